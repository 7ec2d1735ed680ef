// Block-sparse attention forward over per-query-block kept lists, with
// "repeat" heads that attend from anchor rows only and broadcast the result.
//
// Method: CalibAtt (zhichai.net article on CalibAtt, §三 online inference):
// a non-repeat head walks the precomputed kept-block list of each query
// block and skips every other block; a repeat head computes only k anchor
// rows per frame and copies their outputs to the other rows of the frame.
// The repeat broadcast is fused into the store of this kernel instead of a
// separate gather/scatter pass.
//
// One workgroup = one 128-query tile of one head (a query block of a
// non-repeat head, or 128 consecutive anchor queries of a repeat head).
// Per kept key block:
//   S^T = K Q^T on bf16 MFMA (Q held in registers for the whole tile),
//   online softmax in fp32 with exp2,
//   O^T += V^T P^T on bf16 MFMA (P stays in registers).
// K and V tiles are copied global -> LDS by the load unit directly (no
// register round trip). The copy of K for the next kept block starts as
// soon as every wave has finished reading the current K tile and runs under
// the softmax and the P.V product; the copy of V for the next block runs
// under the next S^T product. 64 KiB of LDS per workgroup, two workgroups per
// CU, so one workgroup's softmax overlaps the other's MFMA work.
#include "device_common.h"
#include "kernels.h"

namespace calibatt {

// The running row max is only raised when a block's max exceeds it by more
// than this many powers of two. Probabilities computed against a stale max
// are at most 2^8 and the final division by the row sum cancels the choice
// of reference exactly, so this saves the rescale of the output accumulator
// on almost every block without changing the result.
constexpr float kLazyRescaleLog2 = 8.f;

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(const AttnArgs a) {
  // Dynamic LDS (2 tiles): its contents are written by the copy engine
  // behind the compiler's back, so it must not be a static object the
  // compiler believes it fully sees.
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  uint8_t* const sK = smem;
  uint8_t* const sV = smem + kTileBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const uint32_t ldsK = lds_addr(sK), ldsV = lds_addr(sV);

  // ---- which tile
  const int item = xcd_remap(blockIdx.x, a.n_items);
  const int rep_items = a.n_rep * a.rep_tiles;
  const bool rep = item < rep_items;
  int head, tile;
  if (rep) {
    head = a.heads[item / a.rep_tiles];
    tile = item % a.rep_tiles;
  } else {
    const int j = item - rep_items;
    head = a.heads[a.n_rep + j / a.n_blocks];
    tile = j % a.n_blocks;
  }
  const int N = a.n_tokens, R = a.n_blocks;
  const int64_t st = a.stride_token;
  const int64_t hoff = (int64_t)head * a.stride_head;
  const uint16_t* __restrict__ qh = a.q + hoff;
  const uint16_t* __restrict__ kh = a.k + hoff;
  const uint16_t* __restrict__ vh = a.v + hoff;
  uint16_t* __restrict__ oh = a.o + hoff;

  // ---- this lane's query row
  const int qi = tile * kBlock + wave * 32 + l32;
  bool qvalid;
  int64_t qtok = 0;
  int f = 0, m = 0, x = 0;
  if (rep) {
    qvalid = qi < a.anchor_queries;
    if (qvalid) {
      const int per_frame = a.anchors * a.cols;
      f = qi / per_frame;
      const int rem = qi - f * per_frame;
      m = rem / a.cols;
      x = rem - m * a.cols;
      const int arow = (2 * m + 1) * a.rows / (2 * a.anchors);
      qtok = ((int64_t)f * a.rows + arow) * a.cols + x;
    }
  } else {
    qvalid = qi < N;
    qtok = qi;
  }
  bf16x8 qf[8];
  load_query(qf, qh, st, qtok, qvalid, g);
  // Make the compiler wait for the query loads here, before any tile copy
  // is in flight (it does not see the copies and would otherwise wait for
  // everything outstanding at the first use inside the loop).
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(qf[s]));

  // ---- kept-block range [beg, end): list positions (sparse) or blocks (repeat)
  int beg = 0, end = R;
  if (!rep) {
    const int64_t row = (int64_t)head * R + tile;
    int64_t b = a.offsets[row], e = a.offsets[row + 1];
    b = b < 0 ? 0 : (b > a.nnz ? a.nnz : b);
    e = e < b ? b : (e > a.nnz ? a.nnz : e);
    beg = (int)b;
    end = (int)e;
  }
  // Key block at list position `it`; an index outside [0, R) is loaded as
  // block 0 and contributes nothing (all of its keys are masked). The list
  // is read-only for the kernel's lifetime, so it is read with scalar loads
  // (constant address space), which the tile copies do not wait behind.
  const __attribute__((address_space(4))) int32_t* idx4 =
      (const __attribute__((address_space(4))) int32_t*)a.indices;
  auto block_at = [&](int it) -> int { return rep ? it : idx4[it]; };

  const CopyPlan cp = make_copy_plan(st, lane);
  const float sl = a.scale_log2;
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) oacc[u] = f32x16{};

  int c = 0;
  if (beg < end) {
    c = block_at(beg);
    const int cl = (unsigned)c < (unsigned)R ? c : 0;
    copy_tile<false>(ldsK, kh, cp, cl * kBlock, N, wave, lane);
    copy_tile<true>(ldsV, vh, cp, cl * kBlock, N, wave, lane);
  }

  for (int it = beg; it < end; ++it) {
    const bool has_next = it + 1 < end;
    const int cn = has_next ? block_at(it + 1) : 0;
    const int cnl = (unsigned)cn < (unsigned)R ? cn : 0;
    const int key0 = c * kBlock;
    // valid keys of this block: 0 for an out-of-range index
    const int key_lim = (unsigned)c < (unsigned)R ? (N - key0 < kBlock ? N - key0 : kBlock) : 0;

    // ---- K(it) is in LDS once this lane's copies of it have landed and
    // every wave has passed the barrier (V(it) may still be in flight).
    wait_vmem<kCopiesPerTile>();
    lds_barrier();

    f32x16 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) sacc[t] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // row 32t + l32 has the same swizzle as row l32
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + 32 * t * 256 + k_operand_offset(l32, s, g));
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[t], 0, 0, 0);
      }
    }
    lds_barrier();  // every wave is done with sK
    if (has_next) copy_tile<false>(ldsK, kh, cp, cnl * kBlock, N, wave, lane);

    if (key_lim < kBlock) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (acc_key(t, i, g) >= key_lim) sacc[t][i] = -__builtin_inff();
    }

    // ---- online softmax (log2 units)
    float mx = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, sacc[t][i]);
    mx = pair_max(mx);
    const float mblk = mx * sl;
    const bool up = mblk > m_run + kLazyRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float m_new = up ? mblk : m_run;
      const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int u = 0; u < 4; ++u) oacc[u] *= alpha;
      m_run = m_new;
    }
    const float mref = m_run == -__builtin_inff() ? 0.f : m_run;

    bf16x8 pf[8];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pf[2 * t + (i >> 3)][i & 7] = (__bf16)fast_exp2(__builtin_fmaf(sacc[t][i], sl, -mref));
    // The row sum adds the same bf16-rounded probabilities that enter P.V,
    // so a dominant key's rounding cancels between numerator and denominator
    // (it would not with a stale reference max). Two per dot instruction.
    {
      const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        ls0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[s], pf[s], 0, 1), ones, ls0, false);
        ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[s], pf[s], 2, 3), ones, ls1, false);
        ls0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[s], pf[s], 4, 5), ones, ls0, false);
        ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[s], pf[s], 6, 7), ones, ls1, false);
      }
      l_run += ls0 + ls1;
    }

    // ---- V(it) in LDS (K(it+1) may still be in flight)
    if (has_next) wait_vmem<kCopiesPerTile>();
    else wait_vmem<0>();
    lds_barrier();

#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 vf = v_operand(sV + s * 4096, v_operand_offset(u, lane));
        oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s], oacc[u], 0, 0, 0);
      }
    }
    lds_barrier();  // every wave is done with sV
    if (has_next) copy_tile<true>(ldsV, vh, cp, cnl * kBlock, N, wave, lane);
    c = cn;
  }

  // ---- epilogue: normalise and store (broadcast for repeat heads)
  const float ltot = pair_sum(l_run);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (!qvalid) return;
  u32x2 packed[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      __bf16 h0 = (__bf16)(oacc[u][4 * b + 0] * inv);
      __bf16 h1 = (__bf16)(oacc[u][4 * b + 1] * inv);
      __bf16 h2 = (__bf16)(oacc[u][4 * b + 2] * inv);
      __bf16 h3 = (__bf16)(oacc[u][4 * b + 3] * inv);
      packed[u][b] = u32x2{(uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16),
                           (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16)};
    }
  int y0 = 0, y1 = 1;
  if (rep) {
    y0 = (m * a.rows + a.anchors - 1) / a.anchors;
    y1 = ((m + 1) * a.rows + a.anchors - 1) / a.anchors;
  }
  for (int y = y0; y < y1; ++y) {
    const int64_t tok = rep ? ((int64_t)f * a.rows + y) * a.cols + x : qtok;
    uint16_t* dst = oh + tok * st;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<u32x2*>(dst + 32 * u + 8 * b + 4 * g) = packed[u][b];
  }
}

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(a.n_items), dim3(kThreads), 2 * kTileBytes, stream, a);
  return hipGetLastError();
}

}  // namespace calibatt
