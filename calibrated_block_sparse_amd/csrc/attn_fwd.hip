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
// Per kept key block: stage K (row-major) and V (transposed) in LDS,
// S^T = K Q^T on bf16 MFMA, online softmax in fp32 with exp2, O^T += V^T P^T
// on bf16 MFMA. Two workgroups share a CU so that one's softmax and tile
// loads overlap the other's MFMA work.
#include "device_common.h"
#include "kernels.h"

namespace calibatt {

__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBlock * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kDim * kLdsStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

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

  // ---- kept-block range
  int beg = 0, end = R;
  if (!rep) {
    const int64_t row = (int64_t)head * R + tile;
    int64_t b = a.offsets[row], e = a.offsets[row + 1];
    b = b < 0 ? 0 : (b > a.nnz ? a.nnz : b);
    e = e < b ? b : (e > a.nnz ? a.nnz : e);
    beg = (int)b;
    end = (int)e;
  }

  const float sl = a.scale_log2;
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) oacc[u] = f32x16{};

  for (int it = beg; it < end; ++it) {
    const int c = rep ? it : __builtin_amdgcn_readfirstlane(a.indices[it]);
    if ((unsigned)c >= (unsigned)R) continue;
    const int key0 = c * kBlock;

    __syncthreads();  // previous block's LDS reads are done
    stage_rows(sK, kh, st, key0, N, tid);
    stage_values_transposed(sV, vh, st, key0, N, tid);
    __syncthreads();

    f32x16 sacc[4];
    scores_transposed(sacc, sK, qf, l32, g);
    mask_ragged_keys(sacc, key0, N, g);

    float mx = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, sacc[t][i]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = __builtin_fmaxf(m_run, mx * sl);
    const float alpha = (m_run == -__builtin_inff()) ? 0.f : fast_exp2(m_run - m_new);
    m_run = m_new;

    float lsum = 0.f;
    bf16x8 pf[8];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(sacc[t][i], sl, -m_new));
        lsum += p;
        pf[2 * t + (i >> 3)][i & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int u = 0; u < 4; ++u) oacc[u] *= alpha;

#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sV + (32 * u + l32) * kLdsStride + 16 * s + 8 * g);
        oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s], oacc[u], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: normalise and store (broadcast for repeat heads)
  const float ltot = l_run + __shfl_xor(l_run, 32);
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
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(a.n_items), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace calibatt
