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
// K tiles and transposed V tiles are copied global -> LDS by the load unit
// directly (no register round trip). The copy of K for the next kept block
// starts as soon as every wave has finished reading the current K tile and
// runs under the softmax and the P.V product; the copy of V for the next
// block runs under the next S^T product. 64 KiB of LDS per workgroup, two
// workgroups per CU, so one workgroup's softmax overlaps the other's MFMA
// work.
//
// V is used transposed. The P.V product needs, per lane, eight keys of one
// head-dimension column; reading them out of key-major V in LDS takes
// transposing 8-byte reads, which move half the bytes per LDS cycle of a
// 16-byte read and made LDS bandwidth the bound of the whole kernel. So a
// pre-pass (v_transpose_kernel, HBM-bound, about 1% of the attention time)
// writes every 128-key block of V as a [128 d][128 keys] tile into the
// caller's workspace, keys permuted inside each group of 16 as
// 0-3, 8-11, 4-7, 12-15 -- the order in which a lane holds its
// probabilities. V^T tiles then go through exactly the K-tile path: same
// copy, same swizzle, same 16-byte operand reads.
#include "device_common.h"
#include "kernels.h"


namespace calibatt {

// The running row max is only raised when a block's max exceeds it by more
// than this many powers of two. Probabilities computed against a stale max
// are at most 2^8 and the final division by the row sum cancels the choice
// of reference exactly, so this saves the rescale of the output accumulator
// on almost every block without changing the result.
constexpr float kLazyRescaleLimit = 256.f;  // 2^8

// LDS operand reads kept in flight ahead of the MFMA that uses them.
#ifndef CALIBATT_READ_DEPTH
#define CALIBATT_READ_DEPTH 3
#endif

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Instruction order inside a scheduling region of kM MFMAs that each take
// one LDS operand read: kDepth reads up front, then per MFMA the read kDepth
// ahead and kV vector instructions. Left to itself the compiler issues each
// read right before its MFMA and waits for it, exposing the LDS latency on
// every MFMA.
template <int kM, int kDepth, int kV>
__device__ __forceinline__ void pipeline_reads() {
  __builtin_amdgcn_sched_group_barrier(0x100, kDepth, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < kM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
    if (i + kDepth < kM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (kV > 0) __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);  // VALU
  }
}

// Items, in launch order: tiles of masked repeat heads (repeat heads that
// also keep their block mask, a variant the pages leave open: anchor query
// n attends only to the blocks its own block-row floor(n / 128) keeps), of
// plain repeat heads, then query blocks of block-sparse heads. A masked tile
// builds, in LDS behind the two tiles, a bitmap of kept blocks per query and
// the ascending union of its queries' lists, walks the union, and drops a
// block for a query outside its row by moving that query's reference to
// +inf for the block (its exponentials are exactly 0). kAnyMasked is false
// for launches without masked repeat heads, which then compile to the
// plain loop.
template <bool kAnyMasked>
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
  const bool masked = kAnyMasked && item < a.n_mrep * a.rep_tiles;   // heads[0 .. n_mrep) are masked
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
  // masked repeat tiles: per-query bitmaps [128][W] words, their union [W],
  // the union as an ascending list [R] and its length
  const int W = a.mask_words;
  uint32_t* const bm = reinterpret_cast<uint32_t*>(smem + 2 * kTileBytes);
  uint16_t* const ul = reinterpret_cast<uint16_t*>(bm + 129 * W);
  const int qidx = wave * 32 + l32;
  if (masked) {
    uint32_t* const ub = bm + 128 * W;
    uint32_t* const cnt = reinterpret_cast<uint32_t*>(ul) + (R + 1) / 2;
    for (int i = tid; i < 129 * W; i += kThreads) bm[i] = 0u;
    __syncthreads();
    if (g == 0 && qvalid) {
      const int64_t row = (int64_t)head * R + qtok / kBlock;
      int64_t b = a.offsets[row], e = a.offsets[row + 1];
      b = b < 0 ? 0 : (b > a.nnz ? a.nnz : b);
      e = e < b ? b : (e > a.nnz ? a.nnz : e);
      for (int64_t i = b; i < e; ++i) {
        const int cc = a.indices[i];
        if ((unsigned)cc >= (unsigned)R) continue;
        const uint32_t bit = 1u << (cc & 31);
        bm[qidx * W + (cc >> 5)] |= bit;
        atomicOr(&ub[cc >> 5], bit);
      }
    }
    __syncthreads();
    if (wave == 0) {  // compaction of the union (W <= 64 words)
      uint32_t wv = lane < W ? ub[lane] : 0u;
      const int n = __builtin_popcount(wv);
      int incl = n;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      int pos = incl - n;
      while (wv) {
        const int bit = __builtin_ctz(wv);
        ul[pos++] = (uint16_t)(lane * 32 + bit);
        wv &= wv - 1u;
      }
      if (lane == 63) *cnt = (uint32_t)incl;
    }
    __syncthreads();
    end = (int)__builtin_amdgcn_readfirstlane(*cnt);
  } else if (!rep) {
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
  auto block_at = [&](int it) -> int {
    if (masked) return (int)__builtin_amdgcn_readfirstlane(ul[it]);
    return rep ? it : idx4[it];
  };
  // whether this lane's query keeps the current block (masked repeat tiles)
  bool member = true;

  const CopyPlan cp = make_copy_plan(st, lane);
  const CopyPlan cpt = make_copy_plan(kBlock, lane);   // V^T tiles: 256-byte rows
  const uint16_t* __restrict__ vth = a.vt + (int64_t)head * R * (kBlock * kDim);
  // Per-lane LDS base address of the K operand for d-step s; K rows 32t + l32
  // and V^T rows 32u + l32 share the swizzle of row l32, so the tile, the
  // sub-tile and the K/V choice are compile-time displacements.
  uint32_t kaddr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kaddr[s] = ldsK + (uint32_t)k_operand_offset(l32, s, g);
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
    copy_tile(ldsK, kh, cp, cl * kBlock, N, wave, lane);
    copy_tile(ldsV, vth, cpt, cl * kBlock, R * kBlock, wave, lane);
  }

  // S^T tile t (keys 32t .. 32t+31 of the block x this wave's 32 queries).
  auto qk_tile = [&](f32x16& sa, int t) {
    sa = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 kf = lds_read_b128(kaddr[s] + 8192 * t);
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sa, 0, 0, 0);
    }
  };

  // Probabilities of a score tile against the reference `mref` (16 per
  // lane, as bf16), and their sum into `bsum` (the bf16-rounded values, two
  // per dot instruction). Keys past the end of a ragged block were loaded as
  // copies of key N-1 (their scores repeat a real score of the same block);
  // their probabilities are zeroed and the sum redone afterwards.
  auto probs_tile = [&](const f32x16& sa, bf16x8& p_lo, bf16x8& p_hi, float mref, float& bsum) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p_lo[i] = (__bf16)fast_exp2(__builtin_fmaf(sa[i], sl, -mref));
      p_hi[i] = (__bf16)fast_exp2(__builtin_fmaf(sa[8 + i], sl, -mref));
    }
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    float s0 = 0.f, s1 = 0.f;
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p_lo, p_lo, 0, 1), ones, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p_hi, p_hi, 0, 1), ones, s1, false);
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p_lo, p_lo, 2, 3), ones, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p_hi, p_hi, 2, 3), ones, s1, false);
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p_lo, p_lo, 4, 5), ones, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p_hi, p_hi, 4, 5), ones, s1, false);
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p_lo, p_lo, 6, 7), ones, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p_hi, p_hi, 6, 7), ones, s1, false);
    bsum += s0 + s1;
    // Materialise the probabilities here: left alone the compiler sinks the
    // exponentials into the branches after the rescale test (whose rare path
    // recomputes them).
    asm volatile("" ::"v"(p_lo), "v"(p_hi));
  };

  // O^T += V^T P^T for key groups s0 .. s0+3 (16 keys each). The A operand
  // of lane (l32, g) for output tile u and key group s is V^T row 32u + l32,
  // logical chunk 2s + g: the K-operand address of d-step s, moved to the
  // V^T tile.
  auto pv_steps = [&](const bf16x8 (&pf)[8], int s0) {
#pragma unroll
    for (int s = s0; s < s0 + 4; ++s) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 vf = lds_read_b128(kaddr[s] + kTileBytes + 8192 * u);
        oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s], oacc[u], 0, 0, 0);
      }
    }
  };

  // Row sum (this lane's 64 keys) of the bf16-rounded probabilities that
  // enter P.V, so a dominant key's rounding cancels between numerator and
  // denominator (it would not with a stale reference max).
  auto row_sum = [&](const bf16x8 (&pf)[8]) -> float {
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      ls0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[s], pf[s], 0, 1), ones, ls0, false);
      ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[s], pf[s], 2, 3), ones, ls1, false);
      ls0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[s], pf[s], 4, 5), ones, ls0, false);
      ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[s], pf[s], 6, 7), ones, ls1, false);
    }
    return ls0 + ls1;
  };

  // Zeroes the probabilities of keys at or past key_lim (ragged last block;
  // every key of an out-of-range index). Dword d of pf[s] holds the bf16
  // pair of keys 16s + 8(d/2) + 4g + 2(d%2) + {0, 1}; the mask is built with
  // integer arithmetic (no per-element compares held in scalar registers).
  auto zero_masked_probs = [&](bf16x8 (&pf)[8], int key_lim) {
    const int t0 = key_lim - 4 * g;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 w = __builtin_bit_cast(u32x4, pf[s]);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        int n = t0 - (16 * s + 8 * (d >> 1) + 2 * (d & 1));  // valid keys in the pair
        n = n < 0 ? 0 : (n > 2 ? 2 : n);
        const uint32_t mask = (uint32_t)(n > 0 ? 1 : 0) * 0xffffu | (uint32_t)(n >> 1) * 0xffff0000u;
        w[d] &= mask;
      }
      pf[s] = __builtin_bit_cast(bf16x8, w);
    }
  };

  // Scores of one block (all four tiles stay in registers, so the K tile is
  // free, and the next one can be copied, as soon as the last score MFMA
  // has read it), then its probabilities and this lane's sum of them. The
  // probabilities are taken against the current reference max before
  // anything about the block is known; the reference is only moved (lazy
  // rescale) when some lane's sum exceeds 2^8 -- which bounds every
  // probability by 2^8 without computing the block max -- or on the first
  // block; then the block max is taken from the scores in registers, the
  // output rescaled and the probabilities redone.
  f32x16 sacc[4];
  auto scores = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t) qk_tile(sacc[t], t);
    pipeline_reads<32, CALIBATT_READ_DEPTH, 0>();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto probs = [&](bf16x8 (&pf)[8]) -> float {
    const float mref = !member ? __builtin_inff() : (m_run == -__builtin_inff() ? 0.f : m_run);
    float bsum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) probs_tile(sacc[t], pf[2 * t], pf[2 * t + 1], mref, bsum);
    const bool first = m_run == -__builtin_inff();
    if (__builtin_amdgcn_ballot_w64(first || bsum > kLazyRescaleLimit)) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, sacc[t][i]);
      if (!member) mx = -__builtin_inff();
      const float m_new = __builtin_fmaxf(m_run, pair_max(mx) * sl);
      const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int u = 0; u < 4; ++u) oacc[u] *= alpha;
      m_run = m_new;
      bsum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) probs_tile(sacc[t], pf[2 * t], pf[2 * t + 1], member ? m_run : __builtin_inff(), bsum);
    }
    return bsum;
  };

  for (int it = beg; it < end; ++it) {
    const bool has_next = it + 1 < end;
    const int cn = has_next ? block_at(it + 1) : 0;
    const int cnl = (unsigned)cn < (unsigned)R ? cn : 0;
    const int key0 = c * kBlock;
    // valid keys of this block: 0 for an out-of-range index
    const int key_lim = (unsigned)c < (unsigned)R ? (N - key0 < kBlock ? N - key0 : kBlock) : 0;

    // (lanes past the last anchor query are never stored; they keep every
    // block, as in a plain repeat tile, so they never hold the wave in the
    // rescale path)
    if (masked) member = !qvalid || ((bm[qidx * W + (c >> 5)] >> (c & 31)) & 1u);

    // ---- K(it) is in LDS once this lane's copies of it have landed and
    // every wave has passed the barrier (V(it) may still be in flight).
    wait_vmem<kCopiesPerTile>();
    lds_barrier();

    scores();
    lds_barrier();  // every wave is done with sK: the next K tile copies under the softmax
    if (has_next) copy_tile(ldsK, kh, cp, cnl * kBlock, N, wave, lane);
    bf16x8 pf[8];
    float bsum = probs(pf);
    if (key_lim < kBlock) {
      zero_masked_probs(pf, key_lim);
      bsum = row_sum(pf);
    }
    l_run += bsum;

    // ---- V(it) in LDS (K(it+1) may still be in flight)
    if (has_next) wait_vmem<kCopiesPerTile>();
    else wait_vmem<0>();
    lds_barrier();
    pv_steps(pf, 0);
    pipeline_reads<16, CALIBATT_READ_DEPTH, 0>();
    __builtin_amdgcn_sched_barrier(0);
    pv_steps(pf, 4);
    pipeline_reads<16, CALIBATT_READ_DEPTH, 0>();
    lds_barrier();  // every wave is done with sV
    if (has_next) copy_tile(ldsV, vth, cpt, cnl * kBlock, R * kBlock, wave, lane);
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

// V^T pre-pass: one workgroup per (head, 128-key block). Reads the block's
// rows of V (rows at or past N read as zero), writes the [128 d][128 keys]
// tile with keys permuted inside each group of 16 as 0-3, 8-11, 4-7, 12-15.
// Staged through LDS with rows padded by 4 bytes, so the column reads of
// eight different keys fall in different banks.
__global__ void __launch_bounds__(kThreads) v_transpose_kernel(const VtArgs a) {
  constexpr int kPitch = kDim * 2 + 4;  // bytes per staged key row
  __shared__ __attribute__((aligned(16))) uint8_t tile[kBlock * kPitch];
  const int tid = threadIdx.x;
  const int head = blockIdx.x / a.n_blocks, c = blockIdx.x % a.n_blocks;
  const uint16_t* __restrict__ src = a.v + (int64_t)head * a.stride_head;
  // load: 128 rows x 16 chunks of 16 bytes
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int idx = tid + kThreads * j;
    const int row = idx >> 4, ch = idx & 15;
    const int tok = c * kBlock + row;
    const u32x4 w = tok < a.n_tokens ? load16(src + (int64_t)tok * a.stride_token + ch * 8)
                                     : u32x4{0u, 0u, 0u, 0u};
    uint32_t* d = reinterpret_cast<uint32_t*>(tile + row * kPitch + ch * 16);
    d[0] = w[0]; d[1] = w[1]; d[2] = w[2]; d[3] = w[3];
  }
  __syncthreads();
  // store: task = (pair of d columns, 8-key chunk); chunk cc covers keys
  // 16(cc/2) + 8(e/4) + 4(cc%2) + e%4, e = 0..7
  uint16_t* __restrict__ dst = a.vt + ((int64_t)head * a.n_blocks + c) * (kBlock * kDim);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int task = tid + kThreads * j;
    const int dp = task >> 4, cc = task & 15;
    const int kb = 16 * (cc >> 1) + 4 * (cc & 1);
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int k0 = kb + 8 * (e >> 2) + (e & 3);
      const uint32_t v0 = *reinterpret_cast<const uint32_t*>(tile + k0 * kPitch + dp * 4);
      const uint32_t v1 = *reinterpret_cast<const uint32_t*>(tile + (k0 + 1) * kPitch + dp * 4);
      lo[e >> 1] = (v0 & 0xffffu) | (v1 << 16);            // column 2dp
      hi[e >> 1] = (v0 >> 16) | (v1 & 0xffff0000u);        // column 2dp + 1
    }
    *reinterpret_cast<u32x4*>(dst + (2 * dp) * kBlock + cc * 8) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *reinterpret_cast<u32x4*>(dst + (2 * dp + 1) * kBlock + cc * 8) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  }
}

hipError_t launch_v_transpose(const VtArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.heads * a.n_blocks;
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(v_transpose_kernel, dim3((unsigned)items), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  size_t lds = 2 * kTileBytes;
  if (a.n_mrep == 0) {
    hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3(a.n_items), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
  }
  {
    // masked repeat tiles: bitmaps, union and list behind the two tiles.
    // The dynamic-LDS limit is a per-device attribute of the kernel; it is
    // set on every such launch (a host-side call), so calls from several
    // threads or on several devices need no shared state.
    lds += ((size_t)129 * a.mask_words * 4 + 2 * ((size_t)a.n_blocks + 2) + 4 + 15) / 16 * 16;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<true>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3(a.n_items), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace calibatt
