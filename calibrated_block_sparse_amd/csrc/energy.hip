// Block energy of the post-softmax attention (zhichai.net article on
// CalibAtt, §三 offline calibration steps 1-2):
//   E[r][c] = (1/|I_r|) * sum_{i in I_r} sum_{j in J_c} P_ij,
//   P = softmax(scale * Q K^T) over all N keys.
//
// P is never materialised, and Q K^T is computed once.
//
// energy_partials_kernel: one workgroup (4 waves, 32 query rows each) per
// (head, 128-query tile) walks every key block c and stores, per query row
// i, the block's partial sum  s_c(i) = sum_{j in J_c} 2^(S_ij - m_c(i))  with
// its reference m_c(i) (log2 units, S = scale * log2(e) * q.k), and at the
// end the row's total  l(i) = sum_j 2^(S_ij - m(i))  with its final
// reference m(i). References are integers and move only when a block would
// push a lane's partial past 2^8 (lazy rescale), so every rescale and the
// fix-up's change of reference are exact powers of two.
//
// energy_fixup_kernel: E[r][c] = (1/|I_r|) sum_i s_c(i) 2^(m_c(i) - m(i)) / l(i),
// summed in a fixed order (four consecutive rows per lane, then a butterfly
// over 32 lanes), so the result is bitwise reproducible.
//
// K tiles are copied global -> LDS by the load unit (two buffers: the copy of
// block c+1 runs under the whole computation of block c); operand reads are
// software-pipelined as in the attention kernel.
#include "device_common.h"
#include "kernels.h"

#include <type_traits>

namespace calibatt {

namespace {

constexpr float kEnergyLazyLimit = 256.f;  // a lane's partial may reach 2^8

#ifndef CALIBATT_READ_DEPTH
#define CALIBATT_READ_DEPTH 3
#endif

template <int kM, int kDepth, int kV>
__device__ __forceinline__ void pipeline_reads_e() {
  __builtin_amdgcn_sched_group_barrier(0x100, kDepth, 0);
#pragma unroll
  for (int i = 0; i < kM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + kDepth < kM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (kV > 0) __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
  }
}

__device__ __forceinline__ float pair_sum_e(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float pair_max_e(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace

__global__ void __launch_bounds__(kThreads, 2) energy_partials_kernel(const EnergyArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // two K tiles
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int R = a.n_blocks, N = a.n_tokens;
  const int item = xcd_remap(blockIdx.x, a.heads * R);
  const int head = item / R, tile = item - head * R;
  const int64_t hoff = (int64_t)head * a.stride_head;
  const uint16_t* __restrict__ kh = a.k + hoff;
  const int qi = tile * kBlock + wave * 32 + l32;
  const bool qvalid = qi < N;
  bf16x8 qf[8];
  load_query(qf, a.q + hoff, a.stride_token, qi, qvalid, g);
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(qf[s]));

  const uint32_t lds0 = lds_addr(smem);
  uint32_t kaddr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kaddr[s] = lds0 + (uint32_t)k_operand_offset(l32, s, g);
  const CopyPlan cp = make_copy_plan(a.stride_token, lane);
  const float sl = a.scale_log2;
  const int64_t np = (int64_t)R * kBlock;  // padded rows
  float2* __restrict__ part_out = reinterpret_cast<float2*>(a.partials) + (int64_t)head * R * np + qi;

  float m_run = -__builtin_inff();  // integer-valued once set
  float l_run = 0.f;

  copy_tile(lds0, kh, cp, 0, N, wave, lane);

  // The record of block c is stored at the start of block c+1, after the
  // wait: the wait (vmcnt counts stores too) then never waits for a store
  // issued just before it.
  float prev_row = 0.f, prev_ref = 0.f;
  int prev_c = -1;

  // One block with its K tile in buffer kBuf.
  auto block = [&](auto kBufC, int c) {
    constexpr int kBuf = decltype(kBufC)::value;
    wait_vmem<0>();
    lds_barrier();  // K(c) landed; every wave is done with the other buffer
    if (c + 1 < R) copy_tile(lds0 + (1 - kBuf) * kTileBytes, kh, cp, (c + 1) * kBlock, N, wave, lane);
    if (prev_c >= 0 && g == 0 && qvalid) part_out[(int64_t)prev_c * np] = float2{prev_row, prev_ref};

    f32x16 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 kf = lds_read_b128(kaddr[s] + kBuf * kTileBytes + 8192 * t);
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[t], 0, 0, 0);
      }
    }
    pipeline_reads_e<32, CALIBATT_READ_DEPTH, 0>();
    __builtin_amdgcn_sched_barrier(0);

    // keys at or past N (ragged last block: copies of key N-1) contribute 0
    const int key_lim = N - c * kBlock < kBlock ? N - c * kBlock : kBlock;
    auto partial = [&](float mref) {
      float s0 = 0.f, s1 = 0.f;
      if (key_lim == kBlock) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            s0 += fast_exp2(__builtin_fmaf(sacc[t][i], sl, -mref));
            s1 += fast_exp2(__builtin_fmaf(sacc[t][i + 1], sl, -mref));
          }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            // element i of tile t holds key 32t + 8(i/4) + 4g + i%4
            const int n = key_lim - (32 * t + 8 * (i >> 2) + 4 * g);  // valid keys in its group of 4
            const float e = fast_exp2(__builtin_fmaf(sacc[t][i], sl, -mref));
            s0 += ((i & 3) < n) ? e : 0.f;
          }
      }
      return s0 + s1;
    };
    float mref = m_run == -__builtin_inff() ? 0.f : m_run;
    float ps = partial(mref);
    if (__builtin_amdgcn_ballot_w64(m_run == -__builtin_inff() || ps > kEnergyLazyLimit)) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, sacc[t][i]);
      // integer reference at or above the block max (log2 units)
      const float m_new = __builtin_fmaxf(m_run, __builtin_ceilf(pair_max_e(mx) * sl));
      if (m_new != m_run) {
        l_run = m_run == -__builtin_inff() ? 0.f : __builtin_ldexpf(l_run, (int)(m_run - m_new));
        m_run = m_new;
      }
      mref = m_run;
      ps = partial(mref);
    }
    l_run += ps;
    prev_row = pair_sum_e(ps);
    prev_ref = mref;
    prev_c = c;
  };

  int c = 0;
  for (; c + 1 < R; c += 2) {
    block(std::integral_constant<int, 0>{}, c);
    block(std::integral_constant<int, 1>{}, c + 1);
  }
  if (c < R) block(std::integral_constant<int, 0>{}, c);

  if (prev_c >= 0 && g == 0 && qvalid) part_out[(int64_t)prev_c * np] = float2{prev_row, prev_ref};
  const float ltot = pair_sum_e(l_run);
  if (g == 0 && qvalid) reinterpret_cast<float2*>(a.row_stats)[(int64_t)head * np + qi] = float2{m_run, ltot};
}

// One workgroup per (head, block-row r). Wave w takes key blocks
// 16w .. 16w+15, then 64 further on, ...; its half-wave h the blocks of
// parity h among them. Lane j of the half-wave reads the partials of query
// rows 4j .. 4j+3 of block c (32 contiguous bytes, so a half-wave reads
// block c's 128 partials as one 1 KiB run), sums its four rows in order,
// and the 32 lanes combine by a fixed butterfly.
__global__ void __launch_bounds__(kThreads) energy_fixup_kernel(const EnergyArgs a) {
  __shared__ float s_m[kBlock], s_inv[kBlock];
  const int R = a.n_blocks, N = a.n_tokens;
  const int head = blockIdx.x / R, r = blockIdx.x - head * R;
  const int64_t np = (int64_t)R * kBlock;
  const int rows = (r + 1) * kBlock <= N ? kBlock : N - r * kBlock;
  const float2* __restrict__ st = reinterpret_cast<const float2*>(a.row_stats) + (int64_t)head * np + r * kBlock;
  if ((int)threadIdx.x < kBlock) {
    // rows past N were never written: reference 0 and factor 0
    const bool ok = (int)threadIdx.x < rows;
    const float2 v = ok ? st[threadIdx.x] : float2{0.f, 1.f};
    s_m[threadIdx.x] = v.x;
    s_inv[threadIdx.x] = ok ? 1.f / v.y : 0.f;
  }
  __syncthreads();
  const float inv_rows = 1.f / (float)rows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, j = lane & 31;
  const int i0 = 4 * j;
  const float2* __restrict__ part =
      reinterpret_cast<const float2*>(a.partials) + (int64_t)head * R * np + r * kBlock + i0;
  float* out = a.energy + ((int64_t)head * R + r) * R;
  float f[4], m[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[k] = s_inv[i0 + k];
    m[k] = s_m[i0 + k];
  }
  // Each half-wave takes kFixCols key blocks per pass and issues all their
  // loads before summing, so several reads are in flight per wave.
  constexpr int kFixCols = 8;
  for (int c0 = 2 * kFixCols * wave; c0 < R; c0 += 2 * kFixCols * (kThreads / 64)) {
    float4 v[kFixCols][2];
#pragma unroll
    for (int u = 0; u < kFixCols; ++u) {
      const int c = c0 + 2 * u + half;
      if (c < R) {
        const float4* p = reinterpret_cast<const float4*>(part + (int64_t)c * np);
        v[u][0] = p[0];
        v[u][1] = p[1];
      } else {
        v[u][0] = v[u][1] = float4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < kFixCols; ++u) {
      const int c = c0 + 2 * u + half;
      float acc = 0.f;
      if (c < R) {
        const float s[4] = {v[u][0].x, v[u][0].z, v[u][1].x, v[u][1].z};
        const float e[4] = {v[u][0].y, v[u][0].w, v[u][1].y, v[u][1].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (i0 + k < rows) acc = __builtin_fmaf(s[k], __builtin_ldexpf(f[k], (int)(e[k] - m[k])), acc);
      }
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 32);
      if (j == 0 && c < R) out[c] = acc * inv_rows;
    }
  }
}

// ---------------------------------------------------------------------------
// Spatial similarity of a head (zhichai.net article on CalibAtt, §二
// observation 4 and §三: one score s per (t, l, h); the pages give no
// formula). From the partials above: the profile of spatial row (f, y) is
// rho[c] = (1/W) sum over its W query tokens i of P_i(block c), with
// P_i(block c) = s_c(i) 2^(m_c(i) - m(i)) / l(i); s is the mean over frames
// and non-anchor rows of cos(rho_{f,y}, rho_{f,a(y)}).

// Butterfly sum over the 64 lanes (same order on every lane and call).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// One workgroup per (head, spatial row); wave w takes key blocks w, w+4, ...,
// lane x the row's tokens x, x+64, ...
__global__ void __launch_bounds__(kThreads) row_profile_kernel(const SimArgs a) {
  extern __shared__ float s_row[];  // cols x (m, 1/l)
  const int R = a.n_blocks, W = a.cols, FR = a.frames * a.rows;
  const int head = blockIdx.x / FR, fy = blockIdx.x - head * FR;
  const int64_t np = (int64_t)R * kBlock;
  const int64_t i0 = (int64_t)fy * W;
  const float2* __restrict__ st = reinterpret_cast<const float2*>(a.row_stats) + (int64_t)head * np + i0;
  for (int x = threadIdx.x; x < W; x += kThreads) {
    const float2 v = st[x];
    s_row[2 * x] = v.x;
    s_row[2 * x + 1] = 1.f / v.y;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float2* __restrict__ part = reinterpret_cast<const float2*>(a.partials) + (int64_t)head * R * np + i0;
  float* out = a.profiles + ((int64_t)head * FR + fy) * R;
  const float inv_w = 1.f / (float)W;
  // Each wave takes kProfileCols consecutive key blocks at a time and issues
  // all their loads before any sum, so that many reads are in flight; the
  // sum of each block is still lane x over x, x+64, ... then the butterfly.
  constexpr int kProfileCols = 4;
  for (int c0 = wave * kProfileCols; c0 < R; c0 += (kThreads / 64) * kProfileCols) {
    float acc[kProfileCols];
#pragma unroll
    for (int u = 0; u < kProfileCols; ++u) acc[u] = 0.f;
    for (int x = lane; x < W; x += 64) {
      const float mi = s_row[2 * x], inv_l = s_row[2 * x + 1];
      float2 v[kProfileCols];
#pragma unroll
      for (int u = 0; u < kProfileCols; ++u)
        v[u] = c0 + u < R ? part[(int64_t)(c0 + u) * np + x] : float2{0.f, mi};
#pragma unroll
      for (int u = 0; u < kProfileCols; ++u)
        acc[u] = __builtin_fmaf(v[u].x, __builtin_ldexpf(inv_l, (int)(v[u].y - mi)), acc[u]);
    }
#pragma unroll
    for (int u = 0; u < kProfileCols; ++u) acc[u] = wave_sum(acc[u]);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < kProfileCols; ++u)
        if (c0 + u < R) out[c0 + u] = acc[u] * inv_w;
    }
  }
}

// One workgroup of 16 waves per head; wave w takes the spatial rows w,
// w+16, ... of all frames (in order), lanes the key blocks; per-wave sums
// are combined in wave order.
constexpr int kSimThreads = 1024;

__global__ void __launch_bounds__(kSimThreads) similarity_kernel(const SimArgs a) {
  __shared__ float s_sum[kSimThreads / 64];
  __shared__ int s_cnt[kSimThreads / 64];
  const int R = a.n_blocks, FR = a.frames * a.rows;
  const int head = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* prof = a.profiles + (int64_t)head * FR * R;
  float total = 0.f;
  int count = 0;
  for (int fy = wave; fy < FR; fy += kSimThreads / 64) {
    const int f = fy / a.rows, y = fy - f * a.rows;
    const int m = y * a.anchors / a.rows;
    const int ay = (2 * m + 1) * a.rows / (2 * a.anchors);  // anchor row of y's segment
    if (ay == y) continue;
    const float* u = prof + (int64_t)fy * R;
    const float* w = prof + (int64_t)(f * a.rows + ay) * R;
    float dot = 0.f, uu = 0.f, ww = 0.f;
    for (int c = lane; c < R; c += 64) {
      dot = __builtin_fmaf(u[c], w[c], dot);
      uu = __builtin_fmaf(u[c], u[c], uu);
      ww = __builtin_fmaf(w[c], w[c], ww);
    }
    dot = wave_sum(dot);
    uu = wave_sum(uu);
    ww = wave_sum(ww);
    total += dot / __builtin_sqrtf(uu * ww);
    ++count;
  }
  if (lane == 0) {
    s_sum[wave] = total;
    s_cnt[wave] = count;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    int n = 0;
    for (int w = 0; w < kSimThreads / 64; ++w) {
      t += s_sum[w];
      n += s_cnt[w];
    }
    a.similarity[head] = n == 0 ? 1.f : t / (float)n;
  }
}

hipError_t launch_spatial_similarity(const SimArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.heads * a.frames * a.rows;
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_profile_kernel, dim3((unsigned)items), dim3(kThreads),
                     (size_t)a.cols * 2 * sizeof(float), stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(similarity_kernel, dim3(a.heads), dim3(kSimThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_block_energy(const EnergyArgs& a, hipStream_t stream) {
  const int items = a.heads * a.n_blocks;
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(energy_partials_kernel, dim3(items), dim3(kThreads), 2 * kTileBytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(energy_fixup_kernel, dim3(items), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace calibatt
