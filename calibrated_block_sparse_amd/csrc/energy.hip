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
// summed in ascending i, so the result is bitwise reproducible.
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

  copy_tile<false>(lds0, kh, cp, 0, N, wave, lane);

  // One block with its K tile in buffer kBuf.
  auto block = [&](auto kBufC, int c) {
    constexpr int kBuf = decltype(kBufC)::value;
    wait_vmem<0>();
    lds_barrier();  // K(c) landed; every wave is done with the other buffer
    if (c + 1 < R) copy_tile<false>(lds0 + (1 - kBuf) * kTileBytes, kh, cp, (c + 1) * kBlock, N, wave, lane);

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
    const float row = pair_sum_e(ps);
    if (g == 0 && qvalid) part_out[(int64_t)c * np] = float2{row, mref};
  };

  int c = 0;
  for (; c + 1 < R; c += 2) {
    block(std::integral_constant<int, 0>{}, c);
    block(std::integral_constant<int, 1>{}, c + 1);
  }
  if (c < R) block(std::integral_constant<int, 0>{}, c);

  const float ltot = pair_sum_e(l_run);
  if (g == 0 && qvalid) reinterpret_cast<float2*>(a.row_stats)[(int64_t)head * np + qi] = float2{m_run, ltot};
}

__global__ void __launch_bounds__(kThreads) energy_fixup_kernel(const EnergyArgs a) {
  __shared__ float s_m[kBlock], s_inv[kBlock];
  const int R = a.n_blocks, N = a.n_tokens;
  const int head = blockIdx.x / R, r = blockIdx.x - head * R;
  const int64_t np = (int64_t)R * kBlock;
  const int rows = (r + 1) * kBlock <= N ? kBlock : N - r * kBlock;
  const float2* __restrict__ st = reinterpret_cast<const float2*>(a.row_stats) + (int64_t)head * np + r * kBlock;
  if ((int)threadIdx.x < rows) {
    const float2 v = st[threadIdx.x];
    s_m[threadIdx.x] = v.x;
    s_inv[threadIdx.x] = 1.f / v.y;
  }
  __syncthreads();
  const float inv_rows = 1.f / (float)rows;
  const float2* __restrict__ part =
      reinterpret_cast<const float2*>(a.partials) + (int64_t)head * R * np + r * kBlock;
  float* out = a.energy + ((int64_t)head * R + r) * R;
  for (int c = threadIdx.x; c < R; c += kThreads) {
    const float2* p = part + (int64_t)c * np;
    float acc = 0.f;
    for (int i = 0; i < rows; ++i) {
      const float2 v = p[i];
      acc = __builtin_fmaf(v.x, __builtin_ldexpf(s_inv[i], (int)(v.y - s_m[i])), acc);
    }
    out[c] = acc * inv_rows;
  }
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
