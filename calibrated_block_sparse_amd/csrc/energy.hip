// Block energy of the post-softmax attention (zhichai.net article on
// CalibAtt, §三 offline calibration steps 1-2):
//   E[r][c] = (1/|I_r|) * sum_{i in I_r} sum_{j in J_c} P_ij,
//   P = softmax(scale * Q K^T) over all N keys.
//
// P is never materialised. Pass 1 walks every key block of a query tile and
// keeps, per query row, the running max (log2 units) and the running sum of
// exp2 (online, as in the attention kernel). Pass 2 walks the key blocks
// again, forms exp2(s - m_i) / l_i in fp32 and reduces each 128 x 128 tile
// to one number: lane-local sums, a wave reduction, and a fixed-order sum
// of the four waves at the end, so the result is bitwise reproducible.
#include "device_common.h"
#include "kernels.h"

namespace calibatt {

constexpr int kMaxBlocksEnergy = 2048;

__device__ __forceinline__ void tile_of(int item, int R, int& head, int& tile) {
  head = item / R;
  tile = item - head * R;
}

__global__ void __launch_bounds__(kThreads, 2) energy_stats_kernel(const EnergyArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBlock * kLdsStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int R = a.n_blocks, N = a.n_tokens;
  int head, tile;
  tile_of(xcd_remap(blockIdx.x, a.heads * R), R, head, tile);
  const int64_t hoff = (int64_t)head * a.stride_head;
  const int qi = tile * kBlock + wave * 32 + l32;
  bf16x8 qf[8];
  load_query(qf, a.q + hoff, a.stride_token, qi, qi < N, g);

  const float sl = a.scale_log2;
  float m_run = -__builtin_inff(), l_run = 0.f;
  for (int c = 0; c < R; ++c) {
    const int key0 = c * kBlock;
    __syncthreads();
    stage_rows(sK, a.k + hoff, a.stride_token, key0, N, tid);
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
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) lsum += fast_exp2(__builtin_fmaf(sacc[t][i], sl, -m_new));
    l_run = l_run * alpha + lsum;
    m_run = m_new;
  }
  const float ltot = l_run + __shfl_xor(l_run, 32);
  if (g == 0) {
    const int64_t idx = (int64_t)head * R * kBlock + qi;
    a.row_max[idx] = m_run;
    a.row_sum[idx] = ltot;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ void __launch_bounds__(kThreads, 2) energy_tiles_kernel(const EnergyArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBlock * kLdsStride];
  __shared__ float sE[4][kMaxBlocksEnergy];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int R = a.n_blocks, N = a.n_tokens;
  int head, tile;
  tile_of(xcd_remap(blockIdx.x, a.heads * R), R, head, tile);
  const int64_t hoff = (int64_t)head * a.stride_head;
  const int qi = tile * kBlock + wave * 32 + l32;
  const bool qvalid = qi < N;
  bf16x8 qf[8];
  load_query(qf, a.q + hoff, a.stride_token, qi, qvalid, g);
  const int64_t sidx = (int64_t)head * R * kBlock + qi;
  const float mi = qvalid ? a.row_max[sidx] : 0.f;
  const float inv_l = qvalid ? 1.f / a.row_sum[sidx] : 0.f;

  const float sl = a.scale_log2;
  for (int c = 0; c < R; ++c) {
    const int key0 = c * kBlock;
    __syncthreads();
    stage_rows(sK, a.k + hoff, a.stride_token, key0, N, tid);
    __syncthreads();
    f32x16 sacc[4];
    scores_transposed(sacc, sK, qf, l32, g);
    mask_ragged_keys(sacc, key0, N, g);
    float part = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) part += fast_exp2(__builtin_fmaf(sacc[t][i], sl, -mi));
    part = wave_sum(part * inv_l);
    if (lane == 0) sE[wave][c] = part;
  }
  __syncthreads();
  const int rows = (tile + 1) * kBlock <= N ? kBlock : N - tile * kBlock;
  const float inv_rows = 1.f / (float)rows;
  float* out = a.energy + ((int64_t)head * R + tile) * R;
  for (int c = tid; c < R; c += kThreads)
    out[c] = (((sE[0][c] + sE[1][c]) + sE[2][c]) + sE[3][c]) * inv_rows;
}

hipError_t launch_block_energy(const EnergyArgs& a, hipStream_t stream) {
  const int items = a.heads * a.n_blocks;
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(energy_stats_kernel, dim3(items), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(energy_tiles_kernel, dim3(items), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace calibatt
