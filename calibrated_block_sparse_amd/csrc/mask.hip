// Greedy selection with vote accumulation, vote binarisation, and
// compilation of a block mask into per-query-block kept lists (CSR).
//
// Method: zhichai.net article on CalibAtt, §三 offline calibration: for each
// query block-row, the fewest key blocks whose cumulative energy reaches
// eps(t), taken from the largest energy down; the per-prompt masks are
// averaged over the calibration prompts and binarised at rho; the result is
// a static skip list per (timestep, layer, head).
//
// Selection is exact integer arithmetic: energies become multiples of 2^-40
// (nearest, ties to even), keys (energy << 11 | 2047 - column) are sorted
// by a workgroup bitonic sort in LDS, and an integer prefix scan finds the
// shortest prefix reaching eps. Equal energies therefore order by ascending
// column and the answer does not depend on summation order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace calibatt {

constexpr int kSelThreads = 256;
constexpr int kSelMax = 2048;          // padded row length (power of two)
constexpr int kColBits = 11;
constexpr uint64_t kColMask = (1u << kColBits) - 1;

__device__ __forceinline__ uint64_t quantize_energy(float e) {
  // e * 2^40 is exact in fp64; rint rounds to nearest, ties to even.
  double x = __builtin_rint((double)e * 1099511627776.0);
  if (!(x > 0.0)) x = 0.0;                               // negatives and NaN
  const double top = 2199023255551.0;                    // 2^41 - 1
  if (x > top) x = top;
  return (uint64_t)x;
}

__global__ void __launch_bounds__(kSelThreads) select_votes_kernel(
    const float* __restrict__ energy, int n_draws, int heads, int R, uint64_t eps_fx,
    uint8_t* __restrict__ votes, int32_t* __restrict__ n_sel) {
  __shared__ uint64_t skey[kSelMax];
  __shared__ uint64_t sscan[kSelThreads];
  __shared__ int svote[kSelMax];
  __shared__ int s_nstar;

  const int tid = threadIdx.x;
  const int row = blockIdx.x;            // h * R + r
  int P = 64;
  while (P < R) P <<= 1;
  uint8_t* vrow = votes + (int64_t)row * R;
  for (int c = tid; c < R; c += kSelThreads) svote[c] = vrow[c];

  const int chunk = (R + kSelThreads - 1) / kSelThreads;
  for (int d = 0; d < n_draws; ++d) {
    const float* erow = energy + ((int64_t)d * heads * R + row) * (int64_t)R;
    for (int i = tid; i < P; i += kSelThreads)
      skey[i] = i < R ? (quantize_energy(erow[i]) << kColBits) | (uint64_t)(kColMask - i) : 0ull;
    if (tid == 0) s_nstar = R;
    __syncthreads();

    // Bitonic sort, ascending; the greedy order is read from the top down.
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P; i += kSelThreads) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint64_t x = skey[i], y = skey[ixj];
            const bool up = (i & k) == 0;
            if (up ? (x > y) : (x < y)) {
              skey[i] = y;
              skey[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }

    // Greedy position p (0 = largest energy) lives at skey[P - 1 - p].
    // Thread t owns positions [t*chunk, (t+1)*chunk).
    uint64_t local = 0;
    const int p0 = tid * chunk;
    for (int p = p0; p < p0 + chunk && p < R; ++p) local += skey[P - 1 - p] >> kColBits;
    sscan[tid] = local;
    __syncthreads();
    // Inclusive Hillis-Steele scan of the 256 thread sums.
    for (int off = 1; off < kSelThreads; off <<= 1) {
      const uint64_t add = tid >= off ? sscan[tid - off] : 0ull;
      __syncthreads();
      sscan[tid] += add;
      __syncthreads();
    }
    uint64_t acc = sscan[tid] - local;    // exclusive prefix
    for (int p = p0; p < p0 + chunk && p < R; ++p) {
      acc += skey[P - 1 - p] >> kColBits;
      if (acc >= eps_fx) {
        atomicMin(&s_nstar, p + 1);
        break;
      }
    }
    __syncthreads();
    const int nstar = s_nstar;
    for (int p = tid; p < nstar; p += kSelThreads) {
      const int c = (int)(kColMask - (skey[P - 1 - p] & kColMask));
      svote[c] += 1;                      // columns are distinct within a draw
    }
    if (tid == 0 && n_sel) n_sel[(int64_t)d * heads * R + row] = nstar;
    __syncthreads();
  }
  for (int c = tid; c < R; c += kSelThreads) vrow[c] = (uint8_t)(svote[c] > 255 ? 255 : svote[c]);
}

hipError_t launch_select_votes(const float* energy, int32_t n_draws, int32_t heads,
                               int32_t n_blocks, uint64_t eps_fx, uint8_t* votes,
                               int32_t* n_sel, hipStream_t stream) {
  const int64_t rows = (int64_t)heads * n_blocks;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(select_votes_kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, stream,
                     energy, n_draws, heads, n_blocks, eps_fx, votes, n_sel);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row counts. One wave per row. mode 0: count mask != 0. mode 1: keep iff
// votes * rho_den >= rho_num * n_prompts, an empty row keeps its most-voted
// (lowest) column; the binarised row is written to mask_out. The count of row
// i goes to offsets[i + 1].

__global__ void __launch_bounds__(256) row_counts_kernel(
    const uint8_t* __restrict__ src, int rows, int R, int mode, int n_prompts, int rho_num,
    int rho_den, uint8_t* __restrict__ mask_out, int32_t* __restrict__ offsets) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* s = src + (int64_t)row * R;
  const int need = rho_num * n_prompts;
  int cnt = 0, best_v = -1, best_c = 0;
  for (int c = lane; c < R; c += 64) {
    const int v = s[c];
    const bool keep = mode == 0 ? v != 0 : v * rho_den >= need;
    cnt += keep;
    if (v > best_v) { best_v = v; best_c = c; }  // lane-local: first max in column order
  }
  for (int off = 32; off >= 1; off >>= 1) {
    cnt += __shfl_xor(cnt, off);
    const int ov = __shfl_xor(best_v, off), oc = __shfl_xor(best_c, off);
    if (ov > best_v || (ov == best_v && oc < best_c)) { best_v = ov; best_c = oc; }
  }
  const bool fallback = mode == 1 && cnt == 0;
  if (mode == 1) {
    uint8_t* mrow = mask_out + (int64_t)row * R;
    for (int c = lane; c < R; c += 64) {
      const int v = s[c];
      mrow[c] = (uint8_t)((v * rho_den >= need) || (fallback && c == best_c));
    }
  }
  if (lane == 0) offsets[row + 1] = fallback ? 1 : cnt;
}

hipError_t launch_row_counts(const uint8_t* src, int32_t rows, int32_t n_blocks, int mode,
                             int32_t n_prompts, int32_t rho_num, int32_t rho_den,
                             uint8_t* mask_out, int32_t* offsets, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_counts_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, src, rows,
                     n_blocks, mode, n_prompts, rho_num, rho_den, mask_out, offsets);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// In-place scan: offsets[1..rows] hold counts; afterwards offsets[i] is the
// exclusive prefix (offsets[0] = 0, offsets[rows] = nnz). One workgroup.

constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(kScanThreads) offsets_scan_kernel(int32_t* __restrict__ offsets,
                                                                    int rows) {
  __shared__ int32_t s[kScanThreads];
  const int tid = threadIdx.x;
  const int per = (rows + kScanThreads - 1) / kScanThreads;
  const int b = tid * per;
  const int e = min(b + per, rows);
  int32_t local = 0;
  for (int i = b; i < e; ++i) local += offsets[i + 1];
  s[tid] = local;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t add = tid >= off ? s[tid - off] : 0;
    __syncthreads();
    s[tid] += add;
    __syncthreads();
  }
  int32_t run = s[tid] - local;
  for (int i = b; i < e; ++i) {
    run += offsets[i + 1];
    offsets[i + 1] = run;
  }
  if (tid == 0) offsets[0] = 0;
}

hipError_t launch_offsets_scan(int32_t* offsets, int32_t rows, hipStream_t stream) {
  hipLaunchKernelGGL(offsets_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, offsets, rows);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Compaction: one wave per row writes the kept columns in ascending order.

__global__ void __launch_bounds__(256) compact_kernel(const uint8_t* __restrict__ mask, int rows,
                                                      int R, const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ indices) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* mrow = mask + (int64_t)row * R;
  int32_t base = offsets[row];
  for (int c0 = 0; c0 < R; c0 += 64) {
    const int c = c0 + lane;
    const bool keep = c < R && mrow[c] != 0;
    const uint64_t bal = __ballot(keep);
    if (keep) indices[base + __popcll(bal & ((1ull << lane) - 1ull))] = c;
    base += __popcll(bal);
  }
}

hipError_t launch_compact(const uint8_t* mask, int32_t rows, int32_t n_blocks,
                          const int32_t* offsets, int32_t* indices, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(compact_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, mask, rows,
                     n_blocks, offsets, indices);
  return hipGetLastError();
}

}  // namespace calibatt
