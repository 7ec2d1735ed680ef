// Kernel argument blocks and launchers (internal; the public interface is
// include/calibatt.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/calibatt.h"

namespace calibatt {

constexpr int kMaxHeadsPerLaunch = 256;
constexpr int kMaxMaskedRepeatBlocks = 896;  // R limit of masked repeat heads (LDS bitmaps)

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* vt;        // V^T tiles [heads][R][128 d][128 keys] (workspace)
  uint16_t* o;
  int64_t stride_head;
  int64_t stride_token;
  const int32_t* offsets;
  const int32_t* indices;
  int64_t nnz;
  float scale_log2;          // softmax scale * log2(e)
  int32_t n_tokens;
  int32_t n_blocks;
  int32_t n_rep;             // repeat heads in this launch (listed first in heads[])
  int32_t n_mrep;            // of which masked repeat heads (listed first of all)
  int32_t n_sparse;          // non-repeat heads in this launch
  int32_t rep_tiles;         // query tiles per repeat head
  int32_t n_items;           // n_rep * rep_tiles + n_sparse * n_blocks
  int32_t frames, rows, cols, anchors;
  int32_t anchor_queries;    // frames * anchors * cols
  int32_t mask_words;        // ceil(R/32): bitmap words of masked repeat tiles
  int32_t heads[kMaxHeadsPerLaunch];
};

struct VtArgs {
  const uint16_t* v;
  uint16_t* vt;
  int64_t stride_head;
  int64_t stride_token;
  int32_t heads;
  int32_t n_tokens;
  int32_t n_blocks;
};

struct EnergyArgs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t stride_head;
  int64_t stride_token;
  float* partials;           // float2 [heads][R][R*128]: (block partial sum, its reference)
  float* row_stats;          // float2 [heads][R*128]: (final reference, row sum)
  float* energy;             // [heads][R][R]
  float scale_log2;
  int32_t n_tokens;
  int32_t n_blocks;
  int32_t heads;
};

struct SimArgs {
  const float* partials;     // energy workspace: float2 [heads][R][R*128]
  const float* row_stats;    // energy workspace: float2 [heads][R*128]
  float* profiles;           // [heads][frames*rows][R]
  float* similarity;         // [heads]
  int32_t heads, n_tokens, n_blocks;
  int32_t frames, rows, cols, anchors;
};

// Error reporting of the C ABI (thread-local message, returned status).
int api_fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int api_ok();

// Checks a video grid for repeat heads and the similarity score: it covers
// n_tokens, 1 <= anchors <= rows, and every anchor row lies in the segment
// it serves.
int check_grid(const char* fn, const calibatt_grid& g, int32_t n_tokens);

hipError_t launch_v_transpose(const VtArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream);
hipError_t launch_block_energy(const EnergyArgs& a, hipStream_t stream);
hipError_t launch_spatial_similarity(const SimArgs& a, hipStream_t stream);
hipError_t launch_mfma_probe(float* sink, int64_t iters, int32_t workgroups, hipStream_t stream);

hipError_t launch_select_votes(const float* energy, int32_t n_draws, int32_t heads,
                               int32_t n_blocks, uint64_t eps_fx, uint8_t* votes,
                               int32_t* n_sel, hipStream_t stream);
// mode 0: count nonzero mask entries; mode 1: binarise votes into mask, then count.
hipError_t launch_row_counts(const uint8_t* src, int32_t rows, int32_t n_blocks, int mode,
                             int32_t n_prompts, int32_t rho_num, int32_t rho_den,
                             uint8_t* mask_out, int32_t* offsets, hipStream_t stream);
hipError_t launch_offsets_scan(int32_t* offsets, int32_t rows, hipStream_t stream);
hipError_t launch_compact(const uint8_t* mask, int32_t rows, int32_t n_blocks,
                          const int32_t* offsets, int32_t* indices, hipStream_t stream);

}  // namespace calibatt
