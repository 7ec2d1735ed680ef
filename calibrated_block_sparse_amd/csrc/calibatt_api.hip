// C ABI of libcalibatt.so: argument validation, work decomposition and
// launches. The declarations and their contracts are in include/calibatt.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "../../include/calibatt.h"
#include "kernels.h"

using namespace calibatt;

namespace calibatt {

// The calling thread's last error message, in a fixed buffer: recording
// one never allocates.
thread_local char g_last_error[512];

int api_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int api_ok() {
  g_last_error[0] = '\0';
  return CALIBATT_OK;
}

// Anchor A(m) = floor((2m+1) rows / (2k)) serves the rows y with
// floor(y k / rows) = m. A repeat head hands each anchor's output to the
// other rows of its frame, so every anchor row must lie in the segment it
// serves: floor(A(m) k / rows) == m for every m. This always holds when
// k == rows or rows >= 2k - 1 (then A(m) k / rows >= m + 1/2 - (2k-1)/(2 rows));
// for rows/2 < k < rows it holds for some geometries and fails for others
// (rows = 10, k = 9: row 1 would take row 0's output).
int check_grid(const char* fn, const calibatt_grid& g, int32_t n_tokens) {
  if (g.frames <= 0 || g.rows <= 0 || g.cols <= 0 ||
      (int64_t)g.frames * g.rows * g.cols != n_tokens)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: grid %dx%dx%d does not cover N=%d", fn, g.frames,
                    g.rows, g.cols, n_tokens);
  if (g.anchors < 1 || g.anchors > g.rows)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: anchors %d not in [1, rows=%d]", fn, g.anchors,
                    g.rows);
  for (int64_t m = 0; m < g.anchors; ++m) {
    const int64_t a = (2 * m + 1) * g.rows / (2 * (int64_t)g.anchors);
    if (a * g.anchors / g.rows != m)
      return api_fail(CALIBATT_ERR_UNSUPPORTED,
                      "%s: %d anchors in %d rows: anchor row %lld would not serve its own segment %lld",
                      fn, g.anchors, g.rows, (long long)a, (long long)m);
  }
  return CALIBATT_OK;
}

}  // namespace calibatt

namespace {

int hip_fail(hipError_t e, const char* what) {
  return api_fail(CALIBATT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shared checks of the bf16 [heads][N][128] tensor arguments.
int check_tensor_layout(const char* fn, int32_t heads, int32_t n_tokens, int32_t head_dim,
                        int64_t stride_head, int64_t stride_token) {
  if (heads < 0 || n_tokens < 0)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: heads (%d) and n_tokens (%d) must be >= 0", fn,
                heads, n_tokens);
  if (head_dim != CALIBATT_HEAD_DIM)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (only %d)", fn, head_dim,
                CALIBATT_HEAD_DIM);
  if (stride_token < head_dim || stride_head < 0 || stride_token % 8 || stride_head % 8)
    return api_fail(CALIBATT_ERR_INVALID_ARG,
                "%s: strides (head %lld, token %lld) must be multiples of 8 with token >= %d", fn,
                (long long)stride_head, (long long)stride_token, head_dim);
  // the tile copies address the 128 rows of a block with 32-bit byte
  // offsets from the block's first row
  if (stride_token > CALIBATT_MAX_STRIDE_TOKEN)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: stride_token %lld > %d", fn,
                    (long long)stride_token, CALIBATT_MAX_STRIDE_TOKEN);
  return CALIBATT_OK;
}

}  // namespace

extern "C" {

const char* calibatt_last_error(void) { return calibatt::g_last_error; }

int32_t calibatt_abi_version(void) { return 8; }


size_t calibatt_sparse_attn_fwd_workspace(int32_t heads, int32_t n_tokens) {
  if (heads <= 0 || n_tokens <= 0) return 0;
  return (size_t)heads * (size_t)ceil_div(n_tokens, CALIBATT_BLOCK) * CALIBATT_BLOCK *
         CALIBATT_HEAD_DIM * 2;
}

// Attention launches over V^T tiles already in `vt` (no validation of vt's
// contents). Shared by calibatt_sparse_attn_fwd and _fwd_vt.
static int attn_core(const char* fn, const void* q, const void* k, const void* vt, void* o,
                     int32_t heads, int32_t n_tokens, int64_t stride_head, int64_t stride_token,
                     float scale, const int32_t* kv_offsets, const int32_t* kv_indices, int64_t nnz,
                     const uint8_t* repeat_flags, const calibatt_grid* grid, hipStream_t stream) {
  if (!q || !k || !o) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null q/k/o", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(o))
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: q/k/o must be 16-byte aligned", fn);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  if (nnz < 0) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: nnz < 0", fn);

  const int32_t R = (int32_t)ceil_div(n_tokens, CALIBATT_BLOCK);
  if ((int64_t)heads * R > 0x7fffffff) return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: too many tiles", fn);
  int32_t count[3] = {0, 0, 0};  // heads with flag 0 (block-sparse), 1 (repeat), 2 (masked repeat)
  for (int32_t h = 0; h < heads; ++h) {
    const int f = repeat_flags ? repeat_flags[h] : 0;
    if (f > 2)
      return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: repeat flag %d of head %d is not 0, 1 or 2", fn, f, h);
    ++count[f];
  }
  if (count[2] > 0 && R > kMaxMaskedRepeatBlocks)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: masked repeat heads need R <= %d (R = %d)", fn,
                    kMaxMaskedRepeatBlocks, R);

  AttnArgs a;
  std::memset(&a, 0, sizeof a);
  if (count[1] > 0 || count[2] > 0) {
    if (!grid) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: repeat heads need a grid", fn);
    const int grc = check_grid(fn, *grid, n_tokens);
    if (grc) return grc;
    a.frames = grid->frames;
    a.rows = grid->rows;
    a.cols = grid->cols;
    a.anchors = grid->anchors;
    a.anchor_queries = grid->frames * grid->anchors * grid->cols;
  }
  if ((count[0] > 0 || count[2] > 0) && (!kv_offsets || (!kv_indices && nnz > 0)))
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null kept-block list", fn);

  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.vt = static_cast<const uint16_t*>(vt);
  a.o = static_cast<uint16_t*>(o);
  a.stride_head = stride_head;
  a.stride_token = stride_token;
  a.offsets = kv_offsets;
  a.indices = kv_indices;
  a.nnz = nnz;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.n_tokens = n_tokens;
  a.n_blocks = R;
  a.rep_tiles = (int32_t)ceil_div(a.anchor_queries, CALIBATT_BLOCK);

  // Launch in chunks of at most kMaxHeadsPerLaunch heads: masked repeat
  // heads, plain repeat heads (the longest tiles first), then block-sparse,
  // each kind in ascending head order. The heads of a kind are found by a
  // cursor over the flags, so the call allocates nothing on the host either.
  a.mask_words = (int32_t)ceil_div(R, 32);
  auto next_of = [&](int kind, int32_t from) {
    int32_t h = from;
    while (h < heads && (repeat_flags ? repeat_flags[h] : 0) != kind) ++h;
    return h;
  };
  int32_t hm = next_of(2, 0), hr = next_of(1, 0), hs = next_of(0, 0);
  while (hm < heads || hr < heads || hs < heads) {
    int n = 0;
    a.n_mrep = a.n_rep = a.n_sparse = 0;
    for (; n < kMaxHeadsPerLaunch && hm < heads; hm = next_of(2, hm + 1)) { a.heads[n++] = hm; ++a.n_mrep; }
    for (; n < kMaxHeadsPerLaunch && hr < heads; hr = next_of(1, hr + 1)) a.heads[n++] = hr;
    a.n_rep = n;
    for (; n < kMaxHeadsPerLaunch && hs < heads; hs = next_of(0, hs + 1)) { a.heads[n++] = hs; ++a.n_sparse; }
    const int64_t items = (int64_t)a.n_rep * a.rep_tiles + (int64_t)a.n_sparse * R;
    if (items > 0x7fffffff) return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: too many tiles", fn);
    a.n_items = (int32_t)items;
    hipError_t e = launch_attn_fwd(a, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
  }
  return api_ok();
}

static int check_workspace(const char* fn, int32_t heads, int32_t n_tokens, const void* ws,
                           size_t ws_bytes) {
  const size_t need = calibatt_sparse_attn_fwd_workspace(heads, n_tokens);
  if (!ws || ws_bytes < need)
    return api_fail(CALIBATT_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 15u)
    return api_fail(CALIBATT_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned", fn);
  return CALIBATT_OK;
}

int calibatt_prepare_vt(const void* v, int32_t heads, int32_t n_tokens, int32_t head_dim,
                        int64_t stride_head, int64_t stride_token, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const char* fn = "calibatt_prepare_vt";
  int rc = check_tensor_layout(fn, heads, n_tokens, head_dim, stride_head, stride_token);
  if (rc) return rc;
  if (heads == 0 || n_tokens == 0) return api_ok();
  rc = check_workspace(fn, heads, n_tokens, workspace, workspace_bytes);
  if (rc) return rc;
  if (!v) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null v", fn);
  if (!aligned16(v)) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: v must be 16-byte aligned", fn);
  const int32_t R = (int32_t)ceil_div(n_tokens, CALIBATT_BLOCK);
  if ((int64_t)heads * R > 0x7fffffff) return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: too many tiles", fn);
  VtArgs t;
  t.v = static_cast<const uint16_t*>(v);
  t.vt = static_cast<uint16_t*>(workspace);
  t.stride_head = stride_head;
  t.stride_token = stride_token;
  t.heads = heads;
  t.n_tokens = n_tokens;
  t.n_blocks = R;
  hipError_t e = launch_v_transpose(t, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return api_ok();
}

int calibatt_sparse_attn_fwd_vt(const void* q, const void* k, const void* vt, void* o,
                                int32_t heads, int32_t n_tokens, int32_t head_dim,
                                int64_t stride_head, int64_t stride_token, float scale,
                                const int32_t* kv_offsets, const int32_t* kv_indices, int64_t nnz,
                                const uint8_t* repeat_flags, const calibatt_grid* grid,
                                size_t vt_bytes, void* stream) {
  const char* fn = "calibatt_sparse_attn_fwd_vt";
  int rc = check_tensor_layout(fn, heads, n_tokens, head_dim, stride_head, stride_token);
  if (rc) return rc;
  if (heads == 0 || n_tokens == 0) return api_ok();
  rc = check_workspace(fn, heads, n_tokens, vt, vt_bytes);
  if (rc) return rc;
  return attn_core(fn, q, k, vt, o, heads, n_tokens, stride_head, stride_token, scale, kv_offsets,
                   kv_indices, nnz, repeat_flags, grid, static_cast<hipStream_t>(stream));
}

// Everything the full attention call needs from its arguments besides the
// tensor layout and the workspace, checked before anything is enqueued.
static int check_attn_inputs(const char* fn, const void* q, const void* k, const void* v,
                             const void* o, int32_t heads, int32_t n_tokens, float scale,
                             const int32_t* kv_offsets, const int32_t* kv_indices, int64_t nnz,
                             const uint8_t* repeat_flags, const calibatt_grid* grid) {
  if (!q || !k || !v || !o) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null q/k/v/o", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: q/k/v/o must be 16-byte aligned", fn);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  if (nnz < 0) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: nnz < 0", fn);
  bool any_rep = false, any_sparse = false;
  for (int32_t h = 0; h < heads; ++h) {
    const int f = repeat_flags ? repeat_flags[h] : 0;
    if (f > 2)
      return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: repeat flag %d of head %d is not 0, 1 or 2", fn, f, h);
    if (f == 2 && ceil_div(n_tokens, CALIBATT_BLOCK) > kMaxMaskedRepeatBlocks)
      return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: masked repeat heads need R <= %d", fn,
                      kMaxMaskedRepeatBlocks);
    (f ? any_rep : any_sparse) = true;
    if (f == 2) any_sparse = true;  // its lists are read too
  }
  if (any_rep) {
    if (!grid) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: repeat heads need a grid", fn);
    const int grc = check_grid(fn, *grid, n_tokens);
    if (grc) return grc;
  }
  if (any_sparse && (!kv_offsets || (!kv_indices && nnz > 0)))
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null kept-block list", fn);
  if ((int64_t)heads * ceil_div(n_tokens, CALIBATT_BLOCK) > 0x7fffffff)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: too many tiles", fn);
  return CALIBATT_OK;
}

int calibatt_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, int32_t heads,
                             int32_t n_tokens, int32_t head_dim, int64_t stride_head,
                             int64_t stride_token, float scale, const int32_t* kv_offsets,
                             const int32_t* kv_indices, int64_t nnz,
                             const uint8_t* repeat_flags, const calibatt_grid* grid,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "calibatt_sparse_attn_fwd";
  int rc = check_tensor_layout(fn, heads, n_tokens, head_dim, stride_head, stride_token);
  if (rc) return rc;
  if (heads == 0 || n_tokens == 0) return api_ok();
  rc = check_workspace(fn, heads, n_tokens, workspace, workspace_bytes);
  if (rc) return rc;
  // validate everything the attention needs before enqueuing the pre-pass
  rc = check_attn_inputs(fn, q, k, v, o, heads, n_tokens, scale, kv_offsets, kv_indices, nnz,
                         repeat_flags, grid);
  if (rc) return rc;
  rc = calibatt_prepare_vt(v, heads, n_tokens, head_dim, stride_head, stride_token, workspace,
                           workspace_bytes, stream);
  if (rc) return rc;
  return attn_core(fn, q, k, workspace, o, heads, n_tokens, stride_head, stride_token, scale,
                   kv_offsets, kv_indices, nnz, repeat_flags, grid, static_cast<hipStream_t>(stream));
}

size_t calibatt_block_energy_workspace(int32_t heads, int32_t n_tokens) {
  if (heads <= 0 || n_tokens <= 0) return 0;
  const size_t R = (size_t)ceil_div(n_tokens, CALIBATT_BLOCK);
  // per (head, key block, padded query row) and per (head, padded query row): two floats each
  return (size_t)2 * sizeof(float) * (size_t)heads * R * CALIBATT_BLOCK * (R + 1);
}

int calibatt_block_energy(const void* q, const void* k, float* energy, int32_t heads,
                          int32_t n_tokens, int32_t head_dim, int64_t stride_head,
                          int64_t stride_token, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const char* fn = "calibatt_block_energy";
  int rc = check_tensor_layout(fn, heads, n_tokens, head_dim, stride_head, stride_token);
  if (rc) return rc;
  if (heads == 0 || n_tokens == 0) return api_ok();
  if (!q || !k || !energy) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null q/k/energy", fn);
  if (!aligned16(q) || !aligned16(k))
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: q/k must be 16-byte aligned", fn);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  const int64_t R = ceil_div(n_tokens, CALIBATT_BLOCK);
  if (R > CALIBATT_MAX_BLOCKS)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: %lld blocks > %d", fn, (long long)R,
                CALIBATT_MAX_BLOCKS);
  if ((int64_t)heads * R > 0x7fffffff) return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: too many tiles", fn);
  // heads go in chunks of as many as the workspace holds (all at once when
  // it holds them all; the results do not depend on the chunking)
  const size_t per_head = calibatt_block_energy_workspace(1, n_tokens);
  if (!workspace || workspace_bytes < per_head)
    return api_fail(CALIBATT_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu (one head)", fn,
                    workspace_bytes, per_head);
  if (reinterpret_cast<uintptr_t>(workspace) & 15u)
    return api_fail(CALIBATT_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned", fn);
  const int32_t chunk = workspace_bytes / per_head >= (size_t)heads ? heads
                                                                     : (int32_t)(workspace_bytes / per_head);
  for (int32_t h0 = 0; h0 < heads; h0 += chunk) {
    const int32_t hc = heads - h0 < chunk ? heads - h0 : chunk;
    EnergyArgs a;
    a.q = static_cast<const uint16_t*>(q) + (int64_t)h0 * stride_head;
    a.k = static_cast<const uint16_t*>(k) + (int64_t)h0 * stride_head;
    a.stride_head = stride_head;
    a.stride_token = stride_token;
    a.partials = static_cast<float*>(workspace);
    a.row_stats = a.partials + (size_t)2 * hc * R * R * CALIBATT_BLOCK;
    a.energy = energy + (int64_t)h0 * R * R;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    a.n_tokens = n_tokens;
    a.n_blocks = (int32_t)R;
    a.heads = hc;
    hipError_t e = launch_block_energy(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
  }
  return api_ok();
}

int calibatt_spatial_similarity(const void* energy_workspace, size_t workspace_bytes,
                                int32_t heads, int32_t n_tokens, const calibatt_grid* grid,
                                float* row_profiles, float* similarity, void* stream) {
  const char* fn = "calibatt_spatial_similarity";
  if (heads < 0 || n_tokens < 0)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: heads (%d) and n_tokens (%d) must be >= 0", fn,
                    heads, n_tokens);
  if (heads == 0 || n_tokens == 0) return api_ok();
  if (!grid) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null grid", fn);
  const int grc = check_grid(fn, *grid, n_tokens);
  if (grc) return grc;
  if (grid->cols > 8192)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: %d columns > 8192", fn, grid->cols);
  const int64_t R = ceil_div(n_tokens, CALIBATT_BLOCK);
  if (R > CALIBATT_MAX_BLOCKS)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: %lld blocks > %d", fn, (long long)R,
                    CALIBATT_MAX_BLOCKS);
  if ((int64_t)heads * grid->frames * grid->rows > 0x7fffffff)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: too many spatial rows", fn);
  if (!row_profiles || !similarity)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null row_profiles/similarity", fn);
  const size_t need = calibatt_block_energy_workspace(heads, n_tokens);
  if (!energy_workspace || workspace_bytes < need)
    return api_fail(CALIBATT_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(energy_workspace) & 7u)
    return api_fail(CALIBATT_ERR_WORKSPACE, "%s: workspace must be 8-byte aligned", fn);
  SimArgs a;
  a.partials = static_cast<const float*>(energy_workspace);
  a.row_stats = a.partials + (size_t)2 * heads * R * R * CALIBATT_BLOCK;
  a.profiles = row_profiles;
  a.similarity = similarity;
  a.heads = heads;
  a.n_tokens = n_tokens;
  a.n_blocks = (int32_t)R;
  a.frames = grid->frames;
  a.rows = grid->rows;
  a.cols = grid->cols;
  a.anchors = grid->anchors;
  hipError_t e = launch_spatial_similarity(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return api_ok();
}

uint64_t calibatt_eps_fx(double t, double T, double A, double C, double k) {
  const double eps = A + (C - A) * std::exp(-k * t / T);
  const double x = std::nearbyint(eps * 1099511627776.0);  // default mode: ties to even
  if (!(x > 0.0)) return 0;
  if (x >= 18446744073709551615.0) return ~0ull;
  return (uint64_t)x;
}

int calibatt_build_mask(const float* energy, int32_t n_draws, int32_t heads, int32_t n_blocks,
                        uint64_t eps_fx, uint8_t* votes, int32_t* n_sel, void* stream) {
  const char* fn = "calibatt_build_mask";
  if (n_draws < 0 || heads < 0 || n_blocks < 0)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: negative size", fn);
  if (n_draws == 0 || heads == 0 || n_blocks == 0) return api_ok();
  if (n_blocks > CALIBATT_MAX_BLOCKS)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: %d blocks > %d", fn, n_blocks, CALIBATT_MAX_BLOCKS);
  if (!energy || !votes) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null energy/votes", fn);
  if ((int64_t)heads * n_blocks > 0x7fffffff) return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: too many rows", fn);
  hipError_t e = launch_select_votes(energy, n_draws, heads, n_blocks, eps_fx, votes, n_sel,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return api_ok();
}

static int compile_common(const char* fn, const uint8_t* src, int mode, int32_t heads,
                          int32_t n_blocks, int32_t n_prompts, int32_t rho_num, int32_t rho_den,
                          uint8_t* mask, int32_t* kv_offsets, int32_t* kv_indices,
                          int64_t* nnz_out, void* stream) {
  if (heads < 0 || n_blocks < 0) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: negative size", fn);
  const int64_t rows = (int64_t)heads * n_blocks;
  if (rows * n_blocks >= 0x7fffffffLL)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: heads*R*R must be < 2^31", fn);
  if (!kv_offsets) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null kv_offsets", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (rows == 0) {
    e = launch_offsets_scan(kv_offsets, 0, s);  // writes offsets[0] = 0
    if (e != hipSuccess) return hip_fail(e, fn);
  } else {
    if (!src || !kv_indices || (mode == 1 && !mask))
      return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null input/output", fn);
    e = launch_row_counts(src, (int32_t)rows, n_blocks, mode, n_prompts, rho_num, rho_den, mask,
                          kv_offsets, s);
    if (e == hipSuccess) e = launch_offsets_scan(kv_offsets, (int32_t)rows, s);
    if (e == hipSuccess)
      e = launch_compact(mode == 1 ? mask : src, (int32_t)rows, n_blocks, kv_offsets, kv_indices, s);
    if (e != hipSuccess) return hip_fail(e, fn);
  }
  if (nnz_out) {
    int32_t nnz = 0;
    e = hipMemcpyAsync(&nnz, kv_offsets + rows, sizeof nnz, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, fn);
    *nnz_out = nnz;
  }
  return api_ok();
}

int calibatt_finalize_mask(const uint8_t* votes, int32_t heads, int32_t n_blocks,
                           int32_t n_prompts, int32_t rho_num, int32_t rho_den, uint8_t* mask,
                           int32_t* kv_offsets, int32_t* kv_indices, int64_t* nnz_out,
                           void* stream) {
  const char* fn = "calibatt_finalize_mask";
  if (n_prompts < 1 || n_prompts > 255)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: n_prompts %d not in [1, 255]", fn, n_prompts);
  if (rho_den < 1 || rho_num < 0 || rho_num > rho_den || rho_den > (1 << 20))
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: rho %d/%d invalid", fn, rho_num, rho_den);
  return compile_common(fn, votes, 1, heads, n_blocks, n_prompts, rho_num, rho_den, mask,
                        kv_offsets, kv_indices, nnz_out, stream);
}

int calibatt_compile_skiplist(const uint8_t* mask, int32_t heads, int32_t n_blocks,
                              int32_t* kv_offsets, int32_t* kv_indices, int64_t* nnz_out,
                              void* stream) {
  return compile_common("calibatt_compile_skiplist", mask, 0, heads, n_blocks, 0, 0, 1, nullptr,
                        kv_offsets, kv_indices, nnz_out, stream);
}

int calibatt_validate_skiplist(const int32_t* kv_offsets, const int32_t* kv_indices, int64_t nnz,
                               int32_t heads, int32_t n_blocks) {
  const char* fn = "calibatt_validate_skiplist";
  if (heads < 0 || n_blocks < 0 || nnz < 0)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: negative size", fn);
  if (!kv_offsets || (nnz > 0 && !kv_indices))
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null pointer", fn);
  const int64_t rows = (int64_t)heads * n_blocks;
  if (kv_offsets[0] != 0) return api_fail(CALIBATT_ERR_BAD_SKIPLIST, "%s: offsets[0] = %d", fn, kv_offsets[0]);
  if (kv_offsets[rows] != nnz)
    return api_fail(CALIBATT_ERR_BAD_SKIPLIST, "%s: offsets[%lld] = %d != nnz %lld", fn,
                (long long)rows, kv_offsets[rows], (long long)nnz);
  // Every offset must lie in [0, nnz] before any index is read: offsets such
  // as [0, R, 0] pass the end checks but would send row 0 past the array.
  for (int64_t r = 1; r < rows; ++r) {
    if (kv_offsets[r] < 0 || kv_offsets[r] > nnz)
      return api_fail(CALIBATT_ERR_BAD_SKIPLIST, "%s: offsets[%lld] = %d outside [0, nnz = %lld]",
                      fn, (long long)r, kv_offsets[r], (long long)nnz);
  }
  for (int64_t r = 0; r < rows; ++r) {
    const int32_t b = kv_offsets[r], e = kv_offsets[r + 1];
    if (e < b) return api_fail(CALIBATT_ERR_BAD_SKIPLIST, "%s: row %lld: offsets decrease", fn, (long long)r);
    if (e - b > n_blocks)
      return api_fail(CALIBATT_ERR_BAD_SKIPLIST, "%s: row %lld: %d entries > R", fn, (long long)r, e - b);
    for (int32_t i = b; i < e; ++i) {
      const int32_t c = kv_indices[i];
      if (c < 0 || c >= n_blocks)
        return api_fail(CALIBATT_ERR_BAD_SKIPLIST, "%s: row %lld: index %d out of [0, %d)", fn,
                    (long long)r, c, n_blocks);
      if (i > b && c <= kv_indices[i - 1])
        return api_fail(CALIBATT_ERR_BAD_SKIPLIST, "%s: row %lld: indices not ascending", fn, (long long)r);
    }
  }
  return api_ok();
}

int calibatt_mfma_rate_probe(float* sink, int64_t iters, int32_t workgroups, void* stream) {
  if (!sink) return api_fail(CALIBATT_ERR_INVALID_ARG, "calibatt_mfma_rate_probe: sink is NULL");
  if (iters < 0 || workgroups < 0)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "calibatt_mfma_rate_probe: iters (%lld) and workgroups (%d) must be >= 0",
                (long long)iters, workgroups);
  if (workgroups == 0) return api_ok();
  const hipError_t e = launch_mfma_probe(sink, iters, workgroups, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "calibatt_mfma_rate_probe");
  return api_ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Attention without allocation or workspace (calibatt_sparse_attn_fwd_noalloc).
//
// The V^T tiles go to `scratch`, a file-scope device array of
// CALIBATT_NOALLOC_SCRATCH_BYTES that every device the library runs on holds
// for the life of the process. In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and only that
// address is ever handed to a kernel.

static __device__ __align__(256) uint8_t scratch[CALIBATT_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_addr;  // device -> its copy of `scratch`

// Device address of `scratch` on the device `stream` belongs to.
int scratch_address(const char* fn, hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, fn);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  const auto it = g_scratch_addr.find(dev);
  if (it != g_scratch_addr.end()) {
    *out = it->second;
    return CALIBATT_OK;
  }
  int cur = -1;
  if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_fail(e, fn);
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, fn);
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
  if (e != hipSuccess) return hip_fail(e, fn);
  if (back != hipSuccess) return hip_fail(back, fn);
  if (!p) return api_fail(CALIBATT_ERR_HIP, "%s: no device address for the scratch array", fn);
  g_scratch_addr.emplace(dev, p);
  *out = p;
  return CALIBATT_OK;
}

}  // namespace

extern "C" int calibatt_sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                                int32_t heads, int32_t n_tokens, int32_t head_dim,
                                                int64_t stride_head, int64_t stride_token, float scale,
                                                const int32_t* kv_offsets, const int32_t* kv_indices,
                                                int64_t nnz, const uint8_t* repeat_flags,
                                                const calibatt_grid* grid, void* stream) {
  const char* fn = "calibatt_sparse_attn_fwd_noalloc";
  int rc = check_tensor_layout(fn, heads, n_tokens, head_dim, stride_head, stride_token);
  if (rc) return rc;
  if (heads == 0 || n_tokens == 0) return api_ok();
  const int64_t R = ceil_div(n_tokens, CALIBATT_BLOCK);
  constexpr int64_t kTile = (int64_t)CALIBATT_BLOCK * CALIBATT_HEAD_DIM * 2;
  constexpr int64_t kMaxTiles = (int64_t)CALIBATT_NOALLOC_SCRATCH_BYTES / kTile;
  if (R > kMaxTiles)
    return api_fail(CALIBATT_ERR_UNSUPPORTED,
                    "%s: N = %d needs %lld V^T tiles per head; the %d-byte scratch holds %lld "
                    "(N <= %lld)", fn, n_tokens, (long long)R, CALIBATT_NOALLOC_SCRATCH_BYTES,
                    (long long)kMaxTiles, (long long)(kMaxTiles * CALIBATT_BLOCK));
  rc = check_attn_inputs(fn, q, k, v, o, heads, n_tokens, scale, kv_offsets, kv_indices, nnz,
                         repeat_flags, grid);
  if (rc) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  void* vt = nullptr;
  if ((rc = scratch_address(fn, st, &vt))) return rc;
  // heads in equal chunks whose V^T tiles fit the scratch; each chunk's
  // pre-pass and attention run back to back on the stream
  const int64_t fit = kMaxTiles / R;
  const int64_t chunks = ceil_div(heads, fit);
  const int32_t per = (int32_t)ceil_div(heads, chunks);
  for (int32_t h0 = 0; h0 < heads; h0 += per) {
    const int32_t hc = heads - h0 < per ? heads - h0 : per;
    const int64_t off = (int64_t)h0 * stride_head;
    VtArgs t;
    t.v = static_cast<const uint16_t*>(v) + off;
    t.vt = static_cast<uint16_t*>(vt);
    t.stride_head = stride_head;
    t.stride_token = stride_token;
    t.heads = hc;
    t.n_tokens = n_tokens;
    t.n_blocks = (int32_t)R;
    const hipError_t e = launch_v_transpose(t, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    rc = attn_core(fn, static_cast<const uint16_t*>(q) + off, static_cast<const uint16_t*>(k) + off,
                   vt, static_cast<uint16_t*>(o) + off, hc, n_tokens, stride_head, stride_token,
                   scale, kv_offsets ? kv_offsets + (int64_t)h0 * R : nullptr, kv_indices, nnz,
                   repeat_flags ? repeat_flags + h0 : nullptr, grid, st);
    if (rc) return rc;
  }
  return api_ok();
}
