/*
 * calibatt.h - C ABI of the MI355X (gfx950) calibrated block-sparse attention
 * library (libcalibatt.so).
 *
 * The method (CalibAtt) is described on the page "让视频生成快 1.58 倍，却不改一行
 * 模型代码：CalibAtt 的"注意力考古学"" (zhichai.net), cited here as [CalibAtt blog],
 * and in the abstract of "Accelerating Text-to-Video Generation with
 * Calibrated Sparse Attention", cited as [abstract].
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Block size B = 128 tokens and head dimension D = 128 are fixed
 *   ([CalibAtt blog] §二 observation 1). R = ceil(N / 128) blocks per
 *   sequence; when N is not a multiple of 128 the last block is ragged: keys
 *   at or past N take no part in any softmax and query rows past N are
 *   never written.
 * - Tensors are bf16 (raw 16-bit storage, passed as void*), laid out as
 *   [heads][N][D] with element strides stride_head and stride_token; D is
 *   contiguous. Base pointers must be 16-byte aligned and both strides
 *   multiples of 8 elements; stride_token may not exceed
 *   CALIBATT_MAX_STRIDE_TOKEN (CALIBATT_ERR_UNSUPPORTED). Batch is folded
 *   into heads.
 * - Every pointer named "device" is device memory owned by the caller. The
 *   library allocates no device memory and keeps no state between calls
 *   except the thread-local error string, the host memory of a mask bank
 *   handle (calibatt_bank_open .. calibatt_bank_close) and the scratch of
 *   calibatt_sparse_attn_fwd_noalloc: a static device array of
 *   CALIBATT_NOALLOC_SCRATCH_BYTES that each device holds from the
 *   library's load to the end of the process, and its device address,
 *   looked up once per device.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *   and is asynchronous unless an entry point says otherwise. Argument
 *   errors are reported before anything is enqueued; launch failures return
 *   CALIBATT_ERR_HIP. Nothing throws across this interface.
 * - Calls that overlap on one device and write the same memory race.
 */
#ifndef CALIBATT_H
#define CALIBATT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CALIBATT_OK = 0,
  CALIBATT_ERR_INVALID_ARG = -1,  /* null pointer, bad size, bad alignment */
  CALIBATT_ERR_UNSUPPORTED = -2,  /* D != 128, sizes beyond the limits below */
  CALIBATT_ERR_BAD_SKIPLIST = -3, /* malformed kept-block list (validators) */
  CALIBATT_ERR_WORKSPACE = -4,    /* workspace missing or too small */
  CALIBATT_ERR_HIP = -5,          /* a HIP runtime call or launch failed */
  CALIBATT_ERR_IO = -6            /* mask bank file missing, unreadable or corrupt */
};

#define CALIBATT_BLOCK 128
#define CALIBATT_HEAD_DIM 128
#define CALIBATT_MAX_BLOCKS 2047 /* R limit of the selection kernels */
#define CALIBATT_MAX_STRIDE_TOKEN 8388608 /* elements between tokens (2^23) */
#define CALIBATT_NOALLOC_SCRATCH_BYTES 268435456 /* device scratch of _noalloc (256 MiB per device) */

/* Latent video grid of a sequence: token n = f*rows*cols + y*cols + x
 * (frame-major, row-major inside a frame; [CalibAtt blog] §六). `anchors`
 * is k, the number of anchor rows a repeat head computes per frame. */
typedef struct calibatt_grid {
  int32_t frames;
  int32_t rows;
  int32_t cols;
  int32_t anchors;
} calibatt_grid;

/* Message of this thread's last call that returned a status: its error, or
 * "" when it succeeded. The buffer is per thread and stays valid until the
 * thread's next such call. */
const char* calibatt_last_error(void);

/* Interface version (increments on any change of the declared interface:
 * entry points, their arguments, structures, codes or contracts). Version 2
 * added the workspace of calibatt_sparse_attn_fwd, version 3 its two halves
 * calibatt_prepare_vt and calibatt_sparse_attn_fwd_vt, version 4 the
 * single-pass energy workspace and calibatt_mfma_rate_probe, version 5 the
 * mask bank (calibatt_bank_*) and CALIBATT_ERR_IO, version 6
 * calibatt_spatial_similarity, version 7 masked repeat heads (flag 2),
 * version 8 calibatt_sparse_attn_fwd_noalloc, energy workspaces down to one
 * head (heads then run in chunks) and the per-anchor grid rule. */
int32_t calibatt_abi_version(void);

/*
 * Block-sparse attention forward with optional repeat heads.
 *
 * Non-repeat head h: for each query block r, attend only to the key blocks
 * kv_indices[kv_offsets[h*R + r] .. kv_offsets[h*R + r + 1]) and skip all
 * others ([CalibAtt blog] §三 online inference: a precomputed skip list tells
 * the kernel which blocks to compute; [abstract]: selected connections are
 * computed densely, unselected ones skipped). The result equals softmax
 * attention with the logits of skipped blocks at -inf; a query block with an
 * empty list gets zeros. Lists should be ascending; the order only affects
 * rounding.
 *
 * Repeat head h (repeat_flags[h] == 1; [CalibAtt blog] §二 observation 4,
 * §三): only the `anchors` anchor rows of every frame are computed, densely
 * over all N keys, and each output token (f, y, x) receives the output of
 * query (f, a(y), x), where A(m) = floor((2m+1)*rows / (2*anchors)) and
 * a(y) = A(floor(y*anchors / rows)). Its CSR rows are ignored.
 *
 * Masked repeat head (repeat_flags[h] == 2; a variant, the pages name no
 * mask for repeat heads): as a repeat head, but anchor query n attends only
 * to the key blocks that its block-row floor(n / 128) keeps in the head's
 * CSR lists (zeros for a row that keeps nothing). Needs R <= 896.
 *
 *   q, k, v      device bf16 [heads][N][128] (strides as above), inputs
 *   o            device bf16, same layout and strides, output
 *   scale        softmax scale (> 0), e.g. 1/sqrt(128)
 *   kv_offsets   device int32 [heads*R + 1], non-decreasing, first 0
 *   kv_indices   device int32 [nnz], key block indices in [0, R)
 *   nnz          number of entries of kv_indices. Ranges are clamped to
 *                [0, nnz) and indices outside [0, R) are skipped, so a
 *                malformed list cannot read out of bounds; its result is
 *                unspecified (check lists with calibatt_validate_skiplist).
 *   repeat_flags host uint8 [heads] or NULL (no repeat heads): 0 block
 *                sparse, 1 repeat, 2 masked repeat; other values give
 *                CALIBATT_ERR_INVALID_ARG
 *   grid         host pointer, required iff a repeat flag is set:
 *                frames*rows*cols == N and 1 <= anchors <= rows
 *                (CALIBATT_ERR_INVALID_ARG otherwise); every anchor row
 *                must lie in the segment it serves, floor(A(m)*anchors/rows)
 *                == m, so that it keeps its own output (always true when
 *                anchors == rows or rows >= 2*anchors - 1;
 *                CALIBATT_ERR_UNSUPPORTED otherwise)
 *   workspace    device, 16-byte aligned, at least
 *                calibatt_sparse_attn_fwd_workspace(heads, N) bytes; the call
 *                first writes V there as [heads][R][128 d][128 keys] tiles
 *                (transposed per key block, zero past N) and the attention
 *                reads V only from there. Its contents after the call are
 *                unspecified; calls sharing one workspace must not overlap.
 * kv_offsets / kv_indices may be NULL when every head has flag 1.
 * heads == 0 or N == 0 is a no-op. A workspace that is missing, too small or
 * misaligned gives CALIBATT_ERR_WORKSPACE.
 * The call enqueues kernel launches only (no memset, copy or allocation), so
 * it can be captured in a HIP graph on `stream`. repeat_flags, grid, heads
 * and N are read on the host at capture time and fixed in the graph; the
 * device buffers are read at every replay.
 */
int calibatt_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o,
                             int32_t heads, int32_t n_tokens, int32_t head_dim,
                             int64_t stride_head, int64_t stride_token, float scale,
                             const int32_t* kv_offsets, const int32_t* kv_indices,
                             int64_t nnz, const uint8_t* repeat_flags,
                             const calibatt_grid* grid, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace calibatt_sparse_attn_fwd needs: heads * R *
 * 128 * 128 * 2 (one bf16 V^T tile per head and key block). 0 when heads or
 * n_tokens is not positive.
 */
size_t calibatt_sparse_attn_fwd_workspace(int32_t heads, int32_t n_tokens);

/*
 * First half of calibatt_sparse_attn_fwd: writes the V^T tiles of v
 * ([heads][N][128] bf16, strides as above) into workspace (layout and size
 * as described there). Enqueued on `stream`; errors as for the full call.
 */
int calibatt_prepare_vt(const void* v, int32_t heads, int32_t n_tokens, int32_t head_dim,
                        int64_t stride_head, int64_t stride_token, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Second half of calibatt_sparse_attn_fwd: the attention with V taken from
 * vt, which calibatt_prepare_vt filled for the same heads and N (its
 * contents are not checked). Arguments otherwise as for the full call; the
 * results are identical bit for bit. For callers that prepare V^T on another
 * stream or reuse it for several query sets.
 */
int calibatt_sparse_attn_fwd_vt(const void* q, const void* k, const void* vt, void* o,
                                int32_t heads, int32_t n_tokens, int32_t head_dim,
                                int64_t stride_head, int64_t stride_token, float scale,
                                const int32_t* kv_offsets, const int32_t* kv_indices,
                                int64_t nnz, const uint8_t* repeat_flags,
                                const calibatt_grid* grid, size_t vt_bytes, void* stream);

/*
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments and results as calibatt_sparse_attn_fwd (bit
 * for bit) without workspace / workspace_bytes. The V^T tiles go to a
 * device array inside the library of CALIBATT_NOALLOC_SCRATCH_BYTES, which
 * each device the library runs on holds until the process ends (its address
 * is looked up on the first call on a device; no allocation is made by this
 * call). Heads are processed in equal chunks whose tiles fit it (at most
 * floor(8192 / R) heads per chunk: one V^T pre-pass and one attention
 * launch per chunk), so N may not exceed 8192 * 128 = 1,048,576 tokens
 * (CALIBATT_ERR_UNSUPPORTED beyond). Every call on a device shares that
 * device's array: calls that overlap on one device (on different streams,
 * or from several threads) race and give wrong results; nothing in the
 * array needs to start at any value. Capturable in a HIP graph like the
 * full call (kernel launches only) once a first call on the device has
 * looked up the array's address.
 */
int calibatt_sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                     int32_t heads, int32_t n_tokens, int32_t head_dim,
                                     int64_t stride_head, int64_t stride_token, float scale,
                                     const int32_t* kv_offsets, const int32_t* kv_indices,
                                     int64_t nnz, const uint8_t* repeat_flags,
                                     const calibatt_grid* grid, void* stream);

/*
 * Bytes of device workspace calibatt_block_energy needs: 8 * heads * R*128 *
 * (R + 1) -- a (partial sum, reference) pair of fp32 per head, key block and
 * padded query row, and a (reference, row sum) pair per head and padded
 * query row (2.69 GB for 40 heads at N = 32760).
 */
size_t calibatt_block_energy_workspace(int32_t heads, int32_t n_tokens);

/*
 * Block energy of the post-softmax attention ([CalibAtt blog] §三 offline
 * calibration, steps 1-2): with P = softmax(scale * Q K^T) over all N keys,
 *   energy[h][r][c] = (1/|I_r|) * sum_{i in I_r} sum_{j in J_c} P_ij,
 * where I_r, J_c are the query / key tokens of blocks r, c (|I_r| = 128
 * except on a ragged last block-row, so every block-row sums to one).
 *
 *   q, k       device bf16 [heads][N][128], strides as above
 *   energy     device fp32 [heads][R][R], output (dense, row-major)
 *   workspace  device, 16-byte aligned, at least
 *              calibatt_block_energy_workspace(1, N) bytes. Heads are
 *              processed in chunks of as many as it holds
 *              (workspace_bytes / calibatt_block_energy_workspace(1, N),
 *              all of them when it holds calibatt_block_energy_workspace(
 *              heads, N)); the energies do not depend on the chunking. Only
 *              a workspace that held every head can be passed on to
 *              calibatt_spatial_similarity.
 */
int calibatt_block_energy(const void* q, const void* k, float* energy,
                          int32_t heads, int32_t n_tokens, int32_t head_dim,
                          int64_t stride_head, int64_t stride_token, float scale,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Spatial similarity score of each head ([CalibAtt blog] §二 observation 4:
 * the spatial rows of a frame attend alike; §三: a score s per (t, l, h), a
 * head above gamma = 0.87 computes only k anchor rows per frame). The pages
 * give no formula; the reading implemented:
 *   profile of spatial row (f, y): rho[c] = (1/cols) * sum over the row's
 *     cols query tokens i of sum_{j in J_c} P_ij  (P as for the energy);
 *   s[h] = mean over frames f and non-anchor rows y of the cosine of
 *     rho_{f,y} and rho_{f,a(y)}, anchors A(m) = floor((2m+1) rows / (2k)),
 *     a(y) = A(floor(y k / rows)) (as for repeat heads); 1 when every row is
 *     an anchor.
 * It reads the partial sums calibatt_block_energy leaves in its workspace:
 * call it after calibatt_block_energy for the same q, k, heads and N on the
 * same stream, with that workspace, before the workspace is reused (one
 * Q K^T pass serves both). Averaging over prompts and the comparison with
 * gamma are the caller's.
 *
 *   energy_workspace  device, as filled by calibatt_block_energy
 *   grid              frames*rows*cols == N, 1 <= anchors <= rows, cols <= 8192,
 *                     every anchor row in the segment it serves (as for
 *                     calibatt_sparse_attn_fwd)
 *   row_profiles      device fp32 [heads][frames*rows][R], output
 *   similarity        device fp32 [heads], output
 */
int calibatt_spatial_similarity(const void* energy_workspace, size_t workspace_bytes,
                                int32_t heads, int32_t n_tokens, const calibatt_grid* grid,
                                float* row_profiles, float* similarity, void* stream);

/*
 * Threshold eps(t) = A + (C - A) * exp(-k * t / T) ([CalibAtt blog] §三)
 * as an integer multiple of 2^-40, rounded to nearest (ties to even).
 * Host function, synchronous.
 */
uint64_t calibatt_eps_fx(double t, double T, double A, double C, double k);

/*
 * Greedy selection and vote accumulation ([CalibAtt blog] §三 offline
 * calibration step 3 and the mean over prompts). For every draw p, head h
 * and block-row r: energies are rounded to multiples of 2^-40 (nearest,
 * ties to even), ordered by energy descending and column ascending, and the
 * shortest prefix whose integer sum reaches eps_fx (>=) is selected (the
 * whole row if none does). votes[h][r][c] is incremented by one for every
 * selected block, saturating at 255.
 *
 *   energy   device fp32 [n_draws][heads][R][R], input
 *   eps_fx   threshold in units of 2^-40 (see calibatt_eps_fx)
 *   votes    device uint8 [heads][R][R], read and updated in place
 *   n_sel    device int32 [n_draws][heads][R] (selected count n*) or NULL
 * 1 <= R <= CALIBATT_MAX_BLOCKS.
 */
int calibatt_build_mask(const float* energy, int32_t n_draws, int32_t heads,
                        int32_t n_blocks, uint64_t eps_fx, uint8_t* votes,
                        int32_t* n_sel, void* stream);

/*
 * Binarise averaged votes and compile kept-block lists ([CalibAtt blog] §三:
 * M_bar = votes / |D| binarised at rho; §三 online inference: static skip
 * list per (timestep, layer, head)). Keeps (r, c) iff
 * votes * rho_den >= rho_num * n_prompts; a block-row left empty keeps its
 * most-voted column (lowest index on ties). Then compiles as
 * calibatt_compile_skiplist.
 *
 *   votes       device uint8 [heads][R][R]
 *   n_prompts   |D|, 1..255; rho = rho_num / rho_den with 0 <= rho_num <= rho_den, rho_den >= 1
 *   mask        device uint8 [heads][R][R], output (0/1)
 *   kv_offsets  device int32 [heads*R + 1], output
 *   kv_indices  device int32, capacity heads*R*R, output
 *   nnz_out     host int64* or NULL. When non-NULL the call waits for the
 *               stream and stores the number of kept blocks.
 */
int calibatt_finalize_mask(const uint8_t* votes, int32_t heads, int32_t n_blocks,
                           int32_t n_prompts, int32_t rho_num, int32_t rho_den,
                           uint8_t* mask, int32_t* kv_offsets, int32_t* kv_indices,
                           int64_t* nnz_out, void* stream);

/*
 * Compile a block mask into per-query-block kept lists (CSR): row h*R + r
 * lists the columns c with mask[h][r][c] != 0 in ascending order.
 *
 *   mask        device uint8 [heads][R][R]
 *   kv_offsets  device int32 [heads*R + 1], output
 *   kv_indices  device int32, capacity heads*R*R, output
 *   nnz_out     as for calibatt_finalize_mask
 * heads*R*R must be below 2^31.
 */
int calibatt_compile_skiplist(const uint8_t* mask, int32_t heads, int32_t n_blocks,
                              int32_t* kv_offsets, int32_t* kv_indices,
                              int64_t* nnz_out, void* stream);

/*
 * Check a kept-block list held in HOST memory: offsets[0] == 0,
 * non-decreasing, offsets[heads*R] == nnz, every index in [0, R) and
 * strictly ascending within a row. Returns CALIBATT_OK or
 * CALIBATT_ERR_BAD_SKIPLIST (message names the first offending row).
 * Synchronous, touches no device.
 */
int calibatt_validate_skiplist(const int32_t* kv_offsets, const int32_t* kv_indices,
                               int64_t nnz, int32_t heads, int32_t n_blocks);

/*
 * Mask bank ([CalibAtt blog] §一: calibration compiles one static mask per
 * (timestep, layer, head); §三 online inference: each attention call fetches
 * the kept-block list or repeat flag of its (t, l, h) from a table, making
 * no decision at run time). A bank holds, for T timesteps x L layers, the
 * index of an entry; an entry is what one attention call over H heads needs:
 * repeat flags and kept-block lists (CSR as for calibatt_sparse_attn_fwd).
 * Several (t, l) may share an entry.
 *
 * File layout (little-endian, version 1):
 *   [0, 128)      header: char magic[8] = "CBSMBNK1"; u32 version = 1;
 *                 u32 header bytes = 128; i32 steps T, layers L, heads H,
 *                 n_tokens N, n_blocks R = ceil(N/128), frames, rows, cols,
 *                 anchors (all four 0 when the bank has no grid),
 *                 n_entries E; i64 table offset; i64 file bytes;
 *                 u64 FNV-1a-64 of bytes [128, file bytes); zeros to 128.
 *   [128, ...)    i32 entry[T][L]
 *   table         E x { i64 payload offset, i64 nnz, u64 FNV-1a-64 of the payload }
 *   payloads      each at a multiple of 256 bytes: u8 repeat_flags[H]
 *                 (0, 1 or 2), zeros to a multiple of 4, i32 kv_offsets[H*R + 1],
 *                 i32 kv_indices[nnz]; zeros to the next 256 bytes.
 * The file ends at the end of the last padded payload.
 */
typedef struct calibatt_bank calibatt_bank; /* opaque host object */

typedef struct calibatt_bank_info {
  int32_t steps, layers, heads, n_tokens, n_blocks, n_entries;
  calibatt_grid grid;   /* all zero when the bank has no grid */
  int64_t total_nnz;    /* sum of nnz over entries */
  size_t device_bytes;  /* size of the buffer calibatt_bank_upload needs */
} calibatt_bank_info;

typedef struct calibatt_bank_entry {
  int32_t entry;               /* entry index */
  const uint8_t* repeat_flags; /* host, [H]; valid until calibatt_bank_close */
  const int32_t* kv_offsets;   /* [H*R + 1], host or device (see lookup) */
  const int32_t* kv_indices;   /* [nnz] */
  int64_t nnz;
} calibatt_bank_entry;

/*
 * Write a bank file (synchronous host I/O; written to path + ".tmp" and
 * renamed over path). entry_of: host int32 [steps*layers], values in
 * [0, n_entries). Per entry e (host arrays): repeat_flags[e] uint8 [heads]
 * or NULL (no repeat head; repeat_flags itself may be NULL), kv_offsets[e]
 * int32 [heads*R + 1], kv_indices[e] int32 [kv_offsets[e][heads*R]]. Lists
 * must pass calibatt_validate_skiplist (else CALIBATT_ERR_BAD_SKIPLIST);
 * flags must be 0, 1 or 2 (as for calibatt_sparse_attn_fwd), and any
 * repeat flag needs a grid covering n_tokens (anchor rules as for
 * calibatt_sparse_attn_fwd).
 * I/O failures give CALIBATT_ERR_IO.
 */
int calibatt_bank_write(const char* path, int32_t steps, int32_t layers, int32_t heads,
                        int32_t n_tokens, const calibatt_grid* grid, int32_t n_entries,
                        const int32_t* entry_of, const uint8_t* const* repeat_flags,
                        const int32_t* const* kv_offsets, const int32_t* const* kv_indices);

/*
 * Read and check a bank file (magic, version, sizes, both checksums, every
 * list and flag); on success *out is a new handle owning the file's bytes in
 * host memory. Corrupt or unreadable files give CALIBATT_ERR_IO, malformed
 * lists CALIBATT_ERR_BAD_SKIPLIST; *out is then NULL.
 */
int calibatt_bank_open(const char* path, calibatt_bank** out);

/* Free a handle (NULL is ignored). Device buffers it was uploaded to stay the caller's. */
void calibatt_bank_close(calibatt_bank* bank);

int calibatt_bank_get_info(const calibatt_bank* bank, calibatt_bank_info* out);

/*
 * Copy every entry's lists into `device` (caller-owned, 256-byte aligned, at
 * least info.device_bytes) with an asynchronous copy on `stream`, and
 * remember it for lookups with on_device = 1. The buffer must outlive those
 * lookups' use; uploading again rebinds the handle to the new buffer.
 */
int calibatt_bank_upload(calibatt_bank* bank, void* device, size_t bytes, void* stream);

/*
 * The entry of timestep t and layer l: O(1), no I/O, no device work.
 * on_device = 0 returns host pointers into the handle; 1 returns pointers
 * into the uploaded buffer (CALIBATT_ERR_INVALID_ARG if none). repeat_flags
 * is always host memory, as calibatt_sparse_attn_fwd takes it.
 */
int calibatt_bank_lookup(const calibatt_bank* bank, int32_t t, int32_t l, int32_t on_device,
                         calibatt_bank_entry* out);

/* ===========================================================================
 * Diagnostics (not part of the method; no page defines them)
 * ===========================================================================
 */

/*
 * Matrix-core rate probe: runs `workgroups` workgroups of four
 * waves, each wave issuing iters x 8 independent bf16 32x32x16 MFMAs with
 * register operands (32768 FLOP each), i.e.
 *   workgroups * 4 * iters * 8 * 32768 FLOP,
 * so that timing it on `stream` gives the matrix-core rate the device
 * sustains under pure MFMA load. sink: device fp32[1], practically never
 * written. Returns CALIBATT_ERR_INVALID_ARG for a NULL sink or negative
 * sizes.
 */
int calibatt_mfma_rate_probe(float* sink, int64_t iters, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CALIBATT_H */
