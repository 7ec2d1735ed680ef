/* A plain C user of libcalibatt: only include/calibatt.h and the shared
 * library, no Python or torch. Exercises the host-side entry points (no GPU
 * needed): version, eps fixed point, list validation, argument errors that
 * are reported before anything is launched, and a mask-bank round trip.
 * Prints "ok" and exits 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "calibatt.h"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s (last error: %s)\n",  \
              __LINE__, #cond, calibatt_last_error());                     \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

int main(int argc, char** argv) {
  const char* bank_path = argc > 1 ? argv[1] : "consumer_bank.cbsm";

  CHECK(calibatt_abi_version() >= 7);

  /* eps(t) = A + (C - A) exp(-k t / T) as rint(eps * 2^40): eps(0) = C */
  CHECK(calibatt_eps_fx(0.0, 50.0, 0.84, 0.99, 5.0) == 1088516511498ull);

  /* two heads, N = 300 tokens (R = 3 blocks): head 0 keeps the diagonal,
   * head 1 keeps everything in row 0 and nothing in rows 1 and 2 */
  const int32_t H = 2, N = 300, R = 3;
  int32_t off[7] = {0, 1, 2, 3, 6, 6, 6};
  int32_t idx[6] = {0, 1, 2, 0, 1, 2};
  CHECK(calibatt_validate_skiplist(off, idx, 6, H, R) == CALIBATT_OK);
  int32_t bad_idx[6] = {0, 1, 2, 1, 0, 2}; /* not ascending in row (1, 0) */
  CHECK(calibatt_validate_skiplist(off, bad_idx, 6, H, R) == CALIBATT_ERR_BAD_SKIPLIST);

  /* argument errors come back before any device work: head_dim 64 */
  CHECK(calibatt_sparse_attn_fwd((void*)4096, (void*)4096, (void*)4096, (void*)4096, H, N, 64,
                                 (int64_t)N * 128, 128, 0.1f, off, idx, 6, NULL, NULL,
                                 (void*)4096, calibatt_sparse_attn_fwd_workspace(H, N),
                                 NULL) == CALIBATT_ERR_UNSUPPORTED);
  CHECK(strstr(calibatt_last_error(), "head_dim") != NULL);
  CHECK(calibatt_sparse_attn_fwd_workspace(H, N) == (size_t)H * R * 128 * 128 * 2);

  /* a one-step, two-layer bank: layer 0 -> entry 0, layer 1 -> entry 1
   * (entry 1 marks head 1 as a repeat head on a 3 x 10 x 10 grid) */
  int32_t off1[7] = {0, 3, 6, 9, 10, 11, 12};
  int32_t idx1[12] = {0, 1, 2, 0, 1, 2, 0, 1, 2, 0, 1, 2};
  const uint8_t flags1[2] = {0, 1};
  const int32_t entry_of[2] = {0, 1};
  const uint8_t* flags[2] = {NULL, flags1};
  const int32_t* offs[2] = {off, off1};
  const int32_t* idxs[2] = {idx, idx1};
  const calibatt_grid grid = {3, 10, 10, 5};
  CHECK(calibatt_bank_write(bank_path, 1, 2, H, N, &grid, 2, entry_of, flags, offs, idxs) ==
        CALIBATT_OK);
  calibatt_bank* bank = NULL;
  CHECK(calibatt_bank_open(bank_path, &bank) == CALIBATT_OK && bank != NULL);
  if (bank) {
    calibatt_bank_info info;
    CHECK(calibatt_bank_get_info(bank, &info) == CALIBATT_OK);
    CHECK(info.steps == 1 && info.layers == 2 && info.heads == H && info.n_tokens == N);
    CHECK(info.n_blocks == R && info.n_entries == 2 && info.total_nnz == 18);
    CHECK(info.grid.frames == 3 && info.grid.anchors == 5);
    calibatt_bank_entry e;
    CHECK(calibatt_bank_lookup(bank, 0, 1, 0, &e) == CALIBATT_OK);
    CHECK(e.entry == 1 && e.nnz == 12 && e.repeat_flags[1] == 1 && e.repeat_flags[0] == 0);
    CHECK(memcmp(e.kv_offsets, off1, sizeof off1) == 0 && memcmp(e.kv_indices, idx1, sizeof idx1) == 0);
    CHECK(calibatt_bank_lookup(bank, 0, 0, 0, &e) == CALIBATT_OK);
    CHECK(e.entry == 0 && e.nnz == 6 && memcmp(e.kv_indices, idx, sizeof idx) == 0);
    CHECK(calibatt_bank_lookup(bank, 1, 0, 0, &e) == CALIBATT_ERR_INVALID_ARG);
    calibatt_bank_close(bank);
  }
  calibatt_bank_close(NULL);

  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
