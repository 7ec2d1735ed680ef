// Mask bank: the static kept-block lists and repeat flags of every
// (timestep, layer, head), written once after calibration and looked up per
// attention call (zhichai.net article on CalibAtt, §一: calibration compiles
// a static mask per (t, l, h); §三 online inference: each call fetches the
// mask or repeat flag of its (t, l, h), no decision is made at run time).
//
// Host code only. The on-disk layout is documented in include/calibatt.h.
// A bank is read whole into host memory, every entry is checked (checksum,
// list structure, flags, grid), and calibatt_bank_upload copies the payloads
// into one caller-owned device buffer laid out exactly as in the file, so a
// lookup is two array reads and pointer arithmetic.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/calibatt.h"
#include "kernels.h"

using calibatt::api_fail;
using calibatt::api_ok;
using calibatt::check_grid;

namespace {

constexpr char kMagic[8] = {'C', 'B', 'S', 'M', 'B', 'N', 'K', '1'};
constexpr uint32_t kVersion = 1;
constexpr int64_t kHeaderBytes = 128;
constexpr int64_t kPayloadAlign = 256;
constexpr int64_t kTableEntryBytes = 24;

// 64-bit FNV-1a (Fowler, Noll, Vo): offset basis 0xcbf29ce484222325, prime
// 0x100000001b3, one xor-then-multiply per byte.
uint64_t fnv1a64(const uint8_t* p, size_t n) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

struct Header {
  char magic[8];
  uint32_t version;
  uint32_t header_bytes;
  int32_t steps, layers, heads, n_tokens, n_blocks;
  int32_t frames, rows, cols, anchors;
  int32_t n_entries;
  int64_t table_offset;
  int64_t file_bytes;
  uint64_t checksum;  // FNV-1a 64 of bytes [header_bytes, file_bytes)
};
static_assert(sizeof(Header) == 8 + 4 + 4 + 10 * 4 + 8 + 8 + 8, "packed header");
static_assert(sizeof(Header) <= kHeaderBytes, "header fits");

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int64_t flags_bytes(int32_t heads) { return round_up(heads, 4); }

int64_t payload_bytes(int32_t heads, int32_t n_blocks, int64_t nnz) {
  return flags_bytes(heads) + 4 * ((int64_t)heads * n_blocks + 1) + 4 * nnz;
}

// Checks shared by the writer and the reader: sizes, grid, flags, lists.
int check_shape(const char* fn, int32_t steps, int32_t layers, int32_t heads, int32_t n_tokens,
                int32_t n_entries) {
  if (steps < 1 || layers < 1 || heads < 1 || n_tokens < 1 || n_entries < 1)
    return api_fail(CALIBATT_ERR_INVALID_ARG,
                    "%s: steps %d, layers %d, heads %d, n_tokens %d, entries %d must be >= 1", fn,
                    steps, layers, heads, n_tokens, n_entries);
  const int64_t R = (n_tokens + CALIBATT_BLOCK - 1) / CALIBATT_BLOCK;
  if ((int64_t)heads * R * R >= (int64_t)1 << 31 || (int64_t)steps * layers >= (int64_t)1 << 28)
    return api_fail(CALIBATT_ERR_UNSUPPORTED, "%s: bank too large", fn);
  return CALIBATT_OK;
}

int check_entry(const char* fn, int32_t e, const uint8_t* flags, const int32_t* off,
                const int32_t* idx, int32_t heads, int32_t n_blocks, const calibatt_grid* grid,
                int32_t n_tokens) {
  bool any_rep = false;
  for (int32_t h = 0; h < heads; ++h) {
    if (flags[h] > 2)
      return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: entry %d: repeat flag of head %d is %d", fn, e,
                      h, flags[h]);
    any_rep = any_rep || flags[h];
  }
  if (any_rep) {
    if (!grid) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: entry %d has repeat heads but the bank has no grid", fn, e);
    const int rc = check_grid(fn, *grid, n_tokens);
    if (rc) return rc;
  }
  const int64_t nnz = off[(int64_t)heads * n_blocks];
  const int rc = calibatt_validate_skiplist(off, idx, nnz, heads, n_blocks);
  if (rc) {
    const std::string msg = calibatt_last_error();
    return api_fail(rc, "%s: entry %d: %s", fn, e, msg.c_str());
  }
  return CALIBATT_OK;
}

}  // namespace

struct calibatt_bank {
  Header hdr;
  std::vector<uint8_t> file;            // the whole file
  std::vector<int32_t> entry_of;        // [steps * layers]
  std::vector<int64_t> payload_offset;  // per entry, byte offset in the file
  std::vector<int64_t> nnz;             // per entry
  int64_t payload_begin = 0;            // first payload byte (device copy starts here)
  void* device = nullptr;               // uploaded copy of [payload_begin, file end)
};

extern "C" {

int calibatt_bank_write(const char* path, int32_t steps, int32_t layers, int32_t heads,
                        int32_t n_tokens, const calibatt_grid* grid, int32_t n_entries,
                        const int32_t* entry_of, const uint8_t* const* repeat_flags,
                        const int32_t* const* kv_offsets, const int32_t* const* kv_indices) {
  const char* fn = "calibatt_bank_write";
  if (!path || !entry_of || !kv_offsets || !kv_indices)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null argument", fn);
  int rc = check_shape(fn, steps, layers, heads, n_tokens, n_entries);
  if (rc) return rc;
  if (grid && (rc = check_grid(fn, *grid, n_tokens))) return rc;
  const int32_t R = (n_tokens + CALIBATT_BLOCK - 1) / CALIBATT_BLOCK;
  for (int64_t i = 0; i < (int64_t)steps * layers; ++i)
    if (entry_of[i] < 0 || entry_of[i] >= n_entries)
      return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: (t, l) = (%lld, %lld) maps to entry %d of %d", fn,
                      (long long)(i / layers), (long long)(i % layers), entry_of[i], n_entries);
  const std::vector<uint8_t> no_flags(heads, 0);
  std::vector<int64_t> nnz(n_entries);
  for (int32_t e = 0; e < n_entries; ++e) {
    if (!kv_offsets[e]) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: entry %d: null kv_offsets", fn, e);
    nnz[e] = kv_offsets[e][(int64_t)heads * R];
    if (nnz[e] > 0 && !kv_indices[e])
      return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: entry %d: null kv_indices", fn, e);
    const uint8_t* fl = repeat_flags && repeat_flags[e] ? repeat_flags[e] : no_flags.data();
    if ((rc = check_entry(fn, e, fl, kv_offsets[e], kv_indices[e], heads, R, grid, n_tokens))) return rc;
  }

  // layout: header | map | table | payloads (each 256-byte aligned)
  const int64_t map_offset = kHeaderBytes;
  const int64_t table_offset = map_offset + 4 * (int64_t)steps * layers;
  int64_t pos = round_up(table_offset + kTableEntryBytes * n_entries, kPayloadAlign);
  std::vector<int64_t> poff(n_entries);
  for (int32_t e = 0; e < n_entries; ++e) {
    poff[e] = pos;
    pos = round_up(pos + payload_bytes(heads, R, nnz[e]), kPayloadAlign);
  }
  const int64_t file_bytes = pos;
  std::vector<uint8_t> buf(file_bytes, 0);
  std::memcpy(buf.data() + map_offset, entry_of, 4 * (size_t)steps * layers);
  for (int32_t e = 0; e < n_entries; ++e) {
    uint8_t* p = buf.data() + poff[e];
    const uint8_t* fl = repeat_flags && repeat_flags[e] ? repeat_flags[e] : no_flags.data();
    std::memcpy(p, fl, heads);
    p += flags_bytes(heads);
    std::memcpy(p, kv_offsets[e], 4 * ((size_t)heads * R + 1));
    p += 4 * ((int64_t)heads * R + 1);
    if (nnz[e] > 0) std::memcpy(p, kv_indices[e], 4 * (size_t)nnz[e]);
    uint8_t* t = buf.data() + table_offset + kTableEntryBytes * e;
    const uint64_t sum = fnv1a64(buf.data() + poff[e], (size_t)payload_bytes(heads, R, nnz[e]));
    std::memcpy(t, &poff[e], 8);
    std::memcpy(t + 8, &nnz[e], 8);
    std::memcpy(t + 16, &sum, 8);
  }
  Header h{};
  std::memcpy(h.magic, kMagic, 8);
  h.version = kVersion;
  h.header_bytes = (uint32_t)kHeaderBytes;
  h.steps = steps;
  h.layers = layers;
  h.heads = heads;
  h.n_tokens = n_tokens;
  h.n_blocks = R;
  if (grid) {
    h.frames = grid->frames;
    h.rows = grid->rows;
    h.cols = grid->cols;
    h.anchors = grid->anchors;
  }
  h.n_entries = n_entries;
  h.table_offset = table_offset;
  h.file_bytes = file_bytes;
  h.checksum = fnv1a64(buf.data() + kHeaderBytes, (size_t)(file_bytes - kHeaderBytes));
  std::memcpy(buf.data(), &h, sizeof h);

  // write beside the target, then rename over it
  const std::string tmp = std::string(path) + ".tmp";
  FILE* f = std::fopen(tmp.c_str(), "wb");
  if (!f) return api_fail(CALIBATT_ERR_IO, "%s: cannot open %s for writing", fn, tmp.c_str());
  const size_t wrote = std::fwrite(buf.data(), 1, buf.size(), f);
  const bool closed = std::fclose(f) == 0;
  if (wrote != buf.size() || !closed) {
    std::remove(tmp.c_str());
    return api_fail(CALIBATT_ERR_IO, "%s: short write to %s", fn, tmp.c_str());
  }
  if (std::rename(tmp.c_str(), path) != 0) {
    std::remove(tmp.c_str());
    return api_fail(CALIBATT_ERR_IO, "%s: cannot rename %s to %s", fn, tmp.c_str(), path);
  }
  return api_ok();
}

int calibatt_bank_open(const char* path, calibatt_bank** out) {
  const char* fn = "calibatt_bank_open";
  if (!path || !out) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null argument", fn);
  *out = nullptr;
  FILE* f = std::fopen(path, "rb");
  if (!f) return api_fail(CALIBATT_ERR_IO, "%s: cannot open %s", fn, path);
  std::vector<uint8_t> buf;
  uint8_t chunk[1 << 16];
  size_t n;
  while ((n = std::fread(chunk, 1, sizeof chunk, f)) > 0) buf.insert(buf.end(), chunk, chunk + n);
  const bool err = std::ferror(f) != 0;
  std::fclose(f);
  if (err) return api_fail(CALIBATT_ERR_IO, "%s: read error on %s", fn, path);
  if ((int64_t)buf.size() < kHeaderBytes)
    return api_fail(CALIBATT_ERR_IO, "%s: %s is %zu bytes, shorter than a header", fn, path, buf.size());
  Header h;
  std::memcpy(&h, buf.data(), sizeof h);
  if (std::memcmp(h.magic, kMagic, 8) != 0)
    return api_fail(CALIBATT_ERR_IO, "%s: %s is not a mask bank", fn, path);
  if (h.version != kVersion || h.header_bytes != kHeaderBytes)
    return api_fail(CALIBATT_ERR_IO, "%s: %s has version %u (header %u bytes); this library reads version %u", fn,
                    path, h.version, h.header_bytes, kVersion);
  if (h.file_bytes != (int64_t)buf.size())
    return api_fail(CALIBATT_ERR_IO, "%s: %s is %zu bytes, header says %lld", fn, path, buf.size(),
                    (long long)h.file_bytes);
  if (fnv1a64(buf.data() + kHeaderBytes, buf.size() - kHeaderBytes) != h.checksum)
    return api_fail(CALIBATT_ERR_IO, "%s: %s: checksum mismatch", fn, path);
  // a file that passed its checksum but fails a check of its contents is
  // reported as corrupt (CALIBATT_ERR_IO) with the check's message
  auto corrupt = [&]() {
    const std::string why = calibatt_last_error();
    return api_fail(CALIBATT_ERR_IO, "%s: %s: %s", fn, path, why.c_str());
  };
  int rc = check_shape(fn, h.steps, h.layers, h.heads, h.n_tokens, h.n_entries);
  if (rc) return corrupt();
  const int32_t R = (h.n_tokens + CALIBATT_BLOCK - 1) / CALIBATT_BLOCK;
  if (h.n_blocks != R)
    return api_fail(CALIBATT_ERR_IO, "%s: %s: n_blocks %d != ceil(N/128) = %d", fn, path, h.n_blocks, R);
  const int64_t map_bytes = 4 * (int64_t)h.steps * h.layers;
  if (h.table_offset != kHeaderBytes + map_bytes ||
      h.table_offset + kTableEntryBytes * (int64_t)h.n_entries > h.file_bytes)
    return api_fail(CALIBATT_ERR_IO, "%s: %s: bad entry table offset", fn, path);
  calibatt_grid grid{h.frames, h.rows, h.cols, h.anchors};
  const bool has_grid = h.frames != 0 || h.rows != 0 || h.cols != 0 || h.anchors != 0;
  if (has_grid && check_grid(fn, grid, h.n_tokens)) return corrupt();

  auto* b = new calibatt_bank;
  b->hdr = h;
  b->entry_of.resize((size_t)h.steps * h.layers);
  std::memcpy(b->entry_of.data(), buf.data() + kHeaderBytes, (size_t)map_bytes);
  for (size_t i = 0; i < b->entry_of.size(); ++i)
    if (b->entry_of[i] < 0 || b->entry_of[i] >= h.n_entries) {
      const int32_t bad = b->entry_of[i];
      delete b;
      return api_fail(CALIBATT_ERR_IO, "%s: %s: (t, l) #%zu maps to entry %d of %d", fn, path, i,
                      bad, h.n_entries);
    }
  b->payload_offset.resize(h.n_entries);
  b->nnz.resize(h.n_entries);
  b->payload_begin = h.file_bytes;
  for (int32_t e = 0; e < h.n_entries; ++e) {
    const uint8_t* t = buf.data() + h.table_offset + kTableEntryBytes * e;
    int64_t off, nnz;
    uint64_t sum;
    std::memcpy(&off, t, 8);
    std::memcpy(&nnz, t + 8, 8);
    std::memcpy(&sum, t + 16, 8);
    const int64_t bytes = nnz >= 0 && nnz <= (int64_t)h.heads * R * R ? payload_bytes(h.heads, R, nnz) : -1;
    if (bytes < 0 || off % kPayloadAlign || off < h.table_offset + kTableEntryBytes * (int64_t)h.n_entries ||
        off > h.file_bytes - bytes) {
      delete b;
      return api_fail(CALIBATT_ERR_IO, "%s: %s: entry %d: bad offset or size", fn, path, e);
    }
    if (fnv1a64(buf.data() + off, (size_t)bytes) != sum) {
      delete b;
      return api_fail(CALIBATT_ERR_IO, "%s: %s: entry %d: checksum mismatch", fn, path, e);
    }
    const uint8_t* flags = buf.data() + off;
    const int32_t* kvo = reinterpret_cast<const int32_t*>(flags + flags_bytes(h.heads));
    const int32_t* kvi = kvo + (int64_t)h.heads * R + 1;
    if (kvo[(int64_t)h.heads * R] != nnz) {
      delete b;
      return api_fail(CALIBATT_ERR_IO, "%s: %s: entry %d: list length %d != table nnz %lld", fn, path, e,
                      kvo[(int64_t)h.heads * R], (long long)nnz);
    }
    if ((rc = check_entry(fn, e, flags, kvo, kvi, h.heads, R, has_grid ? &grid : nullptr, h.n_tokens))) {
      delete b;
      return rc == CALIBATT_ERR_BAD_SKIPLIST ? rc : corrupt();
    }
    b->payload_offset[e] = off;
    b->nnz[e] = nnz;
    if (off < b->payload_begin) b->payload_begin = off;
  }
  b->file = std::move(buf);
  *out = b;
  return api_ok();
}

void calibatt_bank_close(calibatt_bank* bank) { delete bank; }

int calibatt_bank_get_info(const calibatt_bank* bank, calibatt_bank_info* out) {
  if (!bank || !out) return api_fail(CALIBATT_ERR_INVALID_ARG, "calibatt_bank_get_info: null argument");
  const Header& h = bank->hdr;
  out->steps = h.steps;
  out->layers = h.layers;
  out->heads = h.heads;
  out->n_tokens = h.n_tokens;
  out->n_blocks = h.n_blocks;
  out->n_entries = h.n_entries;
  out->grid = calibatt_grid{h.frames, h.rows, h.cols, h.anchors};
  out->total_nnz = 0;
  for (int64_t v : bank->nnz) out->total_nnz += v;
  out->device_bytes = (size_t)(h.file_bytes - bank->payload_begin);
  return api_ok();
}

int calibatt_bank_upload(calibatt_bank* bank, void* device, size_t bytes, void* stream) {
  const char* fn = "calibatt_bank_upload";
  if (!bank || !device) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null argument", fn);
  const size_t need = (size_t)(bank->hdr.file_bytes - bank->payload_begin);
  if (bytes < need) return api_fail(CALIBATT_ERR_WORKSPACE, "%s: %zu bytes < %zu", fn, bytes, need);
  if (reinterpret_cast<uintptr_t>(device) % kPayloadAlign)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: device buffer must be %lld-byte aligned", fn,
                    (long long)kPayloadAlign);
  const hipError_t e = hipMemcpyAsync(device, bank->file.data() + bank->payload_begin, need,
                                      hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return api_fail(CALIBATT_ERR_HIP, "%s: hipMemcpyAsync: %s", fn, hipGetErrorString(e));
  bank->device = device;
  return api_ok();
}

int calibatt_bank_lookup(const calibatt_bank* bank, int32_t t, int32_t l, int32_t on_device,
                         calibatt_bank_entry* out) {
  const char* fn = "calibatt_bank_lookup";
  if (!bank || !out) return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: null argument", fn);
  const Header& h = bank->hdr;
  if (t < 0 || t >= h.steps || l < 0 || l >= h.layers)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: (t, l) = (%d, %d) outside %d x %d", fn, t, l, h.steps,
                    h.layers);
  if (on_device && !bank->device)
    return api_fail(CALIBATT_ERR_INVALID_ARG, "%s: bank not uploaded", fn);
  const int32_t e = bank->entry_of[(size_t)t * h.layers + l];
  const int64_t off = bank->payload_offset[e];
  const uint8_t* host = bank->file.data() + off;
  const uint8_t* base = on_device
      ? static_cast<const uint8_t*>(bank->device) + (off - bank->payload_begin)
      : host;
  out->entry = e;
  out->repeat_flags = host;
  out->kv_offsets = reinterpret_cast<const int32_t*>(base + flags_bytes(h.heads));
  out->kv_indices = out->kv_offsets + (int64_t)h.heads * h.n_blocks + 1;
  out->nnz = bank->nnz[e];
  return api_ok();
}

}  // extern "C"
