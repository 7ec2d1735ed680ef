// Device-side building blocks shared by the attention and energy kernels
// (gfx950, wave64). Internal header: not part of the C ABI.
//
// Tile geometry. A workgroup of 256 threads (4 waves) owns one 128-row query
// tile; wave w owns rows 32w..32w+31. Scores are computed transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 so that every lane ends up
// holding one query row (lane % 32) and 64 of the 128 key columns of a block
// (the other 64 live in lane ^ 32). Row max / sum then need a single
// cross-lane exchange, and the softmax rescale of the output accumulator is a
// per-lane scalar.
//
// 32x32 MFMA accumulator layout (16 fp32 per lane): lane l, element i holds
// row 8*(i/4) + 4*(l/32) + (i%4), column l%32. A-operand lane l supplies row
// l%32 and B-operand lane l supplies column l%32, each with an 8-element
// k-slot chosen by l/32; since both operands of a product are loaded with
// the same (lane group, element) -> k mapping, the sum over k is the same
// whatever order the hardware contracts them in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace calibatt {

constexpr int kBlock = 128;       // tokens per block (B)
constexpr int kDim = 128;         // head dimension (D)
constexpr int kThreads = 256;     // 4 waves

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Work-item order across XCDs. Workgroups are dispatched round-robin over
// the 8 XCDs (workgroup i -> XCD i % 8). Inside every run of 8*S workgroup
// ids this map hands each XCD S consecutive work items, so the tiles that
// share an XCD's L2 at a given time are neighbouring query blocks of one
// head and reuse the same key/value blocks. The last partial run is left in
// order. S = CALIBATT_XCD_RUN (0 disables the remap).
#ifndef CALIBATT_XCD_RUN
#define CALIBATT_XCD_RUN 32
#endif
__device__ __forceinline__ int xcd_remap(int id, int n_items) {
  constexpr int kXcd = 8, kPer = CALIBATT_XCD_RUN, kSpan = kXcd * kPer;
  if (kPer == 0) return id;
  const int base = (id / kSpan) * kSpan;
  if (base + kSpan > n_items) return id;
  const int local = id - base;
  return base + (local % kXcd) * kPer + local / kXcd;
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Query fragment (B operand of S^T = K Q^T) for one lane: row `tok` of q,
// d = 16*s + 8*g .. +7 for s = 0..7. Zero when !valid.
__device__ __forceinline__ void load_query(bf16x8 (&qf)[8], const uint16_t* __restrict__ q,
                                           int64_t stride_token, int64_t tok, bool valid,
                                           int g) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u32x4 w = valid ? load16(q + tok * stride_token + 16 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u};
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Asynchronous tile staging (direct global -> LDS copies, no registers).
//
// A 128 x 128 bf16 tile occupies 32 KiB of LDS: row r (token key0 + r) at
// byte r*256, its sixteen 16-byte chunks permuted by an XOR swizzle so that
// the reads the MFMA operands need hit distinct LDS banks:
//   physical chunk = logical chunk ^ (r % 16)
// so the 16-byte operand reads of 16 consecutive rows hit distinct banks
// (K tiles, and V^T tiles, which take the same path).
// One global_load_lds_dwordx4 moves 64 lanes x 16 B into 1 KiB of LDS (lane
// i to byte 16*i of the block M0 points at), i.e. four rows. Wave w copies
// rows 32w .. 32w+31 with eight such instructions; instruction j covers rows
// 32w + 4j + (lane / 16), lane % 16 being the physical chunk.
//
// The copies are issued from inline assembly on purpose: the compiler
// cannot tell which LDS buffer a copy writes and would otherwise wait for
// every copy in flight before any LDS read or barrier, which serialises the
// prefetch. Completion is tracked by hand with s_waitcnt vmcnt (copies
// retire in issue order) followed by a workgroup barrier. Setting M0 needs
// one wait state before the copy that reads it.

constexpr int kTileBytes = kBlock * kDim * 2;   // 32 KiB
constexpr int kCopiesPerTile = 8;               // per wave

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Wave-uniform value pinned to a scalar register (asm "s" operands would
// otherwise print a vector register the compiler chose to keep it in).
__device__ __forceinline__ uint32_t uni(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// 16 bytes per lane from a per-lane 64-bit address into LDS [lds + 16*lane]
// (lds wave-uniform).
__device__ __forceinline__ void copy16_vaddr(uint32_t lds, const void* vaddr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(uni(lds)), "v"(vaddr) : "memory", "m0");
}

#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence: this wave's LDS reads have
// returned, then every wave of the workgroup arrives. (A __syncthreads fence
// would also wait for all copies in flight.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Per-lane source offsets of the fast copy path, fixed for the kernel.
// Instruction j of a wave covers rows 32w + 4j + sub (sub = lane / 16) with
// physical chunk p = lane % 16. The swizzle is (row % 16) = 4(j%4) + sub:
// logical chunk p ^ sub ^ 4(j%4), i.e. the j = 0 offset with bits 6-7 flipped
// by (j%4) << 6 -- valid while a row's byte offset has zero low 8 bits, so the
// fast path requires row_bytes % 256 == 0 (other strides take the per-lane
// path).
struct CopyPlan {
  uint32_t k_off;      // row sub, chunk p ^ sub
  int64_t row_bytes;   // stride_token * 2
  bool fast;           // row_bytes % 256 == 0
};

__device__ __forceinline__ CopyPlan make_copy_plan(int64_t stride_token, int lane) {
  CopyPlan cp;
  const int sub = lane >> 4, p = lane & 15;
  cp.row_bytes = stride_token * 2;
  cp.k_off = (uint32_t)(sub * cp.row_bytes + ((p ^ sub) << 4));
  cp.fast = (cp.row_bytes & 255) == 0;
  return cp;
}

// Buffer resource over `base` with the largest record count (the fast copy
// path only addresses rows that exist; the range check never fires).
__device__ __forceinline__ u32x4 make_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = uni((uint32_t)a);
  r[1] = uni((uint32_t)(a >> 32) & 0xffffu);  // stride 0 (raw buffer)
  r[2] = 0xffffffffu;
  r[3] = 0x00020000u;                          // untyped 32-bit data
  return r;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// Eight copies of rows 32*wave .. +31 of a full K tile (rsrc over the
// tile's first row, soff = byte offset of row 32*wave). Instruction j reads
// with offset k ^ ((j % 4) << 6) at row base 32*wave + 4j.
__device__ __forceinline__ void copy_k_fast(uint32_t lds, u32x4 rs, uint32_t soff, uint32_t step4,
                                            uint32_t k) {
  uint32_t t0, t1;
  asm volatile(
      "s_mov_b32 m0, %[lds]\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[k], %[rs], %[so] offen lds\n\t"
      "v_xor_b32 %[t0], 0x40, %[k]\n\t"
      "s_add_u32 %[so], %[so], %[st]\n\ts_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[t0], %[rs], %[so] offen lds\n\t"
      "v_xor_b32 %[t1], 0x80, %[k]\n\t"
      "s_add_u32 %[so], %[so], %[st]\n\ts_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[t1], %[rs], %[so] offen lds\n\t"
      "v_xor_b32 %[t0], 0xc0, %[k]\n\t"
      "s_add_u32 %[so], %[so], %[st]\n\ts_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[t0], %[rs], %[so] offen lds\n\t"
      "s_add_u32 %[so], %[so], %[st]\n\ts_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[k], %[rs], %[so] offen lds\n\t"
      "v_xor_b32 %[t1], 0x40, %[k]\n\t"
      "s_add_u32 %[so], %[so], %[st]\n\ts_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[t1], %[rs], %[so] offen lds\n\t"
      "v_xor_b32 %[t0], 0x80, %[k]\n\t"
      "s_add_u32 %[so], %[so], %[st]\n\ts_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[t0], %[rs], %[so] offen lds\n\t"
      "v_xor_b32 %[t1], 0xc0, %[k]\n\t"
      "s_add_u32 %[so], %[so], %[st]\n\ts_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[t1], %[rs], %[so] offen lds"
      : [so] "+s"(soff), [t0] "=&v"(t0), [t1] "=&v"(t1)
      : [lds] "s"(uni(lds)), [rs] "s"(rs), [st] "s"(uni(step4)), [k] "v"(k)
      : "memory", "m0", "scc");
}

#pragma clang diagnostic pop

// Issues this wave's eight copies of the tile whose first token row is
// key0. Rows at or past n_tokens are read from row n_tokens - 1 instead
// (their scores repeat a real score of the block and their probabilities are
// zeroed, so those values never matter).
__device__ __forceinline__ void copy_tile(uint32_t lds_tile, const uint16_t* __restrict__ src,
                                          const CopyPlan& cp, int key0, int n_tokens, int wave,
                                          int lane) {
  const uint32_t lds = lds_tile + wave * (kCopiesPerTile * 1024);
  if (cp.fast && key0 + kBlock <= n_tokens) {
    const u32x4 rs = make_rsrc(reinterpret_cast<const char*>(src) + (int64_t)key0 * cp.row_bytes);
    const uint32_t soff = uni((uint32_t)(32 * wave) * (uint32_t)cp.row_bytes);
    copy_k_fast(lds, rs, soff, 4u * (uint32_t)cp.row_bytes, cp.k_off);
  } else {
    const int sub = lane >> 4, p = lane & 15;
#pragma unroll
    for (int j = 0; j < kCopiesPerTile; ++j) {
      const int row = 32 * wave + 4 * j + sub;
      const int tok = key0 + row < n_tokens ? key0 + row : n_tokens - 1;
      copy16_vaddr(lds + 1024 * j,
                   reinterpret_cast<const char*>(src) + (int64_t)tok * cp.row_bytes + (p ^ (row & 15)) * 16);
    }
  }
}

// LDS byte offset of the K operand for d-step s (0..7) of a lane whose
// A-operand row is `row` (r % 16 == row % 16) and lane group g.
__device__ __forceinline__ int k_operand_offset(int row, int s, int g) {
  return row * 256 + ((((2 * s + g) ^ (row & 15))) << 4);
}

typedef __attribute__((address_space(3))) const uint8_t* lds_cptr;

// LDS loads at an LDS byte address. Callers pass a per-lane base plus a
// compile-time displacement, which the compiler folds into the instruction's
// 16-bit offset field (so one base register serves many loads).
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>((lds_cptr)(uintptr_t)addr);
}

}  // namespace calibatt
