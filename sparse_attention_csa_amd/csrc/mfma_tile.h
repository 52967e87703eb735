// LDS row tiles of 512-wide bf16 entries and the MFMA operand reads on them,
// shared by the two attention kernels (attend_mfma.hip: all rows of a split
// through every wavefront; attend_rows.hip: rows divided among wavefronts).
//
// Tile layout.  A row is 1 KB, unpadded; its 16-byte chunk g is stored at
// chunk position g ^ swz(r % 16), r the row within the tile.  The DMA applies
// the permutation by choosing which global chunk each lane fetches.  swz
// keeps both read patterns free of bank conflicts: the score reads (16 rows,
// one 16-byte chunk per lane, ds_read_b128) and the value reads
// (ds_read_b64_tr_b16: 4 rows x 4 columns per lane group).
#pragma once

#include "common.h"

namespace csa {
namespace tile {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

constexpr int kC = 512;        // entry / head dim
constexpr int kRowB = kC * 2;  // bytes per row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 20.f;  // log2 headroom of the weights over the reference max

// s_waitcnt vmcnt(N), lgkmcnt / expcnt not waited (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int wait_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// C[16x16] += A[16x32] B[32x16]
CSA_DEV f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// C[16x16] += A[16x16] B[16x16]
CSA_DEV f32x4_t mfma16(i16x4_t a, i16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

CSA_DEV bf16x8_t lds8(const char* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// ds_read_b64_tr_b16: lane (i, g) of a 16x4 lane grid gets column i of the
// 4x16 block whose rows start at the lane group's addresses
CSA_DEV i16x4_t ld_tr(const char* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

CSA_DEV bf16x8_t cat8(i16x4_t a, i16x4_t b) {
  i16x8_t v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// chunk permutation of a tile row (r % 16): a bijection on 0..15 with
//   bits 0..3 = r2, r0, r1, r2 ^ r3
CSA_DEV int swz(int r) {
  return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) | ((((r >> 2) ^ (r >> 3)) & 1) << 3);
}

// one lane's 16 bytes of a 1 KB row: global chunk (lane ^ sw) lands at LDS
// chunk lane of the row
CSA_DEV void dma_row(const uint16_t* src_row, char* lds_row, int lane, int sw) {
  __builtin_amdgcn_global_load_lds(
      (const void __attribute__((address_space(1)))*)(src_row + 8 * (lane ^ sw)),
      (void __attribute__((address_space(3)))*)(lds_row), 16, 0, 0);
}

// The same DMA written out, M0 set by hand.  The compiler does not see an
// LDS DMA here, so it adds no waits of its own before LDS reads (with the
// builtin it waits for every DMA in flight before any read of the same LDS
// object, including the younger tiles of a ring); the caller waits for the
// tile explicitly (s_waitcnt vmcnt) before reading it, and before writing
// LDS that a DMA may still target.  No output registers: the data goes to
// LDS only.  (gfx950 needs one wait state between the M0 write and the DMA.)
CSA_DEV void dma_row_m0(const uint16_t* src_row, uint32_t lds_row, int lane, int sw) {
  const uint16_t* p = src_row + 8 * (lane ^ sw);
  __asm__ __volatile__("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(p), "s"(lds_row)
                       : "memory");
}

// Any 16 bytes per lane, DMA'd to LDS bytes lds_base + 16 lane (same
// rules as dma_row_m0; lds_base is wavefront-uniform).
CSA_DEV void dma16_m0(const void* p, uint32_t lds_base) {
  __asm__ __volatile__("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(p), "s"(lds_base)
                       : "memory");
}

// LDS byte address of a pointer into a __shared__ object
CSA_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Per-lane byte offsets of the two read patterns in a tile whose 16-row
// block starts at offset 0 (lane = 16 lg + li).
//  score reads: row li, chunk 4ks + lg, i.e. byte (64 ks) ^ s_x with
//    s_x < 256, = 256 (ks / 4) + ((64 (ks % 4)) ^ s_x): s_base[ks % 4]
//  value reads: rows 4lg .. 4lg+3 (lane row 4lg + li/4), columns
//    16dt + 4(li%4) .., byte (32 dt) ^ t_x = 256 (dt / 8) + ((32 (dt % 8)) ^ t_x):
//    t_base[dt % 8]
struct Bases {
  int s[4];
  int t[8];
};
CSA_DEV Bases lane_bases(int li, int lg) {
  Bases b;
  const int s_x = 16 * (lg ^ swz(li));
  const int tr_row = 4 * lg + (li >> 2);
  const int t_x = 16 * (((li >> 1) & 1) ^ swz(tr_row));
#pragma unroll
  for (int u = 0; u < 4; ++u) b.s[u] = li * kRowB + ((64 * u) ^ s_x);
#pragma unroll
  for (int u = 0; u < 8; ++u) b.t[u] = tr_row * kRowB + 8 * (li & 1) + ((32 * u) ^ t_x);
  return b;
}

}  // namespace tile
}  // namespace csa
