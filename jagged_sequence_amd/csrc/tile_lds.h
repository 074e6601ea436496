// Row-major bf16 tiles in LDS for D = 128, filled straight from global memory and read either
// row-wise (16-byte MFMA operands) or transposed (ds_read_b64_tr_b16).
//
// A tile row is 128 bf16 = 256 bytes = 16 chunks of 16 bytes, rows packed with no padding. Chunk c of
// row r is stored at chunk position c ^ swz(r), swz(r) = ((r & 3) << 2) | ((r >> 2) & 3), a bijection
// of r mod 16. With it, (a) the 16 lanes of a quarter-wave that read one logical chunk of 16
// different rows hit 16 different bank groups, and (b) a transposing read, which touches 4
// consecutive rows x 4 consecutive chunks per half-wave, also covers all banks exactly once.
//
// Loads use buffer_load ... lds: lane i of a wave writes 16 bytes at (wave-uniform LDS base) + 16 i,
// so one instruction fills 4 rows (1 KB); rows past the jagged end are out of the buffer range and
// arrive as zeros. No registers are used for staging.
//
// The loads are issued as inline assembly, outside the compiler's view. The compiler cannot tell one
// LDS tile from another, so for a load into LDS that it knows of it waits for the load to land
// before the wave's next LDS read of any tile, which would expose the whole latency of the next
// tile's prefetch. Hidden from it, the loads are waited for only where the kernels say so: every
// consumer of a tile sits behind wait_vm() in each wave followed by a workgroup barrier.
#pragma once

#include "device_common.h"

namespace jfa {

constexpr int kRowBytes = 256;  // D = 128 bf16

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ lds_ptr_t to_lds(const void* p) { return (lds_ptr_t)p; }

// Byte offsets (within the slice) and LDS row for instruction u of a wave filling a tile of
// `rows_per_wave` rows: lane covers row 4 u + lane/16 of the wave's rows and the logical chunk that
// lands at physical position lane % 16.
struct TileLoader {
  uint32_t voff[4];  // per u: row_in_tile * rs * 2 + logical chunk * 16 (without the tile's first row)
};

// Each wave fills rows [16 wave, 16 wave + 16) of a 64-row tile with 4 instructions.
__device__ __forceinline__ TileLoader make_loader64(int wave, int lane, int rs) {
  TileLoader t;
  const int q = lane >> 4, p = lane & 15;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 16 * wave + 4 * u + q;  // row within the tile; r & 15 = 4 u + q
    const int c = p ^ swz(r);
    t.voff[u] = (uint32_t)(r * rs * 2 + c * 16);
  }
  return t;
}

// One buffer_load_dwordx4 ... lds of 16 bytes per lane: lane i's bytes at `voff` of the buffer land
// at LDS byte address `lds` + 16 i. M0 carries the wave-uniform LDS address (set by the compiler just
// before); the s_nop covers the wait state required between an SALU write of M0 and the load reading it.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t src, uint32_t voff, const unsigned char* lds) {
  const uint32_t m0v = (uint32_t)(uintptr_t)to_lds(lds);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" : : "{m0}"(m0v), "v"(voff), "s"(src) : "memory");
}

// The same for 4 bytes per lane: lane i's bytes at `voff` land at `lds` + 4 i (one 256-byte row).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t src, uint32_t voff, const void* lds) {
  const uint32_t m0v = (uint32_t)(uintptr_t)to_lds(lds);
  asm volatile("s_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" : : "{m0}"(m0v), "v"(voff), "s"(src) : "memory");
}

// Issue the loads of a 64-row tile whose first row is `row0` of the slice into LDS at `tile`.
__device__ __forceinline__ void load_tile64(const TileLoader& t, __amdgpu_buffer_rsrc_t src, int row0, int rs,
                                            unsigned char* tile, int wave) {
  const uint32_t base = (uint32_t)(row0 * rs * 2);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    dma16(src, base + t.voff[u], tile + (16 * wave + 4 * u) * kRowBytes);
}

// Each of 8 waves fills rows [8 wave, 8 wave + 8) of a 64-row tile with 2 instructions.
__device__ __forceinline__ TileLoader make_loader64_w8(int wave, int lane, int rs) {
  TileLoader t;
  const int q = lane >> 4, p = lane & 15;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 8 * wave + 4 * u + q;
    const int c = p ^ swz(r);
    t.voff[u] = (uint32_t)(r * rs * 2 + c * 16);
  }
  t.voff[2] = t.voff[3] = 0;
  return t;
}

__device__ __forceinline__ void load_tile64_w8(const TileLoader& t, __amdgpu_buffer_rsrc_t src, int row0, int rs,
                                               unsigned char* tile, int wave) {
  const uint32_t base = (uint32_t)(row0 * rs * 2);
#pragma unroll
  for (int u = 0; u < 2; ++u)
    dma16(src, base + t.voff[u], tile + (8 * wave + 4 * u) * kRowBytes);
}

// Wait for this wave's outstanding global loads (including loads into LDS).
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0); }

// Wait on the vector-memory counter only, until at most N of this wave's vector memory operations
// are outstanding. Loads complete in issue order, so once at most N operations are left, every
// load followed by at least N loads has landed: with the next tile's N loads issued after the
// current tile's, this waits for the current tile and leaves the next one in flight.
template <int N>
__device__ __forceinline__ void wait_vm_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// Row operand: lane reads logical chunk (2 kb + hh) of tile row `r`: byte address
// r * 256 + (((2 kb + hh) ^ swz(r)) << 4) = (r * 256 + ((hh ^ swz(r)) << 4)) ^ (kb << 5).
__device__ __forceinline__ uint32_t row_operand_base(int r, int hh) {
  return (uint32_t)(r * kRowBytes + ((hh ^ swz(r)) << 4));
}

__device__ __forceinline__ bf16x8 lds_read16(const unsigned char* tile, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(tile + off);
}

// Transposed operand of a 32x32x16 MFMA from a k-major tile (row = contraction index, column = m):
// lane l receives X[k0 + 8 (l/32) + 4 half + 0..3][m0 + l % 32] for half = 0, 1 (8 values). Within
// each 16-lane group, lane s supplies the address of X[k0 + 8 (g/2) + 4 half + s/4][m0 + 16 (g%2) + 4 (s%4)],
// g = lane / 16. For m0 = 32 db and k0 a multiple of 16 the byte address is
// 256 k0 + (T[half] ^ (64 db)) with the lane constant T computed here.
__device__ __forceinline__ void tr_operand_bases(int lane, uint32_t (&T)[2]) {
  const int g = lane >> 4, s = lane & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int rr = 8 * (g >> 1) + 4 * half + (s >> 2);  // row within the 16-row group
    const int col = 16 * (g & 1) + 4 * (s & 3);         // column within the 32-column block
    const int c = col >> 3, w = col & 7;
    T[half] = (uint32_t)(rr * kRowBytes + ((c ^ swz(rr)) << 4) + 2 * w);
  }
}

__device__ __forceinline__ bf16x8 lds_read_tr(const unsigned char* tile, uint32_t off0, uint32_t off1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + off0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + off1));
  typedef __attribute__((ext_vector_type(8))) short s16x8;
  const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Stores a wave's 32-row x 128-column tile, held in the MFMA accumulator layout (lane l: row l % 32;
// register r of block db: column 32 db + 8 (r / 4) + 4 (l / 32) + r % 4), as bf16 rows through an
// 8 KB LDS area `stg` that no other wave uses meanwhile. Held directly, a lane owns 4-column pieces
// of its row, so a store instruction would touch 32 rows with 16 bytes each; staged, each store
// writes 4 whole 256-byte rows. The 16-byte chunk c of row r sits at c ^ (r & 15), which keeps both
// the writes and the reads free of bank conflicts. Row r (< nrows) goes to row_ptr(r).
template <class RowPtr>
__device__ __forceinline__ void store_rows_staged(unsigned char* stg, const f32x16 (&acc)[4], float mul, int lane,
                                                  int nrows, RowPtr row_ptr) {
  const int r = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 4 * db + g;
      *reinterpret_cast<uint2*>(stg + r * kRowBytes + ((c ^ (r & 15)) << 4) + 8 * hh) =
          make_uint2(pack2_bf16(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                     pack2_bf16(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul));
    }
  wave_lds_fence();
  const int cc = lane & 15;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int row = 4 * it + (lane >> 4);
    const uint4 x = *reinterpret_cast<const uint4*>(stg + row * kRowBytes + ((cc ^ (row & 15)) << 4));
    if (row < nrows) *reinterpret_cast<uint4*>(row_ptr(row) + cc * 16) = x;
  }
}

}  // namespace jfa
