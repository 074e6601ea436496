// Device helpers shared by the gfx950 attention kernels: MFMA wrappers, bf16 packing, the
// relative-distance bucket, activations built from exp2 and reciprocal, and tile loaders.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "jfa_internal.h"

namespace jfa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// 32x32x16 bf16 MFMA, fp32 accumulate. Operand lane layout (gfx950): lane l holds row (A) or
// column (B) l%32 and the 8 contraction elements 8*(l/32)..+7; the accumulator holds column l%32
// and rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Accumulator row m = 8*(r/4) + 4*(l/32) + r%4 is loaded from operand row kappa(m) (bits 2 and 3
// swapped). Then accumulator registers 8c..8c+7 of lane l hold operand rows 16c + 8*(l/32) + 0..7,
// which is exactly the B-operand layout of the next MFMA whose contraction runs over those rows:
// scores computed this way feed the second product straight from registers.
__device__ __forceinline__ int kappa(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Operand row held by accumulator register r of lane-half hh after the kappa load.
__device__ __forceinline__ int acc_row(int r, int hh) { return 16 * (r >> 3) + 8 * hh + (r & 7); }

__device__ __forceinline__ bf16x8 lds_load8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    f32x2 f = {x[j], x[j + 1]};
    bf16x2 p = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
    r[j] = p[0];
    r[j + 1] = p[1];
  }
  return r;
}

// acc + the sum of the 32 bf16 values in p (v_dot2c_f32_bf16 against (1, 1): two values per
// instruction, fp32 accumulation).
__device__ __forceinline__ float rowsum_bf16(const bf16x8 (&p)[4], float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float acc2 = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 8; j += 4) {
      acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[c][j], p[c][j + 1]}, one, acc, false);
      acc2 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[c][j + 2], p[c][j + 3]}, one, acc2, false);
    }
  return acc + acc2;
}

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Relative-distance bucket: exact below 16, then four equal-width buckets per octave, capped at 63.
// (Also built for the host, where a test compares it with the reference bucket over every distance.)
__host__ __device__ __forceinline__ int rel_bucket(int d) {
  d = d < 0 ? -d : d;
  const int e = 31 - __builtin_clz(d | 16);  // floor(log2 d) for d >= 16; the select below covers d < 16
  const int b = 16 + 4 * (e - 4) + ((d >> (e - 2)) & 3);
  return d < 16 ? d : (b < 63 ? b : 63);
}

// First distance of bucket u >= 16: 2^e + m 2^(e - 2) with e = 4 + (u - 16) / 4, m = (u - 16) % 4
// (the inverse of rel_bucket on its logarithmic part; bucket 63 also takes every larger distance).
__host__ __device__ __forceinline__ int rel_bucket_start(int u) {
  const int e = 4 + ((u - 16) >> 2), m = (u - 16) & 3;
  return (1 << e) + (m << (e - 2));
}

// Score activations for GDPA. sigma(z) = 1 / (1 + 2^(-z log2 e)); SiLU(x) = x sigma(x);
// GELU_tanh(x) = x sigma(2u), u = sqrt(2/pi) (x + 0.044715 x^3), using 1 + tanh(u) = 2 sigma(2u).
// Only the exp2 and reciprocal units are used, no tanh.
constexpr float kGeluK2 = 2.0f * 0.7978845608028654f;  // 2 sqrt(2/pi)
constexpr float kGeluC = 0.044715f;
// The exponent of sigma(2u) is -log2(e) 2u = x (kGeluE1 + kGeluE3 x^2); (2u)' = kGeluK2 + kGeluD3 x^2.
constexpr float kGeluE1 = -kLog2e * kGeluK2;
constexpr float kGeluE3 = -kLog2e * kGeluK2 * kGeluC;
constexpr float kGeluD3 = 3.0f * kGeluK2 * kGeluC;

template <int ACT>
__device__ __forceinline__ float act_fwd(float x) {
  if (ACT == kSilu) {
    return x * fast_rcp(1.0f + fast_exp2(-kLog2e * x));
  } else {
    const float x2 = x * x;
    return x * fast_rcp(1.0f + fast_exp2(x * __builtin_fmaf(kGeluE3, x2, kGeluE1)));
  }
}

// act(x) and act'(x) together: SiLU' = sigma + x sigma (1 - sigma) = sigma + f (1 - sigma);
// GELU_tanh' = sigma(2u) + x sigma(2u) (1 - sigma(2u)) (2u)'.
template <int ACT>
__device__ __forceinline__ void act_fwd_grad(float x, float& f, float& g) {
  if (ACT == kSilu) {
    const float sg = fast_rcp(1.0f + fast_exp2(-kLog2e * x));
    f = x * sg;
    g = __builtin_fmaf(f, 1.0f - sg, sg);
  } else {
    const float x2 = x * x;
    const float sg = fast_rcp(1.0f + fast_exp2(x * __builtin_fmaf(kGeluE3, x2, kGeluE1)));  // sigma(2u)
    const float dz = __builtin_fmaf(kGeluD3, x2, kGeluK2);                                    // (2u)'
    f = x * sg;
    g = __builtin_fmaf(f * (1.0f - sg), dz, sg);
  }
}

// Store 4 consecutive fp32 values as bf16 (8 bytes) or fp32 (16 bytes).
__device__ __forceinline__ void store4(void* base, size_t idx, float a, float b, float c, float d, int f32) {
  if (f32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx) = make_float4(a, b, c, d);
  } else {
    uint2 w = make_uint2(pack2_bf16(a, b), pack2_bf16(c, d));
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + idx) = w;
  }
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// A work record (item or split group), read through the constant address space: the list is never
// written while a kernel runs, and the promise lets the compiler fetch the record with scalar loads.
struct WorkRec {
  int b, h, tile, lo, hi, slot, qs, Lq, ks, Lkv, first;
};
__device__ __forceinline__ WorkRec load_item(const int32_t* list, int i) {
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  const cptr r = (cptr)(list + (size_t)i * kItemInts);
  return {r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7], r[8], r[9], r[10]};
}
__device__ __forceinline__ WorkRec load_group(const int32_t* list, int i) {
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  const cptr r = (cptr)(list + (size_t)i * kGroupInts);
  // group layout: b, h, tile, slot0, R, qs, Lq, ks, Lkv (slot0 and R returned in lo and hi)
  return {r[0], r[1], r[2], r[3], r[4], -1, r[5], r[6], r[7], r[8], 0};
}

// Band visibility (window W and / or block Bk, with or without the causal limit). Query i and key
// j are visible together iff band_key_lo(i) <= j <= band_key_hi(i), equivalently iff
// band_row_lo(j) <= i <= band_row_hi(j); every bound is non-decreasing in its argument, so the
// bounds of a run of rows (keys) are those of its first and last. Positions are within-sequence;
// the sequence's key (row) count clips the upper bound, so one test also masks the ragged tail.
__device__ __forceinline__ int band_key_lo(int i, Band b) {
  int lo = 0;
  if (b.window) lo = max(lo, i - b.window + 1);
  if (b.block) lo = max(lo, (i / b.block) * b.block);
  return lo;
}
__device__ __forceinline__ int band_key_hi(int i, int Lkv, Band b) {
  int hi = Lkv - 1;
  if (b.causal) hi = min(hi, i);
  else if (b.window) hi = min(hi, i + b.window - 1);
  if (b.block) hi = min(hi, (i / b.block) * b.block + b.block - 1);
  return hi;
}
__device__ __forceinline__ int band_row_lo(int j, Band b) {
  int lo = 0;
  if (b.causal) lo = j;
  else if (b.window) lo = max(lo, j - b.window + 1);
  if (b.block) lo = max(lo, (j / b.block) * b.block);
  return lo;
}
__device__ __forceinline__ int band_row_hi(int j, int Lq, Band b) {
  int hi = Lq - 1;
  if (b.window) hi = min(hi, j + b.window - 1);
  if (b.block) hi = min(hi, (j / b.block) * b.block + b.block - 1);
  return hi;
}

// Buffer resource over the rows of one (sequence, head) slice of a [T, H, D] bf16 tensor: `base`
// points at row 0 of the slice, rows are `rs` elements apart and `rows` of them are valid. Loads
// past the last valid row fall outside the resource's byte range and return zeros, so tails of
// jagged sequences need no branch and never read a neighbouring sequence.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const uint16_t* base, int rows, int rs, int D) {
  const uint32_t bytes = rows > 0 ? (uint32_t)((rows - 1) * rs + D) * 2u : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes at byte offset `off` of a buffer resource (zeros when out of range).
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

// Keeps the compiler from moving LDS accesses of one wave across this point; the hardware
// executes one wave's LDS instructions in order, so a wave may then read what it just wrote.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-wave diagonal bias vector. The relative-position bias of a 32-query x 64-key wave tile
// depends only on d = i - j, which takes 95 consecutive values there. Each wave writes
// vec[t] = T[bucket(|d0 + t|)] * mul for t in [0, 95) (two entries per lane) and then loads every
// score's bias with plain LDS reads, no per-score bucket arithmetic.
constexpr int kDiagLen = 96;
__device__ __forceinline__ void fill_diag(float* vec, const float* tab, int d0, float mul, int lane) {
  vec[lane] = tab[rel_bucket(d0 + lane)] * mul;
  if (lane < kDiagLen - 64) vec[64 + lane] = tab[rel_bucket(d0 + 64 + lane)] * mul;
}

// Bias gradient: dT[u] sums dS over the scores whose relative distance falls in bucket u (one bin
// for the per-head scalar). Each lane keeps a running sum for its current bucket in registers;
// when its bucket changes, the sum is added to this wave's bins as a 2^-32 fixed-point integer.
// Integer addition is associative, so the bins and the global totals built from them do not depend
// on the order in which lanes, waves or workgroups add: the result is deterministic.
constexpr int kDbiasBins = 64;
__device__ __forceinline__ unsigned long long to_fixed(float x) {
  return (unsigned long long)__float2ll_rn(x * 4294967296.0f);  // exact scaling by 2^32
}
struct DbiasLane {
  int u = -1;
  float s = 0.0f;
  __device__ __forceinline__ void flush(unsigned long long* bins) {
    if (u >= 0 && s != 0.0f) atomicAdd(bins + u, to_fixed(s));
    u = -1;
    s = 0.0f;
  }
  __device__ __forceinline__ void add(unsigned long long* bins, int bucket, float v) {
    if (bucket != u) {
      flush(bins);
      u = bucket;
    }
    s += v;
  }
  // Eight scores at relative distances d, d + 1, ..., d + 7 (one bucket unless the run crosses a
  // bucket boundary or zero).
  template <bool BUCKET>
  __device__ __forceinline__ void add_run(unsigned long long* bins, int d, const float (&v)[8]) {
    if (!BUCKET) {
      add(bins, 0, ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7])));
      return;
    }
    const int ulo = rel_bucket(d), uhi = rel_bucket(d + 7);
    if ((d >= 0 || d + 7 <= 0) && ulo == uhi) {
      add(bins, ulo, ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7])));
    } else if (d >= 32) {
      // Buckets are at least 8 wide from distance 32 on, so the run crosses exactly one bucket edge:
      // distances below the first distance of bucket uhi go to ulo, the rest to uhi.
      const int k = rel_bucket_start(uhi) - d;  // 1..7
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lo += j < k ? v[j] : 0.0f;
        hi += j < k ? 0.0f : v[j];
      }
      add(bins, ulo, lo);
      add(bins, uhi, hi);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) add(bins, rel_bucket(d + j), v[j]);
    }
  }
};

// Pack element e (0..7) of four 8-element bf16 rows into 4 consecutive bf16 (a column slice).
__device__ __forceinline__ uint2 column4(const uint4 (&r)[4], int e) {
  auto half = [&](const uint4& x) -> uint32_t {
    uint32_t w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
  };
  return make_uint2(half(r[0]) | (half(r[1]) << 16), half(r[2]) | (half(r[3]) << 16));
}

}  // namespace jfa
