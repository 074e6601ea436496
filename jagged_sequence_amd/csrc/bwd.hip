// Backward pass of jagged attention on gfx950 (aihot.vn GEM page, "Jagged Sequence Flash
// Attention": efficient backward passes; kerneldigest.dev page, "Arquitectura del Sistema":
// backward-pass parallelisation). Two attention kernels, run in this order:
//   dQ:    one workgroup per (sequence, head, 128-query tile) work item, looping over 64-key tiles;
//          it also forms Delta = <dO_i, O_i> for the dK/dV kernel;
//   dK/dV: at head dim 128 a persistent kernel (one workgroup per CU) that takes (sequence, head,
//          128-key tile) items from per-XCD work queues and loops over 64-query tiles; at head dim 64,
//          or when every sequence has a single query tile, one workgroup per item.
// Both recompute the scores from Q, K and the forward log-sum-exp. dQ needs no atomics: each query
// tile has one owner. Split items write fp32 partials that fixed-order sums combine, so results do
// not depend on scheduling. The only atomics are the queue counters (which item runs where, never
// what is computed) and, for the optional bias gradient, 64-bit fixed-point sums whose integer
// additions give the same total in any order.
//
// Gradients (per visible pair, s = scale <q_i, k_j> + bias):
//   softmax: P = exp(s - lse_i), dP = <dO_i, v_j>, dS = P (dP - Delta_i), Delta_i = <dO_i, O_i>
//   GDPA:    P = act(s) / Lkv,   dP = <dO_i, v_j>, dS = dP act'(s) / Lkv
//   dV_j += P dO_i,  dK_j += scale dS q_i,  dQ_i += scale dS k_j
#include <type_traits>

#include <algorithm>

#include "device_common.h"
#include "tile_lds.h"

namespace jfa {
namespace {

// ---------------------------------------------------------------- Delta_i = <dO_i, O_i>
// Dot product of one lane's dO elements (NKB groups of 8: elements 16 kb + 0..7 from `base`) with the
// same elements of the forward output (bf16 or fp32), in fp32.
template <int NKB>
__device__ __forceinline__ float row_dot_out(const BwdArgs& a, size_t base, const bf16x8 (&df)[NKB]) {
  // The dtype branch sits outside the loops and every load is issued before the first use, so the
  // row costs one memory round trip rather than one per 16-byte piece.
  float acc = 0.0f;
  if (a.out_f32) {
    const float* op = reinterpret_cast<const float*>(a.out) + base;
    float4 x[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      x[kb][0] = *reinterpret_cast<const float4*>(op + 16 * kb);
      x[kb][1] = *reinterpret_cast<const float4*>(op + 16 * kb + 4);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const float o[8] = {x[kb][0].x, x[kb][0].y, x[kb][0].z, x[kb][0].w,
                          x[kb][1].x, x[kb][1].y, x[kb][1].z, x[kb][1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += (float)df[kb][j] * o[j];
    }
  } else {
    const uint16_t* op = reinterpret_cast<const uint16_t*>(a.out) + base;
    uint4 x[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) x[kb] = load16(op + 16 * kb);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint32_t xw[4] = {x[kb].x, x[kb].y, x[kb].z, x[kb].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc += (float)df[kb][2 * j] * __builtin_bit_cast(float, xw[j] << 16);
        acc += (float)df[kb][2 * j + 1] * __builtin_bit_cast(float, xw[j] & 0xffff0000u);
      }
    }
  }
  return acc;
}

// 4 rows x 8 dims of a [T, H, D] tensor: loaded so that one thread can store them both row-major
// (4 x 16 bytes) and transposed (8 x 8 bytes). Lanes take consecutive row groups (g fastest), so the
// transposed 8-byte writes of a wave spread over all LDS banks.
template <int D, int ROWS>
struct Units {
  static constexpr int CPR = D / 8;
  static constexpr int N = (ROWS / 4) * CPR;
  uint4 r[4];
};

template <int D, int ROWS>
__device__ __forceinline__ void load_units(Units<D, ROWS>& u, __amdgpu_buffer_rsrc_t src, int rs, int row0, int tid) {
  constexpr int CPR = D / 8, N = Units<D, ROWS>::N;
  constexpr int G = ROWS / 4;
  if (N >= kThreads || tid < N) {
    const int g = tid % G, dg = tid / G;
#pragma unroll
    for (int j = 0; j < 4; ++j) u.r[j] = buf_load16(src, (uint32_t)((row0 + 4 * g + j) * rs + dg * 8) * 2u);
  }
}

template <int D, int ROWS>
__device__ __forceinline__ void store_units(const Units<D, ROWS>& u, __bf16* rowmajor, int RS, __bf16* trans, int TS,
                                            int tid) {
  constexpr int N = Units<D, ROWS>::N, G = ROWS / 4;
  if (N >= kThreads || tid < N) {
    const int g = tid % G, dg = tid / G;
    if (rowmajor) {
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&rowmajor[(4 * g + j) * RS + dg * 8]) = u.r[j];
    }
    if (trans) {
#pragma unroll
      for (int e = 0; e < 8; ++e) *reinterpret_cast<uint2*>(&trans[(dg * 8 + e) * TS + 4 * g]) = column4(u.r, e);
    }
  }
}

// ---------------------------------------------------------------- dQ, query-tile parallel
template <int D>
struct alignas(16) DqSmem {
  static constexpr int RS = D + 8, TS = kDqBN + 8;
  __bf16 k[kDqBN * RS];
  __bf16 kt[D * TS];
  __bf16 v[kDqBN * RS];
  float tab[kBuckets];
  float diag[4][kDiagLen];
};

template <int D, int ACT, int BIAS, int MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a) {
  constexpr int BM = kDqBM, BN = kDqBN, NKB = D / 16, NDB = D / 32;
  constexpr int RS = DqSmem<D>::RS, TS = DqSmem<D>::TS;
  constexpr bool SOFTMAX = ACT == kSoftmax;
  constexpr bool CAUSAL = MASK == kMaskCausal, BAND = MASK == kMaskBand;
  __shared__ DqSmem<D> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const WorkRec w = load_item(a.dq_items, blockIdx.x);
  const int h = w.h, t = w.tile, k0 = w.lo, k1 = w.hi, slot = w.slot;
  const int qs = w.qs, Lq = w.Lq, ks = w.ks, Lkv = w.Lkv;
  const int rs = a.H * D;
  const int row0 = t * BM + wave * 32;
  const int qi = row0 + l32;
  // Band: this lane's row sees keys [klo, khi]; the wave's rows together see keys within
  // [wlo, whi], and every one of them sees all of [wlo_all, whi_all].
  int klo = 0, khi = 0, wlo = 0, whi = 0, wlo_all = 0, whi_all = 0;
  if (BAND) {
    klo = band_key_lo(qi, a.band);
    khi = band_key_hi(qi, Lkv, a.band);
    wlo = band_key_lo(row0, a.band);
    whi = band_key_hi(row0 + 31, Lkv, a.band);
    wlo_all = band_key_lo(row0 + 31, a.band);
    whi_all = band_key_hi(row0, Lkv, a.band);
  }

  const float inv_scale = 1.0f / a.scale;
  if (BIAS == kBiasBucket && tid < kBuckets) sm.tab[tid] = a.bias[h * kBuckets + tid];
  const float bias_c = (BIAS == kBiasScalar) ? a.bias[h] : 0.0f;
  const float acc0 = (BIAS == kBiasScalar && !SOFTMAX) ? bias_c * inv_scale : 0.0f;

  bf16x8 qf[NKB], df[NKB];
  {
    const __amdgpu_buffer_rsrc_t qr = slice_rsrc(a.q + (size_t)(a.q_shared ? 0 : qs) * rs + h * D, Lq, rs, D);
    const __amdgpu_buffer_rsrc_t gr = slice_rsrc(a.dout + (size_t)qs * rs + h * D, Lq, rs, D);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint32_t off = (uint32_t)(qi * rs + kb * 16 + hh * 8) * 2u;
      qf[kb] = as_bf16x8(buf_load16(qr, off));
      df[kb] = as_bf16x8(buf_load16(gr, off));
    }
  }
  float nlse2 = kNegInf, dlt = 0.0f;  // -lse in log2 units; -inf makes every P of the row 0
  if (SOFTMAX) {
    // Delta_i = <dO_i, O_i>: this lane's half of the row, then the other half from lane ^ 32. The
    // first piece of the query tile (w.first) also stores it for the dK/dV kernel, which runs after.
    float part = 0.0f;
    if (qi < Lq) {
      const float l = a.lse[(size_t)h * a.Tq + qs + qi];
      nlse2 = l == kNegInf ? kNegInf : -(l - (BIAS == kBiasScalar ? bias_c : 0.0f)) * kLog2e;
      part = row_dot_out<NKB>(a, ((size_t)(qs + qi) * a.H + h) * D + hh * 8, df);
    }
    dlt = part + __shfl_xor(part, 32);
    if (w.first && hh == 0 && qi < Lq) a.delta[(size_t)h * a.Tq + qs + qi] = dlt;
  }
  const float smul = SOFTMAX ? a.scale * kLog2e : a.scale;
  const float invL = Lkv > 0 ? 1.0f / (float)Lkv : 0.0f;

  f32x16 qacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) qacc[db] = f32x16{};

  const __amdgpu_buffer_rsrc_t kr = slice_rsrc(a.k + (size_t)ks * rs + h * D, Lkv, rs, D);
  const __amdgpu_buffer_rsrc_t vr = slice_rsrc(a.v + (size_t)ks * rs + h * D, Lkv, rs, D);
  Units<D, kDqBN> uk, uv;
  if (k0 < k1) {
    load_units<D, kDqBN>(uk, kr, rs, k0 * BN, tid);
    load_units<D, kDqBN>(uv, vr, rs, k0 * BN, tid);
  }
  for (int kt = k0; kt < k1; ++kt) {
    const int key0 = kt * BN;
    __syncthreads();
    store_units<D, kDqBN>(uk, sm.k, RS, sm.kt, TS, tid);
    store_units<D, kDqBN>(uv, sm.v, RS, nullptr, 0, tid);
    if (BIAS == kBiasBucket) fill_diag(sm.diag[wave], sm.tab, row0 - key0 - (BN - 1), inv_scale, lane);
    __syncthreads();
    if (kt + 1 < k1) {
      load_units<D, kDqBN>(uk, kr, rs, (kt + 1) * BN, tid);
      load_units<D, kDqBN>(uv, vr, rs, (kt + 1) * BN, tid);
    }

    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      if (BIAS == kBiasBucket) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const float* dv = &sm.diag[wave][63 - 32 * sb + l32 - 16 * c - 8 * hh];
#pragma unroll
          for (int j = 0; j < 8; ++j) sacc[sb][8 * c + j] = dv[-j];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] = acc0;
      }
      pacc[sb] = f32x16{};
      const __bf16* kp = &sm.k[(32 * sb + kappa(l32)) * RS + hh * 8];
      const __bf16* vp = &sm.v[(32 * sb + kappa(l32)) * RS + hh * 8];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc[sb] = mfma32(lds_load8(kp + kb * 16), qf[kb], sacc[sb]);
        pacc[sb] = mfma32(lds_load8(vp + kb * 16), df[kb], pacc[sb]);
      }
    }

    const bool need_mask = BAND ? (wlo_all > key0 || whi_all < key0 + BN - 1)
                                : (key0 + BN > Lkv) || (CAUSAL && key0 + BN - 1 > row0);
    float ds[2][16];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float d;
        if (SOFTMAX) {
          const float p = fast_exp2(__builtin_fmaf(sacc[sb][r], smul, nlse2));
          d = p * (pacc[sb][r] - dlt);
        } else {
          float f, g;
          act_fwd_grad<ACT>(sacc[sb][r] * smul, f, g);
          d = pacc[sb][r] * g * invL;
        }
        if (need_mask) {
          const int key = key0 + 32 * sb + acc_row(r, hh);
          d = (BAND ? (key < klo || key > khi) : (key >= Lkv || (CAUSAL && key > qi))) ? 0.0f : d;
        }
        ds[sb][r] = d;
      }
    }
    bf16x8 dsb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) dsb[c] = pack8(&ds[c >> 1][8 * (c & 1)]);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const __bf16* kp = &sm.kt[(32 * db + l32) * TS + 8 * hh];
#pragma unroll
      for (int c = 0; c < 4; ++c) qacc[db] = mfma32(lds_load8(kp + 16 * c), dsb[c], qacc[db]);
    }
  }

  if (slot < 0) {
    if (qi < Lq) {
      const size_t base = ((size_t)(qs + qi) * a.H + h) * D;
      const float sc = a.scale;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(a.dq, base + 32 * db + 8 * g + 4 * hh, qacc[db][4 * g] * sc, qacc[db][4 * g + 1] * sc,
                 qacc[db][4 * g + 2] * sc, qacc[db][4 * g + 3] * sc, a.grad_f32);
    }
  } else if (qi < Lq) {  // the fixed-order sums read the rows of the sequence only
    float* po = a.part_dq + ((size_t)slot * BM + wave * 32 + l32) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * g + 4 * hh) =
            make_float4(qacc[db][4 * g], qacc[db][4 * g + 1], qacc[db][4 * g + 2], qacc[db][4 * g + 3]);
  }
}

// D = 128 dQ with a two-stage LDS ring: K and V tiles are loaded straight into LDS (swizzled
// row-major) one tile ahead of the compute; K^T for dQ += dS K comes from transposing LDS reads.
struct alignas(16) DqSmem2 {
  unsigned char kv[2][2][kDqBN * kRowBytes];  // [stage][0 = K, 1 = V]
  float tab[kBuckets];
  float diag[4][kDiagLen];
};

template <int ACT, int BIAS, int MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel2(BwdArgs a) {
  constexpr int D = 128, BM = kDqBM, BN = kDqBN, NKB = D / 16, NDB = D / 32;
  constexpr bool SOFTMAX = ACT == kSoftmax;
  constexpr bool CAUSAL = MASK == kMaskCausal, BAND = MASK == kMaskBand;
  __shared__ DqSmem2 sm;

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The dK/dV kernel, which runs after this one, takes its items from a queue whose counters
  // start at zero.
  if (blockIdx.x == 0 && threadIdx.x < kQueueCounters && a.kv_queue) a.kv_queue[threadIdx.x] = 0;
  const WorkRec w = load_item(a.dq_items, blockIdx.x);
  const int h = w.h, t = w.tile, k0 = w.lo, k1 = w.hi, slot = w.slot;
  const int qs = w.qs, Lq = w.Lq, ks = w.ks, Lkv = w.Lkv;
  const int rs = a.H * D;
  const int row0 = t * BM + wave * 32;
  const int qi = row0 + l32;
  // Band: this lane's row sees keys [klo, khi]; the wave's rows together see keys within
  // [wlo, whi], and every one of them sees all of [wlo_all, whi_all].
  int klo = 0, khi = 0, wlo = 0, whi = 0, wlo_all = 0, whi_all = 0;
  if (BAND) {
    klo = band_key_lo(qi, a.band);
    khi = band_key_hi(qi, Lkv, a.band);
    wlo = band_key_lo(row0, a.band);
    whi = band_key_hi(row0 + 31, Lkv, a.band);
    wlo_all = band_key_lo(row0 + 31, a.band);
    whi_all = band_key_hi(row0, Lkv, a.band);
  }

  const float inv_scale = 1.0f / a.scale;
  // The bias table is written to LDS after the other prologue loads are issued (its round trip
  // overlaps theirs).
  const float tabv = (BIAS == kBiasBucket && tid < kBuckets) ? a.bias[h * kBuckets + tid] : 0.0f;
  const float bias_c = (BIAS == kBiasScalar) ? a.bias[h] : 0.0f;
  const float acc0 = (BIAS == kBiasScalar && !SOFTMAX) ? bias_c * inv_scale : 0.0f;

  // The first key tile is requested before anything else, so that its latency overlaps the
  // fragment loads and the Delta computation below.
  const __amdgpu_buffer_rsrc_t kr = slice_rsrc(a.k + (size_t)ks * rs + h * D, Lkv, rs, D);
  const __amdgpu_buffer_rsrc_t vr = slice_rsrc(a.v + (size_t)ks * rs + h * D, Lkv, rs, D);
  const TileLoader ld = make_loader64(wave, lane, rs);
  if (k0 < k1) {
    load_tile64(ld, kr, k0 * BN, rs, sm.kv[0][0], wave);
    load_tile64(ld, vr, k0 * BN, rs, sm.kv[0][1], wave);
  }

  bf16x8 qf[NKB], df[NKB];
  {
    const __amdgpu_buffer_rsrc_t qr = slice_rsrc(a.q + (size_t)(a.q_shared ? 0 : qs) * rs + h * D, Lq, rs, D);
    const __amdgpu_buffer_rsrc_t gr = slice_rsrc(a.dout + (size_t)qs * rs + h * D, Lq, rs, D);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint32_t off = (uint32_t)(qi * rs + kb * 16 + hh * 8) * 2u;
      qf[kb] = as_bf16x8(buf_load16(qr, off));
      df[kb] = as_bf16x8(buf_load16(gr, off));
    }
  }
  float nlse2 = kNegInf, dlt = 0.0f;  // -lse in log2 units; -inf makes every P of the row 0
  if (SOFTMAX) {
    // Delta_i = <dO_i, O_i>: this lane's half of the row, then the other half from lane ^ 32. The
    // first piece of the query tile (w.first) also stores it for the dK/dV kernel, which runs after.
    float part = 0.0f;
    if (qi < Lq) {
      const float l = a.lse[(size_t)h * a.Tq + qs + qi];
      nlse2 = l == kNegInf ? kNegInf : -(l - (BIAS == kBiasScalar ? bias_c : 0.0f)) * kLog2e;
      part = row_dot_out<NKB>(a, ((size_t)(qs + qi) * a.H + h) * D + hh * 8, df);
    }
    dlt = part + __shfl_xor(part, 32);
    if (w.first && hh == 0 && qi < Lq) a.delta[(size_t)h * a.Tq + qs + qi] = dlt;
  }
  const float smul = SOFTMAX ? a.scale * kLog2e : a.scale;
  const float invL = Lkv > 0 ? 1.0f / (float)Lkv : 0.0f;

  f32x16 qacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) qacc[db] = f32x16{};

  const uint32_t raddr = row_operand_base(kappa(l32), hh);
  uint32_t T[2];
  tr_operand_bases(lane, T);

  // Wave 0 writes the bias table; every wave reads it in the first tile's diagonal fill.
  if (BIAS == kBiasBucket) {
    if (tid < kBuckets) sm.tab[tid] = tabv;
    __syncthreads();
  }
  // One kv tile; ST (compile-time) is the ring stage holding it.
  auto tile = [&](const int kt, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    const int key0 = kt * BN;
    // A tile with no visible pair for this wave's rows (past the diagonal, or outside the band), or a
    // wave whose rows all lie past the sequence's end, contributes nothing.
    const bool wskip =
        row0 >= Lq || (CAUSAL ? key0 > row0 + 31 : (BAND ? (key0 > whi || key0 + BN - 1 < wlo) : false));
    wait_vm();
    // Bias of score (qi, key) at diag[31 - l32 + key - key0], ascending in register order.
    if (BIAS == kBiasBucket && !wskip)
      fill_diag(sm.diag[wave], sm.tab, key0 - row0 - 31, inv_scale, lane);
    __syncthreads();
    if (kt + 1 < k1) {
      load_tile64(ld, kr, (kt + 1) * BN, rs, sm.kv[ST ^ 1][0], wave);
      load_tile64(ld, vr, (kt + 1) * BN, rs, sm.kv[ST ^ 1][1], wave);
    }
    // Such a tile's work is skipped (the wave has taken part in the barrier and the loads above),
    // which leaves the SIMD to the other workgroup's wave.
    if (wskip) return;
    const unsigned char* Kt = sm.kv[ST][0];
    const unsigned char* Vt = sm.kv[ST][1];

    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      if (BIAS == kBiasBucket) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const float* dv = &sm.diag[wave][31 - l32 + 32 * sb + 16 * c + 8 * hh];
#pragma unroll
          for (int j = 0; j < 8; ++j) sacc[sb][8 * c + j] = dv[j];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] = acc0;
      }
      pacc[sb] = f32x16{};
    }
    // K and V operands are requested two steps ahead of their products (a step is one S and one dP
    // product), so each product finds its operand loaded instead of waiting for a read issued just
    // before it.
    bf16x8 kop[2 * NKB], vop[2 * NKB];
#pragma unroll
    for (int s = 0; s < 2 * NKB; ++s) {
      const uint32_t off = (raddr ^ (uint32_t)((s % NKB) << 5)) + (s / NKB) * 32 * kRowBytes;
      kop[s] = lds_read16(Kt, off);
      vop[s] = lds_read16(Vt, off);
    }
#pragma unroll
    for (int s = 0; s < 2 * NKB; ++s) {
      sacc[s / NKB] = mfma32(kop[s], qf[s % NKB], sacc[s / NKB]);
      pacc[s / NKB] = mfma32(vop[s], df[s % NKB], pacc[s / NKB]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + (BIAS == kBiasBucket ? 16 : 0), 0);
#pragma unroll
    for (int s = 0; s < 2 * NKB - 2; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

    const bool need_mask = BAND ? (wlo_all > key0 || whi_all < key0 + BN - 1)
                                : (key0 + BN > Lkv) || (CAUSAL && key0 + BN - 1 > row0);
    float ds[2][16];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float d;
        if (SOFTMAX) {
          const float p = fast_exp2(__builtin_fmaf(sacc[sb][r], smul, nlse2));
          d = p * (pacc[sb][r] - dlt);
        } else {
          float f, g;
          act_fwd_grad<ACT>(sacc[sb][r] * smul, f, g);
          d = pacc[sb][r] * g;  // (the 1 / Lkv of the GDPA gradient is applied to dQ at the end)
        }
        ds[sb][r] = d;
      }
    }
    if (need_mask) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * sb + acc_row(r, hh);
          ds[sb][r] = (BAND ? (key < klo || key > khi) : (key >= Lkv || (CAUSAL && key > qi))) ? 0.0f : ds[sb][r];
        }
    }
    bf16x8 dsb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) dsb[c] = pack8(&ds[c >> 1][8 * (c & 1)]);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t base = (uint32_t)(c * 16 * kRowBytes);
        qacc[db] = mfma32(lds_read_tr(Kt, base + (T[0] ^ (uint32_t)(64 * db)), base + (T[1] ^ (uint32_t)(64 * db))),
                          dsb[c], qacc[db]);
      }
  };
  for (int kt = k0; kt < k1; kt += 2) {
    tile(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < k1) tile(kt + 1, std::integral_constant<int, 1>{});
  }

  const float gscale = SOFTMAX ? 1.0f : invL;  // GDPA: the accumulators lack the factor 1 / Lkv of dS
  if (slot < 0 && !a.grad_f32) {
    // bf16 rows through the ring stage that the last tile did not use (every wave finished reading
    // it before the last tile's barrier, and no load went into it since): 8 KB per wave.
    const int free_st = ((k1 - 1 - k0) & 1) ^ 1;
    char* dst = static_cast<char*>(a.dq);
    const int H = a.H;
    store_rows_staged(&sm.kv[free_st][0][0] + wave * (32 * kRowBytes), qacc, a.scale * gscale, lane, Lq - row0,
                      [&](int r) { return dst + (((size_t)(qs + row0 + r) * H + h) * D) * 2; });
  } else if (slot < 0) {
    if (qi < Lq) {
      const size_t base = ((size_t)(qs + qi) * a.H + h) * D;
      const float sc = a.scale * gscale;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(a.dq, base + 32 * db + 8 * g + 4 * hh, qacc[db][4 * g] * sc, qacc[db][4 * g + 1] * sc,
                 qacc[db][4 * g + 2] * sc, qacc[db][4 * g + 3] * sc, a.grad_f32);
    }
  } else if (qi < Lq) {  // the fixed-order sums read the rows of the sequence only
    float* po = a.part_dq + ((size_t)slot * BM + wave * 32 + l32) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * g + 4 * hh) =
            make_float4(qacc[db][4 * g] * gscale, qacc[db][4 * g + 1] * gscale, qacc[db][4 * g + 2] * gscale,
                        qacc[db][4 * g + 3] * gscale);
  }
}

// ---------------------------------------------------------------- dK/dV, key-tile parallel
template <int D>
struct alignas(16) KvSmem {
  static constexpr int RS = D + 8, TS = kKvBM + 8;
  __bf16 q[kKvBM * RS];
  __bf16 qt[D * TS];
  __bf16 g[kKvBM * RS];
  __bf16 gt[D * TS];
  float lse2[kKvBM];
  float dlt[kKvBM];
  float tab[kBuckets];
  float diag[4][kDiagLen];
  unsigned long long dbh[4][kDbiasBins];  // per-wave bias-gradient bins (fixed point)
};

template <int D, int ACT, int BIASX, int MK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BM = kKvBM, BN = kKvBN, NKB = D / 16, NDB = D / 32;
  constexpr int RS = KvSmem<D>::RS, TS = KvSmem<D>::TS;
  constexpr bool SOFTMAX = ACT == kSoftmax;
  constexpr bool CAUSAL = MK == kMaskCausal, BAND = MK == kMaskBand;
  constexpr int BIAS = BIASX & 3;
  constexpr bool DBIAS = (BIASX & kBiasGrad) != 0;
  __shared__ KvSmem<D> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const WorkRec w = load_item(a.kv_items, blockIdx.x);
  const int h = w.h, kt = w.tile, q0 = w.lo, q1 = w.hi, slot = w.slot;
  const int qs = w.qs, Lq = w.Lq, ks = w.ks, Lkv = w.Lkv;
  const int rs = a.H * D;
  const int key_w = kt * BN + wave * 32;  // first key of this wave
  const int kj = key_w + l32;
  // Band: this lane's key is seen by rows [rlo, rhi]; every key of the wave by all of
  // [wr_all_lo, wr_all_hi].
  int rlo = 0, rhi = 0, wr_all_lo = 0, wr_all_hi = 0;
  if (BAND) {
    rlo = band_row_lo(kj, a.band);
    rhi = band_row_hi(kj, Lq, a.band);
    wr_all_lo = band_row_lo(key_w + 31, a.band);
    wr_all_hi = band_row_hi(key_w, Lq, a.band);
  }

  const float inv_scale = 1.0f / a.scale;
  if (BIAS == kBiasBucket && tid < kBuckets) sm.tab[tid] = a.bias[h * kBuckets + tid];
  DbiasLane dbl;
  if (DBIAS) sm.dbh[wave][lane] = 0ull;
  const float bias_c = (BIAS == kBiasScalar) ? a.bias[h] : 0.0f;
  const float acc0 = (BIAS == kBiasScalar && !SOFTMAX) ? bias_c * inv_scale : 0.0f;

  bf16x8 kf[NKB], vf[NKB];
  {
    const __amdgpu_buffer_rsrc_t kr = slice_rsrc(a.k + (size_t)ks * rs + h * D, Lkv, rs, D);
    const __amdgpu_buffer_rsrc_t vr = slice_rsrc(a.v + (size_t)ks * rs + h * D, Lkv, rs, D);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint32_t off = (uint32_t)(kj * rs + kb * 16 + hh * 8) * 2u;
      kf[kb] = as_bf16x8(buf_load16(kr, off));
      vf[kb] = as_bf16x8(buf_load16(vr, off));
    }
  }
  const float smul = SOFTMAX ? a.scale * kLog2e : a.scale;
  const float invL = Lkv > 0 ? 1.0f / (float)Lkv : 0.0f;
  const float lse_shift = (SOFTMAX && BIAS == kBiasScalar) ? bias_c : 0.0f;

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const __amdgpu_buffer_rsrc_t qsr = slice_rsrc(a.q + (size_t)(a.q_shared ? 0 : qs) * rs + h * D, Lq, rs, D);
  const __amdgpu_buffer_rsrc_t gsr = slice_rsrc(a.dout + (size_t)qs * rs + h * D, Lq, rs, D);
  Units<D, kKvBM> uq, ug;
  float pl = 0.0f, pd = 0.0f;
  auto load_stats = [&](int qt) {
    if (SOFTMAX && tid < BM) {
      const int q = qt * BM + tid;
      pl = kNegInf;  // -lse in log2 units; -inf makes P of rows past the end 0
      pd = 0.0f;
      if (q < Lq) {
        const float l = a.lse[(size_t)h * a.Tq + qs + q];
        pl = l == kNegInf ? kNegInf : -(l - lse_shift) * kLog2e;
        pd = a.delta[(size_t)h * a.Tq + qs + q];
      }
    }
  };
  if (q0 < q1) {
    load_units<D, kKvBM>(uq, qsr, rs, q0 * BM, tid);
    load_units<D, kKvBM>(ug, gsr, rs, q0 * BM, tid);
    load_stats(q0);
  }
  for (int qt = q0; qt < q1; ++qt) {
    const int qrow0 = qt * BM;
    __syncthreads();
    store_units<D, kKvBM>(uq, sm.q, RS, sm.qt, TS, tid);
    store_units<D, kKvBM>(ug, sm.g, RS, sm.gt, TS, tid);
    if (SOFTMAX && tid < BM) {
      sm.lse2[tid] = pl;
      sm.dlt[tid] = pd;
    }
    if (BIAS == kBiasBucket) fill_diag(sm.diag[wave], sm.tab, qrow0 - key_w - 31, inv_scale, lane);
    __syncthreads();
    if (qt + 1 < q1) {
      load_units<D, kKvBM>(uq, qsr, rs, (qt + 1) * BM, tid);
      load_units<D, kKvBM>(ug, gsr, rs, (qt + 1) * BM, tid);
      load_stats(qt + 1);
    }

    // Two 32-query blocks, one after the other (keeps the score temporaries of one block live):
    // S = Q K^T and dP = dO V^T with lane column = key kj and register r = query
    // qrow0 + 32 qb + acc_row(r, hh); then dV += P^T dO and dK += dS^T Q over those 32 queries.
    const bool need_mask = (key_w + 32 > Lkv) || (CAUSAL && key_w + 31 > qrow0) ||
                           (BAND && (wr_all_lo > qrow0 || wr_all_hi < qrow0 + BM - 1));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 sacc, pacc = f32x16{};
      if (BIAS == kBiasBucket) {
        // d = qi - kj = (qrow0 - key_w - 31) + (31 + 32 qb + 16 c + 8 hh + j - l32)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const float* dvp = &sm.diag[wave][31 + 32 * qb + 16 * c + 8 * hh - l32];
#pragma unroll
          for (int j = 0; j < 8; ++j) sacc[8 * c + j] = dvp[j];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = acc0;
      }
      const __bf16* qp = &sm.q[(32 * qb + kappa(l32)) * RS + hh * 8];
      const __bf16* gp = &sm.g[(32 * qb + kappa(l32)) * RS + hh * 8];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc = mfma32(lds_load8(qp + kb * 16), kf[kb], sacc);
        pacc = mfma32(lds_load8(gp + kb * 16), vf[kb], pacc);
      }

      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int c8 = 0; c8 < 2; ++c8) {
        const int rbase = 32 * qb + 16 * c8 + 8 * hh;  // 8 consecutive query rows of this lane
        float l8[8], d8[8], pv[8], dsv[8];
        if (SOFTMAX) {
          const float4 x0 = *reinterpret_cast<const float4*>(&sm.lse2[rbase]);
          const float4 x1 = *reinterpret_cast<const float4*>(&sm.lse2[rbase + 4]);
          const float4 y0 = *reinterpret_cast<const float4*>(&sm.dlt[rbase]);
          const float4 y1 = *reinterpret_cast<const float4*>(&sm.dlt[rbase + 4]);
          l8[0] = x0.x; l8[1] = x0.y; l8[2] = x0.z; l8[3] = x0.w; l8[4] = x1.x; l8[5] = x1.y; l8[6] = x1.z; l8[7] = x1.w;
          d8[0] = y0.x; d8[1] = y0.y; d8[2] = y0.z; d8[3] = y0.w; d8[4] = y1.x; d8[5] = y1.y; d8[6] = y1.z; d8[7] = y1.w;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * c8 + j;
          float pj, dj;
          if (SOFTMAX) {
            pj = fast_exp2(__builtin_fmaf(sacc[r], smul, l8[j]));
            dj = pj * (pacc[r] - d8[j]);
          } else {
            float f, g;
            act_fwd_grad<ACT>(sacc[r] * smul, f, g);
            pj = f * invL;
            dj = pacc[r] * g * invL;
          }
          if (need_mask || !SOFTMAX) {
            const int qi = qrow0 + rbase + j;
            const bool masked =
                (need_mask && (kj >= Lkv || (CAUSAL && kj > qi) || (BAND && (qi < rlo || qi > rhi)))) ||
                (!SOFTMAX && qi >= Lq);
            pj = masked ? 0.0f : pj;
            dj = masked ? 0.0f : dj;
          }
          pv[j] = pj;
          dsv[j] = dj;
        }
        pb[c8] = pack8(pv);
        dsb[c8] = pack8(dsv);
        if (DBIAS) dbl.add_run<BIAS == kBiasBucket>(sm.dbh[wave], qrow0 + rbase - kj, dsv);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const __bf16* gtp = &sm.gt[(32 * db + l32) * TS + 32 * qb + 8 * hh];
        const __bf16* qtp = &sm.qt[(32 * db + l32) * TS + 32 * qb + 8 * hh];
#pragma unroll
        for (int c8 = 0; c8 < 2; ++c8) {
          dv[db] = mfma32(lds_load8(gtp + 16 * c8), pb[c8], dv[db]);
          dk[db] = mfma32(lds_load8(qtp + 16 * c8), dsb[c8], dk[db]);
        }
      }
    }
  }

  if (DBIAS) {
    dbl.flush(sm.dbh[wave]);
    wave_lds_fence();
    constexpr int NB = BIAS == kBiasBucket ? kDbiasBins : 1;
    if (lane < NB) {
      const unsigned long long x = sm.dbh[wave][lane];
      if (x) atomicAdd(a.dbias_acc + (size_t)h * NB + lane, x);
    }
  }

  // Accumulator register r of d-block db: dimension 32 db + 8 (r/4) + 4 hh + r%4, key kj.
  if (slot < 0) {
    if (kj < Lkv) {
      const size_t base = ((size_t)(ks + kj) * a.H + h) * D;
      const float sc = a.scale;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const size_t i = base + 32 * db + 8 * g + 4 * hh;
          store4(a.dk, i, dk[db][4 * g] * sc, dk[db][4 * g + 1] * sc, dk[db][4 * g + 2] * sc, dk[db][4 * g + 3] * sc,
                 a.grad_f32);
          store4(a.dv, i, dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3], a.grad_f32);
        }
    }
  } else {
    const size_t prow = (size_t)slot * BN + wave * 32 + l32;
    float* pk = a.part_dk + prow * D;
    float* pv = a.part_dv + prow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = 32 * db + 8 * g + 4 * hh;
        *reinterpret_cast<float4*>(pk + i) = make_float4(dk[db][4 * g], dk[db][4 * g + 1], dk[db][4 * g + 2], dk[db][4 * g + 3]);
        *reinterpret_cast<float4*>(pv + i) = make_float4(dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]);
      }
  }
}

// D = 128 dK/dV with wave pairs. An 8-wave workgroup owns 128 keys; waves p and p + 4 share keys
// 32 p .. 32 p + 31 and sit on the same SIMD. Wave p (A) holds K and accumulates dV: S = Q K^T,
// P = softmax probabilities (or act(S)/Lkv), dV += P^T dO. Wave p + 4 (B) holds V and accumulates dK:
// dP = dO V^T, dS = P (dP - Delta) (or dP act'(S)/Lkv), dK += dS^T Q. P (and act'(S)/Lkv) pass from
// A to B through LDS between two barriers. Each wave keeps one operand and one accumulator set, so
// two waves fit per SIMD and A's exponentials overlap B's matrix products. Q and dO tiles are loaded
// straight into a two-stage LDS ring (swizzled row-major, no staging registers) one tile ahead of the
// compute; the Q^T and dO^T operands come from transposing LDS reads.
template <bool ONEBAR, bool GDPA, int NP>
struct alignas(16) KvSmem2;

// Two barriers per tile: a two-stage Q/dO ring and one hand-off buffer (NP wave pairs).
template <bool GDPA, int NP>
struct alignas(16) KvSmem2<false, GDPA, NP> {
  static constexpr int NPG = GDPA ? 2 : 1;      // P, and act'/Lkv for GDPA
  unsigned char qg[2][2][kKvBM * kRowBytes];    // [stage][0 = Q, 1 = dO]
  float lse2[2][kKvBM];                         // -lse in log2 units (softmax)
  float dlt[2][kKvBM];
  uint4 xch[1][NP][NPG][2][2][64];              // [buffer][pair][P / act'][q block][8-row half][lane]: 8 bf16
  float tab[kBuckets];
  float diag[NP][kDiagLen];
  unsigned long long dbh[NP][kDbiasBins];       // per-B-wave bias-gradient bins (fixed point)
  unsigned char bkt[2][NP][kDiagLen];           // bucket of every distance of the bias window
};

// One barrier per tile: a three-stage ring and three hand-off buffers (152 KB). The small arrays
// come first so that their LDS offsets fit the immediates of ds_read / ds_read2; the ring stages
// are reached through a wave-uniform base offset.
template <bool GDPA, int NP>
struct alignas(16) KvSmem2<true, GDPA, NP> {
  static constexpr int NPG = 1;  // P (softmax) or act'/Lkv (GDPA; A parks its own P in the next buffer)
  float diag[NP][kDiagLen];  // first: the 8-byte pair reads of a lane's bias window share one base
  float tab[kBuckets];
  unsigned long long dbh[NP][kDbiasBins];
  float lse2[3][kKvBM];
  float dlt[3][kKvBM];
  uint4 xch[3][NP][NPG][2][2][64];
  unsigned char qg[3][2][kKvBM * kRowBytes];
  unsigned char bkt[2][NP][kDiagLen];  // bucket of every distance of the bias window (tile parity)
};

// A wave-uniform value the compiler cannot fold into address immediates.
__device__ __forceinline__ uint32_t uniform_opaque(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// A per-lane value the compiler must treat as new at this point (so that what is derived from it
// is recomputed here instead of being kept live across the loop).
__device__ __forceinline__ int lane_opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void unpack8(uint4 w, float (&x)[8]) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __builtin_bit_cast(float, v[j] << 16);
    x[2 * j + 1] = __builtin_bit_cast(float, v[j] & 0xffff0000u);
  }
}

// The per-wave bias window (see fill_diag) together with the bucket of each of its distances, which
// the bias gradient of the same key block and query tile reads instead of computing them again.
__device__ __forceinline__ void fill_diag_buckets(float* vec, unsigned char* bkt, const float* tab, int d0, float mul,
                                                  int lane) {
  const int u0 = rel_bucket(d0 + lane);
  vec[lane] = tab[u0] * mul;
  bkt[lane] = (unsigned char)u0;
  if (lane < kDiagLen - 64) {
    const int u1 = rel_bucket(d0 + 64 + lane);
    vec[64 + lane] = tab[u1] * mul;
    bkt[64 + lane] = (unsigned char)u1;
  }
}

// DbiasLane::add_run for the bucket table with the buckets of distances d .. d + 7 read from bt[0..7].
__device__ __forceinline__ void add_run_buckets(DbiasLane& dbl, unsigned long long* bins, int d,
                                                const unsigned char* bt, const float (&v)[8]) {
  const int ulo = bt[0], uhi = bt[7];
  if ((d >= 0 || d + 7 <= 0) && ulo == uhi) {
    dbl.add(bins, ulo, ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7])));
  } else if (d >= 32) {
    // buckets are at least 8 wide from distance 32 on: one edge inside the run
    const int k = rel_bucket_start(uhi) - d;  // 1..7
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo += j < k ? v[j] : 0.0f;
      hi += j < k ? 0.0f : v[j];
    }
    dbl.add(bins, ulo, lo);
    dbl.add(bins, uhi, hi);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) dbl.add(bins, bt[j], v[j]);
  }
}

// NP wave pairs per workgroup own NP x 32 keys: NP = 4 (128 keys, 8 waves, one workgroup per CU) in
// general; NP = 2 (64 keys, 4 waves, two workgroups per CU, about 75 KB of LDS) when every sequence
// has a single query tile, where an item is one latency-bound pass and two resident workgroups
// overlap one's loads with the other's work.
// With NP = 4 the hand-off carries one array per tile (P for softmax; act'/Lkv for GDPA, whose A
// wave parks its own P in the next tile's buffer), so a third ring stage and three hand-off buffers fit in LDS
// and one barrier per query tile suffices. The short form (NP = 2), whose items have a single query
// tile, keeps two barriers per tile.
template <int ACT, int NP>
struct DkdvShape {
  static constexpr bool ONEBAR = NP == 4;
  using Smem = KvSmem2<ONEBAR, ACT != kSoftmax, NP>;
};

// One dK/dV item (the key tile and query-tile range at position `item` of the list) by the whole
// workgroup. Its first LDS access follows a barrier that every wave has passed after the previous
// item's last LDS access.
// Work-queue hooks: `claim_next()` runs when the item's tile loop ends and `take_next(token)` after
// its epilogue, so that the queue's round trip overlaps the epilogue's stores. (Claiming earlier
// would hide it better but would hold the claimed item back for a whole item, which lengthens the
// tail of the run.)
template <int ACT, int BIASX, int MK, int NP, class Claim, class Take>
__device__ __forceinline__ void dkdv_item2(const __attribute__((address_space(4))) BwdArgs& a,
                                           typename DkdvShape<ACT, NP>::Smem& sm, int item, const int wave,
                                           Claim claim_next, Take take_next) {
  constexpr int D = 128, BM = kKvBM, BN = 32 * NP, NKB = D / 16, NDB = D / 32;
  constexpr int BIAS = BIASX & 3;
  constexpr bool DBIAS = (BIASX & kBiasGrad) != 0;
  constexpr bool SOFTMAX = ACT == kSoftmax;
  constexpr bool ONEBAR = DkdvShape<ACT, NP>::ONEBAR;
  // GDPA with one barrier per tile hands B only act'/Lkv (in buffer t % 3) and parks A's own P of
  // tile t in buffer (t + 1) % 3: nobody reads that buffer between A's phase 1 of t and A's phase 2 of
  // t (B read it for tile t - 2, before the barrier of tile t - 1), and A itself overwrites it with
  // act'/Lkv of tile t + 1 only after phase 2 of t.
  constexpr bool P_NEXT = ONEBAR && ACT != kSoftmax;
  constexpr bool CAUSAL = MK == kMaskCausal, BAND = MK == kMaskBand;
  using Smem = typename DkdvShape<ACT, NP>::Smem;

  // Lane constants are derived anew for every item from the lane counter (no register holds the
  // thread index across the persistent loop, and nothing derived from it is hoisted out of it).
  // lane_now() recomputes the lane index (two VALU) where a use sits far from the others.
  auto lane_now = [] { return lane_opaque((int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u))); };
  const int lane = lane_now();
  const int tid = wave * 64 + lane, hh = lane >> 5, l32 = lane & 31;
  const int pair = wave % NP;
  const bool isB = wave >= NP;
  const WorkRec w = load_item(a.kv_items, item);
  const int h = w.h, kt = w.tile, q0 = w.lo, q1 = w.hi, slot = w.slot;
  const int qs = w.qs, Lq = w.Lq, ks = w.ks, Lkv = w.Lkv;
  const int rs = a.H * D;
  const int key_w = kt * BN + pair * 32;  // first key of this pair
  const int kj = key_w + l32;
  // Band: every key of the pair is seen by all rows of [wr_all_lo, wr_all_hi] (wave-uniform). The
  // limits are read from the argument segment where they are used.
  auto band = [&] { return Band{a.band.window, a.band.block, a.band.causal}; };
  int wr_all_lo = 0, wr_all_hi = 0;
  if (BAND) {
    wr_all_lo = band_row_lo(key_w + 31, band());
    wr_all_hi = band_row_hi(key_w, Lq, band());
  }

  const float inv_scale = 1.0f / a.scale;
  // The bias table (256 bytes) comes into LDS by the same kind of load as the tiles (wave 0), so
  // no register waits for it; the prologue's wait and barrier publish it.
  auto load_table = [&] {
    if (BIAS == kBiasBucket && wave == 0) {
      const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.bias) + h * kBuckets,
                                                                          (short)0, kBuckets * 4, 0x00020000);
      dma4(tr, (uint32_t)lane_now() * 4u, sm.tab);
    }
  };
  DbiasLane dbl;  // B waves: running bias-gradient sum of this lane
  if (DBIAS && isB) sm.dbh[pair][lane] = 0ull;
  const float bias_c = (BIAS == kBiasScalar) ? a.bias[h] : 0.0f;
  const float acc0 = (BIAS == kBiasScalar && !SOFTMAX) ? bias_c * inv_scale : 0.0f;

  bf16x8 frag[NKB];  // A: K fragment, B: V fragment (B operand, lane = key)
  {
    const __amdgpu_buffer_rsrc_t fr = slice_rsrc((isB ? a.v : a.k) + (size_t)ks * rs + h * D, Lkv, rs, D);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) frag[kb] = as_bf16x8(buf_load16(fr, (uint32_t)(kj * rs + kb * 16 + hh * 8) * 2u));
  }
  const float smul = SOFTMAX ? a.scale * kLog2e : a.scale;
  const float invL = Lkv > 0 ? 1.0f / (float)Lkv : 0.0f;
  const float lse_shift = (SOFTMAX && BIAS == kBiasScalar) ? bias_c : 0.0f;

  f32x16 acc[NDB];  // A: dV, B: dK (unscaled)
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  const __amdgpu_buffer_rsrc_t qsr = slice_rsrc(a.q + (size_t)(a.q_shared ? 0 : qs) * rs + h * D, Lq, rs, D);
  const __amdgpu_buffer_rsrc_t gsr = slice_rsrc(a.dout + (size_t)qs * rs + h * D, Lq, rs, D);
  const uint32_t raddr = row_operand_base(kappa(l32), hh);
  uint32_t T[2];
  tr_operand_bases(lane, T);

  // Statistics of a query tile (softmax): lse and Delta of its 64 rows come into the tile's stage
  // with the tile itself (one 256-byte load each, by wave 0). After the wait that precedes the
  // tile's publishing barrier, wave 0 turns lse into -lse in log2 units in place (rows past the end
  // read zeros and get -inf, which makes their P 0) and Delta into -Delta, the initial value of the
  // B waves' dP accumulators, so that dP - Delta comes out of the products.
  const __amdgpu_buffer_rsrc_t lser =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.lse) + (size_t)h * a.Tq + qs, (short)0, Lq * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t dltr =
      __builtin_amdgcn_make_buffer_rsrc(a.delta + (size_t)h * a.Tq + qs, (short)0, Lq * 4, 0x00020000);
  auto fix_stats = [&](int qt, int stg) {
    if (SOFTMAX && wave == 0) {
      const int r = lane_now();
      const float x = sm.lse2[stg][r];
      sm.lse2[stg][r] = (qt * BM + r < Lq && x != kNegInf) ? -(x - lse_shift) * kLog2e : kNegInf;
      sm.dlt[stg][r] = -sm.dlt[stg][r];
    }
  };
  auto issue_tile = [&](int qt, int stg) {
    if (SOFTMAX && wave == 0) {
      const uint32_t so = (uint32_t)(qt * BM + lane_now()) * 4u;
      dma4(lser, so, sm.lse2[stg]);
      dma4(dltr, so, sm.dlt[stg]);
    }
    // loader offsets recomputed per tile (two VALU each) rather than held in registers
    if constexpr (NP == 4) {
      const TileLoader ld = make_loader64_w8(wave, lane_now(), rs);
      load_tile64_w8(ld, qsr, qt * BM, rs, sm.qg[stg][0], wave);
      load_tile64_w8(ld, gsr, qt * BM, rs, sm.qg[stg][1], wave);
    } else {
      const TileLoader ld = make_loader64(wave, lane_now(), rs);
      load_tile64(ld, qsr, qt * BM, rs, sm.qg[stg][0], wave);
      load_tile64(ld, gsr, qt * BM, rs, sm.qg[stg][1], wave);
    }
  };
  auto fill = [&](int qt) {
    if (BIAS == kBiasBucket && !isB) {
      if constexpr (DBIAS)
        fill_diag_buckets(sm.diag[pair], sm.bkt[qt & 1][pair], sm.tab, qt * BM - key_w - 31, inv_scale, lane_now());
      else
        fill_diag(sm.diag[pair], sm.tab, qt * BM - key_w - 31, inv_scale, lane_now());
    }
  };

  auto stage_ptr = [&](auto st_tag, int which) -> const unsigned char* {
    constexpr int ST = decltype(st_tag)::value;
    if constexpr (ONEBAR)
      return sm.qg[0][which] + uniform_opaque((uint32_t)(ST * 2 * kKvBM * kRowBytes));
    else
      return sm.qg[ST][which];
  };

  // ---- phase 1. A: S = Q K^T, probabilities, hand-off to B. B: dP = dO V^T.
  auto phase1 = [&](const int qt, auto st_tag, auto xb_tag, f32x16 (&pacc)[2]) {
    constexpr int ST = decltype(st_tag)::value, XB = decltype(xb_tag)::value;
    constexpr int PB = P_NEXT ? (XB + 1) % 3 : XB;  // buffer of A's P
    const int qrow0 = qt * BM;
    const unsigned char* Qt = stage_ptr(st_tag, 0);
    const unsigned char* Gt = stage_ptr(st_tag, 1);
    if (!isB) {
      auto run = [&](auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        // Band: rows [rlo, rhi] see this lane's key (derived here, on masked tiles only).
        int rlo = 0, rhi = 0;
        if (MASK && BAND) {
          const int kjm = key_w + (lane_now() & 31);
          rlo = band_row_lo(kjm, band());
          rhi = band_row_hi(kjm, Lq, band());
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          f32x16 sacc;
          if (BIAS == kBiasBucket) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const float* dvp = &sm.diag[pair][31 + 32 * qb + 16 * c + 8 * hh - l32];
#pragma unroll
              for (int j = 0; j < 8; ++j) sacc[8 * c + j] = dvp[j];
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = acc0;
          }
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            sacc = mfma32(lds_read16(Qt, (raddr ^ (uint32_t)(kb << 5)) + qb * 32 * kRowBytes), frag[kb], sacc);
#pragma unroll
          for (int c8 = 0; c8 < 2; ++c8) {
            const int rbase = 32 * qb + 16 * c8 + 8 * hh;  // 8 consecutive query rows of this lane
            float pv[8], gv[8];
            if (SOFTMAX) {
              const float* ls = sm.lse2[ST];
              const float4 x0 = *reinterpret_cast<const float4*>(&ls[rbase]);
              const float4 x1 = *reinterpret_cast<const float4*>(&ls[rbase + 4]);
              const float l8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
              for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(__builtin_fmaf(sacc[8 * c8 + j], smul, l8[j]));
            } else {
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                float f, g;
                act_fwd_grad<ACT>(sacc[8 * c8 + j] * smul, f, g);
                pv[j] = f;  // (the 1 / Lkv of GDPA is applied to dV and dK at the end)
                gv[j] = g;
              }
            }
            // Rows past the sequence's end need no mask: their dO rows read as zeros, so they add
            // nothing to dV and their dP, hence dS, is zero (softmax: their P is zero already).
            if (MASK) {
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                // row index from a fresh lane index: this path runs on diagonal tiles only
                const int qi = qrow0 + 32 * qb + 16 * c8 + 8 * (lane_now() >> 5) + j;
                const bool masked = kj >= Lkv || (CAUSAL && kj > qi) || (BAND && (qi < rlo || qi > rhi));
                pv[j] = masked ? 0.0f : pv[j];
                if (!SOFTMAX) gv[j] = masked ? 0.0f : gv[j];
              }
            }
            sm.xch[PB][pair][0][qb][c8][lane] = __builtin_bit_cast(uint4, pack8(pv));
            if (!SOFTMAX) sm.xch[XB][pair][Smem::NPG - 1][qb][c8][lane] = __builtin_bit_cast(uint4, pack8(gv));
          }
        }
      };
      if ((key_w + 32 > Lkv) || (CAUSAL && key_w + 31 > qrow0) ||
          (BAND && (wr_all_lo > qrow0 || wr_all_hi < qrow0 + BM - 1)))
        run(std::true_type{});
      else
        run(std::false_type{});
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (SOFTMAX) {
          // -Delta of the accumulator's rows (register 8 c + j: row 32 qb + 16 c + 8 hh + j)
#pragma unroll
          for (int c8 = 0; c8 < 2; ++c8) {
            const float* dl = &sm.dlt[ST][32 * qb + 16 * c8 + 8 * hh];
            const float4 y0 = *reinterpret_cast<const float4*>(dl);
            const float4 y1 = *reinterpret_cast<const float4*>(dl + 4);
            pacc[qb][8 * c8 + 0] = y0.x; pacc[qb][8 * c8 + 1] = y0.y; pacc[qb][8 * c8 + 2] = y0.z;
            pacc[qb][8 * c8 + 3] = y0.w; pacc[qb][8 * c8 + 4] = y1.x; pacc[qb][8 * c8 + 5] = y1.y;
            pacc[qb][8 * c8 + 6] = y1.z; pacc[qb][8 * c8 + 7] = y1.w;
          }
        } else {
          pacc[qb] = f32x16{};
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          pacc[qb] = mfma32(lds_read16(Gt, (raddr ^ (uint32_t)(kb << 5)) + qb * 32 * kRowBytes), frag[kb], pacc[qb]);
      }
    }
  };

  // ---- phase 2. A: dV += P^T dO (P read back from the hand-off buffer). B: dS, dK += dS^T Q.
  auto phase2 = [&](const int qt, auto st_tag, auto xb_tag, const f32x16 (&pacc)[2]) {
    constexpr int ST = decltype(st_tag)::value, XB = decltype(xb_tag)::value;
    constexpr int PB = P_NEXT ? (XB + 1) % 3 : XB;  // buffer of A's P
    const int qrow0 = qt * BM;
    const unsigned char* Qt = stage_ptr(st_tag, 0);
    const unsigned char* Gt = stage_ptr(st_tag, 1);
    if (!isB) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int c8 = 0; c8 < 2; ++c8) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, sm.xch[PB][pair][0][qb][c8][lane]);
          const uint32_t base = (uint32_t)((32 * qb + 16 * c8) * kRowBytes);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = mfma32(lds_read_tr(Gt, base + (T[0] ^ (uint32_t)(64 * db)), base + (T[1] ^ (uint32_t)(64 * db))),
                             pb, acc[db]);
        }
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        bf16x8 dsb[2];
#pragma unroll
        for (int c8 = 0; c8 < 2; ++c8) {
          float dsv[8];
          if (SOFTMAX) {
            float pv[8];
            unpack8(sm.xch[XB][pair][0][qb][c8][lane], pv);
#pragma unroll
            for (int j = 0; j < 8; ++j) dsv[j] = pv[j] * pacc[qb][8 * c8 + j];  // pacc = dP - Delta
          } else {
            float gv[8];
            unpack8(sm.xch[XB][pair][Smem::NPG - 1][qb][c8][lane], gv);
#pragma unroll
            for (int j = 0; j < 8; ++j) dsv[j] = pacc[qb][8 * c8 + j] * gv[j];
          }
          dsb[c8] = pack8(dsv);
          if (DBIAS) {
            if (!SOFTMAX)
#pragma unroll
              for (int j = 0; j < 8; ++j) dsv[j] *= invL;
            const int d = qrow0 + 32 * qb + 16 * c8 + 8 * hh - kj;
            if constexpr (BIAS == kBiasBucket)  // distance d sits at 31 + d - qrow0 + key_w of A's window
              add_run_buckets(dbl, sm.dbh[pair], d, &sm.bkt[qt & 1][pair][31 + 32 * qb + 16 * c8 + 8 * hh - l32], dsv);
            else
              dbl.add_run<false>(sm.dbh[pair], d, dsv);
          }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int c8 = 0; c8 < 2; ++c8) {
            const uint32_t base = (uint32_t)((32 * qb + 16 * c8) * kRowBytes);
            acc[db] = mfma32(lds_read_tr(Qt, base + (T[0] ^ (uint32_t)(64 * db)), base + (T[1] ^ (uint32_t)(64 * db))),
                             dsb[c8], acc[db]);
          }
      }
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if constexpr (ONEBAR) {
    // Tile t lives in ring stage and hand-off buffer (t - q0) % 3. Step t: phase 1 of t; wait for
    // tile t+1 (loaded during step t-1) and publish its statistics; barrier; load tile t+2 into the
    // stage tile t-1 used; phase 2 of t. Every wave is past phase 2 of t-1 when the barrier of step
    // t releases, so the stage and buffers it overwrites are free, and A's phase 1 of t+1 may run
    // while B still finishes phase 2 of t.
    if (q0 < q1) issue_tile(q0, 0);
    if (q0 + 1 < q1) issue_tile(q0 + 1, 1);
    load_table();
    wait_vm();
    if (q0 < q1) fix_stats(q0, 0);
    __syncthreads();  // also publishes wave 0's bias table, which the first fill reads
    if (q0 < q1) fill(q0);  // the A wave reads its own window: no barrier needed before phase 1
    auto step = [&](const int qt, auto st_tag) {
      constexpr int ST = decltype(st_tag)::value;
      f32x16 pacc[2];
      phase1(qt, st_tag, st_tag, pacc);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm();
      if (qt + 1 < q1) fix_stats(qt + 1, (ST + 1) % 3);
      __syncthreads();
      if (qt + 2 < q1) issue_tile(qt + 2, (ST + 2) % 3);
      phase2(qt, st_tag, st_tag, pacc);
      if (qt + 1 < q1) fill(qt + 1);
      // Keep the compiler from hoisting the next tile's loads into this phase (register pressure).
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int qt = q0; qt < q1; qt += 3) {
      step(qt, I0{});
      if (qt + 1 < q1) step(qt + 1, I1{});
      if (qt + 2 < q1) step(qt + 2, I2{});
    }
  } else {
    // Two barriers per tile: the first publishes the tile and retires the other stage, the second
    // publishes the hand-off buffer.
    if (q0 < q1) issue_tile(q0, 0);
    load_table();
    // Wave 0 loads the bias table (and the B waves cleared their gradient bins); A waves read the
    // table in the first tile's diagonal fill.
    if (BIAS == kBiasBucket) {
      wait_vm();
      __syncthreads();
    }
    auto step = [&](const int qt, auto st_tag) {
      constexpr int ST = decltype(st_tag)::value;
      wait_vm();
      fix_stats(qt, ST);
      fill(qt);
      __syncthreads();
      if (qt + 1 < q1) issue_tile(qt + 1, ST ^ 1);
      f32x16 pacc[2];
      phase1(qt, st_tag, I0{}, pacc);
      __syncthreads();
      phase2(qt, st_tag, I0{}, pacc);
    };
    for (int qt = q0; qt < q1; qt += 2) {
      step(qt, I0{});
      if (qt + 1 < q1) step(qt + 1, I1{});
    }
  }

  const int token = claim_next();
  // The epilogue derives its lane values afresh: kept from the prologue they would be spilled
  // across the item, and their reloads here would make the next item's first loads wait.
  const int le = lane_now(), hhe = le >> 5, kje = key_w + (le & 31);
  if (DBIAS && isB) {
    dbl.flush(sm.dbh[pair]);
    wave_lds_fence();
    constexpr int NB = BIAS == kBiasBucket ? kDbiasBins : 1;
    if (le < NB) {
      const unsigned long long x = sm.dbh[pair][le];
      if (x) atomicAdd(a.dbias_acc + (size_t)h * NB + le, x);
    }
  }

  // Accumulator register r of d-block db: dimension 32 db + 8 (r/4) + 4 hh + r%4, key kj. GDPA: the
  // accumulators lack the factor 1 / Lkv of P and dS.
  const float gscale = SOFTMAX ? 1.0f : (Lkv > 0 ? 1.0f / (float)Lkv : 0.0f);
  const float sc = (isB ? a.scale : 1.0f) * gscale;
  if (slot < 0 && !a.grad_f32) {
    // bf16 rows go out through LDS as whole rows. Once every wave is past the last tile the Q / dO
    // ring is free: 8 KB per wave.
    __syncthreads();
    char* dst = static_cast<char*>(isB ? a.dk : a.dv);
    const int H = a.H;
    store_rows_staged(&sm.qg[0][0][0] + wave * (32 * kRowBytes), acc, sc, le, Lkv - key_w,
                      [&](int r) { return dst + (((size_t)(ks + key_w + r) * H + h) * D) * 2; });
  } else if (slot < 0) {
    if (kje < Lkv) {
      void* dst = isB ? a.dk : a.dv;
      const size_t base = ((size_t)(ks + kje) * a.H + h) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(dst, base + 32 * db + 8 * g + 4 * hhe, acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc,
                 acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc, a.grad_f32);
    }
  } else {
    float* pp = (isB ? a.part_dk : a.part_dv) + ((size_t)slot * BN + pair * 32 + (le & 31)) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(pp + 32 * db + 8 * g + 4 * hhe) =
            make_float4(acc[db][4 * g] * gscale, acc[db][4 * g + 1] * gscale, acc[db][4 * g + 2] * gscale,
                        acc[db][4 * g + 3] * gscale);
  }
  take_next(token);
}

// dQ of one split group (b, h, tile, slot0, R) by NT threads: NT / BM threads per row, each summing
// its columns over r = 0..R-1 in that order.
template <int D, int NT>
__device__ __forceinline__ void reduce_dq_group(const WorkRec& g, const float* part_dq, void* dq, int H, float scale,
                                                int grad_f32, int tid) {
  constexpr int BM = kDqBM, TPR = NT / BM, COLS = D / TPR;
  const int h = g.h, t = g.tile, slot0 = g.lo, R = g.hi;
  const int row = tid / TPR, part = tid % TPR;
  const int qi = t * BM + row;
  if (qi >= g.Lq) return;
  float acc[COLS];
#pragma unroll
  for (int d = 0; d < COLS; ++d) acc[d] = 0.0f;
  for (int r = 0; r < R; ++r) {
    const float* p = part_dq + ((size_t)(slot0 + r) * BM + row) * D + part * COLS;
#pragma unroll
    for (int d = 0; d < COLS; d += 4) {
      float4 x = *reinterpret_cast<const float4*>(p + d);
      acc[d] += x.x; acc[d + 1] += x.y; acc[d + 2] += x.z; acc[d + 3] += x.w;
    }
  }
  const size_t base = ((size_t)(g.qs + qi) * H + h) * D + part * COLS;
#pragma unroll
  for (int d = 0; d < COLS; d += 4)
    store4(dq, base + d, acc[d] * scale, acc[d + 1] * scale, acc[d + 2] * scale, acc[d + 3] * scale, grad_f32);
}

// Work queue of the dK/dV kernel. The items, in dispatch order, are dealt into kQueues queues:
// position p goes to queue p % kQueues, the XCD whose L2 the dispatch order keeps the item's sequence
// in. A workgroup takes items from the queue of the XCD it runs on and, once that is exhausted, from
// the others; the counters only grow, so every item is taken exactly once and every workgroup
// reaches the end when all queues are exhausted. Used by lane 0 of wave 0 only.
struct ItemQueue {
  int* ctr;        // kQueues counters, zero when the kernel starts
  int n;           // items in the list
  int home;        // queue of this workgroup's XCD
  unsigned empty;  // queues seen exhausted
  __device__ int claim(int x) { return __hip_atomic_fetch_add(ctr + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
  // list position of index i of queue x, or -1 (and x noted as exhausted)
  __device__ int position(int x, int i) {
    const int p = x + kQueues * i;
    if (i >= 0 && p < n) return p;  // (a negative index can only come from uncleared counters)
    empty |= 1u << x;
    return -1;
  }
  __device__ int next() {
#pragma nounroll
    for (int k = 0; k < kQueues; ++k) {
      const int x = (home + k) % kQueues;
      if (empty & (1u << x)) continue;
      const int p = position(x, claim(x));
      if (p >= 0) return p;
    }
    return -1;
  }
};

__device__ __forceinline__ int xcd_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(20, 0, 4)" : "=s"(v));  // XCC_ID
  return (int)v;
}

// Persistent dK/dV kernel (NP = 4): as many workgroups as the GPU holds at once, each running items
// from the work queue until none is left. Next to one workgroup per item this removes the gap between a
// workgroup's end and the next one's start, and the queue balances what the items really cost.
template <int ACT, int BIASX, int MK, int NP>
__global__ __attribute__((amdgpu_flat_work_group_size(NP * 128, NP * 128), amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel2(BwdArgs a) {
  __shared__ typename DkdvShape<ACT, NP>::Smem sm;
  __shared__ int next_item;
  __shared__ unsigned empty_queues;
  // The arguments are read through a pointer made opaque at every item, so that they are loaded
  // again (scalar loads) for each item instead of being held in registers across the whole loop;
  // likewise the queue state lives in LDS and the XCD is read again where needed.
  typedef const __attribute__((address_space(4))) BwdArgs* ArgPtr;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (NP == 2) {
    // The short form (single-tile items, two workgroups per CU) runs one item per workgroup: the
    // second resident workgroup already covers one's start and end, and the queue would only add
    // its round trips.
    ArgPtr ap = (ArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
    dkdv_item2<ACT, BIASX, MK, NP>(*ap, sm, blockIdx.x, wave, [] { return 0; }, [](int) {});
    return;
  }
  if (threadIdx.x == 0) {
    ItemQueue q{a.kv_queue, a.kv_n, xcd_id() % kQueues, 0u};
    next_item = q.next();
    empty_queues = q.empty;
  }
  __syncthreads();
  for (;;) {
    const int item = __builtin_amdgcn_readfirstlane(next_item);
    if (item < 0) break;
    // BwdArgs is the kernel's only argument: it starts the kernel-argument segment
    ArgPtr ap = (ArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ap));
    auto leader = [&]() { return wave == 0 && __builtin_amdgcn_mbcnt_lo(~0u, 0u) == 0; };
    // The home queue's next index is claimed when the item's tile loop ends and resolved after its
    // epilogue (or, with the home queue exhausted, an item is taken from another queue).
    auto claim = [&]() -> int {
      const int home = xcd_id() % kQueues;
      if (!leader() || (empty_queues & (1u << home))) return -1;
      // (the opaque zero keeps the compiler from rewriting the uniform-address atomic into a
      // wave-wide one whose result it would wait for on the spot)
      return __hip_atomic_fetch_add(ap->kv_queue + home + lane_opaque(0), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto take = [&](int claimed) {
      if (!leader()) return;
      const int home = xcd_id() % kQueues;
      ItemQueue q{ap->kv_queue, ap->kv_n, home, empty_queues};
      int p = claimed >= 0 ? q.position(home, claimed) : -1;
      if (p < 0) p = q.next();
      next_item = p;
      empty_queues = q.empty;
    };
    dkdv_item2<ACT, BIASX, MK, NP>(*ap, sm, item, wave, claim, take);
    __syncthreads();
  }
  // The fixed-order sums of split dQ pieces (written by the dQ kernel, which has finished) are taken
  // here by the workgroups that run out of items first, in the time the others finish theirs.
  __syncthreads();  // every wave has read the last next_item before it is reused
  ArgPtr ap = (ArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(ap));
  const int n_red = ap->dq_reduce_n;
  for (;;) {
    if (threadIdx.x == 0)
      next_item = n_red > 0 ? __hip_atomic_fetch_add(ap->kv_queue + kQueues, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : 0;
    __syncthreads();
    const int gi = __builtin_amdgcn_readfirstlane(next_item);
    __syncthreads();  // everyone has read next_item before it is written again
    if (gi >= n_red) break;
    reduce_dq_group<128, NP * 128>(load_group(ap->dq_groups, gi), ap->part_dq, ap->dq, ap->H, ap->scale, ap->grad_f32,
                                   threadIdx.x);
  }
}

// ---------------------------------------------------------------- fused backward, short query sets
// D = 128, every sequence with at most 64 queries (a single query tile). One workgroup per dQ item
// (sequence, head, range of 64-key tiles) keeps the sequence's Q and dO tiles in LDS for the whole
// item and streams the range's K and V tiles through a three-stage ring, each tile read once. Per
// tile: waves 0-1 (A) form S = Q K^T and P for keys 32 a .. 32 a + 31 and dV = P^T dO; waves 2-3 (B)
// form dP = dO V^T, dS and dK = dS^T Q for the same keys (softmax: A hands B the probabilities and
// dS = P (dP - Delta); GDPA: A hands B act'(S) / Lkv and dS = dP act'(S) / Lkv); all four waves
// then add dS K to dQ (wave w: dimensions 32 w .. 32 w + 31). Since every query of the sequence is
// in the tile, a tile's dK and dV are complete and stored at once; only dQ of split ranges (and of
// shared queries, summed over sequences) needs partial sums. Against separate dQ and dK/dV passes
// this reads K and V once instead of twice (aihot.vn GEM page, "Generalized Dot-Product Attention
// (GDPA)": short and asymmetric key / value sets, and PMA's shared seed queries).
struct alignas(16) FusedSmem {
  float lse2[kKvBM];                        // -lse in log2 units
  float dlt[kKvBM];                         // Delta
  float tab[kBuckets];
  float diag[2][kDiagLen];                  // per A wave: bias values of its 95 distances
  unsigned long long dbh[2][kDbiasBins];    // per B wave: bias-gradient bins (fixed point)
  uint4 xch[2][2][2][64];                   // [key half][query block][8-row half][lane]: P or act'/Lkv (bf16)
  unsigned char dst[64 * kRowBytes];        // dS^T: row = key of the tile, 64 queries (swizzled rows)
  unsigned char qg[2][kKvBM * kRowBytes];   // Q, dO
  unsigned char kv[3][2][64 * kRowBytes];   // ring: [stage][K, V]
};

template <int ACT, int BIASX, int MK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_fused_kernel(BwdArgs a) {
  constexpr int D = 128, BM = kKvBM, BN = 64, NKB = D / 16, NDB = D / 32;
  constexpr int BIAS = BIASX & 3;
  constexpr bool DBIAS = (BIASX & kBiasGrad) != 0;
  constexpr bool CAUSAL = MK == kMaskCausal;
  constexpr bool SOFTMAX = ACT == kSoftmax;
  constexpr int kLoadsPerTile = 8;  // dma16 instructions per wave per K / V tile (4 rows x 4, twice)
  __shared__ FusedSmem sm;

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool isB = wave >= 2;
  const int half = wave & 1;  // A / B: key half of the tile
  const WorkRec w = load_item(a.dq_items, blockIdx.x);
  const int h = w.h, k0 = w.lo, k1 = w.hi, slot = w.slot;
  const int qs = w.qs, Lq = w.Lq, ks = w.ks, Lkv = w.Lkv;
  const int H = a.H, rs = H * D;
  const float inv_scale = 1.0f / a.scale;
  const float smul = SOFTMAX ? a.scale * kLog2e : a.scale;
  const float bias_c = (BIAS == kBiasScalar) ? a.bias[h] : 0.0f;
  const float lse_shift = (SOFTMAX && BIAS == kBiasScalar) ? bias_c : 0.0f;
  // GDPA: a per-head scalar bias enters the scores (in units of the unscaled score)
  const float acc0 = (!SOFTMAX && BIAS == kBiasScalar) ? bias_c * inv_scale : 0.0f;
  const float invL = Lkv > 0 ? 1.0f / (float)Lkv : 0.0f;

  // ---- item prologue: Q and dO tiles, statistics, bias table, first two K / V tiles
  const __amdgpu_buffer_rsrc_t qsr = slice_rsrc(a.q + (size_t)(a.q_shared ? 0 : qs) * rs + h * D, Lq, rs, D);
  const __amdgpu_buffer_rsrc_t gsr = slice_rsrc(a.dout + (size_t)qs * rs + h * D, Lq, rs, D);
  const __amdgpu_buffer_rsrc_t ksr = slice_rsrc(a.k + (size_t)ks * rs + h * D, Lkv, rs, D);
  const __amdgpu_buffer_rsrc_t vsr = slice_rsrc(a.v + (size_t)ks * rs + h * D, Lkv, rs, D);
  const TileLoader ld = make_loader64(wave, lane, rs);
  load_tile64(ld, qsr, 0, rs, sm.qg[0], wave);
  load_tile64(ld, gsr, 0, rs, sm.qg[1], wave);
  if (SOFTMAX && wave == 0) {
    const __amdgpu_buffer_rsrc_t lser = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.lse) + (size_t)h * a.Tq + qs, (short)0, Lq * 4, 0x00020000);
    dma4(lser, (uint32_t)lane * 4u, sm.lse2);
  }
  if (BIAS == kBiasBucket && wave == 1) {
    const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.bias) + h * kBuckets,
                                                                        (short)0, kBuckets * 4, 0x00020000);
    dma4(tr, (uint32_t)lane * 4u, sm.tab);
  }
  auto issue = [&](int kt, int stg) {
    load_tile64(ld, ksr, kt * BN, rs, sm.kv[stg][0], wave);
    load_tile64(ld, vsr, kt * BN, rs, sm.kv[stg][1], wave);
  };
  if (k0 < k1) issue(k0, 0);
  if (k0 + 1 < k1) issue(k0 + 1, 1);
  // Delta_i = <dO_i, O_i> (softmax): four threads per row, 32 dimensions each.
  if (SOFTMAX) {
    const int row = tid >> 2, part = tid & 3;
    float acc = 0.0f;
    if (row < Lq) {
      const size_t base = ((size_t)(qs + row) * H + h) * D + part * 32;
      const uint16_t* gp = a.dout + base;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 g = load16(gp + 8 * c);
        float gv[8], ov[8];
        unpack8(g, gv);
        if (a.out_f32) {
          const float4 o0 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.out) + base + 8 * c);
          const float4 o1 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.out) + base + 8 * c + 4);
          ov[0] = o0.x; ov[1] = o0.y; ov[2] = o0.z; ov[3] = o0.w; ov[4] = o1.x; ov[5] = o1.y; ov[6] = o1.z; ov[7] = o1.w;
        } else {
          unpack8(load16(static_cast<const uint16_t*>(a.out) + base + 8 * c), ov);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += gv[j] * ov[j];
      }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (part == 0) sm.dlt[row] = acc;
  }
  if (DBIAS && isB) sm.dbh[half][lane] = 0ull;
  wait_vm();
  if (SOFTMAX && wave == 0) {
    const float x = sm.lse2[lane];
    sm.lse2[lane] = (lane < Lq && x != kNegInf) ? -(x - lse_shift) * kLog2e : kNegInf;
  }
  __syncthreads();

  const uint32_t raddr = row_operand_base(kappa(l32), hh);  // Q / dO rows as A operands
  uint32_t T[2];
  tr_operand_bases(lane, T);
  DbiasLane dbl;
  f32x16 dqa[2];  // dQ^T of dimensions 32 wave .. + 31, query blocks 0 and 1 (unscaled)
  dqa[0] = f32x16{};
  dqa[1] = f32x16{};

  f32x16 acc[NDB];  // A: dV, B: dK of the current tile (dK unscaled)
  // NQB: 32-row query blocks with rows (the second only when the sequence has more than 32 queries)
  auto tile = [&](const int kt, auto st_tag, auto nqb_tag) {
    constexpr int ST = decltype(st_tag)::value;
    constexpr bool qb1 = decltype(nqb_tag)::value == 2;
    // Outstanding at this point: tile kt's loads, then tile kt + 1's (and the previous tile's
    // stores). Loads complete in order, so with at most kLoadsPerTile operations left tile kt has
    // landed (tile kt + 1 may still be in flight).
    if (kt + 1 < k1)
      wait_vm_keep<kLoadsPerTile>();
    else
      wait_vm();
    __syncthreads();  // tile kt is published; every wave is done with the previous tile's LDS data
    if (kt + 2 < k1) issue(kt + 2, (ST + 2) % 3);
    const unsigned char* Kt = sm.kv[ST][0];
    const unsigned char* Vt = sm.kv[ST][1];
    const int key_w = kt * BN + 32 * half;  // first key of this wave's half
    const int kj = key_w + l32;
    // the wave's 32 keys as B operands (lane = key): K for A waves, V for B waves
    bf16x8 frag[NKB];
    {
      const unsigned char* src = isB ? Vt : Kt;
      const uint32_t fb = row_operand_base(32 * half + l32, hh);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) frag[kb] = lds_read16(src, fb ^ (uint32_t)(kb << 5));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    bf16x8 pk[2][2];  // A: P, B: dS, as B operands [query block][16-row step]
    f32x16 pacc[2];   // B: dP
    if (!isB) {
      if (BIAS == kBiasBucket) fill_diag(sm.diag[half], sm.tab, -key_w - 31, inv_scale, lane);
      const bool need_mask = (key_w + 32 > Lkv) || (CAUSAL && key_w + 31 > 0);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (qb == 1 && !qb1) break;
        f32x16 sacc;
        if (BIAS == kBiasBucket) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const float* dvp = &sm.diag[half][31 + 32 * qb + 16 * c + 8 * hh - l32];
#pragma unroll
            for (int j = 0; j < 8; ++j) sacc[8 * c + j] = dvp[j];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = acc0;
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          sacc = mfma32(lds_read16(sm.qg[0], (raddr ^ (uint32_t)(kb << 5)) + qb * 32 * kRowBytes), frag[kb], sacc);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int rbase = 32 * qb + 16 * c + 8 * hh;
          float pv[8], gv[8];
          if (SOFTMAX) {
            const float4 x0 = *reinterpret_cast<const float4*>(&sm.lse2[rbase]);
            const float4 x1 = *reinterpret_cast<const float4*>(&sm.lse2[rbase + 4]);
            const float l8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(__builtin_fmaf(sacc[8 * c + j], smul, l8[j]));
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              float f, g;
              act_fwd_grad<ACT>(sacc[8 * c + j] * smul, f, g);
              pv[j] = f;  // (the 1 / Lkv of GDPA is applied to dV, dK and dQ at the end)
              gv[j] = g;
            }
          }
          // Rows past the sequence's end need no mask: their dO rows read as zeros, so they add
          // nothing to dV and their dP, hence dS, is zero (softmax: their P is zero already).
          if (need_mask) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int qi = rbase + j;
              const bool masked = kj >= Lkv || (CAUSAL && kj > qi);
              pv[j] = masked ? 0.0f : pv[j];
              if (!SOFTMAX) gv[j] = masked ? 0.0f : gv[j];
            }
          }
          pk[qb][c] = pack8(pv);
          sm.xch[half][qb][c][lane] = SOFTMAX ? __builtin_bit_cast(uint4, pk[qb][c]) : __builtin_bit_cast(uint4, pack8(gv));
        }
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (qb == 1 && !qb1) break;
        pacc[qb] = f32x16{};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          pacc[qb] = mfma32(lds_read16(sm.qg[1], (raddr ^ (uint32_t)(kb << 5)) + qb * 32 * kRowBytes), frag[kb], pacc[qb]);
      }
    }
    __syncthreads();  // P is published
    if (!isB) {
      // dV^T += dO^T P
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s == 2 && !qb1) break;
        const uint32_t base = (uint32_t)(16 * s * kRowBytes);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = mfma32(lds_read_tr(sm.qg[1], base + (T[0] ^ (uint32_t)(64 * db)), base + (T[1] ^ (uint32_t)(64 * db))),
                           pk[s >> 1][s & 1], acc[db]);
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (qb == 1 && !qb1) break;
          const int rbase = 32 * qb + 16 * c + 8 * hh;
          float hv[8];  // softmax: P; GDPA: act'(S) / Lkv
          unpack8(sm.xch[half][qb][c][lane], hv);
          float dsv[8];
          if (SOFTMAX) {
            const float4 y0 = *reinterpret_cast<const float4*>(&sm.dlt[rbase]);
            const float4 y1 = *reinterpret_cast<const float4*>(&sm.dlt[rbase + 4]);
            const float d8[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) dsv[j] = hv[j] * (pacc[qb][8 * c + j] - d8[j]);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) dsv[j] = pacc[qb][8 * c + j] * hv[j];
          }
          pk[qb][c] = pack8(dsv);
          // dS^T row (this lane's key), logical chunk rbase / 8 of the query columns
          const int r = 32 * half + l32;
          *reinterpret_cast<uint4*>(&sm.dst[r * kRowBytes + (((rbase >> 3) ^ swz(r)) << 4)]) =
              __builtin_bit_cast(uint4, pk[qb][c]);
          if (DBIAS) {
            if (!SOFTMAX)
#pragma unroll
              for (int j = 0; j < 8; ++j) dsv[j] *= invL;
            dbl.add_run<BIAS == kBiasBucket>(sm.dbh[half], rbase - kj, dsv);
          }
        }
      // dK^T += Q^T dS
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s == 2 && !qb1) break;
        const uint32_t base = (uint32_t)(16 * s * kRowBytes);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = mfma32(lds_read_tr(sm.qg[0], base + (T[0] ^ (uint32_t)(64 * db)), base + (T[1] ^ (uint32_t)(64 * db))),
                           pk[s >> 1][s & 1], acc[db]);
      }
    }
    __syncthreads();  // dS^T is published
    // dQ^T (dimensions 32 wave ..) += K^T dS^T over the tile's 64 keys
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t base = (uint32_t)(16 * s * kRowBytes);
      const bf16x8 kop = lds_read_tr(Kt, base + (T[0] ^ (uint32_t)(64 * wave)), base + (T[1] ^ (uint32_t)(64 * wave)));
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (qb == 1 && !qb1) break;
        dqa[qb] = mfma32(kop, lds_read_tr(sm.dst, base + (T[0] ^ (uint32_t)(64 * qb)), base + (T[1] ^ (uint32_t)(64 * qb))),
                         dqa[qb]);
      }
    }
    // The tile's dV (A) or dK (B) is complete: store it. bf16 rows go out through LDS as whole
    // rows (a lane's accumulators hold 4-element pieces of its key's row): once every wave is done
    // with this stage, its K and V tiles (32 KB) give each wave 8 KB; the stage is reloaded only
    // after the next tile's first barrier.
    void* dstp = isB ? a.dk : a.dv;
    const float sc = (isB ? a.scale : 1.0f) * (SOFTMAX ? 1.0f : invL);
    if (!a.grad_f32) {
      __syncthreads();
      store_rows_staged(sm.kv[ST][0] + wave * (32 * kRowBytes), acc, sc, lane, Lkv - key_w,
                        [&](int r) { return static_cast<char*>(dstp) + (((size_t)(ks + key_w + r) * H + h) * D) * 2; });
    } else if (kj < Lkv) {
      const size_t base = ((size_t)(ks + kj) * H + h) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(dstp, base + 32 * db + 8 * g + 4 * hh, acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc,
                 acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc, 1);
    }
  };
  auto loop = [&](auto nqb_tag) {
    for (int kt = k0; kt < k1; kt += 3) {
      tile(kt, std::integral_constant<int, 0>{}, nqb_tag);
      if (kt + 1 < k1) tile(kt + 1, std::integral_constant<int, 1>{}, nqb_tag);
      if (kt + 2 < k1) tile(kt + 2, std::integral_constant<int, 2>{}, nqb_tag);
    }
  };
  if (Lq > 32)
    loop(std::integral_constant<int, 2>{});
  else
    loop(std::integral_constant<int, 1>{});

  if (DBIAS && isB) {
    dbl.flush(sm.dbh[half]);
    wave_lds_fence();
    constexpr int NB = BIAS == kBiasBucket ? kDbiasBins : 1;
    if (lane < NB) {
      const unsigned long long x = sm.dbh[half][lane];
      if (x) atomicAdd(a.dbias_acc + (size_t)h * NB + lane, x);
    }
  }
  // dQ: accumulator register r of query block qb holds dimension 32 wave + 8 (r/4) + 4 hh + r%4 of
  // query row 32 qb + lane % 32.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = 32 * qb + l32;
    if (qi >= Lq) continue;
    const float gs = SOFTMAX ? 1.0f : invL;  // GDPA: dS lacks its factor 1 / Lkv
    if (slot < 0) {
      const size_t base = ((size_t)(qs + qi) * H + h) * D + 32 * wave;
      const float sc = a.scale * gs;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(a.dq, base + 8 * g + 4 * hh, dqa[qb][4 * g] * sc, dqa[qb][4 * g + 1] * sc, dqa[qb][4 * g + 2] * sc,
               dqa[qb][4 * g + 3] * sc, a.grad_f32);
    } else {
      float* pp = a.part_dq + ((size_t)slot * kDqBM + qi) * D + 32 * wave;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(pp + 8 * g + 4 * hh) =
            make_float4(dqa[qb][4 * g] * gs, dqa[qb][4 * g + 1] * gs, dqa[qb][4 * g + 2] * gs, dqa[qb][4 * g + 3] * gs);
    }
  }
}

// ---------------------------------------------------------------- fixed-order partial sums
// One workgroup per split group.
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_dq_kernel(BwdArgs a) {
  reduce_dq_group<D, 256>(load_group(a.dq_groups, blockIdx.x), a.part_dq, a.dq, a.H, a.scale, a.grad_f32,
                          threadIdx.x);
}

// The same sums for groups with many pieces (shared queries: one piece per sequence): one workgroup
// per (group, row); lane group k of the workgroup adds pieces k, k + NL, k + 2 NL, ... of 4-column
// slices, and the NL lane groups' sums are added in a fixed tree order, so the result does not
// depend on scheduling.
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_dq_wide_kernel(BwdArgs a) {
  constexpr int BM = kDqBM, NQ = D / 4, NL = 256 / NQ;
  const int gi = blockIdx.x / BM, row = blockIdx.x % BM;
  const WorkRec g = load_group(a.dq_groups, gi);
  const int qi = g.tile * BM + row;
  if (qi >= g.Lq) return;
  const int slot0 = g.lo, R = g.hi;
  const int cq = threadIdx.x % NQ, k = threadIdx.x / NQ;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
  for (int r = k; r < R; r += NL) {
    const float4 x = *reinterpret_cast<const float4*>(a.part_dq + ((size_t)(slot0 + r) * BM + row) * D + 4 * cq);
    acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
  }
  __shared__ float4 red[NL][NQ];
  red[k][cq] = acc;
  __syncthreads();
  if (k == 0) {
#pragma unroll
    for (int st = 1; st < NL; st *= 2)  // pairwise tree: ((0 + 1) + (2 + 3)) + ...
#pragma unroll
      for (int i = 0; i < NL; i += 2 * st) {
        red[i][cq].x += red[i + st][cq].x;
        red[i][cq].y += red[i + st][cq].y;
        red[i][cq].z += red[i + st][cq].z;
        red[i][cq].w += red[i + st][cq].w;
      }
    const float4 t = red[0][cq];
    const size_t base = ((size_t)(g.qs + qi) * a.H + g.h) * D + 4 * cq;
    store4(a.dq, base, t.x * a.scale, t.y * a.scale, t.z * a.scale, t.w * a.scale, a.grad_f32);
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_dkdv_kernel(BwdArgs a) {
  constexpr int HALF = D / 2;
  const int BN = a.kv_bn;
  const WorkRec g = load_group(a.kv_groups, blockIdx.x);
  const int h = g.h, kt = g.tile, slot0 = g.lo, R = g.hi;
  const int ks = g.ks, Lkv = g.Lkv;
  const int row = threadIdx.x >> 1, part = threadIdx.x & 1;
  const int kj = kt * BN + row;
  if (row >= BN || kj >= Lkv) return;
  for (int which = 0; which < 2; ++which) {
    const float* src = which == 0 ? a.part_dk : a.part_dv;
    float acc[HALF];
#pragma unroll
    for (int d = 0; d < HALF; ++d) acc[d] = 0.0f;
    for (int r = 0; r < R; ++r) {
      const float* p = src + ((size_t)(slot0 + r) * BN + row) * D + part * HALF;
#pragma unroll
      for (int d = 0; d < HALF; d += 4) {
        float4 x = *reinterpret_cast<const float4*>(p + d);
        acc[d] += x.x; acc[d + 1] += x.y; acc[d + 2] += x.z; acc[d + 3] += x.w;
      }
    }
    const size_t base = ((size_t)(ks + kj) * a.H + h) * D + part * HALF;
    const float sc = which == 0 ? a.scale : 1.0f;
    void* dst = which == 0 ? a.dk : a.dv;
#pragma unroll
    for (int d = 0; d < HALF; d += 4)
      store4(dst, base + d, acc[d] * sc, acc[d + 1] * sc, acc[d + 2] * sc, acc[d + 3] * sc, a.grad_f32);
  }
}

// ---------------------------------------------------------------- bias gradient
// The fixed-point accumulators are cleared by a kernel (not a memset) so that a captured graph
// replays correctly; the finishing kernel converts them to fp32. Without a gradient variant of
// the dK/dV kernel (softmax with a per-head scalar, whose exact gradient is 0) the cleared totals
// come out as 0.
__global__ __launch_bounds__(256) void bwd_dbias_clear_kernel(BwdArgs a, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n && a.dbias_acc) a.dbias_acc[i] = 0ull;
  if (i < kQueueCounters && a.kv_queue) a.kv_queue[i] = 0;  // for backward passes with no dQ items
}

__global__ __launch_bounds__(256) void bwd_dbias_finish_kernel(BwdArgs a, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) a.dbias[i] = (float)((double)(long long)a.dbias_acc[i] * (1.0 / 4294967296.0));
}

// ---------------------------------------------------------------- dispatch
// D = 128 runs the LDS-ring kernels; D = 64 the register-staged ones.
constexpr int kDkdvThreads128 = 512;
template <int D, int ACT, int BIASX, int MK, int NP = 4>
constexpr auto dkdv_select =
    D == 128 ? &bwd_dkdv_kernel2<ACT, BIASX, MK, NP> : &bwd_dkdv_kernel<D, ACT, BIASX, MK>;
template <int D, int ACT, int BIAS, int MK>
constexpr auto dq_select = D == 128 ? &bwd_dq_kernel2<ACT, BIAS, MK> : &bwd_dq_kernel<D, ACT, BIAS, MK>;


#define JFA_DISPATCH_MODES(KERNEL, m, n, s, a)                                                          \
  [&]() -> hipError_t {                                                                                 \
    auto go = [&](auto kern) {                                                                          \
      hipLaunchKernelGGL(kern, dim3(n), dim3(block), 0, s, a);                                          \
      return hipGetLastError();                                                                         \
    };                                                                                                  \
    if (m.D == 64) {                                                                                    \
      JFA_DISPATCH_ACT(KERNEL, 64, m, go)                                                               \
    } else {                                                                                            \
      JFA_DISPATCH_ACT(KERNEL, 128, m, go)                                                              \
    }                                                                                                   \
  }()

#define JFA_DISPATCH_ACT(KERNEL, DD, m, go)                                                             \
  switch (m.act) {                                                                                      \
    case kSoftmax: JFA_DISPATCH_BIAS(KERNEL, DD, kSoftmax, m, go)                                       \
    case kSilu: JFA_DISPATCH_BIAS(KERNEL, DD, kSilu, m, go)                                             \
    default: JFA_DISPATCH_BIAS(KERNEL, DD, kGeluTanh, m, go)                                            \
  }

#define JFA_GO_MASK(KERNEL, DD, AA, BB, m, go)                                                          \
  switch (m.mask_kind()) {                                                                              \
    case kMaskBand: return go(KERNEL<DD, AA, BB, kMaskBand>);                                           \
    case kMaskCausal: return go(KERNEL<DD, AA, BB, kMaskCausal>);                                       \
    default: return go(KERNEL<DD, AA, BB, kMaskNone>);                                                  \
  }
#define JFA_DISPATCH_BIAS(KERNEL, DD, AA, m, go)                                                        \
  switch (m.bias) {                                                                                     \
    case kBiasNone: JFA_GO_MASK(KERNEL, DD, AA, kBiasNone, m, go)                                       \
    case kBiasScalar: JFA_GO_MASK(KERNEL, DD, AA, kBiasScalar, m, go)                                   \
    default: JFA_GO_MASK(KERNEL, DD, AA, kBiasBucket, m, go)                                            \
  }

// The dK/dV kernels also come in bias-gradient variants (bias | kBiasGrad).
#define JFA_GO_CAUSAL(KERNEL, DD, AA, BB, m, go)                                                   \
  if constexpr (DD == 128 && AA == kSoftmax) {                                                     \
    if (m.kv_short) {                                                                              \
      switch (m.mask_kind()) {                                                                     \
        case kMaskBand: return go(KERNEL<DD, AA, BB, kMaskBand, 2>);                               \
        case kMaskCausal: return go(KERNEL<DD, AA, BB, kMaskCausal, 2>);                           \
        default: return go(KERNEL<DD, AA, BB, kMaskNone, 2>);                                      \
      }                                                                                            \
    }                                                                                              \
  }                                                                                                \
  JFA_GO_MASK(KERNEL, DD, AA, BB, m, go)
#define JFA_DISPATCH_BIAS_GRAD(KERNEL, DD, AA, m, go)                                       \
  switch (m.bias | (m.dbias && !(m.bias == kBiasScalar && AA == kSoftmax) ? kBiasGrad : 0)) { \
    case kBiasNone: JFA_GO_CAUSAL(KERNEL, DD, AA, kBiasNone, m, go)                         \
    case kBiasScalar: JFA_GO_CAUSAL(KERNEL, DD, AA, kBiasScalar, m, go)                     \
    case kBiasBucket: JFA_GO_CAUSAL(KERNEL, DD, AA, kBiasBucket, m, go)                     \
    case kBiasScalar | kBiasGrad: JFA_GO_CAUSAL(KERNEL, DD, AA, kBiasScalar | kBiasGrad, m, go) \
    default: JFA_GO_CAUSAL(KERNEL, DD, AA, kBiasBucket | kBiasGrad, m, go)                  \
  }
#define JFA_DISPATCH_ACT_GRAD(KERNEL, DD, m, go)                                \
  switch (m.act) {                                                              \
    case kSoftmax: JFA_DISPATCH_BIAS_GRAD(KERNEL, DD, kSoftmax, m, go)          \
    case kSilu: JFA_DISPATCH_BIAS_GRAD(KERNEL, DD, kSilu, m, go)                \
    default: JFA_DISPATCH_BIAS_GRAD(KERNEL, DD, kGeluTanh, m, go)               \
  }

}  // namespace


hipError_t launch_bwd_dq(const BwdArgs& a, const Modes& m, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int block = kThreads;
  return JFA_DISPATCH_MODES(dq_select, m, n, s, a);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, const Modes& m, int n, int resident, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int block = m.D == 128 ? (m.kv_short ? kDkdvThreads128 / 2 : kDkdvThreads128) : kThreads;
  const int grid = (m.D == 128 && !m.kv_short) ? std::max(1, std::min(n, resident)) : n;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(block), 0, s, a);
    return hipGetLastError();
  };
  if (m.D == 64) {
    JFA_DISPATCH_ACT_GRAD(dkdv_select, 64, m, go)
  } else {
    JFA_DISPATCH_ACT_GRAD(dkdv_select, 128, m, go)
  }
}

hipError_t launch_bwd_fused(const BwdArgs& a, const Modes& m, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(n), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  };
  auto by_mask = [&](auto act_tag, auto bias_tag) {
    constexpr int A = decltype(act_tag)::value, BX = decltype(bias_tag)::value;
    return m.causal ? go(bwd_fused_kernel<A, BX, kMaskCausal>) : go(bwd_fused_kernel<A, BX, kMaskNone>);
  };
  auto by_bias = [&](auto act_tag) {
    constexpr int A = decltype(act_tag)::value;
    using I = std::integral_constant<int, 0>;
    // under softmax a per-head scalar has a zero gradient: no gradient variant
    const bool grad = m.dbias && !(A == kSoftmax && m.bias == kBiasScalar);
    switch (m.bias | (grad ? kBiasGrad : 0)) {
      case kBiasNone: return by_mask(act_tag, I{});
      case kBiasScalar: return by_mask(act_tag, std::integral_constant<int, kBiasScalar>{});
      case kBiasBucket: return by_mask(act_tag, std::integral_constant<int, kBiasBucket>{});
      case kBiasScalar | kBiasGrad:
        if constexpr (A != kSoftmax) return by_mask(act_tag, std::integral_constant<int, kBiasScalar | kBiasGrad>{});
        return by_mask(act_tag, std::integral_constant<int, kBiasScalar>{});
      default: return by_mask(act_tag, std::integral_constant<int, kBiasBucket | kBiasGrad>{});
    }
  };
  switch (m.act) {
    case kSoftmax: return by_bias(std::integral_constant<int, kSoftmax>{});
    case kSilu: return by_bias(std::integral_constant<int, kSilu>{});
    default: return by_bias(std::integral_constant<int, kGeluTanh>{});
  }
}

hipError_t launch_bwd_dbias_clear(const BwdArgs& a, const Modes& m, hipStream_t s) {
  const int n = a.dbias_acc ? a.H * (m.bias == kBiasBucket ? kDbiasBins : 1) : 0;
  const int threads = std::max(n, kQueueCounters);
  hipLaunchKernelGGL(bwd_dbias_clear_kernel, dim3((threads + 255) / 256), dim3(256), 0, s, a, n);
  return hipGetLastError();
}

hipError_t launch_bwd_dbias_finish(const BwdArgs& a, const Modes& m, hipStream_t s) {
  const int n = a.H * (m.bias == kBiasBucket ? kDbiasBins : 1);
  hipLaunchKernelGGL(bwd_dbias_finish_kernel, dim3((n + 255) / 256), dim3(256), 0, s, a, n);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce_dq(const BwdArgs& a, const Modes& m, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (m.D == 64)
    hipLaunchKernelGGL(bwd_reduce_dq_kernel<64>, dim3(n), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_reduce_dq_kernel<128>, dim3(n), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce_dq_wide(const BwdArgs& a, const Modes& m, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (m.D == 64)
    hipLaunchKernelGGL(bwd_reduce_dq_wide_kernel<64>, dim3(n * kDqBM), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_reduce_dq_wide_kernel<128>, dim3(n * kDqBM), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce_dkdv(const BwdArgs& a, const Modes& m, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (m.D == 64)
    hipLaunchKernelGGL(bwd_reduce_dkdv_kernel<64>, dim3(n), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_reduce_dkdv_kernel<128>, dim3(n), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

int occupancy_dq(const Modes& m) {
  int n = 0;
  hipError_t e = m.D == 64
                     ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, bwd_dq_kernel<64, kSoftmax, kBiasBucket, kMaskCausal>, kThreads, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, bwd_dq_kernel2<kSoftmax, kBiasBucket, kMaskCausal>, kThreads, 0);
  return (e == hipSuccess && n > 0) ? n : 1;
}

int occupancy_dkdv(const Modes& m) {
  int n = 0;
  hipError_t e = m.D == 64
                     ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, bwd_dkdv_kernel<64, kSoftmax, kBiasBucket, kMaskCausal>, kThreads, 0)
                     : m.kv_short ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                                        &n, dkdv_select<128, kSoftmax, kBiasScalar, kMaskNone, 2>, kDkdvThreads128 / 2, 0)
                                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                                        &n, dkdv_select<128, kSoftmax, kBiasBucket, kMaskCausal>, kDkdvThreads128, 0);
  return (e == hipSuccess && n > 0) ? n : 1;
}

}  // namespace jfa
