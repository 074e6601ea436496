// Forward pass of jagged attention on gfx950.
//
// One workgroup (4 waves) runs one work item: a 128-row query tile of one (sequence, head) over a
// range of 64-key tiles. Each wave owns 32 query rows. Per key tile:
//   S^T = K Q^T            (32x32x16 bf16 MFMA; K rows from LDS in kappa order, Q^T from registers)
//   score -> log2 domain, bias added, mask by -inf only on tiles that straddle the sequence end
//            or the diagonal (aihot.vn GEM page, "Jagged Sequence Flash Attention": no padding;
//            kerneldigest.dev page, "Arquitectura del Sistema": masking by subtraction)
//   online softmax (running max / sum per query lane) or the GDPA activation
//            (aihot.vn GEM page, "Generalized Dot-Product Attention (GDPA)")
//   O^T += V^T P^T         (V^T from LDS, P^T straight from the score registers)
// The query of lane l is column l%32 of every accumulator, so row statistics reduce inside the
// lane plus one exchange with lane l^32.
#include "device_common.h"
#include "tile_lds.h"

namespace jfa {
namespace {

template <int D>
struct alignas(16) FwdSmem {
  static constexpr int KS = D + 8;          // K row stride (bf16): 16-byte reads are conflict free
  static constexpr int VS = kFwdBN + 8;     // V^T row stride
  __bf16 k[kFwdBN * KS];
  __bf16 vt[D * VS];
  float tab[kBuckets];
  float diag[4][kDiagLen];
};

template <int D>
struct KvRegs {
  static constexpr int KCH = kFwdBN * D / 8 / kThreads;  // 16-byte K chunks per thread
  uint4 k[KCH];
  uint4 v[4];                                           // 4 keys x 8 dims, stored transposed
};

// Global -> registers for one 64-key tile. Rows past the sequence end read as zeros.
template <int D>
__device__ __forceinline__ void load_kv(KvRegs<D>& r, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int rs,
                                        int key0, int tid) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int u = 0; u < KvRegs<D>::KCH; ++u) {
    const int c = tid + kThreads * u, row = c / CPR, col = c % CPR;
    r.k[u] = buf_load16(kr, (uint32_t)((key0 + row) * rs + col * 8) * 2u);
  }
  constexpr int UNITS = (kFwdBN / 4) * CPR, G = kFwdBN / 4;
  if (UNITS >= kThreads || tid < UNITS) {
    const int kg = tid % G, dg = tid / G;  // key groups fastest: transposed LDS writes hit distinct banks
#pragma unroll
    for (int j = 0; j < 4; ++j) r.v[j] = buf_load16(vr, (uint32_t)((key0 + 4 * kg + j) * rs + dg * 8) * 2u);
  }
}

template <int D>
__device__ __forceinline__ void store_kv(const KvRegs<D>& r, FwdSmem<D>& sm, int tid) {
  constexpr int CPR = D / 8, KS = FwdSmem<D>::KS, VS = FwdSmem<D>::VS;
#pragma unroll
  for (int u = 0; u < KvRegs<D>::KCH; ++u) {
    const int c = tid + kThreads * u, row = c / CPR, col = c % CPR;
    *reinterpret_cast<uint4*>(&sm.k[row * KS + col * 8]) = r.k[u];
  }
  constexpr int UNITS = (kFwdBN / 4) * CPR, G = kFwdBN / 4;
  if (UNITS >= kThreads || tid < UNITS) {
    const int kg = tid % G, dg = tid / G;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint2*>(&sm.vt[(dg * 8 + e) * VS + 4 * kg]) = column4(r.v, e);
  }
}

// Softmax keeps a running row maximum m and rescales O and l only when a tile's maximum exceeds m
// by more than 2^kLazy: otherwise probabilities are taken against the stale m (bounded by 2^kLazy,
// exact in fp32 and as relative-precision bf16 operands), which skips most rescales.
constexpr float kLazy = 8.0f;

template <int D, int ACT, int BIAS, int MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdArgs a) {
  constexpr int BM = kFwdBM, BN = kFwdBN, NKB = D / 16, NDB = D / 32;
  constexpr int KS = FwdSmem<D>::KS, VS = FwdSmem<D>::VS;
  constexpr bool SOFTMAX = ACT == kSoftmax;
  constexpr bool CAUSAL = MASK == kMaskCausal, BAND = MASK == kMaskBand;
  __shared__ FwdSmem<D> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const WorkRec w = load_item(a.items, blockIdx.x);
  const int h = w.h, t = w.tile, k0 = w.lo, k1 = w.hi, slot = w.slot;
  const int qs = w.qs, Lq = w.Lq, ks = w.ks, Lkv = w.Lkv;
  const int rs = a.H * D;
  const int row0 = t * BM + wave * 32;
  const int qi = row0 + l32;
  const float inv_scale = 1.0f / a.scale;
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

  if (BIAS == kBiasBucket && tid < kBuckets) sm.tab[tid] = a.bias[h * kBuckets + tid];
  const float bias_c = (BIAS == kBiasScalar) ? a.bias[h] : 0.0f;
  // the bias enters as the accumulator's initial value, in units of the unscaled score
  const float acc0 = (BIAS == kBiasScalar && !SOFTMAX) ? bias_c * inv_scale : 0.0f;

  bf16x8 qf[NKB];
  {
    const __amdgpu_buffer_rsrc_t qr = slice_rsrc(a.q + (size_t)(a.q_shared ? 0 : qs) * rs + h * D, Lq, rs, D);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) qf[kb] = as_bf16x8(buf_load16(qr, (uint32_t)(qi * rs + kb * 16 + hh * 8) * 2u));
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;
  const float smul = SOFTMAX ? a.scale * kLog2e : a.scale;

  const __amdgpu_buffer_rsrc_t kr = slice_rsrc(a.k + (size_t)ks * rs + h * D, Lkv, rs, D);
  const __amdgpu_buffer_rsrc_t vr = slice_rsrc(a.v + (size_t)ks * rs + h * D, Lkv, rs, D);
  KvRegs<D> pf;
  if (k0 < k1) load_kv<D>(pf, kr, vr, rs, k0 * BN, tid);

  for (int kt = k0; kt < k1; ++kt) {
    const int key0 = kt * BN;
    __syncthreads();
    store_kv<D>(pf, sm, tid);
    if (BIAS == kBiasBucket) fill_diag(sm.diag[wave], sm.tab, row0 - key0 - (BN - 1), inv_scale, lane);
    __syncthreads();
    if (kt + 1 < k1) load_kv<D>(pf, kr, vr, rs, (kt + 1) * BN, tid);

    // S^T tile: lane = query qi, register r of block sb = key key0 + 32 sb + acc_row(r, hh).
    f32x16 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      if (BIAS == kBiasBucket) {
        // d = qi - key = (row0 - key0 - 63) + (63 - 32 sb + l32 - 16 c - 8 hh - j)
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
      const __bf16* kp = &sm.k[(32 * sb + kappa(l32)) * KS + hh * 8];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[sb] = mfma32(lds_load8(kp + kb * 16), qf[kb], sacc[sb]);
    }

    const bool need_mask = BAND ? (wlo_all > key0 || whi_all < key0 + BN - 1)
                                : (key0 + BN > Lkv) || (CAUSAL && key0 + BN - 1 > row0);
    if (need_mask) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * sb + acc_row(r, hh);
          const bool masked = BAND ? (key < klo || key > khi) : (key >= Lkv || (CAUSAL && key > qi));
          sacc[sb][r] = masked ? (SOFTMAX ? kNegInf : __builtin_nanf("")) : sacc[sb][r];
        }
    }

    float p[2][16];
    if (SOFTMAX) {
      float mx = kNegInf;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * smul;
      if (__ballot(mx > m_run + kLazy)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == kNegInf ? 0.0f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_run = m_new;
      }
      const float nm = m_run == kNegInf ? 0.0f : -m_run;
      float lsum = 0.0f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(__builtin_fmaf(sacc[sb][r], smul, nm));
          p[sb][r] = e;
          lsum += e;
        }
      l_run += lsum;
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = sacc[sb][r];
          p[sb][r] = x != x ? 0.0f : act_fwd<ACT>(x * smul);  // masked scores carry NaN
        }
    }

    bf16x8 pb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) pb[c] = pack8(&p[c >> 1][8 * (c & 1)]);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const __bf16* vp = &sm.vt[(32 * db + l32) * VS + 8 * hh];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[db] = mfma32(lds_load8(vp + 16 * c), pb[c], o[db]);
    }
  }

  // Epilogue. Accumulator register r of d-block db holds dimension 32 db + 8 (r/4) + 4 hh + r%4.
  float inv;
  float l_tot = 0.0f;
  if (SOFTMAX) {
    l_tot = l_run + __shfl_xor(l_run, 32);
    inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  } else {
    inv = (slot < 0 && Lkv > 0) ? 1.0f / (float)Lkv : 1.0f;
  }
  if (slot < 0) {
    if (qi < Lq) {
      const size_t base = ((size_t)(qs + qi) * a.H + h) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(a.out, base + 32 * db + 8 * g + 4 * hh, o[db][4 * g] * inv, o[db][4 * g + 1] * inv,
                 o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv, a.out_f32);
      if (SOFTMAX && hh == 0)
        a.lse[(size_t)h * a.Tq + qs + qi] =
            l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 + (BIAS == kBiasScalar ? bias_c : 0.0f) : kNegInf;
    }
  } else {
    const int prow = wave * 32 + l32;
    float* po = a.part_o + ((size_t)slot * BM + prow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * g + 4 * hh) =
            make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
    if (SOFTMAX && hh == 0)
      a.part_lse[(size_t)slot * BM + prow] = l_tot > 0.0f ? m_run + fast_log2(l_tot) : kNegInf;
  }
}

// D = 128 forward with a two-stage LDS ring: K and V tiles are loaded straight into LDS
// (swizzled row-major, no staging registers) one tile ahead of the compute, with one barrier per
// tile; V^T operands come from transposing LDS reads of the row-major V tile.
struct alignas(16) FwdSmem2 {
  unsigned char kv[2][2][kFwdBN * kRowBytes];  // [stage][0 = K, 1 = V]
  float tab[kBuckets];
  float diag[4][kDiagLen];
};

template <int ACT, int BIAS, int MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel2(FwdArgs a) {
  constexpr int D = 128, BM = kFwdBM, BN = kFwdBN, NKB = D / 16, NDB = D / 32;
  constexpr bool SOFTMAX = ACT == kSoftmax;
  constexpr bool CAUSAL = MASK == kMaskCausal, BAND = MASK == kMaskBand;
  __shared__ FwdSmem2 sm;

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const WorkRec w = load_item(a.items, blockIdx.x);
  const int h = w.h, t = w.tile, k0 = w.lo, k1 = w.hi, slot = w.slot;
  const int qs = w.qs, Lq = w.Lq, ks = w.ks, Lkv = w.Lkv;
  const int rs = a.H * D;
  const int row0 = t * BM + wave * 32;
  const int qi = row0 + l32;
  const float inv_scale = 1.0f / a.scale;
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

  // The bias table is loaded here and written to LDS after the other prologue loads are issued, so
  // that its round trip overlaps theirs.
  const float tabv = (BIAS == kBiasBucket && tid < kBuckets) ? a.bias[h * kBuckets + tid] : 0.0f;
  const float bias_c = (BIAS == kBiasScalar) ? a.bias[h] : 0.0f;
  const float acc0 = (BIAS == kBiasScalar && !SOFTMAX) ? bias_c * inv_scale : 0.0f;

  bf16x8 qf[NKB];
  {
    const __amdgpu_buffer_rsrc_t qr = slice_rsrc(a.q + (size_t)(a.q_shared ? 0 : qs) * rs + h * D, Lq, rs, D);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) qf[kb] = as_bf16x8(buf_load16(qr, (uint32_t)(qi * rs + kb * 16 + hh * 8) * 2u));
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;
  const float smul = SOFTMAX ? a.scale * kLog2e : a.scale;

  const __amdgpu_buffer_rsrc_t kr = slice_rsrc(a.k + (size_t)ks * rs + h * D, Lkv, rs, D);
  const __amdgpu_buffer_rsrc_t vr = slice_rsrc(a.v + (size_t)ks * rs + h * D, Lkv, rs, D);
  const TileLoader ld = make_loader64(wave, lane, rs);
  const uint32_t kaddr = row_operand_base(kappa(l32), hh);  // K row kappa(l32) (+ 32 sb rows)
  uint32_t T[2];
  tr_operand_bases(lane, T);

  if (k0 < k1) {
    load_tile64(ld, kr, k0 * BN, rs, sm.kv[0][0], wave);
    load_tile64(ld, vr, k0 * BN, rs, sm.kv[0][1], wave);
  }
  // Wave 0 writes the bias table; every wave reads it in the first tile's diagonal fill.
  if (BIAS == kBiasBucket) {
    if (tid < kBuckets) sm.tab[tid] = tabv;
    __syncthreads();
  }
  // One kv tile. ST is the ring stage holding tile kt (compile-time, so every LDS address is a
  // loop-invariant register plus an immediate offset).
  auto tile = [&](const int kt, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    const int key0 = kt * BN;
    // A tile with no visible pair for this wave's rows (past the diagonal, or outside the band), or a
    // wave whose rows all lie past the sequence's end, contributes nothing.
    const bool wskip =
        row0 >= Lq || (CAUSAL ? key0 > row0 + 31 : (BAND ? (key0 > whi || key0 + BN - 1 < wlo) : false));
    wait_vm();
    // Bias of score (qi, key) sits at diag[qi - key + 31 - (row0 - key0)] = diag[31 - l32 + key - key0]:
    // ascending in the accumulator's register order.
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

    f32x16 sacc[2];
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
    }
    // K operands are requested four products ahead of their MFMAs (the two 32-key blocks alternate),
    // so each product finds its operand loaded instead of waiting for a read issued just before it.
    bf16x8 kop[2 * NKB];
#pragma unroll
    for (int s = 0; s < 2 * NKB; ++s)
      kop[s] = lds_read16(Kt, (kaddr ^ (uint32_t)((s >> 1) << 5)) + (s & 1) * 32 * kRowBytes);
#pragma unroll
    for (int s = 0; s < 2 * NKB; ++s) sacc[s & 1] = mfma32(kop[s], qf[s >> 1], sacc[s & 1]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + (BIAS == kBiasBucket ? 16 : 0), 0);
#pragma unroll
    for (int s = 0; s < 2 * NKB - 4; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

    const bool need_mask = BAND ? (wlo_all > key0 || whi_all < key0 + BN - 1)
                                : (key0 + BN > Lkv) || (CAUSAL && key0 + BN - 1 > row0);
    if (need_mask) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * sb + acc_row(r, hh);
          const bool masked = BAND ? (key < klo || key > khi) : (key >= Lkv || (CAUSAL && key > qi));
          sacc[sb][r] = masked ? (SOFTMAX ? kNegInf : __builtin_nanf("")) : sacc[sb][r];
        }
    }

    float p[2][16];
    if (SOFTMAX) {
      float mx = kNegInf;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * smul;
      if (__ballot(mx > m_run + kLazy)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == kNegInf ? 0.0f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_run = m_new;
      }
      const float nm = m_run == kNegInf ? 0.0f : -m_run;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[sb][r] = fast_exp2(__builtin_fmaf(sacc[sb][r], smul, nm));
    } else if (need_mask) {  // masked scores carry NaN (only on tiles that needed the mask)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = sacc[sb][r];
          p[sb][r] = x != x ? 0.0f : act_fwd<ACT>(x * smul);
        }
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[sb][r] = act_fwd<ACT>(sacc[sb][r] * smul);
    }

    bf16x8 pb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) pb[c] = pack8(&p[c >> 1][8 * (c & 1)]);
    // The row sum adds the bf16 weights the P V product uses, two per instruction.
    if (SOFTMAX) l_run = rowsum_bf16(pb, l_run);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t base = (uint32_t)(c * 16 * kRowBytes);
        o[db] = mfma32(lds_read_tr(Vt, base + (T[0] ^ (uint32_t)(64 * db)), base + (T[1] ^ (uint32_t)(64 * db))), pb[c],
                       o[db]);
      }
  };
  for (int kt = k0; kt < k1; kt += 2) {
    tile(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < k1) tile(kt + 1, std::integral_constant<int, 1>{});
  }

  float inv;
  float l_tot = 0.0f;
  if (SOFTMAX) {
    l_tot = l_run + __shfl_xor(l_run, 32);
    inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  } else {
    inv = (slot < 0 && Lkv > 0) ? 1.0f / (float)Lkv : 1.0f;
  }
  if (slot < 0) {
    if (qi < Lq && SOFTMAX && hh == 0)
      a.lse[(size_t)h * a.Tq + qs + qi] =
          l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 + (BIAS == kBiasScalar ? bias_c : 0.0f) : kNegInf;
    if (!a.out_f32) {
      // bf16 rows through the ring stage that the last tile did not use (every wave finished reading
      // it before the last tile's barrier, and no load went into it since): 8 KB per wave. Each lane
      // scales its row by its own 1 / l.
      const int free_st = ((k1 - 1 - k0) & 1) ^ 1;
      char* dst = static_cast<char*>(a.out);
      const int H = a.H;
      store_rows_staged(&sm.kv[free_st][0][0] + wave * (32 * kRowBytes), o, inv, lane, Lq - row0,
                        [&](int r) { return dst + (((size_t)(qs + row0 + r) * H + h) * D) * 2; });
    } else if (qi < Lq) {
      const size_t base = ((size_t)(qs + qi) * a.H + h) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(a.out, base + 32 * db + 8 * g + 4 * hh, o[db][4 * g] * inv, o[db][4 * g + 1] * inv,
                 o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv, a.out_f32);
    }
  } else if (qi < Lq) {  // the combine reads the rows of the sequence only
    const int prow = wave * 32 + l32;
    float* po = a.part_o + ((size_t)slot * BM + prow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * g + 4 * hh) =
            make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
    if (SOFTMAX && hh == 0)
      a.part_lse[(size_t)slot * BM + prow] = l_tot > 0.0f ? m_run + fast_log2(l_tot) : kNegInf;
  }
}

// Merge the pieces of split items in fixed order r = 0..R-1:
//   softmax: lse* = log2 sum_r 2^lse_r,  O = sum_r 2^(lse_r - lse*) O_r   (O_r normalised per piece)
//   GDPA:    O = (sum_r O_r) / Lkv
// The kernel is a chain of dependent memory round trips (record, pieces, output), so everything a
// thread needs is requested up front: the log-sum-exps of up to kCombinePre pieces and the rows of
// the first two pieces, before any arithmetic.
constexpr int kCombineThreads = 512;  // 4 threads per row
constexpr int kCombinePre = 8;

template <int D, int ACT, int BIAS>
__global__ __launch_bounds__(kCombineThreads) void fwd_combine_kernel(FwdArgs a) {
  constexpr int BM = kFwdBM, TPR = kCombineThreads / BM, COLS = D / TPR, NC = COLS / 4;
  constexpr bool SOFTMAX = ACT == kSoftmax;
  const WorkRec g = load_group(a.groups, blockIdx.x);
  const int h = g.h, t = g.tile, slot0 = g.lo, R = g.hi;
  const int qs = g.qs, Lq = g.Lq, Lkv = g.Lkv;
  const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
  const int qi = t * BM + row;
  if (qi >= Lq) return;
  const size_t stride = (size_t)BM * D;
  const float* p0 = a.part_o + ((size_t)slot0 * BM + row) * D + part * COLS;
  float4 x0[NC], x1[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) x0[c] = *reinterpret_cast<const float4*>(p0 + 4 * c);
  if (R > 1) {
#pragma unroll
    for (int c = 0; c < NC; ++c) x1[c] = *reinterpret_cast<const float4*>(p0 + stride + 4 * c);
  }
  const float* pl = a.part_lse + (size_t)slot0 * BM + row;
  float lp[kCombinePre];  // indexed with unrolled (constant) r only
  if (SOFTMAX) {
#pragma unroll
    for (int r = 0; r < kCombinePre; ++r) {
      lp[r] = kNegInf;
      if (r < R) lp[r] = pl[(size_t)r * BM];
    }
  }

  float acc[COLS];
#pragma unroll
  for (int d = 0; d < COLS; ++d) acc[d] = 0.0f;
  auto add = [&](const float4 (&x)[NC], float w) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      acc[4 * c] += w * x[c].x;
      acc[4 * c + 1] += w * x[c].y;
      acc[4 * c + 2] += w * x[c].z;
      acc[4 * c + 3] += w * x[c].w;
    }
  };
  auto add_piece = [&](int r, float w) {
    if (r == 0) {
      add(x0, w);
    } else if (r == 1) {
      add(x1, w);
    } else {
      float4 x[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) x[c] = *reinterpret_cast<const float4*>(p0 + (size_t)r * stride + 4 * c);
      add(x, w);
    }
  };
  float lse2 = kNegInf;
  if (SOFTMAX) {
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < kCombinePre; ++r) mx = fmaxf(mx, lp[r]);
    for (int r = kCombinePre; r < R; ++r) mx = fmaxf(mx, pl[(size_t)r * BM]);
    if (mx != kNegInf) {
      float sum = 0.0f;
#pragma unroll
      for (int r = 0; r < kCombinePre; ++r)
        if (r < R) sum += fast_exp2(lp[r] - mx);
      for (int r = kCombinePre; r < R; ++r) sum += fast_exp2(pl[(size_t)r * BM] - mx);
      lse2 = mx + fast_log2(sum);
#pragma unroll
      for (int r = 0; r < kCombinePre; ++r)
        if (r < R) add_piece(r, fast_exp2(lp[r] - lse2));
      for (int r = kCombinePre; r < R; ++r) add_piece(r, fast_exp2(pl[(size_t)r * BM] - lse2));
    }
  } else {
    for (int r = 0; r < R; ++r) add_piece(r, 1.0f);
    const float inv = Lkv > 0 ? 1.0f / (float)Lkv : 0.0f;
#pragma unroll
    for (int d = 0; d < COLS; ++d) acc[d] *= inv;
  }
  const size_t base = ((size_t)(qs + qi) * a.H + h) * D + part * COLS;
#pragma unroll
  for (int d = 0; d < COLS; d += 4) store4(a.out, base + d, acc[d], acc[d + 1], acc[d + 2], acc[d + 3], a.out_f32);
  if (SOFTMAX && part == 0)
    a.lse[(size_t)h * a.Tq + qs + qi] =
        lse2 == kNegInf ? kNegInf : lse2 * kLn2 + (BIAS == kBiasScalar ? a.bias[h] : 0.0f);
}

template <int D, int ACT, int BIAS, int MASK>
hipError_t fwd_launch_t(const FwdArgs& a, int n, hipStream_t s) {
  if (D == 128)
    hipLaunchKernelGGL((fwd_kernel2<ACT, BIAS, MASK>), dim3(n), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_kernel<D, ACT, BIAS, MASK>), dim3(n), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, int ACT, int BIAS>
hipError_t fwd_launch_c(const FwdArgs& a, const Modes& m, int n, hipStream_t s) {
  switch (m.mask_kind()) {
    case kMaskBand: return fwd_launch_t<D, ACT, BIAS, kMaskBand>(a, n, s);
    case kMaskCausal: return fwd_launch_t<D, ACT, BIAS, kMaskCausal>(a, n, s);
    default: return fwd_launch_t<D, ACT, BIAS, kMaskNone>(a, n, s);
  }
}

template <int D, int ACT>
hipError_t fwd_launch_b(const FwdArgs& a, const Modes& m, int n, hipStream_t s) {
  switch (m.bias) {
    case kBiasNone: return fwd_launch_c<D, ACT, kBiasNone>(a, m, n, s);
    case kBiasScalar: return fwd_launch_c<D, ACT, kBiasScalar>(a, m, n, s);
    default: return fwd_launch_c<D, ACT, kBiasBucket>(a, m, n, s);
  }
}

template <int D>
hipError_t fwd_launch_a(const FwdArgs& a, const Modes& m, int n, hipStream_t s) {
  switch (m.act) {
    case kSoftmax: return fwd_launch_b<D, kSoftmax>(a, m, n, s);
    case kSilu: return fwd_launch_b<D, kSilu>(a, m, n, s);
    default: return fwd_launch_b<D, kGeluTanh>(a, m, n, s);
  }
}

template <int D, int ACT>
hipError_t comb_launch_b(const FwdArgs& a, const Modes& m, int n, hipStream_t s) {
  if (m.bias == kBiasScalar)
    hipLaunchKernelGGL((fwd_combine_kernel<D, ACT, kBiasScalar>), dim3(n), dim3(kCombineThreads), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_combine_kernel<D, ACT, kBiasNone>), dim3(n), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t comb_launch_a(const FwdArgs& a, const Modes& m, int n, hipStream_t s) {
  switch (m.act) {
    case kSoftmax: return comb_launch_b<D, kSoftmax>(a, m, n, s);
    case kSilu: return comb_launch_b<D, kSilu>(a, m, n, s);
    default: return comb_launch_b<D, kGeluTanh>(a, m, n, s);
  }
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a, const Modes& m, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  return m.D == 64 ? fwd_launch_a<64>(a, m, n_items, s) : fwd_launch_a<128>(a, m, n_items, s);
}

hipError_t launch_forward_combine(const FwdArgs& a, const Modes& m, int n_groups, hipStream_t s) {
  if (n_groups <= 0) return hipSuccess;
  return m.D == 64 ? comb_launch_a<64>(a, m, n_groups, s) : comb_launch_a<128>(a, m, n_groups, s);
}

int occupancy_forward(const Modes& m) {
  int n = 0;
  hipError_t e;
  if (m.D == 64)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_kernel<64, kSoftmax, kBiasBucket, kMaskCausal>, kThreads, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_kernel2<kSoftmax, kBiasBucket, kMaskCausal>, kThreads, 0);
  return (e == hipSuccess && n > 0) ? n : 1;
}

}  // namespace jfa
