// MXFP8 forward pass of jagged softmax attention on gfx950 (kerneldigest.dev page, "Arquitectura
// del Sistema": attention in MXFP8 with block quantisation and the probabilities P converted to
// MXFP8 online).
//
// Format: blocks of 32 elements share a power-of-two scale 2^(floor(log2 amax) - 8) (an E8M0 byte);
// elements are FP8 E4M3 (x / scale rounded to nearest even, saturated at 448). Q and K are quantised
// in blocks of 32 features of a row, V in blocks of 32 consecutive keys of one feature counted from
// the sequence's first key, P in blocks of 32 consecutive keys of a row. Products run on the scaled
// MFMA v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation.
//
// Operand layout of that MFMA with FP8 operands (measured on the device with an in-bounds one-wave
// probe): lane l holds row (A) / column (B) l % 32; its 32 bytes are contraction indices
// k = 16 (l / 32) + 0..15 (bytes 0..15) and k = 32 + 16 (l / 32) + 0..15 (bytes 16..31); the 32-k block
// kb = k / 32 is scaled by the scale byte of lane half kb of the same row / column. The accumulator
// layout is that of the bf16 32x32 products.
#include "device_common.h"
#include "tile_lds.h"

namespace jfa {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ f32x16 mfma_mx(const i32x8& a, int sa, const i32x8& b, int sb, f32x16 c) {
  // formats 0 / 0: both operands FP8 E4M3; op_sel 0: scale byte 0 of each lane's scale register
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// E8M0 byte and the reciprocal scale of a block with largest magnitude amax (>= 0, finite):
// scale = 2^(e - 8) with e = floor(log2 amax), clamped at 2^-127 (all-zero and tiny blocks).
__device__ __forceinline__ void mx_scale(float amax, int& byte, float& inv) {
  const int eb = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 255);  // e + 127 for a normal amax
  byte = eb >= 8 ? eb - 8 : 0;
  inv = __builtin_bit_cast(float, (uint32_t)(eb >= 8 ? 262 - eb : 254) << 23);  // 1 / scale
}

// Four values to E4M3 bytes (round to nearest even; the caller has already saturated them).
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = 0;
  w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float sat448(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// ---------------------------------------------------------------- quantisation
// Q or K: four lanes per block of 32 consecutive bf16 values (32 features of one row and head),
// eight values each, so that a wave reads 1 KB and writes 512 bytes contiguously; the block's
// largest magnitude is exchanged among the four lanes.
__global__ __launch_bounds__(256) void mx_quantize_rows_kernel(const uint16_t* x, uint8_t* xq, uint8_t* xs,
                                                               long long n_blocks) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long i = t >> 2;  // block
  const int part = (int)(t & 3);
  const bool valid = i < n_blocks;
  float v[8];
  if (valid) {
    const uint4 w = *reinterpret_cast<const uint4*>(x + t * 8);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_lo(u[j]);
      v[2 * j + 1] = bf16_hi(u[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  if (!valid) return;
  int byte;
  float inv;
  mx_scale(amax, byte, inv);
  const uint32_t o0 = pack4_fp8(sat448(v[0] * inv), sat448(v[1] * inv), sat448(v[2] * inv), sat448(v[3] * inv));
  const uint32_t o1 = pack4_fp8(sat448(v[4] * inv), sat448(v[5] * inv), sat448(v[6] * inv), sat448(v[7] * inv));
  *reinterpret_cast<uint2*>(xq + t * 8) = make_uint2(o0, o1);
  if (part == 0) xs[i] = (uint8_t)byte;
}

// V: one workgroup per (64-key tile of a sequence, head); thread (d, g) quantises keys
// [32 g, 32 g + 32) of feature d. The tile is stored transposed, one 64-byte row per feature, with
// the keys in the order the PV product's A operand takes them: byte r of a row holds key
//   32 (r / 16 % 2) + 16 (r / 8 % 2) + 8 (r / 32) + r % 8,
// so the lane of half hh reads its 32 bytes contiguously at 32 hh. Scales: [tile][h][g][d].
__global__ __launch_bounds__(256) void mx_quantize_v_kernel(const uint16_t* v, const int32_t* tiles, int H,
                                                            uint8_t* vq, uint8_t* vs) {
  const int tile = blockIdx.x, h = blockIdx.y, d = threadIdx.x & 127, g = threadIdx.x >> 7;
  const int key0 = tiles[2 * tile], nvalid = tiles[2 * tile + 1];  // absolute first key row, keys in it
  float x[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int kk = 32 * g + j;
    x[j] = kk < nvalid ? bf16_lo(v[((size_t)(key0 + kk) * H + h) * 128 + d]) : 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
  int byte;
  float inv;
  mx_scale(amax, byte, inv);
  // keys 32 g + 16 b + 8 hh + j go to byte 32 hh + 16 g + 8 b + j
  uint32_t o[2][4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int j0 = 16 * b + 8 * hh + 4 * q;
        o[hh][2 * b + q] = pack4_fp8(sat448(x[j0] * inv), sat448(x[j0 + 1] * inv), sat448(x[j0 + 2] * inv), sat448(x[j0 + 3] * inv));
      }
  uint8_t* row = vq + (((size_t)tile * H + h) * 128 + d) * 64;
  *reinterpret_cast<uint4*>(row + 16 * g) = make_uint4(o[0][0], o[0][1], o[0][2], o[0][3]);
  *reinterpret_cast<uint4*>(row + 32 + 16 * g) = make_uint4(o[1][0], o[1][1], o[1][2], o[1][3]);
  vs[(((size_t)tile * H + h) * 2 + g) * 128 + d] = (uint8_t)byte;
}

// ---------------------------------------------------------------- forward
// LDS per stage of a three-stage ring (tile kt + 2 is loaded while tile kt is used): K tile 64
// keys x 128 bytes (16-byte chunk c of row r at c ^ (r & 7)), V^T tile 128 features x 64 bytes
// (chunk c of row r at c ^ ((r >> 1) & 3)), K scales (one word per key: its four feature blocks),
// V scales ([g][d] bytes).
struct alignas(16) MxSmem {
  unsigned char k[3][64 * 128];
  unsigned char vt[3][128 * 64];
  uint32_t ksc[3][64];
  unsigned char vsc[3][256];
  float tab[kBuckets];
  float diag[4][kDiagLen];
};

// Integer-valued running maximum (log2 units): a power-of-two rescale then commutes with the block
// quantisation of P, and a lazy threshold skips most rescales.
constexpr float kLazyMx = 8.0f;

template <int BIAS, int MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fwd_mx_kernel(MxArgs a) {
  constexpr int D = 128, BM = kFwdBM, BN = kFwdBN, NDB = D / 32;
  constexpr bool CAUSAL = MASK == kMaskCausal, BAND = MASK == kMaskBand;
  __shared__ MxSmem sm;

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const WorkRec w = load_item(a.f.items, blockIdx.x);
  const int h = w.h, t = w.tile, k0 = w.lo, k1 = w.hi, slot = w.slot;
  const int qs = w.qs, Lq = w.Lq, ks = w.ks, Lkv = w.Lkv;
  const int vtile0 = a.f.items[(size_t)blockIdx.x * kItemInts + 11];  // first 64-key tile of the sequence
  const int H = a.f.H;
  const int row0 = t * BM + wave * 32;
  const int qi = row0 + l32;
  const float inv_scale = 1.0f / a.f.scale;
  int klo = 0, khi = 0, wlo = 0, whi = 0, wlo_all = 0, whi_all = 0;
  if (BAND) {
    klo = band_key_lo(qi, a.f.band);
    khi = band_key_hi(qi, Lkv, a.f.band);
    wlo = band_key_lo(row0, a.f.band);
    whi = band_key_hi(row0 + 31, Lkv, a.f.band);
    wlo_all = band_key_lo(row0 + 31, a.f.band);
    whi_all = band_key_hi(row0, Lkv, a.f.band);
  }
  const float tabv = (BIAS == kBiasBucket && tid < kBuckets) ? a.f.bias[h * kBuckets + tid] : 0.0f;
  const float acc0 = (BIAS == kBiasScalar) ? a.f.bias[h] * inv_scale : 0.0f;  // in units of the unscaled score

  // Q fragment (B operand of S^T = K Q^T): for product m, bytes 0..15 are features 64 m + 16 hh + 0..15
  // and bytes 16..31 features 64 m + 32 + 16 hh + 0..15; scale: feature block 2 m + hh.
  i32x8 qf[2];
  int qsc[2];
  {
    const __amdgpu_buffer_rsrc_t qr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.qq) + ((size_t)qs * H + h) * D, (short)0,
                                          Lq > 0 ? (int)((Lq - 1) * H * D + D) : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t sr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.qs) + ((size_t)qs * H + h) * 4, (short)0,
                                          Lq > 0 ? (int)((Lq - 1) * H * 4 + 4) : 0, 0x00020000);
    typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t off = (uint32_t)(qi * H * D + 64 * m + 16 * hh);
      const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0);
      const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(qr, off + 32, 0, 0);
      qf[m] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    const uint32_t sw = __builtin_amdgcn_raw_buffer_load_b32(sr, (uint32_t)(qi * H * 4), 0, 0);
    qsc[0] = (int)((sw >> (8 * hh)) & 255);
    qsc[1] = (int)((sw >> (8 * (2 + hh))) & 255);
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;
  const float smul = a.f.scale * kLog2e;

  // K tile rows and scales, V^T tile and scales, loaded straight into LDS one tile ahead.
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.kq) + ((size_t)ks * H + h) * D, (short)0, Lkv > 0 ? (int)((Lkv - 1) * H * D + D) : 0,
      0x00020000);
  const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.ks) + ((size_t)ks * H + h) * 4, (short)0, Lkv > 0 ? (int)((Lkv - 1) * H * 4 + 4) : 0,
      0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.vq), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t vsr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.vs), (short)0, -1, 0x00020000);
  auto issue = [&](int kt, int st) {
    const int key0 = kt * BN;
    // K: 512 chunks of 16 bytes, two per lane; LDS slot i = 16 lane + 1024 wave (+ 4096 for u = 1)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 256 * u + 64 * wave + lane;  // slot
      const int r = i >> 3, cp = i & 7, c = cp ^ (r & 7);
      dma16(kr, (uint32_t)((key0 + r) * H * D + 16 * c), &sm.k[st][(256 * u + 64 * wave) * 16]);
    }
    // V^T: 512 chunks; slot i -> feature row r = i / 4, physical chunk i % 4 holds logical chunk
    // (i % 4) ^ ((r >> 1) & 3)
    const size_t vbase = ((size_t)(vtile0 + kt) * H + h) * (128 * 64);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 256 * u + 64 * wave + lane;
      const int r = i >> 2, cp = i & 3, c = cp ^ ((r >> 1) & 3);
      dma16(vr, (uint32_t)(vbase + 64 * r + 16 * c), &sm.vt[st][(256 * u + 64 * wave) * 16]);
    }
    if (wave == 0) dma4(ksr, (uint32_t)((key0 + lane) * H * 4), sm.ksc[st]);
    if (wave == 1) dma4(vsr, (uint32_t)(((size_t)(vtile0 + kt) * H + h) * 256 + 4 * lane), sm.vsc[st]);
  };

  if (k0 < k1) issue(k0, 0);
  if (k0 + 1 < k1) issue(k0 + 1, 1);
  if (BIAS == kBiasBucket) {
    if (tid < kBuckets) sm.tab[tid] = tabv;
    __syncthreads();
  }
  const int kr0 = kappa(l32);
  auto tile = [&](const int kt, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    const int key0 = kt * BN;
    const bool wskip =
        row0 >= Lq || (CAUSAL ? key0 > row0 + 31 : (BAND ? (key0 > whi || key0 + BN - 1 < wlo) : false));
    // Tile kt has landed once at most the next tile's loads are outstanding (four per wave, five
    // for the waves that also load the scales).
    if (kt + 1 >= k1)
      wait_vm();
    else if (wave < 2)
      wait_vm_keep<5>();
    else
      wait_vm_keep<4>();
    if (BIAS == kBiasBucket && !wskip) fill_diag(sm.diag[wave], sm.tab, key0 - row0 - 31, inv_scale, lane);
    __syncthreads();
    if (kt + 2 < k1) issue(kt + 2, (ST + 2) % 3);
    if (wskip) return;

    // S^T: A = K rows kappa(l32) + 32 sb; product m takes features 64 m + 16 hh (+ 32).
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
        // a per-head scalar enters the scores (it does not commute with the quantisation of P)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] = acc0;
      }
      const int r = kr0 + 32 * sb;
      const unsigned char* krow = &sm.k[ST][r * 128];
      const uint32_t ksw = sm.ksc[ST][r];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint4 lo = *reinterpret_cast<const uint4*>(krow + 16 * ((4 * m + hh) ^ (r & 7)));
        const uint4 hi = *reinterpret_cast<const uint4*>(krow + 16 * ((4 * m + 2 + hh) ^ (r & 7)));
        const i32x8 ka = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sacc[sb] = mfma_mx(ka, (int)((ksw >> (8 * (2 * m + hh))) & 255), qf[m], qsc[m], sacc[sb]);
      }
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
          sacc[sb][r] = masked ? kNegInf : sacc[sb][r];
        }
    }
    // Largest score of each 32-key block of the row (the lane's 16 and lane l^32's 16).
    float bm[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      bm[sb] = sacc[sb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) bm[sb] = fmaxf(bm[sb], sacc[sb][r]);
      bm[sb] = fmaxf(bm[sb], __shfl_xor(bm[sb], 32));
    }
    const float mx = fmaxf(bm[0], bm[1]) * smul;
    if (__ballot(mx > m_run + kLazyMx)) {
      const float m_new = ceilf(fmaxf(m_run, mx));
      const float alpha = m_new == kNegInf ? 0.0f : fast_exp2(m_run - m_new);  // a power of two
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_run = m_new;
    }
    const float nm = m_run == kNegInf ? 0.0f : -m_run;
    // P blocks: keys 32 sb .. 32 sb + 31 of the row, 16 values in each lane half. P~ = 2^x with
    // x = s smul - m_run, so the block's largest P~ is 2^xb (xb from its largest score) and its scale
    // exponent is se = max(floor(xb) - 8, -127) with no need to look at the P~ values themselves; the
    // scaled elements P~ / 2^se = 2^(x - se) come straight out of the exponential, and the row sum of
    // P~ is the block sums of the scaled elements times 2^se. A block with no visible key has
    // xb = -inf: its elements are 0 and its scale byte 0.
    float lsum = 0.0f;
    int pscb[2];
    i32x8 pb;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const float xb = __builtin_fmaf(bm[sb], smul, nm);
      const float se = bm[sb] == kNegInf ? -127.0f : fmaxf(floorf(xb) - 8.0f, -127.0f);
      pscb[sb] = (int)se + 127;
      const float c = nm - se;  // integers: exact
      float pq[16], bsum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = fast_exp2(__builtin_fmaf(sacc[sb][r], smul, c));
        bsum += x;
        pq[r] = fminf(x, 448.0f);
      }
      lsum += __builtin_ldexpf(bsum, (int)se);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pb[4 * sb + q] = (int)pack4_fp8(pq[4 * q], pq[4 * q + 1], pq[4 * q + 2], pq[4 * q + 3]);
    }
    l_run += lsum;
    const int psc = hh ? pscb[1] : pscb[0];  // lane half hh scales contraction block hh = keys 32 hh ..
    // O^T += V^T P^T: A = V^T rows 32 db + l32, the lane half's 32 bytes at 32 hh.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int r = 32 * db + l32;
      const unsigned char* vrow = &sm.vt[ST][r * 64];
      const int sw = (r >> 1) & 3;
      const uint4 lo = *reinterpret_cast<const uint4*>(vrow + 16 * ((2 * hh) ^ sw));
      const uint4 hi = *reinterpret_cast<const uint4*>(vrow + 16 * ((2 * hh + 1) ^ sw));
      const i32x8 va = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      o[db] = mfma_mx(va, (int)sm.vsc[ST][128 * hh + r], pb, psc, o[db]);
    }
  };
  for (int kt = k0; kt < k1; kt += 3) {
    tile(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < k1) tile(kt + 1, std::integral_constant<int, 1>{});
    if (kt + 2 < k1) tile(kt + 2, std::integral_constant<int, 2>{});
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (slot < 0) {
    if (qi < Lq) {
      if (hh == 0)
        a.f.lse[(size_t)h * a.f.Tq + qs + qi] =
            l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
      const size_t base = ((size_t)(qs + qi) * H + h) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(a.f.out, base + 32 * db + 8 * g + 4 * hh, o[db][4 * g] * inv, o[db][4 * g + 1] * inv,
                 o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv, a.f.out_f32);
    }
  } else if (qi < Lq) {
    const int prow = wave * 32 + l32;
    float* po = a.f.part_o + ((size_t)slot * BM + prow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * g + 4 * hh) =
            make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
    if (hh == 0) a.f.part_lse[(size_t)slot * BM + prow] = l_tot > 0.0f ? m_run + fast_log2(l_tot) : kNegInf;
  }
}

template <int BIAS>
hipError_t mx_launch_b(const MxArgs& a, const Modes& m, int n, hipStream_t s) {
  switch (m.mask_kind()) {
    case kMaskBand: hipLaunchKernelGGL((fwd_mx_kernel<BIAS, kMaskBand>), dim3(n), dim3(kThreads), 0, s, a); break;
    case kMaskCausal: hipLaunchKernelGGL((fwd_mx_kernel<BIAS, kMaskCausal>), dim3(n), dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((fwd_mx_kernel<BIAS, kMaskNone>), dim3(n), dim3(kThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quantize(const MxArgs& a, int Tq, int Tkv, int n_vtiles, hipStream_t s) {
  // four blocks of 32 features per row and head, four lanes per block
  const long long nq = (long long)Tq * a.f.H * 4, nk = (long long)Tkv * a.f.H * 4;
  if (nq > 0)
    hipLaunchKernelGGL(mx_quantize_rows_kernel, dim3((unsigned)((4 * nq + 255) / 256)), dim3(256), 0, s, a.f.q, a.qq, a.qs, nq);
  if (nk > 0)
    hipLaunchKernelGGL(mx_quantize_rows_kernel, dim3((unsigned)((4 * nk + 255) / 256)), dim3(256), 0, s, a.f.k, a.kq, a.ks, nk);
  if (n_vtiles > 0)
    hipLaunchKernelGGL(mx_quantize_v_kernel, dim3(n_vtiles, a.f.H), dim3(256), 0, s, a.f.v, a.vtiles, a.f.H, a.vq, a.vs);
  return hipGetLastError();
}

hipError_t launch_forward_mx(const MxArgs& a, const Modes& m, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  switch (m.bias) {
    case kBiasNone: return mx_launch_b<kBiasNone>(a, m, n_items, s);
    case kBiasScalar: return mx_launch_b<kBiasScalar>(a, m, n_items, s);
    default: return mx_launch_b<kBiasBucket>(a, m, n_items, s);
  }
}

}  // namespace jfa
