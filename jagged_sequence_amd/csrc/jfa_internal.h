// Internal interface between the host planner / ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace jfa {

// Tile geometry. Query-tile kernels (forward, dQ) run 4 waves x 32 query rows = 128 rows and walk
// the keys 64 at a time; the dK/dV kernel runs 4 waves x 32 keys = 128 keys and walks the queries
// 64 at a time. Every wave owns 32 rows/columns of one 32x32 MFMA block.
constexpr int kFwdBM = 128, kFwdBN = 64;
constexpr int kDqBM = 128, kDqBN = 64;
constexpr int kKvBM = 64, kKvBN = 128;
// When every sequence has at most kKvBM queries (one query tile), dK/dV items are latency bound;
// softmax with D = 128 then uses half-width items (64 keys, 4-wave workgroups, two per CU).
constexpr int kKvBNShort = 64;
constexpr int kThreads = 256;
// Device work records carry the sequence's offsets and lengths, so a workgroup starts with a single
// load of its record (no dependent load of the offset arrays):
//   item:  b, h, tile, lo, hi, slot, qs, Lq, ks, Lkv, first, 0 x 5
//          (first = 1 on an unsplit item and on the first piece of a split one)
//   group: b, h, tile, slot0, R, qs, Lq, ks, Lkv, 0 x 7
constexpr int kItemInts = 16;
constexpr int kGroupInts = 16;
constexpr int kBuckets = 64;
// Largest (sequence, head) slice of a [T, H, D] tensor the kernels address with 32-bit offsets.
constexpr long long kMaxSliceElems = 1ll << 30;
// Work queues of the persistent dK/dV kernel (D = 128): one per XCD, then one counter of the dQ
// partial-sum tasks that the same kernel takes once its items are exhausted.
constexpr int kQueues = 8;
constexpr int kQueueCounters = kQueues + 1;

enum Act { kSoftmax = 0, kSilu = 1, kGeluTanh = 2 };
// Mask template argument of the attention kernels. kMaskBand covers a window and / or a block
// limit (with or without the causal limit, given at run time): every lane derives the interval of
// positions it may pair with, so one comparison pair masks a score whatever limits are on.
enum MaskKind { kMaskNone = 0, kMaskCausal = 1, kMaskBand = 2 };

// Run-time limits of kMaskBand (0 = off).
struct Band {
  int window;
  int block;
  int causal;
};
enum BiasKind { kBiasNone = 0, kBiasScalar = 1, kBiasBucket = 2 };

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* bias;
  void* out;
  float* lse;
  float* part_o;    // [slots][kFwdBM][D] fp32: per-piece normalised output (softmax) or raw sum (GDPA)
  float* part_lse;  // [slots][kFwdBM] fp32: per-piece log2-sum-exp2 (softmax)
  const int32_t* items;
  const int32_t* groups;
  int H;
  int Tq;
  float scale;
  int out_f32;
  Band band;
  int q_shared;  // every sequence reads query rows from row 0 of q (shared queries); out and lse stay per sequence
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* bias;
  const void* out;
  const float* lse;
  const uint16_t* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;    // [H][Tq] fp32 (softmax): Delta = rowsum(dO * O), written by the dQ kernel
  float* part_dq;  // [slots][kDqBM][D]
  float* part_dk;  // [slots][kKvBN][D]
  float* part_dv;  // [slots][kKvBN][D]
  unsigned long long* dbias_acc;  // [H][bins] bias-gradient sums in 2^-32 fixed point (two's complement)
  float* dbias;                   // [H][bins] output (bins = 64 for the bucket table, 1 for the scalar)
  const int32_t* dq_items;
  const int32_t* dq_groups;
  const int32_t* kv_items;
  const int32_t* kv_groups;
  int H;
  int Tq;
  int Tkv;
  float scale;
  int out_f32;
  int grad_f32;
  int kv_bn;  // keys per dK/dV item (kKvBN or kKvBNShort)
  int* kv_queue;  // kQueueCounters counters of the dK/dV work queue (D = 128); the dQ kernel zeroes them
  int kv_n;       // dK/dV items
  int dq_reduce_n;  // dQ split groups whose fixed-order sums the persistent dK/dV kernel takes (else 0)
  Band band;
  int q_shared;  // query rows shared by every sequence (read from row 0 of q); dq is summed over sequences
};

// MXFP8 forward: the forward arguments plus the quantised copies (in the forward workspace).
struct MxArgs {
  FwdArgs f;
  uint8_t* qq;  // [Tq][H][D] E4M3
  uint8_t* qs;  // [Tq][H][D / 32] E8M0
  uint8_t* kq;  // [Tkv][H][D] E4M3
  uint8_t* ks;  // [Tkv][H][D / 32] E8M0
  uint8_t* vq;  // [tiles][H][D][64] E4M3, transposed 64-key tiles of every sequence
  uint8_t* vs;  // [tiles][H][2][D] E8M0
  const int32_t* vtiles;  // [tiles][2]: first key row (absolute) and keys in the tile
};

struct Modes {
  int D;
  int act;
  int bias;
  int causal;
  int dbias;     // the bias gradient is requested
  int kv_short;  // dK/dV items of kKvBNShort keys (D = 128, every Lq <= kKvBM)
  int band;      // a window or block limit is on (kMaskBand kernels)
  int mask_kind() const { return band ? kMaskBand : (causal ? kMaskCausal : kMaskNone); }
};

// Bias template argument of the dK/dV kernels: kBiasScalar / kBiasBucket, plus kBiasGrad when the
// kernel also accumulates the bias gradient.
constexpr int kBiasGrad = 4;

// Launchers (defined next to their kernels). Each returns the hipGetLastError() of its launch.
hipError_t launch_forward(const FwdArgs& a, const Modes& m, int n_items, hipStream_t s);
hipError_t launch_forward_combine(const FwdArgs& a, const Modes& m, int n_groups, hipStream_t s);
// n_items dK/dV items; at D = 128 the kernel is persistent and runs min(n_items, resident)
// workgroups (resident = how many the GPU holds at once).
hipError_t launch_bwd_dkdv(const BwdArgs& a, const Modes& m, int n_items, int resident, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, const Modes& m, int n_items, hipStream_t s);
hipError_t launch_bwd_reduce_dq(const BwdArgs& a, const Modes& m, int n_groups, hipStream_t s);
// The same fixed-order sums spread over one workgroup per (group, row), for groups of many pieces.
hipError_t launch_bwd_reduce_dq_wide(const BwdArgs& a, const Modes& m, int n_groups, hipStream_t s);
// Fused backward of plans whose sequences all have at most kKvBM queries (D = 128, no band limits):
// one workgroup per dQ item computes dQ (or its partial) and the dK / dV of the item's keys.
hipError_t launch_bwd_fused(const BwdArgs& a, const Modes& m, int n_items, hipStream_t s);
hipError_t launch_bwd_reduce_dkdv(const BwdArgs& a, const Modes& m, int n_groups, hipStream_t s);
// Clears the bias-gradient totals (when a.dbias_acc is set) and the dK/dV queue counters.
hipError_t launch_bwd_dbias_clear(const BwdArgs& a, const Modes& m, hipStream_t s);
hipError_t launch_bwd_dbias_finish(const BwdArgs& a, const Modes& m, hipStream_t s);

}  // namespace jfa

#include "jfa.h"

namespace jfa {

// jfa_backward with a workspace obtained from `workspace(bytes, &status)` after the argument checks
// (which may refuse the size with a status); no timing and no use-tracking events are recorded.
jfa_status backward_into(jfa_plan_s* P, const void* q, const void* k, const void* v, const int32_t* q_offsets,
                         const int32_t* kv_offsets, const float* bias, const void* out, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* dbias,
                         void* (*workspace)(size_t, jfa_status*), hipStream_t s);
// Sets the thread's last-error text and returns s.
jfa_status set_error(jfa_status s, const char* msg);

// MXFP8 forward (D = 128, softmax): quantisation of Q, K and V, then the attention kernel.
hipError_t launch_mx_quantize(const MxArgs& a, int Tq, int Tkv, int n_vtiles, hipStream_t s);
hipError_t launch_forward_mx(const MxArgs& a, const Modes& m, int n_items, hipStream_t s);

// Resident workgroups per CU of each kernel for the given modes (occupancy query).
int occupancy_forward(const Modes& m);
int occupancy_dq(const Modes& m);
int occupancy_dkdv(const Modes& m);

}  // namespace jfa
