// Allocation-free backward pass: jfa_backward with the workspace taken from a static device array of
// fixed size instead of the caller, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array (`scratch`) exists once per GPU the library runs on and lives until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only a stand-in for the
// symbol): on the first call on a device, with that device current, its device address is looked
// up with hipGetSymbolAddress and kept per device; launches get that address.
//
// The backward kernels need nothing in the workspace to start at zero from an earlier call: the dQ
// kernel (or a clear kernel) zeroes the dK/dV work-queue counters and the bias-gradient totals
// before they are used, and every other region (Delta, split partial results) is written before it
// is read. Calls that overlap on one GPU (several streams or threads at once) share the array and
// race; they must be ordered by the caller.
#include <mutex>
#include <vector>

#include "jfa.h"
#include "jfa_internal.h"

constexpr size_t kScratchBytes = JFA_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
std::vector<void*> g_scratch;  // device address of `scratch`, per device (nullptr: not looked up yet)

// Device address of this device's scratch array (looked up once per device, device current).
void* scratch_address(size_t need, jfa_status* st) {
  if (need > kScratchBytes) {
    *st = jfa::set_error(JFA_ERR_WORKSPACE,
                         "the plan's backward workspace exceeds the allocation-free scratch array "
                         "(JFA_NOALLOC_SCRATCH_BYTES); use jfa_backward with a workspace");
    return nullptr;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = jfa::set_error(JFA_ERR_HIP, "hipGetDevice failed");
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *st = jfa::set_error(JFA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  *st = JFA_OK;
  return g_scratch[dev];
}

}  // namespace

extern "C" jfa_status jfa_backward_noalloc(jfa_plan_t plan, const void* q, const void* k, const void* v,
                                           const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias,
                                           const void* out, const float* lse, const void* dout, void* dq, void* dk,
                                           void* dv, float* dbias, jfa_stream_t stream) {
  return jfa::backward_into(plan, q, k, v, q_offsets, kv_offsets, bias, out, lse, dout, dq, dk, dv, dbias,
                            scratch_address, (hipStream_t)stream);
}
