// am_compact_head_noalloc: am_compact_head with its scratch in a fixed device array of this
// library instead of a caller-supplied workspace, for callers that cannot allocate device
// memory (code captured into graphs, tight serving loops, harnesses that forbid it).
//
// The array `scratch` below is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy (kNoallocScratchBytes) from the first call on that device until the
// process ends. In host code its name only stands in for the symbol; the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with that device
// current, and is the only form in which host code hands the array to kernels. All calls on
// one GPU share that GPU's copy: calls that overlap on one GPU (different streams, or other
// host threads) race on it and must be serialized by the caller. Nothing in it needs to
// start at zero: every kernel of the path writes what it later reads, and the few counters
// the path uses are cleared by its own launches.
#include <mutex>

#include "../../include/am.h"
#include "am_internal.hpp"

namespace {

constexpr size_t kNoallocScratchBytes = AM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (taken on the first call on that device).
am_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return AM_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return AM_ERR_DEVICE;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return AM_OK;
}

}  // namespace

extern "C" am_status am_compact_head_noalloc(const am_problem* p, const void* Q, const void* K,
                                             const void* V, int64_t t, const am_options* opt,
                                             int32_t* idx, void* Ck, float* beta, float* Cv,
                                             float* lse_out, float* O_out, float* score_out,
                                             float* resid_out, int32_t* head_status,
                                             am_stream_t stream) {
  // the problem's workspace need, validated like am_compact_head's arguments (0: invalid)
  const size_t need = am_workspace_bytes(p, t, AM_CALL_COMPACT);
  if (need == 0) {
    // let am_compact_head report the precise error; it launches nothing on invalid input
    return am_compact_head(p, Q, K, V, t, opt, idx, Ck, beta, Cv, lse_out, O_out, score_out,
                           resid_out, head_status, nullptr, 0, stream);
  }
  if (need > kNoallocScratchBytes) return AM_ERR_WORKSPACE;
  void* ws = nullptr;
  const am_status st = scratch_ptr(&ws);
  if (st != AM_OK) return st;
  return am_compact_head(p, Q, K, V, t, opt, idx, Ck, beta, Cv, lse_out, O_out, score_out,
                         resid_out, head_status, ws, kNoallocScratchBytes, stream);
}
