// Decode attention that allocates nothing: its workspace is a file-scope
// device array (one copy on every GPU the library runs on, held until the
// process ends) instead of a caller buffer, for callers that cannot allocate
// device memory (code under stream capture, tight serving loops).  The
// array's device address is looked up once per device with
// hipGetSymbolAddress, with that device current; host code uses only that
// address, never the array's name.  The decode kernels write every
// workspace byte they read (the prepared queries, then the split-K
// partials), so nothing in it has to start at zero.  All calls on one GPU
// share its array: calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tq_internal.h"

namespace {

constexpr size_t kScratchBytes = TQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on `device` (looked up on the first call for
// that device, with the device current).
tq_status scratch_on(int device, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return TQ_EDEVICE;
    if (hipSetDevice(device) != hipSuccess) return TQ_EDEVICE;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return TQ_EDEVICE;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return TQ_OK;
}

}  // namespace

extern "C" tq_status tq_decode_attend_noalloc(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                                              int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                              const tq_kv_view* kv, float softmax_scale, float* out,
                                              void* stream) {
  if (!kcb || !vcb || !kv) return TQ_EINVAL;
  if (kcb->device < 0 || kcb->device >= kMaxDevices) return TQ_EINVAL;
  if (B < 0 || Hq < 0 || kv->max_tokens < 0) return TQ_EINVAL;
  const size_t need = tq_workspace_size(kcb, TQ_OP_DECODE, int64_t(B) * Hq, kv->max_tokens, Hkv);
  if (need > kScratchBytes) return TQ_EWORKSPACE;
  void* ws = nullptr;
  const tq_status st = scratch_on(kcb->device, &ws);
  if (st != TQ_OK) return st;
  return tq::decode_attend_ws(kcb, vcb, q, q_dtype, B, Hq, Hkv, kv, softmax_scale, out, ws, kScratchBytes, stream);
}
