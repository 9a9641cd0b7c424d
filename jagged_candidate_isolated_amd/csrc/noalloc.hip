// Full-sequence forward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
// plan and kernels as rr_attn_fwd, with what rr_attn_fwd keeps in its workspace (the plan,
// and for wide-tile batches the key-norm bounds) in a file-scope device array instead of a
// caller-provided workspace.
//
// Each GPU the library runs on holds its own copy of the array (kScratchBytes) until the
// process ends.  Host code never uses the array's name as an address: on the first
// call on a device (with that device current) the device address is looked up with
// hipGetSymbolAddress and kept per device.  Every call on a GPU shares that GPU's array
// and overwrites the plan the previous call left there; the plan, and any bounds a call
// reads, are rewritten in full by that call (nothing must start at zero), so calls in
// stream order are independent, while calls that overlap on one GPU (other streams or
// threads) race.
#include <mutex>

#include "rr_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // the device address of `scratch` on each device

// The current device's copy of `scratch` into *out; RR_OK or RR_EHIP.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RR_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RR_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RR_OK;
}

}  // namespace

extern "C" {

size_t rr_attn_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

int rr_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, const int32_t* offsets,
                        const int32_t* cand_start, const uint8_t* valid, int attend_padded_history, int32_t B,
                        int32_t T, int32_t H, int32_t d, int dtype, float scale, hipStream_t stream) {
  const size_t need = rr_attn_workspace_bytes(B, T, H, d);
  if (need == 0 || B == 0 || T == 0 || H == 0) {
    // invalid sizes, or an empty call: rr_attn_fwd returns its error (or RR_OK) from the
    // host-side checks before it would touch a workspace
    return rr_attn_fwd(q, k, v, o, offsets, cand_start, valid, attend_padded_history, B, T, H, d, dtype, scale,
                       nullptr, 0, stream);
  }
  if (need > kScratchBytes) return RR_EUNSUPPORTED;
  void* ws = nullptr;
  const int r = scratch_on_current_device(&ws);
  if (r != RR_OK) return r;
  return rr_attn_fwd(q, k, v, o, offsets, cand_start, valid, attend_padded_history, B, T, H, d, dtype, scale, ws,
                     kScratchBytes, stream);
}

}  // extern "C"
