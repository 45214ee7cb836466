// noalloc.hip - smoe_moe_layer_noalloc: one whole layer call that allocates
// nothing and takes no workspace argument, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The scratch the layer's kernels need (the status word and tickets, logits,
// prepped activations and their sums and token scales, h, per-pair outputs,
// the decode metadata) lives in `scratch` below: a file-scope device array of
// kScratchBytes, which every GPU the library runs on holds until the process
// ends.  Its device address is taken once per device with
// hipGetSymbolAddress (the array's name is a host-side stand-in in host
// code, never a device address) and kept per device; that set-up also
// clears the status area with a fill kernel on the caller's stream.
//
// All calls on one GPU share that GPU's array and it keeps the last call's
// contents: calls that may overlap on one GPU (different streams, or host
// threads without ordering) race on it.  Calls ordered on one stream are
// fine; the kernels' tickets return to zero at the end of every call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "smoe_internal.hpp"

#define SMOE_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;   // 16 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` per device

// The current device's address of `scratch`, setting it up on first use:
// hipGetSymbolAddress with that device current, then the status area (the
// workspace's first 256 bytes: status bits and tickets) cleared by a fill
// kernel on `s`, ahead of the call's own kernels.
hipError_t scratch_for_current_device(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255) != 0) return hipErrorInvalidValue;
    err = smoe::launch_fill_u32(static_cast<uint32_t*>(p), 0u, 64, s);
    if (err != hipSuccess) return err;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

SMOE_API size_t smoe_noalloc_scratch_bytes(void) { return kScratchBytes; }

SMOE_API int smoe_moe_layer_noalloc(const smoe_layer_desc* desc, const void* router_w,
                                    const smoe_experts* experts, const float* x, int32_t B,
                                    const float* residual, float* out, float* logits,
                                    int32_t* topk_idx, float* topk_w, const smoe_union* un,
                                    void* stream) {
  // the size check needs a valid descriptor and batch; layer_setup repeats
  // both checks together with the rest
  if (desc == nullptr) return SMOE_EINVAL;
  const size_t need = smoe_workspace_size(desc, B < 1 ? 1 : B);
  if (B >= 1 && B <= SMOE_MAX_BATCH && need > kScratchBytes) return SMOE_EWORKSPACE;
  // validate everything before touching the device (nothing is set up or
  // launched for a call that fails here); the scratch is only named by its
  // size, so any 256-byte aligned placeholder address passes the checks
  smoe::RouteArgs r;
  smoe::FfnArgs a;
  void* const placeholder = reinterpret_cast<void*>((uintptr_t)256);
  int rc = smoe::layer_setup(desc, router_w, experts, x, B, residual, out, logits, topk_idx,
                             topk_w, un, placeholder, kScratchBytes, &r, &a);
  if (rc != SMOE_OK || B == 0) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (scratch_for_current_device(s, &ws) != hipSuccess) return SMOE_EHIP;
  rc = smoe::layer_setup(desc, router_w, experts, x, B, residual, out, logits, topk_idx, topk_w,
                         un, ws, kScratchBytes, &r, &a);
  if (rc != SMOE_OK) return rc;
  return smoe::launch_layer(r, a, s) == hipSuccess ? SMOE_OK : SMOE_EHIP;
}
