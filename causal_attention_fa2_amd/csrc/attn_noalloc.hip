// attn_noalloc.hip -- attn_bwd_qk_noalloc: the backward of attn_bwd_qk with its workspace taken
// from a file-scope device array instead of a caller-provided buffer, for callers that cannot
// allocate device memory (code under stream capture, serving loops, harnesses that forbid it).
//
// The array is `scratch` below: every device the library runs on holds its own copy, placed by the
// HIP runtime when the library's code object is loaded there and held until the process ends.
// Its address differs per device and is not the host-side symbol: it is looked up once per device
// with hipGetSymbolAddress (with that device current) and only that address is handed to kernels.
// The backward writes every word of its workspace before reading it, so nothing in the array has
// to be cleared between calls. All calls on one device share the array: calls that overlap in time
// on one device (different streams, or different host threads without ordering) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn.h"
#include "launch.h"

namespace {

static_assert(ATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device ordinal

// Device that work enqueued on `stream` runs on: the stream's own device, or the current device
// for the null stream.
int stream_device(void* stream, int* dev) {
  if (stream != nullptr) return hipStreamGetDevice(static_cast<hipStream_t>(stream), dev) == hipSuccess ? 0 : -1;
  return hipGetDevice(dev) == hipSuccess ? 0 : -1;
}

// Device address of `scratch` on `dev`, looked up on the first call for that device.
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return -1;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return -1;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return -1;
    if (e != hipSuccess || p == nullptr) return -1;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return 0;
}

}  // namespace

extern "C" int attn_bwd_qk_noalloc(int dtype, const void* q, const void* k, const void* v,
                                   const void* o, const float* lse, const void* dout, void* dq,
                                   void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk,
                                   int D, int causal, int window, int sink, float scale,
                                   void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_INVALID;
  const int st = fa::check_args(dtype, B, Hq, Hkv, Sq, Sk, D, causal, window, sink, scale);
  if (st != ATTN_OK) return st;
  // the head-split partials and the row vectors must fit; the sink split is used when it fits too
  if (fa::bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, D) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
    return ATTN_ERR_SCRATCH;
  int dev = -1;
  void* ws = nullptr;
  if (stream_device(stream, &dev) != 0 || scratch_on(dev, &ws) != 0) return ATTN_ERR_DEVICE;
  return attn_bwd_qk(dtype, q, k, v, o, lse, dout, dq, dk, dv, ws,
                     (size_t)ATTN_NOALLOC_SCRATCH_BYTES, B, Hq, Hkv, Sq, Sk, D, causal, window,
                     sink, scale, stream);
}
