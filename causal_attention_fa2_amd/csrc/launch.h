// launch.h -- host-side interface between the C ABI (attn_api.cpp) and the kernel launchers.
#ifndef ATTN_LAUNCH_H_
#define ATTN_LAUNCH_H_

#include <stddef.h>

namespace fa {

enum { kF32 = 0, kBF16 = 1 };

struct Args {
  int dtype;
  const void* q;
  const void* k;
  const void* v;
  const void* o_in;   // backward: forward output
  void* o;            // forward: output
  float* lse;         // forward: output; backward: input
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;       // backward workspace: rowsum(dO * O), [B, Hq, S]
  int B, Hq, Hkv, S, D;
  int causal, window;
  float scale;
  void* stream;
};

// Tells the launch observer (attn_set_launch_hook) that `kernel` is about to be / has been
// enqueued on `stream`.
void notify_launch(const char* kernel, int after, void* stream);

// Each returns 0 on success, -1 if the HIP runtime reported a launch error.
int launch_fwd(const Args& a);
int launch_bwd(const Args& a);

inline size_t bwd_workspace_bytes(int B, int Hq, int S) {
  size_t delta = (size_t)B * Hq * S * sizeof(float);
  return (delta + 255) / 256 * 256;
}

}  // namespace fa

#endif  // ATTN_LAUNCH_H_
