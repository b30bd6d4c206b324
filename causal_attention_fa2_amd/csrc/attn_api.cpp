// attn_api.cpp -- the extern "C" entry points declared in include/attn.h.
//
// Every argument check runs on the host before anything is enqueued, so a rejected call has no
// side effects. Readings of the definition that the checks enforce: Hq must be a multiple of Hkv
// (query heads split into equal contiguous groups, Grip paragraph of the "KYNETRA FOUNDRY" page);
// window 0 means no window and a window needs the causal mask (the single window parameter of
// "CUDA-LLM: A GitHub Repository for Development", section "The custom CUDA kernel", only ever
// narrows causal attention); with fewer queries than keys the queries are the last Sq positions
// (same section: one kernel for prefill and for one-token decode against a cache), and more
// queries than keys is not defined; sink keys ("KYNETRA FOUNDRY", Vaultecho paragraph) are a count
// >= 0 of leading keys that stay visible beside the window; a paged cache ("KYNETRA FOUNDRY",
// paged-KV paragraph) uses power-of-two blocks of at least 16 tokens; packed documents (page
// "Build a standalone, production grade system that trains a 4,...", curriculum section) take
// the causal mask, no sinks and at most kMaxDocs documents per batch row.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn.h"
#include "launch.h"

namespace {

attn_launch_hook_t g_hook = nullptr;
void* g_hook_user = nullptr;

}  // namespace

namespace fa {
int check_args(int dtype, int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int window,
               int sink, float scale) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk <= 0 || D <= 0) return ATTN_ERR_INVALID;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID;
  if (window < 0 || sink < 0) return ATTN_ERR_INVALID;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID;
  if (!causal && window > 0) return ATTN_ERR_UNSUPPORTED;
  // the kernels take a row's maximum of the raw scores and scale it afterwards: needs scale > 0
  if (!(scale > 0.f)) return ATTN_ERR_UNSUPPORTED;
  if (Sq > Sk) return ATTN_ERR_UNSUPPORTED;  // the queries are the last Sq of Sk positions
  const int64_t q_elems = (int64_t)B * Hq * Sq * D, kv_elems = (int64_t)B * Hkv * Sk * D;
  if (q_elems >= ((int64_t)1 << 31) || kv_elems >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

void notify_launch(const char* kernel, int after, void* stream) {
  attn_launch_hook_t h = g_hook;
  if (h) h(kernel, after, stream, g_hook_user);
}
}  // namespace fa

extern "C" {

void attn_set_launch_hook(attn_launch_hook_t hook, void* user) {
  g_hook_user = user;
  g_hook = hook;
}


int attn_fwd_qk(int dtype, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                int Hq, int Hkv, int Sq, int Sk, int D, int causal, int window, int sink,
                float scale, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID;
  int st = fa::check_args(dtype, B, Hq, Hkv, Sq, Sk, D, causal, window, sink, scale);
  if (st != ATTN_OK) return st;
  fa::Args a{};
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Sk = Sk;
  a.D = D;
  a.causal = causal;
  a.window = window;
  a.sink = sink;
  a.scale = scale;
  a.stream = stream;
  return fa::launch_fwd(a) == 0 ? ATTN_OK : ATTN_ERR_DEVICE;
}

int attn_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse, int B,
             int Hq, int Hkv, int S, int D, int causal, int window, float scale, void* stream) {
  return attn_fwd_qk(dtype, q, k, v, o, lse, B, Hq, Hkv, S, S, D, causal, window, 0, scale, stream);
}

size_t attn_bwd_qk_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
  if (fa::check_args(ATTN_BF16, B, Hq, Hkv, Sq, Sk, D, 1, 0, 0, 1.0f) != ATTN_OK) return 0;
  return fa::bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, D);
}

size_t attn_bwd_qk_workspace_bytes_for(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                                       int window, int sink) {
  if (fa::check_args(ATTN_BF16, B, Hq, Hkv, Sq, Sk, D, causal, window, sink, 1.0f) != ATTN_OK) return 0;
  return fa::bwd_workspace_bytes_for(B, Hq, Hkv, Sq, Sk, D, causal, window, sink);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D) {
  return attn_bwd_qk_workspace_bytes(B, Hq, Hkv, S, S, D);
}

int attn_bwd_qk(int dtype, const void* q, const void* k, const void* v, const void* o,
                const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                int window, int sink, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return ATTN_ERR_INVALID;
  int st = fa::check_args(dtype, B, Hq, Hkv, Sq, Sk, D, causal, window, sink, scale);
  if (st != ATTN_OK) return st;
  if (workspace_bytes < fa::bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)) return ATTN_ERR_INVALID;
  fa::Args a{};
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o_in = o;
  a.lse = const_cast<float*>(lse);
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const size_t row_bytes = fa::delta_bytes(B, Hq, Sq);
  a.delta = static_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + row_bytes);
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * row_bytes);
  // a workspace sized by attn_bwd_qk_workspace_bytes_for holds, after the rest, the sink-split
  // slots or the stored dS (a mask has at most one of the two; the stored dS is used in bf16)
  const size_t base_bytes = fa::bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, D);
  const size_t full_bytes = fa::bwd_workspace_bytes_for(B, Hq, Hkv, Sq, Sk, D, causal, window, sink);
  if (full_bytes > base_bytes && workspace_bytes >= full_bytes) {
    char* extra = static_cast<char*>(workspace) + base_bytes;
    if (fa::ds_bytes(B, Hq, Hkv, Sq, Sk, D, causal, window, sink) == 0) {
      a.xpart = reinterpret_cast<float*>(extra);
    } else if (dtype == fa::kBF16) {
      a.dsm = fa::ds_map(Hq, Hkv, Sq, Sk, causal);
      a.dsm.ds = reinterpret_cast<uint16_t*>(extra);
    }
  }
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Sk = Sk;
  a.D = D;
  a.causal = causal;
  a.window = window;
  a.sink = sink;
  a.scale = scale;
  a.stream = stream;
  return fa::launch_bwd(a) == 0 ? ATTN_OK : ATTN_ERR_DEVICE;
}

int attn_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D, int causal, int window,
             float scale, void* stream) {
  return attn_bwd_qk(dtype, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq,
                     Hkv, S, S, D, causal, window, 0, scale, stream);
}

int attn_fwd_paged(int dtype, const void* q, const void* k_pool, const void* v_pool,
                   const int* block_table, const int* seqlen_k, void* o, float* lse, int B, int Hq,
                   int Hkv, int Sq, int D, int block_size, int max_blocks, int num_blocks,
                   int causal, int window, int sink, float scale, void* stream) {
  if (!q || !k_pool || !v_pool || !block_table || !seqlen_k || !o || !lse) return ATTN_ERR_INVALID;
  if (block_size <= 0 || max_blocks <= 0 || num_blocks <= 0) return ATTN_ERR_INVALID;
  if ((block_size & (block_size - 1)) != 0 || block_size < 16 || block_size > (1 << 20))
    return ATTN_ERR_UNSUPPORTED;
  const int64_t capacity = (int64_t)max_blocks * block_size;  // keys one sequence can hold
  if (capacity >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;
  // Sk = Sq here only for the shared checks; each sequence's own Sk comes from seqlen_k
  int st = fa::check_args(dtype, B, Hq, Hkv, Sq, Sq, D, causal, window, sink, scale);
  if (st != ATTN_OK) return st;
  if (Sq > capacity) return ATTN_ERR_UNSUPPORTED;
  fa::Args a{};
  a.dtype = dtype;
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Sk = Sq;  // replaced per sequence on the device
  a.D = D;
  a.causal = causal;
  a.window = window;
  a.sink = sink;
  a.scale = scale;
  a.stream = stream;
  a.paged = true;
  a.pg.table = block_table;
  a.pg.seqlen = seqlen_k;
  a.pg.shift = __builtin_ctz((unsigned)block_size);
  a.pg.max_blocks = max_blocks;
  a.pg.num_blocks = num_blocks;
  return fa::launch_fwd(a) == 0 ? ATTN_OK : ATTN_ERR_DEVICE;
}

int attn_fwd_varlen(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int n_docs, int B, int Hq, int Hkv, int S, int D,
                    int window, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return ATTN_ERR_INVALID;
  if (n_docs <= 0) return ATTN_ERR_INVALID;
  if (n_docs > fa::kMaxDocs) return ATTN_ERR_UNSUPPORTED;
  int st = fa::check_args(dtype, B, Hq, Hkv, S, S, D, 1, window, 0, scale);
  if (st != ATTN_OK) return st;
  fa::Args a{};
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = S;
  a.Sk = S;
  a.D = D;
  a.causal = 1;
  a.window = window;
  a.scale = scale;
  a.stream = stream;
  a.docs.cu = cu_seqlens;
  a.docs.n = n_docs;
  return fa::launch_fwd(a) == 0 ? ATTN_OK : ATTN_ERR_DEVICE;
}

int attn_bwd_varlen(int dtype, const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, const int* cu_seqlens, int n_docs,
                    int B, int Hq, int Hkv, int S, int D, int window, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace || !cu_seqlens)
    return ATTN_ERR_INVALID;
  if (n_docs <= 0) return ATTN_ERR_INVALID;
  if (n_docs > fa::kMaxDocs) return ATTN_ERR_UNSUPPORTED;
  int st = fa::check_args(dtype, B, Hq, Hkv, S, S, D, 1, window, 0, scale);
  if (st != ATTN_OK) return st;
  if (workspace_bytes < fa::bwd_workspace_bytes(B, Hq, Hkv, S, S, D)) return ATTN_ERR_INVALID;
  fa::Args a{};
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o_in = o;
  a.lse = const_cast<float*>(lse);
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const size_t row_bytes = fa::delta_bytes(B, Hq, S);
  a.delta = static_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + row_bytes);
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * row_bytes);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = S;
  a.Sk = S;
  a.D = D;
  a.causal = 1;
  a.window = window;
  a.scale = scale;
  a.stream = stream;
  a.docs.cu = cu_seqlens;
  a.docs.n = n_docs;
  return fa::launch_bwd(a) == 0 ? ATTN_OK : ATTN_ERR_DEVICE;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int max_keys, int D) {
  if (fa::check_args(ATTN_BF16, B, Hq, Hkv, Sq, max_keys, D, 1, 0, 0, 1.0f) != ATTN_OK) return 0;
  if ((Hq / Hkv) * Sq > 32) return 0;
  return fa::decode_workspace_bytes(B, Hq, Hkv, Sq, max_keys, D);
}

int attn_decode_fwd(int dtype, const void* q, const void* k, const void* v, const int* block_table,
                    const int* seqlen_k, void* o, float* lse, void* workspace,
                    size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                    int block_size, int max_blocks, int num_blocks, int causal, int window, int sink,
                    float scale, void* stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return ATTN_ERR_INVALID;
  const bool paged = block_table != nullptr || seqlen_k != nullptr;
  if (paged && (!block_table || !seqlen_k)) return ATTN_ERR_INVALID;
  fa::Args a{};
  int max_keys = Sk;
  if (paged) {
    if (block_size <= 0 || max_blocks <= 0 || num_blocks <= 0) return ATTN_ERR_INVALID;
    if ((block_size & (block_size - 1)) != 0 || block_size < 16 || block_size > (1 << 20))
      return ATTN_ERR_UNSUPPORTED;
    const int64_t capacity = (int64_t)max_blocks * block_size;
    if (capacity >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;
    max_keys = (int)capacity;
    a.paged = true;
    a.pg.table = block_table;
    a.pg.seqlen = seqlen_k;
    a.pg.shift = __builtin_ctz((unsigned)block_size);
    a.pg.max_blocks = max_blocks;
    a.pg.num_blocks = num_blocks;
  }
  int st = fa::check_args(dtype, B, Hq, Hkv, Sq, max_keys, D, causal, window, sink, scale);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16 || (Hq / Hkv) * Sq > 32) return ATTN_ERR_UNSUPPORTED;
  if (workspace_bytes < fa::decode_workspace_bytes(B, Hq, Hkv, Sq, max_keys, D)) return ATTN_ERR_INVALID;
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Sk = max_keys;  // the dense key count; replaced per sequence on the device when paged
  a.D = D;
  a.causal = causal;
  a.window = window;
  a.sink = sink;
  a.scale = scale;
  a.stream = stream;
  return fa::launch_decode(a, static_cast<float*>(workspace), max_keys) == 0 ? ATTN_OK
                                                                              : ATTN_ERR_DEVICE;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_DEVICE: return "HIP runtime error at launch";
    case ATTN_ERR_SCRATCH: return "problem needs more than the static scratch buffer holds";
    default: return "unknown status";
  }
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
