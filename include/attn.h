/*
 * attn.h -- C ABI of the MI355X (gfx950) causal / sliding-window grouped-query attention library
 * (libattn.so): a tiled forward that writes O and the per-row log-sum-exp, and a backward that
 * takes dO and writes dQ, dK and dV.
 *
 * What the calls compute:
 *   "KYNETRA FOUNDRY" page, FlashAttention paragraph: for each query tile the kernel streams key /
 *   value tiles through on-chip memory with a running-max / running-sum softmax, never writing the
 *   S x S score matrix to HBM; numerics are those of plain attention; the backward recomputes tiles.
 *   Same page, Grip paragraph: query heads are partitioned into groups that share one K/V head.
 *   Same page, decoder-block paragraph: the causal mask is strict left-to-right.
 *   "CUDA-LLM: A GitHub Repository for Development", section "The custom CUDA kernel": one window
 *   parameter switches between full-causal and sliding-window attention; the backward recomputes the
 *   softmax probabilities from the saved log-sum-exp; the kernel also takes fewer queries than keys
 *   (Sq <= Sk), for a prefill chunk or a one-token decode step against a cache.
 *   "KYNETRA FOUNDRY" page, Vaultecho paragraph: beside the sliding window a few persistent sink
 *   tokens at the start of the sequence stay attended. Same page, paged-KV paragraph: a sequence's
 *   K/V cache lives in fixed-size blocks anywhere in a global pool, found through a per-sequence
 *   block table (attn_fwd_paged).
 *   "Build a standalone, production grade system that trains a 4,..." (page-4 prompt), curriculum
 *   section: documents are packed contiguously into fixed-length buffers with document-boundary
 *   index arrays, attention being reset at each boundary (attn_fwd_varlen / attn_bwd_varlen).
 *
 * Definitions (for b < B, query head h < Hq, KV head g = h / (Hq / Hkv), rows i < Sq, keys j < Sk;
 * the queries are the last Sq positions, query i standing at p = i + Sk - Sq):
 *   visible(i, j) = (causal == 0 || j <= p) && (window == 0 || p - j < window || j < sink)
 *   x_ij   = scale * <Q[b,h,i,:], K[b,g,j,:]>            (visible j only)
 *   lse_i  = ln( sum_j exp(x_ij) )                       (natural log of the scaled scores)
 *   P_ij   = exp(x_ij - lse_i),  O_i = sum_j P_ij V[b,g,j,:]
 *   dQ_i   = scale * sum_j dS_ij K_j,  dK_j = scale * sum_{h in group(g)} sum_i dS_ij Q_i,
 *   dV_j   = sum_{h in group(g)} sum_i P_ij dO_i,  with dS_ij = P_ij (<dO_i, V_j> - <dO_i, O_i>).
 *   A window W >= 1 lets query i see keys p-W+1 .. p (W counts the diagonal). W = 0: no window.
 *   A single query (Sq = 1) sees every key causally, or the last W (plus the sink keys).
 *   sink >= 0 counts the leading keys that stay visible once the window has moved past them; it only
 *   matters with a window (without one every earlier key is visible anyway).
 *   attn_fwd / attn_bwd are the square case Sq = Sk = S of attn_fwd_qk / attn_bwd_qk.
 *
 * Layout: Q, O, dO, dQ are [B, Hq, Sq, D]; K, V, dK, dV are [B, Hkv, Sk, D]; lse is [B, Hq, Sq].
 * All are dense and contiguous with D fastest, element type `dtype` (lse is always float32).
 *
 * Ownership and execution: every pointer is a DEVICE pointer owned by the caller. The library
 * never allocates (its one static array, attn_bwd_qk_noalloc's scratch, is placed by the HIP
 * runtime on each device where the library's code is loaded), never synchronises the host, keeps no per-call state, and enqueues all of its
 * work on `stream` (a hipStream_t; NULL = the default stream). Outputs must not alias inputs.
 * Calls on different streams may run concurrently; results are deterministic (no atomics).
 *
 * Errors: arguments are checked on the host before anything is enqueued; a failed check returns a
 * status and enqueues nothing. A launch failure reported by the HIP runtime returns
 * ATTN_ERR_DEVICE. Faults during execution surface at the caller's next synchronisation.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 8

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,     /* null pointer, size <= 0, Hq % Hkv != 0, window < 0, sink < 0,
                               non-finite scale, workspace too small, n_docs <= 0 */
  ATTN_ERR_UNSUPPORTED = 2, /* D not 64 or 128, unknown dtype, window > 0 without causal,
                               Sq > Sk, B*Hq*Sq*D or B*Hkv*Sk*D >= 2^31, a paged block size
                               that is not a power of two in [16, 2^20], n_docs > 2047,
                               scale <= 0 (the kernels take each row's maximum of the raw scores
                               before scaling, which needs scale > 0) */
  ATTN_ERR_DEVICE = 3,      /* the HIP runtime reported an error for a launch */
  ATTN_ERR_SCRATCH = 4      /* attn_bwd_qk_noalloc: the problem needs more workspace than its
                               static scratch array holds (ATTN_NOALLOC_SCRATCH_BYTES) */
} attn_status_t;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* Forward. Reads q [B,Hq,S,D], k and v [B,Hkv,S,D]; writes o [B,Hq,S,D] (dtype, fp32 accumulation
 * rounded to nearest even) and lse [B,Hq,S] (float32, natural log). */
int attn_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int S, int D, int causal, int window, float scale,
             void* stream);

/* Bytes of device workspace attn_bwd needs for these sizes: the per-row delta = rowsum(dO * O)
 * and lse * log2(e) (B*Hq*S fp32 each, 256-byte aligned) and, when the dK/dV pass splits a
 * query-head group across workgroups, fp32 partial sums of dK and dV (2 * parts * B*Hkv*S*D
 * fp32). Returns 0 for sizes attn_bwd would reject. */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D);

/* Backward. o and lse must be exactly what attn_fwd wrote for the same q, k, v and arguments.
 * dout [B,Hq,S,D] is the gradient of the loss with respect to o. Writes dq [B,Hq,S,D] and dk, dv
 * [B,Hkv,S,D]; all three are fully overwritten (not accumulated into). `workspace` is a device
 * buffer of at least attn_bwd_workspace_bytes(...) bytes; its contents on entry do not matter.
 * One of attn_bwd_qk_workspace_bytes_for(B, Hq, Hkv, S, S, D, causal, window, 0) bytes also holds
 * the stored dS where that is used (see there). */
int attn_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes,
             int B, int Hq, int Hkv, int S, int D, int causal, int window, float scale,
             void* stream);

/* Forward with Sq queries against Sk >= Sq keys (bottom-right causal alignment) and `sink` sink
 * keys (see above). Reads q [B,Hq,Sq,D], k and v [B,Hkv,Sk,D]; writes o [B,Hq,Sq,D] and lse
 * [B,Hq,Sq]. attn_fwd is this call with Sq = Sk = S and sink = 0. */
int attn_fwd_qk(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int window, int sink,
                float scale, void* stream);

/* Workspace bytes of attn_bwd_qk: delta and lse * log2(e) (B*Hq*Sq fp32 each, 256-byte aligned)
 * and, when the head group is split, 2 * parts * B*Hkv*Sk*D fp32. 0 for rejected sizes. */
size_t attn_bwd_qk_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D);

/* Workspace bytes of attn_bwd_qk for these exact mask arguments: attn_bwd_qk_workspace_bytes(...)
 * plus one of two optional regions that attn_bwd_qk uses only when workspace_bytes is at least
 * this size (otherwise it runs without, same results up to summation order and rounding):
 *  - with a window and 1 <= sink <= 128 sink keys, the sink split of the bf16 dK/dV pass. Every
 *    query past the window still sees the sink keys, so the first 128-key tile has many times the
 *    work of any other; the split shares its query range among several workgroups whose fp32
 *    partial sums (2 * chunks * parts * B*Hkv*128*D) a small reduce adds in a fixed order.
 *  - with neither a window nor sink keys, D = 128 and Sk >= 2048, the stored dS (bf16 only; fp32
 *    calls leave it unused; where it was measured to pay):
 *    the dK/dV pass writes every 32 x 32 block of dS = P o (dP - delta) it forms, rounded to bf16
 *    as it enters dK, and the dQ pass computes dQ = scale * dS K from them instead of recomputing
 *    the score and dP tiles ("KYNETRA FOUNDRY" page, FlashAttention paragraph, has the backward
 *    recompute them: here that is the pass without this region). B*Hq * (sum over 32-row query
 *    blocks i of the key blocks up to the one holding position 32i + 31 + Sk - Sq, all of them
 *    without the causal mask) * 2048 bytes -- 1.08 GB for B=1, Hq=64, S=4096 -- and none above
 *    4 GiB. dQ then differs from the recomputing pass by the bf16 rounding of P before dS is
 *    formed (dK and dV are the same bits either way).
 * 0 for rejected sizes. */
size_t attn_bwd_qk_workspace_bytes_for(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                                       int window, int sink);

/* Backward with Sq queries against Sk >= Sq keys and `sink` sink keys. dout, dq are
 * [B,Hq,Sq,D]; dk, dv [B,Hkv,Sk,D] (keys no query sees get exact zeros). Same contract as
 * attn_bwd otherwise; o and lse come from attn_fwd_qk with the same arguments. */
int attn_bwd_qk(int dtype, const void* q, const void* k, const void* v, const void* o,
                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes,
                int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int window, int sink,
                float scale, void* stream);

/* For callers that cannot allocate device memory (code under stream capture, serving loops,
 * harnesses that forbid hipMalloc): attn_bwd_qk with the same arguments minus the workspace, which
 * comes from a static device array of ATTN_NOALLOC_SCRATCH_BYTES (one per device, held until the
 * process ends; enough for B=1, Hq=64, Hkv=8, S=4096, D=128 with its head split). Results are
 * bitwise those of attn_bwd_qk given a workspace of that size. Returns ATTN_ERR_SCRATCH, before
 * enqueueing anything, when attn_bwd_qk_workspace_bytes(...) exceeds the array; the sink split or
 * stored dS is used only when attn_bwd_qk_workspace_bytes_for(...) fits. Allocates nothing. Every call on one
 * device uses that device's array (the device of `stream`, or the current device for NULL), so
 * calls that overlap in time on one device race; nothing needs clearing between calls. */
#define ATTN_NOALLOC_SCRATCH_BYTES (72u << 20)
int attn_bwd_qk_noalloc(int dtype, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int window,
                        int sink, float scale, void* stream);

/* Forward against a paged K/V cache. k_pool and v_pool are [num_blocks, Hkv, block_size, D]
 * (dtype); block_table is int32 [B, max_blocks]: logical block t of sequence b (its tokens
 * t*block_size .. +block_size-1) is pool block block_table[b*max_blocks + t]; seqlen_k is int32
 * [B]: sequence b has seqlen_k[b] keys, and its Sq queries are its last Sq positions
 * (p = i + seqlen_k[b] - Sq; causal, window and sink as above). q, o are [B,Hq,Sq,D], lse
 * [B,Hq,Sq]. block_size is a power of two >= 16. The table and lengths are device arrays that
 * the host does not read: a length outside [Sq, max_blocks*block_size] is clamped into it and a
 * table entry outside [0, num_blocks) is clamped into it, so a malformed table cannot make the
 * kernel read outside the pools (the results are then unspecified). Blocks may be shared
 * between sequences (read-only here). */
int attn_fwd_paged(int dtype, const void* q, const void* k_pool, const void* v_pool,
                   const int* block_table, const int* seqlen_k, void* o, float* lse,
                   int B, int Hq, int Hkv, int Sq, int D, int block_size, int max_blocks,
                   int num_blocks, int causal, int window, int sink, float scale, void* stream);

/* Packed documents (causal). Each batch row of q, k, v ([B,Hq,S,D], [B,Hkv,S,D]) holds documents
 * back to back; cu_seqlens is int32 [B, n_docs + 1] with 0 = c_0 <= c_1 <= ... <= c_n_docs = S
 * (empty documents allowed; rows with fewer documents repeat S at the end). Key j is visible to
 * query i of the same row only if both lie in the same document [c_k, c_{k+1}), j <= i, and
 * (window == 0 || i - j < window). n_docs <= 2047. cu_seqlens is a device array the host does
 * not read: its values are clamped into [0, S] and a non-monotone array gives unspecified (but
 * in-bounds) results. Outputs and workspace as attn_fwd / attn_bwd (attn_bwd_workspace_bytes). */
int attn_fwd_varlen(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int n_docs, int B, int Hq, int Hkv, int S, int D,
                    int window, float scale, void* stream);
int attn_bwd_varlen(int dtype, const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, const int* cu_seqlens, int n_docs,
                    int B, int Hq, int Hkv, int S, int D, int window, float scale, void* stream);

/* Key-split forward for decode-shaped problems: the same result as attn_fwd_qk (dense k, v
 * [B,Hkv,Sk,D]; block_table = seqlen_k = NULL) or attn_fwd_paged (block_table, seqlen_k and the
 * pool arguments as there; Sk is then ignored), up to rounding, computed by many workgroups each
 * taking 128 keys of one (batch, KV head) for all of its (Hq/Hkv) * Sq query rows, then a merge
 * of their partial maxima, sums and outputs in a fixed order. Needs bf16 and
 * (Hq / Hkv) * Sq <= 32 (else ATTN_ERR_UNSUPPORTED). workspace: at least
 * attn_decode_workspace_bytes(B, Hq, Hkv, Sq, max_keys, D) bytes, max_keys = Sk (dense) or
 * max_blocks * block_size (paged); returns 0 for unsupported sizes. */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int max_keys, int D);
int attn_decode_fwd(int dtype, const void* q, const void* k, const void* v, const int* block_table,
                    const int* seqlen_k, void* o, float* lse, void* workspace,
                    size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                    int block_size, int max_blocks, int num_blocks, int causal, int window,
                    int sink, float scale, void* stream);

/* Optional launch observer, for profiling. When set, every entry point calls
 * hook(kernel, 0, stream, user) just before and hook(kernel, 1, stream, user) just after it
 * enqueues each of its kernels ("attn_fwd", "attn_bwd_prep" (the delta rows; only with a stored
 * dS), "attn_bwd_dq" (which otherwise forms the delta rows, and with a stored dS also adds the
 * head-part partials of a split head group), "attn_bwd_dkdv", "attn_bwd_dkdv_reduce" (only when
 * the head group is split and dS is not stored), "attn_bwd_dkdv_chunks" (only when the sink key
 * tile is split), "attn_decode", "attn_decode_combine"),
 * on the calling thread, so the hook can record timing events on `stream` around exactly one
 * kernel. NULL (the default) turns it off. The setting is process-wide; set it while no other
 * thread is calling the library. */
typedef void (*attn_launch_hook_t)(const char* kernel, int after, void* stream, void* user);
void attn_set_launch_hook(attn_launch_hook_t hook, void* user);

/* Static, NUL-terminated description of a status code. */
const char* attn_status_string(int status);

/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
