"""ctypes binding of libattn.so: the C-ABI calls under the same names, taking torch tensors.

Argument marshalling only: every step of the attention path runs in the HIP kernels behind
the C ABI. torch supplies device memory (tensor.data_ptr()) and the stream
(torch.cuda.current_stream().cuda_stream, a hipStream_t on ROCm). There is no fallback: if the
library is missing or not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_DEVICE, ATTN_ERR_SCRATCH = 0, 1, 2, 3, 4
ATTN_NOALLOC_SCRATCH_BYTES = 72 << 20  # size of attn_bwd_qk_noalloc's static scratch array
ATTN_F32, ATTN_BF16 = 0, 1

_lib = None
_hook_ref = None

# void (*)(const char* kernel, int after, void* stream, void* user)
LAUNCH_HOOK = ctypes.CFUNCTYPE(None, ctypes.c_char_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p)


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m causal_attention_fa2_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.attn_fwd.restype = i
    lib.attn_bwd.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                             i, i, i, i, i, i, i, f, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_qk.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_qk.restype = i
    lib.attn_bwd_qk.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                i, i, i, i, i, i, i, i, i, f, vp]
    lib.attn_bwd_qk.restype = i
    lib.attn_bwd_qk_noalloc.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        i, i, i, i, i, i, i, i, i, f, vp]
    lib.attn_bwd_qk_noalloc.restype = i
    lib.attn_bwd_qk_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.attn_bwd_qk_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_qk_workspace_bytes_for.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.attn_bwd_qk_workspace_bytes_for.restype = ctypes.c_size_t
    lib.attn_fwd_paged.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, i,
                                   f, vp]
    lib.attn_fwd_paged.restype = i
    lib.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode_fwd.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i, i, i, i, i, i,
                                    i, i, i, i, i, i, f, vp]
    lib.attn_decode_fwd.restype = i
    lib.attn_fwd_varlen.argtypes = [i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_varlen.restype = i
    lib.attn_bwd_varlen.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, i,
                                    i, i, i, i, i, i, f, vp]
    lib.attn_bwd_varlen.restype = i
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = i
    lib.attn_set_launch_hook.argtypes = [LAUNCH_HOOK, vp]
    lib.attn_set_launch_hook.restype = None
    if path is None:
        _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


status_string = attn_status_string


def attn_abi_version() -> int:
    return int(load_library().attn_abi_version())


def attn_set_launch_hook(fn) -> None:
    """fn(kernel: str, after: int, stream: int) is called just before (after=0) and just after
    (after=1) each kernel the library enqueues; None removes it."""
    global _hook_ref
    lib = load_library()
    if fn is None:
        lib.attn_set_launch_hook(LAUNCH_HOOK(), None)
        _hook_ref = None
        return

    def tramp(kernel, after, stream, user):
        fn(kernel.decode(), int(after), int(stream or 0))

    _hook_ref = LAUNCH_HOOK(tramp)  # keep the trampoline alive while the library holds it
    lib.attn_set_launch_hook(_hook_ref, None)


def attn_bwd_workspace_bytes(B: int, Hq: int, Hkv: int, S: int, D: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, Hq, Hkv, S, D))


def attn_bwd_qk_workspace_bytes(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, D: int) -> int:
    return int(load_library().attn_bwd_qk_workspace_bytes(B, Hq, Hkv, Sq, Sk, D))


def attn_bwd_qk_workspace_bytes_for(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, D: int,
                                    causal: bool = True, window: int = 0, sink: int = 0) -> int:
    """Workspace bytes of attn_bwd_qk for these mask arguments (room for the sink split)."""
    return int(load_library().attn_bwd_qk_workspace_bytes_for(B, Hq, Hkv, Sq, Sk, D, int(bool(causal)),
                                                               int(window), int(sink)))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_tensor(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}")


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _fwd_args(q, k, v, o, lse, causal, window, scale):
    import torch
    if not q.is_contiguous() or q.device.type != "cuda":
        raise ValueError("q must be a contiguous GPU tensor")
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    _check_tensor("k", k, (B, Hkv, Sk, D), q.dtype, q.device)
    _check_tensor("v", v, (B, Hkv, Sk, D), q.dtype, q.device)
    _check_tensor("o", o, (B, Hq, Sq, D), q.dtype, q.device)
    _check_tensor("lse", lse, (B, Hq, Sq), torch.float32, q.device)
    scale = D ** -0.5 if scale is None else float(scale)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    return ptrs, (B, Hq, Hkv, Sq, Sk, D), (int(bool(causal)), int(window), scale)


def attn_fwd(q, k, v, o, lse, causal: bool = True, window: int = 0, scale: float | None = None,
             stream=None) -> None:
    """Calls attn_fwd: q [B,Hq,S,D], k/v [B,Hkv,S,D] -> o [B,Hq,S,D] (q's dtype), lse [B,Hq,S] f32."""
    ptrs, (B, Hq, Hkv, Sq, Sk, D), tail = _fwd_args(q, k, v, o, lse, causal, window, scale)
    if Sq != Sk:
        raise ValueError("attn_fwd takes as many queries as keys; use attn_fwd_qk")
    st = load_library().attn_fwd(_dtype_code(q), *ptrs, B, Hq, Hkv, Sq, D, *tail, _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd")


def attn_fwd_qk(q, k, v, o, lse, causal: bool = True, window: int = 0, scale: float | None = None,
                stream=None, sink: int = 0) -> None:
    """Calls attn_fwd_qk: q [B,Hq,Sq,D], k/v [B,Hkv,Sk,D] with Sq <= Sk (the queries are the last
    Sq positions), `sink` leading keys kept visible beside the window -> o [B,Hq,Sq,D],
    lse [B,Hq,Sq] f32."""
    ptrs, (B, Hq, Hkv, Sq, Sk, D), (c, w, sc) = _fwd_args(q, k, v, o, lse, causal, window, scale)
    st = load_library().attn_fwd_qk(_dtype_code(q), *ptrs, B, Hq, Hkv, Sq, Sk, D, c, w, int(sink), sc,
                                    _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_qk")


def attn_fwd_paged(q, k_pool, v_pool, block_table, seqlen_k, o, lse, causal: bool = True,
                   window: int = 0, scale: float | None = None, stream=None, sink: int = 0) -> None:
    """Calls attn_fwd_paged: q [B,Hq,Sq,D]; k_pool/v_pool [num_blocks,Hkv,block_size,D] (q's
    dtype); block_table int32 [B, max_blocks]; seqlen_k int32 [B] -> o [B,Hq,Sq,D], lse [B,Hq,Sq]."""
    import torch
    if not q.is_contiguous() or q.device.type != "cuda":
        raise ValueError("q must be a contiguous GPU tensor")
    B, Hq, Sq, D = q.shape
    nb, Hkv, bs = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    _check_tensor("k_pool", k_pool, (nb, Hkv, bs, D), q.dtype, q.device)
    _check_tensor("v_pool", v_pool, (nb, Hkv, bs, D), q.dtype, q.device)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _check_tensor("block_table", block_table, tuple(block_table.shape), torch.int32, q.device)
    _check_tensor("seqlen_k", seqlen_k, (B,), torch.int32, q.device)
    _check_tensor("o", o, (B, Hq, Sq, D), q.dtype, q.device)
    _check_tensor("lse", lse, (B, Hq, Sq), torch.float32, q.device)
    scale = D ** -0.5 if scale is None else float(scale)
    st = load_library().attn_fwd_paged(
        _dtype_code(q), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
        seqlen_k.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Sq, D, bs,
        block_table.shape[1], nb, int(bool(causal)), int(window), int(sink), scale, _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_paged")


def attn_decode_workspace_bytes(B: int, Hq: int, Hkv: int, Sq: int, max_keys: int, D: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, Hq, Hkv, Sq, max_keys, D))


def attn_decode_fwd(q, k, v, o, lse, workspace, causal: bool = True, window: int = 0,
                    scale: float | None = None, stream=None, sink: int = 0, block_table=None,
                    seqlen_k=None) -> None:
    """Calls attn_decode_fwd (key-split forward, bf16, (Hq/Hkv)*Sq <= 32). Dense: k/v
    [B,Hkv,Sk,D]. Paged: k/v pools [num_blocks,Hkv,block_size,D] with block_table int32
    [B,max_blocks] and seqlen_k int32 [B]. workspace: uint8 tensor of at least
    attn_decode_workspace_bytes(B, Hq, Hkv, Sq, max_keys, D) bytes (max_keys = Sk, or
    max_blocks * block_size when paged)."""
    import torch
    if not q.is_contiguous() or q.device.type != "cuda":
        raise ValueError("q must be a contiguous GPU tensor")
    B, Hq, Sq, D = q.shape
    paged = block_table is not None
    if paged:
        nb, Hkv, bs = k.shape[0], k.shape[1], k.shape[2]
        _check_tensor("k", k, (nb, Hkv, bs, D), q.dtype, q.device)
        _check_tensor("v", v, (nb, Hkv, bs, D), q.dtype, q.device)
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be [B, max_blocks]")
        _check_tensor("block_table", block_table, tuple(block_table.shape), torch.int32, q.device)
        _check_tensor("seqlen_k", seqlen_k, (B,), torch.int32, q.device)
        Sk, maxb, tptr, lptr = 0, block_table.shape[1], block_table.data_ptr(), seqlen_k.data_ptr()
    else:
        Hkv, Sk = k.shape[1], k.shape[2]
        _check_tensor("k", k, (B, Hkv, Sk, D), q.dtype, q.device)
        _check_tensor("v", v, (B, Hkv, Sk, D), q.dtype, q.device)
        nb = bs = maxb = 0
        tptr = lptr = None
    _check_tensor("o", o, (B, Hq, Sq, D), q.dtype, q.device)
    _check_tensor("lse", lse, (B, Hq, Sq), torch.float32, q.device)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    scale = D ** -0.5 if scale is None else float(scale)
    st = load_library().attn_decode_fwd(
        _dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), tptr, lptr, o.data_ptr(),
        lse.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(), B, Hq,
        Hkv, Sq, Sk, D, bs, maxb, nb, int(bool(causal)), int(window), int(sink), scale,
        _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_fwd")


def _docs_arg(cu_seqlens, B, device):
    import torch
    if cu_seqlens.dim() != 2 or cu_seqlens.shape[0] != B or cu_seqlens.shape[1] < 2:
        raise ValueError("cu_seqlens must be [B, n_docs + 1]")
    _check_tensor("cu_seqlens", cu_seqlens, tuple(cu_seqlens.shape), torch.int32, device)
    return cu_seqlens.data_ptr(), cu_seqlens.shape[1] - 1


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, window: int = 0, scale: float | None = None,
                    stream=None) -> None:
    """Calls attn_fwd_varlen (causal, packed documents): cu_seqlens int32 [B, n_docs + 1]."""
    ptrs, (B, Hq, Hkv, Sq, Sk, D), (_, w, sc) = _fwd_args(q, k, v, o, lse, True, window, scale)
    if Sq != Sk:
        raise ValueError("packed documents take as many queries as keys")
    cu, n = _docs_arg(cu_seqlens, B, q.device)
    st = load_library().attn_fwd_varlen(_dtype_code(q), *ptrs, cu, n, B, Hq, Hkv, Sq, D, w, sc,
                                        _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_varlen")


def attn_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens, window: int = 0,
                    scale: float | None = None, stream=None) -> None:
    """Calls attn_bwd_varlen; workspace as for attn_bwd (attn_bwd_workspace_bytes)."""
    ptrs, (B, Hq, Hkv, Sq, Sk, D), (_, w, sc) = _bwd_args(q, k, v, o, lse, dout, dq, dk, dv,
                                                          workspace, True, window, scale)
    if Sq != Sk:
        raise ValueError("packed documents take as many queries as keys")
    cu, n = _docs_arg(cu_seqlens, B, q.device)
    st = load_library().attn_bwd_varlen(_dtype_code(q), *ptrs, cu, n, B, Hq, Hkv, Sq, D, w, sc,
                                        _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_varlen")


def _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, window, scale):
    """Checks the tensors and returns (pointers, sizes, mask arguments); workspace=None leaves the
    workspace pointer and size out of the pointers."""
    import torch
    if not q.is_contiguous() or q.device.type != "cuda":
        raise ValueError("q must be a contiguous GPU tensor")
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    for name, t, shp in (("k", k, (B, Hkv, Sk, D)), ("v", v, (B, Hkv, Sk, D)),
                         ("o", o, (B, Hq, Sq, D)), ("dout", dout, (B, Hq, Sq, D)),
                         ("dq", dq, (B, Hq, Sq, D)), ("dk", dk, (B, Hkv, Sk, D)),
                         ("dv", dv, (B, Hkv, Sk, D))):
        _check_tensor(name, t, shp, q.dtype, q.device)
    _check_tensor("lse", lse, (B, Hq, Sq), torch.float32, q.device)
    scale = D ** -0.5 if scale is None else float(scale)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    if workspace is not None:
        if workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ptrs += (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    return ptrs, (B, Hq, Hkv, Sq, Sk, D), (int(bool(causal)), int(window), scale)


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal: bool = True, window: int = 0,
             scale: float | None = None, stream=None) -> None:
    """Calls attn_bwd; dq/dk/dv are overwritten. workspace: a uint8 GPU tensor of at least
    attn_bwd_workspace_bytes(...) bytes."""
    ptrs, (B, Hq, Hkv, Sq, Sk, D), tail = _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, workspace,
                                                    causal, window, scale)
    if Sq != Sk:
        raise ValueError("attn_bwd takes as many queries as keys; use attn_bwd_qk")
    st = load_library().attn_bwd(_dtype_code(q), *ptrs, B, Hq, Hkv, Sq, D, *tail, _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")


def attn_bwd_qk(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal: bool = True,
                window: int = 0, scale: float | None = None, stream=None, sink: int = 0) -> None:
    """Calls attn_bwd_qk (Sq <= Sk, `sink` sink keys); dq/dk/dv are overwritten. workspace: a uint8
    GPU tensor of at least attn_bwd_qk_workspace_bytes(...) bytes."""
    ptrs, (B, Hq, Hkv, Sq, Sk, D), (c, w, sc) = _bwd_args(q, k, v, o, lse, dout, dq, dk, dv,
                                                          workspace, causal, window, scale)
    st = load_library().attn_bwd_qk(_dtype_code(q), *ptrs, B, Hq, Hkv, Sq, Sk, D, c, w, int(sink), sc,
                                    _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_qk")


def attn_bwd_qk_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal: bool = True, window: int = 0,
                        scale: float | None = None, stream=None, sink: int = 0) -> None:
    """Calls attn_bwd_qk_noalloc: attn_bwd_qk without a workspace argument (the library's static
    per-device scratch array serves instead; nothing is allocated). Raises AttnError with status
    ATTN_ERR_SCRATCH when the problem needs more than ATTN_NOALLOC_SCRATCH_BYTES."""
    ptrs, (B, Hq, Hkv, Sq, Sk, D), (c, w, sc) = _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, None,
                                                          causal, window, scale)
    st = load_library().attn_bwd_qk_noalloc(_dtype_code(q), *ptrs, B, Hq, Hkv, Sq, Sk, D, c, w,
                                            int(sink), sc, _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_qk_noalloc")


# ---------------------------------------------------------------- allocation conveniences
def forward(q, k, v, causal: bool = True, window: int = 0, scale: float | None = None, stream=None,
            sink: int = 0):
    """Allocates o and lse with torch, then calls attn_fwd (attn_fwd_qk when k has more rows than
    q or there are sink keys). Returns (o, lse)."""
    import torch
    B, Hq, Sq, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if k.shape[2] == Sq and not sink:
        attn_fwd(q, k, v, o, lse, causal, window, scale, stream)
    else:
        attn_fwd_qk(q, k, v, o, lse, causal, window, scale, stream, sink)
    return o, lse


def backward(q, k, v, o, lse, dout, causal: bool = True, window: int = 0,
             scale: float | None = None, stream=None, workspace=None, sink: int = 0):
    """Allocates dq, dk, dv (and the workspace if none is given), then calls attn_bwd
    (attn_bwd_qk when k has more rows than q or there are sink keys)."""
    import torch
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if workspace is None:
        workspace = torch.empty(max(1, attn_bwd_qk_workspace_bytes_for(B, Hq, Hkv, Sq, Sk, D, causal, window,
                                                                        sink)),
                                dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if Sk == Sq and not sink:
        attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, window, scale, stream)
    else:
        attn_bwd_qk(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, window, scale, stream, sink)
    return dq, dk, dv
