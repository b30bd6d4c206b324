"""The C-ABI library without a GPU: it loads, exports every function include/attn.h declares,
and rejects invalid arguments on the host before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
PKG = os.path.join(ROOT, "causal_attention_fa2_amd")

import causal_attention_fa2_amd as fa  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from causal_attention_fa2_amd.build import build
        build()
    return fa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == ["attn_abi_version", "attn_bwd", "attn_bwd_qk", "attn_bwd_qk_noalloc",
                     "attn_bwd_qk_workspace_bytes",
                     "attn_bwd_qk_workspace_bytes_for",
                     "attn_bwd_varlen", "attn_bwd_workspace_bytes", "attn_decode_fwd",
                     "attn_decode_workspace_bytes", "attn_fwd", "attn_fwd_paged", "attn_fwd_qk",
                     "attn_fwd_varlen", "attn_set_launch_hook", "attn_status_string"]
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_version_and_status_strings(lib):
    assert fa.attn_abi_version() == 8
    assert fa.attn_status_string(0) == "ok"
    assert fa.attn_status_string(1) == "invalid argument"
    assert fa.attn_status_string(2) == "unsupported configuration"
    assert fa.attn_status_string(3) == "HIP runtime error at launch"
    assert fa.attn_status_string(4) == "problem needs more than the static scratch buffer holds"
    assert fa.attn_status_string(99) == "unknown status"


def _parts(B, Hq, Hkv, S):
    """Head-group split of the dK/dV pass: key tiles of 128 paired, >= 256 workgroups wanted."""
    pairs = (-(-S // 128) + 1) // 2
    hs, G = 1, Hq // Hkv
    while B * Hkv * pairs * hs < 256 and G % (2 * hs) == 0:
        hs *= 2
    return hs


def test_workspace_bytes(lib):
    for shp in ((1, 64, 8, 4096, 128), (4, 16, 16, 1024, 64), (1, 16, 16, 8192, 64),
                (1, 64, 8, 32768, 128), (1, 4, 2, 300, 64), (1, 2, 2, 64, 64)):
        B, Hq, Hkv, S, D = shp
        hs = _parts(B, Hq, Hkv, S)
        rows = (B * Hq * S * 4 + 255) // 256 * 256  # delta, then lse * log2(e)
        part = 2 * hs * B * Hkv * S * D * 4 if hs > 1 else 0
        assert fa.attn_bwd_workspace_bytes(*shp) == 2 * rows + part, shp
    assert _parts(1, 64, 8, 4096) == 2 and _parts(1, 64, 8, 32768) == 1
    assert fa.attn_bwd_workspace_bytes(1, 64, 8, 4096, 128) == 2 * 64 * 4096 * 4 + 2 * 2 * 8 * 4096 * 128 * 4
    assert fa.attn_bwd_workspace_bytes(1, 2, 2, 3, 64) == 512  # two row arrays, 256-byte aligned
    assert fa.attn_bwd_workspace_bytes(1, 3, 2, 64, 64) == 0   # Hq % Hkv != 0
    assert fa.attn_bwd_workspace_bytes(1, 2, 2, 64, 96) == 0   # unsupported D


def test_qk_workspace_bytes(lib):
    """Row arrays follow the queries, partial sums (split head groups) follow the keys."""
    for B, Hq, Hkv, Sq, Sk, D in ((1, 64, 8, 1024, 4096, 128), (1, 64, 8, 1, 4096, 128),
                                  (2, 8, 2, 100, 300, 64), (1, 4, 4, 7, 7, 64), (1, 64, 8, 4096, 4096, 128)):
        hs = _parts(B, Hq, Hkv, Sk)
        rows = (B * Hq * Sq * 4 + 255) // 256 * 256
        part = 2 * hs * B * Hkv * Sk * D * 4 if hs > 1 else 0
        assert fa.attn_bwd_qk_workspace_bytes(B, Hq, Hkv, Sq, Sk, D) == 2 * rows + part
        if Sq == Sk:
            assert fa.attn_bwd_qk_workspace_bytes(B, Hq, Hkv, Sq, Sk, D) == \
                fa.attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, D)
    assert fa.attn_bwd_qk_workspace_bytes(1, 2, 2, 65, 64, 64) == 0  # more queries than keys
    assert fa.attn_bwd_qk_workspace_bytes(1, 2, 2, 0, 64, 64) == 0
    assert fa.attn_bwd_qk_workspace_bytes(1, 2, 2, 64, 0, 64) == 0


def _sink_chunks(B, Hq, Hkv, Sq, Sk, D, window, sink):
    """Chunks of key tile 0's query range in the sink split (query tiles of 64 rows; 1 = no
    split):
    only when tile 0's workgroup (its range plus an ordinary tile's, times the heads of a part)
    would exceed 1.1x a compute unit's share of the work (256 units); chunks of a quarter of an
    ordinary tile's range, at most 64 of them."""
    if window <= 0 or sink <= 0 or sink > 128:
        return 1
    off, c1, br = Sk - Sq, min(128, Sk) - 1, 64

    def rng(s):  # query tiles holding a row that sees some key in [0, c1] (causal)
        lo = max(0, off) - off
        hi = (Sk - 1 if s > 0 else min(Sk - 1, c1 + window - 1)) - off
        return (lo // br, hi // br) if hi >= lo else (1, 0)
    lo0, hi0 = rng(sink)
    lo1, hi1 = rng(0)
    nq0, nq1 = hi0 - lo0 + 1, max(hi1 - lo1 + 1, 1)
    if nq0 <= nq1:
        return 1
    hs = _parts(B, Hq, Hkv, Sk)
    hpg = Hq // Hkv // hs
    pairs = (-(-Sk // 128) + 1) // 2
    heavy = (nq0 + nq1) * hpg
    share = B * Hkv * hs * pairs * 2 * nq1 * hpg // 256
    if heavy * 10 <= share * 11:
        return 1
    c_len = (nq1 + 3) // 4
    if -(-nq0 // c_len) > 64:
        c_len = -(-nq0 // 64)
    return -(-nq0 // c_len)


def test_qk_workspace_bytes_for(lib):
    """Without a window or without sinks it is attn_bwd_qk_workspace_bytes; with both it adds the
    chunk slots: 2 (dK, dV) x chunks x head parts x B*Hkv x 128 keys x D fp32."""
    for B, Hq, Hkv, Sq, Sk, D, window, sink in ((1, 64, 8, 8192, 8192, 128, 1024, 4),
                                                (1, 8, 2, 1024, 1024, 128, 128, 4),
                                                (2, 4, 2, 300, 700, 64, 50, 1),
                                                (1, 64, 8, 4096, 4096, 128, 0, 4),
                                                (1, 64, 8, 4096, 4096, 128, 256, 0),
                                                (1, 4, 2, 640, 640, 128, 70, 130),
                                                (1, 64, 8, 8192, 8192, 64, 1024, 4),
                                                (1, 8, 2, 2048, 2048, 64, 128, 4)):
        base = fa.attn_bwd_qk_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)
        nc = _sink_chunks(B, Hq, Hkv, Sq, Sk, D, window, sink)
        extra = 2 * nc * _parts(B, Hq, Hkv, Sk) * B * Hkv * 128 * D * 4 if nc > 1 else 0
        got = fa.attn_bwd_qk_workspace_bytes_for(B, Hq, Hkv, Sq, Sk, D, True, window, sink)
        assert got == base + extra, (B, Hq, Hkv, Sq, Sk, D, window, sink, nc)
    # the sliding-window workload with 4 sinks: tile 0 is seen by all 128 query tiles, any other
    # tile by 18, so 26 chunks of 5; with 16 batch rows the ordinary work outweighs tile 0: no split
    assert _sink_chunks(1, 64, 8, 8192, 8192, 128, 1024, 4) == 26
    assert fa.attn_bwd_qk_workspace_bytes_for(1, 64, 8, 8192, 8192, 128, True, 1024, 4) == \
        fa.attn_bwd_qk_workspace_bytes(1, 64, 8, 8192, 8192, 128) + 2 * 26 * 8 * 128 * 128 * 4
    assert _sink_chunks(16, 64, 8, 8192, 8192, 128, 1024, 4) == 1
    assert fa.attn_bwd_qk_workspace_bytes_for(16, 64, 8, 8192, 8192, 128, True, 1024, 4) == \
        fa.attn_bwd_qk_workspace_bytes(16, 64, 8, 8192, 8192, 128)
    assert fa.attn_bwd_qk_workspace_bytes_for(1, 2, 2, 65, 64, 64, True, 8, 1) == 0  # rejected
    assert fa.attn_bwd_qk_workspace_bytes_for(1, 2, 2, 64, 64, 64, True, 8, -1) == 0


def _stored_ds_bytes(B, Hq, Sq, Sk, D, causal, window, sink):
    """Room for the stored dS: per (batch, query head) and 64-row query tile, two 2 KB blocks (its two
    32-row halves) per 32-key block from key 0 up to the one holding the position the tile's last
    nominal row stands at (row 64t + 63 at position 64t + 63 + Sk - Sq), all key blocks without the
    causal mask; none with a window or sink keys, for D = 64, below 2048 keys, or beyond 4 GiB."""
    if window or sink or D != 128 or Sk < 2048:
        return 0
    nkb = -(-Sk // 32)
    entries = 0
    for t in range(-(-Sq // 64)):
        last = (64 * t + 63 + Sk - Sq) // 32 if causal else nkb - 1
        entries += min(nkb, last + 1)
    n = B * Hq * entries * 4096
    return n if n <= 4 << 30 else 0


def test_qk_workspace_bytes_for_stored_ds(lib):
    """Without a window and sink keys attn_bwd_qk_workspace_bytes_for adds the stored dS after the
    plain workspace (attn_bwd_qk_workspace_bytes stays the plain size)."""
    for B, Hq, Hkv, Sq, Sk, D, causal in ((1, 64, 8, 4096, 4096, 128, True), (1, 64, 8, 4096, 4096, 128, False),
                                          (2, 4, 2, 300, 2100, 128, True), (1, 8, 2, 2049, 2049, 128, True),
                                          (1, 4, 4, 7, 2048, 128, True), (1, 4, 2, 33, 2047, 128, True),
                                          (3, 6, 2, 2130, 2130, 128, False), (1, 64, 8, 8192, 8192, 128, True),
                                          (1, 64, 8, 32768, 32768, 128, True), (1, 64, 8, 1, 4096, 128, True),
                                          (1, 16, 16, 8192, 8192, 64, True), (4, 16, 16, 1024, 1024, 64, True),
                                          (1, 64, 8, 1024, 1024, 128, True)):
        base = fa.attn_bwd_qk_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)
        got = fa.attn_bwd_qk_workspace_bytes_for(B, Hq, Hkv, Sq, Sk, D, causal, 0, 0)
        assert got == base + _stored_ds_bytes(B, Hq, Sq, Sk, D, causal, 0, 0), (B, Hq, Sq, Sk, D, causal)
    # the 64-head S = 4096 causal problem: tiles t = 0 .. 63 hold 2t + 2 key blocks
    assert _stored_ds_bytes(1, 64, 4096, 4096, 128, True, 0, 0) == 64 * 4160 * 4096
    # S = 8192 would need 4.3 GB (> 4 GiB): no stored dS
    assert _stored_ds_bytes(1, 64, 8192, 8192, 128, True, 0, 0) == 0
    assert fa.attn_bwd_qk_workspace_bytes_for(1, 64, 8, 8192, 8192, 128, True, 0, 0) == \
        fa.attn_bwd_qk_workspace_bytes(1, 64, 8, 8192, 8192, 128)
    # one decode-like query row against 4096 keys: one tile of all 128 key blocks per head
    assert _stored_ds_bytes(1, 64, 1, 4096, 128, True, 0, 0) == 64 * 128 * 4096
    # where it does not pay: D = 64, or fewer than 2048 keys
    assert _stored_ds_bytes(1, 16, 8192, 8192, 64, True, 0, 0) == 0
    assert _stored_ds_bytes(1, 64, 1024, 1024, 128, True, 0, 0) == 0
    assert _stored_ds_bytes(1, 4, 33, 2047, 128, True, 0, 0) == 0 < _stored_ds_bytes(1, 4, 7, 2048, 128, True, 0, 0)


P = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def fwd(lib, dtype=1, ptrs=(P, P, P, P, P), B=1, Hq=2, Hkv=2, S=64, D=64, causal=1, window=0,
        scale=0.125):
    return lib.attn_fwd(dtype, *ptrs, B, Hq, Hkv, S, D, causal, window, scale, None)


def bwd(lib, ws_bytes=0, ptrs=(P,) * 10, B=1, Hq=2, Hkv=2, S=64, D=64, causal=1, window=0,
        scale=0.125, dtype=1):
    return lib.attn_bwd(dtype, *ptrs, ws_bytes, B, Hq, Hkv, S, D, causal, window, scale, None)


def test_fwd_validation(lib):
    INV, UNS = fa.ATTN_ERR_INVALID, fa.ATTN_ERR_UNSUPPORTED
    for i in range(5):
        ptrs = [P] * 5
        ptrs[i] = None
        assert fwd(lib, ptrs=ptrs) == INV
    assert fwd(lib, B=0) == INV
    assert fwd(lib, S=-1) == INV
    assert fwd(lib, Hq=3, Hkv=2) == INV
    assert fwd(lib, window=-1) == INV
    assert fwd(lib, scale=float("nan")) == INV
    assert fwd(lib, scale=float("inf")) == INV
    assert fwd(lib, causal=2) == INV
    assert fwd(lib, D=96) == UNS
    assert fwd(lib, dtype=7) == UNS
    assert fwd(lib, causal=0, window=4) == UNS
    assert fwd(lib, B=1, Hq=64, Hkv=8, S=262144, D=128) == UNS  # 2^31 elements
    # the kernels scale each row's maximum of the raw scores: a scale <= 0 is refused
    assert fwd(lib, scale=0.0) == UNS
    assert fwd(lib, scale=-0.125) == UNS
    assert fwd(lib, scale=float("-inf")) == INV


def test_bwd_validation(lib):
    INV, UNS = fa.ATTN_ERR_INVALID, fa.ATTN_ERR_UNSUPPORTED
    need = fa.attn_bwd_workspace_bytes(1, 2, 2, 64, 64)
    for i in range(10):
        ptrs = [P] * 10
        ptrs[i] = None
        assert bwd(lib, need, ptrs=ptrs) == INV
    assert bwd(lib, need - 1) == INV
    assert bwd(lib, need, Hq=4, Hkv=3) == INV
    assert bwd(lib, need, D=32) == UNS
    assert bwd(lib, need, causal=0, window=1) == UNS
    assert bwd(lib, need, scale=0.0) == UNS
    assert bwd(lib, need, scale=-0.125) == UNS


def fwd_qk(lib, dtype=1, ptrs=(P, P, P, P, P), B=1, Hq=2, Hkv=2, Sq=16, Sk=64, D=64, causal=1,
           window=0, scale=0.125, sink=0):
    return lib.attn_fwd_qk(dtype, *ptrs, B, Hq, Hkv, Sq, Sk, D, causal, window, sink, scale, None)


def bwd_qk(lib, ws_bytes=0, ptrs=(P,) * 10, B=1, Hq=2, Hkv=2, Sq=16, Sk=64, D=64, causal=1,
           window=0, scale=0.125, dtype=1, sink=0):
    return lib.attn_bwd_qk(dtype, *ptrs, ws_bytes, B, Hq, Hkv, Sq, Sk, D, causal, window, sink,
                           scale, None)


def test_qk_validation(lib):
    INV, UNS = fa.ATTN_ERR_INVALID, fa.ATTN_ERR_UNSUPPORTED
    for i in range(5):
        ptrs = [P] * 5
        ptrs[i] = None
        assert fwd_qk(lib, ptrs=ptrs) == INV
    assert fwd_qk(lib, Sq=0) == INV
    assert fwd_qk(lib, Sk=0) == INV
    assert fwd_qk(lib, Sq=65, Sk=64) == UNS        # more queries than keys is not defined
    assert fwd_qk(lib, window=8, sink=-1) == INV
    assert fwd_qk(lib, window=0, sink=-3) == INV
    assert fwd_qk(lib, Hq=3, Hkv=2) == INV
    assert fwd_qk(lib, causal=0, window=4) == UNS
    assert fwd_qk(lib, D=96) == UNS
    # each tensor below 2^31 elements: K/V [1, 8, 2^21, 128] is exactly 2^31
    assert fwd_qk(lib, B=1, Hq=64, Hkv=8, Sq=1, Sk=1 << 21, D=128) == UNS
    assert fwd_qk(lib, B=1, Hq=64, Hkv=8, Sq=1 << 18, Sk=1 << 18, D=128) == UNS
    need = fa.attn_bwd_qk_workspace_bytes(1, 2, 2, 16, 64, 64)
    assert need > 0
    for i in range(10):
        ptrs = [P] * 10
        ptrs[i] = None
        assert bwd_qk(lib, need, ptrs=ptrs) == INV
    assert bwd_qk(lib, need - 1) == INV
    assert bwd_qk(lib, need, Sq=65) == UNS
    assert bwd_qk(lib, need, window=4, sink=-1) == INV
    assert bwd_qk(lib, need, D=32) == UNS


def bwd_noalloc(lib, ptrs=(P,) * 9, B=1, Hq=2, Hkv=2, Sq=16, Sk=64, D=64, causal=1, window=0,
                scale=0.125, dtype=1, sink=0):
    return lib.attn_bwd_qk_noalloc(dtype, *ptrs, B, Hq, Hkv, Sq, Sk, D, causal, window, sink, scale,
                                   None)


def test_noalloc_validation(lib):
    """Argument checks as attn_bwd_qk; a problem whose workspace exceeds the static array is refused
    with ATTN_ERR_SCRATCH before any HIP call (so this runs without a GPU)."""
    INV, UNS, SCR = fa.ATTN_ERR_INVALID, fa.ATTN_ERR_UNSUPPORTED, fa.ATTN_ERR_SCRATCH
    header = open(HEADER).read()
    assert re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \(72u << 20\)", header)
    assert fa.ATTN_NOALLOC_SCRATCH_BYTES == 72 << 20
    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = None
        assert bwd_noalloc(lib, ptrs=ptrs) == INV
    assert bwd_noalloc(lib, Sq=65) == UNS
    assert bwd_noalloc(lib, D=32) == UNS
    assert bwd_noalloc(lib, scale=0.0) == UNS
    assert bwd_noalloc(lib, window=4, sink=-1) == INV
    assert bwd_noalloc(lib, Hq=3) == INV
    # the S=4096, 64/8-head, D=128 backward fits with its head split (2 MiB rows + 64 MiB partials)
    assert fa.attn_bwd_qk_workspace_bytes(1, 64, 8, 4096, 4096, 128) == 66 << 20
    # S=6144 splits the head group too: 2 x 2 x 8 x 6144 x 128 fp32 = 96 MiB of partials
    big = (1, 64, 8, 6144, 6144, 128)
    assert fa.attn_bwd_qk_workspace_bytes(*big) > fa.ATTN_NOALLOC_SCRATCH_BYTES
    assert bwd_noalloc(lib, B=1, Hq=64, Hkv=8, Sq=6144, Sk=6144, D=128) == SCR
    # row arrays alone beyond the array: 2 x 128 heads x 2^17 rows fp32 = 128 MiB
    assert bwd_noalloc(lib, B=1, Hq=128, Hkv=128, Sq=1 << 17, Sk=1 << 17, D=64) == SCR
    # argument errors take precedence over the size check
    assert bwd_noalloc(lib, B=1, Hq=64, Hkv=8, Sq=6144, Sk=6144, D=96) == UNS


def fwd_paged(lib, dtype=1, ptrs=(P,) * 7, B=2, Hq=4, Hkv=2, Sq=1, D=128, bs=16, max_blocks=8,
              num_blocks=20, causal=1, window=0, sink=0, scale=0.125):
    return lib.attn_fwd_paged(dtype, *ptrs, B, Hq, Hkv, Sq, D, bs, max_blocks, num_blocks, causal,
                              window, sink, scale, None)


def test_paged_validation(lib):
    INV, UNS = fa.ATTN_ERR_INVALID, fa.ATTN_ERR_UNSUPPORTED
    for i in range(7):
        ptrs = [P] * 7
        ptrs[i] = None
        assert fwd_paged(lib, ptrs=ptrs) == INV
    assert fwd_paged(lib, bs=0) == INV
    assert fwd_paged(lib, max_blocks=0) == INV
    assert fwd_paged(lib, num_blocks=0) == INV
    assert fwd_paged(lib, bs=24) == UNS            # not a power of two
    assert fwd_paged(lib, bs=8) == UNS             # below 16
    assert fwd_paged(lib, bs=1 << 21) == UNS
    assert fwd_paged(lib, bs=1 << 20, max_blocks=1 << 11) == UNS  # 2^31 keys per sequence
    assert fwd_paged(lib, Sq=129, bs=16, max_blocks=8) == UNS     # more queries than any sequence holds
    assert fwd_paged(lib, Hq=3) == INV
    assert fwd_paged(lib, sink=-1, window=4) == INV
    assert fwd_paged(lib, causal=0, window=4) == UNS
    assert fwd_paged(lib, D=96) == UNS


def test_varlen_validation(lib):
    INV, UNS = fa.ATTN_ERR_INVALID, fa.ATTN_ERR_UNSUPPORTED

    def fv(ptrs=(P,) * 6, n=3, B=1, Hq=2, Hkv=2, S=64, D=64, window=0, scale=0.125, dtype=1):
        return lib.attn_fwd_varlen(dtype, *ptrs[:5], ptrs[5], n, B, Hq, Hkv, S, D, window, scale, None)

    for i in range(6):
        ptrs = [P] * 6
        ptrs[i] = None
        assert fv(ptrs=ptrs) == INV
    assert fv(n=0) == INV
    assert fv(n=2048) == UNS
    assert fv(window=-1) == INV
    assert fv(D=80) == UNS
    need = fa.attn_bwd_workspace_bytes(1, 2, 2, 64, 64)

    def bv(ws=need, ptrs=(P,) * 11, n=3, S=64):
        return lib.attn_bwd_varlen(1, *ptrs[:10], ws, ptrs[10], n, 1, 2, 2, S, 64, 0, 0.125, None)

    for i in range(11):
        ptrs = [P] * 11
        ptrs[i] = None
        assert bv(ptrs=ptrs) == INV
    assert bv(ws=need - 1) == INV
    assert bv(n=-1) == INV


def test_decode_workspace_and_validation(lib):
    INV, UNS = fa.ATTN_ERR_INVALID, fa.ATTN_ERR_UNSUPPORTED
    # chunks of 128 keys x B x Hkv x R packed rows x (D + 2) floats
    assert fa.attn_decode_workspace_bytes(1, 64, 8, 1, 4096, 128) == 32 * 8 * 8 * 130 * 4
    assert fa.attn_decode_workspace_bytes(2, 8, 2, 3, 300, 64) == 3 * 2 * 2 * 12 * 66 * 4
    assert fa.attn_decode_workspace_bytes(1, 64, 8, 5, 4096, 128) == 0   # 40 packed rows
    need = fa.attn_decode_workspace_bytes(1, 64, 8, 1, 4096, 128)

    def dec(ws=need, dtype=1, table=None, lens=None, Hq=64, Sq=1, Sk=4096, bs=0, maxb=0, nb=0, ptrs=(P,) * 6):
        q, k, v, o, lse, w = ptrs
        return lib.attn_decode_fwd(dtype, q, k, v, table, lens, o, lse, w, ws, 1, Hq, 8, Sq, Sk, 128, bs,
                                   maxb, nb, 1, 0, 0, 0.125, None)

    for i in range(6):
        ptrs = [P] * 6
        ptrs[i] = None
        assert dec(ptrs=ptrs) == INV
    assert dec(ws=need - 1) == INV
    assert dec(dtype=0) == UNS                 # bf16 only
    assert dec(Sq=5) == UNS                    # 8 heads x 5 queries > 32 packed rows
    assert dec(table=P) == INV                 # paged needs both the table and the lengths
    assert dec(table=P, lens=P, bs=24, maxb=8, nb=4) == UNS
    assert dec(table=P, lens=P, bs=16, maxb=0, nb=4) == INV


def test_launch_hook_set_and_clear(lib):
    seen = []
    fa.attn_set_launch_hook(lambda k, a, s: seen.append((k, a)))
    assert fwd(lib, D=96) == fa.ATTN_ERR_UNSUPPORTED  # rejected calls enqueue nothing
    assert seen == []
    fa.attn_set_launch_hook(None)


def test_missing_library_raises(tmp_path):
    with pytest.raises(RuntimeError):
        fa.load_library(str(tmp_path / "nope.so"))


def test_product_never_touches_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, flags=re.M), f
                assert "oracle." not in text, f
