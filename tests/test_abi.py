"""The C ABI without a GPU: the library loads, exports every function that
include/fa.h declares, and rejects bad arguments before enqueuing anything.

Only argument-error paths are called here: they return before any HIP call,
so they run on a machine without a GPU."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def L():
    import exact_attention_34_amd as fa
    if not os.path.exists(fa.library_path()):
        from exact_attention_34_amd import build
        build.build()
    return fa.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def _status(name):
    text = open(HEADER).read()
    return int(re.search(r"#define\s+%s\s+\(?(-?\d+)\)?" % name, text).group(1))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert "fa_fwd" in names and "fa_bwd" in names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.fa_abi_version() == _status("FA_ABI_VERSION")
    for code in (0, -1, -2, -3, -4, -5):
        s = L.fa_status_str(code).decode()
        assert s and s != "unknown status"
    assert L.fa_status_str(7).decode() == "unknown status"


# Fake, 16-byte-aligned "device" addresses: never dereferenced, because every
# call below fails its argument checks first.
A = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)
NUL = ctypes.c_void_p(0)

INVALID = _status("FA_ERR_INVALID_ARG")
UNSUP = _status("FA_ERR_UNSUPPORTED")
WS = _status("FA_ERR_WORKSPACE")


def fwd(L, dtype=2, B=1, H=1, N=16, d=64, q=A, k=A, v=A, scale=0.125, causal=0, o=A2,
        lse=A2):
    return L.fa_fwd(dtype, B, H, N, d, q, k, v, scale, causal, o, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(N=0), INVALID),
    (dict(d=0), INVALID), (dict(d=96), UNSUP), (dict(d=256), UNSUP),
    (dict(dtype=3), UNSUP), (dict(dtype=-1), UNSUP),
    (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID),
    (dict(scale=math.nan), INVALID), (dict(scale=math.inf), INVALID),
    (dict(causal=2), INVALID), (dict(causal=-1), INVALID),
    (dict(q=NUL), INVALID), (dict(k=NUL), INVALID), (dict(v=NUL), INVALID),
    (dict(o=NUL), INVALID), (dict(lse=NUL), INVALID),
    (dict(q=MIS), INVALID), (dict(o=MIS), INVALID),
    (dict(B=1 << 12, H=1 << 12, N=1 << 10, d=128), INVALID),  # 2^34 rows
    (dict(B=1 << 16, H=1 << 15, N=1, d=64), INVALID),  # B*H*N = 2^31 rows
    (dict(B=1, H=1, N=1 << 24, d=128), INVALID),  # one slice of 2^31 elements
])
def test_fwd_rejects(L, kw, code):
    assert fwd(L, **kw) == code


def _bwd(L, dtype=2, N=16, d=64, ws=A, ws_bytes=None, causal=0, scale=0.125, dq=A2, lse=A2):
    if ws_bytes is None:
        ws_bytes = L.fa_bwd_workspace_bytes(dtype, 1, 1, N, d)
    return L.fa_bwd(dtype, 1, 1, N, d, A, A, A, A, A, lse, scale, causal, dq, A2, A2, ws,
                    ws_bytes, None)


def test_bwd_rejects(L):
    assert _bwd(L, dtype=0) == UNSUP          # fp32 backward is not built
    assert _bwd(L, d=32) == UNSUP
    assert _bwd(L, N=-3) == INVALID
    assert _bwd(L, scale=math.nan) == INVALID
    assert _bwd(L, causal=5) == INVALID
    assert _bwd(L, ws=NUL) == INVALID
    assert _bwd(L, dq=MIS) == INVALID
    assert _bwd(L, lse=NUL) == INVALID
    need = L.fa_bwd_workspace_bytes(2, 1, 1, 16, 64)
    assert _bwd(L, ws_bytes=need - 1) == WS


def test_bwd_halves_reject(L):
    """fa_bwd_dq_ws and fa_bwd_dkdv_ws check their arguments as fa_bwd does,
    before any HIP call."""
    need = L.fa_bwd_workspace_bytes(2, 1, 1, 16, 64)
    dq = lambda dtype=2, N=16, d=64, scale=0.125, causal=0, o=A, lse=A2, dqp=A2, ws=A, wb=need: \
        L.fa_bwd_dq_ws(dtype, 1, 1, N, d, A, A, A, o, A, lse, scale, causal, dqp, ws, wb, None)
    kv = lambda dtype=2, N=16, d=64, scale=0.125, causal=0, dk=A2, ws=A, wb=need: \
        L.fa_bwd_dkdv_ws(dtype, 1, 1, N, d, A, A, A, A, scale, causal, dk, A2, ws, wb, None)
    for f in (dq, kv):
        assert f(dtype=0) == UNSUP and f(d=32) == UNSUP
        assert f(N=0) == INVALID and f(scale=math.inf) == INVALID and f(causal=3) == INVALID
        assert f(ws=NUL) == INVALID and f(ws=MIS) == INVALID
        assert f(wb=need - 1) == WS
    assert dq(o=NUL) == INVALID and dq(lse=NUL) == INVALID and dq(dqp=MIS) == INVALID
    assert kv(dk=NUL) == INVALID


SCRATCH = _status("FA_ERR_SCRATCH")
MAX_ROWS = 1 << 22   # FA_BWD_NOALLOC_MAX_ROWS


def test_noalloc_rejects(L):
    """fa_bwd_noalloc checks its arguments as fa_bwd does and refuses problems
    with more rows than its static scratch holds, before any HIP call."""
    nb = lambda dtype=2, B=1, H=1, N=16, d=64, scale=0.125, causal=0, dq=A2, lse=A2: \
        L.fa_bwd_noalloc(dtype, B, H, N, d, A, A, A, A, A, lse, scale, causal, dq, A2, A2, None)
    assert "(1 << 22)" in open(HEADER).read()
    assert nb(dtype=0) == UNSUP and nb(d=32) == UNSUP
    assert nb(N=0) == INVALID and nb(scale=-1.0) == INVALID and nb(causal=2) == INVALID
    assert nb(dq=MIS) == INVALID and nb(lse=NUL) == INVALID
    assert nb(B=1, H=1, N=MAX_ROWS + 1) == SCRATCH
    assert nb(B=2, H=32, N=MAX_ROWS // 64 + 1) == SCRATCH
    assert nb(B=64, H=64, N=1025, d=128) == SCRATCH


def test_stage_entry_points_reject(L):
    assert L.fa_bwd_preprocess(2, 1, 1, 0, 64, A, A, A, None) == INVALID
    assert L.fa_bwd_preprocess(2, 1, 1, 8, 64, A, NUL, A, None) == INVALID
    assert L.fa_bwd_preprocess(0, 1, 1, 8, 64, A, A, A, None) == UNSUP
    assert L.fa_bwd_dkdv(1, 1, 1, 8, 64, A, A, A, A, A, A, 0.1, 3, A, A, None) == INVALID
    assert L.fa_bwd_dkdv(0, 1, 1, 8, 64, A, A, A, A, A, A, 0.1, 0, A, A, None) == UNSUP
    assert L.fa_bwd_dkdv(2, 1, 1, 8, 64, A, A, A, A, A, A, 0.1, 0, MIS, A, None) == INVALID
    assert L.fa_bwd_dkdv(2, 1, 1, 8, 64, A, A, A, A, A, NUL, 0.1, 0, A, A, None) == INVALID
    assert L.fa_bwd_dq(2, 1, 1, 8, 64, A, A, A, A, A, A, -0.5, 0, A, None) == INVALID
    assert L.fa_bwd_dq(2, 1, 1, 8, 96, A, A, A, A, A, A, 0.5, 0, A, None) == UNSUP
    assert L.fa_bwd_dq(2, 1, 1, 8, 64, A, A, A, A, A, A, 0.5, 0, NUL, None) == INVALID
    assert L.fa_bwd_dq_d(2, 1, 1, 8, 64, A, A, A, NUL, A, A, A, 0.5, 0, A, None) == INVALID
    assert L.fa_bwd_dq_d(2, 1, 1, 8, 64, A, A, A, A, A, A, NUL, 0.5, 0, A, None) == INVALID
    assert L.fa_bwd_dq_d(2, 1, 1, 8, 64, A, A, A, A, A, A, A, 0.5, 0, MIS, None) == INVALID
    assert L.fa_bwd_dq_d(0, 1, 1, 8, 64, A, A, A, A, A, A, A, 0.5, 0, A, None) == UNSUP
    assert L.fa_bwd_dq_d(2, 1, 1, 8, 64, A, A, A, A, A, A, A, 0.5, 2, A, None) == INVALID


@pytest.mark.parametrize("dtype,B,H,N,d", [(2, 1, 1, 1, 64), (1, 2, 3, 1000, 128),
                                          (2, 16, 32, 2048, 128),
                                          (2, 41, 400, 1024, 128)])  # tensors past 4 GiB
def test_workspace_bytes(L, dtype, B, H, N, d):
    """fp32 D [B,H,N] and fp32 LSE * log2(e) [B,H,N], each rounded up to 256 bytes."""
    dbytes = -(-B * H * N * 4 // 256) * 256
    assert L.fa_bwd_workspace_bytes(dtype, B, H, N, d) == 2 * dbytes
    assert L.fa_bwd_workspace_bytes(0, B, H, N, d) == 0     # fp32: no backward
    assert L.fa_bwd_workspace_bytes(dtype, B, H, N, 80) == 0
    assert L.fa_bwd_workspace_bytes(dtype, 1 << 16, 1 << 15, 1, d) == 0  # 2^31 rows


def test_binding_fails_loudly_without_gpu_tensors():
    """The Python face rejects CPU tensors instead of computing anything."""
    import torch
    import exact_attention_34_amd as fa
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)


def _split(L, dtype=2, N=16, d=64, nsplit=2, ws=A, ws_bytes=None, causal=0, o=A2):
    if ws_bytes is None:
        ws_bytes = L.fa_fwd_splitkv_workspace_bytes(dtype, 1, 1, N, d, nsplit,
                                                    causal if causal in (0, 1) else 0)
    return L.fa_fwd_splitkv(dtype, 1, 1, N, d, A, A, A, 0.125, causal, nsplit, o, A2, ws,
                            ws_bytes, None)


def test_splitkv_rejects(L):
    assert _split(L, dtype=0, ws_bytes=1 << 20) == UNSUP     # no fp32 split path
    assert _split(L, d=96, ws_bytes=1 << 20) == UNSUP
    assert _split(L, nsplit=-1, ws_bytes=1 << 20) == INVALID
    assert _split(L, nsplit=65, ws_bytes=1 << 20) == INVALID
    assert _split(L, causal=3) == INVALID
    assert _split(L, ws=NUL) == INVALID
    assert _split(L, o=MIS) == INVALID
    need = L.fa_fwd_splitkv_workspace_bytes(2, 1, 1, 16, 64, 2, 0)
    assert need > 0
    assert L.fa_fwd_splitkv_workspace_bytes(2, 1, 1, 16, 64, 2, 2) == 0
    assert _split(L, ws_bytes=need - 1) == WS


@pytest.mark.parametrize("N,nsplit,parts", [(1000, 4, 4), (100, 4, 2), (64, 3, 1),
                                             (65, 64, 2), (8192, 5, 5), (8192, 64, 64)])
def test_splitkv_parts_and_workspace(L, N, nsplit, parts):
    """Key tiles of 64 are divided evenly over at most nsplit non-empty ranges;
    the workspace holds every part's fp32 O and LSE."""
    for causal in (0, 1):
        assert L.fa_fwd_splitkv_parts(2, 3, N, nsplit, causal) == parts
        ob = -(-parts * 2 * 3 * N * 128 * 4 // 256) * 256
        lb = -(-parts * 2 * 3 * N * 4 // 256) * 256
        assert L.fa_fwd_splitkv_workspace_bytes(2, 2, 3, N, 128, nsplit, causal) == ob + lb
        assert L.fa_fwd_splitkv_workspace_bytes(0, 2, 3, N, 128, nsplit, causal) == 0
        assert L.fa_fwd_splitkv_parts(2, 3, N, -1, causal) == 0
    assert L.fa_fwd_splitkv_parts(2, 3, N, nsplit, 2) == 0


@pytest.mark.parametrize("B,H,N,causal,parts", [
    (1, 4, 8192, 0, 1),    # 256 query blocks: one per compute unit, no split
    (1, 4, 8192, 1, 2),    # 128 causal pair units: two ranges
    (1, 1, 8192, 0, 4),    # 64 blocks
    (1, 1, 8192, 1, 8),    # 32 pair units
    (2, 8, 1024, 0, 1),    # ranges would be shorter than 16 key tiles
    (16, 32, 2048, 1, 1),  # thousands of units
    (1, 2, 4096, 1, 4)])   # 32 pair units; 64 key tiles give at most 4 ranges
def test_self_attention_split_choice(L, B, H, N, causal, parts):
    """fa_fwd_splitkv with nsplit = 0 splits only when the unsplit forward's
    workgroups (128-row blocks, paired under the causal mask) number fewer
    than the compute units (256 without a device), with ranges of at least
    16 key tiles."""
    assert L.fa_fwd_splitkv_parts(B, H, N, 0, causal) == parts


@pytest.mark.parametrize("B,H,Nk,parts", [(16, 32, 8192, 1), (1, 32, 32768, 8), (4, 8, 65536, 8),
                                           (8, 8, 8192, 4), (1, 1, 300, 1), (1, 1, 100000, 63)])
def test_decoding_split_choice(L, B, H, Nk, parts):
    """Decoding (Nq = 1) with nsplit = 0: about one workgroup per compute unit
    (256 without a device), ranges of at least 256 keys, at most 64 requested
    (whole 64-key tiles divided evenly: 100000 keys in 64 requested ranges
    make 63 of 25 tiles)."""
    assert L.fa_fwd_kvcache_parts(B, H, 1, Nk, 0, 1) == parts


def test_lse_merge_rejects(L):
    m = lambda dtype=0, parts=2, rows=10, d=64, op=A, lp=A, o=A2, lse=A2: L.fa_lse_merge(
        dtype, parts, rows, d, op, lp, o, lse, None)
    assert m(parts=0) == INVALID
    assert m(rows=0) == INVALID
    assert m(d=96) == UNSUP
    assert m(dtype=3) == UNSUP
    assert m(op=NUL) == INVALID
    assert m(lp=NUL) == INVALID
    assert m(o=MIS) == INVALID
    assert m(lse=NUL) == INVALID


def test_kvcache_rejects(L):
    k = lambda dtype=2, Nq=4, Nk=100, d=64, causal=1, nsplit=0, ws=A, nb=1 << 24, o=A2: \
        L.fa_fwd_kvcache(dtype, 1, 2, Nq, Nk, d, A, A, A, 0.125, causal, nsplit, o, A2, ws, nb,
                         None)
    assert k(Nq=101) == INVALID          # causal needs Nq <= Nk
    assert k(Nq=0) == INVALID and k(Nk=0) == INVALID
    assert k(dtype=0) == UNSUP and k(d=80) == UNSUP
    assert k(nsplit=65) == INVALID
    assert k(ws=NUL) == INVALID and k(o=MIS) == INVALID
    assert k(nb=16) == WS
    assert L.fa_fwd_kvcache_workspace_bytes(2, 1, 2, 4, 100, 64, 2, 1) > 0
    assert L.fa_fwd_kvcache_workspace_bytes(0, 1, 2, 4, 100, 64, 2, 1) == 0
    # Nq > Nk is allowed without the mask (every query sees every key), not
    # with it
    assert L.fa_fwd_kvcache_workspace_bytes(2, 1, 2, 300, 100, 64, 2, 0) > 0
    assert L.fa_fwd_kvcache_workspace_bytes(2, 1, 2, 300, 100, 64, 2, 1) == 0
    assert L.fa_fwd_kvcache_parts(1, 2, 4, 100, 2, 3) == 0


@pytest.mark.parametrize("Nq,Nk,nsplit,parts", [(1, 8192, 8, 8), (7, 100, 4, 2), (512, 8192, 3, 3)])
def test_kvcache_parts_and_workspace(L, Nq, Nk, nsplit, parts):
    """Ranges are cut from the Nk keys; the workspace holds fp32 O and LSE for
    the Nq query rows of every part."""
    for causal in (0, 1):
        assert L.fa_fwd_kvcache_parts(2, 3, Nq, Nk, nsplit, causal) == parts
        ob = -(-parts * 6 * Nq * 128 * 4 // 256) * 256
        lb = -(-parts * 6 * Nq * 4 // 256) * 256
        assert L.fa_fwd_kvcache_workspace_bytes(2, 2, 3, Nq, Nk, 128, nsplit, causal) == ob + lb


# ---------------------------------------------------------------------------
# Standard attention (stores S and P)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,ld", [(1, 128), (128, 128), (129, 256), (1000, 1024), (2048, 2048)])
def test_std_row_stride_and_bytes(L, N, ld):
    """N x N arrays have rows of N rounded up to 128 elements; P is 16-bit, S
    fp32, the backward workspace dS (16-bit) then D (fp32), each part padded
    to 256 bytes."""
    r = lambda x: -(-x // 256) * 256
    assert L.fa_std_row_stride(N) == ld
    B, H, d = 2, 3, 64
    assert L.fa_std_p_bytes(2, B, H, N, d) == B * H * N * ld * 2
    assert L.fa_std_fwd_workspace_bytes(1, B, H, N, d) == r(B * H * N * ld * 4)
    assert L.fa_std_bwd_workspace_bytes(2, B, H, N, d) == r(B * H * N * ld * 2) + r(B * H * N * 4)
    assert L.fa_std_p_bytes(0, B, H, N, d) == 0            # fp32 is not built
    assert L.fa_std_fwd_workspace_bytes(2, B, H, N, 96) == 0
    assert L.fa_std_bwd_workspace_bytes(2, 0, H, N, d) == 0


def _std_fwd(L, dtype=2, N=16, d=64, scale=0.125, causal=0, o=A2, P=A2, ws=A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.fa_std_fwd_workspace_bytes(dtype, 1, 1, N, d)
    return L.fa_std_fwd(dtype, 1, 1, N, d, A, A, A, scale, causal, o, A2, P, ws, ws_bytes,
                        None)


def _std_bwd(L, dtype=2, N=16, d=64, scale=0.125, P=A, dq=A2, ws=A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.fa_std_bwd_workspace_bytes(dtype, 1, 1, N, d)
    return L.fa_std_bwd(dtype, 1, 1, N, d, A, A, A, A, A, P, scale, dq, A2, A2, ws, ws_bytes,
                        None)


def test_std_rejects(L):
    assert _std_fwd(L, dtype=0) == UNSUP
    assert _std_fwd(L, d=32) == UNSUP
    assert _std_fwd(L, N=0) == INVALID
    assert _std_fwd(L, scale=math.inf) == INVALID
    assert _std_fwd(L, causal=2) == INVALID
    assert _std_fwd(L, o=MIS) == INVALID
    assert _std_fwd(L, P=NUL) == INVALID
    assert _std_fwd(L, ws=ctypes.c_void_p(0x10010)) == INVALID   # workspace not 256-aligned
    assert _std_fwd(L, ws_bytes=L.fa_std_fwd_workspace_bytes(2, 1, 1, 16, 64) - 1) == WS
    # B*H*N*d < 2^31, but 64 slices of 65536 x 65536 reach the 2^38 limit
    assert L.fa_std_fwd(2, 8, 8, 1 << 16, 64, A, A, A, 0.1, 0, A2, A2, A2, A, 1 << 62,
                        None) == INVALID
    assert L.fa_std_p_bytes(2, 8, 8, 1 << 16, 64) == 0
    assert _std_bwd(L, dtype=0) == UNSUP
    assert _std_bwd(L, scale=0.0) == INVALID
    assert _std_bwd(L, P=MIS) == INVALID
    assert _std_bwd(L, dq=NUL) == INVALID
    assert _std_bwd(L, ws=NUL) == INVALID
    assert _std_bwd(L, ws_bytes=L.fa_std_bwd_workspace_bytes(2, 1, 1, 16, 64) - 1) == WS
