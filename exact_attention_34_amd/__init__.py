"""Exact attention (forward and recompute backward) on AMD MI355X.

A thin ctypes binding over ``libfa.so``, whose C ABI is declared in
``include/fa.h``. This module only marshals arguments: it checks tensors,
allocates the outputs with torch on the tensors' device, and passes raw
pointers plus torch's current HIP stream to the library. Every step of the
computation runs in the library's HIP kernels; there is no other code path.
If the library has not been built, every call raises.
"""
import ctypes
import math
import os

import torch

__all__ = ["fwd", "fwd_splitkv", "fwd_splitkv_parts", "fwd_splitkv_workspace_bytes",
           "fwd_kvcache", "fwd_kvcache_parts", "fwd_kvcache_workspace_bytes", "lse_merge",
           "bwd", "bwd_dq_ws", "bwd_dkdv_ws", "bwd_noalloc", "bwd_preprocess", "bwd_dkdv",
           "bwd_dq", "bwd_dq_d", "bwd_workspace_bytes", "FAError", "library_path", "lib",
           "F32", "F16", "BF16"]

F32, F16, BF16 = 0, 1, 2
_CODES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
_lib = None


class FAError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, fn, code):
        msg = lib().fa_status_str(code).decode() if _lib is not None else str(code)
        super().__init__("%s failed: %s (%d)" % (fn, msg, code))
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libfa.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libfa.so is not built; run __graft_entry__.build() "
                          "(or python exact_attention_34_amd/build.py)")
    L = ctypes.CDLL(_LIB_PATH)
    i, f, p, z = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    L.fa_abi_version.restype = i
    L.fa_status_str.argtypes = [i]
    L.fa_status_str.restype = ctypes.c_char_p
    L.fa_fwd.argtypes = [i, i, i, i, i, p, p, p, f, i, p, p, p]
    L.fa_fwd.restype = i
    L.fa_fwd_splitkv.argtypes = [i, i, i, i, i, p, p, p, f, i, i, p, p, p, z, p]
    L.fa_fwd_splitkv.restype = i
    L.fa_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.fa_fwd_splitkv_workspace_bytes.restype = z
    L.fa_fwd_splitkv_parts.argtypes = [i, i, i, i, i]
    L.fa_fwd_splitkv_parts.restype = i
    L.fa_fwd_kvcache.argtypes = [i, i, i, i, i, i, p, p, p, f, i, i, p, p, p, z, p]
    L.fa_fwd_kvcache.restype = i
    L.fa_fwd_kvcache_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    L.fa_fwd_kvcache_workspace_bytes.restype = z
    L.fa_fwd_kvcache_parts.argtypes = [i, i, i, i, i, i]
    L.fa_fwd_kvcache_parts.restype = i
    L.fa_lse_merge.argtypes = [i, i, ctypes.c_longlong, i, p, p, p, p, p]
    L.fa_lse_merge.restype = i
    L.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    L.fa_bwd_workspace_bytes.restype = z
    L.fa_bwd.argtypes = [i, i, i, i, i, p, p, p, p, p, p, f, i, p, p, p, p, z, p]
    L.fa_bwd.restype = i
    L.fa_bwd_dq_ws.argtypes = [i, i, i, i, i, p, p, p, p, p, p, f, i, p, p, z, p]
    L.fa_bwd_dq_ws.restype = i
    L.fa_bwd_dkdv_ws.argtypes = [i, i, i, i, i, p, p, p, p, f, i, p, p, p, z, p]
    L.fa_bwd_dkdv_ws.restype = i
    L.fa_bwd_noalloc.argtypes = [i, i, i, i, i, p, p, p, p, p, p, f, i, p, p, p, p]
    L.fa_bwd_noalloc.restype = i
    L.fa_bwd_preprocess.argtypes = [i, i, i, i, i, p, p, p, p]
    L.fa_bwd_preprocess.restype = i
    L.fa_bwd_dkdv.argtypes = [i, i, i, i, i, p, p, p, p, p, p, f, i, p, p, p]
    L.fa_bwd_dkdv.restype = i
    L.fa_bwd_dq.argtypes = [i, i, i, i, i, p, p, p, p, p, p, f, i, p, p]
    L.fa_bwd_dq.restype = i
    L.fa_bwd_dq_d.argtypes = [i, i, i, i, i, p, p, p, p, p, p, p, f, i, p, p]
    L.fa_bwd_dq_d.restype = i
    L.fa_std_row_stride.argtypes = [i]
    L.fa_std_row_stride.restype = i
    for name in ("fa_std_p_bytes", "fa_std_fwd_workspace_bytes", "fa_std_bwd_workspace_bytes"):
        getattr(L, name).argtypes = [i, i, i, i, i]
        getattr(L, name).restype = z
    L.fa_std_fwd.argtypes = [i, i, i, i, i, p, p, p, f, i, p, p, p, p, z, p]
    L.fa_std_fwd.restype = i
    L.fa_std_bwd.argtypes = [i, i, i, i, i, p, p, p, p, p, p, f, p, p, p, p, z, p]
    L.fa_std_bwd.restype = i
    _lib = L
    return L


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_qkv(*ts):
    t0 = ts[0]
    if t0.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in ts:
        if t.shape != t0.shape or t.dtype != t0.dtype or t.device != t0.device:
            raise ValueError("tensors must share shape, dtype and device")
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if t0.dtype not in _CODES:
        raise ValueError("unsupported dtype %s" % t0.dtype)
    return (_CODES[t0.dtype],) + tuple(t0.shape)


def _check_rows(t, name, ref):
    """A per-row fp32 vector (LSE or D) that the kernels index as [B, H, N]
    on ref's device: anything else would be read or written out of bounds."""
    B, H, N = ref.shape[:3]
    if (not isinstance(t, torch.Tensor) or t.shape != (B, H, N) or t.dtype != torch.float32
            or t.device != ref.device or not t.is_contiguous()):
        raise ValueError("%s must be a contiguous fp32 [B, H, N] tensor on %s"
                         % (name, ref.device))


def _workspace(ws, nbytes, ref):
    """The caller's workspace (device memory on ref's device, contiguous, at
    least nbytes) or a new one."""
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=ref.device)
    if (not isinstance(ws, torch.Tensor) or ws.device != ref.device or not ws.is_contiguous()
            or ws.numel() * ws.element_size() < nbytes):
        raise ValueError("workspace must be a contiguous tensor of at least %d bytes on %s"
                         % (nbytes, ref.device))
    return ws


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _call(fn, *args):
    rc = getattr(lib(), fn)(*args)
    if rc != 0:
        raise FAError(fn, rc)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def fwd(q, k, v, scale=None, causal=False):
    """O, LSE = attention(q, k, v). q, k, v: [B, H, N, d] on the GPU."""
    dt, B, H, N, d = _check_qkv(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _call("fa_fwd", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _scale(scale, d),
          int(bool(causal)), _ptr(o), _ptr(lse), _stream(q))
    return o, lse


def fwd_splitkv_workspace_bytes(dtype, B, H, N, d, nsplit=0, causal=False):
    return int(lib().fa_fwd_splitkv_workspace_bytes(_CODES[dtype], B, H, N, d, int(nsplit),
                                                   int(bool(causal))))


def fwd_splitkv_parts(B, H, N, nsplit=0, causal=False):
    """Key ranges fwd_splitkv uses for this nsplit (0: the library's choice)."""
    return int(lib().fa_fwd_splitkv_parts(B, H, N, int(nsplit), int(bool(causal))))


def fwd_splitkv(q, k, v, scale=None, causal=False, nsplit=0, workspace=None):
    """O, LSE as fwd(), with each row's keys split into ranges swept by separate
    workgroups and the partial results merged (nsplit=0: the library picks)."""
    dt, B, H, N, d = _check_qkv(q, k, v)
    nbytes = fwd_splitkv_workspace_bytes(q.dtype, B, H, N, d, nsplit, causal)
    workspace = _workspace(workspace, nbytes, q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _call("fa_fwd_splitkv", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _scale(scale, d),
          int(bool(causal)), int(nsplit), _ptr(o), _ptr(lse), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(q))
    return o, lse


def fwd_kvcache_workspace_bytes(dtype, B, H, Nq, Nk, d, nsplit=0, causal=True):
    return int(lib().fa_fwd_kvcache_workspace_bytes(_CODES[dtype], B, H, Nq, Nk, d,
                                                   int(nsplit), int(bool(causal))))


def fwd_kvcache_parts(B, H, Nq, Nk, nsplit=0, causal=True):
    return int(lib().fa_fwd_kvcache_parts(B, H, Nq, Nk, int(nsplit), int(bool(causal))))


def fwd_kvcache(q, k, v, scale=None, causal=True, nsplit=0, workspace=None):
    """O, LSE of Nq new queries ([B, H, Nq, d]) over Nk cached keys and values
    ([B, H, Nk, d]); under the causal mask query i sits at position Nk-Nq+i."""
    for t in (q, k, v):
        if (t.dim() != 4 or not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype
                or t.device != q.device):
            raise ValueError("expected contiguous GPU tensors [B, H, n, d] of one dtype "
                             "on one device")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, d]")
    if q.dtype not in _CODES:
        raise ValueError("unsupported dtype %s" % q.dtype)
    nbytes = fwd_kvcache_workspace_bytes(q.dtype, B, H, Nq, Nk, d, nsplit, causal)
    workspace = _workspace(workspace, nbytes, q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _call("fa_fwd_kvcache", _CODES[q.dtype], B, H, Nq, Nk, d, _ptr(q), _ptr(k), _ptr(v),
          _scale(scale, d), int(bool(causal)), int(nsplit), _ptr(o), _ptr(lse),
          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q))
    return o, lse


def lse_merge(o_parts, lse_parts, out_dtype=torch.float32):
    """Merge partial results over disjoint key sets.

    o_parts: fp32 [P, rows, d]; lse_parts: fp32 [P, rows] (-inf: empty part).
    Returns (o [rows, d] in out_dtype, lse fp32 [rows])."""
    if o_parts.dim() != 3 or lse_parts.shape != o_parts.shape[:2]:
        raise ValueError("expected o_parts [P, rows, d] and lse_parts [P, rows]")
    for t in (o_parts, lse_parts):
        if (t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous()
                or t.device != o_parts.device):
            raise ValueError("parts must be contiguous fp32 GPU tensors on one device")
    if out_dtype not in _CODES:
        raise ValueError("unsupported dtype %s" % out_dtype)
    P, rows, d = o_parts.shape
    o = torch.empty((rows, d), dtype=out_dtype, device=o_parts.device)
    lse = torch.empty(rows, dtype=torch.float32, device=o_parts.device)
    _call("fa_lse_merge", _CODES[out_dtype], P, rows, d, _ptr(o_parts), _ptr(lse_parts),
          _ptr(o), _ptr(lse), _stream(o_parts))
    return o, lse


def bwd_workspace_bytes(dtype, B, H, N, d):
    return int(lib().fa_bwd_workspace_bytes(_CODES[dtype], B, H, N, d))


def bwd(q, k, v, o, do, lse, scale=None, causal=False, workspace=None):
    """dQ, dK, dV of attention given dO, and O, LSE from fwd()."""
    dt, B, H, N, d = _check_qkv(q, k, v, o, do)
    _check_rows(lse, "lse", q)
    nbytes = bwd_workspace_bytes(q.dtype, B, H, N, d)
    workspace = _workspace(workspace, nbytes, q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _call("fa_bwd", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
          _ptr(lse), _scale(scale, d), int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q))
    return dq, dk, dv


def bwd_dq_ws(q, k, v, o, do, lse, dq, workspace, scale=None, causal=False):
    """The first launch of bwd: dQ, with D and the scaled LSE written into
    `workspace` (a bwd_workspace_bytes() buffer) for bwd_dkdv_ws."""
    dt, B, H, N, d = _check_qkv(q, k, v, o, do, dq)
    _check_rows(lse, "lse", q)
    if workspace is None:
        raise ValueError("bwd_dq_ws needs the workspace that bwd_dkdv_ws will read")
    workspace = _workspace(workspace, bwd_workspace_bytes(q.dtype, B, H, N, d), q)
    _call("fa_bwd_dq_ws", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
          _ptr(lse), _scale(scale, d), int(bool(causal)), _ptr(dq), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(q))


def bwd_dkdv_ws(q, k, v, do, dk, dv, workspace, scale=None, causal=False):
    """The second launch of bwd: dK and dV, reading what bwd_dq_ws wrote into
    `workspace` for the same inputs."""
    dt, B, H, N, d = _check_qkv(q, k, v, do, dk, dv)
    if workspace is None:
        raise ValueError("bwd_dkdv_ws reads the workspace that bwd_dq_ws wrote")
    workspace = _workspace(workspace, bwd_workspace_bytes(q.dtype, B, H, N, d), q)
    _call("fa_bwd_dkdv_ws", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(do),
          _scale(scale, d), int(bool(causal)), _ptr(dk), _ptr(dv), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(q))


def bwd_noalloc(q, k, v, o, do, lse, scale=None, causal=False, out=None):
    """bwd() through fa_bwd_noalloc: D lives in the library's static scratch
    instead of a workspace. out: optional (dq, dk, dv) tensors to write into
    (shaped like q, contiguous, on q's device); else they are allocated here."""
    dt, B, H, N, d = _check_qkv(q, k, v, o, do)
    _check_rows(lse, "lse", q)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    else:
        _check_qkv(q, *out)
    dq, dk, dv = out
    _call("fa_bwd_noalloc", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
          _ptr(lse), _scale(scale, d), int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv),
          _stream(q))
    return dq, dk, dv


def bwd_preprocess(o, do, dvec):
    """Stage 1 of bwd: dvec = rowsum(dO o O), fp32 [B, H, N]."""
    dt, B, H, N, d = _check_qkv(o, do)
    _check_rows(dvec, "dvec", o)
    _call("fa_bwd_preprocess", dt, B, H, N, d, _ptr(o), _ptr(do), _ptr(dvec), _stream(o))


def bwd_dkdv(q, k, v, do, lse, dvec, dk, dv, scale=None, causal=False):
    """Stage 2 of bwd: dK and dV (key blocks outer)."""
    dt, B, H, N, d = _check_qkv(q, k, v, do, dk, dv)
    _check_rows(lse, "lse", q)
    _check_rows(dvec, "dvec", q)
    _call("fa_bwd_dkdv", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse),
          _ptr(dvec), _scale(scale, d), int(bool(causal)), _ptr(dk), _ptr(dv), _stream(q))


def bwd_dq_d(q, k, v, o, do, lse, dvec, dq, scale=None, causal=False):
    """Stage 3 with stage 1 folded in: dQ, and dvec = rowsum(dO o O) written
    for a bwd_dkdv that follows."""
    dt, B, H, N, d = _check_qkv(q, k, v, o, do, dq)
    _check_rows(lse, "lse", q)
    _check_rows(dvec, "dvec", q)
    _call("fa_bwd_dq_d", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
          _ptr(lse), _ptr(dvec), _scale(scale, d), int(bool(causal)), _ptr(dq), _stream(q))


def bwd_dq(q, k, v, do, lse, dvec, dq, scale=None, causal=False):
    """Stage 3 of bwd: dQ (query blocks outer)."""
    dt, B, H, N, d = _check_qkv(q, k, v, do, dq)
    _check_rows(lse, "lse", q)
    _check_rows(dvec, "dvec", q)
    _call("fa_bwd_dq", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse),
          _ptr(dvec), _scale(scale, d), int(bool(causal)), _ptr(dq), _stream(q))


def std_row_stride(N):
    """Row stride (elements) of the N x N arrays of the standard path."""
    return int(lib().fa_std_row_stride(N))


def std_p_bytes(dtype, B, H, N, d):
    return int(lib().fa_std_p_bytes(_CODES[dtype], B, H, N, d))


def std_fwd_workspace_bytes(dtype, B, H, N, d):
    return int(lib().fa_std_fwd_workspace_bytes(_CODES[dtype], B, H, N, d))


def std_bwd_workspace_bytes(dtype, B, H, N, d):
    return int(lib().fa_std_bwd_workspace_bytes(_CODES[dtype], B, H, N, d))


def std_fwd(q, k, v, scale=None, causal=False, workspace=None):
    """O, LSE, P of standard attention that stores S and P in device memory.
    P is [B, H, N, std_row_stride(N)] in q's dtype (padding columns zero)."""
    dt, B, H, N, d = _check_qkv(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    P = torch.empty((B, H, N, std_row_stride(N)), dtype=q.dtype, device=q.device)
    workspace = _workspace(workspace, std_fwd_workspace_bytes(q.dtype, B, H, N, d), q)
    _call("fa_std_fwd", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _scale(scale, d),
          int(bool(causal)), _ptr(o), _ptr(lse), _ptr(P), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(q))
    return o, lse, P


def std_bwd(q, k, v, o, do, P, scale=None, workspace=None):
    """dQ, dK, dV of the standard path from the stored P of std_fwd()."""
    dt, B, H, N, d = _check_qkv(q, k, v, o, do)
    if (P.shape != (B, H, N, std_row_stride(N)) or P.dtype != q.dtype or not P.is_contiguous()
            or P.device != q.device):
        raise ValueError("P must be std_fwd's [B, H, N, row stride] array")
    workspace = _workspace(workspace, std_bwd_workspace_bytes(q.dtype, B, H, N, d), q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _call("fa_std_bwd", dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(P),
          _scale(scale, d), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(q))
    return dq, dk, dv
