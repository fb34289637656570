"""ctypes binding of libcsa.so: argument marshalling only.

Each function here has the name of the C entry point it calls and does no
arithmetic of its own: it checks that tensors are on the GPU, contiguous and
of one dtype, takes their data pointers and the current HIP stream, and
raises CsaError on a non-zero return code.  Output and scratch tensors are
allocated with torch when the caller does not pass them.  There is no CPU
path: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSA_LIBRARY names another build of the same library (the host-sanitizer
# build the CPU tests load); by default the in-tree libcsa.so.
LIB_PATH = os.environ.get("CSA_LIBRARY") or os.path.join(_HERE, "libcsa.so")

CSA_F32 = 0
CSA_BF16 = 1
CSA_FP8 = 2   # OCP E4M3 (torch.float8_e4m3fn): indexer queries and keys only
_DT = {torch.float32: CSA_F32, torch.bfloat16: CSA_BF16, torch.float8_e4m3fn: CSA_FP8}

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_int = ctypes.c_int
_sz = ctypes.c_size_t
_f32 = ctypes.c_float

# name -> (restype, argtypes); mirrors include/csa.h
SIGNATURES = {
    "csa_version": (ctypes.c_char_p, []),
    "csa_strerror": (ctypes.c_char_p, [_int]),
    "csa_debug_enabled": (_int, []),
    "csa_debug_set_entry_limit": (_int, [ctypes.c_int64]),
    "csa_compress": (_int, [_vp] * 8 + [_i64] * 4 + [_int, _int, _vp, _i64, _vp]),
    "csa_index_topk": (_int, [_vp, _vp, _vp, _i64] + [_i64] * 8 + [_int, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_workspace_size": (_sz, [_i64] * 4),
    "csa_index_topk_noalloc": (_int, [_vp, _vp, _vp, _i64] + [_i64] * 8 + [_int, _vp, _vp, _vp]),
    "csa_index_topk_mxfp4": (_int, [_vp] * 5 + [_i64] * 9 + [_vp, _vp, _vp, _sz, _vp]),
    "csa_quantize_mxfp4": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp]),
    "csa_grouped_out_proj": (_int, [_vp, _vp, _vp] + [_i64] * 6 + [_int, _vp, _vp, _vp]),
    "csa_norm_rope": (_int, [_vp, _i64, _vp, _i64, _vp, _f32, _i64, _i64, _i64, _i64, ctypes.c_double,
                             _i64, _i64, _int, _vp]),
    "csa_attend": (_int, [_vp, _vp, _i64, _vp, _vp, _i64, _i64, _vp] + [_i64] * 10
                   + [_f32, _int, _vp, _sz, _vp, _vp]),
    "csa_attend_norm_rope": (_int, [_vp, _vp, _f32, _i64, ctypes.c_double, _vp, _i64, _vp, _vp, _i64, _i64, _vp]
                             + [_i64] * 10 + [_f32, _int, _vp, _sz, _vp, _vp]),
    "csa_attend_workspace_size": (_sz, [_i64] * 9 + [_int]),
    "hca_attend": (_int, [_vp, _vp, _i64, _vp, _i64, _i64, _vp] + [_i64] * 9
                   + [_f32, _int, _vp, _sz, _vp, _vp]),
    "hca_attend_workspace_size": (_sz, [_i64] * 8 + [_int]),
    "hca_attend_norm_rope": (_int, [_vp, _vp, _f32, _i64, ctypes.c_double, _vp, _i64, _vp, _i64, _i64, _vp]
                             + [_i64] * 9 + [_f32, _int, _vp, _sz, _vp, _vp]),
    "hca_layer": (_int, [_vp] * 6 + [_i64] * 6 + [_f32, _int, _vp, _vp, _sz, _vp, _vp]),
    "hca_layer_workspace_size": (_sz, [_i64] * 6 + [_int]),
    "csa_paged_block_bytes": (_sz, [_i64] * 4),
    "csa_paged_state_bytes": (_sz, [_i64] * 5),
    "csa_paged_append": (_int, [_vp, _vp, _i64, _vp, _i64, _vp, _vp, _i64] + [_vp] * 15 + [_i64] * 5
                         + [_int, _vp]),
    "csa_paged_index_topk": (_int, [_vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp] + [_i64] * 8
                             + [_int, _vp, _vp, _vp, _sz, _vp]),
    "csa_paged_attend": (_int, [_vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp] + [_i64] * 9
                         + [_f32, _int, _vp, _sz, _vp, _vp]),
    "csa_paged_attend_workspace_size": (_sz, [_i64] * 4),
    "hca_paged_attend": (_int, [_vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp] + [_i64] * 8
                         + [_f32, _int, _vp, _sz, _vp, _vp]),
    "hca_paged_attend_workspace_size": (_sz, [_i64] * 4),
    "csa_quantize_kv_fp8": (_int, [_vp, _i64, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _vp]),
    "csa_attend_fp8kv": (_int, [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _vp] + [_i64] * 11
                         + [_f32, _vp, _sz, _vp, _vp]),
    "csa_attend_fp8kv_workspace_size": (_sz, [_i64] * 9),
    "csa_attend_backward": (_int, [_vp, _vp, _i64, _vp, _vp, _i64, _i64, _vp, _vp] + [_i64] * 10
                            + [_f32, _int, _int, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _sz, _vp]),
    "csa_attend_backward_workspace_size": (_sz, [_i64] * 6),
    "hca_attend_backward": (_int, [_vp, _vp, _i64, _vp, _i64, _i64, _vp, _vp] + [_i64] * 9
                            + [_f32, _int, _int, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _sz, _vp]),
    "hca_attend_backward_workspace_size": (_sz, [_i64] * 6),
    "csa_compress_backward": (_int, [_vp] * 9 + [_i64] * 4 + [_int, _int] + [_vp] * 9 + [_sz, _vp]),
    "csa_compress_backward_workspace_size": (_sz, [_i64] * 3),
    "csa_block_pool_create": (_vp, [_i64]),
    "csa_block_pool_destroy": (None, [_vp]),
    "csa_block_pool_alloc": (_int, [_vp, _i64, _vp]),
    "csa_block_pool_release": (_int, [_vp, _i64, _vp]),
    "csa_block_pool_available": (_i64, [_vp]),
}


class CsaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} ({code})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcsa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m long_context_compressed_csa_amd.build`")
        _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """A build of the library at `path` (e.g. the CSA_DEBUG build,
    libcsa_debug.so) with every entry point's prototype set; not cached."""
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def strerror(code: int) -> str:
    return load_library().csa_strerror(code).decode()


def version() -> str:
    return load_library().csa_version().decode()


# ----------------------------------------------------------------- helpers --

def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _dtype(*ts):
    dts = {t.dtype for t in ts if t is not None}
    if len(dts) != 1:
        raise ValueError(f"tensors must share one dtype, got {dts}")
    dt = dts.pop()
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    return _DT[dt]


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(rc, where):
    if rc != 0:
        raise CsaError(rc, where)


def _f32c(t, name):
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    return _ptr(t)


def _batched(t, nd):
    """View [..] as having a leading batch dim when it is missing."""
    return t if t is None or t.dim() == nd else t.unsqueeze(0)


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    # 256-byte alignment is guaranteed by the caching allocator
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ------------------------------------------------------------ entry points --

def csa_compress(Ca, Cb, Za, Zb, Ba, Bb, m, prev_Cb=None, prev_Zb=None, out=None,
                 overlap=True, stream=None):
    """Compressor (overlap=True: CSA form; False: HCA pooling, pass Cb=Zb=Bb=None).

    Streams [b, n, c] or [n, c]; biases [m, c]; returns [b, n//m, c] (or
    [n//m, c] for 2-D inputs) unless `out` is given.
    """
    squeeze = Ca.dim() == 2
    Ca, Cb, Za, Zb = (_batched(x, 3) for x in (Ca, Cb, Za, Zb))
    prev_Cb, prev_Zb = _batched(prev_Cb, 3), _batched(prev_Zb, 3)
    b, n, c = Ca.shape
    dt = _dtype(Ca, Cb, Za, Zb, Ba, Bb, prev_Cb, prev_Zb)
    out_bstride = 0
    if out is None:
        out = torch.empty((b, n // m, c), dtype=Ca.dtype, device=Ca.device)
        ret = out[0] if squeeze else out
    else:
        ret = out
        o3 = _batched(out, 3)
        if o3.dtype != Ca.dtype or not o3.is_cuda:
            raise ValueError("out must be a GPU tensor of the input dtype")
        if o3.shape != (b, n // m, c) or o3.stride(2) != 1 or o3.stride(1) != c:
            raise ValueError("out must be [b, n//m, c] with dense rows")
        out_bstride = o3.stride(0) if b > 1 else 0
        out = o3
    lib = load_library()
    rc = lib.csa_compress(_ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), _ptr(Ba), _ptr(Bb),
                          _ptr(prev_Cb), _ptr(prev_Zb), b, n, c, m, 1 if overlap else 0, dt,
                          out.data_ptr(), out_bstride, _stream(stream))
    _check(rc, "csa_compress")
    return ret


CSA_SCORE_BF16 = 0x100


def csa_index_topk(qI, w, KIcomp, t0, m, k, n_comp=None, score=False, idx=None,
                   workspace=None, stream=None, bf16_scores=False):
    """Indexer scores + top-k.  qI [b, n_q, n_hI, c_I]; w [b, n_q, n_hI] f32;
    KIcomp [b, cap, c_I] (first n_comp rows used).  Returns idx int32
    [b, n_q, k] (and the scores when score=True).  bf16_scores: select on
    scores rounded to bfloat16 (CSA_SCORE_BF16)."""
    qI, w, KIcomp = _batched(qI, 4), _batched(w, 3), _batched(KIcomp, 3)
    b, n_q, nh, cI = qI.shape
    n_comp = KIcomp.shape[1] if n_comp is None else n_comp
    dt = _dtype(qI, KIcomp) | (CSA_SCORE_BF16 if bf16_scores else 0)
    lib = load_library()
    need = lib.csa_index_topk_workspace_size(b, n_q, n_comp, k)
    if workspace is None:
        workspace = _workspace(max(need, 256), qI.device)
    if idx is None:
        idx = torch.empty((b, n_q, k), dtype=torch.int32, device=qI.device)
    sc = torch.empty((b, n_q, k), dtype=torch.float32, device=qI.device) if score else None
    rc = lib.csa_index_topk(_ptr(qI), _f32c(w, "w"), _ptr(KIcomp), KIcomp.stride(0), b, n_q, t0,
                            n_comp, nh, cI, m, k, dt, _ptr(idx), _ptr(sc), _ptr(workspace),
                            workspace.numel(), _stream(stream))
    _check(rc, "csa_index_topk")
    return (idx, sc) if score else idx


def csa_index_topk_noalloc(qI, w, KIcomp, t0, m, k, n_comp=None, score=False, idx=None, stream=None):
    """csa_index_topk on the library's own per-GPU scratch (no workspace
    argument and no allocation for scratch; outputs are allocated here unless
    given).  Calls that overlap on one GPU race on that scratch."""
    qI, w, KIcomp = _batched(qI, 4), _batched(w, 3), _batched(KIcomp, 3)
    b, n_q, nh, cI = qI.shape
    n_comp = KIcomp.shape[1] if n_comp is None else n_comp
    dt = _dtype(qI, KIcomp)
    lib = load_library()
    if idx is None:
        idx = torch.empty((b, n_q, k), dtype=torch.int32, device=qI.device)
    sc = torch.empty((b, n_q, k), dtype=torch.float32, device=qI.device) if score else None
    rc = lib.csa_index_topk_noalloc(_ptr(qI), _f32c(w, "w"), _ptr(KIcomp), KIcomp.stride(0), b, n_q, t0, n_comp,
                                    nh, cI, m, k, dt, _ptr(idx), _ptr(sc), _stream(stream))
    _check(rc, "csa_index_topk_noalloc")
    return (idx, sc) if score else idx


def csa_index_topk_mxfp4(qI, qI_scale, w, KIcomp, KI_scale, t0, m, k, n_comp=None, score=False, idx=None,
                         workspace=None, stream=None):
    """Indexer scores + top-k over OCP MXFP4 queries and keys.  qI [b, n_q,
    n_hI, c_I/2] uint8 E2M1 pairs and qI_scale [b, n_q, n_hI, c_I/32] uint8
    E8M0; w [b, n_q, n_hI] f32; KIcomp [b, cap, c_I/2] and KI_scale [b, cap,
    c_I/32] uint8 (first n_comp rows used).  Returns idx int32 [b, n_q, k]
    (and the scores when score=True)."""
    qI, qI_scale, w = _batched(qI, 4), _batched(qI_scale, 4), _batched(w, 3)
    KIcomp, KI_scale = _batched(KIcomp, 3), _batched(KI_scale, 3)
    for t, name in ((qI, "qI"), (qI_scale, "qI_scale"), (KIcomp, "KIcomp"), (KI_scale, "KI_scale")):
        if t.dtype != torch.uint8:
            raise ValueError(f"{name} must be uint8 (packed E2M1 codes or E8M0 scales)")
    b, n_q, nh, half = qI.shape
    cI = 2 * half
    if KIcomp.shape[1] != KI_scale.shape[1] or KIcomp.shape[2] != half or KI_scale.shape[2] * 32 != cI:
        raise ValueError("KIcomp / KI_scale shapes do not match qI")
    n_comp = KIcomp.shape[1] if n_comp is None else n_comp
    lib = load_library()
    need = lib.csa_index_topk_workspace_size(b, n_q, n_comp, k)
    if workspace is None:
        workspace = _workspace(max(need, 256), qI.device)
    if idx is None:
        idx = torch.empty((b, n_q, k), dtype=torch.int32, device=qI.device)
    sc = torch.empty((b, n_q, k), dtype=torch.float32, device=qI.device) if score else None
    rc = lib.csa_index_topk_mxfp4(_ptr(qI), _ptr(qI_scale), _f32c(w, "w"), _ptr(KIcomp), _ptr(KI_scale),
                                  KIcomp.shape[1], b, n_q, t0, n_comp, nh, cI, m, k, _ptr(idx), _ptr(sc),
                                  _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "csa_index_topk_mxfp4")
    return (idx, sc) if score else idx


def csa_quantize_mxfp4(x, codes=None, scales=None, stream=None):
    """OCP MXFP4 encoding of x [..., c] (float32 or bf16, c a multiple of 32)
    along its last dimension.  Returns (codes [..., c/2], scales [..., c/32])
    uint8; given output tensors (any leading shape, rows flattened) are
    filled in place."""
    c = x.shape[-1]
    rows = x.numel() // c
    if codes is None:
        codes = torch.empty((*x.shape[:-1], c // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((*x.shape[:-1], c // 32), dtype=torch.uint8, device=x.device)
    lib = load_library()
    rc = lib.csa_quantize_mxfp4(_ptr(x), c, rows, c, _dtype(x, x), _ptr(codes), c // 2, _ptr(scales), c // 32,
                                _stream(stream))
    _check(rc, "csa_quantize_mxfp4")
    return codes, scales


def csa_norm_rope(x, gamma=None, eps=1e-6, rope_dims=64, base=10000.0, pos0=0, pos_step=1, out=None,
                  stream=None):
    """RMSNorm (gamma [c] float32, or None for none) and rotary embedding of
    the last rope_dims dimensions of every vector of x [rows, c] or
    [rows, heads, c]; row r at position pos0 + r * pos_step.  Returns out
    (x itself when out is x: in place)."""
    c = x.shape[-1]
    rows = x.shape[0] if x.dim() > 1 else 1
    heads = x.numel() // (rows * c) if x.numel() else 1
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    lib = load_library()
    g = None if gamma is None else _f32c(gamma, "gamma")
    rc = lib.csa_norm_rope(_ptr(x), heads * c, _ptr(out), heads * c, g, float(eps), rows, heads, c,
                           int(rope_dims), float(base), int(pos0), int(pos_step), _dtype(x, out), _stream(stream))
    _check(rc, "csa_norm_rope")
    return out


def csa_grouped_out_proj(o, WG, WO, mid=None, out=None, stream=None):
    """Grouped output projection: o [n, n_h, c]; WG [g, d_g, (n_h/g)*c];
    WO [d, g*d_g], all bf16.  Returns (mid [n, g*d_g], out [n, d])."""
    n, n_h, c = o.shape
    g, d_g, _ = WG.shape
    d = WO.shape[0]
    if mid is None:
        mid = torch.empty((n, g * d_g), dtype=o.dtype, device=o.device)
    if out is None:
        out = torch.empty((n, d), dtype=o.dtype, device=o.device)
    if WG.shape[2] * g != n_h * c or WO.shape[1] != g * d_g:
        raise ValueError("weight shapes do not match o")
    lib = load_library()
    rc = lib.csa_grouped_out_proj(_ptr(o), _ptr(WG), _ptr(WO), n, n_h, c, g, d_g, d, _dtype(o, WG, WO, mid, out),
                                  _ptr(mid), _ptr(out), _stream(stream))
    _check(rc, "csa_grouped_out_proj")
    return mid, out


def csa_attend(q, Ccomp, idx, kv_raw, sink, t0, m, n_win, scale=None, raw_pos0=0,
               n_comp=None, n_raw=None, out=None, workspace=None, stream=None):
    """CSA main attention.  q [b, n_q, n_h, c]; Ccomp [b, cap, c]; idx
    [b, n_q, k] int32; kv_raw [b, rows, c] (row j at position raw_pos0+j);
    sink [n_h] f32.  Returns out [b, n_q, n_h, c]."""
    q, Ccomp, idx, kv_raw = _batched(q, 4), _batched(Ccomp, 3), _batched(idx, 3), _batched(kv_raw, 3)
    b, n_q, n_h, c = q.shape
    k = idx.shape[2]
    n_comp = Ccomp.shape[1] if n_comp is None else n_comp
    n_raw = kv_raw.shape[1] if n_raw is None else n_raw
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    dt = _dtype(q, Ccomp, kv_raw)
    if idx.dtype != torch.int32:
        raise ValueError("idx must be int32")
    lib = load_library()
    need = lib.csa_attend_workspace_size(b, n_q, t0, n_comp, n_h, c, k, m, n_win, dt)
    if workspace is None:
        workspace = _workspace(need, q.device)
    if out is None:
        out = torch.empty_like(q)
    rc = lib.csa_attend(_ptr(q), _ptr(Ccomp), Ccomp.stride(0), _ptr(idx), _ptr(kv_raw),
                        kv_raw.stride(0), raw_pos0, _f32c(sink, "sink"), b, n_q, t0, n_comp, n_raw,
                        n_h, c, k, m, n_win, scale, dt, _ptr(workspace),
                        0 if workspace is None else workspace.numel(), _ptr(out), _stream(stream))
    _check(rc, "csa_attend")
    return out


def csa_attend_norm_rope(q, gamma_q, eps, rope_dims, base, Ccomp, idx, kv_raw, sink, t0, m, n_win,
                         scale=None, raw_pos0=0, n_comp=None, n_raw=None, out=None, workspace=None,
                         stream=None):
    """csa_attend on raw query heads: each head is RMS-normalised with gain
    gamma_q [c] f32 and its last rope_dims dimensions rotated at its position
    inside the kernel; the output's last rope_dims dimensions are turned back
    by -t before they are stored.  Other arguments as csa_attend."""
    q, Ccomp, idx, kv_raw = _batched(q, 4), _batched(Ccomp, 3), _batched(idx, 3), _batched(kv_raw, 3)
    b, n_q, n_h, c = q.shape
    k = idx.shape[2]
    n_comp = Ccomp.shape[1] if n_comp is None else n_comp
    n_raw = kv_raw.shape[1] if n_raw is None else n_raw
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    dt = _dtype(q, Ccomp, kv_raw)
    if idx.dtype != torch.int32:
        raise ValueError("idx must be int32")
    lib = load_library()
    need = lib.csa_attend_workspace_size(b, n_q, t0, n_comp, n_h, c, k, m, n_win, dt)
    if workspace is None:
        workspace = _workspace(need, q.device)
    if out is None:
        out = torch.empty_like(q)
    rc = lib.csa_attend_norm_rope(_ptr(q), _f32c(gamma_q, "gamma_q"), eps, rope_dims, base, _ptr(Ccomp),
                                  Ccomp.stride(0), _ptr(idx), _ptr(kv_raw), kv_raw.stride(0), raw_pos0,
                                  _f32c(sink, "sink"), b, n_q, t0, n_comp, n_raw, n_h, c, k, m, n_win, scale,
                                  dt, _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                  _ptr(out), _stream(stream))
    _check(rc, "csa_attend_norm_rope")
    return out


def hca_attend_norm_rope(q, gamma_q, eps, rope_dims, base, Ccomp, kv_raw, sink, t0, m_prime, n_win, scale=None,
                         raw_pos0=0, n_comp=None, n_raw=None, out=None, workspace=None, stream=None):
    """hca_attend on raw query heads, normalised (gain gamma_q [c] f32) and
    rotated on their last rope_dims dimensions inside the kernel; the
    output's rotated dimensions turned back by -t.  Other arguments as
    hca_attend."""
    q, Ccomp, kv_raw = _batched(q, 4), _batched(Ccomp, 3), _batched(kv_raw, 3)
    b, n_q, n_h, c = q.shape
    n_comp = Ccomp.shape[1] if n_comp is None else n_comp
    n_raw = kv_raw.shape[1] if n_raw is None else n_raw
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    dt = _dtype(q, Ccomp, kv_raw)
    lib = load_library()
    need = lib.hca_attend_workspace_size(b, n_q, t0, n_comp, n_h, c, m_prime, n_win, dt)
    if workspace is None:
        workspace = _workspace(need, q.device)
    if out is None:
        out = torch.empty_like(q)
    rc = lib.hca_attend_norm_rope(_ptr(q), _f32c(gamma_q, "gamma_q"), eps, rope_dims, base, _ptr(Ccomp),
                                  Ccomp.stride(0), _ptr(kv_raw), kv_raw.stride(0), raw_pos0, _f32c(sink, "sink"), b,
                                  n_q, t0, n_comp, n_raw, n_h, c, m_prime, n_win, scale, dt, _ptr(workspace),
                                  0 if workspace is None else workspace.numel(), _ptr(out), _stream(stream))
    _check(rc, "hca_attend_norm_rope")
    return out


def hca_attend(q, Ccomp, kv_raw, sink, t0, m_prime, n_win, scale=None, raw_pos0=0,
               n_comp=None, n_raw=None, out=None, workspace=None, stream=None):
    """HCA dense attention over every completed entry plus the window."""
    q, Ccomp, kv_raw = _batched(q, 4), _batched(Ccomp, 3), _batched(kv_raw, 3)
    b, n_q, n_h, c = q.shape
    n_comp = Ccomp.shape[1] if n_comp is None else n_comp
    n_raw = kv_raw.shape[1] if n_raw is None else n_raw
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    dt = _dtype(q, Ccomp, kv_raw)
    lib = load_library()
    need = lib.hca_attend_workspace_size(b, n_q, t0, n_comp, n_h, c, m_prime, n_win, dt)
    if workspace is None:
        workspace = _workspace(need, q.device)
    if out is None:
        out = torch.empty_like(q)
    rc = lib.hca_attend(_ptr(q), _ptr(Ccomp), Ccomp.stride(0), _ptr(kv_raw), kv_raw.stride(0),
                        raw_pos0, _f32c(sink, "sink"), b, n_q, t0, n_comp, n_raw, n_h, c, m_prime,
                        n_win, scale, dt, _ptr(workspace),
                        0 if workspace is None else workspace.numel(), _ptr(out), _stream(stream))
    _check(rc, "hca_attend")
    return out


def hca_layer(C, Z, B, q, kv_raw, sink, m_prime, n_win, scale=None, Ccomp=None, out=None,
              workspace=None, stream=None):
    """Whole HCA prefill: pooling compressor then dense attention for every
    position.  C, Z, kv_raw [b, n, c]; q [b, n, n_h, c]; returns (Ccomp, out)."""
    C, Z, q, kv_raw = _batched(C, 3), _batched(Z, 3), _batched(q, 4), _batched(kv_raw, 3)
    b, n, c = C.shape
    n_h = q.shape[2]
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    dt = _dtype(C, Z, B, q, kv_raw)
    lib = load_library()
    need = lib.hca_layer_workspace_size(b, n, n_h, c, m_prime, n_win, dt)
    if workspace is None:
        workspace = _workspace(need, q.device)
    if Ccomp is None:
        Ccomp = torch.empty((b, n // m_prime, c), dtype=C.dtype, device=C.device)
    if out is None:
        out = torch.empty_like(q)
    rc = lib.hca_layer(_ptr(C), _ptr(Z), _ptr(B), _ptr(q), _ptr(kv_raw), _f32c(sink, "sink"), b, n,
                       c, m_prime, n_h, n_win, scale, dt, _ptr(Ccomp), _ptr(workspace),
                       0 if workspace is None else workspace.numel(), _ptr(out), _stream(stream))
    _check(rc, "hca_layer")
    return Ccomp, out


# ----------------------------------------------- heterogeneous decode cache --

class BlockPool:
    """The library's host-side block allocator (csa_block_pool_*)."""

    def __init__(self, n_blocks):
        self._lib = load_library()
        self._p = self._lib.csa_block_pool_create(int(n_blocks))
        if not self._p:
            raise CsaError(-1, "csa_block_pool_create")

    def alloc(self, n):
        ids = (ctypes.c_int32 * max(1, n))()
        _check(self._lib.csa_block_pool_alloc(self._p, n, ids), "csa_block_pool_alloc")
        return list(ids)[:n]

    def release(self, ids):
        arr = (ctypes.c_int32 * max(1, len(ids)))(*ids)
        _check(self._lib.csa_block_pool_release(self._p, len(ids), arr), "csa_block_pool_release")

    def available(self):
        return self._lib.csa_block_pool_available(self._p)

    def close(self):
        if self._p:
            self._lib.csa_block_pool_destroy(self._p)
            self._p = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PagedCache:
    """Device arrays of the heterogeneous decode cache: the block pool array
    and one state per request slot (their layouts are the library's).
    Argument marshalling only; the caller fills `table` [slots, bt_stride]
    int32 from a BlockPool."""

    def __init__(self, n_blocks, slots, bt_stride, c=512, c_I=128, m=4, m_prime=128, n_win=128,
                 device="cuda"):
        lib = load_library()
        self.c, self.c_I, self.m, self.m_prime, self.n_win = c, c_I, m, m_prime, n_win
        self.block_bytes = lib.csa_paged_block_bytes(c, c_I, m, m_prime)
        self.state_bytes = lib.csa_paged_state_bytes(c, c_I, m, m_prime, n_win)
        if not self.block_bytes or not self.state_bytes:
            raise CsaError(-2, "paged cache geometry")
        self.n_blocks, self.slots, self.bt_stride = n_blocks, slots, bt_stride
        self.blocks = torch.empty(n_blocks * self.block_bytes // 2, dtype=torch.bfloat16, device=device)
        self.state = torch.empty(slots * self.state_bytes // 2, dtype=torch.bfloat16, device=device)
        self.table = torch.zeros((slots, bt_stride), dtype=torch.int32, device=device)


def csa_paged_append(cache, pos, tok, biases, req_slot=None, stream=None):
    """tok: dict of [b, c] / [b, c_I] bf16 rows Ca, Cb, Za, Zb, ICa, ICb, IZa,
    IZb, C_h, Z_h; biases: Ba, Bb [m, c], IBa, IBb [m, c_I], B_h [m', c];
    pos [b] int64 (positions of the tokens)."""
    if pos.dtype != torch.int64:
        raise ValueError("pos must be int64")
    if req_slot is not None and req_slot.dtype != torch.int32:
        raise ValueError("req_slot must be int32")
    b = pos.shape[0]
    lib = load_library()
    rc = lib.csa_paged_append(_ptr(cache.state), _ptr(cache.blocks), cache.n_blocks, _ptr(cache.table),
                              cache.bt_stride, _ptr(req_slot), _ptr(pos), b,
                              *(_ptr(tok[x]) for x in ("Ca", "Cb", "Za", "Zb", "ICa", "ICb", "IZa", "IZb", "C_h", "Z_h")),
                              *(_ptr(biases[x]) for x in ("Ba", "Bb", "IBa", "IBb", "B_h")),
                              cache.c, cache.c_I, cache.m, cache.m_prime, cache.n_win, CSA_BF16, _stream(stream))
    _check(rc, "csa_paged_append")


def csa_paged_index_topk(cache, qI, w, pos, n_comp_max, k, req_slot=None, score=False, idx=None, workspace=None,
                         stream=None):
    """qI [b, n_hI, c_I] bf16, w [b, n_hI] f32; returns idx [b, k] int32
    (entry numbers) and the scores when score=True."""
    b, nh, cI = qI.shape
    lib = load_library()
    need = lib.csa_index_topk_workspace_size(b, 1, n_comp_max, k)
    if workspace is None:
        workspace = _workspace(max(need, 256), qI.device)
    if idx is None:
        idx = torch.empty((b, k), dtype=torch.int32, device=qI.device)
    sc = torch.empty((b, k), dtype=torch.float32, device=qI.device) if score else None
    rc = lib.csa_paged_index_topk(_ptr(qI), _f32c(w, "w"), _ptr(cache.blocks), cache.n_blocks, _ptr(cache.table),
                                  cache.bt_stride, _ptr(req_slot), _ptr(pos), b, n_comp_max, nh, cI, cache.c,
                                  cache.m, cache.m_prime, k, _dtype(qI, qI), _ptr(idx), _ptr(sc), _ptr(workspace),
                                  workspace.numel(), _stream(stream))
    _check(rc, "csa_paged_index_topk")
    return (idx, sc) if score else idx


def csa_paged_attend(cache, q, idx, sink, pos, n_comp_max, scale=None, req_slot=None, out=None, workspace=None,
                     stream=None):
    """q [b, n_h, c] bf16, idx [b, k] int32; returns out [b, n_h, c]."""
    b, n_h, c = q.shape
    k = idx.shape[1]
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    lib = load_library()
    need = lib.csa_paged_attend_workspace_size(b, n_h, k, cache.n_win)
    if workspace is None:
        workspace = _workspace(need, q.device)
    if out is None:
        out = torch.empty_like(q)
    rc = lib.csa_paged_attend(_ptr(q), _ptr(cache.blocks), cache.n_blocks, _ptr(cache.table), cache.bt_stride,
                              _ptr(req_slot), _ptr(pos), _ptr(idx), _ptr(cache.state), _f32c(sink, "sink"), b,
                              n_comp_max, n_h, c, cache.c_I, k, cache.m, cache.m_prime, cache.n_win, scale,
                              _dtype(q, q), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                              _ptr(out), _stream(stream))
    _check(rc, "csa_paged_attend")
    return out


def hca_paged_attend(cache, q, sink, pos, n_hca_max, scale=None, req_slot=None, out=None, workspace=None,
                     stream=None):
    """q [b, n_h, c] bf16; returns out [b, n_h, c]."""
    b, n_h, c = q.shape
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    lib = load_library()
    need = lib.hca_paged_attend_workspace_size(b, n_h, n_hca_max, cache.n_win)
    if workspace is None:
        workspace = _workspace(need, q.device)
    if out is None:
        out = torch.empty_like(q)
    rc = lib.hca_paged_attend(_ptr(q), _ptr(cache.blocks), cache.n_blocks, _ptr(cache.table), cache.bt_stride,
                              _ptr(req_slot), _ptr(pos), _ptr(cache.state), _f32c(sink, "sink"), b, n_hca_max, n_h,
                              c, cache.c_I, cache.m, cache.m_prime, cache.n_win, scale, _dtype(q, q),
                              _ptr(workspace), 0 if workspace is None else workspace.numel(), _ptr(out),
                              _stream(stream))
    _check(rc, "hca_paged_attend")
    return out


# ------------------------------------------------------------ backward pass --

def csa_attend_backward(q, Ccomp, idx, kv_raw, sink, dout, t0, m, n_win, scale=None, raw_pos0=0, n_comp=None,
                        n_raw=None, accumulate=False, grads=None, workspace=None, stream=None):
    """Gradients of csa_attend: returns (dq, dCcomp, dkv_raw, dsink), float32,
    shaped like q, Ccomp, kv_raw and sink.  `grads` (that tuple) receives
    them in place; with accumulate=True the last three are added to."""
    q, Ccomp, idx, kv_raw, dout = (_batched(q, 4), _batched(Ccomp, 3), _batched(idx, 3), _batched(kv_raw, 3),
                                   _batched(dout, 4))
    return _attend_backward(False, q, Ccomp, idx, kv_raw, sink, dout, t0, m, n_win, scale, raw_pos0, n_comp, n_raw,
                            accumulate, grads, workspace, stream)


def hca_attend_backward(q, Ccomp, kv_raw, sink, dout, t0, m_prime, n_win, scale=None, raw_pos0=0, n_comp=None,
                        n_raw=None, accumulate=False, grads=None, workspace=None, stream=None):
    """Gradients of hca_attend (see csa_attend_backward)."""
    q, Ccomp, kv_raw, dout = _batched(q, 4), _batched(Ccomp, 3), _batched(kv_raw, 3), _batched(dout, 4)
    return _attend_backward(True, q, Ccomp, None, kv_raw, sink, dout, t0, m_prime, n_win, scale, raw_pos0, n_comp,
                            n_raw, accumulate, grads, workspace, stream)


def _attend_backward(dense, q, Ccomp, idx, kv_raw, sink, dout, t0, m, n_win, scale, raw_pos0, n_comp, n_raw,
                     accumulate, grads, workspace, stream):
    b, n_q, n_h, c = q.shape
    n_comp = Ccomp.shape[1] if n_comp is None else n_comp
    n_raw = kv_raw.shape[1] if n_raw is None else n_raw
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    dt = _dtype(q, Ccomp, kv_raw, dout)
    lib = load_library()
    k = 0 if dense else idx.shape[2]
    need = (lib.hca_attend_backward_workspace_size(b, n_q, n_h, c, n_comp, n_win) if dense
            else lib.csa_attend_backward_workspace_size(b, n_q, n_h, c, k, n_win))
    if workspace is None:
        workspace = _workspace(max(need, 256), q.device)
    if grads is None:
        f = dict(dtype=torch.float32, device=q.device)
        grads = (torch.empty(q.shape, **f), torch.zeros(Ccomp.shape, **f), torch.zeros(kv_raw.shape, **f),
                 torch.zeros(n_h, **f))
    dq, dC, dR, ds = grads
    for t_ in grads:
        if t_.dtype != torch.float32:
            raise ValueError("gradients are float32")
    dC3, dR3 = _batched(dC, 3), _batched(dR, 3)
    if dense:
        rc = lib.hca_attend_backward(_ptr(q), _ptr(Ccomp), Ccomp.stride(0), _ptr(kv_raw), kv_raw.stride(0), raw_pos0,
                                     _f32c(sink, "sink"), _ptr(dout), b, n_q, t0, n_comp, n_raw, n_h, c, m, n_win,
                                     scale, dt, int(accumulate), _ptr(dq), _ptr(dC3), dC3.stride(0), _ptr(dR3),
                                     dR3.stride(0), _ptr(ds), _ptr(workspace), workspace.numel(), _stream(stream))
    else:
        if idx.dtype != torch.int32:
            raise ValueError("idx must be int32")
        rc = lib.csa_attend_backward(_ptr(q), _ptr(Ccomp), Ccomp.stride(0), _ptr(idx), _ptr(kv_raw), kv_raw.stride(0),
                                     raw_pos0, _f32c(sink, "sink"), _ptr(dout), b, n_q, t0, n_comp, n_raw, n_h, c, k,
                                     m, n_win, scale, dt, int(accumulate), _ptr(dq), _ptr(dC3), dC3.stride(0),
                                     _ptr(dR3), dR3.stride(0), _ptr(ds), _ptr(workspace), workspace.numel(),
                                     _stream(stream))
    _check(rc, "hca_attend_backward" if dense else "csa_attend_backward")
    return grads


def csa_compress_backward(Ca, Cb, Za, Zb, Ba, Bb, m, dCcomp, prev_Cb=None, prev_Zb=None, overlap=True,
                          workspace=None, stream=None):
    """Gradients of csa_compress: dict of float32 tensors dCa, dZa, dBa (and
    dCb, dZb, dBb, plus dprev_Cb, dprev_Zb when the state is given)."""
    Ca, Cb, Za, Zb = (_batched(x, 3) for x in (Ca, Cb, Za, Zb))
    prev_Cb, prev_Zb = _batched(prev_Cb, 3), _batched(prev_Zb, 3)
    dCcomp = _batched(dCcomp, 3)
    b, n, c = Ca.shape
    dt = _dtype(Ca, Cb, Za, Zb, Ba, Bb, prev_Cb, prev_Zb)
    f = dict(dtype=torch.float32, device=Ca.device)
    g = {"dCa": torch.empty((b, n, c), **f), "dZa": torch.empty((b, n, c), **f), "dBa": torch.empty((m, c), **f)}
    if overlap:
        g.update({"dCb": torch.empty((b, n, c), **f), "dZb": torch.empty((b, n, c), **f),
                  "dBb": torch.empty((m, c), **f)})
        if prev_Cb is not None:
            g.update({"dprev_Cb": torch.empty((b, m, c), **f), "dprev_Zb": torch.empty((b, m, c), **f)})
    lib = load_library()
    need = lib.csa_compress_backward_workspace_size(n, c, m)
    if workspace is None:
        workspace = _workspace(max(need, 256), Ca.device)
    rc = lib.csa_compress_backward(_ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), _ptr(Ba), _ptr(Bb), _ptr(prev_Cb),
                                   _ptr(prev_Zb), _f32c(dCcomp, "dCcomp"), b, n, c, m, 1 if overlap else 0, dt,
                                   *(_ptr(g.get(x)) for x in ("dCa", "dCb", "dZa", "dZb", "dBa", "dBb", "dprev_Cb",
                                                              "dprev_Zb")),
                                   _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "csa_compress_backward")
    return g


# --------------------------------------------------------- FP8 KV entries --

def csa_quantize_kv_fp8(x, rope_dims=64, stream=None):
    """Encode entries x [..., c] (float32 or bf16): returns (codes [..., c - r]
    uint8, rope [..., r] bf16, scale [...] float32)."""
    c = x.shape[-1]
    rows = x.numel() // c
    lead = x.shape[:-1]
    codes = torch.empty((*lead, c - rope_dims), dtype=torch.uint8, device=x.device)
    rope = torch.empty((*lead, rope_dims), dtype=torch.bfloat16, device=x.device)
    scale = torch.empty(lead, dtype=torch.float32, device=x.device)
    lib = load_library()
    rc = lib.csa_quantize_kv_fp8(_ptr(x), c, rows, c, rope_dims, _dtype(x, x), _ptr(codes), c - rope_dims, _ptr(rope),
                                 rope_dims, _ptr(scale), _stream(stream))
    _check(rc, "csa_quantize_kv_fp8")
    return codes, rope, scale


def csa_attend_fp8kv(q, codes, rope, scale, idx, kv_raw, sink, t0, m, n_win, sm_scale=None, raw_pos0=0, n_comp=None,
                     n_raw=None, out=None, workspace=None, stream=None):
    """csa_attend over FP8-stored entries (codes [b, cap, c - r], rope
    [b, cap, r], scale [b, cap])."""
    q, idx, kv_raw = _batched(q, 4), _batched(idx, 3), _batched(kv_raw, 3)
    codes, rope = _batched(codes, 3), _batched(rope, 3)
    scale = scale if scale.dim() == 2 else scale.unsqueeze(0)
    b, n_q, n_h, c = q.shape
    k = idx.shape[2]
    r = rope.shape[2]
    n_comp = codes.shape[1] if n_comp is None else n_comp
    n_raw = kv_raw.shape[1] if n_raw is None else n_raw
    sm_scale = 1.0 / math.sqrt(c) if sm_scale is None else sm_scale
    if idx.dtype != torch.int32 or codes.dtype != torch.uint8 or scale.dtype != torch.float32:
        raise ValueError("idx int32, codes uint8, scale float32")
    lib = load_library()
    need = lib.csa_attend_fp8kv_workspace_size(b, n_q, t0, n_comp, n_h, c, k, m, n_win)
    if workspace is None:
        workspace = _workspace(max(need, 256), q.device)
    if out is None:
        out = torch.empty_like(q)
    rc = lib.csa_attend_fp8kv(_ptr(q), _ptr(codes), _ptr(rope), _ptr(scale), codes.shape[1], _ptr(idx), _ptr(kv_raw),
                              kv_raw.stride(0), raw_pos0, _f32c(sink, "sink"), b, n_q, t0, n_comp, n_raw, n_h, c, r, k,
                              m, n_win, sm_scale, _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream))
    _check(rc, "csa_attend_fp8kv")
    return out
