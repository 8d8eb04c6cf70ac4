"""fp64 CPU oracle for the multi-scale deformable attention core.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code with
the HIP library. Inputs (numpy arrays or CPU torch tensors, fp32 / bf16 / fp64)
are upcast exactly to float64; every result is float64 numpy.

The C code in ``msda_oracle.c`` cites the passages of the pages each function
follows. Pins for every function live in ``tests/test_oracle_*.py``.
"""
import contextlib
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    src_m = os.path.getmtime(_build.SRC)
    if not os.path.exists(path) or os.path.getmtime(path) < src_m:
        _build.build()
    _lib = _bind(ctypes.CDLL(path))
    return _lib


@contextlib.contextmanager
def swapped_library(path):
    """Run the oracle functions against another build of the oracle source
    (used by the mutation tests, which plant mistakes in a copy)."""
    global _lib
    saved = _load()
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _bind(lib):
    lib.msda_oracle_set_threads.restype = None
    lib.msda_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.msda_oracle_level_start_index.restype = ctypes.c_int64
    lib.msda_oracle_level_start_index.argtypes = [ctypes.c_int, _i64p, _i64p]
    lib.msda_oracle_reference_points_encoder.restype = None
    lib.msda_oracle_reference_points_encoder.argtypes = [ctypes.c_int, ctypes.c_int, _i64p, _f64p, _f64p]
    lib.msda_oracle_reference_points_decoder.restype = None
    lib.msda_oracle_reference_points_decoder.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, _f64p, _f64p, _f64p]
    lib.msda_oracle_sampling_locations.restype = None
    lib.msda_oracle_sampling_locations.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_int, _i64p, _f64p, _f64p, _f64p]
    lib.msda_oracle_softmax.restype = None
    lib.msda_oracle_softmax.argtypes = [ctypes.c_int64, ctypes.c_int, _f64p, _f64p]
    lib.msda_oracle_masked_fill.restype = None
    lib.msda_oracle_masked_fill.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.POINTER(ctypes.c_ubyte), _f64p, _f64p]
    lib.msda_oracle_softmax_backward.restype = None
    lib.msda_oracle_softmax_backward.argtypes = [ctypes.c_int64, ctypes.c_int, _f64p, _f64p, _f64p]
    lib.msda_oracle_sampling_locations_backward.restype = None
    lib.msda_oracle_sampling_locations_backward.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                            ctypes.c_int, _i64p, _f64p, _f64p, _f64p]
    lib.msda_oracle_sampling_locations_box.restype = None
    lib.msda_oracle_sampling_locations_box.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                       ctypes.c_int, _f64p, _f64p, _f64p]
    lib.msda_oracle_sampling_locations_box_backward.restype = None
    lib.msda_oracle_sampling_locations_box_backward.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                                                ctypes.c_int, ctypes.c_int, _f64p, _f64p, _f64p,
                                                                _f64p, _f64p]
    lib.msda_oracle_forward.restype = None
    lib.msda_oracle_forward.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, _i64p, _i64p, _f64p, _f64p, _f64p,
                                        _i64p, ctypes.c_int64, _f64p]
    lib.msda_oracle_backward.restype = None
    lib.msda_oracle_backward.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, _i64p, _i64p, _f64p, _f64p, _f64p, _f64p,
                                         _f64p, _f64p, _f64p]
    return lib


@contextlib.contextmanager
def threads(n):
    """Run the forward and backward on n host threads inside the block
    (results are bit-identical to one thread's: each output element is
    computed by one thread in the serial order)."""
    lib = _load()
    lib.msda_oracle_set_threads(int(n))
    try:
        yield
    finally:
        lib.msda_oracle_set_threads(1)


def _f64(x):
    """Exact upcast to a contiguous float64 numpy array (bf16 via torch)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().cpu().to(torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _p(a, t):
    return a.ctypes.data_as(t)


def level_start_index(spatial_shapes):
    """Exclusive prefix sum of H_l*W_l; returns (lsi [L] int64, S)."""
    shapes = _i64(spatial_shapes).reshape(-1, 2)
    L = shapes.shape[0]
    lsi = np.zeros(L, dtype=np.int64)
    S = _load().msda_oracle_level_start_index(L, _p(shapes, _i64p), _p(lsi, _i64p))
    return lsi, int(S)


def reference_points_encoder(spatial_shapes, valid_ratios):
    """[B,S,L,2] reference points, every pixel of every level a query."""
    shapes = _i64(spatial_shapes).reshape(-1, 2)
    vr = _f64(valid_ratios)
    B, L, _ = vr.shape
    assert L == shapes.shape[0]
    S = int((shapes[:, 0] * shapes[:, 1]).sum())
    out = np.empty((B, S, L, 2), dtype=np.float64)
    _load().msda_oracle_reference_points_encoder(B, L, _p(shapes, _i64p), _p(vr, _f64p), _p(out, _f64p))
    return out


def reference_points_decoder(u, valid_ratios):
    """[B,Nq,L,2] = u[b,q,None,:] * valid_ratios[b,None,l,:]."""
    u = _f64(u)
    vr = _f64(valid_ratios)
    B, Nq, _ = u.shape
    L = vr.shape[1]
    out = np.empty((B, Nq, L, 2), dtype=np.float64)
    _load().msda_oracle_reference_points_decoder(B, Nq, L, _p(u, _f64p), _p(vr, _f64p), _p(out, _f64p))
    return out


def sampling_locations(spatial_shapes, ref, offset_px):
    """loc = ref + offset_px / (W_l, H_l); ref [B,Nq,L,2], offsets [B,Nq,M,L,K,2]."""
    shapes = _i64(spatial_shapes).reshape(-1, 2)
    ref = _f64(ref)
    off = _f64(offset_px)
    B, Nq, M, L, K, _ = off.shape
    assert ref.shape == (B, Nq, L, 2)
    out = np.empty_like(off)
    _load().msda_oracle_sampling_locations(B, Nq, M, L, K, _p(shapes, _i64p), _p(ref, _f64p),
                                           _p(off, _f64p), _p(out, _f64p))
    return out


def softmax(logits, n):
    """Softmax over trailing groups of n entries (n = L*K)."""
    x = _f64(logits)
    shape = x.shape
    flat = x.reshape(-1, n)
    out = np.empty_like(flat)
    _load().msda_oracle_softmax(flat.shape[0], n, _p(flat, _f64p), _p(out, _f64p))
    return out.reshape(shape)


def masked_fill(x, key_padding_mask):
    """x [B,S,...] with the rows of the padded positions (mask [B,S] nonzero)
    set to zero: the module's masked_fill of the value before the core, and
    the backward of that step for a gradient of the same shape."""
    v = _f64(x)
    try:
        import torch
        if isinstance(key_padding_mask, torch.Tensor):
            key_padding_mask = key_padding_mask.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    mask = np.ascontiguousarray(np.asarray(key_padding_mask).astype(np.uint8))
    B, S = v.shape[:2]
    assert mask.shape == (B, S)
    C = int(np.prod(v.shape[2:])) if v.ndim > 2 else 1
    out = np.empty_like(v)
    _load().msda_oracle_masked_fill(B, S, C, mask.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)),
                                    _p(v, _f64p), _p(out, _f64p))
    return out


def softmax_backward(attn, grad_attn, n):
    """grad_logits for A = softmax(logits) over trailing groups of n entries."""
    a = _f64(attn)
    g = _f64(grad_attn)
    assert a.shape == g.shape
    fa, fg = a.reshape(-1, n), g.reshape(-1, n)
    out = np.empty_like(fa)
    _load().msda_oracle_softmax_backward(fa.shape[0], n, _p(fa, _f64p), _p(fg, _f64p), _p(out, _f64p))
    return out.reshape(a.shape)


def sampling_locations_backward(spatial_shapes, grad_loc):
    """(grad_ref [B,Nq,L,2], grad_offset_px [B,Nq,M,L,K,2]) of loc = ref + offset_px / (W_l, H_l)."""
    shapes = _i64(spatial_shapes).reshape(-1, 2)
    gl = _f64(grad_loc)
    B, Nq, M, L, K, _ = gl.shape
    gref = np.empty((B, Nq, L, 2), dtype=np.float64)
    goff = np.empty_like(gl)
    _load().msda_oracle_sampling_locations_backward(B, Nq, M, L, K, _p(shapes, _i64p), _p(gl, _f64p),
                                                    _p(gref, _f64p), _p(goff, _f64p))
    return gref, goff


def sampling_locations_box(ref, offset):
    """loc = ref[..., :2] + offset / K * ref[..., 2:] * 0.5; ref [B,Nq,L,4], offsets [B,Nq,M,L,K,2]."""
    ref = _f64(ref)
    off = _f64(offset)
    B, Nq, M, L, K, _ = off.shape
    assert ref.shape == (B, Nq, L, 4)
    out = np.empty_like(off)
    _load().msda_oracle_sampling_locations_box(B, Nq, M, L, K, _p(ref, _f64p), _p(off, _f64p), _p(out, _f64p))
    return out


def sampling_locations_box_backward(ref, offset, grad_loc):
    """(grad_ref [B,Nq,L,4], grad_offset [B,Nq,M,L,K,2]) of sampling_locations_box."""
    ref = _f64(ref)
    off = _f64(offset)
    gl = _f64(grad_loc)
    B, Nq, M, L, K, _ = off.shape
    gref = np.empty((B, Nq, L, 4), dtype=np.float64)
    goff = np.empty_like(off)
    _load().msda_oracle_sampling_locations_box_backward(B, Nq, M, L, K, _p(ref, _f64p), _p(off, _f64p),
                                                        _p(gl, _f64p), _p(gref, _f64p), _p(goff, _f64p))
    return gref, goff


def forward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
            query_ids=None):
    """Core forward: out [B,Nq,M*D] (or [len(query_ids), M*D] for a subset)."""
    shapes = _i64(spatial_shapes).reshape(-1, 2)
    lsi = _i64(level_start_index)
    v = _f64(value)
    loc = _f64(sampling_locations)
    A = _f64(attention_weights)
    B, S, M, D = v.shape
    _, Nq, _, L, K, _ = loc.shape
    assert A.shape == (B, Nq, M, L, K)
    if query_ids is not None:
        ids = _i64(query_ids).reshape(-1)
        out = np.empty((ids.shape[0], M * D), dtype=np.float64)
        idp, nid = _p(ids, _i64p), ids.shape[0]
    else:
        out = np.empty((B, Nq, M * D), dtype=np.float64)
        idp, nid = None, 0
    _load().msda_oracle_forward(B, S, Nq, M, D, L, K, _p(shapes, _i64p), _p(lsi, _i64p),
                                _p(v, _f64p), _p(loc, _f64p), _p(A, _f64p), idp, nid,
                                _p(out, _f64p))
    return out


def backward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
             grad_output):
    """Core backward: (grad_value [B,S,M,D], grad_loc [B,Nq,M,L,K,2], grad_attn [B,Nq,M,L,K])."""
    shapes = _i64(spatial_shapes).reshape(-1, 2)
    lsi = _i64(level_start_index)
    v = _f64(value)
    loc = _f64(sampling_locations)
    A = _f64(attention_weights)
    G = _f64(grad_output)
    B, S, M, D = v.shape
    _, Nq, _, L, K, _ = loc.shape
    assert G.shape == (B, Nq, M * D)
    gv = np.empty_like(v)
    gl = np.empty_like(loc)
    ga = np.empty_like(A)
    _load().msda_oracle_backward(B, S, Nq, M, D, L, K, _p(shapes, _i64p), _p(lsi, _i64p),
                                 _p(v, _f64p), _p(loc, _f64p), _p(A, _f64p), _p(G, _f64p),
                                 _p(gv, _f64p), _p(gl, _f64p), _p(ga, _f64p))
    return gv, gl, ga
