"""ctypes binding of libmsda.so (the C ABI of include/msda.h).

Argument marshalling only: tensors become device pointers, sizes become an
``msda_shape``, the current HIP stream is passed through, and outputs are
allocated with torch (device memory is PyTorch's plumbing here). Every step of
the computation runs in the HIP kernels of libmsda.so; there is no other path.
If the library is missing or fails to load, every call raises.
"""
import ctypes
import os
import re
import weakref
from typing import Optional, Sequence, Tuple, Union

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsda.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "msda.h")

MSDA_OK = 0
MSDA_E_NULL = -1
MSDA_E_DIM = -2
MSDA_E_SHAPE = -3
MSDA_E_LEVEL_INDEX = -4
MSDA_E_UNSUPPORTED = -5
MSDA_E_ALIGN = -6
MSDA_E_HIP = -7
MSDA_E_WORKSPACE = -8
MSDA_F32 = 0
MSDA_BF16 = 1
MSDA_BWD_ACCUMULATE = 1
MSDA_MAX_LEVELS = 16


class MSDAError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str, call: str):
        super().__init__(f"{call} failed: {name} ({status}): {detail}")
        self.status = status


class msda_shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("channels", ctypes.c_int32),
        ("levels", ctypes.c_int32),
        ("points", ctypes.c_int32),
        ("num_value", ctypes.c_int64),
        ("num_query", ctypes.c_int64),
        ("spatial_shapes", ctypes.POINTER(ctypes.c_int64)),
        ("level_start_index", ctypes.POINTER(ctypes.c_int64)),
    ]


_lib = None
_vp = ctypes.c_void_p
_shp = ctypes.POINTER(msda_shape)
_i64p = ctypes.POINTER(ctypes.c_int64)


def declared_symbols():
    """Names of the entry points include/msda.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"MSDA_API\s+[\w\s\*]*?\b(msda_\w+)\s*\(", text)))


def load():
    """Load libmsda.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libmsda.so not found at {LIB_PATH}; build it with "
            "`python -m scale_deformable_attention_msdeformattn_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.msda_abi_version.restype = ctypes.c_int
    lib.msda_abi_version.argtypes = []
    lib.msda_status_string.restype = ctypes.c_char_p
    lib.msda_status_string.argtypes = [ctypes.c_int]
    lib.msda_last_error.restype = ctypes.c_char_p
    lib.msda_last_error.argtypes = []
    lib.msda_level_start_index.restype = ctypes.c_int
    lib.msda_level_start_index.argtypes = [ctypes.c_int32, _i64p, _i64p, _i64p]
    lib.msda_reference_points.restype = ctypes.c_int
    lib.msda_reference_points.argtypes = [_shp, _vp, _vp, _vp, _vp]
    lib.msda_sampling_locations.restype = ctypes.c_int
    lib.msda_sampling_locations.argtypes = [_shp, _vp, _vp, _vp, _vp]
    lib.msda_attention_softmax.restype = ctypes.c_int
    lib.msda_attention_softmax.argtypes = [_shp, _vp, _vp, _vp]
    lib.msda_prologue.restype = ctypes.c_int
    lib.msda_prologue.argtypes = [_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.msda_forward.restype = ctypes.c_int
    lib.msda_forward.argtypes = [_shp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp]
    lib.msda_backward_workspace_size.restype = ctypes.c_int
    lib.msda_backward_workspace_size.argtypes = [_shp, ctypes.POINTER(ctypes.c_size_t)]
    lib.msda_backward_plan.restype = ctypes.c_int
    lib.msda_backward_plan.argtypes = [_shp] + [ctypes.POINTER(ctypes.c_uint32)] * 3
    lib.msda_backward.restype = ctypes.c_int
    lib.msda_backward.argtypes = [_shp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                  ctypes.c_uint, _vp]
    lib.msda_backward_noalloc.restype = ctypes.c_int
    lib.msda_backward_noalloc.argtypes = [_shp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_uint, _vp]
    lib.msda_forward_fused.restype = ctypes.c_int
    lib.msda_forward_fused.argtypes = [_shp, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp]
    lib.msda_backward_fused.restype = ctypes.c_int
    lib.msda_backward_fused.argtypes = [_shp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp, ctypes.c_size_t, ctypes.c_uint, _vp]
    lib.msda_timing_enable.restype = ctypes.c_int
    lib.msda_timing_enable.argtypes = [ctypes.c_int]
    lib.msda_timing_reset.restype = ctypes.c_int
    lib.msda_timing_reset.argtypes = []
    lib.msda_timing_read.restype = ctypes.c_int
    lib.msda_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_char_p),
                                     ctypes.POINTER(ctypes.c_double), _i64p]
    _lib = lib
    return lib


def _check(status: int, call: str):
    if status != MSDA_OK:
        lib = load()
        raise MSDAError(status, lib.msda_status_string(status).decode(),
                        lib.msda_last_error().decode(), call)


class Shape:
    """Host-side sizes of one call, kept alive while the C call runs."""

    def __init__(self, spatial_shapes, batch, heads, channels, points, num_query,
                 level_start_index=None):
        shapes = _host_i64(spatial_shapes).reshape(-1, 2)
        self.levels = int(shapes.shape[0])
        self._shapes = (ctypes.c_int64 * (2 * self.levels))(*[int(v) for v in shapes.reshape(-1).tolist()])
        if level_start_index is None:
            lsi, S = level_start_index_host(shapes)
        else:
            lsi = [int(v) for v in _host_i64(level_start_index).reshape(-1).tolist()]
            S = int(sum(int(h) * int(w) for h, w in shapes.tolist()))
        self._lsi = (ctypes.c_int64 * max(1, len(lsi)))(*lsi)
        self.c = msda_shape(int(batch), int(heads), int(channels), self.levels, int(points), int(S),
                            int(num_query), ctypes.cast(self._shapes, _i64p), ctypes.cast(self._lsi, _i64p))

    @property
    def ptr(self):
        return ctypes.byref(self.c)


def _host_i64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.int64)
    return torch.as_tensor(x, dtype=torch.int64)


# Host copies of small integer tensors that live on the device (spatial
# shapes, level start indices), so that a call does not wait on the device to
# read them again: keyed by the tensor object, dropped when it is freed, and
# read again when its version counter has moved (any in-place write).
_DEV_INTS = {}


def _ints(x) -> tuple:
    """The values of a small integer array, flattened, as Python ints."""
    if isinstance(x, torch.Tensor) and x.device.type != "cpu":
        key = id(x)
        e = _DEV_INTS.get(key)
        if e is not None and e[0]() is x and e[1] == x._version:
            return e[2]
        vals = tuple(x.detach().to("cpu", torch.int64).reshape(-1).tolist())
        _DEV_INTS[key] = (weakref.ref(x, lambda _r, k=key: _DEV_INTS.pop(k, None)), x._version, vals)
        return vals
    if isinstance(x, tuple) and all(type(v) is int for v in x):
        return x
    return tuple(_host_i64(x).reshape(-1).tolist())


# Shape objects per distinct set of sizes: building one (ctypes arrays, the
# level start index) costs more than the launches of a small call.
_SHAPES = {}
_SHAPES_MAX = 256


def _shape(spatial_shapes, batch, heads, channels, points, num_query, level_start_index=None, num_value=None):
    sv = _ints(spatial_shapes)
    lv = None if level_start_index is None else _ints(level_start_index)
    key = (sv, lv, int(batch), int(heads), int(channels), int(points), int(num_query), num_value)
    sh = _SHAPES.get(key)
    if sh is None:
        sh = Shape(sv, batch, heads, channels, points, num_query, lv)
        if num_value is not None:
            sh.c.num_value = int(num_value)  # the library checks it against sum H_l*W_l
        if len(_SHAPES) >= _SHAPES_MAX:
            _SHAPES.clear()
        _SHAPES[key] = sh
    return sh


def level_start_index_host(spatial_shapes) -> Tuple[list, int]:
    """(level_start_index as a list, S) computed by the library's host helper."""
    shapes = _host_i64(spatial_shapes).reshape(-1, 2)
    L = int(shapes.shape[0])
    arr = (ctypes.c_int64 * (2 * L))(*[int(v) for v in shapes.reshape(-1).tolist()])
    lsi = (ctypes.c_int64 * max(1, L))()
    S = ctypes.c_int64()
    _check(load().msda_level_start_index(L, arr, lsi, ctypes.byref(S)), "msda_level_start_index")
    return [lsi[i] for i in range(L)], S.value


def _dev(t: torch.Tensor, name: str, dtype=torch.float32) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    return t if t.is_contiguous() else t.contiguous()


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# --------------------------------------------------------------------------
# Entry points, same names as the C ABI.
# --------------------------------------------------------------------------

def msda_reference_points(spatial_shapes, valid_ratios: Optional[torch.Tensor] = None,
                          query_ref: Optional[torch.Tensor] = None, batch: Optional[int] = None,
                          device=None) -> torch.Tensor:
    """Reference points [B, Nq, L, 2]. Encoder mode when query_ref is None
    (every pixel of every level is a query, Nq = S); decoder mode with
    query_ref = u [B, Nq, 2]. valid_ratios [B, L, 2] or None (all ones)."""
    sv = _ints(spatial_shapes)
    L = len(sv) // 2
    ref_dev = valid_ratios if valid_ratios is not None else query_ref
    if valid_ratios is not None:
        valid_ratios = _dev(valid_ratios, "valid_ratios")
        B = valid_ratios.shape[0]
        if tuple(valid_ratios.shape) != (B, L, 2):
            raise ValueError(f"valid_ratios must be [B, {L}, 2], got {tuple(valid_ratios.shape)}")
    if query_ref is not None:
        query_ref = _dev(query_ref, "query_ref")
        B, Nq = query_ref.shape[0], query_ref.shape[1]
        if query_ref.dim() != 3 or query_ref.shape[2] != 2:
            raise ValueError("query_ref must be [B, Nq, 2]")
    else:
        B = valid_ratios.shape[0] if valid_ratios is not None else int(batch)
        Nq = sum(sv[2 * i] * sv[2 * i + 1] for i in range(L))
    if valid_ratios is not None and valid_ratios.shape[0] != B:
        raise ValueError("valid_ratios and query_ref disagree on the batch size")
    device = ref_dev.device if ref_dev is not None else torch.device(device or "cuda")
    out = torch.empty(B, Nq, L, 2, dtype=torch.float32, device=device)
    sh = _shape(sv, B, 1, 1, 1, Nq)
    _check(load().msda_reference_points(sh.ptr, _p(valid_ratios), _p(query_ref), _p(out), _stream(out)),
           "msda_reference_points")
    return out


def msda_sampling_locations(spatial_shapes, reference_points: torch.Tensor,
                            offsets_px: torch.Tensor) -> torch.Tensor:
    """loc [B,Nq,M,L,K,2] = ref[B,Nq,L,2] + offsets_px / (W_l, H_l)."""
    ref = _dev(reference_points, "reference_points")
    off = _dev(offsets_px, "offsets_px")
    if off.dim() != 6 or off.shape[-1] != 2:
        raise ValueError("offsets_px must be [B, Nq, M, L, K, 2]")
    B, Nq, M, L, K, _ = off.shape
    if tuple(ref.shape) != (B, Nq, L, 2):
        raise ValueError(f"reference_points must be [{B}, {Nq}, {L}, 2], got {tuple(ref.shape)}")
    out = torch.empty_like(off)
    sh = _shape(spatial_shapes, B, M, 1, K, Nq)
    if sh.levels != L:
        raise ValueError("spatial_shapes and offsets_px disagree on the level count")
    _check(load().msda_sampling_locations(sh.ptr, _p(ref), _p(off), _p(out), _stream(out)),
           "msda_sampling_locations")
    return out


def msda_attention_softmax(spatial_shapes, logits: torch.Tensor, points: int) -> torch.Tensor:
    """Softmax of logits [B,Nq,M,L*K] over L*K -> weights [B,Nq,M,L,K]."""
    x = _dev(logits, "logits")
    sv = _ints(spatial_shapes)
    L = len(sv) // 2
    B, Nq, M, LK = x.shape
    if LK != L * points:
        raise ValueError(f"logits last dim {LK} != L*K = {L * points}")
    out = torch.empty(B, Nq, M, L, points, dtype=torch.float32, device=x.device)
    sh = _shape(sv, B, M, 1, points, Nq)
    _check(load().msda_attention_softmax(sh.ptr, _p(x), _p(out), _stream(out)), "msda_attention_softmax")
    return out


def msda_prologue(spatial_shapes, offsets_px: torch.Tensor, logits: torch.Tensor,
                  valid_ratios: Optional[torch.Tensor] = None, query_ref: Optional[torch.Tensor] = None):
    """Reference points, sampling locations and attention weights in one call:
    (ref [B,Nq,L,2], loc [B,Nq,M,L,K,2], weights [B,Nq,M,L,K]), the same bits
    as msda_reference_points, msda_sampling_locations and
    msda_attention_softmax in turn. Encoder mode when query_ref is None."""
    off = _dev(offsets_px, "offsets_px")
    x = _dev(logits, "logits")
    if off.dim() != 6 or off.shape[-1] != 2:
        raise ValueError("offsets_px must be [B, Nq, M, L, K, 2]")
    B, Nq, M, L, K, _ = off.shape
    if tuple(x.shape) != (B, Nq, M, L * K):
        raise ValueError(f"logits must be [{B}, {Nq}, {M}, {L * K}], got {tuple(x.shape)}")
    if valid_ratios is not None:
        valid_ratios = _dev(valid_ratios, "valid_ratios")
        if tuple(valid_ratios.shape) != (B, L, 2):
            raise ValueError(f"valid_ratios must be [{B}, {L}, 2], got {tuple(valid_ratios.shape)}")
    if query_ref is not None:
        query_ref = _dev(query_ref, "query_ref")
        if tuple(query_ref.shape) != (B, Nq, 2):
            raise ValueError(f"query_ref must be [{B}, {Nq}, 2], got {tuple(query_ref.shape)}")
    sh = _shape(spatial_shapes, B, M, 1, K, Nq)
    if sh.levels != L:
        raise ValueError("spatial_shapes and offsets_px disagree on the level count")
    ref = torch.empty(B, Nq, L, 2, dtype=torch.float32, device=off.device)
    loc = torch.empty_like(off)
    w = torch.empty(B, Nq, M, L, K, dtype=torch.float32, device=off.device)
    _check(load().msda_prologue(sh.ptr, _p(valid_ratios), _p(query_ref), _p(off), _p(x), _p(ref), _p(loc), _p(w),
                                _stream(off)), "msda_prologue")
    return ref, loc, w


def _core_shape(value, spatial_shapes, level_start_index, loc, attn):
    if value.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"value must be float32 or bfloat16 (got {value.dtype})")
    value = _dev(value, "value", None)
    loc = _dev(loc, "sampling_locations")
    attn = _dev(attn, "attention_weights")
    if value.dim() != 4:
        raise ValueError("value must be [B, S, M, D]")
    B, S, M, D = value.shape
    if loc.dim() != 6 or loc.shape[0] != B or loc.shape[2] != M or loc.shape[-1] != 2:
        raise ValueError(f"sampling_locations must be [{B}, Nq, {M}, L, K, 2], got {tuple(loc.shape)}")
    _, Nq, _, L, K, _ = loc.shape
    if tuple(attn.shape) != (B, Nq, M, L, K):
        raise ValueError(f"attention_weights must be {(B, Nq, M, L, K)}, got {tuple(attn.shape)}")
    sh = _shape(spatial_shapes, B, M, D, K, Nq, level_start_index, S)
    if sh.levels != L:
        raise ValueError("spatial_shapes and sampling_locations disagree on the level count")
    vt = MSDA_BF16 if value.dtype == torch.bfloat16 else MSDA_F32
    return value, loc, attn, sh, vt


def msda_forward(value: torch.Tensor, spatial_shapes, level_start_index, sampling_locations: torch.Tensor,
                 attention_weights: torch.Tensor) -> torch.Tensor:
    """Core forward -> output [B, Nq, M*D] fp32."""
    value, loc, attn, sh, vt = _core_shape(value, spatial_shapes, level_start_index, sampling_locations,
                                           attention_weights)
    B, S, M, D = value.shape
    out = torch.empty(B, loc.shape[1], M * D, dtype=torch.float32, device=value.device)
    _check(load().msda_forward(sh.ptr, _p(value), vt, _p(loc), _p(attn), _p(out), _stream(out)),
           "msda_forward")
    return out


def _workspace(sh, device):
    """(workspace tensor, bytes) for a backward of these sizes."""
    nbytes = getattr(sh, "workspace_bytes", None)
    if nbytes is None:
        nbytes = sh.workspace_bytes = msda_backward_workspace_size(sh)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), nbytes


def msda_backward(value: torch.Tensor, spatial_shapes, level_start_index, sampling_locations: torch.Tensor,
                  attention_weights: torch.Tensor, grad_output: torch.Tensor,
                  grad_value: Optional[torch.Tensor] = None):
    """Core backward -> (grad_value [B,S,M,D] fp32, grad_sampling_locations, grad_attention_weights).
    If grad_value is given it is accumulated into (MSDA_BWD_ACCUMULATE)."""
    value, loc, attn, sh, vt = _core_shape(value, spatial_shapes, level_start_index, sampling_locations,
                                           attention_weights)
    B, S, M, D = value.shape
    go = _dev(grad_output, "grad_output")
    if tuple(go.shape) != (B, loc.shape[1], M * D):
        raise ValueError(f"grad_output must be {(B, loc.shape[1], M * D)}, got {tuple(go.shape)}")
    flags = 0
    if grad_value is None:
        grad_value = torch.empty(B, S, M, D, dtype=torch.float32, device=value.device)
    else:
        if grad_value.dtype != torch.float32 or tuple(grad_value.shape) != (B, S, M, D) or \
                not grad_value.is_contiguous():
            raise ValueError("grad_value to accumulate into must be a contiguous fp32 [B,S,M,D] tensor")
        flags = MSDA_BWD_ACCUMULATE
    gl = torch.empty_like(loc)
    ga = torch.empty_like(attn)
    ws, nbytes = _workspace(sh, value.device)
    _check(load().msda_backward(sh.ptr, _p(value), vt, _p(loc), _p(attn), _p(go), _p(grad_value), _p(gl),
                                _p(ga), _p(ws), nbytes, flags, _stream(go)), "msda_backward")
    return grad_value, gl, ga


def msda_backward_noalloc(value: torch.Tensor, spatial_shapes, level_start_index, sampling_locations: torch.Tensor,
                          attention_weights: torch.Tensor, grad_output: torch.Tensor,
                          grad_value: Optional[torch.Tensor] = None):
    """msda_backward through the entry point that allocates nothing (its
    scratch is the library's own device array); outputs as msda_backward."""
    value, loc, attn, sh, vt = _core_shape(value, spatial_shapes, level_start_index, sampling_locations,
                                           attention_weights)
    B, S, M, D = value.shape
    go = _dev(grad_output, "grad_output")
    if tuple(go.shape) != (B, loc.shape[1], M * D):
        raise ValueError(f"grad_output must be {(B, loc.shape[1], M * D)}, got {tuple(go.shape)}")
    flags = 0
    if grad_value is None:
        grad_value = torch.empty(B, S, M, D, dtype=torch.float32, device=value.device)
    else:
        if grad_value.dtype != torch.float32 or tuple(grad_value.shape) != (B, S, M, D) or \
                not grad_value.is_contiguous():
            raise ValueError("grad_value to accumulate into must be a contiguous fp32 [B,S,M,D] tensor")
        flags = MSDA_BWD_ACCUMULATE
    gl = torch.empty_like(loc)
    ga = torch.empty_like(attn)
    _check(load().msda_backward_noalloc(sh.ptr, _p(value), vt, _p(loc), _p(attn), _p(go), _p(grad_value), _p(gl),
                                        _p(ga), flags, _stream(go)), "msda_backward_noalloc")
    return grad_value, gl, ga


def _mask(key_padding_mask, B, S, device):
    """The [B,S] padding mask as a contiguous uint8 device tensor (or None)."""
    if key_padding_mask is None:
        return None
    if tuple(key_padding_mask.shape) != (B, S):
        raise ValueError(f"key_padding_mask must be [{B}, {S}], got {tuple(key_padding_mask.shape)}")
    if key_padding_mask.device != device:
        raise ValueError("key_padding_mask must be on the value's device")
    return key_padding_mask.to(torch.uint8).contiguous()


def msda_forward_fused(value: torch.Tensor, spatial_shapes, level_start_index, reference_points: torch.Tensor,
                       sampling_offsets: torch.Tensor, attention_logits: torch.Tensor,
                       key_padding_mask: Optional[torch.Tensor] = None):
    """Fused forward: locations and the L*K softmax formed inside the core.
    reference_points [B,Nq,L,2] (offsets in pixels of level l) or boxes
    [B,Nq,L,4] (offsets relative to the box size), sampling_offsets
    [B,Nq,M,L,K,2], attention_logits [B,Nq,M,L*K], key_padding_mask [B,S]
    (True = padded: those value rows read as zero) or None ->
    (output [B,Nq,M*D], sampling_locations, attention_weights)."""
    if value.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"value must be float32 or bfloat16 (got {value.dtype})")
    value = _dev(value, "value", None)
    ref = _dev(reference_points, "reference_points")
    off = _dev(sampling_offsets, "sampling_offsets")
    logits = _dev(attention_logits, "attention_logits")
    if value.dim() != 4:
        raise ValueError("value must be [B, S, M, D]")
    B, S, M, D = value.shape
    if off.dim() != 6 or off.shape[0] != B or off.shape[2] != M or off.shape[-1] != 2:
        raise ValueError(f"sampling_offsets must be [{B}, Nq, {M}, L, K, 2], got {tuple(off.shape)}")
    _, Nq, _, L, K, _ = off.shape
    if ref.dim() != 4 or tuple(ref.shape[:3]) != (B, Nq, L) or ref.shape[3] not in (2, 4):
        raise ValueError(f"reference_points must be [{B}, {Nq}, {L}, 2 or 4], got {tuple(ref.shape)}")
    if tuple(logits.shape) != (B, Nq, M, L * K):
        raise ValueError(f"attention_logits must be {(B, Nq, M, L * K)}, got {tuple(logits.shape)}")
    sh = _shape(spatial_shapes, B, M, D, K, Nq, level_start_index, S)
    if sh.levels != L:
        raise ValueError("spatial_shapes and sampling_offsets disagree on the level count")
    vt = MSDA_BF16 if value.dtype == torch.bfloat16 else MSDA_F32
    out = torch.empty(B, Nq, M * D, dtype=torch.float32, device=value.device)
    loc = torch.empty_like(off)
    attn = torch.empty(B, Nq, M, L, K, dtype=torch.float32, device=value.device)
    mask = _mask(key_padding_mask, B, S, value.device)
    _check(load().msda_forward_fused(sh.ptr, _p(value), vt, _p(ref), int(ref.shape[3]), _p(off), _p(logits),
                                     _p(mask), _p(out), _p(loc), _p(attn), _stream(out)), "msda_forward_fused")
    return out, loc, attn


def msda_backward_fused(value: torch.Tensor, spatial_shapes, level_start_index, sampling_locations: torch.Tensor,
                        attention_weights: torch.Tensor, grad_output: torch.Tensor,
                        grad_value: Optional[torch.Tensor] = None, reference_grad: bool = True,
                        box_references: Optional[torch.Tensor] = None,
                        sampling_offsets: Optional[torch.Tensor] = None,
                        key_padding_mask: Optional[torch.Tensor] = None):
    """Backward of msda_forward_fused, from the locations and weights it
    returned -> (grad_value [B,S,M,D], grad_sampling_offsets [B,Nq,M,L,K,2],
    grad_attention_logits [B,Nq,M,L*K], grad_reference_points [B,Nq,L,2|4]
    or None). For 4-d box references pass the boxes and the offsets of the
    forward, and the forward's key_padding_mask if it had one. If grad_value
    is given it is accumulated into."""
    value, loc, attn, sh, vt = _core_shape(value, spatial_shapes, level_start_index, sampling_locations,
                                           attention_weights)
    B, S, M, D = value.shape
    _, Nq, _, L, K, _ = loc.shape
    go = _dev(grad_output, "grad_output")
    if tuple(go.shape) != (B, Nq, M * D):
        raise ValueError(f"grad_output must be {(B, Nq, M * D)}, got {tuple(go.shape)}")
    flags = 0
    if grad_value is None:
        grad_value = torch.empty(B, S, M, D, dtype=torch.float32, device=value.device)
    else:
        if grad_value.dtype != torch.float32 or tuple(grad_value.shape) != (B, S, M, D) or \
                not grad_value.is_contiguous():
            raise ValueError("grad_value to accumulate into must be a contiguous fp32 [B,S,M,D] tensor")
        flags = MSDA_BWD_ACCUMULATE
    dims = 2
    box = off = None
    if box_references is not None:
        dims = 4
        box = _dev(box_references, "box_references")
        off = _dev(sampling_offsets, "sampling_offsets")
        if tuple(box.shape) != (B, Nq, L, 4) or tuple(off.shape) != tuple(loc.shape):
            raise ValueError("box_references must be [B,Nq,L,4] and sampling_offsets [B,Nq,M,L,K,2]")
    goff = torch.empty_like(loc)
    glog = torch.empty(B, Nq, M, L * K, dtype=torch.float32, device=value.device)
    gref = torch.empty(B, Nq, L, dims, dtype=torch.float32, device=value.device) if reference_grad else None
    ws, nbytes = _workspace(sh, value.device)
    mask = _mask(key_padding_mask, B, S, value.device)
    _check(load().msda_backward_fused(sh.ptr, _p(value), vt, _p(loc), _p(attn), _p(box), _p(off), dims, _p(mask),
                                      _p(go),
                                      _p(grad_value), _p(goff), _p(glog), _p(gref), _p(ws), nbytes, flags,
                                      _stream(go)), "msda_backward_fused")
    return grad_value, goff, glog, gref


def msda_backward_workspace_size(shape: "Shape") -> int:
    """Bytes of device workspace msda_backward needs for these sizes."""
    n = ctypes.c_size_t()
    _check(load().msda_backward_workspace_size(shape.ptr, ctypes.byref(n)), "msda_backward_workspace_size")
    return int(n.value)


def msda_backward_plan(shape: "Shape") -> dict:
    """Which levels the backward's tiled fast path would sum from their samples
    ('dense'), give tiles too small to sort ('direct'), and split over several
    workgroups with float atomics ('split'); lists of level indices."""
    masks = [ctypes.c_uint32() for _ in range(3)]
    _check(load().msda_backward_plan(shape.ptr, *[ctypes.byref(m) for m in masks]), "msda_backward_plan")
    levels = shape.levels
    return {key: [l for l in range(levels) if (m.value >> l) & 1]
            for key, m in zip(("dense", "direct", "split"), masks)}


def raw_call(name: str, *args):
    """Call an entry point with raw ctypes arguments and return its status
    (used by the boundary tests; no checks, no exceptions)."""
    return getattr(load(), name)(*args)


def msda_timing_enable(on: bool = True) -> None:
    """Bracket every kernel launch of the library with a HIP event pair on its
    stream (not while the stream is captured)."""
    _check(load().msda_timing_enable(1 if on else 0), "msda_timing_enable")


def msda_timing_reset() -> None:
    _check(load().msda_timing_reset(), "msda_timing_reset")


def msda_timing_read() -> dict:
    """{kernel name: (total milliseconds, launches)} of the timed launches so far."""
    lib = load()
    n = ctypes.c_int(0)
    _check(lib.msda_timing_read(-1, ctypes.byref(n), None, None, None), "msda_timing_read")
    out = {}
    for i in range(n.value):
        name = ctypes.c_char_p()
        ms = ctypes.c_double()
        cnt = ctypes.c_int64()
        _check(lib.msda_timing_read(i, None, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(cnt)),
               "msda_timing_read")
        out[name.value.decode()] = (ms.value, cnt.value)
    return out
