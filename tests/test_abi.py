"""The C-ABI boundary on the CPU: the library loads, exports every entry point
include/msda.h declares, and rejects bad arguments on the host with the
documented status code before any device work. No compute call is made (no
GPU here); every call below fails validation."""
import ctypes
import os
import subprocess

import pytest

from scale_deformable_attention_msdeformattn_amd import _binding as B
from tests.conftest import golden


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from scale_deformable_attention_msdeformattn_amd import build
        build.build()
    return B.load()


def test_exports_every_declared_symbol(lib):
    declared = B.declared_symbols()
    assert set(declared) >= {"msda_reference_points", "msda_forward", "msda_backward",
                             "msda_sampling_locations", "msda_attention_softmax", "msda_status_string"}
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing else leaks out under the msda_ prefix
    assert {n for n in exported if n.startswith("msda_")} == set(declared)


def test_version_and_status_strings(lib):
    assert lib.msda_abi_version() == 11
    assert lib.msda_status_string(0) == b"ok"
    for code in range(-8, 0):
        assert lib.msda_status_string(code) not in (b"", b"unknown status")
    assert lib.msda_status_string(-99) == b"unknown status"


def test_level_start_index_helper_on_page1_pyramid(lib):
    g = golden("pyramid_76x106.json")
    lsi, S = B.level_start_index_host(g["spatial_shapes"])
    assert lsi == g["level_start_index"] and S == g["S"]


def _shape(B_=2, M=8, D=32, K=4, shapes=((76, 106), (38, 53), (19, 27), (8, 13)), S=None, Nq=None, lsi=None):
    S_true = sum(h * w for h, w in shapes)
    if lsi is None:  # exclusive prefix sum, written out so that invalid shapes reach the library
        lsi = [sum(h * w for h, w in shapes[:i]) for i in range(len(shapes))]
    sh = B.Shape(shapes, B_, M, D, K, Nq if Nq is not None else S_true, lsi)
    sh.c.num_value = S_true if S is None else S
    return sh


FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: every call below fails validation first
MISALIGNED = ctypes.c_void_p(0x10002)

# The fake device pointers above must never reach a kernel; these tests are for
# a host without a GPU, where even a validation slip could not launch anything.
cpu_only = pytest.mark.skipif(__import__("torch").cuda.is_available(),
                              reason="fake-pointer validation tests run on a host without a GPU")


def _fwd(lib, sh, value=FAKE, dtype=B.MSDA_F32, loc=FAKE, attn=FAKE, out=FAKE):
    return lib.msda_forward(sh.ptr if sh is not None else None, value, dtype, loc, attn, out, None)


def _bwd(lib, sh, flags=0, value=FAKE, grads=(FAKE, FAKE, FAKE, FAKE), ws=None, ws_bytes=0):
    return lib.msda_backward(sh.ptr, value, B.MSDA_F32, FAKE, FAKE, grads[0], grads[1], grads[2], grads[3],
                             ws, ws_bytes, flags, None)


@cpu_only
def test_null_arguments(lib):
    assert _fwd(lib, None) == B.MSDA_E_NULL
    for kw in ("value", "loc", "attn", "out"):
        assert _fwd(lib, _shape(), **{kw: None}) == B.MSDA_E_NULL, kw
    sh = _shape()
    sh.c.spatial_shapes = None
    assert _fwd(lib, sh) == B.MSDA_E_NULL
    for i in range(4):
        grads = [FAKE] * 4
        grads[i] = None
        assert _bwd(lib, _shape(), grads=tuple(grads)) == B.MSDA_E_NULL
    assert lib.msda_reference_points(_shape().ptr, None, None, None, None) == B.MSDA_E_NULL
    assert lib.msda_sampling_locations(_shape().ptr, FAKE, None, FAKE, None) == B.MSDA_E_NULL
    assert lib.msda_attention_softmax(_shape().ptr, None, FAKE, None) == B.MSDA_E_NULL
    assert b"NULL" in lib.msda_last_error()


@cpu_only
def test_prologue_validates_on_the_host(lib):
    enc = _shape(Nq=None)

    def call(sh, vr=None, u=None, off=FAKE, x=FAKE, ref=FAKE, loc=FAKE, w=FAKE):
        return lib.msda_prologue(sh.ptr, vr, u, off, x, ref, loc, w, None)
    for k in ("off", "x", "ref", "loc", "w"):
        assert call(enc, **{k: None}) == B.MSDA_E_NULL, k
    # encoder reference points need Nq == S; decoder mode (u given) does not
    dec = _shape(Nq=300)
    assert call(dec) == B.MSDA_E_SHAPE
    odd = ctypes.c_void_p(0x10004)   # 4-byte aligned, not 8
    assert call(enc, loc=odd) == B.MSDA_E_ALIGN
    assert call(dec, u=odd) == B.MSDA_E_ALIGN
    assert call(enc, w=ctypes.c_void_p(0x10002)) == B.MSDA_E_ALIGN
    # no queries: nothing to do, no device work
    assert call(_shape(Nq=0), u=FAKE) == B.MSDA_OK


def test_fused_entry_points_validate_on_the_host(lib):
    ptrs = [FAKE] * 6   # ref, offsets, logits, output, loc_out, attn_out

    def fwd(dtype, ref, dims, p, mask=None):
        # (..., ref, dims, offsets, logits, key_padding_mask, output, loc_out, attn_out, stream)
        return lib.msda_forward_fused(_shape().ptr, FAKE, dtype, ref, dims, p[0], p[1], mask, p[2], p[3], p[4], None)
    for i in range(6):
        p = list(ptrs)
        p[i] = None
        assert fwd(B.MSDA_F32, p[0], 2, p[1:]) == B.MSDA_E_NULL, i
    assert fwd(7, FAKE, 2, ptrs[1:]) == B.MSDA_E_UNSUPPORTED
    assert fwd(B.MSDA_F32, FAKE, 3, ptrs[1:]) == B.MSDA_E_UNSUPPORTED
    odd = ctypes.c_void_p(0x10004)   # 4-byte aligned, not 8: (x, y) tensors need 8
    assert fwd(B.MSDA_F32, odd, 2, ptrs[1:]) == B.MSDA_E_ALIGN
    box8 = ctypes.c_void_p(0x10008)  # 8-byte aligned, not 16: boxes need 16
    assert fwd(B.MSDA_F32, box8, 4, ptrs[1:]) == B.MSDA_E_ALIGN
    # a mask (bytes: any alignment) does not change the validation
    assert fwd(B.MSDA_F32, FAKE, 3, ptrs[1:], mask=ctypes.c_void_p(0x10001)) == B.MSDA_E_UNSUPPORTED

    def bwd(g, ref=None, off=None, dims=2, flags=0, mask=None):
        return lib.msda_backward_fused(_shape().ptr, FAKE, B.MSDA_F32, FAKE, FAKE, ref, off, dims, mask, FAKE, *g,
                                       None, 0, flags, None)
    for i in range(3):   # grad_value, grad_offsets, grad_logits required; grad_ref optional
        g = [FAKE, FAKE, FAKE, FAKE]
        g[i] = None
        assert bwd(g) == B.MSDA_E_NULL, i
    assert bwd([FAKE] * 3 + [None], dims=4) == B.MSDA_E_NULL        # boxes need references and offsets
    assert bwd([FAKE] * 3 + [None], dims=5) == B.MSDA_E_UNSUPPORTED
    assert bwd([FAKE] * 3 + [None], flags=0x4) == B.MSDA_E_UNSUPPORTED
    assert bwd([FAKE] * 3 + [None], mask=ctypes.c_void_p(0x10001)) == B.MSDA_E_WORKSPACE
    assert bwd([FAKE] * 3 + [None]) == B.MSDA_E_WORKSPACE


@cpu_only
def test_bad_dimensions(lib):
    for field in ("heads", "channels", "points"):
        sh = _shape()
        setattr(sh.c, field, 0)
        assert _fwd(lib, sh) == B.MSDA_E_DIM, field
    sh = _shape()
    sh.c.num_query = -1
    assert _fwd(lib, sh) == B.MSDA_E_DIM
    sh = _shape()
    sh.c.batch = -2
    assert _fwd(lib, sh) == B.MSDA_E_DIM
    assert _fwd(lib, _shape(shapes=((0, 5), (2, 2)))) == B.MSDA_E_DIM
    # index width: one batch of value at 2^29 elements or more is refused
    big = _shape(B_=1, M=8, D=32, shapes=((2048, 1024),))
    assert _fwd(lib, big) == B.MSDA_E_DIM
    many = _shape(B_=1 << 12, M=8, D=32, shapes=((256, 256),))
    assert _fwd(lib, many) == B.MSDA_E_DIM


@cpu_only
def test_shape_and_level_index_mismatch(lib):
    assert _fwd(lib, _shape(S=10686)) == B.MSDA_E_SHAPE
    assert _fwd(lib, _shape(lsi=[0, 8056, 10070, 10584])) == B.MSDA_E_LEVEL_INDEX
    assert _fwd(lib, _shape(lsi=[0, 2014, 2527, 2631])) == B.MSDA_E_LEVEL_INDEX
    # encoder reference points need Nq == S
    sh = _shape(Nq=300)
    assert lib.msda_reference_points(sh.ptr, None, None, FAKE, None) == B.MSDA_E_SHAPE


@cpu_only
def test_unsupported(lib):
    assert _fwd(lib, _shape(), dtype=7) == B.MSDA_E_UNSUPPORTED
    many_levels = tuple((2, 2) for _ in range(17))
    assert _fwd(lib, _shape(shapes=many_levels)) == B.MSDA_E_UNSUPPORTED
    assert _bwd(lib, _shape(), flags=4) == B.MSDA_E_UNSUPPORTED


@cpu_only
def test_misaligned(lib):
    assert _fwd(lib, _shape(), value=MISALIGNED) == B.MSDA_E_ALIGN
    assert _fwd(lib, _shape(), loc=ctypes.c_void_p(0x10004)) == B.MSDA_E_ALIGN
    assert _fwd(lib, _shape(), out=ctypes.c_void_p(0x10001)) == B.MSDA_E_ALIGN
    assert _bwd(lib, _shape(), grads=(FAKE, MISALIGNED, FAKE, FAKE)) == B.MSDA_E_ALIGN
    assert lib.msda_sampling_locations(_shape().ptr, ctypes.c_void_p(0x10004), FAKE, FAKE, None) == B.MSDA_E_ALIGN
    # bf16 value only needs 2-byte alignment, but an odd address is refused
    assert _fwd(lib, _shape(), value=ctypes.c_void_p(0x10001), dtype=B.MSDA_BF16) == B.MSDA_E_ALIGN


def test_python_binding_refuses_cpu_tensors_and_wrong_dtypes():
    import torch
    v = torch.zeros(1, 80, 2, 4)
    loc = torch.zeros(1, 80, 2, 2, 2, 2)
    a = torch.zeros(1, 80, 2, 2, 2)
    with pytest.raises(ValueError, match="GPU"):
        B.msda_forward(v, [[8, 8], [4, 4]], [0, 64], loc, a)
    with pytest.raises(ValueError, match="float32 or bfloat16"):
        B.msda_forward(v.double(), [[8, 8], [4, 4]], [0, 64], loc, a)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="libmsda.so not found"):
        B.load()


@cpu_only
def test_empty_batch_or_queries_is_a_no_op(lib):
    """B = 0 or Nq = 0: nothing to compute; the call succeeds without touching
    any pointer (NULL tensors are accepted for empty extents)."""
    for field in ("batch", "num_query"):
        sh = _shape()
        setattr(sh.c, field, 0)
        assert _fwd(lib, sh, value=None, loc=None, attn=None, out=None) == B.MSDA_OK, field
        assert lib.msda_sampling_locations(sh.ptr, None, None, None, None) == B.MSDA_OK
        assert lib.msda_attention_softmax(sh.ptr, None, None, None) == B.MSDA_OK
    sh = _shape()
    sh.c.batch = 0
    assert _bwd(lib, sh, grads=(None, None, None, None)) == B.MSDA_OK


@cpu_only
def test_backward_workspace_size_and_check(lib):
    """The encoder sizes take the tiled backward: it needs a workspace, and a
    missing or short one is refused before any device work."""
    sh = _shape()
    n = B.msda_backward_workspace_size(sh)
    # records (4 per sample) dominate: 4 * 4 B * B*Nq*M*L*K
    assert n >= 16 * 2 * 10687 * 8 * 16
    assert _bwd(lib, sh) == B.MSDA_E_WORKSPACE
    assert _bwd(lib, sh, ws=FAKE, ws_bytes=n - 1) == B.MSDA_E_WORKSPACE
    assert _bwd(lib, sh, ws=ctypes.c_void_p(0x10010), ws_bytes=n) == B.MSDA_E_ALIGN
    # sizes without a fast path need none
    assert B.msda_backward_workspace_size(_shape(M=3, D=5)) == 0
    assert lib.msda_backward_workspace_size(sh.ptr, None) == B.MSDA_E_NULL


def test_timing_entry_points_without_launches(lib):
    """The timing aid works on the host alone: no launches, no entries."""
    assert lib.msda_timing_reset() == 0
    assert lib.msda_timing_enable(1) == 0
    assert lib.msda_timing_enable(0) == 0
    n = ctypes.c_int(-5)
    assert lib.msda_timing_read(-1, ctypes.byref(n), None, None, None) == 0
    assert n.value == 0
    assert lib.msda_timing_read(0, ctypes.byref(n), None, None, None) == -2  # MSDA_E_DIM
    assert B.msda_timing_read() == {}


@cpu_only
def test_backward_plan_per_level(lib):
    """The planner's choice of path per level, from the sizes alone (host
    only). The GPU tests of each path rely on these shapes taking it."""
    # the encoder pyramid: the two coarse levels are dense, the fine ones sorted tiles
    assert B.msda_backward_plan(_shape()) == {"dense": [2, 3], "direct": [], "split": []}
    # one 46x46 level (over 2048 pixels, so never dense) at about 94 samples per
    # pixel: 2x2 tiles without the sort, their ~850 records split over two workgroups
    assert B.msda_backward_plan(_shape(B_=1, shapes=((46, 46),), Nq=50000)) == \
        {"dense": [], "direct": [0], "split": [0]}
    # ... at about 80 samples per pixel: 2x2 tiles, one workgroup each
    assert B.msda_backward_plan(_shape(B_=1, shapes=((46, 46),), Nq=42320)) == \
        {"dense": [], "direct": [0], "split": []}
    # sizes off the fast path (M*D != 256): no plan
    assert B.msda_backward_plan(_shape(M=3, D=5)) == {"dense": [], "direct": [], "split": []}
    # empty calls have no plan either, and NULL outputs are allowed
    assert B.msda_backward_plan(_shape(B_=0)) == {"dense": [], "direct": [], "split": []}
    assert lib.msda_backward_plan(_shape().ptr, None, None, None) == B.MSDA_OK


@cpu_only
def test_backward_noalloc_validates_on_the_host(lib):
    """msda_backward_noalloc refuses bad arguments, and sizes whose workspace
    exceeds its fixed scratch, before any device work."""
    f = lib.msda_backward_noalloc

    def call(sh, flags=0, grads=(FAKE, FAKE, FAKE, FAKE), value=FAKE):
        return f(sh.ptr, value, B.MSDA_F32, FAKE, FAKE, *grads, flags, None)

    sh = _shape()
    assert call(sh, flags=0x2) == B.MSDA_E_UNSUPPORTED
    assert call(sh, grads=(FAKE, None, FAKE, FAKE)) == B.MSDA_E_NULL
    assert call(sh, grads=(FAKE, FAKE, MISALIGNED, FAKE)) == B.MSDA_E_ALIGN
    assert call(sh, value=None) == B.MSDA_E_NULL
    assert call(_shape(B_=0)) == B.MSDA_OK
    # the large-batch pyramid at B=8 needs far more workspace than the scratch
    big = _shape(B_=8, shapes=((100, 167), (50, 84), (25, 42), (13, 21)))
    need = B.msda_backward_workspace_size(big)
    assert need > 160 * 2**20
    assert call(big) == B.MSDA_E_WORKSPACE
    assert b"scratch" in lib.msda_last_error()
    # the encoder step's backward fits
    assert B.msda_backward_workspace_size(_shape()) <= 160 * 2**20
