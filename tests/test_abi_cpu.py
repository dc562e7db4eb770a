"""CPU tests of the C ABI: the library loads, exports every entry point declared in
include/fa.h, and rejects invalid arguments with the documented status before any HIP
call (so these run on a host without a GPU)."""

import ctypes
import os
import re

import pytest

from exact_io_aware_19_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared():
    with open(HEADER) as f:
        src = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(fa_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail(f"{_lib.LIB_PATH} not built; run python -m exact_io_aware_19_amd.build")
    return _lib.load()


def test_header_declares_the_boundary():
    assert _declared() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.fa_status_string(code).decode().startswith(name)
    assert lib.fa_status_string(12345).decode() == "unknown fa_status"


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced on error paths


def _fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, scale=0.125, causal=0):
    return lib.fa_forward(q, k, v, o, lse, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
        (dict(B=0), -2), (dict(H=0), -2), (dict(N=0), -2), (dict(N=-5), -2), (dict(B=1 << 20, H=1 << 11), -2),
        (dict(d=96), -3), (dict(d=0), -3), (dict(d=256), -3),
        (dict(scale=float("inf")), -4), (dict(scale=float("-inf")), -4), (dict(scale=float("nan")), -4),
        (dict(q=FAKE + 8), -7), (dict(lse=FAKE + 2), -7),
        # a zero or negative scale passes validation: the alignment error behind it is reported
        (dict(scale=0.0, q=FAKE + 8), -7), (dict(scale=-1.0, q=FAKE + 8), -7), (dict(scale=-0.0, lse=FAKE + 2), -7),
    ],
)
def test_forward_rejects(lib, kw, status):
    assert _fwd(lib, **kw) == status


def test_forward_kvlen_rejects(lib):
    assert lib.fa_forward_kvlen(None, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 0.1, 0, FAKE, None) == -1
    assert lib.fa_forward_kvlen(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 80, 0.1, 0, FAKE, None) == -3


def test_workspace_size(lib):
    B, H, N, d = 2, 3, 100, 128
    nw = (N + 255) // 256 * 256  # rows per head, padded to the dQ pass's 256-row blocks
    want = 2 * 4 * B * H * nw  # D_i and LSE_i * log2(e), fp32
    assert lib.fa_backward_workspace_size(B, H, N, d) == want
    assert lib.fa_backward_workspace_size(0, H, N, d) == 0
    assert lib.fa_backward_workspace_size(B, H, N, 72) == 0


def _bwd(lib, ws=FAKE, ws_bytes=None, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=1, N=16, d=64,
             scale=0.125, causal=0)
    a.update(kw)
    need = lib.fa_backward_workspace_size(a["B"], a["H"], a["N"], a["d"]) if a["N"] > 0 else 0
    return lib.fa_backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"],
                           a["H"], a["N"], a["d"], a["scale"], a["causal"], ws,
                           need if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("missing", ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"])
def test_backward_rejects_null(lib, missing):
    assert _bwd(lib, **{missing: None}) == -1


def test_backward_rejects_bad_args(lib):
    assert _bwd(lib, d=32) == -3
    assert _bwd(lib, N=0) == -2
    assert _bwd(lib, scale=float("nan")) == -4
    assert _bwd(lib, scale=float("-inf")) == -4
    assert _bwd(lib, scale=0.0, ws=FAKE + 16) == -7  # any finite scale is accepted
    assert _bwd(lib, scale=-2.0, ws=FAKE + 16) == -7
    assert _bwd(lib, ws=None) == -5
    assert _bwd(lib, ws_bytes=16) == -5
    assert _bwd(lib, ws=FAKE + 16) == -7
    assert _bwd(lib, dq=FAKE + 4) == -7
    assert lib.fa_backward_kvlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 0.1, 0, FAKE,
                                 None, 0, None) == -5


@pytest.mark.parametrize("name", ["fa_backward_dq_pass", "fa_backward_dkdv_pass"])
def test_backward_passes_validate_like_backward(lib, name):
    fn = getattr(lib, name)
    need = lib.fa_backward_workspace_size(1, 1, 16, 64)

    def call(q=FAKE, d=64, N=16, ws=FAKE, ws_bytes=need, kv=None):
        return fn(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, N, d, 0.125, 0, kv, ws, ws_bytes, None)

    assert call(q=None) == -1
    assert call(d=32) == -3
    assert call(N=0) == -2
    assert call(ws=None) == -5
    assert call(ws_bytes=need - 1) == -5
    assert call(ws=FAKE + 16) == -7


def _fwd_off(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Nq=16, Nk=40, d=64, scale=0.125, causal=1,
             q_offset=24):
    return lib.fa_forward_offset(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, q_offset, None, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), -1), (dict(k=None), -1), (dict(lse=None), -1),
        (dict(Nq=0), -2), (dict(Nk=0), -2), (dict(Nk=-1), -2), (dict(q_offset=-1), -2), (dict(B=0), -2),
        (dict(q_offset=(1 << 31) - 200), -2),
        (dict(Nk=1 << 26, d=128), -2),
        (dict(d=32), -3), (dict(scale=float("nan")), -4), (dict(v=FAKE + 4), -7), (dict(lse=FAKE + 1), -7),
    ],
)
def test_forward_offset_rejects_invalid_arguments(lib, kw, status):
    assert _fwd_off(lib, **kw) == status


@pytest.mark.parametrize("H,Hkv,status", [(4, 3, -8), (4, 0, -8), (4, -2, -8), (4, 5, -8), (0, 1, -2)])
def test_gqa_entry_points_reject_bad_kv_heads(lib, H, Hkv, status):
    assert lib.fa_forward_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, H, Hkv, 16, 64, 0.125, 0, None, None) == status
    need = lib.fa_backward_workspace_size(1, max(H, 1), 16, 64)
    assert lib.fa_backward_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, H, Hkv, 16, 64, 0.125, 0,
                               None, FAKE, need, None) == status


def test_gqa_entry_points_validate_like_the_others(lib):
    assert lib.fa_forward_gqa(None, FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 16, 64, 0.125, 0, None, None) == -1
    assert lib.fa_forward_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 16, 96, 0.125, 0, None, None) == -3
    assert lib.fa_forward_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 16, 64, float("nan"), 0, None, None) == -4
    assert lib.fa_forward_gqa(FAKE, FAKE + 8, FAKE, FAKE, FAKE, 1, 4, 2, 16, 64, 0.1, 0, None, None) == -7
    need = lib.fa_backward_gqa_workspace_size(1, 4, 2, 16, 64)

    def bwd(ws=FAKE, ws_bytes=need, dk=FAKE):
        return lib.fa_backward_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dk, FAKE, 1, 4, 2, 16, 64, 0.125, 0,
                                   None, ws, ws_bytes, None)

    assert bwd(dk=None) == -1
    assert bwd(ws=None) == -5
    assert bwd(ws_bytes=need - 1) == -5
    assert bwd(dk=FAKE + 4) == -7


def test_gqa_workspace_size(lib):
    B, H, N, d = 2, 16, 4096, 128
    stats = 2 * 4 * B * H * ((N + 255) // 256 * 256)
    # enough (key block, K/V head) pairs: statistics only, like the ungrouped size
    assert lib.fa_backward_gqa_workspace_size(B, H, H, N, d) == lib.fa_backward_workspace_size(B, H, N, d) == stats
    assert lib.fa_backward_gqa_workspace_size(4, H, 8, N, d) == 2 * 4 * 4 * H * ((N + 255) // 256 * 256)
    # MQA at B=2: 64 pairs < 512 workgroups -> 8 splits, fp32 partial dK and dV each
    assert lib.fa_backward_gqa_workspace_size(B, H, 1, N, d) == stats + 2 * 8 * B * 1 * N * d * 4
    # never more splits than query heads per group
    assert lib.fa_backward_gqa_workspace_size(1, 2, 1, 128, 64) == 2 * 4 * 2 * 256 + 2 * 2 * 1 * 128 * 64 * 4
    assert lib.fa_backward_gqa_workspace_size(B, H, 3, N, d) == 0
    assert lib.fa_backward_gqa_workspace_size(B, H, 1, N, 80) == 0
    need = lib.fa_backward_gqa_workspace_size(1, 2, 1, 128, 64)
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 128, 64, 0.125, 0, None, FAKE)
    assert lib.fa_backward_gqa(*args, need - 1, None) == -5


def _fp8(lib, q8=FAKE, sq=FAKE, k8=FAKE, sk=FAKE, v8t=FAKE, sv=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=128,
         scale=0.125, causal=0):
    return lib.fa_forward_fp8(q8, sq, k8, sk, v8t, sv, o, lse, B, H, N, d, scale, causal, None, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q8=None), -1), (dict(sq=None), -1), (dict(k8=None), -1), (dict(sk=None), -1), (dict(v8t=None), -1),
        (dict(sv=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
        (dict(N=0), -2), (dict(B=0), -2), (dict(d=96), -3), (dict(scale=float("inf")), -4), (dict(scale=float("nan")), -4),
        (dict(scale=0.0, q8=FAKE + 8), -7), (dict(scale=-0.5, q8=FAKE + 8), -7), (dict(q8=FAKE + 8), -7), (dict(v8t=FAKE + 4), -7), (dict(sk=FAKE + 2), -7), (dict(lse=FAKE + 1), -7),
    ],
)
def test_forward_fp8_rejects(lib, kw, status):
    assert _fp8(lib, **kw) == status


def test_fp8_quantizers_reject(lib):
    q = lib.fa_fp8_quantize_qk
    assert q(None, FAKE, FAKE, None, 1.0, 1, 1, 16, 128, None) == -1
    assert q(FAKE, None, FAKE, None, 1.0, 1, 1, 16, 128, None) == -1
    assert q(FAKE, FAKE, None, None, 1.0, 1, 1, 16, 128, None) == -1
    assert q(FAKE, FAKE, FAKE, None, 1.0, 1, 1, 16, 32, None) == -3
    assert q(FAKE, FAKE, FAKE, None, 0.0, 1, 1, 16, 128, None) == -4
    assert q(FAKE, FAKE, FAKE, None, float("inf"), 1, 1, 16, 128, None) == -4
    assert q(FAKE, FAKE + 8, FAKE, None, 1.0, 1, 1, 16, 128, None) == -7
    assert q(FAKE, FAKE, FAKE, FAKE + 2, 1.0, 1, 1, 16, 128, None) == -7
    v = lib.fa_fp8_quantize_v
    assert v(None, FAKE, FAKE, 1, 1, 16, 64, None) == -1
    assert v(FAKE, FAKE, FAKE, 1, 0, 16, 64, None) == -2
    assert v(FAKE, FAKE, FAKE, 1, 1, 16, 48, None) == -3
    assert v(FAKE, FAKE + 4, FAKE, 1, 1, 16, 64, None) == -7


MICRO_HEADER = os.path.join(ROOT, "include", "fa_micro.h")


def test_micro_library_exports_every_declared_symbol():
    """The machine-microbenchmark library (include/fa_micro.h) loads and exports every
    declared entry point; its argument checks return -1 before any HIP call."""
    from exact_io_aware_19_amd.build import MICRO_LIB_PATH

    if not os.path.exists(MICRO_LIB_PATH):
        pytest.fail(f"{MICRO_LIB_PATH} not built; run python -m exact_io_aware_19_amd.build")
    with open(MICRO_HEADER) as f:
        names = sorted(set(re.findall(r"^\s*int\s+(fa_micro_\w+)\s*\(", f.read(), re.M)))
    assert names == ["fa_micro_atomic_tiles", "fa_micro_coexec", "fa_micro_exp", "fa_micro_grid_blocks",
                     "fa_micro_lds_read", "fa_micro_mfma_bf16", "fa_micro_mfma_fp8_tile", "fa_micro_mfma_order"]
    lib = ctypes.CDLL(MICRO_LIB_PATH)
    for name in names:
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr), name
    vp, i = ctypes.c_void_p, ctypes.c_int
    for name in ("fa_micro_mfma_bf16", "fa_micro_exp", "fa_micro_lds_read"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, i, i, vp]
        assert fn(None, 1, 1, None) == -1
        assert fn(vp(16), 0, 1, None) == -1
        assert fn(vp(16), 1, 0, None) == -1
    lib.fa_micro_atomic_tiles.argtypes = [vp, i, i, i, vp]
    assert lib.fa_micro_atomic_tiles(None, 1, 1, 1, None) == -1
    assert lib.fa_micro_atomic_tiles(vp(16), 0, 1, 1, None) == -1
    lib.fa_micro_coexec.argtypes = [vp, i, i, i, i, i, vp]
    for args in ((None, 1, 3, 0, 1, 1), (vp(16), 1, 0, 0, 1, 1), (vp(16), 1, 4, 0, 1, 1), (vp(16), 1, 3, 4, 1, 1), (vp(16), 1, 3, -1, 1, 1),
                 (vp(16), 1, 3, 0, 0, 1), (vp(16), 1, 3, 0, 1, 0), (vp(16), 0, 3, 0, 1, 1)):
        assert lib.fa_micro_coexec(*args, None) == -1, args
    lib.fa_micro_mfma_order.argtypes = [vp, vp, i, i, i, vp]
    for args in ((None, vp(16), 1, 0, 1), (vp(16), None, 1, 0, 1), (vp(16), vp(16), 0, 0, 1), (vp(16), vp(16), 1, -1, 1),
                 (vp(16), vp(16), 1, 4, 1), (vp(16), vp(16), 1, 0, 0)):
        assert lib.fa_micro_mfma_order(*args, None) == -1, args
    lib.fa_micro_mfma_fp8_tile.argtypes = [vp, vp, vp, vp, vp]
    for k in range(4):
        ptrs = [vp(16)] * 4
        ptrs[k] = None
        assert lib.fa_micro_mfma_fp8_tile(*ptrs, None) == -1


def _noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=1, N=16, d=64,
             scale=0.125, causal=0, kv=None)
    a.update(kw)
    return lib.fa_backward_noalloc(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                   a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["kv"], None)


def test_backward_noalloc_validates_before_any_hip_call(lib):
    """Argument errors and the scratch limit (FA_NOALLOC_SCRATCH_BYTES = 16 MiB of row
    statistics: 2^21 padded rows) are reported on the host, without a GPU."""
    assert _lib.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert _noalloc(lib, dv=None) == -1
    assert _noalloc(lib, N=0) == -2
    assert _noalloc(lib, d=96) == -3
    assert _noalloc(lib, scale=float("nan")) == -4
    # 32 heads x 65536 rows = 2^21 rows fill the scratch exactly: accepted (the
    # misaligned dq behind it is what gets reported); one more head is too many
    assert lib.fa_backward_workspace_size(1, 32, 65536, 64) == _lib.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, H=32, N=65536, dq=FAKE + 4) == -7
    assert _noalloc(lib, H=33, N=65536) == -5
    assert _noalloc(lib, B=2, H=16, N=65537) == -5
    assert _noalloc(lib, scale=-1.0, lse=FAKE + 2) == -7
