"""GPU checks of the machine microbenchmarks (include/fa_micro.h): each kernel computes
exactly what its header says, so the rates the bench derives from them count real work.
Small grids and iteration counts; the expected values are worked out here in Python."""

import ctypes
import os

import numpy as np
import pytest

from tests import parity as P

pytestmark = pytest.mark.gpu

BLOCKS = 6  # workgroups of 256 threads


@pytest.fixture(scope="module")
def micro():
    from exact_io_aware_19_amd.build import MICRO_LIB_PATH

    if not os.path.exists(MICRO_LIB_PATH):
        pytest.fail(f"{MICRO_LIB_PATH} not built; run python -m exact_io_aware_19_amd.build")
    lib = ctypes.CDLL(MICRO_LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    for name in ("fa_micro_mfma_bf16", "fa_micro_exp", "fa_micro_lds_read"):
        getattr(lib, name).argtypes = [vp, i, i, vp]
        getattr(lib, name).restype = i
    lib.fa_micro_atomic_tiles.argtypes = [vp, i, i, i, vp]
    lib.fa_micro_atomic_tiles.restype = i
    lib.fa_micro_grid_blocks.restype = i
    return lib


def _run(gpu, fn, *args):
    import torch

    out = torch.full((BLOCKS * 256,), -1.0, dtype=torch.float32, device=gpu)
    assert fn(out.data_ptr(), BLOCKS, *args, None) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_grid_blocks(gpu, micro):
    import torch

    P.say("micro grid blocks")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert micro.fa_micro_grid_blocks() == 2 * cus


def test_mfma_loop_sums(gpu, micro):
    # every operand element is bf16 2^-10: one 32x32x16 product adds 16 * 2^-20 = 2^-16 to
    # each of a lane's 16 accumulators; 8 chains x 16 accumulators x iters products
    P.say("micro mfma")
    iters = 40
    out = _run(gpu, micro.fa_micro_mfma_bf16, iters)
    np.testing.assert_array_equal(out, np.float32(8 * 16 * iters * 2.0**-16))


def test_exp_loop_values(gpu, micro):
    # 16 chains x <- 2^(-x) per thread from x0 = 0.25 + 0.03 k + 1e-6 tid; the map is a
    # contraction (|d/dx| <= ln2 * 2^-0.25 < 0.6), so rounding differences stay small
    P.say("micro exp")
    iters = 25
    out = _run(gpu, micro.fa_micro_exp, iters)
    tid = np.arange(256, dtype=np.float64)
    x = 0.25 + 0.03 * np.arange(16)[:, None] + 1e-6 * tid[None, :]
    for _ in range(iters):
        x = np.exp2(-x)
    want = np.tile(x.sum(axis=0), BLOCKS)
    np.testing.assert_allclose(out, want, rtol=2e-5, atol=0)


def test_lds_read_xor(gpu, micro):
    # tile unit u (16 bytes) holds (u, 3u, 5u, 7u); thread t reads, per iteration i and
    # k < 8, unit (t % 64) + 64 (t // 64) + (i % 64) + 256 k, XOR-accumulating the words
    P.say("micro lds")
    iters = 70
    out = _run(gpu, micro.fa_micro_lds_read, iters)
    want = np.zeros(256)
    for t in range(256):
        acc = [0, 0, 0, 0]
        for i in range(iters):
            for k in range(8):
                u = (t % 64) + 64 * (t // 64) + (i % 64) + 256 * k
                acc = [a ^ (m * u) for a, m in zip(acc, (1, 3, 5, 7))]
        want[t] = float(acc[0] ^ acc[1] ^ acc[2] ^ acc[3])
    np.testing.assert_array_equal(out, np.tile(want, BLOCKS).astype(np.float32))


def test_atomic_tiles_counts(gpu, micro):
    # workgroup w adds 1.0 to every element of tiles (w + t) % ntiles, t < tiles: each
    # tile ends with the number of (w, t) pairs that hit it
    import torch

    P.say("micro atomics")
    ntiles, tiles, blocks = 5, 3, 7
    buf = torch.zeros(ntiles * 64 * 128, dtype=torch.float32, device=gpu)
    for _ in range(2):  # two calls accumulate
        assert micro.fa_micro_atomic_tiles(buf.data_ptr(), ntiles, blocks, tiles, None) == 0
    torch.cuda.synchronize()
    hits = np.zeros(ntiles)
    for w in range(blocks):
        for t in range(tiles):
            hits[(w + t) % ntiles] += 2
    got = buf.cpu().numpy().reshape(ntiles, 64 * 128)
    np.testing.assert_array_equal(got, np.repeat(hits[:, None], 64 * 128, axis=1).astype(np.float32))


def _chains(kind, iters):
    x = 0.25 + 0.03 * np.arange(16)[:, None] + 1e-6 * np.arange(256)[None, :]
    for _ in range(iters):
        x = np.exp2(-x) if kind == "exp" else x * 0.999 + 1e-4
    return x.sum(axis=0)


@pytest.mark.parametrize("mode", [1, 2, 3])
@pytest.mark.parametrize("valu_kind", [2, 3], ids=["exp_beside_fma", "exp_fma_one_wave"])
def test_coexec_exp_fma_values(gpu, micro, mode, valu_kind):
    # exp2 chains (mfma_iters iterations) and FMA chains (valu_iters) on two waves of one
    # SIMD (kind 2) or interleaved in one wave (kind 3); out: exp sums, then FMA sums
    import torch

    P.say(f"micro coexec mode {mode} kind {valu_kind}")
    micro.fa_micro_coexec.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    micro.fa_micro_coexec.restype = ctypes.c_int
    blocks, it_e, it_f = 3, 30, 40
    out = torch.full((blocks * 512,), -1.0, dtype=torch.float32, device=gpu)
    assert micro.fa_micro_coexec(out.data_ptr(), blocks, mode, valu_kind, it_e, it_f, None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(blocks, 512)
    for half, bit, kind, it in ((0, 1, "exp", it_e), (1, 2, "fma", it_f)):
        part = got[:, 256 * half:256 * (half + 1)]
        if mode & bit:
            np.testing.assert_allclose(part, np.tile(_chains(kind, it), (blocks, 1)), rtol=2e-5, atol=0)
        else:
            np.testing.assert_array_equal(part, np.float32(0))


@pytest.mark.parametrize("mode", [1, 2, 3])
@pytest.mark.parametrize("valu_kind", [0, 1], ids=["exp", "fma"])
def test_coexec_values(gpu, micro, mode, valu_kind):
    # waves 0-3: the MFMA chains (sum 8 * 16 * iters * 2^-16 per lane) when mode bit 0 is
    # set; waves 4-7: 16 chains per lane of exp2(-x) or fma(x, 0.999, 1e-4) when bit 1 is
    import torch

    P.say(f"micro coexec mode {mode} kind {valu_kind}")
    micro.fa_micro_coexec.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    micro.fa_micro_coexec.restype = ctypes.c_int
    blocks, it_m, it_v = 3, 30, 40
    out = torch.full((blocks * 512,), -1.0, dtype=torch.float32, device=gpu)
    assert micro.fa_micro_coexec(out.data_ptr(), blocks, mode, valu_kind, it_m, it_v, None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(blocks, 512)
    want_m = np.float32(8 * 16 * it_m * 2.0**-16) if mode & 1 else np.float32(0)
    np.testing.assert_array_equal(got[:, :256], want_m)
    if mode & 2:
        x = 0.25 + 0.03 * np.arange(16)[:, None] + 1e-6 * np.arange(256)[None, :]
        for _ in range(it_v):
            x = np.exp2(-x) if valu_kind == 0 else x * 0.999 + 1e-4
        np.testing.assert_allclose(got[:, 256:], np.tile(x.sum(axis=0), (blocks, 1)), rtol=2e-5, atol=0)
    else:
        np.testing.assert_array_equal(got[:, 256:], np.float32(0))


def _fp8_tile(gpu, micro, a8, b8, c0):
    import torch

    micro.fa_micro_mfma_fp8_tile.argtypes = [ctypes.c_void_p] * 5
    micro.fa_micro_mfma_fp8_tile.restype = ctypes.c_int
    ta = torch.from_numpy(np.ascontiguousarray(a8, dtype=np.uint8)).to(gpu)
    tb = torch.from_numpy(np.ascontiguousarray(b8, dtype=np.uint8)).to(gpu)
    tc0 = torch.from_numpy(np.ascontiguousarray(c0, dtype=np.float32)).to(gpu)
    tc = torch.full((32, 32), np.nan, dtype=torch.float32, device=gpu)
    assert micro.fa_micro_mfma_fp8_tile(ta.data_ptr(), tb.data_ptr(), tc0.data_ptr(), tc.data_ptr(), None) == 0
    torch.cuda.synchronize()
    return tc.cpu().numpy().astype(np.float64)


def _finite_codes(rng, shape, lo=0x00, hi=0x7E):
    """Random E4M3 codes with magnitude codes in [lo, hi] (0x7F, NaN, excluded), random sign."""
    mag = rng.integers(lo, hi, size=shape, endpoint=True).astype(np.uint8)
    return mag | (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)


def test_mfma_fp8_accumulation_precision(gpu, micro):
    """Exact products and sums of the fp8 product on a wide spread of magnitudes: one
    dominant product (448 x 448) per output beside 63 small ones, random codes, and a
    large accumulator start; reports the error relative to the largest |product| of each
    output.  Measured: at most 2^-11.8 of it (fp32 summation would stay within about
    2^-18); the FP8 forward's parity bound takes 2^-10, which this asserts."""
    from oracle import fp8 as O

    P.say("micro mfma fp8 precision")
    rng = np.random.default_rng(515)
    cases = {}
    a8, b8 = _finite_codes(rng, (32, 64)), _finite_codes(rng, (32, 64))
    cases["random"] = (a8, b8, np.zeros((32, 32)))
    a8, b8 = _finite_codes(rng, (32, 64), 0x08, 0x50), _finite_codes(rng, (32, 64), 0x08, 0x50)
    a8[:, 0], b8[:, 0] = 0x7E, 0x7E
    cases["dominant"] = (a8, b8, np.zeros((32, 32)))
    a8, b8 = _finite_codes(rng, (32, 64), 0x08, 0x50), _finite_codes(rng, (32, 64), 0x08, 0x50)
    a8[:, 0], b8[:, 0] = 0x7E, 0x7E
    a8[:, 1], b8[:, 1] = 0x7E, 0xFE  # +448^2 - 448^2: the small products are the exact sum
    cases["cancel"] = (a8, b8, np.zeros((32, 32)))
    a8, b8 = _finite_codes(rng, (32, 64), 0x08, 0x50), _finite_codes(rng, (32, 64), 0x08, 0x50)
    cases["big_start"] = (a8, b8, np.full((32, 32), 2.0**17))
    for name, (a8, b8, c0) in cases.items():
        a, b = O.e4m3_decode(a8), O.e4m3_decode(b8)
        exact = a @ b.T + c0
        got = _fp8_tile(gpu, micro, a8, b8, c0)
        big = np.maximum(np.max(np.abs(a[:, None, :] * b[None, :, :]), axis=2), np.abs(c0))
        err = np.abs(got - exact)
        rel = err / big
        small = exact - np.where(np.abs(c0) > 0, c0, 0.0)
        P.say(f"  {name}: max |err| {err.max():.3e}, max |err|/max|term| {rel.max():.3e} "
              f"(2^{np.log2(max(rel.max(), 1e-300)):.1f}), exact outputs {np.mean(err == 0):.2f}, "
              f"mean signed err/|small| {np.mean((got - exact) / np.maximum(np.abs(small), 1e-30)):.3e}")
        assert np.all(np.isfinite(got))
        assert rel.max() <= 2.0**-10, name


def test_mfma_order_sums_and_ticks(gpu, micro):
    """The product-order probe: chain k's products add u_k = 2^-16 (1 + k/128) to each of
    its accumulator elements, so each variant's per-thread total follows from its product
    counts (exact in fp32 at 20 blocks); the forward's order with LDS operands computes
    what it computes from registers; 32 products of 32 cycles each take at least 1024
    shader-clock ticks per block, and no order beats independent chains."""
    import torch

    vp, i = ctypes.c_void_p, ctypes.c_int
    micro.fa_micro_mfma_order.argtypes = [vp, vp, i, i, i, vp]
    micro.fa_micro_mfma_order.restype = i
    blocks, iters = 4, 20
    u = [2.0**-16 * (1 + k / 128) for k in range(8)]
    pv = sum(16 * 4 * iters * u[k] for k in range(4))  # P.V accumulators at the end
    expected = {
        0: pv + sum(16 * 4 * iters * u[4 + k] for k in range(4)),
        1: iters * (8 * u[4] + 8 * u[5]) + pv + 16 * 8 * (u[4] + u[5]),
        2: iters * ((4 * u[4] + 4 * u[6]) + (4 * u[5] + 4 * u[7])) + pv + 16 * 4 * sum(u[4:8]),
    }
    expected[3] = expected[1]

    def run(variant, n):
        ticks = torch.zeros(blocks * 4, dtype=torch.int64, device=gpu)
        sink = torch.full((blocks * 256,), -1.0, dtype=torch.float32, device=gpu)
        assert micro.fa_micro_mfma_order(ticks.data_ptr(), sink.data_ptr(), blocks, variant, n, None) == 0
        torch.cuda.synchronize()
        return ticks.cpu().numpy() / n, sink.cpu().numpy()

    per_block = {}
    for variant in range(4):
        P.say(f"micro mfma order variant {variant}")
        t, sink = run(variant, iters)
        np.testing.assert_array_equal(sink, np.float32(expected[variant]))
        assert (t >= 0.97 * 1024).all(), (variant, t)
        t, _ = run(variant, 400)
        assert (t >= 0.97 * 1024).all(), (variant, t)
        per_block[variant] = float(np.median(t))
    P.say(f"  ticks per 32 products (400 blocks): {per_block}")
    assert per_block[0] <= 1.25 * 1024
    assert min(per_block[1], per_block[2], per_block[3]) >= 0.98 * per_block[0]
