"""FP8 quantisation and FP8-input attention, plain CPU definitions -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may import this
module.  It shares no code with the HIP path and never touches a GPU.

What the pages fix
------------------
The FlashAttention-3 generation adds an FP8 forward with *block quantisation* and
*incoherent processing*, and reports an FP8 numerical error 2.6x below a baseline FP8
attention ("FlashAttention" concept wiki page, section FA3 (3) and the fourth
cross-cutting insight on FP8 stability: FP8 inputs with FP32 accumulation).  Nothing
more is on the pages: no format, block size, transform or error metric.  Readings taken
here (each listed with its reason in the design notes of the repository):

* FP8 format: OCP E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
  subnormals, no infinities, the all-ones exponent-and-mantissa pattern is NaN, largest
  finite 448.  Conversion from fp32 rounds to nearest, ties to even, and saturates at
  +-448 (the quantiser never asks for more than 448 before rounding).
* Block quantisation of Q and K: one fp32 scale per block of 64 consecutive rows of a
  head (the key/value tile the kernel streams); scale = amax / 448, code =
  e4m3(x * (448 / amax)), each a single fp32 operation.  A block of zeros has scale 0
  and codes 0.
* V: one fp32 scale per (head, head-dimension column) over all rows of the head, same
  formulas; the column scale multiplies output column c once at the end.
* Incoherent processing: rows of Q and K are multiplied by diag(signs) and then by the
  unnormalised d x d Sylvester-Hadamard matrix (entries +-1) before quantisation; signs
  is a random +-1 vector shared by Q and K, so (Q D H)(K D H)^T = d Q K^T.  The factor
  1/d is folded into Q's block scales (exact, d a power of two).  The transform is the
  fast Walsh-Hadamard butterfly in fp32 with a fixed order: stage h = 1, 2, 4, ..., d/2,
  pairs (i, i + h) inside blocks of 2h, (a, b) -> (a + b, a - b).  Every output is a
  fixed sequence of fp32 additions, so the GPU reaches the same bits.
* FP8 attention = exact attention (the plain fp64 definition in ``oracle.ref``) of the
  dequantised inputs code * scale.  The GPU additionally rounds P to E4M3 before P V;
  that rounding is not emulated (it depends on hardware exp2), and the tolerance of the
  tests is derived from its half-ulp instead.
"""

import numpy as np

from . import ref

__all__ = [
    "E4M3_MAX",
    "e4m3_encode",
    "e4m3_decode",
    "fwht_fp32",
    "quantize_blocks",
    "quantize_columns",
    "dequantize_blocks",
    "dequantize_columns",
    "attention_forward_fp8",
    "QBLOCK",
]

E4M3_MAX = 448.0
QBLOCK = 64  # rows per Q/K scale block


def e4m3_decode(codes):
    """fp64 values of OCP E4M3 codes (uint8 array); 0x7F and 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x):
    """Round fp32 values to OCP E4M3 codes: nearest, ties to even, saturating at +-448.

    Normal range (|x| >= 2^-6): the fp32 mantissa is rounded from 23 to 3 bits (RNE),
    which may carry into the exponent.  Subnormal range (|x| < 2^-6): the code is the
    integer rint(|x| * 2^9) in [0, 8] -- code 8 is the smallest normal, 2^-6.
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    sign = ((bits >> 31) & 1).astype(np.uint8)
    a = np.abs(x).astype(np.float32)
    abits = a.view(np.uint32).astype(np.uint64)
    # normal: RNE to 3 mantissa bits
    lsb = (abits >> 20) & 1
    r = (abits + 0x7FFFF + lsb) & ~np.uint64(0xFFFFF)
    exp = (r >> 23).astype(np.int64) - 127 + 7
    man = ((r >> 20) & 7).astype(np.int64)
    normal_code = (exp << 3) | man
    sub_code = np.rint(a.astype(np.float64) * 512.0).astype(np.int64)
    code = np.where(a < np.float32(2.0 ** -6), sub_code, normal_code)
    code = np.minimum(code, 0x7E)  # saturate at 448
    return (code.astype(np.uint8) | (sign << 7)).astype(np.uint8)


def fwht_fp32(x, signs=None):
    """Unnormalised fast Walsh-Hadamard transform of the last axis in fp32, after an
    optional multiplication by a +-1 sign vector.  Equals (x * signs) @ H_d for the
    Sylvester-Hadamard matrix H_d (H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]])."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    assert d & (d - 1) == 0, "d must be a power of two"
    if signs is not None:
        y = (y * np.asarray(signs, dtype=np.float32)).astype(np.float32)
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return y


def _amax_inv_scale(amax, post_scale):
    amax = np.asarray(amax, dtype=np.float32)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1.0))
    inv = np.where(nz, np.float32(E4M3_MAX) / safe, np.float32(0.0)).astype(np.float32)
    scale = np.where(nz, safe / np.float32(E4M3_MAX), np.float32(0.0)).astype(np.float32)
    scale = (scale * np.float32(post_scale)).astype(np.float32)
    return inv, scale


def quantize_blocks(x, signs=None, post_scale=1.0, block=QBLOCK):
    """Block quantisation of Q or K.

    x: [B,H,N,d] values (fp32-representable, e.g. bf16 inputs); signs: None (no
    rotation) or a +-1 vector of length d (incoherent processing).  Returns
    (codes uint8 [B,H,N,d], scales fp32 [B,H,ceil(N/block)]) with
    dequantised = code * scale.
    """
    y = np.asarray(x, dtype=np.float32)
    if signs is not None:
        y = fwht_fp32(y, signs)
    B, H, N, d = y.shape
    nb = -(-N // block)
    pad = nb * block - N
    yp = np.concatenate([y, np.zeros((B, H, pad, d), np.float32)], axis=2) if pad else y
    amax = np.abs(yp.reshape(B, H, nb, block * d)).max(axis=-1)
    inv, scale = _amax_inv_scale(amax, post_scale)
    inv_rows = np.repeat(inv, block, axis=2)[:, :, :N]
    codes = e4m3_encode((y * inv_rows[..., None]).astype(np.float32))
    return codes, scale


def quantize_columns(x):
    """Column quantisation of V: one scale per (b, h, column) over all N rows.

    Returns (codes uint8 [B,H,N,d], scales fp32 [B,H,d])."""
    y = np.asarray(x, dtype=np.float32)
    amax = np.abs(y).max(axis=2)  # [B,H,d]
    inv, scale = _amax_inv_scale(amax, 1.0)
    codes = e4m3_encode((y * inv[:, :, None, :]).astype(np.float32))
    return codes, scale


def dequantize_blocks(codes, scales, block=QBLOCK):
    N = codes.shape[2]
    s = np.repeat(np.asarray(scales, np.float64), block, axis=2)[:, :, :N]
    return e4m3_decode(codes) * s[..., None]


def dequantize_columns(codes, scales):
    return e4m3_decode(codes) * np.asarray(scales, np.float64)[:, :, None, :]


def attention_forward_fp8(q8, sq, k8, sk, v8, sv, scale, causal=False, kv_len=None):
    """Exact fp64 attention of the dequantised FP8 inputs: O [B,H,N,d], LSE [B,H,N]."""
    q = dequantize_blocks(q8, sq)
    k = dequantize_blocks(k8, sk)
    v = dequantize_columns(v8, sv)
    return ref.attention_forward(q, k, v, scale, causal=causal, kv_len=kv_len)
