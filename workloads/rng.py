"""Seeded, counter-based synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and stores them in the storage dtypes the kernels read
(fp32, bf16, OCP fp8 e4m3fn, OCP MXFP4, and KV rows mixing fp8 and bf16).  It holds none of the attention method's arithmetic: no
softmax, no pooling, no scoring.  Both the HIP path and the CPU oracle receive the very
bytes produced here.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; finaliser constants as published by Vigna for splitmix64.c)
used in counter mode.  Element i of tensor `tid` under `seed` is

    key   = mix64(mix64(seed) ^ tid)
    u64_i = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)          (mod 2**64)

so any element can be produced independently of the others (chunked, multi-threaded,
bit-reproducible).  Uniforms take the top 53 bits: u = (u64 >> 11) * 2**-53 in [0, 1).
Normals use the Box-Muller transform on the pair of uniforms drawn at counters 2i and
2i + 1:  z_i = sqrt(-2 ln(1 - u_2i)) * cos(2 pi u_{2i+1}), evaluated in float64.

Rounding to storage: float64 -> float32 (IEEE round-to-nearest-even), then
float32 -> bf16 round-to-nearest-even on the bit pattern, or float32 -> e4m3fn
round-to-nearest-even with saturation to +-448, or float32 -> MXFP4 (OCP Microscaling
Formats v1.0: blocks of 32 consecutive values of a row share one E8M0 scale 2^X with
X = floor(log2(max |v|)) - 2, the largest E2M1 exponent; each v / 2^X is rounded to the
nearest E2M1 value, ties to the even code, saturating at +-6).

MXFP4 storage of a tensor whose rows hold c values (c % 32 == 0): all rows' element bytes
first, c/2 bytes per row with value 2i in the low nibble of byte i and 2i+1 in the high
nibble, then all rows' scales, c/32 E8M0 bytes per row; one flat uint8 array.

Mixed-precision KV storage (fp8 + bf16) of rows of c values: per row c - 64 e4m3fn bytes
(values 0 .. c-65), then the last 64 values as bf16 (little-endian): c + 64 bytes a row,
uint8 [..., c + 64].  Each part is rounded as its dtype alone.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Storage dtype codes; the values match the C-ABI enum csa_dtype.
F32, BF16, FP8, MXFP4, KV_FP8_BF16 = 0, 1, 2, 3, 4
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8_e4m3", MXFP4: "mxfp4", KV_FP8_BF16: "kv_fp8_bf16"}
KV_ROPE = 64   # trailing values of a mixed KV row kept in bf16
MX_BLOCK = 32
NP_STORAGE = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}

_CHUNK = 1 << 20


def mix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = (x ^ (x >> np.uint64(30))) * _M1
        x = (x ^ (x >> np.uint64(27))) * _M2
    return x ^ (x >> np.uint64(31))


def stream_key(seed: int, tid: int) -> np.uint64:
    k = mix64(np.array([seed], dtype=np.uint64))[0]
    return mix64(np.array([k ^ np.uint64(tid)], dtype=np.uint64))[0]


def raw_u64(seed: int, tid: int, start: int, count: int) -> np.ndarray:
    key = stream_key(seed, tid)
    ctr = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(key + ctr * GOLDEN)


def _uniform_chunk(seed, tid, start, count):
    return (raw_u64(seed, tid, start, count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def _normal_chunk(seed, tid, start, count):
    u = _uniform_chunk(seed, tid, 2 * start, 2 * count)
    u1 = 1.0 - u[0::2]
    u2 = u[1::2]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


# ---------------------------------------------------------------- storage rounding
def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (NaN kept quiet)."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    with np.errstate(over="ignore"):
        out = ((b + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_grid():
    # all finite non-negative e4m3fn values, ascending, with their codes
    vals, codes = [], []
    for code in range(0x7F):  # 0x7F is NaN
        e, mant = code >> 3, code & 7
        v = mant * 2.0 ** -9 if e == 0 else (1 + mant / 8) * 2.0 ** (e - 7)
        vals.append(v)
        codes.append(code)
    return np.array(vals), np.array(codes, dtype=np.uint8)


_E4M3_VALS, _E4M3_CODES = _e4m3_grid()


def f32_to_e4m3_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn code, round to nearest even, saturating at +-448."""
    x = np.asarray(x32, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_E4M3_VALS, a, side="left")  # first grid value >= a
    hi = np.minimum(hi, len(_E4M3_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    vhi, vlo = _E4M3_VALS[hi], _E4M3_VALS[lo]
    exact = vhi == a
    dlo, dhi = a - vlo, vhi - a
    pick_hi = exact | (dhi < dlo) | ((dhi == dlo) & ((_E4M3_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _E4M3_CODES[hi], _E4M3_CODES[lo]).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    return code | sign


def e4m3_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    mag = _E4M3_VALS[np.minimum(b & 0x7F, 0x7E)].astype(np.float32)
    mag = np.where((b & 0x7F) == 0x7F, np.float32(np.nan), mag)
    return np.where(b & 0x80, -mag, mag).astype(np.float32)


# E2M1 magnitudes by code 0..7 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit;
# exponent 0 is subnormal: 0.5 * mantissa)
_E2M1_VALS = np.array([(m * 0.5) if e == 0 else (1 + m / 2) * 2.0 ** (e - 1) for e in range(4) for m in range(2)])


def f32_to_mxfp4(x32: np.ndarray) -> np.ndarray:
    """float32 [..., c] -> MXFP4 storage (flat uint8: element bytes of every row, then scales)."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    c = x.shape[-1]
    assert c % MX_BLOCK == 0
    blocks = x.reshape(-1, c // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    # floor(log2(amax)) exactly from the binary exponent (frexp: amax = f * 2^e, f in [0.5, 1))
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.clip(np.where(amax > 0, e - 1 - 2, -127), -127, 127)
    scaled = blocks / np.ldexp(1.0, X)[..., None]
    a = np.minimum(np.abs(scaled), 6.0)
    hi = np.minimum(np.searchsorted(_E2M1_VALS, a, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    vhi, vlo = _E2M1_VALS[hi], _E2M1_VALS[lo]
    pick_hi = (vhi == a) | (vhi - a < a - vlo) | ((vhi - a == a - vlo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8) | (np.signbit(scaled).astype(np.uint8) << np.uint8(3))
    code = code.reshape(-1, c)
    packed = (code[:, 0::2] | (code[:, 1::2] << np.uint8(4))).astype(np.uint8)
    scales = (X + 127).astype(np.uint8).reshape(-1, c // MX_BLOCK)
    return np.concatenate([packed.reshape(-1), scales.reshape(-1)])


def mxfp4_to_f32(buf: np.ndarray, rows: int, c: int) -> np.ndarray:
    """MXFP4 storage of `rows` rows of c values -> float32 [rows, c] (scale 255 is NaN)."""
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    assert buf.size == rows * (c // 2 + c // MX_BLOCK)
    packed = buf[: rows * c // 2].reshape(rows, c // 2)
    scales = buf[rows * c // 2:].reshape(rows, c // MX_BLOCK).astype(np.int64)
    code = np.empty((rows, c), dtype=np.uint8)
    code[:, 0::2] = packed & 0xF
    code[:, 1::2] = packed >> 4
    mag = _E2M1_VALS[code & 7]
    v = np.where(code & 8, -mag, mag) * np.repeat(np.ldexp(1.0, scales - 127), MX_BLOCK, axis=1)
    v = np.where(np.repeat(scales == 255, MX_BLOCK, axis=1), np.nan, v)
    return v.astype(np.float32)


def mxfp4_rows(buf: np.ndarray, rows: int, c: int, r0: int, r1: int) -> np.ndarray:
    """Rows r0 .. r1-1 of an MXFP4 storage of `rows` rows of c values, as a storage of their own."""
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    eb, sb = c // 2, c // MX_BLOCK
    return np.concatenate([buf[r0 * eb:r1 * eb], buf[rows * eb + r0 * sb:rows * eb + r1 * sb]])


def f32_to_kv_fp8_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 [..., c] -> mixed KV storage uint8 [..., c + 64]."""
    x32 = np.asarray(x32, dtype=np.float32)
    c = x32.shape[-1]
    assert c >= KV_ROPE
    out = np.empty(x32.shape[:-1] + (c + KV_ROPE,), dtype=np.uint8)
    out[..., : c - KV_ROPE] = f32_to_e4m3_bits(x32[..., : c - KV_ROPE])
    bf = np.ascontiguousarray(f32_to_bf16_bits(x32[..., c - KV_ROPE:]).astype("<u2"))
    out[..., c - KV_ROPE:] = bf.view(np.uint8).reshape(x32.shape[:-1] + (2 * KV_ROPE,))
    return out


def kv_fp8_bf16_to_f32(buf: np.ndarray, c: int) -> np.ndarray:
    """Mixed KV storage uint8 [..., c + 64] -> float32 [..., c]."""
    buf = np.asarray(buf, dtype=np.uint8)
    assert buf.shape[-1] == c + KV_ROPE
    out = np.empty(buf.shape[:-1] + (c,), dtype=np.float32)
    out[..., : c - KV_ROPE] = e4m3_bits_to_f32(buf[..., : c - KV_ROPE])
    bf = np.ascontiguousarray(buf[..., c - KV_ROPE:]).view("<u2")
    out[..., c - KV_ROPE:] = bf16_bits_to_f32(bf)
    return out


def to_storage(x64: np.ndarray, dtype: int) -> np.ndarray:
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return x32
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    if dtype == FP8:
        return f32_to_e4m3_bits(x32)
    raise ValueError(dtype)


def storage_to_f32(a: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.asarray(a, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits_to_f32(a)
    if dtype == FP8:
        return e4m3_bits_to_f32(a)
    raise ValueError(dtype)


# ---------------------------------------------------------------- tensor draws
def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def _fill(shape, dtype, fn):
    count = int(np.prod(shape))
    out = np.empty(count, dtype=NP_STORAGE[dtype])
    starts = list(range(0, count, _CHUNK))

    def work(s):
        e = min(count, s + _CHUNK)
        out[s:e] = to_storage(fn(s, e - s), dtype)

    if len(starts) <= 1:
        for s in starts:
            work(s)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, starts))
    return out.reshape(shape)


def normal(seed: int, tid: int, shape, dtype: int = F32, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) samples in storage dtype `dtype`, as a numpy array of the storage type
    (MXFP4: the flat storage of rows of shape[-1] values; the same draws as the other dtypes)."""
    if dtype == MXFP4:
        return f32_to_mxfp4(_fill(shape, F32, lambda s, c: std * _normal_chunk(seed, tid, s, c)))
    if dtype == KV_FP8_BF16:   # uint8 [..., c + 64]; drawn and converted a block of rows at a time
        c = int(shape[-1])
        rows = int(np.prod(shape[:-1]))
        out = np.empty((rows, c + KV_ROPE), dtype=np.uint8)
        step = max(1, _CHUNK // c)

        def work(r0):
            r1 = min(rows, r0 + step)
            x = (std * _normal_chunk(seed, tid, r0 * c, (r1 - r0) * c)).astype(np.float32)
            out[r0:r1] = f32_to_kv_fp8_bf16(x.reshape(r1 - r0, c))

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(0, rows, step)))
        return out.reshape(tuple(shape[:-1]) + (c + KV_ROPE,))
    return _fill(shape, dtype, lambda s, c: std * _normal_chunk(seed, tid, s, c))


def uniform(seed: int, tid: int, shape, dtype: int = F32, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    return _fill(shape, dtype, lambda s, c: lo + (hi - lo) * _uniform_chunk(seed, tid, s, c))
