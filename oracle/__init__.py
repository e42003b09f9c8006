"""Python face of the CPU oracle (oracle/csa_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg
use it to produce expected values.  The product package never imports it.

Every function takes numpy arrays holding the *stored* bytes (float32, bf16 as uint16,
e4m3fn as uint8) plus their dtype code, decodes them exactly to float64 in C, and returns
float64 results (compressed entries rounded to the requested storage dtype, as the
next stage would read them).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csa_oracle.c")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD_DIR, "libcsa_oracle.so")

F32, BF16, FP8, MXFP4, KV_FP8_BF16 = 0, 1, 2, 3, 4
KEEP_DOUBLE = -1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math; OpenMP across independent rows)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-Wall", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=False)
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        D = ctypes.c_double
        sig = {
            "oracle_num_threads": ([], I),
            "oracle_decode": ([P, I, I64, P], I),
            "oracle_decode_mxfp4": ([P, I64, I, P], I),
            "oracle_decode_kv_fp8_bf16": ([P, I64, I, P], I),
            "oracle_rope": ([P, I64, I64, I, I, I, I64, I64, D, I], None),
            "oracle_round": ([P, I, I64], I),
            "oracle_csa_compress": ([P, P, P, P, P, P, I64, I64, I, I, I, P], None),
            "oracle_hca_compress": ([P, P, P, I64, I64, I, I, I, P], None),
            "oracle_index_scores": ([P, P, P, I64, I64, P, I64, I, I, I, P], None),
            "oracle_topk": ([P, I64, I64, P, I64, I, I, P, P], None),
            "oracle_sparse_mqa": ([P, P, P, I64, I64, I64, I, I, I, D, P, P], None),
            "oracle_hca_dense_mqa": ([P, P, I64, I64, P, I64, I, I, I, D, P, P], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().oracle_num_threads()


def decode(a: np.ndarray, dtype: int) -> np.ndarray:
    """Stored values -> exact float64 (the oracle's own decoder)."""
    if isinstance(a, np.ndarray) and a.dtype == np.float64:
        return a
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, dtype=np.float64)
    if lib().oracle_decode(_p(a), dtype, a.size, _p(out)) != 0:
        raise ValueError(f"bad dtype {dtype}")
    return out


def decode_mxfp4(buf: np.ndarray, shape) -> np.ndarray:
    """MXFP4 storage (flat uint8: element bytes of every row, then the scales) of a tensor of
    logical shape `shape` (rows of shape[-1] values) -> exact float64 of that shape."""
    shape = tuple(int(d) for d in shape)
    c = shape[-1]
    rows = int(np.prod(shape[:-1]))
    buf = np.ascontiguousarray(buf, dtype=np.uint8).reshape(-1)
    if c % 32 != 0 or buf.size != rows * (c // 2 + c // 32):
        raise ValueError(f"MXFP4 buffer of {buf.size} bytes does not hold shape {shape}")
    out = np.empty(shape, dtype=np.float64)
    if lib().oracle_decode_mxfp4(_p(buf), rows, c, _p(out)) != 0:
        raise ValueError("bad MXFP4 shape")
    return out


def decode_kv_fp8_bf16(buf: np.ndarray, c: int) -> np.ndarray:
    """Mixed-precision KV rows (uint8 [..., c + 64]: c - 64 e4m3 bytes, then 64 bf16 values)
    -> exact float64 [..., c]."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    if c < 64 or buf.shape[-1] != c + 64:
        raise ValueError(f"rows of {buf.shape[-1]} bytes do not hold {c} mixed values")
    rows = int(np.prod(buf.shape[:-1]))
    out = np.empty(buf.shape[:-1] + (c,), dtype=np.float64)
    if lib().oracle_decode_kv_fp8_bf16(_p(buf), rows, c, _p(out)) != 0:
        raise ValueError("bad mixed KV shape")
    return out


def rope(x, pos0: int, pos_step: int = 1, d: int = 64, base: float = 10000.0, inverse: bool = False,
         dtype: int = F32):
    """Partial RoPE of x [batch, T, H, c] (or [batch, T, c]) -> float64, same shape."""
    out = np.array(_d(x, dtype), dtype=np.float64, copy=True, order="C")
    shp = out.shape
    batch, T = shp[0], shp[1]
    H, c = (1, shp[2]) if out.ndim == 3 else (shp[2], shp[3])
    lib().oracle_rope(_p(out), batch, T, H, c, d, pos0, pos_step, float(base), 1 if inverse else 0)
    return out


def round_to(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float64 values to the nearest value of storage type `dtype` (f32, bf16 or fp8 e4m3fn,
    nearest-even, fp8 saturating at +-448)."""
    out = np.array(x, dtype=np.float64, copy=True, order="C")
    if lib().oracle_round(_p(out), dtype, out.size) != 0:
        raise ValueError(f"bad dtype {dtype}")
    return out


def _d(a, dtype):
    return np.ascontiguousarray(decode(a, dtype), dtype=np.float64)


def csa_compress(Ca, Cb, Za, Zb, Ba, Bb, m: int, in_dtype: int = F32, out_dtype: int = KEEP_DOUBLE):
    """[batch, n, c] streams -> [batch, n // m, c] compressed entries (float64)."""
    Ca, Cb, Za, Zb = (_d(x, in_dtype) for x in (Ca, Cb, Za, Zb))
    Ba, Bb = _d(Ba, F32), _d(Bb, F32)
    batch, n, c = Ca.shape
    assert Ba.shape == (m, c) and Bb.shape == (m, c)
    out = np.empty((batch, n // m, c), dtype=np.float64)
    lib().oracle_csa_compress(_p(Ca), _p(Cb), _p(Za), _p(Zb), _p(Ba), _p(Bb), batch, n, m, c, out_dtype,
                              _p(out))
    return out


def hca_compress(C, Z, B, m_prime: int, in_dtype: int = F32, out_dtype: int = KEEP_DOUBLE):
    C, Z = _d(C, in_dtype), _d(Z, in_dtype)
    B = _d(B, F32)
    batch, n, c = C.shape
    assert B.shape == (m_prime, c)
    out = np.empty((batch, n // m_prime, c), dtype=np.float64)
    lib().oracle_hca_compress(_p(C), _p(Z), _p(B), batch, n, m_prime, c, out_dtype, _p(out))
    return out


def _qpos(T, q_pos0, qpos):
    if qpos is None:
        qpos = q_pos0 + np.arange(T, dtype=np.int64)
    qpos = np.ascontiguousarray(qpos, dtype=np.int64)
    assert qpos.shape == (T,)
    return qpos


def index_scores(qI, w, kI, m: int, q_pos0: int = 0, qk_dtype: int = F32, qpos=None):
    """Indexer scores [batch, T, N]; -inf where the entry is not visible to the query."""
    qI, kI = _d(qI, qk_dtype), _d(kI, qk_dtype)
    w = _d(w, F32)
    batch, T, H_I, c_I = qI.shape
    N = kI.shape[1]
    assert kI.shape == (batch, N, c_I) and w.shape == (batch, T, H_I)
    qp = _qpos(T, q_pos0, qpos)
    out = np.empty((batch, T, N), dtype=np.float64)
    lib().oracle_index_scores(_p(qI), _p(w), _p(kI), batch, T, _p(qp), N, H_I, c_I, m, _p(out))
    return out


def topk(scores, m: int, k: int, q_pos0: int = 0, qpos=None):
    """(idx int32 [batch, T, k] ascending, -1 padded; sel float64 [batch, T, k])."""
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    batch, T, N = scores.shape
    qp = _qpos(T, q_pos0, qpos)
    idx = np.empty((batch, T, k), dtype=np.int32)
    sel = np.empty((batch, T, k), dtype=np.float64)
    lib().oracle_topk(_p(scores), batch, T, _p(qp), N, m, k, _p(idx), _p(sel))
    return idx, sel


def _sink(sink, H):
    """Per-head sink logits as float64 [H] (None: no sink)."""
    if sink is None:
        return None
    s = np.ascontiguousarray(sink, dtype=np.float64)
    assert s.shape == (H,)
    return s


def sparse_mqa(q, kv, idx, scale: float, dtype: int = F32, sink=None, window=None):
    """window: (win_kv [batch, W, c], win_pos0, q_pos0, n_win) — the sliding-window branch (the
    notes page §1.3): query t (position p = q_pos0 + t) also attends, in the same softmax, to
    the raw rows at positions p - n_win + 1 .. p that win_kv holds.  Written as the plain
    union: the raw rows are appended to the entries and their ids to the row's list."""
    q, kv = _d(q, dtype), _d(kv, dtype)
    if window is not None:
        wkv, wp0, qp0, n_win = window
        wkv = _d(wkv, dtype)
        batch, T = q.shape[0], q.shape[1]
        N, W = kv.shape[1], wkv.shape[1]
        idx = np.where((idx >= 0) & (idx < N), idx, -1).astype(np.int32)
        wid = np.full((batch, T, n_win), -1, np.int32)
        for t in range(T):
            for j in range(n_win):
                pw = qp0 + t - n_win + 1 + j
                if pw >= 0 and wp0 <= pw < wp0 + W:
                    wid[:, t, j] = N + (pw - wp0)
        kv = np.concatenate([kv, wkv], axis=1)
        idx = np.concatenate([idx, wid], axis=2)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    batch, T, H, c = q.shape
    N = kv.shape[1]
    k = idx.shape[2]
    assert kv.shape == (batch, N, c) and idx.shape == (batch, T, k)
    out = np.empty((batch, T, H, c), dtype=np.float64)
    sk = _sink(sink, H)
    lib().oracle_sparse_mqa(_p(q), _p(kv), _p(idx), batch, T, N, H, c, k, float(scale),
                            None if sk is None else _p(sk), _p(out))
    return out


def hca_dense_mqa(q, kv, m_prime: int, scale: float, q_pos0: int = 0, dtype: int = F32, qpos=None, sink=None,
                  window=None):
    """Dense causal MQA over the HCA entries each query may see (m'(s+1)-1 <= p).
    window: (win_kv [batch, W, c], win_pos0, n_win) — the sliding-window branch, which the notes
    page §1.3 gives to HCA as to CSA: written as the plain union, i.e. the query's visible
    entries listed explicitly and handed, with the window, to the sparse oracle."""
    if window is not None:
        assert qpos is None
        wkv, wp0, n_win = window
        batch, T = q.shape[0], q.shape[1]
        N = kv.shape[1]
        idx = np.full((batch, T, max(N, 1)), -1, np.int32)
        for t in range(T):
            nv = min(N, (q_pos0 + t + 1) // m_prime)
            idx[:, t, :nv] = np.arange(nv, dtype=np.int32)
        return sparse_mqa(q, kv, idx, scale, dtype=dtype, sink=sink, window=(wkv, wp0, q_pos0, n_win))
    q, kv = _d(q, dtype), _d(kv, dtype)
    batch, T, H, c = q.shape
    N = kv.shape[1]
    assert kv.shape == (batch, N, c)
    qp = _qpos(T, q_pos0, qpos)
    out = np.empty((batch, T, H, c), dtype=np.float64)
    sk = _sink(sink, H)
    lib().oracle_hca_dense_mqa(_p(q), _p(kv), batch, T, _p(qp), N, H, c, m_prime, float(scale),
                               None if sk is None else _p(sk), _p(out))
    return out
