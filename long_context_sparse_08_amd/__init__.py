"""libcsa — CSA / HCA attention hot path (DeepSeek-V4 style) on AMD MI355X (gfx950).

A thin ctypes binding over `_build/libcsa.so`: each function checks the tensors it is
given, allocates outputs with torch when the caller passes none, and calls the C entry
point of the same name on torch's current HIP stream.  All computation happens in the HIP
kernels of the library; there is no CPU fallback.  Importing this module fails loudly if
the library has not been built (`python long_context_sparse_08_amd/build.py`).
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libcsa.so")

CSA_F32, CSA_BF16, CSA_FP8_E4M3, CSA_MXFP4, CSA_KV_FP8_BF16 = 0, 1, 2, 3, 4
STATUS = {0: "CSA_OK", -1: "CSA_ERR_INVALID_ARG", -2: "CSA_ERR_UNSUPPORTED", -3: "CSA_ERR_WORKSPACE",
          -4: "CSA_ERR_HIP", -5: "CSA_ERR_TOO_LARGE"}
NOALLOC_SCRATCH_BYTES = 32 << 20   # CSA_NOALLOC_SCRATCH_BYTES

ENTRY_POINTS = ("csa_compress", "hca_compress", "csa_index_topk_workspace_size", "csa_index_topk",
                "csa_index_topk_noalloc",
                "csa_index_scores", "csa_topk_workspace_size", "csa_topk", "csa_sparse_mqa_workspace_size", "csa_sparse_mqa",
                "hca_dense_mqa", "csa_sparse_mqa_sink", "hca_dense_mqa_sink", "csa_sparse_mqa_swa", "csa_rope", "csa_compress_step", "hca_dense_mqa_swa", "hca_compress_step", "csa_compress_step_kv_index", "csa_status_string",
                "csa_version")


class CsaError(RuntimeError):
    def __init__(self, name: str, status: int, msg: str):
        super().__init__(f"{name} failed with {STATUS.get(status, status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libcsa is not built ({LIB_PATH} missing); run `python long_context_sparse_08_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sig = {
        "csa_compress": ([P, P, P, P, P, P, I64, I64, I, I, I, P, I, P], I),
        "hca_compress": ([P, P, P, I64, I64, I, I, I, P, I, P], I),
        "csa_index_topk_workspace_size": ([I64, I64, I64, I, I], SZ),
        "csa_index_topk": ([P, P, P, I64, I64, I64, I64, I, I, I, I, I, P, P, P, SZ, P], I),
        "csa_index_topk_noalloc": ([P, P, P, I64, I64, I64, I64, I, I, I, I, I, P, P, P], I),
        "csa_index_scores": ([P, P, P, I64, I64, I64, I64, I, I, I, I, P, P], I),
        "csa_topk_workspace_size": ([I64, I64, I64, I], SZ),
        "csa_topk": ([P, I64, I64, I64, I64, I64, I, I, P, P, P, SZ, P], I),
        "csa_sparse_mqa_workspace_size": ([I64, I64, I, I, I, I], SZ),
        "csa_sparse_mqa": ([P, P, P, I64, I64, I64, I, I, I, F, I, P, P, SZ, P], I),
        "hca_dense_mqa": ([P, P, I64, I64, I64, I64, I, I, I, F, I, P, P], I),
        "csa_sparse_mqa_sink": ([P, P, P, I64, I64, I64, I, I, I, F, P, I, P, P, SZ, P], I),
        "csa_rope": ([P, I64, I64, I, I, I, I64, I64, F, I, I, P], I),
        "csa_compress_step": ([P, P, P, P, P, P, I64, I64, I, I, I, P, I64, I, P], I),
        "csa_sparse_mqa_swa": ([P, P, P, I64, I64, I64, I, I, I, F, P, P, I64, I64, I64, I, I, P, P, SZ, P], I),
        "hca_dense_mqa_sink": ([P, P, I64, I64, I64, I64, I, I, I, F, P, I, P, P], I),
        "hca_dense_mqa_swa": ([P, P, I64, I64, I64, I64, I, I, I, F, P, P, I64, I64, I, I, P, P], I),
        "hca_compress_step": ([P, P, P, I64, I64, I, I, I, P, I64, I, P], I),
        "csa_compress_step_kv_index": ([P, P, P, P, P, P, I, P, I64, I, P, P, P, P, P, P, I, P, I64, I, I64, I64, I, I, P],
                                       I),
        "csa_status_string": ([I], ctypes.c_char_p),
        "csa_version": ([], I),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()


def _check(name: str, rc: int):
    if rc != 0:
        raise CsaError(name, rc, lib.csa_status_string(rc).decode())


def _dt(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return CSA_F32
    if x.dtype == torch.bfloat16:
        return CSA_BF16
    if x.dtype in (torch.float8_e4m3fn, torch.uint8):
        return CSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {x.dtype}")


_TORCH_DT = {CSA_F32: torch.float32, CSA_BF16: torch.bfloat16}


class MXFP4:
    """An indexer operand in the library's MXFP4 storage (csa_dtype CSA_MXFP4): `data` is the
    flat uint8 device buffer (the E2M1 element bytes of every row, then every row's E8M0
    scales), `shape` the logical shape whose last dimension is the row length."""

    def __init__(self, data: torch.Tensor, shape):
        self.data = data
        self.shape = tuple(int(d) for d in shape)
        c = self.shape[-1]
        rows = 1
        for d in self.shape[:-1]:
            rows *= d
        if data.dtype != torch.uint8 or c % 32 != 0 or data.numel() != rows * (c // 2 + c // 32):
            raise ValueError(f"an MXFP4 buffer of logical shape {self.shape} holds {rows * (c // 2 + c // 32)} bytes")


class KVFp8Bf16:
    """KV entries in the library's mixed-precision storage (csa_dtype CSA_KV_FP8_BF16): `data`
    is a uint8 device tensor [batch, N, c + 64] whose rows hold c - 64 e4m3 bytes, then the
    last 64 values as bf16; `c` is the logical row length."""

    def __init__(self, data: torch.Tensor, c: int):
        self.data = data
        self.c = int(c)
        if data.dtype != torch.uint8 or data.dim() != 3 or data.shape[-1] != self.c + 64:
            raise ValueError(f"mixed KV rows of {tuple(data.shape)} bytes do not hold {c} values")
        self.shape = (data.shape[0], data.shape[1], self.c)
        self.device = data.device


def _qk(qI, kI):
    """(q tensor, k tensor, q shape, k shape, csa dtype) of the indexer operands."""
    if isinstance(qI, MXFP4) or isinstance(kI, MXFP4):
        if not (isinstance(qI, MXFP4) and isinstance(kI, MXFP4)):
            raise TypeError("qI and kI must both be MXFP4")
        return qI.data, kI.data, qI.shape, kI.shape, CSA_MXFP4
    _need(_dt(qI) == _dt(kI), "qI and kI must have one dtype")
    return qI, kI, tuple(qI.shape), tuple(kI.shape), _dt(qI)


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libcsa takes device tensors only")
        if not t.is_contiguous():
            raise ValueError("libcsa takes contiguous tensors only")
        dev = t.device if dev is None else dev
        if t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _check_out(t, shape, dtype, what):
    """A caller-supplied buffer must have exactly the shape and dtype the call reads or writes
    (the C ABI sees only its address)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{what}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _p(t):
    return None if t is None else t.data_ptr()


def version() -> int:
    return lib.csa_version()


def csa_compress(Ca, Cb, Za, Zb, Ba, Bb, m: int, out=None, out_dtype=None):
    """[batch, n, c] streams (f32/bf16), [m, c] fp32 biases -> [batch, n // m, c] (f32, bf16 or
    fp8 e4m3 as uint8)."""
    _need(Ca.dim() == 3, "streams are [batch, n, c]")
    batch, n, c = Ca.shape
    for nm, t in (("Cb", Cb), ("Za", Za), ("Zb", Zb)):
        _check_out(t, Ca.shape, Ca.dtype, nm)
    _check_out(Ba, (m, c), torch.float32, "Ba")
    _check_out(Bb, (m, c), torch.float32, "Bb")
    if out is not None:
        _need(tuple(out.shape) == (batch, n // m, c), f"out: expected shape {(batch, n // m, c)}")
    dev = _dev(Ca, Cb, Za, Zb, Ba, Bb, out)
    if out is None:
        out = torch.empty((batch, n // m, c), dtype=out_dtype or Ca.dtype, device=dev)
    _check("csa_compress", lib.csa_compress(_p(Ca), _p(Cb), _p(Za), _p(Zb), _p(Ba), _p(Bb), batch, n, m, c, _dt(Ca),
                                            _p(out), _dt(out), _stream(dev)))
    return out


def hca_compress(C, Z, B, m_prime: int, out=None, out_dtype=None):
    """[batch, n, c] stream and scores, [m', c] fp32 biases -> [batch, n // m', c]."""
    _need(C.dim() == 3, "streams are [batch, n, c]")
    batch, n, c = C.shape
    _check_out(Z, C.shape, C.dtype, "Z")
    _check_out(B, (m_prime, c), torch.float32, "B")
    if out is not None:
        _need(tuple(out.shape) == (batch, n // m_prime, c), f"out: expected shape {(batch, n // m_prime, c)}")
    dev = _dev(C, Z, B, out)
    if out is None:
        out = torch.empty((batch, n // m_prime, c), dtype=out_dtype or C.dtype, device=dev)
    _check("hca_compress", lib.hca_compress(_p(C), _p(Z), _p(B), batch, n, m_prime, c, _dt(C), _p(out), _dt(out),
                                            _stream(dev)))
    return out


def csa_index_topk_workspace_size(batch: int, T: int, N: int, H_I: int, k: int) -> int:
    return int(lib.csa_index_topk_workspace_size(batch, T, N, H_I, k))


def workspace_for(batch, T, N, H_I, k, device) -> torch.Tensor:
    nbytes = csa_index_topk_workspace_size(batch, T, N, H_I, k)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def csa_index_topk(qI, w, kI, q_pos0: int, m: int, k: int, idx=None, sel_scores=None, workspace=None,
                   want_scores: bool = True):
    """qI [batch, T, H_I, c_I], w [batch, T, H_I] fp32, kI [batch, N, c_I] -> (idx, sel_scores).
    qI and kI: tensors of one dtype (f32, bf16, e4m3 as uint8) or both MXFP4."""
    qt, kt, qs, ks, qk_dt = _qk(qI, kI)
    _need(len(qs) == 4 and len(ks) == 3, "qI is [batch, T, H_I, c_I], kI [batch, N, c_I]")
    batch, T, H_I, c_I = qs
    N = ks[1]
    _need(ks == (batch, N, c_I), f"kI: expected shape {(batch, N, c_I)}")
    _check_out(w, (batch, T, H_I), torch.float32, "w")
    _check_out(idx, (batch, T, k), torch.int32, "idx")
    _check_out(sel_scores, (batch, T, k), torch.float32, "sel_scores")
    if workspace is not None:
        _need(workspace.dtype == torch.uint8 and workspace.dim() == 1, "workspace is a flat uint8 tensor")
    dev = _dev(qt, w, kt, idx, sel_scores, workspace)
    if idx is None:
        idx = torch.empty((batch, T, k), dtype=torch.int32, device=dev)
    if sel_scores is None and want_scores:
        sel_scores = torch.empty((batch, T, k), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = workspace_for(batch, T, N, H_I, k, dev)
    _check("csa_index_topk", lib.csa_index_topk(_p(qt), _p(w), _p(kt), batch, T, q_pos0, N, H_I, c_I, m, k, qk_dt,
                                                _p(idx), _p(sel_scores), _p(workspace), workspace.numel(),
                                                _stream(dev)))
    return idx, sel_scores


def csa_index_topk_noalloc(qI, w, kI, q_pos0: int, m: int, k: int, idx=None, sel_scores=None,
                           want_scores: bool = True):
    """csa_index_topk without a workspace: the library's fixed per-GPU scratch serves instead
    (for callers that cannot allocate; calls on one GPU must not overlap).  Runs on the
    tensors' device, which must be torch's current device."""
    qt, kt, qs, ks, qk_dt = _qk(qI, kI)
    _need(len(qs) == 4 and len(ks) == 3, "qI is [batch, T, H_I, c_I], kI [batch, N, c_I]")
    batch, T, H_I, c_I = qs
    N = ks[1]
    _need(ks == (batch, N, c_I), f"kI: expected shape {(batch, N, c_I)}")
    _check_out(w, (batch, T, H_I), torch.float32, "w")
    _check_out(idx, (batch, T, k), torch.int32, "idx")
    _check_out(sel_scores, (batch, T, k), torch.float32, "sel_scores")
    dev = _dev(qt, w, kt, idx, sel_scores)
    if dev.index != torch.cuda.current_device():
        raise ValueError("csa_index_topk_noalloc runs on the current device: call torch.cuda.set_device first")
    if idx is None:
        idx = torch.empty((batch, T, k), dtype=torch.int32, device=dev)
    if sel_scores is None and want_scores:
        sel_scores = torch.empty((batch, T, k), dtype=torch.float32, device=dev)
    _check_out(idx, (batch, T, k), torch.int32, "idx")
    if sel_scores is not None:
        _check_out(sel_scores, (batch, T, k), torch.float32, "sel_scores")
    _check("csa_index_topk_noalloc", lib.csa_index_topk_noalloc(_p(qt), _p(w), _p(kt), batch, T, q_pos0, N, H_I, c_I,
                                                                m, k, qk_dt, _p(idx), _p(sel_scores), _stream(dev)))
    return idx, sel_scores


def csa_index_scores(qI, w, kI, q_pos0: int, m: int, scores=None):
    """The indexer scores alone: [batch, T, N] fp32, -inf where the entry is not visible."""
    qt, kt, qs, ks, qk_dt = _qk(qI, kI)
    _need(len(qs) == 4 and len(ks) == 3, "qI is [batch, T, H_I, c_I], kI [batch, N, c_I]")
    batch, T, H_I, c_I = qs
    N = ks[1]
    _need(ks == (batch, N, c_I), f"kI: expected shape {(batch, N, c_I)}")
    _check_out(w, (batch, T, H_I), torch.float32, "w")
    _check_out(scores, (batch, T, N), torch.float32, "scores")
    dev = _dev(qt, w, kt, scores)
    if scores is None:
        scores = torch.empty((batch, T, N), dtype=torch.float32, device=dev)
    _check("csa_index_scores", lib.csa_index_scores(_p(qt), _p(w), _p(kt), batch, T, q_pos0, N, H_I, c_I, m, qk_dt,
                                                    _p(scores), _stream(dev)))
    return scores


def csa_topk(scores, q_pos0: int, m: int, k: int, idx=None, sel_scores=None, workspace=None,
             want_scores: bool = True):
    """scores [batch, T, N] fp32 (N % 4 == 0 for 16-byte rows) -> (idx, sel_scores)."""
    _need(scores.dim() == 3 and scores.dtype == torch.float32, "scores are [batch, T, N] fp32")
    batch, T, N = scores.shape
    _need(N % 4 == 0, "score rows must hold a multiple of 4 entries (16-byte rows)")
    _check_out(idx, (batch, T, k), torch.int32, "idx")
    _check_out(sel_scores, (batch, T, k), torch.float32, "sel_scores")
    dev = _dev(scores, idx, sel_scores, workspace)
    if idx is None:
        idx = torch.empty((batch, T, k), dtype=torch.int32, device=dev)
    if sel_scores is None and want_scores:
        sel_scores = torch.empty((batch, T, k), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(int(lib.csa_topk_workspace_size(batch, T, N, k)), 16), dtype=torch.uint8,
                                device=dev)
    _check("csa_topk", lib.csa_topk(_p(scores), N, batch, T, q_pos0, N, m, k, _p(idx), _p(sel_scores),
                                    _p(workspace), workspace.numel(), _stream(dev)))
    return idx, sel_scores


def csa_sparse_mqa_workspace_size(batch: int, T: int, H: int, c: int, k: int, dtype: int) -> int:
    return int(lib.csa_sparse_mqa_workspace_size(batch, T, H, c, k, dtype))


def mqa_workspace_for(q: torch.Tensor, k: int, dtype: int | None = None):
    batch, T, H, c = q.shape
    nbytes = csa_sparse_mqa_workspace_size(batch, T, H, c, k, _dt(q) if dtype is None else dtype)
    return None if nbytes == 0 else torch.empty(nbytes, dtype=torch.uint8, device=q.device)


def _sink(sink, H, dev):
    if sink is None:
        return None
    _check_out(sink, (H,), torch.float32, "sink")
    _need(sink.device == dev and sink.is_contiguous(), "sink: a contiguous tensor on the call's device")
    return sink


def csa_sparse_mqa(q, kv, idx, scale: float, out=None, workspace=None, sink=None, window=None):
    """q [batch, T, H, c], kv [batch, N, c] (or KVFp8Bf16 with bf16 q), idx [batch, T, k] int32
    -> out [batch, T, H, c].  sink: optional fp32 [H] per-head sink logits (attention sink).
    window: optional (win_kv [batch, W, c], win_pos0, q_pos0, n_win), the sliding-window branch."""
    mixed = isinstance(kv, KVFp8Bf16)
    kvt = kv.data if mixed else kv
    _need(q.dim() == 4 and idx.dim() == 3, "q is [batch, T, H, c], idx [batch, T, k]")
    batch, T, H, c = q.shape
    N = kv.shape[1]
    k = idx.shape[2]
    if mixed:
        _need(q.dtype == torch.bfloat16 and kv.c == c and kvt.shape[0] == batch, "mixed KV rows take bf16 q of width c")
        dt = CSA_KV_FP8_BF16
    else:
        _check_out(kv, (batch, N, c), q.dtype, "kv")
        dt = _dt(q)
    _check_out(idx, (batch, T, k), torch.int32, "idx")
    _check_out(out, (batch, T, H, c), q.dtype, "out")
    wkv, W, wp0, qp0, n_win = None, 0, 0, 0, 0
    if window is not None:
        wkv, wp0, qp0, n_win = window
        _need(wkv.dim() == 3, "win_kv is [batch, W, c]")
        _check_out(wkv, (batch, wkv.shape[1], c), q.dtype, "win_kv")
        W = wkv.shape[1]
    _check_out(sink, (H,), torch.float32, "sink")
    dev = _dev(q, kvt, idx, out, workspace, wkv)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = mqa_workspace_for(q, k + n_win, dt)
    ws_bytes = 0 if workspace is None else workspace.numel()
    sk = _sink(sink, H, dev)
    _check("csa_sparse_mqa", lib.csa_sparse_mqa_swa(_p(q), _p(kvt), _p(idx), batch, T, N, H, c, k, float(scale), _p(sk),
                                                    _p(wkv), W, wp0, qp0, n_win, dt, _p(out), _p(workspace), ws_bytes,
                                                    _stream(dev)))
    return out


def csa_compress_step(Ca, Cb, Za, Zb, Ba, Bb, block: int, cache):
    """Decode-step CSA compression: the state streams [batch, 2m, c] (blocks block-1 and block;
    [batch, m, c] when block == 0) -> row `block` of cache [batch, rows, c], in place."""
    batch, m, c = _step_state(Ca, Cb, Za, Zb, Ba, Bb, block, cache, "KV")
    dev = _dev(Ca, Cb, Za, Zb, Ba, Bb, cache)
    _check("csa_compress_step", lib.csa_compress_step(_p(Ca), _p(Cb), _p(Za), _p(Zb), _p(Ba), _p(Bb), batch, block, m, c,
                                                      _dt(Ca), _p(cache), cache.shape[1], _dt(cache), _stream(dev)))
    return cache


def _step_state(Ca, Cb, Za, Zb, Ba, Bb, block: int, cache, what: str):
    # the checks of csa_compress_step for one state and its cache; returns (batch, m, c)
    _need(Ca.dim() == 3 and Ba.dim() == 2 and cache.dim() == 3,
          f"{what}: state [batch, rows, c], biases [m, c], cache 3-d")
    batch, ns, c = Ca.shape
    m = Ba.shape[0]
    _need(ns == (2 * m if block > 0 else m), f"{what} state: {2 * m if block > 0 else m} tokens per sequence")
    for nm, t in (("Cb", Cb), ("Za", Za), ("Zb", Zb)):
        _check_out(t, Ca.shape, Ca.dtype, f"{what} {nm}")
    _check_out(Ba, (m, c), torch.float32, f"{what} Ba")
    _check_out(Bb, (m, c), torch.float32, f"{what} Bb")
    _need(cache.shape[0] == batch and cache.shape[2] == c and 0 <= block < cache.shape[1],
          f"{what} cache: row `block` of [batch, rows, c]")
    return batch, m, c


def csa_compress_step_kv_index(kv_state, kv_cache, ki_state, ki_cache, block: int):
    """The decode-step compression of one CSA layer: kv_state = (Ca, Cb, Za, Zb, Ba, Bb) and
    ki_state = (ICa, ICb, IZa, IZb, IBa, IBb), each as csa_compress_step takes it, -> row `block`
    of kv_cache and of ki_cache, in place (one launch at m = 4; the same bits as two
    csa_compress_step calls)."""
    _need(len(kv_state) == 6 and len(ki_state) == 6, "states are (Ca, Cb, Za, Zb, Ba, Bb)")
    batch, m, c = _step_state(*kv_state, block, kv_cache, "KV")
    bi, mi, ci = _step_state(*ki_state, block, ki_cache, "index-key")
    _need(bi == batch and mi == m, "both states: the same batch and m")
    _need(ki_state[0].dtype == kv_state[0].dtype, "both states: the same dtype")
    dev = _dev(*kv_state, kv_cache, *ki_state, ki_cache)
    _check("csa_compress_step_kv_index",
           lib.csa_compress_step_kv_index(*[_p(t) for t in kv_state], c, _p(kv_cache), kv_cache.shape[1], _dt(kv_cache),
                                          *[_p(t) for t in ki_state], ci, _p(ki_cache), ki_cache.shape[1],
                                          _dt(ki_cache), batch, block, m, _dt(kv_state[0]), _stream(dev)))
    return kv_cache, ki_cache


def csa_rope(x, pos0: int, pos_step: int = 1, d: int = 64, base: float = 10000.0, inverse: bool = False):
    """Partial RoPE in place on x [batch, T, H, c] (or [batch, T, c] KV rows): the last d
    channels of row (b, t) turn by position pos0 + t * pos_step (inverse: its negative)."""
    dev = _dev(x)
    if x.dim() == 3:
        batch, T, c = x.shape
        H = 1
    else:
        batch, T, H, c = x.shape
    _check("csa_rope", lib.csa_rope(_p(x), batch, T, H, c, d, pos0, pos_step, float(base), 1 if inverse else 0, _dt(x),
                                    _stream(dev)))
    return x


def hca_dense_mqa(q, kv, q_pos0: int, m_prime: int, scale: float, out=None, sink=None, window=None):
    """q [batch, T, H, c], kv [batch, N, c] HCA entries -> out [batch, T, H, c] (dense causal MQA).
    sink: optional fp32 [H]; window: optional (win_kv [batch, W, c], win_pos0, n_win), the
    sliding-window branch over the raw rows at positions p - n_win + 1 .. p."""
    mixed = isinstance(kv, KVFp8Bf16)
    kvt = kv.data if mixed else kv
    _need(q.dim() == 4, "q is [batch, T, H, c]")
    batch, T, H, c = q.shape
    N = kv.shape[1]
    if mixed:
        _need(q.dtype == torch.bfloat16 and kv.c == c and kvt.shape[0] == batch, "mixed KV rows take bf16 q of width c")
        dt = CSA_KV_FP8_BF16
    else:
        _check_out(kv, (batch, N, c), q.dtype, "kv")
        dt = _dt(q)
    _check_out(out, (batch, T, H, c), q.dtype, "out")
    wkv, W, wp0, n_win = None, 0, 0, 0
    if window is not None:
        wkv, wp0, n_win = window
        _need(wkv.dim() == 3, "win_kv is [batch, W, c]")
        _check_out(wkv, (batch, wkv.shape[1], c), q.dtype, "win_kv")
        W = wkv.shape[1]
    _check_out(sink, (H,), torch.float32, "sink")
    dev = _dev(q, kvt, out, wkv)
    if out is None:
        out = torch.empty_like(q)
    sk = _sink(sink, H, dev)
    _check("hca_dense_mqa", lib.hca_dense_mqa_swa(_p(q), _p(kvt), batch, T, q_pos0, N, H, c, m_prime, float(scale),
                                                  _p(sk), _p(wkv), W, wp0, n_win, dt, _p(out), _stream(dev)))
    return out


def hca_compress_step(C, Z, B, block: int, cache):
    """Decode-step HCA compression: the state streams [batch, m', c] (the raw tokens of block
    `block`) -> row `block` of cache [batch, rows, c], in place."""
    _need(C.dim() == 3 and cache.dim() == 3, "state [batch, m', c], cache [batch, rows, c]")
    batch, mp, c = C.shape
    _check_out(Z, C.shape, C.dtype, "Z")
    _check_out(B, (mp, c), torch.float32, "B")
    _need(cache.shape[0] == batch and cache.shape[2] == c and 0 <= block < cache.shape[1], "cache: row `block` of [batch, rows, c]")
    dev = _dev(C, Z, B, cache)
    _check("hca_compress_step", lib.hca_compress_step(_p(C), _p(Z), _p(B), batch, block, mp, c, _dt(C), _p(cache),
                                                      cache.shape[1], _dt(cache), _stream(dev)))
    return cache
