"""The three hot-path pipelines as sequences of libcsa calls, with every output and workspace
allocated once up front (so a step allocates nothing and can be timed or graph-captured).

    CsaPrefill  compress KV + compress index keys -> index/top-k -> sparse MQA
    CsaDecode   index/top-k over a pre-compressed context -> sparse MQA (one new token per
                sequence); every m-th step the new token completes a block, and that step
                first compresses the block's KV entry and index-key entry from the state
                (the raw streams of the last two blocks) into the caches
    HcaChunk    HCA compression of the whole context -> dense causal MQA for a query chunk

Inputs are device tensors in their storage dtypes (bf16 as torch.bfloat16, fp8 e4m3fn as
torch.uint8 bytes, fp32).  Only marshalling happens here; the arithmetic is in libcsa.
"""
from __future__ import annotations

import math

import torch

from . import (CSA_KV_FP8_BF16, KVFp8Bf16, csa_compress, csa_compress_step_kv_index, csa_index_topk, csa_sparse_mqa,
               hca_compress, hca_dense_mqa, mqa_workspace_for, workspace_for)


class CsaPrefill:
    def __init__(self, inp: dict, m: int, k: int, q_pos0: int = 0, scale: float | None = None):
        self.inp, self.m, self.k, self.q_pos0 = inp, m, k, q_pos0
        Ca, q, qI = inp["Ca"], inp["q"], inp["qI"]
        batch, n, c = Ca.shape
        _, T, H, _ = q.shape
        H_I, c_I = qI.shape[2], qI.shape[3]
        N = n // m
        dev = Ca.device
        self.scale = 1.0 / math.sqrt(c) if scale is None else scale
        self.kv = torch.empty((batch, N, c), dtype=Ca.dtype, device=dev)
        self.kI = torch.empty((batch, N, c_I), dtype=inp["ICa"].dtype, device=dev)
        self.idx = torch.empty((batch, T, k), dtype=torch.int32, device=dev)
        self.sel = torch.empty((batch, T, k), dtype=torch.float32, device=dev)
        self.ws = workspace_for(batch, T, N, H_I, k, dev)
        self.mqa_ws = mqa_workspace_for(q, k)
        self.out = torch.empty_like(q)

    def compress(self):
        i = self.inp
        csa_compress(i["Ca"], i["Cb"], i["Za"], i["Zb"], i["Ba"], i["Bb"], self.m, out=self.kv)
        csa_compress(i["ICa"], i["ICb"], i["IZa"], i["IZb"], i["IBa"], i["IBb"], self.m, out=self.kI)

    def select(self):
        i = self.inp
        csa_index_topk(i["qI"], i["w"], self.kI, self.q_pos0, self.m, self.k, idx=self.idx, sel_scores=self.sel,
                       workspace=self.ws)

    def attend(self):
        csa_sparse_mqa(self.inp["q"], self.kv, self.idx, self.scale, out=self.out, workspace=self.mqa_ws)

    def run(self):
        self.compress()
        self.select()
        self.attend()
        return self.out


class CsaDecode:
    def __init__(self, inp: dict, m: int, k: int, q_pos0: int, scale: float | None = None):
        self.inp, self.m, self.k, self.q_pos0 = inp, m, k, q_pos0
        kv, q, qI = inp["kv"], inp["q"], inp["qI"]
        batch, N, c = kv.shape
        _, T, H, _ = q.shape
        H_I = qI.shape[2]
        dev = kv.device
        self.scale = 1.0 / math.sqrt(c) if scale is None else scale
        self.idx = torch.empty((batch, T, k), dtype=torch.int32, device=dev)
        self.sel = torch.empty((batch, T, k), dtype=torch.float32, device=dev)
        self.ws = workspace_for(batch, T, N, H_I, k, dev)
        self.mqa_ws = mqa_workspace_for(q, k, CSA_KV_FP8_BF16 if isinstance(kv, KVFp8Bf16) else None)
        self.out = torch.empty_like(q)

    def select(self):
        i = self.inp
        csa_index_topk(i["qI"], i["w"], i["kI"], self.q_pos0, self.m, self.k, idx=self.idx, sel_scores=self.sel,
                       workspace=self.ws)

    def attend(self):
        csa_sparse_mqa(self.inp["q"], self.inp["kv"], self.idx, self.scale, out=self.out, workspace=self.mqa_ws)

    def can_compress(self) -> bool:
        """The inputs hold a decode state for the KV and the index-key caches."""
        return all(nm in self.inp for nm in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb", "ICa", "ICb", "IZa", "IZb",
                                             "IBa", "IBb"))

    def compress(self):
        """The entries of the block the newest token completes: the block is the last one of
        the caches (entry N-1), computed from the state of its two blocks and written in place."""
        i = self.inp
        blk = i["kv"].shape[1] - 1
        csa_compress_step_kv_index([i[k] for k in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")], i["kv"],
                                   [i[k] for k in ("ICa", "ICb", "IZa", "IZb", "IBa", "IBb")], i["kI"], blk)

    def run(self):
        self.select()
        self.attend()
        return self.out

    def run_steps(self, compress: bool = True):
        """m decode steps: the last one's token completes a block, so that step compresses its
        entries first (one compression every m steps; compress=False leaves it out, to time the
        same steps without it)."""
        for j in range(self.m):
            if compress and j == self.m - 1:
                self.compress()
            self.select()
            self.attend()
        return self.out


class CsaCompress:
    """CSA compression of whole sequences (the step of a prefill that builds the KV cache)."""

    def __init__(self, inp: dict, m: int):
        self.inp, self.m = inp, m
        batch, n, c = inp["Ca"].shape
        self.kv = torch.empty((batch, n // m, c), dtype=inp["Ca"].dtype, device=inp["Ca"].device)

    def run(self):
        i = self.inp
        return csa_compress(i["Ca"], i["Cb"], i["Za"], i["Zb"], i["Ba"], i["Bb"], self.m, out=self.kv)


class HcaChunk:
    def __init__(self, inp: dict, m_prime: int, q_pos0: int, scale: float | None = None):
        self.inp, self.mp, self.q_pos0 = inp, m_prime, q_pos0
        C, q = inp["C"], inp["q"]
        batch, n, c = C.shape
        dev = C.device
        self.scale = 1.0 / math.sqrt(c) if scale is None else scale
        self.kv = torch.empty((batch, n // m_prime, c), dtype=C.dtype, device=dev)
        self.out = torch.empty_like(q)

    def compress(self):
        i = self.inp
        hca_compress(i["C"], i["Z"], i["B"], self.mp, out=self.kv)

    def attend(self):
        hca_dense_mqa(self.inp["q"], self.kv, self.q_pos0, self.mp, self.scale, out=self.out)

    def run(self):
        self.compress()
        self.attend()
        return self.out
