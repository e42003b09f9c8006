"""The five workload shapes and the recipe that fills them with seeded synthetic values.

Shapes mirror DeepSeek-V4-Flash (top-k 512) and V4-Pro (top-k 1024, 1M context) as
listed in the model-configuration table of the notes page "DeepSeek-V4: 迈向高效百万级上下文
智能" (notes.kuangjux.top).  The pages evaluate on 1M-token quality suites that need
trained weights; these tensors stand in for them with the same shapes and no data from
any suite.  Distributions: streams, queries and keys ~N(0,1); position biases
~N(0, 0.1^2); indexer head weights ~U(0,1).  Seed of config i is 1000 + i; each tensor
has a fixed id (the TID table below).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import rng

F32, BF16, FP8, MXFP4, KV_FP8_BF16 = rng.F32, rng.BF16, rng.FP8, rng.MXFP4, rng.KV_FP8_BF16

# tensor ids, fixed forever (changing one changes every input)
TID = {
    "Ca": 1, "Cb": 2, "Za": 3, "Zb": 4, "Ba": 5, "Bb": 6,
    "ICa": 7, "ICb": 8, "IZa": 9, "IZb": 10, "IBa": 11, "IBb": 12,
    "q": 13, "qI": 14, "w": 15,
    "kv": 16, "kI": 17,
    "C": 18, "Z": 19, "B": 20,
}


@dataclass
class Config:
    name: str
    kind: str            # "csa_prefill" | "csa_decode" | "hca_chunk"
    batch: int
    dt: int              # storage dtype of streams, compressed entries, q and outputs
    c: int               # KV width (head dim)
    H: int               # query heads
    k: int = 0           # top-k
    n: int = 0           # raw tokens compressed in this config (0: context given pre-compressed)
    m: int = 4           # CSA compression ratio
    m_prime: int = 128   # HCA compression ratio
    H_I: int = 0         # indexer heads
    c_I: int = 0         # indexer head dim
    qk_dt: int = F32     # indexer q / key dtype
    kv_dt: int = -1      # storage of the compressed KV entries given to decode (-1: dt)
    T: int = 0           # query tokens per sequence
    q_pos0: int = 0      # absolute position of query 0
    N: int = 0           # compressed entries per sequence
    seed: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.c)


CONFIGS = {
    "cfg0_tiny": Config("cfg0_tiny", "csa_prefill", batch=1, dt=F32, c=64, H=4, k=8, n=256, m=4,
                        H_I=2, c_I=32, qk_dt=F32, T=256, q_pos0=0, N=64, seed=1000),
    "cfg1_csa_prefill": Config("cfg1_csa_prefill", "csa_prefill", batch=1, dt=BF16, c=512, H=64, k=512,
                               n=8192, m=4, H_I=64, c_I=128, qk_dt=BF16, T=8192, q_pos0=0, N=2048,
                               seed=1001),
    "cfg2_csa_decode_128k": Config("cfg2_csa_decode_128k", "csa_decode", batch=32, dt=BF16, c=512, H=128,
                                   k=1024, m=4, H_I=64, c_I=128, qk_dt=FP8, T=1, q_pos0=131072,
                                   N=32768, seed=1002),
    "cfg3_hca_chunk_1m": Config("cfg3_hca_chunk_1m", "hca_chunk", batch=1, dt=BF16, c=512, H=64,
                                n=1 << 20, m_prime=128, T=4096, q_pos0=(1 << 20) - 4096, N=8192,
                                seed=1003),
    "cfg4_csa_decode_1m": Config("cfg4_csa_decode_1m", "csa_decode", batch=8, dt=BF16, c=512, H=128,
                                 k=1024, m=4, H_I=64, c_I=128, qk_dt=FP8, T=1, q_pos0=1 << 20,
                                 N=262144, seed=1004),
    # the decode at a 128K context with the indexer's q and keys in MXFP4 (the notes page's
    # §2.4: the indexer's QK path in FP4); the same seed and draws as the fp8 decode, so its
    # selection can be compared with that one
    "cfg2_csa_decode_128k_mxfp4": Config("cfg2_csa_decode_128k_mxfp4", "csa_decode", batch=32, dt=BF16, c=512,
                                         H=128, k=1024, m=4, H_I=64, c_I=128, qk_dt=MXFP4, T=1,
                                         q_pos0=131072, N=32768, seed=1002),
    # CSA compression alone over a 1M-token sequence (4 GiB of bf16 streams): the compressor's
    # bandwidth at full size; T counts the raw tokens compressed per step
    "s1_csa_compress_1m": Config("s1_csa_compress_1m", "csa_compress", batch=1, dt=BF16, c=512, H=0, n=1 << 20, m=4,
                                 T=1 << 20, seed=1005),
    # the decode at a 128K context with the KV entries in the mixed storage (the notes page's
    # §1.3: RoPE channels in bf16, the others in fp8); same seed and draws as the bf16 decode
    "cfg2_csa_decode_128k_kvmixed": Config("cfg2_csa_decode_128k_kvmixed", "csa_decode", batch=32, dt=BF16, c=512,
                                           H=128, k=1024, m=4, H_I=64, c_I=128, qk_dt=FP8, T=1,
                                           q_pos0=131072, N=32768, seed=1002, kv_dt=KV_FP8_BF16),
}
ORDER = list(CONFIGS)


def shapes(cfg: Config) -> dict:
    """name -> (shape, dtype, distribution) for every input tensor of `cfg`."""
    B, c = cfg.batch, cfg.c
    s = {}
    if cfg.kind == "csa_prefill":
        n, m, cI = cfg.n, cfg.m, cfg.c_I
        for nm in ("Ca", "Cb", "Za", "Zb"):
            s[nm] = ((B, n, c), cfg.dt, ("normal", 1.0))
        for nm in ("Ba", "Bb"):
            s[nm] = ((m, c), F32, ("normal", 0.1))
        for nm in ("ICa", "ICb", "IZa", "IZb"):
            s[nm] = ((B, n, cI), cfg.dt, ("normal", 1.0))
        for nm in ("IBa", "IBb"):
            s[nm] = ((m, cI), F32, ("normal", 0.1))
    if cfg.kind == "csa_compress":
        for nm in ("Ca", "Cb", "Za", "Zb"):
            s[nm] = ((B, cfg.n, c), cfg.dt, ("normal", 1.0))
        for nm in ("Ba", "Bb"):
            s[nm] = ((cfg.m, c), F32, ("normal", 0.1))
    if cfg.kind == "csa_decode":
        s["kv"] = ((B, cfg.N, c), cfg.dt if cfg.kv_dt < 0 else cfg.kv_dt, ("normal", 1.0))
        s["kI"] = ((B, cfg.N, cfg.c_I), cfg.qk_dt, ("normal", 1.0))
        # the decode state: raw streams of the last two blocks (2m tokens), from which the step
        # whose token completes a block computes the new KV entry and index-key entry (caches
        # in bf16 / fp8; no state for caches stored in other formats)
        m2 = 2 * cfg.m
        if cfg.kv_dt < 0:
            for nm in ("Ca", "Cb", "Za", "Zb"):
                s[nm] = ((B, m2, c), cfg.dt, ("normal", 1.0))
            for nm in ("Ba", "Bb"):
                s[nm] = ((cfg.m, c), F32, ("normal", 0.1))
        if cfg.qk_dt in (F32, BF16, FP8):
            for nm in ("ICa", "ICb", "IZa", "IZb"):
                s[nm] = ((B, m2, cfg.c_I), cfg.dt, ("normal", 1.0))
            for nm in ("IBa", "IBb"):
                s[nm] = ((cfg.m, cfg.c_I), F32, ("normal", 0.1))
    if cfg.kind in ("csa_prefill", "csa_decode"):
        s["q"] = ((B, cfg.T, cfg.H, c), cfg.dt, ("normal", 1.0))
        s["qI"] = ((B, cfg.T, cfg.H_I, cfg.c_I), cfg.qk_dt, ("normal", 1.0))
        s["w"] = ((B, cfg.T, cfg.H_I), F32, ("uniform", 0.0, 1.0))
    if cfg.kind == "hca_chunk":
        s["C"] = ((B, cfg.n, c), cfg.dt, ("normal", 1.0))
        s["Z"] = ((B, cfg.n, c), cfg.dt, ("normal", 1.0))
        s["B"] = ((cfg.m_prime, c), F32, ("normal", 0.1))
        s["q"] = ((B, cfg.T, cfg.H, c), cfg.dt, ("normal", 1.0))
    return s


def make_tensor(cfg: Config, name: str, seed: int | None = None) -> np.ndarray:
    shape, dt, dist = shapes(cfg)[name]
    sd = cfg.seed if seed is None else seed
    if dist[0] == "normal":
        return rng.normal(sd, TID[name], shape, dt, std=dist[1])
    return rng.uniform(sd, TID[name], shape, dt, lo=dist[1], hi=dist[2])


def make_inputs(cfg: Config, names=None, seed: int | None = None) -> dict:
    names = list(shapes(cfg)) if names is None else names
    return {nm: make_tensor(cfg, nm, seed) for nm in names}


def scaled(cfg: Config, **over) -> Config:
    """A copy of `cfg` with some fields replaced (small parity shapes of the same kind)."""
    d = dict(cfg.__dict__)
    d.update(over)
    d["name"] = over.get("name", cfg.name + "_scaled")
    return Config(**d)
