"""Writes tests/golden/mxfp4_recall_cfg2.txt: how much of the fp8 indexer's top-k the MXFP4
indexer's top-k keeps, on the 128K-context decode workload (all 32 sequences, the same seeded
draws quantised to each format).  Both selections are the oracle's (the GPU matches the
oracle bit for bit on MXFP4 and fp8 inputs), so this calls only oracle/ and the input
generator.  Context, not a target: the notes page "DeepSeek-V4: 迈向高效百万级上下文智能"
(§2.4) quotes 99.7% KV-entry recall for the top-k on bf16 scores of a trained model; FP4 keys
of random data are coarser.

    python tests/golden/mxfp4_recall.py
"""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import CONFIGS, make_inputs, rng  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mxfp4_recall_cfg2.txt")


def main():
    f8, f4 = CONFIGS["cfg2_csa_decode_128k"], CONFIGS["cfg2_csa_decode_128k_mxfp4"]
    h8 = make_inputs(f8, names=["qI", "kI", "w"])
    h4 = make_inputs(f4, names=["qI", "kI", "w"])
    q4 = oracle.decode_mxfp4(h4["qI"], (f4.batch, f4.T, f4.H_I, f4.c_I))
    k4 = oracle.decode_mxfp4(h4["kI"], (f4.batch, f4.N, f4.c_I))
    per_row = []
    for b in range(f8.batch):
        s8 = oracle.index_scores(h8["qI"][b:b + 1], h8["w"][b:b + 1], h8["kI"][b:b + 1], f8.m, q_pos0=f8.q_pos0,
                                 qk_dtype=rng.FP8)
        s4 = oracle.index_scores(q4[b:b + 1], h4["w"][b:b + 1], k4[b:b + 1], f4.m, q_pos0=f4.q_pos0)
        i8, _ = oracle.topk(s8, f8.m, f8.k, q_pos0=f8.q_pos0)
        i4, _ = oracle.topk(s4, f4.m, f4.k, q_pos0=f4.q_pos0)
        per_row.append(len(set(i8.ravel()) & set(i4.ravel())) / f8.k)
    per_row = np.array(per_row)
    lines = ["# MXFP4 vs fp8 indexer: fraction of the fp8 top-k the MXFP4 top-k keeps",
             "# workload: cfg2_csa_decode_128k (32 sequences, 32768 entries, H_I 64 x 128, top-k 1024),",
             "# the same draws quantised to fp8 e4m3 and to MXFP4; oracle selections; written by",
             "# tests/golden/mxfp4_recall.py",
             f"recall_mean {per_row.mean():.6f}",
             f"recall_min {per_row.min():.6f}",
             f"recall_max {per_row.max():.6f}",
             "per_sequence " + " ".join(f"{x:.6f}" for x in per_row)]
    open(OUT, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines[4:7]))


if __name__ == "__main__":
    main()
