"""Helpers for the GPU parity tests: moving generator output to the device and the
tolerance rules the comparisons use.

Tolerances (from the workload contract):
  fp32 paths : |gpu - oracle| <= 1e-5 * max(|oracle|, 1), elementwise;
  bf16 / fp8 : |gpu - oracle| <= 2e-2, elementwise, on unit-scale outputs;
  top-k, fp32 : indices bit-exact (ties to the lower index);
  top-k, low precision : recall >= 0.99 over all rows, and every index present in one set
      but not the other has an oracle score within 1e-2 of the row's k-th oracle score.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

F32, BF16, FP8 = 0, 1, 2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: int, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == BF16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    if t.dtype == torch.uint8:
        return t.numpy()
    return t.numpy().astype(np.float64) if t.is_floating_point() else t.numpy()


def assert_fp32_close(got, ref, what=""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref) / np.maximum(np.abs(ref), 1.0)
    worst = float(err.max()) if err.size else 0.0
    say(f"  {what}: max scaled err {worst:.3e} (limit 1e-5) over {err.size} values")
    assert worst <= 1e-5, (what, worst, np.unravel_index(np.argmax(err), err.shape))


def assert_abs_close(got, ref, tol=2e-2, what=""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    worst = float(err.max()) if err.size else 0.0
    say(f"  {what}: max abs err {worst:.3e} (limit {tol}) over {err.size} values")
    assert worst <= tol, (what, worst, np.unravel_index(np.argmax(err), err.shape))


def check_topk_recall(gpu_idx, ref_idx, ref_scores_rows, k, window=1e-2, min_recall=0.99, what=""):
    """gpu_idx, ref_idx: [rows, k] int32 (-1 pads); ref_scores_rows: [rows, N] oracle scores."""
    hit = total = 0
    for r in range(ref_idx.shape[0]):
        a = set(int(x) for x in gpu_idx[r] if x >= 0)
        b = set(int(x) for x in ref_idx[r] if x >= 0)
        assert len(a) == len(b), (what, r, len(a), len(b))
        hit += len(a & b)
        total += len(b)
        if a != b:
            kth = np.min(ref_scores_rows[r][sorted(b)])
            for s in a ^ b:
                gap = abs(ref_scores_rows[r][s] - kth)
                assert gap <= window, (what, r, s, gap)
        assert np.all(np.diff(gpu_idx[r][gpu_idx[r] >= 0]) > 0), (what, r, "not ascending")
        assert np.all(gpu_idx[r][len(a):] == -1), (what, r, "bad padding")
    recall = hit / max(total, 1)
    say(f"  {what}: recall {recall:.5f} over {ref_idx.shape[0]} rows")
    assert recall >= min_recall, (what, recall)
    return recall
