"""csa_index_topk_noalloc (the index + top-k call for callers that cannot allocate: its scratch
is the library's fixed per-GPU array) against csa_index_topk with a caller workspace, through
the C ABI.  Each case makes two calls in a row on the same GPU, the second with a smaller
input, so the second call runs on the scratch the first one left behind: both must equal the
workspace entry point's indices and scores exactly (the same kernels on the same inputs)."""
import numpy as np
import pytest
import torch

import long_context_sparse_08_amd as csa
from tests._util import BF16, F32, FP8, from_dev, say, to_dev
from workloads import rng

pytestmark = pytest.mark.gpu


def _inputs(seed, batch, T, N, H, cI, dt):
    qI = rng.normal(seed, 1, (batch, T, H, cI), dt)
    kI = rng.normal(seed, 2, (batch, N, cI), dt)
    w = rng.uniform(seed, 3, (batch, T, H), F32)
    return to_dev(qI, dt), to_dev(w, F32), to_dev(kI, dt)


# (batch, T, q_pos0, N, H_I, c_I, m, k, dtype): first call, then a smaller second call
PAIRS = [
    # 128K decode batch (register-staged selection), then 1M-entry rows (several workgroups
    # per row: the selection's counters must be cleared again on the reused scratch)
    ((16, 1, 4 * 32768, 32768, 64, 128, 4, 1024, FP8), (2, 1, 4 * 300000, 300000, 64, 128, 4, 1024, FP8)),
    # group maxima rows, then short decode rows of a different k
    ((4, 1, 4 * 100000, 100000, 64, 128, 4, 2048, FP8), (3, 2, 4 * 9000 - 2, 9000, 64, 128, 4, 512, FP8)),
    # prefill-shaped bf16 rows, then a smaller prefill chunk with rows shorter than k
    ((1, 64, 4000, 1200, 64, 128, 4, 256, BF16), (1, 16, 100, 200, 32, 128, 4, 64, BF16)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "N%d_then_N%d" % (p[0][3], p[1][3]))
def test_noalloc_matches_workspace_entry_point(pair):
    torch.cuda.set_device(0)
    for j, (batch, T, p0, N, H, cI, m, k, dt) in enumerate(pair):
        say(f"csa_index_topk_noalloc call {j}: batch={batch} T={T} q_pos0={p0} N={N} H_I={H} k={k} dt={dt}")
        assert csa.csa_index_topk_workspace_size(batch, T, N, H, k) <= csa.NOALLOC_SCRATCH_BYTES
        qI, w, kI = _inputs(3000 + 7 * j + N, batch, T, N, H, cI, dt)
        ref_idx, ref_sel = csa.csa_index_topk(qI, w, kI, p0, m, k)
        # poison the outputs: every element must be written by the call
        idx = torch.full((batch, T, k), 12345, dtype=torch.int32, device="cuda")
        sel = torch.full((batch, T, k), 7.5, dtype=torch.float32, device="cuda")
        got_idx, got_sel = csa.csa_index_topk_noalloc(qI, w, kI, p0, m, k, idx=idx, sel_scores=sel)
        torch.cuda.synchronize()
        gi, ri = from_dev(got_idx), from_dev(ref_idx)
        gs, rs = from_dev(got_sel), from_dev(ref_sel)
        say(f"  rows {batch * T}: idx equal {np.array_equal(gi, ri)}, scores equal {np.array_equal(gs, rs)}")
        assert np.array_equal(gi, ri)
        assert np.array_equal(gs, rs)
        # the selection itself is sane: ascending ids, -1 padding only at the end
        for r in gi.reshape(-1, k)[:4]:
            v = r[r >= 0]
            assert np.all(np.diff(v) > 0) and np.all(r[len(v):] == -1)


def test_noalloc_rejects_calls_beyond_its_scratch():
    # an 8K-token prefill (8192 score rows of 2048 entries) needs more than the fixed scratch:
    # a clear error, nothing launched, and the next call still works
    torch.cuda.set_device(0)
    batch, T, N, H, cI, k = 1, 8192, 2048, 64, 128, 512
    assert csa.csa_index_topk_workspace_size(batch, T, N, H, k) > csa.NOALLOC_SCRATCH_BYTES
    qI = torch.zeros((batch, T, H, cI), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((batch, T, H), dtype=torch.float32, device="cuda")
    kI = torch.zeros((batch, N, cI), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(csa.CsaError) as e:
        csa.csa_index_topk_noalloc(qI, w, kI, 0, 4, k)
    assert e.value.status == -5
    qs, ws, ks = _inputs(3999, 2, 1, 5000, 64, 128, FP8)
    a, _ = csa.csa_index_topk(qs, ws, ks, 4 * 5000, 4, 300)
    b, _ = csa.csa_index_topk_noalloc(qs, ws, ks, 4 * 5000, 4, 300)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
