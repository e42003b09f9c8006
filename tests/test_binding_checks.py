"""The Python binding rejects caller buffers whose shape or dtype differs from what the call
reads or writes, with a ValueError, before it reaches the C ABI (which sees only addresses).
CPU tensors suffice: these checks run before the device check, and nothing is launched."""
import pytest
import torch

import long_context_sparse_08_amd as csa

f32, bf16, u8, i32 = torch.float32, torch.bfloat16, torch.uint8, torch.int32


def z(*shape, dtype=f32):
    return torch.zeros(shape, dtype=dtype)


def test_compress_arguments():
    S = z(1, 64, 16)
    with pytest.raises(ValueError, match="Cb"):
        csa.csa_compress(S, z(1, 60, 16), S, S, z(4, 16), z(4, 16), 4)
    with pytest.raises(ValueError, match="Ba"):
        csa.csa_compress(S, S, S, S, z(4, 8), z(4, 16), 4)
    with pytest.raises(ValueError, match="out"):
        csa.csa_compress(S, S, S, S, z(4, 16), z(4, 16), 4, out=z(1, 15, 16))
    with pytest.raises(ValueError, match="B"):
        csa.hca_compress(S, S, z(4, 16, dtype=bf16), 4)
    with pytest.raises(ValueError, match="Zb"):
        csa.csa_compress_step(z(1, 8, 16), z(1, 8, 16), z(1, 8, 16), z(1, 4, 16), z(4, 16), z(4, 16), 3, z(1, 9, 16))
    with pytest.raises(ValueError, match="cache"):
        csa.csa_compress_step(*(z(1, 8, 16),) * 4, z(4, 16), z(4, 16), 9, z(1, 9, 16))
    with pytest.raises(ValueError, match="B"):
        csa.hca_compress_step(z(1, 8, 16), z(1, 8, 16), z(4, 16), 0, z(1, 2, 16))


def test_layer_step_compression_arguments():
    S = z(1, 8, 16)
    st = (S, S, S, S, z(4, 16), z(4, 16))
    with pytest.raises(ValueError, match="index-key Zb"):
        csa.csa_compress_step_kv_index(st, z(1, 9, 16), (S, S, S, z(1, 4, 16), z(4, 16), z(4, 16)), z(1, 9, 16), 3)
    with pytest.raises(ValueError, match="KV cache"):
        csa.csa_compress_step_kv_index(st, z(1, 3, 16), st, z(1, 9, 16), 3)
    with pytest.raises(ValueError, match="same batch"):
        S2 = z(2, 8, 16)
        csa.csa_compress_step_kv_index(st, z(1, 9, 16), (S2, S2, S2, S2, z(4, 16), z(4, 16)), z(2, 9, 16), 3)
    with pytest.raises(ValueError, match="same dtype"):
        Sb = z(1, 8, 16, dtype=bf16)
        csa.csa_compress_step_kv_index(st, z(1, 9, 16), (Sb, Sb, Sb, Sb, z(4, 16), z(4, 16)),
                                       z(1, 9, 16, dtype=bf16), 3)
    with pytest.raises(ValueError, match="states are"):
        csa.csa_compress_step_kv_index(st[:5], z(1, 9, 16), st, z(1, 9, 16), 3)


def test_indexer_and_selection_arguments():
    qI, kI, w = z(2, 1, 4, 32, dtype=u8), z(2, 100, 32, dtype=u8), z(2, 1, 4)
    with pytest.raises(ValueError, match="w"):
        csa.csa_index_topk(qI, z(2, 1, 3), kI, 400, 4, 8)
    with pytest.raises(ValueError, match="idx"):
        csa.csa_index_topk(qI, w, kI, 400, 4, 8, idx=z(2, 1, 8, dtype=torch.int64))
    with pytest.raises(ValueError, match="sel_scores"):
        csa.csa_index_topk(qI, w, kI, 400, 4, 8, sel_scores=z(2, 1, 7))
    with pytest.raises(ValueError, match="kI"):
        csa.csa_index_topk(qI, w, z(3, 100, 32, dtype=u8), 400, 4, 8)
    with pytest.raises(ValueError, match="one dtype"):
        csa.csa_index_topk(qI, w, z(2, 100, 32, dtype=bf16), 400, 4, 8)
    with pytest.raises(ValueError, match="idx"):
        csa.csa_index_topk_noalloc(qI, w, kI, 400, 4, 8, idx=z(2, 1, 9, dtype=i32))
    with pytest.raises(ValueError, match="scores"):
        csa.csa_index_scores(qI, w, kI, 400, 4, scores=z(2, 1, 99))
    with pytest.raises(ValueError, match="idx"):
        csa.csa_topk(z(2, 1, 100), 400, 4, 8, idx=z(2, 1, 8))
    with pytest.raises(ValueError, match="multiple of 4"):
        csa.csa_topk(z(2, 1, 99), 400, 4, 8)


def test_attention_arguments():
    q, kv, idx = z(2, 3, 4, 64), z(2, 50, 64), z(2, 3, 8, dtype=i32)
    with pytest.raises(ValueError, match="out"):
        csa.csa_sparse_mqa(q, kv, idx, 0.1, out=z(2, 3, 4, 32))
    with pytest.raises(ValueError, match="idx"):
        csa.csa_sparse_mqa(q, kv, z(2, 3, 8, dtype=torch.int64), 0.1)
    with pytest.raises(ValueError, match="kv"):
        csa.csa_sparse_mqa(q, z(2, 50, 32), idx, 0.1)
    with pytest.raises(ValueError, match="win_kv"):
        csa.csa_sparse_mqa(q, kv, idx, 0.1, window=(z(2, 10, 32), 0, 0, 4))
    with pytest.raises(ValueError, match="sink"):
        csa.csa_sparse_mqa(q, kv, idx, 0.1, sink=z(5))
    with pytest.raises(ValueError, match="out"):
        csa.hca_dense_mqa(q, kv, 0, 128, 0.1, out=z(2, 3, 4, 64, dtype=bf16))
    with pytest.raises(ValueError, match="win_kv"):
        csa.hca_dense_mqa(q, kv, 0, 128, 0.1, window=(z(1, 10, 64), 0, 4))
    with pytest.raises(ValueError, match="mixed"):
        csa.hca_dense_mqa(q, csa.KVFp8Bf16(z(2, 50, 128, dtype=u8), 64), 0, 128, 0.1)
