"""Pins for the CPU oracle: closed forms, invariants, special cases that reduce to a library
routine, and facts the pages state.  None of these re-types the oracle's own formula; each
is chosen so that a plausible slip (wrong window, swapped stream, dropped term, wrong bias
offset, wrong mask boundary, wrong tie rule, missing scale) fails at least one of them.

Sources: "DeepSeek-V4: 迈向高效百万级上下文智能" (notes.kuangjux.top) §1.1 steps 1-2 and
§1.2; the mlpod.com summary of the DeepSeek-V4 report §2.3.1-§2.3.2.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax

from workloads import rng

F32, BF16, FP8 = 0, 1, 2
R = np.random.RandomState


def randn(shape, seed, std=1.0):
    return (R(seed).randn(*shape) * std).astype(np.float64)


# ----------------------------------------------------------------------------- storage
def test_decode_bf16_matches_torch(orc):
    bits = R(0).randint(0, 1 << 16, size=20000).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = orc.decode(bits, BF16)
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]) and np.isnan(got[~ok]).all()


def test_round_to_e4m3_matches_torch_and_saturates(orc):
    """Rounding to fp8 e4m3fn (the storage of fp8 compressed indexer keys): every code's value,
    every midpoint between neighbouring codes (ties go to the even code), random values and
    subnormals round as torch's float8_e4m3fn cast does inside the format's range; beyond
    +-448 the oracle saturates (448 is the largest finite e4m3fn value, +-464 the overflow
    midpoint), checked by hand."""
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()   # +0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    r = np.random.RandomState(5)
    x = np.concatenate([vals, mids, r.uniform(-448, 448, 5000), r.uniform(-0.02, 0.02, 2000), r.randn(2000)])
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).float().to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(orc.round_to(x.astype(np.float32).astype(np.float64), 2), ref)
    got = orc.round_to(np.array([448.0, 449.0, 463.9, 500.0, 1e6, -500.0, -1e9, 2.0 ** -10, 3 * 2.0 ** -11]), 2)
    assert np.array_equal(got, [448.0, 448.0, 448.0, 448.0, 448.0, -448.0, -448.0, 0.0, 2.0 ** -9])


def test_decode_e4m3_matches_torch_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = orc.decode(codes, FP8)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~ok)
    assert np.array_equal(got[ok], ref[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


# MXFP4 (the notes page's §2.4: the indexer's QK path in MXFP4): OCP Microscaling Formats
# v1.0 — E2M1 elements (its table of values), one E8M0 scale per 32 elements.
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # codes 0..7, the spec's FP4 E2M1 values


def test_decode_kv_fp8_bf16_layout(orc):
    """Mixed KV rows (the notes page §1.3: RoPE channels in bf16, the rest in fp8; RoPE on the
    last 64 channels): c - 64 e4m3 bytes, then 64 little-endian bf16 values.  Values from the
    formats' definitions: e4m3 0x38 = 1, 0xB8 = -1, 0x01 = 2^-9 (subnormal), 0x08 = 2^-6,
    0x7E = 448; bf16 0x3F80 = 1, 0xC040 = -3, 0x0001 = 2^-133."""
    c = 128
    buf = np.zeros((2, c + 64), np.uint8)
    buf[0, :5] = [0x38, 0xB8, 0x01, 0x08, 0x7E]
    buf[1, c - 65] = 0x38                       # the last fp8 channel of row 1
    bf = np.zeros((2, 64), np.uint16)
    bf[0, 0], bf[0, 63], bf[1, 1] = 0x3F80, 0xC040, 0x0001
    buf[:, c - 64:] = bf.astype("<u2").view(np.uint8).reshape(2, 128)
    dec = orc.decode_kv_fp8_bf16(buf, c)
    exp = np.zeros((2, c))
    exp[0, :5] = [1.0, -1.0, 2.0 ** -9, 2.0 ** -6, 448.0]
    exp[1, c - 65] = 1.0
    exp[0, c - 64], exp[0, c - 1], exp[1, c - 63] = 1.0, -3.0, 2.0 ** -133
    assert np.array_equal(dec, exp)


def test_kv_fp8_bf16_generator_rounds_each_part_as_torch(orc):
    """The generator's mixed rows, decoded by the oracle, equal torch's own roundings of the
    same float32 draws: float8_e4m3fn for the first c - 64 channels, bfloat16 for the rest."""
    x = rng.normal(7, 3, (6, 512), rng.F32)
    dec = orc.decode_kv_fp8_bf16(rng.f32_to_kv_fp8_bf16(x), 512)
    t = torch.from_numpy(x)
    assert np.array_equal(dec[:, :448], t[:, :448].to(torch.float8_e4m3fn).double().numpy())
    assert np.array_equal(dec[:, 448:], t[:, 448:].to(torch.bfloat16).double().numpy())
    assert np.array_equal(rng.kv_fp8_bf16_to_f32(rng.f32_to_kv_fp8_bf16(x), 512), dec.astype(np.float32))


def test_decode_mxfp4_elements_match_the_spec_table(orc):
    # one row of 32 values holding all 16 codes twice, scale 2^0: code 8 + j is -(code j)
    codes = np.concatenate([np.arange(16), np.arange(16)[::-1]]).astype(np.uint8)
    buf = np.concatenate([(codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), np.array([127], np.uint8)])
    got = orc.decode_mxfp4(buf, (1, 32))[0]
    want = np.array([E2M1_SPEC[c & 7] * (-1.0 if c & 8 else 1.0) for c in codes])
    assert np.array_equal(got, want) and np.signbit(got[8]) and not np.signbit(got[0])


def test_decode_mxfp4_scales_match_torch_e8m0(orc):
    # element code 2 (1.0) everywhere: the decoded value is the block scale; 255 is NaN
    scales = np.arange(256, dtype=np.uint8)
    buf = np.concatenate([np.full(256 * 16, 0x22, np.uint8), scales])
    got = orc.decode_mxfp4(buf, (256, 32))
    ref = torch.from_numpy(scales).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(np.isnan(got[:, 0]), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], np.repeat(ref[ok, None], 32, axis=1))


def test_decode_mxfp4_layout_nibbles_blocks_and_rows(orc):
    # 3 rows of 64 values: value 2i in the low nibble of byte i, block b of row r uses scale
    # byte r * 2 + b of the scale region that follows all rows' element bytes
    r = R(7)
    codes = r.randint(0, 16, size=(3, 64)).astype(np.uint8)
    sc = r.randint(120, 135, size=(3, 2)).astype(np.uint8)
    buf = np.concatenate([(codes[:, 0::2] | (codes[:, 1::2] << 4)).reshape(-1), sc.reshape(-1)]).astype(np.uint8)
    got = orc.decode_mxfp4(buf, (3, 64))
    for row in range(3):
        for j in range(64):
            c = codes[row, j]
            v = E2M1_SPEC[c & 7] * (-1.0 if c & 8 else 1.0) * 2.0 ** (int(sc[row, j // 32]) - 127)
            assert got[row, j] == v, (row, j)


def test_mxfp4_quantizer_follows_the_mx_conversion_rule():
    # the input generator's rounding to MXFP4 (storage only): scale 2^(floor(log2 amax) - 2),
    # elements rounded to the nearest E2M1 value, ties to the even code, saturating at 6
    x = np.zeros((2, 32), np.float32)
    x[0, :6] = [0.1, -0.25, 1.3, 6.0, -7.9, 0.75]        # amax 7.9: scale 2^0
    x[1, :4] = [1000.0, 250.0, -96.0, 31.0]               # amax 1000: floor(log2) 9 -> 2^7
    buf = rng.f32_to_mxfp4(x)
    assert list(buf[-2:]) == [127, 134]
    v = rng.mxfp4_to_f32(buf, 2, 32)
    assert list(v[0, :6]) == [0.0, -0.0, 1.5, 6.0, -6.0, 1.0]   # 0.75: tie 0.5 / 1.0 -> even code 2
    # 1000/128 = 7.8 -> 6 (saturates); 250/128 -> 2; -96/128 = -0.75: tie -> even code 2 (1.0);
    # 31/128 = 0.24 -> 0
    assert list(v[1, :4]) == [768.0, 256.0, -128.0, 0.0]
    # values already on the grid come back exactly
    on = (np.array(E2M1_SPEC * 4, np.float32) * np.float32(2.0 ** -3)).reshape(1, 32)
    assert np.array_equal(rng.mxfp4_to_f32(rng.f32_to_mxfp4(on), 1, 32), on)


def test_round_bf16_matches_torch_and_ties_to_even(orc):
    x = (R(1).randn(50000) * np.exp(R(2).uniform(-30, 30, 50000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(orc.round_to(x.astype(np.float64), BF16), ref)
    # exact halfway points: 1 + 2^-8 lies between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3*2^-8 lies between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    got = orc.round_to(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]), BF16)
    assert list(got) == [1.0, 1 + 2.0 ** -6, -1.0]


def test_round_f32_matches_numpy(orc):
    x = R(3).randn(10000) * 1e3
    assert np.array_equal(orc.round_to(x, F32), x.astype(np.float32).astype(np.float64))


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 1234567: first five outputs as published with the reference
    # implementation (used by the input generator in counter mode).
    seed = np.uint64(1234567)
    with np.errstate(over="ignore"):
        got = rng.mix64(seed + np.arange(1, 6, dtype=np.uint64) * rng.GOLDEN)
    assert [int(v) for v in got] == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                                     4593380528125082431, 16408922859458223821]


# ----------------------------------------------------------------------------- CSA compress
def _streams(batch, n, c, seed):
    return [randn((batch, n, c), seed + i) for i in range(4)]


def test_csa_weights_sum_to_one(orc):
    # C == 1 on both streams -> every entry is exactly a convex weight sum == 1 for any Z, B
    batch, n, m, c = 2, 37, 4, 6
    _, _, Za, Zb = _streams(batch, n, c, 10)
    Ba, Bb = randn((m, c), 20, 0.1), randn((m, c), 21, 0.1)
    ones = np.ones((batch, n, c))
    out = orc.csa_compress(ones, ones, Za * 3, Zb * 3, Ba, Bb, m)
    assert out.shape == (batch, n // m, c)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


def test_csa_uniform_scores_give_mean_pooling(orc):
    # Z = 0, B = 0: entry i = (sum of Ca over window i + sum of Cb over window i-1) / (2m);
    # block 0 has no previous window, so it is the mean of Ca over window 0.
    batch, n, m, c = 2, 40, 4, 5
    Ca, Cb, _, _ = _streams(batch, n, c, 30)
    z = np.zeros((batch, n, c))
    b0 = np.zeros((m, c))
    out = orc.csa_compress(Ca, Cb, z, z, b0, b0, m)
    N = n // m
    exp = np.empty_like(out)
    for i in range(N):
        a = Ca[:, m * i:m * (i + 1)].sum(1)
        if i == 0:
            exp[:, i] = a / m
        else:
            exp[:, i] = (a + Cb[:, m * (i - 1):m * i].sum(1)) / (2 * m)
    np.testing.assert_allclose(out, exp, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("m", [2, 4])
def test_csa_one_hot_scores_pick_the_right_token_and_stream(orc, m):
    # A dominant score (+60) on one token selects that token's value from the matching stream.
    batch, n, c = 1, 8 * m, 3
    Ca, Cb, _, _ = _streams(batch, n, c, 40)
    N = n // m
    zb0, B0 = np.zeros((batch, n, c)), np.zeros((m, c))
    for r in range(m):
        Za = np.zeros((batch, n, c))
        Za[:, r::m, :] = 60.0          # offset r of every a-window
        out = orc.csa_compress(Ca, Cb, Za, zb0 - 60.0, B0, B0, m)
        np.testing.assert_allclose(out[0], Ca[0, r::m][:N], rtol=1e-12, atol=1e-12)
        Zb = np.zeros((batch, n, c))
        Zb[:, r::m, :] = 60.0          # offset r of every b-window (window i-1 of entry i)
        out = orc.csa_compress(Ca, Cb, zb0 - 60.0, Zb, B0, B0, m)
        np.testing.assert_allclose(out[0, 1:], Cb[0, r::m][:N - 1], rtol=1e-12, atol=1e-12)
        # block 0 has no b window: only the (now heavily down-weighted, equal) a-scores remain
        np.testing.assert_allclose(out[0, 0], Ca[0, :m].mean(0), rtol=1e-12, atol=1e-12)


def test_csa_position_bias_is_indexed_by_offset_and_channel(orc):
    batch, n, m, c = 1, 24, 4, 4
    Ca, Cb, _, _ = _streams(batch, n, c, 50)
    z = np.zeros((batch, n, c))
    N = n // m
    for r in range(m):
        Ba = np.zeros((m, c))
        Bb = np.zeros((m, c))
        Ba[r, 2] = 60.0                # only channel 2 gets the bias at offset r
        Bb[:, 2] = -60.0
        out = orc.csa_compress(Ca, Cb, z, z, Ba, Bb, m)
        np.testing.assert_allclose(out[0, :, 2], Ca[0, r::m, 2][:N], rtol=1e-12, atol=1e-12)
        # the other channels are untouched by that bias: plain mean pooling
        i = 3
        mean = (Ca[0, m * i:m * (i + 1), 0].sum() + Cb[0, m * (i - 1):m * i, 0].sum()) / (2 * m)
        np.testing.assert_allclose(out[0, i, 0], mean, rtol=1e-13)


def test_csa_shift_invariance_and_tail_and_batch(orc):
    batch, n, m, c = 3, 43, 4, 7       # 43 = 10 blocks + 3 tail tokens
    Ca, Cb, Za, Zb = _streams(batch, n, c, 60)
    Ba, Bb = randn((m, c), 61, 0.1), randn((m, c), 62, 0.1)
    out = orc.csa_compress(Ca, Cb, Za, Zb, Ba, Bb, m)
    np.testing.assert_allclose(orc.csa_compress(Ca, Cb, Za + 5.0, Zb + 5.0, Ba, Bb, m), out, rtol=1e-12)
    # tail tokens (40..42) influence nothing
    Ca2 = Ca.copy(); Ca2[:, 40:] = 99.0
    Za2 = Za.copy(); Za2[:, 40:] = 99.0
    np.testing.assert_array_equal(orc.csa_compress(Ca2, Cb, Za2, Zb, Ba, Bb, m), out)
    # sequences are independent and each equals its own single-sequence run
    one = orc.csa_compress(Ca[1:2], Cb[1:2], Za[1:2], Zb[1:2], Ba, Bb, m)
    np.testing.assert_array_equal(one[0], out[1])


def test_csa_block0_with_m1_is_identity(orc):
    # m = 1 and block 0: a single a-token, no b window -> the entry is that token exactly.
    # With the b window masked (Zb = -inf) every entry is its own a-token.
    batch, n, c = 1, 9, 3
    Ca, Cb, Za, Zb = _streams(batch, n, c, 70)
    Ba, Bb = randn((1, c), 71), randn((1, c), 72)
    out = orc.csa_compress(Ca, Cb, Za, Zb, Ba, Bb, 1)
    np.testing.assert_array_equal(out[0, 0], Ca[0, 0])
    out = orc.csa_compress(Ca, Cb, Za, np.full_like(Zb, -np.inf), Ba, Bb, 1)
    np.testing.assert_array_equal(out, Ca)


def test_compress_entry_counts_at_one_million_tokens(orc):
    # The pages: 1M (=10^6) tokens become 250k CSA entries (m=4) and ~7800 HCA entries
    # (m'=128).  Fixture: tests/golden/entry_counts.txt.
    import os
    rows = {}
    path = os.path.join(os.path.dirname(__file__), "golden", "entry_counts.txt")
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            name, n, ratio, entries = line.split()[:4]
            rows[name] = (int(n), int(ratio), int(entries))
    n, m, want = rows["csa"]
    one = np.ones((1, n, 1))
    z = np.zeros((1, n, 1))
    assert orc.csa_compress(one, one, z, z, np.zeros((m, 1)), np.zeros((m, 1)), m).shape[1] == want
    n, mp, want = rows["hca"]
    assert orc.hca_compress(one, z, np.zeros((mp, 1)), mp).shape[1] == want
    assert abs(want - 7800) < 0.01 * 7800


# ----------------------------------------------------------------------------- HCA compress
def test_hca_m1_identity_and_weights_sum_to_one(orc):
    batch, n, c = 2, 11, 5
    C, Z = randn((batch, n, c), 80), randn((batch, n, c), 81)
    B = randn((1, c), 82)
    np.testing.assert_array_equal(orc.hca_compress(C, Z, B, 1), C)
    mp = 5
    out = orc.hca_compress(np.ones_like(C), Z * 4, randn((mp, c), 83), mp)
    assert out.shape == (batch, 2, c)
    np.testing.assert_allclose(out, 1.0, atol=1e-14)


def test_hca_mean_pooling_one_hot_and_no_overlap(orc):
    batch, n, mp, c = 1, 3 * 16 + 5, 16, 4
    C = randn((batch, n, c), 90)
    z, b0 = np.zeros((batch, n, c)), np.zeros((mp, c))
    out = orc.hca_compress(C, z, b0, mp)
    exp = np.stack([C[0, mp * i:mp * (i + 1)].mean(0) for i in range(3)])
    np.testing.assert_allclose(out[0], exp, rtol=1e-13, atol=1e-15)
    B = np.zeros((mp, c)); B[7] = 60.0
    np.testing.assert_allclose(orc.hca_compress(C, z, B, mp)[0], C[0, 7::mp][:3], rtol=1e-12, atol=1e-12)
    # no overlap: entry 1 ignores window 0 and window 2
    C2 = C.copy(); C2[:, :mp] = 50.0; C2[:, 2 * mp:] = -50.0
    np.testing.assert_array_equal(orc.hca_compress(C2, z, b0, mp)[0, 1], out[0, 1])


# ----------------------------------------------------------------------------- indexer
def _mask(T, N, ratio, qpos):
    s = np.arange(N)[None, :]
    return ratio * (s + 1) - 1 <= np.asarray(qpos)[:, None]


def test_indexer_single_head_is_relu_of_matmul(orc):
    batch, T, N, cI, m = 2, 30, 9, 8, 4
    qI, kI = randn((batch, T, 1, cI), 100), randn((batch, N, cI), 101)
    w = np.ones((batch, T, 1))
    got = orc.index_scores(qI, w, kI, m)
    vis = _mask(T, N, m, np.arange(T))
    for b in range(batch):
        ref = np.maximum(np.matmul(qI[b, :, 0], kI[b].T), 0.0)
        np.testing.assert_allclose(got[b][vis], ref[vis], rtol=1e-13, atol=1e-13)
        assert np.all(np.isneginf(got[b][~vis]))


def test_indexer_linear_in_head_weights_and_one_hot_heads(orc):
    batch, T, N, H, cI, m = 1, 20, 5, 3, 6, 4
    qI, kI = randn((batch, T, H, cI), 110), randn((batch, N, cI), 111)
    w1, w2 = R(112).uniform(0, 1, (batch, T, H)), R(113).uniform(-1, 1, (batch, T, H))
    vis = _mask(T, N, m, np.arange(T))
    s1, s2 = orc.index_scores(qI, w1, kI, m), orc.index_scores(qI, w2, kI, m)
    s12 = orc.index_scores(qI, w1 + 2.5 * w2, kI, m)
    np.testing.assert_allclose(s12[0][vis], (s1 + 2.5 * s2)[0][vis], rtol=1e-12, atol=1e-12)
    for h in range(H):
        e = np.zeros((batch, T, H)); e[..., h] = 1.0
        ref = np.maximum(np.matmul(qI[0, :, h], kI[0].T), 0.0)
        np.testing.assert_allclose(orc.index_scores(qI, e, kI, m)[0][vis], ref[vis], rtol=1e-13, atol=1e-13)
    perm = [2, 0, 1]
    np.testing.assert_allclose(orc.index_scores(qI[:, :, perm], w1[..., perm], kI, m)[0][vis], s1[0][vis],
                               rtol=1e-13)


def test_indexer_causal_boundary(orc):
    # entry s becomes visible exactly at position m(s+1)-1 and not one token earlier
    m, N, cI = 4, 6, 4
    T = m * N + 3
    qI, kI = randn((1, T, 2, cI), 120), randn((1, N, cI), 121)
    w = np.ones((1, T, 2))
    sc = orc.index_scores(qI, w, kI, m)
    for s in range(N):
        assert np.isneginf(sc[0, m * (s + 1) - 2, s])
        assert np.isfinite(sc[0, m * (s + 1) - 1, s])
    # changing an invisible key changes nothing
    kI2 = kI.copy(); kI2[0, 5] = 100.0
    t = m * 5 - 1   # sees s < 5
    np.testing.assert_array_equal(orc.index_scores(qI, w, kI2, m)[0, t], sc[0, t])
    # explicit positions (sampling) agree with the contiguous run
    sub = np.array([3, 17, 26])
    got = orc.index_scores(qI[:, sub], w[:, sub], kI, m, qpos=sub)
    np.testing.assert_array_equal(got[0], sc[0, sub])


# ----------------------------------------------------------------------------- top-k
def _topk_by_stable_sort(scores, vis, k):
    idx = np.full(k, -1, dtype=np.int32)
    cand = np.nonzero(vis)[0]
    order = cand[np.argsort(-scores[cand], kind="stable")]   # stable: equal scores keep index order
    keep = np.sort(order[:k])
    idx[:len(keep)] = keep
    return idx


def test_topk_equals_full_stable_sort_with_ties(orc):
    batch, T, N, m, k = 2, 60, 14, 4, 5
    # integer-valued scores -> many exact ties
    sc = R(130).randint(0, 4, (batch, T, N)).astype(np.float64)
    idx, sel = orc.topk(sc, m, k)
    for b in range(batch):
        for t in range(T):
            vis = m * (np.arange(N) + 1) - 1 <= t
            ref = _topk_by_stable_sort(sc[b, t], vis, k)
            assert np.array_equal(idx[b, t], ref), (b, t)
            good = ref >= 0
            np.testing.assert_array_equal(sel[b, t][good], sc[b, t][ref[good]])
            assert np.all(np.isneginf(sel[b, t][~good]))


def test_topk_all_visible_when_k_large_and_ties_lower_index(orc):
    N, k, m = 10, 16, 4
    sc = np.zeros((1, 3, N))
    idx, _ = orc.topk(sc, m, k, q_pos0=1000)
    assert list(idx[0, 0]) == list(range(N)) + [-1] * (k - N)
    idx, _ = orc.topk(sc, m, 3, q_pos0=1000)
    assert list(idx[0, 0]) == [0, 1, 2]          # all tied -> lowest indices
    idx, _ = orc.topk(sc, m, 3, q_pos0=2)         # position 2 < m-1: nothing visible
    assert list(idx[0, 0]) == [-1, -1, -1]


# ----------------------------------------------------------------------------- sparse MQA
def test_sparse_mqa_special_cases(orc):
    batch, T, N, H, c, k = 1, 4, 12, 3, 8, 5
    q, kv = randn((batch, T, H, c), 140), randn((batch, N, c), 141)
    scale = 0.3
    # one selected entry -> exactly that row
    idx = np.full((batch, T, k), -1, np.int32); idx[0, :, 2] = [3, 7, 0, 11]
    out = orc.sparse_mqa(q, kv, idx, scale)
    for t, s in enumerate([3, 7, 0, 11]):
        np.testing.assert_allclose(out[0, t], np.broadcast_to(kv[0, s], (H, c)), rtol=1e-15)
    # q = 0 -> mean of the selected rows
    sel = np.array([[1, 4, 5, 9, 10]] * T, np.int32)[None]
    out = orc.sparse_mqa(np.zeros_like(q), kv, sel, scale)
    np.testing.assert_allclose(out[0, 0, 0], kv[0, [1, 4, 5, 9, 10]].mean(0), rtol=1e-13)
    # permuting / padding the id list changes nothing
    base = orc.sparse_mqa(q, kv, sel, scale)
    perm = sel[:, :, ::-1].copy()
    np.testing.assert_allclose(orc.sparse_mqa(q, kv, perm, scale), base, rtol=1e-12, atol=1e-14)
    padded = np.concatenate([sel, np.full((1, T, 3), -1, np.int32)], axis=2)
    np.testing.assert_allclose(orc.sparse_mqa(q, kv, padded, scale), base, rtol=1e-12, atol=1e-14)
    # empty selection -> zeros
    assert not orc.sparse_mqa(q, kv, np.full((1, T, k), -1, np.int32), scale).any()


def test_sparse_mqa_two_entries_logistic_closed_form(orc):
    # two entries: weights are the logistic function of the scaled logit difference
    c, scale = 6, 0.37
    q, kv = randn((1, 1, 1, c), 150), randn((1, 2, c), 151)
    out = orc.sparse_mqa(q, kv, np.array([[[0, 1]]], np.int32), scale)
    d = scale * (q[0, 0, 0] @ kv[0, 0] - q[0, 0, 0] @ kv[0, 1])
    p0 = 1.0 / (1.0 + np.exp(-d))
    np.testing.assert_allclose(out[0, 0, 0], p0 * kv[0, 0] + (1 - p0) * kv[0, 1], rtol=1e-13)


def test_sparse_mqa_identical_rows(orc):
    kv = np.broadcast_to(randn((1, 1, 8), 160), (1, 9, 8)).copy()
    q = randn((1, 2, 4, 8), 161)
    out = orc.sparse_mqa(q, kv, np.array([[[0, 3, 8], [2, 5, -1]]], np.int32), 0.5)
    np.testing.assert_allclose(out, np.broadcast_to(kv[0, 0], out.shape), rtol=1e-14)


# ----------------------------------------------------------------------------- dense MQA
def _dense_attention(q, kv, ratio, scale, qpos):
    # brute force with a library softmax over an explicit mask
    T, H, c = q.shape[1:]
    N = kv.shape[1]
    out = np.zeros(q.shape)
    vis = _mask(T, N, ratio, qpos)
    for b in range(q.shape[0]):
        logits = scale * np.einsum("thc,sc->ths", q[b], kv[b])
        logits = np.where(vis[:, None, :], logits, -np.inf)
        has = vis.any(1)
        p = softmax(logits[has], axis=-1)
        out[b, has] = np.einsum("ths,sc->thc", p, kv[b])
    return out


def test_hca_dense_mqa_equals_masked_full_attention(orc):
    batch, T, N, H, c, mp = 2, 7, 9, 3, 8, 16
    q, kv = randn((batch, T, H, c), 170), randn((batch, N, c), 171)
    q_pos0 = 20                      # positions 20..26: 1 entry visible until 31
    qpos = np.array([0, 14, 15, 31, 47, 100, 143])
    got = orc.hca_dense_mqa(q, kv, mp, 0.25, qpos=qpos)
    np.testing.assert_allclose(got, _dense_attention(q, kv, mp, 0.25, qpos), rtol=1e-12, atol=1e-14)
    assert not got[:, :2].any()      # positions 0 and 14 see nothing
    got = orc.hca_dense_mqa(q, kv, mp, 0.25, q_pos0=q_pos0)
    np.testing.assert_allclose(got, _dense_attention(q, kv, mp, 0.25, q_pos0 + np.arange(T)), rtol=1e-12,
                               atol=1e-14)


def test_sparse_mqa_over_all_visible_equals_dense_csa_mask(orc):
    # selecting every visible entry turns sparse MQA into dense causal MQA under the CSA mask
    batch, T, N, H, c, m = 1, 30, 7, 2, 5, 4
    q, kv = randn((batch, T, H, c), 180), randn((batch, N, c), 181)
    idx, _ = orc.topk(np.zeros((batch, T, N)), m, N)
    np.testing.assert_allclose(orc.sparse_mqa(q, kv, idx, 0.4), orc.hca_dense_mqa(q, kv, m, 0.4),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(orc.sparse_mqa(q, kv, idx, 0.4), _dense_attention(q, kv, m, 0.4, np.arange(T)),
                               rtol=1e-12, atol=1e-14)


def test_attention_sink_closed_forms(orc):
    """Attention sink (the notes page §1.3, the mlpod page §2.3.3 item 4): the softmax
    denominator gains exp(z'_h).  One entry with logit l gives the weight 1 / (1 + exp(z' - l))
    (logistic); a sink far below every logit changes nothing; a query with no entry stays 0;
    heads keep their own sink."""
    c = 4
    q = np.zeros((1, 2, 2, c))
    q[0, :, 0, 0] = 1.0                 # head 0 of both queries: logit = scale * kv[s, 0]
    q[0, :, 1, 1] = 1.0                 # head 1: logit = scale * kv[s, 1]
    kv = np.array([[[2.0, 1.0, -1.0, 0.5], [0.0, -3.0, 4.0, 1.0]]])
    idx = np.array([[[0, -1], [-1, -1]]], np.int32)   # query 1 selects nothing
    scale, sink = 0.5, np.array([0.3, -2.0])
    out = orc.sparse_mqa(q, kv, idx, scale, sink=sink)
    for h, logit in ((0, 1.0), (1, 0.5)):
        wgt = 1.0 / (1.0 + np.exp(sink[h] - logit))
        assert np.allclose(out[0, 0, h], wgt * kv[0, 0], rtol=1e-15, atol=0)
    assert not out[0, 1].any()
    far = orc.sparse_mqa(q, kv, np.array([[[0, 1], [1, 0]]], np.int32), scale, sink=np.array([-1e300, -1e300]))
    assert np.array_equal(far, orc.sparse_mqa(q, kv, np.array([[[0, 1], [1, 0]]], np.int32), scale))


def test_dense_mqa_with_sink_equals_sparse_over_the_visible_entries(orc):
    r = np.random.RandomState(5)
    T, N, H, c, mp, p0 = 6, 9, 3, 8, 4, 10
    q, kv = r.randn(1, T, H, c), r.randn(1, N, c)
    sink = r.randn(H)
    dense = orc.hca_dense_mqa(q, kv, mp, 0.3, q_pos0=p0, sink=sink)
    idx = np.full((1, T, N), -1, np.int32)
    for t in range(T):
        vis = [s for s in range(N) if mp * (s + 1) - 1 <= p0 + t]
        idx[0, t, :len(vis)] = vis
    assert np.allclose(dense, orc.sparse_mqa(q, kv, idx, 0.3, sink=sink), rtol=1e-13, atol=1e-15)
    # and the sink lowers every weight: the output is the no-sink output times sum/(sum + e^z')
    plain = orc.hca_dense_mqa(q, kv, mp, 0.3, q_pos0=p0)
    assert np.all(np.abs(dense) <= np.abs(plain) + 1e-15)


def test_rope_pairs_frequencies_and_relative_positions(orc):
    """Partial RoPE (the notes page §1.3: the last 64 channels; rotation as in RoFormer):
    unit vectors on pair 0 and pair 1 land on (cos, sin) of p and p * base^(-2/d); the leading
    channels stay; position 0 is the identity; the inverse undoes it; and rotated dot products
    depend only on the position difference (the property RoPE exists for)."""
    c, d, base, p = 96, 64, 10000.0, 37
    x = np.zeros((1, 1, c))
    x[0, 0, c - d] = 1.0                        # pair 0, first channel
    x[0, 0, c - d + 3] = 1.0                    # pair 1, second channel
    x[0, 0, 5] = 2.5                            # outside the rotated part
    y = orc.rope(x, p, d=d, base=base)
    a1 = p * base ** (-2.0 / d)
    assert np.allclose(y[0, 0, c - d:c - d + 4], [np.cos(p), np.sin(p), -np.sin(a1), np.cos(a1)], rtol=0, atol=1e-15)
    assert y[0, 0, 5] == 2.5 and not y[0, 0, c - d + 4:].any()
    r = np.random.RandomState(3)
    v = r.randn(2, 3, 4, c)
    assert np.array_equal(orc.rope(v, 0, pos_step=0), v)
    assert np.allclose(orc.rope(orc.rope(v, 1000, 7), 1000, 7, inverse=True), v, rtol=0, atol=1e-12)
    a, b = r.randn(1, 1, c), r.randn(1, 1, c)
    lhs = (orc.rope(a, 5000)[..., c - d:] * orc.rope(b, 4321)[..., c - d:]).sum()
    rhs = (orc.rope(a, 5000 - 4321)[..., c - d:] * b[..., c - d:]).sum()
    assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(rhs))


def test_sliding_window_branch(orc):
    """Sliding-window branch (the notes page §1.3: each query also attends to the most recent
    n_win uncompressed tokens): with nothing selected it is causal attention over the last n_win
    raw rows (scipy softmax, written here independently); n_win = 0 changes nothing; a window
    row and a selected entry share one softmax (the union equals attention over both rows)."""
    r = np.random.RandomState(11)
    B, T, H, c, W, n_win = 1, 6, 2, 8, 10, 4
    q, wkv, kv = r.randn(B, T, H, c), r.randn(B, W, c), r.randn(B, 5, c)
    idx = np.full((B, T, 3), -1, np.int32)
    out = orc.sparse_mqa(q, kv, idx, 0.4, window=(wkv, 0, 2, n_win))
    for t in range(T):
        p = 2 + t
        rows = [j for j in range(W) if p - n_win + 1 <= j <= p]
        for h in range(H):
            w = softmax(0.4 * wkv[0, rows] @ q[0, t, h])
            assert np.allclose(out[0, t, h], w @ wkv[0, rows], rtol=1e-12, atol=1e-14)
    sel = r.randint(0, 5, size=(B, T, 3)).astype(np.int32)
    sel[..., 1] = -1
    assert np.array_equal(orc.sparse_mqa(q, kv, sel, 0.4, window=(wkv, 0, 2, 0)), orc.sparse_mqa(q, kv, sel, 0.4))
    one = np.zeros((B, T, 1), np.int32)          # entry 0 selected by every query
    both = orc.sparse_mqa(q, kv, one, 0.4, window=(wkv, 3, 3, 1))   # plus the row at its own position
    for t in range(T):
        rows = np.stack([kv[0, 0], wkv[0, t]])
        for h in range(H):
            w = softmax(0.4 * rows @ q[0, t, h])
            assert np.allclose(both[0, t, h], w @ rows, rtol=1e-12, atol=1e-14)


def test_dense_mqa_with_window_equals_masked_attention_over_both(orc):
    """HCA dense attention plus the sliding-window branch (the notes page §1.3 gives the window
    to HCA too): brute force over the concatenation [HCA entries, raw rows] with an explicit
    mask (entry s iff m'(s+1)-1 <= p; raw row j iff its position lies in [p - n_win + 1, p]) and
    scipy's softmax, written here independently of the oracle.  Covers queries that see no
    entry (window only), window rows whose tokens an entry also covers, and a sink."""
    r = np.random.RandomState(21)
    B, T, H, c, mp, N, W, n_win = 2, 7, 3, 8, 4, 6, 12, 5
    q0, wp0 = 2, 1                     # queries at positions 2..8; raw rows at positions 1..12
    q, kv, wkv = r.randn(B, T, H, c), r.randn(B, N, c), r.randn(B, W, c)
    sink = r.randn(H)
    for sk in (None, sink):
        out = orc.hca_dense_mqa(q, kv, mp, 0.3, q_pos0=q0, sink=sk, window=(wkv, wp0, n_win))
        for b in range(B):
            for t in range(T):
                p = q0 + t
                rows = [kv[b, s] for s in range(N) if mp * (s + 1) - 1 <= p]
                rows += [wkv[b, j] for j in range(W) if p - n_win + 1 <= wp0 + j <= p]
                rows = np.stack(rows)
                for h in range(H):
                    z = 0.3 * rows @ q[b, t, h]
                    if sk is None:
                        wgt = softmax(z)
                    else:
                        e = np.exp(z - z.max())
                        wgt = e / (e.sum() + np.exp(sk[h] - z.max()))
                    assert np.allclose(out[b, t, h], wgt @ rows, rtol=1e-12, atol=1e-13)
    # n_win = 0 is plain dense attention
    assert np.allclose(orc.hca_dense_mqa(q, kv, mp, 0.3, q_pos0=q0, window=(wkv, wp0, 0)),
                       orc.hca_dense_mqa(q, kv, mp, 0.3, q_pos0=q0), rtol=1e-13, atol=1e-14)
