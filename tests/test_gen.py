"""Checks of the seeded input generator (shared by the oracle and the GPU tests)."""
import numpy as np
import torch

import gen
from gen import configs


def test_counter_based_and_deterministic():
    a = gen.normal(7, gen.TAG_X, 1000, (500,))
    b = gen.normal(7, gen.TAG_X, 0, (2000,))
    np.testing.assert_array_equal(a, b[1000:1500])  # element i does not depend on the fill range
    assert not np.array_equal(a, gen.normal(8, gen.TAG_X, 1000, (500,)))
    assert not np.array_equal(a, gen.normal(7, gen.TAG_WG, 1000, (500,)))
    assert gen.normal(7, gen.TAG_X, 1003, (1,))[0] == gen.lib().gen_normal(7, gen.TAG_X, 1003, 1.0)


def test_segments_fill_matches_plain_fill():
    n, seg = 7, 1000
    src = np.array([5, 100000, 3, 77, 0, 999999, 12345], dtype=np.uint64)
    dst = np.zeros(n * seg + 10, dtype=np.uint16)
    off = np.arange(n, dtype=np.int64)[::-1] * seg + 3
    gen.fill_segments_ptr(3, gen.TAG_WD, src, seg, 0.5, gen.BF16, dst.ctypes.data, off)
    for s in range(n):
        want = gen.normal(3, gen.TAG_WD, int(src[s]), (seg,), 0.5, gen.BF16)
        np.testing.assert_array_equal(dst[off[s]:off[s] + seg], want)


def test_normal_moments_and_support():
    z = gen.normal(1, gen.TAG_MISC, 0, (2_000_000,))
    assert abs(z.mean()) < 3e-3 and abs(z.var() - 1.0) < 3e-3
    assert np.all(np.abs(z) <= 6.0)
    # Irwin-Hall(12) kurtosis is 3 - 1.2/12 = 2.9
    assert abs(np.mean(z ** 4) - 2.9) < 0.03
    s = gen.normal(1, gen.TAG_MISC, 0, (100_000,), sd=1 / 64)
    np.testing.assert_array_equal(s, z[:100_000] * np.float32(1 / 64))


def test_bf16_is_round_to_nearest_even_of_fp32():
    f = gen.normal(2, gen.TAG_WG, 0, (100_000,), 0.03)
    b = gen.normal(2, gen.TAG_WG, 0, (100_000,), 0.03, gen.BF16)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_rank_perm_is_a_permutation_and_zipf_bias():
    r = gen.rank_perm(5, gen.TAG_RANK, 256)
    np.testing.assert_array_equal(np.sort(r), np.arange(1, 257))
    b = gen.zipf_bias(5, gen.TAG_RANK, 256, 0.2, 1.1)
    np.testing.assert_allclose(b, -0.2 * 1.1 * np.log(r.astype(np.float64)), rtol=1e-6, atol=1e-7)


def test_routing_logits_keep_topk_gap():
    w = configs.with_(configs.DECODE, T=512)
    lg = configs.gen_logits(w)
    s = -np.sort(-lg, axis=1)
    assert np.all(s[:, w.k - 1].astype(np.float64) - s[:, w.k].astype(np.float64) >= 1e-3)
    # the Zipf tilt makes low ranks popular
    rank = gen.rank_perm(w.seed, gen.TAG_RANK, w.E)
    top = np.argsort(-lg, axis=1)[:, :w.k].ravel()
    counts = np.bincount(top, minlength=w.E)
    assert counts[np.argsort(rank)[:16]].sum() > counts[np.argsort(rank)[-16:]].sum()


def test_markov_routing_locality():
    w = configs.LRU_DECODE
    ids, _ = gen.markov_routing(w.seed, 40, 2, w.T, w.E, w.k, w.p_stay, w.zipf_s)
    for row in ids.reshape(-1, w.k):
        assert len(set(row.tolist())) == w.k
    same = np.mean(ids[1:] == ids[:-1])
    assert 0.65 < same < 0.85  # p_stay = 0.7 plus Zipf re-draws that land on the same id
