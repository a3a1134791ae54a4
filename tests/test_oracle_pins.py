"""Pins of the oracle's layer arithmetic against things other than itself.

Every test here runs on the CPU.  Each checks the oracle against a library
routine, a closed form, a special case or brute force, chosen so that a dropped
term, a wrong sign, a wrong index or a transposed operand fails at least one.
"""
import numpy as np
import pytest
from scipy.special import expit, softmax

import gen
import oracle


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- top-k routing (a2)
@pytest.mark.parametrize("E,k", [(8, 2), (16, 5), (33, 7), (64, 16), (5, 5)])
def test_route_ids_equal_bruteforce_full_sort(E, k):
    """ids = the first k of Python's sorted() by (-logit, id): brute force on tiny inputs."""
    r = _rng(E * 100 + k)
    T = 40
    lg = r.integers(-3, 4, size=(T, E)).astype(np.float32) * 0.5  # many exact ties
    lg[0, :] = 0.0
    lg[1, ::2] = -0.0  # signed zeros compare equal to +0
    ids, _ = oracle.route(lg, k)
    for t in range(T):
        want = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
        assert list(ids[t]) == want
    # the same order from a library stable sort of the negated logits
    np.testing.assert_array_equal(ids, np.argsort(-lg, axis=1, kind="stable")[:, :k])


def test_route_all_equal_logits_gives_lowest_ids_and_uniform_gate():
    lg = np.full((3, 10), 0.25, dtype=np.float32)
    ids, w = oracle.route(lg, 4)
    np.testing.assert_array_equal(ids, np.tile(np.arange(4), (3, 1)))
    np.testing.assert_array_equal(w, np.full((3, 4), 1.0 / 4.0))


def test_gate_k1_is_exactly_one():
    lg = _rng(1).standard_normal((20, 12)).astype(np.float32)
    ids, w = oracle.route(lg, 1)
    np.testing.assert_array_equal(ids[:, 0], np.argmax(lg, axis=1))
    np.testing.assert_array_equal(w, np.ones((20, 1)))


def test_gate_k2_equals_logistic_of_logit_gap():
    """k=2: w0 = sigma(l0 - l1), w1 = sigma(l1 - l0) (closed form of a 2-way softmax)."""
    lg = (_rng(2).standard_normal((50, 9)) * 3).astype(np.float32)
    ids, w = oracle.route(lg, 2)
    l0 = lg[np.arange(50), ids[:, 0]].astype(np.float64)
    l1 = lg[np.arange(50), ids[:, 1]].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], expit(l0 - l1), rtol=1e-14, atol=0)
    np.testing.assert_allclose(w[:, 1], expit(l1 - l0), rtol=1e-13, atol=1e-300)
    assert np.all(w[:, 0] >= w[:, 1])


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (256, 6), (128, 8)])
def test_gate_is_full_softmax_renormalised_over_topk(E, k):
    """w = softmax over all E (scipy), restricted to the chosen ids and renormalised."""
    lg = (_rng(E + k).standard_normal((30, E)) * 2).astype(np.float32)
    ids, w = oracle.route(lg, k)
    full = softmax(lg.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids, axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=k * 2.0 ** -52)
    assert np.all(np.diff(w, axis=1) <= 0)  # descending logits -> descending gates


# ---------------------------------------------------------------- grouping (a5)
@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (16, 2, 8), (37, 6, 256), (300, 8, 128), (5, 3, 64)])
def test_permute_against_library_routines(T, k, E):
    r = _rng(T * k + E)
    ids = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = oracle.permute(ids, E)
    flat = ids.ravel()
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(perm, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(inv[perm], np.arange(T * k))
    assert counts.sum() == T * k and offsets[-1] == T * k


def test_permute_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 8]], dtype=np.int32), 8)
    with pytest.raises(ValueError):
        oracle.permute(np.array([[-1, 0]], dtype=np.int32), 8)


# ---------------------------------------------------------------- expert FFN (a6) and combine (a7)
def _silu(z):
    return z * expit(z)


def _dense_swiglu(x, wg, wu, wd):
    """Textbook dense SwiGLU FFN with float64 numpy matmuls."""
    x, wg, wu, wd = (np.asarray(a, dtype=np.float64) for a in (x, wg, wu, wd))
    return (_silu(x @ wg.T) * (x @ wu.T)) @ wd.T


def _experts(seed, E, d, f, dtype=np.float32):
    r = _rng(seed)
    ex = {}
    for e in range(E):
        ex[e] = tuple((r.standard_normal(s) / np.sqrt(d)).astype(np.float32)
                      for s in ((f, d), (f, d), (d, f)))
    return ex


def test_single_expert_layer_equals_dense_swiglu():
    """E=1, k=1: the layer is one dense SwiGLU FFN (d != f catches a transposed operand)."""
    T, d, f = 7, 24, 40
    x = _rng(3).standard_normal((T, d)).astype(np.float32)
    ex = _experts(4, 1, d, f)
    table = oracle.ExpertTable(1, ex)
    ids, w, out = oracle.moe_layer(x, np.zeros((T, 1), np.float32), 1, table)
    np.testing.assert_array_equal(ids, 0)
    np.testing.assert_array_equal(w, 1.0)
    np.testing.assert_allclose(out, _dense_swiglu(x, *ex[0]), rtol=1e-12, atol=1e-14)


def test_equal_logits_all_experts_is_mean_of_dense_ffns():
    """k=E with all logits equal: out = mean over experts of the dense FFNs."""
    T, d, f, E = 5, 16, 20, 4
    x = _rng(5).standard_normal((T, d)).astype(np.float32)
    ex = _experts(6, E, d, f)
    table = oracle.ExpertTable(E, ex)
    _, w, out = oracle.moe_layer(x, np.full((T, E), 1.5, np.float32), E, table)
    np.testing.assert_array_equal(w, 0.25)
    want = np.mean([_dense_swiglu(x, *ex[e]) for e in range(E)], axis=0)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)


def test_two_experts_weighted_sum_with_logistic_gates():
    """k=2 of E=3: out = sigma(l0-l1) FFN_a + sigma(l1-l0) FFN_b with a, b the two largest."""
    T, d, f, E = 6, 12, 18, 3
    x = _rng(7).standard_normal((T, d)).astype(np.float32)
    lg = _rng(8).standard_normal((T, E)).astype(np.float32)
    ex = _experts(9, E, d, f)
    table = oracle.ExpertTable(E, ex)
    ids, _, out = oracle.moe_layer(x, lg, 2, table)
    for t in range(T):
        a, b = np.argsort(-lg[t], kind="stable")[:2]
        ga = expit(float(lg[t, a]) - float(lg[t, b]))
        want = ga * _dense_swiglu(x[t:t + 1], *ex[a]) + (1 - ga) * _dense_swiglu(x[t:t + 1], *ex[b])
        np.testing.assert_allclose(out[t], want[0], rtol=1e-12, atol=1e-13)


def test_silu_closed_form_values():
    """d=f=1, all weights 1: y = x * SiLU(x); SiLU(1) = e/(1+e), SiLU(-1) = -1/(1+e)."""
    x = np.array([[1.0], [-1.0], [0.0]], dtype=np.float32)
    one = np.ones((1, 1), np.float32)
    table = oracle.ExpertTable(1, {0: (one, one, one)})
    _, _, out = oracle.moe_layer(x, np.zeros((3, 1), np.float32), 1, table)
    e = np.e
    np.testing.assert_allclose(out[:, 0], [e / (1 + e), 1 / (1 + e), 0.0], rtol=1e-15, atol=0)


def test_expert_ffn_rows_match_dense_per_assignment():
    T, d, f, E, k = 9, 16, 24, 5, 2
    x = _rng(10).standard_normal((T, d)).astype(np.float32)
    ex = _experts(11, E, d, f)
    table = oracle.ExpertTable(E, ex)
    ids, _ = oracle.route(_rng(12).standard_normal((T, E)).astype(np.float32), k)
    assign = np.arange(T * k, dtype=np.int32)[::-1].copy()
    y = oracle.expert_ffn(x, ids, table, assign)
    for q, a in enumerate(assign):
        t, e = a // k, ids.ravel()[a]
        np.testing.assert_allclose(y[q], _dense_swiglu(x[t:t + 1], *ex[e])[0], rtol=1e-12,
                                   atol=1e-14)


def test_bf16_weights_are_upcast_exactly():
    """bf16 bit patterns give the same result as their exact fp32 upcast."""
    T, d, f, E, k = 4, 16, 8, 2, 1
    xb = gen.normal(1, gen.TAG_X, 0, (T, d), 1.0, gen.BF16)
    exb = {e: (gen.normal(1, gen.TAG_WG, e * 1000, (f, d), 0.25, gen.BF16),
               gen.normal(1, gen.TAG_WU, e * 1000, (f, d), 0.25, gen.BF16),
               gen.normal(1, gen.TAG_WD, e * 1000, (d, f), 0.25, gen.BF16)) for e in range(E)}
    exf = {e: tuple(gen.bf16_bits_to_f32(a) for a in v) for e, v in exb.items()}
    lg = _rng(13).standard_normal((T, E)).astype(np.float32)
    _, _, ob = oracle.moe_layer(xb, lg, k, oracle.ExpertTable(E, exb))
    _, _, of = oracle.moe_layer(gen.bf16_bits_to_f32(xb), lg, k, oracle.ExpertTable(E, exf))
    np.testing.assert_array_equal(ob, of)


def test_layer_is_equivariant_under_token_permutation():
    """Permuting the rows of x and logits permutes ids, w and out (bit-exact)."""
    T, d, f, E, k = 12, 16, 24, 6, 3
    x = _rng(14).standard_normal((T, d)).astype(np.float32)
    lg = _rng(15).standard_normal((T, E)).astype(np.float32)
    table = oracle.ExpertTable(E, _experts(16, E, d, f))
    ids, w, out = oracle.moe_layer(x, lg, k, table)
    p = _rng(17).permutation(T)
    ids2, w2, out2 = oracle.moe_layer(x[p], lg[p], k, table)
    np.testing.assert_array_equal(ids2, ids[p])
    np.testing.assert_array_equal(w2, w[p])
    np.testing.assert_array_equal(out2, out[p])


def test_combine_one_hot_gate_selects_rows():
    T, k, d = 6, 3, 5
    yperm = _rng(18).standard_normal((T * k, d))
    inv = _rng(19).permutation(T * k).astype(np.int32)
    w = np.zeros((T, k))
    w[:, 1] = 1.0
    out = oracle.combine(yperm, inv, w)
    np.testing.assert_array_equal(out, yperm[inv.reshape(T, k)[:, 1]])


def test_combine_composed_with_ffn_equals_layer():
    T, d, f, E, k = 10, 16, 12, 6, 3
    x = _rng(20).standard_normal((T, d)).astype(np.float32)
    lg = _rng(21).standard_normal((T, E)).astype(np.float32)
    table = oracle.ExpertTable(E, _experts(22, E, d, f))
    ids, w, out = oracle.moe_layer(x, lg, k, table)
    _, _, perm, inv = oracle.permute(ids, E)
    yperm = oracle.expert_ffn(x, ids, table, perm)
    np.testing.assert_allclose(oracle.combine(yperm, inv, w), out, rtol=1e-13, atol=1e-15)


def test_router_logits_against_float64_matmul():
    x = _rng(23).standard_normal((16, 256)).astype(np.float32)
    wr = (_rng(24).standard_normal((8, 256)) / 16).astype(np.float32)
    lg = oracle.router_logits(x, wr)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T
    np.testing.assert_allclose(lg, ref, rtol=2 ** -23, atol=1e-7)
