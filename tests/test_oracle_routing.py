"""Pins of the oracle's router, top-k gating and bucketing: brute force over subsets,
special cases, 50-digit decimal arithmetic and textbook library routines."""
import itertools
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
import synth


def _brute_topk(l, k):
    """The unique k-subset S with l_i > l_j, or l_i == l_j and i < j, for every i in S and
    j outside S; returned in (-l, index) order by pairwise comparison (selection sort)."""
    E = len(l)
    found = []
    for S in itertools.combinations(range(E), k):
        out = [j for j in range(E) if j not in S]
        if all(l[i] > l[j] or (l[i] == l[j] and i < j) for i in S for j in out):
            found.append(list(S))
    assert len(found) == 1
    S = found[0]
    ordered = []
    while S:
        best = S[0]
        for c in S[1:]:
            if l[c] > l[best] or (l[c] == l[best] and c < best):
                best = c
        ordered.append(best)
        S.remove(best)
    return ordered


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_topk_brute_force_subsets(k):
    rng = np.random.default_rng(11 + k)
    for trial in range(40):
        l = rng.standard_normal((1, 8))
        if trial % 4 == 0:   # exact ties
            l[0, rng.integers(8)] = l[0, rng.integers(8)]
            l[0, 5] = l[0, 2]
        ids, g = oracle.topk_softmax(l, k)
        assert list(ids[0]) == _brute_topk(list(l[0]), k)


def test_gates_equal_renormalised_full_softmax():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((6, 32)) * 3
    ids, g = oracle.topk_softmax(l, 5)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    for t in range(6):
        sel = p[t, ids[t]]
        assert np.allclose(g[t], sel / sel.sum(), rtol=1e-14, atol=0)
        assert abs(g[t].sum() - 1.0) < 1e-15 * 4
        assert np.all(np.diff(g[t]) <= 0)   # descending logits -> descending gates


def test_gates_decimal_50_digits():
    getcontext().prec = 50
    rng = np.random.default_rng(9)
    l = rng.standard_normal((3, 10))
    ids, g = oracle.topk_softmax(l, 4)
    for t in range(3):
        z = [Decimal(float(l[t, e])).exp() for e in ids[t]]
        s = sum(z)
        for j in range(4):
            assert abs(float(z[j] / s) - g[t, j]) <= 2e-16


def test_k1_and_k_equals_E():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((5, 7))
    ids, g = oracle.topk_softmax(l, 1)
    assert np.all(g == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(l, axis=1))
    ids, g = oracle.topk_softmax(l, 7)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    for t in range(5):
        assert sorted(ids[t]) == list(range(7))
        assert np.allclose(g[t], p[t, ids[t]], rtol=1e-14)


def test_duplicate_router_rows_tie_to_lower_index():
    rng = np.random.default_rng(6)
    H, E = 64, 8
    W = rng.standard_normal((E, H)).astype(np.float32)
    W[5] = W[2]          # experts 2 and 5 always tie exactly
    W[7] = W[2]
    x = rng.standard_normal((20, H)).astype(np.float32)
    l = oracle.router_logits(x.astype(np.float64), W, None)
    assert np.array_equal(l[:, 2], l[:, 5]) and np.array_equal(l[:, 2], l[:, 7])
    ids, _ = oracle.topk_softmax(l, 3)
    for t in range(20):
        pos = {int(e): j for j, e in enumerate(ids[t])}
        for a, b in [(2, 5), (5, 7), (2, 7)]:
            if a in pos and b in pos:
                assert pos[a] < pos[b]
            if b in pos:
                assert a in pos   # the lower index is never dropped in favour of the higher


def test_router_logits_decimal_exact():
    """fp32 x and W products are exact in decimal; the oracle must be within fp64 rounding."""
    getcontext().prec = 60
    rng = np.random.default_rng(8)
    H, E, T = 96, 5, 3
    x = rng.standard_normal((T, H)).astype(np.float32)
    W = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    l = oracle.router_logits(x.astype(np.float64), W, b)
    for t in range(T):
        for e in range(E):
            exact = sum(Decimal(float(x[t, h])) * Decimal(float(W[e, h])) for h in range(H)) + Decimal(float(b[e]))
            mag = sum(abs(float(x[t, h]) * float(W[e, h])) for h in range(H)) + abs(float(b[e]))
            assert abs(Decimal(l[t, e]) - exact) <= Decimal(H * 2.0 ** -52 * mag)


def test_bf16_activation_decoding():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    v = oracle.activations_f64(bits, oracle.X_BF16)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 3.140625 and v[3] == 0 and np.signbit(v[4])
    assert v[5] == (2 - 2 ** -7) * 2.0 ** 127


@pytest.mark.parametrize("has_shared", [0, 1])
def test_bucket_against_library_routines(has_shared):
    rng = np.random.default_rng(12)
    for T, k, E in [(1, 4, 128), (17, 8, 256), (64, 2, 8), (300, 6, 40), (5, 1, 3)]:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets, perm, inv = oracle.bucket(ids, E, has_shared)
        flat = ids.reshape(-1)
        expert_of = np.concatenate([flat, np.full(T * has_shared, E)])
        assert np.array_equal(counts, np.bincount(expert_of, minlength=E + 1))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
        assert np.array_equal(perm, np.argsort(expert_of, kind="stable"))
        assert np.array_equal(perm[inv], np.arange(perm.size))
        assert np.array_equal(inv[perm], np.arange(perm.size))
        assert counts.sum() == T * k + T * has_shared
        for e in range(E + 1):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.all(expert_of[seg] == e) and np.all(np.diff(seg) > 0)


def test_shared_gate_weights():
    x = np.array([[1.0, 2.0], [0.0, 0.0], [-3.0, 1.0]])
    w = np.array([0.5, -0.25])
    s = oracle.shared_weights(x, w)
    assert np.allclose(s, [0.5, 0.5, 1 / (1 + np.exp(1.75))], rtol=1e-15)
    assert np.all(oracle.shared_weights(x, None) == 1.0)


# ---------------------------------------------------------------------------
# Marginal-expert omission ("Nebula" page, "Benchmark results": a 10% threshold)
# ---------------------------------------------------------------------------
def test_omission_hand_worked_row():
    """Logits 0, -1, -2, -3, -5 with k = 4: gates e^-j / (1 + e^-1 + e^-2 + e^-3), i.e.
    0.6439, 0.2369, 0.0871, 0.0321; at 10 % the last two go and the kept ones become
    1 / (1 + e^-1) and e^-1 / (1 + e^-1)."""
    l = np.array([[0.0, -1.0, -2.0, -3.0, -5.0]])
    ids, g = oracle.topk_softmax(l, 4)
    assert np.array_equal(ids[0], [0, 1, 2, 3])
    s = 1 + np.exp(-1) + np.exp(-2) + np.exp(-3)
    assert np.allclose(g[0], [1 / s, np.exp(-1) / s, np.exp(-2) / s, np.exp(-3) / s], rtol=1e-15, atol=0)
    ids2, g2 = oracle.omit_marginal(ids, g, 0.1)
    assert np.array_equal(ids2[0], [0, 1, -1, -1])
    assert np.allclose(g2[0], [1 / (1 + np.exp(-1)), np.exp(-1) / (1 + np.exp(-1)), 0, 0], rtol=1e-15, atol=0)


def test_omission_zero_threshold_keeps_everything():
    rng = np.random.default_rng(5)
    l = rng.normal(size=(20, 16))
    ids, g = oracle.topk_softmax(l, 6)
    ids2, g2 = oracle.omit_marginal(ids, g, 0.0)
    assert np.array_equal(ids2, ids) and np.array_equal(g2, g)


def test_omission_definition_brute_force():
    """On random rows: a pair is omitted exactly when its gate is below tau and it is not
    the first; every kept pair keeps its expert; kept gates sum to 1 and keep their
    ratios (renormalised by the kept total)."""
    rng = np.random.default_rng(6)
    for tau in (0.05, 0.1, 0.2, 0.5):
        l = rng.normal(scale=2.0, size=(40, 24))
        ids, g = oracle.topk_softmax(l, 8)
        ids2, g2 = oracle.omit_marginal(ids, g, tau)
        for t in range(40):
            kept = [j for j in range(8) if j == 0 or g[t, j] >= tau]
            assert all(ids2[t, j] == (ids[t, j] if j in kept else -1) for j in range(8))
            assert abs(g2[t].sum() - 1.0) < 1e-15
            tot = sum(g[t, j] for j in kept)
            assert all(abs(g2[t, j] - g[t, j] / tot) < 1e-16 for j in kept)
            assert all(g2[t, j] == 0.0 for j in range(8) if j not in kept)


def test_omission_threshold_one_is_top1_routing():
    """tau = 1 keeps only the first pair (its gate is below 1 whenever k > 1 and the
    logits are finite) with weight 1: the layer equals the same layer routed top-1."""
    import copy
    spec = synth.small_spec("om1", 6, 64, 32, 6, 3, synth.WFMT_CB4, has_shared=1, bias="normal", seed=13)
    layer = synth.make_layer(spec)
    x = synth.make_x(spec)
    r = oracle.moe_forward(layer, x, spec.x_dtype, omit_below=1.0)
    l1 = copy.copy(layer)
    l1.spec = copy.copy(layer.spec)
    l1.spec.top_k = 1
    r1 = oracle.moe_forward(l1, x, spec.x_dtype)
    assert np.array_equal(r["ids"][:, 0], r1["ids"][:, 0]) and np.all(r["ids"][:, 1:] == -1)
    assert np.array_equal(r["y"], r1["y"])


def test_omission_bucketing_leaves_omitted_pairs_out():
    ids = np.array([[3, -1, 0], [3, 1, -1]], dtype=np.int32)
    counts, offsets, perm, inv = oracle.bucket(ids, 4, 1)
    assert list(counts) == [1, 1, 0, 2, 2]
    assert list(offsets) == [0, 1, 2, 2, 4, 6]
    assert list(perm) == [2, 4, 0, 3, 6, 7]
    assert list(inv) == [2, -1, 0, 3, 1, -1, 4, 5]
