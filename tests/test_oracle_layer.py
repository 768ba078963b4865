"""Pins of the oracle's whole-layer output: a dense evaluation of every expert masked by
the gates (a different algorithm: no bucketing), 50-digit decimal arithmetic on a tiny
layer, closed forms for single-nonzero weights, and invariants."""
import copy
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
import packing
import synth


def _dense_masked(layer, x, x_dtype):
    """y = sum over ALL experts e of M[t,e] * FFN_e(x_t) + s_t * FFN_shared(x_t), where
    M[t,e] is the gate of e for token t if selected, else 0."""
    x64 = oracle.activations_f64(x, x_dtype)
    T, E, k, I, H = x64.shape[0], layer.n_experts, layer.top_k, layer.inter, layer.hidden
    l = oracle.router_logits(x64, layer.router_w, layer.router_b)
    ids, g = oracle.topk_softmax(l, k)
    M = np.zeros((T, E))
    for t in range(T):
        M[t, ids[t]] = g[t]
    y = np.zeros((T, H))
    for e in range(E):
        wgu = oracle.dequant(layer.wfmt, layer.gate_up[e], layer.codebook, 2 * I, H)
        wd = oracle.dequant(layer.wfmt, layer.down[e], layer.codebook, H, I)
        a = x64 @ wgu.T
        hh = (a[:, :I] / (1 + np.exp(-a[:, :I]))) * a[:, I:]
        y += M[:, e:e + 1] * (hh @ wd.T)
    if layer.has_shared:
        wgu = oracle.dequant(layer.wfmt, layer.gate_up[E], layer.codebook, 2 * I, H)
        wd = oracle.dequant(layer.wfmt, layer.down[E], layer.codebook, H, I)
        a = x64 @ wgu.T
        hh = (a[:, :I] / (1 + np.exp(-a[:, :I]))) * a[:, I:]
        s = np.ones(T) if layer.shared_gate_w is None else \
            1 / (1 + np.exp(-(x64 @ layer.shared_gate_w.astype(np.float64))))
        y += s[:, None] * (hh @ wd.T)
    return y


CASES = [
    # name, T, H, I, E, k, wfmt, shared, x dtype, bias, shared_gate
    ("cb4_f32", 5, 64, 32, 8, 2, synth.WFMT_CB4, 0, synth.X_F32, "none", False),
    ("cb4_shared", 6, 96, 64, 6, 3, synth.WFMT_CB4, 1, synth.X_BF16, "normal", False),
    ("cb4_shared_gate", 4, 64, 32, 5, 2, synth.WFMT_CB4, 1, synth.X_BF16, "zipf", True),
    ("mx_bf16", 3, 128, 64, 8, 4, synth.WFMT_MXFP4, 0, synth.X_BF16, "normal", False),
    ("mx_k1", 7, 64, 64, 4, 1, synth.WFMT_MXFP4, 1, synth.X_F32, "none", False),
    ("mx_kE", 2, 64, 32, 4, 4, synth.WFMT_MXFP4, 0, synth.X_BF16, "none", False),
]


def _mk(case, seed=21):
    name, T, H, I, E, k, wfmt, sh, xd, bias, sg = case
    spec = synth.small_spec(name, T, H, I, E, k, wfmt, has_shared=sh, x_dtype=xd, bias=bias, seed=seed)
    layer = synth.make_layer(spec, shared_gate=sg)
    return spec, layer, synth.make_x(spec)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dense_masked_evaluation(case):
    spec, layer, x = _mk(case)
    r = oracle.moe_forward(layer, x, spec.x_dtype)
    yd = _dense_masked(layer, x, spec.x_dtype)
    scale = np.abs(yd).max()
    assert scale > 0
    assert np.abs(r["y"] - yd).max() <= 1e-12 * scale


def _decimal_layer(layer, x, x_dtype, digits=50):
    """The tiny layer in 50-digit decimal arithmetic, decoding the packed bytes with the
    OCP table and fp16 fields written out independently of the oracle."""
    getcontext().prec = digits
    E2M1 = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]

    def dec_matrix(packed, rows, cols):
        p = bytes(np.asarray(packed, dtype=np.uint8))
        off = ((rows * cols // 2) + 255) // 256 * 256
        out = []
        for r in range(rows):
            row = []
            for c in range(cols):
                byte = p[(r * cols + c) // 2]
                code = byte & 0xF if c % 2 == 0 else byte >> 4
                bi = (r * cols + c) // 32
                if layer.wfmt == synth.WFMT_MXFP4:
                    s = Decimal(2) ** (p[off + bi] - 127)
                    v = Decimal(E2M1[code])
                else:
                    bits = p[off + 2 * bi] | (p[off + 2 * bi + 1] << 8)
                    ex, fr = (bits >> 10) & 31, bits & 1023
                    s = (Decimal(1024 + fr) * Decimal(2) ** (ex - 25)) if ex else Decimal(fr) * Decimal(2) ** -24
                    s = -s if bits >> 15 else s
                    v = Decimal(int(layer.codebook[code]))
                row.append(s * v)
            out.append(row)
        return out

    if x_dtype == synth.X_BF16:
        xs = [[Decimal(float(np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0])) for b in r] for r in x]
    else:
        xs = [[Decimal(float(v)) for v in r] for r in x]
    T, H, I, E, k = len(xs), layer.hidden, layer.inter, layer.n_experts, layer.top_k
    W = [[Decimal(float(v)) for v in r] for r in layer.router_w]
    b = [Decimal(float(v)) for v in layer.router_b] if layer.router_b is not None else [Decimal(0)] * E
    logits = [[sum(xs[t][h] * W[e][h] for h in range(H)) + b[e] for e in range(E)] for t in range(T)]
    y = [[Decimal(0)] * H for _ in range(T)]
    mats = {}
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t][e], e))[:k]
        z = [(logits[t][e] - logits[t][order[0]]).exp() for e in order]
        zs = sum(z)
        experts = [(e, z[j] / zs) for j, e in enumerate(order)]
        if layer.has_shared:
            experts.append((E, Decimal(1)))
        for e, gate in experts:
            if e not in mats:
                mats[e] = (dec_matrix(layer.gate_up[e], 2 * I, H), dec_matrix(layer.down[e], H, I))
            gu, dn = mats[e]
            a = [sum(gu[i][h] * xs[t][h] for h in range(H)) for i in range(2 * I)]
            hh = [a[i] / (1 + (-a[i]).exp()) * a[I + i] for i in range(I)]
            for n in range(H):
                y[t][n] += gate * sum(dn[n][i] * hh[i] for i in range(I))
    return np.array([[float(v) for v in r] for r in y])


@pytest.mark.parametrize("wfmt,xd,sh", [(synth.WFMT_CB4, synth.X_F32, 1), (synth.WFMT_MXFP4, synth.X_BF16, 0)])
def test_decimal_50_digits_tiny_layer(wfmt, xd, sh):
    spec = synth.small_spec("dec", 2, 32, 32, 4, 2, wfmt, has_shared=sh, x_dtype=xd, bias="normal", seed=5)
    layer = synth.make_layer(spec)
    x = synth.make_x(spec)
    y_exact = _decimal_layer(layer, x, spec.x_dtype)
    y = oracle.moe_forward(layer, x, spec.x_dtype)["y"]
    assert np.abs(y - y_exact).max() <= 1e-13 * np.abs(y_exact).max()


def _packed_from_dense_codes(wfmt, codes, scale_byte_or_bits):
    rows, cols = codes.shape
    return packing.pack(wfmt, codes, np.full((rows, cols // 32), scale_byte_or_bits))


def test_single_nonzero_closed_form():
    """gate row i reads x_a, up row i reads x_b, down row n reads h_i (all weight 1):
    the expert output is silu(x_a) * x_b at position n, times its gate."""
    H, I, E, k, T = 64, 32, 3, 2, 4
    spec = synth.small_spec("one", T, H, I, E, k, synth.WFMT_MXFP4, x_dtype=synth.X_F32, seed=3)
    layer = synth.make_layer(spec)
    ONE = 2  # E2M1 code of 1.0
    placement = {0: (5, 40, 7, 3), 1: (63, 0, 12, 50), 2: (10, 10, 31, 0)}  # e: (a, b, i, n)
    for e, (a, b, i, n) in placement.items():
        gu = np.zeros((2 * I, H), dtype=np.uint8)
        gu[i, a] = ONE
        gu[I + i, b] = ONE
        dn = np.zeros((H, I), dtype=np.uint8)
        dn[n, i] = ONE
        layer.gate_up[e] = _packed_from_dense_codes(synth.WFMT_MXFP4, gu, 127)
        layer.down[e] = _packed_from_dense_codes(synth.WFMT_MXFP4, dn, 127)
    x = synth.make_x(spec)
    r = oracle.moe_forward(layer, x, synth.X_F32)
    x64 = x.astype(np.float64)
    want = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(r["ids"][t, j])
            a, b, i, n = placement[e]
            want[t, n] += r["gates"][t, j] * (x64[t, a] / (1 + np.exp(-x64[t, a]))) * x64[t, b]
    assert np.allclose(r["y"], want, rtol=1e-14, atol=0)


def test_zero_weights_give_exact_zero():
    spec = synth.small_spec("zero", 3, 64, 32, 4, 2, synth.WFMT_CB4, has_shared=1, seed=4)
    layer = synth.make_layer(spec)
    for e in range(5):
        layer.gate_up[e] = layer.gate_up[e].copy()
        nc = 2 * 32 * 64 // 2
        layer.gate_up[e][nc:] = 0   # every fp16 scale = +0
    x = synth.make_x(spec)
    y = oracle.moe_forward(layer, x, spec.x_dtype)["y"]
    assert np.all(y == 0)


def test_linear_in_gates_and_fixed_routing():
    spec, layer, x = _mk(CASES[1])
    r = oracle.moe_forward(layer, x, spec.x_dtype)
    g1 = r["gates"] * 0.25
    g2 = r["gates"] * 0.75 + 0.1
    y1 = oracle.moe_forward(layer, x, spec.x_dtype, ids=r["ids"], gates=g1)["y"]
    y2 = oracle.moe_forward(layer, x, spec.x_dtype, ids=r["ids"], gates=g2)["y"]
    y12 = oracle.moe_forward(layer, x, spec.x_dtype, ids=r["ids"], gates=g1 + g2)["y"]
    # the shared expert enters y1, y2 and y12 once each
    sh = oracle.moe_forward(layer, x, spec.x_dtype, ids=r["ids"], gates=np.zeros_like(g1))["y"]
    assert np.allclose(y1 + y2 - sh, y12, rtol=1e-12, atol=1e-12 * np.abs(y12).max())
    y = oracle.moe_forward(layer, x, spec.x_dtype, ids=r["ids"], gates=r["gates"])["y"]
    assert np.array_equal(y, r["y"])


def test_relabelling_experts_leaves_y_unchanged():
    spec, layer, x = _mk(CASES[3])
    r = oracle.moe_forward(layer, x, spec.x_dtype)
    perm = np.random.default_rng(1).permutation(spec.n_experts)
    L2 = copy.copy(layer)
    L2.router_w = layer.router_w[perm]
    L2.router_b = layer.router_b[perm] if layer.router_b is not None else None
    L2.gate_up = [layer.gate_up[p] for p in perm] + layer.gate_up[spec.n_experts:]
    L2.down = [layer.down[p] for p in perm] + layer.down[spec.n_experts:]
    r2 = oracle.moe_forward(L2, x, spec.x_dtype)
    assert np.array_equal(perm[r2["ids"]], r["ids"])
    assert np.allclose(r2["y"], r["y"], rtol=1e-14, atol=1e-14 * np.abs(r["y"]).max())


def test_rms_rescale_closed_forms():
    a = 1000.0
    y = np.array([[a, -a, a, -a] * 8, [2.0] * 32])
    out = oracle.rms_rescale(y)
    # rms is |a| (resp. 2): the result is +-1 up to eps/2a^2, which rounds to exactly +-1
    assert np.all(out[0, 0::2] == 0x3F80) and np.all(out[0, 1::2] == 0xBF80)
    assert np.all(out[1] == 0x3F80)
    # a vector with known mean square: [3, 4] -> mean 12.5, 3/sqrt(12.5) = 0.8485...
    out = oracle.rms_rescale(np.array([[3.0, 4.0]]), eps=0.0)
    want = synth.f32_to_bf16_bits(np.array([3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], dtype=np.float32))
    assert np.array_equal(out[0], want)
    # eps is added to the mean, inside the square root: a row of c with c^2 == eps gives
    # c / sqrt(2 c^2) = 1/sqrt(2) = 0.70710..., whose nearest bf16 is 0x3F35 (0.70703125)
    c = np.sqrt(oracle.RMS_EPS)
    assert np.all(oracle.rms_rescale(np.full((1, 64), c)) == 0x3F35)
    # a half-way case: 1 + 2^-8 lies midway between bf16 1.0 and 1.0078125 and rounds to even
    q = oracle.rms_quotient(np.array([[1.0 + 2.0 ** -8, 1.0 - 2.0 ** -8]]), eps=0.0)
    assert abs(q[0, 0] - (1.0 + 2.0 ** -8) / np.sqrt(1.0 + 2.0 ** -16)) < 1e-15


def test_forward_expert_map_on_threads_gives_the_same_values():
    """The per-expert products are independent: evaluating them on a thread pool gives
    the values of the one-after-another evaluation, bit for bit."""
    from concurrent.futures import ThreadPoolExecutor
    spec = synth.small_spec("map", 9, 128, 64, 8, 3, synth.WFMT_CB4, has_shared=1, bias="normal")
    layer = synth.make_layer(spec, shared_gate=True)
    x = synth.make_x(spec)
    r1 = oracle.moe_forward(layer, x, spec.x_dtype)
    with ThreadPoolExecutor(4) as ex:
        r2 = oracle.moe_forward(layer, x, spec.x_dtype, map_fn=ex.map)
    assert np.array_equal(r1["y"], r2["y"]) and np.array_equal(r1["o"], r2["o"])


@pytest.mark.parametrize("case", CASES[:4], ids=[c[0] for c in CASES[:4]])
def test_omission_dense_masked_evaluation(case):
    """With omission the layer is the dense masked evaluation whose mask holds the
    renormalised gates of the kept pairs (a different algorithm: no bucketing)."""
    spec, layer, x = _mk(case, seed=33)
    tau = 0.9 / spec.top_k
    r = oracle.moe_forward(layer, x, spec.x_dtype, omit_below=tau)
    x64 = oracle.activations_f64(x, spec.x_dtype)
    ids, g = oracle.topk_softmax(oracle.router_logits(x64, layer.router_w, layer.router_b), spec.top_k)
    T, E, I, H = x.shape[0], spec.n_experts, spec.inter, spec.hidden
    y = np.zeros((T, H))
    for t in range(T):
        keep = [j for j in range(spec.top_k) if j == 0 or g[t, j] >= tau]
        tot = sum(g[t, j] for j in keep)
        for j in keep:
            e = ids[t, j]
            wgu = oracle.dequant(layer.wfmt, layer.gate_up[e], layer.codebook, 2 * I, H)
            wd = oracle.dequant(layer.wfmt, layer.down[e], layer.codebook, H, I)
            a = x64[t] @ wgu.T
            y[t] += g[t, j] / tot * (((a[:I] / (1 + np.exp(-a[:I]))) * a[I:]) @ wd.T)
    if layer.has_shared:
        wgu = oracle.dequant(layer.wfmt, layer.gate_up[E], layer.codebook, 2 * I, H)
        wd = oracle.dequant(layer.wfmt, layer.down[E], layer.codebook, H, I)
        a = x64 @ wgu.T
        sw = np.ones(T) if layer.shared_gate_w is None else \
            1 / (1 + np.exp(-(x64 @ layer.shared_gate_w.astype(np.float64))))
        y += sw[:, None] * (((a[:, :I] / (1 + np.exp(-a[:, :I]))) * a[:, I:]) @ wd.T)
    assert (r["ids"] == -1).any(), "the case should omit some pairs"
    assert np.abs(r["y"] - y).max() <= 1e-12 * np.abs(y).max()
