"""Helpers shared by the GPU parity tests: upload, oracle comparison rules."""
from __future__ import annotations

import numpy as np

import oracle

TOL_REL = 2e-3
TOL_ABS = 1e-5
NEAR_TIE = 2.0 ** -40


def y_tolerance(y_ref: np.ndarray) -> float:
    """Per-element bound |gpu - oracle| <= 2e-3 * max|oracle| + 1e-5 (max over the call's y)."""
    return TOL_REL * float(np.abs(y_ref).max()) + TOL_ABS


def assert_y_close(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = ""):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = y_tolerance(y_ref)
    worst = float(err.max()) if err.size else 0.0
    assert np.isfinite(y_gpu).all(), f"{what}: non-finite GPU output"
    assert worst <= tol, f"{what}: max |gpu - oracle| = {worst:.4e} > tol {tol:.4e}"
    return worst, tol


def routing_mismatches(layer, x64: np.ndarray, ids_gpu: np.ndarray, ids_ref: np.ndarray, logits_ref: np.ndarray,
                       gates_pre=None, omit_below: float = 0.0):
    """Tokens whose GPU ids differ from the oracle's.  Returns (excused, unexcused): a
    mismatch is excused only when every differing position is a near-tie the fp64
    evaluation cannot order independently of summation order:
    |l_a - l_b| <= 2^-40 * sum_h |x_h W_eh| (+|b_e|), or, with omission, a pair whose
    oracle gate before omission lies within 2^-40 of the threshold (kept on one side,
    omitted on the other)."""
    excused, bad = [], []
    W = np.asarray(layer.router_w, dtype=np.float64)
    b = None if layer.router_b is None else np.abs(np.asarray(layer.router_b, dtype=np.float64))
    for t in np.nonzero(np.any(ids_gpu != ids_ref, axis=1))[0]:
        mag = np.abs(x64[t])[None, :] @ np.abs(W).T
        mag = mag[0] + (b if b is not None else 0.0)
        ok = True
        for j in range(ids_ref.shape[1]):
            a_, b_ = int(ids_ref[t, j]), int(ids_gpu[t, j])
            if a_ == b_:
                continue
            if (a_ < 0 or b_ < 0) and gates_pre is not None and omit_below > 0 and \
                    abs(gates_pre[t, j] - omit_below) <= NEAR_TIE * omit_below:
                continue
            if not (0 <= a_ < W.shape[0] and 0 <= b_ < W.shape[0]):
                ok = False
                break
            gap = abs(logits_ref[t, a_] - logits_ref[t, b_])
            if gap > NEAR_TIE * max(mag[a_], mag[b_]):
                ok = False
                break
        (excused if ok else bad).append(int(t))
    return excused, bad


def check_forward(layer, x, x_dtype, y_gpu, dbg, ref=None, tokens=None, what="", omit_below: float = 0.0):
    """Compare one moe_forward call with the oracle: ids exact (near-ties excused and
    re-checked with the GPU's routing), gates within 1e-6, bucketing exact (the perm
    entries past the placed pairs are -1), y within tolerance.  `tokens` restricts the y
    and routing comparison to a sample.  omit_below: the layer's omission threshold (the
    fp32 value the descriptor holds)."""
    T = x.shape[0]
    ref = oracle.moe_forward(layer, x, x_dtype, omit_below=omit_below) if ref is None else ref
    x64 = oracle.activations_f64(x, x_dtype)
    ids_gpu = dbg["ids"].cpu().numpy()
    gates_gpu = dbg["gates"].cpu().numpy()
    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    gates_pre = None
    if omit_below > 0:
        gates_pre = oracle.topk_softmax(ref["logits"][sel] if tokens is None else ref["logits"], layer.top_k)[1]
    excused, bad = routing_mismatches(layer, x64[sel], ids_gpu[sel], ref["ids"], ref["logits"], gates_pre, omit_below)
    assert not bad, f"{what}: expert ids differ from the oracle for tokens {bad[:8]}"
    keep = np.setdiff1d(np.arange(len(sel)), excused)
    assert np.abs(gates_gpu[sel][keep] - ref["gates"][keep]).max(initial=0) <= 1e-6, f"{what}: gates"
    if tokens is None:
        placed = int(ref["offsets"][-1])
        perm = dbg["perm"].cpu().numpy()
        assert np.array_equal(dbg["counts"].cpu().numpy(), ref["counts"]), f"{what}: counts"
        assert np.array_equal(dbg["offsets"].cpu().numpy(), ref["offsets"]), f"{what}: offsets"
        assert np.array_equal(perm[:placed], ref["perm"]), f"{what}: perm"
        assert np.all(perm[placed:] == -1), f"{what}: perm past the placed pairs"
    yg = y_gpu.cpu().numpy()[sel]
    yr = ref["y"].copy()
    if excused:
        alt = oracle.moe_forward(layer, x[sel], x_dtype, ids=ids_gpu[sel], gates=gates_gpu[sel].astype(np.float64))
        yr[excused] = alt["y"][excused]
    return assert_y_close(yg, yr, what), len(excused)


MIDPOINT_REL = 2.0 ** -40


def bf16_near_midpoint(q: np.ndarray, rel: float = MIDPOINT_REL) -> np.ndarray:
    """True where the fp64 value q lies within rel * |q| of a point midway between two
    adjacent bfloat16 values: there the rounding direction depends on the last bits of
    the fp64 evaluation (its summation order), not on the definition."""
    q = np.asarray(q, dtype=np.float64)
    m, _ = np.frexp(q)                    # q = m * 2^e, 0.5 <= |m| < 1
    scaled = np.abs(m) * 256.0            # bf16 keeps 8 significant bits
    frac = scaled - np.floor(scaled)
    return np.abs(frac - 0.5) <= rel * scaled


def assert_rescale_exact(got_bits: np.ndarray, y: np.ndarray, what: str = "") -> int:
    """The GPU's bf16 RMS rescale of y equals the oracle's bit for bit, except where the
    oracle's fp64 quotient sits within 2^-40 of a bf16 rounding midpoint (there the
    two may round apart by one step).  Returns the number of excused elements."""
    y = np.asarray(y, dtype=np.float64)
    want = oracle.rms_rescale(y).astype(np.int32)
    got = np.asarray(got_bits).view(np.uint16).astype(np.int32)
    near = bf16_near_midpoint(oracle.rms_quotient(y))
    diff = got != want
    bad = diff & ~(near & (np.abs(got - want) <= 1))
    assert not bad.any(), f"{what}: {int(bad.sum())} rescaled values differ from the oracle's"
    return int(near.sum())
