"""GPU parity of marginal-expert omission ("Nebula" page, "Benchmark results": experts
whose gate falls under 10 % are dropped as marginal): routed pairs whose gate is below the
threshold are left out and the kept gates renormalised, on every kernel path, against
the oracle's omission."""
import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import synth
from parity_util import check_forward

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TAU = float(np.float32(0.1))  # the descriptor holds an fp32 threshold


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_mixture_experts_amd as qq
    qq.lib()
    return qq


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(q, spec, tau, path=0, layer=None, shared_gate=False):
    layer = synth.make_layer(spec, shared_gate=shared_gate) if layer is None else layer
    x = synth.make_x(spec)
    dl = q.DeviceLayer.from_layer(layer, omit_below=tau)
    y, dbg = q.forward(dl, _dev(x), spec.x_dtype, path=path, debug=True)
    torch.cuda.synchronize()
    return layer, x, y, dbg


@pytest.mark.parametrize("path", [0, 1, 2])
def test_omission_verify_window(q, path):
    """The verify window (Zipf-skewed routing) at 10 %: 57 of 136 routed pairs kept."""
    spec = synth.CONFIGS["c3"]
    layer, x, y, dbg = _run(q, spec, TAU, path=path)
    assert (dbg["ids"].cpu().numpy() == -1).sum() > 0
    (err, tol), nex = check_forward(layer, x, spec.x_dtype, y, dbg, what=f"c3 omit path={path}", omit_below=TAU)
    assert nex == 0


@pytest.mark.parametrize("path", [0, 1, 2])
@pytest.mark.parametrize("T,H,I,E,k,wfmt,shared,xd,tau", [
    (1, 512, 4096, 24, 4, synth.WFMT_MXFP4, 0, synth.X_BF16, 0.2),      # one token, long down rows: o mailbox
    (1, 384, 768, 24, 6, synth.WFMT_MXFP4_PS, 1, synth.X_F32, 0.15),    # packed scales, shared gate
    (4, 256, 1024, 16, 8, synth.WFMT_CB4, 1, synth.X_BF16, 0.12),       # router/route kernel, ticketed combine
    (5, 128, 64, 1024, 16, synth.WFMT_MXFP4, 1, synth.X_BF16, 0.06),    # arrival flags (no mailbox)
    (13, 160, 96, 12, 3, synth.WFMT_MXFP4, 1, synth.X_BF16, 0.3),       # split route
    (40, 256, 128, 16, 4, synth.WFMT_CB4, 1, synth.X_F32, 0.25),        # grouped
    (3, 64, 32, 8, 2, synth.WFMT_CB4, 0, synth.X_F32, 1.0),             # tau = 1: top-1 routing
])
def test_omission_paths(q, T, H, I, E, k, wfmt, shared, xd, tau, path):
    if path == 1 and T > 32:
        pytest.skip("the decode kernels take at most 32 tokens")
    spec = synth.small_spec(f"om{T}_{E}", T, H, I, E, k, wfmt, has_shared=shared, x_dtype=xd, bias="normal",
                            seed=900 + T + E)
    tau32 = float(np.float32(tau))
    layer, x, y, dbg = _run(q, spec, tau32, path=path, shared_gate=bool(shared))
    check_forward(layer, x, spec.x_dtype, y, dbg, what=f"omit T={T} E={E} tau={tau} path={path}",
                  omit_below=tau32)


def test_omission_zero_threshold_is_unchanged(q):
    spec = synth.CONFIGS["c3"]
    layer = synth.make_layer(spec)
    x = _dev(synth.make_x(spec))
    y0 = q.forward(q.DeviceLayer.from_layer(layer), x, spec.x_dtype)
    y1 = q.forward(q.DeviceLayer.from_layer(layer, omit_below=0.0), x, spec.x_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_omission_router_and_bucket_exports(q):
    """moe_router_topk reports omitted pairs as id -1, weight 0; moe_bucket leaves ids -1
    out of the buckets and fills perm past the placed pairs with -1."""
    spec = synth.CONFIGS["c3"]
    layer = synth.make_layer(spec, experts=[])
    x = synth.make_x(spec)
    dl = q.DeviceLayer.from_layer(layer, omit_below=TAU)
    ids, w = q.router_topk(dl, _dev(x), spec.x_dtype)
    x64 = oracle.activations_f64(x, spec.x_dtype)
    ids_ref, g_ref = oracle.omit_marginal(*oracle.topk_softmax(
        oracle.router_logits(x64, layer.router_w, layer.router_b), spec.top_k), TAU)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(w.cpu().numpy() - g_ref).max() <= 1e-6
    counts, offsets, perm = q.bucket(dl, ids)
    c, o, p, _ = oracle.bucket(ids_ref, spec.n_experts, spec.has_shared)
    assert np.array_equal(counts.cpu().numpy(), c) and np.array_equal(offsets.cpu().numpy(), o)
    pg = perm.cpu().numpy()
    assert np.array_equal(pg[:o[-1]], p) and np.all(pg[o[-1]:] == -1)


def test_omission_prefill_chunk_full_size(q):
    """The CB4 prefill chunk (T = 1,024) at 10 %: every token against the oracle."""
    spec = synth.CONFIGS["c5a"]
    layer, x, y, dbg = _run(q, spec, TAU)
    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        ref = oracle.moe_forward(layer, x, spec.x_dtype, map_fn=ex.map, omit_below=TAU)
    (err, tol), nex = check_forward(layer, x, spec.x_dtype, y, dbg, ref=ref, what="c5a omit", omit_below=TAU)
    assert nex == 0
