"""GPU parity: the HIP path (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest

import oracle
import packing
import synth
from parity_util import assert_rescale_exact, check_forward

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

q = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global q
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_mixture_experts_amd as qq
    qq.lib()  # fails loudly when the library is not built
    q = qq


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(spec, layer=None, x=None, path=0):
    layer = synth.make_layer(spec) if layer is None else layer
    x = synth.make_x(spec) if x is None else x
    dl = q.DeviceLayer.from_layer(layer)
    y, dbg = q.forward(dl, _dev(x), spec.x_dtype, path=path, debug=True)
    torch.cuda.synchronize()
    return layer, x, dl, y, dbg


# ---------------------------------------------------------------------------
# dequantisation: bit-exact
# ---------------------------------------------------------------------------
def test_dequant_mxfp4_bit_exact_all_codes_and_scales():
    rows, cols = 256, 96                 # 16 row tiles, 3 blocks per row (a partial step)
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    # row r uses E8M0 = min(r, 252) for its blocks: every finite scale byte appears
    scales = np.repeat(np.minimum(np.arange(rows), 252).astype(np.uint8)[:, None], cols // 32, axis=1)
    buf = packing.pack(packing.MXFP4, codes, scales)
    assert buf.size == q.packed_bytes(q.WFMT_MXFP4, rows, cols)
    out = q.dequant(q.WFMT_MXFP4, _dev(buf), rows, cols).cpu().numpy()
    ref = oracle.dequant(oracle.WFMT_MXFP4, buf, None, rows, cols)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)  # exact in fp32
    assert np.array_equal(out.view(np.uint32), ref.astype(np.float32).view(np.uint32))


def test_dequant_cb4_bit_exact_all_fp16_scales():
    rows, cols = 2048, 32 * 32          # 65,536 blocks: one per fp16 pattern
    cb = synth.make_codebook(77, 0)
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 10) & 31) != 31
    bits = np.where(finite, bits, 0x3C00).astype(np.uint16)
    buf = packing.pack(packing.CB4, codes, bits.reshape(rows, cols // 32))
    out = q.dequant(q.WFMT_CB4, _dev(buf), rows, cols, codebook=_dev(cb)).cpu().numpy()
    ref = oracle.dequant(oracle.WFMT_CB4, buf, cb, rows, cols)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    assert np.array_equal(out.view(np.uint32), ref.astype(np.float32).view(np.uint32))


def test_dequant_cb4_grouped_table_bit_exact():
    """The grouped (prefill) kernels' own CB4 decode (their replicated codebook table and
    lookup) over every fp16 scale pattern and every code, bit for bit against the oracle."""
    rows, cols = 2048, 32 * 32
    cb = synth.make_codebook(78, 0)
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 10) & 31) != 31
    bits = np.where(finite, bits, 0x3C00).astype(np.uint16)
    buf = packing.pack(packing.CB4, codes, bits.reshape(rows, cols // 32))
    out = q.dequant_grouped(q.WFMT_CB4, _dev(buf), rows, cols, codebook=_dev(cb)).cpu().numpy()
    ref = oracle.dequant(oracle.WFMT_CB4, buf, cb, rows, cols)
    assert np.array_equal(out.view(np.uint32), ref.astype(np.float32).view(np.uint32))
    with pytest.raises(q.MoeError):
        q.dequant_grouped(q.WFMT_MXFP4, _dev(buf), rows, cols)


# ---------------------------------------------------------------------------
# routing and bucketing: exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", ["c1", "c2", "c3"])
def test_router_topk_matches_oracle(cfg):
    spec = synth.CONFIGS[cfg]
    layer = synth.make_layer(spec, experts=[])
    x = synth.make_x(spec)
    dl = q.DeviceLayer.from_layer(layer)
    ids, w = q.router_topk(dl, _dev(x), spec.x_dtype)
    torch.cuda.synchronize()
    x64 = oracle.activations_f64(x, spec.x_dtype)
    l = oracle.router_logits(x64, layer.router_w, layer.router_b)
    ids_ref, g_ref = oracle.topk_softmax(l, spec.top_k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(w.cpu().numpy() - g_ref).max() <= 1e-6


def test_router_exact_ties_go_to_lower_index():
    spec = synth.small_spec("tie", 9, 256, 64, 40, 6, synth.WFMT_CB4, bias="none")
    layer = synth.make_layer(spec, experts=[])
    layer.router_w[17] = layer.router_w[3]
    layer.router_w[33] = layer.router_w[3]
    layer.router_w[9] = layer.router_w[30]
    x = synth.make_x(spec)
    dl = q.DeviceLayer.from_layer(layer)
    ids, w = q.router_topk(dl, _dev(x), spec.x_dtype)
    l = oracle.router_logits(oracle.activations_f64(x, spec.x_dtype), layer.router_w, None)
    ids_ref, g_ref = oracle.topk_softmax(l, spec.top_k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)


@pytest.mark.parametrize("T,k,E,shared", [(1, 4, 128, 0), (17, 8, 256, 1), (1024, 8, 256, 1), (1024, 4, 128, 0),
                                          (300, 3, 7, 1), (5, 16, 1024, 0)])
def test_bucket_matches_oracle(T, k, E, shared):
    rng = np.random.default_rng(T + k + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    spec = synth.small_spec("b", T, 64, 32, E, k, synth.WFMT_MXFP4, has_shared=shared)
    layer = synth.make_layer(spec, experts=[])
    dl = q.DeviceLayer.from_layer(layer)
    counts, offsets, perm = q.bucket(dl, _dev(ids))
    c, o, p, _ = oracle.bucket(ids, E, shared)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy(), p)


# ---------------------------------------------------------------------------
# the whole layer
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", ["c1", "c2", "c3"])
def test_forward_decode_configs(cfg):
    spec = synth.CONFIGS[cfg]
    layer, x, dl, y, dbg = _run(spec)
    (err, tol), nex = check_forward(layer, x, spec.x_dtype, y, dbg, what=cfg)
    print(f"{cfg}: max err {err:.3e} tol {tol:.3e} near-ties {nex}")
    assert nex == 0, f"{cfg}: {nex} near-tie tokens on the seeded workload"


SWEEP_T = [1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129]


@pytest.mark.parametrize("path", [0, 1, 2])
@pytest.mark.parametrize("wfmt", [synth.WFMT_MXFP4, synth.WFMT_CB4])
@pytest.mark.parametrize("T", SWEEP_T)
def test_forward_token_sweep(wfmt, T, path):
    """Every tile threshold of the token dimension (16-row MFMA tiles, 4 tiles per pass),
    with a ragged K (H = 160: 5 blocks of 32, not a multiple of 4) for MXFP4.  path 0
    picks the decode kernels up to 10 (MXFP4) or 32 (CB4) tokens; path 1 forces them
    (up to 32 tokens); path 2 forces the grouped kernels."""
    if path == 1 and T > 32:
        pytest.skip("the decode kernels take at most 32 tokens")
    H = 160 if wfmt == synth.WFMT_MXFP4 else 256
    spec = synth.small_spec(f"sweep{T}", T, H, 96, 12, 3, wfmt, has_shared=1, x_dtype=synth.X_BF16,
                            bias="normal", seed=100 + T)
    layer, x, dl, y, dbg = _run(spec, path=path)
    check_forward(layer, x, spec.x_dtype, y, dbg, what=f"T={T} path={path}")


@pytest.mark.parametrize("xd", [synth.X_BF16, synth.X_F32])
@pytest.mark.parametrize("T", [40, 129])
def test_prefill_cb4_ragged_steps(T, xd):
    """The grouped CB4 kernels on K ranges that end in a partial k-step (H = 224: seven
    32-blocks, the last step three; I = 160: five): each row tile's codes of a step arrive
    as one 16-byte load of block 4 s + g, the partial step's missing block clamped to the
    row's last, and the four scales as 2-byte loads."""
    spec = synth.small_spec(f"cb4rag{T}_{xd}", T, 224, 160, 12, 3, synth.WFMT_CB4, has_shared=1, x_dtype=xd,
                            bias="normal", seed=700 + T + xd)
    layer, x, dl, y, dbg = _run(spec, path=2)
    check_forward(layer, x, spec.x_dtype, y, dbg, what=f"CB4 ragged steps T={T} x_dtype={xd}")


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3"])
def test_decode_and_grouped_paths_agree(cfg):
    """Both kernel paths on the same decode-sized inputs, each within tolerance of the oracle."""
    spec = synth.CONFIGS[cfg]
    layer = synth.make_layer(spec)
    x = synth.make_x(spec)
    dl = q.DeviceLayer.from_layer(layer)
    ref = oracle.moe_forward(layer, x, spec.x_dtype)
    for path in (1, 2):
        y, dbg = q.forward(dl, _dev(x), spec.x_dtype, path=path, debug=True)
        torch.cuda.synchronize()
        check_forward(layer, x, spec.x_dtype, y, dbg, ref=ref, what=f"{cfg} path={path}")


def test_decode_path_rejects_large_batches():
    spec = synth.small_spec("big", 40, 64, 32, 4, 2, synth.WFMT_CB4)
    layer = synth.make_layer(spec)
    dl = q.DeviceLayer.from_layer(layer)
    with pytest.raises(q.MoeError) as ei:
        q.forward(dl, _dev(synth.make_x(spec)), spec.x_dtype, path=1)
    assert ei.value.status == q.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("xd", [synth.X_F32, synth.X_BF16])
def test_forward_shared_gate_and_fp32_inputs(xd):
    spec = synth.small_spec("sg", 21, 256, 64, 9, 2, synth.WFMT_CB4, has_shared=1, x_dtype=xd, bias="zipf")
    layer = synth.make_layer(spec, shared_gate=True)
    layer, x, dl, y, dbg = _run(spec, layer=layer)
    check_forward(layer, x, spec.x_dtype, y, dbg, what="shared gate")


@pytest.mark.parametrize("xd", [synth.X_F32, synth.X_BF16])
def test_mxfp4_grouped_activation_planes(xd):
    """The block-scaled MXFP4 grouped path (fp8 activation planes: two for bf16 x, three
    for fp32 x, one E8M0 scale per row; h in three planes per 256-column chunk) with a
    ragged K (H = 160), h chunks padded past I = 96, a shared gate, an all-zero token and
    tokens holding one entry 2^12 times the rest of the row (the row scale then leaves
    the small entries fewer bits)."""
    spec = synth.small_spec("mxplanes", 40, 160, 96, 12, 3, synth.WFMT_MXFP4, has_shared=1, x_dtype=xd,
                            bias="normal", seed=321)
    layer = synth.make_layer(spec, shared_gate=True)
    x = synth.make_x(spec).copy()
    x[0] = 0
    for t, col in ((1, 0), (2, 77), (3, 159)):
        if xd == synth.X_F32:
            x[t, col] *= 4096.0
        else:  # a bf16 value times 2^12: the exponent field plus 12 (exact)
            x[t, col] = np.uint16(int(x[t, col]) + (12 << 7))
    layer, x, dl, y, dbg = _run(spec, layer=layer, x=x, path=2)
    check_forward(layer, x, spec.x_dtype, y, dbg, what=f"mxfp4 planes xd={xd}")


@pytest.mark.parametrize("H,I,k,shared,wfmt,xd", [
    (512, 4096, 4, 0, synth.WFMT_MXFP4, synth.X_BF16),   # K = I over several k-step chunks per wave
    (384, 768, 2, 1, synth.WFMT_MXFP4, synth.X_F32),     # 3 slots, fp32 x planes, ragged last k-step group
    (256, 1024, 4, 1, synth.WFMT_CB4, synth.X_F32),      # codebook weights, shared gate
    (256, 1024, 8, 1, synth.WFMT_CB4, synth.X_BF16),     # 9 slots
    (4096, 640, 12, 0, synth.WFMT_MXFP4, synth.X_BF16),  # I = 640 (5 k-steps): the short-row kernel and its
                                                         # ticketed combine, 64 x 12 blocks
])
def test_one_token_long_rows(H, I, k, shared, wfmt, xd):
    """One token: the split-K down kernel with its mailbox combine over several slot counts,
    both weight formats and both activation types (and one case of the short-row kernel)."""
    spec = synth.small_spec(f"t1_{H}_{I}_{k}", 1, H, I, 24, k, wfmt, has_shared=shared, x_dtype=xd,
                            bias="normal", seed=7 * I + k)
    layer = synth.make_layer(spec, shared_gate=bool(shared))
    layer, x, dl, y, dbg = _run(spec, layer=layer)
    check_forward(layer, x, spec.x_dtype, y, dbg, what=f"one token H={H} I={I} k={k}")


@pytest.mark.parametrize("path", [0, 2])
@pytest.mark.parametrize("T,H,I,E,k,wfmt,shared,xd", [
    (5, 128, 64, 1024, 16, synth.WFMT_MXFP4, 1, synth.X_BF16),   # most experts, largest top-k
    (1, 128, 64, 1024, 16, synth.WFMT_MXFP4, 1, synth.X_BF16),   # the logit mailbox with 16 candidates a lane
    (2, 128, 64, 300, 8, synth.WFMT_CB4, 0, synth.X_F32),        # the mailbox with 5 candidates a lane
    (40, 128, 64, 1024, 16, synth.WFMT_CB4, 1, synth.X_F32),
    (3, 16384, 64, 4, 2, synth.WFMT_CB4, 0, synth.X_BF16),       # largest H: 128 k-steps of gate/up
    (3, 64, 16384, 4, 2, synth.WFMT_MXFP4, 1, synth.X_F32),      # largest I: 128 k-steps of down
    (64, 16384, 64, 4, 2, synth.WFMT_MXFP4, 1, synth.X_BF16),
    (64, 64, 16384, 4, 2, synth.WFMT_MXFP4, 0, synth.X_F32),     # 64 h scale chunks, the LDS table's size
    (64, 64, 16384, 4, 2, synth.WFMT_CB4, 1, synth.X_BF16),
])
def test_forward_at_size_limits(T, H, I, E, k, wfmt, shared, xd, path):
    """The library's largest supported experts count, top-k, hidden and intermediate
    sizes, on the automatic path (decode kernels up to 32 tokens) and the grouped one."""
    spec = synth.small_spec(f"lim{T}_{H}_{I}_{E}", T, H, I, E, k, wfmt, has_shared=shared, x_dtype=xd,
                            bias="normal", seed=T + H + I + E)
    layer = synth.make_layer(spec, shared_gate=bool(shared))
    layer, x, dl, y, dbg = _run(spec, layer=layer, path=path)
    check_forward(layer, x, spec.x_dtype, y, dbg, what=f"limits T={T} H={H} I={I} E={E} k={k} path={path}")


@pytest.mark.parametrize("wfmt", [synth.WFMT_MXFP4, synth.WFMT_CB4])
@pytest.mark.parametrize("T", [2, 4, 20])
def test_decode_down_two_tiles(wfmt, T):
    """The split-K down projection from 2 tokens covers two 16-row tiles per block (one
    ticket per 32 columns): H = 224 gives 7 such blocks per expert.  I = 1152 is 9 k-steps,
    past the short-row kernel."""
    spec = synth.small_spec(f"dn2_{T}", T, 224, 1152, 16, 4, wfmt, has_shared=1, x_dtype=synth.X_BF16,
                            bias="normal", seed=300 + T)
    layer = synth.make_layer(spec)
    layer, x, dl, y, dbg = _run(spec, layer=layer, path=1)
    check_forward(layer, x, spec.x_dtype, y, dbg, what=f"two-tile down T={T} wfmt={wfmt}")


@pytest.mark.parametrize("case,wfmt,T,H,I,E,k", [
    ("same", synth.WFMT_CB4, 32, 2048, 512, 64, 4),        # 32 pairs per expert, 7 rows a pass: 5 passes each
    ("same_wide", synth.WFMT_CB4, 32, 256, 256, 64, 4),    # one 32-row pass: rows past the record's 24 from perm
    ("same", synth.WFMT_MXFP4, 24, 2880, 256, 32, 4),      # 24 pairs per expert, 7 rows a pass: 4 passes each
    ("distinct", synth.WFMT_MXFP4, 32, 512, 256, 1024, 8),  # nearly every pair its own expert: the item bound
])
def test_decode_work_items_at_the_bounds(case, wfmt, T, H, I, E, k):
    """The decode gate/up grid has one row per work item (one staging pass of one active
    expert) up to a bound over every routing.  "same": a router bias of +50 sends every
    token to experts 0..k-1, so each takes T pairs in several passes (and the shared expert
    as many); "distinct": 256 pairs over 1,024 experts with no bias, so most pairs have an
    expert of their own and the item count approaches its bound."""
    spec = synth.small_spec(f"items_{case}_{T}_{H}", T, H, I, E, k, wfmt, has_shared=1, x_dtype=synth.X_BF16,
                            bias="none" if case == "distinct" else "normal", seed=500 + T + H)
    layer = synth.make_layer(spec)
    if case.startswith("same"):
        rb = np.zeros(E, dtype=np.float32)
        rb[:k] = 50.0 + np.arange(k, dtype=np.float32)
        layer.router_b = rb
    layer, x, dl, y, dbg = _run(spec, layer=layer, path=1)
    ids = dbg["ids"].cpu().numpy().reshape(T, k)
    if case.startswith("same"):
        assert (np.sort(ids, axis=1) == np.arange(k)).all()
    else:
        assert len(np.unique(ids)) > 0.7 * T * k
    check_forward(layer, x, spec.x_dtype, y, dbg, what=f"work items {case} T={T} H={H} wfmt={wfmt}")


@pytest.mark.parametrize("wfmt", [synth.WFMT_MXFP4, synth.WFMT_CB4])
@pytest.mark.parametrize("T,path,H", [(1, 0, 512), (4, 0, 512), (7, 0, 512), (9, 0, 512), (40, 0, 512), (4, 2, 512),
                                      (1, 0, 6144), (4, 0, 6144)])
def test_forward_rms_equals_rescale_then_forward(wfmt, T, path, H):
    """moe_forward_rms (the rescale folded into the router kernel below 8 decode tokens,
    the rescale kernel first otherwise) gives the bits of moe_rms_rescale followed by
    moe_forward on the same path, and with the residual add y_prev plus those bits; the
    two-step result is checked against the oracle.  H = 6144 takes the folded rescale's
    form for rows longer than a thread's registers hold (16 values of 256 threads)."""
    spec = synth.small_spec(f"rms{T}_{H}", T, H, 1024, 16, 4, wfmt, has_shared=1, x_dtype=synth.X_BF16,
                            bias="normal", seed=40 + T)
    layer = synth.make_layer(spec, shared_gate=True)
    dl = q.DeviceLayer.from_layer(layer)
    rng = np.random.default_rng(900 + T)
    y_prev = _dev((rng.standard_normal((T, H)) * rng.uniform(0.1, 20.0, (T, 1))).astype(np.float32))
    x = q.rms_rescale(y_prev)
    y2, dbg = q.forward(dl, x, synth.X_BF16, path=path, debug=True)
    y1 = q.forward_rms(dl, y_prev, 1e-6, path=path)
    y3 = q.forward_rms(dl, y_prev, 1e-6, path=path, residual=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y3, y_prev + y1)  # the residual add follows the finished combine, in fp32
    xb = x.cpu().numpy().view(np.uint16)
    check_forward(layer, xb, synth.X_BF16, y2, dbg, what=f"rms T={T} path={path}")


def test_forward_deterministic_and_batch_invariant():
    spec = synth.CONFIGS["c3"]
    layer, x, dl, y, dbg = _run(spec)
    y2 = q.forward(dl, _dev(x), spec.x_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    # token 5 alone gives the same bits as inside the batch
    y1 = q.forward(dl, _dev(x[5:6]), spec.x_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y1[0], y[5])


@pytest.mark.parametrize("cfg", ["c2", "c3"])
def test_graph_replay_matches_eager(cfg):
    """The forward captured in a HIP graph: every replay, with eager work and syncs in
    between, gives the eager result bit for bit."""
    spec = synth.CONFIGS[cfg]
    layer, x, dl, y_eager, _ = _run(spec)
    xt = _dev(x)
    ws = dl.workspace(spec.T)
    y = torch.empty_like(y_eager)
    q.forward(dl, xt, spec.x_dtype, y=y, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.forward(dl, xt, spec.x_dtype, y=y, ws=ws)
    for r in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r}"
        # eager work on the same workspace between replays
        q.forward(dl, xt, spec.x_dtype, y=torch.empty_like(y), ws=ws)
        torch.cuda.synchronize()


def test_forward_zero_tokens_is_noop():
    spec = synth.CONFIGS["c1"]
    layer = synth.make_layer(spec)
    dl = q.DeviceLayer.from_layer(layer)
    x = torch.empty((0, spec.hidden), dtype=torch.float32, device="cuda")
    y = q.forward(dl, x, spec.x_dtype)
    assert y.shape == (0, spec.hidden)


@pytest.mark.parametrize("cfg,T", [("c5a", None), ("c5b", None), ("c3", 136)])
def test_forward_prefill_full_size(cfg, T):
    """Full shapes on the grouped path, every token compared with the oracle: the two
    prefill chunks (T = 1024) and the batched verify round (the verify layer with 8
    requests x 17 tokens, T = 136).  The oracle's expert products run on a thread pool
    (the same values as one after another)."""
    import dataclasses
    import os
    from concurrent.futures import ThreadPoolExecutor
    spec = synth.CONFIGS[cfg] if T is None else dataclasses.replace(synth.CONFIGS[cfg], T=T)
    layer, x, dl, y, dbg = _run(spec)
    del dl
    nthr = min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(nthr) as ex:
        ref = oracle.moe_forward(layer, x, spec.x_dtype, map_fn=ex.map)
    (err, tol), nex = check_forward(layer, x, spec.x_dtype, y, dbg, ref=ref, what=cfg)
    print(f"{cfg} T={spec.T}: max err {err:.3e} tol {tol:.3e} near-ties {nex}")
    assert nex == 0, f"{cfg}: {nex} near-tie tokens on the seeded workload"


@pytest.mark.parametrize("T,H", [(4, 2880), (3, 2048), (1, 160), (5, 4096), (2, 6000)])
def test_rms_rescale_bit_exact(T, H):
    """The rescale kernel's bf16 output equals the oracle's rounding of the fp64 quotient
    y / sqrt(mean(y^2) + eps), bit for bit, over rows of very different scales (rows of up
    to 4,096 columns kept in registers, longer ones read twice)."""
    rng = np.random.default_rng(4 + T + H)
    y = (rng.standard_normal((T, H)) * np.exp(rng.uniform(-20, 20, (T, 1)))).astype(np.float32)
    out = q.rms_rescale(_dev(y), eps=oracle.RMS_EPS).cpu().numpy()
    near = assert_rescale_exact(out, y, what=f"rescale T={T} H={H}")
    print(f"rescale T={T} H={H}: bit-exact, {near} values near a rounding midpoint")


# ---------------------------------------------------------------------------
# 36 stacked gpt-oss-shaped layers (every expert of every layer resident, ~61 GB)
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def stacked_layers():
    spec = synth.CONFIGS["c4"]
    layers = [q.DeviceLayer.from_layer(synth.make_layer(spec, layer=l)) for l in range(spec.n_layers)]
    yield spec, layers
    del layers
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 4])
def test_stacked_layers_teacher_forced(stacked_layers, T):
    """Each layer's y, RMS-rescaled on the GPU, is the next layer's x.  Layers (every one
    at one token, every third at four) are compared with the oracle fed the GPU's own
    input to that layer (a near-tie at one layer cannot then compound), and every
    rescale is compared with the oracle's bit for bit."""
    spec, layers = stacked_layers
    ws = layers[0].workspace(T)
    xs = [_dev(synth.make_x(spec, T=T, layer=0))]
    ys, dbgs = [], []
    for l in range(spec.n_layers):
        y, dbg = q.forward(layers[l], xs[l], spec.x_dtype, ws=ws, debug=True)
        ys.append(y)
        dbgs.append(dbg)
        if l + 1 < spec.n_layers:
            xs.append(q.rms_rescale(y))
    torch.cuda.synchronize()
    for l in range(spec.n_layers - 1):
        assert_rescale_exact(xs[l + 1].cpu().numpy(), ys[l].cpu().numpy(), what=f"rescale after layer {l}")
    import os
    from concurrent.futures import ThreadPoolExecutor
    check = range(spec.n_layers) if T == 1 else range(0, spec.n_layers, 3)
    pool = ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0))))
    for l in check:
        x_l = xs[l].cpu().numpy().view(np.uint16)
        router = synth.make_layer(spec, layer=l, experts=[])
        ids_ref, _ = oracle.topk_softmax(
            oracle.router_logits(oracle.activations_f64(x_l, spec.x_dtype), router.router_w, router.router_b),
            spec.top_k)
        used = np.union1d(ids_ref.ravel(), dbgs[l]["ids"].cpu().numpy().ravel())
        host = synth.make_layer(spec, layer=l, experts=used)
        ref = oracle.moe_forward(host, x_l, spec.x_dtype, map_fn=pool.map)
        (err, tol), nex = check_forward(host, x_l, spec.x_dtype, ys[l], dbgs[l], ref=ref,
                                        what=f"stacked layer {l}, T={T}")
        assert nex == 0, f"stacked layer {l}: {nex} near-tie tokens"
