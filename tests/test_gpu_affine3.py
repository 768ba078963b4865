"""GPU parity of the 3-bit affine group-64 format (one fp16 scale and bias per 64 values:
"Running Qwen3.8-Flash-Next on a 32 GB Mac with Transformers", "Where every weight
lives"): dequantisation against the oracle's exact values, and the layer (decode kernels,
chunks of 32 tokens above that) against the oracle."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import packing
import synth
from parity_util import assert_y_close, check_forward

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_mixture_experts_amd as qq
    qq.lib()
    return qq


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("rows,cols", [(16, 128), (64, 2560), (48, 640)])
def test_dequant_affine3(q, rows, cols):
    """fp32 out = the fp32 rounding of the exact s q + b, over scales and biases of both
    signs and many magnitudes (subnormal and largest fp16 included)."""
    rng = np.random.default_rng(rows + cols)
    qq = rng.integers(0, 8, (rows, cols), dtype=np.uint8)
    s = (rng.uniform(-2, 2, (rows, cols // 64)) * np.exp2(rng.integers(-20, 12, (rows, cols // 64)))).astype(np.float16)
    b = (rng.uniform(-2, 2, (rows, cols // 64)) * np.exp2(rng.integers(-20, 12, (rows, cols // 64)))).astype(np.float16)
    s[0, 0], b[0, 0] = np.float16(6.0e-8), np.float16(-65504.0)
    buf = packing.pack_affine3(qq, s.view(np.uint16), b.view(np.uint16))
    assert buf.size == q.packed_bytes(q.WFMT_AFF3, rows, cols)
    out = q.dequant(q.WFMT_AFF3, _dev(buf), rows, cols).cpu().numpy()
    ref = oracle.dequant(oracle.WFMT_AFF3, buf, None, rows, cols)
    assert np.array_equal(out.view(np.uint32), ref.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("T,H,I,E,k,shared,xd", [
    (1, 256, 1024, 16, 4, 0, synth.X_BF16),    # one token, long down rows: split-K down, o mailbox
    (1, 384, 128, 12, 3, 1, synth.X_F32),      # one token, short down rows, fp32 x planes, shared gate
    (4, 256, 512, 24, 6, 1, synth.X_BF16),     # router/route kernel
    (9, 128, 256, 40, 8, 1, synth.X_BF16),     # split route
    (17, 512, 256, 32, 8, 1, synth.X_F32),     # two token tiles
    (32, 128, 128, 8, 2, 0, synth.X_BF16),     # the decode kernels' largest batch
])
def test_affine3_decode_forward(q, T, H, I, E, k, shared, xd):
    spec = synth.small_spec(f"a3_{T}_{H}_{I}", T, H, I, E, k, synth.WFMT_AFF3, has_shared=shared, x_dtype=xd,
                            bias="normal", seed=700 + T + H)
    layer = synth.make_layer(spec, shared_gate=bool(shared))
    x = synth.make_x(spec)
    dl = q.DeviceLayer.from_layer(layer)
    y, dbg = q.forward(dl, _dev(x), xd, debug=True)
    torch.cuda.synchronize()
    check_forward(layer, x, xd, y, dbg, what=f"affine3 T={T} H={H} I={I}")


@pytest.mark.parametrize("T", [40, 70])
def test_affine3_chunked_batches(q, T):
    """More than 32 tokens: the decode kernels on chunks of 32; y for every token against
    the oracle, the ids through the router export; the grouped path and the bucketing
    outputs of such a call are refused."""
    spec = synth.small_spec(f"a3c{T}", T, 256, 256, 16, 4, synth.WFMT_AFF3, has_shared=1, bias="normal", seed=T)
    layer = synth.make_layer(spec, shared_gate=True)
    x = synth.make_x(spec)
    dl = q.DeviceLayer.from_layer(layer)
    y = q.forward(dl, _dev(x), spec.x_dtype)
    ids, _ = q.router_topk(dl, _dev(x), spec.x_dtype)
    torch.cuda.synchronize()
    ref = oracle.moe_forward(layer, x, spec.x_dtype)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_y_close(y.cpu().numpy(), ref["y"], what=f"affine3 chunked T={T}")
    for kw in (dict(path=q.PATH_PREFILL), dict(debug=True)):
        with pytest.raises(q.MoeError) as ei:
            q.forward(dl, _dev(x), spec.x_dtype, **kw)
        assert ei.value.status == q.MOE_ERR_UNSUPPORTED
    # the rescaled-input entry point on chunks: the bits of the rescale, then the forward
    y_prev = _dev(np.random.default_rng(T).standard_normal((T, spec.hidden)).astype(np.float32))
    y1 = q.forward_rms(dl, y_prev, 1e-6)
    y2 = q.forward(dl, q.rms_rescale(y_prev), synth.X_BF16)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_affine3_page_layer_verify_window(q):
    """The Mac page's layer (hidden 2,560, 512 routed experts of which 10 are kept, intermediate 640,
    a shared expert) with its 3-bit experts at the 17-token verify window, in full."""
    spec = synth.CONFIGS["aff3"]
    layer = synth.make_layer(spec)
    x = synth.make_x(spec)
    dl = q.DeviceLayer.from_layer(layer)
    y, dbg = q.forward(dl, _dev(x), spec.x_dtype, debug=True)
    torch.cuda.synchronize()
    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        ref = oracle.moe_forward(layer, x, spec.x_dtype, map_fn=ex.map)
    (err, tol), nex = check_forward(layer, x, spec.x_dtype, y, dbg, ref=ref, what="aff3")
    assert nex == 0
