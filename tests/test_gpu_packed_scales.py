"""GPU parity of the MXFP4 packed scale store (one base E8M0 byte per row plus a 4-bit
delta per block): decoding is bit-exact against the oracle, and the layer gives the same
y bits as the raw MXFP4 store of the same codes and scales on every kernel path ("How
Neural runs a 120-billion-parameter model on one gaming PC", section "Correctness": only
the scales change encoding in the packed store, and the outputs match bit for bit)."""
import dataclasses

import numpy as np
import pytest

import oracle
import packing
import synth
from parity_util import check_forward

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


@pytest.mark.parametrize("rows,cols", [(256, 96), (64, 2880), (48, 160)])
def test_dequant_packed_scales_bit_exact(q, rows, cols):
    rng = np.random.default_rng(rows + cols)
    codes = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    base = np.minimum(np.arange(rows), 237)[:, None]           # bases 0 .. 237: E8M0 up to 252
    e8 = (base + rng.integers(0, 16, (rows, cols // 32))).astype(np.uint8)
    buf = packing.pack_scale_store(codes, e8)
    assert buf.size == q.packed_bytes(q.WFMT_MXFP4_PS, rows, cols)
    out = q.dequant(q.WFMT_MXFP4_PS, _dev(buf), rows, cols).cpu().numpy()
    ref = oracle.dequant(oracle.WFMT_MXFP4_PS, buf, None, rows, cols)
    assert np.array_equal(out.view(np.uint32), ref.astype(np.float32).view(np.uint32))


def _pair(spec, shared_gate=False):
    raw = synth.make_layer(spec, shared_gate=shared_gate)
    ps = synth.make_layer(synth.with_packed_scales(spec), shared_gate=shared_gate)
    return raw, ps


@pytest.mark.parametrize("path", [0, 1, 2])
@pytest.mark.parametrize("T,xd", [(1, synth.X_BF16), (4, synth.X_F32), (9, synth.X_BF16), (17, synth.X_BF16),
                                  (40, synth.X_F32), (129, synth.X_BF16)])
def test_packed_scales_same_bits_as_raw(q, T, xd, path):
    """Ragged K (H = 160, I = 96: partial last k-steps), a shared expert with a gate."""
    if path == 1 and T > 32:
        pytest.skip("the decode kernels take at most 32 tokens")
    spec = synth.small_spec(f"ps{T}", T, 160, 96, 12, 3, synth.WFMT_MXFP4, has_shared=1, x_dtype=xd,
                            bias="normal", seed=500 + T)
    raw, ps = _pair(spec, shared_gate=True)
    x = _dev(synth.make_x(spec))
    y_raw = q.forward(q.DeviceLayer.from_layer(raw), x, xd, path=path)
    y_ps, dbg = q.forward(q.DeviceLayer.from_layer(ps), x, xd, path=path, debug=True)
    torch.cuda.synchronize()
    assert torch.equal(y_ps, y_raw)
    check_forward(ps, synth.make_x(spec), xd, y_ps, dbg, what=f"packed scales T={T} path={path}")


@pytest.mark.parametrize("cfg,T", [("c2", 1), ("c2", 4), ("c5b", 1024)])
def test_packed_scales_full_size_same_bits_as_raw(q, cfg, T):
    """The gpt-oss-shaped layer at decode (one and four tokens) and the 1,024-token prefill
    chunk: y from the packed scale store equals y from the raw store bit for bit (the raw
    store's y is checked against the oracle by the other parity tests)."""
    spec = dataclasses.replace(synth.CONFIGS[cfg], T=T)
    raw, ps = _pair(spec)
    x = _dev(synth.make_x(spec))
    dl = q.DeviceLayer.from_layer(raw)
    y_raw = q.forward(dl, x, spec.x_dtype)
    del dl
    dl = q.DeviceLayer.from_layer(ps)
    y_ps = q.forward(dl, x, spec.x_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y_ps, y_raw)
