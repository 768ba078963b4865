"""moe_forward_noalloc (the workspace from the library's per-device scratch array) against
moe_forward with a caller workspace, through the C ABI: the same kernels, so the same y
bits, on two calls in a row, the second with a smaller input; the second call is also
checked against the oracle."""
import pytest

import synth
from parity_util import check_forward

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_mixture_experts_amd as qq
    qq.lib()  # fails loudly when the library is not built
    return qq


def _spec(name):
    if name in synth.CONFIGS:
        return synth.CONFIGS[name]
    if name == "small_mx":
        return synth.small_spec("na_mx", 40, 160, 96, 12, 3, synth.WFMT_MXFP4, has_shared=1, bias="normal", seed=61)
    return synth.small_spec("na_cb", 24, 256, 128, 16, 4, synth.WFMT_CB4, has_shared=1, x_dtype=synth.X_F32,
                            bias="zipf", seed=62)


@pytest.mark.parametrize("cfg,T1,T2,path", [
    ("c2", 1, 1, 0),          # one token: router/route kernel, one-token mailbox combine
    ("c3", 17, 5, 0),         # verify window, then a smaller batch on the same scratch
    ("small_mx", 40, 9, 0),   # grouped path, then the decode path
    ("small_cb", 24, 3, 2),   # grouped path forced, fp32 x, codebook weights
])
def test_noalloc_matches_forward(q, cfg, T1, T2, path):
    spec = _spec(cfg)
    layer = synth.make_layer(spec, shared_gate=bool(spec.has_shared))
    dl = q.DeviceLayer.from_layer(layer)
    for call, T in enumerate((T1, T2)):
        x = synth.make_x(spec, T=T, stream=call)
        xt = torch.from_numpy(x).cuda()
        y_ref, dbg = q.forward(dl, xt, spec.x_dtype, path=path, debug=True)
        y_na = q.forward_noalloc(dl, xt, spec.x_dtype, path=path)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ref), f"{cfg} call {call} (T={T}): y differs from moe_forward"
    (err, tol), _ = check_forward(layer, x, spec.x_dtype, y_na, dbg, what=f"{cfg} no-alloc T={T2}")
    print(f"{cfg}: T={T1} then T={T2} bit-identical to moe_forward; max err {err:.3e} (tol {tol:.3e})")


def test_noalloc_rejects_workspace_beyond_scratch(q):
    """A call whose workspace exceeds the scratch array is refused before anything runs."""
    spec = synth.small_spec("na_big", 2048, 1024, 256, 8, 4, synth.WFMT_MXFP4)
    dl = q.DeviceLayer.from_layer(synth.make_layer(spec))
    assert dl.workspace_bytes(spec.T) > 32 << 20
    x = torch.zeros((spec.T, spec.hidden), dtype=torch.int16, device="cuda")
    with pytest.raises(q.MoeError) as ei:
        q.forward_noalloc(dl, x, spec.x_dtype)
    assert ei.value.status == q.MOE_ERR_WORKSPACE
