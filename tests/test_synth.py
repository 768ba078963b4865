"""The seeded generator: reproducible, and drawing from the stated distributions."""
import numpy as np

import synth


def test_reproducible_and_seed_sensitive():
    spec = synth.small_spec("s", 3, 64, 32, 4, 2, synth.WFMT_CB4, has_shared=1, bias="zipf")
    a, b = synth.make_layer(spec), synth.make_layer(spec)
    for e in range(5):
        assert np.array_equal(a.gate_up[e], b.gate_up[e]) and np.array_equal(a.down[e], b.down[e])
    assert np.array_equal(a.router_w, b.router_w) and np.array_equal(a.codebook, b.codebook)
    spec2 = synth.small_spec("s", 3, 64, 32, 4, 2, synth.WFMT_CB4, has_shared=1, bias="zipf", seed=8)
    c = synth.make_layer(spec2)
    assert not np.array_equal(a.gate_up[0], c.gate_up[0])
    # a subset of experts regenerates the same bytes
    d = synth.make_layer(spec, experts=[2])
    assert d.gate_up[0] is None and np.array_equal(d.gate_up[2], a.gate_up[2])
    assert np.array_equal(d.gate_up[4], a.gate_up[4])  # shared expert always present


def test_distributions():
    spec = synth.small_spec("d", 3, 256, 128, 4, 2, synth.WFMT_MXFP4)
    L = synth.make_layer(spec)
    buf = L.gate_up[0]
    off = synth.scale_plane_offset(256, 256)
    u = buf[off:off + 256 * 256 // 32]
    assert u.min() == 118 and u.max() == 124
    codes = buf[:256 * 128]
    nib = np.concatenate([codes & 15, codes >> 4])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.8 * nib.size / 16
    spec = synth.small_spec("d", 3, 256, 128, 4, 2, synth.WFMT_CB4)
    L = synth.make_layer(spec)
    s = L.down[1][synth.scale_plane_offset(256, 128):].view(np.float16).astype(np.float64)
    assert s.min() >= 0.0099 and s.max() <= 0.0501
    cb = L.codebook
    assert cb.dtype == np.int8 and len(set(cb.tolist())) == 16 and np.all(np.diff(cb.astype(int)) > 0)


def test_zipf_prior_is_a_log_distribution():
    b = synth.zipf_log_prior(1003, 0, 256, 1.1)
    p = np.exp(b.astype(np.float64))
    assert abs(p.sum() - 1) < 1e-5
    srt = np.sort(p)[::-1]
    assert abs(srt[0] / srt[1] - 2 ** 1.1) < 1e-4


def test_bf16_inputs_are_rne_of_normals():
    spec = synth.CONFIGS["c2"]
    x = synth.make_x(spec)
    assert x.dtype == np.uint16 and x.shape == (1, 2880)


def test_small_spec_keeps_the_format():
    for wfmt in (synth.WFMT_MXFP4, synth.WFMT_CB4, synth.WFMT_MXFP4_PS, synth.WFMT_AFF3):
        spec = synth.small_spec("f", 2, 128, 128, 4, 2, wfmt)
        layer = synth.make_layer(spec)
        assert layer.wfmt == wfmt
        assert layer.gate_up[0].size == synth.packed_nbytes(wfmt, 256, 128)
