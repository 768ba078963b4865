"""The C ABI on the host (no GPU): the library loads, exports every symbol the header
declares, and its validation rejects bad arguments before anything is enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest

import quantized_mixture_experts_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moeq.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(q.LIB_PATH):
        from quantized_mixture_experts_amd import build
        build.build()
    return q.lib()


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(q.EXPORTED)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_packed_bytes(L):
    assert q.packed_bytes(q.WFMT_MXFP4, 5760, 2880) + q.packed_bytes(q.WFMT_MXFP4, 2880, 2880) == 13_219_200
    assert q.packed_bytes(q.WFMT_CB4, 16, 160) == 1440
    assert q.packed_bytes(q.WFMT_CB4, 16, 100) == 0
    assert q.packed_bytes(99, 16, 64) == 0
    assert q.packed_bytes(q.WFMT_MXFP4, 0, 64) == 0
    assert q.packed_bytes(q.WFMT_MXFP4, 8, 64) == 0   # rows come in tiles of 16


FAKE = 0x10000  # a non-null, 256-aligned stand-in for device pointers (never dereferenced)


def layer(**kw):
    d = dict(hidden=256, inter=128, n_experts=8, top_k=2, wfmt=q.WFMT_CB4, has_shared=0,
             router_w=FAKE, router_b=None, gate_up=FAKE, down=FAKE, codebook=FAKE, shared_gate_w=None,
             omit_below=0.0)
    d.update(kw)
    return q.MoeLayerC(*[d[f] for f, _ in q.MoeLayerC._fields_])


def ws_bytes(L, lay, T):
    return L.moe_workspace_bytes(ctypes.byref(lay), T)


@pytest.mark.parametrize("bad,status", [
    (dict(hidden=100), q.MOE_ERR_INVALID_ARG), (dict(inter=0), q.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), q.MOE_ERR_UNSUPPORTED), (dict(top_k=0), q.MOE_ERR_INVALID_ARG),
    (dict(n_experts=2000, top_k=2), q.MOE_ERR_UNSUPPORTED), (dict(wfmt=7), q.MOE_ERR_INVALID_ARG),
    (dict(codebook=None), q.MOE_ERR_INVALID_ARG), (dict(wfmt=q.WFMT_MXFP4), q.MOE_ERR_INVALID_ARG),
    (dict(omit_below=-0.1), q.MOE_ERR_INVALID_ARG), (dict(omit_below=1.5), q.MOE_ERR_INVALID_ARG),
    (dict(omit_below=float("nan")), q.MOE_ERR_INVALID_ARG),
    (dict(router_w=None), q.MOE_ERR_INVALID_ARG), (dict(gate_up=None), q.MOE_ERR_INVALID_ARG),
    (dict(router_w=FAKE + 4), q.MOE_ERR_ALIGNMENT), (dict(has_shared=2), q.MOE_ERR_INVALID_ARG),
    (dict(hidden=32768), q.MOE_ERR_UNSUPPORTED),
])
def test_forward_rejects_bad_layers(L, bad, status):
    lay = layer(**bad)
    assert ws_bytes(L, lay, 4) == 0
    r = L.moe_forward(ctypes.byref(lay), FAKE, q.DT_F32, 4, FAKE, FAKE, 1 << 30, None, 0,
                      None, None, None, None, None)
    assert r == status


def test_forward_rejects_bad_calls(L):
    lay = layer()
    need = ws_bytes(L, lay, 4)
    assert need > 0
    f = lambda x=FAKE, dt=q.DT_F32, T=4, y=FAKE, ws=FAKE, n=need, path=0, ids=None: L.moe_forward(
        ctypes.byref(lay), x, dt, T, y, ws, n, None, path, ids, None, None, None, None)
    assert f(x=None) == q.MOE_ERR_INVALID_ARG
    assert f(y=None) == q.MOE_ERR_INVALID_ARG
    assert f(dt=5) == q.MOE_ERR_INVALID_ARG
    assert f(dt=2) == q.MOE_ERR_INVALID_ARG  # the rescaled-input mode only through moe_forward_rms
    assert f(T=-1) == q.MOE_ERR_INVALID_ARG
    assert f(T=1 << 20) == q.MOE_ERR_UNSUPPORTED
    assert f(path=9) == q.MOE_ERR_INVALID_ARG
    assert f(x=FAKE + 8) == q.MOE_ERR_ALIGNMENT
    assert f(ids=FAKE + 2) == q.MOE_ERR_ALIGNMENT
    assert f(ws=None) == q.MOE_ERR_WORKSPACE
    assert f(n=need - 1) == q.MOE_ERR_WORKSPACE
    assert f(ws=FAKE + 16) == q.MOE_ERR_ALIGNMENT
    assert f(T=0) == q.MOE_OK     # nothing is enqueued for zero tokens


def test_forward_rms_rejects_bad_calls(L):
    lay = layer()
    need = ws_bytes(L, lay, 4)
    Y = FAKE + 256
    f = lambda yp=FAKE, eps=1e-6, res=0, T=4, y=Y, ws=FAKE, n=need, path=0: L.moe_forward_rms(
        ctypes.byref(lay), yp, eps, res, T, y, ws, n, None, path, None)
    assert f(eps=-1.0) == q.MOE_ERR_INVALID_ARG
    assert f(res=2) == q.MOE_ERR_INVALID_ARG
    assert f(eps=float("nan")) == q.MOE_ERR_INVALID_ARG
    assert f(y=FAKE) == q.MOE_ERR_INVALID_ARG          # y_prev may not be y
    assert f(yp=None) == q.MOE_ERR_INVALID_ARG
    assert f(yp=FAKE + 8) == q.MOE_ERR_ALIGNMENT
    assert f(path=9) == q.MOE_ERR_INVALID_ARG
    assert f(n=need - 1) == q.MOE_ERR_WORKSPACE
    assert f(T=0) == q.MOE_OK


def test_router_and_bucket_validation(L):
    lay = layer()
    need = ws_bytes(L, lay, 3)
    assert L.moe_router_topk(ctypes.byref(lay), FAKE, q.DT_BF16, 3, None, FAKE, FAKE, need, None) == q.MOE_ERR_INVALID_ARG
    assert L.moe_router_topk(ctypes.byref(lay), FAKE, q.DT_BF16, 3, FAKE, FAKE, FAKE, 8, None) == q.MOE_ERR_WORKSPACE
    assert L.moe_router_topk(ctypes.byref(lay), FAKE, q.DT_BF16, 0, FAKE, FAKE, FAKE, need, None) == q.MOE_OK
    assert L.moe_bucket(ctypes.byref(lay), FAKE, 3, FAKE, None, FAKE, FAKE, need, None) == q.MOE_ERR_INVALID_ARG
    assert L.moe_bucket(ctypes.byref(lay), FAKE + 1, 3, FAKE, FAKE, FAKE, FAKE, need, None) == q.MOE_ERR_ALIGNMENT
    assert L.moe_bucket(ctypes.byref(lay), FAKE, 0, FAKE, FAKE, FAKE, FAKE, need, None) == q.MOE_OK


def test_dequant_and_rescale_validation(L):
    assert L.moe_dequant(q.WFMT_CB4, FAKE, None, 16, 64, FAKE, None) == q.MOE_ERR_INVALID_ARG
    assert L.moe_dequant(q.WFMT_MXFP4, FAKE, None, 16, 48, FAKE, None) == q.MOE_ERR_INVALID_ARG
    assert L.moe_dequant(q.WFMT_MXFP4, FAKE, None, 4, 64, FAKE, None) == q.MOE_ERR_INVALID_ARG
    assert L.moe_dequant(q.WFMT_MXFP4, FAKE + 4, None, 16, 64, FAKE, None) == q.MOE_ERR_ALIGNMENT
    assert L.moe_dequant(9, FAKE, None, 16, 64, FAKE, None) == q.MOE_ERR_INVALID_ARG
    # the grouped path's decode export: CB4 only, otherwise moe_dequant's checks
    assert L.moe_dequant_grouped(q.WFMT_MXFP4, FAKE, None, 16, 64, FAKE, None) == q.MOE_ERR_UNSUPPORTED
    assert L.moe_dequant_grouped(q.WFMT_CB4, FAKE, None, 16, 64, FAKE, None) == q.MOE_ERR_INVALID_ARG
    assert L.moe_dequant_grouped(q.WFMT_CB4, FAKE, FAKE, 16, 48, FAKE, None) == q.MOE_ERR_INVALID_ARG
    assert L.moe_dequant_grouped(q.WFMT_CB4, FAKE + 4, FAKE, 16, 64, FAKE, None) == q.MOE_ERR_ALIGNMENT
    assert L.moe_rms_rescale(FAKE, 2, 0, 1e-6, FAKE, None) == q.MOE_ERR_INVALID_ARG
    assert L.moe_rms_rescale(None, 2, 8, 1e-6, FAKE, None) == q.MOE_ERR_INVALID_ARG
    assert L.moe_rms_rescale(FAKE, 0, 8, 1e-6, FAKE, None) == q.MOE_OK


def test_status_strings(L):
    for s in range(-5, 1):
        assert q.status_str(s) not in ("", "unknown status")
    assert q.status_str(-99) == "unknown status"


def test_workspace_grows_with_tokens(L):
    lay = layer()
    assert ws_bytes(L, lay, 0) < ws_bytes(L, lay, 1) < ws_bytes(L, lay, 1024)


def test_workspace_covers_header_and_fp8_planes(L):
    """The fixed header (arrival flags + the decode router's logit mailbox: 18,432 bytes)
    comes first, and the activation regions also hold the MXFP4 prefill's fp8 planes,
    which exceed the bf16 planes for small H and I (rows padded to 128 / 256 columns)."""
    T = 64
    lay = layer(hidden=32, inter=32, n_experts=8, top_k=2, wfmt=q.WFMT_MXFP4, codebook=None, has_shared=1)
    P = T * 2 + T
    need = ws_bytes(L, lay, T)
    assert need >= 18432 + (3 * T * 128 + T) + (3 * P * 256 + P)
    assert ws_bytes(L, layer(), 1) >= 18432


# ---------------------------------------------------------------------------
# The header's storage definition, followed literally, gives the bytes the generator and
# the test encoder write (so a caller packing by the header feeds the kernels correctly).
# ---------------------------------------------------------------------------
HEADER_FORMULAS = [
    "start at byte t*8*K + 1024*s + (16*g + m)*16",
    "entry t*16*nkb + 64*s + i of the plane",
    "MXFP4: i = 16*g + m, entries are bytes (byte S + entry)",
    "CB4:   i = m*r + g, entries are little-endian fp16 (bytes S + 2*entry, +1)",
    "scale plane at byte S = round_up(N*K/2, 256)",
]


def _pack_by_header(wfmt, codes, scales):
    """Element by element, as include/moeq.h states the layout."""
    N, K = codes.shape
    nkb = K // 32
    S = (N * K // 2 + 255) // 256 * 256
    out = bytearray(S + N * nkb * (1 if wfmt == q.WFMT_MXFP4 else 2))
    for row in range(N):
        t, m = row // 16, row % 16
        for b in range(nkb):
            s, g = b // 4, b % 4
            r = min(4, nkb - 4 * s)
            base = t * 8 * K + 1024 * s + (16 * g + m) * 16
            for j in range(16):   # byte j: element 2j low nibble, 2j+1 high nibble
                out[base + j] = int(codes[row, 32 * b + 2 * j]) | (int(codes[row, 32 * b + 2 * j + 1]) << 4)
            i = 16 * g + m if wfmt == q.WFMT_MXFP4 else m * r + g
            entry = t * 16 * nkb + 64 * s + i
            v = int(scales[row, b])
            if wfmt == q.WFMT_MXFP4:
                out[S + entry] = v
            else:
                out[S + 2 * entry], out[S + 2 * entry + 1] = v & 0xFF, v >> 8
    return np.frombuffer(bytes(out), dtype=np.uint8)


@pytest.mark.parametrize("wfmt", [q.WFMT_MXFP4, q.WFMT_CB4])
@pytest.mark.parametrize("N,K", [(16, 32), (32, 160), (48, 256)])
def test_header_layout_matches_encoders(wfmt, N, K):
    import numpy as np_
    import packing
    import synth
    text = " ".join(open(HEADER).read().split())
    for f in HEADER_FORMULAS:
        assert " ".join(f.split()) in text, f"header no longer states: {f}"
    rng = np_.random.default_rng(N + K + wfmt)
    codes = rng.integers(0, 16, (N, K), dtype=np_.uint8)
    if wfmt == q.WFMT_MXFP4:
        scales = rng.integers(118, 125, (N, K // 32)).astype(np_.uint8)
    else:
        scales = rng.uniform(0.01, 0.05, (N, K // 32)).astype(np_.float16).view(np_.uint16)
    got = _pack_by_header(wfmt, codes, scales)
    assert got.size == q.packed_bytes(wfmt, N, K)
    assert np_.array_equal(got, packing.pack(wfmt, codes, scales))
    code_rows = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np_.uint8)
    assert np_.array_equal(got, synth.to_tile_major(code_rows, scales, wfmt))


def test_noalloc_validates_before_touching_the_gpu(L):
    """moe_forward_noalloc checks its arguments and the scratch size on the host first."""
    lay = layer(hidden=2880, inter=2880, n_experts=128, top_k=4, wfmt=q.WFMT_MXFP4, codebook=None)
    assert ws_bytes(L, lay, 1024) > 32 << 20
    assert L.moe_forward_noalloc(ctypes.byref(lay), FAKE, q.DT_BF16, 1024, FAKE, None, 0) == q.MOE_ERR_WORKSPACE
    assert L.moe_forward_noalloc(ctypes.byref(lay), FAKE, 7, 1, FAKE, None, 0) == q.MOE_ERR_INVALID_ARG
    assert L.moe_forward_noalloc(ctypes.byref(lay), FAKE, q.DT_BF16, -1, FAKE, None, 0) == q.MOE_ERR_INVALID_ARG
    assert L.moe_forward_noalloc(ctypes.byref(lay), FAKE, q.DT_BF16, 0, None, None, 0) == q.MOE_OK


def test_packed_scale_store_bytes_and_validation(L):
    """The packed scale store: the page's 12,839,040 bytes per gpt-oss-120B expert, and
    like MXFP4 it takes no codebook."""
    ps = q.WFMT_MXFP4_PS
    assert q.packed_bytes(ps, 5760, 2880) + q.packed_bytes(ps, 2880, 2880) == 12_839_040
    assert q.packed_bytes(ps, 16, 96) == 768 + 16 + 16 * 3 // 2
    assert q.packed_bytes(ps, 8, 64) == 0
    lay = layer(wfmt=ps, codebook=FAKE)
    assert ws_bytes(L, lay, 4) == 0
    lay = layer(wfmt=ps, codebook=None)
    assert ws_bytes(L, lay, 4) > 0


def test_affine3_bytes_and_validation(L):
    a3 = q.WFMT_AFF3
    assert q.packed_bytes(a3, 1280, 2560) + q.packed_bytes(a3, 2560, 640) == 2_150_400
    assert q.packed_bytes(a3, 16, 96) == 0          # columns in steps of 128
    assert ws_bytes(L, layer(wfmt=a3, codebook=None, hidden=256, inter=128), 4) > 0
    assert ws_bytes(L, layer(wfmt=a3, codebook=None, hidden=256, inter=96), 4) == 0
    assert ws_bytes(L, layer(wfmt=a3, codebook=FAKE, hidden=256, inter=128), 4) == 0
    assert L.moe_dequant(a3, FAKE, None, 16, 64, FAKE, None) == q.MOE_ERR_INVALID_ARG
