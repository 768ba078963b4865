"""Seeded synthetic inputs for the routed MoE layer.

This module only draws random inputs and writes them in the packed storage
layout; it computes none of the layer's arithmetic (no decoding, routing,
projection or combine).  Both the CPU oracle (through the tests) and the GPU
library (through the tests and the benchmark) consume what it produces.

Packed storage of one quantised matrix with N rows (a multiple of 16) and K
columns (a multiple of 32), blocks of 32 consecutive values along a row; byte j
of a block's 16 code bytes holds element 2j in its low nibble and element 2j+1
in its high nibble.  The storage is tile-major: rows go in tiles of 16, a row's
blocks in steps of 4 (the last step of a row may hold fewer, r = nkb - 4s).

* code plane: tile t, step s is one unit at byte t*8K + s*1024 holding, for
  block g < r of the step and row m < 16 of the tile, the block's 16 code
  bytes at (16g + m)*16 inside the unit;
* scale plane: starts at round_up(N*K/2, 256); tile t, step s is one unit at
  scale index t*16*nkb + 64*s; inside it MXFP4 keeps the E8M0 byte of (block g,
  row m) at 16g + m and CB4 keeps the little-endian fp16 bits of (row m, block
  g) at m*r + g (units of two bytes).

The total size equals the row-major size (N*K/2 code bytes + N*K/32 scales).

Shapes follow the pages' models: gpt-oss-120B (hidden 2880, 128 experts,
top-4, 36 layers; "Neural Server" page, "What it runs on and what it runs")
and a Flash-Next-like layer (256 routed experts plus one shared expert,
top-8), with decode windows of at most 17 tokens and 1,024-token prefill
chunks.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence

import numpy as np

WFMT_MXFP4 = 1
WFMT_CB4 = 2
WFMT_MXFP4_PS = 3   # MXFP4 codes with the packed scale store
WFMT_AFF3 = 4       # 3-bit affine, groups of 64 with an fp16 scale and bias
X_F32 = 0
X_BF16 = 1

# tensor ids inside one (config, layer, expert) seed tuple
_T_CODES_GU, _T_SCALES_GU, _T_CODES_D, _T_SCALES_D = 0, 1, 2, 3
_T_ROUTER_W, _T_ROUTER_B, _T_X, _T_CODEBOOK, _T_PERM, _T_SHGATE = 10, 11, 12, 13, 14, 15
_SHARED_SLOT = 100_000  # expert index used in the seed tuple of the shared expert


def round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def scale_plane_offset(rows: int, cols: int) -> int:
    return round_up(rows * cols // 2, 256)


def packed_nbytes(wfmt: int, rows: int, cols: int) -> int:
    nblk = rows * cols // 32
    if wfmt == WFMT_AFF3:
        return round_up(rows * cols * 3 // 8, 256) + rows * (cols // 64) * 4
    if wfmt == WFMT_MXFP4_PS:
        return scale_plane_offset(rows, cols) + rows + nblk // 2
    return scale_plane_offset(rows, cols) + nblk * (1 if wfmt == WFMT_MXFP4 else 2)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def random_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    """n uniformly distributed bytes (both nibbles uniform over 16 codes)."""
    words = rng.bit_generator.random_raw((n + 7) // 8)
    return words.view(np.uint8)[:n].copy() if n % 8 else words.view(np.uint8)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


@dataclasses.dataclass
class WeightSpec:
    wfmt: int
    scale_lo: float = 0.01      # CB4: fp16 scale ~ U(lo, hi)
    scale_hi: float = 0.05
    e8m0_lo: int = 118          # MXFP4: E8M0 byte uniform in [lo, hi]
    e8m0_hi: int = 124


@dataclasses.dataclass
class LayerSpec:
    name: str
    T: int
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    has_shared: int
    weights: WeightSpec
    x_dtype: int
    router_std: float
    bias: str                   # "none" | "normal" | "zipf"
    bias_std: float = 0.0
    zipf_s: float = 1.1
    n_layers: int = 1
    seed: int = 0


def to_tile_major(code_rows: np.ndarray, scale_rows: np.ndarray, wfmt: int) -> np.ndarray:
    """Arrange row-major code bytes [N][K/2] and scales [N][K/32] (uint8 E8M0 or uint16
    fp16 bits) into the packed tile-major storage described in the module docstring."""
    N, half = code_rows.shape
    nkb = half // 16
    assert N % 16 == 0 and scale_rows.shape == (N, nkb)
    T = N // 16
    codes = code_rows.reshape(T, 16, nkb, 16)                   # tile, row m, block, byte
    code_units, scale_units = [], []
    for s in range(0, nkb, 4):
        r = min(4, nkb - s)
        code_units.append(codes[:, :, s:s + r, :].transpose(0, 2, 1, 3).reshape(T, r * 256))
        sc = scale_rows.reshape(T, 16, nkb)[:, :, s:s + r]       # tile, row m, block g
        if wfmt == WFMT_MXFP4:
            scale_units.append(sc.transpose(0, 2, 1).reshape(T, r * 16))
        else:
            scale_units.append(sc.reshape(T, 16 * r))
    code_plane = np.concatenate(code_units, axis=1).reshape(-1)
    scale_plane = np.concatenate(scale_units, axis=1).reshape(-1)
    out = np.zeros(packed_nbytes(wfmt, N, nkb * 32), dtype=np.uint8)
    out[:code_plane.size] = code_plane
    off = scale_plane_offset(N, nkb * 32)
    sb = scale_plane.astype(np.uint8 if wfmt == WFMT_MXFP4 else np.dtype("<u2")).view(np.uint8)
    out[off:off + sb.size] = sb
    return out


def to_packed_scale_store(code_rows: np.ndarray, e8m0_rows: np.ndarray) -> np.ndarray:
    """MXFP4 codes [N][K/2] and E8M0 bytes [N][K/32] in the packed scale store: the raw
    store's code plane, then at the scale-plane offset one base byte per row (the row's
    smallest E8M0 byte) and one 4-bit delta per block (E8M0 - base), the delta of block
    (row, b) at the nibble whose index is the block's entry in the raw tile-major scale
    plane (low nibble first).  Rows whose E8M0 bytes span more than 15 are refused."""
    N, nkb = e8m0_rows.shape
    e = e8m0_rows.astype(np.int64)
    base = e.min(axis=1)
    delta = e - base[:, None]
    if delta.max(initial=0) > 15:
        raise ValueError("a row's E8M0 bytes span more than 15: not representable in the packed scale store")
    raw = to_tile_major(code_rows, delta.astype(np.uint8), WFMT_MXFP4)  # deltas in the raw scale order
    off = scale_plane_offset(N, nkb * 32)
    d = raw[off:off + N * nkb]
    out = np.zeros(packed_nbytes(WFMT_MXFP4_PS, N, nkb * 32), dtype=np.uint8)
    out[:off] = raw[:off]
    out[off:off + N] = base.astype(np.uint8)
    out[off + N:] = (d[0::2] | (d[1::2] << 4)).astype(np.uint8)
    return out


def to_affine3(q: np.ndarray, sbits: np.ndarray, bbits: np.ndarray) -> np.ndarray:
    """3-bit codes q [N][K] (0..7), fp16 scale and bias bits [N][K/64] in the 3-bit affine
    storage: rows in tiles of 16, columns in steps of 128 (K % 128 == 0); the lane
    l = 16 g + m of unit (tile t, step s) owns 12 bytes (three little-endian words) at
    t*6K + 768 s + 12 l holding the 32 values of row m at columns 32 j + 8 g + i
    (j, i < 4, 8): pair P = 4 j + i // 2, member i % 2; pairs 0..14 at bits
    3 (P % 5) + 16 (i % 2) of word P // 5, pair 15 with bit k of q at bit 15 + 16 (i % 2)
    of word k.  Then, at round_up(N K 3/8, 256), per (t, s) 128 bytes: row m's
    (scale, bias) of the step's two groups at 8 m."""
    N, K = q.shape
    assert N % 16 == 0 and K % 128 == 0
    q = q.astype(np.uint32).reshape(N // 16, 16, K // 128, 4, 4, 8)   # t, m, s, j, g, i
    q = q.transpose(0, 2, 4, 1, 3, 5).reshape(N // 16, K // 128, 64, 16, 2)  # t, s, lane, P, half
    words = np.zeros((N // 16, K // 128, 64, 3), dtype=np.uint32)
    for P in range(15):
        for half in range(2):
            words[..., P // 5] |= q[..., P, half] << np.uint32(3 * (P % 5) + 16 * half)
    for k in range(3):
        for half in range(2):
            words[..., k] |= ((q[..., 15, half] >> np.uint32(k)) & np.uint32(1)) << np.uint32(15 + 16 * half)
    code = words.astype("<u4").view(np.uint8).reshape(-1)
    off = round_up(N * K * 3 // 8, 256)
    out = np.zeros(packed_nbytes(WFMT_AFF3, N, K), dtype=np.uint8)
    out[:code.size] = code
    sb = np.stack([sbits.reshape(N // 16, 16, K // 128, 2), bbits.reshape(N // 16, 16, K // 128, 2)], axis=-1)
    sb = sb.transpose(0, 2, 1, 3, 4).astype("<u2").reshape(-1)            # t, s, m, group, (s, b)
    out[off:off + 2 * sb.size] = sb.view(np.uint8)
    return out


def make_packed(spec: WeightSpec, rows: int, cols: int, seed_key: Sequence[int],
                codes_tid: int, scales_tid: int) -> np.ndarray:
    """One packed matrix [rows][cols].  The code bytes (row-major, both nibbles uniform) and
    the scales (row-major) are drawn first, then stored tile-major."""
    assert cols % 32 == 0 and rows % 16 == 0
    nblk = rows * cols // 32
    if spec.wfmt == WFMT_AFF3:
        # q uniform over 0..7; s ~ U(lo, hi) and b = -s (3.5 + U(-0.5, 0.5)), both rounded to fp16
        q = _rng(*seed_key, codes_tid).integers(0, 8, size=(rows, cols), dtype=np.uint8)
        srng = _rng(*seed_key, scales_tid)
        sc = srng.uniform(spec.scale_lo, spec.scale_hi, size=(rows, cols // 64))
        bias = -sc * (3.5 + srng.uniform(-0.5, 0.5, size=sc.shape))
        return to_affine3(q, sc.astype(np.float16).view(np.uint16), bias.astype(np.float16).view(np.uint16))
    code_rows = random_bytes(_rng(*seed_key, codes_tid), rows * cols // 2).reshape(rows, cols // 2)
    srng = _rng(*seed_key, scales_tid)
    if spec.wfmt in (WFMT_MXFP4, WFMT_MXFP4_PS):
        sc = srng.integers(spec.e8m0_lo, spec.e8m0_hi + 1, size=nblk, dtype=np.uint8)
    else:
        sc = srng.uniform(spec.scale_lo, spec.scale_hi, size=nblk).astype(np.float16).view(np.uint16)
    if spec.wfmt == WFMT_MXFP4_PS:  # the same draws as the raw MXFP4 store, re-encoded
        return to_packed_scale_store(code_rows, sc.reshape(rows, cols // 32))
    return to_tile_major(code_rows, sc.reshape(rows, cols // 32), spec.wfmt)


def make_codebook(seed: int, layer: int) -> np.ndarray:
    """16 distinct integers from [-127, 127], drawn with the seed, sorted ascending (int8)."""
    rng = _rng(seed, layer, 0, _T_CODEBOOK)
    vals = rng.choice(np.arange(-127, 128), size=16, replace=False)
    return np.sort(vals).astype(np.int8)


def zipf_log_prior(seed: int, layer: int, n_experts: int, s: float) -> np.ndarray:
    """Per-expert bias ln p, p the Zipf(s) rank probabilities over a seeded rank permutation."""
    ranks = np.arange(1, n_experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    perm = _rng(seed, layer, 0, _T_PERM).permutation(n_experts)
    return np.log(p[perm]).astype(np.float32)


@dataclasses.dataclass
class Layer:
    """Host copy of one synthetic layer (all arrays numpy)."""
    spec: LayerSpec
    layer_index: int
    router_w: np.ndarray                    # [E][H] float32
    router_b: Optional[np.ndarray]          # [E] float32 or None
    gate_up: List[np.ndarray]               # E(+1) packed [2I][H] uint8
    down: List[np.ndarray]                  # E(+1) packed [H][I] uint8
    codebook: Optional[np.ndarray]          # [16] int8 (CB4) or None
    shared_gate_w: Optional[np.ndarray]     # [H] float32 or None

    @property
    def hidden(self): return self.spec.hidden
    @property
    def inter(self): return self.spec.inter
    @property
    def n_experts(self): return self.spec.n_experts
    @property
    def top_k(self): return self.spec.top_k
    @property
    def wfmt(self): return self.spec.weights.wfmt
    @property
    def has_shared(self): return self.spec.has_shared


def _expert_pair(spec: LayerSpec, layer: int, e: int):
    key = (spec.seed, layer, e)
    gu = make_packed(spec.weights, 2 * spec.inter, spec.hidden, key, _T_CODES_GU, _T_SCALES_GU)
    dn = make_packed(spec.weights, spec.hidden, spec.inter, key, _T_CODES_D, _T_SCALES_D)
    return gu, dn


def make_layer(spec: LayerSpec, layer: int = 0, experts: Optional[Sequence[int]] = None,
               threads: Optional[int] = None, shared_gate: bool = False) -> Layer:
    """Generate one layer.  `experts` restricts which routed experts get weights
    (the others are left as None, for CPU runs that only need the selected ones)."""
    E, H = spec.n_experts, spec.hidden
    rw = _rng(spec.seed, layer, 0, _T_ROUTER_W).normal(0.0, spec.router_std, size=(E, H)).astype(np.float32)
    if spec.bias == "normal":
        rb = _rng(spec.seed, layer, 0, _T_ROUTER_B).normal(0.0, spec.bias_std, size=E).astype(np.float32)
    elif spec.bias == "zipf":
        rb = zipf_log_prior(spec.seed, layer, E, spec.zipf_s)
    else:
        rb = None
    want = list(range(E)) if experts is None else sorted(set(int(e) for e in experts))
    slots = want + ([_SHARED_SLOT] if spec.has_shared else [])
    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max(1, nthr)) as ex:
        pairs = list(ex.map(lambda e: _expert_pair(spec, layer, e), slots))
    gate_up: List[Optional[np.ndarray]] = [None] * (E + spec.has_shared)
    down: List[Optional[np.ndarray]] = [None] * (E + spec.has_shared)
    for e, (gu, dn) in zip(slots, pairs):
        idx = E if e == _SHARED_SLOT else e
        gate_up[idx], down[idx] = gu, dn
    cb = make_codebook(spec.seed, layer) if spec.weights.wfmt == WFMT_CB4 else None
    sg = None
    if shared_gate and spec.has_shared:
        sg = _rng(spec.seed, layer, 0, _T_SHGATE).normal(0.0, spec.router_std, size=H).astype(np.float32)
    return Layer(spec, layer, rw, rb, gate_up, down, cb, sg)


def make_x(spec: LayerSpec, T: Optional[int] = None, layer: int = 0, stream: int = 0) -> np.ndarray:
    """Activations [T][H]: float32 for X_F32, uint16 bfloat16 bits for X_BF16 (RNE of N(0,1) fp32)."""
    T = spec.T if T is None else T
    v = _rng(spec.seed, layer, stream, _T_X).standard_normal(size=(T, spec.hidden)).astype(np.float32)
    return v if spec.x_dtype == X_F32 else f32_to_bf16_bits(v)


# ---------------------------------------------------------------------------
# The five workloads.  Seeds are 1000 + config number.
# ---------------------------------------------------------------------------
_CB4 = WeightSpec(WFMT_CB4, 0.01, 0.05)
_MX = WeightSpec(WFMT_MXFP4, e8m0_lo=118, e8m0_hi=124)

CONFIGS = {
    # tiny 4-bit codebook layer, fp32 activations
    "c1": LayerSpec("c1_tiny_cb4", T=4, hidden=256, inter=128, n_experts=8, top_k=2, has_shared=0,
                    weights=_CB4, x_dtype=X_F32, router_std=0.05, bias="none", seed=1001),
    # gpt-oss-120B-shaped decode layer, MXFP4 experts
    "c2": LayerSpec("c2_gptoss_mxfp4_decode", T=1, hidden=2880, inter=2880, n_experts=128, top_k=4,
                    has_shared=0, weights=_MX, x_dtype=X_BF16, router_std=0.02, bias="normal",
                    bias_std=0.5, seed=1002),
    # Flash-Next-like draft/verify window, CB4, shared expert, Zipf routing prior
    "c3": LayerSpec("c3_flashnext_cb4_verify", T=17, hidden=2048, inter=512, n_experts=256, top_k=8,
                    has_shared=1, weights=_CB4, x_dtype=X_BF16, router_std=0.02, bias="zipf",
                    zipf_s=1.1, seed=1003),
    # 36 stacked c2 layers
    "c4": LayerSpec("c4_gptoss_36layer_decode", T=1, hidden=2880, inter=2880, n_experts=128, top_k=4,
                    has_shared=0, weights=_MX, x_dtype=X_BF16, router_std=0.02, bias="normal",
                    bias_std=0.5, n_layers=36, seed=1004),
    # prefill chunks, no bias
    "c5a": LayerSpec("c5a_prefill_cb4", T=1024, hidden=2048, inter=512, n_experts=256, top_k=8,
                     has_shared=1, weights=_CB4, x_dtype=X_BF16, router_std=0.02, bias="none", seed=1005),
    # the layer of "Running Qwen3.8-Flash-Next on a 32 GB Mac with Transformers" (hidden
    # 2,560, 512 routed experts of which 10 are kept, intermediate 640, one shared expert) with its
    # 3-bit affine group-64 experts, at the verify window's 17 tokens
    "aff3": LayerSpec("aff3_flashnext_3bit_verify", T=17, hidden=2560, inter=640, n_experts=512, top_k=10,
                      has_shared=1, weights=WeightSpec(WFMT_AFF3, 0.01, 0.05), x_dtype=X_BF16, router_std=0.02,
                      bias="zipf", zipf_s=1.1, seed=1007),
    "c5b": LayerSpec("c5b_prefill_mxfp4", T=1024, hidden=2880, inter=2880, n_experts=128, top_k=4,
                     has_shared=0, weights=_MX, x_dtype=X_BF16, router_std=0.02, bias="none", seed=1006),
}


def small_spec(name: str, T: int, hidden: int, inter: int, n_experts: int, top_k: int, wfmt: int,
               has_shared: int = 0, x_dtype: int = X_BF16, bias: str = "none", seed: int = 7,
               router_std: float = 0.05, bias_std: float = 0.5) -> LayerSpec:
    """A layer shape for parity sweeps (several tiles plus ragged tails, seconds on the CPU)."""
    if wfmt in (WFMT_MXFP4, WFMT_MXFP4_PS):
        w = WeightSpec(wfmt, e8m0_lo=118, e8m0_hi=124)
    elif wfmt in (WFMT_CB4, WFMT_AFF3):
        w = WeightSpec(wfmt, 0.01, 0.05)
    else:
        raise ValueError("unknown weight format")
    return LayerSpec(name, T=T, hidden=hidden, inter=inter, n_experts=n_experts, top_k=top_k,
                     has_shared=has_shared, weights=w, x_dtype=x_dtype, router_std=router_std,
                     bias=bias, bias_std=bias_std, seed=seed)


def with_packed_scales(spec: LayerSpec) -> LayerSpec:
    """The same MXFP4 layer (same seeds, so the same codes and E8M0 values) stored in the
    packed scale store."""
    assert spec.weights.wfmt == WFMT_MXFP4
    w = dataclasses.replace(spec.weights, wfmt=WFMT_MXFP4_PS)
    return dataclasses.replace(spec, name=spec.name + "_packed_scales", weights=w)
