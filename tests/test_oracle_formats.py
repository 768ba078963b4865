"""Pins of the oracle's format decoding against closed forms, library routines and
the byte counts the pages print."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import packing
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# FP4 E2M1 code points as the OCP Microscaling v1.0 spec tabulates them.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _one_block_matrix(codes, scale, wfmt):
    """A 16x32 packed matrix whose row 0 holds the given block; rows 1..15 hold code 0
    with unit scales.  Built with the test-side encoder."""
    c = np.zeros((16, 32), dtype=np.uint8)
    c[0] = codes
    sc = np.full((16, 1), 127 if wfmt == oracle.WFMT_MXFP4 else 0x3C00)
    sc[0, 0] = scale
    buf = packing.pack(wfmt, c, sc)
    assert buf.size == oracle.packed_size(wfmt, 16, 32)
    return buf


def test_block_bytes_land_where_the_storage_definition_says():
    """Row 0's block is the first 16 bytes of the code plane: byte j = element 2j (low
    nibble) | element 2j+1 (high nibble); its scale is the first scale entry."""
    codes = [(5 * i + 1) % 16 for i in range(32)]
    buf = _one_block_matrix(codes, 124, oracle.WFMT_MXFP4)
    assert list(buf[:16]) == [codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(16)]
    assert buf[256] == 124


def test_mxfp4_hand_block_unit_scale():
    codes = list(range(16)) + list(range(16))
    w = oracle.dequant(oracle.WFMT_MXFP4, _one_block_matrix(codes, 127, oracle.WFMT_MXFP4), None, 16, 32)
    assert list(w[0, :16]) == E2M1_TABLE
    assert list(w[0, 16:]) == E2M1_TABLE
    # code 8 is negative zero
    assert np.signbit(w[0, 8]) and w[0, 8] == 0.0
    assert not np.signbit(w[0, 0])


def test_mxfp4_hand_block_eighth_scale():
    codes = [15 - (i % 16) for i in range(32)]
    w = oracle.dequant(oracle.WFMT_MXFP4, _one_block_matrix(codes, 124, oracle.WFMT_MXFP4), None, 16, 32)
    expect = [E2M1_TABLE[c] / 8.0 for c in codes]
    assert list(w[0]) == expect


def test_e2m1_e8m0_exhaustive_closed_form():
    for u in range(256):
        for c in range(16):
            got = float(oracle.e2m1_value(c) * oracle.e8m0_value(u))
            if u == 255:
                assert math.isnan(got)
                continue
            want = math.ldexp(E2M1_TABLE[c], u - 127)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (c, u)


def test_fp16_scale_exhaustive_vs_numpy_half():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.fp16_value(bits)
    lib = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


@pytest.mark.parametrize("scale_bits,factor", [(0x3C00, 1.0), (0x3800, 0.5), (0x0001, 2.0 ** -24),
                                               (0xC000, -2.0), (0x7BFF, 65504.0)])
def test_cb4_hand_block(scale_bits, factor):
    cb = np.array([-127, -100, -64, -33, -17, -8, -3, -1, 0, 2, 5, 9, 21, 47, 88, 127], dtype=np.int8)
    codes = [(7 * i + 3) % 16 for i in range(32)]
    w = oracle.dequant(oracle.WFMT_CB4, _one_block_matrix(codes, scale_bits, oracle.WFMT_CB4), cb, 16, 32)
    assert list(w[0]) == [float(cb[c]) * factor for c in codes]


def test_cb4_exhaustive_scale_times_index():
    """Every fp16 scale pattern times every codebook entry, against numpy's half decoding."""
    cb = np.array(sorted(np.random.default_rng(5).choice(np.arange(-127, 128), 16, replace=False)),
                  dtype=np.int8)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s = bits.view(np.float16).astype(np.float64)
    # one 32-value row per fp16 pattern: 65,536 rows x 32 cols, indices 0..15 twice per row
    rows = 65536
    codes = np.tile(np.tile(np.arange(16, dtype=np.uint8), 2), (rows, 1))
    buf = packing.pack(oracle.WFMT_CB4, codes, bits.reshape(rows, 1))
    w = oracle.dequant(oracle.WFMT_CB4, buf, cb, rows, 32)
    with np.errstate(invalid="ignore"):
        want = s[:, None] * cb.astype(np.float64)[np.tile(np.arange(16), 2)][None, :]
    both_nan = np.isnan(w) & np.isnan(want)
    assert np.array_equal(np.isnan(w), np.isnan(want))
    assert np.array_equal(w[~both_nan], want[~both_nan])


def test_packed_sizes_match_page_figures():
    g = json.load(open(os.path.join(GOLDEN, "page_byte_counts.json")))
    H = I = 2880
    expert = oracle.packed_size(oracle.WFMT_MXFP4, 2 * I, H) + oracle.packed_size(oracle.WFMT_MXFP4, H, I)
    assert expert == g["mxfp4_expert_bytes"]["value"] == 13_219_200
    per_token = g["experts_touched_per_token"]["value"] * expert
    assert per_token == 1_903_564_800
    assert abs(per_token - g["experts_touched_per_token"]["approx_bytes"]) / 1.9e9 < 0.01
    cb = g["cb4_rows_bytes"]
    assert oracle.packed_size(oracle.WFMT_CB4, cb["rows"], cb["values_per_row"]) == cb["value"] == 1440
    assert oracle.packed_size(oracle.WFMT_CB4, 16, 32) - 256 + 16 * 16 == 16 * g["q4_0_bytes_per_32"]["value"]
    # the generator writes the same sizes
    assert synth.packed_nbytes(synth.WFMT_MXFP4, 2 * I, H) + synth.packed_nbytes(synth.WFMT_MXFP4, H, I) == expert


def test_packed_scale_store_size_is_the_pages():
    """One gpt-oss-120B expert in the packed scale store (gate/up [5760][2880] plus down
    [2880][2880]) takes exactly the 12,839,040 bytes the page prints, in the oracle's and
    the generator's size functions alike."""
    g = json.load(open(os.path.join(GOLDEN, "page_byte_counts.json")))
    H = I = 2880
    want = g["mxfp4_packed_scale_expert_bytes"]["value"]
    assert oracle.packed_size(oracle.WFMT_MXFP4_PS, 2 * I, H) + oracle.packed_size(oracle.WFMT_MXFP4_PS, H, I) == want
    assert synth.packed_nbytes(synth.WFMT_MXFP4_PS, 2 * I, H) + synth.packed_nbytes(synth.WFMT_MXFP4_PS, H, I) == want
    # one byte per row plus half a byte per 32-value block, on top of the raw code bytes
    rows = 2 * I + H
    assert rows * H // 2 + rows + rows * (H // 32) // 2 == want


def test_packed_scale_store_hand_encoded_tile():
    """16 rows x 64 columns (2 blocks per row), every code 2 (E2M1 1.0) except code 11
    (-1.5) in element 0 of each row; row m has base byte 110 + m and deltas (m % 4, 15).
    The bytes are placed by hand: bases at the scale offset, then block b of row m's
    delta at nibble 16 b + m (low nibble first)."""
    rows, cols = 16, 64
    S = (rows * cols // 2 + 255) // 256 * 256          # 512
    buf = np.zeros(S + rows + rows * 2 // 2, dtype=np.uint8)
    for m in range(rows):
        for b in range(2):
            at = (16 * b + m) * 16                      # one tile, one step: block b of row m
            buf[at:at + 16] = 0x22
        buf[(16 * 0 + m) * 16] = 0x2B                   # element 0 -> code 11, element 1 -> code 2
        buf[S + m] = 110 + m
    for m in range(rows):
        for b, d in ((0, m % 4), (1, 15)):
            i = 16 * b + m
            buf[S + rows + i // 2] |= d if i % 2 == 0 else d << 4
    assert buf.size == oracle.packed_size(oracle.WFMT_MXFP4_PS, rows, cols)
    w = oracle.dequant(oracle.WFMT_MXFP4_PS, buf, None, rows, cols)
    for m in range(rows):
        s0 = 2.0 ** (110 + m + m % 4 - 127)
        s1 = 2.0 ** (110 + m + 15 - 127)
        assert w[m, 0] == -1.5 * s0 and np.all(w[m, 1:32] == s0)
        assert np.all(w[m, 32:] == s1)


@pytest.mark.parametrize("rows,cols", [(16, 32), (32, 160), (48, 512)])
def test_packed_scale_store_decodes_like_the_raw_store(rows, cols):
    """The page's claim of bit-identical outputs: the same codes and E8M0 values give the
    same dense matrix from the raw and the packed store (E8M0 spans up to 15 per row)."""
    rng = np.random.default_rng(rows + cols)
    codes = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    lo = rng.integers(100, 140, (rows, 1))
    e8 = (lo + rng.integers(0, 16, (rows, cols // 32))).astype(np.uint8)
    raw = packing.pack(packing.MXFP4, codes, e8)
    ps = packing.pack_scale_store(codes, e8)
    code_rows = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(ps, synth.to_packed_scale_store(code_rows, e8))
    assert np.array_equal(oracle.dequant(oracle.WFMT_MXFP4, raw, None, rows, cols),
                          oracle.dequant(oracle.WFMT_MXFP4_PS, ps, None, rows, cols))


def test_packed_scale_store_refuses_wide_rows():
    code_rows = np.zeros((16, 32), dtype=np.uint8)
    e8 = np.full((16, 2), 120, dtype=np.uint8)
    e8[3, 1] = 136                                      # span 16 in row 3
    with pytest.raises(ValueError):
        synth.to_packed_scale_store(code_rows, e8)


@pytest.mark.parametrize("wfmt", [oracle.WFMT_MXFP4, oracle.WFMT_CB4])
def test_layout_single_nonzero_positions(wfmt):
    """One nonzero code at (r, c) lands at (r, c) and only its own block's scale
    multiplies it: checks nibble order, the tile-major code units (two tiles, a partial
    last step of 3 blocks) and the 256-aligned scale plane (rows*cols/2 = 1536 is not
    a multiple of 256 in general; here it is, the partial step covers the other case)."""
    rows, cols = 32, 96
    cb = np.arange(-8, 8, dtype=np.int8) * 3  # index 8 -> 0
    zero_code = 0 if wfmt == oracle.WFMT_MXFP4 else 8
    one_code = 2 if wfmt == oracle.WFMT_MXFP4 else 9   # e2m1(2) = 1.0; cb[9] = 3
    one_val = 1.0 if wfmt == oracle.WFMT_MXFP4 else 3.0
    unit = 127 if wfmt == oracle.WFMT_MXFP4 else 0x3C00
    for r, c in [(0, 0), (0, 1), (17, 33), (31, 95), (3, 64), (16, 70)]:
        codes = np.full((rows, cols), zero_code, dtype=np.uint8)
        codes[r, c] = one_code
        scales = np.full((rows, cols // 32), unit)
        w = oracle.dequant(wfmt, packing.pack(wfmt, codes, scales), cb, rows, cols)
        want = np.zeros((rows, cols))
        want[r, c] = one_val
        assert np.array_equal(w, want)
        scales[r, c // 32] = 130 if wfmt == oracle.WFMT_MXFP4 else 0x4400
        scale = 8.0 if wfmt == oracle.WFMT_MXFP4 else 4.0
        w = oracle.dequant(wfmt, packing.pack(wfmt, codes, scales), cb, rows, cols)
        assert w[r, c] == one_val * scale and np.count_nonzero(w) == 1


@pytest.mark.parametrize("wfmt", [oracle.WFMT_MXFP4, oracle.WFMT_CB4])
@pytest.mark.parametrize("rows,cols", [(16, 32), (32, 96), (48, 160), (16, 2880)])
def test_generator_packer_matches_test_encoder(wfmt, rows, cols):
    """The generator's reshape-based packer and the test-side loop encoder agree byte for byte."""
    rng = np.random.default_rng(rows + cols + wfmt)
    codes = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    if wfmt == oracle.WFMT_MXFP4:
        sc = rng.integers(0, 256, (rows, cols // 32), dtype=np.uint8)
    else:
        sc = rng.integers(0, 65536, (rows, cols // 32)).astype(np.uint16)
    code_rows = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(synth.to_tile_major(code_rows, sc, wfmt), packing.pack(wfmt, codes, sc))


def test_bf16_rounding_two_implementations():
    """The oracle's nearest-even bf16 rounding against the generator's integer-bit rounding."""
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(4000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e4).astype(np.float32),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 - 2 ** -9, 3.0], dtype=np.float32)])
    assert np.array_equal(oracle.round_to_bf16_bits(v.astype(np.float64)), synth.f32_to_bf16_bits(v))
    # ties go to even
    assert oracle.round_to_bf16_bits(np.array([1 + 2 ** -8]))[0] == 0x3F80
    assert oracle.round_to_bf16_bits(np.array([1 + 3 * 2 ** -8]))[0] == 0x3F82


# ---------------------------------------------------------------------------
# 3-bit affine, group 64 ("Running Qwen3.8-Flash-Next on a 32 GB Mac with Transformers")
# ---------------------------------------------------------------------------
def test_affine3_size_is_the_pages():
    """An expert of the page's model (hidden 2,560, intermediate 640) in 3-bit codes with
    one 16-bit scale and one 16-bit bias for each group of 64 values: 3.5 bits per weight, 2,150,400 B, the page's
    2.15 MB per expert."""
    g = json.load(open(os.path.join(GOLDEN, "page_byte_counts.json")))["affine3_expert_bytes"]
    H, I = g["shape"]["hidden"], g["shape"]["inter"]
    got = oracle.packed_size(oracle.WFMT_AFF3, 2 * I, H) + oracle.packed_size(oracle.WFMT_AFF3, H, I)
    assert got == g["value"] == 3 * H * I * 7 // 16
    assert round(got / 1e6, 2) == 2.15
    assert synth.packed_nbytes(synth.WFMT_AFF3, 2 * I, H) + synth.packed_nbytes(synth.WFMT_AFF3, H, I) == got


def test_affine3_hand_encoded_tile():
    """One 16 x 128 unit placed by hand: q = 5 at (row 3, column 45) (j 1, g 1, i 5: lane
    19, pair 6, high member: bits 19..21 of word 1), q = 6 at (row 0, column 127) (lane
    48, pair 15, high member: bit 31 of words 1 and 2), scale 2 and bias -1 for row 3's
    first group, every other scale and bias 0."""
    rows, cols = 16, 128
    code = 768
    buf = np.zeros(code + 16 * 2 * 4, dtype=np.uint8)
    buf[12 * 19 + 4 + 2] = 5 << 3                 # word 1 of lane 19, bits 16..23: q at bit 19
    buf[12 * 48 + 4 + 3] |= 0x80                  # bit 31 of word 1 of lane 48: bit 1 of q
    buf[12 * 48 + 8 + 3] |= 0x80                  # bit 31 of word 2: bit 2 of q
    buf[code + 8 * 3: code + 8 * 3 + 4] = [0x00, 0x40, 0x00, 0xBC]   # s = 2.0, b = -1.0
    assert buf.size == oracle.packed_size(oracle.WFMT_AFF3, rows, cols)
    w = oracle.dequant(oracle.WFMT_AFF3, buf, None, rows, cols)
    want = np.zeros((rows, cols))
    want[3, :64] = -1.0
    want[3, 45] = 2.0 * 5 - 1.0
    want[0, 127] = 0.0 * 6 + 0.0                   # scale 0 there: check the code separately
    assert np.array_equal(w, want)
    q, s, b = oracle.affine3_fields(buf, rows, cols)
    assert q[3, 45] == 5 and q[0, 127] == 6 and q.sum() == 11


def test_affine3_values_exact_and_encoders_agree():
    """s * q + b of fp16 s, b and 3-bit q is exact in fp64 (at most 43 significant bits):
    checked against rational arithmetic; the test encoder and the generator's agree."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    q = rng.integers(0, 8, (32, 256), dtype=np.uint8)
    s = rng.uniform(-3, 3, (32, 4)).astype(np.float16)
    s[0, 0], s[1, 1] = np.float16(6.0e-8), np.float16(65504.0)      # smallest subnormal, largest finite
    b = rng.uniform(-3, 3, (32, 4)).astype(np.float16)
    b[0, 0], b[1, 1] = np.float16(-65504.0), np.float16(6.0e-8)
    sb, bb = s.view(np.uint16), b.view(np.uint16)
    buf = packing.pack_affine3(q, sb, bb)
    assert np.array_equal(buf, synth.to_affine3(q, sb, bb))
    w = oracle.dequant(oracle.WFMT_AFF3, buf, None, 32, 256)
    for r, c in [(0, 0), (1, 64 + 7), (5, 200), (31, 255), (17, 130)]:
        exact = Fraction(float(s[r, c // 64])) * int(q[r, c]) + Fraction(float(b[r, c // 64]))
        assert Fraction(w[r, c]) == exact
