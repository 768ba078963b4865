"""Plain fp64 CPU oracle of the routed MoE feed-forward layer over block-quantised experts.

TEST INFRASTRUCTURE ONLY.  The parity tests, the smoke check and the CPU-baseline
leg of the benchmark use this module; the GPU library never imports or calls it,
and it shares no code with the GPU library.  It is written to be checked by eye:
each function is the plain definition of one step, in float64, with numpy's
matmul/exp as the only library primitives.

What the layer computes, in the order the pages describe it:

* the router turns each token's hidden state into one logit per expert and
  keeps k experts with their normalised weights ("Nebula" page, "How it works":
  the router assigns normalised weights to each expert; "How Neural runs a
  120-billion-parameter model on one gaming PC", section "How one token and one
  prompt are processed": the router kernels emit 4 expert ids and 4 weights);
* (token, expert) pairs are grouped by expert, and each selected expert is read
  once for all of its tokens (NInfer Qwen3.8-Flash-Next page, MoE execution
  notes: the pairs are sorted by expert on the device and an expert's weights
  serve every token routed to it; Neural page, "Prompt processing": the
  device groups tokens by expert);
* each expert runs a fused gate/up projection, the middle activation, and a
  down projection (NInfer page, MoE execution notes: the fused gate/up kernel
  and the down pass row by row over all of a token's experts);
* the weighted expert outputs are summed per token (NInfer page, MoE execution
  notes: the sum of the weighted outputs is independent of which expert
  completes first), plus an always-on shared expert where the layer has one
  ("Running Qwen3.8-Flash-Next on a 32 GB Mac with Transformers",
  "Architecture": each layer has 512 routed experts and a single shared one).

Where the pages leave a step open the plainest reading is taken:

* MXFP4 element = E2M1(code) * 2^(u-127), u the block's E8M0 byte (OCP
  Microscaling Formats v1.0; the pages only name "MXFP4", Neural page, "What it
  runs on and what it runs");
* CB4 element = fp16(scale) * codebook[index], 32 values per block with one fp16
  scale and 16 bytes of 4-bit indices, 18 bytes per 32 values (NInfer page,
  n-gram table paragraph: 16 rows of 160 values take 1,440 bytes in IQ4_NL);
  the 16-entry int8 codebook is an input (a seeded sorted table stands in for
  the real IQ4_NL table, which the pages do not list);
* nibble order: low nibble = even element; per matrix a code plane then a
  scale plane, each stored tile-major (16-row tiles, 4-block steps; see
  storage_index) so that one 16-row step of codes is one contiguous 1 KB unit;
  gate_up = [gate rows; up rows] concatenated;
* activation = SwiGLU, h = silu(gate) * up, silu(a) = a / (1 + exp(-a));
* top-k order = descending logit, ties to the lower expert index; gates =
  softmax over the k kept logits; a router bias is added to the logit;
* bucket order inside an expert = increasing pair id p = t*k + j; the shared
  expert is bucket E with pairs T*k + t;
* the shared expert's weight is 1, or sigmoid(w_sg . x_t) when a shared-gate
  vector is given ("Nebula" page, components table: an F32 shared expert gate).

Every function here is pinned by CPU tests against something other than itself
(closed forms of the formats, brute force over subsets, a dense masked
evaluation, 50-digit decimal arithmetic, library sorts).  The RMS rescale
helper between stacked layers is pinned by closed forms as well.
"""

from __future__ import annotations

import math

import numpy as np

WFMT_MXFP4 = 1
WFMT_CB4 = 2
WFMT_MXFP4_PS = 3   # MXFP4 codes with the packed scale store (one base byte per row + 4-bit deltas)
WFMT_AFF3 = 4       # 3-bit affine codes, groups of 64 values with an fp16 scale and an fp16 bias
X_F32 = 0
X_BF16 = 1


# ---------------------------------------------------------------------------
# Formats
# ---------------------------------------------------------------------------

def e2m1_value(code):
    """FP4 E2M1 (OCP MX v1.0): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
    exponent 0 is subnormal: m * 0.5; otherwise (1 + m/2) * 2^(e-1).  Code 8 is -0."""
    c = np.asarray(code, dtype=np.int64)
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(sign == 1, -mag, mag)


def e8m0_value(u):
    """E8M0 scale (OCP MX v1.0): 2^(u - 127); byte 255 encodes NaN."""
    u = np.asarray(u, dtype=np.int64)
    with np.errstate(invalid="ignore"):
        return np.where(u == 255, np.nan, np.exp2(u - 127.0))


def fp16_value(bits):
    """IEEE binary16 bits -> value (sign, 5-bit exponent with bias 15, 10-bit fraction)."""
    b = np.asarray(bits, dtype=np.int64)
    sign = np.where((b >> 15) & 1 == 1, -1.0, 1.0)
    ex = (b >> 10) & 0x1F
    fr = (b & 0x3FF).astype(np.float64)
    normal = (1024.0 + fr) * np.exp2(ex - 25.0)
    subnormal = fr * 2.0 ** -24
    special = np.where(fr == 0, np.inf, np.nan)
    return sign * np.where(ex == 0, subnormal, np.where(ex == 31, special, normal))


def bf16_value(bits):
    """bfloat16 bits -> value: the upper 16 bits of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def packed_size(wfmt: int, rows: int, cols: int) -> int:
    """Bytes of one packed matrix: code plane, padded to 256 bytes, then the scale plane
    (MXFP4: a byte per block; CB4: two bytes per block; packed scale store: a byte per row
    plus half a byte per block)."""
    if cols % 32 or rows % 16:
        raise ValueError("rows must be a multiple of 16 and cols a multiple of 32")
    code_bytes = rows * cols // 2
    scale_off = (code_bytes + 255) // 256 * 256
    nblocks = rows * cols // 32
    if wfmt == WFMT_MXFP4_PS:
        return scale_off + rows + nblocks // 2
    if wfmt == WFMT_AFF3:
        if cols % 128:
            raise ValueError("the 3-bit affine format needs cols a multiple of 128")
        code_bytes = rows * cols * 3 // 8
        return (code_bytes + 255) // 256 * 256 + rows * (cols // 64) * 4
    return scale_off + nblocks * (1 if wfmt == WFMT_MXFP4 else 2)


def storage_index(wfmt: int, rows: int, cols: int):
    """Where the tile-major storage keeps each block (row, b), b < cols/32:
    (byte offset of its 16 code bytes, index of its scale in the scale plane).
    Rows form tiles of 16 and a row's blocks form steps of 4 (the last step may hold
    r < 4 blocks).  Tile t, step s is one 1,024-byte code unit at t*8*cols + 1024*s,
    block g of the step for row m at (16g + m)*16 inside it; its scales are one unit at
    index t*16*nblk + 64*s, MXFP4 ordered (g, m) -> 16g + m, CB4 ordered (m, g) -> m*r + g."""
    nkb = cols // 32
    row = np.arange(rows)[:, None]
    b = np.arange(nkb)[None, :]
    t, m = row // 16, row % 16
    st, g = b // 4, b % 4
    r = np.minimum(4, nkb - 4 * st)
    code_off = t * 8 * cols + 1024 * st + (16 * g + m) * 16
    unit = t * 16 * nkb + 64 * st
    scale_idx = unit + (16 * g + m if wfmt == WFMT_MXFP4 else m * r + g)
    return code_off, scale_idx


def packed_scale_store_exponents(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """E8M0 byte of every block [rows][cols/32] of a matrix in the packed scale store.

    The store keeps the MXFP4 code plane and replaces the scale plane by one base byte per
    row followed by one 4-bit delta per block, each block's E8M0 byte being base + delta
    ("How Neural runs a 120-billion-parameter model on one gaming PC", section "What it
    runs on and what it runs": 12,839,040 bytes per expert in the packed-scale store
    against 13,219,200 raw; section "Correctness": only the scales are stored in a new
    encoding and the outputs match bit for bit).  The page gives the byte count and the identity;
    the placement is this reading's: at the raw store's scale-plane offset S, the bases
    as N bytes in row order, then the deltas, one nibble per block, at nibble index equal
    to the block's index in the raw MXFP4 scale plane (storage_index), byte S + N + i // 2,
    low nibble for even i."""
    code_bytes = rows * cols // 2
    S = (code_bytes + 255) // 256 * 256
    nkb = cols // 32
    _, idx = storage_index(WFMT_MXFP4, rows, cols)
    base = packed[S:S + rows].astype(np.int64)
    dbytes = packed[S + rows:S + rows + rows * nkb // 2].astype(np.int64)
    delta = np.where(idx % 2 == 0, dbytes[idx // 2] & 0xF, dbytes[idx // 2] >> 4)
    return base[:, None] + delta


def affine3_fields(packed: np.ndarray, rows: int, cols: int):
    """The 3-bit codes q [rows][cols] and the fp16 scale and bias bit patterns
    [rows][cols/64] of a matrix in the 3-bit affine format.

    The format is the one "Running Qwen3.8-Flash-Next on a 32 GB Mac with Transformers"
    names ("Where every weight lives": 3-bit MLX affine, group 64, 2.15 MB per expert;
    "Quality": about 3.5 bits per weight with scales and biases): each group of 64
    consecutive values of a row has a 16-bit scale s and bias b, and a value is
    s * q + b with a 3-bit code q.  The pages do not give the bit packing; the reading:
    rows in tiles of 16 (t, m = row // 16, row % 16), columns in steps of 128 (cols % 128
    == 0).  For column c of step st, with cc = c - 128 st, j = cc // 32, g = (cc % 32) // 8,
    i = cc % 8: the lane l = 16 g + m of unit (t, st) owns 12 bytes, three little-endian
    32-bit words, at byte t*6*cols + 768*st + 12*l; the value is member i % 2 of pair
    P = 4 j + i // 2; for P < 15 it sits at bits 3 (P % 5) + 16 (i % 2) .. +2 of word P // 5,
    for P = 15 bit k of q is bit 15 + 16 (i % 2) of word k.  The scale plane starts at
    round_up(rows*cols*3/8, 256); unit (t, st) is 128 bytes at t*cols + 128*st, row m's
    8 bytes at 8 m: s and b of the step's first group (columns 0..63), then of its
    second, fp16 little-endian."""
    packed = np.asarray(packed, dtype=np.uint8)
    soff = (rows * cols * 3 // 8 + 255) // 256 * 256
    row = np.arange(rows)[:, None]
    col = np.arange(cols)[None, :]
    t, m = row // 16, row % 16
    st, cc = col // 128, col % 128
    j, g, i = cc // 32, (cc % 32) // 8, cc % 8
    lane = 16 * g + m
    base = t * 6 * cols + 768 * st + 12 * lane
    P = 4 * j + i // 2
    half = i % 2
    words = packed[:soff].view("<u4")
    w = [words[(base + 4 * k) // 4].astype(np.int64) for k in range(3)]
    q_lo = np.zeros((rows, cols), dtype=np.int64)
    for k in range(3):   # words 0, 1, 2 hold pairs 0..4, 5..9, 10..14
        sel = (P // 5) == k
        q_lo = np.where(sel & (P < 15), (w[k] >> (3 * (P % 5) + 16 * half)) & 7, q_lo)
    q15 = sum(((w[k] >> (15 + 16 * half)) & 1) << k for k in range(3))
    q = np.where(P == 15, q15, q_lo)
    sp = packed[soff:soff + rows * (cols // 64) * 4].view("<u2")
    G = np.arange(cols // 64)[None, :]
    sidx = (row // 16) * (cols // 64) * 32 + 64 * (G // 2) + 4 * (row % 16) + 2 * (G % 2)
    return q, sp[sidx], sp[sidx + 1]


def dequant(wfmt: int, packed: np.ndarray, codebook, rows: int, cols: int) -> np.ndarray:
    """Dense fp64 [rows][cols] from one packed matrix (every element exact in fp64)."""
    packed = np.asarray(packed, dtype=np.uint8)
    if wfmt == WFMT_AFF3:
        q, sbits, bbits = affine3_fields(packed, rows, cols)
        s = np.repeat(fp16_value(sbits), 64, axis=1)
        b = np.repeat(fp16_value(bbits), 64, axis=1)
        return s * q + b   # exact: fp16 * 3-bit + fp16 needs at most 43 significant bits
    code_bytes = rows * cols // 2
    scale_off = (code_bytes + 255) // 256 * 256
    nblocks = rows * cols // 32
    code_off, scale_idx = storage_index(WFMT_MXFP4 if wfmt == WFMT_MXFP4_PS else wfmt, rows, cols)
    # the 16 code bytes of every block, in block order: [rows][cols/32][16]
    blk = packed[code_off[:, :, None] + np.arange(16)[None, None, :]].astype(np.int64)
    nib = np.empty((rows, cols // 32, 32), dtype=np.int64)
    nib[:, :, 0::2] = blk & 0xF   # element 2j: low nibble of byte j
    nib[:, :, 1::2] = blk >> 4    # element 2j+1: high nibble
    if wfmt == WFMT_MXFP4:
        scales = e8m0_value(packed[scale_off:scale_off + nblocks][scale_idx])
        vals = e2m1_value(nib)
    elif wfmt == WFMT_MXFP4_PS:
        scales = e8m0_value(packed_scale_store_exponents(packed, rows, cols))
        vals = e2m1_value(nib)
    elif wfmt == WFMT_CB4:
        sbits = packed[scale_off:scale_off + 2 * nblocks].view("<u2")[scale_idx]
        scales = fp16_value(sbits)
        vals = np.asarray(codebook, dtype=np.int64)[nib].astype(np.float64)
    else:
        raise ValueError("unknown weight format")
    w = vals * scales[:, :, None]
    return w.reshape(rows, cols)


def activations_f64(x, x_dtype: int) -> np.ndarray:
    if x_dtype == X_F32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if x_dtype == X_BF16:
        return bf16_value(np.asarray(x, dtype=np.uint16))
    raise ValueError("unknown activation dtype")


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------

def router_logits(x64: np.ndarray, router_w, router_b) -> np.ndarray:
    """l[t,e] = sum_h x[t,h] * W_r[e,h] + b[e], fp64."""
    l = x64 @ np.asarray(router_w, dtype=np.float64).T
    if router_b is not None:
        l = l + np.asarray(router_b, dtype=np.float64)[None, :]
    return l


def topk_softmax(logits: np.ndarray, k: int):
    """Per token: the k largest logits ordered by (-logit, expert index); gates are the
    softmax over those k logits (equal to the full softmax renormalised over the k)."""
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))  # primary -logit, then index
        sel = order[:k]
        ids[t] = sel
        z = np.exp(logits[t, sel] - logits[t, sel[0]])
        gates[t] = z / z.sum()
    return ids, gates


def shared_weights(x64: np.ndarray, shared_gate_w) -> np.ndarray:
    """Weight of the always-on shared expert: 1, or sigmoid(w . x_t) with a gate vector."""
    if shared_gate_w is None:
        return np.ones(x64.shape[0])
    z = x64 @ np.asarray(shared_gate_w, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def omit_marginal(ids: np.ndarray, gates: np.ndarray, tau: float):
    """Marginal-expert omission ("Nebula" page, "Benchmark results": experts under a
    10% gate are dropped as marginal).  The page gives the threshold, not what happens to the
    remaining weights; the reading taken: a routed pair whose softmax gate is below tau is
    left out (the first, largest one never is), and the kept gates are renormalised to sum
    to 1.  Omitted pairs get id -1 and gate 0.  tau = 0 keeps every pair unchanged."""
    ids = np.array(ids, dtype=np.int32, copy=True)
    gates = np.array(gates, dtype=np.float64, copy=True)
    if tau <= 0.0:
        return ids, gates
    T, k = ids.shape
    for t in range(T):
        keep = [j == 0 or gates[t, j] >= tau for j in range(k)]
        total = sum(gates[t, j] for j in range(k) if keep[j])
        for j in range(k):
            if keep[j]:
                gates[t, j] = gates[t, j] / total
            else:
                ids[t, j] = -1
                gates[t, j] = 0.0
    return ids, gates


def bucket(ids: np.ndarray, n_experts: int, has_shared: int):
    """Counting sort of pairs p = t*k + j by expert (stable: increasing p in a bucket).
    Shared-expert pairs p = T*k + t form bucket E; pairs with id -1 (omitted) are in no
    bucket.  Returns counts [E+1], offsets [E+2] (exclusive prefix sums; offsets[E+1] =
    the pairs placed), perm (the placed pair ids in bucket order), inv (position of each
    pair in perm, -1 for an omitted pair)."""
    T, k = ids.shape
    expert_of = list(int(e) for e in ids.reshape(-1))
    if has_shared:
        expert_of += [n_experts] * T
    P = len(expert_of)
    counts = np.zeros(n_experts + 1, dtype=np.int32)
    for e in expert_of:
        if e >= 0:
            counts[e] += 1
    offsets = np.zeros(n_experts + 2, dtype=np.int32)
    for e in range(n_experts + 1):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:n_experts + 1].copy()
    perm = np.empty(offsets[n_experts + 1], dtype=np.int32)
    for p in range(P):
        e = expert_of[p]
        if e < 0:
            continue
        perm[fill[e]] = p
        fill[e] += 1
    inv = np.full(P, -1, dtype=np.int32)
    for i in range(perm.shape[0]):
        inv[perm[i]] = i
    return counts, offsets, perm, inv


# ---------------------------------------------------------------------------
# Experts and combine
# ---------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def expert_ffn(w_gate_up: np.ndarray, w_down: np.ndarray, X: np.ndarray):
    """One expert on the rows of X [n][H]: gate/up projection, SwiGLU, down projection.
    Returns (h [n][I], o [n][H])."""
    I = w_gate_up.shape[0] // 2
    a = X @ w_gate_up.T
    h = silu(a[:, :I]) * a[:, I:]
    return h, h @ w_down.T


def moe_forward(layer, x, x_dtype: int, ids=None, gates=None, want_h: bool = False, map_fn=map,
                omit_below: float = 0.0):
    """The whole layer for the tokens in x.  When `ids`/`gates` are given, routing is
    taken from them (steps after routing only; an id of -1 is an omitted pair).
    omit_below > 0 applies the marginal-expert omission to the computed routing.
    Returns a dict with y [T][H] fp64 and every intermediate the GPU library exposes.
    The experts' products are independent of each other; `map_fn` evaluates them (the
    builtin map: one after another; a thread pool's map gives the same values)."""
    H, I, E, k = layer.hidden, layer.inter, layer.n_experts, layer.top_k
    x64 = activations_f64(x, x_dtype)
    T = x64.shape[0]
    logits = router_logits(x64, layer.router_w, layer.router_b)
    if ids is None:
        ids, gates = topk_softmax(logits, k)
        ids, gates = omit_marginal(ids, gates, omit_below)
    ids = np.asarray(ids, dtype=np.int32).reshape(T, k)
    gates = np.asarray(gates, dtype=np.float64).reshape(T, k)
    s = shared_weights(x64, layer.shared_gate_w) if layer.has_shared else None
    counts, offsets, perm, inv = bucket(ids, E, layer.has_shared)
    P = T * k + (T if layer.has_shared else 0)   # every pair id (omitted ones keep zero rows)

    def one_expert(e):
        pairs = perm[offsets[e]:offsets[e + 1]]
        tokens = np.where(pairs < T * k, pairs // k, pairs - T * k)
        wgu = dequant(layer.wfmt, layer.gate_up[e], layer.codebook, 2 * I, H)
        wd = dequant(layer.wfmt, layer.down[e], layer.codebook, H, I)
        h, oe = expert_ffn(wgu, wd, x64[tokens])
        return pairs, h, oe

    o = np.zeros((P, H))
    h_all = np.zeros((P, I)) if want_h else None
    used = [e for e in range(E + layer.has_shared) if counts[e] > 0]
    for pairs, h, oe in map_fn(one_expert, used):
        o[pairs] = oe
        if want_h:
            h_all[pairs] = h
    y = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            if ids[t, j] >= 0:
                y[t] += gates[t, j] * o[t * k + j]
        if layer.has_shared:
            y[t] += s[t] * o[T * k + t]
    return dict(y=y, logits=logits, ids=ids, gates=gates, shared_w=s, counts=counts,
                offsets=offsets, perm=perm, inv=inv, h=h_all, o=o)


# eps of the rescale as the library receives it: an fp32 number (1e-6 rounded to fp32)
RMS_EPS = float(np.float32(1e-6))


def rms_quotient(y: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """y / sqrt(mean(y^2) + eps) per token (row), in float64."""
    y = np.asarray(y, dtype=np.float64)
    return y / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + eps)


def rms_rescale(y: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Input of the next stacked layer: the fp64 quotient y / sqrt(mean(y^2) + eps) per
    token, rounded to bfloat16 (nearest, ties to even).  Returns uint16 bits."""
    return round_to_bf16_bits(rms_quotient(y, eps))


def round_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even); returns the bits.
    bfloat16 keeps 8 significant bits: with val = m * 2^e (0.5 <= |m| < 1), the result is
    round_half_even(m * 2^8) * 2^(e-8).  Normal range only (|val| >= 2^-126)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    flat_v, flat_o = v.reshape(-1), out.reshape(-1)
    for i, val in enumerate(flat_v):
        m, e = math.frexp(float(val))
        r = math.ldexp(round(m * 256.0), e - 8)   # Python's round() is half-to-even
        bits32 = int(np.array([r], dtype=np.float32).view(np.uint32)[0])  # exact: 8 bits
        flat_o[i] = bits32 >> 16
    return out
