"""Test-side encoder of the packed tile-major storage, written from its definition
independently of the generator's packer (which a test compares with this one).

Definition: rows in tiles of 16, a row's 32-value blocks in steps of 4 (the last step
may hold r < 4).  Code unit (tile t, step s) starts at byte t*8*cols + 1024*s and holds
block g of the step for row m at (16g + m)*16.  The scale plane starts at
round_up(rows*cols/2, 256); scale unit (t, s) starts at index t*16*nblk + 64*s and holds
MXFP4 (g, m) at 16g + m, CB4 (m, g) at m*r + g.
"""
import numpy as np

MXFP4, CB4, MXFP4_PS, AFF3 = 1, 2, 3, 4


def pack(wfmt, codes, scales):
    """codes: [rows][cols] 4-bit values; scales: [rows][cols/32] E8M0 bytes (MXFP4) or fp16
    bit patterns (CB4).  Returns the packed bytes."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    assert rows % 16 == 0 and cols % 32 == 0
    nblk = cols // 32
    code_bytes = rows * cols // 2
    scale_off = (code_bytes + 255) // 256 * 256
    sbytes = 1 if wfmt == MXFP4 else 2
    out = np.zeros(scale_off + rows * nblk * sbytes, dtype=np.uint8)
    pairs = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8).reshape(rows, nblk, 16)
    sc = np.asarray(scales).reshape(rows, nblk)
    splane = np.zeros(rows * nblk, dtype=np.uint8 if wfmt == MXFP4 else np.uint16)
    for row in range(rows):
        t, m = divmod(row, 16)
        for b in range(nblk):
            s, g = divmod(b, 4)
            r = min(4, nblk - 4 * s)
            at = t * 8 * cols + 1024 * s + (16 * g + m) * 16
            out[at:at + 16] = pairs[row, b]
            unit = t * 16 * nblk + 64 * s
            splane[unit + (16 * g + m if wfmt == MXFP4 else m * r + g)] = sc[row, b]
    out[scale_off:] = splane.astype("<u2" if wfmt == CB4 else np.uint8).view(np.uint8)
    return out


def pack_scale_store(codes, e8m0):
    """The packed scale store of MXFP4 codes [rows][cols] and E8M0 bytes [rows][cols/32],
    block by block: the raw code plane, then at the scale-plane offset the row bases
    (smallest E8M0 byte of the row), then per block the nibble base-relative exponent at
    nibble index = the block's raw scale index (low nibble first)."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    nblk = cols // 32
    e8m0 = np.asarray(e8m0).reshape(rows, nblk).astype(int)
    raw = pack(MXFP4, codes, np.zeros((rows, nblk), dtype=np.uint8))
    scale_off = (rows * cols // 2 + 255) // 256 * 256
    out = np.zeros(scale_off + rows + rows * nblk // 2, dtype=np.uint8)
    out[:scale_off] = raw[:scale_off]
    for row in range(rows):
        base = min(e8m0[row])
        out[scale_off + row] = base
        t, m = divmod(row, 16)
        for b in range(nblk):
            s, g = divmod(b, 4)
            i = t * 16 * nblk + 64 * s + 16 * g + m
            d = e8m0[row, b] - base
            assert 0 <= d <= 15
            at = scale_off + rows + i // 2
            out[at] |= (d if i % 2 == 0 else d << 4)
    return out


def pack_affine3(q, sbits, bbits):
    """The 3-bit affine storage of codes q [rows][cols] (0..7) and fp16 scale/bias bit
    patterns [rows][cols/64], value by value: tiles of 16 rows, steps of 128 columns; for
    column c of step st (cc = c - 128 st, j = cc // 32, g = cc % 32 // 8, i = cc % 8) the
    word holding it is one of three at byte t*6*cols + 768 st + 12 (16 g + m); pair
    P = 4 j + i // 2, member i % 2; P < 15: bits 3 (P % 5) + 16 (i % 2) of word P // 5;
    P = 15: bit k of q at bit 15 + 16 (i % 2) of word k.  Scales and biases at
    round_up(rows*cols*3/8, 256) + t*cols + 128 st + 8 m + 4 (group in step) (+2: bias)."""
    q = np.asarray(q)
    rows, cols = q.shape
    code = (rows * cols * 3 // 8 + 255) // 256 * 256
    out = np.zeros(code + rows * (cols // 64) * 4, dtype=np.uint8)
    words = np.zeros(code // 4, dtype=np.uint64)
    for row in range(rows):
        t, m = divmod(row, 16)
        for c in range(cols):
            st, cc = divmod(c, 128)
            j, r32 = divmod(cc, 32)
            g, i = divmod(r32, 8)
            base = (t * 6 * cols + 768 * st + 12 * (16 * g + m)) // 4
            P, half = 4 * j + i // 2, i % 2
            v = int(q[row, c])
            if P < 15:
                words[base + P // 5] |= v << (3 * (P % 5) + 16 * half)
            else:
                for k in range(3):
                    words[base + k] |= ((v >> k) & 1) << (15 + 16 * half)
    out[:code] = words.astype("<u4").view(np.uint8)
    for row in range(rows):
        t, m = divmod(row, 16)
        for G in range(cols // 64):
            st, gg = divmod(G, 2)
            at = code + t * cols + 128 * st + 8 * m + 4 * gg
            for k, v in ((0, int(sbits[row, G])), (2, int(bbits[row, G]))):
                out[at + k], out[at + k + 1] = v & 0xFF, v >> 8
    return out
