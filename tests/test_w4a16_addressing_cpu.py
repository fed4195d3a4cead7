"""Host model of the many-token W4A16 kernels' buffer addressing (csrc/w4a16.hip,
``w4a16_big_kernel`` and the 256 x 256 ``w4a16_tile_kernel``): every load the hardware may perform
stays inside its tensor.

A raw buffer load (stride 0) returns zero without touching memory when its per-lane offset is at
or past the descriptor's ``num_records``; the scalar offset is added to the address but is not part
of that range check. So a load is safe when either the per-lane offset is out of range, or the
whole access ``base + voffset + soffset .. + size`` lies inside the tensor. This model repeats the
kernel's index arithmetic (block, wave, lane, row tile j, group g) for the shapes of the GPU parity
tests and checks that condition for the activations, codes, float16 steps and packed zero points.
"""
import numpy as np
import pytest

GROUP = 128
BIG_TOKENS = 128
WAVES = 4


def _nj(n_tokens):
    return 4 if n_tokens > 512 else 1


def _check_x(n_tokens, d_in, ld_x):
    """Activations: a block's 128 tokens, 8 DMA loads per wave and group."""
    x_bytes = ((n_tokens - 1) * ld_x + d_in) * 2
    lane = np.arange(64)
    G = d_in // GROUP
    for by in range((n_tokens + BIG_TOKENS - 1) // BIG_TOKENS):
        tok0 = by * BIG_TOKENS
        base = tok0 * ld_x * 2
        valid = min(BIG_TOKENS, n_tokens - tok0)
        nrec = valid * ld_x * 2
        for wave in range(WAVES):
            for j in range(8):
                tr = 32 * wave + 16 * (j >> 2) + 4 * (j & 3) + (lane >> 4)
                voff = tr * ld_x * 2 + (((lane & 15) ^ (tr & 15)) * 16)
                for g in range(G):
                    soff = g * GROUP * 2
                    live = voff < nrec
                    end = base + voff + soff + 16
                    assert np.all(~live | ((base + voff + soff >= 0) & (end <= x_bytes))), (by, wave, j, g)


def _check_rows(n_tokens, d_in, d_out, row_step_in_voffset=True):
    """Codes, steps and zero points of each wave's 16 NJ rows. Returns the number of live accesses
    outside their tensor (0 for the kernel's layout)."""
    nj = _nj(n_tokens)
    G, GZ = d_in // GROUP, (d_in // GROUP + 1) // 2
    rows_per_wave = 16 * nj
    lane = np.arange(64)
    n, kq = lane & 15, lane >> 4
    tensors = {  # (bytes per row, per-lane in-row offset, size, offset of group g)
        "codes": (d_in // 2, kq * 16, 16, lambda g: g * (GROUP // 2)),
        "steps": (G * 2, 0 * lane, 2, lambda g: g * 2),
        "zeros": (GZ, 0 * lane, 1, lambda g: g >> 1),
    }
    bad = 0
    for bx in range((d_out + 64 * nj - 1) // (64 * nj)):
        for wave in range(WAVES):
            row0 = bx * (4 * rows_per_wave) + wave * rows_per_wave
            vrows = max(0, min(rows_per_wave, d_out - row0))
            r0 = min(row0, d_out - 1)
            for name, (row_bytes, inrow, size, goff) in tensors.items():
                total = d_out * row_bytes
                base = r0 * row_bytes
                nrec = vrows * row_bytes
                for j in range(nj):
                    for g in range(G):
                        if row_step_in_voffset:
                            voff = (16 * j + n) * row_bytes + inrow
                            soff = goff(g)
                        else:  # row tile step in the scalar offset (unchecked by the range test)
                            voff = n * row_bytes + inrow
                            soff = 16 * j * row_bytes + goff(g)
                        live = voff < nrec
                        lo = base + voff + soff
                        bad += int(np.sum(live & ((lo < 0) | (lo + size > total))))
    return bad


SHAPES = [
    (33, 384, 300), (128, 256, 256), (300, 1152, 520), (129, 128, 17),
    (600, 384, 300), (513, 128, 520), (1024, 256, 300), (1300, 384, 520), (2049, 128, 17),
    (4096, 4096, 12288),
]


@pytest.mark.parametrize("n_tokens,d_in,d_out", SHAPES)
def test_weight_loads_stay_inside(n_tokens, d_in, d_out):
    assert _check_rows(n_tokens, d_in, d_out) == 0


@pytest.mark.parametrize("n_tokens,d_in,ld_x", [(33, 384, 384), (129, 128, 128), (1300, 384, 392),
                                                 (2049, 128, 136), (300, 1152, 1152)])
def test_activation_loads_stay_inside(n_tokens, d_in, ld_x):
    _check_x(n_tokens, d_in, ld_x)


def test_model_detects_row_steps_outside_the_range_check():
    # with the 16-row step in the scalar offset, rows 32..63 of a 17-row matrix would be read
    assert _check_rows(2049, 128, 17, row_step_in_voffset=False) > 0


# ------------------------------------------------------------------ the 256 x 256 tile kernel (>= 1024 tokens)

TILE = 256


def _swz(row):
    return (row & 7) ^ ((row >> 3) & 1)


def _check_tile(n_tokens, d_in, d_out, ld_x):
    """Activation DMA (8 loads per wave and K step, the row in the per-lane offset, the K step in the
    scalar one) and the per-thread codes / step / zero-point loads of every tile."""
    x_bytes = ((n_tokens - 1) * ld_x + d_in) * 2
    G, GZ = d_in // 128, (d_in // 128 + 1) // 2
    k_steps = d_in // 64
    lane = np.arange(64)
    tid = np.arange(256)
    bad = 0
    for tm in range((n_tokens + TILE - 1) // TILE):
        m0 = tm * TILE
        rows_a = min(TILE, n_tokens - m0)
        base = m0 * ld_x * 2
        nrec = (rows_a - 1) * ld_x * 2 + d_in * 2
        for wave in range(4):
            for j in range(8):
                row = (4 * j + wave) * 8 + (lane >> 3)
                voff = row * ld_x * 2 + (((lane & 7) ^ _swz(row)) << 4)
                live = voff < nrec
                for ks in range(k_steps):
                    lo = base + voff + ks * 128
                    bad += int(np.sum(live & ((lo < 0) | (lo + 16 > x_bytes))))
    for tn in range((d_out + TILE - 1) // TILE):
        n0 = tn * TILE
        vrows = max(0, min(TILE, d_out - n0))
        r0 = min(n0, d_out - 1)
        for row_bytes, inrow, size, soffs in (
                (d_in // 2, 0, 16, [ks * 32 for ks in range(k_steps)]),
                (d_in // 2, 16, 16, [ks * 32 for ks in range(k_steps)]),
                (G * 2, 0, 2, [(ks >> 1) * 2 for ks in range(k_steps)]),
                (GZ, 0, 1, [ks >> 2 for ks in range(k_steps)])):
            total = d_out * row_bytes
            voff = tid * row_bytes + inrow
            live = voff < vrows * row_bytes
            for so in soffs:
                lo = r0 * row_bytes + voff + so
                bad += int(np.sum(live & ((lo < 0) | (lo + size > total))))
    return bad


@pytest.mark.parametrize("n_tokens,d_in,d_out,ld_x", [
    (1024, 256, 300, 256), (1300, 384, 520, 384), (2049, 128, 17, 128), (1100, 384, 300, 392),
    (4096, 4096, 12288, 4096), (1024, 11008, 4096, 11008)])
def test_tile_kernel_loads_stay_inside(n_tokens, d_in, d_out, ld_x):
    assert _check_tile(n_tokens, d_in, d_out, ld_x) == 0


# ------------------------------------------------------------------ the one-token kernel

GEMV_WAVES, GEMV_DEPTH, GEMV_BLOCKS, GEMV_MAX_IN = 8, 8, 512, 32768


def _gemv_launch(d_in, d_out):
    W = (d_in // 128 + 15) // 16
    rpw = (d_out + GEMV_WAVES * GEMV_BLOCKS - 1) // (GEMV_WAVES * GEMV_BLOCKS)
    return W, rpw, (d_out + GEMV_WAVES * rpw - 1) // (GEMV_WAVES * rpw)


def _check_gemv(d_in, d_out):
    """Every wave's prefetch ring (D windows ahead, loads past the wave's last window clamped to it),
    its consumption order, the activation staging and the LDS reads. Returns how often each (row,
    window) was consumed and each row written."""
    G, GZ = d_in // 128, (d_in // 128 + 1) // 2
    W, rpw, blocks = _gemv_launch(d_in, d_out)
    assert W * 4096 <= 65536
    lane = np.arange(64)
    lg = lane >> 2
    consumed = np.zeros((d_out, W), int)
    written = np.zeros(d_out, int)
    code_bytes, n_steps, n_zeros = d_out * d_in // 2, d_out * G, d_out * GZ
    c = np.arange(GEMV_MAX_IN // 8)  # staging: chunk c -> LDS slot, only chunks below W 256 stored
    cc = c & 255
    slot = (c >> 8) * 256 + (cc & 3) * 64 + (cc >> 2)
    stored = c < W * 256
    assert np.all(slot[stored] < W * 256) and len(set(slot[stored])) == W * 256
    assert np.all((c[stored] * 8 >= d_in) | (c[stored] * 8 + 8 <= d_in))  # a chunk is wholly in x or past it
    for b in range(blocks):
        for wave in range(GEMV_WAVES):
            r0 = (b * GEMV_WAVES + wave) * rpw
            r1 = min(r0 + rpw, d_out)
            n_items = (r1 - r0) * W if r1 > r0 else 0
            ld = {"row": r0, "win": 0, "count": 0}

            def load():
                inside = ld["count"] < n_items
                o = ld["row"] if inside else r1 - 1
                g = np.minimum((ld["win"] if inside else W - 1) * 16 + lg, G - 1)
                a = o * (d_in // 2) + g * 64 + (lane & 3) * 16
                assert o >= 0 and np.all(a >= 0) and np.all(a + 16 <= code_bytes)
                assert np.all(o * G + g < n_steps) and np.all(o * GZ + (g >> 1) < n_zeros)
                ld["count"] += 1
                ld["win"] += 1
                if ld["win"] == W:
                    ld["win"], ld["row"] = 0, ld["row"] + 1

            for _ in range(GEMV_DEPTH):  # unconditional: a wave without rows re-reads the last row
                load()
            crow, cwin = r0, 0
            for base in range(0, n_items, GEMV_DEPTH):
                for u in range(GEMV_DEPTH):
                    if base + u < n_items:
                        consumed[crow, cwin] += 1
                        assert np.all(cwin * 256 + lane + 64 * 3 < W * 256)
                        cwin += 1
                        if cwin == W:
                            written[crow] += 1
                            cwin, crow = 0, crow + 1
                    if base + GEMV_DEPTH < n_items:
                        load()
    return consumed, written


@pytest.mark.parametrize("d_in,d_out", [(128, 1), (128, 17), (2176, 300), (640, 1), (1920, 8193), (4224, 4097),
                                        (32768, 40), (4096, 12288), (28672, 8192), (11008, 4096), (256, 40000)])
def test_one_token_kernel_loads_and_coverage(d_in, d_out):
    consumed, written = _check_gemv(d_in, d_out)
    assert np.all(consumed == 1) and np.all(written == 1)


def test_one_token_diagonal_lanes():
    # the 16x16 accumulator's diagonal sits in lanes 20 q + i (q, i < 4), element i, one per lane
    lane = np.arange(64)
    i = (lane & 15) - 4 * (lane >> 4)
    diag = (i >= 0) & (i < 4)
    rows, cols = 4 * (lane[diag] >> 4) + i[diag], lane[diag] & 15
    assert np.array_equal(rows, cols) and sorted(rows) == list(range(16))


def test_one_token_dequant_identity():
    # the nibble pairs placed in float16 mantissas and the two fused multiply-adds reproduce
    # (q - zero) * step exactly in float32, for every code, zero point and a spread of float16 steps
    # (subnormal, smallest normal, 1, largest); float64 evaluates the fma exactly
    steps = np.array([2.0 ** -24, 2.0 ** -14, 0.00123, 1.0, 3.5, 65504.0], np.float16).astype(np.float64)
    q = np.arange(16)
    for w in [0x76543210, 0xFEDCBA98, 0x0F0F0F0F, 0xF0F0F0F0]:
        nib = [(w >> (4 * e)) & 15 for e in range(8)]
        w8 = w >> 8
        h = [(w & 0x000F000F) | 0x64006400, (w & 0x00F000F0) | 0x64006400,
             (w8 & 0x000F000F) | 0x64006400, (w8 & 0x00F000F0) | 0x64006400]
        halves = np.array([[x & 0xFFFF, x >> 16] for x in h], np.uint16).view(np.float16).astype(np.float64)
        # h0 = (1024 + q0, 1024 + q4), h1 = (1024 + 16 q1, 1024 + 16 q5), h2 / h3 likewise for 2, 6 / 3, 7
        assert np.array_equal(halves[0], 1024 + np.array([nib[0], nib[4]]))
        assert np.array_equal(halves[1], 1024 + 16 * np.array([nib[1], nib[5]]))
        assert np.array_equal(halves[2], 1024 + np.array([nib[2], nib[6]]))
        assert np.array_equal(halves[3], 1024 + 16 * np.array([nib[3], nib[7]]))
    for s in steps:
        for z in range(16):
            c0 = np.float32(-(1024 + z) * s)
            c16 = np.float32(-(64 + z) * s)
            assert c0 == -(1024 + z) * s and c16 == -(64 + z) * s  # the constants are exact in float32
            v0 = np.float32((1024 + q) * np.float64(np.float32(s)) + np.float64(c0))
            v1 = np.float32((1024 + 16 * q) * np.float64(np.float32(s * 0.0625)) + np.float64(c16))
            want = (q - z) * s
            assert np.array_equal(v0.astype(np.float64), want) and np.array_equal(v1.astype(np.float64), want)


def test_one_token_row_ranges_at_the_largest_d_out():
    # the ABI admits d_out up to 2^31 - 257; there the last wave's row range would end at 2^31, so the
    # kernel forms it in 64 bits and clamps to d_out: every wave's [r0, r1) stays inside [0, d_out],
    # the ranges tile the rows, and the host's grid arithmetic needs 64 bits as well
    d_out = 0x7FFFFFFF - 256
    per = GEMV_WAVES * GEMV_BLOCKS
    assert d_out + per - 1 > 2**31 - 1  # the host's rounding up overflows 32 bits
    W, rpw, blocks = _gemv_launch(128, d_out)
    assert blocks * GEMV_WAVES * rpw >= d_out and (blocks - 1) * GEMV_WAVES * rpw < d_out
    ends = []
    for wv in range(blocks * GEMV_WAVES):
        r0l = wv * rpw
        r0, r1 = min(r0l, d_out), min(r0l + rpw, d_out)
        assert 0 <= r0 <= r1 <= d_out <= 2**31 - 1
        ends.append((r0, r1))
    assert max(wv * rpw + rpw for wv in range(blocks * GEMV_WAVES)) > 2**31 - 1  # why 64 bits
    assert ends[0][0] == 0 and ends[-1][1] == d_out
    assert all(a[1] == b[0] for a, b in zip(ends, ends[1:]))
