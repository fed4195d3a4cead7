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
