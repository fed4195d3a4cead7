"""Pins of the GPU-vs-oracle comparison rules (oracle/parity.py) on planted cases.

Every parity verdict passes through these functions, so each is checked here against hand
values: a tie band that is too wide or too narrow, an inverted exemption mask, a zero-point tie
that does not exempt its whole group, or a wrong side of the k* tolerance fails one of them.
The rules follow the stated parity bar: codes and zero points bit-exact except within 1e-5 of a
rounding tie (round half to even, gsyq.cn section 二 ``pseudo_quantize_int4``), k* equal unless
the oracle's losses differ by less than 1e-6 relative (msModelSlim 缩放因子搜索流程: the ratio
with the smallest error is chosen).
"""
import numpy as np
import pytest

from oracle import awq_oracle as O
from oracle import parity as P


# ------------------------------------------------------------------ tie band

@pytest.mark.parametrize("v,want", [
    (3.5, True), (3.5 + 1e-6, True), (3.5 - 1e-6, True), (-2.5 + 1e-6, True), (-0.5, True),
    (3.5 + 2e-5, False), (3.5 - 2e-5, False), (3.0, False), (-2.0, False), (0.25, False),
    (7.5 + 1.1e-5, False),
])
def test_near_half_band(v, want):
    assert bool(P.near_half(np.array([v]))[0]) is want


def test_near_half_band_is_the_stated_one():
    assert P.TIE_BAND == 1e-5
    v = 12.5 + np.array([0.9e-5, -0.9e-5, 1.1e-5, -1.1e-5])
    assert P.near_half(v).tolist() == [True, True, False, False]


def test_exempt_masks_element_and_group():
    g = 4
    t = np.array([[0.0, 1.5 + 1e-6, 2.2, 3.0, 0.1, 0.2, 0.3, 0.4]])   # element 1 near a tie
    zt = np.array([[1.0, 2.5 - 3e-6]])                                  # group 1's zero near a tie
    em, gm = P.exempt_masks(t, zt, g)
    assert gm.tolist() == [[False, True]]
    assert em.tolist() == [[False, True, False, False, True, True, True, True]]


# ------------------------------------------------------------------ code comparison

def _pack_case():
    """Two rows of two 4-wide groups with known ties: row 0 group 0 has t = 2.5 exactly at
    element 2 (step 0.5, y = 1.25); row 1 group 1 has -min/step = 2.5 (the zero-point tie)."""
    W = np.array([[-1.5, 0.3, 1.25, 6.0, -1.5, 0.3, 1.0, 6.0],
                  [-1.5, 0.3, 1.0, 6.0, -1.25, 0.0, 2.0, 6.25]])
    pq = O.quantize_pack(W, np.ones(8), 4)
    em, gm = P.exempt_masks(pq.t, pq.zt, 4)
    assert em[0, 2] and not em[0, 1] and gm[1, 1] and not gm[0, 0]
    return pq, em, gm


def _gpu_copy(pq):
    return pq.q.copy(), pq.qscales.astype(np.float32).copy(), pq.zeros.copy()


def test_compare_codes_identical():
    pq, em, _ = _pack_case()
    q, st, z = _gpu_copy(pq)
    c = P.compare_codes(O.pack_int4(q), st, z, pq, 4)
    assert c["mismatch"] == 0 and c["zero_mismatch"] == 0 and c["raw_code_diff"] == 0
    assert c["exempt_elements"] == int(em.sum()) and c["exempt_groups"] == 1
    assert c["step_max_rel"] < P.STEP_RTOL


def test_compare_codes_counts_a_planted_non_exempt_mismatch():
    pq, em, _ = _pack_case()
    q, st, z = _gpu_copy(pq)
    assert not em[0, 1]
    q[0, 1] ^= 1
    c = P.compare_codes(O.pack_int4(q), st, z, pq, 4)
    assert c["mismatch"] == 1 and c["raw_code_diff"] == 1


def test_compare_codes_ignores_a_planted_exempt_mismatch():
    pq, em, _ = _pack_case()
    q, st, z = _gpu_copy(pq)
    assert em[0, 2]
    q[0, 2] = 6 if q[0, 2] == 5 else 5            # the other side of the tie
    q[1, 5] = (q[1, 5] + 1) % 16                   # inside the zero-point-tie group
    c = P.compare_codes(O.pack_int4(q), st, z, pq, 4)
    assert c["mismatch"] == 0 and c["raw_code_diff"] == 2


def test_compare_codes_zero_points():
    pq, _, gm = _pack_case()
    q, st, z = _gpu_copy(pq)
    z[1, 1] += 1                                   # exempt group: not counted
    c = P.compare_codes(O.pack_int4(q), st, z, pq, 4)
    assert c["zero_mismatch"] == 0
    z[0, 1] += 1                                   # non-exempt group: counted
    c = P.compare_codes(O.pack_int4(q), st, z, pq, 4)
    assert c["zero_mismatch"] == 1


def test_compare_codes_step_error_is_reported():
    pq, _, _ = _pack_case()
    q, st, z = _gpu_copy(pq)
    st64 = pq.qscales.copy()
    st64[0, 0] *= 1 + 3e-6
    c = P.compare_codes(O.pack_int4(q), st64, z, pq, 4)
    assert abs(c["step_max_rel"] - 3e-6) < 1e-9 and c["step_max_rel"] > P.STEP_RTOL


def test_unpack_codes_nibble_order():
    # E1's bytes: codes 0 3 15 3 -> 0x30 0x3F (low nibble = even element)
    assert P.unpack_codes(np.array([[0x30, 0x3F]], np.uint8)).tolist() == [[0, 3, 15, 3]]


# ------------------------------------------------------------------ chosen ratio

def test_kstar_ok_edges():
    lo = np.array([2.0, 1.0, 1.0 + 0.9e-6, 1.0 + 1.1e-6, 0.5])
    assert P.KSTAR_RTOL == 1e-6
    assert P.kstar_ok(1, 1, lo)
    assert P.kstar_ok(2, 1, lo)           # within 1e-6 relative of the oracle's minimum
    assert not P.kstar_ok(3, 1, lo)       # just outside
    assert not P.kstar_ok(0, 1, lo)
    assert P.kstar_ok(4, 1, lo)           # a strictly lower oracle loss is no error of the GPU's


# ------------------------------------------------------------------ delta tolerance

def test_delta_tolerance_terms():
    g = 2
    d_or = np.array([[256.0, 0.0, 0.0, 0.0]])
    W = np.array([[0.0, 0.0, 2.0 ** 40, 0.0]])
    qscales = np.array([[2.0 ** 16, 2.0]])
    s = np.array([1.0, 2.0 ** 16, 1.0, 4.0])
    tol = P.delta_tolerance(d_or, W, qscales, s, g)
    # 2^-8|d| + 2^-16 step/s + 2^-40|w|, step taken from each element's group
    assert tol.tolist() == [[1.0 + 1.0, 2.0 ** -16 * 2.0 ** 16 / 2.0 ** 16,
                             2.0 ** -16 * 2.0 + 1.0, 2.0 ** -16 * 2.0 / 4.0]]


def test_max_rel():
    assert P.max_rel([1.0, 2.0], [1.0, 2.0]) == 0.0
    assert P.max_rel([1.1, 2.0], [1.0, 2.0]) == pytest.approx(0.1)
    assert P.max_rel([], []) == 0.0
