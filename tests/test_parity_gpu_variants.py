"""GPU parity of the grid and quantizer variants, through the C ABI, against the CPU oracle
(oracle/awq_variants.py): the three candidate-scale formulas over explicit ratio lists, the
per-channel weight statistic of the duo formula, the two per-row quantizers, and the search
composed from them.

* Candidate scales within 1e-12 relative (float64 pow and sums, ulp-level differences only).
* Per-row quantizer deltas bit-exact: the kernels take every rounding decision as the float64
  definition does and form the same float64 value, which both sides round to float32 and then to
  the storage dtype. The oracle is fed the GPU's candidate scales so both start from the same s.
* Losses within 1e-3 relative, k* equal up to oracle near-ties, as in the main search."""
import numpy as np
import pytest

from oracle import awq_export as XP
from oracle import awq_oracle as O
from oracle import awq_variants as V
from oracle import parity as P
from workloads import custom_workload, f32_to_bf16_bits, make_w, make_x, to_f32, to_torch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_quantization_mean_amd import binding
    binding.load_library()
    return binding


def _gpu_parts(w, parts, separate=False):
    wt = to_torch(w, "cuda")
    out, r = [], 0
    for i, p in enumerate(parts):
        if separate:
            buf = torch.zeros((p + 5, wt.shape[1]), dtype=wt.dtype, device="cuda")
            buf[2:2 + p].copy_(wt[r:r + p])
            out.append(buf[2:2 + p])
        else:
            out.append(wt[r:r + p])
        r += p
    return out


def _same_nan_rel(got, want):
    got, want = np.asarray(got), np.asarray(want)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    return P.max_rel(got[m], want[m]) if m.any() else 0.0


def _stored(d64, dtype):
    """float64 delta -> float32 (nearest even) -> storage dtype bits, as the kernels store it."""
    d32 = np.asarray(d64, np.float64).astype(np.float32)
    return XP.f32_to_bf16_rne(d32) if dtype == "bf16" else d32.view(np.uint32)


def _gpu_bits(t, dtype):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else t.numpy().view(np.uint32)


GRIDS = {"ms20": V.grid_ms(20), "linspace20": V.grid_linspace(20), "tenths": V.grid_tenths()}


@pytest.mark.parametrize("formula", [V.FORMULA_MSMODELSLIM, V.FORMULA_RMS, V.FORMULA_DUO])
@pytest.mark.parametrize("grid", sorted(GRIDS))
def test_candidate_scales_formulas(B, formula, grid):
    rng = np.random.default_rng(31 + formula)
    d_in = 640
    a = np.exp(rng.normal(-1.0, 1.5, d_in))
    a[[3, 77]] = 0.0            # channels that never fire: a^r = 0 below every floor
    a[[5, 500]] *= 200.0        # outlier channels
    wm = np.abs(rng.normal(0, 0.02, d_in)) + 1e-4
    wm[9] = 0.0                 # an all-zero weight column (wm^(1-r) = 0 for r < 1)
    ratios = GRIDS[grid]
    at = torch.from_numpy(a).cuda()
    wt = torch.from_numpy(wm).cuda()
    got = B.awq_candidate_scales_ex(at, ratios, formula, w_mean=wt).cpu().numpy()
    want = np.stack([V.candidate_scales(formula, a, r, wm) for r in ratios])
    rel = P.max_rel(got, want)
    print(f"[gpu variants] formula {formula} grid {grid}: max rel {rel:.2e}", flush=True)
    assert rel < 1e-12
    if formula == V.FORMULA_MSMODELSLIM and grid == "ms20":
        # the msModelSlim grid through the general kernel equals the main step bit for bit
        main = B.awq_candidate_scales(at, 20).cpu().numpy()
        assert np.array_equal(got, main)


def test_candidate_scales_nonfinite_statistic(B):
    a = np.linspace(0.01, 3.0, 256)
    a[17] = np.nan
    wm = np.full(256, 0.02)
    at, wt = torch.from_numpy(a).cuda(), torch.from_numpy(wm).cuda()
    for formula in (V.FORMULA_MSMODELSLIM, V.FORMULA_RMS, V.FORMULA_DUO):
        ratios = [0.0, 0.3, 1.0]
        got = B.awq_candidate_scales_ex(at, ratios, formula, w_mean=wt).cpu().numpy()
        with np.errstate(invalid="ignore"):
            want = np.stack([V.candidate_scales(formula, a, r, wm) for r in ratios])
        assert _same_nan_rel(got, want) < 1e-12


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("separate", [False, True])
def test_weight_mean(B, dtype, separate):
    wl = custom_workload(16, 384, 520, dtype, config_id=301)
    w = make_w(wl)
    parts = (200, 136, 184)
    got = B.awq_weight_mean(_gpu_parts(w, parts, separate)).cpu().numpy()
    want = V.weight_mean(to_f32(w).astype(np.float64))
    print(f"[gpu variants] weight mean ({dtype}, separate={separate}): max rel {P.max_rel(got, want):.2e}",
          flush=True)
    assert P.max_rel(got, want) < 1e-11


@pytest.mark.parametrize("quantizer", [V.QUANT_INT4_ROW, V.QUANT_INT8_ROW_SYM])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("separate", [False, True])
def test_row_quantizer_delta_bit_exact(B, quantizer, dtype, separate):
    # d_in = 640: one full 512-channel slice and a 128-channel tail per lane sweep
    wl = custom_workload(300, 640, 520, dtype, outlier_channels=3, config_id=302)
    x, w = make_x(wl), make_w(wl).copy()
    w[4, :] = 0                                                               # zero row
    w[6, :] = f32_to_bf16_bits(np.full(640, 0.03125, np.float32)) if dtype == "bf16" else \
        np.full(640, 0.03125, np.float32)                                     # constant row
    if dtype == "bf16":
        w[8, :] = f32_to_bf16_bits(np.abs(to_f32(w[8, :])) + np.float32(0.01))  # one-signed row
    else:
        w[8, :] = np.abs(w[8, :]) + np.float32(0.01)
    parts = (200, 136, 184)
    wp = _gpu_parts(w, parts, separate)
    act = B.awq_act_stats(to_torch(x, "cuda"))
    ratios = V.grid_linspace(7)
    cs = B.awq_candidate_scales_ex(act, ratios, V.FORMULA_MSMODELSLIM)
    delta = B.awq_quant_delta_ex(wp, cs, quantizer)
    torch.cuda.synchronize()
    W = to_f32(w).astype(np.float64)
    cs_np = cs.cpu().numpy()
    print(f"[gpu variants] row quantizer {quantizer} ({dtype}, separate={separate}): 7 candidates", flush=True)
    for k in range(len(ratios)):
        d_or = V.restore(W, cs_np[k], quantizer) - W
        want = _stored(d_or, dtype)
        got = _gpu_bits(delta[k], dtype)
        n_bad = int((got != want).sum())
        if n_bad:
            r, c = np.argwhere(got != want)[0]
            print(f"  k={k}: {n_bad} elements differ, first ({r},{c}) oracle {d_or[r, c]!r}", flush=True)
        assert n_bad == 0


def test_int4_group_quantizer_is_the_main_step(B):
    wl = custom_workload(64, 384, 300, "bf16", config_id=303)
    w = make_w(wl)
    wp = _gpu_parts(w, (300,))
    a = torch.from_numpy(np.exp(np.random.default_rng(5).normal(0, 1, 384))).cuda()
    cs = B.awq_candidate_scales_ex(a, V.grid_tenths(), V.FORMULA_RMS)
    d1 = B.awq_quant_delta_ex(wp, cs, V.QUANT_INT4_GROUP)
    d2 = B.awq_quant_delta(wp, cs)
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))


COMBOS = [
    # (formula, quantizer, grid): the pages' own pairings, plus cross terms
    (V.FORMULA_MSMODELSLIM, V.QUANT_INT4_GROUP, "ms20"),
    (V.FORMULA_DUO, V.QUANT_INT4_ROW, "linspace20"),
    (V.FORMULA_RMS, V.QUANT_INT4_GROUP, "tenths"),
    (V.FORMULA_MSMODELSLIM, V.QUANT_INT8_ROW_SYM, "ms20"),
    (V.FORMULA_DUO, V.QUANT_INT4_GROUP, "linspace20"),
]


@pytest.mark.parametrize("formula,quantizer,grid", COMBOS)
def test_search_ex_against_oracle(B, formula, quantizer, grid):
    wl = custom_workload(600, 384, 520, "bf16", outlier_channels=4, config_id=304)
    x, w = make_x(wl), make_w(wl)
    parts = (200, 136, 184)
    ratios = GRIDS[grid]
    xt = to_torch(x, "cuda")
    wp = _gpu_parts(w, parts)
    act = B.awq_act_stats(xt)
    wm = B.awq_weight_mean(wp) if formula == V.FORMULA_DUO else None
    print(f"[gpu variants] search formula {formula} quantizer {quantizer} grid {grid}", flush=True)
    res = B.awq_search_scales_ex(xt, wp, act, ratios, formula, quantizer, w_mean=wm, cand_per_pass=7)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in res.items()}
    X, W = to_f32(x).astype(np.float64), to_f32(w).astype(np.float64)
    scales, losses, k_or, best = V.search(X, W, ratios, formula, quantizer)
    assert P.max_rel(g["cand_scales"], scales) < 1e-12
    rel = P.max_rel(g["losses"], losses)
    k = int(g["best_info"][0])
    print(f"  losses max rel {rel:.2e}; k* gpu {k} oracle {k_or}", flush=True)
    assert rel < P.LOSS_RTOL
    assert int(g["best_info"][1]) == 0
    assert P.kstar_ok(k, k_or, losses)
    assert np.array_equal(g["best_scales"], g["cand_scales"][k])
    if formula == V.FORMULA_MSMODELSLIM and quantizer == V.QUANT_INT4_GROUP:
        main = B.awq_search_scales(xt, wp, act, 20, cand_per_pass=7)
        torch.cuda.synchronize()
        for key in ("cand_scales", "losses", "best_scales", "best_info"):
            assert np.array_equal(main[key].cpu().numpy(), g[key]), key


def test_no_finite_loss_keeps_unit_scales(B):
    wl = custom_workload(300, 256, 260, "bf16", config_id=305)
    x = make_x(wl).copy()
    x[5, 17] = 0x7FC0  # bf16 NaN: every ratio above 0 gives NaN scales, hence NaN losses
    w = make_w(wl)
    xt = to_torch(x, "cuda")
    wp = _gpu_parts(w, (260,))
    act = B.awq_act_stats(xt)
    res = B.awq_search_scales_ex(xt, wp, act, [0.25, 0.5, 0.75], V.FORMULA_MSMODELSLIM, V.QUANT_INT8_ROW_SYM)
    torch.cuda.synchronize()
    assert np.all(np.isnan(res["losses"].cpu().numpy()))
    assert list(res["best_info"].cpu().numpy()) == [0, 1]
    assert np.all(res["best_scales"].cpu().numpy() == 1.0)
    X, W = to_f32(x).astype(np.float64), to_f32(w).astype(np.float64)
    with np.errstate(invalid="ignore"):
        _, _, _, best = V.search(X, W, [0.25, 0.5, 0.75], V.FORMULA_MSMODELSLIM, V.QUANT_INT8_ROW_SYM)
    assert np.all(best == 1.0)


@pytest.mark.parametrize("quantizer", [V.QUANT_INT4_ROW, V.QUANT_INT8_ROW_SYM])
def test_row_quantizer_full_size_sampled_rows(B, quantizer):
    # the bench layer (7B fused QKV: 12288 x 4096 bf16), all 20 candidates in one launch as the bench
    # times it; 24 sampled rows (part boundaries included) bit-exact against the oracle
    from workloads import workload
    wl = workload(2)
    w = make_w(wl)
    wt = to_torch(w, "cuda")
    parts = [wt[0:4096], wt[4096:8192], wt[8192:12288]]
    rng = np.random.default_rng(12)
    a = np.exp(rng.normal(0.0, 1.0, 4096))
    a[rng.integers(0, 4096, 41)] *= 60.0
    cs = B.awq_candidate_scales_ex(torch.from_numpy(a).cuda(), V.grid_ms(20), V.FORMULA_MSMODELSLIM)
    print(f"[gpu variants] full-size row quantizer {quantizer}: 12288 x 4096, 20 candidates", flush=True)
    delta = B.awq_quant_delta_ex(parts, cs, quantizer)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 4095, 4096, 8191, 8192, 12287], rng.integers(0, 12288, 18)]))
    cs_np = cs.cpu().numpy()
    W = to_f32(w[rows]).astype(np.float64)
    for k in (0, 7, 19):
        d_or = V.restore(W, cs_np[k], quantizer) - W
        got = _gpu_bits(delta[k][torch.from_numpy(rows).cuda()], "bf16")
        assert np.array_equal(got, _stored(d_or, "bf16")), (k, int((got != _stored(d_or, "bf16")).sum()))
