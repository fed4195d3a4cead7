"""GPU parity of the Gram form of the loss (csrc/gram.hip and the error GEMM's kStore / kQuad
epilogues) against the float64 oracle, through the C ABI.

The oracle's loss is the definition, mean((X W^T - X What^T)^2); the Gram form reaches the same
value as sum_o delta[o] (X^T X) delta[o]^T / (N d_out). Checked here:
* G = X^T X against its float64 definition element by element, and its scale exponent;
* the float16 delta against the oracle's What - W (float16 rounding instead of bfloat16);
* every ratio's loss against the oracle's (1e-3) and k* by the pinned rule, on shapes with more
  tokens than input channels (ragged token counts, ragged 256-tiles in d_in and d_out, fused
  parts, several passes), both step by step and inside awq_search_scales, which chooses the Gram
  form for these sizes;
* non-finite weights: every loss NaN and the ones fallback, as the direct form gives.
"""
import numpy as np
import pytest

from oracle import awq_oracle as O
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


def _parts(wt, parts):
    out, r = [], 0
    for p in parts:
        out.append(wt[r:r + p])
        r += p
    return out


def _f16_from_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.float16).astype(np.float64)


@pytest.mark.parametrize("n_tokens,d_in,x_kind", [(1000, 384, "normal"), (2048, 512, "student_t3"),
                                                   (130, 128, "normal")])
def test_gram_matrix(B, n_tokens, d_in, x_kind):
    wl = custom_workload(n_tokens, d_in, 256, "bf16", x_kind=x_kind, outlier_channels=3, config_id=300)
    x = make_x(wl)
    print(f"[gpu gram] G of x{x.shape} {x_kind}", flush=True)
    g16, gexp = B.awq_gram(to_torch(x, "cuda"))
    torch.cuda.synchronize()
    X = to_f32(x).astype(np.float64)
    G = X.T @ X
    e = int(gexp.cpu()[0])
    dmax = np.max(np.diag(G))
    assert 2.0 ** 13 <= dmax * 2.0 ** e < 2.0 ** 14  # the largest entry scales into [2^13, 2^14)
    got = _f16_from_bits(g16) * 2.0 ** -e
    # the 256 x 256 blocks on the diagonal are stored halved (a float16 product): undo it exactly
    blk = np.arange(d_in) // 256
    diag = blk[:, None] == blk[None, :]
    got = np.where(diag, 2.0 * got, got)
    A = np.abs(X).T @ np.abs(X)
    # float16 rounding (2^-11 relative, 2^-25 absolute below the normal range, in scaled units; the
    # halving adds at most 2^-25 there, doubled when undone) and float32 accumulation over the
    # tokens (at most n 2^-24 of the sum of |products|)
    tol = 2.0 ** -11 * np.abs(G) + np.where(diag, 3.0, 1.0) * 2.0 ** -25 * 2.0 ** -e + n_tokens * 2.0 ** -24 * A
    assert np.all(np.abs(got - G) <= tol)
    assert np.all(np.abs(got - got.T) <= 2 * tol)  # both halves of the symmetric product


def test_delta_f16_against_oracle(B):
    wl = custom_workload(700, 384, 600, "bf16", n_grid=4, config_id=301)
    x, w = make_x(wl), make_w(wl)
    xt, wt = to_torch(x, "cuda"), to_torch(w, "cuda")
    wp = _parts(wt, (128, 300, 172))
    act = B.awq_act_stats(xt)
    cs = B.awq_candidate_scales(act, 4)
    d16, dexp = B.awq_quant_delta_f16(wp, cs)
    torch.cuda.synchronize()
    X, W = to_f32(x).astype(np.float64), to_f32(w).astype(np.float64)
    a = O.act_mean(X)
    ex = dexp.cpu().numpy()
    for k in range(4):
        s = O.candidate_scales(a, k / 4)
        d_or = O.quantize_restore(W, s, 128) - W
        pk = O.quantize_pack(W, s, 128)
        em, _ = P.exempt_masks(pk.t, pk.zt)
        raw = _f16_from_bits(d16[k])
        assert np.all(np.isfinite(raw)) and np.max(np.abs(raw)) <= 2.0 ** 14
        got = raw * 2.0 ** -int(ex[k])
        # the bfloat16 tolerance's terms with float16's rounding: 2^-11 |delta|, plus half of
        # float16's subnormal spacing in scaled units
        tol = P.delta_tolerance(d_or, W, pk.qscales, s) - 2.0 ** -8 * np.abs(d_or) + \
            2.0 ** -11 * np.abs(d_or) + 2.0 ** -25 * 2.0 ** -int(ex[k])
        bad = ~((np.abs(got - d_or) <= tol) | em)
        assert not bad.any(), (k, int(bad.sum()))
        # the scale is not needlessly small: the largest delta uses the upper float16 range
        assert np.max(np.abs(raw)) >= 2.0 ** 4


def _gram_losses(B, xt, wp, n_grid, cpp):
    n_tokens = xt.shape[0]
    d_out = sum(p.shape[0] for p in wp)
    act = B.awq_act_stats(xt)
    cs = B.awq_candidate_scales(act, n_grid)
    g16, gexp = B.awq_gram(xt)
    tiles = B.awq_error_tiles(n_tokens, d_out)
    sse = torch.empty((n_grid, tiles), dtype=torch.float64, device="cuda")
    for k0 in range(0, n_grid, cpp):
        nk = min(cpp, n_grid - k0)
        d16, dexp = B.awq_quant_delta_f16(wp, cs[k0:k0 + nk])
        B.awq_gram_error_sse(g16, gexp, d16, dexp, n_tokens, sse[k0:k0 + nk])
    losses, best, info = B.awq_loss_argmin(sse, n_tokens, d_out, cs)
    torch.cuda.synchronize()
    return losses.cpu().numpy(), info.cpu().numpy(), act.cpu().numpy(), sse.cpu().numpy()


GRAM_CASES = [
    # n_tokens, d_in, parts, n_grid, cpp, x_kind
    (2048, 512, (512,), 20, 20, "normal"),
    (1000, 384, (300,), 8, 3, "student_t3"),
    (1500, 256, (128, 256, 96), 12, 12, "normal"),
    (4096, 256, (256,), 20, 7, "student_t3"),
    # 34 row tiles of G, the last 128 wide: 17 pairs of row tiles in the quadratic form
    (8600, 8576, (200,), 2, 2, "normal"),
    # 3 row tiles, the last 128 wide: one pair and the middle row
    (1200, 640, (300, 212), 6, 3, "student_t3"),
    # 4 row tiles x 200 columns: 400 pairs over 256 compute units, one full chunk of first tiles and
    # partners, then a partial one
    (1100, 1024, (2560,), 20, 20, "normal"),
]


@pytest.mark.parametrize("n_tokens,d_in,parts,n_grid,cpp,x_kind", GRAM_CASES)
def test_gram_losses_against_oracle(B, n_tokens, d_in, parts, n_grid, cpp, x_kind):
    d_out = sum(parts)
    wl = custom_workload(n_tokens, d_in, d_out, "bf16", n_grid=n_grid, x_kind=x_kind, outlier_channels=3,
                         config_id=302)
    x, w = make_x(wl), make_w(wl)
    print(f"[gpu gram] losses x{x.shape} parts={parts} n_grid={n_grid} cpp={cpp} {x_kind}", flush=True)
    xt, wt = to_torch(x, "cuda"), to_torch(w, "cuda")
    wp = _parts(wt, parts)
    losses, info, _, sse = _gram_losses(B, xt, wp, n_grid, cpp)
    X, W = to_f32(x).astype(np.float64), to_f32(w).astype(np.float64)
    ref = O.search_scales(X, W, 128, n_grid)
    rel = P.max_rel(losses, ref.losses)
    print(f"  losses max rel err {rel:.3e}; k* gpu {info[0]} oracle {ref.best_k}", flush=True)
    assert rel < P.LOSS_RTOL
    assert int(info[1]) == 0
    assert P.kstar_ok(int(info[0]), ref.best_k, ref.losses)
    # each candidate's own tiles, then zeros up to the direct form's tile count
    own = ((d_in + 255) // 256) * ((d_out + 255) // 256)
    assert np.all(sse[:, own:] == 0.0)


@pytest.mark.parametrize("cpp", [None, 5])
def test_search_scales_takes_the_gram_form(B, cpp):
    n_tokens, d_in, d_out, n_grid = 4096, 256, 512, 20
    assert B.awq_search_loss_form(B.AWQ_DTYPE_BF16, n_tokens, d_in, d_out, n_grid) == B.AWQ_LOSS_GRAM
    wl = custom_workload(n_tokens, d_in, d_out, "bf16", n_grid=n_grid, x_kind="student_t3", outlier_channels=4,
                         config_id=303)
    x, w = make_x(wl), make_w(wl)
    print(f"[gpu gram] awq_search_scales x{x.shape} d_out={d_out} cpp={cpp}", flush=True)
    xt, wt = to_torch(x, "cuda"), to_torch(w, "cuda")
    wp = _parts(wt, (200, 312))
    act = B.awq_act_stats(xt)
    res = B.awq_search_scales(xt, wp, act, n_grid, cand_per_pass=cpp)
    torch.cuda.synchronize()
    X, W = to_f32(x).astype(np.float64), to_f32(w).astype(np.float64)
    ref = O.search_scales(X, W, 128, n_grid)
    losses = res["losses"].cpu().numpy()
    info = res["best_info"].cpu().numpy()
    rel = P.max_rel(losses, ref.losses)
    print(f"  losses max rel err {rel:.3e}; k* gpu {info[0]} oracle {ref.best_k}", flush=True)
    assert rel < P.LOSS_RTOL
    assert int(info[1]) == 0 and P.kstar_ok(int(info[0]), ref.best_k, ref.losses)
    assert np.array_equal(res["best_scales"].cpu().numpy(), res["cand_scales"].cpu().numpy()[int(info[0])])
    # the same losses as the step-by-step Gram form (one code path, one rounding)
    steps, _, _, _ = _gram_losses(B, xt, wp, n_grid, cpp or n_grid)
    assert np.array_equal(losses, steps)


@pytest.mark.parametrize("quant", [None, "int4_row", "int8_row_sym"])
def test_gram_form_with_nonfinite_weights(B, quant):
    n_tokens, d_in, d_out, n_grid = 4096, 256, 256, 20
    wl = custom_workload(n_tokens, d_in, d_out, "bf16", n_grid=n_grid, config_id=304)
    x, w = make_x(wl), make_w(wl)
    w = w.copy()
    w[17, 40] = f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    print(f"[gpu gram] NaN weight, quantizer {quant or 'int4_group'}", flush=True)
    xt, wt = to_torch(x, "cuda"), to_torch(w, "cuda")
    act = B.awq_act_stats(xt)
    if quant is None:
        res = B.awq_search_scales(xt, [wt], act, n_grid)
    else:
        q_c = B.AWQ_QUANT_INT4_ROW if quant == "int4_row" else B.AWQ_QUANT_INT8_ROW_SYM
        res = B.awq_search_scales_ex(xt, [wt], act, [k / n_grid for k in range(n_grid)],
                                     B.AWQ_FORMULA_MSMODELSLIM, q_c)
    torch.cuda.synchronize()
    info = res["best_info"].cpu().numpy()
    assert np.all(np.isnan(res["losses"].cpu().numpy()))
    assert int(info[0]) == 0 and int(info[1]) == B.AWQ_INFO_ALL_NONFINITE
    assert np.all(res["best_scales"].cpu().numpy() == 1.0)


@pytest.mark.parametrize("formula,grid,quant", [("rms", "tenths", "int4_group"), ("duo", "linspace", "int4_group"),
                                                ("duo", "linspace", "int4_row"), ("ms", "ms", "int8_row_sym"),
                                                ("ms", "tenths", "int4_row")])
def test_search_ex_takes_the_gram_form(B, formula, grid, quant):
    # the variant search runs the same loss code with every quantizer (its delta in float16 with a
    # power-of-two scale): a formula, grid and quantizer of the pages, in the Gram regime, against the
    # variant oracle
    from oracle import awq_variants as V
    n_tokens, d_in, d_out = 4096, 256, 384
    ratios = {"tenths": V.grid_tenths(), "linspace": V.grid_linspace(16), "ms": V.grid_ms(20)}[grid]
    f_c = {"rms": B.AWQ_FORMULA_RMS, "duo": B.AWQ_FORMULA_DUO, "ms": B.AWQ_FORMULA_MSMODELSLIM}[formula]
    f_o = {"rms": V.FORMULA_RMS, "duo": V.FORMULA_DUO, "ms": V.FORMULA_MSMODELSLIM}[formula]
    q_c = {"int4_group": B.AWQ_QUANT_INT4_GROUP, "int4_row": B.AWQ_QUANT_INT4_ROW,
           "int8_row_sym": B.AWQ_QUANT_INT8_ROW_SYM}[quant]
    q_o = {"int4_group": V.QUANT_INT4_GROUP, "int4_row": V.QUANT_INT4_ROW, "int8_row_sym": V.QUANT_INT8_ROW_SYM}[quant]
    assert B.awq_search_loss_form(B.AWQ_DTYPE_BF16, n_tokens, d_in, d_out, len(ratios)) == B.AWQ_LOSS_GRAM
    wl = custom_workload(n_tokens, d_in, d_out, "bf16", x_kind="student_t3", outlier_channels=3, config_id=305)
    x, w = make_x(wl), make_w(wl)
    print(f"[gpu gram] awq_search_scales_ex {formula} {grid} {quant} x{x.shape}", flush=True)
    xt, wt = to_torch(x, "cuda"), to_torch(w, "cuda")
    act = B.awq_act_stats(xt)
    wm = B.awq_weight_mean([wt]) if formula == "duo" else None
    res = B.awq_search_scales_ex(xt, [wt], act, ratios, f_c, q_c, w_mean=wm)
    torch.cuda.synchronize()
    X, W = to_f32(x).astype(np.float64), to_f32(w).astype(np.float64)
    _, ref_losses, ref_k, _ = V.search(X, W, ratios, f_o, q_o)
    losses = res["losses"].cpu().numpy()
    info = res["best_info"].cpu().numpy()
    rel = P.max_rel(losses, ref_losses)
    print(f"  losses max rel err {rel:.3e}; k* gpu {info[0]} oracle {ref_k}", flush=True)
    assert rel < P.LOSS_RTOL and P.kstar_ok(int(info[0]), ref_k, ref_losses)


@pytest.mark.parametrize("quant", ["int4_group", "int4_row", "int8_row_sym"])
def test_gram_form_with_tiny_weights(B, quant):
    # weights around 1e-8: the quantizers' step floor (1e-8) decides, so most codes are 0 or +-1 and
    # delta is about as large as the weights; the float16 delta's scale comes from the bound's
    # additive constant, which must still keep every value finite and in range
    from oracle import awq_variants as V
    n_tokens, d_in, d_out, n_grid = 4096, 256, 384, 10
    wl = custom_workload(n_tokens, d_in, d_out, "bf16", n_grid=n_grid, outlier_channels=3, config_id=307)
    x, w = make_x(wl), make_w(wl)
    w = f32_to_bf16_bits((to_f32(w) * 1e-6).astype(np.float32))
    ratios = V.grid_ms(n_grid)
    q_c = {"int4_group": B.AWQ_QUANT_INT4_GROUP, "int4_row": B.AWQ_QUANT_INT4_ROW,
           "int8_row_sym": B.AWQ_QUANT_INT8_ROW_SYM}[quant]
    q_o = {"int4_group": V.QUANT_INT4_GROUP, "int4_row": V.QUANT_INT4_ROW, "int8_row_sym": V.QUANT_INT8_ROW_SYM}[quant]
    assert B.awq_search_loss_form(B.AWQ_DTYPE_BF16, n_tokens, d_in, d_out, n_grid) == B.AWQ_LOSS_GRAM
    print(f"[gpu gram] tiny weights, quantizer {quant}", flush=True)
    xt, wt = to_torch(x, "cuda"), to_torch(w, "cuda")
    act = B.awq_act_stats(xt)
    res = B.awq_search_scales_ex(xt, [wt], act, ratios, B.AWQ_FORMULA_MSMODELSLIM, q_c)
    torch.cuda.synchronize()
    X, W = to_f32(x).astype(np.float64), to_f32(w).astype(np.float64)
    _, ref_losses, ref_k, _ = V.search(X, W, ratios, V.FORMULA_MSMODELSLIM, q_o)
    losses = res["losses"].cpu().numpy()
    info = res["best_info"].cpu().numpy()
    assert np.all(np.isfinite(losses)) and np.all(ref_losses > 0)
    rel = P.max_rel(losses, ref_losses)
    print(f"  losses max rel err {rel:.3e}; k* gpu {info[0]} oracle {ref_k}", flush=True)
    assert rel < P.LOSS_RTOL and P.kstar_ok(int(info[0]), ref_k, ref_losses)


def test_gram_search_in_a_hip_graph(B):
    # the Gram form adds only kernels (transpose, fills, scale choices) to the step: the whole layer
    # captured once and replayed on new activations equals eager runs bit for bit
    n_tokens, d_in, d_out, n_grid = 4096, 256, 512, 8
    assert B.awq_search_loss_form(B.AWQ_DTYPE_BF16, n_tokens, d_in, d_out, n_grid) == B.AWQ_LOSS_GRAM
    wl = custom_workload(n_tokens, d_in, d_out, "bf16", n_grid=n_grid, outlier_channels=3, config_id=306)
    x, w = make_x(wl), make_w(wl)
    print("[gpu gram] HIP graph of the Gram-form layer", flush=True)
    wt = to_torch(w, "cuda")
    wp = _parts(wt, (200, 312))
    x_in = to_torch(x, "cuda").clone()
    x_variants = [x_in.clone(), (x_in.float() * 0.25).to(torch.bfloat16), x_in.flip(0).contiguous()]
    B.awq_layer(x_in, wp, n_grid=n_grid)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = B.awq_layer(x_in, wp, n_grid=n_grid)
    for rep in range(2):
        for xv in x_variants:
            want = {k: v.cpu().numpy() for k, v in B.awq_layer(xv, wp, n_grid=n_grid).items()}
            x_in.copy_(xv)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for key in ("losses", "best_info", "best_scales", "codes", "qscales", "zeros"):
                assert np.array_equal(captured[key].cpu().numpy(), want[key], equal_nan=True), (rep, key)
