"""GPU parity at the full workload sizes (7B fused QKV, 7B down_proj, 70B fused gate+up, 70B
down_proj stress), in the launch configuration the benchmark times: every candidate in one
quantize->delta launch and one error-GEMM launch, through the C ABI step by step.

The oracle cannot run these searches whole on the host (up to 1.2 PFLOP in float64), so it
checks outputs it can compute one by one:
* the activation statistic over all tokens and every candidate's scales, in full;
* 256 x 256 tiles of the error matrix of chosen candidates (their sums of squares);
* whole row stripes of the error matrix (all tokens x the rows of three 256-row tiles) for the
  chosen ratio and its two neighbours, whose sums of squares are compared with the GPU's;
* delta and the final codes, steps and zero points on sampled weight rows;
and the GPU's own outputs must satisfy what holds at any size: each loss is the fixed-order sum
of its tiles over N * d_out, and k* is the first strict minimum of the losses.
For the 7B QKV layer the oracle's loss over all rows is also computed for k* and its
neighbours, and k* must be a minimum of the oracle's own losses among them.
"""
import numpy as np
import pytest

from oracle import awq_oracle as O
from oracle import parity as P
from workloads import make_w, make_x, to_f32, to_torch, workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_quantization_mean_amd import binding
    binding.load_library()
    return binding


def _f64(a):
    return to_f32(a).astype(np.float64)


def _oracle_act_mean(x_np, block=4096):
    """Mean of |X| over all tokens: the oracle's statistic on row blocks, weighted by block size."""
    n = x_np.shape[0]
    acc = np.zeros(x_np.shape[1])
    for r0 in range(0, n, block):
        blk = _f64(x_np[r0:r0 + block])
        acc += O.act_mean(blk) * (blk.shape[0] / n)
    return acc


def _oracle_sse(x_np, w_rows, s, block=2048):
    """Sum over all tokens and the given weight rows of (X W^T - X What^T)^2, using the oracle's
    output MSE on token blocks."""
    w_hat = O.quantize_restore(w_rows, s, 128)
    tot = 0.0
    for r0 in range(0, x_np.shape[0], block):
        xb = _f64(x_np[r0:r0 + block])
        tot += O.output_mse(xb, w_rows, w_hat) * xb.shape[0] * w_rows.shape[0]
    return tot


def _run(B, wl):
    print(f"[gpu full] {wl.name}: X {wl.n_tokens}x{wl.d_in} W {wl.d_out}x{wl.d_in} n_grid {wl.n_grid}", flush=True)
    x_np, w_np = make_x(wl), make_w(wl)
    xt = to_torch(x_np, "cuda")
    wt = to_torch(w_np, "cuda")
    parts = list(wl.parts) or [wl.d_out]
    wp, r = [], 0
    for p in parts:
        wp.append(wt[r:r + p])
        r += p
    act = B.awq_act_stats(xt)
    cand = B.awq_candidate_scales(act, wl.n_grid)
    delta = B.awq_quant_delta(wp, cand, wl.group_size)
    sse = B.awq_error_sse(xt, delta)
    losses, best, info = B.awq_loss_argmin(sse, wl.n_tokens, wl.d_out, cand)
    pk = B.awq_quantize_pack(wp, best, wl.group_size)
    torch.cuda.synchronize()
    g = {"act_mean": act.cpu().numpy(), "cand": cand.cpu().numpy(), "sse": sse.cpu().numpy(),
         "losses": losses.cpu().numpy(), "best": best.cpu().numpy(), "info": info.cpu().numpy(),
         "codes": pk["codes"].cpu().numpy(), "qscales": pk["qscales"].cpu().numpy(),
         "zeros": pk["zeros"].cpu().numpy()}
    return x_np, w_np, g, delta


def _check(B, cid, full_row_losses=False):
    wl = workload(cid)
    x_np, w_np, g, delta = _run(B, wl)
    n, G = wl.n_grid, wl.d_in // 128
    tiles_m, tiles_n = (wl.n_tokens + 255) // 256, (wl.d_out + 255) // 256

    # statistic and candidate scales, in full
    a = _oracle_act_mean(x_np)
    rel = P.max_rel(g["act_mean"], a)
    print(f"  act_mean max rel err {rel:.2e}", flush=True)
    assert rel < P.ACT_RTOL and rel < 1e-11
    S = np.stack([O.candidate_scales(a, k / n) for k in range(n)])
    assert P.max_rel(g["cand"], S) < 1e-12

    # properties of the GPU's own outputs
    sse = g["sse"].reshape(n, tiles_m, tiles_n)
    want = g["sse"].sum(axis=1) / (wl.n_tokens * wl.d_out)
    assert P.max_rel(g["losses"], want) < 1e-12
    k = int(g["info"][0])
    assert int(g["info"][1]) == 0
    assert k == O.select_best(g["losses"].tolist())
    assert np.array_equal(g["best"], g["cand"][k])
    print(f"  k* = {k}; losses {np.array2string(g['losses'], precision=4)}", flush=True)

    # sampled tiles of the error matrix
    rng = np.random.default_rng(cid)
    picks = [(k, 0, 0), (k, tiles_m - 1, tiles_n - 1), (0, tiles_m // 2, tiles_n // 3),
             (n - 1, int(rng.integers(tiles_m)), int(rng.integers(tiles_n)))]
    for (kk, tm, tn) in picks:
        rows = slice(tn * 256, min(wl.d_out, (tn + 1) * 256))
        toks = slice(tm * 256, min(wl.n_tokens, (tm + 1) * 256))
        w_rows = _f64(w_np[rows])
        xw = _f64(x_np[toks])
        w_hat = O.quantize_restore(w_rows, S[kk], 128)
        want = O.output_mse(xw, w_rows, w_hat) * xw.shape[0] * w_rows.shape[0]
        got = float(sse[kk, tm, tn])
        print(f"  tile (k={kk}, tm={tm}, tn={tn}): gpu {got:.6e} oracle {want:.6e} rel {abs(got - want) / want:.2e}",
              flush=True)
        assert abs(got - want) <= P.LOSS_RTOL * want

    # whole row stripes (all tokens) for k* and its neighbours
    stripe_tiles = sorted({0, tiles_n // 2, tiles_n - 1})
    stripe_rows = np.concatenate([np.arange(t * 256, min(wl.d_out, (t + 1) * 256)) for t in stripe_tiles])
    w_rows = _f64(w_np[stripe_rows])
    ks = [kk for kk in (k - 1, k, k + 1) if 0 <= kk < n]
    or_sse = {}
    for kk in ks:
        or_sse[kk] = _oracle_sse(x_np, w_rows, S[kk])
        got = float(sse[kk][:, stripe_tiles].sum())
        print(f"  stripe k={kk}: gpu {got:.6e} oracle {or_sse[kk]:.6e} rel {abs(got - or_sse[kk]) / or_sse[kk]:.2e}",
              flush=True)
        assert abs(got - or_sse[kk]) <= P.LOSS_RTOL * or_sse[kk]

    # delta on sampled rows (k* and the last candidate)
    samp = np.unique(np.concatenate([np.arange(0, wl.d_out, max(1, wl.d_out // 48)), [wl.d_out - 1]]))
    W_s = _f64(w_np[samp])
    for kk in (k, n - 1):
        d_gpu = delta[kk][torch.as_tensor(samp, device=delta.device)].float().cpu().numpy()
        d_or = O.quantize_restore(W_s, S[kk], 128) - W_s
        pq = O.quantize_pack(W_s, S[kk], 128)
        em, _ = P.exempt_masks(pq.t, pq.zt)
        err = np.abs(d_gpu - d_or)
        assert np.all((err <= P.delta_tolerance(d_or, W_s, pq.qscales, S[kk])) | em)

    # final codes, steps and zero points on sampled rows
    pq = O.quantize_pack(W_s, S[k], 128)
    c = P.compare_codes(g["codes"][samp], g["qscales"][samp], g["zeros"][samp], pq)
    print(f"  codes on {len(samp)} rows: {c}", flush=True)
    assert c["mismatch"] == 0 and c["zero_mismatch"] == 0 and c["step_max_rel"] < P.STEP_RTOL

    if full_row_losses:
        W = _f64(w_np)
        for kk in ks:
            want = _oracle_sse(x_np, W, S[kk]) / (wl.n_tokens * wl.d_out)
            got = float(g["losses"][kk])
            print(f"  full loss k={kk}: gpu {got:.8e} oracle {want:.8e} rel {abs(got - want) / want:.2e}", flush=True)
            assert abs(got - want) <= P.LOSS_RTOL * want
            or_sse[kk] = want
        # the chosen ratio is a minimum of the oracle's own losses among its neighbours
        for kk in ks:
            assert or_sse[k] <= or_sse[kk] * (1 + P.KSTAR_RTOL)
    return g


@pytest.mark.timeout(900)
def test_full_7b_qkv_fused(B):
    _check(B, 2, full_row_losses=True)


@pytest.mark.timeout(900)
def test_full_7b_down_proj(B):
    _check(B, 3)


@pytest.mark.timeout(900)
def test_full_70b_gate_up_fused(B):
    _check(B, 4)


@pytest.mark.timeout(900)
def test_full_70b_down_proj_stress(B):
    _check(B, 5)
