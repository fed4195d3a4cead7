"""GPU parity: every step of the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs. Sizes here are ones the oracle finishes in seconds while still
spanning several 256-wide tiles and ragged tails; full-size workloads are in
test_parity_gpu_full.py."""
import numpy as np
import pytest

from oracle import awq_oracle as O
from oracle import parity as P
from workloads import custom_workload, f32_to_bf16_bits, make_w, make_x, to_f32, to_torch, workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_quantization_mean_amd import binding
    binding.load_library()  # must be built wherever a GPU is present: raises otherwise
    return binding


def _case(wl, parts=None):
    x = make_x(wl)
    w = make_w(wl)
    parts = parts or (wl.d_out,)
    assert sum(parts) == wl.d_out
    return x, w, parts


def _gpu_parts(w, parts, separate=False):
    """Row slices of one stacked device matrix, or (separate) copies placed apart in memory, which
    makes the kernels look up each row's part."""
    wt = to_torch(w, "cuda")
    out, r = [], 0
    if separate:
        gap = 3  # rows of padding between parts
        buf = torch.zeros((wt.shape[0] + gap * (len(parts) + 1), wt.shape[1]), dtype=wt.dtype, device="cuda")
        for i, p in enumerate(parts):
            o = r + gap * (i + 1)
            buf[o:o + p].copy_(wt[r:r + p])
            out.append(buf[o:o + p])
            r += p
        return out
    for p in parts:
        out.append(wt[r:r + p])
        r += p
    return out


def _run_gpu(B, x, w, parts, n_grid, cand_per_pass=None, separate=False):
    print(f"[gpu case] x{tuple(x.shape)} {x.dtype} w{tuple(w.shape)} parts={parts} n_grid={n_grid} "
          f"cpp={cand_per_pass} separate={separate}", flush=True)
    xt = to_torch(x, "cuda")
    wp = _gpu_parts(w, parts, separate)
    act = B.awq_act_stats(xt)
    res = B.awq_search_scales(xt, wp, act, n_grid, cand_per_pass=cand_per_pass)
    pk = B.awq_quantize_pack(wp, res["best_scales"])
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in res.items()}
    out.update({k: v.cpu().numpy() for k, v in pk.items()})
    out["act_mean"] = act.cpu().numpy()
    return out, xt, wp


def _check_full(B, x, w, parts, n_grid, cand_per_pass=None, per_candidate_codes=True, separate=False):
    g, xt, wp = _run_gpu(B, x, w, parts, n_grid, cand_per_pass, separate)
    X, W = to_f32(x).astype(np.float64), to_f32(w).astype(np.float64)
    ref = O.search_scales(X, W, 128, n_grid)
    assert P.max_rel(g["act_mean"], ref.act_mean) < P.ACT_RTOL
    assert P.max_rel(g["act_mean"], ref.act_mean) < 1e-11  # float64 sums of exact values
    assert P.max_rel(g["cand_scales"], ref.scales) < 1e-12
    loss_rel = P.max_rel(g["losses"], ref.losses)
    print(f"  losses max rel err {loss_rel:.3e}; k* gpu {g['best_info'][0]} oracle {ref.best_k}", flush=True)
    assert loss_rel < P.LOSS_RTOL
    k = int(g["best_info"][0])
    assert int(g["best_info"][1]) == 0
    assert P.kstar_ok(k, ref.best_k, ref.losses)
    assert np.array_equal(g["best_scales"], g["cand_scales"][k])
    pk = O.quantize_pack(W, ref.scales[k], 128)
    c = P.compare_codes(g["codes"], g["qscales"], g["zeros"], pk)
    print(f"  final codes: {c}", flush=True)
    assert c["mismatch"] == 0 and c["zero_mismatch"] == 0 and c["step_max_rel"] < P.STEP_RTOL
    if per_candidate_codes:
        cs = torch.from_numpy(g["cand_scales"]).cuda()
        for kk in range(n_grid):
            pg = B.awq_quantize_pack(wp, cs[kk])
            torch.cuda.synchronize()
            pk = O.quantize_pack(W, ref.scales[kk], 128)
            c = P.compare_codes(pg["codes"].cpu().numpy(), pg["qscales"].cpu().numpy(),
                                pg["zeros"].cpu().numpy(), pk)
            assert c["mismatch"] == 0 and c["zero_mismatch"] == 0 and c["step_max_rel"] < P.STEP_RTOL, (kk, c)
    return g, ref, xt, wp


def test_config1_tiny_fp32_end_to_end(B):
    wl = workload(1)
    x, w, parts = _case(wl)
    g, ref, _, _ = _check_full(B, x, w, parts, wl.n_grid)
    assert ref.best_k > 0  # the two x50 channels make a non-trivial scale win
    assert ref.losses[ref.best_k] <= ref.losses[0]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("separate", [False, True])
def test_ragged_fused_parts(B, dtype, separate):
    wl = custom_workload(600, 384, 520, dtype, n_grid=7, outlier_channels=4, config_id=101)
    x, w, parts = _case(wl, (200, 136, 184))
    _check_full(B, x, w, parts, 7, separate=separate)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_ragged_tile(B, dtype):
    wl = custom_workload(100, 128, 40, dtype, n_grid=3, outlier_channels=1, config_id=102)
    x, w, parts = _case(wl)
    _check_full(B, x, w, parts, 3)


def test_n_grid_one_is_plain_rtn(B):
    wl = custom_workload(300, 256, 300, "bf16", n_grid=1, config_id=103)
    x, w, parts = _case(wl)
    g, ref, _, _ = _check_full(B, x, w, parts, 1)
    assert int(g["best_info"][0]) == 0 and np.all(g["best_scales"] == 1.0)


def test_degenerate_and_one_signed_groups(B):
    wl = custom_workload(260, 256, 270, "bf16", n_grid=5, config_id=104)
    x, w, parts = _case(wl)
    w = w.copy()
    w[3, :] = 0                      # all-zero rows: step floor 1e-8, zero 0, codes 0
    w[7, :128] = 0x3F00              # a constant group (0.5 in bf16)
    w[11, 128:] = f32_to_bf16_bits(np.abs(to_f32(w[11, 128:])) + np.float32(0.05))  # one-signed group
    _check_full(B, x, w, parts, 5)


def test_candidate_passes_are_bitwise_identical(B):
    wl = custom_workload(520, 256, 512, "bf16", n_grid=6, config_id=105)
    x, w, parts = _case(wl)
    outs = [_run_gpu(B, x, w, parts, 6, cpp)[0] for cpp in (1, 4, 6, 6)]
    for o in outs[1:]:
        assert np.array_equal(o["losses"], outs[0]["losses"])
        assert np.array_equal(o["codes"], outs[0]["codes"])
        assert np.array_equal(o["best_info"], outs[0]["best_info"])


def test_delta_and_tile_sums_against_oracle(B):
    wl = custom_workload(700, 256, 600, "bf16", n_grid=4, config_id=106)
    x, w, parts = _case(wl)
    xt = to_torch(x, "cuda")
    wp = _gpu_parts(w, parts)
    act = B.awq_act_stats(xt)
    cs = B.awq_candidate_scales(act, 4)
    delta = B.awq_quant_delta(wp, cs)
    sse = B.awq_error_sse(xt, delta)
    torch.cuda.synchronize()
    X, W = to_f32(x).astype(np.float64), to_f32(w).astype(np.float64)
    a = O.act_mean(X)
    d_gpu = delta.float().cpu().numpy()
    tiles_n = (600 + 255) // 256
    for k in range(4):
        s = O.candidate_scales(a, k / 4)
        d_or = O.quantize_restore(W, s, 128) - W
        pk = O.quantize_pack(W, s, 128)
        em, _ = P.exempt_masks(pk.t, pk.zt)
        err = np.abs(d_gpu[k] - d_or)
        bad = ~((err <= P.delta_tolerance(d_or, W, pk.qscales, s)) | em)
        if bad.any():
            r, c = np.argwhere(bad)[0]
            print(f"  k={k}: {int(bad.sum())} delta elements off, first at ({r},{c}): gpu {d_gpu[k][r, c]!r} "
                  f"oracle {d_or[r, c]!r} w {W[r, c]!r} t {pk.t[r, c]!r} zt {pk.zt[r, c // 128]!r} "
                  f"step {pk.qscales[r, c // 128]!r}", flush=True)
        assert not bad.any()
        E = X @ d_or.T
        for tm in range(3):
            for tn in range(tiles_n):
                blk = E[tm * 256:(tm + 1) * 256, tn * 256:(tn + 1) * 256]
                want = float((blk ** 2).sum())
                got = float(sse[k, tm * tiles_n + tn].item())
                assert abs(got - want) <= P.LOSS_RTOL * want, (k, tm, tn, got, want)


def test_nonfinite_activation_falls_back_to_unit_scales(B):
    wl = custom_workload(300, 256, 260, "bf16", n_grid=4, config_id=107)
    x, w, parts = _case(wl)
    x = x.copy()
    x[5, 17] = 0x7FC0  # bf16 NaN
    g, _, _ = _run_gpu(B, x, w, parts, 4)
    assert np.isnan(g["act_mean"][17]) and np.isfinite(np.delete(g["act_mean"], 17)).all()
    assert np.all(g["cand_scales"][0] == 1.0) and np.all(np.isnan(g["cand_scales"][1:]))
    assert np.all(np.isnan(g["losses"]))
    assert list(g["best_info"]) == [0, 1]
    assert np.all(g["best_scales"] == 1.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_activation_channels_end_to_end(B, dtype):
    """Channels whose activations are all zero have act_mean 0: s = 0^0 = 1 at r = 0 and the floor
    1e-4 at r > 0, which the normaliser turns into extreme group scales (msModelSlim 算法公式); the
    whole search and the pack still match the oracle."""
    wl = custom_workload(500, 384, 300, dtype, n_grid=6, outlier_channels=3, config_id=111)
    x, w, parts = _case(wl)
    x = x.copy()
    x[:, [4, 130, 383]] = 0
    g, ref, _, _ = _check_full(B, x, w, parts, 6)
    assert np.all(g["act_mean"][[4, 130, 383]] == 0.0)
    assert np.all(ref.scales[1:, 4] == ref.scales[1:].min(axis=1))  # the floored channel is the minimum


def test_nonfinite_weights_end_to_end(B):
    """NaN and +/-Inf weights: their groups' steps are NaN / infinite, every loss is NaN (the group's
    restored values reach every token's output), so the search keeps the unit scales (gsyq section 二)
    and flags it; the pack at ones matches the oracle: codes and zero points of those groups 0, the
    others bit-exact; delta of those groups NaN."""
    wl = custom_workload(300, 384, 260, "bf16", n_grid=5, outlier_channels=2, config_id=112)
    x, w, parts = _case(wl)
    w = w.copy()
    w[3, 5] = 0x7FC0                        # NaN in row 3, group 0
    w[17, 200] = 0x7F80                     # +Inf in row 17, group 1
    w[250, 300], w[250, 301] = 0xFF80, 0x7F80  # -Inf and +Inf in row 250, group 2
    g, xt, wp = _run_gpu(B, x, w, parts, 5)
    assert np.all(np.isnan(g["losses"]))
    assert list(g["best_info"]) == [0, 1]
    assert np.all(g["best_scales"] == 1.0)
    W = to_f32(w).astype(np.float64)
    with np.errstate(invalid="ignore"):
        pk = O.quantize_pack(W, np.ones(384), 128)
    assert np.array_equal(P.unpack_codes(g["codes"]), pk.q)
    assert np.array_equal(g["zeros"], pk.zeros)
    qs = g["qscales"].astype(np.float64)
    nan_w = np.isnan(pk.qscales)
    assert np.array_equal(np.isnan(qs), nan_w) and nan_w[3, 0]
    fin = np.isfinite(pk.qscales)
    assert np.array_equal(np.isinf(qs), np.isinf(pk.qscales)) and not fin[17, 1] and not fin[250, 2]
    assert np.max(np.abs(qs[fin] - pk.qscales[fin]) / pk.qscales[fin]) < P.STEP_RTOL
    # delta at two candidates: NaN on exactly the non-finite groups, the rest within tolerance
    cand = torch.from_numpy(np.stack([np.ones(384), O.candidate_scales(g["act_mean"], 0.4)])).cuda()
    d = B.awq_quant_delta(wp, cand, 128)
    torch.cuda.synchronize()
    for kk in range(2):
        sk = cand[kk].cpu().numpy()
        with np.errstate(invalid="ignore"):
            d_or = O.quantize_restore(W, sk, 128) - W
            pq = O.quantize_pack(W, sk, 128)
        d_gpu = d[kk].float().cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isnan(d_gpu), np.isnan(d_or))
        ok = np.isfinite(d_or)
        em, _ = P.exempt_masks(pq.t, pq.zt)
        tol = P.delta_tolerance(d_or, W, np.nan_to_num(pq.qscales), sk)
        assert np.all((np.abs(d_gpu - d_or) <= tol) | em | ~ok)


def test_repeat_runs_are_bitwise_identical(B):
    wl = custom_workload(1024, 512, 768, "bf16", n_grid=5, config_id=108)
    x, w, parts = _case(wl)
    a = _run_gpu(B, x, w, parts, 5)[0]
    b = _run_gpu(B, x, w, parts, 5)[0]
    for key in ("act_mean", "losses", "codes", "qscales", "zeros", "best_info"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_side_stream_matches_default_stream(B):
    # every entry point enqueues on the stream it is given (torch's current stream by default)
    wl = custom_workload(700, 384, 520, "bf16", n_grid=6, config_id=110)
    x, w, parts = _case(wl)
    xt = to_torch(x, "cuda")
    wp = _gpu_parts(w, parts)
    torch.cuda.synchronize()
    want = {k: v.cpu().numpy() for k, v in B.awq_layer(xt, wp, n_grid=6).items()}
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = B.awq_layer(xt, wp, n_grid=6)
    side.synchronize()
    act = B.awq_act_stats(xt, stream=side)
    res = B.awq_search_scales(xt, wp, act, 6, stream=side)
    res.update(B.awq_quantize_pack(wp, res["best_scales"], stream=side))
    side.synchronize()
    for key in ("act_mean", "losses", "best_info", "best_scales", "codes", "qscales", "zeros"):
        assert np.array_equal(got[key].cpu().numpy(), want[key], equal_nan=True), key
        if key != "act_mean":
            assert np.array_equal(res[key].cpu().numpy(), want[key], equal_nan=True), key
    assert np.array_equal(act.cpu().numpy(), want["act_mean"])


def test_concurrent_searches_on_two_streams(B):
    # the library keeps no device state between calls: two layers searched at once on two streams
    # (each with its own workspace) give what each gives alone
    cases = []
    for cid, (n, d_in, d_out) in ((111, (600, 256, 384)), (112, (900, 384, 260))):
        wl = custom_workload(n, d_in, d_out, "bf16", n_grid=5, config_id=cid)
        x, w, parts = _case(wl)
        cases.append((to_torch(x, "cuda"), _gpu_parts(w, parts)))
    alone = [{k: v.cpu().numpy() for k, v in B.awq_layer(xt, wp, n_grid=5).items()} for xt, wp in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    outs = []
    for (xt, wp), st in zip(cases, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            outs.append(B.awq_layer(xt, wp, n_grid=5))
    for st in streams:
        st.synchronize()
    for got, want in zip(outs, alone):
        for key in ("act_mean", "losses", "best_info", "codes", "qscales", "zeros"):
            assert np.array_equal(got[key].cpu().numpy(), want[key], equal_nan=True), key


def test_whole_layer_in_a_hip_graph(B):
    # the library allocates nothing, issues no memset or copy and never synchronizes, so the whole
    # layer can be captured once and replayed; every replay (new activations copied into the captured
    # input, eager work and synchronizations in between) must equal an eager run on the same input
    wl = custom_workload(640, 384, 520, "bf16", n_grid=6, outlier_channels=4, config_id=113)
    x, w, parts = _case(wl)
    wp = _gpu_parts(w, parts)
    x_in = to_torch(x, "cuda").clone()
    x_variants = [x_in.clone(), (x_in.float() * 0.5).to(torch.bfloat16), x_in.flip(0).contiguous()]
    B.awq_layer(x_in, wp, n_grid=6)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = B.awq_layer(x_in, wp, n_grid=6)
    for rep in range(2):
        for xv in x_variants:
            want = {k: v.cpu().numpy() for k, v in B.awq_layer(xv, wp, n_grid=6).items()}  # eager
            x_in.copy_(xv)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for key in ("act_mean", "losses", "best_info", "best_scales", "codes", "qscales", "zeros"):
                assert np.array_equal(captured[key].cpu().numpy(), want[key], equal_nan=True), (rep, key)


def test_host_side_errors_do_not_launch(B):
    wl = custom_workload(64, 128, 32, "bf16", n_grid=2, config_id=109)
    x, w, parts = _case(wl)
    xt = to_torch(x, "cuda")
    with pytest.raises(B.AwqError) as e:
        B.awq_search_scales(xt, _gpu_parts(w, parts), torch.zeros(128, dtype=torch.float64, device="cuda"),
                            n_grid=2, group_size=64)
    assert e.value.status == 5
    with pytest.raises(B.AwqError) as e:
        B.awq_act_stats(xt[:0])
    assert e.value.status == 3
