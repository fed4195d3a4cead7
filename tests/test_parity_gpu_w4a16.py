"""GPU parity of the W4A16 consumer (awq_w4a16_gemm) against the CPU oracle (oracle/awq_w4a16.py).

* Exact-arithmetic inputs (small-integer activations, power-of-two float16 steps): every product and
  every partial sum is exact in float32, so the output must equal the oracle bit for bit, whatever
  the summation order — this checks every index, nibble, zero point and step of the dequantization
  and the layout of the matrix-core fragments.
* The real chain (search -> pack -> float16 export -> consumer fed X / s) on workload-shaped inputs:
  |Y - Y_oracle| <= K 2^-24 sum_c |x_c| |w_hat_c| (+ one rounding of the output when it is 16-bit):
  the products of two 16-bit operands are exact in float32 and each of the at most K additions into
  an output rounds once.
The one-token kernel (whole rows per wave, 1 KiB windows, up to 32768 inputs), the few-token kernel
(<= 32 tokens) and both shapes of the many-token kernel (16 rows per wave up to 512 tokens, 64
beyond) are covered, with ragged tokens, rows and group counts."""
import numpy as np
import pytest

from oracle import awq_export as XP
from oracle import awq_oracle as O
from oracle import awq_w4a16 as Q
from workloads import custom_workload, make_w, make_x, to_f32, to_torch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_quantization_mean_amd import binding
    binding.load_library()
    return binding


def _exact_case(rng, n_tokens, d_in, d_out):
    """Activations in [-8, 8] (exact in bf16 and f16), codes and zero points uniform, steps 2^-8..2^-4."""
    g = d_in // 128
    x = rng.integers(-8, 9, (n_tokens, d_in)).astype(np.float64)
    q = rng.integers(0, 16, (d_out, d_in))
    z = rng.integers(0, 16, (d_out, g))
    steps = (2.0 ** rng.integers(-8, -3, (d_out, g))).astype(np.float16)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    zp = np.zeros((d_out, (g + 1) // 2), np.uint8)
    zp |= z[:, 0::2].astype(np.uint8)
    if g > 1:
        zp[:, : g // 2] |= z[:, 1::2].astype(np.uint8) << 4
    return x, codes, steps.view(np.uint16), zp


def _dev(codes, sb, zp):
    return (torch.from_numpy(codes).cuda(), torch.from_numpy(sb.view(np.int16)).cuda(), torch.from_numpy(zp).cuda())


def _x_torch(x, operand):
    dt = torch.bfloat16 if operand == "bf16" else torch.float16
    return torch.from_numpy(np.asarray(x, np.float32)).to(dt).cuda()


def _out_bits(y, operand):
    y = y.cpu()
    if y.dtype == torch.float32:
        return y.numpy().view(np.uint32)
    return y.view(torch.int16).numpy().view(np.uint16)


def _want_bits(yref, out, operand):
    y32 = np.asarray(yref, np.float64).astype(np.float32)
    assert np.array_equal(y32.astype(np.float64), yref)  # the exact-arithmetic case really is exact
    if out == "f32":
        return y32.view(np.uint32)
    if operand == "bf16":
        return XP.f32_to_bf16_rne(y32)
    return y32.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("operand", ["bf16", "f16"])
@pytest.mark.parametrize("out", ["f32", "same"])
@pytest.mark.parametrize("n_tokens,d_in,d_out", [
    (1, 128, 16), (1, 2176, 300), (1, 640, 1), (1, 1920, 8193), (1, 4224, 4097),  # one-token kernel: ragged
    (1, 32768, 40),                                                                # windows and row runs, LDS full
    (1, 32896, 24),                                                                # d_in past its LDS: few-token kernel
    (5, 384, 300), (16, 1152, 272), (17, 256, 40), (32, 640, 33),                  # few-token kernel,
    (5, 256, 8209), (16, 384, 8192), (32, 128, 8200), (2, 640, 12289),            # two row tiles per wave,
    (20, 256, 8209),                                                               # and two token tiles
    (33, 384, 300), (128, 256, 256), (300, 1152, 520), (129, 128, 17),            # many-token kernel,
    (600, 384, 300), (513, 128, 520),                                              # 16 or 64 rows per wave
    (1024, 256, 300), (1300, 384, 520), (2049, 128, 17),                           # several token blocks
])
def test_exact_arithmetic_bit_exact(B, operand, out, n_tokens, d_in, d_out):
    rng = np.random.default_rng(n_tokens * 1000 + d_in + d_out)
    x, codes, sb, zp = _exact_case(rng, n_tokens, d_in, d_out)
    xt = _x_torch(x, operand)
    od = torch.float32 if out == "f32" else xt.dtype
    print(f"[gpu w4a16] exact case tokens={n_tokens} d_in={d_in} d_out={d_out} {operand} out={out}", flush=True)
    y = B.awq_w4a16_gemm(xt, *_dev(codes, sb, zp), out_dtype=od)
    torch.cuda.synchronize()
    yref = Q.w4a16_matmul(x, codes, sb, zp, operand)
    got, want = _out_bits(y, operand), _want_bits(yref, out, operand)
    bad = got != want
    if bad.any():
        i, o = np.argwhere(bad)[0]
        print(f"  {int(bad.sum())} of {bad.size} differ; first ({i},{o}): gpu {y[i, o].item()!r} oracle {yref[i, o]!r}",
              flush=True)
    assert not bad.any()


def test_strided_activations_and_output(B):
    rng = np.random.default_rng(77)
    x, codes, sb, zp = _exact_case(rng, 40, 256, 48)
    xt_full = torch.zeros((40, 264), dtype=torch.bfloat16, device="cuda")
    xt_full[:, :256] = _x_torch(x, "bf16")
    y_full = torch.full((40, 56), -7.0, dtype=torch.float32, device="cuda")
    B.awq_w4a16_gemm(xt_full[:, :256], *_dev(codes, sb, zp), y=y_full[:, :48])
    torch.cuda.synchronize()
    yref = Q.w4a16_matmul(x, codes, sb, zp, "bf16")
    assert np.array_equal(y_full[:, :48].cpu().numpy().astype(np.float64), yref)
    assert torch.all(y_full[:, 48:] == -7.0)  # outside ld_y's used columns nothing is written


def test_strided_operands_tile_kernel(B):
    # 1100 tokens (the 256 x 256 tile kernel), activations and output with row pitches beyond their widths
    rng = np.random.default_rng(78)
    x, codes, sb, zp = _exact_case(rng, 1100, 384, 300)
    xt_full = torch.zeros((1100, 392), dtype=torch.bfloat16, device="cuda")
    xt_full[:, :384] = _x_torch(x, "bf16")
    y_full = torch.full((1100, 320), -7.0, dtype=torch.float32, device="cuda")
    B.awq_w4a16_gemm(xt_full[:, :384], *_dev(codes, sb, zp), y=y_full[:, :300])
    torch.cuda.synchronize()
    yref = Q.w4a16_matmul(x, codes, sb, zp, "bf16")
    assert np.array_equal(y_full[:, :300].cpu().numpy().astype(np.float64), yref)
    assert torch.all(y_full[:, 300:] == -7.0)


def _chain(B, wl, parts, n_tokens_use):
    """search -> pack -> float16 export on the GPU; returns device export + host copies."""
    x, w = make_x(wl), make_w(wl)
    xt = to_torch(x, "cuda")
    wt = to_torch(w, "cuda")
    wp, r = [], 0
    for p in parts:
        wp.append(wt[r:r + p])
        r += p
    act = B.awq_act_stats(xt)
    res = B.awq_search_scales(xt, wp, act, wl.n_grid)
    pk = B.awq_quantize_pack(wp, res["best_scales"])
    ex = B.awq_export_fp16(pk["qscales"], pk["zeros"])
    torch.cuda.synchronize()
    s = res["best_scales"].cpu().numpy()
    # the layer input divided by the scales (the fold into the previous operator), in bf16
    xs = to_f32(x[:n_tokens_use]).astype(np.float64) / s[None, :]
    return xs, pk["codes"], ex["steps_f16"], ex["zeros_u4"]


@pytest.mark.parametrize("n_tokens", [1, 16, 32, 33, 200])
def test_real_chain_within_accumulation_bound(B, n_tokens):
    wl = custom_workload(512, 384, 520, "bf16", n_grid=8, outlier_channels=4, config_id=401)
    xs, codes, sb, zp = _chain(B, wl, (200, 136, 184), n_tokens)
    xt = torch.from_numpy(xs.astype(np.float32)).to(torch.bfloat16).cuda()
    print(f"[gpu w4a16] real chain tokens={n_tokens}", flush=True)
    y = B.awq_w4a16_gemm(xt, codes, sb, zp).cpu().numpy().astype(np.float64)
    xq = xt.float().cpu().numpy().astype(np.float64)
    c, s_, z = codes.cpu().numpy(), sb.cpu().numpy().view(np.uint16), zp.cpu().numpy()
    yref = Q.w4a16_matmul(xq, c, s_, z, "bf16")
    tol = 384 * 2.0 ** -24 * Q.abs_product_sums(xq, c, s_, z, "bf16")
    err = np.abs(y - yref)
    print(f"  max err {err.max():.3e}, max err / bound {(err / np.maximum(tol, 1e-300)).max():.3e}", flush=True)
    assert np.all(err <= tol)


@pytest.mark.parametrize("n_tokens", [1, 16, 4096])
def test_full_size_7b_qkv(B, n_tokens):
    # the bench layer's shape: 12288 x 4096 codes; the oracle checks 48 sampled tokens
    rng = np.random.default_rng(9)
    d_in, d_out = 4096, 12288
    q = rng.integers(0, 16, (d_out, d_in))
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    g = d_in // 128
    sb = (np.abs(rng.normal(0.002, 0.0005, (d_out, g))) + 1e-4).astype(np.float16).view(np.uint16)
    zp = rng.integers(0, 256, (d_out, g // 2)).astype(np.uint8)
    x = rng.standard_normal((n_tokens, d_in)).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16).cuda()
    print(f"[gpu w4a16] full size 12288 x 4096, tokens={n_tokens}", flush=True)
    y = B.awq_w4a16_gemm(xt, *_dev(codes, sb, zp), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([[0, n_tokens - 1], rng.integers(0, n_tokens, 46)]))
    xq = xt.float().cpu().numpy().astype(np.float64)[pick]
    yref = Q.w4a16_matmul(xq, codes, sb, zp, "bf16")
    tol = d_in * 2.0 ** -24 * Q.abs_product_sums(xq, codes, sb, zp, "bf16") + 2.0 ** -8 * np.abs(yref)
    got = y.float().cpu().numpy().astype(np.float64)[pick]
    err = np.abs(got - yref)
    print(f"  max err / bound {(err / tol).max():.3e}", flush=True)
    assert np.all(err <= tol)


@pytest.mark.parametrize("operand,n_tokens", [("bf16", 1), ("f16", 1), ("bf16", 16), ("f16", 7), ("bf16", 27)])
def test_decode_70b_down_proj_shape(B, operand, n_tokens):
    # decode on the 70B down_proj's shape (8192 rows x 28672 inputs, 224 groups = 14 windows per row),
    # one token (whole-row windows) and several (two row tiles per wave; 27 tokens: two token tiles per
    # block): every output against the accumulation bound on 96 sampled rows, all outputs finite
    rng = np.random.default_rng(11 + n_tokens)
    d_in, d_out = 28672, 8192
    g = d_in // 128
    codes = rng.integers(0, 256, (d_out, d_in // 2), dtype=np.uint8)
    sb = (np.abs(rng.normal(0.002, 0.0005, (d_out, g))) + 1e-4).astype(np.float16).view(np.uint16)
    zp = rng.integers(0, 256, (d_out, g // 2)).astype(np.uint8)
    x = rng.standard_normal((n_tokens, d_in)).astype(np.float32)
    xt = _x_torch(x, operand)
    print(f"[gpu w4a16] {n_tokens} tokens, 8192 x 28672, {operand}", flush=True)
    y = B.awq_w4a16_gemm(xt, *_dev(codes, sb, zp), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    rows = np.unique(np.concatenate([[0, 1, d_out - 1], rng.integers(0, d_out, 93)]))
    xq = xt.float().cpu().numpy().astype(np.float64)
    yref = Q.w4a16_matmul(xq, codes[rows], sb[rows], zp[rows], operand)
    tol = d_in * 2.0 ** -24 * Q.abs_product_sums(xq, codes[rows], sb[rows], zp[rows], operand)
    err = np.abs(got[:, rows] - yref)
    print(f"  max err / bound {(err / tol).max():.3e}", flush=True)
    assert np.all(err <= tol)


@pytest.mark.parametrize("n_tokens,d_in,d_out", [(1, 640, 300), (5, 384, 8200), (1100, 256, 300)])
def test_nonfinite_activations(B, n_tokens, d_in, d_out):
    # a NaN, +inf and -inf at one input each of three tokens (one token: the -inf alone): those
    # tokens' outputs are NaN or +-inf
    # (inf times a zero weight is NaN, otherwise the one infinite term decides the sign), the same
    # pattern as the float64 oracle whatever the order of the additions; the other tokens are finite
    rng = np.random.default_rng(n_tokens + d_out)
    x, codes, sb, zp = _exact_case(rng, n_tokens, d_in, d_out)
    bad = {0: np.nan, n_tokens // 2: np.inf, n_tokens - 1: -np.inf}
    for t, v in bad.items():
        x[t, 7 + 3 * t % (d_in - 8)] = v
    xt = _x_torch(x, "bf16")
    print(f"[gpu w4a16] non-finite activations, tokens={n_tokens} d_in={d_in} d_out={d_out}", flush=True)
    y = B.awq_w4a16_gemm(xt, *_dev(codes, sb, zp), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    with np.errstate(invalid="ignore"):
        want = Q.w4a16_matmul(x, codes, sb, zp, "bf16")
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(want) & (want > 0))
    assert np.array_equal(np.isinf(got) & (got < 0), np.isinf(want) & (want < 0))
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])  # exact-arithmetic inputs elsewhere
