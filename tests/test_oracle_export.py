"""Pins for the oracle of the steps either side of the search (statistic over batches, source
fold, deployment form), from hand-worked values and identities of the pages (CPU only)."""
import numpy as np
import pytest

from oracle import awq_export as X
from oracle import awq_oracle as O


def test_statistic_over_batches_hand_values():
    # |X| over three tokens in two batches: channel 0 = (1 + 3 + 5) / 3, channel 1 = (2 + 4 + 6) / 3
    b1 = np.array([[1.0, -2.0], [3.0, 4.0]])
    b2 = np.array([[-5.0, 6.0]])
    assert np.array_equal(X.act_sums(b1), [4.0, 6.0])
    assert np.array_equal(X.act_mean_batches([b1, b2]), [3.0, 4.0])


def test_statistic_does_not_depend_on_the_split():
    rng = np.random.default_rng(3)
    x = np.round(rng.standard_normal((97, 5)) * 64) / 64  # exact binary fractions: exact sums
    whole = X.act_mean_batches([x])
    for cuts in ([10, 50], [1, 2, 3, 96], [48]):
        parts = np.split(x, cuts)
        assert np.array_equal(X.act_mean_batches(parts), whole)
    assert np.array_equal(whole, np.abs(x).sum(axis=0) / 97)
    with pytest.raises(ValueError):
        X.act_mean_batches([])


def test_fold_hand_values_and_direction():
    src = np.array([[1.0, 2.0], [3.0, 6.0]])
    assert np.array_equal(X.fold_scales(src, [2.0, 3.0], "f32"), np.array([[0.5, 1.0], [1.0, 2.0]], np.float32))
    # a vector (a norm weight) is one column
    assert np.array_equal(X.fold_scales(np.array([4.0, 9.0]), [2.0, 3.0], "f32")[:, 0], [2.0, 3.0])


def test_fold_bf16_rounding_hand_values():
    # 1/3 in float32 is 0x3EAAAAAB -> low half 0xAAAB above the midpoint -> 0x3EAB
    assert X.fold_scales(np.array([[1.0]]), [3.0], "bf16")[0, 0] == 0x3EAB
    # exact ties go to the even neighbour: 0x3F808000 -> 0x3F80, 0x3F818000 -> 0x3F82
    assert X.fold_scales(np.array([[1.00390625]]), [1.0], "bf16")[0, 0] == 0x3F80
    assert X.fold_scales(np.array([[1.01171875]]), [1.0], "bf16")[0, 0] == 0x3F82
    # overflow to infinity, NaN stays NaN
    assert X.fold_scales(np.array([[3.0e38]]), [1e-3], "bf16")[0, 0] == 0x7F80
    assert (X.fold_scales(np.array([[np.nan]]), [1.0], "bf16")[0, 0] & 0x7FC0) == 0x7FC0


def test_fold_keeps_the_layer_output():
    # gsyq section 四: (x * gamma) W^T == (x * gamma / s) (W * s)^T; the fold must divide the source
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 16))
    gamma = rng.uniform(0.5, 2.0, 16)
    W = rng.standard_normal((9, 16))
    s = rng.uniform(0.1, 10.0, 16)
    ref = (x * gamma) @ W.T
    g2 = X.fold_scales(gamma, s, "f32")[:, 0].astype(np.float64)
    got = (x * g2) @ (W * s).T
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-6)
    wrong = (x * gamma * s) @ (W * s).T
    assert not np.allclose(wrong, ref, rtol=1e-2)
    # the source linear of linear-linear / up-down: its output rows are divided
    W1 = rng.standard_normal((16, 11))
    h = rng.standard_normal((3, 11))
    ref2 = (h @ W1.T) @ W.T
    got2 = (h @ X.fold_scales(W1, s, "f32").astype(np.float64).T) @ (W * s).T
    assert np.allclose(got2, ref2, rtol=1e-5, atol=1e-5)


def test_export_fp16_hand_values():
    qs = np.array([[0.1, 1e-5, 70000.0, 0.5]], np.float32)
    zeros = np.array([[3, 16, -1, 15]])
    hb, packed, bad_z, bad_s = X.export_fp16(qs, zeros)
    assert list(hb[0]) == [0x2E66, 0x00A8, 0x7C00, 0x3800]
    assert list(packed[0]) == [0x03 | (0x0F << 4), 0x00 | (0x0F << 4)]
    assert bad_z == 2 and bad_s == 2
    hb, packed, bad_z, bad_s = X.export_fp16(np.ones((1, 3), np.float32), np.array([[1, 2, 3]]))
    assert list(packed[0]) == [0x21, 0x03] and bad_z == 0 and bad_s == 0


def test_export_of_an_oracle_pack_unpacks_to_its_codes_parameters():
    rng = np.random.default_rng(9)
    W = rng.standard_normal((4, 256)) * 0.02
    pq = O.quantize_pack(W, np.ones(256), 128)
    hb, packed, bad_z, bad_s = X.export_fp16(pq.qscales.astype(np.float32), pq.zeros)
    assert bad_z == 0 and bad_s == 0
    lo, hi = packed & 0xF, packed >> 4
    assert np.array_equal(np.stack([lo, hi], -1).reshape(4, -1)[:, :2], pq.zeros)
    assert np.allclose(hb.view(np.float16).astype(np.float64), pq.qscales, rtol=2.0 ** -11)


# ------------------------------------------------------------------ output-value subgraph, grouped KV heads

def _attention(x, wq, wk, wv, wo, n_heads, n_kv, hd):
    """Causal multi-head attention with grouped KV heads in float64: query head h reads KV head
    h // (n_heads / n_kv) (consecutive query heads share a KV head); output x_attn W_o^T."""
    T = x.shape[0]
    g = n_heads // n_kv
    q = (x @ wq.T).reshape(T, n_heads, hd)
    k = (x @ wk.T).reshape(T, n_kv, hd)
    v = (x @ wv.T).reshape(T, n_kv, hd)
    out = np.empty((T, n_heads, hd))
    mask = np.tril(np.ones((T, T), dtype=bool))
    for h in range(n_heads):
        kv = h // g
        sc = q[:, h, :] @ k[:, kv, :].T / np.sqrt(hd)
        sc = np.where(mask, sc, -np.inf)
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, kv, :]
    return out.reshape(T, n_heads * hd), out.reshape(T, n_heads * hd) @ wo.T


@pytest.mark.parametrize("n_heads,n_kv", [(4, 4), (4, 2), (6, 3), (4, 1), (8, 2)])
def test_ov_fold_keeps_the_attention_output(n_heads, n_kv):
    """v_proj rows divided by the group scales and o_proj columns multiplied by the tied scales give
    the same block output (the identity of gsyq section 一 through the attention mix), for MHA,
    GQA and MQA; this fixes which query heads share a KV head's scale."""
    rng = np.random.default_rng(n_heads * 10 + n_kv)
    hd, d_model, T = 8, 16, 7
    wq = rng.standard_normal((n_heads * hd, d_model)) * 0.3
    wk = rng.standard_normal((n_kv * hd, d_model)) * 0.3
    wv = rng.standard_normal((n_kv * hd, d_model)) * 0.3
    wo = rng.standard_normal((d_model, n_heads * hd)) * 0.3
    x = rng.standard_normal((T, d_model))
    xo, y = _attention(x, wq, wk, wv, wo, n_heads, n_kv, hd)
    a = np.abs(xo).mean(axis=0)
    s = O.candidate_scales(X.tie_heads(a, n_heads, n_kv, hd), 0.5)
    t = X.head_group_scales(s, n_heads, n_kv, hd)
    assert t.shape == (n_kv * hd,)
    _, y2 = _attention(x, wq, wk, wv / t[:, None], wo * s[None, :], n_heads, n_kv, hd)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-12)
    if n_kv < n_heads:
        # untied scales (each query head its own) cannot be folded into the shared value rows
        s_untied = O.candidate_scales(a, 0.5)
        t_untied = X.head_group_scales(s_untied, n_heads, n_kv, hd)
        _, y3 = _attention(x, wq, wk, wv / t_untied[:, None], wo * s_untied[None, :], n_heads, n_kv, hd)
        assert np.max(np.abs(y3 - y)) > 1e-6


def test_tie_heads_hand_values():
    # 4 query heads, 2 KV heads, head_dim 2: heads (0, 1) share KV head 0, (2, 3) share KV head 1
    a = np.array([1.0, 2.0, 3.0, 6.0, 10.0, 20.0, 30.0, 60.0])
    assert X.tie_heads(a, 4, 2, 2).tolist() == [2.0, 4.0, 2.0, 4.0, 20.0, 40.0, 20.0, 40.0]
    assert X.head_group_scales(X.tie_heads(a, 4, 2, 2), 4, 2, 2).tolist() == [2.0, 4.0, 20.0, 40.0]
    # MHA: the identity; MQA: every head takes the mean over all heads
    assert np.array_equal(X.tie_heads(a, 4, 4, 2), a)
    assert X.tie_heads(a, 4, 1, 2).tolist() == [11.0, 22.0] * 4
    with pytest.raises(ValueError):
        X.tie_heads(a, 4, 3, 2)


def test_tied_search_reduces_to_the_main_search_for_mha():
    rng = np.random.default_rng(21)
    Xa = rng.standard_normal((40, 256))
    Xa[:, 7] *= 40.0
    W = rng.standard_normal((16, 256)) * 0.02
    r1 = X.search_scales_tied(Xa, W, 2, 2, 128, 128, 6)
    r0 = O.search_scales(Xa, W, 128, 6)
    np.testing.assert_array_equal(r1.scales, r0.scales)
    np.testing.assert_allclose(r1.losses, r0.losses, rtol=1e-12)
    assert r1.best_k == r0.best_k
    # with two query heads per KV head the chosen scales are equal across each group
    r2 = X.search_scales_tied(Xa, W, 2, 1, 128, 128, 6)
    assert np.array_equal(r2.best_scales[:128], r2.best_scales[128:])
