"""Pins of the CPU oracle: checks that tie it to what the pages and the
mathematics fix, independent of the oracle's own code.  Each ``pin_*`` raises
AssertionError when the oracle is wrong.  They look oracle functions up on the
module at call time, so a mutation test can plant a mistake in the oracle and
see which pins catch it."""

import json
import math
import os

import numpy as np

import brute
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _rows(rng, n, h, d, spread=True):
    x = rng.standard_normal((n, h, d))
    if spread:  # per-row scales over several decades, as the workloads draw them
        x *= np.exp(rng.uniform(np.log(1e-3), np.log(30.0), size=(n, h, 1)))
    return x


def _gamma(rng, d):
    return 1.0 + 0.1 * rng.standard_normal(d)


# ---------------------------------------------------------------- QK-Norm

def pin_rms_closed_form():
    """rms(x_hat / gamma) = sqrt(ms / (ms + eps)) for every row; a zero row maps to 0."""
    rng = _rng(1)
    x = _rows(rng, 40, 4, 128)
    x[3, 2] = 0.0
    g = _gamma(rng, 128)
    eps = 1e-6
    y = A.rms_norm_heads(x, g, eps)
    ms = np.mean(x * x, axis=-1)
    got = np.sqrt(np.mean((y / g) ** 2, axis=-1))
    want = np.sqrt(ms / (ms + eps))
    assert np.allclose(got, want, rtol=1e-12, atol=0), "per-row RMS after norm"
    assert np.all(y[3, 2] == 0.0), "zero row"
    # eps must matter for tiny rows: ms = 1e-8 gives rms 0.00995, not 1
    tiny = np.full((1, 1, 128), 1e-4)
    r = np.sqrt(np.mean(A.rms_norm_heads(tiny, np.ones(128), eps) ** 2))
    assert abs(r - math.sqrt(1e-8 / (1e-8 + eps))) < 1e-12, "eps inside the root"


def pin_rms_l2_norm():
    """[OZ] §20.1: with gamma = 1 the L2 norm of a normed head is sqrt(d * ms / (ms + eps)) ~ sqrt(d)."""
    gd = golden("rmsnorm_l2.json")
    rng = _rng(2)
    x = _rows(rng, 20, 3, 128, spread=False) * 5.0
    y = A.rms_norm_heads(x, np.ones(128), 1e-6)
    ms = np.mean(x * x, axis=-1)
    want = np.sqrt(128 * ms / (ms + 1e-6))
    assert np.allclose(np.linalg.norm(y, axis=-1), want, rtol=1e-12)
    assert abs(np.sqrt(128) - gd["sqrt_d"]) < 1e-15
    assert np.allclose(np.linalg.norm(y, axis=-1), gd["sqrt_d"], rtol=1e-6)


def pin_rms_scale_invariance():
    """x_hat(c x) = x / sqrt(ms + eps / c^2) * gamma: QK-Norm removes a head's scale."""
    rng = _rng(3)
    x = _rows(rng, 16, 2, 128, spread=False)
    g = _gamma(rng, 128)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    for c in (0.1, 30.0):
        got = A.rms_norm_heads(c * x, g, 1e-6)
        want = x / np.sqrt(ms + 1e-6 / c ** 2) * g
        assert np.allclose(got, want, rtol=1e-12, atol=1e-15)


def pin_norm_axis_per_head():
    """[OZ] §20.1 / [NW]: the norm runs over each head's own d; scaling one head leaves others alone."""
    rng = _rng(4)
    x = _rows(rng, 4, 4, 128, spread=False)
    g = _gamma(rng, 128)
    y0 = A.rms_norm_heads(x, g, 1e-6)
    x2 = x.copy()
    x2[:, 1] *= 100.0
    y1 = A.rms_norm_heads(x2, g, 1e-6)
    assert np.array_equal(y0[:, [0, 2, 3]], y1[:, [0, 2, 3]]), "other heads unchanged"


# ---------------------------------------------------------------- RoPE

def pin_rope_closed_values():
    """Pair 0 at position 1 turns by exactly 1 rad (omega_0 = 1): e_0 -> (cos 1, sin 1) on
    dims (0, 64) and e_64 -> (-sin 1, cos 1); omega_63 = theta^(-126/128)."""
    gd = golden("rope_closed_values.json")
    d = gd["head_dim"]
    e0 = np.zeros((1, 1, d)); e0[0, 0, 0] = 1.0
    e64 = np.zeros((1, 1, d)); e64[0, 0, 64] = 1.0
    y = A.rope_rotate_half(e0, [1], 1e6)[0, 0]
    assert abs(y[0] - gd["cos_1"]) < 1e-16 and abs(y[64] - gd["sin_1"]) < 1e-16
    assert np.count_nonzero(y) == 2
    y = A.rope_rotate_half(e64, [1], 1e6)[0, 0]
    assert abs(y[0] + gd["sin_1"]) < 1e-16 and abs(y[64] - gd["cos_1"]) < 1e-16
    for th, key in ((1e6, "1e6"), (1e7, "1e7")):
        w = A.rope_inv_freq(d, th)
        assert w[0] == gd["omega_0"]
        assert abs(w[63] - gd["omega_63"][key]) <= 1e-15 * gd["omega_63"][key] * 4
    # the last pair (63, 127) at position p turns by p * omega_63
    e63 = np.zeros((1, 1, d)); e63[0, 0, 63] = 1.0
    p = 4000
    y = A.rope_rotate_half(e63, [p], 1e6)[0, 0]
    ang = p * gd["omega_63"]["1e6"]
    assert abs(y[63] - math.cos(ang)) < 1e-15 and abs(y[127] - math.sin(ang)) < 1e-15


def pin_rope_pair_norm():
    """Each rotated pair keeps its length: y_i^2 + y_{i+64}^2 = x_i^2 + x_{i+64}^2."""
    rng = _rng(5)
    x = _rows(rng, 64, 3, 128, spread=False)
    pos = rng.integers(0, 40000, size=64)
    y = A.rope_rotate_half(x, pos, 1e6)
    a = x[..., :64] ** 2 + x[..., 64:] ** 2
    b = y[..., :64] ** 2 + y[..., 64:] ** 2
    assert np.allclose(a, b, rtol=1e-13, atol=0)


def pin_rope_position_zero():
    """Position 0 is the identity, exactly."""
    rng = _rng(6)
    x = _rows(rng, 5, 2, 128)
    y = A.rope_rotate_half(x, np.zeros(5, dtype=np.int64), 1e6)
    assert np.array_equal(x, y)


def pin_rope_shift_invariance():
    """<R(m+c) q, R(n+c) k> = <R(m) q, R(n) k>: scores depend only on m - n."""
    rng = _rng(7)
    q = _rows(rng, 8, 1, 128, spread=False)
    k = _rows(rng, 8, 1, 128, spread=False)
    m = rng.integers(0, 500, size=8)
    n = rng.integers(0, 500, size=8)
    for c in (1, 37, 1000):
        s0 = np.einsum("ihd,ihd->ih", A.rope_rotate_half(q, m, 1e6), A.rope_rotate_half(k, n, 1e6))
        s1 = np.einsum("ihd,ihd->ih", A.rope_rotate_half(q, m + c, 1e6), A.rope_rotate_half(k, n + c, 1e6))
        assert np.allclose(s0, s1, rtol=0, atol=1e-10)


# ---------------------------------------------------------------- order

def pin_order_demo():
    """Norm then RoPE vs RoPE then norm: equal when gamma is pair-symmetric
    (gamma_i = gamma_{i+64}, e.g. gamma = 1), different for a general gamma."""
    rng = _rng(8)
    x = _rows(rng, 16, 2, 128)
    pos = np.arange(16)
    g = _gamma(rng, 128)
    gs = np.concatenate([g[:64], g[:64]])
    a = A.qk_norm_rope(x, gs, pos, 1e-6, 1e6, "norm_rope")
    b = A.qk_norm_rope(x, gs, pos, 1e-6, 1e6, "rope_norm")
    assert np.max(np.abs(a - b)) < 1e-12, "orders agree for pair-symmetric gamma"
    a = A.qk_norm_rope(x, g, pos, 1e-6, 1e6, "norm_rope")
    b = A.qk_norm_rope(x, g, pos, 1e-6, 1e6, "rope_norm")
    assert np.max(np.abs(a - b)) > 1e-2, "orders differ for a general gamma"
    # and the default (norm -> RoPE) equals normalising first, then rotating
    want = A.rope_rotate_half(A.rms_norm_heads(x, g, 1e-6), pos, 1e6)
    got = A.qk_norm_rope(x, g, pos, 1e-6, 1e6)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- attention

def _case(seed, lengths, hq, hkv, d=128, vscale=1.0):
    rng = _rng(seed)
    n = sum(lengths)
    q = _rows(rng, n, hq, d)
    k = _rows(rng, n, hkv, d)
    v = rng.standard_normal((n, hkv, d)) * vscale
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, k, v, _gamma(rng, d), _gamma(rng, d), cu


def pin_softmax_rows():
    """Causal softmax rows sum to 1 and are exactly 0 above the diagonal."""
    rng = _rng(9)
    s = rng.standard_normal((30, 30)) * 8
    p = A.causal_softmax(s, np.arange(30), np.arange(30))
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(p[np.triu_indices(30, 1)] == 0.0)
    assert np.all(p[np.tril_indices(30)] > 0.0)
    # rectangular: queries at positions 5..7 over keys 0..7
    p = A.causal_softmax(rng.standard_normal((3, 8)), np.arange(5, 8), np.arange(8))
    assert np.all(p[0, 6:] == 0) and np.all(p[1, 7:] == 0) and np.all(p[2] > 0)


def pin_first_row_is_v0():
    """The first token of every packed sequence sees one key: o_0 = v_0 of its KV head, exactly."""
    lengths = [5, 1, 7]
    q, k, v, gq, gk, cu = _case(10, lengths, 4, 2)
    o = A.attention_prefill(q, k, v, gq, gk, cu, 4, 2)
    for s in range(3):
        for t in range(4):
            assert np.array_equal(o[cu[s], t], v[cu[s], t // 2])


def pin_gqa_head_map():
    """[QA] §2.2 worked example (32/8: heads 1-4 -> group 1, 5-8 -> group 2), and in the
    attention: changing KV head u changes exactly query heads u*g .. u*g+g-1."""
    gd = golden("gqa_head_groups.json")
    for t1, u1 in gd["one_based_examples"]:
        assert A.kv_head_for_q_head(t1 - 1, gd["n_q_heads"], gd["n_kv_heads"]) + 1 == u1
    lengths = [6]
    q, k, v, gq, gk, cu = _case(11, lengths, 8, 2)
    o0 = A.attention_prefill(q, k, v, gq, gk, cu, 8, 2)
    v2 = v.copy()
    v2[:, 1] += 1.0
    o1 = A.attention_prefill(q, k, v2, gq, gk, cu, 8, 2)
    changed = [t for t in range(8) if not np.array_equal(o0[:, t], o1[:, t])]
    assert changed == [4, 5, 6, 7], changed


def pin_gqa_equals_mha_on_repeated_kv():
    """[XW] §7.2.1: GQA equals MHA after repeat-interleaving K and V g times; g = Hq is MQA."""
    lengths = [4, 9]
    q, k, v, gq, gk, cu = _case(12, lengths, 8, 2)
    o_gqa = A.attention_prefill(q, k, v, gq, gk, cu, 8, 2)
    o_mha = A.attention_prefill(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), gq, gk, cu, 8, 8)
    assert np.max(np.abs(o_gqa - o_mha)) < 1e-13
    o_mqa = A.attention_prefill(q, k[:, :1], v[:, :1], gq, gk, cu, 8, 1)
    o_rep = A.attention_prefill(q, np.repeat(k[:, :1], 8, axis=1), np.repeat(v[:, :1], 8, axis=1),
                                gq, gk, cu, 8, 8)
    assert np.max(np.abs(o_mqa - o_rep)) < 1e-13


def pin_brute_force(d=8):
    """Scalar loops (tests/brute.py) on two ragged sequences equal the vectorised oracle."""
    lengths = [3, 6]
    q, k, v, gq, gk, cu = _case(13 + d, lengths, 4, 2, d=d, vscale=3.0)
    o = A.attention_prefill(q, k, v, gq, gk, cu, 4, 2, eps=1e-6, theta=1e6)
    b = np.array(brute.prefill(q.tolist(), k.tolist(), v.tolist(), gq.tolist(), gk.tolist(),
                               lengths, 4, 2, 1e-6, 1e6))
    assert np.max(np.abs(o - b)) < 1e-12, np.max(np.abs(o - b))


def pin_causality():
    """[OZ] §20.8: changing future tokens leaves earlier outputs unchanged (difference exactly 0)."""
    gd = golden("cache_protocol.json")
    lengths = [12]
    q, k, v, gq, gk, cu = _case(14, lengths, 4, 2)
    o0 = A.attention_prefill(q, k, v, gq, gk, cu, 4, 2)
    i = 6
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[i + 1:] += 3.0
    k2[i + 1:] *= -2.0
    v2[i + 1:] += 5.0
    o1 = A.attention_prefill(q2, k2, v2, gq, gk, cu, 4, 2)
    assert float(np.max(np.abs(o0[:i + 1] - o1[:i + 1]))) == gd["future_token_change_past_diff"]
    assert np.max(np.abs(o0[i + 1:] - o1[i + 1:])) > 0.1


def pin_packing_invariance():
    """A sequence gives the same output alone or packed with others (no cross-sequence attention,
    positions restart at 0)."""
    lengths = [7, 5, 9]
    q, k, v, gq, gk, cu = _case(15, lengths, 4, 2)
    o = A.attention_prefill(q, k, v, gq, gk, cu, 4, 2)
    a, b = cu[1], cu[2]
    o1 = A.attention_prefill(q[a:b], k[a:b], v[a:b], gq, gk, np.array([0, b - a]), 4, 2)
    assert np.array_equal(o[a:b], o1)


def pin_decode_is_last_prefill_row():
    """One decode step over a cache of L rotated keys equals row L of a prefill over L + 1 tokens."""
    L = 9
    q, k, v, gq, gk, cu = _case(16, [L + 1], 8, 2)
    o = A.attention_prefill(q, k, v, gq, gk, cu, 8, 2)
    k_hat_cache = A.qk_norm_rope(k[:L], gk, np.arange(L), 1e-6, 1e6)
    od = A.attention_decode(q[L:], k[L:], v[L:], gq, gk, [k_hat_cache], [v[:L]], [L], 8, 2)
    assert np.max(np.abs(od[0] - o[L])) < 1e-12


def pin_chunked_append():
    """[OZ] §20.9: appending [0:2], [2:5], [5:6] against the cache equals one full pass."""
    gd = golden("cache_protocol.json")
    q, k, v, gq, gk, cu = _case(17, [6], 4, 2)
    full = A.attention_prefill(q, k, v, gq, gk, cu, 4, 2)
    kc = np.zeros((0, 2, 128))
    vc = np.zeros((0, 2, 128))
    outs = []
    for a, b in gd["chunks"]:
        o, kh = A.attention_append(q[a:b], k[a:b], v[a:b], gq, gk, kc, vc, a, 4, 2)
        outs.append(o)
        kc = np.concatenate([kc, kh])
        vc = np.concatenate([vc, v[a:b]])
    assert np.max(np.abs(np.concatenate(outs) - full)) < 1e-12
    assert kc.shape[0] == 6


def pin_uniform_scores_prefix_mean():
    """All-zero query heads normalise to 0 (eps avoids 0/0), every score is 0, and each output
    row is the plain mean of v_0 .. v_i."""
    q, k, v, gq, gk, cu = _case(18, [10], 4, 2)
    q[:] = 0.0
    o = A.attention_prefill(q, k, v, gq, gk, cu, 4, 2)
    for t in range(4):
        pm = np.cumsum(v[:, t // 2], axis=0) / np.arange(1, 11)[:, None]
        assert np.max(np.abs(o[:, t] - pm)) < 1e-13


def pin_sdpa_cross_check():
    """A textbook library routine: torch's CPU scaled_dot_product_attention in float64 with
    is_causal on the oracle's normed+rotated Q/K and repeat-interleaved K/V."""
    import torch
    lengths = [33]
    q, k, v, gq, gk, cu = _case(19, lengths, 8, 2, vscale=10.0)
    o = A.attention_prefill(q, k, v, gq, gk, cu, 8, 2)
    pos = np.arange(33)
    qh = torch.from_numpy(A.qk_norm_rope(q, gq, pos, 1e-6, 1e6)).permute(1, 0, 2)
    kh = torch.from_numpy(A.qk_norm_rope(k, gk, pos, 1e-6, 1e6)).permute(1, 0, 2)
    vv = torch.from_numpy(v).permute(1, 0, 2)
    kh = kh.repeat_interleave(4, dim=0).contiguous()
    vv = vv.repeat_interleave(4, dim=0).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qh.contiguous(), kh, vv, is_causal=True)
    assert np.max(np.abs(ref.permute(1, 0, 2).numpy() - o)) < 1e-12


def pin_rows_api_matches_full():
    """The sampled-row entry point equals the full prefill rows it samples."""
    q, k, v, gq, gk, cu = _case(20, [40], 8, 2)
    o = A.attention_prefill(q, k, v, gq, gk, cu, 8, 2)
    rows = np.array([0, 17, 39])
    r = A.attention_prefill_rows(q[rows], k, v, gq, gk, rows, [1, 6], 8, 2)
    assert np.max(np.abs(r - o[rows][:, [1, 6]])) < 1e-13


ALL_PINS = [
    pin_rms_closed_form, pin_rms_l2_norm, pin_rms_scale_invariance, pin_norm_axis_per_head,
    pin_rope_closed_values, pin_rope_pair_norm, pin_rope_position_zero, pin_rope_shift_invariance,
    pin_order_demo, pin_softmax_rows, pin_first_row_is_v0, pin_gqa_head_map,
    pin_gqa_equals_mha_on_repeated_kv, pin_brute_force, pin_causality, pin_packing_invariance,
    pin_decode_is_last_prefill_row, pin_chunked_append, pin_uniform_scores_prefix_mean,
    pin_sdpa_cross_check, pin_rows_api_matches_full,
]
