"""Pins of the oracle's attention sublayer (projections around the core):
scalar brute force, identity weights that reduce it to the core, the head
order of the concatenation, the page's head_dim-128 scale at the 0.6B shape,
the cache protocol through the projections, and the sampled-row entry.  Like
``pins.py``, they look the oracle up at call time so that mutation tests can
plant a mistake and see which pin catches it."""

import numpy as np

import brute
import pins
from oracle import attention as A
from oracle import layer as Y


def _layer_case(seed, lengths, hidden, hq, hkv, d):
    rng = np.random.default_rng(seed)
    n = sum(lengths)
    x = rng.standard_normal((n, hidden))
    w_q = rng.standard_normal((hq * d, hidden)) / np.sqrt(hidden)
    w_k = rng.standard_normal((hkv * d, hidden)) / np.sqrt(hidden)
    w_v = rng.standard_normal((hkv * d, hidden)) / np.sqrt(hidden)
    w_o = rng.standard_normal((hidden, hq * d)) / np.sqrt(hq * d)
    gq = 1.0 + 0.1 * rng.standard_normal(d)
    gk = 1.0 + 0.1 * rng.standard_normal(d)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return x, w_q, w_k, w_v, w_o, gq, gk, cu


def pin_linear_brute():
    """y = x W^T for W [out, in], against scalar loops (out != in, so a transposed
    W cannot pass)."""
    rng = np.random.default_rng(40)
    x = rng.standard_normal((5, 7))
    w = rng.standard_normal((3, 7))
    b = np.array(brute.linear(x.tolist(), w.tolist()))
    assert np.max(np.abs(Y.linear(x, w) - b)) < 1e-12


def pin_layer_brute():
    """The whole sublayer against scalar loops (two ragged sequences, GQA)."""
    lengths = [3, 4]
    x, w_q, w_k, w_v, w_o, gq, gk, cu = _layer_case(41, lengths, 12, 4, 2, 8)
    y = Y.attention_layer_prefill(x, w_q, w_k, w_v, w_o, gq, gk, cu, 4, 2, head_dim=8, eps=1e-6, theta=1e6)
    b = np.array(brute.layer_prefill(x.tolist(), w_q.tolist(), w_k.tolist(), w_v.tolist(), w_o.tolist(),
                                     gq.tolist(), gk.tolist(), lengths, 4, 2, 8, 1e-6, 1e6))
    assert y.shape == (7, 12)
    assert np.max(np.abs(y - b)) < 1e-12, np.max(np.abs(y - b))


def pin_layer_identity():
    """hidden = Hq d, W_q = W_o = I and W_k, W_v picking feature blocks: the
    sublayer is the core applied to x viewed as heads."""
    hq, hkv, d = 4, 2, 8
    lengths = [5, 3]
    rng = np.random.default_rng(42)
    n = sum(lengths)
    x = rng.standard_normal((n, hq * d))
    eye = np.eye(hq * d)
    w_k = eye[:hkv * d]            # k = the first Hkv heads' features of x
    w_v = eye[hq * d - hkv * d:]   # v = the last Hkv heads' features of x
    gq = 1.0 + 0.1 * rng.standard_normal(d)
    gk = 1.0 + 0.1 * rng.standard_normal(d)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    y = Y.attention_layer_prefill(x, eye, w_k, w_v, eye, gq, gk, cu, hq, hkv, head_dim=d)
    xh = x.reshape(n, hq, d)
    o = A.attention_prefill(xh, xh[:, :hkv], xh[:, hq - hkv:], gq, gk, cu, hq, hkv)
    assert np.max(np.abs(y - o.reshape(n, hq * d))) < 1e-13


def pin_head_order_of_concat():
    """With W_o zero outside the column block of head t, y depends on head t's
    output only: y = o_t W_o[:, t d:(t+1) d]^T."""
    hq, hkv, d, hidden = 4, 2, 8, 12
    x, w_q, w_k, w_v, w_o, gq, gk, cu = _layer_case(43, [6], hidden, hq, hkv, d)
    t = 2
    w_sel = np.zeros_like(w_o)
    w_sel[:, t * d:(t + 1) * d] = w_o[:, t * d:(t + 1) * d]
    y = Y.attention_layer_prefill(x, w_q, w_k, w_v, w_sel, gq, gk, cu, hq, hkv, head_dim=d)
    q = (x @ w_q.T).reshape(6, hq, d)
    k = (x @ w_k.T).reshape(6, hkv, d)
    v = (x @ w_v.T).reshape(6, hkv, d)
    o = A.attention_prefill(q, k, v, gq, gk, cu, hq, hkv)
    assert np.max(np.abs(y - o[:, t] @ w_o[:, t * d:(t + 1) * d].T)) < 1e-13


def pin_scale_uses_head_dim():
    """The 0.6B shape of the page: emb 1024, 16 heads, head_dim 128 -> a
    2048-wide query projection and the scale 1/sqrt(128), not
    1/sqrt(1024 / 16).  Checked on that head geometry (hidden 1024) with two
    tokens; raising the scores' scale changes the result."""
    gd = pins.golden("layer_shapes.json")["qwen3_0p6b"]
    hidden, hq, hkv, d = gd["hidden"], gd["n_q_heads"], gd["n_kv_heads"], gd["head_dim"]
    x, w_q, w_k, w_v, w_o, gq, gk, cu = _layer_case(44, [2], hidden, hq, hkv, d)
    assert (x @ w_q.T).shape[1] == gd["q_width"]
    y = Y.attention_layer_prefill(x, w_q, w_k, w_v, w_o, gq, gk, cu, hq, hkv, head_dim=d)
    y_fixed = Y.attention_layer_prefill(x, w_q, w_k, w_v, w_o, gq, gk, cu, hq, hkv, head_dim=d,
                                        scale=1.0 / np.sqrt(gd["scale_head_dim"]))
    y_emb = Y.attention_layer_prefill(x, w_q, w_k, w_v, w_o, gq, gk, cu, hq, hkv, head_dim=d,
                                      scale=1.0 / np.sqrt(hidden / hq))
    assert np.max(np.abs(y - y_fixed)) < 1e-14
    assert np.max(np.abs(y - y_emb)) > 1e-6


def pin_layer_chunked_append():
    """Appending [0:2], [2:5], [5:6] through the sublayer against the cache
    equals one pass ("第 20 章" §20.9 protocol, with the projections)."""
    gd = pins.golden("cache_protocol.json")
    x, w_q, w_k, w_v, w_o, gq, gk, cu = _layer_case(45, [6], 16, 4, 2, 8)
    full = Y.attention_layer_prefill(x, w_q, w_k, w_v, w_o, gq, gk, cu, 4, 2, head_dim=8)
    kc, vc, outs = np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), []
    for a, b in gd["chunks"]:
        y, kh, v = Y.attention_layer_append(x[a:b], w_q, w_k, w_v, w_o, gq, gk, kc, vc, a, 4, 2, head_dim=8)
        outs.append(y)
        kc, vc = np.concatenate([kc, kh]), np.concatenate([vc, v])
    assert np.max(np.abs(np.concatenate(outs) - full)) < 1e-12


def pin_layer_rows_api_matches_full():
    """The sampled-row entry point equals the full sublayer rows it samples."""
    x, w_q, w_k, w_v, w_o, gq, gk, cu = _layer_case(46, [30], 16, 4, 2, 8)
    y = Y.attention_layer_prefill(x, w_q, w_k, w_v, w_o, gq, gk, cu, 4, 2, head_dim=8)
    rows = np.array([0, 11, 29])
    r = Y.attention_layer_prefill_rows(x, w_q, w_k, w_v, w_o, gq, gk, rows, 4, 2, head_dim=8)
    assert np.max(np.abs(r - y[rows])) < 1e-13


LAYER_PINS = [
    pin_linear_brute, pin_layer_brute, pin_layer_identity, pin_head_order_of_concat, pin_scale_uses_head_dim,
    pin_layer_chunked_append, pin_layer_rows_api_matches_full,
]


# ------------------------------------------------------------------ the gated sublayer

from oracle import gated as G  # noqa: E402


def _gated_layer_case(seed, lengths, hidden, hq, hkv, d, rot):
    rng = np.random.default_rng(seed)
    n = sum(lengths)
    x = rng.standard_normal((n, hidden))
    w_q = rng.standard_normal((hq * 2 * d, hidden)) / np.sqrt(hidden)
    w_k = rng.standard_normal((hkv * d, hidden)) / np.sqrt(hidden)
    w_v = rng.standard_normal((hkv * d, hidden)) / np.sqrt(hidden)
    w_o = rng.standard_normal((hidden, hq * d)) / np.sqrt(hq * d)
    qw = 0.1 * rng.standard_normal(d)
    kw = 0.1 * rng.standard_normal(d)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return x, w_q, w_k, w_v, w_o, qw, kw, cu


def pin_gated_layer_brute():
    """The gated sublayer against scalar loops (two ragged sequences, GQA,
    partial rotation)."""
    lengths = [3, 4]
    x, w_q, w_k, w_v, w_o, qw, kw, cu = _gated_layer_case(47, lengths, 12, 4, 2, 8, 4)
    y = G.gated_attention_layer_prefill(x, w_q, w_k, w_v, w_o, qw, kw, cu, 4, 2, head_dim=8, eps=1e-6, theta=1e7,
                                        rot_dim=4)
    b = np.array(brute.gated_layer_prefill(x.tolist(), w_q.tolist(), w_k.tolist(), w_v.tolist(), w_o.tolist(),
                                           qw.tolist(), kw.tolist(), lengths, 4, 2, 8, 1e-6, 1e7, 4))
    assert y.shape == (7, 12)
    assert np.max(np.abs(y - b)) < 1e-12, np.max(np.abs(y - b))


def pin_gated_layer_identity():
    """hidden = Hq 2d and W_q = I: head h's query is x's features 2hd .. 2hd+d-1
    and its gate the next d; W_k, W_v pick feature blocks; W_o = [I; 0].  The
    sublayer is then the gated core on those views of x."""
    hq, hkv, d, rot = 4, 2, 8, 4
    lengths = [5, 3]
    rng = np.random.default_rng(48)
    n = sum(lengths)
    x = rng.standard_normal((n, hq * 2 * d))
    eye = np.eye(hq * 2 * d)
    w_k = eye[d:d + hkv * d]        # k = features d .. d + Hkv d - 1
    w_v = eye[-hkv * d:]            # v = the last Hkv d features
    w_o = eye[:, :hq * d]           # y[:, :Hq d] = the merged heads, the rest 0
    qw = 0.1 * rng.standard_normal(d)
    kw = 0.1 * rng.standard_normal(d)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    y = G.gated_attention_layer_prefill(x, eye, w_k, w_v, w_o, qw, kw, cu, hq, hkv, head_dim=d, rot_dim=rot)
    heads = x.reshape(n, hq, 2 * d)
    q, gate = heads[..., :d], heads[..., d:]
    k = x[:, d:d + hkv * d].reshape(n, hkv, d)
    v = x[:, -hkv * d:].reshape(n, hkv, d)
    o = G.gated_attention_prefill(q, gate, k, v, qw, kw, cu, hq, hkv, rot_dim=rot)
    assert np.max(np.abs(y[:, :hq * d] - o.reshape(n, hq * d))) < 1e-13
    assert np.max(np.abs(y[:, hq * d:])) == 0.0


def pin_gated_layer_page_shape():
    """The Qwen3-Next-80B-A3B global layer of the page's model table: hidden
    2048, 16 / 2 heads of 256, q_proj 8192 wide (doubled), k/v 512, o_proj
    from 4096; two tokens through the oracle at that shape, and with the gate
    saturated open (every gate pre-activation +40, sigmoid = 1 to 1e-17) the
    output is o_proj of the ungated attention of the same projections."""
    gd = pins.golden("layer_shapes.json")["qwen3_next_80b_a3b"]
    hidden, hq, hkv, d, rot = gd["hidden"], gd["n_q_heads"], gd["n_kv_heads"], gd["head_dim"], gd["rotary_dim"]
    x, w_q, w_k, w_v, w_o, qw, kw, cu = _gated_layer_case(49, [2], hidden, hq, hkv, d, rot)
    assert w_q.shape[0] == gd["q_proj_width"] == hq * 2 * d
    assert w_k.shape[0] == gd["kv_proj_width"] and w_o.shape[1] == gd["o_proj_in"]
    q, gate, k, v = G.gated_qkv_projection(x, w_q, w_k, w_v, hq, hkv, d)
    assert q.shape == gate.shape == (2, hq, d) and k.shape == v.shape == (2, hkv, d)
    # open every gate: the gate rows of W_q become zero, x gains no bias, so use a
    # shifted copy whose gate half is +40 through a rank-one term on a constant feature
    x1 = np.concatenate([x, np.ones((2, 1))], axis=1)
    wq1 = np.concatenate([w_q, np.zeros((w_q.shape[0], 1))], axis=1)
    for h in range(hq):
        wq1[2 * h * d + d:2 * (h + 1) * d, :] = 0.0
        wq1[2 * h * d + d:2 * (h + 1) * d, -1] = 40.0
    wk1 = np.concatenate([w_k, np.zeros((w_k.shape[0], 1))], axis=1)
    wv1 = np.concatenate([w_v, np.zeros((w_v.shape[0], 1))], axis=1)
    y = G.gated_attention_layer_prefill(x1, wq1, wk1, wv1, w_o, qw, kw, cu, hq, hkv, head_dim=d, theta=gd["theta"],
                                        rot_dim=rot)
    assert y.shape == (2, hidden)
    qo, _, ko, vo = G.gated_qkv_projection(x1, wq1, wk1, wv1, hq, hkv, d)
    ref = np.zeros((2, hq, d))
    for i in range(2):  # the ungated attention, row by row, from the oracle's own pieces
        qh = G.gated_qk_norm_rope(qo[i:i + 1], qw, [i], 1e-6, gd["theta"], rot)
        kh = G.gated_qk_norm_rope(ko[:i + 1], kw, np.arange(i + 1), 1e-6, gd["theta"], rot)
        ref[i] = A._attend(qh, kh, vo[:i + 1], np.array([i]), np.arange(i + 1), hq, hkv, 1.0 / np.sqrt(d))[0]
    assert np.max(np.abs(y - ref.reshape(2, hq * d) @ w_o.T)) < 1e-12


def pin_gated_layer_chunked_append():
    """Appending [0:2], [2:5], [5:6] through the gated sublayer against the
    cache equals one pass ("第 20 章" §20.9 protocol, with the projections)."""
    gd = pins.golden("cache_protocol.json")
    x, w_q, w_k, w_v, w_o, qw, kw, cu = _gated_layer_case(50, [6], 16, 4, 2, 8, 4)
    full = G.gated_attention_layer_prefill(x, w_q, w_k, w_v, w_o, qw, kw, cu, 4, 2, head_dim=8, rot_dim=4)
    kc, vc, outs = np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), []
    for a, b in gd["chunks"]:
        y, kh, v = G.gated_attention_layer_append(x[a:b], w_q, w_k, w_v, w_o, qw, kw, kc, vc, a, 4, 2, head_dim=8,
                                                  rot_dim=4)
        outs.append(y)
        kc, vc = np.concatenate([kc, kh]), np.concatenate([vc, v])
    assert np.max(np.abs(np.concatenate(outs) - full)) < 1e-12


def pin_gated_layer_rows_api_matches_full():
    """The sampled-row entry point equals the full gated sublayer rows it samples."""
    x, w_q, w_k, w_v, w_o, qw, kw, cu = _gated_layer_case(51, [30], 16, 4, 2, 8, 4)
    y = G.gated_attention_layer_prefill(x, w_q, w_k, w_v, w_o, qw, kw, cu, 4, 2, head_dim=8, rot_dim=4)
    rows = np.array([0, 11, 29])
    r = G.gated_attention_layer_prefill_rows(x, w_q, w_k, w_v, w_o, qw, kw, rows, 4, 2, head_dim=8, rot_dim=4)
    assert np.max(np.abs(r - y[rows])) < 1e-13


GATED_LAYER_PINS = [
    pin_gated_layer_brute, pin_gated_layer_identity, pin_gated_layer_page_shape, pin_gated_layer_chunked_append,
    pin_gated_layer_rows_api_matches_full,
]
