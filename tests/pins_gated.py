"""Pins of the oracle's gated global-attention layer (Qwen3-Next / Qwen3.5):
closed forms, pass-through and reduction properties, the pages' printed sizes
and brute force, each independent of the oracle's own code.  Like ``pins.py``,
they look the oracle up at call time so that mutation tests can plant a
mistake and see which pin catches it."""

import math

import numpy as np

import brute
import pins
from oracle import attention as A
from oracle import gated as G


def _case(seed, lengths, hq, hkv, d=256, rot=64):
    rng = np.random.default_rng(seed)
    n = sum(lengths)
    q = rng.standard_normal((n, hq, d)) * np.exp(rng.uniform(-3, 3, size=(n, hq, 1)))
    gate = rng.standard_normal((n, hq, d)) * 2.0
    k = rng.standard_normal((n, hkv, d)) * np.exp(rng.uniform(-3, 3, size=(n, hkv, 1)))
    v = rng.standard_normal((n, hkv, d))
    qw = 0.1 * rng.standard_normal(d)
    kw = 0.1 * rng.standard_normal(d)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, gate, k, v, qw, kw, cu


def pin_rotary_width():
    """[OZ] §20.4: head_dim 256 with factor 0.25 rotates 64 coordinates (rounded to even)."""
    gd = pins.golden("gated_layer.json")
    assert G.rotary_dim(gd["head_dim"], gd["partial_rotary_factor"]) == gd["rotary_dim"]
    assert G.rotary_dim(100, 0.25) == 24 and G.rotary_dim(128, 1.0) == 128


def pin_zero_centred_norm():
    """x_hat * (1 + w): rms(y / (1 + w)) = sqrt(ms / (ms + eps)) per row; w = 0 is the
    plain unit-RMS row; a zero row stays 0."""
    rng = np.random.default_rng(30)
    x = rng.standard_normal((20, 3, 256)) * np.exp(rng.uniform(-4, 4, size=(20, 3, 1)))
    x[2, 1] = 0.0
    w = 0.2 * rng.standard_normal(256)
    eps = 1e-6
    y = G.rms_norm_zero_centred(x, w, eps)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.sqrt(np.mean((y / (1 + w)) ** 2, axis=-1)), np.sqrt(ms / (ms + eps)), rtol=1e-12, atol=0)
    assert np.all(y[2, 1] == 0.0)
    y0 = G.rms_norm_zero_centred(x, np.zeros(256), eps)
    assert np.allclose(np.sqrt(np.mean(y0 ** 2, axis=-1)), np.sqrt(ms / (ms + eps)), rtol=1e-12, atol=0)


def pin_partial_rope():
    """Coordinates rot .. d-1 pass bit for bit; each rotated pair (i, i + rot/2) keeps its norm;
    pair 0 turns by exactly p radians (frequency 1) and pair rot/2 - 1 by
    p * theta^(-(rot-2)/rot) -- the denominator is rot, not d ([OZ] §20.4); with rot = d it is
    the full rotate-half RoPE."""
    rng = np.random.default_rng(31)
    d, rot, theta = 256, 64, 1e7
    x = rng.standard_normal((9, 2, d))
    pos = np.array([0, 1, 2, 3, 5, 100, 1000, 12345, 32767])
    y = G.rope_partial(x, pos, theta, rot)
    assert np.array_equal(y[..., rot:], x[..., rot:])
    h = rot // 2
    n0 = x[..., :h] ** 2 + x[..., h:rot] ** 2
    n1 = y[..., :h] ** 2 + y[..., h:rot] ** 2
    assert np.allclose(n0, n1, rtol=1e-13, atol=0)
    assert np.array_equal(y[0], x[0])  # position 0 is the identity
    e = np.zeros((3, 1, d))
    e[:, 0, 0] = 1.0
    e[:, 0, h - 1] = 1.0
    ye = G.rope_partial(e, [1, 2, 7], theta, rot)
    for j, p in enumerate([1, 2, 7]):
        assert abs(math.atan2(ye[j, 0, h], ye[j, 0, 0]) - math.remainder(p * 1.0, 2 * math.pi)) < 1e-12
        want = math.remainder(p * theta ** (-(rot - 2) / rot), 2 * math.pi)
        assert abs(math.atan2(ye[j, 0, rot - 1], ye[j, 0, h - 1]) - want) < 1e-12
    full = G.rope_partial(x, pos, theta, d)
    assert np.max(np.abs(full - A.rope_rotate_half(x, pos, theta))) < 1e-13


def pin_split_per_head():
    """[OZ] §20.4: q_proj's 2Hd output splits inside each head -- head h's query is slice
    [2hd, 2hd + d) and its gate [2hd + d, 2(h+1)d); cutting the whole vector in two halves
    instead puts some heads' gates into queries."""
    H, d = 4, 8
    row = np.arange(2 * H * d, dtype=np.float64)[None, :]
    q, g = G.split_query_gate(row, H, d)
    for h in range(H):
        assert np.array_equal(q[0, h], np.arange(2 * h * d, 2 * h * d + d))
        assert np.array_equal(g[0, h], np.arange(2 * h * d + d, 2 * (h + 1) * d))
    halves = row[:, :H * d].reshape(1, H, d)
    assert not np.array_equal(halves, q)


def pin_gate_values():
    """The gate is an elementwise sigmoid: gate 0 halves the output exactly, gate ln 3 scales
    it by 3/4, a gate of 40 leaves it unchanged to 1e-15."""
    lengths = [5, 3]
    q, gate, k, v, qw, kw, cu = _case(32, lengths, 4, 2, d=16, rot=8)
    base = G.gated_attention_prefill(q, np.full(q.shape, 40.0), k, v, qw, kw, cu, 4, 2, rot_dim=8)
    half = G.gated_attention_prefill(q, np.zeros(q.shape), k, v, qw, kw, cu, 4, 2, rot_dim=8)
    q34 = G.gated_attention_prefill(q, np.full(q.shape, math.log(3.0)), k, v, qw, kw, cu, 4, 2, rot_dim=8)
    assert np.max(np.abs(half - 0.5 * base)) < 1e-15
    assert np.max(np.abs(q34 - 0.75 * base)) < 1e-14
    s = G.sigmoid(np.array([0.0, math.log(3.0), -math.log(3.0)]))
    assert np.allclose(s, [0.5, 0.75, 0.25], rtol=0, atol=1e-16)


def pin_gated_reduces_to_qwen3():
    """With rot = d, w = gamma - 1 and a saturated gate the layer is the Qwen3 attention core."""
    lengths = [6, 4]
    q, gate, k, v, qw, kw, cu = _case(33, lengths, 8, 2, d=128, rot=128)
    o = G.gated_attention_prefill(q, np.full(q.shape, 40.0), k, v, qw, kw, cu, 8, 2, eps=1e-6, theta=1e6,
                                  rot_dim=128)
    r = A.attention_prefill(q, k, v, 1.0 + qw, 1.0 + kw, cu, 8, 2, eps=1e-6, theta=1e6)
    assert np.max(np.abs(o - r)) < 1e-12


def pin_gated_brute_force(d=8, rot=4):
    """Scalar loops (tests/brute.py) on two ragged sequences equal the vectorised layer."""
    lengths = [3, 5]
    q, gate, k, v, qw, kw, cu = _case(34 + d, lengths, 4, 2, d=d, rot=rot)
    o = G.gated_attention_prefill(q, gate, k, v, qw, kw, cu, 4, 2, eps=1e-6, theta=1e7, rot_dim=rot)
    b = np.array(brute.gated_prefill(q.tolist(), gate.tolist(), k.tolist(), v.tolist(), qw.tolist(),
                                     kw.tolist(), lengths, 4, 2, 1e-6, 1e7, rot))
    assert np.max(np.abs(o - b)) < 1e-12, np.max(np.abs(o - b))


def pin_gated_chunked_append():
    """Appending [0:2], [2:5], [5:6] against the cache equals one pass ([OZ] §20.9 protocol)."""
    gd = pins.golden("cache_protocol.json")
    q, gate, k, v, qw, kw, cu = _case(35, [6], 4, 2)
    full = G.gated_attention_prefill(q, gate, k, v, qw, kw, cu, 4, 2)
    kc = np.zeros((0, 2, 256))
    vc = np.zeros((0, 2, 256))
    outs = []
    for a, b in gd["chunks"]:
        o, kh = G.gated_attention_append(q[a:b], gate[a:b], k[a:b], v[a:b], qw, kw, kc, vc, a, 4, 2)
        outs.append(o)
        kc = np.concatenate([kc, kh])
        vc = np.concatenate([vc, v[a:b]])
    assert np.max(np.abs(np.concatenate(outs) - full)) < 1e-12


def pin_global_layer_kv_bytes():
    """[NW] Qwen3-Next: the 12 global layers keep 2 x 12 x 2 x 256 x 2 B = 24 KiB of K and V
    per token (the KV accounting at head_dim 256)."""
    from attention_qk_norm_amd import accounting
    gd = pins.golden("gated_layer.json")
    assert accounting.kv_bytes_per_token(gd["kv_heads"], head_dim=gd["head_dim"],
                                         layers=gd["global_layers"]) == gd["kv_bytes_per_token_global_layers"]


def pin_gated_rows_api_matches_full():
    """The sampled-row entry point equals the full prefill rows it samples."""
    q, gate, k, v, qw, kw, cu = _case(36, [40], 8, 2)
    o = G.gated_attention_prefill(q, gate, k, v, qw, kw, cu, 8, 2)
    rows = np.array([0, 17, 39])
    r = G.gated_attention_prefill_rows(q[rows], gate[rows], k, v, qw, kw, rows, [1, 6], 8, 2)
    assert np.max(np.abs(r - o[rows][:, [1, 6]])) < 1e-13


GATED_PINS = [
    pin_rotary_width, pin_zero_centred_norm, pin_partial_rope, pin_split_per_head, pin_gate_values,
    pin_gated_reduces_to_qwen3, pin_gated_brute_force, pin_gated_chunked_append, pin_global_layer_kv_bytes,
    pin_gated_rows_api_matches_full,
]
