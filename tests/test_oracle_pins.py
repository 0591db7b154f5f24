"""The oracle against its pins (CPU only)."""

import numpy as np
import pytest

import pins
from oracle import attention as A


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_brute_force_full_head_dim():
    pins.pin_brute_force(d=128)


# ------------------------------------------------------------------ mutations
# Each plants one plausible mistake in the oracle (on the CPU) and checks that
# at least one pin fails, so the pins would have caught it.

def _rope_sign_flip(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * A.rope_inv_freq(x.shape[-1], theta)
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    return np.concatenate([x[..., :h] * c + x[..., h:] * s, x[..., h:] * c - x[..., :h] * s], -1)


def _rope_interleaved(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * A.rope_inv_freq(d, theta)
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = a * c - b * s
    y[..., 1::2] = b * c + a * s
    return y


def _rope_wrong_freq(head_dim, theta):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -i / head_dim)


def _norm_eps_outside(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * gamma


def _norm_all_heads(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=(-2, -1), keepdims=True)
    return x / np.sqrt(ms + eps) * gamma


def _norm_no_gamma(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _kv_modulo(t, n_q_heads, n_kv_heads):
    return t % n_kv_heads


def _softmax_strict_mask(scores, q_pos, k_pos):
    vis = np.asarray(k_pos)[None, :] < np.asarray(q_pos)[:, None]
    vis[:, 0] = True
    s = np.where(vis, scores, -np.inf)
    e = np.where(vis, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def _softmax_no_mask(scores, q_pos, k_pos):
    s = np.asarray(scores, dtype=np.float64)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


_orig_qk = A.qk_norm_rope


def _order_swapped(x, gamma, positions, eps, theta, order="norm_rope"):
    other = "rope_norm" if order == "norm_rope" else "norm_rope"
    return _orig_qk(x, gamma, positions, eps, theta, other)


_orig_attend = A._attend


def _attend_wrong_scale(q_hat, k_hat, v, q_pos, k_pos, hq, hkv, scale, heads=None):
    return _orig_attend(q_hat, k_hat, v, q_pos, k_pos, hq, hkv, scale * scale * 128 / 64 ** 0.5, heads)


MUTATIONS = {
    "rope_sign_flip": ("rope_rotate_half", _rope_sign_flip),
    "rope_interleaved_pairs": ("rope_rotate_half", _rope_interleaved),
    "rope_freq_missing_factor_2": ("rope_inv_freq", _rope_wrong_freq),
    "norm_eps_outside_root": ("rms_norm_heads", _norm_eps_outside),
    "norm_over_all_heads": ("rms_norm_heads", _norm_all_heads),
    "norm_gamma_dropped": ("rms_norm_heads", _norm_no_gamma),
    "gqa_modulo_map": ("kv_head_for_q_head", _kv_modulo),
    "mask_off_by_one": ("causal_softmax", _softmax_strict_mask),
    "mask_missing": ("causal_softmax", _softmax_no_mask),
    "order_swapped": ("qk_norm_rope", _order_swapped),
    "scale_wrong": ("_attend", _attend_wrong_scale),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(A, attr, fn)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    try:
        pins.pin_brute_force(d=128)
    except (AssertionError, ValueError):
        failed.append("pin_brute_force_d128")
    assert failed, f"no pin caught the planted mistake {name}"


# ------------------------------------------------------------------ gated global-attention layer

import pins_gated  # noqa: E402
from oracle import gated as G  # noqa: E402


@pytest.mark.parametrize("pin", pins_gated.GATED_PINS, ids=lambda f: f.__name__)
def test_gated_pin(pin):
    pin()


def test_gated_brute_force_full_width():
    pins_gated.pin_gated_brute_force(d=32, rot=8)


def _rope_partial_full_denominator(x, positions, theta, rot_dim):
    # frequency denominator head_dim instead of rot_dim (the proportional-RoPE convention)
    x = np.asarray(x, dtype=np.float64)
    d, h = x.shape[-1], rot_dim // 2
    inv = np.power(float(theta), -(2.0 * np.arange(h)) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :h], x[..., h:rot_dim]
    return np.concatenate([a * c - b * s, b * c + a * s, x[..., rot_dim:]], axis=-1)


def _rope_partial_all_dims(x, positions, theta, rot_dim):
    return A.rope_rotate_half(x, positions, theta)


def _norm_plain_gamma(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w)


def _split_halves(q_proj_out, n_heads, head_dim):
    y = np.asarray(q_proj_out, dtype=np.float64).reshape(-1, 2 * n_heads * head_dim)
    return (y[:, :n_heads * head_dim].reshape(-1, n_heads, head_dim),
            y[:, n_heads * head_dim:].reshape(-1, n_heads, head_dim))


def _sigmoid_tanh(x):
    return np.tanh(np.asarray(x, dtype=np.float64))


GATED_MUTATIONS = {
    "rope_full_denominator": ("rope_partial", _rope_partial_full_denominator),
    "rope_all_dims": ("rope_partial", _rope_partial_all_dims),
    "norm_gamma_not_one_plus_w": ("rms_norm_zero_centred", _norm_plain_gamma),
    "gate_split_across_heads": ("split_query_gate", _split_halves),
    "gate_tanh": ("sigmoid", _sigmoid_tanh),
}


@pytest.mark.parametrize("name", sorted(GATED_MUTATIONS))
def test_gated_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = GATED_MUTATIONS[name]
    monkeypatch.setattr(G, attr, fn)
    failed = []
    for pin in pins_gated.GATED_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"


# ------------------------------------------------------------------ the sublayer (projections)

import pins_layer  # noqa: E402
from oracle import layer as Y  # noqa: E402


@pytest.mark.parametrize("pin", pins_layer.LAYER_PINS, ids=lambda f: f.__name__)
def test_layer_pin(pin):
    pin()


def _linear_untransposed(x, w):
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64)


def _split_heads_dim_major(y, n_heads, head_dim):
    y = np.asarray(y, dtype=np.float64)
    return y.reshape(y.shape[0], head_dim, n_heads).transpose(0, 2, 1)


def _merge_heads_dim_major(o):
    o = np.asarray(o, dtype=np.float64)
    return o.transpose(0, 2, 1).reshape(o.shape[0], -1)


LAYER_MUTATIONS = {
    "linear_without_transpose": ("linear", _linear_untransposed),
    "split_heads_dim_major": ("split_heads", _split_heads_dim_major),
    "merge_heads_dim_major": ("merge_heads", _merge_heads_dim_major),
}


@pytest.mark.parametrize("name", sorted(LAYER_MUTATIONS))
def test_layer_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = LAYER_MUTATIONS[name]
    monkeypatch.setattr(Y, attr, fn)
    failed = []
    for pin in pins_layer.LAYER_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"


# ------------------------------------------------------------------ the gated sublayer

@pytest.mark.parametrize("pin", pins_layer.GATED_LAYER_PINS, ids=lambda f: f.__name__)
def test_gated_layer_pin(pin):
    pin()


def _split_query_gate_swapped(q_proj_out, n_heads, head_dim):
    y = np.asarray(q_proj_out, dtype=np.float64).reshape(-1, n_heads, 2 * head_dim)
    return y[..., head_dim:], y[..., :head_dim]


GATED_LAYER_MUTATIONS = {
    "gate_split_across_heads": (G, "split_query_gate", _split_halves),
    "query_gate_swapped": (G, "split_query_gate", _split_query_gate_swapped),
    "linear_without_transpose": (Y, "linear", _linear_untransposed),
    "split_heads_dim_major": (Y, "split_heads", _split_heads_dim_major),
    "merge_heads_dim_major": (Y, "merge_heads", _merge_heads_dim_major),
}


@pytest.mark.parametrize("name", sorted(GATED_LAYER_MUTATIONS))
def test_gated_layer_planted_mistake_is_caught(name, monkeypatch):
    mod, attr, fn = GATED_LAYER_MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    failed = []
    for pin in pins_layer.GATED_LAYER_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
