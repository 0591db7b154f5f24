"""Plain float64 definitions of the gated global-attention layer of the
Qwen3-Next / Qwen3.5 models (test infrastructure; see ``oracle/__init__.py``).

Page references used below:
  [NW]  "14. Qwen 家族：从 QKV 偏置到混合注意力" (niuwancheng.cn): section
        "Qwen3-Next：混合注意力、高稀疏 MoE 与 MTP" -- the global layers double
        the q_proj width (half query, half gate), multiply the attention output
        by sigmoid(gate) before o_proj, use head_dim 256; the norm is the
        zero-centred x_hat * (1 + weight) with the weight initialised to 0.
  [OZ]  "第 20 章 Qwen3 与 Qwen3.5" (book.ozine.me): §20.4 -- the norm scale is
        1 + w; q_proj's 2Hd output is split into query and gate inside each
        head; z = Attn(Q, K, V) * sigmoid(gate); Q/K are normed per head, then
        rotated; only the first d_r coordinates rotate, d_r = head_dim times
        the partial rotary factor rounded to even, and the frequency exponent
        uses d_r, not head_dim, as its denominator (head_dim 256 with factor
        0.25 rotates 64 coordinates).

Readings:
  * the rotated coordinates rotate-half among themselves: pairs (i, i + d_r/2)
    for i < d_r/2, frequency theta^(-2i/d_r); coordinates d_r .. d-1 pass;
  * "split inside each head": head h of the q_proj output owns the slice
    [2hd, 2(h+1)d), its first d values are the query and the next d the gate;
  * the gate multiplies the attention output of the same head and dim;
  * everything else (GQA map, causal mask, scale 1/sqrt(d), packing, cache
    protocol) is the Qwen3 definition of ``oracle/attention.py``.

Nothing is rounded anywhere in this module.
"""

import numpy as np

from . import attention as _A
from . import layer as _L

_f64 = _A._f64


def rotary_dim(head_dim, partial_rotary_factor):
    """d_r: head_dim x factor, rounded down to an even count ([OZ] §20.4)."""
    r = int(head_dim * partial_rotary_factor)
    return r - (r % 2)


def rms_norm_zero_centred(x, w, eps):
    """Each row / sqrt(mean of its squares + eps), times (1 + w) ([NW]
    Qwen3-Next "稳定性"; [OZ] §20.4)."""
    x = _f64(x)
    w = _f64(w)
    mean_sq = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(mean_sq + eps) * (1.0 + w)


def rope_partial(x, positions, theta, rot_dim):
    """Rotate-half RoPE on the first ``rot_dim`` coordinates of every row, with
    frequencies theta^(-2i/rot_dim); the other coordinates pass unchanged
    ([OZ] §20.4 partial_rotary_factor)."""
    x = _f64(x)
    d = x.shape[-1]
    if rot_dim % 2 or not 0 < rot_dim <= d:
        raise ValueError("rot_dim must be even and in (0, head_dim]")
    h = rot_dim // 2
    pos = np.asarray(positions, dtype=np.float64).reshape(-1)
    if pos.shape[0] != x.shape[0]:
        raise ValueError("one position per token row")
    i = np.arange(h, dtype=np.float64)
    inv = np.power(float(theta), -(2.0 * i) / rot_dim)
    angle = pos[:, None] * inv[None, :]
    c = np.cos(angle)[:, None, :]
    s = np.sin(angle)[:, None, :]
    a, b = x[..., :h], x[..., h:rot_dim]
    return np.concatenate([a * c - b * s, b * c + a * s, x[..., rot_dim:]], axis=-1)


def gated_qk_norm_rope(x, w, positions, eps, theta, rot_dim):
    """Zero-centred QK-Norm, then partial RoPE ([OZ] §20.4: norm per head, then
    rotation)."""
    return rope_partial(rms_norm_zero_centred(x, w, eps), positions, theta, rot_dim)


def split_query_gate(q_proj_out, n_heads, head_dim):
    """Per-head split of a ``[n, n_heads * 2 * head_dim]`` q_proj output into
    query and gate, each ``[n, n_heads, head_dim]`` ([OZ] §20.4: reshape to
    2d per head, then cut each head's slice in two)."""
    y = _f64(q_proj_out).reshape(-1, n_heads, 2 * head_dim)
    return y[..., :head_dim], y[..., head_dim:]


def sigmoid(x):
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def gated_attention_prefill(q, gate, k, v, q_w, k_w, cu_seqlens, n_q_heads, n_kv_heads,
                            eps=1e-6, theta=1e7, rot_dim=64, scale=None):
    """Causal GQA over packed sequences with zero-centred QK-Norm, partial RoPE
    and the per-head output gate: o = Attn(q_hat, k_hat, v) * sigmoid(gate)
    ([NW]; [OZ] §20.4).  q, gate ``[n_tok, Hq, d]``; k, v ``[n_tok, Hkv, d]``."""
    q, gate, k, v = _f64(q), _f64(gate), _f64(k), _f64(v)
    _A._check_heads(q, k, v, n_q_heads, n_kv_heads)
    if gate.shape != q.shape:
        raise ValueError("gate must have the query's shape")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    sc = _A._scale(q.shape[-1], scale)
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(cu.shape[0] - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        pos = np.arange(b - a)
        qh = gated_qk_norm_rope(q[a:b], q_w, pos, eps, theta, rot_dim)
        kh = gated_qk_norm_rope(k[a:b], k_w, pos, eps, theta, rot_dim)
        out[a:b] = _A._attend(qh, kh, v[a:b], pos, pos, n_q_heads, n_kv_heads, sc) * sigmoid(gate[a:b])
    return out


def gated_attention_prefill_rows(q_rows, gate_rows, k_seq, v_seq, q_w, k_w, rows, heads, n_q_heads, n_kv_heads,
                                 eps=1e-6, theta=1e7, rot_dim=64, scale=None):
    """Selected output rows of ONE sequence, each by the same definition as
    :func:`gated_attention_prefill`.  ``q_rows``/``gate_rows`` hold the query
    and gate rows of ``rows`` only (``[len(rows), Hq, d]``); ``k_seq``/``v_seq``
    hold keys 0 .. max(rows).  Returns ``[len(rows), len(heads), d]``."""
    q_rows, gate_rows, k_seq, v_seq = _f64(q_rows), _f64(gate_rows), _f64(k_seq), _f64(v_seq)
    rows = np.asarray(rows, dtype=np.int64)
    heads = list(heads)
    nk = int(rows.max()) + 1
    if k_seq.shape[0] < nk or v_seq.shape[0] < nk:
        raise ValueError("keys up to the last requested row are needed")
    sc = _A._scale(q_rows.shape[-1], scale)
    qh = gated_qk_norm_rope(q_rows, q_w, rows, eps, theta, rot_dim)
    kh = gated_qk_norm_rope(k_seq[:nk], k_w, np.arange(nk), eps, theta, rot_dim)
    out = _A._attend(qh, kh, v_seq[:nk], rows, np.arange(nk), n_q_heads, n_kv_heads, sc, heads=heads)
    return out * sigmoid(gate_rows[:, heads, :])


def gated_attention_append(q_new, gate_new, k_new, v_new, q_w, k_w, k_hat_cache, v_cache, start_pos,
                           n_q_heads, n_kv_heads, eps=1e-6, theta=1e7, rot_dim=64, scale=None):
    """New tokens of ONE sequence against its cache of ``start_pos`` normed and
    rotated keys (the Qwen3 cache protocol, [OZ] §20.3), with this layer's
    norm, rotation and gate.  Returns ``(out [n, Hq, d], k_hat_new)``."""
    q_new, gate_new, k_new, v_new = _f64(q_new), _f64(gate_new), _f64(k_new), _f64(v_new)
    k_hat_cache, v_cache = _f64(k_hat_cache), _f64(v_cache)
    start = int(start_pos)
    if k_hat_cache.shape[0] != start or v_cache.shape[0] != start:
        raise ValueError("cache must hold exactly start_pos tokens")
    n = q_new.shape[0]
    pos = start + np.arange(n)
    sc = _A._scale(q_new.shape[-1], scale)
    qh = gated_qk_norm_rope(q_new, q_w, pos, eps, theta, rot_dim)
    kh_new = gated_qk_norm_rope(k_new, k_w, pos, eps, theta, rot_dim)
    keys = np.concatenate([k_hat_cache, kh_new], axis=0)
    vals = np.concatenate([v_cache, v_new], axis=0)
    out = _A._attend(qh, keys, vals, pos, np.arange(start + n), n_q_heads, n_kv_heads, sc)
    return out * sigmoid(gate_new), kh_new


def gated_qkv_projection(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim=256):
    """The gated layer's projections: q_proj gives 2 * head_dim values per
    query head, split inside each head into query and gate ([NW] Qwen3-Next:
    q_proj's width doubled, half query, half gate; [OZ] §20.4); k_proj and
    v_proj as in the Qwen3 layers.  w_q is ``[n_q_heads * 2 * head_dim,
    hidden]``.  Returns (q, gate, k, v)."""
    q, gate = split_query_gate(_L.linear(x, w_q), n_q_heads, head_dim)
    return (q, gate, _L.split_heads(_L.linear(x, w_k), n_kv_heads, head_dim),
            _L.split_heads(_L.linear(x, w_v), n_kv_heads, head_dim))


def gated_attention_layer_prefill(x, w_q, w_k, w_v, w_o, q_w, k_w, cu_seqlens, n_q_heads, n_kv_heads,
                                  head_dim=256, eps=1e-6, theta=1e7, rot_dim=64, scale=None):
    """The gated global-attention sublayer over packed sequences: the
    projections above, the gated core, then o_proj on the gated heads
    concatenated in order (the attention output is multiplied by
    sigmoid(gate) before o_proj: [NW]; [OZ] §20.4).  x ``[n_tok, hidden]`` ->
    ``[n_tok, hidden]``; w_o is ``[hidden, n_q_heads * head_dim]``."""
    q, gate, k, v = gated_qkv_projection(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim)
    o = gated_attention_prefill(q, gate, k, v, q_w, k_w, cu_seqlens, n_q_heads, n_kv_heads, eps=eps, theta=theta,
                                rot_dim=rot_dim, scale=scale)
    return _L.linear(_L.merge_heads(o), w_o)


def gated_attention_layer_prefill_rows(x_seq, w_q, w_k, w_v, w_o, q_w, k_w, rows, n_q_heads, n_kv_heads,
                                       head_dim=256, eps=1e-6, theta=1e7, rot_dim=64, scale=None):
    """Selected output rows of ONE sequence, each by the same definition as
    :func:`gated_attention_layer_prefill`; ``x_seq`` holds the sequence's
    hidden rows 0 .. max(rows).  Returns ``[len(rows), hidden]``."""
    x_seq = _f64(x_seq)
    rows = np.asarray(rows, dtype=np.int64)
    nk = int(rows.max()) + 1
    q, gate = split_query_gate(_L.linear(x_seq[rows], w_q), n_q_heads, head_dim)
    k = _L.split_heads(_L.linear(x_seq[:nk], w_k), n_kv_heads, head_dim)
    v = _L.split_heads(_L.linear(x_seq[:nk], w_v), n_kv_heads, head_dim)
    o = gated_attention_prefill_rows(q, gate, k, v, q_w, k_w, rows, range(n_q_heads), n_q_heads, n_kv_heads,
                                     eps=eps, theta=theta, rot_dim=rot_dim, scale=scale)
    return _L.linear(_L.merge_heads(o), w_o)


def gated_attention_layer_append(x_new, w_q, w_k, w_v, w_o, q_w, k_w, k_hat_cache, v_cache, start_pos,
                                 n_q_heads, n_kv_heads, head_dim=256, eps=1e-6, theta=1e7, rot_dim=64, scale=None):
    """New tokens of ONE sequence through the gated sublayer against its cache
    of ``start_pos`` normed and rotated keys and values.  Returns ``(y [n,
    hidden], k_hat_new, v_new)``."""
    q, gate, k, v = gated_qkv_projection(x_new, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim)
    o, kh = gated_attention_append(q, gate, k, v, q_w, k_w, k_hat_cache, v_cache, start_pos, n_q_heads, n_kv_heads,
                                   eps=eps, theta=theta, rot_dim=rot_dim, scale=scale)
    return _L.linear(_L.merge_heads(o), w_o), kh, v
