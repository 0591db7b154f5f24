"""Plain float64 definitions of the whole attention sublayer around the core:
the q/k/v projections before it and o_proj after it (test infrastructure; see
``oracle/__init__.py``).

Page references used below:
  [QN]  "Qwen3" notes (transformers modeling_qwen3 excerpt): q_proj, k_proj,
        v_proj and o_proj are bias-free linear maps (hidden -> H * head_dim and
        back); each projection output is viewed as [..., heads, head_dim];
        the data flow is qkv_proj -> split -> RMSNorm(Q, K) -> RoPE ->
        attention -> o_proj.
  [XW]  "7.2 Qwen3 全规模实现" §7.2.1 GQA + QKNorm listing: W_query / W_key /
        W_value applied to x, viewed per head, QK-Norm before RoPE, the heads'
        context vectors concatenated in head order and passed through
        out_proj; the softmax scale uses the fixed head_dim (128), not
        emb_dim / num_heads (the 0.6B model: emb 1024, 16 heads, q width 2048).
  [NW]  "14. Qwen 家族：从 QKV 偏置到混合注意力", model table: Qwen3 has no QKV
        bias (QK-Norm replaced it); hidden sizes 1024 / 4096 / 5120 ...

Readings:
  * a linear map with weight W [out, in] computes y = x W^T (no bias);
  * head h of a projection output owns the features h*d .. (h+1)*d - 1, and
    the attention output rows of the heads are concatenated in head order
    before o_proj;
  * everything between the projections is ``oracle/attention.py``.

Nothing is rounded anywhere in this module.
"""

import numpy as np

from . import attention as _A

_f64 = _A._f64


def linear(x, w):
    """Bias-free linear map: y = x W^T for W of shape [out, in] ([QN], [XW])."""
    x, w = _f64(x), _f64(w)
    if x.shape[-1] != w.shape[1]:
        raise ValueError("x's last dim must equal W's input width")
    return x @ w.T


def split_heads(y, n_heads, head_dim):
    """[n, heads * d] -> [n, heads, d]: head h owns features h*d .. (h+1)*d - 1."""
    y = _f64(y)
    if y.shape[-1] != n_heads * head_dim:
        raise ValueError("width is not heads * head_dim")
    return y.reshape(y.shape[0], n_heads, head_dim)


def merge_heads(o):
    """[n, heads, d] -> [n, heads * d], heads concatenated in order ([XW])."""
    o = _f64(o)
    return o.reshape(o.shape[0], o.shape[1] * o.shape[2])


def qkv_projection(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim=128):
    """The three projections, each split into heads ([QN])."""
    return (split_heads(linear(x, w_q), n_q_heads, head_dim),
            split_heads(linear(x, w_k), n_kv_heads, head_dim),
            split_heads(linear(x, w_v), n_kv_heads, head_dim))


def attention_layer_prefill(x, w_q, w_k, w_v, w_o, q_gamma, k_gamma, cu_seqlens, n_q_heads, n_kv_heads,
                            head_dim=128, eps=1e-6, theta=1e6, scale=None, order="norm_rope"):
    """The attention sublayer over packed sequences: projections, the core
    (QK-Norm, RoPE, causal GQA), o_proj.  x [n_tok, hidden] -> y [n_tok, hidden]."""
    q, k, v = qkv_projection(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim)
    o = _A.attention_prefill(q, k, v, q_gamma, k_gamma, cu_seqlens, n_q_heads, n_kv_heads, eps=eps, theta=theta,
                             scale=scale, order=order)
    return linear(merge_heads(o), w_o)


def attention_layer_prefill_rows(x_seq, w_q, w_k, w_v, w_o, q_gamma, k_gamma, rows, n_q_heads, n_kv_heads,
                                 head_dim=128, eps=1e-6, theta=1e6, scale=None, order="norm_rope"):
    """Selected output rows of ONE sequence, each by the same definition as
    :func:`attention_layer_prefill`; ``x_seq`` holds the sequence's hidden rows
    0 .. max(rows).  Returns ``[len(rows), hidden]``."""
    x_seq = _f64(x_seq)
    rows = np.asarray(rows, dtype=np.int64)
    nk = int(rows.max()) + 1
    q = split_heads(linear(x_seq[rows], w_q), n_q_heads, head_dim)
    k = split_heads(linear(x_seq[:nk], w_k), n_kv_heads, head_dim)
    v = split_heads(linear(x_seq[:nk], w_v), n_kv_heads, head_dim)
    o = _A.attention_prefill_rows(q, k, v, q_gamma, k_gamma, rows, range(n_q_heads), n_q_heads, n_kv_heads,
                                  eps=eps, theta=theta, scale=scale, order=order)
    return linear(merge_heads(o), w_o)


def attention_layer_append(x_new, w_q, w_k, w_v, w_o, q_gamma, k_gamma, k_hat_cache, v_cache, start_pos,
                           n_q_heads, n_kv_heads, head_dim=128, eps=1e-6, theta=1e6, scale=None, order="norm_rope"):
    """New tokens of ONE sequence through the sublayer against its cache of
    ``start_pos`` rotated keys and values.  Returns ``(y [n, hidden], k_hat_new,
    v_new)`` (the cache entries the new tokens add)."""
    q, k, v = qkv_projection(x_new, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim)
    o, kh = _A.attention_append(q, k, v, q_gamma, k_gamma, k_hat_cache, v_cache, start_pos, n_q_heads, n_kv_heads,
                                eps=eps, theta=theta, scale=scale, order=order)
    return linear(merge_heads(o), w_o), kh, v
