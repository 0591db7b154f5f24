"""Plain float64 definitions of the attention-sublayer core (test infrastructure).

Page references used below:
  [QA]  "Transformer 20. Qwen 3 架构拆解" (m.nlpx.cn): §2.2 (attention, GQA index
        formula, scaled dot product), §2.3 (RMSNorm), §2.4 (RoPE base).
  [RL]  "Qwen3" notes on the Transformers model (llm.rainlin.net): section
        "QK-Norm" and the ``Qwen3Attention`` excerpt (norm on the per-head view,
        then RoPE, then the cache update).
  [NW]  "14. Qwen 家族：从 QKV 偏置到混合注意力" (niuwancheng.cn): section
        "Qwen3：去掉偏置，改用 QK-Norm" (one RMSNorm per 128-dim head, before RoPE).
  [XW]  "7.2 Qwen3 全规模实现" (paper.xwysyy.cn): §7.2.1 core components -- the
        RMSNorm, RoPE (frequency table, rotate-half) and GQA + QKNorm listings,
        and the causal mask built in the model.
  [OZ]  "第 20 章 Qwen3 与 Qwen3.5" (book.ozine.me): §20.1 (norm axis = each
        head's own d, then RoPE, then GQA expansion), §20.3 (cache protocol:
        rotate the new K at start_pos, never re-rotate old K; rectangular mask
        from pos_start), §20.9 (chunked-append equivalence).

Readings where the pages are silent or disagree:
  * order: norm then RoPE ([RL], [NW], [XW], [OZ]); [QA] claims RoPE then norm.
    Both are available through ``order`` (the library too, as params.order).
  * eps sits inside the square root, added to the mean square ([XW] RMSNorm;
    the [QA] §2.3 formula is garbled).
  * one gamma of length head_dim for Q and one for K, shared by all heads.
  * RoPE pairs (i, i + d/2) (rotate-half), frequency theta^(-2i/d); the angle is
    taken exactly in float64 here.
  * KV head of query head t is floor(t / g) (0-based form of the [QA] formula).
  * packed sequences are independent; positions restart at 0 in each.
  * softmax scale 1/sqrt(head_dim) ([XW] note after the GQA listing; [OZ] §20.1).

Shapes: token-major ``[n_tok, heads, head_dim]`` arrays.  Any float input is
converted exactly to float64; nothing is rounded anywhere in this module.
"""

import numpy as np

_ROW_BLOCK = 512  # query rows evaluated per matrix product (memory bound only)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kv_head_for_q_head(t, n_q_heads, n_kv_heads):
    """KV head (0-based) that query head ``t`` reads.

    [QA] §2.2 gives the 1-based rule "group floor((t-1)/g)+1" with
    g = h_q / h_kv (heads 1-4 share the first group for 32/8); [XW] §7.2.1
    expands K and V by repeat-interleaving each KV head ``group_size`` times,
    which is the same map.  0-based: floor(t / g).
    """
    if n_kv_heads <= 0 or n_q_heads % n_kv_heads != 0:
        raise ValueError("n_q_heads must be a positive multiple of n_kv_heads")
    g = n_q_heads // n_kv_heads
    return t // g


def rms_norm_heads(x, gamma, eps):
    """RMSNorm of every row along its last axis ([XW] §7.2.1 RMSNorm; [OZ] §20.1).

    Each row (one head of one token) is divided by sqrt(mean of its squares +
    eps) and multiplied elementwise by ``gamma`` (length head_dim, no bias).
    """
    x = _f64(x)
    gamma = _f64(gamma)
    mean_sq = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(mean_sq + eps) * gamma


def rope_inv_freq(head_dim, theta):
    """Rotation frequencies theta^(-2i/d) for i = 0 .. d/2-1 ([XW] §7.2.1 RoPE)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -(2.0 * i) / head_dim)


def rope_rotate_half(x, positions, theta):
    """Rotate-half RoPE ([XW] §7.2.1 RoPE: angles duplicated over both halves,
    result = x*cos + cat(-x2, x1)*sin).

    ``x`` is ``[n, heads, d]``; row n is at position ``positions[n]``.  Pair
    (i, i+d/2) turns by the angle positions[n] * theta^(-2i/d):
        y_i       = x_i cos - x_{i+d/2} sin
        y_{i+d/2} = x_{i+d/2} cos + x_i sin
    """
    x = _f64(x)
    d = x.shape[-1]
    h = d // 2
    pos = np.asarray(positions, dtype=np.float64).reshape(-1)
    if pos.shape[0] != x.shape[0]:
        raise ValueError("one position per token row")
    angle = pos[:, None] * rope_inv_freq(d, theta)[None, :]
    c = np.cos(angle)[:, None, :]
    s = np.sin(angle)[:, None, :]
    first, second = x[..., :h], x[..., h:]
    return np.concatenate([first * c - second * s, second * c + first * s], axis=-1)


def qk_norm_rope(x, gamma, positions, eps, theta, order="norm_rope"):
    """QK-Norm then RoPE on ``[n, heads, d]`` rows ([RL] "QK-Norm"; [NW] Qwen3
    section; [XW] GQA listing; [OZ] §20.1).  ``order="rope_norm"`` gives the
    other order that [QA] §2.2 / §6 describe, for the order demonstration."""
    if order == "norm_rope":
        return rope_rotate_half(rms_norm_heads(x, gamma, eps), positions, theta)
    if order == "rope_norm":
        return rms_norm_heads(rope_rotate_half(x, positions, theta), gamma, eps)
    raise ValueError("order must be 'norm_rope' or 'rope_norm'")


def causal_softmax(scores, q_pos, k_pos):
    """Softmax over keys with the causal mask ([XW] §7.2.1: entries above the
    diagonal set to -inf before softmax; [OZ] §20.3: rectangular mask when the
    queries start at pos_start).  Key j is visible to query i iff
    k_pos[j] <= q_pos[i].  Every query must see at least one key."""
    scores = _f64(scores)
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    if not visible.any(axis=1).all():
        raise ValueError("a query row sees no key")
    masked = np.where(visible, scores, -np.inf)
    row_max = masked.max(axis=1, keepdims=True)
    e = np.where(visible, np.exp(masked - row_max), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def _attend(q_hat, k_hat, v, q_pos, k_pos, n_q_heads, n_kv_heads, scale, heads=None):
    """Softmax attention of rotated queries over rotated keys, per query head
    with its GQA KV head ([XW] §7.2.1 GQA listing: Q K^T, mask, softmax of the
    scaled scores, times V).  q_hat [Lq, Hq, d], k_hat/v [Lk, Hkv, d]."""
    heads = range(n_q_heads) if heads is None else heads
    heads = list(heads)
    lq = q_hat.shape[0]
    out = np.empty((lq, len(heads), q_hat.shape[-1]), dtype=np.float64)
    q_pos = np.asarray(q_pos)
    k_pos = np.asarray(k_pos)
    for hi, t in enumerate(heads):
        u = kv_head_for_q_head(t, n_q_heads, n_kv_heads)
        kt = k_hat[:, u, :]
        vu = v[:, u, :]
        for r0 in range(0, lq, _ROW_BLOCK):
            r1 = min(lq, r0 + _ROW_BLOCK)
            s = (q_hat[r0:r1, t, :] @ kt.T) * scale
            p = causal_softmax(s, q_pos[r0:r1], k_pos)
            out[r0:r1, hi, :] = p @ vu
    return out


def _check_heads(q, k, v, n_q_heads, n_kv_heads):
    if q.shape[1] != n_q_heads or k.shape[1] != n_kv_heads or v.shape[1] != n_kv_heads:
        raise ValueError("head counts do not match the arrays")
    kv_head_for_q_head(0, n_q_heads, n_kv_heads)


def _scale(head_dim, scale):
    return 1.0 / np.sqrt(head_dim) if scale is None else float(scale)


def attention_prefill(q, k, v, q_gamma, k_gamma, cu_seqlens, n_q_heads, n_kv_heads,
                      eps=1e-6, theta=1e6, scale=None, order="norm_rope"):
    """Causal GQA attention over packed sequences.

    q ``[n_tok, Hq, d]``, k and v ``[n_tok, Hkv, d]``; sequence s owns tokens
    cu_seqlens[s] .. cu_seqlens[s+1]-1 at positions 0 .. L_s-1.  Returns the
    float64 output ``[n_tok, Hq, d]`` (before any output projection).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check_heads(q, k, v, n_q_heads, n_kv_heads)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    sc = _scale(q.shape[-1], scale)
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(cu.shape[0] - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        pos = np.arange(b - a)
        qh = qk_norm_rope(q[a:b], q_gamma, pos, eps, theta, order)
        kh = qk_norm_rope(k[a:b], k_gamma, pos, eps, theta, order)
        out[a:b] = _attend(qh, kh, v[a:b], pos, pos, n_q_heads, n_kv_heads, sc)
    return out


def attention_prefill_rows(q_seq, k_seq, v_seq, q_gamma, k_gamma, rows, heads,
                           n_q_heads, n_kv_heads, eps=1e-6, theta=1e6, scale=None,
                           order="norm_rope"):
    """Selected output rows of ONE sequence, each by the same definition as
    :func:`attention_prefill`.  ``q_seq`` holds the sequence's query rows for
    ``rows`` only (``[len(rows), Hq, d]``); ``k_seq``/``v_seq`` hold keys
    0 .. max(rows).  Returns ``[len(rows), len(heads), d]``."""
    q_seq, k_seq, v_seq = _f64(q_seq), _f64(k_seq), _f64(v_seq)
    rows = np.asarray(rows, dtype=np.int64)
    nk = int(rows.max()) + 1
    if k_seq.shape[0] < nk or v_seq.shape[0] < nk:
        raise ValueError("keys up to the last requested row are needed")
    sc = _scale(q_seq.shape[-1], scale)
    qh = qk_norm_rope(q_seq, q_gamma, rows, eps, theta, order)
    kh = qk_norm_rope(k_seq[:nk], k_gamma, np.arange(nk), eps, theta, order)
    return _attend(qh, kh, v_seq[:nk], rows, np.arange(nk), n_q_heads, n_kv_heads, sc,
                   heads=heads)


def attention_append(q_new, k_new, v_new, q_gamma, k_gamma, k_hat_cache, v_cache,
                     start_pos, n_q_heads, n_kv_heads, eps=1e-6, theta=1e6,
                     scale=None, order="norm_rope"):
    """New tokens of ONE sequence attending to its cache plus themselves.

    [OZ] §20.3: the new K is normed and rotated at start_pos .. start_pos+n-1,
    then joined to the cached K, which already carries its rotation and is not
    rotated again; the mask is rectangular from pos_start.  [RL] excerpt: the
    cache receives K after RoPE.  ``k_hat_cache`` ``[start_pos, Hkv, d]`` holds
    the rotated keys of positions 0 .. start_pos-1, ``v_cache`` their values.
    Returns ``(out [n, Hq, d], k_hat_new [n, Hkv, d])``.
    """
    q_new, k_new, v_new = _f64(q_new), _f64(k_new), _f64(v_new)
    k_hat_cache, v_cache = _f64(k_hat_cache), _f64(v_cache)
    start = int(start_pos)
    if k_hat_cache.shape[0] != start or v_cache.shape[0] != start:
        raise ValueError("cache must hold exactly start_pos tokens")
    _check_heads(q_new, k_new, v_new, n_q_heads, n_kv_heads)
    n = q_new.shape[0]
    pos = start + np.arange(n)
    sc = _scale(q_new.shape[-1], scale)
    qh = qk_norm_rope(q_new, q_gamma, pos, eps, theta, order)
    kh_new = qk_norm_rope(k_new, k_gamma, pos, eps, theta, order)
    keys = np.concatenate([k_hat_cache, kh_new], axis=0)
    vals = np.concatenate([v_cache, v_new], axis=0)
    out = _attend(qh, keys, vals, pos, np.arange(start + n), n_q_heads, n_kv_heads, sc)
    return out, kh_new


def attention_decode(q, k, v, q_gamma, k_gamma, k_hat_caches, v_caches, start_pos,
                     n_q_heads, n_kv_heads, eps=1e-6, theta=1e6, scale=None,
                     order="norm_rope"):
    """One new token per sequence (``q [n_seq, Hq, d]``, ``k``/``v``
    ``[n_seq, Hkv, d]``) against per-sequence caches of ``start_pos[i]``
    rotated keys: :func:`attention_append` with n = 1 for each sequence.
    Returns ``[n_seq, Hq, d]``."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    out = np.empty(q.shape, dtype=np.float64)
    for i in range(q.shape[0]):
        o, _ = attention_append(q[i:i + 1], k[i:i + 1], v[i:i + 1], q_gamma, k_gamma,
                                k_hat_caches[i], v_caches[i], start_pos[i],
                                n_q_heads, n_kv_heads, eps, theta, scale, order)
        out[i] = o[0]
    return out
