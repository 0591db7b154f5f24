"""Scalar brute force of the attention core, in pure Python (``math`` only), for
tiny shapes.  Written independently of ``oracle/`` (no shared code): loops over
every token, head, key and dimension, straight from the definitions -- RMSNorm
per head row with eps inside the root, rotate-half RoPE with frequency
theta^(-2i/d), scores scaled by 1/sqrt(d), causal softmax, weighted sum of V,
query head t reading KV head floor(t / g)."""

import math


def _norm_row(row, gamma, eps):
    ms = sum(x * x for x in row) / len(row)
    r = 1.0 / math.sqrt(ms + eps)
    return [row[i] * r * gamma[i] for i in range(len(row))]


def _rope_row(row, pos, theta):
    d = len(row)
    h = d // 2
    out = [0.0] * d
    for i in range(h):
        ang = pos * theta ** (-(2.0 * i) / d)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = row[i] * c - row[i + h] * s
        out[i + h] = row[i + h] * c + row[i] * s
    return out


def prefill(q, k, v, q_gamma, k_gamma, lengths, n_q_heads, n_kv_heads, eps, theta):
    """q[t][h][d], k/v[t][h][d] nested lists (packed tokens).  Returns o[t][h][d]."""
    g = n_q_heads // n_kv_heads
    d = len(q[0][0])
    scale = 1.0 / math.sqrt(d)
    out = []
    base = 0
    for L in lengths:
        qh = [[_rope_row(_norm_row(q[base + i][t], q_gamma, eps), i, theta)
               for t in range(n_q_heads)] for i in range(L)]
        kh = [[_rope_row(_norm_row(k[base + j][u], k_gamma, eps), j, theta)
               for u in range(n_kv_heads)] for j in range(L)]
        for i in range(L):
            row = []
            for t in range(n_q_heads):
                u = t // g
                s = [sum(qh[i][t][e] * kh[j][u][e] for e in range(d)) * scale for j in range(i + 1)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = sum(w)
                row.append([sum(w[j] * v[base + j][u][e] for j in range(i + 1)) / z for e in range(d)])
            out.append(row)
        base += L
    return out


def _norm_row_zero_centred(row, w, eps):
    ms = sum(x * x for x in row) / len(row)
    r = 1.0 / math.sqrt(ms + eps)
    return [row[i] * r * (1.0 + w[i]) for i in range(len(row))]


def _rope_row_partial(row, pos, theta, rot):
    out = list(row)
    h = rot // 2
    for i in range(h):
        ang = pos * theta ** (-(2.0 * i) / rot)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = row[i] * c - row[i + h] * s
        out[i + h] = row[i + h] * c + row[i] * s
    return out


def gated_prefill(q, gate, k, v, q_w, k_w, lengths, n_q_heads, n_kv_heads, eps, theta, rot):
    """The gated global-attention layer: zero-centred norm (scale 1 + w), RoPE on
    the first ``rot`` coordinates with frequency theta^(-2i/rot), causal GQA
    softmax attention, output times 1 / (1 + exp(-gate))."""
    g = n_q_heads // n_kv_heads
    d = len(q[0][0])
    scale = 1.0 / math.sqrt(d)
    out = []
    base = 0
    for L in lengths:
        qh = [[_rope_row_partial(_norm_row_zero_centred(q[base + i][t], q_w, eps), i, theta, rot)
               for t in range(n_q_heads)] for i in range(L)]
        kh = [[_rope_row_partial(_norm_row_zero_centred(k[base + j][u], k_w, eps), j, theta, rot)
               for u in range(n_kv_heads)] for j in range(L)]
        for i in range(L):
            row = []
            for t in range(n_q_heads):
                u = t // g
                s = [sum(qh[i][t][e] * kh[j][u][e] for e in range(d)) * scale for j in range(i + 1)]
                m = max(s)
                wts = [math.exp(x - m) for x in s]
                z = sum(wts)
                row.append([sum(wts[j] * v[base + j][u][e] for j in range(i + 1)) / z
                            / (1.0 + math.exp(-gate[base + i][t][e])) for e in range(d)])
            out.append(row)
        base += L
    return out


def linear(x, w):
    """y[t][o] = sum_i x[t][i] * w[o][i] (bias-free linear map, W stored [out][in])."""
    return [[sum(row[i] * w[o][i] for i in range(len(row))) for o in range(len(w))] for row in x]


def layer_prefill(x, w_q, w_k, w_v, w_o, q_gamma, k_gamma, lengths, n_q_heads, n_kv_heads, head_dim, eps, theta):
    """The attention sublayer: projections, head split (head h = features
    h*d .. h*d+d-1), the core above, heads concatenated in order, o_proj."""
    def heads(rows, n):
        return [[[r[h * head_dim + e] for e in range(head_dim)] for h in range(n)] for r in rows]
    q = heads(linear(x, w_q), n_q_heads)
    k = heads(linear(x, w_k), n_kv_heads)
    v = heads(linear(x, w_v), n_kv_heads)
    o = prefill(q, k, v, q_gamma, k_gamma, lengths, n_q_heads, n_kv_heads, eps, theta)
    merged = [[o[t][h][e] for h in range(n_q_heads) for e in range(head_dim)] for t in range(len(o))]
    return linear(merged, w_o)


def gated_layer_prefill(x, w_q, w_k, w_v, w_o, q_w, k_w, lengths, n_q_heads, n_kv_heads, head_dim, eps, theta,
                        rot):
    """The gated sublayer: q_proj gives 2 * head_dim values per query head, the
    first head_dim of them the query and the next head_dim the gate; k_proj
    and v_proj split into heads of head_dim; the gated layer above; heads
    concatenated in order; o_proj."""
    qp = linear(x, w_q)
    q = [[[r[2 * h * head_dim + e] for e in range(head_dim)] for h in range(n_q_heads)] for r in qp]
    gate = [[[r[2 * h * head_dim + head_dim + e] for e in range(head_dim)] for h in range(n_q_heads)] for r in qp]
    k = [[[r[h * head_dim + e] for e in range(head_dim)] for h in range(n_kv_heads)] for r in linear(x, w_k)]
    v = [[[r[h * head_dim + e] for e in range(head_dim)] for h in range(n_kv_heads)] for r in linear(x, w_v)]
    o = gated_prefill(q, gate, k, v, q_w, k_w, lengths, n_q_heads, n_kv_heads, eps, theta, rot)
    merged = [[o[t][h][e] for h in range(n_q_heads) for e in range(head_dim)] for t in range(len(o))]
    return linear(merged, w_o)
