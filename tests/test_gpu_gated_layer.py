"""GPU parity of the gated global-attention sublayer (Qwen3-Next / Qwen3.5,
head_dim 256) through the C-ABI against the CPU oracle
(``oracle.gated_attention_layer_prefill``): the fused projection (per query
head its query and gate, raw; key heads zero-centred-normed and partially
rotated at each token's position into the cache; value heads), the gated core
and o_proj.

Tolerances as for the Qwen3 sublayer: y per element max 2e-2 and mean 2e-3
(x ~ N(0,1), weights N(0,1)/sqrt(fan-in): unit-scale q, k, v, gate and y);
the cached K̂ within the projection's error carried through the norm and the
rotation to first order, plus one bf16 rounding; V within the linear map's
bound.  Chunked appends through the sublayer equal one pass bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from attention_qk_norm_amd import binding as B
from attention_qk_norm_amd import inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_util as U
else:  # collected on a CPU-only machine: every test here is deselected by -m "not gpu"
    U = None

BF = torch.bfloat16
D = 256


def _inputs(cid, hq, hkv, lengths, hidden, rot, gate=True):
    spec = inputs.gated_spec(cid, "bf16", hq, hkv, lengths, rot=rot)
    w_qkv, w_o = inputs.layer_weights(spec, hidden)
    if not gate:  # query rows only: drop each head's gate rows
        q = w_qkv[:hq * 2 * D].reshape(hq, 2, D, hidden)[:, 0].reshape(hq * D, hidden)
        w_qkv = np.concatenate([q, w_qkv[hq * 2 * D:]])
    x = inputs.layer_x(spec, hidden)
    gq, gk = inputs.gammas(spec)
    return spec, x, w_qkv, w_o, gq, gk


def _params(spec, gate=True):
    p = B.make_gated_params(spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, rope_theta=spec.theta, rotary_dim=spec.rot)
    p.output_gate = 1 if gate else 0
    return p


def _oracle(spec, x, w_qkv, w_o, gq, gk, cu, gate=True, rows=None):
    hq, hkv = spec.n_q_heads, spec.n_kv_heads
    qw = hq * (2 if gate else 1) * D
    wq, wk, wv = w_qkv[:qw], w_qkv[qw:qw + hkv * D], w_qkv[qw + hkv * D:]
    if gate:
        if rows is None:
            return oracle.gated_attention_layer_prefill(x, wq, wk, wv, w_o, gq, gk, cu, hq, hkv, head_dim=D,
                                                        eps=spec.eps, theta=spec.theta, rot_dim=spec.rot)
        return oracle.gated_attention_layer_prefill_rows(x, wq, wk, wv, w_o, gq, gk, rows, hq, hkv, head_dim=D,
                                                         eps=spec.eps, theta=spec.theta, rot_dim=spec.rot)
    # no output gate: plain heads of 256 and the gate saturated open (sigmoid = 1)
    q = oracle.split_heads(oracle.linear(x, wq), hq, D)
    k = oracle.split_heads(oracle.linear(x, wk), hkv, D)
    v = oracle.split_heads(oracle.linear(x, wv), hkv, D)
    o = oracle.gated_attention_prefill(q, np.full(q.shape, 40.0), k, v, gq, gk, cu, hq, hkv, eps=spec.eps,
                                       theta=spec.theta, rot_dim=spec.rot)
    return oracle.linear(oracle.merge_heads(o), w_o)


GATED_LAYER_SMALL = [
    # id, Hq, Hkv, lengths, hidden, rot
    (300, 16, 2, [1, 63, 64, 65, 200], 512, 64),   # the Qwen3-Next grouping (g = 8), tile edges, ragged tail
    (301, 4, 4, [130, 7], 256, 32),                 # g = 1
    (302, 8, 1, [257], 384, 128),                   # g = 8, hidden 3 x 128, rotary 128
]


@pytest.mark.parametrize("cid,hq,hkv,lengths,hidden,rot", GATED_LAYER_SMALL, ids=[str(c[0]) for c in GATED_LAYER_SMALL])
@pytest.mark.parametrize("with_cache", [False, True])
def test_gated_layer_small(cid, hq, hkv, lengths, hidden, rot, with_cache):
    spec, x, w_qkv, w_o, gq, gk = _inputs(cid, hq, hkv, lengths, hidden, rot)
    U.say(f"gated sublayer {cid} Hq={hq} Hkv={hkv} lengths={lengths} hidden={hidden} rot={rot} cache={with_cache}")
    p = _params(spec)
    cu = spec.cu_seqlens()
    kc = vc = None
    if with_cache:
        kc = torch.full((spec.n_seq, hkv, max(lengths) + 5, D), 7.0, dtype=BF, device=U.DEV)
        vc = torch.full_like(kc, 7.0)
    y = B.attention_layer(p, U.up(x, BF), U.up(w_qkv, BF), U.up(w_o, BF), U.up(gq, BF), U.up(gk, BF),
                          torch.from_numpy(cu).to(U.DEV), cu, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    ref = _oracle(spec, x, w_qkv, w_o, gq, gk, cu)
    err = np.abs(U.down(y) - ref)
    print(f"gated layer {cid}: max {err.max():.3e} mean {err.mean():.3e} (|y_ref| max {np.abs(ref).max():.2f})")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    if with_cache:
        qw = hq * 2 * D
        wk, wv = w_qkv[qw:qw + hkv * D], w_qkv[qw + hkv * D:]
        kref = x.astype(np.float64) @ wk.astype(np.float64).T
        kb = 2.0 ** -8 * np.abs(kref) + hidden * 2.0 ** -23 * (np.abs(x).astype(np.float64) @
                                                                  np.abs(wk).astype(np.float64).T)
        vref = x.astype(np.float64) @ wv.astype(np.float64).T
        vb = 2.0 ** -8 * np.abs(vref) + hidden * 2.0 ** -23 * (np.abs(x).astype(np.float64) @
                                                                  np.abs(wv).astype(np.float64).T)
        for s in range(spec.n_seq):
            a, b = cu[s], cu[s + 1]
            L = b - a
            kr3 = kref[a:b].reshape(L, hkv, D)
            kh = oracle.gated_qk_norm_rope(kr3, gk, np.arange(L), spec.eps, spec.theta, rot)
            got_k = U.down(kc[s, :, :L].permute(1, 0, 2))
            # the projection error carried through the norm (first order) and the
            # rotation, with the scale 1 + w, plus one rounding to bf16
            rms = np.sqrt(np.mean(kr3 ** 2, axis=-1, keepdims=True) + spec.eps)
            emax = kb[a:b].reshape(L, hkv, D).max(axis=-1, keepdims=True)
            kbound = 2.0 * np.abs(1.0 + gk).max() * (emax / rms) * (1.0 + np.abs(kr3).max(axis=-1, keepdims=True) / rms) \
                + 2.0 ** -8 * np.abs(kh) + 1e-6
            assert np.all(np.abs(got_k - kh) <= kbound), np.abs(got_k - kh).max()
            got_v = U.down(vc[s, :, :L].permute(1, 0, 2))
            assert np.all(np.abs(got_v - vref[a:b].reshape(L, hkv, D)) <= vb[a:b].reshape(L, hkv, D))
            assert bool((kc[s, :, L:] == 7.0).all()) and bool((vc[s, :, L:] == 7.0).all())


def test_gated_layer_without_output_gate():
    """head_dim 256 with output_gate = 0: q_proj gives head_dim values per head
    (no gate rows) and the attention output goes to o_proj as it is."""
    spec, x, w_qkv, w_o, gq, gk = _inputs(303, 8, 2, [100, 37], 256, 64, gate=False)
    U.say("gated sublayer without the output gate")
    p = _params(spec, gate=False)
    cu = spec.cu_seqlens()
    y = B.attention_layer(p, U.up(x, BF), U.up(w_qkv, BF), U.up(w_o, BF), U.up(gq, BF), U.up(gk, BF),
                          torch.from_numpy(cu).to(U.DEV), cu)
    torch.cuda.synchronize()
    ref = _oracle(spec, x, w_qkv, w_o, gq, gk, cu, gate=False)
    err = np.abs(U.down(y) - ref)
    print(f"ungated d256 layer: max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_gated_layer_append_in_chunks_equals_one_pass():
    """A prompt through the gated sublayer in ragged chunks (with the cache)
    gives the one-pass rows bit for bit, and the oracle's append rows."""
    spec, x, w_qkv, w_o, gq, gk = _inputs(304, 16, 2, [190, 77], 256, 64)
    U.say("gated sublayer: chunked append vs one pass")
    p = _params(spec)
    cu = spec.cu_seqlens()
    cap = 200
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(U.DEV)
    args = (U.up(w_qkv, BF), U.up(w_o, BF), U.up(gq, BF), U.up(gk, BF))
    kc1 = torch.zeros(2, 2, cap, D, dtype=BF, device=U.DEV)
    vc1 = torch.zeros_like(kc1)
    y1 = B.attention_layer(p, U.up(x, BF), *args, dev(cu), cu, k_cache=kc1, v_cache=vc1)
    kc2, vc2 = torch.zeros_like(kc1), torch.zeros_like(kc1)
    splits = [[0, 64, 65, 190], [0, 1, 77]]
    y2 = torch.empty_like(y1)
    for c in range(3):
        lo = [sp[min(c, len(sp) - 1)] for sp in splits]
        hi = [sp[min(c + 1, len(sp) - 1)] for sp in splits]
        new = [h - l for l, h in zip(lo, hi)]
        rows = np.concatenate([np.arange(cu[s] + lo[s], cu[s] + hi[s]) for s in range(2)]).astype(np.int64)
        if len(rows) == 0:
            continue
        cu_new = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
        sp_h = np.array(lo, dtype=np.int32)
        yc = B.attention_layer(p, U.up(x[rows], BF), *args, dev(cu_new), cu_new, start_pos=dev(sp_h),
                               start_pos_host=sp_h, k_cache=kc2, v_cache=vc2)
        y2[torch.from_numpy(rows).to(U.DEV)] = yc
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)
    # and the oracle's append of the last chunk of sequence 0 (65 cached tokens, 125 new)
    qw = 16 * 2 * D
    wq, wk, wv = w_qkv[:qw], w_qkv[qw:qw + 2 * D], w_qkv[qw + 2 * D:]
    kh = oracle.gated_qk_norm_rope((x[:65] @ wk.T.astype(np.float64)).reshape(65, 2, D), gk, np.arange(65), spec.eps,
                                   spec.theta, 64)
    vv = (x[:65] @ wv.T.astype(np.float64)).reshape(65, 2, D)
    ref, _, _ = oracle.gated_attention_layer_append(x[65:190], wq, wk, wv, w_o, gq, gk, kh, vv, 65, 16, 2, head_dim=D,
                                                    eps=spec.eps, theta=spec.theta, rot_dim=64)
    err = np.abs(U.down(y2[65:190]) - ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())


def test_gated_layer_full_size_sampled():
    """The Qwen3-Next-80B-A3B gated sublayer (hidden 2048, 16 / 2 heads of 256,
    rotary 64, theta 1e7) at 4 x 4096 tokens, in the launch configuration the
    benchmark times: sampled rows of one sequence against the oracle, and
    run-to-run determinism."""
    spec = inputs.gated_layer_case_spec()
    hidden = inputs.LAYER_HIDDEN[spec.case_id]
    U.say("gated sublayer full size 4x4096 hidden 2048")
    w_qkv, w_o = inputs.layer_weights(spec, hidden)
    x = inputs.layer_x(spec, hidden)
    gq, gk = inputs.gammas(spec)
    p = _params(spec)
    cu = spec.cu_seqlens()
    kc = torch.empty(4, 2, 4096, D, dtype=BF, device=U.DEV)
    vc = torch.empty_like(kc)
    args = (p, U.up(x, BF), U.up(w_qkv, BF), U.up(w_o, BF), U.up(gq, BF), U.up(gk, BF),
            torch.from_numpy(cu).to(U.DEV), cu)
    y = B.attention_layer(*args, k_cache=kc, v_cache=vc)
    y2 = B.attention_layer(*args, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    s = 3
    rows = U.sample_rows(4096, np.random.default_rng(13), n_blocks=1, block=8)
    U.say(f"  oracle rows of sequence {s}: {len(rows)}")
    xs = inputs.layer_x(spec, hidden, seq=s, lo=0, hi=int(rows.max()) + 1)
    ref = _oracle(spec, xs, w_qkv, w_o, gq, gk, None, rows=rows)
    got = U.down(y[cu[s] + torch.from_numpy(rows).to(U.DEV)])
    err = np.abs(got - ref)
    print(f"gated sublayer full size: max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_gated_layer_rope_then_norm():
    """order = 1 at head_dim 256: the projection's key epilogue and the core's
    query prologue rotate first and norm after (scale 1 + w applied after the
    rotation).  Reference composed from the oracle's pinned pieces: the gated
    projections, rope_partial, rms_norm_zero_centred, causal_softmax per head
    with its KV group, sigmoid(gate), o_proj; the cached K̂ checked as well."""
    hq, hkv, lengths, hidden, rot = 8, 2, [70, 129], 256, 64
    spec, x, w_qkv, w_o, gq, gk = _inputs(305, hq, hkv, lengths, hidden, rot)
    U.say("gated sublayer, RoPE then norm")
    p = _params(spec)
    p.order = 1
    cu = spec.cu_seqlens()
    kc = torch.zeros(spec.n_seq, hkv, max(lengths), D, dtype=BF, device=U.DEV)
    vc = torch.zeros_like(kc)
    y = B.attention_layer(p, U.up(x, BF), U.up(w_qkv, BF), U.up(w_o, BF), U.up(gq, BF), U.up(gk, BF),
                          torch.from_numpy(cu).to(U.DEV), cu, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    qw = hq * 2 * D
    q, gate, k, v = oracle.gated_qkv_projection(x, w_qkv[:qw], w_qkv[qw:qw + hkv * D], w_qkv[qw + hkv * D:], hq, hkv)
    o = np.zeros(q.shape)
    for s in range(spec.n_seq):
        a, b = cu[s], cu[s + 1]
        pos = np.arange(b - a)
        qh = oracle.rms_norm_zero_centred(oracle.rope_partial(q[a:b], pos, spec.theta, rot), gq, spec.eps)
        kh = oracle.rms_norm_zero_centred(oracle.rope_partial(k[a:b], pos, spec.theta, rot), gk, spec.eps)
        for t in range(hq):
            u = oracle.kv_head_for_q_head(t, hq, hkv)
            pr = oracle.causal_softmax(qh[:, t] @ kh[:, u].T / np.sqrt(D), pos, pos)
            o[a:b, t] = (pr @ v[a:b, u]) * oracle.sigmoid(gate[a:b, t])
        # the projection's fp32 error carried through the rotation (norm-preserving)
        # and the norm to first order, with the scale 1 + w, plus one bf16 rounding
        wk = w_qkv[qw:qw + hkv * D].astype(np.float64)
        kb = (hidden * 2.0 ** -23 * (np.abs(x[a:b]).astype(np.float64) @ np.abs(wk).T)).reshape(b - a, hkv, D)
        kr = k[a:b]
        rms = np.sqrt(np.mean(kr ** 2, axis=-1, keepdims=True) + spec.eps)
        kbound = 2.0 * np.abs(1.0 + gk).max() * (kb.max(axis=-1, keepdims=True) / rms) * \
            (1.0 + np.abs(kr).max(axis=-1, keepdims=True) / rms) + 2.0 ** -8 * np.abs(kh) + 1e-6
        got_k = U.down(kc[s, :, :b - a].permute(1, 0, 2))
        assert np.all(np.abs(got_k - kh) <= kbound), np.abs(got_k - kh).max()
    ref = oracle.linear(oracle.merge_heads(o), w_o)
    err = np.abs(U.down(y) - ref)
    print(f"gated layer rope->norm: max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
