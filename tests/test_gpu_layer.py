"""GPU parity of the attention sublayer (q/k/v projections with the fused
QK-Norm + RoPE + cache-write epilogue, the core, o_proj) and of the bf16
linear map, against the CPU oracle (``oracle.layer``), through the C-ABI.

Tolerances:
  * linear: every output within 2^-8 |y_ref| + k 2^-23 sum_i |x_i w_i| (fp32
    accumulation of exact bf16 products, then one rounding to bf16, with a
    factor 2 of slack on both terms);
  * cached K̂ and V from the fused projection: the same bound on the
    projection, carried through the norm and rotation (one rounding to bf16);
  * sublayer output y: per element max 2e-2 and mean 2e-3 (the bf16 gate of
    the core).  x ~ N(0,1) and weights N(0,1)/sqrt(fan-in) give q, k, v and y
    unit scale; y's error is the attention output's error mixed by o_proj's
    rows of unit norm, which keeps its scale, plus one bf16 rounding.
Chunked appends through the sublayer equal one pass bit for bit."""

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


def linear_bound(x, w, k):
    """2^-8 |y| + k 2^-23 (|x| |w|^T), elementwise (float64)."""
    y = x.astype(np.float64) @ w.astype(np.float64).T
    mag = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    return y, 2.0 ** -8 * np.abs(y) + k * 2.0 ** -23 * mag


# Every width takes the four-wave tile form: one, two and an odd number of K
# steps, ragged last row and column tiles (a column tile of 128), the q/k/v
# width of Qwen3-8B.  The last five shapes take the XCD block walks over
# 256 x 256 tiles: 4 x 8 blocks in 4 x 2 regions (one and two block columns per
# region), and 8 x 4 blocks in 8 x 1 regions with the per-XCD column-block
# rotation (one, three and six block columns).  The eight-wave form serves the
# q/k/v epilogues, tested with the sublayers.
@pytest.mark.parametrize("m,n,k", [(1, 128, 64), (255, 384, 128), (257, 256, 1024), (1000, 640, 320),
                                   (4096, 1024, 4096), (1, 4096, 64), (257, 4224, 128), (1000, 4096, 320),
                                   (300, 6144, 4096), (4096, 4096, 64), (4096, 8192, 64), (16384, 1024, 64),
                                   (16384, 3072, 64), (16384, 6144, 64)])
def test_linear(m, n, k):
    rng = np.random.default_rng(m + n + k)
    x = inputs.round_to_bf16(rng.standard_normal((m, k)).astype(np.float32))
    w = inputs.round_to_bf16((rng.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32))
    U.say(f"linear m={m} n={n} k={k}")
    y = B.linear(U.up(x, BF), U.up(w, BF))
    torch.cuda.synchronize()
    ref, bound = linear_bound(x, w, k)
    err = np.abs(U.down(y) - ref)
    print(f"linear {m}x{n}x{k}: max err {err.max():.3e}, max err / bound {(err / bound).max():.3f}")
    assert np.all(err <= bound)


def _layer_inputs(cid, hq, hkv, lengths, hidden, theta=1e6):
    spec = inputs.custom_spec(cid, "bf16", hq, hkv, lengths, theta=theta)
    w_qkv, w_o = inputs.layer_weights(spec, hidden)
    x = inputs.layer_x(spec, hidden)
    gq, gk = inputs.gammas(spec)
    return spec, x, w_qkv, w_o, gq, gk


def _split_w(spec, w_qkv):
    d = spec.head_dim
    a, b = spec.n_q_heads * d, (spec.n_q_heads + spec.n_kv_heads) * d
    return w_qkv[:a], w_qkv[a:b], w_qkv[b:]


LAYER_SMALL = [
    # id, Hq, Hkv, lengths, hidden
    (200, 4, 2, [1, 63, 64, 65, 200], 256),   # g = 2, tile edges, a ragged tail of the token tiles
    (201, 16, 8, [300, 129], 1024),            # the Qwen3-0.6B head geometry (hidden 1024, q width 2048)
    (202, 8, 1, [257], 384),                   # g = 8, hidden 3 x 128
]


@pytest.mark.parametrize("cid,hq,hkv,lengths,hidden", LAYER_SMALL, ids=[str(c[0]) for c in LAYER_SMALL])
@pytest.mark.parametrize("with_cache", [False, True])
def test_attention_layer_small(cid, hq, hkv, lengths, hidden, with_cache):
    spec, x, w_qkv, w_o, gq, gk = _layer_inputs(cid, hq, hkv, lengths, hidden)
    U.say(f"attention layer case {cid} Hq={hq} Hkv={hkv} lengths={lengths} hidden={hidden} cache={with_cache}")
    p = U.params(spec)
    cu = spec.cu_seqlens()
    kc = vc = None
    if with_cache:
        kc = torch.full((spec.n_seq, hkv, max(lengths) + 5, 128), 7.0, dtype=BF, device=U.DEV)
        vc = torch.full_like(kc, 7.0)
    y = B.attention_layer(p, U.up(x, BF), U.up(w_qkv, BF), U.up(w_o, BF), U.up(gq, BF), U.up(gk, BF),
                          torch.from_numpy(cu).to(U.DEV), cu, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    wq, wk, wv = _split_w(spec, w_qkv)
    ref = oracle.attention_layer_prefill(x, wq, wk, wv, w_o, gq, gk, cu, hq, hkv, eps=spec.eps, theta=spec.theta)
    got = U.down(y)
    err = np.abs(got - ref)
    print(f"layer {cid}: max {err.max():.3e} mean {err.mean():.3e} (|y_ref| max {np.abs(ref).max():.2f})")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    if with_cache:
        # K̂ and V in the cache: the fused projection's epilogue, checked per token
        kref, kb = linear_bound(x, wk, hidden)
        vref, vb = linear_bound(x, wv, hidden)
        for s in range(spec.n_seq):
            a, b = cu[s], cu[s + 1]
            L = b - a
            kh = oracle.qk_norm_rope(kref[a:b].reshape(L, hkv, 128), gk, np.arange(L), spec.eps, spec.theta)
            got_k = U.down(kc[s, :, :L].permute(1, 0, 2))
            # First-order propagation of the projection error e (|e_i| <= eps_i) through
            # the norm and the rotation.  k/r(k), r = sqrt(mean k^2 + eps), moves by
            # e_i/r - k_i (k.e)/(d r^3), and |k.e| <= |k| |e| <= sqrt(d) r sqrt(d) max eps,
            # so each coordinate moves by at most (max eps / r)(1 + max_i |k_i| / r);
            # the rotation adds two coordinates (|cos| + |sin| <= 2 with gamma),
            # and the result is rounded once to bf16 (2^-9 |k|, doubled for slack).
            kr3 = kref[a:b].reshape(L, hkv, 128)
            rms = np.sqrt(np.mean(kr3 ** 2, axis=-1, keepdims=True) + spec.eps)
            emax = kb[a:b].reshape(L, hkv, 128).max(axis=-1, keepdims=True)
            kbound = 2.0 * np.abs(gk).max() * (emax / rms) * (1.0 + np.abs(kr3).max(axis=-1, keepdims=True) / rms) \
                + 2.0 ** -8 * np.abs(kh) + 1e-6
            assert np.all(np.abs(got_k - kh) <= kbound), np.abs(got_k - kh).max()
            got_v = U.down(vc[s, :, :L].permute(1, 0, 2))
            assert np.all(np.abs(got_v - vref[a:b].reshape(L, hkv, 128)) <= vb[a:b].reshape(L, hkv, 128))
            assert bool((kc[s, :, L:] == 7.0).all()) and bool((vc[s, :, L:] == 7.0).all())


def test_attention_layer_append_in_chunks_equals_one_pass():
    """A prompt run through the sublayer in ragged chunks (with the cache) gives
    the one-pass rows bit for bit, and the oracle's append rows."""
    spec, x, w_qkv, w_o, gq, gk = _layer_inputs(203, 8, 2, [190, 77], 256)
    U.say("attention layer: chunked append vs one pass")
    p = U.params(spec)
    cu = spec.cu_seqlens()
    cap = 200
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(U.DEV)
    args = (U.up(w_qkv, BF), U.up(w_o, BF), U.up(gq, BF), U.up(gk, BF))
    kc1 = torch.zeros(2, 2, cap, 128, dtype=BF, device=U.DEV)
    vc1 = torch.zeros_like(kc1)
    y1 = B.attention_layer(p, U.up(x, BF), *args, dev(cu), cu, k_cache=kc1, v_cache=vc1)
    kc2 = torch.zeros_like(kc1)
    vc2 = torch.zeros_like(kc1)
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
    wq, wk, wv = _split_w(spec, w_qkv)
    kh = oracle.qk_norm_rope((x[:65] @ wk.T.astype(np.float64)).reshape(65, 2, 128), gk, np.arange(65), spec.eps,
                             spec.theta)
    vv = (x[:65] @ wv.T.astype(np.float64)).reshape(65, 2, 128)
    ref, _, _ = oracle.attention_layer_append(x[65:190], wq, wk, wv, w_o, gq, gk, kh, vv, 65, 8, 2, eps=spec.eps,
                                              theta=spec.theta)
    err = np.abs(U.down(y2[65:190]) - ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())


def test_attention_layer_full_size_sampled():
    """The Qwen3-8B sublayer (hidden 4096, 32 / 8 heads) at 4 x 4096 tokens, in
    the launch configuration the benchmark times: sampled rows of one sequence
    against the oracle, and run-to-run determinism."""
    spec = inputs.layer_case_spec()
    hidden = inputs.LAYER_HIDDEN[spec.case_id]
    U.say("attention layer full size 4x4096 hidden 4096")
    w_qkv, w_o = inputs.layer_weights(spec, hidden)
    x = inputs.layer_x(spec, hidden)
    gq, gk = inputs.gammas(spec)
    p = U.params(spec)
    cu = spec.cu_seqlens()
    kc = torch.empty(4, 8, 4096, 128, dtype=BF, device=U.DEV)
    vc = torch.empty_like(kc)
    args = (p, U.up(x, BF), U.up(w_qkv, BF), U.up(w_o, BF), U.up(gq, BF), U.up(gk, BF),
            torch.from_numpy(cu).to(U.DEV), cu)
    y = B.attention_layer(*args, k_cache=kc, v_cache=vc)
    y2 = B.attention_layer(*args, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    s = 2
    rows = U.sample_rows(4096, np.random.default_rng(12), n_blocks=1, block=8)
    wq, wk, wv = _split_w(spec, w_qkv)
    ref = oracle.attention_layer_prefill_rows(x[cu[s]:cu[s + 1]], wq, wk, wv, w_o, gq, gk, rows, 32, 8,
                                              eps=spec.eps, theta=spec.theta)
    got = U.down(y[cu[s] + torch.from_numpy(rows).to(U.DEV)])
    err = np.abs(got - ref)
    print(f"layer full size seq {s}: max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
