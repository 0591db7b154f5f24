"""GPU parity of the gated global-attention layer (Qwen3-Next / Qwen3.5: head_dim
256, zero-centred QK-Norm, partial RoPE, per-head sigmoid output gate) against
the CPU oracle (``oracle.gated``), through the C-ABI.

The kernels read the query and the gate from the q_proj output layout (per
head the query, then the gate), which the tests build with
``inputs.q_proj_rows``; the oracle takes the two halves separately.

Tolerances as for the Qwen3 layers: fp32 inputs max-abs 1e-4 (raw); bf16
inputs, per query head, max |o - o_ref| / max(1, s_v) <= 2e-2 and mean <= 2e-3
(the gate scales every output by at most 1, so the bound carries over).  Cache
writes are checked bit for bit against the library's own norm+RoPE entry."""

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


def gparams(spec, **kw):
    kw.setdefault("rotary_dim", spec.rot)
    return B.make_gated_params(spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, rope_theta=spec.theta, **kw)


def check(got, ref, spec, label):
    if spec.dtype == "f32":
        err = np.abs(got - ref).max()
        print(f"{label}: max {err:.3e}")
        assert err <= 1e-4, (label, err)
    else:
        print(U.bf16_gate(got, ref, spec, label=label))


def q_proj(x):
    return inputs.q_proj_rows(x["q"], x["gate"])


# ------------------------------------------------------------------ norm + partial RoPE

@pytest.mark.parametrize("dtype,rot,order", [("f32", 64, 0), ("bf16", 64, 0), ("bf16", 32, 0), ("f32", 128, 0),
                                             ("bf16", 256, 0), ("f32", 64, 1), ("bf16", 64, 1)])
def test_gated_qk_norm_rope(dtype, rot, order):
    spec = inputs.gated_spec(160 + rot + order, dtype, 4, 2, [37, 300], rot=rot)
    x = inputs.prefill_inputs(spec)
    rng = np.random.default_rng(5)
    pos = np.concatenate([np.arange(37), rng.integers(0, 262144, size=300)]).astype(np.int32)
    U.say(f"gated qk_norm_rope {dtype} rot={rot} order={order} n_tok={len(pos)}")
    dt = U.torch_dtype(spec)
    qo, ko = B.qk_norm_rope(gparams(spec, order=order), U.up(q_proj(x), dt), U.up(x["k"], dt),
                            U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt), torch.from_numpy(pos).to(U.DEV))
    torch.cuda.synchronize()
    assert qo.shape == (len(pos), 4, 256)
    for got, raw, w, name in ((qo, x["q"], x["q_gamma"], "q"), (ko, x["k"], x["k_gamma"], "k")):
        if order == 0:
            ref = oracle.gated_qk_norm_rope(raw, w, pos, spec.eps, spec.theta, rot)
        else:  # RoPE first, then the zero-centred norm
            ref = oracle.rms_norm_zero_centred(oracle.rope_partial(raw, pos, spec.theta, rot), w, spec.eps)
        got = U.down(got)
        err = np.abs(got - ref)
        if dtype == "f32":
            assert err.max() <= 2e-5, (name, err.max())
        else:  # one rounding to bf16: half an ulp of the value, plus fp32 slack
            assert np.all(err <= np.abs(ref) * 2.0 ** -8 + 1e-5), (name, err.max())
        if rot < 256:  # the coordinates past rot are only normed
            tail = oracle.rms_norm_zero_centred(raw, w, spec.eps)[..., rot:]
            assert np.abs(got[..., rot:] - tail).max() <= (2e-5 if dtype == "f32" else
                                                            2.0 ** -8 * np.abs(tail).max())


# ------------------------------------------------------------------ prefill

GATED_PREFILL = [
    # id, dtype, Hq, Hkv, lengths, rot
    (170, "bf16", 16, 2, [1, 63, 64, 65, 200, 517], 64),   # g = 8 (Qwen3-Next grouping), tile edges, ragged tail
    (171, "bf16", 8, 8, [130, 7], 64),                      # g = 1
    (172, "bf16", 16, 1, [260], 64),                        # g = 16
    (173, "bf16", 24, 4, [97, 250], 32),                    # g = 6
    (174, "bf16", 8, 2, [150, 33], 256),                    # full rotation
    (175, "bf16", 128, 1, [40, 3], 128),                    # g = 128: one token per workgroup
    (176, "f32", 16, 2, [1, 65, 200], 64),
    (177, "f32", 4, 4, [77], 256),
]


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths,rot", GATED_PREFILL, ids=[str(c[0]) for c in GATED_PREFILL])
def test_gated_prefill_small(cid, dtype, hq, hkv, lengths, rot):
    run_gated_prefill(cid, dtype, hq, hkv, lengths, rot)


def run_gated_prefill(cid, dtype, hq, hkv, lengths, rot):
    spec = inputs.gated_spec(cid, dtype, hq, hkv, lengths, rot=rot)
    x = inputs.prefill_inputs(spec)
    U.say(f"gated prefill case {cid} {dtype} Hq={hq} Hkv={hkv} lengths={lengths} rot={rot}")
    dt = U.torch_dtype(spec)
    cu = torch.from_numpy(x["cu_seqlens"]).to(U.DEV)
    out = B.prefill(gparams(spec), U.up(q_proj(x), dt), U.up(x["k"], dt), U.up(x["v"], dt),
                    U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt), cu, x["cu_seqlens"])
    torch.cuda.synchronize()
    ref = oracle.gated_attention_prefill(x["q"], x["gate"], x["k"], x["v"], x["q_gamma"], x["k_gamma"],
                                         x["cu_seqlens"], hq, hkv, eps=spec.eps, theta=spec.theta, rot_dim=rot)
    check(U.down(out), ref, spec, f"gated prefill {cid}")


def test_gated_prefill_large_magnitude_v():
    """V times 2^118 on the head_dim-256 kernel's static-bound path: its weights
    2^(score - B) are <= 1, so the fp32 accumulators stay finite.  The output
    divided by 2^118 meets the literal bounds (the gate scales by at most 1)."""
    spec = inputs.gated_spec(179, "bf16", 16, 2, [1, 65, 200, 517], rot=64, v_scaled=False)
    x = dict(inputs.prefill_inputs(spec))
    big = 2.0 ** 118
    x["v"] = (x["v"] * np.float32(big)).astype(np.float32)
    U.say("gated prefill, large-magnitude V")
    dt = torch.bfloat16
    cu = torch.from_numpy(x["cu_seqlens"]).to(U.DEV)
    out = B.prefill(gparams(spec), U.up(q_proj(x), dt), U.up(x["k"], dt), U.up(x["v"], dt),
                    U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt), cu, x["cu_seqlens"])
    torch.cuda.synchronize()
    ref = oracle.gated_attention_prefill(x["q"], x["gate"], x["k"], x["v"], x["q_gamma"], x["k_gamma"],
                                         x["cu_seqlens"], 16, 2, eps=spec.eps, theta=spec.theta, rot_dim=64)
    got = U.down(out)
    assert np.isfinite(got).all()
    err = np.abs(got - ref) / big
    print(f"gated large V: max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_dim_256_without_gate(dtype):
    """output_gate = 0: the plain attention of the head_dim-256 layer (the
    oracle's gate saturated at +inf, where sigmoid is exactly 1), q given
    without gate halves; also with the plain norm scale (norm_offset 0)."""
    spec = inputs.gated_spec(178, dtype, 8, 2, [90, 140], rot=64)
    x = inputs.prefill_inputs(spec)
    dt = U.torch_dtype(spec)
    cu = torch.from_numpy(x["cu_seqlens"]).to(U.DEV)
    inf = np.full(x["q"].shape, np.inf)
    for offset in (1.0, 0.0):
        U.say(f"head_dim 256 prefill without gate, {dtype}, norm_offset={offset}")
        p = gparams(spec, output_gate=0)
        p.norm_offset = offset
        w = 1.0 + x["q_gamma"] if offset == 0.0 else x["q_gamma"]  # scale 1 + w either way
        wk = 1.0 + x["k_gamma"] if offset == 0.0 else x["k_gamma"]
        out = B.prefill(p, U.up(x["q"], dt), U.up(x["k"], dt), U.up(x["v"], dt), U.up(w, dt), U.up(wk, dt), cu,
                        x["cu_seqlens"])
        torch.cuda.synchronize()
        if dtype == "bf16" and offset == 0.0:  # 1 + w rounded to bf16 is what the kernel saw
            w_used, wk_used = inputs.round_to_bf16(w.astype(np.float32)) - 1.0, \
                inputs.round_to_bf16(wk.astype(np.float32)) - 1.0
        else:
            w_used, wk_used = x["q_gamma"], x["k_gamma"]
        ref = oracle.gated_attention_prefill(x["q"], inf, x["k"], x["v"], w_used, wk_used, x["cu_seqlens"], 8, 2,
                                             eps=spec.eps, theta=spec.theta, rot_dim=64)
        check(U.down(out), ref, spec, f"no gate, offset {offset}")


def test_gated_prefill_online_softmax_path():
    """Norm weights lifted so that the logit bound exceeds the static-bound
    limit: the kernel takes the online softmax (one entry of each weight is
    raised, so the bf16 error stays that of the Qwen3 case)."""
    spec = inputs.gated_spec(179, "bf16", 16, 2, [300, 129], rot=64)
    x = inputs.prefill_inputs(spec)
    x["q_gamma"] = x["q_gamma"].copy()
    x["k_gamma"] = x["k_gamma"].copy()
    x["q_gamma"][5] = 1.0   # scale 2
    x["k_gamma"][70] = 0.75  # scale 1.75: bound ~ 0.0902 * 256 * 3.5 > 60
    U.say("gated prefill, online softmax path")
    dt = torch.bfloat16
    cu = torch.from_numpy(x["cu_seqlens"]).to(U.DEV)
    out = B.prefill(gparams(spec), U.up(q_proj(x), dt), U.up(x["k"], dt), U.up(x["v"], dt),
                    U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt), cu, x["cu_seqlens"])
    torch.cuda.synchronize()
    ref = oracle.gated_attention_prefill(x["q"], x["gate"], x["k"], x["v"], x["q_gamma"], x["k_gamma"],
                                         x["cu_seqlens"], 16, 2, eps=spec.eps, theta=spec.theta, rot_dim=64)
    check(U.down(out), ref, spec, "gated online")


def test_gated_prefill_full_size_sampled():
    """A Qwen3-Next global layer at 4 x 4096 tokens (16 query heads, 2 KV heads,
    head_dim 256, rot 64), in the launch configuration the benchmark times;
    sampled rows of every sequence against the oracle, plus first-row and
    determinism checks."""
    spec = inputs.gated_case_spec(inputs.GATED_PREFILL_CASE)
    x = inputs.prefill_inputs(spec)
    U.say("gated prefill full size 4x4096 16/2 d256")
    dt = torch.bfloat16
    cu = torch.from_numpy(x["cu_seqlens"]).to(U.DEV)
    args = (gparams(spec), U.up(q_proj(x), dt), U.up(x["k"], dt), U.up(x["v"], dt), U.up(x["q_gamma"], dt),
            U.up(x["k_gamma"], dt), cu, x["cu_seqlens"])
    out = B.prefill(*args)
    out2 = B.prefill(*args)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    got = U.down(out)
    rng = np.random.default_rng(11)
    heads = [0, 7, 8, 15]
    for s in range(spec.n_seq):
        rows = U.sample_rows(4096, rng, n_blocks=1, block=8)
        a = int(x["cu_seqlens"][s])
        ref = oracle.gated_attention_prefill_rows(x["q"][a + rows], x["gate"][a + rows], x["k"][a:a + 4096],
                                                  x["v"][a:a + 4096], x["q_gamma"], x["k_gamma"], rows, heads,
                                                  16, 2, eps=spec.eps, theta=spec.theta, rot_dim=64)
        print(U.bf16_gate(got[a + rows][:, heads], ref, spec, heads=heads, label=f"seq {s}"))


# ------------------------------------------------------------------ append and decode

def _gated_cache(spec, x, kraw, vraw, capacity):
    """Cache tensors holding, per sequence, the keys normed and rotated by the
    library's own norm+RoPE entry, and the raw values."""
    dt = U.torch_dtype(spec)
    kc = torch.full((spec.n_seq, spec.n_kv_heads, capacity, 256), 7.0, dtype=dt, device=U.DEV)
    vc = torch.full_like(kc, 7.0)
    for i, (kr, vr) in enumerate(zip(kraw, vraw)):
        L = kr.shape[0]
        if L == 0:
            continue
        pos = torch.arange(L, dtype=torch.int32, device=U.DEV)
        _, kh = B.qk_norm_rope(gparams(spec), None, U.up(kr, dt), None, U.up(x["k_gamma"], dt), pos)
        kc[i, :, :L] = kh.permute(1, 0, 2)
        vc[i, :, :L] = U.up(vr, dt).permute(1, 0, 2)
    torch.cuda.synchronize()
    return kc, vc


GATED_APPEND = [
    # id, dtype, Hq, Hkv, lengths (prefix + new), prefix lengths
    (180, "bf16", 16, 2, [300, 70, 400, 5], [37, 0, 256, 4]),
    (181, "f32", 8, 2, [150, 70], [64, 3]),
]


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths,splits", GATED_APPEND, ids=[str(c[0]) for c in GATED_APPEND])
def test_gated_append(cid, dtype, hq, hkv, lengths, splits):
    run_gated_append(cid, dtype, hq, hkv, lengths, splits, 64)


def run_gated_append(cid, dtype, hq, hkv, lengths, splits, rot):
    spec = inputs.gated_spec(cid, dtype, hq, hkv, lengths, rot=rot)
    x = inputs.prefill_inputs(spec)
    U.say(f"gated append case {cid} {dtype} Hq={hq} Hkv={hkv} lengths={lengths} prefixes={splits} rot={rot}")
    cu = x["cu_seqlens"]
    qp = q_proj(x)
    kc, vc = _gated_cache(spec, x, [x["k"][cu[s]:cu[s] + splits[s]] for s in range(spec.n_seq)],
                          [x["v"][cu[s]:cu[s] + splits[s]] for s in range(spec.n_seq)], max(lengths) + 9)
    new = [lengths[s] - splits[s] for s in range(spec.n_seq)]
    cu_new = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    sel = np.concatenate([np.arange(cu[s] + splits[s], cu[s + 1]) for s in range(spec.n_seq)]).astype(np.int64)
    dt = U.torch_dtype(spec)
    sp = np.asarray(splits, dtype=np.int32)
    out = B.append(gparams(spec), U.up(qp[sel], dt), U.up(x["k"][sel], dt), U.up(x["v"][sel], dt),
                   U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt), kc, vc, torch.from_numpy(sp).to(U.DEV),
                   torch.from_numpy(cu_new).to(U.DEV), sp, cu_new)
    torch.cuda.synchronize()
    ref = []
    for s in range(spec.n_seq):
        a, b, c = cu[s], cu[s] + splits[s], cu[s + 1]
        kh = oracle.gated_qk_norm_rope(x["k"][a:b], x["k_gamma"], np.arange(splits[s]), spec.eps, spec.theta, rot)
        o, _ = oracle.gated_attention_append(x["q"][b:c], x["gate"][b:c], x["k"][b:c], x["v"][b:c], x["q_gamma"],
                                             x["k_gamma"], kh, x["v"][a:b], splits[s], hq, hkv, eps=spec.eps,
                                             theta=spec.theta, rot_dim=rot)
        ref.append(o)
    check(U.down(out), np.concatenate(ref), spec, f"gated append {cid}")
    # the cache holds every token's rotated key and its value, and nothing past the sequence
    for s in range(spec.n_seq):
        L = lengths[s]
        pos = torch.arange(L, dtype=torch.int32, device=U.DEV)
        _, kh = B.qk_norm_rope(gparams(spec), None, U.up(x["k"][cu[s]:cu[s + 1]], dt), None,
                               U.up(x["k_gamma"], dt), pos)
        torch.cuda.synchronize()
        assert torch.equal(kc[s, :, :L], kh.permute(1, 0, 2))
        assert torch.equal(vc[s, :, :L], U.up(x["v"][cu[s]:cu[s + 1]], dt).permute(1, 0, 2))
        assert bool((kc[s, :, L:] == 7.0).all()) and bool((vc[s, :, L:] == 7.0).all())


GATED_DECODE = [
    (190, "bf16", 16, 2, [0, 1, 31, 32, 33, 127, 128, 1000, 2500]),
    (191, "bf16", 32, 2, [5, 700, 1029]),
    (192, "f32", 16, 2, [0, 1, 65, 300]),
]


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths", GATED_DECODE, ids=[str(c[0]) for c in GATED_DECODE])
def test_gated_decode(cid, dtype, hq, hkv, lengths):
    run_gated_decode(cid, dtype, hq, hkv, lengths, 64)


def run_gated_decode(cid, dtype, hq, hkv, lengths, rot):
    spec = inputs.gated_spec(cid, dtype, hq, hkv, lengths, kind="decode", rot=rot)
    x = inputs.decode_new_token(spec)
    U.say(f"gated decode case {cid} {dtype} Hq={hq} Hkv={hkv} lengths={lengths} rot={rot}")
    raws = inputs.decode_cache_raw_all(spec)
    kc, vc = _gated_cache(spec, x, [r[0] for r in raws], [r[1] for r in raws], max(lengths) + 7)
    dt = U.torch_dtype(spec)
    sp = x["start_pos"]
    out = B.decode(gparams(spec), U.up(q_proj(x), dt), U.up(x["k"], dt), U.up(x["v"], dt),
                   U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt), kc, vc, torch.from_numpy(sp).to(U.DEV), sp)
    torch.cuda.synchronize()
    ref = []
    for i, L in enumerate(lengths):
        kr, vr = raws[i]
        kh = oracle.gated_qk_norm_rope(kr, x["k_gamma"], np.arange(L), spec.eps, spec.theta, rot)
        o, _ = oracle.gated_attention_append(x["q"][i:i + 1], x["gate"][i:i + 1], x["k"][i:i + 1],
                                             x["v"][i:i + 1], x["q_gamma"], x["k_gamma"], kh, vr, L, hq, hkv,
                                             eps=spec.eps, theta=spec.theta, rot_dim=rot)
        ref.append(o[0])
    check(U.down(out), np.stack(ref), spec, f"gated decode {cid}")
    # the new key and value were appended at start_pos, rotated there
    for i, L in enumerate(lengths):
        _, kh = B.qk_norm_rope(gparams(spec), None, U.up(x["k"][i:i + 1], dt), None, U.up(x["k_gamma"], dt),
                               torch.tensor([L], dtype=torch.int32, device=U.DEV))
        torch.cuda.synchronize()
        assert torch.equal(kc[i, :, L], kh[0])
        assert torch.equal(vc[i, :, L], U.up(x["v"][i], dt))


# ------------------------------------------------------------------ seeded shape sweep

# group sizes the head_dim-256 tiles accept (128 bf16 prefill rows, 64 fp32
# rows, 16 decode rows) and the rotary widths of the boundary
SWEEP_PREFILL_G = {"bf16": [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24, 32, 64, 128], "f32": [1, 2, 3, 8, 16, 64]}
SWEEP_DECODE_G = {"bf16": [1, 2, 3, 4, 6, 8, 12, 16], "f32": [1, 3, 8]}
SWEEP_ROT = [32, 64, 128, 256]


def _sweep(kind, n_cases, first_id, dtypes):
    """Cases drawn from a fixed generator: each dtype walks a shuffled list of
    group sizes and rotary widths; 1-8 KV heads (at most 128 query heads);
    ragged lengths with about one empty sequence in ten; at least one new token."""
    rng = np.random.default_rng([0x6A7E, first_id])
    table = SWEEP_DECODE_G if kind == "decode" else SWEEP_PREFILL_G
    g_order = {d: [] for d in dtypes}
    r_order = {d: [] for d in dtypes}
    cases = []
    for i in range(n_cases):
        dtype = dtypes[i % len(dtypes)]
        if not g_order[dtype]:
            g_order[dtype] = [int(v) for v in rng.permutation(table[dtype])]
        if not r_order[dtype]:
            r_order[dtype] = [int(v) for v in rng.permutation(SWEEP_ROT)]
        g, rot = g_order[dtype].pop(), r_order[dtype].pop()
        hkv = int(rng.choice([h for h in (1, 2, 4, 8) if g * h <= 128]))
        n_max, l_max = (6, 2500) if kind == "decode" else (4, 500)
        while True:
            n = int(rng.integers(1, n_max + 1))
            lengths = rng.integers(1, l_max + 1, size=n)
            lengths[rng.random(n) < 0.1] = 0
            lengths = [int(v) for v in lengths]
            splits = [int(rng.integers(0, L + 1)) for L in lengths]
            if kind == "decode" or sum(lengths) - (sum(splits) if kind == "append" else 0) > 0:
                break
        extra = (splits,) if kind == "append" else ()
        cases.append((first_id + i, dtype, g * hkv, hkv, lengths) + extra + (rot,))
    return cases


def _sid(c):
    return f"{c[0]}-{c[1]}-h{c[2]}x{c[3]}-rot{c[-1]}"


SWEEP_PREFILL = _sweep("prefill", 14, 400, ["bf16", "bf16", "bf16", "f32"])
SWEEP_APPEND = _sweep("append", 6, 430, ["bf16", "bf16", "f32"])
SWEEP_DECODE = _sweep("decode", 8, 460, ["bf16", "bf16", "bf16", "f32"])


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths,rot", SWEEP_PREFILL, ids=[_sid(c) for c in SWEEP_PREFILL])
def test_gated_sweep_prefill(cid, dtype, hq, hkv, lengths, rot):
    run_gated_prefill(cid, dtype, hq, hkv, lengths, rot)


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths,splits,rot", SWEEP_APPEND, ids=[_sid(c) for c in SWEEP_APPEND])
def test_gated_sweep_append(cid, dtype, hq, hkv, lengths, splits, rot):
    run_gated_append(cid, dtype, hq, hkv, lengths, splits, rot)


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths,rot", SWEEP_DECODE, ids=[_sid(c) for c in SWEEP_DECODE])
def test_gated_sweep_decode(cid, dtype, hq, hkv, lengths, rot):
    run_gated_decode(cid, dtype, hq, hkv, lengths, rot)
