"""GPU parity of libqwattn against the CPU oracle, through the C-ABI.

Tolerances: fp32 inputs max-abs 1e-4 (raw); bf16 inputs, per query head,
max |o - o_ref| / max(1, s_v) <= 2e-2 and mean <= 2e-3 where s_v is the
head's V scale (the raw values are printed); with unscaled V the bound is
the plain absolute one.  Integer-exact properties (causality, packing,
determinism, the first row, cache writes) are checked bit for bit."""

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


# ------------------------------------------------------------------ norm + RoPE

@pytest.mark.parametrize("dtype,theta", [("f32", 1e6), ("bf16", 1e6), ("bf16", 1e7)])
def test_qk_norm_rope(dtype, theta):
    spec = inputs.custom_spec(101, dtype, 8, 2, [37, 300], theta=theta)
    x = inputs.prefill_inputs(spec)
    rng = np.random.default_rng(3)
    pos = np.concatenate([np.arange(37), rng.integers(0, 131072, size=300)]).astype(np.int32)
    pos[-1] = 32767
    U.say(f"qk_norm_rope {dtype} theta={theta} n_tok={len(pos)}")
    dt = U.torch_dtype(spec)
    qo, ko = B.qk_norm_rope(U.params(spec), U.up(x["q"], dt), U.up(x["k"], dt), U.up(x["q_gamma"], dt),
                            U.up(x["k_gamma"], dt), torch.from_numpy(pos).to(U.DEV))
    torch.cuda.synchronize()
    for got, raw, g, name in ((qo, x["q"], x["q_gamma"], "q"), (ko, x["k"], x["k_gamma"], "k")):
        ref = oracle.qk_norm_rope(raw, g, pos, spec.eps, theta)
        got = U.down(got)
        err = np.abs(got - ref)
        if dtype == "f32":
            assert err.max() <= 2e-5, (name, err.max())
        else:  # one rounding to bf16: half an ulp of the value, plus fp32 slack
            assert np.all(err <= np.abs(ref) * 2.0 ** -8 + 1e-5), (name, err.max())
        # position 0 is the identity of the normed row
        z = np.where(pos == 0)[0]
        if len(z):
            nrm = oracle.rms_norm_heads(raw[z], g, spec.eps)
            assert np.abs(got[z] - nrm).max() <= (2e-5 if dtype == "f32" else 2.0 ** -8 * np.abs(nrm).max())


def test_qk_norm_rope_in_place_and_k_only():
    spec = inputs.custom_spec(102, "bf16", 4, 4, [50])
    x = inputs.prefill_inputs(spec)
    pos = np.arange(50, dtype=np.int32)
    U.say("qk_norm_rope in place / k only")
    dt = torch.bfloat16
    k = U.up(x["k"], dt)
    _, ko = B.qk_norm_rope(U.params(spec), None, U.up(x["k"], dt), None, U.up(x["k_gamma"], dt),
                           torch.from_numpy(pos).to(U.DEV))
    B.qk_norm_rope(U.params(spec), None, k, None, U.up(x["k_gamma"], dt), torch.from_numpy(pos).to(U.DEV),
                   k_out=k)
    torch.cuda.synchronize()
    assert torch.equal(k, ko)


# ------------------------------------------------------------------ prefill

PREFILL_SMALL = [
    # id, dtype, Hq, Hkv, lengths
    (110, "bf16", 8, 2, [1, 63, 64, 65, 200, 517]),   # g = 4, tile edges and a ragged tail
    (111, "bf16", 4, 4, [130, 7]),                    # g = 1 (MHA)
    (112, "bf16", 16, 2, [300, 129]),                 # g = 8
    (113, "bf16", 16, 1, [260]),                      # g = 16 (MQA over 16 heads)
    (114, "bf16", 10, 2, [97, 250]),                  # g = 5 (Qwen3-14B-like grouping)
    (115, "f32", 8, 2, [1, 63, 64, 65, 200]),
    (116, "f32", 6, 3, [77]),
]


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths", PREFILL_SMALL, ids=[str(c[0]) for c in PREFILL_SMALL])
def test_prefill_small(cid, dtype, hq, hkv, lengths):
    spec = inputs.custom_spec(cid, dtype, hq, hkv, lengths)
    x = inputs.prefill_inputs(spec)
    U.say(f"prefill case {cid} {dtype} Hq={hq} Hkv={hkv} lengths={lengths}")
    out = U.down(U.run_prefill(spec, x))
    ref = oracle.attention_prefill(x["q"], x["k"], x["v"], x["q_gamma"], x["k_gamma"], x["cu_seqlens"], hq, hkv,
                                   eps=spec.eps, theta=spec.theta)
    if dtype == "f32":
        assert np.abs(out - ref).max() <= 1e-4, np.abs(out - ref).max()
    else:
        print(U.bf16_gate(out, ref, spec, label=f"case {cid}"))


def test_prefill_config0_f32():
    spec = inputs.case_spec(0)
    x = inputs.prefill_inputs(spec)
    U.say("prefill config 0 (f32, 1x128, 16/8)")
    out = U.down(U.run_prefill(spec, x))
    ref = oracle.attention_prefill(x["q"], x["k"], x["v"], x["q_gamma"], x["k_gamma"], x["cu_seqlens"], 16, 8,
                                   eps=spec.eps, theta=spec.theta)
    err = np.abs(out - ref).max()
    print("config 0 max abs", err, "max |o|", np.abs(ref).max())
    assert err <= 1e-4


def test_prefill_unscaled_v_literal_bound():
    """q and k scaled per head, v ~ N(0,1): the literal 2e-2 / 2e-3 bounds."""
    spec = inputs.custom_spec(117, "bf16", 8, 2, [700, 333], v_scaled=False)
    x = inputs.prefill_inputs(spec)
    U.say("prefill unscaled-V companion")
    out = U.down(U.run_prefill(spec, x))
    ref = oracle.attention_prefill(x["q"], x["k"], x["v"], x["q_gamma"], x["k_gamma"], x["cu_seqlens"], 8, 2,
                                   eps=spec.eps, theta=spec.theta)
    err = np.abs(out - ref)
    print("unscaled V: max", err.max(), "mean", err.mean())
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_prefill_first_row_and_causality_bitwise():
    spec = inputs.custom_spec(118, "bf16", 8, 2, [150, 90])
    x = inputs.prefill_inputs(spec)
    U.say("prefill first-row / causality")
    out0 = U.run_prefill(spec, x)
    cu = x["cu_seqlens"]
    # first token of each sequence sees one key: o_0 = v_0 exactly
    for s in range(2):
        for t in range(8):
            assert torch.equal(out0[cu[s], t], U.up(x["v"][cu[s], t // 4], torch.bfloat16))
    # changing tokens after row i of sequence 0 leaves rows <= i bit-identical
    i = 70
    x2 = dict(x)
    for key in ("q", "k", "v"):
        a = x[key].copy()
        a[i + 1:cu[1]] = inputs.round_to_bf16(a[i + 1:cu[1]] * -1.5 + 0.25)
        x2[key] = a
    out1 = U.run_prefill(spec, x2)
    assert torch.equal(out0[:i + 1], out1[:i + 1])
    assert torch.equal(out0[cu[1]:], out1[cu[1]:])  # the other sequence is untouched too
    assert not torch.equal(out0[i + 1:cu[1]], out1[i + 1:cu[1]])


def test_prefill_packing_invariance_and_determinism():
    spec = inputs.custom_spec(119, "bf16", 8, 2, [100, 333, 64])
    x = inputs.prefill_inputs(spec)
    U.say("prefill packing invariance / determinism")
    out_a = U.run_prefill(spec, x)
    out_b = U.run_prefill(spec, x)
    assert torch.equal(out_a, out_b)
    cu = x["cu_seqlens"]
    solo = dict(x)
    for key in ("q", "k", "v"):
        solo[key] = x[key][cu[1]:cu[2]]
    solo["cu_seqlens"] = np.array([0, 333], dtype=np.int32)
    out_s = U.run_prefill(spec, solo)
    assert torch.equal(out_a[cu[1]:cu[2]], out_s)


def test_prefill_cache_write():
    spec = inputs.custom_spec(120, "bf16", 8, 2, [45, 130])
    x = inputs.prefill_inputs(spec)
    U.say("prefill with cache write")
    kc = torch.full((2, 2, 160, 128), 7.0, dtype=torch.bfloat16, device=U.DEV)
    vc = torch.full_like(kc, 7.0)
    out_c = U.run_prefill(spec, x, kc, vc)
    out_n = U.run_prefill(spec, x)
    assert torch.equal(out_c, out_n)
    cu = x["cu_seqlens"]
    for s in range(2):
        L = spec.lengths[s]
        pos = torch.arange(L, dtype=torch.int32, device=U.DEV)
        _, kh = B.qk_norm_rope(U.params(spec), None, U.up(x["k"][cu[s]:cu[s + 1]], torch.bfloat16), None,
                               U.up(x["k_gamma"], torch.bfloat16), pos)
        torch.cuda.synchronize()
        assert torch.equal(kc[s, :, :L], kh.permute(1, 0, 2))
        assert torch.equal(vc[s, :, :L], U.up(x["v"][cu[s]:cu[s + 1]], torch.bfloat16).permute(1, 0, 2))
        assert bool((kc[s, :, L:] == 7.0).all()) and bool((vc[s, :, L:] == 7.0).all())


def test_prefill_empty_and_zero_length():
    spec = inputs.custom_spec(121, "bf16", 8, 2, [0, 5, 0, 70, 0])
    x = inputs.prefill_inputs(spec)
    U.say("prefill with empty sequences")
    out = U.down(U.run_prefill(spec, x))
    ref = oracle.attention_prefill(x["q"], x["k"], x["v"], x["q_gamma"], x["k_gamma"], x["cu_seqlens"], 8, 2,
                                   eps=spec.eps, theta=spec.theta)
    U.bf16_gate(out, ref, spec, label="empty seqs")
    # n_seq = 0 is a no-op
    p = U.params(spec)
    z = torch.zeros(0, 8, 128, dtype=torch.bfloat16, device=U.DEV)
    B.prefill(p, z, z[:, :2], z[:, :2], U.up(x["q_gamma"], torch.bfloat16), U.up(x["k_gamma"], torch.bfloat16),
              torch.zeros(1, dtype=torch.int32, device=U.DEV), [0])


def test_prefill_online_softmax_path():
    """One large gamma entry each in q and k lifts the launch-wide QK-Norm
    logit bound, scale * log2(e) * 128 * max|gamma_q| * max|gamma_k| (+1/64),
    above 60 in log2 units, so the bf16 kernel runs its online (running-max)
    softmax instead of the static-bound one, while typical logits stay the
    configs' size (scaling every gamma instead sharpens the softmax until bf16
    operands alone exceed the tolerance).  Same tolerance as every bf16 case;
    the first row of each sequence is still exactly v_0."""
    spec = inputs.custom_spec(122, "bf16", 8, 2, [1, 64, 65, 200, 517])
    x = dict(inputs.prefill_inputs(spec))
    x["q_gamma"] = x["q_gamma"].copy()
    x["k_gamma"] = x["k_gamma"].copy()
    x["q_gamma"][5] = 3.5
    x["k_gamma"][70] = -3.0
    bound = (1.0 / np.sqrt(128.0)) * np.log2(np.e) * 128.0 * np.abs(x["q_gamma"]).max() * \
        np.abs(x["k_gamma"]).max() * (1.0 + 1.0 / 64)
    assert bound > 60.0, bound
    U.say(f"prefill online-softmax path (logit bound {bound:.1f} in log2 units)")
    out_t = U.run_prefill(spec, x)
    out = U.down(out_t)
    ref = oracle.attention_prefill(x["q"], x["k"], x["v"], x["q_gamma"], x["k_gamma"], x["cu_seqlens"], 8, 2,
                                   eps=spec.eps, theta=spec.theta)
    print(U.bf16_gate(out, ref, spec, label="online path"))
    cu = x["cu_seqlens"]
    for s in range(len(spec.lengths)):
        for t in range(8):
            assert torch.equal(out_t[cu[s], t], U.up(x["v"][cu[s], t // 4], torch.bfloat16))


V_BIG = 2.0 ** 118


@pytest.mark.parametrize("online", [False, True], ids=["static", "online"])
def test_prefill_large_magnitude_v(online):
    """V near the top of the bf16 range (v ~ N(0, 1) times 2^118, about 3e35 per
    unit): the static-bound weights 2^(score - B) and the online weights
    2^(score - max) are both <= 1, so the fp32 accumulators hold sums of a few
    hundred weighted v's and stay finite (weights 2^score, up to 2^B with B
    near 28 here, would overflow them).  Same bounds as every bf16 case, on
    the output divided by 2^118; the first row of every sequence is v_0
    exactly.  ``online`` lifts the launch-wide logit bound past 60 with one
    large gamma entry in q and k, as in the online-path test."""
    spec = inputs.custom_spec(124, "bf16", 8, 2, [1, 64, 65, 200, 517], v_scaled=False)
    x = dict(inputs.prefill_inputs(spec))
    x["v"] = (x["v"] * np.float32(V_BIG)).astype(np.float32)  # exact: a power of two
    if online:
        x["q_gamma"] = x["q_gamma"].copy()
        x["k_gamma"] = x["k_gamma"].copy()
        x["q_gamma"][5] = 3.5
        x["k_gamma"][70] = -3.0
    bound = (1.0 / np.sqrt(128.0)) * np.log2(np.e) * 128.0 * np.abs(x["q_gamma"]).max() * \
        np.abs(x["k_gamma"]).max() * (1.0 + 1.0 / 64)
    assert (bound > 60.0) == online, bound
    U.say(f"prefill large-magnitude V, {'online' if online else 'static-bound'} softmax (bound {bound:.1f})")
    out_t = U.run_prefill(spec, x)
    out = U.down(out_t)
    ref = oracle.attention_prefill(x["q"], x["k"], x["v"], x["q_gamma"], x["k_gamma"], x["cu_seqlens"], 8, 2,
                                   eps=spec.eps, theta=spec.theta)
    assert np.isfinite(out).all()
    err = np.abs(out - ref) / V_BIG
    print(f"large V ({'online' if online else 'static'}): max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    cu = x["cu_seqlens"]
    for s in range(len(spec.lengths)):
        for t in range(8):
            assert torch.equal(out_t[cu[s], t], U.up(x["v"][cu[s], t // 4], torch.bfloat16))


def test_prefill_many_short_sequences():
    """2100 packed sequences of 0..9 tokens: the plan kernel's large-plan path
    (more sequences than its LDS arrays hold), empty sequences included."""
    rng = np.random.default_rng(123)
    lengths = rng.integers(0, 10, size=2100).tolist()
    spec = inputs.custom_spec(123, "bf16", 8, 2, lengths)
    x = inputs.prefill_inputs(spec)
    U.say(f"prefill with {len(lengths)} short sequences ({sum(lengths)} tokens)")
    out = U.down(U.run_prefill(spec, x))
    ref = oracle.attention_prefill(x["q"], x["k"], x["v"], x["q_gamma"], x["k_gamma"], x["cu_seqlens"], 8, 2,
                                   eps=spec.eps, theta=spec.theta)
    print(U.bf16_gate(out, ref, spec, label="many short sequences"))


@pytest.mark.parametrize("v_scaled", [True, False], ids=["v-scaled", "v-unscaled"])
@pytest.mark.parametrize("case_id", [1, 3, 4])
def test_prefill_full_size_sampled(case_id, v_scaled):
    """Full-size standard workloads in the benchmark's launch configuration;
    seeded row samples of every sequence checked against the oracle.  With the
    V heads scaled (the workload as specified) the error is divided by
    max(1, s_v); with V unscaled (q and k still scaled per head, which is what
    stresses QK-Norm) the literal absolute bounds 2e-2 max / 2e-3 mean hold."""
    spec = inputs.case_spec(case_id, v_scaled=v_scaled)
    U.say(f"prefill config {case_id} full size: {spec.workload} (generating inputs)")
    x = inputs.prefill_inputs(spec)
    U.say(f"prefill config {case_id} full size: launching ({spec.n_tok} tokens)")
    out = U.run_prefill(spec, x)
    rng = np.random.default_rng(case_id)
    heads = np.arange(spec.n_q_heads)
    seqs = range(spec.n_seq) if spec.n_seq <= 4 else sorted(set([0, spec.n_seq - 1]) |
                                                             set(rng.choice(spec.n_seq, 3, replace=False).tolist()))
    cu = x["cu_seqlens"]
    for s in seqs:
        rows = U.sample_rows(spec.lengths[s], rng)
        U.say(f"  oracle rows seq {s} ({len(rows)} rows, L={spec.lengths[s]})")
        ref = U.oracle_rows(spec, s, rows, heads)
        got = U.down(out[cu[s] + rows])
        print(case_id, s, U.bf16_gate(got, ref, spec, label=f"config {case_id} seq {s}"))
        if not v_scaled:
            err = np.abs(got - ref)
            assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())


# ------------------------------------------------------------------ append (chunked prefill)

APPEND_CASES = [
    # id, dtype, Hq, Hkv, lengths (prefix + new), prefix lengths
    (140, "bf16", 8, 2, [300, 70, 400, 5], [37, 0, 256, 4]),   # ragged prefixes, one append of a single token
    (141, "bf16", 32, 8, [700, 129], [512, 1]),                 # g = 4 (Qwen3-8B grouping)
    (142, "bf16", 16, 1, [333], [100]),                         # g = 16
    (143, "f32", 8, 2, [150, 70], [64, 3]),                     # fp32 path
]


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths,splits", APPEND_CASES, ids=[str(c[0]) for c in APPEND_CASES])
def test_append_against_cache(cid, dtype, hq, hkv, lengths, splits):
    """New tokens at start_pos .. attend to the cached keys and causally to each
    other (rectangular mask); the oracle appends to its own cache."""
    spec = inputs.custom_spec(cid, dtype, hq, hkv, lengths)
    x = inputs.prefill_inputs(spec)
    U.say(f"append case {cid} {dtype} Hq={hq} Hkv={hkv} lengths={lengths} prefixes={splits}")
    out, kc, vc, ref, _ = U.append_case(spec, x, splits, max(lengths) + 9)
    got = U.down(out)
    if dtype == "f32":
        assert np.abs(got - ref).max() <= 1e-4, np.abs(got - ref).max()
    else:
        sv = np.maximum(1.0, U.v_scale_per_q_head(spec))
        err = np.abs(got - ref) / sv[None, :, None]
        print(f"case {cid}: scaled max {err.max():.3e} mean {err.mean():.3e}")
        assert err.max() <= 2e-2 and err.mean() <= 2e-3
    # the cache holds every token's rotated key and its value, and nothing past the sequence
    dt = U.torch_dtype(spec)
    cu = x["cu_seqlens"]
    for s in range(spec.n_seq):
        L = lengths[s]
        pos = torch.arange(L, dtype=torch.int32, device=U.DEV)
        _, kh = B.qk_norm_rope(U.params(spec), None, U.up(x["k"][cu[s]:cu[s + 1]], dt), None,
                               U.up(x["k_gamma"], dt), pos)
        torch.cuda.synchronize()
        assert torch.equal(kc[s, :, :L], kh.permute(1, 0, 2))
        assert torch.equal(vc[s, :, :L], U.up(x["v"][cu[s]:cu[s + 1]], dt).permute(1, 0, 2))
        assert bool((kc[s, :, L:] == 7.0).all()) and bool((vc[s, :, L:] == 7.0).all())


def test_append_in_chunks_equals_one_prefill():
    """Appending a prompt in chunks [0:2], [2:5], [5:6] and then in larger
    ragged chunks gives the single-pass prefill rows, as the pages' own
    KV-cache check has it.  Here bit for bit: a row's keys are visited in the
    same 64-key tiles from slot 0 either way, and masked keys add exact zeros."""
    spec = inputs.custom_spec(144, "bf16", 8, 2, [300])
    x = inputs.prefill_inputs(spec)
    dt = torch.bfloat16
    p = U.params(spec)
    full = U.down(U.run_prefill(spec, x))
    U.say("append in chunks vs one prefill")
    kc = torch.zeros(1, 2, 320, 128, dtype=dt, device=U.DEV)
    vc = torch.zeros_like(kc)
    g = lambda name: U.up(x[name], dt)
    outs = []
    for a, b in ((0, 2), (2, 5), (5, 6), (6, 70), (70, 71), (71, 300)):
        sp = np.array([a], dtype=np.int32)
        cn = np.array([0, b - a], dtype=np.int32)
        o = B.append(p, U.up(x["q"][a:b], dt), U.up(x["k"][a:b], dt), U.up(x["v"][a:b], dt), g("q_gamma"),
                     g("k_gamma"), kc, vc, torch.from_numpy(sp).to(U.DEV), torch.from_numpy(cn).to(U.DEV), sp, cn)
        outs.append(U.down(o))
    torch.cuda.synchronize()
    got = np.concatenate(outs)
    sv = np.maximum(1.0, U.v_scale_per_q_head(spec))
    err = np.abs(got - full) / sv[None, :, None]
    print(f"chunks vs one pass: scaled max {err.max():.3e}; bitwise equal rows {np.mean(np.all(got == full, axis=(1, 2))):.2f}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    assert np.array_equal(got, full)


def test_append_capacity_rejection_leaves_cache():
    """An append that would run past the cache is rejected and changes nothing."""
    spec = inputs.custom_spec(145, "bf16", 8, 2, [40])
    x = inputs.prefill_inputs(spec)
    dt = torch.bfloat16
    kc = torch.full((1, 2, 40, 128), 3.0, dtype=dt, device=U.DEV)
    vc = torch.full_like(kc, 3.0)
    before = (kc.clone(), vc.clone())
    sp = np.array([30], dtype=np.int32)
    cn = np.array([0, 11], dtype=np.int32)
    U.say("append past capacity")
    with pytest.raises(B.QwattnError):
        B.append(U.params(spec), U.up(x["q"][:11], dt), U.up(x["k"][:11], dt), U.up(x["v"][:11], dt),
                 U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt), kc, vc, torch.from_numpy(sp).to(U.DEV),
                 torch.from_numpy(cn).to(U.DEV), sp, cn)
    torch.cuda.synchronize()
    assert torch.equal(kc, before[0]) and torch.equal(vc, before[1])


# ------------------------------------------------------------------ RoPE-then-norm order (params.order = 1)

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_norm_order_all_entry_points(dtype):
    """params.order = 1 (RoPE first, then QK-Norm) on every entry point against
    the oracle's order="rope_norm"; with the configs' non-pair-symmetric gamma
    the two orders give different outputs, and the library follows each."""
    spec = inputs.custom_spec(146 if dtype == "bf16" else 147, dtype, 8, 2, [1, 70, 200])
    x = inputs.prefill_inputs(spec)
    dt = U.torch_dtype(spec)
    p1 = U.params(spec, order=1)
    cu = x["cu_seqlens"]
    U.say(f"RoPE-then-norm order, {dtype}")
    kw = dict(eps=spec.eps, theta=spec.theta)

    def check(got, ref, label):
        if dtype == "f32":
            assert np.abs(got - ref).max() <= 1e-4, (label, np.abs(got - ref).max())
        else:
            sv = np.maximum(1.0, U.v_scale_per_q_head(spec))
            err = np.abs(got - ref) / sv[None, :, None]
            assert err.max() <= 2e-2 and err.mean() <= 2e-3, (label, err.max(), err.mean())

    # standalone rows
    pos = np.arange(cu[-1], dtype=np.int32) % 97
    qo, ko = B.qk_norm_rope(p1, U.up(x["q"], dt), U.up(x["k"], dt), U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt),
                            torch.from_numpy(pos).to(U.DEV))
    torch.cuda.synchronize()
    for got, raw, g in ((qo, x["q"], x["q_gamma"]), (ko, x["k"], x["k_gamma"])):
        ref = oracle.qk_norm_rope(raw, g, pos, spec.eps, spec.theta, order="rope_norm")
        tol = 2e-5 if dtype == "f32" else None
        got = U.down(got)
        if tol:
            assert np.abs(got - ref).max() <= tol
        else:
            assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-5)
    # prefill (with a cache, which then serves the append and decode below)
    cap = 210
    kc = torch.zeros(3, 2, cap, 128, dtype=dt, device=U.DEV)
    vc = torch.zeros_like(kc)
    out = B.prefill(p1, U.up(x["q"], dt), U.up(x["k"], dt), U.up(x["v"], dt), U.up(x["q_gamma"], dt),
                    U.up(x["k_gamma"], dt), torch.from_numpy(cu).to(U.DEV), cu, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    ref1 = oracle.attention_prefill(x["q"], x["k"], x["v"], x["q_gamma"], x["k_gamma"], cu, 8, 2,
                                    order="rope_norm", **kw)
    ref0 = oracle.attention_prefill(x["q"], x["k"], x["v"], x["q_gamma"], x["k_gamma"], cu, 8, 2, **kw)
    check(U.down(out), ref1, "prefill")
    assert np.abs(ref1 - ref0).max() > 0.1  # the orders really differ here
    # one more token per sequence, once through append and once through decode
    rng = np.random.default_rng(7)
    qn = inputs.round_to_bf16(rng.standard_normal((3, 8, 128))) if dtype == "bf16" else \
        rng.standard_normal((3, 8, 128)).astype(np.float32)
    kn = inputs.round_to_bf16(rng.standard_normal((3, 2, 128))) if dtype == "bf16" else \
        rng.standard_normal((3, 2, 128)).astype(np.float32)
    vn = inputs.round_to_bf16(rng.standard_normal((3, 2, 128))) if dtype == "bf16" else \
        rng.standard_normal((3, 2, 128)).astype(np.float32)
    sp = np.array(spec.lengths, dtype=np.int32)
    refs = []
    for i in range(3):
        a, b = cu[i], cu[i + 1]
        kh = oracle.qk_norm_rope(x["k"][a:b], x["k_gamma"], np.arange(b - a), spec.eps, spec.theta,
                                 order="rope_norm")
        o, _ = oracle.attention_append(qn[i:i + 1], kn[i:i + 1], vn[i:i + 1], x["q_gamma"], x["k_gamma"], kh,
                                       x["v"][a:b], sp[i], 8, 2, order="rope_norm", **kw)
        refs.append(o[0])
    ref = np.stack(refs)
    cn = np.arange(4, dtype=np.int32)
    kc2, vc2 = kc.clone(), vc.clone()
    o_app = B.append(p1, U.up(qn, dt), U.up(kn, dt), U.up(vn, dt), U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt),
                     kc2, vc2, torch.from_numpy(sp).to(U.DEV), torch.from_numpy(cn).to(U.DEV), sp, cn)
    o_dec = B.decode(p1, U.up(qn, dt), U.up(kn, dt), U.up(vn, dt), U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt),
                     kc, vc, torch.from_numpy(sp).to(U.DEV), sp)
    torch.cuda.synchronize()
    check(U.down(o_app), ref, "append")
    check(U.down(o_dec), ref, "decode")
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2)  # both wrote the same new key and value


# ------------------------------------------------------------------ decode

DECODE_SMALL = [
    (130, "bf16", 8, 2, [0, 1, 31, 32, 33, 127, 128, 1000, 2500]),
    (131, "bf16", 32, 8, [5, 700, 1029]),
    (132, "bf16", 16, 1, [300, 64]),
    (133, "f32", 8, 2, [0, 1, 65, 300]),
]


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths", DECODE_SMALL, ids=[str(c[0]) for c in DECODE_SMALL])
def test_decode_small(cid, dtype, hq, hkv, lengths):
    spec = inputs.custom_spec(cid, dtype, hq, hkv, lengths, kind="decode")
    x = inputs.decode_new_token(spec)
    cap = max(lengths) + 7
    U.say(f"decode case {cid} {dtype} Hq={hq} Hkv={hkv} lengths={lengths}")
    kc, vc, raws = U.build_decode_cache(spec, x, cap)
    dt = U.torch_dtype(spec)
    sp = x["start_pos"]
    out = B.decode(U.params(spec), U.up(x["q"], dt), U.up(x["k"], dt), U.up(x["v"], dt), U.up(x["q_gamma"], dt),
                   U.up(x["k_gamma"], dt), kc, vc, torch.from_numpy(sp).to(U.DEV), sp)
    torch.cuda.synchronize()
    ref = U.oracle_decode(spec, x, raws, range(spec.n_seq))
    got = U.down(out)
    if dtype == "f32":
        assert np.abs(got - ref).max() <= 1e-4, np.abs(got - ref).max()
    else:
        print(U.bf16_gate(got, ref, spec, label=f"decode {cid}"))
    # the new key and value were appended at start_pos, rotated there
    for i, L in enumerate(lengths):
        _, kh = B.qk_norm_rope(U.params(spec), None, U.up(x["k"][i:i + 1], dt), None, U.up(x["k_gamma"], dt),
                               torch.tensor([L], dtype=torch.int32, device=U.DEV))
        torch.cuda.synchronize()
        assert torch.equal(kc[i, :, L], kh[0])
        assert torch.equal(vc[i, :, L], U.up(x["v"][i], dt))


def test_decode_matches_last_prefill_row():
    """Prefill over L+1 tokens vs prefill over L (filling the cache) + one decode step."""
    L = 777
    spec = inputs.custom_spec(134, "bf16", 8, 2, [L + 1])
    x = inputs.prefill_inputs(spec)
    U.say("decode vs last prefill row")
    full = U.run_prefill(spec, x)
    kc = torch.zeros(1, 2, L + 1, 128, dtype=torch.bfloat16, device=U.DEV)
    vc = torch.zeros_like(kc)
    head = dict(x)
    for key in ("q", "k", "v"):
        head[key] = x[key][:L]
    head["cu_seqlens"] = np.array([0, L], dtype=np.int32)
    U.run_prefill(spec, head, kc, vc)
    dt = torch.bfloat16
    sp = np.array([L], dtype=np.int32)
    out = B.decode(U.params(spec), U.up(x["q"][L:], dt), U.up(x["k"][L:], dt), U.up(x["v"][L:], dt),
                   U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt), kc, vc, torch.from_numpy(sp).to(U.DEV), sp)
    torch.cuda.synchronize()
    U.bf16_gate(U.down(out), U.down(full[L:]), spec, label="decode vs prefill")


def test_decode_capacity_rejection_leaves_cache():
    """An over-long append is rejected and leaves the cache untouched."""
    spec = inputs.custom_spec(135, "bf16", 8, 2, [5, 9], kind="decode")
    x = inputs.decode_new_token(spec)
    U.say("decode capacity rejection")
    kc, vc, _ = U.build_decode_cache(spec, x, 9)
    k0, v0 = kc.clone(), vc.clone()
    dt = torch.bfloat16
    sp = x["start_pos"]
    with pytest.raises(B.QwattnError) as ei:
        B.decode(U.params(spec), U.up(x["q"], dt), U.up(x["k"], dt), U.up(x["v"], dt), U.up(x["q_gamma"], dt),
                 U.up(x["k_gamma"], dt), kc, vc, torch.from_numpy(sp).to(U.DEV), sp)
    assert ei.value.status == B.ERR_CAPACITY
    torch.cuda.synchronize()
    assert torch.equal(kc, k0) and torch.equal(vc, v0)


@pytest.mark.parametrize("v_scaled", [True, False], ids=["v-scaled", "v-unscaled"])
def test_decode_config2_full_size_sampled(v_scaled):
    """Qwen3-8B decode, 64 sequences with contexts U[1024, 32768], in the
    benchmark's launch configuration; 4 sequences checked against the oracle
    (unscaled V: the literal absolute bounds)."""
    spec = inputs.case_spec(2, v_scaled=v_scaled)
    x = inputs.decode_new_token(spec)
    cap = (max(spec.lengths) + 1 + 63) // 64 * 64
    U.say(f"decode config 2: building cache ({sum(spec.lengths)} tokens, capacity {cap})")
    kc, vc, _ = U.build_decode_cache(spec, x, cap)
    dt = torch.bfloat16
    sp = x["start_pos"]
    U.say("decode config 2: launching")
    out = B.decode(U.params(spec), U.up(x["q"], dt), U.up(x["k"], dt), U.up(x["v"], dt), U.up(x["q_gamma"], dt),
                   U.up(x["k_gamma"], dt), kc, vc, torch.from_numpy(sp).to(U.DEV), sp)
    torch.cuda.synchronize()
    order = np.argsort(spec.lengths)
    seqs = sorted({int(order[0]), int(order[-1]), 7, 40})
    U.say(f"decode config 2: oracle for sequences {seqs}")
    raws = inputs.decode_cache_raw_all(spec, seqs)
    ref = U.oracle_decode(spec, x, raws, seqs)
    got = U.down(out[seqs])
    print(U.bf16_gate(got, ref, spec, label="config 2"))
    if not v_scaled:
        err = np.abs(got - ref)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
