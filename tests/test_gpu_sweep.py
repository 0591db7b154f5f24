"""Seeded random shapes for prefill, append and decode, against the oracle.

The hand-picked cases in the other GPU tests cover the tile edges one at a
time; this sweep draws head counts, group sizes (including the ones that do
not divide a tile evenly: 3, 6, 7, 12, 24), sequence counts and ragged
lengths from a fixed generator, so the case list is the same on every run and
each case is named by its shape.  Tolerances are the same as the hand-picked
cases: fp32 max-abs 1e-4, bf16 max/mean 2e-2 / 2e-3 scaled by max(1, s_v)."""

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

# group sizes the prefill tiles (256 bf16 rows, 64 fp32 rows) and decode (16 rows) accept
PREFILL_G = {"bf16": [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24, 32, 64], "f32": [1, 2, 3, 5, 8, 16, 64]}
DECODE_G = {"bf16": [1, 2, 3, 4, 5, 6, 7, 8, 12, 16], "f32": [1, 3, 4, 8]}


def _heads(rng, g, max_hq=64):
    hkv = int(rng.choice([h for h in (1, 2, 4, 8) if g * h <= max_hq]))
    return g * hkv, hkv


def _lengths(rng, n_max, l_max, zero_p=0.1):
    n = int(rng.integers(1, n_max + 1))
    ls = rng.integers(1, l_max + 1, size=n)
    ls[rng.random(n) < zero_p] = 0
    return [int(x) for x in ls]


def _draw(kind, n_cases, first_id, dtypes):
    """Every group size of the table appears once before any repeats (per dtype);
    at least one token is new in every case (an empty call is its own test)."""
    rng = np.random.default_rng([0x5EE9, first_id])
    table = DECODE_G if kind == "decode" else PREFILL_G
    order = {d: [] for d in dtypes}
    cases = []
    for i in range(n_cases):
        dtype = dtypes[i % len(dtypes)]
        if not order[dtype]:
            order[dtype] = [int(g) for g in rng.permutation(table[dtype])]
        hq, hkv = _heads(rng, order[dtype].pop())
        while True:
            lengths = _lengths(rng, 6, 3000) if kind == "decode" else _lengths(rng, 4, 600)
            splits = [int(rng.integers(0, L + 1)) for L in lengths]
            if kind == "decode" or sum(lengths) - (sum(splits) if kind == "append" else 0) > 0:
                break
        if kind == "append":
            cases.append((first_id + i, dtype, hq, hkv, lengths, splits))
        else:
            cases.append((first_id + i, dtype, hq, hkv, lengths))
    return cases


def _name(c):
    return f"{c[0]}-{c[1]}-h{c[2]}x{c[3]}"


SWEEP_PREFILL = _draw("prefill", 17, 300, ["bf16", "bf16", "bf16", "f32"])
SWEEP_APPEND = _draw("append", 8, 330, ["bf16", "bf16", "bf16", "f32"])
SWEEP_DECODE = _draw("decode", 12, 360, ["bf16", "bf16", "bf16", "f32"])


def _gate(got, ref, spec, label):
    if spec.dtype == "f32":
        err = np.abs(got - ref).max() if got.size else 0.0
        assert err <= 1e-4, f"{label}: max abs {err:.3e}"
    elif got.size:
        print(U.bf16_gate(got, ref, spec, label=label))


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths", SWEEP_PREFILL, ids=[_name(c) for c in SWEEP_PREFILL])
def test_sweep_prefill(cid, dtype, hq, hkv, lengths):
    spec = inputs.custom_spec(cid, dtype, hq, hkv, lengths)
    x = inputs.prefill_inputs(spec)
    U.say(f"sweep prefill {cid} {dtype} Hq={hq} Hkv={hkv} lengths={lengths}")
    out = U.down(U.run_prefill(spec, x))
    ref = oracle.attention_prefill(x["q"], x["k"], x["v"], x["q_gamma"], x["k_gamma"], x["cu_seqlens"], hq, hkv,
                                   eps=spec.eps, theta=spec.theta)
    _gate(out, ref, spec, f"sweep prefill {cid}")


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths,splits", SWEEP_APPEND, ids=[_name(c) for c in SWEEP_APPEND])
def test_sweep_append(cid, dtype, hq, hkv, lengths, splits):
    spec = inputs.custom_spec(cid, dtype, hq, hkv, lengths)
    x = inputs.prefill_inputs(spec)
    U.say(f"sweep append {cid} {dtype} Hq={hq} Hkv={hkv} lengths={lengths} prefixes={splits}")
    out, kc, vc, ref, _ = U.append_case(spec, x, splits, max(lengths) + 5)
    _gate(U.down(out), ref, spec, f"sweep append {cid}")
    # nothing was written past the end of any sequence
    for s, L in enumerate(lengths):
        assert bool((kc[s, :, L:] == 7.0).all()) and bool((vc[s, :, L:] == 7.0).all())


@pytest.mark.parametrize("cid,dtype,hq,hkv,lengths", SWEEP_DECODE, ids=[_name(c) for c in SWEEP_DECODE])
def test_sweep_decode(cid, dtype, hq, hkv, lengths):
    spec = inputs.custom_spec(cid, dtype, hq, hkv, lengths, kind="decode")
    x = inputs.decode_new_token(spec)
    U.say(f"sweep decode {cid} {dtype} Hq={hq} Hkv={hkv} lengths={lengths}")
    kc, vc, raws = U.build_decode_cache(spec, x, max(lengths) + 3)
    dt = U.torch_dtype(spec)
    sp = x["start_pos"]
    out = B.decode(U.params(spec), U.up(x["q"], dt), U.up(x["k"], dt), U.up(x["v"], dt), U.up(x["q_gamma"], dt),
                   U.up(x["k_gamma"], dt), kc, vc, torch.from_numpy(sp).to(U.DEV), sp)
    torch.cuda.synchronize()
    ref = U.oracle_decode(spec, x, raws, range(spec.n_seq))
    _gate(U.down(out), ref, spec, f"sweep decode {cid}")
