"""qwattn_decode_noalloc (the decode entry point that allocates nothing: its
scratch is the library's fixed device array) against qwattn_decode with a
workspace, through the C ABI: two calls in a row on one device, the second
with fewer sequences and shorter contexts, each must give qwattn_decode's
output and cache bit for bit (the same kernels on the same chunking) -- which
meets the bf16 bound against the oracle that qwattn_decode's own tests hold
(also checked here on a few sequences).  The rejection of sizes beyond the
array is a host check, tested on the CPU with the other validation cases."""

import numpy as np
import pytest
import torch

from attention_qk_norm_amd import binding as B
from attention_qk_norm_amd import inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_util as U
else:  # collected on a CPU-only machine: deselected by -m "not gpu"
    U = None


def _decode_pair(spec, cap, seed):
    """The same decode call through both entry points, each on its own copy of
    the cache; returns both outputs and both caches."""
    x = inputs.decode_new_token(spec)
    kc, vc, raws = U.build_decode_cache(spec, x, cap)
    dt = torch.bfloat16
    p = U.params(spec)
    sp_h = x["start_pos"]
    sp = torch.from_numpy(sp_h).to(U.DEV)
    args = (U.up(x["q"], dt), U.up(x["k"], dt), U.up(x["v"], dt), U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt))
    kc2, vc2 = kc.clone(), vc.clone()
    U.say(f"decode_noalloc vs decode: {spec.n_seq} sequences, contexts {min(spec.lengths)}..{max(spec.lengths)}")
    ref = B.decode(p, *args, kc, vc, sp, sp_h)
    got = B.decode_noalloc(p, *args, kc2, vc2, sp, sp_h)
    torch.cuda.synchronize()
    return x, raws, ref, got, (kc, vc), (kc2, vc2)


def test_decode_noalloc_two_calls_match_decode():
    # first call: 12 sequences with contexts up to 9000 keys (several chunks each)
    big = inputs.custom_spec(400, "bf16", 32, 8, [1, 2047, 2048, 2049, 9000, 5000, 0, 77, 4096, 6000, 3333, 8191],
                             kind="decode")
    x, raws, ref, got, (kc, vc), (kc2, vc2) = _decode_pair(big, 9024, 400)
    assert torch.equal(got, ref)
    assert torch.equal(kc2, kc) and torch.equal(vc2, vc)
    seqs = [0, 4, 11]
    want = U.oracle_decode(big, x, [raws[i] for i in seqs], seqs)
    print(U.bf16_gate(U.down(got[seqs]), want, big, label="noalloc call 1"))
    # second call, smaller: 3 sequences, shorter contexts; the array still holds
    # the first call's partials, which must not leak into this one
    small = inputs.custom_spec(401, "bf16", 32, 8, [300, 1, 1500], kind="decode")
    x, raws, ref, got, (kc, vc), (kc2, vc2) = _decode_pair(small, 1536, 401)
    assert torch.equal(got, ref)
    assert torch.equal(kc2, kc) and torch.equal(vc2, vc)
    want = U.oracle_decode(small, x, raws, list(range(3)))
    print(U.bf16_gate(U.down(got), want, small, label="noalloc call 2"))


def test_decode_noalloc_gated_layer_matches_decode():
    """The head_dim-256 gated layer (gate applied in the merge) through both entry points."""
    spec = inputs.gated_spec(402, "bf16", 16, 2, [700, 40, 2500], kind="decode", rot=64)
    x = inputs.decode_new_token(spec)
    dt = torch.bfloat16
    p = B.make_gated_params(16, 2, eps=spec.eps, rope_theta=spec.theta, rotary_dim=64)
    cap = 2560
    kc = torch.zeros(3, 2, cap, 256, dtype=dt, device=U.DEV)
    vc = torch.zeros_like(kc)
    for i, (kr, vr) in enumerate(inputs.decode_cache_raw_all(spec)):
        L = spec.lengths[i]
        _, kh = B.qk_norm_rope(p, None, U.up(kr, dt), None, U.up(x["k_gamma"], dt),
                               torch.arange(L, dtype=torch.int32, device=U.DEV))
        kc[i, :, :L] = kh.permute(1, 0, 2)
        vc[i, :, :L] = U.up(vr, dt).permute(1, 0, 2)
    kc2, vc2 = kc.clone(), vc.clone()
    sp_h = x["start_pos"]
    sp = torch.from_numpy(sp_h).to(U.DEV)
    args = (U.up(inputs.q_proj_rows(x["q"], x["gate"]), dt), U.up(x["k"], dt), U.up(x["v"], dt),
            U.up(x["q_gamma"], dt), U.up(x["k_gamma"], dt))
    U.say("decode_noalloc vs decode: gated layer, 3 sequences")
    ref = B.decode(p, *args, kc, vc, sp, sp_h)
    got = B.decode_noalloc(p, *args, kc2, vc2, sp, sp_h)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(kc2, kc) and torch.equal(vc2, vc)
