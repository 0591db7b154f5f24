"""Helpers for the GPU parity tests: upload seeded inputs, run the library
through its C-ABI binding, and score results against the oracle."""

import sys

import numpy as np
import torch

import oracle
from attention_qk_norm_amd import binding as B
from attention_qk_norm_amd import inputs

DEV = torch.device("cuda:0")


def say(msg):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(spec):
    return torch.bfloat16 if spec.dtype == "bf16" else torch.float32


def up(a, dtype):
    """Host float32 array (already representable in dtype) -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype)


def down(t):
    return t.float().cpu().numpy().astype(np.float64)


def params(spec, **kw):
    return B.make_params(spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, rope_theta=spec.theta, **kw)


def v_scale_per_q_head(spec):
    _, _, sv = inputs.head_scales(spec)
    return sv[np.arange(spec.n_q_heads) // spec.g].astype(np.float64)


def bf16_gate(got, ref, spec, heads=None, max_tol=2e-2, mean_tol=2e-3, label=""):
    """Per query head t, errors divided by max(1, s_v of t's KV head) must meet the
    max / mean bounds (a bf16 output cannot meet an absolute bound once V is
    scaled up to 30; with s_v <= 1 this is the absolute bound)."""
    heads = np.arange(spec.n_q_heads) if heads is None else np.asarray(heads)
    s = np.maximum(1.0, v_scale_per_q_head(spec)[heads])
    err = np.abs(got - ref) / s[None, :, None]
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    mx, mn = float(err.max()), float(err.mean())
    raw = float(np.abs(got - ref).max())
    assert mx <= max_tol and mn <= mean_tol, f"{label}: scaled max {mx:.3e} mean {mn:.3e} (raw max {raw:.3e})"
    return mx, mn, raw


def run_prefill(spec, x, k_cache=None, v_cache=None):
    dt = torch_dtype(spec)
    p = params(spec)
    cu = torch.from_numpy(x["cu_seqlens"]).to(DEV)
    out = B.prefill(p, up(x["q"], dt), up(x["k"], dt), up(x["v"], dt), up(x["q_gamma"], dt),
                    up(x["k_gamma"], dt), cu, x["cu_seqlens"], k_cache=k_cache, v_cache=v_cache)
    torch.cuda.synchronize()
    return out


def build_decode_cache(spec, x, capacity, seqs=None):
    """Fill a [n_seq][Hkv][capacity][128] cache with the rotated raw cache keys
    (through qk_norm_rope at positions 0 .. L-1) and the raw values."""
    dt = torch_dtype(spec)
    p = params(spec)
    n = spec.n_seq
    kc = torch.zeros(n, spec.n_kv_heads, capacity, 128, dtype=dt, device=DEV)
    vc = torch.zeros_like(kc)
    kg = up(x["k_gamma"], dt)
    seqs = range(n) if seqs is None else seqs
    raws = inputs.decode_cache_raw_all(spec, seqs)
    for i, (kr, vr) in zip(seqs, raws):
        L = spec.lengths[i]
        if L == 0:
            continue
        pos = torch.arange(L, dtype=torch.int32, device=DEV)
        _, kh = B.qk_norm_rope(p, None, up(kr, dt), None, kg, pos)
        kc[i, :, :L] = kh.permute(1, 0, 2)
        vc[i, :, :L] = up(vr, dt).permute(1, 0, 2)
    torch.cuda.synchronize()
    return kc, vc, raws


def oracle_decode(spec, x, raws, seqs):
    """Oracle decode of the sequences ``seqs``; raws[j] = raw cache (k, v) of seqs[j]."""
    out = []
    for j, i in enumerate(seqs):
        L = spec.lengths[i]
        kr, vr = raws[j]
        kh = oracle.qk_norm_rope(kr, x["k_gamma"], np.arange(L), spec.eps, spec.theta)
        o = oracle.attention_decode(x["q"][i:i + 1], x["k"][i:i + 1], x["v"][i:i + 1], x["q_gamma"],
                                    x["k_gamma"], [kh], [vr], [L], spec.n_q_heads, spec.n_kv_heads,
                                    eps=spec.eps, theta=spec.theta)
        out.append(o[0])
    return np.stack(out)


def sample_rows(L, rng, n_blocks=2, block=16):
    """First and last rows plus a few seeded blocks of a sequence of length L."""
    rows = set(range(min(L, block))) | set(range(max(0, L - block), L))
    for _ in range(n_blocks):
        a = int(rng.integers(0, max(1, L - block)))
        rows |= set(range(a, min(L, a + block)))
    return np.array(sorted(rows))


def oracle_rows(spec, seq, rows, heads):
    """Oracle output rows of one sequence of a prefill case (keys regenerated)."""
    runs, start = [], 0
    for j in range(1, len(rows) + 1):  # contiguous runs of the sorted rows
        if j == len(rows) or rows[j] != rows[j - 1] + 1:
            runs.append((int(rows[start]), int(rows[j - 1]) + 1))
            start = j
    q = np.concatenate([inputs.prefill_seq_rows(spec, seq, a, b, "q") for a, b in runs])
    k = inputs.prefill_seq_rows(spec, seq, 0, int(rows.max()) + 1, "k")
    v = inputs.prefill_seq_rows(spec, seq, 0, int(rows.max()) + 1, "v")
    gq, gk = inputs.gammas(spec)
    return oracle.attention_prefill_rows(q, k, v, gq, gk, rows, heads, spec.n_q_heads, spec.n_kv_heads,
                                         eps=spec.eps, theta=spec.theta)


def append_case(spec, x, splits, cap):
    """Prefix of each sequence by prefill (cache written), then its remaining
    tokens as one append.  splits[s] = prefix length of sequence s.  Returns the
    append output [n_new][Hq][128], the cache and the oracle's output."""
    dt = torch_dtype(spec)
    p = params(spec)
    n = spec.n_seq
    cu = x["cu_seqlens"]
    kc = torch.full((n, spec.n_kv_heads, cap, 128), 7.0, dtype=dt, device=DEV)
    vc = torch.full_like(kc, 7.0)
    pre = [np.arange(cu[s], cu[s] + splits[s]) for s in range(n)]
    new = [np.arange(cu[s] + splits[s], cu[s + 1]) for s in range(n)]
    cu_pre = np.concatenate([[0], np.cumsum([len(r) for r in pre])]).astype(np.int32)
    cu_new = np.concatenate([[0], np.cumsum([len(r) for r in new])]).astype(np.int32)
    ip, inew = np.concatenate(pre).astype(np.int64), np.concatenate(new).astype(np.int64)
    g = lambda name: up(x[name], dt)
    if cu_pre[-1] > 0:
        B.prefill(p, up(x["q"][ip], dt), up(x["k"][ip], dt), up(x["v"][ip], dt), g("q_gamma"), g("k_gamma"),
                  torch.from_numpy(cu_pre).to(DEV), cu_pre, k_cache=kc, v_cache=vc)
    sp = np.array(splits, dtype=np.int32)
    out = B.append(p, up(x["q"][inew], dt), up(x["k"][inew], dt), up(x["v"][inew], dt), g("q_gamma"),
                   g("k_gamma"), kc, vc, torch.from_numpy(sp).to(DEV), torch.from_numpy(cu_new).to(DEV),
                   sp, cu_new)
    torch.cuda.synchronize()
    ref = []
    for s in range(n):
        a, b, c = cu[s], cu[s] + splits[s], cu[s + 1]
        kh = oracle.qk_norm_rope(x["k"][a:b], x["k_gamma"], np.arange(splits[s]), spec.eps, spec.theta)
        o, _ = oracle.attention_append(x["q"][b:c], x["k"][b:c], x["v"][b:c], x["q_gamma"], x["k_gamma"], kh,
                                       x["v"][a:b], splits[s], spec.n_q_heads, spec.n_kv_heads, eps=spec.eps,
                                       theta=spec.theta)
        ref.append(o)
    return out, kc, vc, np.concatenate(ref), cu_new
