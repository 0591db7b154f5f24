"""Benchmark of the attention-sublayer core on one MI355X.

One step = the whole hot path on synthetic Qwen3-shaped inputs resident in HBM:
  * qwattn_prefill on the Qwen3-32B-shaped long prefill (B=1 x T=32768, Hq=64,
    Hkv=8, bf16): norm+RoPE of K into a KV cache, the tile plan, and the causal
    GQA attention kernel with the fused Q norm+RoPE prologue;
  * qwattn_decode on the Qwen3-8B-shaped decode (64 sequences, contexts
    U[1024, 32768], bf16 cache): the new-token prologue, split-K attention and
    the combine.
Prints one JSON line.  ``value`` is prefill attention TFLOP/s of the long
prefill over the whole call (algorithmic flops: unmasked causal pairs only);
the decode KV-read GB/s sits under ``decode``.  The other prefill workloads
(Qwen3-8B 4 x 4096 and the Qwen3-235B-A22B-attention ragged batch) are timed
after the steps, each with its own roofline, under ``prefill_workloads``.
The line also carries chunked-prefill (``append``), the gated head_dim-256
layer of Qwen3-Next (``gated``: prefill and decode) and the whole attention
sublayer with its projections (``layer`` for Qwen3-8B, ``gated_layer`` for
the Qwen3-Next global-attention sublayer) figures, and the CPU oracle timed on
bounded samples (``cpu_baseline`` for the long prefill, ``decode.cpu_baseline``).

    python bench.py [--steps K] [--warmup W] [--prefill-case {1,3,4}] [--extra-prefill 1,4|none]
                    [--no-decode] [--no-cpu-baseline] [--no-append] [--no-gated] [--no-layer] [--gpus 1]
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E (published)
FP32_PEAK_TFLOPS = 157.3         # MI355X fp32 vector / MFMA (published)
HEADLINE_PREFILL = 3             # the long prefill: 1 x 32768 tokens, 64 / 8 heads
EXTRA_PREFILL = "1,4"            # the other prefill workloads, timed beside the steps


class HipEvents:
    """hipEvent_t pairs through the HIP runtime (recorded by the library on its stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def recorded_traffic(kernel, source, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summaries (profiles/hbm_traffic_*.md), or None when none
    was taken for the current kernel source."""
    import glob
    import hashlib
    path = os.path.join(ROOT, "attention_qk_norm_amd", "csrc", source)
    sha = hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "hbm_traffic_*.md"))):
        text = open(f).read()
        if "```json" not in text:
            continue
        block = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        for rec in block.values():
            if (rec.get("kernel_id") == kernel and rec.get("workload") == workload and
                    rec.get("source_sha256_16") == sha):
                return {"bytes": int(rec["read_bytes"]) + int(rec["write_bytes"]),
                        "read_bytes": int(rec["read_bytes"]), "write_bytes": int(rec["write_bytes"]),
                        "from": os.path.relpath(f, ROOT)}
    return None


def measure_peaks(dev, src):
    """The MFMA rate and HBM read bandwidth this GPU sustains in this run (the
    library's measurement aids, best of 3, timed with the library's hook): a
    register-only MFMA loop on every SIMD, and one nontemporal read of `src`."""
    import torch
    from attention_qk_norm_amd import binding as B
    ev = HipEvents()
    sink = torch.zeros(1, dtype=torch.float32, device=dev)

    def best_ms(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(3):
            a, b = ev.create(), ev.create()
            B.set_timing_events(a, b)
            fn()
            torch.cuda.synchronize()
            ms.append(ev.elapsed_ms(a, b))
        return min(ms)

    iters = 20000
    mfma = B.mfma_probe_flops(iters) / best_ms(lambda: B.mfma_probe(iters, sink)) / 1e9
    nbytes = B.hbm_read_probe(src, sink)
    hbm = nbytes / best_ms(lambda: B.hbm_read_probe(src, sink)) / 1e6
    return {"mfma_tflops": round(mfma, 1), "hbm_read_gbs": round(hbm, 1), "hbm_read_bytes": nbytes}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def pct(v):
    """p10 / median / p90 of timed iterations (ms)."""
    return [round(float(x), 4) for x in np.percentile(v, [10, 50, 90])]


def setup_prefill(case_id, dev):
    import torch
    from attention_qk_norm_amd import binding as B, inputs
    spec = inputs.case_spec(case_id)
    log(f"prefill workload: {spec.workload}; generating inputs")
    x = inputs.prefill_inputs(spec)
    bf = torch.bfloat16
    up = lambda a: torch.from_numpy(a).to(dev).to(bf)
    st = dict(spec=spec, q=up(x["q"]), k=up(x["k"]), v=up(x["v"]), qg=up(x["q_gamma"]), kg=up(x["k_gamma"]),
              cu=torch.from_numpy(x["cu_seqlens"]).to(dev), cu_h=x["cu_seqlens"])
    del x
    cap = (max(spec.lengths) + 63) // 64 * 64
    st["kc"] = torch.empty(spec.n_seq, spec.n_kv_heads, cap, 128, dtype=bf, device=dev)
    st["vc"] = torch.empty_like(st["kc"])
    st["out"] = torch.empty_like(st["q"])
    p = B.make_params(spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, rope_theta=spec.theta)
    nbytes = B.prefill_workspace_size(p, B.BF16, spec.n_seq, spec.n_tok, max(spec.lengths), True)
    st["ws"] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    st["params"] = p
    return st


def run_prefill(st):
    from attention_qk_norm_amd import binding as B
    B.prefill(st["params"], st["q"], st["k"], st["v"], st["qg"], st["kg"], st["cu"], st["cu_h"], out=st["out"],
              k_cache=st["kc"], v_cache=st["vc"], workspace=st["ws"])


def prefill_record(spec, call_all, kern_all, peaks=None):
    """Throughput of a prefill workload: over the whole call (``value``) and of
    the attention kernel against the bf16 MFMA peak (``roofline``)."""
    from attention_qk_norm_amd import accounting
    flops = accounting.prefill_flops(spec.lengths, spec.n_q_heads)
    call_ms, kern_ms = float(np.mean(call_all)), float(np.mean(kern_all))
    achieved = flops / (kern_ms * 1e-3) / 1e12
    roof = {"kernel": "k_prefill_bf16", "bound": "mfma", "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": recorded_traffic("k_prefill_bf16", "k_prefill.hip", spec.workload),
            "kernel_ms": round(kern_ms, 4), "kernel_ms_p10_p50_p90": pct(kern_all), "algorithmic_flops": flops}
    if peaks is not None:
        roof["measured_peak"] = {"value": peaks["mfma_tflops"], "unit": "TFLOP/s",
                                 "frac": round(achieved / peaks["mfma_tflops"], 4),
                                 "how": "register-only v_mfma_f32_32x32x16_bf16 loop, one wave per SIMD on "
                                        "every CU, this run (qwattn_mfma_probe)"}
    value = flops / (call_ms * 1e-3) / 1e12
    return {"metric": "prefill attention TFLOP/s", "unit": "TFLOP/s", "workload": spec.workload,
            "value": round(value, 2), "call_ms": round(call_ms, 4), "call_ms_p10_p50_p90": pct(call_all),
            "frac_mfma_peak": round(value / MFMA_BF16_PEAK_TFLOPS, 4), "roofline": roof}


def setup_decode(case_id, dev):
    import torch
    from attention_qk_norm_amd import binding as B, inputs
    spec = inputs.case_spec(case_id)
    log(f"decode workload: {spec.workload}; generating cache ({sum(spec.lengths)} tokens)")
    x = inputs.decode_new_token(spec)
    bf = torch.bfloat16
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(bf)
    p = B.make_params(spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, rope_theta=spec.theta)
    cap = (max(spec.lengths) + 1 + 63) // 64 * 64
    kc = torch.zeros(spec.n_seq, spec.n_kv_heads, cap, 128, dtype=bf, device=dev)
    vc = torch.zeros_like(kc)
    kg = up(x["k_gamma"])
    t0 = time.time()
    batch = 8
    for b0 in range(0, spec.n_seq, batch):
        seqs = list(range(b0, min(spec.n_seq, b0 + batch)))
        for i, (kr, vr) in zip(seqs, inputs.decode_cache_raw_all(spec, seqs)):
            L = spec.lengths[i]
            pos = torch.arange(L, dtype=torch.int32, device=dev)
            _, kh = B.qk_norm_rope(p, None, up(kr), None, kg, pos)
            kc[i, :, :L] = kh.permute(1, 0, 2)
            vc[i, :, :L] = up(vr).permute(1, 0, 2)
        torch.cuda.synchronize()
    log(f"decode cache built in {time.time() - t0:.1f}s")
    sp = x["start_pos"]
    st = dict(spec=spec, x=x, params=p, q=up(x["q"]), k=up(x["k"]), v=up(x["v"]), qg=up(x["q_gamma"]), kg=kg,
              kc=kc, vc=vc, sp=torch.from_numpy(sp).to(dev), sp_h=sp)
    st["out"] = torch.empty_like(st["q"])
    nbytes = B.decode_workspace_size(p, B.BF16, spec.n_seq, int(sp.sum()))
    st["ws"] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return st


def run_decode(st):
    from attention_qk_norm_amd import binding as B
    B.decode(st["params"], st["q"], st["k"], st["v"], st["qg"], st["kg"], st["kc"], st["vc"], st["sp"], st["sp_h"],
             out=st["out"], workspace=st["ws"])


def warm_up(run, seconds=0.3, max_calls=4000):
    """Calls `run` for `seconds` of wall time (at least twice) before a timed
    measurement: after the host-side input generation has left the GPU idle,
    its clock takes a fraction of a second of load to come back up, and calls
    timed earlier run up to 20% slow."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < 2 or (time.perf_counter() - t0 < seconds and n < max_calls):
        run()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _timed_lists(run, n_calls):
    """Per-call times (torch events around the call) and dominant-kernel times
    (the library's timing hook: HIP events on its stream), in ms."""
    import torch
    from attention_qk_norm_amd import binding as B
    ev = HipEvents()
    kev = [(ev.create(), ev.create()) for _ in range(n_calls)]
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_calls)]
    torch.cuda.synchronize()
    for (ka, kb), (ca, cb) in zip(kev, cev):
        B.set_timing_events(ka, kb)
        ca.record()
        run()
        cb.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in cev], [ev.elapsed_ms(a, b) for a, b in kev]


def _timed(run, n_calls):
    """Mean call time and mean dominant-kernel time, in ms."""
    c, k = _timed_lists(run, n_calls)
    return float(np.mean(c)), float(np.mean(k))


def measure_prefill_workload(case_id, dev, n_calls=20):
    """One prefill workload on its own: warm-up calls, then n_calls timed."""
    import torch
    st = setup_prefill(case_id, dev)
    warm_up(lambda: run_prefill(st))
    c, k = _timed_lists(lambda: run_prefill(st), n_calls)
    rec = prefill_record(st["spec"], c, k)
    del st
    torch.cuda.empty_cache()
    return rec


def measure_append(dev, n_calls=20, new_tokens=512):
    """Chunked prefill against the cache (qwattn_append), on the 4 x 4096
    workload: each sequence's first 4096 - new_tokens tokens are prefilled into
    the cache, then its last new_tokens tokens are appended (timed; every call
    rewrites the same cache slots)."""
    import torch
    from attention_qk_norm_amd import accounting, binding as B, inputs
    spec = inputs.case_spec(1)
    x = inputs.prefill_inputs(spec)
    bf = torch.bfloat16
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(bf)
    cu = x["cu_seqlens"]
    split = [L - new_tokens for L in spec.lengths]
    pre = np.concatenate([np.arange(cu[s], cu[s] + split[s]) for s in range(spec.n_seq)])
    new = np.concatenate([np.arange(cu[s] + split[s], cu[s + 1]) for s in range(spec.n_seq)])
    cu_pre = np.concatenate([[0], np.cumsum(split)]).astype(np.int32)
    cu_new = np.arange(spec.n_seq + 1, dtype=np.int32) * new_tokens
    p = B.make_params(spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, rope_theta=spec.theta)
    cap = (max(spec.lengths) + 63) // 64 * 64
    kc = torch.empty(spec.n_seq, spec.n_kv_heads, cap, 128, dtype=bf, device=dev)
    vc = torch.empty_like(kc)
    qg, kg = up(x["q_gamma"]), up(x["k_gamma"])
    B.prefill(p, up(x["q"][pre]), up(x["k"][pre]), up(x["v"][pre]), qg, kg, torch.from_numpy(cu_pre).to(dev),
              cu_pre, k_cache=kc, v_cache=vc)
    q, k, v = up(x["q"][new]), up(x["k"][new]), up(x["v"][new])
    sp_h = np.array(split, dtype=np.int32)
    sp, cn = torch.from_numpy(sp_h).to(dev), torch.from_numpy(cu_new).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(B.append_workspace_size(p, B.BF16, spec.n_seq, int(cu_new[-1]), new_tokens),
                     dtype=torch.uint8, device=dev)
    run = lambda: B.append(p, q, k, v, qg, kg, kc, vc, sp, cn, sp_h, cu_new, out=out, workspace=ws)
    warm_up(run)
    ev = HipEvents()
    kev = [(ev.create(), ev.create()) for _ in range(n_calls)]
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_calls)]
    torch.cuda.synchronize()
    for (ka, kb), (ca, cb) in zip(kev, cev):
        B.set_timing_events(ka, kb)
        ca.record()
        run()
        cb.record()
    torch.cuda.synchronize()
    flops = accounting.append_flops(split, [new_tokens] * spec.n_seq, spec.n_q_heads)
    k_ms = float(np.mean([ev.elapsed_ms(a, b) for a, b in kev]))
    c_ms = float(np.mean([a.elapsed_time(b) for a, b in cev]))
    workload = f"qwen3-8b-append-bf16 {spec.n_seq}x({split[0]} cached + {new_tokens} new) Hq{spec.n_q_heads} Hkv{spec.n_kv_heads}"
    return {"metric": "append attention TFLOP/s", "unit": "TFLOP/s", "workload": workload,
            "value": round(flops / (c_ms * 1e-3) / 1e12, 2), "call_ms": round(c_ms, 4),
            "roofline": {"kernel": "k_prefill_bf16", "bound": "mfma", "achieved": round(flops / (k_ms * 1e-3) / 1e12, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (k_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "kernel_ms": round(k_ms, 4), "algorithmic_flops": flops,
                         "traffic": recorded_traffic("k_prefill_bf16", "k_prefill.hip", workload)}}


def measure_gated(dev, n_calls=20):
    """The gated global layer of Qwen3-Next (head_dim 256, 16 query / 2 KV heads,
    rotary 64 of 256, zero-centred norm, sigmoid output gate): prefill of
    4 x 4096 tokens into a cache, and one decode step of 64 sequences with
    contexts U[1024, 32768]."""
    import torch
    from attention_qk_norm_amd import accounting, binding as B, inputs
    bf = torch.bfloat16
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(bf)
    res = {}

    spec = inputs.gated_case_spec(inputs.GATED_PREFILL_CASE)
    log(f"gated prefill workload: {spec.workload}")
    x = inputs.prefill_inputs(spec)
    p = B.make_gated_params(spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, rope_theta=spec.theta, rotary_dim=spec.rot)
    q, k, v = up(inputs.q_proj_rows(x["q"], x["gate"])), up(x["k"]), up(x["v"])
    qg, kg = up(x["q_gamma"]), up(x["k_gamma"])
    cu, cu_h = torch.from_numpy(x["cu_seqlens"]).to(dev), x["cu_seqlens"]
    cap = (max(spec.lengths) + 63) // 64 * 64
    kc = torch.empty(spec.n_seq, spec.n_kv_heads, cap, 256, dtype=bf, device=dev)
    vc = torch.empty_like(kc)
    out = torch.empty(spec.n_tok, spec.n_q_heads, 256, dtype=bf, device=dev)
    ws = torch.empty(B.prefill_workspace_size(p, B.BF16, spec.n_seq, spec.n_tok, max(spec.lengths), True),
                     dtype=torch.uint8, device=dev)
    run = lambda: B.prefill(p, q, k, v, qg, kg, cu, cu_h, out=out, k_cache=kc, v_cache=vc, workspace=ws)
    warm_up(run)
    c_ms, k_ms = _timed(run, n_calls)
    flops = accounting.prefill_flops(spec.lengths, spec.n_q_heads, head_dim=256)
    res["prefill"] = {
        "metric": "gated prefill attention TFLOP/s", "unit": "TFLOP/s", "workload": spec.workload,
        "value": round(flops / (c_ms * 1e-3) / 1e12, 2), "call_ms": round(c_ms, 4),
        "roofline": {"kernel": "k_prefill_wide", "bound": "mfma", "achieved": round(flops / (k_ms * 1e-3) / 1e12, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (k_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic("k_prefill_wide", "k_prefill_wide.hip", spec.workload),
                     "kernel_ms": round(k_ms, 4), "algorithmic_flops": flops}}
    del q, k, v, kc, vc, out, ws

    spec = inputs.gated_case_spec(inputs.GATED_DECODE_CASE)
    log(f"gated decode workload: {spec.workload}; building the cache")
    x = inputs.decode_new_token(spec)
    cap = (max(spec.lengths) + 1 + 63) // 64 * 64
    kc = torch.zeros(spec.n_seq, spec.n_kv_heads, cap, 256, dtype=bf, device=dev)
    vc = torch.zeros_like(kc)
    kg = up(x["k_gamma"])
    for b0 in range(0, spec.n_seq, 8):
        seqs = list(range(b0, min(spec.n_seq, b0 + 8)))
        for i, (kr, vr) in zip(seqs, inputs.decode_cache_raw_all(spec, seqs)):
            L = spec.lengths[i]
            _, kh = B.qk_norm_rope(p, None, up(kr), None, kg, torch.arange(L, dtype=torch.int32, device=dev))
            kc[i, :, :L] = kh.permute(1, 0, 2)
            vc[i, :, :L] = up(vr).permute(1, 0, 2)
        torch.cuda.synchronize()
    sp_h = x["start_pos"]
    sp = torch.from_numpy(sp_h).to(dev)
    q, k, v, qg = up(inputs.q_proj_rows(x["q"], x["gate"])), up(x["k"]), up(x["v"]), up(x["q_gamma"])
    out = torch.empty(spec.n_seq, spec.n_q_heads, 256, dtype=bf, device=dev)
    ws = torch.empty(B.decode_workspace_size(p, B.BF16, spec.n_seq, int(sp_h.sum())), dtype=torch.uint8, device=dev)
    run = lambda: B.decode(p, q, k, v, qg, kg, kc, vc, sp, sp_h, out=out, workspace=ws)
    warm_up(run)
    c_ms, k_ms = _timed(run, n_calls)
    kv = accounting.decode_kv_read_bytes(spec.lengths, spec.n_kv_heads, head_dim=256)
    res["decode"] = {
        "metric": "gated decode KV-read GB/s", "unit": "GB/s", "workload": spec.workload,
        "value": round(kv / (c_ms * 1e-3) / 1e9, 1), "call_ms": round(c_ms, 4), "kv_read_bytes": kv,
        "roofline": {"kernel": "k_decode_split", "bound": "hbm", "achieved": round(kv / (k_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kv / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("k_decode_split", "k_decode.hip", spec.workload),
                     "kernel_ms": round(k_ms, 4)}}
    return res


def measure_layer(dev, n_calls=20, gated=False):
    """A whole attention sublayer on the 4 x 4096 prefill with the cache write:
    the fused q/k/v projection, the core and o_proj in one
    qwattn_attention_layer call; the o_proj GEMM is also timed on its own
    through qwattn_linear.  Qwen3-8B (hidden 4096, 32 / 8 heads of 128), or
    with ``gated`` the global-attention sublayer of Qwen3-Next-80B-A3B (hidden
    2048, 16 / 2 heads of 256, q_proj giving each head's query and gate,
    rotary 64, sigmoid output gate)."""
    import torch
    from attention_qk_norm_amd import accounting, binding as B, inputs
    bf = torch.bfloat16
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(bf)
    spec = inputs.gated_layer_case_spec() if gated else inputs.layer_case_spec()
    hidden = inputs.LAYER_HIDDEN[spec.case_id]
    d = spec.head_dim
    q_w = 2 * d if gated else d
    log(f"sublayer workload: {spec.workload}")
    w_qkv, w_o = inputs.layer_weights(spec, hidden)
    x = up(inputs.layer_x(spec, hidden))
    w_qkv, w_o = up(w_qkv), up(w_o)
    gq, gk = (up(g) for g in inputs.gammas(spec))
    if gated:
        p = B.make_gated_params(spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, rope_theta=spec.theta,
                                rotary_dim=spec.rot)
    else:
        p = B.make_params(spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, rope_theta=spec.theta)
    cu_h = spec.cu_seqlens()
    cu = torch.from_numpy(cu_h).to(dev)
    kc = torch.empty(spec.n_seq, spec.n_kv_heads, max(spec.lengths), d, dtype=bf, device=dev)
    vc = torch.empty_like(kc)
    y = torch.empty(spec.n_tok, hidden, dtype=bf, device=dev)
    ws = torch.empty(B.attention_layer_workspace_size(p, B.BF16, hidden, spec.n_seq, spec.n_tok, max(spec.lengths),
                                                      True), dtype=torch.uint8, device=dev)
    run = lambda: B.attention_layer(p, x, w_qkv, w_o, gq, gk, cu, cu_h, y=y, k_cache=kc, v_cache=vc, workspace=ws)
    warm_up(run)
    c_ms, qkv_ms = _timed(run, n_calls)
    o_in = torch.empty(spec.n_tok, spec.n_q_heads * d, dtype=bf, device=dev).normal_()
    run_o = lambda: B.linear(o_in, w_o, y=y)
    warm_up(run_o)
    _, o_ms = _timed(run_o, n_calls)
    qkv_flops = 2 * spec.n_tok * hidden * (spec.n_q_heads * q_w + 2 * spec.n_kv_heads * d)
    o_flops = 2 * spec.n_tok * spec.n_q_heads * d * hidden
    attn_flops = accounting.prefill_flops(spec.lengths, spec.n_q_heads, head_dim=d)
    total = qkv_flops + attn_flops + o_flops
    gemm = lambda f, ms: {"achieved": round(f / (ms * 1e-3) / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(f / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                          "kernel_ms": round(ms, 4), "algorithmic_flops": f}
    kname = "k_gemm_qkv_gated" if gated else "k_gemm_qkv"
    what = "query|gate, k, v" if gated else "q/k/v"
    return {"metric": f"attention sublayer TFLOP/s ({what} projection + core + o_proj)", "unit": "TFLOP/s",
            "workload": spec.workload, "value": round(total / (c_ms * 1e-3) / 1e12, 2), "call_ms": round(c_ms, 4),
            "algorithmic_flops": total,
            "roofline": dict(kernel=f"k_gemm<{'qkv_gated' if gated else 'qkv'}> (fused {what} projection)",
                             bound="mfma", **gemm(qkv_flops, qkv_ms),
                             traffic=recorded_traffic(kname, "k_gemm.hip", spec.workload)),
            "o_proj": dict(kernel="k_gemm<plain> via qwattn_linear", bound="mfma", **gemm(o_flops, o_ms),
                           traffic=recorded_traffic("k_gemm_plain", "k_gemm.hip", spec.workload))}


def measure_fp32_parity(dev, n_calls=50):
    """The fp32 parity workload (Qwen3-0.6B heads: 1 x 128 tokens, 16 / 8 heads,
    fp32 in and out, fp32 arithmetic throughout): its time, and its share of
    the fp32 peak as information only (67.6 MFLOP is a few microseconds of
    work, so the launches dominate)."""
    import torch
    from attention_qk_norm_amd import accounting, binding as B, inputs
    spec = inputs.case_spec(0)
    x = inputs.prefill_inputs(spec)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, k, v, qg, kg = (up(x[n]) for n in ("q", "k", "v", "q_gamma", "k_gamma"))
    cu_h = x["cu_seqlens"]
    cu = torch.from_numpy(cu_h).to(dev)
    p = B.make_params(spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, rope_theta=spec.theta)
    out = torch.empty_like(q)
    ws = torch.empty(B.prefill_workspace_size(p, B.F32, spec.n_seq, spec.n_tok, max(spec.lengths), False),
                     dtype=torch.uint8, device=dev)
    run = lambda: B.prefill(p, q, k, v, qg, kg, cu, cu_h, out=out, workspace=ws)
    warm_up(run, seconds=0.1)
    c_ms, k_ms = _timed(run, n_calls)
    flops = accounting.prefill_flops(spec.lengths, spec.n_q_heads)
    return {"metric": "fp32 prefill TFLOP/s (parity workload; information only)", "unit": "TFLOP/s",
            "workload": spec.workload, "dtype": "f32", "value": round(flops / (c_ms * 1e-3) / 1e12, 4),
            "call_ms": round(c_ms, 4), "kernel_ms": round(k_ms, 4), "algorithmic_flops": flops,
            "kernel_frac_fp32_peak": round(flops / (k_ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 5),
            "fp32_peak_tflops": FP32_PEAK_TFLOPS}


def copy_calibration(dev):
    """One 1 GiB device-to-device copy, whose counter readings scale the
    FETCH_SIZE / WRITE_SIZE figures of a counter run."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return {"read": 1 << 30, "write": 1 << 30}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return None


def stratified_rows(L, block, stride, rng):
    """Query rows of a stratified sample: the rows of each sequence are cut into
    blocks of `block` rows, the blocks into strata of `stride` consecutive
    blocks; one block per stratum is drawn, and the last block is always in."""
    n_blocks = (L + block - 1) // block
    picks = set()
    for s0 in range(0, n_blocks, stride):
        picks.add(int(rng.integers(s0, min(n_blocks, s0 + stride))))
    picks.add(n_blocks - 1)
    return np.concatenate([np.arange(b * block, min(L, (b + 1) * block)) for b in sorted(picks)])


def cpu_baseline_prefill(spec, stride=16, block=128, seed=0x51A7):
    """The oracle, as it stands, on a seeded stratified sample of the prefill
    workload: 1 in `stride` query-row blocks of every sequence (all query
    heads, the sequence's last block always in), each row by the oracle's
    definition with every key it sees.  Its time scaled by all causal pairs
    over the sampled pairs is the extrapolated time of the whole workload."""
    import oracle
    from attention_qk_norm_amd import accounting, inputs
    rng = np.random.default_rng(seed)
    gq, gk = inputs.gammas(spec)
    dt, pairs = 0.0, 0
    n_rows = 0
    for sq in range(spec.n_seq):
        L = spec.lengths[sq]
        rows = stratified_rows(L, block, stride, rng)
        starts = sorted(set(int(r) // block * block for r in rows))
        q = np.concatenate([inputs.prefill_seq_rows(spec, sq, a, min(L, a + block), "q") for a in starts])
        k = inputs.prefill_seq_rows(spec, sq, 0, int(rows.max()) + 1, "k")
        v = inputs.prefill_seq_rows(spec, sq, 0, int(rows.max()) + 1, "v")
        t0 = time.perf_counter()
        oracle.attention_prefill_rows(q, k, v, gq, gk, rows, np.arange(spec.n_q_heads), spec.n_q_heads,
                                      spec.n_kv_heads, eps=spec.eps, theta=spec.theta)
        dt += time.perf_counter() - t0
        pairs += int((rows + 1).sum())
        n_rows += len(rows)
    total_pairs = accounting.prefill_pairs(spec.lengths)
    flops = accounting.prefill_flops(spec.lengths, spec.n_q_heads)
    full_s = dt * total_pairs / pairs
    return {"value": flops / full_s / 1e12, "unit": "TFLOP/s", "cores": os.cpu_count(), "blas_threads": _blas_threads(),
            "kind": "oracle", "seconds": round(dt, 2), "extrapolated_seconds": round(full_s, 1),
            "sample": f"{spec.workload}: seeded stratified sample of 1 in {stride} query-row blocks of {block} rows "
                      f"per sequence (the last block always in), {n_rows} rows x all {spec.n_q_heads} query heads "
                      f"({pairs / total_pairs:.4f} of the causal pairs), each row with every key it sees; numpy "
                      "float64 oracle; time extrapolated by causal pairs (labelled: extrapolated)"}


def cpu_baseline_decode(spec, n_sample=8, seed=0x51A7):
    """The oracle's decode on a seeded sample of the batch's sequences (their
    caches' keys normed and rotated by the oracle beforehand, untimed: a cache
    holds them so), in KV-read GB/s over the sampled sequences' cache bytes."""
    import oracle
    from attention_qk_norm_amd import accounting, inputs
    rng = np.random.default_rng(seed)
    seqs = sorted(rng.choice(spec.n_seq, size=min(n_sample, spec.n_seq), replace=False).tolist())
    x = inputs.decode_new_token(spec)
    raws = inputs.decode_cache_raw_all(spec, seqs)
    dt = 0.0
    for i, (kr, vr) in zip(seqs, raws):
        L = spec.lengths[i]
        kh = oracle.qk_norm_rope(kr, x["k_gamma"], np.arange(L), spec.eps, spec.theta)
        t0 = time.perf_counter()
        oracle.attention_decode(x["q"][i:i + 1], x["k"][i:i + 1], x["v"][i:i + 1], x["q_gamma"], x["k_gamma"],
                                [kh], [vr], [L], spec.n_q_heads, spec.n_kv_heads, eps=spec.eps, theta=spec.theta)
        dt += time.perf_counter() - t0
    kv = accounting.decode_kv_read_bytes([spec.lengths[i] for i in seqs], spec.n_kv_heads)
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": os.cpu_count(), "blas_threads": _blas_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{spec.workload}: {len(seqs)} seeded sequences of the 64 ({sum(spec.lengths[i] for i in seqs)} "
                      "cached tokens), one decode step each; numpy float64 oracle, KV bytes read over its time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefill-case", type=int, default=HEADLINE_PREFILL, choices=[1, 3, 4],
                    help="the prefill workload of the step (default: the long prefill)")
    ap.add_argument("--extra-prefill", default=EXTRA_PREFILL,
                    help="comma-separated prefill workloads timed beside the steps, or 'none'")
    ap.add_argument("--decode-case", type=int, default=2)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip the chunked-prefill (append) measurement")
    ap.add_argument("--no-gated", action="store_true", help="skip the gated-layer (head_dim 256) measurements")
    ap.add_argument("--no-layer", action="store_true", help="skip the whole-sublayer (projections) measurement")
    ap.add_argument("--only", choices=["append", "gated", "layer", "gated_layer"],
                    help="profiling aid: run only this measurement and print its record (no step, not a bench line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one 1 GiB device-to-device copy kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention core shards by KV head or sequence with no "
              "exchange between GPUs, so one GPU's share at its real shape is what is timed (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    extra = [] if args.extra_prefill in ("", "none") else [int(c) for c in args.extra_prefill.split(",")]
    extra = [c for c in extra if c != args.prefill_case]

    import torch
    from attention_qk_norm_amd import accounting, binding as B
    B.load()
    dev = torch.device("cuda:0")
    if args.only:
        rec = {"append": measure_append, "gated": measure_gated, "layer": measure_layer,
               "gated_layer": lambda d: measure_layer(d, gated=True)}[args.only](dev)
        if args.copy_calibration:
            rec["copy_calibration_bytes"] = copy_calibration(dev)
        print(json.dumps({args.only: rec}), flush=True)
        return
    pre = setup_prefill(args.prefill_case, dev)
    dec = None if args.no_decode else setup_decode(args.decode_case, dev)
    ev = HipEvents()
    n = args.steps
    pre_ev = [(ev.create(), ev.create()) for _ in range(n)]
    dec_ev = [(ev.create(), ev.create()) for _ in range(n)]
    call_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]

    def step(i=None):
        if i is not None:
            B.set_timing_events(*pre_ev[i])
            call_ev[i][0].record()
        run_prefill(pre)
        if i is not None:
            call_ev[i][1].record()
        if dec is not None:
            if i is not None:
                B.set_timing_events(*dec_ev[i])
                call_ev[i][2].record()
            run_decode(dec)
            if i is not None:
                call_ev[i][3].record()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {n} steps")
    t0 = time.perf_counter()
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    log("measured peaks (MFMA loop, streaming read)")
    # the read source must dwarf the 256 MB Infinity Cache: the decode K cache
    # (4.3 GB at the 64-sequence workload), else a temporary 2 GiB buffer
    peaks = measure_peaks(dev, dec["kc"] if dec is not None else torch.ones(1 << 29, dtype=torch.int32, device=dev))

    spec = pre["spec"]
    headline = prefill_record(spec, [e[0].elapsed_time(e[1]) for e in call_ev],
                              [ev.elapsed_ms(a, b) for a, b in pre_ev], peaks)
    rec = {
        "metric": "prefill attention TFLOP/s (causal GQA with fused QK-Norm+RoPE)",
        "value": headline["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": round(wall / n * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec.workload, "global_batch": spec.n_seq, "seq_len": max(spec.lengths),
                   "n_q_heads": spec.n_q_heads, "n_kv_heads": spec.n_kv_heads, "head_dim": 128,
                   "rope_theta": spec.theta, "parallelism": "single-gpu",
                   "decode_workload": None if dec is None else dec["spec"].workload},
        "prefill_call_ms": headline["call_ms"],
        "prefill_call_ms_p10_p50_p90": headline["call_ms_p10_p50_p90"],
        "prefill_frac_mfma_peak": headline["frac_mfma_peak"],
        "roofline": headline["roofline"],
    }
    if dec is not None:
        ds = dec["spec"]
        kv_bytes = accounting.decode_kv_read_bytes(ds.lengths, ds.n_kv_heads)
        split_all = [ev.elapsed_ms(a, b) for a, b in dec_ev]
        dec_call_all = [e[2].elapsed_time(e[3]) for e in call_ev]
        split_ms = float(np.mean(split_all))
        dec_call_ms = float(np.mean(dec_call_all))
        rec["decode"] = {
            "metric": "decode KV-read GB/s", "unit": "GB/s", "workload": ds.workload,
            "value": round(kv_bytes / (dec_call_ms * 1e-3) / 1e9, 1), "call_ms": round(dec_call_ms, 4),
            "call_ms_p10_p50_p90": pct(dec_call_all),
            "frac_hbm_peak": round(kv_bytes / (dec_call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kv_read_bytes": kv_bytes,
            "roofline": {"kernel": "k_decode_split", "bound": "hbm",
                         "achieved": round(kv_bytes / (split_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(kv_bytes / (split_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": recorded_traffic("k_decode_split", "k_decode.hip", ds.workload),
                         "kernel_ms": round(split_ms, 4), "kernel_ms_p10_p50_p90": pct(split_all),
                         "measured_peak": {"value": peaks["hbm_read_gbs"], "unit": "GB/s",
                                           "frac": round(kv_bytes / (split_ms * 1e-3) / 1e9 / peaks["hbm_read_gbs"], 4),
                                           "how": f"one nontemporal streaming read of {peaks['hbm_read_bytes']} bytes "
                                                  "(the K cache), this run (qwattn_hbm_read_probe)"}},
        }
    del pre, dec
    torch.cuda.empty_cache()
    if extra:
        rec["prefill_workloads"] = {}
        for c in extra:
            log(f"prefill workload {c}")
            rec["prefill_workloads"][str(c)] = measure_prefill_workload(c, dev)
    if not args.no_append:
        log("append (chunked prefill) measurement")
        rec["append"] = measure_append(dev)
    if not args.no_gated:
        torch.cuda.empty_cache()
        log("gated-layer measurements")
        rec["gated"] = measure_gated(dev)
    if not args.no_layer:
        torch.cuda.empty_cache()
        log("sublayer measurement")
        rec["layer"] = measure_layer(dev)
        if not args.no_gated:
            torch.cuda.empty_cache()
            log("gated sublayer measurement")
            rec["gated_layer"] = measure_layer(dev, gated=True)
    log("fp32 parity workload")
    rec["fp32_parity"] = measure_fp32_parity(dev)
    if args.copy_calibration:
        rec["copy_calibration_bytes"] = copy_calibration(dev)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a stratified sample of the prefill workload")
        rec["cpu_baseline"] = cpu_baseline_prefill(spec)
        if "decode" in rec:
            from attention_qk_norm_amd import inputs
            log("timing the CPU oracle on a sample of the decode workload")
            rec["decode"]["cpu_baseline"] = cpu_baseline_decode(inputs.case_spec(args.decode_case))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
