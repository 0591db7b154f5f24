"""Seeded synthetic inputs for the attention-sublayer core.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the method's arithmetic.  Both the HIP path and the CPU oracle
consume exactly the values it returns (float32 numpy arrays whose values are
already representable in the case's dtype, so the bf16 upload and the float64
oracle conversion are both exact).

Recipe (every draw is reproducible on its own, so any sequence or token block
of a full-size case can be regenerated without drawing the rest):
  * seed key ``[0x51A7, case_id, stream, ...]`` for ``numpy.random.PCG64``
    through ``SeedSequence``;
  * stream 0: sequence lengths; stream 1: per-head scales
    s = exp(U(ln 0.1, ln 30)) for q (Hq), k (Hkv), v (Hkv); stream 2: gamma_q
    and gamma_k = 1 + 0.1 N(0, 1) over head_dim;
  * streams 3, 4, 5: q, k, v rows, N(0, 1) float32 times the head's scale,
    drawn per (sequence, 1024-token block); streams 6, 7: the raw K and V
    already in a decode cache, per (sequence, 1024-token block);
  * bf16 cases round every value to bf16 with round-to-nearest-even.
Gated-layer cases (head_dim 256, the Qwen3-Next / Qwen3.5 global layers) use
the same streams at head_dim 256, norm weights w = 0.1 N(0, 1) (the
zero-centred norm scales by 1 + w, so the scales match the Qwen3 cases), and
stream 8: the output-gate pre-activations, 2 N(0, 1) per (token, head, dim)
(sigmoid then spans about 0.02 .. 0.98).
Sublayer cases (projections around the core): stream 9, the layer input rows
x ~ N(0, 1) per (sequence, 1024-token block); streams 10 and 11, the stacked
q/k/v weight and the o_proj weight, N(0, 1) / sqrt(fan-in) per 1024-row block
(so q, k, v and y come out with unit scale).
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 0x51A7
HEAD_DIM = 128
BLOCK_TOKENS = 1024

S_LENGTHS, S_SCALES, S_GAMMA, S_Q, S_K, S_V, S_CACHE_K, S_CACHE_V, S_GATE, S_X, S_WQKV, S_WO = range(12)
GATED_HEAD_DIM = 256
GATE_SCALE = 2.0


def round_to_bf16(x):
    """float32 array -> float32 array holding the nearest bf16 values (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x):
    """bf16-exact float32 array -> int16 array of its bf16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16).view(np.int16)


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL


@dataclass
class CaseSpec:
    """Shape and distribution of one synthetic case."""
    case_id: int
    workload: str
    dtype: str                 # "f32" or "bf16"
    n_q_heads: int
    n_kv_heads: int
    theta: float
    kind: str                  # "prefill" or "decode"
    lengths: list = field(default_factory=list)   # prefill: per-sequence L; decode: cached L_i
    eps: float = 1e-6
    head_dim: int = HEAD_DIM
    v_scaled: bool = True      # False: v ~ N(0, 1) unscaled (q, k still scaled)
    pos_offset: int = 0
    gated: bool = False        # gated global layer: zero-centred norm, partial RoPE, output gate
    rot: int = HEAD_DIM        # rotated coordinates

    @property
    def g(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_seq(self):
        return len(self.lengths)

    @property
    def n_tok(self):
        return int(sum(self.lengths)) if self.kind == "prefill" else len(self.lengths)

    def cu_seqlens(self):
        cu = np.zeros(len(self.lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.lengths)
        return cu


def _lengths(case_id, rule):
    rng = _rng(SEED_ROOT, case_id, S_LENGTHS)
    kind = rule[0]
    if kind == "fixed":
        return [int(x) for x in rule[1]]
    if kind == "uniform":          # integers in [lo, hi]
        _, n, lo, hi = rule
        return [int(x) for x in rng.integers(lo, hi + 1, size=n)]
    if kind == "loguniform":       # round(exp(U(ln lo, ln hi)))
        _, n, lo, hi = rule
        return [int(round(math.exp(x))) for x in rng.uniform(math.log(lo), math.log(hi), size=n)]
    raise ValueError(rule)


# The five Qwen3-shaped workloads (head_dim 128 throughout).
_CASE_TABLE = {
    0: ("qwen3-0.6b-layer-f32 B1 T128 Hq16 Hkv8", "f32", 16, 8, 1e6, "prefill", ("fixed", [128])),
    1: ("qwen3-8b-prefill-bf16 B4 T4096 Hq32 Hkv8", "bf16", 32, 8, 1e6, "prefill", ("fixed", [4096] * 4)),
    2: ("qwen3-8b-decode-bf16 64seq ctx U[1024,32768] Hq32 Hkv8", "bf16", 32, 8, 1e6, "decode",
        ("uniform", 64, 1024, 32768)),
    3: ("qwen3-32b-long-prefill-bf16 B1 T32768 Hq64 Hkv8", "bf16", 64, 8, 1e6, "prefill", ("fixed", [32768])),
    4: ("qwen3-235b-a22b-attn-ragged-prefill-bf16 16seq L logU[256,16384] Hq64 Hkv4", "bf16", 64, 4, 1e7,
        "prefill", ("loguniform", 16, 256, 16384)),
}


def case_spec(case_id, v_scaled=True):
    """Spec of one of the five standard workloads."""
    workload, dtype, hq, hkv, theta, kind, rule = _CASE_TABLE[case_id]
    return CaseSpec(case_id=case_id, workload=workload, dtype=dtype, n_q_heads=hq, n_kv_heads=hkv,
                    theta=theta, kind=kind, lengths=_lengths(case_id, rule), v_scaled=v_scaled)


def custom_spec(case_id, dtype, n_q_heads, n_kv_heads, lengths, kind="prefill", theta=1e6,
                v_scaled=True, eps=1e-6):
    """Spec for a test shape; ``case_id`` (>= 100 by convention) seeds it."""
    return CaseSpec(case_id=case_id, workload=f"custom-{case_id}", dtype=dtype,
                    n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, theta=theta, kind=kind,
                    lengths=[int(x) for x in lengths], v_scaled=v_scaled, eps=eps)


# The gated global layer of Qwen3-Next-80B-A3B (2 KV heads, head_dim 256,
# partial rotary factor 0.25; 16 query heads) at the prefill shape of the
# Qwen3-8B workload, and a 64-sequence decode over the same context mix.
GATED_PREFILL_CASE = 5
GATED_DECODE_CASE = 6


def gated_case_spec(case_id):
    """Spec of the gated-layer workloads (prefill 5, decode 6)."""
    if case_id == GATED_PREFILL_CASE:
        return gated_spec(case_id, "bf16", 16, 2, [4096] * 4, rot=64,
                          workload="qwen3-next-global-layer-prefill-bf16 B4 T4096 Hq16 Hkv2 d256 rot64")
    if case_id == GATED_DECODE_CASE:
        return gated_spec(case_id, "bf16", 16, 2, _lengths(case_id, ("uniform", 64, 1024, 32768)), kind="decode",
                          rot=64, workload="qwen3-next-global-layer-decode-bf16 64seq ctx U[1024,32768] Hq16 Hkv2 d256")
    raise ValueError(case_id)


# The attention sublayer of Qwen3-8B (hidden 4096, 32 / 8 heads) at the
# 4 x 4096 prefill shape, and the gated global-attention sublayer of
# Qwen3-Next-80B-A3B (hidden 2048, 16 / 2 heads of 256, 25% rotary, theta 1e7)
# at the same token shape.
LAYER_CASE = 7
GATED_LAYER_CASE = 8
LAYER_HIDDEN = {LAYER_CASE: 4096, GATED_LAYER_CASE: 2048}


def layer_case_spec():
    spec = case_spec(1)
    spec.case_id = LAYER_CASE
    spec.workload = "qwen3-8b-attention-sublayer-bf16 B4 T4096 hidden4096 Hq32 Hkv8"
    return spec


def gated_layer_case_spec():
    return gated_spec(GATED_LAYER_CASE, "bf16", 16, 2, [4096] * 4, rot=64,
                      workload="qwen3-next-gated-sublayer-bf16 B4 T4096 hidden2048 Hq16 Hkv2 d256 rot64")


def _weight(spec, stream, rows, cols):
    out = np.empty((rows, cols), dtype=np.float32)

    def run(b):
        r1 = min(rows, b + BLOCK_TOKENS)
        w = _rng(SEED_ROOT, spec.case_id, stream, b // BLOCK_TOKENS).standard_normal((r1 - b, cols), dtype=np.float32)
        out[b:r1] = _store(w * np.float32(1.0 / math.sqrt(cols)), spec.dtype)

    list(_pool().map(run, range(0, rows, BLOCK_TOKENS)))
    return out


def layer_weights(spec, hidden):
    """(w_qkv [Hq q_w + 2 Hkv d, hidden], w_o [hidden, Hq d]): the stacked q/k/v
    projection weights and the o_proj weight, each stored [out][in]; q_w = d,
    or 2 d for a gated layer (per query head its query rows, then its gate
    rows)."""
    d = spec.head_dim
    q_w = 2 * d if spec.gated else d
    return (_weight(spec, S_WQKV, spec.n_q_heads * q_w + 2 * spec.n_kv_heads * d, hidden),
            _weight(spec, S_WO, hidden, spec.n_q_heads * d))


def layer_x(spec, hidden, seq=None, lo=0, hi=None):
    """Layer input rows: all sequences packed [n_tok, hidden], or rows lo..hi-1
    of sequence ``seq``."""
    def rows(s, a, b):
        L = spec.lengths[s]
        out = np.empty((b - a, hidden), dtype=np.float32)
        for blk in range(a // BLOCK_TOKENS, (b - 1) // BLOCK_TOKENS + 1 if b > a else 0):
            s0 = blk * BLOCK_TOKENS
            n = min(BLOCK_TOKENS, L - s0)
            x = _store(_rng(SEED_ROOT, spec.case_id, S_X, s, blk).standard_normal((n, hidden), dtype=np.float32),
                       spec.dtype)
            c0, c1 = max(a, s0), min(b, s0 + n)
            out[c0 - a:c1 - a] = x[c0 - s0:c1 - s0]
        return out

    if seq is not None:
        return rows(seq, lo, spec.lengths[seq] if hi is None else hi)
    cu = spec.cu_seqlens()
    out = np.empty((int(cu[-1]), hidden), dtype=np.float32)

    def run(s):
        out[cu[s]:cu[s + 1]] = rows(s, 0, spec.lengths[s])

    list(_pool().map(run, range(spec.n_seq)))
    return out


def gated_spec(case_id, dtype, n_q_heads, n_kv_heads, lengths, kind="prefill", theta=1e7, rot=64,
               v_scaled=True, eps=1e-6, workload=None):
    """Spec of a gated global-attention layer shape (head_dim 256)."""
    return CaseSpec(case_id=case_id, workload=workload or f"gated-{case_id}", dtype=dtype,
                    n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, theta=theta, kind=kind,
                    lengths=[int(x) for x in lengths], v_scaled=v_scaled, eps=eps,
                    head_dim=GATED_HEAD_DIM, gated=True, rot=rot)


def _store(x, dtype):
    return round_to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def head_scales(spec):
    """Per-head scales (s_q [Hq], s_k [Hkv], s_v [Hkv]) as float32."""
    rng = _rng(SEED_ROOT, spec.case_id, S_SCALES)
    lo, hi = math.log(0.1), math.log(30.0)
    sq = np.exp(rng.uniform(lo, hi, size=spec.n_q_heads)).astype(np.float32)
    sk = np.exp(rng.uniform(lo, hi, size=spec.n_kv_heads)).astype(np.float32)
    sv = np.exp(rng.uniform(lo, hi, size=spec.n_kv_heads)).astype(np.float32)
    if not spec.v_scaled:
        sv = np.ones_like(sv)
    return sq, sk, sv


def gammas(spec):
    """(gamma_q, gamma_k), each 1 + 0.1 N(0, 1) over head_dim, in the case dtype
    (gated layers: the zero-centred weights w = 0.1 N(0, 1))."""
    rng = _rng(SEED_ROOT, spec.case_id, S_GAMMA)
    base = 0.0 if spec.gated else 1.0
    gq = base + 0.1 * rng.standard_normal(spec.head_dim)
    gk = base + 0.1 * rng.standard_normal(spec.head_dim)
    return _store(gq.astype(np.float32), spec.dtype), _store(gk.astype(np.float32), spec.dtype)


def _gate_scale(spec):
    return np.full(spec.n_q_heads, GATE_SCALE, dtype=np.float32)


def _block(spec, stream, seq, blk, n, heads, scale):
    rng = _rng(SEED_ROOT, spec.case_id, stream, seq, blk)
    x = rng.standard_normal((n, heads, spec.head_dim), dtype=np.float32)
    x *= scale[None, :, None]
    return _store(x, spec.dtype)


def seq_rows(spec, stream, seq, length, heads, scale, lo=0, hi=None):
    """Rows lo..hi-1 of one sequence's tensor for ``stream`` ([hi-lo, heads, d])."""
    hi = length if hi is None else hi
    out = np.empty((hi - lo, heads, spec.head_dim), dtype=np.float32)
    b0, b1 = lo // BLOCK_TOKENS, (hi - 1) // BLOCK_TOKENS if hi > lo else -1
    for b in range(b0, b1 + 1):
        a = b * BLOCK_TOKENS
        n = min(BLOCK_TOKENS, length - a)
        blk = _block(spec, stream, seq, b, n, heads, scale)
        s0, s1 = max(lo, a), min(hi, a + n)
        out[s0 - lo:s1 - lo] = blk[s0 - a:s1 - a]
    return out


def _packed(spec, stream, heads, scale):
    """Tensor of all sequences packed token-major: [n_tok, heads, d]."""
    cu = spec.cu_seqlens()
    out = np.empty((int(cu[-1]), heads, spec.head_dim), dtype=np.float32)
    jobs = []
    for s, length in enumerate(spec.lengths):
        for b in range(0, (length + BLOCK_TOKENS - 1) // BLOCK_TOKENS):
            jobs.append((s, b, length))

    def run(job):
        s, b, length = job
        a = b * BLOCK_TOKENS
        n = min(BLOCK_TOKENS, length - a)
        out[cu[s] + a:cu[s] + a + n] = _block(spec, stream, s, b, n, heads, scale)

    list(_pool().map(run, jobs))
    return out


def prefill_inputs(spec):
    """dict(q, k, v, q_gamma, k_gamma, cu_seqlens) for a prefill case."""
    assert spec.kind == "prefill"
    sq, sk, sv = head_scales(spec)
    gq, gk = gammas(spec)
    x = dict(q=_packed(spec, S_Q, spec.n_q_heads, sq),
             k=_packed(spec, S_K, spec.n_kv_heads, sk),
             v=_packed(spec, S_V, spec.n_kv_heads, sv),
             q_gamma=gq, k_gamma=gk, cu_seqlens=spec.cu_seqlens())
    if spec.gated:
        x["gate"] = _packed(spec, S_GATE, spec.n_q_heads, _gate_scale(spec))
    return x


def q_proj_rows(q, gate):
    """The q_proj output layout of a gated layer: per head the query, then the
    gate ([n, H, d] twice -> [n, H, 2d])."""
    return np.ascontiguousarray(np.concatenate([q, gate], axis=-1))


def prefill_seq_rows(spec, seq, lo, hi, which):
    """Rows lo..hi-1 of sequence ``seq`` of 'q', 'k' or 'v' (for sampled checks)."""
    sq, sk, sv = head_scales(spec)
    stream, heads, scale = {"q": (S_Q, spec.n_q_heads, sq), "k": (S_K, spec.n_kv_heads, sk),
                            "v": (S_V, spec.n_kv_heads, sv),
                            "gate": (S_GATE, spec.n_q_heads, _gate_scale(spec))}[which]
    return seq_rows(spec, stream, seq, spec.lengths[seq], heads, scale, lo, hi)


def decode_new_token(spec):
    """dict(q [n_seq,Hq,d], k, v [n_seq,Hkv,d], q_gamma, k_gamma, start_pos) for a decode case.

    The new token of sequence i is drawn as row L_i of that sequence's q/k/v
    streams, so it is the token that follows its cached context."""
    assert spec.kind == "decode"
    sq, sk, sv = head_scales(spec)
    gq, gk = gammas(spec)
    q = np.stack([seq_rows(spec, S_Q, i, L + 1, spec.n_q_heads, sq, L, L + 1)[0]
                  for i, L in enumerate(spec.lengths)])
    k = np.stack([seq_rows(spec, S_K, i, L + 1, spec.n_kv_heads, sk, L, L + 1)[0]
                  for i, L in enumerate(spec.lengths)])
    v = np.stack([seq_rows(spec, S_V, i, L + 1, spec.n_kv_heads, sv, L, L + 1)[0]
                  for i, L in enumerate(spec.lengths)])
    x = dict(q=q, k=k, v=v, q_gamma=gq, k_gamma=gk, start_pos=np.asarray(spec.lengths, dtype=np.int32))
    if spec.gated:
        x["gate"] = np.stack([seq_rows(spec, S_GATE, i, L + 1, spec.n_q_heads, _gate_scale(spec), L, L + 1)[0]
                              for i, L in enumerate(spec.lengths)])
    return x


def decode_cache_raw(spec, seq):
    """Raw (not yet normed or rotated) K and the V of sequence ``seq``'s cached
    context, positions 0 .. L-1: two ``[L, Hkv, d]`` arrays."""
    _, sk, sv = head_scales(spec)
    L = spec.lengths[seq]
    return (seq_rows(spec, S_CACHE_K, seq, L, spec.n_kv_heads, sk),
            seq_rows(spec, S_CACHE_V, seq, L, spec.n_kv_heads, sv))


def decode_cache_raw_all(spec, seqs=None):
    """decode_cache_raw for many sequences, drawn in parallel; list of (k, v)."""
    seqs = range(spec.n_seq) if seqs is None else seqs
    return list(_pool().map(lambda i: decode_cache_raw(spec, i), list(seqs)))
