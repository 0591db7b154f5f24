"""The entry points under HIP graph capture.

The library allocates nothing, copies nothing and never synchronises inside a
call (the caller passes the workspace), so a prefill and a decode can be
captured once and replayed.  Each replay is checked bit for bit against an
eager call on the same inputs (every kernel is deterministic), with eager work,
synchronisations and new input values between the replays."""

import pytest
import torch

from attention_qk_norm_amd import binding as B
from attention_qk_norm_amd import inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_util as U
else:  # collected on a CPU-only machine: every test here is deselected by -m "not gpu"
    U = None


def _prefill_set(cid, spec_lengths):
    spec = inputs.custom_spec(cid, "bf16", 8, 2, spec_lengths)
    x = inputs.prefill_inputs(spec)
    return spec, {n: U.up(x[n], torch.bfloat16) for n in ("q", "k", "v", "q_gamma", "k_gamma")}, x["cu_seqlens"]


def _decode_set(cid, lengths):
    spec = inputs.custom_spec(cid, "bf16", 32, 8, lengths, kind="decode")
    x = inputs.decode_new_token(spec)
    return spec, x, {n: U.up(x[n], torch.bfloat16) for n in ("q", "k", "v", "q_gamma", "k_gamma")}


def test_prefill_and_decode_replay_in_a_graph():
    lengths = [300, 77, 513]
    spec, a, cu_h = _prefill_set(150, lengths)
    _, b, _ = _prefill_set(151, lengths)  # second input set, same shapes
    p = U.params(spec)
    cap = max(lengths) + 3
    cu = torch.from_numpy(cu_h).to(U.DEV)
    ws_p = torch.empty(B.prefill_workspace_size(p, B.BF16, spec.n_seq, spec.n_tok, max(lengths), True),
                       dtype=torch.uint8, device=U.DEV)

    dlen = [5, 700, 1029, 64]
    dspec, dx, da = _decode_set(152, dlen)
    _, _, db = _decode_set(153, dlen)
    dp = U.params(dspec)
    kc0, vc0, _ = U.build_decode_cache(dspec, dx, max(dlen) + 5)
    sp_h = dx["start_pos"]
    sp = torch.from_numpy(sp_h).to(U.DEV)
    ws_d = torch.empty(B.decode_workspace_size(dp, B.BF16, dspec.n_seq, int(sp_h.sum())), dtype=torch.uint8,
                       device=U.DEV)

    # the captured calls read these buffers and write these outputs
    gin = {n: t.clone() for n, t in a.items()}
    gdin = {n: t.clone() for n, t in da.items()}
    g_out = torch.empty(spec.n_tok, 8, 128, dtype=torch.bfloat16, device=U.DEV)
    g_kc = torch.full((spec.n_seq, 2, cap, 128), 7.0, dtype=torch.bfloat16, device=U.DEV)
    g_vc = torch.full_like(g_kc, 7.0)
    g_dout = torch.empty(dspec.n_seq, 32, 128, dtype=torch.bfloat16, device=U.DEV)
    g_dkc, g_dvc = kc0.clone(), vc0.clone()

    def calls(pin, din, out, kc, vc, dout, dkc, dvc):
        B.prefill(p, pin["q"], pin["k"], pin["v"], pin["q_gamma"], pin["k_gamma"], cu, cu_h, out=out,
                  k_cache=kc, v_cache=vc, workspace=ws_p)
        B.decode(dp, din["q"], din["k"], din["v"], din["q_gamma"], din["k_gamma"], dkc, dvc, sp, sp_h, out=dout,
                 workspace=ws_d)

    def eager(pin, din):
        out = torch.empty_like(g_out)
        kc, vc = torch.full_like(g_kc, 7.0), torch.full_like(g_vc, 7.0)
        dout = torch.empty_like(g_dout)
        dkc, dvc = kc0.clone(), vc0.clone()
        calls(pin, din, out, kc, vc, dout, dkc, dvc)
        torch.cuda.synchronize()
        return out, kc, vc, dout, dkc, dvc

    U.say("graph: eager warm-up on a side stream, then capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls(gin, gdin, g_out, g_kc, g_vc, g_dout, g_dkc, g_dvc)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(gin, gdin, g_out, g_kc, g_vc, g_dout, g_dkc, g_dvc)
    torch.cuda.synchronize()

    for r, (pin, din) in enumerate([(a, da), (b, db), (a, da), (b, db)]):
        U.say(f"graph replay {r}")
        for n in gin:
            gin[n].copy_(pin[n])
        for n in gdin:
            gdin[n].copy_(din[n])
        g_out.fill_(-3.0)
        g_dout.fill_(-3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = eager(pin, din)  # eager work between the replays
        got = (g_out, g_kc, g_vc, g_dout, g_dkc, g_dvc)
        for name, x, y in zip(("out", "k_cache", "v_cache", "decode out", "decode k_cache", "decode v_cache"),
                              got, ref):
            assert torch.equal(x, y), f"replay {r}: {name} differs from the eager call"
    assert bool(torch.isfinite(g_out.float()).all()) and bool(torch.isfinite(g_dout.float()).all())


@pytest.mark.parametrize("gated", [False, True], ids=["qwen3", "gated"])
def test_attention_layer_replay_in_a_graph(gated):
    """The sublayer (q/k/v projection GEMM with the norm/RoPE/cache epilogue,
    attention, o_proj GEMM) captured once and replayed on two input sets: the
    Qwen3 form (head_dim 128), and the gated form (head_dim 256: query|gate
    rows, zero-centred key norm and partial rotation in the epilogue, whose
    key heads add their sums of squares across waves through LDS)."""
    hidden, lengths = (512, [300, 129]) if gated else (1024, [300, 129])
    hq, hkv = (8, 2) if gated else (16, 8)
    make = (lambda cid: inputs.gated_spec(cid, "bf16", hq, hkv, lengths, rot=64)) if gated else \
        (lambda cid: inputs.custom_spec(cid, "bf16", hq, hkv, lengths))
    spec = make(156 if gated else 154)
    d = spec.head_dim
    w_qkv, w_o = inputs.layer_weights(spec, hidden)
    gq, gk = inputs.gammas(spec)
    bf = torch.bfloat16
    xs = [U.up(inputs.layer_x(spec, hidden), bf), U.up(inputs.layer_x(make(157 if gated else 155), hidden), bf)]
    w_qkv, w_o, gq, gk = U.up(w_qkv, bf), U.up(w_o, bf), U.up(gq, bf), U.up(gk, bf)
    p = B.make_gated_params(hq, hkv, eps=spec.eps, rope_theta=spec.theta, rotary_dim=spec.rot) if gated else U.params(spec)
    cu_h = spec.cu_seqlens()
    cu = torch.from_numpy(cu_h).to(U.DEV)
    cap = max(lengths) + 5
    ws = torch.empty(B.attention_layer_workspace_size(p, B.BF16, hidden, spec.n_seq, spec.n_tok, max(lengths), True),
                     dtype=torch.uint8, device=U.DEV)
    g_x = xs[0].clone()
    g_y = torch.empty(spec.n_tok, hidden, dtype=bf, device=U.DEV)
    g_kc = torch.full((spec.n_seq, hkv, cap, d), 7.0, dtype=bf, device=U.DEV)
    g_vc = torch.full_like(g_kc, 7.0)

    def call(x, y, kc, vc):
        B.attention_layer(p, x, w_qkv, w_o, gq, gk, cu, cu_h, y=y, k_cache=kc, v_cache=vc, workspace=ws)

    U.say("graph: sublayer warm-up on a side stream, then capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(g_x, g_y, g_kc, g_vc)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(g_x, g_y, g_kc, g_vc)
    torch.cuda.synchronize()
    for r, x in enumerate([xs[0], xs[1], xs[0]]):
        U.say(f"graph sublayer replay {r}")
        g_x.copy_(x)
        g_y.fill_(-3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y = torch.empty_like(g_y)
        kc, vc = torch.full_like(g_kc, 7.0), torch.full_like(g_vc, 7.0)
        call(x, y, kc, vc)
        torch.cuda.synchronize()
        assert torch.equal(g_y, y), f"replay {r}: y differs from the eager call"
        assert torch.equal(g_kc, kc) and torch.equal(g_vc, vc), f"replay {r}: cache differs from the eager call"
