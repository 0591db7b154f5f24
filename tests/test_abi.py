"""The C-ABI library on the CPU: it loads, exports every entry point the header
declares, and rejects invalid calls before touching a GPU (no call here
reaches a HIP runtime function: validation fails first)."""

import ctypes
import os
import re

import pytest

from attention_qk_norm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qwattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qwattn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"qwattn_qk_norm_rope", "qwattn_prefill", "qwattn_decode", "qwattn_append"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.qwattn_abi_version() == 6
    for st in range(6):
        assert lib.qwattn_status_str(st)


F = ctypes.c_void_p(0x100000)   # never dereferenced: every call below fails validation
ODD = ctypes.c_void_p(0x100002)


def cu(*vals):
    return (ctypes.c_int32 * len(vals))(*vals)


def prefill(lib, p, cu_h, n_seq, q=F, cache=(None, None, None), ws=F, ws_bytes=1 << 30, dtype=1):
    kc, vc, d = cache
    return lib.qwattn_prefill(ctypes.byref(p), dtype, q, F, F, F, F, F, cu_h, n_seq, F, kc, vc,
                              ctypes.byref(d) if d is not None else None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=30, n_kv_heads=8), B.ERR_INVALID_ARG),
    (dict(n_q_heads=0, n_kv_heads=8), B.ERR_INVALID_ARG),
    (dict(n_q_heads=32, n_kv_heads=8, head_dim=64), B.ERR_UNSUPPORTED),
    (dict(n_q_heads=32, n_kv_heads=8, order=2), B.ERR_INVALID_ARG),
    (dict(n_q_heads=32, n_kv_heads=8, rope_theta=1.0), B.ERR_INVALID_ARG),
    (dict(n_q_heads=32, n_kv_heads=8, eps=-1.0), B.ERR_INVALID_ARG),
])
def test_bad_params(lib, kw, status):
    p = B.make_params(**kw)
    assert prefill(lib, p, cu(0, 5), 1) == status
    assert lib.qwattn_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=128, rotary_dim=64), B.ERR_UNSUPPORTED),       # partial rotation runs at head_dim 256
    (dict(head_dim=128, norm_offset=1.0), B.ERR_UNSUPPORTED),
    (dict(head_dim=128, output_gate=1), B.ERR_UNSUPPORTED),
    (dict(head_dim=256, rotary_dim=48), B.ERR_UNSUPPORTED),       # 32, 64, 128, 256 only
    (dict(head_dim=256, rotary_dim=258), B.ERR_INVALID_ARG),
    (dict(head_dim=256, rotary_dim=63), B.ERR_INVALID_ARG),
    (dict(head_dim=256, rotary_dim=-64), B.ERR_INVALID_ARG),
    (dict(head_dim=256, output_gate=2), B.ERR_INVALID_ARG),
    (dict(head_dim=256, norm_offset=float("nan")), B.ERR_INVALID_ARG),
])
def test_gated_layer_params(lib, kw, status):
    """The gated-layer options (partial rotary, zero-centred norm, output gate)
    are validated before anything runs."""
    p = B.make_params(16, 2, **kw)
    assert prefill(lib, p, cu(0, 5), 1) == status
    assert lib.qwattn_last_error()


def test_gated_layer_params_accepted(lib):
    """Valid gated-layer parameters pass validation (the call then stops at a
    later check: here the workspace size)."""
    for rot in (0, 32, 64, 128, 256):
        p = B.make_params(16, 2, head_dim=256, rotary_dim=rot, norm_offset=1.0, output_gate=1)
        assert prefill(lib, p, cu(0, 5), 1, ws_bytes=16) == B.ERR_WORKSPACE
    p = B.make_gated_params(16, 2)
    assert (p.head_dim, p.rotary_dim, p.norm_offset, p.output_gate) == (256, 64, 1.0, 1)
    assert B.prefill_workspace_size(p, B.BF16, 1, 5, 5, False) > 0
    # the rotated-K buffer scales with head_dim 256; the bf16 tile is 128 rows at head_dim 256
    a = B.prefill_workspace_size(p, B.BF16, 4, 16384, 4096, False)
    b = B.prefill_workspace_size(p, B.BF16, 4, 16384, 4096, True)
    assert a - b >= 16384 * 2 * 256 * 2
    assert prefill(lib, B.make_gated_params(256, 1), cu(0, 5), 1) == B.ERR_UNSUPPORTED  # g > 128
    # a gated query may not be normalised in place (q_out would overlap the gates)
    f = lib.qwattn_qk_norm_rope
    assert f(ctypes.byref(p), 1, F, None, F, None, F, 4, F, None, None) == B.ERR_INVALID_ARG
    # the cache rows must hold head_dim 256
    d = B.CacheDesc(2 * 100 * 128, 100 * 128, 128, 100)
    assert prefill(lib, p, cu(0, 5), 1, cache=(F, F, d)) == B.ERR_INVALID_ARG


def test_bad_lengths_pointers_workspace(lib):
    p = B.make_params(32, 8)
    assert prefill(lib, p, cu(1, 5), 1) == B.ERR_INVALID_ARG          # cu[0] != 0
    assert prefill(lib, p, cu(0, 5, 3), 2) == B.ERR_INVALID_ARG       # decreasing
    assert prefill(lib, p, cu(0, 5), 1, q=ODD) == B.ERR_INVALID_ARG   # misaligned
    assert prefill(lib, p, cu(0, 5), 1, q=None) == B.ERR_INVALID_ARG  # NULL
    assert prefill(lib, p, cu(0, 5), 1, ws_bytes=16) == B.ERR_WORKSPACE
    assert prefill(lib, p, cu(0, 5), 1, ws=None) == B.ERR_WORKSPACE
    d = B.CacheDesc(8 * 4 * 128, 4 * 128, 128, 4)                      # capacity 4 < 5 tokens
    assert prefill(lib, p, cu(0, 5), 1, cache=(F, F, d)) == B.ERR_CAPACITY
    assert prefill(lib, p, cu(0, 5), 1, cache=(F, None, d)) == B.ERR_INVALID_ARG
    d2 = B.CacheDesc(8 * 8 * 130, 8 * 130, 130, 8)                     # rows not 16-byte aligned
    assert prefill(lib, p, cu(0, 5), 1, cache=(F, F, d2)) == B.ERR_INVALID_ARG
    assert prefill(lib, p, cu(0), 0) == B.OK                           # n_seq = 0: no-op
    assert prefill(lib, B.make_params(512, 1), cu(0, 5), 1) == B.ERR_UNSUPPORTED  # g > 256


def test_decode_capacity_overflow_rejected(lib):
    """An append past the cache capacity is an error with nothing enqueued."""
    p = B.make_params(32, 8)
    d = B.CacheDesc(8 * 100 * 128, 100 * 128, 128, 100)
    sp = cu(3, 99, 100)
    r = lib.qwattn_decode(ctypes.byref(p), 1, F, F, F, F, F, F, F, ctypes.byref(d), F, sp, 3, F, F, 1 << 30, None)
    assert r == B.ERR_CAPACITY
    assert b"sequence 2" in lib.qwattn_last_error()
    sp = cu(3, -1)
    r = lib.qwattn_decode(ctypes.byref(p), 1, F, F, F, F, F, F, F, ctypes.byref(d), F, sp, 2, F, F, 1 << 30, None)
    assert r == B.ERR_INVALID_ARG
    r = lib.qwattn_decode(ctypes.byref(B.make_params(64, 2)), 1, F, F, F, F, F, F, F, ctypes.byref(d), F,
                          cu(3), 1, F, F, 1 << 30, None)
    assert r == B.ERR_UNSUPPORTED  # g = 32 > 16 on the bf16 decode path


def append(lib, p, sp_h, cu_h, n_seq, cache, sp=F, q=F, ws_bytes=1 << 30, dtype=1):
    kc, vc, d = cache
    return lib.qwattn_append(ctypes.byref(p), dtype, q, F, F, F, F, kc, vc, ctypes.byref(d) if d else None, sp, sp_h,
                             F, cu_h, n_seq, F, F, ws_bytes, None)


def test_append_validation(lib):
    """Appends past the capacity, negative positions, a missing cache or missing
    positions are rejected before anything is enqueued."""
    p = B.make_params(32, 8)
    d = B.CacheDesc(8 * 100 * 128, 100 * 128, 128, 100)
    c = (F, F, d)
    assert append(lib, p, cu(90, 10), cu(0, 10, 101), 2, c) == B.ERR_CAPACITY     # 90 + 10 fits, 10 + 91 > 100
    assert b"sequence 1" in lib.qwattn_last_error()
    assert append(lib, p, cu(90, 0), cu(0, 11, 20), 2, c) == B.ERR_CAPACITY      # 90 + 11 > 100
    assert b"sequence 0" in lib.qwattn_last_error()
    assert append(lib, p, cu(-1, 0), cu(0, 1, 2), 2, c) == B.ERR_INVALID_ARG     # negative position
    assert append(lib, p, cu(0, 0), cu(0, 1, 2), 2, (None, None, None)) == B.ERR_INVALID_ARG  # no cache
    assert append(lib, p, None, cu(0, 1, 2), 2, c) == B.ERR_INVALID_ARG          # no host positions
    assert append(lib, p, cu(0, 0), cu(0, 1, 2), 2, c, sp=None) == B.ERR_INVALID_ARG
    assert append(lib, p, cu(0, 0), cu(1, 1, 2), 2, c) == B.ERR_INVALID_ARG      # cu[0] != 0
    assert append(lib, p, cu(0, 0), cu(0, 1, 2), 2, c, ws_bytes=16) == B.ERR_WORKSPACE
    assert append(lib, p, cu(), cu(0), 0, c) == B.OK                              # n_seq = 0: no-op
    assert B.append_workspace_size(p, B.BF16, 2, 20, 11) == B.prefill_workspace_size(p, B.BF16, 2, 20, 11, True)


def test_workspace_sizes(lib):
    p = B.make_params(32, 8)
    a = B.prefill_workspace_size(p, B.BF16, 4, 16384, 4096, False)
    b = B.prefill_workspace_size(p, B.BF16, 4, 16384, 4096, True)
    assert a > b > 0
    assert a - b >= 16384 * 8 * 128 * 2  # the rotated-K buffer when no cache is given
    assert B.prefill_workspace_size(B.make_params(30, 8), B.BF16, 4, 16384, 4096, False) == 0
    assert B.decode_workspace_size(p, B.BF16, 64, 1 << 20) > 64 * 32 * 128 * 2
    assert B.decode_workspace_size(p, 7, 64, 1 << 20) == 0


def test_qk_norm_rope_validation(lib):
    p = B.make_params(8, 2)
    f = lib.qwattn_qk_norm_rope
    assert f(ctypes.byref(p), 1, None, None, F, F, F, 10, None, None, None) == B.ERR_INVALID_ARG
    assert f(ctypes.byref(p), 1, F, None, F, F, F, 10, None, None, None) == B.ERR_INVALID_ARG
    assert f(ctypes.byref(p), 1, F, None, F, None, F, -1, F, None, None) == B.ERR_INVALID_ARG
    assert f(ctypes.byref(p), 1, F, None, F, None, F, 0, F, None, None) == B.OK


def test_probe_validation(lib):
    """The measurement aids reject bad arguments before any device query."""
    assert lib.qwattn_mfma_probe(0, F, None) == B.ERR_INVALID_ARG
    assert lib.qwattn_mfma_probe(-4, F, None) == B.ERR_INVALID_ARG
    assert lib.qwattn_mfma_probe(16, None, None) == B.ERR_INVALID_ARG
    assert lib.qwattn_mfma_probe(16, ODD, None) == B.ERR_INVALID_ARG
    assert lib.qwattn_mfma_probe_flops(0) == 0.0
    assert lib.qwattn_hbm_read_probe(F, 0, F, None) == B.ERR_INVALID_ARG
    assert lib.qwattn_hbm_read_probe(F, 24, F, None) == B.ERR_INVALID_ARG
    assert lib.qwattn_hbm_read_probe(None, 1 << 20, F, None) == B.ERR_INVALID_ARG
    assert lib.qwattn_hbm_read_probe(ODD, 1 << 20, F, None) == B.ERR_INVALID_ARG
    assert lib.qwattn_hbm_read_probe(F, 1 << 20, None, None) == B.ERR_INVALID_ARG


def test_cache_row_stride_beyond_32bit_tile_offsets(lib):
    """A cache whose token stride would overflow the kernels' 32-bit row offsets
    inside a 64-slot tile is rejected (not silently wrapped), for prefill,
    append and decode; the largest accepted stride passes that check."""
    p = B.make_params(32, 8)
    big = (1 << 26) // 2 + 64  # bf16 elements: one slot row > 64 MiB
    for stride_tok, status in ((big, B.ERR_UNSUPPORTED), ((1 << 26) // 2, B.ERR_WORKSPACE)):
        d = B.CacheDesc(stride_tok * 8 * 2, stride_tok * 2, stride_tok, 2)
        assert prefill(lib, p, cu(0, 2), 1, cache=(F, F, d), ws_bytes=16) == status
        if status == B.ERR_UNSUPPORTED:
            assert b"32-bit" in lib.qwattn_last_error()
        assert append(lib, p, cu(0), cu(0, 2), 1, (F, F, d), ws_bytes=16) == status
        r = lib.qwattn_decode(ctypes.byref(p), 1, F, F, F, F, F, F, F, ctypes.byref(d), F, cu(1), 1, F, F, 16, None)
        assert r == status
    # fp32 rows are 4 bytes per element: half the element stride hits the same limit
    d = B.CacheDesc(big * 8, big // 2 + 32, big // 2 + 32, 2)
    assert prefill(lib, p, cu(0, 2), 1, cache=(F, F, d), dtype=0) == B.ERR_UNSUPPORTED


def test_cache_extent_and_head_bounds(lib):
    """Strides or extents past 2^56 elements (which would overflow 64-bit
    offsets further on) and head counts past 32768 are rejected."""
    p = B.make_params(32, 8)
    d = B.CacheDesc(1 << 60, 128, 128, 2)
    assert prefill(lib, p, cu(0, 2), 1, cache=(F, F, d)) == B.ERR_INVALID_ARG
    d = B.CacheDesc(1 << 54, 128, 128, 2)                 # 4 x 2^54 + ... > 2^56
    assert prefill(lib, p, cu(0, 1, 1, 1, 1, 2), 5, cache=(F, F, d)) == B.ERR_INVALID_ARG
    assert b"extent" in lib.qwattn_last_error()
    d = B.CacheDesc(1 << 50, 1 << 47, (1 << 25) + 8, 1 << 20)  # extent ~2^50: fine; rows > 64 MiB: not
    assert prefill(lib, p, cu(0, 2), 1, cache=(F, F, d)) == B.ERR_UNSUPPORTED
    assert prefill(lib, B.make_params(65536, 65536), cu(0, 2), 1) == B.ERR_UNSUPPORTED
    assert B.prefill_workspace_size(B.make_params(65536, 8192), B.BF16, 1, 5, 5, False) == 0


def test_linear_and_layer_inner_dimension_bounds(lib):
    """Projections whose inner dimension would overflow the 32-bit panel row
    offsets, or whose tile grid is too large, are rejected."""
    f = lib.qwattn_linear
    assert f(1, F, F, 0, 128, 1 << 23, F, None) == B.OK             # the largest inner dimension (m = 0: no-op)
    assert f(1, F, F, 16, 128, (1 << 23) + 64, F, None) == B.ERR_UNSUPPORTED
    assert f(1, F, F, 1 << 31, 128, 64, F, None) == B.ERR_UNSUPPORTED
    assert f(1, F, F, (1 << 31) - 1, (1 << 31) - 128, 64, F, None) == B.ERR_UNSUPPORTED  # too many tiles
    p = B.make_params(32, 8)
    assert B.attention_layer_workspace_size(p, B.BF16, (1 << 23) + 128, 1, 5, 5, False) == 0
    assert B.attention_layer_workspace_size(p, B.BF16, 4096, 1, 5, 5, False) > 0


def test_decode_workspace_size_is_monotone(lib):
    """A decode workspace sized for a total of start positions serves every
    smaller total (the chunk length the call picks shrinks with the total, so
    the bound on the chunk count must not)."""
    for hkv, hq in ((8, 32), (2, 16), (1, 16), (4, 64)):
        for dt, d in ((B.BF16, 128), (B.F32, 128), (B.BF16, 256)):
            p = B.make_params(hq, hkv) if d == 128 else B.make_gated_params(hq, hkv)
            for n_seq in (1, 7, 64):
                prev = 0
                totals = sorted(set([0, 1, 100, 127, 128, 129] + [int(x) for x in
                                    __import__("numpy").geomspace(1, 1 << 24, 400)] +
                                    [c * m * ((2048 + hkv - 1) // hkv) + e for c in (128, 256, 512, 1024, 2048)
                                     for m in (1, 2) for e in (-n_seq - 1, -n_seq, -n_seq + 1, 0)]))
                for t in totals:
                    if t < 0:
                        continue
                    sz = B.decode_workspace_size(p, dt, n_seq, t)
                    assert sz >= prev, (hkv, dt, d, n_seq, t, sz, prev)
                    prev = sz


def test_decode_noalloc_validation_and_size_limit(lib):
    """The no-allocation decode validates like qwattn_decode, and sizes whose
    scratch exceeds the fixed array are rejected before anything is enqueued
    (no GPU is touched: the check precedes the scratch lookup)."""
    p = B.make_params(32, 8)
    d = B.CacheDesc(8 * 100 * 128, 100 * 128, 128, 100)
    f = lib.qwattn_decode_noalloc
    assert f(ctypes.byref(p), 1, F, F, F, F, F, F, F, ctypes.byref(d), F, cu(3, 99, 100), 3, F, None) == B.ERR_CAPACITY
    assert f(ctypes.byref(B.make_params(64, 2)), 1, F, F, F, F, F, F, F, ctypes.byref(d), F, cu(3), 1, F,
             None) == B.ERR_UNSUPPORTED
    assert f(ctypes.byref(p), 1, None, None, None, None, None, None, None, None, None, None, 0, None, None) == B.OK
    limit = 67108864
    # the largest total whose scratch fits, and one more chunk's worth
    p16 = B.make_params(16, 1)
    # (only over-limit sizes are called: a call that passed every check would
    # launch kernels, and these pointers are fake)
    for n_seq, total, ok in ((1, 16_000_000, True), (1, 16_500_000, False), (2, 8_300_000 * 2, False)):
        need = B.decode_workspace_size(p16, B.BF16, n_seq, total)
        assert (need <= limit) == ok, (n_seq, total, need)
        if ok:
            continue
        each = total // n_seq
        sp = (ctypes.c_int32 * n_seq)(*([each] * n_seq))
        big = B.CacheDesc((each + 1) * 128, (each + 1) * 128, 128, each + 1)
        r = f(ctypes.byref(p16), 1, F, F, F, F, F, F, F, ctypes.byref(big), F, sp, n_seq, F, None)
        assert r == B.ERR_WORKSPACE
        assert b"fixed scratch" in lib.qwattn_last_error()
