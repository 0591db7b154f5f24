"""ctypes binding of libqwattn (argument marshalling only: every step of the
path runs in the library's HIP kernels).  The names follow the C entry points
declared in include/qwattn.h.

Tensors are torch tensors on the current HIP device; the call is enqueued on
``torch.cuda.current_stream()``.  The library is loaded on first use and a
missing build raises, so nothing falls back to another implementation."""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libqwattn.so")
_lib = None

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_WORKSPACE, ERR_HIP = range(6)
F32, BF16 = 0, 1
HEAD_DIM = 128
HEAD_DIM_GATED = 256


class Params(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("eps", ctypes.c_float), ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("order", ctypes.c_int32), ("rotary_dim", ctypes.c_int32), ("norm_offset", ctypes.c_float),
                ("output_gate", ctypes.c_int32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("stride_seq", ctypes.c_int64), ("stride_head", ctypes.c_int64), ("stride_tok", ctypes.c_int64),
                ("capacity", ctypes.c_int32)]


class QwattnError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"libqwattn status {status}: {detail}")


def lib_path():
    return _LIB_PATH


def load(path=None):
    """Load libqwattn.so (raises if it is not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libqwattn is not built ({p} missing): run __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pp, pc = ctypes.POINTER(Params), ctypes.POINTER(CacheDesc)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.qwattn_qk_norm_rope.argtypes = [pp, i32, vp, vp, vp, vp, vp, i64, vp, vp, vp]
    lib.qwattn_qk_norm_rope.restype = i32
    lib.qwattn_prefill.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp, ip, i32, vp, vp, vp, pc, vp, sz, vp]
    lib.qwattn_prefill.restype = i32
    lib.qwattn_decode.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp, vp, pc, vp, ip, i32, vp, vp, sz, vp]
    lib.qwattn_decode.restype = i32
    lib.qwattn_decode_noalloc.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp, vp, pc, vp, ip, i32, vp, vp]
    lib.qwattn_decode_noalloc.restype = i32
    lib.qwattn_append.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp, vp, pc, vp, ip, vp, ip, i32, vp, vp, sz, vp]
    lib.qwattn_append.restype = i32
    lib.qwattn_append_workspace_size.argtypes = [pp, i32, i32, i64, i32]
    lib.qwattn_append_workspace_size.restype = sz
    lib.qwattn_prefill_workspace_size.argtypes = [pp, i32, i32, i64, i32, i32]
    lib.qwattn_prefill_workspace_size.restype = sz
    lib.qwattn_decode_workspace_size.argtypes = [pp, i32, i32, i64]
    lib.qwattn_decode_workspace_size.restype = sz
    lib.qwattn_linear.argtypes = [i32, vp, vp, i64, i32, i32, vp, vp]
    lib.qwattn_linear.restype = i32
    lib.qwattn_attention_layer.argtypes = [pp, i32, i32, vp, vp, vp, vp, vp, vp, ip, i32, vp, ip, vp, vp, vp, pc,
                                           vp, sz, vp]
    lib.qwattn_attention_layer.restype = i32
    lib.qwattn_attention_layer_workspace_size.argtypes = [pp, i32, i32, i32, i64, i32, i32]
    lib.qwattn_attention_layer_workspace_size.restype = sz
    lib.qwattn_mfma_probe.argtypes = [i32, vp, vp]
    lib.qwattn_mfma_probe.restype = i32
    lib.qwattn_mfma_probe_flops.argtypes = [i32]
    lib.qwattn_mfma_probe_flops.restype = ctypes.c_double
    lib.qwattn_hbm_read_probe.argtypes = [vp, i64, vp, vp]
    lib.qwattn_hbm_read_probe.restype = i32
    lib.qwattn_status_str.argtypes = [i32]
    lib.qwattn_status_str.restype = ctypes.c_char_p
    lib.qwattn_last_error.argtypes = []
    lib.qwattn_last_error.restype = ctypes.c_char_p
    lib.qwattn_set_timing_events.argtypes = [vp, vp]
    lib.qwattn_set_timing_events.restype = i32
    lib.qwattn_abi_version.argtypes = []
    lib.qwattn_abi_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def make_params(n_q_heads, n_kv_heads, eps=1e-6, rope_theta=1e6, softmax_scale=0.0, head_dim=HEAD_DIM, order=0,
                rotary_dim=0, norm_offset=0.0, output_gate=0):
    return Params(n_q_heads, n_kv_heads, head_dim, eps, rope_theta, softmax_scale, order, rotary_dim, norm_offset,
                  output_gate)


def make_gated_params(n_q_heads, n_kv_heads, eps=1e-6, rope_theta=1e7, rotary_dim=64, softmax_scale=0.0, order=0,
                      output_gate=1):
    """A gated global-attention layer (Qwen3-Next / Qwen3.5): head_dim 256,
    zero-centred QK-Norm, partial RoPE, per-head sigmoid output gate."""
    return make_params(n_q_heads, n_kv_heads, eps=eps, rope_theta=rope_theta, softmax_scale=softmax_scale,
                       head_dim=HEAD_DIM_GATED, order=order, rotary_dim=rotary_dim, norm_offset=1.0,
                       output_gate=output_gate)


def _out_like(params, q):
    """Output tensor for a call whose queries are q (q carries the gate halves
    when params.output_gate is set)."""
    return torch.empty(q.shape[0], params.n_q_heads, params.head_dim, dtype=q.dtype, device=q.device)


def _check(status):
    if status != OK:
        raise QwattnError(status, _lib.qwattn_last_error().decode())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name):
    if t is not None and (not t.is_cuda or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def cache_desc(k_cache):
    """Descriptor of a [n_seq][n_kv_heads][capacity][head_dim] cache tensor (strides may vary)."""
    s = k_cache.stride()
    return CacheDesc(s[0], s[1], s[2], k_cache.shape[2])


def _check_cache_pair(params, k_cache, v_cache):
    if v_cache is None or k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must share one shape and stride layout")
    if k_cache.dim() != 4 or k_cache.shape[3] != params.head_dim or k_cache.stride(3) != 1:
        raise ValueError("cache must be [n_seq][n_kv_heads][capacity][head_dim] with the last dim contiguous")


def qk_norm_rope(params, q, k, q_gamma, k_gamma, positions, q_out=None, k_out=None):
    """QK-Norm then RoPE of q [n_tok, Hq, d] (gated: [n_tok, Hq, 2d]) and/or
    k [n_tok, Hkv, d] at ``positions``."""
    lib = load()
    ref = q if q is not None else k
    for t, n in ((q, "q"), (k, "k"), (q_gamma, "q_gamma"), (k_gamma, "k_gamma"), (positions, "positions")):
        _dev(t, n)
    if q is not None and q_out is None:
        q_out = _out_like(params, q)
    if k is not None and k_out is None:
        k_out = torch.empty_like(k)
    n_tok = ref.shape[0]
    _check(lib.qwattn_qk_norm_rope(ctypes.byref(params), _dtype_code(ref), _ptr(q), _ptr(k), _ptr(q_gamma),
                                   _ptr(k_gamma), _ptr(positions), n_tok, _ptr(q_out), _ptr(k_out), _stream()))
    return q_out, k_out


def set_timing_events(begin, end):
    """Raw hipEvent_t handles (ints) recorded around the next call's dominant kernel."""
    _check(load().qwattn_set_timing_events(ctypes.c_void_p(begin) if begin else None,
                                           ctypes.c_void_p(end) if end else None))


def prefill_workspace_size(params, dtype_code, n_seq, n_tok, max_seqlen, with_cache):
    return load().qwattn_prefill_workspace_size(ctypes.byref(params), dtype_code, n_seq, n_tok, max_seqlen,
                                                1 if with_cache else 0)


def decode_workspace_size(params, dtype_code, n_seq, total_start_pos):
    return load().qwattn_decode_workspace_size(ctypes.byref(params), dtype_code, n_seq, total_start_pos)


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def prefill(params, q, k, v, q_gamma, k_gamma, cu_seqlens, cu_seqlens_host=None, out=None,
            k_cache=None, v_cache=None, workspace=None):
    """Causal GQA prefill over packed sequences.  ``cu_seqlens`` is a device
    int32 tensor [n_seq + 1]; ``cu_seqlens_host`` the same values on the host
    (a list, numpy array or CPU tensor; read from the device when omitted)."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_gamma, "q_gamma"), (k_gamma, "k_gamma"),
                 (cu_seqlens, "cu_seqlens")):
        _dev(t, n)
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.cpu()
    cu_h = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    n_seq = cu_h.numel() - 1
    n_tok = int(cu_h[-1]) if n_seq > 0 else 0
    max_len = int((cu_h[1:] - cu_h[:-1]).max()) if n_seq > 0 else 0
    dt = _dtype_code(q)
    if out is None:
        out = _out_like(params, q)
    desc = None
    if k_cache is not None:
        _check_cache_pair(params, k_cache, v_cache)
        desc = cache_desc(k_cache)
    nbytes = prefill_workspace_size(params, dt, n_seq, n_tok, max_len, k_cache is not None)
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib.qwattn_prefill(ctypes.byref(params), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(q_gamma), _ptr(k_gamma),
                              ctypes.c_void_p(cu_seqlens.data_ptr()),
                              cu_h.numpy().ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n_seq, _ptr(out),
                              _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc) if desc else None,
                              ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream()))
    return out


def append_workspace_size(params, dtype_code, n_seq, n_new, max_new):
    return load().qwattn_append_workspace_size(ctypes.byref(params), dtype_code, n_seq, n_new, max_new)


def append(params, q, k, v, q_gamma, k_gamma, k_cache, v_cache, start_pos, cu_new, start_pos_host=None,
           cu_new_host=None, out=None, workspace=None):
    """Multi-token append against the cache: sequence s adds the tokens
    cu_new[s] .. cu_new[s+1]-1 at positions start_pos[s] ..; their k̂/v go to
    those cache slots and each new query attends to slots 0 .. its position."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_gamma, "q_gamma"), (k_gamma, "k_gamma"),
                 (start_pos, "start_pos"), (cu_new, "cu_new")):
        _dev(t, n)
    sp_h = torch.as_tensor(start_pos.cpu() if start_pos_host is None else start_pos_host,
                           dtype=torch.int32).contiguous()
    cu_h = torch.as_tensor(cu_new.cpu() if cu_new_host is None else cu_new_host, dtype=torch.int32).contiguous()
    n_seq = sp_h.numel()
    if cu_h.numel() != n_seq + 1:
        raise ValueError("cu_new must hold n_seq + 1 offsets")
    n_new = int(cu_h[-1]) if n_seq > 0 else 0
    max_new = int((cu_h[1:] - cu_h[:-1]).max()) if n_seq > 0 else 0
    dt = _dtype_code(q)
    if out is None:
        out = _out_like(params, q)
    _check_cache_pair(params, k_cache, v_cache)
    desc = cache_desc(k_cache)
    nbytes = append_workspace_size(params, dt, n_seq, n_new, max_new)
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib.qwattn_append(ctypes.byref(params), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(q_gamma), _ptr(k_gamma),
                             _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
                             ctypes.c_void_p(start_pos.data_ptr()),
                             sp_h.numpy().ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                             ctypes.c_void_p(cu_new.data_ptr()),
                             cu_h.numpy().ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n_seq, _ptr(out),
                             ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream()))
    return out


def decode(params, q, k, v, q_gamma, k_gamma, k_cache, v_cache, start_pos, start_pos_host=None, out=None,
           workspace=None):
    """One new token per sequence against the cache; appends k̂/v at start_pos."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_gamma, "q_gamma"), (k_gamma, "k_gamma"),
                 (start_pos, "start_pos")):
        _dev(t, n)
    if start_pos_host is None:
        start_pos_host = start_pos.cpu()
    sp_h = torch.as_tensor(start_pos_host, dtype=torch.int32).contiguous()
    n_seq = sp_h.numel()
    dt = _dtype_code(q)
    if out is None:
        out = _out_like(params, q)
    _check_cache_pair(params, k_cache, v_cache)
    desc = cache_desc(k_cache)
    nbytes = decode_workspace_size(params, dt, n_seq, int(sp_h.sum()))
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib.qwattn_decode(ctypes.byref(params), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(q_gamma), _ptr(k_gamma),
                             _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
                             ctypes.c_void_p(start_pos.data_ptr()),
                             sp_h.numpy().ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n_seq, _ptr(out),
                             ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream()))
    return out


def decode_noalloc(params, q, k, v, q_gamma, k_gamma, k_cache, v_cache, start_pos, start_pos_host=None, out=None):
    """qwattn_decode without a workspace: the library's fixed device scratch
    (QWATTN_DECODE_NOALLOC_SCRATCH_BYTES per device) instead."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_gamma, "q_gamma"), (k_gamma, "k_gamma"),
                 (start_pos, "start_pos")):
        _dev(t, n)
    if start_pos_host is None:
        start_pos_host = start_pos.cpu()
    sp_h = torch.as_tensor(start_pos_host, dtype=torch.int32).contiguous()
    if out is None:
        out = _out_like(params, q)
    _check_cache_pair(params, k_cache, v_cache)
    desc = cache_desc(k_cache)
    _check(lib.qwattn_decode_noalloc(ctypes.byref(params), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(q_gamma),
                                     _ptr(k_gamma), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
                                     ctypes.c_void_p(start_pos.data_ptr()),
                                     sp_h.numpy().ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), sp_h.numel(),
                                     _ptr(out), _stream()))
    return out


def linear(x, w, y=None):
    """y = x W^T (bf16): x [m, k], w [n, k] (the weight as stored), y [m, n]."""
    lib = load()
    _dev(x, "x")
    _dev(w, "w")
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("x and w disagree on the input width")
    if y is None:
        y = torch.empty(m, n, dtype=x.dtype, device=x.device)
    _check(lib.qwattn_linear(_dtype_code(x), _ptr(x), _ptr(w), m, n, k, _ptr(y), _stream()))
    return y


def mfma_probe(iters, sink):
    """Measurement aid: the register-only MFMA loop (see qwattn.h); sink is a
    float32 device tensor of at least one element."""
    lib = load()
    _dev(sink, "sink")
    _check(lib.qwattn_mfma_probe(iters, _ptr(sink), _stream()))


def mfma_probe_flops(iters):
    return load().qwattn_mfma_probe_flops(iters)


def hbm_read_probe(src, sink, nbytes=None):
    """Measurement aid: reads nbytes (default: all of src, rounded down to 16)
    of the device tensor src once with nontemporal loads."""
    lib = load()
    _dev(src, "src")
    _dev(sink, "sink")
    total = src.numel() * src.element_size()
    nbytes = (total if nbytes is None else nbytes) // 16 * 16
    if nbytes > total:
        raise ValueError("nbytes exceeds src")
    _check(lib.qwattn_hbm_read_probe(_ptr(src), nbytes, _ptr(sink), _stream()))
    return nbytes


def attention_layer_workspace_size(params, dtype_code, hidden, n_seq, n_tok, max_seqlen, with_cache):
    return load().qwattn_attention_layer_workspace_size(ctypes.byref(params), dtype_code, hidden, n_seq, n_tok,
                                                        max_seqlen, 1 if with_cache else 0)


def attention_layer(params, x, w_qkv, w_o, q_gamma, k_gamma, cu_seqlens, cu_seqlens_host=None, start_pos=None,
                    start_pos_host=None, y=None, k_cache=None, v_cache=None, workspace=None):
    """The attention sublayer (q/k/v projections, QK-Norm, RoPE, causal GQA,
    o_proj) over packed sequences x [n_tok, hidden]; with ``start_pos`` an
    append against the cache.  w_qkv stacks the q, k and v projection weights
    ([out][in] each); w_o is the o_proj weight."""
    lib = load()
    for t, nm in ((x, "x"), (w_qkv, "w_qkv"), (w_o, "w_o"), (q_gamma, "q_gamma"), (k_gamma, "k_gamma"),
                  (cu_seqlens, "cu_seqlens"), (start_pos, "start_pos")):
        _dev(t, nm)
    cu_h = torch.as_tensor(cu_seqlens.cpu() if cu_seqlens_host is None else cu_seqlens_host,
                           dtype=torch.int32).contiguous()
    n_seq = cu_h.numel() - 1
    n_tok = int(cu_h[-1]) if n_seq > 0 else 0
    max_len = int((cu_h[1:] - cu_h[:-1]).max()) if n_seq > 0 else 0
    sp_h = None
    if start_pos is not None:
        sp_h = torch.as_tensor(start_pos.cpu() if start_pos_host is None else start_pos_host,
                               dtype=torch.int32).contiguous()
    hidden = x.shape[1]
    dt = _dtype_code(x)
    if y is None:
        y = torch.empty(n_tok, hidden, dtype=x.dtype, device=x.device)
    desc = None
    if k_cache is not None:
        _check_cache_pair(params, k_cache, v_cache)
        desc = cache_desc(k_cache)
    nbytes = attention_layer_workspace_size(params, dt, hidden, n_seq, n_tok, max_len, k_cache is not None)
    ws = _workspace(nbytes, x.device, workspace)
    _check(lib.qwattn_attention_layer(
        ctypes.byref(params), dt, hidden, _ptr(x), _ptr(w_qkv), _ptr(w_o), _ptr(q_gamma), _ptr(k_gamma),
        ctypes.c_void_p(cu_seqlens.data_ptr()), cu_h.numpy().ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n_seq,
        _ptr(start_pos), None if sp_h is None else sp_h.numpy().ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        _ptr(y), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc) if desc else None,
        ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream()))
    return y
