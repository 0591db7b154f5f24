// C-ABI of libqwattn: argument validation, planning, workspace layout and
// launches.  Every check runs before the first HIP call, so an invalid call
// enqueues nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/qwattn.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_ev_begin = nullptr, g_ev_end = nullptr;

// Records the timing hook around one launch and clears it.
template <class F>
hipError_t timed_launch(hipStream_t st, F&& launch) {
  hipEvent_t b = g_ev_begin, e = g_ev_end;
  g_ev_begin = g_ev_end = nullptr;
  hipError_t r;
  if (b && (r = hipEventRecord(b, st)) != hipSuccess) return r;
  if ((r = launch()) != hipSuccess) return r;
  if (e && (r = hipEventRecord(e, st)) != hipSuccess) return r;
  return hipSuccess;
}

qwattn_status fail(qwattn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

qwattn_status hip_fail(hipError_t e, const char* what) {
  return fail(QWATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Rotated coordinates: rotary_dim, 0 meaning all of head_dim.
int rot_dim(const qwattn_params* p) { return p->rotary_dim ? p->rotary_dim : p->head_dim; }

// Elements between consecutive query head rows of q: the query and, with the
// output gate, the gate that follows it.
int q_row(const qwattn_params* p) { return p->output_gate ? 2 * p->head_dim : p->head_dim; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Compute units of the current device.
hipError_t cu_count(int* n) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev);
  return e;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int elem_bytes(qwattn_dtype dt) { return dt == QWATTN_BF16 ? 2 : 4; }

// The tile copies address the rows of one K/V tile (64 rows in prefill, 32 in
// decode; 256 rows of an operand panel in the projections) from a scalar base
// with 32-bit per-lane byte offsets, row * row stride + column, so 64 row
// strides (256 for the projections) must fit in 32 bits.
constexpr int64_t kMaxTileRowBytes = (int64_t(1) << 32) / 64;  // 64 MiB per K/V row
constexpr int64_t kMaxGemmRowElems = (int64_t(1) << 32) / 256 / 2;  // bf16 operand row of a projection
// Bounds that keep every element offset and size product far inside int64.
constexpr int32_t kMaxHeads = 32768;
constexpr int64_t kMaxCacheElems = int64_t(1) << 56;

qwattn_status check_params(const qwattn_params* p, qwattn_dtype dt) {
  if (!p) return fail(QWATTN_ERR_INVALID_ARG, "params is NULL");
  if (dt != QWATTN_F32 && dt != QWATTN_BF16) return fail(QWATTN_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (p->n_q_heads <= 0 || p->n_kv_heads <= 0)
    return fail(QWATTN_ERR_INVALID_ARG, "head counts must be positive (n_q_heads=%d, n_kv_heads=%d)",
                p->n_q_heads, p->n_kv_heads);
  if (p->n_q_heads > kMaxHeads)
    return fail(QWATTN_ERR_UNSUPPORTED, "n_q_heads=%d > %d", p->n_q_heads, kMaxHeads);
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(QWATTN_ERR_INVALID_ARG, "n_q_heads=%d is not a multiple of n_kv_heads=%d", p->n_q_heads,
                p->n_kv_heads);
  if (p->head_dim != QWATTN_HEAD_DIM && p->head_dim != QWATTN_HEAD_DIM_GATED)
    return fail(QWATTN_ERR_UNSUPPORTED, "head_dim=%d (128 and 256 are supported)", p->head_dim);
  if (!(p->eps >= 0.f) || !std::isfinite(p->eps)) return fail(QWATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!(p->rope_theta > 1.0) || !std::isfinite(p->rope_theta))
    return fail(QWATTN_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  if (!(p->softmax_scale >= 0.f) || !std::isfinite(p->softmax_scale))
    return fail(QWATTN_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (p->order != 0 && p->order != 1) return fail(QWATTN_ERR_INVALID_ARG, "order must be 0 or 1");
  const int rot = rot_dim(p);
  if (rot <= 0 || rot > p->head_dim || rot % 2)
    return fail(QWATTN_ERR_INVALID_ARG, "rotary_dim=%d must be even and in (0, head_dim]", p->rotary_dim);
  if (!std::isfinite(p->norm_offset)) return fail(QWATTN_ERR_INVALID_ARG, "norm_offset must be finite");
  if (p->output_gate != 0 && p->output_gate != 1) return fail(QWATTN_ERR_INVALID_ARG, "output_gate must be 0 or 1");
  if (p->head_dim == QWATTN_HEAD_DIM) {
    if (rot != QWATTN_HEAD_DIM || p->norm_offset != 0.f || p->output_gate)
      return fail(QWATTN_ERR_UNSUPPORTED,
                  "head_dim 128 takes full rotation, norm_offset 0 and no output gate (the gated-layer options "
                  "run at head_dim 256)");
  } else if (rot != 32 && rot != 64 && rot != 128 && rot != 256) {
    return fail(QWATTN_ERR_UNSUPPORTED, "rotary_dim=%d at head_dim 256 (32, 64, 128 and 256 are supported)", rot);
  }
  return QWATTN_OK;
}

qwattn_status check_ptr(const void* p, const char* name, uintptr_t align = 16) {
  if (!p) return fail(QWATTN_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(QWATTN_ERR_INVALID_ARG, "%s is not %d-byte aligned", name, (int)align);
  return QWATTN_OK;
}

// A cache of n_seq sequences x n_kv heads x capacity slots.
qwattn_status check_cache(const qwattn_cache_desc* c, const void* kc, const void* vc, qwattn_dtype dt,
                          int head_dim, int n_seq, int n_kv) {
  qwattn_status st;
  if ((st = check_ptr(kc, "k_cache")) || (st = check_ptr(vc, "v_cache"))) return st;
  if (!c) return fail(QWATTN_ERR_INVALID_ARG, "cache descriptor is NULL");
  if (c->capacity <= 0) return fail(QWATTN_ERR_INVALID_ARG, "cache capacity must be positive");
  if (c->stride_seq <= 0 || c->stride_head <= 0 || c->stride_tok <= 0)
    return fail(QWATTN_ERR_INVALID_ARG, "cache strides must be positive");
  if (c->stride_seq > kMaxCacheElems || c->stride_head > kMaxCacheElems || c->stride_tok > kMaxCacheElems)
    return fail(QWATTN_ERR_INVALID_ARG, "cache stride beyond 2^56 elements");
  const int64_t es = elem_bytes(dt);
  if ((c->stride_seq * es) % 16 || (c->stride_head * es) % 16 || (c->stride_tok * es) % 16)
    return fail(QWATTN_ERR_INVALID_ARG, "cache strides must keep rows 16-byte aligned");
  if (c->stride_tok < head_dim) return fail(QWATTN_ERR_INVALID_ARG, "cache stride_tok < head_dim");
  if (c->stride_tok * es > kMaxTileRowBytes)
    return fail(QWATTN_ERR_UNSUPPORTED,
                "cache stride_tok of %lld bytes > %lld: the kernels address a tile's 64 rows with 32-bit offsets",
                (long long)(c->stride_tok * es), (long long)kMaxTileRowBytes);
  // Offset of the last element the call may touch, exactly (128-bit).
  const __int128 last = (__int128)(n_seq > 0 ? n_seq - 1 : 0) * c->stride_seq +
                        (__int128)(n_kv > 0 ? n_kv - 1 : 0) * c->stride_head +
                        (__int128)(c->capacity - 1) * c->stride_tok + head_dim;
  if (last > kMaxCacheElems) return fail(QWATTN_ERR_INVALID_ARG, "cache extent beyond 2^56 elements");
  return QWATTN_OK;
}

// theta^(-2i/rot) for i < rot/2 (the rest zero).
qw::RopeFreq rope_freq(const qwattn_params* p) {
  qw::RopeFreq r{};
  const int rot = rot_dim(p);
  for (int i = 0; i < rot / 2; ++i) r.w[i] = std::pow(p->rope_theta, -(2.0 * i) / rot);
  return r;
}

float scale_log2e(const qwattn_params* p) {
  const double sc = p->softmax_scale > 0.f ? (double)p->softmax_scale : 1.0 / std::sqrt((double)p->head_dim);
  return (float)(sc * 1.4426950408889634);
}

// Query rows per attention workgroup.
int prefill_rows(const qwattn_params* p, qwattn_dtype dt) {
  if (dt != QWATTN_BF16) return qw::kAttnF32Rows;
  return p->head_dim == QWATTN_HEAD_DIM ? qw::kPrefillRows : qw::kWideRows;
}

// The norm+RoPE fields every launch shares.
void set_norm(qw::NormRopeArgs& a, const qwattn_params* p) {
  a.eps = p->eps;
  a.order = p->order;
  a.head_dim = p->head_dim;
  a.rot = rot_dim(p);
  a.gamma_offset = p->norm_offset;
  a.rope = rope_freq(p);
  a.in_row[0] = q_row(p);
  a.in_row[1] = a.in_row[2] = p->head_dim;
}

// ------------------------------------------------------------------ prefill plan
struct PrefillPlan {
  int g = 1, bm_tok = 1, max_tiles = 0, n_items = 0;
  size_t off_khat = 0, off_qhat = 0, off_scratch = 0, off_items = 0, off_flag = 0, total = 0;
};

// Workspace layout; n_items / max_tiles are upper bounds when `exact` is false.
PrefillPlan prefill_layout(const qwattn_params* p, qwattn_dtype dt, int n_seq, int64_t n_tok, int max_tiles,
                           int64_t n_items, bool with_cache) {
  PrefillPlan pl;
  pl.g = p->n_q_heads / p->n_kv_heads;
  pl.bm_tok = std::max(1, prefill_rows(p, dt) / pl.g);
  pl.max_tiles = max_tiles;
  pl.n_items = (int)n_items;
  size_t off = 0;
  pl.off_khat = off;
  if (!with_cache) off = align256(off + (size_t)n_tok * p->n_kv_heads * p->head_dim * elem_bytes(dt));
  pl.off_qhat = off;
  if (dt == QWATTN_F32) off = align256(off + (size_t)n_tok * p->n_q_heads * p->head_dim * 4);
  pl.off_scratch = off;
  off = align256(off + (size_t)(4 * ((int64_t)max_tiles + 1) + n_seq) * 4);
  pl.off_items = off;
  off = align256(off + (size_t)n_items * sizeof(qw::PrefillItem));
  pl.off_flag = off;
  off = align256(off + 8);  // the softmax form and its weight shift
  pl.total = off;
  return pl;
}

// ------------------------------------------------------------------ decode plan
// Keys per split-K chunk: the largest that still gives about 2048 workgroups
// (a few per CU); larger chunks spread each workgroup's fixed work (query
// load, merge, partial write) over more keys.
int decode_chunk(int64_t total_keys, int n_kv_heads) {
  for (int c : {2048, 1024, 512, 256})
    if ((total_keys / c) * n_kv_heads >= 2048) return c;
  return qw::kDecodeKeysPerPass;
}

struct DecodeLayout {
  int chunk = 0;
  int64_t max_chunks = 0;
  size_t off_qhat = 0, off_chunk = 0, off_chunk_seq = 0, off_part = 0, total = 0;
};

// Chunks a call with n_seq sequences and total_keys keys may need: at least
// sum_i ceil(keys_i / chunk) <= total_keys / chunk + n_seq for its own chunk,
// and no fewer than a call with fewer keys could need, so that a workspace
// sized for some total serves every smaller total.  A smaller total can pick
// a smaller chunk: chunk c < 2048 is picked only while
// (total / 2c) * n_kv < 2048, i.e. for totals below 2c * ceil(2048 / n_kv),
// where it makes fewer than 2 * ceil(2048 / n_kv) chunks (+ n_seq).
int64_t decode_max_chunks(int64_t total_keys, int n_seq, int n_kv) {
  const int chunk = decode_chunk(total_keys, n_kv);
  int64_t most = total_keys / chunk;
  if (chunk > qw::kDecodeKeysPerPass) most = std::max<int64_t>(most, 2 * ((2048 + n_kv - 1) / n_kv));
  return most + n_seq;
}

DecodeLayout decode_layout(const qwattn_params* p, qwattn_dtype dt, int n_seq, int64_t total_start_pos) {
  DecodeLayout d;
  const int64_t total_keys = total_start_pos + n_seq;
  d.chunk = decode_chunk(total_keys, p->n_kv_heads);
  d.max_chunks = decode_max_chunks(total_keys, n_seq, p->n_kv_heads);
  size_t off = 0;
  d.off_qhat = off;
  off = align256(off + (size_t)n_seq * p->n_q_heads * p->head_dim * elem_bytes(dt));
  d.off_chunk = off;
  off = align256(off + (size_t)(n_seq + 1) * 4);
  d.off_chunk_seq = off;
  off = align256(off + (size_t)d.max_chunks * 4);
  d.off_part = off;
  if (dt == QWATTN_BF16)
    off = align256(off + (size_t)d.max_chunks * p->n_q_heads * qw::part_stride(p->head_dim) * 4);
  d.total = off;
  return d;
}

}  // namespace

extern "C" {

int qwattn_abi_version(void) { return QWATTN_ABI_VERSION; }

qwattn_status qwattn_set_timing_events(void* begin, void* end) {
  if (!begin != !end) return fail(QWATTN_ERR_INVALID_ARG, "timing events must be both set or both NULL");
  g_ev_begin = (hipEvent_t)begin;
  g_ev_end = (hipEvent_t)end;
  return QWATTN_OK;
}

const char* qwattn_last_error(void) { return g_last_error.c_str(); }

const char* qwattn_status_str(qwattn_status s) {
  switch (s) {
    case QWATTN_OK: return "ok";
    case QWATTN_ERR_INVALID_ARG: return "invalid argument";
    case QWATTN_ERR_UNSUPPORTED: return "unsupported";
    case QWATTN_ERR_CAPACITY: return "cache capacity exceeded";
    case QWATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case QWATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

qwattn_status qwattn_qk_norm_rope(const qwattn_params* params, qwattn_dtype dtype, const void* q, const void* k,
                                  const void* q_gamma, const void* k_gamma, const int32_t* positions,
                                  int64_t n_tok, void* q_out, void* k_out, void* stream) {
  g_last_error.clear();
  qwattn_status st;
  if ((st = check_params(params, dtype))) return st;
  if (n_tok < 0) return fail(QWATTN_ERR_INVALID_ARG, "n_tok < 0");
  if (!q && !k) return fail(QWATTN_ERR_INVALID_ARG, "q and k are both NULL");
  if (!q != !q_out) return fail(QWATTN_ERR_INVALID_ARG, "q and q_out must be both set or both NULL");
  if (!k != !k_out) return fail(QWATTN_ERR_INVALID_ARG, "k and k_out must be both set or both NULL");
  if (q && ((st = check_ptr(q, "q")) || (st = check_ptr(q_out, "q_out")) || (st = check_ptr(q_gamma, "q_gamma"))))
    return st;
  if (q && params->output_gate && q == q_out)
    return fail(QWATTN_ERR_INVALID_ARG, "q_out may not alias q when q carries the output gate");
  if (k && ((st = check_ptr(k, "k")) || (st = check_ptr(k_out, "k_out")) || (st = check_ptr(k_gamma, "k_gamma"))))
    return st;
  if ((st = check_ptr(positions, "positions", 4))) return st;
  if (n_tok == 0) return QWATTN_OK;

  qw::NormRopeArgs a{};
  a.x[0] = q; a.x[1] = k; a.x[2] = nullptr;
  a.out[0] = q_out; a.out[1] = k_out;
  a.gamma[0] = q_gamma; a.gamma[1] = k_gamma;
  a.heads[0] = q ? params->n_q_heads : 0;
  a.heads[1] = k ? params->n_kv_heads : 0;
  a.heads[2] = 0;
  a.pos = positions;
  a.mode = qw::kPosExplicit;
  a.n_tok = n_tok;
  set_norm(a, params);
  hipError_t e = qw::launch_normrope(dtype == QWATTN_BF16, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "norm+RoPE launch");
  return QWATTN_OK;
}

size_t qwattn_prefill_workspace_size(const qwattn_params* params, qwattn_dtype dtype, int32_t n_seq, int64_t n_tok,
                                     int32_t max_seqlen, int32_t with_cache) {
  if (check_params(params, dtype) || n_seq < 0 || n_tok < 0 || max_seqlen < 0) return 0;
  const int g = params->n_q_heads / params->n_kv_heads;
  const int bm = std::max(1, prefill_rows(params, dtype) / g);
  const int max_tiles = (int)(((int64_t)max_seqlen + bm - 1) / bm);
  const int64_t n_items = n_tok / bm + n_seq;
  return prefill_layout(params, dtype, n_seq, n_tok, max_tiles, n_items, with_cache != 0).total;
}

}  // extern "C"

namespace {

// Sizes of a prefill / append call, from the validated host lengths.
struct SeqPlan {
  int64_t n_tok = 0;
  int bm = 1, max_tiles = 0;
  int64_t n_items = 0;
  bool append = false, any_cache = false;
};

// Checks shared by prefill, append and the sublayer: group size, lengths,
// positions and cache capacity (nothing is enqueued on failure).  n_seq == 0
// and n_tok == 0 return QWATTN_OK with sp.n_tok == 0.
qwattn_status check_sequences(const qwattn_params* params, qwattn_dtype dtype, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_host, int32_t n_seq, const int32_t* start_pos,
                              const int32_t* start_pos_host, const void* k_cache, const void* v_cache,
                              const qwattn_cache_desc* cache, SeqPlan& sp) {
  qwattn_status st;
  sp.append = start_pos != nullptr || start_pos_host != nullptr;
  const int g = params->n_q_heads / params->n_kv_heads;
  const int rows = prefill_rows(params, dtype);
  if (g > rows) return fail(QWATTN_ERR_UNSUPPORTED, "group size %d > %d", g, rows);
  if (n_seq < 0) return fail(QWATTN_ERR_INVALID_ARG, "n_seq < 0");
  if (n_seq == 0) return QWATTN_OK;
  if (!cu_seqlens_host) return fail(QWATTN_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
  if (cu_seqlens_host[0] != 0) return fail(QWATTN_ERR_INVALID_ARG, "cu_seqlens[0] = %d, must be 0", cu_seqlens_host[0]);
  for (int s = 0; s < n_seq; ++s)
    if (cu_seqlens_host[s + 1] < cu_seqlens_host[s])
      return fail(QWATTN_ERR_INVALID_ARG, "cu_seqlens decreases at %d", s + 1);
  if ((st = check_ptr(cu_seqlens, "cu_seqlens", 4))) return st;
  sp.any_cache = k_cache || v_cache || cache;
  if (sp.append) {
    if (!start_pos || !start_pos_host) return fail(QWATTN_ERR_INVALID_ARG, "start_pos and start_pos_host are both needed");
    if ((st = check_ptr(start_pos, "start_pos", 4))) return st;
    if (!sp.any_cache) return fail(QWATTN_ERR_INVALID_ARG, "an append needs the KV cache");
  }
  if (sp.any_cache) {
    if ((st = check_cache(cache, k_cache, v_cache, dtype, params->head_dim, n_seq, params->n_kv_heads))) return st;
    for (int s = 0; s < n_seq; ++s) {
      const int64_t p0 = sp.append ? start_pos_host[s] : 0;
      const int64_t L = cu_seqlens_host[s + 1] - cu_seqlens_host[s];
      if (p0 < 0) return fail(QWATTN_ERR_INVALID_ARG, "start_pos[%d] = %lld < 0", s, (long long)p0);
      if (p0 + L > cache->capacity)
        return fail(QWATTN_ERR_CAPACITY, "sequence %d: %lld + %lld tokens exceed cache capacity %d", s,
                    (long long)p0, (long long)L, cache->capacity);
    }
  }
  sp.n_tok = cu_seqlens_host[n_seq];
  sp.bm = std::max(1, rows / g);
  for (int s = 0; s < n_seq; ++s) {
    const int nt = (int)(((int64_t)cu_seqlens_host[s + 1] - cu_seqlens_host[s] + sp.bm - 1) / sp.bm);
    sp.max_tiles = std::max(sp.max_tiles, nt);
    sp.n_items += nt;
  }
  if (sp.n_items * params->n_kv_heads > 0x7fffffffLL) return fail(QWATTN_ERR_UNSUPPORTED, "too many tiles");
  return QWATTN_OK;
}

qwattn_status check_workspace(const void* workspace, size_t workspace_bytes, size_t need) {
  if (need > 0 && (!workspace || !aligned(workspace, 256)))
    return fail(QWATTN_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < need)
    return fail(QWATTN_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  return QWATTN_OK;
}

// Where the attention reads its rotated keys and values: a cache (rows by
// sequence) or packed buffers [n_tok][Hkv][d] (rows by token).
struct KvSource {
  const void* khat;
  int64_t ks_seq, ks_head, ks_tok;
  int k_packed;
  const void* v;
  int64_t vs_seq, vs_head, vs_tok;
  int v_packed;
};

KvSource cache_source(const qwattn_cache_desc* c, const void* k_cache, const void* v_cache) {
  return {k_cache, c->stride_seq, c->stride_head, c->stride_tok, 0,
          v_cache, c->stride_seq, c->stride_head, c->stride_tok, 0};
}

KvSource packed_source(const void* khat, const void* v, const qwattn_params* p) {
  const int64_t D = p->head_dim;
  return {khat, 0, D, p->n_kv_heads * D, 1, v, 0, D, p->n_kv_heads * D, 1};
}

// The tile plan and the attention kernel: q raw (bf16 path, normed and rotated
// in the prologue) or q̂ (fp32 path, in the workspace), keys and values from kv.
qwattn_status launch_attention(const qwattn_params* params, qwattn_dtype dtype, const void* q, const void* q_gamma,
                               const void* k_gamma, const KvSource& kv, const int32_t* cu_seqlens,
                               const int32_t* start_pos, int32_t n_seq, const SeqPlan& sp, const PrefillPlan& pl,
                               char* ws, void* out, hipStream_t strm, bool timed) {
  const int64_t D = params->head_dim;
  qw::PlanArgs pa{};
  pa.cu = cu_seqlens;
  pa.n_seq = n_seq;
  pa.bm_tok = sp.bm;
  pa.max_tiles = sp.max_tiles;
  pa.n_items = (int)sp.n_items;
  pa.scratch = (int32_t*)(ws + pl.off_scratch);
  pa.start_pos = start_pos;  // NULL for a prefill
  pa.items = (qw::PrefillItem*)(ws + pl.off_items);
  if (dtype == QWATTN_BF16) {
    pa.q_gamma = q_gamma;
    pa.k_gamma = k_gamma;
    pa.scale_log2e = scale_log2e(params);
    pa.gamma_offset = params->norm_offset;
    pa.head_dim = params->head_dim;
    pa.static_flag = (int32_t*)(ws + pl.off_flag);
  }
  hipError_t e;
  if ((e = qw::launch_prefill_plan(pa, strm)) != hipSuccess) return hip_fail(e, "plan launch");

  qw::PrefillArgs a{};
  a.q = q;
  a.q_row = q_row(params);
  a.gate = params->output_gate ? (const char*)q + D * elem_bytes(dtype) : nullptr;
  a.q_gamma = q_gamma;
  a.k_gamma = k_gamma;
  a.qhat = ws + pl.off_qhat;
  a.khat = kv.khat;
  a.ks_seq = kv.ks_seq; a.ks_head = kv.ks_head; a.ks_tok = kv.ks_tok;
  a.k_packed = kv.k_packed;
  a.v = kv.v;
  a.vs_seq = kv.vs_seq; a.vs_head = kv.vs_head; a.vs_tok = kv.vs_tok;
  a.v_packed = kv.v_packed;
  a.cu = cu_seqlens;
  a.start_pos = start_pos;  // NULL for a prefill
  a.items = pa.items;
  a.static_flag = pa.static_flag;
  a.out = out;
  a.n_seq = n_seq;
  a.Hq = params->n_q_heads;
  a.Hkv = params->n_kv_heads;
  a.g = params->n_q_heads / params->n_kv_heads;
  a.bm_tok = sp.bm;
  a.decode = 0;
  a.scale_log2e = scale_log2e(params);
  a.eps = params->eps;
  a.order = params->order;
  a.head_dim = params->head_dim;
  a.rot = rot_dim(params);
  a.gamma_offset = params->norm_offset;
  a.rope = rope_freq(params);
  auto launch = [&] {
    if (dtype != QWATTN_BF16) return qw::launch_attn_f32(a, (int)sp.n_items, strm);
    return D == QWATTN_HEAD_DIM ? qw::launch_prefill_bf16(a, (int)sp.n_items, strm)
                                : qw::launch_prefill_wide(a, (int)sp.n_items, strm);
  };
  e = timed ? timed_launch(strm, launch) : launch();
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return QWATTN_OK;
}

// Prefill, or (start_pos set) an append of new tokens at start_pos[s] .. against
// the cache: the norm+RoPE pass for K (and V into the cache), then the plan and
// the attention, with positions offset per sequence.
qwattn_status prefill_or_append(const qwattn_params* params, qwattn_dtype dtype, const void* q, const void* k,
                                const void* v, const void* q_gamma, const void* k_gamma, const int32_t* cu_seqlens,
                                const int32_t* cu_seqlens_host, int32_t n_seq, const int32_t* start_pos,
                                const int32_t* start_pos_host, void* out, void* k_cache, void* v_cache,
                                const qwattn_cache_desc* cache, void* workspace, size_t workspace_bytes,
                                void* stream) {
  qwattn_status st;
  if ((st = check_params(params, dtype))) return st;
  SeqPlan sp;
  if ((st = check_sequences(params, dtype, cu_seqlens, cu_seqlens_host, n_seq, start_pos, start_pos_host, k_cache,
                            v_cache, cache, sp)))
    return st;
  if (n_seq == 0) return QWATTN_OK;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(q_gamma, "q_gamma")) || (st = check_ptr(k_gamma, "k_gamma")) || (st = check_ptr(out, "out")))
    return st;
  if (sp.n_tok == 0) return QWATTN_OK;
  const PrefillPlan pl = prefill_layout(params, dtype, n_seq, sp.n_tok, sp.max_tiles, sp.n_items, sp.any_cache);
  if ((st = check_workspace(workspace, workspace_bytes, pl.total))) return st;

  hipStream_t strm = (hipStream_t)stream;
  char* ws = (char*)workspace;

  // 1) norm + RoPE of K (and of Q for the fp32 path); K̂ -> cache or workspace, V -> cache
  qw::NormRopeArgs nr{};
  nr.x[0] = q; nr.x[1] = k; nr.x[2] = v;
  nr.out[0] = ws + pl.off_qhat;
  nr.out[1] = sp.any_cache ? nullptr : (void*)(ws + pl.off_khat);
  nr.gamma[0] = q_gamma; nr.gamma[1] = k_gamma;
  nr.heads[0] = dtype == QWATTN_F32 ? params->n_q_heads : 0;
  nr.heads[1] = params->n_kv_heads;
  nr.heads[2] = sp.any_cache ? params->n_kv_heads : 0;
  if (sp.any_cache) {
    nr.k_cache = k_cache; nr.v_cache = v_cache;
    nr.cs_seq = cache->stride_seq; nr.cs_head = cache->stride_head; nr.cs_tok = cache->stride_tok;
  }
  nr.cu = cu_seqlens;
  nr.pos = start_pos;  // NULL for a prefill
  nr.n_seq = n_seq;
  nr.mode = qw::kPosPacked;
  nr.n_tok = sp.n_tok;
  set_norm(nr, params);
  hipError_t e = qw::launch_normrope(dtype == QWATTN_BF16, nr, strm);
  if (e != hipSuccess) return hip_fail(e, "norm+RoPE launch");

  // 2) plan + attention.  K̂ from the cache or the workspace; V from the cache
  // for an append (the earlier tokens' values live only there), else the input.
  KvSource kv = sp.any_cache ? cache_source(cache, k_cache, v_cache) : packed_source(ws + pl.off_khat, v, params);
  if (!sp.append) {
    const KvSource pv = packed_source(nullptr, v, params);
    kv.v = v; kv.vs_seq = pv.vs_seq; kv.vs_head = pv.vs_head; kv.vs_tok = pv.vs_tok; kv.v_packed = 1;
  }
  return launch_attention(params, dtype, q, q_gamma, k_gamma, kv, cu_seqlens, start_pos, n_seq, sp, pl, ws, out,
                          strm, true);
}

// Workspace of the sublayer: the prefill plan (and K̂ without a cache), then
// raw q ([n_tok][Hq][q_row]: with the output gate each head's query, then its
// gate), the attention output ([n_tok][Hq][head_dim]), and V without a cache;
// all bf16.
struct LayerPlan {
  PrefillPlan pl;
  size_t off_q = 0, off_o = 0, off_v = 0, total = 0;
};

LayerPlan layer_layout(const qwattn_params* p, int n_seq, int64_t n_tok, int max_tiles, int64_t n_items,
                       bool with_cache) {
  LayerPlan lp;
  lp.pl = prefill_layout(p, QWATTN_BF16, n_seq, n_tok, max_tiles, n_items, with_cache);
  size_t off = lp.pl.total;
  lp.off_q = off;
  off = align256(off + (size_t)n_tok * p->n_q_heads * q_row(p) * 2);
  lp.off_o = off;
  off = align256(off + (size_t)n_tok * p->n_q_heads * p->head_dim * 2);
  lp.off_v = off;
  if (!with_cache) off = align256(off + (size_t)n_tok * p->n_kv_heads * p->head_dim * 2);
  lp.total = off;
  return lp;
}

// A GEMM's operand rows must keep 256 rows' offsets within 32 bits (see
// kMaxGemmRowElems), and its tile grid within one launch.
qwattn_status check_gemm_shape(int64_t m, int64_t n, int64_t k) {
  if (k > kMaxGemmRowElems)
    return fail(QWATTN_ERR_UNSUPPORTED, "inner dimension %lld > %lld: operand panels use 32-bit row offsets",
                (long long)k, (long long)kMaxGemmRowElems);
  if (m > 0x7fffffffLL || ((m + 255) / 256) * ((n + 255) / 256) > 0x7fffffffLL)
    return fail(QWATTN_ERR_UNSUPPORTED, "GEMM of %lld x %lld has too many tiles", (long long)m, (long long)n);
  return QWATTN_OK;
}

qwattn_status check_layer_params(const qwattn_params* params, qwattn_dtype dtype, int32_t hidden) {
  qwattn_status st;
  if ((st = check_params(params, dtype))) return st;
  if (dtype != QWATTN_BF16) return fail(QWATTN_ERR_UNSUPPORTED, "the sublayer runs in bf16");
  if (params->head_dim == QWATTN_HEAD_DIM_GATED && rot_dim(params) > 128)
    return fail(QWATTN_ERR_UNSUPPORTED, "the head_dim-256 sublayer rotates at most 128 leading dims (rotary_dim=%d)",
                rot_dim(params));
  if (hidden <= 0 || hidden % 128)
    return fail(hidden <= 0 ? QWATTN_ERR_INVALID_ARG : QWATTN_ERR_UNSUPPORTED,
                "hidden=%d must be a positive multiple of 128", hidden);
  // the q/k/v projection reads rows of hidden values, o_proj rows of Hq * head_dim
  return check_gemm_shape(0, 0, std::max<int64_t>(hidden, (int64_t)params->n_q_heads * params->head_dim));
}

// y = x W^T launch (plain epilogue).
hipError_t launch_linear(const void* x, const void* w, int64_t m, int n, int k, void* y, hipStream_t strm) {
  qw::GemmArgs g{};
  g.x = (const uint16_t*)x;
  g.w = (const uint16_t*)w;
  g.M = m; g.N = n; g.K = k;
  g.ldx = k; g.ldw = k;
  g.y = (uint16_t*)y;
  g.ldy = n;
  return qw::launch_gemm(g, qw::kGemmPlain, strm);
}

// ------------------------------------------------------------------ decode
struct DecodeArgsIn {
  const qwattn_params* params;
  qwattn_dtype dtype;
  const void *q, *k, *v, *q_gamma, *k_gamma;
  void *k_cache, *v_cache;
  const qwattn_cache_desc* cache;
  const int32_t *start_pos, *start_pos_host;
  int32_t n_seq;
  void* out;
};

struct DecodeCall {
  DecodeLayout dl;
  int64_t total_chunks = 0;
};

// Every check of a decode call (nothing is enqueued); n_seq == 0 passes.
qwattn_status decode_check(const DecodeArgsIn& in, DecodeCall& dc) {
  const qwattn_params* params = in.params;
  qwattn_status st;
  if ((st = check_params(params, in.dtype))) return st;
  const int g = params->n_q_heads / params->n_kv_heads;
  if (in.dtype == QWATTN_BF16 && g > 16) return fail(QWATTN_ERR_UNSUPPORTED, "decode group size %d > 16", g);
  if (in.dtype == QWATTN_F32 && g > qw::kAttnF32Rows)
    return fail(QWATTN_ERR_UNSUPPORTED, "group size %d > %d for fp32", g, qw::kAttnF32Rows);
  if (in.n_seq < 0) return fail(QWATTN_ERR_INVALID_ARG, "n_seq < 0");
  if (in.n_seq == 0) return QWATTN_OK;
  if ((st = check_ptr(in.q, "q")) || (st = check_ptr(in.k, "k")) || (st = check_ptr(in.v, "v")) ||
      (st = check_ptr(in.q_gamma, "q_gamma")) || (st = check_ptr(in.k_gamma, "k_gamma")) ||
      (st = check_ptr(in.out, "out")) || (st = check_ptr(in.start_pos, "start_pos", 4)))
    return st;
  if (!in.start_pos_host) return fail(QWATTN_ERR_INVALID_ARG, "start_pos_host is NULL");
  if ((st = check_cache(in.cache, in.k_cache, in.v_cache, in.dtype, params->head_dim, in.n_seq, params->n_kv_heads)))
    return st;
  int64_t total = 0;
  for (int i = 0; i < in.n_seq; ++i) {
    const int sp = in.start_pos_host[i];
    if (sp < 0) return fail(QWATTN_ERR_INVALID_ARG, "start_pos[%d] = %d < 0", i, sp);
    if ((int64_t)sp + 1 > in.cache->capacity)
      return fail(QWATTN_ERR_CAPACITY, "sequence %d: start_pos %d + 1 exceeds cache capacity %d", i, sp,
                  in.cache->capacity);
    total += sp;
  }
  dc.dl = decode_layout(params, in.dtype, in.n_seq, total);
  dc.total_chunks = 0;
  for (int i = 0; i < in.n_seq; ++i) dc.total_chunks += ((int64_t)in.start_pos_host[i] + dc.dl.chunk) / dc.dl.chunk;
  if (dc.total_chunks * params->n_kv_heads > 0x7fffffffLL) return fail(QWATTN_ERR_UNSUPPORTED, "too many chunks");
  return QWATTN_OK;
}

// The launches of a checked decode call, with its scratch at ws (dc.dl.total bytes).
qwattn_status decode_launch(const DecodeArgsIn& in, const DecodeCall& dc, char* ws, hipStream_t strm) {
  const qwattn_params* params = in.params;
  const DecodeLayout& dl = dc.dl;
  const int g = params->n_q_heads / params->n_kv_heads;
  const int64_t D = params->head_dim;
  const qwattn_cache_desc* cache = in.cache;
  const void* gate = params->output_gate ? (const char*)in.q + D * elem_bytes(in.dtype) : nullptr;

  // 1) prologue: q̂ -> scratch; k̂ (rotated at start_pos) and v -> cache slot start_pos
  qw::NormRopeArgs nr{};
  nr.x[0] = in.q; nr.x[1] = in.k; nr.x[2] = in.v;
  nr.out[0] = ws + dl.off_qhat;
  nr.out[1] = nullptr;
  nr.gamma[0] = in.q_gamma; nr.gamma[1] = in.k_gamma;
  nr.heads[0] = params->n_q_heads;
  nr.heads[1] = params->n_kv_heads;
  nr.heads[2] = params->n_kv_heads;
  nr.k_cache = in.k_cache; nr.v_cache = in.v_cache;
  nr.cs_seq = cache->stride_seq; nr.cs_head = cache->stride_head; nr.cs_tok = cache->stride_tok;
  nr.pos = in.start_pos;
  nr.n_seq = in.n_seq;
  nr.mode = qw::kPosDecode;
  nr.n_tok = in.n_seq;
  set_norm(nr, params);
  hipError_t e = qw::launch_normrope(in.dtype == QWATTN_BF16, nr, strm);
  if (e != hipSuccess) return hip_fail(e, "decode prologue launch");

  if (in.dtype == QWATTN_BF16) {
    qw::DecodeArgs a{};
    a.qhat = (const uint16_t*)(ws + dl.off_qhat);
    a.gate = (const uint16_t*)gate;
    a.q_row = q_row(params);
    a.head_dim = params->head_dim;
    a.k_cache = (const uint16_t*)in.k_cache;
    a.v_cache = (const uint16_t*)in.v_cache;
    a.cs_seq = cache->stride_seq; a.cs_head = cache->stride_head; a.cs_tok = cache->stride_tok;
    a.start_pos = in.start_pos;
    a.chunk_off = (const int32_t*)(ws + dl.off_chunk);
    a.chunk_seq = (const int32_t*)(ws + dl.off_chunk_seq);
    a.partial = (float*)(ws + dl.off_part);
    a.out = (uint16_t*)in.out;
    a.n_seq = in.n_seq;
    a.Hq = params->n_q_heads;
    a.Hkv = params->n_kv_heads;
    a.g = g;
    a.chunk = dl.chunk;
    a.scale_log2e = scale_log2e(params);
    if ((e = qw::launch_decode_plan(in.start_pos, in.n_seq, dl.chunk, (int)dl.max_chunks,
                                    (int32_t*)(ws + dl.off_chunk), (int32_t*)(ws + dl.off_chunk_seq), strm)) !=
        hipSuccess)
      return hip_fail(e, "decode plan launch");
    if ((e = timed_launch(strm, [&] { return qw::launch_decode_split(a, (int)dc.total_chunks, strm); })) !=
        hipSuccess)
      return hip_fail(e, "decode split launch");
    if ((e = qw::launch_decode_combine(a, strm)) != hipSuccess) return hip_fail(e, "decode combine launch");
  } else {
    qw::PrefillArgs a{};
    a.qhat = ws + dl.off_qhat;
    a.gate = gate;
    a.q_row = q_row(params);
    a.head_dim = params->head_dim;
    a.khat = in.k_cache;
    a.ks_seq = cache->stride_seq; a.ks_head = cache->stride_head; a.ks_tok = cache->stride_tok;
    a.k_packed = 0;
    a.v = in.v_cache;
    a.vs_seq = cache->stride_seq; a.vs_head = cache->stride_head; a.vs_tok = cache->stride_tok;
    a.v_packed = 0;
    a.start_pos = in.start_pos;
    a.out = in.out;
    a.n_seq = in.n_seq;
    a.Hq = params->n_q_heads;
    a.Hkv = params->n_kv_heads;
    a.g = g;
    a.bm_tok = 1;
    a.decode = 1;
    a.scale_log2e = scale_log2e(params);
    a.eps = params->eps;
    if ((e = timed_launch(strm, [&] { return qw::launch_attn_f32(a, in.n_seq, strm); })) != hipSuccess)
      return hip_fail(e, "decode attention launch");
  }
  return QWATTN_OK;
}

}  // namespace

extern "C" {

qwattn_status qwattn_prefill(const qwattn_params* params, qwattn_dtype dtype, const void* q, const void* k,
                             const void* v, const void* q_gamma, const void* k_gamma, const int32_t* cu_seqlens,
                             const int32_t* cu_seqlens_host, int32_t n_seq, void* out, void* k_cache,
                             void* v_cache, const qwattn_cache_desc* cache, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return prefill_or_append(params, dtype, q, k, v, q_gamma, k_gamma, cu_seqlens, cu_seqlens_host, n_seq, nullptr,
                           nullptr, out, k_cache, v_cache, cache, workspace, workspace_bytes, stream);
}

size_t qwattn_append_workspace_size(const qwattn_params* params, qwattn_dtype dtype, int32_t n_seq, int64_t n_new,
                                    int32_t max_new) {
  return qwattn_prefill_workspace_size(params, dtype, n_seq, n_new, max_new, 1);
}

qwattn_status qwattn_append(const qwattn_params* params, qwattn_dtype dtype, const void* q, const void* k,
                            const void* v, const void* q_gamma, const void* k_gamma, void* k_cache, void* v_cache,
                            const qwattn_cache_desc* cache, const int32_t* start_pos, const int32_t* start_pos_host,
                            const int32_t* cu_new, const int32_t* cu_new_host, int32_t n_seq, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (n_seq > 0 && (!start_pos || !start_pos_host))
    return fail(QWATTN_ERR_INVALID_ARG, "start_pos and start_pos_host must be set");
  if (n_seq > 0 && (!k_cache || !v_cache || !cache)) return fail(QWATTN_ERR_INVALID_ARG, "an append needs the KV cache");
  return prefill_or_append(params, dtype, q, k, v, q_gamma, k_gamma, cu_new, cu_new_host, n_seq, start_pos,
                           start_pos_host, out, k_cache, v_cache, cache, workspace, workspace_bytes, stream);
}

size_t qwattn_decode_workspace_size(const qwattn_params* params, qwattn_dtype dtype, int32_t n_seq,
                                    int64_t total_start_pos) {
  if (check_params(params, dtype) || n_seq < 0 || total_start_pos < 0) return 0;
  return decode_layout(params, dtype, n_seq, total_start_pos).total;
}

qwattn_status qwattn_decode(const qwattn_params* params, qwattn_dtype dtype, const void* q, const void* k,
                            const void* v, const void* q_gamma, const void* k_gamma, void* k_cache, void* v_cache,
                            const qwattn_cache_desc* cache, const int32_t* start_pos, const int32_t* start_pos_host,
                            int32_t n_seq, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  const DecodeArgsIn in{params, dtype, q, k, v, q_gamma, k_gamma, k_cache, v_cache, cache, start_pos, start_pos_host,
                        n_seq, out};
  DecodeCall dc;
  qwattn_status st;
  if ((st = decode_check(in, dc))) return st;
  if (n_seq == 0) return QWATTN_OK;
  if (!workspace || !aligned(workspace, 256))
    return fail(QWATTN_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < dc.dl.total)
    return fail(QWATTN_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, dc.dl.total);
  return decode_launch(in, dc, (char*)workspace, (hipStream_t)stream);
}

qwattn_status qwattn_decode_noalloc(const qwattn_params* params, qwattn_dtype dtype, const void* q, const void* k,
                                    const void* v, const void* q_gamma, const void* k_gamma, void* k_cache,
                                    void* v_cache, const qwattn_cache_desc* cache, const int32_t* start_pos,
                                    const int32_t* start_pos_host, int32_t n_seq, void* out, void* stream) {
  static_assert(qw::kNoAllocScratchBytes == QWATTN_DECODE_NOALLOC_SCRATCH_BYTES, "scratch size");
  g_last_error.clear();
  const DecodeArgsIn in{params, dtype, q, k, v, q_gamma, k_gamma, k_cache, v_cache, cache, start_pos, start_pos_host,
                        n_seq, out};
  DecodeCall dc;
  qwattn_status st;
  if ((st = decode_check(in, dc))) return st;
  if (n_seq == 0) return QWATTN_OK;
  if (dc.dl.total > qw::kNoAllocScratchBytes)
    return fail(QWATTN_ERR_WORKSPACE,
                "qwattn_decode_noalloc: these sizes need %zu bytes of scratch; the fixed scratch holds %zu "
                "(call qwattn_decode with a workspace)",
                dc.dl.total, (size_t)qw::kNoAllocScratchBytes);
  void* scratch = nullptr;
  if (const hipError_t e = qw::decode_scratch(&scratch)) return hip_fail(e, "fixed scratch lookup");
  return decode_launch(in, dc, (char*)scratch, (hipStream_t)stream);
}

qwattn_status qwattn_mfma_probe(int32_t iters, float* sink, void* stream) {
  g_last_error.clear();
  qwattn_status st;
  if (iters <= 0) return fail(QWATTN_ERR_INVALID_ARG, "iters must be positive");
  if ((st = check_ptr(sink, "sink", 4))) return st;
  int n_cu = 0;
  if (const hipError_t e = cu_count(&n_cu)) return hip_fail(e, "device query");
  hipStream_t strm = (hipStream_t)stream;
  const hipError_t e =
      timed_launch(strm, [&] { return qw::launch_mfma_probe(n_cu, (int)(((int64_t)iters + 3) / 4), sink, strm); });
  if (e != hipSuccess) return hip_fail(e, "MFMA probe launch");
  return QWATTN_OK;
}

double qwattn_mfma_probe_flops(int32_t iters) {
  int n_cu = 0;
  if (iters <= 0 || cu_count(&n_cu) != hipSuccess) return 0.0;
  // workgroups x 4 waves x rounds x 32 MFMAs x 32 x 32 x 16 x 2 flops
  return (double)n_cu * 4 * ((((int64_t)iters + 3) / 4) * 32) * 32768.0;
}

qwattn_status qwattn_hbm_read_probe(const void* src, int64_t bytes, float* sink, void* stream) {
  g_last_error.clear();
  qwattn_status st;
  if (bytes <= 0 || bytes % 16) return fail(QWATTN_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if ((st = check_ptr(src, "src")) || (st = check_ptr(sink, "sink", 4))) return st;
  int n_cu = 0;
  if (const hipError_t e = cu_count(&n_cu)) return hip_fail(e, "device query");
  hipStream_t strm = (hipStream_t)stream;
  const hipError_t e = timed_launch(strm, [&] { return qw::launch_read_probe(32 * n_cu, src, bytes / 16, sink, strm); });
  if (e != hipSuccess) return hip_fail(e, "HBM read probe launch");
  return QWATTN_OK;
}

qwattn_status qwattn_linear(qwattn_dtype dtype, const void* x, const void* w, int64_t m, int32_t n, int32_t k,
                            void* y, void* stream) {
  g_last_error.clear();
  qwattn_status st;
  if (dtype != QWATTN_BF16) return fail(QWATTN_ERR_UNSUPPORTED, "qwattn_linear runs in bf16");
  if (m < 0 || n <= 0 || k <= 0) return fail(QWATTN_ERR_INVALID_ARG, "m >= 0, n > 0 and k > 0 are required");
  if (n % 128 || k % 64)
    return fail(QWATTN_ERR_UNSUPPORTED, "n=%d must be a multiple of 128 and k=%d of 64", n, k);
  if ((st = check_gemm_shape(m, n, k))) return st;
  if ((st = check_ptr(x, "x")) || (st = check_ptr(w, "w")) || (st = check_ptr(y, "y"))) return st;
  if (m == 0) return QWATTN_OK;
  hipStream_t strm = (hipStream_t)stream;
  const hipError_t e = timed_launch(strm, [&] { return launch_linear(x, w, m, n, k, y, strm); });
  if (e != hipSuccess) return hip_fail(e, "linear launch");
  return QWATTN_OK;
}

size_t qwattn_attention_layer_workspace_size(const qwattn_params* params, qwattn_dtype dtype, int32_t hidden,
                                             int32_t n_seq, int64_t n_tok, int32_t max_seqlen, int32_t with_cache) {
  if (check_layer_params(params, dtype, hidden) || n_seq < 0 || n_tok < 0 || max_seqlen < 0) return 0;
  const int g = params->n_q_heads / params->n_kv_heads;
  const int bm = std::max(1, prefill_rows(params, dtype) / g);
  const int max_tiles = (int)(((int64_t)max_seqlen + bm - 1) / bm);
  return layer_layout(params, n_seq, n_tok, max_tiles, n_tok / bm + n_seq, with_cache != 0).total;
}

qwattn_status qwattn_attention_layer(const qwattn_params* params, qwattn_dtype dtype, int32_t hidden, const void* x,
                                     const void* w_qkv, const void* w_o, const void* q_gamma, const void* k_gamma,
                                     const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t n_seq,
                                     const int32_t* start_pos, const int32_t* start_pos_host, void* y, void* k_cache,
                                     void* v_cache, const qwattn_cache_desc* cache, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  qwattn_status st;
  if ((st = check_layer_params(params, dtype, hidden))) return st;
  SeqPlan sp;
  if ((st = check_sequences(params, dtype, cu_seqlens, cu_seqlens_host, n_seq, start_pos, start_pos_host, k_cache,
                            v_cache, cache, sp)))
    return st;
  if (n_seq == 0) return QWATTN_OK;
  if ((st = check_ptr(x, "x")) || (st = check_ptr(w_qkv, "w_qkv")) || (st = check_ptr(w_o, "w_o")) ||
      (st = check_ptr(q_gamma, "q_gamma")) || (st = check_ptr(k_gamma, "k_gamma")) || (st = check_ptr(y, "y")))
    return st;
  if (sp.n_tok == 0) return QWATTN_OK;
  if ((st = check_gemm_shape(sp.n_tok,
                             (int64_t)params->n_q_heads * q_row(params) + 2 * params->n_kv_heads * params->head_dim,
                             hidden)))
    return st;
  const LayerPlan lp = layer_layout(params, n_seq, sp.n_tok, sp.max_tiles, sp.n_items, sp.any_cache);
  if ((st = check_workspace(workspace, workspace_bytes, lp.total))) return st;

  hipStream_t strm = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int D = params->head_dim, Hq = params->n_q_heads, Hkv = params->n_kv_heads;

  // 1) x W_qkv^T: raw q (and gate) -> workspace; K̂ (normed, rotated at each
  // token's position) and V -> the cache, or packed workspace buffers
  qw::GemmArgs g{};
  g.x = (const uint16_t*)x;
  g.w = (const uint16_t*)w_qkv;
  g.M = sp.n_tok;
  g.N = Hq * q_row(params) + 2 * Hkv * D;
  g.q_width = q_row(params);
  g.rot = rot_dim(params);
  g.gamma_offset = params->norm_offset;
  g.K = hidden;
  g.ldx = hidden; g.ldw = hidden;
  g.Hq = Hq; g.Hkv = Hkv;
  g.q_out = (uint16_t*)(ws + lp.off_q);
  if (sp.any_cache) {
    g.k_cache = (uint16_t*)k_cache; g.v_cache = (uint16_t*)v_cache;
    g.cs_seq = cache->stride_seq; g.cs_head = cache->stride_head; g.cs_tok = cache->stride_tok;
  } else {
    g.k_out = (uint16_t*)(ws + lp.pl.off_khat);
    g.v_out = (uint16_t*)(ws + lp.off_v);
  }
  g.cu = cu_seqlens;
  g.n_seq = n_seq;
  g.start_pos = start_pos;  // NULL for a prefill
  g.k_gamma = (const uint16_t*)k_gamma;
  g.eps = params->eps;
  g.order = params->order;
  g.rope = rope_freq(params);
  const int epi = D == QWATTN_HEAD_DIM ? qw::kGemmQkv : qw::kGemmQkvGated;
  hipError_t e = timed_launch(strm, [&] { return qw::launch_gemm(g, epi, strm); });
  if (e != hipSuccess) return hip_fail(e, "qkv projection launch");

  // 2) plan + attention -> O [n_tok][Hq][head_dim] in the workspace
  const KvSource kv = sp.any_cache ? cache_source(cache, k_cache, v_cache)
                                   : packed_source(ws + lp.pl.off_khat, ws + lp.off_v, params);
  if ((st = launch_attention(params, dtype, ws + lp.off_q, q_gamma, k_gamma, kv, cu_seqlens, start_pos, n_seq, sp,
                             lp.pl, ws, ws + lp.off_o, strm, false)))
    return st;

  // 3) o_proj: y = O W_o^T (O's heads concatenated in order)
  if ((e = launch_linear(ws + lp.off_o, w_o, sp.n_tok, hidden, Hq * D, y, strm)) != hipSuccess)
    return hip_fail(e, "o_proj launch");
  return QWATTN_OK;
}

}  // extern "C"
