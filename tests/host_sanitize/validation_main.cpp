// Drives every entry point of libqwattn's validation layer (qwattn_api.cpp,
// built host-only with AddressSanitizer and UndefinedBehaviorSanitizer, the
// kernels replaced by stubs.cpp):
//  * invalid calls must return their status and launch nothing (the error
//    convention of "第 20 章 Qwen3 与 Qwen3.5" §20.9: a rejected append leaves
//    the cache and the position as they were);
//  * valid calls with host arrays and workspaces of exactly the declared
//    sizes must succeed, and the stubs then write every workspace byte the
//    kernels would, so any layout overrun is reported by the sanitizer.
// Prints "ok <n> checks" and exits 0, or names the failed check and exits 1.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "qwattn.h"
#include "stubs.h"

namespace {

int checks = 0, failures = 0;

void expect(bool ok, const char* what, int line) {
  ++checks;
  if (!ok) {
    ++failures;
    std::fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", line, what, qwattn_last_error());
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// Fake device pointers (never dereferenced), 256-byte aligned.
void* const D = reinterpret_cast<void*>(0x100000);
void* const D2 = reinterpret_cast<void*>(0x200000);
void* const ODD = reinterpret_cast<void*>(0x100002);

// Host buffer of exactly n bytes at a 256-byte aligned address (the workspace).
struct HostWs {
  void* raw = nullptr;
  void* p = nullptr;
  size_t n = 0;
  explicit HostWs(size_t bytes) : n(bytes) {
    if (bytes) {
      raw = std::aligned_alloc(256, (bytes + 255) & ~size_t(255));
      p = raw;
    }
  }
  ~HostWs() { std::free(raw); }
};

qwattn_params params(int hq, int hkv, int d = 128) {
  qwattn_params p{};
  p.n_q_heads = hq;
  p.n_kv_heads = hkv;
  p.head_dim = d;
  p.eps = 1e-6f;
  p.rope_theta = d == 128 ? 1e6 : 1e7;
  if (d == 256) {
    p.rotary_dim = 64;
    p.norm_offset = 1.f;
    p.output_gate = 1;
  }
  return p;
}

qwattn_cache_desc cache(int n_kv, int cap, int d) {
  return qwattn_cache_desc{(int64_t)n_kv * cap * d, (int64_t)cap * d, d, cap};
}

int launched() {
  const int n = stub::launches;
  stub::launches = 0;
  return n;
}

void prefill_cases() {
  for (qwattn_dtype dt : {QWATTN_BF16, QWATTN_F32})
    for (int d : {128, 256})
      for (int with_cache : {0, 1})
        for (auto shape : {std::vector<int>{1, 1}, {32, 8}, {64, 4}, {16, 2}}) {
          const qwattn_params p = params(shape[0], shape[1], d);
          const std::vector<int> lens = {0, 5, 700, 1, 257, 0, 3000};
          const int n_seq = (int)lens.size();
          int32_t* cu = new int32_t[n_seq + 1];
          cu[0] = 0;
          int mx = 0;
          for (int s = 0; s < n_seq; ++s) {
            cu[s + 1] = cu[s] + lens[s];
            mx = std::max(mx, lens[s]);
          }
          stub::n_tok = cu[n_seq];
          const size_t need = qwattn_prefill_workspace_size(&p, dt, n_seq, cu[n_seq], mx, with_cache);
          EXPECT(need > 0);
          HostWs ws(need);
          const qwattn_cache_desc c = cache(shape[1], 3000, d);
          qwattn_status st = qwattn_prefill(&p, dt, D, D, D, D, D, (int32_t*)D, cu, n_seq, D2, with_cache ? D : nullptr,
                                            with_cache ? D : nullptr, with_cache ? &c : nullptr, ws.p, ws.n, nullptr);
          EXPECT(st == QWATTN_OK);
          EXPECT(launched() >= 3);
          // one byte short: rejected, nothing launched
          // (the size function bounds the tile count from above, so one byte
          // less than its answer can still be enough; 256 bytes never is)
          st = qwattn_prefill(&p, dt, D, D, D, D, D, (int32_t*)D, cu, n_seq, D2, with_cache ? D : nullptr,
                              with_cache ? D : nullptr, with_cache ? &c : nullptr, ws.p, 256, nullptr);
          EXPECT(st == QWATTN_ERR_WORKSPACE);
          EXPECT(launched() == 0);
          delete[] cu;
        }
}

void append_cases() {
  const qwattn_params p = params(32, 8);
  const int n_seq = 3;
  int32_t* sp = new int32_t[n_seq]{0, 100, 4000};
  int32_t* cu = new int32_t[n_seq + 1]{0, 64, 64, 160};
  const qwattn_cache_desc c = cache(8, 4096, 128);
  stub::n_tok = 160;
  const size_t need = qwattn_append_workspace_size(&p, QWATTN_BF16, n_seq, 160, 96);
  HostWs ws(need);
  EXPECT(qwattn_append(&p, QWATTN_BF16, D, D, D, D, D, D, D, &c, (int32_t*)D, sp, (int32_t*)D, cu, n_seq, D2, ws.p,
                       ws.n, nullptr) == QWATTN_OK);
  EXPECT(launched() == 3);
  // 4000 + 96 > 4096: capacity, nothing launched
  sp[2] = 4001;
  EXPECT(qwattn_append(&p, QWATTN_BF16, D, D, D, D, D, D, D, &c, (int32_t*)D, sp, (int32_t*)D, cu, n_seq, D2, ws.p,
                       ws.n, nullptr) == QWATTN_ERR_CAPACITY);
  EXPECT(launched() == 0);
  sp[2] = -1;
  EXPECT(qwattn_append(&p, QWATTN_BF16, D, D, D, D, D, D, D, &c, (int32_t*)D, sp, (int32_t*)D, cu, n_seq, D2, ws.p,
                       ws.n, nullptr) == QWATTN_ERR_INVALID_ARG);
  EXPECT(qwattn_append(&p, QWATTN_BF16, D, D, D, D, D, nullptr, D, &c, (int32_t*)D, sp, (int32_t*)D, cu, n_seq, D2,
                       ws.p, ws.n, nullptr) == QWATTN_ERR_INVALID_ARG);
  EXPECT(launched() == 0);
  delete[] sp;
  delete[] cu;
}

void decode_cases() {
  for (qwattn_dtype dt : {QWATTN_BF16, QWATTN_F32})
    for (int d : {128, 256})
      for (auto shape : {std::vector<int>{32, 8}, {16, 2}, {16, 1}, {64, 4}}) {
        if (dt == QWATTN_F32 && d == 256) continue;
        const qwattn_params p = params(shape[0], shape[1], d);
        // a workspace sized for the largest total serves every smaller one,
        // across the totals where the chunk length changes
        const int n_seq = 5;
        int32_t* sp = new int32_t[n_seq];
        const int64_t big = 5 * 300000;
        const size_t need = qwattn_decode_workspace_size(&p, dt, n_seq, big);
        EXPECT(need > 0);
        HostWs ws(need);
        const qwattn_cache_desc c = cache(shape[1], 300001, d);
        for (int64_t each : {0LL, 1LL, 127LL, 128LL, 1000LL, 6000LL, 26000LL, 52000LL, 104000LL, 300000LL}) {
          for (int i = 0; i < n_seq; ++i) sp[i] = (int32_t)(each - i % 2 * (each > 0));
          EXPECT(qwattn_decode(&p, dt, D, D, D, D, D, D, D, &c, (int32_t*)D, sp, n_seq, D2, ws.p, ws.n, nullptr) ==
                 QWATTN_OK);
          EXPECT(launched() >= 2);
          // the same call on the fixed scratch, when its sizes fit there
          int64_t tot = 0;
          for (int i = 0; i < n_seq; ++i) tot += sp[i];
          const bool fits = qwattn_decode_workspace_size(&p, dt, n_seq, tot) <= QWATTN_DECODE_NOALLOC_SCRATCH_BYTES;
          EXPECT(qwattn_decode_noalloc(&p, dt, D, D, D, D, D, D, D, &c, (int32_t*)D, sp, n_seq, D2, nullptr) ==
                 (fits ? QWATTN_OK : QWATTN_ERR_WORKSPACE));
          EXPECT(fits ? launched() >= 2 : launched() == 0);
        }
        sp[3] = 300001;  // start_pos + 1 > capacity
        EXPECT(qwattn_decode(&p, dt, D, D, D, D, D, D, D, &c, (int32_t*)D, sp, n_seq, D2, ws.p, ws.n, nullptr) ==
               QWATTN_ERR_CAPACITY);
        EXPECT(launched() == 0);
        sp[3] = 5;
        EXPECT(qwattn_decode(&p, dt, D, D, D, D, D, D, D, &c, (int32_t*)D, sp, n_seq, D2, ws.p, 16, nullptr) ==
               QWATTN_ERR_WORKSPACE);
        EXPECT(qwattn_decode(&p, dt, D, D, D, D, D, D, D, &c, (int32_t*)D, sp, n_seq, D2, ODD, ws.n, nullptr) ==
               QWATTN_ERR_WORKSPACE);
        EXPECT(launched() == 0);
        delete[] sp;
      }
}

void noalloc_limit_cases() {
  // 16 query / 1 KV head: the scratch of about 16.3 million keys fills the array
  const qwattn_params p = params(16, 1);
  for (int32_t each : {16000000, 16500000}) {
    int32_t* sp = new int32_t[1]{each};
    const qwattn_cache_desc c = cache(1, each + 1, 128);
    const qwattn_status st =
        qwattn_decode_noalloc(&p, QWATTN_BF16, D, D, D, D, D, D, D, &c, (int32_t*)D, sp, 1, D2, nullptr);
    EXPECT(st == (each == 16000000 ? QWATTN_OK : QWATTN_ERR_WORKSPACE));
    EXPECT(launched() == (each == 16000000 ? 4 : 0));
    delete[] sp;
  }
}

void layer_and_linear_cases() {
  const qwattn_params p = params(32, 8);
  for (int with_cache : {0, 1}) {
    const int n_seq = 2;
    int32_t* cu = new int32_t[n_seq + 1]{0, 300, 301};
    stub::n_tok = 301;
    const size_t need = qwattn_attention_layer_workspace_size(&p, QWATTN_BF16, 4096, n_seq, 301, 300, with_cache);
    HostWs ws(need);
    const qwattn_cache_desc c = cache(8, 512, 128);
    EXPECT(qwattn_attention_layer(&p, QWATTN_BF16, 4096, D, D, D, D, D, (int32_t*)D, cu, n_seq, nullptr, nullptr, D2,
                                  with_cache ? D : nullptr, with_cache ? D : nullptr, with_cache ? &c : nullptr, ws.p,
                                  ws.n, nullptr) == QWATTN_OK);
    EXPECT(launched() == 4);
    if (with_cache) {  // an append through the sublayer
      int32_t* sp = new int32_t[n_seq]{100, 211};
      EXPECT(qwattn_attention_layer(&p, QWATTN_BF16, 4096, D, D, D, D, D, (int32_t*)D, cu, n_seq, (int32_t*)D, sp, D2,
                                    D, D, &c, ws.p, ws.n, nullptr) == QWATTN_OK);
      EXPECT(launched() == 4);
      sp[1] = 512;  // 512 + 1 > capacity 512
      EXPECT(qwattn_attention_layer(&p, QWATTN_BF16, 4096, D, D, D, D, D, (int32_t*)D, cu, n_seq, (int32_t*)D, sp, D2,
                                    D, D, &c, ws.p, ws.n, nullptr) == QWATTN_ERR_CAPACITY);
      EXPECT(launched() == 0);
      delete[] sp;
    }
    delete[] cu;
  }
  // the gated sublayer (head_dim 256, query and gate per head), with and without the cache
  for (int with_cache : {0, 1}) {
    const qwattn_params pg = params(16, 2, 256);
    const int n_seq = 3;
    int32_t* cu = new int32_t[n_seq + 1]{0, 100, 100, 613};
    stub::n_tok = 613;
    const size_t need = qwattn_attention_layer_workspace_size(&pg, QWATTN_BF16, 2048, n_seq, 613, 513, with_cache);
    EXPECT(need > 0);
    HostWs ws(need);
    const qwattn_cache_desc c = cache(2, 600, 256);
    EXPECT(qwattn_attention_layer(&pg, QWATTN_BF16, 2048, D, D, D, D, D, (int32_t*)D, cu, n_seq, nullptr, nullptr,
                                  D2, with_cache ? D : nullptr, with_cache ? D : nullptr, with_cache ? &c : nullptr,
                                  ws.p, ws.n, nullptr) == QWATTN_OK);
    EXPECT(launched() == 4);
    delete[] cu;
  }
  qwattn_params pr = params(16, 2, 256);
  pr.rotary_dim = 256;  // the fused gated projection rotates at most 128 dims
  EXPECT(qwattn_attention_layer_workspace_size(&pr, QWATTN_BF16, 2048, 1, 5, 5, 0) == 0);
  EXPECT(qwattn_attention_layer(&p, QWATTN_F32, 4096, D, D, D, D, D, (int32_t*)D, nullptr, 0, nullptr, nullptr, D2,
                                nullptr, nullptr, nullptr, nullptr, 0, nullptr) == QWATTN_ERR_UNSUPPORTED);
  EXPECT(qwattn_linear(QWATTN_BF16, D, D, 1000, 384, 4096, D2, nullptr) == QWATTN_OK);
  EXPECT(launched() == 1);
  EXPECT(qwattn_linear(QWATTN_BF16, D, D, 1000, 383, 4096, D2, nullptr) == QWATTN_ERR_UNSUPPORTED);
  EXPECT(qwattn_linear(QWATTN_BF16, D, D, 1000, 384, (1 << 23) + 64, D2, nullptr) == QWATTN_ERR_UNSUPPORTED);
  EXPECT(qwattn_linear(QWATTN_BF16, D, D, -1, 384, 64, D2, nullptr) == QWATTN_ERR_INVALID_ARG);
  EXPECT(qwattn_linear(QWATTN_BF16, ODD, D, 10, 384, 64, D2, nullptr) == QWATTN_ERR_INVALID_ARG);
  EXPECT(launched() == 0);
}

void invalid_param_cases() {
  int32_t* cu = new int32_t[2]{0, 5};
  const qwattn_cache_desc c = cache(8, 100, 128);
  auto pre = [&](const qwattn_params* p, qwattn_dtype dt, const qwattn_cache_desc* cd) {
    return qwattn_prefill(p, dt, D, D, D, D, D, (int32_t*)D, cu, 1, D2, cd ? D : nullptr, cd ? D : nullptr, cd, D,
                          1 << 30, nullptr);
  };
  EXPECT(pre(nullptr, QWATTN_BF16, nullptr) == QWATTN_ERR_INVALID_ARG);
  qwattn_params p = params(32, 8);
  EXPECT(pre(&p, (qwattn_dtype)7, nullptr) == QWATTN_ERR_INVALID_ARG);
  p.n_q_heads = 30;
  EXPECT(pre(&p, QWATTN_BF16, nullptr) == QWATTN_ERR_INVALID_ARG);
  p = params(32, 8);
  p.head_dim = 64;
  EXPECT(pre(&p, QWATTN_BF16, nullptr) == QWATTN_ERR_UNSUPPORTED);
  p = params(32, 8);
  p.eps = -1.f;
  EXPECT(pre(&p, QWATTN_BF16, nullptr) == QWATTN_ERR_INVALID_ARG);
  p = params(1 << 16, 1 << 16);
  EXPECT(pre(&p, QWATTN_BF16, nullptr) == QWATTN_ERR_UNSUPPORTED);
  p = params(512, 1);
  EXPECT(pre(&p, QWATTN_BF16, nullptr) == QWATTN_ERR_UNSUPPORTED);  // g > 256
  p = params(32, 8);
  qwattn_cache_desc bad = c;
  bad.stride_tok = (1 << 25) + 8;  // a 64-slot tile's row offsets would not fit 32 bits
  bad.stride_head = bad.stride_tok * 100;
  bad.stride_seq = bad.stride_head * 8;
  EXPECT(pre(&p, QWATTN_BF16, &bad) == QWATTN_ERR_UNSUPPORTED);
  bad = c;
  bad.stride_seq = int64_t(1) << 62;  // would overflow the element offsets
  EXPECT(pre(&p, QWATTN_BF16, &bad) == QWATTN_ERR_INVALID_ARG);
  bad = c;
  bad.stride_tok = 130;  // rows not 16-byte aligned
  EXPECT(pre(&p, QWATTN_BF16, &bad) == QWATTN_ERR_INVALID_ARG);
  bad = c;
  bad.capacity = 4;  // 5 tokens do not fit
  EXPECT(pre(&p, QWATTN_BF16, &bad) == QWATTN_ERR_CAPACITY);
  cu[0] = 1;
  EXPECT(pre(&p, QWATTN_BF16, nullptr) == QWATTN_ERR_INVALID_ARG);
  cu[0] = 0;
  EXPECT(qwattn_prefill(&p, QWATTN_BF16, ODD, D, D, D, D, (int32_t*)D, cu, 1, D2, nullptr, nullptr, nullptr, D,
                        1 << 30, nullptr) == QWATTN_ERR_INVALID_ARG);
  EXPECT(qwattn_qk_norm_rope(&p, QWATTN_BF16, nullptr, nullptr, D, D, (int32_t*)D, 4, nullptr, nullptr, nullptr) ==
         QWATTN_ERR_INVALID_ARG);
  EXPECT(qwattn_set_timing_events(D, nullptr) == QWATTN_ERR_INVALID_ARG);
  EXPECT(qwattn_mfma_probe(0, (float*)D, nullptr) == QWATTN_ERR_INVALID_ARG);
  EXPECT(qwattn_hbm_read_probe(D, 24, (float*)D, nullptr) == QWATTN_ERR_INVALID_ARG);
  EXPECT(launched() == 0);
  // valid standalone calls and the measurement aids, with the timing hook set
  EXPECT(qwattn_set_timing_events(D, D2) == QWATTN_OK);
  EXPECT(qwattn_qk_norm_rope(&p, QWATTN_BF16, D, D, D, D, (int32_t*)D, 4, D2, D2, nullptr) == QWATTN_OK);
  EXPECT(qwattn_mfma_probe(100, (float*)D, nullptr) == QWATTN_OK);
  EXPECT(qwattn_mfma_probe_flops(100) > 0.0);
  EXPECT(qwattn_hbm_read_probe(D, 1 << 20, (float*)D, nullptr) == QWATTN_OK);
  EXPECT(launched() == 3);
  for (int s = 0; s <= 6; ++s) EXPECT(std::strlen(qwattn_status_str((qwattn_status)s)) > 0);
  EXPECT(qwattn_abi_version() == QWATTN_ABI_VERSION);
  delete[] cu;
}

}  // namespace

int main() {
  invalid_param_cases();
  prefill_cases();
  append_cases();
  decode_cases();
  noalloc_limit_cases();
  layer_and_linear_cases();
  if (failures) {
    std::fprintf(stderr, "%d of %d checks failed\n", failures, checks);
    return 1;
  }
  std::printf("ok %d checks\n", checks);
  return 0;
}
