// QK-Norm then rotate-half RoPE over token rows (HBM-bound).
//
// QK-Norm: each 128-value head row is divided by sqrt(mean of squares + eps),
// the mean taken in fp32, then scaled by gamma ("7.2 Qwen3 全规模实现" §7.2.1
// RMSNorm; "Qwen3" notes, "QK-Norm").  RoPE: dims i and i+64 of a row at
// position p turn by p * theta^(-2i/128) ("7.2 Qwen3 全规模实现" §7.2.1 RoPE).
// The norm comes first, as four of the five pages print it.
//
// A workgroup owns up to 8 consecutive tokens (one when there are few).  It
// first tabulates cos/sin of its tokens' 64 angles in LDS (shared by every head
// of a token), then 16-lane
// groups walk the token rows: lane j of a group holds dims 4j..4j+3 and
// 64+4j..64+4j+3, so each lane owns whole rotation pairs and the row's sum of
// squares is a 16-lane reduction.  Loads and stores are 8-byte (bf16) or
// 16-byte (fp32) per lane, 128 contiguous bytes per half-row.
#include "kernels.h"

namespace qw {
namespace {

constexpr int kMaxTokens = 8;  // tokens per workgroup (fewer for small inputs)
constexpr int kRowsInFlight = 4;

template <class S>
__global__ __launch_bounds__(256) void k_normrope(NormRopeArgs a, int tb) {
  using T = typename S::T;
  __shared__ float cos_t[kMaxTokens][kHalf];
  __shared__ float sin_t[kMaxTokens][kHalf];
  __shared__ int tok_seq[kMaxTokens];
  __shared__ int tok_pos[kMaxTokens];

  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.x * tb;
  const int nt = (int)min((int64_t)tb, a.n_tok - tok0);

  if (tid < nt) {
    const int64_t n = tok0 + tid;
    int s = 0, p;
    if (a.mode == kPosPacked) {
      int lo = 0, hi = a.n_seq;  // first index with cu[idx] > n, minus one
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)a.cu[mid + 1] <= n) lo = mid + 1; else hi = mid;
      }
      s = lo;
      p = (int)(n - a.cu[s]);
    } else if (a.mode == kPosDecode) {
      s = (int)n;
      p = a.pos[n];
    } else {
      p = a.pos[n];
    }
    tok_seq[tid] = s;
    tok_pos[tid] = p;
  }
  __syncthreads();
  for (int e = tid; e < nt * kHalf; e += 256) {
    const int t = e / kHalf, i = e % kHalf;
    float c, s;
    rope_cos_sin(tok_pos[t], a.rope.w[i], c, s);
    cos_t[t][i] = c;
    sin_t[t][i] = s;
  }
  __syncthreads();

  const int grp = tid >> 4, j = tid & 15;
  float gam[2][8];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    if (a.heads[w] > 0) {
      float lo4[4], hi4[4];
      load4((const T*)a.gamma[w] + 4 * j, lo4);
      load4((const T*)a.gamma[w] + kHalf + 4 * j, hi4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { gam[w][e] = lo4[e]; gam[w][4 + e] = hi4[e]; }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gam[w][e] = 0.f;
    }
  }

  const int Hq = a.heads[0], Hk = a.heads[1], Hv = a.heads[2];
  const int Ht = Hq + Hk + Hv;
  const int n_rows = nt * Ht;
  // Each 16-lane group takes rows grp, grp + 16, ...; kRowsInFlight rows are
  // loaded before any is reduced, to keep several loads in flight per lane.
  for (int r0 = grp; r0 < n_rows; r0 += 16 * kRowsInFlight) {
    float x1[kRowsInFlight][4], x2[kRowsInFlight][4];
#pragma unroll
    for (int i = 0; i < kRowsInFlight; ++i) {
      const int r = r0 + 16 * i;
      if (r < n_rows) {
        const int t = r / Ht;
        int h = r - t * Ht;
        const int which = h < Hq ? 0 : (h < Hq + Hk ? 1 : 2);
        h -= which == 0 ? 0 : (which == 1 ? Hq : Hq + Hk);
        const T* src = (const T*)a.x[which] + ((tok0 + t) * a.heads[which] + h) * kD;
        load4(src + 4 * j, x1[i]);
        load4(src + kHalf + 4 * j, x2[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kRowsInFlight; ++i) {
      const int r = r0 + 16 * i;
      if (r >= n_rows) break;  // uniform across the 16-lane group
      const int t = r / Ht;
      int h = r - t * Ht;
      const int64_t n = tok0 + t;
      const int which = h < Hq ? 0 : (h < Hq + Hk ? 1 : 2);
      h -= which == 0 ? 0 : (which == 1 ? Hq : Hq + Hk);
      const int seq = tok_seq[t], pos = tok_pos[t];
      if (which == 2) {  // V: copied into the cache slot as is
        T* dst = (T*)a.v_cache + seq * a.cs_seq + h * a.cs_head + (int64_t)pos * a.cs_tok;
        store4(dst + 4 * j, x1[i]);
        store4(dst + kHalf + 4 * j, x2[i]);
        continue;
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += x1[i][e] * x1[i][e] + x2[i][e] * x2[i][e];
      ss = row16_sum(ss);
      const float inv = rsqrtf(ss * (1.0f / kD) + a.eps);
      float y1[4], y2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a1 = x1[i][e] * inv * gam[which][e];
        const float a2 = x2[i][e] * inv * gam[which][4 + e];
        const float c = cos_t[t][4 * j + e], sn = sin_t[t][4 * j + e];
        y1[e] = a1 * c - a2 * sn;
        y2[e] = a2 * c + a1 * sn;
      }
      T* dst;
      if (which == 1 && a.k_cache)
        dst = (T*)a.k_cache + seq * a.cs_seq + h * a.cs_head + (int64_t)pos * a.cs_tok;
      else
        dst = (T*)a.out[which] + (n * a.heads[which] + h) * kD;
      store4(dst + 4 * j, y1);
      store4(dst + kHalf + 4 * j, y2);
    }
  }
}

}  // namespace

hipError_t launch_normrope(bool bf16, const NormRopeArgs& a, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  // Few tokens (decode): one token per workgroup, so the rows spread over CUs.
  const int tb = a.n_tok >= 4096 ? kMaxTokens : (a.n_tok >= 1024 ? 2 : 1);
  const int64_t blocks = (a.n_tok + tb - 1) / tb;
  if (bf16)
    hipLaunchKernelGGL(k_normrope<BF16>, dim3((unsigned)blocks), dim3(256), 0, st, a, tb);
  else
    hipLaunchKernelGGL(k_normrope<F32>, dim3((unsigned)blocks), dim3(256), 0, st, a, tb);
  return hipGetLastError();
}

}  // namespace qw
