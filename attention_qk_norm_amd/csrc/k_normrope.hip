// QK-Norm then rotate-half RoPE over token rows (HBM-bound).
//
// QK-Norm: each 128-value head row is divided by sqrt(mean of squares + eps),
// the mean taken in fp32, then scaled by gamma ("7.2 Qwen3 全规模实现" §7.2.1
// RMSNorm; "Qwen3" notes, "QK-Norm").  RoPE: dims i and i+64 of a row at
// position p turn by p * theta^(-2i/128) ("7.2 Qwen3 全规模实现" §7.2.1 RoPE).
// The norm comes first, as four of the five pages print it; order = 1 gives the
// other order ("Transformer 20. Qwen 3 架构拆解" §2.2: RoPE, then the norm).
//
// A workgroup owns `tb` consecutive tokens (16 for large inputs, down to one
// for a decode step).  It first finds each token's sequence and position, then
// tabulates cos/sin of the tokens' 64 angles in LDS (shared by every head of a
// token).  A 16-lane group then walks whole rows: lane j holds dims 8j..8j+7
// (one 16-byte load per row in bf16), its rotation partners sit in lane j ^ 8
// and arrive by one DPP row rotation, and the row's sum of squares is a 16-lane
// reduction.  Each group serves one token (or a share of its heads when a
// workgroup has fewer than 16 tokens) and keeps that token's cos/sin in
// registers across the heads; four rows are loaded before any is reduced.
// Tensor selection (q, k, v) is a uniform outer loop, so every address base is
// a scalar.
#include "kernels.h"

namespace qw {
namespace {

constexpr int kMaxTokens = 16;    // tokens per workgroup
constexpr int kRowsInFlight = 4;  // rows loaded per group before any is reduced
constexpr int kCuStage = 2048;    // sequence offsets staged in LDS (packed mode)

// 8 consecutive values of a row <-> registers.  bf16: one 16-byte access.
__device__ __forceinline__ void load8(const uint16_t* p, uint32_t (&raw)[8]) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  raw[0] = v[0]; raw[1] = v[1]; raw[2] = v[2]; raw[3] = v[3];
}
__device__ __forceinline__ void load8(const float* p, uint32_t (&raw)[8]) {
  const u32x4 v0 = *reinterpret_cast<const u32x4*>(p);
  const u32x4 v1 = *reinterpret_cast<const u32x4*>(p + 4);
  raw[0] = v0[0]; raw[1] = v0[1]; raw[2] = v0[2]; raw[3] = v0[3];
  raw[4] = v1[0]; raw[5] = v1[1]; raw[6] = v1[2]; raw[7] = v1[3];
}
__device__ __forceinline__ void store_raw8(uint16_t* p, const uint32_t (&raw)[8]) {
  *reinterpret_cast<u32x4*>(p) = u32x4{raw[0], raw[1], raw[2], raw[3]};
}
__device__ __forceinline__ void store_raw8(float* p, const uint32_t (&raw)[8]) {
  *reinterpret_cast<u32x4*>(p) = u32x4{raw[0], raw[1], raw[2], raw[3]};
  *reinterpret_cast<u32x4*>(p + 4) = u32x4{raw[4], raw[5], raw[6], raw[7]};
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&y)[8]) {
  *reinterpret_cast<u32x4*>(p) = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                       pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
}
__device__ __forceinline__ void store8(float* p, const float (&y)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{y[4], y[5], y[6], y[7]};
}
// Raw registers -> 8 floats, and the partner lane's (j ^ 8) values.
template <class S>
__device__ __forceinline__ void unpack8(const uint32_t (&raw)[8], float (&x)[8]) {
  if constexpr (S::kBytes == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[2 * e] = bf16_lo(raw[e]); x[2 * e + 1] = bf16_hi(raw[e]); }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(raw[e]);
  }
}
template <class S>
__device__ __forceinline__ void partner8(const uint32_t (&raw)[8], uint32_t (&out)[8]) {
  constexpr int n = S::kBytes == 2 ? 4 : 8;
#pragma unroll
  for (int e = 0; e < n; ++e)  // row_ror 8: lane j of each 16-lane row reads lane (j + 8) % 16
    out[e] = (uint32_t)__builtin_amdgcn_mov_dpp((int)raw[e], 0x128, 0xF, 0xF, false);
}

template <class S>
__global__ __launch_bounds__(256) void k_normrope(NormRopeArgs a, int tb) {
  using T = typename S::T;
  __shared__ float2 cs_t[kMaxTokens][kHalf];  // (cos, sin) of token t, angle i
  __shared__ int tok_seq[kMaxTokens];
  __shared__ int tok_pos[kMaxTokens];
  __shared__ int cu_s[kCuStage];

  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.x * tb;
  const int nt = (int)min((int64_t)tb, a.n_tok - tok0);

  // ---- sequence and position of each token
  const bool staged = a.mode == kPosPacked && a.n_seq < kCuStage;
  if (staged) {
    for (int i = tid; i <= a.n_seq; i += 256) cu_s[i] = a.cu[i];
    __syncthreads();
  }
  if (tid < nt) {
    const int64_t n = tok0 + tid;
    int s = 0, p;
    if (a.mode == kPosPacked) {
      int lo = 0, hi = a.n_seq;  // last s with cu[s] <= n: first index with cu[idx+1] > n
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int c = staged ? cu_s[mid + 1] : a.cu[mid + 1];
        if ((int64_t)c <= n) lo = mid + 1; else hi = mid;
      }
      s = lo;
      p = (int)(n - (staged ? cu_s[s] : a.cu[s])) + (a.pos ? a.pos[s] : 0);  // append: from start_pos[s]
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
  {
    const double w = a.rope.w[tid & (kHalf - 1)];  // 256 is a multiple of 64: one angle index per thread
    for (int e = tid; e < nt * kHalf; e += 256) {
      float c, s;
      rope_cos_sin(tok_pos[e / kHalf], w, c, s);
      cs_t[e / kHalf][e % kHalf] = make_float2(c, s);
    }
  }
  __syncthreads();

  // ---- rows: group g serves token g / G and heads (g % G) + G k, G = 16 / tb
  const int grp = tid >> 4, j = tid & 15;
  const int G = kHalf / 4 / tb;  // 16 / tb
  const int t = grp / G, sub = grp - t * G;
  if (t >= nt) return;  // no barrier below
  const int64_t n = tok0 + t;
  const int seq = tok_seq[t], pos = tok_pos[t];
  const float sgn = j < 8 ? -1.f : 1.f;  // own dim in the first half: own*c - partner*s
  float cs[8], sn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 v = cs_t[t][8 * (j & 7) + e];
    cs[e] = v.x;
    sn[e] = v.y;
  }

#pragma unroll
  for (int which = 0; which < 3; ++which) {
    const int H = a.heads[which];
    if (H == 0) continue;
    const T* src = (const T*)a.x[which] + n * H * kD + 8 * j;
    float go[8], gp[8];  // gamma of the lane's own dims and of its partners
    if (which < 2) {
      uint32_t r[8];
      load8((const T*)a.gamma[which] + 8 * j, r);
      unpack8<S>(r, go);
      load8((const T*)a.gamma[which] + 8 * (j ^ 8), r);
      unpack8<S>(r, gp);
    }
    for (int h0 = sub; h0 < H; h0 += G * kRowsInFlight) {
      uint32_t raw[kRowsInFlight][8];
#pragma unroll
      for (int i = 0; i < kRowsInFlight; ++i) {
        const int h = h0 + G * i;
        if (h < H) load8(src + h * kD, raw[i]);
      }
#pragma unroll
      for (int i = 0; i < kRowsInFlight; ++i) {
        const int h = h0 + G * i;
        if (h >= H) break;  // uniform across the 16-lane group
        if (which == 2) {   // V: copied into the cache slot as is
          T* dst = (T*)a.v_cache + seq * a.cs_seq + h * a.cs_head + (int64_t)pos * a.cs_tok + 8 * j;
          store_raw8(dst, raw[i]);
          continue;
        }
        uint32_t praw[8];
        partner8<S>(raw[i], praw);
        float xo[8], xp[8];
        unpack8<S>(raw[i], xo);
        unpack8<S>(praw, xp);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += xo[e] * xo[e];
        ss = row16_sum(ss);
        const float inv = rsqrtf(ss * (1.0f / kD) + a.eps);
        // RMS is rotation-invariant, so one inv serves both orders; they differ
        // in whether gamma scales the dims before the rotation (norm first) or
        // after it (RoPE first).
        float y[8];
        if (a.order == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float own = xo[e] * inv * go[e];
            const float par = xp[e] * inv * gp[e];
            y[e] = own * cs[e] + sgn * (par * sn[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = (xo[e] * cs[e] + sgn * (xp[e] * sn[e])) * inv * go[e];
        }
        T* dst;
        if (which == 1 && a.k_cache)
          dst = (T*)a.k_cache + seq * a.cs_seq + h * a.cs_head + (int64_t)pos * a.cs_tok;
        else
          dst = (T*)a.out[which] + (n * H + h) * kD;
        store8(dst + 8 * j, y);
      }
    }
  }
}

}  // namespace

hipError_t launch_normrope(bool bf16, const NormRopeArgs& a, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  // Enough workgroups to cover the chip: 16 tokens each for large inputs, down
  // to one token each (a decode step), so the rows spread over the CUs.
  int tb = kMaxTokens;
  while (tb > 1 && a.n_tok < (int64_t)tb * 1024) tb >>= 1;
  const int64_t blocks = (a.n_tok + tb - 1) / tb;
  if (bf16)
    hipLaunchKernelGGL(k_normrope<BF16>, dim3((unsigned)blocks), dim3(256), 0, st, a, tb);
  else
    hipLaunchKernelGGL(k_normrope<F32>, dim3((unsigned)blocks), dim3(256), 0, st, a, tb);
  return hipGetLastError();
}

}  // namespace qw
