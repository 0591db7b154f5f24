// QK-Norm then rotate-half RoPE over token rows (HBM-bound).
//
// QK-Norm: each head row is divided by sqrt(mean of squares + eps), the mean
// taken in fp32, then scaled by gamma ("7.2 Qwen3 全规模实现" §7.2.1 RMSNorm;
// "Qwen3" notes, "QK-Norm") -- or, in the gated layers of Qwen3-Next /
// Qwen3.5, by 1 + gamma (the zero-centred norm; "第 20 章 Qwen3 与 Qwen3.5"
// §20.4).  RoPE: dims i and i + rot/2 of a row at position p turn by
// p * theta^(-2i/rot), i < rot/2 ("7.2 Qwen3 全规模实现" §7.2.1 RoPE, where
// rot = head_dim = 128); the gated layers turn only the first rot of their
// 256 coordinates and pass the rest ("第 20 章" §20.4).  The norm comes first,
// as four of the five pages print it; order = 1 gives the other order
// ("Transformer 20. Qwen 3 架构拆解" §2.2: RoPE, then the norm).
//
// A workgroup owns `tb` consecutive tokens (16 for large inputs, down to one
// for a decode step).  It first finds each token's sequence and position, then
// tabulates cos/sin of the tokens' rot/2 angles in LDS (shared by every head
// of a token).  A 16-lane group then walks whole rows: lane j holds the D/16
// dims from D/16 * j on (16-byte accesses); the rotation partners of its dims
// sit in lane j +- off, off = (rot/2) / (D/16), and arrive by one lane exchange
// (a DPP row rotation when off = 8); the row's sum of squares is a 16-lane
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

// N consecutive values of a row held as raw dwords (16-byte accesses).
template <class S, int N>
struct Row {
  static constexpr int kWords = N * S::kBytes / 4;
  uint32_t w[kWords];
};
template <class S, int N>
__device__ __forceinline__ void load_row(const typename S::T* p, Row<S, N>& r) {
#pragma unroll
  for (int i = 0; i < Row<S, N>::kWords / 4; ++i) {
    const u32x4 v = reinterpret_cast<const u32x4*>(p)[i];
    r.w[4 * i] = v[0]; r.w[4 * i + 1] = v[1]; r.w[4 * i + 2] = v[2]; r.w[4 * i + 3] = v[3];
  }
}
template <class S, int N>
__device__ __forceinline__ void store_row(typename S::T* p, const Row<S, N>& r) {
#pragma unroll
  for (int i = 0; i < Row<S, N>::kWords / 4; ++i)
    reinterpret_cast<u32x4*>(p)[i] = u32x4{r.w[4 * i], r.w[4 * i + 1], r.w[4 * i + 2], r.w[4 * i + 3]};
}
template <class S, int N>
__device__ __forceinline__ void unpack(const Row<S, N>& r, float (&x)[N]) {
  if constexpr (S::kBytes == 2) {
#pragma unroll
    for (int e = 0; e < N / 2; ++e) { x[2 * e] = bf16_lo(r.w[e]); x[2 * e + 1] = bf16_hi(r.w[e]); }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] = __uint_as_float(r.w[e]);
  }
}
template <class S, int N>
__device__ __forceinline__ void store_vals(typename S::T* p, const float (&y)[N]) {
  Row<S, N> r;
  if constexpr (S::kBytes == 2) {
#pragma unroll
    for (int e = 0; e < N / 2; ++e) r.w[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) r.w[e] = __float_as_uint(y[e]);
  }
  store_row<S, N>(p, r);
}

template <class S, int D>
__global__ __launch_bounds__(256) void k_normrope(NormRopeArgs a, int tb) {
  using T = typename S::T;
  constexpr int DPL = D / 16;  // dims per lane
  __shared__ float2 cs_t[kMaxTokens][D / 2];  // (cos, sin) of token t, angle i
  __shared__ int tok_seq[kMaxTokens];
  __shared__ int tok_pos[kMaxTokens];
  __shared__ int cu_s[kCuStage];

  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.x * tb;
  const int nt = (int)min((int64_t)tb, a.n_tok - tok0);
  const int half = a.rot / 2;  // angles per token

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
  for (int e = tid; e < nt * half; e += 256) {
    float c, s;
    rope_cos_sin(tok_pos[e / half], a.rope.w[e % half], c, s);
    cs_t[e / half][e % half] = make_float2(c, s);
  }
  __syncthreads();

  // ---- rows: group g serves token g / G and heads (g % G) + G k, G = 16 / tb
  const int grp = tid >> 4, j = tid & 15;
  const int G = kMaxTokens / tb;
  const int t = grp / G, sub = grp - t * G;
  if (t >= nt) return;  // no barrier below
  const int64_t n = tok0 + t;
  const int seq = tok_seq[t], pos = tok_pos[t];
  // Dims i < rot/2 (lanes j < off) pair with i + rot/2 (lanes off .. 2 off - 1);
  // lanes from 2 off on hold unrotated dims (cos 1, sin 0, partner = self).
  const int off = half / DPL;
  const bool first = j < off, turned = j < 2 * off;
  const int pj = first ? j + off : (turned ? j - off : j);
  const int partner = (tid & 63 & ~15) | pj;
  const bool dpp = off == 8;  // partner = j ^ 8 for every lane: one DPP row rotation
  const float sgn = first ? -1.f : 1.f;  // own dim in the first half: own*c - partner*s
  float cs[DPL], sn[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const float2 v = turned ? cs_t[t][DPL * (first ? j : j - off) + e] : make_float2(1.f, 0.f);
    cs[e] = v.x;
    sn[e] = v.y;
  }

#pragma unroll
  for (int which = 0; which < 3; ++which) {
    const int H = a.heads[which];
    if (H == 0) continue;
    const int64_t in_row = a.in_row[which];
    const T* src = (const T*)a.x[which] + n * H * in_row + DPL * j;
    float go[DPL], gp[DPL];  // norm scale of the lane's own dims and of its partner's
    if (which < 2) {
      Row<S, DPL> r;
      load_row<S, DPL>((const T*)a.gamma[which] + DPL * j, r);
      unpack<S, DPL>(r, go);
      load_row<S, DPL>((const T*)a.gamma[which] + DPL * pj, r);
      unpack<S, DPL>(r, gp);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        go[e] += a.gamma_offset;
        gp[e] += a.gamma_offset;
      }
    }
    for (int h0 = sub; h0 < H; h0 += G * kRowsInFlight) {
      Row<S, DPL> raw[kRowsInFlight];
#pragma unroll
      for (int i = 0; i < kRowsInFlight; ++i) {
        const int h = h0 + G * i;
        if (h < H) load_row<S, DPL>(src + h * in_row, raw[i]);
      }
#pragma unroll
      for (int i = 0; i < kRowsInFlight; ++i) {
        const int h = h0 + G * i;
        if (h >= H) break;  // uniform across the 16-lane group
        if (which == 2) {   // V: copied into the cache slot as is
          T* dst = (T*)a.v_cache + seq * a.cs_seq + h * a.cs_head + (int64_t)pos * a.cs_tok + DPL * j;
          store_row<S, DPL>(dst, raw[i]);
          continue;
        }
        Row<S, DPL> praw;
        if (dpp) {
#pragma unroll
          for (int e = 0; e < Row<S, DPL>::kWords; ++e)  // row_ror 8: lane j reads lane (j + 8) % 16
            praw.w[e] = (uint32_t)__builtin_amdgcn_mov_dpp((int)raw[i].w[e], 0x128, 0xF, 0xF, false);
        } else {
#pragma unroll
          for (int e = 0; e < Row<S, DPL>::kWords; ++e) praw.w[e] = (uint32_t)__shfl((int)raw[i].w[e], partner, 64);
        }
        float xo[DPL], xp[DPL];
        unpack<S, DPL>(raw[i], xo);
        unpack<S, DPL>(praw, xp);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) ss += xo[e] * xo[e];
        ss = row16_sum(ss);
        const float inv = rsqrtf(ss * (1.0f / D) + a.eps);
        // RMS is rotation-invariant, so one inv serves both orders; they differ
        // in whether the norm scale applies to the dims before the rotation
        // (norm first) or after it (RoPE first).
        float y[DPL];
        if (a.order == 0) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) {
            const float own = xo[e] * inv * go[e];
            const float par = xp[e] * inv * gp[e];
            y[e] = own * cs[e] + sgn * (par * sn[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < DPL; ++e) y[e] = (xo[e] * cs[e] + sgn * (xp[e] * sn[e])) * inv * go[e];
        }
        T* dst;
        if (which == 1 && a.k_cache)
          dst = (T*)a.k_cache + seq * a.cs_seq + h * a.cs_head + (int64_t)pos * a.cs_tok;
        else
          dst = (T*)a.out[which] + (n * H + h) * D;
        store_vals<S, DPL>(dst + DPL * j, y);
      }
    }
  }
}

template <class S>
hipError_t launch_t(const NormRopeArgs& a, int tb, int64_t blocks, hipStream_t st) {
  if (a.head_dim == kMaxD)
    hipLaunchKernelGGL((k_normrope<S, kMaxD>), dim3((unsigned)blocks), dim3(256), 0, st, a, tb);
  else
    hipLaunchKernelGGL((k_normrope<S, kD>), dim3((unsigned)blocks), dim3(256), 0, st, a, tb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_normrope(bool bf16, const NormRopeArgs& a, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  // Enough workgroups to cover the chip: 16 tokens each for large inputs, down
  // to one token each (a decode step), so the rows spread over the CUs.
  int tb = kMaxTokens;
  while (tb > 1 && a.n_tok < (int64_t)tb * 1024) tb >>= 1;
  const int64_t blocks = (a.n_tok + tb - 1) / tb;
  return bf16 ? launch_t<BF16>(a, tb, blocks, st) : launch_t<F32>(a, tb, blocks, st);
}

}  // namespace qw
