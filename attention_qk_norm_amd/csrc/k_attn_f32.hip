// Causal grouped-query attention in fp32 throughout (fp32 inputs): the same
// definition as the bf16 prefill ("7.2 Qwen3 全规模实现" §7.2.1 GQA + QKNorm;
// "Transformer 20. Qwen 3 架构拆解" §2.2), computed with fp32 FMAs so that no
// operand is rounded below fp32.  It serves fp32 prefill and fp32 decode.
//
// Queries arrive already normed and rotated (fp32, from the norm+RoPE pass);
// keys already normed and rotated (cache or workspace).  A workgroup owns one
// (sequence, KV head) and up to 64 query rows = tokens x the g heads of the
// group; four lanes share a row, each holding a quarter of its dims (32 of 128,
// or 64 of 256), so a score is that many FMAs plus a 4-lane reduction.  K and V
// tiles (32 keys at head_dim 128, 16 at 256) are staged in LDS and read as
// broadcasts.  Online softmax in fp32 (exp2 with log2(e) folded into the
// scale); the gated layers ("第 20 章 Qwen3 与 Qwen3.5" §20.4) then multiply
// each output row by sigmoid of its gate row.  Decode mode: one query token per sequence at start_pos, keys
// 0 .. start_pos of the cache (the new key already appended).  Prefill mode
// with start_pos set (an append): sequence s's rows are new tokens at
// start_pos[s] .., attending to cache slots 0 .. their own position.
#include "kernels.h"

namespace qw {
namespace {

template <int D>
__global__ __launch_bounds__(256) void k_attn_f32(PrefillArgs a) {
  constexpr int kKeys = 4096 / D;  // keys per LDS tile
  constexpr int DPL = D / 4;       // dims per lane
  __shared__ __attribute__((aligned(16))) float kt[kKeys][D];
  __shared__ __attribute__((aligned(16))) float vt[kKeys][D];

  const int tid = threadIdx.x;
  const int u = blockIdx.x % a.Hkv;
  int s, qt;
  if (a.decode) {
    s = blockIdx.x / a.Hkv;
    qt = 0;
  } else {
    const PrefillItem item = a.items[blockIdx.x / a.Hkv];
    s = item.s;
    qt = item.qt;
  }
  if (s < 0 || s >= a.n_seq) return;
  int row_base, L, pos0;
  if (a.decode) {
    row_base = s;        // query row index in qhat / out
    pos0 = a.start_pos[s];
    L = 1;
  } else {
    row_base = a.cu[s];
    pos0 = a.start_pos ? a.start_pos[s] : 0;  // an append: new tokens at start_pos ..
    L = a.cu[s + 1] - row_base;
  }
  const int tok_base = qt * a.bm_tok;
  if (qt < 0 || tok_base >= L || pos0 < 0) return;
  const int n_kv = pos0 + min(L, tok_base + a.bm_tok);

  const int r = tid >> 2, sub = tid & 3;
  const int hoff = r % a.g, toff = r / a.g;
  const int qtok = tok_base + toff;
  const bool valid = toff < a.bm_tok && qtok < L;
  const int qpos = valid ? pos0 + qtok : 0x3fffffff;
  const int t_head = u * a.g + hoff;

  float q[DPL], o[DPL];
  if (valid) {
    const float* src = (const float*)a.qhat + ((int64_t)(row_base + qtok) * a.Hq + t_head) * D + DPL * sub;
#pragma unroll
    for (int e = 0; e < DPL; e += 4) {
      f32x4 x = *reinterpret_cast<const f32x4*>(src + e);
      q[e] = x[0]; q[e + 1] = x[1]; q[e + 2] = x[2]; q[e + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < DPL; ++e) q[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  const float* kbase = (const float*)a.khat + u * a.ks_head +
                       (a.k_packed ? (int64_t)row_base * a.ks_tok : (int64_t)s * a.ks_seq);
  const float* vbase = (const float*)a.v + u * a.vs_head +
                       (a.v_packed ? (int64_t)row_base * a.vs_tok : (int64_t)s * a.vs_seq);

  for (int k0 = 0; k0 < n_kv; k0 += kKeys) {
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m) {  // 1024 16-byte chunks per tile and tensor
      const int c = tid + 256 * m;
      const int row = c / (D / 4), col = (c % (D / 4)) * 4;
      const int key = k0 + row;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (key < n_kv) {
        kx = *reinterpret_cast<const f32x4*>(kbase + (int64_t)key * a.ks_tok + col);
        vx = *reinterpret_cast<const f32x4*>(vbase + (int64_t)key * a.vs_tok + col);
      }
      *reinterpret_cast<f32x4*>(&kt[row][col]) = kx;
      *reinterpret_cast<f32x4*>(&vt[row][col]) = vx;
    }
    __syncthreads();

    float sc[kKeys];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc = fmaf(q[e], kt[j][DPL * sub + e], acc);
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      float x = acc * a.scale_log2e;
      if (k0 + j > qpos) x = -INFINITY;
      sc[j] = x;
      mt = fmaxf(mt, x);
    }
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = exp2f(sc[j] - m_new);
      psum += p;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(p, vt[j][DPL * sub + e], o[e]);
    }
    l_run = l_run * alpha + psum;
  }

  if (valid) {
    const float inv_l = 1.0f / l_run;
    const int64_t row = (int64_t)(row_base + qtok) * a.Hq + t_head;
    float* dst = (float*)a.out + row * D + DPL * sub;
    const float* gp = a.gate ? (const float*)a.gate + row * a.q_row + DPL * sub : nullptr;
#pragma unroll
    for (int e = 0; e < DPL; e += 4) {
      f32x4 x = {o[e] * inv_l, o[e + 1] * inv_l, o[e + 2] * inv_l, o[e + 3] * inv_l};
      if (gp) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(gp + e);
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] /= 1.0f + expf(-gv[c]);
      }
      *reinterpret_cast<f32x4*>(dst + e) = x;
    }
  }
}

}  // namespace

hipError_t launch_attn_f32(const PrefillArgs& a, int n_items, hipStream_t st) {
  if (n_items <= 0) return hipSuccess;
  const int64_t blocks = (int64_t)n_items * a.Hkv;
  if (a.head_dim == kMaxD)
    hipLaunchKernelGGL(k_attn_f32<kMaxD>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_attn_f32<kD>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace qw
