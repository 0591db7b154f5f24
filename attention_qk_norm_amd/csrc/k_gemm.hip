// Bias-free linear maps of the attention sublayer, bf16 in / fp32 accumulate,
// MFMA on gfx950: y = x W^T with W stored [out][in] ("Qwen3" notes, the
// Qwen3Attention excerpt: q_proj, k_proj, v_proj, o_proj; "7.2 Qwen3 全规模实现"
// §7.2.1 listing).
//
// Two epilogues:
//  * plain: y rounded to bf16 (o_proj, or any projection);
//  * qkv: the fused q/k/v projection.  Its output columns are head blocks of
//    128: Hq query heads, then Hkv key heads, then Hkv value heads (the three
//    weights stacked).  Query blocks are written raw (the attention kernel's
//    prologue norms and rotates them); key blocks are QK-Normed and rotated at
//    the token's position straight from the fp32 accumulators and written to
//    the KV cache (or a packed buffer); value blocks go to the cache as they
//    are.  So K and V reach HBM once, already in their cached form
//    ("Qwen3" notes: qkv_proj -> split -> RMSNorm(Q, K) -> RoPE).
//
// Tiling: a workgroup (4 waves) computes a 256-token x 256-column tile as
// C^T = W X^T with v_mfma_f32_32x32x16_bf16 (A = W fragment, B = X fragment,
// both 16-byte reads from LDS).  Wave w covers 128 tokens ((w >> 1) half) x
// 128 columns ((w & 1) half: exactly one head block), as 4 x 4 accumulators of
// 32 x 32.  In the transposed accumulator a lane owns ONE token (lane % 32) and
// 64 of the head block's 128 columns (the other 64 sit in lane ^ 32), and
// columns c and c + 64 (a RoPE pair) share a lane, so the norm is a lane-local
// sum plus one lane-pair exchange and the rotation is register-local.
//
// K steps of 64: the x and W tiles (256 rows x 128 B each) go HBM -> LDS
// directly (global_load_lds_dwordx4) into a two-stage ring of padded 1 KB
// blocks (row r in block r % 32, slot r / 32; 16-byte skew between blocks, so
// the 16 rows of a fragment read land in 16 distinct bank groups).
#include "kernels.h"

namespace qw {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kBlk = 1040;                 // 1 KB block (8 rows x 128 B) + 16 B skew
constexpr int kTile = 32 * kBlk;           // one 256 x 64 operand tile
constexpr int kStageBytes = 2 * kTile;     // x tile, then W tile
constexpr int kSmem = 2 * kStageBytes;     // two stages
// qkv: after the ring, the key norm scale (128 floats) and the RoPE
// frequencies (64 doubles), read per lane in the epilogue.
constexpr int kGammaOff = kSmem, kFreqOff = kSmem + 512, kSmemQkv = kSmem + 1024;
static_assert(kSmemQkv <= 160 * 1024, "LDS per workgroup");

__device__ __forceinline__ bf16x8 lds_load_b128(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

// Direct HBM -> LDS copy of 16 bytes per lane (lane l's bytes land at
// lds_base + 16 l; M0 holds the wave-uniform base, one wait state after
// writing it).  Inline assembly, so the compiler does not wait for every
// outstanding copy before each LDS read: the K loop waits for its own copies.
__device__ __forceinline__ void load_lds16_async(uint32_t lds_base, const void* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_base), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

// Sequence and position of packed token n: last s with cu[s] <= n.
__device__ __forceinline__ void token_position(const GemmArgs& a, int64_t n, int& s, int& pos) {
  int lo = 0, hi = a.n_seq;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)a.cu[mid + 1] <= n) lo = mid + 1; else hi = mid;
  }
  s = lo;
  pos = (int)(n - a.cu[s]) + (a.start_pos ? a.start_pos[s] : 0);
}

template <int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  lds_u8* lds = (lds_u8*)(smem);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wt = w >> 1, wc = w & 1;
  const int n = lane & 31, hg = lane >> 5;

  // Consecutive workgroups take consecutive column tiles of one token tile;
  // the 8 XCDs receive workgroups round-robin, so each XCD keeps a fixed
  // subset of the weight column tiles in its L2 while the token tiles stream.
  const int tiles_n = (a.N + kBN - 1) / kBN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int64_t row0 = (int64_t)tm * kBM;
  const int col0 = tn * kBN;

  const char* xbase = (const char*)(a.x + row0 * a.ldx);
  const char* wbase = (const char*)(a.w + (int64_t)col0 * a.ldw);
  const int64_t xrow = a.ldx * 2, wrow = a.ldw * 2;  // bytes per row
  const int last_x = (int)min((int64_t)kBM - 1, a.M - 1 - row0);
  const int last_w = min(kBN - 1, a.N - 1 - col0);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  // Wave w fills blocks 8w .. 8w+7 of both tiles; rows past the matrix repeat
  // its last row (their results are never stored).
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    const uint32_t xdst = lds0 + stage * kStageBytes, wdst = xdst + kTile;
    const char* xk = xbase + (int64_t)kt * kBK * 2;
    const char* wk = wbase + (int64_t)kt * kBK * 2;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int blk = wu * 8 + m;
      const int r = blk + 32 * (lane >> 3);
      load_lds16_async(xdst + blk * kBlk, xk, (uint32_t)(min(r, last_x) * xrow) + (lane & 7) * 16);
      load_lds16_async(wdst + blk * kBlk, wk, (uint32_t)(min(r, last_w) * wrow) + (lane & 7) * 16);
    }
  };

  f32x16 acc[4][4];  // [column block jc][token block it]
#pragma unroll
  for (int jc = 0; jc < 4; ++jc)
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[jc][it][j] = 0.f;

  // Fragment (row block b of the wave's half, k16 step s): row 32b + n of the
  // half -> block n, slot 4 half + b; 16-byte chunk 2s + hg.
  const int xoff = n * kBlk + hg * 16 + wt * 512;
  const int woff = n * kBlk + hg * 16 + wc * 512;
  const int nk = a.K / kBK;
  issue(0, 0);
  float* gk_lds = (float*)(smem + kGammaOff);
  double* w_lds = (double*)(smem + kFreqOff);
  if constexpr (EPI == kGemmQkv) {  // published by the loop's first barrier
    if (tid < 128) gk_lds[tid] = bf16_to_f32(a.k_gamma[tid]);
    else if (tid < 192) w_lds[tid - 128] = a.rope.w[tid - 128];
  }
  for (int kt = 0; kt < nk; ++kt) {
    // Only step kt's copies are outstanding here; once this thread's part has
    // landed, the barrier publishes everyone's part and frees the other stage.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
    const lds_u8* xs = lds + (kt & 1) * kStageBytes;
    const lds_u8* ws = xs + kTile;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      bf16x8 wf[4], xf[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        wf[b] = lds_load_b128(ws + woff + b * 128 + s * 32);
        xf[b] = lds_load_b128(xs + xoff + b * 128 + s * 32);
      }
#pragma unroll
      for (int jc = 0; jc < 4; ++jc)
#pragma unroll
        for (int it = 0; it < 4; ++it)
          acc[jc][it] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[jc], xf[it], acc[jc][it], 0, 0, 0);
    }
  }

  // ---- epilogue.  acc[jc][it][j]: token row0 + 128 wt + 32 it + n, column
  // col0 + 128 wc + 32 jc + 8 (j / 4) + 4 hg + j % 4.
  const int ccol = col0 + 128 * wc;  // the wave's first column (a head block in the qkv form)
  if (ccol >= a.N) return;
  if constexpr (EPI == kGemmPlain) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t tok = row0 + 128 * wt + 32 * it + n;
      if (tok >= a.M) continue;
      uint16_t* dst = a.y + tok * a.ldy + ccol + 4 * hg;
#pragma unroll
      for (int jc = 0; jc < 4; ++jc)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg)
          *reinterpret_cast<u32x2*>(dst + 32 * jc + 8 * jg) =
              u32x2{pack_bf16x2(acc[jc][it][4 * jg], acc[jc][it][4 * jg + 1]),
                    pack_bf16x2(acc[jc][it][4 * jg + 2], acc[jc][it][4 * jg + 3])};
    }
  } else {
    const int hh = ccol / 128;  // head block: query, key or value head
    const bool is_q = hh < a.Hq, is_k = !is_q && hh < a.Hq + a.Hkv;
    const int kv = is_k ? hh - a.Hq : hh - a.Hq - a.Hkv;
    // norm scale of column 32 jc + 8 (j / 4) + 4 hg + j % 4
    auto gk = [&](int jc, int j) __attribute__((always_inline)) { return gk_lds[32 * jc + 8 * (j >> 2) + 4 * hg + (j & 3)]; };
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t tok = row0 + 128 * wt + 32 * it + n;
      const bool valid = tok < a.M;
      float x[4][16];
#pragma unroll
      for (int jc = 0; jc < 4; ++jc)
#pragma unroll
        for (int j = 0; j < 16; ++j) x[jc][j] = acc[jc][it][j];
      uint16_t* dst;
      if (is_q) {
        dst = a.q_out + (tok * a.Hq + hh) * 128;
      } else {
        int s = 0, pos = 0;
        if (valid) token_position(a, tok, s, pos);
        if (is_k) {
          // QK-Norm from the fp32 accumulators; RMS is rotation-invariant, so
          // one inv serves both orders, which differ in whether the norm scale
          // applies before or after the rotation.
          float ss = 0.f;
#pragma unroll
          for (int jc = 0; jc < 4; ++jc)
#pragma unroll
            for (int j = 0; j < 16; ++j) ss += x[jc][j] * x[jc][j];
          ss = pair_sum(ss);
          const float inv = rsqrtf(ss * (1.0f / 128) + a.eps);
          if (a.order == 0)
#pragma unroll
            for (int jc = 0; jc < 4; ++jc)
#pragma unroll
              for (int j = 0; j < 16; ++j) x[jc][j] *= inv * gk(jc, j);
          // RoPE: columns d and d + 64 (blocks jc and jc + 2) turn by pos * w_d;
          // the angle is reduced in fp64 (whole turns removed exactly) and
          // evaluated by the hardware sine/cosine, which take turns.
#pragma unroll
          for (int jc = 0; jc < 2; ++jc)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const double wfreq = w_lds[32 * jc + 8 * (j >> 2) + 4 * hg + (j & 3)];
              const double t = (double)pos * (wfreq * 0.15915494309189535);
              const float r = (float)(t - rint(t));
              const float c = __builtin_amdgcn_cosf(r), sn = __builtin_amdgcn_sinf(r);
              const float y1 = x[jc][j], y2 = x[jc + 2][j];
              x[jc][j] = y1 * c - y2 * sn;
              x[jc + 2][j] = y2 * c + y1 * sn;
            }
          if (a.order != 0)
#pragma unroll
            for (int jc = 0; jc < 4; ++jc)
#pragma unroll
              for (int j = 0; j < 16; ++j) x[jc][j] *= inv * gk(jc, j);
        }
        uint16_t* cache = is_k ? a.k_cache : a.v_cache;
        if (cache)
          dst = cache + s * a.cs_seq + kv * a.cs_head + (int64_t)pos * a.cs_tok;
        else
          dst = (is_k ? a.k_out : a.v_out) + (tok * a.Hkv + kv) * 128;
      }
      if (!valid) continue;
      dst += 4 * hg;
#pragma unroll
      for (int jc = 0; jc < 4; ++jc)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg)
          *reinterpret_cast<u32x2*>(dst + 32 * jc + 8 * jg) =
              u32x2{pack_bf16x2(x[jc][4 * jg], x[jc][4 * jg + 1]), pack_bf16x2(x[jc][4 * jg + 2], x[jc][4 * jg + 3])};
    }
  }
}

template <int EPI>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)k_gemm<EPI>, hipFuncAttributeMaxDynamicSharedMemorySize, kSmemQkv);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
  hipLaunchKernelGGL(k_gemm<EPI>, dim3((unsigned)tiles), dim3(256), kSmemQkv, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int epilogue, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  return epilogue == kGemmQkv ? launch_t<kGemmQkv>(a, st) : launch_t<kGemmPlain>(a, st);
}

}  // namespace qw
