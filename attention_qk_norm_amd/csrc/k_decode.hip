// Split-K decode over a bf16 KV cache (HBM-bound), head_dim 128 or 256.
//
// One new query token per sequence attends to the cache slots 0 .. start_pos[i]
// of its KV head, the new key having been normed, rotated at start_pos and
// appended by the prologue ("第 20 章 Qwen3 与 Qwen3.5" §20.3: only the new K is
// rotated; cached keys already carry their rotation).  The key axis of every
// (sequence, KV head) is cut into chunks; a workgroup streams one chunk, its four
// waves taking interleaved 32-key blocks, and leaves a partial (m, l,
// acc[head_dim]) per query head.  A second kernel merges the partials with the exact softmax
// identity o = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c.
//
// Per 32-key block a wave computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16
// (A = K rows loaded straight from HBM as 16-byte fragments, B = the g <= 16
// query heads of the group, resident), so each lane owns one head column and
// the softmax is lane-local plus two lane swaps.  The probabilities, rounded to
// bf16, are the B operand of O^T = V^T P^T; V goes HBM -> the wave's own LDS
// slot directly (no staging registers) and comes back transposed through
// ds_read_b64_tr_b16.
// Every K and V byte is read once, in 16-byte lane loads.  The gated layers
// ("第 20 章 Qwen3 与 Qwen3.5" §20.4) multiply the merged output by sigmoid of
// the gate in the merge kernel.
#include "kernels.h"

namespace qw {
namespace {

constexpr int kBlockKeys = 32;

// V block in LDS: 32 rows x 2D bytes.  The transposed reads of one half-wave
// touch 8 rows x 32 bytes; XOR-ing the 16-byte chunk with (row & 7) << 1 spreads
// those 8 rows over the 8 32-byte windows of a 256-byte bank line.
template <int D>
__device__ __forceinline__ int v_swz(int row, int chunk) {
  return row * (2 * D) + ((chunk ^ ((row & 7) << 1)) << 4);
}

// Dynamic LDS: the four waves' V blocks, later reused for the merge.
template <int D>
constexpr int decode_smem_bytes() {
  return 4 * kBlockKeys * 2 * D + 4 * 2 * 16 * 4;
}

// Direct HBM -> LDS copy of 16 bytes per lane (lane l's bytes land at
// lds_base + 16 l; M0 holds the wave-uniform base, one wait state after
// writing it).  Inline assembly, so the compiler does not wait for every
// outstanding copy before each LDS read; the loop waits for its own copies.
__device__ __forceinline__ void load_lds16_async(uint32_t lds_base, const void* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(lds_base), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

template <int D>
__global__ __launch_bounds__(256) void k_decode_split(DecodeArgs a) {
  constexpr int KF = D / 32;  // K / Q fragments per 16 x 32-dim slice row
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int u = blockIdx.x % a.Hkv;
  const int cg = blockIdx.x / a.Hkv;
  const int i = a.chunk_seq[cg];  // chunk_off[i] <= cg < chunk_off[i + 1]
  if (i < 0 || i >= a.n_seq) return;
  const int n_keys = a.start_pos[i] + 1;
  const int kbeg = (cg - a.chunk_off[i]) * a.chunk;
  const int kend = min(n_keys, kbeg + a.chunk);

  const int hh = lane & 15, q4 = lane >> 4;  // head column, lane group
  const bool hvalid = hh < a.g;

  // query fragments: B[k = dim 32kk + 8q4 + e][n = head hh]
  bf16x8 qf[KF];
  {
    const uint16_t* src = a.qhat + ((int64_t)i * a.Hq + u * a.g + (hvalid ? hh : 0)) * D + 8 * q4;
#pragma unroll
    for (int kk = 0; kk < KF; ++kk) {
      u32x4 raw = hvalid ? *reinterpret_cast<const u32x4*>(src + 32 * kk) : u32x4{0, 0, 0, 0};
      qf[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const uint16_t* kb = a.k_cache + (int64_t)i * a.cs_seq + u * a.cs_head;
  const uint16_t* vb = a.v_cache + (int64_t)i * a.cs_seq + u * a.cs_head;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // w is wave-uniform: keep it (and b0) in SGPRs
  lds_u8* vs = (lds_u8*)(smem) + wu * kBlockKeys * 2 * D;
  const uint32_t vs_lds = (uint32_t)(uintptr_t)vs;

  f32x4 o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;

  // transposed-read coordinates: group q4 reads rows 4 q4 + (lam >> 2) (+16)
  const int lam = lane & 15;
  const int v_row = 4 * q4 + (lam >> 2);
  const int v_col = 4 * (lam & 3);  // + 16 db, elements

  for (int b0 = kbeg + wu * kBlockKeys; b0 < kend; b0 += 4 * kBlockKeys) {
    // V rows of the block go HBM -> this wave's LDS slot directly, in the
    // swizzled layout: copy m fills LDS bytes 1024 m + 16 lane, i.e. row r,
    // chunk position cp, which holds global chunk cp ^ ((r & 7) << 1).  Keys
    // past kend repeat the last key (masked below, and finite).  Issued first:
    // the K loads after them complete later, so the wait the compiler puts in
    // front of the score MFMAs also covers these copies.
    {
      constexpr int CPR = D / 8;  // 16-byte chunks per row
      const char* vblk = (const char*)(vb + (int64_t)b0 * a.cs_tok);
      const int last = kend - 1 - b0;
#pragma unroll
      for (int m = 0; m < D / 16; ++m) {
        const int o = 1024 * m + 16 * lane;
        const int r = o / (2 * D), cp = (o % (2 * D)) / 16;
        const int c = cp ^ ((r & 7) << 1);
        load_lds16_async(vs_lds + 1024 * m, vblk, (uint32_t)(min(r, last) * a.cs_tok * 2) + c * 16);
      }
      static_assert(CPR * 16 == 2 * D, "row bytes");
    }
    // K fragments: A[m = key b0 + 16 sb + hh][k = dim 32kk + 8 q4 + e]
    u32x4 kr[2][KF];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int key = b0 + 16 * sb + hh;
#pragma unroll
      for (int kk = 0; kk < KF; ++kk)
        kr[sb][kk] = key < kend ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                      kb + (int64_t)key * a.cs_tok + 32 * kk + 8 * q4))
                                : u32x4{0, 0, 0, 0};
    }
    f32x4 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      sacc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KF; ++kk)
        sacc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[sb][kk]), qf[kk],
                                                          sacc[sb], 0, 0, 0);
    }
    // this wave's V copies have landed (only this wave reads its slot)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // softmax over the block: sacc[sb][j] = key b0 + 16sb + 4q4 + j of head hh
    float sv[8];
    float mt = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = b0 + 16 * sb + 4 * q4 + j;
        const float x = key < kend ? sacc[sb][j] * a.scale_log2e : -INFINITY;
        sv[4 * sb + j] = x;
        mt = fmaxf(mt, x);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    // The row sum adds the bf16-rounded weights the PV MFMA uses: numerator and
    // denominator sum the same weights.
    float psum = 0.f;
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pf[e] = (__bf16)__builtin_amdgcn_exp2f(sv[e] - m_new);  // virtual key 8 q4 + e
      psum += (float)pf[e];
    }
    l_run = l_run * alpha + psum;

    // O^T[d][head] += V^T[d][keys] P^T[keys][head]
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int col = 16 * db + v_col;
      const int off = (col & 7) * 2;
      const bf16x8 va = concat_tr16(lds_read_tr16(vs + v_swz<D>(v_row, col >> 3) + off),
                                    lds_read_tr16(vs + v_swz<D>(v_row + 16, col >> 3) + off));
#pragma unroll
      for (int j = 0; j < 4; ++j) o[db][j] *= alpha;
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, o[db], 0, 0, 0);
    }
  }

  // ---- merge the four waves: m is uniform over a head's lane groups; l is not
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();
  float* ob = reinterpret_cast<float*>(smem);           // [4 waves][16 heads][D]
  float* ml = ob + 4 * 16 * D;                           // [4 waves][2][16]
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) ob[(w * 16 + hh) * D + 16 * db + 4 * q4 + j] = o[db][j];
  if (q4 == 0) {
    ml[(w * 2 + 0) * 16 + hh] = m_run;
    ml[(w * 2 + 1) * 16 + hh] = l_run;
  }
  __syncthreads();
  for (int e = tid; e < a.g * D; e += 256) {
    const int h = e / D, d = e % D;
    float M = -1e30f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, ml[(ww * 2) * 16 + h]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = __builtin_amdgcn_exp2f(ml[(ww * 2) * 16 + h] - M);
      acc += f * ob[(ww * 16 + h) * D + d];
      lsum += f * ml[(ww * 2 + 1) * 16 + h];
    }
    float* dst = a.partial + ((int64_t)cg * a.Hq + u * a.g + h) * (D + 4);
    dst[d] = acc;
    if (d == 0) {
      dst[D] = M;
      dst[D + 1] = lsum;
    }
  }
}

// One wave per (sequence, query head): merge its chunks' partials.  The lanes
// first take the chunks' maxima in parallel; the weighted sum then walks the
// chunks with four loads in flight, each lane owning D/64 of the dims.
template <int D>
__global__ __launch_bounds__(64) void k_decode_combine(DecodeArgs a) {
  constexpr int N = D / 64;
  const int i = blockIdx.x / a.Hq, t = blockIdx.x % a.Hq;
  const int lane = threadIdx.x;
  const int c0 = a.chunk_off[i], c1 = a.chunk_off[i + 1];
  const float* base = a.partial + t * (D + 4);
  const int64_t cstride = (int64_t)a.Hq * (D + 4);
  float M = -1e30f;
  for (int c = c0 + lane; c < c1; c += 64) M = fmaxf(M, base[c * cstride + D]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  float acc[N], lsum = 0.f;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int c = c0; c < c1; ++c) {
    const float* p = base + c * cstride;
    const float f = __builtin_amdgcn_exp2f(p[D] - M);
    lsum += f * p[D + 1];
#pragma unroll
    for (int e = 0; e < N; ++e) acc[e] += f * p[N * lane + e];
  }
  const float inv = 1.0f / lsum;
  float y[N];
#pragma unroll
  for (int e = 0; e < N; ++e) y[e] = acc[e] * inv;
  if (a.gate) {  // gated layers: times sigmoid(gate) at the same dims
    const uint16_t* gp = a.gate + ((int64_t)i * a.Hq + t) * a.q_row + N * lane;
#pragma unroll
    for (int e = 0; e < N; ++e) y[e] /= 1.0f + __expf(-bf16_to_f32(gp[e]));
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(a.out + ((int64_t)i * a.Hq + t) * D + N * lane);
#pragma unroll
  for (int e = 0; e < N / 2; ++e) dst[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
}

// chunk_off[i] = sum_{i' < i} ceil((start_pos[i'] + 1) / chunk); one workgroup.
__global__ __launch_bounds__(1024) void k_decode_plan(const int32_t* start_pos, int n_seq, int chunk, int max_chunks,
                                                      int32_t* chunk_off, int32_t* chunk_seq) {
  __shared__ int tmp[16];
  int carry = 0;
  for (int base = 0; base < n_seq; base += 1024) {
    const int i = base + threadIdx.x;
    const int v = i < n_seq ? (start_pos[i] + chunk) / chunk : 0;
    int total;
    const int ex = block_exclusive_scan(v, tmp, &total);
    if (i < n_seq) {
      chunk_off[i] = carry + ex;
      // the sequence of every chunk, so a split workgroup needs no search
      // (clamped to what the host sized, so a device/host mismatch cannot
      // write out of bounds)
      for (int c = carry + ex; c < min(carry + ex + v, max_chunks); ++c) chunk_seq[c] = i;
    }
    carry += total;
  }
  if (threadIdx.x == 0) chunk_off[n_seq] = carry;
  for (int c = carry + threadIdx.x; c < max_chunks; c += 1024) chunk_seq[c] = -1;  // no sequence
}

}  // namespace

hipError_t launch_decode_plan(const int32_t* start_pos, int n_seq, int chunk, int max_chunks, int32_t* chunk_off,
                              int32_t* chunk_seq, hipStream_t st) {
  hipLaunchKernelGGL(k_decode_plan, dim3(1), dim3(1024), 0, st, start_pos, n_seq, chunk, max_chunks, chunk_off,
                     chunk_seq);
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs& a, int total_chunks, hipStream_t st) {
  if (total_chunks <= 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)total_chunks * a.Hkv));
  if (a.head_dim == kMaxD) {
    static const hipError_t attr = hipFuncSetAttribute((const void*)k_decode_split<kMaxD>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       decode_smem_bytes<kMaxD>());
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_decode_split<kMaxD>, grid, dim3(256), decode_smem_bytes<kMaxD>(), st, a);
  } else {
    hipLaunchKernelGGL(k_decode_split<kD>, grid, dim3(256), decode_smem_bytes<kD>(), st, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t st) {
  if (a.n_seq <= 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)a.n_seq * a.Hq));
  if (a.head_dim == kMaxD)
    hipLaunchKernelGGL(k_decode_combine<kMaxD>, grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(k_decode_combine<kD>, grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace qw
