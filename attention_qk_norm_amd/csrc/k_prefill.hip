// Causal grouped-query attention prefill, bf16 in / fp32 math, MFMA on gfx950.
//
// What it computes ("7.2 Qwen3 全规模实现" §7.2.1 GQA + QKNorm listing;
// "Transformer 20. Qwen 3 架构拆解" §2.2): for query head t of a packed sequence
// and its KV head u = floor(t / g), o_i = sum_j softmax_j(q_i . k_j / sqrt(128)) v_j
// over keys j <= i of the same sequence, with q already QK-normed and rotated
// (done here, in the prologue) and k read already normed and rotated (written by
// the norm+RoPE pass into the cache or the workspace).
//
// Layout of the work: a workgroup (4 waves) owns one KV head u of one sequence
// and a query tile of bm_tok tokens x g heads = up to 128 rows, so every K/V
// tile staged in LDS serves all g heads of the group.  Each wave holds 32 rows.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// A = a K fragment from LDS, B = the wave's resident bf16 Q fragments.  In the
// 32x32 accumulator each lane then owns ONE query row (lane % 32) and 16 keys,
// so the softmax max and sum are lane-local plus one lane-half swap, and the
// accumulator, rounded to bf16, is directly the B operand of O^T = V^T P^T once
// the key order inside each 16-key slice is permuted consistently on the V side.
// V stays row-major in LDS; its transposed A operand comes from gfx950's
// ds_read_b64_tr_b16 (two per fragment).  Online softmax in fp32 with exp2 and
// log2(e) folded into the scale; tiles entirely above the diagonal are never
// visited, and only tiles crossing it are masked.
#include "kernels.h"

namespace qw {
namespace {

constexpr int kTileKeys = 64;
constexpr int kRowBytes = kD * 2;  // one bf16 row in LDS


__device__ __forceinline__ bf16x8 lds_load_b128(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

// Byte offset of (row, 16-byte chunk) in a K tile: chunk ^ (row & 15) makes the
// 32 rows of one MFMA fragment read hit 16 distinct chunk slots per 16 lanes.
__device__ __forceinline__ int k_swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 15)) << 4);
}
// V tile: the transposed reads touch 8 consecutive rows x 64 bytes; XOR-ing the
// chunk with (row & 3) << 2 puts the 4 rows of each half-wave in different
// 64-byte bank windows.
__device__ __forceinline__ int v_swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row & 3) << 2)) << 4);
}

__global__ __launch_bounds__(256, 1) void k_prefill_bf16(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kTileKeys * kRowBytes];
  lds_u8* ks = (lds_u8*)(smem);
  lds_u8* vs = ks + kTileKeys * kRowBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int u = blockIdx.x % a.Hkv;
  const int2 item = a.items[blockIdx.x / a.Hkv];
  const int s = item.x, qt = item.y;
  if (s < 0 || s >= a.n_seq) return;
  const int seq0 = a.cu[s];
  const int L = a.cu[s + 1] - seq0;
  const int tok_base = qt * a.bm_tok;
  if (qt < 0 || tok_base >= L) return;
  const int n_kv = min(L, tok_base + a.bm_tok);

  // ---- this lane's query row
  const int n = lane & 31, hg = lane >> 5;
  const int r = w * 32 + n;
  const int hoff = r / a.bm_tok, toff = r - hoff * a.bm_tok;
  const int qtok = tok_base + toff;
  const bool valid = hoff < a.g && qtok < L;
  const int qpos = valid ? qtok : 0x3fffffff;  // padding rows see every key
  const int t_head = u * a.g + hoff;
  int wave_min = qpos;
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) wave_min = min(wave_min, __shfl_xor(wave_min, m, 64));

  // ---- prologue: QK-Norm + RoPE of the query row, kept as bf16 MFMA fragments.
  // Lane (n, hg) holds dims 16kk + 8hg + e (kk < 8, e < 8); dims i and i + 64 of
  // a rotation pair sit in fragments kk and kk + 4 of the same lane.
  bf16x8 qf[8];
  {
    float x[8][8];
    if (valid) {
      const uint16_t* src = (const uint16_t*)a.q + ((int64_t)(seq0 + qtok) * a.Hq + t_head) * kD + 8 * hg;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        u32x4 raw = *reinterpret_cast<const u32x4*>(src + 16 * kk);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[kk][2 * e] = bf16_lo(raw[e]);
          x[kk][2 * e + 1] = bf16_hi(raw[e]);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[kk][e] = 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[kk][e] * x[kk][e];
    ss = pair_sum(ss);  // lane l ^ 32 holds the other half of the row
    const float inv = rsqrtf(ss * (1.0f / kD) + a.eps);
    const uint16_t* gsrc = (const uint16_t*)a.q_gamma + 8 * hg;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 gr = *reinterpret_cast<const u32x4*>(gsrc + 16 * kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[kk][2 * e] *= inv * bf16_lo(gr[e]);
        x[kk][2 * e + 1] *= inv * bf16_hi(gr[e]);
      }
    }
    const int p = valid ? qtok : 0;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float c, sn;
        rope_cos_sin(p, a.rope.w[16 * kk + 8 * hg + e], c, sn);
        const float y1 = x[kk][e], y2 = x[kk + 4][e];
        x[kk][e] = y1 * c - y2 * sn;
        x[kk + 4][e] = y2 * c + y1 * sn;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)x[kk][e];
  }

  // ---- K/V sources for (sequence s, KV head u)
  const uint16_t* kbase = (const uint16_t*)a.khat + u * a.ks_head +
                          (a.k_packed ? (int64_t)seq0 * a.ks_tok : (int64_t)s * a.ks_seq);
  const uint16_t* vbase = (const uint16_t*)a.v + u * a.vs_head +
                          (a.v_packed ? (int64_t)seq0 * a.vs_tok : (int64_t)s * a.vs_seq);

  // Each thread stages 4 of the 1024 16-byte chunks of a 64-key K tile and of V.
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int c = tid + 256 * m;
      const int row = c >> 4, col = c & 15;
      const int key = t * kTileKeys + row;
      if (key < n_kv) {
        kreg[m] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * a.ks_tok + col * 8);
        vreg[m] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * a.vs_tok + col * 8);
      } else {
        kreg[m] = u32x4{0, 0, 0, 0};
        vreg[m] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int c = tid + 256 * m;
      const int row = c >> 4, col = c & 15;
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(ks + k_swz(row, col)) = kreg[m];
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(vs + v_swz(row, col)) = vreg[m];
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  // transposed-read coordinates of this lane inside a V tile (see the header)
  const int G = lane >> 4, lam = lane & 15;
  const int v_row0 = 4 * (G >> 1) + (lam >> 2);    // + 16 kk (+ 8 for the upper half)
  const int v_col0 = 16 * (G & 1) + 4 * (lam & 3);  // + 32 db, in elements

  const int n_tiles = (n_kv + kTileKeys - 1) / kTileKeys;
  load_tile(0);
  for (int t = 0; t < n_tiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(t + 1);

    // S^T = K Q^T for the tile's two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.f;
      const int krow = 32 * kb + n;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 ka = lds_load_b128(ks + k_swz(krow, 2 * kk + hg));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], sacc[kb], 0, 0, 0);
      }
    }

    // online softmax; sacc[kb][j] is key 64t + 32kb + 8(j/4) + 4hg + j%4 of row n
    const int key0 = t * kTileKeys;
    const bool diag = key0 + kTileKeys - 1 > wave_min;
    float sv[32];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = sacc[kb][j] * a.scale_log2e;
        if (diag) {
          const int key = key0 + 32 * kb + 8 * (j >> 2) + 4 * hg + (j & 3);
          if (key > qpos) x = -INFINITY;
        }
        sv[kb * 16 + j] = x;
        mt = fmaxf(mt, x);
      }
    mt = pair_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float pv = __builtin_amdgcn_exp2f(sv[i] - m_new);
      sv[i] = pv;
      psum += pv;
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[db][j] *= alpha;

    // P^T fragments: slice kk (16 keys) = registers 8(kk%2) .. +7 of block kk/2
    bf16x8 pf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i) pf[kk][i] = (__bf16)sv[(kk >> 1) * 16 + 8 * (kk & 1) + i];

    // O^T += V^T P^T; the A operand (V^T rows d, keys in the permuted slice order)
    // comes from two transposed 8-byte LDS reads per fragment.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int row = 16 * kk + v_row0;
        const int col = 32 * db + v_col0;
        const int off = (col & 7) * 2;
        const bf16x8 va = concat_tr16(lds_read_tr16(vs + v_swz(row, col >> 3) + off),
                                      lds_read_tr16(vs + v_swz(row + 8, col >> 3) + off));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kk], o[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O^T block db, register j = dim 32db + 8(j/4) + 4hg + j%4 of row n
  const float l_tot = pair_sum(l_run);
  const float inv_l = 1.0f / l_tot;
  if (valid) {
    uint16_t* dst = (uint16_t*)a.out + ((int64_t)(seq0 + qtok) * a.Hq + t_head) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = 32 * db + 8 * jg + 4 * hg;
        u32x2 pk = {pack_bf16x2(o[db][4 * jg] * inv_l, o[db][4 * jg + 1] * inv_l),
                    pack_bf16x2(o[db][4 * jg + 2] * inv_l, o[db][4 * jg + 3] * inv_l)};
        *reinterpret_cast<u32x2*>(dst + d) = pk;
      }
  }
}

// Work list, heaviest tiles first.  Tiles are ordered by query-tile index
// descending (the cost of tile qt is min(L, (qt+1) bm_tok) keys), and within
// one index by sequence length descending.  With nt_s = ceil(L_s / bm_tok):
//   cnt_gt[q] = #{s : nt_s > q},  off[q] = sum_{q' > q} cnt_gt[q'],
//   rank_s    = cnt_gt[nt_s] + (arrival order among equal nt_s),
// and tile (s, qt) lands at off[qt] + rank_s -- a bijection onto 0..n_items-1
// (the order among equal lengths varies from run to run; the results do not).
// One workgroup of 1024 threads; scratch holds 4 (max_tiles + 1) + n_seq ints.
// Lengths are clamped to what the host sized, so a device/host mismatch cannot
// write out of bounds.
__global__ __launch_bounds__(1024) void k_prefill_plan(PlanArgs a) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int nb = a.max_tiles + 1;
  int32_t* hist = a.scratch;
  int32_t* cnt_gt = hist + nb;
  int32_t* off = cnt_gt + nb;
  int32_t* tie = off + nb;
  int32_t* rank = tie + nb;
  auto n_tiles_of = [&](int s) {
    const int L = max(0, a.cu[s + 1] - a.cu[s]);
    return min(a.max_tiles, (L + a.bm_tok - 1) / a.bm_tok);
  };
  for (int i = tid; i < nb; i += 1024) { hist[i] = 0; tie[i] = 0; }
  __syncthreads();
  for (int s = tid; s < a.n_seq; s += 1024) atomicAdd(&hist[n_tiles_of(s)], 1);
  __syncthreads();
  // two suffix sums: cnt_gt[q] = sum_{n > q} hist[n]; off[q] = sum_{q' > q} cnt_gt[q']
  const int per = (nb + 1023) / 1024;
  for (int pass = 0; pass < 2; ++pass) {
    const int32_t* in = pass == 0 ? hist : cnt_gt;
    int32_t* outp = pass == 0 ? cnt_gt : off;
    const int lo = min(nb, tid * per), hi = min(nb, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += in[i];
    part[tid] = sum;
    __syncthreads();
    if (tid == 0) {  // exclusive suffix over the 1024 partial sums
      int acc = 0;
      for (int i = 1023; i >= 0; --i) { const int v = part[i]; part[i] = acc; acc += v; }
    }
    __syncthreads();
    int acc = part[tid];
    for (int i = hi - 1; i >= lo; --i) { outp[i] = acc; acc += in[i]; }
    __syncthreads();
  }
  for (int s = tid; s < a.n_seq; s += 1024) {
    const int nt = n_tiles_of(s);
    rank[s] = cnt_gt[nt] + atomicAdd(&tie[nt], 1);
  }
  __syncthreads();
  for (int s = 0; s < a.n_seq; ++s) {
    const int nt = n_tiles_of(s);
    const int rk = rank[s];
    for (int q = tid; q < nt; q += 1024) {
      const int pos = off[q] + rk;
      if (pos < a.n_items) a.items[pos] = make_int2(s, q);
    }
  }
}

}  // namespace

hipError_t launch_prefill_plan(const PlanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_prefill_plan, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, int n_items, hipStream_t st) {
  if (n_items <= 0) return hipSuccess;
  const int64_t blocks = (int64_t)n_items * a.Hkv;
  hipLaunchKernelGGL(k_prefill_bf16, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace qw
