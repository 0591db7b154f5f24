// Causal grouped-query attention prefill, bf16 in / fp32 math, MFMA on gfx950.
//
// What it computes ("7.2 Qwen3 全规模实现" §7.2.1 GQA + QKNorm listing;
// "Transformer 20. Qwen 3 架构拆解" §2.2): for query head t of a packed sequence
// and its KV head u = floor(t / g), o_i = sum_j softmax_j(q_i . k_j / sqrt(128)) v_j
// over keys j <= i of the same sequence, with q already QK-normed and rotated
// (done here, in the prologue) and k read already normed and rotated (written by
// the norm+RoPE pass into the cache or the workspace).
//
// Work layout: a workgroup (4 waves) owns one KV head u of one sequence and a
// query tile of bm_tok tokens x g heads = up to 256 rows, so every K/V tile
// staged in LDS serves all g heads of the group.  Each wave holds 64 rows as two
// 32-row blocks, so every K or V fragment it reads from LDS feeds two MFMAs (the
// LDS pipe, not the bytes, limits the fragment reads on gfx950).
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// A = a K fragment from LDS, B = the wave's resident bf16 Q fragments.  In the
// 32x32 accumulator each lane then owns ONE query row (lane % 32) and 16 keys,
// so the softmax is lane-local plus one lane-pair exchange, and the
// probabilities, rounded to bf16, are directly the B operand of O^T = V^T P^T
// once the key order inside each 16-key slice is permuted the same way on the V
// side.  V stays row-major in LDS; its transposed A operand comes from gfx950's
// ds_read_b64_tr_b16 (two per fragment).
//
// K/V tiles of 64 keys go HBM -> LDS directly (global_load_lds_dwordx4, no
// staging registers) into a three-stage ring: tiles t+1 and t+2 land while tile
// t is used, tile t+2's copies issued during tile t's first MFMAs.
//
// Softmax: QK-Norm bounds every logit.  The query rows are pre-multiplied by
// c = scale * log2(e) before their bf16 rounding, so the MFMA scores are in
// log2 units, and |score| <= c * 128 * max|gamma_q| * max|gamma_k| (query rows
// have norm <= sqrt(128) max|gamma_q|, rotated keys <= sqrt(128) max|gamma_k|,
// RoPE keeps norms; a small margin covers the bf16 roundings).  When that bound
// is <= 60, the weights are p = 2^(score - B), B the bound rounded up to an
// integer: every p lies in [2^-120, 1], a normal float in fp32 and in bf16, so
// softmax needs no running maximum and no rescaling, and the tile pipelines at
// 32-key granularity.  The shift costs no instruction: the first score MFMA of
// a tile takes -B as its accumulator input instead of 0, and the exponential
// is taken of the accumulator itself.  With p <= 1 the PV accumulators have
// the range of the online form.  Otherwise the
// kernel runs the usual online softmax.  Both are exactly softmax; only
// rounding differs.  The row sum adds the bf16-rounded weights the PV MFMA
// uses, so every output row is an exact convex combination of V rows.  Tiles
// entirely above a wave's diagonal are skipped; only tiles crossing it are
// masked.
#include <type_traits>

#include "kernels.h"

namespace qw {
namespace {

constexpr int kTileKeys = 64;
constexpr float kStaticBoundMax = 60.f;             // log2 units

// LDS tile layout.  Row r of a 64-row tile lives in 1 KB block r % 16, slot
// r / 16 (256 B per slot); blocks are padded apart (K: 1040 B, V: 1088 B).
// A direct global->LDS load fills one whole block (lane l -> slot l / 16,
// 16-byte chunk l % 16).  Every fragment read is then one per-lane base plus
// compile-time offsets, and the rows read together land in distinct banks:
//  * K (b128 reads, 16 consecutive rows at one chunk): the 16 B block skew
//    spreads the 16 rows over all 16 chunk slots of a 256 B bank line;
//  * V (transposed b64 reads, 4 consecutive rows x 64 B per half-wave): the
//    64 B block skew puts the 4 rows in the 4 windows of a bank line.
constexpr int kKBlk = 1040, kVBlk = 1088;
constexpr int kKTile = 16 * kKBlk, kVTile = 16 * kVBlk;
constexpr int kStageBytes = kKTile + kVTile;
// Three-stage ring: tile t is read while tiles t+1 and t+2 are in flight.
constexpr int kStages = 3;
constexpr int kLoadsPerTile = 8;  // direct loads per lane per tile (4 K blocks, 4 V blocks)
constexpr int kPlanLdsTiles = 2047;  // plans up to this many tiles per sequence ...
constexpr int kPlanLdsSeqs = 2047;   // ... and sequences run entirely in LDS
constexpr int kRopeRow = kHalf + 2;  // float2 entries per row of the cos/sin table (16 B pad)
// Dynamic LDS: the K/V ring, or the prologue's cos/sin table if that is larger
// (bm_tok = 256 / g tokens; at most 256).
constexpr int kPrefillSmemMax = kPrefillRows * kRopeRow * 8 > kStages * kStageBytes ? kPrefillRows * kRopeRow * 8
                                                                                  : kStages * kStageBytes;
static_assert(kPrefillSmemMax <= 160 * 1024, "LDS per workgroup");
inline int prefill_smem_bytes(int bm_tok) { return bm_tok * kRopeRow * 8 > kStages * kStageBytes ? bm_tok * kRopeRow * 8 : kStages * kStageBytes; }

__device__ __forceinline__ bf16x8 lds_load_b128(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

// Direct HBM -> LDS copy of 16 bytes per lane: lane l's bytes, read from
// gbase + voff, land at LDS address lds_base + 16 l (M0 holds the wave-uniform
// base; one wait state after writing M0).  Written as inline assembly so the
// compiler does not put a wait for every outstanding copy in front of each LDS
// read: the tile loop waits for its own copies (s_waitcnt vmcnt) before the
// barrier that publishes a tile.
__device__ __forceinline__ void load_lds16_async(uint32_t lds_base, const void* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_base), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

__global__ __launch_bounds__(256, 1) void k_prefill_bf16(const PrefillItem* __restrict__ items, int hkv, PrefillArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // kStages x (K, V)
  lds_u8* lds = (lds_u8*)(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  // Consecutive workgroups take the KV heads of one work item, so each XCD
  // (workgroups are dealt round-robin over the 8 XCDs) keeps to its own heads
  // and their K/V stay in its L2.
  const int u = blockIdx.x % hkv;
  const PrefillItem item = items[blockIdx.x / hkv];
  const int s = item.s, qt = item.qt;
  const int seq0 = item.seq0;
  const int L = item.len;
  const int tok_base = qt * a.bm_tok;
  // Position of the sequence's first row: 0 for a prefill; for an append the
  // rows are new tokens at start_pos .., the keys are cache slots 0 .. and the
  // mask is rectangular.
  const int p0 = item.p0;
  if ((s < 0) | (s >= a.n_seq) | (qt < 0) | (tok_base >= L) | (p0 < 0)) return;
  const int n_kv = p0 + min(L, tok_base + a.bm_tok);

  // ---- this lane's two query rows (blocks qb = 0, 1 of the wave)
  const int n = lane & 31, hg = lane >> 5;
  int qpos[2], qtok[2], t_head[2];
  bool valid[2];
  int wave_min = 0x3fffffff, wave_max = -1;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = w * 64 + qb * 32 + n;
    const int hoff = r / a.bm_tok, toff = r - hoff * a.bm_tok;
    qtok[qb] = tok_base + toff;
    valid[qb] = hoff < a.g && qtok[qb] < L;
    qpos[qb] = valid[qb] ? p0 + qtok[qb] : 0x3fffffff;  // padding rows see every key
    t_head[qb] = u * a.g + hoff;
    wave_min = min(wave_min, qpos[qb]);
    wave_max = max(wave_max, valid[qb] ? p0 + qtok[qb] : -1);
  }
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) {
    wave_min = min(wave_min, __shfl_xor(wave_min, m, 64));
    wave_max = max(wave_max, __shfl_xor(wave_max, m, 64));
  }

  // ---- K/V sources for (sequence s, KV head u)
  const uint16_t* kbase = (const uint16_t*)a.khat + u * a.ks_head +
                          (a.k_packed ? (int64_t)seq0 * a.ks_tok : (int64_t)s * a.ks_seq);
  const uint16_t* vbase = (const uint16_t*)a.v + u * a.vs_head +
                          (a.v_packed ? (int64_t)seq0 * a.vs_tok : (int64_t)s * a.vs_seq);

  // Each wave fills blocks 4w .. 4w+3 of K and of V per tile.  A lane's byte
  // offset inside a tile is fixed; the tile base is uniform (scalar).  Keys
  // past n_kv (last tile only) repeat the last key: they are masked, and stay
  // finite.
  const int64_t kstride = a.ks_tok * 2, vstride = a.vs_tok * 2;  // bytes per key row
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int row = (w * 4 + m) + 16 * (lane >> 4);
    koff[m] = (uint32_t)(row * kstride) + (lane & 15) * 16;
    voff[m] = (uint32_t)(row * vstride) + (lane & 15) * 16;
  }
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  // TileCopy: one tile's copies for this lane (K blocks 4w .. 4w+3, then V),
  // addresses formed in advance so the static tile can issue them one at a
  // time between its MFMAs.
  struct TileCopy {
    uint32_t kdst, vdst;
    const char *ksrc, *vsrc;
    uint32_t off[kLoadsPerTile];
  };
  auto tile_copy = [&](int t, int stage) __attribute__((always_inline)) {
    TileCopy c;
    c.kdst = lds0 + stage * kStageBytes + wu * 4 * kKBlk;
    c.vdst = lds0 + stage * kStageBytes + kKTile + wu * 4 * kVBlk;
    c.ksrc = (const char*)kbase + (int64_t)t * kTileKeys * kstride;
    c.vsrc = (const char*)vbase + (int64_t)t * kTileKeys * vstride;
    const bool tail = (t + 1) * kTileKeys > n_kv;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      c.off[m] = koff[m];
      c.off[4 + m] = voff[m];
      if (tail) {
        const int r = min(w * 4 + m + 16 * (lane >> 4), n_kv - 1 - t * kTileKeys);
        c.off[m] = (uint32_t)(r * kstride) + (lane & 15) * 16;
        c.off[4 + m] = (uint32_t)(r * vstride) + (lane & 15) * 16;
      }
    }
    return c;
  };
  // copy i (0 .. 7): K block 4w + i (i < 4), then V block 4w + i - 4
  auto issue_copy = [&](const TileCopy& c, int i) __attribute__((always_inline)) {
    if (i < 4) load_lds16_async(c.kdst + i * kKBlk, c.ksrc, c.off[i]);
    else load_lds16_async(c.vdst + (i - 4) * kVBlk, c.vsrc, c.off[i]);
  };
  auto issue_tile = [&](int t, int stage) __attribute__((always_inline)) {
    const TileCopy c = tile_copy(t, stage);
#pragma unroll
    for (int i = 0; i < kLoadsPerTile; ++i) issue_copy(c, i);
  };
  const int n_tiles = (n_kv + kTileKeys - 1) / kTileKeys;

  // ---- prologue: QK-Norm + RoPE of each query row, kept as bf16 MFMA fragments.
  // Lane (n, hg) holds dims 16kk + 8hg + e (kk < 8, e < 8); dims i and i + 64 of
  // a rotation pair sit in fragments kk and kk + 4 of the same lane.
  bf16x8 qf[2][8];
  // The launch-wide logit bound (decided once by the plan kernel) picks the
  // softmax form.
  const bool use_static = a.static_flag[0] != 0;
  // Static-bound form: each tile's score accumulators start at -B (B the
  // launch's logit bound, an integer), so its weights come out as 2^(score - B).
  f32x16 neg_bound;
  {
    const float nb = __int_as_float(a.static_flag[1]);
#pragma unroll
    for (int j = 0; j < 16; ++j) neg_bound[j] = nb;
  }
  const float c_log2 = a.scale_log2e;
  // QK-Norm + RoPE of one query row, times c = scale * log2(e) (so the MFMA
  // scores come out in log2 units), into bf16 fragments.  Called once per query
  // block with static arguments, so the fragment arrays stay in registers.
  // cos/sin of the workgroup's bm_tok positions (tok_base ..) at the 64 RoPE
  // angles, tabulated once in LDS (the K/V stages are not in use yet) and
  // shared by the g heads of each token.  Rows are padded by 16 bytes so the
  // 16 lanes of a b128 read pass hit distinct banks.
  // When the table fits in one ring stage (g >= 4) it goes to stage 2, which
  // the first tile copies do not touch: tiles 0 and 1 and the query rows are
  // then already in flight while the table is computed.  (Stage 2 first
  // receives tile 2, after the loop's first barrier.)
  const bool early = a.bm_tok * kRopeRow * 8 <= kStageBytes;
  float2* const rope_t = (float2*)(smem + (early ? 2 * kStageBytes : 0));
  u32x4 qraw[2][8];  // raw bf16 query rows: dims 16kk + 8hg .. +7
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const uint16_t* src = (const uint16_t*)a.q + ((int64_t)(seq0 + (valid[qb] ? qtok[qb] : 0)) * a.Hq +
                                                  (valid[qb] ? t_head[qb] : 0)) * kD + 8 * hg;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qraw[qb][kk] = *reinterpret_cast<const u32x4*>(src + 16 * kk);
  }
  u32x4 graw[8];  // gamma_q at the same dims
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) graw[kk] = *reinterpret_cast<const u32x4*>((const uint16_t*)a.q_gamma + 8 * hg + 16 * kk);
  if (early) {
    issue_tile(0, 0);
    if (n_tiles > 1) issue_tile(1, 1);
  }
  // The angle is reduced in fp64 (whole turns removed exactly) and evaluated
  // by the hardware sine/cosine, which take turns: errors near 1e-6, far below
  // the bf16 rounding of the fragments they feed.  Wave w fills angles
  // 16w .. 16w+15 for every token (lane = token), so the angle index is uniform
  // and its frequency comes through a scalar load: no vector-memory wait, which
  // would also wait for the query rows and tiles issued above, precedes it.
  {
    constexpr int kPerWave = kHalf / 4;
    for (int t0 = 0; t0 < a.bm_tok; t0 += 64) {
      const int t = t0 + lane;
      const double pos = (double)(p0 + tok_base + t);
#pragma unroll
      for (int k = 0; k < kPerWave; ++k) {
        const int i = wu * kPerWave + k;
        const double turns = a.rope.w[i] * 0.15915494309189535;  // w / (2 pi)
        const double x = pos * turns;
        const float r = (float)(x - rint(x));  // in [-1/2, 1/2] turn
        if (t < a.bm_tok) rope_t[t * kRopeRow + i] = make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
      }
    }
  }
  __syncthreads();
  auto row_prologue = [&](bool ok, int tok, const u32x4 (&raw)[8], bf16x8 (&frag)[8]) __attribute__((always_inline)) {
    float x[8][8];
    if (ok) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[kk][2 * e] = bf16_lo(raw[kk][e]);
          x[kk][2 * e + 1] = bf16_hi(raw[kk][e]);
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
    // RMS is rotation-invariant, so one inv serves both orders; they differ in
    // whether gamma scales the dims before the rotation (norm first, order 0)
    // or after it (RoPE first, order 1).
    auto scale = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[kk][2 * e] *= inv * bf16_lo(graw[kk][e]);
          x[kk][2 * e + 1] *= inv * bf16_hi(graw[kk][e]);
        }
      }
    };
    if (a.order == 0) scale();
    const float2* cs = rope_t + (ok ? tok - tok_base : 0) * kRopeRow + 8 * hg;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 v = cs[16 * kk + e];
        const float y1 = x[kk][e], y2 = x[kk + 4][e];
        x[kk][e] = y1 * v.x - y2 * v.y;
        x[kk + 4][e] = y2 * v.x + y1 * v.y;
      }
    }
    if (a.order != 0) scale();
    // The fragments are only ever MFMA B operands, which gfx950 reads from
    // AGPRs directly: writing them there keeps the 64 registers out of the
    // VGPR file that the tile loop fills with scores, weights and O.
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t v = pack_bf16x2(x[kk][2 * e] * c_log2, x[kk][2 * e + 1] * c_log2);
        asm("v_accvgpr_write_b32 %0, %1" : "=a"(w4[e]) : "v"(v));
      }
      frag[kk] = __builtin_bit_cast(bf16x8, w4);
    }
  };
  row_prologue(valid[0], qtok[0], qraw[0], qf[0]);
  __builtin_amdgcn_sched_barrier(0);
  row_prologue(valid[1], qtok[1], qraw[1], qf[1]);
  if (!early) {
    __syncthreads();  // every wave is done with the table before tiles land on it
    issue_tile(0, 0);
    if (n_tiles > 1) issue_tile(1, 1);
  }


  f32x16 o[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[qb][db][j] = 0.f;
  float m_run[2] = {-1e30f, -1e30f}, l_run[2] = {0.f, 0.f};

  // Per-lane LDS bases of the fragment reads (everything else is an immediate).
  // K: row 32kb + n, chunk 2kk + hg.  V (transposed): row 16kk + v_row0 (+8),
  // dims 32db + v_col0 .. +3.
  const int G = lane >> 4, lam = lane & 15;
  const int v_row0 = 4 * (G >> 1) + (lam >> 2);
  const int v_col0 = 16 * (G & 1) + 4 * (lam & 3);
  const int k_base = (n & 15) * kKBlk + (n >> 4) * 256 + hg * 16;
  const int v_base = v_row0 * kVBlk + v_col0 * 2;


  // One tile with the online softmax (running max, rescaled accumulators):
  // S^T = K Q^T, softmax in place on the accumulators, O^T += V^T P^T.
  auto tile = [&](const lds_u8* ks, const lds_u8* vs, int key0) __attribute__((always_inline)) {
    f32x16 sacc[2][2];  // [key block kb][query block qb]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[kb][qb][j] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ka = lds_load_b128(ks + k_base + kb * 512 + kk * 32);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qb][kk], sacc[kb][qb], 0, 0, 0);
      }
    }
    // sacc[kb][qb][j] is key key0 + 32kb + 8(j/4) + 4hg + j%4 of row (qb, n)
    const bool diag = key0 + kTileKeys - 1 > wave_min;
    bf16x8 pf[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (diag) {  // key0 + 32kb + 8(j/4) + 4hg + j%4 > qpos  <=>  constant > lim
        const int lim = qpos[qb] - key0 - 4 * hg;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (32 * kb + 8 * (j >> 2) + (j & 3) > lim) sacc[kb][qb][j] = -INFINITY;
      }
      float m_use;
      {
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sacc[kb][qb][j]);
        mt = pair_max(mt);
        const float m_new = fmaxf(m_run[qb], mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) o[qb][db][j] *= alpha;
        m_use = m_new;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          sacc[kb][qb][j] = __builtin_amdgcn_exp2f(sacc[kb][qb][j] - m_use);
      // P^T fragments: slice kk (16 keys) = registers 8(kk%2) .. +7 of block kk/2.
      // The row sum adds the bf16-rounded weights the MFMA uses, so every output
      // row is an exact convex combination of V rows.
      float psum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 w4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w4[e] = pack_bf16x2(sacc[kk >> 1][qb][8 * (kk & 1) + 2 * e], sacc[kk >> 1][qb][8 * (kk & 1) + 2 * e + 1]);
          psum = sum_bf16x2(w4[e], psum);
        }
        pf[qb][kk] = __builtin_bit_cast(bf16x8, w4);
      }
      l_run[qb] += psum;
    }
    // O^T += V^T P^T; each V fragment (two transposed reads) feeds both query blocks
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const lds_u8* vp = vs + v_base + kk * 256 + db * 64;
        const bf16x8 va = concat_tr16(lds_read_tr16(vp), lds_read_tr16(vp + 8 * kVBlk));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[qb][kk], o[qb][db], 0, 0, 0);
      }
    }
  };

  // Static-bound tile, software-pipelined at 32-key granularity and issued in
  // a fixed order.  With the bound there is no row maximum, so the weights of
  // keys 0..31 are formed while the S MFMAs of keys 32..63 run, and those of
  // keys 32..63 while the PV MFMAs of keys 0..31 run:
  //   S(keys 0-31) | S(keys 32-63) + exp(0-31) | PV(0-31) + exp(32-63) | PV(32-63)
  // One wave per SIMD issues in order, so the order is the schedule: every MFMA
  // is followed by a quarter of one weight group (two keys) for the VALU to
  // run under it, and every step issues the LDS fragment read that is needed
  // three steps later.  sched_barrier keeps the compiler from regrouping them.
  auto static_tile = [&](const lds_u8* ks, const lds_u8* vs, int key0, auto diag_tag, const TileCopy& next) __attribute__((always_inline)) {
    constexpr bool kDiag = decltype(diag_tag)::value;
    f32x16 sacc[2][2];  // [key block kb][query block qb]
    bf16x8 pf[2][4];    // [qb][16-key slice kk]
    u32x4 w4[2][2][2];  // [kb][qb][h]: weights being packed into pf[qb][2kb + h]
    float psum[2] = {0.f, 0.f};
    bf16x8 kf[16];      // K fragment (kb, kk) at 8kb + kk
    bf16x8 vf[16];      // V fragment (kk, db) at 4kk + db
    auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
    auto kread = [&](int i) __attribute__((always_inline)) {
      kf[i] = lds_load_b128(ks + k_base + (i >> 3) * 512 + (i & 7) * 32);
    };
    auto vread = [&](int i) __attribute__((always_inline)) {
      const lds_u8* vp = vs + v_base + (i >> 2) * 256 + (i & 3) * 64;
      vf[i] = concat_tr16(lds_read_tr16(vp), lds_read_tr16(vp + 8 * kVBlk));
    };
    auto smfma = [&](int kb, int kk, int qb) __attribute__((always_inline)) {
      sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[8 * kb + kk], qf[qb][kk],
                                                             kk == 0 ? neg_bound : sacc[kb][qb], 0, 0, 0);
    };
    auto pmfma = [&](int i, int qb) __attribute__((always_inline)) {
      o[qb][i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf[qb][i >> 2], o[qb][i & 3], 0, 0, 0);
    };
    // Weight pair m (0..15) of key block kb: query block m / 8, registers
    // j = 2(m % 8), +1 of sacc[kb][qb], i.e. keys key0 + 32kb + 8(j/4) + 4hg + j%4.
    auto weights = [&](int kb, int m) __attribute__((always_inline)) {
      const int qb = m >> 3, j = 2 * (m & 7), h = j >> 3, e = (j & 7) >> 1;
      float x0 = sacc[kb][qb][j], x1 = sacc[kb][qb][j + 1];
      if constexpr (kDiag) {  // key > qpos  <=>  constant > lim
        const int lim = qpos[qb] - key0 - 4 * hg - 32 * kb;
        if (8 * (j >> 2) + (j & 3) > lim) x0 = -INFINITY;
        if (8 * ((j + 1) >> 2) + ((j + 1) & 3) > lim) x1 = -INFINITY;
      }
      w4[kb][qb][h][e] = pack_bf16x2(__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1));
      psum[qb] = sum_bf16x2(w4[kb][qb][h][e], psum[qb]);
      if (e == 3) pf[qb][2 * kb + h] = __builtin_bit_cast(bf16x8, w4[kb][qb][h]);
    };

    kread(0);
    kread(1);
    kread(2);
    fence();
    // S(keys 0-31); the reads run ahead into the K fragments of keys 32-63
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      smfma(0, kk, 0);
      smfma(0, kk, 1);
      kread(kk + 3);
      issue_copy(next, kk);  // tile t+2's copies, one per two MFMAs
      fence();
    }
    // S(keys 32-63) + weights of keys 0-31; then the first V fragments
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      smfma(1, kk, 0);
      weights(0, 2 * kk);
      fence();
      smfma(1, kk, 1);
      weights(0, 2 * kk + 1);
      if (kk < 5)
        kread(8 + kk + 3);
      else
        vread(kk - 5);
      fence();
    }
    // PV(keys 0-31) + weights of keys 32-63
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pmfma(i, 0);
      weights(1, 2 * i);
      fence();
      pmfma(i, 1);
      weights(1, 2 * i + 1);
      vread(i + 3);
      fence();
    }
    // PV(keys 32-63)
#pragma unroll
    for (int i = 8; i < 16; ++i) {
      pmfma(i, 0);
      pmfma(i, 1);
      if (i + 3 < 16) vread(i + 3);
      fence();
    }
    l_run[0] += psum[0];
    l_run[1] += psum[1];
  };

  auto run = [&](auto static_tag) __attribute__((always_inline)) {
    constexpr bool kStatic = decltype(static_tag)::value;
    int stage = 0;
    for (int t = 0; t < n_tiles; ++t, stage = stage == kStages - 1 ? 0 : stage + 1) {
      // This thread's part of tile t is in LDS once at most tile t+1's copies
      // are outstanding; the barrier then publishes everyone's part and frees
      // the stage of tile t-1, which receives tile t+2.
      static_assert(kLoadsPerTile == 8, "vmcnt immediate below");
      if (t + 1 < n_tiles)
        __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      const int next = stage == 0 ? 2 : stage - 1;  // the stage tile t+2 goes to
      const int key0 = t * kTileKeys;
      const lds_u8* ks = lds + stage * kStageBytes;
      if (kStatic && key0 <= wave_max) {
        // The static tile issues tile t+2's copies one per two MFMAs of its
        // first phase rather than in a burst here.  Past the last tile it
        // copies the last tile again into the free stage (in bounds, never
        // read), so the tile has no branch.
        const TileCopy nc = tile_copy(min(t + 2, n_tiles - 1), next);
        if (key0 + kTileKeys - 1 > wave_min)
          static_tile(ks, ks + kKTile, key0, std::true_type{}, nc);
        else
          static_tile(ks, ks + kKTile, key0, std::false_type{}, nc);
        continue;
      }
      if (t + 2 < n_tiles) issue_tile(t + 2, next);
      if (key0 > wave_max) continue;        // every key of the tile is in this wave's future
      if constexpr (!kStatic) tile(ks, ks + kKTile, key0);
    }
  };
  if (use_static)
    run(std::true_type{});
  else
    run(std::false_type{});
  // the repeat copies issued during the last tiles land before the ring is reused
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---- epilogue: O^T block db, register j = dim 32db + 8(j/4) + 4hg + j%4 of
  // row (qb, n).  The normalised rows are staged in LDS (the ring is free once
  // every wave is past its last tile; no copy is in flight then) and leave as
  // whole rows: 16 lanes x 16 B per row, and the g heads of a token, adjacent
  // in out, go out together.  Stored straight from the accumulators, every
  // store instruction touched 32 rows 2*Hq*128 bytes apart.
  constexpr int kORow = 2 * kD + 16;  // bytes per staged row (16 B pad)
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float inv_l = 1.0f / pair_sum(l_run[qb]);
    lds_u8* orow = lds + (w * 64 + qb * 32 + n) * kORow;  // row r = hoff * bm_tok + toff
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = 32 * db + 8 * jg + 4 * hg;
        u32x2 pk = {pack_bf16x2(o[qb][db][4 * jg] * inv_l, o[qb][db][4 * jg + 1] * inv_l),
                    pack_bf16x2(o[qb][db][4 * jg + 2] * inv_l, o[qb][db][4 * jg + 3] * inv_l)};
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(orow + 2 * d) = pk;
      }
  }
  __syncthreads();
  const int n_chunks = a.bm_tok * a.g * (kD / 8);  // 16-byte chunks, ordered (token, head, chunk)
  // row / g by one multiply: (row + 1/2) / g lies at least 1/(2g) >= 2^-9 from
  // an integer and the float error is below 2^-15 for row < 256.
  const float inv_g = 1.0f / (float)a.g;
#pragma unroll 4
  for (int c = tid; c < n_chunks; c += 256) {
    const int row = c >> 4, part = c & 15;
    const int toff = (int)(((float)row + 0.5f) * inv_g), hoff = row - toff * a.g;
    if (tok_base + toff < L) {
      const u32x4 v =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(lds + (hoff * a.bm_tok + toff) * kORow + 16 * part);
      uint16_t* dst = (uint16_t*)a.out + ((int64_t)(seq0 + tok_base + toff) * a.Hq + u * a.g + hoff) * kD + 8 * part;
      *reinterpret_cast<u32x4*>(dst) = v;
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
  __shared__ int tmp[16];
  // Small plans (the usual case) keep every array in LDS; larger ones use the
  // caller's scratch.
  __shared__ int32_t lds_arr[4 * (kPlanLdsTiles + 1) + 2 * (kPlanLdsSeqs + 1)];
  const int tid = threadIdx.x;
  const int nb = a.max_tiles + 1;
  const bool small = a.max_tiles <= kPlanLdsTiles && a.n_seq <= kPlanLdsSeqs;
  int32_t* hist = small ? lds_arr : a.scratch;
  int32_t* cnt_gt = hist + nb;
  int32_t* off = cnt_gt + nb;
  int32_t* tie = off + nb;
  int32_t* rank = tie + nb;
  int32_t* cu = small ? rank + a.n_seq : nullptr;  // staged offsets (small plans)
  if (small)
    for (int i = tid; i <= a.n_seq; i += 1024) cu[i] = a.cu[i];
  for (int i = tid; i < nb; i += 1024) { hist[i] = 0; tie[i] = 0; }
  __syncthreads();
  auto cu_at = [&](int i) { return small ? cu[i] : a.cu[i]; };
  auto n_tiles_of = [&](int s) {
    const int L = max(0, cu_at(s + 1) - cu_at(s));
    return min(a.max_tiles, (L + a.bm_tok - 1) / a.bm_tok);
  };
  for (int s = tid; s < a.n_seq; s += 1024) atomicAdd(&hist[n_tiles_of(s)], 1);
  __syncthreads();
  // two suffix sums, 1024 entries at a time from the top (thread order runs
  // from high to low index, so a prefix scan over threads is a suffix sum):
  //   cnt_gt[q] = sum_{n > q} hist[n];  off[q] = sum_{q' > q} cnt_gt[q']
  for (int pass = 0; pass < 2; ++pass) {
    const int32_t* in = pass == 0 ? hist : cnt_gt;
    int32_t* outp = pass == 0 ? cnt_gt : off;
    int carry = 0;
    for (int base = ((nb - 1) / 1024) * 1024; base >= 0; base -= 1024) {
      const int i = base + 1023 - tid;
      const int v = i < nb ? in[i] : 0;
      int total;
      const int ex = block_exclusive_scan(v, tmp, &total);
      if (i < nb) outp[i] = carry + ex;
      carry += total;
    }
    __syncthreads();
  }
  for (int s = tid; s < a.n_seq; s += 1024) {
    const int nt = n_tiles_of(s);
    rank[s] = cnt_gt[nt] + atomicAdd(&tie[nt], 1);
  }
  __syncthreads();
  if (tid >= 960 && a.static_flag) {
    // (the last wave, while the others write the list) the largest norm scale
    // |gamma_offset + gamma| of q and of k.  Every rotated query row has norm
    // <= sqrt(d) times the q maximum and every rotated key <= sqrt(d) times the
    // k maximum (the normed row has RMS 1 and RoPE keeps norms), so with the
    // query rows pre-scaled by c = scale * log2(e), |score| <= c * d * max_q *
    // max_k, plus a margin for the bf16 roundings.  Within 60 (log2 units)
    // every p = 2^score is a normal float, and the prefill runs its
    // static-bound softmax.
    const int l = tid - 960;
    const uint16_t* gk = (const uint16_t*)a.k_gamma;
    const uint16_t* gq = (const uint16_t*)a.q_gamma;
    float kmax = 0.f, qmax = 0.f;
    for (int i = l; i < a.head_dim; i += 64) {
      kmax = fmaxf(kmax, fabsf(a.gamma_offset + bf16_to_f32(gk[i])));
      qmax = fmaxf(qmax, fabsf(a.gamma_offset + bf16_to_f32(gq[i])));
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      kmax = fmaxf(kmax, __shfl_xor(kmax, m, 64));
      qmax = fmaxf(qmax, __shfl_xor(qmax, m, 64));
    }
    if (l == 0) {
      const float bound = a.scale_log2e * (float)a.head_dim * qmax * kmax * (1.0f + 1.0f / 64);
      const bool ok = bound <= kStaticBoundMax;
      // the weights are 2^(score - B), B = the bound rounded up: in [2^-120, 1]
      a.static_flag[0] = ok;
      a.static_flag[1] = __float_as_int(ok ? -ceilf(bound) : 0.f);
    }
  }
  for (int s = 0; s < a.n_seq; ++s) {
    const int nt = n_tiles_of(s);
    const int rk = rank[s];
    const int seq0 = cu_at(s), len = cu_at(s + 1) - seq0;
    const int p0 = a.start_pos ? a.start_pos[s] : 0;
    for (int q = tid; q < nt; q += 1024) {
      const int pos = off[q] + rk;
      if (pos < a.n_items) {
        PrefillItem it;
        it.s = s; it.qt = q; it.seq0 = seq0; it.len = len; it.p0 = p0;
        it.pad0 = it.pad1 = it.pad2 = 0;
        a.items[pos] = it;
      }
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
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)k_prefill_bf16, hipFuncAttributeMaxDynamicSharedMemorySize, kPrefillSmemMax);
  if (attr != hipSuccess) return attr;
  const int64_t blocks = (int64_t)n_items * a.Hkv;
  hipLaunchKernelGGL(k_prefill_bf16, dim3((unsigned)blocks), dim3(256), prefill_smem_bytes(a.bm_tok), st,
                     (const PrefillItem*)a.items, a.Hkv, a);
  return hipGetLastError();
}

}  // namespace qw
