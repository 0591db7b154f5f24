// Causal grouped-query attention prefill at head_dim 256 (the gated global
// layers of Qwen3-Next / Qwen3.5), bf16 in / fp32 math, MFMA on gfx950.
//
// What it computes ("14. Qwen 家族：从 QKV 偏置到混合注意力", section on
// Qwen3-Next; "第 20 章 Qwen3 与 Qwen3.5" §20.4): for query head t and its KV head
// u = floor(t / g), o_i = sigmoid(gate_i) * sum_j softmax_j(q_i . k_j / sqrt(256)) v_j
// over keys j <= i of the same sequence.  q is normed with the scale
// norm_offset + gamma (1 + w for the zero-centred norm) and rotated on its first
// `rot` coordinates only (pairs (i, i + rot/2), frequency theta^(-2i/rot)); this
// happens here, in the prologue.  k arrives normed and rotated the same way (the
// norm+RoPE pass wrote it to the cache or the workspace).  Without a gate the
// output is the plain attention.
//
// Work layout: a workgroup (4 waves, one per SIMD) owns one KV head u of one
// sequence and a query tile of bm_tok tokens x g heads = up to 128 rows; every
// K/V tile staged in LDS serves all g heads of the group.  Each wave holds one
// 32-row block.  At head_dim 256 a wave's O accumulators (32 rows x 256 dims)
// and resident Q fragments fill the register file that two 32-row blocks use at
// head_dim 128, so every LDS fragment read feeds one MFMA here.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
// (A = a K fragment from LDS, B = the wave's resident bf16 Q fragments): each
// lane owns one query row (lane % 32) and 16 keys of every 32-key block, so the
// softmax is lane-local plus one lane-pair exchange, and the probabilities,
// rounded to bf16, are directly the B operand of O^T = V^T P^T once the key
// order inside each 16-key slice is permuted the same way on the V side (V^T
// fragments come from gfx950's transposed LDS read, ds_read_b64_tr_b16).
//
// K/V tiles of 64 keys (32 KB each) go HBM -> LDS directly
// (global_load_lds_dwordx4) into a two-stage ring: tile t+1 lands while tile t
// is used, its copies issued one per two score MFMAs of tile t.
//
// Softmax: as in the head_dim-128 kernel, the query rows are pre-multiplied by
// c = scale * log2(e); when the launch-wide bound c * 256 * max|scale_q| *
// max|scale_k| (plus a rounding margin) is <= 60, p = 2^(score - B), B that
// bound rounded up, lies in [2^-120, 1] and needs no running maximum (the
// static-bound form, decided by the plan kernel; the first score MFMA of a
// tile starts its accumulator at -B); otherwise the online softmax runs.  The row sum adds the bf16-rounded weights that the PV MFMA uses.
#include <type_traits>

#include "kernels.h"

namespace qw {
namespace {

constexpr int kW = 256;          // head_dim
constexpr int kTileKeys = 64;
// LDS tile layout: row r of a 64-row tile (512 bytes) lives in 1 KB block
// r % 32, slot r / 32; blocks are padded apart (K: 1040 B, V: 1088 B).  A direct
// global->LDS load fills one whole block (lane l -> slot l / 32, 16-byte chunk
// l % 32).  Consecutive rows then sit in consecutive blocks, so
//  * K (b128 reads, 16 consecutive rows at one chunk): the 16 B block skew
//    spreads the 16 rows over the 16 chunk slots of a 256 B bank line;
//  * V (transposed b64 reads, 4 consecutive rows x 64 B per half-wave): the
//    64 B skew puts the 4 rows in the 4 windows of a bank line.
constexpr int kBlocks = 32;
constexpr int kKBlk = 1040, kVBlk = 1088;
constexpr int kKTile = kBlocks * kKBlk, kVTile = kBlocks * kVBlk;
constexpr int kStageBytes = kKTile + kVTile;
constexpr int kStages = 2;
constexpr int kSmem = kStages * kStageBytes;
static_assert(kSmem <= 160 * 1024, "LDS per workgroup");
constexpr int kBlocksPerWave = kBlocks / 4;  // per tensor and tile
constexpr float kStaticBoundMax = 60.f;      // log2 units

__device__ __forceinline__ bf16x8 lds_load_b128(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

// Direct HBM -> LDS copy of 16 bytes per lane (lane l's bytes land at
// lds_base + 16 l; M0 holds the wave-uniform base, one wait state after writing
// it).  Inline assembly, so the compiler does not put a wait for every
// outstanding copy in front of each LDS read: the tile loop waits for its own
// copies (s_waitcnt vmcnt(0)) before the barrier that publishes a tile.
__device__ __forceinline__ void load_lds16_async(uint32_t lds_base, const void* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_base), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

// QK-Norm and partial RoPE of the lane's half query row (dims 16kk + 8hg + e,
// kk < 16, e < 8), times c, into bf16 MFMA B fragments (AGPRs).  Dims i and
// i + ROT/2 of a rotation pair sit in fragments kk and kk + ROT/32 of the same
// lane; fragments from ROT/16 on pass unrotated.
template <int ROT>
__device__ __forceinline__ void q_prologue(const PrefillArgs& a, const u32x4 (&raw)[16], const u32x4 (&graw)[16],
                                           bool ok, int pos, int hg, bf16x8 (&frag)[16]) {
  constexpr int RH = ROT / 32;
  float x[16][8];
#pragma unroll
  for (int kk = 0; kk < 16; ++kk)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[kk][2 * e] = ok ? bf16_lo(raw[kk][e]) : 0.f;
      x[kk][2 * e + 1] = ok ? bf16_hi(raw[kk][e]) : 0.f;
    }
  float ss = 0.f;
#pragma unroll
  for (int kk = 0; kk < 16; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[kk][e] * x[kk][e];
  ss = pair_sum(ss);  // lane l ^ 32 holds the other half of the row
  const float inv = rsqrtf(ss * (1.0f / kW) + a.eps);
  auto scale = [&](int kk) __attribute__((always_inline)) {
    const u32x4 gr = graw[kk];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[kk][2 * e] *= inv * (a.gamma_offset + bf16_lo(gr[e]));
      x[kk][2 * e + 1] *= inv * (a.gamma_offset + bf16_hi(gr[e]));
    }
  };
  // RMS is rotation-invariant, so one inv serves both orders; they differ in
  // whether the norm scale applies before the rotation (order 0) or after it.
  if (a.order == 0)
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) scale(kk);
  // The angle p * w_i is reduced in fp64 (whole turns removed exactly) and
  // evaluated by the hardware sine/cosine, which take turns.
  const double turn = 0.15915494309189535;  // 1 / (2 pi)
#pragma unroll
  for (int kk = 0; kk < RH; ++kk) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i0 = 16 * kk + e;  // angle index of hg = 0; hg = 1 adds 8
      const double w = hg ? a.rope.w[i0 + 8] : a.rope.w[i0];
      const double t = (double)pos * (w * turn);
      const float r = (float)(t - rint(t));
      const float c = __builtin_amdgcn_cosf(r), s = __builtin_amdgcn_sinf(r);
      const float y1 = x[kk][e], y2 = x[kk + RH][e];
      x[kk][e] = y1 * c - y2 * s;
      x[kk + RH][e] = y2 * c + y1 * s;
    }
  }
  if (a.order != 0)
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) scale(kk);
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    u32x4 w4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t v = pack_bf16x2(x[kk][2 * e] * a.scale_log2e, x[kk][2 * e + 1] * a.scale_log2e);
      asm("v_accvgpr_write_b32 %0, %1" : "=a"(w4[e]) : "v"(v));
    }
    frag[kk] = __builtin_bit_cast(bf16x8, w4);
  }
}

__global__ __launch_bounds__(256, 1) void k_prefill_wide(const PrefillItem* __restrict__ items, int hkv, PrefillArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // kStages x (K, V)
  lds_u8* lds = (lds_u8*)(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  // Consecutive workgroups take the KV heads of one work item (the XCD
  // round-robin then keeps each XCD on its own heads' K/V in its L2).
  const int u = blockIdx.x % hkv;
  const PrefillItem item = items[blockIdx.x / hkv];
  const int s = item.s, qt = item.qt, seq0 = item.seq0, L = item.len, p0 = item.p0;
  const int tok_base = qt * a.bm_tok;
  if ((s < 0) | (s >= a.n_seq) | (qt < 0) | (tok_base >= L) | (p0 < 0)) return;
  const int n_kv = p0 + min(L, tok_base + a.bm_tok);

  // ---- this lane's query row
  const int n = lane & 31, hg = lane >> 5;
  const int r = w * 32 + n;
  const int hoff = r / a.bm_tok, toff = r - hoff * a.bm_tok;
  const int qtok = tok_base + toff;
  const bool valid = hoff < a.g && qtok < L;
  const int qpos = valid ? p0 + qtok : 0x3fffffff;  // padding rows see every key
  const int t_head = u * a.g + hoff;
  int wave_min = qpos, wave_max = valid ? qpos : -1;
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
  const int64_t kstride = a.ks_tok * 2, vstride = a.vs_tok * 2;  // bytes per key row
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  // Wave w fills blocks 8w .. 8w+7 of K and of V.  Keys past n_kv (last tile
  // only) repeat the last key: they are masked, and stay finite.
  // TileCopy: one tile's copies for this lane, addresses formed in advance so
  // the static tile can issue them one at a time between its MFMAs.
  struct TileCopy {
    uint32_t kdst, vdst;
    const char *ksrc, *vsrc;
    uint32_t ko[kBlocksPerWave], vo[kBlocksPerWave];
  };
  auto tile_copy = [&](int t, int stage) __attribute__((always_inline)) {
    TileCopy c;
    c.kdst = lds0 + stage * kStageBytes + wu * kBlocksPerWave * kKBlk;
    c.vdst = lds0 + stage * kStageBytes + kKTile + wu * kBlocksPerWave * kVBlk;
    c.ksrc = (const char*)kbase + (int64_t)t * kTileKeys * kstride;
    c.vsrc = (const char*)vbase + (int64_t)t * kTileKeys * vstride;
    const int last = n_kv - 1 - t * kTileKeys;  // last valid row of the tile
#pragma unroll
    for (int m = 0; m < kBlocksPerWave; ++m) {
      const int row = min(wu * kBlocksPerWave + m + 32 * (lane >> 5), last);
      c.ko[m] = (uint32_t)(row * kstride) + (lane & 31) * 16;
      c.vo[m] = (uint32_t)(row * vstride) + (lane & 31) * 16;
    }
    return c;
  };
  // copy i (0 .. 15) of a tile: K block 8w + i/2 (i even), V block 8w + i/2 (i odd)
  auto issue_copy = [&](const TileCopy& c, int i) __attribute__((always_inline)) {
    const int m = i >> 1;
    if (i & 1) load_lds16_async(c.vdst + m * kVBlk, c.vsrc, c.vo[m]);
    else load_lds16_async(c.kdst + m * kKBlk, c.ksrc, c.ko[m]);
  };
  auto issue_tile = [&](int t, int stage) __attribute__((always_inline)) {
    const TileCopy c = tile_copy(t, stage);
#pragma unroll
    for (int i = 0; i < 2 * kBlocksPerWave; ++i) issue_copy(c, i);
  };
  const int n_tiles = (n_kv + kTileKeys - 1) / kTileKeys;

  // ---- prologue: raw query row (16-byte loads), first tile, then norm + RoPE
  u32x4 qraw[16];
  {
    const int64_t row = (int64_t)(seq0 + (valid ? qtok : 0)) * a.Hq + (valid ? t_head : 0);
    const uint16_t* src = (const uint16_t*)a.q + row * a.q_row + 8 * hg;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qraw[kk] = *reinterpret_cast<const u32x4*>(src + 16 * kk);
  }
  u32x4 graw[16];  // the norm weights at the same dims, requested with the rows
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) graw[kk] = *reinterpret_cast<const u32x4*>((const uint16_t*)a.q_gamma + 8 * hg + 16 * kk);
  issue_tile(0, 0);
  bf16x8 qf[16];
  const int qp = valid ? qpos : 0;
  switch (a.rot) {
    case 32: q_prologue<32>(a, qraw, graw, valid, qp, hg, qf); break;
    case 64: q_prologue<64>(a, qraw, graw, valid, qp, hg, qf); break;
    case 128: q_prologue<128>(a, qraw, graw, valid, qp, hg, qf); break;
    default: q_prologue<256>(a, qraw, graw, valid, qp, hg, qf); break;
  }
  const bool use_static = a.static_flag[0] != 0;
  // Static-bound form: each tile's score accumulators start at -B (B the
  // launch's logit bound, an integer), so its weights come out as 2^(score - B).
  f32x16 neg_bound;
  {
    const float nb = __int_as_float(a.static_flag[1]);
#pragma unroll
    for (int j = 0; j < 16; ++j) neg_bound[j] = nb;
  }

  f32x16 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  // Per-lane LDS bases of the fragment reads (everything else is an immediate).
  // K fragment (kb, kk): key 32kb + n -> block n, slot kb; dims 16kk + 8hg.
  // V fragment (kk, db), transposed: keys 16kk + v_row0 (+8), dims 32db + v_col0 .. +3.
  const int G = lane >> 4, lam = lane & 15;
  const int v_row0 = 4 * (G >> 1) + (lam >> 2);
  const int v_col0 = 16 * (G & 1) + 4 * (lam & 3);
  const int k_base = n * kKBlk + hg * 16;
  const int v_base = v_row0 * kVBlk + v_col0 * 2;

  // One 64-key tile: S^T = K Q^T (keys 0-31, then 32-63, so the weights of the
  // first half can form while the second half's MFMAs run), the softmax in
  // place, O^T += V^T P^T.
  auto tile = [&](const lds_u8* ks, const lds_u8* vs, int key0, auto static_tag, auto diag_tag)
                  __attribute__((always_inline)) {
    constexpr bool kStatic = decltype(static_tag)::value;
    constexpr bool kDiag = decltype(diag_tag)::value;
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = kStatic ? neg_bound : f32x16{};
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const bf16x8 ka = lds_load_b128(ks + k_base + kb * 512 + kk * 32);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], sacc[kb], 0, 0, 0);
      }
    }
    // sacc[kb][j] is key key0 + 32kb + 8(j/4) + 4hg + j%4 of row n
    if constexpr (kDiag) {
      const int lim = qpos - key0 - 4 * hg;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (32 * kb + 8 * (j >> 2) + (j & 3) > lim) sacc[kb][j] = -INFINITY;
    }
    float m_use = 0.f;
    if constexpr (!kStatic) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sacc[kb][j]);
      mt = pair_max(mt);
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
      m_use = m_new;
    }
    // P^T fragments: slice kk (16 keys) = registers 8(kk%2) .. +7 of block kk/2.
    bf16x8 pf[4];
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = sacc[kk >> 1][8 * (kk & 1) + 2 * e], x1 = sacc[kk >> 1][8 * (kk & 1) + 2 * e + 1];
        w4[e] = kStatic ? pack_bf16x2(__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1))
                        : pack_bf16x2(__builtin_amdgcn_exp2f(x0 - m_use), __builtin_amdgcn_exp2f(x1 - m_use));
        psum = sum_bf16x2(w4[e], psum);
      }
      pf[kk] = __builtin_bit_cast(bf16x8, w4);
    }
    l_run += psum;
    // O^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const lds_u8* vp = vs + v_base + 16 * (kk & 1) * kVBlk + (kk >> 1) * 512 + db * 64;
        const bf16x8 va = concat_tr16(lds_read_tr16(vp), lds_read_tr16(vp + 8 * kVBlk));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kk], o[db], 0, 0, 0);
      }
    }
  };

  // Static-bound tile in a fixed issue order (the weights need no row
  // maximum, so they can form while MFMAs run):
  //   S(keys 0-31) | S(keys 32-63) + weights(0-31) | PV(0-31) + weights(32-63) | PV(32-63)
  // With one wave per SIMD the issue order is the schedule: every MFMA is
  // followed by the LDS fragment read needed kLead MFMAs later and, in the
  // middle phases, by half a weight pair; sched_barrier keeps the compiler
  // from regrouping them.
  constexpr int kLead = 6;
  auto static_tile = [&](const lds_u8* ks, const lds_u8* vs, int key0, auto diag_tag, const TileCopy& next) __attribute__((always_inline)) {
    constexpr bool kDiag = decltype(diag_tag)::value;
    f32x16 sacc[2];
    bf16x8 pf[4];
    u32x4 w4[2][2];
    float psum = 0.f;
    bf16x8 kf[32];  // K fragment (kb, kk) at 16 kb + kk
    bf16x8 vf[32];  // V fragment (kk, db) at 8 kk + db
    auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
    auto kread = [&](int i) __attribute__((always_inline)) {
      kf[i] = lds_load_b128(ks + k_base + (i >> 4) * 512 + (i & 15) * 32);
    };
    auto vread = [&](int i) __attribute__((always_inline)) {
      const int kk = i >> 3, db = i & 7;
      const lds_u8* vp = vs + v_base + 16 * (kk & 1) * kVBlk + (kk >> 1) * 512 + db * 64;
      vf[i] = concat_tr16(lds_read_tr16(vp), lds_read_tr16(vp + 8 * kVBlk));
    };
    // fragment read r of the tile's stream: K fragments 0..31, then V 0..31
    auto fread = [&](int r) __attribute__((always_inline)) {
      if (r < 32) kread(r);
      else if (r < 64) vread(r - 32);
    };
    auto smfma = [&](int kb, int kk) __attribute__((always_inline)) {
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[16 * kb + kk], qf[kk], kk == 0 ? neg_bound : sacc[kb], 0, 0, 0);
    };
    auto pmfma = [&](int i) __attribute__((always_inline)) {
      o[i & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf[i >> 3], o[i & 7], 0, 0, 0);
    };
    // Weight pair m (0..7) of key block kb: registers j = 2m, 2m+1 of sacc[kb],
    // keys key0 + 32kb + 8(j/4) + 4hg + j%4; slice 2kb + j/8 of P^T.
    auto weights = [&](int kb, int m) __attribute__((always_inline)) {
      const int j = 2 * m, h = j >> 3, e = (j & 7) >> 1;
      float x0 = sacc[kb][j], x1 = sacc[kb][j + 1];
      if constexpr (kDiag) {  // key > qpos  <=>  constant > lim
        const int lim = qpos - key0 - 4 * hg - 32 * kb;
        if (8 * (j >> 2) + (j & 3) > lim) x0 = -INFINITY;
        if (8 * ((j + 1) >> 2) + ((j + 1) & 3) > lim) x1 = -INFINITY;
      }
      w4[kb][h][e] = pack_bf16x2(__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1));
      psum = sum_bf16x2(w4[kb][h][e], psum);
      if (e == 3) pf[2 * kb + h] = __builtin_bit_cast(bf16x8, w4[kb][h]);
    };
#pragma unroll
    for (int r = 0; r < kLead; ++r) fread(r);
    fence();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {  // S(keys 0-31)
      smfma(0, kk);
      fread(kk + kLead);
      if (kk & 1) issue_copy(next, kk >> 1);
      fence();
    }
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {  // S(keys 32-63) + weights of keys 0-31
      smfma(1, kk);
      if (kk & 1) weights(0, kk >> 1);
      fread(16 + kk + kLead);
      if (kk & 1) issue_copy(next, 8 + (kk >> 1));
      fence();
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // PV(keys 0-31) + weights of keys 32-63
      pmfma(i);
      if (i & 1) weights(1, i >> 1);
      fread(32 + i + kLead);
      fence();
    }
#pragma unroll
    for (int i = 16; i < 32; ++i) {  // PV(keys 32-63)
      pmfma(i);
      fread(32 + i + kLead);
      fence();
    }
    l_run += psum;
  };

  auto run = [&](auto static_tag) __attribute__((always_inline)) {
    for (int t = 0; t < n_tiles; ++t) {
      // Only tile t's copies are outstanding here; once this thread's part
      // has landed, the barrier publishes everyone's part and frees the stage
      // of tile t-1, which receives tile t+1.
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      const int key0 = t * kTileKeys;
      const lds_u8* ks = lds + (t & 1) * kStageBytes;
      constexpr bool kStatic = decltype(static_tag)::value;
      if (kStatic && key0 <= wave_max) {
        // The static tile issues tile t+1's 16 copies one per two score MFMAs
        // over its first half rather than in a burst here: a burst fills the
        // copy queue and stalls the in-order issue of the first MFMAs.  Past
        // the last tile it copies the last tile again into the free stage (in
        // bounds, never read), so the tile has no branch.
        const TileCopy next = tile_copy(min(t + 1, n_tiles - 1), (t + 1) & 1);
        if (key0 + kTileKeys - 1 > wave_min)
          static_tile(ks, ks + kKTile, key0, std::true_type{}, next);
        else
          static_tile(ks, ks + kKTile, key0, std::false_type{}, next);
        continue;
      }
      if (t + 1 < n_tiles) issue_tile(t + 1, (t + 1) & 1);
      if (key0 > wave_max) continue;  // every key of the tile is in this wave's future
      if constexpr (!kStatic) {
        if (key0 + kTileKeys - 1 > wave_min)
          tile(ks, ks + kKTile, key0, static_tag, std::true_type{});
        else
          tile(ks, ks + kKTile, key0, static_tag, std::false_type{});
      }
    }
  };
  if (use_static)
    run(std::true_type{});
  else
    run(std::false_type{});
  // the repeat copies issued during the last tile land before the ring is reused
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---- epilogue: O^T block db, register j = dim 32db + 8(j/4) + 4hg + j%4 of
  // row n.  The normalised rows are staged in LDS as fp32 (the ring is free
  // once every wave is past its last tile; no copy is in flight then) and leave
  // as whole rows, 16 B per lane, the g heads of a token together, with the
  // gate read the same way.  Straight from the accumulators every gate load and
  // output store touched 32 rows far apart.  The gate multiplies by a
  // reciprocal (1 ulp) before the single rounding to bf16.
  constexpr int kORow = 4 * kW + 16;  // bytes per staged fp32 row (16 B pad)
  static_assert(128 * kORow <= kSmem, "the staged rows fit in the ring");
  // Output chunks (16 B of 8 dims), ordered (token, head, chunk): thread tid
  // takes chunks tid + 256 i.  Their gate values are requested first, all at
  // once, so that one memory latency overlaps the staging below instead of
  // one per few chunks in the store loop.
  constexpr int kChunkIters = 128 * (kW / 8) / 256;
  const int n_chunks = a.bm_tok * a.g * (kW / 8);
  // row / g by one multiply: (row + 1/2) / g lies at least 1/(2g) >= 2^-9 from
  // an integer and the float error is below 2^-15 for row < 256.
  const float inv_g = 1.0f / (float)a.g;
  u32x4 gate_raw[kChunkIters];
  if (a.gate) {
#pragma unroll
    for (int i = 0; i < kChunkIters; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 5, part = c & 31;
      const int tf = (int)(((float)row + 0.5f) * inv_g), hf = row - tf * a.g;
      const bool ok = c < n_chunks && tok_base + tf < L;
      const int64_t grow = (int64_t)(seq0 + (ok ? tok_base + tf : 0)) * a.Hq + u * a.g + (ok ? hf : 0);
      gate_raw[i] = *reinterpret_cast<const u32x4*>((const uint16_t*)a.gate + grow * a.q_row + 8 * part);
    }
  }
  const float inv_l = 1.0f / pair_sum(l_run);
  __syncthreads();
  {
    lds_u8* orow = lds + r * kORow;  // r = hoff * bm_tok + toff
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = 32 * db + 8 * jg + 4 * hg;
        *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(orow + 4 * d) =
            f32x4{o[db][4 * jg] * inv_l, o[db][4 * jg + 1] * inv_l, o[db][4 * jg + 2] * inv_l,
                  o[db][4 * jg + 3] * inv_l};
      }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kChunkIters; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 5, part = c & 31;
    const int tf = (int)(((float)row + 0.5f) * inv_g), hf = row - tf * a.g;
    if (c < n_chunks && tok_base + tf < L) {
      const lds_u8* src = lds + (hf * a.bm_tok + tf) * kORow + 32 * part;
      const f32x4 y0 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(src);
      const f32x4 y1 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(src + 16);
      float y[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      const int64_t grow = (int64_t)(seq0 + tok_base + tf) * a.Hq + u * a.g + hf;
      if (a.gate) {  // times sigmoid(gate) at the same dims
        const u32x4 gr = gate_raw[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[2 * e] *= __builtin_amdgcn_rcpf(1.0f + __expf(-bf16_lo(gr[e])));
          y[2 * e + 1] *= __builtin_amdgcn_rcpf(1.0f + __expf(-bf16_hi(gr[e])));
        }
      }
      *reinterpret_cast<u32x4*>((uint16_t*)a.out + grow * kW + 8 * part) =
          u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
    }
  }
}

}  // namespace

hipError_t launch_prefill_wide(const PrefillArgs& a, int n_items, hipStream_t st) {
  if (n_items <= 0) return hipSuccess;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)k_prefill_wide, hipFuncAttributeMaxDynamicSharedMemorySize, kSmem);
  if (attr != hipSuccess) return attr;
  const int64_t blocks = (int64_t)n_items * a.Hkv;
  hipLaunchKernelGGL(k_prefill_wide, dim3((unsigned)blocks), dim3(256), kSmem, st, (const PrefillItem*)a.items, a.Hkv, a);
  return hipGetLastError();
}

}  // namespace qw
