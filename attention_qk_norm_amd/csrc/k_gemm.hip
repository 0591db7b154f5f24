// Bias-free linear maps of the attention sublayer, bf16 in / fp32 accumulate,
// MFMA on gfx950: y = x W^T with W stored [out][in] ("Qwen3" notes, the
// Qwen3Attention excerpt: q_proj, k_proj, v_proj, o_proj; "7.2 Qwen3 全规模实现"
// §7.2.1 listing).
//
// Three epilogues:
//  * plain: y rounded to bf16 (o_proj, or any projection);
//  * qkv: the fused q/k/v projection.  Its output columns are head blocks of
//    128: Hq query heads, then Hkv key heads, then Hkv value heads (the three
//    weights stacked).  Query blocks are written raw (the attention kernel's
//    prologue norms and rotates them); key blocks are QK-Normed and rotated at
//    the token's position straight from the fp32 accumulators and written to
//    the KV cache (or a packed buffer); value blocks go to the cache as they
//    are.  So K and V reach HBM once, already in their cached form
//    ("Qwen3" notes: qkv_proj -> split -> RMSNorm(Q, K) -> RoPE);
//  * gated qkv: the same for the gated global layers of Qwen3-Next / Qwen3.5
//    (head_dim 256; "14. Qwen 家族" Qwen3-Next section; "第 20 章" §20.4):
//    q_proj gives 2 x 256 values per query head, the query then the gate,
//    written raw; key heads get the zero-centred norm (scale 1 + w) and the
//    partial rotation of their leading dims; value heads go as they are.
//
// Tiling: a workgroup computes a 256-token x 256-column tile as C^T = W X^T
// with v_mfma_f32_32x32x16_bf16 (A = W fragment, B = X fragment, both 16-byte
// reads from LDS), in one of two forms:
//  * eight waves (two per SIMD), each 64 tokens ((w >> 1) quarter) x 128
//    columns ((w & 1) half), 4 x 2 accumulators of 32 x 32: 6 fragment reads
//    per 8 MFMAs;
//  * four waves (one per SIMD), each 128 tokens x 128 columns, 4 x 4
//    accumulators (in AGPRs): 8 fragment reads per 16 MFMAs, so the LDS reads
//    take a third less.
// In both the tiles go HBM -> LDS directly (global_load_lds_dwordx4, no staging
// registers) into a two-stage ring; the barrier that publishes K step kt+1
// sits before the last k16 step of K step kt, whose fragments are already in
// registers, and the copies of K step kt+2 go out one per two MFMAs, half after
// that barrier and half in the first k16 step of K step kt+1, each with at
// least two k16 steps to land before the barrier that needs it.
// The plain epilogue takes the four-wave form, the q/k/v epilogues the
// eight-wave form.  Every epilogue stages the finished tile in LDS (the ring is
// idle by then) and stores whole rows.
// Either way a wave owns exactly one head block of 128 columns, and in the
// transposed accumulator a lane owns ONE token (lane % 32) and 64 of the
// block's 128 columns (the other 64 sit in lane ^ 32), and columns c and
// c + 64 (a RoPE pair) share a lane, so the norm is a lane-local sum plus one
// lane-pair exchange and the rotation is register-local.  The LDS ring holds
// padded 1 KB blocks (row r in block r % 32, slot r / 32; 16-byte skew between
// blocks, so the 16 rows of a fragment read land in 16 distinct bank groups).
#include <type_traits>

#include "kernels.h"

namespace qw {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kBlk = 1040;                 // 1 KB block (8 rows x 128 B) + 16 B skew
constexpr int kTile = 32 * kBlk;           // one 256 x 64 operand tile
constexpr int kStageBytes = 2 * kTile;     // x tile, then W tile
constexpr int kSmem = 2 * kStageBytes;     // two stages
// qkv: after the ring, the key norm scale (up to 256 floats) and the RoPE
// frequencies (64 doubles), read per lane in the epilogue; gated qkv: then the
// halves of the keys' sums of squares ([8 token blocks of 32][32 tokens][2 halves]).
constexpr int kGammaOff = kSmem, kFreqOff = kSmem + 1024, kSsOff = kSmem + 1536, kSmemQkv = kSmem + 1536 + 2048;
static_assert(kSmemQkv <= 160 * 1024, "LDS per workgroup");

__device__ __forceinline__ bf16x8 lds_load_b128(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

// Direct HBM -> LDS copy of 16 bytes per lane: lane l's bytes, read from
// gbase + voff, land at LDS address lds_base + 16 l (M0 holds the wave-uniform
// base; one wait state after writing M0).  Inline assembly, so the compiler
// does not wait for every outstanding copy before each LDS read: the K loop
// waits for its own copies (s_waitcnt vmcnt) before the barrier that
// publishes a K step.
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

// WAVES: 8 (64 tokens x 128 columns per wave) or 4 (128 x 128).
template <int EPI, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 1) void k_gemm(GemmArgs a) {
  constexpr int kThreads = WAVES * 64;
  constexpr int kTB = WAVES == 8 ? 2 : 4;  // token blocks of 32 per wave
  constexpr int kWT = 32 * kTB;            // tokens per wave
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  lds_u8* lds = (lds_u8*)(smem);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wt = w >> 1, wc = w & 1;  // token part (kWT tokens), column half (128 columns)
  const int n = lane & 31, hg = lane >> 5;

  // Tile order, XCD-aware.  Workgroups are dealt round-robin to the 8 XCDs
  // (blockIdx b runs on XCD b % 8), each with its own L2, and an XCD holds 32
  // of them at once (one per CU).  The tile grid is cut into 8 regions, one
  // per XCD, so an XCD streams only its region's panels of x and W.  Where the
  // region divides into blocks of 32 tiles (4 token tiles x 8 column tiles, or
  // 8 x 4), it is walked block by block: the 32 workgroups an XCD runs
  // together then read 12 panels (4 + 8) for their 32 tiles, the fewest any
  // shape allows.  With 8 x 1 regions every XCD covers every column block, so
  // XCD x starts at column block x: the key and value heads of a q/k/v
  // projection (its last columns, whose epilogue is the heaviest) are then
  // spread over the launch instead of falling on every CU at once.  Otherwise
  // the region is walked row by row; failing even that, consecutive
  // workgroups take consecutive column tiles.
  const int tiles_n = (a.N + kBN - 1) / kBN;
  const int tiles_m = (int)((a.M + kBM - 1) / kBM);
  int tm, tn;
  const int x = blockIdx.x & 7, idx = blockIdx.x >> 3;
  if (tiles_m % 16 == 0 && tiles_n % 16 == 0) {
    // regions: 4 x 2 (a quarter of the token tiles, half of the column tiles); blocks 4 x 8
    const int rm = tiles_m / 4, rn = tiles_n / 2, blk = idx >> 5, in = idx & 31, bpr = rn / 8;
    tm = (x >> 1) * rm + (blk / bpr) * 4 + (in >> 3);
    tn = (x & 1) * rn + (blk % bpr) * 8 + (in & 7);
  } else if (tiles_m % 64 == 0 && tiles_n % 4 == 0) {
    // regions: 8 x 1 (an eighth of the token tiles, every column tile); blocks 8 x 4
    const int rm = tiles_m / 8, blk = idx >> 5, in = idx & 31, bpr = tiles_n / 4;
    tm = x * rm + (blk / bpr) * 8 + (in >> 2);
    tn = ((blk % bpr + x) % bpr) * 4 + (in & 3);
  } else if (tiles_m % 4 == 0 && tiles_n % 2 == 0) {
    const int rn = tiles_n / 2;
    tm = (x >> 1) * (tiles_m / 4) + idx / rn;
    tn = (x & 1) * rn + idx % rn;
  } else {
    tm = blockIdx.x / tiles_n;
    tn = blockIdx.x - tm * tiles_n;
  }
  const int64_t row0 = (int64_t)tm * kBM;
  const int col0 = tn * kBN;

  const char* xbase = (const char*)(a.x + row0 * a.ldx);
  const char* wbase = (const char*)(a.w + (int64_t)col0 * a.ldw);
  const int64_t xrow = a.ldx * 2, wrow = a.ldw * 2;  // bytes per row
  const int last_x = (int)min((int64_t)kBM - 1, a.M - 1 - row0);
  const int last_w = min(kBN - 1, a.N - 1 - col0);
  f32x16 acc[4][kTB];  // [column block jc][token block it]
#pragma unroll
  for (int jc = 0; jc < 4; ++jc)
#pragma unroll
    for (int it = 0; it < kTB; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[jc][it][j] = 0.f;

  // Fragment (k16 step s): tile row r -> block r % 32, slot r / 32; 16-byte
  // chunk 2s + hg.  Token block it of the wave: row kWT wt + 32 it + n (slot
  // kTB wt + it); column block jc: row 128 wc + 32 jc + n (slot 4 wc + jc).
  const int xoff = n * kBlk + hg * 16 + wt * kTB * 128;
  const int woff = n * kBlk + hg * 16 + wc * 512;
  const int nk = a.K / kBK;
  float* gk_lds = (float*)(smem + kGammaOff);
  double* w_lds = (double*)(smem + kFreqOff);
  if constexpr (EPI == kGemmQkv) {  // published by the first barrier below
    if (tid < 128) gk_lds[tid] = bf16_to_f32(a.k_gamma[tid]);
    if (tid < 64) w_lds[tid] = a.rope.w[tid];
  } else if constexpr (EPI >= kGemmQkvGated) {
    if (tid < 256) gk_lds[tid] = a.gamma_offset + bf16_to_f32(a.k_gamma[tid]);
    if (tid < 64) w_lds[tid] = a.rope.w[tid];
  }
  bf16x8 wf[2][4], xf[2][kTB];
  auto read = [&](int kt, int s, int r) __attribute__((always_inline)) {
    // order: W 0, x 0 .. kTB-1, W 1..3 -- the first MFMAs of a step need W 0 and every x
    const lds_u8* xs = lds + (kt & 1) * kStageBytes;
    const lds_u8* ws = xs + kTile;
    const int buf = s & 1;
    if (r == 0) wf[buf][0] = lds_load_b128(ws + woff + s * 32);
    else if (r <= kTB) xf[buf][r - 1] = lds_load_b128(xs + xoff + (r - 1) * 128 + s * 32);
    else wf[buf][r - kTB] = lds_load_b128(ws + woff + (r - kTB) * 128 + s * 32);
  };
  constexpr int kReads = 4 + kTB;  // fragment reads per k16 step

  if constexpr (WAVES == 8) {
    // Copies: wave w fills blocks 4w .. 4w+3 of both tiles; lane l carries
    // slot l / 8 (row blk + 32 (l / 8)), 16-byte chunk l % 8 -- its LDS address
    // inside the block is 16 l.  Rows past the matrix repeat its last row
    // (their results are never stored).  The schedule is the four-wave form's:
    // the barrier that publishes K step kt+1 sits before K step kt's last k16
    // step, and K step kt+2's 8 copies per lane go out one per two MFMAs, half
    // after that barrier and half in K step kt+1's first k16 step.
    uint32_t xo[4], wo[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = w * 4 + m + 32 * (lane >> 3);
      xo[m] = (uint32_t)(min(r, last_x) * xrow) + (lane & 7) * 16;
      wo[m] = (uint32_t)(min(r, last_w) * wrow) + (lane & 7) * 16;
    }
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    // copy m (0 .. 7) of K step kt: x block 4w + m (m < 4), then W block 4w + m - 4
    auto copy = [&](int kt, int m) __attribute__((always_inline)) {
      const uint32_t dst = lds0 + (kt & 1) * kStageBytes + (m < 4 ? 0 : kTile) + (wu * 4 + (m & 3)) * kBlk;
      const char* src = (m < 4 ? xbase : wbase) + (int64_t)kt * kBK * 2;
      load_lds16_async(dst, src, m < 4 ? xo[m] : wo[m - 4]);
    };
    // K step 0 and the first half of K step 1; wait for step 0.
#pragma unroll
    for (int m = 0; m < 8; ++m) copy(0, m);
    if (nk > 1) {
#pragma unroll
      for (int m = 0; m < 4; ++m) copy(1, m);
      __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kReads; ++r) read(0, 0, r);
    // The 8 MFMAs of k16 step s, each followed by fn(i); sched_barrier keeps
    // the order, so every read and copy has the MFMAs after it to land; the two
    // waves of a SIMD interleave their streams.
    auto mfmas = [&](int s, auto fn) __attribute__((always_inline)) {
      const int buf = s & 1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int jc = i >> 1, it = i & 1;
        acc[jc][it] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][jc], xf[buf][it], acc[jc][it], 0, 0, 0);
        fn(i);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // One K step; kMore / kMore2 say whether K steps kt+1 / kt+2 exist
    // (compile-time in the steady state, so the MFMA stream has no branches).
    auto step = [&](int kt, auto more_tag, auto more2_tag) __attribute__((always_inline)) {
      constexpr bool kMore = decltype(more_tag)::value, kMore2 = decltype(more2_tag)::value;
      // k16 steps 0..2; the 6 fragments of step s+1 are read during step s, and
      // k16 step 0 sends the second half of K step kt+1's copies.
      mfmas(0, [&](int i) __attribute__((always_inline)) {
        if (i < kReads) read(kt, 1, i);
        if constexpr (kMore)
          if ((i & 1) == 0) copy(kt + 1, 4 + (i >> 1));
      });
#pragma unroll
      for (int s = 1; s < 3; ++s)
        mfmas(s, [&](int i) __attribute__((always_inline)) {
          if (i < kReads) read(kt, s + 1, i);
        });
      if constexpr (kMore) {
        // This wave's copies of K step kt+1 have landed; the barrier publishes
        // everyone's and (its fragment reads done) frees stage kt & 1.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
      }
      // k16 step 3 from registers; meanwhile the first fragments of K step
      // kt+1 and the first half of K step kt+2's copies into the freed stage.
      mfmas(3, [&](int i) __attribute__((always_inline)) {
        if constexpr (kMore)
          if (i < kReads) read(kt + 1, 0, i);
        if constexpr (kMore2)
          if ((i & 1) == 0) copy(kt + 2, i >> 1);
      });
    };
    int kt = 0;
    for (; kt + 2 < nk; ++kt) step(kt, std::true_type{}, std::true_type{});
    if (kt + 1 < nk) step(kt++, std::true_type{}, std::false_type{});
    step(kt, std::false_type{}, std::false_type{});
  } else {
    // Copies: wave w fills blocks 8w .. 8w+7 of both tiles; lane l carries
    // slot l / 8 (row blk + 32 (l / 8)), 16-byte chunk l % 8 -- its LDS
    // address inside the block is 16 l.  Rows past the matrix repeat its last
    // row (their results are never stored).
    uint32_t xo[8], wo[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int r = w * 8 + m + 32 * (lane >> 3);
      xo[m] = (uint32_t)(min(r, last_x) * xrow) + (lane & 7) * 16;
      wo[m] = (uint32_t)(min(r, last_w) * wrow) + (lane & 7) * 16;
    }
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    // copy m (0 .. 15) of K step kt: x block 8w + m (m < 8), then W block 8w + m - 8
    auto copy = [&](int kt, int m) __attribute__((always_inline)) {
      const uint32_t dst = lds0 + (kt & 1) * kStageBytes + (m < 8 ? 0 : kTile) + (wu * 8 + (m & 7)) * kBlk;
      const char* src = (m < 8 ? xbase : wbase) + (int64_t)kt * kBK * 2;
      load_lds16_async(dst, src, m < 8 ? xo[m] : wo[m - 8]);
    };
    // K step 0 and the first half of K step 1 (the second half goes out
    // during K step 0); wait for step 0.
#pragma unroll
    for (int m = 0; m < 16; ++m) copy(0, m);
    if (nk > 1) {
#pragma unroll
      for (int m = 0; m < 8; ++m) copy(1, m);
      __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kReads; ++r) read(0, 0, r);
    // The 16 MFMAs of k16 step s, each followed by fn(i); sched_barrier keeps
    // the order, so every read and copy has the MFMAs after it to land.
    auto mfmas = [&](int s, auto fn) __attribute__((always_inline)) {
      const int buf = s & 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int jc = i >> 2, it = i & 3;
        acc[jc][it] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][jc], xf[buf][it], acc[jc][it], 0, 0, 0);
        fn(i);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // One K step; kMore / kMore2 say whether K steps kt+1 / kt+2 exist
    // (compile-time in the steady state, so the MFMA stream has no branches).
    auto step = [&](int kt, auto more_tag, auto more2_tag) __attribute__((always_inline)) {
      constexpr bool kMore = decltype(more_tag)::value, kMore2 = decltype(more2_tag)::value;
      // k16 steps 0..2; the 8 fragments of step s+1 are read during step s, and
      // k16 step 0 sends the second half of K step kt+1's copies.
      mfmas(0, [&](int i) __attribute__((always_inline)) {
        if (i < 8) read(kt, 1, i);
        if constexpr (kMore)
          if ((i & 1) == 0) copy(kt + 1, 8 + (i >> 1));
      });
#pragma unroll
      for (int s = 1; s < 3; ++s)
        mfmas(s, [&](int i) __attribute__((always_inline)) {
          if (i < 8) read(kt, s + 1, i);
        });
      if constexpr (kMore) {
        // This wave's copies of K step kt+1 have landed; the barrier publishes
        // everyone's and (its fragment reads done) frees stage kt & 1.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
      }
      // k16 step 3 from registers; meanwhile the first fragments of K step
      // kt+1 and the first half of K step kt+2's copies into the freed stage.
      mfmas(3, [&](int i) __attribute__((always_inline)) {
        if constexpr (kMore)
          if (i < 8) read(kt + 1, 0, i);
        if constexpr (kMore2)
          if ((i & 1) == 0) copy(kt + 2, i >> 1);
      });
    };
    int kt = 0;
    for (; kt + 2 < nk; ++kt) step(kt, std::true_type{}, std::true_type{});
    if (kt + 1 < nk) step(kt++, std::true_type{}, std::false_type{});
    step(kt, std::false_type{}, std::false_type{});
  }

  // ---- epilogue.  acc[jc][it][j]: token row0 + kWT wt + 32 it + n, column
  // col0 + 128 wc + 32 jc + 8 (j / 4) + 4 hg + j % 4.
  const int ccol = col0 + 128 * wc;  // the wave's first column (a head block in the qkv form)
  // The gated q/k/v epilogue (head_dim 256).  Column regions -- tiles never
  // straddle them, every width being a multiple of 256 -- are: Hq query rows of
  // q_width values, written raw to q_out [M][Hq][q_width]; Hkv key heads, normed
  // and partially rotated at each token's position; Hkv value heads.  A head of
  // 256 spans the tile: wave (wt, wc) holds dims 128 wc .. 128 wc + 127 of its kWT
  // tokens, so a key's sum of squares adds the two waves' halves through LDS (the
  // branch is uniform over the workgroup, so its barrier is too), and the
  // rotated dims (at most 128) all lie in the waves with wc = 0.  acc[jc][it][j]:
  // token row0 + kWT wt + 32 it + n, column 32 jc + 8 (j / 4) + 4 hg + j % 4 of the
  // wave's 128.
  if constexpr (EPI >= kGemmQkvGated) {
    // one instantiation per rotary width: 32, 64 or 128 leading dims turn
    constexpr int ROT = EPI == kGemmQkvGated ? 32 : EPI == kGemmQkvGated + 1 ? 64 : 128;
    // As in the other epilogues the finished rows are staged in LDS (row r,
    // 16-byte chunk c at position c ^ (r % 16)) and leave whole: a query tile is
    // 512 contiguous bytes of each token's q_out row, a key or value tile one
    // head of 256 dims, i.e. one cache slot.  The (sequence, position) of each
    // token sits in the 2 KB of the ring past the staged rows.
    auto slot = [](int r, int c) __attribute__((always_inline)) { return r * 512 + ((c ^ (r & 15)) << 4); };
    typedef __attribute__((address_space(3))) int32_t lds_i32;
    lds_i32* meta = (lds_i32*)(lds + kBM * 512);  // [256][2]: sequence, position
    static_assert(kBM * 512 + kBM * 8 <= kSmem, "staged rows and positions fit in the ring");
    const int qcols = a.Hq * a.q_width;
    const bool q_tile = col0 < qcols;  // query (and gate) values, raw
    constexpr int D = kMaxD;
    const bool is_k = !q_tile && col0 < qcols + a.Hkv * D;
    const int kv = q_tile ? 0 : (col0 - qcols) / D - (is_k ? 0 : a.Hkv);
    float inv[kTB] = {};
    if (is_k) {
      float* ss_lds = (float*)(smem + kSsOff);
#pragma unroll
      for (int it = 0; it < kTB; ++it) {
        float ss = 0.f;
#pragma unroll
        for (int jc = 0; jc < 4; ++jc)
#pragma unroll
          for (int j = 0; j < 16; ++j) ss += acc[jc][it][j] * acc[jc][it][j];
        ss = pair_sum(ss);  // lane n ^ 32 holds the other 64 of the wave's 128 dims
        if (hg == 0) ss_lds[((wt * kTB + it) * 32 + n) * 2 + wc] = ss;
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < kTB; ++it) {
        const float* p = ss_lds + ((wt * kTB + it) * 32 + n) * 2;
        inv[it] = rsqrtf((p[0] + p[1]) * (1.0f / D) + a.eps);
      }
    }
    __syncthreads();  // every wave's last fragment reads are done
#pragma unroll
    for (int it = 0; it < kTB; ++it) {
      const int r = kWT * wt + 32 * it + n;
      const int64_t tok = row0 + r;
      float x[4][16];
#pragma unroll
      for (int jc = 0; jc < 4; ++jc)
#pragma unroll
        for (int j = 0; j < 16; ++j) x[jc][j] = acc[jc][it][j];
      if (!q_tile) {
        int s = 0, pos = 0;
        if (tok < a.M) token_position(a, tok, s, pos);
        if (is_k) {
          // norm scale 1 + w (the table holds gamma_offset + gamma); RMS is
          // rotation-invariant, so one inv serves both orders
          auto scale = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int jc = 0; jc < 4; ++jc)
#pragma unroll
              for (int j = 0; j < 16; ++j) x[jc][j] *= inv[it] * gk_lds[128 * wc + 32 * jc + 8 * (j >> 2) + 4 * hg + (j & 3)];
          };
          // dims c and c + rot/2 (c < rot/2) turn by pos * w_c, the angle reduced
          // in fp64 and evaluated by the hardware sine/cosine, which take turns
          auto turn = [&](int jc1, int j1, int jc2, int j2) __attribute__((always_inline)) {
            const int c = 32 * jc1 + 8 * (j1 >> 2) + 4 * hg + (j1 & 3);
            const double t = (double)pos * (w_lds[c] * 0.15915494309189535);
            const float rr = (float)(t - rint(t));
            const float cs = __builtin_amdgcn_cosf(rr), sn = __builtin_amdgcn_sinf(rr);
            const float y1 = x[jc1][j1], y2 = x[jc2][j2];
            x[jc1][j1] = y1 * cs - y2 * sn;
            x[jc2][j2] = y2 * cs + y1 * sn;
          };
          if (a.order == 0) scale();
          if (wc == 0) {
            if constexpr (ROT == 128) {
#pragma unroll
              for (int jc = 0; jc < 2; ++jc)
#pragma unroll
                for (int j = 0; j < 16; ++j) turn(jc, j, jc + 2, j);
            } else if constexpr (ROT == 64) {
#pragma unroll
              for (int j = 0; j < 16; ++j) turn(0, j, 1, j);
            } else {
#pragma unroll
              for (int j = 0; j < 8; ++j) turn(0, j, 0, j + 8);
            }
          }
          if (a.order != 0) scale();
        }
        if (wc == 0 && hg == 0) {
          meta[2 * r] = s;
          meta[2 * r + 1] = pos;
        }
      }
#pragma unroll
      for (int jc = 0; jc < 4; ++jc)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg)
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(lds + slot(r, 16 * wc + 4 * jc + jg) + 8 * hg) =
              u32x2{pack_bf16x2(x[jc][4 * jg], x[jc][4 * jg + 1]), pack_bf16x2(x[jc][4 * jg + 2], x[jc][4 * jg + 3])};
    }
    __syncthreads();
    // A thread keeps one chunk column c and walks the rows r0, r0 + kThreads / 32, ...
    constexpr int kRowStep = kThreads / 32;
    const int c = tid & 31, r0 = tid >> 5;
    uint16_t* cache = is_k ? a.k_cache : a.v_cache;
    uint16_t* base = q_tile ? a.q_out + row0 * qcols + col0 + 8 * c
                            : (cache ? cache + kv * a.cs_head : (is_k ? a.k_out : a.v_out) + (row0 * a.Hkv + kv) * D) + 8 * c;
    const int64_t step = q_tile ? (int64_t)qcols : (int64_t)a.Hkv * D;  // per row, without a cache
#pragma unroll
    for (int i = 0; i < kBM / kRowStep; ++i) {
      const int r = r0 + kRowStep * i;
      if (row0 + r >= a.M) continue;
      uint16_t* dst = (q_tile || !cache) ? base + r * step
                                         : base + meta[2 * r] * a.cs_seq + (int64_t)meta[2 * r + 1] * a.cs_tok;
      *reinterpret_cast<u32x4*>(dst) =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(lds + slot(r, c));
    }
    return;
  }
  if constexpr (EPI == kGemmPlain) {
    // The tile leaves as whole rows: the accumulators go to LDS as bf16 (the
    // ring is idle once every wave is past its last K step), then each wave
    // stores two rows of 512 B per instruction.  Straight from the
    // accumulators, each store instruction touched 32 rows 16 B apart.  Row r
    // holds its 16-byte chunk c (columns 8c .. 8c+7) at position c ^ (r % 16),
    // so the full-row reads are conflict-free.
    auto slot = [](int r, int c) __attribute__((always_inline)) { return r * 512 + ((c ^ (r & 15)) << 4); };
    __syncthreads();  // every wave's last fragment reads are done
#pragma unroll
    for (int it = 0; it < kTB; ++it) {
      const int r = kWT * wt + 32 * it + n;
#pragma unroll
      for (int jc = 0; jc < 4; ++jc)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg)
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(lds + slot(r, 16 * wc + 4 * jc + jg) + 8 * hg) =
              u32x2{pack_bf16x2(acc[jc][it][4 * jg], acc[jc][it][4 * jg + 1]),
                    pack_bf16x2(acc[jc][it][4 * jg + 2], acc[jc][it][4 * jg + 3])};
    }
    __syncthreads();
    // A thread keeps one chunk column c and walks the rows r0, r0 + kThreads / 32, ...
    constexpr int kRowStep = kThreads / 32;
    const int rows = (int)min((int64_t)kBM, a.M - row0), c = tid & 31, r0 = tid >> 5;
    if (8 * c < a.N - col0) {
      uint16_t* dst = a.y + row0 * a.ldy + col0 + 8 * c;
#pragma unroll
      for (int i = 0; i < kBM / kRowStep; ++i) {
        const int r = r0 + kRowStep * i;
        if (r < rows)
          *reinterpret_cast<u32x4*>(dst + r * a.ldy) =
              *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(lds + slot(r, c));
      }
    }
  } else {
    // The two column halves of the tile are head blocks: query, key or value.
    // Keys are normed and rotated here from the fp32 accumulators; then, as in
    // the plain tile, the rows are staged in LDS and leave whole: each 256-byte
    // head row to q_out (query) or to the token's cache slot (key, value).  The
    // (sequence, position) of every token goes through LDS from the wave that
    // looked it up: the tile's last column half, a key or value block whenever
    // either half is.
    auto slot = [](int r, int c) __attribute__((always_inline)) { return r * 512 + ((c ^ (r & 15)) << 4); };
    typedef __attribute__((address_space(3))) int32_t lds_i32;
    lds_i32* meta = (lds_i32*)(lds + kSsOff);  // [256][2]: sequence, position
    const bool half_ok = ccol < a.N;
    const int hh = ccol / 128;  // this wave's head block
    const bool is_q = hh < a.Hq, is_k = !is_q && hh < a.Hq + a.Hkv;
    const bool publisher = !is_q && (wc == 1 || col0 + 128 >= a.N);
    // norm scale of column 32 jc + 8 (j / 4) + 4 hg + j % 4
    auto gk = [&](int jc, int j) __attribute__((always_inline)) { return gk_lds[32 * jc + 8 * (j >> 2) + 4 * hg + (j & 3)]; };
    __syncthreads();  // every wave's last fragment reads are done
#pragma unroll
    for (int it = 0; it < kTB; ++it) {
      const int r = kWT * wt + 32 * it + n;
      const int64_t tok = row0 + r;
      float x[4][16];
#pragma unroll
      for (int jc = 0; jc < 4; ++jc)
#pragma unroll
        for (int j = 0; j < 16; ++j) x[jc][j] = acc[jc][it][j];
      int s = 0, pos = 0;
      if (!is_q && half_ok) {
        if (tok < a.M) token_position(a, tok, s, pos);
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
              const float rr = (float)(t - rint(t));
              const float c = __builtin_amdgcn_cosf(rr), sn = __builtin_amdgcn_sinf(rr);
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
      }
      if (publisher && hg == 0) {
        meta[2 * r] = s;
        meta[2 * r + 1] = pos;
      }
      if (half_ok)
#pragma unroll
        for (int jc = 0; jc < 4; ++jc)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg)
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(lds + slot(r, 16 * wc + 4 * jc + jg) + 8 * hg) =
                u32x2{pack_bf16x2(x[jc][4 * jg], x[jc][4 * jg + 1]), pack_bf16x2(x[jc][4 * jg + 2], x[jc][4 * jg + 3])};
    }
    __syncthreads();
    // A thread keeps one chunk column c (and so one head block) and walks the
    // rows r0, r0 + kThreads / 32, ...; everything but the row is set up once.
    constexpr int kRowStep = kThreads / 32;
    const int c = tid & 31, r0 = tid >> 5;
    const int hb = (col0 >> 7) + (c >> 4);  // the chunk's head block
    if (128 * hb < a.N) {
      if (hb < a.Hq) {
        uint16_t* dst = a.q_out + (row0 * a.Hq + hb) * 128 + 8 * (c & 15);
        const int64_t step = (int64_t)a.Hq * 128;
#pragma unroll
        for (int i = 0; i < kBM / kRowStep; ++i) {
          const int r = r0 + kRowStep * i;
          if (row0 + r < a.M)
            *reinterpret_cast<u32x4*>(dst + r * step) =
                *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(lds + slot(r, c));
        }
      } else {
        const bool k_blk = hb < a.Hq + a.Hkv;
        const int kv = k_blk ? hb - a.Hq : hb - a.Hq - a.Hkv;
        uint16_t* cache = k_blk ? a.k_cache : a.v_cache;
        uint16_t* packed = (k_blk ? a.k_out : a.v_out) + (row0 * a.Hkv + kv) * 128 + 8 * (c & 15);
        uint16_t* slot0 = cache ? cache + kv * a.cs_head + 8 * (c & 15) : nullptr;
#pragma unroll
        for (int i = 0; i < kBM / kRowStep; ++i) {
          const int r = r0 + kRowStep * i;
          if (row0 + r >= a.M) continue;
          uint16_t* dst = cache ? slot0 + meta[2 * r] * a.cs_seq + (int64_t)meta[2 * r + 1] * a.cs_tok
                                : packed + (int64_t)r * a.Hkv * 128;
          *reinterpret_cast<u32x4*>(dst) =
              *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(lds + slot(r, c));
        }
      }
    }
  }
}

template <int EPI, int WAVES>
hipError_t launch_w(const GemmArgs& a, hipStream_t st) {
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)k_gemm<EPI, WAVES>, hipFuncAttributeMaxDynamicSharedMemorySize, kSmemQkv);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
  hipLaunchKernelGGL((k_gemm<EPI, WAVES>), dim3((unsigned)tiles), dim3(WAVES * 64), kSmemQkv, st, a);
  return hipGetLastError();
}

// The plain epilogue takes the four-wave form (1-4% ahead of the eight-wave
// form at every width measured); the q/k/v epilogues take the eight-wave form,
// whose second wave per SIMD covers the norm, rotation and position lookups
// (1% ahead on the Qwen3-8B projection), and where the gated epilogue fits
// without spills.
template <int EPI>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  if constexpr (EPI == kGemmPlain) return launch_w<EPI, 4>(a, st);
  else return launch_w<EPI, 8>(a, st);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int epilogue, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (epilogue == kGemmQkvGated) {
    if (a.rot == 32) return launch_t<kGemmQkvGated>(a, st);
    if (a.rot == 64) return launch_t<kGemmQkvGated + 1>(a, st);
    return launch_t<kGemmQkvGated + 2>(a, st);
  }
  return epilogue == kGemmQkv ? launch_t<kGemmQkv>(a, st) : launch_t<kGemmPlain>(a, st);
}

}  // namespace qw
