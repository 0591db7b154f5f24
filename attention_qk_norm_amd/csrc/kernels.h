// Kernel argument blocks and host-side launchers of libqwattn.  Launchers return
// hipSuccess or the launch error; they do no validation (the C-ABI layer does).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace qw {

// ---------------------------------------------------------------- norm + RoPE
// Row sources: tensor 0 = q (normed, rotated), 1 = k (normed, rotated),
// 2 = v (copied unchanged into the cache).  heads[i] == 0 skips tensor i.
enum NormRopeMode : int {
  kPosExplicit = 0,  // token n at position pos[n]; outputs contiguous
  kPosPacked = 1,    // token n in sequence s (from cu), position n - cu[s] (+ pos[s] if pos is set)
  kPosDecode = 2,    // token n is sequence n's new token, at position pos[n]
};

struct NormRopeArgs {
  const void* x[3];
  int in_row[3];            // elements between consecutive head rows of x[i] (head_dim, or 2 head_dim for a gated q)
  void* out[2];             // contiguous q / k outputs (k unused when k_cache set)
  const void* gamma[2];
  int heads[3];
  void* k_cache;            // when set, rotated k goes to cache(seq, head, pos)
  void* v_cache;            // when set (and heads[2] > 0), v goes to cache(seq, head, pos)
  int64_t cs_seq, cs_head, cs_tok;
  const int32_t* pos;
  const int32_t* cu;
  int n_seq;
  int mode;
  int64_t n_tok;
  float eps;
  int order;                // 0: QK-Norm then RoPE; 1: RoPE then QK-Norm
  int head_dim;             // 128 or 256
  int rot;                  // rotated coordinates (pairs (i, i + rot/2)); head_dim for Qwen3
  float gamma_offset;       // 0: scale = gamma; 1: zero-centred norm, scale = 1 + gamma
  RopeFreq rope;            // theta^(-2i/rot)
};

hipError_t launch_normrope(bool bf16, const NormRopeArgs& a, hipStream_t st);

// ---------------------------------------------------------------- prefill
// One entry of the work list: query tile qt of sequence s, with what a
// workgroup needs next (its rows' token offset and count, and the position of
// the sequence's first row), so that it starts with a single dependent load.
struct PrefillItem {
  int32_t s, qt, seq0, len, p0, pad0, pad1, pad2;
};
// Work list of (sequence, query tile) pairs, heaviest first.
struct PlanArgs {
  const int32_t* cu;
  int n_seq;
  int bm_tok;        // query tokens per tile
  int max_tiles;     // max over sequences of ceil(L / bm_tok)
  int n_items;       // sum over sequences of ceil(L / bm_tok)
  int32_t* scratch;  // 4 * (max_tiles + 1) + n_seq ints
  const int32_t* start_pos;  // NULL, or (an append) the position of each sequence's first row
  PrefillItem* items;
  // bf16 path: the QK-Norm logit bound of the launch decides the softmax form
  const void* q_gamma;       // NULL on the fp32 path
  const void* k_gamma;
  float scale_log2e;
  float gamma_offset;        // norm scale = gamma_offset + gamma
  int head_dim;
  int32_t* static_flag;      // out: [0] 1 when the static-bound softmax applies; [1] the
                             // float -B, B its logit bound rounded up (the weights are
                             // 2^(score - B))
};
hipError_t launch_prefill_plan(const PlanArgs& a, hipStream_t st);

struct PrefillArgs {
  const void* q;            // raw queries; row (token n, head t) at q + (n*Hq + t)*q_row
  int q_row;                // head_dim, or 2 head_dim when the rows carry the output gate
  const void* gate;         // NULL, or the gate rows (q + head_dim, same strides): out *= sigmoid(gate)
  const void* q_gamma;
  const void* k_gamma;      // bf16 path: bounds the rotated-key norms
  const void* qhat;         // fp32 path: normed+rotated q [n_tok][Hq][head_dim] (fp32)
  const void* khat;         // rotated keys; row (s, h, j) at khat + h*ks_head + base(s) + j*ks_tok
  int64_t ks_seq, ks_head, ks_tok;
  int k_packed;             // 1: base(s) = cu[s]*ks_tok; 0: base(s) = s*ks_seq
  const void* v;            // V rows; row (s, h, j) at v + h*vs_head + base(s) + j*vs_tok
  int64_t vs_seq, vs_head, vs_tok;
  int v_packed;
  const int32_t* cu;        // packed: sequence offsets; decode: unused
  const int32_t* start_pos; // decode (fp32 path): position of each sequence's new token;
                            // prefill: NULL, or (an append) position of each sequence's first row
  const PrefillItem* items;
  const int32_t* static_flag;  // bf16 path: written by the plan kernel ([0] form, [1] shift)
  void* out;
  int n_seq, Hq, Hkv, g, bm_tok;
  int decode;               // fp32 path: items are (seq, 0), one query token at start_pos
  float scale_log2e;        // softmax scale * log2(e)
  float eps;
  int order;                // bf16 Q prologue: 0 QK-Norm then RoPE, 1 RoPE then QK-Norm
  int head_dim;             // 128 or 256
  int rot;                  // bf16 Q prologue: rotated coordinates
  float gamma_offset;       // bf16 Q prologue: norm scale = gamma_offset + gamma
  RopeFreq rope;
};
constexpr int kPrefillRows = 256;  // query rows (g heads x bm_tok tokens) per workgroup
constexpr int kWideRows = 128;     // the same for head_dim 256
constexpr int kAttnF32Rows = 64;   // fp32 path: query rows per workgroup
hipError_t launch_prefill_bf16(const PrefillArgs& a, int n_items, hipStream_t st);
hipError_t launch_prefill_wide(const PrefillArgs& a, int n_items, hipStream_t st);
hipError_t launch_attn_f32(const PrefillArgs& a, int n_items, hipStream_t st);

// ---------------------------------------------------------------- decode
struct DecodeArgs {
  const uint16_t* qhat;     // normed+rotated new queries [n_seq][Hq][head_dim] (bf16)
  const uint16_t* gate;     // NULL, or gate rows: (seq i, head t) at gate + (i*Hq + t)*q_row
  int q_row;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int64_t cs_seq, cs_head, cs_tok;
  const int32_t* start_pos; // keys of sequence i: slots 0 .. start_pos[i] (inclusive)
  const int32_t* chunk_off; // [n_seq + 1] prefix of chunk counts
  const int32_t* chunk_seq; // [total chunks] sequence of each chunk
  float* partial;           // [total_chunks][Hq][head_dim + 4]: accumulators, m, l, 2 pad floats
  uint16_t* out;            // [n_seq][Hq][head_dim]
  int n_seq, Hq, Hkv, g;
  int head_dim;             // 128 or 256
  int chunk;                // keys per split (multiple of kDecodeKeysPerPass)
  float scale_log2e;
};
inline int part_stride(int head_dim) { return head_dim + 4; }
constexpr int kDecodeKeysPerPass = 128;  // 4 waves x 32 keys
hipError_t launch_decode_plan(const int32_t* start_pos, int n_seq, int chunk, int max_chunks, int32_t* chunk_off,
                              int32_t* chunk_seq, hipStream_t st);
hipError_t launch_decode_split(const DecodeArgs& a, int total_chunks, hipStream_t st);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t st);

// ---------------------------------------------------------------- projections
// y = x W^T, bf16 operands, fp32 accumulation.  x [M][K] (row stride ldx), W
// [N][K] (row stride ldw); K a multiple of 64, N a multiple of 128.
enum GemmEpilogue : int {
  kGemmPlain = 0,     // y [M][N] (row stride ldy, a multiple of 8), rounded to bf16
  kGemmQkv = 1,       // columns = Hq query, Hkv key, Hkv value head blocks of 128
  kGemmQkvGated = 2,  // columns = Hq query rows of q_width (query, then gate), Hkv key and Hkv
                      // value heads of 256 (the gated layers)
};
struct GemmArgs {
  const uint16_t* x;
  const uint16_t* w;
  int64_t M;
  int N, K;
  int64_t ldx, ldw;
  uint16_t* y;              // plain
  int64_t ldy;
  int Hq, Hkv;              // qkv: head blocks
  int q_width;              // gated qkv: values per query head in the q_proj output (256, or 512
                            // with the output gate: the query, then the gate)
  int rot;                  // gated qkv: rotated leading dims of a key head (32, 64 or 128)
  float gamma_offset;       // gated qkv: key norm scale = gamma_offset + gamma
  uint16_t* q_out;          // qkv: raw queries [M][Hq][128] (gated: [M][Hq][q_width])
  uint16_t* k_out;          // qkv: normed+rotated keys [M][Hkv][d] when k_cache is NULL
  uint16_t* v_out;          // qkv: values [M][Hkv][d] when v_cache is NULL
  uint16_t* k_cache;        // qkv: cache rows (seq, head, pos) as in NormRopeArgs
  uint16_t* v_cache;
  int64_t cs_seq, cs_head, cs_tok;
  const int32_t* cu;        // qkv: packed sequence offsets [n_seq + 1]
  int n_seq;
  const int32_t* start_pos; // qkv: NULL, or (an append) each sequence's first position
  const uint16_t* k_gamma;
  float eps;
  int order;
  RopeFreq rope;
};
hipError_t launch_gemm(const GemmArgs& a, int epilogue, hipStream_t st);

// ---------------------------------------------------------------- fixed scratch
// Device scratch for the entry points that allocate nothing: this many bytes
// per device, at the address decode_scratch returns for the current device
// (looked up once per device; shared by every such call on that device).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t decode_scratch(void** ptr);

// ---------------------------------------------------------------- measurement aids
hipError_t launch_mfma_probe(int n_wg, int iters4, float* sink, hipStream_t st);
hipError_t launch_read_probe(int n_wg, const void* src, int64_t n16, float* sink, hipStream_t st);

}  // namespace qw
