// Device-side helpers shared by the libqwattn kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qw {

constexpr int kD = 128;       // head_dim of the Qwen3 layers
constexpr int kHalf = kD / 2; // their RoPE pairs (i, i + 64)
constexpr int kMaxD = 256;    // head_dim of the gated (Qwen3-Next / Qwen3.5) layers

// RoPE frequencies theta^(-2i/rot), i < rot/2 (rot = the rotated coordinates,
// the whole head for Qwen3), computed by the host in double.
struct RopeFreq {
  double w[kMaxD / 2];
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Two floats -> packed bf16 pair (round to nearest even, one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// cos and sin of pos * w: the angle is formed and reduced to [-pi, pi] in
// double (two-constant Cody-Waite with 2*pi split in a high and a low double),
// then evaluated in fp32.  Keeps the error near one fp32 ulp at any position.
__device__ __forceinline__ void rope_cos_sin(int pos, double w, float& c, float& s) {
  const double phi = (double)pos * w;
  const double k = rint(phi * 0.15915494309189535);  // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, phi);          // 2 pi, high part
  r = fma(-k, 2.4492935982947064e-16, r);              // 2 pi, low part
  sincosf((float)r, &s, &c);
}

// Sum over each group of 16 consecutive lanes (one DPP row): butterfly within
// quads, then rotations by 4 and 8 inside the row; every lane ends with the sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror 4
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror 8
  return x;
}

// Exclusive prefix sum over a 1024-thread block (each thread one value);
// `tmp` is 16 ints of LDS.  Returns the thread's exclusive prefix and writes the
// block total to *total.  Every thread of the block must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  int wsum = 0, all = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = tmp[i];
    wsum += i < w ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return wsum + inc - v;
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < width; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <int width>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int m = 1; m < width; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// Reductions over the lane pair (l, l ^ 32) with one v_permlane32_swap: the
// swap exchanges the upper half of its first operand with the lower half of its
// second, so across its two results every lane sees its own value and its
// partner's (in lane-dependent order) -- combine both, never pick one.
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// acc + lo + hi of a packed bf16 pair, in one v_dot2c_f32_bf16 against (1, 1).
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u), acc,
                                         false);
}

// gfx950 transposed LDS read: within each 16-lane group, lane i receives
// element (i % 4) of the 8 bytes that lanes 4r + i/4 (r = 0..3) point at, as
// its elements r = 0..3.  Returned as two dwords.
__device__ __forceinline__ u32x2 lds_read_tr16(const lds_u8* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>(const_cast<lds_u8*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Two transposed reads -> one 8 x bf16 MFMA operand (whole-dword moves only).
__device__ __forceinline__ bf16x8 concat_tr16(u32x2 lo, u32x2 hi) {
  u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// Load / store helpers for the two storage types.
struct F32 {
  typedef float T;
  static constexpr int kBytes = 4;
};
struct BF16 {
  typedef uint16_t T;
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ void load4(const float* p, float (&x)[4]) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
}
__device__ __forceinline__ void load4(const uint16_t* p, float (&x)[4]) {
  u32x2 v = *reinterpret_cast<const u32x2*>(p);
  x[0] = bf16_lo(v[0]); x[1] = bf16_hi(v[0]); x[2] = bf16_lo(v[1]); x[3] = bf16_hi(v[1]);
}
__device__ __forceinline__ void store4(float* p, const float (&x)[4]) {
  f32x4 v = {x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p) = v;
}
__device__ __forceinline__ void store4(uint16_t* p, const float (&x)[4]) {
  u32x2 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  *reinterpret_cast<u32x2*>(p) = v;
}

}  // namespace qw
