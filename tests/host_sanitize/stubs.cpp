// Host-only stand-ins for the kernel launchers and for the four HIP runtime
// calls the validation layer makes, so that qwattn_api.cpp runs under
// AddressSanitizer and UndefinedBehaviorSanitizer on a machine with no GPU.
//
// Device pointers in these runs are small fake addresses that nothing ever
// dereferences.  The workspace is host memory of exactly the size the caller
// was told to allocate, so each launcher below writes every workspace byte its
// kernel would write (and reads what it would read): a workspace layout that
// runs past the end becomes a heap-buffer-overflow report.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>

#include "kernels.h"
#include "stubs.h"

namespace stub {
int launches = 0;
int64_t n_tok = 0;
int64_t total_chunks = 0;
int n_cu = 256;
unsigned sink = 0;

bool is_host(const void* p) { return reinterpret_cast<uintptr_t>(p) >= kHostFloor; }

void write(const void* p, size_t bytes) {
  if (is_host(p) && bytes) std::memset(const_cast<void*>(p), 0x5a, bytes);
}

void read(const void* p, size_t bytes) {
  if (!is_host(p)) return;
  const unsigned char* b = static_cast<const unsigned char*>(p);
  for (size_t i = 0; i < bytes; i += 61) sink += b[i];
  if (bytes) sink += b[bytes - 1];
}
}  // namespace stub

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = stub::n_cu;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub error"; }
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

namespace qw {

hipError_t launch_normrope(bool bf16, const NormRopeArgs& a, hipStream_t) {
  ++stub::launches;
  const size_t es = bf16 ? 2 : 4;
  // mode kPosDecode handles one token per sequence; the others n_tok rows
  const int64_t rows = a.n_tok;
  if (a.heads[0] > 0) stub::write(a.out[0], rows * a.heads[0] * a.head_dim * es);
  if (a.heads[1] > 0 && !a.k_cache) stub::write(a.out[1], rows * a.heads[1] * a.head_dim * es);
  return hipSuccess;
}

hipError_t launch_prefill_plan(const PlanArgs& a, hipStream_t) {
  ++stub::launches;
  stub::write(a.scratch, (4 * ((int64_t)a.max_tiles + 1) + a.n_seq) * sizeof(int32_t));
  stub::write(a.items, (size_t)a.n_items * sizeof(PrefillItem));
  if (a.static_flag) stub::write(a.static_flag, 2 * sizeof(int32_t));
  return hipSuccess;
}

static hipError_t attention(const PrefillArgs& a, int n_items, bool bf16) {
  ++stub::launches;
  const size_t es = bf16 ? 2 : 4;
  stub::read(a.items, (size_t)n_items * sizeof(PrefillItem));
  if (a.static_flag) stub::read(a.static_flag, 2 * sizeof(int32_t));
  if (!bf16) stub::read(a.qhat, stub::n_tok * a.Hq * a.head_dim * 4);
  if (a.k_packed) stub::read(a.khat, stub::n_tok * a.Hkv * a.head_dim * es);
  if (a.v_packed) stub::read(a.v, stub::n_tok * a.Hkv * a.head_dim * es);
  stub::write(a.out, stub::n_tok * a.Hq * a.head_dim * es);
  return hipSuccess;
}
hipError_t launch_prefill_bf16(const PrefillArgs& a, int n, hipStream_t) { return attention(a, n, true); }
hipError_t launch_prefill_wide(const PrefillArgs& a, int n, hipStream_t) { return attention(a, n, true); }
hipError_t launch_attn_f32(const PrefillArgs& a, int n, hipStream_t) {
  if (a.decode) {  // one query row per sequence, q̂ fp32 in the workspace
    ++stub::launches;
    stub::read(a.qhat, (size_t)a.n_seq * a.Hq * a.head_dim * 4);
    return hipSuccess;
  }
  return attention(a, n, false);
}

hipError_t launch_decode_plan(const int32_t*, int n_seq, int, int max_chunks, int32_t* chunk_off, int32_t* chunk_seq,
                              hipStream_t) {
  ++stub::launches;
  stub::write(chunk_off, ((size_t)n_seq + 1) * sizeof(int32_t));
  stub::write(chunk_seq, (size_t)max_chunks * sizeof(int32_t));
  return hipSuccess;
}

hipError_t launch_decode_split(const DecodeArgs& a, int total_chunks, hipStream_t) {
  ++stub::launches;
  stub::total_chunks = total_chunks;
  stub::read(a.qhat, (size_t)a.n_seq * a.Hq * a.head_dim * 2);
  stub::read(a.chunk_seq, (size_t)total_chunks * sizeof(int32_t));
  stub::write(a.partial, (size_t)total_chunks * a.Hq * part_stride(a.head_dim) * sizeof(float));
  return hipSuccess;
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t) {
  ++stub::launches;
  stub::read(a.chunk_off, ((size_t)a.n_seq + 1) * sizeof(int32_t));
  stub::read(a.partial, (size_t)stub::total_chunks * a.Hq * part_stride(a.head_dim) * sizeof(float));
  return hipSuccess;
}

hipError_t launch_gemm(const GemmArgs& a, int epilogue, hipStream_t) {
  ++stub::launches;
  stub::read(a.x, (size_t)a.M * a.ldx * 2);
  if (epilogue == kGemmPlain) {
    stub::write(a.y, (size_t)a.M * a.ldy * 2);
  } else {
    const size_t d = epilogue == kGemmQkvGated ? 256 : 128;
    const size_t qw = epilogue == kGemmQkvGated ? (size_t)a.q_width : d;
    stub::write(a.q_out, (size_t)a.M * a.Hq * qw * 2);
    if (!a.k_cache) stub::write(a.k_out, (size_t)a.M * a.Hkv * d * 2);
    if (!a.v_cache) stub::write(a.v_out, (size_t)a.M * a.Hkv * d * 2);
  }
  return hipSuccess;
}

// The fixed scratch: host memory of exactly the device array's size.
hipError_t decode_scratch(void** ptr) {
  static void* p = std::aligned_alloc(256, kNoAllocScratchBytes);
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_mfma_probe(int, int, float*, hipStream_t) {
  ++stub::launches;
  return hipSuccess;
}
hipError_t launch_read_probe(int, const void*, int64_t, float*, hipStream_t) {
  ++stub::launches;
  return hipSuccess;
}

}  // namespace qw
