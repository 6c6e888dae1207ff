// Internal helpers shared by the library's translation units: error state,
// argument checks, bf16 conversion and wave-level primitives for gfx950
// (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- errors
void set_error(const std::string& msg);
void clear_error();

inline moe_status fail(moe_status st, const std::string& msg) {
  set_error(msg);
  return st;
}

// Checks the launch that was just enqueued.
moe_status check_launch(const char* what);

#define MOE_REQUIRE(cond, status, msg)             \
  do {                                             \
    if (!(cond)) return ::moe::fail((status), (msg)); \
  } while (0)

inline hipStream_t as_stream(moe_stream_t s) {
  return reinterpret_cast<hipStream_t>(s);
}

// ---------------------------------------------------------------- index record
// Out-of-range indices met by this translation unit's kernels: MOE_IDXERR_*
// bits, OR-ed in by the kernel that met one.  Each unit (and each device) has
// its own copy; moe_index_errors reads and clears them all.
[[maybe_unused]] static __device__ unsigned int g_index_flags;

__device__ __forceinline__ void note_index_error(unsigned int bits) {
  atomicOr(&g_index_flags, bits);
}

// Host side: this unit's record on the current device, copied on `st`, which
// is then waited for; cleared afterwards when `clear` is set.
[[maybe_unused]] static moe_status take_index_flags(hipStream_t st, unsigned int* bits,
                                                    bool clear) {
  unsigned int v = 0;
  hipError_t e =
      hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_index_flags), sizeof v, 0, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess && clear && v != 0) {
    static const unsigned int zero = 0;
    e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_index_flags), &zero, sizeof zero, 0,
                               hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
  }
  if (e != hipSuccess) return fail(MOE_ERR_HIP, std::string("moe_index_errors: ") + hipGetErrorString(e));
  *bits |= v;
  return MOE_OK;
}

// The units whose kernels read indices from caller buffers.
moe_status index_record_route(hipStream_t st, unsigned int* bits, bool clear);
moe_status index_record_count(hipStream_t st, unsigned int* bits, bool clear);
moe_status index_record_move(hipStream_t st, unsigned int* bits, bool clear);
moe_status index_record_gemm(hipStream_t st, unsigned int* bits, bool clear);

inline size_t dtype_size(moe_dtype t) { return t == MOE_BF16 ? 2 : 4; }
inline bool dtype_ok(moe_dtype t) { return t == MOE_F32 || t == MOE_BF16; }

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
// bf16 values are carried as raw 16-bit patterns.
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest, ties to even; NaN stays NaN (quiet).  gfx950 converts in
// one instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> two packed bf16 in one dword (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- math
// sigmoid(z) = 1 / (1 + e^-z) from the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32; about 1 ulp each).  Saturates to 0 / 1 for large
// |z|.  Every kernel that evaluates SwiGLU uses this one, so fused and
// separate evaluations agree bit for bit.
__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum across the 64 lanes.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
}

}  // namespace moe
