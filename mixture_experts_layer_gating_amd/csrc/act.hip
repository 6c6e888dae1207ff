// SwiGLU activation between the two expert projections, and its gradient
// [Summary, Method details / key design: optimised activation function].
//
// h[m, :] = [G | U] (gate columns [0, F), up columns [F, 2F));
// a = silu(G) * U, silu(z) = z * sigmoid(z).  Elementwise and HBM-bound:
// each thread handles one 16-byte chunk of G and the matching chunk of U.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kActBlock = 256;

struct alignas(16) V16 {
  uint32_t w[4];
};

template <typename T>
struct Elems {
  static constexpr int N = 16 / sizeof(T);
};

// Streamed loads (STREAM): non-temporal, for inputs read for the last time
// in the pass; the hint keeps them from displacing other data in the caches
// (and made the backward kernel 8% faster on the MI355X).
template <bool STREAM = false, typename T>
__device__ __forceinline__ void load_f32(const T* p, float* f) {
  V16 v;
  if constexpr (STREAM) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) v.w[i] = w[i];
  } else {
    v = *reinterpret_cast<const V16*>(p);
  }
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = lo_bf16(v.w[i]);
      f[2 * i + 1] = hi_bf16(v.w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v.w[i]);
  }
}

template <typename T>
__device__ __forceinline__ void store_f32(T* p, const float* f) {
  V16 v;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v.w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v.w[i] = __float_as_uint(f[i]);
  }
  *reinterpret_cast<V16*>(p) = v;
}

// Flat 32-bit index over (row, 16-byte chunk of the gate half), one chunk per
// thread per grid-stride step.
template <typename T>
__global__ __launch_bounds__(kActBlock) void act_fwd_kernel(const T* __restrict__ h, int M, int F,
                                                            T* __restrict__ a) {
  constexpr int N = Elems<T>::N;
  const int cpr = F / N;
  const int total = M * cpr;
  for (int i = blockIdx.x * kActBlock + threadIdx.x; i < total; i += gridDim.x * kActBlock) {
    const int m = i / cpr, c = i - m * cpr;
    const T* hr = h + static_cast<size_t>(m) * 2 * F + c * N;
    float g[N], u[N], o[N];
    load_f32(hr, g);
    load_f32(hr + F, u);
#pragma unroll
    for (int e = 0; e < N; ++e) o[e] = g[e] * sigmoid_fast(g[e]) * u[e];
    store_f32(a + static_cast<size_t>(m) * F + c * N, o);
  }
}

// dh = [dG | dU] from h and da; with SCALED also the activation itself,
// recomputed from h and scaled by a per-row factor: a_s[m, :] = row_scale[m]
// * silu(G) * U, rounded once.  a_s feeds GEMM 2's weight gradient when the
// combine's gradient is read through the row map instead of being written
// (the gate weight moves from dc to a).  Each thread takes two chunks per
// grid-stride step and issues both chunks' loads before using either (3%
// faster than one chunk at T*k = 128 Ki rows, F = 1536).
template <typename T, bool SCALED>
__global__ __launch_bounds__(kActBlock) void act_bwd_kernel(
    const T* __restrict__ h, const T* __restrict__ da, const float* __restrict__ row_scale, int M,
    int F, T* __restrict__ dh, T* __restrict__ a_s) {
  constexpr int N = Elems<T>::N;
  const int cpr = F / N;
  const int total = M * cpr;
  const int stride = gridDim.x * kActBlock;
  for (int i0 = blockIdx.x * kActBlock + threadIdx.x; i0 < total; i0 += 2 * stride) {
    float g[2][N], u[2][N], d[2][N], rs[2];
    int m[2], c[2];
    bool live[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      // A chunk past the end repeats chunk i0's loads and is not stored.
      const int i = i0 + r * stride;
      live[r] = i < total;
      m[r] = (live[r] ? i : i0) / cpr;
      c[r] = (live[r] ? i : i0) - m[r] * cpr;
      const T* hr = h + static_cast<size_t>(m[r]) * 2 * F + c[r] * N;
      load_f32<true>(hr, g[r]);  // h and da are not read again in the pass
      load_f32<true>(hr + F, u[r]);
      load_f32<true>(da + static_cast<size_t>(m[r]) * F + c[r] * N, d[r]);
      rs[r] = SCALED ? row_scale[m[r]] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (!live[r]) continue;
      float dg[N], du[N], o[N];
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float s = sigmoid_fast(g[r][e]);
        dg[e] = d[r][e] * u[r][e] * s * (1.f + g[r][e] * (1.f - s));
        du[e] = d[r][e] * g[r][e] * s;
        o[e] = rs[r] * (g[r][e] * s * u[r][e]);
      }
      T* dr = dh + static_cast<size_t>(m[r]) * 2 * F + c[r] * N;
      store_f32(dr, dg);
      store_f32(dr + F, du);
      if constexpr (SCALED) store_f32(a_s + static_cast<size_t>(m[r]) * F + c[r] * N, o);
    }
  }
}

int act_grid(int M, int F, moe_dtype dt) {
  // One chunk per thread, capped at 32 workgroups per compute unit.
  const long long chunks = static_cast<long long>(M) * F * static_cast<long long>(dtype_size(dt)) / 16;
  long long b = (chunks + kActBlock - 1) / kActBlock;
  if (b > 256LL * 32) b = 256LL * 32;
  return static_cast<int>(b < 1 ? 1 : b);
}

moe_status check_act(int M, int F, moe_dtype dt) {
  MOE_REQUIRE(M >= 1 && F >= 1, MOE_ERR_INVALID_ARG, "M and F must be >= 1");
  MOE_REQUIRE(static_cast<long long>(M) * F < (1ll << 31), MOE_ERR_UNSUPPORTED,
              "M*F must be < 2^31");
  MOE_REQUIRE(dtype_ok(dt), MOE_ERR_UNSUPPORTED, "unknown dtype");
  MOE_REQUIRE(F % 8 == 0, MOE_ERR_UNSUPPORTED, "F must be a multiple of 8");
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_act_fwd(const void* h, int M, int F, moe_dtype dtype, void* a,
                                  moe_stream_t stream) {
  clear_error();
  if (moe_status s = check_act(M, F, dtype)) return s;
  MOE_REQUIRE(h && a, MOE_ERR_INVALID_ARG, "moe_act_fwd: null pointer");
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(act_fwd_kernel<uint16_t>, dim3(act_grid(M, F, dtype)), dim3(kActBlock), 0,
                       as_stream(stream), static_cast<const uint16_t*>(h), M, F,
                       static_cast<uint16_t*>(a));
  else
    hipLaunchKernelGGL(act_fwd_kernel<float>, dim3(act_grid(M, F, dtype)), dim3(kActBlock), 0,
                       as_stream(stream), static_cast<const float*>(h), M, F,
                       static_cast<float*>(a));
  return check_launch("moe_act_fwd");
}

extern "C" moe_status moe_act_bwd(const void* h, const void* da, int M, int F, moe_dtype dtype,
                                  void* dh, moe_stream_t stream) {
  clear_error();
  if (moe_status s = check_act(M, F, dtype)) return s;
  MOE_REQUIRE(h && da && dh, MOE_ERR_INVALID_ARG, "moe_act_bwd: null pointer");
  const dim3 grid(act_grid(M, F, dtype)), block(kActBlock);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL((act_bwd_kernel<uint16_t, false>), grid, block, 0, as_stream(stream),
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(da), nullptr,
                       M, F, static_cast<uint16_t*>(dh), nullptr);
  else
    hipLaunchKernelGGL((act_bwd_kernel<float, false>), grid, block, 0, as_stream(stream),
                       static_cast<const float*>(h), static_cast<const float*>(da), nullptr, M, F,
                       static_cast<float*>(dh), nullptr);
  return check_launch("moe_act_bwd");
}

extern "C" moe_status moe_act_bwd_scaled(const void* h, const void* da, const float* row_scale,
                                         int M, int F, moe_dtype dtype, void* dh, void* a_scaled,
                                         moe_stream_t stream) {
  clear_error();
  if (moe_status s = check_act(M, F, dtype)) return s;
  MOE_REQUIRE(h && da && row_scale && dh && a_scaled, MOE_ERR_INVALID_ARG,
              "moe_act_bwd_scaled: null pointer");
  const dim3 grid(act_grid(M, F, dtype)), block(kActBlock);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL((act_bwd_kernel<uint16_t, true>), grid, block, 0, as_stream(stream),
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(da),
                       row_scale, M, F, static_cast<uint16_t*>(dh),
                       static_cast<uint16_t*>(a_scaled));
  else
    hipLaunchKernelGGL((act_bwd_kernel<float, true>), grid, block, 0, as_stream(stream),
                       static_cast<const float*>(h), static_cast<const float*>(da), row_scale, M,
                       F, static_cast<float*>(dh), static_cast<float*>(a_scaled));
  return check_launch("moe_act_bwd_scaled");
}
