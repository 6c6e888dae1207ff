// Softmax top-k expert selection and its backward pass.
//
// Expert selection is the first step of the MoE forward pass [Summary,
// Method details / technical framework].  Definitions used: softmax over all
// E experts of z = logits + bias; slot j takes the j-th largest z, ties to
// the lower expert index; weights are the selected probabilities, optionally
// renormalised; a forced assignment (forced uniform routing, [Brief,
// Limitations]) replaces the selection.
//
// Layout: one 64-lane wavefront per token, expert e held by lane e % 64 in
// register slot e / 64.  Selection is k rounds of a wave-wide (value, index)
// arg-max; nothing is written to global memory but the outputs.
#include <float.h>
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteBlock = 256;  // 4 tokens per block

// Order used for selection: larger value first, then lower index.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return (va > vb) || (va == vb && ia < ib);
}

template <int EPL>
__global__ __launch_bounds__(kRouteBlock) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E,
    int k, int renorm, const int32_t* __restrict__ forced, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, float* __restrict__ probs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kRouteBlock / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const float* row = logits + static_cast<size_t>(t) * E;

  float z[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    if (e < E) {
      float v = row[e];
      if (bias) v = v + bias[e];
      z[i] = v;
    } else {
      z[i] = -INFINITY;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) m = fmaxf(m, z[i]);
  m = wave_max(m);
  float ex[EPL];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    ex[i] = (e < E) ? expf(z[i] - m) : 0.f;
    s += ex[i];
  }
  s = wave_sum(s);
  if (probs) {
    float* prow = probs + static_cast<size_t>(t) * E;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = i * kWave + lane;
      if (e < E) prow[e] = ex[i] / s;
    }
  }

  // Selected ids and their (unnormalised) probabilities, kept in lane j.
  int my_id = 0;
  float my_p = 0.f;
  if (forced) {
    if (lane < k) {
      const int e = forced[static_cast<size_t>(t) * k + lane];
      float v = row[e];
      if (bias) v = v + bias[e];
      my_id = e;
      my_p = expf(v - m) / s;
    }
  } else {
    uint32_t taken = 0;  // bit i: register slot i already selected
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = i * kWave + lane;
        if (e < E && !(taken & (1u << i)) && better(z[i], e, bv, bi)) {
          bv = z[i];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      // Every lane now holds the winner (bv, bi).
      if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
      if (lane == j) {
        my_id = bi;
        my_p = expf(bv - m) / s;
      }
    }
  }
  if (renorm) {
    // Sum over j in increasing order, identical in every lane.
    float tot = 0.f;
    for (int j = 0; j < k; ++j) tot += __shfl(my_p, j, kWave);
    my_p = my_p / tot;
  }
  if (lane < k) {
    idx_out[static_cast<size_t>(t) * k + lane] = my_id;
    w_out[static_cast<size_t>(t) * k + lane] = my_p;
  }
}

template <int EPL, typename OutT>
__global__ __launch_bounds__(kRouteBlock) void route_topk_bwd_kernel(
    const float* __restrict__ probs, const int32_t* __restrict__ idx,
    const float* __restrict__ dw, int T, int E, int k, int renorm, OutT* __restrict__ dz) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kRouteBlock / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const float* prow = probs + static_cast<size_t>(t) * E;
  const int32_t* irow = idx + static_cast<size_t>(t) * k;
  const float* drow = dw + static_cast<size_t>(t) * k;

  // Lane j < k holds slot j: its expert, probability and d(prob).
  int my_id = 0;
  float my_p = 0.f, my_dw = 0.f;
  if (lane < k) {
    my_id = irow[lane];
    my_p = prow[my_id];
    my_dw = drow[lane];
  }
  float my_dp = my_dw;
  if (renorm) {
    float S = 0.f;
    for (int j = 0; j < k; ++j) S += __shfl(my_p, j, kWave);
    float c = 0.f;
    for (int j = 0; j < k; ++j) c += __shfl(my_dw, j, kWave) * (__shfl(my_p, j, kWave) / S);
    my_dp = (my_dw - c) / S;
  }
  // <p, dp> over the selected experts only (dp is zero elsewhere).
  float pdp = (lane < k) ? my_p * my_dp : 0.f;
  pdp = wave_sum(pdp);

  float dp[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) dp[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = __shfl(my_id, j, kWave);
    const float v = __shfl(my_dp, j, kWave);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (e == i * kWave + lane) dp[i] += v;
  }
  OutT* zrow = dz + static_cast<size_t>(t) * E;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    if (e < E) {
      const float g = prow[e] * (dp[i] - pdp);
      if constexpr (sizeof(OutT) == 2)
        zrow[e] = f32_to_bf16(g);
      else
        zrow[e] = g;
    }
  }
}

template <int EPL>
void launch_route(int T, dim3 grid, hipStream_t st, const float* logits, const float* bias,
                  int E, int k, int renorm, const int32_t* forced, int32_t* idx, float* w,
                  float* probs) {
  hipLaunchKernelGGL(route_topk_kernel<EPL>, grid, dim3(kRouteBlock), 0, st, logits, bias, T, E,
                     k, renorm, forced, idx, w, probs);
}

template <int EPL>
void launch_route_bwd(int T, dim3 grid, hipStream_t st, const float* probs, const int32_t* idx,
                      const float* dw, int E, int k, int renorm, void* dz, moe_dtype dt) {
  if (dt == MOE_BF16)
    hipLaunchKernelGGL((route_topk_bwd_kernel<EPL, uint16_t>), grid, dim3(kRouteBlock), 0, st,
                       probs, idx, dw, T, E, k, renorm, static_cast<uint16_t*>(dz));
  else
    hipLaunchKernelGGL((route_topk_bwd_kernel<EPL, float>), grid, dim3(kRouteBlock), 0, st,
                       probs, idx, dw, T, E, k, renorm, static_cast<float*>(dz));
}

moe_status check_route_sizes(int T, int E, int k) {
  MOE_REQUIRE(T >= 1, MOE_ERR_INVALID_ARG, "T must be >= 1");
  MOE_REQUIRE(E >= 1, MOE_ERR_INVALID_ARG, "E must be >= 1");
  MOE_REQUIRE(E <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, "E exceeds 1024");
  MOE_REQUIRE(k >= 1 && k <= E, MOE_ERR_INVALID_ARG, "need 1 <= k <= E");
  MOE_REQUIRE(k <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED, "k exceeds 32");
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route_topk(const float* logits, const float* bias, int T, int E, int k,
                                     int renorm, const int32_t* forced_idx, int32_t* topk_idx,
                                     float* topk_w, float* probs, moe_stream_t stream) {
  clear_error();
  if (moe_status st = check_route_sizes(T, E, k)) return st;
  MOE_REQUIRE(logits && topk_idx && topk_w, MOE_ERR_INVALID_ARG,
              "moe_route_topk: null logits/topk_idx/topk_w");
  const dim3 grid((T + 3) / 4);
  hipStream_t st = as_stream(stream);
  const int epl = (E + kWave - 1) / kWave;
  if (epl <= 1)
    launch_route<1>(T, grid, st, logits, bias, E, k, renorm, forced_idx, topk_idx, topk_w, probs);
  else if (epl <= 2)
    launch_route<2>(T, grid, st, logits, bias, E, k, renorm, forced_idx, topk_idx, topk_w, probs);
  else if (epl <= 4)
    launch_route<4>(T, grid, st, logits, bias, E, k, renorm, forced_idx, topk_idx, topk_w, probs);
  else if (epl <= 8)
    launch_route<8>(T, grid, st, logits, bias, E, k, renorm, forced_idx, topk_idx, topk_w, probs);
  else
    launch_route<16>(T, grid, st, logits, bias, E, k, renorm, forced_idx, topk_idx, topk_w, probs);
  return check_launch("moe_route_topk");
}

extern "C" moe_status moe_route_topk_bwd(const float* probs, const int32_t* topk_idx,
                                         const float* dtopk_w, int T, int E, int k, int renorm,
                                         void* dlogits, moe_dtype dlogits_dtype,
                                         moe_stream_t stream) {
  clear_error();
  if (moe_status st = check_route_sizes(T, E, k)) return st;
  MOE_REQUIRE(probs && topk_idx && dtopk_w && dlogits, MOE_ERR_INVALID_ARG,
              "moe_route_topk_bwd: null pointer");
  MOE_REQUIRE(dtype_ok(dlogits_dtype), MOE_ERR_UNSUPPORTED, "moe_route_topk_bwd: bad dtype");
  const dim3 grid((T + 3) / 4);
  hipStream_t st = as_stream(stream);
  const int epl = (E + kWave - 1) / kWave;
  if (epl <= 1)
    launch_route_bwd<1>(T, grid, st, probs, topk_idx, dtopk_w, E, k, renorm, dlogits, dlogits_dtype);
  else if (epl <= 2)
    launch_route_bwd<2>(T, grid, st, probs, topk_idx, dtopk_w, E, k, renorm, dlogits, dlogits_dtype);
  else if (epl <= 4)
    launch_route_bwd<4>(T, grid, st, probs, topk_idx, dtopk_w, E, k, renorm, dlogits, dlogits_dtype);
  else if (epl <= 8)
    launch_route_bwd<8>(T, grid, st, probs, topk_idx, dtopk_w, E, k, renorm, dlogits, dlogits_dtype);
  else
    launch_route_bwd<16>(T, grid, st, probs, topk_idx, dtopk_w, E, k, renorm, dlogits, dlogits_dtype);
  return check_launch("moe_route_topk_bwd");
}
