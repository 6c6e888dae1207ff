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
// arg-max; nothing is written to global memory but the outputs.  With at
// most 64 experts a token takes 8 lanes instead (8 tokens per wavefront,
// lane g of a group holding experts g*V .. g*V + V - 1, V = ceil(E / 8)):
// the same k rounds, each a scan of V registers and a 3-step arg-max across
// the group, at an eighth of the wavefronts.
#include <float.h>
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteBlock = 256;  // 4 tokens per block

// Order used for selection: larger value first, then lower index.  A NaN
// ranks below every number (-inf included) and NaNs among themselves by
// index, so a token whose logits hold NaNs still gets k distinct ids in
// [0, E) -- the order of a stable descending sort that puts NaNs last.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  const bool na = va != va, nb = vb != vb;
  if (na || nb) return nb && (!na || ia < ib);
  return (va > vb) || (va == vb && ia < ib);
}

// Start of an arg-max: worse than every candidate (NaN, with an index above
// any expert's).
constexpr int kNoExpert = 0x7fffffff;

// An expert id read from a caller's buffer (forced ids, the backward pass's
// topk_idx) outside [0, E) is a caller error; it is clamped so that no read
// or row index derived from it leaves its buffer, and recorded.
__device__ __forceinline__ int clamp_expert(int e, int E) {
  if (e >= 0 && e < E) return e;
  note_index_error(MOE_IDXERR_EXPERT);
  return e < 0 ? 0 : E - 1;
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
      const int e = clamp_expert(forced[static_cast<size_t>(t) * k + lane], E);
      float v = row[e];
      if (bias) v = v + bias[e];
      my_id = e;
      my_p = expf(v - m) / s;
    }
  } else {
    uint32_t taken = 0;  // bit i: register slot i already selected
    for (int j = 0; j < k; ++j) {
      float bv = __builtin_nanf("");
      int bi = kNoExpert;
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

// At most 64 experts: 8 lanes per token (see the layout note above).  Same
// definitions as route_topk_kernel; the softmax sum is taken in a different
// order (per lane, then across the 8 lanes).
constexpr int kGroup = 8;  // lanes per token

template <int V>
__global__ __launch_bounds__(kRouteBlock) void route_topk_small_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E,
    int k, int renorm, const int32_t* __restrict__ forced, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, float* __restrict__ probs) {
  constexpr int kSlots = MOE_MAX_TOPK / kGroup;  // output slots per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane & (kGroup - 1);
  const int t = blockIdx.x * (kRouteBlock / kGroup) + static_cast<int>(threadIdx.x / kGroup);
  // Whole groups leave together (all 8 lanes share t), so the shuffles below
  // only ever read lanes of live groups.
  if (t >= T) return;
  const float* row = logits + static_cast<size_t>(t) * E;

  float z[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = g * V + v;
    if (e < E) {
      float x = row[e];
      if (bias) x = x + bias[e];
      z[v] = x;
    } else {
      z[v] = -INFINITY;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int v = 0; v < V; ++v) m = fmaxf(m, z[v]);
#pragma unroll
  for (int o = kGroup / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  float ex[V];
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    ex[v] = (g * V + v < E) ? expf(z[v] - m) : 0.f;
    s += ex[v];
  }
#pragma unroll
  for (int o = kGroup / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (probs) {
    float* prow = probs + static_cast<size_t>(t) * E;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (g * V + v < E) prow[g * V + v] = ex[v] / s;
  }

  // Slot j goes to lane j % 8 of the group, register j / 8.
  int my_id[kSlots];
  float my_p[kSlots];
#pragma unroll
  for (int q = 0; q < kSlots; ++q) {
    my_id[q] = 0;
    my_p[q] = 0.f;
  }
  if (forced) {
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      const int j = q * kGroup + g;
      if (j < k) {
        const int e = clamp_expert(forced[static_cast<size_t>(t) * k + j], E);
        float x = row[e];
        if (bias) x = x + bias[e];
        my_id[q] = e;
        my_p[q] = expf(x - m) / s;
      }
    }
  } else {
    uint32_t taken = 0;  // bit v: register v already selected
    for (int j = 0; j < k; ++j) {
      float bv = __builtin_nanf("");
      int bi = kNoExpert;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int e = g * V + v;
        if (e < E && !(taken & (1u << v)) && better(z[v], e, bv, bi)) {
          bv = z[v];
          bi = e;
        }
      }
#pragma unroll
      for (int o = kGroup / 2; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      // Every lane of the group now holds the winner (bv, bi).
      if (bi / V == g) taken |= 1u << (bi - g * V);
      if ((j & (kGroup - 1)) == g) {
        const float p = expf(bv - m) / s;
#pragma unroll
        for (int q = 0; q < kSlots; ++q)
          if (q == j / kGroup) {
            my_id[q] = bi;
            my_p[q] = p;
          }
      }
    }
  }
  if (renorm) {
    // Sum over j in increasing order, identical in every lane of the group.
    const int base = lane & ~(kGroup - 1);
    float tot = 0.f;
    for (int j = 0; j < k; ++j) {
      float pj = 0.f;
#pragma unroll
      for (int q = 0; q < kSlots; ++q) {
        const float x = __shfl(my_p[q], base + (j & (kGroup - 1)), kWave);
        if (q == j / kGroup) pj = x;
      }
      tot += pj;
    }
#pragma unroll
    for (int q = 0; q < kSlots; ++q) my_p[q] = my_p[q] / tot;
  }
#pragma unroll
  for (int q = 0; q < kSlots; ++q) {
    const int j = q * kGroup + g;
    if (j < k) {
      idx_out[static_cast<size_t>(t) * k + j] = my_id[q];
      w_out[static_cast<size_t>(t) * k + j] = my_p[q];
    }
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
    my_id = clamp_expert(irow[lane], E);
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
  hipStream_t st = as_stream(stream);
  if (E <= kWave) {
    // 8 lanes per token, 32 tokens per block
    const dim3 g8((T + kRouteBlock / kGroup - 1) / (kRouteBlock / kGroup));
    const int v = (E + kGroup - 1) / kGroup;
#define MOE_SMALL(VV)                                                                         \
  hipLaunchKernelGGL(route_topk_small_kernel<VV>, g8, dim3(kRouteBlock), 0, st, logits, bias, T, \
                     E, k, renorm, forced_idx, topk_idx, topk_w, probs)
    if (v <= 1) MOE_SMALL(1);
    else if (v <= 2) MOE_SMALL(2);
    else if (v <= 4) MOE_SMALL(4);
    else MOE_SMALL(8);
#undef MOE_SMALL
    return check_launch("moe_route_topk");
  }
  const dim3 grid((T + 3) / 4);
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

namespace moe {
moe_status index_record_route(hipStream_t st, unsigned int* bits, bool clear) {
  return take_index_flags(st, bits, clear);
}
}  // namespace moe
