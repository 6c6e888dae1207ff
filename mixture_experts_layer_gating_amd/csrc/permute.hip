// Token permutation into expert-contiguous order, the weighted combine back
// to token order, and the combine's backward pass.
//
// The grouped GEMM consumes the tokens of each expert as one contiguous block
// of rows [Brief, Core method]; these kernels move rows between token order
// and that expert-sorted order.  They are HBM-bound: every thread moves
// 16-byte chunks, consecutive threads take consecutive chunks of a row, so
// each row is read and written as whole cache lines.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMoveBlock = 256;

struct alignas(16) Vec16 {
  uint32_t w[4];
};

// Loads of rows that the kernel streams through are non-temporal: each
// chunk is read once here, and the hint keeps the streamed bytes from
// displacing other data in the caches (it also made these kernels 8-14%
// faster on the MI355X).
__device__ __forceinline__ Vec16 ld16_stream(const void* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  Vec16 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.w[i] = w[i];
  return v;
}
__device__ __forceinline__ void st16(void* p, const Vec16& v) {
  *reinterpret_cast<Vec16*>(p) = v;
}

// Elements per 16-byte chunk: 8 bf16 or 4 fp32.
template <typename T>
struct Chunk;
template <>
struct Chunk<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(const Vec16& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = lo_bf16(v.w[i]);
      f[2 * i + 1] = hi_bf16(v.w[i]);
    }
  }
  __device__ static Vec16 pack(const float* f) {
    Vec16 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v.w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
  }
};
template <>
struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static void unpack(const Vec16& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v.w[i]);
  }
  __device__ static Vec16 pack(const float* f) {
    Vec16 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v.w[i] = __float_as_uint(f[i]);
    return v;
  }
};

// A dest entry names a row of the T*k-row permuted array; one outside it
// (a caller error) is neither read nor written, and is recorded.
__device__ __forceinline__ bool row_ok(int d, unsigned rows) {
  return static_cast<unsigned>(d) < rows;
}

// xp[dest[t*k + j], :] = x[t, :] for every slot (t, j): each token row is
// read once and written to its k rows (the same result as gathering
// xp[p] = x[src[p] / k]).  One workgroup per token row, threads on
// consecutive 16-byte chunks; stores do not wait, so k of them per load keep
// the memory system busy.
__global__ __launch_bounds__(kMoveBlock) void permute_kernel(const char* __restrict__ x,
                                                             const int32_t* __restrict__ dest,
                                                             int Tn, int k, int chunks_per_row,
                                                             char* __restrict__ xp) {
  const size_t row_bytes = static_cast<size_t>(chunks_per_row) * 16;
  const unsigned rows = static_cast<unsigned>(Tn) * static_cast<unsigned>(k);
  bool bad = false;
  for (int t = blockIdx.x; t < Tn; t += gridDim.x) {
    const char* in = x + static_cast<size_t>(t) * row_bytes;
    const int32_t* drow = dest + static_cast<size_t>(t) * k;
    for (int c = threadIdx.x; c < chunks_per_row; c += kMoveBlock) {
      const Vec16 v = ld16_stream(in + c * 16);
      for (int j = 0; j < k; ++j) {
        const int d = drow[j];
        if (row_ok(d, rows))
          st16(xp + static_cast<size_t>(d) * row_bytes + c * 16, v);
        else
          bad = true;
      }
    }
  }
  if (bad) note_index_error(MOE_IDXERR_ROW);
}

constexpr int kUnroll = 8;  // slots whose loads are issued together

// y[t, :] = sum_j w[t, j] * yp[dest[t*k + j], :]  (w == nullptr -> weight 1)
// with fp32 accumulation in increasing j.  One workgroup per output row; the
// loads of up to 8 slots are issued before any of them is used.
template <typename T>
__global__ __launch_bounds__(kMoveBlock) void unpermute_kernel(const char* __restrict__ yp,
                                                               const int32_t* __restrict__ dest,
                                                               const float* __restrict__ w,
                                                               int Tn, int k, int chunks_per_row,
                                                               char* __restrict__ y) {
  constexpr int N = Chunk<T>::N;
  const size_t row_bytes = static_cast<size_t>(chunks_per_row) * 16;
  const unsigned rows = static_cast<unsigned>(Tn) * static_cast<unsigned>(k);
  bool bad = false;
  for (int t = blockIdx.x; t < Tn; t += gridDim.x) {
    const int32_t* drow = dest + static_cast<size_t>(t) * k;
    const float* wrow = w ? w + static_cast<size_t>(t) * k : nullptr;
    for (int c = threadIdx.x; c < chunks_per_row; c += kMoveBlock) {
      float acc[N];
#pragma unroll
      for (int q = 0; q < N; ++q) acc[q] = 0.f;
      for (int j0 = 0; j0 < k; j0 += kUnroll) {
        Vec16 raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (j0 + u < k) {
            // An out-of-range row reads row 0 and contributes zeros.
            const int d = drow[j0 + u];
            const bool ok = row_ok(d, rows);
            bad |= !ok;
            raw[u] = ld16_stream(yp + static_cast<size_t>(ok ? d : 0) * row_bytes + c * 16);
            if (!ok) raw[u] = Vec16{};
          }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (j0 + u < k) {
            const float wt = wrow ? wrow[j0 + u] : 1.f;
            float v[N];
            Chunk<T>::unpack(raw[u], v);
#pragma unroll
            for (int q = 0; q < N; ++q) acc[q] = fmaf(wt, v[q], acc[q]);
          }
        }
      }
      st16(y + static_cast<size_t>(t) * row_bytes + c * 16, Chunk<T>::pack(acc));
    }
  }
  if (bad) note_index_error(MOE_IDXERR_ROW);
}

// One block per token: dyp rows of its k slots (unless !WRITE_DYP) and the
// k dot products dw.
template <typename T, bool WRITE_DYP>
__global__ __launch_bounds__(kMoveBlock) void unpermute_bwd_kernel(
    const char* __restrict__ dy, const char* __restrict__ yp, const int32_t* __restrict__ dest,
    const float* __restrict__ w, int k, unsigned rows, int chunks_per_row,
    char* __restrict__ dyp, float* __restrict__ dw) {
  constexpr int N = Chunk<T>::N;
  __shared__ float part[kMoveBlock / kWave][MOE_MAX_TOPK];
  const int t = blockIdx.x;
  const size_t row_bytes = static_cast<size_t>(chunks_per_row) * 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const char* dyrow = dy + static_cast<size_t>(t) * row_bytes;
  const int32_t* drow = dest + static_cast<size_t>(t) * k;
  const float* wrow = w + static_cast<size_t>(t) * k;
  float dot[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) dot[j] = 0.f;
  bool bad = false;
  for (int c = threadIdx.x; c < chunks_per_row; c += kMoveBlock) {
    float g[N];
    Chunk<T>::unpack(ld16_stream(dyrow + c * 16), g);
#pragma unroll
    for (int j0 = 0; j0 < MOE_MAX_TOPK; j0 += kUnroll) {
      if (j0 >= k) break;
      Vec16 raw[kUnroll];
      int dd[kUnroll];
      bool ok[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (j0 + u < k) {
          // An out-of-range row is not written and reads as zeros (dw gets
          // nothing from it).
          dd[u] = drow[j0 + u];
          ok[u] = row_ok(dd[u], rows);
          bad |= !ok[u];
          raw[u] = ld16_stream(yp + static_cast<size_t>(ok[u] ? dd[u] : 0) * row_bytes + c * 16);
          if (!ok[u]) raw[u] = Vec16{};
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (j0 + u < k) {
          const float wt = wrow[j0 + u];
          float v[N], o[N];
          Chunk<T>::unpack(raw[u], v);
#pragma unroll
          for (int q = 0; q < N; ++q) {
            dot[j0 + u] = fmaf(g[q], v[q], dot[j0 + u]);
            o[q] = wt * g[q];
          }
          if (WRITE_DYP && ok[u])
            st16(dyp + static_cast<size_t>(dd[u]) * row_bytes + c * 16, Chunk<T>::pack(o));
        }
      }
    }
  }
  if (bad) note_index_error(MOE_IDXERR_ROW);
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j < k) {
      const float v = wave_sum(dot[j]);
      if (lane == 0) part[wid][j] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < k) {
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < kMoveBlock / kWave; ++q) acc += part[q][threadIdx.x];
    dw[static_cast<size_t>(t) * k + threadIdx.x] = acc;
  }
}

// out[p] = w[src[p]]: the gate weights in the expert-sorted row order (one
// float per row; an entry of src outside [0, n) gives 0 and is recorded).
__global__ __launch_bounds__(kMoveBlock) void gather_scale_kernel(const float* __restrict__ w,
                                                                  const int32_t* __restrict__ src,
                                                                  int n, float* __restrict__ out) {
  bool bad = false;
  for (int p = blockIdx.x * kMoveBlock + threadIdx.x; p < n; p += gridDim.x * kMoveBlock) {
    const int s = src[p];
    const bool ok = row_ok(s, static_cast<unsigned>(n));
    bad |= !ok;
    out[p] = ok ? w[s] : 0.f;
  }
  if (bad) note_index_error(MOE_IDXERR_ROW);
}

int row_grid(long long rows) {
  // One workgroup per row, capped at 32 per compute unit (256 CUs).
  long long b = rows;
  if (b > 256LL * 32) b = 256LL * 32;
  return static_cast<int>(b < 1 ? 1 : b);
}

moe_status check_move(int T, int k, int d, moe_dtype dt) {
  MOE_REQUIRE(T >= 1 && k >= 1 && d >= 1, MOE_ERR_INVALID_ARG, "T, k, d must be >= 1");
  MOE_REQUIRE(k <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED, "k exceeds 32");
  MOE_REQUIRE(dtype_ok(dt), MOE_ERR_UNSUPPORTED, "unknown dtype");
  MOE_REQUIRE(d % 8 == 0, MOE_ERR_UNSUPPORTED, "d must be a multiple of 8");
  MOE_REQUIRE(static_cast<long long>(T) * k < (1ll << 31), MOE_ERR_UNSUPPORTED,
              "T*k must be < 2^31");
  return MOE_OK;
}

}  // namespace

moe_status index_record_move(hipStream_t st, unsigned int* bits, bool clear) {
  return take_index_flags(st, bits, clear);
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_permute(const void* x, const int32_t* dest, int T, int k, int d,
                                  moe_dtype dtype, void* xp, moe_stream_t stream) {
  clear_error();
  if (moe_status s = check_move(T, k, d, dtype)) return s;
  MOE_REQUIRE(x && dest && xp, MOE_ERR_INVALID_ARG, "moe_permute: null pointer");
  const int cpr = static_cast<int>(d * dtype_size(dtype) / 16);
  hipLaunchKernelGGL(permute_kernel, dim3(row_grid(T)), dim3(kMoveBlock), 0, as_stream(stream),
                     static_cast<const char*>(x), dest, T, k, cpr, static_cast<char*>(xp));
  return check_launch("moe_permute");
}

extern "C" moe_status moe_unpermute(const void* yp, const int32_t* dest, const float* w, int T,
                                    int k, int d, moe_dtype dtype, void* y, moe_stream_t stream) {
  clear_error();
  if (moe_status s = check_move(T, k, d, dtype)) return s;
  MOE_REQUIRE(yp && dest && y, MOE_ERR_INVALID_ARG, "moe_unpermute: null pointer");
  const int cpr = static_cast<int>(d * dtype_size(dtype) / 16);
  const dim3 grid(row_grid(T));
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(unpermute_kernel<uint16_t>, grid, dim3(kMoveBlock), 0, as_stream(stream),
                       static_cast<const char*>(yp), dest, w, T, k, cpr, static_cast<char*>(y));
  else
    hipLaunchKernelGGL(unpermute_kernel<float>, grid, dim3(kMoveBlock), 0, as_stream(stream),
                       static_cast<const char*>(yp), dest, w, T, k, cpr, static_cast<char*>(y));
  return check_launch("moe_unpermute");
}

extern "C" moe_status moe_unpermute_bwd(const void* dy, const void* yp, const int32_t* dest,
                                        const float* w, int T, int k, int d, moe_dtype dtype,
                                        void* dyp, float* dw, moe_stream_t stream) {
  clear_error();
  if (moe_status s = check_move(T, k, d, dtype)) return s;
  MOE_REQUIRE(dy && yp && dest && w && dw, MOE_ERR_INVALID_ARG,
              "moe_unpermute_bwd: null pointer");
  const int cpr = static_cast<int>(d * dtype_size(dtype) / 16);
  const unsigned rows = static_cast<unsigned>(T) * static_cast<unsigned>(k);
  const dim3 grid(T), block(kMoveBlock);
  hipStream_t st = as_stream(stream);
  const char* dyc = static_cast<const char*>(dy);
  const char* ypc = static_cast<const char*>(yp);
  char* dypc = static_cast<char*>(dyp);
#define MOE_UBWD(TT, WD)                                                                       \
  hipLaunchKernelGGL((unpermute_bwd_kernel<TT, WD>), grid, block, 0, st, dyc, ypc, dest, w, k, \
                     rows, cpr, dypc, dw)
  if (dtype == MOE_BF16) {
    if (dyp) MOE_UBWD(uint16_t, true); else MOE_UBWD(uint16_t, false);
  } else {
    if (dyp) MOE_UBWD(float, true); else MOE_UBWD(float, false);
  }
#undef MOE_UBWD
  return check_launch("moe_unpermute_bwd");
}

extern "C" moe_status moe_gather_scale(const float* w, const int32_t* src, int n, float* out,
                                       moe_stream_t stream) {
  clear_error();
  MOE_REQUIRE(n >= 1, MOE_ERR_INVALID_ARG, "moe_gather_scale: n must be >= 1");
  MOE_REQUIRE(w && src && out, MOE_ERR_INVALID_ARG, "moe_gather_scale: null pointer");
  long long g = (static_cast<long long>(n) + kMoveBlock - 1) / kMoveBlock;
  if (g > 2048) g = 2048;
  hipLaunchKernelGGL(gather_scale_kernel, dim3(static_cast<unsigned>(g)), dim3(kMoveBlock), 0,
                     as_stream(stream), w, src, n, out);
  return check_launch("moe_gather_scale");
}
