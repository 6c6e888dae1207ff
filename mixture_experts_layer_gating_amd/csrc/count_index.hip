// Token counting and index generation [Brief, Core method: dedicated GPU
// kernels count each expert's tokens and generate the indices that feed the
// grouped GEMM].
//
// Output (flat slot s = t*k + j, expert topk_idx[s]):
//   counts[e], offsets[e] (exclusive scan, offsets[E] = T*k),
//   dest[s] = row of slot s in expert-sorted order, src = inverse of dest.
// Inside an expert's rows the slots keep increasing s (a stable sort), which
// makes the result unique and deterministic.  No global atomics are used;
// ranks come from wavefront ballots and LDS-staged scans.
//
// Three launches (two when the histogram table's reads stay small, see
// ci_scan_scatter_kernel: each scatter block then does its own scan):
//   1. count:   block b histograms its chunk of slots in LDS
//               -> blk_cnt[e][b]                                  (workspace)
//   2. scan:    one block: totals -> counts, offsets; per expert an exclusive
//               scan over blocks -> blk_off[e][b] = first row of block b's
//               slots of expert e.  Each expert gets a power-of-two group of
//               threads (inside one wave) that each sum a run of blocks.
//   3. scatter: block b re-reads its chunk; each wave ranks its slots with a
//               64-lane match mask (one ballot per expert-id bit), adds the
//               running per-(wave, expert) count and the block offset, and
//               writes dest and src.
#include <mutex>
#include <string>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCiBlock = 256;                 // 4 waves
constexpr int kCiWaves = kCiBlock / kWave;
constexpr int kCiChunk = 512;                 // slots per block (many blocks in flight)
constexpr int kCiSub = kCiChunk / kCiWaves;   // slots per wave
constexpr int kScanBlock = 1024;

inline int num_chunks(long long Tk) { return static_cast<int>((Tk + kCiChunk - 1) / kCiChunk); }

// Expert id of a slot.  Ids outside [0, E) are a caller error (the routing
// kernel never writes one); they are clamped, so that counts still sum to
// T*k, dest / src stay a permutation and every row index derived from them
// stays inside its buffer, and recorded.
__device__ __forceinline__ int load_id(const int32_t* __restrict__ ids, int s, int E) {
  const int id = ids[s];
  if (id >= 0 && id < E) return id;
  note_index_error(MOE_IDXERR_EXPERT);
  return id < 0 ? 0 : E - 1;
}

__global__ __launch_bounds__(kCiBlock) void ci_count_kernel(const int32_t* __restrict__ ids,
                                                            int Tk, int E, int nblk,
                                                            int32_t* __restrict__ blk_cnt) {
  extern __shared__ int32_t hist[];  // [E]
  for (int e = threadIdx.x; e < E; e += kCiBlock) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kCiChunk;
  const int end = min(base + kCiChunk, Tk);
  for (int s = base + threadIdx.x; s < end; s += kCiBlock) atomicAdd(&hist[load_id(ids, s, E)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kCiBlock)
    blk_cnt[static_cast<size_t>(e) * nblk + blockIdx.x] = hist[e];
}

__global__ __launch_bounds__(kScanBlock) void ci_scan_kernel(const int32_t* __restrict__ blk_cnt,
                                                             int E, int nblk,
                                                             int32_t* __restrict__ blk_off,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets) {
  __shared__ int32_t tot_s[MOE_MAX_EXPERTS];
  __shared__ int32_t base_s[MOE_MAX_EXPERTS];
  const int lane = threadIdx.x & (kWave - 1);
  // tpe threads per expert: a power of two with E * tpe <= kScanBlock (E <=
  // 1024 = kScanBlock) and tpe <= 64, so an expert's threads share a wave.
  int tpe = 1;
  while (tpe < kWave && 2 * tpe * E <= kScanBlock) tpe *= 2;
  const int per_t = (nblk + tpe - 1) / tpe;
  const int e = threadIdx.x / tpe, sub = threadIdx.x % tpe;
  const bool act = e < E;
  const int b0 = min(nblk, sub * per_t), b1 = min(nblk, b0 + per_t);
  const int32_t* row = blk_cnt + static_cast<size_t>(act ? e : 0) * nblk;
  // A thread's block counts are loaded kBatch at a time, all in flight
  // together (a loop of single loads waits once per block); runs of up to
  // kBatch blocks (the common case: T*k <= 16 Ki slots per expert thread)
  // keep them in registers for the second pass.
  constexpr int kBatch = 8;
  int held[kBatch];
  int part = 0;
  if (act) {
    for (int b = b0; b < b1; b += kBatch) {
#pragma unroll
      for (int q = 0; q < kBatch; ++q) held[q] = b + q < b1 ? row[b + q] : 0;
#pragma unroll
      for (int q = 0; q < kBatch; ++q) part += held[q];
    }
  }
  // Inclusive scan over the expert's tpe threads, then its total.
  int inc = part;
  for (int o = 1; o < tpe; o <<= 1) {
    const int n = __shfl_up(inc, o, tpe);
    if (sub >= o) inc += n;
  }
  const int tot = __shfl(inc, tpe - 1, tpe);
  if (act && sub == 0) tot_s[e] = tot;
  __syncthreads();
  // Exclusive scan of the totals over experts (wave 0).
  if (threadIdx.x < kWave) {
    int carry = 0;
    for (int c = 0; c < E; c += kWave) {
      const int v = c + lane < E ? tot_s[c + lane] : 0;
      const int iv = wave_inclusive_scan(v, lane);
      if (c + lane < E) base_s[c + lane] = carry + iv - v;
      carry += __shfl(iv, kWave - 1, kWave);
    }
    if (lane == 0) offsets[E] = carry;
  }
  __syncthreads();
  if (act) {
    const int base = base_s[e];
    if (sub == 0) {
      counts[e] = tot;
      offsets[e] = base;
    }
    int32_t* orow = blk_off + static_cast<size_t>(e) * nblk;
    int run = base + inc - part;
    for (int b = b0; b < b1; b += kBatch) {
      if (b1 - b0 > kBatch) {  // reload this batch (held has the last one)
#pragma unroll
        for (int q = 0; q < kBatch; ++q) held[q] = b + q < b1 ? row[b + q] : 0;
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        if (b + q < b1) orow[b + q] = run;
        run += held[q];
      }
    }
  }
}

// Lanes of the wave whose id equals this lane's id (only among lanes with
// valid == true).  One ballot per id bit.
__device__ __forceinline__ uint64_t match_mask(int id, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (id >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    m &= bit ? ones : ~ones;
  }
  return valid ? m : 0ull;
}

// Ranks of block blockIdx.x's slots.  `first(e)` is the first row of this
// block's slots of expert e; run is LDS of kCiWaves * E ints.
template <class First>
__device__ __forceinline__ void scatter_block(const int32_t* __restrict__ ids, int Tk, int E,
                                              int nbits, First first, int32_t* run,
                                              int32_t* __restrict__ dest,
                                              int32_t* __restrict__ src) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kCiWaves * E; i += kCiBlock) run[i] = 0;
  __syncthreads();
  const int wbase = blockIdx.x * kCiChunk + wid * kCiSub;
  const int wend = min(wbase + kCiSub, Tk);
  int32_t* myrun = run + wid * E;
  const uint64_t lt = lanemask_lt(lane);

  // Pass 1: per-(wave, expert) counts of this block's chunk.
  for (int s0 = wbase; s0 < wend; s0 += kWave) {
    const int s = s0 + lane;
    const bool valid = s < wend;
    const int id = valid ? load_id(ids, s, E) : 0;
    const uint64_t m = match_mask(id, valid, nbits);
    if (valid && (m & lt) == 0) myrun[id] += __popcll(m);
  }
  __syncthreads();
  // Exclusive scan over waves, seeded with the block's first row per expert.
  for (int e = threadIdx.x; e < E; e += kCiBlock) {
    int acc = first(e);
    for (int w = 0; w < kCiWaves; ++w) {
      const int c = run[w * E + e];
      run[w * E + e] = acc;
      acc += c;
    }
  }
  __syncthreads();
  // Pass 2: final rows.
  for (int s0 = wbase; s0 < wend; s0 += kWave) {
    const int s = s0 + lane;
    const bool valid = s < wend;
    const int id = valid ? load_id(ids, s, E) : 0;
    const uint64_t m = match_mask(id, valid, nbits);
    int row = 0;
    if (valid) row = myrun[id] + __popcll(m & lt);
    // All lanes have read the running count before the leader advances it.
    __builtin_amdgcn_wave_barrier();
    if (valid && (m & lt) == 0) myrun[id] += __popcll(m);
    if (valid) {
      dest[s] = row;
      src[row] = s;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(kCiBlock) void ci_scatter_kernel(
    const int32_t* __restrict__ ids, int Tk, int E, int nbits, int nblk,
    const int32_t* __restrict__ blk_off, int32_t* __restrict__ dest, int32_t* __restrict__ src) {
  extern __shared__ int32_t run[];  // [kCiWaves][E]
  scatter_block(ids, Tk, E, nbits,
                [&](int e) { return blk_off[static_cast<size_t>(e) * nblk + blockIdx.x]; }, run,
                dest, src);
}

// Scan and scatter in one launch, for histogram tables whose reads stay small
// (E <= 1024 and E * nblk^2 <= kFusedReads; every workload here): every block
// sums the block histograms itself -- all blocks before it, and all blocks
// for the totals -- so no separate single-block scan is launched.  Block 0
// also writes counts and offsets.  Same arithmetic as ci_scan_kernel
// (integer sums), so the same result.  (The separate single-block scan took
// 56 us at the large-expert shape, E = 128 x 256 blocks; its lanes read runs
// of counts 128 bytes apart, one cache line each.)
constexpr int kFusedExperts = 1024;
// Every block reads the whole E x nblk table, so the fused path reads
// E * nblk^2 ints from L2 in all; above this the separate scan is cheaper.
constexpr long long kFusedReads = 1ll << 24;
// Tables up to this many ints are summed thread-per-expert (WAVE_ROWS =
// false): many experts with few blocks each (sparse small groups: 14 us in
// all against 35 us wave-per-expert, OLMoE-like 16.6 against 19.1 us);
// larger ones wave-per-expert (large-expert shape: 27 us against 69 us with
// the separate scan).
constexpr int kThreadRowsTable = 16384;

template <bool WAVE_ROWS>
__global__ __launch_bounds__(kCiBlock) void ci_scan_scatter_kernel(
    const int32_t* __restrict__ ids, int Tk, int E, int nbits, int nblk,
    const int32_t* __restrict__ blk_cnt, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dest, int32_t* __restrict__ src) {
  __shared__ int32_t before_s[kFusedExperts];
  __shared__ int32_t base_s[kFusedExperts];
  __shared__ int32_t run[kCiWaves * kFusedExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int me = static_cast<int>(blockIdx.x);
  if constexpr (!WAVE_ROWS) {
    // Small tables: tpe threads per expert, a power of two <= 64 with
    // E * tpe <= kCiBlock (an expert's threads share a wave), each summing a
    // run of blocks, 32 loads in flight at a time.
    int tpe = 1;
    while (tpe < kWave && 2 * tpe * E <= kCiBlock) tpe *= 2;
    const int per_t = (nblk + tpe - 1) / tpe;
    const int e = threadIdx.x / tpe, sub = threadIdx.x % tpe;
    const bool act = e < E;
    const int b0 = min(nblk, sub * per_t), b1 = min(nblk, b0 + per_t);
    const int32_t* row = blk_cnt + static_cast<size_t>(act ? e : 0) * nblk;
    int before = 0, total = 0;
    if (act) {
      constexpr int kBatch = 32;
      for (int b = b0; b < b1; b += kBatch) {
        int v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) v[q] = b + q < b1 ? row[b + q] : 0;
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          total += v[q];
          before += b + q < me ? v[q] : 0;
        }
      }
    }
    for (int o = tpe / 2; o > 0; o >>= 1) {
      total += __shfl_xor(total, o, kWave);
      before += __shfl_xor(before, o, kWave);
    }
    if (act && sub == 0) {
      base_s[e] = total;  // the totals first; the scan below turns them into offsets
      before_s[e] = before;
    }
  } else {
    // Larger tables: each wave takes experts wid, wid + 4, ...: its 64 lanes
    // read 64 consecutive block counts of the expert's row per load (whole
    // cache lines), eight experts by four runs of 64 blocks -- 32 loads in
    // flight per lane -- then two wave sums give the expert's total and the
    // part from the blocks before this one.  (Four experts by one run, one
    // memory round trip per four loads: the whole call took 36.5 us at 128
    // experts x 256 blocks, against 26.9 us now.)
    constexpr int kEx = 8, kRuns = 4;
    for (int e0 = wid; e0 < E; e0 += kCiWaves * kEx) {
      int total[kEx], before[kEx];
#pragma unroll
      for (int x = 0; x < kEx; ++x) total[x] = before[x] = 0;
      for (int b0 = 0; b0 < nblk; b0 += kRuns * kWave) {
        int v[kEx][kRuns];
#pragma unroll
        for (int x = 0; x < kEx; ++x) {
          const int e = e0 + x * kCiWaves;
#pragma unroll
          for (int r = 0; r < kRuns; ++r) {
            const int b = b0 + r * kWave + lane;
            v[x][r] = (e < E && b < nblk) ? blk_cnt[static_cast<size_t>(e) * nblk + b] : 0;
          }
        }
#pragma unroll
        for (int x = 0; x < kEx; ++x)
#pragma unroll
          for (int r = 0; r < kRuns; ++r) {
            total[x] += v[x][r];
            before[x] += b0 + r * kWave + lane < me ? v[x][r] : 0;
          }
      }
#pragma unroll
      for (int x = 0; x < kEx; ++x) {
        const int e = e0 + x * kCiWaves;
        const int tot = wave_sum_int(total[x]);
        const int bef = wave_sum_int(before[x]);
        if (e < E && lane == 0) {
          base_s[e] = tot;  // the totals first; the scan below turns them into offsets
          before_s[e] = bef;
        }
      }
    }
  }
  __syncthreads();
  // Exclusive scan of the totals over experts (wave 0).
  if (threadIdx.x < kWave) {
    int carry = 0;
    for (int c = 0; c < E; c += kWave) {
      const int v = c + lane < E ? base_s[c + lane] : 0;
      const int iv = wave_inclusive_scan(v, lane);
      if (c + lane < E) {
        base_s[c + lane] = carry + iv - v;
        if (me == 0) {
          counts[c + lane] = v;
          offsets[c + lane] = carry + iv - v;
        }
      }
      carry += __shfl(iv, kWave - 1, kWave);
    }
    if (me == 0 && lane == 0) offsets[E] = carry;
  }
  __syncthreads();
  scatter_block(ids, Tk, E, nbits, [&](int x) { return base_s[x] + before_s[x]; }, run, dest,
                src);
}

int id_bits(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_count_index_workspace_size(int T, int k, int E) {
  if (T < 1 || k < 1 || E < 1) return 0;
  const long long Tk = static_cast<long long>(T) * k;
  const size_t nblk = static_cast<size_t>(num_chunks(Tk));
  // blk_cnt and blk_off, each [E][nblk] int32, 256-byte aligned halves.
  const size_t half = ((static_cast<size_t>(E) * nblk * 4 + 255) / 256) * 256;
  return 2 * half;
}

namespace moe {
namespace {

moe_status check_count_index(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                             int32_t* offsets, int32_t* dest, int32_t* src) {
  MOE_REQUIRE(T >= 1 && k >= 1 && E >= 1, MOE_ERR_INVALID_ARG,
              "moe_count_index: T, k, E must be >= 1");
  MOE_REQUIRE(k <= E, MOE_ERR_INVALID_ARG, "moe_count_index: need k <= E");
  MOE_REQUIRE(E <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, "moe_count_index: E exceeds 1024");
  const long long Tk = static_cast<long long>(T) * k;
  MOE_REQUIRE(Tk < (1ll << 31), MOE_ERR_UNSUPPORTED, "moe_count_index: T*k must be < 2^31");
  MOE_REQUIRE(topk_idx && counts && offsets && dest && src, MOE_ERR_INVALID_ARG,
              "moe_count_index: null pointer");
  return MOE_OK;
}

// The launches of moe_count_index over a validated workspace of `need` bytes
// (every word of it is written before it is read: no clearing needed).
moe_status count_index_launch(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                              int32_t* offsets, int32_t* dest, int32_t* src, void* ws,
                              size_t need, moe_stream_t stream) {
  const long long Tk = static_cast<long long>(T) * k;
  const int nblk = num_chunks(Tk);
  int32_t* blk_cnt = static_cast<int32_t*>(ws);
  int32_t* blk_off = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + need / 2);
  hipStream_t st = as_stream(stream);
  hipLaunchKernelGGL(ci_count_kernel, dim3(nblk), dim3(kCiBlock), E * sizeof(int32_t), st,
                     topk_idx, static_cast<int>(Tk), E, nblk, blk_cnt);
  if (moe_status s = check_launch("moe_count_index/count")) return s;
  if (E <= kFusedExperts &&
      static_cast<long long>(E) * nblk * static_cast<long long>(nblk) <= kFusedReads) {
    if (static_cast<long long>(E) * nblk <= kThreadRowsTable && E <= kCiBlock)
      hipLaunchKernelGGL(ci_scan_scatter_kernel<false>, dim3(nblk), dim3(kCiBlock), 0, st,
                         topk_idx, static_cast<int>(Tk), E, id_bits(E), nblk, blk_cnt, counts,
                         offsets, dest, src);
    else
      hipLaunchKernelGGL(ci_scan_scatter_kernel<true>, dim3(nblk), dim3(kCiBlock), 0, st,
                         topk_idx, static_cast<int>(Tk), E, id_bits(E), nblk, blk_cnt, counts,
                         offsets, dest, src);
    return check_launch("moe_count_index/scan+scatter");
  }
  hipLaunchKernelGGL(ci_scan_kernel, dim3(1), dim3(kScanBlock), 0, st, blk_cnt, E, nblk, blk_off,
                     counts, offsets);
  if (moe_status s = check_launch("moe_count_index/scan")) return s;
  hipLaunchKernelGGL(ci_scatter_kernel, dim3(nblk), dim3(kCiBlock),
                     kCiWaves * E * sizeof(int32_t), st, topk_idx, static_cast<int>(Tk), E,
                     id_bits(E), nblk, blk_off, dest, src);
  return check_launch("moe_count_index/scatter");
}

// Scratch of moe_count_index_noalloc: one copy per GPU, held until the
// process ends.  Host code never names this array in a device context (on
// the host its name is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  MOE_REQUIRE(err == hipSuccess, MOE_ERR_HIP,
              std::string("moe_count_index_noalloc: hipGetDevice: ") + hipGetErrorString(err));
  MOE_REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED,
              "moe_count_index_noalloc: device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    MOE_REQUIRE(err == hipSuccess && p != nullptr, MOE_ERR_HIP,
                std::string("moe_count_index_noalloc: hipGetSymbolAddress: ") +
                    hipGetErrorString(err));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

moe_status index_record_count(hipStream_t st, unsigned int* bits, bool clear) {
  return take_index_flags(st, bits, clear);
}

}  // namespace moe

extern "C" moe_status moe_count_index(const int32_t* topk_idx, int T, int k, int E,
                                      int32_t* counts, int32_t* offsets, int32_t* dest,
                                      int32_t* src, void* ws, size_t ws_bytes,
                                      moe_stream_t stream) {
  clear_error();
  if (moe_status s = check_count_index(topk_idx, T, k, E, counts, offsets, dest, src)) return s;
  const size_t need = moe_count_index_workspace_size(T, k, E);
  MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE,
              "moe_count_index: workspace too small");
  MOE_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 15) == 0, MOE_ERR_WORKSPACE,
              "moe_count_index: workspace must be 16-byte aligned");
  return count_index_launch(topk_idx, T, k, E, counts, offsets, dest, src, ws, need, stream);
}

extern "C" moe_status moe_count_index_noalloc(const int32_t* topk_idx, int T, int k, int E,
                                              int32_t* counts, int32_t* offsets, int32_t* dest,
                                              int32_t* src, moe_stream_t stream) {
  clear_error();
  if (moe_status s = check_count_index(topk_idx, T, k, E, counts, offsets, dest, src)) return s;
  const size_t need = moe_count_index_workspace_size(T, k, E);
  MOE_REQUIRE(need <= MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_UNSUPPORTED,
              "moe_count_index_noalloc: the block tables of this shape exceed the static "
              "scratch (moe_count_index_workspace_size(T, k, E) must be <= "
              "MOE_NOALLOC_SCRATCH_BYTES); use moe_count_index with a workspace");
  void* ws = nullptr;
  if (moe_status s = scratch_of_current_device(&ws)) return s;
  return count_index_launch(topk_idx, T, k, E, counts, offsets, dest, src, ws, need, stream);
}
