// Grouped GEMM over all experts in one launch [Brief, Core method: the
// experts' matrix products are merged into a grouped GEMM; Summary, Method
// details / key design: optimised matrix multiplication].
//
// Rows [offsets[e], offsets[e+1]) of the token-major operands belong to
// expert e.  `offsets` is read on the device: each workgroup derives its
// (expert, row tile, column tile) from it, so the host never waits for the
// routing result.  Three operand layouts cover the forward and backward
// passes (b = per-expert weights [E, K, N]):
//
//   NN  c[rows e]  = a[rows e]  @ b[e]          forward (reduction over K)
//   NT  da[rows e] = dc[rows e] @ b[e]^T        input gradient (over N)
//   TN  db[e]      = a[rows e]^T @ dc[rows e]   weight gradient (over rows)
//
// bf16 path (gemm_mfma_kernel): v_mfma_f32_32x32x16_bf16 on tiles of up to
// 256x256 outputs, 8 waves (2x4, 128x64 per wave, two per SIMD) for the big
// tiles; smaller tiles for small shapes.  Operands go from global memory
// straight into LDS (buffer_load ... lds, one 1 KB wave instruction at a
// time), four reduction steps of 32 in flight:
//   * k-contiguous operands (a in NN, both in NT) in two "pair" buffers of
//     [rows][64] (two steps each; whole 128-byte lines per request), read
//     with ds_read_b128 through an XOR swizzle of the 16-byte chunk;
//   * k-strided operands (b in NN, both in TN) in four "quad" buffers of
//     [32][cols], read with gfx950's transposing ds_read_b64_tr_b16.
// Waits are counted vmcnt waits plus one barrier per step; the MFMAs are
// interleaved with the next half-step's fragment reads and loads.  The
// epilogue converts and stores through buffer descriptors over the tile's
// valid rows (GEMM 1 can apply SwiGLU there).  Workgroups are mapped so that
// each of the 8 XCDs (own L2) walks a contiguous range of tiles, which keeps
// one expert's weights and rows in one L2; weight-gradient tile rows are
// dealt over the XCDs in pairs, the hottest experts' first (balance under
// skewed routing: a weight-gradient tile is as long as its expert's row
// count).  Shapes with few output tiles reduce the weight gradient in row
// slices (partials in a workspace, summed in slice order).
//
// Float32 (and shapes whose K or N is not a multiple of 8) run on a plain
// LDS-tiled 64x64 kernel on the float32 matrix cores (gemm_f32_kernel:
// operands converted to float32 in LDS, v_mfma_f32_32x32x2_f32) with the same
// tile resolution.
#include <math.h>

#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

enum Mode { kNN = 0, kNT = 1, kTN = 2 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const void* x;    // NN: a [M,K]   NT: dc [M,N]  TN: a [M,K]
  const void* y;    // NN: b [E,K,N] NT: b [E,K,N] TN: dc [M,N]
  const void* add;  // NT: optional addend [M,K]
  void* out;        // NN: c [M,N]   NT: da [M,K]  TN: db [E,K,N] or split partials
  const int32_t* offsets;
  int M, K, N, E;
  int ntm;    // TN: row tiles over K
  int ntn;    // column tiles
  int split;  // TN: reduction slices (partials written to out as [split][E][K][N])
  void* out2;  // NN with the SwiGLU epilogue: act [M, N / 2]
  // Gathered x operand (GEMM 1 and its weight gradient without a permuted
  // copy of x): logical row p of x is physical row xrows[p] / xdiv of the
  // x array, which has xphys rows.  xrows == nullptr: x is used as is.
  const int32_t* xrows;
  int xdiv;
  int xphys;
  unsigned xmagic;  // ceil(2^32 / xdiv) mod 2^32 (see div_rows)
  int xshift;       // log2(xdiv) when xdiv is a power of two, else -1
  int hot_first;    // TN, E <= 256: take the groups in hot-first order (group_at)
  int row_group;    // NN / NT: tile order inside a group (see find_row_tile); 0 = row-major
  // Gathered y operand (the weight gradient reading its dc through a row
  // map): logical row p of y is physical row yrows[p] / ydiv of an array of
  // yphys rows.  yrows == nullptr: y is used as is.
  const int32_t* yrows;
  int ydiv;
  int yphys;
  unsigned ymagic;
  int yshift;
  // NT: output row p is multiplied by row_scale[p] before rounding (nullptr:
  // no scale).
  const float* row_scale;
};

// ------------------------------------------------------------------ tiles
// Row-tiled modes (NN, NT): every wave finds which expert owns this
// workgroup's row tile (the same answer in each wave, so no LDS and no
// barrier are needed, and small tiles keep their LDS footprint at a multiple
// of the operand buffers).  Tiles are counted per expert as
// ceil(rows_e / BM); expert e owns logical tiles [ntn * first_row_tile_e,
// ntn * (first_row_tile_e + tiles_e)), ordered inside by order_in_group;
// workgroup b runs on XCD b % 8 and takes logical tile
// (b % 8) * ceil(n / 8) + b / 8, so each XCD walks a contiguous range of
// experts.  Up to kHeld * 64 experts the offsets are loaded once (all loads in
// flight together) and kept in registers.
struct RowTile {
  int found, e, mt_local, nt, g0, g1;  // wave-uniform
};

// Position of the tile at index `local` among a group's te * ntn tiles.
// group_rows = 0: row-major (all ntn column tiles of a row tile in turn).
// Otherwise the group's row tiles are taken in bands of group_rows, and each
// band column by column: the ~32 tiles an XCD runs at once then cover a few
// row tiles and a few column tiles of one group (e.g. 8 x 4) instead of two
// row tiles and every column tile, so fewer distinct operand slabs stream
// through that XCD's L2 at a time.
__device__ __forceinline__ void order_in_group(int local, int te, int ntn, int group_rows,
                                               int& mt_local, int& nt) {
  if (group_rows <= 0) {
    mt_local = local / ntn;
    nt = local - mt_local * ntn;
    return;
  }
  const int band = local / (group_rows * ntn);
  const int rows = min(group_rows, te - band * group_rows);
  const int w = local - band * group_rows * ntn;
  nt = w / rows;
  mt_local = band * group_rows + (w - nt * rows);
}

// A group whose offsets are reversed or leave [0, M] (a caller error) gets
// no tiles; every workgroup sees it, and the first thread of each records it.
__device__ __forceinline__ bool group_ok(int o0, int o1, int M) {
  return o0 >= 0 && o0 <= o1 && o1 <= M;
}

template <int BM>
__device__ RowTile find_row_tile(const int32_t* __restrict__ offsets, int E, int M, int ntn,
                                 int group_rows, int lane) {
  constexpr int kHeld = 4;
  const bool held = E <= kHeld * kWave;
  int o0[kHeld], o1[kHeld], tiles[kHeld], incl[kHeld];
  int total = 0;
  bool bad = false;
  if (held) {
#pragma unroll
    for (int c = 0; c < kHeld; ++c) {
      const int e = c * kWave + lane;
      o0[c] = e < E ? offsets[e] : 0;
      o1[c] = e < E ? offsets[e + 1] : 0;
      if (!group_ok(o0[c], o1[c], M)) {
        bad = true;
        o0[c] = o1[c] = 0;
      }
    }
#pragma unroll
    for (int c = 0; c < kHeld; ++c) {
      tiles[c] = (o1[c] - o0[c] + BM - 1) / BM;
      incl[c] = 0;
      if (c * kWave < E) {
        incl[c] = wave_inclusive_scan(tiles[c], lane);
        total += __shfl(incl[c], kWave - 1, kWave);
      }
    }
  } else {
    for (int c = 0; c < E; c += kWave) {
      const int e = c + lane;
      int n = 0;
      if (e < E) {
        const int a0 = offsets[e], a1 = offsets[e + 1];
        if (group_ok(a0, a1, M))
          n = (a1 - a0 + BM - 1) / BM;
        else
          bad = true;
      }
      total += wave_sum_int(n);
    }
  }
  if (__ballot(bad) != 0 && threadIdx.x == 0) note_index_error(MOE_IDXERR_GROUP);
  const long long n_act = static_cast<long long>(total) * ntn;
  const long long per = (n_act + 7) / 8;
  const long long rank = blockIdx.x >> 3;
  const long long L = static_cast<long long>(blockIdx.x & 7) * per + rank;
  int found = 0, e_found = 0, mt_local = 0, nt = 0, g0 = 0, g1 = 0;
  if (rank < per && L < n_act) {
    // Group e owns logical tiles [ntn * excl_e, ntn * (excl_e + tiles_e)), so
    // the row tile L / ntn (counted over all groups) names the group; the
    // tile's place inside the group follows order_in_group.
    const int mt = static_cast<int>(L / ntn);
    int excl_found = 0, te_found = 0;
    int carry = 0;
    if (held) {
#pragma unroll
      for (int c = 0; c < kHeld; ++c) {
        if (found || c * kWave >= E) continue;
        const int excl = carry + incl[c] - tiles[c];
        const bool hit = tiles[c] > 0 && mt >= excl && mt < excl + tiles[c];
        const uint64_t bal = __ballot(hit);
        if (bal) {
          const int srcl = __builtin_ctzll(bal);
          e_found = c * kWave + srcl;
          excl_found = __shfl(excl, srcl, kWave);
          te_found = __shfl(tiles[c], srcl, kWave);
          g0 = __shfl(o0[c], srcl, kWave);
          g1 = __shfl(o1[c], srcl, kWave);
          found = 1;
        }
        carry += __shfl(incl[c], kWave - 1, kWave);
      }
    } else {
      for (int c = 0; c < E; c += kWave) {
        const int e = c + lane;
        int a0 = e < E ? offsets[e] : 0;
        int a1 = e < E ? offsets[e + 1] : 0;
        if (!group_ok(a0, a1, M)) a0 = a1 = 0;
        const int n = (a1 - a0 + BM - 1) / BM;
        const int inc = wave_inclusive_scan(n, lane);
        const int excl = carry + inc - n;
        const bool hit = n > 0 && mt >= excl && mt < excl + n;
        const uint64_t bal = __ballot(hit);
        if (bal) {
          const int srcl = __builtin_ctzll(bal);
          e_found = __shfl(e, srcl, kWave);
          excl_found = __shfl(excl, srcl, kWave);
          te_found = __shfl(n, srcl, kWave);
          g0 = __shfl(a0, srcl, kWave);
          g1 = __shfl(a1, srcl, kWave);
          found = 1;
          break;
        }
        carry += __shfl(inc, kWave - 1, kWave);
      }
    }
    if (found) {
      const int local = static_cast<int>(L - static_cast<long long>(excl_found) * ntn);
      order_in_group(local, te_found, ntn, group_rows, mt_local, nt);
    }
  }
  return RowTile{found, e_found, mt_local, nt, g0, g1};
}

struct TileInfo {
  int e, i0, j0, r_lo, r_hi, g0, g1, slice;
};

// Weight-gradient tiles reduce over all rows of their group, so a hot group's
// tiles are long; started last, they leave the other compute units idle at
// the end of the launch.  Hot-first order: groups with at least 6, 4, 3, 2
// and 1.5 times the mean row count, bucket by bucket, then the rest, by index
// within a bucket (the longest tiles start first, without a sort).  Groups
// below 1.5 times the mean keep their index order.  Returns the group at
// position `pos` of that order; E <= 256.  Run by every wave (wave-uniform).
__device__ int group_at(const int32_t* __restrict__ offsets, int E, int pos, int lane) {
  constexpr int kRuns = 4;                          // runs of 64 groups
  constexpr int kTimes2[] = {12, 8, 6, 4, 3};       // bucket bounds, x2
  constexpr int kBuckets = 6;
  const long long total = offsets[E] - offsets[0];  // all rows (uniform)
  int bucket[kRuns];
#pragma unroll
  for (int c = 0; c < kRuns; ++c) {
    const int e = c * kWave + lane;
    bucket[c] = -1;  // past E: in no bucket
    if (e < E) {
      const long long n2e = 2ll * (offsets[e + 1] - offsets[e]) * E;  // 2 n_e E vs th2 * total
      int b = kBuckets - 1;
#pragma unroll
      for (int q = kBuckets - 2; q >= 0; --q)
        if (n2e >= kTimes2[q] * total) b = q;
      bucket[c] = b;
    }
  }
  const uint64_t below = (1ull << lane) - 1ull;
  for (int b = 0; b < kBuckets; ++b) {
#pragma unroll
    for (int c = 0; c < kRuns; ++c) {
      const uint64_t m = __ballot(bucket[c] == b);
      const int cnt = __popcll(m);
      if (pos < cnt) {
        const bool hit = bucket[c] == b && __popcll(m & below) == pos;
        return c * kWave + __builtin_ctzll(__ballot(hit));
      }
      pos -= cnt;
    }
  }
  return 0;  // pos >= E: not reached (callers pass pos < E)
}

// Returns false if this workgroup has no tile.  Must be called by all threads.
constexpr int kTnDeal = 2;  // weight-gradient tile rows dealt to an XCD at a time

template <int MODE, int BM>
__device__ bool resolve_tile(const GemmArgs& p, TileInfo& t) {
  if constexpr (MODE == kTN) {
    // Tile rows (slice, e, row tile) are dealt over the XCDs in pairs --
    // XCD x takes rows 2x, 2x + 1, 2x + 16, 2x + 17, ... with all ntn column
    // tiles of each -- so every XCD gets a share of every group however
    // unevenly the rows are spread over the groups (the reduction of a big
    // group is as long as its row count), while each group's column operand
    // is read by a few XCDs only.  (Single rows balance a skewed routing
    // slightly better but cost the even one more L2 traffic; groups of four
    // balance worse.)
    const long long per_e = static_cast<long long>(p.ntm) * p.ntn;
    const long long nrows = static_cast<long long>(p.ntm) * p.E * p.split;
    const long long rank = blockIdx.x >> 3;
    const long long gsz = static_cast<long long>(kTnDeal) * p.ntn;
    const long long within = rank % gsz;
    const long long R = ((rank / gsz) * 8 + (blockIdx.x & 7)) * kTnDeal + within / p.ntn;
    if (R >= nrows) return false;
    const long long L = R * p.ntn + within % p.ntn;
    const long long per_slice = per_e * p.E;
    t.slice = static_cast<int>(L / per_slice);
    const long long rem0 = L - static_cast<long long>(t.slice) * per_slice;
    const int pos = static_cast<int>(rem0 / per_e);
    const int rem = static_cast<int>(rem0 - static_cast<long long>(pos) * per_e);
    t.e = p.hot_first ? group_at(p.offsets, p.E, pos, threadIdx.x & (kWave - 1)) : pos;
    const int mt = rem / p.ntn;
    const int nt = rem - mt * p.ntn;
    t.i0 = mt * BM;
    t.g0 = p.offsets[t.e];
    t.g1 = p.offsets[t.e + 1];
    if (!group_ok(t.g0, t.g1, p.M)) {
      // No rows: the tile's weight gradient is written as zeros.
      if (threadIdx.x == 0) note_index_error(MOE_IDXERR_GROUP);
      t.g0 = t.g1 = 0;
    }
    const int len = t.g1 - t.g0;
    // Slice s reduces rows [g0 + s*chunk, g0 + (s+1)*chunk), chunk a multiple of 64.
    const int chunk = ((len + p.split - 1) / p.split + 63) / 64 * 64;
    t.r_lo = min(t.g1, t.g0 + t.slice * chunk);
    t.r_hi = min(t.g1, t.r_lo + chunk);
    t.j0 = nt;  // column tile index; scaled by the caller
    return true;
  } else {
    const int lane = threadIdx.x & (kWave - 1);
    const RowTile r = find_row_tile<BM>(p.offsets, p.E, p.M, p.ntn, p.row_group, lane);
    if (!r.found) return false;
    t.e = r.e;
    t.g0 = r.g0;
    t.g1 = r.g1;
    t.i0 = t.g0 + r.mt_local * BM;
    t.j0 = r.nt;
    t.r_lo = 0;
    t.r_hi = (MODE == kNN) ? p.K : p.N;
    t.slice = 0;
    return true;
  }
}

// ------------------------------------------------------------------ MFMA path
// Tiles of BM x BN outputs, reduction in steps of kBK = 32.  Operand tiles go
// from global memory straight into LDS (buffer_load_dwordx4 ... lds: each wave
// instruction fills 1 KB of LDS, lane i writing bytes [16 i, 16 i + 16)); the
// LDS layout is chosen through each lane's source address.  Out-of-range
// elements come back as zeros from the buffer descriptor's range check, so the
// main loop has no branches.
//
// The load path is bound by the number of cache lines in flight per compute
// unit, so every load fetches whole 128-byte lines:
//   k-contiguous operand ("pair" buffers): two buffers of [O][64] (two
//     reduction steps, 128 B per row), refilled every other step.  16-byte
//     chunk c of row r is stored at chunk c ^ ((r >> 1) & 7); MFMA fragments
//     (8 consecutive k of one row) are read with ds_read_b128, and 16
//     consecutive rows at one chunk cover all 64 banks.
//   k-strided operand ("quad" buffers; the reduction index is not contiguous
//     in memory): four buffers of [32][O] (one step each, as the tile lies in
//     memory, O >= 64 elements = whole lines).  16-byte unit u of row k is
//     stored at u ^ swz_t(k).  Fragments are read with two ds_read_b64_tr_b16:
//     within each 16 lanes, lane s reads 4 elements of row k0 + s/4 at column
//     n0 + 4 (s % 4), and the instruction returns to lane s the 4
//     consecutive-k elements of column n0 + s -- the MFMA operand layout.
// Every wave waits for its own fragment reads of step s before the barrier
// that ends step s, so the buffers of step s are free right after it: quad
// loads for step s + 4 and (at odd s) pair loads for steps s + 3, s + 4 go out
// then, three and two steps before they are read.
constexpr int kBK = 32;
constexpr int kThreads = 256;           // float32 kernel: 4 waves per block
constexpr unsigned kOOB = 0x80000000u;  // buffer offset that is always out of range
constexpr int kCpolNonTemporal = 2;     // cache-policy operand of buffer stores: nt

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Buffer descriptor over [base, base + bytes).  Base and size are the same in
// every lane; readfirstlane keeps the descriptor in scalar registers (a value
// the compiler computes with vector instructions would otherwise make it wrap
// every load in a loop over distinct descriptors).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
  const int n = bytes > 0x7ffffff0LL ? 0x7ffffff0 : static_cast<int>(bytes < 0 ? 0 : bytes);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// s_waitcnt vmcnt(N) lgkmcnt(0): this wave's LDS reads done and at most N of
// its global loads outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
}

// Pair buffers: physical 16-byte chunk of logical chunk c (0..7) of row r.
__device__ __forceinline__ int swz_p(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <int O>
__device__ __forceinline__ int swz_t(int k) {
  // O >= 128: a row spans >= 16 units (all banks), rows k..k+3 are spread by
  // XOR-ing the unit with 4 (k % 4).  O == 64: rows of 8 units alternate bank
  // halves, so only (k / 2) % 2 is needed.
  if constexpr (O >= 128)
    return 4 * (k & 3);
  else
    return 4 * ((k >> 1) & 1);
}

// Operand descriptor: element (o, r) lives at
//   k-contiguous: base + o * ld + r           (o from 0 = the tile's first row)
//   k-strided:    base + (r - r_lo) * ld + o  (o from 0 = the tile's first column)
struct Operand {
  const uint16_t* base;
  long long ld;
  int o_valid;  // number of valid o from the tile's first one (glu: hidden units)
  // SwiGLU weights [K, 2F]: tile column o is hidden unit f = (o / 64) * 32 +
  // o % 32 of the gate half (o / 32 even) or of the up half (o / 32 odd),
  // i.e. memory column (o / 32 % 2) * glu_f + glu_j0 + f.  glu_f = 0: plain.
  int glu_f;
  int glu_j0;
  // Gathered rows (loaders with GX): logical row p (k-contiguous: tile row;
  // k-strided: reduction row) is physical row rows[p] / rdiv of base, which
  // has `phys` rows; col0 is added to every column (k-strided).
  const int32_t* rows;
  int rdiv;
  int phys;
  int col0;
  unsigned rmagic;  // ceil(2^32 / rdiv) mod 2^32
  int rshift;       // log2(rdiv) when rdiv is a power of two, else -1
};

// n / d for 0 <= n < 2^31, 1 <= d, with m = ceil(2^32 / d) mod 2^32: the
// high half of n * m is n / d or n / d + 1 (the excess of m over 2^32 / d
// adds less than n / 2^32 < 1/2), one correction each way makes it exact;
// d = 1 (m wraps to 0) is passed through.  A handful of instructions instead
// of a full 32-bit division.
__device__ __forceinline__ int div_rows(int n, int d, unsigned m) {
  const unsigned un = static_cast<unsigned>(n), ud = static_cast<unsigned>(d);
  unsigned q = __umulhi(un, m);
  q -= (q * ud > un) ? 1u : 0u;
  q += ((q + 1u) * ud <= un) ? 1u : 0u;
  return d == 1 ? n : static_cast<int>(q);
}

// Loads of one operand, shared by the NW waves of the workgroup.  A k-strided
// operand loads one reduction step (O x 32 elements, O / 16 wave
// instructions) per call; a k-contiguous one loads a pair of steps (O x 64
// elements, O / 8 wave instructions).
template <bool STRIDED, int O, int NW, bool GX = false>
struct DmaLoader {
  static constexpr int kSpan = STRIDED ? kBK : 2 * kBK;  // reduction elements per call
  static constexpr int kTotal = O * kSpan * 2 / 1024;     // 1 KB wave instructions per call
  static constexpr int kPerWave = kTotal >= NW ? kTotal / NW : 1;
  // Vector-memory loads per call and wave: the LDS loads, plus (gathered
  // k-strided operand) the row-map loads of the call four ahead.
  static constexpr int kLoadsPerCall = kPerWave * ((GX && STRIDED) ? 2 : 1);
  static_assert(kTotal % NW == 0 || kTotal < NW, "chunks must split evenly over waves");
  static_assert(NW % 2 == 0, "pair chunk mapping assumes an even number of waves");
  __amdgpu_buffer_rsrc_t rsrc;
  unsigned voff[kPerWave];  // byte offset at call index 0 (kOOB: lane out of range)
  int lds_off[kPerWave];    // element offset in the buffer (wave-uniform)
  int klim;                 // k-contiguous: this lane's chunk loaded for call indices < klim
  unsigned step;            // bytes per call index
  // Gathered k-strided operand: this lane's row within a call (per q), the
  // tile's reduction range, the row map, and a ring of the physical rows of
  // the next four calls (slot = call index % 4).
  int grow[GX && STRIDED ? kPerWave : 1];
  int g_lo, g_hi, g_div, g_shift, g_phys;
  unsigned g_magic;
  unsigned g_lim;  // row-map entries must lie below this (x_phys * x_div)
  bool g_bad;      // k-contiguous: this lane met a row-map entry outside [0, g_lim)
  uint64_t g_badmask;  // k-strided: OR of the lane masks of bad entries (wave-uniform)
  unsigned ld_bytes;
  __amdgpu_buffer_rsrc_t g_rs;  // the row map
  int ring[GX && STRIDED ? kPerWave : 1][4];

  __device__ __forceinline__ void init(const Operand& op, int r_lo, int r_hi) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    g_bad = false;
    g_badmask = 0;
    if constexpr (GX) {
      // An entry at or past x_phys * x_div (or negative) is a caller error:
      // its row reads as zeros (physical row x_phys, just past the range)
      // and is recorded.
      const long long lim = static_cast<long long>(op.phys) * op.rdiv;
      g_lim = static_cast<unsigned>(lim < 0x80000000LL ? lim : 0x80000000LL);
      g_phys = op.phys;
    }
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
      const int cid = q * NW + w;  // 1 KB piece of the buffer
      lds_off[q] = cid * 512;
      const int pos = cid * 1024 + lane * 16;  // byte position in the buffer
      if constexpr (!STRIDED) {
        // Row cid * 8 + lane / 8; its logical chunk c for physical chunk
        // lane % 8 depends on the row only through (row / 2) % 8, i.e. on the
        // lane and the parity of cid -- the same for every q (NW is even).
        const int row = pos / (kSpan * 2);
        const int c = swz_p(row, lane & 7);
        // Chunk [c * 8, c * 8 + 8) of call i lies inside the reduction range
        // while r_lo + i * 64 + c * 8 + 8 <= r_hi.
        const int room = r_hi - r_lo - c * 8 - 8;
        klim = room >= 0 ? room / kSpan + 1 : 0;
        int prow = row;  // physical row
        if constexpr (GX) {
          prow = 0;
          if (row < op.o_valid) {
            const int raw = op.rows[row];
            if (static_cast<unsigned>(raw) < g_lim) {
              prow = div_rows(raw, op.rdiv, op.rmagic);
            } else {
              prow = op.phys;
              g_bad = true;
            }
          }
        }
        voff[q] = row < op.o_valid ? static_cast<unsigned>((prow * op.ld + c * 8) * 2) : kOOB;
      } else {
        // Rows past the reduction range fall outside the buffer range; so do
        // columns past the operand (kOOB + i * step stays above the range,
        // which is below 2^31 bytes).
        const int row = pos / (O * 2);
        const int u = ((pos % (O * 2)) / 16) ^ swz_t<O>(row);
        int col = u * 8;
        bool valid;
        if (op.glu_f) {
          const int blk = col >> 5, f = (blk >> 1) * 32 + (col & 31);
          valid = f + 8 <= op.o_valid;
          col = (blk & 1) * op.glu_f + op.glu_j0 + f;
        } else {
          valid = col + 8 <= op.o_valid;
        }
        if constexpr (GX) {
          // row is this lane's row within a call; the physical row comes
          // from the ring at issue time.
          grow[q] = row;
          voff[q] = valid ? static_cast<unsigned>((op.col0 + col) * 2) : kOOB;
        } else {
          voff[q] = valid ? static_cast<unsigned>((row * op.ld + col) * 2) : kOOB;
        }
      }
    }
    if constexpr (GX) {
      rsrc = make_rsrc(op.base, static_cast<long long>(op.phys) * op.ld * 2);
      step = STRIDED ? 0u : static_cast<unsigned>(kSpan * 2);
      if constexpr (STRIDED) {
        g_lo = r_lo;
        g_hi = r_hi;
        g_magic = op.rmagic;
        g_shift = op.rshift;
        ld_bytes = static_cast<unsigned>(op.ld * 2);
        g_div = op.rdiv;
        g_rs = make_rsrc(op.rows, static_cast<long long>(r_hi > 0 ? r_hi : 1) * 4);
        // Row maps of calls 0..3; the prologue's issues fetch those of 4..7.
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) fetch_rows(sl, sl);
      }
    } else if constexpr (!STRIDED) {
      const int rows = op.o_valid < O ? (op.o_valid < 0 ? 0 : op.o_valid) : O;
      rsrc = make_rsrc(op.base, static_cast<long long>(rows) * op.ld * 2);
      step = kSpan * 2;
    } else {
      rsrc = make_rsrc(op.base, static_cast<long long>(r_hi - r_lo) * op.ld * 2);
      step = static_cast<unsigned>(kSpan * op.ld * 2);
    }
  }

  // Gathered k-strided operand: load the row-map entries of call i into ring
  // slot sl.  Every lane loads (a clamped index past the range), so each call
  // issues the same number of loads, which the counted waits rely on.
  __device__ __forceinline__ void fetch_rows(int i, int sl) {
    if constexpr (GX && STRIDED) {
#pragma unroll
      for (int q = 0; q < kPerWave; ++q) {
        const int r = min(g_lo + i * kBK + grow[q], g_hi - 1);
        ring[q][sl] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(
            g_rs, static_cast<unsigned>(r < 0 ? 0 : r) * 4u, 0, 0));
      }
    }
  }

  // Gathered k-strided operand: turn ring slot sl (row-map entries, landed)
  // into physical rows.  Called at the start of the step that issues from
  // that slot, so the division runs beside the MFMAs instead of in front of
  // the loads.
  __device__ __forceinline__ void prepare(int sl) {
    if constexpr (GX && STRIDED) {
      // Entries out of range become row g_phys, whose loads fall past the
      // buffer range (zeros); a wave-wide mask of such lanes is kept in
      // scalar registers for the record.  With a shift the clamp is a minimum: a valid entry
      // (below g_phys << g_shift) shifts to below g_phys, a larger one to at
      // least g_phys, a negative one (arithmetic shift) to a negative value,
      // i.e. a large unsigned one.
      if (g_shift >= 0) {  // uniform: a power-of-two divisor is a shift
#pragma unroll
        for (int q = 0; q < kPerWave; ++q) {
          const unsigned sh = static_cast<unsigned>(ring[q][sl] >> g_shift);
          const unsigned prow = min(sh, static_cast<unsigned>(g_phys));
          g_badmask |= __ballot(prow == static_cast<unsigned>(g_phys));
          ring[q][sl] = static_cast<int>(prow);
        }
      } else {
#pragma unroll
        for (int q = 0; q < kPerWave; ++q) {
          const unsigned raw = static_cast<unsigned>(ring[q][sl]);
          const int prow = raw < g_lim ? div_rows(static_cast<int>(raw), g_div, g_magic) : g_phys;
          g_badmask |= __ballot(prow == g_phys);
          ring[q][sl] = prow;
        }
      }
      // Pin the results here: otherwise the compiler sinks the division to
      // just before the load that uses it, after the step's barrier.
#pragma unroll
      for (int q = 0; q < kPerWave; ++q) asm volatile("" : "+v"(ring[q][sl]));
    }
  }

  // Issue the loads of call index i (a step, or a pair of steps) into `buf`;
  // sl = i % 4, a compile-time constant at every call site (gathered
  // k-strided operand: the ring slot holding call i's rows, refilled with
  // those of call i + 4).
  __device__ __forceinline__ void issue(uint16_t* buf, int i, int sl = 0) {
    if (kTotal < NW && static_cast<int>(threadIdx.x / kWave) >= kTotal) return;
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
      unsigned off;
      if constexpr (GX && STRIDED) {
        const int r = g_lo + i * kBK + grow[q];
        const int prow = ring[q][sl];  // prepared
        // prow < 2^24 and the row stride < 2^24 bytes (checked on the host):
        // a full-rate 24-bit multiply.
        off = (r < g_hi && voff[q] != kOOB)
                  ? voff[q] + __umul24(static_cast<unsigned>(prow), ld_bytes)
                  : kOOB;
      } else if constexpr (STRIDED) {
        off = voff[q] + static_cast<unsigned>(i) * step;
      } else {
        off = i < klim ? voff[q] + static_cast<unsigned>(i) * step : kOOB;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(buf + lds_off[q]), 16, off, 0,
                                               0, 0);
    }
    if constexpr (GX && STRIDED) fetch_rows(i + 4, sl);
  }
};

// MFMA fragment addressing: 8 consecutive k (16 kk .. 16 kk + 15, split by
// lane half) of row / column `32 i` of this wave's part of the buffer, for the
// step that is half h of a pair buffer (k-contiguous) or a whole quad buffer
// (k-strided).  The lane-dependent part of each LDS element offset is
// computed once per tile; the rest is a compile-time constant that lands in
// the instruction's offset field.  The lane part goes through an empty asm
// statement so that every fragment read stays a plain offset from its buffer
// array: the compiler then keeps the LDS alias information that lets it wait
// only for the DMA loads of the buffer being read (when it derives one read's
// address from another's, it drops that information and waits for all loads
// in flight).
template <bool STRIDED, int O, int N>
struct FragAddr {
  int idx[STRIDED ? N : 4];

  __device__ __forceinline__ void init(int wbase, int lane) {
    if constexpr (!STRIDED) {
      // [O][64] buffer; wbase % 32 == 0, so the swizzle depends on the lane only
      const int row = wbase + (lane & 31);
#pragma unroll
      for (int hk = 0; hk < 4; ++hk) {
        const int chunk = hk * 2 + (lane >> 5);  // hk = 2 h + kk
        idx[hk] = row * 2 * kBK + (swz_p(row, chunk) << 3);
        asm volatile("" : "+v"(idx[hk]));
      }
    } else {
      // [32][O] buffer; lane s of each 16 reads row k0 + s / 4, 4 columns from
      // n0 + 4 (s % 4); the k0 + 4 and k0 + 16 rows share k0's swizzle.
      const int g = lane >> 4, s = lane & 15;
      const int k0 = 8 * (g >> 1) + (s >> 2);
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const int col = wbase + j * 32 + 16 * (g & 1) + 4 * (s & 3);
        idx[j] = k0 * O + (((col >> 3) ^ swz_t<O>(k0)) << 3) + (col & 7);
        asm volatile("" : "+v"(idx[j]));
      }
    }
  }

  __device__ __forceinline__ bf16x8 read(const uint16_t* buf, int i, int h, int kk) const {
    if constexpr (!STRIDED) {
      const u32x4 v =
          *reinterpret_cast<const u32x4*>(buf + idx[h * 2 + kk] + i * 32 * 2 * kBK);
      return __builtin_bit_cast(bf16x8, v);
    } else {
      const uint16_t* p0 = buf + idx[i] + kk * 16 * O;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p0);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p0 + 4 * O));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, v);
    }
  }
};

template <int MI, int NI>
struct Frags {
  bf16x8 a[MI], b[NI];
};

// Buffers of one operand: four quad buffers or two pair buffers.
struct Bufs {
  uint16_t* b[4];
};

// Buffer and pair half holding reduction step s (mod 4) of an operand.
template <bool STRIDED>
__device__ __forceinline__ const uint16_t* step_buf(const Bufs& B, int s) {
  return STRIDED ? B.b[s & 3] : B.b[(s >> 1) & 1];
}

// Fragments of step s (mod 4), k-slice kk: the first MIV 32-row blocks of this
// wave's rows (the rest of the wave's rows are past the end of its group) and
// all its columns.
template <int MIV, bool XS, bool YS, int MI, int NI, class XA, class YA>
__device__ __forceinline__ void read_frags(Frags<MI, NI>& f, const Bufs& xb, const Bufs& yb,
                                           int s, int kk, const XA& xa, const YA& ya) {
  if constexpr (MIV > 0) {
    const uint16_t* xt = step_buf<XS>(xb, s);
    const uint16_t* yt = step_buf<YS>(yb, s);
#pragma unroll
    for (int i = 0; i < MIV; ++i) f.a[i] = xa.read(xt, i, s & 1, kk);
#pragma unroll
    for (int j = 0; j < NI; ++j) f.b[j] = ya.read(yt, j, s & 1, kk);
  }
}

template <int MIV, int MI, int NI>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[MI][NI], const Frags<MI, NI>& f) {
#pragma unroll
  for (int i = 0; i < MIV; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Loads that belong to reduction step t (t % 4 == s, a compile-time
// constant): quad operands load step t into quad buffer s; when t is odd, pair
// operands load steps t - 1, t (pair (t - 1) / 2) into pair buffer
// ((t - 1) / 2) % 2 -- two steps ahead of the quad loads of step t - 1, since a
// pair buffer frees up only after both steps of the pair it held.
template <bool XS, bool YS, class XL, class YL>
__device__ __forceinline__ void issue_step(XL& xl, YL& yl, const Bufs& xb, const Bufs& yb, int s,
                                           int t) {
  if ((s & 1) == 1) {
    if constexpr (!XS) xl.issue(xb.b[(s >> 1) & 1], t >> 1);
    if constexpr (!YS) yl.issue(yb.b[(s >> 1) & 1], t >> 1);
  }
  if constexpr (XS) xl.issue(xb.b[s & 3], t, s & 3);
  if constexpr (YS) yl.issue(yb.b[s & 3], t, s & 3);
}

// Scheduling pattern for a half step: each MFMA followed by up to two LDS
// fragment reads and one global load.  The next half's fragments are then
// all requested within the first MFMAs and have the rest of the half to
// arrive, and the eight waves spread their LDS reads over the half instead of
// all reading in one burst.  (Left to itself the compiler sinks each read to
// just before its use and the MFMAs wait on LDS latency.)
template <int NM>
__device__ __forceinline__ void interleave_mfma_ds() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
  }
}

// The reduction loop of one workgroup tile.  Every wave issues its share of
// the loads and takes part in every barrier; only the MFMAs (and fragment
// reads) of row blocks past the end of the group are left out.
//
// Step s:  read k-slice 1 of step s, interleaved with the MFMAs on slice 0 |
// wait for this wave's reads and for the loads step s + 1 needs, barrier |
// issue the loads of step s + 4 and read slice 0 of step s + 1, interleaved
// with the MFMAs on slice 1.  Loads go out in step order (a step's pair
// before its quads), so what step s + 1 needs -- its quads, issued with step
// s + 1, and when s + 1 is even its pair, issued with step s + 2 -- has
// landed once no more than the loads of the later steps up to s + 3 are
// outstanding.  Steps past the reduction range load zeros; the loop runs a
// multiple of 4 steps.
template <int MIV, bool XS, bool YS, int MI, int NI, class XL, class YL, class XA, class YA>
__device__ __forceinline__ void reduce_tile(f32x16 (&acc)[MI][NI], XL& xl, YL& yl,
                                            const XA& xa, const YA& ya, const Bufs& xb,
                                            const Bufs& yb, int nk) {
  constexpr int LQ = (XS ? XL::kLoadsPerCall : 0) + (YS ? YL::kLoadsPerCall : 0);  // per quad step
  constexpr int LP = (XS ? 0 : XL::kLoadsPerCall) + (YS ? 0 : YL::kLoadsPerCall);  // per pair
  // Prologue: steps 0..3 in flight (pairs 0 and 1 with steps 1 and 3), step
  // 0 landed everywhere.
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    xl.prepare(s);
    yl.prepare(s);
    issue_step<XS, YS>(xl, yl, xb, yb, s, s);
  }
  wait_vmcnt<3 * LQ + LP>();
  __builtin_amdgcn_s_barrier();
  Frags<MI, NI> f0, f1;
  read_frags<MIV, XS, YS>(f0, xb, yb, 0, 0, xa, ya);
  // Four steps per iteration; the last iteration, when the reduction is
  // not a multiple of four steps, runs as a separate copy that leaves out
  // the MFMAs of the steps past the end (their operands are zeros), so the
  // full iterations keep their fixed schedule.
  auto four_steps = [&](int kt, auto guarded) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool live = !decltype(guarded)::value || kt + s < nk;
      xl.prepare(s);  // gathered operands: rows of the call this step issues
      yl.prepare(s);
      read_frags<MIV, XS, YS>(f1, xb, yb, s, 1, xa, ya);
      if (live) mfma_step<MIV>(acc, f0);
      interleave_mfma_ds<MIV * NI>();
      __builtin_amdgcn_sched_barrier(0);
      // Issued after the loads step s + 1 needs: steps s + 2 and s + 3, minus
      // the pair of step s + 2 when that is the pair step s + 1 needs.
      if ((s & 1) == 0)
        wait_vmcnt_lgkm0<2 * LQ + LP>();
      else
        wait_vmcnt_lgkm0<2 * LQ>();
      __builtin_amdgcn_s_barrier();
      issue_step<XS, YS>(xl, yl, xb, yb, s, kt + s + 4);
      read_frags<MIV, XS, YS>(f0, xb, yb, s + 1, 0, xa, ya);
      if (live) mfma_step<MIV>(acc, f1);
      interleave_mfma_ds<MIV * NI>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int kt = 0;
  for (; kt + 4 <= nk; kt += 4) four_steps(kt, std::false_type{});
  if (kt < nk) four_steps(kt, std::true_type{});
  // Drain the loads of the last steps before the workgroup's LDS is released.
  wait_vmcnt<0>();
}

// Workgroup: WGM x WGN waves, each computing a (BM / WGM) x (BN / WGN) piece.
// GLU (NN, bf16): the SwiGLU variant of GEMM 1 -- the tile's columns are
// interleaved 32-column blocks of gate and up weights for 128 hidden units
// (see Operand), so every wave holds the gate and the up value of the same
// units in the same lanes; the epilogue stores h and act = silu(g) * u.
// GX: the x operand is gathered through p.xrows (GEMM 1 with the SwiGLU
// epilogue, and the weight gradient).
template <int MODE, int BM, int BN, int WGM, int WGN, typename OutT, bool GLU = false,
          bool GX = false, bool GY = false>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_mfma_kernel(GemmArgs p) {
  constexpr bool XS = (MODE == kTN);  // x operand k-strided in memory
  constexpr bool YS = (MODE != kNT);  // y operand k-strided in memory
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MI = WM / 32, NI = WN / 32;
  static_assert(!GLU || (MODE == kNN && NI == 2 && sizeof(OutT) == 2),
                "the SwiGLU epilogue pairs a wave's two column blocks");
  static_assert(!GX || GLU || MODE == kTN || MODE == kNT,
                "gathered x: GEMM 1 with SwiGLU, data and weight gradients");
  static_assert(!GY || (MODE == kTN && !GX), "gathered y: weight gradient, x not gathered");
  // Elements per buffer: four quad buffers (k-strided) or two pair buffers.
  constexpr int XBE = XS ? BM * kBK : BM * 2 * kBK;
  constexpr int YBE = YS ? BN * kBK : BN * 2 * kBK;
  // One array per buffer: the compiler then tracks each buffer's loads
  // separately and waits only for the ones a read depends on.
  __shared__ __attribute__((aligned(1024))) uint16_t xb0[XBE];
  __shared__ __attribute__((aligned(1024))) uint16_t xb1[XBE];
  __shared__ alignas(XS ? 1024 : 16) uint16_t xb2[XS ? XBE : 8];
  __shared__ alignas(XS ? 1024 : 16) uint16_t xb3[XS ? XBE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t yb0[YBE];
  __shared__ __attribute__((aligned(1024))) uint16_t yb1[YBE];
  __shared__ alignas(YS ? 1024 : 16) uint16_t yb2[YS ? YBE : 8];
  __shared__ alignas(YS ? 1024 : 16) uint16_t yb3[YS ? YBE : 8];

  TileInfo t;
  if (!resolve_tile<MODE, BM>(p, t)) return;
  // The tile is the same for the whole workgroup; say so, so that buffer
  // descriptors built from it live in scalar registers.
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.i0 = __builtin_amdgcn_readfirstlane(t.i0);
  t.j0 = __builtin_amdgcn_readfirstlane(t.j0);
  t.r_lo = __builtin_amdgcn_readfirstlane(t.r_lo);
  t.r_hi = __builtin_amdgcn_readfirstlane(t.r_hi);
  t.g0 = __builtin_amdgcn_readfirstlane(t.g0);
  t.g1 = __builtin_amdgcn_readfirstlane(t.g1);
  const int j0 = t.j0 * (GLU ? BN / 2 : BN);  // GLU: first hidden unit of the tile
  const long long KN = static_cast<long long>(p.K) * p.N;

  Operand xo{}, yo{};
  if constexpr (GLU) {
    const int F = p.N / 2;
    if constexpr (GX)
      xo = {static_cast<const uint16_t*>(p.x), p.K, t.g1 - t.i0, 0, 0, p.xrows + t.i0, p.xdiv,
            p.xphys, 0, p.xmagic, p.xshift};
    else
      xo = {static_cast<const uint16_t*>(p.x) + static_cast<long long>(t.i0) * p.K, p.K,
            t.g1 - t.i0, 0, 0};
    yo = {static_cast<const uint16_t*>(p.y) + t.e * KN, p.N, F - j0, F, j0};
  } else if constexpr (MODE == kNN) {
    xo = {static_cast<const uint16_t*>(p.x) + static_cast<long long>(t.i0) * p.K, p.K,
          t.g1 - t.i0, 0, 0};
    yo = {static_cast<const uint16_t*>(p.y) + t.e * KN + j0, p.N, p.N - j0, 0, 0};
  } else if constexpr (MODE == kNT) {
    if constexpr (GX)
      xo = {static_cast<const uint16_t*>(p.x), p.N, t.g1 - t.i0, 0, 0, p.xrows + t.i0, p.xdiv,
            p.xphys, 0, p.xmagic, p.xshift};
    else
      xo = {static_cast<const uint16_t*>(p.x) + static_cast<long long>(t.i0) * p.N, p.N,
            t.g1 - t.i0, 0, 0};
    yo = {static_cast<const uint16_t*>(p.y) + t.e * KN + static_cast<long long>(j0) * p.N, p.N,
          p.K - j0, 0, 0};
  } else if constexpr (GY) {
    xo = {static_cast<const uint16_t*>(p.x) + static_cast<long long>(t.r_lo) * p.K + t.i0, p.K,
          p.K - t.i0, 0, 0};
    yo = {static_cast<const uint16_t*>(p.y), p.N, p.N - j0, 0, 0, p.yrows, p.ydiv, p.yphys, j0,
          p.ymagic, p.yshift};
  } else if constexpr (GX) {
    xo = {static_cast<const uint16_t*>(p.x), p.K, p.K - t.i0, 0, 0, p.xrows, p.xdiv, p.xphys,
          t.i0, p.xmagic, p.xshift};
    yo = {static_cast<const uint16_t*>(p.y) + static_cast<long long>(t.r_lo) * p.N + j0, p.N,
          p.N - j0, 0, 0};
  } else {
    xo = {static_cast<const uint16_t*>(p.x) + static_cast<long long>(t.r_lo) * p.K + t.i0, p.K,
          p.K - t.i0, 0, 0};
    yo = {static_cast<const uint16_t*>(p.y) + static_cast<long long>(t.r_lo) * p.N + j0, p.N,
          p.N - j0, 0, 0};
  }
  DmaLoader<XS, BM, NW, GX> xl;
  DmaLoader<YS, BN, NW, GY> yl;
  xl.init(xo, t.r_lo, t.r_hi);
  yl.init(yo, t.r_lo, t.r_hi);

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int wm = wid / WGN, wn = wid % WGN;
  FragAddr<XS, BM, MI> xa;
  FragAddr<YS, BN, NI> ya;
  xa.init(wm * WM, lane);
  ya.init(wn * WN, lane);

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (t.r_hi - t.r_lo + kBK - 1) / kBK;
  if (nk > 0) {
    const Bufs xb = {{xb0, xb1, xb2, xb3}};
    const Bufs yb = {{yb0, yb1, yb2, yb3}};
    // Row blocks of this wave that hold rows of the tile (partial last tiles
    // of a group, or of K in the weight-gradient layout).
    const int rows = (MODE == kTN) ? p.K - t.i0 : t.g1 - t.i0;
    const int rem = rows - wm * WM;
    const int miv = rem <= 0 ? 0 : (rem >= WM ? MI : (rem + 31) / 32);
#define MOE_REDUCE(V) reduce_tile<V, XS, YS, MI, NI>(acc, xl, yl, xa, ya, xb, yb, nk)
    if (miv == MI) {
      MOE_REDUCE(MI);
    } else if constexpr (MI == 4) {
      if (miv == 3) MOE_REDUCE(3);
      else if (miv == 2) MOE_REDUCE(2);
      else if (miv == 1) MOE_REDUCE(1);
      else MOE_REDUCE(0);
    } else if constexpr (MI == 2) {
      if (miv == 1) MOE_REDUCE(1);
      else MOE_REDUCE(0);
    } else {
      MOE_REDUCE(0);
    }
#undef MOE_REDUCE
  }
  if constexpr (GX) {
    if ((__ballot(xl.g_bad) | xl.g_badmask) != 0 && lane == 0) note_index_error(MOE_IDXERR_GATHER);
  }
  if constexpr (GY) {
    if (yl.g_badmask != 0 && lane == 0) note_index_error(MOE_IDXERR_GATHER);
  }

  if constexpr (GLU) {
    // acc[i][0]: gate, acc[i][1]: up, of hidden unit j0 + wn * 32 + l % 32.
    // act is computed from the stored (bf16) h values, as the separate
    // activation kernel does.  Stores go through buffer descriptors over the
    // tile's valid rows of h and act (rows past the group are dropped); a
    // lane past the last hidden unit starts from an out-of-range offset.
    const int F = p.N / 2;
    const int rows = min(BM, t.g1 - t.i0);
    const __amdgpu_buffer_rsrc_t h_rs =
        make_rsrc(static_cast<uint16_t*>(p.out) + static_cast<long long>(t.i0) * p.N,
                  static_cast<long long>(rows) * p.N * 2);
    const __amdgpu_buffer_rsrc_t a_rs =
        make_rsrc(static_cast<uint16_t*>(p.out2) + static_cast<long long>(t.i0) * F,
                  static_cast<long long>(rows) * F * 2);
    const int f = j0 + wn * 32 + (lane & 31);
    const int lrow = wm * WM + (lane >> 5) * 4;
    const unsigned h_off = f < F ? static_cast<unsigned>((lrow * p.N + f) * 2) : kOOB;
    const unsigned a_off = f < F ? static_cast<unsigned>((lrow * F + f) * 2) : kOOB;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row_c = i * 32 + (r >> 2) * 8 + (r & 3);
        const unsigned ho = h_off + static_cast<unsigned>(row_c * p.N * 2);
        const unsigned ao = a_off + static_cast<unsigned>(row_c * F * 2);
        const uint16_t gb = f32_to_bf16(acc[i][0][r]), ub = f32_to_bf16(acc[i][1][r]);
        __builtin_amdgcn_raw_buffer_store_b16(gb, h_rs, ho, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(ub, h_rs, ho + static_cast<unsigned>(F * 2), 0, 0);
        const float g = bf16_to_f32(gb), u = bf16_to_f32(ub);
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(g * sigmoid_fast(g) * u), a_rs, ao, 0,
                                              0);
      }
    }
    return;
  }

  // Epilogue.  32x32 accumulator layout: lane l, register r holds
  // row (r/4)*8 + (l/32)*4 + r%4, column l%32.  Consecutive lanes write
  // consecutive columns, so each store instruction covers two 64-byte row
  // segments (bf16).  (Whole-tile stores leave every compute unit at once;
  // wider per-lane stores only make that burst denser.)  The stores go
  // through a buffer descriptor over the tile's valid rows, so rows past the
  // group (or past K) fall outside it and the hardware drops them; a lane
  // whose column is past the matrix gets an out-of-range offset.  Offsets
  // are 32-bit: row and column constants fold into scalar registers, and no
  // store needs a branch.
  {
    constexpr int SZ = sizeof(OutT);
    // Weight gradients are not read again in the pass: non-temporal stores
    // keep them from displacing the activations that the next kernels read
    // from the caches (full layer -0.7%).  Other results are read by the
    // next kernel and keep the default policy.
    constexpr int kOutCpol = MODE == kTN ? kCpolNonTemporal : 0;
    const int ld = (MODE == kNT) ? p.K : p.N;  // output row length
    const int row_end = (MODE == kTN) ? p.K : t.g1;
    const int rows = min(BM, row_end - t.i0);
    long long first;  // element index of the tile's (0, 0)
    if constexpr (MODE == kTN)
      first = (static_cast<long long>(t.slice) * p.E + t.e) * KN +
              static_cast<long long>(t.i0) * p.N + j0;
    else
      first = static_cast<long long>(t.i0) * ld + j0;
    const __amdgpu_buffer_rsrc_t out_rs =
        make_rsrc(static_cast<char*>(p.out) + first * SZ,
                  (static_cast<long long>(rows) * ld - j0) * SZ);
    // NT addend (or an empty range when there is none; never read then)
    const __amdgpu_buffer_rsrc_t add_rs =
        make_rsrc(MODE == kNT && p.add ? static_cast<const char*>(p.add) + first * 2
                                       : static_cast<const char*>(p.out),
                  MODE == kNT && p.add ? (static_cast<long long>(rows) * ld - j0) * 2 : 0);
    // Per lane and column block: its byte offset in the tile, or kOOB; the
    // row's offset (a multiple of the row length, below 2^31) is added to it,
    // which keeps kOOB-based offsets out of range.
    unsigned col_off[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int col = wn * WN + j * 32 + (lane & 31);
      col_off[j] = j0 + col < ld
                       ? static_cast<unsigned>(((wm * WM + (lane >> 5) * 4) * ld + col) * SZ)
                       : kOOB;
    }
    // Gathered NT (the data gradient of GEMM 2 reading dy through the row
    // map): output row p is scaled by row_scale[p] (the slot's gate weight)
    // before rounding; the scales of this lane's rows of block i are loaded
    // once for all its column blocks.
    constexpr bool kScaled = MODE == kNT && GX;
    const __amdgpu_buffer_rsrc_t sc_rs =
        make_rsrc(kScaled ? static_cast<const void*>(p.row_scale + t.i0) : p.out,
                  kScaled ? static_cast<long long>(rows) * 4 : 0);
    const unsigned sc_lane = static_cast<unsigned>((wm * WM + (lane >> 5) * 4) * 4);
    // The stores, with the (NT) addend read from the same offsets.
    auto store_all = [&](auto with_add) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        float sc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[r] = 1.f;
          if constexpr (kScaled)
            sc[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                sc_rs, sc_lane + static_cast<unsigned>((i * 32 + (r >> 2) * 8 + (r & 3)) * 4), 0,
                0));
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          // A block's addend values are all read before any of its stores
          // (the compiler cannot move a read across a possibly aliasing store).
          float addv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row_c = i * 32 + (r >> 2) * 8 + (r & 3);
            const unsigned off = col_off[j] + static_cast<unsigned>(row_c * ld * SZ);
            addv[r] = 0.f;
            if constexpr (decltype(with_add)::value)
              addv[r] = bf16_to_f32(static_cast<uint16_t>(
                  __builtin_amdgcn_raw_buffer_load_b16(add_rs, off, 0, 0)));
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row_c = i * 32 + (r >> 2) * 8 + (r & 3);
            const unsigned off = col_off[j] + static_cast<unsigned>(row_c * ld * SZ);
            float v = acc[i][j][r];
            if constexpr (kScaled) v *= sc[r];
            if constexpr (decltype(with_add)::value) v += addv[r];
            if constexpr (SZ == 2)
              __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), out_rs, off, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), out_rs, off, 0, kOutCpol);
          }
        }
      }
    };
    if (MODE == kNT && p.add)
      store_all(std::true_type{});
    else
      store_all(std::false_type{});
  }
}

// ------------------------------------------------------------------ float32 path
template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) {
  return bf16_to_f32(v);
}

constexpr int kSimtTile = 64;
constexpr int kSimtBK = 16;

template <int MODE, typename InT, typename OutT>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs p) {
  __shared__ float xs[kSimtBK][kSimtTile + 4];
  __shared__ float ys[kSimtBK][kSimtTile + 4];
  TileInfo t;
  if (!resolve_tile<MODE, kSimtTile>(p, t)) return;
  const int j0 = t.j0 * kSimtTile;
  const long long KN = static_cast<long long>(p.K) * p.N;
  const InT* X = static_cast<const InT*>(p.x);
  const InT* Y = static_cast<const InT*>(p.y);
  // (o, r) addressing as in the MFMA path.
  long long xld, yld;
  int xolim, yolim;
  bool xt, yt;
  if (MODE == kNN) {
    xld = p.K; xolim = t.g1; xt = false;
    Y += t.e * KN; yld = p.N; yolim = p.N; yt = true;
  } else if (MODE == kNT) {
    xld = p.N; xolim = t.g1; xt = false;
    Y += t.e * KN; yld = p.N; yolim = p.K; yt = false;
  } else {
    xld = p.K; xolim = p.K; xt = true;
    yld = p.N; yolim = p.N; yt = true;
  }
  // Four waves, each a 32x32 quarter of the 64x64 tile on the float32 matrix
  // cores (v_mfma_f32_32x32x2_f32: lane l supplies the row (column) l % 32 at
  // reduction index l / 32 of each operand).
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int wm = wv >> 1, wn = wv & 1;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  for (int r0 = t.r_lo; r0 < t.r_hi; r0 += kSimtBK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = threadIdx.x + q * kThreads;
      // direct: r fastest (contiguous); transposed: o fastest.
      int o, r;
      if (!xt) { o = idx / kSimtBK; r = idx % kSimtBK; } else { o = idx % kSimtTile; r = idx / kSimtTile; }
      int oa = t.i0 + o, ra = r0 + r;
      float v = 0.f;
      if (oa < xolim && ra < t.r_hi)
        v = to_f32(xt ? X[static_cast<long long>(ra) * xld + oa] : X[static_cast<long long>(oa) * xld + ra]);
      xs[r][o] = v;
      if (!yt) { o = idx / kSimtBK; r = idx % kSimtBK; } else { o = idx % kSimtTile; r = idx / kSimtTile; }
      oa = j0 + o;
      ra = r0 + r;
      v = 0.f;
      if (oa < yolim && ra < t.r_hi)
        v = to_f32(yt ? Y[static_cast<long long>(ra) * yld + oa] : Y[static_cast<long long>(oa) * yld + ra]);
      ys[r][o] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kSimtBK; kk += 2) {
      const float a = xs[kk + (lane >> 5)][wm * 32 + (lane & 31)];
      const float b = ys[kk + (lane >> 5)][wn * 32 + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // 32x32 accumulator layout: lane l, register r holds row
  // (r / 4) * 8 + (l / 32) * 4 + r % 4, column l % 32 of the wave's block.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    {
      const int row = wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      const int col = wn * 32 + (lane & 31);
      const int ra = t.i0 + row, ca = j0 + col;
      float v = acc[r];
      if (MODE == kNN) {
        if (ra < t.g1 && ca < p.N) {
          const long long o = static_cast<long long>(ra) * p.N + ca;
          if constexpr (sizeof(OutT) == 2) static_cast<uint16_t*>(p.out)[o] = f32_to_bf16(v);
          else static_cast<float*>(p.out)[o] = v;
        }
      } else if (MODE == kNT) {
        if (ra < t.g1 && ca < p.K) {
          const long long o = static_cast<long long>(ra) * p.K + ca;
          if (p.add) v += to_f32(static_cast<const InT*>(p.add)[o]);
          if constexpr (sizeof(OutT) == 2) static_cast<uint16_t*>(p.out)[o] = f32_to_bf16(v);
          else static_cast<float*>(p.out)[o] = v;
        }
      } else {
        if (ra < p.K && ca < p.N)
          static_cast<float*>(p.out)[t.e * KN + static_cast<long long>(ra) * p.N + ca] = v;
      }
    }
  }
}

// Sum of split-K partials: db[i] = sum_s part[s][i], in increasing s.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           long long n, int split,
                                                           float* __restrict__ db) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += gridDim.x * 256LL) {
    // Eight partials loaded at a time (all in flight), summed in slice order.
    float s = 0.f;
    for (int q0 = 0; q0 < split; q0 += 8) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = q0 + q < split ? part[(q0 + q) * n + i] : 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q0 + q < split) s += v[q];
    }
    db[i] = s;
  }
}

// ------------------------------------------------------------------ host side
struct Cfg {
  int bm, bn;
};

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Row tiles per band of the row-tiled tile order (order_in_group).  Measured
// (interleaved runs, whole layer): large-expert step 16.05 ms with row-major
// order, 15.68 ms with bands of 4, 15.60 ms with bands of 8 (GEMM 1's data
// gradient -8%, GEMM 2 forward -6%); OLMoE-like 3.015 / 3.016 / 2.98 ms.
constexpr int kRowGroup = 8;
int row_group_rows() { return kRowGroup; }

// Tile shape for the row-tiled modes from the mean rows per expert and the
// number of output columns.
Cfg pick_row_cfg(int M, int E, int ncols) {
  const double mean = static_cast<double>(M) / E;
  if (ncols <= 64) return {64, 64};
  if (mean < 96.0) return ncols >= 256 ? Cfg{64, 256} : Cfg{64, 64};
  const long long tiles256 = (ceil_div(M, 256) + E) * ceil_div(ncols, 256);
  if (tiles256 >= 512) return {256, 256};
  // Fewer 128x128 tiles than compute units (the large-expert router's
  // logits: 16384 x 128 outputs, 129 tiles) leave most of the chip idle;
  // 64x64 tiles (several per CU) spread the same work four times wider.
  const long long tiles128 = (ceil_div(M, 128) + E) * ceil_div(ncols, 128);
  if (tiles128 < 256) return {64, 64};
  return {128, 128};
}

Cfg pick_tn_cfg(int K, int N, int E) {
  if (N <= 64 || K <= 64) return {64, 64};
  const long long tiles256 = ceil_div(K, 256) * ceil_div(N, 256) * E;
  if (tiles256 >= 512) return {256, 256};
  return {128, 128};
}

int pick_split(int M, int K, int N, int E) {
  const Cfg c = pick_tn_cfg(K, N, E);
  const long long tiles = ceil_div(K, c.bm) * ceil_div(N, c.bn) * E;
  if (tiles >= 512) return 1;
  const long long mean_rows = M / E;
  long long s = ceil_div(512, tiles);
  const long long by_rows = mean_rows / 256;  // at least 4 stages of 64 rows per slice
  if (s > by_rows) s = by_rows;
  if (s > 64) s = 64;
  return static_cast<int>(s < 1 ? 1 : s);
}

// Wavefront grid of the MFMA workgroup for each tile shape (matches the
// instantiations launched by dispatch_mfma).
struct Waves {
  int m, n;
};
Waves waves_of(Cfg c) {
  if (c.bm == 256 && c.bn == 256) return {2, 4};
  if (c.bm == 64 && c.bn == 256) return {1, 4};
  return {2, 2};
}

// The MFMA kernels address operands through buffer descriptors with 32-bit
// byte offsets: every operand (and one expert's weights) stays below 2^31
// bytes.  Larger shapes take the float32 kernel.
bool mfma_ok(moe_dtype dt, int M, int K, int N) {
  const long long lim = 1ll << 30;  // elements of 2 bytes
  // Tile-relative store offsets (up to 256 rows of a float32 row of K or N
  // elements, added to the out-of-range base 2^31) must stay below 2^32.
  const int row_lim = 1 << 20;
  return dt == MOE_BF16 && K % 8 == 0 && N % 8 == 0 && K < row_lim && N < row_lim &&
         static_cast<long long>(M) * K < lim && static_cast<long long>(M) * N < lim &&
         static_cast<long long>(K) * N < lim;
}

// The MFMA kernels move 16-byte vectors: operands and results start on
// 16-byte boundaries (null pointers pass).
bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }

template <int MODE, int BM, int BN, int WGM, int WGN, typename OutT, bool GLU = false,
          bool GX = false, bool GY = false>
void launch_mfma(GemmArgs p, long long tiles_upper, hipStream_t st) {
  const long long grid = ceil_div(tiles_upper, 8) * 8;
  hipLaunchKernelGGL((gemm_mfma_kernel<MODE, BM, BN, WGM, WGN, OutT, GLU, GX, GY>),
                     dim3(static_cast<unsigned>(grid)), dim3(64 * WGM * WGN), 0, st, p);
}

template <int MODE, typename OutT, bool GX = false, bool GY = false>
void dispatch_mfma(Cfg c, GemmArgs p, hipStream_t st) {
  const int ncols = (MODE == kNN) ? p.N : (MODE == kNT ? p.K : p.N);
  p.ntn = static_cast<int>(ceil_div(ncols, c.bn));
  p.row_group = row_group_rows();
  long long upper;
  if (MODE == kTN) {
    // 8 XCDs x (tile rows per XCD, whole deals) x ntn
    p.ntm = static_cast<int>(ceil_div(p.K, c.bm));
    upper = ceil_div(static_cast<long long>(p.ntm) * p.E * p.split, 8 * kTnDeal) * 8 * kTnDeal *
            p.ntn;
  } else {
    upper = (ceil_div(p.M, c.bm) + p.E) * p.ntn;
  }
  if (c.bm == 256 && c.bn == 256)
    launch_mfma<MODE, 256, 256, 2, 4, OutT, false, GX, GY>(p, upper, st);
  else if (c.bm == 128 && c.bn == 128)
    launch_mfma<MODE, 128, 128, 2, 2, OutT, false, GX, GY>(p, upper, st);
  else if (c.bm == 64 && c.bn == 256)
    launch_mfma<MODE, 64, 256, 1, 4, OutT, false, GX, GY>(p, upper, st);
  else
    launch_mfma<MODE, 64, 64, 2, 2, OutT, false, GX, GY>(p, upper, st);
}

// GEMM 1 with the SwiGLU epilogue: tiles of 128 hidden units (gate and up
// columns interleaved), which needs two 32-column blocks per wave.
Cfg pick_glu_cfg(int M, int E, int N) {
  const Cfg c = pick_row_cfg(M, E, N);
  return c.bn == 64 ? Cfg{128, 128} : c;
}

template <bool GX = false>
void dispatch_glu(Cfg c, GemmArgs p, hipStream_t st) {
  p.ntn = static_cast<int>(ceil_div(p.N / 2, c.bn / 2));
  p.row_group = row_group_rows();
  const long long upper = (ceil_div(p.M, c.bm) + p.E) * p.ntn;
  if (c.bm == 256 && c.bn == 256)
    launch_mfma<kNN, 256, 256, 2, 4, uint16_t, true, GX>(p, upper, st);
  else if (c.bm == 64 && c.bn == 256)
    launch_mfma<kNN, 64, 256, 1, 4, uint16_t, true, GX>(p, upper, st);
  else
    launch_mfma<kNN, 128, 128, 2, 2, uint16_t, true, GX>(p, upper, st);
}

template <int MODE, typename InT, typename OutT>
void launch_simt(GemmArgs p, hipStream_t st) {
  const int ncols = (MODE == kNN) ? p.N : (MODE == kNT ? p.K : p.N);
  p.ntn = static_cast<int>(ceil_div(ncols, kSimtTile));
  p.split = 1;
  long long upper;
  if (MODE == kTN) {
    // 8 XCDs x (tile rows per XCD, whole deals) x ntn
    p.ntm = static_cast<int>(ceil_div(p.K, kSimtTile));
    upper = ceil_div(static_cast<long long>(p.ntm) * p.E, 8 * kTnDeal) * 8 * kTnDeal * p.ntn;
  } else {
    upper = (ceil_div(p.M, kSimtTile) + p.E) * p.ntn;
  }
  const long long grid = ceil_div(upper, 8) * 8;
  hipLaunchKernelGGL((gemm_f32_kernel<MODE, InT, OutT>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, st, p);
}

// Row map of a gathered operand: logical row p is physical row rows[p] / div
// of an array of `phys` rows of `ld` elements.  The MFMA loaders address it
// with 32-bit byte offsets.
// ceil(2^32 / d) mod 2^32 for div_rows.
unsigned div_magic(int d) {
  const unsigned long long dd = static_cast<unsigned long long>(d < 1 ? 1 : d);
  return static_cast<unsigned>(((1ull << 32) + dd - 1) / dd);
}

// log2(d) for a power of two d, else -1.
int div_shift(int d) {
  if (d < 1 || (d & (d - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < d) ++s;
  return s;
}

moe_status check_gather(const char* fn, const int32_t* rows, int div, int phys, int ld) {
  (void)fn;
  MOE_REQUIRE(rows != nullptr, MOE_ERR_INVALID_ARG, "gathered operand: null row map");
  MOE_REQUIRE(div >= 1 && phys >= 1, MOE_ERR_INVALID_ARG,
              "gathered operand: row divisor and physical rows must be >= 1");
  MOE_REQUIRE(static_cast<long long>(phys) * ld < (1ll << 30) && phys < (1 << 24) &&
                  ld < (1 << 23),
              MOE_ERR_UNSUPPORTED,
              "gathered operand: needs physical rows * row length < 2^30, rows < 2^24 and row "
              "length < 2^23");
  return MOE_OK;
}

moe_status check_gemm(const void* offsets, int M, int K, int N, int E, moe_dtype dt) {
  MOE_REQUIRE(offsets != nullptr, MOE_ERR_INVALID_ARG, "grouped gemm: null offsets");
  MOE_REQUIRE(M >= 1 && K >= 1 && N >= 1 && E >= 1, MOE_ERR_INVALID_ARG,
              "grouped gemm: M, K, N, E must be >= 1");
  MOE_REQUIRE(dtype_ok(dt), MOE_ERR_UNSUPPORTED, "grouped gemm: unknown dtype");
  MOE_REQUIRE(static_cast<long long>(M) * (K > N ? K : N) < (1ll << 40), MOE_ERR_UNSUPPORTED,
              "grouped gemm: operand too large");
  MOE_REQUIRE(static_cast<long long>(E) * K * N < (1ll << 40), MOE_ERR_UNSUPPORTED,
              "grouped gemm: weight tensor too large");
  return MOE_OK;
}

}  // namespace

moe_status index_record_gemm(hipStream_t st, unsigned int* bits, bool clear) {
  return take_index_flags(st, bits, clear);
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_grouped_gemm_workspace_size(int M, int K, int N, int E, moe_dtype dtype) {
  if (M < 1 || K < 1 || N < 1 || E < 1 || !mfma_ok(dtype, M, K, N)) return 0;
  const int s = pick_split(M, K, N, E);
  if (s <= 1) return 0;
  return static_cast<size_t>(s) * E * K * N * sizeof(float);
}

extern "C" moe_status moe_grouped_gemm_plan(int product, int M, int K, int N, int E,
                                            moe_dtype dtype, int* tile_m, int* tile_n,
                                            int* waves_m, int* waves_n, int* split, int* mfma) {
  clear_error();
  MOE_REQUIRE(product >= 0 && product <= 3, MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_plan: product must be 0, 1, 2 or 3");
  MOE_REQUIRE(M >= 1 && K >= 1 && N >= 1 && E >= 1, MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_plan: sizes must be >= 1");
  MOE_REQUIRE(dtype_ok(dtype), MOE_ERR_UNSUPPORTED, "moe_grouped_gemm_plan: unknown dtype");
  const bool m = mfma_ok(dtype, M, K, N);
  Cfg c{kSimtTile, kSimtTile};
  int s = 1;
  if (m) {
    if (product == 0) c = pick_row_cfg(M, E, N);
    else if (product == 3) c = pick_glu_cfg(M, E, N);
    else if (product == 1) c = pick_row_cfg(M, E, K);
    else {
      c = pick_tn_cfg(K, N, E);
      s = pick_split(M, K, N, E);
    }
  }
  int wgm = 0, wgn = 0;
  if (m) {
    const Waves w = waves_of(c);
    wgm = w.m;
    wgn = w.n;
  }
  if (tile_m) *tile_m = c.bm;
  if (tile_n) *tile_n = c.bn;
  if (waves_m) *waves_m = wgm;
  if (waves_n) *waves_n = wgn;
  if (split) *split = s;
  if (mfma) *mfma = m ? 1 : 0;
  return MOE_OK;
}

extern "C" moe_status moe_grouped_gemm_swiglu_fwd(const void* a, const void* b,
                                                  const int32_t* offsets, int M, int K, int F,
                                                  int E, moe_dtype dtype, void* h, void* act,
                                                  moe_stream_t stream) {
  clear_error();
  MOE_REQUIRE(F >= 1 && F <= (1 << 29), MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_swiglu_fwd: F out of range");
  const int N = 2 * F;
  if (moe_status s = check_gemm(offsets, M, K, N, E, dtype)) return s;
  MOE_REQUIRE(a && b && h && act, MOE_ERR_INVALID_ARG, "moe_grouped_gemm_swiglu_fwd: null pointer");
  MOE_REQUIRE(F % 8 == 0, MOE_ERR_UNSUPPORTED,
              "moe_grouped_gemm_swiglu_fwd: F must be a multiple of 8");
  if (mfma_ok(dtype, M, K, N)) {
    MOE_REQUIRE(aligned16(a) && aligned16(b) && aligned16(h) && aligned16(act),
                MOE_ERR_INVALID_ARG,
                "moe_grouped_gemm_swiglu_fwd: bf16 operands and results must be 16-byte aligned");
    GemmArgs p{a, b, nullptr, h, offsets, M, K, N, E, 0, 0, 1, act};
    dispatch_glu(pick_glu_cfg(M, E, N), p, as_stream(stream));
    return check_launch("moe_grouped_gemm_swiglu_fwd");
  }
  // Shapes the MFMA path does not take: the GEMM, then the activation kernel.
  if (moe_status s = moe_grouped_gemm_fwd(a, b, offsets, M, K, N, E, dtype, h, dtype, nullptr, 0,
                                          stream))
    return s;
  return moe_act_fwd(h, M, F, dtype, act, stream);
}

extern "C" moe_status moe_grouped_gemm_swiglu_fwd_gather(
    const void* x, const int32_t* x_rows, int x_div, int x_phys, const void* b,
    const int32_t* offsets, int M, int K, int F, int E, moe_dtype dtype, void* h, void* act,
    moe_stream_t stream) {
  clear_error();
  MOE_REQUIRE(F >= 1 && F <= (1 << 29), MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_swiglu_fwd_gather: F out of range");
  const int N = 2 * F;
  if (moe_status s = check_gemm(offsets, M, K, N, E, dtype)) return s;
  MOE_REQUIRE(x && b && h && act, MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_swiglu_fwd_gather: null pointer");
  if (moe_status s = check_gather("moe_grouped_gemm_swiglu_fwd_gather", x_rows, x_div, x_phys, K))
    return s;
  MOE_REQUIRE(F % 8 == 0 && mfma_ok(dtype, M, K, N), MOE_ERR_UNSUPPORTED,
              "moe_grouped_gemm_swiglu_fwd_gather: needs the bf16 MFMA path (K, F multiples of 8)");
  MOE_REQUIRE(aligned16(x) && aligned16(b) && aligned16(h) && aligned16(act), MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_swiglu_fwd_gather: operands and results must be 16-byte aligned");
  GemmArgs p{x, b, nullptr, h, offsets, M, K, N, E, 0, 0, 1, act, x_rows, x_div, x_phys,
             div_magic(x_div), div_shift(x_div)};
  dispatch_glu<true>(pick_glu_cfg(M, E, N), p, as_stream(stream));
  return check_launch("moe_grouped_gemm_swiglu_fwd_gather");
}

extern "C" moe_status moe_grouped_gemm_fwd(const void* a, const void* b, const int32_t* offsets,
                                           int M, int K, int N, int E, moe_dtype ab_dtype,
                                           void* c, moe_dtype c_dtype, void* ws, size_t ws_bytes,
                                           moe_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  clear_error();
  if (moe_status s = check_gemm(offsets, M, K, N, E, ab_dtype)) return s;
  MOE_REQUIRE(a && b && c, MOE_ERR_INVALID_ARG, "moe_grouped_gemm_fwd: null pointer");
  MOE_REQUIRE(dtype_ok(c_dtype), MOE_ERR_UNSUPPORTED, "moe_grouped_gemm_fwd: bad c_dtype");
  MOE_REQUIRE(!(ab_dtype == MOE_F32 && c_dtype == MOE_BF16), MOE_ERR_UNSUPPORTED,
              "moe_grouped_gemm_fwd: float32 inputs need a float32 output");
  if (mfma_ok(ab_dtype, M, K, N))
    MOE_REQUIRE(aligned16(a) && aligned16(b) && aligned16(c), MOE_ERR_INVALID_ARG,
                "moe_grouped_gemm_fwd: bf16 operands and result must be 16-byte aligned");
  GemmArgs p{a, b, nullptr, c, offsets, M, K, N, E, 0, 0, 1};
  hipStream_t st = as_stream(stream);
  if (mfma_ok(ab_dtype, M, K, N)) {
    const Cfg cfg = pick_row_cfg(M, E, N);
    if (c_dtype == MOE_BF16) dispatch_mfma<kNN, uint16_t>(cfg, p, st);
    else dispatch_mfma<kNN, float>(cfg, p, st);
  } else if (ab_dtype == MOE_BF16) {
    if (c_dtype == MOE_BF16) launch_simt<kNN, uint16_t, uint16_t>(p, st);
    else launch_simt<kNN, uint16_t, float>(p, st);
  } else {
    launch_simt<kNN, float, float>(p, st);
  }
  return check_launch("moe_grouped_gemm_fwd");
}

namespace moe {
namespace {

moe_status grouped_gemm_bwd(const void* a, const int32_t* a_rows, int a_div, int a_phys,
                            const void* b, const void* dc, const int32_t* offsets, int M, int K,
                            int N, int E, moe_dtype dtype, void* da, const void* da_add,
                            float* db, void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (moe_status s = check_gemm(offsets, M, K, N, E, dtype)) return s;
  MOE_REQUIRE(dc != nullptr, MOE_ERR_INVALID_ARG, "moe_grouped_gemm_bwd: null dc");
  MOE_REQUIRE(da == nullptr || b != nullptr, MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_bwd: da needs b");
  MOE_REQUIRE(db == nullptr || a != nullptr, MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_bwd: db needs a");
  const bool use_mfma = mfma_ok(dtype, M, K, N);
  if (use_mfma)
    MOE_REQUIRE(aligned16(a) && aligned16(b) && aligned16(dc) && aligned16(da) &&
                    aligned16(da_add) && aligned16(db),
                MOE_ERR_INVALID_ARG,
                "moe_grouped_gemm_bwd: bf16 operands and results must be 16-byte aligned");
  int split = 1;
  if (db && use_mfma) {
    split = pick_split(M, K, N, E);
    if (split > 1) {
      const size_t need = moe_grouped_gemm_workspace_size(M, K, N, E, dtype);
      MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE,
                  "moe_grouped_gemm_bwd: workspace too small");
      MOE_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 15) == 0, MOE_ERR_WORKSPACE,
                  "moe_grouped_gemm_bwd: workspace must be 16-byte aligned");
    }
  }
  hipStream_t st = as_stream(stream);
  if (da) {
    GemmArgs p{dc, b, da_add, da, offsets, M, K, N, E, 0, 0, 1};
    if (use_mfma) {
      dispatch_mfma<kNT, uint16_t>(pick_row_cfg(M, E, K), p, st);
    } else if (dtype == MOE_BF16) {
      launch_simt<kNT, uint16_t, uint16_t>(p, st);
    } else {
      launch_simt<kNT, float, float>(p, st);
    }
    if (moe_status s = check_launch("moe_grouped_gemm_bwd/da")) return s;
  }
  if (db) {
    if (use_mfma) {
      // Hot-first group order for groups long enough that their tiles'
      // lengths matter (at least 128 rows on average).
      const int hot_first = split == 1 && E >= 2 && E <= 256 && M / E >= 128 ? 1 : 0;
      GemmArgs p{a, dc, nullptr, split > 1 ? ws : static_cast<void*>(db), offsets, M, K, N, E,
                 0, 0, split, nullptr, a_rows, a_div, a_phys, div_magic(a_div),
                 div_shift(a_div), hot_first};
      if (a_rows)
        dispatch_mfma<kTN, float, true>(pick_tn_cfg(K, N, E), p, st);
      else
        dispatch_mfma<kTN, float>(pick_tn_cfg(K, N, E), p, st);
      if (moe_status s = check_launch("moe_grouped_gemm_bwd/db")) return s;
      if (split > 1) {
        const long long n = static_cast<long long>(E) * K * N;
        long long g = ceil_div(n, 256);
        if (g > 8192) g = 8192;
        hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<unsigned>(g)), dim3(256), 0, st,
                           static_cast<const float*>(ws), n, split, db);
      }
    } else {
      GemmArgs p{a, dc, nullptr, db, offsets, M, K, N, E, 0, 0, 1};
      if (dtype == MOE_BF16) launch_simt<kTN, uint16_t, float>(p, st);
      else launch_simt<kTN, float, float>(p, st);
    }
    if (moe_status s = check_launch("moe_grouped_gemm_bwd/db")) return s;
  }
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_grouped_gemm_bwd(const void* a, const void* b, const void* dc,
                                           const int32_t* offsets, int M, int K, int N, int E,
                                           moe_dtype dtype, void* da, const void* da_add,
                                           float* db, void* ws, size_t ws_bytes,
                                           moe_stream_t stream) {
  clear_error();
  return grouped_gemm_bwd(a, nullptr, 1, 0, b, dc, offsets, M, K, N, E, dtype, da, da_add, db, ws,
                          ws_bytes, stream);
}

extern "C" moe_status moe_grouped_gemm_bwd_gather(const void* a, const int32_t* a_rows,
                                                  int a_div, int a_phys, const void* b,
                                                  const void* dc, const int32_t* offsets, int M,
                                                  int K, int N, int E, moe_dtype dtype, void* da,
                                                  const void* da_add, float* db, void* ws,
                                                  size_t ws_bytes, moe_stream_t stream) {
  clear_error();
  if (moe_status s = check_gather("moe_grouped_gemm_bwd_gather", a_rows, a_div, a_phys, K))
    return s;
  MOE_REQUIRE(mfma_ok(dtype, M, K, N), MOE_ERR_UNSUPPORTED,
              "moe_grouped_gemm_bwd_gather: needs the bf16 MFMA path (K, N multiples of 8)");
  return grouped_gemm_bwd(a, a_rows, a_div, a_phys, b, dc, offsets, M, K, N, E, dtype, da, da_add,
                          db, ws, ws_bytes, stream);
}

extern "C" moe_status moe_grouped_gemm_bwd_scaled_gather(
    const void* a_scaled, const void* b, const void* dy, const int32_t* dc_rows, int dc_div,
    int dc_phys, const float* row_scale, const int32_t* offsets, int M, int K, int N, int E,
    moe_dtype dtype, void* da, float* db, void* ws, size_t ws_bytes, moe_stream_t stream) {
  clear_error();
  if (moe_status s = check_gemm(offsets, M, K, N, E, dtype)) return s;
  MOE_REQUIRE(dy != nullptr && row_scale != nullptr, MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_bwd_scaled_gather: null dy or row_scale");
  MOE_REQUIRE(da == nullptr || b != nullptr, MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_bwd_scaled_gather: da needs b");
  MOE_REQUIRE(db == nullptr || a_scaled != nullptr, MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_bwd_scaled_gather: db needs a_scaled");
  if (moe_status s = check_gather("moe_grouped_gemm_bwd_scaled_gather", dc_rows, dc_div, dc_phys, N))
    return s;
  MOE_REQUIRE(mfma_ok(dtype, M, K, N), MOE_ERR_UNSUPPORTED,
              "moe_grouped_gemm_bwd_scaled_gather: needs the bf16 MFMA path (K, N multiples of 8)");
  MOE_REQUIRE(aligned16(a_scaled) && aligned16(b) && aligned16(dy) && aligned16(da) &&
                  aligned16(db),
              MOE_ERR_INVALID_ARG,
              "moe_grouped_gemm_bwd_scaled_gather: operands and results must be 16-byte aligned");
  int split = 1;
  if (db) {
    split = pick_split(M, K, N, E);
    if (split > 1) {
      const size_t need = moe_grouped_gemm_workspace_size(M, K, N, E, dtype);
      MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE,
                  "moe_grouped_gemm_bwd_scaled_gather: workspace too small");
      MOE_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 15) == 0, MOE_ERR_WORKSPACE,
                  "moe_grouped_gemm_bwd_scaled_gather: workspace must be 16-byte aligned");
    }
  }
  hipStream_t st = as_stream(stream);
  const unsigned magic = div_magic(dc_div);
  const int shift = div_shift(dc_div);
  if (da) {
    // da = diag(row_scale) (dy_g @ b^T): the NT kernel with its x operand
    // gathered and the scale in the epilogue.
    GemmArgs p{dy, b, nullptr, da, offsets, M, K, N, E, 0, 0, 1, nullptr, dc_rows, dc_div,
               dc_phys, magic, shift};
    p.row_scale = row_scale;
    dispatch_mfma<kNT, uint16_t, true>(pick_row_cfg(M, E, K), p, st);
    if (moe_status s = check_launch("moe_grouped_gemm_bwd_scaled_gather/da")) return s;
  }
  if (db) {
    // db = a_scaled^T @ dy_g: the TN kernel with its y operand gathered.
    const int hot_first = split == 1 && E >= 2 && E <= 256 && M / E >= 128 ? 1 : 0;
    GemmArgs p{a_scaled, dy, nullptr, split > 1 ? ws : static_cast<void*>(db), offsets, M, K,
               N, E, 0, 0, split};
    p.hot_first = hot_first;
    p.yrows = dc_rows;
    p.ydiv = dc_div;
    p.yphys = dc_phys;
    p.ymagic = magic;
    p.yshift = shift;
    dispatch_mfma<kTN, float, false, true>(pick_tn_cfg(K, N, E), p, st);
    if (moe_status s = check_launch("moe_grouped_gemm_bwd_scaled_gather/db")) return s;
    if (split > 1) {
      const long long n = static_cast<long long>(E) * K * N;
      long long g = ceil_div(n, 256);
      if (g > 8192) g = 8192;
      hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<unsigned>(g)), dim3(256), 0, st,
                         static_cast<const float*>(ws), n, split, db);
      if (moe_status s = check_launch("moe_grouped_gemm_bwd_scaled_gather/db")) return s;
    }
  }
  return MOE_OK;
}
