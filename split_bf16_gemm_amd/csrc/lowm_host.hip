// lowm_host.hip -- host side of the low-M split-K bf16 GEMM for AMD Instinct
// MI355X (gfx950): argument validation, tactic and split_k choice, workspace
// sizing, launch, the consumer-side wait of the push epilogue, and the C ABI
// of include/lowm.h.  The kernels are in lowm_kernels.cuh, instantiated per
// output kind in lowm_inst_*.hip.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "lowm_types.h"

namespace lowm {

const Table& table() {
  static const Table t = [] {
    Table x{};
    fill_table_bf16(x);
    fill_table_f32(x);
    fill_table_push(x);
    return x;
  }();
  return t;
}

thread_local int g_last_hip_error = 0;
StressArgs g_stress = {0u, -1, -1, 0, 0, -1, 0u, nullptr};
// Workgroups the trace buffer has room for (stress build; 0 without one).
size_t g_trace_capacity = 0;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_sizes(int M, int N, int K, int S) {
  if (M <= 0 || N <= 0 || K <= 0 || S < 1) return LOWM_ERR_INVALID_ARG;
  if (M > LOWM_MAX_M || S > LOWM_MAX_SPLIT_K) return LOWM_ERR_UNSUPPORTED;
  if (K % (kVecK * S) != 0) return LOWM_ERR_UNSUPPORTED;
  return LOWM_OK;
}

size_t counter_bytes(int N) { return (size_t)4 * kCtrStride * ((N + 15) / 16); }
// Every tile width 16*RG divides this, so tiles * BN <= round_up(N, kPartialPad).
constexpr size_t kPartialPad = 64;

int variant_index(const lowm_tactic& t) {
  for (int i = 0; i < kNumVariants; ++i)
    if (kVariants[i].stage == t.stage && kVariants[i].unroll == t.unroll &&
        kVariants[i].stages == t.stages)
      return i;
  return -1;
}

int rows_index(int rows) { return rows % 16 == 0 ? rg_index(rows / 16) : -1; }

KernelFn lookup(bool f32out, int act, int M, const lowm_tactic& t, bool push = false) {
  if (t.waves != kWaves) return nullptr;
  const int ri = rows_index(t.rows);
  const int vi = variant_index(t);
  if (ri < 0 || vi < 0 || M < 1 || M > LOWM_MAX_M) return nullptr;
  return table().fn[push ? kOutPush : f32out ? kOutF32 : kOutBf16][act][(M + 15) / 16 - 1][ri][vi];
}

// Largest activation slice staged in LDS (bytes, padding included).
constexpr size_t kActLdsMax = 48 * 1024;
size_t act_lds_bytes(int M, int nvec) { return (size_t)M * (nvec + 1) * 16; }

// The kernel a launch with tactic t runs (defined below).
KernelFn select_kernel(bool f32out, int M, int S, int nvec, const lowm_tactic& t,
                       size_t* dyn_lds, bool push = false);

// Default tactic, in order: quarter-rows tiles for 49..64 rows without
// split-K where their grid fits the device once, quarter tiles where the
// rules below name them, panel tiles above 16 rows, line-pair tiles, the
// register ring.
// Line-pair tiles (the default for M <= 4 with split-K, where the K slice is
// whole 64-K line pairs per wavefront): 16 rows, a ring of 4 slots for
// M <= 4 with 8..15 pairs per wavefront and of 2 otherwise.  Measured on
// MI355X at the three shapes of the pages (N 6144 K 4096 split_k 2,
// N 2304 K 12288 split_k 4, N 49152 K 4096 split_k 2) and M 1 at split_k
// 2..8: 2-11 % faster than the quarter tiles there (the tile's last rank
// folds without the exchange's round trips), 19-25 % faster than the
// register ring.
// Register ring (slices that are not whole 64-K steps): tiles of 16 weight
// rows for M <= 16 and 32 above (two row groups share each activation load);
// each of the four wavefronts streams cpw = ceil(chunks / 4) contiguous
// chunks of its slice.  When cpw <= 16 the best ring issues the whole range
// in its first stage (unroll = the smallest power of two >= cpw, 2 stages);
// for longer ranges a 4-chunk, 2-stage ring beats deeper ones.  Fall back to
// other rings, then the LDS variants, when the build has no such
// instantiation for this M.
int pick(int M, int N, int K, int S, lowm_tactic* t, bool push = false) {
  const int rc = check_sizes(M, N, K, S);
  if (rc != LOWM_OK) return rc;
  const int nvec = K / S / kVecK;
  const int cpw = ((nvec + 3) / 4 + kWaves - 1) / kWaves;
  const int act = (nvec % 64 == 0 && act_lds_bytes(M, nvec) <= kActLdsMax) ? 1 : 0;
  int first_unroll = 4;
  if (cpw <= 16) {
    while (first_unroll < cpw) first_unroll *= 2;
  }
  const Variant first = {kStageReg, first_unroll, 2};
  static const Variant others[] = {{kStageReg, 4, 2}, {kStageReg, 8, 2}, {kStageLds, 4, 2},
                                   {kStageLds, 4, 3}};
  t->rows = M <= 16 ? 16 : 32;
  // The launch stages the activation slice in LDS when `act` is 1 and the
  // build has that instantiation, else it loads activation operands from L2;
  // the tactic must exist in the mode the launch will use.
  auto provides = [&](const Variant& v) {
    t->stage = v.stage;
    t->unroll = v.unroll;
    t->stages = v.stages;
    t->waves = kWaves;
    for (int f = 0; f < 2; ++f) {
      const bool f32 = f == 1;
      if (!(act && lookup(f32, 1, M, *t)) && !lookup(f32, 0, M, *t)) return false;
    }
    return true;
  };
  // Quarter tiles (each wavefront one quarter of the K slice for the whole
  // tile, both operands through its own LDS ring).  Measured on MI355X
  // (bench.py --tactic-matrix) at M 1..64, N 1536..24576, K 4096..16384,
  // split_k 1..8 against the line-pair and panel tiles:
  //   - split_k 1, M <= 32: 32-row tiles (16-row tiles above 16 rows where
  //     that still gives no more than 192 workgroups): M 16, N 6144, K 4096
  //     10.9 us against 12.3 (line pairs), M 32 12.9 against 13.8 (panel),
  //     M 4 10.1 against 10.5, M 16 N 24576 32.0 against 33.4.  Ring 4 where
  //     every workgroup fits on the device at once (at most 256 32-row
  //     workgroups up to 16 rows, where ring 3 would fit two per CU; always
  //     above, where both fit one): M 1 / 4 / 8 / 32, N 6144 9.61 / 9.80 /
  //     10.01 / 12.83 us against 9.86 / 10.00 / 10.18 / 12.96 with ring 3;
  //   - split_k >= 2, 4 < M <= 16: the tile width and ring by the number of
  //     32-row workgroups W: <= 96 rows 16 ring 3, <= 192 rows 32 ring 3,
  //     then rows 48 ring 3 where those number <= 256 (one per CU), else
  //     rows 48 ring 2 up to split_k 4 and rows 32 ring 2 above (M 16 N 6144
  //     split_k 2 / 4 / 8: 11.6 / 12.3 / 15.5 us; split_k 2 with rows 16
  //     ring 2 12.6, M 8 11.4 against 11.6; in two or more rounds rows 48
  //     ring 2 beat rows 32 ring 2 by 1.6-3 % at split_k 2 and 4, M 16
  //     N 12288 / 24576 split_k 2 19.3 / 36.7 against 19.9 / 37.7, and lose
  //     by 5 % at split_k 8, M 8 / 16 N 6144 15.6 / 16.4 against 14.9 / 15.6);
  //   - split_k 1, M > 32 (where the quarter-rows tiles above do not
  //     apply): the tile width of 16..64 rows with the fewest rounds of 256
  //     workgroups times rows loaded per K step (activation blocks plus
  //     weight rows); ring 3 where it fits, else 2.  Every measured winner
  //     is that choice: M 64 N 8192 / 12288 / 16384 / 24576 rows 32 / 48 /
  //     64 / 48 (18.1 / 23.7 / 29.2 / 45.5 us, the others 18.1-24.5 /
  //     26.2-31.5 / 35.1-40.6 / 50.6-52.3), M 40 N 6144 rows 32 (14.7),
  //     M 40 N 24576 and M 48 N 12288 rows 48 (37.6, 20.8 against 45.0-46.0
  //     and 23.6-28.9);
  //   - split_k 2, 16 < M <= 32: the width with the fewest rounds times rows
  //     loaded (as for 33..64 rows below), ring 3; it picks every measured
  //     winner: M 32 N 3072 / 6144 / 12288 rows 32 / 48 / 48 (10.1 / 13.2 /
  //     25.1 us, the best other width 11.5 / 14.2 / 26.8), M 24 N 24576
  //     rows 64 (44.6, against 45.0 for rows 32).
  // The line-pair tiles stay faster for M <= 4 with split_k >= 2 (their last
  // rank folds without the exchange's round trips), the panel tiles for
  // M > 32 with split-K and for split_k >= 4 above 16 rows.  Every choice
  // below depends on N only through the tile width and ring, which do not
  // change the summation order, so a batched launch (picked for its
  // narrowest GEMM) gives each GEMM the bits of its single call.
  if (nvec % 32 == 0) {
    const long w16 = (long)((N + 15) / 16) * S;
    const long w32 = (long)((N + 31) / 32) * S;
    const long w48 = (long)((N + 47) / 48) * S;
    auto quarter = [&](int rows, int ring) {
      t->rows = rows;
      return provides({kStageQuarter, 2, ring});
    };
    // The tile width of 16..64 weight rows whose workgroups move the fewest
    // bytes in all: rounds of up to 256 workgroups (one per CU) times the rows
    // each loads per K step (its 16-row blocks of activations plus its weight
    // rows); returns the width in 16-row groups.
    auto fewest_rows = [&]() {
      const long act_rows = 16L * ((M + 15) / 16);
      int best = 1;
      long best_cost = 0;
      for (int nb = 1; nb <= 4; ++nb) {
        const long wgs = (long)((N + 16 * nb - 1) / (16 * nb)) * S;
        const long cost = (wgs + 255) / 256 * (act_rows + 16 * nb);
        if (nb == 1 || cost < best_cost) {
          best = nb;
          best_cost = cost;
        }
      }
      return best;
    };
    // Quarter-rows tiles for 49..64 rows without split-K (not for the push
    // epilogue): two workgroups per tile, one per 32-row block, and the
    // narrowest tile width (16..48 columns) at which the blocks fill the 256
    // CUs once; otherwise the rules below.  Measured on MI355X (bench.py
    // --tactic-matrix) at M 64, K 4096 against the quarter tiles: N 2048 /
    // 4096 / 6144 9.3 / 12.2 / 15.4 us against 13.3 / 14.2 / 17.0; N 6144
    // K 8192 29.8 against 31.6; N 2304 K 12288 31.0 against 35.2.  Each
    // workgroup moves 32 activation rows and 16..48 weight rows per K step
    // where the quarter tiles move M and 16..32: at 33..48 rows that is no
    // fewer bytes (M 40, N 6144: 15.5 against 14.7), and at N 8192 the
    // 64-column blocks lose to 32-row quarter tiles (18.7 against 18.1).
    // Same summation order, so the same bits, as the quarter tiles.
    if (M > 48 && S == 1 && !push) {
      const long blocks = (M + 31) / 32;
      for (int nb = 1; nb <= 3; ++nb)
        if ((long)((N + 16 * nb - 1) / (16 * nb)) * blocks <= 256) {
          t->rows = 16 * nb;
          t->stage = kStageQuarterRows;
          t->unroll = 2;
          t->stages = nb == 1 ? 4 : 3;
          t->waves = kWaves;
          bool ok = true;
          for (int f = 0; f < 2; ++f) {
            size_t dyn = 0;
            ok = ok && select_kernel(f == 1, M, 1, nvec, *t, &dyn) != nullptr;
          }
          if (ok) return LOWM_OK;
          break;
        }
    }
    if (M <= 16 && S == 1) {
      if ((w32 <= 256 && quarter(32, 4)) || quarter(32, 3)) return LOWM_OK;
    } else if (M > 4 && M <= 16) {
      if (w32 <= 96 ? quarter(16, 3)
                    : w32 <= 192 ? quarter(32, 3)
                                 : w48 <= 256 ? quarter(48, 3)
                                              : S <= 4 ? quarter(48, 2) : quarter(32, 2))
        return LOWM_OK;
    } else if (M > 16 && M <= 32 && S == 1) {
      if (w16 <= 192 ? quarter(16, 3) : (quarter(32, 4) || quarter(32, 3))) return LOWM_OK;
    } else if (M > 32 && S == 1) {
      const int best = fewest_rows();
      const int ring = best <= 2 || (best == 3 && M <= 48) ? 3 : 2;
      if (quarter(16 * best, ring) || quarter(16 * best, 2)) return LOWM_OK;
    } else if (M > 16 && M <= 32 && S == 2) {
      if (quarter(16 * fewest_rows(), 3)) return LOWM_OK;
    }
  }
  // More than 16 activation rows: panel tiles (the activation operand of a
  // step shared in LDS by the four wavefronts), ring of 4 steps.  Measured on
  // MI355X at M 32 and M 64, N 6144, K 4096, split_k 1..8: 1.3-2.1x faster
  // than the line-pair and register tiles at every point; rings of 3 and 6
  // are within a few percent, 3 slower at M 64.  64-row tiles: with split-K
  // they beat the 32-row tiles whose wavefront pairs split the K slice in
  // halves (split_k 2, M 32 / M 64: 15.1 / 18.5 us against 15.7 / 21.3),
  // which win only without split-K, where the quarter tiles win in turn.
  if (M > 16 && nvec % 8 == 0) {
    t->rows = 64;
    if (provides({kStagePanel, 2, 4})) return LOWM_OK;
  }
  if (nvec % 32 == 0 && M <= 32) {
    const int pairs = nvec / 32;   // line pairs per wavefront
    if (!(M > 16 && pairs >= 16)) {
      const int ring = (M <= 4 && pairs >= 8 && pairs < 16) ? 4 : 2;
      t->rows = 16;
      if (provides({kStageLine, 2, ring})) return LOWM_OK;
    }
  }
  t->rows = M <= 16 ? 16 : 32;
  if (provides(first)) return LOWM_OK;
  for (const Variant& v : others)
    if (provides(v)) return LOWM_OK;
  return LOWM_ERR_UNSUPPORTED;
}

// split_k for a shape, from a table of the fastest measured on MI355X
// (bench.py --split-sweep: the default tactic for each split_k, W streamed
// from HBM through a rotated pool, median of 3 x 40 calls): M 4, 8, 16, 32
// and 64, N 768 .. 24576, K 2048 .. 16384, split_k 1, 2, 4, 8.  A shape
// takes its nearest grid point in log2 N and log2 K and the row of the next
// measured M at or above its own.  On the grid every entry is the fastest
// split_k; some neighbours are within a few percent of each other.  split_k
// pays when the tiles are few and K is long; the larger the partials (M),
// the less often.
constexpr int kSplitRows = 5;
constexpr int kSplitRowM[kSplitRows] = {4, 8, 16, 32, 64};
constexpr unsigned char kBestSplit[kSplitRows][6][4] = {
    // M <= 4            K: 2048 4096 8192 16384
    {{4, 4, 4, 8},    // N 768
     {4, 4, 4, 4},    // N 1536
     {2, 2, 2, 4},    // N 3072
     {1, 1, 2, 8},    // N 6144
     {1, 2, 2, 8},    // N 12288
     {1, 1, 2, 8}},   // N 24576
    // 4 < M <= 8
    {{4, 4, 8, 8},
     {2, 8, 4, 4},
     {2, 2, 4, 4},
     {1, 1, 2, 4},
     {1, 1, 2, 4},
     {1, 1, 2, 4}},
    // 8 < M <= 16
    {{4, 4, 8, 8},
     {4, 4, 4, 8},
     {2, 4, 4, 4},
     {1, 1, 2, 4},
     {1, 2, 2, 4},
     {1, 1, 2, 4}},
    // 16 < M <= 32
    {{2, 2, 2, 8},
     {1, 2, 2, 8},
     {1, 1, 2, 4},
     {1, 1, 2, 2},
     {1, 1, 2, 4},
     {1, 1, 2, 1}},
    // 32 < M <= 64
    {{1, 1, 1, 8},
     {1, 1, 1, 8},
     {1, 1, 4, 4},
     {1, 1, 1, 2},
     {1, 1, 1, 1},
     {1, 1, 1, 2}}};

int nearest_log2_index(double x, double base, int last) {
  const int i = (int)floor(log2(x / base) + 0.5);
  return i < 0 ? 0 : (i > last ? last : i);
}

int pick_split(int M, int N, int K, int* split_k) {
  if (!split_k) return LOWM_ERR_INVALID_ARG;
  int rc = check_sizes(M, N, K, 1);
  if (rc != LOWM_OK) return rc;
  int row = 0;
  while (row < kSplitRows - 1 && M > kSplitRowM[row]) ++row;
  int S = kBestSplit[row][nearest_log2_index(N, 768.0, 5)][nearest_log2_index(K, 2048.0, 3)];
  // the largest power of two <= S that K allows (a whole number of 16-byte
  // vectors per slice), preferring slices that are whole line pairs
  while (S > 1 && K % (kVecK * S) != 0) S /= 2;
  while (S > 1 && (K / S) % 256 != 0 && K % 256 == 0) S /= 2;
  *split_k = S;
  return LOWM_OK;
}

// The kernel a launch with tactic t runs: the activation slice is staged in
// LDS when it is small and whole 1 KB pieces (and the build has that
// instantiation); otherwise the wavefronts load activation operands from L2.
KernelFn select_kernel(bool f32out, int M, int S, int nvec, const lowm_tactic& t,
                       size_t* dyn_lds, bool push) {
  *dyn_lds = 0;
  // quarter-rows tiles: the quarter kernel of 16*unroll activation rows,
  // launched with H = ceil(M / (16*unroll)) workgroups per tile (split_k 1;
  // no push epilogue, whose flags every block of a tile would raise)
  if (t.stage == kStageQuarterRows) {
    if (S != 1 || push || t.unroll < 1 || t.unroll > 4 || nvec % 32 != 0) return nullptr;
    lowm_tactic q = t;
    q.stage = kStageQuarter;
    q.unroll = 2;
    return lookup(f32out, 0, M < 16 * t.unroll ? M : 16 * t.unroll, q);
  }
  // line-pair tiles stream whole 64-K line pairs per wavefront; panel tiles
  // whole 64-K steps of the slice (of each half of it with 32-row tiles)
  if (t.stage == kStageLine && nvec % 32 != 0) return nullptr;
  if (t.stage == kStagePanel && nvec % (t.rows == 32 ? 16 : 8) != 0) return nullptr;
  if (t.stage == kStageQuarter && nvec % 32 != 0) return nullptr;
  if (nvec % 64 == 0 && act_lds_bytes(M, nvec) <= kActLdsMax) {
    if (KernelFn fn = lookup(f32out, 1, M, t, push)) {
      *dyn_lds = act_lds_bytes(M, nvec);
      return fn;
    }
  }
  *dyn_lds = 0;
  return lookup(f32out, 0, M, t, push);
}

size_t workspace_bytes(int M, int N, int K, int S) {
  if (check_sizes(M, N, K, S) != LOWM_OK || S == 1) return 0;
  // counters for up to ceil(N/16) tiles, then [tiles][split_k][M][BN] fp32
  // partials; tiles * BN never exceeds N rounded up to 64, a multiple of
  // every tile width.  Both parts are multiples of 256 bytes.
  return counter_bytes(N) +
         (size_t)S * (size_t)M * round_up((size_t)N, kPartialPad) * sizeof(float);
}

// The push epilogue of a single-GEMM launch (bf16 output).
struct PushSpec {
  void* dst;
  int ld;
  uint32_t* flags;
  uint32_t value;
};

// [lo, hi) of the bytes a row-major [rows, cols] array with row pitch ld
// elements of `elem` bytes spans.
inline void byte_span(const void* p, int rows, int cols, int ld, size_t elem, uintptr_t* lo,
                      uintptr_t* hi) {
  *lo = (uintptr_t)p;
  *hi = *lo + ((size_t)(rows - 1) * (size_t)ld + (size_t)cols) * elem;
}

bool overlap(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) {
  return a0 < b1 && b0 < a1;
}

int check_push(const PushSpec& p, const void* C, int M, int N) {
  if (!p.dst || !p.flags || p.value == 0 || p.ld < N) return LOWM_ERR_INVALID_ARG;
  if (((uintptr_t)p.dst & 1) || ((uintptr_t)p.flags & 3)) return LOWM_ERR_UNSUPPORTED;
  uintptr_t c0, c1, d0, d1, f0, f1;
  byte_span(C, M, N, N, 2, &c0, &c1);
  byte_span(p.dst, M, N, p.ld, 2, &d0, &d1);
  byte_span(p.flags, 1, (N + 15) / 16, 0, 4, &f0, &f1);
  if (overlap(c0, c1, d0, d1) || overlap(c0, c1, f0, f1) || overlap(d0, d1, f0, f1))
    return LOWM_ERR_INVALID_ARG;
  return LOWM_OK;
}

// Outputs the launch writes must not overlap anything it reads or writes
// besides themselves: no C_g may overlap any A, W or other C of the launch,
// nor the workspace, and the workspace may overlap no operand.  (Inputs may
// be shared or overlap each other: they are only read.)
int check_overlaps(const lowm_gemm_desc* gemms, int count, bool f32out, int M, int K, int S,
                   const void* workspace) {
  const size_t celem = f32out ? 4 : 2;
  uintptr_t w0 = 0, w1 = 0;
  if (S > 1) {
    size_t ws = 0;
    for (int g = 0; g < count; ++g) ws += workspace_bytes(M, gemms[g].N, K, S);
    w0 = (uintptr_t)workspace;
    w1 = w0 + ws;
  }
  for (int g = 0; g < count; ++g) {
    uintptr_t c0, c1;
    byte_span(gemms[g].C, M, gemms[g].N, gemms[g].N, celem, &c0, &c1);
    if (S > 1 && overlap(c0, c1, w0, w1)) return LOWM_ERR_INVALID_ARG;
    for (int h = 0; h < count; ++h) {
      uintptr_t a0, a1, b0, b1;
      byte_span(gemms[h].A, M, K, K, 2, &a0, &a1);
      byte_span(gemms[h].W, gemms[h].N, K, K, 2, &b0, &b1);
      if (overlap(c0, c1, a0, a1) || overlap(c0, c1, b0, b1)) return LOWM_ERR_INVALID_ARG;
      if (S > 1 && g == 0 && (overlap(w0, w1, a0, a1) || overlap(w0, w1, b0, b1)))
        return LOWM_ERR_INVALID_ARG;
      if (h != g) {
        uintptr_t d0, d1;
        byte_span(gemms[h].C, M, gemms[h].N, gemms[h].N, celem, &d0, &d1);
        if (overlap(c0, c1, d0, d1)) return LOWM_ERR_INVALID_ARG;
      }
    }
  }
  return LOWM_OK;
}

// One launch of `count` GEMMs sharing M, K, split_k, the output type and the
// tactic; the single-GEMM entry points are the count == 1 case.  GEMM g's
// workspace follows GEMM g-1's (each is workspace_bytes of its own sizes).
// `push` (single bf16 GEMM only) adds the push epilogue.
int launch_batch(const lowm_gemm_desc* gemms, int count, bool f32out, int M, int K, int S,
                 void* workspace, hipStream_t stream, const lowm_tactic* tactic,
                 const PushSpec* push = nullptr) {
  if (!gemms || count < 1) return LOWM_ERR_INVALID_ARG;
  if (count > kMaxBatch) return LOWM_ERR_UNSUPPORTED;
  if (push && (count != 1 || f32out)) return LOWM_ERR_INVALID_ARG;
  for (int g = 0; g < count; ++g)
    if (!gemms[g].A || !gemms[g].W || !gemms[g].C) return LOWM_ERR_INVALID_ARG;
  int rc = LOWM_OK;
  for (int g = 0; g < count; ++g) {
    rc = check_sizes(M, gemms[g].N, K, S);
    if (rc != LOWM_OK) return rc;
  }
  if (S > 1 && !workspace) return LOWM_ERR_WORKSPACE;
  for (int g = 0; g < count; ++g) {
    if (((uintptr_t)gemms[g].A | (uintptr_t)gemms[g].W) & 15) return LOWM_ERR_UNSUPPORTED;
    if ((uintptr_t)gemms[g].C & (f32out ? 3 : 1)) return LOWM_ERR_UNSUPPORTED;
  }
  if (S > 1 && ((uintptr_t)workspace & 15)) return LOWM_ERR_UNSUPPORTED;
  rc = check_overlaps(gemms, count, f32out, M, K, S, workspace);
  if (rc != LOWM_OK) return rc;
  if (push) {
    rc = check_push(*push, gemms[0].C, M, gemms[0].N);
    if (rc != LOWM_OK) return rc;
  }

  lowm_tactic t;
  if (tactic) {
    t = *tactic;
  } else {
    // One tactic serves every GEMM of the launch: pick it for the narrowest
    // (N only sets the tile width and ring, which keep the summation order).
    int n_min = gemms[0].N;
    for (int g = 1; g < count; ++g) n_min = gemms[g].N < n_min ? gemms[g].N : n_min;
    rc = pick(M, n_min, K, S, &t, push != nullptr);
    if (rc != LOWM_OK) return rc;
  }
  const int nvec = K / S / kVecK;
  size_t dyn_lds = 0;
  const KernelFn fn = select_kernel(f32out, M, S, nvec, t, &dyn_lds, push != nullptr);
  if (!fn) return LOWM_ERR_UNSUPPORTED;

  const int BN = t.rows;
  Batch bt{};
  size_t grid = 0, ws_off = 0;
  for (int g = 0; g < count; ++g) {
    GemmSlot& sl = bt.g[g];
    const int N = gemms[g].N;
    sl.A = static_cast<const uint16_t*>(gemms[g].A);
    sl.W = static_cast<const uint16_t*>(gemms[g].W);
    sl.C = gemms[g].C;
    sl.N = N;
    char* ws = static_cast<char*>(workspace) + ws_off;
    sl.ctr = S > 1 ? reinterpret_cast<uint32_t*>(ws) : nullptr;
    sl.part = S > 1 ? reinterpret_cast<uint32_t*>(ws + counter_bytes(N)) : nullptr;
    ws_off += workspace_bytes(M, N, K, S);
    const size_t tiles = (size_t)((N + BN - 1) / BN);
    const size_t blocks = t.stage == kStageQuarterRows ? (M + 16 * t.unroll - 1) / (16 * t.unroll) : 1;
    grid += round_up(tiles, kXcds) * (size_t)S * blocks;
    if (grid > 0x7fffffffu) return LOWM_ERR_UNSUPPORTED;
    sl.bid_end = (int)grid;
  }
  for (int g = count; g < kMaxBatch; ++g) bt.g[g] = bt.g[count - 1];
  // a traced launch (stress build) must fit the trace buffer it writes
  if (g_stress.trace && grid > g_trace_capacity) return LOWM_ERR_INVALID_ARG;

  Args a{};
  a.A = bt.g[0].A;
  a.W = bt.g[0].W;
  a.C = bt.g[0].C;
  a.M = M;
  a.N = bt.g[0].N;
  a.K = K;
  a.S = S;
  a.nvec = nvec;
  a.batch = count;
  a.ctr = bt.g[0].ctr;
  a.part = bt.g[0].part;
  a.bid_base = 0;
  a.push = push ? static_cast<uint16_t*>(push->dst) : nullptr;
  a.flags = push ? push->flags : nullptr;
  a.push_ld = push ? push->ld : 0;
  a.flag_value = push ? push->value : 0u;
  a.stress = g_stress;

  void* kargs[] = {&a, &bt};
  hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)grid),
                                   dim3(kThreads), kargs, dyn_lds, stream);
  if (err == hipSuccess) err = hipGetLastError();
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return LOWM_ERR_LAUNCH;
  }
  return LOWM_OK;
}

// ---------------------------------------------------------------------------
// Built-in workspace of the no-allocation entry point: a file-scope device
// array, one copy per GPU the library runs on, held until the process ends.
// In host code `scratch` names a host-side stand-in, never the device memory:
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that address is ever passed on.
// The array is zero when the library is loaded onto a device, and every
// launch that completes returns every word it used (counters and partial
// slots) to zero, exactly as with a caller's workspace: each call finds it
// all zero without any clearing.  Calls that overlap in time on one GPU
// (two streams) share it and race.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = LOWM_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the device `stream` belongs to.
int scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t err = hipStreamGetDevice(stream, &dev);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return LOWM_ERR_LAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return LOWM_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = 0;
      err = hipGetDevice(&cur);
      if (err == hipSuccess && cur != dev) err = hipSetDevice(dev);
      if (err == hipSuccess) {
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
          const hipError_t back = hipSetDevice(cur);
          if (err == hipSuccess) err = back;
        }
      }
      if (err != hipSuccess || !p) {
        g_last_hip_error = (int)err;
        return LOWM_ERR_LAUNCH;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return LOWM_OK;
}

int launch(const void* A, const void* W, void* C, bool f32out, int M, int N, int K, int S,
           void* workspace, hipStream_t stream, const lowm_tactic* tactic,
           const PushSpec* push = nullptr) {
  const lowm_gemm_desc one = {A, W, C, N};
  return launch_batch(&one, 1, f32out, M, K, S, workspace, stream, tactic, push);
}

// Consumer side of the push epilogue: one wavefront polls the flags with
// system-scope loads until each holds `value` or `ticks` of the 100 MHz
// real-time counter have passed, then writes how many flags it did not see
// set (0: all were).  Every poll of a flag is a fresh load; a flag once seen
// is not polled again.
constexpr int kWaitFlagsPerLane = 64;
constexpr int kMaxWaitFlags = kWave * kWaitFlagsPerLane;
constexpr uint32_t kMaxWaitUs = 10u * 1000u * 1000u;

__global__ __launch_bounds__(kWave) void lowm_push_wait_kernel(const uint32_t* flags, int n,
                                                                uint32_t value, uint64_t ticks,
                                                                int* missing) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int lane = threadIdx.x;
  uint64_t pending = 0;   // bit j: flag lane + 64 j not yet seen
  for (int j = 0; j < kWaitFlagsPerLane; ++j)
    if (lane + kWave * j < n) pending |= 1ull << j;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    for (int j = 0; j < kWaitFlagsPerLane; ++j) {
      if (!(pending >> j & 1)) continue;
      const uint32_t f = __hip_atomic_load(flags + lane + kWave * j, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM);
      if (f == value) pending &= ~(1ull << j);
    }
    if (__all(pending == 0)) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(8);
  }
  int left = __popcll(pending);
  for (int off = kWave / 2; off > 0; off >>= 1) left += __shfl_xor(left, off);
  if (lane == 0) missing[0] = left;
#endif
}

int push_wait(const uint32_t* flags, int n, uint32_t value, uint32_t timeout_us, int* missing,
              hipStream_t stream) {
  if (!flags || !missing || n < 1 || value == 0) return LOWM_ERR_INVALID_ARG;
  if (n > kMaxWaitFlags || timeout_us > kMaxWaitUs) return LOWM_ERR_UNSUPPORTED;
  if (((uintptr_t)flags & 3) || ((uintptr_t)missing & 3)) return LOWM_ERR_UNSUPPORTED;
  const uint64_t ticks = (uint64_t)timeout_us * 100u;
  void* kargs[] = {&flags, &n, &value, const_cast<uint64_t*>(&ticks), &missing};
  hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&lowm_push_wait_kernel),
                                   dim3(1), dim3(kWave), kargs, 0, stream);
  if (err == hipSuccess) err = hipGetLastError();
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return LOWM_ERR_LAUNCH;
  }
  return LOWM_OK;
}

}  // namespace lowm

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

int lowm_gemm_splitk(const void* A, const void* W, void* C, int M, int N, int K, int split_k,
                     void* workspace, void* stream) {
  return lowm::launch(A, W, C, false, M, N, K, split_k, workspace,
                      static_cast<hipStream_t>(stream), nullptr);
}

int lowm_gemm_splitk_noalloc(const void* A, const void* W, void* C, int M, int N, int K,
                             int split_k, void* stream) {
  int rc = lowm::check_sizes(M, N, K, split_k);
  if (rc != LOWM_OK) return rc;
  if (!A || !W || !C) return LOWM_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (split_k > 1) {
    if (lowm::workspace_bytes(M, N, K, split_k) > lowm::kScratchBytes) return LOWM_ERR_SCRATCH;
    rc = lowm::scratch_address(static_cast<hipStream_t>(stream), &ws);
    if (rc != LOWM_OK) return rc;
  }
  return lowm::launch(A, W, C, false, M, N, K, split_k, ws, static_cast<hipStream_t>(stream),
                      nullptr);
}

int lowm_gemm_splitk_f32out(const void* A, const void* W, float* C, int M, int N, int K,
                            int split_k, void* workspace, void* stream) {
  return lowm::launch(A, W, C, true, M, N, K, split_k, workspace,
                      static_cast<hipStream_t>(stream), nullptr);
}

int lowm_gemm_splitk_ex(const void* A, const void* W, void* C, int M, int N, int K,
                        int split_k, void* workspace, void* stream, const lowm_tactic* tactic) {
  return lowm::launch(A, W, C, false, M, N, K, split_k, workspace,
                      static_cast<hipStream_t>(stream), tactic);
}

int lowm_gemm_splitk_f32out_ex(const void* A, const void* W, float* C, int M, int N, int K,
                               int split_k, void* workspace, void* stream,
                               const lowm_tactic* tactic) {
  return lowm::launch(A, W, C, true, M, N, K, split_k, workspace,
                      static_cast<hipStream_t>(stream), tactic);
}

size_t lowm_gemm_splitk_workspace_bytes(int M, int N, int K, int split_k) {
  return lowm::workspace_bytes(M, N, K, split_k);
}

int lowm_gemm_splitk_push(const void* A, const void* W, void* C, int M, int N, int K,
                          int split_k, void* workspace, void* push, int push_ld,
                          uint32_t* flags, uint32_t flag_value, void* stream,
                          const lowm_tactic* tactic) {
  const lowm::PushSpec ps = {push, push_ld, flags, flag_value};
  return lowm::launch(A, W, C, false, M, N, K, split_k, workspace,
                      static_cast<hipStream_t>(stream), tactic, &ps);
}

int lowm_push_wait(const uint32_t* flags, int n_flags, uint32_t flag_value,
                   uint32_t timeout_us, int* missing, void* stream) {
  return lowm::push_wait(flags, n_flags, flag_value, timeout_us, missing,
                         static_cast<hipStream_t>(stream));
}

int lowm_gemm_splitk_batched(const lowm_gemm_desc* gemms, int count, int M, int K,
                             int split_k, void* workspace, void* stream) {
  return lowm::launch_batch(gemms, count, false, M, K, split_k, workspace,
                            static_cast<hipStream_t>(stream), nullptr);
}

size_t lowm_gemm_splitk_batched_workspace_bytes(const lowm_gemm_desc* gemms, int count, int M,
                                                int K, int split_k) {
  if (!gemms || count < 1 || count > LOWM_MAX_BATCH) return 0;
  size_t total = 0;
  for (int g = 0; g < count; ++g) {
    if (lowm::check_sizes(M, gemms[g].N, K, split_k) != LOWM_OK) return 0;
    total += lowm::workspace_bytes(M, gemms[g].N, K, split_k);
  }
  return total;
}

int lowm_pick_split_k(int M, int N, int K, int* split_k) {
  return lowm::pick_split(M, N, K, split_k);
}

int lowm_check_launch(int M, int N, int K, int split_k, int f32out, const lowm_tactic* tactic) {
  int rc = lowm::check_sizes(M, N, K, split_k);
  if (rc != LOWM_OK) return rc;
  lowm_tactic t;
  if (tactic) {
    t = *tactic;
  } else {
    rc = lowm::pick(M, N, K, split_k, &t);
    if (rc != LOWM_OK) return rc;
  }
  size_t dyn = 0;
  return lowm::select_kernel(f32out != 0, M, split_k, K / split_k / lowm::kVecK, t, &dyn)
             ? LOWM_OK
             : LOWM_ERR_UNSUPPORTED;
}

int lowm_pick_tactic(int M, int N, int K, int split_k, lowm_tactic* out) {
  if (!out) return LOWM_ERR_INVALID_ARG;
  return lowm::pick(M, N, K, split_k, out);
}

const char* lowm_strerror(int code) {
  switch (code) {
    case LOWM_OK: return "success";
    case LOWM_ERR_INVALID_ARG:
      return "invalid argument (NULL operand, size <= 0, split_k < 1, or an output that "
             "overlaps an operand, another output or the workspace)";
    case LOWM_ERR_UNSUPPORTED:
      return "unsupported (M > 64, K not a multiple of 8*split_k, split_k > 256, misaligned "
             "pointer, or a tactic the library does not provide)";
    case LOWM_ERR_WORKSPACE: return "split_k > 1 needs a workspace";
    case LOWM_ERR_LAUNCH: return "a HIP call failed (see lowm_last_hip_error)";
    case LOWM_ERR_SCRATCH:
      return "the sizes need more workspace than the built-in scratch of "
             "lowm_gemm_splitk_noalloc (LOWM_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

int lowm_last_hip_error(void) { return lowm::g_last_hip_error; }

int lowm_workspace_status(const void* workspace, int N, void* stream, int* faulted_tiles,
                          int* open_tiles) {
  if (!workspace || N <= 0 || !faulted_tiles || !open_tiles) return LOWM_ERR_INVALID_ARG;
  const size_t lines = (size_t)(N + 15) / 16;
  std::vector<uint32_t> host(lines * lowm::kCtrStride);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipMemcpyAsync(host.data(), workspace, host.size() * sizeof(uint32_t),
                                  hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) {
    lowm::g_last_hip_error = (int)err;
    return LOWM_ERR_LAUNCH;
  }
  int faulted = 0, open = 0;
  for (size_t t = 0; t < lines; ++t) {
    const uint32_t* line = host.data() + t * lowm::kCtrStride;
    faulted += line[lowm::kFaultWord] != 0u;
    open += line[0] != 0u;
  }
  *faulted_tiles = faulted;
  *open_tiles = open;
  return LOWM_OK;
}

#ifdef LOWM_STRESS
// Stress build only: where, on whom and how long the kernels stall.  Applies
// to every later launch from any thread; not thread-safe.
int lowm_stress_configure(unsigned site_mask, int rank, int wave, int tile_mod, int tile_sel,
                          int step, unsigned delay_ns) {
  if (delay_ns > 5000000u) return LOWM_ERR_INVALID_ARG;  // at most 5 ms per stall
  lowm::g_stress.site_mask = site_mask;
  lowm::g_stress.rank = rank;
  lowm::g_stress.wave = wave;
  lowm::g_stress.tile_mod = tile_mod;
  lowm::g_stress.tile_sel = tile_sel;
  lowm::g_stress.step = step;
  lowm::g_stress.ticks = delay_ns / 10u;  // s_memrealtime: 100 MHz
  return LOWM_OK;
}

// Stress build only: record per-workgroup timestamps and ids into `buf`
// (device memory, 10 uint64 per workgroup of the grid: entry, first stage,
// loop end, reduced, arrived, end, CU id, XCD id, tile, rank), which holds
// `workgroups` such records; a launch whose grid is larger returns
// LOWM_ERR_INVALID_ARG before any HIP call.  NULL stops tracing.
int lowm_stress_trace(void* buf, size_t workgroups) {
  if (buf && workgroups == 0) return LOWM_ERR_INVALID_ARG;
  lowm::g_stress.trace = static_cast<uint64_t*>(buf);
  lowm::g_trace_capacity = buf ? workgroups : 0;
  return LOWM_OK;
}
#endif

}  // extern "C"
