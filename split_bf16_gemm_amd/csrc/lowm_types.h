// lowm_types.h -- types shared by the kernel translation units and the host
// side of the low-M split-K bf16 GEMM (gfx950).  No device code here.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "lowm.h"

namespace lowm {

constexpr int kWave = 64;        // lanes per wavefront
constexpr int kWaves = 4;        // wavefronts per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kVecK = 8;         // bf16 per 16-byte vector
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kCtrStride = 64;   // uint32 words between tile counters (256 bytes)
constexpr int kFaultWord = 1;    // word of a counter line that flags a failed fold
constexpr int kProbeRanks = 3;   // early probe: at most 3 peers (split_k <= 4)
constexpr uint32_t kProbeTicks = 2000;  // ... polled for at most 20 us (100 MHz clock)
// An owner that finds a peer's slot still unpublished after the counter said
// every peer had arrived re-reads it for at most this long (100 MHz clock).
constexpr uint32_t kFoldPollTicks = 100000;   // 1 ms

enum Stage : int {
  kStageLds = LOWM_STAGE_LDS,
  kStageReg = LOWM_STAGE_REG,
  kStageLine = LOWM_STAGE_LINE,
  kStagePanel = LOWM_STAGE_PANEL,
  kStageQuarter = LOWM_STAGE_QUARTER,
  kStageQuarterRows = LOWM_STAGE_QUARTER_ROWS
};

// ---------------------------------------------------------------------------
// Stress instrumentation (acted on only in the -DLOWM_STRESS build)
// ---------------------------------------------------------------------------
enum StressSite : uint32_t {
  kSiteEntry = 1u,        // a wavefront stalls before its first load
  kSiteStageRead = 2u,    // after the stage wait, before reading the stage
  kSiteReduce = 4u,       // before writing its sums for the wavefront reduction
  kSitePublish = 8u,      // before storing the rank partial and arriving
  kSiteFold = 16u,        // owner: after the arrival count, before reading partials
  // A rank arrives first and stores its partial only after the stall (unless
  // the arrival made it the owner), as if its stores had landed that late.
  kSiteLatePublish = 32u,
};

struct StressArgs {
  uint32_t site_mask;     // OR of StressSite
  int rank;               // -1: any rank
  int wave;               // -1: any wavefront
  int tile_mod;           // stall tiles with tile % tile_mod == tile_sel
  int tile_sel;
  int step;               // kSiteStageRead: only this step (-1: every step)
  uint32_t ticks;         // stall length in s_memrealtime ticks (100 MHz)
  uint64_t* trace;        // optional per-workgroup timestamps (kTraceSlots each)
};

// Timestamp trace of the stress build: per workgroup, s_memrealtime (100 MHz)
// at these points, then the hardware ids of the CU and XCD it ran on and the
// (tile, rank) it worked on (kTraceSlots 64-bit words per workgroup).  The
// timestamps are global stores, counted by the same vector-memory counter as
// the loads whose completion the explicit s_waitcnt of the LDS-ring variants
// assumes: a traced launch measures timing only, its output is not checked.
enum TraceSlot : int {
  kTraceEntry = 0, kTraceFirstStage = 1, kTraceLoopEnd = 2, kTraceReduced = 3,
  kTraceArrived = 4, kTraceEnd = 5, kTraceHwId = 6, kTraceXccId = 7, kTraceTile = 8,
  kTraceRank = 9, kTraceSlots = 10
};

struct Args {
  // Every field a single-GEMM launch reads sits in the first 64 bytes of the
  // argument segment, so each workgroup's start waits for one scalar line.
  const uint16_t* A;
  const uint16_t* W;
  void* C;
  uint32_t* ctr;          // [ceil(N/16)] arrival counters, kCtrStride words apart
  uint32_t* part;         // encoded fp32 partial slots
  int M, N, K, S;
  int nvec;               // 16-byte vectors per rank slice: K / S / 8
  int batch;              // GEMMs in the launch; 1: these fields describe the only one
  // Set by gemm_args in the kernel, never read from the argument segment.
  int bid_base;           // first workgroup of this GEMM in a batched launch
  // push epilogue (its own instantiation, bf16 output)
  uint16_t* push;         // exchange buffer, element (m, n) at push[m * push_ld + n]
  uint32_t* flags;        // [ceil(N / 16)] one per 16 output columns
  int push_ld;
  uint32_t flag_value;
  StressArgs stress;
};
static_assert(offsetof(Args, batch) + sizeof(int) <= 64, "hot fields leave the first line");

// Batched launch: up to kMaxBatch independent GEMMs with one M, K and split_k
// in one grid.  GEMM g owns the workgroups [bid_end of g-1, bid_end of g),
// each range a multiple of 8 so that the ranks of a tile still share an XCD.
constexpr int kMaxBatch = LOWM_MAX_BATCH;
struct GemmSlot {
  const uint16_t* A;
  const uint16_t* W;
  void* C;
  uint32_t* ctr;
  uint32_t* part;
  int N;
  int bid_end;
};
struct Batch {
  GemmSlot g[kMaxBatch];  // read only when Args::batch > 1
};

// ---------------------------------------------------------------------------
// The kernel table: every instantiation the build provides, by output kind,
// activation mode, M block count, tile rows and variant.
// ---------------------------------------------------------------------------
struct Variant {
  int stage, unroll, stages;
};
constexpr Variant kVariants[] = {
    {kStageLds, 4, 2},   {kStageLds, 4, 3},   {kStageReg, 4, 2},   {kStageReg, 8, 2},
    {kStageReg, 16, 2},  {kStageLine, 2, 2},  {kStageLine, 2, 3},  {kStageLine, 2, 4},
    {kStagePanel, 2, 3}, {kStagePanel, 2, 4}, {kStagePanel, 2, 6},
    {kStageQuarter, 2, 2}, {kStageQuarter, 2, 3}, {kStageQuarter, 2, 4},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

// Rows per tile the build provides: 16 * RG for RG in kRowGroups (line-pair,
// register and LDS tiles 16 or 32; quarter tiles 16, 32, 48 or 64; panel
// tiles 64 with 16 per wavefront, or 32 with 16 per pair of wavefronts).
constexpr int kRowGroups[] = {1, 2, 3, 4};
constexpr int kNumRowGroups = sizeof(kRowGroups) / sizeof(kRowGroups[0]);
constexpr int rg_index(int rg) {
  for (int i = 0; i < kNumRowGroups; ++i)
    if (kRowGroups[i] == rg) return i;
  return -1;
}

typedef void (*KernelFn)(Args, Batch);

// table[out][act][MB-1][rg_index][variant]; out 0 bf16, 1 fp32, 2 bf16 + push
enum OutKind : int { kOutBf16 = 0, kOutF32 = 1, kOutPush = 2, kNumOutKinds = 3 };
struct Table {
  KernelFn fn[kNumOutKinds][2][4][kNumRowGroups][kNumVariants];
};

// Each output kind's kernels live in a translation unit of their own, which
// fills its part of the table.
void fill_table_bf16(Table& t);
void fill_table_f32(Table& t);
void fill_table_push(Table& t);

}  // namespace lowm
