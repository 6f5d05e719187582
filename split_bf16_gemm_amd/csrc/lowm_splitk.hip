// lowm_splitk.hip -- low-M split-K bf16 GEMM for AMD Instinct MI355X (gfx950).
//
//   C[m][n] = sum_k A[m][k] * W[n][k]        A [M,K], W [N,K] bf16, row-major
//
// The problem is the one the TensorRT-LLM PR "Fix two synchronization gaps in
// the MiniMax M3 low-M split-K GEMM" works on (Description; Hardware
// verification): a handful of activation rows against a large bf16 weight,
// K cut into split_k slices whose fp32 partials one owner adds.  The design
// here is gfx950's own:
//
//  * One workgroup = (output tile of BN = 16*RG weight rows) x (one K slice,
//    "rank").  Its four wavefronts share the slice; each streams its share of
//    W once from HBM and feeds bf16 MFMA 16x16x32 with W as the 16-column
//    operand and the M activation rows, zero-padded to 16 per block, as the
//    16-row operand, accumulating fp32 in registers.  M <= 64 is 1..4 MFMA
//    row blocks.
//  * W reaches the MFMA either through an LDS ring of NS stages filled with
//    direct-to-LDS loads (global_load_lds_dwordx4) and shared by the whole
//    workgroup, or straight into a ring of NS register stages per wavefront.
//    In the LDS ring a stage is refilled only after a workgroup barrier that
//    every wavefront reaches once its reads of that stage have completed: a
//    per-wavefront wait is not enough when the stage is shared (Triton issue
//    "warpgroup_mma_wait does not properly synchronize across warpgroups";
//    cuLA PR "Fix SM90 WY input buffer reuse before WGMMA completion").
//  * The wavefronts' sums are added through LDS in wavefront order.
//  * split_k > 1: every rank stores its fp32 partial in the workspace, makes
//    it visible at agent scope (release), and counts itself in the tile's
//    arrival counter with a relaxed atomic.  The rank that sees split_k-1
//    earlier arrivals is the owner: it reads the peers' partials after the
//    count (acquire), adds the partials in rank order 0..split_k-1 (its own
//    from registers, at its own position), rounds once to bf16 and returns
//    the counter and the tile's partial slots to zero.  A slot word holds the
//    complement of the partial's bits, so zero means "not published"; the
//    whole workspace is zero between launches.  Where split_k is 2..4 and a
//    tile has at most 64 elements, the grid is rank-major and the tile's last
//    rank polls its peers' slots for a bounded time instead of publishing: a
//    published slot is visible long before the publisher's acknowledgement
//    and arrival come back from the loaded memory system.  Each counter sits
//    on its own 256-byte line: device-scope atomics on one line are
//    serialised where they execute, so tiles do not share lines.  Scope
//    matters (PR, Description item 2: a release and an acquire synchronize
//    only when each one's scope includes the other thread); the acquire is
//    carried by device-scope loads issued on the owner's path only (PR,
//    Description item 2, on the cost of an acquiring wait).  No workgroup
//    waits for another without a bound.
//
// Built twice from this source: liblowm.so, and liblowm_stress.so with
// -DLOWM_STRESS, which adds bounded s_sleep stalls at chosen sites, ranks,
// wavefronts and tiles (the stall-injection method of the PR's Hardware
// verification).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "lowm.h"

namespace lowm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;        // lanes per wavefront
constexpr int kWaves = 4;        // wavefronts per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kVecK = 8;         // bf16 per 16-byte vector
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kCtrStride = 64;   // uint32 words between tile counters (256 bytes)
constexpr int kProbeRanks = 3;   // early probe: at most 3 peers (split_k <= 4)
constexpr uint32_t kProbeTicks = 2000;  // ... polled for at most 20 us (100 MHz clock)

enum Stage : int {
  kStageLds = LOWM_STAGE_LDS,
  kStageReg = LOWM_STAGE_REG,
  kStageWave = LOWM_STAGE_WAVE,
  kStageLine = LOWM_STAGE_LINE
};

// ---------------------------------------------------------------------------
// Stress instrumentation (compiled only with -DLOWM_STRESS)
// ---------------------------------------------------------------------------
enum StressSite : uint32_t {
  kSiteEntry = 1u,        // a wavefront stalls before its first load
  kSiteStageRead = 2u,    // after the stage barrier, before reading the stage
  kSiteReduce = 4u,       // before writing its sums for the wavefront reduction
  kSitePublish = 8u,      // before storing the rank partial and arriving
  kSiteFold = 16u,        // owner: after the acquire, before reading partials
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
// at these points, then the hardware ids of the CU and XCD it ran on.  The
// timestamps are global stores, counted by the same vector-memory counter as
// the loads whose completion the explicit s_waitcnt of the LDS-ring variants
// assumes: a traced launch measures timing only, its output is not checked.
enum TraceSlot : int {
  kTraceEntry = 0, kTraceFirstStage = 1, kTraceLoopEnd = 2, kTraceReduced = 3,
  kTraceArrived = 4, kTraceEnd = 5, kTraceHwId = 6, kTraceXccId = 7, kTraceSlots = 8
};

struct Args {
  // Every field a single-GEMM launch reads sits in the first 64 bytes of the
  // argument segment, so each workgroup's start waits for one scalar line.
  const uint16_t* A;
  const uint16_t* W;
  void* C;
  uint32_t* ctr;          // [tiles] arrival counters, kCtrStride words apart
  uint32_t* part;         // [tiles][S][M*BN] encoded fp32 partials
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

// The Args of the GEMM this workgroup belongs to.
__device__ __forceinline__ Args gemm_args(const Args& a, const Batch& bt) {
  Args b = a;
  b.bid_base = 0;
  if (a.batch > 1) {
    int g = 0;
#pragma unroll
    for (int i = 0; i < kMaxBatch - 1; ++i)
      if (i < a.batch - 1 && (int)blockIdx.x >= bt.g[i].bid_end) g = i + 1;
    const GemmSlot& s = bt.g[g];
    b.A = s.A;
    b.W = s.W;
    b.C = s.C;
    b.ctr = s.ctr;
    b.part = s.part;
    b.N = s.N;
    b.bid_base = g > 0 ? bt.g[g - 1].bid_end : 0;
  }
  return b;
}

#ifdef LOWM_STRESS
__device__ __forceinline__ void stall_ticks(uint32_t ticks) {
  // Bounded: s_memrealtime is a free-running 100 MHz counter.
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(16);
}
__device__ __forceinline__ void maybe_stall(const StressArgs& st, uint32_t site, int rank,
                                            int wave, int tile, int step) {
  if (!(st.site_mask & site)) return;
  if (st.rank >= 0 && st.rank != rank) return;
  if (st.wave >= 0 && st.wave != wave) return;
  if (st.tile_mod > 1 && tile % st.tile_mod != st.tile_sel) return;
  if (site == kSiteStageRead && st.step >= 0 && st.step != step) return;
  stall_ticks(st.ticks);
}
#define LOWM_STALL(site, step) maybe_stall(a.stress, (site), rank, wave, tile, (step))
#define LOWM_TRACE(slot)                                                              \
  do {                                                                                \
    if (a.stress.trace && threadIdx.x == 0)                                           \
      a.stress.trace[(size_t)blockIdx.x * kTraceSlots + (slot)] =                      \
          __builtin_amdgcn_s_memrealtime();                                           \
  } while (0)
#define LOWM_TRACE_IDS()                                                              \
  do {                                                                                \
    if (a.stress.trace && threadIdx.x == 0) {                                         \
      a.stress.trace[(size_t)blockIdx.x * kTraceSlots + kTraceHwId] =                  \
          __builtin_amdgcn_s_getreg(4 | (31 << 11));                                  \
      a.stress.trace[(size_t)blockIdx.x * kTraceSlots + kTraceXccId] =                 \
          __builtin_amdgcn_s_getreg(20 | (31 << 11));                                 \
    }                                                                                 \
  } while (0)
#else
#define LOWM_STALL(site, step) ((void)0)
#define LOWM_TRACE(slot) ((void)0)
#define LOWM_TRACE_IDS() ((void)0)
#endif

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]<<14
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}
// A workgroup barrier that does not drain outstanding global loads (a HIP
// __syncthreads() would wait for vmcnt(0) and empty the prefetch ring).  The
// memory clobber keeps the compiler from moving loads or stores across it.
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_barrier" ::: "memory"); }
// Keeps a group of prefetch loads where it is issued: without it the compiler
// sinks each load down to its first use, NS-1 steps later, and the register
// ring degenerates into load-then-wait.
__device__ __forceinline__ void pin_issue() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Cache-policy operand of the whole-line direct-to-LDS loads of W: `nt`.
// Each W byte is read once per launch; with whole-line requests the hint
// streams faster than the default policy (measured read-only on MI355X in
// this kernel's geometry: 9.0 vs 9.7 us for 48 MiB).
constexpr int kStreamAux = 2;

// A 16-byte LDS read the compiler does not see as one.  Used for slots that
// direct-to-LDS loads fill, which the code orders by explicit waits: left to
// itself the compiler adds a wait for every outstanding load before some of
// these reads.  The value is usable only after lds_wait() on it.
__device__ __forceinline__ u32x4 lds_read_opaque(const u32x4* p) {
  const uint32_t addr =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) u32x4*)p;
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
// 24 wait states after the last MFMA that writes any of `acc` (2 or 4
// accumulators), before anything reads them.  Reading an MFMA result needs
// wait states that the compiler inserts itself, but it was seen to omit them
// on a path that branches from the last MFMA straight to the accumulator
// reads (the first register then held its value from before the last two
// MFMAs).  The accumulators are operands, so every MFMA producing them is
// issued before these no-ops and every read comes after.
template <int N>
__device__ __forceinline__ void mfma_settle(f32x4 (&acc)[N]) {
  if constexpr (N == 1) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0]));
  else if constexpr (N == 2)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0]), "+a"(acc[1]));
  else if constexpr (N == 4)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
  else static_assert(N == 1 || N == 2 || N == 4, "mfma_settle: 1, 2 or 4 accumulators");
}

// Waits for every outstanding LDS operation; the values read by
// lds_read_opaque pass through it, so their uses cannot move above it.
template <int N>
__device__ __forceinline__ void lds_wait(u32x4 (&v)[N]) {
  if constexpr (N == 1) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]) : : "memory");
  else if constexpr (N == 2)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]) : : "memory");
  else if constexpr (N == 4)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3])
                 : : "memory");
  else static_assert(N == 1 || N == 2 || N == 4, "lds_wait: 1, 2 or 4 values");
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Output kinds a kernel is instantiated for: bf16, fp32, and bf16 with the
// push epilogue (a separate instantiation, so the plain kernels carry no
// trace of it).
struct PushBf16 {};
template <typename OutT> struct OutStore { using type = OutT; };
template <> struct OutStore<PushBf16> { using type = __bf16; };
template <typename OutT>
constexpr bool kPush = std::is_same<OutT, PushBf16>::value;

template <typename T>
__device__ __forceinline__ T to_out(float v);
template <>
__device__ __forceinline__ float to_out<float>(float v) { return v; }
template <>
__device__ __forceinline__ __bf16 to_out<__bf16>(float v) {
  return static_cast<__bf16>(v);  // v_cvt_pk_bf16_f32: round to nearest even
}

// ---------------------------------------------------------------------------
// split-K fold helpers
// ---------------------------------------------------------------------------
// Partial slots.  A slot word holds the complement of the bits of an fp32
// partial, so the all-zero word means "not published".  The caller zero-fills
// the workspace once; every tile's owner returns each slot it read, and its
// own, to zero, so every launch starts with an all-zero partial region.  A
// slot read before its rank wrote it therefore decodes as a NaN (~0), and a
// late rank can tell from the slots alone whether a peer has published.  The
// one fp32 pattern whose complement is zero (0xFFFFFFFF, a NaN) is stored as
// the canonical NaN.
__device__ __forceinline__ uint32_t enc_partial(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  return ~(b == 0xFFFFFFFFu ? 0x7FC00000u : b);
}
__device__ __forceinline__ float dec_partial(uint32_t w) { return __builtin_bit_cast(float, ~w); }

// Device-scope (sc1) accesses of the slots: written through the XCD's L2 to
// where every XCD reads, and read from there.
__device__ __forceinline__ uint32_t load_slot(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_slot(uint32_t* p, uint32_t w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The owner's value of one output element: the S rank partials of this tile
// (slot r at slots[r * E + e]) added in rank order 0..S-1, with this rank's
// own partial `own` at its own position.  The S-1 peers' slots are loaded
// unconditionally (peer i is rank i, or i+1 past the owner) and before the
// first add, so the loads overlap; a load under a branch would be waited for
// inside it.  Loads only: the caller stores C and clears the slots after all
// its folds, so that no wait for these loads also waits for stores.
template <int SN>
__device__ __forceinline__ float fold_ranks_n(const uint32_t* slots, size_t E, int e, int rank,
                                              float own) {
  uint32_t w[SN - 1];
#pragma unroll
  for (int i = 0; i < SN - 1; ++i)
    w[i] = load_slot(slots + (size_t)(i < rank ? i : i + 1) * E + e);
  float v = (rank == 0) ? own : dec_partial(w[0]);
#pragma unroll
  for (int r = 1; r < SN; ++r)
    v += (r == rank) ? own : dec_partial(r < rank ? w[r < SN - 1 ? r : 0] : w[r - 1]);
  return v;
}

__device__ __forceinline__ float fold_ranks(const uint32_t* slots, size_t E, int e, int S,
                                            int rank, float own) {
  switch (S) {
    case 2: return fold_ranks_n<2>(slots, E, e, rank, own);
    case 3: return fold_ranks_n<3>(slots, E, e, rank, own);
    case 4: return fold_ranks_n<4>(slots, E, e, rank, own);
    case 8: return fold_ranks_n<8>(slots, E, e, rank, own);
    default: break;
  }
  float v = 0.f;
  for (int r = 0; r < S; ++r) {
    const uint32_t w = load_slot(slots + (size_t)r * E + e);
    const float p = (r == rank) ? own : dec_partial(w);
    v = (r == 0) ? p : v + p;
  }
  return v;
}

// Every rank's slot of element e back to zero, once the owner has read them
// (the owner's own too: it published before it knew it was the owner).
__device__ __forceinline__ void clear_slots(uint32_t* slots, size_t E, int e, int S) {
  for (int r = 0; r < S; ++r) store_slot(slots + (size_t)r * E + e, 0u);
}

// Whether a split-K tile's last rank polls its peers' slots instead of
// publishing (see workgroup_epilogue): split_k 2..4 and tiles of at most 64
// elements (one per lane).
__device__ __forceinline__ bool early_probe(const Args& a, int BN) {
  return a.S > 1 && a.S - 1 <= kProbeRanks && a.M * BN <= kWave;
}

// Source of probe load i of a lane: peer i's slot of the lane's element
// where this wavefront probes and both exist, else a harmless word of A (so
// that every wavefront can issue the same number of loads).
__device__ __forceinline__ const uint32_t* probe_src(const Args& a, int E, int tile, int lane,
                                                     int i, bool probing) {
  if (probing && i < a.S - 1 && lane < E)
    return a.part + ((size_t)tile * a.S + i) * E + lane;
  return reinterpret_cast<const uint32_t*>(a.A);
}

// a0: workgroup -> (output tile, rank).  Workgroups are dealt to the 8 XCDs
// round-robin; every rank of a tile gets the same blockIdx % 8, hence one
// XCD.  Where the early probe applies the order is rank-major: the GEMM's
// first T8 workgroups are rank 0 of tiles 0..T8-1, the next T8 rank 1, and
// so on (T8 = tiles rounded up to a multiple of 8), so a tile's later ranks
// tend to end their streams after its earlier ones have published.
// Elsewhere the ranks of a tile are dispatched 8 workgroups apart.
__device__ __forceinline__ void decode_tile(const Args& a, int BN, int& tile, int& rank) {
  const int bid = (int)blockIdx.x - a.bid_base;
  if (early_probe(a, BN)) {
    const int t8 = ((a.N + BN - 1) / BN + kXcds - 1) / kXcds * kXcds;
    rank = bid / t8;
    tile = bid - rank * t8;
  } else {
    const int q = bid / kXcds;
    rank = q % a.S;
    tile = (q / a.S) * kXcds + (bid % kXcds);
  }
}

// Register/LDS budget of a tactic.  Kept in one place so the host picker and
// the instantiation filter agree.
//
// LDS variant: a stage is BN weight rows x 512 K (1 KB of each row), stored
// row by row at a pitch of 1040 bytes; each direct-to-LDS instruction moves
// one 1 KB contiguous piece of one row.  Each wavefront consumes 4 of the
// stage's 16 MFMA chunks, so U is 4.
// REG variant: a step is 4*U chunks; wavefront w loads chunks 4j+w.
// ACT: 1 = the workgroup's activation slice A[0:M, slice] is moved into LDS
// once (direct-to-LDS, 1 KB pieces) before the W stream starts; 0 = each
// wavefront loads its activation operands from L2 alongside each W group.
template <int MB, int RG, int STAGE, int U, int NS, int ACT>
struct Shape {
  static constexpr int BN = 16 * RG;
  static constexpr int kPitch = 65;                     // u32x4 per LDS row (1040 B)
  static constexpr int WU = kWaves * U;                 // chunks per step
  static constexpr int slot_elems = (STAGE == kStageLds) ? BN * kPitch : 1;
  static constexpr int red_floats = kWaves * RG * MB * 4 * kWave;
  // the wavefront reduction reuses stage 0 when it is large enough
  static constexpr bool red_in_ring = STAGE == kStageLds && slot_elems * 4 >= red_floats;
  // vector-memory ops of one pipeline group, per wavefront
  static constexpr int group_loads = ((STAGE == kStageLds) ? BN / kWaves : U * RG) +
                                     (ACT ? 0 : U * MB);
  static constexpr int lds_bytes = (STAGE == kStageLds ? NS * slot_elems * 16 : 0) +
                                   (red_in_ring ? 0 : red_floats * 4);
  static constexpr int stage_vgprs =
      NS * U * 4 * ((ACT ? 0 : MB) + (STAGE == kStageReg ? RG : 0));
  static constexpr bool valid =
      lds_bytes <= 128 * 1024 && stage_vgprs <= 224 && NS >= 2 && NS <= 4 &&
      (STAGE == kStageReg || U == 4) && (NS - 1) * group_loads <= 63 && (!ACT || MB <= 2);
};

template <int N>
__device__ __forceinline__ void wait_groups(int younger) {
  // at most `younger` (0..3) groups of N ops may still be outstanding
  if (younger <= 0) wait_vmcnt<0>();
  else if (younger == 1) wait_vmcnt<N>();
  else if (younger == 2) wait_vmcnt<2 * N <= 63 ? 2 * N : 63>();
  else wait_vmcnt<3 * N <= 63 ? 3 * N : 63>();
}

// a6: the owner's store of output element (m, n), to C and, with the push
// epilogue, to the exchange buffer.  The pushed copy is written with
// system-scope stores (sc0 sc1: through every cache to memory), so once they
// are acknowledged a flag store publishes them to any observer.
template <typename OutT>
__device__ __forceinline__ void store_out(const Args& a, int m, int n, float v) {
  using T = typename OutStore<OutT>::type;
  const T o = to_out<T>(v);
  static_cast<T*>(a.C)[(size_t)m * a.N + n] = o;
  if constexpr (kPush<OutT>)
    __hip_atomic_store(a.push + (size_t)m * a.push_ld + n, __builtin_bit_cast(uint16_t, o),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Push epilogue, called by the one wavefront that stored the tile at
// columns n0 .. n0+16*RG-1: once every pushed store of it is acknowledged,
// set the flag of each of its 16-column groups to the caller's value.
template <int RG, typename OutT>
__device__ __forceinline__ void publish_flags(const Args& a, int n0, int lane) {
  if constexpr (kPush<OutT>) {
    wait_vmcnt0();
    pin_issue();
    if (lane < RG && n0 + 16 * lane < a.N)
      __hip_atomic_store(a.flags + n0 / 16 + lane, a.flag_value, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// ---------------------------------------------------------------------------
// The epilogue of a workgroup of kWaves wavefronts, each holding its own sums
// of the tile (acc, MFMA D layout).  The sums are added through LDS in
// wavefront order; wavefront 0 then stores C (split_k 1), or publishes the
// rank partial and, as the owner, folds the ranks (split_k > 1).  `red` is
// room for kWaves*RG*MB*4*64 floats that no wavefront still reads.
// ---------------------------------------------------------------------------
template <int MB, int RG, typename OutT>
__device__ __forceinline__ void workgroup_epilogue(const Args& a, const f32x4 (&acc)[RG][MB],
                                                   float* red, int wave, int lane, int tile,
                                                   int rank, int n0,
                                                   uint32_t (&probe)[kProbeRanks], bool probed) {
  constexpr int BN = 16 * RG;
  auto red_at = [&](int w, int rg, int b, int i, int ln) -> float& {
    return red[(((w * RG + rg) * MB + b) * 4 + i) * kWave + ln];
  };
  LOWM_STALL(kSiteReduce, 0);
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) red_at(wave, rg, b, i, lane) = acc[rg][b][i];

  // Early probe (split_k 2..4, tiles of at most 64 elements): wavefront 0 of
  // the last rank loads the peers' slots of its element, unless the caller's
  // main loop already did (`probed`), before the barrier, so the loads
  // overlap the wavefront reduction.  Words without a peer or an element
  // count as published.
  const int E = a.M * BN;
  uint32_t* slots = a.part + (size_t)tile * a.S * E;
  const bool probing = early_probe(a, BN) && rank == a.S - 1;
  if (wave == 0 && probing && !probed) {
#pragma unroll
    for (int i = 0; i < kProbeRanks; ++i) probe[i] = load_slot(probe_src(a, E, tile, lane, i, true));
  }
  auto probe_seen = [&](int i) { return i >= a.S - 1 || lane >= E || probe[i] != 0u; };

  // Every wavefront's sums are in LDS after the barrier; wavefront 0 carries
  // on alone.  (A variant where the last wavefront to arrive at an LDS
  // counter carried on, with no barrier, measured slower.)
  wait_lgkmcnt0();
  barrier_keep_loads();
  if (wave != 0) return;
  LOWM_TRACE(kTraceReduced);

  // Wavefront 0 owns the epilogue.  Output element e of the tile is
  // (m, nl) = (e / BN, e % BN).  The MFMA keeps D[row][col] in lane
  // col + 16*(row/4), register row % 4; rows are activation rows, columns
  // weight rows.
  auto red_pos = [&](int e) -> float& {   // wavefront 0's sum of element e
    const int m = e / BN, nl = e - (e / BN) * BN;
    const int b = m >> 4, mm = m & 15;
    return red_at(0, nl >> 4, b, mm & 3, (nl & 15) + 16 * (mm >> 2));
  };
  auto rank_sum = [&](int e) {
    const int m = e / BN, nl = e - (e / BN) * BN;
    const int b = m >> 4, mm = m & 15;
    const int ln = (nl & 15) + 16 * (mm >> 2), rg = nl >> 4, i = mm & 3;
    float p = red_at(0, rg, b, i, ln);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) p += red_at(w, rg, b, i, ln);
    return p;
  };
  if (a.S == 1) {
    for (int e = lane; e < E; e += kWave) {
      const int m = e / BN, n = n0 + (e - m * BN);
      if (n < a.N) store_out<OutT>(a, m, n, rank_sum(e));
    }
    publish_flags<RG, OutT>(a, n0, lane);
    LOWM_TRACE(kTraceEnd);
    return;
  }

  uint32_t* ctr = a.ctr + (size_t)tile * kCtrStride;
  LOWM_STALL(kSitePublish, 0);
  if (probing) {
    // The last rank (rank-major dispatch: issued after every peer of its
    // tile on the same XCD) polls until every peer's slot holds its partial,
    // for at most kProbeTicks; a peer's slot is visible without its
    // publish acknowledgement and arrival, which the loaded memory system
    // delays by microseconds.  Past the limit it publishes and arrives like
    // any rank, so the result never depends on the dispatch order.
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
      bool seen = true;
#pragma unroll
      for (int i = 0; i < kProbeRanks; ++i) seen = seen && probe_seen(i);
      if (__all(seen)) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > kProbeTicks) break;
      __builtin_amdgcn_s_sleep(2);
#pragma unroll
      for (int i = 0; i < kProbeRanks; ++i)
        if (!probe_seen(i)) probe[i] = load_slot(slots + (size_t)i * E + lane);
    }
    bool seen = true;
#pragma unroll
    for (int i = 0; i < kProbeRanks; ++i) seen = seen && probe_seen(i);
    if (__all(seen)) {
      // Every peer has published: this rank is the owner without publishing
      // or arriving.  No peer can become the owner, since only the S-1 peers
      // arrive and the last of them sees S-2 earlier arrivals.  The fold is
      // the same rank-order sum as the owner's below, this rank's partial
      // last.  (Traced as a rank that never arrived.)
      //
      // Subtract the S-1 arrivals of the peers: whenever theirs land, the
      // counter is back at zero for the next launch.  (Issued first: later,
      // the compiler would wait for the stores below before it.)
      if (lane == 0)
        __hip_atomic_fetch_add(ctr, (uint32_t)(1 - a.S), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      LOWM_STALL(kSiteFold, 0);
      if (lane < E) {
        float v = dec_partial(probe[0]);
#pragma unroll
        for (int i = 1; i < kProbeRanks; ++i)
          if (i < a.S - 1) v += dec_partial(probe[i]);
        v += rank_sum(lane);
        const int m = lane / BN, n = n0 + (lane - m * BN);
        if (n < a.N) store_out<OutT>(a, m, n, v);  // a6
#pragma unroll
        for (int i = 0; i < kProbeRanks; ++i)
          if (i < a.S - 1) store_slot(slots + (size_t)i * E + lane, 0u);
      }
      publish_flags<RG, OutT>(a, n0, lane);
      LOWM_TRACE(kTraceEnd);
      return;
    }
  }

  // a4: publish this rank's partial, then arrive.  The partial is written
  // with device-scope stores (sc1: written through this XCD's L2 to where
  // every XCD sees it) and the arrival is issued only after all of them are
  // acknowledged (vmcnt(0)): the release is carried by the stores' own
  // scope, so no cache-wide write-back is needed.
  for (int e = lane; e < E; e += kWave) store_slot(slots + (size_t)rank * E + e, enc_partial(rank_sum(e)));
  wait_vmcnt0();
  pin_issue();
  uint32_t before = 0;
  if (lane == 0)
    before = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  before = __builtin_amdgcn_readfirstlane(before);
  LOWM_TRACE(kTraceArrived);
  if (before != (uint32_t)(a.S - 1)) {   // not the last rank: done
    LOWM_TRACE(kTraceEnd);
    return;
  }

  // a5: the owner.  The peers' partials are read with device-scope loads
  // (sc1), issued only after the arrival count is known, so they observe
  // every partial whose arrival was counted; no cache-wide invalidate.  The
  // fold is in rank order with this rank's partial, from LDS, at its own
  // position; every slot read goes back to zero.
  LOWM_STALL(kSiteFold, 0);
  // Two passes: the folds (global loads only, four elements' loads in
  // flight at once; each result replaces the element's wavefront-0 sum in
  // LDS, which nothing else reads), then the stores of C and the clearing
  // of the slots, which nothing waits for.  Past the tile's end a lane folds
  // its first element again and keeps nothing.
  auto fold_pass = [&](auto sn_c) {
    constexpr int SN = decltype(sn_c)::value;
    for (int e0 = lane; e0 < E; e0 += 4 * kWave) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kWave < E ? e0 + u * kWave : e0;
        v[u] = SN > 0 ? fold_ranks_n<(SN > 0 ? SN : 2)>(slots, E, e, rank, rank_sum(e))
                      : fold_ranks(slots, E, e, a.S, rank, rank_sum(e));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + u * kWave < E) red_pos(e0 + u * kWave) = v[u];
    }
  };
  switch (a.S) {
    case 2: fold_pass(std::integral_constant<int, 2>{}); break;
    case 3: fold_pass(std::integral_constant<int, 3>{}); break;
    case 4: fold_pass(std::integral_constant<int, 4>{}); break;
    case 8: fold_pass(std::integral_constant<int, 8>{}); break;
    default: fold_pass(std::integral_constant<int, 0>{}); break;
  }
  for (int e = lane; e < E; e += kWave) {
    const int m = e / BN, n = n0 + (e - m * BN);
    if (n < a.N) store_out<OutT>(a, m, n, red_pos(e));  // a6
    clear_slots(slots, E, e, a.S);
  }
  publish_flags<RG, OutT>(a, n0, lane);
  // Every rank has arrived: the tile's counter is zero again for the next
  // launch.
  if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  LOWM_TRACE(kTraceEnd);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int MB, int RG, int STAGE, int U, int NS, int ACT, typename OutT>
__device__ __forceinline__ void kernel_body(const Args& a) {
  using SH = Shape<MB, RG, STAGE, U, NS, ACT>;
  constexpr int BN = SH::BN;
  constexpr int kSlot = SH::slot_elems;
  constexpr int kPitch = SH::kPitch;
  constexpr int G = SH::group_loads;
  constexpr bool kLds = STAGE == kStageLds;

  // LDS stages are distinct objects so the compiler can tell that a refill of
  // one stage does not alias reads of another and needs no extra wait.
  __shared__ u32x4 ring0[kSlot];
  __shared__ u32x4 ring1[kLds ? kSlot : 1];
  __shared__ u32x4 ring2[(kLds && NS > 2) ? kSlot : 1];
  __shared__ u32x4 ring3[(kLds && NS > 3) ? kSlot : 1];
  __shared__ float red_own[SH::red_in_ring ? 1 : SH::red_floats];
  // activation slice (ACT): M rows of nvec+1 vectors, sized at launch
  extern __shared__ u32x4 act_lds[];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;     // which 16-byte vector of a 32-wide K chunk
  const int l16 = lane & 15;   // row within a 16-row MFMA operand

  int tile, rank;
  decode_tile(a, BN, tile, rank);
  LOWM_TRACE(kTraceEntry);
  LOWM_TRACE_IDS();
  if (tile * BN >= a.N) return;
  const int n0 = tile * BN;
  const int Ks = a.nvec * kVecK;
  const size_t k0 = (size_t)rank * Ks;
  const int nvec = a.nvec;

  // K order.  LDS variant: each tile starts its slice at a different 512-wide
  // stage and wraps around, so the workgroups in flight spread over the
  // columns of W.  REG variant: wavefront w owns the contiguous chunk range
  // [w*cpw, (w+1)*cpw) of the slice and streams it front to back, so the
  // loads it issues back to back cover its 16 rows x U*64 contiguous bytes.
  const int nunits = kLds ? (nvec + 63) / 64 : (nvec + 3) / 4;
  const int rot = kLds ? (int)(((unsigned)tile * 5u) % (unsigned)nunits) : 0;
  auto phys = [&](int u) { return u < nunits ? (u + rot < nunits ? u + rot : u + rot - nunits) : -1; };
  const bool whole = kLds ? (nvec % 64 == 0) : (nvec % 4 == 0);
  const int cpw = (nunits + kWaves - 1) / kWaves;            // REG: chunks per wavefront
  const int nsteps = kLds ? nunits : (cpw + U - 1) / U;

  // Activation rows of this lane per 16-row block; rows >= M are clamped to
  // row 0 and masked to zero.
  const uint16_t* arow[MB];
  int arow_lds[MB];
  bool a_ok[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int m = 16 * b + l16;
    a_ok[b] = m < a.M;
    arow[b] = a.A + (size_t)(a_ok[b] ? m : 0) * a.K + k0;
    arow_lds[b] = (a_ok[b] ? m : 0) * (nvec + 1);
  }
  // Element offset of vector v of the slice, clamped into the slice.
  auto voff = [&](int v) { return (v < nvec ? v : nvec - 1) * kVecK; };

  f32x4 acc[RG][MB];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[rg][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[ACT ? 1 : NS][U][MB];
  u32x4 wreg[kLds ? 1 : NS][U][RG];

  // REG variant: this lane's W rows.
  const uint16_t* wrow[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    int n = n0 + 16 * rg + l16;
    n = n < a.N ? n : a.N - 1;
    wrow[rg] = a.W + (size_t)n * a.K + k0;
  }
  // LDS variant: the rows this wavefront moves into each stage (rows wave,
  // wave+4, ...), lane i carrying bytes [16i, 16i+16) of the row's 1 KB.
  constexpr int kRowsPerWave = BN / kWaves;
  const uint16_t* drow[kLds ? kRowsPerWave : 1];
  if constexpr (kLds) {
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      int n = n0 + wave + kWaves * i;
      n = n < a.N ? n : a.N - 1;
      drow[i] = a.W + (size_t)n * a.K + k0;
    }
  }

  auto slot_ptr = [&](auto slot_c) -> u32x4* {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (SL == 0) return ring0;
    else if constexpr (SL == 1) return ring1;
    else if constexpr (SL == 2) return ring2;
    else return ring3;
  };

  // Vector index (within the slice) of this lane's operand for chunk j of
  // step s, or -1 past the end of the slice (or of this wavefront's range).
  auto operand_vec = [&](int s, int j) {
    if constexpr (kLds) {
      const int p = phys(s);
      return p < 0 ? -1 : p * 64 + (wave * U + j) * 4 + g;
    } else {
      const int c = s * U + j;
      const int chunk = wave * cpw + c;
      return (c < cpw && chunk < nunits) ? chunk * 4 + g : -1;
    }
  };
  // REG variant: where a load past the end of this wavefront's range reads
  // instead (its own last chunk, just loaded, so it hits in L2).
  auto load_vec = [&](int s, int j) {
    const int c = s * U + j;
    int chunk = wave * cpw + (c < cpw ? c : cpw - 1);
    chunk = chunk < nunits ? chunk : nunits - 1;
    return chunk * 4 + g;
  };

  // Issue the loads of step s (< nsteps) into stage slot SL.
  auto issue = [&](auto slot_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (kLds) {
      u32x4* slot = slot_ptr(slot_c);
      const int off = voff(phys(s) * 64 + lane);
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        // one contiguous 1 KB piece of row (wave + 4i); lane i's 16 bytes
        // land at base + 16*i
        __builtin_amdgcn_global_load_lds(
            drow[i] + off,
            (__attribute__((address_space(3))) void*)(slot + (wave + kWaves * i) * kPitch), 16,
            0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int off = voff(load_vec(s, j));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) wreg[SL][j][rg] = load16(wrow[rg] + off);
      }
    }
    if constexpr (!ACT) {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int off = voff(kLds ? max(operand_vec(s, j), 0) : load_vec(s, j));
#pragma unroll
        for (int b = 0; b < MB; ++b) areg[SL][j][b] = load16(arow[b] + off);
      }
    }
    pin_issue();
  };

  // Multiply-accumulate step s out of stage slot SL.  MASK: some operand of
  // the step may lie outside the slice (ragged K or a step past the end).
  auto compute_impl = [&](auto slot_c, auto mask_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int v = operand_vec(s, j);
      bool v_ok = true;
      if constexpr (MASK) v_ok = v >= 0 && v < nvec;
      u32x4 wv[RG];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        if constexpr (kLds) {
          const u32x4* slot = slot_ptr(slot_c);
          wv[rg] = slot[(16 * rg + l16) * kPitch + (wave * U + j) * 4 + g];
        } else {
          wv[rg] = wreg[SL][j][rg];
        }
        if constexpr (MASK) wv[rg] = v_ok ? wv[rg] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        u32x4 av;
        if constexpr (ACT) {
          av = act_lds[arow_lds[b] + (v_ok ? v : 0)];
        } else {
          av = areg[SL][j][b];
        }
        av = (a_ok[b] && v_ok) ? av : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) acc[rg][b] = mfma(av, wv[rg], acc[rg][b]);
      }
    }
  };
  auto compute = [&](auto slot_c, int s) {
    // every operand of the step lies inside the slice: no masking needed
    const bool full =
        whole && (kLds ? s < nunits : ((s + 1) * U <= cpw && (wave + 1) * cpw <= nunits));
    if (full)
      compute_impl(slot_c, std::false_type{}, s);
    else
      compute_impl(slot_c, std::true_type{}, s);
  };

  // One pipeline step: wait for stage s, refill the stage step s-1 used with
  // step s+NS-1 (if there is one), compute step s.
  auto step = [&](auto slot_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int NEXT = (SL + NS - 1) % NS;
    if constexpr (kLds) {
      // Own loads of stage s have landed once only the younger groups
      // (at most NS-2, fewer near the end) are outstanding ...
      const int younger = min(NS - 2, nsteps - 1 - s);
      wait_groups<G>(younger);
      // ... every wavefront's reads of the previous stage have completed ...
      wait_lgkmcnt0();
      // ... and after the barrier both hold for the whole workgroup, so the
      // stage read in step s-1 may be refilled and stage s may be read.
      barrier_keep_loads();
      LOWM_STALL(kSiteStageRead, s);
    }
    if (s == 0) LOWM_TRACE(kTraceFirstStage);
    if (s + NS - 1 < nsteps) issue(std::integral_constant<int, NEXT>{}, s + NS - 1);
    compute(slot_c, s);
  };

  // The arrival counter starts at zero before any wavefront can reach the
  // end: set here, published by the first barrier every variant executes
  // (the stage barrier, the activation barrier, or the one below).

  LOWM_STALL(kSiteEntry, 0);

  // ACT: the activation slice goes to LDS first, 1 KB pieces spread over the
  // wavefronts (every wavefront issues the same number; surplus issues repeat
  // the last piece into its own place).
  if constexpr (ACT) {
    const int ppr = nvec / 64;                      // pieces per row
    const int total = a.M * ppr;
    const int per_wave = (total + kWaves - 1) / kWaves;
    for (int i = 0; i < per_wave; ++i) {
      int idx = wave + kWaves * i;
      idx = idx < total ? idx : total - 1;
      const int m = idx / ppr, p = idx - (idx / ppr) * ppr;
      __builtin_amdgcn_global_load_lds(
          a.A + (size_t)m * a.K + k0 + p * 512 + lane * kVecK,
          (__attribute__((address_space(3))) void*)(act_lds + m * (nvec + 1) + p * 64), 16, 0, 0);
    }
  }

  // Prologue: groups 0 .. NS-2 (as many as there are steps).
  issue(std::integral_constant<int, 0>{}, 0);
  if constexpr (NS > 2) {
    if (1 < nsteps) issue(std::integral_constant<int, 1>{}, 1);
  }
  if constexpr (NS > 3) {
    if (2 < nsteps) issue(std::integral_constant<int, 2>{}, 2);
  }
  if constexpr (ACT && !kLds) {
    // The register variant has no stage barrier: wait here until the
    // activation pieces (older than every group) have landed, then make all
    // wavefronts' pieces visible to all.
    wait_groups<G>(min(NS - 1, nsteps));
    wait_lgkmcnt0();
    barrier_keep_loads();
  }

  for (int s = 0; s < nsteps; s += NS) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 >= nsteps) break;
    step(std::integral_constant<int, 1 % NS>{}, s + 1);
    if constexpr (NS > 2) {
      if (s + 2 >= nsteps) break;
      step(std::integral_constant<int, 2 % NS>{}, s + 2);
    }
    if constexpr (NS > 3) {
      if (s + 3 >= nsteps) break;
      step(std::integral_constant<int, 3 % NS>{}, s + 3);
    }
  }
  LOWM_TRACE(kTraceLoopEnd);

  // Wavefront reduction through LDS, added in wavefront order below.  In the
  // LDS variant it reuses stage 0, which every wavefront must have finished
  // reading first.
  float* red = SH::red_in_ring ? reinterpret_cast<float*>(ring0) : red_own;
  if constexpr (SH::red_in_ring) {
    wait_lgkmcnt0();
    barrier_keep_loads();
  }
  uint32_t probe[kProbeRanks];
  workgroup_epilogue<MB, RG, OutT>(a, acc, red, wave, lane, tile, rank, n0, probe, false);
}

// ---------------------------------------------------------------------------
// Line-pair tiles: W goes global -> LDS with direct-to-LDS loads in which
// every request is a whole 128-byte line and carries the non-temporal hint
// (each W byte is read once).  One load moves 8 rows x 128 B; two of them,
// a "line pair", hold 16 rows x 64 K, the operands of two MFMA chunks.  Each
// wavefront streams its own contiguous quarter of the K slice through a ring
// of R line-pair slots that only it reads, so the main loop has no workgroup
// barrier: a slot is refilled after the wavefront's own reads of it have
// completed (lgkmcnt), and read after the loads that fill it have landed
// (vmcnt) -- both waits explicit, since the compiler does not order reads of
// LDS after direct-to-LDS loads.  The activation operands go global ->
// registers with each line pair.
//
// LDS layout of a slot: per row group, the two 8-row pieces at a pitch of
// 1088 B (64 B of padding); within a piece, row q's 128 B line at q*128.
// Lane 8q+j of a load writes position j of row q and fetches 16-byte piece
// (j - q/2) mod 8 of that row's line: a rotation that makes the MFMA-layout
// reads (16 rows at one K offset) fall in distinct LDS banks.
// ---------------------------------------------------------------------------
template <int MB, int RG, int R>
struct LineShape {
  static constexpr int BN = 16 * RG;
  static constexpr int kPiecePitch = 68;                 // u32x4 (1088 B)
  static constexpr int slot_elems = RG * 2 * kPiecePitch;  // one wavefront's slot
  static constexpr int red_floats = kWaves * RG * MB * 4 * kWave;
  static constexpr int lds_bytes = kWaves * R * slot_elems * 16 + red_floats * 4;
  static constexpr int a_vgprs = R * 2 * MB * 4;
  // vector-memory ops per line pair: 2 W loads per row group, 2 A loads per
  // activation block
  static constexpr int pair_loads = 2 * RG + 2 * MB;
  static constexpr bool valid = R >= 2 && R <= 4 && MB <= 2 && lds_bytes <= 48 * 1024 &&
                                a_vgprs <= 64 && (R - 1) * pair_loads <= 63;
};

// The ring slots arrive as distinct restrict-qualified pointers: once the
// body is inlined they carry alias scopes, from which the compiler sees that
// a refill of one slot does not alias reads of another, and adds no wait of
// its own beyond the explicit ones.
template <int MB, int RG, int R, typename OutT>
__device__ __forceinline__ void line_tile_body(const Args& a, u32x4* __restrict__ ring0,
                                               u32x4* __restrict__ ring1,
                                               u32x4* __restrict__ ring2,
                                               u32x4* __restrict__ ring3,
                                               float* __restrict__ red) {
  using SH = LineShape<MB, RG, R>;
  constexpr int BN = SH::BN;
  constexpr int kSlot = SH::slot_elems;
  constexpr int kPP = SH::kPiecePitch;
  constexpr int G = SH::pair_loads;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;
  const int l16 = lane & 15;

  int tile, rank;
  decode_tile(a, BN, tile, rank);
  LOWM_TRACE(kTraceEntry);
  LOWM_TRACE_IDS();
  if (tile * BN >= a.N) return;
  const int n0 = tile * BN;
  const int nvec = a.nvec;
  // line pairs (64 K each) per wavefront; the launch requires nvec % 32 == 0
  const int P = nvec / 32;
  const size_t kw = (size_t)rank * nvec * kVecK + (size_t)wave * P * 64;

  // Activation rows of this lane per 16-row block.  Rows >= M read row 0:
  // MFMA output rows are independent and rows >= M are never stored, so
  // their operands need no masking (and the operand registers no select,
  // which would make the compiler wait for them at the top of the loop).
  const uint16_t* arow[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int m = 16 * b + l16;
    arow[b] = a.A + (size_t)(m < a.M ? m : 0) * a.K + kw + g * kVecK;
  }
  // Load sources: row 8i+qr of row group rg, rotated piece of its line.
  const int qr = lane >> 3;
  const int piece = ((lane & 7) - (qr >> 1)) & 7;
  const uint16_t* wsrc[RG][2];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int n = n0 + 16 * rg + 8 * i + qr;
      n = n < a.N ? n : a.N - 1;
      wsrc[rg][i] = a.W + (size_t)n * a.K + kw + piece * kVecK;
    }
  // MFMA-layout read offsets within a slot: row l16, piece 4c+g of the line.
  int rpos[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    rpos[c] = (l16 >> 3) * kPP + (l16 & 7) * 8 + ((4 * c + g + ((l16 & 7) >> 1)) & 7);

  f32x4 acc[RG][MB];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[rg][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 areg[R][2][MB];

  auto slot_ptr = [&](auto slot_c) -> u32x4* {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (SL == 0) return ring0 + wave * kSlot;
    else if constexpr (SL == 1) return ring1 + wave * kSlot;
    else if constexpr (SL == 2) return ring2 + wave * kSlot;
    else return ring3 + wave * kSlot;
  };
  // Line pair p (< P) into slot SL: 2*RG direct-to-LDS loads, then the
  // activation operands of its two chunks.
  auto issue = [&](auto slot_c, int p) {
    constexpr int SL = decltype(slot_c)::value;
    u32x4* slot = slot_ptr(slot_c);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(
            wsrc[rg][i] + (size_t)p * 64,
            (__attribute__((address_space(3))) void*)(slot + (rg * 2 + i) * kPP), 16, 0,
            kStreamAux);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < MB; ++b) areg[SL][c][b] = load16(arow[b] + (size_t)p * 64 + c * 32);
    pin_issue();
  };
  // Step p (line pair p) out of slot SL: wait until pair p has landed (at
  // most YOUNGER pairs issued after it still in flight), read it, multiply,
  // then refill the slot with pair p+R when REFILL says there is one.
  // The last rank's probe of its peers' slots (see workgroup_epilogue) is
  // issued inside the loop, once the second-to-last line pair has landed, so
  // that its latency overlaps the last pair's.  Every wavefront issues the
  // same kProbeRanks loads (harmless ones where it does not probe) so the
  // wait counts stay compile-time constants: after the probe, a step's wait
  // allows kProbeRanks more outstanding operations.
  const int E = a.M * BN;
  const bool probing = early_probe(a, BN) && rank == a.S - 1 && wave == 0;
  const uint32_t* psrc[kProbeRanks];
#pragma unroll
  for (int i = 0; i < kProbeRanks; ++i) psrc[i] = probe_src(a, E, tile, lane, i, probing);
  uint32_t probe[kProbeRanks];
  auto issue_probe = [&]() {
#pragma unroll
    for (int i = 0; i < kProbeRanks; ++i) probe[i] = load_slot(psrc[i]);
    pin_issue();
  };
  auto step = [&](auto slot_c, auto younger_c, auto extra_c, auto probe_c, int p,
                  bool refill) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int YOUNGER = decltype(younger_c)::value;
    constexpr int EXTRA = decltype(extra_c)::value;
    const u32x4* slot = slot_ptr(slot_c);
    wait_vmcnt<YOUNGER * G + EXTRA>();
    if constexpr (decltype(probe_c)::value) issue_probe();
    LOWM_STALL(kSiteStageRead, p);
    if (p == 0) LOWM_TRACE(kTraceFirstStage);
    // both chunks' W operands (the reads are complete after lds_wait, so the
    // refill below cannot overwrite them early)
    u32x4 wv[2 * RG];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) wv[c * RG + rg] = lds_read_opaque(slot + rg * 2 * kPP + rpos[c]);
    lds_wait(wv);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          acc[rg][b] = mfma(areg[SL][c][b], wv[c * RG + rg], acc[rg][b]);
    if (refill) issue(slot_c, p + R);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using YR = std::integral_constant<int, R - 1>;

  LOWM_STALL(kSiteEntry, 0);
  // Steady state: whole ring cycles in which every step refills its slot, so
  // R pairs are always in flight and each wait count is the same constant.
  // The first cycle runs before the loop: straight-line code keeps the
  // compiler's own waits for the activation registers exact.
  using NoProbe = std::false_type;
  auto cycle = [&](int p) {
    step(I0{}, YR{}, I0{}, NoProbe{}, p, true);
    step(I1{}, YR{}, I0{}, NoProbe{}, p + 1, true);
    if constexpr (R > 2) step(I2{}, YR{}, I0{}, NoProbe{}, p + 2, true);
    if constexpr (R > 3) step(I3{}, YR{}, I0{}, NoProbe{}, p + 3, true);
  };
  int p0 = 0;
  if (P >= 2 * R) {
    // prologue: the first R pairs, unconditionally
    issue(I0{}, 0);
    issue(I1{}, 1);
    if constexpr (R > 2) issue(I2{}, 2);
    if constexpr (R > 3) issue(I3{}, 3);
    cycle(0);
    for (p0 = R; p0 + 2 * R <= P; p0 += R) cycle(p0);
  } else {
    // prologue: as many of the first R pairs as there are
    issue(I0{}, 0);
    if (1 < P) issue(I1{}, 1);
    if constexpr (R > 2) {
      if (2 < P) issue(I2{}, 2);
    }
    if constexpr (R > 3) {
      if (3 < P) issue(I3{}, 3);
    }
  }
  // Tail: the REM = P - p0 remaining pairs (1 .. 2R-1), all issued or
  // issued by these steps; one straight-line sequence per REM, so every wait
  // count and refill is a constant.
  auto tail_step = [&](auto rem_c, auto i_c) {
    constexpr int REM = decltype(rem_c)::value;
    constexpr int I = decltype(i_c)::value;
    if constexpr (I < REM) {
      constexpr int YOUNGER = (REM - 1 - I) < (R - 1) ? (REM - 1 - I) : (R - 1);
      // the probe goes out after the second-to-last pair's wait (no refill
      // follows it), so only the last step's wait allows for it
      constexpr int EXTRA = (I == REM - 1) ? kProbeRanks : 0;
      constexpr bool PROBE = (REM >= 2 && I == REM - 2);
      step(std::integral_constant<int, I % R>{}, std::integral_constant<int, YOUNGER>{},
           std::integral_constant<int, EXTRA>{}, std::integral_constant<bool, PROBE>{}, p0 + I,
           I + R < REM);
    }
  };
  auto tail = [&](auto rem_c) {
    if constexpr (decltype(rem_c)::value == 1) issue_probe();
    tail_step(rem_c, I0{});
    tail_step(rem_c, I1{});
    tail_step(rem_c, I2{});
    tail_step(rem_c, I3{});
    tail_step(rem_c, std::integral_constant<int, 4>{});
    tail_step(rem_c, std::integral_constant<int, 5>{});
    tail_step(rem_c, std::integral_constant<int, 6>{});
  };
  static_assert(2 * R - 1 <= 7, "tail covers at most 7 pairs");
  switch (P - p0) {
    case 1: tail(std::integral_constant<int, 1>{}); break;
    case 2: tail(std::integral_constant<int, 2>{}); break;
    case 3: tail(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr (2 * R - 1 >= 4) tail(std::integral_constant<int, 4>{}); break;
    case 5: if constexpr (2 * R - 1 >= 5) tail(std::integral_constant<int, 5>{}); break;
    case 6: if constexpr (2 * R - 1 >= 6) tail(std::integral_constant<int, 6>{}); break;
    case 7: if constexpr (2 * R - 1 >= 7) tail(std::integral_constant<int, 7>{}); break;
    default: break;
  }
  mfma_settle(reinterpret_cast<f32x4(&)[RG * MB]>(acc));
  LOWM_TRACE(kTraceLoopEnd);
  workgroup_epilogue<MB, RG, OutT>(a, acc, red, wave, lane, tile, rank, n0, probe, true);
}

template <int MB, int RG, int R, typename OutT>
__global__ __launch_bounds__(kThreads) void lowm_line_kernel(Args a0, Batch bt) {
#if defined(__HIP_DEVICE_COMPILE__)
  const Args a = gemm_args(a0, bt);
  using SH = LineShape<MB, RG, R>;
  // one LDS object per ring slot (all wavefronts' copies of that slot)
  __shared__ u32x4 ring0[kWaves * SH::slot_elems];
  __shared__ u32x4 ring1[kWaves * SH::slot_elems];
  __shared__ u32x4 ring2[R > 2 ? kWaves * SH::slot_elems : 1];
  __shared__ u32x4 ring3[R > 3 ? kWaves * SH::slot_elems : 1];
  __shared__ float red[SH::red_floats];
  line_tile_body<MB, RG, R, OutT>(a, ring0, ring1, ring2, ring3, red);
#endif
}

// ---------------------------------------------------------------------------
// Wavefront tiles: one wavefront is the whole workgroup and owns a tile of
// BN = 16*RG weight rows for its entire K slice, so no wavefront waits for
// another: no LDS stage barrier and no wavefront reduction.  W streams into a
// ring of NS register stages of U 32-wide chunks (16 B per lane per chunk and
// row group); the ring is issued unconditionally (past the end of the slice
// the addresses repeat the slice's last vector and the products are masked),
// so the loop body has no branches and the compiler's wait counts stay exact.
// ---------------------------------------------------------------------------
template <int MB, int RG, int U, int NS, int ACT>
struct WaveShape {
  static constexpr int BN = 16 * RG;
  static constexpr int stage_vgprs = NS * U * 4 * (RG + (ACT ? 0 : MB));
  static constexpr bool valid = NS >= 2 && NS <= 4 && stage_vgprs <= 256 && (!ACT || MB <= 2);
};

template <int MB, int RG, int U, int NS, int ACT, typename OutT>
__device__ __forceinline__ void wave_tile_body(const Args& a) {
  constexpr int BN = 16 * RG;
  extern __shared__ u32x4 act_lds[];   // ACT: M rows of nvec+1 vectors

  const int lane = threadIdx.x;
  const int wave = 0;
  (void)wave;
  const int g = lane >> 4;
  const int l16 = lane & 15;

  int tile, rank;
  decode_tile(a, BN, tile, rank);
  LOWM_TRACE(kTraceEntry);
  LOWM_TRACE_IDS();
  if (tile * BN >= a.N) return;
  const int n0 = tile * BN;
  const int nvec = a.nvec;
  const size_t k0 = (size_t)rank * nvec * kVecK;
  const int nchunks = (nvec + 3) / 4;
  const int rot = (int)(((unsigned)tile * 5u) % (unsigned)nchunks);
  const bool whole = nvec % 4 == 0;
  const int nsteps = (nchunks + U - 1) / U;

  const uint16_t* wrow[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    int n = n0 + 16 * rg + l16;
    n = n < a.N ? n : a.N - 1;
    wrow[rg] = a.W + (size_t)n * a.K + k0;
  }
  const uint16_t* arow[MB];
  int arow_lds[MB];
  bool a_ok[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int m = 16 * b + l16;
    a_ok[b] = m < a.M;
    arow[b] = a.A + (size_t)(a_ok[b] ? m : 0) * a.K + k0;
    arow_lds[b] = (a_ok[b] ? m : 0) * (nvec + 1);
  }

  LOWM_STALL(kSiteEntry, 0);
  if constexpr (ACT) {
    // the activation slice to LDS, 1 KB pieces; read back only after the
    // explicit wait below the prologue (the compiler does not order a read
    // of LDS after a direct-to-LDS load that writes it)
    const int ppr = nvec / 64;
    const int total = a.M * ppr;
    for (int idx = 0; idx < total; ++idx) {
      const int m = idx / ppr, p = idx - (idx / ppr) * ppr;
      __builtin_amdgcn_global_load_lds(
          a.A + (size_t)m * a.K + k0 + p * 512 + lane * kVecK,
          (__attribute__((address_space(3))) void*)(act_lds + m * (nvec + 1) + p * 64), 16, 0, 0);
    }
  }

  // chunk c of the slice in this tile's rotated order; -1 past the end
  auto phys = [&](int c) {
    return c < nchunks ? (c + rot < nchunks ? c + rot : c + rot - nchunks) : -1;
  };
  auto voff = [&](int v) { return (v < nvec ? v : nvec - 1) * kVecK; };

  f32x4 acc[2][RG][MB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[h][rg][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wreg[NS][U][RG];
  u32x4 areg[ACT ? 1 : NS][U][MB];

  auto issue = [&](auto slot_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = phys(s * U + j);
      const int off = voff((p < 0 ? nchunks - 1 : p) * 4 + g);
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) wreg[SL][j][rg] = load16(wrow[rg] + off);
      if constexpr (!ACT) {
#pragma unroll
        for (int b = 0; b < MB; ++b) areg[SL][j][b] = load16(arow[b] + off);
      }
    }
    pin_issue();
  };

  auto compute_impl = [&](auto slot_c, auto mask_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = phys(s * U + j);
      const int v = p * 4 + g;
      bool v_ok = true;
      if constexpr (MASK) v_ok = p >= 0 && v < nvec;
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        u32x4 av;
        if constexpr (ACT) av = act_lds[arow_lds[b] + (v_ok ? v : 0)];
        else av = areg[SL][j][b];
        av = (a_ok[b] && v_ok) ? av : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          u32x4 wv = wreg[SL][j][rg];
          if constexpr (MASK) wv = v_ok ? wv : u32x4{0u, 0u, 0u, 0u};
          acc[j & 1][rg][b] = mfma(av, wv, acc[j & 1][rg][b]);
        }
      }
    }
  };
  auto step = [&](auto slot_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int NEXT = (SL + NS - 1) % NS;
    issue(std::integral_constant<int, NEXT>{}, s + NS - 1);
    if (whole && (s + 1) * U <= nchunks)
      compute_impl(slot_c, std::false_type{}, s);
    else
      compute_impl(slot_c, std::true_type{}, s);
  };

  issue(std::integral_constant<int, 0>{}, 0);
  if constexpr (NS > 2) issue(std::integral_constant<int, 1>{}, 1);
  if constexpr (NS > 3) issue(std::integral_constant<int, 2>{}, 2);
  if constexpr (ACT) {
    // The activation pieces went out before the NS-1 prologue groups: once
    // at most those groups' loads are outstanding, the pieces are in LDS.
    wait_vmcnt<(NS - 1) * U * RG>();
  }
  for (int s = 0; s < nsteps; s += NS) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
    if constexpr (NS > 2) step(std::integral_constant<int, 2>{}, s + 2);
    if constexpr (NS > 3) step(std::integral_constant<int, 3>{}, s + 3);
  }
  wait_vmcnt0();
  LOWM_TRACE(kTraceLoopEnd);

  // This lane's sums: block b, register i is D[4g+i][l16] = C[16b+4g+i][n0+16rg+l16].
  f32x4 sum[RG][MB];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int b = 0; b < MB; ++b) sum[rg][b] = acc[0][rg][b] + acc[1][rg][b];

  if (a.S == 1) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 16 * b + 4 * g + i, n = n0 + 16 * rg + l16;
          if (m < a.M && n < a.N) store_out<OutT>(a, m, n, sum[rg][b][i]);
        }
    publish_flags<RG, OutT>(a, n0, lane);
    LOWM_TRACE(kTraceEnd);
    return;
  }

  // a4: publish (device-scope stores, all acknowledged before the arrival)
  LOWM_STALL(kSitePublish, 0);
  const int E = a.M * BN;
  uint32_t* slots = a.part + (size_t)tile * a.S * E;
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * b + 4 * g + i, nl = 16 * rg + l16;
        if (m < a.M) store_slot(slots + (size_t)rank * E + m * BN + nl, enc_partial(sum[rg][b][i]));
      }
  wait_vmcnt0();
  pin_issue();
  uint32_t before = 0;
  if (lane == 0)
    before = __hip_atomic_fetch_add(a.ctr + (size_t)tile * kCtrStride, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  before = __builtin_amdgcn_readfirstlane(before);
  LOWM_TRACE(kTraceArrived);
  if (before != (uint32_t)(a.S - 1)) {
    LOWM_TRACE(kTraceEnd);
    return;
  }

  // a5/a6: the owner folds in rank order (its own partial from registers)
  // and returns every slot it read to zero
  LOWM_STALL(kSiteFold, 0);
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * b + 4 * g + i, nl = 16 * rg + l16;
        if (m < a.M) sum[rg][b][i] = fold_ranks(slots, E, m * BN + nl, a.S, rank, sum[rg][b][i]);
      }
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * b + 4 * g + i, nl = 16 * rg + l16, n = n0 + nl;
        if (m >= a.M) continue;
        if (n < a.N) store_out<OutT>(a, m, n, sum[rg][b][i]);
        clear_slots(slots, E, m * BN + nl, a.S);
      }
  publish_flags<RG, OutT>(a, n0, lane);
  if (lane == 0)
    __hip_atomic_store(a.ctr + (size_t)tile * kCtrStride, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  LOWM_TRACE(kTraceEnd);
}

template <int MB, int RG, int U, int NS, int ACT, typename OutT>
__global__ __launch_bounds__(kWave) void lowm_wave_kernel(Args a, Batch bt) {
#if defined(__HIP_DEVICE_COMPILE__)
  wave_tile_body<MB, RG, U, NS, ACT, OutT>(gemm_args(a, bt));
#endif
}

// The body uses device-only builtins (direct-to-LDS loads), which the host
// pass cannot instantiate; it only needs the launch stub there.
template <int MB, int RG, int STAGE, int U, int NS, int ACT, typename OutT>
__global__ __launch_bounds__(kThreads) void lowm_splitk_kernel(Args a, Batch bt) {
#if defined(__HIP_DEVICE_COMPILE__)
  kernel_body<MB, RG, STAGE, U, NS, ACT, OutT>(gemm_args(a, bt));
#endif
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Variant {
  int stage, unroll, stages;
};
// The register/LDS variants this build provides.
constexpr Variant kVariants[] = {
    {kStageLds, 4, 2},  {kStageLds, 4, 3},  {kStageReg, 8, 2},  {kStageReg, 4, 3},
    {kStageReg, 4, 4},  {kStageReg, 16, 2}, {kStageReg, 4, 2},  {kStageWave, 4, 4},
    {kStageWave, 8, 2}, {kStageLine, 2, 2}, {kStageLine, 2, 3}, {kStageLine, 2, 4},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

typedef void (*KernelFn)(Args, Batch);

template <int MB, int RG, int VI, int ACT, typename OutT>
KernelFn kernel_for() {
  constexpr Variant v = kVariants[VI];
  if constexpr (v.stage == kStageLine) {
    // no staged activation slice: instantiated for act 0 only
    if constexpr (ACT == 0 && LineShape<MB, RG, v.stages>::valid)
      return lowm_line_kernel<MB, RG, v.stages, OutT>;
    else
      return nullptr;
  } else if constexpr (v.stage == kStageWave) {
    if constexpr (WaveShape<MB, RG, v.unroll, v.stages, ACT>::valid)
      return lowm_wave_kernel<MB, RG, v.unroll, v.stages, ACT, OutT>;
    else
      return nullptr;
  } else if constexpr (Shape<MB, RG, v.stage, v.unroll, v.stages, ACT>::valid) {
    return lowm_splitk_kernel<MB, RG, v.stage, v.unroll, v.stages, ACT, OutT>;
  } else {
    return nullptr;
  }
}

template <int MB, int RG, int ACT, typename OutT, int... VI>
void fill_row(KernelFn* row, std::integer_sequence<int, VI...>) {
  ((row[VI] = kernel_for<MB, RG, VI, ACT, OutT>()), ...);
}

// Rows per tile the build provides: 16 * RG for RG in kRowGroups.
constexpr int kRowGroups[] = {1, 2, 4};
constexpr int kNumRowGroups = sizeof(kRowGroups) / sizeof(kRowGroups[0]);
constexpr int rg_index(int rg) {
  for (int i = 0; i < kNumRowGroups; ++i)
    if (kRowGroups[i] == rg) return i;
  return -1;
}

// table[out][act][MB-1][rg_index][variant]; out 0 bf16, 1 fp32, 2 bf16 + push
enum OutKind : int { kOutBf16 = 0, kOutF32 = 1, kOutPush = 2, kNumOutKinds = 3 };
struct Table {
  KernelFn fn[kNumOutKinds][2][4][kNumRowGroups][kNumVariants];
};
template <typename OutT, int MB, int RG>
void fill_one(Table& t, int out) {
  constexpr int ri = rg_index(RG);
  fill_row<MB, RG, 0, OutT>(t.fn[out][0][MB - 1][ri], std::make_integer_sequence<int, kNumVariants>{});
  fill_row<MB, RG, 1, OutT>(t.fn[out][1][MB - 1][ri], std::make_integer_sequence<int, kNumVariants>{});
}
template <typename OutT, int MB>
void fill_mb(Table& t, int out) {
  fill_one<OutT, MB, 1>(t, out);
  fill_one<OutT, MB, 2>(t, out);
  fill_one<OutT, MB, 4>(t, out);
}
template <typename OutT>
void fill_out(Table& t, int out) {
  fill_mb<OutT, 1>(t, out);
  fill_mb<OutT, 2>(t, out);
  fill_mb<OutT, 3>(t, out);
  fill_mb<OutT, 4>(t, out);
}
const Table& table() {
  static const Table t = [] {
    Table x{};
    fill_out<__bf16>(x, kOutBf16);
    fill_out<float>(x, kOutF32);
    fill_out<PushBf16>(x, kOutPush);
    return x;
  }();
  return t;
}

thread_local int g_last_hip_error = 0;
StressArgs g_stress = {0u, -1, -1, 0, 0, -1, 0u, nullptr};

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

int threads_of(const lowm_tactic& t) { return t.stage == kStageWave ? kWave : kThreads; }

KernelFn lookup(bool f32out, int act, int M, const lowm_tactic& t, bool push = false) {
  if (t.waves != (t.stage == kStageWave ? 1 : kWaves)) return nullptr;
  const int ri = rows_index(t.rows);
  const int vi = variant_index(t);
  if (ri < 0 || vi < 0 || M < 1 || M > LOWM_MAX_M) return nullptr;
  return table().fn[push ? kOutPush : f32out ? kOutF32 : kOutBf16][act][(M + 15) / 16 - 1][ri][vi];
}

// Largest activation slice staged in LDS (bytes, padding included).
constexpr size_t kActLdsMax = 48 * 1024;
size_t act_lds_bytes(int M, int nvec) { return (size_t)M * (nvec + 1) * 16; }

// Default tactic.  Where the K slice is whole 64-K line pairs per wavefront
// (K / split_k % 256 == 0) and M <= 32: line-pair tiles of 16 rows, a ring of
// 4 slots for M <= 4 with 8..15 pairs per wavefront and of 2 otherwise; not
// for M > 16 with 16 or more pairs, where the register ring below is faster.
// Measured on MI355X at N 6144, K 4096, M 1..32, split_k 1..8, and at
// N 2304 K 12288 split_k 4 and N 49152 K 4096 split_k 2: the line tiles
// beat the register ring by 3-30 % everywhere else.
// Otherwise tiles of 16 weight rows for M <= 16 and 32 above (two row
// groups share each activation load) in a register ring: each of the four
// wavefronts streams cpw = ceil(chunks / 4) contiguous chunks of its slice.
// When cpw <= 16 the best ring issues the whole range in its first stage
// (unroll = the smallest power of two >= cpw, 2 stages); for longer ranges a
// 4-chunk, 2-stage ring beats deeper ones.  Fall back to other rings, then
// the single-wavefront and LDS variants, when the build has no such
// instantiation for this M.
int pick(int M, int N, int K, int S, lowm_tactic* t) {
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
  static const Variant others[] = {{kStageReg, 4, 2},  {kStageReg, 4, 3},  {kStageReg, 8, 2},
                                   {kStageWave, 4, 4}, {kStageWave, 8, 2}, {kStageLds, 4, 2},
                                   {kStageLds, 4, 3}};
  t->rows = M <= 16 ? 16 : 32;
  // The launch stages the activation slice in LDS when `act` is 1 and the
  // build has that instantiation, else it loads activation operands from L2;
  // the tactic must exist in the mode the launch will use.
  auto provides = [&](const Variant& v) {
    t->stage = v.stage;
    t->unroll = v.unroll;
    t->stages = v.stages;
    t->waves = v.stage == kStageWave ? 1 : kWaves;
    for (int f = 0; f < 2; ++f) {
      const bool f32 = f == 1;
      if (!(act && lookup(f32, 1, M, *t)) && !lookup(f32, 0, M, *t)) return false;
    }
    return true;
  };
  if (nvec % 32 == 0 && M <= 32) {
    const int pairs = nvec / 32;   // line pairs per wavefront
    // Measured on MI355X: 32-row line tiles beat 16-row ones only without
    // split-K, for 5..16 activation rows, 16 line pairs per wavefront and at
    // least 192 tiles (M 16, N 6144, K 4096: 12.3 vs 14.4 us; M 16, N 24576:
    // 32.9 vs 40.5); with split_k 2..8, other slice lengths or fewer tiles
    // they lose.
    if (S == 1 && M > 4 && M <= 16 && pairs == 16 && (N + 31) / 32 >= 192) {
      t->rows = 32;
      if (provides({kStageLine, 2, 2})) return LOWM_OK;
    }
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

// split_k for a shape, from a table of the fastest measured on MI355X (default
// tactic for each split_k, W streamed from HBM): M 4 and 16, N 768 .. 24576,
// K 2048 .. 16384, split_k 1, 2, 4, 8.  A shape takes its nearest grid point
// in log2 N and log2 K; M <= 8 uses the M 4 row, larger M the M 16 row.  On
// the grid every entry is the fastest split_k; off it, the neighbours were
// within 10 % of each other's best.  split_k pays when the tiles are few and
// K is long; for M 16 the larger partials make it pay less often.
constexpr unsigned char kBestSplit[2][6][4] = {
    // M <= 8            K: 2048 4096 8192 16384
    {{1, 4, 4, 8},    // N 768
     {2, 2, 4, 4},    // N 1536
     {1, 2, 2, 4},    // N 3072
     {1, 2, 2, 8},    // N 6144
     {1, 1, 2, 8},    // N 12288
     {1, 1, 2, 8}},   // N 24576
    // M > 8
    {{1, 4, 4, 4},
     {1, 2, 8, 8},
     {1, 1, 4, 4},
     {1, 1, 2, 4},
     {1, 1, 1, 1},
     {1, 1, 1, 1}}};

int nearest_log2_index(double x, double base, int last) {
  const int i = (int)floor(log2(x / base) + 0.5);
  return i < 0 ? 0 : (i > last ? last : i);
}

int pick_split(int M, int N, int K, int* split_k) {
  if (!split_k) return LOWM_ERR_INVALID_ARG;
  int rc = check_sizes(M, N, K, 1);
  if (rc != LOWM_OK) return rc;
  int S = kBestSplit[M <= 8 ? 0 : 1][nearest_log2_index(N, 768.0, 5)]
                    [nearest_log2_index(K, 2048.0, 3)];
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
KernelFn select_kernel(bool f32out, int M, int nvec, const lowm_tactic& t, size_t* dyn_lds,
                       bool push = false) {
  *dyn_lds = 0;
  // line-pair tiles stream whole 64-K line pairs per wavefront
  if (t.stage == kStageLine && nvec % 32 != 0) return nullptr;
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
  return counter_bytes(N) + (size_t)S * (size_t)M * round_up((size_t)N, kPartialPad) * sizeof(float);
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

int check_push(const PushSpec& p, const void* C, int M, int N) {
  if (!p.dst || !p.flags || p.value == 0 || p.ld < N) return LOWM_ERR_INVALID_ARG;
  if (((uintptr_t)p.dst & 1) || ((uintptr_t)p.flags & 3)) return LOWM_ERR_UNSUPPORTED;
  uintptr_t c0, c1, d0, d1, f0, f1;
  byte_span(C, M, N, N, 2, &c0, &c1);
  byte_span(p.dst, M, N, p.ld, 2, &d0, &d1);
  byte_span(p.flags, 1, (N + 15) / 16, 0, 4, &f0, &f1);
  auto overlap = [](uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) {
    return a0 < b1 && b0 < a1;
  };
  if (overlap(c0, c1, d0, d1) || overlap(c0, c1, f0, f1) || overlap(d0, d1, f0, f1))
    return LOWM_ERR_INVALID_ARG;
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
  if (push) {
    rc = check_push(*push, gemms[0].C, M, gemms[0].N);
    if (rc != LOWM_OK) return rc;
  }

  lowm_tactic t;
  if (tactic) {
    t = *tactic;
  } else {
    // One tactic serves every GEMM of the launch: pick it for the narrowest
    // (the only rule that depends on N asks for enough tiles).
    int n_min = gemms[0].N;
    for (int g = 1; g < count; ++g) n_min = gemms[g].N < n_min ? gemms[g].N : n_min;
    rc = pick(M, n_min, K, S, &t);
    if (rc != LOWM_OK) return rc;
  }
  const int nvec = K / S / kVecK;
  size_t dyn_lds = 0;
  const KernelFn fn = select_kernel(f32out, M, nvec, t, &dyn_lds, push != nullptr);
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
    grid += round_up(tiles, kXcds) * (size_t)S;
    if (grid > 0x7fffffffu) return LOWM_ERR_UNSUPPORTED;
    sl.bid_end = (int)grid;
  }
  for (int g = count; g < kMaxBatch; ++g) bt.g[g] = bt.g[count - 1];

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
                                   dim3(threads_of(t)), kargs, dyn_lds, stream);
  if (err == hipSuccess) err = hipGetLastError();
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return LOWM_ERR_LAUNCH;
  }
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
  return lowm::select_kernel(f32out != 0, M, K / split_k / lowm::kVecK, t, &dyn)
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
    case LOWM_ERR_INVALID_ARG: return "invalid argument (NULL operand, size <= 0, split_k < 1)";
    case LOWM_ERR_UNSUPPORTED:
      return "unsupported (M > 64, K not a multiple of 8*split_k, split_k > 256, misaligned "
             "pointer, or tactic not in this build)";
    case LOWM_ERR_WORKSPACE: return "split_k > 1 needs a workspace";
    case LOWM_ERR_LAUNCH: return "kernel launch failed (see lowm_last_hip_error)";
    default: return "unknown error code";
  }
}

int lowm_last_hip_error(void) { return lowm::g_last_hip_error; }

#ifdef LOWM_STRESS
// Stress build only: where, on whom and how long the kernels stall.  Applies
// to every later launch from any thread; not thread-safe.
int lowm_stress_configure(unsigned site_mask, int rank, int wave, int tile_mod, int tile_sel,
                          int step, unsigned delay_ns) {
  if (delay_ns > 1000000u) return LOWM_ERR_INVALID_ARG;  // at most 1 ms per stall
  lowm::g_stress.site_mask = site_mask;
  lowm::g_stress.rank = rank;
  lowm::g_stress.wave = wave;
  lowm::g_stress.tile_mod = tile_mod;
  lowm::g_stress.tile_sel = tile_sel;
  lowm::g_stress.step = step;
  lowm::g_stress.ticks = delay_ns / 10u;  // s_memrealtime: 100 MHz
  return LOWM_OK;
}

// Stress build only: record per-workgroup timestamps into `buf` (device
// memory, 8 uint64 per workgroup of the grid; NULL stops tracing).
int lowm_stress_trace(void* buf) {
  lowm::g_stress.trace = static_cast<uint64_t*>(buf);
  return LOWM_OK;
}
#endif

}  // extern "C"
