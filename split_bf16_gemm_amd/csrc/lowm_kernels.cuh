// lowm_kernels.cuh -- device code of the low-M split-K bf16 GEMM for AMD
// Instinct MI355X (gfx950): helpers, the split-K exchange, and the kernel
// templates.  Included by the per-output-kind translation units
// (lowm_inst_*.hip), each of which instantiates its kernels and fills its
// part of the kernel table.
//
//   C[m][n] = sum_k A[m][k] * W[n][k]        A [M,K], W [N,K] bf16, row-major
//
// The problem is the one the TensorRT-LLM PR "Fix two synchronization gaps in
// the MiniMax M3 low-M split-K GEMM" works on (Description; Hardware
// verification): a handful of activation rows against a large bf16 weight,
// K cut into split_k slices whose fp32 partials one owner adds.  The design
// here is gfx950's own:
//
//  * One workgroup = (output tile of BN weight rows) x (one K slice, "rank").
//    Its four wavefronts stream W once from HBM and feed bf16 MFMA 16x16x32
//    with W as the 16-column operand and the M activation rows, in blocks of
//    16, as the 16-row operand, accumulating fp32 in registers.  M <= 64 is
//    1..4 MFMA row blocks.
//  * Tile kinds (tactics):
//      LINE   W global -> LDS in whole 128-byte lines (non-temporal
//             direct-to-LDS loads) into a ring private to each wavefront;
//             the wavefronts split the K slice; activation operands straight
//             from memory into registers.  The default for M <= 4 with
//             split-K.
//      QUARTER each wavefront one quarter of the K slice for the whole tile,
//             weight and activation rows alike through its own LDS ring with
//             the same whole-line loads; the quarter sums are added in order
//             through LDS and each wavefront then owns 16 output columns.
//             The default without split-K and for 5..32 rows with it (as
//             the host's tactic rules state).
//      PANEL  64-row tiles, each wavefront owning 16 of them for the whole K
//             slice; W as in LINE, and the activation panel of each 64-K
//             step loaded once per workgroup into an LDS ring that all four
//             wavefronts read, refilled only after a workgroup barrier.
//             Each wavefront then owns its 16 output columns through the
//             exchange as well.  The default above 32 rows with split-K.
//      REG    W global -> a register ring per wavefront (any K slice).
//      LDS    W global -> an LDS ring of NS stages shared by the workgroup,
//             a stage refilled only after a workgroup barrier that every
//             wavefront reaches once its reads of it have completed: a
//             per-wavefront wait is not enough when the stage is shared
//             (Triton issue "warpgroup_mma_wait does not properly
//             synchronize across warpgroups"; cuLA PR "Fix SM90 WY input
//             buffer reuse before WGMMA completion").
//  * split_k > 1: every rank stores its fp32 partial in the workspace slots
//    and counts itself in the arrival counter of its columns with a relaxed
//    device-scope atomic.  The rank that sees split_k-1 earlier arrivals is
//    the owner: it reads the peers' slots, adds the partials in rank order
//    0..split_k-1 (its own from registers, at its own position), rounds once
//    to bf16 and returns the counter and the slots to zero.  A slot word
//    holds the complement of the partial's bits, so zero means "not
//    published": each slot is its own single-copy-atomic object, written
//    once per launch, and the owner re-reads any slot it still finds zero
//    (bounded) instead of relying on an ordering between the counter and the
//    slots.  Where split_k is 2..4 and a tile has at most 64 elements, the
//    grid is rank-major and the tile's last rank polls its peers' slots for a
//    bounded time instead of publishing.  Scope matters (PR, Description
//    item 2: a release and an acquire synchronize only when each one's scope
//    includes the other thread): every exchanged access is at device
//    ("agent") scope, the one that spans all XCDs.  No workgroup waits for
//    another without a bound.
//
// Built as liblowm.so; as liblowm_stress.so with -DLOWM_STRESS, which adds
// bounded s_sleep stalls at chosen sites, ranks, wavefronts and tiles (the
// stall-injection method of the PR's Hardware verification); and, when asked
// for, as liblowm_fenced.so with -DLOWM_FENCED, a comparison build whose
// exchange uses a release arrival and an acquire fence.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "lowm_types.h"

namespace lowm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
__device__ __forceinline__ bool stress_selected(const StressArgs& st, uint32_t site, int rank,
                                                int wave, int tile, int step) {
  if (!(st.site_mask & site)) return false;
  if (st.rank >= 0 && st.rank != rank) return false;
  if (st.wave >= 0 && st.wave != wave) return false;
  if (st.tile_mod > 1 && tile % st.tile_mod != st.tile_sel) return false;
  if (site == kSiteStageRead && st.step >= 0 && st.step != step) return false;
  return true;
}
__device__ __forceinline__ void maybe_stall(const StressArgs& st, uint32_t site, int rank,
                                            int wave, int tile, int step) {
  if (stress_selected(st, site, rank, wave, tile, step)) stall_ticks(st.ticks);
}
#define LOWM_STALL(site, step) maybe_stall(a.stress, (site), rank, wave, tile, (step))
#define LOWM_LATE_PUBLISH() stress_selected(a.stress, kSiteLatePublish, rank, wave, tile, 0)
#define LOWM_LATE_STALL() stall_ticks(a.stress.ticks)
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
      a.stress.trace[(size_t)blockIdx.x * kTraceSlots + kTraceTile] = (uint64_t)tile; \
      a.stress.trace[(size_t)blockIdx.x * kTraceSlots + kTraceRank] = (uint64_t)rank; \
    }                                                                                 \
  } while (0)
#else
#define LOWM_STALL(site, step) ((void)0)
#define LOWM_LATE_PUBLISH() false
#define LOWM_LATE_STALL() ((void)0)
#define LOWM_TRACE(slot) ((void)0)
#define LOWM_TRACE_IDS() ((void)0)
#endif

// The fenced build (-DLOWM_FENCED, a comparison build, never the default):
// the arrival is a release RMW and the owner issues an acquire fence before
// it reads its peers' partials, the textbook pairing at agent scope.  The
// default build needs neither (each slot is written once per launch and
// read until it is non-zero), and the compiler's agent-scope release and
// acquire write back and invalidate this XCD's whole L2.
#ifdef LOWM_FENCED
#define LOWM_ARRIVE_ORDER __ATOMIC_RELEASE
#define LOWM_OWNER_FENCE() __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent")
#else
#define LOWM_ARRIVE_ORDER __ATOMIC_RELAXED
#define LOWM_OWNER_FENCE() ((void)0)
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
// 24 wait states after the last MFMA that writes any of `acc`, before
// anything reads them.  Reading an MFMA result needs
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
  else if constexpr (N == 3)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]));
  else if constexpr (N == 4)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
  else {
    // in groups of four: each group's no-ops follow the MFMAs that write it
    mfma_settle(reinterpret_cast<f32x4(&)[4]>(acc[0]));
    mfma_settle(reinterpret_cast<f32x4(&)[N - 4]>(acc[4]));
  }
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
  else {
    // any count: the wait, then an empty asm per value that the value's uses
    // depend on (volatile asm statements keep their order)
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
  }
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

// The owner's fold.  For each of its NE elements e[j] (slot r of element e
// at slots[r * E + e]) the S rank partials are added in rank order
// 0..S-1, with this rank's own partial (v[j] on entry) at its own position;
// v[j] holds the sum on exit.  The peers' slots (peer i is rank i, or i+1
// past the owner) are all loaded before the first add, so the loads overlap;
// a load under a branch would be waited for inside it.  Loads only: the
// caller stores C and clears the slots after its folds, so that no wait for
// these loads also waits for stores.
//
// The arrival counter only says when to look.  What the owner adds is what
// each slot holds, and a slot is its own single-copy-atomic 32-bit object
// that is zero until its rank writes it, once, in this launch.  So any
// non-zero word read is that rank's partial, whatever order the memory
// system made the counter and the slots visible in.  A word still zero is
// re-read, with s_sleep between reads, for at most kFoldPollTicks of the
// 100 MHz clock; one that stays zero is added as it is (it decodes as a NaN,
// so C shows it) and the tile's fault word is set for the host to find.
__device__ __forceinline__ const uint32_t* peer_slot(const uint32_t* slots, size_t E, int e,
                                                     int rank, int i) {
  return slots + (size_t)(i < rank ? i : i + 1) * E + e;
}

// Re-reads, with s_sleep between rounds and for at most kFoldPollTicks, the
// words of w still zero; word k came from slot(base, k).  The base pointer
// passes through an empty asm each round, so the addresses are recomputed
// on this rare path instead of being kept live in registers for the whole
// kernel.  A word that stays zero sets the fault word.
template <int NW, typename Slot>
__device__ __forceinline__ void await_published(uint32_t (&w)[NW], const uint32_t* base,
                                                Slot slot, uint32_t* fault) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  bool zero = true;
  while (true) {
    __builtin_amdgcn_s_sleep(4);
    asm volatile("" : "+v"(base));
#pragma unroll
    for (int k = 0; k < NW; ++k)
      if (w[k] == 0u)
        w[k] = __hip_atomic_load(slot(base, k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    zero = false;
#pragma unroll
    for (int k = 0; k < NW; ++k) zero = zero || w[k] == 0u;
    if (!__any(zero)) return;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kFoldPollTicks) break;
  }
  if (zero) __hip_atomic_store(fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int SN, int NE>
__device__ __forceinline__ void fold_owner_n(const uint32_t* slots, size_t E, const int (&e)[NE],
                                             int rank, float (&v)[NE], uint32_t* fault) {
  constexpr int NW = NE * (SN - 1);
  auto slot = [&](const uint32_t* base, int k) {
    return peer_slot(base, E, e[k / (SN - 1)], rank, k % (SN - 1));
  };
  uint32_t w[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) w[k] = load_slot(slot(slots, k));
  bool zero = false;
#pragma unroll
  for (int k = 0; k < NW; ++k) zero = zero || w[k] == 0u;
  if (__builtin_expect(__any(zero), 0)) await_published(w, slots, slot, fault);
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    const uint32_t* wj = w + j * (SN - 1);
    float acc = (rank == 0) ? v[j] : dec_partial(wj[0]);
#pragma unroll
    for (int r = 1; r < SN; ++r)
      acc += (r == rank) ? v[j] : dec_partial(r < rank ? wj[r < SN - 1 ? r : 0] : wj[r - 1]);
    v[j] = acc;
  }
}

// Any other split_k: one element and one peer at a time (a slow path; the
// measured split_k choices are 2, 3, 4 and 8).
template <int NE>
__device__ __forceinline__ void fold_owner_any(const uint32_t* slots, size_t E,
                                               const int (&e)[NE], int S, int rank,
                                               float (&v)[NE], uint32_t* fault) {
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    float acc = 0.f;
    for (int r = 0; r < S; ++r) {
      float p = v[j];
      if (r != rank) {
        auto slot = [&](const uint32_t* base, int) { return base + (size_t)r * E + e[j]; };
        uint32_t w[1] = {load_slot(slot(slots, 0))};
        if (__any(w[0] == 0u)) await_published(w, slots, slot, fault);
        p = dec_partial(w[0]);
      }
      acc = (r == 0) ? p : acc + p;
    }
    v[j] = acc;
  }
}

template <int NE>
__device__ __forceinline__ void fold_owner(const uint32_t* slots, size_t E, const int (&e)[NE],
                                           int S, int rank, float (&v)[NE], uint32_t* fault) {
  switch (S) {
    case 2: fold_owner_n<2>(slots, E, e, rank, v, fault); break;
    case 3: fold_owner_n<3>(slots, E, e, rank, v, fault); break;
    case 4: fold_owner_n<4>(slots, E, e, rank, v, fault); break;
    case 8: fold_owner_n<8>(slots, E, e, rank, v, fault); break;
    default: fold_owner_any(slots, E, e, S, rank, v, fault); break;
  }
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
// XCD.  Where the last rank probes its peers (rank_major) the order is
// rank-major: the GEMM's first T8 workgroups are rank 0 of tiles 0..T8-1, the
// next T8 rank 1, and so on (T8 = tiles rounded up to a multiple of 8), so a
// tile's later ranks tend to end their streams after its earlier ones have
// published.  Elsewhere the ranks of a tile are dispatched 8 workgroups
// apart.
__device__ __forceinline__ void decode_tile(const Args& a, int BN, bool rank_major, int& tile,
                                            int& rank) {
  const int bid = (int)blockIdx.x - a.bid_base;
  if (rank_major) {
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

// Wait until at most min(younger, YMAX) groups of N vector-memory operations
// issued after the oldest outstanding group are still in flight (younger < 0
// counts as 0).
template <int N, int YMAX>
__device__ __forceinline__ void wait_younger(int younger) {
  static_assert(YMAX >= 0 && YMAX <= 7 && YMAX * N <= 63, "vmcnt is 6 bits");
  younger = younger < YMAX ? younger : YMAX;
  switch (younger) {
    case 7: if constexpr (YMAX >= 7) { wait_vmcnt<7 * N>(); break; } [[fallthrough]];
    case 6: if constexpr (YMAX >= 6) { wait_vmcnt<6 * N>(); break; } [[fallthrough]];
    case 5: if constexpr (YMAX >= 5) { wait_vmcnt<5 * N>(); break; } [[fallthrough]];
    case 4: if constexpr (YMAX >= 4) { wait_vmcnt<4 * N>(); break; } [[fallthrough]];
    case 3: if constexpr (YMAX >= 3) { wait_vmcnt<3 * N>(); break; } [[fallthrough]];
    case 2: if constexpr (YMAX >= 2) { wait_vmcnt<2 * N>(); break; } [[fallthrough]];
    case 1: if constexpr (YMAX >= 1) { wait_vmcnt<N>(); break; } [[fallthrough]];
    default: wait_vmcnt<0>(); break;
  }
}

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
    for (int i = 0; i < kProbeRanks; ++i)
      probe[i] = load_slot(probe_src(a, E, tile, lane, i, true));
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
  // every XCD reads), and the arrival follows at once, without waiting for
  // their acknowledgement: the owner does not rely on an order between the
  // count and the slots (a slot it still finds zero is re-read until this
  // rank's store lands), so the publisher pays one round trip, not two
  // (measured 0.1-0.3 us per call on the counter-path shapes, no change
  // elsewhere).
  const bool late = LOWM_LATE_PUBLISH();
  if (!late)
    for (int e = lane; e < E; e += kWave)
      store_slot(slots + (size_t)rank * E + e, enc_partial(rank_sum(e)));
  pin_issue();
  uint32_t before = 0;
  if (lane == 0)
    before = __hip_atomic_fetch_add(ctr, 1u, LOWM_ARRIVE_ORDER, __HIP_MEMORY_SCOPE_AGENT);
  before = __builtin_amdgcn_readfirstlane(before);
  LOWM_TRACE(kTraceArrived);
  if (late) {   // stress build only: the partial lands after the arrival
    if (before != (uint32_t)(a.S - 1)) LOWM_LATE_STALL();
    for (int e = lane; e < E; e += kWave)
      store_slot(slots + (size_t)rank * E + e, enc_partial(rank_sum(e)));
  }
  if (before != (uint32_t)(a.S - 1)) {   // not the last rank: done
    LOWM_TRACE(kTraceEnd);
    return;
  }

  // a5: the owner.  The peers' partials are read with device-scope loads;
  // a slot still zero is re-read (fold_owner).  The fold is in rank order
  // with this rank's partial, from LDS, at its own position; every slot read
  // goes back to zero.
  LOWM_STALL(kSiteFold, 0);
  LOWM_OWNER_FENCE();
  // Two passes: the folds (global loads only, four elements' loads in
  // flight at once; each result replaces the element's wavefront-0 sum in
  // LDS, which nothing else reads), then the stores of C and the clearing
  // of the slots, which nothing waits for.  Past the tile's end a lane folds
  // its first element again and keeps nothing.
  uint32_t* fault = ctr + kFaultWord;
  auto fold_pass = [&](auto sn_c) {
    constexpr int SN = decltype(sn_c)::value;
    for (int e0 = lane; e0 < E; e0 += 4 * kWave) {
      int e[4];
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        e[u] = e0 + u * kWave < E ? e0 + u * kWave : e0;
        v[u] = rank_sum(e[u]);
      }
      if constexpr (SN > 0) fold_owner_n<SN>(slots, E, e, rank, v, fault);
      else fold_owner_any(slots, E, e, a.S, rank, v, fault);
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
  decode_tile(a, BN, early_probe(a, BN), tile, rank);
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
  auto phys = [&](int u) {
    return u < nunits ? (u + rot < nunits ? u + rot : u + rot - nunits) : -1;
  };
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
  decode_tile(a, BN, early_probe(a, BN), tile, rank);
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
      for (int rg = 0; rg < RG; ++rg)
        wv[c * RG + rg] = lds_read_opaque(slot + rg * 2 * kPP + rpos[c]);
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
// Panel tiles (M > 16): a workgroup's tile is 64 weight rows, 16 per
// wavefront, and every wavefront walks the rank's whole K slice in steps of
// 64 K.  With 17..64 activation rows the activation operand of a step
// (16*MB rows x 64 K) outweighs the weight operand of one wavefront (16 rows
// x 64 K), so it is loaded once per workgroup, as 2*MB whole-line pieces of
// 8 rows x 128 B spread over the wavefronts, into an LDS ring that all four
// wavefronts read (the activation "panel").  The weight rows stream as in
// the line-pair tiles: whole-line non-temporal direct-to-LDS loads into a
// slot only this wavefront reads.  Ring slot s holds step p = s (mod R) of
// both.  (Measured on MI355X and not adopted: the weights straight into a
// register ring in the MFMA operand layout, and 32 columns per wavefront;
// both were slower at every M 32 / M 64 sweep shape.)
//
// Step p: each wavefront waits for its own loads of step p (vmcnt), then a
// workgroup barrier makes every wavefront's panel pieces of step p visible
// to all and guarantees that every wavefront has completed its reads of
// step p-1 (each waits for its LDS reads before it multiplies), so the slot
// step p-1 used is refilled with step p+R-1 right after the barrier.  A
// stage is never refilled before all of its readers are done (the lesson of
// the Triton issue "warpgroup_mma_wait does not properly synchronize across
// warpgroups" and of the cuLA PR "Fix SM90 WY input buffer reuse before
// WGMMA completion").  No load is issued past the end of the slice, so the
// ring drains in the last R-2 steps and no load is in flight at the end.
//
// Each wavefront owns its 16 output columns to the end: no wavefront
// reduction, and with split_k > 1 it publishes, arrives and (as the owner)
// folds its 16-column strip, with the counter of that strip.
// ---------------------------------------------------------------------------
template <int MB, int R, int KW>
struct PanelShape {
  static constexpr int WN = kWaves / KW;               // wavefronts along N (16 columns each)
  static constexpr int BN = 16 * WN;                    // weight rows per workgroup tile
  static constexpr int kPP = 68;                        // u32x4 per 8-row piece (1088 B)
  static constexpr int w_slot = 2 * kPP;                // one wavefront's weight step
  static constexpr int a_half = 2 * MB * kPP;           // the activation panel of one K part
  static constexpr int a_slot = KW * a_half;            // ... of a step (all KW parts)
  static constexpr int slot_elems = kWaves * w_slot + a_slot;
  static constexpr int a_pieces = KW * 2 * MB;          // panel pieces per step
  static constexpr int a_loads = (a_pieces + kWaves - 1) / kWaves;   // ... per wavefront
  static constexpr int step_loads = 2 + a_loads;        // vector-memory ops per step per wavefront
  static constexpr int lds_bytes = R * slot_elems * 16;
  static constexpr int red_floats = (KW - 1) * WN * MB * 4 * kWave;   // K-part reduction
  static constexpr bool valid = MB >= 2 && MB <= 4 && R >= 3 && R <= 8 && (KW == 1 || KW == 2) &&
                                (R - 1) * step_loads <= 63 && lds_bytes <= 128 * 1024 &&
                                red_floats * 4 <= lds_bytes;
};

template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<0>) .. f(integral_constant<N-1>), in order
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// The epilogue of one wavefront that holds the whole K-slice sums of a
// 16-column strip (columns nw .. nw+15) for every activation row: block b,
// register i of `acc` is C[16b + 4g + i][nw + l16] at lane (g, l16).
// split_k 1 stores C; otherwise the strip is published to its slots and
// folded by the last of its ranks to arrive, through the strip's own counter.
template <int MB, typename OutT>
__device__ __forceinline__ void strip_epilogue(const Args& a, f32x4 (&acc)[MB], int nw, int rank,
                                               int tile, int wave, int lane) {
  (void)tile;
  (void)wave;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  if (nw >= a.N) return;               // this wavefront's columns lie past the end of C
  // This lane's sums: block b, register i is C[16b + 4g + i][nw + l16].
  const int n = nw + l16;
  if (a.S == 1) {
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * b + 4 * g + i;
        if (m < a.M && n < a.N) store_out<OutT>(a, m, n, acc[b][i]);
      }
    publish_flags<1, OutT>(a, nw, lane);
    LOWM_TRACE(kTraceEnd);
    return;
  }

  // a4: publish this wavefront's partial strip (element (m, c) at word
  // 16m + c of the rank's slot), then arrive on the strip's counter.
  const int strip = nw >> 4;
  const int E = a.M * 16;
  uint32_t* slots = a.part + (size_t)strip * a.S * E;
  uint32_t* ctr = a.ctr + (size_t)strip * kCtrStride;
  LOWM_STALL(kSitePublish, 0);
  auto publish = [&] {
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * b + 4 * g + i;
        if (m < a.M) store_slot(slots + (size_t)rank * E + 16 * m + l16, enc_partial(acc[b][i]));
      }
  };
  const bool late = LOWM_LATE_PUBLISH();
  if (!late) publish();
  pin_issue();           // arrive at once: the owner re-reads any slot still zero
  uint32_t before = 0;
  if (lane == 0)
    before = __hip_atomic_fetch_add(ctr, 1u, LOWM_ARRIVE_ORDER, __HIP_MEMORY_SCOPE_AGENT);
  before = __builtin_amdgcn_readfirstlane(before);
  LOWM_TRACE(kTraceArrived);
  if (late) {   // stress build only: the partial lands after the arrival
    if (before != (uint32_t)(a.S - 1)) LOWM_LATE_STALL();
    publish();
  }
  if (before != (uint32_t)(a.S - 1)) {
    LOWM_TRACE(kTraceEnd);
    return;
  }

  // a5/a6: the owner folds its strip in rank order (its own partial from
  // registers), stores C and returns every slot and the counter to zero.
  // The peers' slots of BPC blocks of 4 rows per lane are loaded at once
  // (all blocks for split_k 2..4, one at a time above: two at split_k 8
  // measured 0.2-0.4 us slower), so the fold waits for one round trip per
  // group, not per block.  Rows >= M fold row 0
  // again and keep nothing.
  LOWM_STALL(kSiteFold, 0);
  LOWM_OWNER_FENCE();
  uint32_t* fault = ctr + kFaultWord;
  float out[MB][4];
  auto fold_blocks = [&](auto sn_c, auto bpc_c, int b0) {
    constexpr int SN = decltype(sn_c)::value;
    constexpr int BPC = decltype(bpc_c)::value;
    int e[4 * BPC];
    float v[4 * BPC];
#pragma unroll
    for (int j = 0; j < BPC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * (b0 + j) + 4 * g + i;
        e[4 * j + i] = 16 * (m < a.M ? m : 0) + l16;
        v[4 * j + i] = acc[b0 + j][i];
      }
    if constexpr (SN > 0) fold_owner_n<SN>(slots, E, e, rank, v, fault);
    else fold_owner_any(slots, E, e, a.S, rank, v, fault);
#pragma unroll
    for (int j = 0; j < BPC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[b0 + j][i] = v[4 * j + i];
  };
  auto fold_all = [&](auto sn_c) {
    constexpr int SN = decltype(sn_c)::value;
    constexpr int BPC0 = (SN == 2 || SN == 3 || SN == 4) ? MB : 1;
    constexpr int BPC = BPC0 < MB ? BPC0 : MB;
#pragma unroll
    for (int b0 = 0; b0 + BPC <= MB; b0 += BPC)
      fold_blocks(sn_c, std::integral_constant<int, BPC>{}, b0);
    if constexpr (MB % BPC != 0)
      fold_blocks(sn_c, std::integral_constant<int, MB % BPC>{}, MB - MB % BPC);
  };
  switch (a.S) {
    case 2: fold_all(std::integral_constant<int, 2>{}); break;
    case 3: fold_all(std::integral_constant<int, 3>{}); break;
    case 4: fold_all(std::integral_constant<int, 4>{}); break;
    case 8: fold_all(std::integral_constant<int, 8>{}); break;
    default: fold_all(std::integral_constant<int, 0>{}); break;
  }
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * b + 4 * g + i;
      if (m >= a.M) continue;
      if (n < a.N) store_out<OutT>(a, m, n, out[b][i]);
      clear_slots(slots, E, 16 * m + l16, a.S);
    }
  publish_flags<1, OutT>(a, nw, lane);
  if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  LOWM_TRACE(kTraceEnd);
}

template <int MB, int R, int KW, typename OutT>
__device__ __forceinline__ void panel_tile_body(const Args& a, u32x4* __restrict__ ring) {
  using SH = PanelShape<MB, R, KW>;
  constexpr int BN = SH::BN;
  constexpr int kPP = SH::kPP;
  constexpr int kSlot = SH::slot_elems;
  constexpr int G = SH::step_loads;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;
  const int l16 = lane & 15;

  int tile, rank;
  decode_tile(a, BN, false, tile, rank);
  LOWM_TRACE(kTraceEntry);
  LOWM_TRACE_IDS();
  if (tile * BN >= a.N) return;        // a whole workgroup past the end (grid padding)
  // Wavefront (wn, kh): 16 columns wn of the tile, K part kh of the slice
  // (KW 2: the slice's two halves, added in order after the main loop).
  const int wn = wave % SH::WN, kh = wave / SH::WN;
  const int n0 = tile * BN;
  const int nw = n0 + 16 * wn;         // this wavefront's first column
  const int nvec = a.nvec;
  const int P = nvec / (8 * KW);       // steps per K part; the launch requires nvec % (8*KW) == 0
  const size_t kr = (size_t)rank * nvec * kVecK;   // the rank's slice
  const size_t kpart = (size_t)P * 64;             // elements per K part

  // Line loads: lane 8q + j fetches 16-byte piece (j - q/2) mod 8 of row q of
  // an 8-row piece and lands at position j of that row in LDS, so that the
  // MFMA-layout reads (16 rows at one K offset) fall in distinct banks.
  const int qr = lane >> 3;
  const int piece = ((lane & 7) - (qr >> 1)) & 7;
  // Weight sources: row 8i + qr of this wavefront's 16, rotated piece.
  const uint16_t* wsrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int n = nw + 8 * i + qr;
    n = n < a.N ? n : a.N - 1;
    wsrc[i] = a.W + (size_t)n * a.K + kr + kh * kpart + piece * kVecK;
  }
  // This wavefront's panel pieces: j = wave + 4t (clamped: with MB 3 the
  // last piece is loaded by more than one wavefront, with identical data,
  // and every copy lands before the barrier that publishes the stage).
  // Piece j is K part j / (2*MB), activation rows 8*(j % (2*MB)) .. +7; rows
  // >= M read row M-1: MFMA output rows are independent and rows >= M are
  // never stored.
  const uint16_t* asrc[SH::a_loads];
  int apos[SH::a_loads];
#pragma unroll
  for (int t = 0; t < SH::a_loads; ++t) {
    int j = wave + kWaves * t;
    j = j < SH::a_pieces ? j : SH::a_pieces - 1;
    const int jk = j / (2 * MB), jj = j - jk * (2 * MB);
    int m = 8 * jj + qr;
    m = m < a.M ? m : a.M - 1;
    asrc[t] = a.A + (size_t)m * a.K + kr + jk * kpart + piece * kVecK;
    apos[t] = kWaves * SH::w_slot + j * kPP;
  }
  // MFMA-layout read offsets within a pair of 8-row pieces: row l16, piece 4c+g.
  int rpos[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    rpos[c] = (l16 >> 3) * kPP + (l16 & 7) * 8 + ((4 * c + g + ((l16 & 7) >> 1)) & 7);

  f32x4 acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto slot_ptr = [&](int sl) -> u32x4* { return ring + sl * kSlot; };
  // Step p's loads into slot SL: this wavefront's two weight pieces, then
  // its share of the panel.
  auto issue = [&](auto slot_c, int p) {
    constexpr int SL = decltype(slot_c)::value;
    u32x4* slot = slot_ptr(SL);
    const size_t off = (size_t)p * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(
          wsrc[i] + off,
          (__attribute__((address_space(3))) void*)(slot + wave * SH::w_slot + i * kPP), 16, 0,
          kStreamAux);
#pragma unroll
    for (int t = 0; t < SH::a_loads; ++t)
      __builtin_amdgcn_global_load_lds(asrc[t] + off,
                                       (__attribute__((address_space(3))) void*)(slot + apos[t]),
                                       16, 0, 0);
    pin_issue();
  };
  // Step p out of slot SL (= p mod R).  YOUNGER: how many later steps'
  // loads may still be in flight once step p's have landed; REFILL: whether
  // step p+R-1 exists (both compile-time, so that every wait count is a
  // constant and the compiler adds none of its own).
  auto step = [&](auto slot_c, auto younger_c, auto refill_c, int p) {
    constexpr int SL = decltype(slot_c)::value;
    // this wavefront's loads of step p have landed ...
    wait_vmcnt<decltype(younger_c)::value * G>();
    // ... and after the barrier every wavefront's have, and every wavefront
    // has finished reading step p-1's slot
    barrier_keep_loads();
    LOWM_STALL(kSiteStageRead, p);
    if (p == 0) LOWM_TRACE(kTraceFirstStage);
    if constexpr (decltype(refill_c)::value)
      issue(std::integral_constant<int, (SL + R - 1) % R>{}, p + R - 1);
    const u32x4* slot = slot_ptr(SL);
    u32x4 v[2 + 2 * MB];                    // weight chunks 0, 1, then panel (c, b)
#pragma unroll
    for (int c = 0; c < 2; ++c) v[c] = lds_read_opaque(slot + wave * SH::w_slot + rpos[c]);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < MB; ++b)
        v[2 + c * MB + b] =
            lds_read_opaque(slot + kWaves * SH::w_slot + kh * SH::a_half + 2 * b * kPP + rpos[c]);
    lds_wait(v);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[b] = mfma(v[2 + c * MB + b], v[c], acc[b]);
  };

  LOWM_STALL(kSiteEntry, 0);
  // Steady state: whole ring cycles of R steps in which every step refills
  // the slot its predecessor read, so R-1 steps are always in flight and
  // every wait count is the same constant.  The first cycle runs before the
  // loop, after an unconditional prologue of R-1 steps, and the last
  // REM = P - p0 steps (R-1 .. 2R-2) run as straight-line code, one sequence
  // per REM: every issue is then unconditional where it happens.
  using T = std::true_type;
  auto cycle = [&](int p0) {
    static_for<R>([&](auto s_c) {
      step(s_c, std::integral_constant<int, R - 2>{}, T{}, p0 + decltype(s_c)::value);
    });
  };
  auto tail = [&](auto rem_c, int p0) {
    constexpr int REM = decltype(rem_c)::value;
    static_for<REM>([&](auto i_c) {
      constexpr int I = decltype(i_c)::value;
      constexpr int YOUNGER = (REM - 1 - I) < (R - 2) ? (REM - 1 - I) : (R - 2);
      step(std::integral_constant<int, I % R>{},
           std::integral_constant<int, YOUNGER>{},
           std::integral_constant<bool, (I + R - 1 < REM)>{}, p0 + I);
    });
  };
  int p0 = 0;
  if (P >= 2 * R - 1) {
    static_for<R - 1>([&](auto s_c) { issue(s_c, decltype(s_c)::value); });
    cycle(0);
    for (p0 = R; p0 + 2 * R - 1 <= P; p0 += R) cycle(p0);
  } else {
    // fewer steps than a prologue plus a cycle: issue what exists
    static_for<R - 1>([&](auto s_c) {
      if (decltype(s_c)::value < P) issue(s_c, decltype(s_c)::value);
    });
  }
  // p0 is a multiple of R, so the tail's slots start at 0
  static_assert(2 * R - 2 <= 14, "the tail covers at most 14 steps");
  switch (P - p0) {
#define LOWM_PANEL_TAIL(n) \
    case n: if constexpr (n <= 2 * R - 2) tail(std::integral_constant<int, n>{}, p0); break;
    LOWM_PANEL_TAIL(1) LOWM_PANEL_TAIL(2) LOWM_PANEL_TAIL(3) LOWM_PANEL_TAIL(4)
    LOWM_PANEL_TAIL(5) LOWM_PANEL_TAIL(6) LOWM_PANEL_TAIL(7) LOWM_PANEL_TAIL(8)
    LOWM_PANEL_TAIL(9) LOWM_PANEL_TAIL(10) LOWM_PANEL_TAIL(11) LOWM_PANEL_TAIL(12)
    LOWM_PANEL_TAIL(13) LOWM_PANEL_TAIL(14)
#undef LOWM_PANEL_TAIL
    default: break;
  }
  mfma_settle(acc);
  LOWM_TRACE(kTraceLoopEnd);
  if constexpr (KW == 2) {
    // The two K halves of each strip: the second half's sums go through LDS
    // (the ring, which every wavefront has finished reading once all reach
    // the barrier) and are added to the first's, in that order; the first
    // half's wavefront carries on alone.
    float* red = reinterpret_cast<float*>(ring);
    auto red_at = [&](int b, int i) -> float& {
      return red[((wn * MB + b) * 4 + i) * kWave + lane];
    };
    barrier_keep_loads();
    if (kh == 1) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_at(b, i) = acc[b][i];
    }
    wait_lgkmcnt0();
    barrier_keep_loads();
    if (kh == 1) return;
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b][i] = acc[b][i] + red_at(b, i);
    LOWM_TRACE(kTraceReduced);
  }

  strip_epilogue<MB, OutT>(a, acc, nw, rank, tile, wave, lane);
}

template <int MB, int R, int KW, typename OutT>
__global__ __launch_bounds__(kThreads) void lowm_panel_kernel(Args a0, Batch bt) {
#if defined(__HIP_DEVICE_COMPILE__)
  const Args a = gemm_args(a0, bt);
  __shared__ u32x4 ring[R * PanelShape<MB, R, KW>::slot_elems];
  panel_tile_body<MB, R, KW, OutT>(a, ring);
#endif
}

// ---------------------------------------------------------------------------
// Quarter tiles: the four wavefronts split the rank's K slice into four
// contiguous quarters, and each streams, for its quarter, both operands of
// the whole tile (16*NB weight rows and the M activation rows) through a
// ring of R slots of its own, one 64-K step per slot, with whole-line
// direct-to-LDS loads (8 rows x 128 B each, rotated as in the line-pair
// tiles so that the MFMA-layout reads of 16 rows fall in distinct banks).
// No workgroup barrier in the main loop; every operand byte is written to
// and read from LDS once (the panel tiles read each activation byte once per
// wavefront).  After the loop the four quarter sums of each 16-column strip
// are added in wavefront (K) order through LDS by the strip's wavefront,
// whose strip epilogue stores or exchanges it.
// ---------------------------------------------------------------------------
template <int MB, int NB, int R>
struct QuarterShape {
  static constexpr int BN = 16 * NB;             // weight rows per workgroup tile
  static constexpr int kPP = 68;                 // u32x4 per 8-row piece (1088 B)
  static constexpr int G = 2 * (NB + MB);        // 8-row pieces (loads) per step
  static constexpr int slot_elems = G * kPP;     // one wavefront's step
  static constexpr int lds_bytes = kWaves * R * slot_elems * 16;
  static constexpr int red_floats = kWaves * NB * MB * 4 * kWave;
  static constexpr bool valid = MB >= 1 && MB <= 4 && NB >= 1 && NB <= 4 &&
                                R >= 2 && R <= 8 && (R - 1) * G <= 63 &&
                                lds_bytes <= 160 * 1024 && red_floats * 4 <= lds_bytes;
};

template <int MB, int NB, int R, typename OutT>
__device__ __forceinline__ void quarter_tile_body(const Args& a0, u32x4* __restrict__ lds) {
  using SH = QuarterShape<MB, NB, R>;
  constexpr int BN = SH::BN;
  constexpr int G = SH::G;
  constexpr int kPP = SH::kPP;
  constexpr int kSlot = SH::slot_elems;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;
  const int l16 = lane & 15;

  // A launch whose M exceeds the 16*MB rows of the kernel (the quarter-rows
  // tiles, split_k 1) gives each tile H workgroups, one per block of 16*MB
  // activation rows; block h is decoded as one more rank of the tile, so the
  // blocks of a tile share an XCD and the later ones find its W rows in the
  // L2.  Each block is then a GEMM of its own rows: A and C start at row
  // 16*MB*h.  With H = 1 (every other launch) nothing changes.
  const int H = (a0.M + 16 * MB - 1) / (16 * MB);
  int tile, rank;
  {
    Args d = a0;
    d.S = a0.S * H;
    decode_tile(d, BN, false, tile, rank);
  }
  const int h = rank / a0.S;
  rank -= h * a0.S;
  Args a = a0;
  if (H > 1) {
    const int m0 = 16 * MB * h;
    a.A = a0.A + (size_t)m0 * a0.K;
    a.C = static_cast<typename OutStore<OutT>::type*>(a0.C) + (size_t)m0 * a0.N;
    a.M = a0.M - m0 < 16 * MB ? a0.M - m0 : 16 * MB;
  }
  LOWM_TRACE(kTraceEntry);
  LOWM_TRACE_IDS();
  if (tile * BN >= a.N) return;        // a whole workgroup past the end (grid padding)
  const int n0 = tile * BN;
  // Steps per quarter; the launch requires nvec % 32 == 0 (whole steps).
  const int P = a.nvec / 32;
  const size_t k0 = (size_t)rank * a.nvec * kVecK + (size_t)wave * P * 64;
  u32x4* ring = lds + wave * R * kSlot;

  // Piece t of a step: 8 rows x 128 B, weight rows n0 + 8t .. for t < 2*NB,
  // then activation rows 8(t - 2*NB) ..; lane 8q + j fetches 16-byte piece
  // (j - q/2) mod 8 of row q, which lands at position j of that row.  Rows
  // past the end read the last row: MFMA rows and columns are independent,
  // and results outside C are never stored.
  const int qr = lane >> 3;
  const int piece = ((lane & 7) - (qr >> 1)) & 7;
  const uint16_t* src[G];
#pragma unroll
  for (int t = 0; t < G; ++t) {
    if (t < 2 * NB) {
      int n = n0 + 8 * t + qr;
      n = n < a.N ? n : a.N - 1;
      src[t] = a.W + (size_t)n * a.K + k0 + piece * kVecK;
    } else {
      int m = 8 * (t - 2 * NB) + qr;
      m = m < a.M ? m : a.M - 1;
      src[t] = a.A + (size_t)m * a.K + k0 + piece * kVecK;
    }
  }
  // MFMA-layout read offsets within a 16-row block: row l16, piece 4c+g.
  int rpos[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    rpos[c] = (l16 >> 3) * kPP + (l16 & 7) * 8 + ((4 * c + g + ((l16 & 7) >> 1)) & 7);

  f32x4 acc[NB * MB];                  // [j][b]: column block j, row block b
#pragma unroll
  for (int i = 0; i < NB * MB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](auto slot_c, int p) {
    constexpr int SL = decltype(slot_c)::value;
    u32x4* slot = ring + SL * kSlot;
    const size_t off = (size_t)p * 64;
    static_for<G>([&](auto t_c) {
      constexpr int t = decltype(t_c)::value;
      __builtin_amdgcn_global_load_lds(src[t] + off,
                                       (__attribute__((address_space(3))) void*)(slot + t * kPP),
                                       16, 0, t < 2 * NB ? kStreamAux : 0);
    });
    pin_issue();
  };
  // Step p out of slot SL (= p mod R).  YOUNGER: how many later steps' loads
  // may still be in flight once step p's have landed; REFILL: whether step
  // p+R-1 exists; it goes into the slot step p-1 read, whose reads completed
  // before its MFMAs (both compile-time, so every wait count is a constant).
  auto step = [&](auto slot_c, auto younger_c, auto refill_c, int p) {
    constexpr int SL = decltype(slot_c)::value;
    wait_vmcnt<decltype(younger_c)::value * G>();
    LOWM_STALL(kSiteStageRead, p);
    if (p == 0) LOWM_TRACE(kTraceFirstStage);
    if constexpr (decltype(refill_c)::value)
      issue(std::integral_constant<int, (SL + R - 1) % R>{}, p + R - 1);
    const u32x4* slot = ring + SL * kSlot;
    u32x4 v[2 * (NB + MB)];            // chunk c: weight blocks, then activation blocks
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < NB + MB; ++t)
        v[c * (NB + MB) + t] = lds_read_opaque(slot + 2 * t * kPP + rpos[c]);
    lds_wait(v);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
          acc[j * MB + b] =
              mfma(v[c * (NB + MB) + NB + b], v[c * (NB + MB) + j], acc[j * MB + b]);
  };

  LOWM_STALL(kSiteEntry, 0);
  using T = std::true_type;
  auto cycle = [&](int p0) {
    static_for<R>([&](auto s_c) {
      step(s_c, std::integral_constant<int, R - 2>{}, T{}, p0 + decltype(s_c)::value);
    });
  };
  auto tail = [&](auto rem_c, int p0) {
    constexpr int REM = decltype(rem_c)::value;
    static_for<REM>([&](auto i_c) {
      constexpr int I = decltype(i_c)::value;
      constexpr int YOUNGER = (REM - 1 - I) < (R - 2) ? (REM - 1 - I) : (R - 2);
      step(std::integral_constant<int, I % R>{}, std::integral_constant<int, YOUNGER>{},
           std::integral_constant<bool, (I + R - 1 < REM)>{}, p0 + I);
    });
  };
  int p0 = 0;
  if (P >= 2 * R - 1) {
    static_for<R - 1>([&](auto s_c) { issue(s_c, decltype(s_c)::value); });
    cycle(0);
    for (p0 = R; p0 + 2 * R - 1 <= P; p0 += R) cycle(p0);
  } else {
    static_for<R - 1>([&](auto s_c) {
      if (decltype(s_c)::value < P) issue(s_c, decltype(s_c)::value);
    });
  }
  static_assert(2 * R - 2 <= 14, "the tail covers at most 14 steps");
  switch (P - p0) {
#define LOWM_QUARTER_TAIL(n) \
    case n: if constexpr (n <= 2 * R - 2) tail(std::integral_constant<int, n>{}, p0); break;
    LOWM_QUARTER_TAIL(1) LOWM_QUARTER_TAIL(2) LOWM_QUARTER_TAIL(3) LOWM_QUARTER_TAIL(4)
    LOWM_QUARTER_TAIL(5) LOWM_QUARTER_TAIL(6) LOWM_QUARTER_TAIL(7) LOWM_QUARTER_TAIL(8)
    LOWM_QUARTER_TAIL(9) LOWM_QUARTER_TAIL(10) LOWM_QUARTER_TAIL(11) LOWM_QUARTER_TAIL(12)
    LOWM_QUARTER_TAIL(13) LOWM_QUARTER_TAIL(14)
#undef LOWM_QUARTER_TAIL
    default: break;
  }
  mfma_settle(acc);
  LOWM_TRACE(kTraceLoopEnd);

  // The quarter sums through LDS (the rings, once every wavefront is done
  // with its own): wavefront w's block (j, b), register i at
  // red[(((w * NB + j) * MB + b) * 4 + i) * 64 + lane]; strip j's wavefront
  // adds the four quarters in order 0..3.
  float* red = reinterpret_cast<float*>(lds);
  __syncthreads();
  LOWM_STALL(kSiteReduce, 0);
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(((wave * NB + j) * MB + b) * 4 + i) * kWave + lane] = acc[j * MB + b][i];
  __syncthreads();
  if (wave >= NB) return;
  f32x4 sum[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = red[((wave * MB + b) * 4 + i) * kWave + lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w)
        v += red[(((w * NB + wave) * MB + b) * 4 + i) * kWave + lane];
      sum[b][i] = v;
    }
  LOWM_TRACE(kTraceReduced);
  strip_epilogue<MB, OutT>(a, sum, n0 + 16 * wave, rank, tile, wave, lane);
}

template <int MB, int NB, int R, typename OutT>
__global__ __launch_bounds__(kThreads) void lowm_quarter_kernel(Args a0, Batch bt) {
#if defined(__HIP_DEVICE_COMPILE__)
  const Args a = gemm_args(a0, bt);
  __shared__ u32x4 lds[kWaves * R * QuarterShape<MB, NB, R>::slot_elems];
  quarter_tile_body<MB, NB, R, OutT>(a, lds);
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
// Instantiation: the kernel of (MB, RG, variant VI, activation mode ACT,
// output kind OutT), or nullptr where the build provides none.
// ---------------------------------------------------------------------------
template <int MB, int RG, int VI, int ACT, typename OutT>
KernelFn kernel_for() {
  constexpr Variant v = kVariants[VI];
  if constexpr (v.stage == kStageLine) {
    // no staged activation slice: instantiated for act 0 only
    if constexpr (ACT == 0 && LineShape<MB, RG, v.stages>::valid)
      return lowm_line_kernel<MB, RG, v.stages, OutT>;
    else
      return nullptr;
  } else if constexpr (v.stage == kStagePanel) {
    // 64-row tiles (16 rows per wavefront, each the whole K slice) or 32-row
    // tiles (16 rows per pair of wavefronts, each half the K slice);
    // activation panel in LDS
    constexpr int KW = RG == 4 ? 1 : 2;
    if constexpr (ACT == 0 && (RG == 4 || RG == 2) && PanelShape<MB, v.stages, KW>::valid)
      return lowm_panel_kernel<MB, v.stages, KW, OutT>;
    else
      return nullptr;
  } else if constexpr (v.stage == kStageQuarter) {
    // 16 * RG weight rows per tile, the K slice in quarters per wavefront;
    // no staged activation slice
    if constexpr (ACT == 0 && QuarterShape<MB, RG, v.stages>::valid)
      return lowm_quarter_kernel<MB, RG, v.stages, OutT>;
    else
      return nullptr;
  } else if constexpr (RG <= 2 && Shape<MB, RG, v.stage, v.unroll, v.stages, ACT>::valid) {
    return lowm_splitk_kernel<MB, RG, v.stage, v.unroll, v.stages, ACT, OutT>;
  } else {
    return nullptr;
  }
}

template <int MB, int RG, int ACT, typename OutT, int... VI>
void fill_row(KernelFn* row, std::integer_sequence<int, VI...>) {
  ((row[VI] = kernel_for<MB, RG, VI, ACT, OutT>()), ...);
}
template <typename OutT, int MB, int RG>
void fill_one(Table& t, int out) {
  constexpr int ri = rg_index(RG);
  constexpr auto vis = std::make_integer_sequence<int, kNumVariants>{};
  fill_row<MB, RG, 0, OutT>(t.fn[out][0][MB - 1][ri], vis);
  fill_row<MB, RG, 1, OutT>(t.fn[out][1][MB - 1][ri], vis);
}
template <typename OutT, int MB>
void fill_mb(Table& t, int out) {
  fill_one<OutT, MB, 1>(t, out);
  fill_one<OutT, MB, 2>(t, out);
  fill_one<OutT, MB, 3>(t, out);
  fill_one<OutT, MB, 4>(t, out);
}
// Every kernel of output kind OutT into row `out` of the table.
template <typename OutT>
void fill_out(Table& t, int out) {
  fill_mb<OutT, 1>(t, out);
  fill_mb<OutT, 2>(t, out);
  fill_mb<OutT, 3>(t, out);
  fill_mb<OutT, 4>(t, out);
}

}  // namespace lowm
