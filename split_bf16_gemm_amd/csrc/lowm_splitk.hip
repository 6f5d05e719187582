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
//    earlier arrivals is the owner: one acquire fence, then it adds the
//    partials in rank order 0..split_k-1 (its own from registers, at its own
//    position), rounds once to bf16 and resets the counter.  Scope matters
//    (PR, Description item 2: a release and an acquire synchronize only when
//    each one's scope includes the other thread); the acquire is issued once,
//    on the owner's path only, never in a polling loop (PR, Description item
//    2, on the cost of an acquiring wait).  No workgroup waits for another.
//
// Built twice from this source: liblowm.so, and liblowm_stress.so with
// -DLOWM_STRESS, which adds bounded s_sleep stalls at chosen sites, ranks,
// wavefronts and tiles (the stall-injection method of the PR's Hardware
// verification).

#include <hip/hip_runtime.h>

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
constexpr int kChunkK = 32;      // K of one MFMA 16x16x32
constexpr int kVecK = 8;         // bf16 per 16-byte vector
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dealt round-robin

enum Stage : int { kStageLds = LOWM_STAGE_LDS, kStageReg = LOWM_STAGE_REG };

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
};

struct Args {
  const uint16_t* A;
  const uint16_t* W;
  void* C;
  uint32_t* ctr;          // [tiles] arrival counters
  float* part;            // [tiles][S][M*BN] fp32 partials
  int M, N, K, S;
  int nvec;               // 16-byte vectors per rank slice: K / S / 8
  int nchunks;            // MFMA chunks per rank slice: ceil(nvec / 4)
  int nsteps;             // pipeline steps per rank slice
  int tiles;              // ceil(N / BN)
  StressArgs stress;
};

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
#else
#define LOWM_STALL(site, step) ((void)0)
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

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <typename OutT>
__device__ __forceinline__ OutT to_out(float v);
template <>
__device__ __forceinline__ float to_out<float>(float v) { return v; }
template <>
__device__ __forceinline__ __bf16 to_out<__bf16>(float v) {
  return static_cast<__bf16>(v);  // v_cvt_pk_bf16_f32: round to nearest even
}

// Register/LDS budget of a tactic.  Kept in one place so the host picker and
// the instantiation filter agree.
template <int MB, int RG, int STAGE, int U, int NS>
struct Shape {
  static constexpr int BN = 16 * RG;
  static constexpr int WU = kWaves * U;                 // chunks per step
  static constexpr int slot_elems = WU * RG * kWave;    // u32x4 per LDS stage
  static constexpr int group_loads = U * (RG + MB);     // vmem ops per group
  static constexpr int lds_bytes = (STAGE == kStageLds ? NS * slot_elems * 16 : 0) +
                                   kWaves * RG * MB * 4 * kWave * 4;
  static constexpr int stage_vgprs =
      NS * U * 4 * (MB + (STAGE == kStageReg ? RG : 0));
  static constexpr bool valid =
      lds_bytes <= 160 * 1024 && stage_vgprs <= 224 &&
      (STAGE == kStageReg || (NS - 2) * group_loads <= 63) && NS >= 2 && NS <= 4;
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int MB, int RG, int STAGE, int U, int NS, typename OutT>
__device__ __forceinline__ void kernel_body(const Args& a) {
  using SH = Shape<MB, RG, STAGE, U, NS>;
  constexpr int BN = SH::BN;
  constexpr int WU = SH::WU;
  constexpr int kSlot = (STAGE == kStageLds) ? SH::slot_elems : 1;

  // LDS stages are distinct objects so the compiler can tell that a refill of
  // one stage does not alias reads of another and needs no extra wait.
  __shared__ u32x4 ring0[kSlot];
  __shared__ u32x4 ring1[kSlot];
  __shared__ u32x4 ring2[(NS > 2) ? kSlot : 1];
  __shared__ u32x4 ring3[(NS > 3) ? kSlot : 1];
  __shared__ float red[kWaves][RG][MB][4][kWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;     // which 16-byte vector of a 32-wide K chunk
  const int l16 = lane & 15;   // row within a 16-row MFMA operand

  // a0: blockIdx -> (tile, rank).  Workgroups are dealt to the 8 XCDs
  // round-robin; the ranks of one tile share blockIdx % 8, hence one XCD.
  const int bid = blockIdx.x;
  const int q = bid / kXcds;
  const int rank = q % a.S;
  const int tile = (q / a.S) * kXcds + (bid % kXcds);
  if (tile >= a.tiles) return;
  const int n0 = tile * BN;
  const int Ks = a.nvec * kVecK;
  const size_t k0 = (size_t)rank * Ks;

  // Per-lane operand rows.  Out-of-range rows are clamped to a valid row so
  // every load stays in bounds; their results are masked (act) or land only
  // in output columns that are never stored (W).
  const uint16_t* wrow[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    int n = n0 + 16 * rg + l16;
    n = n < a.N ? n : a.N - 1;
    wrow[rg] = a.W + (size_t)n * a.K + k0;
  }
  const uint16_t* arow[MB];
  bool a_ok[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int m = 16 * b + l16;
    a_ok[b] = m < a.M;
    arow[b] = a.A + (size_t)(a_ok[b] ? m : 0) * a.K + k0;
  }
  const int last_off = (a.nvec - 1) * kVecK;

  // Element offset of this lane's vector in chunk c (clamped into the slice).
  auto vec_off = [&](int c) {
    const int off = c * kChunkK + g * kVecK;
    return off < last_off ? off : last_off;
  };
  // Chunks a wavefront loads (and, in the register variant, consumes) in step
  // s: the four wavefronts' j-th loads are adjacent, so together they sweep
  // 16 rows x 256 contiguous bytes.
  auto load_chunk = [&](int s, int j) { return s * WU + j * kWaves + wave; };
  // Chunks a wavefront consumes in step s of the LDS variant.
  auto lds_chunk = [&](int s, int j) { return s * WU + wave * U + j; };

  f32x4 acc[RG][MB];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[rg][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Register stages: activation operands always, W operands in the register
  // variant.
  u32x4 areg[NS][U][MB];
  u32x4 wreg[(STAGE == kStageReg) ? NS : 1][U][RG];

  auto slot_ptr = [&](auto slot_c) -> u32x4* {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (SL == 0) return ring0;
    else if constexpr (SL == 1) return ring1;
    else if constexpr (SL == 2) return ring2;
    else return ring3;
  };

  // Issue the loads of step s into stage slot SL.  Always issued, even past
  // the last step (addresses clamped), so the number of vector-memory ops
  // after any group is a compile-time constant.
  auto issue = [&](auto slot_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (STAGE == kStageLds) {
      u32x4* slot = slot_ptr(slot_c);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int cl = j * kWaves + wave;                 // chunk within the step
        const int off = vec_off(load_chunk(s, j));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          // lane i's 16 bytes land at base + 16*i
          __builtin_amdgcn_global_load_lds(
              wrow[rg] + off,
              (__attribute__((address_space(3))) void*)(slot + (cl * RG + rg) * kWave), 16, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int off = vec_off(lds_chunk(s, j));
#pragma unroll
        for (int b = 0; b < MB; ++b) areg[SL][j][b] = load16(arow[b] + off);
      }
    } else {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int off = vec_off(load_chunk(s, j));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) wreg[SL][j][rg] = load16(wrow[rg] + off);
#pragma unroll
        for (int b = 0; b < MB; ++b) areg[SL][j][b] = load16(arow[b] + off);
      }
    }
    pin_issue();
  };

  // Multiply-accumulate step s out of stage slot SL.
  auto compute = [&](auto slot_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
    // Every chunk of the step is whole and inside the slice: no masking.
    const bool full = (s + 1) * WU * 4 <= a.nvec;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int c = (STAGE == kStageLds) ? lds_chunk(s, j) : load_chunk(s, j);
      const bool v_ok = full || (c * 4 + g < a.nvec);
      u32x4 wv[RG];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        if constexpr (STAGE == kStageLds) {
          const u32x4* slot = slot_ptr(slot_c);
          wv[rg] = slot[((wave * U + j) * RG + rg) * kWave + lane];
        } else {
          wv[rg] = wreg[SL][j][rg];
        }
        if (!full) wv[rg] = v_ok ? wv[rg] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        u32x4 av = areg[SL][j][b];
        av = (a_ok[b] && v_ok) ? av : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) acc[rg][b] = mfma(av, wv[rg], acc[rg][b]);
      }
    }
  };

  // One pipeline step: wait for stage s, refill the stage step s-1 used with
  // step s+NS-1, compute step s.
  auto step = [&](auto slot_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int NEXT = (SL + NS - 1) % NS;
    if constexpr (STAGE == kStageLds) {
      // Own loads of stage s have landed once at most the NS-2 younger groups
      // are outstanding ...
      wait_vmcnt<(NS - 2) * SH::group_loads>();
      // ... every wavefront's reads of the previous stage have completed ...
      wait_lgkmcnt0();
      // ... and after the barrier both hold for the whole workgroup, so the
      // stage read in step s-1 may be refilled and stage s may be read.
      barrier_keep_loads();
      LOWM_STALL(kSiteStageRead, s);
    }
    issue(std::integral_constant<int, NEXT>{}, s + NS - 1);
    compute(slot_c, s);
  };

  LOWM_STALL(kSiteEntry, 0);

  // Prologue: groups 0 .. NS-2.
  issue(std::integral_constant<int, 0>{}, 0);
  if constexpr (NS > 2) issue(std::integral_constant<int, 1>{}, 1);
  if constexpr (NS > 3) issue(std::integral_constant<int, 2>{}, 2);

  for (int s = 0; s < a.nsteps; s += NS) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 >= a.nsteps) break;
    step(std::integral_constant<int, 1 % NS>{}, s + 1);
    if constexpr (NS > 2) {
      if (s + 2 >= a.nsteps) break;
      step(std::integral_constant<int, 2 % NS>{}, s + 2);
    }
    if constexpr (NS > 3) {
      if (s + 3 >= a.nsteps) break;
      step(std::integral_constant<int, 3 % NS>{}, s + 3);
    }
  }
  // No load may still be writing into LDS or registers when the wavefront
  // moves on (the trailing groups are clamped re-reads of the last chunk).
  wait_vmcnt0();

  // Wavefront reduction through LDS, added in wavefront order below.
  LOWM_STALL(kSiteReduce, 0);
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][rg][b][i][lane] = acc[rg][b][i];
  wait_lgkmcnt0();
  barrier_keep_loads();
  if (wave != 0) return;

  // Wavefront 0 owns the epilogue.  Output element e of the tile is (m, nl) =
  // (e / BN, e % BN).  The MFMA keeps D[row][col] in lane col + 16*(row/4),
  // register row % 4; rows are activation rows, columns weight rows.
  const int E = a.M * BN;
  auto rank_sum = [&](int e) {
    const int m = e / BN, nl = e - (e / BN) * BN;
    const int b = m >> 4, mm = m & 15;
    const int ln = (nl & 15) + 16 * (mm >> 2), rg = nl >> 4, i = mm & 3;
    float p = red[0][rg][b][i][ln];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) p += red[w][rg][b][i][ln];
    return p;
  };
  OutT* C = static_cast<OutT*>(a.C);

  if (a.S == 1) {
    for (int e = lane; e < E; e += kWave) {
      const int m = e / BN, n = n0 + (e - m * BN);
      if (n < a.N) C[(size_t)m * a.N + n] = to_out<OutT>(rank_sum(e));
    }
    return;
  }

  // a4: publish this rank's partial, then arrive.
  LOWM_STALL(kSitePublish, 0);
  float* slots = a.part + (size_t)tile * a.S * E;
  for (int e = lane; e < E; e += kWave) slots[(size_t)rank * E + e] = rank_sum(e);
  // Release at agent scope: the partial is written back past this XCD's L2
  // before the arrival can be observed (buffer_wbl2 + vmcnt(0)).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  uint32_t before = 0;
  if (lane == 0)
    before = __hip_atomic_fetch_add(a.ctr + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  before = __builtin_amdgcn_readfirstlane(before);
  if (before != (uint32_t)(a.S - 1)) return;   // not the last rank: done

  // a5: the owner.  One acquire at agent scope (buffer_inv), then the fold in
  // rank order with this rank's partial taken from LDS at its own position.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  LOWM_STALL(kSiteFold, 0);
  for (int e = lane; e < E; e += kWave) {
    const float own = rank_sum(e);
    float v = (rank == 0) ? own : slots[e];
    for (int r = 1; r < a.S; ++r) v += (r == rank) ? own : slots[(size_t)r * E + e];
    const int m = e / BN, n = n0 + (e - m * BN);
    if (n < a.N) C[(size_t)m * a.N + n] = to_out<OutT>(v);  // a6
  }
  // The tile's counter is zero again for the next launch.
  if (lane == 0) __hip_atomic_store(a.ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The body uses device-only builtins (direct-to-LDS loads), which the host
// pass cannot instantiate; it only needs the launch stub there.
template <int MB, int RG, int STAGE, int U, int NS, typename OutT>
__global__ __launch_bounds__(kThreads) void lowm_splitk_kernel(Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  kernel_body<MB, RG, STAGE, U, NS, OutT>(a);
#endif
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Variant {
  int stage, unroll, stages;
};
// The register/LDS variants this build provides (any rows in {16,32,64}).
constexpr Variant kVariants[] = {
    {kStageLds, 2, 4}, {kStageLds, 2, 3}, {kStageLds, 4, 3}, {kStageLds, 1, 4},
    {kStageReg, 2, 4}, {kStageReg, 4, 3}, {kStageReg, 4, 4}, {kStageReg, 2, 3},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

typedef void (*KernelFn)(Args);

template <int MB, int RG, int VI, typename OutT>
KernelFn kernel_for() {
  constexpr Variant v = kVariants[VI];
  if constexpr (Shape<MB, RG, v.stage, v.unroll, v.stages>::valid)
    return lowm_splitk_kernel<MB, RG, v.stage, v.unroll, v.stages, OutT>;
  else
    return nullptr;
}

template <int MB, int RG, typename OutT, int... VI>
void fill_row(KernelFn* row, std::integer_sequence<int, VI...>) {
  ((row[VI] = kernel_for<MB, RG, VI, OutT>()), ...);
}

// table[out][MB-1][rg_index][variant]
struct Table {
  KernelFn fn[2][4][3][kNumVariants];
};
template <typename OutT, int MB, int RG>
void fill_one(Table& t, int out) {
  constexpr int ri = RG == 1 ? 0 : RG == 2 ? 1 : 2;
  fill_row<MB, RG, OutT>(t.fn[out][MB - 1][ri], std::make_integer_sequence<int, kNumVariants>{});
}
template <typename OutT>
void fill_out(Table& t, int out) {
  fill_one<OutT, 1, 1>(t, out); fill_one<OutT, 1, 2>(t, out); fill_one<OutT, 1, 4>(t, out);
  fill_one<OutT, 2, 1>(t, out); fill_one<OutT, 2, 2>(t, out); fill_one<OutT, 2, 4>(t, out);
  fill_one<OutT, 3, 1>(t, out); fill_one<OutT, 3, 2>(t, out); fill_one<OutT, 3, 4>(t, out);
  fill_one<OutT, 4, 1>(t, out); fill_one<OutT, 4, 2>(t, out); fill_one<OutT, 4, 4>(t, out);
}
const Table& table() {
  static const Table t = [] {
    Table x{};
    fill_out<__bf16>(x, 0);
    fill_out<float>(x, 1);
    return x;
  }();
  return t;
}

thread_local int g_last_hip_error = 0;
StressArgs g_stress = {0u, -1, -1, 0, 0, -1, 0u};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_sizes(int M, int N, int K, int S) {
  if (M <= 0 || N <= 0 || K <= 0 || S < 1) return LOWM_ERR_INVALID_ARG;
  if (M > LOWM_MAX_M || S > LOWM_MAX_SPLIT_K) return LOWM_ERR_UNSUPPORTED;
  if (K % (kVecK * S) != 0) return LOWM_ERR_UNSUPPORTED;
  return LOWM_OK;
}

size_t counter_bytes(int N) { return round_up((size_t)4 * ((N + 15) / 16), 256); }

int variant_index(const lowm_tactic& t) {
  for (int i = 0; i < kNumVariants; ++i)
    if (kVariants[i].stage == t.stage && kVariants[i].unroll == t.unroll &&
        kVariants[i].stages == t.stages)
      return i;
  return -1;
}

int rows_index(int rows) { return rows == 16 ? 0 : rows == 32 ? 1 : rows == 64 ? 2 : -1; }

KernelFn lookup(bool f32out, int M, const lowm_tactic& t) {
  if (t.waves != kWaves) return nullptr;
  const int ri = rows_index(t.rows);
  const int vi = variant_index(t);
  if (ri < 0 || vi < 0 || M < 1 || M > LOWM_MAX_M) return nullptr;
  return table().fn[f32out ? 1 : 0][(M + 15) / 16 - 1][ri][vi];
}

// Default tactic: enough weight rows per tile that re-reading the activation
// slice per tile stays below the weight traffic, and the first variant in a
// preference list that this build provides for that shape.
int pick(int M, int N, int K, int S, lowm_tactic* t) {
  const int rc = check_sizes(M, N, K, S);
  if (rc != LOWM_OK) return rc;
  static const Variant pref[] = {{kStageReg, 4, 3}, {kStageReg, 2, 4}, {kStageReg, 2, 3},
                                 {kStageLds, 2, 4}, {kStageLds, 1, 4}};
  t->waves = kWaves;
  t->rows = M <= 16 ? 16 : (M <= 32 ? 32 : 64);
  for (const Variant& v : pref) {
    t->stage = v.stage;
    t->unroll = v.unroll;
    t->stages = v.stages;
    if (lookup(false, M, *t) && lookup(true, M, *t)) return LOWM_OK;
  }
  return LOWM_ERR_UNSUPPORTED;
}

int launch(const void* A, const void* W, void* C, bool f32out, int M, int N, int K, int S,
           void* workspace, hipStream_t stream, const lowm_tactic* tactic) {
  if (!A || !W || !C) return LOWM_ERR_INVALID_ARG;
  int rc = check_sizes(M, N, K, S);
  if (rc != LOWM_OK) return rc;
  if (S > 1 && !workspace) return LOWM_ERR_WORKSPACE;
  if (((uintptr_t)A | (uintptr_t)W) & 15) return LOWM_ERR_UNSUPPORTED;
  if ((uintptr_t)C & (f32out ? 3 : 1)) return LOWM_ERR_UNSUPPORTED;
  if (S > 1 && ((uintptr_t)workspace & 15)) return LOWM_ERR_UNSUPPORTED;

  lowm_tactic t;
  if (tactic) {
    t = *tactic;
  } else {
    rc = pick(M, N, K, S, &t);
    if (rc != LOWM_OK) return rc;
  }
  const KernelFn fn = lookup(f32out, M, t);
  if (!fn) return LOWM_ERR_UNSUPPORTED;

  const int BN = t.rows;
  const int WU = kWaves * t.unroll;
  Args a;
  a.A = static_cast<const uint16_t*>(A);
  a.W = static_cast<const uint16_t*>(W);
  a.C = C;
  a.M = M;
  a.N = N;
  a.K = K;
  a.S = S;
  a.nvec = K / S / kVecK;
  a.nchunks = (a.nvec + 3) / 4;
  a.nsteps = (a.nchunks + WU - 1) / WU;
  a.tiles = (N + BN - 1) / BN;
  a.ctr = S > 1 ? static_cast<uint32_t*>(workspace) : nullptr;
  a.part = S > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + counter_bytes(N))
                 : nullptr;
  a.stress = g_stress;

  const size_t tiles_pad = round_up((size_t)a.tiles, kXcds);
  const size_t grid = tiles_pad * (size_t)S;
  if (grid > 0x7fffffffu) return LOWM_ERR_UNSUPPORTED;
  void* kargs[] = {&a};
  hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)grid),
                                   dim3(kThreads), kargs, 0, stream);
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
  if (lowm::check_sizes(M, N, K, split_k) != LOWM_OK || split_k == 1) return 0;
  // counters for up to ceil(N/16) tiles, then [tiles][split_k][M][BN] fp32
  // partials; tiles * BN never exceeds N rounded up to 64.
  return lowm::counter_bytes(N) +
         (size_t)split_k * (size_t)M * lowm::round_up((size_t)N, 64) * sizeof(float);
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
#endif

}  // extern "C"
