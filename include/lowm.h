/*
 * lowm.h -- C ABI of the low-M split-K bf16 GEMM for AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (TensorRT-LLM PR "Fix two synchronization gaps in the MiniMax
 * M3 low-M split-K GEMM", Description item 2 and Hardware verification):
 *
 *     C[m][n] = sum_{k=0}^{K-1} A[m][k] * W[n][k]        (C = A * W^T)
 *
 * with A [M, K] and W [N, K] bf16, fp32 accumulation and a bf16 (or fp32)
 * result.  The K range is cut into split_k equal contiguous slices; each slice
 * ("rank") produces an fp32 partial of the output tile and one owner adds the
 * partials, always in rank order 0, 1, ..., split_k-1, then rounds once to
 * bf16 (round-to-nearest-even) and is the only writer of C.  The owner is the
 * last rank of the tile to arrive (a per-tile counter in the workspace), or,
 * for split_k 2..4 and line-pair, register or LDS tiles of M x (tile rows)
 * <= 64 elements (M <= 4 with the 16-row line-pair tiles that are the default
 * there), the tile's last rank when it finds every peer's partial already in
 * the workspace.  That rank polls for at most 20 us
 * and then arrives like any other, so no workgroup waits for another without
 * a bound and any grid size completes.
 *
 * Layouts: A, W and C are dense row-major with no padding: element (m, k) of A
 * at A + m*K + k, (n, k) of W at W + n*K + k, (m, n) of C at C + m*N + n.
 * C must not overlap A, W or the workspace (A and W may overlap: they are
 * only read); a launch given overlapping buffers returns LOWM_ERR_INVALID_ARG.
 *
 * Ownership: the caller owns every buffer.  The library allocates nothing,
 * frees nothing and keeps no mutable global state (a per-device table of
 * compute-unit counts is read once).  All entry points that launch work are
 * asynchronous on `stream` (a hipStream_t; NULL is the null stream): they
 * validate their arguments on the host before any HIP call, enqueue one
 * kernel and return.  Execution errors surface at the caller's next
 * synchronisation.
 *
 * Workspace (split_k > 1 only): an opaque device buffer of
 * lowm_gemm_splitk_workspace_bytes(M, N, K, split_k) bytes, 256-byte aligned,
 * holding one arrival counter per output tile, each on its own 256-byte line
 * (256 * ceil(N / 16) bytes), followed by the partial slots (one 32-bit word
 * per rank and tile element: the complement of the fp32 partial's bits, so
 * that zero means "not published").  Zero it once before first use
 * (hipMemset).  Every launch that completes leaves the whole workspace zero
 * again (the owner resets its tile's counter and every slot of the tile), so
 * it can be reused by the next launch, of any shape, without clearing; a
 * caller must not write to it between launches.  One workspace per in-flight
 * launch: launches that overlap in time (two streams) must not share one.
 * After a launch that did not complete, zero it again.
 *
 * Errors: every int-returning function returns LOWM_OK (0) or a negative
 * LOWM_ERR_* code; lowm_strerror() names it and lowm_last_hip_error() gives
 * the hipError_t behind LOWM_ERR_LAUNCH on the calling thread.
 */
#ifndef LOWM_H
#define LOWM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOWM_OK 0
/* A NULL operand pointer, M, N or K <= 0, split_k < 1, or an output C whose
 * bytes overlap A, W, another output of the launch or the workspace (or a
 * workspace that overlaps A or W). */
#define LOWM_ERR_INVALID_ARG (-1)
/* Outside what the kernels support: M > 64 (the low-M regime); K not a
 * multiple of 8 * split_k (every rank's slice must be a non-empty whole number
 * of 16-byte vectors); split_k > 256; A, W or the workspace not 16-byte
 * aligned; C not aligned to its element size; a tactic the build lacks. */
#define LOWM_ERR_UNSUPPORTED (-2)
/* split_k > 1 with a NULL workspace. */
#define LOWM_ERR_WORKSPACE (-3)
/* A HIP call failed: the kernel launch, or the stream synchronisation or
 * copy of lowm_workspace_status; see lowm_last_hip_error(). */
#define LOWM_ERR_LAUNCH (-4)
/* lowm_gemm_splitk_noalloc: the sizes need a workspace larger than
 * LOWM_SCRATCH_BYTES. */
#define LOWM_ERR_SCRATCH (-5)

/* Largest M the kernels accept. */
#define LOWM_MAX_M 64
/* Largest split_k the kernels accept. */
#define LOWM_MAX_SPLIT_K 256

/*
 * C (bf16 [M, N]) = A (bf16 [M, K]) * W (bf16 [N, K])^T, fp32 accumulation,
 * split_k equal K slices folded in rank order by the last-arriving rank
 * (PR "Fix two synchronization gaps in the MiniMax M3 low-M split-K GEMM",
 * Description item 2: each rank's fp32 partial over its part of K, summed
 * by one owner; Hardware verification: bf16 operands and output).
 * `workspace` may be NULL when split_k == 1.  `stream` is a hipStream_t.
 */
int lowm_gemm_splitk(const void* A, const void* W, void* C,
                     int M, int N, int K, int split_k,
                     void* workspace, void* stream);

/*
 * The same product with an fp32 result: C is float [M, N].  Same kernel and
 * summation order; only the final store differs, so the bf16 entry point's
 * output is exactly this result rounded to nearest-even.  The fp32 sum is
 * what the pages check against: the PR's Hardware verification compares
 * each output with the fp32 product of the same operands, and the integer
 * closed form of the Triton issue "warpgroup_mma_wait does not properly
 * synchronize across warpgroups" (Describe the bug) is exact only in fp32.
 */
int lowm_gemm_splitk_f32out(const void* A, const void* W, float* C,
                            int M, int N, int K, int split_k,
                            void* workspace, void* stream);

/*
 * Bytes of workspace a launch with these sizes needs: 0 when split_k == 1,
 * else the counters (256 bytes per 16 columns of C) plus the fp32 partials,
 * split_k * M * round_up(N, 64) floats.  Returns 0 as well for arguments the
 * launch would reject.  The workspace carries the split-K exchange that the
 * PR's Description item 2 runs through a shared-memory mailbox inside a
 * 2-CTA cluster; gfx950 has neither, so the partials and the arrival counts
 * go through device memory instead.  Host-only; no HIP call.
 */
size_t lowm_gemm_splitk_workspace_bytes(int M, int N, int K, int split_k);

/*
 * Batched launch (the pages' kernel runs with programmatic dependent launch,
 * which lets the next kernel start while this one is in its main loop: PR,
 * Description item 1 and Hardware verification; ROCm has no such launch, and
 * this entry point hides the same launch gaps by running several GEMMs of
 * one layer in one launch): `count` (1 .. LOWM_MAX_BATCH) independent products
 * C_g = A_g * W_g^T that share M, K, split_k and the bf16 output, in one
 * kernel launch (one launch gap instead of `count`; the GEMMs' tails
 * overlap).  Each GEMM is exactly what lowm_gemm_splitk computes for it: one
 * tactic serves the launch (the default for M, K, split_k and the narrowest
 * N_g), whose per-element summation order equals the single call's, so each
 * output is bitwise the single call's.  The workspace (split_k > 1) is the concatenation, in
 * order, of each GEMM's own workspace of lowm_gemm_splitk_workspace_bytes
 * (M, N_g, K, split_k) bytes; lowm_gemm_splitk_batched_workspace_bytes gives
 * the total.  Zero it once; every completed launch leaves it reusable.
 * Errors as lowm_gemm_splitk, checked for every GEMM before any HIP call;
 * count < 1 or a NULL `gemms` is LOWM_ERR_INVALID_ARG, count > LOWM_MAX_BATCH
 * LOWM_ERR_UNSUPPORTED.
 */
#define LOWM_MAX_BATCH 8
typedef struct lowm_gemm_desc {
    const void* A;   /* bf16 [M, K] */
    const void* W;   /* bf16 [N, K] */
    void* C;         /* bf16 [M, N] */
    int N;
} lowm_gemm_desc;

int lowm_gemm_splitk_batched(const lowm_gemm_desc* gemms, int count, int M, int K,
                             int split_k, void* workspace, void* stream);

/* Total workspace bytes of a batched launch (0 when split_k == 1, or for
 * arguments the launch would reject). */
size_t lowm_gemm_splitk_batched_workspace_bytes(const lowm_gemm_desc* gemms, int count,
                                                int M, int K, int split_k);

/* Static text naming an error code.  (Error reporting of the host launch
 * path; the PR's Description item 1 has the host guarantee a non-empty K
 * loop, which this library checks and reports as LOWM_ERR_UNSUPPORTED.) */
const char* lowm_strerror(int code);

/* hipError_t of the most recent failed HIP call on the calling thread (0 if
 * none); the cause behind LOWM_ERR_LAUNCH. */
int lowm_last_hip_error(void);

/* Status of a split-K workspace: failure detection for the exchange (the
 * defects of PR "Fix two synchronization gaps in the MiniMax M3 low-M
 * split-K GEMM", Description items 1 and 2, were lost or stale reads).
 * Each 256-byte counter line of the workspace holds, in word 0, the tile's
 * arrival count and, in word 1, its fault word.
 * An owner that still finds a peer's partial slot unpublished 1 ms after
 * every peer has arrived stops waiting, folds the slot as it reads it and
 * sets the fault word; the library never clears a fault word.  That
 * launch's C is invalid for the tile, and the workspace must be zeroed
 * before its next use (the late partial may still land in it).  A
 * non-zero arrival count after the stream has drained means a launch that
 * did not complete.
 *
 * Waits for the work queued on `stream` (hipStreamSynchronize), copies the
 * ceil(N / 16) counter lines of `workspace` (a workspace last used by a
 * launch with N output columns and split_k > 1) to the host and stores the
 * number of tiles with a set fault word in *faulted_tiles and the number
 * with a non-zero arrival count in *open_tiles.  For a batched workspace,
 * call it on each GEMM's part: GEMM g's begins after the
 * lowm_gemm_splitk_workspace_bytes of GEMMs 0..g-1.  (The built-in scratch
 * of lowm_gemm_splitk_noalloc is not reachable from here.)  A NULL pointer
 * or N <= 0 is LOWM_ERR_INVALID_ARG (no HIP call); a failed synchronisation
 * or copy is LOWM_ERR_LAUNCH. */
int lowm_workspace_status(const void* workspace, int N, void* stream, int* faulted_tiles,
                          int* open_tiles);

/*
 * Tactic: how a launch tiles the problem.  lowm_gemm_splitk picks one from
 * (M, N, K, split_k); the _ex entry points take it explicitly, for tuning
 * sweeps and for tests that cover every variant.  Any tactic gives a correct
 * result; the summation order (and so the low bits of random-input results)
 * depends on it.  The pages ship fixed tactics per split_k (TensorRT-LLM PR
 * "Fix two synchronization gaps in the MiniMax M3 low-M split-K GEMM",
 * Hardware verification); these are this library's own.
 *   stage      LOWM_STAGE_LINE: W goes global -> LDS in whole 128-byte lines
 *              (8 rows x 128 B per direct-to-LDS load, non-temporal); each
 *              wavefront streams its own quarter of the K slice through a
 *              ring of `stages` slots of 16 rows x 64 K that only it reads,
 *              with no barrier in the main loop; activation operands go
 *              straight into registers.  unroll must be 2; the K slice must
 *              be a multiple of 256 (K / split_k % 256 == 0).  rows 16, or
 *              32 with 2 stages; M <= 32.
 *              LOWM_STAGE_PANEL: tiles of 64 rows, 16 per wavefront, each
 *              wavefront walking the whole K slice (or of 32 rows, 16 per
 *              pair of wavefronts, each of the pair walking one half of the
 *              slice, the halves added in order); W as in LINE (a ring slot
 *              per wavefront), the activation operand of each 64-K step
 *              ("panel") loaded once per workgroup into an LDS ring of
 *              `stages` steps that all wavefronts read, refilled only after a
 *              workgroup barrier.  rows 64 or 32, unroll 2, stages 3, 4 or 6;
 *              17 <= M <= 64; the K slice a multiple of 64 (rows 64) or 128
 *              (rows 32).
 *              LOWM_STAGE_QUARTER: each wavefront streams one quarter of
 *              the K slice for the whole tile, both operands (W rows and
 *              activation rows) through a ring of `stages` 64-K slots of its
 *              own in LDS, with whole-line direct-to-LDS loads; no barrier in
 *              the main loop; the four quarter sums are added in order
 *              through LDS at the end.  rows 16, 32, 48 or 64, unroll 2, stages
 *              2, 3 or 4 (where LDS and the wait counter allow); the K slice
 *              a multiple of 256.
 *              LOWM_STAGE_QUARTER_ROWS: QUARTER tiles whose workgroups each
 *              take one block of 16 * unroll activation rows (the last block
 *              may be shorter): ceil(M / (16 * unroll)) workgroups per tile,
 *              on one XCD, each streaming the tile's W rows (the blocks after
 *              the first find them in the L2) and only its own activation
 *              rows.  The same summation order, so the same bits, as
 *              QUARTER.  rows 16, 32, 48 or 64, unroll 1..4, stages as
 *              QUARTER; split_k 1 only; not with the push epilogue (every
 *              block of a tile would raise its flags).
 *              LOWM_STAGE_LDS: W goes global -> an LDS ring of `stages`
 *              stages shared by the workgroup; a stage holds 512 K of each of
 *              the tile's rows, each direct-to-LDS load moving 1 KB of one
 *              row; a stage is refilled only after a workgroup barrier that
 *              every wavefront reaches once its reads of it are done.  unroll
 *              must be 4; stages 2 or 3.
 *              LOWM_STAGE_REG: W goes global -> registers, a ring of
 *              `stages` register stages per wavefront, `unroll` 32-wide K
 *              chunks (4, 8 or 16) per wavefront per stage; each wavefront
 *              streams its own contiguous quarter of the K slice.  stages 2.
 *   rows       W rows (output columns) per workgroup tile: 16 or 32 (LINE,
 *              LDS, REG), 64 or 32 (PANEL), 16, 32, 48 or 64 (QUARTER,
 *              QUARTER_ROWS).
 *   waves      wavefronts per workgroup: always 4.
 *   unroll     see stage.
 *   stages     ring depth, see stage.
 * A tactic the build does not provide for the launch's M and K slice is
 * LOWM_ERR_UNSUPPORTED.
 */
#define LOWM_STAGE_LDS 0
#define LOWM_STAGE_REG 1
#define LOWM_STAGE_LINE 3
#define LOWM_STAGE_PANEL 4
#define LOWM_STAGE_QUARTER 5
#define LOWM_STAGE_QUARTER_ROWS 6
typedef struct lowm_tactic {
    int stage;
    int rows;
    int waves;
    int unroll;
    int stages;
} lowm_tactic;

/* The tactic lowm_gemm_splitk would use for these sizes (written to *out).
 * Returns LOWM_OK or an error code for sizes it would reject.  Host-only.
 * (The push entry point picks the same way but never takes
 * LOWM_STAGE_QUARTER_ROWS: it uses the QUARTER or PANEL tiles the rules give
 * without that family.)
 * (The PR ships one fixed tactic per split_k, Hardware verification; this
 * one is chosen per shape from measurements on MI355X.) */
int lowm_pick_tactic(int M, int N, int K, int split_k, lowm_tactic* out);

/* Host-only: a split_k for these sizes (written to *split_k), chosen from a
 * table of the fastest split_k measured on MI355X (bench.py --split-sweep)
 * over M 4, 8, 16, 32 and 64, N 768 .. 24576, K 2048 .. 16384 (nearest
 * grid point in log2 N and log2 K, the row of the next measured M at or
 * above M), reduced to a power of two that K allows.  Any split_k is
 * correct; this one minimises time per call.  (The PR ships split_k 1 and 2,
 * Hardware verification.)  Returns LOWM_OK, or the error code a launch would
 * return for M, N, K. */
int lowm_pick_split_k(int M, int N, int K, int* split_k);

/* Host-only: LOWM_OK if a launch with these sizes, output type (f32out != 0:
 * fp32) and tactic (NULL: the default) would find a kernel in the library, else
 * the error code the launch would return for them (the host-side checks of
 * lowm_gemm_splitk, including the PR's non-empty K loop of Description
 * item 1).  No HIP call is made. */
int lowm_check_launch(int M, int N, int K, int split_k, int f32out,
                      const lowm_tactic* tactic);

/* lowm_gemm_splitk / _f32out with an explicit tactic (NULL: the default),
 * the same product (PR, Description item 2) in another summation order.
 * LOWM_ERR_UNSUPPORTED for a tactic the library does not provide. */
int lowm_gemm_splitk_ex(const void* A, const void* W, void* C,
                        int M, int N, int K, int split_k,
                        void* workspace, void* stream, const lowm_tactic* tactic);
int lowm_gemm_splitk_f32out_ex(const void* A, const void* W, float* C,
                               int M, int N, int K, int split_k,
                               void* workspace, void* stream,
                               const lowm_tactic* tactic);

/*
 * Push epilogue.  The pages name a push epilogue among the shipped variants
 * of the kernel (split_k 1 and 2, with and without it) and state that only
 * the owner of an output tile publishes it, without defining it further
 * (TensorRT-LLM PR "Fix two synchronization gaps in the MiniMax M3 low-M
 * split-K GEMM", Hardware verification and Test Coverage).  Reading taken
 * here: the owner of each output tile (the last-arriving rank; every
 * workgroup when split_k == 1) writes its bf16 tile to C as
 * lowm_gemm_splitk does and also to a caller-given exchange buffer, for
 * instance where the next operation of a tensor-parallel layer reads it, and
 * then raises a flag per 16 output columns so that a consumer can start on
 * the columns that are ready.
 *
 *   push      bf16 exchange buffer: element (m, n) goes to push[m * push_ld + n];
 *             push_ld >= N elements; 2-byte aligned.
 *   flags     uint32 [ceil(N / 16)]: flag j covers columns 16j .. 16j+15;
 *             4-byte aligned.
 *   flag_value  non-zero value written to each flag.
 *
 * The pushed elements are written with system-scope stores and a flag is
 * written, also at system scope, only after every pushed store of its
 * columns has been acknowledged: an observer that reads flag j == flag_value
 * with a system-scope (or, on this device, device-scope) load and then reads
 * those columns with such loads sees the final values.  The library never
 * resets the flags: the consumer clears them, or the caller uses a new
 * flag_value per call.  C, the exchange buffer and the flags must not
 * overlap (LOWM_ERR_INVALID_ARG).  Output C and all other arguments and
 * errors are as lowm_gemm_splitk_ex (tactic NULL: the default).
 */
int lowm_gemm_splitk_push(const void* A, const void* W, void* C, int M, int N, int K,
                          int split_k, void* workspace, void* push, int push_ld,
                          uint32_t* flags, uint32_t flag_value, void* stream,
                          const lowm_tactic* tactic);

/*
 * Consumer side of the push epilogue (the publication the PR's Hardware
 * verification and Test Coverage name, read as above): enqueues on `stream`
 * one wavefront that polls flags[0 .. n_flags-1] with system-scope loads
 * until each equals flag_value, or until timeout_us microseconds have
 * passed, and then writes to the device int *missing the number of flags it
 * did not see set (0: all were).  Work enqueued after it on `stream` runs
 * after it.  `flags` must hold at least n_flags words (the library cannot
 * check this: a shorter buffer is read past its end); n_flags 1 .. 4096,
 * timeout_us <= 10,000,000, flag_value non-zero; the wait is bounded whether
 * or not any producer runs.
 */
int lowm_push_wait(const uint32_t* flags, int n_flags, uint32_t flag_value,
                   uint32_t timeout_us, int* missing, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the product
 * of lowm_gemm_splitk, bit for bit the same kernels, tactic and summation
 * order, with the split-K workspace taken from a buffer built into the
 * library instead of the caller's.  No hipMalloc, hipFree or other
 * allocation happens in this call.
 *
 * The buffer is a device array of LOWM_SCRATCH_BYTES per GPU, held from the
 * library's first call on that GPU until the process ends; its device
 * address is looked up once per GPU (on the device `stream` belongs to).  It
 * is zero when loaded, and every launch that completes returns every word it
 * used to zero, so each call finds it clear.  All calls on one GPU share it:
 * calls that overlap in time on that GPU (two streams, or two threads) race
 * and must not be issued.  Sizes whose workspace
 * (lowm_gemm_splitk_workspace_bytes) exceeds LOWM_SCRATCH_BYTES return
 * LOWM_ERR_SCRATCH before any HIP call; other arguments and errors as
 * lowm_gemm_splitk.  split_k == 1 uses no workspace.
 */
#define LOWM_SCRATCH_BYTES (16u << 20)
int lowm_gemm_splitk_noalloc(const void* A, const void* W, void* C,
                             int M, int N, int K, int split_k, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LOWM_H */
