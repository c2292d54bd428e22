/*
 * arepi.h -- C ABI of the MI355X (gfx950) fused all-reduce epilogue library.
 *
 * Three operations of a tensor-parallel layer, each one hand-written HIP
 * kernel, plus the calls that arm, feed and emulate the peers on one GPU:
 *
 *   arepi_gemm_rs_fused      row-parallel bf16 GEMM whose epilogue finishes the
 *                            reduce-scatter of this rank's owner segment, gated
 *                            per flag tile by a readiness bitmask.
 *   arepi_gemm_rs_ring       the same GEMM as one hop of a push-ring
 *                            reduce-scatter (one upstream partial per row).
 *   arepi_ar_rmsnorm_lamport all-reduce combine + RMSNorm where the data is its
 *                            own arrival flag (Lamport -0.0 sentinel).
 *   arepi_combine_reduce     weighted top-k combine of expert outputs.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers into row-major, contiguous
 *     buffers owned by the caller, 16-byte aligned.  Arrays of pointers marked
 *     HOST are host arrays whose elements are device pointers.  bf16 data is
 *     passed as uint16_t bit patterns.
 *   - Every call validates all arguments before launching anything.  On bad
 *     arguments it launches nothing, returns a negative arepi_status and records
 *     a message naming the argument, the value given and the allowed range
 *     (read it with arepi_last_error(), thread-local).
 *   - Launches are asynchronous on `stream` (a hipStream_t; NULL is the legacy
 *     default stream).  Device-side status words are read by the caller after
 *     synchronising.  The library allocates no device memory.  Its only state
 *     is the per-thread error message, a per-device cache of the wall-clock
 *     rate, and the static staging of arepi_ar_rmsnorm_lamport_noalloc.
 *   - Spin waits are bounded: `spin_limit` > 0 is the number of polls before a
 *     wait gives up; <= 0 selects a deadline of one second of the device's
 *     constant-rate wall clock (s_memrealtime, its rate read from the runtime)
 *     from the start of the wait.  A wait that gives up ORs
 *     AREPI_STATUS_TIMEOUT into *status (when status is non-NULL) and the
 *     kernel finishes normally, with the affected outputs unspecified.
 */
#ifndef AREPI_H
#define AREPI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *arepi_stream_t; /* same type as hipStream_t */

typedef enum {
    AREPI_OK = 0,
    AREPI_EINVAL = -1,       /* null pointer, negative size, shape mismatch, misalignment */
    AREPI_EUNSUPPORTED = -2, /* valid request outside what the kernels implement */
    AREPI_ELAUNCH = -3       /* the HIP runtime refused the launch */
} arepi_status;

/* Memory scope of readiness flags: AGENT when producer and consumer share one
 * GPU, SYSTEM when the producer is another device. */
enum { AREPI_SCOPE_AGENT = 0, AREPI_SCOPE_SYSTEM = 1 };

/* Bits ORed into a device status word. */
enum { AREPI_STATUS_TIMEOUT = 1u };

/* Compute-tile choice for arepi_gemm_rs_fused (0 = chosen from the shape).
 * BMxBN is the output tile of one workgroup; the _S variants walk K in
 * 32-wide steps through an S-stage LDS ring (the others: 64-wide, 2 stages;
 * 64x128_S4: 64-wide, 4 stages). */
enum {
    AREPI_TILE_AUTO = 0,
    AREPI_TILE_256x256 = 1,
    AREPI_TILE_128x256 = 2,
    AREPI_TILE_128x128 = 3,
    AREPI_TILE_64x128 = 4,
    AREPI_TILE_32x256 = 5,
    AREPI_TILE_256x256_S4 = 6,
    AREPI_TILE_256x128_S3 = 7,
    AREPI_TILE_128x256_S3 = 8,
    AREPI_TILE_128x128_S4 = 9,
    AREPI_TILE_256x256_W8 = 10, /* 8 waves (two per SIMD), BK 32, 4 stages */
    AREPI_TILE_256x256_W8_K64 = 11, /* 8 waves, BK 64, 2 stages: half the barriers per K */
    AREPI_TILE_64x128_S4 = 12,      /* BK 64, 4 stages (96 KiB of LDS): one workgroup per CU */
    /* ORed into an explicit tile: when every segment is a whole number of
     * half-blocks (BM/2 rows, BM >= 64), a workgroup takes two half-blocks and
     * the owner segment's half-blocks are each paired with a non-owner one,
     * which spreads the owner rows' peer reads over twice as many workgroups.
     * Without it (and for other shapes) each workgroup's rows are one
     * contiguous block. */
    AREPI_TILE_PAIRED_ROWS = 0x200,
    /* ORed into any tile_cfg (AUTO included): the owner tiles clear each
     * ready_in bit they waited for, so ready_in is all zero again when the
     * call ends and the next call can use it without a separate clear.  A
     * tile clears its bits only after every load of the data under them has
     * returned (at the end of its epilogue), so a bit that reads clear also
     * says its slot of recv may be refilled for the next call.  Needs the
     * flag tiles to nest inside the compute tiles, as ready_out does. */
    AREPI_TILE_CONSUME_READY = 0x400,
    /* ORed into a contiguous tile_cfg (AUTO included) of arepi_gemm_rs_fused:
     * the owner segment's row blocks come first in the schedule instead of
     * last.  Last suits partials that land while the GEMM runs (the owner
     * tiles wait for them as late as possible); first suits partials already
     * landed when the call starts: in a grid of several rounds the owner
     * tiles' longer epilogue (R-1 partials read per tile) then overlaps the
     * later rounds instead of forming the last one.  Not with
     * AREPI_TILE_PAIRED_ROWS, not for the push ring or the fp8 form. */
    AREPI_TILE_OWNER_FIRST = 0x800,
    /* ORed into AREPI_TILE_256x256_W8_K64 (or AUTO where that tile is the
     * automatic choice) of arepi_gemm_rs_fused, for grids of several rounds:
     * the owner segment runs as 128x256 tiles (same eight waves, half the
     * rows each) in workgroups after all the others, so each owner workgroup
     * reads half the peers' bytes and the last round, which holds them, ends
     * sooner.  Needs R >= 2, the segment height a multiple of 256, the
     * contiguous owner-last layout, and (with ready_out or consumption) flag
     * tiles nesting in 128x256 tiles.  AREPI_TILE_AUTO turns it on by itself
     * where it applies and adds no round of workgroups. */
    AREPI_TILE_OWNER_HALF = 0x1000
};

/* Message describing the last failed call on this thread ("" if none). */
const char *arepi_last_error(void);

/* Library version string. */
const char *arepi_version(void);

/* ------------------------------------------------------------------------ *
 * GEMM + reduce-scatter epilogue.
 *
 * Defined by DeepGEMM PR #1 "Fused ring RS: per-tile bitmask + drain-ring with
 * owner-boundary flush" (description: per-tile readiness replaces the
 * per-segment flag; the epilogue adds the peers' partials of the owner
 * segment) and ROCm/mori PR #662 (PR description: row-parallel wo_b GEMM fused
 * with its all-reduce).  Here the combine is the direct sum over the R-1 peers.
 *
 * One rank of R computes its full local product C = X . W (fp32 accumulate):
 *   x        bf16 [M,K]                X_r
 *   w        bf16 [K,N]                W_r (row-major [K,N])
 *   recv     HOST array of R device pointers; recv[p] is bf16 [M/R,N], peer p's
 *            partial of this rank's owner segment; recv[owner] is ignored.
 *   ready_in u32 [R][words]; bit t (word t/32, bit t%32) of peer p says flag
 *            tile t of recv[p] has landed.  Read-only, unless tile_cfg has
 *            AREPI_TILE_CONSUME_READY (then the owner-segment bits this call
 *            waited for are cleared before it ends).  Flag tiles are
 *            flag_tile_m x flag_tile_n pieces of a segment, clipped at its
 *            edges, numbered row-major; words = arepi_gemm_rs_flag_words().
 *   out      bf16 [M/R,N]: out[i,n] = bf16(C[owner*M/R + i, n] + sum over
 *            p != owner of recv[p][i,n]) (fp32 adds, round-to-nearest-even).
 *   send     bf16 [M,N] or NULL: rows outside the owner segment receive
 *            bf16(C) -- this rank's outgoing partials; owner rows untouched.
 *   ready_out u32 [R][words] or NULL (requires send): after the call every
 *            flag tile of every non-owner segment has its bit set, each set
 *            with a release at `scope` once that tile's send rows are stored.
 *   status   device u32 or NULL; spin_limit as above.
 * Owner tiles wait for their ready_in bits with an acquire at `scope`.  A
 * workgroup holding owner rows and rows of other segments stores and publishes
 * those other rows before it waits (a wait ahead of that publication could
 * close a cycle across ranks whose such workgroups wait on each other).
 * Constraints: 1 <= R <= 8, 0 <= owner < R, M % R == 0, M >= 1, N >= 8,
 * N % 8 == 0, K >= 8, K % 8 == 0, flag tiles >= 1x1.  With ready_out, flag
 * tiles must nest inside the compute tiles (see arepi_gemm_rs_supports).
 * ------------------------------------------------------------------------ */
int arepi_gemm_rs_supports(int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                           int flag_tile_n, int publish, int tile_cfg);

/* u32 words per peer of ready_in / ready_out, or a negative status. */
int64_t arepi_gemm_rs_flag_words(int64_t M, int64_t N, int R, int flag_tile_m, int flag_tile_n);

/* Compute tile (AREPI_TILE_*) the automatic choice picks for a shape, or a
 * negative status.  With AREPI_TILE_AUTO, arepi_gemm_rs_fused also applies
 * AREPI_TILE_OWNER_HALF where it can and it adds no round of workgroups
 * (at most 256 per round); passing the returned tile explicitly does not. */
int arepi_gemm_rs_pick_tile(int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                            int flag_tile_n, int publish);

/* Work assignment of arepi_gemm_rs_fused for a shape (for tests and
 * diagnostics): returns the number of workgroups W, or a negative status.  If
 * rows is non-NULL (capacity >= 6*W int64 entries), workgroup b (in launch
 * order) gets rows[6b..6b+5] = {row block, column block, first row of chunk A,
 * rows of A, first row of chunk B, rows of B}; the workgroup computes the
 * output rows of both chunks over columns [column block * BN, + BN).  Row
 * block -1 marks an owner half-height tile (AREPI_TILE_OWNER_HALF). */
int64_t arepi_gemm_rs_schedule(int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                               int flag_tile_n, int publish, int tile_cfg, int64_t *rows,
                               int64_t capacity);

int arepi_gemm_rs_fused(const uint16_t *x, const uint16_t *w, const uint16_t *const *recv,
                        uint32_t *ready_in, uint16_t *out, uint16_t *send,
                        uint32_t *ready_out, int64_t M, int64_t N, int64_t K, int R, int owner,
                        int flag_tile_m, int flag_tile_n, int scope, int tile_cfg,
                        uint32_t *status, int64_t spin_limit, arepi_stream_t stream);

/* ------------------------------------------------------------------------ *
 * GEMM + reduce-scatter epilogue, push-ring form.
 *
 * Defined by DeepGEMM PR #1 "Fused ring RS: per-tile bitmask + drain-ring with
 * owner-boundary flush" (description): the reduce-scatter runs as a ring in
 * which each rank adds its own partial tile to the running partial it
 * received from upstream and pushes the sum downstream; the owner of a segment
 * is the last rank of its chain.  Reading taken: rank r receives from r-1 and
 * sends to r+1 (mod R), so the segment this rank starts is
 * chain = (owner - 1) mod R, and partials travel as bf16.
 *
 * Arguments as for arepi_gemm_rs_fused, except:
 *   upstream HOST array of R device pointers; upstream[d] is bf16 [M/R,N], the
 *            running partial of segment d from the upstream rank;
 *            upstream[chain] is ignored (with R = 1 nothing is read).
 *   ready_in u32 [R][words]; bit t of entry d says flag tile t of upstream[d]
 *            has landed (consumed as in arepi_gemm_rs_fused with
 *            AREPI_TILE_CONSUME_READY).
 *   out      bf16 [M/R,N]: out[i,n] = bf16(C[owner*M/R + i, n] + upstream[owner][i,n]).
 *   send     bf16 [M,N], required: a row i of segment d != owner receives
 *            bf16(C[i,n] + upstream[d][i - d*M/R, n]), or bf16(C[i,n]) when
 *            d == chain (one fp32 add, then round-to-nearest-even).
 *   ready_out as for arepi_gemm_rs_fused (every segment d != owner).
 * Every tile that adds an upstream partial waits for its ready_in bits with an
 * acquire at `scope`.  Tiles run segment by segment in ring order: chain first,
 * then chain-1, ..., owner last.
 * Constraints: those of arepi_gemm_rs_fused, plus (M/R) % 8 == 0 when R > 1;
 * AREPI_TILE_PAIRED_ROWS is refused (EUNSUPPORTED).  With ready_out, every row
 * block must lie in one segment (tile rows dividing M/R): a tile publishes a
 * segment only after that segment's upstream partial arrived, so a tile over
 * two segments would hold each publication behind the other's arrival, a
 * cycle across the ranks of a ring (EUNSUPPORTED otherwise).
 * ------------------------------------------------------------------------ */
int arepi_gemm_rs_ring_supports(int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                                int flag_tile_n, int publish, int tile_cfg);

/* Compute tile (AREPI_TILE_*) the automatic choice of arepi_gemm_rs_ring
 * picks for a shape, or a negative status.  With publish set it only takes
 * tiles whose row blocks each lie in one segment (see arepi_gemm_rs_ring). */
int arepi_gemm_rs_ring_pick_tile(int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                                 int flag_tile_n, int publish);

int arepi_gemm_rs_ring(const uint16_t *x, const uint16_t *w, const uint16_t *const *upstream,
                       uint32_t *ready_in, uint16_t *out, uint16_t *send, uint32_t *ready_out,
                       int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                       int flag_tile_n, int scope, int tile_cfg, uint32_t *status,
                       int64_t spin_limit, arepi_stream_t stream);

/* ------------------------------------------------------------------------ *
 * GEMM + reduce-scatter epilogue, fp8 block-scaled local product.
 *
 * Defined by ROCm/mori PR #662, the blockscale commit (X quantised 1x128 along
 * K, W 128x128, fp32 scales; the scales vary along K, so the local product is
 * sum over K blocks b of xs[m,b] * ws[n/128,b] * d_b with d_b the fp8 product
 * of block b; applied with the running rescale t_b = t_{b-1}*(s_{b-1}/s_b) +
 * d_b, out = t_last * s_last), and by its re-review finding that the gfx950
 * matrix atom reads OCP e4m3fn bytes.
 *   x   e4m3fn bytes [M,K]            X_r
 *   xs  fp32 [M][K/128]               row-major, finite
 *   wt  e4m3fn bytes [N,K]            W_r TRANSPOSED (K contiguous)
 *   ws  fp32 [ceil(N/128)][K/128]     row-major, finite
 * A zero scale is accepted for a block whose fp8 data are all zero (what a
 * quantiser emits for an all-zero block, e.g. padding rows): the block adds
 * nothing, and the running rescale carries the previous non-zero scale
 * across it.  A zero scale over non-zero data, and non-finite scales, give
 * unspecified outputs.
 * The reduce-scatter epilogue and every other argument are those of
 * arepi_gemm_rs_fused (direct sum over the R-1 peers).  The compute tile is
 * 256x256 (tile_cfg may only carry AREPI_TILE_CONSUME_READY; with ready_out,
 * flag tiles must nest inside 256x256 tiles).  Constraints:
 * those of arepi_gemm_rs_fused plus K % 128 == 0; xs 4-byte aligned.
 * e4m3fnuz bytes are not this encoding (the same bits decode to other values).
 * ------------------------------------------------------------------------ */
int arepi_gemm_rs_fp8_supports(int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                               int flag_tile_n, int publish, int tile_cfg);

int arepi_gemm_rs_fp8(const uint8_t *x, const float *xs, const uint8_t *wt, const float *ws,
                      const uint16_t *const *recv, uint32_t *ready_in, uint16_t *out, uint16_t *send,
                      uint32_t *ready_out, int64_t M, int64_t N, int64_t K, int R, int owner,
                      int flag_tile_m, int flag_tile_n, int scope, int tile_cfg, uint32_t *status,
                      int64_t spin_limit, arepi_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Lamport all-reduce + RMSNorm.
 *
 * Defined by ROCm/aiter PR #4977 "[HIP] Single-kernel Lamport fused all-reduce
 * + RMSNorm (opt-in)", Approach section: staging is armed with -0.0 (bf16
 * 0x8000); producers map -0.0 to +0.0 before storing; a consumer treats a
 * 16-byte pack as arrived only when none of its words is 0x8000, consumes it
 * and re-arms it.  The staging area is private to these calls.
 * ------------------------------------------------------------------------ */

/* Arm: write 0x8000 into every one of `elems` bf16 words of staging.  Call once
 * before first use, outside any graph capture (after that the consumer keeps
 * the area armed). */
int arepi_lamport_prefill(uint16_t *staging, int64_t elems, arepi_stream_t stream);

/* Emulated producers for one GPU: for each slot s < S, copy src[s] (bf16
 * [M,N]) into staging[s] one tile_m x tile_n tile at a time, in the order
 * order[s][0..tiles-1] (device int32, a permutation of the row-major tile
 * ids), canonicalising every 0x8000 word to 0x0000 and storing with
 * device-coherent stores at `scope`.  No fence: the data is the flag.
 * src and staging are [S][M][N]. */
int arepi_lamport_publish(const uint16_t *src, uint16_t *staging, const int32_t *order, int S,
                          int64_t M, int64_t N, int tile_m, int tile_n, int scope,
                          arepi_stream_t stream);

/* Consumer: staging [S][M][N] (armed, being or already published), gamma bf16
 * [N], out bf16 [M,N].  Per row i: s = sum over slots 0..S-1 (fp32) once each
 * pack has arrived; out = bf16(s * (1/sqrt(mean(s^2) + eps)) * gamma).  Every
 * consumed pack is re-armed, so staging is all 0x8000 again on return.
 * Constraints: 1 <= S <= 8, N % 8 == 0, 8 <= N <= 16384. */
int arepi_ar_rmsnorm_lamport(uint16_t *staging, const uint16_t *gamma, uint16_t *out, int64_t M,
                             int64_t N, int S, float eps, int scope, uint32_t *status,
                             int64_t spin_limit, arepi_stream_t stream);

/* Largest staging (S*M*N*2 bytes) of arepi_ar_rmsnorm_lamport_noalloc: 32 MiB,
 * e.g. S = 8 slots of up to 292 rows at N = 7168. */
#define AREPI_LAMPORT_NOALLOC_BYTES (32LL * 1024 * 1024)

/* The consumer above with the staging held by the library, for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation).  The staging is a static device
 * array of AREPI_LAMPORT_NOALLOC_BYTES, one per GPU, laid out as [S][M][N]
 * for the M, N, S of each call.  The call allocates nothing and calls no
 * allocating routine.
 *   - The first call on a device (with that device current) resolves the
 *     array's address and arms all of it with 0x8000 by a fill kernel on
 *     `stream`; make that first call outside graph capture (M = 0 does only
 *     this) and order it before any publication into the array.
 *   - When `staging` is non-NULL it receives the array's device address on the
 *     current device: producers publish into it (arepi_lamport_publish, or a
 *     peer's stores) exactly as into a caller-owned staging.
 *   - Every call on one GPU shares that GPU's array and it keeps the last
 *     call's contents: the consumer re-arms every pack it consumes, so it is
 *     armed again after a call that did not time out.  After a time-out re-arm
 *     it with arepi_lamport_prefill on the returned address.  Calls that
 *     overlap on one GPU (two streams, two threads) race on the array.
 * gamma, out, M, N, S, eps, scope, status, spin_limit are as in
 * arepi_ar_rmsnorm_lamport.  S*M*N*2 above AREPI_LAMPORT_NOALLOC_BYTES is
 * refused with AREPI_EUNSUPPORTED before anything is launched. */
int arepi_ar_rmsnorm_lamport_noalloc(const uint16_t *gamma, uint16_t *out, int64_t M, int64_t N, int S,
                                     float eps, int scope, uint32_t *status, int64_t spin_limit,
                                     uint16_t **staging, arepi_stream_t stream);

/* Two-phase form (same page, Approach: "phase A" is the reduce-scatter with
 * cross-device stores, "phase B" the consumer; Correctness notes: every block
 * finishes its producer work before it polls, and the grid is clamped to the
 * workgroups that can be resident at once).  R ranks each hold a partial
 * inputs[r] (bf16 [M,N]); every rank has a private staging[r] (bf16 [M,N],
 * armed with arepi_lamport_prefill).  One call on rank `rank`:
 *   phase A: the flattened tensor is cut into R parts of ceil(M*N/8/R) 16-byte
 *     packs; for each pack of part `rank`, T = bf16(sum over r of inputs[r])
 *     (fp32, ranks ascending, round-to-nearest-even), 0x8000 words mapped to
 *     0x0000, stored into EVERY staging[d] with device-coherent stores at
 *     `scope` (no fence: the data is the flag);
 *   phase B: every pack of staging[rank] is waited for (it arrives from the
 *     phase A of the rank owning its part), re-armed, and per row
 *     out = bf16(T * (1/sqrt(mean(T^2) + eps)) * gamma).
 * HOST arrays inputs/staging hold R device pointers.  staging[rank] is all
 * 0x8000 again on return; the other ranks' staging receive part `rank`.
 * Ordering between calls (a peer's phase A of the next call must not land
 * before this call has re-armed) is the caller's: on one GPU stream order, or
 * an event between the calls.  Constraints: 1 <= R <= 8, 0 <= rank < R,
 * N % 8 == 0, 8 <= N <= 16384, M*N*2 < 2 GiB.  Waits are bounded by
 * spin_limit (AREPI_STATUS_TIMEOUT in *status). */
int arepi_ar_rmsnorm_lamport_2phase(const uint16_t *const *inputs, uint16_t *const *staging,
                                    const uint16_t *gamma, uint16_t *out, int64_t M, int64_t N, int R,
                                    int rank, float eps, int scope, uint32_t *status,
                                    int64_t spin_limit, arepi_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Weighted top-k combine.
 *
 * The expert-output reduction of DeepEP's intranode combine (DeepEP PR #527,
 * "Fix the MultiStages for intranode combine": a multi-stage pipeline whose
 * stages are issued and waited on independently):
 *   out[t,h] = bf16( sum_{k<E} gate[t,k] * x[t,k,h] )    (fp32 accumulate)
 *   x bf16 [T,E,H], gate fp32 [T,E], out bf16 [T,H].
 * Constraints: 1 <= E <= 16, H % 8 == 0.  This entry point streams the
 * expert rows through registers (two work units in flight per thread,
 * nontemporal loads and stores).
 * ------------------------------------------------------------------------ */
int arepi_combine_reduce(const uint16_t *x, const float *gate, uint16_t *out, int64_t T, int E,
                         int64_t H, arepi_stream_t stream);

/* The same combine through the LDS-staged pipeline: each wave owns S stages of
 * E x 1 KiB filled by direct-to-LDS loads and waits for one stage at a time
 * (the stage-per-issuer structure of the DeepEP fix above).  Same arguments,
 * constraints and results as arepi_combine_reduce (identical bits: both add
 * the experts in ascending order with the same fused multiply-adds). */
int arepi_combine_reduce_lds(const uint16_t *x, const float *gate, uint16_t *out, int64_t T, int E,
                             int64_t H, arepi_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Test-only peer emulation on one GPU (prefixed emu_ so it is never mistaken
 * for the method).  For each item j < n_items, order[j] = (peer p, flag tile
 * t): copy flag tile t of src[p] (bf16 [M/R,N]) into recv[p], then set bit t
 * of ready_in[p] with a release at `scope`.  src and recv are HOST arrays of R
 * device pointers (entry `owner` ignored); ready_in must be zero beforehand.
 * Items go in batches of items_per_release consecutive entries of order: a
 * batch's tiles are copied, then one release at `scope` precedes the batch's
 * bits (1 = a release per tile).  workgroups = 0 lands every batch at once
 * (one workgroup each); workgroups = G > 0 lands them G at a time, in order,
 * which paces the arrivals like a link of bounded rate and leaves the other
 * compute units to the consumer.
 * resident: NULL, or a device uint32 [2] (zero before first use) through
 * which every producer workgroup announces its start, for
 * arepi_emu_producer_gate.
 * Errors: EINVAL for bad shapes, NULL pointers, workgroups < 0 or
 * items_per_release < 1.
 * ------------------------------------------------------------------------ */
int arepi_emu_peer_producer(const uint16_t *const *src, uint16_t *const *recv, uint32_t *ready_in,
                            const int32_t *order, int64_t n_items, int64_t M, int64_t N, int R,
                            int owner, int flag_tile_m, int flag_tile_n, int scope, int workgroups,
                            int items_per_release, uint32_t *resident, arepi_stream_t stream);

/* Test-only: the emulated peers of `steps` consecutive consumer calls in one
 * launch, so that the producer is resident once for all of them.  Step s
 * lands the n_items items of orders[s % n_orders] (device int32
 * [n_orders][n_items][2]) exactly as arepi_emu_peer_producer does, copying
 * from src[p] + (s % n_orders) * src_step elements (src_step >= 0, a multiple
 * of 8; 0: the same partials every step).  go: device uint32, 0 before the
 * launch.  Pacing, one of two:
 *   credit = 0 (signals): step s starts once *go >= s; the consumer's stream
 *     raises it with arepi_emu_signal(go, s, ...) once the consumer of step
 *     s-1 has ended and no longer reads recv or ready_in;
 *   credit = 1: go is the producer's own count of landed (workgroup, step)
 *     pairs; step s starts once every producer workgroup has landed step
 *     s-1, and then each batch waits until the ready_in bits of its items are
 *     clear, i.e. consumed.  The consumer must pass AREPI_TILE_CONSUME_READY,
 *     whose owner tiles clear a bit only after the tile's data has been
 *     read, so a slot is refilled as soon as it is free and no signal is
 *     needed between consumer calls.
 * The consumer of step s-1 needs nothing from step s, so every wait ends;
 * each is bounded by spin_limit (encoding above), and on expiry the producer
 * ORs AREPI_STATUS_TIMEOUT into *status (status may be NULL) and stops.
 * Issue it with `resident` and arepi_emu_producer_gate before the first
 * consumer.  Errors: those of arepi_emu_peer_producer, plus go NULL, credit
 * not 0 or 1, steps < 1, n_orders < 1, a bad src_step, or (credit = 1)
 * steps x launched workgroups reaching 2^32. */
int arepi_emu_peer_producer_steps(const uint16_t *const *src, uint16_t *const *recv, uint32_t *ready_in,
                                  const int32_t *orders, int n_orders, int64_t n_items, int64_t M, int64_t N,
                                  int R, int owner, int flag_tile_m, int flag_tile_n, int scope, int workgroups,
                                  int items_per_release, uint32_t *resident, uint32_t *go, int credit,
                                  int steps, int64_t src_step, uint32_t *status, int64_t spin_limit,
                                  arepi_stream_t stream);

/* Test-only: a stream with a hardware queue of its own, for the emulated
 * producer.  The HIP runtime hands ordinary streams out of a small pool of
 * hardware queues, so two of them may share one, and a queue runs its
 * kernels in order; a stream created with a compute-unit mask gets a queue
 * that is never pooled.  The mask here enables every compute unit.  Default
 * priority.  Destroy with arepi_emu_stream_destroy. */
int arepi_emu_stream_create(arepi_stream_t *stream);
int arepi_emu_stream_destroy(arepi_stream_t stream);

/* Test-only: one thread stores `value` into *flag (device uint32, relaxed,
 * agent scope) once everything issued before it on `stream` has ended. */
int arepi_emu_signal(uint32_t *flag, uint32_t value, arepi_stream_t stream);

/* Test-only forward-progress gate for a consumer that waits on the emulated
 * producer on the same GPU (the aiter PR #4977 Correctness notes: producer
 * work must not be left unscheduled behind spinning consumers).  Launch it on
 * the consumer's stream after the producer (issued with the same `resident`)
 * and before the consumer: one wave waits until every producer workgroup has
 * started, then zeroes resident for the next step.  The producer waits only
 * for consumers of earlier steps (or, within one call, not at all), which
 * need nothing from it, so once resident it finishes, whatever registers the
 * consumer's workgroups take.  Issue the producer first in host order: when the two
 * streams share one hardware queue, the queue then runs producer, gate and
 * consumer in turn.  The next producer on the same `resident` must be
 * ordered after this gate.  The wait is bounded by spin_limit (encoding as
 * above); on expiry AREPI_STATUS_TIMEOUT is ORed into *status (status may be
 * NULL) and resident is left as it is. */
int arepi_emu_producer_gate(uint32_t *resident, uint32_t *status, int64_t spin_limit,
                            arepi_stream_t stream);

/* Test-only: phase A of the two-phase Lamport call for rank `rank` alone
 * (stands in for a peer GPU's phase A on one GPU).  Same arguments and
 * constraints as arepi_ar_rmsnorm_lamport_2phase; never waits. */
int arepi_emu_lamport_phase_a(const uint16_t *const *inputs, uint16_t *const *staging, int64_t M,
                              int64_t N, int R, int rank, int scope, arepi_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* AREPI_H */
