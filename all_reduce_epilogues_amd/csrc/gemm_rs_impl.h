// gemm_rs_impl.h -- shared body of the GEMM + reduce-scatter kernels for gfx950
// (direct-sum form in gemm_rs.hip, push-ring form in gemm_rs_ring.hip).
//
// What it computes follows DeepGEMM PR #1 "Fused ring RS: per-tile bitmask +
// drain-ring with owner-boundary flush" (description) and ROCm/mori PR #662
// (PR description, fused GEMM + all-reduce of the wo_b projection), in the
// direct-sum form: each rank computes its full local product C = X.W; the owner
// segment's tiles add the R-1 peer partials in the epilogue, all other rows are
// stored as this rank's outgoing partials.
//
// Design (gfx950, not a translation of the pages' sm100 / FlyDSL kernels):
//  * Workgroup tile BM x BN of 4 or 8 waves, each wave a WM x WN block of
//    32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16, fp32 accumulators).  The
//    8-wave 256x256 tile runs two waves per SIMD: one wave issues MFMAs while
//    the other waits on its loads.
//  * K is walked in BK-wide steps through an S-stage LDS ring filled by
//    direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds, issued as inline
//    asm so the compiler adds no waits of its own); a stage is read only after
//    an exact vmcnt wait and a barrier.  Out-of-range offsets zero-fill the
//    M, N and K tails.  With S >= 3 a step's loads are spread between its MFMA
//    groups instead of being issued as one burst.
//  * X [M,K] is K-contiguous in LDS and read with 16-byte swizzled reads.  W
//    [K,N] stays N-contiguous in LDS and is read with the gfx950 transpose
//    read (ds_read_b64_tr_b16), which yields the B-operand layout directly.
//    MFMAs and operand reads of the next sub-step are interleaved with
//    scheduling groups.
//  * Rows: a row block is two half-blocks (chunks) of BM/2 rows, interleaved
//    between the wave rows.  Optionally (AREPI_TILE_PAIRED_ROWS) an owner
//    half-block is paired with a non-owner one; or (AREPI_TILE_OWNER_HALF)
//    the owner rows run as half-height tiles of the same waves after all the
//    other workgroups.
//  * Epilogue, chosen per workgroup at entry (no-owner / owner-chunk-A /
//    owner-rows-anywhere bodies): accumulators go through LDS one 32-row slab
//    at a time and come back row-contiguous; owner rows wait for their peers'
//    flag-tile bits (one lane per (peer, tile), relaxed polls, one acquire),
//    add the peers' packs (fetched several units ahead with row-coalesced
//    loads, ascending rank order, fp32) and store to `out`; other rows are
//    stored to `send`.  With consumption, an owner tile clears the bits it
//    waited for at its end, once every load of the data under them has
//    returned.  Stores are buffer stores whose out-of-range offsets
//    drop lanes, so the code has no data-dependent branches around memory
//    operations.  No per-tile drain on `out` (the kernel end is its release);
//    a drain + balanced barrier + one release precede the ready_out bits.
//  * Tile order: row blocks rotated so the owner segment comes last (the
//    destination-rotated order of the mori page's tile-order commit), grouped
//    G row blocks at a time, and remapped so that the blocks one XCD runs
//    together are neighbours (shared X rows / W columns in that XCD's L2).
#ifndef AREPI_GEMM_RS_IMPL_H
#define AREPI_GEMM_RS_IMPL_H

#include <algorithm>
#include <string>

#include "arepi_internal.h"

namespace arepi {
namespace {


constexpr int kMaxR = 8;
constexpr int kXcds = 8;

struct GemmRsParams {
    const uint16_t *x;
    const uint16_t *w;
    const uint16_t *peer[kMaxR - 1];  // peer partials in ascending rank order, owner skipped
    int npeers;                       // R - 1
    uint32_t *ready_in;
    uint16_t *out;
    uint16_t *send;
    uint32_t *ready_out;
    uint32_t *status;
    int64_t M, N, K, seg;
    int64_t ftiles_n;  // flag tiles per segment row band
    int64_t fwords;    // u32 words per peer
    int64_t spin_limit;  // bound of each wait: > 0 polls, < 0 ticks of the wall clock
    int R, owner, ftm, ftn;
    int system_scope;
    int nRB, nCB, ob1, group, xcd_chunk, nWG;
    // Owner half-height tiles (contiguous layout only): the owner segment's
    // row blocks are not among the nRB scheduled by tile_of_block (nrot is
    // the count the rotation runs over, nRB + the owner's blocks); instead
    // nextra workgroups after the nWG others each take BM/2 owner rows of one
    // column block, so the owner tiles' peer reads are split over twice as
    // many workgroups.  nextra = 0 otherwise, and nrot = nRB.
    int nrot, nextra;
    // Row blocks are two chunks of CK rows (A, B).  Contiguous: block b is rows
    // [b*BM, (b+1)*BM).  Paired (seg a multiple of CK, R >= 2): chunks never
    // straddle a segment; the first npure blocks pair two non-owner chunks, the
    // next nleft (0/1) hold one non-owner chunk, the last nc pair owner chunk i
    // with a non-owner chunk, so the owner rows' peer reads are spread over nc
    // row blocks instead of seg/BM.
    int paired, nc, npure, nleft;
    int consume;  // owner tiles clear the ready_in bits they waited for
    // Push-ring form only: up[d] is the running partial of segment d received
    // from the upstream rank (up[chain] unused), chain = (owner - 1) mod R is
    // the segment this rank starts, and row blocks run in descending order
    // from the chain segment's last one (ob1), so the owner segment is last.
    const uint16_t *up[kMaxR];
    int ring, chain;
    // fp8 block-scaled form only: x and w hold e4m3fn bytes, X [M,K] and W
    // transposed [N,K]; xs [M][K/128] and ws [ceil(N/128)][K/128] fp32 scales
    const float *xs, *ws;
};


typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// X tile rows are BK*2 bytes (CH = BK/8 chunks of 16 bytes); chunk c of row r
// sits at c ^ ((r / (16/CH)) % CH): the 16 consecutive rows that one 16-lane
// group reads at one logical chunk hit 16 distinct 16-byte bank groups.
template <int CH>
__device__ __forceinline__ int swz_a(int r) { return (r / (16 / CH)) % CH; }
// W tile rows are BN*2 bytes (BN/8 chunks); chunk c of row k sits at
// c ^ (4 * (k & 3)): the four rows and four chunks one transpose read touches
// per 16-lane group land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz_b(int k) { return 4 * (k & 3); }

// s_waitcnt vmcnt(0) with a memory clobber (the compiler neither drops it nor
// moves memory operations across it).
__device__ __forceinline__ void wait_vmcnt_zero() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void drain_stores() { wait_vmcnt_zero(); }
// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt and
// lgkmcnt left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}


// Raw buffer resource (base, no stride, num_records bytes, gfx9 word 3).
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    i32x4 r = {(int)(uint32_t)b, (int)(uint32_t)(b >> 32), (int)bytes, kBufferDword3};
    return r;
}

// 16-byte direct-to-LDS load: lane i's 16 bytes from rsrc + voff + soff land
// at LDS byte lds_base + 16*i.  Issued as asm so the compiler does not add
// its own conservative waits between these loads and LDS reads; every stage
// is drained explicitly (wait_vmcnt_zero + barrier) before it is read.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_base, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// Rows of a chunk that starts at `first` and holds at most CK rows.
__host__ __device__ __forceinline__ int rows_left(int64_t M, int64_t first, int CK) {
    const int64_t n = M - first;
    return n <= 0 ? 0 : n < CK ? (int)n : CK;
}

// Global first row and row count of the two chunks of row block rb (shared by
// the kernel and the host-side schedule query).
__host__ __device__ __forceinline__ void chunks_of_block(const GemmRsParams &p, int BM, int CK, int rb, int64_t &a0,
                                                         int &alen, int64_t &b0, int &blen) {
    if (!p.paired) {
        a0 = (int64_t)rb * BM;
        b0 = a0 + CK;
        alen = rows_left(p.M, a0, CK);
        blen = CK < BM ? rows_left(p.M, b0, CK) : 0;
        return;
    }
    // non-owner chunk j: segment owner+1+j/nc (mod R), chunk j%nc of it
    auto other = [&](int j) { return (int64_t)((p.owner + 1 + j / p.nc) % p.R) * p.seg + (int64_t)(j % p.nc) * CK; };
    const int tail = (p.R - 2) * p.nc;  // non-owner chunks before the ones paired with owner chunks
    alen = blen = CK;
    if (rb < p.npure) {
        a0 = other(2 * rb);
        b0 = other(2 * rb + 1);
    } else if (rb < p.npure + p.nleft) {
        a0 = other(tail - 1);
        b0 = 0;
        blen = 0;
    } else {
        const int i = rb - p.npure - p.nleft;
        a0 = (int64_t)p.owner * p.seg + (int64_t)i * CK;
        b0 = other(tail + i);
    }
}

__host__ __device__ __forceinline__ void tile_of_block(const GemmRsParams &p, int b, int &rb, int &cb) {
    // XCD-aware remap inside rounds of 8*C blocks: consecutive schedule
    // entries land on the same XCD (blocks are dealt to XCDs round-robin), so
    // the blocks one XCD runs share X rows and W columns in its L2.  A last,
    // partial round of 8*C' blocks is remapped the same way with C' in place
    // of C (left in order when its size is not a multiple of 8).
    const int C = p.xcd_chunk;
    const int round = kXcds * C;
    int s = b;
    const int r = b / round, j = b % round;
    const int in_round = min(round, p.nWG - r * round);  // blocks of b's round
    if (in_round % kXcds == 0) s = r * round + (j % kXcds) * (in_round / kXcds) + j / kXcds;
    // G row blocks at a time, column-major inside the group.
    const int per_group = p.group * p.nCB;
    const int g = s / per_group, within = s % per_group;
    const int gsz = p.group < p.nRB - g * p.group ? p.group : p.nRB - g * p.group;
    const int pos = g * p.group + within % gsz;
    cb = within / gsz;
    // rotated so that the owner's row blocks come last: ascending from the
    // block after the owner's (direct sum; with owner half-height tiles the
    // owner's blocks are past the nRB positions and never reached), descending
    // from the chain segment's last block (push ring: the order in which a
    // ring hands the segments on)
    rb = p.ring ? (p.ob1 - pos % p.nRB + p.nRB) % p.nRB : (p.ob1 + pos) % p.nrot;
}

// Workgroup b >= nWG of the owner half-height tiles: half-block h of the
// owner segment (BM/2 rows from owner*seg + h*BM/2), column block cb.  The
// half-blocks of one column block are consecutive entries, and the entries
// are remapped as tile_of_block remaps a round (when their count is a
// multiple of 8), so that consecutive entries land on one XCD and share its
// L2's copy of the W column block.
__host__ __device__ __forceinline__ void owner_half_of_block(const GemmRsParams &p, int b, int &h, int &cb) {
    const int j = b - p.nWG, nh = p.nextra / p.nCB;
    const int s = p.nextra % kXcds == 0 ? (j % kXcds) * (p.nextra / kXcds) + j / kXcds : j;
    h = s % nh;
    cb = s / nh;
}

// LDS bytes of one workgroup: S stages of [X tile | W tile].
template <int BM, int BN, int BK, int S>
constexpr int lds_bytes() { return S * (BM * BK * 2 + BK * BN * 2); }

// Kinds of workgroup, fixed at entry so that each body has straight-line code
// around the accumulators (a conditional update of them makes the compiler copy
// all of them through vector registers).
// kRing: push-ring form, every row outside the chain segment adds the
// upstream partial of its own segment.
// kOwnerChunkAPub, kOwnerAnywherePub: as kOwnerChunkA / kOwnerRowsAnywhere for
// a tile that also holds rows of other segments and publishes them
// (ready_out): those rows are stored and published before the readiness wait.
enum {
    kNoOwnerRows = 0,
    kOwnerChunkA = 1,
    kOwnerRowsAnywhere = 2,
    kRing = 3,
    kOwnerChunkAPub = 4,
    kOwnerAnywherePub = 5
};

template <int BM, int BN, int WM, int WN, int BK, int S, int WPE, int PEERS, int KIND, bool FP8 = false>
__device__ __forceinline__ void gemm_rs_body(const GemmRsParams &p, uint8_t *smem, int rb, int cb, int64_t a0,
                                             int alen, int64_t b0, int blen) {
    constexpr int NWN = BN / WN;
    constexpr int NW = (BM / WM) * NWN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int CH = BK / 8;                    // 16-byte chunks per X row in LDS
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;  // one stage
    constexpr int A_INSTR = A_BYTES / 1024 / NW;  // 1 KiB direct-to-LDS loads per wave and step
    constexpr int B_INSTR = B_BYTES / 1024 / NW;
    constexpr int NDMA = A_INSTR + B_INSTR;
    constexpr int A_RPI = 64 / CH;                // X rows per load instruction
    constexpr int B_CPR = BN / 8;                 // 16-byte chunks per W row in LDS
    constexpr int B_RPI = 64 / B_CPR;             // W rows per load instruction
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int LDS_BYTES = S * STAGE;
    constexpr int EPS = WN + 8;                   // epilogue LDS row stride (floats)
    // epilogue slab rows: the largest of 32/16/8 whose per-wave fp32 slabs fit the stages
    constexpr int ER = (NW * 32 * EPS * 4 <= LDS_BYTES) ? 32 : (NW * 16 * EPS * 4 <= LDS_BYTES) ? 16 : 8;
    static_assert(CH == 4 || CH == 8, "BK must be 32 or 64");
    static_assert(A_INSTR >= 1 && A_INSTR * NW * 1024 == A_BYTES, "X stage split");
    static_assert(B_INSTR >= 1 && B_INSTR * NW * 1024 == B_BYTES, "W stage split");
    static_assert(B_CPR >= 16 && B_CPR <= 64, "W swizzle needs 16..64 chunks per row");
    static_assert(NW * ER * EPS * 4 <= LDS_BYTES, "epilogue slabs must fit the stage memory");
    static_assert(S >= 2 && (S - 2) * NDMA < 64, "stage count vs vmcnt range");

    static_assert(LDS_BYTES == lds_bytes<BM, BN, BK, S>(), "stage layout");
    // S stages [X | W] x S (in `smem`); the epilogue reuses the same memory.
    typedef __attribute__((address_space(3))) uint8_t lds_t;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    (void)rb;
    const int64_t n0 = (int64_t)cb * BN;
    const int64_t M = p.M, N = p.N, K = p.K;
    // The tile's BM rows are two chunks A and B of CK rows, interleaved in
    // blocks of IL rows so that every wave row holds as many rows of A as of B
    // (an owner chunk's epilogue work is shared by all waves).
    constexpr int IL = BM >= 64 ? (WM >= 64 ? WM / 2 : WM) : BM;
    constexpr int CK = BM >= 64 ? BM / 2 : BM;
    static_assert(BM < 64 || (BM / (2 * IL)) * IL == CK, "chunk interleave");
    // global row of tile row v, or -1 past the end of its chunk
    auto row_of = [&](int v) -> int64_t {
        const int idx = (v / (2 * IL)) * IL + v % IL;
        return ((v / IL) & 1) ? (idx < blen ? b0 + idx : -1) : (idx < alen ? a0 + idx : -1);
    };

    // Buffer resources over X and W: a load whose offset is out of range
    // returns zeros, which fills the M, N and K tails without branches.
    const i32x4 xr = buffer_rsrc(p.x, (uint32_t)(M * K * 2));
    const i32x4 wr = buffer_rsrc(p.w, (uint32_t)(K * N * 2));
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy for LDS bases
    constexpr uint32_t kOob = 0x80000000u;

    // Per-lane source of each load.  X: instruction i covers A_RPI rows of the
    // stage; lane -> (row, physical chunk) and loads the logical chunk the
    // read-side swizzle expects.  W: instruction i covers B_RPI rows.  The
    // per-lane byte offset is fixed for the whole K loop (rows/columns past M
    // or N get an out-of-range offset); k0 goes into the scalar offset.
    auto a_row_of = [&](int i) { return (wave * A_INSTR + i) * A_RPI + lane / CH; };
    auto a_col_of = [&](int i) { return ((lane % CH) ^ swz_a<CH>(a_row_of(i))) * 8; };
    auto b_row_of = [&](int i) { return (wave * B_INSTR + i) * B_RPI + lane / B_CPR; };
    uint32_t a_off[A_INSTR], b_off[B_INSTR];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
        const int64_t gm = row_of(a_row_of(i));
        a_off[i] = (gm >= 0) ? (uint32_t)((gm * K + a_col_of(i)) * 2) : kOob;
    }
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
        const int r = b_row_of(i);
        const int64_t gn = n0 + ((lane % B_CPR) ^ swz_b(r)) * 8;
        b_off[i] = (gn < N) ? (uint32_t)((r * N + gn) * 2) : kOob;
    }
    const int64_t w_kstride = N * 2;  // bytes of W per k
    auto b_k_of = [&](int i) { return b_row_of(i); };

    lds_t *const S0 = (lds_t *)smem;
    auto lds_addr = [](const lds_t *ptr) { return (uint32_t)(uintptr_t)ptr; };
    const int KT = (int)((K + BK - 1) / BK);
    // Loads of K step kt into stage kt % S.  Every call issues exactly NDMA
    // instructions per wave (steps past the end load nothing but zeros, with
    // out-of-range offsets) so the vmcnt arithmetic below is uniform.
    auto issue_step = [&](int kt) {
        const lds_t *st = S0 + (kt % S) * STAGE;
        const uint32_t la = lds_addr(st) + wave_u * A_INSTR * 1024;
        const uint32_t lb = lds_addr(st + A_BYTES) + wave_u * B_INSTR * 1024;
        const int64_t k0 = (int64_t)kt * BK;
        if (k0 + BK <= K) {  // full step: precomputed offsets, k0 in soffset
            const uint32_t sa = (uint32_t)(k0 * 2), sb = (uint32_t)(k0 * w_kstride);
#pragma unroll
            for (int i = 0; i < A_INSTR; ++i) dma16(xr, la + i * 1024, a_off[i], sa);
#pragma unroll
            for (int i = 0; i < B_INSTR; ++i) dma16(wr, lb + i * 1024, b_off[i], sb);
        } else {  // partial or past-the-end step: every lane checks its own k
#pragma unroll
            for (int i = 0; i < A_INSTR; ++i) {
                const bool in = a_off[i] != kOob && k0 + a_col_of(i) < K;
                dma16(xr, la + i * 1024, in ? a_off[i] + (uint32_t)(k0 * 2) : kOob, 0);
            }
#pragma unroll
            for (int i = 0; i < B_INSTR; ++i) {
                const bool in = b_off[i] != kOob && k0 + b_k_of(i) < K;
                dma16(wr, lb + i * 1024, in ? b_off[i] + (uint32_t)(k0 * w_kstride) : kOob, 0);
            }
        }
    };
    // The same loads one instruction at a time (d < NDMA), so that they can be
    // spread between the MFMAs of a step.
    struct StepLoads {
        uint32_t la, lb, sa, sb;
        int64_t k0;
        bool full;
    };
    auto step_loads = [&](int kt) {
        const lds_t *st = S0 + (kt % S) * STAGE;
        StepLoads sl;
        sl.la = lds_addr(st) + wave_u * A_INSTR * 1024;
        sl.lb = lds_addr(st + A_BYTES) + wave_u * B_INSTR * 1024;
        sl.k0 = (int64_t)kt * BK;
        sl.full = sl.k0 + BK <= K;
        sl.sa = sl.full ? (uint32_t)(sl.k0 * 2) : 0u;
        sl.sb = sl.full ? (uint32_t)(sl.k0 * w_kstride) : 0u;
        return sl;
    };
    auto issue_one = [&](const StepLoads &sl, int d) {
        if (d < A_INSTR) {
            const int i = d;
            const bool in = a_off[i] != kOob && sl.k0 + a_col_of(i) < K;
            const uint32_t vo = sl.full ? a_off[i] : in ? a_off[i] + (uint32_t)(sl.k0 * 2) : kOob;
            dma16(xr, sl.la + i * 1024, vo, sl.sa);
        } else {
            const int i = d - A_INSTR;
            const bool in = b_off[i] != kOob && sl.k0 + b_k_of(i) < K;
            const uint32_t vo = sl.full ? b_off[i] : in ? b_off[i] + (uint32_t)(sl.k0 * w_kstride) : kOob;
            dma16(wr, sl.lb + i * 1024, vo, sl.sb);
        }
    };
    // wait until this wave's loads of the oldest outstanding step have landed,
    // leaving the S-2 younger steps in flight
    auto wait_oldest_step = [&]() { wait_vmcnt<(S - 2) * NDMA>(); };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    // MFMA operands: X rows with 16-byte swizzled reads; W columns with the
    // gfx950 transpose read -- in each 16-lane group, lane (4a+b) receives
    // element b of the 8-byte rows read by lanes a, a+4, a+8, a+12, so lanes
    // that read 4 consecutive n of rows k..k+3 end up holding 4 consecutive k
    // of one column, the B-operand layout.
    const int g16 = lane >> 4, s16 = lane & 15;
    const int b_n_lane = 16 * (g16 & 1) + 4 * (s16 & 3);  // n offset of this lane's 8-byte read
    const int b_k_lane = 8 * (g16 >> 1) + (s16 >> 2);     // k offset (+4 for the upper half)
    struct Frag {
        bf16x8 a[TM], b[TN];
    };
    auto load_frag = [&](const lds_t *As, int kk, Frag &f) {
        const lds_t *Bs = As + A_BYTES;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * WM + i * 32 + (lane & 31);
            const int c = kk * 2 + (lane >> 5);
            f.a[i] = *(const __attribute__((address_space(3))) bf16x8 *)(As + r * (BK * 2) + ((c ^ swz_a<CH>(r)) << 4));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = wn * WN + j * 32 + b_n_lane;
            bf16x4 h[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int k = kk * 16 + b_k_lane + 4 * half;
                const lds_t *src = Bs + k * (BN * 2) + (((n >> 3) ^ swz_b(k)) << 4) + (n & 7) * 2;
                h[half] = __builtin_bit_cast(
                    bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)src));
            }
            f.b[j] = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    // Operand reads of piece pc (of TM): A row block pc and the W columns j
    // with j*TM/TN == pc.
    auto load_frag_piece = [&](const lds_t *As, int kk, Frag &f, int pc) {
        const lds_t *Bs = As + A_BYTES;
        {
            const int i = pc;
            const int r = wm * WM + i * 32 + (lane & 31);
            const int c = kk * 2 + (lane >> 5);
            f.a[i] = *(const __attribute__((address_space(3))) bf16x8 *)(As + r * (BK * 2) + ((c ^ swz_a<CH>(r)) << 4));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            if ((j * TM) / TN != pc) continue;
            const int n = wn * WN + j * 32 + b_n_lane;
            bf16x4 h[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int k = kk * 16 + b_k_lane + 4 * half;
                const lds_t *src = Bs + k * (BN * 2) + (((n >> 3) ^ swz_b(k)) << 4) + (n & 7) * 2;
                h[half] = __builtin_bit_cast(
                    bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)src));
            }
            f.b[j] = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    auto reads_in_piece = [](int pc) {
        int n = 1;
        for (int j = 0; j < TN; ++j) n += ((j * TM) / TN == pc) ? 2 : 0;
        return n;
    };
    auto mma_row = [&](const Frag &f, int i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    };
    auto mma = [&](const Frag &f) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    };
    // Scheduling groups: after each MFMA one LDS operand read, so the reads of
    // the next sub-step overlap the MFMAs of the current one (the compiler's
    // default is to drain each read right before its first use).
    constexpr int NREAD = TM + 2 * TN;  // LDS reads per sub-step
    constexpr int NMMA = TM * TN;       // MFMAs per sub-step
    constexpr int NK = BK / 16;         // MFMA sub-steps per K step
    static_assert(NK % 2 == 0, "sub-step parity must repeat across K steps");
    // the S >= 3 rings issue a step's loads spread through the step
    constexpr bool kSpreadLoads = S >= 3;
    constexpr int kHalf = (NDMA + 1) / 2;  // loads of a step issued before its stage barrier
    auto interleave = [&]() {
#pragma unroll
        for (int n = 0; n < NMMA; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
            if (n < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
    };

    // ---- mainloop: an S-stage ring.  Step t computes from stage t%S while the
    // loads of steps t+1..t+S-1 are in flight; at its top it issues step
    // t+S-1 into the stage step t-1 used (free since the barrier that ended
    // step t-1).  The pipeline is rotated across the barrier: sub-step 0's
    // operands of step t were read right after the previous barrier, and the
    // last sub-step's MFMAs of step t run after the barrier that publishes step
    // t+1, overlapping its first operand reads.  Before that barrier every wave
    // has its own loads of step t+1 landed (vmcnt) and its LDS reads of stage
    // t%S done (the barrier's lgkmcnt wait).
    if constexpr (!FP8) {
    Frag f[2];
#pragma unroll
    for (int s0 = 0; s0 < S - 1; ++s0) issue_step(s0);
    wait_oldest_step();
    __syncthreads();
    // Two-stage ring: step t+1's loads go out right after the barrier that
    // frees their stage (the one step t-1 used), ahead of the operand reads
    // and the last MFMAs of step t-1.
    // (With two stages every wait is vmcnt(0), so steps past the end can be
    // skipped without upsetting the wait arithmetic.)
    if constexpr (!kSpreadLoads)
        if (S - 1 < KT) issue_step(S - 1);
    load_frag(S0, 0, f[0]);
    for (int t = 0; t < KT; ++t) {
        const lds_t *X = S0 + (t % S) * STAGE;
        if constexpr (kSpreadLoads) {
            // Step t+S-1's loads are spread over the step: the first and the
            // last sub-step run in TM pieces (one MFMA row plus its share of the
            // next operand reads), each piece followed by its share of the
            // loads (half of them before the stage barrier, half after).
            const StepLoads sl = step_loads(t + S - 1);
            auto pieces = [&](const lds_t *src, int kk_next, Frag &fn, const Frag &fc, int d0) {
#pragma unroll
                for (int pc = 0; pc < TM; ++pc) {
                    load_frag_piece(src, kk_next, fn, pc);
                    mma_row(fc, pc);
#pragma unroll
                    for (int n = 0; n < TN; ++n) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                        if (n < reads_in_piece(pc)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int d = d0 + (pc * kHalf) / TM; d < d0 + ((pc + 1) * kHalf) / TM; ++d)
                        if (d < NDMA) issue_one(sl, d);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            pieces(X, 1, f[1], f[0], 0);
#pragma unroll
            for (int kk = 1; kk + 1 < NK; ++kk) {
                load_frag(X, kk + 1, f[(kk + 1) & 1]);
                mma(f[kk & 1]);
                interleave();
            }
            // step t+1's loads are done once at most the younger ones are in flight
            wait_vmcnt<(S - 3) * NDMA + kHalf>();
            __syncthreads();
            pieces(S0 + ((t + 1) % S) * STAGE, 0, f[0], f[(NK - 1) & 1], kHalf);
        } else {
#pragma unroll
            for (int kk = 0; kk + 1 < NK; ++kk) {
                load_frag(X, kk + 1, f[(kk + 1) & 1]);
                mma(f[kk & 1]);
                interleave();
            }
            wait_oldest_step();
            __syncthreads();
            if (t + S < KT) issue_step(t + S);  // into stage t % S, free since this barrier
            // (after the last step this reads operands that are never used)
            load_frag(S0 + ((t + 1) % S) * STAGE, 0, f[0]);
            mma(f[(NK - 1) & 1]);
            interleave();
        }
    }
    } else {
        // ---- fp8 e4m3fn block-scaled mainloop.  X [M,K] and W transposed
        // [N,K] (both K-contiguous bytes); one 128-wide K block per step
        // through an S-stage LDS ring of [BM][128] + [BN][128] bytes whose
        // 16-byte chunks are XOR-swizzled by row, filled by direct-to-LDS
        // loads as in the bf16 ring.  Each block's product d_b is accumulated
        // on the 64-wide fp8 MFMA into the one accumulator set, which carries
        // the running sum rescaled: after block b, acc *= s_b / s_{b+1}
        // (s_b = xs[m,b] * ws[n/128,b]), and after the last block acc *=
        // s_last, so acc ends at sum_b s_b * d_b.  The tile spans NCB
        // 128-column scale blocks (n0 a multiple of 128) and each wave's
        // columns lie in one of them.  The kernel allocates, past the stages, S
        // scale areas of 2 KiB and 2*NCB*BM floats of factors.
        constexpr int NCB = BN / 128;
        static_assert(NCB * 128 == BN && 128 % WN == 0, "a wave's columns lie in one W scale block");
        // Chunk c of tile row v sits at c ^ swz8(v).  Two 128-byte rows share a
        // 256-byte line of the 64 banks; ((v >> 1) & 7) sends the 16 rows of
        // one parity to 8 positions twice each, so the 16-byte operand reads of
        // 32 consecutive rows take the minimum passes.
        auto swz8 = [](int v) { return (v >> 1) & 7; };
        constexpr int ROWB = 128;  // bytes of one tile row per step
        constexpr int A8 = BM * ROWB, B8 = BN * ROWB, ST8 = A8 + B8;
        static_assert(S * ST8 == LDS_BYTES, "the fp8 stages fill the stage memory");
        constexpr int AI = A8 / (NW * 1024), BI = B8 / (NW * 1024);  // 1 KiB load instructions per wave per step
        static_assert(AI * NW * 1024 == A8 && BI * NW * 1024 == B8, "fp8 tile split");
        static_assert(BM == 4 * 64 && NW >= 5, "scale loads: four waves of row scales and one column scale");
        constexpr int ND8 = AI + BI + 1;  // loads per wave per step (operands, then one of scales)
        static_assert(S >= 2 && (S - 2) * ND8 < 64, "stage count vs vmcnt range");
        constexpr int SCL = 2048;  // bytes of one stage's scale area: 8 waves x 64 lanes x 4
        const int KB = (int)(K / 128);
        const int nb = (int)(n0 / 128);
        // byte offsets are 32-bit: M*K, N*K < 2^30 and M*KB*4 < 2^31 (host-checked)
        const i32x4 x8r = buffer_rsrc(p.x, (uint32_t)(M * K));
        const i32x4 w8r = buffer_rsrc(p.w, (uint32_t)(N * K));
        const i32x4 xsr = buffer_rsrc(p.xs, (uint32_t)(M * KB * 4));
        const i32x4 wsr = buffer_rsrc(p.ws, (uint32_t)(((N + 127) / 128) * KB * 4));
        // Per-lane sources.  Instruction i of a wave fills 1 KiB: 8 tile rows
        // of 8 chunks; the lane writes physical chunk lane%8 of its row and
        // loads the logical chunk the read side expects there.
        uint32_t xo[AI], wo[BI];
#pragma unroll
        for (int i = 0; i < AI; ++i) {
            const int v = (wave * AI + i) * 8 + lane / 8;
            const int64_t gm = row_of(v);
            xo[i] = gm >= 0 ? (uint32_t)(gm * K + (((lane & 7) ^ swz8(v)) << 4)) : kOob;
        }
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const int v = (wave * BI + i) * 8 + lane / 8;
            const int64_t gn = n0 + v;
            wo[i] = gn < N ? (uint32_t)(gn * K + (((lane & 7) ^ swz8(v)) << 4)) : kOob;
        }
        // Scales ride one block ahead: the loads of step kt bring block kt+1's
        // scales into stage kt's scale area -- waves 0..3 the row scales of
        // tile rows 64*wave + lane (slot = tile row), wave 4 lane c the
        // column scale of the tile's scale block c (slot 256 + c); every other
        // lane, and scale blocks past N, read nothing (zeros).
        const int NBW = (int)((N + 127) / 128);
        const i32x4 sr = wave_u < 4 ? xsr : wsr;
        uint32_t so;
        {
            const int64_t gm = wave < 4 ? row_of(wave * 64 + lane) : -1;
            so = wave < 4 ? (gm >= 0 ? (uint32_t)(gm * KB * 4) : kOob)
                          : (wave == 4 && lane < NCB && nb + lane < NBW ? (uint32_t)((int64_t)(nb + lane) * KB * 4)
                                                                       : kOob);
        }
        lds_t *const SC = S0 + LDS_BYTES;                                   // [S][SCL]
        float *const fac = reinterpret_cast<float *>(smem + LDS_BYTES + S * SCL);  // [2][NCB][BM]
        auto dma4 = [](i32x4 rsrc, uint32_t lds_base, uint32_t voff, uint32_t soff) {
            asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                         :
                         : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff)
                         : "memory", "m0");
        };
        // Loads of step kt into stage kt % S: exactly ND8 per wave for every kt
        // (past the last block every offset is out of range and loads zeros),
        // so the vmcnt arithmetic is uniform.
        auto issue8 = [&](int kt) {
            const lds_t *st = S0 + (kt % S) * ST8;
            const uint32_t la = lds_addr(st) + wave_u * AI * 1024;
            const uint32_t lb = lds_addr(st + A8) + wave_u * BI * 1024;
            const bool in = kt < KB;
            // (kt is uniform; readfirstlane tells the compiler so for the scalar operands)
            const uint32_t k0 = __builtin_amdgcn_readfirstlane(in ? (uint32_t)kt * 128u : 0u);
            const uint32_t la_u = __builtin_amdgcn_readfirstlane(la), lb_u = __builtin_amdgcn_readfirstlane(lb);
#pragma unroll
            for (int i = 0; i < AI; ++i) dma16(x8r, la_u + i * 1024, in ? xo[i] : kOob, k0);
#pragma unroll
            for (int i = 0; i < BI; ++i) dma16(w8r, lb_u + i * 1024, in ? wo[i] : kOob, k0);
            const bool sin = kt + 1 < KB;
            dma4(sr, __builtin_amdgcn_readfirstlane(lds_addr(SC + (kt % S) * SCL) + wave_u * 256), sin ? so : kOob,
                 __builtin_amdgcn_readfirstlane(sin ? (uint32_t)(kt + 1) * 4u : 0u));
        };
        // Factors: thread t < BM keeps its row's current scale s_b and the
        // column scales in registers; in step b (after issuing the next
        // step's loads) it reads block b+1's from the scale area of stage b%S
        // (landed with step b's operands) and writes the factors applied after
        // block b, s_b/s_{b+1} (or s_last after the last block), one per scale
        // block, into fac buffer b&1; the barrier that ends the step publishes
        // them.  One reciprocal per row and K block and one per scale block.
        // Rows past M and scale blocks past N get factor 1 (their products
        // are zero).  A zero scale (what a quantiser emits for an all-zero
        // block, e.g. padding rows) is not taken as the running unit: the
        // unit in effect carries over it (factor 1 across the block), so a
        // zero-scale block whose fp8 data are zero adds nothing, as in the
        // plain block sum, and the ratios stay finite.  Before the first
        // non-zero scale the unit is 1.
        const int64_t frow = tid < BM ? row_of(tid) : -1;
        auto unit = [](float raw, float carried) { return raw != 0.0f ? raw : carried; };
        float rs = frow >= 0 ? unit(p.xs[frow * KB], 1.0f) : 1.0f;
        float cs[NCB];
#pragma unroll
        for (int c = 0; c < NCB; ++c) cs[c] = nb + c < NBW ? unit(p.ws[(int64_t)(nb + c) * KB], 1.0f) : 1.0f;
        asm volatile("" ::"v"(rs), "v"(cs[0]), "v"(cs[NCB - 1]));  // the loads land before the first direct-to-LDS load
        auto write_factor = [&](int b) {
            if (tid < BM) {
                const float *sc = reinterpret_cast<const float *>(smem + LDS_BYTES + (b % S) * SCL);
                const bool more = b + 1 < KB;
                const float rn = more && frow >= 0 ? unit(sc[tid], rs) : 1.0f;
                // ratios through v_rcp_f32 (within 1 ulp; exact for powers of two)
                const float rr = more ? rs * __builtin_amdgcn_rcpf(rn) : rs;
#pragma unroll
                for (int c = 0; c < NCB; ++c) {
                    const float cn = more && nb + c < NBW ? unit(sc[256 + c], cs[c]) : 1.0f;
                    fac[((b & 1) * NCB + c) * BM + tid] = rr * (more ? cs[c] * __builtin_amdgcn_rcpf(cn) : cs[c]);
                    cs[c] = cn;
                }
                rs = rn;
            }
        };
        auto apply_factor = [&](int b) {
            const float *fb = fac + ((b & 1) * NCB + (wn * WN) / 128) * BM;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float f = fb[wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)];
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j][r] *= f;
                }
        };
#pragma unroll
        for (int s0 = 0; s0 < S - 1; ++s0) issue8(s0);
        wait_vmcnt<(S - 2) * ND8>();
        __syncthreads();
        for (int b = 0; b < KB; ++b) {
            // stage b%S holds block b's operands and block b+1's scales
            issue8(b + S - 1);  // into stage (b-1)%S, free since the barrier that ended step b-1
            write_factor(b);    // (reads stage b%S's scales, which issue8 does not touch)
            const lds_t *As = S0 + (b % S) * ST8;
            const lds_t *Bs = As + A8;
            // Two 64-wide MFMA steps per block (v_mfma_scale_f32_32x32x64_f8f6f4
            // with unit scales: the full fp8 rate on gfx950, where the 16-wide
            // fp8 MFMA runs at the bf16 rate).  Lane half h of step s takes
            // chunks 4s+h and 4s+2+h of its row (read as 16 bytes each) as its
            // 32 operand bytes.  A and B use the same k assignment, so each
            // step sums the products of all 64 k of its four chunks.
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                i32x4 aq[2][TM], bq[2][TN];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int c = 4 * s + 2 * q + (lane >> 5);
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        const int v = wm * WM + i * 32 + (lane & 31);
                        aq[q][i] = *(const __attribute__((address_space(3))) i32x4 *)(As + v * ROWB + ((c ^ swz8(v)) << 4));
                    }
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int v = wn * WN + j * 32 + (lane & 31);
                        bq[q][j] = *(const __attribute__((address_space(3))) i32x4 *)(Bs + v * ROWB + ((c ^ swz8(v)) << 4));
                    }
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const i32x8 a = __builtin_shufflevector(aq[0][i], aq[1][i], 0, 1, 2, 3, 4, 5, 6, 7);
                        const i32x8 b8 = __builtin_shufflevector(bq[0][j], bq[1][j], 0, 1, 2, 3, 4, 5, 6, 7);
                        // formats 0/0: e4m3fn operands; scales 127: 2^0 in E8M0
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b8, acc[i][j], 0, 0, 0, 127, 0, 127);
                    }
            }
            // step b+1's loads are done once at most the younger ones are in flight
            wait_vmcnt<(S - 2) * ND8>();
            __syncthreads();
            // after block b: acc *= s_b / s_{b+1} (s_last after the last block)
            apply_factor(b);
        }
    }
    wait_vmcnt_zero();
    __syncthreads();  // the stages are reused by the epilogue below

    // each wave stages its epilogue slabs in its own part of the (now idle) stages
    float *const ep = reinterpret_cast<float *>(smem) + wave * ER * EPS;

    // ---- epilogue -----------------------------------------------------------------
    // Row and byte offsets are 32-bit: M*N*2, M*K*2 and K*N*2 are below 2 GiB.
    const bool sys = p.system_scope != 0;
    const int seg = (int)p.seg, Ni = (int)N, N2 = 2 * (int)N;
    const int oseg0 = p.owner * seg, oseg1 = oseg0 + seg;
    // the tile's rows as up to two ranges [r0[h], r1[h]) (one when B follows
    // A; empty ranges have r0 == r1); loops over h are unrolled so that these
    // stay in registers
    auto row_ranges = [](int xa0, int xalen, int xb0, int xblen, int (&q0)[2], int (&q1)[2]) {
        if (xalen > 0 && xblen > 0 && xb0 == xa0 + xalen) {
            q0[0] = xa0, q1[0] = xa0 + xalen + xblen, q0[1] = q1[1] = 0;
        } else {
            q0[0] = xa0, q1[0] = xa0 + max(xalen, 0);
            q0[1] = xb0, q1[1] = xb0 + max(xblen, 0);
        }
    };
    int r0[2], r1[2];
    row_ranges((int)a0, alen, (int)b0, blen, r0, r1);
    constexpr bool has_owner = KIND != kNoOwnerRows;  // tiles that wait for and add partials
    constexpr bool kRingK = KIND == kRing;
    bool has_other = false;
#pragma unroll
    for (int h = 0; h < 2; ++h) has_other |= r0[h] < r1[h] && (r0[h] < oseg0 || r1[h] > oseg1);
    const int tc0 = (int)(n0 / p.ftn), ntc = (int)((min(n0 + BN, N) - 1) / p.ftn) - tc0 + 1;

    // The (source, flag tile) items this tile adds: with_items(fn) calls
    // fn(count, item), item(k, word, bit) giving item k's ready_in word and bit.
    // (The row ranges are recomputed here, so that they need not stay live
    // through the drain for the clears at the end.)
    auto with_items = [&](bool launder, auto &&fn) {
        // launder: hide the tile's row ranges from the compiler, so that
        // nothing computed from them for the wait is kept live to the end
        int xa0 = (int)a0, xalen = alen, xb0 = (int)b0, xblen = blen;
        if (launder) asm volatile("" : "+s"(xa0), "+s"(xalen), "+s"(xb0), "+s"(xblen));
        int r0[2], r1[2];
        row_ranges(xa0, xalen, xb0, xblen, r0, r1);
        if constexpr (kRingK) {
            // Ring: the flag tiles of the upstream partial of every segment
            // the tile's rows touch, except the chain segment.  Walks the
            // (range, segment) pieces in order; returns the item count and,
            // for 0 <= k < count, item k's word and bit.
            auto walk = [&](int k, uint32_t *&word, uint32_t &bit) {
                int seen = 0;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (r0[h] >= r1[h]) continue;
                    const int d0 = r0[h] / seg, d1 = (r1[h] - 1) / seg;
                    for (int d = d0; d <= d1; ++d) {
                        if (d == p.chain) continue;
                        const int s0 = d * seg;
                        const int lr0 = max(r0[h], s0) - s0, lr1 = min(r1[h], s0 + seg) - s0;
                        const int tr0 = lr0 / p.ftm, n = ((lr1 - 1) / p.ftm - tr0 + 1) * ntc;
                        if (k >= seen && k < seen + n) {
                            const int ti = k - seen;
                            const int t = (tr0 + ti / ntc) * (int)p.ftiles_n + tc0 + ti % ntc;
                            word = p.ready_in + (int64_t)d * p.fwords + (t >> 5);
                            bit = 1u << (t & 31);
                        }
                        seen += n;
                    }
                }
                return seen;
            };
            uint32_t *w0 = nullptr, b0_ = 0;
            fn(walk(-1, w0, b0_), walk);
        } else {
            int tr0[2] = {0, 0}, th[2] = {0, 0};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (!(r0[h] < r1[h] && r0[h] < oseg1 && r1[h] > oseg0)) continue;
                const int lr0 = max(r0[h], oseg0) - oseg0, lr1 = min(r1[h], oseg1) - oseg0;
                tr0[h] = lr0 / p.ftm;
                th[h] = ((lr1 - 1) / p.ftm - tr0[h] + 1) * ntc;
            }
            const int per_peer = th[0] + th[1], items = p.npeers * per_peer;
            // word and bit of item k
            auto item = [&](int k, uint32_t *&word, uint32_t &bit) {
                const int slot = k / per_peer;
                int ti = k % per_peer;
                const int h = ti < th[0] ? 0 : 1;
                ti -= h ? th[0] : 0;
                const int t = ((h ? tr0[1] : tr0[0]) + ti / ntc) * (int)p.ftiles_n + tc0 + ti % ntc;
                const int rank = slot < p.owner ? slot : slot + 1;
                word = p.ready_in + (int64_t)rank * p.fwords + (t >> 5);
                bit = 1u << (t & 31);
            };
            fn(items, item);
        }
    };

    auto wait_ready = [&]() {
    if constexpr (has_owner) {
        // Wait until every flag tile this tile adds is set: one item per
        // lane, all polled at once with relaxed loads, then one acquire.
        if (wave == 0) {
            with_items(false, [&](int items, auto item) {
                int64_t spins = 0;
                const uint64_t t0 = spin_clock();
                for (int k = lane; k < items; k += 64) {
                    uint32_t *word, bit;
                    item(k, word, bit);
                    while (!(load_relaxed(word, sys) & bit)) {
                        if (spin_expired(p.spin_limit, spins, t0)) {
                            if (p.status) atomicOr(p.status, (uint32_t)AREPI_STATUS_TIMEOUT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                }
            });
            fence_acquire(sys);
        }
        __syncthreads();
    }
    };

    // Consumption: clear the bits waited for, at the end of the tile, once
    // every wave has drained (barrier): by then every load of the peers' data
    // has returned, so a bit that reads clear also says its slot of recv may
    // be refilled.  Each flag tile lies under exactly one workgroup's rows and
    // columns when bits are consumed (checked on the host), so no other
    // workgroup waits for the bits cleared here; the kernel's end makes the
    // clears visible to whatever the stream runs next.
    auto consume_ready = [&]() {
    if constexpr (has_owner) {
        if (!p.consume) return;
        __syncthreads();
        if (wave == 0)
            with_items(true, [&](int items, auto item) {
                for (int k = lane; k < items; k += 64) {
                    uint32_t *word, bit;
                    item(k, word, bit);
                    fetch_and_relaxed(word, ~bit, sys);
                }
            });
    }
    };

    const int wm_u = wave_u / NWN;
    // Chunk (hb: false = A, true = B) and row inside it of this wave's row
    // wm*WM + t (t < WM, a multiple of 8).  When WM is a multiple of 2*IL the
    // chunk depends on t alone, which keeps it a compile-time constant.
    constexpr bool kStaticHalves = WM % (2 * IL) == 0;
    auto chunk_pos = [&](int t, bool &hb, int &idx) {
        if constexpr (kStaticHalves) {
            hb = (t / IL) & 1;
            idx = wm_u * (WM / 2) + (t / (2 * IL)) * IL + t % IL;
        } else {
            const unsigned v = (unsigned)(wm_u * WM + t);
            hb = (v / IL) & 1;
            idx = (int)((v / (2 * IL)) * IL + v % IL);
        }
    };

    // ---- staging, peer combine and stores ---------------------------------------
    // Each wave drains its accumulators one ER-row slab at a time through its
    // own LDS region (no workgroup barrier: a wave's LDS operations complete in
    // order) and finishes row-contiguous 16-byte packs ("units": one pack per
    // lane, RPS rows x WN columns per wave).  All LDS reads of a slab are
    // issued before its packs are used.  Row bases of a unit are wave-uniform
    // scalars; each lane adds a fixed byte offset.
    //  * Owner rows add the peers' partials (bf16 -> fp32, ascending rank
    //    order) to the fp32 accumulator, then round once.  The peers' packs
    //    are fetched D units ahead with row-coalesced buffer loads; lanes whose
    //    row is not an owner row and slots past R-1 use an out-of-range offset
    //    (the load returns zeros) and have their bits ORed with 0x80008000, so
    //    they add -0.0, which leaves every value unchanged.
    //  * Ring: every row outside the chain segment adds the one upstream
    //    partial of its own segment the same way (one slot, its buffer chosen
    //    per unit), whichever destination the row has.
    //  * A pack is stored with buffer stores whose offset is out of range
    //    (nothing is written) for the destination its row does not belong to
    //    and for rows or columns past the end.
    //  * When the owner chunk is A and the halves are static, the B half-blocks
    //    (no owner rows) are drained first, while the first peer packs load.
    constexpr int CPR = WN / 8;     // 16-byte chunks per epilogue row
    constexpr int RPS = 64 / CPR;   // rows per unit
    constexpr int STEPS = ER / RPS; // units per slab
    constexpr int NQ = 32 / ER;     // slabs per 32-row MFMA block
    constexpr int UPB = NQ * STEPS; // units per 32-row block
    static_assert(STEPS >= 1 && STEPS * RPS == ER, "epilogue step split");
    static_assert(!kRingK || RPS <= 8, "ring units must fit the 8-row segment alignment");
    constexpr bool kPubFirst = KIND == kOwnerChunkAPub || KIND == kOwnerAnywherePub;
    constexpr bool kAOnly = (KIND == kOwnerChunkA || KIND == kOwnerChunkAPub) && kStaticHalves;
    auto block_is_a = [](int i) { return !(((i * 32) / IL) & 1); };
    // owner-candidate blocks, in drain order
    constexpr int NOB = KIND == kNoOwnerRows ? 0 : kAOnly ? (TM + 1) / 2 : TM;
    auto cand_block = [&](int c) {
        if constexpr (kAOnly) {
            int n = 0;
            for (int i = 0; i < TM; ++i)
                if (block_is_a(i) && n++ == c) return i;
            return 0;
        } else {
            return c;
        }
    };
    constexpr int NOU = NOB * UPB;  // owner-candidate units
    constexpr int DW = (WPE != 1 ? 1 : 2) * (PEERS <= 1 ? 8 : PEERS <= 3 ? 4 : 2);
    constexpr int D = NOU < DW ? NOU : DW;  // prefetch depth in units
    constexpr int DP = D > 0 ? D : 1;       // ring-buffer size of the prefetched packs
    const int lane_r = lane / CPR, ch = lane % CPR;
    const int gc = (int)n0 + wn * WN + ch * 8;
    const bool col_ok = gc < Ni;
    const int lane_off = lane_r * N2 + gc * 2;  // byte offset of this lane inside a unit
    const __amdgpu_buffer_rsrc_t out_rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.out, 0, seg * N2, kBufferDword3);
    const __amdgpu_buffer_rsrc_t send_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.send ? p.send : p.out), 0, p.send ? (int)(M * N2) : 0, kBufferDword3);
    // Unit (block i, slab q, step st): first global row (scalar) and how many of its RPS rows exist.
    auto unit_rows = [&](int i, int q, int st, int &row0, int &nrows) {
        bool hb;
        int idx;
        chunk_pos(i * 32 + q * ER + st * RPS, hb, idx);
        row0 = (hb ? (int)b0 : (int)a0) + idx;
        nrows = min(max((hb ? blen : alen) - idx, 0), RPS);
    };
    // byte offset of this lane's pack of a unit in the owner segment, or out of range
    auto owner_off = [&](int row0, int nrows) -> uint32_t {
        const int row = row0 + lane_r;
        const bool own = col_ok && lane_r < nrows && row >= oseg0 && row < oseg1;
        return own ? (uint32_t)((row0 - oseg0) * N2 + lane_off) : kOob;
    };
    // Ring: a unit's rows lie in one segment (the segment height is a multiple
    // of the unit height, checked on the host), so its segment d, and with it
    // the upstream buffer, is a wave-uniform scalar.  Offset of this lane's
    // pack in up[d], or out of range (chain segment, missing rows or columns).
    auto ring_seg = [&](int row0) { return __builtin_amdgcn_readfirstlane(row0 / seg); };
    auto ring_off = [&](int row0, int nrows) -> uint32_t {
        const int d = ring_seg(row0);
        const bool in = col_ok && lane_r < nrows && d != p.chain;
        return in ? (uint32_t)((row0 - d * seg) * N2 + lane_off) : kOob;
    };
    auto comb_off = [&](int row0, int nrows) -> uint32_t {
        if constexpr (kRingK)
            return ring_off(row0, nrows);
        else
            return owner_off(row0, nrows);
    };
    auto up_rsrc = [&](int d) {
        const uint16_t *q = p.up[0];
#pragma unroll
        for (int k = 1; k < kMaxR; ++k) q = d == k ? p.up[k] : q;
        return __builtin_amdgcn_make_buffer_rsrc((void *)(q ? q : p.x), 0, q ? seg * N2 : 0, kBufferDword3);
    };
    __amdgpu_buffer_rsrc_t prs[PEERS];
    uint32_t pneg[PEERS];  // 0x80008000 for slots past R-1 (they add -0.0)
    i32x4 pk[DP][PEERS];
    auto prefetch = [&](int ou) {  // ou = owner-candidate unit
        const int i = cand_block(ou / UPB), q = (ou % UPB) / STEPS, st = ou % STEPS;
        int row0, nrows;
        unit_rows(i, q, st, row0, nrows);
        const uint32_t off = comb_off(row0, nrows);
        if constexpr (kRingK) {
            static_assert(PEERS == 1, "the ring adds one upstream partial");
            pk[ou % DP][0] = __builtin_bit_cast(
                i32x4, __builtin_amdgcn_raw_buffer_load_b128(up_rsrc(ring_seg(row0)), off, 0, kAuxNontemporal));
        } else {
#pragma unroll
            for (int sl = 0; sl < PEERS; ++sl)
                pk[ou % DP][sl] = __builtin_bit_cast(
                    i32x4, __builtin_amdgcn_raw_buffer_load_b128(prs[sl], off, 0, kAuxNontemporal));
        }
    };
    if constexpr (NOU > 0) {
        const int recv_bytes = seg * N2;
#pragma unroll
        for (int sl = 0; sl < PEERS; ++sl) {  // slots hold the peers in ascending rank order
            const bool valid = sl < p.npeers;
            if constexpr (!kRingK)  // (the ring picks its resource per unit)
                prs[sl] = __builtin_amdgcn_make_buffer_rsrc((void *)(valid ? p.peer[sl] : p.x), 0,
                                                            valid ? recv_bytes : 0, kBufferDword3);
            pneg[sl] = (kRingK || valid) ? 0u : 0x80008000u;
        }
    }
    // the first D units' peer packs (after the readiness wait)
    auto start_prefetch = [&]() {
        if constexpr (NOU > 0) {
#pragma unroll
            for (int ou = 0; ou < D; ++ou) prefetch(ou);
        }
    };
    // Drain block i; `c` is its index among the owner-candidate blocks, or -1.
    // `rows` selects the rows stored: kAllRows, kOtherRows (rows outside the
    // owner segment, no peers added) or kOwnRows (owner rows only).
    enum { kAllRows = 0, kOtherRows = 1, kOwnRows = 2 };
    auto drain_block = [&](int i, int c, int rows) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            // accumulator register r of a 32x32 tile holds row 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    if (NQ == 1 || row / ER == q) ep[(row % ER) * EPS + j * 32 + (lane & 31)] = acc[i][j][r];
                }
            float v[STEPS][8];
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                const float *src = ep + (st * RPS + lane_r) * EPS + ch * 8;
                const float4 v0 = *reinterpret_cast<const float4 *>(src);
                const float4 v1 = *reinterpret_cast<const float4 *>(src + 4);
                v[st][0] = v0.x, v[st][1] = v0.y, v[st][2] = v0.z, v[st][3] = v0.w;
                v[st][4] = v1.x, v[st][5] = v1.y, v[st][6] = v1.z, v[st][7] = v1.w;
            }
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                int row0, nrows;
                unit_rows(i, q, st, row0, nrows);
                const int row = row0 + lane_r;
                const bool ok = col_ok && lane_r < nrows;
                const bool own = row >= oseg0 && row < oseg1;
                if (c >= 0) {  // compile-time after unrolling
                    const int ou = c * UPB + q * STEPS + st;
                    const uint32_t lane_neg = comb_off(row0, nrows) == kOob ? 0x80008000u : 0u;
#pragma unroll
                    for (int sl = 0; sl < PEERS; ++sl) {
                        const uint32_t neg = lane_neg | pneg[sl];
                        const i32x4 w4 = pk[ou % DP][sl];
                        float f[8];
                        unpack8(make_uint4((uint32_t)w4.x | neg, (uint32_t)w4.y | neg, (uint32_t)w4.z | neg,
                                           (uint32_t)w4.w | neg),
                                f);
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[st][e] = v[st][e] + f[e];
                    }
                    if (ou + D < NOU) prefetch(ou + D);
                }
                const uint4 q8 = pack8(v[st]);
                const i32x4 qv = {(int)q8.x, (int)q8.y, (int)q8.z, (int)q8.w};
                if constexpr (has_owner)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        qv, out_rs, (ok && own && rows != kOtherRows) ? (uint32_t)((row0 - oseg0) * N2 + lane_off) : kOob,
                        0, kAuxNontemporal);
                __builtin_amdgcn_raw_buffer_store_b128(
                    qv, send_rs, (ok && !own && rows != kOwnRows) ? (uint32_t)(row0 * N2 + lane_off) : kOob, 0,
                    kAuxNontemporal);
            }
        }
    };

    // Publish the send tiles: drain this thread's stores, balanced barrier, one
    // release, then relaxed bit sets.
    auto publish = [&]() {
        drain_stores();
        __syncthreads();
        if (wave == 0) {
            fence_release(sys);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (r0[h] >= r1[h]) continue;
                const int d0 = r0[h] / seg, d1 = (r1[h] - 1) / seg;
                for (int d = d0; d <= d1; ++d) {
                    if (d == p.owner) continue;
                    const int s0 = d * seg;
                    const int lr0 = max(r0[h], s0) - s0, lr1 = min(r1[h], s0 + seg) - s0;
                    const int tr0 = lr0 / p.ftm, tr1 = (lr1 - 1) / p.ftm;
                    const int items = (tr1 - tr0 + 1) * ntc;
                    uint32_t *words = p.ready_out + (int64_t)d * p.fwords;
                    for (int it = lane; it < items; it += 64) {
                        const int t = (tr0 + it / ntc) * (int)p.ftiles_n + tc0 + it % ntc;
                        fetch_or_relaxed(words + (t >> 5), 1u << (t & 31), sys);
                    }
                }
            }
        }
    };
    const bool publishes = p.ready_out && has_other;

    // A tile with owner rows and rows of other segments publishes the other
    // segments' rows before it waits (kPubFirst): across ranks, a wait placed
    // before that publication could close a cycle (this rank's owner rows
    // waiting on a peer whose own such tile waits on this rank's publication).
    // Its accumulators are staged twice: other rows, publish, wait, owner rows.
    if constexpr (kRingK) {
        // (the ring refuses tiles that span segments when it publishes)
        wait_ready();
        start_prefetch();
#pragma unroll
        for (int i = 0; i < TM; ++i) drain_block(i, i, kAllRows);
        if (publishes) publish();
    } else if constexpr (kAOnly) {
        // chunk B holds no owner rows, chunk A only owner rows
        if constexpr (kPubFirst) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                if (!block_is_a(i)) drain_block(i, -1, kAllRows);
            publish();
            wait_ready();
            start_prefetch();
        } else {
            wait_ready();
            start_prefetch();
#pragma unroll
            for (int i = 0; i < TM; ++i)
                if (!block_is_a(i)) drain_block(i, -1, kAllRows);
        }
#pragma unroll
        for (int c = 0; c < NOB; ++c) drain_block(cand_block(c), c, kAllRows);
        if (!kPubFirst && publishes) publish();
    } else if constexpr (kPubFirst) {
#pragma unroll
        for (int i = 0; i < TM; ++i) drain_block(i, -1, kOtherRows);
        publish();
        wait_ready();
        start_prefetch();
#pragma unroll
        for (int i = 0; i < TM; ++i) drain_block(i, i, kOwnRows);
    } else if constexpr (has_owner) {
        wait_ready();
        start_prefetch();
#pragma unroll
        for (int i = 0; i < TM; ++i) drain_block(i, i, kAllRows);
        if (publishes) publish();
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) drain_block(i, -1, kAllRows);
        if (publishes) publish();
    }
    consume_ready();
}

// ---- host side --------------------------------------------------------------------

struct TileCfg {
    int id, BM, BN;
    int slots;   // workgroups co-resident on one CU (LDS / register bound)
    double eff;  // relative per-CU throughput used by the automatic choice
    bool one_wave = false;  // chosen automatically only when every tile is resident at once
};
// eff: sustained per-CU throughput relative to the 4-stage 256x256 tile, from
// timing the tp=4 / tp=8 workloads on MI355X (contiguous rows).  64x128_s4
// beats 64x128 when each CU runs one tile (tp=8 M=256: 32 against 34.5 us)
// and loses when a CU has two (M=512: 54 against 44 us, where 64x128 keeps
// both resident side by side), hence one_wave.
constexpr TileCfg kTiles[] = {
    {AREPI_TILE_256x256_W8_K64, 256, 256, 1, 1.14},
    {AREPI_TILE_256x256_W8, 256, 256, 1, 1.08},
    {AREPI_TILE_256x256_S4, 256, 256, 1, 1.00},
    {AREPI_TILE_256x256, 256, 256, 1, 0.96},
    {AREPI_TILE_256x128_S3, 256, 128, 2, 0.95},
    {AREPI_TILE_128x256, 128, 256, 1, 0.97},
    {AREPI_TILE_128x256_S3, 128, 256, 2, 0.93},
    {AREPI_TILE_128x128_S4, 128, 128, 2, 0.80},
    {AREPI_TILE_128x128, 128, 128, 2, 0.75},
    {AREPI_TILE_64x128_S4, 64, 128, 1, 0.64, true},
    {AREPI_TILE_64x128, 64, 128, 3, 0.60},
    {AREPI_TILE_32x256, 32, 256, 2, 0.40},
};

const TileCfg *find_tile(int id) {
    for (const auto &t : kTiles)
        if (t.id == id) return &t;
    return nullptr;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Every flag tile (of every segment) must lie inside one row block of BM rows
// (or chunk, in the paired layout: the same test with BM = CK) and one column
// block of BN, so that one workgroup can publish it.
bool flags_nest(int64_t M, int64_t N, int R, int ftm, int ftn, int BM, int BN) {
    const int64_t seg = M / R;
    for (int64_t c = 0; c * ftn < N; ++c) {
        const int64_t s = c * ftn, e = std::min<int64_t>(s + ftn, N) - 1;
        if (s / BN != e / BN) return false;
    }
    for (int d = 0; d < R; ++d) {
        for (int64_t k = 0; k * ftm < seg; ++k) {
            const int64_t s = d * seg + k * ftm, e = d * seg + std::min<int64_t>((k + 1) * ftm, seg) - 1;
            if (s / BM != e / BM) return false;
        }
    }
    return true;
}

int validate_shape(int64_t M, int64_t N, int64_t K, int R, int owner, int ftm, int ftn) {
    auto bad = [](const std::string &m) { return fail(AREPI_EINVAL, "arepi_gemm_rs: " + m); };
    if (R < 1 || R > kMaxR) return bad("R=" + std::to_string(R) + " outside [1, 8]");
    if (owner < 0 || owner >= R)
        return bad("owner=" + std::to_string(owner) + " outside [0, R-1=" + std::to_string(R - 1) + "]");
    if (M < 1) return bad("M=" + std::to_string(M) + " must be >= 1");
    if (M % R) return bad("M=" + std::to_string(M) + " is not a multiple of R=" + std::to_string(R));
    if (N < 8 || N % 8) return bad("N=" + std::to_string(N) + " must be a positive multiple of 8");
    if (K < 8 || K % 8) return bad("K=" + std::to_string(K) + " must be a positive multiple of 8");
    if (ftm < 1 || ftn < 1)
        return bad("flag tile " + std::to_string(ftm) + "x" + std::to_string(ftn) + " must be at least 1x1");
    // X, W and each peer partial are addressed with 32-bit buffer offsets
    const int64_t lim = int64_t(1) << 31;
    if (M * K * 2 >= lim || K * N * 2 >= lim || M * N * 2 >= lim)
        return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs: X [M,K], W [K,N] and send [M,N] must each be below 2 GiB");
    return AREPI_OK;
}

// Chunk rows of a BM-row block (two chunks per block from BM = 64 up).
int chunk_rows(int BM) { return BM >= 64 ? BM / 2 : BM; }

// Whether the paired row layout applies: two or more ranks, segments made of
// whole chunks, and (when publishing) flag tiles nested in chunks.
bool use_paired(int64_t M, int64_t N, int R, int ftm, int ftn, int BM, int BN, bool publish, bool contiguous) {
    const int CK = chunk_rows(BM);
    if (contiguous || R < 2 || CK == BM) return false;
    if ((M / R) % CK) return false;
    return !publish || flags_nest(M, N, R, ftm, ftn, CK, BN);
}

// whole_segments: only tiles whose row blocks each lie in one segment (the
// push ring's condition for publishing).
int pick_tile(int64_t M, int64_t N, int64_t K, int R, int ftm, int ftn, bool publish, bool whole_segments = false) {
    (void)K;
    int best = -1;
    double best_cost = 0;
    for (const auto &t : kTiles) {
        if (publish && !flags_nest(M, N, R, ftm, ftn, t.BM, t.BN)) continue;
        if (whole_segments && R > 1 && (M / R) % t.BM) continue;
        const int64_t count = cdiv(M, t.BM) * cdiv(N, t.BN);
        if (t.one_wave && count > 256 * (int64_t)t.slots) continue;
        // waves of co-resident tiles x time of one wave; a wave with fewer
        // tiles than slots on each CU runs fewer of them side by side
        const int64_t waves = cdiv(count, 256 * (int64_t)t.slots);
        const int64_t per_cu = std::min<int64_t>(t.slots, cdiv(count, 256));
        const double cost = (double)waves * per_cu * t.BM * t.BN / t.eff;
        if (best < 0 || cost < best_cost) {
            best = t.id;
            best_cost = cost;
        }
    }
    return best;
}

// Launch geometry (everything but the pointers) for tile t.
int plan(GemmRsParams &p, const TileCfg *t, int64_t M, int64_t N, int64_t K, int R, int owner, int ftm, int ftn,
         bool publish, bool contiguous, bool owner_first = false, bool owner_half = false) {
    p.M = M;
    p.N = N;
    p.K = K;
    p.seg = M / R;
    p.ftiles_n = cdiv(N, ftn);
    p.fwords = cdiv(cdiv(p.seg, ftm) * p.ftiles_n, 32);
    p.R = R;
    p.owner = owner;
    p.ftm = ftm;
    p.ftn = ftn;
    p.nCB = (int)cdiv(N, t->BN);
    p.paired = use_paired(M, N, R, ftm, ftn, t->BM, t->BN, publish, contiguous);
    if (p.paired) {
        // non-owner chunks paired with each other first, owner chunks paired last
        const int CK = chunk_rows(t->BM);
        p.nc = (int)(p.seg / CK);
        p.npure = (R - 2) * p.nc / 2;
        p.nleft = (R - 2) * p.nc % 2;
        p.nRB = p.npure + p.nleft + p.nc;
        p.ob1 = 0;
    } else {
        p.nRB = (int)cdiv(M, t->BM);
        // first row block after the owner's: the rotation puts the owner's
        // last; or (owner_first) the owner's first row block, which puts them
        // first
        p.ob1 = owner_first ? (int)(((int64_t)owner * p.seg / t->BM) % p.nRB)
                            : (int)(cdiv((int64_t)(owner + 1) * p.seg, t->BM) % p.nRB);
    }
    p.group = 4;
    p.xcd_chunk = 32;
    const int64_t nwg = (int64_t)p.nRB * p.nCB;
    if (nwg > (int64_t)1 << 30) return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs: too many tiles");
    p.nWG = (int)nwg;
    p.nrot = p.nRB;
    p.nextra = 0;
    if (owner_half) {
        // the owner's seg/BM whole row blocks leave the rotation, which then
        // reaches only the others; 2*seg/BM half-blocks per column come after
        const int k = (int)(p.seg / t->BM);
        p.nRB -= k;
        p.nWG = p.nRB * p.nCB;
        p.nextra = 2 * k * p.nCB;
    }
    return AREPI_OK;
}

// Tiles with an owner half-height form (AREPI_TILE_OWNER_HALF): the 8-wave
// 256x256 BK 64 tile and the 4-wave 128x256 tile.
bool has_owner_half(int id) { return id == AREPI_TILE_256x256_W8_K64 || id == AREPI_TILE_128x256; }

// Whether AREPI_TILE_OWNER_HALF can apply to tile id: whole owner row blocks,
// and, when bits are consumed, flag tiles nesting in the half-height owner
// tiles (each must lie under one workgroup; owner tiles publish nothing).
bool owner_half_fits(int64_t M, int64_t N, int R, int ftm, int ftn, bool consume, int id) {
    if (!has_owner_half(id) || R < 2) return false;
    const TileCfg *t = find_tile(id);
    return (M / R) % t->BM == 0 && (!consume || flags_nest(M, N, R, ftm, ftn, t->BM / 2, t->BN));
}

// Tile id, row layout and options of a validated tile_cfg.
struct CfgChoice {
    const TileCfg *t;
    int id;
    bool contiguous, consume, nest, owner_first, owner_half;
};
CfgChoice decode_cfg(int64_t M, int64_t N, int64_t K, int R, int ftm, int ftn, bool publish, int tile_cfg,
                     bool whole_segments = false) {
    CfgChoice c{};
    c.consume = (tile_cfg & AREPI_TILE_CONSUME_READY) != 0;
    c.nest = publish || c.consume;
    c.contiguous = (tile_cfg & AREPI_TILE_PAIRED_ROWS) == 0;
    c.owner_first = (tile_cfg & AREPI_TILE_OWNER_FIRST) != 0;
    c.owner_half = (tile_cfg & AREPI_TILE_OWNER_HALF) != 0;
    const int id = tile_cfg &
                   ~(AREPI_TILE_PAIRED_ROWS | AREPI_TILE_CONSUME_READY | AREPI_TILE_OWNER_FIRST | AREPI_TILE_OWNER_HALF);
    c.id = id == AREPI_TILE_AUTO ? pick_tile(M, N, K, R, ftm, ftn, c.nest, whole_segments && publish) : id;
    c.t = find_tile(c.id);
    // The automatic choice (direct form, contiguous owner-last layout) also
    // runs the owner rows as half-height tiles where that adds no round of
    // workgroups: tp=8 M = 2048, 4096, 8192 measured 13%, 7% and 6% faster;
    // the one-round tp=4 share would need a second round.
    if (id == AREPI_TILE_AUTO && !whole_segments && c.contiguous && !c.owner_first &&
        owner_half_fits(M, N, R, ftm, ftn, c.consume, c.id)) {
        const int64_t ncb = cdiv(N, c.t->BN), plain = cdiv(M, c.t->BM) * ncb;
        const int64_t half = plain + (M / R / c.t->BM) * ncb;
        const int64_t round = 256 * (int64_t)c.t->slots;
        if (cdiv(half, round) <= cdiv(plain, round)) c.owner_half = true;
    }
    return c;
}

}  // namespace
}  // namespace arepi

#endif  // AREPI_GEMM_RS_IMPL_H
