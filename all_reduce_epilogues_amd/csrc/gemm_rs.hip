// gemm_rs.hip -- row-parallel bf16 GEMM with a fused reduce-scatter epilogue
// for gfx950 (MI355X).
//
// What it computes follows DeepGEMM PR #1 "Fused ring RS: per-tile bitmask +
// drain-ring with owner-boundary flush" (description) and ROCm/mori PR #662
// (PR description, fused GEMM + all-reduce of the wo_b projection), in the
// direct-sum form: each rank computes its full local product C = X.W; the owner
// segment's tiles add the R-1 peer partials in the epilogue, all other rows are
// stored as this rank's outgoing partials.
//
// Design (gfx950, not a translation of the pages' sm100 / FlyDSL kernels):
//  * Workgroup tile BM x BN, 4 waves of 64 lanes, each wave a WM x WN block of
//    32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16, fp32 accumulators).
//  * K is walked in BK = 64 steps through a two-stage LDS ring: the next
//    step's global loads are issued into registers before the current step's
//    MFMAs and written to the other LDS stage after them, one barrier per step.
//  * X [M,K] is K-contiguous and goes to LDS as is.  W [K,N] is N-contiguous;
//    each thread loads a 4(k) x 8(n) block and transposes it in registers so
//    the LDS copy is K-contiguous per column, which is what the MFMA B operand
//    reads (8 consecutive k per lane).
//  * LDS rows are 128 bytes (64 bf16); the eight 16-byte chunks of a row are
//    XOR-swizzled by (row ^ row>>3) & 7 so that both the 16-byte MFMA operand
//    reads (32 consecutive rows, one chunk) and the 16-byte X writes avoid
//    bank conflicts.
//  * Epilogue: the accumulators (4 consecutive rows per lane in the MFMA
//    layout) are staged through LDS one 32-row slab at a time and read back
//    row-contiguous, so every global access is a 16-byte, row-coalesced pack.
//    Owner rows wait for their peers' flag-tile bits (relaxed polls, one
//    acquire), then add the peers in ascending rank order (fp32) and store to
//    `out`; other rows are converted and stored to `send`.  No per-tile drain
//    on `out` (the kernel end is its release); a drain + balanced barrier +
//    one release precede the ready_out bits of `send` tiles.
//  * Tile order: row blocks rotated so the owner segment comes last (the
//    destination-rotated order of the mori page's tile-order commit), grouped
//    G row blocks at a time, and remapped so that the blocks one XCD runs
//    together are neighbours (shared X rows / W columns in that XCD's L2).
#include <algorithm>
#include <string>

#include "arepi_internal.h"

namespace arepi {
namespace {

constexpr int BK = 64;
constexpr int kMaxR = 8;
constexpr int kXcds = 8;

struct GemmRsParams {
    const uint16_t *x;
    const uint16_t *w;
    const uint16_t *peer[kMaxR - 1];  // peer partials in ascending rank order, owner skipped
    int npeers;                       // R - 1
    const uint32_t *ready_in;
    uint16_t *out;
    uint16_t *send;
    uint32_t *ready_out;
    uint32_t *status;
    int64_t M, N, K, seg;
    int64_t ftiles_n;  // flag tiles per segment row band
    int64_t fwords;    // u32 words per peer
    int64_t spin_limit;
    int R, owner, ftm, ftn;
    int system_scope;
    int nRB, nCB, ob1, group, xcd_chunk, nWG;
};

// gfx9 buffer-resource word 3 (raw, untyped 32-bit data format).
constexpr int kBufferDword3 = 0x00020000;

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

typedef int i32x4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ void tile_of_block(const GemmRsParams &p, int b, int &rb, int &cb) {
    // XCD-aware remap inside full rounds of 8*C blocks: consecutive schedule
    // entries land on the same XCD (blocks are dealt to XCDs round-robin).
    const int C = p.xcd_chunk;
    const int round = kXcds * C;
    int s = b;
    if ((b / round + 1) * round <= p.nWG) {
        const int r = b / round, j = b % round;
        s = r * round + (j % kXcds) * C + j / kXcds;
    }
    // G row blocks at a time, column-major inside the group.
    const int per_group = p.group * p.nCB;
    const int g = s / per_group, within = s % per_group;
    const int gsz = min(p.group, p.nRB - g * p.group);
    const int pos = g * p.group + within % gsz;
    cb = within / gsz;
    rb = (p.ob1 + pos) % p.nRB;  // rotated: owner row blocks come last
}

// WPE: waves per SIMD the register allocation targets (1 = one big-tile
// workgroup per CU; 2 = two co-resident workgroups; 0 = no target).
template <int BM, int BN, int WM, int WN, int BK, int S, int WPE, int PEERS>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1, WPE > 0 ? WPE : 8)))
    gemm_rs_kernel(const GemmRsParams p) {
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

    // S stages [X | W] x S; the epilogue reuses the same memory.
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
    typedef __attribute__((address_space(3))) uint8_t lds_t;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    int rb, cb;
    tile_of_block(p, blockIdx.x, rb, cb);
    const int64_t m0 = (int64_t)rb * BM, n0 = (int64_t)cb * BN;
    const int64_t M = p.M, N = p.N, K = p.K;

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
        const int64_t gm = m0 + a_row_of(i);
        a_off[i] = (gm < M) ? (uint32_t)((gm * K + a_col_of(i)) * 2) : kOob;
    }
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
        const int r = b_row_of(i);
        const int64_t gn = n0 + ((lane % B_CPR) ^ swz_b(r)) * 8;
        b_off[i] = (gn < N) ? (uint32_t)((r * N + gn) * 2) : kOob;
    }

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
            const uint32_t sa = (uint32_t)(k0 * 2), sb = (uint32_t)(k0 * N * 2);
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
                const bool in = b_off[i] != kOob && k0 + b_row_of(i) < K;
                dma16(wr, lb + i * 1024, in ? b_off[i] + (uint32_t)(k0 * N * 2) : kOob, 0);
            }
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
    Frag f[2];
#pragma unroll
    for (int s0 = 0; s0 < S - 1; ++s0) issue_step(s0);
    wait_oldest_step();
    __syncthreads();
    load_frag(S0, 0, f[0]);
    for (int t = 0; t < KT; ++t) {
        const lds_t *X = S0 + (t % S) * STAGE;
        issue_step(t + S - 1);
#pragma unroll
        for (int kk = 0; kk + 1 < NK; ++kk) {
            load_frag(X, kk + 1, f[(kk + 1) & 1]);
            mma(f[kk & 1]);
            interleave();
        }
        wait_oldest_step();
        __syncthreads();
        // (after the last step this reads operands that are never used)
        load_frag(S0 + ((t + 1) % S) * STAGE, 0, f[0]);
        mma(f[(NK - 1) & 1]);
        interleave();
    }
    wait_vmcnt_zero();
    __syncthreads();  // the stages are reused by the epilogue below

    // each wave stages its epilogue slabs in its own part of the (now idle) stages
    float *const ep = reinterpret_cast<float *>(smem) + wave * ER * EPS;

    // ---- epilogue -----------------------------------------------------------------
    const bool sys = p.system_scope != 0;
    const int64_t m1 = min(m0 + BM, M);
    const int64_t oseg0 = (int64_t)p.owner * p.seg, oseg1 = oseg0 + p.seg;
    const bool has_owner = m0 < oseg1 && m1 > oseg0;
    const bool has_other = m0 < oseg0 || m1 > oseg1;

    if (has_owner) {
        // Wait until every peer's flag tiles under this tile's owner rows are set.
        if (wave == 0 && lane < p.R && lane != p.owner) {
            const int64_t lr0 = max(m0, oseg0) - oseg0, lr1 = min(m1, oseg1) - oseg0;
            const int64_t tr0 = lr0 / p.ftm, tr1 = (lr1 - 1) / p.ftm;
            const int64_t tc0 = n0 / p.ftn, tc1 = (min(n0 + BN, N) - 1) / p.ftn;
            const uint32_t *words = p.ready_in + (int64_t)lane * p.fwords;
            int64_t spins = 0;
            bool gave_up = false;
            for (int64_t tr = tr0; tr <= tr1 && !gave_up; ++tr) {
                for (int64_t tc = tc0; tc <= tc1 && !gave_up; ++tc) {
                    const int64_t t = tr * p.ftiles_n + tc;
                    const uint32_t bit = 1u << (t & 31);
                    while (!(load_relaxed(words + (t >> 5), sys) & bit)) {
                        if (++spins > p.spin_limit) {
                            if (p.status) atomicOr(p.status, (uint32_t)AREPI_STATUS_TIMEOUT);
                            gave_up = true;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                }
            }
            fence_acquire(sys);
        }
        __syncthreads();
    }

    // Each wave drains its accumulators one ER-row slab at a time through its
    // own LDS region (no workgroup barrier: a wave's LDS operations complete in
    // order) and finishes row-contiguous 16-byte packs.  The peers' partials of
    // owner rows are independent of the accumulators, so they are fetched D
    // units ahead (a unit = one 16-byte pack per lane) with branch-free buffer
    // loads; out-of-range and non-owner lanes use an out-of-range offset.
    constexpr int CPR = WN / 8;     // 16-byte chunks per epilogue row
    constexpr int RPS = 64 / CPR;   // rows per unit
    constexpr int STEPS = ER / RPS; // units per slab
    constexpr int NQ = 32 / ER;     // slabs per 32-row MFMA block
    constexpr int NU = TM * NQ * STEPS;
    constexpr int kPeers = PEERS;       // peer slots compiled in (>= R - 1)
    constexpr int DW = WPE != 1 ? (PEERS <= 3 ? 4 : 2) : (PEERS <= 3 ? 8 : 4);
    constexpr int D = NU < DW ? NU : DW;  // prefetch depth in units
    static_assert(STEPS >= 1 && STEPS * RPS == ER, "epilogue step split");
    const uint32_t recv_bytes = (uint32_t)(p.seg * N * 2);
    __amdgpu_buffer_rsrc_t prs[kPeers];
    bool pvalid[kPeers];
#pragma unroll
    for (int sl = 0; sl < kPeers; ++sl) {  // slots hold the peers in ascending rank order
        pvalid[sl] = sl < p.npeers;
        prs[sl] = __builtin_amdgcn_make_buffer_rsrc((void *)(pvalid[sl] ? p.peer[sl] : p.x), 0,
                                                    pvalid[sl] ? (int)recv_bytes : 0, kBufferDword3);
    }
    auto unit_pos = [&](int u, int64_t &gr, int64_t &gc, int &row, int &ch) {
        const int i = u / (NQ * STEPS), q = (u / STEPS) % NQ, st = u % STEPS;
        row = st * RPS + lane / CPR;
        ch = lane % CPR;
        gr = m0 + wm * WM + i * 32 + q * ER + row;
        gc = n0 + wn * WN + ch * 8;
    };
    auto prefetch = [&](int u, i32x4 (&pk)[kPeers]) {
        int64_t gr, gc;
        int row, ch;
        unit_pos(u, gr, gc, row, ch);
        const bool own = gr >= oseg0 && gr < oseg1 && gc < N;
        const uint32_t off = own ? (uint32_t)(((gr - oseg0) * N + gc) * 2) : kOob;
#pragma unroll
        for (int sl = 0; sl < kPeers; ++sl)
            if (pvalid[sl])
                pk[sl] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(prs[sl], off, 0, kAuxNontemporal));
    };
    i32x4 pk[D][kPeers];
    if (has_owner) {
#pragma unroll
        for (int u = 0; u < D; ++u) prefetch(u, pk[u]);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int i = u / (NQ * STEPS), q = (u / STEPS) % NQ;
        if (u % STEPS == 0) {
            // accumulator register r of a 32x32 tile holds row 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    if (row / ER == q) ep[(row % ER) * EPS + j * 32 + (lane & 31)] = acc[i][j][r];
                }
        }
        int64_t gr, gc;
        int row, ch;
        unit_pos(u, gr, gc, row, ch);
        if (gr < M && gc < N) {
            const float4 v0 = *reinterpret_cast<const float4 *>(ep + row * EPS + ch * 8);
            const float4 v1 = *reinterpret_cast<const float4 *>(ep + row * EPS + ch * 8 + 4);
            float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            if (gr >= oseg0 && gr < oseg1) {
#pragma unroll
                for (int sl = 0; sl < kPeers; ++sl) {
                    if (pvalid[sl]) {
                        float f[8];
                        const i32x4 w4 = pk[u % D][sl];
                        unpack8(make_uint4(w4.x, w4.y, w4.z, w4.w), f);
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = v[e] + f[e];
                    }
                }
                store16_nt(p.out + (gr - oseg0) * N + gc, pack8(v));
            } else if (p.send) {
                store16_nt(p.send + gr * N + gc, pack8(v));
            }
        }
        if (has_owner && u + D < NU) prefetch(u + D, pk[u % D]);
    }

    // Publish the send tiles: drain this thread's stores, balanced barrier, one
    // release, then relaxed bit sets.
    if (p.ready_out && has_other) {
        drain_stores();
        __syncthreads();
        if (wave == 0) {
            fence_release(sys);
            const int64_t d0 = m0 / p.seg, d1 = (m1 - 1) / p.seg;
            const int64_t tc0 = n0 / p.ftn, tc1 = (min(n0 + BN, N) - 1) / p.ftn;
            const int64_t ntc = tc1 - tc0 + 1;
            for (int64_t d = d0; d <= d1; ++d) {
                if (d == p.owner) continue;
                const int64_t s0 = d * p.seg;
                const int64_t lr0 = max(m0, s0) - s0, lr1 = min(m1, s0 + p.seg) - s0;
                const int64_t tr0 = lr0 / p.ftm, tr1 = (lr1 - 1) / p.ftm;
                const int64_t items = (tr1 - tr0 + 1) * ntc;
                uint32_t *words = p.ready_out + d * p.fwords;
                for (int64_t it = lane; it < items; it += 64) {
                    const int64_t t = (tr0 + it / ntc) * p.ftiles_n + tc0 + it % ntc;
                    fetch_or_relaxed(words + (t >> 5), 1u << (t & 31), sys);
                }
            }
        }
    }
}

// ---- host side --------------------------------------------------------------------

struct TileCfg {
    int id, BM, BN;
    int slots;   // workgroups co-resident on one CU (LDS / register bound)
    double eff;  // relative per-CU throughput used by the automatic choice
};
// eff: sustained per-CU throughput relative to the best tile, from timing the
// tp=4 / tp=8 workloads on MI355X; cost = waves of tiles x tile area / eff.
constexpr TileCfg kTiles[] = {
    {AREPI_TILE_256x256_S4, 256, 256, 1, 1.00},
    {AREPI_TILE_128x256_S3, 128, 256, 2, 0.98},
    {AREPI_TILE_256x128_S3, 256, 128, 2, 0.97},
    {AREPI_TILE_256x256, 256, 256, 1, 0.93},
    {AREPI_TILE_128x128_S4, 128, 128, 2, 0.82},
    {AREPI_TILE_128x256, 128, 256, 1, 0.80},
    {AREPI_TILE_128x128, 128, 128, 2, 0.75},
    {AREPI_TILE_64x128, 64, 128, 3, 0.60},
    {AREPI_TILE_32x256, 32, 256, 2, 0.40},
};

const TileCfg *find_tile(int id) {
    for (const auto &t : kTiles)
        if (t.id == id) return &t;
    return nullptr;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Every flag tile (of every segment) must lie inside one compute tile, so that
// one workgroup can publish it.
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
    if (M * K * 2 >= lim || K * N * 2 >= lim || (M / R) * N * 2 >= lim)
        return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs: X, W and each peer partial must be below 2 GiB");
    return AREPI_OK;
}

int pick_tile(int64_t M, int64_t N, int64_t K, int R, int ftm, int ftn, bool publish) {
    (void)K;
    int best = -1;
    double best_cost = 0;
    for (const auto &t : kTiles) {
        if (publish && !flags_nest(M, N, R, ftm, ftn, t.BM, t.BN)) continue;
        const int64_t count = cdiv(M, t.BM) * cdiv(N, t.BN);
        // waves of co-resident tiles x work per CU per wave / efficiency
        const double cost = (double)cdiv(count, 256 * t.slots) * t.slots * t.BM * t.BN / t.eff;
        if (best < 0 || cost < best_cost) {
            best = t.id;
            best_cost = cost;
        }
    }
    return best;
}

template <int BM, int BN, int WM, int WN, int BK, int S, int WPE>
void launch(const GemmRsParams &p, hipStream_t stream) {
    constexpr int NT = (BM / WM) * (BN / WN) * 64;
    if (p.npeers <= 3)
        hipLaunchKernelGGL((gemm_rs_kernel<BM, BN, WM, WN, BK, S, WPE, 3>), dim3(p.nWG), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_rs_kernel<BM, BN, WM, WN, BK, S, WPE, kMaxR - 1>), dim3(p.nWG), dim3(NT), 0,
                           stream, p);
}

}  // namespace
}  // namespace arepi

using namespace arepi;

extern "C" int64_t arepi_gemm_rs_flag_words(int64_t M, int64_t N, int R, int flag_tile_m,
                                            int flag_tile_n) {
    if (R < 1 || R > kMaxR || M < 1 || M % R || N < 1 || flag_tile_m < 1 || flag_tile_n < 1)
        return fail(AREPI_EINVAL, "arepi_gemm_rs_flag_words: bad geometry");
    const int64_t tiles = cdiv(M / R, flag_tile_m) * cdiv(N, flag_tile_n);
    ok();
    return cdiv(tiles, 32);
}

extern "C" int arepi_gemm_rs_pick_tile(int64_t M, int64_t N, int64_t K, int R, int owner,
                                       int flag_tile_m, int flag_tile_n, int publish) {
    int rc = validate_shape(M, N, K, R, owner, flag_tile_m, flag_tile_n);
    if (rc) return rc;
    const int t = pick_tile(M, N, K, R, flag_tile_m, flag_tile_n, publish != 0);
    if (t < 0)
        return fail(AREPI_EUNSUPPORTED,
                    "arepi_gemm_rs: no compute tile holds whole flag tiles of " + std::to_string(flag_tile_m) +
                        "x" + std::to_string(flag_tile_n) + " (needed when ready_out is given)");
    ok();
    return t;
}

extern "C" int arepi_gemm_rs_supports(int64_t M, int64_t N, int64_t K, int R, int owner,
                                      int flag_tile_m, int flag_tile_n, int publish, int tile_cfg) {
    int rc = validate_shape(M, N, K, R, owner, flag_tile_m, flag_tile_n);
    if (rc) return rc;
    if (tile_cfg == AREPI_TILE_AUTO) {
        rc = arepi_gemm_rs_pick_tile(M, N, K, R, owner, flag_tile_m, flag_tile_n, publish);
        return rc < 0 ? rc : ok();
    }
    const TileCfg *t = find_tile(tile_cfg);
    if (!t) return fail(AREPI_EINVAL, "arepi_gemm_rs: tile_cfg=" + std::to_string(tile_cfg) + " is not an AREPI_TILE_* value");
    if (publish && !flags_nest(M, N, R, flag_tile_m, flag_tile_n, t->BM, t->BN))
        return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs: flag tiles " + std::to_string(flag_tile_m) + "x" +
                                            std::to_string(flag_tile_n) + " straddle " + std::to_string(t->BM) +
                                            "x" + std::to_string(t->BN) + " compute tiles");
    return ok();
}

extern "C" int arepi_gemm_rs_fused(const uint16_t *x, const uint16_t *w, const uint16_t *const *recv,
                                   const uint32_t *ready_in, uint16_t *out, uint16_t *send,
                                   uint32_t *ready_out, int64_t M, int64_t N, int64_t K, int R, int owner,
                                   int flag_tile_m, int flag_tile_n, int scope, int tile_cfg,
                                   uint32_t *status, int64_t spin_limit, arepi_stream_t stream) {
    const bool publish = ready_out != nullptr;
    int rc = arepi_gemm_rs_supports(M, N, K, R, owner, flag_tile_m, flag_tile_n, publish, tile_cfg);
    if (rc) return rc;
    auto bad = [](const std::string &m) { return fail(AREPI_EINVAL, "arepi_gemm_rs_fused: " + m); };
    if (!x || !w || !out) return bad("x, w and out must be non-NULL");
    if (!aligned16(x) || !aligned16(w) || !aligned16(out)) return bad("x, w and out must be 16-byte aligned");
    if (send && !aligned16(send)) return bad("send must be 16-byte aligned");
    if (publish && !send) return bad("ready_out needs send (the tiles it publishes)");
    if (scope != AREPI_SCOPE_AGENT && scope != AREPI_SCOPE_SYSTEM)
        return bad("scope=" + std::to_string(scope) + " is neither AREPI_SCOPE_AGENT nor AREPI_SCOPE_SYSTEM");
    if (R > 1) {
        if (!recv) return bad("recv must be a host array of R device pointers");
        if (!ready_in) return bad("ready_in must be non-NULL when R > 1");
        for (int p = 0; p < R; ++p) {
            if (p == owner) continue;
            if (!recv[p]) return bad("recv[" + std::to_string(p) + "] is NULL");
            if (!aligned16(recv[p])) return bad("recv[" + std::to_string(p) + "] must be 16-byte aligned");
        }
    }
    const int cfg = tile_cfg == AREPI_TILE_AUTO ? pick_tile(M, N, K, R, flag_tile_m, flag_tile_n, publish) : tile_cfg;
    const TileCfg *t = find_tile(cfg);

    GemmRsParams p{};
    p.x = x;
    p.w = w;
    p.npeers = 0;
    for (int i = 0; i < R; ++i)
        if (i != owner) p.peer[p.npeers++] = recv[i];
    p.ready_in = ready_in;
    p.out = out;
    p.send = send;
    p.ready_out = ready_out;
    p.status = status;
    p.M = M;
    p.N = N;
    p.K = K;
    p.seg = M / R;
    p.ftiles_n = cdiv(N, flag_tile_n);
    p.fwords = cdiv(cdiv(p.seg, flag_tile_m) * p.ftiles_n, 32);
    p.spin_limit = spin_limit > 0 ? spin_limit : kDefaultSpinLimit;
    p.R = R;
    p.owner = owner;
    p.ftm = flag_tile_m;
    p.ftn = flag_tile_n;
    p.system_scope = scope == AREPI_SCOPE_SYSTEM;
    p.nRB = (int)cdiv(M, t->BM);
    p.nCB = (int)cdiv(N, t->BN);
    // first row block after the owner's: the rotation puts the owner's last
    p.ob1 = (int)(cdiv((int64_t)(owner + 1) * p.seg, t->BM) % p.nRB);
    p.group = 4;
    p.xcd_chunk = 32;
    const int64_t nwg = (int64_t)p.nRB * p.nCB;
    if (nwg > (int64_t)1 << 30) return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_fused: too many tiles");
    p.nWG = (int)nwg;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (cfg) {
        case AREPI_TILE_256x256: launch<256, 256, 128, 128, 64, 2, 1>(p, s); break;
        case AREPI_TILE_128x256: launch<128, 256, 64, 128, 64, 2, 1>(p, s); break;
        case AREPI_TILE_128x128: launch<128, 128, 64, 64, 64, 2, 0>(p, s); break;
        case AREPI_TILE_64x128: launch<64, 128, 32, 64, 64, 2, 0>(p, s); break;
        case AREPI_TILE_32x256: launch<32, 256, 32, 64, 64, 2, 0>(p, s); break;
        case AREPI_TILE_256x256_S4: launch<256, 256, 128, 128, 32, 4, 1>(p, s); break;
        case AREPI_TILE_256x128_S3: launch<256, 128, 128, 64, 32, 3, 2>(p, s); break;
        case AREPI_TILE_128x256_S3: launch<128, 256, 64, 128, 32, 3, 2>(p, s); break;
        case AREPI_TILE_128x128_S4: launch<128, 128, 64, 64, 32, 4, 2>(p, s); break;
        default: return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_fused: no kernel for tile " + std::to_string(cfg));
    }
    return check_launch("arepi_gemm_rs_fused");
}
