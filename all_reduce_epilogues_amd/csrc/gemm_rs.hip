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
    const uint16_t *recv[kMaxR];
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

__device__ __forceinline__ uint32_t dword_of(const uint4 &v, int d) {
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// 16-byte load, or zeros when `pred` is false (returned by value so the
// compiler never needs the address of a zero constant).
__device__ __forceinline__ uint4 load16_or_zero(const uint16_t *p, bool pred) {
    uint4 r = make_uint4(0u, 0u, 0u, 0u);
    if (pred) r = *reinterpret_cast<const uint4 *>(p);
    return r;
}

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
// Offset (in bf16 elements) of 16-byte chunk c of row r of a [rows][BK] tile.
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 3); }

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

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64, 1)
    gemm_rs_kernel(const GemmRsParams p) {
    constexpr int NWN = BN / WN;
    constexpr int NT = (BM / WM) * NWN * 64;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int A_LD = BM * (BK / 8) / NT;        // 16-byte X chunks per thread
    constexpr int B_LD = (BK / 4) * (BN / 8) / NT;  // 4x8 W blocks per thread
    constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
    constexpr int EPS = WN + 8;                      // epilogue LDS row stride (floats)
    static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the thread count");
    static_assert(A_LD * NT == BM * (BK / 8) && B_LD * NT == (BK / 4) * (BN / 8), "uneven load split");
    static_assert((BM / WM) * NWN * 32 * EPS * 4 <= 2 * (A_ELEMS + B_ELEMS) * 2, "epilogue LDS");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (A_ELEMS + B_ELEMS)];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    int rb, cb;
    tile_of_block(p, blockIdx.x, rb, cb);
    const int64_t m0 = (int64_t)rb * BM, n0 = (int64_t)cb * BN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const uint16_t *__restrict__ x = p.x;
    const uint16_t *__restrict__ w = p.w;

    uint4 ra[A_LD];
    uint4 rw[B_LD][4];

    auto load_tile = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int q = tid + i * NT;
            const int64_t gm = m0 + (q >> 3), gk = k0 + (q & 7) * 8;
            ra[i] = load16_or_zero(x + gm * K + gk, gm < M && gk < K);
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int q = tid + i * NT;
            const int kb4 = (q & 1) + 2 * ((q >> 1) / (BN / 8));
            const int nb = (q >> 1) % (BN / 8);
            const int64_t gn = n0 + nb * 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t gk = k0 + kb4 * 4 + j;
                rw[i][j] = load16_or_zero(w + gk * N + gn, gk < K && gn < N);
            }
        }
    };

    auto store_tile = [&](int buf) {
        uint16_t *As = smem + buf * (A_ELEMS + B_ELEMS);
        uint16_t *Bs = As + A_ELEMS;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int q = tid + i * NT;
            *reinterpret_cast<uint4 *>(As + lds_off(q >> 3, q & 7)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int q = tid + i * NT;
            const int kb4 = (q & 1) + 2 * ((q >> 1) / (BN / 8));
            const int nb = (q >> 1) % (BN / 8);
#pragma unroll
            for (int jn = 0; jn < 8; ++jn) {
                const int d = jn >> 1;
                const uint32_t w0 = dword_of(rw[i][0], d), w1 = dword_of(rw[i][1], d);
                const uint32_t w2 = dword_of(rw[i][2], d), w3 = dword_of(rw[i][3], d);
                uint32_t lo, hi;
                if (jn & 1) {
                    lo = (w0 >> 16) | (w1 & 0xffff0000u);
                    hi = (w2 >> 16) | (w3 & 0xffff0000u);
                } else {
                    lo = (w0 & 0xffffu) | (w1 << 16);
                    hi = (w2 & 0xffffu) | (w3 << 16);
                }
                const int n = nb * 8 + jn;
                *reinterpret_cast<uint2 *>(Bs + lds_off(n, kb4 >> 1) + (kb4 & 1) * 4) = make_uint2(lo, hi);
            }
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    auto compute = [&](int buf) {
        const uint16_t *As = smem + buf * (A_ELEMS + B_ELEMS);
        const uint16_t *Bs = As + A_ELEMS;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int kc = kk * 2 + (lane >> 5);
            bf16x8 a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = *reinterpret_cast<const bf16x8 *>(As + lds_off(wm * WM + i * 32 + (lane & 31), kc));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b[j] = *reinterpret_cast<const bf16x8 *>(Bs + lds_off(wn * WN + j * 32 + (lane & 31), kc));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    // ---- mainloop ---------------------------------------------------------------
    const int KT = (int)((K + BK - 1) / BK);
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        if (more) load_tile((int64_t)(kt + 1) * BK);
        compute(kt & 1);
        if (more) store_tile((kt + 1) & 1);
        __syncthreads();
    }

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

    float *ep = reinterpret_cast<float *>(smem) + wave * 32 * EPS;
    constexpr int CPR = WN / 8;     // 16-byte chunks per epilogue row
    constexpr int RPS = 64 / CPR;   // rows per step
    constexpr int STEPS = 32 / RPS;
    const int R = p.R, owner = p.owner;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                ep[row * EPS + j * 32 + (lane & 31)] = acc[i][j][r];
            }
        __syncthreads();
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int row = st * RPS + lane / CPR, ch = lane % CPR;
            const int64_t gr = m0 + wm * WM + i * 32 + row;
            const int64_t gc = n0 + wn * WN + ch * 8;
            if (gr < M && gc < N) {
                const float4 v0 = *reinterpret_cast<const float4 *>(ep + row * EPS + ch * 8);
                const float4 v1 = *reinterpret_cast<const float4 *>(ep + row * EPS + ch * 8 + 4);
                float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                if (gr >= oseg0 && gr < oseg1) {
                    const int64_t off = (gr - oseg0) * N + gc;
#pragma unroll
                    for (int pr = 0; pr < kMaxR; ++pr) {
                        if (pr < R && pr != owner) {
                            float f[8];
                            unpack8(*reinterpret_cast<const uint4 *>(p.recv[pr] + off), f);
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] = v[e] + f[e];
                        }
                    }
                    *reinterpret_cast<uint4 *>(p.out + off) = pack8(v);
                } else if (p.send) {
                    *reinterpret_cast<uint4 *>(p.send + gr * N + gc) = pack8(v);
                }
            }
        }
        __syncthreads();
    }

    // Publish the send tiles: drain this thread's stores, balanced barrier, one
    // release, then relaxed bit sets.
    if (p.ready_out && has_other) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if (wave == 0) {
            fence_release(sys);
            const int64_t d0 = m0 / p.seg, d1 = (m1 - 1) / p.seg;
            const int64_t tc0 = n0 / p.ftn, tc1 = (min(n0 + BN, N) - 1) / p.ftn;
            const int64_t ntc = tc1 - tc0 + 1;
            for (int64_t d = d0; d <= d1; ++d) {
                if (d == owner) continue;
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
    double eff;  // relative per-CU throughput used by the automatic choice
};
constexpr TileCfg kTiles[] = {
    {AREPI_TILE_256x256, 256, 256, 1.00},
    {AREPI_TILE_128x256, 128, 256, 0.92},
    {AREPI_TILE_128x128, 128, 128, 0.80},
    {AREPI_TILE_64x128, 64, 128, 0.55},
    {AREPI_TILE_32x256, 32, 256, 0.50},
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
    if (M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 31))
        return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs: dimensions above 2^31 are not supported");
    return AREPI_OK;
}

int pick_tile(int64_t M, int64_t N, int64_t K, int R, int ftm, int ftn, bool publish) {
    (void)K;
    int best = -1;
    double best_cost = 0;
    for (const auto &t : kTiles) {
        if (publish && !flags_nest(M, N, R, ftm, ftn, t.BM, t.BN)) continue;
        const int64_t count = cdiv(M, t.BM) * cdiv(N, t.BN);
        const double cost = (double)cdiv(count, 256) * t.BM * t.BN / t.eff;
        if (best < 0 || cost < best_cost) {
            best = t.id;
            best_cost = cost;
        }
    }
    return best;
}

template <int BM, int BN, int WM, int WN>
void launch(const GemmRsParams &p, hipStream_t stream) {
    constexpr int NT = (BM / WM) * (BN / WN) * 64;
    hipLaunchKernelGGL((gemm_rs_kernel<BM, BN, WM, WN>), dim3(p.nWG), dim3(NT), 0, stream, p);
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
    for (int i = 0; i < kMaxR; ++i) p.recv[i] = (i < R && i != owner && recv) ? recv[i] : nullptr;
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
        case AREPI_TILE_256x256: launch<256, 256, 128, 128>(p, s); break;
        case AREPI_TILE_128x256: launch<128, 256, 64, 128>(p, s); break;
        case AREPI_TILE_128x128: launch<128, 128, 64, 64>(p, s); break;
        case AREPI_TILE_64x128: launch<64, 128, 32, 64>(p, s); break;
        case AREPI_TILE_32x256: launch<32, 256, 32, 64>(p, s); break;
        default: return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_fused: no kernel for tile " + std::to_string(cfg));
    }
    return check_launch("arepi_gemm_rs_fused");
}
