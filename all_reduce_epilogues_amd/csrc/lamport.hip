// lamport.hip -- Lamport-sentinel all-reduce + RMSNorm for gfx950.
//
// Protocol from ROCm/aiter PR #4977 "[HIP] Single-kernel Lamport fused
// all-reduce + RMSNorm (opt-in)" (Approach section; bring-up commit notes on
// arming outside graph capture and on a private staging area):
//   * staging words are armed with -0.0 (bf16 0x8000);
//   * a producer maps 0x8000 to 0x0000 on the final bf16 bits and stores with
//     no fence -- the data is its own flag, and word order inside a pack does
//     not matter because a half-landed pack still shows a sentinel;
//   * a consumer treats a 16-byte pack as arrived when none of its eight words
//     is 0x8000, consumes it and re-arms it (each pack has exactly one consumer
//     thread, so the re-arm needs no extra synchronisation).
//
// gfx950 mapping: the publisher's stores are device-coherent 8-byte atomics
// (relaxed, agent or system scope; the compiler emits sc1 stores), so a
// consumer polling from another XCD sees them while the publisher runs.  The
// consumer reads each pack once with a plain 16-byte load and only polls
// coherently (sc1 loads) when the pack still shows a sentinel.
//
// Consumer layout: one workgroup of NT threads per row; thread t owns packs
// t, t+NT, ... of the row (coalesced 16-byte columns, PPT of them), keeps the
// fp32 slot sums of its packs in registers, reduces sum(s^2) across the
// workgroup (wave shuffles, then LDS), and writes the normalised row.  The
// launch takes NT = 256 with one pack per thread up to 256 packs (N <= 2048),
// NT = 512 with two up to 1024 packs (N = 7168: 896 packs), and NT = 512
// with four above that.  (Other row widths, persistent row loops and a
// slot-interleaved staging layout measured slower or equal on MI355X.)
#include <algorithm>
#include <mutex>
#include <string>

#include "arepi_internal.h"

namespace arepi {
namespace {

constexpr uint64_t kSent4 = 0x8000800080008000ull;
constexpr uint32_t kSent2 = 0x80008000u;

// True when any 16-bit lane of v holds the sentinel (exact: the classic
// zero-lane test is exact for the "some lane is zero" decision).
__device__ __forceinline__ bool has_sentinel(uint64_t v) {
    const uint64_t t = v ^ kSent4;
    return ((t - 0x0001000100010001ull) & ~t & 0x8000800080008000ull) != 0;
}

// Map every 0x8000 half of a 32-bit word to 0x0000.
__device__ __forceinline__ uint32_t canon2(uint32_t u) {
    const uint32_t lo = ((u & 0xffffu) == 0x8000u) ? 0u : (u & 0xffffu);
    const uint32_t hi = ((u >> 16) == 0x8000u) ? 0u : (u & 0xffff0000u);
    return lo | hi;
}

__global__ void prefill_kernel(uint4 *__restrict__ dst, int64_t n16, uint16_t *__restrict__ tail,
                               int64_t n_tail) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const uint4 s = make_uint4(kSent2, kSent2, kSent2, kSent2);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = s;
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < n_tail) tail[threadIdx.x] = 0x8000u;
}

// One workgroup per (slot, position in that slot's publication order).
__global__ void __launch_bounds__(256) publish_kernel(const uint16_t *__restrict__ src,
                                                     uint16_t *__restrict__ staging,
                                                     const int32_t *__restrict__ order, int64_t M,
                                                     int64_t N, int tile_m, int tile_n,
                                                     int64_t tiles_n, int64_t tiles, int system) {
    const int64_t slot = blockIdx.x / tiles;
    const int64_t pos = blockIdx.x % tiles;
    const int64_t t = order[slot * tiles + pos];
    if (t < 0 || t >= tiles) return;  // not a tile id: publishes nothing
    const int64_t r0 = (t / tiles_n) * tile_m, c0 = (t % tiles_n) * tile_n;
    const int64_t rows = min((int64_t)tile_m, M - r0);
    const int64_t packs = (min((int64_t)tile_n, N - c0)) / 8;
    const uint16_t *s = src + slot * M * N;
    uint16_t *d = staging + slot * M * N;
    const bool sys = system != 0;
    for (int64_t i = threadIdx.x; i < rows * packs; i += blockDim.x) {
        const int64_t off = (r0 + i / packs) * N + c0 + (i % packs) * 8;
        const uint4 q = *reinterpret_cast<const uint4 *>(s + off);
        const uint64_t lo = (uint64_t)canon2(q.x) | ((uint64_t)canon2(q.y) << 32);
        const uint64_t hi = (uint64_t)canon2(q.z) | ((uint64_t)canon2(q.w) << 32);
        uint64_t *p = reinterpret_cast<uint64_t *>(d + off);
        store64_coherent(p, lo, sys);
        store64_coherent(p + 1, hi, sys);
    }
}

// Consumer.  A kernel launch is an acquire at agent scope, so inside this
// launch a plain load of a staging pack returns either the sentinel or data
// published during the launch -- never an older payload.
//
// Fast pass (no branches, so the compiler's memory-counter waits stay exact):
// one nontemporal 16-byte buffer load per (pack, slot), the S loads of pack
// j+1 in flight while pack j is checked and summed; a pack whose S slots all
// arrived is re-armed at once.  Packs past the row end and slots past S use an
// out-of-range offset: the load returns zeros (no sentinel, adds +0) and the
// store is dropped.  A pack in which any slot still shows a sentinel is
// neither summed for good nor re-armed; it is marked and redone after the fast
// pass, slot by slot in the same order, polling with device-coherent loads
// (which observe a producer running concurrently on another XCD) until the
// pack lands or the spin budget runs out.  Every pack has exactly one consumer
// thread, so re-arming needs no extra synchronisation; the kernel end
// releases the re-arms before any later publication into the same staging.
constexpr uint32_t kOob = 0x80000000u;  // at or past every resource's size (host-checked)

__device__ __forceinline__ uint64_t lo64(const i32x4 v) { return (uint64_t)(uint32_t)v[0] | ((uint64_t)(uint32_t)v[1] << 32); }
__device__ __forceinline__ uint64_t hi64(const i32x4 v) { return (uint64_t)(uint32_t)v[2] | ((uint64_t)(uint32_t)v[3] << 32); }
__device__ __forceinline__ void add8(float (&acc)[8], uint64_t lo, uint64_t hi) {
    const uint4 v = make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
    float f[8];
    unpack8(v, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + f[e];
}

template <int PPT, int NT>
__global__ void __launch_bounds__(NT) ar_rmsnorm_kernel(uint16_t *__restrict__ staging,
                                                        const uint16_t *__restrict__ gamma,
                                                        uint16_t *__restrict__ out, int64_t M,
                                                        int64_t N, int S, float eps, int system,
                                                        uint32_t *status, int64_t spin_limit) {
    __shared__ float red[NT / 64];
    const int tid = threadIdx.x;
    const int packs = (int)(N / 8);
    // Byte offsets are 32-bit: 8 * M * N * 2 <= 2^31 (host-checked), so the
    // offset of any of the 8 slots stays below kOob, and slots past S fall
    // outside the resource (S planes) without a test.
    const uint32_t plane2 = (uint32_t)(M * N * 2), row2 = (uint32_t)((int64_t)blockIdx.x * N * 2);
    const __amdgpu_buffer_rsrc_t st_rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)staging, 0, (int)(plane2 * (uint32_t)S), kBufferDword3);
    const bool sys = system != 0;
    const i32x4 armed = {(int)kSent2, (int)kSent2, (int)kSent2, (int)kSent2};
    // slot-0 offset of this thread's pack j, or kOob past the row end
    auto pack_off = [&](int j) {
        const int pk = tid + j * NT;
        return pk < packs ? row2 + (uint32_t)pk * 16u : kOob;
    };

    float s[PPT][8];
    uint32_t bad = 0;  // bit j: pack j still showed a sentinel in the fast pass
    i32x4 q[2][8];
    auto issue = [&](int j, i32x4 (&d)[8]) {
        const uint32_t o = pack_off(j);
#pragma unroll
        for (int sl = 0; sl < 8; ++sl)
            d[sl] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(st_rs, o + (uint32_t)sl * plane2,
                                                                                    0, kAuxNontemporal));
    };
    issue(0, q[0]);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        if (j + 1 < PPT) issue(j + 1, q[(j + 1) & 1]);
        bool b = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) s[j][e] = 0.f;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            const uint64_t lo = lo64(q[j & 1][sl]), hi = hi64(q[j & 1][sl]);
            b |= has_sentinel(lo) | has_sentinel(hi);
            add8(s[j], lo, hi);
        }
        bad |= (uint32_t)b << j;
        const uint32_t o = b ? kOob : pack_off(j);
#pragma unroll
        for (int sl = 0; sl < 8; ++sl)
            __builtin_amdgcn_raw_buffer_store_b128(armed, st_rs, o + (uint32_t)sl * plane2, 0, kAuxNontemporal);
    }

    // Slow pass: packs that had not fully landed, redone in slot order.
    if (bad) {
        int64_t spins = 0;
        const uint64_t t0 = spin_clock();
        bool gave_up = false;
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            if (!((bad >> j) & 1u)) continue;
#pragma unroll
            for (int e = 0; e < 8; ++e) s[j][e] = 0.f;
            uint16_t *base = staging + (int64_t)blockIdx.x * N + (int64_t)(tid + j * NT) * 8;
            for (int sl = 0; sl < S; ++sl) {
                uint64_t *p64 = reinterpret_cast<uint64_t *>(base + (int64_t)sl * M * N);
                uint64_t lo = load64_coherent(p64, sys), hi = load64_coherent(p64 + 1, sys);
                while (!gave_up && (has_sentinel(lo) || has_sentinel(hi))) {
                    if (spin_expired(spin_limit, spins, t0)) {
                        gave_up = true;
                        if (status) atomicOr(status, (uint32_t)AREPI_STATUS_TIMEOUT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                    lo = load64_coherent(p64, sys);
                    hi = load64_coherent(p64 + 1, sys);
                }
                add8(s[j], lo, hi);
                store16_nt(base + (int64_t)sl * M * N, make_uint4(kSent2, kSent2, kSent2, kSent2));
            }
        }
    }

    // workgroup sum of s^2 (pack-major, then element order, per thread)
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < PPT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = ss + s[j][e] * s[j][e];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) tot = tot + red[w];
    const float r = 1.0f / sqrtf(tot / (float)N + eps);

    const __amdgpu_buffer_rsrc_t g_rs = __builtin_amdgcn_make_buffer_rsrc((void *)gamma, 0, (int)(N * 2), kBufferDword3);
    const __amdgpu_buffer_rsrc_t o_rs = __builtin_amdgcn_make_buffer_rsrc((void *)out, 0, (int)plane2, kBufferDword3);
    i32x4 g[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int pk = tid + j * NT;
        g[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             g_rs, pk < packs ? (uint32_t)pk * 16u : kOob, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int pk = tid + j * NT;
        float gf[8], y[8];
        unpack8(make_uint4((uint32_t)g[j][0], (uint32_t)g[j][1], (uint32_t)g[j][2], (uint32_t)g[j][3]), gf);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (s[j][e] * r) * gf[e];
        const uint4 o = pack8(y);
        const i32x4 ov = {(int)o.x, (int)o.y, (int)o.z, (int)o.w};
        __builtin_amdgcn_raw_buffer_store_b128(ov, o_rs, pk < packs ? row2 + (uint32_t)pk * 16u : kOob, 0,
                                               kAuxNontemporal);
    }
}

// ---- two-phase form (ROCm/aiter PR #4977, Approach: phase A is the
// reduce-scatter with cross-device stores, phase B the consumer) ------------
//
// R ranks each hold a partial in[r] [M,N]; every rank has its own staging
// [M,N] (armed with the sentinel).  The flattened tensor is cut into R parts
// of ceil(P/R) 16-byte packs.  One launch on rank `rank`:
//  Phase A: for each pack of part `rank`, add the R partials in fp32 (ranks
//    ascending), round once to bf16, map -0.0 to +0.0 and store the pack into
//    EVERY rank's staging (device-coherent 16-byte stores; no fence: the data
//    is the flag).
//  Phase B: each row of this rank's staging -- whose packs come from every
//    rank's phase A -- is consumed as in the one-shot consumer with one slot:
//    a plain load first, a coherent re-poll for packs still armed, re-arm of
//    every pack consumed, then RMSNorm of the bf16 values into out.
// Phase B of one block waits for phase A work of other blocks of the same
// launch, so the launch is persistent: the grid is clamped to the workgroups
// that can be resident at once, and every block finishes all of its phase A
// work (which waits for nothing) before it polls.  Both phases are
// grid-stride loops; phase A has no barriers, phase B's trip count is
// block-uniform and each row ends with a barrier (the reduction slots are
// reused by the next row).
constexpr int kMaxRanks = 8;
// Cache-policy operands of device-coherent 16-byte stores: sc1 (agent scope)
// and sc0 sc1 (system scope), the bits the compiler gives the scoped relaxed
// atomic stores of the same scope (checked against the emitted assembly).
constexpr int kAuxCoherentAgent = 16;
constexpr int kAuxCoherentSystem = 17;

struct Lamport2Params {
    const uint16_t *in[kMaxRanks];
    uint16_t *stg[kMaxRanks];
    const uint16_t *gamma;
    uint16_t *out;
    uint32_t *status;
    int64_t M, N, spin_limit;
    int R, rank, system, phase_b;
    float eps;
};

template <int PPT, int NT>
__global__ void __launch_bounds__(NT) lamport2_kernel(const Lamport2Params p) {
    __shared__ float red[NT / 64];
    const int tid = threadIdx.x;
    const bool sys = p.system != 0;
    const int64_t total = p.M * p.N / 8;  // 16-byte packs
    const int64_t q = (total + p.R - 1) / p.R;
    const int64_t a0 = min(total, q * p.rank), a1 = min(total, a0 + q);
    const uint32_t plane2 = (uint32_t)(p.M * p.N * 2);

    // ---- phase A ----
    // Two packs per thread and iteration (the second one GS packs further),
    // so each thread has 2R loads in flight.
    const int64_t GS = (int64_t)gridDim.x * NT;
    auto reduce_pack = [&](const uint4 (&v)[kMaxRanks]) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int r = 0; r < kMaxRanks; ++r)
            if (r < p.R) {
                float f[8];
                unpack8(v[r], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = acc[e] + f[e];
            }
        const uint4 t = pack8(acc);
        const i32x4 c = {(int)canon2(t.x), (int)canon2(t.y), (int)canon2(t.z), (int)canon2(t.w)};
        return c;
    };
    auto store_pack = [&](const i32x4 c, int64_t k) {
#pragma unroll
        for (int d = 0; d < kMaxRanks; ++d)
            if (d < p.R) {
                const __amdgpu_buffer_rsrc_t rs =
                    __builtin_amdgcn_make_buffer_rsrc((void *)p.stg[d], 0, (int)plane2, kBufferDword3);
                if (sys)
                    __builtin_amdgcn_raw_buffer_store_b128(c, rs, (uint32_t)(k * 16), 0, kAuxCoherentSystem);
                else
                    __builtin_amdgcn_raw_buffer_store_b128(c, rs, (uint32_t)(k * 16), 0, kAuxCoherentAgent);
            }
    };
    for (int64_t k = a0 + (int64_t)blockIdx.x * NT + tid; k < a1; k += 2 * GS) {
        const bool two = k + GS < a1;
        const int64_t k2 = two ? k + GS : k;  // (clamped: loaded, never stored)
        uint4 v[kMaxRanks], w[kMaxRanks];
#pragma unroll
        for (int r = 0; r < kMaxRanks; ++r)
            if (r < p.R) {
                v[r] = load16_nt(p.in[r] + k * 8);
                w[r] = load16_nt(p.in[r] + k2 * 8);
            }
        store_pack(reduce_pack(v), k);
        const i32x4 c2 = reduce_pack(w);
        if (two) store_pack(c2, k2);
    }
    if (!p.phase_b) return;

    // ---- phase B ----
    const int packs = (int)(p.N / 8);
    uint16_t *const mine = p.stg[p.rank];
    const __amdgpu_buffer_rsrc_t st_rs = __builtin_amdgcn_make_buffer_rsrc((void *)mine, 0, (int)plane2, kBufferDword3);
    const __amdgpu_buffer_rsrc_t g_rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.gamma, 0, (int)(p.N * 2), kBufferDword3);
    const __amdgpu_buffer_rsrc_t o_rs = __builtin_amdgcn_make_buffer_rsrc((void *)p.out, 0, (int)plane2, kBufferDword3);
    const i32x4 armed = {(int)kSent2, (int)kSent2, (int)kSent2, (int)kSent2};
    int64_t spins = 0;
    bool gave_up = false;
    // The plain loads of the block's next row are issued before the current
    // row is reduced and written, so they are in flight across its barriers
    // (a pack that is still armed when loaded goes to the slow pass, as any).
    auto load_row = [&](int64_t row, i32x4 (&dst)[PPT]) {
        const uint32_t r2 = row < p.M ? (uint32_t)(row * p.N * 2) : 0u;
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int pk = tid + j * NT;
            const uint32_t off = row < p.M && pk < packs ? r2 + (uint32_t)pk * 16u : kOob;
            dst[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(st_rs, off, 0, kAuxNontemporal));
        }
    };
    i32x4 qv[PPT];
    load_row(blockIdx.x, qv);
    for (int64_t row = blockIdx.x; row < p.M; row += gridDim.x) {
        const uint32_t row2 = (uint32_t)(row * p.N * 2);
        auto pack_off = [&](int j) {
            const int pk = tid + j * NT;
            return pk < packs ? row2 + (uint32_t)pk * 16u : kOob;
        };
        i32x4 qn[PPT];
        load_row(row + gridDim.x, qn);
        float s[PPT][8];
        uint32_t bad = 0;
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const uint64_t lo = lo64(qv[j]), hi = hi64(qv[j]);
            const bool b = has_sentinel(lo) | has_sentinel(hi);
#pragma unroll
            for (int e = 0; e < 8; ++e) s[j][e] = 0.f;
            add8(s[j], lo, hi);
            bad |= (uint32_t)b << j;
            __builtin_amdgcn_raw_buffer_store_b128(armed, st_rs, b ? kOob : pack_off(j), 0, kAuxNontemporal);
        }
        // slow pass: packs that had not landed, polled coherently
        if (bad) {
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                if (!((bad >> j) & 1u)) continue;
                uint16_t *base = mine + row * p.N + (int64_t)(tid + j * NT) * 8;
                uint64_t *p64 = reinterpret_cast<uint64_t *>(base);
                uint64_t lo = load64_coherent(p64, sys), hi = load64_coherent(p64 + 1, sys);
                const uint64_t t0 = spin_clock();
                while (!gave_up && (has_sentinel(lo) || has_sentinel(hi))) {
                    if (spin_expired(p.spin_limit, spins, t0)) {
                        gave_up = true;
                        if (p.status) atomicOr(p.status, (uint32_t)AREPI_STATUS_TIMEOUT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                    lo = load64_coherent(p64, sys);
                    hi = load64_coherent(p64 + 1, sys);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) s[j][e] = 0.f;
                add8(s[j], lo, hi);
                store16_nt(base, make_uint4(kSent2, kSent2, kSent2, kSent2));
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < PPT; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = ss + s[j][e] * s[j][e];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
        if ((tid & 63) == 0) red[tid >> 6] = ss;
        __syncthreads();
        float tot = red[0];
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) tot = tot + red[w];
        const float r = 1.0f / sqrtf(tot / (float)p.N + p.eps);
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int pk = tid + j * NT;
            const i32x4 g = __builtin_bit_cast(
                i32x4, __builtin_amdgcn_raw_buffer_load_b128(g_rs, pk < packs ? (uint32_t)pk * 16u : kOob, 0, 0));
            float gf[8], y[8];
            unpack8(make_uint4((uint32_t)g[0], (uint32_t)g[1], (uint32_t)g[2], (uint32_t)g[3]), gf);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (s[j][e] * r) * gf[e];
            const uint4 o = pack8(y);
            const i32x4 ov = {(int)o.x, (int)o.y, (int)o.z, (int)o.w};
            __builtin_amdgcn_raw_buffer_store_b128(ov, o_rs, pack_off(j), 0, kAuxNontemporal);
        }
        __syncthreads();  // red[] is rewritten by the next row
#pragma unroll
        for (int j = 0; j < PPT; ++j) qv[j] = qn[j];
    }
}

template <int PPT, int NT>
int launch_lamport2(const Lamport2Params &p, hipStream_t s) {
    // persistent grid: at most the workgroups resident at once
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, lamport2_kernel<PPT, NT>, NT, 0) != hipSuccess ||
        cus < 1 || per_cu < 1)
        return fail(AREPI_ELAUNCH, "arepi_ar_rmsnorm_lamport_2phase: occupancy query failed");
    const int64_t total = p.M * p.N / 8, q = (total + p.R - 1) / p.R;
    int64_t want = std::max<int64_t>(p.phase_b ? p.M : 1, (q + NT - 1) / NT);
    const int64_t grid = std::min<int64_t>(want, (int64_t)cus * per_cu);
    hipLaunchKernelGGL((lamport2_kernel<PPT, NT>), dim3((unsigned)std::max<int64_t>(grid, 1)), dim3(NT), 0, s, p);
    return check_launch("arepi_ar_rmsnorm_lamport_2phase");
}

}  // namespace
}  // namespace arepi

using namespace arepi;

extern "C" int arepi_lamport_prefill(uint16_t *staging, int64_t elems, arepi_stream_t stream) {
    if (elems < 0) return fail(AREPI_EINVAL, "arepi_lamport_prefill: elems=" + std::to_string(elems) + " must be >= 0");
    if (elems == 0) return ok();
    if (!staging) return fail(AREPI_EINVAL, "arepi_lamport_prefill: staging is NULL");
    if (!aligned16(staging)) return fail(AREPI_EINVAL, "arepi_lamport_prefill: staging must be 16-byte aligned");
    const int64_t n16 = elems / 8, tail = elems % 8;
    int64_t grid = (n16 + 255) / 256;
    if (grid > 8192) grid = 8192;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<uint4 *>(staging), n16, staging + n16 * 8, tail);
    return check_launch("arepi_lamport_prefill");
}

extern "C" int arepi_lamport_publish(const uint16_t *src, uint16_t *staging, const int32_t *order, int S,
                                     int64_t M, int64_t N, int tile_m, int tile_n, int scope,
                                     arepi_stream_t stream) {
    auto bad = [](const std::string &m) { return fail(AREPI_EINVAL, "arepi_lamport_publish: " + m); };
    if (S < 1 || S > 8) return bad("S=" + std::to_string(S) + " outside [1, 8]");
    if (M < 0) return bad("M=" + std::to_string(M) + " must be >= 0");
    if (N < 8 || N % 8) return bad("N=" + std::to_string(N) + " must be a positive multiple of 8");
    if (tile_m < 1 || tile_n < 8 || tile_n % 8)
        return bad("tile " + std::to_string(tile_m) + "x" + std::to_string(tile_n) +
                   " needs tile_m >= 1 and tile_n a positive multiple of 8");
    if (scope != AREPI_SCOPE_AGENT && scope != AREPI_SCOPE_SYSTEM) return bad("scope must be AGENT or SYSTEM");
    if (M == 0) return ok();
    if (!src || !staging || !order) return bad("src, staging and order must be non-NULL");
    if (!aligned16(src) || !aligned16(staging)) return bad("src and staging must be 16-byte aligned");
    const int64_t tiles_n = (N + tile_n - 1) / tile_n;
    const int64_t tiles = ((M + tile_m - 1) / tile_m) * tiles_n;
    if (tiles * S > (int64_t)1 << 31) return fail(AREPI_EUNSUPPORTED, "arepi_lamport_publish: too many tiles");
    hipLaunchKernelGGL(publish_kernel, dim3((unsigned)(tiles * S)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), src, staging, order, M, N, tile_m, tile_n, tiles_n,
                       tiles, scope == AREPI_SCOPE_SYSTEM ? 1 : 0);
    return check_launch("arepi_lamport_publish");
}

// Shared validation and launch of the two consumer entry points.
static int check_consumer(const char *who, int64_t M, int64_t N, int S, float eps, int scope) {
    auto bad = [who](const std::string &m) { return fail(AREPI_EINVAL, std::string(who) + ": " + m); };
    if (S < 1 || S > 8) return bad("S=" + std::to_string(S) + " outside [1, 8]");
    if (M < 0) return bad("M=" + std::to_string(M) + " must be >= 0");
    if (N < 8 || N % 8) return bad("N=" + std::to_string(N) + " must be a positive multiple of 8");
    if (N > 16384)
        return fail(AREPI_EUNSUPPORTED, std::string(who) + ": N=" + std::to_string(N) + " above 16384");
    if (!(eps >= 0.0f)) return bad("eps must be >= 0");
    if (scope != AREPI_SCOPE_AGENT && scope != AREPI_SCOPE_SYSTEM) return bad("scope must be AGENT or SYSTEM");
    return AREPI_OK;
}

static int launch_consumer(const char *who, uint16_t *staging, const uint16_t *gamma, uint16_t *out, int64_t M,
                           int64_t N, int S, float eps, int scope, uint32_t *status, int64_t spin_limit,
                           hipStream_t s) {
    if (M * N * 2 * 8 > (int64_t)1 << 31)
        return fail(AREPI_EUNSUPPORTED,
                    std::string(who) + ": one staging slot (M*N*2 bytes) must be at most 256 MiB");
    const int64_t packs = N / 8;
    const int64_t lim = spin_bound(spin_limit);
    const int sys = scope == AREPI_SCOPE_SYSTEM ? 1 : 0;
    const int ppt = (int)((packs + 255) / 256);
#define AREPI_RMS_LAUNCH(P, T)                                                                                   \
    hipLaunchKernelGGL((ar_rmsnorm_kernel<P, T>), dim3((unsigned)M), dim3(T), 0, s, staging, gamma, out, M, N, S, \
                       eps, sys, status, lim)
    // 512-thread rows from 257 packs up: at N = 7168 (896 packs, two per
    // thread) this timed ~1% faster than 256 threads with four packs each
    if (ppt <= 1)
        AREPI_RMS_LAUNCH(1, 256);
    else if (packs <= 1024)
        AREPI_RMS_LAUNCH(2, 512);
    else
        AREPI_RMS_LAUNCH(4, 512);
#undef AREPI_RMS_LAUNCH
    return check_launch(who);
}

extern "C" int arepi_ar_rmsnorm_lamport(uint16_t *staging, const uint16_t *gamma, uint16_t *out, int64_t M,
                                        int64_t N, int S, float eps, int scope, uint32_t *status,
                                        int64_t spin_limit, arepi_stream_t stream) {
    const char *who = "arepi_ar_rmsnorm_lamport";
    if (const int rc = check_consumer(who, M, N, S, eps, scope)) return rc;
    if (M == 0) return ok();
    if (!staging || !gamma || !out)
        return fail(AREPI_EINVAL, std::string(who) + ": staging, gamma and out must be non-NULL");
    if (!aligned16(staging) || !aligned16(gamma) || !aligned16(out))
        return fail(AREPI_EINVAL, std::string(who) + ": staging, gamma and out must be 16-byte aligned");
    return launch_consumer(who, staging, gamma, out, M, N, S, eps, scope, status, spin_limit,
                           reinterpret_cast<hipStream_t>(stream));
}

// ---- consumer with library-held staging ---------------------------------------
//
// For callers that cannot allocate device memory.  The staging is a fixed-size
// static device array; every GPU the library runs on holds its own copy at its
// own address.  In host code the array's name is only a host-side stand-in, so
// host code never hands it to a kernel: the device address is resolved once
// per device with hipGetSymbolAddress (with that device current) and kept.
static __device__ __align__(256) uint16_t scratch[AREPI_LAMPORT_NOALLOC_BYTES / 2];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint16_t *g_scratch[kMaxDevices];  // per device: resolved (and armed) address
}  // namespace

// Address of the current device's staging.  The first call on a device arms
// the whole array with the sentinel (a fill kernel on `s`); from then on the
// consumer keeps what it reads armed.
static int noalloc_staging(const char *who, hipStream_t s, uint16_t **ptr) {
    int dev = -1;
    const hipError_t de = hipGetDevice(&dev);
    if (de != hipSuccess) return fail(AREPI_ELAUNCH, std::string(who) + ": hipGetDevice: " + hipGetErrorString(de));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(AREPI_EUNSUPPORTED, std::string(who) + ": device " + std::to_string(dev) + " beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(AREPI_ELAUNCH, std::string(who) + ": hipGetSymbolAddress(scratch): " + hipGetErrorString(e));
        constexpr int64_t n16 = AREPI_LAMPORT_NOALLOC_BYTES / 16;
        hipLaunchKernelGGL(prefill_kernel, dim3(2048), dim3(256), 0, s, static_cast<uint4 *>(p), n16,
                           static_cast<uint16_t *>(p), (int64_t)0);
        if (const int rc = check_launch(who)) return rc;
        g_scratch[dev] = static_cast<uint16_t *>(p);
    }
    *ptr = g_scratch[dev];
    return AREPI_OK;
}

extern "C" int arepi_ar_rmsnorm_lamport_noalloc(const uint16_t *gamma, uint16_t *out, int64_t M, int64_t N, int S,
                                                float eps, int scope, uint32_t *status, int64_t spin_limit,
                                                uint16_t **staging, arepi_stream_t stream) {
    const char *who = "arepi_ar_rmsnorm_lamport_noalloc";
    if (const int rc = check_consumer(who, M, N, S, eps, scope)) return rc;
    const int64_t cap = AREPI_LAMPORT_NOALLOC_BYTES;
    if (M > cap / ((int64_t)S * N * 2))
        return fail(AREPI_EUNSUPPORTED, std::string(who) + ": S*M*N*2 = " + std::to_string((int64_t)S * N * 2) +
                                            "*" + std::to_string(M) + " bytes exceeds the " + std::to_string(cap) +
                                            "-byte static staging");
    if (M > 0 && (!gamma || !out)) return fail(AREPI_EINVAL, std::string(who) + ": gamma and out must be non-NULL");
    if (M > 0 && (!aligned16(gamma) || !aligned16(out)))
        return fail(AREPI_EINVAL, std::string(who) + ": gamma and out must be 16-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint16_t *st = nullptr;
    if (const int rc = noalloc_staging(who, s, &st)) return rc;
    if (staging) *staging = st;
    if (M == 0) return ok();
    return launch_consumer(who, st, gamma, out, M, N, S, eps, scope, status, spin_limit, s);
}

// Shared validation of the two-phase entry points.
static int lamport2_params(const char *who, const uint16_t *const *inputs, uint16_t *const *staging, int64_t M,
                           int64_t N, int R, int rank, int scope, Lamport2Params &p) {
    auto bad = [who](const std::string &m) { return fail(AREPI_EINVAL, std::string(who) + ": " + m); };
    if (R < 1 || R > kMaxRanks) return bad("R=" + std::to_string(R) + " outside [1, 8]");
    if (rank < 0 || rank >= R) return bad("rank=" + std::to_string(rank) + " outside [0, R-1]");
    if (M < 0) return bad("M=" + std::to_string(M) + " must be >= 0");
    if (N < 8 || N % 8) return bad("N=" + std::to_string(N) + " must be a positive multiple of 8");
    if (N > 16384) return fail(AREPI_EUNSUPPORTED, std::string(who) + ": N=" + std::to_string(N) + " above 16384");
    if (scope != AREPI_SCOPE_AGENT && scope != AREPI_SCOPE_SYSTEM) return bad("scope must be AGENT or SYSTEM");
    if (M * N * 2 >= (int64_t)1 << 31)
        return fail(AREPI_EUNSUPPORTED, std::string(who) + ": one [M,N] buffer must be below 2 GiB");
    if (!inputs || !staging) return bad("inputs and staging must be host arrays of R device pointers");
    for (int r = 0; r < R; ++r) {
        if (!inputs[r] || !staging[r])
            return bad("inputs[" + std::to_string(r) + "] and staging[" + std::to_string(r) + "] must be non-NULL");
        if (!aligned16(inputs[r]) || !aligned16(staging[r])) return bad("buffers must be 16-byte aligned");
        p.in[r] = inputs[r];
        p.stg[r] = staging[r];
    }
    p.M = M;
    p.N = N;
    p.R = R;
    p.rank = rank;
    p.system = scope == AREPI_SCOPE_SYSTEM ? 1 : 0;
    return AREPI_OK;
}

extern "C" int arepi_ar_rmsnorm_lamport_2phase(const uint16_t *const *inputs, uint16_t *const *staging,
                                               const uint16_t *gamma, uint16_t *out, int64_t M, int64_t N, int R,
                                               int rank, float eps, int scope, uint32_t *status,
                                               int64_t spin_limit, arepi_stream_t stream) {
    const char *who = "arepi_ar_rmsnorm_lamport_2phase";
    Lamport2Params p{};
    int rc = lamport2_params(who, inputs, staging, M, N, R, rank, scope, p);
    if (rc) return rc;
    if (!(eps >= 0.0f)) return fail(AREPI_EINVAL, std::string(who) + ": eps must be >= 0");
    if (M == 0) return ok();
    if (!gamma || !out || !aligned16(gamma) || !aligned16(out))
        return fail(AREPI_EINVAL, std::string(who) + ": gamma and out must be non-NULL and 16-byte aligned");
    p.gamma = gamma;
    p.out = out;
    p.status = status;
    p.eps = eps;
    p.spin_limit = spin_bound(spin_limit);
    p.phase_b = 1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int64_t packs = N / 8;
    if (packs <= 256) return launch_lamport2<1, 256>(p, s);
    if (packs <= 512) return launch_lamport2<2, 256>(p, s);
    if (packs <= 1024) return launch_lamport2<4, 256>(p, s);
    return launch_lamport2<8, 256>(p, s);
}

extern "C" int arepi_emu_lamport_phase_a(const uint16_t *const *inputs, uint16_t *const *staging, int64_t M,
                                         int64_t N, int R, int rank, int scope, arepi_stream_t stream) {
    Lamport2Params p{};
    int rc = lamport2_params("arepi_emu_lamport_phase_a", inputs, staging, M, N, R, rank, scope, p);
    if (rc) return rc;
    if (M == 0) return ok();
    p.phase_b = 0;
    return launch_lamport2<1, 256>(p, reinterpret_cast<hipStream_t>(stream));
}
