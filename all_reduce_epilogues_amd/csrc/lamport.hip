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
// gfx950 mapping: the publisher's stores and the consumer's polls and re-arm
// stores are device-coherent 8-byte atomics (relaxed, agent or system scope),
// which the compiler lowers to sc1 global loads/stores: they are not served
// from an XCD's non-coherent L2 copy, so a pack written from another XCD is
// seen, and a re-arm can never be written back over a later publication.
//
// Consumer layout: one 256-thread workgroup per row; thread t owns packs
// t, t+256, ... of the row (coalesced 16-byte columns), keeps the fp32 slot sums
// of its packs in registers, reduces sum(s^2) across the workgroup (wave
// shuffles, then LDS), and writes the normalised row.
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

template <int PPT>
__global__ void __launch_bounds__(256) ar_rmsnorm_kernel(uint16_t *__restrict__ staging,
                                                        const uint16_t *__restrict__ gamma,
                                                        uint16_t *__restrict__ out, int64_t M,
                                                        int64_t N, int S, float eps, int system,
                                                        uint32_t *status, int64_t spin_limit) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t packs = N / 8;
    const int64_t plane = M * N;
    const bool sys = system != 0;
    float s[PPT][8];
    float ss = 0.f;
    int64_t spins = 0;
    bool gave_up = false;

#pragma unroll
    for (int j = 0; j < PPT; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[j][e] = 0.f;
        const int64_t pk = tid + (int64_t)j * 256;
        if (pk < packs) {
            uint64_t *base = reinterpret_cast<uint64_t *>(staging + row * N + pk * 8);
            uint64_t lo[8], hi[8];
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                if (sl < S) {
                    lo[sl] = load64_coherent(base + sl * (plane / 4), sys);
                    hi[sl] = load64_coherent(base + sl * (plane / 4) + 1, sys);
                }
            }
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                if (sl < S) {
                    // spin until the pack has landed (bounded)
                    while (!gave_up && (has_sentinel(lo[sl]) || has_sentinel(hi[sl]))) {
                        if (++spins > spin_limit) {
                            gave_up = true;
                            if (status) atomicOr(status, (uint32_t)AREPI_STATUS_TIMEOUT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                        lo[sl] = load64_coherent(base + sl * (plane / 4), sys);
                        hi[sl] = load64_coherent(base + sl * (plane / 4) + 1, sys);
                    }
                    const uint4 q = make_uint4((uint32_t)lo[sl], (uint32_t)(lo[sl] >> 32), (uint32_t)hi[sl],
                                               (uint32_t)(hi[sl] >> 32));
                    float f[8];
                    unpack8(q, f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) s[j][e] = s[j][e] + f[e];
                    // re-arm the consumed pack
                    store64_coherent(base + sl * (plane / 4), kSent4, sys);
                    store64_coherent(base + sl * (plane / 4) + 1, kSent4, sys);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = ss + s[j][e] * s[j][e];
        }
    }
    // workgroup sum of s^2
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float r = 1.0f / sqrtf(tot / (float)N + eps);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int64_t pk = tid + (int64_t)j * 256;
        if (pk < packs) {
            const uint4 g = *reinterpret_cast<const uint4 *>(gamma + pk * 8);
            float gf[8], y[8];
            unpack8(g, gf);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (s[j][e] * r) * gf[e];
            *reinterpret_cast<uint4 *>(out + row * N + pk * 8) = pack8(y);
        }
    }
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

extern "C" int arepi_ar_rmsnorm_lamport(uint16_t *staging, const uint16_t *gamma, uint16_t *out, int64_t M,
                                        int64_t N, int S, float eps, int scope, uint32_t *status,
                                        int64_t spin_limit, arepi_stream_t stream) {
    auto bad = [](const std::string &m) { return fail(AREPI_EINVAL, "arepi_ar_rmsnorm_lamport: " + m); };
    if (S < 1 || S > 8) return bad("S=" + std::to_string(S) + " outside [1, 8]");
    if (M < 0) return bad("M=" + std::to_string(M) + " must be >= 0");
    if (N < 8 || N % 8) return bad("N=" + std::to_string(N) + " must be a positive multiple of 8");
    if (N > 16384) return fail(AREPI_EUNSUPPORTED, "arepi_ar_rmsnorm_lamport: N=" + std::to_string(N) + " above 16384");
    if (!(eps >= 0.0f)) return bad("eps must be >= 0");
    if (scope != AREPI_SCOPE_AGENT && scope != AREPI_SCOPE_SYSTEM) return bad("scope must be AGENT or SYSTEM");
    if (M == 0) return ok();
    if (!staging || !gamma || !out) return bad("staging, gamma and out must be non-NULL");
    if (!aligned16(staging) || !aligned16(gamma) || !aligned16(out))
        return bad("staging, gamma and out must be 16-byte aligned");
    if (M > (int64_t)1 << 31) return fail(AREPI_EUNSUPPORTED, "arepi_ar_rmsnorm_lamport: M above 2^31");
    const int64_t packs = N / 8;
    const int ppt = (int)((packs + 255) / 256);
    const int64_t lim = spin_limit > 0 ? spin_limit : kDefaultSpinLimit;
    const int sys = scope == AREPI_SCOPE_SYSTEM ? 1 : 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (ppt <= 1)
        hipLaunchKernelGGL(ar_rmsnorm_kernel<1>, dim3((unsigned)M), dim3(256), 0, s, staging, gamma, out, M, N, S,
                           eps, sys, status, lim);
    else if (ppt <= 2)
        hipLaunchKernelGGL(ar_rmsnorm_kernel<2>, dim3((unsigned)M), dim3(256), 0, s, staging, gamma, out, M, N, S,
                           eps, sys, status, lim);
    else if (ppt <= 4)
        hipLaunchKernelGGL(ar_rmsnorm_kernel<4>, dim3((unsigned)M), dim3(256), 0, s, staging, gamma, out, M, N, S,
                           eps, sys, status, lim);
    else
        hipLaunchKernelGGL(ar_rmsnorm_kernel<8>, dim3((unsigned)M), dim3(256), 0, s, staging, gamma, out, M, N, S,
                           eps, sys, status, lim);
    return check_launch("arepi_ar_rmsnorm_lamport");
}
