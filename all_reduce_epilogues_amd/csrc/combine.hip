// combine.hip -- weighted top-k combine through a multi-stage LDS pipeline
// (gfx950).
//
//   out[t,h] = bf16( sum_{k<E} gate[t,k] * x[t,k,h] ),  fp32 accumulate.
//
// The pipeline idea follows DeepEP PR #527 ("Fix the MultiStages for intranode
// combine"): a multi-stage buffer only overlaps if every stage is issued and
// waited on independently, instead of one issuer serialising all stages.  On
// gfx950 that maps to direct-to-LDS loads (global_load_lds_dwordx4), which
// put data in LDS without holding registers: each wave owns S stages of
// E x 1 KiB, issues stage i+S-1 before it consumes stage i, and waits with
// an exact vmcnt that leaves the younger stages in flight.  A lane only ever
// reads back the 16 bytes it loaded itself, so no barrier is needed; the
// read-back uses explicit ds_read_b128 with its own lgkmcnt wait so the
// compiler's conservative LDS-DMA wait does not collapse the pipeline.
//
// This LDS-staged pipeline is the arepi_combine_reduce_lds entry point; the
// default arepi_combine_reduce uses the register-pipelined kernel further down.
//
// Work unit ("chunk"): one token t and 512 consecutive h (64 lanes x 8).  The
// grid is a fixed set of single-wave workgroups (5 per CU: 32 KiB of LDS each
// at E=8, S=4) looping over chunks with a grid stride.  Expert rows are read
// once, so the loads and the output stores are nontemporal (streaming).
#include <string>

#include "arepi_internal.h"

namespace arepi {
namespace {

constexpr int kStages = 4;
constexpr int kChunkH = 512;  // h values per chunk (64 lanes x 8)

__device__ __forceinline__ u32x4 ds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left free (gfx9 encoding: vmcnt low
// bits [3:0], high bits [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int E>
__device__ __forceinline__ void wait_stages_after(int n_after) {
    // n_after younger stages (E loads each) may stay in flight
    switch (n_after) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<E>(); break;
        case 2: wait_vmcnt<2 * E>(); break;
        default: wait_vmcnt<3 * E>(); break;
    }
}

template <int E>
__global__ void __launch_bounds__(64) combine_kernel(const uint16_t *__restrict__ x,
                                                    const float *__restrict__ gate,
                                                    uint16_t *__restrict__ out, int64_t T, int64_t H,
                                                    int64_t chunks_per_token) {
    static_assert(E >= 1 && 3 * E < 64, "E out of range for the vmcnt budget");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x;
    const int64_t n_chunks = T * chunks_per_token;
    const int64_t stride = gridDim.x;
    const int64_t first = blockIdx.x;
    const int64_t n_mine = first < n_chunks ? (n_chunks - 1 - first) / stride + 1 : 0;

    auto lds_stage = [&](int s) {
        return (__attribute__((address_space(3))) uint8_t *)(lds) + s * (E * 1024);
    };
    auto issue = [&](int64_t i) {
        const int64_t c = first + i * stride;
        const int64_t t = c / chunks_per_token;
        const int64_t h = (c % chunks_per_token) * kChunkH + lane * 8;
        const int s = (int)(i % kStages);
        // lanes past H re-load their token's first pack (never stored), so every
        // stage issues exactly E load instructions for the vmcnt arithmetic
        const uint16_t *src = x + (t * E) * H + (h < H ? h : 0);
#pragma unroll
        for (int k = 0; k < E; ++k)
            __builtin_amdgcn_global_load_lds(src + (int64_t)k * H,
                                             (__attribute__((address_space(3))) void *)(lds_stage(s) + k * 1024),
                                             16, 0, kAuxNontemporal);
    };

    for (int64_t i = 0; i < kStages - 1 && i < n_mine; ++i) issue(i);
    for (int64_t i = 0; i < n_mine; ++i) {
        if (i + kStages - 1 < n_mine) issue(i + kStages - 1);
        const int64_t left = n_mine - 1 - i;
        wait_stages_after<E>((int)(left < kStages - 1 ? left : kStages - 1));

        const int64_t c = first + i * stride;
        const int64_t t = c / chunks_per_token;
        const int64_t h = (c % chunks_per_token) * kChunkH + lane * 8;
        const uint32_t base = (uint32_t)(uintptr_t)lds_stage((int)(i % kStages)) + lane * 16;
        u32x4 q[E];
#pragma unroll
        for (int k = 0; k < E; ++k) q[k] = ds_read16(base + k * 1024);
        float g[E];
#pragma unroll
        for (int k = 0; k < E; ++k) g[k] = gate[t * E + k];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < E; ++k) {
            float f[8];
            unpack8(make_uint4(q[k].x, q[k].y, q[k].z, q[k].w), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = acc[e] + g[k] * f[e];
        }
        if (h < H) store16_nt(out + t * H + h, pack8(acc));
    }
}

// Register-pipelined variant (the default entry point): one thread = one
// 16-byte column pack of one token; each thread keeps the E expert loads of
// two work units in flight (two stages in registers) with nontemporal loads,
// and the output store is nontemporal too.  On MI355X this streams at ~6 TB/s,
// above the LDS-staged pipeline above, because no LDS round trip and no
// per-wave stage bookkeeping sit between the loads and the FMAs.
template <int E, int UNITS>
__global__ void __launch_bounds__(256) combine_regs_kernel(const uint16_t *__restrict__ x,
                                                           const float *__restrict__ gate,
                                                           uint16_t *__restrict__ out, int64_t T, int64_t H) {
    const int64_t packs = H / 8, units = T * packs;
    const int64_t stride = (int64_t)gridDim.x * 256 * UNITS;
    for (int64_t u0 = (int64_t)blockIdx.x * 256 * UNITS + threadIdx.x; u0 < units; u0 += stride) {
        uint4 q[UNITS][E];
        int64_t tt[UNITS], hh[UNITS];
#pragma unroll
        for (int r = 0; r < UNITS; ++r) {
            const int64_t u = min(u0 + (int64_t)r * 256, units - 1);  // clamped: never stored
            tt[r] = u / packs;
            hh[r] = (u % packs) * 8;
#pragma unroll
            for (int k = 0; k < E; ++k) q[r][k] = load16_nt(x + (tt[r] * E + k) * H + hh[r]);
        }
#pragma unroll
        for (int r = 0; r < UNITS; ++r) {
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const float g = gate[tt[r] * E + k];
                float f[8];
                unpack8(q[r][k], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = acc[e] + g * f[e];
            }
            if (u0 + (int64_t)r * 256 < units) store16_nt(out + tt[r] * H + hh[r], pack8(acc));
        }
    }
}

template <int E>
int launch_regs(const uint16_t *x, const float *gate, uint16_t *out, int64_t T, int64_t H, hipStream_t s) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    constexpr int UNITS = E <= 8 ? 2 : 1;
    const int64_t units = T * (H / 8);
    int64_t grid = (units + 256 * UNITS - 1) / (256 * UNITS);
    if (grid > (int64_t)cus * 16) grid = (int64_t)cus * 16;
    hipLaunchKernelGGL((combine_regs_kernel<E, UNITS>), dim3((unsigned)grid), dim3(256), 0, s, x, gate, out, T, H);
    return check_launch("arepi_combine_reduce");
}

template <int E>
int launch(const uint16_t *x, const float *gate, uint16_t *out, int64_t T, int64_t H, hipStream_t s) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
    const int64_t cpt = (H + kChunkH - 1) / kChunkH;
    const int64_t n_chunks = T * cpt;
    const size_t lds = (size_t)kStages * E * 1024;
    const int per_cu = (int)((160 * 1024) / lds) > 0 ? (int)((160 * 1024) / lds) : 1;
    int64_t grid = (int64_t)cus * (per_cu < 8 ? per_cu : 8);
    if (grid > n_chunks) grid = n_chunks;
    hipLaunchKernelGGL((combine_kernel<E>), dim3((unsigned)grid), dim3(64), lds, s, x, gate, out, T, H, cpt);
    return check_launch("arepi_combine_reduce_lds");
}

}  // namespace
}  // namespace arepi

using namespace arepi;

static int combine_validate(const char *who, const uint16_t *x, const float *gate, uint16_t *out, int64_t T,
                            int E, int64_t H) {
    auto bad = [who](const std::string &m) { return fail(AREPI_EINVAL, std::string(who) + ": " + m); };
    if (T < 0) return bad("T=" + std::to_string(T) + " must be >= 0");
    if (E < 1 || E > 16)
        return fail(AREPI_EUNSUPPORTED, std::string(who) + ": E=" + std::to_string(E) + " outside [1, 16]");
    if (H < 8 || H % 8) return bad("H=" + std::to_string(H) + " must be a positive multiple of 8");
    if (T == 0) return 1;  // nothing to do
    if (!x || !gate || !out) return bad("x, gate and out must be non-NULL");
    if (!aligned16(x) || !aligned16(out)) return bad("x and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(gate) & 3u) != 0) return bad("gate must be 4-byte aligned");
    return AREPI_OK;
}

#define AREPI_E_CASES(F)                                                                                  \
    F(1) F(2) F(3) F(4) F(5) F(6) F(7) F(8) F(9) F(10) F(11) F(12) F(13) F(14) F(15) F(16)

extern "C" int arepi_combine_reduce(const uint16_t *x, const float *gate, uint16_t *out, int64_t T, int E,
                                    int64_t H, arepi_stream_t stream) {
    const int rc = combine_validate("arepi_combine_reduce", x, gate, out, T, E, H);
    if (rc < 0) return rc;
    if (rc == 1) return ok();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (E) {
#define AREPI_CASE(e) \
    case e: return launch_regs<e>(x, gate, out, T, H, s);
        AREPI_E_CASES(AREPI_CASE)
#undef AREPI_CASE
    }
    return fail(AREPI_EUNSUPPORTED, "arepi_combine_reduce: unreachable E");
}

extern "C" int arepi_combine_reduce_lds(const uint16_t *x, const float *gate, uint16_t *out, int64_t T, int E,
                                        int64_t H, arepi_stream_t stream) {
    const int rc = combine_validate("arepi_combine_reduce_lds", x, gate, out, T, E, H);
    if (rc < 0) return rc;
    if (rc == 1) return ok();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (E) {
#define AREPI_CASE(e) \
    case e: return launch<e>(x, gate, out, T, H, s);
        AREPI_E_CASES(AREPI_CASE)
#undef AREPI_CASE
    }
    return fail(AREPI_EUNSUPPORTED, "arepi_combine_reduce_lds: unreachable E");
}
