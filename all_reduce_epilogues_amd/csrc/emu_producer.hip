// emu_producer.hip -- stands in for the R-1 peer ranks on one GPU (tests and
// benchmark only).  A workgroup lands a batch of (peer, flag tile) items: it
// copies those tiles of the peers' partials into recv[peer], drains its
// stores, meets the workgroup barrier, and one thread publishes the batch's
// bits after one release -- the per-tile readiness of DeepGEMM PR #1 "Fused
// ring RS: per-tile bitmask", in the place of a per-segment flag.  A release
// at agent scope writes back the L2 of the XCD it runs on, which a remote
// peer's release would not do to this GPU; batching several tiles per release
// keeps that cost of the emulation down.
#include <algorithm>
#include <string>
#include <vector>

#include "arepi_internal.h"

namespace arepi {
namespace {

constexpr int kMaxR = 8;

struct EmuParams {
    const uint16_t *src[kMaxR];
    uint16_t *recv[kMaxR];
    uint32_t *ready_in;
    const int32_t *order;  // [n_orders][n_items][2] = (peer, tile)
    int64_t n_items, seg, N, ftiles_n, ftiles, fwords;
    int ftm, ftn, R, owner, system_scope;
    int per_release;  // items landed per release
    uint32_t *resident;  // NULL, or [2]: workgroups started, grid size
    // several steps in one launch: step s uses order s % n_orders.  Signal
    // mode: step s starts once *go >= s (go NULL: no wait).  Credit mode: go
    // counts the producer's own (workgroup, step) completions; step s starts
    // once every workgroup has finished step s-1 (*go >= s * grid), then each
    // batch waits until its items' bits are clear (the consumer clears a bit
    // once it has read that tile).  Both are needed: with the order changing
    // between steps, a bit that is clear because another workgroup has not
    // yet landed that tile for step s-1 is not a credit.
    uint32_t *go;
    int steps, n_orders;
    int credit;
    // step s copies from src[peer] + (s % n_orders) * src_step elements
    int64_t src_step;
    uint32_t *status;
    int64_t spin_limit;
};

__device__ bool item_valid(const EmuParams &p, const int32_t *order, const int64_t item, int &peer, int64_t &t) {
    peer = order[2 * item];
    t = order[2 * item + 1];
    return peer >= 0 && peer < p.R && peer != p.owner && t >= 0 && t < p.ftiles;
}

// Copies one (peer, flag tile) item with the whole workgroup (no drain).
__device__ void copy_item(const EmuParams &p, const int32_t *order, const int64_t item, const int64_t src_off) {
    int peer;
    int64_t t;
    if (!item_valid(p, order, item, peer, t)) return;  // uniform across the workgroup
    const int64_t r0 = (t / p.ftiles_n) * p.ftm, c0 = (t % p.ftiles_n) * p.ftn;
    const int64_t rows = min((int64_t)p.ftm, p.seg - r0);
    const int64_t packs = min((int64_t)p.ftn, p.N - c0) / 8;
    const uint16_t *s = nullptr;
    uint16_t *d = nullptr;
#pragma unroll
    for (int i = 0; i < kMaxR; ++i)
        if (i == peer) {
            s = p.src[i] + src_off;
            d = p.recv[i];
        }
    // 16-byte packs, eight per thread in flight (streaming loads and stores).
    // Whole rounds of 256 x 8 packs run without per-pack predicates: a store
    // under a branch would make the compiler wait for every load in flight.
    const int ppr = (int)packs, total = (int)rows * ppr;
    auto at = [&](int i) { return (r0 + i / ppr) * p.N + c0 + (i % ppr) * 8; };
    int base = 0;
    for (; base + 256 * 8 <= total; base += 256 * 8) {
        uint4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = load16_nt(s + at(base + (int)threadIdx.x + k * 256));
#pragma unroll
        for (int k = 0; k < 8; ++k) store16_nt(d + at(base + (int)threadIdx.x + k * 256), v[k]);
    }
    if (base < total) {
        uint4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = base + (int)threadIdx.x + k * 256;
            if (i < total) v[k] = load16_nt(s + at(i));
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = base + (int)threadIdx.x + k * 256;
            if (i < total) store16_nt(d + at(i), v[k]);
        }
    }
}

// Batch j is items [j*K, j*K + K) in order (K = per_release).  Workgroup g
// lands batches g, g + G, g + 2G, ... (G = grid size), so a grid smaller than
// the batch count paces the landing like a link of bounded rate.  Each batch:
// copies, drain, barrier, one release, then its bits.
// Its waves share the GPU with the GEMM it feeds, whose owner tiles spin on
// these bits.  A workgroup waits only between steps (for a signal, or for
// the other workgroups and then for credits), and what it waits for comes
// from a consumer of an earlier step, which needs nothing from it, so once it
// is resident it finishes.
// With `resident` given, every workgroup announces itself on arrival, so that
// emu_gate_kernel can hold the consumer back until the whole grid has started.
__global__ void __launch_bounds__(256) emu_producer_kernel(const EmuParams p) {
    if (p.resident && threadIdx.x == 0) {
        __hip_atomic_store(p.resident + 1, gridDim.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(p.resident, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __shared__ int stop;
    const int64_t K = p.per_release, batches = (p.n_items + K - 1) / K;
    const bool sys = p.system_scope != 0;
    for (int st = 0; st < p.steps; ++st) {
        if (p.go) {
            // signal mode: wait for the consumer of step st-1 to be done with
            // recv and ready_in; credit mode: wait for every producer
            // workgroup to have landed step st-1
            const uint32_t need = p.credit ? (uint32_t)st * gridDim.x : (uint32_t)st;
            if (threadIdx.x == 0) {
                int64_t n = 0;
                const uint64_t t0 = spin_clock();
                stop = 0;
                while (load_relaxed(p.go, false) < need) {
                    if (spin_expired(p.spin_limit, n, t0)) {
                        stop = 1;
                        if (p.status) atomicOr(p.status, (uint32_t)AREPI_STATUS_TIMEOUT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __syncthreads();
            if (stop) return;
        }
        const int32_t *order = p.order + (int64_t)(st % p.n_orders) * p.n_items * 2;
        const int64_t src_off = (int64_t)(st % p.n_orders) * p.src_step;
        for (int64_t j = blockIdx.x; j < batches; j += gridDim.x) {
            const int64_t i0 = j * K, i1 = min(i0 + K, p.n_items);
            if (p.credit) {
                // wait until the consumer has read what the batch's slots hold
                // (a bit still set belongs to the previous step); the copies
                // below are issued only once the loop has seen every bit clear
                if (threadIdx.x < 64) {
                    int64_t n = 0;
                    const uint64_t t0 = spin_clock();
                    bool expired = false;
                    for (int64_t item = i0 + threadIdx.x; item < i1 && !expired; item += 64) {
                        int peer;
                        int64_t t;
                        if (!item_valid(p, order, item, peer, t)) continue;
                        const uint32_t *w = p.ready_in + (int64_t)peer * p.fwords + (t >> 5);
                        while (load_relaxed(w, sys) & (1u << (t & 31))) {
                            if (spin_expired(p.spin_limit, n, t0)) {
                                expired = true;
                                break;
                            }
                            __builtin_amdgcn_s_sleep(2);
                        }
                    }
                    const bool any = __builtin_amdgcn_ballot_w64(expired) != 0;
                    if (threadIdx.x == 0) {
                        stop = any ? 1 : 0;
                        if (any && p.status) atomicOr(p.status, (uint32_t)AREPI_STATUS_TIMEOUT);
                    }
                }
                __syncthreads();
                if (stop) return;
            }
            for (int64_t item = i0; item < i1; ++item) copy_item(p, order, item, src_off);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (threadIdx.x == 0) {
                fence_release(sys);
                for (int64_t item = i0; item < i1; ++item) {
                    int peer;
                    int64_t t;
                    if (item_valid(p, order, item, peer, t))
                        fetch_or_relaxed(p.ready_in + (int64_t)peer * p.fwords + (t >> 5), 1u << (t & 31), sys);
                }
            }
        }
        if (p.credit && threadIdx.x == 0) {
            // this workgroup's bits of step st are set (the atomics have
            // completed) before it counts the step as landed
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __hip_atomic_fetch_add(p.go, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// One thread: *flag = value after everything before it on the stream.
__global__ void emu_signal_kernel(uint32_t *flag, uint32_t value) {
    __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave, launched on the consumer's stream between the producer and the
// consumer: waits until every producer workgroup has started (resident[0]
// reaches the grid size in resident[1]), then returns the pair to zero.  The
// consumer is queued behind it, so it cannot take the compute units before
// the producer holds its own; the producer never waits, so it then finishes
// whatever the consumer's workgroups occupy.
__global__ void __launch_bounds__(64) emu_gate_kernel(uint32_t *resident, uint32_t *status, int64_t spin_limit) {
    if (threadIdx.x != 0) return;
    int64_t n = 0;
    const uint64_t t0 = spin_clock();
    for (;;) {
        const uint32_t g = load_relaxed(resident + 1, false);
        const uint32_t c = load_relaxed(resident, false);
        if (g != 0 && c >= g) {
            __hip_atomic_fetch_sub(resident, g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(resident + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        if (spin_expired(spin_limit, n, t0)) {
            if (status) atomicOr(status, (uint32_t)AREPI_STATUS_TIMEOUT);
            return;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

}  // namespace
}  // namespace arepi

using namespace arepi;

static int emu_launch(const char *who, const uint16_t *const *src, uint16_t *const *recv, uint32_t *ready_in,
                      const int32_t *order, int64_t n_items, int64_t M, int64_t N, int R, int owner,
                      int flag_tile_m, int flag_tile_n, int scope, int workgroups, int items_per_release,
                      uint32_t *resident, uint32_t *go, int steps, int n_orders, bool credit,
                      int64_t src_step, uint32_t *status, int64_t spin_limit, arepi_stream_t stream) {
    auto bad = [who](const std::string &m) { return fail(AREPI_EINVAL, std::string(who) + ": " + m); };
    if (R < 1 || R > kMaxR) return bad("R=" + std::to_string(R) + " outside [1, 8]");
    if (owner < 0 || owner >= R) return bad("owner outside [0, R-1]");
    if (M < 1 || M % R) return bad("M must be a positive multiple of R");
    if (N < 8 || N % 8) return bad("N must be a positive multiple of 8");
    if (flag_tile_m < 1 || flag_tile_n < 8 || flag_tile_n % 8)
        return bad("flag tile needs flag_tile_m >= 1 and flag_tile_n a positive multiple of 8");
    if (scope != AREPI_SCOPE_AGENT && scope != AREPI_SCOPE_SYSTEM) return bad("scope must be AGENT or SYSTEM");
    if (n_items < 0 || n_items > (int64_t)1 << 30) return bad("n_items out of range");
    if (workgroups < 0) return bad("workgroups must be >= 0 (0: one per batch)");
    if (items_per_release < 1) return bad("items_per_release must be >= 1");
    if (steps < 1 || n_orders < 1) return bad("steps and n_orders must be >= 1");
    if (src_step < 0 || src_step % 8) return bad("src_step must be a non-negative multiple of 8");
    if (n_items == 0) return ok();
    if (!src || !recv || !ready_in || !order) return bad("src, recv, ready_in and order must be non-NULL");
    EmuParams p{};
    for (int i = 0; i < R; ++i) {
        if (i == owner) continue;
        if (!src[i] || !recv[i]) return bad("src/recv entry " + std::to_string(i) + " is NULL");
        if (!aligned16(src[i]) || !aligned16(recv[i])) return bad("src/recv must be 16-byte aligned");
        p.src[i] = src[i];
        p.recv[i] = recv[i];
    }
    p.ready_in = ready_in;
    p.order = order;
    p.n_items = n_items;
    p.seg = M / R;
    p.N = N;
    p.ftiles_n = (N + flag_tile_n - 1) / flag_tile_n;
    p.ftiles = ((p.seg + flag_tile_m - 1) / flag_tile_m) * p.ftiles_n;
    p.fwords = (p.ftiles + 31) / 32;
    p.ftm = flag_tile_m;
    p.ftn = flag_tile_n;
    p.R = R;
    p.owner = owner;
    p.system_scope = scope == AREPI_SCOPE_SYSTEM ? 1 : 0;
    p.per_release = items_per_release;
    p.resident = resident;
    p.go = go;
    p.steps = steps;
    p.n_orders = n_orders;
    p.credit = credit ? 1 : 0;
    p.src_step = src_step;
    p.status = status;
    p.spin_limit = spin_bound(spin_limit);
    const int64_t batches = (n_items + items_per_release - 1) / items_per_release;
    const int64_t groups = workgroups == 0 ? batches : std::min<int64_t>(workgroups, batches);
    if (credit && (int64_t)steps * groups >= ((int64_t)1 << 32))
        return bad("steps x workgroups must stay below 2^32 (the 32-bit landed-step count)");
    hipLaunchKernelGGL(emu_producer_kernel, dim3((unsigned)groups), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), p);
    return check_launch(who);
}

extern "C" int arepi_emu_peer_producer(const uint16_t *const *src, uint16_t *const *recv, uint32_t *ready_in,
                                       const int32_t *order, int64_t n_items, int64_t M, int64_t N, int R,
                                       int owner, int flag_tile_m, int flag_tile_n, int scope,
                                       int workgroups, int items_per_release, uint32_t *resident,
                                       arepi_stream_t stream) {
    return emu_launch("arepi_emu_peer_producer", src, recv, ready_in, order, n_items, M, N, R, owner,
                      flag_tile_m, flag_tile_n, scope, workgroups, items_per_release, resident, nullptr, 1, 1,
                      false, 0, nullptr, 0, stream);
}

extern "C" int arepi_emu_peer_producer_steps(const uint16_t *const *src, uint16_t *const *recv,
                                             uint32_t *ready_in, const int32_t *orders, int n_orders,
                                             int64_t n_items, int64_t M, int64_t N, int R, int owner,
                                             int flag_tile_m, int flag_tile_n, int scope, int workgroups,
                                             int items_per_release, uint32_t *resident, uint32_t *go, int credit,
                                             int steps, int64_t src_step, uint32_t *status, int64_t spin_limit,
                                             arepi_stream_t stream) {
    if (!go) return fail(AREPI_EINVAL, "arepi_emu_peer_producer_steps: go must be non-NULL");
    if (credit != 0 && credit != 1) return fail(AREPI_EINVAL, "arepi_emu_peer_producer_steps: credit must be 0 or 1");
    return emu_launch("arepi_emu_peer_producer_steps", src, recv, ready_in, orders, n_items, M, N, R, owner,
                      flag_tile_m, flag_tile_n, scope, workgroups, items_per_release, resident, go, steps,
                      n_orders, credit != 0, src_step, status, spin_limit, stream);
}

extern "C" int arepi_emu_signal(uint32_t *flag, uint32_t value, arepi_stream_t stream) {
    if (!flag) return fail(AREPI_EINVAL, "arepi_emu_signal: flag must be non-NULL");
    if (reinterpret_cast<uintptr_t>(flag) & 3u) return fail(AREPI_EINVAL, "arepi_emu_signal: flag must be 4-byte aligned");
    hipLaunchKernelGGL(emu_signal_kernel, dim3(1), dim3(1), 0, reinterpret_cast<hipStream_t>(stream), flag, value);
    return check_launch("arepi_emu_signal");
}

extern "C" int arepi_emu_producer_gate(uint32_t *resident, uint32_t *status, int64_t spin_limit,
                                       arepi_stream_t stream) {
    if (!resident) return fail(AREPI_EINVAL, "arepi_emu_producer_gate: resident must be non-NULL");
    if (reinterpret_cast<uintptr_t>(resident) & 7u)
        return fail(AREPI_EINVAL, "arepi_emu_producer_gate: resident must be 8-byte aligned");
    hipLaunchKernelGGL(emu_gate_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), resident,
                       status, spin_bound(spin_limit));
    return check_launch("arepi_emu_producer_gate");
}

extern "C" int arepi_emu_stream_create(arepi_stream_t *stream) {
    if (!stream) return fail(AREPI_EINVAL, "arepi_emu_stream_create: stream must be non-NULL");
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return fail(AREPI_ELAUNCH, "arepi_emu_stream_create: device query failed");
    // every compute unit enabled: the mask only buys the queue of its own
    std::vector<uint32_t> mask((cus + 31) / 32, 0u);
    for (int c = 0; c < cus; ++c) mask[c / 32] |= 1u << (c % 32);
    hipStream_t s = nullptr;
    const hipError_t e = hipExtStreamCreateWithCUMask(&s, (uint32_t)mask.size(), mask.data());
    if (e != hipSuccess)
        return fail(AREPI_ELAUNCH, std::string("arepi_emu_stream_create: ") + hipGetErrorString(e));
    *stream = reinterpret_cast<arepi_stream_t>(s);
    return ok();
}

extern "C" int arepi_emu_stream_destroy(arepi_stream_t stream) {
    if (!stream) return fail(AREPI_EINVAL, "arepi_emu_stream_destroy: stream must be non-NULL");
    const hipError_t e = hipStreamDestroy(reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(AREPI_ELAUNCH, std::string("arepi_emu_stream_destroy: ") + hipGetErrorString(e));
    return ok();
}
