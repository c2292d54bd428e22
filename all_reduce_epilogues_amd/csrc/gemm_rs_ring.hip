// gemm_rs_ring.hip -- row-parallel bf16 GEMM whose epilogue is one hop of a
// push ring reduce-scatter, for gfx950 (MI355X), and its C entry points.
//
// What it computes follows DeepGEMM PR #1 "Fused ring RS: per-tile bitmask +
// drain-ring with owner-boundary flush" (description): each rank takes the
// running partial of a segment from its upstream neighbour, adds its own
// partial tile in the GEMM epilogue and pushes the sum on; the owner of a
// segment is the last rank of that segment's chain and ends with the full
// sum.  Rank r receives from r-1 and sends to r+1 (mod R); the segment a rank
// starts, chain = (owner - 1) mod R, has no upstream partial.  Per row of
// segment d of the local product C = X.W (fp32, then one bf16 rounding):
//     d == owner: out  = bf16(C + up[owner])
//     d == chain: send = bf16(C)
//     otherwise:  send = bf16(C + up[d])
// Readiness is per flag tile, as in the direct form: bit t of ready_in[d] says
// flag tile t of up[d] has landed; ready_out[d] is set for every segment this
// rank pushes on (every d != owner).
//
// The mainloop, staging, stores and publication are the direct form's
// (gemm_rs_impl.h); what differs is the epilogue's source (one upstream
// partial per row, chosen by the row's segment, for every tile but those of
// the chain segment) and the tile order (segments in the order a ring hands
// them on: chain first, owner last).
#include "gemm_rs_impl.h"

namespace arepi {
namespace {

template <int BM, int BN, int WM, int WN, int BK, int S, int WPE>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1, WPE > 0 ? WPE : 8)))
    gemm_rs_ring_kernel(const GemmRsParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[lds_bytes<BM, BN, BK, S>()];
    constexpr int CK = BM >= 64 ? BM / 2 : BM;
    int rb, cb;
    tile_of_block(p, blockIdx.x, rb, cb);
    int64_t a0, b0;
    int alen, blen;
    chunks_of_block(p, BM, CK, rb, a0, alen, b0, blen);
    // a tile whose rows all lie in the chain segment has nothing to add
    const int64_t c0 = (int64_t)p.chain * p.seg, c1 = c0 + p.seg;
    const bool chain_a = alen <= 0 || (a0 >= c0 && a0 + alen <= c1);
    const bool chain_b = blen <= 0 || (b0 >= c0 && b0 + blen <= c1);
    if (chain_a && chain_b)
        gemm_rs_body<BM, BN, WM, WN, BK, S, WPE, 1, kNoOwnerRows>(p, smem, rb, cb, a0, alen, b0, blen);
    else
        gemm_rs_body<BM, BN, WM, WN, BK, S, WPE, 1, kRing>(p, smem, rb, cb, a0, alen, b0, blen);
}

template <int BM, int BN, int WM, int WN, int BK, int S, int WPE>
void launch_ring(const GemmRsParams &p, hipStream_t stream) {
    constexpr int NT = (BM / WM) * (BN / WN) * 64;
    hipLaunchKernelGGL((gemm_rs_ring_kernel<BM, BN, WM, WN, BK, S, WPE>), dim3(p.nWG), dim3(NT), 0, stream, p);
}

// Rows per epilogue unit never exceed this (64 lanes / 16-byte chunks per
// wave row); a segment height that is a multiple of it keeps every unit inside
// one segment.
constexpr int kRingRowAlign = 8;

}  // namespace
}  // namespace arepi

using namespace arepi;

extern "C" int arepi_gemm_rs_ring_supports(int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                                           int flag_tile_n, int publish, int tile_cfg) {
    if (tile_cfg & AREPI_TILE_PAIRED_ROWS)
        return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_ring: AREPI_TILE_PAIRED_ROWS applies to the direct form only");
    if (tile_cfg & (AREPI_TILE_OWNER_FIRST | AREPI_TILE_OWNER_HALF))
        return fail(AREPI_EINVAL, "arepi_gemm_rs_ring: AREPI_TILE_OWNER_FIRST and AREPI_TILE_OWNER_HALF are not "
                                  "options of the ring order");
    int rc = arepi_gemm_rs_supports(M, N, K, R, owner, flag_tile_m, flag_tile_n, publish, tile_cfg);
    if (rc) return rc;
    if (R > 1 && (M / R) % kRingRowAlign)
        return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_ring: segment height M/R=" + std::to_string(M / R) +
                                            " must be a multiple of " + std::to_string(kRingRowAlign));
    // When it publishes, a tile waits for its segments' upstream partials
    // before it publishes them on; a tile spanning two segments would make each
    // segment's publication wait for the other's arrival, which across the
    // ranks of a ring closes a cycle.  So each row block must lie in one
    // segment (the segment height a multiple of the tile height).
    if (publish && R > 1) {
        const int id = tile_cfg & ~AREPI_TILE_CONSUME_READY;
        if (id == AREPI_TILE_AUTO) {
            if (pick_tile(M, N, K, R, flag_tile_m, flag_tile_n, true, true) < 0)
                return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_ring: no compute tile fits whole in one segment of " +
                                                    std::to_string(M / R) + " rows with whole flag tiles");
        } else if ((M / R) % find_tile(id)->BM) {
            return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_ring: with ready_out, tile rows " +
                                                std::to_string(find_tile(id)->BM) + " must divide the segment height " +
                                                std::to_string(M / R));
        }
    }
    return ok();
}

extern "C" int arepi_gemm_rs_ring_pick_tile(int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                                            int flag_tile_n, int publish) {
    int rc = arepi_gemm_rs_ring_supports(M, N, K, R, owner, flag_tile_m, flag_tile_n, publish, AREPI_TILE_AUTO);
    if (rc) return rc;
    const int t = pick_tile(M, N, K, R, flag_tile_m, flag_tile_n, publish != 0, publish != 0);
    ok();
    return t;
}

extern "C" int arepi_gemm_rs_ring(const uint16_t *x, const uint16_t *w, const uint16_t *const *upstream,
                                  uint32_t *ready_in, uint16_t *out, uint16_t *send, uint32_t *ready_out,
                                  int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                                  int flag_tile_n, int scope, int tile_cfg, uint32_t *status, int64_t spin_limit,
                                  arepi_stream_t stream) {
    const bool publish = ready_out != nullptr;
    int rc = arepi_gemm_rs_ring_supports(M, N, K, R, owner, flag_tile_m, flag_tile_n, publish, tile_cfg);
    if (rc) return rc;
    // one rank: nothing comes from upstream, the ring is the plain GEMM
    if (R == 1)
        return arepi_gemm_rs_fused(x, w, nullptr, ready_in, out, send, ready_out, M, N, K, R, owner, flag_tile_m,
                                   flag_tile_n, scope, tile_cfg, status, spin_limit, stream);
    auto bad = [](const std::string &m) { return fail(AREPI_EINVAL, "arepi_gemm_rs_ring: " + m); };
    if (!x || !w || !out) return bad("x, w and out must be non-NULL");
    if (!aligned16(x) || !aligned16(w) || !aligned16(out)) return bad("x, w and out must be 16-byte aligned");
    if (!send) return bad("send must be non-NULL (every non-owner row is pushed on)");
    if (!aligned16(send)) return bad("send must be 16-byte aligned");
    if (scope != AREPI_SCOPE_AGENT && scope != AREPI_SCOPE_SYSTEM)
        return bad("scope=" + std::to_string(scope) + " is neither AREPI_SCOPE_AGENT nor AREPI_SCOPE_SYSTEM");
    if (!upstream) return bad("upstream must be a host array of R device pointers");
    if (!ready_in) return bad("ready_in must be non-NULL when R > 1");
    const int chain = (owner + R - 1) % R;
    for (int d = 0; d < R; ++d) {
        if (d == chain) continue;
        if (!upstream[d]) return bad("upstream[" + std::to_string(d) + "] is NULL");
        if (!aligned16(upstream[d])) return bad("upstream[" + std::to_string(d) + "] must be 16-byte aligned");
    }
    const CfgChoice c = decode_cfg(M, N, K, R, flag_tile_m, flag_tile_n, publish, tile_cfg, /*whole_segments=*/true);

    GemmRsParams p{};
    p.x = x;
    p.w = w;
    p.npeers = 1;
    for (int d = 0; d < R; ++d) p.up[d] = d == chain ? nullptr : upstream[d];
    p.ready_in = ready_in;
    p.out = out;
    p.send = send;
    p.ready_out = ready_out;
    p.status = status;
    p.spin_limit = spin_bound(spin_limit);
    p.system_scope = scope == AREPI_SCOPE_SYSTEM;
    p.consume = c.consume ? 1 : 0;
    rc = plan(p, c.t, M, N, K, R, owner, flag_tile_m, flag_tile_n, c.nest, /*contiguous=*/true);
    if (rc) return rc;
    p.ring = 1;
    p.chain = chain;
    p.ob1 = (int)((((int64_t)chain + 1) * p.seg - 1) / c.t->BM);  // the chain segment's last row block

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (c.id) {
        case AREPI_TILE_256x256: launch_ring<256, 256, 128, 128, 64, 2, 1>(p, s); break;
        case AREPI_TILE_128x256: launch_ring<128, 256, 64, 128, 64, 2, 1>(p, s); break;
        case AREPI_TILE_128x128: launch_ring<128, 128, 64, 64, 64, 2, 0>(p, s); break;
        case AREPI_TILE_64x128: launch_ring<64, 128, 32, 64, 64, 2, 0>(p, s); break;
        case AREPI_TILE_32x256: launch_ring<32, 256, 32, 64, 64, 2, 0>(p, s); break;
        case AREPI_TILE_256x256_S4: launch_ring<256, 256, 128, 128, 32, 4, 1>(p, s); break;
        case AREPI_TILE_256x128_S3: launch_ring<256, 128, 128, 64, 32, 3, 2>(p, s); break;
        case AREPI_TILE_128x256_S3: launch_ring<128, 256, 64, 128, 32, 3, 2>(p, s); break;
        case AREPI_TILE_128x128_S4: launch_ring<128, 128, 64, 64, 32, 4, 2>(p, s); break;
        case AREPI_TILE_256x256_W8: launch_ring<256, 256, 128, 64, 32, 4, 2>(p, s); break;
        case AREPI_TILE_256x256_W8_K64: launch_ring<256, 256, 128, 64, 64, 2, 2>(p, s); break;
        case AREPI_TILE_64x128_S4: launch_ring<64, 128, 32, 64, 64, 4, 0>(p, s); break;
        default: return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_ring: no kernel for tile " + std::to_string(c.id));
    }
    return check_launch("arepi_gemm_rs_ring");
}
