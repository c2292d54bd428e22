// gemm_rs.hip -- row-parallel bf16 GEMM with a fused reduce-scatter epilogue
// for gfx950 (MI355X), direct-sum form, and its C entry points.
//
// What it computes follows DeepGEMM PR #1 "Fused ring RS: per-tile bitmask +
// drain-ring with owner-boundary flush" (description) and ROCm/mori PR #662
// (PR description, fused GEMM + all-reduce of the wo_b projection), in the
// direct-sum form: each rank computes its full local product C = X.W; the owner
// segment's tiles add the R-1 peer partials in the epilogue, all other rows are
// stored as this rank's outgoing partials.  The kernel body, tile schedule and
// host-side planning are shared with the push-ring form (gemm_rs_impl.h).
#include "gemm_rs_impl.h"

namespace arepi {
namespace {

// WPE: waves per SIMD the register allocation targets (1 = one big-tile
// workgroup per CU; 2 = two co-resident workgroups; 0 = no target).
template <int BM, int BN, int WM, int WN, int BK, int S, int WPE, int PEERS>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1, WPE > 0 ? WPE : 8)))
    gemm_rs_kernel(const GemmRsParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[lds_bytes<BM, BN, BK, S>()];
    constexpr int CK = BM >= 64 ? BM / 2 : BM;
    int rb, cb;
    tile_of_block(p, blockIdx.x, rb, cb);
    int64_t a0, b0;
    int alen, blen;
    chunks_of_block(p, BM, CK, rb, a0, alen, b0, blen);
    const int64_t oseg0 = (int64_t)p.owner * p.seg, oseg1 = oseg0 + p.seg;
    const bool own_a = alen > 0 && a0 < oseg1 && a0 + alen > oseg0;
    const bool own_b = blen > 0 && b0 < oseg1 && b0 + blen > oseg0;
    if (!own_a && !own_b)
        gemm_rs_body<BM, BN, WM, WN, BK, S, WPE, PEERS, kNoOwnerRows>(p, smem, rb, cb, a0, alen, b0, blen);
    else if (p.paired)  // paired half-blocks: only chunk A can be an owner chunk
        gemm_rs_body<BM, BN, WM, WN, BK, S, WPE, PEERS, kOwnerChunkA>(p, smem, rb, cb, a0, alen, b0, blen);
    else
        gemm_rs_body<BM, BN, WM, WN, BK, S, WPE, PEERS, kOwnerRowsAnywhere>(p, smem, rb, cb, a0, alen, b0, blen);
}

template <int BM, int BN, int WM, int WN, int BK, int S, int WPE>
void launch(const GemmRsParams &p, hipStream_t stream) {
    constexpr int NT = (BM / WM) * (BN / WN) * 64;
    if (p.npeers <= 1)
        hipLaunchKernelGGL((gemm_rs_kernel<BM, BN, WM, WN, BK, S, WPE, 1>), dim3(p.nWG), dim3(NT), 0, stream, p);
    else if (p.npeers <= 3)
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
    const bool consume = (tile_cfg & AREPI_TILE_CONSUME_READY) != 0;
    // consuming readiness bits needs the same nesting as publishing them
    const bool nest = publish || consume;
    if ((tile_cfg & ~AREPI_TILE_CONSUME_READY) == AREPI_TILE_AUTO) {
        rc = arepi_gemm_rs_pick_tile(M, N, K, R, owner, flag_tile_m, flag_tile_n, nest);
        return rc < 0 ? rc : ok();
    }
    const bool contiguous = (tile_cfg & AREPI_TILE_PAIRED_ROWS) == 0;
    const int id = tile_cfg & ~(AREPI_TILE_PAIRED_ROWS | AREPI_TILE_CONSUME_READY);
    const TileCfg *t = id == AREPI_TILE_AUTO ? nullptr : find_tile(id);
    if (!t) return fail(AREPI_EINVAL, "arepi_gemm_rs: tile_cfg=" + std::to_string(tile_cfg) + " is not an AREPI_TILE_* value");
    if (nest && !flags_nest(M, N, R, flag_tile_m, flag_tile_n, t->BM, t->BN) &&
        !use_paired(M, N, R, flag_tile_m, flag_tile_n, t->BM, t->BN, true, contiguous))
        return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs: flag tiles " + std::to_string(flag_tile_m) + "x" +
                                            std::to_string(flag_tile_n) + " straddle " + std::to_string(t->BM) +
                                            "x" + std::to_string(t->BN) + " compute tiles");
    return ok();
}

extern "C" int arepi_gemm_rs_fused(const uint16_t *x, const uint16_t *w, const uint16_t *const *recv,
                                   uint32_t *ready_in, uint16_t *out, uint16_t *send,
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
    const CfgChoice c = decode_cfg(M, N, K, R, flag_tile_m, flag_tile_n, publish, tile_cfg);
    const int cfg = c.id;

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
    p.spin_limit = spin_bound(spin_limit);
    p.system_scope = scope == AREPI_SCOPE_SYSTEM;
    p.consume = c.consume ? 1 : 0;
    rc = plan(p, c.t, M, N, K, R, owner, flag_tile_m, flag_tile_n, c.nest, c.contiguous);
    if (rc) return rc;

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
        case AREPI_TILE_256x256_W8: launch<256, 256, 128, 64, 32, 4, 2>(p, s); break;
        case AREPI_TILE_256x256_W8_K64: launch<256, 256, 128, 64, 64, 2, 2>(p, s); break;
        default: return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_fused: no kernel for tile " + std::to_string(cfg));
    }
    return check_launch("arepi_gemm_rs_fused");
}

extern "C" int64_t arepi_gemm_rs_schedule(int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                                          int flag_tile_n, int publish, int tile_cfg, int64_t *rows,
                                          int64_t capacity) {
    int rc = arepi_gemm_rs_supports(M, N, K, R, owner, flag_tile_m, flag_tile_n, publish, tile_cfg);
    if (rc) return rc;
    const CfgChoice c = decode_cfg(M, N, K, R, flag_tile_m, flag_tile_n, publish != 0, tile_cfg);
    const TileCfg *t = c.t;
    GemmRsParams p{};
    rc = plan(p, t, M, N, K, R, owner, flag_tile_m, flag_tile_n, c.nest, c.contiguous);
    if (rc) return rc;
    if (rows) {
        if (capacity < (int64_t)p.nWG * 6)
            return fail(AREPI_EINVAL, "arepi_gemm_rs_schedule: capacity " + std::to_string(capacity) + " < 6 x " +
                                          std::to_string(p.nWG) + " workgroups");
        const int CK = chunk_rows(t->BM);
        for (int b = 0; b < p.nWG; ++b) {
            int rb, cb, alen, blen;
            int64_t a0, b0;
            tile_of_block(p, b, rb, cb);
            chunks_of_block(p, t->BM, CK, rb, a0, alen, b0, blen);
            int64_t *r = rows + (int64_t)b * 6;
            r[0] = rb, r[1] = cb, r[2] = a0, r[3] = alen, r[4] = b0, r[5] = blen;
        }
    }
    ok();
    return p.nWG;
}
