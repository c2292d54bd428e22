// gemm_rs_fp8.hip -- fp8 (e4m3fn) block-scaled GEMM with the fused
// reduce-scatter epilogue, for gfx950 (MI355X), and its C entry point.
//
// What it computes follows ROCm/mori PR #662 (the blockscale commit of the
// fused wo_b GEMM + all-reduce: X quantised 1x128 along K, W 128x128, fp32
// scales; the running-rescale accumulator t_b = t_{b-1} * (s_{b-1}/s_b) + d_b,
// out = t_last * s_last, which needs no second accumulator) and the re-review
// finding that the gfx950 matrix atom reads the OCP e4m3fn encoding (e4m3fnuz
// bytes are not accepted).  The reduce-scatter epilogue is the direct-sum form
// of gemm_rs.hip; the mainloop is the fp8 branch of the shared body
// (gemm_rs_impl.h), on a 256x256 tile of eight 128x64 waves (one workgroup per
// CU; per MFMA a 128x64 wave reads a third fewer LDS bytes than a 64x64 one,
// and the wide tile loads half the operand bytes per FLOP of 128x128).
#include "gemm_rs_impl.h"

namespace arepi {
namespace {

// MIXED: the instantiation that can run a workgroup holding owner rows beside
// published rows of other segments (published before its readiness wait).
template <int PEERS, bool MIXED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) gemm_rs_fp8_kernel(const GemmRsParams p) {
    // two stages, their 2 KiB scale areas, then 2 x 2 x 256 factors
    __shared__ __attribute__((aligned(1024))) uint8_t smem[lds_bytes<256, 256, 64, 2>() + 2 * 2048 + 2 * 2 * 256 * 4];
    constexpr int BM = 256, CK = 128;
    int rb, cb;
    tile_of_block(p, blockIdx.x, rb, cb);
    int64_t a0, b0;
    int alen, blen;
    chunks_of_block(p, BM, CK, rb, a0, alen, b0, blen);
    const int64_t oseg0 = (int64_t)p.owner * p.seg, oseg1 = oseg0 + p.seg;
    const bool own_a = alen > 0 && a0 < oseg1 && a0 + alen > oseg0;
    const bool own_b = blen > 0 && b0 < oseg1 && b0 + blen > oseg0;
    if (!own_a && !own_b) {
        gemm_rs_body<256, 256, 128, 64, 64, 2, 2, PEERS, kNoOwnerRows, true>(p, smem, rb, cb, a0, alen, b0, blen);
        return;
    }
    if constexpr (MIXED) {
        const bool other_a = alen > 0 && (a0 < oseg0 || a0 + alen > oseg1);
        const bool other_b = blen > 0 && (b0 < oseg0 || b0 + blen > oseg1);
        if (p.ready_out != nullptr && (other_a || other_b)) {
            gemm_rs_body<256, 256, 128, 64, 64, 2, 2, PEERS, kOwnerAnywherePub, true>(p, smem, rb, cb, a0, alen, b0,
                                                                                    blen);
            return;
        }
    }
    gemm_rs_body<256, 256, 128, 64, 64, 2, 2, PEERS, kOwnerRowsAnywhere, true>(p, smem, rb, cb, a0, alen, b0, blen);
}

}  // namespace
}  // namespace arepi

using namespace arepi;

extern "C" int arepi_gemm_rs_fp8_supports(int64_t M, int64_t N, int64_t K, int R, int owner, int flag_tile_m,
                                          int flag_tile_n, int publish, int tile_cfg) {
    int rc = validate_shape(M, N, K, R, owner, flag_tile_m, flag_tile_n);
    if (rc) return rc;
    if (K % 128) return fail(AREPI_EINVAL, "arepi_gemm_rs_fp8: K=" + std::to_string(K) + " must be a multiple of 128");
    if (tile_cfg & ~AREPI_TILE_CONSUME_READY)
        return fail(AREPI_EUNSUPPORTED,
                    "arepi_gemm_rs_fp8: tile_cfg may only carry AREPI_TILE_CONSUME_READY (the tile is 256x256)");
    const bool nest = publish || (tile_cfg & AREPI_TILE_CONSUME_READY);
    if (nest && !flags_nest(M, N, R, flag_tile_m, flag_tile_n, 256, 256))
        return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_fp8: flag tiles " + std::to_string(flag_tile_m) + "x" +
                                            std::to_string(flag_tile_n) + " straddle 256x256 compute tiles");
    return ok();
}

extern "C" int arepi_gemm_rs_fp8(const uint8_t *x, const float *xs, const uint8_t *wt, const float *ws,
                                 const uint16_t *const *recv, uint32_t *ready_in, uint16_t *out, uint16_t *send,
                                 uint32_t *ready_out, int64_t M, int64_t N, int64_t K, int R, int owner,
                                 int flag_tile_m, int flag_tile_n, int scope, int tile_cfg, uint32_t *status,
                                 int64_t spin_limit, arepi_stream_t stream) {
    const bool publish = ready_out != nullptr;
    int rc = arepi_gemm_rs_fp8_supports(M, N, K, R, owner, flag_tile_m, flag_tile_n, publish, tile_cfg);
    if (rc) return rc;
    auto bad = [](const std::string &m) { return fail(AREPI_EINVAL, "arepi_gemm_rs_fp8: " + m); };
    if (!x || !xs || !wt || !ws || !out) return bad("x, xs, wt, ws and out must be non-NULL");
    if (!aligned16(x) || !aligned16(wt) || !aligned16(out)) return bad("x, wt and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(xs) | reinterpret_cast<uintptr_t>(ws)) & 3)
        return bad("xs and ws must be 4-byte aligned");
    if (send && !aligned16(send)) return bad("send must be 16-byte aligned");
    if (publish && !send) return bad("ready_out needs send (the tiles it publishes)");
    if (scope != AREPI_SCOPE_AGENT && scope != AREPI_SCOPE_SYSTEM)
        return bad("scope=" + std::to_string(scope) + " is neither AREPI_SCOPE_AGENT nor AREPI_SCOPE_SYSTEM");
    if (M * (K / 128) * 4 >= (int64_t)1 << 31) return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_fp8: xs too large");
    if (R > 1) {
        if (!recv) return bad("recv must be a host array of R device pointers");
        if (!ready_in) return bad("ready_in must be non-NULL when R > 1");
        for (int q = 0; q < R; ++q) {
            if (q == owner) continue;
            if (!recv[q]) return bad("recv[" + std::to_string(q) + "] is NULL");
            if (!aligned16(recv[q])) return bad("recv[" + std::to_string(q) + "] must be 16-byte aligned");
        }
    }
    GemmRsParams p{};
    p.x = reinterpret_cast<const uint16_t *>(x);
    p.w = reinterpret_cast<const uint16_t *>(wt);
    p.xs = xs;
    p.ws = ws;
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
    p.consume = (tile_cfg & AREPI_TILE_CONSUME_READY) ? 1 : 0;
    rc = plan(p, find_tile(AREPI_TILE_256x256_W8_K64), M, N, K, R, owner, flag_tile_m, flag_tile_n,
              publish || p.consume, /*contiguous=*/true);
    if (rc) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // a 256-row block mixes owner rows with published rows only when ready_out
    // is given and the segment height is not a multiple of 256
    if (ready_out && R > 1 && p.seg % 256) {
        if (p.npeers <= 1)
            hipLaunchKernelGGL((gemm_rs_fp8_kernel<1, true>), dim3(p.nWG), dim3(512), 0, s, p);
        else if (p.npeers <= 3)
            hipLaunchKernelGGL((gemm_rs_fp8_kernel<3, true>), dim3(p.nWG), dim3(512), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_rs_fp8_kernel<kMaxR - 1, true>), dim3(p.nWG), dim3(512), 0, s, p);
    } else {
        if (p.npeers <= 1)
            hipLaunchKernelGGL((gemm_rs_fp8_kernel<1, false>), dim3(p.nWG), dim3(512), 0, s, p);
        else if (p.npeers <= 3)
            hipLaunchKernelGGL((gemm_rs_fp8_kernel<3, false>), dim3(p.nWG), dim3(512), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_rs_fp8_kernel<kMaxR - 1, false>), dim3(p.nWG), dim3(512), 0, s, p);
    }
    return check_launch("arepi_gemm_rs_fp8");
}
