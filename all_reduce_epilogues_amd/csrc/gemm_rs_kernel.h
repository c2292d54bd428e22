// gemm_rs_kernel.h -- the direct-form GEMM + reduce-scatter kernel entry and
// its launch by compute tile, shared by the two translation units that
// instantiate it: gemm_rs.hip (workgroups whose rows never mix owner rows with
// published rows of other segments) and gemm_rs_mixed.hip (the instantiation
// that also carries the bodies for such mixed workgroups, which stage their
// accumulators twice and need more registers).
#ifndef AREPI_GEMM_RS_KERNEL_H
#define AREPI_GEMM_RS_KERNEL_H

#include "gemm_rs_impl.h"

namespace arepi {
namespace {

// WPE: waves per SIMD the register allocation targets (1 = one big-tile
// workgroup per CU; 2 = two co-resident workgroups; 0 = no target).
// MIXED: the instantiation that can run a workgroup holding owner rows and
// published rows of other segments (those rows are published before the
// readiness wait); without it such a workgroup never occurs.
template <int BM, int BN, int WM, int WN, int BK, int S, int WPE, int PEERS, bool MIXED>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1, WPE > 0 ? WPE : 8)))
    gemm_rs_kernel(const GemmRsParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[lds_bytes<BM, BN, BK, S>()];
    constexpr int CK = BM >= 64 ? BM / 2 : BM;
    // The 8-wave 256x256 BK 64 tile and the 4-wave 128x256 tile can run the
    // owner segment as half-height tiles (BM/2 x BN with the same waves, WM/2
    // rows each) in the workgroups after the nWG others.
    constexpr bool kHalfOwner = BN == 256 && BK == 64 && S == 2 &&
                                ((BM == 256 && WM == 128 && WN == 64) || (BM == 128 && WM == 64 && WN == 128));
    if constexpr (kHalfOwner) {
        if ((int)blockIdx.x >= p.nWG) {
            int h, hcb;
            owner_half_of_block(p, blockIdx.x, h, hcb);
            const int64_t h0 = (int64_t)p.owner * p.seg + (int64_t)h * (BM / 2);
            gemm_rs_body<BM / 2, BN, WM / 2, WN, BK, S, WPE, PEERS, kOwnerRowsAnywhere>(p, smem, -1, hcb, h0, BM / 4,
                                                                                      h0 + BM / 4, BM / 4);
            return;
        }
    } else {
        if ((int)blockIdx.x >= p.nWG) return;  // (the host never launches extra workgroups for this tile)
    }
    int rb, cb;
    tile_of_block(p, blockIdx.x, rb, cb);
    int64_t a0, b0;
    int alen, blen;
    chunks_of_block(p, BM, CK, rb, a0, alen, b0, blen);
    const int64_t oseg0 = (int64_t)p.owner * p.seg, oseg1 = oseg0 + p.seg;
    const bool own_a = alen > 0 && a0 < oseg1 && a0 + alen > oseg0;
    const bool own_b = blen > 0 && b0 < oseg1 && b0 + blen > oseg0;
    if (!own_a && !own_b) {
        gemm_rs_body<BM, BN, WM, WN, BK, S, WPE, PEERS, kNoOwnerRows>(p, smem, rb, cb, a0, alen, b0, blen);
        return;
    }
    if constexpr (MIXED) {
        // rows of other segments beside owner rows, published: those go first
        const bool other_a = alen > 0 && (a0 < oseg0 || a0 + alen > oseg1);
        const bool other_b = blen > 0 && (b0 < oseg0 || b0 + blen > oseg1);
        if (p.ready_out != nullptr && (other_a || other_b)) {
            if (p.paired)  // paired half-blocks: only chunk A can be an owner chunk
                gemm_rs_body<BM, BN, WM, WN, BK, S, WPE, PEERS, kOwnerChunkAPub>(p, smem, rb, cb, a0, alen, b0, blen);
            else
                gemm_rs_body<BM, BN, WM, WN, BK, S, WPE, PEERS, kOwnerAnywherePub>(p, smem, rb, cb, a0, alen, b0,
                                                                                  blen);
            return;
        }
    }
    if (p.paired)
        gemm_rs_body<BM, BN, WM, WN, BK, S, WPE, PEERS, kOwnerChunkA>(p, smem, rb, cb, a0, alen, b0, blen);
    else
        gemm_rs_body<BM, BN, WM, WN, BK, S, WPE, PEERS, kOwnerRowsAnywhere>(p, smem, rb, cb, a0, alen, b0, blen);
}

template <int BM, int BN, int WM, int WN, int BK, int S, int WPE, bool MIXED>
void launch(const GemmRsParams &p, hipStream_t stream) {
    constexpr int NT = (BM / WM) * (BN / WN) * 64;
    const dim3 grid(p.nWG + p.nextra);  // the owner half-height workgroups come after the others
    if (p.npeers <= 1)
        hipLaunchKernelGGL((gemm_rs_kernel<BM, BN, WM, WN, BK, S, WPE, 1, MIXED>), grid, dim3(NT), 0, stream, p);
    else if (p.npeers <= 3)
        hipLaunchKernelGGL((gemm_rs_kernel<BM, BN, WM, WN, BK, S, WPE, 3, MIXED>), grid, dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_rs_kernel<BM, BN, WM, WN, BK, S, WPE, kMaxR - 1, MIXED>), grid, dim3(NT), 0, stream,
                           p);
}

// Launches tile `cfg`; false if there is no kernel for it.
template <bool MIXED>
bool launch_tile(int cfg, const GemmRsParams &p, hipStream_t s) {
    switch (cfg) {
        case AREPI_TILE_256x256: launch<256, 256, 128, 128, 64, 2, 1, MIXED>(p, s); return true;
        case AREPI_TILE_128x256: launch<128, 256, 64, 128, 64, 2, 1, MIXED>(p, s); return true;
        case AREPI_TILE_128x128: launch<128, 128, 64, 64, 64, 2, 0, MIXED>(p, s); return true;
        case AREPI_TILE_64x128: launch<64, 128, 32, 64, 64, 2, 0, MIXED>(p, s); return true;
        case AREPI_TILE_32x256: launch<32, 256, 32, 64, 64, 2, 0, MIXED>(p, s); return true;
        case AREPI_TILE_256x256_S4: launch<256, 256, 128, 128, 32, 4, 1, MIXED>(p, s); return true;
        case AREPI_TILE_256x128_S3: launch<256, 128, 128, 64, 32, 3, 2, MIXED>(p, s); return true;
        case AREPI_TILE_128x256_S3: launch<128, 256, 64, 128, 32, 3, 2, MIXED>(p, s); return true;
        case AREPI_TILE_128x128_S4: launch<128, 128, 64, 64, 32, 4, 2, MIXED>(p, s); return true;
        case AREPI_TILE_256x256_W8: launch<256, 256, 128, 64, 32, 4, 2, MIXED>(p, s); return true;
        case AREPI_TILE_256x256_W8_K64: launch<256, 256, 128, 64, 64, 2, 2, MIXED>(p, s); return true;
        case AREPI_TILE_64x128_S4: launch<64, 128, 32, 64, 64, 4, 0, MIXED>(p, s); return true;
        default: return false;
    }
}

}  // namespace

// Defined in gemm_rs_mixed.hip: launch_tile<true>.  The parameters travel as
// an opaque pointer: GemmRsParams is local to each translation unit (the same
// standard-layout definition in both).
bool launch_gemm_rs_mixed(int cfg, const void *params, hipStream_t s);

}  // namespace arepi

#endif  // AREPI_GEMM_RS_KERNEL_H
