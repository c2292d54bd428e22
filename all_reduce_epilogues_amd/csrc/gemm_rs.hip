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
#include "gemm_rs_kernel.h"


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
    if ((tile_cfg & AREPI_TILE_OWNER_FIRST) && (tile_cfg & AREPI_TILE_PAIRED_ROWS))
        return fail(AREPI_EINVAL, "arepi_gemm_rs: AREPI_TILE_OWNER_FIRST needs the contiguous row layout");
    if (tile_cfg & AREPI_TILE_OWNER_HALF) {
        // owner rows as half-height tiles (256x256_w8_k64 and 128x256 only)
        if (tile_cfg & (AREPI_TILE_PAIRED_ROWS | AREPI_TILE_OWNER_FIRST))
            return fail(AREPI_EINVAL, "arepi_gemm_rs: AREPI_TILE_OWNER_HALF needs the contiguous, owner-last layout");
        const bool consume_h = (tile_cfg & AREPI_TILE_CONSUME_READY) != 0;
        int base = tile_cfg & ~(AREPI_TILE_OWNER_HALF | AREPI_TILE_CONSUME_READY);
        if (base == AREPI_TILE_AUTO) {
            base = arepi_gemm_rs_pick_tile(M, N, K, R, owner, flag_tile_m, flag_tile_n, publish || consume_h);
            if (base < 0) return base;
        }
        if (!has_owner_half(base))
            return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs: AREPI_TILE_OWNER_HALF applies to AREPI_TILE_256x256_W8_K64 "
                                            "and AREPI_TILE_128x256 (explicit, or as the automatic choice)");
        const int bm = find_tile(base)->BM;
        if (R < 2 || (M / R) % bm)
            return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs: AREPI_TILE_OWNER_HALF needs R >= 2 and the segment "
                                            "height M/R a multiple of " + std::to_string(bm));
        if (!owner_half_fits(M, N, R, flag_tile_m, flag_tile_n, consume_h, base))
            return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs: AREPI_TILE_OWNER_HALF: consumed flag tiles " +
                                                std::to_string(flag_tile_m) + "x" + std::to_string(flag_tile_n) +
                                                " straddle the " + std::to_string(bm / 2) + "-row owner tiles");
        tile_cfg = (tile_cfg & AREPI_TILE_CONSUME_READY) | base;
    }
    tile_cfg &= ~AREPI_TILE_OWNER_FIRST;
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
    rc = plan(p, c.t, M, N, K, R, owner, flag_tile_m, flag_tile_n, c.nest, c.contiguous, c.owner_first,
              c.owner_half);
    if (rc) return rc;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // a workgroup can mix owner rows with published rows of other segments
    // only when ready_out is given and either half-blocks are paired or a row
    // block straddles a segment boundary
    const int BM = c.t->BM;
    const bool mixed = ready_out && R > 1 && (p.paired || p.seg % BM != 0);
    const bool launched = mixed ? launch_gemm_rs_mixed(cfg, &p, s) : launch_tile<false>(cfg, p, s);
    if (!launched) return fail(AREPI_EUNSUPPORTED, "arepi_gemm_rs_fused: no kernel for tile " + std::to_string(cfg));
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
    rc = plan(p, t, M, N, K, R, owner, flag_tile_m, flag_tile_n, c.nest, c.contiguous, c.owner_first,
              c.owner_half);
    if (rc) return rc;
    const int total = p.nWG + p.nextra;
    if (rows) {
        if (capacity < (int64_t)total * 6)
            return fail(AREPI_EINVAL, "arepi_gemm_rs_schedule: capacity " + std::to_string(capacity) + " < 6 x " +
                                          std::to_string(total) + " workgroups");
        const int CK = chunk_rows(t->BM);
        for (int b = 0; b < total; ++b) {
            int rb, cb, alen, blen;
            int64_t a0, b0;
            if (b < p.nWG) {
                tile_of_block(p, b, rb, cb);
                chunks_of_block(p, t->BM, CK, rb, a0, alen, b0, blen);
            } else {
                // owner half-height tile: row block -1, two chunks of BM/4 rows
                int h;
                owner_half_of_block(p, b, h, cb);
                rb = -1;
                a0 = (int64_t)owner * p.seg + (int64_t)h * (t->BM / 2);
                alen = blen = t->BM / 4;
                b0 = a0 + alen;
            }
            int64_t *r = rows + (int64_t)b * 6;
            r[0] = rb, r[1] = cb, r[2] = a0, r[3] = alen, r[4] = b0, r[5] = blen;
        }
    }
    ok();
    return total;
}
