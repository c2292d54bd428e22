/*
 * oracle.c -- plain CPU oracle for the fused all-reduce epilogues.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP kernels behind include/arepi.h) never calls it and shares no code,
 * header, table or helper with it.
 *
 * Every function here is the plain definition of what the method computes,
 * written as slow, obviously-correct loops:
 *   - fp32 accumulation with a fixed summation order (the order each function
 *     states), compiled with -ffp-contract=off and no fast-math, so every
 *     multiply and add is a separately rounded IEEE binary32 operation;
 *   - bf16 values are handled as their raw 16-bit patterns; bf16 -> fp32 is the
 *     exact 16-bit shift and fp32 -> bf16 is round-to-nearest-even;
 *   - OpenMP splits work over output rows only, so threading never changes any
 *     element's arithmetic.
 *
 * Sources (web pages; the section named is where the fact is stated):
 *   [P1] DeepGEMM PR #1 "Fused ring RS: per-tile bitmask + drain-ring with
 *        owner-boundary flush" -- description (per-tile readiness instead of a
 *        per-segment flag; the owner segment ends with the full sum).
 *   [P2] ROCm/mori PR #662 "Fuse DSV4-Pro wo_b's GEMM with its all-reduce over
 *        cco SDMA" -- PR description, self_test commit, second review.
 *   [P4] ROCm/aiter PR #4977 "Single-kernel Lamport fused all-reduce + RMSNorm"
 *        -- Approach section and the correctness notes of the bring-up commit.
 *   [P5] DeepEP PR #527 (issue #613 mirror) "Fix the MultiStages for intranode
 *        combine" -- description.
 *
 * Readings where the pages leave a step open (also listed with the design
 * notes of the repository):
 *   - the GEMM-RS rank computes its full local product X_r.W_r [M,N]; rows of
 *     the owner segment get the peer partials added, all other rows are this
 *     rank's outgoing partials for their owners;
 *   - fp32 -> bf16 conversion is round-to-nearest-even;
 *   - summation orders: GEMM k ascending, then the local accumulator plus the
 *     peer partials in ascending rank order skipping the owner; Lamport slots
 *     0..S-1; combine experts 0..E-1;
 *   - RMSNorm: y = x * (1/sqrt(mean(x^2) + eps)) * gamma, mean over the row;
 *   - combine: y[t,h] = sum_k gate[t,k] * x[t,k,h], gate applied as given.
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- bf16 <-> fp32 --------------------------------------------------------- */

/* bf16 is the upper half of a binary32 pattern: widening is exact. */
static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round-to-nearest-even to the upper 16 bits.  A NaN becomes a quiet NaN with
 * its sign kept; overflow past the largest finite bf16 rounds to infinity as
 * IEEE rounding requires (the carry walks into the exponent). */
static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

void oracle_bf16_from_f32(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

void oracle_f32_from_bf16(const uint16_t *in, float *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_f32(in[i]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- GEMM + reduce-scatter epilogue ([P1] description, [P2] PR description) --
 *
 * One rank r of R holds X_r [M,K] and W_r [K,N] (both row-major bf16).  Its
 * local partial is C_r = X_r . W_r, accumulated in fp32 with k ascending.  The
 * M rows are split into R equal segments of seg = M/R rows; segment d belongs
 * to rank d.  For the owner segment this rank finishes the reduce-scatter:
 *     out[i,n] = bf16( C_r[owner*seg + i, n] + sum_{p != owner} recv[p][i,n] )
 * (local accumulator first, then peers in ascending rank order, fp32 adds).
 * Every other row i is this rank's outgoing partial for the owner of its
 * segment:  send[i,n] = bf16( C_r[i,n] ).
 *
 * recv is an array of R pointers to [seg,N] bf16 buffers; recv[owner] is never
 * read.  send may be NULL.  Only rows [row_begin, row_end) of C_r are computed
 * (so large shapes can be sampled a row band at a time).
 *
 * The bf16 x bf16 product has at most 16 significant bits, so it is exact in
 * fp32 and a fused multiply-add would give the same bits as the separate
 * multiply and add written here.
 *
 * Returns 0, or -1 on bad arguments.  The loop nest runs k outside n so that a
 * row of W is read contiguously; each element's own sum is still k ascending.
 */
int oracle_gemm_rs(const uint16_t *x, const uint16_t *w, const uint16_t *const *recv,
                   uint16_t *out, uint16_t *send, int64_t M, int64_t N, int64_t K, int R,
                   int owner, int64_t row_begin, int64_t row_end) {
    if (M < 0 || N < 0 || K < 0 || R < 1 || owner < 0 || owner >= R) return -1;
    if (M % R != 0) return -1;
    if (row_begin < 0 || row_end > M || row_begin > row_end) return -1;
    const int64_t seg = M / R;
    int bad = 0;
#pragma omp parallel
    {
        float *acc = (float *)malloc((size_t)(N > 0 ? N : 1) * sizeof(float));
        if (!acc) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = row_begin; i < row_end; ++i) {
                for (int64_t n = 0; n < N; ++n) acc[n] = 0.0f;
                for (int64_t k = 0; k < K; ++k) {
                    const float xv = bf16_to_f32(x[i * K + k]);
                    const uint16_t *wrow = w + k * N;
                    for (int64_t n = 0; n < N; ++n) acc[n] = acc[n] + xv * bf16_to_f32(wrow[n]);
                }
                const int64_t d = i / seg;
                if (d == owner) {
                    const int64_t li = i - (int64_t)owner * seg;
                    for (int64_t n = 0; n < N; ++n) {
                        float t = acc[n];
                        for (int p = 0; p < R; ++p) {
                            if (p == owner) continue;
                            t = t + bf16_to_f32(recv[p][li * N + n]);
                        }
                        out[li * N + n] = f32_to_bf16_rne(t);
                    }
                } else if (send) {
                    for (int64_t n = 0; n < N; ++n) send[i * N + n] = f32_to_bf16_rne(acc[n]);
                }
            }
            free(acc);
        }
    }
    return bad ? -1 : 0;
}

/* ---- fp8 block-scaled form of the local product ([P2] blockscale commit) ------
 *
 * Operands are fp8 e4m3fn bytes (the OCP encoding: sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent 0 is subnormal, S.1111.111 is NaN, no
 * infinities; 0x38 is 1.0, largest finite 448).  X is quantised in 1x128
 * blocks along K with fp32 scales xs [M][K/128] (row-major); W is held
 * transposed, wt [N][K] (K contiguous), quantised in 128x128 blocks with fp32
 * scales ws [ceil(N/128)][K/128].  The local product is the plain definition
 *     C[m,n] = sum_{b} (xs[m,b] * ws[n/128,b]) * d_b[m,n],
 *     d_b[m,n] = sum_{k in block b} dec(x[m,k]) * dec(wt[n,k])
 * in fp32: k ascending inside a block (a product of two e4m3 values is exact
 * in fp32), blocks ascending, the scale product formed first.  The
 * reduce-scatter epilogue on C is that of oracle_gemm_rs. */
float oracle_fp8_e4m3fn_to_f32(uint8_t b) {
    const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
    float v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexpf((float)m, -9); /* m/8 * 2^-6 */
    else
        v = ldexpf((float)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

int oracle_gemm_rs_fp8(const uint8_t *x, const float *xs, const uint8_t *wt, const float *ws,
                       const uint16_t *const *recv, uint16_t *out, uint16_t *send, int64_t M, int64_t N,
                       int64_t K, int R, int owner, int64_t row_begin, int64_t row_end) {
    if (M < 0 || N < 0 || K < 0 || K % 128 || R < 1 || owner < 0 || owner >= R || M % R) return -1;
    if (row_begin < 0 || row_end > M || row_begin > row_end) return -1;
    const int64_t seg = M / R, KB = K / 128;
    float lut[256];
    for (int i = 0; i < 256; ++i) lut[i] = oracle_fp8_e4m3fn_to_f32((uint8_t)i);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = row_begin; i < row_end; ++i) {
        const int64_t d = i / seg, li = i - d * seg;
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t b = 0; b < KB; ++b) {
                float db = 0.0f;
                for (int64_t k = b * 128; k < (b + 1) * 128; ++k) db = db + lut[x[i * K + k]] * lut[wt[n * K + k]];
                const float s = xs[i * KB + b] * ws[(n / 128) * KB + b];
                acc = acc + s * db;
            }
            if (d == owner) {
                float t = acc;
                for (int p = 0; p < R; ++p)
                    if (p != owner) t = t + bf16_to_f32(recv[p][li * N + n]);
                out[li * N + n] = f32_to_bf16_rne(t);
            } else if (send) {
                send[i * N + n] = f32_to_bf16_rne(acc);
            }
        }
    }
    return 0;
}

/* ---- push-ring form of the same reduce-scatter ([P1] description) ----------
 *
 * In the ring of [P1] each rank takes the running partial of a segment from
 * its upstream neighbour, adds its own partial and pushes the sum downstream;
 * the owner of the segment is the last rank of that chain and ends with the
 * full sum.  Reading taken here: rank r receives from rank r-1 and sends to
 * rank r+1 (mod R), so the chain of segment d runs d+1, d+2, ..., d; rank r
 * starts the chain of segment chain = (r - 1) mod R, which has no upstream
 * partial; the partials travel as bf16 (rounded at every hop).
 *
 * upstream is an array of R pointers to [seg,N] bf16 buffers: upstream[d] is
 * the running partial of segment d received from the upstream rank
 * (upstream[chain] is never read; with R = 1 nothing is read).
 *     out[i,n]  = bf16( C_r[owner*seg + i, n] + upstream[owner][i,n] )
 *     send[i,n] = bf16( C_r[i,n] + upstream[d][i - d*seg, n] )  (row i in segment d)
 *     send[i,n] = bf16( C_r[i,n] )                                (row i in segment chain)
 * C_r is accumulated exactly as in oracle_gemm_rs (fp32, k ascending), and
 * the local accumulator comes first in every add.
 */
int oracle_gemm_rs_ring(const uint16_t *x, const uint16_t *w, const uint16_t *const *upstream,
                        uint16_t *out, uint16_t *send, int64_t M, int64_t N, int64_t K, int R,
                        int owner, int64_t row_begin, int64_t row_end) {
    if (M < 0 || N < 0 || K < 0 || R < 1 || owner < 0 || owner >= R) return -1;
    if (M % R != 0) return -1;
    if (row_begin < 0 || row_end > M || row_begin > row_end) return -1;
    const int64_t seg = M / R;
    const int chain = (owner + R - 1) % R;
    int bad = 0;
#pragma omp parallel
    {
        float *acc = (float *)malloc((size_t)(N > 0 ? N : 1) * sizeof(float));
        if (!acc) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = row_begin; i < row_end; ++i) {
                for (int64_t n = 0; n < N; ++n) acc[n] = 0.0f;
                for (int64_t k = 0; k < K; ++k) {
                    const float xv = bf16_to_f32(x[i * K + k]);
                    const uint16_t *wrow = w + k * N;
                    for (int64_t n = 0; n < N; ++n) acc[n] = acc[n] + xv * bf16_to_f32(wrow[n]);
                }
                const int64_t d = i / seg, li = i - d * seg;
                const int adds = R > 1 && d != chain;
                if (d == owner) {
                    for (int64_t n = 0; n < N; ++n) {
                        float t = acc[n];
                        if (adds) t = t + bf16_to_f32(upstream[d][li * N + n]);
                        out[li * N + n] = f32_to_bf16_rne(t);
                    }
                } else if (send) {
                    for (int64_t n = 0; n < N; ++n) {
                        float t = acc[n];
                        if (adds) t = t + bf16_to_f32(upstream[d][li * N + n]);
                        send[i * N + n] = f32_to_bf16_rne(t);
                    }
                }
            }
            free(acc);
        }
    }
    return bad ? -1 : 0;
}

/* ---- per-tile readiness bitmask ([P1] title and description) ---------------
 *
 * Each segment is cut into flag tiles of ftm x ftn (clipped at the segment's
 * bottom and right edges), numbered row-major within the segment:
 *     tiles = ceil(seg/ftm) * ceil(N/ftn),  words = ceil(tiles/32).
 * Bit t of a segment's word array is flag tile t (word t/32, bit t%32).
 */
int64_t oracle_flag_tiles(int64_t M, int64_t N, int R, int64_t ftm, int64_t ftn) {
    if (R < 1 || M % R != 0 || ftm < 1 || ftn < 1 || M < 0 || N < 0) return -1;
    const int64_t seg = M / R;
    return ((seg + ftm - 1) / ftm) * ((N + ftn - 1) / ftn);
}

int64_t oracle_flag_words(int64_t M, int64_t N, int R, int64_t ftm, int64_t ftn) {
    const int64_t t = oracle_flag_tiles(M, N, R, ftm, ftn);
    return t < 0 ? -1 : (t + 31) / 32;
}

/* Expected ready_out after one full call: every flag tile of every non-owner
 * segment published (its bit set), the owner's own words untouched (zero),
 * padding bits zero.  words is [R][W] u32. */
int oracle_ready_out(int64_t M, int64_t N, int R, int owner, int64_t ftm, int64_t ftn,
                     uint32_t *words) {
    const int64_t tiles = oracle_flag_tiles(M, N, R, ftm, ftn);
    if (tiles < 0 || owner < 0 || owner >= R) return -1;
    const int64_t W = (tiles + 31) / 32;
    memset(words, 0, (size_t)(R * W) * sizeof(uint32_t));
    for (int d = 0; d < R; ++d) {
        if (d == owner) continue;
        for (int64_t t = 0; t < tiles; ++t) words[d * W + t / 32] |= 1u << (t % 32);
    }
    return 0;
}

/* ---- Lamport sentinel, canonicalisation, AR + RMSNorm ([P4] Approach) -------
 *
 * The staging slots are armed with the bf16 pattern of -0.0 (0x8000).  A
 * producer never stores that pattern: before the store it maps -0.0 to +0.0
 * on the final bf16 bits.  So a word still holding 0x8000 means "not arrived". */
#define LAMPORT_SENTINEL_BF16 0x8000u

void oracle_lamport_canon(const uint16_t *src, uint16_t *dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = (src[i] == LAMPORT_SENTINEL_BF16) ? 0u : src[i];
}

/* Fill a staging area with the sentinel (arming). */
void oracle_lamport_arm(uint16_t *staging, int64_t n) {
    for (int64_t i = 0; i < n; ++i) staging[i] = LAMPORT_SENTINEL_BF16;
}

/* Consumer: S partial buffers src[S][M][N] (as the producers hand them over,
 * before canonicalisation), gamma [N], out [M,N].  For each row i:
 *     s[n]  = sum_{p=0..S-1} canon(src[p][i,n])         (fp32, p ascending)
 *     ms    = (sum_{n ascending} s[n]*s[n]) / N          (fp32)
 *     r     = 1 / sqrt(ms + eps)                         (fp32, correctly rounded)
 *     out   = bf16( (s[n] * r) * gamma[n] )
 * Rows [row_begin, row_end) only.  Returns 0 or -1. */
int oracle_ar_rmsnorm(const uint16_t *src, const uint16_t *gamma, uint16_t *out, int64_t M,
                      int64_t N, int S, float eps, int64_t row_begin, int64_t row_end) {
    if (M < 0 || N < 1 || S < 1 || row_begin < 0 || row_end > M || row_begin > row_end) return -1;
    int bad = 0;
#pragma omp parallel
    {
        float *s = (float *)malloc((size_t)N * sizeof(float));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = row_begin; i < row_end; ++i) {
                for (int64_t n = 0; n < N; ++n) s[n] = 0.0f;
                for (int p = 0; p < S; ++p) {
                    const uint16_t *row = src + ((int64_t)p * M + i) * N;
                    for (int64_t n = 0; n < N; ++n) {
                        const uint16_t v = (row[n] == LAMPORT_SENTINEL_BF16) ? 0u : row[n];
                        s[n] = s[n] + bf16_to_f32(v);
                    }
                }
                float ss = 0.0f;
                for (int64_t n = 0; n < N; ++n) ss = ss + s[n] * s[n];
                const float ms = ss / (float)N;
                const float r = 1.0f / sqrtf(ms + eps);
                for (int64_t n = 0; n < N; ++n)
                    out[i * N + n] = f32_to_bf16_rne((s[n] * r) * bf16_to_f32(gamma[n]));
            }
            free(s);
        }
    }
    return bad ? -1 : 0;
}

/* ---- two-phase Lamport AR + RMSNorm ([P4] Approach: phase A, then phase B) ---
 *
 * Phase A is a reduce-scatter with cross-device stores: the [M,N] tensor is
 * cut into R parts, the rank owning a part adds the R ranks' partials of its
 * elements, rounds the sum once to bf16, maps -0.0 to +0.0 and stores the
 * result into every rank's staging.  Which rank owns which part changes no
 * value (each element's sum is the same), so once every part has landed each
 * staging holds
 *     T[i,n] = canon( bf16( sum_{r=0..R-1} x[r][i,n] ) )   (fp32, r ascending)
 * x is [R][M][N], the ranks' inputs.  Rows [row_begin, row_end) only.
 * Returns 0 or -1. */
int oracle_lamport_reduce(const uint16_t *x, uint16_t *t, int64_t M, int64_t N, int R,
                          int64_t row_begin, int64_t row_end) {
    if (M < 0 || N < 1 || R < 1 || row_begin < 0 || row_end > M || row_begin > row_end) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = row_begin; i < row_end; ++i) {
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int r = 0; r < R; ++r) acc = acc + bf16_to_f32(x[((int64_t)r * M + i) * N + n]);
            const uint16_t b = f32_to_bf16_rne(acc);
            t[i * N + n] = (b == LAMPORT_SENTINEL_BF16) ? 0u : b;
        }
    }
    return 0;
}

/* Phase B is the one-slot consumer above applied to T: per row,
 *     ms = (sum_n T^2) / N,  r = 1/sqrt(ms + eps),  out = bf16((T * r) * gamma)
 * so the two-phase result differs from the one-shot one only by the bf16
 * rounding of the sum before the norm. */
int oracle_ar_rmsnorm_2phase(const uint16_t *x, const uint16_t *gamma, uint16_t *out, int64_t M,
                             int64_t N, int R, float eps, int64_t row_begin, int64_t row_end) {
    if (M < 0 || N < 1 || R < 1 || row_begin < 0 || row_end > M || row_begin > row_end) return -1;
    const int64_t rows = row_end - row_begin;
    uint16_t *t = (uint16_t *)malloc((size_t)(rows > 0 ? rows : 1) * (size_t)N * sizeof(uint16_t));
    if (!t) return -1;
    /* T of the requested rows only, as a [rows, N] block */
    int rc = 0;
    for (int64_t i = 0; i < rows && rc == 0; ++i) {
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int r = 0; r < R; ++r) acc = acc + bf16_to_f32(x[((int64_t)r * M + row_begin + i) * N + n]);
            const uint16_t b = f32_to_bf16_rne(acc);
            t[i * N + n] = (b == LAMPORT_SENTINEL_BF16) ? 0u : b;
        }
    }
    if (rows > 0) rc = oracle_ar_rmsnorm(t, gamma, out + row_begin * N, rows, N, 1, eps, 0, rows);
    free(t);
    return rc;
}

/* ---- weighted top-k combine ([P5] description: the intranode combine) -------
 *
 * x [T][E][H] bf16 (the E expert outputs of each token, contiguous per token),
 * gate [T][E] fp32, out [T][H] bf16:
 *     out[t,h] = bf16( sum_{k=0..E-1} gate[t,k] * x[t,k,h] )    (fp32, k ascending)
 * Tokens [t_begin, t_end) only.  Returns 0 or -1. */
int oracle_combine(const uint16_t *x, const float *gate, uint16_t *out, int64_t T, int E,
                   int64_t H, int64_t t_begin, int64_t t_end) {
    if (T < 0 || E < 1 || H < 0 || t_begin < 0 || t_end > T || t_begin > t_end) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = t_begin; t < t_end; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int k = 0; k < E; ++k)
                acc = acc + gate[t * E + k] * bf16_to_f32(x[((int64_t)t * E + k) * H + h]);
            out[t * H + h] = f32_to_bf16_rne(acc);
        }
    }
    return 0;
}
