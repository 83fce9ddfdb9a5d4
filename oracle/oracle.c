/*
 * oracle.c -- plain, slow CPU oracle for the fused add + argmax readout.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package
 * smoke check and the benchmark's CPU-baseline leg may load this library.  It
 * shares no code, header, table or helper with the GPU library: the GPU path
 * never includes, links or calls it, and it never calls the GPU path.
 *
 * What it computes (XPress kernels page, "fused_add_argmax_to_blk" and the two
 * stage kernels "_xpress_add_argmax_partial_kernel" and
 * "_xpress_add_argmax_reduce_to_blk_kernel"):
 *
 *   for every draft row r = n*(B-1) + b   (0 <= n < N, 0 <= b < B-1)
 *     s_v = bf16( base[r, v] + bias[r, v] ),  v = 0 .. V-1
 *     blk[n, 1 + b] = lowest v with s_v == max_u s_u
 *   blk[n, 0] (the verified anchor) and every other byte are left alone.
 *
 * Readings where the pages leave a step open (each one is listed with its
 * reason in the design notes):
 *   - the sum is the exact sum of the two bf16 values rounded once to bf16
 *     with round-to-nearest, ties-to-even (the stage-1 kernel rounds the sum to
 *     the input dtype; the top-C kernel widens to fp32 first and says the
 *     full-vocab path does the same).  Here the sum is formed in binary64 and
 *     then rounded to bf16 by an explicit integer-grid rounding written below.
 *     binary64 carries 53 >= 2*8+2 significant bits, so rounding first to
 *     binary64 and then to bf16 gives the same bf16 as rounding the exact sum
 *     once (the double-rounding innocuity bound for addition);
 *   - subnormal bf16 values are kept, never flushed;
 *   - values compare as real numbers: -0 equals +0;
 *   - on equal maxima the lowest vocabulary index wins (what an argmax over
 *     the chunk followed by a strict ">" scan over chunks in ascending order
 *     yields);
 *   - NaN inputs are outside the contract; a NaN sum never wins here, at any
 *     position: the scan starts from -inf at index 0 and takes only a
 *     strictly greater value, so a row of NaN and -inf sums reports index 0.
 *
 * Everything is single-threaded and unvectorised on purpose.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* ---------------------------------------------------------------------------
 * bf16 decoding, from the field definition.
 *
 * A bf16 is 1 sign bit, 8 exponent bits (bias 127) and 7 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-133   (2^-126 * f/128)
 *   exponent 1..254 : normal,    value = (128 + fraction) * 2^(e - 127 - 7)
 *   exponent 255    : infinity (fraction 0) or NaN.
 * Every bf16 value is exactly representable in binary64.
 * ------------------------------------------------------------------------- */
double oracle_bf16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xFF;
    int f = h & 0x7F;
    double mag;
    if (e == 0xFF) {
        mag = (f == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        mag = ldexp((double)f, -133);
    } else {
        mag = ldexp((double)(128 + f), e - 127 - 7);
    }
    return sign ? -mag : mag;
}

/* ---------------------------------------------------------------------------
 * Round a binary64 value to the nearest bf16, ties to even (IEEE 754
 * roundTiesToEven), keeping subnormals and overflowing to infinity.
 *
 * The bf16 values in the binade [2^k, 2^(k+1)) (k >= -126) are the integer
 * multiples of the quantum q = 2^(k-7); below 2^-126 the quantum stays at
 * 2^-133 (the subnormal range).  So: pick q, scale x by 1/q (exact, q is a
 * power of two), round that real number to an integer with ties going to the
 * even integer, scale back.  A result of magnitude >= 2^128 is infinity
 * (the value rounded as if the exponent were unbounded exceeds the largest
 * finite bf16).
 * ------------------------------------------------------------------------- */
uint16_t oracle_bf16_from_double(double x)
{
    if (isnan(x)) {
        return 0x7FC0; /* a quiet NaN; outside the contract */
    }
    uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    double a = fabs(x);
    if (a == 0.0) {
        return sign; /* +0 or -0 as given */
    }
    if (isinf(a)) {
        return sign | 0x7F80;
    }
    int e2;
    (void)frexp(a, &e2);  /* a = m * 2^e2, m in [0.5, 1) */
    int k = e2 - 1;       /* a in [2^k, 2^(k+1)) */
    if (k > 127) {
        return sign | 0x7F80; /* at least 2^128: beyond every finite bf16 */
    }
    if (k < -126) {
        k = -126; /* subnormal range shares the smallest normal quantum */
    }
    double scaled = ldexp(a, 7 - k); /* a / q, exact */
    double lo = floor(scaled);
    double frac = scaled - lo;       /* exact: scaled < 2^53 */
    double m = lo;
    if (frac > 0.5) {
        m = lo + 1.0;
    } else if (frac == 0.5) {
        /* halfway: take the even neighbour */
        m = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;
    }
    /* m is an integer in [0, 256]: 256 means the value rounded up into the
     * next binade, whose significand is 128 with the exponent one higher. */
    if (m >= 256.0) {
        m = 128.0;
        k += 1;
    }
    if (m == 0.0) {
        return sign; /* cannot happen for a nonzero sum of bf16s; kept total */
    }
    if (m < 128.0) {
        /* only possible at k == -126: a subnormal, exponent field 0 */
        return sign | (uint16_t)m;
    }
    int efield = k + 127;
    if (efield >= 0xFF) {
        return sign | 0x7F80; /* overflow to infinity */
    }
    return sign | (uint16_t)(efield << 7) | (uint16_t)((int)m - 128);
}

/* Element-wise oracle_bf16_from_double over n values. */
void oracle_bf16_from_double_many(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        out[i] = oracle_bf16_from_double(x[i]);
    }
}

/* The rounded sum of one pair: bf16(a + b), formed in binary64. */
uint16_t oracle_bf16_sum(uint16_t a, uint16_t b)
{
    double s = oracle_bf16_to_double(a) + oracle_bf16_to_double(b);
    return oracle_bf16_from_double(s);
}

/* Element-wise rounded sums of n pairs (used by the pins on the oracle). */
void oracle_bf16_sum_many(const uint16_t* a, const uint16_t* b, uint16_t* out,
                          int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        out[i] = oracle_bf16_sum(a[i], b[i]);
    }
}

/* All rounded sums a_vals[i] + b for every one of the 65536 bf16 patterns b:
 * out[i * 65536 + b].  Used for the exhaustive pin of the element rounding. */
void oracle_bf16_sum_grid(const uint16_t* a_vals, int64_t n_a, uint16_t* out)
{
    for (int64_t i = 0; i < n_a; ++i) {
        for (int64_t b = 0; b < 65536; ++b) {
            out[i * 65536 + b] = oracle_bf16_sum(a_vals[i], (uint16_t)b);
        }
    }
}

/* Argmax of one row: the lowest v whose rounded sum equals the row maximum.
 * The scan runs v = 0 .. V-1 from the incumbent (-inf, index 0) and replaces
 * it only on a strictly greater value, which is exactly "first maximum"; a
 * NaN sum compares false and never replaces it.  V >= 1. */
int64_t oracle_add_argmax_row(const uint16_t* base_row, const uint16_t* bias_row,
                              int64_t V)
{
    int64_t best_v = 0;
    double best = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        double s = oracle_bf16_to_double(oracle_bf16_sum(base_row[v], bias_row[v]));
        if (s > best) {
            best = s;
            best_v = v;
        }
    }
    return best_v;
}

/* The whole readout on host buffers.
 *   base, bias : bf16 bit patterns, N*(B-1) rows, row strides in elements
 *   blk        : int64 [N, B] row-major; blk[n*B + 1 + b] is written for
 *                every row r = n*(B-1) + b; slot 0 is never touched.
 * Returns 0, or -1 on arguments that describe no valid layout. */
int oracle_add_argmax_to_blk(const uint16_t* base, const uint16_t* bias,
                             int64_t* blk, int64_t N, int64_t B, int64_t V,
                             int64_t stride_base_r, int64_t stride_bias_r)
{
    if (N < 0 || B < 1 || V < 1 || stride_base_r < V || stride_bias_r < V) {
        return -1;
    }
    int64_t rows = N * (B - 1);
    for (int64_t r = 0; r < rows; ++r) {
        int64_t n = r / (B - 1);
        int64_t b = r % (B - 1);
        blk[n * B + 1 + b] = oracle_add_argmax_row(base + r * stride_base_r,
                                                   bias + r * stride_bias_r, V);
    }
    return 0;
}

/* Rows [r0, r1) only, writing idx_out[r - r0]; lets a caller spread a large
 * workload over several host threads without changing the arithmetic. */
int oracle_add_argmax_rows(const uint16_t* base, const uint16_t* bias,
                           int64_t* idx_out, int64_t r0, int64_t r1, int64_t V,
                           int64_t stride_base_r, int64_t stride_bias_r)
{
    if (r0 < 0 || r1 < r0 || V < 1 || stride_base_r < V || stride_bias_r < V) {
        return -1;
    }
    for (int64_t r = r0; r < r1; ++r) {
        idx_out[r - r0] = oracle_add_argmax_row(base + r * stride_base_r,
                                                bias + r * stride_bias_r, V);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Top-C readout (XPress kernels page, "_xpress_topc_argmax_to_blk_kernel" and
 * "fused_topc_argmax_to_blk"): each draft row r = n*(B-1) + j carries C
 * candidates -- their base logits base_c[r, c], refiner bias bias_c[r, c]
 * and vocabulary ids cand[r, c], all three [N, B-1, C] contiguous.  The
 * winner is the first c maximising bf16(base_c + bias_c) (the same element
 * rule and tie rule as the full-vocabulary readout), and its id is written
 * to blk[n, 1 + j]:
 *     blk[n*B + 1 + j] = cand[r*C + first_argmax_c]
 * Slot 0 and all other memory are untouched.  Returns 0, or -1 on sizes that
 * describe no valid layout.
 * ------------------------------------------------------------------------- */
int oracle_topc_argmax_to_blk(const uint16_t* base_c, const uint16_t* bias_c,
                              const int64_t* cand, int64_t* blk, int64_t N,
                              int64_t B, int64_t C)
{
    if (N < 0 || B < 1 || C < 1) {
        return -1;
    }
    int64_t rows = N * (B - 1);
    for (int64_t r = 0; r < rows; ++r) {
        int64_t n = r / (B - 1);
        int64_t j = r % (B - 1);
        int64_t best = oracle_add_argmax_row(base_c + r * C, bias_c + r * C, C);
        blk[n * B + 1 + j] = cand[r * C + best];
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Readout with the refiner bias computed in place (XPress kernels page,
 * module description: logits = base + x @ W2, the readout matmul, followed by
 * the argmax; the fused add + argmax consumes its bf16 result as bias):
 *
 *   bias[r, v] = bf16( sum_k x[r, k] * w[v, k] )      (the matmul's bf16 output)
 *   s[r, v]    = bf16( base[r, v] + bias[r, v] )
 *   blk[n, 1 + b] = first argmax_v s[r, v],   r = n*(B-1) + b
 *
 * x is [rows, R] and w is [V, R] (the head weight, one row per vocabulary id),
 * both bf16 and row-major; base has row stride stride_base_r.  Reading: the
 * dot product is the exact real sum rounded once to bf16 (the matmul
 * accumulates in fp32 and rounds its output to bf16; the exact value is its
 * plain definition).  Here each product of two bf16 values is exact in
 * binary64 and the sum is formed in binary64, which is exact for the
 * dyadic test inputs and within 2^-53 relative of the exact sum otherwise.
 * ------------------------------------------------------------------------- */
uint16_t oracle_dot_bf16(const uint16_t* x_row, const uint16_t* w_row, int64_t R)
{
    double acc = 0.0;
    for (int64_t k = 0; k < R; ++k) {
        acc += oracle_bf16_to_double(x_row[k]) * oracle_bf16_to_double(w_row[k]);
    }
    return oracle_bf16_from_double(acc);
}

/* Element-wise bf16 decoding of n patterns into binary64. */
void oracle_bf16_to_double_many(const uint16_t* h, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        out[i] = oracle_bf16_to_double(h[i]);
    }
}

/* First argmax of bf16(base + bf16(x_row . w[v])) over v = 0 .. V-1, with
 * x_row [R] and w [V, R] given decoded to binary64 (oracle_bf16_to_double:
 * every bf16 value is exact there, so decoding once is a change of storage,
 * not of the arithmetic).  Each product of two bf16 values is exact in
 * binary64; the sum over k runs in order k = 0 .. R-1 and is rounded once
 * to bf16 (the matmul's bf16 output), then added to base and rounded again.
 * The incumbent starts at (-inf, index 0) and only a strictly greater value
 * replaces it, as in the readout above. */
static int64_t gemm_scan_row(const uint16_t* base_row, const double* x_row,
                             const double* w, int64_t V, int64_t R)
{
    int64_t best_v = 0;
    double best = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        const double* wv = w + v * R;
        double acc = 0.0;
        for (int64_t k = 0; k < R; ++k) {
            acc += x_row[k] * wv[k];
        }
        uint16_t bias = oracle_bf16_from_double(acc);
        double sum = oracle_bf16_to_double(oracle_bf16_sum(base_row[v], bias));
        if (sum > best) {
            best = sum;
            best_v = v;
        }
    }
    return best_v;
}

/* Rows [r0, r1) on decoded operands: xd [rows, R] and wd [V, R] binary64
 * (oracle_bf16_to_double_many of x and w); idx_out[r - r0] = first argmax
 * of row r. */
int oracle_gemm_argmax_rows_decoded(const uint16_t* base, const double* xd, const double* wd,
                                    int64_t* idx_out, int64_t r0, int64_t r1, int64_t V,
                                    int64_t R, int64_t stride_base_r)
{
    if (r0 < 0 || r1 < r0 || V < 1 || R < 1 || stride_base_r < V) {
        return -1;
    }
    for (int64_t r = r0; r < r1; ++r) {
        idx_out[r - r0] = gemm_scan_row(base + r * stride_base_r, xd + r * R, wd, V, R);
    }
    return 0;
}

/* Rows [r0, r1) on bf16 operands: decodes x's rows r0 .. r1-1 and all of w,
 * then scans each row.  Returns 0, -1 on invalid sizes, -2 when out of host
 * memory. */
int oracle_gemm_argmax_rows(const uint16_t* base, const uint16_t* x, const uint16_t* w,
                            int64_t* idx_out, int64_t r0, int64_t r1, int64_t V,
                            int64_t R, int64_t stride_base_r)
{
    if (r0 < 0 || r1 < r0 || V < 1 || R < 1 || stride_base_r < V) {
        return -1;
    }
    double* wd = (double*)malloc(sizeof(double) * (size_t)(V * R));
    double* xd = (double*)malloc(sizeof(double) * (size_t)((r1 - r0) * R + 1));
    if (!wd || !xd) {
        free(wd);
        free(xd);
        return -2;
    }
    oracle_bf16_to_double_many(w, wd, V * R);
    oracle_bf16_to_double_many(x + r0 * R, xd, (r1 - r0) * R);
    int rc = oracle_gemm_argmax_rows_decoded(base + r0 * stride_base_r, xd, wd, idx_out, 0,
                                             r1 - r0, V, R, stride_base_r);
    free(wd);
    free(xd);
    return rc;
}

/* ---------------------------------------------------------------------------
 * Latent stage of one Jacobi pass (XPress kernels page, module description and
 * "_xpress_latent_kernel", both revisions): for every block n and slot b < B,
 * with R latent channels and an MLP of H hidden units,
 *
 *   prev[b]  = am1[n] for b = 0, blk[n, b-1] otherwise   (previous slot's token)
 *   x[b, r]  = xh[n, b, r] + sum_k w1[prev[b], k] * wlat[r, k]
 *   u[b, r]  = sum_j mixl[b, j, r] * x[j, r]               (folded causal mixer)
 *   g[b, h]  = sum_r bf16(u[b, r]) * wg[h, r]
 *   v[b, h]  = sum_r bf16(u[b, r]) * wu[h, r]
 *   f[b, h]  = g * sigmoid(g) * v                          (SwiGLU)
 *   o[b, r]  = u[b, r] + sum_h bf16(f[b, h]) * wd[r, h]    (MLP with residual)
 *   out[n, b-1, r] = bf16(o[b, r]),  b = 1 .. B-1
 *
 * All tensors are bf16 bit patterns except blk / am1 (int64).  Weight layouts
 * are out-major (one row per output unit): wlat [R, R], wg / wu [H, R],
 * wd [R, H]; mixl is [B, B, R] (zero above the diagonal for a causal mixer, but
 * every j < B is summed, as the page's mixer loop does); xh is [N, B, R]; w1 is
 * [V, R]; out is [N, B-1, R].  Slot 0 is the anchor: its x feeds the mixer of
 * the later slots but no latent is written for it.
 *
 * Reading: the page's kernel keeps x, u, g, v and the residual sum in fp32 and
 * rounds to bf16 at exactly three places: u before the MLP, the SwiGLU product
 * before the down projection, and the output.  The plain definition of each
 * fp32 quantity is its exact real value; here it is formed in binary64 (every
 * product of two bf16 values is exact there) and the sigmoid is the C
 * library's exp.
 *
 * Optional outputs (NULL to skip), binary64 before any rounding:
 *   xs [N, B, R], us [N, B, R], gs / vs / fs [N, B-1, H], os [N, B-1, R].
 * Returns 0, -1 on invalid sizes or a token id outside [0, V), -2 when out of
 * host memory.
 * ------------------------------------------------------------------------- */
int oracle_latent_pass(const int64_t* blk, const int64_t* am1, const uint16_t* xh,
                       const uint16_t* w1, const uint16_t* wlat, const uint16_t* mixl,
                       const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                       uint16_t* out, int64_t N, int64_t B, int64_t R, int64_t H,
                       int64_t V, double* xs, double* us, double* gs, double* vs,
                       double* fs, double* os)
{
    if (N < 0 || B < 2 || R < 1 || H < 1 || V < 1) {
        return -1;
    }
    /* the weights decoded to binary64 once (a change of storage, not of the
       arithmetic below) */
    double* dlat = (double*)malloc(sizeof(double) * (size_t)(R * R));
    double* dmix = (double*)malloc(sizeof(double) * (size_t)(B * B * R));
    double* dg = (double*)malloc(sizeof(double) * (size_t)(H * R));
    double* du = (double*)malloc(sizeof(double) * (size_t)(H * R));
    double* dd = (double*)malloc(sizeof(double) * (size_t)(R * H));
    double* emb = (double*)malloc(sizeof(double) * (size_t)R);
    double* x = (double*)malloc(sizeof(double) * (size_t)(B * R));
    double* u = (double*)malloc(sizeof(double) * (size_t)(B * R));
    double* ub = (double*)malloc(sizeof(double) * (size_t)R);
    double* m = (double*)malloc(sizeof(double) * (size_t)H);
    int rc = 0;
    if (!dlat || !dmix || !dg || !du || !dd || !emb || !x || !u || !ub || !m) {
        rc = -2;
        goto done;
    }
    for (int64_t i = 0; i < R * R; ++i) dlat[i] = oracle_bf16_to_double(wlat[i]);
    for (int64_t i = 0; i < B * B * R; ++i) dmix[i] = oracle_bf16_to_double(mixl[i]);
    for (int64_t i = 0; i < H * R; ++i) {
        dg[i] = oracle_bf16_to_double(wg[i]);
        du[i] = oracle_bf16_to_double(wu[i]);
        dd[i] = oracle_bf16_to_double(wd[i]);
    }
    for (int64_t n = 0; n < N; ++n) {
        /* embedding of the previous slot's token, projected, plus the cache */
        for (int64_t b = 0; b < B; ++b) {
            int64_t tok = (b == 0) ? am1[n] : blk[n * B + b - 1];
            if (tok < 0 || tok >= V) {
                rc = -1;
                goto done;
            }
            for (int64_t k = 0; k < R; ++k) {
                emb[k] = oracle_bf16_to_double(w1[tok * R + k]);
            }
            for (int64_t r = 0; r < R; ++r) {
                double acc = oracle_bf16_to_double(xh[(n * B + b) * R + r]);
                for (int64_t k = 0; k < R; ++k) {
                    acc += emb[k] * dlat[r * R + k];
                }
                x[b * R + r] = acc;
            }
        }
        /* folded causal mixer, per channel */
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t r = 0; r < R; ++r) {
                double acc = 0.0;
                for (int64_t j = 0; j < B; ++j) {
                    acc += dmix[(b * B + j) * R + r] * x[j * R + r];
                }
                u[b * R + r] = acc;
            }
        }
        if (xs != NULL || us != NULL) {
            for (int64_t i = 0; i < B * R; ++i) {
                if (xs != NULL) xs[n * B * R + i] = x[i];
                if (us != NULL) us[n * B * R + i] = u[i];
            }
        }
        /* SwiGLU MLP with residual, for the slots that are read out */
        for (int64_t b = 1; b < B; ++b) {
            int64_t row = n * (B - 1) + b - 1;
            for (int64_t r = 0; r < R; ++r) {
                ub[r] = oracle_bf16_to_double(oracle_bf16_from_double(u[b * R + r]));
            }
            for (int64_t h = 0; h < H; ++h) {
                double g = 0.0, v = 0.0;
                for (int64_t r = 0; r < R; ++r) {
                    g += ub[r] * dg[h * R + r];
                    v += ub[r] * du[h * R + r];
                }
                double f = g / (1.0 + exp(-g)) * v;
                m[h] = oracle_bf16_to_double(oracle_bf16_from_double(f));
                if (gs != NULL) gs[row * H + h] = g;
                if (vs != NULL) vs[row * H + h] = v;
                if (fs != NULL) fs[row * H + h] = f;
            }
            for (int64_t r = 0; r < R; ++r) {
                double acc = u[b * R + r];
                for (int64_t h = 0; h < H; ++h) {
                    acc += m[h] * dd[r * H + h];
                }
                if (os != NULL) os[row * R + r] = acc;
                out[row * R + r] = oracle_bf16_from_double(acc);
            }
        }
    }
done:
    free(dlat);
    free(dmix);
    free(dg);
    free(du);
    free(dd);
    free(emb);
    free(x);
    free(u);
    free(ub);
    free(m);
    return rc;
}
