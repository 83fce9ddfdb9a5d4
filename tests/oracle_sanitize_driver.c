/*
 * oracle_sanitize_driver.c -- runs the CPU oracle (oracle/oracle.c) on jobs
 * read from stdin, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: every buffer is allocated at exactly the size
 * the call may touch, so an out-of-bounds access, a use of uninitialised
 * heap or undefined arithmetic in the oracle stops the run.  Test
 * infrastructure only (tests/test_oracle_sanitized.py builds and drives it).
 *
 * One job per line, integers in decimal (bf16 patterns as integers):
 *   sum a b                               -> bf16(a + b)
 *   row V base[V] bias[V]                 -> first argmax
 *   blk N B V sb sbi base[rows*sb] bias[rows*sbi] blk[N*B]   (buffers are
 *       allocated at (rows-1)*stride + V only; blk at N*B)   -> blk[N*B]
 *   topc C base[C] bias[C] cand[C]        -> winning id (N = 1, B = 2)
 *   gemm V R x[R] w[V*R] base[V]          -> argmax (bf16 route), argmax
 *                                            (decoded route)
 *   latent N B R H V blk[N*B] am1[N] xh[N*B*R] w1[V*R] wlat[R*R]
 *          mixl[B*B*R] wg[H*R] wu[H*R] wd[R*H]  -> out[N*(B-1)*R]
 * Each output line is the results separated by spaces.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_bf16_sum(uint16_t a, uint16_t b);
int64_t oracle_add_argmax_row(const uint16_t* base_row, const uint16_t* bias_row, int64_t V);
int oracle_add_argmax_to_blk(const uint16_t* base, const uint16_t* bias, int64_t* blk,
                             int64_t N, int64_t B, int64_t V, int64_t stride_base_r,
                             int64_t stride_bias_r);
int oracle_topc_argmax_to_blk(const uint16_t* base_c, const uint16_t* bias_c,
                              const int64_t* cand, int64_t* blk, int64_t N, int64_t B, int64_t C);
void oracle_bf16_to_double_many(const uint16_t* h, double* out, int64_t n);
int oracle_gemm_argmax_rows(const uint16_t* base, const uint16_t* x, const uint16_t* w,
                            int64_t* idx_out, int64_t r0, int64_t r1, int64_t V, int64_t R,
                            int64_t stride_base_r);
int oracle_gemm_argmax_rows_decoded(const uint16_t* base, const double* xd, const double* wd,
                                    int64_t* idx_out, int64_t r0, int64_t r1, int64_t V,
                                    int64_t R, int64_t stride_base_r);
int oracle_latent_pass(const int64_t* blk, const int64_t* am1, const uint16_t* xh,
                       const uint16_t* w1, const uint16_t* wlat, const uint16_t* mixl,
                       const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                       uint16_t* out, int64_t N, int64_t B, int64_t R, int64_t H, int64_t V,
                       double* xs, double* us, double* gs, double* vs, double* fs, double* os);

static int64_t next_int(void)
{
    long long v;
    if (scanf("%lld", &v) != 1) {
        fprintf(stderr, "driver: truncated job\n");
        exit(2);
    }
    return (int64_t)v;
}

static uint16_t* read_u16(int64_t n)
{
    uint16_t* p = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = (uint16_t)next_int();
    return p;
}

static int64_t* read_i64(int64_t n)
{
    int64_t* p = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = next_int();
    return p;
}

/* a strided [rows, stride] buffer read whole, copied into an allocation of
 * exactly (rows - 1) * stride + V elements */
static uint16_t* read_rows(int64_t rows, int64_t stride, int64_t V)
{
    uint16_t* all = read_u16(rows * stride);
    int64_t n = (rows - 1) * stride + V;
    uint16_t* p = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n);
    memcpy(p, all, sizeof(uint16_t) * (size_t)n);
    free(all);
    return p;
}

int main(void)
{
    char op[16];
    while (scanf("%15s", op) == 1) {
        if (strcmp(op, "sum") == 0) {
            uint16_t a = (uint16_t)next_int(), b = (uint16_t)next_int();
            printf("%u\n", (unsigned)oracle_bf16_sum(a, b));
        } else if (strcmp(op, "row") == 0) {
            int64_t V = next_int();
            uint16_t* a = read_u16(V);
            uint16_t* b = read_u16(V);
            printf("%lld\n", (long long)oracle_add_argmax_row(a, b, V));
            free(a);
            free(b);
        } else if (strcmp(op, "blk") == 0) {
            int64_t N = next_int(), B = next_int(), V = next_int();
            int64_t sb = next_int(), sbi = next_int();
            int64_t rows = N * (B - 1);
            uint16_t* a = read_rows(rows, sb, V);
            uint16_t* b = read_rows(rows, sbi, V);
            int64_t* blk = read_i64(N * B);
            int rc = oracle_add_argmax_to_blk(a, b, blk, N, B, V, sb, sbi);
            printf("%d", rc);
            for (int64_t i = 0; i < N * B; ++i) printf(" %lld", (long long)blk[i]);
            printf("\n");
            free(a);
            free(b);
            free(blk);
        } else if (strcmp(op, "topc") == 0) {
            int64_t C = next_int();
            uint16_t* a = read_u16(C);
            uint16_t* b = read_u16(C);
            int64_t* cand = read_i64(C);
            int64_t blk[2] = {-7, -1};
            int rc = oracle_topc_argmax_to_blk(a, b, cand, blk, 1, 2, C);
            printf("%d %lld %lld\n", rc, (long long)blk[0], (long long)blk[1]);
            free(a);
            free(b);
            free(cand);
        } else if (strcmp(op, "gemm") == 0) {
            int64_t V = next_int(), R = next_int();
            uint16_t* x = read_u16(R);
            uint16_t* w = read_u16(V * R);
            uint16_t* base = read_u16(V);
            int64_t i1 = -1, i2 = -1;
            int rc1 = oracle_gemm_argmax_rows(base, x, w, &i1, 0, 1, V, R, V);
            double* xd = (double*)malloc(sizeof(double) * (size_t)R);
            double* wd = (double*)malloc(sizeof(double) * (size_t)(V * R));
            oracle_bf16_to_double_many(x, xd, R);
            oracle_bf16_to_double_many(w, wd, V * R);
            int rc2 = oracle_gemm_argmax_rows_decoded(base, xd, wd, &i2, 0, 1, V, R, V);
            printf("%d %lld %d %lld\n", rc1, (long long)i1, rc2, (long long)i2);
            free(x);
            free(w);
            free(base);
            free(xd);
            free(wd);
        } else if (strcmp(op, "latent") == 0) {
            int64_t N = next_int(), B = next_int(), R = next_int(), H = next_int(), V = next_int();
            int64_t* blk = read_i64(N * B);
            int64_t* am1 = read_i64(N);
            uint16_t* xh = read_u16(N * B * R);
            uint16_t* w1 = read_u16(V * R);
            uint16_t* wlat = read_u16(R * R);
            uint16_t* mixl = read_u16(B * B * R);
            uint16_t* wg = read_u16(H * R);
            uint16_t* wu = read_u16(H * R);
            uint16_t* wd = read_u16(R * H);
            int64_t nout = N * (B - 1) * R;
            uint16_t* out = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(nout > 0 ? nout : 1));
            int rc = oracle_latent_pass(blk, am1, xh, w1, wlat, mixl, wg, wu, wd, out, N, B, R,
                                        H, V, NULL, NULL, NULL, NULL, NULL, NULL);
            printf("%d", rc);
            for (int64_t i = 0; rc == 0 && i < nout; ++i) printf(" %u", (unsigned)out[i]);
            printf("\n");
            free(blk);
            free(am1);
            free(xh);
            free(w1);
            free(wlat);
            free(mixl);
            free(wg);
            free(wu);
            free(wd);
            free(out);
        } else {
            fprintf(stderr, "driver: unknown job %s\n", op);
            return 2;
        }
        fflush(stdout);
    }
    return 0;
}
