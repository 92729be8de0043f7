/*
 * The fp64 oracle's entry points on small seeded inputs, for a build with the
 * host sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer).  Every input
 * and output goes to the file named by argv[1] as records
 *     int64 count, int32 kind (0 = float32, 1 = float64, 2 = int64), data
 * so that the test can rerun the plain oracle build on the same inputs and
 * compare.  Also checks that bad sizes are refused.  Exit status 0 = done.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_run(int64_t n_seq, const int64_t *row0, const int64_t *len, int64_t row_step,
                   int64_t H, int64_t dk, int64_t dv, const float *q, const float *k,
                   const float *v, const float *beta, const float *log_alpha, const double *s0,
                   double *o, double *o_mag, double *s_final, int n_threads);
int kda_oracle_backward(int64_t n_seq, const int64_t *row0, const int64_t *len, int64_t row_step,
                        int64_t H, int64_t dk, int64_t dv, const float *q, const float *k,
                        const float *v, const float *beta, const float *log_alpha,
                        const double *s0, const double *d_o, const double *d_sT, double *dq,
                        double *dkk, double *dvv, double *dbeta, double *dla, double *ds0,
                        int n_threads);
int kda_oracle_prepare(int64_t rows, int64_t H, int64_t dk, const float *q_raw, const float *k_raw,
                       const float *b_raw, const float *a_raw, int round, float *q, float *k,
                       float *beta, float *log_alpha);

static FILE *out;
static uint64_t rng = 0x9e3779b97f4a7c15ull;

static double uniform(void) /* [0, 1) */
{
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng >> 11) / 9007199254740992.0;
}

static void put(const void *p, int64_t count, int32_t kind)
{
    const size_t size = kind == 0 ? 4 : 8;
    fwrite(&count, 8, 1, out);
    fwrite(&kind, 4, 1, out);
    if (count > 0) fwrite(p, size, (size_t)count, out);
}

static float *floats(int64_t n, double lo, double hi)
{
    float *x = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i) x[i] = (float)(lo + (hi - lo) * uniform());
    return x;
}

static double *doubles(int64_t n, double lo, double hi)
{
    double *x = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * uniform();
    return x;
}

#define CHECK(cond)                                                                \
    do {                                                                           \
        if (!(cond)) {                                                             \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);     \
            return 1;                                                              \
        }                                                                          \
    } while (0)

/* packed sequences of the given lengths, rows one after another */
static int packed_case(int64_t n_seq, const int64_t *len, int64_t H, int64_t dk, int64_t dv,
                       int with_state, int with_mag, int threads)
{
    int64_t *row0 = (int64_t *)malloc((size_t)n_seq * 8), rows = 0;
    for (int64_t n = 0; n < n_seq; ++n) {
        row0[n] = rows;
        rows += len[n];
    }
    float *q = floats(rows * H * dk, -0.3, 0.3), *k = floats(rows * H * dk, -0.3, 0.3);
    float *v = floats(rows * H * dv, -1.0, 1.0), *beta = floats(rows * H, 0.05, 0.95);
    float *la = floats(rows * H * dk, -2.0, 0.0);
    double *s0 = with_state ? doubles(n_seq * H * dk * dv, -0.5, 0.5) : NULL;
    double *d_o = doubles(rows * H * dv, -1.0, 1.0), *d_sT = doubles(n_seq * H * dk * dv, -0.2, 0.2);
    double *o = doubles(rows * H * dv, 0.0, 0.0), *mag = with_mag ? doubles(rows * H * dv, 0.0, 0.0) : NULL;
    double *s1 = doubles(n_seq * H * dk * dv, 0.0, 0.0);
    CHECK(kda_oracle_run(n_seq, row0, len, 1, H, dk, dv, q, k, v, beta, la, s0, o, mag, s1, threads) == 0);
    double *dq = doubles(rows * H * dk, 0, 0), *dk_ = doubles(rows * H * dk, 0, 0);
    double *dv_ = doubles(rows * H * dv, 0, 0), *db = doubles(rows * H, 0, 0);
    double *dla = doubles(rows * H * dk, 0, 0), *ds0 = doubles(n_seq * H * dk * dv, 0, 0);
    CHECK(kda_oracle_backward(n_seq, row0, len, 1, H, dk, dv, q, k, v, beta, la, s0, d_o, d_sT, dq,
                              dk_, dv_, db, dla, ds0, threads) == 0);
    const int64_t dims[5] = {n_seq, rows, H, dk, dv};
    put(dims, 5, 2);
    put(len, n_seq, 2);
    put(q, rows * H * dk, 0);
    put(k, rows * H * dk, 0);
    put(v, rows * H * dv, 0);
    put(beta, rows * H, 0);
    put(la, rows * H * dk, 0);
    put(s0, with_state ? n_seq * H * dk * dv : 0, 1);
    put(d_o, rows * H * dv, 1);
    put(d_sT, n_seq * H * dk * dv, 1);
    put(o, rows * H * dv, 1);
    put(mag, with_mag ? rows * H * dv : 0, 1);
    put(s1, n_seq * H * dk * dv, 1);
    put(dq, rows * H * dk, 1);
    put(dk_, rows * H * dk, 1);
    put(dv_, rows * H * dv, 1);
    put(db, rows * H, 1);
    put(dla, rows * H * dk, 1);
    put(ds0, n_seq * H * dk * dv, 1);
    free(row0); free(q); free(k); free(v); free(beta); free(la); free(s0); free(d_o); free(d_sT);
    free(o); free(mag); free(s1); free(dq); free(dk_); free(dv_); free(db); free(dla); free(ds0);
    return 0;
}

static int prepare_case(int64_t rows, int64_t H, int64_t dk)
{
    float *qr = floats(rows * H * dk, -2, 2), *kr = floats(rows * H * dk, -2, 2);
    float *br = floats(rows * H, -6, 6), *ar = floats(rows * H * dk, -30, 30);
    memset(qr, 0, (size_t)dk * sizeof(float)); /* a zero vector stays zero */
    float *q = floats(rows * H * dk, 0, 0), *k = floats(rows * H * dk, 0, 0);
    float *b = floats(rows * H, 0, 0), *la = floats(rows * H * dk, 0, 0);
    CHECK(kda_oracle_prepare(rows, H, dk, qr, kr, br, ar, 1, q, k, b, la) == 0);
    const int64_t dims[3] = {rows, H, dk};
    put(dims, 3, 2);
    put(qr, rows * H * dk, 0);
    put(kr, rows * H * dk, 0);
    put(br, rows * H, 0);
    put(ar, rows * H * dk, 0);
    put(q, rows * H * dk, 0);
    put(k, rows * H * dk, 0);
    put(b, rows * H, 0);
    put(la, rows * H * dk, 0);
    free(qr); free(kr); free(br); free(ar); free(q); free(k); free(b); free(la);
    return 0;
}

int main(int argc, char **argv)
{
    if (argc != 2) return 2;
    out = fopen(argv[1], "wb");
    if (!out) return 2;
    const int64_t mixed[5] = {0, 1, 70, 5, 129};
    const int64_t one[1] = {3};
    const int64_t none[2] = {0, 0};
    if (packed_case(5, mixed, 2, 16, 12, 1, 1, 3)) return 1;
    if (packed_case(1, one, 1, 128, 128, 0, 0, 1)) return 1;
    if (packed_case(2, none, 2, 8, 8, 1, 1, 2)) return 1;
    if (prepare_case(7, 3, 16)) return 1;
    /* refused sizes */
    const int64_t bad_len[1] = {-1}, row0[1] = {0};
    float f = 0.f;
    double d = 0.0;
    CHECK(kda_oracle_run(-1, row0, one, 1, 1, 1, 1, &f, &f, &f, &f, &f, NULL, &d, NULL, &d, 1) == -1);
    CHECK(kda_oracle_run(1, row0, bad_len, 1, 1, 1, 1, &f, &f, &f, &f, &f, NULL, &d, NULL, &d, 1) == -1);
    CHECK(kda_oracle_run(1, row0, one, 1, 0, 1, 1, &f, &f, &f, &f, &f, NULL, &d, NULL, &d, 1) == -1);
    CHECK(kda_oracle_backward(1, row0, bad_len, 1, 1, 1, 1, &f, &f, &f, &f, &f, NULL, &d, NULL, &d,
                              &d, &d, &d, &d, NULL, 1) == -1);
    CHECK(kda_oracle_prepare(-1, 1, 1, &f, &f, &f, &f, 1, &f, &f, &f, &f) == -1);
    fclose(out);
    printf("oracle driver done\n");
    return 0;
}
