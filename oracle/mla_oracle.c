/*
 * mla_oracle.c -- plain, slow fp64 CPU reference for paged MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header, table
 * or helper with the GPU path.
 *
 * What it computes (the plain definition; no blocking, fusion or reordering):
 *
 *   Multi-head latent attention decode over a paged latent cache, as released
 *   in "DeepSeek publica FlashMLA como codigo abierto" (release bullets: MLA
 *   decoding kernel, BF16, paged KV cache with block size 64, variable
 *   sequence lengths).  Every cached token is one latent row of d_qk bf16
 *   values (512 compressed dims followed by 64 rope dims).  All h_q query
 *   heads read the same row: the key is the whole row, the value is its
 *   first d_v entries.  Token j of sequence b lives in physical page
 *   block_table[b][j / page], row j % page.
 *
 *   For every sequence b, query i < s_q and head h:
 *     L      = n_b                      (no mask)
 *            = n_b - s_q + 1 + i        (causal: query i sits at absolute
 *                                        position n_b - s_q + i and sees keys
 *                                        up to and including that position)
 *     s_j    = scale * sum_d q[b,i,h,d] * k_j[d]            for j < L
 *     m      = max_j s_j,   w_j = exp(s_j - m),   l = sum_j w_j
 *     out    = (sum_j w_j * k_j[0:d_v]) / l
 *     lse    = m + ln(l)
 *   An empty key set gives out = 0 and lse = -inf (the log of an empty sum).
 *
 *   Split-KV merge (used to check partial results): each contiguous key range
 *   r of a row has its own (o_r, lse_r) from the formula above; with
 *   M = max_r lse_r, lse = M + ln(sum_r exp(lse_r - M)) and
 *   out = sum_r exp(lse_r - lse) * o_r.  All-empty gives out 0, lse -inf.
 *
 *   Absorption bmm ("[Attention] MLA get rid of materialization", PR
 *   description: the absorbed W_Q_UK / W_UV_O products are not materialized;
 *   the up-projections are applied as sequential batched matmuls instead):
 *     y[b,h,n] = sum_k x[b,h,k] * W[h,k,n]
 *
 *   FP8 weights for the absorption bmm (the same PR description: weights
 *   stored in fp8 are decompressed to 16-bit floats before the bmm, since no
 *   fp8 bmm is used).  The pages fix neither the fp8 format nor the scale
 *   granularity; the reading taken here: OCP FP8 E4M3 codes (sign, 4-bit
 *   exponent with bias 7, 3-bit mantissa; exponent field 0 holds the
 *   subnormals m * 2^-9; S.1111.111 is NaN; no infinities) with one fp32
 *   scale per 128 x 128 block of each head's K x N matrix, decompressed as
 *     W[h,k,n] = bf16( e4m3(code[h,k,n]) * scale[h, k / 128, n / 128] )
 *   where the product is exact and bf16() rounds it once, to nearest even.
 *
 *   Materialized absorbed weights (the products the same PR description
 *   decides not to precompute; the fp64 products themselves are formed in
 *   oracle/materialize.py) are stored as bf16: oracle_round_bf16_array
 *   rounds each fp64 value once, to nearest even.
 *
 * Precision: inputs that are bf16 in the product (cache rows, weights) are
 * passed as raw bf16 bit patterns and widened exactly to fp64 here;
 * activations are passed as fp64.  All arithmetic is fp64 and nothing is
 * rounded on the way out.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC mla_oracle.c -o liboracle.so -lm
 * (no -ffast-math: IEEE semantics are part of the definition).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* Exact widening of a bf16 bit pattern: it is the top half of an fp32. */
static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int oracle_max_threads(void) { return omp_get_max_threads(); }

/* Number of keys query i of a sequence of length n may see. */
static int64_t visible_keys(int64_t n, int s_q, int i, int causal)
{
    int64_t L = causal ? n - s_q + 1 + i : n;
    return L < 0 ? 0 : L;
}

/*
 * Attention of every (b, i, h) row over the keys j with
 * key_begin[b] <= j < min(key_end[b], L) (L as above).  Passing NULL for
 * key_begin / key_end means 0 / n_b, i.e. the full decode.
 *
 *   q           fp64 [batch][s_q][h_q][d_qk]
 *   kv_cache    bf16 bits [num_pages][page][d_qk]
 *   block_table int32 [batch][bt_stride]
 *   seqlens     int32 [batch]
 *   out         fp64 [batch][s_q][h_q][d_v]
 *   lse         fp64 [batch][s_q][h_q]
 *
 * Returns 0, or -1 if a needed block-table entry is outside [0, num_pages)
 * or a length is negative or beyond the block table (nothing is read then
 * for that row; the caller treats any nonzero return as a failed check).
 */
int oracle_attend(const double *q, const uint16_t *kv_cache, int64_t num_pages,
                  const int32_t *block_table, int64_t bt_stride,
                  const int32_t *seqlens, int batch, int s_q, int h_q,
                  int d_qk, int d_v, int page, float scale, int causal,
                  const int64_t *key_begin, const int64_t *key_end,
                  double *out, double *lse)
{
    const double scale64 = (double)scale;
    const int64_t rows = (int64_t)batch * s_q * h_q;
    int err = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t r = 0; r < rows; ++r) {
        const int b = (int)(r / ((int64_t)s_q * h_q));
        const int i = (int)((r / h_q) % s_q);
        const int64_t n = seqlens[b];
        const double *qrow = q + r * d_qk;
        double *orow = out + r * d_v;

        int64_t lo = key_begin ? key_begin[b] : 0;
        int64_t hi = key_end ? key_end[b] : n;
        const int64_t L = visible_keys(n, s_q, i, causal);
        if (hi > L) hi = L;
        if (lo < 0) lo = 0;

        for (int e = 0; e < d_v; ++e) orow[e] = 0.0;
        lse[r] = -INFINITY;
        if (n < 0 || n > bt_stride * (int64_t)page) { err |= 1; continue; }
        if (hi <= lo) continue;

        /* pointers to the key rows of this row's key range */
        const int64_t cnt = hi - lo;
        const uint16_t **krow = (const uint16_t **)malloc((size_t)cnt * sizeof *krow);
        double *s = (double *)malloc((size_t)cnt * sizeof *s);
        int bad = 0;
        for (int64_t t = 0; t < cnt; ++t) {
            const int64_t j = lo + t;
            const int64_t phys = block_table[(int64_t)b * bt_stride + j / page];
            if (phys < 0 || phys >= num_pages) { bad = 1; break; }
            krow[t] = kv_cache + (phys * page + j % page) * d_qk;
        }
        if (bad) { free(krow); free(s); err |= 1; continue; }

        /* logits */
        for (int64_t t = 0; t < cnt; ++t) {
            double dot = 0.0;
            for (int d = 0; d < d_qk; ++d)
                dot += qrow[d] * bf16_bits_to_double(krow[t][d]);
            s[t] = scale64 * dot;
        }
        /* softmax with the max subtracted, then the weighted sum of values */
        double m = s[0];
        for (int64_t t = 1; t < cnt; ++t)
            if (s[t] > m) m = s[t];
        double l = 0.0;
        for (int64_t t = 0; t < cnt; ++t) {
            const double w = exp(s[t] - m);
            l += w;
            for (int e = 0; e < d_v; ++e)
                orow[e] += w * bf16_bits_to_double(krow[t][e]);
        }
        for (int e = 0; e < d_v; ++e) orow[e] /= l;
        lse[r] = m + log(l);
        free(krow);
        free(s);
    }
    return err ? -1 : 0;
}

/*
 * Merge n_parts partial results per row.
 *   o_parts   fp64 [n_parts][rows][d_v]
 *   lse_parts fp64 [n_parts][rows]      (-inf marks an empty part)
 *   out       fp64 [rows][d_v], lse fp64 [rows]
 */
void oracle_combine(const double *o_parts, const double *lse_parts, int n_parts,
                    int64_t rows, int d_v, double *out, double *lse)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int p = 0; p < n_parts; ++p)
            if (lse_parts[p * rows + r] > M) M = lse_parts[p * rows + r];
        double *orow = out + r * d_v;
        for (int e = 0; e < d_v; ++e) orow[e] = 0.0;
        if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
        double total = 0.0;
        for (int p = 0; p < n_parts; ++p)
            total += exp(lse_parts[p * rows + r] - M);
        const double L = M + log(total);
        lse[r] = L;
        for (int p = 0; p < n_parts; ++p) {
            const double lp = lse_parts[p * rows + r];
            if (lp == -INFINITY) continue;
            const double w = exp(lp - L);
            const double *op = o_parts + ((int64_t)p * rows + r) * d_v;
            for (int e = 0; e < d_v; ++e) orow[e] += w * op[e];
        }
    }
}

/* OCP FP8 E4M3 code to its exact value. */
double oracle_e4m3_to_double(uint8_t code)
{
    const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);               /* subnormal: m * 2^-9 */
    else v = ldexp(1.0 + m / 8.0, e - 7);                /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* Round a double to the nearest bf16 (8 significant bits, fp32's exponent
 * range, ties to even) and return its bit pattern. */
uint16_t oracle_double_to_bf16(double x)
{
    if (isnan(x)) return 0x7FC0;
    const int neg = signbit(x);
    double a = fabs(x), r;
    if (a == 0.0) return neg ? 0x8000 : 0;
    int e;
    frexp(a, &e);                       /* a = f * 2^e, f in [0.5, 1) */
    if (e - 1 < -126) {
        r = nearbyint(ldexp(a, 133)) * ldexp(1.0, -133);   /* subnormal step 2^-133 */
    } else {
        r = ldexp(nearbyint(ldexp(a, 8 - e)), e - 8);       /* 8 significant bits */
    }
    if (r >= ldexp(1.0, 128)) return neg ? 0xFF80 : 0x7F80;  /* overflow: infinity */
    float f = (float)r;                 /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)((u >> 16) | (neg ? 0x8000u : 0u));
}

/*
 * Decompress block-scaled fp8 weights to bf16 bits.
 *   code  [heads][K][N] E4M3 codes
 *   scale [heads][ceil(K / blk)][ceil(N / blk)] fp32
 *   w     [heads][K][N] bf16 bits (output)
 */
/* x[i] rounded once to bf16 (nearest even), for n values: the storage of
 * weights that are products of other weights (materialized absorption). */
void oracle_round_bf16_array(const double *x, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_double_to_bf16(x[i]);
}

void oracle_dequant_fp8(const uint8_t *code, const float *scale, int heads, int K, int N,
                        int blk, uint16_t *w)
{
    const int kb = (K + blk - 1) / blk, nb = (N + blk - 1) / blk;
    for (int h = 0; h < heads; ++h)
        for (int k = 0; k < K; ++k)
            for (int n = 0; n < N; ++n) {
                const int64_t i = ((int64_t)h * K + k) * N + n;
                const double sc = scale[((int64_t)h * kb + k / blk) * nb + n / blk];
                w[i] = oracle_double_to_bf16(oracle_e4m3_to_double(code[i]) * sc);
            }
}

/*
 * Batched per-head matmul y[b,h,:] = x[b,h,:] . W[h]  (fp64).
 *   x  fp64 [batch][heads][K]
 *   w  bf16 bits [heads][K][N]
 *   y  fp64 [batch][heads][N]
 */
void oracle_absorb_bmm(const double *x, const uint16_t *w, int batch, int heads,
                       int K, int N, double *y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)batch * heads; ++bh) {
        const int h = (int)(bh % heads);
        const double *xr = x + bh * K;
        const uint16_t *wh = w + (int64_t)h * K * N;
        double *yr = y + bh * N;
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += xr[k] * bf16_bits_to_double(wh[(int64_t)k * N + n]);
            yr[n] = acc;
        }
    }
}
