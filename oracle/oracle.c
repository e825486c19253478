/*
 * CPU oracle for online INT8 W8A8 linear layers, the routed int8 MoE layer and
 * the Hadamard-domain (fwht128, u8 group scale under a bf16 row scale) variant.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the HIP
 * library.  Every step is written the slow, obvious way, in the order the
 * method states it, so a reader can check it against the sources by eye.
 *
 * Sources (web pages; titles abbreviated):
 *   [ATOM]  "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5,
 *            with working MTP" (ATOM pull request), sections "Changes" and
 *            the intro paragraph on the precision split.
 *   [QUARK] "Qwen3.6-27B-Quark-W8A8-INT8" model card, "Quantization Scheme"
 *            table and "Quantization Details" list.
 *   [IQ8R]  "Qwen3.6-35B-A3B IQ8R - radiance container" card, the file table
 *            ("Trunk", "Experts", "Activations" rows) and the recipe under
 *            "How this file was made".
 *
 * Numeric conventions (the pages give no precision; these are the readings):
 *   - scales and the dense/MoE epilogues are fp32 with IEEE division, round to
 *     nearest even, no FMA contraction (built with -ffp-contract=off);
 *   - integer dot products are exact (int64 sums, stored as int32 where the
 *     value provably fits);
 *   - routing and SiLU are evaluated in fp64 and rounded once to fp32;
 *   - the g256 epilogue is evaluated in fp64 from an exact int64 group sum.
 * Inputs are assumed finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32.  bf16 is the top half of an fp32 bit pattern.              */
/* ------------------------------------------------------------------------ */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round an fp32 value to the nearest bf16, ties to even (finite inputs). */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

EXPORT int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel loops that follow (the results do not depend on it). */
EXPORT void orc_set_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

EXPORT void orc_bf16_round(const float *x, int64_t n, uint16_t *y)
{
    for (int64_t i = 0; i < n; i++) y[i] = f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* O1: symmetric per-row int8 quantisation.                                   */
/* [QUARK] "Quantization Scheme": activations INT8 per token, symmetric,      */
/* dynamic; weights INT8 per channel (ch_axis=0), symmetric.                  */
/* [IQ8R] "Trunk" row: codes -127..127, round to nearest; recipe clamp=sym.   */
/* scale = amax / 127 in fp32; code = round-half-even(x / scale) (a true      */
/* division), clamped to [-127, 127].  An all-zero row gets scale 0, codes 0. */
/* ------------------------------------------------------------------------ */
static void quant_row_f32(const float *v, int64_t K, int8_t *q, float *s_out)
{
    float amax = 0.0f;
    for (int64_t k = 0; k < K; k++) {
        float a = fabsf(v[k]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int64_t k = 0; k < K; k++) q[k] = 0;
        *s_out = 0.0f;
        return;
    }
    float s = amax / 127.0f;
    for (int64_t k = 0; k < K; k++) {
        float t = v[k] / s;
        float r = nearbyintf(t); /* default rounding mode: nearest, ties even */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[k] = (int8_t)r;
    }
    *s_out = s;
}

EXPORT void orc_quant_rows_f32(const float *x, int64_t M, int64_t K, int64_t ldx,
                               int8_t *q, int64_t ldq, float *s)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) quant_row_f32(x + m * ldx, K, q + m * ldq, s + m);
}

EXPORT void orc_quant_rows_bf16(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                int8_t *q, int64_t ldq, float *s)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float *row = (float *)malloc((size_t)K * sizeof(float));
        for (int64_t k = 0; k < K; k++) row[k] = bf16_to_f32(x[m * ldx + k]);
        quant_row_f32(row, K, q + m * ldq, s + m);
        free(row);
    }
}

/* ------------------------------------------------------------------------ */
/* O3: int8 x int8 -> int32 contraction over K, then the fp32 epilogue       */
/* y = bf16( (float(acc) * sa[m]) * sw[n] ).                                  */
/* [ATOM] "Changes": per-token int8 activations against int8 weights with     */
/* per-channel fp32 scales; output bf16.  Weights are [N, K], K contiguous.   */
/* ------------------------------------------------------------------------ */
static int64_t dot_i8(const int8_t *a, const int8_t *b, int64_t K)
{
    int64_t sum = 0;
    for (int64_t k = 0; k < K; k++) sum += (int64_t)a[k] * (int64_t)b[k];
    return sum;
}

static uint16_t epilogue_bf16(int32_t acc, float sa, float sw)
{
    float v = (float)acc;
    v = v * sa;
    v = v * sw;
    return f32_to_bf16(v);
}

EXPORT void orc_gemm_i32(const int8_t *qa, int64_t lda, const int8_t *qw, int64_t ldw,
                         int64_t M, int64_t N, int64_t K, int32_t *acc, int64_t ldc)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            acc[m * ldc + n] = (int32_t)dot_i8(qa + m * lda, qw + n * ldw, K);
}

EXPORT void orc_epilogue(const int32_t *acc, int64_t ldc, const float *sa, const float *sw,
                         int64_t M, int64_t N, uint16_t *y, int64_t ldy)
{
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * ldy + n] = epilogue_bf16(acc[m * ldc + n], sa[m], sw[n]);
}

EXPORT void orc_gemm_w8a8(const int8_t *qa, const float *sa, int64_t lda, const int8_t *qw,
                          const float *sw, int64_t ldw, int64_t M, int64_t N, int64_t K,
                          uint16_t *y, int64_t ldy)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            int32_t acc = (int32_t)dot_i8(qa + m * lda, qw + n * ldw, K);
            y[m * ldy + n] = epilogue_bf16(acc, sa[m], sw[n]);
        }
}

/* Selected outputs only: point p is (ms[p], ns[p]).  Used to check results at
 * sizes where the full product is too slow on the host. */
EXPORT void orc_gemm_w8a8_points(const int8_t *qa, const float *sa, int64_t lda,
                                 const int8_t *qw, const float *sw, int64_t ldw, int64_t K,
                                 const int64_t *ms, const int64_t *ns, int64_t P,
                                 int32_t *acc_out, uint16_t *y_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; p++) {
        int64_t m = ms[p], n = ns[p];
        int32_t acc = (int32_t)dot_i8(qa + m * lda, qw + n * ldw, K);
        if (acc_out) acc_out[p] = acc;
        if (y_out) y_out[p] = epilogue_bf16(acc, sa[m], sw[n]);
    }
}

/* O1 then O3: the whole online W8A8 linear, bf16 in, bf16 out. */
EXPORT void orc_linear_w8a8(const uint16_t *x, int64_t M, int64_t K, const int8_t *qw,
                            const float *sw, int64_t N, uint16_t *y)
{
    int8_t *q = (int8_t *)malloc((size_t)(M * K));
    float *s = (float *)malloc((size_t)M * sizeof(float));
    orc_quant_rows_bf16(x, M, K, K, q, K, s);
    orc_gemm_w8a8(q, s, K, qw, sw, K, M, N, K, y, N);
    free(q);
    free(s);
}

/* ------------------------------------------------------------------------ */
/* O4: router.  [ATOM] "Changes", fused_moe_triton.py bullet: routing comes   */
/* first in the int8 MoE forward.  Softmax over the E expert logits, keep the */
/* top-k, renormalise the kept probabilities to sum to one.                   */
/* Selection is on the logits (softmax is monotonic): slot j holds the j-th   */
/* largest logit; equal logits go to the lower expert index.  Probabilities   */
/* and weights are computed in fp64 and rounded once to fp32.                 */
/* ------------------------------------------------------------------------ */
EXPORT void orc_route_topk(const float *logits, int64_t T, int64_t E, int64_t k,
                           int32_t *ids, float *w)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        double *p = (double *)malloc((size_t)E * sizeof(double));
        /* selection: repeatedly take the best remaining expert */
        for (int64_t j = 0; j < k; j++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep lower index */
            }
            taken[best] = 1;
            ids[t * k + j] = (int32_t)best;
        }
        /* softmax over all E, in index order */
        double mx = l[0];
        for (int64_t e = 1; e < E; e++)
            if (l[e] > mx) mx = l[e];
        double z = 0.0;
        for (int64_t e = 0; e < E; e++) {
            p[e] = exp((double)l[e] - mx);
            z += p[e];
        }
        for (int64_t e = 0; e < E; e++) p[e] = p[e] / z;
        /* renormalise over the kept experts, in slot order */
        double kept = 0.0;
        for (int64_t j = 0; j < k; j++) kept += p[ids[t * k + j]];
        for (int64_t j = 0; j < k; j++) w[t * k + j] = (float)(p[ids[t * k + j]] / kept);
        free(p);
        free(taken);
    }
}

/* O5: how many (token, slot) pairs each expert receives. */
EXPORT void orc_expert_counts(const int32_t *ids, int64_t n_pairs, int64_t E, int32_t *counts)
{
    for (int64_t e = 0; e < E; e++) counts[e] = 0;
    for (int64_t r = 0; r < n_pairs; r++) counts[ids[r]] += 1;
}

/* ------------------------------------------------------------------------ */
/* O6..O10: routed int8 MoE forward, given the routing (ids, w).              */
/* [ATOM] "Changes", fused_moe_triton.py bullet, in its order:                */
/*   per-token int8 quant of x -> gemm1 over w13 with gated SiLU, the w13     */
/*   rows interleaved (row 2i = gate_i, row 2i+1 = up_i) -> per-token int8    */
/*   requant of each (token, slot) row -> gemm2 over w2 -> weighted combine.  */
/* [ATOM] moe.py bullet: int8 w13/w2 with per-channel fp32 scales.            */
/* Layouts: x [T,H] bf16; w13 [E, 2I, H] int8, s13 [E, 2I]; w2 [E, H, I]      */
/* int8, s2 [E, H]; ids/w [T, k]; out [T, H] bf16.  Pair r = t*k + j.         */
/* The optional intermediates (NULL to skip) are written in pair order:       */
/* qx [T,H], sx [T], acc1 [T*k, 2I], act [T*k, I], qa [T*k, I], sa2 [T*k],    */
/* acc2 [T*k, H], y2 [T*k, H].                                                */
/* ------------------------------------------------------------------------ */
static float silu_times_up(float g, float u)
{
    /* SiLU(g) = g * sigmoid(g) = g / (1 + e^-g), in fp64, rounded to fp32 */
    float sg = (float)((double)g / (1.0 + exp(-(double)g)));
    return sg * u;
}

EXPORT void orc_moe_forward(const uint16_t *x, const int32_t *ids, const float *w,
                            const int8_t *w13, const float *s13, const int8_t *w2,
                            const float *s2, int64_t T, int64_t H, int64_t E, int64_t I,
                            int64_t k, uint16_t *out, int8_t *qx_out, float *sx_out,
                            int32_t *acc1_out, float *act_out, int8_t *qa_out,
                            float *sa2_out, int32_t *acc2_out, float *y2_out)
{
    (void)E;
    const int64_t I2 = 2 * I;
    int8_t *qx = (int8_t *)malloc((size_t)(T * H));
    float *sx = (float *)malloc((size_t)T * sizeof(float));
    float *y2 = (float *)malloc((size_t)(T * k * H) * sizeof(float));

    /* O6: quantise each token once; all its pairs reuse the codes */
    orc_quant_rows_bf16(x, T, H, H, qx, H, sx);

#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < T * k; r++) {
        int64_t t = r / k;
        int64_t e = ids[r];
        const int8_t *we13 = w13 + e * I2 * H;
        const float *se13 = s13 + e * I2;
        const int8_t *we2 = w2 + e * H * I;
        const float *se2 = s2 + e * H;
        float *h = (float *)malloc((size_t)I2 * sizeof(float));
        float *act = (float *)malloc((size_t)I * sizeof(float));
        int8_t *qa = (int8_t *)malloc((size_t)I);
        float sa2;

        /* O7: gemm1, dequantise, gated SiLU over the interleaved rows */
        for (int64_t c = 0; c < I2; c++) {
            int32_t acc = (int32_t)dot_i8(qx + t * H, we13 + c * H, H);
            if (acc1_out) acc1_out[r * I2 + c] = acc;
            float v = (float)acc;
            v = v * sx[t];
            v = v * se13[c];
            h[c] = v;
        }
        for (int64_t i = 0; i < I; i++) act[i] = silu_times_up(h[2 * i], h[2 * i + 1]);
        if (act_out) memcpy(act_out + r * I, act, (size_t)I * sizeof(float));

        /* O8: per-row requant of the activation */
        quant_row_f32(act, I, qa, &sa2);
        if (qa_out) memcpy(qa_out + r * I, qa, (size_t)I);
        if (sa2_out) sa2_out[r] = sa2;

        /* O9: gemm2 and dequantise */
        for (int64_t c = 0; c < H; c++) {
            int32_t acc = (int32_t)dot_i8(qa, we2 + c * I, I);
            if (acc2_out) acc2_out[r * H + c] = acc;
            float v = (float)acc;
            v = v * sa2;
            v = v * se2[c];
            y2[r * H + c] = v;
        }
        free(h);
        free(act);
        free(qa);
    }

    /* O10: weighted combine, fp32, slot order, one rounding to bf16 */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int64_t c = 0; c < H; c++) {
            float acc = 0.0f;
            for (int64_t j = 0; j < k; j++) {
                float term = w[t * k + j] * y2[(t * k + j) * H + c];
                acc = acc + term;
            }
            out[t * H + c] = f32_to_bf16(acc);
        }

    if (qx_out) memcpy(qx_out, qx, (size_t)(T * H));
    if (sx_out) memcpy(sx_out, sx, (size_t)T * sizeof(float));
    if (y2_out) memcpy(y2_out, y2, (size_t)(T * k * H) * sizeof(float));
    free(qx);
    free(sx);
    free(y2);
}

/* ------------------------------------------------------------------------ */
/* O14: dense W8A8 MLP block.  [ATOM] intro (A8W8 for all dense GEMMs of the   */
/* 27B dense model) with the gated-SiLU / requant order of its "Changes",     */
/* fused_moe_triton.py bullet, applied to the dense gate_up and down linears:  */
/*   per-token int8 quant of x -> gate_up GEMM (rows interleaved: 2i = gate_i, */
/*   2i+1 = up_i) dequantised in fp32 -> act_i = SiLU(gate_i) * up_i ->         */
/*   per-token int8 requant of the act row -> down GEMM -> bf16.               */
/* Layouts: x [M,K] bf16; wgu [2I,K] int8, sgu [2I]; wd [N,I] int8, sd [N];    */
/* y [M,N] bf16.  Optional intermediates (NULL to skip): qx [M,K], sx [M],     */
/* acc1 [M,2I], act [M,I], qa [M,I], sa [M], acc2 [M,N].                       */
/* ------------------------------------------------------------------------ */
EXPORT void orc_mlp_forward(const uint16_t *x, int64_t M, int64_t K, const int8_t *wgu,
                            const float *sgu, int64_t I, const int8_t *wd, const float *sd,
                            int64_t N, uint16_t *y, int8_t *qx_out, float *sx_out,
                            int32_t *acc1_out, float *act_out, int8_t *qa_out, float *sa_out,
                            int32_t *acc2_out)
{
    const int64_t I2 = 2 * I;
    int8_t *qx = (int8_t *)malloc((size_t)(M * K));
    float *sx = (float *)malloc((size_t)M * sizeof(float));

    /* per-token quant of the input rows */
    orc_quant_rows_bf16(x, M, K, K, qx, K, sx);

#pragma omp parallel for schedule(dynamic)
    for (int64_t m = 0; m < M; m++) {
        float *h = (float *)malloc((size_t)I2 * sizeof(float));
        float *act = (float *)malloc((size_t)I * sizeof(float));
        int8_t *qa = (int8_t *)malloc((size_t)I);
        float sa;

        /* gate_up GEMM, dequantised */
        for (int64_t c = 0; c < I2; c++) {
            int32_t acc = (int32_t)dot_i8(qx + m * K, wgu + c * K, K);
            if (acc1_out) acc1_out[m * I2 + c] = acc;
            float v = (float)acc;
            v = v * sx[m];
            v = v * sgu[c];
            h[c] = v;
        }
        /* SiLU(gate) * up over the interleaved rows */
        for (int64_t i = 0; i < I; i++) act[i] = silu_times_up(h[2 * i], h[2 * i + 1]);
        if (act_out) memcpy(act_out + m * I, act, (size_t)I * sizeof(float));

        /* per-token requant of the activation row */
        quant_row_f32(act, I, qa, &sa);
        if (qa_out) memcpy(qa_out + m * I, qa, (size_t)I);
        if (sa_out) sa_out[m] = sa;

        /* down GEMM and the bf16 epilogue */
        for (int64_t n = 0; n < N; n++) {
            int32_t acc = (int32_t)dot_i8(qa, wd + n * I, I);
            if (acc2_out) acc2_out[m * N + n] = acc;
            y[m * N + n] = epilogue_bf16(acc, sa, sd[n]);
        }
        free(h);
        free(act);
        free(qa);
    }
    if (qx_out) memcpy(qx_out, qx, (size_t)(M * K));
    if (sx_out) memcpy(sx_out, sx, (size_t)M * sizeof(float));
    free(qx);
    free(sx);
}

/* ------------------------------------------------------------------------ */
/* fp32 -> IEEE binary16 bit pattern, round to nearest even (finite inputs;  */
/* magnitudes from 65520 up become infinity, below 2^-14 subnormal).          */
/* ------------------------------------------------------------------------ */
static uint16_t f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    float a = fabsf(f);
    if (a >= 65520.0f) return (uint16_t)(sign | 0x7c00u);
    if (a < 0x1p-14f) {
        /* subnormal: units of 2^-24 (the scaling is exact), rounded to even */
        float m = nearbyintf(a * 0x1p24f);
        return (uint16_t)(sign | (uint16_t)m);
    }
    uint32_t au = u & 0x7fffffffu;
    uint32_t e = (au >> 23) - 127u + 15u;   /* 1 .. 30 */
    uint32_t m = au & 0x7fffffu;
    uint32_t h = (e << 10) | (m >> 13);
    uint32_t rest = m & 0x1fffu;          /* the 13 dropped mantissa bits */
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u; /* may carry into e */
    return (uint16_t)(sign | h);
}

static float f16_to_f32(uint16_t h)
{
    uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    float v;
    if (e == 0) v = ldexpf((float)m, -24);
    else if (e == 31) v = INFINITY;
    else v = ldexpf((float)(m | 0x400u), (int)e - 25);
    return (h & 0x8000u) ? -v : v;
}

EXPORT void orc_f32_to_f16(const float *x, int64_t n, uint16_t *y)
{
    for (int64_t i = 0; i < n; i++) y[i] = f32_to_f16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* O15: int8 KV-cache quantisation with an f16 scale per token and head.     */
/* [IQ8R] "Serve": kv-cache-dtype i8 stores the attention cache as int8 with  */
/* an f16 scale per token and head.  Per (token t, head h), the D values      */
/* x[t, h, :] (bf16):                                                         */
/*   s = f16(amax / 127)  (amax/127 in fp32, then rounded to f16, even ties); */
/*   code = clamp(round_half_even(x / float(s)), -127, 127), 0 where s == 0.  */
/* The codes are formed against the stored f16 scale, so code * s is the     */
/* value the cache holds.  Precondition: amax / 127 < 65520 (finite scale).  */
/* Token t goes to cache row slots[t] (slots NULL: row t; a negative slot    */
/* skips the token).  x rows have stride ldt elements (heads contiguous);    */
/* q rows stride ldq, s rows stride lds.                                      */
/* ------------------------------------------------------------------------ */
EXPORT void orc_kv_quant_i8(const uint16_t *x, int64_t T, int64_t Hk, int64_t D, int64_t ldt,
                            const int32_t *slots, int8_t *q, int64_t ldq, uint16_t *s,
                            int64_t lds)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        int64_t row = slots ? (int64_t)slots[t] : t;
        if (row < 0) continue;
        for (int64_t h = 0; h < Hk; h++) {
            const uint16_t *xr = x + t * ldt + h * D;
            float amax = 0.0f;
            for (int64_t d = 0; d < D; d++) {
                float a = fabsf(bf16_to_f32(xr[d]));
                if (a > amax) amax = a;
            }
            uint16_t sh = f32_to_f16(amax / 127.0f);
            float sf = f16_to_f32(sh);
            s[row * lds + h] = sh;
            for (int64_t d = 0; d < D; d++) {
                int8_t c = 0;
                if (sf != 0.0f) {
                    float r = nearbyintf(bf16_to_f32(xr[d]) / sf);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    c = (int8_t)r;
                }
                q[row * ldq + h * D + d] = c;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O11: fwht128.  [IQ8R] "Trunk" row: each 128 of K rotated by the            */
/* unnormalised Hadamard; recipe transform=fwht128.  Fast Walsh-Hadamard      */
/* butterfly in fp32, natural (Sylvester) order, stages h = 1, 2, ..., 64;    */
/* at each stage every pair (i, i+h) with (i & h) == 0 becomes                */
/* (v[i] + v[i+h], v[i] - v[i+h]).                                            */
/* ------------------------------------------------------------------------ */
static void fwht128_block(float *v)
{
    for (int h = 1; h < 128; h <<= 1)
        for (int i = 0; i < 128; i++)
            if ((i & h) == 0) {
                float a = v[i];
                float b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

/* In place on fp32 rows; K must be a multiple of 128. */
EXPORT void orc_fwht128_rows(float *v, int64_t M, int64_t K, int64_t ldv)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t b = 0; b < K; b += 128) fwht128_block(v + m * ldv + b);
}

/* [IQ8R] "Activations" row: int8 activations under the same rotation.
 * O11 on each 128-block of the bf16 row, then O1 over the whole rotated row. */
EXPORT void orc_fwht128_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                              int8_t *q, int64_t ldq, float *s)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float *row = (float *)malloc((size_t)K * sizeof(float));
        for (int64_t k = 0; k < K; k++) row[k] = bf16_to_f32(x[m * ldx + k]);
        for (int64_t b = 0; b < K; b += 128) fwht128_block(row + b);
        quant_row_f32(row, K, q + m * ldq, s + m);
        free(row);
    }
}

/* ------------------------------------------------------------------------ */
/* O12: rotated weight preparation with a u8 scale per row per 256 of K      */
/* under a bf16 scale per row.  [IQ8R] "Trunk" row and the recipe line        */
/* "rtn codes=i8 group=256 scale=u8 scale2=bf16 block2=1x* transform=fwht128  */
/* clamp=sym".  Per row n of W [N, K] (fp32):                                 */
/*   w' = fwht128 of each 128-block;                                          */
/*   per group g of 256: a_g = max |w'|, s_g = a_g / 127;                     */
/*   s2 = bf16(max_g s_g / 255);                                              */
/*   su8_g = 0 for an all-zero group, else clamp(round(s_g / s2), 1, 255);    */
/*   eff_g = s2 * su8_g;  code = clamp(round(w' / eff_g), -127, 127).         */
/* A row whose s2 rounds to zero gets zero codes and zero scales.             */
/* ------------------------------------------------------------------------ */
EXPORT void orc_weight_prep_g256(const float *W, int64_t N, int64_t K, int8_t *qw,
                                 uint8_t *su8, uint16_t *s2)
{
    const int64_t G = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        float *row = (float *)malloc((size_t)K * sizeof(float));
        float *sg = (float *)malloc((size_t)G * sizeof(float));
        memcpy(row, W + n * K, (size_t)K * sizeof(float));
        for (int64_t b = 0; b < K; b += 128) fwht128_block(row + b);
        float smax = 0.0f;
        for (int64_t g = 0; g < G; g++) {
            float a = 0.0f;
            for (int64_t k = g * 256; k < (g + 1) * 256; k++) {
                float v = fabsf(row[k]);
                if (v > a) a = v;
            }
            sg[g] = a / 127.0f;
            if (sg[g] > smax) smax = sg[g];
        }
        uint16_t s2b = f32_to_bf16(smax / 255.0f);
        float s2f = bf16_to_f32(s2b);
        s2[n] = s2b;
        for (int64_t g = 0; g < G; g++) {
            uint8_t u = 0;
            if (s2f != 0.0f && sg[g] != 0.0f) {
                float r = nearbyintf(sg[g] / s2f);
                if (r < 1.0f) r = 1.0f;
                if (r > 255.0f) r = 255.0f;
                u = (uint8_t)r;
            }
            su8[n * G + g] = u;
            float eff = s2f * (float)u;
            for (int64_t k = g * 256; k < (g + 1) * 256; k++) {
                int8_t c = 0;
                if (eff != 0.0f) {
                    float r = nearbyintf(row[k] / eff);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    c = (int8_t)r;
                }
                qw[n * K + k] = c;
            }
        }
        free(row);
        free(sg);
    }
}

/* ------------------------------------------------------------------------ */
/* O16: rotated weight preparation with a bf16 scale per row per 128 of K    */
/* (the routed experts and the shared expert's down projection).  [IQ8R]     */
/* "Experts" row (int8 on the same rotated grid with a bf16 scale per row    */
/* and 128 of K) and the recipe lines ffn_gate_up_exps / ffn_down_exps /     */
/* ffn_down_shexp (codes=i8 group=128 scale=bf16 transform=fwht128 clamp=sym).*/
/* Per row n of W [N, K] (fp32): w' = fwht128 of each 128-block (a group is   */
/* one block); s_g = bf16(max |w'| over the group / 127); code =              */
/* clamp(round(w' / float(s_g)), -127, 127), 0 where s_g is 0.  The codes are  */
/* formed against the stored bf16 scale.                                      */
/* ------------------------------------------------------------------------ */
EXPORT void orc_weight_prep_g128(const float *W, int64_t N, int64_t K, int8_t *qw, uint16_t *s)
{
    const int64_t G = K / 128;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        float *row = (float *)malloc((size_t)K * sizeof(float));
        memcpy(row, W + n * K, (size_t)K * sizeof(float));
        for (int64_t b = 0; b < K; b += 128) fwht128_block(row + b);
        for (int64_t g = 0; g < G; g++) {
            float a = 0.0f;
            for (int64_t k = g * 128; k < (g + 1) * 128; k++) {
                float v = fabsf(row[k]);
                if (v > a) a = v;
            }
            uint16_t sb = f32_to_bf16(a / 127.0f);
            float sf = bf16_to_f32(sb);
            s[n * G + g] = sb;
            for (int64_t k = g * 128; k < (g + 1) * 128; k++) {
                int8_t c = 0;
                if (sf != 0.0f) {
                    float r = nearbyintf(row[k] / sf);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    c = (int8_t)r;
                }
                qw[n * K + k] = c;
            }
        }
        free(row);
    }
}

/* O17: g128 GEMM, one output: the exact int32 sum of each 128-group times   */
/* that group's bf16 scale, summed in fp64 in group order, then times the    */
/* activation row scale and 2^-7 (undoing <Hx, Hw> = 128 <x, w>), in fp64,    */
/* rounded once to fp32.                                                      */
static float g128_one(const int8_t *a, const int8_t *wrow, const uint16_t *srow, int64_t K,
                      float sa)
{
    double t = 0.0;
    for (int64_t g = 0; g < K / 128; g++) {
        int64_t accg = dot_i8(a + g * 128, wrow + g * 128, 128);
        t = t + (double)accg * (double)bf16_to_f32(srow[g]);
    }
    t = t * (double)sa;
    t = t * 0.0078125;
    return (float)t;
}

EXPORT void orc_gemm_g128(const int8_t *qa, const float *sa, int64_t M, int64_t K,
                          const int8_t *qw, const uint16_t *s, int64_t N, float *y)
{
    const int64_t G = K / 128;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = g128_one(qa + m * K, qw + n * K, s + n * G, K, sa[m]);
}

/* O18: rotated requant of an fp32 row: fwht128 of each 128-block, then the   */
/* per-row quant O1 over the whole rotated row.  [IQ8R] "Activations" row     */
/* (int8 activations under the same rotation): the down projection's input   */
/* lives on the rotated grid of its weights.                                  */
static void rot_quant_row_f32(const float *v, int64_t K, int8_t *q, float *s_out)
{
    float *row = (float *)malloc((size_t)K * sizeof(float));
    memcpy(row, v, (size_t)K * sizeof(float));
    for (int64_t b = 0; b < K; b += 128) fwht128_block(row + b);
    quant_row_f32(row, K, q, s_out);
    free(row);
}

EXPORT void orc_rot_quant_rows_f32(const float *x, int64_t M, int64_t K, int8_t *q, float *s)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) rot_quant_row_f32(x + m * K, K, q + m * K, s + m);
}

/* ------------------------------------------------------------------------ */
/* O19: routed experts in the Hadamard domain.  [IQ8R] "Experts" and         */
/* "Activations" rows: the 256 routed experts int8 on the rotated grid with a */
/* bf16 scale per row and 128 of K, reading the codes the trunk's quantisers  */
/* write; with the [ATOM] order (routing given) -> quant -> gemm1 with the     */
/* gated SiLU over interleaved w13 -> per-token requant -> gemm2 -> combine:  */
/*   qx, sx = fwht128 + per-token quant of x (O11 + O1, the trunk's codes);    */
/*   per pair r = t*k + j, e = ids[t,j]:                                       */
/*     h[c] = g128(qx[t], w13[e,c], s13[e,c], sx[t])   (O17), c < 2I;          */
/*     act_i = silu(h[2i]) * h[2i+1];                                         */
/*     qa, sa2 = fwht128 + per-row quant of act (O18);                        */
/*     y2[c] = g128(qa, w2[e,c], s2[e,c], sa2), c < H;                        */
/*   out[t,h] = bf16( (sum_j w[t,j] * y2[(t,j),h], fp32, slot order)          */
/*                    + shared[t,h] )   (shared: the shared expert, O20, or    */
/*                                       no term when NULL)                   */
/* Layouts: w13 [E, 2I, H] int8, s13 bf16 [E, 2I, H/128]; w2 [E, H, I],        */
/* s2 bf16 [E, H, I/128]; shared fp32 [T, H].  Intermediates as O6..O10        */
/* (NULL to skip): qx, sx, act, qa, sa2, y2.                                  */
/* ------------------------------------------------------------------------ */
EXPORT void orc_moe_rot_forward(const uint16_t *x, const int32_t *ids, const float *w,
                                const int8_t *w13, const uint16_t *s13, const int8_t *w2,
                                const uint16_t *s2, int64_t T, int64_t H, int64_t E, int64_t I,
                                int64_t k, const float *shared, uint16_t *out, int8_t *qx_out,
                                float *sx_out, float *act_out, int8_t *qa_out, float *sa2_out,
                                float *y2_out)
{
    (void)E;
    const int64_t I2 = 2 * I, GH = H / 128, GI = I / 128;
    int8_t *qx = (int8_t *)malloc((size_t)(T * H));
    float *sx = (float *)malloc((size_t)T * sizeof(float));
    float *y2 = (float *)malloc((size_t)(T * k * H) * sizeof(float));
    orc_fwht128_quant(x, T, H, H, qx, H, sx);

#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < T * k; r++) {
        int64_t t = r / k;
        int64_t e = ids[r];
        float *h = (float *)malloc((size_t)I2 * sizeof(float));
        float *act = (float *)malloc((size_t)I * sizeof(float));
        int8_t *qa = (int8_t *)malloc((size_t)I);
        float sa2;
        for (int64_t c = 0; c < I2; c++)
            h[c] = g128_one(qx + t * H, w13 + (e * I2 + c) * H, s13 + (e * I2 + c) * GH, H,
                            sx[t]);
        for (int64_t i = 0; i < I; i++) act[i] = silu_times_up(h[2 * i], h[2 * i + 1]);
        if (act_out) memcpy(act_out + r * I, act, (size_t)I * sizeof(float));
        rot_quant_row_f32(act, I, qa, &sa2);
        if (qa_out) memcpy(qa_out + r * I, qa, (size_t)I);
        if (sa2_out) sa2_out[r] = sa2;
        for (int64_t c = 0; c < H; c++)
            y2[r * H + c] = g128_one(qa, w2 + (e * H + c) * I, s2 + (e * H + c) * GI, I, sa2);
        free(h);
        free(act);
        free(qa);
    }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int64_t c = 0; c < H; c++) {
            float acc = 0.0f;
            for (int64_t j = 0; j < k; j++) {
                float term = w[t * k + j] * y2[(t * k + j) * H + c];
                acc = acc + term;
            }
            if (shared) acc = acc + shared[t * H + c];
            out[t * H + c] = f32_to_bf16(acc);
        }
    if (qx_out) memcpy(qx_out, qx, (size_t)(T * H));
    if (sx_out) memcpy(sx_out, sx, (size_t)T * sizeof(float));
    if (y2_out) memcpy(y2_out, y2, (size_t)(T * k * H) * sizeof(float));
    free(qx);
    free(sx);
    free(y2);
}

/* ------------------------------------------------------------------------ */
/* O20: the shared expert in the Hadamard domain.  [IQ8R] "Experts" row: the  */
/* shared expert like the routed ones, its gate/up projection as the trunk's  */
/* linears; recipe ffn_gate_up_shexp (group=256 scale=u8 scale2=bf16, as O12)  */
/* and ffn_down_shexp (group=128 scale=bf16, as O16):                          */
/*   qx, sx = fwht128 + per-token quant of x (the trunk's codes);              */
/*   h[c] = float( sum_g su8[c,g] acc_g * sx * s2[c] * 2^-7 )  (O13 in fp64,    */
/*          rounded to fp32 instead of bf16), c < 2Is, rows 2i = gate_i;      */
/*   act_i = silu(h[2i]) * h[2i+1]; qa, sa = O18(act);                        */
/*   y[t,n] = g128(qa, wd[n], sd[n], sa)   (fp32 [T, H]).                      */
/* ------------------------------------------------------------------------ */
EXPORT void orc_shared_expert(const uint16_t *x, int64_t T, int64_t H, int64_t Is,
                              const int8_t *wgu, const uint8_t *su8, const uint16_t *s2,
                              const int8_t *wd, const uint16_t *sd, float *y, float *act_out)
{
    const int64_t I2 = 2 * Is, G = H / 256, GI = Is / 128;
    int8_t *qx = (int8_t *)malloc((size_t)(T * H));
    float *sx = (float *)malloc((size_t)T * sizeof(float));
    orc_fwht128_quant(x, T, H, H, qx, H, sx);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        float *h = (float *)malloc((size_t)I2 * sizeof(float));
        float *act = (float *)malloc((size_t)Is * sizeof(float));
        int8_t *qa = (int8_t *)malloc((size_t)Is);
        float sa;
        for (int64_t c = 0; c < I2; c++) {
            int64_t tsum = 0;
            for (int64_t g = 0; g < G; g++)
                tsum += (int64_t)su8[c * G + g] *
                        dot_i8(qx + t * H + g * 256, wgu + c * H + g * 256, 256);
            double v = (double)tsum * (double)sx[t];
            v = v * (double)bf16_to_f32(s2[c]);
            v = v * 0.0078125;
            h[c] = (float)v;
        }
        for (int64_t i = 0; i < Is; i++) act[i] = silu_times_up(h[2 * i], h[2 * i + 1]);
        if (act_out) memcpy(act_out + t * Is, act, (size_t)Is * sizeof(float));
        rot_quant_row_f32(act, Is, qa, &sa);
        for (int64_t n = 0; n < H; n++) y[t * H + n] = g128_one(qa, wd + n * Is, sd + n * GI, Is, sa);
        free(h);
        free(act);
        free(qa);
    }
    free(qx);
    free(sx);
}

/* ------------------------------------------------------------------------ */
/* O21: the router gate in bf16.  [ATOM] intro (precision split): the router  */
/* gate stays BF16.  logits[t,e] = sum_h x[t,h] * wg[e,h] with bf16 operands; */
/* the products are exact in fp64 and are summed in fp64 in index order,      */
/* then rounded once to fp32.                                                 */
/* ------------------------------------------------------------------------ */
EXPORT void orc_router_gate_bf16(const uint16_t *x, const uint16_t *wg, int64_t T, int64_t H,
                                 int64_t E, float *logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int64_t e = 0; e < E; e++) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; h++)
                acc = acc + (double)bf16_to_f32(x[t * H + h]) * (double)bf16_to_f32(wg[e * H + h]);
            logits[t * E + e] = (float)acc;
        }
}

/* ------------------------------------------------------------------------ */
/* O13: g256 GEMM in the rotated domain.  Per output (m, n):                  */
/*   acc_g = sum over the 256 k of group g of qa[m,k] * qw[n,k]  (exact);     */
/*   T = sum_g su8[n,g] * acc_g                                  (int64);     */
/*   y = bf16( float( T * sa[m] * s2[n] * 2^-7 ) )              (fp64).       */
/* The 2^-7 undoes <Hx, Hw> = 128 <x, w> for the unnormalised transform.      */
/* ------------------------------------------------------------------------ */
static uint16_t g256_one(const int8_t *a, const int8_t *wrow, const uint8_t *su8row,
                         int64_t K, float sa, uint16_t s2b, int64_t *tsum_out)
{
    int64_t tsum = 0;
    for (int64_t g = 0; g < K / 256; g++) {
        int64_t accg = dot_i8(a + g * 256, wrow + g * 256, 256);
        tsum += (int64_t)su8row[g] * accg;
    }
    if (tsum_out) *tsum_out = tsum;
    double v = (double)tsum * (double)sa;
    v = v * (double)bf16_to_f32(s2b);
    v = v * 0.0078125;
    return f32_to_bf16((float)v);
}

EXPORT void orc_gemm_g256(const int8_t *qa, const float *sa, int64_t M, int64_t K,
                          const int8_t *qw, const uint8_t *su8, const uint16_t *s2, int64_t N,
                          uint16_t *y, int64_t *tsum)
{
    const int64_t G = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = g256_one(qa + m * K, qw + n * K, su8 + n * G, K, sa[m], s2[n],
                                    tsum ? tsum + m * N + n : NULL);
}

EXPORT void orc_gemm_g256_points(const int8_t *qa, const float *sa, int64_t K,
                                 const int8_t *qw, const uint8_t *su8, const uint16_t *s2,
                                 const int64_t *ms, const int64_t *ns, int64_t P,
                                 uint16_t *y, int64_t *tsum)
{
    const int64_t G = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; p++) {
        int64_t m = ms[p], n = ns[p];
        y[p] = g256_one(qa + m * K, qw + n * K, su8 + n * G, K, sa[m], s2[n],
                        tsum ? tsum + p : NULL);
    }
}
