/*
 * Plain CPU oracle of the Kimi-K2 routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do. It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * What it computes (sources are the Open Model Atlas pages on Kimi K2):
 *   - the layer: each token's output is the router-weighted sum of the
 *     outputs of its selected experts, plus the shared expert applied to
 *     every token ("Mixture of experts" page, experts inspector, Direct
 *     evidence "moe-forward"; Code: forward and moe_infer);
 *   - one expert: down(silu(gate x) * up x), three bias-free linear maps
 *     with weight[out][in] layout ("SwiGLU output" page, evidence "mlp",
 *     class DeepseekV3MLP; "Element-wise product" page, formula h = a (.) u);
 *   - weight storage: FP8 e4m3 with one scale per 128 x 128 block, and
 *     dynamic activation quantisation ("Input features" page, evidence
 *     "linear", quantization_config).
 *
 * Precision. Every dot product is formed in double. The products of two
 * e4m3 values and their 128-term block sums are exact in double (each
 * product is a multiple of 2^-18 below 2^18, a block sum stays below 2^25),
 * so the only roundings are the double-precision scale products and sums.
 * The two quantisation points take their decision in float32: the value is
 * rounded to float, the group scale is fl32(amax / 448) and the code is the
 * round-to-nearest-even, saturating e4m3 encoding of fl32(v / scale), with
 * IEEE float division. The final output is rounded once from double to
 * bfloat16, round-to-nearest-even.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_SHAPE 2
#define ORC_ERR_BAD_ID 5
#define ORC_ERR_DUP_ID 6
#define ORC_ERR_NOMEM 9

#define GROUP 128 /* quantisation block edge, weight_block_size [128, 128] */
#define E4M3_MAX 448.0f

/* ---------------------------------------------------------------------
 * OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits. Exponent field 0 holds subnormals m * 2^-9. The code with
 * exponent 15 and mantissa 7 is NaN; there is no infinity, so the largest
 * finite magnitude is 1.75 * 2^8 = 448.
 * ------------------------------------------------------------------- */
double orc_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int ex = (code >> 3) & 0xF;
    int man = code & 0x7;
    double mag;
    if (ex == 0xF && man == 0x7)
        return NAN;
    if (ex == 0)
        mag = ldexp((double)man, -9);
    else
        mag = ldexp(1.0 + man / 8.0, ex - 7);
    return sign ? -mag : mag;
}

/* Round-to-nearest, ties to the even code, saturating at +-448.
 * Written as a search over the 127 finite non-negative codes (0x00..0x7E),
 * whose values increase with the code: pick the closest; on an exact tie pick
 * the code whose lowest bit is 0. The sign is carried over, so -0 and
 * negative values that round to zero give 0x80. */
uint8_t orc_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    if (a >= E4M3_MAX)
        return (uint8_t)(sign | 0x7E);
    int best = 0;
    double best_d = a; /* distance to code 0 */
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(a - orc_e4m3_decode((uint8_t)c));
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(sign | best);
}

/* bfloat16 -> float: the 16 stored bits are the upper half of a float32. */
float orc_bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* double -> bfloat16, one rounding, nearest with ties to even. bfloat16 has
 * an 8-bit significand and float32's exponent range (normals down to 2^-126,
 * subnormal quantum 2^-133). */
uint16_t orc_bf16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7FC0;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    int q = e - 8;
    if (q < -133)
        q = -133;
    double m = nearbyint(ldexp(a, -q)); /* default rounding mode: ties to even */
    double r = ldexp(m, q);
    float f = (float)r; /* exact: at most 9 significant bits; overflow gives inf */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* ---------------------------------------------------------------------
 * Dynamic quantisation of a row to e4m3 with one float32 scale per
 * 128-element group: scale = amax / 448, code = e4m3(v / scale); an all-zero
 * group gets scale 1, so its codes are the (signed) zeros.
 * ("Input features" page, evidence "linear": activation_scheme dynamic,
 * fmt e4m3.) The pages do not speak of NaN. Reading taken: a NaN has no
 * magnitude, so amax is taken over the other values (a NaN never passes the
 * comparison below), and a NaN value is encoded like any other, as the NaN
 * code (v / scale is NaN).
 * ------------------------------------------------------------------- */
static void quant_group_f32(const float* v, int n, uint8_t* q, float* s)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    float scale = amax > 0.0f ? amax / E4M3_MAX : 1.0f;
    *s = scale;
    for (int i = 0; i < n; ++i) {
        float t = v[i] / scale;
        q[i] = orc_e4m3_encode(t);
    }
}

/* Quantise rows x[rows][cols] given as bfloat16 bits. cols % 128 == 0.
 * q[rows][cols] codes, s[rows][cols/128] scales. */
int orc_quant_rows_bf16(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* s)
{
    if (rows < 0 || cols <= 0 || cols % GROUP)
        return ORC_ERR_SHAPE;
    float buf[GROUP];
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < cols / GROUP; ++g) {
            for (int i = 0; i < GROUP; ++i)
                buf[i] = orc_bf16_to_float(x[r * cols + g * GROUP + i]);
            quant_group_f32(buf, GROUP, q + r * cols + g * GROUP, s + r * (cols / GROUP) + g);
        }
    return ORC_OK;
}

/* Same quantiser for float32 rows (used for the product h). */
int orc_quant_rows_f32(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* s)
{
    if (rows < 0 || cols <= 0 || cols % GROUP)
        return ORC_ERR_SHAPE;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < cols / GROUP; ++g)
            quant_group_f32(x + r * cols + g * GROUP, GROUP, q + r * cols + g * GROUP,
                            s + r * (cols / GROUP) + g);
    return ORC_OK;
}

/* ---------------------------------------------------------------------
 * RMSNorm of bfloat16 rows with a bfloat16 gain per feature, the norm the
 * block applies before its FFN ("Input features" page, evidence "rmsnorm":
 * DeepseekV3RMSNorm, computed in float32 and returned in the input dtype,
 * then scaled by the gain; evidence "block": post_attention_layernorm feeds
 * the mlp). Per row of length n:
 *   v   = fl32(mean of x_i^2)              (sum and division in double)
 *   r   = fl32(1 / sqrt(fl32(v + eps)))    (double, one rounding)
 *   t_i = bf16(fl32(x_i * r))              (back to the input dtype)
 *   y_i = bf16(g_i * t_i)                  (g_i * t_i is exact in float32)
 * The page fixes float32 for the normalisation but neither the summation
 * order of the mean nor the rounding of the reciprocal square root; these
 * are the readings taken here. y[rows][cols] bf16 bits.
 * ------------------------------------------------------------------- */
int orc_rmsnorm_rows(const uint16_t* x, const uint16_t* gain, float eps, int64_t rows,
                     int64_t cols, uint16_t* y)
{
    if (rows < 0 || cols <= 0)
        return ORC_ERR_SHAPE;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * cols;
        double ss = 0.0;
        for (int64_t i = 0; i < cols; ++i) {
            double v = (double)orc_bf16_to_float(xr[i]);
            ss += v * v;
        }
        float var = (float)(ss / (double)cols);
        float t = var + eps;
        float rs = (float)(1.0 / sqrt((double)t));
        for (int64_t i = 0; i < cols; ++i) {
            float xn = orc_bf16_to_float(xr[i]) * rs;
            float tb = orc_bf16_to_float(orc_bf16_from_double((double)xn));
            float g = orc_bf16_to_float(gain[i]);
            y[r * cols + i] = orc_bf16_from_double((double)(g * tb));
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------
 * Dispatch ("Mixture of experts" page, Code: moe_infer): count the tokens
 * routed to each expert, order the flat (token, choice) slots s = n*K + k by
 * expert, and keep the inverse so outputs can be scattered back. The pages
 * sort with an unspecified tie order; this oracle fixes it to ascending s
 * within an expert (a stable sort), which makes the order unique.
 *
 * counts[E], offsets[E+1] (offsets[0] = 0, offsets[e+1] = offsets[e] +
 * counts[e]), sorted_slot[N*K] (position -> slot), slot_pos[N*K]
 * (slot -> position). Ids must lie in [0, E) and be distinct within a row.
 * ------------------------------------------------------------------- */
int orc_dispatch(const int32_t* ids, int64_t N, int32_t K, int32_t E, int32_t* counts,
                 int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos)
{
    if (N < 0 || K < 1 || E < 1 || K > E)
        return ORC_ERR_SHAPE;
    for (int64_t n = 0; n < N; ++n)
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = ids[n * K + k];
            if (e < 0 || e >= E)
                return ORC_ERR_BAD_ID;
            for (int32_t j = 0; j < k; ++j)
                if (ids[n * K + j] == e)
                    return ORC_ERR_DUP_ID;
        }
    for (int32_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t s = 0; s < N * K; ++s)
        counts[ids[s]] += 1;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!fill)
        return ORC_ERR_NOMEM;
    for (int32_t e = 0; e < E; ++e)
        fill[e] = offsets[e];
    for (int64_t s = 0; s < N * K; ++s) {
        int32_t p = fill[ids[s]]++;
        sorted_slot[p] = (int32_t)s;
        slot_pos[s] = p;
    }
    free(fill);
    return ORC_OK;
}

/* ---------------------------------------------------------------------
 * One FP8 linear map y = W x with W[out][in] e4m3 codes and scales
 * ws[out/128][in/128], and x given as e4m3 codes xq[in] with per-group
 * scales xs[in/128] (the dequantised operand is code * scale).
 *   y[o] = sum_kb (xs[kb] * ws[o/128][kb]) * sum_{i in kb} dec(xq[i]) dec(W[o][i])
 * All in double; the inner block sum is exact.
 * ------------------------------------------------------------------- */
static void fp8_linear(const double* xdec, const float* xs, int64_t in, const uint8_t* W,
                       const float* ws, int64_t out, const double* lut, double* y)
{
    int64_t kbn = in / GROUP;
    for (int64_t o = 0; o < out; ++o) {
        const uint8_t* row = W + o * in;
        const float* srow = ws + (o / GROUP) * kbn;
        double acc = 0.0;
        for (int64_t kb = 0; kb < kbn; ++kb) {
            double blk = 0.0;
            for (int64_t i = kb * GROUP; i < (kb + 1) * GROUP; ++i)
                blk += xdec[i] * lut[row[i]];
            acc += ((double)xs[kb] * (double)srow[kb]) * blk;
        }
        y[o] = acc;
    }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One SwiGLU expert on one quantised token: y = down(silu(gate x) * up x),
 * with the product h re-quantised per 128 features before the down map.
 * scratch: 3*d_ff + d_ff doubles/floats handled inside. */
static void expert_forward(const double* xdec, const float* xs, int64_t d, int64_t d_ff,
                           const uint8_t* wg, const float* sg, const uint8_t* wu,
                           const float* su, const uint8_t* wd, const float* sd,
                           const double* lut, double* g, double* u, float* h, uint8_t* hq,
                           float* hs, double* hdec, double* y)
{
    fp8_linear(xdec, xs, d, wg, sg, d_ff, lut, g);
    fp8_linear(xdec, xs, d, wu, su, d_ff, lut, u);
    for (int64_t j = 0; j < d_ff; ++j)
        h[j] = (float)(silu(g[j]) * u[j]); /* a = silu(g), h = a (.) u */
    orc_quant_rows_f32(h, 1, d_ff, hq, hs);
    for (int64_t j = 0; j < d_ff; ++j)
        hdec[j] = lut[hq[j]];
    fp8_linear(hdec, hs, d_ff, wd, sd, d, lut, y);
}

/* ---------------------------------------------------------------------
 * The layer, per token (a per-token loop over the token's K experts):
 *   out[n] = bf16( sum_{k<K} w[n][k] * E_{ids[n][k]}(x_n)  [+ S(x_n)] )
 * with x_n quantised once per token, the routed sum formed in ascending k
 * and the shared expert S (if given) added after it.
 *
 * x[N][d] bf16 bits; ids/w [N][K]; routed weights stacked over experts:
 * wg, wu [E][d_ff][d], sg, su [E][d_ff/128][d/128], wd [E][d][d_ff],
 * sd [E][d/128][d_ff/128]. Shared expert (all NULL to omit) has the same
 * layout with E = 1 and its own intermediate size sh_dff.
 * residual[N][d] bf16 (NULL to omit): the block's second residual addition
 * ("Input features" page, evidence "block": hidden = residual + mlp(...)),
 * added after the shared expert, before the one rounding.
 * tokens: list of token indices to evaluate (NULL = all N, in order);
 * out_bf16[n_eval][d] and, if non-NULL, out_f64[n_eval][d] (before rounding).
 * n_threads <= 0 uses the OpenMP default.
 * ------------------------------------------------------------------- */
int orc_moe_forward(const uint16_t* x, int64_t N, int32_t d, const int32_t* ids, const float* w,
                    int32_t K, int32_t E, int32_t d_ff, const uint8_t* wg, const float* sg,
                    const uint8_t* wu, const float* su, const uint8_t* wd, const float* sd,
                    const uint8_t* sh_wg, const float* sh_sg, const uint8_t* sh_wu,
                    const float* sh_su, const uint8_t* sh_wd, const float* sh_sd, int32_t sh_dff,
                    const uint16_t* residual, const int64_t* tokens, int64_t n_eval,
                    uint16_t* out_bf16, double* out_f64, int32_t n_threads)
{
    if (N < 0 || d <= 0 || d % GROUP || K < 0 || E < 1 || K > E || d_ff <= 0 || d_ff % GROUP)
        return ORC_ERR_SHAPE;
    int has_shared = sh_wg != NULL;
    if (has_shared && (sh_dff <= 0 || sh_dff % GROUP))
        return ORC_ERR_SHAPE;
    if (tokens == NULL)
        n_eval = N;
    for (int64_t t = 0; t < n_eval; ++t) {
        int64_t n = tokens ? tokens[t] : t;
        if (n < 0 || n >= N)
            return ORC_ERR_SHAPE;
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = ids[n * K + k];
            if (e < 0 || e >= E)
                return ORC_ERR_BAD_ID;
            for (int32_t j = 0; j < k; ++j)
                if (ids[n * K + j] == e)
                    return ORC_ERR_DUP_ID;
        }
    }
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = orc_e4m3_decode((uint8_t)c);

    const int64_t D = d, F = d_ff;
    const int64_t maxF = (has_shared && sh_dff > d_ff) ? sh_dff : d_ff;
    const int64_t ex_w = F * D;                    /* bytes per projection per expert */
    const int64_t ex_s = (F / GROUP) * (D / GROUP); /* scales per projection per expert */
    int err = ORC_OK;

#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel
#endif
    {
        double* xdec = (double*)malloc(sizeof(double) * D);
        float* xs = (float*)malloc(sizeof(float) * (D / GROUP));
        uint8_t* xq = (uint8_t*)malloc(D);
        double* g = (double*)malloc(sizeof(double) * maxF);
        double* u = (double*)malloc(sizeof(double) * maxF);
        float* h = (float*)malloc(sizeof(float) * maxF);
        uint8_t* hq = (uint8_t*)malloc(maxF);
        float* hs = (float*)malloc(sizeof(float) * (maxF / GROUP));
        double* hdec = (double*)malloc(sizeof(double) * maxF);
        double* y = (double*)malloc(sizeof(double) * D);
        double* acc = (double*)malloc(sizeof(double) * D);
        if (!xdec || !xs || !xq || !g || !u || !h || !hq || !hs || !hdec || !y || !acc) {
#ifdef _OPENMP
#pragma omp critical
#endif
            err = ORC_ERR_NOMEM;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t t = 0; t < n_eval; ++t) {
                int64_t n = tokens ? tokens[t] : t;
                orc_quant_rows_bf16(x + n * D, 1, D, xq, xs);
                for (int64_t i = 0; i < D; ++i)
                    xdec[i] = lut[xq[i]];
                for (int64_t o = 0; o < D; ++o)
                    acc[o] = 0.0;
                for (int32_t k = 0; k < K; ++k) {
                    int64_t e = ids[n * K + k];
                    expert_forward(xdec, xs, D, F, wg + e * ex_w, sg + e * ex_s, wu + e * ex_w,
                                   su + e * ex_s, wd + e * ex_w, sd + e * ex_s, lut, g, u, h, hq,
                                   hs, hdec, y);
                    double wk = (double)w[n * K + k];
                    for (int64_t o = 0; o < D; ++o)
                        acc[o] += wk * y[o];
                }
                if (has_shared) {
                    expert_forward(xdec, xs, D, sh_dff, sh_wg, sh_sg, sh_wu, sh_su, sh_wd, sh_sd,
                                   lut, g, u, h, hq, hs, hdec, y);
                    for (int64_t o = 0; o < D; ++o)
                        acc[o] += y[o];
                }
                if (residual)
                    for (int64_t o = 0; o < D; ++o)
                        acc[o] += (double)orc_bf16_to_float(residual[n * D + o]);
                for (int64_t o = 0; o < D; ++o) {
                    out_bf16[t * D + o] = orc_bf16_from_double(acc[o]);
                    if (out_f64)
                        out_f64[t * D + o] = acc[o];
                }
            }
        }
        free(xdec); free(xs); free(xq); free(g); free(u); free(h);
        free(hq); free(hs); free(hdec); free(y); free(acc);
    }
    return err;
}

/* ---------------------------------------------------------------------
 * Single expert rows: for each pair (tokens[i], experts[i]) evaluate the
 * expert on the quantised token and return y (double, before any rounding)
 * and, if the pointers are non-NULL, the e4m3 codes and scales of the
 * requantised product h. Layouts as in orc_moe_forward.
 * y[n_rows][d], hq[n_rows][d_ff], hs[n_rows][d_ff/128].
 * ------------------------------------------------------------------- */
int orc_expert_rows(const uint16_t* x, int64_t N, int32_t d, int32_t E, int32_t d_ff,
                    const uint8_t* wg, const float* sg, const uint8_t* wu, const float* su,
                    const uint8_t* wd, const float* sd, const int64_t* tokens,
                    const int32_t* experts, int64_t n_rows, double* y, uint8_t* hq_out,
                    float* hs_out, int32_t n_threads)
{
    if (N < 0 || d <= 0 || d % GROUP || E < 1 || d_ff <= 0 || d_ff % GROUP || n_rows < 0)
        return ORC_ERR_SHAPE;
    for (int64_t i = 0; i < n_rows; ++i) {
        if (tokens[i] < 0 || tokens[i] >= N)
            return ORC_ERR_SHAPE;
        if (experts[i] < 0 || experts[i] >= E)
            return ORC_ERR_BAD_ID;
    }
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = orc_e4m3_decode((uint8_t)c);
    const int64_t D = d, F = d_ff;
    const int64_t ex_w = F * D, ex_s = (F / GROUP) * (D / GROUP);
    int err = ORC_OK;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel
#endif
    {
        double* xdec = (double*)malloc(sizeof(double) * D);
        float* xs = (float*)malloc(sizeof(float) * (D / GROUP));
        uint8_t* xq = (uint8_t*)malloc(D);
        double* g = (double*)malloc(sizeof(double) * F);
        double* u = (double*)malloc(sizeof(double) * F);
        float* h = (float*)malloc(sizeof(float) * F);
        uint8_t* hq = (uint8_t*)malloc(F);
        float* hs = (float*)malloc(sizeof(float) * (F / GROUP));
        double* hdec = (double*)malloc(sizeof(double) * F);
        if (!xdec || !xs || !xq || !g || !u || !h || !hq || !hs || !hdec) {
#ifdef _OPENMP
#pragma omp critical
#endif
            err = ORC_ERR_NOMEM;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t i = 0; i < n_rows; ++i) {
                int64_t e = experts[i];
                orc_quant_rows_bf16(x + tokens[i] * D, 1, D, xq, xs);
                for (int64_t j = 0; j < D; ++j)
                    xdec[j] = lut[xq[j]];
                expert_forward(xdec, xs, D, F, wg + e * ex_w, sg + e * ex_s, wu + e * ex_w,
                               su + e * ex_s, wd + e * ex_w, sd + e * ex_s, lut, g, u, h, hq, hs,
                               hdec, y + i * D);
                if (hq_out)
                    memcpy(hq_out + i * F, hq, F);
                if (hs_out)
                    memcpy(hs_out + i * (F / GROUP), hs, sizeof(float) * (F / GROUP));
            }
        }
        free(xdec); free(xs); free(xq); free(g); free(u); free(h); free(hq); free(hs); free(hdec);
    }
    return err;
}

/* Threads an OpenMP parallel region gets with the given request (for the
 * benchmark's report of the cores the oracle used). */
int orc_threads(int32_t n_threads)
{
#ifdef _OPENMP
    int got = 1;
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel
    {
#pragma omp single
        got = omp_get_num_threads();
    }
    return got;
#else
    (void)n_threads;
    return 1;
#endif
}
