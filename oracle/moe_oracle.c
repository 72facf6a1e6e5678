/*
 * moe_oracle.c -- plain, slow CPU oracle of one sparse MoE layer's forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP path, and the HIP path never calls it.
 *
 * What it computes, token by token (every token is independent):
 *   1. logits a[e] = sum_h x[h] * Wg[e][h], accumulated in double, rounded to
 *      fp32 (the gate is computed in FP32: page "MAX 中 Step-3.5-Flash
 *      架构解析…", section "MoE：共享专家、sigmoid 路由与激活裁剪", the
 *      Step3p5MoEGate paragraph).
 *   2. scores s[e] = sigmoid(a[e]) in fp32; corrected c[e] = s[e] + bias[e]
 *      (fp32 add; the bias is a learnable fp32 per-expert vector, same
 *      paragraph).
 *   3. the k experts with the largest corrected score are selected, ordered
 *      by (c descending, index ascending); NaN ranks below every number;
 *      indices are clamped to [0, E-1] (same paragraph: top-k on corrected
 *      scores, index clamp as a NaN/Inf guard).
 *   4. the weight of a selected expert is its *raw* score s (not c); if
 *      norm_expert_weight, the k weights are divided by their sum; they are
 *      always multiplied by router_scaling_factor (same paragraph; the
 *      config table gives norm_expert_weight and the 3.0 factor).
 *   5. each selected expert e: g = W13[e][0:I] x, u = W13[e][I:2I] x,
 *      h = act(g, u, L), y = W2[e] h (clipped SwiGLU on the concatenated
 *      gate|up projection, same section; gate rows first is this oracle's
 *      reading of "concatenated").
 *   6. shared expert: y_sh = Ws2 act(Ws13 x, L_shared) (always-on MLP of
 *      width share_expert_dim, same section).
 *   7. out = sum_j w_j y_j + y_sh.
 *
 * act(g, u, L) = silu(g) * u when L == 0 (config table: limit 0 means no
 * clipping); otherwise min(silu(g), L) * clamp(u, -L, L).  The pages only say
 * the SwiGLU is "clipped" with a per-layer limit; clamping each factor is this
 * oracle's reading.
 *
 * FP8 mode (routed experts stored as OCP E4M3FN codes with one fp32 scale per
 * 128x128 weight block: miles page "Step-5-Preview", section 1 Model
 * Introduction): the true weight is decode(q) * scale (the trainer's
 * dequantisation on load).  The inputs of both routed projections (x, and h)
 * are quantised per (row, 128-column group): s_a = amax / 448 (1 if amax is
 * 0), q_a = E4M3FN_RNE_saturating(a / s_a), a' = decode(q_a) * s_a.  The pages
 * do not say how activations meet FP8 weights; this dynamic per-group
 * quantisation is the oracle's reading.  Router and shared expert stay bf16.
 *
 * Precision: inputs are bf16 (or E4M3 codes) / fp32; every dot product is
 * accumulated in double and each intermediate tensor is rounded to fp32.
 * Parity of this file is pinned by the CPU tests (closed forms, brute force,
 * textbook special cases); see the test suite.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t H, E, k, I, Is;
    float scale;
    int32_t norm;
    float limit, limit_shared;
    int32_t fp8;
} orc_cfg;

/* ---- scalar helpers --------------------------------------------------- */

uint16_t orc_bf16_round(float f);

static float bf16_val(uint16_t v) {
    uint32_t u = ((uint32_t)v) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* OCP 8-bit floating point, E4M3FN flavour: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
 * (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities; largest finite
 * magnitude is 1.75 * 2^8 = 448. */
double orc_e4m3_decode(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round-to-nearest-even, saturating encode: the finite code nearest to v;
 * on an exact tie the code with an even mantissa (even code) wins; anything
 * beyond 448 in magnitude becomes +-448; NaN maps to the NaN code. */
uint8_t orc_e4m3_encode(float v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 0x7F; ++c) {          /* all non-negative finite codes */
        double d = fabs(orc_e4m3_decode((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = c;
        }
    }
    return sign | (uint8_t)best;
}

double orc_silu(double g) { return g / (1.0 + exp(-g)); }

/* clipped SwiGLU, see the header comment */
double orc_act(double g, double u, double L) {
    double sg = orc_silu(g);
    if (L == 0.0) return sg * u;
    if (sg > L) sg = L;
    if (u > L) u = L;
    if (u < -L) u = -L;
    return sg * u;
}

/* per (row, 128-group) dynamic E4M3 quantise-dequantise of a fp32 row, in place */
static void quant_row_fp8(float* a, int n) {
    for (int g0 = 0; g0 < n; g0 += 128) {
        float amax = 0.f;
        for (int i = g0; i < g0 + 128 && i < n; ++i) {
            float m = fabsf(a[i]);
            if (m > amax) amax = m;
        }
        float sa = amax > 0.f ? amax / 448.0f : 1.0f;
        for (int i = g0; i < g0 + 128 && i < n; ++i) {
            float r = a[i] / sa;
            a[i] = (float)orc_e4m3_decode(orc_e4m3_encode(r)) * sa;
        }
    }
}

/* "a ranks above b" for the top-k order: larger value first, NaN last,
 * equal values -> lower index first */
static int ranks_above(float ca, int ia, float cb, int ib) {
    int na = isnan(ca), nb = isnan(cb);
    if (na && nb) return ia < ib;
    if (na) return 0;
    if (nb) return 1;
    if (ca > cb) return 1;
    if (ca < cb) return 0;
    return ia < ib;
}

/* ---- routing ------------------------------------------------------------ */

/* logits, raw scores s and corrected scores c of one token over all E experts */
static void score_token(const orc_cfg* c, const uint16_t* xt, const uint16_t* wg, const float* bias,
                        float* logits_out, float* corr_out, float* s_buf, float* c_buf) {
    const int H = c->H, E = c->E;
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        const uint16_t* we = wg + (size_t)e * H;
        for (int h = 0; h < H; ++h) acc += (double)bf16_val(xt[h]) * (double)bf16_val(we[h]);
        float a = (float)acc;
        float s = (float)(1.0 / (1.0 + exp(-(double)a)));
        s_buf[e] = s;
        c_buf[e] = bias ? s + bias[e] : s;
        if (logits_out) logits_out[e] = a;
        if (corr_out) corr_out[e] = c_buf[e];
    }
}

/* selection: k rounds, each picks the best expert not yet chosen */
static void select_topk(const orc_cfg* c, const float* c_buf, int32_t* ids) {
    const int E = c->E, k = c->k;
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || ranks_above(c_buf[e], e, c_buf[best], best)) best = e;
        }
        if (best < 0) best = 0;
        if (best > E - 1) best = E - 1;
        taken[best] = 1;
        ids[j] = best;
    }
    free(taken);
}

/* the k weights of the chosen experts from their raw scores */
static void weigh(const orc_cfg* c, const float* s_buf, const int32_t* ids, float* w) {
    const int k = c->k;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += (double)s_buf[ids[j]];
    for (int j = 0; j < k; ++j) {
        double v = (double)s_buf[ids[j]];
        if (c->norm) v = (double)(float)(v / sum);
        w[j] = (float)(v * (double)c->scale);
    }
}

/* Routing of one token.  With ids_in == NULL the k experts are chosen from
 * the corrected scores.  With ids_in given (routing replay: miles page
 * "Step-5-Preview", section 5.2 Algorithm, where the trainer reuses the
 * rollout's expert choices) the choice is taken as given, each id clamped to
 * [0, E-1] as the selection's own guard does, and only the weights are
 * computed, from the current raw scores.  That the replayed choice keeps the
 * weights of the model being run is this oracle's reading: the page says only
 * that the expert choices are replayed. */
static void route_token(const orc_cfg* c, const uint16_t* xt, const uint16_t* wg,
                        const float* bias, const int32_t* ids_in, int32_t* ids, float* w,
                        float* logits_out, float* corr_out, float* s_buf, float* c_buf) {
    score_token(c, xt, wg, bias, logits_out, corr_out, s_buf, c_buf);
    if (ids_in) {
        for (int j = 0; j < c->k; ++j) {
            int e = ids_in[j];
            ids[j] = e < 0 ? 0 : (e > c->E - 1 ? c->E - 1 : e);
        }
    } else {
        select_topk(c, c_buf, ids);
    }
    weigh(c, s_buf, ids, w);
}

/* Route T tokens.  x [T,H] bf16, wg [E,H] bf16, bias [E] fp32 ->
 * ids [T,k] int32, w [T,k] fp32; logits/corrected [T,E] fp32 if non-NULL.
 * ids_in [T,k] (optional): replayed expert choices; bias is then unused. */
int orc_route(const orc_cfg* c, int64_t T, const uint16_t* x, const uint16_t* wg,
              const float* bias, const int32_t* ids_in, int32_t* ids, float* w, float* logits,
              float* corrected) {
    if (!c || c->k < 1 || c->k > c->E) return 1;
#pragma omp parallel
    {
        float* s_buf = (float*)malloc(sizeof(float) * (size_t)c->E);
        float* c_buf = (float*)malloc(sizeof(float) * (size_t)c->E);
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < T; ++t)
            route_token(c, x + t * c->H, wg, bias, ids_in ? ids_in + t * c->k : NULL, ids + t * c->k,
                        w + t * c->k,
                        logits ? logits + t * c->E : NULL, corrected ? corrected + t * c->E : NULL,
                        s_buf, c_buf);
        free(s_buf);
        free(c_buf);
    }
    return 0;
}

/* ---- expert MLPs --------------------------------------------------------- */

/* weight element (row n, column kk) of a [N,K] matrix: bf16, or FP8 code x
 * the fp32 scale of its 128x128 block */
static float wval(const void* W, const float* Ws, int K, int n, int kk, int fp8) {
    if (!fp8) return bf16_val(((const uint16_t*)W)[(size_t)n * K + kk]);
    uint8_t q = ((const uint8_t*)W)[(size_t)n * K + kk];
    float s = Ws[(size_t)(n / 128) * (K / 128) + kk / 128];
    return (float)orc_e4m3_decode(q) * s;
}

/* y[H] = W2 act(W13 xin, L), xin fp32 [H]; W13 [2N,H], W2 [H,N].
 * round_gu: g and u are rounded to bf16 before the activation (a training
 * forward that keeps them in bf16 for its backward). */
static void mlp(const orc_cfg* c, int N, const float* xin, const void* W13, const float* S13,
                const void* W2, const float* S2, float L, int fp8, float* hbuf, float* y, int round_gu) {
    const int H = c->H;
    for (int i = 0; i < N; ++i) {
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
            g += (double)wval(W13, S13, H, i, h, fp8) * (double)xin[h];
            u += (double)wval(W13, S13, H, N + i, h, fp8) * (double)xin[h];
        }
        float gf = (float)g, uf = (float)u;
        if (round_gu) {
            gf = bf16_val(orc_bf16_round(gf));
            uf = bf16_val(orc_bf16_round(uf));
        }
        hbuf[i] = (float)orc_act((double)gf, (double)uf, (double)L);
    }
    if (fp8) quant_row_fp8(hbuf, N);
    for (int o = 0; o < H; ++o) {
        double acc = 0.0;
        for (int i = 0; i < N; ++i) acc += (double)wval(W2, S2, N, o, i, fp8) * (double)hbuf[i];
        y[o] = (float)acc;
    }
}

/*
 * Full layer for n tokens (rows tok[0..n-1] of x, or 0..n-1 if tok is NULL).
 * out [n,H] fp32; ids [n,k]; w [n,k]; y_routed [n,k,H] and y_shared [n,H]
 * (fp32, optional) expose the per-expert outputs for the tests.
 * w13: [E,2I,H] bf16 or E4M3 codes; w13s [E,2I/128,H/128] (FP8 only);
 * w2: [E,H,I]; w2s [E,H/128,I/128]; ws13 [2Is,H] bf16; ws2 [H,Is] bf16.
 * ids_in [T,k] (optional, indexed by token like x): replayed expert choices,
 * see route_token.
 */
int orc_layer(const orc_cfg* c, int64_t n, const int64_t* tok, const uint16_t* x,
              const uint16_t* wg, const float* bias, const int32_t* ids_in, const void* w13, const float* w13s,
              const void* w2, const float* w2s, const uint16_t* ws13, const uint16_t* ws2,
              float* out, int32_t* ids, float* w, float* y_routed, float* y_shared, int32_t round_gu) {
    if (!c || c->k < 1 || c->k > c->E) return 1;
    const int H = c->H, E = c->E, k = c->k, I = c->I, Is = c->Is;
    const size_t esz = c->fp8 ? 1 : 2;
    int err = 0;
#pragma omp parallel
    {
        float* s_buf = (float*)malloc(sizeof(float) * (size_t)E);
        float* c_buf = (float*)malloc(sizeof(float) * (size_t)E);
        float* xin = (float*)malloc(sizeof(float) * (size_t)H);
        float* xq = (float*)malloc(sizeof(float) * (size_t)H);
        int hmax = I > Is ? I : Is;
        float* hbuf = (float*)malloc(sizeof(float) * (size_t)(hmax > 0 ? hmax : 1));
        float* y = (float*)malloc(sizeof(float) * (size_t)H);
        double* acc = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            int64_t t = tok ? tok[r] : r;
            const uint16_t* xt = x + t * H;
            int32_t* id = ids + r * k;
            float* wt = w + r * k;
            route_token(c, xt, wg, bias, ids_in ? ids_in + t * k : NULL, id, wt, NULL, NULL, s_buf, c_buf);
            for (int h = 0; h < H; ++h) xin[h] = bf16_val(xt[h]);
            memcpy(xq, xin, sizeof(float) * (size_t)H);
            if (c->fp8) quant_row_fp8(xq, H);
            for (int h = 0; h < H; ++h) acc[h] = 0.0;
            for (int j = 0; j < k; ++j) {
                int e = id[j];
                const char* W13e = (const char*)w13 + (size_t)e * 2 * I * H * esz;
                const char* W2e = (const char*)w2 + (size_t)e * H * I * esz;
                const float* S13 = c->fp8 ? w13s + (size_t)e * (2 * I / 128) * (H / 128) : NULL;
                const float* S2 = c->fp8 ? w2s + (size_t)e * (H / 128) * (I / 128) : NULL;
                mlp(c, I, xq, W13e, S13, W2e, S2, c->limit, c->fp8, hbuf, y, round_gu);
                if (y_routed) memcpy(y_routed + (r * k + j) * H, y, sizeof(float) * (size_t)H);
                for (int h = 0; h < H; ++h) acc[h] += (double)wt[j] * (double)y[h];
            }
            if (Is > 0) {
                mlp(c, Is, xin, ws13, NULL, ws2, NULL, c->limit_shared, 0, hbuf, y, round_gu);
                if (y_shared) memcpy(y_shared + r * H, y, sizeof(float) * (size_t)H);
                for (int h = 0; h < H; ++h) acc[h] += (double)y[h];
            } else if (y_shared) {
                memset(y_shared + r * H, 0, sizeof(float) * (size_t)H);
            }
            for (int h = 0; h < H; ++h) out[r * H + h] = (float)acc[h];
        }
        free(s_buf); free(c_buf); free(xin); free(xq); free(hbuf); free(y); free(acc);
    }
    return err;
}

/* Per-expert token counts and the expert-major, token-ascending row order of
 * the (token, slot) pairs: the plain definition of the permutation.
 * ids [T,k] -> counts [E], offsets [E+1] (exclusive prefix sum),
 * row_to_pair [T*k] (row r holds pair p = t*k + j), pair_to_row [T*k]. */
int orc_permute(int64_t T, int32_t k, int32_t E, const int32_t* ids, int32_t* counts,
                int32_t* offsets, int32_t* row_to_pair, int32_t* pair_to_row) {
    const int64_t P = T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (ids[p] < 0 || ids[p] >= E) return 1;
        counts[ids[p]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
    for (int64_t p = 0; p < P; ++p) {      /* pairs in ascending order -> stable */
        int e = ids[p];
        int32_t r = offsets[e] + fill[e]++;
        row_to_pair[r] = (int32_t)p;
        pair_to_row[p] = r;
    }
    free(fill);
    return 0;
}

/* ---- the steps either side of the layer --------------------------------- */

/* fp32 -> bf16 bit pattern, round to nearest, ties to even (NaN stays NaN) */
uint16_t orc_bf16_round(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Zero-centred RMSNorm in front of the MoE layer (MAX page, the model
 * overview and the weight-adaptation notes: the block's norms are
 * zero-centred RMSNorms with weight_offset 1, i.e. the stored weight g is
 * used as 1 + g; the AutoModel page's benchmark table keeps norms and the
 * residual stream in FP32).  Per row of the fp32 residual r [T,H]:
 *   x[h] = r[h] / sqrt(mean_h r^2 + eps) * (1 + g[h])
 * with the mean in double, the result rounded to fp32 and then to bf16 (the
 * layer's input dtype).  eps is not printed on the pages; it is an input. */
int orc_rmsnorm(int64_t T, int32_t H, const float* r, const float* g, float eps, uint16_t* x) {
    if (T < 0 || H < 1) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float* rt = r + t * H;
        double ss = 0.0;
        for (int h = 0; h < H; ++h) ss += (double)rt[h] * (double)rt[h];
        double inv = 1.0 / sqrt(ss / (double)H + (double)eps);
        for (int h = 0; h < H; ++h) {
            float y = (float)((double)rt[h] * inv * (1.0 + (double)g[h]));
            x[t * H + h] = orc_bf16_round(y);
        }
    }
    return 0;
}

/* Static balanced routing (AutoModel page, benchmark table: the Step-5
 * benchmark runs with a fake, balanced, static expert routing).  The page
 * gives no rule; this oracle's reading is the round-robin that deals the T*k
 * (token, slot) pairs to the experts in turn: pair p = t*k + j goes to expert
 * p mod E.  Every expert gets floor(T*k/E) or one more pair, and the k
 * experts of one token are distinct because k <= E. */
int orc_balanced_ids(int64_t T, int32_t k, int32_t E, int32_t* ids) {
    if (k < 1 || k > E || T < 0) return 1;
    for (int64_t p = 0; p < T * k; ++p) ids[p] = (int32_t)(p % E);
    return 0;
}

/* ---- backward of the layer (bf16 experts) -------------------------------
 *
 * The gradient of the forward above with respect to x, the router weight and
 * every expert weight, given dL/dout (the trainer's side of the method: the
 * AutoModel page's benchmark and the miles page's BF16 trainer run forward,
 * backward and optimizer).  The expert choice is a discrete function of the
 * scores and passes no gradient; the routing bias only steers that choice,
 * so it has none.  Everything here is computed in double from the bf16
 * inputs (the forward's fp32 roundings are not repeated), so the result is
 * the exact gradient up to double rounding:
 *   w_j = scale * s_j / S (S = sum of the k chosen raw scores; S -> 1 without
 *         normalisation), s_j = sigmoid(a_j)
 *   dy_j = w_j dout;  dw_j = dout . y_j
 *   dh_j = W2_e^T dy_j;  (dg, du) = act'(g, u) dh_j;  dx += W13_e^T dgu_j
 *   dW2_e += dy_j h_j^T;  dW13_e += dgu_j x^T
 *   ds_j = scale/S (dw_j - sum_j' dw_j' s_j' / S)   (scale dw_j without norm)
 *   da_j = ds_j s_j (1 - s_j);  dW_router[e_j] += da_j x;  dx += da_j W_router[e_j]
 *   shared: dhs = Ws2^T dout, (dgs, dus) = act'(gs, us) dhs, dx += Ws13^T dgus,
 *           dWs2 += dout hs^T, dWs13 += dgus x^T
 * act'(g, u, L): with L = 0, dg = u silu'(g), du = silu(g); with L > 0 each
 * clamp passes the gradient where its input lies in the clamp's range, ends
 * included (the convention of torch's clamp), else none:
 *   dg = clamp(u) silu'(g) [silu(g) <= L],  du = min(silu(g), L) [|u| <= L].
 * silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g))).
 * Slots are treated one by one, so a replayed choice holding an expert twice
 * gets the sum of both slots' terms.
 * round_gu: the pre-activations (g, u) are rounded to bf16 before the
 * activation and its derivative, as a training forward that keeps them in
 * bf16 computes; the gradient then passes through the rounding as through
 * the identity.  The clamps' pass/stop decisions are taken on those bf16
 * values on both sides.
 */
static double sigm(double a) { return 1.0 / (1.0 + exp(-a)); }

void orc_act_grad(double g, double u, double L, double* dg, double* du) {
    double sg = sigm(g);
    double silu = g * sg, dsilu = sg * (1.0 + g * (1.0 - sg));
    if (L == 0.0) {
        *dg = u * dsilu;
        *du = silu;
        return;
    }
    double uc = u > L ? L : (u < -L ? -L : u);
    double sc = silu > L ? L : silu;
    *dg = silu <= L ? uc * dsilu : 0.0;
    *du = (u >= -L && u <= L) ? sc : 0.0;
}

/* per token: everything the weight gradients need, and dx */
typedef struct {
    double *dgu, *h, *w, *da, *dgus, *hs, *dx;   /* [k,2I], [k,I], [k], [k], [2Is], [Is], [H] */
} tok_grads;

static double round_bf16_d(double v) {
    const uint16_t b = orc_bf16_round((float)v);
    return (double)bf16_val(b);
}

static void token_backward(const orc_cfg* c, const double* x, const uint16_t* wg, const int32_t* ids,
                           const uint16_t* w13, const uint16_t* w2, const uint16_t* ws13, const uint16_t* ws2,
                           const float* dout, tok_grads* o, double* buf, int round_gu) {
    const int H = c->H, k = c->k, I = c->I, Is = c->Is;
    double* s = buf;               /* k */
    double* dw = s + k;            /* k */
    double* gu = dw + k;           /* 2 max(I, Is) */
    double* dh = gu + 2 * (I > Is ? I : Is);
    double* y = dh + (I > Is ? I : Is);   /* H */
    double S = 0.0;
    for (int j = 0; j < k; ++j) {
        const uint16_t* we = wg + (size_t)ids[j] * H;
        double a = 0.0;
        for (int h = 0; h < H; ++h) a += x[h] * (double)bf16_val(we[h]);
        s[j] = sigm(a);
        S += s[j];
    }
    if (!c->norm) S = 1.0;
    for (int h = 0; h < H; ++h) o->dx[h] = 0.0;
    for (int j = 0; j < k; ++j) {
        const int e = ids[j];
        const uint16_t* W13 = w13 + (size_t)e * 2 * I * H;
        const uint16_t* W2 = w2 + (size_t)e * H * I;
        double* hj = o->h + (size_t)j * I;
        double* dgu = o->dgu + (size_t)j * 2 * I;
        o->w[j] = (double)c->scale * s[j] / S;
        for (int n = 0; n < 2 * I; ++n) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h) acc += (double)bf16_val(W13[(size_t)n * H + h]) * x[h];
            gu[n] = round_gu ? round_bf16_d(acc) : acc;
        }
        for (int i = 0; i < I; ++i) hj[i] = orc_act(gu[i], gu[I + i], (double)c->limit);
        double d = 0.0;
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int i = 0; i < I; ++i) acc += (double)bf16_val(W2[(size_t)h * I + i]) * hj[i];
            y[h] = acc;
            d += (double)dout[h] * acc;
        }
        dw[j] = d;
        for (int i = 0; i < I; ++i) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h) acc += (double)bf16_val(W2[(size_t)h * I + i]) * (double)dout[h];
            dh[i] = o->w[j] * acc;
        }
        for (int i = 0; i < I; ++i) {
            double dg, du;
            orc_act_grad(gu[i], gu[I + i], (double)c->limit, &dg, &du);
            dgu[i] = dh[i] * dg;
            dgu[I + i] = dh[i] * du;
        }
        for (int n = 0; n < 2 * I; ++n) {
            if (dgu[n] == 0.0) continue;
            const uint16_t* row = W13 + (size_t)n * H;
            for (int h = 0; h < H; ++h) o->dx[h] += dgu[n] * (double)bf16_val(row[h]);
        }
    }
    /* router */
    double sdw = 0.0;
    for (int j = 0; j < k; ++j) sdw += dw[j] * s[j] / S;
    for (int j = 0; j < k; ++j) {
        double ds = c->norm ? (double)c->scale / S * (dw[j] - sdw) : (double)c->scale * dw[j];
        o->da[j] = ds * s[j] * (1.0 - s[j]);
        const uint16_t* we = wg + (size_t)ids[j] * H;
        for (int h = 0; h < H; ++h) o->dx[h] += o->da[j] * (double)bf16_val(we[h]);
    }
    /* shared expert */
    if (Is > 0) {
        for (int n = 0; n < 2 * Is; ++n) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h) acc += (double)bf16_val(ws13[(size_t)n * H + h]) * x[h];
            gu[n] = round_gu ? round_bf16_d(acc) : acc;
        }
        for (int i = 0; i < Is; ++i) o->hs[i] = orc_act(gu[i], gu[Is + i], (double)c->limit_shared);
        for (int i = 0; i < Is; ++i) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h) acc += (double)bf16_val(ws2[(size_t)h * Is + i]) * (double)dout[h];
            double dg, du;
            orc_act_grad(gu[i], gu[Is + i], (double)c->limit_shared, &dg, &du);
            o->dgus[i] = acc * dg;
            o->dgus[Is + i] = acc * du;
        }
        for (int n = 0; n < 2 * Is; ++n) {
            if (o->dgus[n] == 0.0) continue;
            const uint16_t* row = ws13 + (size_t)n * H;
            for (int h = 0; h < H; ++h) o->dx[h] += o->dgus[n] * (double)bf16_val(row[h]);
        }
    }
}

/*
 * Backward for selected outputs.  ids: the expert choice (ids_in if given,
 * else the forward's own routing of x).  dout [T,H] fp32.
 *   dx [n_tok, H] for the tokens tok_sel[0..n_tok-1];
 *   dwg [n_exp, H], dw13 [n_exp, 2I, H], dw2 [n_exp, H, I] for the experts
 *     exp_sel[0..n_exp-1] (any of them may be NULL);
 *   dws13 [2Is, H], dws2 [H, Is] if want_shared (they need every token).
 * ids_out [T,k] (optional) receives the choice used.  Sums over tokens run
 * in ascending token order.
 */
int orc_backward(const orc_cfg* c, int64_t T, const uint16_t* x, const uint16_t* wg, const float* bias,
                 const int32_t* ids_in, const uint16_t* w13, const uint16_t* w2, const uint16_t* ws13,
                 const uint16_t* ws2, const float* dout, const int64_t* tok_sel, int64_t n_tok,
                 const int32_t* exp_sel, int32_t n_exp, int32_t want_shared, int32_t round_gu, float* dx,
                 float* dwg, float* dw13, float* dw2, float* dws13, float* dws2, int32_t* ids_out) {
    if (!c || c->fp8 || c->k < 1 || c->k > c->E || T < 0) return 1;
    if (want_shared && c->Is == 0) return 1;
    const int H = c->H, E = c->E, k = c->k, I = c->I, Is = c->Is;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k > 0 ? T * k : 1));
    float* wdummy = (float*)malloc(sizeof(float) * (size_t)(T * k > 0 ? T * k : 1));
    if (orc_route(c, T, x, wg, bias, ids_in, ids, wdummy, NULL, NULL)) return 1;
    free(wdummy);
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)(T * k));
    int32_t* esel = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; ++e) esel[e] = -1;
    for (int i = 0; i < n_exp; ++i) esel[exp_sel[i]] = i;
    /* tokens whose backward is needed, in ascending order */
    int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
    for (int64_t t = 0; t < T; ++t) slot[t] = want_shared ? 1 : 0;
    for (int64_t i = 0; i < n_tok; ++i) slot[tok_sel[i]] = 1;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j)
            if (esel[ids[t * k + j]] >= 0) slot[t] = 1;
    int64_t n_need = 0;
    for (int64_t t = 0; t < T; ++t) slot[t] = slot[t] ? n_need++ : -1;
    const size_t per = (size_t)k * 2 * I + (size_t)k * I + 2 * (size_t)k + 3 * (size_t)Is + (size_t)H;
    double* store = (double*)calloc((size_t)(n_need > 0 ? n_need : 1) * per, sizeof(double));
    tok_grads* tg = (tok_grads*)malloc(sizeof(tok_grads) * (size_t)(n_need > 0 ? n_need : 1));
    for (int64_t i = 0; i < n_need; ++i) {
        double* b = store + (size_t)i * per;
        tg[i].dgu = b; b += (size_t)k * 2 * I;
        tg[i].h = b; b += (size_t)k * I;
        tg[i].w = b; b += k;
        tg[i].da = b; b += k;
        tg[i].dgus = b; b += 2 * (size_t)Is;
        tg[i].hs = b; b += Is;
        tg[i].dx = b;
    }
    const int wide = I > Is ? I : Is;
#pragma omp parallel
    {
        double* xb = (double*)malloc(sizeof(double) * (size_t)H);
        double* buf = (double*)malloc(sizeof(double) * ((size_t)2 * k + 3 * (size_t)wide + (size_t)H));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            if (slot[t] < 0) continue;
            for (int h = 0; h < H; ++h) xb[h] = bf16_val(x[t * H + h]);
            token_backward(c, xb, wg, ids + t * k, w13, w2, ws13, ws2, dout + t * H, &tg[slot[t]], buf, round_gu);
        }
        free(xb);
        free(buf);
    }
    if (dx)
        for (int64_t i = 0; i < n_tok; ++i)
            for (int h = 0; h < H; ++h) dx[i * H + h] = (float)tg[slot[tok_sel[i]]].dx[h];
    /* weight gradients of the selected experts: one output row per task */
    if (n_exp > 0 && (dw13 || dw2 || dwg)) {
#pragma omp parallel
        {
            double* acc = (double*)malloc(sizeof(double) * (size_t)H);
            double* acc2 = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 4)
            for (int64_t task = 0; task < (int64_t)n_exp * (2 * I + H + 1); ++task) {
                const int q = (int)(task / (2 * I + H + 1));
                const int r = (int)(task % (2 * I + H + 1));
                const int e = exp_sel[q];
                if (r < 2 * I) {                 /* dW13_e row r */
                    if (!dw13) continue;
                    for (int h = 0; h < H; ++h) acc[h] = 0.0;
                    for (int64_t t = 0; t < T; ++t)
                        for (int j = 0; j < k; ++j)
                            if (ids[t * k + j] == e) {
                                const double gv = tg[slot[t]].dgu[(size_t)j * 2 * I + r];
                                if (gv == 0.0) continue;
                                for (int h = 0; h < H; ++h) acc[h] += gv * (double)bf16_val(x[t * H + h]);
                            }
                    float* o = dw13 + ((size_t)q * 2 * I + r) * H;
                    for (int h = 0; h < H; ++h) o[h] = (float)acc[h];
                } else if (r < 2 * I + H) {      /* dW2_e row h */
                    if (!dw2) continue;
                    const int hh = r - 2 * I;
                    for (int i = 0; i < I; ++i) acc2[i] = 0.0;
                    for (int64_t t = 0; t < T; ++t)
                        for (int j = 0; j < k; ++j)
                            if (ids[t * k + j] == e) {
                                const double dy = tg[slot[t]].w[j] * (double)dout[t * H + hh];
                                const double* hv = tg[slot[t]].h + (size_t)j * I;
                                for (int i = 0; i < I; ++i) acc2[i] += dy * hv[i];
                            }
                    float* o = dw2 + ((size_t)q * H + hh) * I;
                    for (int i = 0; i < I; ++i) o[i] = (float)acc2[i];
                } else {                         /* router row e */
                    if (!dwg) continue;
                    for (int h = 0; h < H; ++h) acc[h] = 0.0;
                    for (int64_t t = 0; t < T; ++t)
                        for (int j = 0; j < k; ++j)
                            if (ids[t * k + j] == e) {
                                const double d = tg[slot[t]].da[j];
                                for (int h = 0; h < H; ++h) acc[h] += d * (double)bf16_val(x[t * H + h]);
                            }
                    for (int h = 0; h < H; ++h) dwg[(size_t)q * H + h] = (float)acc[h];
                }
            }
            free(acc);
            free(acc2);
        }
    }
    if (want_shared) {
#pragma omp parallel
        {
            double* acc = (double*)malloc(sizeof(double) * (size_t)(H > Is ? H : Is));
#pragma omp for schedule(dynamic, 4)
            for (int64_t task = 0; task < 2 * (int64_t)Is + H; ++task) {
                if (task < 2 * Is) {
                    const int n = (int)task;
                    for (int h = 0; h < H; ++h) acc[h] = 0.0;
                    for (int64_t t = 0; t < T; ++t) {
                        const double gv = tg[slot[t]].dgus[n];
                        if (gv == 0.0) continue;
                        for (int h = 0; h < H; ++h) acc[h] += gv * (double)bf16_val(x[t * H + h]);
                    }
                    for (int h = 0; h < H; ++h) dws13[(size_t)n * H + h] = (float)acc[h];
                } else {
                    const int hh = (int)(task - 2 * Is);
                    for (int i = 0; i < Is; ++i) acc[i] = 0.0;
                    for (int64_t t = 0; t < T; ++t) {
                        const double d = (double)dout[t * H + hh];
                        const double* hv = tg[slot[t]].hs;
                        for (int i = 0; i < Is; ++i) acc[i] += d * hv[i];
                    }
                    for (int i = 0; i < Is; ++i) dws2[(size_t)hh * Is + i] = (float)acc[i];
                }
            }
            free(acc);
        }
    }
    free(store);
    free(tg);
    free(slot);
    free(esel);
    free(ids);
    return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
