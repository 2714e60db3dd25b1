/*
 * oracle.c - plain, slow CPU oracle of the Llama-2 single-token decode step
 * (llama2.c run.c in fp32, runq.c in Q8_0).
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or constant with the GPU library, and parses the weight blob
 * with its own code.
 *
 * Precision. Every tensor the model stores (weights, KV cache, the residual
 * stream and each activation vector handed from one step to the next) is
 * fp32, as in the pages' C engine (the KV cache is an array of float, gitcode
 * porting guide, section "memory optimisation"). Every reduction (sum of
 * squares, dot products, softmax max/sum, the attention weighted sum, the
 * Q8_0 group combine) runs in fp64 and is rounded to fp32 where the model
 * stores the value. Two places run in fp32 because the pages fix them
 * there: the RoPE angle pos*freq and its cosf/sinf (Karpathy tech notes, Q&A
 * page, question on RoPE in C versus PyTorch), and the Q8_0 quantiser
 * (gitcode porting guide, section "1. INT8 quantisation", the quantize
 * listing), where a float max, a float division by 127 and a rounding of a
 * float quotient decide the integer codes.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no -Ofast / -ffast-math: the
 * gitcode guide's Makefile section notes that -Ofast trades precision).
 * Rows of every matvec are split over OpenMP threads; the summation order
 * inside a row is fixed, so results do not depend on the thread count.
 *
 * Readings of the pages where they are silent (each also listed in the design
 * notes): RMSNorm y = g * x / sqrt(mean(x^2) + 1e-5); RoPE rotates interleaved
 * pairs (2j, 2j+1) of each q and k head by pos * 10000^(-2j/hs); attention
 * scores are scaled by 1/sqrt(head_size); query head h reads kv head
 * h / (n_heads / n_kv_heads); SwiGLU is silu(w1 x) * (w3 x); pre-norm
 * residuals; an all-zero Q8_0 group gets scale 0 and codes 0; argmax ties go
 * to the lowest index.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_Q8_0 1
#define OR_Q4_0 2

#define OR_OK 0
#define OR_EINVAL -1
#define OR_EFORMAT -2
#define OR_ENOMEM -3

typedef struct {
    int32_t dim, hidden_dim, n_layers, n_heads, n_kv_heads, vocab_size, seq_len;
} or_config;

/* one matrix: fp32 values, Q8_0 codes, or Q4_0 packed codes (two per
   byte), with one fp32 scale per gs elements */
typedef struct {
    const float* f;
    const int8_t* q;
    const uint8_t* p;
    const float* s;
} or_mat;

typedef struct {
    or_config c;
    int dtype, gs;
    int64_t d, h, L, V, S, nh, nkv, hs, kvd, kvmul;
    or_mat emb, wq, wk, wv, wo, w1, w2, w3, wcls;
    const float *rms_att, *rms_ffn, *rms_final;
    float* kc; /* [L][S][kvd] */
    float* vc;
    /* activations, fp32 as stored by the model */
    float *x, *xb, *q, *k, *v, *o, *y, *h1, *h3, *hb, *logits;
    int8_t* aq; /* quantised activation codes (Q8_0 path) */
    float* as;
    /* trace of one layer's quantised matvec inputs (Q8_0 path) */
    int trace_layer;
    int64_t trace_at; /* layer whose inputs the matvecs record */
    int8_t* tq[4];
    float* ts[4];
    float* tf[4];
} or_model;

/* ---------------------------------------------------------------- parsing */

static int64_t i64abs(int64_t v) { return v < 0 ? -v : v; }

static int take(const uint8_t** p, const uint8_t* end, int64_t bytes, const void** out)
{
    if (bytes < 0 || (int64_t)(end - *p) < bytes) return 0;
    *out = *p;
    *p += bytes;
    return 1;
}

static int take_mat(or_model* m, const uint8_t** p, const uint8_t* end, int64_t n, or_mat* w)
{
    const void* a;
    memset(w, 0, sizeof(*w));
    if (m->dtype == OR_F32) {
        if (!take(p, end, 4 * n, &a)) return 0;
        w->f = (const float*)a;
    } else if (m->dtype == OR_Q8_0) {
        if (!take(p, end, n, &a)) return 0;
        w->q = (const int8_t*)a;
        if (!take(p, end, 4 * (n / m->gs), &a)) return 0;
        w->s = (const float*)a;
    } else {
        if (!take(p, end, n / 2, &a)) return 0;
        w->p = (const uint8_t*)a;
        if (!take(p, end, 4 * (n / 32), &a)) return 0;
        w->s = (const float*)a;
    }
    return 1;
}

/*
 * Open a model over a blob (borrowed, must outlive the model).
 * Header: seven int32 config fields, then the arrays in the llama2.c order
 * (pomoai.com hub page, data-format section). vocab_size < 0 means the
 * classifier is a separate array after the legacy tables (Karpathy tech
 * notes, Q&A page, shared_weights question). The two legacy freq_cis tables,
 * seq_len*head_size/2 floats each, are skipped (same Q&A page, question on
 * skipping freq_cis in memory_map_weights).
 * dtype OR_Q4_0 (gs must be 32) reads the 4-bit variant as a whole model:
 * every matrix, the embedding included, is stored as packed Q4_0 codes
 * [n/2] followed by fp32 scales [n/32] (the group layout described at
 * or_quantize_q40); every matvec quantises its input to Q8_0 with groups of
 * 32 (W4A8, the Q8_0 scheme with 4-bit weights); norm gains, legacy tables,
 * KV cache and activations stay fp32.
 */
int or_open(const void* blob, int64_t nbytes, int dtype, int gs, or_model** out)
{
    *out = NULL;
    if (!blob || nbytes < 28 || (dtype != OR_F32 && dtype != OR_Q8_0 && dtype != OR_Q4_0)) return OR_EINVAL;
    or_model* m = (or_model*)calloc(1, sizeof(or_model));
    if (!m) return OR_ENOMEM;
    memcpy(&m->c, blob, 28);
    m->dtype = dtype;
    m->gs = gs;
    m->d = m->c.dim;
    m->h = m->c.hidden_dim;
    m->L = m->c.n_layers;
    m->nh = m->c.n_heads;
    m->nkv = m->c.n_kv_heads;
    m->V = i64abs(m->c.vocab_size);
    m->S = m->c.seq_len;
    if (m->d <= 0 || m->h <= 0 || m->L <= 0 || m->nh <= 0 || m->nkv <= 0 || m->V <= 0 ||
        m->S <= 0 || m->d % m->nh || m->nh % m->nkv || (m->d / m->nh) % 2) {
        free(m);
        return OR_EINVAL;
    }
    m->hs = m->d / m->nh;
    m->kvd = m->nkv * m->hs;
    m->kvmul = m->nh / m->nkv;
    if (dtype == OR_Q8_0 && (gs <= 0 || m->d % gs || m->h % gs)) {
        free(m);
        return OR_EINVAL;
    }
    /* Q4_0 model: every matrix stored as 4-bit groups of 32 (the reading
       below), every matvec input quantised to Q8_0 with the same groups */
    if (dtype == OR_Q4_0 && (gs != 32 || m->d % 32 || m->h % 32)) {
        free(m);
        return OR_EINVAL;
    }
    const uint8_t* p = (const uint8_t*)blob + 28;
    const uint8_t* end = (const uint8_t*)blob + nbytes;
    const void* a;
    int64_t d = m->d, h = m->h, L = m->L, kvd = m->kvd;
    int ok = take_mat(m, &p, end, m->V * d, &m->emb);
    ok = ok && take(&p, end, 4 * L * d, &a);
    if (ok) m->rms_att = (const float*)a;
    ok = ok && take_mat(m, &p, end, L * d * d, &m->wq);
    ok = ok && take_mat(m, &p, end, L * kvd * d, &m->wk);
    ok = ok && take_mat(m, &p, end, L * kvd * d, &m->wv);
    ok = ok && take_mat(m, &p, end, L * d * d, &m->wo);
    ok = ok && take(&p, end, 4 * L * d, &a);
    if (ok) m->rms_ffn = (const float*)a;
    ok = ok && take_mat(m, &p, end, L * h * d, &m->w1);
    ok = ok && take_mat(m, &p, end, L * d * h, &m->w2);
    ok = ok && take_mat(m, &p, end, L * h * d, &m->w3);
    ok = ok && take(&p, end, 4 * d, &a);
    if (ok) m->rms_final = (const float*)a;
    ok = ok && take(&p, end, 4 * m->S * (m->hs / 2), &a); /* legacy freq_cis_real */
    ok = ok && take(&p, end, 4 * m->S * (m->hs / 2), &a); /* legacy freq_cis_imag */
    if (ok) {
        if (m->c.vocab_size > 0)
            m->wcls = m->emb;
        else
            ok = take_mat(m, &p, end, m->V * d, &m->wcls);
    }
    if (!ok || p != end) {
        free(m);
        return OR_EFORMAT;
    }
    int64_t kvn = L * m->S * kvd;
    m->kc = (float*)calloc((size_t)kvn, sizeof(float));
    m->vc = (float*)calloc((size_t)kvn, sizeof(float));
    int64_t big = d > h ? d : h;
    m->x = (float*)calloc(d, 4);
    m->xb = (float*)calloc(d, 4);
    m->q = (float*)calloc(d, 4);
    m->k = (float*)calloc(kvd, 4);
    m->v = (float*)calloc(kvd, 4);
    m->o = (float*)calloc(d, 4);
    m->y = (float*)calloc(d, 4);
    m->h1 = (float*)calloc(h, 4);
    m->h3 = (float*)calloc(h, 4);
    m->hb = (float*)calloc(h, 4);
    m->logits = (float*)calloc(m->V, 4);
    m->aq = (int8_t*)calloc(big, 1);
    m->as = (float*)calloc(big, 4);
    m->trace_layer = -1;
    if (!m->kc || !m->vc || !m->x || !m->xb || !m->q || !m->k || !m->v || !m->o || !m->y ||
        !m->h1 || !m->h3 || !m->hb || !m->logits || !m->aq || !m->as) {
        /* leak-free enough for a test oracle: release what exists */
        free(m->kc); free(m->vc); free(m->x); free(m->xb); free(m->q); free(m->k);
        free(m->v); free(m->o); free(m->y); free(m->h1); free(m->h3); free(m->hb);
        free(m->logits); free(m->aq); free(m->as); free(m);
        return OR_ENOMEM;
    }
    *out = m;
    return OR_OK;
}

void or_close(or_model* m)
{
    if (!m) return;
    free(m->kc); free(m->vc); free(m->x); free(m->xb); free(m->q); free(m->k);
    free(m->v); free(m->o); free(m->y); free(m->h1); free(m->h3); free(m->hb);
    free(m->logits); free(m->aq); free(m->as);
    for (int i = 0; i < 4; i++) { free(m->tq[i]); free(m->ts[i]); free(m->tf[i]); }
    free(m);
}

void or_reset_kv(or_model* m)
{
    int64_t kvn = m->L * m->S * m->kvd;
    memset(m->kc, 0, (size_t)kvn * 4);
    memset(m->vc, 0, (size_t)kvn * 4);
}

float* or_key_cache(or_model* m) { return m->kc; }
float* or_value_cache(or_model* m) { return m->vc; }
float* or_logits(or_model* m) { return m->logits; }
float* or_residual(or_model* m) { return m->x; }
/* the last layer's attention output o (n_heads*head_size) of the last forward */
float* or_attn_out(or_model* m) { return m->o; }

void or_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int or_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------- the method */

/*
 * Q8_0 (definition from the gitcode porting guide, section "1. INT8
 * quantisation", and the hub page's quantisation section): a vector is cut
 * into groups of gs consecutive values; a group stores one fp32 scale and gs
 * int8 codes, and value i of the group stands for code_i * scale.
 *
 * The scale is the group's largest magnitude divided by 127 (an fp32
 * division), so the largest value maps to +-127.
 */
static float q80_scale_of(const float* v, int gs)
{
    float amax = 0.0f;
    for (int i = 0; i < gs; i++)
        if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
    return amax / 127.0f;
}

/*
 * A code is the nearest integer to the fp32 quotient value / scale, halves
 * rounded away from zero (C's round). A group of zeros has scale 0; its codes
 * are 0 (the quotient would be 0/0).
 */
static int8_t q80_code_of(float v, float scale)
{
    if (scale == 0.0f) return 0;
    const float quotient = v / scale;
    return (int8_t)roundf(quotient);
}

/* Quantise n values (n a multiple of gs): codes q[n], scales s[n/gs]. */
int or_quantize(const float* x, int64_t n, int gs, int8_t* q, float* s)
{
    if (gs <= 0 || n < 0 || n % gs) return OR_EINVAL;
    const int64_t groups = n / gs;
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < groups; g++) {
        const float* v = x + g * gs;
        const float scale = q80_scale_of(v, gs);
        s[g] = scale;
        for (int i = 0; i < gs; i++) q[g * gs + i] = q80_code_of(v[i], scale);
    }
    return OR_OK;
}

/*
 * RMSNorm (pomoai.com hub page, architecture list; it replaces LayerNorm):
 * out_i = g_i * x_i / sqrt(sum(x^2)/n + eps), eps = 1e-5, in fp64, stored fp32.
 */
static void rmsnorm(float* out, const float* x, const float* g, int64_t n)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; i++) ss += (double)x[i] * (double)x[i];
    double r = 1.0 / sqrt(ss / (double)n + 1e-5);
    for (int64_t i = 0; i < n; i++) out[i] = (float)((double)g[i] * ((double)x[i] * r));
}

/*
 * Matrix-vector product out = W x with W row-major [rows][cols] (the
 * hand-written matmul the ainews article's technical section describes; the
 * toy forward pass of the mht18 essay, section 2.3, ends with one).
 * fp32: fp64 dot of fp32 values, stored fp32.
 * Q8_0: x is first quantised (int8 activations; the Q&A page explains the
 * int8 speed-up by integer multiply-adds); per group the int8 dot is exact
 * in integers, then scaled by the weight and activation scales and summed
 * in fp64.
 */
static void matvec_f32_rows(float* out, const float* x, const float* W, int64_t rows, int64_t cols)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; i++) {
        const float* wr = W + i * cols;
        double acc = 0.0;
        for (int64_t j = 0; j < cols; j++) acc += (double)wr[j] * (double)x[j];
        out[i] = (float)acc;
    }
}

static void matvec_q80_rows(float* out, const int8_t* aq, const float* as, const int8_t* Q,
                            const float* S, int64_t rows, int64_t cols, int gs)
{
    int64_t ng = cols / gs;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; i++) {
        const int8_t* qr = Q + i * cols;
        const float* sr = S + i * ng;
        double acc = 0.0;
        for (int64_t g = 0; g < ng; g++) {
            int64_t dot = 0;
            for (int j = 0; j < gs; j++) dot += (int64_t)qr[g * gs + j] * (int64_t)aq[g * gs + j];
            acc += (double)dot * (double)sr[g] * (double)as[g];
        }
        out[i] = (float)acc;
    }
}

static void matvec_q40_rows(float* out, const int8_t* aq, const float* as, const uint8_t* Q,
                            const float* S, int64_t rows, int64_t cols);

static void matvec(or_model* m, float* out, const float* x, const or_mat* w, int64_t woff,
                   int64_t rows, int64_t cols, int trace_slot)
{
    if (m->dtype == OR_F32) {
        matvec_f32_rows(out, x, w->f + woff, rows, cols);
        return;
    }
    if (m->dtype == OR_Q4_0) {
        or_quantize(x, cols, 32, m->aq, m->as);
        matvec_q40_rows(out, m->aq, m->as, w->p + woff / 2, w->s + woff / 32, rows, cols);
        return;
    }
    int gs = m->gs;
    or_quantize(x, cols, gs, m->aq, m->as);
    if (trace_slot >= 0) {
        const int64_t off = m->trace_at * cols;
        memcpy(m->tq[trace_slot] + off, m->aq, (size_t)cols);
        memcpy(m->ts[trace_slot] + off / gs, m->as, (size_t)(cols / gs) * 4);
        memcpy(m->tf[trace_slot] + off, x, (size_t)cols * 4);
    }
    matvec_q80_rows(out, m->aq, m->as, w->q + woff, w->s + woff / gs, rows, cols, gs);
}

/* standalone fp32 matvec out = W x (the same loop the model uses) */
int or_matvec_f32(const float* W, const float* x, int64_t rows, int64_t cols, float* out)
{
    if (rows < 0 || cols < 0) return OR_EINVAL;
    matvec_f32_rows(out, x, W, rows, cols);
    return OR_OK;
}

/* standalone Q8_0 matvec: x is quantised first, as in the model */
int or_matvec_q80(const int8_t* Q, const float* S, const float* x, int64_t rows, int64_t cols,
                  int gs, float* out)
{
    if (gs <= 0 || cols % gs || rows < 0) return OR_EINVAL;
    int8_t* aq = (int8_t*)malloc((size_t)cols);
    float* as = (float*)malloc((size_t)(cols / gs + 1) * 4);
    if (!aq || !as) { free(aq); free(as); return OR_ENOMEM; }
    or_quantize(x, cols, gs, aq, as);
    matvec_q80_rows(out, aq, as, Q, S, rows, cols, gs);
    free(aq);
    free(as);
    return OR_OK;
}

/*
 * ---- 4-bit group quantisation ("Q4_0"). The ainews article (technical
 * deep dive, benchmark and comparison tables) names a 4-bit Q4_0 variant of
 * the engine in a llama.cpp-like format, and the gitcode guide (future
 * optimisation directions) lists 4-bit quantisation after llama.cpp's
 * format as a next step; neither gives the layout. Reading, in the manner of the
 * gitcode guide's Q8_0 listing: groups of 32 values; m is the group's value
 * of largest magnitude (the first one among equal magnitudes); the scale is
 * the fp32 quotient m / -8 (0 for an all-zero group); a code is the fp32
 * quotient x / scale rounded half away from zero and clamped to [-8, 7]
 * (the value m itself maps to -8). Storage per group: 16 bytes, byte b
 * holding code b + 8 in its low nibble and code b + 16 + 8 in its high
 * nibble; the fp32 scales follow as a separate array.
 * A Q4_0 matvec quantises its input to Q8_0 with the same 32-value groups
 * (the W8A8 scheme above with 4-bit weights): each group contributes the
 * exact int32 dot of its codes times the weight scale times the input
 * scale, summed over the groups in fp64.
 */
int or_quantize_q40(const float* x, int64_t n, uint8_t* q, float* s)
{
    if (n < 0 || n % 32) return OR_EINVAL;
    for (int64_t g = 0; g < n / 32; g++) {
        const float* xg = x + g * 32;
        float amax = 0.0f, m = 0.0f;
        for (int i = 0; i < 32; i++) {
            const float a = fabsf(xg[i]);
            if (a > amax) {
                amax = a;
                m = xg[i];
            }
        }
        const float scale = amax == 0.0f ? 0.0f : m / -8.0f;
        s[g] = scale;
        int c[32];
        for (int i = 0; i < 32; i++) {
            int v = 0;
            if (scale != 0.0f) {
                const float r = roundf(xg[i] / scale);
                v = r < -8.0f ? -8 : r > 7.0f ? 7 : (int)r;
            }
            c[i] = v;
        }
        for (int b = 0; b < 16; b++) q[g * 16 + b] = (uint8_t)((c[b] + 8) | ((c[b + 16] + 8) << 4));
    }
    return OR_OK;
}

/* the int32 group dot of 32 packed 4-bit weight codes with 32 int8 input codes */
static int32_t q40_group_dot(const uint8_t* w, const int8_t* xq)
{
    int32_t dot = 0;
    for (int b = 0; b < 16; b++) {
        dot += ((int32_t)(w[b] & 15) - 8) * (int32_t)xq[b];
        dot += ((int32_t)(w[b] >> 4) - 8) * (int32_t)xq[b + 16];
    }
    return dot;
}

int or_group_dots_q40(const uint8_t* wq, const int8_t* xq, int64_t cols, int32_t* out)
{
    if (cols % 32) return OR_EINVAL;
    for (int64_t g = 0; g < cols / 32; g++) out[g] = q40_group_dot(wq + g * 16, xq + g * 32);
    return OR_OK;
}

/* rows of a Q4_0 matvec over already quantised input codes aq / scales as */
static void matvec_q40_rows(float* out, const int8_t* aq, const float* as, const uint8_t* Q,
                            const float* S, int64_t rows, int64_t cols)
{
    const int64_t ng = cols / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; i++) {
        const uint8_t* qr = Q + i * (cols / 2);
        const float* sr = S + i * ng;
        double acc = 0.0;
        for (int64_t g = 0; g < ng; g++)
            acc += (double)q40_group_dot(qr + g * 16, aq + g * 32) * (double)sr[g] * (double)as[g];
        out[i] = (float)acc;
    }
}

/* Q4_0 matvec: Q packed [rows][cols/2], S [rows][cols/32]; x quantised first */
int or_matvec_q40(const uint8_t* Q, const float* S, const float* x, int64_t rows, int64_t cols, float* out)
{
    if (cols % 32 || rows < 0) return OR_EINVAL;
    int8_t* aq = (int8_t*)malloc((size_t)cols + 1);
    float* as = (float*)malloc((size_t)(cols / 32 + 1) * 4);
    if (!aq || !as) {
        free(aq);
        free(as);
        return OR_ENOMEM;
    }
    or_quantize(x, cols, 32, aq, as);
    matvec_q40_rows(out, aq, as, Q, S, rows, cols);
    free(aq);
    free(as);
    return OR_OK;
}

/* the int32 group dot products of one Q8_0 matvec row: out[g] for g < cols/gs */
int or_group_dots(const int8_t* wq, const int8_t* xq, int64_t cols, int gs, int32_t* out)
{
    if (gs <= 0 || cols % gs) return OR_EINVAL;
    for (int64_t g = 0; g < cols / gs; g++) {
        int64_t dot = 0;
        for (int j = 0; j < gs; j++) dot += (int64_t)wq[g * gs + j] * (int64_t)xq[g * gs + j];
        out[g] = (int32_t)dot;
    }
    return OR_OK;
}

/*
 * RoPE computed on the fly (Karpathy tech notes, Q&A page, question on RoPE
 * in C versus PyTorch: the C engine evaluates cosf/sinf of pos*freq in every
 * forward instead of reading a table). Reading: within each head the pairs
 * (2j, 2j+1) rotate by pos * freq_j, freq_j = 10000^(-2j/hs) (computed in
 * fp64, rounded to fp32), angle = (float)pos * freq_j in fp32; cosf and sinf
 * are taken as the fp32 cosine and sine of that fp32 angle, correctly
 * rounded (the fp64 value rounded to fp32), so the result does not depend on
 * one libm's last-bit behaviour; the rotation runs in fp64 and is stored fp32.
 */
static void rope(float* vec, int64_t nheads, int64_t hs, int pos)
{
    for (int64_t hd = 0; hd < nheads; hd++) {
        float* hv = vec + hd * hs;
        for (int64_t j = 0; j < hs / 2; j++) {
            float freq = (float)pow(10000.0, -(double)(2 * j) / (double)hs);
            float ang = (float)pos * freq;
            double c = (double)(float)cos((double)ang), sn = (double)(float)sin((double)ang);
            double a = hv[2 * j], b = hv[2 * j + 1];
            hv[2 * j] = (float)(a * c - b * sn);
            hv[2 * j + 1] = (float)(a * sn + b * c);
        }
    }
}

/* the fp32 frequency table the rope above uses (exposed for tests) */
void or_rope_freqs(int64_t hs, float* out)
{
    for (int64_t j = 0; j < hs / 2; j++) out[j] = (float)pow(10000.0, -(double)(2 * j) / (double)hs);
}

/* apply rope to an arbitrary vector of nheads heads (exposed for tests) */
void or_rope(float* vec, int64_t nheads, int64_t hs, int pos) { rope(vec, nheads, hs, pos); }

/*
 * Attention of one layer over cached positions 0..pos (Karpathy tech notes,
 * Q&A page: the KV-cache question places k, v of position pos at offset
 * loff + pos*kv_dim; the GQA question gives q n_heads*head_size and k, v
 * n_kv_heads*head_size, query heads sharing a kv head). For query head hd
 * and kv head g = hd / kvmul: score_t = q.k_t / sqrt(hs); a = softmax(score);
 * o = sum_t a_t v_t. All in fp64, o stored fp32.
 */
static void attention(or_model* m, int64_t l, int pos)
{
    int64_t hs = m->hs, kvd = m->kvd;
    const float* kl = m->kc + l * m->S * kvd;
    const float* vl = m->vc + l * m->S * kvd;
    double scale = 1.0 / sqrt((double)hs);
    #pragma omp parallel for schedule(static)
    for (int64_t hd = 0; hd < m->nh; hd++) {
        int64_t g = hd / m->kvmul;
        const float* qh = m->q + hd * hs;
        double* sc = (double*)malloc(sizeof(double) * (size_t)(pos + 1));
        double mx = -INFINITY;
        for (int64_t t = 0; t <= pos; t++) {
            const float* kt = kl + t * kvd + g * hs;
            double dot = 0.0;
            for (int64_t i = 0; i < hs; i++) dot += (double)qh[i] * (double)kt[i];
            sc[t] = dot * scale;
            if (sc[t] > mx) mx = sc[t];
        }
        double z = 0.0;
        for (int64_t t = 0; t <= pos; t++) {
            sc[t] = exp(sc[t] - mx);
            z += sc[t];
        }
        /* o_i = sum over t = 0..pos of a_t v_t[i], each sum taken in
           increasing t; the cached rows are read one at a time */
        double* acc = (double*)calloc((size_t)hs, sizeof(double));
        for (int64_t t = 0; t <= pos; t++) {
            const float* vt = vl + t * kvd + g * hs;
            for (int64_t i = 0; i < hs; i++) acc[i] += sc[t] * (double)vt[i];
        }
        for (int64_t i = 0; i < hs; i++) m->o[hd * hs + i] = (float)(acc[i] / z);
        free(acc);
        free(sc);
    }
}

/* residual add x += y, the sum of two stored fp32 vectors, stored fp32 */
static void residual(float* x, const float* y, int64_t n)
{
    for (int64_t i = 0; i < n; i++) x[i] = (float)((double)x[i] + (double)y[i]);
}

/* first index of the largest value (sample_argmax in the gitcode guide's
   embedded main loop); ties go to the lowest index */
int or_argmax(const float* v, int64_t n)
{
    int64_t best = 0;
    for (int64_t i = 1; i < n; i++)
        if (v[i] > v[best]) best = i;
    return (int)best;
}

/* ---- temperature sampling (mht18 essay, section 3.2: the logits go through
   a softmax and the next token is a random draw from that distribution,
   the temperature scaling the logits first; temperature 0 is the greedy
   argmax above).
   Draws: output k of the splitmix64 stream seeded with `seed` (Steele, Lea,
   Flood 2014: state seed + k * 0x9E3779B97F4A7C15 through their finaliser),
   as a uniform on (0, 1): ((bits >> 11) + 1/2) * 2^-53, exact in fp64.
   The draw from softmax(logit / T) is taken by the Gumbel-max rule (Gumbel
   1954; the argmax of logit_i / T + g_i with independent standard Gumbel
   g_i = -log(-log(u_i)) is distributed as softmax(logit / T)): scores in
   fp64, compared after rounding to fp32, ties to the lowest index. Token i at
   position pos uses draw k = pos * n + i + 1. */
uint64_t or_splitmix64(uint64_t seed, uint64_t k)
{
    uint64_t z = seed + k * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

double or_uniform(uint64_t seed, uint64_t k)
{
    return ((double)(or_splitmix64(seed, k) >> 11) + 0.5) * 0x1.0p-53;
}

/* the fp32 score of token i (for the tests' tie margins) */
float or_sample_score(float logit, double temperature, uint64_t seed, int64_t pos, int64_t n, int64_t i)
{
    const double u = or_uniform(seed, (uint64_t)pos * (uint64_t)n + (uint64_t)i + 1u);
    const double g = -log(-log(u));
    return (float)((double)logit / temperature + g);
}

int or_sample(const float* logits, int64_t n, double temperature, uint64_t seed, int64_t pos)
{
    if (temperature == 0.0) return or_argmax(logits, n);
    int64_t best = 0;
    float bv = or_sample_score(logits[0], temperature, seed, pos, n, 0);
    for (int64_t i = 1; i < n; i++) {
        const float s = or_sample_score(logits[i], temperature, seed, pos, n, i);
        if (s > bv) {
            bv = s;
            best = i;
        }
    }
    return (int)best;
}

/* trace buffers hold every layer: slot s of layer l at offset l * size(s) */
static int64_t trace_size(const or_model* m, int slot) { return slot == 3 ? m->h : m->d; }

static void trace_alloc(or_model* m)
{
    for (int i = 0; i < 4; i++) {
        if (!m->tq[i]) {
            int64_t n = m->L * trace_size(m, i);
            m->tq[i] = (int8_t*)calloc(n, 1);
            m->ts[i] = (float*)calloc(n, 4);
            m->tf[i] = (float*)calloc(n, 4);
        }
    }
}

/* record the quantised inputs of layer l's four matvecs (Q8_0 only):
   slot 0 QKV input, 1 output-projection input, 2 W1/W3 input, 3 W2 input;
   l = -2 records every layer, l = -1 stops */
void or_trace_layer(or_model* m, int l)
{
    m->trace_layer = l;
    if (l >= 0 || l == -2) trace_alloc(m);
}

static int64_t trace_off(const or_model* m, int layer, int slot)
{
    return (int64_t)(layer < 0 ? 0 : layer) * trace_size(m, slot);
}

int8_t* or_trace_codes(or_model* m, int slot) { return m->tq[slot] + trace_off(m, m->trace_layer, slot); }
float* or_trace_scales(or_model* m, int slot)
{
    return m->ts[slot] + trace_off(m, m->trace_layer, slot) / m->gs;
}
float* or_trace_input(or_model* m, int slot) { return m->tf[slot] + trace_off(m, m->trace_layer, slot); }
int8_t* or_trace_codes_at(or_model* m, int layer, int slot) { return m->tq[slot] + trace_off(m, layer, slot); }
float* or_trace_scales_at(or_model* m, int layer, int slot)
{
    return m->ts[slot] + trace_off(m, layer, slot) / m->gs;
}
float* or_trace_input_at(or_model* m, int layer, int slot) { return m->tf[slot] + trace_off(m, layer, slot); }

/*
 * One decode step: token at position pos -> logits[V]; writes KV slot pos.
 * Order of the step (pomoai.com hub page architecture list; Q&A page on the
 * KV cache, GQA and RoPE; mht18 essay section 2.3): embedding row; per layer
 * pre-norm attention block (RMSNorm, q/k/v matvecs, RoPE on q and k, K/V
 * cache write, attention, output matvec, residual) and pre-norm SwiGLU block
 * (RMSNorm, w1 and w3 matvecs, silu(w1 x) * w3 x, w2 matvec, residual); final
 * RMSNorm; classifier matvec (the embedding table when vocab_size > 0).
 */
int or_forward(or_model* m, int token, int pos)
{
    if (token < 0 || token >= m->V || pos < 0 || pos >= m->S) return OR_EINVAL;
    int64_t d = m->d, h = m->h, kvd = m->kvd, hs = m->hs;

    /* embedding row; Q8_0 and Q4_0 dequantise it (code times its group scale) */
    if (m->dtype == OR_F32) {
        memcpy(m->x, m->emb.f + (int64_t)token * d, (size_t)d * 4);
    } else if (m->dtype == OR_Q4_0) {
        const uint8_t* pr = m->emb.p + (int64_t)token * d / 2;
        const float* sr = m->emb.s + (int64_t)token * d / 32;
        for (int64_t i = 0; i < d; i++) {
            const int64_t g = i / 32, j = i % 32;
            const uint8_t b = pr[g * 16 + j % 16];
            const int code = (j < 16 ? (b & 15) : (b >> 4)) - 8;
            m->x[i] = (float)((double)code * (double)sr[g]);
        }
    } else {
        const int8_t* qr = m->emb.q + (int64_t)token * d;
        const float* sr = m->emb.s + (int64_t)token * d / m->gs;
        for (int64_t i = 0; i < d; i++)
            m->x[i] = (float)((double)qr[i] * (double)sr[i / m->gs]);
    }

    for (int64_t l = 0; l < m->L; l++) {
        int tr = (m->dtype == OR_Q8_0 && (m->trace_layer == (int)l || m->trace_layer == -2));
        m->trace_at = l;
        rmsnorm(m->xb, m->x, m->rms_att + l * d, d);
        matvec(m, m->q, m->xb, &m->wq, l * d * d, d, d, tr ? 0 : -1);
        matvec(m, m->k, m->xb, &m->wk, l * kvd * d, kvd, d, -1);
        matvec(m, m->v, m->xb, &m->wv, l * kvd * d, kvd, d, -1);
        rope(m->q, m->nh, hs, pos);
        rope(m->k, m->nkv, hs, pos);
        float* kslot = m->kc + (l * m->S + pos) * kvd;
        float* vslot = m->vc + (l * m->S + pos) * kvd;
        memcpy(kslot, m->k, (size_t)kvd * 4);
        memcpy(vslot, m->v, (size_t)kvd * 4);
        attention(m, l, pos);
        matvec(m, m->y, m->o, &m->wo, l * d * d, d, d, tr ? 1 : -1);
        residual(m->x, m->y, d);

        rmsnorm(m->xb, m->x, m->rms_ffn + l * d, d);
        matvec(m, m->h1, m->xb, &m->w1, l * h * d, h, d, tr ? 2 : -1);
        matvec(m, m->h3, m->xb, &m->w3, l * h * d, h, d, -1);
        for (int64_t i = 0; i < h; i++) {
            double z = m->h1[i];
            double silu = z / (1.0 + exp(-z));
            m->hb[i] = (float)(silu * (double)m->h3[i]);
        }
        matvec(m, m->y, m->hb, &m->w2, l * d * h, d, h, tr ? 3 : -1);
        residual(m->x, m->y, d);
    }

    rmsnorm(m->xb, m->x, m->rms_final, d);
    matvec(m, m->logits, m->xb, &m->wcls, 0, m->V, d, -1);
    return OR_OK;
}
