/*
 * synth.c - seeded synthetic inputs for the Llama-2 decode step.
 *
 * This module writes weight blobs and prompt token ids. It holds none of the
 * decode step's arithmetic (no norm, matvec, RoPE, attention or quantisation):
 * both the CPU oracle and the GPU library consume the bytes it writes, and each
 * parses them with its own code.
 *
 * Blob layout (the llama2.c format as the pages describe it: "config header,
 * then contiguous float32 (or int8) arrays", pomoai.com hub page, section on
 * the data format; the sign of vocab_size marks an unshared classifier, Q&A
 * page, shared_weights question; two legacy freq_cis tables of
 * seq_len*head_size/2 floats each, Q&A page, memory_map_weights question):
 *
 *   int32 dim, hidden_dim, n_layers, n_heads, n_kv_heads, vocab_size, seq_len
 *   E[V][d] rms_att[L][d] wq[L][d][d] wk[L][kvd][d] wv[L][kvd][d] wo[L][d][d]
 *   rms_ffn[L][d] w1[L][h][d] w2[L][d][h] w3[L][h][d] rms_final[d]
 *   freq_cis_real[S][hs/2] freq_cis_imag[S][hs/2] (wcls[V][d] if vocab_size<0)
 *
 * In the Q8_0 blob every matrix (E, wq, wk, wv, wo, w1, w2, w3, wcls) is
 * stored as int8 codes[n] followed by fp32 scales[n/GS]; norm gains and the
 * legacy tables stay fp32. In the Q4_0 blob (dtype 2, groups of 32) every
 * matrix is stored as packed 4-bit codes[n/2] (16 bytes per group: byte b
 * holds code b + 8 in its low nibble and code b + 16 + 8 in its high one)
 * followed by fp32 scales[n/32].
 *
 * Values. Every element is a pure function of (seed, tensor id, element
 * index) through the splitmix64 finaliser (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), so any thread
 * count gives the same bytes.
 *   - fp32 matrices, activation vectors and KV-cache fills: a standard
 *     normal variate from one 64-bit draw by the Box-Muller transform (Box
 *     and Muller, "A note on the generation of random normal deviates",
 *     1958): the two 32-bit halves give u1, u2 in (0, 1) as (k + 1/2) 2^-32,
 *     z = sqrt(-2 ln u1) cos(2 pi u2) in fp64, times the sd (0.02 for
 *     weights), rounded to fp32 once: N(0, sd) up to |z| of about 6.7.
 *   - Q8_0 matrices: shaped like the codes of a bell-shaped tensor stored
 *     with one scale per group of GS: in every group one element, at a
 *     drawn index and with a drawn sign, is +-127 (the group's largest
 *     magnitude), and the others are the centred sum mapped with integer
 *     arithmetic to a code of sd ~50, clipped to [-126, 126]; each group
 *     scale is drawn uniformly from [0.75, 1.25] x 0.02/sd(code), so
 *     dequantised weights have sd ~0.02.
 *   - Q4_0 matrices: the centred sum mapped to [-8, 8] with integer
 *     arithmetic and 8 clipped to 7; scales as for Q8_0 with the 4-bit
 *     code's sd.
 *   - norm gains are 1.0; the legacy freq_cis tables are NaN so that a loader
 *     that fails to skip them poisons every logit.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

enum {
    T_EMB = 1, T_RMS_ATT, T_WQ, T_WK, T_WV, T_WO, T_RMS_FFN,
    T_W1, T_W2, T_W3, T_RMS_FINAL, T_FREQ_RE, T_FREQ_IM, T_WCLS,
    T_SCALE_BASE = 32, T_PROMPT = 64, T_GROUP_MAX = 96
};

static inline uint64_t mix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t seed, uint64_t tid, uint64_t i)
{
    return mix64(mix64(mix64(seed) + tid) + i);
}

/* centred sum of four 16-bit fields: integer in [-131070, 131070] */
static inline int64_t bell(uint64_t r)
{
    int64_t s = (int64_t)(r & 0xFFFF) + (int64_t)((r >> 16) & 0xFFFF) +
                (int64_t)((r >> 32) & 0xFFFF) + (int64_t)((r >> 48) & 0xFFFF);
    return s - 131070;
}

/* standard deviation of bell(): 4 * (65536^2 - 1) / 12 under the root */
static double bell_sd(void) { return sqrt(4.0 * (65536.0 * 65536.0 - 1.0) / 12.0); }

/* standard normal variate of one 64-bit draw (Box-Muller, cosine branch) */
static inline double gauss(uint64_t r)
{
    const double u1 = ((double)(r & 0xFFFFFFFFull) + 0.5) * 0x1.0p-32;
    const double u2 = ((double)(r >> 32) + 0.5) * 0x1.0p-32;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

typedef struct {
    int32_t dim, hidden_dim, n_layers, n_heads, n_kv_heads, vocab_size, seq_len;
} synth_config;

static int64_t iabs64(int64_t v) { return v < 0 ? -v : v; }

/* element counts of the blob's arrays, in file order; returns count */
typedef struct { int tid; int64_t n; int is_matrix; } part;

static int parts_of(const synth_config* c, part* p)
{
    int64_t d = c->dim, h = c->hidden_dim, L = c->n_layers, V = iabs64(c->vocab_size);
    int64_t hs = d / c->n_heads, kvd = (int64_t)c->n_kv_heads * hs, S = c->seq_len;
    int k = 0;
    p[k++] = (part){T_EMB, V * d, 1};
    p[k++] = (part){T_RMS_ATT, L * d, 0};
    p[k++] = (part){T_WQ, L * d * d, 1};
    p[k++] = (part){T_WK, L * kvd * d, 1};
    p[k++] = (part){T_WV, L * kvd * d, 1};
    p[k++] = (part){T_WO, L * d * d, 1};
    p[k++] = (part){T_RMS_FFN, L * d, 0};
    p[k++] = (part){T_W1, L * h * d, 1};
    p[k++] = (part){T_W2, L * d * h, 1};
    p[k++] = (part){T_W3, L * h * d, 1};
    p[k++] = (part){T_RMS_FINAL, d, 0};
    p[k++] = (part){T_FREQ_RE, S * (hs / 2), 0};
    p[k++] = (part){T_FREQ_IM, S * (hs / 2), 0};
    if (c->vocab_size < 0) p[k++] = (part){T_WCLS, V * d, 1};
    return k;
}

static int valid(const synth_config* c, int dtype, int gs)
{
    if (c->dim <= 0 || c->hidden_dim <= 0 || c->n_layers <= 0 || c->n_heads <= 0 ||
        c->n_kv_heads <= 0 || c->vocab_size == 0 || c->seq_len <= 0)
        return 0;
    if (c->dim % c->n_heads) return 0;
    if (dtype == 2 && gs != 32) return 0;
    if (dtype == 1 || dtype == 2) {
        /* groups never straddle a matrix row */
        if (gs <= 0 || c->dim % gs || c->hidden_dim % gs) return 0;
        part p[16];
        int n = parts_of(c, p);
        for (int i = 0; i < n; i++)
            if (p[i].is_matrix && p[i].n % gs) return 0;
    }
    return 1;
}

/* total blob bytes; dtype 0 = fp32, 1 = Q8_0 with group size gs, 2 = Q4_0
   (gs 32); -1 if invalid */
int64_t synth_blob_bytes(const synth_config* c, int dtype, int gs)
{
    if (!valid(c, dtype, gs)) return -1;
    part p[16];
    int n = parts_of(c, p);
    int64_t bytes = 7 * 4;
    for (int i = 0; i < n; i++) {
        if (dtype == 1 && p[i].is_matrix)
            bytes += p[i].n + 4 * (p[i].n / gs);
        else if (dtype == 2 && p[i].is_matrix)
            bytes += p[i].n / 2 + 4 * (p[i].n / 32);
        else
            bytes += 4 * p[i].n;
    }
    return bytes;
}

static void fill_f32(float* dst, int64_t n, uint64_t seed, int tid)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) dst[i] = (float)(gauss(draw(seed, (uint64_t)tid, (uint64_t)i)) * 0.02);
}

static void fill_const(float* dst, int64_t n, float v)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) dst[i] = v;
}

/* sd of an 8-bit code before clipping: bell_sd * 173 / 131070 (about 49.9) */
#define CODE8_SPAN 173

static void fill_codes(int8_t* dst, int64_t n, int gs, uint64_t seed, int tid)
{
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n / gs; g++) {
        const uint64_t r = draw(seed, (uint64_t)(T_GROUP_MAX + tid), (uint64_t)g);
        const int64_t at = (int64_t)((r >> 11) % (uint64_t)gs);
        for (int64_t j = 0; j < gs; j++) {
            const int64_t i = g * gs + j;
            int64_t c = bell(draw(seed, (uint64_t)tid, (uint64_t)i)) * CODE8_SPAN / 131070;
            c = c > 126 ? 126 : c < -126 ? -126 : c;
            if (j == at) c = (r >> 63) ? -127 : 127;
            dst[i] = (int8_t)c;
        }
    }
}

/* 4-bit codes of element i: the bell sum mapped to [-8, 8], 8 clipped to 7 */
static inline int code4(uint64_t seed, int tid, int64_t i)
{
    const int64_t c = bell(draw(seed, (uint64_t)tid, (uint64_t)i)) * 8 / 131070;
    return c > 7 ? 7 : (int)c;
}

static void fill_codes4(uint8_t* dst, int64_t n, uint64_t seed, int tid)
{
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n / 32; g++)
        for (int b = 0; b < 16; b++)
            dst[g * 16 + b] = (uint8_t)((code4(seed, tid, g * 32 + b) + 8) |
                                        ((code4(seed, tid, g * 32 + b + 16) + 8) << 4));
}

static void fill_scales_sd(float* dst, int64_t ng, uint64_t seed, int tid, double code_sd)
{
    const double base = 0.02 / code_sd;
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ng; g++) {
        double u = (double)(draw(seed, (uint64_t)(T_SCALE_BASE + tid), (uint64_t)g) >> 11) *
                   (1.0 / 9007199254740992.0);
        dst[g] = (float)(base * (0.75 + 0.5 * u));
    }
}

static void fill_scales(float* dst, int64_t ng, uint64_t seed, int tid)
{
    /* sd of a code: about bell_sd * CODE8_SPAN / 131070, plus the group's
       +-127 (its share of the mean square is 127^2 / gs at gs 64) */
    const double base = 0.02 / 52.0;
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ng; g++) {
        double u = (double)(draw(seed, (uint64_t)(T_SCALE_BASE + tid), (uint64_t)g) >> 11) *
                   (1.0 / 9007199254740992.0);
        dst[g] = (float)(base * (0.75 + 0.5 * u));
    }
}

/*
 * Write the whole blob into out (synth_blob_bytes() bytes).
 * Returns 0, or -1 when the config is invalid.
 */
int synth_fill_blob(const synth_config* c, int dtype, int gs, uint64_t seed, uint8_t* out)
{
    if (!valid(c, dtype, gs)) return -1;
    memcpy(out, c, 7 * 4);
    uint8_t* ptr = out + 7 * 4;
    part p[16];
    int n = parts_of(c, p);
    for (int i = 0; i < n; i++) {
        if (dtype == 2 && p[i].is_matrix) {
            fill_codes4(ptr, p[i].n, seed, p[i].tid);
            ptr += p[i].n / 2;
            /* n / 2 is a multiple of 16: the scales stay 4-byte aligned */
            fill_scales_sd((float*)ptr, p[i].n / 32, seed, p[i].tid, bell_sd() * 8.0 / 131070.0);
            ptr += 4 * (p[i].n / 32);
        } else if (dtype == 1 && p[i].is_matrix) {
            int8_t* q = (int8_t*)ptr;
            fill_codes(q, p[i].n, gs, seed, p[i].tid);
            ptr += p[i].n;
            float* s;
            /* scales follow the codes; the blob keeps 4-byte alignment because
               every code array length is a multiple of gs */
            s = (float*)ptr;
            fill_scales(s, p[i].n / gs, seed, p[i].tid);
            ptr += 4 * (p[i].n / gs);
        } else {
            float* f = (float*)ptr;
            if (p[i].tid == T_RMS_ATT || p[i].tid == T_RMS_FFN || p[i].tid == T_RMS_FINAL)
                fill_const(f, p[i].n, 1.0f);
            else if (p[i].tid == T_FREQ_RE || p[i].tid == T_FREQ_IM)
                fill_const(f, p[i].n, NAN);
            else
                fill_f32(f, p[i].n, seed, p[i].tid);
            ptr += 4 * p[i].n;
        }
    }
    return 0;
}

/* n prompt token ids, uniform over [0, vocab) */
void synth_prompt(uint64_t seed, int32_t n, int32_t vocab, int32_t* out)
{
    for (int32_t i = 0; i < n; i++)
        out[i] = (int32_t)((draw(seed, T_PROMPT, (uint64_t)i) >> 11) % (uint64_t)vocab);
}

/* n fp32 values, N(0, sd), for activation vectors and KV-cache fills */
void synth_normal_f32(uint64_t seed, int32_t tid, int64_t n, double sd, float* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (float)(gauss(draw(seed, (uint64_t)(1000 + tid), (uint64_t)i)) * sd);
}
