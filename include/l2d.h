/*
 * l2d.h - C ABI of the MI355X (gfx950) single-token Llama-2 decode step.
 *
 * The step is llama2.c's forward(token, pos) -> logits, in fp32 (run.c) and
 * in Q8_0 (runq.c: int8 codes with one fp32 scale per group of GS values,
 * activations quantised before every matvec). The interface follows the shape
 * the pages show: build the transformer from a weight file, call
 * forward(transformer, token, pos) for a float* of logits, then take the
 * argmax (gitcode porting guide, embedded main-loop example); quantize(x, n)
 * with a global group size (same guide, INT8 quantisation section); a KV
 * cache that starts zeroed (same guide, memory section).
 *
 * Conventions for every entry point:
 *   - return 0 (L2D_OK) on success or a negative L2D_E* code; nothing here
 *     calls exit() or abort(). l2d_last_error() describes the last failure.
 *   - "device" pointers are HIP device memory on the current device; "host"
 *     pointers are ordinary process memory.
 *   - a context is not thread-safe: one context per host thread/stream.
 *   - all work of a context is enqueued on its stream, in order.
 */
#ifndef L2D_H
#define L2D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define L2D_F32 0  /* fp32 weights and activations (run.c) */
#define L2D_Q8_0 1 /* int8 weight/activation codes, fp32 group scales (runq.c) */
#define L2D_Q4_0 2 /* 4-bit weight codes in groups of 32, fp32 group scales, int8 activations
                      (the 4-bit variant the ainews article names; group_size 32) */

#define L2D_OK 0
#define L2D_EINVAL (-1)  /* bad argument: config, group size, token, pos, size */
#define L2D_EFORMAT (-2) /* blob size or layout does not match its header */
#define L2D_ENOMEM (-3)  /* host or device allocation failed */
#define L2D_EHIP (-4)    /* a HIP runtime call failed */

/*
 * Model configuration. The first seven fields are the blob header, in its
 * order: seven little-endian int32 (pomoai.com hub page, data-format
 * section). head_size = dim / n_heads; kv_dim = n_kv_heads * head_size (Q&A
 * page, GQA question). vocab_size > 0: the classifier is the embedding table;
 * vocab_size < 0: a separate classifier array of |vocab_size| rows follows
 * the legacy tables (Q&A page, shared_weights question).
 */
typedef struct {
    int32_t dim, hidden_dim, n_layers, n_heads, n_kv_heads, vocab_size, seq_len;
    int32_t dtype;      /* L2D_F32, L2D_Q8_0 or L2D_Q4_0 */
    int32_t group_size; /* Q8_0 group size GS (64 for the workloads); 32 for Q4_0; ignored for fp32 */
    double rope_theta;  /* 10000 */
    double norm_eps;    /* 1e-5 */
} l2d_config;

/*
 * Host views of the weights, borrowed from the caller (normally pointers into
 * a blob parsed by l2d_blob_parse). Matrices are row-major [rows][cols] with
 * cols the input size. fp32: the matrix pointer is float*, the *_s scale
 * pointer is NULL. Q8_0: the matrix pointer is int8_t codes[rows*cols] and
 * *_s is float scales[rows*cols/GS], one per group of GS consecutive codes.
 * Q4_0: the matrix pointer is uint8_t packed codes[rows*cols/2], 16 bytes
 * per group of 32 (byte b: code b + 8 in the low nibble, code b + 16 + 8 in
 * the high nibble), *_s float scales[rows*cols/32].
 * Per-layer arrays are stacked over layers: wq is [n_layers][dim][dim], etc.
 */
typedef struct {
    const void* emb;  const float* emb_s;   /* [vocab][dim] */
    const float* rms_att;                   /* [n_layers][dim] */
    const void* wq;   const float* wq_s;    /* [n_layers][dim][dim] */
    const void* wk;   const float* wk_s;    /* [n_layers][kv_dim][dim] */
    const void* wv;   const float* wv_s;    /* [n_layers][kv_dim][dim] */
    const void* wo;   const float* wo_s;    /* [n_layers][dim][dim] */
    const float* rms_ffn;                   /* [n_layers][dim] */
    const void* w1;   const float* w1_s;    /* [n_layers][hidden_dim][dim] */
    const void* w2;   const float* w2_s;    /* [n_layers][dim][hidden_dim] */
    const void* w3;   const float* w3_s;    /* [n_layers][hidden_dim][dim] */
    const float* rms_final;                 /* [dim] */
    const void* wcls; const float* wcls_s;  /* [vocab][dim]; == emb when shared */
} l2d_weights;

typedef struct l2d_ctx l2d_ctx;

/*
 * Parse a weight blob held in host memory (zero-copy: w points into blob).
 * Layout: the seven-int32 header, then emb, rms_att, wq, wk, wv, wo, rms_ffn,
 * w1, w2, w3, rms_final, the two legacy freq_cis tables of
 * seq_len*head_size/2 floats each (skipped: RoPE is computed on the fly,
 * Q&A page, freq_cis question), then wcls when vocab_size < 0. In a Q8_0 blob
 * each matrix is codes[n] then scales[n/GS]; in a Q4_0 blob (group_size 32)
 * packed codes[n/2] then scales[n/32]. cfg gets the header plus dtype,
 * group_size, rope_theta = 10000, norm_eps = 1e-5.
 * Errors: L2D_EINVAL for a bad dtype/GS or an invalid header (dim % n_heads,
 * n_heads % n_kv_heads, odd head_size, GS not dividing dim and hidden_dim,
 * a non-positive field); L2D_EFORMAT when nbytes differs from the size the
 * header implies. All offsets are 64-bit.
 */
int l2d_blob_parse(const void* blob, uint64_t nbytes, int32_t dtype, int32_t group_size,
                   l2d_config* cfg, l2d_weights* w);

/*
 * Create a context on the current HIP device: allocate device weights (in the
 * library's own layout), the zeroed KV cache [n_layers][seq_len][kv_dim] fp32
 * (gitcode guide, memory section; Q&A page, KV-cache question), activations
 * and scratch; copy the weights host->device; capture one decode step as a
 * HIP graph. stream: a hipStream_t to run on, or NULL for a stream the
 * context creates and owns. The host weights may be freed after return.
 * Supported: dim and hidden_dim multiples of 4 (fp32: at most 16000);
 * head_size one of 4, 8, 12, 16, 24, 32, 48, 64, 96, 128 (the attention
 * kernel holds at most four float4 of a key row per lane);
 * n_heads / n_kv_heads in {1, 2, 4, 8};
 * Q8_0 group size a power of two in [16, 256] dividing dim and hidden_dim.
 * Launch-shape settings read from the environment here (tuning only; the
 * results do not depend on them beyond the rounding noted):
 *   L2D_GEMV_WG_PER_CU   matvec workgroups per CU (default 2; bit-identical)
 *   L2D_ATTN_WG_PER_CU   attention workgroups per CU that size the position
 *                        splits (default 3, capped by how many fit on a CU;
 *                        another split changes the fp64 merge order)
 *   L2D_ATTN_GSPLIT      workgroups sharing one kv head's query heads
 *                        (default 2 when 8 query heads share one, else 1;
 *                        bit-identical)
 *   L2D_CHAIN=1          per-phase step with chained launches where
 *                        available (default off; l2d_use_chain;
 *                        bit-identical)
 *   L2D_PREFILL_ATTN_VALU=1  batched prefill uses the vector attention kernel
 *                        for every shape (comparison only; read at each
 *                        prefill launch, not here)
 * Errors: L2D_EINVAL, L2D_ENOMEM (device memory), L2D_EHIP.
 */
int l2d_init(const l2d_config* cfg, const l2d_weights* w, void* stream, l2d_ctx** out);

/*
 * One decode step: the embedding row of token, every layer at position pos
 * (k and v are written to cache slot pos, attention reads slots 0..pos),
 * final norm, classifier and argmax. Returns a device pointer to
 * logits[|vocab_size|] fp32, owned by the context and valid until the next
 * forward; the values are ready once the context's stream has reached this
 * point (l2d_sync). Returns NULL on error (token not in [0, vocab), pos not
 * in [0, seq_len)). Re-running the same (token, pos) rewrites the same cache
 * slot with the same values.
 */
const float* l2d_forward(l2d_ctx* ctx, int32_t token, int32_t pos);

/*
 * Like l2d_forward, with the token taken on the device from the previous
 * step's pick (its argmax, or its sampled token when sampling is on):
 * decoding without a host round trip. pos must be >= 1 and the previous
 * forward of this context must have been at pos - 1.
 */
const float* l2d_forward_greedy(l2d_ctx* ctx, int32_t pos);

/*
 * Batched prompt prefill: the same result as n calls l2d_forward(tokens[i],
 * pos0 + i), i = 0..n-1 (prompt tokens are fed through the forward pass one
 * position after another: gitcode guide, main loop; mht18 essay, section 2.3,
 * the toy forward pass over a sequence), computed as int8 matrix products
 * over chunks of up to 512 tokens (MFMA): for Q8_0 every token's matmul
 * inputs are quantised on their own and every output is the same fp64 sum of
 * exact int32 group dots; for fp32 every output is an fp64 sum of the exact
 * products (fp64 MFMA; the summation order differs, as in the decode step's
 * GEMV); attention of token i covers slots 0..pos0 + i. Writes K/V slots
 * pos0 .. pos0 + n - 1 of every layer and returns, like l2d_forward, the
 * device logits of the last token; l2d_last_token gives its argmax (or
 * sampled token), and l2d_forward_greedy(ctx, pos0 + n) may follow.
 * tokens is a host array of n ids, read before the call returns.
 * Asynchronous on the context's stream; the first call allocates the chunk
 * buffers (about 512 x (3 dim + 2 hidden_dim) x 4 bytes, plus 512 x
 * max(dim, hidden_dim) x 4 for fp32 weights).
 * Needs fp32 weights, or Q8_0 with group size 64, 128 or 256, and
 * n_heads / n_kv_heads dividing 8. Returns NULL on error: n <= 0, pos0 < 0, pos0 + n > seq_len,
 * a token outside [0, vocab), an unsupported model (L2D_EINVAL, see
 * l2d_last_error), L2D_ENOMEM, L2D_EHIP.
 */
const float* l2d_prefill(l2d_ctx* ctx, const int32_t* tokens, int32_t n, int32_t pos0);

/*
 * Group combine of the following prefills' Q8_0 matmuls. fp32 = 0 (the
 * default): each output is the fp64 sum over groups of (exact int32 group
 * dot x weight scale) x input scale, the single-token step's arithmetic, so
 * prefill and token-by-token decoding give identical bits. fp32 = 1: the same
 * sum accumulated in fp32, acc = fma(float(dot), weight scale x input scale,
 * acc) (the pages' runq.c combines a group's integer dot with the two scales
 * in float; hub page, quantisation support; gitcode guide section 1): fewer
 * operations per group, results within the logits tolerance rather than bit
 * for bit. fp32 weights are unaffected. Returns L2D_EINVAL for other values.
 */
int l2d_prefill_combine(l2d_ctx* ctx, int32_t fp32);

/*
 * Next-token selection of the following forwards (mht18 essay, section 3.2:
 * the logits go through a softmax, the next token is a random draw from
 * that distribution, the temperature scaling the logits first).
 * temperature == 0 (the default): the greedy argmax. temperature > 0: the
 * token is drawn from softmax(logits / temperature) by the Gumbel-max rule,
 * fused into the classifier: argmax_i of fp32(logit_i / T + g_i), ties to the
 * lowest index, g_i = -log(-log(u_i)) in fp64, u_i = ((b >> 11) + 1/2) 2^-53
 * with b output k = pos * vocab + i + 1 of the splitmix64 stream seeded with
 * `seed` (Steele, Lea, Flood 2014). The draws depend only on (seed, pos,
 * token index): a run is reproducible. The logits are unchanged;
 * l2d_last_token returns the drawn token. Returns L2D_EINVAL for a negative
 * or non-finite temperature.
 */
int l2d_set_sampling(l2d_ctx* ctx, double temperature, uint64_t seed);

/* Wait for the context's stream. */
int l2d_sync(l2d_ctx* ctx);

/*
 * The last forward's pick: the argmax of its logits, the lowest index among
 * equal maxima (sample_argmax of the gitcode guide's main loop), or with
 * sampling on (l2d_set_sampling) the drawn token. Waits for the stream.
 */
int l2d_last_token(l2d_ctx* ctx, int32_t* token);

/* Copy the last forward's logits to host memory (|vocab_size| floats). Waits. */
int l2d_read_logits(l2d_ctx* ctx, float* host_dst);

/*
 * Q8_0-quantise n fp32 values (device x) into device q[n] and s[n/gs], group
 * by group as the quantize listing of the gitcode porting guide (section
 * "1. INT8 quantisation") does: the group's largest |x|, scale = that / 127
 * (fp32 division), code = round half away from zero of the fp32 quotient x /
 * scale. An all-zero group gets scale 0 and codes 0. stream: hipStream_t or
 * NULL (the null stream). Asynchronous. Errors: L2D_EINVAL when gs <= 0,
 * n < 0 or n % gs != 0, or a pointer is NULL while n > 0.
 */
int l2d_quantize_q80(const float* x, int64_t n, int32_t gs, int8_t* q, float* s, void* stream);

/* Zero the KV cache (the calloc'd state of a fresh run). Asynchronous. */
int l2d_reset_kv(l2d_ctx* ctx);

/* Release everything the context owns. NULL is a no-op. */
void l2d_free(l2d_ctx* ctx);

/* Message for the last error of ctx, or of the calling thread when ctx is NULL. */
const char* l2d_last_error(const l2d_ctx* ctx);

/* ------------------------------------------------------------------------
 * Diagnostics and test hooks. They expose intermediate results of the same
 * kernels the decode step runs; none is needed to decode.
 * ---------------------------------------------------------------------- */

/*
 * Device pointers to the KV cache, [n_layers][seq_len][kv_dim] fp32 each.
 * Writing them (e.g. to place synthetic keys/values at deep positions) is
 * allowed between steps.
 */
int l2d_kv_cache(l2d_ctx* ctx, float** key_cache, float** value_cache);

/*
 * Matvec out = W x with the decode step's GEMV kernel (all device pointers):
 * W is fp32 [rows][cols] (dtype L2D_F32, W_s NULL), Q8_0 int8 codes
 * [rows][cols] or Q4_0 nibbles [rows][cols/2], with fp32 scales W_s
 * [rows][cols/gs]; x is fp32 [cols]; out is fp32 [rows].
 * Q8_0 (gitcode porting guide, INT8 quantisation section): x is quantised
 * inside the kernel with the weights' group size, as in the decode step;
 * gs a power of two in [16, 256].
 * Q4_0 (4-bit variant named in the ainews article's technical deep dive and
 * tables, and as a next step in the gitcode guide; read as): gs must be
 * 32; code c of a group is stored as c + 8 in [0, 15], byte b of a group's
 * 16 bytes holding code b in its low nibble and code b + 16 in its high
 * nibble; the scale is the group's value of largest magnitude divided by
 * -8. x is quantised inside the kernel to Q8_0 with groups of 32, and each
 * output is the fp64 sum over groups of (exact int32 group dot) x weight
 * scale x input scale, rounded to fp32.
 * group_dots, when not NULL (Q8_0 and Q4_0), receives the exact int32 dot of
 * every (row, group): [rows][cols/gs]. rows must be even.
 * Asynchronous on stream (Q8_0 codes are first re-laid-out into a
 * stream-ordered temporary buffer; Q4_0 is read in place).
 */
int l2d_gemv(int32_t dtype, const void* W, const float* W_s, const float* x, int64_t rows,
             int64_t cols, int32_t gs, float* out, int32_t* group_dots, void* stream);

/*
 * l2d_gemv for callers that cannot allocate device memory (code under
 * stream capture, serving loops and harnesses that forbid hipMalloc): same
 * arguments, same kernels, same result bits, and no device allocation.
 * Q8_0 codes are re-laid-out into a fixed scratch array of
 * l2d_gemv_noalloc_max_bytes() bytes (32 MiB) that the library holds on each
 * GPU it runs on until the process ends; rows * cols above that returns
 * L2D_EINVAL (use l2d_gemv). Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, two threads) race and give
 * undefined results; calls on one stream are ordered and safe. fp32 and
 * Q4_0 need no scratch and run as l2d_gemv does. Asynchronous on stream.
 */
int l2d_gemv_noalloc(int32_t dtype, const void* W, const float* W_s, const float* x, int64_t rows,
                     int64_t cols, int32_t gs, float* out, int32_t* group_dots, void* stream);
int64_t l2d_gemv_noalloc_max_bytes(void);

/*
 * Time the matvec kernel of l2d_gemv (dtype L2D_F32 or L2D_Q4_0; Q8_0 codes
 * need the device layout and are timed by l2d_profile_step): reps launches
 * on stream, launch r reading weight copy r % copies (W and W_s are host
 * arrays of `copies` device pointers; W_s may be NULL for fp32), each
 * bracketed by HIP events stamped at the kernel's own start and end.
 * avg_seconds receives the mean kernel duration; out holds the last
 * launch's result. Synchronous. Same argument rules as l2d_gemv.
 */
int l2d_gemv_profile(int32_t dtype, const void* const* W, const float* const* W_s, int32_t copies,
                     const float* x, int64_t rows, int64_t cols, int32_t gs, float* out,
                     int32_t reps, double* avg_seconds, void* stream);

/*
 * Trace the quantised matvec inputs of one layer (Q8_0): after l2d_trace_layer
 * (ctx, layer) the next forwards record, for that layer, the codes and scales
 * the kernels computed for slot 0 (q/k/v input), 1 (output-projection input),
 * 2 (w1/w3 input), 3 (w2 input); l2d_trace_read copies one slot to host
 * (codes n, scales n/gs; n = dim, or hidden_dim for slot 3). layer -1 stops
 * tracing. Tracing runs the step without the captured graph.
 */
int l2d_trace_layer(l2d_ctx* ctx, int32_t layer);
int l2d_trace_read(l2d_ctx* ctx, int32_t slot, int8_t* host_q, float* host_s);

/* The hipStream_t the context enqueues on. */
void* l2d_stream(l2d_ctx* ctx);

/*
 * Run the step at (token, pos) reps times with the kernels launched one by
 * one and HIP events recorded around every launch on the context's stream;
 * avg_seconds[7] receives the mean duration per launch of each kernel class:
 * 0 q/k/v matvec (+norm, RoPE, cache write), 1 attention, 2 output matvec,
 * 3 w1/w3 matvec (+norm, SwiGLU), 4 w2 matvec, 5 classifier (+norm, argmax),
 * 6 step start (embedding row). With chained launches (l2d_use_chain) class
 * 1 is the attention + output matvec launch and class 3 the w1/w3 + w2
 * launch; classes 2 and 4 then read 0. Synchronous.
 */
int l2d_profile_step(l2d_ctx* ctx, int32_t token, int32_t pos, int32_t reps, double* avg_seconds);

/*
 * l2d_prefill with HIP events stamped at every kernel's start and end;
 * avg_seconds[8] receives the mean duration per launch of each kernel class:
 * 0 norm + quantise, 1 q/k/v matmul (+RoPE, cache write), 2 attention,
 * 3 output matmul (+residual), 4 w1/w3 matmul (+SwiGLU), 5 w2 matmul
 * (+residual), 6 last token's step start, 7 classifier. Synchronous.
 */
int l2d_profile_prefill(l2d_ctx* ctx, const int32_t* tokens, int32_t n, int32_t pos0, double* avg_seconds);

/* 1: replay the captured graph (default); 0: launch the step's kernels one by one.
 * Applies when the persistent step kernel is off (l2d_use_persistent). */
int l2d_use_graph(l2d_ctx* ctx, int32_t enable);

/*
 * Chained launches of the per-phase step (the layer loop of the mht18
 * essay, section 2.3, and the Q&A page's question on the KV cache: each
 * layer's attention over positions 0..pos, then its output projection;
 * w1/w3 with SwiGLU, then w2), computed as above with the same arithmetic
 * and order, so the logits equal the kernel-by-kernel step's bit for bit.
 * enable = 1: each layer takes three launches instead of five: q/k/v; the
 * attention and the output projection in one launch; w1/w3 and w2 in one
 * launch. In a chained launch the second phase's workgroups follow the
 * first's in the grid, issue their weight loads, and wait for flags that
 * the first phase's workgroups set once their outputs are stored (the
 * attention's o per kv head column; the Q8_0 codes of the SwiGLU output per
 * group). Available for Q8_0 with group size 64, up to 4 query heads per
 * attention workgroup (whose o fills whole 128-byte lines), dim <= 8192 and
 * the head sizes l2d_init takes; enable = 1 elsewhere returns L2D_EINVAL.
 * Off by default (L2D_CHAIN=1 in the environment at l2d_init turns it on):
 * on MI355X the hand-over through device memory costs as much as the launch
 * boundary it replaces, and the 7B Q8_0 step runs slower chained (449
 * against 472 tok/s at pos 512). Re-captures the step graph
 * (synchronous). A wait that exceeds a bounded number of polls (about a
 * quarter second) gives up, later waits of the step give up at once, and
 * the next l2d_sync, l2d_last_token or l2d_read_logits returns L2D_EHIP.
 */
int l2d_use_chain(l2d_ctx* ctx, int32_t enable);

/* 1 when the per-phase step runs with chained launches, 0 otherwise,
 * L2D_EINVAL for a null context. */
int l2d_chained(const l2d_ctx* ctx);

/*
 * Test hook for the chained launches' failure path, forced from the host:
 * sets their error word as a wait that gave up would. The next chained
 * step's waits that find their flags not yet set give up at once (every
 * workgroup still ends), and the next l2d_sync, l2d_last_token or
 * l2d_read_logits returns L2D_EHIP and clears the word; steps after that
 * are valid again. L2D_EINVAL when chained launches are not available for
 * the context's model. Synchronous.
 */
int l2d_test_chain_fault(l2d_ctx* ctx);

/*
 * The same step as one persistent kernel: a single cooperative launch per
 * l2d_forward / l2d_forward_greedy (the toy forward pass of the mht18 essay,
 * section 2.3, every phase computed as above, with the same arithmetic and
 * order; the logits equal the per-phase kernels' bit for bit except where
 * the attention's position split count differs, which moves only the fp64
 * merge order). Worker waves stream the weights through all matvec phases
 * without a break; control waves wait for the other workgroups' progress
 * flags and run the prologues, epilogues and attention. Available for Q8_0
 * with group size 64 on a device with cooperative launch that can hold one
 * workgroup per CU (dim <= 8192, hidden_dim <= 65536, the head sizes
 * l2d_init takes); enable = 1 elsewhere returns L2D_EINVAL. A wait for
 * another workgroup that exceeds a bounded number of polls (seconds) gives
 * up: every workgroup then ends, and the next l2d_sync, l2d_last_token or
 * l2d_read_logits returns L2D_EHIP and resets the flags. Tracing
 * (l2d_trace_layer) uses the per-phase kernels. Off by default: on MI355X
 * the per-phase kernels are faster.
 */
int l2d_use_persistent(l2d_ctx* ctx, int32_t enable);

/*
 * Diagnostics of the persistent step kernel: run one step at (token, pos)
 * with it, recording the device's real-time clock (100 MHz ticks) at each
 * workgroup's control events and at each worker's phase reports. *events
 * receives E = 1 + 6 (4 n_layers + 1), the control events per workgroup.
 * host (n uint64) receives, for G workgroups (one per CU) and W worker
 * waves each (l2d_stream_shape): [G][E] control stamps (event 0: step
 * start; for phase p, in step order q/k/v, output, w1/w3, w2 per layer,
 * then the classifier: 1 + 6p phase start, 2 + 6p the inputs' producers
 * seen done (their progress flags), 3 + 6p input in LDS for the workers,
 * 4 + 6p all workers done, 5 + 6p results stored and this workgroup's flag
 * published, 6 + 6p (q/k/v phases) attention done and published), then
 * [G][W][4 n_layers + 1] worker report stamps; 0 where an event did not
 * occur. host NULL: only *events is set. Synchronous; L2D_EINVAL when n is
 * too small or the kernel is not available.
 */
int l2d_stream_trace(l2d_ctx* ctx, int32_t token, int32_t pos, uint64_t* host, int64_t n, int64_t* events);

/*
 * Launch shape of the persistent step kernel of this context: workgroups
 * (one per CU) and worker waves per workgroup, the G and W of
 * l2d_stream_trace's buffer. L2D_EINVAL for null arguments or when the
 * kernel is not available for the context's model or device.
 */
int l2d_stream_shape(const l2d_ctx* ctx, int32_t* workgroups, int32_t* workers);

/* 1 when l2d_forward runs the persistent step kernel, 0 when the per-phase
 * kernels run, L2D_EINVAL for a null context. */
int l2d_persistent(const l2d_ctx* ctx);

/*
 * Test hook, host only (no device is touched): run the persistent step
 * kernel's plan for the model cfg (Q8_0, group size 64) and a launch of nwg
 * workgroups on the host, with the same functions the kernel computes its
 * addresses with: every worker wave's weight stream (phase order, rows,
 * chunks, code and scale offsets inside their arrays), every row of every
 * matrix streamed exactly once, workgroup row ranges tiling each matrix,
 * attention position ranges covering 0..pos exactly for every pos, partial
 * slots inside their allocation, LDS within 160 KiB. Returns 0 ("ok" in
 * msg) or L2D_EINVAL with the first problem in msg (msglen bytes, NUL
 * terminated).
 */
int l2d_stream_plan_check(const l2d_config* cfg, int32_t nwg, char* msg, int32_t msglen);

#ifdef __cplusplus
}
#endif

#endif /* L2D_H */
