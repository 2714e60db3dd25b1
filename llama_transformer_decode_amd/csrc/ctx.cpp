// ctx.cpp - the C ABI: context creation, weight upload, the decode step as a
// captured HIP graph, and the diagnostic hooks.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <string>

#include "internal.hpp"
#include "l2d.h"
#include "runtime.hpp"
#include "stream_plan.hpp"

namespace {

thread_local std::string g_err;

}  // namespace

namespace l2d {

int fail(l2d_ctx* ctx, int code, const std::string& msg)
{
    if (ctx)
        ctx->err = msg;
    else
        g_err = msg;
    return code;
}

static bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int validate_config(const l2d_config* c)
{
    auto bad = [](const char* m) { return fail(nullptr, L2D_EINVAL, m); };
    if (c->dim <= 0 || c->hidden_dim <= 0 || c->n_layers <= 0 || c->n_heads <= 0 ||
        c->n_kv_heads <= 0 || c->vocab_size == 0 || c->seq_len <= 0)
        return bad("config: every header field must be positive (vocab_size non-zero)");
    if (c->dim % c->n_heads) return bad("config: dim must be a multiple of n_heads");
    if (c->n_heads % c->n_kv_heads) return bad("config: n_heads must be a multiple of n_kv_heads");
    const int hs = c->dim / c->n_heads;
    if (hs % 2) return bad("config: head_size must be even (RoPE rotates pairs)");
    if (c->dtype != L2D_F32 && c->dtype != L2D_Q8_0 && c->dtype != L2D_Q4_0) return bad("config: unknown dtype");
    if (c->dtype == L2D_Q4_0) {
        if (c->group_size != 32) return bad("config: Q4_0 group size must be 32");
        if (c->dim % 32 || c->hidden_dim % 32) return bad("config: Q4_0 needs dim and hidden_dim multiples of 32");
    }
    if (c->dtype == L2D_Q8_0) {
        const int gs = c->group_size;
        if (!pow2(gs) || gs < 16 || gs > 256)
            return bad("config: Q8_0 group size must be a power of two in [16, 256]");
        if (c->dim % gs || c->hidden_dim % gs)
            return bad("config: Q8_0 group size must divide dim and hidden_dim");
    }
    return L2D_OK;
}

// limits of the kernels beyond the format's own rules
static int check_supported(l2d_ctx* ctx, const l2d_config* c)
{
    const int hs = c->dim / c->n_heads;
    if (c->dim % 4 || c->hidden_dim % 4)
        return fail(ctx, L2D_EINVAL, "init: dim and hidden_dim must be multiples of 4");
    if (hs % 4 || hs > 128) return fail(ctx, L2D_EINVAL, "init: head_size must be a multiple of 4 and <= 128");
    if (c->dtype == L2D_F32 && (c->dim > 16000 || c->hidden_dim > 16000))
        return fail(ctx, L2D_EINVAL, "init: fp32 matvec inputs are limited to 16000 values (64 KiB of LDS)");
    if (c->dim > 65536 || c->hidden_dim > 65536)
        return fail(ctx, L2D_EINVAL, "init: matvec inputs are limited to 65536 values");
    const int G = c->n_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(ctx, L2D_EINVAL, "init: n_heads / n_kv_heads must be 1, 2, 4 or 8");
    if (!attention_supported(G, hs))
        return fail(ctx, L2D_EINVAL,
                    "init: attention supports head sizes 4, 8, 12, 16, 24, 32, 48, 64, 96 and 128 "
                    "(at most 4 float4 of a key row per lane)");
    return L2D_OK;
}

}  // namespace l2d

using namespace l2d;

#define HIP_TRY(ctx, call)                                                                  \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess)                                                               \
            return fail((ctx), L2D_EHIP, std::string(#call ": ") + hipGetErrorString(e_));  \
    } while (0)

namespace {

int dev_alloc(l2d_ctx* ctx, void** p, size_t bytes)
{
    *p = nullptr;
    if (bytes == 0) bytes = 16;
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        char buf[128];
        snprintf(buf, sizeof(buf), "init: hipMalloc of %zu bytes failed", bytes);
        return fail(ctx, e == hipErrorOutOfMemory ? L2D_ENOMEM : L2D_EHIP, buf);
    }
    ctx->allocs.push_back(*p);
    return L2D_OK;
}

#define ALLOC(ptr, bytes)                                               \
    do {                                                                \
        void* p_ = nullptr;                                             \
        int rc_ = dev_alloc(ctx, &p_, (bytes));                         \
        if (rc_ != L2D_OK) return rc_;                                  \
        (ptr) = (decltype(ptr))p_;                                      \
    } while (0)

// host -> device copy of `rows` rows of `width` bytes each, placed at a
// device pitch of `dpitch` bytes: one contiguous upload into a staging
// buffer, then a device-side strided copy
int upload_rows(l2d_ctx* ctx, void* dst, size_t dpitch, const void* src, size_t width, size_t rows,
                void* staging)
{
    HIP_TRY(ctx, hipMemcpyAsync(staging, src, width * rows, hipMemcpyHostToDevice, ctx->stream));
    HIP_TRY(ctx, hipMemcpy2DAsync(dst, dpitch, staging, width, width, rows,
                                  hipMemcpyDeviceToDevice, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    return L2D_OK;
}

// host -> device copy of Q8_0 codes [rows][K] through the staging buffer,
// re-laid-out on the device (group-interleaved rows; source row r lands at
// destination row (r / blk) * stride + off + r % blk)
int upload_q8(l2d_ctx* ctx, void* dst, const void* src, int64_t rows, int64_t K, int64_t blk,
              int64_t stride, int64_t off, void* staging)
{
    HIP_TRY(ctx, hipMemcpyAsync(staging, src, (size_t)(rows * K), hipMemcpyHostToDevice, ctx->stream));
    HIP_TRY(ctx, launch_permute_q8((const int8_t*)staging, (int8_t*)dst, rows, K, ctx->gs, blk, stride,
                                   off, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    return L2D_OK;
}

int upload(l2d_ctx* ctx, void* dst, const void* src, size_t bytes)
{
    HIP_TRY(ctx, hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, ctx->stream));
    return L2D_OK;
}

void release(l2d_ctx* ctx)
{
    if (ctx->exec) hipGraphExecDestroy(ctx->exec);
    if (ctx->graph) hipGraphDestroy(ctx->graph);
    if (ctx->stream) hipStreamSynchronize(ctx->stream);
    for (void* p : ctx->allocs) hipFree(p);
    ctx->allocs.clear();
    if (ctx->own_stream && ctx->stream) hipStreamDestroy(ctx->stream);
    ctx->stream = nullptr;
}

size_t elt(int dt) { return dt == DT_F32 ? 4 : 1; }

// device bytes of n weights of dtype dt (Q4_0: two codes per byte)
size_t mat_bytes(int dt, int64_t n) { return dt == DT_F32 ? (size_t)n * 4 : dt == DT_Q8 ? (size_t)n : (size_t)n / 2; }

// Start/stop events of each launch of the kernel-by-kernel step, by kernel
// class; the events are stamped at the kernel's own start and end.
struct KernelTimer {
    std::vector<hipEvent_t> ev;
    std::vector<int> cls;
    size_t used = 0;
    LaunchEvents cur;

    hipError_t next(int c)
    {
        if (used + 2 > ev.size()) {
            for (int i = 0; i < 2; i++) {
                hipEvent_t e;
                hipError_t r = hipEventCreate(&e);
                if (r != hipSuccess) return r;
                ev.push_back(e);
            }
            cls.resize(ev.size() / 2);
        }
        cls[used / 2] = c;
        cur.start = ev[used];
        cur.stop = ev[used + 1];
        used += 2;
        return hipSuccess;
    }
    ~KernelTimer()
    {
        for (hipEvent_t e : ev) hipEventDestroy(e);
    }
};

enum { KC_QKV = 0, KC_ATTN, KC_WO, KC_W13, KC_W2, KC_CLS, KC_BEGIN, KC_COUNT };

// Final RMSNorm of ctx->x -> classifier -> logits and argmax (or sampled
// token) of the step recorded in the step record.
int enqueue_classifier(l2d_ctx* ctx, KernelTimer* kt, int cls)
{
    GemvParams p;
    memset(&p, 0, sizeof(p));
    p.gs = (int32_t)ctx->gs;
    p.eps = ctx->cfg.norm_eps;
    p.step = ctx->step;
    p.W = ctx->wcls;
    p.Ws = ctx->dt != DT_F32 ? ctx->wcls_s : nullptr;
    p.M = ctx->V;
    p.K = ctx->d;
    p.x = ctx->x;
    p.gain = ctx->rms_final;
    p.out = ctx->logits;
    p.argmax = ctx->argmax;
    if (kt) HIP_TRY(ctx, kt->next(cls));
    HIP_TRY(ctx, launch_gemv(ctx->dt, PRO_NORM, EPI_LOGITS, p, ctx->max_blocks, ctx->stream,
                             kt ? &kt->cur : nullptr));
    return L2D_OK;
}

// All kernels of one decode step after the step-start kernel.
int enqueue_layers(l2d_ctx* ctx, bool tracing, KernelTimer* kt = nullptr)
{
    const int64_t d = ctx->d, h = ctx->h, kvd = ctx->kvd;
    const int64_t nqkv = d + 2 * kvd;
    const int dt = ctx->dt;
    const int64_t gs = ctx->gs;
    hipStream_t s = ctx->stream;
    auto scales = [&](float* base, int64_t off_elems) -> const float* {
        return dt != DT_F32 ? base + off_elems / gs : nullptr;
    };
    for (int64_t l = 0; l < ctx->L; l++) {
        const bool tr = tracing && l == ctx->trace_layer;
        GemvParams p;
        memset(&p, 0, sizeof(p));
        p.gs = (int32_t)gs;
        p.eps = ctx->cfg.norm_eps;
        p.step = ctx->step;

        // RMSNorm -> q/k/v matvec -> RoPE -> KV-cache slot pos
        p.W = (const uint8_t*)ctx->wqkv + mat_bytes(dt, l * nqkv * d);
        p.Ws = scales(ctx->wqkv_s, l * nqkv * d);
        p.M = nqkv;
        p.K = d;
        p.x = ctx->x;
        p.gain = ctx->rms_att + l * d;
        p.out = ctx->q;
        p.kcache = ctx->kc + l * ctx->S * kvd;
        p.vcache = ctx->vc + l * ctx->S * kvd;
        p.d = (int32_t)d;
        p.kvd = (int32_t)kvd;
        p.hs = (int32_t)ctx->hs;
        p.rope = ctx->rope;
        p.trace_q = tr ? ctx->trace_q[0] : nullptr;
        p.trace_s = tr ? ctx->trace_s[0] : nullptr;
        if (kt) HIP_TRY(ctx, kt->next(KC_QKV));
        HIP_TRY(ctx, launch_gemv(ctx->dt, PRO_NORM, EPI_QKV, p, ctx->max_blocks, s, kt ? &kt->cur : nullptr));

        // attention over positions 0..pos
        AttnParams a;
        a.q = ctx->q;
        a.kc = ctx->kc + l * ctx->S * kvd;
        a.vc = ctx->vc + l * ctx->S * kvd;
        a.o = ctx->o;
        a.part_o = ctx->part_o;
        a.part_ml = ctx->part_ml;
        a.ctr = ctx->attn_ctr;
        a.step = ctx->step;
        a.S = (int32_t)ctx->S;
        a.nkv = (int32_t)ctx->nkv;
        a.hs = (int32_t)ctx->hs;
        a.kvd = (int32_t)kvd;
        a.G = (int32_t)ctx->G;
        a.nsplit = ctx->nsplit;
        a.gsplit = ctx->gsplit;
        const bool chain = ctx->use_chain && ctx->chain_ok;
        const int64_t ncol = ctx->nkv * ctx->gsplit;
        ChainArgs ca;
        ca.flags = ctx->chain_flags;
        ca.nflags = (int32_t)ncol;
        ca.pub = ctx->chain_flags;
        ca.err = ctx->chain_err;
        ca.go = ctx->chain_err + 32;
        ca.layer = (int32_t)l;
        ca.nlayers = (int32_t)ctx->L;
        if (!chain) {
            if (kt) HIP_TRY(ctx, kt->next(KC_ATTN));
            HIP_TRY(ctx, launch_attention(a, s, kt ? &kt->cur : nullptr));
        }

        // output projection + residual
        p.W = (const uint8_t*)ctx->wo + mat_bytes(dt, l * d * d);
        p.Ws = scales(ctx->wo_s, l * d * d);
        p.M = d;
        p.K = d;
        p.x = ctx->o;
        p.gain = nullptr;
        p.out = ctx->x;
        p.trace_q = tr ? ctx->trace_q[1] : nullptr;
        p.trace_s = tr ? ctx->trace_s[1] : nullptr;
        if (chain) {
            // attention and the output projection in one launch
            if (kt) HIP_TRY(ctx, kt->next(KC_ATTN));
            HIP_TRY(ctx, launch_attn_wo(a, p, ca, ctx->max_blocks, s, kt ? &kt->cur : nullptr));
        } else {
            if (kt) HIP_TRY(ctx, kt->next(KC_WO));
            HIP_TRY(ctx, launch_gemv(ctx->dt, PRO_PLAIN, EPI_RESID, p, ctx->max_blocks, s, kt ? &kt->cur : nullptr));
        }

        // RMSNorm -> w1/w3 matvec -> SwiGLU
        p.W = (const uint8_t*)ctx->w13 + mat_bytes(dt, l * 2 * h * d);
        p.Ws = scales(ctx->w13_s, l * 2 * h * d);
        p.M = 2 * h;
        p.K = d;
        p.x = ctx->x;
        p.gain = ctx->rms_ffn + l * d;
        p.out = ctx->hb;
        p.trace_q = tr ? ctx->trace_q[2] : nullptr;
        p.trace_s = tr ? ctx->trace_s[2] : nullptr;
        // quantised weights: hb is quantised once, group by group, as the
        // w1/w3 matvec completes it, and the w2 matvec takes the codes
        const bool hbq = dt != DT_F32;
        p.oq = hbq ? ctx->hb_q : nullptr;
        p.os = hbq ? ctx->hb_s : nullptr;
        p.octr = hbq ? ctx->hb_ctr : nullptr;
        p.ogs = (int32_t)gs;
        GemvParams p13 = p;
        if (chain) p13.oq = ctx->chain_hbq;  // one group per 128-byte line
        if (!chain) {
            if (kt) HIP_TRY(ctx, kt->next(KC_W13));
            HIP_TRY(ctx, launch_gemv(ctx->dt, PRO_NORM, EPI_SWIGLU, p, ctx->max_blocks, s, kt ? &kt->cur : nullptr));
        }
        p.oq = nullptr;
        p.os = nullptr;
        p.octr = nullptr;

        // w2 matvec + residual
        p.W = (const uint8_t*)ctx->w2 + mat_bytes(dt, l * d * h);
        p.Ws = scales(ctx->w2_s, l * d * h);
        p.M = d;
        p.K = h;
        p.x = ctx->hb;
        p.xq = hbq ? ctx->hb_q : nullptr;
        p.xs = hbq ? ctx->hb_s : nullptr;
        p.gain = nullptr;
        p.out = ctx->x;
        p.trace_q = tr ? ctx->trace_q[3] : nullptr;
        p.trace_s = tr ? ctx->trace_s[3] : nullptr;
        if (chain) {
            // w1/w3 and w2 in one launch, w2 waiting on the group flags
            GemvParams p2 = p;
            p2.xq = ctx->chain_hbq;
            p2.xs = nullptr;
            ChainArgs cf = ca;
            cf.flags = ctx->chain_flags + ncol;
            cf.nflags = (int32_t)(h / gs);
            cf.pub = ctx->chain_flags + ncol;
            cf.go = ctx->chain_err + 64;
            if (kt) HIP_TRY(ctx, kt->next(KC_W13));
            HIP_TRY(ctx, launch_ffn_chain(p13, p2, cf, ctx->max_blocks, s, kt ? &kt->cur : nullptr));
        } else {
            if (kt) HIP_TRY(ctx, kt->next(KC_W2));
            HIP_TRY(ctx, launch_gemv(ctx->dt, hbq ? PRO_CODES : PRO_PLAIN, EPI_RESID, p, ctx->max_blocks, s,
                                     kt ? &kt->cur : nullptr));
        }
        p.xq = nullptr;
        p.xs = nullptr;
    }
    return enqueue_classifier(ctx, kt, KC_CLS);
}

int setup_stream(l2d_ctx* ctx, int cus);

int capture(l2d_ctx* ctx)
{
    HIP_TRY(ctx, hipStreamBeginCapture(ctx->stream, hipStreamCaptureModeThreadLocal));
    int rc = enqueue_layers(ctx, false);
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(ctx->stream, &g);
    if (rc != L2D_OK) {
        if (g) hipGraphDestroy(g);
        return rc;
    }
    if (e != hipSuccess) return fail(ctx, L2D_EHIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
    ctx->graph = g;
    HIP_TRY(ctx, hipGraphInstantiate(&ctx->exec, g, nullptr, nullptr, 0));
    return L2D_OK;
}

int init_impl(l2d_ctx* ctx, const l2d_config* cfg, const l2d_weights* w, void* stream)
{
    int rc = validate_config(cfg);
    if (rc != L2D_OK) return fail(ctx, rc, g_err);
    rc = check_supported(ctx, cfg);
    if (rc != L2D_OK) return rc;
    ctx->cfg = *cfg;
    ctx->dt = cfg->dtype == L2D_F32 ? DT_F32 : cfg->dtype == L2D_Q8_0 ? DT_Q8 : DT_Q4;
    ctx->d = cfg->dim;
    ctx->h = cfg->hidden_dim;
    ctx->L = cfg->n_layers;
    ctx->V = cfg->vocab_size < 0 ? -(int64_t)cfg->vocab_size : cfg->vocab_size;
    ctx->S = cfg->seq_len;
    ctx->nh = cfg->n_heads;
    ctx->nkv = cfg->n_kv_heads;
    ctx->hs = ctx->d / ctx->nh;
    ctx->kvd = ctx->nkv * ctx->hs;
    ctx->G = ctx->nh / ctx->nkv;
    ctx->gs = ctx->dt != DT_F32 ? cfg->group_size : 1;
    const bool q8 = ctx->dt == DT_Q8;
    const bool quant = ctx->dt != DT_F32;  // scales present (Q8_0, Q4_0)
    if (!w || !w->emb || !w->rms_att || !w->wq || !w->wk || !w->wv || !w->wo || !w->rms_ffn ||
        !w->w1 || !w->w2 || !w->w3 || !w->rms_final || !w->wcls)
        return fail(ctx, L2D_EINVAL, "init: a weight pointer is NULL");
    if (quant && (!w->emb_s || !w->wq_s || !w->wk_s || !w->wv_s || !w->wo_s || !w->w1_s ||
                  !w->w2_s || !w->w3_s || !w->wcls_s))
        return fail(ctx, L2D_EINVAL, "init: a scale pointer is NULL");

    HIP_TRY(ctx, hipGetDevice(&ctx->device));
    int cus = 0;
    HIP_TRY(ctx, hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, ctx->device));
    int per_cu = 2;
    if (const char* e = getenv("L2D_GEMV_WG_PER_CU")) per_cu = atoi(e) > 0 ? atoi(e) : per_cu;
    ctx->max_blocks = cus * per_cu;
    if (stream) {
        ctx->stream = (hipStream_t)stream;
    } else {
        HIP_TRY(ctx, hipStreamCreateWithFlags(&ctx->stream, hipStreamNonBlocking));
        ctx->own_stream = true;
    }

    const int64_t d = ctx->d, h = ctx->h, L = ctx->L, V = ctx->V, kvd = ctx->kvd;
    const int64_t gs = ctx->gs;
    const size_t es = elt(ctx->dt);
    const int dt = ctx->dt;
    const int64_t nqkv = d + 2 * kvd;
    auto sbytes = [&](int64_t n) -> size_t { return quant ? (size_t)(n / gs) * 4 : 0; };
    auto mb = [&](int64_t n) -> size_t { return mat_bytes(dt, n); };

    ALLOC(ctx->emb, mb(V * d));
    if (quant) ALLOC(ctx->emb_s, sbytes(V * d));
    ALLOC(ctx->wqkv, mb(L * nqkv * d));
    if (quant) ALLOC(ctx->wqkv_s, sbytes(L * nqkv * d));
    ALLOC(ctx->wo, mb(L * d * d));
    if (quant) ALLOC(ctx->wo_s, sbytes(L * d * d));
    ALLOC(ctx->w13, mb(L * 2 * h * d));
    if (quant) ALLOC(ctx->w13_s, sbytes(L * 2 * h * d));
    ALLOC(ctx->w2, mb(L * d * h));
    if (quant) ALLOC(ctx->w2_s, sbytes(L * d * h));
    const bool shared = cfg->vocab_size > 0;
    if (!shared) {
        ALLOC(ctx->wcls, mb(V * d));
        if (quant) ALLOC(ctx->wcls_s, sbytes(V * d));
    }
    ALLOC(ctx->rms_att, (size_t)(L * d) * 4);
    ALLOC(ctx->rms_ffn, (size_t)(L * d) * 4);
    ALLOC(ctx->rms_final, (size_t)d * 4);
    ALLOC(ctx->freqs, (size_t)(ctx->hs / 2) * 4);
    ALLOC(ctx->rope, (size_t)ctx->hs * 4);
    const size_t kvbytes = (size_t)(L * ctx->S * kvd) * 4;
    ALLOC(ctx->kc, kvbytes);
    ALLOC(ctx->vc, kvbytes);
    ALLOC(ctx->x, (size_t)d * 4);
    ALLOC(ctx->q, (size_t)d * 4);
    ALLOC(ctx->o, (size_t)d * 4);
    ALLOC(ctx->hb, (size_t)h * 4);
    ALLOC(ctx->hb_q, (size_t)h);
    ALLOC(ctx->hb_s, (size_t)(h / gs + 1) * 4);
    ALLOC(ctx->hb_ctr, (size_t)(h / gs + 1) * kGroupCtrStride * 4);
    ALLOC(ctx->logits, (size_t)V * 4);
    ALLOC(ctx->step, 64);
    ALLOC(ctx->argmax, (size_t)kArgmaxWords * 8);
    // attention position splits: at most about three workgroups per CU over
    // the kv heads (fewer, longer ranges beat more, shorter ones once that
    // fills the chip: measured from pos 128 to 4095 at the 7B and 13B
    // shapes), splits of at least one sub-chunk (the grid is sized once,
    // inactive splits exit), at most 64 splits to merge per head
    {
        const int64_t sc = attention_positions_per_subchunk((int)ctx->hs);
        // 8 query heads per kv head: two workgroups share each kv head (4
        // heads each), so the merge that follows the last range reads half
        // as much per workgroup, and two run at once
        ctx->gsplit = ctx->G == 8 ? 2 : 1;
        if (const char* e = getenv("L2D_ATTN_GSPLIT")) {
            const int v = atoi(e);
            if (v >= 1 && ctx->G % v == 0 && ctx->G / v >= 1) ctx->gsplit = v;
        }
        const int64_t nv = ctx->nkv * ctx->gsplit;
        // no more than can be resident at once: the 4-head instance (70B)
        // fits two per CU, and sizing for three left a second round of
        // workgroups (attention at pos 4095: 41.0 -> 33.3 us per layer)
        int64_t per_cu = 3;
        int resident = attention_blocks_per_cu((int)ctx->G, ctx->gsplit, (int)ctx->hs);
        // chained launches (off by default: on MI355X the 7B Q8_0 step ran
        // 449 tok/s chained against 472 kernel by kernel at pos 512;
        // L2D_CHAIN=1 or l2d_use_chain turns them on). The split count is
        // sized for the lower occupancy of the two attention instances, so
        // switching does not change it.
        ctx->chain_ok = chain_supported(ctx->dt, (int)ctx->gs, ctx->d, ctx->h, (int)ctx->G, ctx->gsplit,
                                        (int)ctx->hs, ctx->max_blocks);
        ctx->use_chain = false;
        if (const char* e = getenv("L2D_CHAIN")) ctx->use_chain = ctx->chain_ok && atoi(e) != 0;
        if (ctx->chain_ok) {
            const int rc2 = attn_wo_blocks_per_cu((int)ctx->G, ctx->gsplit, (int)ctx->hs, ctx->d, (int)ctx->gs);
            if (rc2 > 0 && (resident <= 0 || rc2 < resident)) resident = rc2;
        }
        if (resident > 0 && resident < per_cu) per_cu = resident;
        if (const char* e = getenv("L2D_ATTN_WG_PER_CU")) per_cu = atoi(e) > 0 ? atoi(e) : per_cu;
        int64_t ns = (per_cu * cus + nv / 2) / nv;
        if (ns > 64) ns = 64;
        if (ns > (ctx->S + sc - 1) / sc) ns = (ctx->S + sc - 1) / sc;
        ctx->nsplit = (int)(ns < 1 ? 1 : ns);
    }
    const size_t nparts = (size_t)ctx->nkv * ctx->nsplit * ctx->G;
    ALLOC(ctx->part_o, nparts * ctx->hs * 8);
    ALLOC(ctx->part_ml, nparts * 2 * 8);
    ALLOC(ctx->attn_ctr, (size_t)ctx->nkv * ctx->gsplit * 32 * 4);
    const size_t chain_flag_bytes = (size_t)(ctx->nkv * ctx->gsplit + h / gs + 1) * 4;
    ALLOC(ctx->chain_flags, chain_flag_bytes);
    ALLOC(ctx->chain_err, 96 * 4);
    ALLOC(ctx->chain_hbq, (size_t)(h / gs + 1) * 128);
    for (int i = 0; i < 4; i++) {
        const int64_t n = i == 3 ? h : d;
        ALLOC(ctx->trace_q[i], (size_t)n);
        ALLOC(ctx->trace_s[i], (size_t)(n / gs + 1) * 4);
    }

    // staging buffer for the strided (re-laid-out) uploads: the largest of
    // the arrays that go through it
    size_t stage = 0;
    for (int64_t n : {L * d * d, L * kvd * d, L * h * d, V * d}) {
        if (mb(n) > stage) stage = mb(n);
        if (sbytes(n) > stage) stage = sbytes(n);
    }
    void* staging = nullptr;
    {
        hipError_t e = hipMalloc(&staging, stage);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(ctx, L2D_ENOMEM, "init: no device memory for the upload staging buffer");
        }
    }
    auto up_all = [&]() -> int {
        int r;
        if (q8) {
            // codes: group-interleaved rows, placed by the permute kernel
            const int64_t all = 1ll << 62;
            if ((r = upload_q8(ctx, ctx->emb, w->emb, V, d, all, 0, 0, staging))) return r;
            if ((r = upload_q8(ctx, ctx->wqkv, w->wq, L * d, d, d, nqkv, 0, staging))) return r;
            if ((r = upload_q8(ctx, ctx->wqkv, w->wk, L * kvd, d, kvd, nqkv, d, staging))) return r;
            if ((r = upload_q8(ctx, ctx->wqkv, w->wv, L * kvd, d, kvd, nqkv, d + kvd, staging))) return r;
            if ((r = upload_q8(ctx, ctx->wo, w->wo, L * d, d, all, 0, 0, staging))) return r;
            if ((r = upload_q8(ctx, ctx->w13, w->w1, L * h, d, 1, 2, 0, staging))) return r;
            if ((r = upload_q8(ctx, ctx->w13, w->w3, L * h, d, 1, 2, 1, staging))) return r;
            if ((r = upload_q8(ctx, ctx->w2, w->w2, L * d, h, all, 0, 0, staging))) return r;
            if (!shared && (r = upload_q8(ctx, ctx->wcls, w->wcls, V, d, all, 0, 0, staging))) return r;
            // scales: plain [row][K/gs], rows placed like the codes
            if ((r = upload(ctx, ctx->emb_s, w->emb_s, sbytes(V * d)))) return r;
            const size_t sp = sbytes(nqkv * d);
            if ((r = upload_rows(ctx, ctx->wqkv_s, sp, w->wq_s, sbytes(d * d), L, staging))) return r;
            if ((r = upload_rows(ctx, (uint8_t*)ctx->wqkv_s + sbytes(d * d), sp, w->wk_s,
                                 sbytes(kvd * d), L, staging))) return r;
            if ((r = upload_rows(ctx, (uint8_t*)ctx->wqkv_s + sbytes((d + kvd) * d), sp, w->wv_s,
                                 sbytes(kvd * d), L, staging))) return r;
            if ((r = upload(ctx, ctx->wo_s, w->wo_s, sbytes(L * d * d)))) return r;
            const size_t sb = sbytes(d);
            if ((r = upload_rows(ctx, ctx->w13_s, 2 * sb, w->w1_s, sb, L * h, staging))) return r;
            if ((r = upload_rows(ctx, (uint8_t*)ctx->w13_s + sb, 2 * sb, w->w3_s, sb, L * h, staging))) return r;
            if ((r = upload(ctx, ctx->w2_s, w->w2_s, sbytes(L * d * h)))) return r;
            if (!shared && (r = upload(ctx, ctx->wcls_s, w->wcls_s, sbytes(V * d)))) return r;
        } else {
            // fp32 values, or Q4_0 packed codes (rows read in place)
            const size_t lp = mb(nqkv * d), rw = mb(d);
            if ((r = upload(ctx, ctx->emb, w->emb, mb(V * d)))) return r;
            // q, k, v rows of each layer side by side: [L][d + 2kvd][d]
            if ((r = upload_rows(ctx, ctx->wqkv, lp, w->wq, mb(d * d), L, staging))) return r;
            if ((r = upload_rows(ctx, (uint8_t*)ctx->wqkv + mb(d * d), lp, w->wk, mb(kvd * d), L, staging))) return r;
            if ((r = upload_rows(ctx, (uint8_t*)ctx->wqkv + mb((d + kvd) * d), lp, w->wv, mb(kvd * d), L,
                                 staging))) return r;
            if ((r = upload(ctx, ctx->wo, w->wo, mb(L * d * d)))) return r;
            // w1 / w3 rows interleaved: [L][h][2][d]
            if ((r = upload_rows(ctx, ctx->w13, 2 * rw, w->w1, rw, L * h, staging))) return r;
            if ((r = upload_rows(ctx, (uint8_t*)ctx->w13 + rw, 2 * rw, w->w3, rw, L * h, staging))) return r;
            if ((r = upload(ctx, ctx->w2, w->w2, mb(L * d * h)))) return r;
            if (!shared && (r = upload(ctx, ctx->wcls, w->wcls, mb(V * d)))) return r;
            if (quant) {
                // scales: plain [row][K/32], rows placed like the codes
                if ((r = upload(ctx, ctx->emb_s, w->emb_s, sbytes(V * d)))) return r;
                const size_t sp = sbytes(nqkv * d);
                if ((r = upload_rows(ctx, ctx->wqkv_s, sp, w->wq_s, sbytes(d * d), L, staging))) return r;
                if ((r = upload_rows(ctx, (uint8_t*)ctx->wqkv_s + sbytes(d * d), sp, w->wk_s,
                                     sbytes(kvd * d), L, staging))) return r;
                if ((r = upload_rows(ctx, (uint8_t*)ctx->wqkv_s + sbytes((d + kvd) * d), sp, w->wv_s,
                                     sbytes(kvd * d), L, staging))) return r;
                if ((r = upload(ctx, ctx->wo_s, w->wo_s, sbytes(L * d * d)))) return r;
                const size_t sb = sbytes(d);
                if ((r = upload_rows(ctx, ctx->w13_s, 2 * sb, w->w1_s, sb, L * h, staging))) return r;
                if ((r = upload_rows(ctx, (uint8_t*)ctx->w13_s + sb, 2 * sb, w->w3_s, sb, L * h, staging))) return r;
                if ((r = upload(ctx, ctx->w2_s, w->w2_s, sbytes(L * d * h)))) return r;
                if (!shared && (r = upload(ctx, ctx->wcls_s, w->wcls_s, sbytes(V * d)))) return r;
            }
        }
        if ((r = upload(ctx, ctx->rms_att, w->rms_att, (size_t)(L * d) * 4))) return r;
        if ((r = upload(ctx, ctx->rms_ffn, w->rms_ffn, (size_t)(L * d) * 4))) return r;
        if ((r = upload(ctx, ctx->rms_final, w->rms_final, (size_t)d * 4))) return r;
        return L2D_OK;
    };
    rc = up_all();
    hipStreamSynchronize(ctx->stream);
    hipFree(staging);
    if (rc != L2D_OK) return rc;
    if (shared) {
        ctx->wcls = ctx->emb;
        ctx->wcls_s = ctx->emb_s;
    }

    // RoPE frequencies theta^(-2j/hs), computed in fp64 and rounded once
    {
        std::vector<float> f((size_t)(ctx->hs / 2));
        for (int64_t j = 0; j < ctx->hs / 2; j++)
            f[(size_t)j] = (float)pow(cfg->rope_theta, -(double)(2 * j) / (double)ctx->hs);
        HIP_TRY(ctx, hipMemcpyAsync(ctx->freqs, f.data(), f.size() * 4, hipMemcpyHostToDevice, ctx->stream));
        HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    }
    HIP_TRY(ctx, hipMemsetAsync(ctx->kc, 0, kvbytes, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->vc, 0, kvbytes, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->argmax, 0, (size_t)kArgmaxWords * 8, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->attn_ctr, 0, (size_t)ctx->nkv * ctx->gsplit * 32 * 4, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->hb_ctr, 0, (size_t)(ctx->h / ctx->gs + 1) * kGroupCtrStride * 4, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->step, 0, 64, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->chain_flags, 0, chain_flag_bytes, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->chain_err, 0, 96 * 4, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    rc = capture(ctx);
    if (rc != L2D_OK) return rc;
    return setup_stream(ctx, cus);
}

// The persistent step kernel (Q8_0, group size 64): one workgroup per CU,
// all resident (cooperative launch). Its attention items: the query heads of
// a kv head split over gsplit items when 8 share one (as in the per-phase
// attention kernel), and about one item per workgroup over the position
// splits.
int setup_stream(l2d_ctx* ctx, int cus)
{
    ctx->stream_ok = false;
    ctx->use_stream = false;
    const int gsplit = ctx->G == 8 ? 2 : 1;
    if (!stream_supported(ctx->dt, ctx->gs, ctx->d, ctx->h, (int)ctx->G, gsplit, (int)ctx->hs)) return L2D_OK;
    int coop = 0;
    HIP_TRY(ctx, hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, ctx->device));
    if (!coop) return L2D_OK;
    const int kg = (int)ctx->G / gsplit;
    // the workers' weight base is the q/k/v codes; every matrix kind's codes
    // and scales as byte offsets from it
    const int8_t* base = (const int8_t*)ctx->wqkv;
    auto off = [&](const void* q) { return (int64_t)((intptr_t)q - (intptr_t)base); };
    SPlan sp{ctx->d, ctx->h, ctx->L, ctx->kvd, ctx->V, cus, stream_workers(),
             off(ctx->wqkv), off(ctx->wo), off(ctx->w13), off(ctx->w2), off(ctx->wcls),
             off(ctx->wqkv_s), off(ctx->wo_s), off(ctx->w13_s), off(ctx->w2_s), off(ctx->wcls_s)};
    if (!sd_fits(sp)) return L2D_OK;
    std::vector<SDesc> tab;
    std::vector<int32_t> cnt;
    int64_t stride = 0;
    stream_tables(sp, tab, cnt, &stride);
    const size_t lds = stream_lds_bytes(sp, kg, (int)ctx->hs, stride);
    if (lds > 160 * 1024 || stream_blocks_per_cu(kg, (int)ctx->hs, lds) < 1) return L2D_OK;
    const int64_t cols = ctx->nkv * gsplit;
    const int64_t ns = stream_splits(ctx->nkv, gsplit, cus, ctx->S, (int)ctx->hs);
    ALLOC(ctx->ssync, sizeof(StreamSync));
    ALLOC(ctx->sflags, (size_t)cus * 4);
    ALLOC(ctx->shead_ctr, (size_t)cols * 32 * 4);
    ALLOC(ctx->spart_o, (size_t)cols * ns * kg * ctx->hs * 8);
    ALLOC(ctx->spart_ml, (size_t)cols * ns * kg * 2 * 8);
    ALLOC(ctx->sdummy, 8192);
    ALLOC(ctx->swtab, tab.size() * sizeof(SDesc));
    ALLOC(ctx->swcnt, cnt.size() * sizeof(int32_t));
    HIP_TRY(ctx, hipMemcpyAsync(ctx->swtab, tab.data(), tab.size() * sizeof(SDesc), hipMemcpyHostToDevice, ctx->stream));
    HIP_TRY(ctx, hipMemcpyAsync(ctx->swcnt, cnt.data(), cnt.size() * sizeof(int32_t), hipMemcpyHostToDevice, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->ssync, 0, sizeof(StreamSync), ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->sflags, 0, (size_t)cus * 4, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->shead_ctr, 0, (size_t)cols * 32 * 4, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->sdummy, 0, 8192, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    ctx->swtab_stride = stride;
    ctx->stream_grid = cus;
    ctx->stream_kg = kg;
    ctx->stream_gsplit = gsplit;
    ctx->stream_nsplit = (int)ns;
    ctx->stream_ymax = (int)sp_max_wg_rows(sp);
    ctx->stream_lds = lds;
    ctx->stream_epoch = 0;
    ctx->stream_ok = true;
    return L2D_OK;
}

// One launch of the persistent step kernel for (token, pos).
hipError_t launch_step_kernel(l2d_ctx* ctx, int32_t token, int32_t pos, bool greedy)
{
    const uint32_t nb = stream_epochs((int)ctx->L);
    if (ctx->stream_epoch > (1u << 31) - nb) {
        // the progress flags count up across launches: restart them from zero
        hipError_t e = hipMemsetAsync(ctx->sflags, 0, (size_t)ctx->stream_grid * 4, ctx->stream);
        if (e != hipSuccess) return e;
        ctx->stream_epoch = 0;
    }
    StreamParams p;
    memset(&p, 0, sizeof(p));
    p.d = (int32_t)ctx->d;
    p.h = (int32_t)ctx->h;
    p.L = (int32_t)ctx->L;
    p.nkv = (int32_t)ctx->nkv;
    p.hs = (int32_t)ctx->hs;
    p.kvd = (int32_t)ctx->kvd;
    p.G = (int32_t)ctx->G;
    p.V = (int32_t)ctx->V;
    p.S = (int32_t)ctx->S;
    p.nsplit = ctx->stream_nsplit;
    p.gsplit = ctx->stream_gsplit;
    p.ymax = ctx->stream_ymax;
    p.kmax = (int32_t)(ctx->d > ctx->h ? ctx->d : ctx->h);
    p.eps = ctx->cfg.norm_eps;
    p.emb = (const int8_t*)ctx->emb;
    p.emb_s = ctx->emb_s;
    p.wqkv = (const int8_t*)ctx->wqkv;
    p.wqkv_s = ctx->wqkv_s;
    p.wo = (const int8_t*)ctx->wo;
    p.wo_s = ctx->wo_s;
    p.w13 = (const int8_t*)ctx->w13;
    p.w13_s = ctx->w13_s;
    p.w2 = (const int8_t*)ctx->w2;
    p.w2_s = ctx->w2_s;
    p.wcls = (const int8_t*)ctx->wcls;
    p.wcls_s = ctx->wcls_s;
    p.rms_att = ctx->rms_att;
    p.rms_ffn = ctx->rms_ffn;
    p.rms_final = ctx->rms_final;
    p.freqs = ctx->freqs;
    p.kc = ctx->kc;
    p.vc = ctx->vc;
    p.x = ctx->x;
    p.q = ctx->q;
    p.o = ctx->o;
    p.hb = ctx->hb;
    p.logits = ctx->logits;
    p.step = ctx->step;
    p.argmax = ctx->argmax;
    p.part_o = ctx->spart_o;
    p.part_ml = ctx->spart_ml;
    p.head_ctr = ctx->shead_ctr;
    p.sync = ctx->ssync;
    p.flags = ctx->sflags;
    p.dummy = ctx->sdummy;
    p.wbase = p.wqkv;
    p.wtab = ctx->swtab;
    p.wtab_stride = ctx->swtab_stride;
    p.wcnt = ctx->swcnt;
    p.token = token;
    p.pos = pos;
    p.greedy = greedy ? 1 : 0;
    p.epoch0 = ctx->stream_epoch;
    p.temperature = ctx->temperature;
    p.seed = ctx->seed;
    p.trace = ctx->strace;
    p.trace_n = stream_trace_events((int)ctx->L);
    hipError_t e = launch_stream(p, ctx->stream_kg, ctx->stream_grid, ctx->stream_lds, ctx->stream);
    if (e == hipSuccess) {
        ctx->stream_epoch += nb;
        ctx->stream_pending = true;
    }
    return e;
}

// After a synchronisation: did a wait of a chained launch give up? Then
// the error word is cleared and the error reported (flags need no reset:
// the next step's epoch differs).
int chain_check(l2d_ctx* ctx)
{
    if (!ctx->chain_pending) return L2D_OK;
    ctx->chain_pending = false;
    uint32_t err = 0;
    HIP_TRY(ctx, hipMemcpyAsync(&err, ctx->chain_err, 4, hipMemcpyDeviceToHost, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    if (err == 0) return L2D_OK;
    HIP_TRY(ctx, hipMemsetAsync(ctx->chain_err, 0, 4, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    return fail(ctx, L2D_EHIP, "chained launch: a wait for the first phase gave up; the step's results are invalid");
}

// After a synchronisation: did a wait of the step kernel give up? Then the
// barrier state is reset and the error reported.
int stream_check(l2d_ctx* ctx)
{
    const int rc = chain_check(ctx);
    if (rc != L2D_OK) return rc;
    if (!ctx->stream_pending) return L2D_OK;
    uint32_t err = 0;
    HIP_TRY(ctx, hipMemcpyAsync(&err, ctx->ssync->err, 4, hipMemcpyDeviceToHost, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    ctx->stream_pending = false;
    if (err == 0) return L2D_OK;
    const int64_t cols = ctx->nkv * ctx->stream_gsplit;
    HIP_TRY(ctx, hipMemsetAsync(ctx->ssync, 0, sizeof(StreamSync), ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->sflags, 0, (size_t)ctx->stream_grid * 4, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->shead_ctr, 0, (size_t)cols * 32 * 4, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    ctx->stream_epoch = 0;
    return fail(ctx, L2D_EHIP, "step kernel: a wait for another workgroup gave up; the step's results are invalid");
}

hipError_t begin(l2d_ctx* ctx, int32_t token, int32_t pos, bool greedy,
                 const LaunchEvents* ev = nullptr)
{
    BeginParams b;
    b.emb = ctx->emb;
    b.emb_s = ctx->emb_s;
    b.dtype = ctx->dt;
    b.gs = ctx->gs;
    b.d = (int32_t)ctx->d;
    b.vocab = (int32_t)ctx->V;
    b.x = ctx->x;
    b.step = ctx->step;
    b.argmax = ctx->argmax;
    b.token = token;
    b.pos = pos;
    b.greedy = greedy ? 1 : 0;
    b.temperature = ctx->temperature;
    b.seed = ctx->seed;
    b.freqs = ctx->freqs;
    b.rope = ctx->rope;
    b.hs = (int32_t)ctx->hs;
    return launch_begin(b, ctx->stream, ev);
}

const float* forward_impl(l2d_ctx* ctx, int32_t token, int32_t pos, bool greedy)
{
    if (!ctx) {
        fail(nullptr, L2D_EINVAL, "forward: null context");
        return nullptr;
    }
    if (pos < 0 || pos >= ctx->S) {
        fail(ctx, L2D_EINVAL, "forward: pos outside [0, seq_len)");
        return nullptr;
    }
    if (!greedy && (token < 0 || token >= ctx->V)) {
        fail(ctx, L2D_EINVAL, "forward: token outside [0, vocab)");
        return nullptr;
    }
    if (greedy && (pos < 1 || ctx->last_pos != pos - 1)) {
        fail(ctx, L2D_EINVAL, "forward_greedy: the previous step must be at pos - 1");
        return nullptr;
    }
    const bool tracing = ctx->trace_layer >= 0;
    if (ctx->use_stream && ctx->stream_ok && !tracing) {
        hipError_t e = launch_step_kernel(ctx, token, pos, greedy);
        if (e != hipSuccess) {
            fail(ctx, L2D_EHIP, std::string("step kernel launch: ") + hipGetErrorString(e));
            return nullptr;
        }
        ctx->last_pos = pos;
        return ctx->logits;
    }
    hipError_t e = begin(ctx, token, pos, greedy);
    if (e != hipSuccess) {
        fail(ctx, L2D_EHIP, std::string("begin_step launch: ") + hipGetErrorString(e));
        return nullptr;
    }
    if (ctx->use_graph && !tracing) {
        e = hipGraphLaunch(ctx->exec, ctx->stream);
        if (e != hipSuccess) {
            fail(ctx, L2D_EHIP, std::string("hipGraphLaunch: ") + hipGetErrorString(e));
            return nullptr;
        }
    } else if (enqueue_layers(ctx, tracing) != L2D_OK) {
        return nullptr;
    }
    if (ctx->use_chain && ctx->chain_ok) ctx->chain_pending = true;
    ctx->last_pos = pos;
    return ctx->logits;
}

}  // namespace

namespace l2d {

// Argument checks shared by l2d_gemv, l2d_gemv_noalloc and l2d_gemv_profile; fills p (W, Ws
// left to the caller) and the kernel dtype.
int gemv_setup(int32_t dtype, const float* x, int64_t rows, int64_t cols, int32_t gs,
               bool have_scales, float* out, GemvParams* p, int* dt)
{
    if (dtype != L2D_F32 && dtype != L2D_Q8_0 && dtype != L2D_Q4_0)
        return fail(nullptr, L2D_EINVAL, "gemv: bad dtype");
    if (rows <= 0 || cols <= 0 || rows % 2 || cols % 4 || !x || !out)
        return fail(nullptr, L2D_EINVAL, "gemv: need rows even > 0, cols % 4 == 0, non-null pointers");
    if (dtype == L2D_Q8_0) {
        if (gs < 16 || gs > 256 || (gs & (gs - 1)) || cols % gs || !have_scales)
            return fail(nullptr, L2D_EINVAL, "gemv: Q8_0 needs a power-of-two gs in [16,256] dividing cols");
        if (cols > 65536) return fail(nullptr, L2D_EINVAL, "gemv: cols > 65536");
    } else if (dtype == L2D_Q4_0) {
        if (gs != 32 || cols % 32 || !have_scales) return fail(nullptr, L2D_EINVAL, "gemv: Q4_0 needs gs 32 dividing cols");
        if (cols > 65536) return fail(nullptr, L2D_EINVAL, "gemv: cols > 65536");
    } else if (cols > 16000) {
        return fail(nullptr, L2D_EINVAL, "gemv: fp32 cols > 16000");
    }
    memset(p, 0, sizeof(*p));
    p->M = rows;
    p->K = cols;
    p->gs = dtype == L2D_F32 ? 1 : gs;
    p->x = x;
    p->out = out;
    *dt = dtype == L2D_F32 ? DT_F32 : dtype == L2D_Q8_0 ? DT_Q8 : DT_Q4;
    return L2D_OK;
}

int gemv_grid()
{
    int dev = 0, cus = 0;
    hipGetDevice(&dev);
    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return cus > 0 ? 2 * cus : 512;
}

}  // namespace l2d

extern "C" {

int l2d_init(const l2d_config* cfg, const l2d_weights* w, void* stream, l2d_ctx** out)
{
    if (!out || !cfg) return fail(nullptr, L2D_EINVAL, "init: null argument");
    *out = nullptr;
    l2d_ctx* ctx = new (std::nothrow) l2d_ctx();
    if (!ctx) return fail(nullptr, L2D_ENOMEM, "init: out of host memory");
    int rc = init_impl(ctx, cfg, w, stream);
    if (rc != L2D_OK) {
        g_err = ctx->err;
        release(ctx);
        delete ctx;
        return rc;
    }
    *out = ctx;
    return L2D_OK;
}

const float* l2d_forward(l2d_ctx* ctx, int32_t token, int32_t pos)
{
    return forward_impl(ctx, token, pos, false);
}

const float* l2d_forward_greedy(l2d_ctx* ctx, int32_t pos)
{
    return forward_impl(ctx, 0, pos, true);
}

int l2d_sync(l2d_ctx* ctx)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "sync: null context");
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    return stream_check(ctx);
}

int l2d_last_token(l2d_ctx* ctx, int32_t* token)
{
    if (!ctx || !token) return fail(ctx, L2D_EINVAL, "last_token: null argument");
    if (ctx->last_pos < 0) return fail(ctx, L2D_EINVAL, "last_token: no forward yet");
    unsigned long long slots[kArgmaxSlots * kArgmaxStride];
    HIP_TRY(ctx, hipMemcpyAsync(slots, ctx->argmax + (size_t)(ctx->last_pos & 1) * kArgmaxSlots * kArgmaxStride,
                                sizeof(slots), hipMemcpyDeviceToHost, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    int rc = stream_check(ctx);
    if (rc != L2D_OK) return rc;
    unsigned long long v = 0;
    for (int i = 0; i < kArgmaxSlots; i++)
        if (slots[i * kArgmaxStride] > v) v = slots[i * kArgmaxStride];
    *token = (int32_t)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull));
    return L2D_OK;
}

int l2d_read_logits(l2d_ctx* ctx, float* host_dst)
{
    if (!ctx || !host_dst) return fail(ctx, L2D_EINVAL, "read_logits: null argument");
    HIP_TRY(ctx, hipMemcpyAsync(host_dst, ctx->logits, (size_t)ctx->V * 4, hipMemcpyDeviceToHost,
                                ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    return stream_check(ctx);
}

int l2d_quantize_q80(const float* x, int64_t n, int32_t gs, int8_t* q, float* s, void* stream)
{
    if (gs <= 0 || n < 0 || n % gs) return fail(nullptr, L2D_EINVAL, "quantize_q80: need gs > 0, n >= 0, n % gs == 0");
    if (!((gs <= 64 && (gs & (gs - 1)) == 0) || gs % 64 == 0))
        return fail(nullptr, L2D_EINVAL, "quantize_q80: gs must be a power of two <= 64 or a multiple of 64");
    if (n == 0) return L2D_OK;
    if (!x || !q || !s) return fail(nullptr, L2D_EINVAL, "quantize_q80: null pointer");
    hipError_t e = launch_quantize(x, n, gs, q, s, (hipStream_t)stream);
    if (e != hipSuccess) return fail(nullptr, L2D_EHIP, std::string("quantize_q80: ") + hipGetErrorString(e));
    return L2D_OK;
}

int l2d_reset_kv(l2d_ctx* ctx)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "reset_kv: null context");
    const size_t kvbytes = (size_t)(ctx->L * ctx->S * ctx->kvd) * 4;
    HIP_TRY(ctx, hipMemsetAsync(ctx->kc, 0, kvbytes, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->vc, 0, kvbytes, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->attn_ctr, 0, (size_t)ctx->nkv * ctx->gsplit * 32 * 4, ctx->stream));
    HIP_TRY(ctx, hipMemsetAsync(ctx->hb_ctr, 0, (size_t)(ctx->h / ctx->gs + 1) * kGroupCtrStride * 4, ctx->stream));
    ctx->last_pos = -1;
    return L2D_OK;
}

void l2d_free(l2d_ctx* ctx)
{
    if (!ctx) return;
    release(ctx);
    delete ctx;
}

const char* l2d_last_error(const l2d_ctx* ctx)
{
    return ctx ? ctx->err.c_str() : g_err.c_str();
}

int l2d_kv_cache(l2d_ctx* ctx, float** key_cache, float** value_cache)
{
    if (!ctx || !key_cache || !value_cache) return fail(ctx, L2D_EINVAL, "kv_cache: null argument");
    *key_cache = ctx->kc;
    *value_cache = ctx->vc;
    return L2D_OK;
}


int l2d_gemv(int32_t dtype, const void* W, const float* W_s, const float* x, int64_t rows,
             int64_t cols, int32_t gs, float* out, int32_t* group_dots, void* stream)
{
    GemvParams p;
    int dt = 0;
    int rc = gemv_setup(dtype, x, rows, cols, gs, W_s != nullptr, out, &p, &dt);
    if (rc != L2D_OK) return rc;
    if (!W) return fail(nullptr, L2D_EINVAL, "gemv: null weights");
    hipStream_t st = (hipStream_t)stream;
    void* perm = nullptr;
    if (dtype == L2D_Q8_0) {
        // the kernel reads the device layout: group-interleaved rows
        hipError_t e = hipMallocAsync(&perm, (size_t)(rows * cols), st);
        if (e != hipSuccess) return fail(nullptr, L2D_ENOMEM, "gemv: no device memory for the re-laid-out codes");
        e = launch_permute_q8((const int8_t*)W, (int8_t*)perm, rows, cols, gs, 1ll << 62, 0, 0, st);
        if (e != hipSuccess) {
            (void)hipFreeAsync(perm, st);
            return fail(nullptr, L2D_EHIP, std::string("gemv: ") + hipGetErrorString(e));
        }
    }
    p.W = perm ? perm : W;
    p.Ws = W_s;
    p.group_dots = dtype == L2D_F32 ? nullptr : group_dots;
    hipError_t e = launch_gemv(dt, PRO_PLAIN, EPI_STORE, p, gemv_grid(), st);
    if (perm) (void)hipFreeAsync(perm, st);
    if (e != hipSuccess) return fail(nullptr, L2D_EHIP, std::string("gemv: ") + hipGetErrorString(e));
    return L2D_OK;
}

int l2d_gemv_profile(int32_t dtype, const void* const* W, const float* const* W_s, int32_t copies,
                     const float* x, int64_t rows, int64_t cols, int32_t gs, float* out,
                     int32_t reps, double* avg_seconds, void* stream)
{
    if (!W || copies <= 0 || reps <= 0 || !avg_seconds)
        return fail(nullptr, L2D_EINVAL, "gemv_profile: bad argument");
    if (dtype == L2D_Q8_0)
        return fail(nullptr, L2D_EINVAL, "gemv_profile: Q8_0 codes need the device layout (timed by l2d_profile_step)");
    GemvParams p;
    int dt = 0;
    int rc = gemv_setup(dtype, x, rows, cols, gs, W_s != nullptr, out, &p, &dt);
    if (rc != L2D_OK) return rc;
    for (int i = 0; i < copies; i++)
        if (!W[i] || (dtype == L2D_Q4_0 && !W_s[i])) return fail(nullptr, L2D_EINVAL, "gemv_profile: null copy");
    hipStream_t st = (hipStream_t)stream;
    const int grid = gemv_grid();
    KernelTimer kt;
    for (int r = 0; r < reps; r++) {
        if (kt.next(0) != hipSuccess) return fail(nullptr, L2D_EHIP, "gemv_profile: no events");
        p.W = W[r % copies];
        p.Ws = dtype == L2D_Q4_0 ? W_s[r % copies] : nullptr;
        hipError_t e = launch_gemv(dt, PRO_PLAIN, EPI_STORE, p, grid, st, &kt.cur);
        if (e != hipSuccess) return fail(nullptr, L2D_EHIP, std::string("gemv_profile: ") + hipGetErrorString(e));
    }
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(nullptr, L2D_EHIP, std::string("gemv_profile: ") + hipGetErrorString(e));
    double sum = 0.0;
    for (size_t i = 0; i < kt.used / 2; i++) {
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, kt.ev[2 * i], kt.ev[2 * i + 1]);
        if (e != hipSuccess) return fail(nullptr, L2D_EHIP, std::string("gemv_profile: ") + hipGetErrorString(e));
        sum += ms * 1e-3;
    }
    *avg_seconds = sum / reps;
    return L2D_OK;
}

// ---------------------------------------------------------------- prefill

namespace {

constexpr int kPrefillChunk = 512;  // tokens per batched pass
enum { PC_PREP = 0, PC_QKV, PC_ATTN, PC_WO, PC_W13, PC_W2, PC_START, PC_CLS, PC_COUNT };

bool prefill_supported(const l2d_ctx* ctx)
{
    const bool dt_ok = ctx->dt == DT_F32 || (ctx->dt == DT_Q8 && (ctx->gs == 64 || ctx->gs == 128 || ctx->gs == 256));
    return dt_ok && ctx->d % 4 == 0 && ctx->h % 4 == 0 && prefill_attn_supported((int)ctx->G, (int)ctx->hs);
}

int prefill_buffers(l2d_ctx* ctx)
{
    if (ctx->pf_cap > 0) return L2D_OK;
    int64_t cap = ctx->S < kPrefillChunk ? ctx->S : kPrefillChunk;
    cap = (cap + 15) / 16 * 16;  // whole 16-token tiles of the matmul inputs and attention blocks
    const int64_t kmax = ctx->d > ctx->h ? ctx->d : ctx->h;
    ALLOC(ctx->pf_tok, (size_t)cap * 4);
    ALLOC(ctx->pf_x, (size_t)(cap * ctx->d) * 4);
    ALLOC(ctx->pf_q, (size_t)(cap * ctx->d) * 4);
    ALLOC(ctx->pf_o, (size_t)(cap * ctx->d) * 4);
    ALLOC(ctx->pf_h, (size_t)(cap * ctx->h) * 4);
    // matmul inputs: int8 codes (Q8_0) or normalised fp32 rows (fp32 weights)
    ALLOC(ctx->pf_aq, (size_t)(cap * kmax) * (ctx->dt == DT_F32 ? 4 : 1));
    ALLOC(ctx->pf_as, (size_t)(cap * (kmax / ctx->gs)) * 4);
    ALLOC(ctx->pf_cos, (size_t)(cap * (ctx->hs / 2)) * 4);
    ALLOC(ctx->pf_sin, (size_t)(cap * (ctx->hs / 2)) * 4);
    // rows past a chunk's last token are read (never used) by the attention
    // kernel's last token block: keep them finite
    HIP_TRY(ctx, hipMemsetAsync(ctx->pf_q, 0, (size_t)(cap * ctx->d) * 4, ctx->stream));
    ctx->pf_cap = (int)cap;
    return L2D_OK;
}

// One chunk of m <= pf_cap prompt tokens (already in pf_tok) at positions
// pos .. pos + m - 1: every layer, leaving the residual rows in pf_x and the
// K/V rows in the cache.
int enqueue_prefill_chunk(l2d_ctx* ctx, int m, int pos, KernelTimer* kt)
{
    const int64_t d = ctx->d, h = ctx->h, kvd = ctx->kvd, gs = ctx->gs;
    const int64_t nqkv = d + 2 * kvd;
    const bool f32 = ctx->dt == DT_F32;
    const size_t es = elt(ctx->dt);
    float* xn = (float*)ctx->pf_aq;  // fp32 weights: normalised input rows
    hipStream_t s = ctx->stream;
    auto ev = [&](int c) -> const LaunchEvents* {
        if (!kt) return nullptr;
        if (kt->next(c) != hipSuccess) return nullptr;
        return &kt->cur;
    };
    PrefillEmbedParams e;
    e.emb = ctx->emb;
    e.emb_s = ctx->emb_s;
    e.dtype = ctx->dt;
    e.gs = (int32_t)gs;
    e.d = d;
    e.tokens = ctx->pf_tok;
    e.m = m;
    e.x = ctx->pf_x;
    HIP_TRY(ctx, launch_prefill_embed(e, s));
    HIP_TRY(ctx, launch_prefill_rope(ctx->freqs, (int)ctx->hs, pos, m, ctx->pf_cos, ctx->pf_sin, s));

    auto prep = [&](const float* x, const float* gain, int64_t K) -> hipError_t {
        PrefillPrepParams q;
        q.x = x;
        q.gain = gain;
        q.eps = ctx->cfg.norm_eps;
        q.K = K;
        q.gs = (int32_t)gs;
        q.m = m;
        q.q = ctx->pf_aq;
        q.s = ctx->pf_as;
        q.xo = f32 ? xn : nullptr;
        return launch_prefill_prep(q, gain != nullptr, s, ev(PC_PREP));
    };
    auto scales = [&](float* base, int64_t off_elems) -> const float* {
        return f32 ? nullptr : base + off_elems / gs;
    };
    for (int64_t l = 0; l < ctx->L; l++) {
        PrefillGemmParams g;
        memset(&g, 0, sizeof(g));
        g.dtype = ctx->dt;
        g.gs = (int32_t)gs;
        g.m = m;
        g.combine = ctx->pf_combine;
        g.aq = ctx->pf_aq;
        g.as = ctx->pf_as;

        HIP_TRY(ctx, prep(ctx->pf_x, ctx->rms_att + l * d, d));
        g.a32 = xn;
        g.W = (const uint8_t*)ctx->wqkv + (size_t)(l * nqkv * d) * es;
        g.Ws = scales(ctx->wqkv_s, l * nqkv * d);
        g.N = nqkv;
        g.K = d;
        g.out = ctx->pf_q;
        g.ldo = d;
        g.kcache = ctx->kc + l * ctx->S * kvd;
        g.vcache = ctx->vc + l * ctx->S * kvd;
        g.d = (int32_t)d;
        g.kvd = (int32_t)kvd;
        g.hs = (int32_t)ctx->hs;
        g.pos0 = pos;
        g.rcos = ctx->pf_cos;
        g.rsin = ctx->pf_sin;
        HIP_TRY(ctx, launch_prefill_gemm(EPI_QKV, g, s, ev(PC_QKV)));

        PrefillAttnParams a;
        a.q = ctx->pf_q;
        a.kc = ctx->kc + l * ctx->S * kvd;
        a.vc = ctx->vc + l * ctx->S * kvd;
        a.o = ctx->pf_o;
        a.d = (int32_t)d;
        a.kvd = (int32_t)kvd;
        a.hs = (int32_t)ctx->hs;
        a.G = (int32_t)ctx->G;
        a.nkv = (int32_t)ctx->nkv;
        a.m = m;
        a.pos0 = pos;
        HIP_TRY(ctx, launch_prefill_attn(a, s, ev(PC_ATTN)));

        if (!f32) HIP_TRY(ctx, prep(ctx->pf_o, nullptr, d));
        g.a32 = ctx->pf_o;
        g.W = (const uint8_t*)ctx->wo + (size_t)(l * d * d) * es;
        g.Ws = scales(ctx->wo_s, l * d * d);
        g.N = d;
        g.K = d;
        g.out = ctx->pf_x;
        g.ldo = d;
        HIP_TRY(ctx, launch_prefill_gemm(EPI_RESID, g, s, ev(PC_WO)));

        HIP_TRY(ctx, prep(ctx->pf_x, ctx->rms_ffn + l * d, d));
        g.a32 = xn;
        g.W = (const uint8_t*)ctx->w13 + (size_t)(l * 2 * h * d) * es;
        g.Ws = scales(ctx->w13_s, l * 2 * h * d);
        g.N = 2 * h;
        g.K = d;
        g.out = ctx->pf_h;
        g.ldo = h;
        HIP_TRY(ctx, launch_prefill_gemm(EPI_SWIGLU, g, s, ev(PC_W13)));

        if (!f32) HIP_TRY(ctx, prep(ctx->pf_h, nullptr, h));
        g.a32 = ctx->pf_h;
        g.W = (const uint8_t*)ctx->w2 + (size_t)(l * d * h) * es;
        g.Ws = scales(ctx->w2_s, l * d * h);
        g.N = d;
        g.K = h;
        g.out = ctx->pf_x;
        g.ldo = d;
        HIP_TRY(ctx, launch_prefill_gemm(EPI_RESID, g, s, ev(PC_W2)));
    }
    return L2D_OK;
}

int prefill_impl(l2d_ctx* ctx, const int32_t* tokens, int32_t n, int32_t pos0, KernelTimer* kt)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "prefill: null context");
    if (!tokens || n <= 0 || pos0 < 0 || (int64_t)pos0 + n > ctx->S)
        return fail(ctx, L2D_EINVAL, "prefill: need tokens, n > 0 and 0 <= pos0, pos0 + n <= seq_len");
    for (int32_t i = 0; i < n; i++)
        if (tokens[i] < 0 || tokens[i] >= ctx->V) return fail(ctx, L2D_EINVAL, "prefill: token outside [0, vocab)");
    if (!prefill_supported(ctx))
        return fail(ctx, L2D_EINVAL, "prefill: needs fp32 weights or Q8_0 with group size 64, 128 or 256, "
                                     "and n_heads / n_kv_heads dividing 8");
    int rc = prefill_buffers(ctx);
    if (rc != L2D_OK) return rc;
    int m = 0;
    for (int32_t c0 = 0; c0 < n; c0 += m) {
        m = n - c0 < ctx->pf_cap ? n - c0 : ctx->pf_cap;
        HIP_TRY(ctx, hipMemcpyAsync(ctx->pf_tok, tokens + c0, (size_t)m * 4, hipMemcpyHostToDevice, ctx->stream));
        rc = enqueue_prefill_chunk(ctx, m, pos0 + c0, kt);
        if (rc != L2D_OK) return rc;
    }
    // the last token's step: step record, argmax slots and the classifier on
    // its residual row (the step-start kernel's embedding row is replaced)
    const int32_t last = pos0 + n - 1;
    if (kt) HIP_TRY(ctx, kt->next(PC_START));
    HIP_TRY(ctx, begin(ctx, tokens[n - 1], last, false, kt ? &kt->cur : nullptr));
    HIP_TRY(ctx, hipMemcpyAsync(ctx->x, ctx->pf_x + (size_t)(m - 1) * ctx->d, (size_t)ctx->d * 4,
                                hipMemcpyDeviceToDevice, ctx->stream));
    rc = enqueue_classifier(ctx, kt, PC_CLS);
    if (rc != L2D_OK) return rc;
    ctx->last_pos = last;
    return L2D_OK;
}

}  // namespace

const float* l2d_prefill(l2d_ctx* ctx, const int32_t* tokens, int32_t n, int32_t pos0)
{
    if (prefill_impl(ctx, tokens, n, pos0, nullptr) != L2D_OK) return nullptr;
    return ctx->logits;
}

int l2d_profile_prefill(l2d_ctx* ctx, const int32_t* tokens, int32_t n, int32_t pos0, double* avg_seconds)
{
    if (!ctx || !avg_seconds) return fail(ctx, L2D_EINVAL, "profile_prefill: null argument");
    KernelTimer kt;
    int rc = prefill_impl(ctx, tokens, n, pos0, &kt);
    if (rc != L2D_OK) return rc;
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    double sum[PC_COUNT] = {0};
    int cnt[PC_COUNT] = {0};
    for (size_t i = 0; i < kt.used / 2; i++) {
        float ms = 0.f;
        HIP_TRY(ctx, hipEventElapsedTime(&ms, kt.ev[2 * i], kt.ev[2 * i + 1]));
        sum[kt.cls[i]] += ms * 1e-3;
        cnt[kt.cls[i]] += 1;
    }
    for (int c = 0; c < PC_COUNT; c++) avg_seconds[c] = cnt[c] ? sum[c] / cnt[c] : 0.0;
    return L2D_OK;
}

int l2d_trace_layer(l2d_ctx* ctx, int32_t layer)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "trace_layer: null context");
    if (layer >= ctx->L) return fail(ctx, L2D_EINVAL, "trace_layer: layer out of range");
    ctx->trace_layer = layer < 0 ? -1 : layer;
    return L2D_OK;
}

int l2d_trace_read(l2d_ctx* ctx, int32_t slot, int8_t* host_q, float* host_s)
{
    if (!ctx || slot < 0 || slot > 3 || !host_q || !host_s) return fail(ctx, L2D_EINVAL, "trace_read: bad argument");
    if (ctx->dt != DT_Q8) return fail(ctx, L2D_EINVAL, "trace_read: tracing records Q8_0 codes only");
    const int64_t n = slot == 3 ? ctx->h : ctx->d;
    HIP_TRY(ctx, hipMemcpyAsync(host_q, ctx->trace_q[slot], (size_t)n, hipMemcpyDeviceToHost, ctx->stream));
    HIP_TRY(ctx, hipMemcpyAsync(host_s, ctx->trace_s[slot], (size_t)(n / ctx->gs) * 4,
                                hipMemcpyDeviceToHost, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    return L2D_OK;
}

void* l2d_stream(l2d_ctx* ctx) { return ctx ? (void*)ctx->stream : nullptr; }

int l2d_profile_step(l2d_ctx* ctx, int32_t token, int32_t pos, int32_t reps, double* avg_seconds)
{
    if (!ctx || !avg_seconds || reps <= 0) return fail(ctx, L2D_EINVAL, "profile_step: bad argument");
    if (pos < 0 || pos >= ctx->S || token < 0 || token >= ctx->V)
        return fail(ctx, L2D_EINVAL, "profile_step: token or pos out of range");
    KernelTimer kt;
    for (int r = 0; r < reps; r++) {
        HIP_TRY(ctx, kt.next(KC_BEGIN));
        HIP_TRY(ctx, begin(ctx, token, pos, false, &kt.cur));
        if (ctx->use_chain && ctx->chain_ok) ctx->chain_pending = true;
        int rc = enqueue_layers(ctx, false, &kt);
        if (rc != L2D_OK) return rc;
    }
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    double sum[KC_COUNT] = {0};
    int cnt[KC_COUNT] = {0};
    for (size_t i = 0; i < kt.used / 2; i++) {
        float ms = 0.f;
        HIP_TRY(ctx, hipEventElapsedTime(&ms, kt.ev[2 * i], kt.ev[2 * i + 1]));
        sum[kt.cls[i]] += ms * 1e-3;
        cnt[kt.cls[i]] += 1;
    }
    for (int c = 0; c < KC_COUNT; c++) avg_seconds[c] = cnt[c] ? sum[c] / cnt[c] : 0.0;
    ctx->last_pos = pos;
    return L2D_OK;
}

int l2d_set_sampling(l2d_ctx* ctx, double temperature, uint64_t seed)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "set_sampling: null context");
    if (!(temperature >= 0.0) || !isfinite(temperature))
        return fail(ctx, L2D_EINVAL, "set_sampling: temperature must be finite and >= 0");
    ctx->temperature = temperature;
    ctx->seed = seed;
    return L2D_OK;
}

int l2d_use_persistent(l2d_ctx* ctx, int32_t enable)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "use_persistent: null context");
    if (enable && !ctx->stream_ok)
        return fail(ctx, L2D_EINVAL,
                    "use_persistent: the persistent step kernel is built for Q8_0 with group size 64 "
                    "on a device with cooperative launch; not available for this model or device");
    ctx->use_stream = enable != 0;
    return L2D_OK;
}

int l2d_persistent(const l2d_ctx* ctx)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "persistent: null context");
    return ctx->use_stream && ctx->stream_ok ? 1 : 0;
}

int l2d_stream_trace(l2d_ctx* ctx, int32_t token, int32_t pos, uint64_t* host, int64_t n, int64_t* events)
{
    if (!ctx || !events) return fail(ctx, L2D_EINVAL, "stream_trace: null argument");
    if (!ctx->stream_ok) return fail(ctx, L2D_EINVAL, "stream_trace: the persistent step kernel is not available");
    const int64_t ne = stream_trace_events((int)ctx->L);
    const int64_t NP = 4 * ctx->L + 1;
    const int64_t total = (int64_t)ctx->stream_grid * (ne + stream_workers() * NP);
    *events = ne;
    if (!host) return L2D_OK;  // size query
    if (n < total) return fail(ctx, L2D_EINVAL, "stream_trace: host buffer too small");
    uint64_t* dev = nullptr;
    HIP_TRY(ctx, hipMalloc(&dev, (size_t)total * 8));
    hipError_t me = hipMemsetAsync(dev, 0, (size_t)total * 8, ctx->stream);
    const bool was = ctx->use_stream;
    ctx->use_stream = true;
    ctx->strace = dev;
    const float* r = me == hipSuccess ? forward_impl(ctx, token, pos, false) : nullptr;
    ctx->strace = nullptr;
    ctx->use_stream = was;
    int rc = r ? l2d_sync(ctx) : L2D_EHIP;
    if (rc == L2D_OK) {
        hipError_t e = hipMemcpy(host, dev, (size_t)total * 8, hipMemcpyDeviceToHost);
        if (e != hipSuccess) rc = fail(ctx, L2D_EHIP, std::string("stream_trace: ") + hipGetErrorString(e));
    }
    hipFree(dev);
    return rc;
}

int l2d_stream_shape(const l2d_ctx* ctx, int32_t* workgroups, int32_t* workers)
{
    if (!ctx || !workgroups || !workers) return fail(nullptr, L2D_EINVAL, "stream_shape: null argument");
    if (!ctx->stream_ok) return fail(const_cast<l2d_ctx*>(ctx), L2D_EINVAL, "stream_shape: the persistent step kernel is not available");
    *workgroups = ctx->stream_grid;
    *workers = stream_workers();
    return L2D_OK;
}

int l2d_prefill_combine(l2d_ctx* ctx, int32_t fp32)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "prefill_combine: null context");
    if (fp32 != 0 && fp32 != 1) return fail(ctx, L2D_EINVAL, "prefill_combine: 0 (fp64) or 1 (fp32)");
    ctx->pf_combine = fp32;
    return L2D_OK;
}

int l2d_use_graph(l2d_ctx* ctx, int32_t enable)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "use_graph: null context");
    ctx->use_graph = enable != 0;
    return L2D_OK;
}

int l2d_use_chain(l2d_ctx* ctx, int32_t enable)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "use_chain: null context");
    if (enable && !ctx->chain_ok)
        return fail(ctx, L2D_EINVAL,
                    "use_chain: chained launches are built for Q8_0 with group size 64, at most 4 query "
                    "heads per attention workgroup and dim <= 8192; not available for this model");
    if ((enable != 0) == ctx->use_chain) return L2D_OK;
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    ctx->use_chain = enable != 0;
    // the captured graph holds the launches: capture the step again
    if (ctx->exec) HIP_TRY(ctx, hipGraphExecDestroy(ctx->exec));
    if (ctx->graph) HIP_TRY(ctx, hipGraphDestroy(ctx->graph));
    ctx->exec = nullptr;
    ctx->graph = nullptr;
    return capture(ctx);
}

int l2d_chained(const l2d_ctx* ctx)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "chained: null context");
    return ctx->use_chain && ctx->chain_ok ? 1 : 0;
}

int l2d_test_chain_fault(l2d_ctx* ctx)
{
    if (!ctx) return fail(nullptr, L2D_EINVAL, "test_chain_fault: null context");
    if (!ctx->chain_ok) return fail(ctx, L2D_EINVAL, "test_chain_fault: chained launches are not available");
    const uint32_t one = 1;
    HIP_TRY(ctx, hipMemcpyAsync(ctx->chain_err, &one, 4, hipMemcpyHostToDevice, ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
    ctx->chain_pending = true;
    return L2D_OK;
}

}  // extern "C"
