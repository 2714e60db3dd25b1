// blob.cpp - host-side parser of the llama2.c-style weight blob.
//
// Layout (pomoai.com hub page, data-format section: a header of config
// fields, then contiguous fp32 or int8 arrays): seven int32 header fields,
// then emb, rms_att, wq, wk, wv, wo, rms_ffn, w1, w2, w3, rms_final, two
// legacy freq_cis tables of seq_len*head_size/2 floats each that are skipped
// (Q&A page, freq_cis question), and wcls only when vocab_size < 0 (Q&A page,
// shared_weights question). In a Q8_0 blob each matrix is int8 codes[n]
// followed by fp32 scales[n/GS]; in a Q4_0 blob packed 4-bit codes[n/2]
// followed by fp32 scales[n/32]. Every offset is 64-bit: the Q&A page
// records a pointer-arithmetic overflow at 13B and above.
#include <stdint.h>
#include <string.h>

#include "l2d.h"
#include "runtime.hpp"

namespace {

struct Cursor {
    const uint8_t* p;
    const uint8_t* end;
    bool ok = true;

    const void* take(uint64_t bytes)
    {
        if (!ok || (uint64_t)(end - p) < bytes) {
            ok = false;
            return nullptr;
        }
        const void* r = p;
        p += bytes;
        return r;
    }
};

void take_matrix(Cursor& c, int32_t dtype, int32_t gs, uint64_t n, const void** m, const float** s)
{
    if (dtype == L2D_F32) {
        *m = c.take(n * 4);
        *s = nullptr;
    } else if (dtype == L2D_Q4_0) {
        *m = c.take(n / 2);
        *s = (const float*)c.take((n / 32) * 4);
    } else {
        *m = c.take(n);
        *s = (const float*)c.take((n / (uint64_t)gs) * 4);
    }
}

}  // namespace

extern "C" int l2d_blob_parse(const void* blob, uint64_t nbytes, int32_t dtype, int32_t gs,
                              l2d_config* cfg, l2d_weights* w)
{
    if (!blob || !cfg || !w || nbytes < 28) return l2d::fail(nullptr, L2D_EINVAL, "blob_parse: null pointer or blob shorter than its header");
    if (dtype != L2D_F32 && dtype != L2D_Q8_0 && dtype != L2D_Q4_0)
        return l2d::fail(nullptr, L2D_EINVAL, "blob_parse: dtype must be L2D_F32, L2D_Q8_0 or L2D_Q4_0");
    if (dtype == L2D_Q4_0 && gs != 32) return l2d::fail(nullptr, L2D_EINVAL, "blob_parse: Q4_0 needs group size 32");
    l2d_config c;
    memset(&c, 0, sizeof(c));
    memcpy(&c, blob, 28);
    c.dtype = dtype;
    c.group_size = dtype == L2D_F32 ? 0 : gs;
    c.rope_theta = 10000.0;
    c.norm_eps = 1e-5;
    int rc = l2d::validate_config(&c);
    if (rc != L2D_OK) return rc;

    const uint64_t d = (uint64_t)c.dim, h = (uint64_t)c.hidden_dim, L = (uint64_t)c.n_layers;
    const uint64_t V = (uint64_t)(c.vocab_size < 0 ? -(int64_t)c.vocab_size : c.vocab_size);
    const uint64_t hs = d / (uint64_t)c.n_heads, kvd = (uint64_t)c.n_kv_heads * hs;
    const uint64_t S = (uint64_t)c.seq_len;

    Cursor cur{(const uint8_t*)blob + 28, (const uint8_t*)blob + nbytes};
    l2d_weights o;
    memset(&o, 0, sizeof(o));
    take_matrix(cur, dtype, gs, V * d, &o.emb, &o.emb_s);
    o.rms_att = (const float*)cur.take(L * d * 4);
    take_matrix(cur, dtype, gs, L * d * d, &o.wq, &o.wq_s);
    take_matrix(cur, dtype, gs, L * kvd * d, &o.wk, &o.wk_s);
    take_matrix(cur, dtype, gs, L * kvd * d, &o.wv, &o.wv_s);
    take_matrix(cur, dtype, gs, L * d * d, &o.wo, &o.wo_s);
    o.rms_ffn = (const float*)cur.take(L * d * 4);
    take_matrix(cur, dtype, gs, L * h * d, &o.w1, &o.w1_s);
    take_matrix(cur, dtype, gs, L * d * h, &o.w2, &o.w2_s);
    take_matrix(cur, dtype, gs, L * h * d, &o.w3, &o.w3_s);
    o.rms_final = (const float*)cur.take(d * 4);
    cur.take(S * (hs / 2) * 4);  // legacy freq_cis_real
    cur.take(S * (hs / 2) * 4);  // legacy freq_cis_imag
    if (c.vocab_size > 0) {
        o.wcls = o.emb;
        o.wcls_s = o.emb_s;
    } else {
        take_matrix(cur, dtype, gs, V * d, &o.wcls, &o.wcls_s);
    }
    if (!cur.ok || cur.p != cur.end)
        return l2d::fail(nullptr, L2D_EFORMAT, "blob_parse: blob size does not match the size its header implies");
    *cfg = c;
    *w = o;
    return L2D_OK;
}
