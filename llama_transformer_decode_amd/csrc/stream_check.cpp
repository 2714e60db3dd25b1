// stream_check.cpp - host check of the persistent step kernel's plan: the
// same stream_plan.hpp functions the kernel computes its addresses with, run
// over every wave of a launch, before the kernel ever runs on a device.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "attn_core.hpp"
#include "internal.hpp"
#include "l2d.h"
#include "runtime.hpp"
#include "stream_plan.hpp"

namespace l2d {

// Every worker's chunk table: worker wid = b * nwk + w at tab[wid * stride],
// its items of one layer (kinds q/k/v, output, w1/w3, w2) followed by its
// classifier items; cnt[2 wid] and cnt[2 wid + 1] count them.
void stream_tables(const SPlan& s, std::vector<SDesc>& tab, std::vector<int32_t>& cnt, int64_t* stride)
{
    const int64_t wofs[5] = {s.wo0, s.wo1, s.wo2, s.wo3, s.wo4};
    const int64_t sofs[5] = {s.so0, s.so1, s.so2, s.so3, s.so4};
    const int64_t nw = s.nwg * s.nwk;
    std::vector<std::vector<SDesc>> per((size_t)nw);
    cnt.assign((size_t)(2 * nw), 0);
    int64_t longest = 1;
    for (int64_t b = 0; b < s.nwg; b++) {
        const SRows rows = sp_rows(s, b);
        for (int64_t w = 0; w < s.nwk; w++) {
            const int64_t wid = b * s.nwk + w;
            std::vector<SDesc>& it = per[(size_t)wid];
            for (int k = 0; k < 5; k++) {
                if (k == SK_CLS) cnt[2 * wid] = (int32_t)it.size();
                const SPhase f = sp_phase(s, k < 4 ? k : 4 * s.L);
                const int64_t n = sp_worker_rows(rows.r0[k], rows.r1[k], w, s.nwk);
                const int64_t nch = sp_chunks(f.K);
                const int32_t wl = k == SK_CLS ? 0 : (int32_t)(f.M * f.K);
                const int32_t sl = k == SK_CLS ? 0 : (int32_t)(4 * f.M * (f.K / kSGS));
                if (n == 0) {
                    it.push_back(SDesc{wofs[k], sofs[k], 0, 0, sd_meta(k, false, true, true, 1, 0, 0), 0});
                    continue;
                }
                for (int64_t j = 0; j < n; j++) {
                    const int64_t local = w + j * s.nwk, row = rows.r0[k] + local;
                    for (int64_t c = 0; c < nch; c++) {
                        SDesc e;
                        e.w0 = wofs[k] + sp_code_off(row, f.K, c, 0, 0);
                        e.s0 = sofs[k] + 4 * sp_scale_off(row, f.K, c, 0);
                        e.wl = wl;
                        e.sl = sl;
                        e.meta = sd_meta(k, c == nch - 1, j == 0 && c == 0, false, sp_chunk_groups(f.K, c), c, local);
                        e.pad = 0;
                        it.push_back(e);
                    }
                }
            }
            cnt[2 * wid + 1] = (int32_t)(it.size() - (size_t)cnt[2 * wid]);
            if ((int64_t)it.size() > longest) longest = (int64_t)it.size();
        }
    }
    *stride = longest;
    tab.assign((size_t)(nw * longest), SDesc{0, 0, 0, 0, 0, 0});
    for (int64_t i = 0; i < nw; i++)
        std::copy(per[(size_t)i].begin(), per[(size_t)i].end(), tab.begin() + i * longest);
}

namespace {

struct Check {
    std::string first;
    bool ok() const { return first.empty(); }
    void fail(const char* fmt, long long a = 0, long long b = 0, long long c = 0, long long d = 0)
    {
        if (!first.empty()) return;
        char buf[256];
        snprintf(buf, sizeof(buf), fmt, a, b, c, d);
        first = buf;
    }
};

// bytes of codes of each matrix kind (all layers)
int64_t codes_of(const SPlan& s, int kind)
{
    const SPhase f = sp_phase(s, kind < 4 ? kind : 4 * s.L);
    return kind == SK_CLS ? f.M * f.K : s.L * f.M * f.K;
}

// The chunk tables the kernel walks (stream_tables), expanded over the
// layers, against the plan's enumeration (sp_item): the same items in the
// same order, one phantom item exactly where a worker has no rows of a
// kind, the phase-start and row-end flags where they belong, every code and
// scale load inside its array and its row, every (row, chunk) of layer 0 and
// of the classifier streamed exactly once over all waves.
void check_streams(const SPlan& s, int64_t ymax, Check& ck)
{
    std::vector<SDesc> tab;
    std::vector<int32_t> cnt;
    int64_t stride = 0;
    stream_tables(s, tab, cnt, &stride);
    std::vector<std::vector<int>> seen(5);
    for (int k = 0; k < 5; k++) {
        const SPhase f = sp_phase(s, k < 4 ? k : 4 * s.L);
        seen[k].assign((size_t)(f.M * sp_chunks(f.K)), 0);
    }
    const int64_t wofs[5] = {s.wo0, s.wo1, s.wo2, s.wo3, s.wo4};
    const int64_t sofs[5] = {s.so0, s.so1, s.so2, s.so3, s.so4};
    for (int64_t b = 0; b < s.nwg && ck.ok(); b++) {
        const SRows rows = sp_rows(s, b);
        for (int k = 0; k < 5; k++) {
            const SPhase f = sp_phase(s, k < 4 ? k : 4 * s.L);
            if (rows.r0[k] < 0 || rows.r0[k] > rows.r1[k] || rows.r1[k] > f.M || (rows.r0[k] & 1))
                ck.fail("workgroup %lld kind %lld: rows [%lld, %lld)", b, k, rows.r0[k], rows.r1[k]);
            if (rows.r1[k] - rows.r0[k] > ymax) ck.fail("workgroup %lld kind %lld: %lld rows > ymax", b, k, rows.r1[k] - rows.r0[k]);
            // consecutive workgroups tile [0, M)
            int64_t p0, p1;
            sp_wg_rows(f.M, b + 1 < s.nwg ? b + 1 : b, s.nwg, &p0, &p1);
            if (b + 1 < s.nwg && p0 != rows.r1[k]) ck.fail("kind %lld: gap after workgroup %lld", k, b);
            if (b == 0 && rows.r0[k] != 0) ck.fail("kind %lld: rows do not start at 0", k);
            if (b + 1 == s.nwg && rows.r1[k] != f.M) ck.fail("kind %lld: rows do not end at M", k);
        }
        for (int64_t w = 0; w < s.nwk && ck.ok(); w++) {
            const int64_t wid = b * s.nwk + w;
            const SDesc* t0 = tab.data() + wid * stride;
            const int64_t nL = cnt[2 * wid], nC = cnt[2 * wid + 1];
            if (nL < 4 || nC < 1 || nL + nC > stride) ck.fail("worker %lld: table sizes %lld + %lld", wid, nL, nC);
            const SWork wk = sp_work(s, rows, w);
            int64_t t = 0;  // next item of the enumeration
            int64_t phase = -1;
            for (int64_t l = 0; l <= s.L && ck.ok(); l++) {
                const int64_t i0 = l < s.L ? 0 : nL, i1 = l < s.L ? nL : nL + nC;
                for (int64_t i = i0; i < i1 && ck.ok(); i++) {
                    const SDesc& e = t0[i];
                    const int kind = sd_kind(e.meta);
                    const int64_t p = kind == SK_CLS ? 4 * s.L : 4 * l + kind;
                    if (kind > SK_CLS || (kind == SK_CLS) != (l == s.L))
                        ck.fail("worker %lld: item %lld of layer %lld has kind %lld", wid, i, l, kind);
                    // every phase is entered once, in order, by its first item
                    const bool first = (e.meta & SD_FIRST) != 0;
                    if (first != (p != phase) || (first && p != phase + 1))
                        ck.fail("worker %lld layer %lld item %lld: phase flag (phase %lld after %lld)", wid, l, i, p);
                    phase = p;
                    if (e.meta & SD_PHANTOM) {
                        const int64_t nrows = sp_worker_rows(rows.r0[kind], rows.r1[kind], w, s.nwk);
                        if (nrows != 0 || !first || sd_nb(e.meta) != 1)
                            ck.fail("worker %lld: phantom item of kind %lld with %lld rows", wid, kind, nrows);
                        continue;
                    }
                    if (t >= wk.total) {
                        ck.fail("worker %lld: more table items than the plan's %lld", wid, wk.total);
                        break;
                    }
                    const SItem u = sp_item(s, wk, w, t++);
                    const SPhase f = sp_phase(s, u.p);
                    const int64_t L0 = kind == SK_CLS ? 0 : l;
                    const int64_t w0 = e.w0 + L0 * e.wl, s0 = e.s0 + L0 * e.sl;
                    if (u.p != p || u.kind != kind || u.c != sd_c(e.meta) || u.local != sd_local(e.meta) ||
                        sd_nb(e.meta) != sp_chunk_groups(u.K, u.c) ||
                        ((e.meta & SD_ROWEND) != 0) != (u.c == u.nch - 1) ||
                        w0 != wofs[kind] + u.woff + sp_code_off(u.row, u.K, u.c, 0, 0) ||
                        s0 != sofs[kind] + 4 * (u.soff + sp_scale_off(u.row, u.K, u.c, 0)) ||
                        e.wl != (kind == SK_CLS ? 0 : f.M * f.K) || e.sl != (kind == SK_CLS ? 0 : 4 * f.M * (f.K / kSGS)))
                        ck.fail("worker %lld: table item %lld of layer %lld differs from the plan's item %lld", wid, i, l, t - 1);
                    const int64_t local = u.local, row = u.row;
                    if (local < 0 || local >= rows.r1[kind] - rows.r0[kind] || local >= ymax ||
                        row != rows.r0[kind] + local)
                        ck.fail("worker %lld: local row %lld", wid, local);
                    if (row < 0 || row >= f.M) ck.fail("worker %lld: row %lld of %lld", wid, row, f.M);
                    // what the kernel loads: lanes j < nb read 16 bytes at
                    // w0 + 16 * (nb * q + j), q < 4, and the scale at s0 + 4 j
                    const int64_t nb = sd_nb(e.meta);
                    const int64_t cb = codes_of(s, kind);
                    const int64_t lo = w0 - wofs[kind], hi = w0 - wofs[kind] + 16 * (nb * 3 + nb - 1) + 16;
                    if (lo < 0 || hi > cb) ck.fail("worker %lld: codes [%lld, %lld) out of range", wid, lo, hi);
                    if (lo < u.woff + row * u.K || hi > u.woff + (row + 1) * u.K)
                        ck.fail("worker %lld: chunk leaves row %lld", wid, row);
                    const int64_t slo = s0 - sofs[kind], shi = s0 - sofs[kind] + 4 * nb;
                    if (slo < 0 || shi > 4 * (cb / kSGS)) ck.fail("worker %lld: scales [%lld, %lld)", wid, slo, shi);
                    if (u.p < 4 || u.p == 4 * s.L) {
                        const int k = u.p < 4 ? (int)u.p : 4;
                        seen[k][(size_t)(row * u.nch + u.c)] += 1;
                    }
                }
            }
            if (ck.ok() && (t != wk.total || phase != 4 * s.L))
                ck.fail("worker %lld: table ends at item %lld of %lld, phase %lld", wid, t, wk.total, phase);
        }
    }
    for (int k = 0; k < 5 && ck.ok(); k++)
        for (size_t i = 0; i < seen[k].size(); i++)
            if (seen[k][i] != 1) {
                ck.fail("kind %lld: row-chunk %lld streamed %lld times", k, (long long)i, seen[k][i]);
                break;
            }
}

// attention items: every position 0..pos of every kv head column in exactly
// one active range, partial slots inside their allocation
void check_attention(int64_t nkv, int64_t gsplit, int64_t ns, int64_t S, int hs, Check& ck)
{
    const int sc = attention_positions_per_subchunk(hs);
    const int64_t cols = nkv * gsplit;
    for (int64_t T = 1; T <= S && ck.ok(); T += (T < 256 ? 1 : 97)) {
        int nact = 0;
        const int per = attn_split((int)T, (int)ns, sc, &nact);
        if (nact < 1 || nact > ns) ck.fail("T %lld: %lld active ranges of %lld", T, nact, ns);
        int64_t covered = 0;
        for (int64_t c = 0; c < nact; c++) {
            const int64_t r0 = c * per, n = T - r0 < per ? T - r0 : per;
            if (n <= 0 || r0 + n > T) ck.fail("T %lld: range %lld [%lld, +%lld)", T, c, r0, n);
            covered += n;
        }
        if (covered != T) ck.fail("T %lld: ranges cover %lld positions", T, covered);
        const int64_t last_slot = (cols - 1) * ns + (nact - 1);
        if (last_slot >= cols * ns) ck.fail("T %lld: partial slot %lld", T, last_slot);
    }
}

}  // namespace

}  // namespace l2d

using namespace l2d;

extern "C" int l2d_stream_plan_check(const l2d_config* cfg, int32_t nwg, char* msg, int32_t msglen)
{
    Check ck;
    if (!cfg || nwg <= 0) {
        ck.fail("null config or nwg <= 0");
    } else if (validate_config(cfg) != L2D_OK) {
        ck.fail("invalid config");
    } else {
        const int64_t d = cfg->dim, h = cfg->hidden_dim, L = cfg->n_layers;
        const int64_t nh = cfg->n_heads, nkv = cfg->n_kv_heads, hs = d / nh, kvd = nkv * hs;
        const int64_t V = cfg->vocab_size < 0 ? -(int64_t)cfg->vocab_size : cfg->vocab_size;
        const int G = (int)(nh / nkv);
        const int gsplit = G == 8 ? 2 : 1;
        const SPlan s{d, h, L, kvd, V, nwg, stream_workers(), 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        if (!stream_supported(L2D_Q8_0, cfg->group_size, d, h, G, gsplit, (int)hs) || !sd_fits(s)) {
            ck.fail("model not supported by the step kernel");
        } else {
            const int64_t ymax = sp_max_wg_rows(s);
            check_streams(s, ymax, ck);
            const int64_t ns = stream_splits(nkv, gsplit, nwg, cfg->seq_len, (int)hs);
            check_attention(nkv, gsplit, ns, cfg->seq_len, (int)hs, ck);
            std::vector<SDesc> tab;
            std::vector<int32_t> cnt;
            int64_t stride = 0;
            stream_tables(s, tab, cnt, &stride);
            const size_t lds = stream_lds_bytes(s, G / gsplit, (int)hs, stride);
            if (lds > 160 * 1024) ck.fail("LDS %lld bytes > 160 KiB", (long long)lds);
        }
    }
    if (msg && msglen > 0) {
        snprintf(msg, (size_t)msglen, "%s", ck.ok() ? "ok" : ck.first.c_str());
    }
    return ck.ok() ? L2D_OK : L2D_EINVAL;
}
