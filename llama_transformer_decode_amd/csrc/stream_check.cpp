// stream_check.cpp - host check of the persistent step kernel's plan: the
// same stream_plan.hpp functions the kernel computes its addresses with, run
// over every wave of a launch, before the kernel ever runs on a device.
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "attn_core.hpp"
#include "internal.hpp"
#include "l2d.h"
#include "runtime.hpp"
#include "stream_plan.hpp"

namespace l2d {

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

void check_streams(const SPlan& s, int64_t ymax, Check& ck)
{
    const int64_t NP = sp_phases(s);
    // rows x chunks of the first layer's phases and the classifier, counted
    // over all waves: every one exactly once
    std::vector<std::vector<int>> seen(5);
    for (int k = 0; k < 5; k++) {
        const SPhase f = sp_phase(s, k < 4 ? k : 4 * s.L);
        seen[k].assign((size_t)(f.M * sp_chunks(f.K)), 0);
    }
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
            const SWork wk = sp_work(s, rows, w);
            int64_t last_p = -1, last_row = -1, last_c = -1;
            SKindRun tab[5];
            for (int k = 0; k < 5; k++) tab[k] = sp_kind_run(s, rows, w, k);
            SCur cur;
            sc_begin(cur, tab, w);
            int64_t cur_phase = -1;
            for (int64_t t = 0; t < wk.total && ck.ok(); t++) {
                const SItem u = sp_item(s, wk, w, t);
                // the kernel's incremental cursor walks the same items, with
                // one phantom item in each phase where the worker has no rows
                // (every phase in order)
                while (!cur.end && cur.phantom) {
                    if (sc_phase(cur, s) != cur_phase + 1) ck.fail("workgroup %lld worker %lld: phase skipped", b, w);
                    cur_phase = sc_phase(cur, s);
                    sc_step(cur, s, tab, w);
                }
                if (cur.end || sc_phase(cur, s) != u.p || cur.kind != u.kind || cur.local != u.local ||
                    cur.c != u.c || cur.nch != u.nch || cur.K != u.K ||
                    cur.woff != u.woff + u.row * u.K || cur.soff != u.soff + u.row * (u.K / kSGS) ||
                    sc_groups(cur) != sp_chunk_groups(u.K, u.c))
                    ck.fail("workgroup %lld worker %lld: cursor differs from the plan at item %lld", b, w, t);
                if (sc_phase(cur, s) != cur_phase && sc_phase(cur, s) != cur_phase + 1)
                    ck.fail("workgroup %lld worker %lld: phase skipped", b, w);
                cur_phase = sc_phase(cur, s);
                sc_step(cur, s, tab, w);
                const SPhase f = sp_phase(s, u.p);
                if (u.p < last_p) ck.fail("workgroup %lld worker %lld: phase order at item %lld", b, w, t);
                // a row's chunks are consecutive and in order
                if (u.c > 0 && (u.row != last_row || u.c != last_c + 1 || u.p != last_p))
                    ck.fail("workgroup %lld worker %lld: chunk order at item %lld", b, w, t);
                last_p = u.p;
                last_row = u.row;
                last_c = u.c;
                if (f.kind != u.kind || f.K != u.K || f.woff != u.woff || f.soff != u.soff)
                    ck.fail("workgroup %lld worker %lld phase %lld: item fields", b, w, u.p);
                const int64_t local = u.local;
                const int64_t row = u.row;
                if (local < 0 || local >= rows.r1[u.kind] - rows.r0[u.kind] || local >= ymax ||
                    row != rows.r0[u.kind] + local)
                    ck.fail("workgroup %lld worker %lld: local row %lld", b, w, local);
                if (row < 0 || row >= f.M) ck.fail("workgroup %lld worker %lld: row %lld of %lld", b, w, row, f.M);
                if (u.c < 0 || u.c >= u.nch || u.nch != sp_chunks(u.K))
                    ck.fail("workgroup %lld worker %lld: chunk %lld", b, w, u.c);
                const int64_t cb = codes_of(s, u.kind);
                const int64_t lo = u.woff + sp_code_off(row, u.K, u.c, 0, 0);
                const int64_t hi = u.woff + sp_code_off(row, u.K, u.c, 3, 63) + 16;
                if (lo < 0 || hi > cb) ck.fail("workgroup %lld worker %lld: codes [%lld, %lld) out of range", b, w, lo, hi);
                // the chunk's codes lie inside its row
                if (lo < u.woff + row * u.K || hi > u.woff + (row + 1) * u.K)
                    ck.fail("workgroup %lld worker %lld: chunk leaves row %lld", b, w, row);
                const int64_t slo = u.soff + sp_scale_off(row, u.K, u.c, 0);
                const int64_t shi = u.soff + sp_scale_off(row, u.K, u.c, 63) + 1;
                if (slo < 0 || shi > cb / kSGS) ck.fail("workgroup %lld worker %lld: scales [%lld, %lld)", b, w, slo, shi);
                if (u.p < 4 || u.p == NP - 1) {
                    const int k = u.p < 4 ? (int)u.p : 4;
                    seen[k][(size_t)(row * u.nch + u.c)] += 1;
                }
            }
            while (!cur.end && cur.phantom) {
                if (sc_phase(cur, s) != cur_phase + 1) ck.fail("workgroup %lld worker %lld: phase skipped", b, w);
                cur_phase = sc_phase(cur, s);
                sc_step(cur, s, tab, w);
            }
            if (!cur.end || cur_phase != NP - 1)
                ck.fail("workgroup %lld worker %lld: cursor does not end with the plan", b, w);
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
        if (!stream_supported(L2D_Q8_0, cfg->group_size, d, h, G, gsplit, (int)hs)) {
            ck.fail("model not supported by the step kernel");
        } else {
            const SPlan s{d, h, L, kvd, V, nwg, stream_workers(), 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
            const int64_t ymax = sp_max_wg_rows(s);
            check_streams(s, ymax, ck);
            const int64_t ns = stream_splits(nkv, gsplit, nwg, cfg->seq_len, (int)hs);
            check_attention(nkv, gsplit, ns, cfg->seq_len, (int)hs, ck);
            const size_t lds = stream_lds_bytes(s, G / gsplit, (int)hs);
            if (lds > 160 * 1024) ck.fail("LDS %lld bytes > 160 KiB", (long long)lds);
        }
    }
    if (msg && msglen > 0) {
        snprintf(msg, (size_t)msglen, "%s", ck.ok() ? "ok" : ck.first.c_str());
    }
    return ck.ok() ? L2D_OK : L2D_EINVAL;
}
