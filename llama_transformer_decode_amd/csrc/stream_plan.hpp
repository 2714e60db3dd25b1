// stream_plan.hpp - who touches what in the persistent step kernel
// (stream.hip): the matvec phases of one decode step, the rows each
// workgroup and each worker wave owns, the order in which a worker streams
// its weight chunks, the addresses of those chunks, and the attention work
// items. Every function is __host__ __device__: the kernel computes its
// addresses with them, and the host checker (l2d_stream_plan_check) runs
// the same code over every wave of a launch to prove each access in bounds.
#pragma once

#include <stdint.h>

#ifndef __HIPCC__
#define __host__
#define __device__
#define __forceinline__ inline
#endif

namespace l2d {

constexpr int kSGS = 64;  // Q8_0 group size of the step kernel
constexpr int kSAW = 4;   // control waves per workgroup (prologues, epilogues, attention)

// matvec phases in step order: per layer q/k/v, output, w1/w3, w2; then the
// classifier
enum SKind { SK_QKV = 0, SK_WO = 1, SK_W13 = 2, SK_W2 = 3, SK_CLS = 4 };

struct SPlan {
    int64_t d, h, L, kvd, V;
    int64_t nwg;  // workgroups of the launch
    int64_t nwk;  // worker waves per workgroup
    // where each matrix kind's codes and scales start (bytes), from one base
    // address (the kernel's); 0 for offsets within each array
    int64_t wo0, wo1, wo2, wo3, wo4;
    int64_t so0, so1, so2, so3, so4;
};

struct SPhase {
    int kind;
    int64_t layer, M, K;
    int64_t woff;  // first code of the phase in its weight array (bytes)
    int64_t soff;  // first scale of the phase in its scale array (floats)
};

__host__ __device__ __forceinline__ int64_t sp_phases(SPlan s) { return 4 * s.L + 1; }

__host__ __device__ __forceinline__ SPhase sp_phase(SPlan s, int64_t p)
{
    SPhase f;
    if (p >= 4 * s.L) {
        f.kind = SK_CLS;
        f.layer = 0;
        f.M = s.V;
        f.K = s.d;
    } else {
        f.layer = p / 4;
        f.kind = (int)(p % 4);
        f.M = f.kind == SK_QKV ? s.d + 2 * s.kvd : f.kind == SK_W13 ? 2 * s.h : s.d;
        f.K = f.kind == SK_W2 ? s.h : s.d;
    }
    f.woff = f.layer * f.M * f.K;
    f.soff = f.layer * f.M * (f.K / kSGS);
    return f;
}

// Rows [r0, r1) of workgroup b: a balanced share of the row pairs (the q/k/v
// and w1/w3 epilogues combine rows 2i and 2i+1).
__host__ __device__ __forceinline__ void sp_wg_rows(int64_t M, int64_t b, int64_t nwg, int64_t* r0, int64_t* r1)
{
    const int64_t T = (M + 1) / 2;
    *r0 = 2 * (T * b / nwg);
    const int64_t e = 2 * (T * (b + 1) / nwg);
    *r1 = e < M ? e : M;
}

// largest row count of any workgroup in any phase (LDS size of the results)
__host__ __device__ __forceinline__ int64_t sp_max_wg_rows(SPlan s)
{
    int64_t m = 0;
    const int64_t Ms[4] = {s.d + 2 * s.kvd, s.d, 2 * s.h, s.V};
    for (int i = 0; i < 4; i++) {
        const int64_t T = (Ms[i] + 1) / 2;
        const int64_t r = 2 * ((T + s.nwg - 1) / s.nwg);
        m = r > m ? r : m;
    }
    return m;
}

// Worker w of a workgroup takes rows r0 + w, r0 + w + nwk, ... below r1.
__host__ __device__ __forceinline__ int64_t sp_worker_rows(int64_t r0, int64_t r1, int64_t w, int64_t nwk)
{
    const int64_t n = r1 - r0;
    return n > w ? (n - w + nwk - 1) / nwk : 0;
}

// chunks per row: 64 groups of 64 codes each (the last may hold fewer)
__host__ __device__ __forceinline__ int64_t sp_chunks(int64_t K) { return (K / kSGS + 63) / 64; }

// groups in chunk c of a row of K codes
__host__ __device__ __forceinline__ int64_t sp_chunk_groups(int64_t K, int64_t c)
{
    const int64_t left = K / kSGS - 64 * c;
    return left < 64 ? left : 64;
}

// Byte offset, within a phase's codes, of the 16-byte piece q (0..3) of
// lane j's group in chunk c of row r. Rows are stored group-interleaved:
// chunk c of a row holds groups 64c .. 64c + nb - 1, quarter q of group
// 64c + j at 16 * (nb * q + j). Lanes past the chunk's groups read the last
// group (their contribution is masked).
__host__ __device__ __forceinline__ int64_t sp_code_off(int64_t r, int64_t K, int64_t c, int q, int j)
{
    const int64_t nb = sp_chunk_groups(K, c);
    const int64_t jj = j < nb ? j : nb - 1;
    return r * K + c * 64 * kSGS + 16 * (nb * q + jj);
}

// float offset, within a phase's scales, of lane j's group scale in chunk c of row r
__host__ __device__ __forceinline__ int64_t sp_scale_off(int64_t r, int64_t K, int64_t c, int j)
{
    const int64_t nb = sp_chunk_groups(K, c);
    const int64_t jj = j < nb ? j : nb - 1;
    return r * (K / kSGS) + 64 * c + jj;
}

// Row ranges of one workgroup for the five matrix shapes (they do not
// depend on the layer).
struct SRows {
    int64_t r0[5], r1[5];
};

__host__ __device__ __forceinline__ SRows sp_rows(SPlan s, int64_t b)
{
    SRows r;
#pragma unroll
    for (int k = 0; k < 5; k++) {
        const SPhase f = sp_phase(s, k < 4 ? k : 4 * s.L);
        sp_wg_rows(f.M, b, s.nwg, &r.r0[k], &r.r1[k]);
    }
    return r;
}

// One worker's stream, the same in every layer: its rows of each kind
// (q/k/v, output, w1/w3, w2, classifier), the workgroup's first row of each
// kind, chunks per row (ch_d for inputs of dim values, ch_h for w2's
// hidden_dim), and the running item counts. Named scalars, no arrays: the
// kernel keeps them in scalar registers.
struct SWork {
    int64_t n0, n1, n2, n3, n4;
    int64_t b0, b1, b2, b3, b4;  // first row of each kind in the workgroup
    int64_t ch_d, ch_h;
    int64_t a0, a1, a2, per;     // items of q/k/v; + output; + w1/w3; + w2 (one layer)
    int64_t total;               // items of the whole step
};

__host__ __device__ __forceinline__ SWork sp_work(SPlan s, SRows r, int64_t w)
{
    SWork k;
    k.n0 = sp_worker_rows(r.r0[0], r.r1[0], w, s.nwk);
    k.n1 = sp_worker_rows(r.r0[1], r.r1[1], w, s.nwk);
    k.n2 = sp_worker_rows(r.r0[2], r.r1[2], w, s.nwk);
    k.n3 = sp_worker_rows(r.r0[3], r.r1[3], w, s.nwk);
    k.n4 = sp_worker_rows(r.r0[4], r.r1[4], w, s.nwk);
    k.b0 = r.r0[0];
    k.b1 = r.r0[1];
    k.b2 = r.r0[2];
    k.b3 = r.r0[3];
    k.b4 = r.r0[4];
    k.ch_d = sp_chunks(s.d);
    k.ch_h = sp_chunks(s.h);
    k.a0 = k.n0 * k.ch_d;
    k.a1 = k.a0 + k.n1 * k.ch_d;
    k.a2 = k.a1 + k.n2 * k.ch_d;
    k.per = k.a2 + k.n3 * k.ch_h;
    k.total = s.L * k.per + k.n4 * k.ch_d;
    return k;
}

// Item t of a worker's stream (0 <= t < total): phase, matrix kind, layer,
// the row (and its index among the workgroup's rows), the chunk of the row,
// and where the phase's codes and scales start. Each row's chunks are
// consecutive; phases follow in step order.
struct SItem {
    int64_t p, layer, row, local, c, nch, K, woff, soff;
    int kind;
};

__host__ __device__ __forceinline__ SItem sp_item(SPlan s, SWork k, int64_t w, int64_t t)
{
    // 32-bit arithmetic: a worker streams far fewer than 2^31 items
    const int32_t t32 = (int32_t)t, per = (int32_t)k.per;
    SItem it;
    int32_t r;
    if (t < s.L * k.per) {
        const int32_t layer = t32 / per;
        it.layer = layer;
        r = t32 - layer * per;
        it.kind = r < (int32_t)k.a0 ? SK_QKV : r < (int32_t)k.a1 ? SK_WO : r < (int32_t)k.a2 ? SK_W13 : SK_W2;
        r -= it.kind == SK_QKV ? 0 : it.kind == SK_WO ? (int32_t)k.a0 : it.kind == SK_W13 ? (int32_t)k.a1 : (int32_t)k.a2;
        it.p = 4 * (int64_t)layer + it.kind;
    } else {
        it.kind = SK_CLS;
        it.layer = 0;
        r = (int32_t)(t - s.L * k.per);
        it.p = 4 * s.L;
    }
    const int32_t nch = (int32_t)(it.kind == SK_W2 ? k.ch_h : k.ch_d);
    it.nch = nch;
    const int32_t j = nch == 1 ? r : r / nch;
    it.c = r - j * nch;
    it.local = w + (int64_t)j * s.nwk;
    const int64_t base = it.kind == SK_QKV ? k.b0 : it.kind == SK_WO ? k.b1 : it.kind == SK_W13 ? k.b2
                       : it.kind == SK_W2  ? k.b3 : k.b4;
    it.row = base + it.local;
    const SPhase f = sp_phase(s, it.p);
    it.K = f.K;
    it.woff = f.woff;
    it.soff = f.soff;
    return it;
}

// The kernel's form of a worker's stream: a table of chunk descriptors,
// built on the host from the enumeration above (the items of one layer, then
// the classifier's), so the kernel walks it with one scalar load per chunk
// and no address arithmetic beyond a layer multiply. A worker with no rows of
// a kind gets one phantom item there (it loads a dummy address and computes
// nothing), so every worker passes through every phase in order. The host
// checker expands each table over the layers and requires the items of
// sp_item, in order.
struct SDesc {
    int64_t w0;  // byte offset (from the kernel's weight base) of the chunk's codes in layer 0
    int64_t s0;  // byte offset of the chunk's group scales in layer 0
    int32_t wl;  // code bytes from one layer to the next (0 for the classifier)
    int32_t sl;  // scale bytes from one layer to the next
    uint32_t meta;
    uint32_t pad;
};

// meta word: kind in bits 0-2, flags, groups of the chunk (1..64) in bits
// 6-12, chunk of the row in bits 13-16, the row's index among the
// workgroup's rows in bits 17-31
enum : uint32_t {
    SD_ROWEND = 1u << 3,   // the row's last chunk: reduce and store its sum
    SD_FIRST = 1u << 4,    // the worker's first item of its phase
    SD_PHANTOM = 1u << 5,  // no rows of this kind: load nothing real, compute nothing
};

__host__ __device__ __forceinline__ uint32_t sd_meta(int kind, bool rowend, bool first, bool phantom, int64_t nb,
                                                     int64_t c, int64_t local)
{
    return (uint32_t)kind | (rowend ? SD_ROWEND : 0u) | (first ? SD_FIRST : 0u) | (phantom ? SD_PHANTOM : 0u) |
           ((uint32_t)nb << 6) | ((uint32_t)c << 13) | ((uint32_t)local << 17);
}
__host__ __device__ __forceinline__ int sd_kind(uint32_t m) { return (int)(m & 7u); }
__host__ __device__ __forceinline__ int sd_nb(uint32_t m) { return (int)((m >> 6) & 127u); }
__host__ __device__ __forceinline__ int sd_c(uint32_t m) { return (int)((m >> 13) & 15u); }
__host__ __device__ __forceinline__ int sd_local(uint32_t m) { return (int)(m >> 17); }

// limits of the meta fields and of the per-layer strides
__host__ __device__ __forceinline__ bool sd_fits(SPlan s)
{
    const int64_t kmax = s.d > s.h ? s.d : s.h;
    const int64_t big = 2 * s.h * s.d > s.V * s.d ? 2 * s.h * s.d : s.V * s.d;
    return sp_chunks(kmax) <= 16 && sp_max_wg_rows(s) < 32768 && big < ((int64_t)1 << 31);
}

// Attention work items: (kv head g, query-head subset hsub of gsplit, range
// split of ns); item it covers kv head column vg = it / ns, split it % ns.
__host__ __device__ __forceinline__ int64_t sp_attn_items(int64_t nkv, int64_t gsplit, int64_t ns)
{
    return nkv * gsplit * ns;
}

}  // namespace l2d
