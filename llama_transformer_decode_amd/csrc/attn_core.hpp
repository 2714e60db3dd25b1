// attn_core.hpp - single-query GQA attention over one range of cached
// positions of one kv head, for a workgroup of NT threads. Shared by the
// standalone attention kernel (attn.hip) and the persistent step kernel
// (stream.hip), and by the batched prefill's vector attention kernel.
//
// For query head h and its kv head g = h / G (G = n_heads / n_kv_heads query
// heads share a kv head: Q&A page, GQA question), over cached positions
// t in [r0, r0 + n) (Q&A page, KV-cache question: k, v of position t sit at
// t * kv_dim in the layer's cache):
//     s_t = q_h . k_t / sqrt(hs),  a = softmax(s),  o_h = sum_t a_t v_t.
// The workgroup serves all G query heads of g, so every K/V row is read from
// HBM once per step whatever G is. The range is walked in sub-chunks of SC
// positions, grouped into super-chunks of up to kSuperPos positions. K rows
// stream two sub-chunks ahead across the whole range; the V rows of a
// super-chunk's first two sub-chunks are loaded when its scores start, the
// rest two ahead while its values accumulate. Per super-chunk:
//   scores  per sub-chunk: LPK lanes per position (16-byte loads,
//           interleaved so the LPK lanes read LPK*16 contiguous bytes), G fp64
//           dots, DPP lane sums, into LDS;
//   softmax per head, online in fp64 over super-chunks: the super-chunk's
//           maximum, e^{s - m} for each of its positions, running max m and
//           sum l, rescale factor e^{m_old - m_new} for what was accumulated
//           before (one pass and three barriers per super-chunk);
//   values  per sub-chunk: thread = (float4 column f, position slot), G fp64
//           double4 accumulators.
// On return the slot partial sums of the values sit in LDS (attn_value sums
// them in a fixed order) with the running (m, l) of each head.
//
// Several query tokens at once (batched prefill): the G "heads" of a range
// may be Gt query heads of each of G / Gt consecutive tokens. Head h then
// belongs to token h / Gt, reads its query row at q + (h / Gt) * qstride +
// (h % Gt) * hs, and sees positions t <= last0 + h / Gt only (causal mask:
// later positions score -inf and add exactly nothing). A range starting at
// position 0 keeps every head's running maximum finite from its first
// sub-chunk on.
#pragma once

#include "device.hpp"
#include "internal.hpp"

namespace l2d {

constexpr int kMaxG = 8;    // query heads per kv head held in registers
constexpr int kMaxKPT = 4;  // K float4 per lane per sub-chunk
constexpr int kMaxVPT = 4;  // V float4 per thread per sub-chunk
constexpr int kSuperPos = 128;  // positions per softmax pass (a whole number of sub-chunks)

struct AttnShape {
    int F;      // float4 per head row
    int lpk;    // lanes per position in the score phase
    int sc;     // positions per sub-chunk
    int kpt;    // K float4 per lane
    int slots;  // position slots in the value phase
    int vpt;    // V float4 per thread
    int nred;   // partial sums per output element left in LDS
};

template <int NT>
__host__ __device__ inline AttnShape attn_shape(int hs)
{
    AttnShape a;
    a.F = hs / 4;
    a.lpk = (a.F % 8 == 0) ? 8 : (a.F % 4 == 0) ? 4 : (a.F % 2 == 0) ? 2 : 1;
    a.sc = NT / a.lpk;
    if (a.sc > 128) a.sc = 128;
    a.kpt = a.F / a.lpk;
    a.slots = NT / a.F;
    a.vpt = (a.sc + a.slots - 1) / a.slots;
    a.nred = (64 % a.F) == 0 ? NT / 64 : a.slots;
    return a;
}

// positions per super-chunk: whole sub-chunks, at most kSuperPos (at least one)
__host__ __device__ inline int attn_super_pos(const AttnShape& a)
{
    return a.sc >= kSuperPos ? a.sc : (kSuperPos / a.sc) * a.sc;
}

template <int NT>
__host__ __device__ inline size_t attn_core_lds_bytes(int G, int hs)
{
    const AttnShape a = attn_shape<NT>(hs);
    const size_t q = (((size_t)G * hs * 4) + 15) & ~(size_t)15;
    const size_t sc = (size_t)G * attn_super_pos(a) * 8;
    const size_t stats = (size_t)3 * kMaxG * 8;
    const size_t red = (size_t)a.nred * G * hs * 8;
    return q + sc + stats + red;
}

template <int NT>
inline bool attn_core_supported(int G, int hs)
{
    const AttnShape a = attn_shape<NT>(hs);
    return (G == 1 || G == 2 || G == 4 || G == 8) && hs % 4 == 0 && a.F <= 64 && a.kpt <= kMaxKPT &&
           a.vpt <= kMaxVPT && a.slots >= 1;
}

__device__ __forceinline__ double lanes_sum_f64(double v, int width)
{
    if (width >= 2) {
        const int lo = dpp_xor1(__double2loint(v)), hi = dpp_xor1(__double2hiint(v));
        v += __hiloint2double(hi, lo);
    }
    if (width >= 4) {
        const int lo = dpp_xor2(__double2loint(v)), hi = dpp_xor2(__double2hiint(v));
        v += __hiloint2double(hi, lo);
    }
    // every lane of a quad now holds the same partial sum: the half-row and
    // row mirrors pair it with the other quad / half-row, as xor 4 / xor 8
    if (width >= 8) {
        const int lo = dpp_hmirror(__double2loint(v)), hi = dpp_hmirror(__double2hiint(v));
        v += __hiloint2double(hi, lo);
    }
    if (width >= 16) {
        const int lo = dpp_mirror(__double2loint(v)), hi = dpp_mirror(__double2hiint(v));
        v += __hiloint2double(hi, lo);
    }
    for (int m = 16; m < width; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

struct KBuf {
    f32x4 k[kMaxKPT];
};
struct VBuf {
    f32x4 v[kMaxVPT];
};

// What one range needs: this kv head's G query rows, the layer's caches.
struct AttnRange {
    const float* q;   // [G][hs] query rows of kv head g (written this launch)
    const float* kc;  // layer's key cache [S][kvd]
    const float* vc;
    int kvd, hs, G, g;
    int r0, n;        // positions [r0, r0 + n)
    int fresh;        // the position written in this launch (device-scope loads), or -1
    int Gt;           // query heads per token (= G for a single token)
    int qstride;      // floats between consecutive tokens' query rows
    int last0;        // last position the first token may see (causal limit)
};

// K rows, then V rows, of positions [t0, t0 + n) (n <= sc). Rows written in
// an earlier launch take plain loads; the fresh row a device-scope load.
template <int NT>
__device__ __forceinline__ void load_k(KBuf& b, const AttnRange& r, const AttnShape& a, int t0, int n)
{
    const int tid = threadIdx.x;
    const int tl = tid / a.lpk, sub = tid % a.lpk;
    const bool ok = tl < n;
    const int t = t0 + (ok ? tl : 0);
    const float* row = r.kc + (size_t)t * r.kvd + (size_t)r.g * r.hs;
#pragma unroll
    for (int k = 0; k < kMaxKPT; k++) {
        const bool use = ok && k < a.kpt;
        const float* pk = row + 4 * (sub + a.lpk * k);
        b.k[k] = use ? (t == r.fresh ? ld_dev4(pk) : *(const f32x4*)pk) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

template <int NT>
__device__ __forceinline__ void load_v(VBuf& b, const AttnRange& r, const AttnShape& a, int t0, int n)
{
    const int tid = threadIdx.x;
    const int f = tid % a.F, slot = tid / a.F;
#pragma unroll
    for (int j = 0; j < kMaxVPT; j++) {
        const int tl = slot + a.slots * j;
        const bool ok = slot < a.slots && j < a.vpt && tl < n;
        const int t = t0 + (ok ? tl : 0);
        const float* pv = r.vc + (size_t)t * r.kvd + (size_t)r.g * r.hs + 4 * f;
        b.v[j] = ok ? (t == r.fresh ? ld_dev4(pv) : *(const f32x4*)pv) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// LDS layout of the range computation
template <int NT>
struct AttnLds {
    float* qs;
    double* sc;
    double* m_run;
    double* l_run;
    double* alpha;
    double* red;
    __device__ __forceinline__ AttnLds(unsigned char* smem, int G, int hs, const AttnShape& a)
    {
        qs = (float*)smem;
        sc = (double*)(smem + ((((size_t)G * hs * 4) + 15) & ~(size_t)15));
        m_run = sc + (size_t)G * attn_super_pos(a);
        l_run = m_run + kMaxG;
        alpha = l_run + kMaxG;
        red = alpha + kMaxG;
    }
};

// Barrier of the NT threads running a range: the whole workgroup by default.
struct BlockSync {
    __device__ __forceinline__ void operator()() const { __syncthreads(); }
};

// The range computation; ends with a barrier (sync) after which red, m_run
// and l_run hold the result. sync synchronises the NT threads that run it
// (the workgroup, or a group of its waves).
template <int KG, int NT, class Sync = BlockSync>
__device__ __forceinline__ void attn_range(const AttnRange& r, unsigned char* smem, Sync sync = Sync())
{
    constexpr int G = KG;
    const int hs = r.hs;
    const AttnShape a = attn_shape<NT>(hs);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = r.n, r0 = r.r0;
    const int nsub = (n + a.sc - 1) / a.sc;
    AttnLds<NT> L(smem, G, hs, a);

    const int P = attn_super_pos(a);       // positions per super-chunk
    const int spc = P / a.sc;               // sub-chunks per super-chunk
    const int nsup = (n + P - 1) / P;
    auto sub_n = [&](int s) { return min(a.sc, n - s * a.sc); };

    // the first two sub-chunks' K loads, then q
    KBuf KA, KB;
    VBuf VA, VB;
    load_k<NT>(KA, r, a, r0, sub_n(0));
    if (nsub > 1) load_k<NT>(KB, r, a, r0 + a.sc, sub_n(1));
    for (int i = tid; i < G * hs; i += NT) {
        const int h = i / hs;
        // q written in this launch (fresh >= 0: the persistent step) needs a
        // device-scope load; one written by an earlier launch does not
        const float* qp = r.q + (size_t)(h / r.Gt) * r.qstride + (size_t)(h % r.Gt) * hs + i % hs;
        L.qs[i] = r.fresh >= 0 ? ld_dev(qp) : *qp;
    }
    if (tid < G) {
        L.m_run[tid] = -INFINITY;
        L.l_run[tid] = 0.0;
    }
    sync();

    const double scale = 1.0 / sqrt((double)hs);
    const int vf = tid % a.F, vslot = tid / a.F;
    double ax[KG], ay[KG], az[KG], aw[KG];
#pragma unroll
    for (int h = 0; h < KG; h++) ax[h] = ay[h] = az[h] = aw[h] = 0.0;

    // scores of sub-chunk s into LDS at its offset in the super-chunk, then
    // the K buffer takes sub-chunk s + 2
    auto scores = [&](KBuf& cur, int s, int off) {
        const int t0 = r0 + s * a.sc;
        const int m = sub_n(s);
        const int tl = tid / a.lpk, sub = tid % a.lpk;
        const f32x4* q4 = (const f32x4*)L.qs;
        double sv[KG];
#pragma unroll
        for (int h = 0; h < KG; h++) {
            double acc = 0.0;
#pragma unroll
            for (int k = 0; k < kMaxKPT; k++) {
                if (k < a.kpt) {
                    const f32x4 qv = q4[(size_t)h * a.F + sub + a.lpk * k];
                    const f32x4 kv = cur.k[k];
                    acc += (double)qv.x * (double)kv.x;
                    acc += (double)qv.y * (double)kv.y;
                    acc += (double)qv.z * (double)kv.z;
                    acc += (double)qv.w * (double)kv.w;
                }
            }
            sv[h] = lanes_sum_f64(acc, a.lpk);
        }
        if (sub == 0 && tl < m)
#pragma unroll
            for (int h = 0; h < KG; h++)
                L.sc[(size_t)h * P + off + tl] = t0 + tl <= r.last0 + h / r.Gt ? sv[h] * scale : -INFINITY;
        if (s + 2 < nsub) load_k<NT>(cur, r, a, t0 + 2 * a.sc, sub_n(s + 2));
    };
    // values of sub-chunk s (weights at its offset in the super-chunk), then
    // the V buffer takes sub-chunk s + 2 if it lies in the same super-chunk
    auto values = [&](VBuf& cur, int s, int off, int s_end) {
        const int t0 = r0 + s * a.sc;
        const int m = sub_n(s);
        if (vslot < a.slots) {
#pragma unroll
            for (int j = 0; j < kMaxVPT; j++) {
                const int tl = vslot + a.slots * j;
                if (j < a.vpt && tl < m) {
                    const f32x4 vv = cur.v[j];
#pragma unroll
                    for (int h = 0; h < KG; h++) {
                        const double e = L.sc[(size_t)h * P + off + tl];
                        ax[h] += e * (double)vv.x;
                        ay[h] += e * (double)vv.y;
                        az[h] += e * (double)vv.z;
                        aw[h] += e * (double)vv.w;
                    }
                }
            }
        }
        if (s + 2 < s_end) load_v<NT>(cur, r, a, t0 + 2 * a.sc, sub_n(s + 2));
    };

    for (int c = 0; c < nsup; c++) {
        const int s0 = c * spc, s1 = min(nsub, s0 + spc);
        const int mP = min(P, n - c * P);  // positions of this super-chunk
        // V rows of its first two sub-chunks, in flight during the scores
        load_v<NT>(VA, r, a, r0 + s0 * a.sc, sub_n(s0));
        if (s0 + 1 < s1) load_v<NT>(VB, r, a, r0 + (s0 + 1) * a.sc, sub_n(s0 + 1));
        // scores; K buffer of sub-chunk s is KA for even s, KB for odd
        for (int s = s0; s < s1; s++) {
            if ((s & 1) == 0)
                scores(KA, s, (s - s0) * a.sc);
            else
                scores(KB, s, (s - s0) * a.sc);
        }
        sync();
        // softmax over the super-chunk, one wave per head
        for (int h = wave; h < G; h += NT / kWave) {
            double mx = -INFINITY;
            for (int t = lane; t < mP; t += kWave) mx = fmax(mx, L.sc[(size_t)h * P + t]);
            mx = wave_max(mx);
            const double mo = L.m_run[h];
            const double mn = fmax(mo, mx);
            double l = 0.0;
            for (int t = lane; t < mP; t += kWave) {
                const double e = exp(L.sc[(size_t)h * P + t] - mn);
                L.sc[(size_t)h * P + t] = e;
                l += e;
            }
            l = wave_sum(l);
            if (lane == 0) {
                const double al = exp(mo - mn);  // 0 when mo is -inf
                L.alpha[h] = al;
                L.l_run[h] = L.l_run[h] * al + l;
                L.m_run[h] = mn;
            }
        }
        sync();
        if (vslot < a.slots) {
#pragma unroll
            for (int h = 0; h < KG; h++) {
                const double al = L.alpha[h];
                ax[h] *= al;
                ay[h] *= al;
                az[h] *= al;
                aw[h] *= al;
            }
        }
        // values; V buffer of the super-chunk's i-th sub-chunk is VA for even
        // i, VB for odd
        for (int s = s0; s < s1; s++) {
            if (((s - s0) & 1) == 0)
                values(VA, s, (s - s0) * a.sc, s1);
            else
                values(VB, s, (s - s0) * a.sc, s1);
        }
        sync();  // L.sc is rewritten by the next super-chunk
    }

    // the value accumulators of the position slots, into LDS
    if ((64 % a.F) == 0) {
        // slots within a wave: butterfly over lane bits >= log2(F)
        for (int msk = a.F; msk < kWave; msk <<= 1) {
#pragma unroll
            for (int h = 0; h < KG; h++) {
                ax[h] += __shfl_xor(ax[h], msk, kWave);
                ay[h] += __shfl_xor(ay[h], msk, kWave);
                az[h] += __shfl_xor(az[h], msk, kWave);
                aw[h] += __shfl_xor(aw[h], msk, kWave);
            }
        }
        if (lane < a.F) {
            for (int h = 0; h < G; h++) {
                double* rr = L.red + ((size_t)wave * G + h) * hs + vf * 4;
                rr[0] = ax[h];
                rr[1] = ay[h];
                rr[2] = az[h];
                rr[3] = aw[h];
            }
        }
    } else if (vslot < a.slots) {
        for (int h = 0; h < G; h++) {
            double* rr = L.red + ((size_t)vslot * G + h) * hs + vf * 4;
            rr[0] = ax[h];
            rr[1] = ay[h];
            rr[2] = az[h];
            rr[3] = aw[h];
        }
    }
    sync();
}

// unnormalised value sum of element e (of G*hs) after attn_range, in a fixed order
template <int NT>
__device__ __forceinline__ double attn_value(unsigned char* smem, int G, int hs, int e)
{
    const AttnShape a = attn_shape<NT>(hs);
    AttnLds<NT> L(smem, G, hs, a);
    double acc = 0.0;
    for (int sl = 0; sl < a.nred; sl++) acc += L.red[(size_t)sl * G * hs + e];
    return acc;
}

template <int NT>
__device__ __forceinline__ double attn_m(unsigned char* smem, int G, int hs, int h)
{
    const AttnShape a = attn_shape<NT>(hs);
    return AttnLds<NT>(smem, G, hs, a).m_run[h];
}

template <int NT>
__device__ __forceinline__ double attn_l(unsigned char* smem, int G, int hs, int h)
{
    const AttnShape a = attn_shape<NT>(hs);
    return AttnLds<NT>(smem, G, hs, a).l_run[h];
}

// Positions per split for T = pos + 1 cached positions and NS splits: the
// even share rounded up to a multiple of `round` positions. Returns the
// number of active splits through nact.
__host__ __device__ inline int attn_split(int T, int NS, int round, int* nact)
{
    int per = (T + NS - 1) / NS;
    per = ((per + round - 1) / round) * round;
    *nact = (T + per - 1) / per;
    return per;
}

}  // namespace l2d
