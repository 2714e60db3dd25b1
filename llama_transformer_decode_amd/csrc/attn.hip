// attn.hip - single-query GQA attention over the KV cache, split by position.
//
// For query head h and its kv head g = h / G (G = n_heads / n_kv_heads query
// heads share a kv head: Q&A page, GQA question), over cached positions
// t = 0..pos (Q&A page, KV-cache question: k, v of position t sit at
// t * kv_dim in the layer's cache):
//     s_t = q_h . k_t / sqrt(hs),  a = softmax(s),  o_h = sum_t a_t v_t.
//
// Grid (n_kv_heads, NS): workgroup (g, c) owns a contiguous range of about
// (pos+1)/NS positions (rounded up to whole sub-chunks) of kv head g and serves all G query heads of g, so
// every K/V row is read from HBM once per step whatever G is. The range is
// walked in sub-chunks of SC positions whose K and V rows are loaded two
// sub-chunks ahead (double buffer), so a range of up to 2*SC positions costs
// one HBM round trip. Per sub-chunk:
//   scores  LPK lanes per position (16-byte loads, interleaved so the LPK
//           lanes read LPK*16 contiguous bytes), G fp64 dots, DPP lane sums;
//   softmax per head, online in fp64: running max m and sum l, rescale
//           factor e^{m_old - m_new} for what was accumulated before;
//   values  thread = (float4 column f, position slot), G fp64 double4
//           accumulators.
// The slots are reduced through LDS in a fixed order. One active range: o is
// written directly. Several: each writes (m, l, acc) and a small merge kernel
// launched right after combines them, o = sum_c e^{m_c - M} acc_c /
// sum_c e^{m_c - M} l_c (no atomics or device-scope fences needed).
// Workgroups beyond the active ranges exit at once: the grid is sized once,
// pos is read from device memory, and the same launch serves every position
// of a captured graph.
#include <hip/hip_ext.h>

#include "device.hpp"
#include "internal.hpp"

namespace l2d {

constexpr int kAThreads = 256;
constexpr int kMaxG = 8;    // query heads per kv head held in registers
constexpr int kMaxKPT = 4;  // K float4 per lane per sub-chunk
constexpr int kMaxVPT = 4;  // V float4 per thread per sub-chunk

struct AttnShape {
    int F;      // float4 per head row
    int lpk;    // lanes per position in the score phase
    int sc;     // positions per sub-chunk
    int kpt;    // K float4 per lane
    int slots;  // position slots in the value phase
    int vpt;    // V float4 per thread
};

__host__ __device__ inline AttnShape attn_shape(int hs)
{
    AttnShape a;
    a.F = hs / 4;
    a.lpk = (a.F % 8 == 0) ? 8 : (a.F % 4 == 0) ? 4 : (a.F % 2 == 0) ? 2 : 1;
    a.sc = kAThreads / a.lpk;
    if (a.sc > 128) a.sc = 128;
    a.kpt = a.F / a.lpk;
    a.slots = kAThreads / a.F;
    a.vpt = (a.sc + a.slots - 1) / a.slots;
    return a;
}

int attention_positions_per_subchunk(int hs) { return attn_shape(hs).sc; }

// Positions per split for T = pos + 1 cached positions and NS splits: the
// even share rounded up to whole sub-chunks, so a split is one or more full
// sub-chunks (the last split may be short). Returns the number of active
// splits through nact.
__host__ __device__ inline int attn_split(int T, int NS, int sc, int* nact)
{
    int per = (T + NS - 1) / NS;
    per = ((per + sc - 1) / sc) * sc;
    *nact = (T + per - 1) / per;
    return per;
}

bool attention_supported(int G, int hs)
{
    const AttnShape a = attn_shape(hs);
    return (G == 1 || G == 2 || G == 4 || G == 8) && hs % 4 == 0 && a.F <= 64 && a.kpt <= kMaxKPT &&
           a.vpt <= kMaxVPT && attention_lds_bytes(G, hs, 0) <= 64 * 1024;
}

size_t attention_lds_bytes(int G, int hs, int)
{
    const AttnShape a = attn_shape(hs);
    const size_t q = (((size_t)G * hs * 4) + 15) & ~(size_t)15;
    const size_t sc = (size_t)G * a.sc * 8;
    const size_t stats = (size_t)3 * kMaxG * 8;
    const bool wave_red = (64 % a.F) == 0;
    const size_t red = (size_t)(wave_red ? 4 : a.slots) * G * hs * 8;
    return q + sc + stats + red;
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
    for (int m = 4; m < width; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

struct KVBuf {
    f32x4 k[kMaxKPT];
    f32x4 v[kMaxVPT];
};

__device__ __forceinline__ void load_kv(KVBuf& b, const AttnParams& p, const AttnShape& a, int g,
                                        int t0, int n)
{
    const int tid = threadIdx.x;
    // K: position tid / lpk, float4 columns sub + lpk*k
    {
        const int tl = tid / a.lpk, sub = tid % a.lpk;
        const bool ok = tl < n;
        const f32x4* row = (const f32x4*)(p.kc + (size_t)(t0 + (ok ? tl : 0)) * p.kvd + (size_t)g * p.hs);
#pragma unroll
        for (int k = 0; k < kMaxKPT; k++)
            b.k[k] = (ok && k < a.kpt) ? row[sub + a.lpk * k] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // V: column tid % F, positions slot + slots*j
    {
        const int f = tid % a.F, slot = tid / a.F;
#pragma unroll
        for (int j = 0; j < kMaxVPT; j++) {
            const int tl = slot + a.slots * j;
            const bool ok = slot < a.slots && j < a.vpt && tl < n;
            b.v[j] = ok ? *((const f32x4*)(p.vc + (size_t)(t0 + tl) * p.kvd + (size_t)g * p.hs) + f)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
}

template <int KG>
__global__ __launch_bounds__(kAThreads) void attention_kernel(AttnParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int g = blockIdx.x, split = blockIdx.y;
    const int T = p.step[1] + 1;
    const int NS = p.nsplit;
    int nact;
    const int per = attn_split(T, NS, attn_shape(p.hs).sc, &nact);
    if (split >= nact) return;
    const int r0 = split * per;
    const int n = min(T - r0, per);

    constexpr int G = KG;
    const int hs = p.hs;
    const AttnShape a = attn_shape(hs);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nsub = (n + a.sc - 1) / a.sc;

    float* qs = (float*)smem;
    double* sc = (double*)(smem + ((((size_t)G * hs * 4) + 15) & ~(size_t)15));
    double* m_run = sc + (size_t)G * a.sc;
    double* l_run = m_run + kMaxG;
    double* alpha = l_run + kMaxG;
    double* red = alpha + kMaxG;

    // issue the first two sub-chunks' K/V loads, then q
    KVBuf A, B;
    load_kv(A, p, a, g, r0, min(a.sc, n));
    if (nsub > 1) load_kv(B, p, a, g, r0 + a.sc, min(a.sc, n - a.sc));
    for (int i = tid; i < G * hs; i += kAThreads) qs[i] = p.q[(size_t)g * G * hs + i];
    if (tid < G) {
        m_run[tid] = -INFINITY;
        l_run[tid] = 0.0;
    }
    __syncthreads();

    const double scale = 1.0 / sqrt((double)hs);
    const int vf = tid % a.F, vslot = tid / a.F;
    double ax[KG], ay[KG], az[KG], aw[KG];
#pragma unroll
    for (int h = 0; h < KG; h++) ax[h] = ay[h] = az[h] = aw[h] = 0.0;

    auto step = [&](KVBuf& cur, int s) {
        const int t0 = r0 + s * a.sc;
        const int m = min(a.sc, n - s * a.sc);
        // scores
        {
            const int tl = tid / a.lpk, sub = tid % a.lpk;
            const f32x4* q4 = (const f32x4*)qs;
            double sv[KG];
#pragma unroll
            for (int h = 0; h < KG; h++) {
                double acc = 0.0;
                if (h < G) {
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
                }
                sv[h] = lanes_sum_f64(acc, a.lpk);
            }
            if (sub == 0 && tl < m)
#pragma unroll
                for (int h = 0; h < KG; h++)
                    if (h < G) sc[(size_t)h * a.sc + tl] = sv[h] * scale;
        }
        __syncthreads();
        for (int h = wave; h < G; h += kAThreads / kWave) {
            double mx = -INFINITY;
            for (int t = lane; t < m; t += kWave) mx = fmax(mx, sc[(size_t)h * a.sc + t]);
            mx = wave_max(mx);
            const double mo = m_run[h];
            const double mn = fmax(mo, mx);
            double l = 0.0;
            for (int t = lane; t < m; t += kWave) {
                const double e = exp(sc[(size_t)h * a.sc + t] - mn);
                sc[(size_t)h * a.sc + t] = e;
                l += e;
            }
            l = wave_sum(l);
            if (lane == 0) {
                const double al = exp(mo - mn);  // 0 when mo is -inf
                alpha[h] = al;
                l_run[h] = l_run[h] * al + l;
                m_run[h] = mn;
            }
        }
        __syncthreads();
        // values
        if (vslot < a.slots) {
#pragma unroll
            for (int h = 0; h < KG; h++) {
                if (h < G) {
                    const double al = alpha[h];
                    ax[h] *= al;
                    ay[h] *= al;
                    az[h] *= al;
                    aw[h] *= al;
                }
            }
#pragma unroll
            for (int j = 0; j < kMaxVPT; j++) {
                const int tl = vslot + a.slots * j;
                if (j < a.vpt && tl < m) {
                    const f32x4 vv = cur.v[j];
#pragma unroll
                    for (int h = 0; h < KG; h++) {
                        if (h < G) {
                            const double e = sc[(size_t)h * a.sc + tl];
                            ax[h] += e * (double)vv.x;
                            ay[h] += e * (double)vv.y;
                            az[h] += e * (double)vv.z;
                            aw[h] += e * (double)vv.w;
                        }
                    }
                }
            }
        }
        __syncthreads();
        // refill the buffer just consumed with the sub-chunk after next
        if (s + 2 < nsub) load_kv(cur, p, a, g, t0 + 2 * a.sc, min(a.sc, n - (s + 2) * a.sc));
    };
    for (int s = 0; s < nsub; s += 2) {
        step(A, s);
        if (s + 1 < nsub) step(B, s + 1);
    }

    // reduce the value accumulators over position slots, in a fixed order
    const bool wave_red = (64 % a.F) == 0;
    if (wave_red) {
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
                double* rr = red + ((size_t)wave * G + h) * hs + vf * 4;
                rr[0] = ax[h];
                rr[1] = ay[h];
                rr[2] = az[h];
                rr[3] = aw[h];
            }
        }
    } else if (vslot < a.slots) {
        for (int h = 0; h < G; h++) {
            double* rr = red + ((size_t)vslot * G + h) * hs + vf * 4;
            rr[0] = ax[h];
            rr[1] = ay[h];
            rr[2] = az[h];
            rr[3] = aw[h];
        }
    }
    __syncthreads();
    const int nred = wave_red ? 4 : a.slots;

    if (nact == 1) {
        for (int e = tid; e < G * hs; e += kAThreads) {
            double acc = 0.0;
            for (int sl = 0; sl < nred; sl++) acc += red[(size_t)sl * G * hs + e];
            p.o[(size_t)g * G * hs + e] = (float)(acc / l_run[e / hs]);
        }
        return;
    }
    // Several ranges: write (acc, m, l); the merge kernel that follows in
    // the stream combines them (the kernel boundary orders the stores)
    const size_t pbase = ((size_t)g * NS + split) * G;
    for (int e = tid; e < G * hs; e += kAThreads) {
        double acc = 0.0;
        for (int sl = 0; sl < nred; sl++) acc += red[(size_t)sl * G * hs + e];
        p.part_o[pbase * hs + e] = acc;
    }
    if (tid < G) {
        p.part_ml[(pbase + tid) * 2 + 0] = m_run[tid];
        p.part_ml[(pbase + tid) * 2 + 1] = l_run[tid];
    }
}

// Merge of the split results, o = sum_c e^{m_c - M} acc_c / sum_c e^{m_c - M} l_c
// with M = max_c m_c, in fp64. Four adjacent lanes share an output element
// and take every fourth split; their partial maxima and sums combine by DPP
// in a fixed order. Does nothing when one split covered all positions (the
// attention kernel then wrote o itself).
__global__ __launch_bounds__(256) void attention_merge_kernel(AttnParams p)
{
    const int T = p.step[1] + 1;
    int nact;
    attn_split(T, p.nsplit, attn_shape(p.hs).sc, &nact);
    if (nact == 1) return;
    const int G = p.G, hs = p.hs;
    const int64_t n_out = (int64_t)p.nkv * G * hs;
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 2;
    const int sub = threadIdx.x & 3;
    const int64_t ec = e < n_out ? e : n_out - 1;  // clamped: all lanes join the DPP sums
    const int64_t g = ec / (G * hs);
    const int64_t within = ec % (G * hs);
    const int64_t h = within / hs;
    const size_t base = (size_t)g * p.nsplit;
    // this lane's splits c = sub + 4k (k < 16, NS <= 64), loads issued together
    constexpr int KMAX = 16;
    double m[KMAX], l[KMAX], o[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; k++) {
        const int c = min(sub + 4 * k, nact - 1);
        m[k] = p.part_ml[((base + c) * G + h) * 2];
        l[k] = p.part_ml[((base + c) * G + h) * 2 + 1];
        o[k] = p.part_o[((base + c) * G) * hs + within];
    }
    double M = -INFINITY;
#pragma unroll
    for (int k = 0; k < KMAX; k++)
        if (sub + 4 * k < nact) M = fmax(M, m[k]);
    M = fmax(M, __hiloint2double(dpp_xor1(__double2hiint(M)), dpp_xor1(__double2loint(M))));
    M = fmax(M, __hiloint2double(dpp_xor2(__double2hiint(M)), dpp_xor2(__double2loint(M))));
    double O = 0.0, L = 0.0;
#pragma unroll
    for (int k = 0; k < KMAX; k++) {
        if (sub + 4 * k < nact) {
            const double w = exp(m[k] - M);
            L += w * l[k];
            O += w * o[k];
        }
    }
    O += __hiloint2double(dpp_xor1(__double2hiint(O)), dpp_xor1(__double2loint(O)));
    O += __hiloint2double(dpp_xor2(__double2hiint(O)), dpp_xor2(__double2loint(O)));
    L += __hiloint2double(dpp_xor1(__double2hiint(L)), dpp_xor1(__double2loint(L)));
    L += __hiloint2double(dpp_xor2(__double2hiint(L)), dpp_xor2(__double2loint(L)));
    if (sub == 0 && e < n_out) p.o[e] = (float)(O / L);
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s, const LaunchEvents* ev)
{
    const size_t lds = attention_lds_bytes(p.G, p.hs, 0);
    const dim3 grid(p.nkv, p.nsplit);
    hipEvent_t e0 = ev ? ev->start : nullptr;
#define L2D_ATT(GG)                                                                                \
    if (ev)                                                                                        \
        hipExtLaunchKernelGGL(attention_kernel<GG>, grid, dim3(kAThreads), (uint32_t)lds, s, e0,   \
                              nullptr, 0u, p);                                                     \
    else                                                                                           \
        hipLaunchKernelGGL(attention_kernel<GG>, grid, dim3(kAThreads), lds, s, p);
    switch (p.G) {
    case 1: L2D_ATT(1) break;
    case 2: L2D_ATT(2) break;
    case 4: L2D_ATT(4) break;
    case 8: L2D_ATT(8) break;
    default: return hipErrorInvalidValue;
    }
#undef L2D_ATT
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)p.nkv * p.G * p.hs * 4;
    const dim3 mgrid((unsigned)((threads + 255) / 256));
    if (ev)
        hipExtLaunchKernelGGL(attention_merge_kernel, mgrid, dim3(256), 0u, s, nullptr, ev->stop, 0u, p);
    else
        hipLaunchKernelGGL(attention_merge_kernel, mgrid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace l2d
