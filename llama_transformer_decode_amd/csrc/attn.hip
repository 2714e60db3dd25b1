// attn.hip - single-query GQA attention over the KV cache, split by position.
//
// For query head h and its kv head g = h / G (G = n_heads / n_kv_heads query
// heads share a kv head: Q&A page, GQA question), over cached positions
// t = 0..pos (Q&A page, KV-cache question: k, v of position t sit at
// t * kv_dim in the layer's cache):
//     s_t = q_h . k_t / sqrt(hs),  a = softmax(s),  o_h = sum_t a_t v_t.
//
// Grid (n_kv_heads, nsplit): workgroup (g, c) takes positions
// [c*chunk, (c+1)*chunk) of kv head g for all G query heads of g, so each K/V
// row is read from HBM once per step whatever G is. Within a workgroup:
//   1. scores: LPP lanes per position (16-byte loads of a K row, interleaved
//      so LPP lanes read LPP*16 contiguous bytes), G fp64 dots, LPP-lane
//      butterfly; scores kept in LDS as fp64;
//   2. per head: max, exp, sum over the chunk (fp64, one wave per head);
//   3. values: thread = (float4 column f, position slot), G fp64 double4
//      accumulators, slots reduced through LDS in a fixed order;
//   4. one chunk: write o = acc / l. Several: write (m, l, acc) partials; the
//      last workgroup of kv head g to finish (device-scope counter) merges
//      them, o = sum_c e^{m_c - M} acc_c / sum_c e^{m_c - M} l_c, and resets
//      the counter for the next step.
// Workgroups with no positions (c*chunk > pos) exit at once: the grid is
// sized for seq_len once, and pos is read from device memory, so the same
// launch serves every position of a captured graph.
#include "device.hpp"
#include "internal.hpp"

namespace l2d {

constexpr int kAThreads = 256;

static __host__ __device__ inline int attn_lpp(int F)
{
    // lanes per position for the score phase: up to 4, a power of two dividing F
    return (F % 4 == 0) ? 4 : ((F % 2 == 0) ? 2 : 1);
}

static __host__ __device__ inline int attn_slots(int F, int G, int hs)
{
    // position slots of the value phase, bounded so the fp64 reduction
    // buffer (slots * G * hs doubles) stays within 48 KiB
    int s = kAThreads / F;
    const int cap = (48 * 1024) / (G * hs * 8);
    if (s > cap) s = cap;
    return s < 1 ? 1 : s;
}

size_t attention_lds_bytes(int G, int hs, int chunk)
{
    const int F = hs / 4;
    const size_t q = (size_t)G * hs * 4;
    const size_t sc = (size_t)G * chunk * 8;
    const size_t red = (size_t)attn_slots(F, G, hs) * G * hs * 8;
    return q + sc + red + 64;
}

__global__ __launch_bounds__(kAThreads) void attention_kernel(AttnParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int g = blockIdx.x, split = blockIdx.y;
    const int pos = p.step[1];
    const int T = pos + 1;
    const int chunk = p.chunk;
    const int nact = (T + chunk - 1) / chunk;
    if (split >= nact) return;
    const int t0 = split * chunk;
    const int n = min(T - t0, chunk);
    const int G = p.G, hs = p.hs, F = hs / 4, kvd = p.kvd;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    float* qs = (float*)smem;                                   // [G][hs]
    double* sc = (double*)(smem + (((size_t)G * hs * 4 + 7) & ~(size_t)7));  // [G][chunk]
    double* red = sc + (size_t)G * chunk;                       // [slots][G][hs]
    __shared__ int last_flag;

    // q of the G query heads of kv head g (contiguous: heads g*G .. g*G+G-1)
    for (int i = tid; i < G * hs; i += kAThreads) qs[i] = p.q[(size_t)g * G * hs + i];
    __syncthreads();

    // ---- 1. scores
    const double scale = 1.0 / sqrt((double)hs);
    {
        const int lpp = attn_lpp(F);
        const int ppp = kAThreads / lpp;  // positions per pass
        const int sub = tid % lpp;
        const f32x4* q4 = (const f32x4*)qs;
        for (int base = 0; base < n; base += ppp) {
            const int tl = base + tid / lpp;
            const bool ok = tl < n;
            double s[8];
            for (int h0 = 0; h0 < G; h0 += 8) {
                const int hn = min(8, G - h0);
#pragma unroll
                for (int h = 0; h < 8; h++) s[h] = 0.0;
                if (ok) {
                    const f32x4* k4 = (const f32x4*)(p.kc + (size_t)(t0 + tl) * kvd + (size_t)g * hs);
                    for (int f = sub; f < F; f += lpp) {
                        const f32x4 kv = k4[f];
#pragma unroll
                        for (int h = 0; h < 8; h++) {
                            if (h < hn) {
                                const f32x4 qv = q4[(size_t)(h0 + h) * F + f];
                                s[h] += (double)qv.x * (double)kv.x;
                                s[h] += (double)qv.y * (double)kv.y;
                                s[h] += (double)qv.z * (double)kv.z;
                                s[h] += (double)qv.w * (double)kv.w;
                            }
                        }
                    }
                }
#pragma unroll
                for (int h = 0; h < 8; h++) {
                    double v = s[h];
                    for (int m = 1; m < lpp; m <<= 1) v += __shfl_xor(v, m, kWave);
                    if (ok && sub == 0 && h < hn) sc[(size_t)(h0 + h) * chunk + tl] = v * scale;
                }
            }
        }
    }
    __syncthreads();

    // ---- 2. softmax statistics per head (one wave per head)
    __shared__ double mh[64], lh[64];  // G <= 64
    for (int h = wave; h < G; h += kAThreads / kWave) {
        double m = -INFINITY;
        for (int t = lane; t < n; t += kWave) m = fmax(m, sc[(size_t)h * chunk + t]);
        m = wave_max(m);
        double l = 0.0;
        for (int t = lane; t < n; t += kWave) {
            const double e = exp(sc[(size_t)h * chunk + t] - m);
            sc[(size_t)h * chunk + t] = e;
            l += e;
        }
        l = wave_sum(l);
        if (lane == 0) {
            mh[h] = m;
            lh[h] = l;
        }
    }
    __syncthreads();

    // ---- 3. values: acc_h = sum_t e_t v_t
    const int slots = attn_slots(F, G, hs);
    {
        const int f = tid % F, slot = tid / F;
        const bool active = slot < slots;
        for (int h0 = 0; h0 < G; h0 += 8) {
            const int hn = min(8, G - h0);
            double ax[8], ay[8], az[8], aw[8];
#pragma unroll
            for (int h = 0; h < 8; h++) ax[h] = ay[h] = az[h] = aw[h] = 0.0;
            if (active) {
                for (int tl = slot; tl < n; tl += slots) {
                    const f32x4 vv =
                        *((const f32x4*)(p.vc + (size_t)(t0 + tl) * kvd + (size_t)g * hs) + f);
#pragma unroll
                    for (int h = 0; h < 8; h++) {
                        if (h < hn) {
                            const double e = sc[(size_t)(h0 + h) * chunk + tl];
                            ax[h] += e * (double)vv.x;
                            ay[h] += e * (double)vv.y;
                            az[h] += e * (double)vv.z;
                            aw[h] += e * (double)vv.w;
                        }
                    }
                }
                for (int h = 0; h < hn; h++) {
                    double* rr = red + ((size_t)slot * G + h0 + h) * hs + f * 4;
                    rr[0] = ax[h];
                    rr[1] = ay[h];
                    rr[2] = az[h];
                    rr[3] = aw[h];
                }
            }
        }
    }
    __syncthreads();

    // reduce slots in index order; e = h*hs + i
    if (nact == 1) {
        for (int e = tid; e < G * hs; e += kAThreads) {
            double a = 0.0;
            for (int sl = 0; sl < slots; sl++) a += red[(size_t)sl * G * hs + e];
            const int h = e / hs;
            p.o[(size_t)g * G * hs + e] = (float)(a / lh[h]);
        }
        return;
    }
    const size_t pbase = ((size_t)g * p.nsplit + split) * G;
    for (int e = tid; e < G * hs; e += kAThreads) {
        double a = 0.0;
        for (int sl = 0; sl < slots; sl++) a += red[(size_t)sl * G * hs + e];
        p.part_o[pbase * hs + e] = a;
    }
    if (tid < G) {
        p.part_ml[(pbase + tid) * 2 + 0] = mh[tid];
        p.part_ml[(pbase + tid) * 2 + 1] = lh[tid];
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const int prev = atomicAdd(p.counters + g, 1);
        last_flag = (prev == nact - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();

    // ---- 4. merge the nact partials of kv head g
    for (int e = tid; e < G * hs; e += kAThreads) {
        const int h = e / hs;
        double M = -INFINITY;
        for (int c = 0; c < nact; c++) {
            const size_t b = ((size_t)g * p.nsplit + c) * G + h;
            M = fmax(M, __builtin_nontemporal_load(p.part_ml + b * 2));
        }
        double O = 0.0, L = 0.0;
        for (int c = 0; c < nact; c++) {
            const size_t b = ((size_t)g * p.nsplit + c) * G;
            const double w = exp(__builtin_nontemporal_load(p.part_ml + (b + h) * 2) - M);
            L += w * __builtin_nontemporal_load(p.part_ml + (b + h) * 2 + 1);
            O += w * __builtin_nontemporal_load(p.part_o + b * hs + e);
        }
        p.o[(size_t)g * G * hs + e] = (float)(O / L);
    }
    if (tid == 0) p.counters[g] = 0;
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s)
{
    const size_t lds = attention_lds_bytes(p.G, p.hs, p.chunk);
    hipLaunchKernelGGL(attention_kernel, dim3(p.nkv, p.nsplit), dim3(kAThreads), lds, s, p);
    return hipGetLastError();
}

}  // namespace l2d
