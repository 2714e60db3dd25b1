// attn_decode.hpp - the attention of one decode step, one workgroup's part:
// workgroup (vg, c) of the grid (n_kv_heads * gsplit, NS) runs the attention
// of G/gsplit of the query heads of kv head vg / gsplit over a contiguous
// range of about (pos+1)/NS positions (rounded up to whole sub-chunks; see
// attn_core.hpp for the computation). gsplit > 1 (used for 8 query heads per
// kv head) reads the kv head's K/V rows once per workgroup but halves each
// merge. One active range: o is written directly. Several: each range stores
// its (m, l, acc) with device-scope stores, waits for them to complete and
// counts itself done on its kv head's counter; the range that completes the
// count merges all of them, o = sum_c e^{m_c - M} acc_c / sum_c e^{m_c - M} l_c,
// reading them with device-scope loads, and resets the counter. No fence or
// cache write-back is needed, and no second kernel.
// Workgroups beyond the active ranges exit at once: the grid is sized once,
// pos is read from device memory, and the same launch serves every position
// of a captured graph.
#pragma once

#include <hip/hip_ext.h>

#include "attn_core.hpp"
#include "device.hpp"
#include "internal.hpp"

namespace l2d {

constexpr int kAThreads = 256;

// HS > 0: the head size as a compile-time constant (every shape of the range
// computation folds, with no branches on it); HS = 0: read from p.hs
//
// PUB (the first phase of a chained launch with the output projection): o
// is stored at device scope, and once the workgroup that writes kv head
// column vg's o has its stores complete, it sets flag chain.pub[vg] to the
// launch's epoch.
template <int KG, int HS, bool PUB>
__device__ __forceinline__ void attention_body(const AttnParams& p, int vg, int split, const ChainArgs& chain)
{
    extern __shared__ __align__(16) unsigned char smem[];
    // workgroup (vg, c): kv head g = vg / gsplit, its query heads
    // [hsub * KG, (hsub + 1) * KG), positions of range c
    const int g = vg / p.gsplit, hsub = vg % p.gsplit;
    const size_t qoff = ((size_t)g * p.G + (size_t)hsub * KG) * (HS > 0 ? HS : p.hs);
    const int T = p.step[1] + 1;
    const int NS = p.nsplit;
    int nact;
    const int hs = HS > 0 ? HS : p.hs;
    const int per = attn_split(T, NS, attn_shape<kAThreads>(hs).sc, &nact);
    if (split >= nact) return;
    const int r0 = split * per;
    constexpr int G = KG;
    const int tid = threadIdx.x;

    AttnRange r;
    r.q = p.q + qoff;
    r.kc = p.kc;
    r.vc = p.vc;
    r.kvd = p.kvd;
    r.hs = hs;
    r.G = G;
    r.g = g;
    r.r0 = r0;
    r.n = min(T - r0, per);
    r.fresh = -1;  // the kernel boundary orders the cache write before these loads
    r.Gt = G;  // one query token: no causal mask within the range
    r.qstride = 0;
    r.last0 = 0x3fffffff;
    attn_range<KG, kAThreads>(r, smem);

    // column vg's o is complete (PUB): wait for this workgroup's stores,
    // then set the column's flag
    auto publish = [&]() {
        if constexpr (PUB) {
            wait_vm_all();
            __syncthreads();
            if (tid == 0) st_dev(chain.pub + vg, (uint32_t)p.step[kStepSerial] * (uint32_t)chain.nlayers +
                                                     (uint32_t)chain.layer + 1u);
        }
    };
    auto put_o = [&](int64_t i, float v) {
        if constexpr (PUB) st_dev(p.o + i, v);
        else p.o[i] = v;
    };
    if (nact == 1) {
        for (int e = tid; e < G * hs; e += kAThreads)
            put_o(qoff + e, (float)(attn_value<kAThreads>(smem, G, hs, e) / attn_l<kAThreads>(smem, G, hs, e / hs)));
        publish();
        return;
    }
    // Several ranges: store (acc, m, l) at the device coherence point, then
    // count this range done; the last one merges
    const size_t pbase = ((size_t)vg * NS + split) * G;
    for (int e = tid; e < G * hs; e += kAThreads) st_dev(p.part_o + pbase * hs + e, attn_value<kAThreads>(smem, G, hs, e));
    if (tid < G) {
        st_dev(p.part_ml + (pbase + tid) * 2, attn_m<kAThreads>(smem, G, hs, tid));
        st_dev(p.part_ml + (pbase + tid) * 2 + 1, attn_l<kAThreads>(smem, G, hs, tid));
    }
    wait_vm_all();
    __syncthreads();
    __shared__ int last;
    if (tid == 0) {
        uint32_t* ctr = p.ctr + (size_t)vg * 32;
        const uint32_t done = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = done + 1 == (uint32_t)nact;
        if (last) st_dev(ctr, 0u);  // the next use is a later launch
    }
    __syncthreads();
    if (!last) return;
    // Merge of kv head g's ranges, in fp64. First the weight of every (head,
    // range), w_c = e^{m_c - M} with M the head's maximum, and the head's
    // sum_c w_c l_c: one wavefront per head, a lane per range, fixed-order
    // wave reductions. Then each output element: four adjacent lanes take
    // every fourth range (all their loads issued together) and combine by
    // DPP in a fixed order. Every lane of a wave joins the DPP steps.
    __shared__ double wsh[kMaxG][64];
    __shared__ double lsh[kMaxG];
    const size_t base = (size_t)vg * NS;
    const int sub = tid & 3;
    constexpr int KMAX = 16;  // ranges per lane: NS <= 64
    const int kk = (nact + 3) / 4;  // ranges this lane's loads actually need
    // Output passes of 64 elements (4 lanes each). The partial values of PB
    // passes are loaded together; the first batch goes out with the (m, l)
    // loads below, so for G <= 2 (two passes at head size 128) the merge
    // costs one device round trip, and for G = 8 four instead of sixteen.
    constexpr int PB = KG >= 4 ? 4 : 2;
    const int npass = (G * hs + kAThreads / 4 - 1) / (kAThreads / 4);
    double buf[PB][KMAX];
    auto load_pass = [&](double* o, int ps) {
        const int ec = min(ps * (kAThreads / 4) + (tid >> 2), G * hs - 1);
#pragma unroll
        for (int k = 0; k < KMAX; k++)
            o[k] = (k < kk && ps < npass) ? ld_dev(p.part_o + ((base + min(sub + 4 * k, nact - 1)) * G) * hs + ec)
                                          : 0.0;
    };
#pragma unroll
    for (int q = 0; q < PB; q++) load_pass(buf[q], q);
    for (int t = tid; t < G * 64; t += kAThreads) {
        const int h = t / 64, c = t % 64;
        const bool ok = c < nact;
        const double mc = ok ? ld_dev(p.part_ml + ((base + c) * G + h) * 2) : -INFINITY;
        const double lc = ok ? ld_dev(p.part_ml + ((base + c) * G + h) * 2 + 1) : 0.0;
        const double M = wave_max(mc);
        const double w = ok ? exp(mc - M) : 0.0;
        const double Ls = wave_sum(w * lc);
        wsh[h][c] = w;
        if ((t & 63) == 0) lsh[h] = Ls;
    }
    __syncthreads();
    for (int b0 = 0; b0 < npass; b0 += PB) {
        if (b0 > 0) {
#pragma unroll
            for (int q = 0; q < PB; q++) load_pass(buf[q], b0 + q);
        }
#pragma unroll
        for (int q = 0; q < PB; q++) {
            if (b0 + q < npass) {  // uniform
                const int e = (b0 + q) * (kAThreads / 4) + (tid >> 2);
                const int ec = e < G * hs ? e : G * hs - 1;
                const int h = ec / hs;
                double O = 0.0;
#pragma unroll
                for (int k = 0; k < KMAX; k++)
                    if (sub + 4 * k < nact) O += wsh[h][sub + 4 * k] * buf[q][k];
                O += __hiloint2double(dpp_xor1(__double2hiint(O)), dpp_xor1(__double2loint(O)));
                O += __hiloint2double(dpp_xor2(__double2hiint(O)), dpp_xor2(__double2loint(O)));
                if (sub == 0 && e < G * hs) put_o(qoff + e, (float)(O / lsh[h]));
            }
        }
    }
    publish();
}

}  // namespace l2d
