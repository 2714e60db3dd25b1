// attn.hip - the standalone attention kernels of the kernel-by-kernel step:
// grid (n_kv_heads, NS), workgroup (g, c) runs the attention of kv head g
// over a contiguous range of about (pos+1)/NS positions (rounded up to whole
// sub-chunks; see attn_core.hpp for the computation). One active range: o is
// written directly. Several: each writes (m, l, acc) and a small merge kernel
// launched right after combines them, o = sum_c e^{m_c - M} acc_c /
// sum_c e^{m_c - M} l_c (no atomics or device-scope fences needed).
// Workgroups beyond the active ranges exit at once: the grid is sized once,
// pos is read from device memory, and the same launch serves every position
// of a captured graph.
#include <hip/hip_ext.h>

#include "attn_core.hpp"
#include "device.hpp"
#include "internal.hpp"

namespace l2d {

constexpr int kAThreads = 256;

int attention_positions_per_subchunk(int hs) { return attn_shape<kAThreads>(hs).sc; }

bool attention_supported(int G, int hs)
{
    return attn_core_supported<kAThreads>(G, hs) && attention_lds_bytes(G, hs, 0) <= 64 * 1024;
}

size_t attention_lds_bytes(int G, int hs, int) { return attn_core_lds_bytes<kAThreads>(G, hs); }

template <int KG>
__global__ __launch_bounds__(kAThreads) void attention_kernel(AttnParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int g = blockIdx.x, split = blockIdx.y;
    const int T = p.step[1] + 1;
    const int NS = p.nsplit;
    int nact;
    const int per = attn_split(T, NS, attn_shape<kAThreads>(p.hs).sc, &nact);
    if (split >= nact) return;
    const int r0 = split * per;
    constexpr int G = KG;
    const int hs = p.hs;
    const int tid = threadIdx.x;

    AttnRange r;
    r.q = p.q + (size_t)g * G * hs;
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

    if (nact == 1) {
        for (int e = tid; e < G * hs; e += kAThreads)
            p.o[(size_t)g * G * hs + e] =
                (float)(attn_value<kAThreads>(smem, G, hs, e) / attn_l<kAThreads>(smem, G, hs, e / hs));
        return;
    }
    // Several ranges: write (acc, m, l); the merge kernel that follows in
    // the stream combines them (the kernel boundary orders the stores)
    const size_t pbase = ((size_t)g * NS + split) * G;
    for (int e = tid; e < G * hs; e += kAThreads) p.part_o[pbase * hs + e] = attn_value<kAThreads>(smem, G, hs, e);
    if (tid < G) {
        p.part_ml[(pbase + tid) * 2 + 0] = attn_m<kAThreads>(smem, G, hs, tid);
        p.part_ml[(pbase + tid) * 2 + 1] = attn_l<kAThreads>(smem, G, hs, tid);
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
    attn_split(T, p.nsplit, attn_shape<kAThreads>(p.hs).sc, &nact);
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
