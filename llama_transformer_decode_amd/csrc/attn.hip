// attn.hip - the attention kernel of the kernel-by-kernel step (the
// computation is attention_body in attn_decode.hpp), its launch and its
// occupancy query.
#include "attn_decode.hpp"

namespace l2d {

int attention_positions_per_subchunk(int hs) { return attn_shape<kAThreads>(hs).sc; }

bool attention_supported(int G, int hs)
{
    return attn_core_supported<kAThreads>(G, hs) && attention_lds_bytes(G, hs, 0) <= 64 * 1024;
}

size_t attention_lds_bytes(int G, int hs, int) { return attn_core_lds_bytes<kAThreads>(G, hs); }

template <int KG, int HS>
__global__ __launch_bounds__(kAThreads) void attention_kernel(AttnParams p)
{
    attention_body<KG, HS, false>(p, (int)blockIdx.x, (int)blockIdx.y, ChainArgs{});
}

template <int KG, int HS>
static int blocks_per_cu(size_t lds)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attention_kernel<KG, HS>, kAThreads, lds) != hipSuccess)
        return 0;
    return n;
}

template <int KG>
static int blocks_per_cu_hs(int hs, size_t lds)
{
    return hs == 128 ? blocks_per_cu<KG, 128>(lds) : hs == 64 ? blocks_per_cu<KG, 64>(lds) : blocks_per_cu<KG, 0>(lds);
}

int attention_blocks_per_cu(int G, int gsplit, int hs)
{
    if (gsplit < 1 || G % gsplit) return 0;
    const size_t lds = attention_lds_bytes(G, hs, 0);
    switch (G / gsplit) {
    case 1: return blocks_per_cu_hs<1>(hs, lds);
    case 2: return blocks_per_cu_hs<2>(hs, lds);
    case 4: return blocks_per_cu_hs<4>(hs, lds);
    case 8: return blocks_per_cu_hs<8>(hs, lds);
    default: return 0;
    }
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s, const LaunchEvents* ev)
{
    if (p.nsplit > 64) return hipErrorInvalidValue;  // the merge takes at most 64 ranges
    const size_t lds = attention_lds_bytes(p.G, p.hs, 0);
    if (p.gsplit < 1 || p.G % p.gsplit) return hipErrorInvalidValue;
    const dim3 grid(p.nkv * p.gsplit, p.nsplit);
#define L2D_ATT2(GG, HH)                                                                           \
    if (ev)                                                                                        \
        hipExtLaunchKernelGGL((attention_kernel<GG, HH>), grid, dim3(kAThreads), (uint32_t)lds, s, \
                              ev->start, ev->stop, 0u, p);                                         \
    else                                                                                           \
        hipLaunchKernelGGL((attention_kernel<GG, HH>), grid, dim3(kAThreads), lds, s, p);
#define L2D_ATT(GG)                                                                                \
    if (p.hs == 128) {                                                                             \
        L2D_ATT2(GG, 128)                                                                          \
    } else if (p.hs == 64) {                                                                       \
        L2D_ATT2(GG, 64)                                                                           \
    } else {                                                                                       \
        L2D_ATT2(GG, 0)                                                                            \
    }
    switch (p.G / p.gsplit) {
    case 1: L2D_ATT(1) break;
    case 2: L2D_ATT(2) break;
    case 4: L2D_ATT(4) break;
    case 8: L2D_ATT(8) break;
    default: return hipErrorInvalidValue;
    }
#undef L2D_ATT
#undef L2D_ATT2
    return hipGetLastError();
}

}  // namespace l2d

