// chain.hip - chained launches of the decode step: two consecutive phases of
// a layer in one launch, the second phase's workgroups after the first's in
// the grid (gemv_core.hpp, "chaining"):
//   attention, then the output projection + residual (the projection's
//   workgroups wait for every kv head column's o);
//   w1/w3 + SwiGLU, then w2 + residual (w2's workgroups wait for every Q8_0
//   group of the SwiGLU output).
// The second phase's weight loads go out before its wait, while the first
// phase's last workgroups still run, and the launch boundary between the two
// phases is gone. The arithmetic of both phases is that of their own kernels,
// so the results are bit-identical to the kernel-by-kernel step.
// Built for Q8_0 weights with groups of 64 (the quantised decode step).
#include <algorithm>

#include "attn_decode.hpp"
#include "gemv_core.hpp"

namespace l2d {

static_assert(kAThreads == kThreads, "chained phases share one workgroup size");

// Blocks [0, nattn): attention workgroup (column b % ncol, range b / ncol),
// the order in which the attention kernel's 2-D grid is dispatched; the
// rest: the output projection (one-row tiles, four 16-byte loads per lane).
template <int KG, int HS, int NC>
__global__ __launch_bounds__(kThreads) void attn_wo_kernel(AttnParams a, GemvParams g, ChainArgs c, int nattn)
{
    const int b = (int)blockIdx.x;
    const int ncol = a.nkv * a.gsplit;
    if (b < nattn)
        attention_body<KG, HS, true>(a, b % ncol, b / ncol, c);
    else
        gemv_body<DT_Q8, PRO_PLAIN, EPI_RESID, 1, 4, NC, 2, false, CH_WAIT>(g, b - nattn, (int)gridDim.x - nattn, c);
}

// Blocks [0, n13): w1/w3 (two-row tiles); the rest: w2 (one-row tiles) on
// the codes the w1/w3 phase published.
template <int NC13, int NC2>
__global__ __launch_bounds__(kThreads) void ffn_kernel(GemvParams g13, GemvParams g2, ChainArgs c, int n13)
{
    const int b = (int)blockIdx.x;
    if (b < n13)
        gemv_body<DT_Q8, PRO_NORM, EPI_SWIGLU, 2, 4, NC13, 2, false, CH_PUB>(g13, b, n13, c);
    else
        gemv_body<DT_Q8, PRO_CODES, EPI_RESID, 1, 4, NC2, 2, false, CH_WAIT>(g2, b - n13, (int)gridDim.x - n13, c);
}

namespace {

// the input registers of a matvec over K values: 16-value chunks per thread
// (1, 2, 4; 0 = loaded in batches, plain and code inputs only)
int chunks_per_thread(int64_t K)
{
    const int64_t n = (K / 16 + kThreads - 1) / kThreads;
    return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 0;
}

// workgroups of a matvec with this many tiles (the per-phase kernel's rule)
int gemv_blocks(int64_t tiles, int max_blocks)
{
    int64_t b = (tiles + kWaves - 1) / kWaves;
    if (max_blocks > 0 && b > max_blocks) b = max_blocks;
    return (int)(b < 1 ? 1 : b);
}

int attn_kg(const AttnParams& a) { return a.gsplit >= 1 && a.G % a.gsplit == 0 ? a.G / a.gsplit : 0; }

}  // namespace

bool chain_supported(int dt, int gs, int64_t d, int64_t h, int G, int gsplit, int hs, int max_blocks)
{
    if (dt != DT_Q8 || gs != 64 || d % 64 != 0 || h % 64 != 0) return false;
    if (gsplit < 1 || G % gsplit != 0) return false;
    const int kg = G / gsplit;
    if (kg != 1 && kg != 2 && kg != 4) return false;
    // every 128-byte line of o has one writer (the workgroup of its kv head
    // column), so the output projection can read o with plain loads
    if ((int64_t)kg * hs % 32 != 0) return false;
    // the output projection and w2 take one-row tiles only while every wave
    // gets fewer than six rows (the per-phase kernel's shape rule)
    const int64_t waves = (int64_t)(max_blocks > 0 ? max_blocks : 512) * kWaves;
    if (d >= 6 * waves) return false;
    const int nd = chunks_per_thread(d);
    if (nd != 1 && nd != 2) return false;
    // every w1/w3 workgroup owns rows (so each has read x before w2 writes it)
    if (gemv_blocks(h, max_blocks) * kWaves > h) return false;
    return attention_supported(G, hs);
}

hipError_t launch_attn_wo(const AttnParams& a, const GemvParams& g, const ChainArgs& c, int max_blocks,
                          hipStream_t s, const LaunchEvents* ev)
{
    if (a.nsplit > 64) return hipErrorInvalidValue;
    const int ncol = a.nkv * a.gsplit;
    const int nattn = ncol * a.nsplit;
    const int nwo = gemv_blocks(g.M, max_blocks);
    const size_t lds = std::max(attention_lds_bytes(a.G, a.hs, 0), gemv_lds_bytes(DT_Q8, g.K, g.gs, 0));
    const int nc = chunks_per_thread(g.K);
    const int kg = attn_kg(a);
    const dim3 grid((unsigned)(nattn + nwo));
#define L2D_AW(KG, HS, NC)                                                                                 \
    {                                                                                                      \
        if (ev)                                                                                            \
            hipExtLaunchKernelGGL((attn_wo_kernel<KG, HS, NC>), grid, dim3(kThreads), (uint32_t)lds, s,    \
                                  ev->start, ev->stop, 0u, a, g, c, nattn);                                \
        else                                                                                               \
            hipLaunchKernelGGL((attn_wo_kernel<KG, HS, NC>), grid, dim3(kThreads), lds, s, a, g, c, nattn); \
        return hipGetLastError();                                                                          \
    }
#define L2D_AW_HS(KG, NC)                   \
    {                                       \
        if (a.hs == 128) L2D_AW(KG, 128, NC) \
        if (a.hs == 64) L2D_AW(KG, 64, NC)   \
        L2D_AW(KG, 0, NC)                    \
    }
#define L2D_AW_NC(KG)                   \
    {                                   \
        if (nc == 1) L2D_AW_HS(KG, 1)   \
        if (nc == 2) L2D_AW_HS(KG, 2)   \
    }
    if (kg == 1) L2D_AW_NC(1)
    if (kg == 2) L2D_AW_NC(2)
    if (kg == 4) L2D_AW_NC(4)
#undef L2D_AW_NC
#undef L2D_AW_HS
#undef L2D_AW
    return hipErrorInvalidValue;
}

hipError_t launch_ffn_chain(const GemvParams& g13, const GemvParams& g2, const ChainArgs& c, int max_blocks,
                            hipStream_t s, const LaunchEvents* ev)
{
    const int n13 = gemv_blocks(g13.M / 2, max_blocks);
    const int n2 = gemv_blocks(g2.M, max_blocks);
    const size_t lds = std::max(gemv_lds_bytes(DT_Q8, g13.K, g13.gs, 0), gemv_lds_bytes(DT_Q8, g2.K, g2.gs, 0));
    const int nc13 = chunks_per_thread(g13.K), nc2 = chunks_per_thread(g2.K);
    const dim3 grid((unsigned)(n13 + n2));
#define L2D_FF(A, B)                                                                                       \
    {                                                                                                      \
        if (ev)                                                                                            \
            hipExtLaunchKernelGGL((ffn_kernel<A, B>), grid, dim3(kThreads), (uint32_t)lds, s, ev->start,   \
                                  ev->stop, 0u, g13, g2, c, n13);                                          \
        else                                                                                               \
            hipLaunchKernelGGL((ffn_kernel<A, B>), grid, dim3(kThreads), lds, s, g13, g2, c, n13);         \
        return hipGetLastError();                                                                          \
    }
#define L2D_FF2(A)                  \
    {                               \
        if (nc2 == 1) L2D_FF(A, 1)  \
        if (nc2 == 2) L2D_FF(A, 2)  \
        if (nc2 == 4) L2D_FF(A, 4)  \
        L2D_FF(A, 0)                \
    }
    if (nc13 == 1) L2D_FF2(1)
    if (nc13 == 2) L2D_FF2(2)
#undef L2D_FF2
#undef L2D_FF
    return hipErrorInvalidValue;
}

// attention workgroups of a chained attention + output projection launch
// that can be resident on one CU (the instance the launch would pick)
int attn_wo_blocks_per_cu(int G, int gsplit, int hs, int64_t d, int gs)
{
    if (gsplit < 1 || G % gsplit) return 0;
    const size_t lds = std::max(attention_lds_bytes(G, hs, 0), gemv_lds_bytes(DT_Q8, d, gs, 0));
    const int nc = chunks_per_thread(d);
    int n = 0;
    hipError_t e = hipErrorInvalidValue;
#define L2D_OCC(KG, HS, NC) \
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_wo_kernel<KG, HS, NC>, kThreads, lds)
#define L2D_OCC_HS(KG, NC)                  \
    if (hs == 128) L2D_OCC(KG, 128, NC);    \
    else if (hs == 64) L2D_OCC(KG, 64, NC); \
    else L2D_OCC(KG, 0, NC);
#define L2D_OCC_NC(KG)                 \
    if (nc == 1) { L2D_OCC_HS(KG, 1) } \
    else if (nc == 2) { L2D_OCC_HS(KG, 2) }
    const int kg = G / gsplit;
    if (kg == 1) { L2D_OCC_NC(1) }
    else if (kg == 2) { L2D_OCC_NC(2) }
    else if (kg == 4) { L2D_OCC_NC(4) }
#undef L2D_OCC_NC
#undef L2D_OCC_HS
#undef L2D_OCC
    return e == hipSuccess ? n : 0;
}

}  // namespace l2d
