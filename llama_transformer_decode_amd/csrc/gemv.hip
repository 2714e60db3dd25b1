// gemv.hip - the matvec kernels of the kernel-by-kernel decode step (one
// launch per matvec) and their launch shapes; the computation itself is in
// gemv_core.hpp.
#include "gemv_core.hpp"

namespace l2d {

template <int DT, int PRO, int EPI, int RPW, int U, int NC, int NBUF, bool DBG>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p)
{
    gemv_body<DT, PRO, EPI, RPW, U, NC, NBUF, DBG, CH_NONE>(p, (int)blockIdx.x, (int)gridDim.x, ChainArgs{});
}

size_t gemv_lds_bytes(int dt, int64_t K, int gs, int hs)
{
    return gemv_input_bytes(dt, K, gs) + (size_t)hs * 4;
}

template <int DT, int PRO, int EPI, int RPW, int U, int NC, bool DBG>
static hipError_t launch_t(const GemvParams& p, int blocks, hipStream_t s, const LaunchEvents* ev)
{
    constexpr int NBUF = 2;
    const size_t lds = gemv_lds_bytes(DT, p.K, p.gs, EPI == EPI_QKV ? p.hs : 0);
    if (ev)
        hipExtLaunchKernelGGL((gemv_kernel<DT, PRO, EPI, RPW, U, NC, NBUF, DBG>), dim3((unsigned)blocks),
                              dim3(kThreads), (uint32_t)lds, s, ev->start, ev->stop, 0u, p);
    else
        hipLaunchKernelGGL((gemv_kernel<DT, PRO, EPI, RPW, U, NC, NBUF, DBG>), dim3((unsigned)blocks),
                           dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

// NC: the smallest register budget holding this thread's share of the input
// (fp32: float4 chunks; Q8_0: 16-value chunks; 0 = batched late loads)
template <int DT, int PRO, int EPI, int RPW, int U, bool DBG>
static hipError_t launch_nc(const GemvParams& p, int max_blocks, hipStream_t s, const LaunchEvents* ev)
{
    const int64_t tiles = (p.M + RPW - 1) / RPW;
    int64_t blocks = (tiles + kWaves - 1) / kWaves;
    if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) blocks = 1;
    const int64_t per_thread = DT == DT_F32 ? (p.K / 4 + kThreads - 1) / kThreads
                                            : (p.K / 16 + kThreads - 1) / kThreads;
    const int b = (int)blocks;
    if (per_thread <= 1) return launch_t<DT, PRO, EPI, RPW, U, 1, DBG>(p, b, s, ev);
    if (per_thread <= 2) return launch_t<DT, PRO, EPI, RPW, U, 2, DBG>(p, b, s, ev);
    if (per_thread <= 4) return launch_t<DT, PRO, EPI, RPW, U, 4, DBG>(p, b, s, ev);
    if constexpr (DT == DT_F32) {
        if (per_thread <= 16) return launch_t<DT, PRO, EPI, RPW, U, 16, DBG>(p, b, s, ev);
        return hipErrorInvalidValue;
    } else {
        if (PRO != PRO_NORM) return launch_t<DT, PRO, EPI, RPW, U, 0, DBG>(p, b, s, ev);
        return hipErrorInvalidValue;  // RMSNorm inputs longer than 16384
    }
}

// Launch shape: RPW rows per tile and U 16-byte loads per row per chunk
// (fp32), or U = gs/16 loads per group (Q8_0); every wave gets a contiguous
// share of the tiles; the grid is capped at max_blocks workgroups.
// Measured on MI355X (7B shapes, back-to-back launches): two chunks in the
// ring beat three or four (fewer registers, more waves); fp32 and Q8_0 rows are best
// one per tile when the matrix gives a wave fewer than three two-row tiles
// (output projection, w2), two per tile otherwise. Epilogues that combine a
// row pair (RoPE, SwiGLU) get an even number of rows per tile, or one-row
// tiles handed out in pairs (group sizes 128 and 256).
template <int DT, int PRO, int EPI, bool DBG>
static hipError_t launch_shape(const GemvParams& p, int max_blocks, hipStream_t s, const LaunchEvents* ev)
{
    if constexpr (DT == DT_F32) {
        // one-row tiles on the same rule as Q8_0 (7B output projection and
        // w2: 0.2 and 1.1 us faster than two-row tiles; two-row tiles with
        // 2 or 8 loads and four-row tiles were slower on every shape)
        if constexpr (EPI != EPI_QKV && EPI != EPI_SWIGLU) {
            const int64_t waves = (int64_t)(max_blocks > 0 ? max_blocks : 512) * kWaves;
            if (p.M < 6 * waves) return launch_nc<DT, PRO, EPI, 1, 4, DBG>(p, max_blocks, s, ev);
        }
        return launch_nc<DT, PRO, EPI, 2, 4, DBG>(p, max_blocks, s, ev);
    } else if constexpr (DT == DT_Q4) {
        // four rows of one group per lane: the fastest of RPW 1-8 x U 1-4
        // on every 7B matrix shape (MI355X, 512 and 1024 workgroups)
        if (p.gs != 32) return hipErrorInvalidValue;
        return launch_nc<DT, PRO, EPI, 4, 1, DBG>(p, max_blocks, s, ev);
    } else {
        const int64_t waves = (int64_t)(max_blocks > 0 ? max_blocks : 512) * kWaves;
        switch (p.gs) {
        case 16: return launch_nc<DT, PRO, EPI, 8, 1, DBG>(p, max_blocks, s, ev);
        case 32: return launch_nc<DT, PRO, EPI, 4, 2, DBG>(p, max_blocks, s, ev);
        case 64:
            // the q/k/v and w1/w3 epilogues work on row pairs: RPW stays even
            if constexpr (EPI != EPI_QKV && EPI != EPI_SWIGLU)
                if (p.M < 6 * waves) return launch_nc<DT, PRO, EPI, 1, 4, DBG>(p, max_blocks, s, ev);
            return launch_nc<DT, PRO, EPI, 2, 4, DBG>(p, max_blocks, s, ev);
        case 128: return launch_nc<DT, PRO, EPI, 1, 8, DBG>(p, max_blocks, s, ev);
        case 256: return launch_nc<DT, PRO, EPI, 1, 16, DBG>(p, max_blocks, s, ev);
        default: return hipErrorInvalidValue;
        }
    }
}

hipError_t launch_gemv(int dt, int pro, int epi, const GemvParams& p, int max_blocks,
                       hipStream_t s, const LaunchEvents* ev)
{
#define L2D_CASE(D, P, E)                                                  \
    if (dt == D && pro == P && epi == E) {                                 \
        if (D != DT_F32 && p.group_dots != nullptr)                        \
            return launch_shape<D, P, E, true>(p, max_blocks, s, ev);      \
        return launch_shape<D, P, E, false>(p, max_blocks, s, ev);         \
    }
    L2D_CASE(DT_F32, PRO_NORM, EPI_QKV)
    L2D_CASE(DT_F32, PRO_PLAIN, EPI_RESID)
    L2D_CASE(DT_F32, PRO_NORM, EPI_SWIGLU)
    L2D_CASE(DT_F32, PRO_NORM, EPI_LOGITS)
    L2D_CASE(DT_F32, PRO_PLAIN, EPI_STORE)
    L2D_CASE(DT_Q8, PRO_NORM, EPI_QKV)
    L2D_CASE(DT_Q8, PRO_PLAIN, EPI_RESID)
    L2D_CASE(DT_Q8, PRO_CODES, EPI_RESID)
    L2D_CASE(DT_Q8, PRO_NORM, EPI_SWIGLU)
    L2D_CASE(DT_Q8, PRO_NORM, EPI_LOGITS)
    L2D_CASE(DT_Q8, PRO_PLAIN, EPI_STORE)
    L2D_CASE(DT_Q4, PRO_NORM, EPI_QKV)
    L2D_CASE(DT_Q4, PRO_PLAIN, EPI_RESID)
    L2D_CASE(DT_Q4, PRO_CODES, EPI_RESID)
    L2D_CASE(DT_Q4, PRO_NORM, EPI_SWIGLU)
    L2D_CASE(DT_Q4, PRO_NORM, EPI_LOGITS)
    L2D_CASE(DT_Q4, PRO_PLAIN, EPI_STORE)
#undef L2D_CASE
    return hipErrorInvalidValue;
}

}  // namespace l2d

