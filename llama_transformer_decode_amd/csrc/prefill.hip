// prefill.hip - batched prompt prefill on gfx950: the decode step applied to
// m prompt tokens at once (prompt tokens are fed through the same forward
// pass one position after another: gitcode guide, main loop; mht18 essay,
// section 2.3, the toy forward pass over a sequence). Results equal m
// single-token steps: every token's matvec inputs are quantised on their own
// (Q8_0 per token and group), each row of every matmul is the same fp64 sum
// of exact int32 group dots, in the same group order, and attention of token
// t covers cached positions 0..pos0+t.
//
// What changes is the shape of the work: with m tokens the matvecs become one
// int8 matrix product per weight matrix, C[row][t] = sum_g dot(W_row,g,
// x_t,g) * sw[row][g] * sx[t][g], computed with v_mfma_i32_16x16x64_i8 (one
// 64-value group per instruction, exact int32 result) and combined in fp64
// per group. The weights stream from HBM once per chunk of tokens instead of
// once per token.
//
// Kernels, in the order of a layer:
//   prefill_embed_kernel   x_t = embedding row of token t
//   prefill_prep_kernel    RMSNorm (optional) + Q8_0 quantisation per token row
//   prefill_gemm_kernel    int8 MFMA product + epilogue (q/k/v with RoPE and the
//                          cache write, residual add, SwiGLU)
//   prefill_attn_kernel    causal GQA attention of a block of tokens per kv head
#include <hip/hip_ext.h>

#include "attn_core.hpp"
#include "device.hpp"
#include "internal.hpp"

namespace l2d {

typedef int v4i __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ embedding rows

__global__ __launch_bounds__(256) void prefill_embed_kernel(PrefillEmbedParams p)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int t = blockIdx.y;
    if (i >= p.d) return;
    const int64_t token = p.tokens[t];
    const int64_t off = token * p.d + i;
    float v;
    if (p.dtype == DT_F32) {
        v = ((const float*)p.emb)[off];
    } else {
        const int8_t c = ((const int8_t*)p.emb)[token * p.d + q8_perm_offset(i, p.d, p.gs)];
        v = (float)((double)c * (double)p.emb_s[off / p.gs]);
    }
    p.x[(int64_t)t * p.d + i] = v;
}

hipError_t launch_prefill_embed(const PrefillEmbedParams& p, hipStream_t s)
{
    const dim3 grid((unsigned)((p.d + 255) / 256), (unsigned)p.m);
    hipLaunchKernelGGL(prefill_embed_kernel, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

// ------------------------------------------------------------ RoPE table

// cos / sin of the fp32 angle (pos0 + t) * freq_j, each the fp64 value
// rounded once to fp32 (the same values the decode step's q/k/v epilogue uses)
__global__ __launch_bounds__(256) void prefill_rope_kernel(const float* freqs, int half, int pos0, int m,
                                                         float* rcos, float* rsin)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)m * half) return;
    const int t = (int)(i / half), j = (int)(i % half);
    const float ang = (float)(pos0 + t) * freqs[j];
    rcos[i] = (float)cos((double)ang);
    rsin[i] = (float)sin((double)ang);
}

hipError_t launch_prefill_rope(const float* freqs, int hs, int pos0, int m, float* rcos, float* rsin,
                               hipStream_t s)
{
    const int64_t n = (int64_t)m * (hs / 2);
    hipLaunchKernelGGL(prefill_rope_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, freqs,
                       hs / 2, pos0, m, rcos, rsin);
    return hipGetLastError();
}

// ------------------------------------------------------------ norm + quantise

// One workgroup per token row of K values: optional RMSNorm (fp64 sum of
// squares, v = fp32(g * (x * r)) as in the decode prologue), then Q8_0 codes
// (plain order, [m][K]) and scales ([m][K/gs]) with the decode quantiser:
// one wavefront per group of 64 (gs 64) or per 64-value part of a larger
// group, the group maximum over its lanes.
template <bool NORM>
__global__ __launch_bounds__(256) void prefill_prep_kernel(PrefillPrepParams p)
{
    __shared__ double red[4];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* x = p.x + (int64_t)t * p.K;
    double r = 1.0;
    if (NORM) {
        double ss = 0.0;
        for (int64_t i = tid; i < p.K; i += 256) ss += (double)x[i] * (double)x[i];
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        ss = red[0] + red[1] + red[2] + red[3];
        r = 1.0 / sqrt(ss / (double)p.K + p.eps);
    }
    const int gs = p.gs;
    const int lpg = gs / 16;             // lanes per group, 16 values each
    const int gpw = kWave / lpg;         // groups per wavefront pass
    const int64_t ng = p.K / gs;
    int8_t* q = p.q + (int64_t)t * p.K;
    float* sc = p.s + (int64_t)t * ng;
    for (int64_t g0 = (int64_t)wave * gpw; g0 < ng; g0 += 4 * gpw) {
        const int64_t g = g0 + lane / lpg;
        const bool ok = g < ng;
        const int64_t base = (ok ? g : ng - 1) * gs + (lane % lpg) * 16;
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; k++) {
            const float xv = x[base + k];
            v[k] = NORM ? (float)((double)p.gain[base + k] * ((double)xv * r)) : xv;
        }
        float s;
        const i32x4 codes = quant16(v, lpg, &s);
        if (ok) {
            *(i32x4*)(q + base) = codes;
            if (lane % lpg == 0) sc[g] = s;
        }
    }
}

hipError_t launch_prefill_prep(const PrefillPrepParams& p, bool norm, hipStream_t s, const LaunchEvents* ev)
{
    if (p.gs < 16 || p.gs > 1024 || p.K % p.gs) return hipErrorInvalidValue;
    const auto k = norm ? prefill_prep_kernel<true> : prefill_prep_kernel<false>;
    if (ev)
        hipExtLaunchKernelGGL(k, dim3((unsigned)p.m), dim3(256), 0u, s, ev->start, ev->stop, 0u, p);
    else
        hipLaunchKernelGGL(k, dim3((unsigned)p.m), dim3(256), 0, s, p);
    return hipGetLastError();
}

// ------------------------------------------------------------ int8 MFMA GEMM

// Workgroup tile: 64 weight rows x 64 tokens; wavefront (wr, wt) takes rows
// 32*wr.. and tokens 32*wt.., i.e. 2 x 2 tiles of 16 x 16. Per group of
// gs = 64*U values, tile (i, j) gets U v_mfma_i32_16x16x64_i8 into one int32
// accumulator (exact: at most 256 * 127^2 < 2^31) and then, for each of the
// lane's four outputs, acc += (dot * sw) * sx in fp64 (the oracle's order;
// contraction into an fma is switched off). Operand lanes: lane l holds row
// (token) l % 16 and the 16-byte quarter l / 16 of each 64-value part of the
// group; output lane l holds rows 4*(l/16) + r, r < 4, of column l % 16.
//
// Weights are read in the decode step's group-interleaved layout
// (q8_perm_offset): quarter q of group j of a 64-group block sits at
// 16*nb*q + 16*j. Scales of 16 groups of the tile's rows and tokens are
// staged in LDS, double-buffered, loaded one 16-group stage ahead.
constexpr int kGR = 64, kGT = 64, kGStage = 16;

struct GemmTileLds {
    float sw[2][kGStage][kGR];
    float sx[2][kGStage][kGT];
};

template <int EPI, int U>
__global__ __launch_bounds__(256, 2) void prefill_gemm_kernel(PrefillGemmParams p)
{
#pragma clang fp contract(off)
    __shared__ GemmTileLds L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wt = wave >> 1;
    // XCD-aware order: the token blocks of one row block run on one XCD
    // (workgroup id mod 8), back to back, so its weight tile is read from HBM
    // once and then from that XCD's L2
    const int nrb = (int)((p.N + kGR - 1) / kGR), ntb = (p.m + kGT - 1) / kGT;
    const int id = blockIdx.x, xcd = id % 8, slot = id / 8;
    const int rb = xcd + 8 * (slot / ntb), tb = slot % ntb;
    if (rb >= nrb) return;
    const int64_t row0 = (int64_t)rb * kGR, tok0 = (int64_t)tb * kGT;
    const int64_t K = p.K, gs = p.gs, ng = K / gs;

    // operand addresses: lane's row (token) of each tile and its quarter
    const int rl = lane % 16, ql = lane / 16;
    const int8_t* wrow[2];
    const int8_t* xrow[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int64_t row = row0 + 32 * wr + 16 * i + rl;
        wrow[i] = (const int8_t*)p.W + (row < p.N ? row : p.N - 1) * K;
        const int64_t tok = tok0 + 32 * wt + 16 * i + rl;
        xrow[i] = p.aq + (tok < p.m ? tok : p.m - 1) * K;
    }
    auto load_ops = [&](int64_t g, v4i (&a)[2][U], v4i (&b)[2][U]) {
        const int64_t blk = g / 64, j = g % 64;
        const int64_t nb = (ng - blk * 64) < 64 ? (ng - blk * 64) : 64;
        const int64_t wbase = blk * 64 * gs + 16 * j;
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t q = 4 * u + ql;
#pragma unroll
            for (int i = 0; i < 2; i++) {
                a[i][u] = *(const v4i*)(wrow[i] + wbase + 16 * nb * q);
                b[i][u] = *(const v4i*)(xrow[i] + g * gs + 16 * q);
            }
        }
    };
    // scales of stage st (16 groups) into LDS buffer bf: thread -> (row or
    // token, 4 consecutive groups)
    auto stage_load = [&](int64_t st, float (&w4)[4], float (&x4)[4]) {
        const int who = tid / 4, part = tid % 4;  // 64 rows/tokens x 4 parts of 4 groups
        const int64_t g = st * kGStage + part * 4;
        const int64_t row = row0 + who < p.N ? row0 + who : p.N - 1;
        const int64_t tok = tok0 + who < p.m ? tok0 + who : p.m - 1;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int64_t gg = g + k < ng ? g + k : ng - 1;
            w4[k] = p.Ws[row * ng + gg];
            x4[k] = p.as[tok * ng + gg];
        }
    };
    auto stage_store = [&](int bf, const float (&w4)[4], const float (&x4)[4]) {
        const int who = tid / 4, part = tid % 4;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            L.sw[bf][part * 4 + k][who] = w4[k];
            L.sx[bf][part * 4 + k][who] = x4[k];
        }
    };

    double acc[2][2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) acc[i][j][r] = 0.0;

    const int64_t nst = (ng + kGStage - 1) / kGStage;
    float w4[4], x4[4];
    stage_load(0, w4, x4);
    stage_store(0, w4, x4);
    v4i a[2][U], b[2][U], an[2][U], bn[2][U];
    load_ops(0, a, b);
    __syncthreads();
    for (int64_t st = 0; st < nst; st++) {
        const int bf = (int)(st & 1);
        if (st + 1 < nst) stage_load(st + 1, w4, x4);
        const int64_t gend = (st + 1) * kGStage < ng ? (st + 1) * kGStage : ng;
        for (int64_t g = st * kGStage; g < gend; g++) {
            // next group's operands in flight while this one is used
            load_ops(g + 1 < ng ? g + 1 : g, an, bn);
            const int gi = (int)(g - st * kGStage);
            v4i d[2][2];
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    v4i c = {0, 0, 0, 0};
#pragma unroll
                    for (int u = 0; u < U; u++) c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i][u], b[j][u], c, 0, 0, 0);
                    d[i][j] = c;
                }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const double sx = (double)L.sx[bf][gi][32 * wt + 16 * j + rl];
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    const f32x4 sw4 = *(const f32x4*)&L.sw[bf][gi][32 * wr + 16 * i + 4 * ql];
                    const float swv[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const double t = ((double)d[i][j][r] * (double)swv[r]) * sx;
                        acc[i][j][r] = acc[i][j][r] + t;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int u = 0; u < U; u++) {
                    a[i][u] = an[i][u];
                    b[i][u] = bn[i][u];
                }
        }
        if (st + 1 < nst) {
            stage_store(bf ^ 1, w4, x4);
            __syncthreads();
        }
    }

    // epilogue: lane holds rows row0 + 32wr + 16i + 4ql + r of token
    // tok0 + 32wt + 16j + rl
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int64_t t = tok0 + 32 * wt + 16 * j + rl;
        if (t >= p.m) continue;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int64_t rbase = row0 + 32 * wr + 16 * i + 4 * ql;
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; r++) y[r] = (float)acc[i][j][r];
            if (EPI == EPI_STORE) {
                for (int r = 0; r < 4; r++)
                    if (rbase + r < p.N) p.out[t * p.ldo + rbase + r] = y[r];
            } else if (EPI == EPI_RESID) {
                for (int r = 0; r < 4; r++)
                    if (rbase + r < p.N) {
                        float* o = p.out + t * p.ldo + rbase + r;
                        *o = (float)((double)*o + (double)y[r]);
                    }
            } else if (EPI == EPI_SWIGLU) {
                for (int r = 0; r < 4; r += 2)
                    if (rbase + r + 1 < p.N) {
                        const double z = (double)y[r];
                        const double h3 = (double)y[r + 1];
                        const double silu = z / (1.0 + exp(-z));
                        p.out[t * p.ldo + (rbase + r) / 2] = (float)(silu * h3);
                    }
            } else if (EPI == EPI_QKV) {
                const int64_t pos = p.pos0 + t;
                for (int r = 0; r < 4; r += 2) {
                    const int64_t row = rbase + r;
                    if (row + 1 >= p.N) continue;
                    const float av = y[r], bv = y[r + 1];
                    if (row < p.d + p.kvd) {
                        const int64_t within = row < p.d ? row : row - p.d;
                        const int jj = (int)((within % p.hs) / 2);
                        const double c = (double)p.rcos[t * (p.hs / 2) + jj];
                        const double s = (double)p.rsin[t * (p.hs / 2) + jj];
                        const float ra = (float)((double)av * c - (double)bv * s);
                        const float rb2 = (float)((double)av * s + (double)bv * c);
                        if (row < p.d) {
                            p.out[t * p.ldo + row] = ra;
                            p.out[t * p.ldo + row + 1] = rb2;
                        } else {
                            float* ks = p.kcache + pos * p.kvd + within;
                            ks[0] = ra;
                            ks[1] = rb2;
                        }
                    } else {
                        float* vs = p.vcache + pos * p.kvd + (row - p.d - p.kvd);
                        vs[0] = av;
                        vs[1] = bv;
                    }
                }
            }
        }
    }
}

size_t prefill_gemm_grid(int64_t N, int m)
{
    const int64_t nrb = (N + kGR - 1) / kGR, ntb = (m + kGT - 1) / kGT;
    return (size_t)(8 * ((nrb + 7) / 8) * ntb);
}

template <int EPI>
static hipError_t launch_gemm_epi(const PrefillGemmParams& p, hipStream_t s, const LaunchEvents* ev)
{
    const dim3 grid((unsigned)prefill_gemm_grid(p.N, p.m));
#define L2D_PG(UU)                                                                                   \
    if (ev)                                                                                          \
        hipExtLaunchKernelGGL((prefill_gemm_kernel<EPI, UU>), grid, dim3(256), 0u, s, ev->start,     \
                              ev->stop, 0u, p);                                                      \
    else                                                                                             \
        hipLaunchKernelGGL((prefill_gemm_kernel<EPI, UU>), grid, dim3(256), 0, s, p);
    switch (p.gs) {
    case 64: L2D_PG(1) break;
    case 128: L2D_PG(2) break;
    case 256: L2D_PG(4) break;
    default: return hipErrorInvalidValue;
    }
#undef L2D_PG
    return hipGetLastError();
}

hipError_t launch_prefill_gemm(int epi, const PrefillGemmParams& p, hipStream_t s, const LaunchEvents* ev)
{
    if (p.N <= 0 || p.m <= 0 || p.K % p.gs) return hipErrorInvalidValue;
    switch (epi) {
    case EPI_STORE: return launch_gemm_epi<EPI_STORE>(p, s, ev);
    case EPI_RESID: return launch_gemm_epi<EPI_RESID>(p, s, ev);
    case EPI_SWIGLU: return launch_gemm_epi<EPI_SWIGLU>(p, s, ev);
    case EPI_QKV: return launch_gemm_epi<EPI_QKV>(p, s, ev);
    default: return hipErrorInvalidValue;
    }
}

// ------------------------------------------------------------ attention

// Grid (kv head g, block of TB = KG / G consecutive tokens): one range over
// positions 0..pos0 + last token of the block, its KG "heads" being the G
// query heads of each token, each masked to its own causal limit. K and V
// rows are read once per block of tokens.
constexpr int kPAThreads = 256;

template <int KG>
__global__ __launch_bounds__(kPAThreads) void prefill_attn_kernel(PrefillAttnParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int g = blockIdx.x;
    const int TB = KG / p.G;
    const int t0 = blockIdx.y * TB;
    const int tlast = min(t0 + TB, p.m) - 1;
    AttnRange r;
    r.q = p.q + (size_t)t0 * p.d + (size_t)g * p.G * p.hs;
    r.kc = p.kc;
    r.vc = p.vc;
    r.kvd = p.kvd;
    r.hs = p.hs;
    r.G = KG;
    r.g = g;
    r.r0 = 0;
    r.n = p.pos0 + tlast + 1;
    r.fresh = -1;  // the q/k/v kernel wrote the cache rows before this launch
    r.Gt = p.G;
    r.qstride = p.d;
    r.last0 = p.pos0 + t0;
    // In a last, partial block the heads of tokens past the chunk read query
    // rows of the buffer's zeroed spare rows (its capacity is a multiple of
    // TB tokens); heads do not mix, and their outputs are not written.
    attn_range<KG, kPAThreads>(r, smem);
    for (int e = threadIdx.x; e < KG * p.hs; e += kPAThreads) {
        const int h = e / p.hs;
        const int t = t0 + h / p.G;
        if (t > tlast) continue;
        const int hh = h % p.G;
        p.o[(size_t)t * p.d + ((size_t)g * p.G + hh) * p.hs + e % p.hs] =
            (float)(attn_value<kPAThreads>(smem, KG, p.hs, e) / attn_l<kPAThreads>(smem, KG, p.hs, h));
    }
}

int prefill_attn_heads(int G) { return G <= kMaxG ? kMaxG : G; }

bool prefill_attn_supported(int G, int hs)
{
    return G >= 1 && G <= kMaxG && (kMaxG % G) == 0 && attn_core_supported<kPAThreads>(kMaxG, hs) &&
           attn_core_lds_bytes<kPAThreads>(kMaxG, hs) <= 64 * 1024;
}

hipError_t launch_prefill_attn(const PrefillAttnParams& p, hipStream_t s, const LaunchEvents* ev)
{
    if (!prefill_attn_supported(p.G, p.hs)) return hipErrorInvalidValue;
    const int TB = kMaxG / p.G;
    const dim3 grid((unsigned)p.nkv, (unsigned)((p.m + TB - 1) / TB));
    const size_t lds = attn_core_lds_bytes<kPAThreads>(kMaxG, p.hs);
    if (ev)
        hipExtLaunchKernelGGL(prefill_attn_kernel<kMaxG>, grid, dim3(kPAThreads), (uint32_t)lds, s, ev->start,
                              ev->stop, 0u, p);
    else
        hipLaunchKernelGGL(prefill_attn_kernel<kMaxG>, grid, dim3(kPAThreads), lds, s, p);
    return hipGetLastError();
}

}  // namespace l2d
