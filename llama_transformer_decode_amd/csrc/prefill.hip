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
//   prefill_attn_mfma_kernel  causal attention of 16 query rows (token, head)
//                          of one kv head on the fp64 matrix cores (head
//                          sizes that are multiples of 16, up to 128)
//   prefill_attn_kernel    causal GQA attention of a block of tokens per kv head
//                          (the other head sizes)
#include <hip/hip_ext.h>
#include <stdlib.h>

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
// and scales ([m][K/gs]) with the decode quantiser, 16 values per lane, the
// group maximum over the group's lanes. Codes are stored in the operand
// order of the matmul's MFMA: for each tile of 16 tokens, group g and
// 64-value part u of the group, 1 KiB in which lane l = 16*q + (t % 16)
// holds quarter q of token t's part (so one contiguous 1 KiB load feeds one
// instruction).
template <bool NORM, bool Q8>
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
    if (!Q8) {
        // fp32 weights: the normalised row itself feeds the matmul
        float* xo = p.xo + (int64_t)t * p.K;
        for (int64_t i = tid; i < p.K; i += 256)
            xo[i] = NORM ? (float)((double)p.gain[i] * ((double)x[i] * r)) : x[i];
        return;
    }
    const int gs = p.gs;
    const int lpg = gs / 16;             // lanes per group, 16 values each
    const int gpw = kWave / lpg;         // groups per wavefront pass
    const int64_t ng = p.K / gs;
    const int U = gs / 64;               // 64-value parts per group
    int8_t* q = p.q + (int64_t)(t / 16) * ng * gs * 16;
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
            const int cq = lane % lpg, u = cq / 4, qq = cq % 4;
            *(i32x4*)(q + (((int64_t)g * U + u) * 64 + qq * 16 + t % 16) * 16) = codes;
            if (lane % lpg == 0) sc[g] = s;
        }
    }
}

hipError_t launch_prefill_prep(const PrefillPrepParams& p, bool norm, hipStream_t s, const LaunchEvents* ev)
{
    if (p.xo == nullptr && (p.gs < 64 || p.gs > 256 || p.K % p.gs)) return hipErrorInvalidValue;
    const auto k = p.xo != nullptr ? (norm ? prefill_prep_kernel<true, false> : prefill_prep_kernel<false, false>)
                                   : (norm ? prefill_prep_kernel<true, true> : prefill_prep_kernel<false, true>);
    if (ev)
        hipExtLaunchKernelGGL(k, dim3((unsigned)p.m), dim3(256), 0u, s, ev->start, ev->stop, 0u, p);
    else
        hipLaunchKernelGGL(k, dim3((unsigned)p.m), dim3(256), 0, s, p);
    return hipGetLastError();
}

// ------------------------------------------------------------ int8 MFMA GEMM

// Epilogue of four consecutive output rows rbase..rbase+3 (rbase a multiple
// of 4, so row pairs stay whole) of token t: the decode step's epilogue
// arithmetic, on row-major [m][ldo] outputs.
template <int EPI>
__device__ __forceinline__ void prefill_epilogue(const PrefillGemmParams& p, int64_t t, int64_t rbase,
                                                 const float (&y)[4])
{
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

// Workgroup tile: 64 weight rows x 128 tokens; wavefront (wr, wt) takes rows
// 32*wr.. and tokens 64*wt.., i.e. 2 x 4 tiles of 16 x 16. Per group of
// gs = 64*U values, tile (i, j) gets U v_mfma_i32_16x16x64_i8 into one int32
// accumulator (exact: at most 256 * 127^2 < 2^31) and then, for each of the
// lane's four outputs, acc += (dot * sw) * sx in fp64 (the oracle's order;
// contraction into an fma is switched off). Operand lanes: lane l holds row
// (token) l % 16 and the 16-byte quarter l / 16 of a 64-value part of the
// group; output lane l holds rows 4*(l/16) + r, r < 4, of column l % 16.
//
// Weights (the decode step's group-interleaved rows, q8_perm_offset: quarter
// Q of group j of a 64-group block at 16*nb*Q + 16*j) are staged through LDS
// in steps of 8 64-value parts: the workgroup reads, per row and quarter,
// the step's groups as one contiguous run (a 128-byte line for gs 64) and
// writes them in operand order; the next step's loads are in flight while
// the current one is used (double buffer). Inputs are already in operand
// order (prefill_prep_kernel): one contiguous 1 KiB load per tile, issued
// into a ring of groups ahead of their use. Scales of the step's groups for
// the tile's rows and tokens are staged with the weights.
constexpr int kGR = 64, kGT = 128, kGParts = 8;
constexpr int kTR = 2, kTT = 4;  // 16 x 16 tiles per wavefront: rows, tokens

// Staged weight rows are stored at row ^ gemm_swz(part, quarter). The XOR
// stays within an aligned block of 16 rows, so the 16 lanes of one operand
// read still hit 16 distinct 16-byte bank groups, and each 16 lanes of a
// staging write (8 parts times 2 quarters of the same row) hit 16 distinct
// bank groups instead of one. Only for one 64-value part per group: with 2
// or 4 parts the index arithmetic made those instances spill.
template <int U>
__device__ __forceinline__ int gemm_swz(int part, int quarter) { return U == 1 ? ((quarter & 1) << 3) | (part & 7) : 0; }

struct GemmLds {
    v4i w[2][kGParts][4][kGR];    // [buffer][part][quarter][row], 16 bytes each
    // scales [buffer][group of the step][row or token]; rows padded by 8
    // floats so that a staging write (8 groups of 8 rows or tokens) hits 64
    // distinct banks
    float sw[2][kGParts][kGR + 8];
    float sx[2][kGParts][kGT + 8];
};
// two workgroups per CU (launch bounds) must fit the CU's 160 KiB of LDS
static_assert(2 * sizeof(GemmLds) <= 160 * 1024, "GemmLds");

template <int U>
struct GemmOps {
    v4i b[kTT][U];
};

// CMB 0: each output is the fp64 sum over groups of (dot x sw) x sx, the
// oracle's arithmetic and order (bit-identical results). CMB 1: the same sum
// in fp32, acc = fma(float(dot), sw x sx, acc): one conversion, one multiply
// and one fused multiply-add per output and group instead of four fp64
// operations, held to the logits tolerance instead of bit-identity.
template <int EPI, int U, int CMB>
__global__ __launch_bounds__(256, 2) void prefill_gemm_kernel(PrefillGemmParams p)
{
#pragma clang fp contract(off)
    constexpr int GPS = kGParts / U;  // groups per step
    constexpr int kGRing = U == 1 ? 2 : U == 2 ? 2 : 1;
    extern __shared__ __align__(16) unsigned char gsmem[];
    GemmLds& L = *(GemmLds*)gsmem;
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
    // group indices and offsets within one row fit in 32 bits (K <= 65536)
    const int K = (int)p.K, gs = p.gs, ng = K / gs;
    const int nst = (ng + GPS - 1) / GPS;
    const int rl = lane % 16, ql = lane / 16;

    // ---- weight staging: piece k of this thread = (row, quarter Q, group jg)
    // with jg fastest, so 8 (gs 64) adjacent lanes read one 128-byte run
    constexpr int kPieces = kGR * 4 * kGParts / 256;  // 16-byte pieces per thread (8)
    v4i wreg[kPieces];
    float swreg[(kGR * GPS + 255) / 256], sxreg[(kGT * GPS + 255) / 256];
    auto stage_load = [&](int st) {
        const int g0 = st * GPS;
#pragma unroll
        for (int k = 0; k < kPieces; k++) {
            const int id2 = tid + 256 * k;
            const int jg = id2 % GPS, Q = (id2 / GPS) % (4 * U), r = id2 / (GPS * 4 * U);
            int g = g0 + jg;
            g = g < ng ? g : ng - 1;
            const int blk = g / 64, jj = g % 64;
            const int nb = (ng - blk * 64) < 64 ? (ng - blk * 64) : 64;
            const int64_t row = row0 + r < p.N ? row0 + r : p.N - 1;
            wreg[k] = *(const v4i*)((const int8_t*)p.W + row * K + blk * 64 * gs + 16 * nb * Q + 16 * jj);
        }
#pragma unroll
        for (int k = 0; k < (kGR * GPS + 255) / 256; k++) {
            const int id2 = tid + 256 * k;
            if (id2 < kGR * GPS) {
                const int jg = id2 % GPS, r = id2 / GPS;
                const int g = g0 + jg < ng ? g0 + jg : ng - 1;
                const int64_t row = row0 + r < p.N ? row0 + r : p.N - 1;
                swreg[k] = p.Ws[row * ng + g];
            }
        }
#pragma unroll
        for (int k = 0; k < (kGT * GPS + 255) / 256; k++) {
            const int id2 = tid + 256 * k;
            if (id2 < kGT * GPS) {
                const int jg = id2 % GPS, t = id2 / GPS;
                const int g = g0 + jg < ng ? g0 + jg : ng - 1;
                const int64_t tok = tok0 + t < p.m ? tok0 + t : p.m - 1;
                sxreg[k] = p.as[tok * ng + g];
            }
        }
    };
    auto stage_store = [&](int bf) {
#pragma unroll
        for (int k = 0; k < kPieces; k++) {
            const int id2 = tid + 256 * k;
            const int jg = id2 % GPS, Q = (id2 / GPS) % (4 * U), r = id2 / (GPS * 4 * U);
            L.w[bf][jg * U + Q / 4][Q % 4][r ^ gemm_swz<U>(jg * U + Q / 4, Q % 4)] = wreg[k];
        }
#pragma unroll
        for (int k = 0; k < (kGR * GPS + 255) / 256; k++) {
            const int id2 = tid + 256 * k;
            if (id2 < kGR * GPS) L.sw[bf][id2 % GPS][id2 / GPS] = swreg[k];
        }
#pragma unroll
        for (int k = 0; k < (kGT * GPS + 255) / 256; k++) {
            const int id2 = tid + 256 * k;
            if (id2 < kGT * GPS) L.sx[bf][id2 % GPS][id2 / GPS] = sxreg[k];
        }
    };

    // ---- inputs: tile j of this wavefront = token tile (tok0 + 64wt)/16 + j
    const int8_t* xtile[kTT];
#pragma unroll
    for (int j = 0; j < kTT; j++) {
        int64_t tt = (tok0 + 64 * wt) / 16 + j;
        const int64_t last = (p.m - 1) / 16;
        tt = tt < last ? tt : last;
        xtile[j] = p.aq + tt * (int64_t)ng * gs * 16 + lane * 16;
    }
    auto load_ops = [&](int g, GemmOps<U>& o) {
        const int gc = g < ng ? g : ng - 1;
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
            for (int j = 0; j < kTT; j++) o.b[j][u] = *(const v4i*)(xtile[j] + ((int64_t)gc * U + u) * 1024);
    };

    using Acc = typename std::conditional<CMB == 1, float, double>::type;
    Acc acc[kTR][kTT][4];
#pragma unroll
    for (int i = 0; i < kTR; i++)
#pragma unroll
        for (int j = 0; j < kTT; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) acc[i][j][r] = (Acc)0;

    GemmOps<U> ops[kGRing];
#pragma unroll
    for (int k = 0; k < kGRing; k++) load_ops(k, ops[k]);
    stage_load(0);
    stage_store(0);
    if (nst > 1) stage_load(1);
    __syncthreads();

    auto use_group = [&](const GemmOps<U>& o, int g) {
        const int bf = (g / GPS) & 1, gl = g % GPS;
        // with one part per group every LDS read of the group is issued
        // first, so one wait covers them all (with 2 or 4 parts the extra
        // operands would spill: their reads stay per row tile)
        float sxf[kTT];
        f32x4 sw4[kTR];
        v4i av[kTR][U];
        auto read_rows = [&](int i) {
            sw4[i] = *(const f32x4*)&L.sw[bf][gl][32 * wr + 16 * i + 4 * ql];
#pragma unroll
            for (int u = 0; u < U; u++)
                av[i][u] = L.w[bf][gl * U + u][ql][(32 * wr + 16 * i + rl) ^ gemm_swz<U>(gl * U + u, ql)];
        };
#pragma unroll
        for (int j = 0; j < kTT; j++) sxf[j] = L.sx[bf][gl][64 * wt + 16 * j + rl];
        if constexpr (U == 1) {
#pragma unroll
            for (int i = 0; i < kTR; i++) read_rows(i);
        }
        double sx[kTT];
#pragma unroll
        for (int j = 0; j < kTT; j++) sx[j] = (double)sxf[j];
#pragma unroll
        for (int i = 0; i < kTR; i++) {
            if constexpr (U != 1) read_rows(i);
            const double sw[4] = {(double)sw4[i].x, (double)sw4[i].y, (double)sw4[i].z, (double)sw4[i].w};
            const float swf[4] = {sw4[i].x, sw4[i].y, sw4[i].z, sw4[i].w};
            const v4i* a = av[i];
#pragma unroll
            for (int j = 0; j < kTT; j++) {
                v4i c = {0, 0, 0, 0};
#pragma unroll
                for (int u = 0; u < U; u++) c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], o.b[j][u], c, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    if constexpr (CMB == 1) {
                        acc[i][j][r] = __builtin_fmaf((float)c[r], swf[r] * sxf[j], acc[i][j][r]);
                    } else {
                        const double t = ((double)c[r] * sw[r]) * sx[j];
                        acc[i][j][r] = acc[i][j][r] + t;
                    }
                }
            }
        }
    };

    for (int g0 = 0; g0 < ng; g0 += kGRing) {
#pragma unroll
        for (int k = 0; k < kGRing; k++) {
            const int g = g0 + k;
            if (g < ng) {
                if (g > 0 && g % GPS == 0) {
                    // step g / GPS: its weights and scales (loaded a step
                    // ago) into the buffer last read two steps ago
                    const int st = g / GPS;
                    stage_store(st & 1);
                    __syncthreads();
                    if (st + 1 < nst) stage_load(st + 1);
                }
                use_group(ops[k], g);
            }
            load_ops(g + kGRing, ops[k]);
        }
    }

    // epilogue: lane holds rows row0 + 32wr + 16i + 4ql + r of token
    // tok0 + 64wt + 16j + rl
#pragma unroll
    for (int j = 0; j < kTT; j++) {
        const int64_t t = tok0 + 64 * wt + 16 * j + rl;
        if (t >= p.m) continue;
#pragma unroll
        for (int i = 0; i < kTR; i++) {
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; r++) y[r] = (float)acc[i][j][r];
            prefill_epilogue<EPI>(p, t, row0 + 32 * wr + 16 * i + 4 * ql, y);
        }
    }
}

// fp32 weights: the same tiles on v_mfma_f64_16x16x4f64. A product of two
// fp32 values is exact in fp64, so each output is an fp64 sum of the exact
// products w * x (the oracle's fp32 matvec up to summation order, as in the
// decode step's fp32 GEMV). Output lane l, register r of this instruction
// holds row l/16 + 4r of column l % 16 (checked on MI355X with an in-bounds
// probe); feeding operand row i with weight row 4*(i%4) + i/4 leaves each
// lane four consecutive weight rows, as the epilogues need. Weights and
// inputs are staged through LDS in steps of 32 values of K, double-buffered.
constexpr int kFK = 32;  // K values per step

struct GemmF32Lds {
    float w[2][kFK][kGR];  // [buffer][k][row]
    float x[2][kFK][kGT];  // [buffer][k][token]
};

typedef double v4d __attribute__((ext_vector_type(4)));

template <int EPI>
__global__ __launch_bounds__(256, 2) void prefill_gemm_f32_kernel(PrefillGemmParams p)
{
    __shared__ GemmF32Lds L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wt = wave >> 1;
    const int nrb = (int)((p.N + kGR - 1) / kGR), ntb = (p.m + kGT - 1) / kGT;
    const int id = blockIdx.x, xcd = id % 8, slot = id / 8;
    const int rb = xcd + 8 * (slot / ntb), tb = slot % ntb;
    if (rb >= nrb) return;
    const int64_t row0 = (int64_t)rb * kGR, tok0 = (int64_t)tb * kGT;
    const int K = (int)p.K;
    const int nst = (K + kFK - 1) / kFK;
    const int rl = lane % 16, ql = lane / 16;
    const int perm = 4 * (rl % 4) + rl / 4;  // weight row of operand row rl

    // staging: weights 64 rows x 32 values (2 float4 per thread), inputs
    // 128 tokens x 32 values (4 float4 per thread); 8 lanes read one row's
    // 128 contiguous bytes
    f32x4 wreg[2], xreg[4];
    auto stage_load = [&](int st) {
        const int k0 = st * kFK;
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int id2 = tid + 256 * c, r = id2 / 8, kq = id2 % 8;
            const int64_t row = row0 + r < p.N ? row0 + r : p.N - 1;
            int k = k0 + 4 * kq;
            k = k < K ? k : K - 4;
            wreg[c] = *(const f32x4*)((const float*)p.W + row * K + k);
        }
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int id2 = tid + 256 * c, t = id2 / 8, kq = id2 % 8;
            const int64_t tok = tok0 + t < p.m ? tok0 + t : p.m - 1;
            int k = k0 + 4 * kq;
            k = k < K ? k : K - 4;
            xreg[c] = *(const f32x4*)(p.a32 + tok * K + k);
        }
    };
    auto stage_store = [&](int bf, int st) {
        const int k0 = st * kFK;
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int id2 = tid + 256 * c, r = id2 / 8, kq = id2 % 8;
            const bool ok = k0 + 4 * kq < K;  // values past K contribute zero
            L.w[bf][4 * kq + 0][r] = ok ? wreg[c].x : 0.f;
            L.w[bf][4 * kq + 1][r] = ok ? wreg[c].y : 0.f;
            L.w[bf][4 * kq + 2][r] = ok ? wreg[c].z : 0.f;
            L.w[bf][4 * kq + 3][r] = ok ? wreg[c].w : 0.f;
        }
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int id2 = tid + 256 * c, t = id2 / 8, kq = id2 % 8;
            const bool ok = k0 + 4 * kq < K;
            L.x[bf][4 * kq + 0][t] = ok ? xreg[c].x : 0.f;
            L.x[bf][4 * kq + 1][t] = ok ? xreg[c].y : 0.f;
            L.x[bf][4 * kq + 2][t] = ok ? xreg[c].z : 0.f;
            L.x[bf][4 * kq + 3][t] = ok ? xreg[c].w : 0.f;
        }
    };

    v4d acc[kTR][kTT];
#pragma unroll
    for (int i = 0; i < kTR; i++)
#pragma unroll
        for (int j = 0; j < kTT; j++) acc[i][j] = v4d{0.0, 0.0, 0.0, 0.0};

    stage_load(0);
    stage_store(0, 0);
    if (nst > 1) stage_load(1);
    __syncthreads();
    for (int st = 0; st < nst; st++) {
        const int bf = st & 1;
#pragma unroll
        for (int ks = 0; ks < kFK / 4; ks++) {
            const int kk = 4 * ks + ql;
            double a[kTR], b[kTT];
#pragma unroll
            for (int i = 0; i < kTR; i++) a[i] = (double)L.w[bf][kk][32 * wr + 16 * i + perm];
#pragma unroll
            for (int j = 0; j < kTT; j++) b[j] = (double)L.x[bf][kk][64 * wt + 16 * j + rl];
#pragma unroll
            for (int i = 0; i < kTR; i++)
#pragma unroll
                for (int j = 0; j < kTT; j++) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (st + 1 < nst) {
            stage_store(bf ^ 1, st + 1);
            __syncthreads();
            if (st + 2 < nst) stage_load(st + 2);
        }
    }
#pragma unroll
    for (int j = 0; j < kTT; j++) {
        const int64_t t = tok0 + 64 * wt + 16 * j + rl;
        if (t >= p.m) continue;
#pragma unroll
        for (int i = 0; i < kTR; i++) {
            const float y[4] = {(float)acc[i][j][0], (float)acc[i][j][1], (float)acc[i][j][2], (float)acc[i][j][3]};
            prefill_epilogue<EPI>(p, t, row0 + 32 * wr + 16 * i + 4 * ql, y);
        }
    }
}

size_t prefill_gemm_grid(int64_t N, int m)
{
    const int64_t nrb = (N + kGR - 1) / kGR, ntb = (m + kGT - 1) / kGT;
    return (size_t)(8 * ((nrb + 7) / 8) * ntb);
}

// the staging buffers exceed the default 64 KiB of dynamic LDS
template <int EPI, int U, int CMB>
static hipError_t gemm_lds_attr()
{
    static bool done = false;
    if (!done) {
        hipError_t e = hipFuncSetAttribute((const void*)prefill_gemm_kernel<EPI, U, CMB>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(GemmLds));
        if (e != hipSuccess) return e;
        done = true;
    }
    return hipSuccess;
}

template <int EPI>
static hipError_t launch_gemm_epi(const PrefillGemmParams& p, hipStream_t s, const LaunchEvents* ev)
{
    const dim3 grid((unsigned)prefill_gemm_grid(p.N, p.m));
#define L2D_PG(UU, CC)                                                                               \
    if (hipError_t e_ = gemm_lds_attr<EPI, UU, CC>(); e_ != hipSuccess) return e_;                  \
    if (ev)                                                                                          \
        hipExtLaunchKernelGGL((prefill_gemm_kernel<EPI, UU, CC>), grid, dim3(256),                  \
                              (uint32_t)sizeof(GemmLds), s, ev->start, ev->stop, 0u, p);             \
    else                                                                                             \
        hipLaunchKernelGGL((prefill_gemm_kernel<EPI, UU, CC>), grid, dim3(256), sizeof(GemmLds), s, p);
    if (p.combine == 1) {
        switch (p.gs) {
        case 64: L2D_PG(1, 1) break;
        case 128: L2D_PG(2, 1) break;
        case 256: L2D_PG(4, 1) break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (p.gs) {
        case 64: L2D_PG(1, 0) break;
        case 128: L2D_PG(2, 0) break;
        case 256: L2D_PG(4, 0) break;
        default: return hipErrorInvalidValue;
        }
    }
#undef L2D_PG
    return hipGetLastError();
}

template <int EPI>
static hipError_t launch_gemm_f32_epi(const PrefillGemmParams& p, hipStream_t s, const LaunchEvents* ev)
{
    const dim3 grid((unsigned)prefill_gemm_grid(p.N, p.m));
    if (ev)
        hipExtLaunchKernelGGL(prefill_gemm_f32_kernel<EPI>, grid, dim3(256), 0u, s, ev->start, ev->stop, 0u, p);
    else
        hipLaunchKernelGGL(prefill_gemm_f32_kernel<EPI>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_prefill_gemm(int epi, const PrefillGemmParams& p, hipStream_t s, const LaunchEvents* ev)
{
    if (p.N <= 0 || p.m <= 0) return hipErrorInvalidValue;
    if (p.dtype == DT_F32) {
        if (p.K % 4) return hipErrorInvalidValue;
        switch (epi) {
        case EPI_STORE: return launch_gemm_f32_epi<EPI_STORE>(p, s, ev);
        case EPI_RESID: return launch_gemm_f32_epi<EPI_RESID>(p, s, ev);
        case EPI_SWIGLU: return launch_gemm_f32_epi<EPI_SWIGLU>(p, s, ev);
        case EPI_QKV: return launch_gemm_f32_epi<EPI_QKV>(p, s, ev);
        default: return hipErrorInvalidValue;
        }
    }
    if (p.K % p.gs) return hipErrorInvalidValue;
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
    // the longest ranges (last tokens) first, so the grid ends on short ones
    const int t0 = (gridDim.y - 1 - blockIdx.y) * TB;
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

// Query rows per workgroup: 4 (8 when G = 8), or fewer down to G, the
// most that are a multiple of G and whose LDS fits in 64 KiB; 0 if none.
// Eight rows take 254 VGPRs, one wavefront per SIMD: on MI355X the 7B
// prefill attention ran in 461 us per layer with 8 rows, 264 with 4, 388
// with 2 and 433 with 1.
static int prefill_attn_rows(int G, int hs)
{
    for (int kg = G > 4 ? kMaxG : 4; kg >= 1; kg /= 2)
        if (kg >= G && kg % G == 0 && attn_core_supported<kPAThreads>(kg, hs) &&
            attn_core_lds_bytes<kPAThreads>(kg, hs) <= 64 * 1024)
            return kg;
    return 0;
}

bool prefill_attn_supported(int G, int hs) { return G >= 1 && prefill_attn_rows(G, hs) > 0; }

// ---------------------------------------------------------------- attention on fp64 MFMA
// A head size that is a multiple of 16 (up to 128): a workgroup holds 16
// query rows of one kv head, each a (token, query head) pair of the G query
// heads sharing it (16 tokens when G = 1, 2 tokens of all 8 heads when
// G = 8); its four wavefronts
// take every fourth chunk of 16 positions (so the long, late blocks are
// spread over four SIMDs; two workgroups share a CU). Each computes
// S = Q K^T and O += P V on v_mfma_f64_16x16x4f64 with the online softmax of
// the vector path in fp64 (scaled fp64 scores, running maximum, fp64 exp,
// fixed-order row sums). The four partial (m, l, O) are merged at the end in
// a fixed order, as the decode step merges position ranges. q is converted to
// fp64 once per query row; K and V rows are staged through each wavefront's
// own LDS. Operand rows are fed in the order 4*(i%4) + i/4, so register r of
// lane l ends up with query row 4*(l/16) + r (as in the fp64 prefill matmul).
constexpr int kPMT = 16;            // query rows per workgroup
constexpr int kPMC = 16;            // positions per chunk
constexpr int kPMW = 4;             // wavefronts per workgroup (8 measured slower)
constexpr int kPMHs = 128;          // largest head size
constexpr int kPMSK = kPMHs + 4;    // K row stride in LDS: the B-operand reads hit distinct banks
constexpr int kPMSV = kPMHs + 16;   // V row stride
constexpr int kPMSP = kPMC + 1;     // P row stride (doubles)

struct PrefillMfmaWaveLds {
    float k[kPMC][kPMSK];
    float v[kPMC][kPMSV];
    double pt[kPMT][kPMSP];
};
// after the chunk loop the same bytes hold the wavefront's partial result
struct PrefillMfmaMerge {
    // [lane][4 * tile + register]; the row is padded by one double so that
    // the lanes of a wavefront hit distinct banks (unpadded, every lane of a
    // store or load fell on the same bank pair)
    double o[64][kPMHs / 16 * 4 + 1];
    double m[kPMT], l[kPMT];       // per token
};
static_assert(sizeof(PrefillMfmaMerge) <= sizeof(PrefillMfmaWaveLds), "merge area");

static bool prefill_attn_mfma_ok(int G, int hs)
{
    return (G == 1 || G == 2 || G == 4 || G == 8) && hs % 16 == 0 && hs >= 16 && hs <= kPMHs;
}

// maximum / sum over each aligned group of 16 lanes, identical in every lane
// of the group (quad swaps, half-row mirror, row mirror: each step combines
// a pair of lanes symmetrically, so all lanes see the same operations)
__device__ __forceinline__ double row16_max(double v)
{
    v = fmax(v, dpp_f64<0xB1>(v));
    v = fmax(v, dpp_f64<0x4E>(v));
    v = fmax(v, dpp_f64<0x141>(v));
    return fmax(v, dpp_f64<0x140>(v));
}

__device__ __forceinline__ double row16_sum(double v)
{
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    return v + dpp_f64<0x140>(v);
}

// this wavefront's LDS writes complete before its lanes read them (each
// wavefront owns its staging area; the waves run different chunk counts, so
// no workgroup barrier inside the loop)
__device__ __forceinline__ void lds_wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// NT = head size / 16: every loop below has a compile-time trip count. W
// wavefronts per workgroup. A chunk's K/V rows are loaded when it starts:
// two wavefronts per SIMD (at most 256 registers each) cover each other's
// load latency, where holding the next chunk's rows in registers (one
// wavefront per SIMD) measured slower.
template <int NT, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void prefill_attn_mfma_kernel(PrefillAttnParams p)
{
    constexpr int HS = 16 * NT, NKS = HS / 4, F4ROW = HS / 4;
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    PrefillMfmaWaveLds& L = ((PrefillMfmaWaveLds*)smem)[w];
    const int rl = lane % 16, ql = lane / 16;
    const int perm = 4 * (rl % 4) + rl / 4;
    // the block's 16 operand rows are query rows R0 .. R0 + 15 of kv head g;
    // row R is query head g * G + R % G of token R / G (all G query heads of
    // a kv head share its K/V rows)
    const int g = blockIdx.x, G = p.G;
    const int R0 = (gridDim.y - 1 - blockIdx.y) * kPMT;  // the longest blocks first
    const int tlast = min((R0 + kPMT - 1) / G, p.m - 1);
    const int plast = p.pos0 + tlast;  // the last position any row of the block sees
    const int nch = plast / kPMC + 1;
    const double scale = 1.0 / sqrt((double)HS);

    // Q operand of step ks: row rl, k ql = query row R0 + perm, dimension
    // 4 ks + ql. Tokens past the chunk read the query buffer's zeroed spare
    // rows (it holds whole 16-token tiles, and R0 + 15 < 16 * ceil(m / 16) * G).
    double qa[NKS];
    {
        const int R = R0 + perm;
        const float* qrow = p.q + (size_t)(R / G) * p.d + ((size_t)g * G + R % G) * HS;
#pragma unroll
        for (int ks = 0; ks < NKS; ks++) qa[ks] = (double)qrow[4 * ks + ql];
    }
    // causal limit of the rows this lane's registers hold: row R0 + 4 ql + r
    int tpos[4];
#pragma unroll
    for (int r = 0; r < 4; r++) tpos[r] = p.pos0 + (R0 + 4 * ql + r) / G;
    v4d acc[NT];
#pragma unroll
    for (int j = 0; j < NT; j++) acc[j] = v4d{0.0, 0.0, 0.0, 0.0};
    double mrun[4], lrun[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
        mrun[r] = -INFINITY;
        lrun[r] = 0.0;
    }

    // staging: the chunk's 16 K rows and 16 V rows, NT float4 of each per lane
    f32x4 kr[NT], vr[NT];
    auto stage_load = [&](int c) {
#pragma unroll
        for (int i = 0; i < NT; i++) {
            const int idx = lane + 64 * i, row = idx / F4ROW, col = idx % F4ROW;
            const int pp = min(c * kPMC + row, plast);  // rows past the last one repeat it (masked)
            const size_t off = (size_t)pp * p.kvd + (size_t)g * HS + 4 * col;
            kr[i] = *(const f32x4*)(p.kc + off);
            vr[i] = *(const f32x4*)(p.vc + off);
        }
    };
    auto stage_store = [&]() {
#pragma unroll
        for (int i = 0; i < NT; i++) {
            const int idx = lane + 64 * i, row = idx / F4ROW, col = idx % F4ROW;
            *(f32x4*)&L.k[row][4 * col] = kr[i];
            *(f32x4*)&L.v[row][4 * col] = vr[i];
        }
    };

    for (int c = w; c < nch; c += W) {
        stage_load(c);
        stage_store();
        lds_wave_sync();

        // S = Q K^T: operand B[k ql][col rl] = K[position rl][4 ks + ql]; two
        // interleaved accumulators halve the dependent chain
        v4d s0 = v4d{0.0, 0.0, 0.0, 0.0}, s1 = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int ks = 0; ks < NKS; ks += 2) {
            s0 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks], (double)L.k[rl][4 * ks + ql], s0, 0, 0, 0);
            if (ks + 1 < NKS)
                s1 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks + 1], (double)L.k[rl][4 * ks + 4 + ql], s1, 0, 0, 0);
        }
        const v4d sacc = s0 + s1;

        // causal mask, online softmax; register r is query row R0 + 4 ql + r,
        // lane rl is position c*16 + rl
        const int pp = c * kPMC + rl;
        double pr[4], mn[4], ms[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const double sv = pp <= tpos[r] ? sacc[r] * scale : -INFINITY;
            mn[r] = fmax(mrun[r], row16_max(sv));
            // a token may see none of this wavefront's positions so far (its
            // first chunks lie past it): then every term is 0, not e^(-inf + inf)
            ms[r] = mn[r] == -INFINITY ? 0.0 : mn[r];
            pr[r] = exp(sv - ms[r]);
        }
        // the rescale factor of token 4 ql + r is the same in all 16 lanes of
        // the row: lane rl computes the one of r = rl % 4 and each quad of
        // lanes shares its four by DPP broadcast
        const int ro = rl & 3;
        const double mo = ro == 0 ? mrun[0] : ro == 1 ? mrun[1] : ro == 2 ? mrun[2] : mrun[3];
        const double so = ro == 0 ? ms[0] : ro == 1 ? ms[1] : ro == 2 ? ms[2] : ms[3];
        const double ao = exp(mo - so);  // 0 on the first chunk the token sees
        double alpha[4];
        alpha[0] = dpp_f64<0x00>(ao);
        alpha[1] = dpp_f64<0x55>(ao);
        alpha[2] = dpp_f64<0xAA>(ao);
        alpha[3] = dpp_f64<0xFF>(ao);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            lrun[r] = lrun[r] * alpha[r] + row16_sum(pr[r]);
            mrun[r] = mn[r];
        }
#pragma unroll
        for (int j = 0; j < NT; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) acc[j][r] *= alpha[r];

        // O += P V: P through LDS into operand order, B[k ql][col rl] = V[4 ks + ql][16 j + rl]
#pragma unroll
        for (int r = 0; r < 4; r++) L.pt[4 * ql + r][rl] = pr[r];
        lds_wave_sync();
#pragma unroll
        for (int ks = 0; ks < kPMC / 4; ks++) {
            const double a = L.pt[perm][4 * ks + ql];
#pragma unroll
            for (int j = 0; j < NT; j++)
                acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)L.v[4 * ks + ql][16 * j + rl], acc[j], 0, 0, 0);
        }
        lds_wave_sync();
    }

    // merge the wavefronts' partial results in a fixed order (wave 0..3): a
    // wavefront without chunks contributes m = -inf, l = 0, O = 0
    __syncthreads();
    {
        PrefillMfmaMerge& M = *(PrefillMfmaMerge*)&L;
#pragma unroll
        for (int j = 0; j < NT; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) M.o[lane][4 * j + r] = acc[j][r];
        if (rl == 0)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                M.m[4 * ql + r] = mrun[r];
                M.l[4 * ql + r] = lrun[r];
            }
    }
    __syncthreads();
    // wave w finishes tiles w, w + W, ...
    for (int j = w; j < NT; j += W) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int tk = 4 * ql + r;
            double mw[W], mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < W; u++) {
                mw[u] = ((PrefillMfmaMerge*)&((PrefillMfmaWaveLds*)smem)[u])->m[tk];
                mx = fmax(mx, mw[u]);
            }
            double O = 0.0, Lsum = 0.0;
#pragma unroll
            for (int u = 0; u < W; u++) {
                const PrefillMfmaMerge* Mu = (const PrefillMfmaMerge*)&((PrefillMfmaWaveLds*)smem)[u];
                const double f = exp(mw[u] - mx);  // 0 for a wavefront without chunks
                O += f * Mu->o[lane][4 * j + r];
                Lsum += f * Mu->l[tk];
            }
            const int R = R0 + tk, t = R / G;
            if (t < p.m)
                p.o[(size_t)t * p.d + ((size_t)g * G + R % G) * HS + 16 * j + rl] = (float)(O / Lsum);
        }
    }
}

template <int NT, int W>
static hipError_t prefill_mfma_lds_attr()
{
    static bool done = false;
    if (!done) {
        hipError_t e = hipFuncSetAttribute((const void*)prefill_attn_mfma_kernel<NT, W>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(W * sizeof(PrefillMfmaWaveLds)));
        if (e != hipSuccess) return e;
        done = true;
    }
    return hipSuccess;
}

template <int NT, int W>
static hipError_t launch_prefill_mfma(const PrefillAttnParams& p, hipStream_t s, const LaunchEvents* ev)
{
    if (hipError_t e = prefill_mfma_lds_attr<NT, W>(); e != hipSuccess) return e;
    const dim3 grid((unsigned)p.nkv, (unsigned)(((int64_t)p.m * p.G + kPMT - 1) / kPMT));
    const size_t lds = W * sizeof(PrefillMfmaWaveLds);
    if (ev)
        hipExtLaunchKernelGGL((prefill_attn_mfma_kernel<NT, W>), grid, dim3(64 * W), (uint32_t)lds, s, ev->start,
                              ev->stop, 0u, p);
    else
        hipLaunchKernelGGL((prefill_attn_mfma_kernel<NT, W>), grid, dim3(64 * W), lds, s, p);
    return hipGetLastError();
}

template <int W>
static hipError_t launch_prefill_mfma_w(const PrefillAttnParams& p, hipStream_t s, const LaunchEvents* ev)
{
    switch (p.hs / 16) {
    case 1: return launch_prefill_mfma<1, W>(p, s, ev);
    case 2: return launch_prefill_mfma<2, W>(p, s, ev);
    case 3: return launch_prefill_mfma<3, W>(p, s, ev);
    case 4: return launch_prefill_mfma<4, W>(p, s, ev);
    case 5: return launch_prefill_mfma<5, W>(p, s, ev);
    case 6: return launch_prefill_mfma<6, W>(p, s, ev);
    case 7: return launch_prefill_mfma<7, W>(p, s, ev);
    case 8: return launch_prefill_mfma<8, W>(p, s, ev);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill_attn(const PrefillAttnParams& p, hipStream_t s, const LaunchEvents* ev)
{
    if (prefill_attn_mfma_ok(p.G, p.hs) && !getenv("L2D_PREFILL_ATTN_VALU")) {
        return launch_prefill_mfma_w<kPMW>(p, s, ev);
    }
    const int kg = prefill_attn_rows(p.G, p.hs);
    if (kg == 0) return hipErrorInvalidValue;
    const int TB = kg / p.G;
    const dim3 grid((unsigned)p.nkv, (unsigned)((p.m + TB - 1) / TB));
    const size_t lds = attn_core_lds_bytes<kPAThreads>(kg, p.hs);
#define L2D_PA(KG)                                                                                  \
    if (ev)                                                                                         \
        hipExtLaunchKernelGGL(prefill_attn_kernel<KG>, grid, dim3(kPAThreads), (uint32_t)lds, s,    \
                              ev->start, ev->stop, 0u, p);                                          \
    else                                                                                            \
        hipLaunchKernelGGL(prefill_attn_kernel<KG>, grid, dim3(kPAThreads), lds, s, p);
    switch (kg) {
    case 8: L2D_PA(8) break;
    case 4: L2D_PA(4) break;
    case 2: L2D_PA(2) break;
    case 1: L2D_PA(1) break;
    default: return hipErrorInvalidValue;
    }
#undef L2D_PA
    return hipGetLastError();
}

}  // namespace l2d
