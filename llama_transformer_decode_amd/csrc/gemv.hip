// gemv.hip - batch-1 matrix-vector products of the decode step on gfx950.
//
// One kernel template serves every matvec of the step (q/k/v, output
// projection, w1/w3, w2, classifier: the hand-written row-by-row matmul of
// the ainews article's technical section, over HBM-resident weights):
//
//   prologue  every workgroup builds the input vector in LDS in one parallel
//             pass (16 values per thread): x as is, or RMSNorm(x) (pomoai.com
//             hub page, architecture list), and for Q8_0 the int8 codes and
//             group scales of that vector (gitcode porting guide, INT8
//             quantisation section; the group max is a DPP lane reduction);
//   main loop each wavefront owns a contiguous, balanced range of row tiles
//             (RPW rows each) and streams them in chunks of U 16-byte loads
//             per row, double-buffered: the next chunk is in flight while the
//             current one is consumed, and the first chunk is issued before
//             the prologue so its HBM latency overlaps the prologue. Lanes
//             cover 64 x 16 B = 1 KiB contiguous per load instruction. fp32
//             rows multiply-add into fp64 (a product of two fp32 values is
//             exact in fp64); Q8_0 rows use v_dot4_i32_i8 for exact int32
//             group dots (DPP quad sums), combined in fp64 with the weight
//             and activation scales;
//   epilogue  a DPP wave sum leaves each row's total in lane 63, which
//             finishes the tile: store, residual add, RoPE + KV-cache write,
//             SwiGLU, or classifier + packed argmax.
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace l2d {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// ---------------------------------------------------------------- prologue

// block-wide fp64 sum, fixed order (wave butterfly, then waves 0..3)
__device__ __forceinline__ double block_sum(double v, double* red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_sum(v);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }

// fp32 input vector -> LDS as float4 chunks (thread t takes chunks t, t+256,
// ...). NC: float4 chunks per thread kept in registers for RMSNorm.
template <int PRO, int NC>
__device__ __forceinline__ void prologue_f32(const GemvParams& p, unsigned char* smem)
{
    const int tid = threadIdx.x;
    const int64_t K4 = p.K / 4;
    f32x4* xl = (f32x4*)smem;
    __shared__ double red[kWaves];
    if (PRO == PRO_NORM) {
        f32x4 xv[NC], gv[NC];
#pragma unroll
        for (int j = 0; j < NC; j++) {
            const int64_t c = (int64_t)j * kThreads + tid;
            xv[j] = c < K4 ? ld4(p.x + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
            gv[j] = c < K4 ? ld4(p.gain + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        double ss = 0.0;
#pragma unroll
        for (int j = 0; j < NC; j++) {
            ss += (double)xv[j].x * (double)xv[j].x;
            ss += (double)xv[j].y * (double)xv[j].y;
            ss += (double)xv[j].z * (double)xv[j].z;
            ss += (double)xv[j].w * (double)xv[j].w;
        }
        ss = block_sum(ss, red);
        const double r = 1.0 / sqrt(ss / (double)p.K + p.eps);
#pragma unroll
        for (int j = 0; j < NC; j++) {
            const int64_t c = (int64_t)j * kThreads + tid;
            if (c < K4) {
                f32x4 o;
                o.x = (float)((double)gv[j].x * ((double)xv[j].x * r));
                o.y = (float)((double)gv[j].y * ((double)xv[j].y * r));
                o.z = (float)((double)gv[j].z * ((double)xv[j].z * r));
                o.w = (float)((double)gv[j].w * ((double)xv[j].w * r));
                xl[c] = o;
            }
        }
    } else {
        constexpr int B = 8;  // loads in flight per thread
        for (int64_t base = 0; base < K4; base += (int64_t)B * kThreads) {
            f32x4 v[B];
#pragma unroll
            for (int j = 0; j < B; j++) {
                const int64_t c = base + (int64_t)j * kThreads + tid;
                v[j] = c < K4 ? ld4(p.x + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int j = 0; j < B; j++) {
                const int64_t c = base + (int64_t)j * kThreads + tid;
                if (c < K4) xl[c] = v[j];
            }
        }
    }
    __syncthreads();
}

// quantise one 16-value chunk (this lane's part of a group of lpg lanes)
__device__ __forceinline__ i32x4 quant16(const float* v, int lpg, float* scale_out)
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) m = fmaxf(m, fabsf(v[i]));
    m = lanes_max_f32(m, lpg);
    const float sc = q80_scale(m);
    *scale_out = sc;
    int w[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        uint32_t b = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int q = q80_code(v[4 * k + i], sc);
            b |= ((uint32_t)(q & 0xFF)) << (8 * i);
        }
        w[k] = (int)b;
    }
    return i32x4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ void load16(float* v, const float* src, bool ok)
{
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const f32x4 a = ok ? ld4(src + 4 * k) : f32x4{0.f, 0.f, 0.f, 0.f};
        v[4 * k] = a.x;
        v[4 * k + 1] = a.y;
        v[4 * k + 2] = a.z;
        v[4 * k + 3] = a.w;
    }
}

// Q8_0 input vector -> LDS codes [K] + scales [K/gs] (thread t takes 16-value
// chunks t, t+256, ...; the lpg = gs/16 lanes of a group are adjacent).
// NC: 16-value chunks per thread kept in registers for RMSNorm.
template <int PRO, int NC>
__device__ __forceinline__ void prologue_q8(const GemvParams& p, unsigned char* smem)
{
    const int tid = threadIdx.x;
    const int64_t nq = p.K / 16;
    const int lpg = p.gs / 16;
    i32x4* xq = (i32x4*)smem;
    float* xs = (float*)(smem + p.K);
    __shared__ double red[kWaves];
    if (PRO == PRO_NORM) {
        float xv[NC][16], gv[NC][16];
#pragma unroll
        for (int j = 0; j < NC; j++) {
            const int64_t c = (int64_t)j * kThreads + tid;
            load16(xv[j], p.x + 16 * c, c < nq);
            load16(gv[j], p.gain + 16 * c, c < nq);
        }
        double ss = 0.0;
#pragma unroll
        for (int j = 0; j < NC; j++)
#pragma unroll
            for (int i = 0; i < 16; i++) ss += (double)xv[j][i] * (double)xv[j][i];
        ss = block_sum(ss, red);
        const double r = 1.0 / sqrt(ss / (double)p.K + p.eps);
#pragma unroll
        for (int j = 0; j < NC; j++) {
            const int64_t c = (int64_t)j * kThreads + tid;
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; i++) v[i] = (float)((double)gv[j][i] * ((double)xv[j][i] * r));
            float sc;
            const i32x4 codes = quant16(v, lpg, &sc);
            if (c < nq) {
                xq[c] = codes;
                if ((c & (lpg - 1)) == 0) xs[c / lpg] = sc;
            }
        }
    } else {
        constexpr int B = 4;  // 16-value chunks in flight per thread
        for (int64_t base = 0; base < nq; base += (int64_t)B * kThreads) {
            float v[B][16];
#pragma unroll
            for (int j = 0; j < B; j++) {
                const int64_t c = base + (int64_t)j * kThreads + tid;
                load16(v[j], p.x + 16 * c, c < nq);
            }
#pragma unroll
            for (int j = 0; j < B; j++) {
                const int64_t c = base + (int64_t)j * kThreads + tid;
                float sc;
                const i32x4 codes = quant16(v[j], lpg, &sc);
                if (c < nq) {
                    xq[c] = codes;
                    if ((c & (lpg - 1)) == 0) xs[c / lpg] = sc;
                }
            }
        }
    }
    __syncthreads();
    if (p.trace_q != nullptr && blockIdx.x == 0) {
        for (int64_t c = tid; c < nq; c += kThreads) ((i32x4*)p.trace_q)[c] = xq[c];
        for (int64_t g = tid; g < p.K / p.gs; g += kThreads) p.trace_s[g] = xs[g];
    }
}

// ---------------------------------------------------------------- epilogue

template <int EPI>
__device__ __forceinline__ void gemv_epilogue(const GemvParams& p, int64_t row0, int rpw,
                                              const double* acc, unsigned long long& best)
{
    if (EPI == EPI_STORE) {
        for (int r = 0; r < rpw; r++)
            if (row0 + r < p.M) p.out[row0 + r] = (float)acc[r];
    } else if (EPI == EPI_RESID) {
        for (int r = 0; r < rpw; r++) {
            const int64_t row = row0 + r;
            if (row < p.M) {
                const float y = (float)acc[r];
                p.out[row] = (float)((double)p.out[row] + (double)y);
            }
        }
    } else if (EPI == EPI_LOGITS) {
        for (int r = 0; r < rpw; r++) {
            const int64_t row = row0 + r;
            if (row < p.M) {
                const float y = (float)acc[r];
                p.out[row] = y;
                const unsigned long long key = argmax_pack(y, (uint32_t)row);
                best = key > best ? key : best;
            }
        }
    } else if (EPI == EPI_SWIGLU) {
        // rows (2i, 2i+1) hold w1 row i and w3 row i
        for (int r = 0; r + 1 < rpw; r += 2) {
            const int64_t row = row0 + r;
            if (row + 1 < p.M) {
                const double z = (double)(float)acc[r];
                const double h3 = (double)(float)acc[r + 1];
                const double silu = z / (1.0 + exp(-z));
                p.out[row / 2] = (float)(silu * h3);
            }
        }
    } else if (EPI == EPI_QKV) {
        // rows [0, d) q, [d, d+kvd) k, [d+kvd, d+2kvd) v; pairs (2j, 2j+1)
        // of each q/k head rotate by pos * freq_j (RoPE, computed on the fly)
        const int pos = p.step[1];
        for (int r = 0; r + 1 < rpw; r += 2) {
            const int64_t row = row0 + r;
            if (row + 1 >= p.M) continue;
            const float a = (float)acc[r], b = (float)acc[r + 1];
            if (row < p.d + p.kvd) {
                const int64_t within = row < p.d ? row : row - p.d;
                const int j = (int)((within % p.hs) / 2);
                const float ang = (float)pos * p.freqs[j];
                const double c = (double)(float)cos((double)ang);
                const double s = (double)(float)sin((double)ang);
                const float ra = (float)((double)a * c - (double)b * s);
                const float rb = (float)((double)a * s + (double)b * c);
                if (row < p.d) {
                    p.out[row] = ra;
                    p.out[row + 1] = rb;
                } else {
                    float* kslot = p.kcache + (int64_t)pos * p.kvd + within;
                    kslot[0] = ra;
                    kslot[1] = rb;
                }
            } else {
                float* vslot = p.vcache + (int64_t)pos * p.kvd + (row - p.d - p.kvd);
                vslot[0] = a;
                vslot[1] = b;
            }
        }
    }
}

// ---------------------------------------------------------------- main loop

// One chunk of a tile: U loads of 16 bytes per lane for each of RPW rows.
template <int DT, int RPW, int U>
struct Chunk {
    using V = typename std::conditional<DT == DT_F32, f32x4, i32x4>::type;
    V w[RPW][U];
    float s[RPW][U];  // Q8_0: the weight scale of this lane's group
};

template <int DT, int RPW, int U>
__device__ __forceinline__ void load_chunk(Chunk<DT, RPW, U>& ch, const GemvParams& p, int64_t row0,
                                           int64_t c0, int64_t Kv, int lane, int gshift)
{
#pragma unroll
    for (int uu = 0; uu < U; uu++) {
        const int64_t c = c0 + uu * kWave + lane;
#pragma unroll
        for (int r = 0; r < RPW; r++) {
            const bool ok = c < Kv && row0 + r < p.M;
            if constexpr (DT == DT_F32) {
                const f32x4* W = (const f32x4*)p.W + (row0 + r) * Kv;
                ch.w[r][uu] = ok ? __builtin_nontemporal_load(W + c) : f32x4{0.f, 0.f, 0.f, 0.f};
            } else {
                const i32x4* W = (const i32x4*)p.W + (row0 + r) * Kv;
                ch.w[r][uu] = ok ? __builtin_nontemporal_load(W + c) : i32x4{0, 0, 0, 0};
                const int64_t ngr = (Kv * 16) >> (gshift + 4);
                ch.s[r][uu] = ok ? p.Ws[(row0 + r) * ngr + (c >> gshift)] : 0.0f;
            }
        }
    }
}

template <int DT, int RPW, int U, bool DBG>
__device__ __forceinline__ void use_chunk(const Chunk<DT, RPW, U>& ch, double* acc,
                                          const GemvParams& p, const unsigned char* smem,
                                          int64_t row0, int64_t c0, int64_t Kv, int lane,
                                          int gshift, int lpg)
{
#pragma unroll
    for (int uu = 0; uu < U; uu++) {
        const int64_t c = c0 + uu * kWave + lane;
        const bool ok = c < Kv;
        if constexpr (DT == DT_F32) {
            const f32x4 xv = ok ? ((const f32x4*)smem)[c] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                const f32x4 w = ch.w[r][uu];
                acc[r] += (double)w.x * (double)xv.x;
                acc[r] += (double)w.y * (double)xv.y;
                acc[r] += (double)w.z * (double)xv.z;
                acc[r] += (double)w.w * (double)xv.w;
            }
        } else {
            const i32x4 xv = ok ? ((const i32x4*)smem)[c] : i32x4{0, 0, 0, 0};
            const float* xs = (const float*)(smem + Kv * 16);
            const int64_t g = c >> gshift;
            const double xsg = ok ? (double)xs[g] : 0.0;
            const bool lead = (lane & (lpg - 1)) == 0;
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                int d = dot16_i8(ch.w[r][uu], xv);
                d = lanes_sum_i32(d, lpg);
                const double t = ((double)d * (double)ch.s[r][uu]) * xsg;
                acc[r] += (ok && lead) ? t : 0.0;
                if (DBG && ok && lead && row0 + r < p.M) {
                    const int64_t ngr = (Kv * 16) >> (gshift + 4);
                    p.group_dots[(row0 + r) * ngr + g] = d;
                }
            }
        }
    }
}

template <int DT, int PRO, int EPI, int RPW, int U, int NC, bool DBG>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t Kv = DT == DT_F32 ? p.K / 4 : p.K / 16;  // 16-byte vectors per row
    const int gshift = DT == DT_F32 ? 0 : ilog2(p.gs) - 4;  // vector index -> group
    const int lpg = DT == DT_F32 ? 1 : p.gs / 16;            // lanes per group
    const int64_t CH = (int64_t)kWave * U;                  // vectors per row per chunk
    const int64_t nch = (Kv + CH - 1) / CH;                  // chunks per tile

    // balanced contiguous range of tiles for this wave
    const int64_t tiles = (p.M + RPW - 1) / RPW;
    const int64_t nw = (int64_t)gridDim.x * kWaves;
    const int64_t gw = (int64_t)blockIdx.x * kWaves + wave;
    const int64_t t_beg = tiles * gw / nw, t_end = tiles * (gw + 1) / nw;
    const int64_t iters = (t_end - t_beg) * nch;

    Chunk<DT, RPW, U> A, B;
    if (iters > 0) load_chunk<DT, RPW, U>(A, p, t_beg * RPW, 0, Kv, lane, gshift);

    if constexpr (DT == DT_F32)
        prologue_f32<PRO, NC>(p, smem);
    else
        prologue_q8<PRO, NC>(p, smem);

    double acc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; r++) acc[r] = 0.0;
    unsigned long long best = 0;
    int64_t tile = t_beg, ch = 0;  // position of the chunk in A
    int64_t ntile = t_beg, nchk = 0;

    auto advance = [&](int64_t& t, int64_t& c) {
        if (++c == nch) {
            c = 0;
            ++t;
        }
    };
    auto finish_tile = [&]() {
#pragma unroll
        for (int r = 0; r < RPW; r++) acc[r] = wave_sum_to_last(acc[r]);
        if (lane == kWave - 1) gemv_epilogue<EPI>(p, tile * RPW, RPW, acc, best);
#pragma unroll
        for (int r = 0; r < RPW; r++) acc[r] = 0.0;
    };

    for (int64_t it = 0; it < iters; it += 2) {
        // A holds chunk `it`; fetch it+1 into B, then consume A
        ntile = tile;
        nchk = ch;
        advance(ntile, nchk);
        if (it + 1 < iters) load_chunk<DT, RPW, U>(B, p, ntile * RPW, nchk * CH, Kv, lane, gshift);
        use_chunk<DT, RPW, U, DBG>(A, acc, p, smem, tile * RPW, ch * CH, Kv, lane, gshift, lpg);
        if (ch == nch - 1) finish_tile();
        tile = ntile;
        ch = nchk;
        if (it + 1 >= iters) break;
        // B holds chunk it+1; fetch it+2 into A, then consume B
        ntile = tile;
        nchk = ch;
        advance(ntile, nchk);
        if (it + 2 < iters) load_chunk<DT, RPW, U>(A, p, ntile * RPW, nchk * CH, Kv, lane, gshift);
        use_chunk<DT, RPW, U, DBG>(B, acc, p, smem, tile * RPW, ch * CH, Kv, lane, gshift, lpg);
        if (ch == nch - 1) finish_tile();
        tile = ntile;
        ch = nchk;
    }
    if (EPI == EPI_LOGITS && lane == kWave - 1 && best != 0)
        atomicMax(p.argmax + (p.step[1] & 1), best);
}

size_t gemv_lds_bytes(int dt, int64_t K, int gs)
{
    if (dt == DT_F32) return (size_t)K * 4;
    return (size_t)K + (size_t)(K / gs) * 4;
}

template <int DT, int PRO, int EPI, int RPW, int U, int NC, bool DBG>
static hipError_t launch_t(const GemvParams& p, int blocks, hipStream_t s)
{
    const size_t lds = gemv_lds_bytes(DT, p.K, p.gs);
    hipLaunchKernelGGL((gemv_kernel<DT, PRO, EPI, RPW, U, NC, DBG>), dim3((unsigned)blocks),
                       dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

// Launch shape: RPW rows per tile, U loads per row per chunk, and the grid.
// Every wave gets a contiguous 1/nw share of the tiles; the grid is capped at
// max_blocks workgroups and never exceeds one tile per wave. NC (RMSNorm
// prologues only) is the smallest register budget that holds the input.
template <int DT, int PRO, int EPI, bool DBG>
static hipError_t launch_shape(const GemvParams& p, int max_blocks, hipStream_t s)
{
    constexpr int RPW = DT == DT_F32 ? 2 : 4;
    constexpr int U = DT == DT_F32 ? 4 : 2;
    const int64_t tiles = (p.M + RPW - 1) / RPW;
    int64_t blocks = (tiles + kWaves - 1) / kWaves;
    if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) blocks = 1;
    const int64_t per_thread = DT == DT_F32 ? (p.K / 4 + kThreads - 1) / kThreads
                                            : (p.K / 16 + kThreads - 1) / kThreads;
    if (PRO == PRO_PLAIN || per_thread <= 1)
        return launch_t<DT, PRO, EPI, RPW, U, 1, DBG>(p, (int)blocks, s);
    if (per_thread <= 2) return launch_t<DT, PRO, EPI, RPW, U, 2, DBG>(p, (int)blocks, s);
    if (per_thread <= 4) return launch_t<DT, PRO, EPI, RPW, U, 4, DBG>(p, (int)blocks, s);
    if (DT == DT_F32 && per_thread <= 16)
        return launch_t<DT, PRO, EPI, RPW, U, 16, DBG>(p, (int)blocks, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(int dt, int pro, int epi, const GemvParams& p, int max_blocks,
                       hipStream_t s)
{
#define L2D_CASE(D, P, E)                                                  \
    if (dt == D && pro == P && epi == E) {                                 \
        if (D == DT_Q8 && p.group_dots != nullptr)                         \
            return launch_shape<D, P, E, true>(p, max_blocks, s);          \
        return launch_shape<D, P, E, false>(p, max_blocks, s);             \
    }
    L2D_CASE(DT_F32, PRO_NORM, EPI_QKV)
    L2D_CASE(DT_F32, PRO_PLAIN, EPI_RESID)
    L2D_CASE(DT_F32, PRO_NORM, EPI_SWIGLU)
    L2D_CASE(DT_F32, PRO_NORM, EPI_LOGITS)
    L2D_CASE(DT_F32, PRO_PLAIN, EPI_STORE)
    L2D_CASE(DT_Q8, PRO_NORM, EPI_QKV)
    L2D_CASE(DT_Q8, PRO_PLAIN, EPI_RESID)
    L2D_CASE(DT_Q8, PRO_NORM, EPI_SWIGLU)
    L2D_CASE(DT_Q8, PRO_NORM, EPI_LOGITS)
    L2D_CASE(DT_Q8, PRO_PLAIN, EPI_STORE)
#undef L2D_CASE
    return hipErrorInvalidValue;
}

}  // namespace l2d
