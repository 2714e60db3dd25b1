// gemv.hip - batch-1 matrix-vector products of the decode step on gfx950.
//
// One kernel template serves every matvec of the step (q/k/v, output
// projection, w1/w3, w2, classifier; the hand-written matmul of the ainews
// article's technical section, run per row over HBM-resident weights):
//
//   prologue  every workgroup builds the input vector in LDS: x as is, or
//             RMSNorm(x) (pomoai.com hub page, architecture list), and for
//             Q8_0 the int8 codes + group scales of that vector (gitcode
//             porting guide, INT8 quantisation section);
//   main loop each wavefront owns RPW consecutive rows and streams them with
//             16-byte nontemporal loads, U loads per row in flight, lanes
//             covering 64 x 16 B = 1 KiB contiguous per load instruction;
//             fp32 rows multiply-add into fp64 (a product of two fp32 values
//             is exact in fp64), Q8_0 rows use v_dot4_i32_i8 for exact int32
//             group dots, combined in fp64 with the weight and activation
//             scales;
//   epilogue  lane 0 finishes the rows: store, residual add, RoPE + KV-cache
//             write, SwiGLU, or classifier + packed argmax.
//
// The weights are read exactly once per step; nothing else in the step
// touches HBM in comparable volume, so this kernel's bandwidth is the step's.
#include "device.hpp"
#include "internal.hpp"

namespace l2d {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int DT, int PRO>
__device__ __forceinline__ void gemv_prologue(const GemvParams& p, unsigned char* smem)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t K = p.K;
    __shared__ double red[kWaves];
    double r = 1.0;
    if (PRO == PRO_NORM) {
        // sum of squares in fp64, fixed order: strided per thread, butterfly
        // per wave, then the four waves in index order
        double ss = 0.0;
        for (int64_t i = tid; i < K; i += kThreads) {
            const double v = (double)p.x[i];
            ss += v * v;
        }
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        ss = red[0] + red[1] + red[2] + red[3];
        r = 1.0 / sqrt(ss / (double)K + p.eps);
    }
    auto val = [&](int64_t i) -> float {
        if (PRO == PRO_NORM) return (float)((double)p.gain[i] * ((double)p.x[i] * r));
        return p.x[i];
    };
    if (DT == DT_F32) {
        float* xf = (float*)smem;
        for (int64_t i = tid; i < K; i += kThreads) xf[i] = val(i);
    } else {
        int8_t* xq = (int8_t*)smem;
        float* xs = (float*)(smem + K);
        q80_groups_wave(val, K / p.gs, p.gs, wave, kWaves, xq, xs, lane);
        __syncthreads();
        if (p.trace_q != nullptr && blockIdx.x == 0) {
            for (int64_t i = tid; i < K; i += kThreads) p.trace_q[i] = xq[i];
            for (int64_t g = tid; g < K / p.gs; g += kThreads) p.trace_s[g] = xs[g];
        }
    }
    __syncthreads();
}

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

template <int DT, int PRO, int EPI, int RPW, int U, bool DBG>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    gemv_prologue<DT, PRO>(p, smem);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t K = p.K;
    const int64_t units = (p.M + RPW - 1) / RPW;
    unsigned long long best = 0;

    for (int64_t u = (int64_t)blockIdx.x * kWaves + wave; u < units;
         u += (int64_t)gridDim.x * kWaves) {
        const int64_t row0 = u * RPW;
        double acc[RPW];
#pragma unroll
        for (int r = 0; r < RPW; r++) acc[r] = 0.0;

        if (DT == DT_F32) {
            const int64_t K4 = K / 4;
            const f32x4* W4 = (const f32x4*)p.W + row0 * K4;
            const f32x4* x4 = (const f32x4*)smem;
            for (int64_t c0 = 0; c0 < K4; c0 += (int64_t)kWave * U) {
                f32x4 wv[RPW][U];
#pragma unroll
                for (int uu = 0; uu < U; uu++) {
                    const int64_t c = c0 + uu * kWave + lane;
#pragma unroll
                    for (int r = 0; r < RPW; r++) {
                        const bool ok = c < K4 && row0 + r < p.M;
                        wv[r][uu] = ok ? __builtin_nontemporal_load(W4 + r * K4 + c)
                                       : f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
#pragma unroll
                for (int uu = 0; uu < U; uu++) {
                    const int64_t c = c0 + uu * kWave + lane;
                    if (c < K4) {
                        const f32x4 xv = x4[c];
#pragma unroll
                        for (int r = 0; r < RPW; r++) {
                            acc[r] += (double)wv[r][uu].x * (double)xv.x;
                            acc[r] += (double)wv[r][uu].y * (double)xv.y;
                            acc[r] += (double)wv[r][uu].z * (double)xv.z;
                            acc[r] += (double)wv[r][uu].w * (double)xv.w;
                        }
                    }
                }
            }
        } else {
            const int gs = p.gs;
            const int lpg = gs / 16;  // lanes per group (16 codes per lane per load)
            const int64_t K16 = K / 16;
            const int64_t ngr = K / gs;
            const i32x4* Wq = (const i32x4*)((const int8_t*)p.W + row0 * K);
            const float* Wsr = p.Ws + row0 * ngr;
            const i32x4* xq4 = (const i32x4*)smem;
            const float* xs = (const float*)(smem + K);
            const bool lead = (lane % lpg) == 0;
            for (int64_t c0 = 0; c0 < K16; c0 += (int64_t)kWave * U) {
                i32x4 wv[RPW][U];
                float wsv[RPW][U];
#pragma unroll
                for (int uu = 0; uu < U; uu++) {
                    const int64_t c = c0 + uu * kWave + lane;
                    const int64_t g = (c * 16) / gs;
#pragma unroll
                    for (int r = 0; r < RPW; r++) {
                        const bool ok = c < K16 && row0 + r < p.M;
                        wv[r][uu] = ok ? __builtin_nontemporal_load(Wq + r * K16 + c)
                                       : i32x4{0, 0, 0, 0};
                        wsv[r][uu] = (ok && lead) ? Wsr[r * ngr + g] : 0.0f;
                    }
                }
#pragma unroll
                for (int uu = 0; uu < U; uu++) {
                    const int64_t c = c0 + uu * kWave + lane;
                    const bool ok = c < K16;
                    const int64_t g = (c * 16) / gs;
                    const i32x4 xv = ok ? xq4[c] : i32x4{0, 0, 0, 0};
                    const double xsg = ok ? (double)xs[g] : 0.0;
#pragma unroll
                    for (int r = 0; r < RPW; r++) {
                        int d = dot16_i8(wv[r][uu], xv);
                        d = group_sum_i32(d, lpg);
                        if (ok && lead && row0 + r < p.M) {
                            acc[r] += ((double)d * (double)wsv[r][uu]) * xsg;
                            if (DBG) p.group_dots[(row0 + r) * ngr + g] = d;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RPW; r++) acc[r] = wave_sum(acc[r]);
        if (lane == 0) gemv_epilogue<EPI>(p, row0, RPW, acc, best);
    }
    if (EPI == EPI_LOGITS && lane == 0 && best != 0)
        atomicMax(p.argmax + (p.step[1] & 1), best);
}

size_t gemv_lds_bytes(int dt, int64_t K, int gs)
{
    if (dt == DT_F32) return (size_t)K * 4;
    return (size_t)K + (size_t)(K / gs) * 4;
}

template <int DT, int PRO, int EPI, bool DBG = false>
static hipError_t launch_t(const GemvParams& p, int max_blocks, hipStream_t s)
{
    constexpr int RPW = DT == DT_F32 ? 2 : 4;
    constexpr int U = DT == DT_F32 ? 4 : 2;
    const int64_t units = (p.M + RPW - 1) / RPW;
    int64_t blocks = (units + kWaves - 1) / kWaves;
    if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) blocks = 1;
    const size_t lds = gemv_lds_bytes(DT, p.K, p.gs);
    hipLaunchKernelGGL((gemv_kernel<DT, PRO, EPI, RPW, U, DBG>), dim3((unsigned)blocks),
                       dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_gemv(int dt, int pro, int epi, const GemvParams& p, int max_blocks,
                       hipStream_t s)
{
#define L2D_CASE(D, P, E)                                                  \
    if (dt == D && pro == P && epi == E) {                                 \
        if (D == DT_Q8 && p.group_dots != nullptr)                         \
            return launch_t<D, P, E, true>(p, max_blocks, s);              \
        return launch_t<D, P, E>(p, max_blocks, s);                        \
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
