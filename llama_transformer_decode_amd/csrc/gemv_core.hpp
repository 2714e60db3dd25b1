// gemv_core.hpp - batch-1 matrix-vector products of the decode step on gfx950.
//
// One kernel template serves every matvec of the step (q/k/v, output
// projection, w1/w3, w2, classifier: the hand-written row-by-row matmul of
// the ainews article's technical section, over HBM-resident weights).
//
// Order of work in a workgroup, arranged so that the HBM latency of the
// weights overlaps everything else:
//   1. every thread issues the loads of its share of the input vector (and
//      of the RMSNorm gain);
//   2. every wavefront issues the loads of its first NBUF weight chunks;
//   3. prologue: the input vector is prepared in LDS while those loads are in
//      flight: x as is, or RMSNorm(x) (pomoai.com hub page, architecture
//      list), and for Q8_0 the int8 codes and group scales of that vector
//      (gitcode porting guide, INT8 quantisation section; group max by DPP),
//      or codes and scales the producing kernel already made (PRO_CODES). A
//      scheduling barrier and register holds keep steps 1 and 2 in this
//      order, so the prologue waits for its own loads only;
//   4. main loop over a contiguous, balanced range of row tiles (RPW rows
//      each), as a ring of NBUF chunk buffers: consume a chunk, refill its
//      buffer with the chunk NBUF ahead, then (at a tile's end) reduce and
//      run the epilogue. Every load is unconditional (indices
//      past the end are clamped onto valid memory and their contribution is
//      masked), so each iteration issues the same loads and the compiler's
//      wait counts stay exact: NBUF-1 chunks remain in flight while one is
//      consumed.
// Lanes cover 64 x 16 B = 1 KiB contiguous per load instruction. fp32 rows
// multiply-add into fp64 (a product of two fp32 values is exact in fp64).
// Q8_0 rows are stored group-interleaved (q8_perm_offset) so that each lane
// holds whole groups: v_dot4_i32_i8 gives the exact int32 group dot in one
// lane, combined in fp64 with the weight and activation scales. Q4_0 rows
// need no re-layout: a group is 16 bytes, so one 16-byte load per lane holds
// a whole group; its nibbles are unpacked with two masks and dotted against
// the input's codes, the dot starting from -8 x (the group's input code sum)
// to undo the +8 offset of the stored nibbles.
//   epilogue  a DPP wave sum leaves each row's total in lane 63, which
//             finishes the tile: store, residual add, RoPE + KV-cache write,
//             SwiGLU, or classifier + packed argmax.
#pragma once

#include <hip/hip_ext.h>

#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace l2d {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// LDS bytes of the prepared input vector (16-byte aligned end)
__host__ __device__ inline size_t gemv_input_bytes(int dt, int64_t K, int gs)
{
    // fp32: the vector; Q8_0: codes and scales; Q4_0: codes, scales and
    // the offset terms (int32)
    const size_t b = dt == DT_F32 ? (size_t)K * 4
                   : dt == DT_Q8  ? (size_t)K + (size_t)(K / gs) * 4
                                  : (size_t)K + (size_t)(K / gs) * 8;
    return (b + 15) & ~(size_t)15;
}

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

__device__ __forceinline__ int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }

// A chained launch's quantised matvec input (the SwiGLU output's Q8_0
// codes, written by many waves of the launch on every XCD) is stored one
// group per 128-byte line: the group's codes, then its scale. A line then has
// one writer, and a reader's plain load after the wait cannot hit a partial
// copy of it in its XCD's L2 (nothing in the launch reads the line earlier,
// and the launch boundary cleared any older copy).
constexpr int kChainLine = 128;

__device__ __forceinline__ const int8_t* chain_codes(const int8_t* base, int64_t k16, int lpg)
{
    return base + (k16 / lpg) * kChainLine + (k16 % lpg) * 16;
}

__device__ __forceinline__ const float* chain_scale(const int8_t* base, int64_t g)
{
    return (const float*)(base + g * kChainLine + 64);
}

// fp32 input: thread t holds float4 chunks t, t+256, ... (NC of them)
// An empty asm that claims to redefine v: no use of v can be scheduled
// before this point (the loads themselves are not moved).
template <class T>
__device__ __forceinline__ void hold(T& v)
{
    asm volatile("" : "+v"(v));
}

template <int PRO, int NC>
struct InputF32 {
    f32x4 x[NC], g[NC];

    __device__ __forceinline__ void fence()
    {
#pragma unroll
        for (int j = 0; j < NC; j++) {
            hold(x[j]);
            if (PRO == PRO_NORM) hold(g[j]);
        }
    }

    __device__ __forceinline__ void issue(const GemvParams& p)
    {
        const int64_t K4 = p.K / 4;
#pragma unroll
        for (int j = 0; j < NC; j++) {
            const int64_t c = imin((int64_t)j * kThreads + threadIdx.x, K4 - 1);
            x[j] = ld4(p.x + 4 * c);
            if (PRO == PRO_NORM) g[j] = ld4(p.gain + 4 * c);
        }
    }

    __device__ __forceinline__ void finish(const GemvParams& p, unsigned char* smem, double* red, int)
    {
        const int64_t K4 = p.K / 4;
        f32x4* xl = (f32x4*)smem;
        double r = 1.0;
        if (PRO == PRO_NORM) {
            double ss = 0.0;
#pragma unroll
            for (int j = 0; j < NC; j++) {
                const bool ok = (int64_t)j * kThreads + threadIdx.x < K4;
                const f32x4 v = x[j];
                const double s4 = (double)v.x * (double)v.x + (double)v.y * (double)v.y +
                                  (double)v.z * (double)v.z + (double)v.w * (double)v.w;
                ss += ok ? s4 : 0.0;
            }
            ss = block_sum(ss, red);
            r = 1.0 / sqrt(ss / (double)p.K + p.eps);
        }
#pragma unroll
        for (int j = 0; j < NC; j++) {
            const int64_t c = (int64_t)j * kThreads + threadIdx.x;
            if (c < K4) {
                f32x4 o = x[j];
                if (PRO == PRO_NORM) {
                    o.x = (float)((double)g[j].x * ((double)x[j].x * r));
                    o.y = (float)((double)g[j].y * ((double)x[j].y * r));
                    o.z = (float)((double)g[j].z * ((double)x[j].z * r));
                    o.w = (float)((double)g[j].w * ((double)x[j].w * r));
                }
                xl[c] = o;
            }
        }
        __syncthreads();
    }
};

// The four vectors come by value: a pointer into the held input arrays
// lets the optimiser merge their loads across elements, which pins the
// arrays to the stack.
__device__ __forceinline__ void unpack16(float* v, f32x4 a0, f32x4 a1, f32x4 a2, f32x4 a3)
{
    const f32x4 a[4] = {a0, a1, a2, a3};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        v[4 * k] = a[k].x;
        v[4 * k + 1] = a[k].y;
        v[4 * k + 2] = a[k].z;
        v[4 * k + 3] = a[k].w;
    }
}

// Index (in 16-byte units) of 16-value input chunk c in LDS: Q8_0 in the
// group-interleaved order of the weights; Q4_0 (gs 32) in two planes, the
// first 16 codes of every group, then the last 16.
template <int DT>
__device__ __forceinline__ int64_t input_chunk_slot(int64_t c, int64_t K, int gs)
{
    if (DT == DT_Q8) return q8_perm_offset(16 * c, K, gs) / 16;
    return (c & 1) * (K / 32) + (c >> 1);
}

// Workgroup 0 copies the quantised input it holds in LDS to the trace
// buffers, back in plain element order (test hook).
template <int DT>
__device__ __forceinline__ void trace_input(const GemvParams& p, const unsigned char* smem, int bid)
{
    if (p.trace_q == nullptr || bid != 0) return;
    for (int64_t c = threadIdx.x; c < p.K / 16; c += kThreads)
        ((i32x4*)p.trace_q)[c] = ((const i32x4*)smem)[input_chunk_slot<DT>(c, p.K, p.gs)];
    for (int64_t g = threadIdx.x; g < p.K / p.gs; g += kThreads)
        p.trace_s[g] = ((const float*)(smem + p.K))[g];
}

// Quantised input (Q8_0 codes of x for the Q8_0 and Q4_0 matvecs): thread t
// holds 16-value chunks t, t+256, ... (NC of them); lanes of one group
// (lpg = gs/16) are adjacent. Codes go to LDS at input_chunk_slot, scales in
// plain order after them, and for Q4_0 then -8 x each group's code sum.
// NC == 0: the input is too long to hold; it is loaded in batches after the
// weight prefetch instead.
template <int DT, int PRO, int NC>
struct InputQ8 {
    static constexpr int N = NC > 0 ? NC : 1;
    // the RMSNorm gain is held across the weight prefetch only for one chunk
    // per thread; longer inputs load it in the prologue (registers)
    static constexpr bool kHoldGain = PRO == PRO_NORM && NC == 1;
    f32x4 x[N][4], g[N][4];

    __device__ __forceinline__ void fence()
    {
        if (NC == 0) return;
#pragma unroll
        for (int j = 0; j < N; j++)
#pragma unroll
            for (int k = 0; k < 4; k++) {
                hold(x[j][k]);
                if (kHoldGain) hold(g[j][k]);
            }
    }

    __device__ __forceinline__ void issue(const GemvParams& p)
    {
        if (NC == 0) return;
        const int64_t nq = p.K / 16;
#pragma unroll
        for (int j = 0; j < N; j++) {
            const int64_t c = imin((int64_t)j * kThreads + threadIdx.x, nq - 1);
#pragma unroll
            for (int k = 0; k < 4; k++) {
                x[j][k] = ld4(p.x + 16 * c + 4 * k);
                if (kHoldGain) g[j][k] = ld4(p.gain + 16 * c + 4 * k);
            }
        }
    }

    __device__ __forceinline__ void store(const GemvParams& p, unsigned char* smem, int64_t c,
                                          const float* v, int lpg)
    {
        float sc;
        const i32x4 codes = quant16(v, lpg, &sc);
        int csum = 0;
        if (DT == DT_Q4) csum = lanes_sum_i32(dot16_i8(codes, i32x4{0x01010101, 0x01010101, 0x01010101,
                                                                 0x01010101}), lpg);
        if (c < p.K / 16) {
            ((i32x4*)smem)[input_chunk_slot<DT>(c, p.K, p.gs)] = codes;
            if ((c & (lpg - 1)) == 0) {
                ((float*)(smem + p.K))[c / lpg] = sc;
                if (DT == DT_Q4) ((int*)(smem + p.K))[p.K / p.gs + c / lpg] = -8 * csum;
            }
        }
    }

    __device__ __forceinline__ void finish(const GemvParams& p, unsigned char* smem, double* red, int bid)
    {
        const int64_t nq = p.K / 16;
        const int lpg = p.gs / 16;
        if (NC > 0) {
            if (PRO == PRO_NORM && !kHoldGain) {
#pragma unroll
                for (int j = 0; j < N; j++) {
                    const int64_t c = imin((int64_t)j * kThreads + threadIdx.x, nq - 1);
#pragma unroll
                    for (int k = 0; k < 4; k++) g[j][k] = ld4(p.gain + 16 * c + 4 * k);
                }
            }
            double r = 1.0;
            if (PRO == PRO_NORM) {
                double ss = 0.0;
#pragma unroll
                for (int j = 0; j < N; j++) {
                    const bool ok = (int64_t)j * kThreads + threadIdx.x < nq;
                    double s = 0.0;
#pragma unroll
                    for (int k = 0; k < 4; k++)
                        s += (double)x[j][k].x * (double)x[j][k].x + (double)x[j][k].y * (double)x[j][k].y +
                             (double)x[j][k].z * (double)x[j][k].z + (double)x[j][k].w * (double)x[j][k].w;
                    ss += ok ? s : 0.0;
                }
                ss = block_sum(ss, red);
                r = 1.0 / sqrt(ss / (double)p.K + p.eps);
            }
#pragma unroll
            for (int j = 0; j < N; j++) {
                if ((int64_t)j * kThreads < nq) {  // uniform
                    float v[16];
                    unpack16(v, x[j][0], x[j][1], x[j][2], x[j][3]);
                    if (PRO == PRO_NORM) {
                        float gg[16];
                        unpack16(gg, g[j][0], g[j][1], g[j][2], g[j][3]);
#pragma unroll
                        for (int i = 0; i < 16; i++) v[i] = (float)((double)gg[i] * ((double)v[i] * r));
                    }
                    store(p, smem, (int64_t)j * kThreads + threadIdx.x, v, lpg);
                }
            }
        } else {
            // long plain inputs: batches of 4 chunks per thread
            for (int64_t base = 0; base < nq; base += 4 * kThreads) {
                f32x4 a[4][4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int64_t c = imin(base + (int64_t)j * kThreads + threadIdx.x, nq - 1);
#pragma unroll
                    for (int k = 0; k < 4; k++) a[j][k] = ld4(p.x + 16 * c + 4 * k);
                }
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    if (base + (int64_t)j * kThreads < nq) {  // uniform
                        float v[16];
                        unpack16(v, a[j][0], a[j][1], a[j][2], a[j][3]);
                        store(p, smem, base + (int64_t)j * kThreads + threadIdx.x, v, lpg);
                    }
                }
            }
        }
        __syncthreads();
        trace_input<DT>(p, smem, bid);
    }
};

// Already quantised input (PRO_CODES: Q8_0 codes and scales of x, written by
// the producing kernel): the same LDS image as InputQ8 builds, without the
// per-workgroup quantisation. Thread t holds 16-code chunks t, t+256, ...
// PAD: the chained launch's layout (one group per 128-byte line, gs 64)
template <int DT, int NC, bool PAD>
struct InputCodes {
    static constexpr int N = NC > 0 ? NC : 1;
    i32x4 c[N];
    float sc[N];

    __device__ __forceinline__ void fence()
    {
        if (NC == 0) return;
#pragma unroll
        for (int j = 0; j < N; j++) {
            hold(c[j]);
            hold(sc[j]);
        }
    }

    __device__ __forceinline__ void issue(const GemvParams& p)
    {
        if (NC == 0) return;
        const int64_t nq = p.K / 16;
        const int lpg = p.gs / 16;
#pragma unroll
        for (int j = 0; j < N; j++) {
            const int64_t k = imin((int64_t)j * kThreads + threadIdx.x, nq - 1);
            c[j] = PAD ? *(const i32x4*)chain_codes(p.xq, k, lpg) : *(const i32x4*)(p.xq + 16 * k);
            sc[j] = PAD ? *chain_scale(p.xq, k / lpg) : p.xs[k / lpg];
        }
    }

    __device__ __forceinline__ void put(const GemvParams& p, unsigned char* smem, int64_t k, i32x4 codes,
                                        float scale, int lpg)
    {
        int csum = 0;
        if (DT == DT_Q4) csum = lanes_sum_i32(dot16_i8(codes, i32x4{0x01010101, 0x01010101, 0x01010101,
                                                                 0x01010101}), lpg);
        if (k < p.K / 16) {
            ((i32x4*)smem)[input_chunk_slot<DT>(k, p.K, p.gs)] = codes;
            if ((k & (lpg - 1)) == 0) {
                ((float*)(smem + p.K))[k / lpg] = scale;
                if (DT == DT_Q4) ((int*)(smem + p.K))[p.K / p.gs + k / lpg] = -8 * csum;
            }
        }
    }

    __device__ __forceinline__ void finish(const GemvParams& p, unsigned char* smem, double*, int bid)
    {
        const int64_t nq = p.K / 16;
        const int lpg = p.gs / 16;
        if (NC > 0) {
#pragma unroll
            for (int j = 0; j < N; j++)
                if ((int64_t)j * kThreads < nq) put(p, smem, (int64_t)j * kThreads + threadIdx.x, c[j], sc[j], lpg);
        } else {
            for (int64_t base = 0; base < nq; base += 4 * kThreads) {
                i32x4 a[4];
                float b[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int64_t k = imin(base + (int64_t)j * kThreads + threadIdx.x, nq - 1);
                    a[j] = PAD ? *(const i32x4*)chain_codes(p.xq, k, lpg) : *(const i32x4*)(p.xq + 16 * k);
                    b[j] = PAD ? *chain_scale(p.xq, k / lpg) : p.xs[k / lpg];
                }
#pragma unroll
                for (int j = 0; j < 4; j++)
                    if (base + (int64_t)j * kThreads < nq) put(p, smem, base + (int64_t)j * kThreads + threadIdx.x, a[j], b[j], lpg);
            }
        }
        __syncthreads();
        trace_input<DT>(p, smem, bid);
    }
};

// ---------------------------------------------------------------- epilogue

// What the epilogue needs besides the row sums, gathered without global
// loads on the critical path: pos (read once per kernel), the residual values
// of the tile's rows (loaded with the tile's weight chunks) and the RoPE
// cos/sin table of this pos (built in LDS by the prologue).
struct EpiIn {
    int pos;
    const float* res;    // [rpw] residual stream values of the tile's rows
    const float* rcos;   // [hs/2] fp32 cosines of pos * freq_j
    const float* rsin;   // [hs/2] fp32 sines
    double temp;         // EPI_LOGITS: sampling temperature (0: argmax)
    uint64_t seed;       // EPI_LOGITS: sampling seed
};

template <int EPI>
__device__ __forceinline__ void gemv_epilogue(const GemvParams& p, int64_t row0, int rpw,
                                              const double* acc, unsigned long long& best,
                                              const EpiIn& in)
{
    if (EPI == EPI_STORE) {
        for (int r = 0; r < rpw; r++)
            if (row0 + r < p.M) p.out[row0 + r] = (float)acc[r];
    } else if (EPI == EPI_RESID) {
        for (int r = 0; r < rpw; r++) {
            const int64_t row = row0 + r;
            if (row < p.M) {
                const float y = (float)acc[r];
                p.out[row] = (float)((double)in.res[r] + (double)y);
            }
        }
    } else if (EPI == EPI_LOGITS) {
        for (int r = 0; r < rpw; r++) {
            const int64_t row = row0 + r;
            if (row < p.M) {
                const float y = (float)acc[r];
                p.out[row] = y;
                const float kv = sample_key(y, in.temp, in.seed, in.pos, p.M, row);
                const unsigned long long key = argmax_pack(kv, (uint32_t)row);
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
                // device scope: the wave completing a group reads it back
                st_dev(p.out + row / 2, (float)(silu * h3));
            }
        }
    } else if (EPI == EPI_QKV) {
        // rows [0, d) q, [d, d+kvd) k, [d+kvd, d+2kvd) v; pairs (2j, 2j+1)
        // of each q/k head rotate by pos * freq_j (RoPE, computed on the fly)
        const int pos = in.pos;
        for (int r = 0; r + 1 < rpw; r += 2) {
            const int64_t row = row0 + r;
            if (row + 1 >= p.M) continue;
            const float a = (float)acc[r], b = (float)acc[r + 1];
            if (row < p.d + p.kvd) {
                const int64_t within = row < p.d ? row : row - p.d;
                const int j = (int)((within % p.hs) / 2);
                const double c = (double)in.rcos[j];
                const double s = (double)in.rsin[j];
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

// One chunk of a tile.
//   fp32: U loads of 16 bytes per lane for each of RPW rows (64*U float4
//         columns of each row).
//   Q8_0: one block of 64 groups of each of RPW rows in the permuted layout:
//         lane j holds group j of the block, U = gs/16 loads of 16 bytes,
//         plus that group's weight scale.
//   Q4_0: 64*U groups of each of RPW rows: lane j holds groups j, j+64, ...
//         (one 16-byte load each) and their weight scales.
template <int DT, int RPW, int U>
struct Chunk {
    static constexpr int SU = DT == DT_Q4 ? U : 1;
    using V = typename std::conditional<DT == DT_F32, f32x4, i32x4>::type;
    V w[RPW][U];
    float s[RPW][SU];
    float res[RPW];  // residual values of the rows (EPI_RESID)
};

// Loads of one chunk; rows, columns and lanes past the end are clamped onto
// valid addresses (use_chunk masks them), so the sequence never branches.
// A "dummy" chunk (past the wave's last tile: the ring's refills at the end)
// reads the first 16 bytes of the input vector instead, a cache-resident
// address, so it costs no HBM traffic and returns quickly. DW: the first
// bytes of the weights and scales instead (the input vector of a chained
// launch's second phase is not final until its wait ends, and no line of it
// may be loaded into L2 before then).
template <int DT, int EPI, int RPW, int U, bool DW>
__device__ __forceinline__ void load_chunk(Chunk<DT, RPW, U>& ch, const GemvParams& p, int64_t row0,
                                           int64_t chunk, int lane, bool dummy)
{
    const int64_t keep = dummy ? 0 : 1;  // multiplies every offset
    const void* dx = DW ? p.W : (const void*)p.x;
    const float* dxs = DW ? (p.Ws != nullptr ? p.Ws : (const float*)p.W) : p.x;
    if (EPI == EPI_RESID) {
#pragma unroll
        for (int r = 0; r < RPW; r++) ch.res[r] = p.out[imin(row0 + r, p.M - 1) * keep];
    }
    if constexpr (DT == DT_F32) {
        const int64_t Kv = p.K / 4;
        const f32x4* base = dummy ? (const f32x4*)dx : (const f32x4*)p.W;
#pragma unroll
        for (int uu = 0; uu < U; uu++) {
            const int64_t c = imin(chunk * kWave * U + uu * kWave + lane, Kv - 1);
#pragma unroll
            for (int r = 0; r < RPW; r++)
                ch.w[r][uu] = __builtin_nontemporal_load(base + (imin(row0 + r, p.M - 1) * Kv + c) * keep);
        }
    } else if constexpr (DT == DT_Q8) {
        const int64_t ng = p.K / p.gs;
        const int64_t g0 = chunk * 64;
        const int64_t nb = imin(ng - g0, 64);
        const int64_t j = imin(lane, nb - 1);
        const int8_t* base = dummy ? (const int8_t*)dx : (const int8_t*)p.W;
        const float* sbase = dummy ? dxs : p.Ws;
#pragma unroll
        for (int r = 0; r < RPW; r++) {
            const int64_t row = imin(row0 + r, p.M - 1);
            const i32x4* W = (const i32x4*)(base + (row * p.K + g0 * p.gs) * keep);
#pragma unroll
            for (int q = 0; q < U; q++) ch.w[r][q] = __builtin_nontemporal_load(W + (nb * q + j) * keep);
            ch.s[r][0] = sbase[(row * ng + g0 + j) * keep];
        }
    } else {
        const int64_t ng = p.K / 32;
        const i32x4* base = dummy ? (const i32x4*)dx : (const i32x4*)p.W;
        const float* sbase = dummy ? dxs : p.Ws;
#pragma unroll
        for (int r = 0; r < RPW; r++) {
            const int64_t rg = imin(row0 + r, p.M - 1) * ng;
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t g = imin(chunk * kWave * U + u * kWave + lane, ng - 1);
                ch.w[r][u] = __builtin_nontemporal_load(base + (rg + g) * keep);
                ch.s[r][u] = sbase[(rg + g) * keep];
            }
        }
    }
}

template <int DT, int RPW, int U, bool DBG>
__device__ __forceinline__ void use_chunk(const Chunk<DT, RPW, U>& ch, double* acc,
                                          const GemvParams& p, const unsigned char* smem,
                                          int64_t row0, int64_t chunk, int lane, bool valid)
{
    if constexpr (DT == DT_F32) {
        const int64_t Kv = p.K / 4;
#pragma unroll
        for (int uu = 0; uu < U; uu++) {
            const int64_t c = chunk * kWave * U + uu * kWave + lane;
            const f32x4 xl = ((const f32x4*)smem)[imin(c, Kv - 1)];
            const bool ok = valid && c < Kv;
            const f32x4 xv = ok ? xl : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                const f32x4 w = ch.w[r][uu];
                acc[r] += (double)w.x * (double)xv.x;
                acc[r] += (double)w.y * (double)xv.y;
                acc[r] += (double)w.z * (double)xv.z;
                acc[r] += (double)w.w * (double)xv.w;
            }
        }
    } else if constexpr (DT == DT_Q8) {
        const int64_t ng = p.K / p.gs;
        const int64_t g0 = chunk * 64;
        const int64_t nb = imin(ng - g0, 64);
        const int64_t j = imin(lane, nb - 1);
        const bool ok = valid && lane < nb;
        const i32x4* xq = (const i32x4*)(smem + g0 * p.gs);
        i32x4 xv[U];
#pragma unroll
        for (int q = 0; q < U; q++) xv[q] = xq[nb * q + j];
        const double xsg = (double)((const float*)(smem + p.K))[g0 + j];
#pragma unroll
        for (int r = 0; r < RPW; r++) {
            int d = 0;
#pragma unroll
            for (int q = 0; q < U; q++) {
                d = dot4_i8(ch.w[r][q].x, xv[q].x, d);
                d = dot4_i8(ch.w[r][q].y, xv[q].y, d);
                d = dot4_i8(ch.w[r][q].z, xv[q].z, d);
                d = dot4_i8(ch.w[r][q].w, xv[q].w, d);
            }
            const double t = ((double)d * (double)ch.s[r][0]) * xsg;
            acc[r] += ok ? t : 0.0;
            if (DBG && ok && row0 + r < p.M) p.group_dots[(row0 + r) * ng + g0 + lane] = d;
        }
    } else {
        // byte b of a group: code b + 8 in the low nibble, code b + 16 + 8
        // in the high nibble
        constexpr int kLo = 0x0F0F0F0F;
        const int64_t ng = p.K / 32;
        const i32x4* xlo = (const i32x4*)smem;  // codes 0-15 of every group
        const i32x4* xhi = xlo + ng;            // codes 16-31
        const float* xs = (const float*)(smem + p.K);
        const int* xoff = (const int*)(xs + ng);
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t g = chunk * kWave * U + u * kWave + lane;
            const bool ok = valid && g < ng;
            const int64_t gc = imin(g, ng - 1);
            const i32x4 a = xlo[gc], b = xhi[gc];
            const double xsg = (double)xs[gc];
            const int off = xoff[gc];
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                const i32x4 w = ch.w[r][u];
                int d = off;
                d = dot4_i8(w.x & kLo, a.x, d);
                d = dot4_i8(w.y & kLo, a.y, d);
                d = dot4_i8(w.z & kLo, a.z, d);
                d = dot4_i8(w.w & kLo, a.w, d);
                d = dot4_i8((int)((uint32_t)w.x >> 4) & kLo, b.x, d);
                d = dot4_i8((int)((uint32_t)w.y >> 4) & kLo, b.y, d);
                d = dot4_i8((int)((uint32_t)w.z >> 4) & kLo, b.z, d);
                d = dot4_i8((int)((uint32_t)w.w >> 4) & kLo, b.w, d);
                const double t = ((double)d * (double)ch.s[r][u]) * xsg;
                acc[r] += ok ? t : 0.0;
                if (DBG && ok && row0 + r < p.M) p.group_dots[(row0 + r) * ng + g] = d;
            }
        }
    }
}

// ---------------------------------------------------------------- chaining

// Role of a matvec in a chained launch: two phases of a layer in one launch,
// the second phase's workgroups after the first's in the grid. Workgroups
// are dispatched in grid order on each XCD, so every workgroup of the first
// phase has started (and, never waiting itself, will finish) before a
// second-phase workgroup can take its place; the second phase's waits
// therefore always end.
//   CH_NONE  a launch of its own;
//   CH_WAIT  second phase: the weight prefetch goes out first, then the
//            workgroup waits until every producer flag holds this launch's
//            epoch, and only then loads the input vector (plain loads: every
//            128-byte line of it has one writer, which stored it at device
//            scope before setting its flag, and no earlier load of the
//            launch brought the line into this XCD's L2);
//   CH_PUB   first phase of the FFN launch (w1/w3): each Q8_0 group of its
//            output is quantised as in CH_NONE, the codes and scale stored at
//            device scope into the group's own 128-byte line (kChainLine),
//            and then the group's flag is set.
enum { CH_NONE = 0, CH_WAIT = 1, CH_PUB = 2 };

// polls of the producer flags before a wait gives up
constexpr uint32_t kChainSpin = 1u << 18;

// The epoch of this launch of layer c.layer's chained kernel: the step
// serial (advanced by every step-start kernel) times the layer count, plus
// the layer, plus one; distinct for every launch of one layer's kernel
// until the serial wraps, and never the flags' initial 0 before that.
__device__ __forceinline__ uint32_t chain_epoch(const int32_t* step, const ChainArgs& c)
{
    return (uint32_t)step[kStepSerial] * (uint32_t)c.nlayers + (uint32_t)c.layer + 1u;
}

// Wait until every producer flag c.flags[0, c.nflags) holds epoch, then all
// waves of the workgroup meet at a barrier. Only the first workgroup of the
// second phase (bid 0) polls the flags (wave 0, a lane per flag); it then
// sets the go word *c.go to epoch, which every workgroup of the phase polls
// with one lane. (With every workgroup polling every flag, the polls to
// those few lines at the device coherence point slowed the first phase's
// own device-scope traffic.) The wait is bounded: after kChainSpin polls,
// or once another wait has given up (*c.err set), it sets *c.err and
// returns; the host then reports the step invalid.
__device__ __forceinline__ bool chain_poll_err(const ChainArgs& c, uint32_t it)
{
    if (it >= kChainSpin || ((it & 63) == 0 && ld_dev(c.err) != 0u)) {
        st_dev(c.err, 1u);
        return true;
    }
    return false;
}

__device__ __forceinline__ void chain_wait(const ChainArgs& c, uint32_t epoch, int bid)
{
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        bool failed = false;
        if (bid == 0) {
            for (uint32_t it = 0;; it++) {
                bool ok = true;
                for (int i = lane; i < c.nflags; i += kWave) ok = ok && ld_dev(c.flags + i) == epoch;
                if (__all(ok)) break;
                if (chain_poll_err(c, it)) {
                    failed = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            if (lane == 0 && !failed) st_dev(c.go, epoch);
        } else if (lane == 0) {
            for (uint32_t it = 0; ld_dev(c.go) != epoch; it++) {
                if (chain_poll_err(c, it)) break;
                __builtin_amdgcn_s_sleep(4);
            }
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------- matvec

// One workgroup's share of a matvec: workgroup bid of nblk (blockIdx.x of
// gridDim.x when the matvec has a launch of its own).
template <int DT, int PRO, int EPI, int RPW, int U, int NC, int NBUF, bool DBG, int CH>
__device__ __forceinline__ void gemv_body(const GemvParams& p, int bid, int nblk, const ChainArgs& chain)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ double red[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // chunks per tile: 64*U float4 columns (fp32), 64 groups (Q8_0) or
    // 64*U groups (Q4_0)
    const int64_t nch = DT == DT_F32 ? (p.K / 4 + kWave * U - 1) / (kWave * U)
                      : DT == DT_Q8  ? (p.K / p.gs + 63) / 64
                                     : (p.K / 32 + kWave * U - 1) / (kWave * U);
    // balanced contiguous range of tiles for this wave; one-row tiles that
    // feed a row-pair epilogue (RoPE, SwiGLU) are handed out in pairs, and
    // the even row's sum waits in a register for the odd row's
    constexpr bool PAIR1 = RPW == 1 && (EPI == EPI_QKV || EPI == EPI_SWIGLU);
    const int64_t tiles = (p.M + RPW - 1) / RPW;
    const int64_t units = PAIR1 ? tiles / 2 : tiles;
    const int64_t nw = (int64_t)nblk * kWaves;
    const int64_t gw = (int64_t)bid * kWaves + wave;
    const int64_t t_beg = (PAIR1 ? 2 : 1) * (units * gw / nw), t_end = (PAIR1 ? 2 : 1) * (units * (gw + 1) / nw);
    const int64_t iters = (t_end - t_beg) * nch;
    const int pos = (EPI == EPI_QKV || EPI == EPI_LOGITS) ? p.step[kStepPos] : 0;
    uint64_t seed = 0;
    double temp = 0.0;
    if (EPI == EPI_LOGITS) {
        seed = *(const uint64_t*)(p.step + kStepSeed);
        temp = *(const double*)(p.step + kStepTemp);
    }

    // 1. input loads (CH_WAIT: after the wait, below)
    typename std::conditional<PRO == PRO_CODES, InputCodes<DT, NC, CH == CH_WAIT>,
        typename std::conditional<DT == DT_F32, InputF32<PRO, NC>, InputQ8<DT, PRO, NC>>::type>::type in;
    if constexpr (CH != CH_WAIT) in.issue(p);
    // this step's RoPE cos / sin of this thread's pair (q/k/v epilogue),
    // made once per step by the step-start kernel
    float rc = 0.0f, rs = 0.0f;
    if (EPI == EPI_QKV && (int)threadIdx.x < p.hs / 2) {
        rc = p.rope[threadIdx.x];
        rs = p.rope[p.hs / 2 + threadIdx.x];
    }
    // keep every input load ahead of the weight prefetch: the prologue then
    // waits only for its own loads, not for the weights in flight behind them
    __builtin_amdgcn_sched_barrier(0);

    // 2. the first NBUF chunks (dummy loads for a wave with fewer chunks)
    Chunk<DT, RPW, U> buf[NBUF];
    int64_t ltile = t_beg, lch = 0;
    auto load_next = [&](Chunk<DT, RPW, U>& b) {
        load_chunk<DT, EPI, RPW, U, CH == CH_WAIT>(b, p, imin(ltile, tiles - 1) * RPW, lch, lane, ltile >= t_end);
        if (++lch == nch) {
            lch = 0;
            ++ltile;
        }
    };
#pragma unroll
    for (int k = 0; k < NBUF; k++) load_next(buf[k]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (CH == CH_WAIT) {
        // the weights are in flight; now wait for the input's producers
        chain_wait(chain, chain_epoch(p.step, chain), bid);
        in.issue(p);
    } else {
        in.fence();
    }
    hold(rc);
    hold(rs);

    // 3. prologue: this step's RoPE table into LDS, then the input vector
    float* rcos = (float*)(smem + gemv_input_bytes(DT, p.K, p.gs));
    float* rsin = rcos + p.hs / 2;
    if (EPI == EPI_QKV && (int)threadIdx.x < p.hs / 2) {
        rcos[threadIdx.x] = rc;
        rsin[threadIdx.x] = rs;
    }
    in.finish(p, smem, red, bid);

    // 4. main loop: every iteration consumes one buffer and refills it
    double acc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; r++) acc[r] = 0.0;
    unsigned long long best = 0;
    double pend = 0.0;  // PAIR1: the even row of the current pair
    int64_t tile = t_beg, ch = 0;
    for (int64_t it = 0; it < iters; it += NBUF) {
#pragma unroll
        for (int k = 0; k < NBUF; k++) {
            const bool valid = it + k < iters;
            use_chunk<DT, RPW, U, DBG>(buf[k], acc, p, smem, tile * RPW, ch, lane, valid);
            // refill the buffer as soon as its data is consumed: the tile's
            // reduction and epilogue then run with NBUF chunks in flight
            float res[RPW];
#pragma unroll
            for (int r = 0; r < RPW; r++) res[r] = EPI == EPI_RESID ? buf[k].res[r] : 0.0f;
            load_next(buf[k]);
            if (valid && ch == nch - 1) {
#pragma unroll
                for (int r = 0; r < RPW; r++) acc[r] = wave_sum_to_last(acc[r]);
                if (lane == kWave - 1) {
                    const EpiIn ein{pos, res, rcos, rsin, temp, seed};
                    if constexpr (PAIR1) {
                        if ((tile & 1) == 0) {
                            pend = acc[0];
                        } else {
                            const double pr[2] = {pend, acc[0]};
                            gemv_epilogue<EPI>(p, tile - 1, 2, pr, best, ein);
                        }
                    } else {
                        gemv_epilogue<EPI>(p, tile * RPW, RPW, acc, best, ein);
                    }
                }
#pragma unroll
                for (int r = 0; r < RPW; r++) acc[r] = 0.0;
            }
            if (++ch == nch) {
                ch = 0;
                ++tile;
            }
        }
    }
    if (EPI == EPI_SWIGLU && p.oq != nullptr) {
        // this wave stored outputs [rows / 2) of its tile range
        const int64_t r_lo = t_beg * RPW, r_hi = imin(t_end * RPW, p.M);
        if constexpr (CH == CH_PUB)
            quantize_completed_groups<true>(p.out, r_lo / 2, r_hi / 2, p.ogs, p.oq, nullptr, p.octr,
                                            kGroupCtrStride, lane, chain.pub, chain_epoch(p.step, chain));
        else
            quantize_completed_groups<false>(p.out, r_lo / 2, r_hi / 2, p.ogs, p.oq, p.os, p.octr,
                                             kGroupCtrStride, lane, nullptr, 0u);
    }
    if (EPI == EPI_LOGITS) {
        // workgroup maximum, then one atomic into a slot chosen by workgroup
        __shared__ unsigned long long wbest[kWaves];
        if (lane == kWave - 1) wbest[wave] = best;
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long b = wbest[0];
            for (int w = 1; w < kWaves; w++) b = wbest[w] > b ? wbest[w] : b;
            if (b != 0)
                atomicMax(p.argmax + ((size_t)(pos & 1) * kArgmaxSlots + bid % kArgmaxSlots) *
                                         kArgmaxStride,
                          b);
        }
    }
}

}  // namespace l2d
