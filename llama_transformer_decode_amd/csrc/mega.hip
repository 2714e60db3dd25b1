// mega.hip - the whole decode step as one persistent kernel.
//
// One workgroup of 512 threads per CU, launched cooperatively so that all of
// them are resident; the step's phases (the toy forward pass of the mht18
// essay, section 2.3, per layer: RMSNorm + q/k/v matvec + RoPE + cache write,
// attention, output matvec + residual, RMSNorm + w1/w3 matvec + SwiGLU, w2
// matvec + residual; then final RMSNorm + classifier + argmax) run back to
// back, separated by grid barriers instead of kernel boundaries.
//
// Matvec phases: the rows are split in tiles of two rows; each workgroup owns
// a contiguous range of tiles and its eight waves claim tiles from that range
// through an LDS counter, so a wave that gets its data sooner takes more
// tiles. A wave keeps two chunks of weights in flight (16 KiB). The first two
// chunks of the next phase are issued before the barrier that ends the
// current one: weights do not depend on the barrier, so HBM keeps streaming
// while the grid synchronises.
//
// Grid barrier: a workgroup arrives (its stores complete, then one atomic add
// on its XCD's counter), issues its prefetch, then waits until the eight
// counters reach their targets (one load per poll). The wait gives up after
// a bounded number of polls and sets an error word, so every wave ends.
//
// Values passed between workgroups within the launch (activations, the new
// cache row, attention partials) are written and read with device-scope
// accesses (ld_dev / st_dev), which do not go through a stale per-XCD cache.
//
// Attention: work items are (kv head, position range); each item writes its
// unnormalised partial result, and the last range of a kv head to finish
// (atomic count) merges them (o = sum_c e^{m_c - M} acc_c / sum_c e^{m_c - M} l_c).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn_core.hpp"
#include "device.hpp"
#include "internal.hpp"

namespace l2d {

constexpr int kMT = 512;               // threads per workgroup
constexpr int kMW = kMT / kWave;       // waves per workgroup
constexpr uint32_t kSpinLimit = 1u << 22;

// ---------------------------------------------------------------- grid barrier

__device__ __forceinline__ void grid_arrive(MegaSync* s)
{
    wait_vm_all();  // this wave's stores have reached the coherence point
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(&s->arrive[blockIdx.x & 7][0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// true when every workgroup has arrived `epoch` times in total; false after
// the poll limit or when another workgroup gave up
__device__ __forceinline__ bool grid_wait(MegaSync* s, uint32_t epoch)
{
    __shared__ int ok;
    if (threadIdx.x < kWave) {
        const int y = threadIdx.x & 7;
        const uint32_t members = (uint32_t)(((int)gridDim.x - y + 7) / 8);
        const uint32_t target = epoch * members;
        uint32_t n = 0;
        bool good = true;
        while (true) {
            const uint32_t c = ld_dev(&s->arrive[y][0]);
            if (__all(c >= target)) break;
            if (++n > kSpinLimit || ld_dev(&s->err[0]) != 0u) {
                good = false;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (threadIdx.x == 0) {
            ok = good ? 1 : 0;
            if (!good) st_dev(&s->err[0], 1u);
        }
    }
    __syncthreads();
    return ok != 0;
}

// ---------------------------------------------------------------- matvec phase

// One matvec of the step.
struct MV {
    const void* W;      // this layer's rows: fp32 [M][K] or group-interleaved int8 codes
    const float* Ws;    // Q8_0 scales [M][K/64]
    int64_t M, K;
    const float* x;     // input vector [K], written earlier in this launch
    const float* gain;  // RMSNorm gain [K], or nullptr
    float* out;
    int epi;
    float* kslot;       // EPI_QKV: this layer's cache rows at pos
    float* vslot;
};

__device__ __forceinline__ int64_t mmin(int64_t a, int64_t b) { return a < b ? a : b; }

template <int DT>
struct MvPhase {
    static constexpr int RPW = 2;  // rows per tile
    static constexpr int NB = 2;   // chunks in flight per wave
    static constexpr int U = 4;    // 16-byte loads per row per chunk
    using V = typename std::conditional<DT == DT_F32, f32x4, i32x4>::type;

    V w[NB][RPW][U];
    float s[NB][RPW];
    float res[NB][RPW];
    int btile[NB], bch[NB];
    bool bval[NB];
    int cur_tile, cur_ch, wg_beg, wg_end, tiles, nch;
    int* ctr;
    unsigned long long best;

    __device__ __forceinline__ void load(const MV& m, int k)
    {
        const int lane = threadIdx.x & 63;
        if (cur_ch == 0) {
            int t = 0;
            if (lane == 0) t = atomicAdd(ctr, 1);
            cur_tile = wg_beg + __builtin_amdgcn_readfirstlane(t);
        }
        const bool valid = cur_tile < wg_end;
        // past the range: read the first bytes of the input vector instead
        // (cache-resident, no HBM traffic); every load is issued regardless
        const int64_t keep = valid ? 1 : 0;
        const int64_t row0 = (int64_t)min(cur_tile, tiles - 1) * RPW;
        if (m.epi == EPI_RESID) {
#pragma unroll
            for (int r = 0; r < RPW; r++) res[k][r] = ld_dev(m.out + mmin(row0 + r, m.M - 1) * keep);
        }
        if constexpr (DT == DT_F32) {
            const int64_t Kv = m.K / 4;
            const f32x4* base = valid ? (const f32x4*)m.W : (const f32x4*)m.x;
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t c = mmin((int64_t)cur_ch * kWave * U + u * kWave + lane, Kv - 1);
#pragma unroll
                for (int r = 0; r < RPW; r++)
                    w[k][r][u] = __builtin_nontemporal_load(base + (mmin(row0 + r, m.M - 1) * Kv + c) * keep);
            }
        } else {
            const int64_t ng = m.K / 64, g0 = (int64_t)cur_ch * 64;
            const int64_t nb = mmin(ng - g0, 64), j = mmin(lane, nb - 1);
            const int8_t* base = valid ? (const int8_t*)m.W : (const int8_t*)m.x;
            const float* sbase = valid ? m.Ws : m.x;
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                const int64_t row = mmin(row0 + r, m.M - 1);
                const i32x4* Wp = (const i32x4*)(base + (row * m.K + g0 * 64) * keep);
#pragma unroll
                for (int q = 0; q < U; q++) w[k][r][q] = __builtin_nontemporal_load(Wp + (nb * q + j) * keep);
                s[k][r] = sbase[(row * ng + g0 + j) * keep];
            }
        }
        btile[k] = cur_tile;
        bch[k] = cur_ch;
        bval[k] = valid;
        if (++cur_ch == nch) cur_ch = 0;
    }

    // tile range of this workgroup, then the first NB chunks
    __device__ __forceinline__ void prefetch(const MV& m, int* counter)
    {
        ctr = counter;
        nch = DT == DT_F32 ? (int)((m.K / 4 + kWave * U - 1) / (kWave * U)) : (int)((m.K / 64 + 63) / 64);
        tiles = (int)((m.M + RPW - 1) / RPW);
        wg_beg = (int)((int64_t)tiles * blockIdx.x / gridDim.x);
        wg_end = (int)((int64_t)tiles * (blockIdx.x + 1) / gridDim.x);
        cur_tile = wg_beg;
        cur_ch = 0;
        best = 0;
        if (wg_beg == wg_end) return;  // no rows here: nothing to load
#pragma unroll
        for (int k = 0; k < NB; k++) load(m, k);
    }

    // input vector into LDS: fp32 (optionally RMSNorm'ed), or for Q8_0 its
    // group-interleaved codes followed by the group scales
    __device__ __forceinline__ void prologue(const MV& m, double eps, unsigned char* smem, double* red)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const bool norm = m.gain != nullptr;
        if constexpr (DT == DT_F32) {
            constexpr int NC = 8;  // K <= 16384
            const int64_t K4 = m.K / 4;
            const int nc = (int)((K4 + kMT - 1) / kMT);
            f32x4 xv[NC];
#pragma unroll
            for (int j = 0; j < NC; j++)
                if (j < nc) xv[j] = ld_dev4(m.x + 4 * mmin((int64_t)j * kMT + threadIdx.x, K4 - 1));
            double r = 1.0;
            if (norm) {
                double ss = 0.0;
#pragma unroll
                for (int j = 0; j < NC; j++) {
                    if (j < nc && (int64_t)j * kMT + threadIdx.x < K4) {
                        const f32x4 v = xv[j];
                        ss += (double)v.x * (double)v.x + (double)v.y * (double)v.y +
                              (double)v.z * (double)v.z + (double)v.w * (double)v.w;
                    }
                }
                ss = wave_sum(ss);
                if (lane == 0) red[wave] = ss;
                __syncthreads();
                ss = 0.0;
                for (int w8 = 0; w8 < kMW; w8++) ss += red[w8];
                r = 1.0 / sqrt(ss / (double)m.K + eps);
            }
            f32x4* xl = (f32x4*)smem;
#pragma unroll
            for (int j = 0; j < NC; j++) {
                const int64_t c = (int64_t)j * kMT + threadIdx.x;
                if (j < nc && c < K4) {
                    f32x4 o = xv[j];
                    if (norm) {
                        const f32x4 g = *(const f32x4*)(m.gain + 4 * c);
                        o.x = (float)((double)g.x * ((double)o.x * r));
                        o.y = (float)((double)g.y * ((double)o.y * r));
                        o.z = (float)((double)g.z * ((double)o.z * r));
                        o.w = (float)((double)g.w * ((double)o.w * r));
                    }
                    xl[c] = o;
                }
            }
        } else {
            constexpr int NC = 4;  // K <= 32768
            const int64_t nq = m.K / 16;
            const int nc = (int)((nq + kMT - 1) / kMT);
            f32x4 xv[NC][4];
#pragma unroll
            for (int j = 0; j < NC; j++) {
                if (j < nc) {
                    const int64_t c = mmin((int64_t)j * kMT + threadIdx.x, nq - 1);
#pragma unroll
                    for (int q = 0; q < 4; q++) xv[j][q] = ld_dev4(m.x + 16 * c + 4 * q);
                }
            }
            double r = 1.0;
            if (norm) {
                double ss = 0.0;
#pragma unroll
                for (int j = 0; j < NC; j++) {
                    if (j < nc && (int64_t)j * kMT + threadIdx.x < nq) {
#pragma unroll
                        for (int q = 0; q < 4; q++)
                            ss += (double)xv[j][q].x * (double)xv[j][q].x + (double)xv[j][q].y * (double)xv[j][q].y +
                                  (double)xv[j][q].z * (double)xv[j][q].z + (double)xv[j][q].w * (double)xv[j][q].w;
                    }
                }
                ss = wave_sum(ss);
                if (lane == 0) red[wave] = ss;
                __syncthreads();
                ss = 0.0;
                for (int w8 = 0; w8 < kMW; w8++) ss += red[w8];
                r = 1.0 / sqrt(ss / (double)m.K + eps);
            }
#pragma unroll
            for (int j = 0; j < NC; j++) {
                if (j >= nc) break;  // uniform
                const int64_t c = (int64_t)j * kMT + threadIdx.x;
                float v[16];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    v[4 * q] = xv[j][q].x;
                    v[4 * q + 1] = xv[j][q].y;
                    v[4 * q + 2] = xv[j][q].z;
                    v[4 * q + 3] = xv[j][q].w;
                }
                if (norm) {
                    const int64_t cc = mmin(c, nq - 1);
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const f32x4 g = *(const f32x4*)(m.gain + 16 * cc + 4 * q);
                        v[4 * q] = (float)((double)g.x * ((double)v[4 * q] * r));
                        v[4 * q + 1] = (float)((double)g.y * ((double)v[4 * q + 1] * r));
                        v[4 * q + 2] = (float)((double)g.z * ((double)v[4 * q + 2] * r));
                        v[4 * q + 3] = (float)((double)g.w * ((double)v[4 * q + 3] * r));
                    }
                }
                float sc;
                const i32x4 codes = quant16(v, 4, &sc);  // 4 lanes per group of 64
                if (c < nq) {
                    ((i32x4*)smem)[q8_perm_offset(16 * c, m.K, 64) / 16] = codes;
                    if ((c & 3) == 0) ((float*)(smem + m.K))[c / 4] = sc;
                }
            }
        }
        __syncthreads();
    }

    // finished row pair (rows row0, row0 + 1): y0, y1 in lane 63
    __device__ __forceinline__ void epilogue(const MV& m, const MegaParams& P, int k, int64_t row0, double y0,
                                             double y1, const float* rcos, const float* rsin)
    {
        switch (m.epi) {
        case EPI_RESID:
            if (row0 < m.M) st_dev(m.out + row0, (float)((double)res[k][0] + (double)(float)y0));
            if (row0 + 1 < m.M) st_dev(m.out + row0 + 1, (float)((double)res[k][1] + (double)(float)y1));
            break;
        case EPI_SWIGLU:
            if (row0 + 1 < m.M) {
                const double z = (double)(float)y0, h3 = (double)(float)y1;
                st_dev(m.out + row0 / 2, (float)(z / (1.0 + exp(-z)) * h3));
            }
            break;
        case EPI_QKV:
            if (row0 + 1 < m.M) {
                const float a = (float)y0, b = (float)y1;
                if (row0 < (int64_t)P.d + P.kvd) {
                    const int64_t within = row0 < P.d ? row0 : row0 - P.d;
                    const int j = (int)((within % P.hs) / 2);
                    const double c = (double)rcos[j], sn = (double)rsin[j];
                    const float ra = (float)((double)a * c - (double)b * sn);
                    const float rb = (float)((double)a * sn + (double)b * c);
                    float* dst = row0 < P.d ? m.out + row0 : m.kslot + within;
                    st_dev(dst, ra);
                    st_dev(dst + 1, rb);
                } else {
                    float* dst = m.vslot + (row0 - P.d - P.kvd);
                    st_dev(dst, a);
                    st_dev(dst + 1, b);
                }
            }
            break;
        case EPI_LOGITS:
            if (row0 < m.M) {
                const float v = (float)y0;
                m.out[row0] = v;
                const float kv = sample_key(v, P.temperature, P.seed, P.pos, m.M, row0);
                const unsigned long long key = argmax_pack(kv, (uint32_t)row0);
                best = key > best ? key : best;
            }
            if (row0 + 1 < m.M) {
                const float v = (float)y1;
                m.out[row0 + 1] = v;
                const float kv = sample_key(v, P.temperature, P.seed, P.pos, m.M, row0 + 1);
                const unsigned long long key = argmax_pack(kv, (uint32_t)(row0 + 1));
                best = key > best ? key : best;
            }
            break;
        default:
            break;
        }
    }

    // prologue, then consume the chunks (claiming and refilling) until this
    // wave's claims run past the workgroup's range
    __device__ __forceinline__ void run(const MV& m, const MegaParams& P, int* other_counter, unsigned char* smem,
                                        double* red, const float* rcos, const float* rsin)
    {
        if (threadIdx.x == 0) *other_counter = 0;  // the next phase's claims start from zero
        if (wg_beg == wg_end) return;               // uniform: no rows in this workgroup
        prologue(m, P.eps, smem, red);
        const int lane = threadIdx.x & 63;
        double acc[RPW];
#pragma unroll
        for (int r = 0; r < RPW; r++) acc[r] = 0.0;
        bool done = false;
        while (!done) {
#pragma unroll
            for (int k = 0; k < NB; k++) {
                done = done || !bval[k];
                if (done) continue;
                const int ch = bch[k];
                if constexpr (DT == DT_F32) {
                    const int64_t Kv = m.K / 4;
#pragma unroll
                    for (int u = 0; u < U; u++) {
                        const int64_t c = (int64_t)ch * kWave * U + u * kWave + lane;
                        const f32x4 xl = ((const f32x4*)smem)[mmin(c, Kv - 1)];
                        const f32x4 xv = c < Kv ? xl : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int r = 0; r < RPW; r++) {
                            const f32x4 wv = w[k][r][u];
                            acc[r] += (double)wv.x * (double)xv.x;
                            acc[r] += (double)wv.y * (double)xv.y;
                            acc[r] += (double)wv.z * (double)xv.z;
                            acc[r] += (double)wv.w * (double)xv.w;
                        }
                    }
                } else {
                    const int64_t ng = m.K / 64, g0 = (int64_t)ch * 64;
                    const int64_t nb = mmin(ng - g0, 64), j = mmin(lane, nb - 1);
                    const bool ok = lane < nb;
                    const i32x4* xq = (const i32x4*)(smem + g0 * 64);
                    i32x4 xx[U];
#pragma unroll
                    for (int q = 0; q < U; q++) xx[q] = xq[nb * q + j];
                    const double xsg = (double)((const float*)(smem + m.K))[g0 + j];
#pragma unroll
                    for (int r = 0; r < RPW; r++) {
                        int d = 0;
#pragma unroll
                        for (int q = 0; q < U; q++) {
                            d = dot4_i8(w[k][r][q].x, xx[q].x, d);
                            d = dot4_i8(w[k][r][q].y, xx[q].y, d);
                            d = dot4_i8(w[k][r][q].z, xx[q].z, d);
                            d = dot4_i8(w[k][r][q].w, xx[q].w, d);
                        }
                        const double t = ((double)d * (double)s[k][r]) * xsg;
                        acc[r] += ok ? t : 0.0;
                    }
                }
                if (ch == nch - 1) {
#pragma unroll
                    for (int r = 0; r < RPW; r++) acc[r] = wave_sum_to_last(acc[r]);
                    if (lane == kWave - 1) epilogue(m, P, k, (int64_t)btile[k] * RPW, acc[0], acc[1], rcos, rsin);
#pragma unroll
                    for (int r = 0; r < RPW; r++) acc[r] = 0.0;
                }
                load(m, k);
            }
        }
    }
};

// ---------------------------------------------------------------- phases

__device__ __forceinline__ size_t mv_es(int dt) { return dt == DT_F32 ? 4 : 1; }

__device__ __forceinline__ MV mv_qkv(const MegaParams& P, int l)
{
    const int64_t n = (int64_t)P.d + 2 * P.kvd;
    MV m;
    m.W = (const uint8_t*)P.wqkv + (size_t)(l * n * P.d) * mv_es(P.dt);
    m.Ws = P.dt == DT_Q8 ? P.wqkv_s + (size_t)l * n * (P.d / 64) : nullptr;
    m.M = n;
    m.K = P.d;
    m.x = P.x;
    m.gain = P.rms_att + (size_t)l * P.d;
    m.out = P.q;
    m.epi = EPI_QKV;
    m.kslot = P.kc + ((size_t)l * P.S + P.pos) * P.kvd;
    m.vslot = P.vc + ((size_t)l * P.S + P.pos) * P.kvd;
    return m;
}

__device__ __forceinline__ MV mv_wo(const MegaParams& P, int l)
{
    MV m;
    m.W = (const uint8_t*)P.wo + (size_t)((int64_t)l * P.d * P.d) * mv_es(P.dt);
    m.Ws = P.dt == DT_Q8 ? P.wo_s + (size_t)l * P.d * (P.d / 64) : nullptr;
    m.M = P.d;
    m.K = P.d;
    m.x = P.o;
    m.gain = nullptr;
    m.out = P.x;
    m.epi = EPI_RESID;
    m.kslot = m.vslot = nullptr;
    return m;
}

__device__ __forceinline__ MV mv_w13(const MegaParams& P, int l)
{
    MV m;
    m.W = (const uint8_t*)P.w13 + (size_t)((int64_t)l * 2 * P.h * P.d) * mv_es(P.dt);
    m.Ws = P.dt == DT_Q8 ? P.w13_s + (size_t)l * 2 * P.h * (P.d / 64) : nullptr;
    m.M = 2 * (int64_t)P.h;
    m.K = P.d;
    m.x = P.x;
    m.gain = P.rms_ffn + (size_t)l * P.d;
    m.out = P.hb;
    m.epi = EPI_SWIGLU;
    m.kslot = m.vslot = nullptr;
    return m;
}

__device__ __forceinline__ MV mv_w2(const MegaParams& P, int l)
{
    MV m;
    m.W = (const uint8_t*)P.w2 + (size_t)((int64_t)l * P.d * P.h) * mv_es(P.dt);
    m.Ws = P.dt == DT_Q8 ? P.w2_s + (size_t)l * P.d * (P.h / 64) : nullptr;
    m.M = P.d;
    m.K = P.h;
    m.x = P.hb;
    m.gain = nullptr;
    m.out = P.x;
    m.epi = EPI_RESID;
    m.kslot = m.vslot = nullptr;
    return m;
}

__device__ __forceinline__ MV mv_cls(const MegaParams& P)
{
    MV m;
    m.W = P.wcls;
    m.Ws = P.dt == DT_Q8 ? P.wcls_s : nullptr;
    m.M = P.V;
    m.K = P.d;
    m.x = P.x;
    m.gain = P.rms_final;
    m.out = P.logits;
    m.epi = EPI_LOGITS;
    m.kslot = m.vslot = nullptr;
    return m;
}

// position ranges of the attention at T = pos + 1 cached positions
__device__ __forceinline__ int mega_ranges(int T, int nkv, int* per)
{
    int ns = (int)gridDim.x / nkv;
    ns = ns < 1 ? 1 : ns > kMegaSplits ? kMegaSplits : ns;
    int nact;
    *per = attn_split(T, ns, 16, &nact);
    return nact;
}

template <int KG>
__device__ __forceinline__ void attention_phase(const MegaParams& P, int l, unsigned char* smem)
{
    constexpr int G = KG;
    const int hs = P.hs, tid = threadIdx.x;
    const int T = P.pos + 1;
    int per;
    const int nact = mega_ranges(T, P.nkv, &per);
    __shared__ int last;
    for (int it = blockIdx.x; it < P.nkv * nact; it += gridDim.x) {
        const int g = it / nact, c = it % nact;
        AttnRange r;
        r.q = P.q + (size_t)g * G * hs;
        r.kc = P.kc + (size_t)l * P.S * P.kvd;
        r.vc = P.vc + (size_t)l * P.S * P.kvd;
        r.kvd = P.kvd;
        r.hs = hs;
        r.G = G;
        r.g = g;
        r.r0 = c * per;
        r.n = min(T - r.r0, per);
        r.fresh = P.pos;
        r.Gt = G;  // one query token: no causal mask within the range
        r.qstride = 0;
        r.last0 = 0x3fffffff;
        attn_range<KG, kMT>(r, smem);
        float* og = P.o + (size_t)g * G * hs;
        if (nact == 1) {
            for (int e = tid; e < G * hs; e += kMT)
                st_dev(og + e, (float)(attn_value<kMT>(smem, G, hs, e) / attn_l<kMT>(smem, G, hs, e / hs)));
            __syncthreads();  // LDS is reused by the next item
            continue;
        }
        const size_t base = (size_t)g * kMegaSplits;
        for (int e = tid; e < G * hs; e += kMT)
            st_dev(P.part_o + (base + c) * G * hs + e, attn_value<kMT>(smem, G, hs, e));
        if (tid < G) {
            st_dev(P.part_ml + ((base + c) * G + tid) * 2, attn_m<kMT>(smem, G, hs, tid));
            st_dev(P.part_ml + ((base + c) * G + tid) * 2 + 1, attn_l<kMT>(smem, G, hs, tid));
        }
        wait_vm_all();
        __syncthreads();
        if (tid == 0) {
            uint32_t* ctr = P.head_ctr + (size_t)g * 32;
            const uint32_t done = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = done + 1 == (uint32_t)nact;
            if (last) st_dev(ctr, 0u);  // next use is a later layer, after grid barriers
        }
        __syncthreads();
        if (last) {
            // every range of kv head g has stored its partials: merge in a fixed order
            for (int e = tid; e < G * hs; e += kMT) {
                const int h = e / hs;
                double M = -INFINITY;
                for (int cc = 0; cc < nact; cc++) M = fmax(M, ld_dev(P.part_ml + ((base + cc) * G + h) * 2));
                double O = 0.0, Ls = 0.0;
                for (int cc = 0; cc < nact; cc++) {
                    const double wgt = exp(ld_dev(P.part_ml + ((base + cc) * G + h) * 2) - M);
                    Ls += wgt * ld_dev(P.part_ml + ((base + cc) * G + h) * 2 + 1);
                    O += wgt * ld_dev(P.part_o + (base + cc) * G * hs + e);
                }
                st_dev(og + e, (float)(O / Ls));
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- the kernel

template <int DT, int KG>
__global__ __launch_bounds__(kMT, 1) void step_kernel(MegaParams P)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ double red[kMW];
    __shared__ int ctr[2];
    __shared__ float rcos[128], rsin[128];
    __shared__ unsigned long long wbest[kMW];
    __shared__ int tok_sh;
    MegaSync* S = P.sync;
    uint32_t ep = P.epoch0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int pos = P.pos;

    // ---- step start: token, RoPE table of pos, x = embedding row
    if (tid < 2) ctr[tid] = 0;
    if (tid < P.hs / 2) {
        // fp32 cosine / sine of the fp32 angle pos * freq_j, correctly rounded
        const float ang = (float)pos * P.freqs[tid];
        rcos[tid] = (float)cos((double)ang);
        rsin[tid] = (float)sin((double)ang);
    }
    if (wave == 0) {
        int token = P.token;
        if (P.greedy) {
            // argmax of the previous step: maximum over its slots
            const int qq = ((pos - 1) & 1) * kArgmaxSlots;
            unsigned long long v = lane < kArgmaxSlots ? ld_dev(P.argmax + (size_t)(qq + lane) * kArgmaxStride) : 0ull;
            for (int msk = 32; msk >= 1; msk >>= 1) {
                const unsigned long long o = __shfl_xor(v, msk, 64);
                v = o > v ? o : v;
            }
            token = (int)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull));
            if (token < 0 || token >= P.V) token = 0;
        }
        if (lane == 0) tok_sh = token;
    }
    __syncthreads();
    const int token = tok_sh;
    if (blockIdx.x == 0) {
        if (tid == 0) {
            st_dev(P.step + kStepToken, token);
            st_dev(P.step + kStepPos, pos);
            st_dev((unsigned long long*)(P.step + kStepSeed), (unsigned long long)P.seed);
            st_dev((unsigned long long*)(P.step + kStepTemp), (unsigned long long)__double_as_longlong(P.temperature));
        }
        if (tid < kArgmaxSlots) st_dev(P.argmax + ((size_t)(pos & 1) * kArgmaxSlots + tid) * kArgmaxStride, 0ull);
    }
    {
        const int64_t i0 = (int64_t)P.d * blockIdx.x / gridDim.x, i1 = (int64_t)P.d * (blockIdx.x + 1) / gridDim.x;
        for (int64_t i = i0 + tid; i < i1; i += kMT) {
            const int64_t off = (int64_t)token * P.d + i;
            float v;
            if (DT == DT_F32) {
                v = ((const float*)P.emb)[off];
            } else {
                const int8_t c = ((const int8_t*)P.emb)[(int64_t)token * P.d + q8_perm_offset(i, P.d, 64)];
                v = (float)((double)c * (double)P.emb_s[off / 64]);
            }
            st_dev(P.x + i, v);
        }
    }
    // phase sequence: per layer q/k/v, attention, output, w1/w3, w2; then
    // the classifier. One code path serves every matvec phase.
    enum { PH_QKV = 0, PH_ATTN, PH_WO, PH_W13, PH_W2, PH_PER_LAYER };
    const int nph = P.L * PH_PER_LAYER + 1;
    auto make_mv = [&](int i) -> MV {
        const int l = i / PH_PER_LAYER, k = i % PH_PER_LAYER;
        if (i == nph - 1) return mv_cls(P);
        if (k == PH_QKV) return mv_qkv(P, l);
        if (k == PH_WO) return mv_wo(P, l);
        if (k == PH_W13) return mv_w13(P, l);
        return mv_w2(P, l);
    };
    MvPhase<DT> ph;
    int cc = 0;  // LDS claim counter of the next matvec phase (alternates)
    grid_arrive(S);
    ph.prefetch(make_mv(0), &ctr[cc]);
    if (!grid_wait(S, ++ep)) return;
    for (int i = 0; i < nph; i++) {
        const bool attn = i % PH_PER_LAYER == PH_ATTN && i != nph - 1;
        if (attn) {
            attention_phase<KG>(P, i / PH_PER_LAYER, smem);
        } else {
            cc ^= 1;  // the next matvec phase claims from the other counter
            ph.run(make_mv(i), P, &ctr[cc], smem, red, rcos, rsin);
        }
        if (i == nph - 1) break;
        grid_arrive(S);
        // the next phase's first weight chunks (attention has no prefetch)
        if ((i + 1) % PH_PER_LAYER != PH_ATTN || i + 1 == nph - 1) ph.prefetch(make_mv(i + 1), &ctr[cc]);
        if (!grid_wait(S, ++ep)) return;
    }

    // classifier argmax: workgroup maximum, one atomic into a slot of this step's parity
    if (lane == kWave - 1) wbest[wave] = ph.best;
    __syncthreads();
    if (tid == 0) {
        unsigned long long b = wbest[0];
        for (int w8 = 1; w8 < kMW; w8++) b = wbest[w8] > b ? wbest[w8] : b;
        if (b != 0)
            atomicMax(P.argmax + ((size_t)(pos & 1) * kArgmaxSlots + blockIdx.x % kArgmaxSlots) * kArgmaxStride, b);
    }
}

// ---------------------------------------------------------------- host side

bool mega_supported(int dt, int gs, int64_t d, int64_t h, int G, int hs)
{
    if (dt != DT_F32 && dt != DT_Q8) return false;  // built for fp32 and Q8_0 only
    if (dt == DT_Q8 && gs != 64) return false;
    // matvec inputs held in registers by the prologue: 16 (fp32: 4) values
    // per thread in up to 4 (fp32: 8) batches
    const int64_t K = d > h ? d : h;
    if (K > (dt == DT_F32 ? 16384 : 32768)) return false;
    if (hs / 2 > 128) return false;
    return attn_core_supported<kMT>(G, hs);
}

size_t mega_lds_bytes(int dt, int64_t d, int64_t h, int G, int hs)
{
    const int64_t K = d > h ? d : h;
    size_t mv = dt == DT_F32 ? (size_t)K * 4 : (size_t)K + (size_t)(K / 64) * 4;
    mv = (mv + 15) & ~(size_t)15;
    const size_t at = attn_core_lds_bytes<kMT>(G, hs);
    return mv > at ? mv : at;
}

template <int DT>
static const void* kernel_for(int G)
{
    switch (G) {
    case 1: return (const void*)step_kernel<DT, 1>;
    case 2: return (const void*)step_kernel<DT, 2>;
    case 4: return (const void*)step_kernel<DT, 4>;
    case 8: return (const void*)step_kernel<DT, 8>;
    default: return nullptr;
    }
}

static const void* mega_kernel(int dt, int G) { return dt == DT_F32 ? kernel_for<DT_F32>(G) : kernel_for<DT_Q8>(G); }

int mega_blocks_per_cu(int dt, int G, size_t lds)
{
    const void* f = mega_kernel(dt, G);
    if (!f) return 0;
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kMT, lds) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}

hipError_t launch_mega(const MegaParams& p, int grid, size_t lds, hipStream_t s)
{
    const void* f = mega_kernel(p.dt, p.G);
    if (!f) return hipErrorInvalidValue;
    MegaParams arg = p;
    void* args[] = {&arg};
    return hipLaunchCooperativeKernel(f, dim3((unsigned)grid), dim3(kMT), args, (unsigned)lds, s);
}

}  // namespace l2d
