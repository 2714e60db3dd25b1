// device.hpp - wavefront-level helpers for gfx950 (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace l2d {

constexpr int kWave = 64;

// native clang vectors: 16-byte global loads (plain and nontemporal)
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// sum of an int over aligned groups of `width` lanes (width a power of two <= 64)
__device__ __forceinline__ int group_sum_i32(int v, int width)
{
    for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// dot of 4 int8 pairs packed in two 32-bit words, accumulated into c (v_dot4_i32_i8)
__device__ __forceinline__ int dot4_i8(int a, int b, int c)
{
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

__device__ __forceinline__ int dot16_i8(i32x4 a, i32x4 b)
{
    int p = dot4_i8(a.x, b.x, 0);
    p = dot4_i8(a.y, b.y, p);
    p = dot4_i8(a.z, b.z, p);
    p = dot4_i8(a.w, b.w, p);
    return p;
}

// Order-preserving map of a float onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// argmax candidate packed for a 64-bit atomicMax: high word the float key,
// low word the complement of the index, so equal values favour the lower index.
__device__ __forceinline__ unsigned long long argmax_pack(float v, uint32_t idx)
{
    return ((unsigned long long)float_key(v) << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

// Q8_0 quantisation of one group value: the group's scale is wmax / 127
// (IEEE fp32 division), the code is the fp32 quotient rounded half away from
// zero; a zero scale gives code 0.
__device__ __forceinline__ float q80_scale(float wmax) { return wmax / 127.0f; }

__device__ __forceinline__ int q80_code(float x, float scale)
{
    if (scale == 0.0f) return 0;
    return (int)roundf(x / scale);
}

}  // namespace l2d

namespace l2d {

// Wave-cooperative Q8_0 quantisation of groups of gs values (gs a power of
// two in [16, 1024]). A wave handles 64/min(gs,64) groups per iteration;
// iterations first_iter, first_iter + iter_stride, ... cover all ng groups.
// val(i) yields the fp32 value of element i. Codes go to q[i], scales to s[g].
template <class Val>
__device__ __forceinline__ void q80_groups_wave(Val val, int64_t ng, int gs, int64_t first_iter,
                                                int64_t iter_stride, int8_t* q, float* s,
                                                int lane)
{
    const int sw = gs < kWave ? gs : kWave;  // lanes per group
    const int gpw = kWave / sw;               // groups per wave iteration
    const int epl = gs / sw;                  // values per lane
    const int sub = lane % sw;
    for (int64_t it = first_iter; it * gpw < ng; it += iter_stride) {
        const int64_t g = it * gpw + lane / sw;
        const bool ok = g < ng;
        float m = 0.0f;
        if (ok)
            for (int k = 0; k < epl; k++) m = fmaxf(m, fabsf(val(g * gs + sub + k * sw)));
        for (int w = 1; w < sw; w <<= 1) m = fmaxf(m, __shfl_xor(m, w, kWave));
        const float sc = q80_scale(m);
        if (ok) {
            for (int k = 0; k < epl; k++) {
                const int64_t i = g * gs + sub + k * sw;
                q[i] = (int8_t)q80_code(val(i), sc);
            }
            if (sub == 0) s[g] = sc;
        }
    }
}

}  // namespace l2d

namespace l2d {

// Cross-lane moves with DPP quad permutations (VALU, no LDS traffic).
// quad_perm [1,0,3,2]: lane ^ 1; quad_perm [2,3,0,1]: lane ^ 2.
__device__ __forceinline__ int dpp_xor1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_xor2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); }

__device__ __forceinline__ float dpp_xor1f(float v) { return __int_as_float(dpp_xor1(__float_as_int(v))); }
__device__ __forceinline__ float dpp_xor2f(float v) { return __int_as_float(dpp_xor2(__float_as_int(v))); }
// row_half_mirror (lane j <-> 7 - j within 8 lanes) and row_mirror (j <-> 15
// - j within 16): once every lane of a quad (of a half-row) holds the same
// value, they pair it with the other quad (half-row) as xor 4 (xor 8) would
__device__ __forceinline__ int dpp_hmirror(int v) { return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_mirror(int v) { return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false); }

// sum of an int over aligned groups of `width` lanes (power of two <= 64);
// DPP up to 16 lanes, lane shuffles beyond
__device__ __forceinline__ int lanes_sum_i32(int v, int width)
{
    if (width >= 2) v += dpp_xor1(v);
    if (width >= 4) v += dpp_xor2(v);
    if (width >= 8) v += dpp_hmirror(v);
    if (width >= 16) v += dpp_mirror(v);
    for (int m = 16; m < width; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// max of a float over aligned groups of `width` lanes (power of two <= 64)
__device__ __forceinline__ float lanes_max_f32(float v, int width)
{
    if (width >= 2) v = fmaxf(v, dpp_xor1f(v));
    if (width >= 4) v = fmaxf(v, dpp_xor2f(v));
    if (width >= 8) v = fmaxf(v, __int_as_float(dpp_hmirror(__float_as_int(v))));
    if (width >= 16) v = fmaxf(v, __int_as_float(dpp_mirror(__float_as_int(v))));
    for (int m = 16; m < width; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

__device__ __forceinline__ int ilog2(int v) { return 31 - __builtin_clz(v); }

}  // namespace l2d

namespace l2d {

// DPP move of a double (two 32-bit halves); lanes of rows disabled by
// ROW_MASK receive 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROW_MASK, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROW_MASK, 0xF, false);
    return __hiloint2double(hi, lo);
}

// value of lane l of a double (uniform result)
__device__ __forceinline__ double readlane_f64(double v, int l)
{
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}

// fp64 sum over the 64 lanes of a wavefront; every lane gets the total. Fixed
// order, so the result is deterministic: within each row of 16 lanes quad xor
// 1, quad xor 2, half-row mirror, row mirror (DPP, a few cycles each), then the
// four row totals read from lanes 0, 16, 32, 48 and added as (r0 + r1) + (r2 +
// r3).
__device__ __forceinline__ double wave_sum(double v)
{
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// fp64 maximum over the 64 lanes (every lane gets it), the same steps
__device__ __forceinline__ double wave_max(double v)
{
    v = fmax(v, dpp_f64<0xB1>(v));
    v = fmax(v, dpp_f64<0x4E>(v));
    v = fmax(v, dpp_f64<0x141>(v));
    v = fmax(v, dpp_f64<0x140>(v));
    return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

// fp32 maximum over the 64 lanes (every lane gets it)
__device__ __forceinline__ float wave_maxf(float v)
{
    auto mv = [](float x, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
    };
    v = fmaxf(v, mv(v, std::integral_constant<int, 0xB1>()));
    v = fmaxf(v, mv(v, std::integral_constant<int, 0x4E>()));
    v = fmaxf(v, mv(v, std::integral_constant<int, 0x141>()));
    v = fmaxf(v, mv(v, std::integral_constant<int, 0x140>()));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// fp64 sum over the 64 lanes with DPP only (fixed order); the total lands in
// lane 63: quad xor 1, quad xor 2, half-row mirror, row mirror, then
// row_bcast:15 into rows 1 and 3 and row_bcast:31 into rows 2 and 3.
__device__ __forceinline__ double wave_sum_to_last(double v)
{
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    v += dpp_f64<0x142, 0xA>(v);
    v += dpp_f64<0x143, 0xC>(v);
    return v;
}

}  // namespace l2d

namespace l2d {

// Device layout of a Q8_0 row of K codes (group size gs, ng = K/gs groups):
// groups are taken 64 at a time ("blocks"; the last block may hold fewer,
// nb); within a block the 16-byte quarters of its groups are stored quarter
// by quarter: quarter q of group j of the block sits at
//     block_start + 16*nb*q + 16*j,   block_start = 64*gs*block.
// A wavefront reading quarter q of a block with lane j = group j loads 16*nb
// contiguous bytes, and each lane ends up with whole groups.
__host__ __device__ __forceinline__ int64_t q8_perm_offset(int64_t i, int64_t K, int gs)
{
    const int64_t ng = K / gs;
    const int64_t g = i / gs, w = i % gs;
    const int64_t blk = g / 64, j = g % 64;
    const int64_t nb = (ng - blk * 64) < 64 ? (ng - blk * 64) : 64;
    const int64_t q = w / 16, b = w % 16;
    return blk * 64 * gs + 16 * nb * q + 16 * j + b;
}

}  // namespace l2d

namespace l2d {

// Device-scope coherent accesses, for values that one workgroup writes and
// another reads within the same kernel launch (the step kernel's phases):
// relaxed atomics at agent scope, which gfx950 executes with the sc1 cache
// policy (stores reach the device coherence point before they complete,
// loads do not hit a stale copy in a per-XCD cache).
__device__ __forceinline__ float ld_dev(const float* p)
{
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ double ld_dev(const double* p)
{
    return __hip_atomic_load(const_cast<double*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p)
{
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long ld_dev(const unsigned long long* p)
{
    return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// four consecutive floats (16-byte aligned) as two 8-byte device-scope loads
__device__ __forceinline__ f32x4 ld_dev4(const float* p)
{
    unsigned long long* q = (unsigned long long*)const_cast<float*>(p);
    const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                 __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}

__device__ __forceinline__ void st_dev(float* p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_dev(double* p, double v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_dev(int32_t* p, int32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_dev(unsigned long long* p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// wait until every global memory access this wave issued has completed
// (stores acknowledged); also a compiler barrier for memory operations
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// quantise one 16-value chunk (this lane's part of a group of lpg adjacent
// lanes): the group's scale and the 16 codes packed 4 per word
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

// Q8_0 quantisation of a vector y that many waves produce, each wave a
// contiguous range, done once per group instead of by every consumer.

// One wave quantises group y[0, gs) (values read with device-scope loads):
// lane l takes elements l, l + 64, ...; codes to q[0, gs), the scale to *s.
// DEV: the codes and scale are stored at device scope (a reader in the same
// launch on another XCD), codes four to a 32-bit word (gs a multiple of 4);
// the caller lays the group out in a line of its own.
template <bool DEV>
__device__ __forceinline__ void quantize_group_wave(const float* y, int gs, int8_t* q, float* s, int lane)
{
    constexpr int kMaxPer = 4;  // gs <= 256
    float v[kMaxPer];
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxPer; k++) {
        const int i = lane + k * kWave;
        v[k] = i < gs ? ld_dev(y + i) : 0.0f;
        m = fmaxf(m, fabsf(v[k]));
    }
    m = wave_maxf(m);
    const float sc = q80_scale(m);
#pragma unroll
    for (int k = 0; k < kMaxPer; k++) {
        const int i = lane + k * kWave;
        if constexpr (DEV) {
            // lanes 4j .. 4j+3 hold elements 4j .. 4j+3 of this pass: OR
            // their bytes into one word, which lane 4j stores
            const int c = i < gs ? q80_code(v[k], sc) : 0;
            int w = (c & 0xFF) << (8 * (lane & 3));
            w |= dpp_xor1(w);
            w |= dpp_xor2(w);
            if ((lane & 3) == 0 && i < gs) st_dev((uint32_t*)(q + i), (uint32_t)w);
        } else {
            if (i < gs) q[i] = (int8_t)q80_code(v[k], sc);
        }
    }
    if (lane == 0) {
        if constexpr (DEV) st_dev(s, sc);
        else *s = sc;
    }
}

// Called by a whole wave after it has stored y[lo, hi) with device-scope
// stores. For every group of gs values it touched, it adds its count of
// elements to the group's counter (relaxed, device scope, after waiting for
// its stores to complete); the wave that brings a count to gs reads the
// group back, quantises it into q/s and resets the counter for the next
// use. A range holding a whole group quantises it without counting.
// Counter g sits at ctr[g * ctr_stride].
// PUB (a chained launch, whose second phase reads the codes): group g takes
// the 128-byte line q + 128 g (its gs <= 64 codes, then its scale at byte
// 64; s is unused), stored at device scope, and once they are complete the
// group's flag pub[g] is set to epoch.
template <bool PUB>
__device__ __forceinline__ void quantize_completed_groups(const float* y, int64_t lo, int64_t hi, int gs,
                                                          int8_t* q, float* s, uint32_t* ctr,
                                                          int ctr_stride, int lane, uint32_t* pub,
                                                          uint32_t epoch)
{
    if (lo >= hi) return;
    wait_vm_all();
    for (int64_t g = lo / gs; g * gs < hi; g++) {
        const int64_t a = lo > g * gs ? lo : g * gs;
        const int64_t b = hi < (g + 1) * gs ? hi : (g + 1) * gs;
        const uint32_t cnt = (uint32_t)(b - a);
        bool last = cnt == (uint32_t)gs;
        if (!last) {
            uint32_t old = 0;
            if (lane == 0)
                old = __hip_atomic_fetch_add(ctr + g * ctr_stride, cnt, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
            old = __shfl(old, 0, kWave);
            last = old + cnt == (uint32_t)gs;
            if (last && lane == 0) st_dev(ctr + g * ctr_stride, 0u);
        }
        if (last) {
            if constexpr (PUB)
                quantize_group_wave<true>(y + g * gs, gs, q + g * 128, (float*)(q + g * 128 + 64), lane);
            else
                quantize_group_wave<false>(y + g * gs, gs, q + g * gs, s + g, lane);
            if constexpr (PUB) {
                wait_vm_all();
                if (lane == 0) st_dev(pub + g, epoch);
            }
        }
    }
}

}  // namespace l2d

namespace l2d {

// Temperature sampling draws (mht18 essay, section 3.2: a random draw from
// the softmax of the logits, the temperature scaling them): output k of the
// splitmix64 stream seeded with seed (Steele, Lea, Flood 2014), mapped to a
// uniform on (0, 1) as ((bits >> 11) + 1/2) * 2^-53, and its standard Gumbel
// transform -log(-log(u)). argmax_i of logit_i / T + g_i is a draw from
// softmax(logit / T) (Gumbel-max rule).
__host__ __device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t k)
{
    uint64_t z = seed + k * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ double gumbel_at(uint64_t seed, uint64_t k)
{
    const double u = ((double)(splitmix64_at(seed, k) >> 11) + 0.5) * 0x1.0p-53;
    return -log(-log(u));
}

// the value the classifier's argmax compares for token `row` of `n` at
// position pos: the logit itself, or with temperature > 0 its Gumbel-max
// score logit / T + g, rounded to fp32
__device__ __forceinline__ float sample_key(float logit, double temperature, uint64_t seed, int pos, int64_t n,
                                            int64_t row)
{
    if (!(temperature > 0.0)) return logit;
    return (float)((double)logit / temperature + gumbel_at(seed, (uint64_t)pos * (uint64_t)n + (uint64_t)row + 1u));
}

}  // namespace l2d
