// step.hip - the first kernel of a decode step, and the standalone Q8_0
// quantiser.
#include <hip/hip_ext.h>

#include "device.hpp"
#include "internal.hpp"

namespace l2d {

// Step start: record (token, pos) for the captured kernels, clear this
// step's argmax slot, and write the embedding row of token into the residual
// stream x (the first step of the toy forward pass, mht18 essay section
// 2.3). Q8_0 and Q4_0 rows are dequantised: x_i = code_i * scale of its
// group (fp32 product, exact before the one rounding). In greedy mode the token is the
// argmax of the previous step, read from the other argmax slot.
__global__ __launch_bounds__(256) void begin_step_kernel(BeginParams p)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int32_t token = p.token;
    if (p.greedy) {
        // maximum over the previous step's argmax slots (wave 0), broadcast
        __shared__ unsigned long long prev;
        if (threadIdx.x < 64) {
            const int q = ((p.pos - 1) & 1) * kArgmaxSlots;
            unsigned long long v = threadIdx.x < kArgmaxSlots
                                       ? p.argmax[(size_t)(q + threadIdx.x) * kArgmaxStride]
                                       : 0ull;
            for (int m = 32; m >= 1; m >>= 1) {
                const unsigned long long o = __shfl_xor(v, m, 64);
                v = o > v ? o : v;
            }
            if (threadIdx.x == 0) prev = v;
        }
        __syncthreads();
        token = (int32_t)(0xFFFFFFFFu - (uint32_t)(prev & 0xFFFFFFFFull));
        if (token < 0 || token >= p.vocab) token = 0;
    }
    if (i < p.d) {
        const int64_t off = (int64_t)token * p.d + i;
        if (p.dtype == DT_F32) {
            p.x[i] = ((const float*)p.emb)[off];
        } else if (p.dtype == DT_Q8) {
            // codes are stored group-interleaved within the row
            const int8_t c = ((const int8_t*)p.emb)[(int64_t)token * p.d + q8_perm_offset(i, p.d, p.gs)];
            p.x[i] = (float)((double)c * (double)p.emb_s[off / p.gs]);
        } else {
            // Q4_0: byte b of a 32-value group holds codes b and b + 16
            const int64_t g = off / 32, j = off % 32;
            const uint8_t b = ((const uint8_t*)p.emb)[g * 16 + j % 16];
            const int c = (j < 16 ? (b & 15) : (b >> 4)) - 8;
            p.x[i] = (float)((double)c * (double)p.emb_s[g]);
        }
    }
    if (i == 0) {
        p.step[kStepToken] = token;
        p.step[kStepPos] = p.pos;
        *(uint64_t*)(p.step + kStepSeed) = p.seed;
        *(double*)(p.step + kStepTemp) = p.temperature;
        p.step[kStepSerial] += 1;  // a new epoch for this step's chained launches
    }
    if (blockIdx.x == 0 && threadIdx.x < kArgmaxSlots)
        p.argmax[((size_t)(p.pos & 1) * kArgmaxSlots + threadIdx.x) * kArgmaxStride] = 0ull;
    if (blockIdx.x == 0 && (int)threadIdx.x < p.hs / 2) {
        const float ang = (float)p.pos * p.freqs[threadIdx.x];
        p.rope[threadIdx.x] = (float)cos((double)ang);
        p.rope[p.hs / 2 + threadIdx.x] = (float)sin((double)ang);
    }
}

hipError_t launch_begin(const BeginParams& p, hipStream_t s, const LaunchEvents* ev)
{
    const unsigned blocks = (unsigned)((p.d + 255) / 256);
    if (ev)
        hipExtLaunchKernelGGL(begin_step_kernel, dim3(blocks), dim3(256), 0u, s, ev->start, ev->stop, 0u, p);
    else
        hipLaunchKernelGGL(begin_step_kernel, dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

// Q8_0 codes from the plain row-major layout into the device layout: every
// row's codes are group-interleaved (q8_perm_offset), and source row r lands
// at destination row (r / blk) * stride + off + r % blk, which places q, k, v
// rows of a layer side by side and interleaves w1 / w3 rows.
__global__ __launch_bounds__(256) void permute_q8_kernel(const int8_t* src, int8_t* dst, int64_t rows,
                                                        int64_t K, int32_t gs, int64_t blk,
                                                        int64_t stride, int64_t off)
{
    const int64_t nq = K / 16;
    const int64_t total = rows * nq;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / nq, c = i % nq;
        const int64_t drow = (r / blk) * stride + off + r % blk;
        *(i32x4*)(dst + drow * K + q8_perm_offset(16 * c, K, gs)) = *(const i32x4*)(src + r * K + 16 * c);
    }
}

hipError_t launch_permute_q8(const int8_t* src, int8_t* dst, int64_t rows, int64_t K, int32_t gs,
                             int64_t blk, int64_t stride, int64_t off, hipStream_t st)
{
    int64_t blocks = (rows * (K / 16) + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(permute_q8_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, rows, K,
                       gs, blk, stride, off);
    return hipGetLastError();
}

// Standalone quantiser: the same wave-cooperative group code the GEMV
// prologue uses, over a vector in device memory.
__global__ __launch_bounds__(256) void quantize_kernel(const float* x, int64_t n, int32_t gs,
                                                      int8_t* q, float* s)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    auto val = [&](int64_t i) -> float { return x[i]; };
    q80_groups_wave(val, n / gs, gs, wave, nwaves, q, s, lane);
}

hipError_t launch_quantize(const float* x, int64_t n, int32_t gs, int8_t* q, float* s,
                           hipStream_t st)
{
    const int64_t ng = n / gs;
    const int64_t gpw = 64 / (gs < 64 ? gs : 64);
    int64_t iters = (ng + gpw - 1) / gpw;
    int64_t blocks = (iters + 3) / 4;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n, gs, q, s);
    return hipGetLastError();
}

}  // namespace l2d
