// stream.hip - the whole Q8_0 decode step (the toy forward pass of the mht18
// essay, section 2.3: per layer RMSNorm, q/k/v matvec, RoPE, cache write,
// attention, output matvec + residual, RMSNorm, w1/w3 matvec, SwiGLU, w2
// matvec + residual; then the final RMSNorm, the classifier and its argmax)
// as one persistent kernel, one workgroup per CU, launched cooperatively.
//
// Batch-1 decode streams every weight once per token, and which bytes it
// streams does not depend on the token: only the arithmetic on them waits
// for the previous phase. So each workgroup is split in two roles:
//
//   worker waves (kSNW of them) do nothing but stream weight chunks and dot
//   them with the matvec input held in LDS. Each walks a table of chunk
//   descriptors built on the host (one scalar load per chunk) and keeps kSNB
//   chunks in flight in registers; its stream runs through all matvec
//   phases of the step without a break: the loads of the next phase's rows
//   go out while the current phase finishes and while the workgroups wait
//   for each other; only the use of a chunk waits for its phase's input. A
//   worker touches no activation in global memory; it leaves each row's sum
//   in LDS.
//
//   control waves (kSAW of them, 256 threads) run everything else: the wait
//   for the previous phase's outputs, the input of each matvec (RMSNorm and
//   Q8_0 quantisation of the activation vector into LDS, the same arithmetic
//   as the per-phase kernels), the epilogue of the workgroup's rows (RoPE and
//   the cache write, residual add, SwiGLU, logits and argmax) and the
//   attention (split-position GQA ranges with the attn_core computation, the
//   last range of a kv head merging them).
//
// Workgroups hand over through progress flags, not grid barriers: after its
// epilogue (or its attention items) a workgroup waits until its own stores
// are complete and then stores the phase's epoch into its flag; a consumer
// waits until every flag has reached the epoch of the phase it needs, then
// reads the data. Each phase of each layer of each launch has its own epoch,
// so flags only grow. A workgroup with no rows in a phase skips the wait and
// the input: it reads nothing and stores nothing there.
//
// Control and workers meet in LDS only: `ready` (the input of phase p is in
// LDS) and `done` (a worker finished phase p and left its row sums in LDS).
// Values passed between workgroups within the launch use device-scope
// loads and stores (ld_dev / st_dev). Every wait is bounded: a wait that
// gives up sets an error word and every wave leaves.
//
// The row ranges, the attention items and the workers' chunk tables come
// from stream_plan.hpp, whose functions the host checker runs over every
// wave of a launch.
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "attn_core.hpp"
#include "device.hpp"
#include "internal.hpp"
#include "stream_plan.hpp"

namespace l2d {

constexpr int kSA = kSAW * kWave;          // control threads per workgroup
constexpr int kSNW = 4;                    // worker waves per workgroup
constexpr int kSNB = 10;                   // weight chunks in flight per worker
constexpr int kST = kSA + kSNW * kWave;    // threads per workgroup
constexpr uint32_t kGridSpin = 1u << 22;   // polls of the progress flags before giving up
constexpr int kSMaxSplits = 16;            // attention position splits per kv head column
constexpr uint32_t kLdsSpin = 1u << 27;    // LDS polls before giving up

// LDS control words of a workgroup
struct SCtl {
    uint32_t ready;  // the input of phase p is in LDS once ready > p
    uint32_t done;   // phase completions reported by the workers (all of them report every phase)
    uint32_t gbar;   // arrivals at control-group barriers
    uint32_t abort;  // a wait gave up: every wave leaves
    int32_t token;
    int32_t last;    // attention: this workgroup completed its kv head's count
    uint32_t pad[2];
    double red[kSAW];
    unsigned long long best[kSAW];
};

// dynamic LDS layout (byte offsets)
struct SLds {
    size_t tab, rope, y, res, in_q, in_s, attn, total;
};

// tstride: descriptors per worker table (each worker's table is copied to
// LDS when the kernel starts)
__host__ __device__ inline SLds stream_lds_layout(int64_t ymax, int64_t kmax, int64_t hs, size_t attn_bytes,
                                                  int64_t tstride)
{
    SLds o;
    auto up = [](size_t v) { return (v + 15) & ~(size_t)15; };
    o.tab = up(sizeof(SCtl));
    o.rope = o.tab + (size_t)kSNW * (size_t)tstride * sizeof(SDesc);
    o.y = o.rope + up((size_t)hs * 4);
    o.res = o.y + up((size_t)ymax * 4);
    o.in_q = o.res + up((size_t)ymax * 4);
    // the matvec input and the attention range share one area
    o.in_s = o.in_q + up((size_t)kmax);
    const size_t in_end = o.in_s + up((size_t)(kmax / kSGS) * 4);
    o.attn = o.in_q;
    const size_t at_end = o.attn + up(attn_bytes);
    o.total = in_end > at_end ? in_end : at_end;
    return o;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Diagnostics (P.trace set): the real-time clock (100 MHz) at event e of
// this workgroup's control group, by its first thread
__device__ __forceinline__ void trace_ctl(const StreamParams& P, int64_t e)
{
    if (P.trace != nullptr && threadIdx.x == 0)
        P.trace[(int64_t)blockIdx.x * P.trace_n + e] = __builtin_amdgcn_s_memrealtime();
}

// ---------------------------------------------------------------- LDS waits

// a control word: every lane reads the same address; taken from the first
// lane so that the compiler knows the value (and every wait loop's exit) is
// uniform across the wave
__device__ __forceinline__ uint32_t lds_ld(const uint32_t* p)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)__hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

__device__ __forceinline__ void lds_st(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void lds_add(uint32_t* p, uint32_t v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// this wave's LDS writes have completed (and no memory access is moved
// across this point by the compiler)
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Barrier of the kSAW control waves: a monotonic arrival counter in LDS;
// each wave tracks how many arrivals complete its next barrier. Gives up
// (and raises abort) after kLdsSpin polls; returns at once once abort is set.
struct ABar {
    SCtl* c;
    uint32_t& n;
    __device__ __forceinline__ void operator()() const
    {
        n += kSAW;
        lds_fence();
        if (lane_id() == 0) lds_add(&c->gbar, 1u);
        uint32_t k = 0;
        while (lds_ld(&c->gbar) < n) {
            if (lds_ld(&c->abort) != 0u) break;
            if (++k > kLdsSpin) {
                lds_st(&c->abort, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
    }
};

// ---------------------------------------------------------------- workers

struct SChunk {
    i32x4 w[4];  // lane j: the four 16-byte quarters of its group's codes
    float s;     // the group's weight scale
};

// Loads of one table item (desc e, layer `layer`): lane j < nb reads the
// four 16-byte quarters of group j of the chunk at w0 + 16 (nb q + j) and
// its scale at s0 + 4 j; lanes past the chunk's groups repeat the last one.
// A phantom item, or no item at all (live false: past the end of the stream,
// or the step has given up), reads the zeroed dummy buffer instead, so every
// ring slot issues the same loads and the compiler's wait counts stay exact.
// The chunk's meta word goes with it for its use.
__device__ __forceinline__ void sk_issue(SChunk& b, uint32_t& meta, const StreamParams& P, const SDesc& e,
                                         int32_t layer, bool live)
{
    const int lane = lane_id();
    const bool real = live && (e.meta & SD_PHANTOM) == 0u;
    meta = live ? e.meta : SD_PHANTOM;
    const int nb = real ? sd_nb(e.meta) : 1;
    const int8_t* cb = real ? P.wbase + e.w0 + (int64_t)layer * e.wl : P.dummy;
    const int8_t* sb = real ? P.wbase + e.s0 + (int64_t)layer * e.sl : P.dummy;
    const uint32_t j = lane < nb ? (uint32_t)lane : (uint32_t)(nb - 1);
#pragma unroll
    for (int q = 0; q < 4; q++)
        b.w[q] = __builtin_nontemporal_load((const i32x4*)(cb + 16 * nb * q + 16u * j));
    b.s = *(const float*)(sb + 4u * j);
}

// Lane j's term of one chunk: the exact int32 dot of group j with the input
// codes in LDS (two independent partial sums: integer addition is exact, so
// the order does not matter), scaled by the weight and input scales in fp64
// (the per-phase GEMV's arithmetic and order); 0 for lanes past the chunk's
// groups.
__device__ __forceinline__ double sk_term(const SChunk& b, uint32_t m, const unsigned char* in_q,
                                          const float* in_s)
{
    const int lane = lane_id();
    const int nb = sd_nb(m), c = sd_c(m);
    const int j = lane < nb ? lane : nb - 1;
    const i32x4* xq = (const i32x4*)(in_q + c * (64 * kSGS));
    i32x4 xv[4];
#pragma unroll
    for (int q = 0; q < 4; q++) xv[q] = xq[nb * q + j];
    const double xsg = (double)in_s[64 * c + j];
    int d0 = 0, d1 = 0;
#pragma unroll
    for (int q = 0; q < 2; q++) {
        d0 = dot4_i8(b.w[q].x, xv[q].x, d0);
        d1 = dot4_i8(b.w[q + 2].x, xv[q + 2].x, d1);
        d0 = dot4_i8(b.w[q].y, xv[q].y, d0);
        d1 = dot4_i8(b.w[q + 2].y, xv[q + 2].y, d1);
        d0 = dot4_i8(b.w[q].z, xv[q].z, d0);
        d1 = dot4_i8(b.w[q + 2].z, xv[q + 2].z, d1);
        d0 = dot4_i8(b.w[q].w, xv[q].w, d0);
        d1 = dot4_i8(b.w[q + 2].w, xv[q + 2].w, d1);
    }
    const double t = ((double)(d0 + d1) * (double)b.s) * xsg;
    return lane < nb ? t : 0.0;
}

// Use of one chunk: its term added into the row's running sum acc; at the
// row's last chunk the wave sum goes to the row's slot in y.
__device__ __forceinline__ void sk_use(const SChunk& b, uint32_t m, double& acc, const unsigned char* in_q,
                                       const float* in_s, float* y)
{
    acc += sk_term(b, m, in_q, in_s);
    if (m & SD_ROWEND) {
        acc = wave_sum_to_last(acc);
        if (lane_id() == kWave - 1) y[sd_local(m)] = (float)acc;
        acc = 0.0;
    }
}

// LDS byte address of a pointer into the workgroup's LDS
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    typedef __attribute__((address_space(3))) const uint32_t lds_u32;
    return (uint32_t)(uintptr_t)(lds_u32*)p;
}

// Wait until the input of phase q is in LDS (ready > q); false when the step
// gives up (abort set, or kLdsSpin polls). The poll loop is one asm block:
// the compiler sees no loop inside the worker's ring, so its wait counts
// for the weight loads in flight stay exact (a loop there made it wait for
// every load before each chunk). The block waits for its own LDS reads.
__device__ __forceinline__ bool sk_wait_ready(SCtl* c, int64_t q)
{
    static_assert(offsetof(SCtl, ready) == 0 && offsetof(SCtl, abort) == 12, "control word offsets");
    uint32_t t0, t1, rdy, abt, cnt;
    asm volatile(
        "s_mov_b32 %[k], 0\n\t"
        "1:\n\t"
        "ds_read_b32 %[v], %[a]\n\t"
        "ds_read_b32 %[w], %[a] offset:12\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "v_readfirstlane_b32 %[r], %[v]\n\t"
        "v_readfirstlane_b32 %[ab], %[w]\n\t"
        "s_nop 4\n\t"
        "s_cmp_gt_u32 %[r], %[q]\n\t"
        "s_cbranch_scc1 2f\n\t"
        "s_cmp_lg_u32 %[ab], 0\n\t"
        "s_cbranch_scc1 2f\n\t"
        "s_add_u32 %[k], %[k], 1\n\t"
        "s_cmp_gt_u32 %[k], %[lim]\n\t"
        "s_cbranch_scc1 2f\n\t"
        "s_sleep 2\n\t"
        "s_branch 1b\n"
        "2:"
        : [v] "=&v"(t0), [w] "=&v"(t1), [r] "=&s"(rdy), [ab] "=&s"(abt), [k] "=&s"(cnt)
        : [a] "v"(lds_addr(c)), [q] "s"((uint32_t)q), [lim] "s"(kLdsSpin)
        : "scc", "memory");
    return rdy > (uint32_t)q && abt == 0u;
}

// this wave's row sums of its current phase are in LDS
__device__ __forceinline__ void sk_signal_done(SCtl* c)
{
    lds_fence();
    if (lane_id() == 0) lds_add(&c->done, 1u);
}

// Diagnostics: the clock at worker w's report of phase p
__device__ __forceinline__ void trace_worker(const StreamParams& P, int64_t w, int64_t p, int64_t NP)
{
    if (P.trace != nullptr && lane_id() == 0)
        P.trace[(int64_t)gridDim.x * P.trace_n + ((int64_t)blockIdx.x * kSNW + w) * NP + p] =
            __builtin_amdgcn_s_memrealtime();
}

// Move the worker from phase `from` (-1: none yet) to phase `to` (NP: the
// end): report `from` done, then wait for the input of `to`. Every worker
// passes through every phase (a phantom item where it has no rows).
__device__ __forceinline__ bool sk_transition(SCtl* c, int64_t from, int64_t to, int64_t NP)
{
    if (from >= 0) sk_signal_done(c);
    return to >= NP || sk_wait_ready(c, to);
}

__device__ __forceinline__ void stream_worker(const StreamParams& P, unsigned char* smem, const SLds& L,
                                              int64_t w)
{
    SCtl* c = (SCtl*)smem;
    float* y = (float*)(smem + L.y);
    const unsigned char* in_q = smem + L.in_q;
    const float* in_s = (const float*)(smem + L.in_s);
    const int64_t NP = 4 * (int64_t)P.L + 1;
    const int64_t wid = (int64_t)blockIdx.x * kSNW + w;
    // this worker's table, copied into its LDS area once (a scalar load per
    // chunk from global memory waited about 0.5 us behind the weight
    // stream's traffic in L2; an LDS read does not)
    const int32_t nL = __builtin_amdgcn_readfirstlane(P.wcnt[2 * wid]);
    const int32_t nC = __builtin_amdgcn_readfirstlane(P.wcnt[2 * wid + 1]);
    SDesc* tab = (SDesc*)(smem + L.tab) + w * P.wtab_stride;
    {
        const i32x4* src = (const i32x4*)(P.wtab + wid * P.wtab_stride);
        i32x4* dst = (i32x4*)tab;
        for (int i = lane_id(); i < 2 * (nL + nC); i += kWave) dst[i] = src[i];
        lds_fence();
    }
    const int32_t total = P.L * nL + nC;  // far below 2^31 chunks per worker
    // load cursor: table index lt of layer ll; after the last layer (ll ==
    // L) the classifier's items follow at lt = nL, nL + 1, ...
    int32_t lt = 0, ll = 0;
    int32_t issued = 0, used = 0;
    bool ok = true;
    SChunk buf[kSNB];
    uint32_t meta[kSNB];
    // the descriptor of the next chunk to issue, read one refill ahead (a
    // uniform LDS read, made scalar)
    auto fetch = [&](int32_t i) {
        const SDesc* ep = tab + i;
        const i32x4 a = *(const i32x4*)ep;
        const i32x4 b2 = *((const i32x4*)ep + 1);
        SDesc e;
        e.w0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(a.y) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane(a.x));
        e.s0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(a.w) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane(a.z));
        e.wl = __builtin_amdgcn_readfirstlane(b2.x);
        e.sl = __builtin_amdgcn_readfirstlane(b2.y);
        e.meta = (uint32_t)__builtin_amdgcn_readfirstlane(b2.z);
        return e;
    };
    SDesc nxt = fetch(0);
    auto refill = [&](int k) {
        const bool live = ok && issued < total;
        sk_issue(buf[k], meta[k], P, nxt, ll, live);
        if (live) {
            ++issued;
            if (++lt == nL && ll < P.L) {
                ++ll;
                lt = ll < P.L ? 0 : nL;
            }
        }
        nxt = fetch(ok && issued < total ? lt : 0);
    };
#pragma unroll
    for (int k = 0; k < kSNB; k++) refill(k);
    // Each pass uses the kSNB chunks the ring holds, in order, and refills
    // each slot at once with the chunk kSNB ahead. The pass has no early
    // exit: an exit edge inside it made the compiler wait for every load in
    // flight before each chunk.
    int64_t cur = -1;  // the phase being used: every phase starts with a first item
    double acc = 0.0;
    do {
#pragma unroll
        for (int k = 0; k < kSNB; k++) {
            if (ok && used < total) {
                const uint32_t m = meta[k];
                if (m & SD_FIRST) {
                    if (cur >= 0) trace_worker(P, w, cur, NP);
                    ok = sk_transition(c, cur, cur + 1, NP);
                    ++cur;
                }
                if (ok && (m & SD_PHANTOM) == 0u) sk_use(buf[k], m, acc, in_q, in_s, y);
                ++used;
            }
            refill(k);
        }
    } while (ok && used < total);
    if (ok) {
        trace_worker(P, w, cur, NP);
        sk_transition(c, cur, NP, NP);
    }
}

// ---------------------------------------------------------------- control

// Wait until every workgroup's progress flag has reached `epoch` (wave 0
// polls them with device-scope loads; the other control waves wait at the
// control barrier). False when the step gives up.
__device__ __forceinline__ bool ctl_wait_flags(const StreamParams& P, SCtl* c, ABar& bar, uint32_t epoch)
{
    if (threadIdx.x < kWave) {
        const int lane = lane_id();
        const int nwg = (int)gridDim.x;
        uint32_t n = 0;
        bool good = true;
        while (true) {
            uint32_t lo = 0xFFFFFFFFu;
            for (int i = lane; i < nwg; i += kWave) {
                const uint32_t v = ld_dev(P.flags + i);
                lo = v < lo ? v : lo;
            }
            if (__all(lo >= epoch)) break;
            if (++n > kGridSpin || ((n & 63) == 0 && ld_dev(&P.sync->err[0]) != 0u)) {
                good = false;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (!good && lane == 0) {
            st_dev(&P.sync->err[0], 1u);
            lds_st(&c->abort, 1u);
        }
    }
    bar();
    return lds_ld(&c->abort) == 0u;
}

// This workgroup's outputs of the phase with this epoch are stored: every
// control wave waits for its own stores to complete, then the flag moves on.
__device__ __forceinline__ void ctl_publish(const StreamParams& P, ABar& bar, uint32_t epoch)
{
    wait_vm_all();
    bar();
    if (threadIdx.x == 0) st_dev(P.flags + blockIdx.x, epoch);
}

// control-group sum of one double per thread, fixed order (wave butterfly,
// then waves 0..3): the per-phase GEMV prologue's block sum
__device__ __forceinline__ double ctl_sum(double v, SCtl* c, ABar& bar)
{
    v = wave_sum(v);
    if (lane_id() == 0) c->red[threadIdx.x >> 6] = v;
    bar();
    const double t = c->red[0] + c->red[1] + c->red[2] + c->red[3];
    bar();  // red is free again
    return t;
}

// store the Q8_0 codes of 16-value chunk k (of K values) and, from the
// group's first lane, its scale; four adjacent threads hold one group
__device__ __forceinline__ void ctl_put(unsigned char* in_q, float* in_s, int64_t k, int64_t K, const float* v)
{
    float sc;
    const i32x4 codes = quant16(v, kSGS / 16, &sc);
    if (k < K / 16) {
        ((i32x4*)in_q)[q8_perm_offset(16 * k, K, kSGS) / 16] = codes;
        if ((k & 3) == 0) in_s[k / 4] = sc;
    }
}

// 16 values of chunk k of the embedding row of `token` (Q8_0, codes stored
// group-interleaved), dequantised as code x scale
__device__ __forceinline__ void ctl_emb16(const StreamParams& P, int token, int64_t k, float* v)
{
    const int64_t base = (int64_t)token * P.d;
    const i32x4 cw = *(const i32x4*)(P.emb + base + q8_perm_offset(16 * k, P.d, kSGS));
    const double sc = (double)P.emb_s[(base + 16 * k) / kSGS];
    const int wd[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int8_t code = (int8_t)((wd[i / 4] >> (8 * (i % 4))) & 0xFF);
        v[i] = (float)((double)code * sc);
    }
}

__device__ __forceinline__ void ctl_dev16(const float* u, int64_t k, float* v)
{
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const f32x4 a = ld_dev4(u + 16 * k + 4 * q);
        v[4 * q] = a.x;
        v[4 * q + 1] = a.y;
        v[4 * q + 2] = a.z;
        v[4 * q + 3] = a.w;
    }
}

// Matvec input of K = dim values: RMSNorm with gain, then Q8_0 codes into
// LDS (chunk k = t + 256 j of thread t); the values are the embedding row
// of `token` (first layer) or the device vector u.
__device__ __forceinline__ void ctl_input_norm(const StreamParams& P, SCtl* c, ABar& bar, unsigned char* in_q,
                                               float* in_s, const float* u, int token, const float* gain)
{
    constexpr int NC = 2;  // dim <= 8192
    const int64_t K = P.d, nq = K / 16;
    const int t = threadIdx.x;
    float v[NC][16];
#pragma unroll
    for (int j = 0; j < NC; j++) {
        if ((int64_t)j * kSA < nq) {  // uniform
            const int64_t k = (int64_t)j * kSA + t < nq ? (int64_t)j * kSA + t : nq - 1;
            if (u)
                ctl_dev16(u, k, v[j]);
            else
                ctl_emb16(P, token, k, v[j]);
        }
    }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < NC; j++) {
        if ((int64_t)j * kSA < nq) {
            const bool ok = (int64_t)j * kSA + t < nq;
            double s = 0.0;
#pragma unroll
            for (int k4 = 0; k4 < 4; k4++)
                s += (double)v[j][4 * k4] * (double)v[j][4 * k4] + (double)v[j][4 * k4 + 1] * (double)v[j][4 * k4 + 1] +
                     (double)v[j][4 * k4 + 2] * (double)v[j][4 * k4 + 2] +
                     (double)v[j][4 * k4 + 3] * (double)v[j][4 * k4 + 3];
            ss += ok ? s : 0.0;
        }
    }
    ss = ctl_sum(ss, c, bar);
    const double r = 1.0 / sqrt(ss / (double)K + P.eps);
#pragma unroll
    for (int j = 0; j < NC; j++) {
        if ((int64_t)j * kSA < nq) {
            const int64_t k = (int64_t)j * kSA + t;
            const int64_t kc = k < nq ? k : nq - 1;
            float o[16];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const f32x4 g = *(const f32x4*)(gain + 16 * kc + 4 * q);
                o[4 * q] = (float)((double)g.x * ((double)v[j][4 * q] * r));
                o[4 * q + 1] = (float)((double)g.y * ((double)v[j][4 * q + 1] * r));
                o[4 * q + 2] = (float)((double)g.z * ((double)v[j][4 * q + 2] * r));
                o[4 * q + 3] = (float)((double)g.w * ((double)v[j][4 * q + 3] * r));
            }
            ctl_put(in_q, in_s, k, K, o);
        }
    }
}

// Matvec input of K values taken as they are (o, or the SwiGLU output):
// Q8_0 codes into LDS. Each thread loads up to four 16-value chunks before it
// uses any, so a whole input of up to 16384 values costs one round trip.
__device__ __forceinline__ void ctl_input_plain(const float* u, int64_t K, unsigned char* in_q, float* in_s)
{
    constexpr int NJ = 4;
    const int64_t nq = K / 16;
    const int t = threadIdx.x;
    for (int64_t base = 0; base < nq; base += NJ * kSA) {
        float v[NJ][16];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            if (base + (int64_t)j * kSA < nq) {  // uniform
                const int64_t k = base + (int64_t)j * kSA + t;
                ctl_dev16(u, k < nq ? k : nq - 1, v[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NJ; j++)
            if (base + (int64_t)j * kSA < nq) ctl_put(in_q, in_s, base + (int64_t)j * kSA + t, K, v[j]);
    }
}

// publish the input of phase p to the workers
__device__ __forceinline__ void ctl_ready(SCtl* c, ABar& bar, int64_t p)
{
    bar();  // every control wave's LDS writes are complete
    if (threadIdx.x == 0) lds_st(&c->ready, (uint32_t)(p + 1));
}

// wait until the workers have reported `want` phases in total (each worker
// reports every phase once, in order)
__device__ __forceinline__ bool ctl_wait_done(SCtl* c, uint32_t want)
{
    uint32_t k = 0;
    while (lds_ld(&c->done) < want) {
        if (lds_ld(&c->abort) != 0u) return false;
        if (++k > kLdsSpin) {
            lds_st(&c->abort, 1u);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    return true;
}

// Attention of layer l (split-position GQA, the per-phase attention
// kernel's computation and merge), over the items of this workgroup.
template <int KG, int HS>
__device__ __forceinline__ void ctl_attention(const StreamParams& P, int l, SCtl* c, ABar& bar, unsigned char* at)
{
    constexpr int G = KG;
    const int hs = HS > 0 ? HS : P.hs;
    const int tid = threadIdx.x;
    const int T = P.pos + 1;
    const int NS = P.nsplit;
    int nact;
    const int per = attn_split(T, NS, attn_shape<kSA>(hs).sc, &nact);
    const int64_t nitems = sp_attn_items(P.nkv, P.gsplit, NS);
    __shared__ double wsh[kMaxG][64];
    __shared__ double lsh[kMaxG];
    for (int64_t it = blockIdx.x; it < nitems; it += gridDim.x) {
        const int vg = (int)(it / NS), split = (int)(it % NS);
        if (split >= nact) continue;  // uniform over the control group
        const int g = vg / P.gsplit, hsub = vg % P.gsplit;
        const size_t qoff = ((size_t)g * P.G + (size_t)hsub * KG) * hs;
        AttnRange r;
        r.q = P.q + qoff;
        r.kc = P.kc + (size_t)l * P.S * P.kvd;
        r.vc = P.vc + (size_t)l * P.S * P.kvd;
        r.kvd = P.kvd;
        r.hs = hs;
        r.G = G;
        r.g = g;
        r.r0 = split * per;
        r.n = min(T - r.r0, per);
        r.fresh = P.pos;  // this launch wrote slot pos: device-scope loads
        r.Gt = G;
        r.qstride = 0;
        r.last0 = 0x3fffffff;
        attn_range<KG, kSA, ABar>(r, at, bar);
        if (nact == 1) {
            for (int e = tid; e < G * hs; e += kSA)
                st_dev(P.o + qoff + e, (float)(attn_value<kSA>(at, G, hs, e) / attn_l<kSA>(at, G, hs, e / hs)));
            bar();  // LDS is reused by the next item
            continue;
        }
        const size_t pbase = ((size_t)vg * NS + split) * G;
        for (int e = tid; e < G * hs; e += kSA) st_dev(P.part_o + pbase * hs + e, attn_value<kSA>(at, G, hs, e));
        if (tid < G) {
            st_dev(P.part_ml + (pbase + tid) * 2, attn_m<kSA>(at, G, hs, tid));
            st_dev(P.part_ml + (pbase + tid) * 2 + 1, attn_l<kSA>(at, G, hs, tid));
        }
        wait_vm_all();
        bar();
        if (tid == 0) {
            uint32_t* ctr = P.head_ctr + (size_t)vg * 32;
            const uint32_t done = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool last = done + 1 == (uint32_t)nact;
            if (last) st_dev(ctr, 0u);  // the next use is a later layer, after every workgroup's flags moved on
            c->last = last ? 1 : 0;
        }
        bar();
        if (c->last) {
            // merge kv head column vg's ranges in fp64: the weight of every
            // (head, range) w_c = e^{m_c - M}, then four lanes per output
            // element over every fourth range, combined by DPP
            const size_t base = (size_t)vg * NS;
            const int sub = tid & 3;
            constexpr int KMAX = kSMaxSplits / 4;  // ranges per lane
            const int kk = (nact + 3) / 4;
            for (int t = tid; t < G * 64; t += kSA) {
                const int h = t / 64, cc = t % 64;
                const bool ok = cc < nact;
                const double mc = ok ? ld_dev(P.part_ml + ((base + cc) * G + h) * 2) : -INFINITY;
                const double lc = ok ? ld_dev(P.part_ml + ((base + cc) * G + h) * 2 + 1) : 0.0;
                const double M = wave_max(mc);
                const double wgt = ok ? exp(mc - M) : 0.0;
                const double Ls = wave_sum(wgt * lc);
                wsh[h][cc] = wgt;
                if ((t & 63) == 0) lsh[h] = Ls;
            }
            bar();
            const int npass = (G * hs + kSA / 4 - 1) / (kSA / 4);
            for (int ps = 0; ps < npass; ps++) {
                const int e = ps * (kSA / 4) + (tid >> 2);
                const int ec = e < G * hs ? e : G * hs - 1;
                const int h = ec / hs;
                double buf[KMAX];
#pragma unroll
                for (int k = 0; k < KMAX; k++)
                    buf[k] = k < kk ? ld_dev(P.part_o + ((base + min(sub + 4 * k, nact - 1)) * G) * hs + ec) : 0.0;
                double O = 0.0;
#pragma unroll
                for (int k = 0; k < KMAX; k++)
                    if (sub + 4 * k < nact) O += wsh[h][sub + 4 * k] * buf[k];
                O += __hiloint2double(dpp_xor1(__double2hiint(O)), dpp_xor1(__double2loint(O)));
                O += __hiloint2double(dpp_xor2(__double2hiint(O)), dpp_xor2(__double2loint(O)));
                if (sub == 0 && e < G * hs) st_dev(P.o + qoff + e, (float)(O / lsh[h]));
            }
        }
        bar();  // LDS and the flag are reused by the next item
    }
}

// Epoch of phase k (0 q/k/v, 1 attention, 2 output, 3 w1/w3, 4 w2) of
// layer l in this launch
__device__ __forceinline__ uint32_t ep(const StreamParams& P, int l, int k)
{
    return P.epoch0 + 1u + 5u * (uint32_t)l + (uint32_t)k;
}

template <int KG, int HS>
__device__ __forceinline__ void stream_control(const StreamParams& P, SPlan s, unsigned char* smem,
                                               const SLds& L)
{
    SCtl* c = (SCtl*)smem;
    float* rcos = (float*)(smem + L.rope);
    float* rsin = rcos + P.hs / 2;
    float* y = (float*)(smem + L.y);
    // this workgroup's rows of the residual stream x (the rows of the output
    // and w2 matvecs), kept in LDS for the whole step
    float* res = (float*)(smem + L.res);
    unsigned char* in_q = smem + L.in_q;
    float* in_s = (float*)(smem + L.in_s);
    const int tid = threadIdx.x, lane = lane_id();
    const int64_t b = blockIdx.x;
    const SRows rows = sp_rows(s, b);
    const int pos = P.pos;
    uint32_t nbar = 0;
    ABar bar{c, nbar};
    // ---- step start: token, the RoPE table of pos, the embedding row
    if (tid < kWave) {
        int token = P.token;
        if (P.greedy) {
            // the previous step's pick: the maximum over its argmax slots
            const int qq = ((pos - 1) & 1) * kArgmaxSlots;
            unsigned long long v = lane < kArgmaxSlots ? ld_dev(P.argmax + (size_t)(qq + lane) * kArgmaxStride) : 0ull;
            for (int m = 32; m >= 1; m >>= 1) {
                const unsigned long long o = __shfl_xor(v, m, kWave);
                v = o > v ? o : v;
            }
            token = (int)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull));
            if (token < 0 || token >= P.V) token = 0;
        }
        if (lane == 0) c->token = token;
    }
    if (tid < P.hs / 2) {
        // fp32 cosine / sine of the fp32 angle pos * freq_j, each the fp64
        // value rounded once
        const float ang = (float)pos * P.freqs[tid];
        rcos[tid] = (float)cos((double)ang);
        rsin[tid] = (float)sin((double)ang);
    }
    bar();
    const int token = c->token;
    if (b == 0) {
        // the step record, and this step's argmax slots cleared; complete
        // before this workgroup's first flag, which every classifier waits for
        if (tid == 0) {
            st_dev(P.step + kStepToken, token);
            st_dev(P.step + kStepPos, pos);
            st_dev((unsigned long long*)(P.step + kStepSeed), (unsigned long long)P.seed);
            st_dev((unsigned long long*)(P.step + kStepTemp), (unsigned long long)__double_as_longlong(P.temperature));
        }
        if (tid < kArgmaxSlots) st_dev(P.argmax + ((size_t)(pos & 1) * kArgmaxSlots + tid) * kArgmaxStride, 0ull);
    }
    {
        // this workgroup's rows of x = the embedding row
        const int64_t r0 = rows.r0[SK_WO], nr = rows.r1[SK_WO] - r0;
        for (int64_t t = tid; t < nr; t += kSA) {
            const int64_t i = r0 + t;
            const int8_t code = P.emb[(int64_t)token * P.d + q8_perm_offset(i, P.d, kSGS)];
            res[t] = (float)((double)code * (double)P.emb_s[((int64_t)token * P.d + i) / kSGS]);
        }
    }

    trace_ctl(P, 0);
    const int64_t NP = sp_phases(s);
    for (int64_t p = 0; p < NP; p++) {
        const SPhase f = sp_phase(s, p);
        trace_ctl(P, 1 + 6 * p);
        const int l = (int)f.layer;
        const int k = f.kind;
        const int64_t r0 = rows.r0[k], nr = rows.r1[k] - r0;
        // wait for the phase's input, then prepare it in LDS (nothing when
        // this workgroup has no rows here)
        if (nr > 0) {
            uint32_t need = 0;  // 0: nothing to wait for (the embedding row)
            if (k == SK_QKV && l > 0) need = ep(P, l - 1, 4);
            else if (k == SK_WO) need = ep(P, l, 1);
            else if (k == SK_W13) need = ep(P, l, 2);
            else if (k == SK_W2) need = ep(P, l, 3);
            else if (k == SK_CLS) need = ep(P, (int)P.L - 1, 4);
            if (need != 0 && !ctl_wait_flags(P, c, bar, need)) return;
            trace_ctl(P, 2 + 6 * p);
            if (k == SK_QKV)
                ctl_input_norm(P, c, bar, in_q, in_s, l == 0 ? nullptr : P.x, token, P.rms_att + (size_t)l * P.d);
            else if (k == SK_W13)
                ctl_input_norm(P, c, bar, in_q, in_s, P.x, token, P.rms_ffn + (size_t)l * P.d);
            else if (k == SK_CLS)
                ctl_input_norm(P, c, bar, in_q, in_s, P.x, token, P.rms_final);
            else
                ctl_input_plain(k == SK_WO ? P.o : P.hb, f.K, in_q, in_s);
        }
        ctl_ready(c, bar, p);
        trace_ctl(P, 3 + 6 * p);
        if (!ctl_wait_done(c, (uint32_t)((p + 1) * kSNW))) return;
        trace_ctl(P, 4 + 6 * p);
        bar();
        // epilogue of this workgroup's rows
        if (k == SK_QKV) {
            const int64_t d = P.d, kvd = P.kvd;
            float* kslot = P.kc + ((size_t)l * P.S + pos) * kvd;
            float* vslot = P.vc + ((size_t)l * P.S + pos) * kvd;
            for (int64_t k2 = tid; 2 * k2 + 1 < nr; k2 += kSA) {
                const int64_t row = r0 + 2 * k2;
                const float a = y[2 * k2], bb = y[2 * k2 + 1];
                if (row < d + kvd) {
                    // RoPE: rotate the pair (2j, 2j+1) of the head by pos * freq_j
                    const int64_t within = row < d ? row : row - d;
                    const int j = (int)((within % P.hs) / 2);
                    const double cs = (double)rcos[j], sn = (double)rsin[j];
                    const float ra = (float)((double)a * cs - (double)bb * sn);
                    const float rb = (float)((double)a * sn + (double)bb * cs);
                    float* dst = row < d ? P.q + row : kslot + within;
                    st_dev(dst, ra);
                    st_dev(dst + 1, rb);
                } else {
                    float* dst = vslot + (row - d - kvd);
                    st_dev(dst, a);
                    st_dev(dst + 1, bb);
                }
            }
        } else if (k == SK_WO || k == SK_W2) {
            for (int64_t t = tid; t < nr; t += kSA) {
                const float xn = (float)((double)res[t] + (double)y[t]);
                res[t] = xn;
                st_dev(P.x + r0 + t, xn);
            }
        } else if (k == SK_W13) {
            // rows (2i, 2i+1) hold w1 row i and w3 row i
            for (int64_t k2 = tid; 2 * k2 + 1 < nr; k2 += kSA) {
                const double z = (double)y[2 * k2];
                const double h3 = (double)y[2 * k2 + 1];
                const double silu = z / (1.0 + exp(-z));
                st_dev(P.hb + (r0 / 2 + k2), (float)(silu * h3));
            }
        } else {
            // logits and the packed argmax (or Gumbel-max sampling) key
            unsigned long long best = 0;
            for (int64_t t = tid; t < nr; t += kSA) {
                const int64_t row = r0 + t;
                const float yv = y[t];
                P.logits[row] = yv;
                const float kv = sample_key(yv, P.temperature, P.seed, pos, f.M, row);
                const unsigned long long key = argmax_pack(kv, (uint32_t)row);
                best = key > best ? key : best;
            }
            for (int m = 32; m >= 1; m >>= 1) {
                const unsigned long long o = __shfl_xor(best, m, kWave);
                best = o > best ? o : best;
            }
            if (lane == 0) c->best[tid >> 6] = best;
            bar();
            if (tid == 0) {
                unsigned long long bm = c->best[0];
                for (int w8 = 1; w8 < kSAW; w8++) bm = c->best[w8] > bm ? c->best[w8] : bm;
                if (bm != 0)
                    atomicMax(P.argmax + ((size_t)(pos & 1) * kArgmaxSlots + b % kArgmaxSlots) * kArgmaxStride, bm);
            }
            trace_ctl(P, 5 + 6 * p);
            return;
        }
        ctl_publish(P, bar, ep(P, l, k == SK_QKV ? 0 : k == SK_WO ? 2 : k == SK_W13 ? 3 : 4));
        trace_ctl(P, 5 + 6 * p);
        if (k == SK_QKV) {
            // attention of layer l once every workgroup's q/k/v rows are stored
            if (!ctl_wait_flags(P, c, bar, ep(P, l, 0))) return;
            ctl_attention<KG, HS>(P, l, c, bar, smem + L.attn);
            if (lds_ld(&c->abort) != 0u) return;
            ctl_publish(P, bar, ep(P, l, 1));
            trace_ctl(P, 6 + 6 * p);
        }
    }
}

template <int KG, int HS>
__global__ __launch_bounds__(kST) void stream_step_kernel(StreamParams P)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const SPlan s{P.d, P.h, P.L, P.kvd, P.V, (int64_t)gridDim.x, kSNW, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const SLds L = stream_lds_layout(P.ymax, P.kmax, P.hs, attn_core_lds_bytes<kSA>(KG, HS > 0 ? HS : P.hs),
                                     P.wtab_stride);
    SCtl* c = (SCtl*)smem;
    if (threadIdx.x == 0) {
        c->ready = 0;
        c->done = 0;
        c->gbar = 0;
        c->abort = 0;
    }
    __syncthreads();  // the only workgroup-wide barrier: roles never meet at one again
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (wave < kSAW)
        stream_control<KG, HS>(P, s, smem, L);
    else
        stream_worker(P, smem, L, wave - kSAW);
}

// ---------------------------------------------------------------- host side

bool stream_supported(int dt, int gs, int64_t d, int64_t h, int G, int gsplit, int hs)
{
    if (dt != DT_Q8 || gs != kSGS) return false;
    if (d % kSGS || h % kSGS || d > 8192 || h > 65536) return false;
    if (gsplit < 1 || G % gsplit) return false;
    const int kg = G / gsplit;
    if (kg != 1 && kg != 2 && kg != 4 && kg != 8) return false;
    return attn_core_supported<kSA>(kg, hs) && hs / 2 <= kSA;
}

size_t stream_lds_bytes(const SPlan& s, int kg, int hs, int64_t tstride)
{
    const int64_t kmax = s.d > s.h ? s.d : s.h;
    return stream_lds_layout(sp_max_wg_rows(s), kmax, hs, attn_core_lds_bytes<kSA>(kg, hs), tstride).total;
}

template <int KG>
static const void* kernel_hs(int hs)
{
    return hs == 128 ? (const void*)stream_step_kernel<KG, 128>
         : hs == 64  ? (const void*)stream_step_kernel<KG, 64>
                     : (const void*)stream_step_kernel<KG, 0>;
}

static const void* stream_kernel(int kg, int hs)
{
    switch (kg) {
    case 1: return kernel_hs<1>(hs);
    case 2: return kernel_hs<2>(hs);
    case 4: return kernel_hs<4>(hs);
    case 8: return kernel_hs<8>(hs);
    default: return nullptr;
    }
}

int stream_threads() { return kST; }

// attention position splits per kv head column: about one item per
// workgroup, at most kSMaxSplits, at most one split per sub-chunk
int stream_splits(int64_t nkv, int64_t gsplit, int64_t nwg, int64_t S, int hs)
{
    const int64_t cols = nkv * gsplit;
    const int64_t sc = attn_shape<kSA>(hs).sc;
    int64_t ns = (nwg + cols / 2) / cols;
    if (ns > kSMaxSplits) ns = kSMaxSplits;
    if (ns > (S + sc - 1) / sc) ns = (S + sc - 1) / sc;
    return (int)(ns < 1 ? 1 : ns);
}
int stream_workers() { return kSNW; }

int stream_blocks_per_cu(int kg, int hs, size_t lds)
{
    const void* f = stream_kernel(kg, hs);
    if (!f) return 0;
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kST, lds) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}

hipError_t launch_stream(const StreamParams& p, int kg, int grid, size_t lds, hipStream_t st)
{
    const void* f = stream_kernel(kg, p.hs);
    if (!f) return hipErrorInvalidValue;
    StreamParams arg = p;
    void* args[] = {&arg};
    return hipLaunchCooperativeKernel(f, dim3((unsigned)grid), dim3(kST), args, (unsigned)lds, st);
}

}  // namespace l2d
