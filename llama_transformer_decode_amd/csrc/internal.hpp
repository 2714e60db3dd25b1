// internal.hpp - kernel parameter blocks and launchers shared by the runtime
// (ctx.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace l2d {

// DT_Q4: 4-bit weight codes, two per byte, groups of 32 with an fp32 scale
// (matvec only; the input vector is quantised to Q8_0 with groups of 32).
enum Dt { DT_F32 = 0, DT_Q8 = 1, DT_Q4 = 2 };

// The device step record (int32 words), written by the step-start kernel:
// token, pos, then the sampler's seed (uint64) and temperature (fp64; 0 =
// greedy argmax) at 8-byte aligned word offsets, and the step serial, which
// every step-start kernel advances by one (the epochs of chained launches).
enum { kStepToken = 0, kStepPos = 1, kStepSeed = 2, kStepTemp = 4, kStepSerial = 6, kStepWords = 16 };

// The classifier's argmax is kept in kArgmaxSlots packed 64-bit slots per
// step parity (pos & 1), each on its own 128-byte line, so that workgroups
// finishing together do not serialise on one atomic; the step's argmax is
// the maximum over the slots.
constexpr int kArgmaxSlots = 64;
constexpr int kArgmaxStride = 16;  // u64 per slot
constexpr int kArgmaxWords = 2 * kArgmaxSlots * kArgmaxStride;

// spacing of per-group completion counters (uint32): one 64-byte line each
constexpr int kGroupCtrStride = 16;

// GEMV input-vector preparation (the "prologue", run by every workgroup into
// its LDS): PRO_PLAIN takes x as is; PRO_NORM applies RMSNorm with gain;
// PRO_CODES takes x already quantised to Q8_0 (codes xq, scales xs).
enum Pro { PRO_PLAIN = 0, PRO_NORM = 1, PRO_CODES = 2 };

// What happens to each finished output row (the "epilogue").
enum Epi {
    EPI_STORE = 0,   // out[row] = y
    EPI_RESID = 1,   // out[row] += y (residual stream)
    EPI_QKV = 2,     // RoPE on q/k pairs, q -> out, k/v -> cache slot pos
    EPI_SWIGLU = 3,  // rows (2i, 2i+1) = (w1, w3): out[i] = silu(y0) * y1
    EPI_LOGITS = 4,  // out[row] = y and a packed 64-bit argmax
};

struct GemvParams {
    const void* W;     // fp32 [M][K], int8 codes [M][K] or Q4_0 nibbles [M][K/2]
    const float* Ws;   // Q8_0 / Q4_0 scales [M][K/gs]
    int64_t M, K;
    int32_t gs;
    const float* x;     // input vector [K], fp32
    const float* gain;  // RMSNorm gain [K] (PRO_NORM)
    const int8_t* xq;   // PRO_CODES: Q8_0 codes of the input [K], plain order
    const float* xs;    //            and its group scales [K/gs]
    double eps;
    float* out;
    // EPI_QKV
    float* kcache;  // this layer's [seq_len][kv_dim]
    float* vcache;
    int32_t d, kvd, hs;
    const float* rope;    // [hs]: fp32 cos, then sin, of pos * freq_j for this step's pos
    const int32_t* step;  // device step record (kStep*)
    // EPI_LOGITS
    unsigned long long* argmax;  // [2][kArgmaxSlots][kArgmaxStride], parity pos & 1
    // EPI_SWIGLU: when oq is set, the output is also quantised to Q8_0 with
    // groups of ogs (codes oq [M/2], scales os [M/2/ogs]) for the next matvec,
    // each group once, by the wave that completes it (counters octr, zero
    // between launches, kGroupCtrStride apart)
    int8_t* oq;
    float* os;
    uint32_t* octr;
    int32_t ogs;
    // diagnostics
    int32_t* group_dots;  // [M][K/gs] exact int32 group dots (Q8_0, Q4_0; test hook)
    int8_t* trace_q;      // workgroup 0 copies its quantised input here
    float* trace_s;
};

// Optional kernel timing: events stamped at the kernel's own start and end
// (hipExtLaunchKernel), so durations match a hardware kernel trace.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

hipError_t launch_gemv(int dt, int pro, int epi, const GemvParams& p, int max_blocks,
                       hipStream_t s, const LaunchEvents* ev = nullptr);

// A chained launch runs two consecutive phases of a layer (attention and
// the output projection; w1/w3 and w2): the second phase's workgroups follow
// the first's in the grid, prefetch their weights, and wait on flags the
// first phase's workgroups set once their outputs are stored. A flag holds
// the epoch of the launch that set it (chain_epoch: step serial x layers +
// layer + 1), so flags need no reset between launches.
struct ChainArgs {
    const uint32_t* flags;  // the producer flags the second phase waits on
    int32_t nflags;
    uint32_t* pub;          // the flags the first phase sets (the same array)
    uint32_t* go;           // the second phase's first workgroup sets it to the epoch
                            // once every flag holds it; the others poll it
    uint32_t* err;          // set when a wait gives up (zero otherwise)
    int32_t layer, nlayers;
};

// dynamic LDS bytes the GEMV needs for an input of K values (+ the RoPE
// table of a head of hs values for the q/k/v epilogue, else hs = 0)
size_t gemv_lds_bytes(int dt, int64_t K, int gs, int hs);

struct AttnParams {
    const float* q;    // [n_heads * hs]
    const float* kc;   // this layer's [S][kvd]
    const float* vc;
    float* o;          // [n_heads * hs]
    double* part_o;    // [nkv][nsplit][G][hs]
    double* part_ml;   // [nkv][nsplit][G][2]
    uint32_t* ctr;     // [nkv * gsplit][32]: ranges done this launch per (kv head, head subset); zero between launches
    const int32_t* step;
    int32_t S, nkv, hs, kvd, G, nsplit;
    int32_t gsplit;    // workgroups sharing one kv head's G query heads (G / gsplit heads each)
};

hipError_t launch_attention(const AttnParams& p, hipStream_t s, const LaunchEvents* ev = nullptr);
size_t attention_lds_bytes(int G, int hs, int unused);
bool attention_supported(int G, int hs);
int attention_positions_per_subchunk(int hs);
// attention workgroups that can be resident on one CU for this shape (the
// instance the launch would pick), or 0 if the runtime cannot tell
int attention_blocks_per_cu(int G, int gsplit, int hs);

// ---- chained launches (chain.hip): Q8_0 weights, groups of 64

// true when both chained launches serve this shape (the instances built,
// and every w1/w3 workgroup owning rows)
bool chain_supported(int dt, int gs, int64_t d, int64_t h, int G, int gsplit, int hs, int max_blocks);
// attention, then the output projection + residual (wo: PRO_PLAIN, EPI_RESID)
hipError_t launch_attn_wo(const AttnParams& a, const GemvParams& wo, const ChainArgs& c, int max_blocks,
                          hipStream_t s, const LaunchEvents* ev = nullptr);
// w1/w3 + SwiGLU (PRO_NORM, EPI_SWIGLU, output quantised), then w2 +
// residual on its codes (PRO_CODES, EPI_RESID)
hipError_t launch_ffn_chain(const GemvParams& w13, const GemvParams& w2, const ChainArgs& c, int max_blocks,
                            hipStream_t s, const LaunchEvents* ev = nullptr);
// attention workgroups of the chained attention launch resident per CU
int attn_wo_blocks_per_cu(int G, int gsplit, int hs, int64_t d, int gs);

// ---- batched prefill (prefill.hip)

struct PrefillEmbedParams {
    const void* emb;       // embedding table, device layout
    const float* emb_s;    // Q8_0 scales
    int32_t dtype, gs;
    int64_t d;
    const int32_t* tokens; // [m]
    int32_t m;
    float* x;              // [m][d]
};
hipError_t launch_prefill_embed(const PrefillEmbedParams& p, hipStream_t s);

// cos / sin tables [m][hs/2] of positions pos0 .. pos0 + m - 1
hipError_t launch_prefill_rope(const float* freqs, int hs, int pos0, int m, float* rcos, float* rsin,
                               hipStream_t s);

struct PrefillPrepParams {
    const float* x;     // [m][K]
    const float* gain;  // RMSNorm gain [K] (norm only)
    double eps;
    int64_t K;
    int32_t gs, m;
    int8_t* q;          // codes in the matmul's operand order: [m/16][K/gs][gs/64][64 lanes][16]
    float* s;           // [m][K/gs] scales
    float* xo;          // fp32 weights: the normalised rows [m][K] instead of codes (q, s unused)
};
hipError_t launch_prefill_prep(const PrefillPrepParams& p, bool norm, hipStream_t s,
                               const LaunchEvents* ev = nullptr);

struct PrefillGemmParams {
    int32_t dtype;      // DT_Q8 (int8 MFMA) or DT_F32 (fp64 MFMA)
    const void* W;      // Q8_0 codes [N][K], device (group-interleaved) layout, or fp32 [N][K]
    const float* Ws;    // [N][K/gs]
    int64_t N, K;
    int32_t gs, m;
    const int8_t* aq;   // input codes in operand order (prefill_prep_kernel), tiles of 16 tokens
    const float* as;    // [m][K/gs]
    const float* a32;   // fp32 weights: input rows [m][K]
    float* out;         // EPI_STORE / EPI_QKV (q rows) / EPI_SWIGLU: [m][ldo]; EPI_RESID: += into [m][ldo]
    int64_t ldo;
    // EPI_QKV
    float* kcache;      // this layer's [seq_len][kv_dim]
    float* vcache;
    int32_t d, kvd, hs, pos0;
    const float* rcos;  // [m][hs/2]
    const float* rsin;
    // Q8_0 group combine: 0 fp64 (bit-identical to single-token steps), 1 fp32
    int32_t combine;
};
hipError_t launch_prefill_gemm(int epi, const PrefillGemmParams& p, hipStream_t s,
                               const LaunchEvents* ev = nullptr);
size_t prefill_gemm_grid(int64_t N, int m);

struct PrefillAttnParams {
    const float* q;     // [>= m rounded up to the token block][d]
    const float* kc;    // this layer's caches
    const float* vc;
    float* o;           // [m][d]
    int32_t d, kvd, hs, G, nkv, m, pos0;
};
bool prefill_attn_supported(int G, int hs);
hipError_t launch_prefill_attn(const PrefillAttnParams& p, hipStream_t s, const LaunchEvents* ev = nullptr);

struct BeginParams {
    const void* emb;
    const float* emb_s;
    int32_t dtype, gs, d, vocab;
    float* x;
    int32_t* step;
    unsigned long long* argmax;
    int32_t token, pos, greedy;
    double temperature;  // 0: the classifier's argmax picks the token
    uint64_t seed;
    // RoPE table of this step: rope[j] = cos, rope[hs/2 + j] = sin of the
    // fp32 angle pos * freqs[j], each the fp64 value rounded once
    const float* freqs;
    float* rope;
    int32_t hs;
};

hipError_t launch_begin(const BeginParams& p, hipStream_t s, const LaunchEvents* ev = nullptr);

hipError_t launch_permute_q8(const int8_t* src, int8_t* dst, int64_t rows, int64_t K, int32_t gs,
                             int64_t blk, int64_t stride, int64_t off, hipStream_t st);

hipError_t launch_quantize(const float* x, int64_t n, int32_t gs, int8_t* q, float* s,
                           hipStream_t st);

// ---------------------------------------------------------------- step kernel
// The whole Q8_0 decode step as one persistent cooperative kernel
// (stream.hip): worker waves stream the weights, control waves run the grid
// barriers, prologues, epilogues and attention.

// Error word of the step kernel: set when a wait gives up (every wave then
// leaves, and the host reports the step invalid).
struct StreamSync {
    uint32_t err[32];
};

struct SDesc;

struct StreamParams {
    int32_t d, h, L, nkv, hs, kvd, G, V, S;
    int32_t nsplit;  // attention position splits per kv head column
    int32_t gsplit;  // attention items sharing one kv head's query heads
    int32_t ymax;    // row results one workgroup holds in LDS
    int32_t kmax;    // longest matvec input (max(dim, hidden_dim))
    double eps;
    // weights in the library's device layout (Q8_0, group size 64)
    const int8_t* emb;
    const float* emb_s;
    const int8_t* wqkv;
    const float* wqkv_s;
    const int8_t* wo;
    const float* wo_s;
    const int8_t* w13;
    const float* w13_s;
    const int8_t* w2;
    const float* w2_s;
    const int8_t* wcls;
    const float* wcls_s;
    const float* rms_att;
    const float* rms_ffn;
    const float* rms_final;
    const float* freqs;
    // state
    float* kc;
    float* vc;
    float* x;
    float* q;
    float* o;
    float* hb;
    float* logits;
    int32_t* step;
    unsigned long long* argmax;
    double* part_o;      // [nkv * gsplit][nsplit][G / gsplit][hs]
    double* part_ml;     // [nkv * gsplit][nsplit][G / gsplit][2]
    uint32_t* head_ctr;  // [nkv * gsplit][32]: ranges of the column finished (zero between uses)
    StreamSync* sync;
    // progress of each workgroup: the epoch of the last phase whose outputs it
    // has stored (each phase of each layer of each launch has its own epoch)
    uint32_t* flags;
    const int8_t* dummy; // 8 KiB of zeroed device memory: the loads past the end of a worker's stream
    // the workers' chunk tables (stream_tables): worker wid's at
    // wtab[wid * wtab_stride], wcnt[2 wid] items per layer, wcnt[2 wid + 1]
    // classifier items; offsets from wbase
    const int8_t* wbase;
    const SDesc* wtab;
    int64_t wtab_stride;
    const int32_t* wcnt;
    // this launch
    int32_t token, pos, greedy;
    uint32_t epoch0;     // epochs used by earlier launches (the first phase of this one is epoch0 + 1)
    double temperature;  // 0: argmax
    uint64_t seed;
    // diagnostics: when set, clock stamps of each workgroup's control events
    // ([nwg][trace_n]) and of each worker's phase reports ([nwg][workers][phases])
    uint64_t* trace;
    int64_t trace_n;
};

// control events per workgroup in a step kernel trace
inline int64_t stream_trace_events(int L) { return 1 + 6 * (4 * (int64_t)L + 1); }

// epochs one launch of the step kernel uses: five per layer (q/k/v,
// attention, output, w1/w3, w2) and one spare
inline uint32_t stream_epochs(int L) { return 5u * (uint32_t)L + 1u; }

struct SPlan;
void stream_tables(const SPlan& s, std::vector<SDesc>& tab, std::vector<int32_t>& cnt, int64_t* stride);
bool stream_supported(int dt, int gs, int64_t d, int64_t h, int G, int gsplit, int hs);
size_t stream_lds_bytes(const SPlan& s, int kg, int hs, int64_t tstride);
int stream_threads();
int stream_splits(int64_t nkv, int64_t gsplit, int64_t nwg, int64_t S, int hs);
int stream_workers();
// workgroups of the step kernel a CU can hold with this much LDS (0: none)
int stream_blocks_per_cu(int kg, int hs, size_t lds);
hipError_t launch_stream(const StreamParams& p, int kg, int grid, size_t lds, hipStream_t s);

}  // namespace l2d
