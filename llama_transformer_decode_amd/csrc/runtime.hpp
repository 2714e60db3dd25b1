// runtime.hpp - the decode context and host-side helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "internal.hpp"
#include "l2d.h"

namespace l2d {

// record an error message (for ctx, or the calling thread when ctx is null)
// and return code
int fail(l2d_ctx* ctx, int code, const std::string& msg);

// check a config against what the kernels support; returns L2D_OK or L2D_EINVAL
int validate_config(const l2d_config* c);

// argument checks of l2d_gemv and its kernel parameters (weights unset);
// returns L2D_OK or the error recorded for the calling thread
int gemv_setup(int32_t dtype, const float* x, int64_t rows, int64_t cols, int32_t gs,
               bool have_scales, float* out, GemvParams* p, int* dt);

// workgroups of a standalone matvec launch on the current device
int gemv_grid();

}  // namespace l2d

struct l2d_ctx {
    l2d_config cfg;
    int dt;
    int64_t d, h, L, V, S, nh, nkv, hs, kvd, G;
    int gs;
    hipStream_t stream = nullptr;
    bool own_stream = false;
    int device = 0;
    int max_blocks = 0;  // GEMV workgroup cap (CUs x workgroups per CU)

    // device weights, in the library's layout
    void* emb = nullptr;      // [V][d]
    float* emb_s = nullptr;
    void* wqkv = nullptr;     // [L][d + 2 kvd][d]: q rows, then k rows, then v rows
    float* wqkv_s = nullptr;
    void* wo = nullptr;       // [L][d][d]
    float* wo_s = nullptr;
    void* w13 = nullptr;      // [L][2h][d]: row 2i = w1 row i, row 2i+1 = w3 row i
    float* w13_s = nullptr;
    void* w2 = nullptr;       // [L][d][h]
    float* w2_s = nullptr;
    void* wcls = nullptr;     // [V][d], aliases emb when the classifier is shared
    float* wcls_s = nullptr;
    float* rms_att = nullptr;
    float* rms_ffn = nullptr;
    float* rms_final = nullptr;
    float* freqs = nullptr;   // [hs/2]
    float* rope = nullptr;    // [hs]: this step's RoPE cos / sin (step-start kernel)

    // state
    float* kc = nullptr;      // [L][S][kvd]
    float* vc = nullptr;
    float* x = nullptr;       // residual stream [d]
    float* q = nullptr;       // [d]
    float* o = nullptr;       // attention output [d]
    float* hb = nullptr;      // [h]
    int8_t* hb_q = nullptr;   // Q8_0 / Q4_0 models: codes of hb [h], its scales [h/gs],
    float* hb_s = nullptr;    // written by the w1/w3 matvec for the w2 matvec
    uint32_t* hb_ctr = nullptr;  // [h/gs][kGroupCtrStride] group completion counters
    float* logits = nullptr;  // [V]
    int32_t* step = nullptr;  // {token, pos}
    unsigned long long* argmax = nullptr;  // [2][kArgmaxSlots][kArgmaxStride]
    double* part_o = nullptr;
    double* part_ml = nullptr;
    uint32_t* attn_ctr = nullptr;  // [nkv][32] ranges done per kv head (attention merge)
    int nsplit = 0;
    int gsplit = 1;  // workgroups per kv head in decode attention

    // chained launches (attention + output projection, w1/w3 + w2 in one
    // launch each; Q8_0, group size 64)
    bool chain_ok = false;             // supported for this model on this device
    bool use_chain = false;
    bool chain_pending = false;        // chained launches ran since the error word was last read
    uint32_t* chain_flags = nullptr;   // [nkv * gsplit] attention columns, then [h / gs] FFN groups
    uint32_t* chain_err = nullptr;     // [0]: set when a wait of a chained launch gives up;
                                       // [32], [64]: the go words of the two chained launches
    int8_t* chain_hbq = nullptr;       // [h / gs][128 bytes]: SwiGLU output codes, then scale, per group

    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    bool use_graph = true;

    // the persistent step kernel (one cooperative launch per step, Q8_0)
    bool stream_ok = false;       // supported for this model on this device
    bool use_stream = false;
    bool stream_pending = false;  // launched since the error word was last read
    int stream_grid = 0;
    int stream_kg = 1;            // query heads per attention item
    int stream_gsplit = 1;
    int stream_nsplit = 1;
    int stream_ymax = 0;
    size_t stream_lds = 0;
    uint32_t stream_epoch = 0;    // progress-flag epochs used so far
    l2d::StreamSync* ssync = nullptr;
    uint32_t* sflags = nullptr;   // [stream_grid] progress flags
    l2d::SDesc* swtab = nullptr;  // workers' chunk tables
    int32_t* swcnt = nullptr;
    int64_t swtab_stride = 0;
    uint32_t* shead_ctr = nullptr;
    double* spart_o = nullptr;
    double* spart_ml = nullptr;
    int8_t* sdummy = nullptr;
    uint64_t* strace = nullptr;   // diagnostics: clock stamps of the next launch (l2d_stream_trace)

    // batched prefill (allocated by the first l2d_prefill): chunk capacity
    // in tokens (a multiple of 16), token ids, residual rows, q rows,
    // attention outputs, FFN hidden rows, quantised matmul inputs, RoPE tables
    int pf_cap = 0;
    int pf_combine = 0;      // Q8_0 group combine of the prefill matmuls: 0 fp64, 1 fp32
    int32_t* pf_tok = nullptr;
    float* pf_x = nullptr;   // [cap][d]
    float* pf_q = nullptr;   // [cap][d]
    float* pf_o = nullptr;   // [cap][d]
    float* pf_h = nullptr;   // [cap][h]
    int8_t* pf_aq = nullptr; // [cap][max(d, h)]
    float* pf_as = nullptr;  // [cap][max(d, h) / gs]
    float* pf_cos = nullptr; // [cap][hs / 2]
    float* pf_sin = nullptr;

    int trace_layer = -1;
    int8_t* trace_q[4] = {nullptr, nullptr, nullptr, nullptr};
    float* trace_s[4] = {nullptr, nullptr, nullptr, nullptr};

    int32_t last_pos = -1;
    double temperature = 0.0;  // next-token sampling (0: greedy argmax)
    uint64_t seed = 0;
    std::string err;
    std::vector<void*> allocs;
};
