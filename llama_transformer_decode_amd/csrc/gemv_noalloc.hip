// gemv_noalloc.hip - l2d_gemv without any device allocation.
//
// l2d_gemv re-lays Q8_0 codes out into a temporary device buffer (the
// group-interleaved rows the matvec kernel reads) that it allocates and frees
// on the stream. Callers that cannot allocate device memory (code under
// stream capture, tight serving loops, harnesses that forbid it) use
// l2d_gemv_noalloc instead: the re-laid-out codes go to `scratch`, a fixed
// array in device memory that the library's code object holds on every GPU
// it runs on, until the process ends.
//
// Host code never passes the array's name to a kernel or a copy: in host
// code it is a host-side stand-in, not a device address. The device address
// comes from hipGetSymbolAddress, taken once per device (with that device
// current) on the entry point's first call there and kept in dev_scratch.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "internal.hpp"
#include "l2d.h"
#include "runtime.hpp"

namespace l2d {
namespace {

// rows * cols codes at most (32 MiB: a 4096 x 8192 matrix, or the 7B q/k/v
// output projection shapes; the w1/w3 and classifier shapes do not fit)
constexpr int64_t kScratchBytes = 32ll << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) int8_t scratch[kScratchBytes];

std::mutex g_mu;
int8_t* dev_scratch[kMaxDevices] = {};

// device address of `scratch` on the current device, looked up once per
// device; nullptr (error recorded) when the lookup fails
int8_t* scratch_of_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fail(nullptr, L2D_EHIP, "gemv_noalloc: no current device");
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!dev_scratch[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            fail(nullptr, L2D_EHIP, std::string("gemv_noalloc: scratch address: ") + hipGetErrorString(e));
            return nullptr;
        }
        dev_scratch[dev] = (int8_t*)ptr;
    }
    return dev_scratch[dev];
}

}  // namespace
}  // namespace l2d

using namespace l2d;

extern "C" int64_t l2d_gemv_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int l2d_gemv_noalloc(int32_t dtype, const void* W, const float* W_s, const float* x, int64_t rows,
                                int64_t cols, int32_t gs, float* out, int32_t* group_dots, void* stream)
{
    GemvParams p;
    int dt = 0;
    int rc = gemv_setup(dtype, x, rows, cols, gs, W_s != nullptr, out, &p, &dt);
    if (rc != L2D_OK) return rc;
    if (!W) return fail(nullptr, L2D_EINVAL, "gemv_noalloc: null weights");
    hipStream_t st = (hipStream_t)stream;
    const void* wk = W;
    if (dtype == L2D_Q8_0) {
        if (rows > kScratchBytes / cols)
            return fail(nullptr, L2D_EINVAL,
                        "gemv_noalloc: rows x cols = " + std::to_string(rows * cols) +
                            " Q8_0 codes exceed the " + std::to_string(kScratchBytes) +
                            "-byte scratch array (use l2d_gemv)");
        int8_t* buf = scratch_of_current_device();
        if (!buf) return L2D_EHIP;
        // every code of rows x cols is rewritten before the matvec reads it
        hipError_t e = launch_permute_q8((const int8_t*)W, buf, rows, cols, gs, 1ll << 62, 0, 0, st);
        if (e != hipSuccess) return fail(nullptr, L2D_EHIP, std::string("gemv_noalloc: ") + hipGetErrorString(e));
        wk = buf;
    }
    p.W = wk;
    p.Ws = W_s;
    p.group_dots = dtype == L2D_F32 ? nullptr : group_dots;
    hipError_t e = launch_gemv(dt, PRO_PLAIN, EPI_STORE, p, gemv_grid(), st);
    if (e != hipSuccess) return fail(nullptr, L2D_EHIP, std::string("gemv_noalloc: ") + hipGetErrorString(e));
    return L2D_OK;
}
