// Allocation-free form of the dynamic-scale linear: blockint8_linear with its
// workspace (the quantised activations and their scales, staged between the
// quantisation and the GEMM launch) in a fixed device array of this library
// instead of caller-provided buffers.  For callers that cannot allocate
// device memory around the call (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  See include/blockint8.h.
//
// The array, `scratch`, is a file-scope __device__ object: every GPU the
// library runs on holds its own copy until the process ends.  In host code
// its name is only a handle for the symbol, never a device address: the
// address of each device's copy is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/blockint8.h"
#include "internal.hpp"

namespace {

constexpr int64_t kScratchBytes = BI8_NOALLOC_SCRATCH_BYTES;

// [0, align256(M*K)): int8 codes [M, K]; then fp32 scales [M, KB].
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_addr[kMaxDevices];   // device address of `scratch` per device, once looked up

// Device address of the current device's copy of `scratch`.
hipError_t current_scratch(void **addr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int32_t blockint8_linear_noalloc(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws,
                                            const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                                            int32_t block_n, int32_t block_k, void *stream) {
    static const char fn[] = "blockint8_linear_noalloc";
    int32_t s = bi8::check_linear_args(fn, x, ldx, w, ws, bias, y, M, N, K, block_n, block_k);
    if (s) return s;
    if (M == 0) return bi8::call_status(fn, hipSuccess);
    // M <= 2^31 and K <= 2^23: the products below fit in int64
    const int64_t KB = (block_n == 1 && block_k == K) ? 1 : (K + 127) / 128;
    const int64_t codes = (M * K + 255) / 256 * 256;
    const int64_t need = codes + 4 * M * KB;
    if (need > kScratchBytes)
        return bi8::fail_status(BI8_ERR_SHAPE,
                                "%s: M = %lld, K = %lld needs %lld bytes of workspace; the static workspace "
                                "holds %lld (use blockint8_linear with caller-provided workspaces)",
                                fn, (long long)M, (long long)K, (long long)need, (long long)kScratchBytes);
    void *base = nullptr;
    hipError_t e = current_scratch(&base);
    if (e != hipSuccess) return bi8::call_status(fn, e);
    int8_t *xq = static_cast<int8_t *>(base);
    float *xs = reinterpret_cast<float *>(static_cast<unsigned char *>(base) + codes);
    return bi8::call_status(fn, bi8::launch_linear(x, ldx, w, ws, bias, y, M, N, K, block_n, block_k, xq, xs,
                                                   static_cast<hipStream_t>(stream)));
}
