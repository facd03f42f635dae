// Shader-clock probe for the benchmark (measurement support, not part of
// the block-wise INT8 path; built into its own library, libbi8clock.so).
//
// One wave per workgroup records three 64-bit values: the shader-clock cycle
// counter (s_memtime, which advances at the current GFX clock), the
// constant-rate real-time counter (s_memrealtime, at the rate
// hipDeviceAttributeWallClockRate reports) and where the wave ran: the XCD
// id in bits [3:0] and the HW_ID register (CU, shader array and shader
// engine in its bits [15:8]) in bits [63:32].  The cycle counters of
// different compute units are not aligned with each other, so samples are
// compared per compute unit.  Launched with enough workgroups to reach every
// CU just before and just after a timed region on the same stream, the two
// samples of one CU give the average GFX clock there over the region:
//     f = (memtime_after - memtime_before) / (realtime_after - realtime_before)
//         * wall_clock_rate.
//
//   int bi8clock_sample(uint64_t *out, int blocks, void *stream)
//       out: device uint64 [blocks, 3] = (memtime, realtime, place) per
//       workgroup; 1 <= blocks <= 1024.  Returns 0, or -1 on a bad argument,
//       or the HIP error code of the launch.
//   int bi8clock_wall_rate_khz(int device)
//       the real-time counter's rate in kHz (0 if the query fails).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t *out) {
    if (threadIdx.x == 0) {
        const uint64_t t = __builtin_amdgcn_s_memtime();
        const uint64_t r = __builtin_amdgcn_s_memrealtime();
        // hwreg XCC_ID bits [3:0]: the XCD this wave runs on; hwreg HW_ID
        // (all 32 bits): its wave, SIMD, CU, shader array and engine
        const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);
        const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
        out[blockIdx.x * 3 + 0] = t;
        out[blockIdx.x * 3 + 1] = r;
        out[blockIdx.x * 3 + 2] = ((uint64_t)hw << 32) | (xcc & 0xFu);
    }
}

}  // namespace

extern "C" int bi8clock_sample(uint64_t *out, int blocks, void *stream) {
    if (!out || blocks < 1 || blocks > 1024) return -1;
    hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)blocks), dim3(64), 0,
                       static_cast<hipStream_t>(stream), out);
    return (int)hipGetLastError();
}

extern "C" int bi8clock_wall_rate_khz(int device) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) != hipSuccess) return 0;
    return khz;
}
