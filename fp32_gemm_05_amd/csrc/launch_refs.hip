// launch_refs.hip -- two reference kernels of the bench, next to which the SGEMM kernels are
// measured.  Not part of libsgemm: built as liblaunch_refs.so and called only by bench.py and
// fp32_gemm_05_amd/profiling.py.
//
//   * launch_floor: an empty kernel launched with a given grid, workgroup size and LDS
//     allocation.  Timed back to back like the bench times a GEMM, it is the per-launch cost
//     of dispatching that grid at all -- the floor of a launch-latency bound GEMM.
//   * sclk_probe: reads the shader-clock counter (s_memtime) and the constant-rate real-time
//     counter (s_memrealtime) at the start and end of a bounded spin, so that their ratio gives
//     the engine clock at the moment the probe ran, on the stream it ran on.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

__global__ void empty_kernel() {}

// One lane per workgroup times a spin of `ticks` real-time ticks.  The loop ends once the
// real-time counter has advanced by `ticks`, which it always does.
__global__ void __launch_bounds__(64) sclk_probe_kernel(uint64_t ticks, unsigned long long* __restrict__ out) {
    if (threadIdx.x != 0) return;
    const uint64_t r0 = wall_clock64();
    const uint64_t c0 = clock64();
    uint64_t r1 = r0;
    while (r1 - r0 < ticks) r1 = wall_clock64();
    const uint64_t c1 = clock64();
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
}

}  // namespace

extern "C" {

// Launch an empty kernel of nwg workgroups of `threads` threads with lds_bytes of dynamic LDS
// each on `stream`.  Returns 0, -1 on invalid arguments, or the hipError_t of the launch.
__attribute__((visibility("default"))) int launch_floor(int nwg, int threads, int lds_bytes, hipStream_t stream) {
    if (nwg <= 0 || threads <= 0 || threads > 1024 || threads % 64 != 0 || lds_bytes < 0 ||
        lds_bytes > 160 * 1024)
        return -1;
    if (lds_bytes > 64 * 1024) {  // dynamic LDS above 64 KiB must be allowed explicitly
        hipError_t a = hipFuncSetAttribute(reinterpret_cast<const void*>(&empty_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
        if (a != hipSuccess) return (int)a;
    }
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&empty_kernel), dim3((unsigned)nwg),
                                   dim3((unsigned)threads), nullptr, (size_t)lds_bytes, stream);
    return e == hipSuccess ? 0 : (int)e;
}

// Launch the clock probe: nblocks workgroups (workgroup w runs on XCD w % 8), each spinning for
// `ticks` real-time ticks and writing (shader cycles, real-time ticks) of its spin to
// out[2w], out[2w + 1]; out is a device buffer of 2 * nblocks 64-bit values.  The engine clock is
// cycles / ticks * (real-time rate, hipDeviceAttributeWallClockRate).  Returns 0, -1 on invalid
// arguments, or the hipError_t of the launch.
__attribute__((visibility("default"))) int sclk_probe(int nblocks, long ticks, unsigned long long* out,
                                                      hipStream_t stream) {
    if (nblocks <= 0 || nblocks > 4096 || ticks <= 0 || ticks > 100000000L || out == nullptr) return -1;
    uint64_t t = (uint64_t)ticks;
    void* args[] = {&t, &out};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&sclk_probe_kernel), dim3((unsigned)nblocks),
                                   dim3(64), args, 0, stream);
    return e == hipSuccess ? 0 : (int)e;
}

// The real-time counter's rate in kHz on the current device (0 if unknown).
__attribute__((visibility("default"))) int wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

}  // extern "C"
