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
//   * lds_probe: one wave reads LDS at per-lane word offsets from a table; run under rocprofv3
//     with SQ_LDS_BANK_CONFLICT, pairs of lanes that conflict show how the LDS groups the lanes
//     of an access into passes.
//   * mfma_chain: one wave per SIMD issues a dependent chain of MFMAs of one shape and times it
//     in shader cycles: the cycles one MFMA of that shape occupies the matrix pipe, the unit of
//     the ideal K-loop time in the phase profiles.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void empty_kernel() {}

// Four waves per workgroup; wave w of the grid issues n (a multiple of 8) MFMAs of shape `kind`
// (32: v_mfma_f32_32x32x2_f32, 16: v_mfma_f32_16x16x4_f32) as `ilp` interleaved dependent chains
// (1, 2 or 4 accumulators) and writes the shader cycles they took to cycles[w]; every lane writes
// a sum of its accumulators to sink, which keeps the chains from being optimised away.
template <int KIND, int ILP>
__device__ __attribute__((always_inline)) inline float mfma_chain_run(int n, float a, float b) {
    typedef typename std::conditional<KIND == 32, f32x16, f32x4>::type acc_t;
    acc_t acc[ILP];
#pragma unroll
    for (int c = 0; c < ILP; ++c) acc[c] = acc_t{};
    for (int i = 0; i < n; i += 8)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            acc_t& x = acc[u % ILP];
            if constexpr (KIND == 32)
                x = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, x, 0, 0, 0);
            else
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, x, 0, 0, 0);
        }
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < ILP; ++c)
#pragma unroll
        for (int r = 0; r < (KIND == 32 ? 16 : 4); ++r) sum += acc[c][r];
    return sum;
}

__global__ void __launch_bounds__(256) mfma_chain_kernel(int n, int kind, int ilp, unsigned long long* __restrict__ cycles,
                                                        float* __restrict__ sink) {
    const float a = (float)(threadIdx.x & 63) * 1e-3f, b = 1.0f;
    const unsigned long long t0 = clock64();
    float sum;
    if (kind == 32)
        sum = ilp == 1 ? mfma_chain_run<32, 1>(n, a, b) : ilp == 2 ? mfma_chain_run<32, 2>(n, a, b)
                                                                   : mfma_chain_run<32, 4>(n, a, b);
    else
        sum = ilp == 1 ? mfma_chain_run<16, 1>(n, a, b) : ilp == 2 ? mfma_chain_run<16, 2>(n, a, b)
                                                                   : mfma_chain_run<16, 4>(n, a, b);
    const unsigned long long t1 = clock64();
    if ((threadIdx.x & 63) == 0) cycles[blockIdx.x * 4 + (threadIdx.x >> 6)] = t1 - t0;
    sink[blockIdx.x * 256 + threadIdx.x] = sum;
}

// One wave: lane l reads `width` bytes (4, 8 or 16) of a 64 KiB LDS array at float offset idx[l]
// (clamped into the array and to the access's alignment), `reps` times, and writes a sum of what it
// read to out[l].  Each read waits for itself inside its asm block.
__global__ void __launch_bounds__(64) lds_probe_kernel(const int* __restrict__ idx, int width, int reps,
                                                       float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) float lds[16384];
    for (int i = threadIdx.x; i < 16384; i += 64) lds[i] = (float)i;
    __syncthreads();
    const int f = min(max(idx[threadIdx.x], 0), 16380) & ~3;
    const unsigned a = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) float*)(lds + f);
    float s = 0.f;
    for (int r = 0; r < reps; ++r) {
        if (width == 16) {
            f32x4 v;
            asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
            s += v.x + v.y + v.z + v.w;
        } else if (width == 8) {
            f32x2 v;
            asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
            s += v.x + v.y;
        } else {
            float v;
            asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
            s += v;
        }
    }
    out[threadIdx.x] = s;
}

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

// Launch the MFMA chains: nblocks workgroups of 4 waves (nblocks = the CU count gives one wave per
// SIMD), each wave n MFMAs of shape kind (32 or 16) in ilp (1, 2 or 4) interleaved dependent
// chains; cycles: device buffer of 4 * nblocks 64-bit values, sink: device buffer of 256 * nblocks
// floats.  Returns 0, -1 on invalid arguments, or the hipError_t of the launch.
__attribute__((visibility("default"))) int mfma_chain(int nblocks, int n, int kind, int ilp, unsigned long long* cycles,
                                                      float* sink, hipStream_t stream) {
    if (nblocks <= 0 || nblocks > 4096 || n <= 0 || n % 8 != 0 || n > (1 << 20) || (kind != 32 && kind != 16) ||
        (ilp != 1 && ilp != 2 && ilp != 4) || cycles == nullptr || sink == nullptr)
        return -1;
    void* args[] = {&n, &kind, &ilp, &cycles, &sink};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mfma_chain_kernel), dim3((unsigned)nblocks),
                                   dim3(256), args, 0, stream);
    return e == hipSuccess ? 0 : (int)e;
}

// Launch the LDS probe: one wave; idx: device table of 64 float offsets, out: device buffer of 64
// floats.  Returns 0, -1 on invalid arguments, or the hipError_t of the launch.
__attribute__((visibility("default"))) int lds_probe(const int* idx, int width, int reps, float* out,
                                                     hipStream_t stream) {
    if (idx == nullptr || out == nullptr || (width != 4 && width != 8 && width != 16) || reps <= 0 || reps > 4096)
        return -1;
    void* args[] = {&idx, &width, &reps, &out};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&lds_probe_kernel), dim3(1), dim3(64), args, 0, stream);
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
