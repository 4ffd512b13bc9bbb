// hbm_read.hip -- a streaming-read kernel used as the read-bandwidth reference of the
// profiling summaries (what a plain read of a buffer reaches on this GPU), next to which the
// HBM-bound SGEMM workload is judged.  Not part of libsgemm: built as libhbm_read.so and
// called only by fp32_gemm_05_amd/profiling.py.
#include <hip/hip_runtime.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;  // 128-bit loads in flight per thread

// Workgroup w reads the contiguous chunk [w * chunk, (w + 1) * chunk) of n 16-byte elements,
// kInFlight loads per thread at a time, and writes one partial sum per thread (so that the
// loads cannot be dropped).
__global__ void __launch_bounds__(kThreads) hbm_read_kernel(const f32x4* __restrict__ p, long n, long chunk,
                                                             float* __restrict__ out) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const long b = (long)blockIdx.x * chunk;
    const long e = b + chunk < n ? b + chunk : n;
    long i = b + threadIdx.x;
    for (; i + (kInFlight - 1) * kThreads < e; i += kInFlight * kThreads) {
        f32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) v[u] = p[i + u * kThreads];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc += v[u];
    }
    for (; i < e; i += kThreads) acc += p[i];
    out[(long)blockIdx.x * kThreads + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

long chunk_elems(int chunk_kib) { return (long)chunk_kib * 1024 / 16; }

}  // namespace

extern "C" {

// Workgroups of one read of `bytes` in chunks of chunk_kib KiB; the `out` buffer of hbm_read
// needs 256 floats per workgroup.  Returns -1 on invalid arguments.
__attribute__((visibility("default"))) long hbm_read_workgroups(long bytes, int chunk_kib) {
    if (bytes <= 0 || bytes % 16 != 0 || chunk_kib <= 0) return -1;
    const long n = bytes / 16, c = chunk_elems(chunk_kib);
    return (n + c - 1) / c;
}

// Read `bytes` bytes at device address buf (16-byte aligned, bytes a multiple of 16) on
// `stream`; out: device buffer of 256 * hbm_read_workgroups(bytes, chunk_kib) floats.
// Returns 0, -1 on invalid arguments, or the hipError_t of the launch.
__attribute__((visibility("default"))) int hbm_read(const void* buf, long bytes, int chunk_kib, float* out,
                                                    hipStream_t stream) {
    const long nwg = hbm_read_workgroups(bytes, chunk_kib);
    if (nwg <= 0 || nwg > 0x7fffffffL || buf == nullptr || out == nullptr ||
        (reinterpret_cast<unsigned long>(buf) & 15u) != 0)
        return -1;
    const f32x4* p = static_cast<const f32x4*>(buf);
    long n = bytes / 16, chunk = chunk_elems(chunk_kib);
    void* args[] = {&p, &n, &chunk, &out};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&hbm_read_kernel), dim3((unsigned)nwg),
                                   dim3(kThreads), args, 0, stream);
    return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
