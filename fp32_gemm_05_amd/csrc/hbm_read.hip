// hbm_read.hip -- a streaming-read kernel used as the read-bandwidth reference of the
// profiling summaries (what a plain read of a buffer reaches on this GPU), next to which the
// HBM-bound SGEMM workload is compared, and a write of a matrix in the order in which the MFMA
// epilogue stores C (the write reference of the store-heavy shapes).  Not part of libsgemm:
// built as libhbm_read.so and called only by fp32_gemm_05_amd/profiling.py.
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

// Workgroup b writes the 64x64 tile (b / tiles_n, b % tiles_n) of the M x N matrix c (row
// stride ldc) the way the 32x32x2 MFMA epilogue stores it: wave w owns the 32x32 block
// (w / 2, w % 2), and value i of lane l goes to row 8 * (i / 4) + 4 * (l / 32) + i % 4 and
// column l % 32 of the block; NT selects nontemporal stores.
template <bool NT>
__global__ void __launch_bounds__(kThreads) tile_write_kernel(float* __restrict__ c, int ldc, int tiles_n,
                                                               float v) {
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int w = threadIdx.x / 64, l = threadIdx.x % 64;
    const long r0 = (long)tm * 64 + (w / 2) * 32;
    const long c0 = (long)tn * 64 + (w % 2) * 32 + l % 32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const long r = r0 + 8 * (i / 4) + 4 * (l / 32) + i % 4;
        const float x = v + (float)i;
        if (NT)
            __builtin_nontemporal_store(x, c + r * ldc + c0);
        else
            c[r * ldc + c0] = x;
    }
}

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

// Write the M x N matrix at device address c (row stride ldc floats) in 64x64 tiles in the MFMA
// epilogue's store order, with nontemporal stores when nt != 0.  M and N must be positive
// multiples of 64 with N <= ldc and (M / 64) * (N / 64) < 2^31.  Returns 0, -1 on invalid
// arguments, or the hipError_t of the launch.
__attribute__((visibility("default"))) int hbm_write_tiles(float* c, int M, int N, int ldc, int nt,
                                                           hipStream_t stream) {
    if (c == nullptr || M <= 0 || N <= 0 || M % 64 != 0 || N % 64 != 0 || N > ldc) return -1;
    const long nwg = (long)(M / 64) * (N / 64);
    if (nwg > 0x7fffffffL) return -1;
    int tiles_n = N / 64;
    float v = 1.0f;
    void* args[] = {&c, &ldc, &tiles_n, &v};
    const void* k = nt ? reinterpret_cast<const void*>(&tile_write_kernel<true>)
                       : reinterpret_cast<const void*>(&tile_write_kernel<false>);
    hipError_t e = hipLaunchKernel(k, dim3((unsigned)nwg), dim3(kThreads), args, 0, stream);
    return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
