// Streaming-read ceiling of the device, for context next to the verifier's
// throughput: one kernel reads a buffer once with 16-byte non-temporal loads
// (the load form the rows kernel uses) and folds it into one word per
// workgroup so the loads cannot be dropped.  Not part of the verify ABI; the
// benchmark loads it from its own library (libhbmprobe.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void read_kernel(const v4u* __restrict__ p, long nvec, uint32_t* out) {
    const long nthreads = (long)gridDim.x * kThreads;
    long i = (long)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + (kUnroll - 1) * nthreads < nvec; i += kUnroll * nthreads) {
        v4u v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * nthreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < nvec; i += nthreads) {
        const v4u v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t s[kThreads];
    s[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0u;
        for (int k = 0; k < kThreads; ++k) r ^= s[k];
        out[blockIdx.x] = r;
    }
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned) at device address `buf`
// with `grid` workgroups of 256 threads on `stream`; `out` holds `grid` words.
// Returns 0, or 1 for bad arguments, 3 for a launch failure.
int hbm_read_probe(const void* buf, long bytes, uint32_t* out, int grid, void* stream) {
    if (!buf || !out || bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16 || grid < 1) return 1;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const v4u*>(buf), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
