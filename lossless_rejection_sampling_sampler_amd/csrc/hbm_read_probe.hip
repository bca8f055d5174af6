// Streaming-read ceiling of the device, for context next to the verifier's
// throughput: a kernel reads a buffer once with 16-byte loads and folds it into
// one word per workgroup so the loads cannot be dropped.  Several layouts are
// offered so that the ceiling is the best the device shows, not one kernel's:
// grid-stride (consecutive threads of the whole grid on consecutive vectors) or
// one contiguous span per workgroup, 8 or 16 loads in flight per thread, and
// non-temporal or ordinary loads.  Not part of the verify ABI; the benchmark
// loads it from its own library (libhbmprobe.so).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <bool kNT>
__device__ __forceinline__ v4u load16(const v4u* p) {
    if (kNT) return __builtin_nontemporal_load(p);
    return *p;
}

// Grid-stride: thread t of the grid reads vectors t, t + N, t + 2N, ... (N =
// threads in the grid), kUnroll of them per round.
template <int kUnroll, bool kNT>
__global__ __launch_bounds__(kThreads) void read_stride(const v4u* __restrict__ p, long nvec, uint32_t* out) {
    const long nthreads = (long)gridDim.x * kThreads;
    long i = (long)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + (kUnroll - 1) * nthreads < nvec; i += kUnroll * nthreads) {
        v4u v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = load16<kNT>(p + i + u * nthreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < nvec; i += nthreads) {
        const v4u v = load16<kNT>(p + i);
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

// Span: workgroup w reads the contiguous vectors [w n / G, (w + 1) n / G), in
// rounds of kUnroll * 256 consecutive vectors.
template <int kUnroll, bool kNT>
__global__ __launch_bounds__(kThreads) void read_span(const v4u* __restrict__ p, long nvec, uint32_t* out) {
    const long a = (long)blockIdx.x * nvec / gridDim.x, e = (long)(blockIdx.x + 1) * nvec / gridDim.x;
    long i = a + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + (kUnroll - 1) * kThreads < e; i += kUnroll * kThreads) {
        v4u v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = load16<kNT>(p + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < e; i += kThreads) {
        const v4u v = load16<kNT>(p + i);
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

// Chunks: the buffer is cut into chunks of kUnroll * 256 vectors and workgroup
// w reads chunks w, w + G, w + 2G, ... (one contiguous chunk at a time, the
// grid together on a contiguous window).
template <int kUnroll, bool kNT>
__global__ __launch_bounds__(kThreads) void read_chunks(const v4u* __restrict__ p, long nvec, uint32_t* out) {
    constexpr long C = (long)kUnroll * kThreads;
    uint32_t acc = 0u;
    for (long c0 = (long)blockIdx.x * C; c0 < nvec; c0 += (long)gridDim.x * C) {
        const long i = c0 + threadIdx.x;
        if (c0 + C <= nvec) {
            v4u v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) v[u] = load16<kNT>(p + i + u * kThreads);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        } else {
            for (long j = i; j < nvec; j += kThreads) {
                const v4u v = load16<kNT>(p + j);
                acc ^= v.x ^ v.y ^ v.z ^ v.w;
            }
        }
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

typedef void (*Kern)(const v4u*, long, uint32_t*);

// mode 0..7: bit 0 span (else grid-stride), bit 1 ordinary loads (else
// non-temporal), bit 2 16 loads in flight per thread (else 8); mode 8 / 9:
// chunks of 8 / 16 non-temporal loads per thread.
Kern kernel_for(int mode) {
    if (mode == 8) return read_chunks<8, true>;
    if (mode == 9) return read_chunks<16, true>;
    switch (mode & 7) {
        case 0: return read_stride<8, true>;
        case 1: return read_span<8, true>;
        case 2: return read_stride<8, false>;
        case 3: return read_span<8, false>;
        case 4: return read_stride<16, true>;
        case 5: return read_span<16, true>;
        case 6: return read_stride<16, false>;
        default: return read_span<16, false>;
    }
}

bool args_ok(const void* buf, long bytes, const uint32_t* out, int grid) {
    return buf && out && bytes > 0 && bytes % 16 == 0 && reinterpret_cast<uintptr_t>(buf) % 16 == 0 && grid >= 1;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned) at device address `buf`
// with `grid` workgroups of 256 threads on `stream` (grid-stride, 8
// non-temporal loads per thread); `out` holds `grid` words.  Returns 0, or 1
// for bad arguments, 3 for a launch failure.
int hbm_read_probe(const void* buf, long bytes, uint32_t* out, int grid, void* stream) {
    if (!args_ok(buf, bytes, out, grid)) return 1;
    hipLaunchKernelGGL((read_stride<8, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const v4u*>(buf), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

// Times `reps` launches of layout `mode` (0..9, see kernel_for) on the null
// stream after `warmup` untimed ones; *ms receives the mean kernel duration
// from events the dispatches stamp themselves.  Synchronous.  Returns 0, 1 for
// bad arguments, 3 for a HIP failure.
int hbm_read_probe_time(const void* buf, long bytes, uint32_t* out, int grid, int mode, int warmup, int reps,
                        float* ms) {
    if (!args_ok(buf, bytes, out, grid) || mode < 0 || mode > 9 || warmup < 0 || reps < 1 || !ms) return 1;
    const Kern k = kernel_for(mode);
    const v4u* p = static_cast<const v4u*>(buf);
    for (int w = 0; w < warmup; ++w) hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kThreads), 0, 0, p, bytes / 16, out);
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 3;
    double total = 0.0;
    int st = 0;
    for (int r = 0; r < reps && st == 0; ++r) {
        hipExtLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kThreads), 0, 0, a, b, 0, p, bytes / 16, out);
        float t = 0.f;
        if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&t, a, b) != hipSuccess) st = 3;
        total += t;
    }
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    if (st) return st;
    *ms = static_cast<float>(total / reps);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
