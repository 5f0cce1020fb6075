// Streaming-read probe: the HBM read rate this GPU sustains for a plain sequential read, the
// measured ceiling that the projection kernels' GB/s is compared with.  Not part of the
// projection path: built into its own library (libw4a16_probe.so) and called by the benchmark.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Every thread reads UNROLL 16-byte chunks per round, grid-stride over the buffer, and writes one
// word (the XOR of what it read) so the loads cannot be dropped.  chunks = bytes / 16; each
// thread's final write lands in sink[global thread index] (sink has gridDim * blockDim words).
template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, int64_t chunks,
                                                          uint32_t* __restrict__ sink) {
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    uint32_t acc = 0;
    int64_t i = tid;
    for (; i + (UNROLL - 1) * stride < chunks; i += UNROLL * stride) {
        u32x4_t v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < chunks; i += stride) {
        const u32x4_t v = src[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    sink[tid] = acc;
}

}  // namespace

extern "C" {

// Words the sink must hold for a launch of `blocks` workgroups (256 threads each).
int64_t w4a16_probe_sink_words(int blocks) { return static_cast<int64_t>(blocks) * 256; }

// Read `bytes` (a multiple of 16, 16-byte aligned) from device memory `src` once on `stream`;
// `sink` holds w4a16_probe_sink_words(blocks) words.  Returns 0, or 1 for invalid arguments, 7
// when the launch fails.
int w4a16_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int blocks, void* stream) {
    if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0 || blocks < 1)
        return 1;
    hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4_t*>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
