// stream_read.hip -- a plain streaming-read kernel: the HBM bandwidth a
// read-only kernel reaches on this GPU, the practical ceiling the decode
// kernel's rate is compared with.  Built as its own library (libkvq_probe.so);
// not part of the decode path or of its C ABI.
//
// Grid-stride 16-byte loads, U loads in flight per thread; every index is
// checked against the buffer length; one word per thread goes to `sink`, so
// the loads cannot be removed.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int NT = 256;
constexpr int U = 8;

__global__ void __launch_bounds__(NT) stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ sink)
{
    const size_t tid = (size_t)blockIdx.x * NT + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * NT;
    uint32_t acc = 0;
    for (size_t i0 = tid; i0 < n16; i0 += stride * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = i0 + (size_t)u * stride;
            v[u] = i < n16 ? p[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    sink[tid] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at `buf` (16-byte aligned, device) once
// with `blocks` workgroups of 256 threads on `stream`; sink (device) holds
// blocks * 256 words.  Returns 0, or -1 for invalid arguments, -7 when the
// launch fails.
int kvq_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream)
{
    if (!buf || !sink || blocks < 1 || bytes % 16 != 0 || ((uintptr_t)buf % 16) != 0) return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(NT), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
