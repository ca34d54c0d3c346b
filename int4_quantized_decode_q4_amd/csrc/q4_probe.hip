// q4_probe.hip -- a plain streaming read of device memory, the measurement
// ceiling the int4 matmuls are compared against.
//
// The benchmark protocol of the Zero-TVM article ("Zero-TVM：手写 WGSL 着色器在
// 浏览器中运行 Phi-3-mini，挑战编译器霸权", section 性能基准) keeps raw data
// beside each figure; on MI355X the useful context for an HBM-bound kernel is
// what a kernel that only reads the same number of bytes achieves in one
// launch.  This kernel does nothing but that: each 64-lane wavefront reads
// 1 KiB per load instruction (16 bytes per lane, fully coalesced) through a
// buffer resource, keeps two chunks of kProbeUnits loads in flight, and
// folds every word into an xor so no load is dead; each block writes its one
// word to `sink`.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_internal.h"

namespace q4 {

namespace {

constexpr int kProbeUnits = 8;            // 1 KiB loads per chunk per wavefront
constexpr int kProbeChunk = kProbeUnits * 1024;
constexpr int kProbeWaves = 4;            // wavefronts per block
constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer format

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const uint8_t *base, int64_t c,
                                                             int64_t bytes)
{
    // chunks past the end (and the tail past `bytes`) read as zeros
    const int64_t off = c * kProbeChunk;
    const int64_t left = bytes - off;
    const int n = left <= 0 ? 0 : (left < kProbeChunk ? (int)left : kProbeChunk);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base + (n ? off : 0)), (short)0,
                                             n, kBufferWord3);
}

__global__ __launch_bounds__(64 * kProbeWaves) void read_probe_kernel(const uint8_t *__restrict__ src,
                                                                      int64_t bytes, int64_t chunks,
                                                                      uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t step = (int64_t)gridDim.x * kProbeWaves;
    int64_t c = (int64_t)blockIdx.x * kProbeWaves + w;
    v4u a[kProbeUnits], b[kProbeUnits];
    uint32_t acc = 0;
    {
        const __amdgpu_buffer_rsrc_t r = chunk_rsrc(src, c, bytes);
#pragma unroll
        for (int i = 0; i < kProbeUnits; ++i)
            a[i] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, i * 1024, 0);
    }
    while (c < chunks) {
        {
            const __amdgpu_buffer_rsrc_t r = chunk_rsrc(src, c + step, bytes);
#pragma unroll
            for (int i = 0; i < kProbeUnits; ++i) {
                b[i] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, i * 1024, 0);
                acc ^= a[i].x ^ a[i].y ^ a[i].z ^ a[i].w;
            }
            c += step;
        }
        if (c >= chunks)
            break;
        {
            const __amdgpu_buffer_rsrc_t r = chunk_rsrc(src, c + step, bytes);
#pragma unroll
            for (int i = 0; i < kProbeUnits; ++i) {
                a[i] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, i * 1024, 0);
                acc ^= b[i].x ^ b[i].y ^ b[i].z ^ b[i].w;
            }
            c += step;
        }
    }
    // one word per block: the xor of everything its wavefronts read
    __shared__ uint32_t part[kProbeWaves];
    for (int off = 32; off >= 1; off >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if (lane == 0)
        part[w] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int i = 0; i < kProbeWaves; ++i)
            t ^= part[i];
        sink[blockIdx.x] = t;
    }
}

}  // namespace

int64_t read_probe_blocks(int64_t bytes, int cus)
{
    const int64_t chunks = (bytes + kProbeChunk - 1) / kProbeChunk;
    const int64_t groups = (chunks + kProbeWaves - 1) / kProbeWaves;
    const int64_t cap = 2 * (int64_t)cus;   // two blocks of four wavefronts per CU
    return groups < cap ? (groups > 0 ? groups : 1) : cap;
}

hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, int cus,
                             hipStream_t stream)
{
    const int64_t chunks = (bytes + kProbeChunk - 1) / kProbeChunk;
    const int64_t blocks = read_probe_blocks(bytes, cus);
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(64 * kProbeWaves), 0, stream,
                       static_cast<const uint8_t *>(src), bytes, chunks, sink);
    return hipGetLastError();
}

}  // namespace q4
