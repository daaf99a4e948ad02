// Measurement instrument: a plain streaming read of a device buffer, the
// achievable HBM read rate that the decode's weight stream is set against.
//
// Grid-stride loop over 16-byte chunks with nontemporal loads (the decode
// streams its tiles the same way), one load per work-item per iteration, a
// fixed grid of TQ_STREAM_READ_BLOCKS workgroups of 256 work-items.  That
// shape was the fastest of a sweep over grids of 128 - 8192 workgroups, 256
// - 1024 work-items and 1 - 8 loads in flight per work-item on 18 - 33 MB
// buffers.  Each workgroup writes the XOR of the 32-bit words it read, so the
// loads have a defined use and the result can be checked.
#include <hip/hip_runtime.h>

#include "tiledq.h"

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int THREADS = 256;

__global__ __launch_bounds__(THREADS) void k_stream_read(const v4u *__restrict__ src, int64_t n16,
                                                         uint32_t *__restrict__ sink)
{
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n16; i += stride) {
        const v4u v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int o = 32; o > 0; o >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    __shared__ uint32_t wave_acc[THREADS / 64];
    if ((threadIdx.x & 63) == 0)
        wave_acc[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < THREADS / 64; w++)
            r ^= wave_acc[w];
        sink[blockIdx.x] = r;
    }
}

}  // namespace

extern "C" int tq_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (bytes % 16 != 0)
        return TQ_E_SHAPE;
    if (bytes == 0)
        return TQ_OK;
    if (!src || !sink)
        return TQ_E_NULL;
    if ((uintptr_t)src % 16 != 0 || (uintptr_t)sink % 4 != 0)
        return TQ_E_ALIGN;
    k_stream_read<<<TQ_STREAM_READ_BLOCKS, THREADS, 0, stream>>>((const v4u *)src,
                                                                (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_E_LAUNCH;
}
