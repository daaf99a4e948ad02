// Dynamic activation quantization ("Memory buffers": activations are
// quantized on the fly; the vector dot of "Q2_0 Format" runs against Q8_0
// activation tiles).  Per 32-element K block: d = amax/127 (IEEE fp32
// divide), q = round-half-away-from-zero(x * (1/d)), d stored as fp16
// (nearest-even) -- quant32() in tq_internal.h.  One block per 32 lanes.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int THREADS = 256;

template <int DT>
__global__ __launch_bounds__(THREADS) void k_quantize(const void *__restrict__ x, int64_t M,
                                                      int64_t nb, int64_t ldx,
                                                      int8_t *__restrict__ q,
                                                      uint16_t *__restrict__ d)
{
    const int64_t blk = (int64_t)blockIdx.x * (THREADS / 32) + (threadIdx.x >> 5);
    const int j = threadIdx.x & 31;
    if (blk >= M * nb)
        return;                      // uniform across the 32 lanes of a block
    const int64_t m = blk / nb, kt = blk - m * nb;
    int8_t qv;
    uint16_t db;
    quant32(load_x<DT>(x, m * ldx + kt * 32 + j), qv, db);
    q[m * nb * 32 + kt * 32 + j] = qv;
    if (j == 0)
        d[m * nb + kt] = db;
}

}  // namespace

hipError_t launch_quantize(int dtype, const void *x, int64_t M, int64_t K, int64_t ldx,
                           int8_t *q, uint16_t *d, hipStream_t s)
{
    const int64_t nb = K / 32;
    const int64_t blocks = M * nb;
    dim3 grid((unsigned)((blocks + THREADS / 32 - 1) / (THREADS / 32)));
    switch (dtype) {
    case TQ_F32: k_quantize<TQ_F32><<<grid, THREADS, 0, s>>>(x, M, nb, ldx, q, d); break;
    case TQ_BF16: k_quantize<TQ_BF16><<<grid, THREADS, 0, s>>>(x, M, nb, ldx, q, d); break;
    case TQ_F16: k_quantize<TQ_F16><<<grid, THREADS, 0, s>>>(x, M, nb, ldx, q, d); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tq
