// Dynamic activation quantization ("Memory buffers": activations are
// quantized on the fly; the vector dot of "Q2_0 Format" runs against Q8_0
// activation tiles).  Per 32-element K block: d = amax/127 (IEEE fp32
// divide), q = round-half-away-from-zero(x * (1/d)), d stored as fp16
// (nearest-even) -- quant_quad() in tq_internal.h.  One block per quad of
// lanes, 8 consecutive elements per lane.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int THREADS = 256;
constexpr int BPW = THREADS / 4;     // blocks per workgroup: one quad of lanes each

template <int DT>
__global__ __launch_bounds__(THREADS) void k_quantize(const void *__restrict__ x, int64_t M,
                                                      int64_t nb, int64_t ldx,
                                                      int8_t *__restrict__ q,
                                                      uint16_t *__restrict__ d)
{
    const int64_t blk = (int64_t)blockIdx.x * BPW + (threadIdx.x >> 2);
    const int c = threadIdx.x & 3;
    if (blk >= M * nb)
        return;                      // uniform across the quad of a block
    const int64_t m = blk / nb, kt = blk - m * nb;
    float v[8];
    load_x8<DT>(v, x, m * ldx + kt * 32 + 8 * c);
    uint2 qv;
    uint16_t db;
    quant_quad(v, qv, db);
    *(u32x2u *)(q + m * nb * 32 + kt * 32 + 8 * c) = u32x2u{qv.x, qv.y};
    if (c == 0)
        d[m * nb + kt] = db;
}

}  // namespace

hipError_t launch_quantize(int dtype, const void *x, int64_t M, int64_t K, int64_t ldx,
                           int8_t *q, uint16_t *d, hipStream_t s)
{
    const int64_t nb = K / 32;
    const int64_t blocks = M * nb;
    if (!grid_fits((blocks + BPW - 1) / BPW, THREADS))
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)((blocks + BPW - 1) / BPW));
    switch (dtype) {
    case TQ_F32: k_quantize<TQ_F32><<<grid, THREADS, 0, s>>>(x, M, nb, ldx, q, d); break;
    case TQ_BF16: k_quantize<TQ_BF16><<<grid, THREADS, 0, s>>>(x, M, nb, ldx, q, d); break;
    case TQ_F16: k_quantize<TQ_F16><<<grid, THREADS, 0, s>>>(x, M, nb, ldx, q, d); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tq
