// merge.hip -- combine (O, lse) partials computed over disjoint key sets.
//
// The online-softmax fold of lesson 8 "Context Parallelism (CP)", section 3,
// applied to whole shards (the Helix article, phase 1, combines per-device
// partial attention results in one exchange):
//   M = max_p lse_p,  w_p = exp(lse_p - M),
//   lse = M + ln(sum_p w_p),  O = sum_p w_p O_p / sum_p w_p.
// One wave per row; lane j owns dims j, j+64.  The partial lse values of a
// row are read by all lanes (a broadcast), the O partials as coalesced rows.
// The same kernel merges the key-range splits of the prefill, whose LSE is
// laid out [B, Hq, rows].
#include "ra_device.h"

namespace ra {
namespace {

template <int D, bool LSE_BHQ>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
    constexpr int EPL = D / 64;  // elements per lane
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= p.rows) return;
    int64_t lrow = row;  // index of the row's lse
    if (LSE_BHQ) {
        const int64_t bq = row / p.Hq, h = row - bq * p.Hq;
        const int64_t b = bq / p.q_rows, q = bq - b * p.q_rows;
        lrow = (b * p.Hq + h) * p.q_rows + q;
    }

    float M = kNegInf;
    for (int q = 0; q < p.n_parts; ++q) M = fmaxf(M, p.lse_parts[(int64_t)q * p.rows + lrow]);

    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    float W = 0.f;
    if (M != kNegInf) {
        for (int q = 0; q < p.n_parts; ++q) {
            const float lq = p.lse_parts[(int64_t)q * p.rows + lrow];
            if (lq == kNegInf) continue;
            const float wq = __expf(lq - M);
            W += wq;
            const float* op = p.O_parts + ((int64_t)q * p.rows + row) * D;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(wq, op[lane + 64 * e], acc[e]);
        }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    if (p.out_bf16) {
        uint16_t* o = (uint16_t*)p.O + row * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[lane + 64 * e] = __builtin_bit_cast(uint16_t, (__bf16)(acc[e] * inv));
    } else {
        float* o = (float*)p.O + row * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[lane + 64 * e] = acc[e] * inv;
    }
    if (p.lse != nullptr && lane == 0) p.lse[lrow] = W > 0.f ? M + __logf(W) : kNegInf;
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int d, hipStream_t s) {
    const int64_t grid = (p.rows + 3) / 4;
    if (grid <= 0) return hipSuccess;
    if (p.lse_bhq) {
        if (d == 128)
            hipLaunchKernelGGL((merge_kernel<128, true>), dim3((unsigned)grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((merge_kernel<64, true>), dim3((unsigned)grid), dim3(256), 0, s, p);
    } else if (d == 128) {
        hipLaunchKernelGGL((merge_kernel<128, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
    } else {
        hipLaunchKernelGGL((merge_kernel<64, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace ra
