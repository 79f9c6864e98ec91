// merge.hip -- combine (O, lse) partials computed over disjoint key sets.
//
// The online-softmax fold of lesson 8 "Context Parallelism (CP)", section 3,
// applied to whole shards (the Helix article, phase 1, combines per-device
// partial attention results in one exchange):
//   M = max_p lse_p,  w_p = exp(lse_p - M),
//   lse = M + ln(sum_p w_p),  O = sum_p w_p O_p / sum_p w_p.
// One wave per row; lane j owns dims j, j+64.  The parts' lse values are
// read 64 at a time, one per lane, and reduced across the wave; the O
// partials are read as coalesced rows, eight parts in flight.
// The same kernel merges the key-range splits of the prefill, whose LSE is
// laid out [B, Hq, rows], and, for a split ring step, folds them into the
// running state as one more part (the state first), in place: every lane of
// a row reads the row's state before the row's wave writes it.
#include "ra_device.h"

namespace ra {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

template <int D, bool LSE_BHQ>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
    constexpr int EPL = D / 64;  // elements per lane
    constexpr int U = 8;         // partial rows in flight per lane
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= p.rows) return;
    int64_t lrow = row;  // index of the row's lse
    if (LSE_BHQ) {
        const int64_t bq = row / p.Hq, h = row - bq * p.Hq;
        const int64_t b = bq / p.q_rows, q = bq - b * p.q_rows;
        lrow = (b * p.Hq + h) * p.q_rows + q;
    }

    // the parts' lse values, 64 at a time, one per lane (and the state's)
    const float ls = p.lse_state != nullptr ? p.lse_state[lrow] : kNegInf;
    float M = kNegInf;
    for (int q0 = 0; q0 < p.n_parts; q0 += 64) {
        const int q = q0 + lane;
        M = fmaxf(M, q < p.n_parts ? p.lse_parts[(int64_t)q * p.rows + lrow] : kNegInf);
    }
    M = wave_max(M);
    // no part has a key: a running state stays as it is
    if (M == kNegInf && p.lse_state != nullptr) return;
    M = fmaxf(M, ls);

    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    float W = 0.f;
    if (M != kNegInf) {
        if (ls != kNegInf) {  // the state first
            const float ws = __expf(ls - M);
            const float* op = p.O_state + row * D;
            W = ws;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] = ws * op[lane + 64 * e];
        }
        for (int q0 = 0; q0 < p.n_parts; q0 += 64) {
            const int q = q0 + lane;
            const float lq = q < p.n_parts ? p.lse_parts[(int64_t)q * p.rows + lrow] : kNegInf;
            const float wl = lq == kNegInf ? 0.f : __expf(lq - M);  // this lane's part weight
            W += wave_sum(wl);
            const int cnt = min(64, p.n_parts - q0);
            // U independent partial rows in flight; parts of weight 0 read
            // nothing (an empty part's O may be anything finite)
            for (int j0 = 0; j0 < cnt; j0 += U) {
                float wq[U], v[U][EPL];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int j = j0 + u;
                    wq[u] = __shfl(wl, j < cnt ? j : 0, 64);
                    if (j >= cnt) wq[u] = 0.f;
                    const float* op = p.O_parts + ((int64_t)(q0 + j) * p.rows + row) * D;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) v[u][e] = wq[u] != 0.f ? op[lane + 64 * e] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(wq[u], v[u][e], acc[e]);
            }
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

// Few parts (the key-range splits of the prefill, 2-8 ranges): a group of
// D/4 lanes per row, each lane owning 4 consecutive dims, so a wave merges
// 256/D rows at once with all of a row's loads independent and no wave-wide
// reductions.  Parts are folded in order, as above.
constexpr int MERGE_FEW_MAX = 8;

template <int D, bool LSE_BHQ>
__global__ __launch_bounds__(256) void merge_few_kernel(MergeParams p) {
    constexpr int LPR = D / 4;  // lanes per row
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
    const int sub = threadIdx.x % LPR;
    if (row >= p.rows) return;
    int64_t lrow = row;
    if (LSE_BHQ) {
        const int64_t bq = row / p.Hq, h = row - bq * p.Hq;
        const int64_t b = bq / p.q_rows, q = bq - b * p.q_rows;
        lrow = (b * p.Hq + h) * p.q_rows + q;
    }
    float lq[MERGE_FEW_MAX];
    float M = kNegInf;
#pragma unroll
    for (int q = 0; q < MERGE_FEW_MAX; ++q) {
        lq[q] = q < p.n_parts ? p.lse_parts[(int64_t)q * p.rows + lrow] : kNegInf;
        M = fmaxf(M, lq[q]);
    }
    // no part has a key: a running state stays as it is
    if (M == kNegInf && p.lse_state != nullptr) return;
    const float ls = p.lse_state != nullptr ? p.lse_state[lrow] : kNegInf;
    M = fmaxf(M, ls);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float W = 0.f;
    if (M != kNegInf) {
        if (ls != kNegInf) {  // the state first
            const float ws = __expf(ls - M);
            const float4 s4 = *(const float4*)(p.O_state + row * D + 4 * sub);
            W = ws;
            acc = make_float4(ws * s4.x, ws * s4.y, ws * s4.z, ws * s4.w);
        }
        float w[MERGE_FEW_MAX];
        float4 v[MERGE_FEW_MAX];
#pragma unroll
        for (int q = 0; q < MERGE_FEW_MAX; ++q) {
            w[q] = lq[q] == kNegInf ? 0.f : __expf(lq[q] - M);
            v[q] = w[q] != 0.f ? *(const float4*)(p.O_parts + ((int64_t)q * p.rows + row) * D + 4 * sub)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int q = 0; q < MERGE_FEW_MAX; ++q) {
            W += w[q];
            acc.x = __builtin_fmaf(w[q], v[q].x, acc.x);
            acc.y = __builtin_fmaf(w[q], v[q].y, acc.y);
            acc.z = __builtin_fmaf(w[q], v[q].z, acc.z);
            acc.w = __builtin_fmaf(w[q], v[q].w, acc.w);
        }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    if (p.out_bf16) {
        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.x * inv)) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.y * inv)) << 16);
        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.z * inv)) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.w * inv)) << 16);
        *(uint2*)((uint16_t*)p.O + row * D + 4 * sub) = make_uint2(lo, hi);
    } else {
        *(float4*)((float*)p.O + row * D + 4 * sub) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (p.lse != nullptr && sub == 0) p.lse[lrow] = W > 0.f ? M + __logf(W) : kNegInf;
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int d, hipStream_t s) {
    if (p.rows <= 0) return hipSuccess;
    // the few-parts path moves 16-byte (O partials, fp32 O) or 8-byte (bf16 O) units
    const bool aligned = ((uintptr_t)p.O_parts | (uintptr_t)p.O | (uintptr_t)p.O_state) % 16 == 0;
    if (p.n_parts <= MERGE_FEW_MAX && aligned) {
        const int64_t grid = (p.rows * (d / 4) + 255) / 256;
        if (p.lse_bhq) {
            if (d == 128)
                hipLaunchKernelGGL((merge_few_kernel<128, true>), dim3((unsigned)grid), dim3(256), 0, s, p);
            else
                hipLaunchKernelGGL((merge_few_kernel<64, true>), dim3((unsigned)grid), dim3(256), 0, s, p);
        } else if (d == 128) {
            hipLaunchKernelGGL((merge_few_kernel<128, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
        } else {
            hipLaunchKernelGGL((merge_few_kernel<64, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
        }
        return hipGetLastError();
    }
    const int64_t grid = (p.rows + 3) / 4;
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
