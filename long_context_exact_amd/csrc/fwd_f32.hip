// fwd_f32.hip -- blockwise ring-attention forward, fp32 inputs.
//
// Same ring visiting order, causal tile classes and online-softmax fold as
// the bf16 kernel (lesson 8 "Context Parallelism (CP)", sections 2-4), but
// every product and sum stays in fp32 so the result can be held to fp32
// accuracy.  Work-group: 64 queries x 4 threads per query; thread `part`
// owns head dimensions part, part+4, part+8, ... of its query's Q row and O
// accumulator.  Key/value tiles of 16 keys are staged in LDS.
#include "ra_device.h"

namespace ra {
namespace {

constexpr int BM = FWD_F32_BLOCK_M;  // 64 queries
constexpr int BN = 16;               // keys per tile
constexpr int NT = 256;

template <int D>
__global__ __launch_bounds__(NT) void fwd_f32_kernel(FwdParams p) {
    constexpr int DP = D / 4;  // dims per thread
    __shared__ float Ks[BN][D];
    __shared__ float Vs[BN][D];

    const unsigned split = blockIdx.x % (unsigned)p.kv_splits;
    const QTile qt = decode_qtile<BM>(p, blockIdx.x / (unsigned)p.kv_splits);
    const int t = threadIdx.x;
    const int qi = t >> 2, part = t & 3;
    const bool qvalid = qi < qt.rows;
    const int64_t qpos = qt.pos0 + qi;
    const int64_t qmax = qt.pos0 + qt.rows - 1;

    float q[DP], o[DP];
    const float* Qp = (const float*)p.Q + ((qt.b * p.q_rows + qt.q_row0 + qi) * p.Hq + qt.qh) * (int64_t)D;
#pragma unroll
    for (int e = 0; e < DP; ++e) {
        q[e] = qvalid ? Qp[4 * e + part] : 0.f;
        o[e] = 0.f;
    }
    float m_run = kNegInf, l_run = 0.f;

    const int64_t row_stride = (int64_t)p.Hkv * D;
    const float* Kg = (const float*)p.K + ((int64_t)qt.b * p.kv_rows * p.Hkv + qt.kvh) * D;
    const float* Vg = (const float*)p.V + ((int64_t)qt.b * p.kv_rows * p.Hkv + qt.kvh) * D;

    // this work-group's key range: tiles [i0, i0 + cnt) of the visiting order
    const int n_all = kv_count(p, qt.rank, qmax, BN);
    const int i0 = (int)(((int64_t)n_all * split) / p.kv_splits);
    int cnt = (int)(((int64_t)n_all * (split + 1)) / p.kv_splits) - i0;
    KvIter it;
    bool have = cnt > 0 && kv_first(p, qt.rank, qmax, BN, it);
    for (int k = 0; have && k < i0; ++k) have = kv_next(p, qt.rank, qmax, BN, it);
    while (have) {
        const int64_t r0 = it.krow + (int64_t)it.tile * BN;
        const int64_t kpos0 = it.kpos + (int64_t)it.tile * BN;
        const int64_t kleft = p.c - (int64_t)it.tile * BN;
        const int klen = kleft < BN ? (int)kleft : BN;
        __syncthreads();
        for (int idx = t; idx < BN * D / 4; idx += NT) {
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (row < klen) {
                kv = *(const float4*)(Kg + (r0 + row) * row_stride + 4 * c4);
                vv = *(const float4*)(Vg + (r0 + row) * row_stride + 4 * c4);
            }
            *(float4*)&Ks[row][4 * c4] = kv;
            *(float4*)&Vs[row][4 * c4] = vv;
        }
        __syncthreads();

        float s[BN];
        float mx = kNegInf;
#pragma unroll 4
        for (int j = 0; j < BN; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < DP; ++e) acc = __builtin_fmaf(q[e], Ks[j][4 * e + part], acc);
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            const bool ok = j < klen && (!p.causal || kpos0 + j <= qpos);
            s[j] = ok ? acc * p.scale_log2 : kNegInf;
            mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            s[j] = fast_exp2(s[j] - m_use);
            lsum += s[j];
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
#pragma unroll 8
        for (int e = 0; e < DP; ++e) {
            float acc = o[e] * alpha;
#pragma unroll
            for (int j = 0; j < BN; ++j) acc = __builtin_fmaf(s[j], Vs[j][4 * e + part], acc);
            o[e] = acc;
        }
        have = --cnt > 0 && kv_next(p, qt.rank, qmax, BN, it);
    }

    if (qvalid) {
        float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float lse = l_run > 0.f ? m_run * kLn2 + __logf(l_run) : kNegInf;
        float* Op = (float*)p.O + ((qt.b * p.q_rows + qt.q_row0 + qi) * p.Hq + qt.qh) * (int64_t)D +
                    (int64_t)split * p.o_split_stride;
        float* Lp = p.LSE + ((int64_t)qt.b * p.Hq + qt.qh) * p.q_rows + qt.q_row0 + qi +
                    (int64_t)split * p.l_split_stride;
        float w_old = 0.f;
        if (p.fold) {  // fold into the running state (lesson 8 section 3, whole blocks)
            const float lse_old = *Lp;
            const float M = fmaxf(lse_old, lse);
            if (M != kNegInf) {
                const float a = __expf(lse_old - M), b = __expf(lse - M);
                w_old = a / (a + b);
                inv *= b / (a + b);
                lse = M + __logf(a + b);
            }
        }
#pragma unroll
        for (int e = 0; e < DP; ++e)
            Op[4 * e + part] = p.fold ? __builtin_fmaf(w_old, Op[4 * e + part], o[e] * inv) : o[e] * inv;
        // all four threads of the query read the old LSE before the one that
        // writes it: the threads of a query are lanes of one wave, and the
        // store depends on the loaded value
        if (part == 0) *Lp = lse;
    }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t s) {
    const int64_t tiles = (int64_t)p.n_ranks * p.chunks_per_rank * p.tiles_per_chunk;
    const int64_t grid = tiles * p.B * p.Hq * p.kv_splits;
    if (grid <= 0) return hipSuccess;
    if (d == 128)
        hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace ra
