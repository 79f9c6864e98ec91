// decode.hip -- per-shard partial attention of a few query tokens against a
// KV cache split along the sequence (the Helix article's phase 1: each device
// holds a slice of the cache and produces a partial result that one exchange
// later combines).  Output per part: O_p normalised by its own denominator
// and lse_p = m_p + ln l_p, which is exactly what the merge needs.
//
// bf16 kernel: one work-group per (batch, kv head, part).  The Sq x G query
// rows that read this kv head form the 32 MFMA columns (unused columns carry
// zero queries and are never stored).  The part's keys stream through LDS in
// stages of 128 (two 64-key tiles, double-buffered); each of the 4 waves
// takes 32 keys of a stage and keeps its own (m, l, O) state; the four states
// are merged through LDS at the end.  The kernel is bound by HBM: every K/V
// byte is read exactly once.
#include "attn_tile.h"

namespace ra {
namespace {

constexpr int NT = 256;
constexpr int BN = 64;       // keys per tile
constexpr int STAGE = 128;   // keys per stage (two tiles)

template <int D>
__global__ __launch_bounds__(NT) void decode_bf16_kernel(DecodeParams p) {
    using T = Tile<D, BN, NT>;
    constexpr int KB = D / 16, DB = D / 32;
    // [buffer][tile][K | V^T]; reused as fp32 scratch for the final merge
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][2 * T::ELEMS];
    static_assert(sizeof(lds) >= sizeof(float) * (4 * D * 32 + 8 * 32), "merge scratch");

    const int part = blockIdx.x % p.n_parts;
    const int pair = blockIdx.x / p.n_parts;
    const int b = pair / p.Hkv, kvh = pair % p.Hkv;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int h = lane >> 5, m = lane & 31;
    const int R = (int)p.Sq * p.G;

    // MFMA column m <-> query row (position i, head kvh*G + g)
    const bool cvalid = m < R;
    const int ci = cvalid ? m / p.G : 0, cg = cvalid ? m % p.G : 0;
    bf16x8 qop[KB];
    {
        const uint16_t* qp = (const uint16_t*)p.Q +
                             (((int64_t)b * p.Sq + ci) * p.Hq + (int64_t)kvh * p.G + cg) * D;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            uint4 u = cvalid ? *(const uint4*)(qp + kb * 16 + h * 8) : make_uint4(0, 0, 0, 0);
            qop[kb] = __builtin_bit_cast(bf16x8, u);
        }
    }

    int64_t k0 = (int64_t)part * p.part_len;
    int64_t k1 = k0 + p.part_len;
    if (k1 > p.Skv) k1 = p.Skv;
    if (k0 > k1) k0 = k1;
    const int64_t nstages = (k1 - k0 + STAGE - 1) / STAGE;

    const int64_t row_stride = (int64_t)p.Hkv * D;
    const uint16_t* Kg = (const uint16_t*)p.K + ((int64_t)b * p.Skv * p.Hkv + kvh) * D;
    const uint16_t* Vg = (const uint16_t*)p.V + ((int64_t)b * p.Skv * p.Hkv + kvh) * D;

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    typename T::Regs regs[2];
    auto tile_len = [&](int64_t st, int a) -> int {
        const int64_t left = k1 - (k0 + st * STAGE + a * BN);
        return left <= 0 ? 0 : (left < BN ? (int)left : BN);
    };
    auto load_stage = [&](int64_t st) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int64_t r0 = k0 + st * STAGE + a * BN;
            T::load(regs[a], Kg + r0 * row_stride, Vg + r0 * row_stride, row_stride, tile_len(st, a),
                    threadIdx.x);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int a = 0; a < 2; ++a) T::store(regs[a], lds[buf][a], lds[buf][a] + T::ELEMS, threadIdx.x);
    };

    if (nstages > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();

    const int a = w >> 1, kb2 = w & 1;  // this wave's tile and 32-key half
    int buf = 0;
    for (int64_t st = 0; st < nstages; ++st) {
        const bool nxt = st + 1 < nstages;
        if (nxt) load_stage(st + 1);
        const int klen = tile_len(st, a);
        if (klen > kb2 * 32) {
            const uint16_t* Ks = lds[buf][a];
            const uint16_t* Vts = lds[buf][a] + T::ELEMS;
            f32x16 sacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
            const int row = kb2 * 32 + swap_bits23(m);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 av = *(const bf16x8*)(Ks + T::k_off(row, kb * 2 + h));
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qop[kb], sacc, 0, 0, 0);
            }
            if (klen < BN) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kidx = kb2 * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
                    if (kidx >= klen) sacc[r] = kNegInf;
                }
            }
            float mx = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
            mx = xor32_max(mx);
            const float m_new = fmaxf(m_run, mx * p.scale_log2);
            const float m_use = m_new == kNegInf ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            float lsum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(__builtin_fmaf(sacc[r], p.scale_log2, -m_use));
                sacc[r] = e;
                lsum += e;
            }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            bf16x8 pb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int i = 0; i < 8; ++i) pb[kk][i] = (__bf16)sacc[8 * kk + i];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int dim = db * 32 + m;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 av = *(const bf16x8*)(Vts + T::vt_off(dim, 2 * (2 * kb2 + kk) + h));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kk], oacc[db], 0, 0, 0);
                }
            }
        }
        if (nxt) store_stage(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }

    // ---- merge the four waves' states, then write this part's (O, lse)
    const float l_tot = xor32_sum(l_run);
    float* scratch = (float*)&lds[0][0][0];
    float* Ow = scratch;                 // [4][D][32]
    float* mw = scratch + 4 * D * 32;    // [4][32]
    float* lw = mw + 4 * 32;             // [4][32]
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dim = db * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            Ow[(w * D + dim) * 32 + m] = oacc[db][r];
        }
    if (h == 0) {
        mw[w * 32 + m] = m_run;
        lw[w * 32 + m] = l_tot;
    }
    __syncthreads();
    {
        const int n = threadIdx.x & 31;       // column
        const int dg = threadIdx.x >> 5;      // group of D/8 dims
        constexpr int DPT = D / 8;
        if (n < R) {
            float M = kNegInf;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mw[ww * 32 + n]);
            float sc[4];
            float W = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                sc[ww] = M == kNegInf ? 0.f : fast_exp2(mw[ww * 32 + n] - M);
                W += lw[ww * 32 + n] * sc[ww];
            }
            const float inv = W > 0.f ? 1.f / W : 0.f;
            const int i = n / p.G, g = n % p.G;
            const int64_t row = ((int64_t)b * p.Sq + i) * p.Hq + (int64_t)kvh * p.G + g;
            const int64_t rows = (int64_t)p.B * p.Sq * p.Hq;
            float* op = p.O_parts + ((int64_t)part * rows + row) * D + dg * DPT;
#pragma unroll
            for (int e = 0; e < DPT; e += 4) {
                float4 v;
                float* vv = (float*)&v;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int dim = dg * DPT + e + q;
                    float acc = 0.f;
#pragma unroll
                    for (int ww = 0; ww < 4; ++ww) acc += Ow[(ww * D + dim) * 32 + n] * sc[ww];
                    vv[q] = acc * inv;
                }
                *(float4*)(op + e) = v;
            }
            if (dg == 0)
                p.lse_parts[(int64_t)part * rows + row] = W > 0.f ? (M + __log2f(W)) * kLn2 : kNegInf;
        }
    }
}

// fp32 inputs: plain VALU kernel, 4 threads per query row (thread `part4`
// owns dims part4, part4+4, ...), 16 keys per LDS tile.
template <int D>
__global__ __launch_bounds__(128) void decode_f32_kernel(DecodeParams p) {
    constexpr int DP = D / 4, BK = 16;
    __shared__ float Ks[BK][D];
    __shared__ float Vs[BK][D];
    const int part = blockIdx.x % p.n_parts;
    const int pair = blockIdx.x / p.n_parts;
    const int b = pair / p.Hkv, kvh = pair % p.Hkv;
    const int t = threadIdx.x, n = t >> 2, part4 = t & 3;
    const int R = (int)p.Sq * p.G;
    const bool valid = n < R;
    const int i = valid ? n / p.G : 0, g = valid ? n % p.G : 0;
    const int64_t row = ((int64_t)b * p.Sq + i) * p.Hq + (int64_t)kvh * p.G + g;

    float q[DP], o[DP];
    const float* qp = (const float*)p.Q + row * D;
#pragma unroll
    for (int e = 0; e < DP; ++e) {
        q[e] = valid ? qp[4 * e + part4] : 0.f;
        o[e] = 0.f;
    }
    int64_t k0 = (int64_t)part * p.part_len;
    int64_t k1 = k0 + p.part_len;
    if (k1 > p.Skv) k1 = p.Skv;
    if (k0 > k1) k0 = k1;
    const int64_t row_stride = (int64_t)p.Hkv * D;
    const float* Kg = (const float*)p.K + ((int64_t)b * p.Skv * p.Hkv + kvh) * D;
    const float* Vg = (const float*)p.V + ((int64_t)b * p.Skv * p.Hkv + kvh) * D;
    float m_run = kNegInf, l_run = 0.f;
    for (int64_t kb = k0; kb < k1; kb += BK) {
        const int klen = (k1 - kb) < BK ? (int)(k1 - kb) : BK;
        __syncthreads();
        for (int idx = t; idx < BK * D / 4; idx += 128) {
            const int r = idx / (D / 4), c4 = idx % (D / 4);
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (r < klen) {
                kv = *(const float4*)(Kg + (kb + r) * row_stride + 4 * c4);
                vv = *(const float4*)(Vg + (kb + r) * row_stride + 4 * c4);
            }
            *(float4*)&Ks[r][4 * c4] = kv;
            *(float4*)&Vs[r][4 * c4] = vv;
        }
        __syncthreads();
        float s[BK];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < BK; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < DP; ++e) acc = __builtin_fmaf(q[e], Ks[j][4 * e + part4], acc);
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            s[j] = j < klen ? acc * p.scale_log2 : kNegInf;
            mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < BK; ++j) {
            s[j] = fast_exp2(s[j] - m_use);
            lsum += s[j];
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
#pragma unroll
        for (int e = 0; e < DP; ++e) {
            float acc = o[e] * alpha;
#pragma unroll
            for (int j = 0; j < BK; ++j) acc = __builtin_fmaf(s[j], Vs[j][4 * e + part4], acc);
            o[e] = acc;
        }
    }
    if (valid) {
        const int64_t rows = (int64_t)p.B * p.Sq * p.Hq;
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float* op = p.O_parts + ((int64_t)part * rows + row) * D;
#pragma unroll
        for (int e = 0; e < DP; ++e) op[4 * e + part4] = o[e] * inv;
        if (part4 == 0)
            p.lse_parts[(int64_t)part * rows + row] = l_run > 0.f ? m_run * kLn2 + __logf(l_run) : kNegInf;
    }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, int d, hipStream_t s) {
    const int64_t grid = (int64_t)p.B * p.Hkv * p.n_parts;
    if (grid <= 0) return hipSuccess;
    if (d == 128)
        hipLaunchKernelGGL(decode_bf16_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL(decode_bf16_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeParams& p, int d, hipStream_t s) {
    const int64_t grid = (int64_t)p.B * p.Hkv * p.n_parts;
    if (grid <= 0) return hipSuccess;
    if (d == 128)
        hipLaunchKernelGGL(decode_f32_kernel<128>, dim3((unsigned)grid), dim3(128), 0, s, p);
    else
        hipLaunchKernelGGL(decode_f32_kernel<64>, dim3((unsigned)grid), dim3(128), 0, s, p);
    return hipGetLastError();
}

}  // namespace ra
