// decode.hip -- per-shard partial attention of a few query tokens against a
// KV cache split along the sequence (the Helix article's phase 1: each device
// holds a slice of the cache and produces a partial result that one exchange
// later combines).  Output per part: O_p normalised by its own denominator
// and lse_p = m_p + ln l_p, which is exactly what the merge needs.
//
// bf16 kernel: one work-group per (batch, kv head, part).  The Sq x G query
// rows that read this kv head form the 32 MFMA columns (unused columns carry
// zero queries and are never stored).  The part's keys stream through LDS in
// stages of 128; each of the 4 waves takes 32 keys of a stage and keeps its
// own (m, l, O) state, and the four states are merged at the end.  The kernel
// is bound by HBM (every K/V byte is read once), so what matters is the bytes
// in flight: the next stage is loaded into registers while the current one is
// used from a single 64 KB LDS stage, which lets two work-groups share a CU.
// K and V stay row-major in LDS; the PV operand (8 consecutive keys of one
// head dim) comes from two ds_read_b64_tr_b16 transposing reads.
#include "ra_device.h"

namespace ra {
namespace {

constexpr int NT = 256;
constexpr int STAGE = 128;   // keys per stage (4 waves x 32)

typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct DecStage {
    static constexpr int KCH = D / 8;                 // 16-byte chunks per row
    static constexpr int ELEMS = STAGE * D;
    static constexpr int LOADS = STAGE * KCH / NT;    // 16-byte loads per thread per tensor
    static_assert(STAGE * KCH % NT == 0, "stage split");
    // K: chunk c of row r lives at chunk c ^ (r mod KCH) (MFMA operand reads
    // of 32 rows x 2 chunks hit every bank equally).  V: a transposing read
    // touches 8 rows (two groups of 4) x 32 dims; the row swizzle spreads them.
    static __device__ __forceinline__ int k_off(int row, int ch) {
        return row * D + ((ch ^ (row & (KCH - 1))) << 3);
    }
    static __device__ __forceinline__ int v_off(int row, int ch) {
        const int sw = D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
        return row * D + ((ch ^ sw) << 3);
    }
    struct Regs {
        uint4 k[LOADS], v[LOADS];
    };
    // rows [0, klen) of the stage from global memory; rows past klen load as
    // 0.  Load i of thread t covers row t/KCH + i*NT/KCH, chunk t%KCH: one
    // per-thread byte offset against a uniform base that steps NT/KCH rows.
    static __device__ __forceinline__ void load(Regs& r, const uint16_t* Kb, const uint16_t* Vb,
                                                int64_t row_stride, int klen, int t) {
        const int row0 = t / KCH;
        const uint32_t off = (uint32_t)(row0 * row_stride * 2 + (t % KCH) * 16);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const bool ok = row0 + i * (NT / KCH) < klen;
            const int64_t step = (int64_t)i * (NT / KCH) * row_stride;
            r.k[i] = ok ? load_once16((const char*)(Kb + step) + off) : make_uint4(0, 0, 0, 0);
            r.v[i] = ok ? load_once16((const char*)(Vb + step) + off) : make_uint4(0, 0, 0, 0);
        }
    }
    static __device__ __forceinline__ void store(const Regs& r, uint16_t* Ks, uint16_t* Vs, int t) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int id = t + NT * i;
            const int row = id / KCH, ch = id % KCH;
            *(uint4*)(Ks + k_off(row, ch)) = r.k[i];
            *(uint4*)(Vs + v_off(row, ch)) = r.v[i];
        }
    }
};

template <int D>
__global__ __launch_bounds__(NT, 2) void decode_bf16_kernel(DecodeParams p) {
    using T = DecStage<D>;
    constexpr int KB = D / 16, DB = D / 32;
    // [K | V] of one stage; reused as the scratch of the final merge
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::ELEMS];
    static_assert(sizeof(lds) >= sizeof(float) * (3 * DB * 16 * 64 + 3 * 2 * 64), "merge scratch");
    uint16_t* Ks = lds;
    uint16_t* Vs = lds + T::ELEMS;

    const int part = blockIdx.x % p.n_parts;
    const int pair = blockIdx.x / p.n_parts;
    const int b = pair / p.Hkv, kvh = pair % p.Hkv;
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
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

    int64_t k0, k1, base;
    decode_part(p, part, b, kvh, D, k0, k1, base);
    const int64_t nstages = (k1 - k0 + STAGE - 1) / STAGE;

    const int64_t row_stride = (int64_t)p.Hkv * D;
    const uint16_t* Kg = (const uint16_t*)p.K + base;
    const uint16_t* Vg = (const uint16_t*)p.V + base;

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    auto stage_len = [&](int64_t st) -> int {
        const int64_t left = k1 - (k0 + st * STAGE);
        return left <= 0 ? 0 : (left < STAGE ? (int)left : STAGE);
    };
    typename T::Regs regs;
    if (nstages > 0) {
        T::load(regs, Kg + k0 * row_stride, Vg + k0 * row_stride, row_stride, stage_len(0), t);
        T::store(regs, Ks, Vs, t);
    }
    __syncthreads();

    const int krow = 32 * w + swap_bits23(m);   // this lane's K row (MFMA A-operand row m)
    for (int64_t st = 0; st < nstages; ++st) {
        const bool nxt = st + 1 < nstages;
        if (nxt) {
            const int64_t r0 = k0 + (st + 1) * STAGE;
            T::load(regs, Kg + r0 * row_stride, Vg + r0 * row_stride, row_stride, stage_len(st + 1), t);
        }
        const int klen = stage_len(st) - 32 * w;  // this wave's valid keys (may be <= 0)
        if (klen > 0) {
            f32x16 sacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 av = *(const bf16x8*)(Ks + T::k_off(krow, kb * 2 + h));
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qop[kb], sacc, 0, 0, 0);
            }
            // register r holds key 16*(r/8) + 8h + r%8 of the wave's 32
            if (klen < 32) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kidx = 16 * (r >> 3) + 8 * h + (r & 7);
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
            bf16x8 pb[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(__builtin_fmaf(sacc[r], p.scale_log2, -m_use));
                lsum += e;
                pb[r >> 3][r & 7] = (__bf16)e;
            }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            // O^T += V^T P^T: operand (kk, db) = keys 32w + 16kk.., dims 32db..;
            // lane l of 16-lane group g reads rows 8*(g>>1) + (l%16)/4 (+4)
            // and dims 16*(g&1) + 4*(l%4): 4 consecutive keys of one dim each
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int r0 = 32 * w + 16 * kk + 8 * h + ((lane & 15) >> 2);
                    const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(Vs + T::v_off(r0, col >> 3) + (col & 7)));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(Vs + T::v_off(r0 + 4, col >> 3) + (col & 7)));
                    const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kk], oacc[db], 0, 0, 0);
                }
        }
        __syncthreads();
        if (nxt) T::store(regs, Ks, Vs, t);
        __syncthreads();
    }

    // ---- merge the four waves' states in wave 0 (same register layout in
    // every wave, so lane l combines the other waves' lane-l values), then
    // write this part's (O, lse)
    float* scratch = (float*)lds;
    float* Ow = scratch;                       // [3][DB*16][64]
    float* ml = scratch + 3 * DB * 16 * 64;    // [3][2][64]
    if (w > 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) Ow[((w - 1) * DB * 16 + db * 16 + r) * 64 + lane] = oacc[db][r];
        ml[((w - 1) * 2 + 0) * 64 + lane] = m_run;
        ml[((w - 1) * 2 + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (w == 0) {
        float mw[4], lw[4], sc[4];
        mw[0] = m_run;
        lw[0] = l_run;
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            mw[ww] = ml[((ww - 1) * 2 + 0) * 64 + lane];
            lw[ww] = ml[((ww - 1) * 2 + 1) * 64 + lane];
        }
        float M = kNegInf;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mw[ww]);
        float L = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            sc[ww] = M == kNegInf ? 0.f : fast_exp2(mw[ww] - M);
            L += lw[ww] * sc[ww];
        }
        L = xor32_sum(L);  // the two half-waves hold different keys of one query
        const float inv = L > 0.f ? 1.f / L : 0.f;
        if (cvalid) {
            const int64_t row = ((int64_t)b * p.Sq + ci) * p.Hq + (int64_t)kvh * p.G + cg;
            const int64_t rows = (int64_t)p.B * p.Sq * p.Hq;
            float* op = p.O_parts + ((int64_t)part * rows + row) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    float o[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = 4 * g4 + q;
                        float acc = oacc[db][r] * sc[0];
#pragma unroll
                        for (int ww = 1; ww < 4; ++ww) acc += Ow[((ww - 1) * DB * 16 + db * 16 + r) * 64 + lane] * sc[ww];
                        o[q] = acc * inv;
                    }
                    // accumulator registers 4*g4..4*g4+3 hold dims db*32 + 8*g4 + 4h + 0..3
                    *(float4*)(op + db * 32 + 8 * g4 + 4 * h) = make_float4(o[0], o[1], o[2], o[3]);
                }
            if (h == 0)
                p.lse_parts[(int64_t)part * rows + row] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
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
    int64_t k0, k1, base;
    decode_part(p, part, b, kvh, D, k0, k1, base);
    const int64_t row_stride = (int64_t)p.Hkv * D;
    const float* Kg = (const float*)p.K + base;
    const float* Vg = (const float*)p.V + base;
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
