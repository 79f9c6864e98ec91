// fwd_bf16.hip -- blockwise ring-attention forward, bf16 inputs, gfx950 MFMA.
//
// One work-group owns a tile of 128 queries of one head (4 waves x 32
// queries) and keeps its online-softmax state (m, l, O) in registers while
// the key/value tiles of the P resident shards stream past it in ring order
// (lesson 8 "Context Parallelism (CP)", sections 2 and 3).  Per key tile:
//
//   S^T = K Q^T          v_mfma_f32_32x32x16_bf16, fp32 accumulate
//   mask                 only on tiles that cross the causal diagonal or the
//                        ragged end of a chunk
//   m~ = max(m, max S)   in-lane max over the lane's 32 scores + one swap with
//                        the other half-wave (each lane owns one query)
//   P = exp2(S*c - m~)   c = log2(e)/sqrt(d) folded into one FMA
//   l = l*a + sum P      a = exp2(m - m~), lane-partial sums
//   O^T = O^T*a + V^T P^T   v_mfma_f32_32x32x16_bf16 with P rounded to bf16
//
// The score matrix is produced transposed (keys along MFMA rows, queries
// along columns) so each lane holds whole rows of its own query and the
// softmax needs no cross-lane reduction beyond one half-wave swap.  The K
// rows fed to the first MFMA are permuted (bits 2 and 3 of the row index
// swapped) so that the accumulator hands every lane 8 consecutive keys per
// 16-key block: exactly the B operand layout of the second MFMA, with no data
// movement between the two products.
//
// K and V tiles (64 keys) are double-buffered in LDS.  Global loads for tile
// i+1 are issued before the MFMAs of tile i.  K is stored row-major with a
// 16-byte-chunk XOR swizzle; V is stored transposed (V^T, keys contiguous) so
// the second MFMA's A operand is one 16-byte LDS read per lane.
#include "attn_tile.h"

namespace ra {
namespace {

constexpr int BM = FWD_BF16_BLOCK_M;  // queries per work-group
constexpr int BN = 64;                // keys per tile
constexpr int NT = 256;               // threads per work-group

template <int D>
__global__ __launch_bounds__(NT, 1) void fwd_bf16_kernel(FwdParams p) {
    using T = Tile<D, BN, NT>;
    constexpr int KB = D / 16;  // MFMA k-blocks of Q K^T
    constexpr int DB = D / 32;  // 32-dim blocks of O^T
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2 * T::ELEMS];

    const QTile qt = decode_qtile<BM>(p, blockIdx.x);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int h = lane >> 5, m = lane & 31;

    // this lane's query (MFMA column m of the wave's 32 queries)
    const int qi = w * 32 + m;
    const bool qvalid = qi < qt.rows;
    const int64_t qpos = qt.pos0 + qi;
    const int wrows = qt.rows - w * 32;  // valid queries of this wave (may be <= 0)
    const int64_t wq_lo = qt.pos0 + w * 32;
    const int64_t wq_hi = wq_lo + (wrows < 32 ? wrows : 32) - 1;
    const int64_t qmax = qt.pos0 + qt.rows - 1;

    const uint16_t* Q = (const uint16_t*)p.Q;
    bf16x8 qop[KB];
    {
        const uint16_t* qp = Q + ((qt.b * p.q_rows + qt.q_row0 + qi) * p.Hq + qt.qh) * (int64_t)D;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            uint4 u = qvalid ? *(const uint4*)(qp + kb * 16 + h * 8) : make_uint4(0, 0, 0, 0);
            qop[kb] = __builtin_bit_cast(bf16x8, u);
        }
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    const int64_t row_stride = (int64_t)p.Hkv * D;
    const uint16_t* Kg = (const uint16_t*)p.K + ((int64_t)qt.b * p.S * p.Hkv + qt.kvh) * D;
    const uint16_t* Vg = (const uint16_t*)p.V + ((int64_t)qt.b * p.S * p.Hkv + qt.kvh) * D;

    KvIter it;
    bool have = kv_first(p, qt.rank, qmax, BN, it);
    typename T::Regs regs;
    if (have) {
        const int64_t r0 = it.krow + (int64_t)it.tile * BN;
        const int64_t left = p.c - (int64_t)it.tile * BN;
        T::load(regs, Kg + r0 * row_stride, Vg + r0 * row_stride, row_stride,
                left < BN ? (int)left : BN, threadIdx.x);
        T::store(regs, lds[0], lds[0] + T::ELEMS, threadIdx.x);
    }
    __syncthreads();

    int buf = 0;
    while (have) {
        const int64_t kpos0 = it.kpos + (int64_t)it.tile * BN;
        const int64_t kleft = p.c - (int64_t)it.tile * BN;
        const int klen = kleft < BN ? (int)kleft : BN;
        const bool nxt = kv_next(p, qt.rank, qmax, BN, it);
        if (nxt) {
            const int64_t r0 = it.krow + (int64_t)it.tile * BN;
            const int64_t left = p.c - (int64_t)it.tile * BN;
            T::load(regs, Kg + r0 * row_stride, Vg + r0 * row_stride, row_stride,
                    left < BN ? (int)left : BN, threadIdx.x);
        }

        const uint16_t* Ks = lds[buf];
        const uint16_t* Vts = lds[buf] + T::ELEMS;
        const bool active = wrows > 0 && !(p.causal && kpos0 > wq_hi);
        if (active) {
            // ---- S^T = K Q^T (64 keys x 32 queries)
            f32x16 sacc[2];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb2][r] = 0.f;
                const int row = kb2 * 32 + swap_bits23(m);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const bf16x8 a = *(const bf16x8*)(Ks + T::k_off(row, kb * 2 + h));
                    sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[kb], sacc[kb2], 0, 0, 0);
                }
            }
            // ---- mask (diagonal / ragged tiles only); register r of block kb2
            // holds key kb2*32 + 16*(r/8) + 8h + (r%8)
            const bool need_mask = klen < BN || (p.causal && kpos0 + BN - 1 > wq_lo);
            if (need_mask) {
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kidx = kb2 * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
                        const bool ok = kidx < klen && (!p.causal || kpos0 + kidx <= qpos);
                        if (!ok) sacc[kb2][r] = kNegInf;
                    }
            }
            // ---- online softmax update
            float mx = kNegInf;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
            mx = xor32_max(mx);
            const float m_new = fmaxf(m_run, mx * p.scale_log2);
            const float m_use = m_new == kNegInf ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            float lsum = 0.f;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = fast_exp2(__builtin_fmaf(sacc[kb2][r], p.scale_log2, -m_use));
                    sacc[kb2][r] = e;
                    lsum += e;
                }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            // ---- P^T as the B operand: 16-key block kk = registers 8*(kk%2).. of kb2 = kk/2
            bf16x8 pb[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int i = 0; i < 8; ++i) pb[kk][i] = (__bf16)sacc[kk >> 1][8 * (kk & 1) + i];
            // ---- O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int dim = db * 32 + m;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const bf16x8 a = *(const bf16x8*)(Vts + T::vt_off(dim, 2 * kk + h));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], oacc[db], 0, 0, 0);
                }
            }
        }
        if (nxt) T::store(regs, lds[buf ^ 1], lds[buf ^ 1] + T::ELEMS, threadIdx.x);
        __syncthreads();
        buf ^= 1;
        have = nxt;
    }

    // ---- finalize: O = O / l, LSE = m + ln l (natural log)
    const float l_tot = xor32_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qvalid) {
        const int64_t obase = ((qt.b * p.q_rows + qt.q_row0 + qi) * p.Hq + qt.qh) * (int64_t)D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                // accumulator registers 4*g4..4*g4+3 hold dims db*32 + 8*g4 + 4h + 0..3
                const int dim = db * 32 + 8 * g4 + 4 * h;
                const float o0 = oacc[db][4 * g4 + 0] * inv, o1 = oacc[db][4 * g4 + 1] * inv;
                const float o2 = oacc[db][4 * g4 + 2] * inv, o3 = oacc[db][4 * g4 + 3] * inv;
                if (p.o_f32) {
                    *(float4*)((float*)p.O + obase + dim) = make_float4(o0, o1, o2, o3);
                } else {
                    const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o0) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o1) << 16);
                    const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o2) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o3) << 16);
                    *(uint2*)((uint16_t*)p.O + obase + dim) = make_uint2(w0, w1);
                }
            }
        if (h == 0) {
            const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
            p.LSE[((int64_t)qt.b * p.Hq + qt.qh) * p.q_rows + qt.q_row0 + qi] = lse;
        }
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t s) {
    const int64_t tiles = (int64_t)p.n_ranks * p.chunks_per_rank * p.tiles_per_chunk;
    const int64_t grid = tiles * p.B * p.Hq;
    if (grid <= 0) return hipSuccess;
    if (d == 128)
        hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace ra
