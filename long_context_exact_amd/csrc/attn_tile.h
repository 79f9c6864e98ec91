// attn_tile.h -- bf16 key/value tile staging for the MFMA attention kernels.
//
// A tile is BN consecutive key rows of one kv head.  K goes to LDS row-major
// (one row = d bf16) with the 16-byte chunks of row r XOR-swizzled by r, so
// the 32 rows one MFMA operand read touches land in distinct banks.  V goes to
// LDS transposed (V^T, one row per head dimension, BN keys contiguous): the
// PV product contracts over keys, and an MFMA operand must hold 8 consecutive
// contraction elements per lane.  The transpose happens in registers: each
// thread loads 4 consecutive key rows x 8 dims and writes 8 dims x 4 keys.
#pragma once

#include "ra_device.h"

namespace ra {

template <int D, int BN, int NT>
struct Tile {
    static constexpr int KCH = D / 8;              // 16-byte chunks per K row
    static constexpr int K_LOADS = BN * KCH / NT;  // 16-byte K loads per thread
    static constexpr int V_UNITS = (BN / 4) * KCH; // (4 keys x 8 dims) units
    static constexpr int V_LOADS = (V_UNITS + NT - 1) / NT;
    static constexpr int ELEMS = BN * D;           // bf16 elements of K (or V)
    static_assert(BN * KCH % NT == 0, "K tile must split evenly over the threads");
    static_assert(BN % 32 == 0 && BN <= 128, "tile rows");

    struct Regs {
        uint4 k[K_LOADS];
        uint4 v[V_LOADS][4];
    };

    // element offset of K row `row`, 16-byte chunk `ch`
    static __device__ __forceinline__ int k_off(int row, int ch) {
        return row * D + ((ch ^ (row & (KCH - 1))) << 3);
    }
    // element offset of V^T row `dim`, 16-byte chunk `ch` (8 keys)
    static __device__ __forceinline__ int vt_off(int dim, int ch) {
        constexpr int VCH = BN / 8;
        const int sw = (dim ^ (dim >> 3)) & (VCH - 1);
        return dim * BN + ((ch ^ sw) << 3);
    }

    // Global -> registers.  Kb/Vb point at the tile's first row; rows are
    // row_stride elements apart; rows >= klen load as zero.
    static __device__ __forceinline__ void load(Regs& r, const uint16_t* Kb, const uint16_t* Vb,
                                                int64_t row_stride, int klen, int t) {
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int id = t + NT * i;
            const int row = id / KCH, ch = id % KCH;
            r.k[i] = row < klen ? *(const uint4*)(Kb + row * row_stride + ch * 8)
                                : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < V_LOADS; ++u) {
            const int id = t + NT * u;
            if (id < V_UNITS) {
                const int ch = id % KCH, g = id / KCH;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * g + i;
                    r.v[u][i] = row < klen ? *(const uint4*)(Vb + row * row_stride + ch * 8)
                                           : make_uint4(0, 0, 0, 0);
                }
            }
        }
    }

    // Registers -> LDS (Ks: K tile, Vts: V^T tile).
    static __device__ __forceinline__ void store(const Regs& r, uint16_t* Ks, uint16_t* Vts, int t) {
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int id = t + NT * i;
            const int row = id / KCH, ch = id % KCH;
            *(uint4*)(Ks + k_off(row, ch)) = r.k[i];
        }
#pragma unroll
        for (int u = 0; u < V_LOADS; ++u) {
            const int id = t + NT * u;
            if (id < V_UNITS) {
                const int ch = id % KCH, g = id / KCH;  // dims 8ch..8ch+7, keys 4g..4g+3
                const uint32_t* v0 = (const uint32_t*)&r.v[u][0];
                const uint32_t* v1 = (const uint32_t*)&r.v[u][1];
                const uint32_t* v2 = (const uint32_t*)&r.v[u][2];
                const uint32_t* v3 = (const uint32_t*)&r.v[u][3];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // dword j of a key row holds dims 2j (low half) and 2j+1 (high half)
                    const uint32_t lo01 = __builtin_amdgcn_perm(v1[j], v0[j], 0x05040100u);
                    const uint32_t lo23 = __builtin_amdgcn_perm(v3[j], v2[j], 0x05040100u);
                    const uint32_t hi01 = __builtin_amdgcn_perm(v1[j], v0[j], 0x07060302u);
                    const uint32_t hi23 = __builtin_amdgcn_perm(v3[j], v2[j], 0x07060302u);
                    const int d0 = 8 * ch + 2 * j;
                    // keys 4g..4g+3 sit in 16-byte chunk g/2, 8-byte half g%2
                    *(uint2*)(Vts + vt_off(d0, g >> 1) + 4 * (g & 1)) = make_uint2(lo01, lo23);
                    *(uint2*)(Vts + vt_off(d0 + 1, g >> 1) + 4 * (g & 1)) = make_uint2(hi01, hi23);
                }
            }
        }
    }
};

// MFMA row permutation for the QK^T product: swapping bits 2 and 3 of the
// row index makes the 32x32 accumulator give each half-wave 8 consecutive
// keys of every 16-key block (register r of half h <-> key 16*(r/8)+8h+r%8).
__device__ __forceinline__ int swap_bits23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

}  // namespace ra
