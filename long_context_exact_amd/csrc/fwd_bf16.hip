// fwd_bf16.hip -- blockwise ring-attention forward, bf16 inputs, gfx950 MFMA.
//
// One work-group owns a tile of 256 queries of one head (8 waves x 32
// queries, two waves per SIMD) and keeps its online-softmax state (m, l, O)
// in registers while the key/value tiles of the P resident shards stream past
// it in ring order (lesson 8 "Context Parallelism (CP)", sections 2 and 3).
// Per key tile of 64 keys and per wave:
//
//   S^T = K Q^T          v_mfma_f32_32x32x16_bf16, fp32 accumulate
//   mask                 only on tiles that cross the causal diagonal or the
//                        ragged end of a chunk
//   m~ = max(m, max S)   in-lane max over the lane's 32 scores + one
//                        permlane32 swap (each lane owns one query)
//   P = exp2(S*c - m')   c = log2(e)/sqrt(d) folded into one FMA
//   l = l*a + sum P      lane-partial sums, a = exp2(m - m'); a second sum
//                        of the bf16-rounded P (v_dot2 with ones) normalises O
//   O^T = O^T*a + V^T P^T   v_mfma_f32_32x32x16_bf16 with P rounded to bf16
//
// The reference point m' of the exponentials is moved only when the running
// maximum has grown by more than 2^8 since the last move (then P <= 256):
// O and l are always taken relative to the same m', so the result is the
// same; the 64 multiplies of the O rescale are skipped on most tiles.
//
// The score matrix is produced transposed (keys along MFMA rows, queries
// along columns) so each lane holds whole rows of its own query.  The K rows
// fed to the first MFMA are permuted (bits 2 and 3 of the row index swapped)
// so the accumulator hands every lane 8 consecutive keys per 16-key block:
// exactly the B operand of the second MFMA, with no data movement.  V is
// stored transposed in LDS (V^T: keys contiguous, one row per head dim), so
// the PV operand (8 consecutive keys of one dim per lane) is one 16-byte LDS
// read, like the K operand.  The transpose is done in registers while the
// tile is staged, in the VALU phase; transposing LDS reads in the MFMA phase
// would cost it about three times the LDS issue time per operand.
//
// Schedule.  The waves form two groups, 0-3 and 4-7, with one wave of each
// on every SIMD.  An iteration has two phases separated by barriers: an MFMA
// phase (O += V_{i-1} P_{i-1}, then S_i = K_i Q^T) and a VALU phase (softmax
// of S_i, plus staging the next K/V rows).  Group 1 starts one phase late, so
// on every SIMD one wave issues MFMAs while the other runs its exponentials.
// K/V tiles live in a ring of three LDS buffers; each group stages half of
// every tile through registers (tile i+1+group is written in the VALU phase of
// iteration i, and its successor's global loads are issued right after).
#include "ra_device.h"

namespace ra {
namespace {

constexpr int BM = FWD_BF16_BLOCK_M;  // queries per work-group (8 waves x 32)
constexpr int BN = 64;                // keys per tile
constexpr int NT = 512;               // threads per work-group
constexpr int GT = 256;               // threads per wave group
constexpr int NBUF = 3;               // LDS ring depth
constexpr float kLazy = 8.0f;         // log2 headroom before the reference max moves

#ifndef RA_FWD_VT
#define RA_FWD_VT 0       // 1: V transposed in LDS (16-byte PV reads); 0: row-major V, transpose reads
#endif
#ifndef RA_FWD_PIN
#define RA_FWD_PIN 1      // pin the MFMA / operand-read interleave
#endif
#ifndef RA_FWD_AHEAD
#define RA_FWD_AHEAD 4    // MFMA operands read ahead of use in the MFMA phase
#endif

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct KvTileRow {
    static constexpr int KCH = D / 8;                   // 16-byte chunks per row
    static constexpr int HALF = BN / 2;                 // rows staged by one wave group
    static constexpr int LOADS = HALF * KCH / GT;       // 16-byte loads per thread per tensor
    static constexpr int ELEMS = BN * D;
    static constexpr int K_ELEMS = ELEMS, V_ELEMS = ELEMS;
    static_assert(LOADS >= 1 && HALF * KCH % GT == 0, "tile split");

    // K: chunk c of row r lives at chunk c ^ (r mod KCH): the 32 rows x 2
    // chunks of one MFMA operand read hit every bank equally.
    static __device__ __forceinline__ int k_off(int row, int ch) {
        return row * D + ((ch ^ (row & (KCH - 1))) << 3);
    }
    // V: chunk c of row r lives at chunk c ^ s(r); one transpose read touches
    // 8 rows (two groups of 4 consecutive) x 32 dims, spread over all banks.
    static __device__ __forceinline__ int v_sw(int row) {
        return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
    }
    static __device__ __forceinline__ int v_off(int row, int ch) {
        return row * D + ((ch ^ v_sw(row)) << 3);
    }

    struct Regs {
        uint4 k[LOADS];
        uint4 v[LOADS];
    };

    // Rows [32*grp, 32*grp + 32) of a tile, global -> registers; rows at or
    // beyond klen (the ragged end of a chunk) load as zero.
    static __device__ __forceinline__ void load(Regs& r, const uint16_t* Kb, const uint16_t* Vb,
                                                int64_t row_stride, int klen, int grp, int gt) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int id = gt + GT * i;
            const int row = HALF * grp + id / KCH, ch = id % KCH;
            const bool ok = row < klen;
            const int64_t off = row * row_stride + ch * 8;
            r.k[i] = ok ? *(const uint4*)(Kb + off) : make_uint4(0, 0, 0, 0);
            r.v[i] = ok ? *(const uint4*)(Vb + off) : make_uint4(0, 0, 0, 0);
        }
    }
    static __device__ __forceinline__ void store(const Regs& r, uint16_t* Ks, uint16_t* Vs, int grp,
                                                 int gt) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int id = gt + GT * i;
            const int row = HALF * grp + id / KCH, ch = id % KCH;
            *(uint4*)(Ks + k_off(row, ch)) = r.k[i];
            *(uint4*)(Vs + v_off(row, ch)) = r.v[i];
        }
    }
};

// V stored transposed (V^T) with 256-byte rows, for 16-byte PV operand reads.
template <int D>
struct KvTileVt {
    static constexpr int KCH = D / 8;                   // 16-byte chunks per K row
    static constexpr int HALF = BN / 2;                 // keys staged by one wave group
    static constexpr int K_LOADS = HALF * KCH / GT;     // 16-byte K loads per thread
    static constexpr int V_UNITS = (HALF / 2) * KCH;    // (2 keys x 8 dims) V units per half tile
    static constexpr int K_ELEMS = BN * D;
    static constexpr int VT_STRIDE = 2 * BN;            // V^T row pitch in elements (256 bytes)
    static constexpr int V_ELEMS = D * VT_STRIDE;
    static_assert(K_LOADS >= 1 && K_LOADS <= 2 && HALF * KCH % GT == 0 && V_UNITS <= GT, "tile split");

    // K, row-major: chunk c of row r lives at chunk c ^ (r mod KCH); the 32
    // rows x 2 chunks of one MFMA operand read hit every bank equally.
    static __device__ __forceinline__ int k_off(int row, int ch) {
        return row * D + ((ch ^ (row & (KCH - 1))) << 3);
    }
    // V^T: one row per head dimension, BN keys used out of a 256-byte pitch;
    // 8-key chunk c of row d lives at chunk c ^ (d mod 16) ^ ((d >> 4) mod 8).
    // Measured with the LDS bank-conflict counter, the PV operand read (32
    // consecutive dims x 2 chunks) is conflict-free; the staging writes below
    // (4 bytes = 2 keys of one dim, dims 8c+j of the 16 chunks c) cover 64
    // distinct banks.  With the (d mod 16) term alone 8-byte transposed
    // writes conflict 16-way.
    static __device__ __forceinline__ int vt_off(int dim, int ch) {
        return dim * VT_STRIDE + ((ch ^ (dim & 15) ^ ((dim >> 4) & 7)) << 3);
    }

    // Staging of one wave group's half tile (keys 32*grp .. 32*grp+31).  Every
    // thread carries K_LOADS 16-byte chunks of K and one unit of V: 2
    // consecutive keys x 8 dims, transposed in registers on the way to LDS.
    struct Regs {
        uint4 k0, k1, v0, v1;
    };

    static __device__ __forceinline__ void load(Regs& r, const uint16_t* Kb, const uint16_t* Vb,
                                                int64_t row_stride, int klen, int grp, int gt) {
        {
            const int row = HALF * grp + gt / KCH, ch = gt % KCH;
            r.k0 = row < klen ? *(const uint4*)(Kb + row * row_stride + ch * 8) : make_uint4(0, 0, 0, 0);
        }
        if (K_LOADS > 1) {
            const int id = gt + GT;
            const int row = HALF * grp + id / KCH, ch = id % KCH;
            r.k1 = row < klen ? *(const uint4*)(Kb + row * row_stride + ch * 8) : make_uint4(0, 0, 0, 0);
        }
        if (gt < V_UNITS) {
            const int ch = gt % KCH, kp = gt / KCH;
            const int row = HALF * grp + 2 * kp;
            r.v0 = row < klen ? *(const uint4*)(Vb + row * row_stride + ch * 8) : make_uint4(0, 0, 0, 0);
            r.v1 = row + 1 < klen ? *(const uint4*)(Vb + (row + 1) * row_stride + ch * 8)
                                  : make_uint4(0, 0, 0, 0);
        }
    }

    static __device__ __forceinline__ void store(const Regs& r, uint16_t* Ks, uint16_t* Vts, int grp,
                                                 int gt) {
        {
            const int row = HALF * grp + gt / KCH, ch = gt % KCH;
            *(uint4*)(Ks + k_off(row, ch)) = r.k0;
        }
        if (K_LOADS > 1) {
            const int id = gt + GT;
            const int row = HALF * grp + id / KCH, ch = id % KCH;
            *(uint4*)(Ks + k_off(row, ch)) = r.k1;
        }
        if (gt < V_UNITS) {
            const int ch = gt % KCH, kp = gt / KCH;
            const int key0 = HALF * grp + 2 * kp;  // keys key0, key0+1; dims 8ch..8ch+7
            const uint32_t a[4] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w};
            const uint32_t b[4] = {r.v1.x, r.v1.y, r.v1.z, r.v1.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // dword j of a key row holds dims 2j (low half) and 2j+1 (high half)
                const int d0 = 8 * ch + 2 * j;
                *(uint32_t*)(Vts + vt_off(d0, key0 >> 3) + (key0 & 7)) =
                    __builtin_amdgcn_perm(b[j], a[j], 0x05040100u);
                *(uint32_t*)(Vts + vt_off(d0 + 1, key0 >> 3) + (key0 & 7)) =
                    __builtin_amdgcn_perm(b[j], a[j], 0x07060302u);
            }
        }
    }
};

#if RA_FWD_VT
template <int D> using KvTile = KvTileVt<D>;
#else
template <int D> using KvTile = KvTileRow<D>;
#endif

__device__ __forceinline__ i16x4 ds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

__device__ __forceinline__ int swap_bits23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// max / sum of a value over the two half-waves (lanes l and l^32)
__device__ __forceinline__ float halves_max(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

struct TileDesc {
    int64_t krow;  // first K/V row (sharded order)
    int64_t kpos;  // global position of that row
    int klen;      // valid rows of the tile (ragged end of a chunk)
};

__device__ __forceinline__ TileDesc tile_desc(const FwdParams& p, const KvIter& it) {
    TileDesc d;
    const int64_t off = (int64_t)it.tile * BN;
    d.krow = it.krow + off;
    d.kpos = it.kpos + off;
    const int64_t left = p.c - off;
    d.klen = left < BN ? (int)left : BN;
    return d;
}

template <int D>
__global__ __launch_bounds__(NT) void fwd_bf16_kernel(FwdParams p) {
    using T = KvTile<D>;
    constexpr int KB = D / 16;  // MFMA k-blocks of Q K^T
    constexpr int DB = D / 32;  // 32-dim blocks of O^T
    __shared__ __attribute__((aligned(16))) uint16_t ldsK[NBUF][T::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t ldsV[NBUF][T::V_ELEMS];  // V^T, padded rows

    const QTile qt = decode_qtile<BM>(p, blockIdx.x);
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, uniform in the wave
    const int h = lane >> 5, m = lane & 31;
    const int grp = w >> 2, gt = t & (GT - 1);  // wave group; one wave of each per SIMD

    // this lane's query (MFMA column m of the wave's 32 queries)
    const int qi = w * 32 + m;
    const bool qvalid = qi < qt.rows;
    const int64_t qpos = qt.pos0 + qi;
    const int wrows = qt.rows - w * 32;  // valid queries of this wave (may be <= 0)
    const int64_t wq_lo = qt.pos0 + w * 32;
    const int64_t wq_hi = wq_lo + (wrows < 32 ? wrows : 32) - 1;
    const int64_t qmax = qt.pos0 + qt.rows - 1;

    bf16x8 qop[KB];
    {
        const uint16_t* qp = (const uint16_t*)p.Q +
                             ((qt.b * p.q_rows + qt.q_row0 + qi) * p.Hq + qt.qh) * (int64_t)D;
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
    float m_run = kNegInf, l_run = 0.f, lr_run = 0.f;
    const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};

    const int64_t row_stride = (int64_t)p.Hkv * D;
    const uint16_t* Kg = (const uint16_t*)p.K + ((int64_t)qt.b * p.S * p.Hkv + qt.kvh) * D;
    const uint16_t* Vg = (const uint16_t*)p.V + ((int64_t)qt.b * p.S * p.Hkv + qt.kvh) * D;

    // ---- prologue: tile 0 in LDS (both halves), group 1's half of tile 1 in
    // LDS, and each group's next half-tile (1 + grp) in registers
    const int n = kv_count(p, qt.rank, qmax, BN);
    KvIter it_c, it_l;
    typename T::Regs regs;
    if (n > 0) {
        kv_first(p, qt.rank, qmax, BN, it_c);
        it_l = it_c;
        TileDesc d0 = tile_desc(p, it_c);
        T::load(regs, Kg + d0.krow * row_stride, Vg + d0.krow * row_stride, row_stride, d0.klen, grp, gt);
        T::store(regs, ldsK[0], ldsV[0], grp, gt);
        for (int j = 1; j <= 1 + grp && j < n; ++j) {
            kv_next(p, qt.rank, qmax, BN, it_l);
            const TileDesc dj = tile_desc(p, it_l);
            T::load(regs, Kg + dj.krow * row_stride, Vg + dj.krow * row_stride, row_stride, dj.klen,
                    grp, gt);
            if (j < 1 + grp) T::store(regs, ldsK[j], ldsV[j], grp, gt);
        }
    }
    // the first MFMA phase multiplies P = 0 by the V buffer "before" tile 0:
    // zero it so no stale bits (NaN patterns) reach the accumulators
    for (int e = t * 8; e < T::V_ELEMS; e += NT * 8)
        *(uint4*)(&ldsV[NBUF - 1][e]) = make_uint4(0, 0, 0, 0);
    // Drain the prologue's loads here: otherwise the wait-count analysis merges
    // them into the loop header and makes the loop wait on in-flight staging
    // loads at its first MFMA.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (grp == 1) __syncthreads();  // group 1 runs one phase behind group 0

    // P of the previous tile (zero before the first tile, whose "previous" V
    // buffer is zeroed in the prologue, so the first PV product adds 0)
    bf16x8 pb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) pb[kk][i2] = (__bf16)0.f;

    // MFMA phase operands, in issue order: NPV blocks of O^T += V^T P^T (block
    // j: keys 16*(j/DB).., dims 32*(j%DB)..), then NQK blocks of S^T = K Q^T
    // (block j: keys 32*(j/KB).., dims 16*(j%KB)..).  Each operand is one
    // 16-byte LDS read.
    constexpr int NPV = 4 * DB, NQK = 2 * KB, NMF = NPV + NQK;
    auto read_op = [&](int j, int buf) -> bf16x8 {
        if (j < NPV) {
            const int kk = j / DB, db = j % DB;
#if RA_FWD_VT
            return *(const bf16x8*)(ldsV[(buf + NBUF - 1) % NBUF] + T::vt_off(db * 32 + m, 2 * kk + h));
#else
            // transpose reads: lane l of 16-lane group g points at row
            // 8*(g>>1) + (l%16)/4 (+4 for the second read) and dims
            // 16*(g&1) + 4*(l%4); it receives 4 consecutive keys of one dim
            const uint16_t* Vs = ldsV[(buf + NBUF - 1) % NBUF];
            const int r0 = 16 * kk + 8 * (lane >> 5) + ((lane & 15) >> 2);
            const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            const i16x4 lo = ds_read_tr(Vs + T::v_off(r0, col >> 3) + (col & 7));
            const i16x4 hi = ds_read_tr(Vs + T::v_off(r0 + 4, col >> 3) + (col & 7));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#endif
        }
        const int q = j - NPV, kb2 = q / KB, kb = q % KB;
        const int row = kb2 * 32 + swap_bits23(m);
        return *(const bf16x8*)(ldsK[buf] + T::k_off(row, kb * 2 + h));
    };

    constexpr int AHEAD = RA_FWD_AHEAD;  // operands read ahead of their MFMA
    for (int i = 0; i < n; ++i) {
        // ================= MFMA phase: O += V_{i-1} P_{i-1}; S_i = K_i Q^T
        // One straight-line block: every wave runs both products on every
        // tile (a tile wholly in the future of a wave's queries is masked to
        // P = 0 in the VALU phase), so the operand reads can be issued AHEAD
        // MFMAs early and their LDS latency hides behind the matrix pipe.
        const TileDesc dc = tile_desc(p, it_c);
        const int cb = i % NBUF;
        f32x16 sacc[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb2][r] = 0.f;
        bf16x8 ops[AHEAD];
#pragma unroll
        for (int j = 0; j < AHEAD; ++j) ops[j] = read_op(j, cb);
#if RA_FWD_PIN
        // pin the issue order: the first AHEAD operands' reads, then per MFMA
        // the read of the operand AHEAD positions later
        __builtin_amdgcn_sched_group_barrier(0x100, RA_FWD_VT ? AHEAD : 2 * AHEAD, 0);
#endif
#pragma unroll
        for (int j = 0; j < NMF; ++j) {
            const bf16x8 a = ops[j % AHEAD];
            if (j + AHEAD < NMF) ops[j % AHEAD] = read_op(j + AHEAD, cb);
            if (j < NPV) {
                oacc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[j / DB], oacc[j % DB], 0, 0, 0);
            } else {
                const int q = j - NPV;
                sacc[q / KB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[q % KB], sacc[q / KB], 0, 0, 0);
            }
#if RA_FWD_PIN
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (!RA_FWD_VT && j + AHEAD < NPV)
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            else if (j + AHEAD < NMF)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#endif
        }
        __syncthreads();

        // ================= VALU phase: softmax of S_i; stage K/V rows
        {
            // mask (diagonal / ragged tiles only): register r of block kb2
            // holds key kb2*32 + 16*(r/8) + 8h + (r%8); keys >= lim are masked
            const bool need_mask = dc.klen < BN || (p.causal && dc.kpos + BN - 1 > wq_lo);
            if (need_mask) {
                int lim = dc.klen;
                if (p.causal) {
                    const int64_t vis = qpos - dc.kpos + 1;
                    lim = vis < (int64_t)lim ? (vis < 0 ? 0 : (int)vis) : lim;
                }
                lim -= 8 * h;
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int k0 = kb2 * 32 + 16 * (r >> 3) + (r & 7);
                        sacc[kb2][r] = k0 < lim ? sacc[kb2][r] : kNegInf;
                    }
            }
            float mx = kNegInf;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
            mx = halves_max(mx) * p.scale_log2;
            const bool move = mx > m_run + kLazy;
            const float m_ref = move ? mx : m_run;
            const float m_use = m_ref == kNegInf ? 0.f : m_ref;
            if (__builtin_amdgcn_ballot_w64(move) != 0) {
                const float alpha = fast_exp2(m_run - m_use);
                l_run *= alpha;
                lr_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }
            m_run = m_ref;
            // l_run sums the exponentials exactly (for the LSE); lr_run sums
            // the bf16-rounded values the PV product uses (for O), so a
            // dominant key's rounding cancels in O = sum(p V) / sum(p)
            float lsum = 0.f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int i2 = 0; i2 < 8; i2 += 2) {
                    const float e0 = fast_exp2(
                        __builtin_fmaf(sacc[kk >> 1][8 * (kk & 1) + i2], p.scale_log2, -m_use));
                    const float e1 = fast_exp2(
                        __builtin_fmaf(sacc[kk >> 1][8 * (kk & 1) + i2 + 1], p.scale_log2, -m_use));
                    lsum += e0 + e1;
                    bf16x2 pr;
                    pr[0] = (__bf16)e0;
                    pr[1] = (__bf16)e1;
                    lr_run = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes, lr_run, false);
                    pb[kk][i2] = pr[0];
                    pb[kk][i2 + 1] = pr[1];
                }
            l_run += lsum;
        }
        // this group's half of tile i+1+grp -> LDS; then the next half-tile's loads
        const int wi = i + 1 + grp;
        if (wi < n) {
            T::store(regs, ldsK[wi % NBUF], ldsV[wi % NBUF], grp, gt);
            if (wi + 1 < n) {
                kv_next(p, qt.rank, qmax, BN, it_l);
                const TileDesc dl = tile_desc(p, it_l);
                T::load(regs, Kg + dl.krow * row_stride, Vg + dl.krow * row_stride, row_stride,
                        dl.klen, grp, gt);
            }
        }
        __syncthreads();
        if (i + 1 < n) kv_next(p, qt.rank, qmax, BN, it_c);
    }
    // last MFMA phase: O += V_{n-1} P_{n-1}
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
        const bf16x8 a = read_op(j, n % NBUF);
        oacc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[j / DB], oacc[j % DB], 0, 0, 0);
    }
    __syncthreads();
    if (grp == 0) __syncthreads();  // matches group 1's extra barrier

    // ---- finalize: O = O / l, LSE = m + ln l (natural log)
    const float l_tot = halves_sum(l_run);
    const float lr_tot = halves_sum(lr_run);
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
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
