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
//   P = exp2(S*c - m')   c = log2(e)/sqrt(d) folded into one FMA; m' is the
//                        lane's reference point (below)
//   l = l*a + sum P      lane-partial sums; a second sum of the bf16-rounded P
//                        (v_dot2 with ones) normalises O
//   O^T = O^T*a + V^T P^T   v_mfma_f32_32x32x16_bf16 with P rounded to bf16
//
// Reference point.  O and l are kept relative to a reference m' that only
// has to keep the exponentials in range, not equal the running maximum: a
// tile whose 32 exponentials (per lane) sum to at most 2^8 is accepted as it
// is, so most tiles need no max reduction and no O rescale.  Otherwise (also
// at a lane's first finite score, which overflows the sum against the initial
// reference) the slow path takes the true maximum, rescales l and O by
// a = exp2(m' - m'') and recomputes the tile's P.
//
// The score matrix is produced transposed (keys along MFMA rows, queries
// along columns) so each lane holds whole rows of its own query.  The K rows
// fed to the first MFMA are permuted (bits 2 and 3 of the row index swapped)
// so the accumulator hands every lane 8 consecutive keys per 16-key block:
// exactly the B operand of the second MFMA, with no data movement.  V stays
// row-major in LDS; its A operand (8 consecutive keys of one head dim per
// lane) comes from two ds_read_b64_tr_b16 transposing reads.
//
// Schedule.  A wave hides part of its independent VALU work behind its own
// MFMAs (the two pipes overlap only in part), so every wave software-pipelines
// its own loop: in iteration i it issues the MFMAs of S_{i+1} = K_{i+1} Q^T and
// O += V_{i-1} P_{i-1} and, in between them, the softmax of S_i.  The stage
// opens with a PV product whose V operand was read before the barrier, so an
// MFMA is in flight while the K operands arrive and the next loads go out.
// K/V tiles go from global memory straight into rings of four LDS buffers
// (global_load_lds_dwordx4, no staging registers): stage i loads K of tile i+3
// and V of tile i+2, two stages before their use, and waits only for the loads
// of two stages before.  The loop body is unrolled over the ring so
// that every LDS operand address is a per-lane base plus an immediate offset.
#include <type_traits>

#include "ra_device.h"

namespace ra {
namespace {

constexpr int BM = FWD_BF16_BLOCK_M;  // queries per work-group (8 waves x 32)
constexpr int BN = 64;                // keys per tile
constexpr int NW = 8;                 // waves per work-group
constexpr int NT = 64 * NW;           // threads per work-group
constexpr int NBUF = 4;               // LDS ring depth (K and V rings stay below 64 KB each)
constexpr float kSumCap = 256.f;      // largest accepted per-lane tile sum of P
// Initial reference point: finite, so the stage needs no -inf test.  Any
// finite score then overflows the tile sum to +inf and takes the slow path,
// where the rescale factor exp2(kRefInit - m'') is 0.
constexpr float kRefInit = -1e30f;
static_assert(BM == 32 * NW, "32 queries per wave");

#ifndef RA_FWD_AHEAD
#define RA_FWD_AHEAD 3    // LDS operands read ahead of their MFMAs
#endif

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from global memory (uniform base + per-lane byte offset)
// into LDS at lds_base + 16 * lane (lds_base in M0, uniform over the wave).
// Written out so that the compiler's wait-count analysis, which cannot tell
// the ring buffers apart, does not stall every LDS read on the loads in
// flight; the kernel waits for them itself (vmcnt) before the barrier that
// publishes a tile.  M0 is restored afterwards.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(lds_base)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// K/V tile of BN rows x D dims, row-major in LDS with 16-byte chunk swizzles.
template <int D>
struct KvTile {
    static constexpr int KCH = D / 8;               // 16-byte chunks per row
    static constexpr int ELEMS = BN * D;
    static constexpr int ROUNDS = BN * KCH / NT;    // 16-byte loads per thread per tensor
    static constexpr int LOADS = 2 * ROUNDS;        // loads per thread per tile
    static_assert(ROUNDS >= 1 && BN * KCH % NT == 0, "tile split");

    // K: chunk c of row r lives at chunk c ^ (r mod KCH): the 32 rows x 2
    // chunks of one MFMA operand read hit every bank equally.
    static __device__ __forceinline__ int k_swz(int row) { return row & (KCH - 1); }
    // V: one transpose read touches 8 rows (two groups of 4 consecutive) x 32
    // dims; the row-dependent chunk swizzle spreads them over all banks.
    static __device__ __forceinline__ int v_swz(int row) {
        return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
    }
    static __device__ __forceinline__ int k_off(int row, int ch) {
        return row * D + ((ch ^ k_swz(row)) << 3);
    }
    static __device__ __forceinline__ int v_off(int row, int ch) {
        return row * D + ((ch ^ v_swz(row)) << 3);
    }

    // Tile rows [0, BN) global -> LDS with no registers in between: lane l of
    // wave w fills 16-byte chunk NT*r + 64*w + l of the buffer, so it loads
    // the global chunk the swizzle puts there.  Round r covers the rows of
    // round 0 plus r*NT/KCH, a multiple of KCH, so both swizzles repeat and
    // Offs holds only round 0's byte offsets (from the tile's first row).
    static constexpr int ROWS_PER_ROUND = NT / KCH;
    static_assert(ROWS_PER_ROUND % KCH == 0 && ROWS_PER_ROUND % 4 == 0, "swizzles repeat per round");
    struct Offs {
        uint32_t k, v;
    };
    static __device__ __forceinline__ uint32_t chunk_off(int r, int w, int lane, int rows_in,
                                                         uint32_t row_bytes, bool is_v) {
        const int c = NT * r + 64 * w + lane;
        const int row = c / KCH, slot = c % KCH;
        const int sw = is_v ? v_swz(row) : k_swz(row);
        return (row < rows_in ? (uint32_t)row * row_bytes : 0u) + (uint32_t)((slot ^ sw) << 4);
    }
    static __device__ __forceinline__ Offs offsets(int w, int lane, uint32_t row_bytes) {
        Offs o;
        o.k = chunk_off(0, w, lane, BN, row_bytes, false);
        o.v = chunk_off(0, w, lane, BN, row_bytes, true);
        return o;
    }
    // Rows at or past klen (the ragged end of a chunk) repeat row 0: finite
    // data under keys that the mask removes.
    // Load q of a K/V tile pair: q < ROUNDS is round q of K, the rest the
    // rounds of V (so a stage can spread its loads between its MFMAs).  The K
    // and the V tile of one load set belong to different key tiles.  Only a
    // launch whose chunk length is not a multiple of BN (RAGGED) has tiles
    // with fewer than BN rows.
    template <bool RAGGED>
    static __device__ __forceinline__ void load_one(int q, const uint16_t* Kb, int klen, const uint16_t* Vb,
                                                    int vlen, const Offs& o, uint32_t row_bytes,
                                                    const uint16_t* Ks, const uint16_t* Vs, int w, int lane) {
        const bool is_v = q >= ROUNDS;
        const int r = is_v ? q - ROUNDS : q;
        const uint16_t* g = is_v ? Vb : Kb;
        const int len = is_v ? vlen : klen;
        const uint32_t lds = lds_addr((is_v ? Vs : Ks) + (NT * r + 64 * w) * 8);
        if (!RAGGED || len >= BN)
            lds_dma16(g + (int64_t)r * ROWS_PER_ROUND * (row_bytes / 2), is_v ? o.v : o.k, lds);
        else
            lds_dma16(g, chunk_off(r, w, lane, len, row_bytes, is_v), lds);
    }
    template <bool RAGGED>
    static __device__ __forceinline__ void load(const uint16_t* Kb, int klen, const uint16_t* Vb, int vlen,
                                                const Offs& o, uint32_t row_bytes, const uint16_t* Ks,
                                                const uint16_t* Vs, int w, int lane) {
#pragma unroll
        for (int q = 0; q < LOADS; ++q) load_one<RAGGED>(q, Kb, klen, Vb, vlen, o, row_bytes, Ks, Vs, w, lane);
    }
};

// max / sum / or of a value over the two half-waves (lanes l and l^32)
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
__device__ __forceinline__ bool halves_any(bool b) {
    const unsigned u = b ? 1u : 0u;
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return ((unsigned)r[0] | (unsigned)r[1]) != 0u;
}

// ----------------------------------------------------------------------------
// Key-tile cursor, in ring order: step t = 0..P-1 visits shard (rank - t) mod
// P (K/V travel r -> r+1, lesson 8 section 2), its chunks in local order and
// each chunk's tiles in ascending order; under the causal mask only the
// prefix of a chunk up to the tile's last query coordinate is visited.  The
// same order as the generic iterator of the other kernels, in 32-bit fields
// (positions < 2^30): advancing inside a segment is three adds, the segment
// walk runs only at its end.  All fields are uniform across the work-group.
// ----------------------------------------------------------------------------
struct KvCur {
    int t, lc;   // ring step and local chunk of the current segment
    int tl;      // tiles of the segment after the current one
    int krow;    // first K/V row (sharded order) of the current tile
    int kpos;    // mask coordinate of that row (global position when chunked)
    int cleft;   // rows of the chunk from that row on
};

__device__ __forceinline__ bool cur_seg(const FwdParams& p, int rank, int qmax, KvCur& c) {
    int s = rank - c.t;
    if (s < 0) s += p.P;
    const int cl = (int)p.c;
    c.krow = (p.kv_block ? 0 : s * (int)p.n) + c.lc * cl;
    c.kpos = p.striped ? (int)(s > rank) : global_chunk(p.P, p.chunks_per_rank, s, c.lc) * cl;
    int vis = cl;
    if (p.causal) vis = min(max(qmax - c.kpos + 1, 0), cl);
    c.tl = (vis + BN - 1) / BN - 1;
    c.cleft = cl;
    return c.tl >= 0;
}

// next non-empty segment; only called while tiles remain
__device__ __forceinline__ void cur_skip(const FwdParams& p, int rank, int qmax, KvCur& c) {
    do {
        if (++c.lc == p.chunks_per_rank) {
            c.lc = 0;
            ++c.t;
        }
    } while (c.t < p.step_hi && !cur_seg(p, rank, qmax, c));
}

__device__ __forceinline__ void cur_first(const FwdParams& p, int rank, int qmax, KvCur& c) {
    c.t = p.step_lo;
    c.lc = 0;
    if (!cur_seg(p, rank, qmax, c)) cur_skip(p, rank, qmax, c);
}

__device__ __forceinline__ void cur_next(const FwdParams& p, int rank, int qmax, KvCur& c) {
    if (c.tl > 0) {
        --c.tl;
        c.krow += BN;
        c.kpos += BN;
        c.cleft -= BN;
    } else {
        cur_skip(p, rank, qmax, c);
    }
}

// skip k tiles (whole segments at a time)
__device__ __forceinline__ void cur_advance(const FwdParams& p, int rank, int qmax, KvCur& c, int k) {
    while (k > c.tl) {
        k -= c.tl + 1;
        cur_skip(p, rank, qmax, c);
    }
    c.tl -= k;
    c.krow += k * BN;
    c.kpos += k * BN;
    c.cleft -= k * BN;
}

__device__ __forceinline__ int cur_count(const FwdParams& p, int rank, int qmax) {
    KvCur c;
    int n = 0;
    for (c.t = p.step_lo; c.t < p.step_hi; ++c.t)
        for (c.lc = 0; c.lc < p.chunks_per_rank; ++c.lc)
            if (cur_seg(p, rank, qmax, c)) n += c.tl + 1;
    return n;
}

// The loader's cursor: cur_next that also moves the tile's K row pointer, by
// one tile inside a segment and from the segment's first row after a jump.
__device__ __forceinline__ void lc_next(const FwdParams& p, int rank, int qmax, KvCur& c, const uint16_t*& kp,
                                        const uint16_t* Kg, int64_t row_stride) {
    if (c.tl > 0) {
        --c.tl;
        c.krow += BN;
        c.kpos += BN;
        c.cleft -= BN;
        kp += BN * row_stride;
    } else {
        cur_skip(p, rank, qmax, c);
        kp = Kg + c.krow * row_stride;
    }
}

// Masks keys of a tile outside the query's causal window or past a ragged
// chunk end.  Register r of block kb2 holds key kb2*32 + 16*(r/8) + 8h + r%8.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int lim) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int k0 = kb2 * 32 + 16 * (r >> 3) + (r & 7);
            s[kb2][r] = k0 < lim ? s[kb2][r] : kNegInf;
        }
}

// P = exp2(S*c - mu), its exact and bf16-rounded sums.
__device__ __forceinline__ void exp_tile(const f32x16 (&s)[2], float c, float mu, bf16x8 (&pb)[4],
                                         float& lsum, float& lrsum) {
    const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
    lsum = 0.f;
    lrsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i2 = 0; i2 < 8; i2 += 2) {
            const float e0 = fast_exp2(__builtin_fmaf(s[kk >> 1][8 * (kk & 1) + i2], c, -mu));
            const float e1 = fast_exp2(__builtin_fmaf(s[kk >> 1][8 * (kk & 1) + i2 + 1], c, -mu));
            lsum += e0 + e1;
            bf16x2 pr;
            pr[0] = (__bf16)e0;
            pr[1] = (__bf16)e1;
            lrsum = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes, lrsum, false);
            pb[kk][i2] = pr[0];
            pb[kk][i2 + 1] = pr[1];
        }
}

template <int D, bool RAGGED>
__global__ __launch_bounds__(NT) void fwd_bf16_kernel(FwdParams p) {
    using T = KvTile<D>;
    constexpr int KB = D / 16;    // MFMA k-blocks of Q K^T
    constexpr int DB = D / 32;    // 32-dim blocks of O^T
    constexpr int NQK = 2 * KB;   // K operands (MFMAs) of S^T per tile
    constexpr int NPV = 4 * DB;   // V operands (MFMAs) of O^T per tile
    constexpr int NMF = NQK + NPV;
    constexpr int AHEAD = RA_FWD_AHEAD;
    static_assert(AHEAD >= 1 && AHEAD <= NQK, "read-ahead depth");
    // 1 KB alignment leaves the low ten address bits to the in-tile offset,
    // so the swizzle XORs below can act on absolute LDS addresses
    __shared__ __attribute__((aligned(1024))) uint16_t ldsK[NBUF][T::ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t ldsV[NBUF][T::ELEMS];

    // work-group -> (query tile, key range): the splits of one tile are adjacent
    // With XCD grouping the ranges of one tile stay on the tile's XCD
    // (work-group ids 8 apart, as dispatch deals ids round-robin over the 8
    // XCDs), next to each other in its dispatch order.
    unsigned split, qid;
    if (p.xcd_pairs > 0 && p.kv_splits > 1) {
        const unsigned k = blockIdx.x >> 3;
        split = k % (unsigned)p.kv_splits;
        qid = ((k / (unsigned)p.kv_splits) << 3) | (blockIdx.x & 7u);
    } else {
        split = blockIdx.x % (unsigned)p.kv_splits;
        qid = blockIdx.x / (unsigned)p.kv_splits;
    }
    const QTile qt = decode_qtile<BM>(p, qid);
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, uniform in the wave
    const int h = lane >> 5, m = lane & 31;

    // this lane's query (MFMA column m of the wave's 32 queries)
    const int qi = w * 32 + m;
    const int pos0 = (int)qt.pos0;
    const int qpos = pos0 + qi;
    const int wq_lo = pos0 + w * 32;
    const int qmax = pos0 + qt.rows - 1;
    const float c = p.scale_log2;

    bf16x8 qop[KB];
    {
        const uint16_t* qp = (const uint16_t*)p.Q +
                             ((qt.b * p.q_rows + qt.q_row0 + qi) * p.Hq + qt.qh) * (int64_t)D;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const uint4 u = qi < qt.rows ? *(const uint4*)(qp + kb * 16 + h * 8) : make_uint4(0, 0, 0, 0);
            qop[kb] = __builtin_bit_cast(bf16x8, u);
        }
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_ref = kRefInit, l_run = 0.f, lr_run = 0.f;
    f32x16 zero16;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero16[r] = 0.f;

    const int64_t row_stride = (int64_t)p.Hkv * D;
    const uint32_t row_bytes = (uint32_t)(row_stride * 2);
    const uint16_t* Kg = (const uint16_t*)p.K + ((int64_t)qt.b * p.kv_rows * p.Hkv + qt.kvh) * D;
    const uint16_t* Vg = (const uint16_t*)p.V + ((int64_t)qt.b * p.kv_rows * p.Hkv + qt.kvh) * D;
    const typename T::Offs offs = T::offsets(w, lane, row_bytes);

    // ---- prologue.  Stage i issues the loads of K of tile i+3 and V of tile
    // i+2 (two stages before their use), so K of tiles 0-2 and V of tiles 0-1
    // go out here; the V buffer "before" tile 0 is zeroed (the first PV
    // product multiplies P = 0).  Past the work-group's last tile the loads
    // repeat that tile into buffers that no later stage reads, so every stage
    // issues the same number of loads and one wait count fits all stages.
    // This work-group's key range: tiles [i0, i0 + n) of the tile's visiting order.
    const int n_all = cur_count(p, qt.rank, qmax);
    const int i0 = (int)(((int64_t)n_all * split) / p.kv_splits);
    const int n = (int)(((int64_t)n_all * (split + 1)) / p.kv_splits) - i0;
    KvCur it_c, it_l;            // tile i of the loop; the K loader's tile
    const uint16_t* kp_l = Kg;   // K rows of the K loader's tile
    int klen_l = BN;             // rows of that tile inside its chunk
    int64_t voff_l = 0;          // K/V element offset of the V loader's tile (one behind)
    int vlen_l = BN;
    int issued = 0;              // tiles up to and including the K loader's
    // K loader to the next tile (it stays on the last one)
    auto advance_loader = [&]() {
        if (issued < n) {
            lc_next(p, qt.rank, qmax, it_l, kp_l, Kg, row_stride);
            if (RAGGED) klen_l = min(it_l.cleft, BN);
            ++issued;
        }
    };
    if (n > 0) {
        cur_first(p, qt.rank, qmax, it_c);
        cur_advance(p, qt.rank, qmax, it_c, i0);
        it_l = it_c;
        kp_l = Kg + it_l.krow * row_stride;
        klen_l = min(it_l.cleft, BN);
        issued = 1;
        T::template load<RAGGED>(kp_l, klen_l, Vg + (kp_l - Kg), klen_l, offs, row_bytes, ldsK[0], ldsV[0], w, lane);
        advance_loader();
        T::template load<RAGGED>(kp_l, klen_l, Vg + (kp_l - Kg), klen_l, offs, row_bytes, ldsK[1], ldsV[1], w, lane);
        advance_loader();
#pragma unroll
        for (int q = 0; q < T::ROUNDS; ++q)
            T::template load_one<RAGGED>(q, kp_l, klen_l, Vg, BN, offs, row_bytes, ldsK[2], ldsV[2], w, lane);
        // stage 0 loads V of tile 2 (the loader's tile now) and K of tile 3
        voff_l = kp_l - Kg;
        vlen_l = klen_l;
        advance_loader();
    }
    for (int e = t * 8; e < T::ELEMS; e += NT * 8)
        *(uint4*)(&ldsV[NBUF - 1][e]) = make_uint4(0, 0, 0, 0);

    // LDS operand addresses.  Both chunk swizzles are XORs into address bits
    // that the row part leaves clear, so the byte address of an operand is
    // (per-lane base) ^ (constant of its dim block) + (constant of its row
    // block and buffer): twelve XORed bases (eight for K, four for V) and an
    // immediate offset per read.
    //
    // K operand j: keys 32*(j%2).. (rows permuted), dims 16*(j/2)..: the two
    // S^T accumulators alternate, so consecutive MFMAs are independent.  Lane
    // (h, m) reads row 32*(j%2) + swap(m), 16-byte chunk 2*(j/2) + h, stored
    // at chunk (2*(j/2) + h) ^ (row mod KCH) = 2*(j/2) ^ (h ^ (swap(m) mod KCH)).
    const int sm = swap_bits23(m);
    uint32_t kbase = lds_addr(ldsK) + (uint32_t)(sm * 2 * D + 16 * (h ^ (sm & (T::KCH - 1))));
    // V operand j: keys 16*(j/DB).., dims 32*(j%DB)..; lane l of 16-lane group
    // g points at row 8*(g>>1) + (l%16)/4 (+4 for the second read) and dims
    // 16*(g&1) + 4*(l%4); it receives 4 consecutive keys of one dim.  The
    // swizzle flips the 64-byte dim block by v_swz(row)/4, which depends only
    // on the row bits that this base fixes.
    const int vr = 8 * h + ((lane & 15) >> 2);
    uint32_t vbase = lds_addr(ldsV) + (uint32_t)(vr * 2 * D + 64 * (T::v_swz(vr) >> 2) +
                                                 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) +
                                                 8 * (lane & 1));
    // operand j of ring buffer b (b known at compile time)
    auto read_k = [&](int j, int b) -> bf16x8 {
        const uint32_t a = (kbase ^ (uint32_t)(32 * (j >> 1))) + (uint32_t)(b * T::ELEMS * 2 + (j & 1) * 64 * D);
        return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)a;
    };
    auto read_v = [&](int j, int b) -> bf16x8 {
        const uint32_t a = (vbase ^ (uint32_t)(64 * (j % DB))) + (uint32_t)(b * T::ELEMS * 2 + (j / DB) * 32 * D);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)a);
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)(a + 8 * D));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // scores of tile 0
    f32x16 sa[2], sb[2];  // S of tiles i and i+1 (roles swap every iteration)
    bf16x8 pa[4], pb[4];  // P of tiles i-1 and i (roles swap every iteration)
    // K of tile 0 resident: the V of tiles 0-1 and K of tiles 1-2 may still fly
    static_assert(2 * T::LOADS < 16, "wait count fits the vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * T::LOADS));
    __syncthreads();
    // V operand 0 of the next stage's first MFMA (a PV product), read before
    // the barrier that opens the stage: V of tile i-1 has long been resident
    bf16x8 vpre = read_v(0, NBUF - 1);
    if (n > 0) {
#pragma unroll
        for (int j = 0; j < NQK; ++j) {
            const bf16x8 a = read_k(j, 0);
            sa[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[j >> 1], j < 2 ? zero16 : sa[j & 1], 0, 0, 0);
        }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) pa[kk][i2] = (__bf16)0.f;

    // One iteration: tile i, with i % NBUF == SLOT known at compile time.
    // sc / sn: S of tiles i / i+1; pp / pc: P of tiles i-1 / i.
    auto iteration = [&](auto slot, int i, f32x16 (&sc)[2], f32x16 (&sn)[2], bf16x8 (&pp)[4],
                         bf16x8 (&pc)[4]) {
        constexpr int SLOT = decltype(slot)::value;
        // K of tile i+1 resident (the loads of the previous stage may still
        // fly); after the barrier the K buffer of tile i-1 and the V buffer of
        // tile i-2 are free for K of tile i+3 and V of tile i+2
        __builtin_amdgcn_s_waitcnt(0x0F70 | T::LOADS);
        __syncthreads();
        // S_{i+1} from buffer (i+1) (stale data past the last tile: unused)
        constexpr int KBUF = (SLOT + 1) % NBUF, VBUF = (SLOT + NBUF - 1) % NBUF;

        const int klen = RAGGED ? min(it_c.cleft, BN) : BN;
        if ((RAGGED && klen < BN) || (p.causal && it_c.kpos + BN - 1 > wq_lo)) {
            const int lim = p.causal ? min(max(qpos - it_c.kpos + 1, 0), klen) : klen;
            mask_tile(sc, lim - 8 * h);
        }
        // The stage, slot by slot: MFMA slot j is PV operand j/2 (even j) or
        // QK operand j/2 (odd j); behind it the softmax runs one element per
        // slot as a three-step pipeline (FMA of element j+1, exp of element
        // j, sums and bf16 packing of element j-1), so exactly one exp and
        // about three other VALU instructions trail each MFMA and only a few
        // temporaries are live.  sched_barrier keeps this order.
        float lsum = 0.f, lrsum = 0.f;
        {
            // The twelve operand addresses stay in registers; the kernel for
            // ragged chunks, short of registers, recomputes them in every stage.
            if (RAGGED) asm volatile("" : "+v"(kbase), "+v"(vbase));
            const float mu = m_ref;
            const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
            constexpr int NE = 32;            // softmax elements per lane and tile
            constexpr int EPS = NE / NMF;     // elements per MFMA slot
            static_assert(NQK == NPV && EPS * NMF == NE, "slot layout");
            auto read_op = [&](int j) -> bf16x8 { return (j & 1) ? read_k(j >> 1, KBUF) : read_v(j >> 1, VBUF); };
            auto sval = [&](int e) -> float { return sc[e >> 4][e & 15]; };
            float tf[NE], ex[NE];
            bf16x8 ops[AHEAD];
#pragma unroll
            for (int j = 1; j <= AHEAD; ++j) ops[j % AHEAD] = read_op(j);
#pragma unroll
            for (int q = 0; q < EPS; ++q) tf[q] = __builtin_fmaf(sval(q), c, -mu);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j <= NMF; ++j) {
                if (j < NMF) {
                    const bf16x8 a = j == 0 ? vpre : ops[j % AHEAD];
                    const int q = j >> 1;
                    if ((j & 1) == 1)
                        sn[q & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[q >> 1], q < 2 ? zero16 : sn[q & 1],
                                                                            0, 0, 0);
                    else
                        oacc[q % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pp[q / DB], oacc[q % DB], 0, 0, 0);
                    if (j >= 1 && j + AHEAD < NMF) ops[j % AHEAD] = read_op(j + AHEAD);
                    // The loads of K of tile i+3 and V of tile i+2 (the
                    // loader cursor moved at the end of the previous stage):
                    // one behind each even slot from the second on, so that
                    // their scalar work is spread over the stage.
                    if (j >= 2 && (j & 1) == 0 && (j - 2) / 2 < T::LOADS)
                        T::template load_one<RAGGED>((j - 2) / 2, kp_l, klen_l, Vg + voff_l, vlen_l, offs, row_bytes,
                                                     ldsK[(SLOT + 3) % NBUF], ldsV[(SLOT + 2) % NBUF], w, lane);
                }
#pragma unroll
                for (int q = 0; q < EPS; ++q) {
                    const int e1 = (j + 1) * EPS + q, e0 = j * EPS + q, em = (j - 1) * EPS + q;
                    if (e1 < NE) tf[e1] = __builtin_fmaf(sval(e1), c, -mu);
                    if (e0 < NE) ex[e0] = fast_exp2(tf[e0]);
                    if (em >= 0 && em < NE) {
                        lsum = em == 0 ? ex[0] : lsum + ex[em];
                        if (em & 1) {
                            bf16x2 pr;
                            pr[0] = (__bf16)ex[em - 1];
                            pr[1] = (__bf16)ex[em];
                            lrsum = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes, lrsum, false);
                            pc[em >> 3][(em & 7) - 1] = pr[0];
                            pc[em >> 3][em & 7] = pr[1];
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // rare: a lane's sum exceeded the cap, or its first finite score
        const bool slow = lsum > kSumCap;
        if (__builtin_amdgcn_ballot_w64(slow) != 0) {
            const bool need = halves_any(slow);
            float mx = kNegInf;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb2][r]);
            mx = halves_max(mx) * c;
            const float m_new = need ? fmaxf(m_ref, mx) : m_ref;
            const float alpha = need ? fast_exp2(m_ref - m_new) : 1.f;  // 0 at the first finite score
            l_run *= alpha;
            lr_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m_ref = m_new;
            exp_tile(sc, c, m_new, pc, lsum, lrsum);
        }
        l_run += lsum;
        lr_run += lrsum;
        if (i + 1 < n) cur_next(p, qt.rank, qmax, it_c);
        // the next stage loads V of the K loader's tile and K of the one
        // after; this scalar work overlaps the stage's last MFMAs
        voff_l = kp_l - Kg;
        vlen_l = klen_l;
        advance_loader();
        vpre = read_v(0, SLOT);
    };

    static_assert(NBUF == 4, "the loop body is unrolled over the ring");
    for (int i = 0; i < n; i += 4) {
        iteration(std::integral_constant<int, 0>(), i, sa, sb, pa, pb);
        if (i + 1 < n) iteration(std::integral_constant<int, 1>(), i + 1, sb, sa, pb, pa);
        if (i + 2 < n) iteration(std::integral_constant<int, 2>(), i + 2, sa, sb, pa, pb);
        if (i + 3 < n) iteration(std::integral_constant<int, 3>(), i + 3, sb, sa, pb, pa);
    }
    // no load may still be writing LDS when the work-group ends
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (n > 0 && (n - 1) % 2 == 0) {
        // the last tile's P is in the second copy: move it to the first
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) pa[kk] = pb[kk];
    }

    // ---- epilogue: O += V_{n-1} P_{n-1}
    if (n > 0) {
        const int vb = (n - 1) % NBUF;
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
            const bf16x8 a = read_v(j, vb);
            oacc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pa[j / DB], oacc[j % DB], 0, 0, 0);
        }
    }

    // ---- finalize: O = O / l, LSE = m + ln l (natural log); with a running
    // state, fold this result into it (lesson 8 section 3, whole blocks):
    // O = (a O_old + b O_new) / (a + b), a = e^(lse_old - M), b = e^(lse - M)
    const float l_tot = halves_sum(l_run);
    const float lr_tot = halves_sum(lr_run);
    float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    float lse = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : kNegInf;
    // A work-group with no key tile leaves a running state as it is (the fold
    // with an empty block is the identity), and as a key range writes only its
    // lse = -inf: a merge reads no O of a part with weight 0.
    if (qi < qt.rows && !(n == 0 && p.fold)) {
        const int64_t obase = ((qt.b * p.q_rows + qt.q_row0 + qi) * p.Hq + qt.qh) * (int64_t)D +
                              (int64_t)split * p.o_split_stride;
        const int64_t lidx = ((int64_t)qt.b * p.Hq + qt.qh) * p.q_rows + qt.q_row0 + qi +
                             (int64_t)split * p.l_split_stride;
        float w_old = 0.f;
        if (p.fold) {
            const float lse_old = p.LSE[lidx];
            const float M = fmaxf(lse_old, lse);
            if (M != kNegInf) {
                const float a = __expf(lse_old - M), b = __expf(lse - M);
                const float rw = 1.f / (a + b);
                w_old = a * rw;
                inv *= b * rw;
                lse = M + __logf(a + b);
            }
        }
        const bool o_store = !(n == 0 && p.kv_splits > 1);
#pragma unroll
        for (int db = 0; db < DB && o_store; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                // accumulator registers 4*g4..4*g4+3 hold dims db*32 + 8*g4 + 4h + 0..3
                const int dim = db * 32 + 8 * g4 + 4 * h;
                float o0 = oacc[db][4 * g4 + 0] * inv, o1 = oacc[db][4 * g4 + 1] * inv;
                float o2 = oacc[db][4 * g4 + 2] * inv, o3 = oacc[db][4 * g4 + 3] * inv;
                if (p.fold) {
                    const float4 old = *(const float4*)((const float*)p.O + obase + dim);
                    o0 = __builtin_fmaf(w_old, old.x, o0);
                    o1 = __builtin_fmaf(w_old, old.y, o1);
                    o2 = __builtin_fmaf(w_old, old.z, o2);
                    o3 = __builtin_fmaf(w_old, old.w, o3);
                }
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
        // the new LSE depends on the old one, so the load above has returned
        // for every lane of the wave before this store issues
        if (h == 0) p.LSE[lidx] = lse;
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t s) {
    const int64_t tiles = (int64_t)p.n_ranks * p.chunks_per_rank * p.tiles_per_chunk;
    const int64_t grid = tiles * p.B * p.Hq * p.kv_splits;
    if (grid <= 0) return hipSuccess;
    // chunks of a multiple of BN rows have no ragged key tile
    const bool ragged = p.c % BN != 0;
    if (d == 128) {
        if (ragged)
            hipLaunchKernelGGL((fwd_bf16_kernel<128, true>), dim3((unsigned)grid), dim3(NT), 0, s, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<128, false>), dim3((unsigned)grid), dim3(NT), 0, s, p);
    } else {
        if (ragged)
            hipLaunchKernelGGL((fwd_bf16_kernel<64, true>), dim3((unsigned)grid), dim3(NT), 0, s, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<64, false>), dim3((unsigned)grid), dim3(NT), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace ra
