// ra_device.h -- device-side helpers shared by the gfx950 kernels of libra.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// MFMA row permutation for the QK^T product: swapping bits 2 and 3 of the
// row index makes the 32x32 accumulator give each half-wave 8 consecutive
// keys of every 16-key block (register r of half h <-> key 16*(r/8)+8h+r%8),
// which is the layout of the B operand of the following PV product.
__device__ __forceinline__ int swap_bits23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// 16-byte load of data that is read once: the non-temporal hint keeps the
// stream from displacing reused lines and reads HBM faster than a plain load
// (measured on gfx950: 6.6-6.8 TB/s against 6.1-6.2 for a read-only stream).
__device__ __forceinline__ uint4 load_once16(const void* p) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float xor32_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ __forceinline__ float xor32_sum(float x) { return x + __shfl_xor(x, 32, 64); }

// ----------------------------------------------------------------------------
// Round-robin KV blocks (Helix article: new tokens' KV goes to the devices of
// the KV-parallel group in turn, one block each).  Key x is in block
// j = x / block, on shard j mod P, at local row (j / P) * block + x mod block.
// With `total` keys, shard s holds the blocks s, s + P, ... below
// ceil(total / block); only the last block of the sequence can be partial.
// ----------------------------------------------------------------------------
__host__ __device__ inline int64_t rr_shard_len(int64_t total, int64_t block, int P, int s) {
    const int64_t nb = (total + block - 1) / block;
    if (s >= nb) return 0;
    int64_t len = ((nb - 1 - s) / P + 1) * block;
    if ((nb - 1) % P == s) len -= nb * block - total;
    return len;
}

// key range [k0, k1) (shard-local rows) and K/V element offset of one decode part
__device__ __forceinline__ void decode_part(const DecodeParams& p, int part, int b, int kvh, int d,
                                            int64_t& k0, int64_t& k1, int64_t& base) {
    const int s = part / p.parts_per_shard, j = part % p.parts_per_shard;
    const int64_t L = p.rr_block > 0 ? rr_shard_len(p.Skv, p.rr_block, p.n_shards, s) : p.Skv;
    const int64_t plen = (L + p.parts_per_shard - 1) / p.parts_per_shard;
    k0 = (int64_t)j * plen;
    k1 = k0 + plen < L ? k0 + plen : L;
    if (k0 > k1) k0 = k1;
    base = (((int64_t)s * p.B + b) * p.kv_cap * p.Hkv + kvh) * d;
}

// ----------------------------------------------------------------------------
// Chunk maps of the splits (lesson 8, section 4 and its exercise).
//
// With k chunks per rank and kP chunks in all, local chunk lc of rank r is
// global chunk (lc/2) P + r for even lc (picked from the front, one round of
// P per pair) and kP - 1 - (lc/2) P - r for odd lc (picked from the back).
// k = 1 is the contiguous split and k = 2 the usual zig-zag {r, 2P-1-r}.
// The global chunks fall into k bands of P consecutive ids; band b holds the
// even picks lc = 2b for b < ceil(k/2) and the odd picks lc = 2(k-1-b)+1
// above, so a global chunk maps back to (rank, lc) through its band.
// ----------------------------------------------------------------------------
__device__ __forceinline__ int global_chunk(int P, int k, int rank, int lc) {
    const int j = lc >> 1;
    return (lc & 1) ? k * P - 1 - j * P - rank : j * P + rank;
}

__device__ __forceinline__ int band_chunk(int k, int b) {
    return b < (k + 1) / 2 ? 2 * b : 2 * (k - 1 - b) + 1;
}

// ----------------------------------------------------------------------------
// Query tiles of one prefill launch.
//
// Work-group id -> (batch, query head, rank, local chunk, tile).  Tiles are
// handed out heaviest first: under the causal mask the work of a query tile
// grows with its mask coordinate, so tiles are enumerated by descending
// global chunk and, inside a chunk, descending offset (striped split: by
// descending local offset, ranks interleaved, since every rank's tile at one
// offset does the same work).  When the number of (batch, kv head) pairs is a
// multiple of the 8 XCDs, work-group ids are grouped so that all query heads
// reading one kv head run on one XCD (ids are dispatched round-robin over the
// XCDs) and share its L2.
// ----------------------------------------------------------------------------
struct QTile {
    int b, qh, kvh, rank;
    int64_t q_row0;  // first row in the Q/O tensors
    int64_t pos0;    // mask coordinate of the first row
    int rows;        // valid rows (<= BLOCK_M)
};

template <int BM>
__device__ __forceinline__ QTile decode_qtile(const FwdParams& p, unsigned id) {
    QTile t;
    int trank, pair, g;
    if (p.xcd_pairs > 0) {
        const unsigned xcd = id & 7u, k = id >> 3;
        const unsigned per = (unsigned)(p.xcd_pairs * p.G);
        trank = (int)(k / per);
        const unsigned rem = k % per;
        pair = (int)xcd * p.xcd_pairs + (int)(rem / p.G);
        g = (int)(rem % p.G);
    } else {
        const unsigned per = (unsigned)(p.B * p.Hq);
        trank = (int)(id / per);
        const unsigned rem = id % per;
        pair = (int)(rem / p.G);
        g = (int)(rem % p.G);
    }
    t.b = pair / p.Hkv;
    t.kvh = pair % p.Hkv;
    t.qh = t.kvh * p.G + g;
    const int tpc = p.tiles_per_chunk;
    const int k = p.chunks_per_rank;
    int rank, lc, j;
    int64_t pos_chunk;
    if (p.striped) {
        j = tpc - 1 - trank / p.n_ranks;
        rank = p.rank_lo + trank % p.n_ranks;
        lc = 0;
        pos_chunk = 0;
    } else {
        const int cidx = trank / tpc;
        j = tpc - 1 - (trank % tpc);
        if (p.n_ranks == 1) {
            rank = p.rank_lo;
            lc = band_chunk(k, k - 1 - cidx);
        } else {
            const int gch = k * p.P - 1 - cidx;
            const int band = gch / p.P;
            lc = band_chunk(k, band);
            rank = (lc & 1) ? k * p.P - 1 - (lc >> 1) * p.P - gch : gch - band * p.P;
        }
        pos_chunk = (int64_t)global_chunk(p.P, k, rank, lc) * p.c;
    }
    t.rank = rank;
    const int64_t off = (int64_t)j * BM;
    t.q_row0 = (p.q_local ? 0 : (int64_t)rank * p.n) + (int64_t)lc * p.c + off;
    t.pos0 = pos_chunk + off;
    const int64_t left = p.c - off;
    t.rows = left < BM ? (int)left : BM;
    return t;
}

// ----------------------------------------------------------------------------
// Ring visiting order of the key tiles of one query tile.
//
// Step t = 0..P-1 visits shard s = (rank - t) mod P (lesson 8, section 2: K/V
// travel r -> r+1, so after t hops rank r holds the block that started at
// r - t).  Inside a shard the chunks are visited in local order and each
// chunk's key tiles in ascending order.  Under the causal mask only the
// prefix of a chunk whose positions do not exceed the tile's last query is
// visited (in mask coordinates); tiles wholly in the future of every query of
// the tile are skipped.
// All fields are uniform across the work-group.
// ----------------------------------------------------------------------------
struct KvIter {
    int t, lc, tile, ntiles;
    int64_t krow;  // first K/V row (sharded order) of the current chunk
    int64_t kpos;  // mask coordinate of that row
};

__device__ __forceinline__ void kv_seg(const FwdParams& p, int rank, int64_t qmax, int bn,
                                       KvIter& it) {
    int s = rank - it.t;
    if (s < 0) s += p.P;
    it.krow = (p.kv_block ? 0 : (int64_t)s * p.n) + (int64_t)it.lc * p.c;
    it.kpos = p.striped ? (int64_t)(s > rank)
                        : (int64_t)global_chunk(p.P, p.chunks_per_rank, s, it.lc) * p.c;
    int64_t vis = p.c;
    if (p.causal) {
        vis = qmax - it.kpos + 1;
        if (vis < 0) vis = 0;
        if (vis > p.c) vis = p.c;
    }
    it.ntiles = (int)((vis + bn - 1) / bn);
}

__device__ __forceinline__ bool kv_first(const FwdParams& p, int rank, int64_t qmax, int bn,
                                         KvIter& it) {
    it.t = p.step_lo;
    it.lc = 0;
    it.tile = 0;
    kv_seg(p, rank, qmax, bn, it);
    while (it.tile >= it.ntiles) {
        if (++it.lc == p.chunks_per_rank) {
            it.lc = 0;
            if (++it.t == p.step_hi) return false;
        }
        kv_seg(p, rank, qmax, bn, it);
    }
    return true;
}

// Number of key tiles the iteration visits.
__device__ __forceinline__ int kv_count(const FwdParams& p, int rank, int64_t qmax, int bn) {
    KvIter it;
    int n = 0;
    for (it.t = p.step_lo; it.t < p.step_hi; ++it.t)
        for (it.lc = 0; it.lc < p.chunks_per_rank; ++it.lc) {
            kv_seg(p, rank, qmax, bn, it);
            n += it.ntiles;
        }
    return n;
}

__device__ __forceinline__ bool kv_next(const FwdParams& p, int rank, int64_t qmax, int bn,
                                        KvIter& it) {
    ++it.tile;
    while (it.tile >= it.ntiles) {
        if (++it.lc == p.chunks_per_rank) {
            it.lc = 0;
            if (++it.t == p.step_hi) return false;
        }
        it.tile = 0;
        kv_seg(p, rank, qmax, bn, it);
    }
    return true;
}

}  // namespace ra
