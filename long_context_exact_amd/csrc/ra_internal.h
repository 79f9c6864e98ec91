// ra_internal.h -- parameter blocks shared by the host entry points and the
// kernel launchers of libra.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Which query tiles one prefill launch covers and how they are ordered.
//
// The queries of a rank are cut into tiles that never straddle a chunk (a
// rank owns one chunk under the contiguous and the striped split and k under
// zig-zag), so the mask coordinates inside one query tile are consecutive.
// Key tiles likewise stay inside one chunk.
//
// Mask coordinates.  For the chunked splits the coordinate of a token is its
// global position.  Under the striped split rank r holds positions r + iP,
// i = 0..n-1, and a key of shard s at local index j is visible to the query
// at local index i iff s + jP <= r + iP, i.e. j + (s > r) <= i: the query's
// coordinate is i and the key's is j + (s > r).  Either way a key is visible
// iff its coordinate does not exceed the query's, and coordinates advance by
// one per row inside a chunk.
struct FwdParams {
    const void* Q;     // [B, q_rows, Hq, d]
    const void* K;     // [B, S, Hkv, d], sharded order (kv_block: [B, n, Hkv, d])
    const void* V;     // same as K
    void* O;           // [B, q_rows, Hq, d]
    float* LSE;        // [B, Hq, q_rows]
    int64_t S;         // total tokens (all shards)
    int64_t kv_rows;   // rows per batch entry of K/V: S, or n for a block
    int64_t n;         // tokens per shard, S / P
    int64_t c;         // tokens per chunk: n / chunks_per_rank
    int64_t q_rows;    // rows of Q/O/LSE: S for all ranks, n for one rank
    int B, Hq, Hkv, G; // G = Hq / Hkv
    int P;
    int striped;       // 1: token round-robin split (one chunk per rank)
    int causal;
    int o_f32;         // 1: O is fp32, 0: O has the input dtype (bf16)
    int rank_lo;       // first rank of this launch
    int n_ranks;       // ranks in this launch (P for all, 1 for one rank)
    int q_local;       // 1: Q/O/LSE rows are rank-local (row 0 = first row of rank_lo)
    int tiles_per_chunk;   // ceil(c / BLOCK_M)
    int chunks_per_rank;   // k: 1 contiguous or striped, k >= 2 zig-zag
    int xcd_pairs;     // (b, kv head) pairs per XCD group, 0 = no XCD grouping
    // Key-range splits: each query tile's visiting order of key tiles is cut
    // into kv_splits contiguous ranges, one work-group each.  With more than
    // one split, O and LSE point at fp32 partial buffers and split s writes
    // its (O, LSE) partial at offsets s * o_split_stride / s * l_split_stride.
    int kv_splits;
    int64_t o_split_stride, l_split_stride;
    // Ring steps visited: t in [step_lo, step_hi) (0 and P for a whole pass).
    // kv_block = 1: K/V hold only the shard of step step_lo, [B, n, Hkv, d]
    // (a received block), instead of all P shards.  fold = 1: O (fp32) and
    // LSE hold a running state that this launch's result is folded into.
    int step_lo, step_hi;
    int kv_block;
    int fold;
    float scale_log2;  // log2(e) / sqrt(d)
    float scale;       // 1 / sqrt(d)
};

// Decode over a KV cache held as n_shards shard caches (one per device of a
// KV-parallel group): row r of batch entry b of shard s sits at row
// (s * B + b) * kv_cap + r of K and V.  One contiguous cache is one shard
// with kv_cap = Skv.  Under round-robin blocks (rr_block > 0) key x of the
// sequence lives in shard (x / rr_block) mod n_shards, so shard lengths
// follow from Skv alone.  Each shard is cut into parts_per_shard parts.
struct DecodeParams {
    const void* Q;     // [B, Sq, Hq, d]
    const void* K;     // [n_shards, B, kv_cap, Hkv, d]
    const void* V;
    float* O_parts;    // [n_parts, B*Sq*Hq, d]
    float* lse_parts;  // [n_parts, B*Sq*Hq]
    int64_t Sq;
    int64_t Skv;       // keys of the sequence (all shards)
    int64_t kv_cap;    // rows per (shard, batch entry)
    int64_t rr_block;  // 0: one contiguous cache; > 0: round-robin block size
    int B, Hq, Hkv, G;
    int n_parts;       // n_shards * parts_per_shard
    int n_shards, parts_per_shard;
    float scale_log2;
};

struct MergeParams {
    const float* O_parts;
    const float* lse_parts;
    void* O;
    float* lse;
    int64_t rows;
    int n_parts;
    int out_bf16;
    // lse_bhq = 1: rows are (b, q, h) of a [B, q_rows, Hq, d] output whose LSE
    // is laid out [B, Hq, q_rows] (partials and result alike); 0: lse[row]
    int lse_bhq;
    int64_t q_rows;
    int Hq;
    // optional running state, folded in as a first part and overwritten in
    // place: O_state (fp32 rows x d) is then also O, lse_state (laid out like
    // lse) also lse; null when there is none
    const float* O_state;
    const float* lse_state;
};

// Launchers (each returns hipSuccess or the launch error).
hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeParams& p, int d, hipStream_t s);
hipError_t launch_decode_f32(const DecodeParams& p, int d, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, int d, hipStream_t s);
hipError_t launch_kv_append_rr(void* K_cache, void* V_cache, const void* K_new, const void* V_new,
                              int B, int64_t row_bytes, int P, int64_t cap, int64_t len,
                              int64_t n_new, int64_t block, hipStream_t s);
hipError_t launch_head_a2a(const void* src, void* dst, int64_t B, int64_t S, int P, int64_t run_bytes,
                           int inverse, hipStream_t s);
hipError_t launch_layout(const void* src, void* dst, int64_t outer, int64_t S, int64_t inner_bytes,
                         int P, int chunks_per_rank, int striped, int inverse, hipStream_t s);

// Tile shapes of the prefill kernels (the host needs them for the grid).
constexpr int FWD_BF16_BLOCK_M = 256;
constexpr int FWD_F32_BLOCK_M = 64;

}  // namespace ra
