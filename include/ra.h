/*
 * ra.h -- C ABI of the MI355X (gfx950) ring-attention library (libra.so).
 *
 * The library computes the forward pass of exact ring attention for
 * sequence-parallel ranks that are simulated on one GPU: all P key/value
 * shards are resident, and each rank's query block visits them in ring
 * order.  It also computes attention of a few query tokens against a KV cache
 * split into shards, and merges the per-shard (O, lse) partials.
 *
 * Sources (the pages this follows):
 *   [L8]  Lesson 8 "Context Parallelism (CP)", hpc.payai.win: section 1
 *         (sequence split, s_local = s / N_cp, tensors (b, s_local, h)),
 *         section 2 (ring loop: Q_r stays, K/V move r -> r+1, at step t rank r
 *         holds the block from (r - t) mod P), section 3 (online softmax
 *         update of (m, l, O)), section 4 (causal mask j <= i; naive split and
 *         the zig-zag split where rank r holds chunks r and 2P-1-r) and the
 *         exercise (the zig-zag rule for more than two chunks per rank).
 *   [P1]  "Paralelismo de sequencia e atencao de anel", aiunderstanding.org:
 *         every query ends up seeing every key; the result equals full
 *         attention; striped attention is named as another way to balance
 *         the causal work (not defined there).
 *   [HX]  "NVIDIA Helix Parallelism" article, storagereview.com, phase 1: the
 *         KV cache is split along the sequence across devices, each computes a
 *         partial result, and one exchange combines them.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or keeps them.  Every call validates its
 *     arguments, enqueues kernels on `stream` (a hipStream_t passed as void*;
 *     NULL is the default stream) and returns without synchronising.  A
 *     kernel fault surfaces at the caller's next synchronisation.
 *   - Layouts are row-major with the last dimension contiguous.  Sequence
 *     tensors are [B, S, H, d]; d (head dimension) is 64 or 128.
 *   - dtype: RA_DTYPE_F32 (float) or RA_DTYPE_BF16 (bfloat16 bit patterns,
 *     uint16) for Q, K and V.  The attention output O has its own o_dtype:
 *     with bf16 inputs it may be bf16 (rounded to nearest even) or fp32 (the
 *     fp32 accumulator, unrounded); with fp32 inputs it is fp32.  LSE and
 *     partials are fp32.
 *   - The softmax scale is 1/sqrt(d) ([L8] section 1).
 *   - Grouped-query attention: query head h reads key/value head
 *     h / (Hq/Hkv) (contiguous groups; Hq must be a multiple of Hkv).
 *   - LSE is the natural-log softmax denominator of the scaled scores,
 *     m + ln(sum_j exp(s_j - m)); a row that sees no key gets O = 0 and
 *     LSE = -inf.
 *   - Return value: RA_OK (0) or a negative ra_status.  Argument checks run
 *     before any HIP call, so invalid arguments are reported without touching
 *     the device.  ra_last_error() gives a message for the calling thread's
 *     last failure.
 *   - Calls are re-entrant; the only global state is the thread-local error
 *     message and the device scratch of ra_fwd_rank_noalloc (its calls on one
 *     GPU share that scratch).
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RA_OK = 0,
    RA_ERR_INVALID_ARG = -1, /* null pointer, size <= 0, rank out of range, bad enum */
    RA_ERR_UNSUPPORTED = -2, /* valid but not implemented: d, Hq % Hkv, uneven split */
    RA_ERR_HIP = -3          /* a HIP runtime call or kernel launch failed */
} ra_status;

typedef enum {
    RA_LAYOUT_CONTIGUOUS = 0, /* P shards of S/P tokens; shard r = tokens [r*S/P, (r+1)*S/P) */
    RA_LAYOUT_ZIGZAG = 1,     /* 2P chunks of S/(2P) tokens; shard r = [chunk r ; chunk 2P-1-r] */
    RA_LAYOUT_STRIPED = 2     /* tokens dealt round-robin; shard r = positions r, r+P, r+2P, ... */
} ra_layout;

/* Zig-zag with k chunks per rank, 1 <= k <= RA_MAX_CHUNKS_PER_RANK: kP chunks
 * of S/(kP) tokens; shard r = [chunk g(r,0) ; ... ; chunk g(r,k-1)] with
 * g(r, i) = (i/2)P + r for even i and kP-1-(i/2)P-r for odd i ([L8] exercise).
 * RA_LAYOUT_ZIGZAG_K(1) is the contiguous split, RA_LAYOUT_ZIGZAG_K(2) the
 * usual zig-zag. */
#define RA_LAYOUT_ZIGZAG_K(k) (0x100 | (k))
#define RA_MAX_CHUNKS_PER_RANK 64

typedef enum { RA_DTYPE_F32 = 0, RA_DTYPE_BF16 = 1 } ra_dtype;

/*
 * Rank-sharded sequence order.  A sequence tensor "in sharded order" stores
 * shard 0's tokens, then shard 1's, ... (each shard S/P tokens).  Under
 * RA_LAYOUT_CONTIGUOUS this is the natural order.  Under RA_LAYOUT_ZIGZAG
 * shard r holds chunk r followed by chunk 2P-1-r ([L8] section 4B and the
 * exercise's answer, which lists the chunks in that order); under
 * RA_LAYOUT_ZIGZAG_K(k) its k chunks in the order g(r, 0..k-1).  Under
 * RA_LAYOUT_STRIPED shard r holds positions r, r+P, ..., S-P+r in ascending
 * order ([P1] only names striped attention; dealing single tokens
 * round-robin is this library's reading).  The causal mask always compares
 * natural (global) positions ([L8] section 4).
 */

/*
 * ra_fwd_rank -- forward pass of one simulated rank ([L8] sections 2-4).
 *
 * Rank `rank` keeps its query block Q_r fixed and, for t = 0..P-1, attends the
 * resident K/V shard (rank - t) mod P, folding each block into its running
 * online-softmax state; after P steps it writes O_r and LSE_r.
 *
 *   Q_r   [B, S/P, Hq, d]   the rank's local queries (its shard of Q)
 *   K, V  [B, S, Hkv, d]    all P shards, in sharded order
 *   O_r   [B, S/P, Hq, d]   output in o_dtype
 *   LSE_r [B, Hq, S/P]      fp32 output
 *   causal: 0 or 1; layout: ra_layout; dtype, o_dtype: ra_dtype.
 * Requirements: S % P == 0 (contiguous, striped), S % (2P) == 0 (zig-zag),
 * S % (kP) == 0 (RA_LAYOUT_ZIGZAG_K(k)); S < 2^30 for bf16; P <= 4096;
 * 0 <= rank < P; Hq % Hkv == 0; d in {64, 128}.  Q_r/O_r must not alias K/V.
 * For B == 1, Q_r/O_r may point at rows rank*S/P of full sharded tensors.
 * The rows written are bit-identical to the same rows of ra_fwd_all.
 */
int ra_fwd_rank(const void* Q_r, const void* K, const void* V, void* O_r, float* LSE_r,
                int B, int Hq, int Hkv, int64_t S, int d, int P, int rank,
                int causal, int layout, int dtype, int o_dtype, void* stream);

/*
 * ra_fwd_all -- all P simulated ranks in one launch.
 *   Q, O [B, S, Hq, d], K, V [B, S, Hkv, d], LSE [B, Hq, S]; all sequence
 *   dimensions in sharded order.  Same requirements as ra_fwd_rank.
 * Equals the concatenation of ra_fwd_rank over rank = 0..P-1, bit for bit.
 */
int ra_fwd_all(const void* Q, const void* K, const void* V, void* O, float* LSE,
               int B, int Hq, int Hkv, int64_t S, int d, int P,
               int causal, int layout, int dtype, int o_dtype, void* stream);

/*
 * ra_fwd_rank_ws, ra_fwd_all_ws -- ra_fwd_rank / ra_fwd_all with a caller
 * workspace that lets the library split each query tile's walk over the key
 * tiles (the ring order above) into kv_splits contiguous ranges, run them on
 * separate work-groups, and combine the (O, lse) partials of the ranges with
 * the fold of [L8] section 3 (the ra_merge_partials formula).  This keeps the
 * GPU busy when a launch has few query tiles (a short rank share) or when
 * one causal tile does much more work than the rest.
 *   kv_splits  0: automatic (about two work-groups per compute unit, at most
 *              8 ranges, fewer if the workspace is smaller); 1..RA_MAX_KV_SPLITS:
 *              exactly that many ranges (a range may be empty).
 *   workspace  device memory of workspace_bytes, 16-byte aligned, owned by
 *              the caller, not aliasing any tensor argument; its contents on
 *              entry do not matter and are garbage on return.  NULL or too
 *              small: automatic mode uses fewer splits (1 needs none); an
 *              explicit kv_splits fails with RA_ERR_INVALID_ARG.
 * All other arguments and requirements are those of ra_fwd_rank / ra_fwd_all.
 * With one split the result is bit-identical to ra_fwd_rank / ra_fwd_all; for
 * a given kv_splits the rows of ra_fwd_rank_ws equal those of ra_fwd_all_ws
 * bit for bit.  Other split counts agree within rounding.
 */
#define RA_MAX_KV_SPLITS 64

int ra_fwd_rank_ws(const void* Q_r, const void* K, const void* V, void* O_r, float* LSE_r,
                   int B, int Hq, int Hkv, int64_t S, int d, int P, int rank,
                   int causal, int layout, int dtype, int o_dtype,
                   int kv_splits, void* workspace, int64_t workspace_bytes, void* stream);

int ra_fwd_all_ws(const void* Q, const void* K, const void* V, void* O, float* LSE,
                  int B, int Hq, int Hkv, int64_t S, int d, int P,
                  int causal, int layout, int dtype, int o_dtype,
                  int kv_splits, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * ra_fwd_rank_noalloc -- ra_fwd_rank_ws for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The key-range partials go to a scratch array that
 * the library holds in device memory, RA_SCRATCH_BYTES per GPU it runs on,
 * from the first call on that GPU until the process ends; the call itself
 * makes no hipMalloc, hipFree or other allocating call.  The caller still
 * passes the inputs and outputs.
 *   kv_splits: 0 = automatic (as ra_fwd_rank_ws with a workspace of
 *              RA_SCRATCH_BYTES: fewer ranges where their partials would not
 *              fit); 1..RA_MAX_KV_SPLITS = exactly that many, and
 *              RA_ERR_INVALID_ARG (before any HIP call) when their partials,
 *              ra_fwd_workspace_bytes(..., all_ranks = 0, ..., kv_splits),
 *              exceed RA_SCRATCH_BYTES.
 * The result equals ra_fwd_rank_ws with the same kv_splits (and, in automatic
 * mode, a workspace of RA_SCRATCH_BYTES) bit for bit.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be ordered by the caller.  The
 * scratch's contents on entry do not matter; every range rewrites its
 * partials.  All other arguments and requirements are those of ra_fwd_rank.
 */
#define RA_SCRATCH_BYTES ((int64_t)128 << 20)

int ra_fwd_rank_noalloc(const void* Q_r, const void* K, const void* V, void* O_r, float* LSE_r,
                        int B, int Hq, int Hkv, int64_t S, int d, int P, int rank,
                        int causal, int layout, int dtype, int o_dtype, int kv_splits,
                        void* stream);

/*
 * ra_ring_step -- one step of the ring loop of one rank ([L8] section 2),
 * for a deployment where K/V blocks arrive one at a time (a P2P receive
 * buffer) instead of all being resident.
 *
 * At step t rank `rank` holds the K/V block of shard s = (rank - t) mod P.
 * The call attends the rank's queries to that block (causal mask on global
 * positions, as ra_fwd_rank) and folds the result into the running state
 * (O_acc, LSE_acc) with the update of [L8] section 3 applied to the whole
 * block: M = max(lse_old, lse_t), a = e^(lse_old-M), b = e^(lse_t-M),
 * O = (a O_old + b O_t)/(a+b), LSE = M + ln(a+b).
 *   Q_r          [B, S/P, Hq, d]   the rank's local queries (dtype)
 *   K_blk, V_blk [B, S/P, Hkv, d]  shard s's rows in sharded order (dtype)
 *   O_acc        [B, S/P, Hq, d]   fp32 running output, normalised
 *   LSE_acc      [B, Hq, S/P]      fp32 running LSE
 * Step t = 0 initialises the state (its previous contents do not matter);
 * steps t > 0 fold into it and may come in any order after t = 0.  After
 * all P steps O_acc and LSE_acc equal ra_fwd_rank's fp32 output within
 * rounding (the fold reference points differ).  A bf16 copy of O_acc is
 * ra_merge_partials(O_acc, Z, O, NULL, 1, rows, d, RA_DTYPE_BF16) with Z a
 * zero-filled fp32 array of rows = B*(S/P)*Hq entries: one part of weight 1
 * (LSE_acc itself is laid out [B, Hq, S/P], not by row).
 * Requirements: those of ra_fwd_rank, 0 <= t < P; the state must not alias
 * Q_r or the block.  Launches of one rank's steps must be ordered (one
 * stream, or events): each reads and writes the whole state.
 */
int ra_ring_step(const void* Q_r, const void* K_blk, const void* V_blk, float* O_acc,
                 float* LSE_acc, int B, int Hq, int Hkv, int64_t S, int d, int P, int rank,
                 int t, int causal, int layout, int dtype, void* stream);

/*
 * ra_ring_step_ws -- ra_ring_step with key-range splits, for steps whose
 * launch has too few query tiles to fill the GPU (under the causal split,
 * steps t > 0 give work to only some of a rank's tiles).  Each tile's key
 * tiles of the block are cut into kv_splits contiguous ranges, one
 * work-group each, whose fp32 (O, lse) partials go to `workspace`; one merge
 * then folds the ranges and, for t > 0, the running state (as its first
 * part) into (O_acc, LSE_acc), in place ([L8] section 3 applied to the
 * ranges and the state).
 *   kv_splits: 0 = automatic (about two work-groups per compute unit, at
 *              most 8 and at most one per 1024 keys of the block, fewer if
 *              the workspace is smaller), 1..64 = exactly that many
 *              (RA_ERR_INVALID_ARG if the workspace is too small).
 *   workspace: device memory owned by the caller, 16-byte aligned, of
 *              ra_fwd_workspace_bytes(..., all_ranks = 0, ...) bytes for the
 *              same shape and kv_splits (enough for the automatic choice);
 *              NULL with workspace_bytes = 0 runs one range.
 * With one range it is ra_ring_step exactly (bit for bit).  The ranges cost
 * a merge launch and fp32 traffic per step (partials and the state), so
 * they pay only when a step leaves compute units idle and its block is
 * large enough.  Other counts
 * agree with it within rounding.  Requirements and ordering: those of
 * ra_ring_step; the workspace must not alias any tensor, and calls that
 * share it must be ordered.
 */
int ra_ring_step_ws(const void* Q_r, const void* K_blk, const void* V_blk, float* O_acc,
                    float* LSE_acc, int B, int Hq, int Hkv, int64_t S, int d, int P, int rank,
                    int t, int causal, int layout, int dtype, int kv_splits, void* workspace,
                    int64_t workspace_bytes, void* stream);

/*
 * ra_fwd_workspace_bytes -- workspace that ra_fwd_rank_ws and ra_ring_step_ws
 * (all_ranks = 0) or ra_fwd_all_ws (all_ranks = 1) need for kv_splits ranges
 * (0: the automatic choice): kv_splits * rows * (d + 1) * 4 bytes with
 * rows = B * Hq * (S/P or S),
 * 0 for one range.  Returns a negative ra_status for invalid shapes.  No HIP
 * call is made.
 */
int64_t ra_fwd_workspace_bytes(int B, int Hq, int Hkv, int64_t S, int d, int P, int all_ranks,
                               int causal, int layout, int dtype, int kv_splits);

/*
 * ra_merge_partials -- combine (O, lse) partials that were computed over
 * disjoint key sets of the same query rows ([L8] section 3 applied to whole
 * shards; [HX] phase 1):
 *   M = max_p lse_p, w_p = exp(lse_p - M),
 *   lse = M + ln(sum_p w_p), O = sum_p w_p O_p / sum_p w_p.
 * Partials with lse_p = -inf carry weight 0; a row whose partials are all
 * -inf gets O = 0, lse = -inf.
 *   O_parts   [n_parts, rows, d] fp32     lse_parts [n_parts, rows] fp32
 *   O         [rows, d] in out_dtype      lse       [rows] fp32 (may be NULL)
 * Requirements: n_parts >= 1, rows >= 1, d in {64, 128}.
 */
int ra_merge_partials(const float* O_parts, const float* lse_parts, void* O, float* lse,
                      int n_parts, int64_t rows, int d, int out_dtype, void* stream);

/*
 * ra_attn_partial -- per-shard partial attention over a KV cache that is
 * split along the sequence ([HX] phase 1).  Non-causal: every query sees
 * every key of its shard.
 *   Q  [B, Sq, Hq, d]      K, V [B, Skv, Hkv, d]   (dtype)
 *   Skv is cut into n_parts contiguous parts of ceil(Skv / n_parts) keys
 *   (the last part may be shorter or empty); part p covers keys
 *   [p*ceil, min(Skv, (p+1)*ceil)).
 *   O_parts   [n_parts, B*Sq*Hq, d] fp32, row (b*Sq + i)*Hq + h
 *   lse_parts [n_parts, B*Sq*Hq]    fp32
 * Requirements: Sq * (Hq/Hkv) <= 32, n_parts >= 1, d in {64, 128}.
 * An empty part yields O = 0, lse = -inf, which ra_merge_partials ignores.
 */
int ra_attn_partial(const void* Q, const void* K, const void* V, float* O_parts,
                    float* lse_parts, int B, int Hq, int Hkv, int64_t Sq, int64_t Skv,
                    int d, int n_parts, int dtype, void* stream);

/*
 * Round-robin KV cache of a KV-parallel group ([HX]: new tokens' KV is
 * written to the devices of the group in turn, one block of tokens each, so
 * every device's cache grows evenly).  Key x of a sequence is in block
 * j = x / block, held by shard j mod P at shard-local row
 * (j / P) * block + x mod block.  The P shard caches are one tensor
 * [P, B, cap, Hkv, d] (dtype), shard-major, so each shard's cache is one
 * contiguous region as it would be on its own device.
 *
 * ra_kv_append_rr -- write the K/V of n_new new tokens at sequence positions
 * len .. len+n_new-1 into their shards.
 *   K_new, V_new  [B, n_new, Hkv, d]; K_cache, V_cache as above.
 * Rows of other positions are not touched.  All pointers 16-byte aligned.
 * Requirements: len >= 0, n_new >= 1, block >= 1, every shard's length after
 * the append <= cap (shard 0 is the longest), d in {64, 128}.
 */
int ra_kv_append_rr(void* K_cache, void* V_cache, const void* K_new, const void* V_new,
                    int B, int Hkv, int d, int P, int64_t cap, int64_t len, int64_t n_new,
                    int64_t block, int dtype, void* stream);

/*
 * ra_attn_partial_rr -- ra_attn_partial over the round-robin cache of a
 * sequence of `len` keys: every shard is cut into parts_per_shard parts of
 * its own length, part p*parts_per_shard + j covering the j-th range of shard
 * p ([HX] phase 1: each device computes partials over its own cache).
 *   Q [B, Sq, Hq, d]; O_parts [P*parts_per_shard, B*Sq*Hq, d] fp32;
 *   lse_parts [P*parts_per_shard, B*Sq*Hq] fp32.
 * ra_merge_partials over all P*parts_per_shard parts gives the attention of
 * the queries over all len keys.  Requirements as ra_attn_partial, plus
 * len >= 1, block >= 1, the shards' lengths <= cap.
 */
int ra_attn_partial_rr(const void* Q, const void* K_cache, const void* V_cache, float* O_parts,
                       float* lse_parts, int B, int Hq, int Hkv, int64_t Sq, int64_t cap,
                       int64_t len, int64_t block, int P, int parts_per_shard, int d, int dtype,
                       void* stream);

/*
 * ra_layout_gather -- move a sequence tensor between natural order and
 * sharded order ([L8] section 4B and exercise: the zig-zag chunk maps; the
 * striped token map).
 *   src, dst  [outer, S, inner_bytes] viewed as bytes; must not overlap.
 *   inverse = 0: natural -> sharded; inverse = 1: sharded -> natural.
 *   layout RA_LAYOUT_CONTIGUOUS is the identity (a copy).
 * Use outer = B and inner_bytes = H*d*elem for Q/K/V/O, and outer = B*Hq,
 * inner_bytes = 4 for an LSE array [B, Hq, S].
 * Requirements: the split requirements of ra_fwd_rank (S < 2^31 for the
 * striped split), inner_bytes >= 1.
 */
int ra_layout_gather(const void* src, void* dst, int64_t outer, int64_t S,
                     int64_t inner_bytes, int P, int layout, int inverse, void* stream);

/*
 * ra_head_a2a -- the all-to-all of DeepSpeed Ulysses ([L8] section 5): the
 * sequence-sharded tensors are transposed so that rank g holds head group g
 * (H/P heads) of every token; attention then runs per rank over the whole
 * sequence, and the same exchange brings the output back.  On one GPU the
 * P ranks' buffers are one tensor, so the exchange is a transposition:
 *   inverse = 0: src [B, S, P, run] -> dst [P, B, S, run]
 *   inverse = 1: src [P, B, S, run] -> dst [B, S, P, run]
 * where run = run_bytes is one head group of one token (H/P * d * elem for
 * Q/K/V/O).  For an LSE stored [P, B, H/P, S] use S = 1 and run =
 * H/P * S * 4 to reach [B, H, S].  The heads must divide by P (the caller
 * forms run_bytes).  run_bytes a multiple of 16, pointers 16-byte aligned,
 * src and dst must not overlap.
 */
int ra_head_a2a(const void* src, void* dst, int64_t B, int64_t S, int P, int64_t run_bytes,
                int inverse, void* stream);

/* Message describing the calling thread's last non-OK status ("" if none). */
const char* ra_last_error(void);

/* Library version string. */
const char* ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
