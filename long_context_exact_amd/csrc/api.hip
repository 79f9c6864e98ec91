// api.hip -- the extern "C" entry points of libra.so (declared in ra.h):
// argument validation, launch planning and kernel dispatch.  Validation
// happens before any HIP call, so bad arguments are reported without a device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/ra.h"
#include "ra_device.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return RA_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Layout code -> chunks per rank k and the striped flag; checks that S splits.
struct Split {
    int k;        // chunks per rank (1 for the contiguous and the striped split)
    int striped;  // 1: token round-robin
};

int check_split(int layout, int64_t S, int P, Split& sp) {
    sp.k = 1;
    sp.striped = 0;
    if (layout == RA_LAYOUT_CONTIGUOUS) {
    } else if (layout == RA_LAYOUT_ZIGZAG) {
        sp.k = 2;
    } else if (layout == RA_LAYOUT_STRIPED) {
        sp.striped = 1;
    } else if ((layout & ~0xff) == 0x100 && (layout & 0xff) >= 1 &&
               (layout & 0xff) <= RA_MAX_CHUNKS_PER_RANK) {
        sp.k = layout & 0xff;
    } else {
        return fail(RA_ERR_INVALID_ARG, "unknown layout %d", layout);
    }
    if (P > 4096) return fail(RA_ERR_UNSUPPORTED, "P=%d exceeds 4096", P);
    const int64_t parts = (int64_t)sp.k * P;
    if (S % parts != 0)
        return fail(RA_ERR_UNSUPPORTED, "S=%lld does not split into %lld equal chunks", (long long)S,
                    (long long)parts);
    return RA_OK;
}

// Checks shared by ra_fwd_rank and ra_fwd_all.
int check_fwd(const void* Q, const void* K, const void* V, const void* O, const float* LSE, int B,
              int Hq, int Hkv, int64_t S, int d, int P, int causal, int layout, int dtype,
              int o_dtype) {
    if (!Q || !K || !V || !O || !LSE) return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || P <= 0)
        return fail(RA_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d S=%lld P=%d)", B,
                    Hq, Hkv, (long long)S, P);
    if (causal != 0 && causal != 1) return fail(RA_ERR_INVALID_ARG, "causal must be 0 or 1");
    Split sp;
    const int rc = check_split(layout, S, P, sp);
    if (rc != RA_OK) return rc;
    if (dtype != RA_DTYPE_F32 && dtype != RA_DTYPE_BF16)
        return fail(RA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (o_dtype != RA_DTYPE_F32 && o_dtype != RA_DTYPE_BF16)
        return fail(RA_ERR_INVALID_ARG, "unknown output dtype %d", o_dtype);
    if (dtype == RA_DTYPE_F32 && o_dtype != RA_DTYPE_F32)
        return fail(RA_ERR_UNSUPPORTED, "fp32 inputs need an fp32 output");
    if (d != 64 && d != 128) return fail(RA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
    if (Hq % Hkv != 0) return fail(RA_ERR_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (dtype == RA_DTYPE_BF16 && S >= (int64_t(1) << 30))
        return fail(RA_ERR_UNSUPPORTED, "S=%lld: the bf16 kernel keeps positions in 31 bits",
                    (long long)S);
    return RA_OK;
}

ra::FwdParams plan_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                       int Hq, int Hkv, int64_t S, int d, int P, int causal, int layout, int dtype,
                       int o_dtype, int rank_lo, int n_ranks, int q_local) {
    ra::FwdParams p;
    p.Q = Q;
    p.K = K;
    p.V = V;
    p.O = O;
    p.LSE = LSE;
    p.S = S;
    Split sp;
    check_split(layout, S, P, sp);  // validated by check_fwd
    p.n = S / P;
    p.striped = sp.striped;
    p.chunks_per_rank = sp.k;
    p.c = p.n / sp.k;
    p.q_rows = q_local ? p.n : S;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.P = P;
    p.causal = causal;
    p.o_f32 = o_dtype == RA_DTYPE_F32;
    p.rank_lo = rank_lo;
    p.n_ranks = n_ranks;
    p.q_local = q_local;
    const int bm = dtype == RA_DTYPE_BF16 ? ra::FWD_BF16_BLOCK_M : ra::FWD_F32_BLOCK_M;
    p.tiles_per_chunk = (int)((p.c + bm - 1) / bm);
    const int pairs = B * Hkv;
    p.xcd_pairs = (pairs % 8 == 0) ? pairs / 8 : 0;
    p.kv_splits = 1;
    p.o_split_stride = 0;
    p.l_split_stride = 0;
    p.step_lo = 0;
    p.step_hi = P;
    p.kv_block = 0;
    p.kv_rows = S;
    p.fold = 0;
    p.scale = (float)(1.0 / sqrt((double)d));
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    return p;
}

int launch_fwd(const ra::FwdParams& p, int d, int dtype, void* stream) {
    const int64_t tiles = (int64_t)p.n_ranks * p.chunks_per_rank * p.tiles_per_chunk;
    const int64_t grid = tiles * p.B * p.Hq * p.kv_splits;
    if (grid > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "grid of %lld work-groups", (long long)grid);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = dtype == RA_DTYPE_BF16 ? ra::launch_fwd_bf16(p, d, s) : ra::launch_fwd_f32(p, d, s);
    return hip_status(e, "attention kernel launch");
}

// ---- key-range splits -------------------------------------------------------
//
// A launch with fewer query tiles than a few per compute unit leaves CUs idle,
// and under the causal mask its heaviest tile alone sets the time.  Splitting
// every tile's visiting order of key tiles into contiguous ranges, one
// work-group each, and merging the (O, lse) partials with the merge kernel
// (the section 3 fold over the ranges) evens this out.
// Measured on the 8k and 32k-token causal workloads: about two work-groups
// per CU is best; beyond that the fp32 partials cost more traffic than the
// balance gains (8 ranges beat 16 on a 32-tile rank share).
constexpr int kComputeUnits = 256;  // MI355X
constexpr int kAutoMaxSplits = 8;
// One ring step covers one block of S/P keys.  On the 8k-token workload
// (1024-key blocks) eight automatic ranges made the steps 28% slower; on the
// 32k one (4096-key blocks) two ranges made them 9% faster.
constexpr int64_t kAutoMinRangeKeys = 1024;

int64_t fwd_units(const ra::FwdParams& p) {
    return (int64_t)p.n_ranks * p.chunks_per_rank * p.tiles_per_chunk * p.B * p.Hq;
}

// splits the automatic choice asks for: about two work-groups per CU
int auto_splits(const ra::FwdParams& p) {
    const int64_t units = fwd_units(p);
    if (units <= 0 || units >= 4 * kComputeUnits) return 1;
    const int64_t s = (2 * kComputeUnits + units - 1) / units;
    return (int)(s < kAutoMaxSplits ? s : kAutoMaxSplits);
}

// workspace for `splits` partials: fp32 O [splits, rows, d] then LSE [splits, rows]
int64_t split_bytes(const ra::FwdParams& p, int d, int splits) {
    if (splits <= 1) return 0;
    const int64_t rows = (int64_t)p.B * p.q_rows * p.Hq;
    return (int64_t)splits * rows * (d + 1) * (int64_t)sizeof(float);
}

int fwd_split(ra::FwdParams p, int d, int dtype, int o_dtype, int kv_splits, void* ws,
              int64_t ws_bytes, void* stream, int max_auto = kAutoMaxSplits) {
    if (kv_splits < 0 || kv_splits > RA_MAX_KV_SPLITS)
        return fail(RA_ERR_INVALID_ARG, "kv_splits=%d outside [0, %d]", kv_splits, RA_MAX_KV_SPLITS);
    if (ws_bytes < 0) return fail(RA_ERR_INVALID_ARG, "negative workspace size");
    if (ws == nullptr) ws_bytes = 0;
    int splits = kv_splits;
    if (splits == 0) {
        splits = auto_splits(p);
        if (splits > max_auto) splits = max_auto;
        while (splits > 1 && split_bytes(p, d, splits) > ws_bytes) --splits;
    } else if (split_bytes(p, d, splits) > ws_bytes) {
        return fail(RA_ERR_INVALID_ARG, "workspace of %lld bytes, %d splits need %lld",
                    (long long)ws_bytes, splits, (long long)split_bytes(p, d, splits));
    }
    if (splits == 1) return launch_fwd(p, d, dtype, stream);
    if ((uintptr_t)ws % 16 != 0) return fail(RA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    // a ring step past the first folds its ranges and the running state in
    // one merge (the state as its first part, written back in place)
    const int fold = p.fold;
    p.fold = 0;
    const int64_t rows = (int64_t)p.B * p.q_rows * p.Hq;
    if ((rows + 3) / 4 > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "too many rows");
    float* o_parts = (float*)ws;
    float* l_parts = o_parts + (int64_t)splits * rows * d;
    void* O = p.O;
    float* LSE = p.LSE;
    p.O = o_parts;
    p.LSE = l_parts;
    p.o_f32 = 1;
    p.kv_splits = splits;
    p.o_split_stride = rows * d;
    p.l_split_stride = rows;
    // the bf16 kernel keeps a tile's ranges on the tile's XCD; the fp32 one
    // keeps them adjacent in dispatch order, without XCD grouping
    if (dtype != RA_DTYPE_BF16) p.xcd_pairs = 0;
    const int rc = launch_fwd(p, d, dtype, stream);
    if (rc != RA_OK) return rc;
    ra::MergeParams m;
    m.O_parts = o_parts;
    m.lse_parts = l_parts;
    m.O = O;
    m.lse = LSE;
    m.rows = rows;
    m.n_parts = splits;
    m.out_bf16 = o_dtype == RA_DTYPE_BF16;
    m.lse_bhq = 1;
    m.q_rows = p.q_rows;
    m.Hq = p.Hq;
    m.O_state = fold ? (const float*)O : nullptr;
    m.lse_state = fold ? LSE : nullptr;
    return hip_status(ra::launch_merge(m, d, (hipStream_t)stream), "merge kernel launch");
}

// ---- library-owned scratch (ra_fwd_rank_noalloc) ---------------------------
//
// Device memory for the key-range partials of ra_fwd_rank_noalloc, for callers
// that cannot allocate.  Each GPU the library runs on holds its own copy of
// the array until the process ends.  In host code the array's name is only a
// stand-in for the symbol: kernels and copies use the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in scratch_dev.
static __device__ __align__(256) unsigned char scratch[RA_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxScratchDevices] = {};

// Address of the current device's scratch (set up on the first call there).
int scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(RA_ERR_UNSUPPORTED, "device %d: scratch is kept for devices 0..%d", dev,
                    kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (p == nullptr) return fail(RA_ERR_HIP, "hipGetSymbolAddress(scratch) returned no address");
        scratch_dev[dev] = p;
    }
    *out = scratch_dev[dev];
    return RA_OK;
}

}  // namespace

extern "C" {

int ra_fwd_rank(const void* Q_r, const void* K, const void* V, void* O_r, float* LSE_r, int B,
                int Hq, int Hkv, int64_t S, int d, int P, int rank, int causal, int layout, int dtype,
                int o_dtype, void* stream) {
    int rc = check_fwd(Q_r, K, V, O_r, LSE_r, B, Hq, Hkv, S, d, P, causal, layout, dtype, o_dtype);
    if (rc != RA_OK) return rc;
    if (rank < 0 || rank >= P) return fail(RA_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, P);
    ra::FwdParams p = plan_fwd(Q_r, K, V, O_r, LSE_r, B, Hq, Hkv, S, d, P, causal, layout, dtype,
                               o_dtype, rank, 1, 1);
    return launch_fwd(p, d, dtype, stream);
}

int ra_fwd_all(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq,
               int Hkv, int64_t S, int d, int P, int causal, int layout, int dtype, int o_dtype,
               void* stream) {
    int rc = check_fwd(Q, K, V, O, LSE, B, Hq, Hkv, S, d, P, causal, layout, dtype, o_dtype);
    if (rc != RA_OK) return rc;
    ra::FwdParams p = plan_fwd(Q, K, V, O, LSE, B, Hq, Hkv, S, d, P, causal, layout, dtype, o_dtype,
                               0, P, 0);
    return launch_fwd(p, d, dtype, stream);
}

int ra_fwd_rank_ws(const void* Q_r, const void* K, const void* V, void* O_r, float* LSE_r, int B,
                   int Hq, int Hkv, int64_t S, int d, int P, int rank, int causal, int layout,
                   int dtype, int o_dtype, int kv_splits, void* workspace, int64_t workspace_bytes,
                   void* stream) {
    int rc = check_fwd(Q_r, K, V, O_r, LSE_r, B, Hq, Hkv, S, d, P, causal, layout, dtype, o_dtype);
    if (rc != RA_OK) return rc;
    if (rank < 0 || rank >= P) return fail(RA_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, P);
    ra::FwdParams p = plan_fwd(Q_r, K, V, O_r, LSE_r, B, Hq, Hkv, S, d, P, causal, layout, dtype,
                               o_dtype, rank, 1, 1);
    return fwd_split(p, d, dtype, o_dtype, kv_splits, workspace, workspace_bytes, stream);
}

int ra_fwd_rank_noalloc(const void* Q_r, const void* K, const void* V, void* O_r, float* LSE_r, int B,
                        int Hq, int Hkv, int64_t S, int d, int P, int rank, int causal, int layout,
                        int dtype, int o_dtype, int kv_splits, void* stream) {
    int rc = check_fwd(Q_r, K, V, O_r, LSE_r, B, Hq, Hkv, S, d, P, causal, layout, dtype, o_dtype);
    if (rc != RA_OK) return rc;
    if (rank < 0 || rank >= P) return fail(RA_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, P);
    if (kv_splits < 0 || kv_splits > RA_MAX_KV_SPLITS)
        return fail(RA_ERR_INVALID_ARG, "kv_splits=%d outside [0, %d]", kv_splits, RA_MAX_KV_SPLITS);
    ra::FwdParams p = plan_fwd(Q_r, K, V, O_r, LSE_r, B, Hq, Hkv, S, d, P, causal, layout, dtype,
                               o_dtype, rank, 1, 1);
    const int64_t need = split_bytes(p, d, kv_splits);
    if (kv_splits > 1 && need > RA_SCRATCH_BYTES)
        return fail(RA_ERR_INVALID_ARG,
                    "kv_splits=%d needs %lld bytes of partials; the library's scratch holds %lld",
                    kv_splits, (long long)need, (long long)RA_SCRATCH_BYTES);
    void* ws = nullptr;
    rc = scratch_ptr(&ws);
    if (rc != RA_OK) return rc;
    return fwd_split(p, d, dtype, o_dtype, kv_splits, ws, RA_SCRATCH_BYTES, stream);
}

int ra_fwd_all_ws(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq,
                  int Hkv, int64_t S, int d, int P, int causal, int layout, int dtype, int o_dtype,
                  int kv_splits, void* workspace, int64_t workspace_bytes, void* stream) {
    int rc = check_fwd(Q, K, V, O, LSE, B, Hq, Hkv, S, d, P, causal, layout, dtype, o_dtype);
    if (rc != RA_OK) return rc;
    ra::FwdParams p = plan_fwd(Q, K, V, O, LSE, B, Hq, Hkv, S, d, P, causal, layout, dtype, o_dtype,
                               0, P, 0);
    return fwd_split(p, d, dtype, o_dtype, kv_splits, workspace, workspace_bytes, stream);
}

int ra_ring_step(const void* Q_r, const void* K_blk, const void* V_blk, float* O_acc, float* LSE_acc,
                 int B, int Hq, int Hkv, int64_t S, int d, int P, int rank, int t, int causal,
                 int layout, int dtype, void* stream) {
    return ra_ring_step_ws(Q_r, K_blk, V_blk, O_acc, LSE_acc, B, Hq, Hkv, S, d, P, rank, t, causal, layout,
                           dtype, 1, nullptr, 0, stream);
}

int ra_ring_step_ws(const void* Q_r, const void* K_blk, const void* V_blk, float* O_acc, float* LSE_acc,
                    int B, int Hq, int Hkv, int64_t S, int d, int P, int rank, int t, int causal,
                    int layout, int dtype, int kv_splits, void* workspace, int64_t workspace_bytes,
                    void* stream) {
    int rc = check_fwd(Q_r, K_blk, V_blk, O_acc, LSE_acc, B, Hq, Hkv, S, d, P, causal, layout, dtype,
                       RA_DTYPE_F32);
    if (rc != RA_OK) return rc;
    if (rank < 0 || rank >= P) return fail(RA_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, P);
    if (t < 0 || t >= P) return fail(RA_ERR_INVALID_ARG, "step %d outside [0, %d)", t, P);
    ra::FwdParams p = plan_fwd(Q_r, K_blk, V_blk, O_acc, LSE_acc, B, Hq, Hkv, S, d, P, causal, layout,
                               dtype, RA_DTYPE_F32, rank, 1, 1);
    p.step_lo = t;
    p.step_hi = t + 1;
    p.kv_block = 1;
    p.kv_rows = p.n;
    p.fold = t > 0;
    // automatic ranges of at least 1024 keys of the block: below that the
    // partials and the merge cost more than the balance gains
    const int64_t max_auto = p.n / kAutoMinRangeKeys;
    return fwd_split(p, d, dtype, RA_DTYPE_F32, kv_splits, workspace, workspace_bytes, stream,
                     (int)(max_auto < 1 ? 1 : max_auto < kAutoMaxSplits ? max_auto : kAutoMaxSplits));
}

int64_t ra_fwd_workspace_bytes(int B, int Hq, int Hkv, int64_t S, int d, int P, int all_ranks,
                               int causal, int layout, int dtype, int kv_splits) {
    static const char kDummy = 0;
    const void* x = &kDummy;  // shape checks only: no tensor is touched
    int rc = check_fwd(x, x, x, (void*)x, (float*)x, B, Hq, Hkv, S, d, P, causal, layout, dtype,
                       dtype);
    if (rc != RA_OK) return rc;
    if (all_ranks != 0 && all_ranks != 1) return fail(RA_ERR_INVALID_ARG, "all_ranks must be 0 or 1");
    if (kv_splits < 0 || kv_splits > RA_MAX_KV_SPLITS)
        return fail(RA_ERR_INVALID_ARG, "kv_splits=%d outside [0, %d]", kv_splits, RA_MAX_KV_SPLITS);
    ra::FwdParams p = plan_fwd(x, x, x, (void*)x, (float*)x, B, Hq, Hkv, S, d, P, causal, layout,
                               dtype, dtype, 0, all_ranks ? P : 1, all_ranks ? 0 : 1);
    ok();
    return split_bytes(p, d, kv_splits == 0 ? auto_splits(p) : kv_splits);
}

int ra_merge_partials(const float* O_parts, const float* lse_parts, void* O, float* lse,
                      int n_parts, int64_t rows, int d, int out_dtype, void* stream) {
    if (!O_parts || !lse_parts || !O) return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
    if (n_parts <= 0 || rows <= 0)
        return fail(RA_ERR_INVALID_ARG, "n_parts=%d rows=%lld must be positive", n_parts,
                    (long long)rows);
    if (out_dtype != RA_DTYPE_F32 && out_dtype != RA_DTYPE_BF16)
        return fail(RA_ERR_INVALID_ARG, "unknown dtype %d", out_dtype);
    if (d != 64 && d != 128) return fail(RA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
    if ((rows + 3) / 4 > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "too many rows");
    ra::MergeParams p;
    p.O_parts = O_parts;
    p.lse_parts = lse_parts;
    p.O = O;
    p.lse = lse;
    p.rows = rows;
    p.n_parts = n_parts;
    p.out_bf16 = out_dtype == RA_DTYPE_BF16;
    p.lse_bhq = 0;
    p.q_rows = 0;
    p.Hq = 1;
    p.O_state = nullptr;
    p.lse_state = nullptr;
    return hip_status(ra::launch_merge(p, d, (hipStream_t)stream), "merge kernel launch");
}

int ra_attn_partial(const void* Q, const void* K, const void* V, float* O_parts, float* lse_parts,
                    int B, int Hq, int Hkv, int64_t Sq, int64_t Skv, int d, int n_parts, int dtype,
                    void* stream) {
    if (!Q || !K || !V || !O_parts || !lse_parts) return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || n_parts <= 0)
        return fail(RA_ERR_INVALID_ARG, "sizes must be positive");
    if (dtype != RA_DTYPE_F32 && dtype != RA_DTYPE_BF16)
        return fail(RA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (d != 64 && d != 128) return fail(RA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
    if (Hq % Hkv != 0) return fail(RA_ERR_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (Sq * (Hq / Hkv) > 32)
        return fail(RA_ERR_UNSUPPORTED, "Sq*(Hq/Hkv)=%lld exceeds 32 query rows per kv head",
                    (long long)(Sq * (Hq / Hkv)));
    const int64_t grid = (int64_t)B * Hkv * n_parts;
    if (grid > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "grid of %lld work-groups", (long long)grid);
    ra::DecodeParams p;
    p.Q = Q;
    p.K = K;
    p.V = V;
    p.O_parts = O_parts;
    p.lse_parts = lse_parts;
    p.Sq = Sq;
    p.Skv = Skv;
    p.kv_cap = Skv;
    p.rr_block = 0;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.n_parts = n_parts;
    p.n_shards = 1;
    p.parts_per_shard = n_parts;
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = dtype == RA_DTYPE_BF16 ? ra::launch_decode_bf16(p, d, s) : ra::launch_decode_f32(p, d, s);
    return hip_status(e, "decode kernel launch");
}

int ra_kv_append_rr(void* K_cache, void* V_cache, const void* K_new, const void* V_new, int B,
                    int Hkv, int d, int P, int64_t cap, int64_t len, int64_t n_new, int64_t block,
                    int dtype, void* stream) {
    if (!K_cache || !V_cache || !K_new || !V_new) return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
    if (B <= 0 || Hkv <= 0 || P <= 0 || cap <= 0 || n_new <= 0 || block <= 0 || len < 0)
        return fail(RA_ERR_INVALID_ARG, "sizes must be positive (len >= 0)");
    if (dtype != RA_DTYPE_F32 && dtype != RA_DTYPE_BF16)
        return fail(RA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (d != 64 && d != 128) return fail(RA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
    if (P > 4096) return fail(RA_ERR_UNSUPPORTED, "P=%d exceeds 4096", P);
    // shard 0 receives the first block of every round, so it is never shorter
    const int64_t need = ra::rr_shard_len(len + n_new, block, P, 0);
    if (need > cap)
        return fail(RA_ERR_INVALID_ARG, "shard 0 would hold %lld rows, capacity %lld", (long long)need,
                    (long long)cap);
    if (((int64_t)B * n_new + 3) / 4 > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "too many new rows");
    if (((uintptr_t)K_cache | (uintptr_t)V_cache | (uintptr_t)K_new | (uintptr_t)V_new) % 16 != 0)
        return fail(RA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    const int64_t row_bytes = (int64_t)Hkv * d * (dtype == RA_DTYPE_BF16 ? 2 : 4);
    return hip_status(ra::launch_kv_append_rr(K_cache, V_cache, K_new, V_new, B, row_bytes, P, cap,
                                              len, n_new, block, (hipStream_t)stream),
                      "append kernel launch");
}

int ra_attn_partial_rr(const void* Q, const void* K_cache, const void* V_cache, float* O_parts,
                       float* lse_parts, int B, int Hq, int Hkv, int64_t Sq, int64_t cap,
                       int64_t len, int64_t block, int P, int parts_per_shard, int d, int dtype,
                       void* stream) {
    if (!Q || !K_cache || !V_cache || !O_parts || !lse_parts)
        return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || cap <= 0 || len <= 0 || block <= 0 || P <= 0 ||
        parts_per_shard <= 0)
        return fail(RA_ERR_INVALID_ARG, "sizes must be positive");
    if (dtype != RA_DTYPE_F32 && dtype != RA_DTYPE_BF16)
        return fail(RA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (d != 64 && d != 128) return fail(RA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
    if (Hq % Hkv != 0) return fail(RA_ERR_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (Sq * (Hq / Hkv) > 32)
        return fail(RA_ERR_UNSUPPORTED, "Sq*(Hq/Hkv)=%lld exceeds 32 query rows per kv head",
                    (long long)(Sq * (Hq / Hkv)));
    if (P > 4096) return fail(RA_ERR_UNSUPPORTED, "P=%d exceeds 4096", P);
    if (ra::rr_shard_len(len, block, P, 0) > cap)
        return fail(RA_ERR_INVALID_ARG, "%lld keys in blocks of %lld exceed shard capacity %lld",
                    (long long)len, (long long)block, (long long)cap);
    const int64_t n_parts = (int64_t)P * parts_per_shard;
    const int64_t grid = (int64_t)B * Hkv * n_parts;
    if (n_parts > 0x7fffffffLL || grid > 0x7fffffffLL)
        return fail(RA_ERR_UNSUPPORTED, "grid of %lld work-groups", (long long)grid);
    ra::DecodeParams p;
    p.Q = Q;
    p.K = K_cache;
    p.V = V_cache;
    p.O_parts = O_parts;
    p.lse_parts = lse_parts;
    p.Sq = Sq;
    p.Skv = len;
    p.kv_cap = cap;
    p.rr_block = block;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.n_parts = (int)n_parts;
    p.n_shards = P;
    p.parts_per_shard = parts_per_shard;
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = dtype == RA_DTYPE_BF16 ? ra::launch_decode_bf16(p, d, s) : ra::launch_decode_f32(p, d, s);
    return hip_status(e, "decode kernel launch");
}

int ra_layout_gather(const void* src, void* dst, int64_t outer, int64_t S, int64_t inner_bytes, int P,
                     int layout, int inverse, void* stream) {
    if (!src || !dst) return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
    if (outer <= 0 || S <= 0 || inner_bytes <= 0 || P <= 0)
        return fail(RA_ERR_INVALID_ARG, "sizes must be positive");
    Split sp;
    const int rc = check_split(layout, S, P, sp);
    if (rc != RA_OK) return rc;
    if (inverse != 0 && inverse != 1) return fail(RA_ERR_INVALID_ARG, "inverse must be 0 or 1");
    if (sp.striped && S >= (int64_t(1) << 31))
        return fail(RA_ERR_UNSUPPORTED, "S=%lld: the striped gather keeps rows in 32 bits",
                    (long long)S);
    const uint8_t* s0 = (const uint8_t*)src;
    const uint8_t* d0 = (const uint8_t*)dst;
    const int64_t bytes = outer * S * inner_bytes;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(RA_ERR_INVALID_ARG, "src and dst overlap");
    return hip_status(ra::launch_layout(src, dst, outer, S, inner_bytes, P, sp.k, sp.striped,
                                        inverse, (hipStream_t)stream),
                      "layout kernel launch");
}

int ra_head_a2a(const void* src, void* dst, int64_t B, int64_t S, int P, int64_t run_bytes,
                int inverse, void* stream) {
    if (!src || !dst) return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
    if (B <= 0 || S <= 0 || P <= 0 || run_bytes <= 0) return fail(RA_ERR_INVALID_ARG, "sizes must be positive");
    if (inverse != 0 && inverse != 1) return fail(RA_ERR_INVALID_ARG, "inverse must be 0 or 1");
    if (run_bytes % 16 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0)
        return fail(RA_ERR_UNSUPPORTED, "runs of %lld bytes: need 16-byte runs and alignment",
                    (long long)run_bytes);
    const int64_t runs = (int64_t)P * B * S;
    if ((runs * ((run_bytes + 4095) / 4096) + 3) / 4 > 0x7fffffffLL)
        return fail(RA_ERR_UNSUPPORTED, "too many runs");
    const uint8_t* s0 = (const uint8_t*)src;
    const uint8_t* d0 = (const uint8_t*)dst;
    const int64_t bytes = runs * run_bytes;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(RA_ERR_INVALID_ARG, "src and dst overlap");
    return hip_status(ra::launch_head_a2a(src, dst, B, S, P, run_bytes, inverse, (hipStream_t)stream),
                      "all-to-all kernel launch");
}

const char* ra_last_error(void) { return g_err; }

const char* ra_version(void) { return "libra 0.1 (gfx950)"; }

}  // extern "C"
