// layout.hip -- natural <-> rank-sharded sequence order.
//
// Lesson 8 "Context Parallelism (CP)", section 4B and the exercise: with k
// chunks of c = S/(kP) tokens per rank, sharded row r*(S/P) + lc*c + u holds
// natural position g(r, lc)*c + u, where g is the zig-zag chunk map (even
// local chunks picked from the front, odd ones from the back; k = 2 gives
// chunks r and 2P-1-r, k = 1 the identity).  Under the striped split
// sharded row r*(S/P) + i holds natural position r + iP.
//
// Pure data movement.  The chunked splits move whole chunks of c rows, so the
// chunk kernel gives each work-group a contiguous byte range inside one chunk
// and computes the source and destination chunk bases once (scalar
// arithmetic); the threads then stream 16-byte units, read with the
// non-temporal hint (each byte is read once; measured on one box: 5.64 TB/s
// for Q, K, V against 5.32 with plain loads and 5.57 with non-temporal loads
// and stores).  The striped split
// moves single rows: the row kernel gives each wave whole rows and maps each
// destination row to its source once.  The general kernel (any alignment)
// copies 16-, 4- or 1-byte units and maps every destination row to its source.
#include "ra_device.h"

namespace ra {
namespace {

struct LayoutArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t outer, S, row_bytes;
    int64_t n, c;  // tokens per shard, tokens per chunk
    int P, k, striped, inverse;
};

// natural chunk of the sharded chunk slot q = rank * k + lc, and back
__device__ __forceinline__ int64_t natural_chunk(int P, int k, int64_t q) {
    return global_chunk(P, k, (int)(q / k), (int)(q % k));
}
__device__ __forceinline__ int64_t sharded_slot(int P, int k, int64_t g) {
    const int band = (int)(g / P);
    const int lc = band_chunk(k, band);
    const int64_t rank = (lc & 1) ? (int64_t)k * P - 1 - (int64_t)(lc >> 1) * P - g : g - (int64_t)band * P;
    return rank * k + lc;
}

__device__ __forceinline__ int64_t src_row(const LayoutArgs& a, int64_t k) {
    if (a.striped) {
        if (!a.inverse) return (k % a.n) * a.P + k / a.n;  // sharded row r*n + i <- r + iP
        return (k % a.P) * a.n + k / a.P;                  // natural r + iP <- sharded r*n + i
    }
    const int64_t q = k / a.c, u = k % a.c;
    if (!a.inverse) return natural_chunk(a.P, a.k, q) * a.c + u;
    return sharded_slot(a.P, a.k, q) * a.c + u;
}

template <typename U>
__global__ __launch_bounds__(256) void layout_kernel(LayoutArgs a) {
    const int64_t units_per_row = a.row_bytes / (int64_t)sizeof(U);
    const int64_t total = a.outer * a.S * units_per_row;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t u = idx % units_per_row;
        const int64_t rowg = idx / units_per_row;
        const int64_t o = rowg / a.S, k = rowg % a.S;
        const int64_t sk = src_row(a, k);
        const U* s = (const U*)(a.src + (o * a.S + sk) * a.row_bytes);
        U* d = (U*)(a.dst + (o * a.S + k) * a.row_bytes);
        d[u] = s[u];
    }
}

// Chunk-level copy: work-group -> (outer index o, destination chunk q, byte
// range of BYTES_PER_WG inside it).  Chunks are c rows of row_bytes.
constexpr int64_t BYTES_PER_WG = 64 * 1024;

struct ChunkArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t chunk_bytes, seq_bytes;  // one chunk; one outer slice (S rows)
    int nchunks, wgs_per_chunk, P, k, inverse;
};

__global__ __launch_bounds__(256) void layout_chunks_kernel(ChunkArgs a) {
    const int part = (int)(blockIdx.x % (unsigned)a.wgs_per_chunk);
    const unsigned rest = blockIdx.x / (unsigned)a.wgs_per_chunk;
    const int q = (int)(rest % (unsigned)a.nchunks);
    const int64_t o = rest / (unsigned)a.nchunks;
    // source chunk: destination slot q holds natural chunk g(q / k, q % k);
    // destination natural chunk q comes from the slot that holds it
    const int64_t sq = a.inverse ? sharded_slot(a.P, a.k, q) : natural_chunk(a.P, a.k, q);
    const int64_t beg = (int64_t)part * BYTES_PER_WG;
    int64_t len = a.chunk_bytes - beg;
    if (len > BYTES_PER_WG) len = BYTES_PER_WG;
    const uint4* s = (const uint4*)(a.src + o * a.seq_bytes + sq * a.chunk_bytes + beg);
    uint4* d = (uint4*)(a.dst + o * a.seq_bytes + (int64_t)q * a.chunk_bytes + beg);
    const int units = (int)(len >> 4);
#pragma unroll 4
    for (int i = threadIdx.x; i < units; i += 256) d[i] = load_once16(s + i);
}

// Striped row copy: work-group -> (outer index o, ROWS consecutive
// destination rows); wave w copies rows w, w+4, ... of them, 16 bytes a lane.
struct RowArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t row_bytes, seq_bytes;
    unsigned S, n, P;
    int rows_per_wg, wgs_per_seq, inverse;
};

__global__ __launch_bounds__(256) void layout_rows_kernel(RowArgs a) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const unsigned blk = blockIdx.x % (unsigned)a.wgs_per_seq;
    const int64_t o = blockIdx.x / (unsigned)a.wgs_per_seq;
    const unsigned k0 = blk * (unsigned)a.rows_per_wg;
    const int units = (int)(a.row_bytes >> 4);
    for (int rr = w; rr < a.rows_per_wg; rr += 4) {
        const unsigned k = k0 + (unsigned)rr;
        if (k >= a.S) break;
        const unsigned sk = a.inverse ? (k % a.P) * a.n + k / a.P : (k % a.n) * a.P + k / a.n;
        const uint4* s = (const uint4*)(a.src + o * a.seq_bytes + (int64_t)sk * a.row_bytes);
        uint4* d = (uint4*)(a.dst + o * a.seq_bytes + (int64_t)k * a.row_bytes);
        for (int i = lane; i < units; i += 64) d[i] = load_once16(s + i);
    }
}

// Head all-to-all of the Ulysses scheme (lesson 8, section 5): every rank
// sends head group g of its sequence shard to rank g.  With the token's heads
// cut into P runs of run_bytes (H/P heads each), forward moves
// [B, S, P, run] (sequence order, all heads) to [P, B, S, run] (head group
// major: each group holds every token), inverse moves it back.  Work items
// are (destination run, 4 KiB segment of it), one wave each, enumerated in
// destination order; lanes move 16 bytes at a time.  Long runs (an LSE row
// of a head group is S * 4 bytes) are thus spread over many waves.
constexpr int64_t A2A_SEG = 4096;

struct A2AArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t B, S, runs, run_bytes, segs;  // runs = P * B * S; segs per run
    int P, inverse;
};

__global__ __launch_bounds__(256) void head_a2a_kernel(A2AArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= a.runs * a.segs) return;
    const int64_t k = item / a.segs, seg = item - k * a.segs;  // destination run, segment
    int64_t srun;
    if (!a.inverse) {  // k = (g * B + b) * S + x  <-  (b * S + x) * P + g
        const int64_t g = k / (a.B * a.S), bx = k - g * a.B * a.S;
        srun = bx * a.P + g;
    } else {           // k = (b * S + x) * P + g  <-  (g * B + b) * S + x
        const int64_t bx = k / a.P, g = k - bx * a.P;
        srun = g * a.B * a.S + bx;
    }
    const int64_t beg = seg * A2A_SEG;
    int64_t len = a.run_bytes - beg;
    if (len > A2A_SEG) len = A2A_SEG;
    const uint4* s = (const uint4*)(a.src + srun * a.run_bytes + beg);
    uint4* d = (uint4*)(a.dst + k * a.run_bytes + beg);
    const int units = (int)(len >> 4);
    for (int u = lane; u < units; u += 64) d[u] = load_once16(s + u);
}

}  // namespace

hipError_t launch_head_a2a(const void* src, void* dst, int64_t B, int64_t S, int P, int64_t run_bytes,
                           int inverse, hipStream_t s) {
    A2AArgs a;
    a.src = (const uint8_t*)src;
    a.dst = (uint8_t*)dst;
    a.B = B;
    a.S = S;
    a.P = P;
    a.runs = (int64_t)P * B * S;
    a.run_bytes = run_bytes;
    a.segs = (run_bytes + A2A_SEG - 1) / A2A_SEG;
    a.inverse = inverse;
    const int64_t grid = (a.runs * a.segs + 3) / 4;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(head_a2a_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_layout(const void* src, void* dst, int64_t outer, int64_t S, int64_t inner_bytes,
                         int P, int chunks_per_rank, int striped, int inverse, hipStream_t s) {
    LayoutArgs a;
    a.src = (const uint8_t*)src;
    a.dst = (uint8_t*)dst;
    a.outer = outer;
    a.S = S;
    a.row_bytes = inner_bytes;
    a.P = P;
    a.k = chunks_per_rank;
    a.striped = striped;
    a.inverse = inverse;
    a.n = S / P;
    a.c = a.n / chunks_per_rank;
    const int64_t total_bytes = outer * S * inner_bytes;
    if (total_bytes <= 0) return hipSuccess;
    const uintptr_t align = (uintptr_t)src | (uintptr_t)dst;
    if (striped) {
        RowArgs r;
        // about 64 KiB per work-group, whole rows, at least one row per wave
        int64_t rows = BYTES_PER_WG / inner_bytes;
        rows = rows < 4 ? 4 : (rows > 256 ? 256 : rows);
        const int64_t wps = (S + rows - 1) / rows;
        const int64_t grid = outer * wps;
        if (align % 16 == 0 && inner_bytes % 16 == 0 && inner_bytes >= 64 && grid <= 0x7fffffffLL) {
            r.src = (const uint8_t*)src;
            r.dst = (uint8_t*)dst;
            r.row_bytes = inner_bytes;
            r.seq_bytes = S * inner_bytes;
            r.S = (unsigned)S;
            r.n = (unsigned)a.n;
            r.P = (unsigned)P;
            r.rows_per_wg = (int)rows;
            r.wgs_per_seq = (int)wps;
            r.inverse = inverse;
            hipLaunchKernelGGL(layout_rows_kernel, dim3((unsigned)grid), dim3(256), 0, s, r);
            return hipGetLastError();
        }
    } else {
        ChunkArgs c;
        c.chunk_bytes = a.c * inner_bytes;
        c.seq_bytes = S * inner_bytes;
        c.nchunks = chunks_per_rank * P;
        const int64_t wpc = (c.chunk_bytes + BYTES_PER_WG - 1) / BYTES_PER_WG;
        const int64_t grid = outer * c.nchunks * wpc;
        if (align % 16 == 0 && c.chunk_bytes % 16 == 0 && grid <= 0x7fffffffLL) {
            c.src = (const uint8_t*)src;
            c.dst = (uint8_t*)dst;
            c.wgs_per_chunk = (int)wpc;
            c.P = P;
            c.k = chunks_per_rank;
            c.inverse = inverse;
            hipLaunchKernelGGL(layout_chunks_kernel, dim3((unsigned)grid), dim3(256), 0, s, c);
            return hipGetLastError();
        }
    }
    int64_t unit = 1;
    if (inner_bytes % 16 == 0 && align % 16 == 0)
        unit = 16;
    else if (inner_bytes % 4 == 0 && align % 4 == 0)
        unit = 4;
    const int64_t units = total_bytes / unit;
    int64_t grid = (units + 255) / 256;
    if (grid > 256 * 64) grid = 256 * 64;
    if (unit == 16)
        hipLaunchKernelGGL(layout_kernel<uint4>, dim3((unsigned)grid), dim3(256), 0, s, a);
    else if (unit == 4)
        hipLaunchKernelGGL(layout_kernel<uint32_t>, dim3((unsigned)grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(layout_kernel<uint8_t>, dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ra
