// layout.hip -- natural <-> rank-sharded sequence order.
//
// Lesson 8 "Context Parallelism (CP)", section 4B: with 2P chunks of S/(2P)
// tokens, rank r holds chunks r and 2P-1-r (in that local order, as the
// exercise's answer lists them).  Sharded row k = r*(S/P) + lc*c + u holds
// natural position chunk(r, lc)*c + u with chunk(r, 0) = r and
// chunk(r, 1) = 2P-1-r.  The contiguous split is the identity.
//
// Pure data movement.  Both splits move whole chunks of c rows, so the fast
// kernel gives each work-group a contiguous byte range inside one chunk and
// computes the source and destination chunk bases once (scalar arithmetic);
// the threads then stream 16-byte units.  The general kernel (any alignment)
// copies 16-, 4- or 1-byte units and maps every destination row to its source.
#include "ra_device.h"

namespace ra {
namespace {

struct LayoutArgs {
    const uint8_t* src;
    uint8_t* dst;
    int64_t outer, S, row_bytes;
    int64_t n, c;  // tokens per shard, tokens per chunk
    int P, zigzag, inverse;
};

__device__ __forceinline__ int64_t src_row(const LayoutArgs& a, int64_t k) {
    if (!a.zigzag) return k;
    if (!a.inverse) {  // dst sharded row k <- src natural position
        const int64_t r = k / a.n, local = k % a.n;
        const int64_t lc = local / a.c, u = local % a.c;
        const int64_t ch = lc == 0 ? r : 2 * a.P - 1 - r;
        return ch * a.c + u;
    }
    // dst natural position k <- src sharded row
    const int64_t ch = k / a.c, u = k % a.c;
    const int64_t r = ch < a.P ? ch : 2 * a.P - 1 - ch;
    const int64_t lc = ch < a.P ? 0 : 1;
    return r * a.n + lc * a.c + u;
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
    int nchunks, wgs_per_chunk, P, zigzag, inverse;
};

__global__ __launch_bounds__(256) void layout_chunks_kernel(ChunkArgs a) {
    const int part = (int)(blockIdx.x % (unsigned)a.wgs_per_chunk);
    const unsigned rest = blockIdx.x / (unsigned)a.wgs_per_chunk;
    const int q = (int)(rest % (unsigned)a.nchunks);
    const int64_t o = rest / (unsigned)a.nchunks;
    int sq = q;  // source chunk index
    if (a.zigzag) {
        if (!a.inverse) {
            // destination sharded position q = 2r + lc holds natural chunk r or 2P-1-r
            const int r = q >> 1, lc = q & 1;
            sq = lc == 0 ? r : 2 * a.P - 1 - r;
        } else {
            // destination natural chunk q comes from sharded position 2r + lc
            const int r = q < a.P ? q : 2 * a.P - 1 - q;
            sq = 2 * r + (q < a.P ? 0 : 1);
        }
    }
    const int64_t beg = (int64_t)part * BYTES_PER_WG;
    int64_t len = a.chunk_bytes - beg;
    if (len > BYTES_PER_WG) len = BYTES_PER_WG;
    const uint4* s = (const uint4*)(a.src + o * a.seq_bytes + sq * a.chunk_bytes + beg);
    uint4* d = (uint4*)(a.dst + o * a.seq_bytes + (int64_t)q * a.chunk_bytes + beg);
    const int units = (int)(len >> 4);
#pragma unroll 4
    for (int i = threadIdx.x; i < units; i += 256) d[i] = s[i];
}

}  // namespace

hipError_t launch_layout(const void* src, void* dst, int64_t outer, int64_t S, int64_t inner_bytes,
                         int P, int zigzag, int inverse, hipStream_t s) {
    LayoutArgs a;
    a.src = (const uint8_t*)src;
    a.dst = (uint8_t*)dst;
    a.outer = outer;
    a.S = S;
    a.row_bytes = inner_bytes;
    a.P = P;
    a.zigzag = zigzag;
    a.inverse = inverse;
    a.n = S / P;
    a.c = zigzag ? S / (2 * P) : a.n;
    const int64_t total_bytes = outer * S * inner_bytes;
    if (total_bytes <= 0) return hipSuccess;
    const uintptr_t align = (uintptr_t)src | (uintptr_t)dst;
    {
        ChunkArgs c;
        c.chunk_bytes = a.c * inner_bytes;
        c.seq_bytes = S * inner_bytes;
        c.nchunks = zigzag ? 2 * P : P;
        const int64_t wpc = (c.chunk_bytes + BYTES_PER_WG - 1) / BYTES_PER_WG;
        const int64_t grid = outer * c.nchunks * wpc;
        if (align % 16 == 0 && c.chunk_bytes % 16 == 0 && grid <= 0x7fffffffLL) {
            c.src = (const uint8_t*)src;
            c.dst = (uint8_t*)dst;
            c.wgs_per_chunk = (int)wpc;
            c.P = P;
            c.zigzag = zigzag;
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
