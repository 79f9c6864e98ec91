// kvcache.hip -- round-robin append of new tokens' K/V to the shard caches of
// a KV-parallel group (the Helix article: the first block of new tokens goes
// to device 0, the next to device 1, and so on, so every device's cache grows
// evenly).  Token x of the sequence is in block j = x / block, stored by
// shard j mod P at local row (j / P) * block + x mod block.
//
// Pure data movement: one wave per new (batch entry, token) row; its lanes
// copy the row's 16-byte units.  Both caches are laid out
// [P, B, cap, row] so each shard's cache is one contiguous region, as it
// would be on its own device.
#include "ra_device.h"

namespace ra {
namespace {

struct AppendArgs {
    uint8_t* Kc;
    uint8_t* Vc;
    const uint8_t* Kn;
    const uint8_t* Vn;
    int64_t row_bytes, cap, len, n_new, block;
    int B, P;
};

__global__ __launch_bounds__(256) void kv_append_rr_kernel(AppendArgs a) {
    const int64_t id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // b * n_new + i, one wave each
    if (id >= (int64_t)a.B * a.n_new) return;
    const int lane = threadIdx.x & 63;
    const int64_t b = id / a.n_new, i = id - b * a.n_new;
    const int64_t x = a.len + i;    // sequence position of the new token
    const int64_t j = x / a.block;
    const int64_t shard = j % a.P;
    const int64_t row = (j / a.P) * a.block + (x - j * a.block);
    const int64_t dst = ((shard * a.B + b) * a.cap + row) * a.row_bytes;
    const int64_t src = id * a.row_bytes;
    const int units = (int)(a.row_bytes >> 4);
    for (int u = lane; u < units; u += 64) {
        ((uint4*)(a.Kc + dst))[u] = load_once16((const uint4*)(a.Kn + src) + u);
        ((uint4*)(a.Vc + dst))[u] = load_once16((const uint4*)(a.Vn + src) + u);
    }
}

}  // namespace

hipError_t launch_kv_append_rr(void* K_cache, void* V_cache, const void* K_new, const void* V_new,
                              int B, int64_t row_bytes, int P, int64_t cap, int64_t len,
                              int64_t n_new, int64_t block, hipStream_t s) {
    AppendArgs a;
    a.Kc = (uint8_t*)K_cache;
    a.Vc = (uint8_t*)V_cache;
    a.Kn = (const uint8_t*)K_new;
    a.Vn = (const uint8_t*)V_new;
    a.row_bytes = row_bytes;
    a.cap = cap;
    a.len = len;
    a.n_new = n_new;
    a.block = block;
    a.B = B;
    a.P = P;
    const int64_t grid = ((int64_t)B * n_new + 3) / 4;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(kv_append_rr_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ra
