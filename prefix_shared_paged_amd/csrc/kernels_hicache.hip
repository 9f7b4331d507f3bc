// kernels_hicache.hip -- row moves between a host-memory KV tier and the pool.
//
// HiCache keeps KV rows that leave the GPU pool in page-locked host memory
// (the second tier) and brings a matched prefix back into pool slots before
// it is attended ("SGLang：从前端 DSL 到 SRT 服务运行时", section "从 2024 年论文到
// 今天的缓存栈", the HiCache bullet).  Both directions are one gather kernel:
// the GPU reads and writes the page-locked host buffer directly over the host
// link, so scattered rows (page size 1) need no staging copy and no DMA
// descriptor per row.
//
// Work item = one 16-byte chunk of one row of one tensor, numbered
// ((i * n_t + t) * cpr + c) for row move i, tensor t (K then V) and chunk c.
// Consecutive lanes take consecutive chunks of a row, so a wave reads and
// writes contiguous runs of up to 1 KiB on both sides.  Each thread keeps kMoveUnroll loads
// in flight before it stores, which is what a read over the host link needs
// to approach its bandwidth.  Rows whose source or destination index lies
// outside its buffer are skipped: no access is ever made outside the
// buffers the caller described.
#include <algorithm>

#include "common.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMoveThreads = 256;
constexpr int kMoveUnroll = 4;
constexpr int kMoveMaxBlocks = 8192;

// DIR 0: host rows -> pool slots (prefetch); DIR 1: pool slots -> host rows (write-back).
template <int DIR>
__global__ void __launch_bounds__(kMoveThreads) move_rows_kernel(const MoveArgs a) {
    const int64_t total = a.n * a.n_t * a.cpr;
    const int64_t per_block = (int64_t)kMoveThreads * kMoveUnroll;
    for (int64_t base = (int64_t)blockIdx.x * per_block + threadIdx.x; base < total;
         base += (int64_t)gridDim.x * per_block) {
        u32x4 v[kMoveUnroll];
        u32x4 *dst[kMoveUnroll];
#pragma unroll
        for (int u = 0; u < kMoveUnroll; ++u) {
            const int64_t e = base + (int64_t)u * kMoveThreads;
            dst[u] = nullptr;
            if (e >= total) continue;
            const int64_t c = e % a.cpr;
            const int64_t it = e / a.cpr;
            const int t = (int)(it % a.n_t);
            const int64_t i = it / a.n_t;
            const int64_t h = a.host_rows[i];
            const int64_t s = a.slots[i];
            if (h < 0 || h >= a.n_host_rows || s < 0 || s >= a.num_slots) continue;
            const int64_t src_row = DIR == 0 ? h : s;
            const int64_t dst_row = DIR == 0 ? s : h;
            const u32x4 *src = reinterpret_cast<const u32x4 *>(a.src[t] + src_row * a.row_bytes) + c;
            v[u] = *src;
            dst[u] = reinterpret_cast<u32x4 *>(a.dst[t] + dst_row * a.row_bytes) + c;
        }
#pragma unroll
        for (int u = 0; u < kMoveUnroll; ++u)
            if (dst[u]) *dst[u] = v[u];
    }
}

}  // namespace

int launch_move_rows(int dir, const MoveArgs &a, hipStream_t st) {
    if (a.n <= 0) return SGL_OK;
    const int64_t items = a.n * a.n_t * a.cpr;
    const int64_t per_block = (int64_t)kMoveThreads * kMoveUnroll;
    const int blocks = (int)std::min<int64_t>((items + per_block - 1) / per_block, kMoveMaxBlocks);
    if (dir == 0)
        hipLaunchKernelGGL(move_rows_kernel<0>, dim3(blocks), dim3(kMoveThreads), 0, st, a);
    else
        hipLaunchKernelGGL(move_rows_kernel<1>, dim3(blocks), dim3(kMoveThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? SGL_OK : SGL_ERR_HIP;
}
