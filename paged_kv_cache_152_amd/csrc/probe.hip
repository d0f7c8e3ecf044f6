// Streaming read probe: the HBM read rate that 16-byte loads reach, with and
// without the nontemporal hint.  The decode kernels read each cached byte once
// per call, so this is the ceiling their loads face (short of the 8 TB/s peak).
#include "internal.h"

namespace pkv {
namespace {

// Read-only streaming probe: each workgroup takes 16 KiB runs of the buffer
// (four 4 KiB loads per iteration, every wave instruction over 1 KiB of whole
// lines), with or without the nontemporal hint, and XOR-folds the 32-bit words
// it read.  Each wave folds its lanes and XORs one word into *sink, so the
// launch leaves *sink XORed with the XOR of every word of the buffer.
template <bool NT>
__global__ __launch_bounds__(256) void pkv_read_kernel(const uint4* __restrict__ src, int64_t n,
                                                       uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t step = (int64_t)gridDim.x * 1024;
    for (int64_t base = (int64_t)blockIdx.x * 1024; base < n; base += step) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            if (i < n) {
                if constexpr (NT) {
                    typedef uint32_t v4 __attribute__((ext_vector_type(4)));
                    v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4*>(src + i)));
                } else {
                    v[u] = src[i];
                }
            } else {
                v[u] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, 64);
    if ((threadIdx.x & 63) == 0 && acc != 0) atomicXor(sink, acc);
}

// Gathered read: the list's chunk i is chunk order[i] of the buffer, each chunk
// 2^log_rows rows of 4 KiB (256 lanes x 16 bytes), read in list order, eight
// rows per workgroup step (on random 4 KiB chunks eight in flight read faster
// than four; in address order four are best).  Entries outside
// [0, src_chunks) are skipped.  The paged decode kernels read their tiles this
// way, through the block table.
template <bool NT>
__global__ __launch_bounds__(256) void pkv_gather_read_kernel(const uint4* __restrict__ src, int64_t src_chunks,
                                                              const int32_t* __restrict__ order, int64_t n_order,
                                                              int log_rows, uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t n_rows = n_order << log_rows;
    const int64_t row_mask = ((int64_t)1 << log_rows) - 1;
    const int64_t step = (int64_t)gridDim.x * 8;
    // lanes 0-7 of each wave hold the eight list entries of a step, loaded one
    // step ahead and read back with readlane; a row past the list or an entry
    // outside the buffer reads row 0 of chunk 0 (src_chunks >= 1) and its
    // words are masked out
    const int lane = threadIdx.x & 63;
    auto entries = [&](int64_t b) -> int32_t {
        return lane < 8 && b < n_rows ? order[min(b + lane, n_rows - 1) >> log_rows] : 0;
    };
    int32_t mine = entries((int64_t)blockIdx.x * 8);
    for (int64_t base = (int64_t)blockIdx.x * 8; base < n_rows; base += step) {
        int64_t cc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) cc[u] = __builtin_amdgcn_readlane(mine, u);
        uint4 v[8];
        uint32_t keep[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t r = base + u;
            const bool ok = r < n_rows && cc[u] >= 0 && cc[u] < src_chunks;
            keep[u] = ok ? ~0u : 0u;
            const int64_t row = ok ? (cc[u] << log_rows) + (r & row_mask) : 0;
            const uint4* p = src + (row << 8) + threadIdx.x;
            if constexpr (NT) {
                typedef uint32_t v4 __attribute__((ext_vector_type(4)));
                v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4*>(p)));
            } else {
                v[u] = *p;
            }
        }
        mine = entries(base + step);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= (v[u].x ^ v[u].y ^ v[u].z ^ v[u].w) & keep[u];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, 64);
    if ((threadIdx.x & 63) == 0 && acc != 0) atomicXor(sink, acc);
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, bool nontemporal, uint32_t* sink, hipStream_t stream) {
    int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 1023) / 1024;
    // two workgroups per CU: on random data a sweep of 2, 4, 8 and 16 per CU
    // read fastest at two (fewer streams open at once)
    if (blocks > 256 * 2) blocks = 256 * 2;
    const uint4* s = reinterpret_cast<const uint4*>(src);
    void* args[] = {&s, &n, &sink};
    const void* k = nontemporal ? reinterpret_cast<const void*>(pkv_read_kernel<true>)
                                : reinterpret_cast<const void*>(pkv_read_kernel<false>);
    return launch_kernel(k, dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

hipError_t launch_gather_read_probe(const void* src, size_t bytes, bool nontemporal, const int32_t* order,
                                    int64_t n_order, int log_rows, uint32_t* sink, hipStream_t stream) {
    const int64_t n_rows = n_order << log_rows;
    if (n_rows == 0) return hipSuccess;
    int64_t blocks = (n_rows + 7) / 8;
    if (blocks > 256 * 2) blocks = 256 * 2;            // as the streaming read
    const uint4* s = reinterpret_cast<const uint4*>(src);
    int64_t src_chunks = (int64_t)(bytes >> (12 + log_rows));
    if (src_chunks == 0) return hipSuccess;            // every entry is outside the buffer
    void* args[] = {&s, &src_chunks, &order, &n_order, &log_rows, &sink};
    const void* k = nontemporal ? reinterpret_cast<const void*>(pkv_gather_read_kernel<true>)
                                : reinterpret_cast<const void*>(pkv_gather_read_kernel<false>);
    return launch_kernel(k, dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

}  // namespace pkv
