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

}  // namespace pkv
