// kv_append: scatter the new tokens' K and V into their pool slots, and the
// plain copy kernel used to calibrate HBM traffic counters.
//
// Only the new token's K/V are computed each decode step and appended to the
// cache (www.cf-1.com/news/5824798 §1.1; www.mlqm.cn/news/394450 section 四);
// with a pre-allocated pool the append is a store at an index
// (www.mooersco.com/news/1484987 §2.2).  Slot s addresses block s / 16,
// row s % 16 of the [num_blocks][H_kv][16][D] pool.
//
// One thread moves one 16-byte chunk of a destination row.  For an FP8 pool
// the source (bf16 or fp32) is multiplied by the per-head inverse scale in
// fp32 and rounded to OCP E4M3 (nearest, ties to even, saturating at 448,
// NaN -> 0x7F), the storage convention of m.lqnn.cn/news/219451 §4.
#include "internal.h"

namespace pkv {
namespace {

// fp32 -> OCP E4M3 ("FN": bias 7, no infinities, S.1111.111 = NaN, max 448),
// round to nearest, ties to even, values beyond 448 saturate.  Branch-free:
// every case is computed and the right one selected.
//  - Normal codes (|x| >= 2^-6): re-bias the fp32 exponent from 127 to 7 in
//    the bit pattern and drop 20 fraction bits, adding 0x7FFFF plus the kept
//    low bit first, which rounds to nearest even (a carry may step into the
//    next binade, as the value does).
//  - Subnormal codes (|x| < 2^-6): the code is k with value k * 2^-9, so
//    k = rint(|x| * 2^9), exact in fp32 since the scaling is by a power of 2;
//    k = 8 is the smallest normal code, which is where such a rounding lands.
__device__ __forceinline__ uint32_t e4m3_from_f32(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    const uint32_t rb = a - (120u << 23);
    const uint32_t nrm = (rb + 0x7FFFFu + ((rb >> 20) & 1u)) >> 20;
    const float small = __uint_as_float(a < (121u << 23) ? a : (121u << 23));   // |x| clamped to 2^-6
    const uint32_t sub = (uint32_t)__builtin_rintf(small * 512.0f);             // 0 .. 8
    uint32_t code = a >= (121u << 23) ? nrm : sub;
    code = a >= 0x43E00000u ? 0x7Eu : code;            // |x| >= 448 (incl. inf): saturate
    code |= sign;
    return a > 0x7F800000u ? 0x7Fu : code;             // NaN
}

// Same-dtype append: one 16-byte chunk per thread.
__global__ __launch_bounds__(256) void kv_append_copy(AppendParams p, int row_bytes) {
    const int chunks = row_bytes / 16;
    const int64_t per_kv = (int64_t)p.T * p.H_kv * chunks;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= 2 * per_kv) return;
    const int which = idx >= per_kv;                   // 0: K, 1: V
    int64_t rem = idx - which * per_kv;
    const int chunk = (int)(rem % chunks);
    rem /= chunks;
    const int g = (int)(rem % p.H_kv);
    const int t = (int)(rem / p.H_kv);
    const int32_t slot = p.slots[t];
    if (slot < 0 || (int64_t)slot >= p.num_slots) return;
    const int64_t blk = slot / kBlock, row = slot % kBlock;
    const char* src = reinterpret_cast<const char*>(which ? p.v_src : p.k_src) +
                      ((int64_t)t * p.H_kv + g) * row_bytes + (int64_t)chunk * 16;
    char* dst = reinterpret_cast<char*>(which ? p.v_pool : p.k_pool) +
                ((blk * p.H_kv + g) * kBlock + row) * row_bytes + (int64_t)chunk * 16;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

// Quantising append into an FP8 pool: 16 codes (one 16-byte chunk) per thread.
template <int SRC>
__global__ __launch_bounds__(256) void kv_append_fp8(AppendParams p) {
    constexpr int SE = SRC == DT_F32 ? 4 : 2;
    const int chunks = p.D / 16;
    const int64_t per_kv = (int64_t)p.T * p.H_kv * chunks;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= 2 * per_kv) return;
    const int which = idx >= per_kv;
    int64_t rem = idx - which * per_kv;
    const int chunk = (int)(rem % chunks);
    rem /= chunks;
    const int g = (int)(rem % p.H_kv);
    const int t = (int)(rem / p.H_kv);
    const int32_t slot = p.slots[t];
    if (slot < 0 || (int64_t)slot >= p.num_slots) return;
    const int64_t blk = slot / kBlock, row = slot % kBlock;
    const float inv = (which ? p.v_inv : p.k_inv)[g];
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(which ? p.v_src : p.k_src) +
                                                      (((int64_t)t * p.H_kv + g) * p.D + (int64_t)chunk * 16) * SE);
    uint4 raw[SE];                                     // the chunk's 16 source values, 16-byte loads
#pragma unroll
    for (int i = 0; i < SE; ++i) raw[i] = src[i];
    const uint32_t* rw = reinterpret_cast<const uint32_t*>(raw);
    uint32_t words[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t packed = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = 4 * w + k;
            float x;
            if constexpr (SRC == DT_F32) x = __uint_as_float(rw[e]);
            else x = __uint_as_float(e & 1 ? rw[e >> 1] & 0xFFFF0000u : rw[e >> 1] << 16);   // bf16
            packed |= e4m3_from_f32(x * inv) << (8 * k);
        }
        words[w] = packed;
    }
    char* dst = reinterpret_cast<char*>(which ? p.v_pool : p.k_pool) +
                ((blk * p.H_kv + g) * kBlock + row) * p.D + (int64_t)chunk * 16;
    *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
}

// ---------------------------------------------------------------------------
// INT8 per-block min-max (www.mooersco.com/news/1484987 §3.3): codes
// q = round((x - min) / (max - min) * 255) with one (min, max) per (block, KV
// head) tile, separately for K and V.  Every step is fp32 in the formula's
// order, rounded once each (no fused multiply-add), so the codes are exactly
// determined by the values and the order of the calls.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t int8_code(float x, float lo, float hi) {
#pragma clang fp contract(off)
    if (!(hi > lo)) return 0u;
    const float t = (x - lo) / (hi - lo);                        // correctly rounded fp32 division
    const float c = __builtin_rintf(t * 255.0f);                  // round half to even
    if (!(c >= 0.0f)) return 0u;                                  // negative or NaN
    return c >= 255.0f ? 255u : (uint32_t)c;
}

__device__ __forceinline__ float int8_step(float lo, float hi) { return (hi - lo) / 255.0f; }

template <int SRC>
__device__ __forceinline__ float src_value(const void* p, int64_t i) {
    if constexpr (SRC == DT_F32) return reinterpret_cast<const float*>(p)[i];
    else if constexpr (SRC == DT_F16) return (float)reinterpret_cast<const _Float16*>(p)[i];
    else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
}

// Pass 1: each written slot records (this call's epoch, token).
__global__ __launch_bounds__(256) void kv_append_int8_tag(AppendParams p) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= p.T) return;
    const int32_t slot = p.slots[t];
    if (slot < 0 || (int64_t)slot >= p.num_slots) return;
    p.tags[slot] = ((uint64_t)p.epoch << 32) | (uint32_t)t;
}

// Pass 2: one wave per (token, KV head).  The wave of the lowest token of this
// call in a tile encodes the whole tile (K, then V); the others exit.  Lane r
// < 16 learns which token writes row r this call (or none).
template <int SRC>
__global__ __launch_bounds__(64) void kv_append_int8(AppendParams p) {
#pragma clang fp contract(off)   // a re-encoded value is min + code * step, rounded twice
    const int t = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
    const int32_t slot = p.slots[t];
    if (slot < 0 || (int64_t)slot >= p.num_slots) return;
    const int64_t blk = slot / kBlock;
    int writer = -1;
    if (lane < kBlock) {
        const uint64_t tag = p.tags[blk * kBlock + lane];
        if ((uint32_t)(tag >> 32) == p.epoch) writer = (int)(uint32_t)tag;
    }
    int lowest = writer < 0 ? 0x7FFFFFFF : writer;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lowest = min(lowest, __shfl_xor(lowest, o, 64));
    if (lowest != t) return;                             // uniform: another wave owns the tile
    const uint32_t written = (uint32_t)__builtin_amdgcn_ballot_w64(lane < kBlock && writer >= 0) & 0xFFFFu;
    const bool fresh = written & 1u;                     // row 0 written: the tile starts over
    const int D = p.D;
    const int64_t tile = tile_bytes(DT_INT8, D);
    for (int which = 0; which < 2; ++which) {
        uint8_t* base = reinterpret_cast<uint8_t*>(which ? p.v_pool : p.k_pool) + (blk * p.H_kv + g) * tile;
        float* header = reinterpret_cast<float*>(base + (int64_t)kBlock * D);
        const void* src = which ? p.v_src : p.k_src;
        // the range of this call's values in the tile
        float lo = INFINITY, hi = -INFINITY;
        for (int r = 0; r < kBlock; ++r) {
            if (!((written >> r) & 1u)) continue;        // uniform
            const int tr = __shfl(writer, r, 64);
            const int64_t row0 = ((int64_t)tr * p.H_kv + g) * D;
            for (int e = lane; e < D; e += 64) {
                const float x = src_value<SRC>(src, row0 + e);
                lo = fminf(lo, x);
                hi = fmaxf(hi, x);
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            lo = fminf(lo, __shfl_xor(lo, o, 64));
            hi = fmaxf(hi, __shfl_xor(hi, o, 64));
        }
        if (!fresh) {
            const float old_lo = header[0], old_hi = header[1];
            const float new_lo = fminf(old_lo, lo), new_hi = fmaxf(old_hi, hi);
            if (new_lo != old_lo || new_hi != old_hi) {  // the range moved: re-encode the other rows
                const float old_step = int8_step(old_lo, old_hi);
                for (int i = lane; i < kBlock * D; i += 64) {
                    const int r = i / D;
                    if ((written >> r) & 1u) continue;
                    const float v = old_lo + (float)base[i] * old_step;   // two roundings (contract off)
                    base[i] = (uint8_t)int8_code(v, new_lo, new_hi);
                }
            }
            lo = new_lo;
            hi = new_hi;
        }
        for (int r = 0; r < kBlock; ++r) {
            if (!((written >> r) & 1u)) continue;
            const int tr = __shfl(writer, r, 64);
            const int64_t row0 = ((int64_t)tr * p.H_kv + g) * D;
            for (int e = lane; e < D; e += 64) base[r * D + e] = (uint8_t)int8_code(src_value<SRC>(src, row0 + e), lo, hi);
        }
        if (lane == 0) {
            header[0] = lo;
            header[1] = hi;
            header[2] = int8_step(lo, hi);
            header[3] = 0.0f;
        }
    }
}

// Plain copy, 16 bytes per load/store, four independent chunks per thread per step.
__global__ __launch_bounds__(256) void pkv_copy_kernel(uint4* __restrict__ dst,
                                                       const uint4* __restrict__ src, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        dst[i] = a;
        dst[i + stride] = b;
        dst[i + 2 * stride] = c;
        dst[i + 3 * stride] = d;
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

// Copy-on-write: copy whole blocks (all KV heads) src[i] -> dst[i] in both
// pools; blockIdx.y selects the pair, 16 bytes per thread.
__global__ __launch_bounds__(256) void kv_copy_blocks(CopyParams p) {
    const int pair = blockIdx.y;
    const int64_t n16 = p.block_bytes / 16;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (pair >= p.n || i >= 2 * n16) return;
    const bool v = i >= n16;
    const int64_t j = v ? i - n16 : i;
    char* base = reinterpret_cast<char*>(v ? p.v_pool : p.k_pool);
    const uint4* src = reinterpret_cast<const uint4*>(base + (int64_t)p.src[pair] * p.block_bytes);
    uint4* dst = reinterpret_cast<uint4*>(base + (int64_t)p.dst[pair] * p.block_bytes);
    dst[j] = src[j];
}

// Swap staging: blockIdx.y selects the block, 16 bytes per thread over its
// K tile then its V tile.
__global__ __launch_bounds__(256) void kv_move_blocks(MoveParams p) {
    const int b = blockIdx.y;
    const int64_t n16 = p.block_bytes / 16;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= p.n || i >= 2 * n16) return;
    const bool v = i >= n16;
    const int64_t j = v ? i - n16 : i;
    uint4* pool = reinterpret_cast<uint4*>(reinterpret_cast<char*>(v ? p.v_pool : p.k_pool) +
                                           (int64_t)p.ids[b] * p.block_bytes) + j;
    uint4* stage = reinterpret_cast<uint4*>(p.staging + (p.first + b) * 2 * p.block_bytes + (v ? p.block_bytes : 0)) + j;
    if (p.to_pool) *pool = *stage;
    else *stage = *pool;
}

}  // namespace

hipError_t launch_move_blocks(const MoveParams& p, hipStream_t stream) {
    if (p.n <= 0) return hipSuccess;
    MoveParams arg = p;
    void* args[] = {&arg};
    const int64_t threads = 2 * (p.block_bytes / 16);
    return launch_kernel(reinterpret_cast<const void*>(kv_move_blocks),
                           dim3((unsigned)((threads + 255) / 256), (unsigned)p.n), dim3(256), args, 0, stream);
}

hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t stream) {
    if (p.n <= 0) return hipSuccess;
    CopyParams arg = p;
    void* args[] = {&arg};
    const int64_t threads = 2 * (p.block_bytes / 16);
    return launch_kernel(reinterpret_cast<const void*>(kv_copy_blocks),
                           dim3((unsigned)((threads + 255) / 256), (unsigned)p.n), dim3(256), args, 0, stream);
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
    if (p.T <= 0) return hipSuccess;
    AppendParams arg = p;
    if (p.dst_dt == DT_INT8) {
        if (!p.tags || p.epoch == 0) return hipErrorInvalidValue;
        void* args[] = {&arg};
        hipError_t e = launch_kernel(reinterpret_cast<const void*>(kv_append_int8_tag),
                                       dim3((unsigned)((p.T + 255) / 256)), dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
        const void* fn = p.src_dt == DT_F32   ? reinterpret_cast<const void*>(kv_append_int8<DT_F32>)
                         : p.src_dt == DT_F16 ? reinterpret_cast<const void*>(kv_append_int8<DT_F16>)
                                              : reinterpret_cast<const void*>(kv_append_int8<DT_BF16>);
        return launch_kernel(fn, dim3((unsigned)p.T, (unsigned)p.H_kv), dim3(64), args, 0, stream);
    }
    if (p.dst_dt == p.src_dt) {
        int row_bytes = p.D * elem_bytes(p.dst_dt);
        const int64_t threads = 2LL * p.T * p.H_kv * (row_bytes / 16);
        const unsigned blocks = (unsigned)((threads + 255) / 256);
        void* args[] = {&arg, &row_bytes};
        return launch_kernel(reinterpret_cast<const void*>(kv_append_copy), dim3(blocks), dim3(256), args,
                               0, stream);
    }
    if (p.dst_dt == DT_FP8 && (p.src_dt == DT_BF16 || p.src_dt == DT_F32)) {
        const int64_t threads = 2LL * p.T * p.H_kv * (p.D / 16);
        const unsigned blocks = (unsigned)((threads + 255) / 256);
        void* args[] = {&arg};
        const void* fn = p.src_dt == DT_BF16 ? reinterpret_cast<const void*>(kv_append_fp8<DT_BF16>)
                                             : reinterpret_cast<const void*>(kv_append_fp8<DT_F32>);
        return launch_kernel(fn, dim3(blocks), dim3(256), args, 0, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;          // grid-stride beyond 64 workgroups per CU
    uint4* d = reinterpret_cast<uint4*>(dst);
    const uint4* s = reinterpret_cast<const uint4*>(src);
    void* args[] = {&d, &s, &n};
    return launch_kernel(reinterpret_cast<const void*>(pkv_copy_kernel), dim3((unsigned)blocks), dim3(256),
                           args, 0, stream);
}

}  // namespace pkv
