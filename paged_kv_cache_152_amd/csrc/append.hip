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

// The 16 source values of chunk c (16 consecutive elements) of a token's row,
// with 16-byte loads: the source is 16-byte aligned and D is a multiple of 16.
template <int SRC>
__device__ __forceinline__ void src_chunk16(const void* p, int64_t row0, int c, float (&x)[16]) {
    if constexpr (SRC == DT_F32) {
        const uint4* q = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(p) + row0) + 4 * c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 w = q[i];
            x[4 * i] = __uint_as_float(w.x);
            x[4 * i + 1] = __uint_as_float(w.y);
            x[4 * i + 2] = __uint_as_float(w.z);
            x[4 * i + 3] = __uint_as_float(w.w);
        }
    } else {
        const uint4* q = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + row0) + 2 * c;
        uint32_t w[8];
        const uint4 a = q[0], b = q[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (SRC == DT_F16) {
                x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
                x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
            } else {                                                   // bf16
                x[2 * i] = __uint_as_float(w[i] << 16);
                x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        }
    }
}

// Pass 1 of calls over 64 tokens: each written slot records (this call's
// epoch, token).
__global__ __launch_bounds__(256) void kv_append_int8_tag(AppendParams p) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= p.T) return;
    const int32_t slot = p.slots[t];
    if (slot < 0 || (int64_t)slot >= p.num_slots) return;
    p.tags[slot] = ((uint64_t)p.epoch << 32) | (uint32_t)t;
}

constexpr int kInt8ScanTokens = 64;   // calls up to this many tokens find a tile's writers by a scan

// One wave per (token, KV head, K or V).  The wave of the lowest token of this
// call in a tile encodes the whole tile; the others exit.  Lane r < 16
// learns which token writes row r this call (or none): from the slots
// themselves when the call has at most 64 tokens (SCAN: lane j holds token j's
// slot; ties between duplicate slots go to the lower token), else from the
// tags of pass 1.  Work on a tile goes in 16-byte chunks of a row.
template <int SRC, bool SCAN>
__global__ __launch_bounds__(64) void kv_append_int8(AppendParams p) {
#pragma clang fp contract(off)   // a re-encoded value is min + code * step, rounded twice
    __shared__ int row_writer[kBlock];
    const int t = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
    const int32_t slot = p.slots[t];
    if (slot < 0 || (int64_t)slot >= p.num_slots) return;
    const int64_t blk = slot / kBlock;
    int writer = -1;
    if constexpr (SCAN) {
        const int32_t s = lane < p.T ? p.slots[lane] : -1;
        const bool mine = s >= 0 && (int64_t)s < p.num_slots && s / kBlock == blk;
        const int row = mine ? s % kBlock : kBlock;
#pragma unroll
        for (int r = 0; r < kBlock; ++r) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(row == r);
            if (lane == r && m) writer = __builtin_ctzll(m);
        }
    } else if (lane < kBlock) {
        const uint64_t tag = p.tags[blk * kBlock + lane];
        if ((uint32_t)(tag >> 32) == p.epoch) writer = (int)(uint32_t)tag;
    }
    int lowest = writer < 0 ? 0x7FFFFFFF : writer;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lowest = min(lowest, __shfl_xor(lowest, o, 64));
    if (lowest != t) return;                             // uniform: another wave owns the tile
    const uint32_t written = (uint32_t)__builtin_amdgcn_ballot_w64(lane < kBlock && writer >= 0) & 0xFFFFu;
    if (lane < kBlock) row_writer[lane] = writer;
    __syncthreads();
    const bool fresh = written & 1u;                     // row 0 written: the tile starts over
    const int D = p.D, cpr = D / 16, chunks = kBlock * cpr;
    const int64_t tile = tile_bytes(DT_INT8, D);
    {
        const int which = blockIdx.z;                    // 0: K, 1: V
        uint8_t* bbase = reinterpret_cast<uint8_t*>(which ? p.v_pool : p.k_pool) + blk * p.H_kv * tile;
        uint8_t* base = bbase + (int64_t)g * kBlock * D;                 // the codes
        uint4* base4 = reinterpret_cast<uint4*>(base);
        float* header = reinterpret_cast<float*>(bbase + (int64_t)p.H_kv * kBlock * D + kInt8HeaderBytes * g);
        const void* src = which ? p.v_src : p.k_src;
        // the range of this call's values in the tile
        float lo = INFINITY, hi = -INFINITY;
        for (int c = lane; c < chunks; c += 64) {
            const int r = c / cpr;
            if (!((written >> r) & 1u)) continue;
            float x[16];
            src_chunk16<SRC>(src, ((int64_t)row_writer[r] * p.H_kv + g) * D, c - r * cpr, x);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                lo = fminf(lo, x[k]);
                hi = fmaxf(hi, x[k]);
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
                for (int c = lane; c < chunks; c += 64) {
                    if ((written >> (c / cpr)) & 1u) continue;
                    uint4 w = base4[c];
                    uint32_t* wv = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t o = 0;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const float v = old_lo + (float)((wv[i] >> (8 * k)) & 0xFFu) * old_step;  // two roundings
                            o |= int8_code(v, new_lo, new_hi) << (8 * k);
                        }
                        wv[i] = o;
                    }
                    base4[c] = w;
                }
            }
            lo = new_lo;
            hi = new_hi;
        }
        for (int c = lane; c < chunks; c += 64) {
            const int r = c / cpr;
            if (!((written >> r) & 1u)) continue;
            float x[16];
            src_chunk16<SRC>(src, ((int64_t)row_writer[r] * p.H_kv + g) * D, c - r * cpr, x);
            uint32_t wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t o = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) o |= int8_code(x[4 * i + k], lo, hi) << (8 * k);
                wv[i] = o;
            }
            base4[c] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
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
        if (!p.tags || p.epoch == 0 || p.D % 16) return hipErrorInvalidValue;
        void* args[] = {&arg};
        const bool scan = p.T <= kInt8ScanTokens;
        if (!scan) {
            hipError_t e = launch_kernel(reinterpret_cast<const void*>(kv_append_int8_tag),
                                         dim3((unsigned)((p.T + 255) / 256)), dim3(256), args, 0, stream);
            if (e != hipSuccess) return e;
        }
        const void* fn =
            scan ? (p.src_dt == DT_F32   ? reinterpret_cast<const void*>(kv_append_int8<DT_F32, true>)
                    : p.src_dt == DT_F16 ? reinterpret_cast<const void*>(kv_append_int8<DT_F16, true>)
                                         : reinterpret_cast<const void*>(kv_append_int8<DT_BF16, true>))
                 : (p.src_dt == DT_F32   ? reinterpret_cast<const void*>(kv_append_int8<DT_F32, false>)
                    : p.src_dt == DT_F16 ? reinterpret_cast<const void*>(kv_append_int8<DT_F16, false>)
                                         : reinterpret_cast<const void*>(kv_append_int8<DT_BF16, false>));
        return launch_kernel(fn, dim3((unsigned)p.T, (unsigned)p.H_kv, 2), dim3(64), args, 0, stream);
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
