// Paged single-token decode attention for gfx950 (CDNA4, wave64).
//
// What is computed (www.mlqm.cn/news/394450, sections 二 and 四; block table of
// www.cf-1.com/news/5824798 §3.1; GQA of www.mlqm.cn/news/394450 section 六):
// for sequence b and query head h, with G query heads per KV head g = h / G,
//   out[b][h] = sum_j softmax_j(scale * <q[b][h], K_b[j][g]>) * V_b[j][g],
// where token j of sequence b sits in physical block tables[b][j / 16], row
// j % 16, of the pool [num_blocks][H_kv][16][D] (K and V in separate pools).
//
// Work split.  Kernel 1 takes one (partition of the context, KV head, sequence)
// per workgroup of 4 waves.  The workgroup serves all GS query heads of its KV
// head, so every K/V tile is fetched from HBM once per group, not once per
// query head.  Inside a wave, lane l owns row r = l / LPR and a 16-byte chunk
// c = l % LPR of a token's row: one wave-wide load brings RPL token rows of a
// 16-token tile, NLOAD loads bring the whole tile.  Every row of lanes keeps
// its own online-softmax state (running max m, running sum l, accumulator o)
// over the tokens it loads, so the only cross-lane traffic per token is the
// DPP sum of the dot product inside the row.  The next block's K and V are
// loaded before the current one is consumed.  At the end the rows and waves of
// the workgroup merge through LDS, and the workgroup writes either the final
// output (single partition) or (m, l, o) for kernel 2, which merges the
// partitions of a sequence with the same log-sum-exp rule.
//
// Logits are kept in base 2: q is pre-multiplied by scale * log2(e) (and by the
// K scale of an FP8 pool), and exp2 is the hardware v_exp_f32.  For FP8 pools
// the V scale multiplies the merged output.
#include "internal.h"

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <unordered_map>

// Fixed scratch of paged_decode_noalloc (work list and partial results), one
// copy per device for the life of the process.  Host code never passes this
// name to a kernel or a copy: it only stands in for the device array on the
// host side.  noalloc_scratch() below looks up the device address.
static __device__ __align__(256) unsigned char scratch[pkv::kNoAllocScratchBytes];

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elem<DT_F16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_FP8> { static constexpr int bytes = 1; };
template <> struct Elem<DT_INT8> { static constexpr int bytes = 1; };

// Geometry of one (block, KV head) tile [16][D] of storage type DT.
template <int DT, int D> struct Tile {
    static constexpr int E = Elem<DT>::bytes;
    static constexpr int ROW = D * E;                                // bytes of one token row
    static constexpr int BYTES = kBlock * ROW;                       // bytes of the tile's elements
    static constexpr int STRIDE = BYTES + (DT == DT_INT8 ? kInt8HeaderBytes : 0);   // tile to tile
    static constexpr int W = BYTES / 64 >= 16 ? 16 : BYTES / 64;     // bytes per lane per load
    static constexpr int EPL = W / E;                                // elements per lane per load
    static constexpr int LPR = ROW / W;                              // lanes per token row
    static constexpr int RPL = 64 / LPR;                             // token rows per wave load
    static constexpr int NLOAD = kBlock / RPL;                       // loads per tile
    static_assert(BYTES >= 256 && W >= 4, "tile too small for one wave");
    static_assert((LPR & (LPR - 1)) == 0 && LPR <= 32, "row must span a power of two of lanes");
};

template <int W> struct Raw;
template <> struct Raw<4> { using T = uint32_t; static constexpr int words = 1; };
template <> struct Raw<8> { using T = uint2; static constexpr int words = 2; };
template <> struct Raw<16> { using T = uint4; static constexpr int words = 4; };

template <int W>
__device__ __forceinline__ uint32_t word(const typename Raw<W>::T& r, int i) {
    if constexpr (W == 4) return r;
    else return reinterpret_cast<const uint32_t*>(&r)[i];
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Widen the EPL stored elements of one lane chunk to fp32.
template <int DT, int W>
__device__ __forceinline__ void widen(const typename Raw<W>::T& r, float* f) {
    constexpr int NW = Raw<W>::words;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t w = word<W>(r, i);
        if constexpr (DT == DT_F32) {
            f[i] = __uint_as_float(w);
        } else if constexpr (DT == DT_F16) {
            f[2 * i] = f16lo(w);
            f[2 * i + 1] = f16hi(w);
        } else if constexpr (DT == DT_BF16) {
            f[2 * i] = bf16lo(w);
            f[2 * i + 1] = bf16hi(w);
        } else if constexpr (DT == DT_INT8) {  // min-max codes as integers 0..255 (exact)
#pragma unroll
            for (int k = 0; k < 4; ++k) f[4 * i + k] = (float)((w >> (8 * k)) & 0xFFu);
        } else {  // OCP E4M3 -> fp32, two codes per instruction
            auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
            auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
            f[4 * i] = lo[0];
            f[4 * i + 1] = lo[1];
            f[4 * i + 2] = hi[0];
            f[4 * i + 3] = hi[1];
        }
    }
}

template <int QDT>
__device__ __forceinline__ float load_q(const void* q, int64_t i) {
    if constexpr (QDT == DT_F32) return reinterpret_cast<const float*>(q)[i];
    else if constexpr (QDT == DT_F16) return (float)reinterpret_cast<const _Float16*>(q)[i];
    else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(q)[i] << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int QDT>
__device__ __forceinline__ void store_out(void* out, int64_t i, float x) {
    if constexpr (QDT == DT_F32) reinterpret_cast<float*>(out)[i] = x;
    else if constexpr (QDT == DT_F16) reinterpret_cast<_Float16*>(out)[i] = (_Float16)x;
    else reinterpret_cast<uint16_t*>(out)[i] = f32_to_bf16_rne(x);
}

// Sum over the LPR lanes of a row; every lane of the row gets the same value.
// Pairs are combined symmetrically (a+b on one side, b+a on the other), so the
// result is bit-identical across the row.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
    if constexpr (LPR >= 2) v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    if constexpr (LPR >= 4) v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    if constexpr (LPR >= 8) v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    if constexpr (LPR >= 16) v += __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, false); // row_mirror
    if constexpr (LPR >= 32) v += __shfl_xor(v, 16, 64);
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Loads of the cached keys and values.  With NT the nontemporal hint is set:
// each byte is read once per call, and on this part a stream of such loads
// runs at about 6.8 TB/s where plain loads level off near 6.0.  The hint is
// used where one load instruction covers whole 128-byte lines, or half lines
// whose other half the next instruction reads.  A line split over four
// instructions (the 8-byte key loads of E4M3 pools) is fetched more than once
// under the hint, so those loads stay plain.
template <class T, bool NT = true>
__device__ __forceinline__ T load_kv(const char* p) {
    if constexpr (!NT) return *reinterpret_cast<const T*>(p);
    static_assert(sizeof(T) == 16 || sizeof(T) == 8 || sizeof(T) == 4, "16-, 8- or 4-byte loads");
    if constexpr (sizeof(T) == 16) {
        typedef uint32_t v4 __attribute__((ext_vector_type(4)));
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const v4*>(p)));
    } else if constexpr (sizeof(T) == 8) {
        typedef uint32_t v2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const v2*>(p)));
    } else {
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)));
    }
}

// ---------------------------------------------------------------------------
// Pieces shared by both partition kernels.
// ---------------------------------------------------------------------------

// Context length of sequence b, clamped to what the launch was sized for.
__device__ __forceinline__ int clamped_len(const DecodeParams& p, int b) {
    int n = p.lens[b];
    n = n < 0 ? 0 : n;
    n = n > p.max_len ? p.max_len : n;
    return n > p.max_blocks * kBlock ? p.max_blocks * kBlock : n;
}

// Schedule header in the workspace.  The work counter, hammered by atomics,
// has a cache line of its own; the item count and the partition length the
// plan kernel chose sit on another.
constexpr int kSchedCounter = 0;
constexpr int kSchedItems = 32;
constexpr int kSchedPart = 33;

// Partition length in tokens: the plan kernel's choice in planned mode.  Read
// once per workgroup.
__device__ __forceinline__ int part_tokens(const DecodeParams& p) {
    return p.items ? p.sched[kSchedPart] : p.part_tokens;
}

__device__ __forceinline__ int num_parts(int P, int n) { return (n + P - 1) / P; }

// The k = ceil(n / P) partitions of a sequence split its blocks evenly:
// partition i covers blocks [i*nb/k, (i+1)*nb/k), so no partition is a small
// remainder and every one holds at most about P tokens.
struct Range {
    int n, nparts, blk_first, blk_last, pend;
};

__device__ __forceinline__ Range partition_range(const DecodeParams& p, int P, int b, int part) {
    Range R;
    R.n = clamped_len(p, b);
    R.nparts = num_parts(P, R.n);
    const int nb = (R.n + kBlock - 1) / kBlock;
    R.blk_first = (int)((int64_t)part * nb / max(R.nparts, 1));
    R.blk_last = (int)((int64_t)(part + 1) * nb / max(R.nparts, 1));
    R.pend = min(R.n, R.blk_last * kBlock);
    return R;
}

// The physical block ids of one wave's blocks (blk0, blk0 + 4, ...), 64 at a
// time, one entry per lane, fetched with a single vector load and read back
// with readlane.  Loading them up front keeps the table lookups off the path
// between one block's K/V loads and the next.
struct WaveTable {
    int v = -1;
    __device__ __forceinline__ void load(const int32_t* table, int blk0, int nmine, int j0, int lane) {
        const int j = j0 + lane;
        v = j < nmine ? table[blk0 + kDecodeWaves * j] : -1;
    }
    __device__ __forceinline__ int phys(int j) const { return __builtin_amdgcn_readlane(v, j & 63); }
};

// Merge the NS softmax streams of a workgroup (per head: running max s_m,
// running sum s_l, unnormalised accumulator s_o) and write either the final
// output (one partition) or the partition's (m, l, o) for the reduce kernel.
template <int QDT, int D, int GS, int NS>
__device__ __forceinline__ void merge_streams(const DecodeParams& p, const float (*s_m)[GS],
                                              const float (*s_l)[GS], const float (*s_o)[GS][D], int b,
                                              int hq0, int part, bool single, float vscale) {
    for (int i = threadIdx.x; i < GS * D; i += kDecodeWaves * 64) {
        const int h = i / D, d = i % D;
        float M = -INFINITY;
        for (int t = 0; t < NS; ++t) M = fmaxf(M, s_m[t][h]);
        float L = 0.0f, O = 0.0f;
        if (M != -INFINITY) {
            for (int t = 0; t < NS; ++t) {
                const float w = fast_exp2(s_m[t][h] - M);
                L = fmaf(s_l[t][h], w, L);
                O = fmaf(s_o[t][h][d], w, O);
            }
        }
        O *= vscale;
        const int hq = hq0 + h;
        if (single) {
            store_out<QDT>(p.out, ((int64_t)b * p.H_q + hq) * D + d, L > 0.0f ? O / L : 0.0f);
        } else {
            const int64_t slot = ((int64_t)b * p.H_q + hq) * p.max_parts + part;
            p.ws_o[slot * D + d] = O;
            if (d == 0) {
                p.ws_ml[slot * 2] = M;
                p.ws_ml[slot * 2 + 1] = L;
            }
        }
    }
}

template <int QDT, int D, int GS>
__device__ __forceinline__ void zero_output(const DecodeParams& p, int b, int hq0) {
    for (int i = threadIdx.x; i < GS * D; i += kDecodeWaves * 64)
        store_out<QDT>(p.out, ((int64_t)b * p.H_q + hq0) * D + i, 0.0f);
}

// Walk this wave's blocks j = 0 .. nmine-1 through a ring of NB buffers: the
// loads of blocks j+1 .. j+NB-1 are in flight while block j is consumed, and
// no registers are copied (the ring position is a compile-time index).
// fetch(j, buf) issues the loads; consume(j, buf) uses them.
template <int NB, class Buf, class Fetch, class Consume>
__device__ __forceinline__ void pipeline(int nmine, Fetch&& fetch, Consume&& consume) {
    Buf ring[NB];
#pragma unroll
    for (int k = 0; k < NB - 1; ++k)
        if (k < nmine) fetch(k, ring[k]);
    for (int j0 = 0; j0 < nmine; j0 += NB) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int j = j0 + k;
            if (j >= nmine) return;
            if (j + NB - 1 < nmine) fetch(j + NB - 1, ring[(k + NB - 1) % NB]);
            consume(j, ring[k]);
        }
    }
}

// The vector kernel's variant of the two helpers above.  The wave's block ids
// come from scalar loads one block ahead (take(j) returns block j's id, loaded
// during take(j - 1), and starts the load of block j + 1's; past the wave's
// last block it returns -1), and every step fetches, also past the last block
// (fetch then reads block 0 and marks it absent).  With no load behind a
// branch the compiler counts the loads in flight and waits for block j's alone
// before consuming it.  On the matrix-core kernel the same change measured
// slower (table entries through the scalar cache stall its waves); on the
// vector kernel it is faster.
struct ScalarWaveTable {
    const __attribute__((address_space(4))) int32_t* row = nullptr;
    int blk0 = 0, nmine = 0, next = -1;
    __device__ __forceinline__ int entry(int j) const {
        return nmine > 0 ? row[blk0 + kDecodeWaves * min(j, nmine - 1)] : -1;
    }
    __device__ __forceinline__ void init(const int32_t* table, int blk0_, int nmine_) {
        row = (const __attribute__((address_space(4))) int32_t*)table;
        blk0 = blk0_;
        nmine = nmine_;
        next = entry(0);
    }
    __device__ __forceinline__ int take(int j) {
        const int cur = j < nmine ? next : -1;
        next = entry(j + 1);
        return cur;
    }
};

template <int NB, class Buf, class Fetch, class Consume>
__device__ __forceinline__ void pipeline_all(int nmine, Fetch&& fetch, Consume&& consume) {
    Buf ring[NB];
#pragma unroll
    for (int k = 0; k < NB - 1; ++k) fetch(k, ring[k]);
    for (int j0 = 0; j0 < nmine; j0 += NB) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int j = j0 + k;
            if (j >= nmine) return;
            fetch(j + NB - 1, ring[(k + NB - 1) % NB]);
            consume(j, ring[k]);
        }
    }
}

// ---------------------------------------------------------------------------
// Work distribution.
//
// Dense mode (no work list): a grid (partition, head group, sequence), one
// item per workgroup; used when every context fits one partition.
//
// Planned mode: kernel 0 (paged_decode_plan) lists the live (sequence,
// partition) items longest first, and the partition kernel runs a grid only
// as large as the GPU holds at once.  Each workgroup takes one of the first
// gridDim.x items (first_ticket), then further items from an atomic counter,
// until the list is exhausted:
// long partitions start first and short ones fill the tail.  Items are
// expanded over head groups (consecutive virtual items share a partition, so
// the heads of one block are read close together in time).  Which workgroup
// computes an item has no influence on the bits it produces.
// ---------------------------------------------------------------------------
// First ticket of workgroup i of n: workgroups are dealt round-robin over the
// 8 XCDs, so workgroup i takes ticket (i % 8) * (n / 8) + i / 8, and the head
// groups of one (sequence, partition), consecutive tickets, share an XCD and
// its L2 (the INT8 headers of a block sit on one line for all heads).
__device__ __forceinline__ int first_ticket(int i, int n) {
    const int full = n - n % 8;
    return i >= full ? i : (i % 8) * (full / 8) + i / 8;
}

template <class F>
__device__ __forceinline__ void for_each_item(const DecodeParams& p, F&& f) {
    __shared__ int s_next;
    const bool planned = p.items != nullptr;
    const int HG = p.head_groups;
    const int total = planned ? p.sched[kSchedItems] * HG : 1;
    const int P = part_tokens(p);
    int v = planned ? first_ticket((int)blockIdx.x, (int)gridDim.x) : 0;
    while (v < total) {                        // one call site, so the item body is inlined
        int b, part, hgi;
        if (planned) {
            const int2 it = p.items[v / HG];
            b = it.x;
            part = it.y;
            hgi = v % HG;
        } else {
            b = blockIdx.z;
            part = blockIdx.x;
            hgi = blockIdx.y;
        }
        f(b, part, hgi, P);
        if (!planned) break;
        __syncthreads();                       // this item's LDS reads are done
        if (threadIdx.x == 0) s_next = atomicAdd(&p.sched[kSchedCounter], 1) + (int)gridDim.x;
        __syncthreads();
        v = s_next;
    }
}

// Kernel 0: the work list.  Items are bucketed by partition length (in blocks),
// 32 buckets, longest bucket first; a zero-length sequence is one item (its
// output is zeroed).  The header holds the work counter, the item count and
// the partition length used.
//
// The partition length is the host's, except when every context has the same
// length n: then k equal partitions per context give B * head_groups * k
// items of one size, and a k that makes that a whole number of rounds of the
// grid (every workgroup the same number of items, no partly idle last round)
// is taken: the smallest such k with at least one round, up to max_parts
// (automatic partition only; a partition the caller set is kept).
constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 32;

__global__ __launch_bounds__(kPlanThreads) void paged_decode_plan(DecodeParams p) {
    __shared__ int cnt[kPlanBuckets];
    __shared__ int off[kPlanBuckets];
    __shared__ int s_min, s_max, s_P;
    const int tid = threadIdx.x;
    // each thread's first sequence stays in a register (B <= kPlanThreads needs
    // no second read of context_lens)
    const int n0 = tid < p.B ? clamped_len(p, tid) : 0;
    auto len_of = [&](int b) { return b == tid ? n0 : clamped_len(p, b); };
    if (tid < kPlanBuckets) cnt[tid] = 0;
    if (tid == 0) {
        s_min = INT_MAX;
        s_max = 0;
    }
    __syncthreads();
    int lo = INT_MAX, hi = 0;
    for (int b = tid; b < p.B; b += kPlanThreads) {
        const int n = len_of(b);
        lo = min(lo, n);
        hi = max(hi, n);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        lo = min(lo, __shfl_xor(lo, o, 64));
        hi = max(hi, __shfl_xor(hi, o, 64));
    }
    if ((tid & 63) == 0) {
        atomicMin(&s_min, lo);
        atomicMax(&s_max, hi);
    }
    __syncthreads();
    if (tid == 0) {
        int P = p.part_tokens;
        const int n = s_max;
        if (p.choose_parts && n > 0 && s_min == n) {
            const int64_t cols = (int64_t)p.B * p.head_groups;
            const int nb = (n + kBlock - 1) / kBlock;
            for (int k = 1; k <= p.max_parts && k <= nb; ++k) {
                const int Pk = (n + k - 1) / k;
                const int64_t items = cols * num_parts(Pk, n);
                if (items >= p.grid_wgs && items % p.grid_wgs == 0) {
                    P = Pk;
                    break;
                }
            }
        }
        s_P = P;
    }
    __syncthreads();
    const int P = s_P;
    const int max_blk = (P + kBlock - 1) / kBlock + 1;
    auto classify = [&](int b, int& k) {
        const int n = len_of(b);
        k = max(num_parts(P, n), 1);
        const int per = ((n + kBlock - 1) / kBlock + k - 1) / k;   // blocks per partition
        return min(kPlanBuckets - 1, (int)((int64_t)per * kPlanBuckets / (max_blk + 1)));
    };
    for (int b = tid; b < p.B; b += kPlanThreads) {
        int k;
        const int bk = classify(b, k);
        atomicAdd(&cnt[bk], k);
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = kPlanBuckets - 1; i >= 0; --i) {
            off[i] = run;
            run += cnt[i];
        }
        p.sched[kSchedCounter] = 0;
        p.sched[kSchedItems] = run;
        p.sched[kSchedPart] = P;
    }
    __syncthreads();
    for (int b = tid; b < p.B; b += kPlanThreads) {
        int k;
        const int bk = classify(b, k);
        const int base = atomicAdd(&off[bk], k);
        for (int i = 0; i < k; ++i) p.items[base + i] = make_int2(b, i);
    }
}

// ---------------------------------------------------------------------------
// Vector variant: any dtype, head_dim 16/64/128, any group size up to 8.
// ---------------------------------------------------------------------------
template <int NS, int GS, int D>
struct StreamSmem {
    float m[NS][GS];
    float l[NS][GS];
    float o[NS][GS][D];
};

// One work item of the vector variant: partition `part` of sequence b for
// head group hgi (KV head hgi / subs, query heads hq0 .. hq0 + GS - 1).
template <int KDT, int QDT, int D, int GS>
__device__ __forceinline__ void vec_item(const DecodeParams& p, int b, int part, int hgi, int P,
                                         StreamSmem<kDecodeWaves * Tile<KDT, D>::RPL, GS, D>& sm) {
    using TL = Tile<KDT, D>;
    using RawT = typename Raw<TL::W>::T;
    constexpr int EPL = TL::EPL, LPR = TL::LPR, RPL = TL::RPL, NLOAD = TL::NLOAD;
    constexpr int NS = kDecodeWaves * RPL;   // softmax streams per workgroup
    auto& s_m = sm.m;
    auto& s_l = sm.l;
    auto& s_o = sm.o;

    const int subs = p.G / GS;
    const int g = hgi / subs;
    const int hq0 = g * p.G + (hgi % subs) * GS;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane / LPR, c = lane % LPR;

    const Range R = partition_range(p, P, b, part);
    if (R.n == 0) {                      // empty context: out = 0, written by partition 0
        if (part == 0) zero_output<QDT, D, GS>(p, b, hq0);
        return;
    }
    if (part >= R.nparts) return;

    // Query fragment: this lane's EPL dims of each of the GS heads, scaled to base 2.
    float qscale = p.scale * kLog2e;
    if constexpr (KDT == DT_FP8) qscale *= p.k_scale[g];
    float qf[GS][EPL];
#pragma unroll
    for (int h = 0; h < GS; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            qf[h][e] = load_q<QDT>(p.q, ((int64_t)b * p.H_q + hq0 + h) * D + c * EPL + e) * qscale;
    // INT8 pools: a key is min + step * code, so <qf, key> = min * sum(qf) +
    // step * <qf, codes>; sum(qf) over the head is taken once.  The values'
    // min term is kept apart per stream (mv) and added when the streams merge.
    constexpr bool I8 = KDT == DT_INT8;
    float qsum[GS], mv[GS];
#pragma unroll
    for (int h = 0; h < GS; ++h) {
        qsum[h] = 0.0f;
        mv[h] = 0.0f;
        if constexpr (I8) {
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) s += qf[h][e];
            qsum[h] = row_sum<LPR>(s);
        }
    }

    float m[GS], l[GS], acc[GS][EPL];
#pragma unroll
    for (int h = 0; h < GS; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
    }

    const int32_t* table = p.tables + (int64_t)b * p.max_blocks;
    const char* kbase = reinterpret_cast<const char*>(p.k_pool);
    const char* vbase = reinterpret_cast<const char*>(p.v_pool);
    const int lane_off = r * NLOAD * TL::ROW + c * TL::W;
    // a block holds the codes of every KV head, then (INT8) their headers
    const int64_t head_off = (int64_t)g * TL::BYTES;
    const int64_t blk_stride = (int64_t)p.H_kv * TL::STRIDE;
    const int64_t hdr_off = (int64_t)p.H_kv * TL::BYTES + kInt8HeaderBytes * g;
    const int blk0 = R.blk_first + __builtin_amdgcn_readfirstlane(wave);   // uniform: scalar table loads
    const int nmine = blk0 < R.blk_last ? (R.blk_last - blk0 + kDecodeWaves - 1) / kDecodeWaves : 0;
    ScalarWaveTable wt;
    wt.init(table, blk0, nmine);

    struct Buf {
        RawT k[NLOAD], v[NLOAD];
        float4 kh, vh;                   // INT8: tile headers {min, max, step, 0}
        bool ok;
    };
    auto fetch = [&](int j, Buf& B) {
        const int phys = wt.take(j);
        B.ok = phys >= 0 && phys < p.num_blocks;
        const int64_t blk_base = (int64_t)(B.ok ? phys : 0) * blk_stride;   // absent: block 0, unused
        const int64_t off = blk_base + head_off + lane_off;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            B.k[i] = load_kv<RawT>(kbase + off + i * TL::ROW);
            B.v[i] = load_kv<RawT>(vbase + off + i * TL::ROW);
        }
        if constexpr (I8) {
            B.kh = *reinterpret_cast<const float4*>(kbase + blk_base + hdr_off);
            B.vh = *reinterpret_cast<const float4*>(vbase + blk_base + hdr_off);
        }
    };
    auto update = [&](auto masked, int blk, const Buf& B) {
        constexpr bool MASKED = decltype(masked)::value;
        const int tok0 = blk * kBlock + r * NLOAD;   // this row's first token in the block
        float z[GS][NLOAD];
        float vf[NLOAD][EPL];
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            float kf[EPL];
            widen<KDT, TL::W>(B.k[i], kf);
            widen<KDT, TL::W>(B.v[i], vf[i]);
            const bool valid = !MASKED || tok0 + i < R.pend;
#pragma unroll
            for (int h = 0; h < GS; ++h) {
                float d = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) d = fmaf(qf[h][e], kf[e], d);
                d = row_sum<LPR>(d);
                if constexpr (I8) d = fmaf(B.kh.z, d, B.kh.x * qsum[h]);
                z[h][i] = valid ? d : -INFINITY;
            }
            if (MASKED && !valid) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) vf[i][e] = 0.0f;   // select, never 0 * garbage
            }
        }
#pragma unroll
        for (int h = 0; h < GS; ++h) {
            float mx = z[h][0];
#pragma unroll
            for (int i = 1; i < NLOAD; ++i) mx = fmaxf(mx, z[h][i]);
            const float m_new = fmaxf(m[h], mx);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = fast_exp2(m[h] - m_use);
            float psum = 0.0f;
            float pv[NLOAD];
#pragma unroll
            for (int i = 0; i < NLOAD; ++i) {
                pv[i] = fast_exp2(z[h][i] - m_use);
                psum += pv[i];
            }
            l[h] = fmaf(l[h], alpha, psum);
            if constexpr (I8) {
                mv[h] = fmaf(mv[h], alpha, B.vh.x * psum);
#pragma unroll
                for (int i = 0; i < NLOAD; ++i) pv[i] *= B.vh.z;
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float a = acc[h][e] * alpha;
#pragma unroll
                for (int i = 0; i < NLOAD; ++i) a = fmaf(pv[i], vf[i][e], a);
                acc[h][e] = a;
            }
            m[h] = m_new;
        }
    };
    auto consume = [&](int j, const Buf& B) {
        if (!B.ok) return;
        const int blk = blk0 + kDecodeWaves * j;
        if (blk * kBlock + kBlock > R.pend) update(std::integral_constant<bool, true>{}, blk, B);
        else update(std::integral_constant<bool, false>{}, blk, B);
    };
    pipeline_all<2, Buf>(nmine, fetch, consume);

    const int s = wave * RPL + r;
#pragma unroll
    for (int h = 0; h < GS; ++h) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_o[s][h][c * EPL + e] = acc[h][e] + mv[h];
        if (c == 0) {
            s_m[s][h] = m[h];
            s_l[s][h] = l[h];
        }
    }
    __syncthreads();
    float vscale = 1.0f;
    if constexpr (KDT == DT_FP8) vscale = p.v_scale[g];
    merge_streams<QDT, D, GS, NS>(p, s_m, s_l, s_o, b, hq0, part, R.nparts == 1, vscale);
}

template <int KDT, int QDT, int D, int GS>
__global__ __launch_bounds__(kDecodeWaves * 64) void paged_decode_partition(DecodeParams p) {
    __shared__ StreamSmem<kDecodeWaves * Tile<KDT, D>::RPL, GS, D> sm;
    for_each_item(p, [&](int b, int part, int hgi, int P) { vec_item<KDT, QDT, D, GS>(p, b, part, hgi, P, sm); });
}

// ---------------------------------------------------------------------------
// Grouped-query variant (GS >= 3 query heads per KV head, head_dim 128,
// 16-bit or FP8 KV): Q.K^T on the matrix cores, P.V on the vector ALUs.
//
// Per 16-token block a wave issues KS = 4 v_mfma_f32_16x16x32 (bf16 or f16):
// A = the K tile (16 tokens x 32 dims per step), B = the queries (32 dims x 16
// head columns, GS of them live, the rest zero).  Lane l supplies A row
// m = l % 16 (a token) and B column n = l % 16 (a head), both for the dim group
// 8 * (4 s + l / 16) .. +7 of step s, so each lane's A operand is one 16-byte
// (8-byte for FP8) load of a token row.  The 16x16 fp32 result leaves scores
// of tokens 4r .. 4r+3 for head n in lane 16r + n (r = l / 16): exactly the
// tokens whose V rows the lanes of DPP row r load for the P.V update, so each
// head's weight reaches its row with one row_newbcast and every lane
// accumulates 8 output dims for all GS heads.  Each lane (r, n) keeps the
// running max / sum of stream (r, head n); the accumulators of stream (r, h)
// are spread over the 16 lanes of row r.  An FP8 tile is widened to bf16/f16
// (exact) for the MFMA and to fp32 for P.V.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

template <int QDT> struct MfmaIn;
template <> struct MfmaIn<DT_BF16> { using T = bf16x8_t; };
template <> struct MfmaIn<DT_F16> { using T = f16x8_t; };

template <int QDT>
__device__ __forceinline__ f32x4_t mfma16x16x32(const typename MfmaIn<QDT>::T& a, const typename MfmaIn<QDT>::T& b,
                                                f32x4_t c) {
    if constexpr (QDT == DT_BF16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 E4M3 codes (two words) -> 8 bf16 / f16 values, exact.
template <int QDT>
__device__ __forceinline__ typename MfmaIn<QDT>::T fp8x8_to_mfma(uint2 w) {
    uint32_t o[4];
    if constexpr (QDT == DT_BF16) {
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true));
    } else {
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true));
    }
    return __builtin_bit_cast(typename MfmaIn<QDT>::T, make_uint4(o[0], o[1], o[2], o[3]));
}

__device__ __forceinline__ float row_bcast(float v, int src_lane_in_row) {
    // DPP row_newbcast: every lane of a 16-lane row receives lane `src` of that row.
    switch (src_lane_in_row) {
        case 0: return __builtin_amdgcn_update_dpp(0.0f, v, 0x150, 0xF, 0xF, false);
        case 1: return __builtin_amdgcn_update_dpp(0.0f, v, 0x151, 0xF, 0xF, false);
        case 2: return __builtin_amdgcn_update_dpp(0.0f, v, 0x152, 0xF, 0xF, false);
        case 3: return __builtin_amdgcn_update_dpp(0.0f, v, 0x153, 0xF, 0xF, false);
        case 4: return __builtin_amdgcn_update_dpp(0.0f, v, 0x154, 0xF, 0xF, false);
        case 5: return __builtin_amdgcn_update_dpp(0.0f, v, 0x155, 0xF, 0xF, false);
        case 6: return __builtin_amdgcn_update_dpp(0.0f, v, 0x156, 0xF, 0xF, false);
        default: return __builtin_amdgcn_update_dpp(0.0f, v, 0x157, 0xF, 0xF, false);
    }
}

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));   // round to nearest even
}

__device__ __forceinline__ uint32_t row_bcast_u32(uint32_t v, int src_lane_in_row) {
    return __float_as_uint(row_bcast(__uint_as_float(v), src_lane_in_row));
}

// E4M3 codes of two tokens a, b at the same dims as f16 pairs: out[d] =
// (a[d], b[d]), d = 0..7 (words hold dims 4j .. 4j+3).  v_perm_b32 takes bytes
// 0-3 from its second source and 4-7 from its first; the f16 widening is exact.
__device__ __forceinline__ void fp8_token_pairs(const uint2& a, const uint2& b, uint32_t* out) {
    const uint32_t wa[2] = {a.x, a.y}, wb[2] = {b.x, b.y};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t lo = __builtin_amdgcn_perm(wb[j], wa[j], 0x05010400u);   // a0 b0 a1 b1
        const uint32_t hi = __builtin_amdgcn_perm(wb[j], wa[j], 0x07030602u);   // a2 b2 a3 b3
        out[4 * j + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
        out[4 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
        out[4 * j + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
        out[4 * j + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
    }
}

// 8 INT8 min-max codes (two words) -> 8 bf16 / f16 values (integers 0..255, exact).
template <int QDT>
__device__ __forceinline__ typename MfmaIn<QDT>::T u8x8_to_mfma(uint2 w) {
    const uint32_t ws[2] = {w.x, w.y};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t word = ws[j >> 1];
        const int sh = 16 * (j & 1);
        const f32x2_t v = {(float)((word >> sh) & 0xFFu), (float)((word >> (sh + 8)) & 0xFFu)};
        if constexpr (QDT == DT_BF16) o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
        else o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    }
    return __builtin_bit_cast(typename MfmaIn<QDT>::T, make_uint4(o[0], o[1], o[2], o[3]));
}

template <int KDT>
struct GqaTile {
    static constexpr int E = Elem<KDT>::bytes;
    static constexpr int ROW = 128 * E;                  // bytes of a token row
    static constexpr int BYTES = kBlock * ROW;
    static constexpr int STRIDE = BYTES + (KDT == DT_INT8 ? kInt8HeaderBytes : 0);
    static constexpr int KW = 8 * E;                      // bytes per lane per MFMA step (8 dims)
    using KRaw = typename Raw<KW>::T;                     // uint4 (16-bit) or uint2 (FP8)
    using VRaw = typename Raw<KW>::T;
};

template <int KDT, int QDT, int GS>
__device__ __forceinline__ void gqa_item(const DecodeParams& p, int b, int part, int hgi, int P,
                                         StreamSmem<kDecodeWaves * 4, GS, 128>& sm) {
    constexpr int D = 128, KS = 4, NS = kDecodeWaves * 4;
    using TL = GqaTile<KDT>;
    using KRaw = typename TL::KRaw;
    using MT = typename MfmaIn<QDT>::T;
    auto& s_m = sm.m;
    auto& s_l = sm.l;
    auto& s_o = sm.o;

    const int subs = p.G / GS;
    const int g = hgi / subs;
    const int hq0 = g * p.G + (hgi % subs) * GS;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane >> 4, c = lane & 15;      // DPP row; lane within the row

    const Range R = partition_range(p, P, b, part);
    if (R.n == 0) {
        if (part == 0) zero_output<QDT, D, GS>(p, b, hq0);
        return;
    }
    if (part >= R.nparts) return;

    // B operand: head c (zero beyond GS), for step s dims 8 (4 s + r) .. +7, or
    // for INT8 keys 32 r + 8 s .. +7 (a lane then reads its keys as two 16-byte
    // runs).  Q.K^T sums over all dims either way.
    constexpr bool KRUN = KDT == DT_INT8;
    MT qb[KS];
    {
        const uint16_t* q16 = reinterpret_cast<const uint16_t*>(p.q);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            const int d0 = KRUN ? 32 * r + 8 * s : 8 * (4 * s + r);
            if (c < GS)
                raw = *reinterpret_cast<const uint4*>(q16 + ((int64_t)b * p.H_q + hq0 + c) * D + d0);
            qb[s] = __builtin_bit_cast(MT, raw);
        }
    }
    float qscale = p.scale * kLog2e;
    if constexpr (KDT == DT_FP8) qscale *= p.k_scale[g];
    // INT8 pools: <q, key> = min * sum(q) + step * <q, codes> (sum over the head,
    // taken once); the values' min term is kept apart per stream (mv_run).
    constexpr bool I8 = KDT == DT_INT8;
    float qsum = 0.0f, mv_run = 0.0f;
    if constexpr (I8) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) qsum += (float)qb[s][e];
        qsum += __shfl_xor(qsum, 16, 64);
        qsum += __shfl_xor(qsum, 32, 64);
    }

    float m_run = -INFINITY, l_run = 0.0f;   // stream (row r, head c)
    float acc[GS][8];
#pragma unroll
    for (int h = 0; h < GS; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;

    const int32_t* table = p.tables + (int64_t)b * p.max_blocks;
    const char* kbase = reinterpret_cast<const char*>(p.k_pool);
    const char* vbase = reinterpret_cast<const char*>(p.v_pool);
    // a block holds the codes of every KV head, then (INT8) their headers
    const int64_t head_off = (int64_t)g * TL::BYTES;
    const int64_t blk_stride = (int64_t)p.H_kv * TL::STRIDE;
    const int64_t hdr_off = (int64_t)p.H_kv * TL::BYTES + kInt8HeaderBytes * g;
    // K: token c, step s -> bytes KW (4 s + r), or 32 r + 8 s for INT8;
    // V: token 4 r + i, bytes KW c.
    const int k_off = c * TL::ROW + (KRUN ? 32 * r : r * TL::KW);
    const int v_off = (4 * r) * TL::ROW + c * TL::KW;
    const int blk0 = R.blk_first + wave;
    const int nmine = blk0 < R.blk_last ? (R.blk_last - blk0 + kDecodeWaves - 1) / kDecodeWaves : 0;
    WaveTable wt;
    wt.load(table, blk0, nmine, 0, lane);

    struct Buf {
        KRaw k[KS];
        KRaw v[4];
        float4 kh, vh;                   // INT8: tile headers {min, max, step, 0}
        bool ok;
    };
    auto fetch = [&](int j, Buf& B) {
        if ((j & 63) == 0 && j > 0) wt.load(table, blk0, nmine, j, lane);
        const int phys = wt.phys(j);
        B.ok = phys >= 0 && phys < p.num_blocks;
        if (!B.ok) return;
        const int64_t blk_base = (int64_t)phys * blk_stride;
        const int64_t off = blk_base + head_off;
        if constexpr (KRUN) {
#pragma unroll
            for (int s2 = 0; s2 < KS / 2; ++s2) {
                const uint4 w = load_kv<uint4>(kbase + off + k_off + 16 * s2);
                B.k[2 * s2] = make_uint2(w.x, w.y);
                B.k[2 * s2 + 1] = make_uint2(w.z, w.w);
            }
        } else {
#pragma unroll
            for (int s = 0; s < KS; ++s) B.k[s] = load_kv<KRaw, TL::KW == 16>(kbase + off + k_off + s * 4 * TL::KW);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) B.v[i] = load_kv<KRaw>(vbase + off + v_off + i * TL::ROW);
        if constexpr (I8) {
            B.kh = *reinterpret_cast<const float4*>(kbase + blk_base + hdr_off);
            B.vh = *reinterpret_cast<const float4*>(vbase + blk_base + hdr_off);
        }
    };
    auto update = [&](auto masked, int blk, const Buf& B) {
        constexpr bool MASKED = decltype(masked)::value;
        f32x4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            MT a;
            if constexpr (KDT == DT_FP8) a = fp8x8_to_mfma<QDT>(B.k[s]);
            else if constexpr (I8) a = u8x8_to_mfma<QDT>(B.k[s]);
            else a = __builtin_bit_cast(MT, B.k[s]);
            S = mfma16x16x32<QDT>(a, qb[s], S);
        }
        const int tok = blk * kBlock + 4 * r;           // token of S[0] in this lane
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (I8) z[i] = fmaf(B.kh.z, S[i], B.kh.x * qsum) * qscale;
            else z[i] = S[i] * qscale;
            if (MASKED && tok + i >= R.pend) z[i] = -INFINITY;
        }
        const float m_new = fmaxf(fmaxf(m_run, fmaxf(z[0], z[1])), fmaxf(z[2], z[3]));
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(z[i] - m_use);
        l_run = fmaf(l_run, alpha, (pr[0] + pr[1]) + (pr[2] + pr[3]));
        if constexpr (I8) mv_run = fmaf(mv_run, alpha, B.vh.x * ((pr[0] + pr[1]) + (pr[2] + pr[3])));
        m_run = m_new;
        // rescale the accumulators of every stream whose max moved
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f && c < GS) != 0) {
#pragma unroll
            for (int h = 0; h < GS; ++h) {
                const float ah = row_bcast(alpha, h);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= ah;
            }
        }
        if constexpr (KDT != DT_FP8) {
            // 16-bit values: widen to fp32, one FMA per (head, dim, token)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float vf[8];
                widen<KDT, TL::KW>(B.v[i], vf);
                if (MASKED && tok + i >= R.pend) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) vf[e] = 0.0f;   // select, never 0 * garbage
                }
#pragma unroll
                for (int h = 0; h < GS; ++h) {
                    float ph = row_bcast(pr[i], h);
                    if constexpr (I8) ph *= B.vh.z;          // value = min + step * code
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
                }
            }
        } else {
            // E4M3 values: two tokens per v_dot2_f32_f16.  The codes of tokens
            // (4r, 4r+1) at one dim are paired with v_perm_b32 and widened exactly
            // to f16; their weights travel as one f16 pair per head (relative
            // rounding 2^-11 on a weight, far inside the FP8 tolerance).
            const uint32_t pp[2] = {pack_f16x2(pr[0], pr[1]), pack_f16x2(pr[2], pr[3])};
#pragma unroll
            for (int pi = 0; pi < 2; ++pi) {
                uint32_t vp[8];
                fp8_token_pairs(B.v[2 * pi], B.v[2 * pi + 1], vp);
                if (MASKED) {
                    const uint32_t keep = (tok + 2 * pi < R.pend ? 0x0000FFFFu : 0u) |
                                          (tok + 2 * pi + 1 < R.pend ? 0xFFFF0000u : 0u);
#pragma unroll
                    for (int e = 0; e < 8; ++e) vp[e] &= keep;       // select, never 0 * garbage
                }
#pragma unroll
                for (int h = 0; h < GS; ++h) {
                    const f16x2_t wh = __builtin_bit_cast(f16x2_t, row_bcast_u32(pp[pi], h));
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[h][e] = __builtin_amdgcn_fdot2(wh, __builtin_bit_cast(f16x2_t, vp[e]), acc[h][e], false);
                }
            }
        }
    };
    auto consume = [&](int j, const Buf& B) {
        if (!B.ok) return;
        const int blk = blk0 + kDecodeWaves * j;
        if (blk * kBlock + kBlock > R.pend) update(std::integral_constant<bool, true>{}, blk, B);
        else update(std::integral_constant<bool, false>{}, blk, B);
    };
    pipeline<2, Buf>(nmine, fetch, consume);

    // Merge the 16 streams (4 waves x 4 rows) of each head through LDS.
    const int srow = wave * 4 + r;
    if (c < GS) {
        s_m[srow][c] = m_run;
        s_l[srow][c] = l_run;
    }
#pragma unroll
    for (int h = 0; h < GS; ++h) {
        const float mh = I8 ? row_bcast(mv_run, h) : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s_o[srow][h][c * 8 + e] = acc[h][e] + mh;
    }
    __syncthreads();
    float vscale = 1.0f;
    if constexpr (KDT == DT_FP8) vscale = p.v_scale[g];
    merge_streams<QDT, D, GS, NS>(p, s_m, s_l, s_o, b, hq0, part, R.nparts == 1, vscale);
}

template <int KDT, int QDT, int GS>
// Groups up to 5 fit 3 waves per SIMD without spilling; larger ones take 2.
__global__ __launch_bounds__(kDecodeWaves * 64) __attribute__((amdgpu_waves_per_eu(GS <= 5 ? 3 : 2)))
void paged_decode_partition_gqa(DecodeParams p) {
    __shared__ StreamSmem<kDecodeWaves * 4, GS, 128> sm;
    for_each_item(p, [&](int b, int part, int hgi, int P) { gqa_item<KDT, QDT, GS>(p, b, part, hgi, P, sm); });
}

// Wave-wide max / sum; every lane gets the same value (fixed butterfly order).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float lane_bcast(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Kernel 2: merge the partitions of one (sequence, query head) with the same
// rule as the in-workgroup merge: M = max m_t, L = sum l_t 2^(m_t - M),
// out = sum o_t 2^(m_t - M) / L.  Sequences that fit one partition were
// finished by kernel 1 and are skipped here.  Lane t handles partition t's
// (m, l) (64 partitions per sweep); the weights are broadcast from their lanes
// while every lane accumulates its own output dims, so the partial-output
// loads are independent of each other.
template <int QDT, int D>
__global__ __launch_bounds__(64) void paged_decode_reduce(DecodeParams p) {
    constexpr int DPL = D >= 64 ? D / 64 : 1;      // output dims per lane
    const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int nparts = num_parts(part_tokens(p), clamped_len(p, b));
    if (nparts <= 1) return;
    const int64_t base = ((int64_t)b * p.H_q + hq) * p.max_parts;
    const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + base;
    const float* po = p.ws_o + base * D;
    const bool live = D >= 64 || lane < D;

    // Up to kFewParts partitions: every partial output is loaded before the
    // max is known, so those loads overlap the (m, l) load and the two wave
    // reductions instead of waiting for them.  Same operations in the same
    // order as the general loop below, so the same bits.
    constexpr int kFewParts = 16;
    if (nparts <= kFewParts) {
        float ov[kFewParts][DPL];
#pragma unroll
        for (int t = 0; t < kFewParts; ++t)
#pragma unroll
            for (int i = 0; i < DPL; ++i) ov[t][i] = t < nparts && live ? po[(int64_t)t * D + lane + 64 * i] : 0.0f;
        const float2 v = lane < nparts ? ml[lane] : make_float2(-INFINITY, 0.0f);
        const float M = wave_max(v.x);
        float L = 0.0f, o[DPL];
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[i] = 0.0f;
        if (M != -INFINITY) {
            const float w = lane < nparts ? fast_exp2(v.x - M) : 0.0f;
            if (lane < nparts) L = fmaf(v.y, w, L);
#pragma unroll
            for (int t = 0; t < kFewParts; ++t) {
                if (t < nparts) {
                    const float wt = lane_bcast(w, t);
#pragma unroll
                    for (int i = 0; i < DPL; ++i) o[i] = fmaf(ov[t][i], wt, o[i]);
                }
            }
        }
        L = wave_sum(L);
        if (live) {
#pragma unroll
            for (int i = 0; i < DPL; ++i)
                store_out<QDT>(p.out, ((int64_t)b * p.H_q + hq) * D + lane + 64 * i, L > 0.0f ? o[i] / L : 0.0f);
        }
        return;
    }

    float M = -INFINITY;
    for (int t0 = 0; t0 < nparts; t0 += 64)
        if (t0 + lane < nparts) M = fmaxf(M, ml[t0 + lane].x);
    M = wave_max(M);

    float L = 0.0f, o[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] = 0.0f;
    if (M != -INFINITY) {
        for (int t0 = 0; t0 < nparts; t0 += 64) {
            const int t = t0 + lane;
            float w = 0.0f;
            if (t < nparts) {
                const float2 v = ml[t];
                w = fast_exp2(v.x - M);
                L = fmaf(v.y, w, L);
            }
            const int cnt = min(64, nparts - t0);
#pragma unroll 8
            for (int j = 0; j < cnt; ++j) {
                const float wj = lane_bcast(w, j);
                const float* src = po + (int64_t)(t0 + j) * D;
                if (live) {
#pragma unroll
                    for (int i = 0; i < DPL; ++i) o[i] = fmaf(src[lane + 64 * i], wj, o[i]);
                }
            }
        }
    }
    L = wave_sum(L);
    if (live) {
#pragma unroll
        for (int i = 0; i < DPL; ++i)
            store_out<QDT>(p.out, ((int64_t)b * p.H_q + hq) * D + lane + 64 * i, L > 0.0f ? o[i] / L : 0.0f);
    }
}

using KernelFn = void (*)(DecodeParams);

template <int KDT, int QDT, int D>
KernelFn pick_gs(int gs) {
    // groups >= 3 at head_dim 128 with 16-bit / FP8 storage always take the
    // matrix-core variant; do not instantiate vector kernels for them
    constexpr bool kGqaCovers = D == 128 && KDT != DT_F32;
    if (kGqaCovers && gs >= 3) return nullptr;
    switch (gs) {
        case 1: return paged_decode_partition<KDT, QDT, D, 1>;
        case 2: return paged_decode_partition<KDT, QDT, D, 2>;
        default: break;
    }
    if constexpr (!kGqaCovers) {
        switch (gs) {
            case 3: return paged_decode_partition<KDT, QDT, D, 3>;
            case 4: return paged_decode_partition<KDT, QDT, D, 4>;
            case 5: return paged_decode_partition<KDT, QDT, D, 5>;
            case 6: return paged_decode_partition<KDT, QDT, D, 6>;
            case 7: return paged_decode_partition<KDT, QDT, D, 7>;
            case 8: return paged_decode_partition<KDT, QDT, D, 8>;
            default: return nullptr;
        }
    }
    return nullptr;
}

template <int KDT, int QDT>
KernelFn pick_d(int D, int gs) {
    switch (D) {
        case 16: return pick_gs<KDT, QDT, 16>(gs);
        case 64: return pick_gs<KDT, QDT, 64>(gs);
        case 128: return pick_gs<KDT, QDT, 128>(gs);
        default: return nullptr;
    }
}

KernelFn pick_vector(int kdt, int qdt, int D, int gs);

template <int KDT, int QDT>
KernelFn pick_gqa(int gs) {
    switch (gs) {
        case 3: return paged_decode_partition_gqa<KDT, QDT, 3>;
        case 4: return paged_decode_partition_gqa<KDT, QDT, 4>;
        case 5: return paged_decode_partition_gqa<KDT, QDT, 5>;
        case 6: return paged_decode_partition_gqa<KDT, QDT, 6>;
        case 7: return paged_decode_partition_gqa<KDT, QDT, 7>;
        case 8: return paged_decode_partition_gqa<KDT, QDT, 8>;
        default: return nullptr;
    }
}

// Grouped heads with 128-dim heads and 16-bit / FP8 storage take the matrix-core
// variant; everything else the vector variant.
KernelFn pick_partition(int kdt, int qdt, int D, int gs) {
    if (D == 128 && gs >= 3) {
        if (kdt == DT_F16 && qdt == DT_F16) return pick_gqa<DT_F16, DT_F16>(gs);
        if (kdt == DT_BF16 && qdt == DT_BF16) return pick_gqa<DT_BF16, DT_BF16>(gs);
        if (kdt == DT_FP8 && qdt == DT_BF16) return pick_gqa<DT_FP8, DT_BF16>(gs);
        if (kdt == DT_FP8 && qdt == DT_F16) return pick_gqa<DT_FP8, DT_F16>(gs);
        if (kdt == DT_INT8 && qdt == DT_BF16) return pick_gqa<DT_INT8, DT_BF16>(gs);
        if (kdt == DT_INT8 && qdt == DT_F16) return pick_gqa<DT_INT8, DT_F16>(gs);
    }
    return pick_vector(kdt, qdt, D, gs);
}

KernelFn pick_vector(int kdt, int qdt, int D, int gs) {
    if (kdt == DT_F32 && qdt == DT_F32) return pick_d<DT_F32, DT_F32>(D, gs);
    if (kdt == DT_F16 && qdt == DT_F16) return pick_d<DT_F16, DT_F16>(D, gs);
    if (kdt == DT_BF16 && qdt == DT_BF16) return pick_d<DT_BF16, DT_BF16>(D, gs);
    if (kdt == DT_FP8 && qdt == DT_BF16) return pick_d<DT_FP8, DT_BF16>(D, gs);
    if (kdt == DT_FP8 && qdt == DT_F16) return pick_d<DT_FP8, DT_F16>(D, gs);
    if (kdt == DT_INT8 && qdt == DT_BF16) return pick_d<DT_INT8, DT_BF16>(D, gs);
    if (kdt == DT_INT8 && qdt == DT_F16) return pick_d<DT_INT8, DT_F16>(D, gs);
    return nullptr;
}

template <int QDT>
KernelFn pick_reduce_d(int D) {
    switch (D) {
        case 16: return paged_decode_reduce<QDT, 16>;
        case 64: return paged_decode_reduce<QDT, 64>;
        case 128: return paged_decode_reduce<QDT, 128>;
        default: return nullptr;
    }
}

KernelFn pick_reduce(int qdt, int D) {
    switch (qdt) {
        case DT_F32: return pick_reduce_d<DT_F32>(D);
        case DT_F16: return pick_reduce_d<DT_F16>(D);
        case DT_BF16: return pick_reduce_d<DT_BF16>(D);
        default: return nullptr;
    }
}

}  // namespace

int decode_heads_per_wg(int32_t G) {
    if (G <= kMaxGroupPerWg) return G;
    for (int gs = kMaxGroupPerWg; gs >= 1; --gs)
        if (G % gs == 0) return gs;
    return 1;
}

bool decode_supported(int32_t kv_dt, int32_t q_dt, int32_t D, int32_t G) {
    if (G < 1) return false;
    return pick_partition(kv_dt, q_dt, D, decode_heads_per_wg(G)) != nullptr &&
           pick_reduce(q_dt, D) != nullptr;
}

// Workgroups of `fn` that fit on the device at once (cached per kernel).
int resident_workgroups(KernelFn fn) {
    static std::mutex mu;
    static std::unordered_map<const void*, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(reinterpret_cast<const void*>(fn));
    if (it != cache.end()) return it->second;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn),
                                                     kDecodeWaves * 64, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0)
        return 1024;   // not cached: a later call retries the query
    cache[reinterpret_cast<const void*>(fn)] = cus * per_cu;
    return cus * per_cu;
}

int decode_resident_workgroups(int32_t kv_dt, int32_t q_dt, int32_t D, int32_t G) {
    KernelFn fn = pick_partition(kv_dt, q_dt, D, decode_heads_per_wg(G));
    return fn ? resident_workgroups(fn) : 0;
}

hipError_t noalloc_scratch(int device, void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};       // per device, filled on first use (no host allocation)
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device) return hipErrorInvalidDevice;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[device] = p;
    }
    *ptr = addr[device];
    return hipSuccess;
}

hipError_t launch_decode_plan(const DecodeParams& p, hipStream_t stream) {
    DecodeParams arg = p;
    void* args[] = {&arg};
    return launch_kernel(reinterpret_cast<const void*>(paged_decode_plan), dim3(1), dim3(kPlanThreads), args, 0,
                           stream);
}

hipError_t launch_decode_partition(const DecodeParams& p, hipStream_t stream) {
    const int gs = decode_heads_per_wg(p.G);
    KernelFn fn = pick_partition(p.kv_dt, p.q_dt, p.D, gs);
    if (!fn) return hipErrorInvalidValue;
    dim3 grid;
    if (p.items) {
        grid = dim3((unsigned)p.grid_wgs);
    } else {
        grid = dim3((unsigned)p.max_parts, (unsigned)p.head_groups, (unsigned)p.B);
    }
    DecodeParams arg = p;
    void* args[] = {&arg};
    return launch_kernel(reinterpret_cast<const void*>(fn), grid, dim3(kDecodeWaves * 64), args, 0, stream);
}

hipError_t launch_decode_reduce(const DecodeParams& p, hipStream_t stream) {
    KernelFn fn = pick_reduce(p.q_dt, p.D);
    if (!fn) return hipErrorInvalidValue;
    DecodeParams arg = p;
    void* args[] = {&arg};
    return launch_kernel(reinterpret_cast<const void*>(fn), dim3((unsigned)p.H_q, (unsigned)p.B),
                           dim3(64), args, 0, stream);
}

}  // namespace pkv
