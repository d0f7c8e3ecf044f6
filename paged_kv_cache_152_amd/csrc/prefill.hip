// paged_prefill: a chunk of query tokens per sequence attending, through the
// block table, to the cached context and to itself (the prefill stage of
// www.mlqm.cn/news/394450 section 三, chunked as in its section 七; block
// table of www.cf-1.com/news/5824798 §3.1).  Unlike single-token decode this
// is a dense contraction on both sides, so both products run on the matrix
// cores.
//
// Work split.  A workgroup of 4 waves takes one (query tile, head group,
// sequence); the workgroups of one (sequence, head group) are placed on one XCD
// so its L2 serves their repeated reads of the same K/V.  A wave owns 32 query
// rows in two groups of 16: tw = 32 / gs query tokens times the gs query heads
// of one KV head group (row = token * gs + head; rows beyond tw * gs are
// padding).  The four waves walk the same 16-token blocks of the context.
// Each thread moves 1/256 of a block's K and V tile from HBM into registers
// four blocks ahead of use, then into LDS: K as it is stored ([token][dim],
// rows padded against bank conflicts), V transposed ([dim][token]).  Block ids
// come from a per-wave register of 64 table entries.
//
// Per block, with m = 16 tokens, for each row group:
//   S^T = K . Q^T    4 (head_dim 128) or 2 (64) v_mfma_f32_16x16x32: A = the K
//                    tile (lane: token l % 16, 8 dims) from LDS, shared by the
//                    row groups; B = 16 query rows (lane: row l % 16, 8 dims),
//                    held in registers for the whole walk.  Lane l ends with
//                    the logits of tokens 4 (l / 16) .. +3 for row l % 16.
//   online softmax   the running max / sum of a row live in the four lanes
//                    l % 16 = row; two cross-row shuffles per block.  Logits
//                    are in base 2 (exp2), q's scale folded in.
//   O^T += V^T . P^T head_dim / 16 v_mfma_f32_16x16x16: B = P^T, which is
//                    exactly the layout S^T left in the lanes (packed to
//                    16-bit), A = V^T from LDS, shared by the row groups.
// Lane l accumulates output dims 16 mt + 4 (l / 16) + i of row l % 16 of each
// group, so the rescale when a row's max moves is one multiply per
// accumulator.
//
// FP8 pools: K codes are widened exactly to q's 16-bit type for Q.K^T; V codes
// to f16 (exact) for P.V, with P in f16.  The K scale folds into the logit
// scale, the V scale multiplies the output.  Tokens past the context, and
// blocks whose table entry lies outside the pool, are masked by selection and
// their V rows are zeroed in LDS, so no stored garbage reaches the result.
#include "internal.h"

#include <type_traits>

namespace pkv {
namespace {

constexpr int kPfWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

template <int T> struct Vec8;
template <> struct Vec8<DT_BF16> { using T = bf16x8_t; };
template <> struct Vec8<DT_F16> { using T = f16x8_t; };

// S^T step: 16 tokens x 16 rows, 32 dims.
template <int QT>
__device__ __forceinline__ f32x4_t mma_k32(const typename Vec8<QT>::T& a, const typename Vec8<QT>::T& b,
                                           f32x4_t c) {
    if constexpr (QT == DT_BF16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// O^T step: 16 dims x 16 rows, 16 tokens; operands are four 16-bit values.
template <int PT>
__device__ __forceinline__ f32x4_t mma_k16(uint2 a, uint2 b, f32x4_t c) {
    if constexpr (PT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                         __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// Two fp32 -> two 16-bit values of type PT (round to nearest even), packed.
template <int PT>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
    const f32x2_t v = {x, y};
    if constexpr (PT == DT_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// The sum of the two 16-bit values of type PT packed in w, in fp32 (exact widening).
template <int PT>
__device__ __forceinline__ float sum2(uint32_t w) {
    if constexpr (PT == DT_BF16)
        return __builtin_bit_cast(float, w << 16) + __builtin_bit_cast(float, w & 0xffff0000u);
    else {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, w);
        return (float)h[0] + (float)h[1];
    }
}

// 8 E4M3 codes -> 8 values of 16-bit type T, exact.
template <int T>
__device__ __forceinline__ uint4 fp8x8_to(uint2 w) {
    uint32_t o[4];
    if constexpr (T == DT_BF16) {
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
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int QT>
__device__ __forceinline__ uint16_t to_q16(float x) {
    if constexpr (QT == DT_BF16) return bf16_rne(x);
    else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Lane-pair max / sum across the four lanes of a row (l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float across_rows_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float across_rows_sum(float v) {
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
}

// Rows per wave: kRowGroups groups of 16; tiles of K / V staged NR blocks ahead.
constexpr int kRowGroups = 2;
constexpr int kAhead = 4;

// Workgroups of one (sequence, head group) walk the same K/V; keep them on one
// XCD (workgroups are dealt round-robin over the 8 XCDs), so its L2 serves the
// repeats.  Logical index = xcd * (n / 8) + position on that XCD.  Within a
// (sequence, head group) the query tiles go last to first: under the causal
// mask a later tile sees more keys, so the longest workgroups start first and
// the shortest fill the end of the launch (4% shorter launch on a 16 x 512-token
// chunk workload than first to last).
__device__ __forceinline__ int64_t xcd_logical(int64_t i, int64_t n) {
    const int64_t full = n - n % 8;
    if (i >= full) return i;
    return (i % 8) * (full / 8) + i / 8;
}

template <int KDT, int QDT, int D>
__global__ __launch_bounds__(kPfWaves * 64) void paged_prefill_kernel(PrefillParams p) {
    constexpr int KS = D / 32;                 // S^T steps (32 dims each)
    constexpr int MT = D / 16;                 // O^T m-tiles (16 dims each)
    constexpr int R = kRowGroups;
    constexpr int PT = KDT == DT_BF16 ? DT_BF16 : DT_F16;   // type of P and V in P.V
    constexpr int KT = KDT == DT_FP8 ? QDT : KDT;            // type of K in Q.K^T
    constexpr int KE = KDT == DT_FP8 ? 1 : 2;  // bytes per stored K/V element
    constexpr int EPL = D / 16;                // elements of a tile one thread stages (16 threads a token)
    constexpr int KROW = D + 8;                // LDS row of a K or V tile, padded (16-bit elements)
    constexpr float kLazy = 8.0f;              // a row's reference max moves only when exceeded by 2^8
    using QV = typename Vec8<QDT>::T;
    __shared__ __align__(16) uint16_t ks_lds[2][16 * KROW];
    __shared__ __align__(16) uint16_t vs_lds[2][16 * KROW];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane >> 4, c = lane & 15;
    const int gs = p.gs, subs = p.G / gs;
    const int tw = (16 * R) / gs;                            // query tokens per wave
    const int64_t tiles = p.tiles;
    const int64_t n_wg = tiles * p.H_kv * subs * p.n_seqs;
    const int64_t L = xcd_logical(blockIdx.x, n_wg);
    const int tile = (int)(tiles - 1 - L % tiles);          // latest (heaviest under the causal mask) first
    const int hgi = (int)((L / tiles) % ((int64_t)p.H_kv * subs));
    const int s = (int)(L / (tiles * p.H_kv * subs));
    const int g = hgi / subs;
    const int hq0 = g * p.G + (hgi % subs) * gs;

    const int q0 = min(p.q_start[s], p.total_q), q1 = min(max(p.q_start[s + 1], q0), p.total_q);
    const int q_len = q1 - q0;
    int n = p.lens[s];
    n = n < 0 ? 0 : (n > p.max_blocks * kBlock ? p.max_blocks * kBlock : n);
    const int tile0 = tile * kPfWaves * tw;                 // first query token of the workgroup
    if (tile0 >= q_len) return;
    const int tile_last = min(q_len, tile0 + kPfWaves * tw) - 1;
    const int wg_see = p.causal ? n - q_len + tile_last : n - 1;
    const int nblk = wg_see < 0 ? 0 : min((wg_see + kBlock) / kBlock, (n + kBlock - 1) / kBlock);

    // this lane's query rows: group rg holds row rg * 16 + c of the wave
    int i_row[R], see[R];
    bool live[R];
    QV qb[R][KS];
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        const int row = rg * 16 + c;
        i_row[rg] = tile0 + wave * tw + row / gs;
        live[rg] = row < tw * gs && i_row[rg] < q_len;
        const int pos = n - q_len + i_row[rg];
        see[rg] = p.causal ? pos : n - 1;
        const int64_t qrow = ((int64_t)(q0 + i_row[rg]) * p.H_q + hq0 + row % gs) * D;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            if (live[rg]) raw = *reinterpret_cast<const uint4*>(q16 + qrow + 32 * k + 8 * r);
            qb[rg][k] = __builtin_bit_cast(QV, raw);
        }
    }
    float qscale = p.scale * kLog2e;
    float vscale = 1.0f;
    if constexpr (KDT == DT_FP8) {
        qscale *= p.k_scale[g];
        vscale = p.v_scale[g];
    }

    const int32_t* table = p.tables + (int64_t)s * p.max_blocks;
    const char* kbase = reinterpret_cast<const char*>(p.k_pool);
    const char* vbase = reinterpret_cast<const char*>(p.v_pool);
    constexpr int ROW = D * KE;
    constexpr int TILE = kBlock * ROW;
    const int64_t blk_stride = (int64_t)p.H_kv * TILE;
    const int64_t head_off = (int64_t)g * TILE;
    // staging: thread tid moves token tid / 16, elements EPL (tid % 16) .. +EPL-1 of the K and V tiles
    const int st_tok = tid >> 4, st_el = (tid & 15) * EPL;
    const int st_off = st_tok * ROW + st_el * KE;
    using Raw = std::conditional_t<EPL * KE == 16, uint4, std::conditional_t<EPL * KE == 8, uint2, uint32_t>>;
    struct Stage {
        Raw k, v;
        bool ok;
    };
    int tv = -1;                               // table entries of blocks 64 t .. 64 t + 63, one per lane
    int tv_base = -64;
    auto fetch = [&](int j, Stage& st) {
        if (j - tv_base >= 64) {               // uniform: every lane walks the same j
            tv_base = j & ~63;
            tv = tv_base + lane < nblk ? table[tv_base + lane] : -1;
        }
        const int phys = __builtin_amdgcn_readlane(tv, j & 63);
        st.ok = phys >= 0 && phys < p.num_blocks;
        if (!st.ok) return;
        const int64_t off = (int64_t)phys * blk_stride + head_off + st_off;
        st.k = *reinterpret_cast<const Raw*>(kbase + off);
        st.v = *reinterpret_cast<const Raw*>(vbase + off);
    };
    // K tile in K's MFMA type, V tile in PT, both [token][dim] as stored; dead rows zero
    auto stage = [&](int j, const Stage& st, int buf) {
        const bool ok = st.ok && j * kBlock + st_tok < n;
        uint16_t* kd = &ks_lds[buf][st_tok * KROW + st_el];
        uint16_t* vd = &vs_lds[buf][st_tok * KROW + st_el];
        if constexpr (KDT == DT_FP8) {
            if constexpr (EPL == 8) {
                uint4 kw = fp8x8_to<KT>(*reinterpret_cast<const uint2*>(&st.k));
                uint4 vw = fp8x8_to<DT_F16>(*reinterpret_cast<const uint2*>(&st.v));
                if (!ok) kw = vw = make_uint4(0u, 0u, 0u, 0u);
                *reinterpret_cast<uint4*>(kd) = kw;
                *reinterpret_cast<uint4*>(vd) = vw;
            } else {
                const uint32_t kc = *reinterpret_cast<const uint32_t*>(&st.k);
                const uint32_t vc = *reinterpret_cast<const uint32_t*>(&st.v);
                uint2 kw, vw;
                if constexpr (KT == DT_BF16) {
                    kw.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kc, 1.0f, false));
                    kw.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kc, 1.0f, true));
                } else {
                    kw.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(kc, 1.0f, false));
                    kw.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(kc, 1.0f, true));
                }
                vw.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vc, 1.0f, false));
                vw.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vc, 1.0f, true));
                if (!ok) kw = vw = make_uint2(0u, 0u);
                *reinterpret_cast<uint2*>(kd) = kw;
                *reinterpret_cast<uint2*>(vd) = vw;
            }
        } else {
            constexpr int NW = sizeof(Raw) / 4;
            const uint32_t* kw = reinterpret_cast<const uint32_t*>(&st.k);
            const uint32_t* vw = reinterpret_cast<const uint32_t*>(&st.v);
            uint32_t kz[NW], vz[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                kz[w] = ok ? kw[w] : 0u;
                vz[w] = ok ? vw[w] : 0u;
            }
            if constexpr (NW == 4) {
                *reinterpret_cast<uint4*>(kd) = make_uint4(kz[0], kz[1], kz[2], kz[3]);
                *reinterpret_cast<uint4*>(vd) = make_uint4(vz[0], vz[1], vz[2], vz[3]);
            } else {
                *reinterpret_cast<uint2*>(kd) = make_uint2(kz[0], kz[1]);
                *reinterpret_cast<uint2*>(vd) = make_uint2(vz[0], vz[1]);
            }
        }
    };

    f32x4_t acc[R][MT];
    float m_run[R], l_run[R];
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        m_run[rg] = -INFINITY;
        l_run[rg] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rg][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // Rows keep a reference max m_ref that moves only when a logit exceeds it
    // by more than 2^kLazy: the weights exp2(z - m_ref) stay <= 2^kLazy (exact
    // in fp32, the same relative precision in 16-bit), and the accumulators are
    // rescaled only on those moves.  A block every live row sees in full takes
    // the unmasked path.
    const int wg_min_see = p.causal ? n - q_len + tile0 : n - 1;
    auto compute = [&](bool masked, int j, int buf) {
        // K operand (token c, dims 32 k + 8 r), shared by the row groups
        typename Vec8<KT>::T ka[KS];
#pragma unroll
        for (int k = 0; k < KS; ++k)
            ka[k] = *reinterpret_cast<const typename Vec8<KT>::T*>(&ks_lds[buf][c * KROW + 32 * k + 8 * r]);
        const int tok = j * kBlock + 4 * r;
        uint2 pb[R];
#pragma unroll
        for (int rg = 0; rg < R; ++rg) {
            f32x4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < KS; ++k) S = mma_k32<QDT>(__builtin_bit_cast(QV, ka[k]), qb[rg][k], S);
            float z[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool vis = live[rg] && (!masked || (tok + i < n && tok + i <= see[rg]));
                z[i] = vis ? S[i] * qscale : -INFINITY;      // select, never 0 * garbage
            }
            const float m_blk = across_rows_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
            if (__builtin_amdgcn_ballot_w64(m_blk > m_run[rg] + kLazy) != 0) {
                const float m_new = m_blk > m_run[rg] + kLazy ? m_blk : m_run[rg];
                const float alpha = m_new == m_run[rg] ? 1.0f : __builtin_amdgcn_exp2f(m_run[rg] - m_new);
                l_run[rg] *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[rg][mt] *= alpha;
                m_run[rg] = m_new;
            }
            const float m_use = m_run[rg] == -INFINITY ? 0.0f : m_run[rg];
            float pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(z[i] - m_use);
            // l sums the rounded weights P.V multiplies, so the output is a normalised
            // average of those weights and a row's dominant weight carries no rounding
            pb[rg] = make_uint2(pack2<PT>(pr[0], pr[1]), pack2<PT>(pr[2], pr[3]));
            l_run[rg] += across_rows_sum(sum2<PT>(pb[rg].x) + sum2<PT>(pb[rg].y));
        }
        // V^T operand: dim 16 mt + c, tokens 4 r .. 4 r + 3.  ds_read_b64_tr_b16
        // builds, in each 16-lane group, row k from the 4 elements lanes 4k ..
        // 4k + 3 point at and hands lane i element i of rows 0 .. 3; so lane
        // (r, c) points at token 4 r + c / 4, dims 16 mt + 4 (c % 4) .. + 3.
        const uint16_t* vsrc = &vs_lds[buf][(4 * r + (c >> 2)) * KROW + 4 * (c & 3)];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint2 va = __builtin_bit_cast(
                uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (__attribute__((address_space(3))) s16x4_t*)(vsrc + 16 * mt)));
#pragma unroll
            for (int rg = 0; rg < R; ++rg) acc[rg][mt] = mma_k16<PT>(va, pb[rg], acc[rg][mt]);
        }
    };

    // register ring of kAhead blocks in flight; LDS double buffer for the block in use
    Stage ring[kAhead];
#pragma unroll
    for (int k = 0; k < kAhead; ++k)
        if (k < nblk) fetch(k, ring[k]);
    for (int j0 = 0; j0 < nblk; j0 += kAhead) {
#pragma unroll
        for (int k = 0; k < kAhead; ++k) {
            const int j = j0 + k;
            if (j < nblk) {
                stage(j, ring[k], j & 1);
                if (j + kAhead < nblk) fetch(j + kAhead, ring[k]);
                __syncthreads();                             // tiles of block j are in LDS
                compute(!((j + 1) * kBlock <= n && j * kBlock + kBlock - 1 <= wg_min_see), j, j & 1);
            }
        }
    }

    uint16_t* o16 = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        if (!live[rg]) continue;
        const int row = rg * 16 + c;
        const float inv = l_run[rg] > 0.0f ? vscale / l_run[rg] : 0.0f;
        const int64_t orow = ((int64_t)(q0 + i_row[rg]) * p.H_q + hq0 + row % gs) * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            uint16_t e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = to_q16<QDT>(acc[rg][mt][i] * inv);
            *reinterpret_cast<uint2*>(o16 + orow + 16 * mt + 4 * r) =
                make_uint2((uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16));
        }
    }
}

// ---------------------------------------------------------------------------
// 16-bit pools (and E4M3 at head_dim 128): K and V go from HBM straight into
// LDS (global_load_lds_dwordx4, no registers on the way), in kStages LDS
// buffers of one 32-token stage (two blocks) each: while a wave computes one
// stage, the next three are landing, and one wait plus one barrier per stage
// hands the next one over.  The compute is software-pipelined one stage deep
// (S^T of stage j + 1 runs on the matrix cores while the weights of stage j
// are taken on the vector ALUs; see the stage loop).  A stage row is one
// token's head_dim values; its 16-byte chunks are
// XOR-swizzled by row so that the K-operand reads (16 rows, one chunk each)
// and the transposed V reads (4 rows x 32 bytes per 16 lanes) hit distinct
// banks.  Tokens past the context and blocks outside the pool load from a
// zero tile instead, so no stored garbage reaches P.V.
//
// Per 32-token stage, for each row group: S^T of the two blocks on
// 2 x head_dim / 32 v_mfma_f32_16x16x32; the lane then holds the weights of
// tokens 4 (l / 16) .. +3 of both blocks for row l % 16, which is the B layout
// of a 16x16x32 product with k = 8 (l / 16) + i standing for those 8 tokens.
// O^T += V^T . P^T on head_dim / 16 v_mfma_f32_16x16x32, A built from two
// ds_read_b64_tr_b16 (one per block) in the same token order.
constexpr int kStages = 4;

template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
    if constexpr (D == 128) return row & 15;       // 16 chunks a row: rows 0..15 spread over all banks
    else return (row >> 1) & 7;                    // 8 chunks a row: two rows per bank sweep
}

// Wait until at most N of this wave's vector-memory loads are outstanding,
// then meet the other waves.  Written as one asm statement with a memory
// clobber: the compiler neither moves LDS accesses across it nor adds a full
// drain of the LDS-bound loads, as a fenced barrier would.
template <int N>
__device__ __forceinline__ void wait_loads_then_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Maxima of finite-or-minus-infinity values, as one v_maximum3_f32 (IEEE
// maximum: no signalling-NaN quieting, so no extra instruction per operand as
// fmaxf costs).  Never inline asm: a VALU read of a matrix-core result needs
// wait states the hardware does not enforce, and the compiler inserts them only
// for instructions it can see.  An asm v_max3_f32 fed straight from the Q.K^T
// accumulators once read them before the MFMA had written them, so the block
// max, and with it the rescale reference, varied from run to run.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Max across the four lanes of a row (l % 16 equal; v_permlane16_swap pairs
// row r with row r ^ 1, v_permlane32_swap r with r ^ 2) of two values a, b at
// once.  A 32-lane swap of a against b leaves
// a's lanes 0-31 and b's lanes 0-31 in the first result and both upper halves
// in the second, so their max holds a's pair max (lanes l, l + 32) in lanes
// 0-31 and b's in lanes 32-63; a 16-lane swap of that with itself completes
// both four-lane maxes, and a last 32-lane swap copies each half across.
__device__ __forceinline__ void row_max4x2(float a, float b, float& ma, float& mb) {
    const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                                    false, false);
    const float c = __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)s[0]),
                                                  __builtin_bit_cast(float, (uint32_t)s[1]));
    const uint32_t cu = __builtin_bit_cast(uint32_t, c);
    const auto t = __builtin_amdgcn_permlane16_swap(cu, cu, false, false);
    const float d = __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)t[0]),
                                                  __builtin_bit_cast(float, (uint32_t)t[1]));
    const uint32_t du = __builtin_bit_cast(uint32_t, d);
    const auto u = __builtin_amdgcn_permlane32_swap(du, du, false, false);
    ma = __builtin_bit_cast(float, (uint32_t)u[0]);
    mb = __builtin_bit_cast(float, (uint32_t)u[1]);
}

typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

// Eight ds_read_b64_tr_b16, at a[m] and at a[m] + OFF bytes (the same rows of
// the next block), issued without waiting; tr_wait8 later waits for every LDS
// read and hands the registers on through the wait, so nothing reads them
// before the data has landed.  In asm because the compiler, unable to tell
// these reads from the stage loads still landing in other LDS buffers, would
// otherwise drain every outstanding vector-memory load first.
// The reads sit at a + BASE and a + BASE + OFF (immediate offsets, so a stage
// buffer known at compile time costs no address arithmetic).
template <int BASE, int OFF>
__device__ __forceinline__ void tr_issue8(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, u32x2_t (&o)[8]) {
    static_assert(BASE >= 0 && BASE + OFF < 65536, "16-bit LDS offset");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
        "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%13"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "n"(BASE), "n"(BASE + OFF)
        : "memory");
}
// Eight ds_read_b64_tr_b8 at a[0..7] + BASE, issued without waiting (tr_wait8 waits).
template <int BASE>
__device__ __forceinline__ void trb8_issue8(const uint32_t (&a)[8], u32x2_t (&o)[8]) {
    static_assert(BASE >= 0 && BASE < 65536, "16-bit LDS offset");
    asm volatile(
        "ds_read_b64_tr_b8 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b8 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b8 %2, %10 offset:%16\n\t"
        "ds_read_b64_tr_b8 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b8 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b8 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b8 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b8 %7, %15 offset:%16"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "n"(BASE)
        : "memory");
}

template <int V>
struct StageBuf {
    static constexpr int value = V;
};
__device__ __forceinline__ void tr_wait8(u32x2_t (&o)[8]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]), "+v"(o[4]), "+v"(o[5]), "+v"(o[6]), "+v"(o[7])
                 :
                 : "memory");
}

// Direct-to-LDS loads of 16 bytes a lane (global_load_lds_dwordx4: lane l's
// bytes land at LDS byte M0 + 16 l), written as asm.  From the builtin, the
// compiler tracks these loads and, unable to tell which LDS bytes they write,
// makes every later LDS read wait until all of them have landed, which would
// drain the stage ring at every step; the stage loop does its own waiting (a
// vector-memory count, then a barrier, before a stage is read).  The
// instruction writes no register.  An M0 write needs one wait state before
// the load reads it.
// M0 is named as clobbered; these kernels make no other use of it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const char* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds) : "m0");
}
__device__ __forceinline__ void lds_dma16(const char* vaddr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(vaddr), "s"(lds) : "m0");
}
#pragma clang diagnostic pop

template <int KDT, int QDT, int D>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void paged_prefill_dma_kernel(PrefillParams p) {
    constexpr bool F8 = KDT == DT_FP8;         // E4M3 codes: widened as they leave LDS
    constexpr int PT = F8 ? DT_F16 : KDT;      // type of P and V in P.V
    constexpr int KS = D / 32;                 // S^T steps per block (32 dims each)
    constexpr int MT = D / 16;                 // O^T m-tiles (16 dims each)
    constexpr int R = kRowGroups;
    constexpr int ROWB = D * (F8 ? 1 : 2);     // bytes of a token row
    constexpr int SWZ = ROWB / 2;              // chunk_swizzle<SWZ>: the swizzle of a row of ROWB bytes
    constexpr int CH = ROWB / 16;              // 16-byte chunks per row
    constexpr int SROWS = 2 * kBlock;          // token rows per stage
    constexpr int NI = SROWS * CH / (64 * kPfWaves);   // loads per wave per tensor per stage
    constexpr int SB = SROWS * ROWB;           // bytes of one tensor's stage
    constexpr float kLazy = 8.0f;
    static_assert(NI >= 1 && (64 / CH) * NI * kPfWaves == SROWS, "stage rows split evenly over the loads");
    static_assert(F8 ? QDT != KDT : QDT == KDT, "16-bit pools take queries of their own type");
    using QV = typename Vec8<QDT>::T;
    using PV = typename Vec8<PT>::T;
    __shared__ __align__(16) unsigned char k_lds[kStages][SB];
    __shared__ __align__(16) unsigned char v_lds[kStages][SB];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane >> 4, c = lane & 15;
    const int gs = p.gs, subs = p.G / gs;
    const int tw = (16 * R) / gs;                            // query tokens per wave
    const int64_t tiles = p.tiles;
    const int64_t n_wg = tiles * p.H_kv * subs * p.n_seqs;
    const int64_t L = xcd_logical(blockIdx.x, n_wg);
    const int tile = (int)(tiles - 1 - L % tiles);          // latest (heaviest under the causal mask) first
    const int hgi = (int)((L / tiles) % ((int64_t)p.H_kv * subs));
    const int s = (int)(L / (tiles * p.H_kv * subs));
    const int g = hgi / subs;
    const int hq0 = g * p.G + (hgi % subs) * gs;

    const int q0 = min(p.q_start[s], p.total_q), q1 = min(max(p.q_start[s + 1], q0), p.total_q);
    const int q_len = q1 - q0;
    int n = p.lens[s];
    n = n < 0 ? 0 : (n > p.max_blocks * kBlock ? p.max_blocks * kBlock : n);
    const int tile0 = tile * kPfWaves * tw;                 // first query token of the workgroup
    if (tile0 >= q_len) return;
    const int tile_last = min(q_len, tile0 + kPfWaves * tw) - 1;
    const int wg_see = p.causal ? n - q_len + tile_last : n - 1;
    const int nblk = wg_see < 0 ? 0 : min((wg_see + kBlock) / kBlock, (n + kBlock - 1) / kBlock);
    const int n_it = (nblk + 1) >> 1;

    // A negative scale flips q's sign bits (exact) so that the logit scale is
    // positive and the row max can be taken before scaling.
    float scale2 = p.scale * kLog2e;
    float vscale = 1.0f;
    if constexpr (F8) {                        // FP8: the K scale joins the logit scale, the V scale the output
        scale2 *= p.k_scale[g];
        vscale = p.v_scale[g];
    }
    const uint32_t qflip = scale2 < 0.0f ? 0x80008000u : 0u;
    const float qscale = fmaxf(fabsf(scale2), 1e-30f);

    int see[R];
    bool live[R];
    int i_row[R];
    QV qb[R][KS];
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        const int row = rg * 16 + c;
        i_row[rg] = tile0 + wave * tw + row / gs;
        live[rg] = row < tw * gs && i_row[rg] < q_len;
        see[rg] = p.causal ? n - q_len + i_row[rg] : n - 1;
        const int64_t qrow = ((int64_t)(q0 + i_row[rg]) * p.H_q + hq0 + row % gs) * D;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            if (live[rg]) raw = *reinterpret_cast<const uint4*>(q16 + qrow + 32 * k + 8 * r);
            raw.x ^= qflip; raw.y ^= qflip; raw.z ^= qflip; raw.w ^= qflip;
            qb[rg][k] = __builtin_bit_cast(QV, raw);
        }
    }

    // Load geometry: load i of this wave fills stage chunks (wave * NI + i) * 64
    // + lane, i.e. row ld_row, physical chunk lane % CH, holding logical chunk
    // (lane % CH) ^ swizzle(row).  All rows of one load lie in one block.
    const int32_t* table = p.tables + (int64_t)s * p.max_blocks;
    const char* kbase = reinterpret_cast<const char*>(p.k_pool) + (int64_t)g * kBlock * ROWB;
    const char* vbase = reinterpret_cast<const char*>(p.v_pool) + (int64_t)g * kBlock * ROWB;
    const char* zero = reinterpret_cast<const char*>(p.zero_tile);
    const int64_t blk_stride = (int64_t)p.H_kv * kBlock * ROWB;
    const uint32_t blk_stride32 = (uint32_t)blk_stride;        // kv_heads <= 65535: below 2^28
    const int j_whole = n / (2 * kBlock);                       // stages whose 32 tokens all lie in the context
    int ld_off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int slot = (wave * NI + i) * 64 + lane;
        const int row = slot / CH, pch = slot % CH;
        ld_off[i] = (row % kBlock) * ROWB + ((pch ^ chunk_swizzle<SWZ>(row)) * 16);
    }
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto lds_addr = [](const unsigned char* ptr) {     // LDS byte address of a shared-memory pointer
        return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)ptr;
    };
    // Table entries of stage jj (-1 past the visible blocks), read through the
    // scalar cache as constant data one step before the stage's loads use them,
    // so that their latency is not waited out at the hand-over.  Stages past
    // the last one (jj >= n_it) keep the ring's waits uniform: they have no
    // blocks and read the zero tile.
    const __attribute__((address_space(4))) int32_t* ctab =
        (const __attribute__((address_space(4))) int32_t*)table;
    auto entries = [&](int jj, int& ph0, int& ph1) {
        const int b0 = 2 * jj, b1 = 2 * jj + 1;
        const int e0 = ctab[min(b0, nblk - 1)], e1 = ctab[min(b1, nblk - 1)];   // nblk >= 1 here
        ph0 = b0 < nblk ? e0 : -1;
        ph1 = b1 < nblk ? e1 : -1;
    };
    // The loads of stage jj (blocks 2 jj, 2 jj + 1, physical ph0, ph1) into
    // buffer BUF = jj % 4.
    auto issue = [&](int jj, auto BUF, int ph0, int ph1) {
        const bool ok0 = (uint32_t)ph0 < (uint32_t)p.num_blocks, ok1 = (uint32_t)ph1 < (uint32_t)p.num_blocks;
        const bool full = ok0 && ok1 && jj < j_whole;                       // uniform
        constexpr int buf = decltype(BUF)::value;
        if (full) {                            // uniform base + 32-bit lane offset
            // a wave's loads cover 8 consecutive stage rows, all in one block
            static_assert(NI * (64 / CH) <= kBlock && kBlock % (NI * (64 / CH)) == 0, "a wave's rows lie in one block");
            const int h = (wave_u * NI * (64 / CH)) / kBlock;
            const uint64_t base = (uint64_t)(uint32_t)(h ? ph1 : ph0) * blk_stride32;   // ph checked >= 0
            const char* kb = kbase + base;
            const char* vb = vbase + base;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int dst = (wave_u * NI + i) * 64 * 16;                  // bytes
                lds_dma16(kb, (uint32_t)ld_off[i], lds_addr(&k_lds[buf][dst]));
                lds_dma16(vb, (uint32_t)ld_off[i], lds_addr(&v_lds[buf][dst]));
            }
        } else {                               // rows past the context or in a bad block read the zero tile
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int h = ((wave_u * NI + i) * (64 / CH)) / kBlock;
                const int ph = h ? ph1 : ph0;
                const int dst = (wave_u * NI + i) * 64 * 16;
                // formed here, not hoisted out of the loop as 64-bit registers
                uint32_t off = (uint32_t)ld_off[i];
                int ln = lane;
                asm volatile("" : "+v"(off), "+v"(ln));
                const int ld_row = ((wave_u * NI + i) * 64 + ln) / CH;      // stage row of this lane's chunk
                const bool ok = (h ? ok1 : ok0) && 2 * jj * kBlock + ld_row < n;
                const char* ks = ok ? kbase + (int64_t)ph * blk_stride + off : zero + off;
                const char* vs = ok ? vbase + (int64_t)ph * blk_stride + off : zero + off;
                lds_dma16(ks, lds_addr(&k_lds[buf][dst]));
                lds_dma16(vs, lds_addr(&v_lds[buf][dst]));
            }
        }
    };

    f32x4_t acc[R][MT];
    // m_run is the reference max, finite from the start: a row's first block
    // with a visible token moves it (its weights before that are exp2(-inf) = 0,
    // and the rescale factor exp2(kNoMax - m) is 0).
    constexpr float kNoMax = -1e30f;
    // acc_l: the row sums of the weights, as one more 16-dim tile of P.V whose
    // V^T is all ones (every lane of a row then holds its sum; the products
    // are exact and the sum is kept in fp32 like the other tiles)
    float m_run[R];
    f32x4_t acc_l[R];
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        m_run[rg] = kNoMax;
        acc_l[rg] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rg][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const int wg_min_see = p.causal ? n - q_len + tile0 : n - 1;
    // Stage jj needs masking if it reaches past the context or past the diagonal
    // of the workgroup's first query token.
    // Stage jj needs no mask iff 32 (jj + 1) <= min(n, wg_min_see + 1).
    const int j_unmasked = max(0, min(n, wg_min_see + 1)) / (2 * kBlock);
    auto stage_masked = [&](int jj) { return jj >= j_unmasked; };

    // K operand of the stage in buffer BUF, block h: token c, dims 32 k + 8 r ..
    // +7 (16 bytes, or 8 E4M3 codes widened exactly to q's type).
    auto k_read = [&](auto BUF, QV (&ka)[2][KS]) {
        constexpr int buf = decltype(BUF)::value;
        const unsigned char* kt = k_lds[buf];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = h * kBlock + c;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                if constexpr (F8)
                    ka[h][k] = __builtin_bit_cast(QV, fp8x8_to<QDT>(*reinterpret_cast<const uint2*>(
                        kt + row * ROWB + ((2 * k + (r >> 1)) ^ chunk_swizzle<SWZ>(row)) * 16 + (r & 1) * 8)));
                else
                    ka[h][k] = *reinterpret_cast<const QV*>(kt + row * ROWB + ((4 * k + r) ^ chunk_swizzle<SWZ>(row)) * 16);
            }
        }
    };
    // S^T of both blocks for both row groups: lane (r, c) gets the logits of
    // tokens 4 r .. +3 of block 0 (z[rg][0..3]) and of block 1 (z[rg][4..7]) for row c.
    auto s_mma = [&](const QV (&ka)[2][KS], float (&z)[R][8]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int rg = 0; rg < R; ++rg) {
                f32x4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k = 0; k < KS; ++k) S = mma_k32<QDT>(ka[h][k], qb[rg][k], S);
#pragma unroll
                for (int i = 0; i < 4; ++i) z[rg][4 * h + i] = S[i];
            }
        }
    };
    // V^T operand of the stage in buffer BUF, dims 16 mt + c, tokens 4 r .. +3 of
    // block 0 then of block 1.
    // ds_read_b64_tr_b16 builds, in each 16-lane group, row k from the 4
    // elements lanes 4k .. 4k + 3 point at and hands lane i element i of rows
    // 0 .. 3; so lane (r, c) points at token 4 r + c / 4, dims 16 mt + 4 (c % 4).
    // Block 1's rows sit 16 rows (16 * ROWB bytes) after block 0's, with the same swizzle.
    // E4M3 pools: ds_read_b64_tr_b8 builds, in each 16-lane group, row k
    // from the 16 bytes lanes 2k, 2k + 1 point at and hands lane i byte i
    // of rows 0 .. 7.  Lane (r, c) points at the token that k-index
    // 8 r + c / 2 stands for (tokens 4 r .. +3 of block 0, then of block
    // 1), dims 16 mt + 8 (c % 2) .. +7, so one read per m-tile gives the
    // lane its 8 codes of dim 16 mt + c, widened exactly to f16.
    constexpr int NV = F8 ? MT / 8 : MT / 4;          // issue groups of 8 reads
    auto v_issue = [&](auto BUF, u32x2_t (&vh)[NV][8]) {
        constexpr int buf = decltype(BUF)::value;
        const unsigned char* vt = v_lds[0];        // buffer 0's address + buf * SB as an immediate
        if constexpr (F8) {
            const int kk = c >> 1;
            const int trow = kk < 4 ? 4 * r + kk : kBlock + 4 * r + (kk - 4);
            const uint32_t rbase =
                (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(vt + trow * ROWB) + (c & 1) * 8;
            const int sw = chunk_swizzle<SWZ>(trow);
#pragma unroll
            for (int m8 = 0; m8 < MT; m8 += 8) {
                uint32_t a8[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) a8[u] = rbase + (uint32_t)(((m8 + u) ^ sw) * 16);
                trb8_issue8<buf * SB>(a8, vh[m8 / 8]);
            }
        } else {
            const int vrow = 4 * r + (c >> 2);
            const uint32_t vrow_addr =
                (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(vt + vrow * ROWB) + (c & 1) * 8;
#pragma unroll
            for (int m4 = 0; m4 < MT; m4 += 4) {
                uint32_t a[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int lc = 2 * (m4 + u) + ((c & 3) >> 1);
                    a[u] = vrow_addr + (uint32_t)((lc ^ chunk_swizzle<SWZ>(vrow)) * 16);
                }
                tr_issue8<buf * SB, kBlock * ROWB>(a[0], a[1], a[2], a[3], vh[m4 / 4]);
            }
        }
    };
    auto v_wait = [&](u32x2_t (&vh)[NV][8]) {
#pragma unroll
        for (int v = 0; v < NV; ++v) tr_wait8(vh[v]);
    };
    // Mask the logits of stage jj (mask), then take the block max of each row
    // and, where it passes the row's threshold, move the reference max and
    // rescale the row's sum and accumulators (row_update).
    auto mask = [&](bool masked, int jj, float (&z)[R][8]) {
        const int tok = 2 * jj * kBlock + 4 * r;
        if (masked) {                          // one uniform branch for both row groups
#pragma unroll
            for (int rg = 0; rg < R; ++rg) {
                // token tok + (i / 4) * 16 + i % 4 is visible iff that offset <= lim
                const int lim = min(n - 1, see[rg]) - tok;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    z[rg][i] = (i >> 2) * kBlock + (i & 3) <= lim ? z[rg][i] : -INFINITY;   // select, never 0 * garbage
            }
        }
    };
    auto row_update = [&](float (&z)[R][8]) {
        // Lazy reference max: a row's reference moves only when a logit passes
        // it by more than kLazy (weights up to 2^kLazy are fine in every P
        // type).  Each lane tests its own 8 logits; only when some lane of the
        // wave passes is the row max taken across the row's 4 lanes.
        float mx[R];
        bool pass = false;
#pragma unroll
        for (int rg = 0; rg < R; ++rg) {
            mx[rg] = vmax3(vmax3(z[rg][0], z[rg][1], z[rg][2]), vmax3(z[rg][3], z[rg][4], z[rg][5]),
                           __builtin_elementwise_maximum(z[rg][6], z[rg][7]));
            pass = pass || mx[rg] * qscale - m_run[rg] > kLazy;
        }
        if (__builtin_amdgcn_ballot_w64(pass) != 0) {
            static_assert(R == 2, "row maxes are reduced in pairs");
            float rmax[R];
            row_max4x2(mx[0], mx[1], rmax[0], rmax[1]);
#pragma unroll
            for (int rg = 0; rg < R; ++rg) {
                const float m_blk = rmax[rg] * qscale;
                const bool moves = m_blk - m_run[rg] > kLazy;
                if (__builtin_amdgcn_ballot_w64(moves) != 0) {
                    const float m_new = moves ? m_blk : m_run[rg];
                    const float alpha = m_new == m_run[rg] ? 1.0f : __builtin_amdgcn_exp2f(m_run[rg] - m_new);
                    acc_l[rg] *= alpha;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[rg][mt] *= alpha;
                    m_run[rg] = m_new;
                }
            }
        }
    };
    // P = exp2(z * qscale - m) in P.V's 16-bit type.
    auto softmax = [&](const float (&z)[R][8], PV (&pb)[R]) {
#pragma unroll
        for (int rg = 0; rg < R; ++rg) {
            float pr[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(z[rg][i], qscale, -m_run[rg]));
            const uint4 pw = make_uint4(pack2<PT>(pr[0], pr[1]), pack2<PT>(pr[2], pr[3]),
                                        pack2<PT>(pr[4], pr[5]), pack2<PT>(pr[6], pr[7]));
            pb[rg] = __builtin_bit_cast(PV, pw);
        }
    };
    // O^T += V^T . P^T over the stage's 32 tokens, and the row sums of P (the
    // weights P.V multiplies, so that the output is their normalised average).
    const uint32_t one2 = PT == DT_BF16 ? 0x3f803f80u : 0x3c003c00u;
    const PV ones = __builtin_bit_cast(PV, make_uint4(one2, one2, one2, one2));
    auto pv_mma = [&](const u32x2_t (&vh)[NV][8], const PV (&pb)[R]) {
#pragma unroll
        for (int rg = 0; rg < R; ++rg) acc_l[rg] = mma_k32<PT>(ones, pb[rg], acc_l[rg]);
        if constexpr (F8) {
#pragma unroll
            for (int m8 = 0; m8 < MT; m8 += 8) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const PV va = __builtin_bit_cast(PV, fp8x8_to<DT_F16>(make_uint2(vh[m8 / 8][u].x, vh[m8 / 8][u].y)));
#pragma unroll
                    for (int rg = 0; rg < R; ++rg) acc[rg][m8 + u] = mma_k32<PT>(va, pb[rg], acc[rg][m8 + u]);
                }
            }
        } else {
#pragma unroll
            for (int m4 = 0; m4 < MT; m4 += 4) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const PV va = __builtin_bit_cast(PV, make_uint4(vh[m4 / 4][2 * u].x, vh[m4 / 4][2 * u].y,
                                                                     vh[m4 / 4][2 * u + 1].x, vh[m4 / 4][2 * u + 1].y));
#pragma unroll
                    for (int rg = 0; rg < R; ++rg) acc[rg][m4 + u] = mma_k32<PT>(va, pb[rg], acc[rg][m4 + u]);
                }
            }
        }
    };

    // Software pipeline over stages of two blocks.  Step j turns the logits of
    // stage j (already masked, with the row maxes applied) into weights and
    // accumulates P.V of stage j, while it computes the logits of stage j + 1:
    // the matrix cores work on S^T(j + 1) while the vector ALUs take the
    // exponentials of stage j, and on P.V(j) while they take the maxes of
    // stage j + 1, so the two units overlap within one wave.
    //
    // Buffers.  Stage s lives in buffer s % 4.  Its K is read in step s - 1
    // before S^T(s), its V at the end of step s - 1, and both reads are
    // complete before step s begins.  Step j waits until stage j + 1 has
    // landed, meets the other waves (after which no wave reads stage j's
    // buffer), and refills that buffer with stage j + 4: three stages are in
    // flight while one is computed.  Stages past the end are issued too (from
    // the zero tile), so that every wait counts the same loads; they are
    // drained before the workgroup ends.
    constexpr int LPS = 2 * NI;                // loads per stage per wave
    float z[R][8];
    u32x2_t vh[NV][8];
    int nx0 = -1, nx1 = -1;                    // table entries of the next stage to issue
    if (n_it > 0) {
        int e0, e1;
        entries(0, e0, e1);
        issue(0, StageBuf<0>{}, e0, e1);
        entries(1, e0, e1);
        issue(1, StageBuf<1>{}, e0, e1);
        entries(2, e0, e1);
        issue(2, StageBuf<2>{}, e0, e1);
        entries(3, e0, e1);
        issue(3, StageBuf<3>{}, e0, e1);
        entries(4, nx0, nx1);
        wait_loads_then_barrier<(kStages - 1) * LPS>();
        QV ka[2][KS];
        k_read(StageBuf<0>{}, ka);
        s_mma(ka, z);
        mask(stage_masked(0), 0, z);
        row_update(z);
        v_issue(StageBuf<0>{}, vh);
        v_wait(vh);
    }
    static_assert(kStages == 4, "the loop is unrolled over four buffers");
    // Step j < n_it - 1 (the last stage's P.V follows the loop).
    auto step = [&](int j, auto BUF) {
        constexpr int nbuf = (decltype(BUF)::value + 1) % kStages;
        wait_loads_then_barrier<2 * LPS>();
        issue(j + 4, BUF, nx0, nx1);           // (j + 4) % 4 == j % 4
        QV ka[2][KS];
        k_read(StageBuf<nbuf>{}, ka);
        PV pb[R];
        softmax(z, pb);
        // the weights are formed here, beside S^T(j + 1) on the matrix cores,
        // not sunk past the mask branch to where P.V uses them
#pragma unroll
        for (int rg = 0; rg < R; ++rg) asm volatile("" ::"v"(pb[rg]));
        float zn[R][8];
        s_mma(ka, zn);
        mask(stage_masked(j + 1), j + 1, zn);  // before P.V(j), so that P.V and the maxes share a block
        // A wave issuing P.V takes precedence over the other wave of its SIMD
        // (which is then on its exponentials or its stage hand-over), so that
        // the matrix cores are kept fed.
        __builtin_amdgcn_s_setprio(1);
        pv_mma(vh, pb);
        v_issue(StageBuf<nbuf>{}, vh);         // the registers P.V(j) has just read
        row_update(zn);
        v_wait(vh);
        __builtin_amdgcn_s_setprio(0);
        // after the wait for the V reads: a scalar load in flight would make
        // every LDS wait of this step wait for it too
        entries(j + 5, nx0, nx1);
#pragma unroll
        for (int rg = 0; rg < R; ++rg)
#pragma unroll
            for (int i = 0; i < 8; ++i) z[rg][i] = zn[rg][i];
    };
    for (int j = 0; j < n_it - 1; j += kStages) {
        step(j, StageBuf<0>{});
        if (j + 1 < n_it - 1) step(j + 1, StageBuf<1>{});
        if (j + 2 < n_it - 1) step(j + 2, StageBuf<2>{});
        if (j + 3 < n_it - 1) step(j + 3, StageBuf<3>{});
    }
    if (n_it > 0) {
        PV pb[R];
        softmax(z, pb);
        pv_mma(vh, pb);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the stages past the end
    }

    uint16_t* o16 = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        if (!live[rg]) continue;
        const int row = rg * 16 + c;
        const float l = acc_l[rg][0];
        const float inv = l > 0.0f ? vscale / l : 0.0f;
        const int64_t orow = ((int64_t)(q0 + i_row[rg]) * p.H_q + hq0 + row % gs) * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            uint16_t e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = to_q16<QDT>(acc[rg][mt][i] * inv);
            *reinterpret_cast<uint2*>(o16 + orow + 16 * mt + 4 * r) =
                make_uint2((uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16));
        }
    }
}

using KernelFn = void (*)(PrefillParams);

template <int KDT, int QDT>
KernelFn pick_d(int D) {
    switch (D) {
        case 64: return paged_prefill_kernel<KDT, QDT, 64>;
        case 128: return paged_prefill_kernel<KDT, QDT, 128>;
        default: return nullptr;
    }
}

template <int KDT>
KernelFn pick_dma(int D) {
    switch (D) {
        case 64: return paged_prefill_dma_kernel<KDT, KDT, 64>;
        case 128: return paged_prefill_dma_kernel<KDT, KDT, 128>;
        default: return nullptr;
    }
}

// E4M3 pools: the direct-to-LDS kernel at head_dim 128 (a stage of 64-dim
// codes is too small for every lane to move 16 bytes), the register-staged
// kernel at 64.
template <int QDT>
KernelFn pick_fp8(int D) {
    if (D == 128) return paged_prefill_dma_kernel<DT_FP8, QDT, 128>;
    return pick_d<DT_FP8, QDT>(D);
}

KernelFn pick(int kdt, int qdt, int D) {
    if (kdt == DT_F16 && qdt == DT_F16) return pick_dma<DT_F16>(D);
    if (kdt == DT_BF16 && qdt == DT_BF16) return pick_dma<DT_BF16>(D);
    if (kdt == DT_FP8 && qdt == DT_BF16) return pick_fp8<DT_BF16>(D);
    if (kdt == DT_FP8 && qdt == DT_F16) return pick_fp8<DT_F16>(D);
    return nullptr;
}

}  // namespace

bool prefill_supported(int32_t kv_dt, int32_t q_dt, int32_t D) { return pick(kv_dt, q_dt, D) != nullptr; }

int prefill_heads_per_group(int32_t G) {
    if (G <= 16) return G;
    for (int gs = 16; gs >= 1; --gs)
        if (G % gs == 0) return gs;
    return 1;
}

int64_t prefill_tiles(int32_t G, int32_t max_q_len) {
    const int tw = (16 * kRowGroups) / prefill_heads_per_group(G);
    const int per_wg = kPfWaves * tw;
    return ((int64_t)max_q_len + per_wg - 1) / per_wg;
}

int64_t prefill_workgroups(int32_t G, int32_t H_kv, int32_t n_seqs, int32_t max_q_len) {
    return prefill_tiles(G, max_q_len) * H_kv * (G / prefill_heads_per_group(G)) * n_seqs;
}

hipError_t launch_prefill(const PrefillParams& p, int32_t max_q_len, hipStream_t stream) {
    KernelFn fn = pick(p.kv_dt, p.q_dt, p.D);
    if (!fn) return hipErrorInvalidValue;
    const int64_t n_wg = prefill_workgroups(p.G, p.H_kv, p.n_seqs, max_q_len);
    if (n_wg <= 0) return hipSuccess;
    PrefillParams arg = p;
    arg.tiles = prefill_tiles(p.G, max_q_len);
    void* args[] = {&arg};
    return launch_kernel(reinterpret_cast<const void*>(fn), dim3((unsigned)n_wg), dim3(kPfWaves * 64), args, 0,
                           stream);
}

}  // namespace pkv
