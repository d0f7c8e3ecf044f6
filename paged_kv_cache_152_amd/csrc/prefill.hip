// paged_prefill: a chunk of query tokens per sequence attending, through the
// block table, to the cached context and to itself (the prefill stage of
// www.mlqm.cn/news/394450 section 三, chunked as in its section 七; block
// table of www.cf-1.com/news/5824798 §3.1).  Unlike single-token decode this
// is a dense contraction on both sides, so both products run on the matrix
// cores.
//
// Work split.  A workgroup of 4 waves takes one (query tile, head group,
// sequence).  A wave owns 16 query rows: TW = 16 / gs query tokens times the gs
// query heads of one KV head group (row c = token c / gs, head c % gs; rows
// beyond TW * gs are padding).  The four waves walk the same 16-token blocks
// of the context; their K and V tiles come from HBM once per workgroup.
//
// Per block, with m = 16 tokens:
//   S^T = K . Q^T    4 (head_dim 128) or 2 (64) v_mfma_f32_16x16x32: A = the K
//                    tile (lane: token l % 16, 8 dims), straight from HBM;
//                    B = the 16 query rows (lane: row l % 16, 8 dims), held
//                    in registers for the whole walk.  Lane l ends with the
//                    logits of tokens 4 (l / 16) .. +3 for row l % 16.
//   online softmax   the running max / sum of a row live in the four lanes
//                    l % 16 = row; two cross-row shuffles per block.  Logits
//                    are in base 2 (exp2), q's scale folded in.
//   O^T += V^T . P^T head_dim / 16 v_mfma_f32_16x16x16: B = P^T, which is
//                    exactly the layout S^T left in the lanes (packed to
//                    16-bit), A = V^T read from LDS, where the workgroup
//                    wrote the block's V transposed ([dim][token]) once.
// Lane l accumulates output dims 16 mt + 4 (l / 16) + i of row l % 16, so the
// rescale when a row's max moves is one multiply per accumulator.
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

template <int KDT, int QDT, int D>
__global__ __launch_bounds__(kPfWaves * 64) void paged_prefill_kernel(PrefillParams p) {
    constexpr int KS = D / 32;                 // S^T steps (32 dims each)
    constexpr int MT = D / 16;                 // O^T m-tiles (16 dims each)
    constexpr int EPL = D / 16;                // V dims one lane stages per block
    constexpr int PT = KDT == DT_BF16 ? DT_BF16 : DT_F16;   // type of P and V in P.V
    constexpr int KE = KDT == DT_FP8 ? 1 : 2;  // bytes per stored K/V element
    using QV = typename Vec8<QDT>::T;
    // V^T of the current and the next block, [dim][token], 16-bit values of PT
    __shared__ uint16_t vt[2][D][16];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane >> 4, c = lane & 15;
    const int s = blockIdx.z;
    const int gs = p.gs, subs = p.G / gs, TW = 16 / gs;
    const int g = blockIdx.y / subs;
    const int hq0 = g * p.G + (blockIdx.y % subs) * gs;

    const int q0 = min(p.q_start[s], p.total_q), q1 = min(max(p.q_start[s + 1], q0), p.total_q);
    const int q_len = q1 - q0;
    int n = p.lens[s];
    n = n < 0 ? 0 : (n > p.max_blocks * kBlock ? p.max_blocks * kBlock : n);
    const int tile0 = blockIdx.x * kPfWaves * TW;            // first query token of the workgroup
    if (tile0 >= q_len) return;
    const int tile_last = min(q_len, tile0 + kPfWaves * TW) - 1;

    // this lane's query row
    const int i_row = tile0 + wave * TW + c / gs;            // token index within the chunk
    const int h_row = hq0 + c % gs;
    const bool row_live = c < TW * gs && i_row < q_len;
    const int pos = n - q_len + i_row;                       // the row's position in the context
    const int see = p.causal ? pos : n - 1;                  // newest position the row sees

    // the blocks the workgroup needs
    const int wg_see = p.causal ? n - q_len + tile_last : n - 1;
    const int nblk = wg_see < 0 ? 0 : min((wg_see + kBlock) / kBlock, (n + kBlock - 1) / kBlock);

    // Q^T operand: row c, dims 32 k + 8 r .. +7
    QV qb[KS];
    {
        const uint16_t* q16 = reinterpret_cast<const uint16_t*>(p.q);
        const int64_t qrow = ((int64_t)(q0 + i_row) * p.H_q + h_row) * D;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            if (row_live) raw = *reinterpret_cast<const uint4*>(q16 + qrow + 32 * k + 8 * r);
            qb[k] = __builtin_bit_cast(QV, raw);
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
    constexpr int ROW = D * KE;                              // bytes of a token row
    constexpr int TILE = kBlock * ROW;                       // bytes of a (block, head) tile
    const int64_t blk_stride = (int64_t)p.H_kv * TILE;
    const int64_t head_off = (int64_t)g * TILE;
    // K operand of this lane: token c, dims 32 k + 8 r; V staging: token tid / 16, dims EPL (tid % 16)
    const int k_off = c * ROW + 8 * r * KE;
    const int v_tok = tid >> 4, v_dim = (tid & 15) * EPL;
    const int v_off = v_tok * ROW + v_dim * KE;

    using KRaw = std::conditional_t<KDT == DT_FP8, uint2, uint4>;                 // 8 K elements
    using VRaw = std::conditional_t<EPL * KE == 16, uint4, std::conditional_t<EPL * KE == 8, uint2, uint32_t>>;
    struct Stage {
        KRaw k[KS];
        VRaw v;
        bool ok;
    };
    auto fetch = [&](int j, Stage& st) {
        const int phys = table[j];
        st.ok = phys >= 0 && phys < p.num_blocks;
        if (!st.ok) return;
        const int64_t off = (int64_t)phys * blk_stride + head_off;
#pragma unroll
        for (int k = 0; k < KS; ++k) st.k[k] = *reinterpret_cast<const KRaw*>(kbase + off + k_off + 32 * k * KE);
        st.v = *reinterpret_cast<const VRaw*>(vbase + off + v_off);
    };
    // V rows of the block, transposed into LDS as PT values; dead rows are zero
    auto stage_v = [&](int j, const Stage& st, int buf) {
        uint16_t e16[EPL];
        const bool live = st.ok && j * kBlock + v_tok < n;
        if constexpr (KDT == DT_FP8) {
            // EPL codes -> f16
            uint32_t w[EPL / 2];
            if constexpr (EPL == 8) {
                const uint4 f = fp8x8_to<DT_F16>(*reinterpret_cast<const uint2*>(&st.v));
                w[0] = f.x; w[1] = f.y; w[2] = f.z; w[3] = f.w;
            } else {
                const uint32_t code = *reinterpret_cast<const uint32_t*>(&st.v);
                w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(code, 1.0f, false));
                w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(code, 1.0f, true));
            }
#pragma unroll
            for (int e = 0; e < EPL / 2; ++e) {
                e16[2 * e] = (uint16_t)(w[e] & 0xFFFFu);
                e16[2 * e + 1] = (uint16_t)(w[e] >> 16);
            }
        } else {
            const uint32_t* w = reinterpret_cast<const uint32_t*>(&st.v);
#pragma unroll
            for (int e = 0; e < EPL / 2; ++e) {
                e16[2 * e] = (uint16_t)(w[e] & 0xFFFFu);
                e16[2 * e + 1] = (uint16_t)(w[e] >> 16);
            }
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) vt[buf][v_dim + e][v_tok] = live ? e16[e] : (uint16_t)0;
    };

    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    Stage cur, nxt;
    if (nblk > 0) fetch(0, cur);
    for (int j = 0; j < nblk; ++j) {
        const int buf = j & 1;
        stage_v(j, cur, buf);
        if (j + 1 < nblk) fetch(j + 1, nxt);                 // in flight during this block's math
        __syncthreads();                                     // V^T of block j is in LDS

        // S^T = K . Q^T
        f32x4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            QV a;
            if constexpr (KDT == DT_FP8) a = __builtin_bit_cast(QV, fp8x8_to<QDT>(cur.k[k]));
            else a = __builtin_bit_cast(QV, cur.k[k]);
            S = mma_k32<QDT>(a, qb[k], S);
        }
        const int tok = j * kBlock + 4 * r;                  // token of S[0] in this lane
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool vis = cur.ok && row_live && tok + i < n && tok + i <= see;
            z[i] = vis ? S[i] * qscale : -INFINITY;          // select, never 0 * garbage
        }
        const float m_blk = across_rows_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
        const float m_new = fmaxf(m_run, m_blk);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(z[i] - m_use);
        l_run = fmaf(l_run, alpha, across_rows_sum((pr[0] + pr[1]) + (pr[2] + pr[3])));
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
        }
        // O^T += V^T . P^T
        const uint2 pb = make_uint2(pack2<PT>(pr[0], pr[1]), pack2<PT>(pr[2], pr[3]));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint2 va = *reinterpret_cast<const uint2*>(&vt[buf][16 * mt + c][4 * r]);
            acc[mt] = mma_k16<PT>(va, pb, acc[mt]);
        }
        cur = nxt;
    }

    if (!row_live) return;
    const float inv = l_run > 0.0f ? vscale / l_run : 0.0f;
    uint16_t* o16 = reinterpret_cast<uint16_t*>(p.out);
    const int64_t orow = ((int64_t)(q0 + i_row) * p.H_q + h_row) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        uint16_t e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = to_q16<QDT>(acc[mt][i] * inv);
        *reinterpret_cast<uint2*>(o16 + orow + 16 * mt + 4 * r) =
            make_uint2((uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16));
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

KernelFn pick(int kdt, int qdt, int D) {
    if (kdt == DT_F16 && qdt == DT_F16) return pick_d<DT_F16, DT_F16>(D);
    if (kdt == DT_BF16 && qdt == DT_BF16) return pick_d<DT_BF16, DT_BF16>(D);
    if (kdt == DT_FP8 && qdt == DT_BF16) return pick_d<DT_FP8, DT_BF16>(D);
    if (kdt == DT_FP8 && qdt == DT_F16) return pick_d<DT_FP8, DT_F16>(D);
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
    const int tw = 16 / prefill_heads_per_group(G);
    const int per_wg = kPfWaves * tw;
    return ((int64_t)max_q_len + per_wg - 1) / per_wg;
}

hipError_t launch_prefill(const PrefillParams& p, int32_t max_q_len, hipStream_t stream) {
    KernelFn fn = pick(p.kv_dt, p.q_dt, p.D);
    if (!fn) return hipErrorInvalidValue;
    const int64_t tiles = prefill_tiles(p.G, max_q_len);
    if (tiles <= 0 || p.n_seqs <= 0) return hipSuccess;
    PrefillParams arg = p;
    void* args[] = {&arg};
    const unsigned groups = (unsigned)((int64_t)p.H_kv * (p.G / p.gs));
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)tiles, groups, (unsigned)p.n_seqs),
                           dim3(kPfWaves * 64), args, 0, stream);
}

}  // namespace pkv
