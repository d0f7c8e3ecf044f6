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

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elem<DT_F16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_FP8> { static constexpr int bytes = 1; };

// Geometry of one (block, KV head) tile [16][D] of storage type DT.
template <int DT, int D> struct Tile {
    static constexpr int E = Elem<DT>::bytes;
    static constexpr int ROW = D * E;                                // bytes of one token row
    static constexpr int BYTES = kBlock * ROW;                       // bytes of the tile
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

template <int KDT, int QDT, int D, int GS>
__global__ __launch_bounds__(kDecodeWaves * 64) void paged_decode_partition(DecodeParams p) {
    using TL = Tile<KDT, D>;
    using RawT = typename Raw<TL::W>::T;
    constexpr int EPL = TL::EPL, LPR = TL::LPR, RPL = TL::RPL, NLOAD = TL::NLOAD;
    constexpr int NS = kDecodeWaves * RPL;   // softmax streams per workgroup

    __shared__ float s_m[NS][GS];
    __shared__ float s_l[NS][GS];
    __shared__ float s_o[NS][GS][D];

    const int part = blockIdx.x;
    const int subs = p.G / GS;
    const int g = blockIdx.y / subs;
    const int hq0 = g * p.G + (blockIdx.y % subs) * GS;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane / LPR, c = lane % LPR;

    int n = p.lens[b];
    n = n < 0 ? 0 : n;
    n = n > p.max_len ? p.max_len : n;
    n = n > p.max_blocks * kBlock ? p.max_blocks * kBlock : n;
    const int pstart = part * p.part_tokens;
    const bool single = n <= p.part_tokens;
    if (n == 0) {
        // empty context: out = 0 (written once, by partition 0)
        if (part == 0)
            for (int i = tid; i < GS * D; i += kDecodeWaves * 64)
                store_out<QDT>(p.out, ((int64_t)b * p.H_q + hq0) * D + i, 0.0f);
        return;
    }
    if (pstart >= n) return;
    const int pend = min(n, pstart + p.part_tokens);
    const int blk_first = pstart / kBlock;
    const int blk_last = (pend + kBlock - 1) / kBlock;   // exclusive

    // Query fragment: this lane's EPL dims of each of the GS heads, scaled to base 2.
    float qscale = p.scale * kLog2e;
    if constexpr (KDT == DT_FP8) qscale *= p.k_scale[g];
    float qf[GS][EPL];
#pragma unroll
    for (int h = 0; h < GS; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            qf[h][e] = load_q<QDT>(p.q, ((int64_t)b * p.H_q + hq0 + h) * D + c * EPL + e) * qscale;

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
    const int64_t head_off = (int64_t)g * TL::BYTES;
    const int64_t blk_stride = (int64_t)p.H_kv * TL::BYTES;

    RawT kc[NLOAD], vc[NLOAD], kn[NLOAD], vn[NLOAD];
    auto fetch = [&](int blk, RawT* kr, RawT* vr) -> bool {
        const int phys = table[blk];
        if (phys < 0 || phys >= p.num_blocks) return false;
        const int64_t off = (int64_t)phys * blk_stride + head_off + lane_off;
        const char* kp = kbase + off;
        const char* vp = vbase + off;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            kr[i] = *reinterpret_cast<const RawT*>(kp + i * TL::ROW);
            vr[i] = *reinterpret_cast<const RawT*>(vp + i * TL::ROW);
        }
        return true;
    };

    int blk = blk_first + wave;
    bool ok_c = blk < blk_last ? fetch(blk, kc, vc) : false;
    for (; blk < blk_last; blk += kDecodeWaves) {
        const int nblk = blk + kDecodeWaves;
        const bool ok_n = nblk < blk_last ? fetch(nblk, kn, vn) : false;
        if (ok_c) {
            const int tok0 = blk * kBlock + r * NLOAD;   // this row's first token in the block
            const bool partial = blk * kBlock + kBlock > pend;
            float z[GS][NLOAD];
            float vf[NLOAD][EPL];
#pragma unroll
            for (int i = 0; i < NLOAD; ++i) {
                float kf[EPL];
                widen<KDT, TL::W>(kc[i], kf);
                widen<KDT, TL::W>(vc[i], vf[i]);
                const bool valid = !partial || (tok0 + i < pend);
#pragma unroll
                for (int h = 0; h < GS; ++h) {
                    float d = 0.0f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) d = fmaf(qf[h][e], kf[e], d);
                    d = row_sum<LPR>(d);
                    z[h][i] = valid ? d : -INFINITY;
                }
                if (partial && !valid) {
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
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    float a = acc[h][e] * alpha;
#pragma unroll
                    for (int i = 0; i < NLOAD; ++i) a = fmaf(pv[i], vf[i][e], a);
                    acc[h][e] = a;
                }
                m[h] = m_new;
            }
        }
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            kc[i] = kn[i];
            vc[i] = vn[i];
        }
        ok_c = ok_n;
    }

    // Merge the NS streams of this workgroup.
    const int s = wave * RPL + r;
#pragma unroll
    for (int h = 0; h < GS; ++h) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_o[s][h][c * EPL + e] = acc[h][e];
        if (c == 0) {
            s_m[s][h] = m[h];
            s_l[s][h] = l[h];
        }
    }
    __syncthreads();

    float vscale = 1.0f;
    if constexpr (KDT == DT_FP8) vscale = p.v_scale[g];
    for (int i = tid; i < GS * D; i += kDecodeWaves * 64) {
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

// Kernel 2: merge the partitions of one (sequence, query head) with the same
// rule as the in-workgroup merge: M = max m_t, L = sum l_t 2^(m_t - M),
// out = sum o_t 2^(m_t - M) / L.  Sequences that fit one partition were
// finished by kernel 1 and are skipped here.
template <int QDT>
__global__ __launch_bounds__(64) void paged_decode_reduce(DecodeParams p) {
    const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    int n = p.lens[b];
    n = n < 0 ? 0 : n;
    n = n > p.max_len ? p.max_len : n;
    n = n > p.max_blocks * kBlock ? p.max_blocks * kBlock : n;
    const int nparts = (n + p.part_tokens - 1) / p.part_tokens;
    if (nparts <= 1) return;
    const int64_t base = ((int64_t)b * p.H_q + hq) * p.max_parts;
    float M = -INFINITY;
    for (int t = 0; t < nparts; ++t) M = fmaxf(M, p.ws_ml[(base + t) * 2]);
    for (int d = lane; d < p.D; d += 64) {
        float L = 0.0f, O = 0.0f;
        if (M != -INFINITY) {
            for (int t = 0; t < nparts; ++t) {
                const float w = fast_exp2(p.ws_ml[(base + t) * 2] - M);
                L = fmaf(p.ws_ml[(base + t) * 2 + 1], w, L);
                O = fmaf(p.ws_o[(base + t) * p.D + d], w, O);
            }
        }
        store_out<QDT>(p.out, ((int64_t)b * p.H_q + hq) * p.D + d, L > 0.0f ? O / L : 0.0f);
    }
}

using KernelFn = void (*)(DecodeParams);

template <int KDT, int QDT, int D>
KernelFn pick_gs(int gs) {
    switch (gs) {
        case 1: return paged_decode_partition<KDT, QDT, D, 1>;
        case 2: return paged_decode_partition<KDT, QDT, D, 2>;
        case 3: return paged_decode_partition<KDT, QDT, D, 3>;
        case 4: return paged_decode_partition<KDT, QDT, D, 4>;
        case 5: return paged_decode_partition<KDT, QDT, D, 5>;
        case 6: return paged_decode_partition<KDT, QDT, D, 6>;
        case 7: return paged_decode_partition<KDT, QDT, D, 7>;
        case 8: return paged_decode_partition<KDT, QDT, D, 8>;
        default: return nullptr;
    }
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

KernelFn pick_partition(int kdt, int qdt, int D, int gs) {
    if (kdt == DT_F32 && qdt == DT_F32) return pick_d<DT_F32, DT_F32>(D, gs);
    if (kdt == DT_F16 && qdt == DT_F16) return pick_d<DT_F16, DT_F16>(D, gs);
    if (kdt == DT_BF16 && qdt == DT_BF16) return pick_d<DT_BF16, DT_BF16>(D, gs);
    if (kdt == DT_FP8 && qdt == DT_BF16) return pick_d<DT_FP8, DT_BF16>(D, gs);
    if (kdt == DT_FP8 && qdt == DT_F16) return pick_d<DT_FP8, DT_F16>(D, gs);
    return nullptr;
}

KernelFn pick_reduce(int qdt) {
    switch (qdt) {
        case DT_F32: return paged_decode_reduce<DT_F32>;
        case DT_F16: return paged_decode_reduce<DT_F16>;
        case DT_BF16: return paged_decode_reduce<DT_BF16>;
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
           pick_reduce(q_dt) != nullptr;
}

hipError_t launch_decode_partition(const DecodeParams& p, hipStream_t stream) {
    const int gs = decode_heads_per_wg(p.G);
    KernelFn fn = pick_partition(p.kv_dt, p.q_dt, p.D, gs);
    if (!fn) return hipErrorInvalidValue;
    dim3 grid((unsigned)p.max_parts, (unsigned)(p.H_kv * (p.G / gs)), (unsigned)p.B);
    DecodeParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, dim3(kDecodeWaves * 64), args, 0,
                           stream);
}

hipError_t launch_decode_reduce(const DecodeParams& p, hipStream_t stream) {
    KernelFn fn = pick_reduce(p.q_dt);
    if (!fn) return hipErrorInvalidValue;
    DecodeParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)p.H_q, (unsigned)p.B),
                           dim3(64), args, 0, stream);
}

}  // namespace pkv
