// Internal interface between the host core (pool.cpp) and the HIP kernels.
// Not part of the public ABI (include/pagedkv.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;        // tokens per physical block
constexpr int kZeroTileBytes = kBlock * 128 * 2;   // one 16-token tile of the widest 16-bit row
constexpr int kDecodeWaves = 4;   // waves per decode workgroup
constexpr int kMaxGroupPerWg = 8; // query heads one decode workgroup serves

enum Dt : int32_t { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3, DT_INT8 = 4 };

__host__ __device__ inline int elem_bytes(int32_t dt) { return dt == DT_F32 ? 4 : (dt == DT_FP8 || dt == DT_INT8 ? 1 : 2); }

// INT8 min-max tiles carry a 16-byte header {min, max, step = (max - min) / 255, 0}.
// A block of an INT8 pool holds the codes of its kv_heads tiles first
// (kBlock * D bytes each, so every tile's rows stay on 128-byte lines when
// kv_heads is a multiple of 8), then the kv_heads headers: tile (blk, g) has
// its codes at blk * kv_heads * tile_bytes + g * kBlock * D and its header at
// blk * kv_heads * tile_bytes + kv_heads * kBlock * D + 16 g.
constexpr int kInt8HeaderBytes = 16;

// Bytes of one (block, KV head) tile of a pool.
__host__ __device__ inline int64_t tile_bytes(int32_t dt, int32_t D) {
    return (int64_t)kBlock * D * elem_bytes(dt) + (dt == DT_INT8 ? kInt8HeaderBytes : 0);
}

struct AppendParams {
    const int32_t* slots;
    const void* k_src;
    const void* v_src;
    void* k_pool;
    void* v_pool;
    const float* k_inv;   // FP8 pools: per-head 1/scale
    const float* v_inv;
    int64_t num_slots;    // num_blocks * kBlock
    int32_t T, H_kv, D;
    int32_t src_dt, dst_dt;
    uint64_t* tags;       // INT8 pools: per slot (call epoch << 32 | token) of the last call that wrote it
    uint32_t epoch;       // INT8 pools: this call's epoch (never 0)
};

constexpr int kMaxCopiesPerLaunch = 128;

// Copy-on-write block copies, passed by value (no device list needed).
struct CopyParams {
    int32_t src[kMaxCopiesPerLaunch];
    int32_t dst[kMaxCopiesPerLaunch];
    int32_t n;
    void* k_pool;
    void* v_pool;
    int64_t block_bytes;      // bytes of one block over all KV heads (one pool)
};

struct DecodeParams {
    const void* k_pool;
    const void* v_pool;
    const float* k_scale;     // FP8 pools only
    const float* v_scale;
    const void* q;            // [B][H_q][D]
    void* out;                // [B][H_q][D]
    const int32_t* tables;    // [B][max_blocks]
    const int32_t* lens;      // [B]
    float* ws_ml;             // [B][H_q][max_parts][2]  (running max, sum) per partition
    float* ws_o;              // [B][H_q][max_parts][D]  unnormalised partial output
    int32_t* sched;           // planned mode: 256-byte schedule header (work counter, item count,
                              // partition tokens)
    int2* items;              // planned mode: (sequence, partition) work list; NULL = dense grid
    int32_t B, H_q, H_kv, G, D, num_blocks, max_blocks, max_len;
    int32_t part_tokens;      // dense mode: the partition; planned mode: the host's choice
    int32_t max_parts;        // partitions the workspace holds per context
    int32_t grid_wgs;         // planned mode: workgroups of the partition kernel
    int32_t choose_parts;     // planned mode: the plan kernel may shorten the partition
    int32_t head_groups;      // H_kv * (G / heads per workgroup)
    int32_t kv_dt, q_dt;
    float scale;              // softmax scale as given
};

// Swap: whole blocks (all KV heads, K and V) between the pools and a staging
// buffer laid out [block][K tile bytes | V tile bytes], in logical order.
struct MoveParams {
    int32_t ids[kMaxCopiesPerLaunch];   // physical blocks of this launch
    int32_t n;
    int64_t first;                      // staging slot of ids[0]
    void* k_pool;
    void* v_pool;
    char* staging;
    int64_t block_bytes;
    int32_t to_pool;                    // 0: pools -> staging, 1: staging -> pools
};

struct PrefillParams {
    const void* k_pool;
    const void* v_pool;
    const float* k_scale;     // FP8 pools only
    const float* v_scale;
    const void* q;            // [total_q][H_q][D]
    void* out;                // [total_q][H_q][D]
    const int32_t* q_start;   // [n_seqs + 1]
    const int32_t* tables;    // [n_seqs][max_blocks]
    const int32_t* lens;      // [n_seqs] context lengths including the chunk
    const void* zero_tile;    // kZeroTileBytes of zeros: the source of absent tokens
    int32_t n_seqs, total_q, H_q, H_kv, G, D, num_blocks, max_blocks;
    int32_t gs;               // query heads per row group (divides G, at most 16)
    int64_t tiles;            // query tiles per (sequence, head group), set by the launcher
    int32_t kv_dt, q_dt, causal;
    float scale;
};

// Every kernel of the library is launched through launch_kernel (same
// arguments as hipLaunchKernel).  While a timed call has armed an event pair,
// the launches go through hipExtLaunchKernel: the first records the start
// event as its kernel starts and every one records the stop event as its
// kernel ends, so the pair spans exactly the call's kernels.  Two separate
// hipEventRecord calls around the launch would also count the dispatch and
// completion of the event packets themselves (about 5 us a launch).
hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, void** args, size_t shmem, hipStream_t stream);
void arm_launch_events(hipEvent_t start, hipEvent_t stop);
bool disarm_launch_events();   // true if a launch since arming recorded the events

// Launch one kernel each; return hipSuccess or the launch error.
// Unsupported combinations are filtered on the host before these are called.
hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream);
bool decode_supported(int32_t kv_dt, int32_t q_dt, int32_t D, int32_t G);
int decode_heads_per_wg(int32_t G);
// Workgroups of the partition kernel for this combination that fit on the
// current device at once (a nominal 1024 if the device cannot be queried).
int decode_resident_workgroups(int32_t kv_dt, int32_t q_dt, int32_t D, int32_t G);
hipError_t launch_decode_plan(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_partition(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeParams& p, hipStream_t stream);
// Device address of the fixed decode scratch on `device` (which must be the
// current device), looked up once per device and kept; kNoAllocScratchBytes long.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(int device, void** ptr);
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_read_probe(const void* src, size_t bytes, bool nontemporal, uint32_t* sink, hipStream_t stream);
hipError_t launch_gather_read_probe(const void* src, size_t bytes, bool nontemporal, const int32_t* order,
                                    int64_t n_order, int log_rows, uint32_t* sink, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t stream);
hipError_t launch_move_blocks(const MoveParams& p, hipStream_t stream);
bool prefill_supported(int32_t kv_dt, int32_t q_dt, int32_t D);
int prefill_heads_per_group(int32_t G);
int64_t prefill_tiles(int32_t G, int32_t max_q_len);
int64_t prefill_workgroups(int32_t G, int32_t H_kv, int32_t n_seqs, int32_t max_q_len);
hipError_t launch_prefill(const PrefillParams& p, int32_t max_q_len, hipStream_t stream);

}  // namespace pkv
