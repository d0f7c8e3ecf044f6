// Host core of libpagedkv: the block pool, its allocator, argument checks and
// the C ABI declared in include/pagedkv.h.
//
// Allocator (www.cf-1.com/news/5824798 §3.1-§3.3; m.lqnn.cn/news/219451 §3):
// one pool of fixed 16-token blocks, a FIFO free list seeded by the caller, a
// per-sequence block table grown on demand (a block is taken only when a new
// position starts one, so only the last block is ever partly filled), and a
// per-block reference count so several tables can share prefix blocks.  A
// block whose count drops to zero goes to the back of the free list.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <array>
#include <deque>
#include <limits>
#include <list>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

// The library is built with hidden visibility; only the C ABI is exported.
#pragma GCC visibility push(default)
#include "../../include/pagedkv.h"
#pragma GCC visibility pop
#include "internal.h"

static_assert(PKV_NOALLOC_SCRATCH_BYTES == pkv::kNoAllocScratchBytes, "scratch size differs from the header's");

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return PKV_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(PKV_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

struct Seq {
    std::vector<int32_t> blocks;
    int32_t len = 0;
    bool swapped = false;      // blocks live on the host (kv_seq_swap_out); `blocks` is empty
};

constexpr int kMaxTimed = 65536;

struct KernelTimer {
    std::string name;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
    int64_t launches = 0, dropped = 0;
};

}  // namespace

struct kv_pool {
    int32_t num_blocks = 0, block_size = 0, kv_heads = 0, head_dim = 0, dtype = 0, elem = 0;
    bool host_only = true;
    int device = 0;
    void* k_pool = nullptr;
    void* v_pool = nullptr;
    float* scales = nullptr;   // device: k_scale[H], v_scale[H], k_inv[H], v_inv[H]
    void* zero_tile = nullptr; // device: kZeroTileBytes of zeros (paged_prefill reads absent tokens here)
    uint64_t* tags = nullptr;  // device, INT8 pools: per slot, (call epoch << 32 | token) of its last append
    uint32_t epoch = 0;        // INT8 pools: epoch of the last append call
    uint64_t pool_bytes = 0, block_bytes = 0;
    int32_t partition_tokens = 0;

    std::deque<int32_t> free_list;
    std::vector<int32_t> ref;
    std::unordered_map<int32_t, Seq> seqs;
    int32_t next_id = 0;
    int32_t shared = 0;        // blocks with refcount >= 2
    // copy-on-write: (source, destination) block copies owed to the device,
    // performed by the next kv_append / paged_decode / kv_apply_copies
    std::vector<std::pair<int32_t, int32_t>> pending;

    // prefix cache: content key -> block, and per cached block its key and
    // tokens; cached blocks nobody holds wait in `lru` (oldest release first)
    std::unordered_map<uint64_t, int32_t> cache;
    std::vector<uint64_t> block_key;
    std::vector<char> is_cached;
    std::vector<std::array<int32_t, 16>> block_tokens;
    std::list<int32_t> lru;
    std::vector<std::list<int32_t>::iterator> lru_pos;

    // device staging of swaps, grown on demand
    void* staging = nullptr;
    size_t staging_bytes = 0;

    bool profiling = false;
    std::vector<KernelTimer> timers;
    std::vector<hipEvent_t> spare_events;
};

namespace {

bool dtype_known(int32_t dt) { return dt >= PKV_F32 && dt <= PKV_INT8_MINMAX; }

int elem_of(int32_t dt) { return pkv::elem_bytes(dt); }

void ref_inc(kv_pool* p, int32_t b) {
    if (++p->ref[b] == 2) ++p->shared;
}

void ref_dec(kv_pool* p, int32_t b) {
    if (p->ref[b]-- == 2) --p->shared;
}

// Blocks a reservation can draw on: uncached free blocks, then cached blocks
// nobody holds (evicted least recently released first).
size_t available(const kv_pool* p) { return p->free_list.size() + p->lru.size(); }

int32_t take_block(kv_pool* p) {
    int32_t b;
    if (!p->free_list.empty()) {
        b = p->free_list.front();
        p->free_list.pop_front();
    } else {
        b = p->lru.front();                    // evict: forget its content key
        p->lru.pop_front();
        p->cache.erase(p->block_key[b]);
        p->is_cached[b] = 0;
    }
    p->ref[b] = 1;
    return b;
}

// A block's last holder let go: cached blocks stay findable until evicted.
void release_block(kv_pool* p, int32_t b) {
    if (!p->is_cached.empty() && p->is_cached[b]) {
        p->lru.push_back(b);
        p->lru_pos[b] = std::prev(p->lru.end());
    } else {
        p->free_list.push_back(b);
    }
}

int create_common(int32_t num_blocks, int32_t block_size, int32_t kv_heads, int32_t head_dim,
                  int32_t dtype, const int32_t* order, kv_pool_t** out, bool host_only) {
    if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0 || kv_heads <= 0 || head_dim <= 0)
        return fail(PKV_ERR_INVALID_ARG, "sizes must be > 0 (num_blocks %d, block_size %d, kv_heads %d, head_dim %d)",
                    num_blocks, block_size, kv_heads, head_dim);
    if (!dtype_known(dtype)) return fail(PKV_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (block_size != pkv::kBlock) return fail(PKV_ERR_UNSUPPORTED, "block_size must be 16, got %d", block_size);
    if (head_dim != 16 && head_dim != 64 && head_dim != 128)
        return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 16, 64 or 128, got %d", head_dim);
    if ((int64_t)num_blocks * block_size > std::numeric_limits<int32_t>::max())
        return fail(PKV_ERR_INVALID_ARG, "num_blocks * block_size must fit int32 slots");
    if (kv_heads > 65535) return fail(PKV_ERR_INVALID_ARG, "kv_heads too large");
    std::vector<int32_t> ord(num_blocks);
    if (order) {
        std::vector<char> seen(num_blocks, 0);
        for (int32_t i = 0; i < num_blocks; ++i) {
            const int32_t b = order[i];
            if (b < 0 || b >= num_blocks || seen[b])
                return fail(PKV_ERR_INVALID_ARG, "initial_free_order is not a permutation of 0..%d", num_blocks - 1);
            seen[b] = 1;
            ord[i] = b;
        }
    } else {
        for (int32_t i = 0; i < num_blocks; ++i) ord[i] = i;
    }
    kv_pool* p = new (std::nothrow) kv_pool();
    if (!p) return fail(PKV_ERR_DEVICE, "host allocation failed");
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    p->kv_heads = kv_heads;
    p->head_dim = head_dim;
    p->dtype = dtype;
    p->elem = elem_of(dtype);
    p->host_only = host_only;
    p->block_bytes = (uint64_t)pkv::tile_bytes(dtype, head_dim);
    p->pool_bytes = (uint64_t)num_blocks * kv_heads * p->block_bytes;
    p->free_list.assign(ord.begin(), ord.end());
    p->ref.assign(num_blocks, 0);
    if (!host_only) {
        hipError_t e = hipGetDevice(&p->device);
        if (e == hipSuccess) e = hipMalloc(&p->k_pool, p->pool_bytes);
        if (e == hipSuccess) e = hipMalloc(&p->v_pool, p->pool_bytes);
        if (e == hipSuccess) e = hipMemset(p->k_pool, 0, p->pool_bytes);
        if (e == hipSuccess) e = hipMemset(p->v_pool, 0, p->pool_bytes);
        if (e == hipSuccess) e = hipMalloc(&p->zero_tile, pkv::kZeroTileBytes);
        if (e == hipSuccess) e = hipMemset(p->zero_tile, 0, pkv::kZeroTileBytes);
        if (e == hipSuccess && dtype == PKV_INT8_MINMAX) {
            e = hipMalloc(&p->tags, sizeof(uint64_t) * num_blocks * block_size);
            if (e == hipSuccess) e = hipMemset(p->tags, 0, sizeof(uint64_t) * num_blocks * block_size);
        }
        if (e == hipSuccess && dtype == PKV_FP8_E4M3) {
            e = hipMalloc(&p->scales, sizeof(float) * 4 * kv_heads);
            if (e == hipSuccess) {
                std::vector<float> ones(4 * kv_heads, 1.0f);
                e = hipMemcpy(p->scales, ones.data(), sizeof(float) * 4 * kv_heads, hipMemcpyHostToDevice);
            }
        }
        if (e != hipSuccess) {
            int rc = hip_fail(e, "pool device allocation");
            kv_pool_destroy(p);
            return rc;
        }
    }
    *out = p;
    return ok();
}

Seq* find_seq(kv_pool* p, int32_t id) {
    auto it = p->seqs.find(id);
    return it == p->seqs.end() ? nullptr : &it->second;
}

const Seq* find_seq(const kv_pool* p, int32_t id) {
    auto it = p->seqs.find(id);
    return it == p->seqs.end() ? nullptr : &it->second;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// ---------------------------------------------------------------- profiling
hipEvent_t take_event(kv_pool* p) {
    if (!p->spare_events.empty()) {
        hipEvent_t e = p->spare_events.back();
        p->spare_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

KernelTimer& timer_for(kv_pool* p, const char* name) {
    for (auto& t : p->timers)
        if (t.name == name) return t;
    p->timers.push_back(KernelTimer{name, {}, 0, 0});
    return p->timers.back();
}

// Launch `fn` on `stream`; when profiling, the kernels it launches record an
// event pair at their own start and end (launch_kernel).
template <class F>
hipError_t timed_launch(kv_pool* p, const char* name, hipStream_t stream, F&& fn) {
    if (!p->profiling) return fn();
    KernelTimer& t = timer_for(p, name);
    ++t.launches;
    if ((int)t.pending.size() >= kMaxTimed) {
        ++t.dropped;
        return fn();
    }
    hipEvent_t a = take_event(p), b = take_event(p);
    if (!a || !b) {
        ++t.dropped;
        if (a) p->spare_events.push_back(a);
        if (b) p->spare_events.push_back(b);
        return fn();
    }
    pkv::arm_launch_events(a, b);              // the launches inside fn record them
    const hipError_t e = fn();
    if (!pkv::disarm_launch_events()) {        // nothing launched: no timing for this call
        ++t.dropped;
        p->spare_events.push_back(a);
        p->spare_events.push_back(b);
        return e;
    }
    t.pending.emplace_back(a, b);
    return e;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

uint64_t kv_cache_bytes(int32_t layers, int32_t kv_heads, int32_t head_dim, int32_t elem_bytes,
                        int64_t tokens, int64_t seqs) {
    if (layers <= 0 || kv_heads <= 0 || head_dim <= 0 || elem_bytes <= 0 || tokens < 0 || seqs < 0) return 0;
    return 2ull * (uint64_t)layers * (uint64_t)kv_heads * (uint64_t)head_dim * (uint64_t)elem_bytes *
           (uint64_t)tokens * (uint64_t)seqs;
}

int kv_pool_create(int32_t num_blocks, int32_t block_size, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                   const int32_t* initial_free_order, kv_pool_t** out) {
    try {
        return create_common(num_blocks, block_size, kv_heads, head_dim, dtype, initial_free_order, out, false);
    } catch (...) {
        return fail(PKV_ERR_DEVICE, "kv_pool_create: host exception");
    }
}

int kv_pool_create_host_only(int32_t num_blocks, int32_t block_size, int32_t kv_heads, int32_t head_dim,
                             int32_t dtype, const int32_t* initial_free_order, kv_pool_t** out) {
    try {
        return create_common(num_blocks, block_size, kv_heads, head_dim, dtype, initial_free_order, out, true);
    } catch (...) {
        return fail(PKV_ERR_DEVICE, "kv_pool_create_host_only: host exception");
    }
}

int kv_pool_destroy(kv_pool_t* pool) {
    if (!pool) return ok();
    if (!pool->host_only) {
        // teardown: a failing release has nowhere to be reported, so errors are dropped
        for (auto& t : pool->timers)
            for (auto& ev : t.pending) {
                (void)hipEventDestroy(ev.first);
                (void)hipEventDestroy(ev.second);
            }
        for (hipEvent_t e : pool->spare_events) (void)hipEventDestroy(e);
        for (void* mem : {pool->k_pool, pool->v_pool, static_cast<void*>(pool->scales), pool->zero_tile,
                          static_cast<void*>(pool->tags), pool->staging})
            if (mem) (void)hipFree(mem);
    }
    delete pool;
    return ok();
}

int kv_pool_info(const kv_pool_t* p, kv_pool_info_t* out) {
    if (!p || !out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    std::memset(out, 0, sizeof *out);
    out->k_pool = p->k_pool;
    out->v_pool = p->v_pool;
    out->k_scale = p->scales;
    out->v_scale = p->scales ? p->scales + p->kv_heads : nullptr;
    out->pool_bytes = p->pool_bytes;
    out->block_bytes = p->block_bytes;
    out->total_bytes = p->host_only ? 0
                                    : 2 * p->pool_bytes + (p->scales ? 4ull * sizeof(float) * p->kv_heads : 0) +
                                          (uint64_t)pkv::kZeroTileBytes +
                                          (p->tags ? sizeof(uint64_t) * p->num_blocks * p->block_size : 0);
    out->num_blocks = p->num_blocks;
    out->block_size = p->block_size;
    out->kv_heads = p->kv_heads;
    out->head_dim = p->head_dim;
    out->dtype = p->dtype;
    out->elem_bytes = p->elem;
    out->free_blocks = (int32_t)p->free_list.size();
    out->used_blocks = p->num_blocks - out->free_blocks - (int32_t)p->lru.size();
    out->shared_blocks = p->shared;
    out->live_seqs = (int32_t)p->seqs.size();
    out->host_only = p->host_only ? 1 : 0;
    out->partition_tokens = p->partition_tokens;
    out->cached_blocks = (int32_t)p->cache.size();
    out->evictable_blocks = (int32_t)p->lru.size();
    return ok();
}

int kv_pool_set_fp8_scales(kv_pool_t* p, const float* k_scale, const float* v_scale) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    if (p->dtype != PKV_FP8_E4M3) return fail(PKV_ERR_STATE, "scales apply to FP8 pools only");
    if (!k_scale || !v_scale) return fail(PKV_ERR_INVALID_ARG, "NULL scale array");
    const int H = p->kv_heads;
    std::vector<float> h(4 * H);
    for (int i = 0; i < H; ++i) {
        if (!(k_scale[i] > 0.0f) || !std::isfinite(k_scale[i]) || !(v_scale[i] > 0.0f) || !std::isfinite(v_scale[i]))
            return fail(PKV_ERR_INVALID_ARG, "scales must be finite and > 0 (head %d)", i);
        h[i] = k_scale[i];
        h[H + i] = v_scale[i];
        h[2 * H + i] = 1.0f / k_scale[i];
        h[3 * H + i] = 1.0f / v_scale[i];
    }
    if (p->host_only) return ok();
    hipError_t e = hipMemcpy(p->scales, h.data(), sizeof(float) * 4 * H, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "scale upload");
    return ok();
}

// ------------------------------------------------------------------ sequences
int kv_seq_create(kv_pool_t* p, int32_t* seq_id) {
    if (!p || !seq_id) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    if (p->next_id == std::numeric_limits<int32_t>::max()) return fail(PKV_ERR_OUT_OF_RANGE, "sequence ids exhausted");
    try {
        const int32_t id = p->next_id++;
        p->seqs.emplace(id, Seq{});
        *seq_id = id;
    } catch (...) {
        return fail(PKV_ERR_DEVICE, "host allocation failed");
    }
    return ok();
}

int kv_seq_reserve(kv_pool_t* p, int32_t seq, int32_t n_tokens, int32_t* slots) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    Seq* s = find_seq(p, seq);
    if (!s) return fail(PKV_ERR_STATE, "unknown or freed sequence %d", seq);
    if (s->swapped) return fail(PKV_ERR_STATE, "sequence %d is swapped out", seq);
    if (n_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "n_tokens < 0");
    if (n_tokens > 0 && !slots) return fail(PKV_ERR_INVALID_ARG, "slot_mapping_out is NULL");
    const int64_t new_len = (int64_t)s->len + n_tokens;
    if (new_len > std::numeric_limits<int32_t>::max()) return fail(PKV_ERR_OUT_OF_RANGE, "sequence length overflow");
    const int bs = p->block_size;
    // Writing into a partly filled block that another table also holds: copy it
    // first (copy-on-write), so the other holders keep their contents.
    const bool cow = n_tokens > 0 && s->len % bs != 0 && p->ref[s->blocks.back()] > 1;
    const int64_t need = (new_len + bs - 1) / bs - (int64_t)s->blocks.size() + (cow ? 1 : 0);
    if (need > (int64_t)available(p))
        return fail(PKV_ERR_NO_BLOCKS, "need %lld blocks, %zu available", (long long)need, available(p));
    try {
        s->blocks.reserve(s->blocks.size() + (size_t)need);
        if (cow) p->pending.reserve(p->pending.size() + 1);
    } catch (...) {
        return fail(PKV_ERR_DEVICE, "host allocation failed");
    }
    int64_t taken = 0;
    if (cow) {
        const int32_t old = s->blocks.back();
        const int32_t fresh = take_block(p);
        ref_dec(p, old);                       // stays >= 1: the block was shared
        s->blocks.back() = fresh;
        p->pending.emplace_back(old, fresh);
        ++taken;
    }
    for (; taken < need; ++taken) s->blocks.push_back(take_block(p));
    for (int64_t pos = s->len, i = 0; pos < new_len; ++pos, ++i)
        slots[i] = s->blocks[pos / bs] * bs + (int32_t)(pos % bs);
    s->len = (int32_t)new_len;
    return ok();
}

int kv_batch_reserve(kv_pool_t* p, const int32_t* seqs, int32_t n, const int32_t* n_tokens, int32_t* slots) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n < 0");
    if (n == 0) return ok();
    if (!seqs || !slots) return fail(PKV_ERR_INVALID_ARG, "NULL array");
    const int bs = p->block_size;
    // Dry run, replaying kv_seq_reserve's rules: lengths after each request
    // (sequences may repeat), copy-on-write departures (which lower the shared
    // block's count for later requests), total blocks needed.
    int64_t need = 0;
    try {
        std::unordered_map<int32_t, int64_t> len;        // sequence -> simulated length
        std::unordered_map<int32_t, int32_t> left;       // block -> holders that copied away
        std::unordered_map<int32_t, bool> own_last;      // sequence -> last block is now private
        for (int32_t i = 0; i < n; ++i) {
            const int32_t k = n_tokens ? n_tokens[i] : 1;
            if (k < 0) return fail(PKV_ERR_INVALID_ARG, "n_tokens[%d] < 0", i);
            const Seq* s = find_seq(p, seqs[i]);
            if (!s) return fail(PKV_ERR_STATE, "unknown or freed sequence %d", seqs[i]);
            if (s->swapped) return fail(PKV_ERR_STATE, "sequence %d is swapped out", seqs[i]);
            auto it = len.find(seqs[i]);
            const int64_t cur = it == len.end() ? s->len : it->second;
            const int64_t nxt = cur + k;
            if (nxt > std::numeric_limits<int32_t>::max()) return fail(PKV_ERR_OUT_OF_RANGE, "sequence length overflow");
            bool& priv = own_last[seqs[i]];
            if (k > 0 && cur % bs != 0 && !priv) {
                const int32_t last = s->blocks.back();
                if (p->ref[last] - left[last] > 1) {
                    ++need;
                    ++left[last];
                    priv = true;
                }
            }
            const int64_t grown = (nxt + bs - 1) / bs - (cur + bs - 1) / bs;
            if (grown > 0) priv = true;
            need += grown;
            len[seqs[i]] = nxt;
        }
    } catch (...) {
        return fail(PKV_ERR_DEVICE, "host allocation failed");
    }
    if (need > (int64_t)available(p))
        return fail(PKV_ERR_NO_BLOCKS, "batch needs %lld blocks, %zu available", (long long)need, available(p));
    int64_t o = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t k = n_tokens ? n_tokens[i] : 1;
        const int rc = kv_seq_reserve(p, seqs[i], k, slots + o);
        if (rc != PKV_OK) return rc;   // unreachable: the dry run checked every condition
        o += k;
    }
    return ok();
}

int kv_seq_fork(kv_pool_t* p, int32_t parent, int32_t n_shared, int32_t* child) {
    if (!p || !child) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    Seq* s = find_seq(p, parent);
    if (!s) return fail(PKV_ERR_STATE, "unknown or freed sequence %d", parent);
    if (s->swapped) return fail(PKV_ERR_STATE, "sequence %d is swapped out", parent);
    if (n_shared < 0 || n_shared > s->len)
        return fail(PKV_ERR_INVALID_ARG, "fork length %d must be in [0, parent length %d]", n_shared, s->len);
    if (p->next_id == std::numeric_limits<int32_t>::max()) return fail(PKV_ERR_OUT_OF_RANGE, "sequence ids exhausted");
    Seq c;
    try {
        c.blocks.assign(s->blocks.begin(), s->blocks.begin() + (n_shared + p->block_size - 1) / p->block_size);
        c.len = n_shared;
        const int32_t id = p->next_id;
        p->seqs.emplace(id, std::move(c));
        ++p->next_id;
        for (int32_t b : p->seqs[id].blocks) ref_inc(p, b);
        *child = id;
    } catch (...) {
        return fail(PKV_ERR_DEVICE, "host allocation failed");
    }
    return ok();
}

int kv_seq_free(kv_pool_t* p, int32_t seq) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    auto it = p->seqs.find(seq);
    if (it == p->seqs.end()) return fail(PKV_ERR_STATE, "unknown or freed sequence %d", seq);
    // deepest block first: a cached prefix chain then loses its tail before its root
    const std::vector<int32_t>& blocks = it->second.blocks;
    for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) {
        ref_dec(p, *b);
        if (p->ref[*b] == 0) release_block(p, *b);
    }
    p->seqs.erase(it);
    return ok();
}

int kv_seq_length(const kv_pool_t* p, int32_t seq, int32_t* len) {
    if (!p || !len) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    const Seq* s = find_seq(p, seq);
    if (!s) return fail(PKV_ERR_STATE, "unknown or freed sequence %d", seq);
    *len = s->len;
    return ok();
}

int kv_block_tables(const kv_pool_t* p, const int32_t* seqs, int32_t n, int32_t max_blocks, int32_t* tables,
                    int32_t* lens) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    if (n < 0 || max_blocks < 0) return fail(PKV_ERR_INVALID_ARG, "negative size");
    if (n > 0 && (!seqs || !lens || (max_blocks > 0 && !tables))) return fail(PKV_ERR_INVALID_ARG, "NULL array");
    for (int32_t i = 0; i < n; ++i) {
        const Seq* s = find_seq(p, seqs[i]);
        if (!s) return fail(PKV_ERR_STATE, "unknown or freed sequence %d", seqs[i]);
        if (s->swapped) return fail(PKV_ERR_STATE, "sequence %d is swapped out", seqs[i]);
        if ((int64_t)s->blocks.size() > max_blocks)
            return fail(PKV_ERR_OUT_OF_RANGE, "sequence %d has %zu blocks > max_blocks_per_seq %d", seqs[i],
                        s->blocks.size(), max_blocks);
    }
    for (int32_t i = 0; i < n; ++i) {
        const Seq* s = find_seq(p, seqs[i]);
        int32_t* row = tables + (int64_t)i * max_blocks;
        const int32_t nb = (int32_t)s->blocks.size();
        for (int32_t j = 0; j < nb; ++j) row[j] = s->blocks[j];
        for (int32_t j = nb; j < max_blocks; ++j) row[j] = -1;
        lens[i] = s->len;
    }
    return ok();
}

int kv_block_refcount(const kv_pool_t* p, int32_t block, int32_t* out) {
    if (!p || !out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    if (block < 0 || block >= p->num_blocks) return fail(PKV_ERR_INVALID_ARG, "block %d out of range", block);
    *out = p->ref[block];
    return ok();
}

int kv_free_list(const kv_pool_t* p, int32_t* out, int32_t cap, int32_t* n) {
    if (!p || !n) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    *n = (int32_t)p->free_list.size();
    if (cap < *n) return fail(PKV_ERR_OUT_OF_RANGE, "capacity %d < free list length %d", cap, *n);
    if (*n > 0 && !out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
    int32_t i = 0;
    for (int32_t b : p->free_list) out[i++] = b;
    return ok();
}

// ------------------------------------------------------------- prefix cache
uint64_t kv_block_hash(uint64_t parent, uint64_t ns, const int32_t* tokens) {
    // SplitMix64's output function (Steele, Lea, Flood 2014), folded over the
    // parent key, the namespace and the block's 16 tokens.
    auto mix = [](uint64_t x) {
        x += 0x9E3779B97F4A7C15ull;
        x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
        x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
        return x ^ (x >> 31);
    };
    uint64_t h = mix(parent ^ mix(ns));
    if (tokens)
        for (int i = 0; i < pkv::kBlock; ++i) h = mix(h ^ (uint64_t)(uint32_t)tokens[i]);
    return h;
}

int kv_prefix_register(kv_pool_t* p, int32_t seq, const int32_t* tokens, int32_t n_tokens, uint64_t ns,
                       int32_t* n_registered) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    const Seq* s = find_seq(p, seq);
    if (!s) return fail(PKV_ERR_STATE, "unknown or freed sequence %d", seq);
    if (s->swapped) return fail(PKV_ERR_STATE, "sequence %d is swapped out", seq);
    if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return fail(PKV_ERR_INVALID_ARG, "bad token array");
    if (n_tokens > s->len) return fail(PKV_ERR_OUT_OF_RANGE, "%d tokens given, sequence holds %d", n_tokens, s->len);
    const int bs = p->block_size;
    const int32_t nfull = n_tokens / bs;
    int32_t added = 0;
    try {
        if (p->is_cached.empty()) {
            p->is_cached.assign(p->num_blocks, 0);
            p->block_key.assign(p->num_blocks, 0);
            p->block_tokens.resize(p->num_blocks);
            p->lru_pos.resize(p->num_blocks);
        }
        uint64_t key = 0;
        for (int32_t i = 0; i < nfull; ++i) {
            key = kv_block_hash(key, ns, tokens + (int64_t)i * bs);
            const int32_t b = s->blocks[i];
            if (p->cache.count(key) || p->is_cached[b]) continue;   // content already cached, or block keyed
            p->cache.emplace(key, b);
            p->is_cached[b] = 1;
            p->block_key[b] = key;
            std::copy(tokens + (int64_t)i * bs, tokens + (int64_t)(i + 1) * bs, p->block_tokens[b].begin());
            ++added;
        }
    } catch (...) {
        return fail(PKV_ERR_DEVICE, "host allocation failed");
    }
    if (n_registered) *n_registered = added;
    return ok();
}

int kv_seq_create_cached(kv_pool_t* p, const int32_t* tokens, int32_t n_tokens, uint64_t ns, int32_t* seq_id,
                         int32_t* n_cached_tokens) {
    if (!p || !seq_id || !n_cached_tokens) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return fail(PKV_ERR_INVALID_ARG, "bad token array");
    if (p->next_id == std::numeric_limits<int32_t>::max()) return fail(PKV_ERR_OUT_OF_RANGE, "sequence ids exhausted");
    const int bs = p->block_size;
    Seq s;
    try {
        uint64_t key = 0;
        for (int32_t i = 0; (int64_t)(i + 1) * bs <= n_tokens; ++i) {
            key = kv_block_hash(key, ns, tokens + (int64_t)i * bs);
            auto it = p->cache.find(key);
            if (it == p->cache.end()) break;
            const int32_t b = it->second;
            if (!std::equal(tokens + (int64_t)i * bs, tokens + (int64_t)(i + 1) * bs, p->block_tokens[b].begin()))
                break;                                               // a key collision: never share it
            s.blocks.push_back(b);
        }
        const int32_t id = p->next_id;
        p->seqs.emplace(id, Seq{});
        ++p->next_id;
        for (int32_t b : s.blocks) {
            if (p->ref[b] == 0) {                                    // evictable: take it back
                p->lru.erase(p->lru_pos[b]);
                p->ref[b] = 1;
            } else {
                ref_inc(p, b);
            }
        }
        s.len = (int32_t)s.blocks.size() * bs;
        *n_cached_tokens = s.len;
        p->seqs[id] = std::move(s);
        *seq_id = id;
    } catch (...) {
        return fail(PKV_ERR_DEVICE, "host allocation failed");
    }
    return ok();
}

int kv_prefix_evict_all(kv_pool_t* p) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    for (int32_t b : p->lru) {
        p->cache.erase(p->block_key[b]);
        p->is_cached[b] = 0;
        p->free_list.push_back(b);
    }
    p->lru.clear();
    // blocks still held lose their keys now and go to the free list when released
    for (auto it = p->cache.begin(); it != p->cache.end();) {
        p->is_cached[it->second] = 0;
        it = p->cache.erase(it);
    }
    return ok();
}

int kv_pending_copies(const kv_pool_t* p, int32_t* src, int32_t* dst, int32_t cap, int32_t* n) {
    if (!p || !n) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    *n = (int32_t)p->pending.size();
    if (cap < *n) return fail(PKV_ERR_OUT_OF_RANGE, "capacity %d < %d pending copies", cap, *n);
    if (*n > 0 && (!src || !dst)) return fail(PKV_ERR_INVALID_ARG, "NULL array");
    for (int32_t i = 0; i < *n; ++i) {
        src[i] = p->pending[i].first;
        dst[i] = p->pending[i].second;
    }
    return ok();
}

}  // extern "C"

namespace {

// Perform the pending copy-on-write block copies on `stream` (both pools, all
// heads of each block) and clear the list.  Metadata-only pools just clear it.
int flush_copies(kv_pool* p, hipStream_t stream) {
    if (p->pending.empty()) return PKV_OK;
    if (!p->host_only) {
        for (size_t i = 0; i < p->pending.size(); i += pkv::kMaxCopiesPerLaunch) {
            pkv::CopyParams cp{};
            cp.n = (int32_t)std::min<size_t>(pkv::kMaxCopiesPerLaunch, p->pending.size() - i);
            for (int32_t j = 0; j < cp.n; ++j) {
                cp.src[j] = p->pending[i + j].first;
                cp.dst[j] = p->pending[i + j].second;
            }
            cp.k_pool = p->k_pool;
            cp.v_pool = p->v_pool;
            cp.block_bytes = (int64_t)p->kv_heads * p->block_bytes;
            hipError_t e = timed_launch(p, "kv_copy_blocks", stream, [&] { return pkv::launch_copy_blocks(cp, stream); });
            if (e != hipSuccess) return hip_fail(e, "kv_copy_blocks launch");
        }
    }
    p->pending.clear();
    return PKV_OK;
}

}  // namespace

extern "C" {

int kv_apply_copies(kv_pool_t* p, void* stream) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    const int rc = flush_copies(p, reinterpret_cast<hipStream_t>(stream));
    return rc == PKV_OK ? ok() : rc;
}

// ---------------------------------------------------------------- device work
int kv_append(kv_pool_t* p, const int32_t* slot_mapping, int32_t T, const void* k_new, const void* v_new,
              int32_t src_dtype, void* stream) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    if (T < 0) return fail(PKV_ERR_INVALID_ARG, "T < 0");
    if (!dtype_known(src_dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown src dtype %d", src_dtype);
    const bool pairing = (src_dtype == p->dtype && p->dtype != PKV_INT8_MINMAX) ||
                         (p->dtype == PKV_FP8_E4M3 && (src_dtype == PKV_BF16 || src_dtype == PKV_F32)) ||
                         (p->dtype == PKV_INT8_MINMAX &&
                          (src_dtype == PKV_BF16 || src_dtype == PKV_F16 || src_dtype == PKV_F32));
    if (!pairing) return fail(PKV_ERR_UNSUPPORTED, "cannot append dtype %d into a pool of dtype %d", src_dtype, p->dtype);
    if (T > 0 && (!slot_mapping || !k_new || !v_new)) return fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
    if (T > 0 && (!aligned16(k_new) || !aligned16(v_new))) return fail(PKV_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
    if ((int64_t)T * p->kv_heads * p->head_dim > (int64_t)1 << 40) return fail(PKV_ERR_INVALID_ARG, "T too large");
    if (p->host_only) return fail(PKV_ERR_STATE, "host-only pool has no device memory");
    if (T == 0) return ok();
    pkv::AppendParams a{};
    a.slots = slot_mapping;
    a.k_src = k_new;
    a.v_src = v_new;
    a.k_pool = p->k_pool;
    a.v_pool = p->v_pool;
    a.k_inv = p->scales ? p->scales + 2 * p->kv_heads : nullptr;
    a.v_inv = p->scales ? p->scales + 3 * p->kv_heads : nullptr;
    a.num_slots = (int64_t)p->num_blocks * p->block_size;
    a.T = T;
    a.H_kv = p->kv_heads;
    a.D = p->head_dim;
    a.src_dt = src_dtype;
    a.dst_dt = p->dtype;
    if (p->tags) {
        if (++p->epoch == 0) ++p->epoch;      // 0 marks a slot never written
        a.tags = p->tags;
        a.epoch = p->epoch;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int rc = flush_copies(p, s);       // copy-on-write before the new rows land
    if (rc != PKV_OK) return rc;
    hipError_t e = timed_launch(p, "kv_append", s, [&] { return pkv::launch_kv_append(a, s); });
    if (e != hipSuccess) return hip_fail(e, "kv_append launch");
    return ok();
}

}  // extern "C"

namespace {

int32_t resolve_partition(const kv_pool* p, int32_t B, int32_t H_q, int32_t max_len) {
    if (max_len <= 0) return 64;
    if (p->partition_tokens > 0) return p->partition_tokens;
    const int64_t G = H_q / p->kv_heads;
    const int64_t wg_cols = (int64_t)B * p->kv_heads * (G / pkv::decode_heads_per_wg((int32_t)G));
    // Contexts up to 4096 tokens with at least two (sequence, head group)
    // columns per CU run as one partition: a plain grid, no work list, no merge.
    if (max_len <= 4096 && wg_cols >= 512) return ((max_len + 63) / 64) * 64;
    // Otherwise the largest partition in [256, 8192] that still gives >= 2048
    // work items (two to three per resident workgroup).  Multi-partition
    // launches are scheduled longest-first from a work list, so a few long
    // partitions do not stretch the tail, and larger partitions mean fewer item
    // start-ups and less merging.
    int32_t P = 8192;
    while (P > 256 && wg_cols * ((max_len + P - 1) / P) < 2048) P /= 2;
    if (max_len <= P) P = ((max_len + 63) / 64) * 64;
    return P;
}

// Workspace of a launch that spans more than one partition (256-byte aligned
// sections): [schedule header][work list: B*max_parts (sequence, partition)]
// [(m, l): B*H_q*max_parts float2][partial outputs: B*H_q*max_parts*D float].
struct WsLayout {
    size_t items = 0, ml = 0, o = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Partitions per context the workspace holds.  With the automatic partition
// it is twice the host's count, so the plan kernel may pick a shorter
// partition when every context has the same length.
int64_t parts_capacity(const kv_pool* p, int32_t max_len, int32_t P) {
    const int64_t parts = max_len <= 0 ? 1 : (max_len + (int64_t)P - 1) / P;
    return parts <= 1 || p->partition_tokens > 0 ? parts : 2 * parts;
}

WsLayout workspace_for(const kv_pool* p, int32_t B, int32_t H_q, int32_t max_len, int32_t P) {
    WsLayout L;
    const int64_t parts = parts_capacity(p, max_len, P);
    if (parts <= 1 || B <= 0) return L;
    const size_t slots = (size_t)B * H_q * parts;
    L.items = 256;
    L.ml = L.items + align256((size_t)B * parts * 2 * sizeof(int32_t));
    L.o = L.ml + align256(slots * 2 * sizeof(float));
    L.total = L.o + slots * p->head_dim * sizeof(float);
    return L;
}

}  // namespace

extern "C" {

int paged_decode_set_partition(kv_pool_t* p, int32_t partition_tokens) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    if (partition_tokens != 0 && (partition_tokens < 64 || partition_tokens > (1 << 20) || partition_tokens % 64 != 0))
        return fail(PKV_ERR_INVALID_ARG, "partition must be 0 or a multiple of 64 in [64, 1048576]");
    p->partition_tokens = partition_tokens;
    return ok();
}

int32_t paged_decode_partition_tokens(const kv_pool_t* p, int32_t B, int32_t H_q, int32_t max_context_len) {
    if (!p || H_q <= 0 || H_q % p->kv_heads != 0) return 0;
    return resolve_partition(p, B, H_q, max_context_len);
}

size_t paged_decode_workspace_bytes(const kv_pool_t* p, int32_t B, int32_t H_q, int32_t max_context_len) {
    if (!p || B <= 0 || H_q <= 0 || H_q % p->kv_heads != 0) return 0;
    const int32_t max_len = max_context_len;
    return workspace_for(p, B, H_q, max_len, resolve_partition(p, B, H_q, max_len)).total;
}

}  // extern "C"

namespace {

// paged_decode and paged_decode_noalloc.  With `noalloc` the workspace
// arguments are ignored and the library's fixed device scratch serves instead.
int decode_impl(kv_pool_t* p, const void* q, int32_t q_dtype, int32_t B, int32_t H_q, const int32_t* block_tables,
                int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len, float scale,
                void* out, void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    if (B < 0 || B > 65535) return fail(PKV_ERR_INVALID_ARG, "B must be in [0, 65535], got %d", B);
    if (H_q <= 0 || H_q % p->kv_heads != 0)
        return fail(PKV_ERR_INVALID_ARG, "H_q (%d) must be a positive multiple of kv_heads (%d)", H_q, p->kv_heads);
    if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be > 0");
    if (max_context_len < 0) return fail(PKV_ERR_INVALID_ARG, "max_context_len < 0");
    if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite");
    if (!dtype_known(q_dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown q dtype %d", q_dtype);
    const int32_t G = H_q / p->kv_heads;
    if (!pkv::decode_supported(p->dtype, q_dtype, p->head_dim, G))
        return fail(PKV_ERR_UNSUPPORTED, "no decode kernel for pool dtype %d, q dtype %d, head_dim %d, group %d",
                    p->dtype, q_dtype, p->head_dim, G);
    if ((int64_t)p->kv_heads * (G / pkv::decode_heads_per_wg(G)) > 65535)
        return fail(PKV_ERR_INVALID_ARG, "too many query heads for one launch");
    if (B > 0 && (!q || !out || !block_tables || !context_lens)) return fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
    if (B > 0 && (int64_t)max_blocks_per_seq * B > ((int64_t)1 << 40)) return fail(PKV_ERR_INVALID_ARG, "tables too large");
    if (B > 0 && (!aligned16(q) || !aligned16(out))) return fail(PKV_ERR_INVALID_ARG, "q/out must be 16-byte aligned");
    const int32_t max_len = (int32_t)std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * p->block_size);
    const int32_t P = resolve_partition(p, B, H_q, max_len);
    if (max_len > 0 && (max_len + (int64_t)P - 1) / P > (1 << 29))
        return fail(PKV_ERR_INVALID_ARG, "partition of %d tokens is too small for %d tokens", P, max_len);
    const WsLayout ws = workspace_for(p, B, H_q, max_len, P);
    const size_t need = ws.total;
    if (noalloc) {
        if (need > pkv::kNoAllocScratchBytes)
            return fail(PKV_ERR_OUT_OF_RANGE, "these sizes need %zu bytes of scratch; the fixed scratch holds %zu",
                        need, pkv::kNoAllocScratchBytes);
        if (p->host_only) return fail(PKV_ERR_STATE, "host-only pool has no device memory");
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            int cur = -1;
            hipError_t e = hipGetDevice(&cur);
            if (e != hipSuccess) return hip_fail(e, "current device");
            if (cur != p->device)
                return fail(PKV_ERR_INVALID_ARG, "current device %d is not the pool's device %d", cur, p->device);
            e = pkv::noalloc_scratch(cur, &workspace);
            if (e != hipSuccess) return hip_fail(e, "decode scratch address");
            workspace_bytes = pkv::kNoAllocScratchBytes;
        }
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PKV_ERR_INVALID_ARG, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(PKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (p->host_only) return fail(PKV_ERR_STATE, "host-only pool has no device memory");
    if (B == 0) return ok();

    pkv::DecodeParams d{};
    d.k_pool = p->k_pool;
    d.v_pool = p->v_pool;
    d.k_scale = p->scales;
    d.v_scale = p->scales ? p->scales + p->kv_heads : nullptr;
    d.q = q;
    d.out = out;
    d.tables = block_tables;
    d.lens = context_lens;
    char* wsb = reinterpret_cast<char*>(workspace);
    d.sched = need ? reinterpret_cast<int32_t*>(wsb) : nullptr;
    d.items = need ? reinterpret_cast<int2*>(wsb + ws.items) : nullptr;
    d.ws_ml = need ? reinterpret_cast<float*>(wsb + ws.ml) : nullptr;
    d.ws_o = need ? reinterpret_cast<float*>(wsb + ws.o) : nullptr;
    d.B = B;
    d.H_q = H_q;
    d.H_kv = p->kv_heads;
    d.G = G;
    d.D = p->head_dim;
    d.num_blocks = p->num_blocks;
    d.max_blocks = max_blocks_per_seq;
    d.max_len = max_len;
    d.part_tokens = P;
    d.max_parts = (int32_t)parts_capacity(p, max_len, P);
    d.choose_parts = p->partition_tokens == 0;
    d.head_groups = p->kv_heads * (G / pkv::decode_heads_per_wg(G));
    if (need) {
        const int64_t upper = (int64_t)B * d.max_parts * d.head_groups;
        d.grid_wgs = (int32_t)std::min<int64_t>(upper, pkv::decode_resident_workgroups(p->dtype, q_dtype, p->head_dim, G));
    }
    d.kv_dt = p->dtype;
    d.q_dt = q_dtype;
    d.scale = scale;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int rc = flush_copies(p, s);       // tables may point at copied blocks
    if (rc != PKV_OK) return rc;
    hipError_t e = hipSuccess;
    if (d.items) {
        e = timed_launch(p, "paged_decode_plan", s, [&] { return pkv::launch_decode_plan(d, s); });
        if (e != hipSuccess) return hip_fail(e, "paged_decode_plan launch");
    }
    e = timed_launch(p, "paged_decode_partition", s, [&] { return pkv::launch_decode_partition(d, s); });
    if (e != hipSuccess) return hip_fail(e, "paged_decode_partition launch");
    if (d.max_parts > 1) {
        e = timed_launch(p, "paged_decode_reduce", s, [&] { return pkv::launch_decode_reduce(d, s); });
        if (e != hipSuccess) return hip_fail(e, "paged_decode_reduce launch");
    }
    return ok();
}

}  // namespace

extern "C" {

int paged_decode(kv_pool_t* p, const void* q, int32_t q_dtype, int32_t B, int32_t H_q, const int32_t* block_tables,
                 int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len, float scale,
                 void* out, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(p, q, q_dtype, B, H_q, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                       scale, out, workspace, workspace_bytes, stream, false);
}

int paged_decode_noalloc(kv_pool_t* p, const void* q, int32_t q_dtype, int32_t B, int32_t H_q,
                         const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t max_context_len, float scale, void* out, void* stream) {
    return decode_impl(p, q, q_dtype, B, H_q, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                       scale, out, nullptr, 0, stream, true);
}

int paged_prefill(kv_pool_t* p, const void* q, int32_t q_dtype, int32_t n_seqs, int32_t H_q, const int32_t* q_start,
                  int32_t total_q, int32_t max_q_len, const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, float scale, int32_t causal, void* out, void* stream) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    if (n_seqs < 0 || n_seqs > 65535) return fail(PKV_ERR_INVALID_ARG, "n_seqs must be in [0, 65535], got %d", n_seqs);
    if (H_q <= 0 || H_q % p->kv_heads != 0)
        return fail(PKV_ERR_INVALID_ARG, "H_q (%d) must be a positive multiple of kv_heads (%d)", H_q, p->kv_heads);
    if (total_q < 0 || max_q_len < 0) return fail(PKV_ERR_INVALID_ARG, "negative query count");
    if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be > 0");
    if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite");
    if (!dtype_known(q_dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown q dtype %d", q_dtype);
    if (!pkv::prefill_supported(p->dtype, q_dtype, p->head_dim))
        return fail(PKV_ERR_UNSUPPORTED, "no prefill kernel for pool dtype %d, q dtype %d, head_dim %d", p->dtype,
                    q_dtype, p->head_dim);
    const int32_t G = H_q / p->kv_heads;
    const int32_t gs = pkv::prefill_heads_per_group(G);
    if ((int64_t)p->kv_heads * (G / gs) > 65535) return fail(PKV_ERR_INVALID_ARG, "too many query heads for one launch");
    if (pkv::prefill_workgroups(G, p->kv_heads, n_seqs, max_q_len) > INT32_MAX)
        return fail(PKV_ERR_INVALID_ARG, "max_q_len too large");
    const bool work = n_seqs > 0 && total_q > 0 && max_q_len > 0;
    if (work && (!q || !out || !q_start || !block_tables || !context_lens))
        return fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
    if (work && (int64_t)max_blocks_per_seq * n_seqs > ((int64_t)1 << 40))
        return fail(PKV_ERR_INVALID_ARG, "tables too large");
    if (work && (!aligned16(q) || !aligned16(out))) return fail(PKV_ERR_INVALID_ARG, "q/out must be 16-byte aligned");
    if (p->host_only) return fail(PKV_ERR_STATE, "host-only pool has no device memory");
    if (!work) return ok();

    pkv::PrefillParams d{};
    d.k_pool = p->k_pool;
    d.v_pool = p->v_pool;
    d.k_scale = p->scales;
    d.v_scale = p->scales ? p->scales + p->kv_heads : nullptr;
    d.q = q;
    d.out = out;
    d.q_start = q_start;
    d.tables = block_tables;
    d.lens = context_lens;
    d.zero_tile = p->zero_tile;
    d.n_seqs = n_seqs;
    d.total_q = total_q;
    d.H_q = H_q;
    d.H_kv = p->kv_heads;
    d.G = G;
    d.D = p->head_dim;
    d.num_blocks = p->num_blocks;
    d.max_blocks = max_blocks_per_seq;
    d.gs = gs;
    d.kv_dt = p->dtype;
    d.q_dt = q_dtype;
    d.causal = causal != 0;
    d.scale = scale;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int rc = flush_copies(p, s);       // tables may point at copied blocks
    if (rc != PKV_OK) return rc;
    hipError_t e = timed_launch(p, "paged_prefill", s, [&] { return pkv::launch_prefill(d, max_q_len, s); });
    if (e != hipSuccess) return hip_fail(e, "paged_prefill launch");
    return ok();
}

}  // extern "C"

namespace {

// Device staging of at least `bytes` for a swap (the pool keeps the largest so far).
int ensure_staging(kv_pool* p, size_t bytes) {
    if (p->staging_bytes >= bytes) return PKV_OK;
    if (p->staging) {
        hipError_t e = hipFree(p->staging);
        p->staging = nullptr;
        p->staging_bytes = 0;
        if (e != hipSuccess) return hip_fail(e, "staging release");
    }
    hipError_t e = hipMalloc(&p->staging, bytes);
    if (e != hipSuccess) {
        p->staging = nullptr;
        return hip_fail(e, "swap staging allocation");
    }
    p->staging_bytes = bytes;
    return PKV_OK;
}

// Move the blocks `ids` (logical order) between the pools and the staging buffer.
hipError_t move_blocks(kv_pool* p, const std::vector<int32_t>& ids, bool to_pool, hipStream_t s) {
    pkv::MoveParams mp{};
    mp.k_pool = p->k_pool;
    mp.v_pool = p->v_pool;
    mp.staging = reinterpret_cast<char*>(p->staging);
    mp.block_bytes = (int64_t)p->kv_heads * p->block_bytes;    // a whole block: every KV head's tile
    mp.to_pool = to_pool ? 1 : 0;
    for (size_t i = 0; i < ids.size(); i += pkv::kMaxCopiesPerLaunch) {
        const size_t n = std::min<size_t>(pkv::kMaxCopiesPerLaunch, ids.size() - i);
        for (size_t k = 0; k < n; ++k) mp.ids[k] = ids[i + k];
        mp.n = (int32_t)n;
        mp.first = (int64_t)i;
        hipError_t e = pkv::launch_move_blocks(mp, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

size_t swap_bytes_of(const kv_pool* p, int32_t len) {
    return (size_t)((len + p->block_size - 1) / p->block_size) * 2 * p->kv_heads * p->block_bytes;
}

}  // namespace

extern "C" {

int kv_seq_swap_bytes(const kv_pool_t* p, int32_t seq, size_t* bytes) {
    if (!p || !bytes) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    const Seq* s = find_seq(p, seq);
    if (!s) return fail(PKV_ERR_STATE, "unknown or freed sequence %d", seq);
    *bytes = swap_bytes_of(p, s->len);
    return ok();
}

int kv_seq_swap_out(kv_pool_t* p, int32_t seq, void* host_dst, size_t bytes, void* stream) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    Seq* s = find_seq(p, seq);
    if (!s) return fail(PKV_ERR_STATE, "unknown or freed sequence %d", seq);
    if (s->swapped) return fail(PKV_ERR_STATE, "sequence %d is already swapped out", seq);
    const size_t need = swap_bytes_of(p, s->len);
    if (!p->host_only && bytes < need)
        return fail(PKV_ERR_INVALID_ARG, "swap buffer of %zu bytes, %zu needed", bytes, need);
    if (need > 0 && !host_dst && !p->host_only) return fail(PKV_ERR_INVALID_ARG, "host_dst is NULL");
    if (need > 0 && !p->host_only) {
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        int rc = flush_copies(p, st);                  // the blocks may be owed a copy
        if (rc == PKV_OK) rc = ensure_staging(p, need);
        if (rc != PKV_OK) return rc;
        hipError_t e = move_blocks(p, s->blocks, false, st);
        if (e == hipSuccess) e = hipMemcpyAsync(host_dst, p->staging, need, hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e, "swap-out copy");
    }
    for (auto b = s->blocks.rbegin(); b != s->blocks.rend(); ++b) {   // as kv_seq_free: deepest first
        ref_dec(p, *b);
        if (p->ref[*b] == 0) release_block(p, *b);
    }
    s->blocks.clear();
    s->swapped = true;
    return ok();
}

int kv_seq_swap_in(kv_pool_t* p, int32_t seq, const void* host_src, size_t bytes, void* stream) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    Seq* s = find_seq(p, seq);
    if (!s) return fail(PKV_ERR_STATE, "unknown or freed sequence %d", seq);
    if (!s->swapped) return fail(PKV_ERR_STATE, "sequence %d is not swapped out", seq);
    const size_t need = swap_bytes_of(p, s->len);
    if (!p->host_only && bytes < need)
        return fail(PKV_ERR_INVALID_ARG, "swap buffer of %zu bytes, %zu needed", bytes, need);
    if (need > 0 && !host_src && !p->host_only) return fail(PKV_ERR_INVALID_ARG, "host_src is NULL");
    const size_t nb = (size_t)((s->len + p->block_size - 1) / p->block_size);
    if (nb > available(p)) return fail(PKV_ERR_NO_BLOCKS, "swap-in needs %zu blocks, %zu available", nb, available(p));
    std::vector<int32_t> blocks;
    try {
        blocks.reserve(nb);
    } catch (...) {
        return fail(PKV_ERR_DEVICE, "host allocation failed");
    }
    for (size_t i = 0; i < nb; ++i) blocks.push_back(take_block(p));
    if (need > 0 && !p->host_only) {
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        int rc = flush_copies(p, st);
        if (rc == PKV_OK) rc = ensure_staging(p, need);
        hipError_t e = hipSuccess;
        if (rc == PKV_OK) {
            e = hipMemcpyAsync(p->staging, host_src, need, hipMemcpyHostToDevice, st);
            if (e == hipSuccess) e = move_blocks(p, blocks, true, st);
            if (e == hipSuccess) e = hipStreamSynchronize(st);
            if (e != hipSuccess) rc = hip_fail(e, "swap-in copy");
        }
        if (rc != PKV_OK) {                            // give the blocks back; the sequence stays out
            for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) {
                ref_dec(p, *b);
                if (p->ref[*b] == 0) release_block(p, *b);
            }
            return rc;
        }
    }
    s->blocks = std::move(blocks);
    s->swapped = false;
    return ok();
}

int kv_pool_copy_to_host(const kv_pool_t* p, void* k_dst, void* v_dst) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    if (p->host_only) return fail(PKV_ERR_STATE, "host-only pool has no device memory");
    const int rc = flush_copies(const_cast<kv_pool*>(p), nullptr);
    if (rc != PKV_OK) return rc;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess && k_dst) e = hipMemcpy(k_dst, p->k_pool, p->pool_bytes, hipMemcpyDeviceToHost);
    if (e == hipSuccess && v_dst) e = hipMemcpy(v_dst, p->v_pool, p->pool_bytes, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "pool read-back");
    return ok();
}

int pkv_profile_enable(kv_pool_t* p, int32_t on) {
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
    if (p->host_only && on) return fail(PKV_ERR_STATE, "host-only pool launches no kernels");
    p->profiling = on != 0;
    return ok();
}

int pkv_profile_read(kv_pool_t* p, pkv_kernel_stat_t* out, int32_t cap, int32_t* n) {
    if (!p || !n) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    *n = (int32_t)p->timers.size();
    if (cap < *n) return fail(PKV_ERR_OUT_OF_RANGE, "capacity %d < %d kernels", cap, *n);
    if (*n > 0 && !out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
    for (int32_t i = 0; i < *n; ++i) {
        KernelTimer& t = p->timers[i];
        double total = 0.0;
        for (auto& ev : t.pending) {
            float ms = 0.0f;
            hipError_t e = hipEventSynchronize(ev.second);
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev.first, ev.second);
            if (e != hipSuccess) return hip_fail(e, "profile event read");
            total += ms;
            p->spare_events.push_back(ev.first);
            p->spare_events.push_back(ev.second);
        }
        std::memset(&out[i], 0, sizeof out[i]);
        std::snprintf(out[i].name, sizeof out[i].name, "%s", t.name.c_str());
        out[i].launches = t.launches;
        out[i].dropped = t.dropped;
        out[i].total_ms = total;
        t.pending.clear();
        t.launches = 0;
        t.dropped = 0;
    }
    return ok();
}

int pkv_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!dst || !src) return fail(PKV_ERR_INVALID_ARG, "NULL pointer");
    if (bytes % 16 || !aligned16(dst) || !aligned16(src)) return fail(PKV_ERR_INVALID_ARG, "copy needs 16-byte granularity");
    hipError_t e = pkv::launch_copy(dst, src, bytes, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "copy launch");
    return ok();
}

int pkv_read_probe(const void* src, size_t bytes, int32_t nontemporal, const int32_t* order, int64_t n_order,
                   int32_t chunk_bytes, uint32_t* sink, void* stream) {
    if ((!src && bytes) || !sink) return fail(PKV_ERR_INVALID_ARG, "NULL pointer");
    if (bytes % 16 || !aligned16(src)) return fail(PKV_ERR_INVALID_ARG, "read probe needs 16-byte granularity");
    if (reinterpret_cast<uintptr_t>(sink) % 4) return fail(PKV_ERR_INVALID_ARG, "sink must be 4-byte aligned");
    if (nontemporal != 0 && nontemporal != 1) return fail(PKV_ERR_INVALID_ARG, "nontemporal must be 0 or 1");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (!order) {
        e = pkv::launch_read_probe(src, bytes, nontemporal == 1, sink, st);
    } else {
        if (n_order < 0) return fail(PKV_ERR_INVALID_ARG, "n_order must be >= 0");
        if (reinterpret_cast<uintptr_t>(order) % 4) return fail(PKV_ERR_INVALID_ARG, "order must be 4-byte aligned");
        int log_rows = -1;
        for (int k = 0; k <= 18; ++k)
            if (chunk_bytes == (4096 << k)) log_rows = k;
        if (log_rows < 0) return fail(PKV_ERR_INVALID_ARG, "chunk_bytes must be 4096 times a power of two, at most 1 GiB");
        if (bytes % (size_t)chunk_bytes) return fail(PKV_ERR_INVALID_ARG, "bytes must be a multiple of chunk_bytes");
        if (n_order > (INT64_MAX >> (log_rows + 1))) return fail(PKV_ERR_INVALID_ARG, "n_order too large");
        e = pkv::launch_gather_read_probe(src, bytes, nontemporal == 1, order, n_order, log_rows, sink, st);
    }
    if (e != hipSuccess) return hip_fail(e, "read probe launch");
    return ok();
}

}  // extern "C"

namespace pkv {
namespace {
// The event pair a timed call armed on this thread, and whether a launch has
// recorded it yet.
thread_local hipEvent_t t_start = nullptr, t_stop = nullptr;
thread_local bool t_recorded = false;
}  // namespace

void arm_launch_events(hipEvent_t start, hipEvent_t stop) {
    t_start = start;
    t_stop = stop;
    t_recorded = false;
}

bool disarm_launch_events() {
    const bool r = t_recorded;
    t_start = t_stop = nullptr;
    t_recorded = false;
    return r;
}

hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, void** args, size_t shmem, hipStream_t stream) {
    if (!t_stop) return hipLaunchKernel(fn, grid, block, args, shmem, stream);
    const hipError_t e =
        hipExtLaunchKernel(fn, grid, block, args, shmem, stream, t_recorded ? nullptr : t_start, t_stop, 0);
    if (e == hipSuccess) t_recorded = true;
    return e;
}
}  // namespace pkv
