// Chunk store around the fusion path: the load controller that picks the
// recompute ratio, and an HBM tier that keeps recently used chunk caches in
// device memory in front of pinned host memory.
//
// Load controller: CacheBlend explainer (0h-n0.github.io), section
// "パイプライン実行とロードコントローラ".  Recomputing a fraction r costs
// r T_prefill and loading costs T_load = per-token KV bytes * tokens /
// throughput; layer-wise pipelining hides the load when r T_prefill >=
// T_load, hence r* = max(r_min, T_load / T_prefill).
//
// HBM tier: CachedAttention explainer (0h-n0.github.io), section
// "エビクションポリシー" (least recently used entries leave GPU HBM first)
// and Prompt Cache explainer, section "キャッシュヒット率とエビクション"
// (hit rate, LRU eviction).  Entries are whole chunk caches (all layers, K,
// V and, for quantized chunks, their parameters) in one device allocation
// from a memory pool of the tier.  A missed chunk gets a new entry at lookup
// and the fusion's per-layer fetch copies the chunk into it (the staging
// fields of cb_chunk_kv), so every chunk crosses the host link once.
// Entries are allocated and released in the order of the caller's stream:
// a release is queued after every fusion queued before it, so no fusion
// still reads the memory; and the entries a lookup hands out are never
// released by that same lookup.
#include <cmath>
#include <list>
#include <mutex>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include <hip/hip_runtime.h>

#include "host.h"

namespace {

using cb::set_error;

#define CB_HIP_S(call)                                                                 \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess)                                                          \
            return set_error(CB_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

// Least-recently-used bookkeeping over a byte budget (host only).
class LruPolicy {
public:
    explicit LruPolicy(int64_t capacity) : cap_(capacity) {}

    bool contains(uint64_t key) const { return map_.count(key) != 0; }

    // A lookup: a resident key becomes the most recently used.
    bool touch(uint64_t key) {
        auto it = map_.find(key);
        if (it == map_.end()) return false;
        order_.splice(order_.begin(), order_, it->second.first);
        return true;
    }

    // Stores key as the most recently used, evicting least recently used
    // keys outside `keep` until `bytes` fit; the evicted keys are appended
    // to `evicted` in eviction order.  When even evicting every key outside
    // `keep` cannot make room, nothing changes (false).
    bool insert(uint64_t key, int64_t bytes, const std::unordered_set<uint64_t>& keep,
                std::vector<uint64_t>* evicted) {
        if (contains(key) || bytes < 0) return false;
        int64_t room = cap_ - used_;
        for (const auto& kv : map_)
            if (!keep.count(kv.first)) room += kv.second.second;
        if (bytes > room) return false;
        for (auto it = order_.end(); used_ + bytes > cap_ && it != order_.begin();) {
            --it;
            if (keep.count(*it)) continue;
            const uint64_t old = *it;
            used_ -= map_[old].second;
            map_.erase(old);
            it = order_.erase(it);
            evicted->push_back(old);
        }
        order_.push_front(key);
        map_[key] = {order_.begin(), bytes};
        used_ += bytes;
        return true;
    }

    void erase(uint64_t key) {
        auto it = map_.find(key);
        if (it == map_.end()) return;
        used_ -= it->second.second;
        order_.erase(it->second.first);
        map_.erase(it);
    }

    int64_t used() const { return used_; }
    size_t size() const { return map_.size(); }

private:
    int64_t cap_;
    int64_t used_ = 0;
    std::list<uint64_t> order_;   // front = most recently used
    std::unordered_map<uint64_t, std::pair<std::list<uint64_t>::iterator, int64_t>> map_;
};

int64_t code_bytes(int fmt, int64_t elems, int dtype) {
    if (fmt == CB_KV_U8) return elems;
    if (fmt == CB_KV_U4) return elems / 2;
    return elems * (dtype == CB_BF16 ? 2 : 4);
}

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

struct cb_chunk_cache {
    int L = 0, row = 0, dtype = 0, device = 0;
    int64_t capacity = 0;
    LruPolicy lru{0};
    struct Entry {
        void* mem = nullptr;
        cb_chunk_kv dev{};          // the device copy, once filled
        bool committed = false;     // filled by a fusion the caller committed
    };
    std::unordered_map<uint64_t, Entry> entries;
    hipMemPool_t pool = nullptr;
    cb_cache_stat st{};
    std::mutex mu;

    // Device bytes of one entry: K codes/values, V, parameters, 256-aligned.
    int64_t entry_bytes(const cb_chunk_kv& c) const {
        const int64_t elems = (int64_t)L * c.n_tokens * row;
        int64_t b = 2 * round256(code_bytes(c.kv_format, elems, dtype));
        if (c.kv_format != CB_KV_PLAIN) b += round256((int64_t)L * 4 * row * 4);
        return b;
    }
};

extern "C" {

cb_status cb_controller_ratio(double t_prefill_s, double per_token_kv_bytes, int64_t n_tokens,
                              double throughput_bytes_per_s, int32_t r_min_bp, int32_t* r_bp_out) {
    if (!r_bp_out) return set_error(CB_E_INVALID, "r_bp_out is NULL");
    if (!(t_prefill_s > 0) || !(per_token_kv_bytes > 0) || !(throughput_bytes_per_s > 0) ||
        !std::isfinite(t_prefill_s) || !std::isfinite(per_token_kv_bytes) ||
        !std::isfinite(throughput_bytes_per_s) || n_tokens < 0)
        return set_error(CB_E_INVALID, "times, sizes and throughput must be positive and finite");
    if (r_min_bp < 0 || r_min_bp > 10000)
        return set_error(CB_E_INVALID, "r_min_bp %d outside 0..10000", r_min_bp);
    const double bytes = per_token_kv_bytes * (double)n_tokens;
    const double t_load = bytes / throughput_bytes_per_s;
    const double ratio = t_load / t_prefill_s;
    const double bp = std::floor(ratio * 10000.0 + 0.5);
    int32_t r = bp >= 10000.0 ? 10000 : (int32_t)bp;
    if (r < r_min_bp) r = r_min_bp;
    *r_bp_out = r;
    return CB_OK;
}

cb_status cb_cache_replay(int64_t capacity_bytes, int32_t n_batches, const int32_t* batch_sizes,
                          const uint64_t* keys, const int64_t* sizes, int32_t* hits_out,
                          uint64_t* evicted_out, int32_t* evicted_per_batch) {
    if (capacity_bytes < 0 || n_batches < 0) return set_error(CB_E_INVALID, "negative sizes");
    if (n_batches > 0 && (!batch_sizes || !hits_out || !evicted_per_batch))
        return set_error(CB_E_INVALID, "NULL buffer");
    int64_t total = 0;
    for (int b = 0; b < n_batches; ++b) {
        if (batch_sizes[b] < 0) return set_error(CB_E_INVALID, "batch %d has a negative size", b);
        total += batch_sizes[b];
    }
    if (total > 0 && (!keys || !sizes)) return set_error(CB_E_INVALID, "NULL keys/sizes");
    for (int64_t i = 0; i < total; ++i)
        if (sizes[i] < 0) return set_error(CB_E_INVALID, "use %lld has a negative size", (long long)i);
    LruPolicy lru(capacity_bytes);
    std::vector<uint64_t> ev;
    std::unordered_set<uint64_t> keep;
    int64_t at = 0, n_ev = 0;
    for (int b = 0; b < n_batches; ++b) {
        const int n = batch_sizes[b];
        for (int i = 0; i < n; ++i) hits_out[at + i] = lru.touch(keys[at + i]) ? 1 : 0;
        keep.clear();
        keep.insert(keys + at, keys + at + n);
        ev.clear();
        for (int i = 0; i < n; ++i)
            if (!lru.contains(keys[at + i])) lru.insert(keys[at + i], sizes[at + i], keep, &ev);
        if (evicted_out)
            for (uint64_t k : ev) evicted_out[n_ev++] = k;
        evicted_per_batch[b] = (int32_t)ev.size();
        at += n;
    }
    return CB_OK;
}

cb_status cb_cache_create(int32_t n_layers, int32_t row, int32_t dtype, int64_t capacity_bytes,
                          cb_chunk_cache** out) {
    if (!out) return set_error(CB_E_INVALID, "out is NULL");
    *out = nullptr;
    if (n_layers <= 0 || row <= 0 || row % 8 || capacity_bytes < 0)
        return set_error(CB_E_SHAPE, "n_layers, row (a multiple of 8) and capacity must be valid");
    if (dtype != CB_F32 && dtype != CB_BF16) return set_error(CB_E_INVALID, "dtype %d", dtype);
    cb_chunk_cache* c = new cb_chunk_cache();
    c->L = n_layers;
    c->row = row;
    c->dtype = dtype;
    c->capacity = capacity_bytes;
    c->lru = LruPolicy(capacity_bytes);
    hipError_t e = hipGetDevice(&c->device);
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = c->device;
    if (e == hipSuccess) e = hipMemPoolCreate(&c->pool, &props);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        cb_cache_destroy(c);
        return set_error(CB_E_HIP, "HBM tier set-up failed: %s", hipGetErrorString(e));
    }
    uint64_t keep = UINT64_MAX;
    (void)hipMemPoolSetAttribute(c->pool, hipMemPoolAttrReleaseThreshold, &keep);
    *out = c;
    return CB_OK;
}

void cb_cache_destroy(cb_chunk_cache* c) {
    if (!c) return;
    // fusions queued on any stream may still read entries
    (void)hipDeviceSynchronize();
    for (auto& kv : c->entries) (void)hipFree(kv.second.mem);
    if (c->pool) (void)hipMemPoolDestroy(c->pool);
    delete c;
}

cb_status cb_cache_resolve(cb_chunk_cache* c, int32_t n, const uint64_t* keys,
                           const cb_chunk_kv* chunks, cb_chunk_kv* out, int32_t* hits,
                           void* stream) {
    if (!c) return set_error(CB_E_INVALID, "cache is NULL");
    if (n < 0) return set_error(CB_E_INVALID, "n < 0");
    if (n > 0 && (!keys || !chunks || !out)) return set_error(CB_E_INVALID, "NULL buffer");
    for (int i = 0; i < n; ++i) {
        const cb_chunk_kv& h = chunks[i];
        if (!h.on_host) continue;
        if (h.stage_k || h.stage_v || h.stage_qparams)
            return set_error(CB_E_INVALID, "use %d: chunk already has staging buffers", i);
        if (h.n_tokens <= 0 ||
            (h.kv_format != CB_KV_PLAIN && h.kv_format != CB_KV_U8 && h.kv_format != CB_KV_U4))
            return set_error(CB_E_INVALID, "use %d: bad chunk descriptor", i);
    }
    const hipStream_t st = (hipStream_t)stream;
    std::lock_guard<std::mutex> lk(c->mu);
    // entries reserved by a lookup that was never committed hold no data
    for (auto it = c->entries.begin(); it != c->entries.end();) {
        if (it->second.committed) { ++it; continue; }
        CB_HIP_S(hipFreeAsync(it->second.mem, st));
        c->lru.erase(it->first);
        it = c->entries.erase(it);
    }
    for (int i = 0; i < n; ++i) {
        out[i] = chunks[i];
        bool hit = false;
        if (chunks[i].on_host) {
            ++c->st.lookups;
            hit = c->lru.touch(keys[i]);
            if (hit) {
                const cb_chunk_kv& d = c->entries[keys[i]].dev;
                if (d.n_tokens != chunks[i].n_tokens || d.kv_format != chunks[i].kv_format)
                    return set_error(CB_E_INVALID,
                                     "use %d: key names a chunk of another size or format", i);
                out[i] = d;
                ++c->st.hits;
            }
        }
        if (hits) hits[i] = hit ? 1 : 0;
    }
    // reserve entries for the misses; this call's entries are never released here
    std::unordered_set<uint64_t> keep;
    for (int i = 0; i < n; ++i)
        if (chunks[i].on_host) keep.insert(keys[i]);
    std::vector<uint64_t> ev;
    for (int i = 0; i < n; ++i) {
        const cb_chunk_kv& h = chunks[i];
        if (!h.on_host || c->lru.contains(keys[i])) continue;
        const int64_t bytes = c->entry_bytes(h);
        ev.clear();
        if (!c->lru.insert(keys[i], bytes, keep, &ev)) continue;   // no room: stays on host
        for (uint64_t k : ev) {
            CB_HIP_S(hipFreeAsync(c->entries[k].mem, st));
            c->entries.erase(k);
            ++c->st.evicted;
        }
        void* mem = nullptr;
        if (hipMallocFromPoolAsync(&mem, (size_t)bytes, c->pool, st) != hipSuccess) {
            (void)hipGetLastError();
            c->lru.erase(keys[i]);
            continue;                                               // stays on host
        }
        const int64_t layer_elems = (int64_t)h.n_tokens * c->row;
        const int64_t plane = round256(code_bytes(h.kv_format, layer_elems * c->L, c->dtype));
        char* k = (char*)mem;
        cb_chunk_cache::Entry& e = c->entries[keys[i]];
        e.mem = mem;
        e.committed = false;
        e.dev = h;
        e.dev.k = k;
        e.dev.v = k + plane;
        e.dev.on_host = 0;
        e.dev.layer_stride = layer_elems;
        e.dev.qparams = h.kv_format != CB_KV_PLAIN ? (const float*)(k + 2 * plane) : nullptr;
        e.dev.stage_k = e.dev.stage_v = nullptr;
        e.dev.stage_qparams = nullptr;
        out[i].stage_k = k;
        out[i].stage_v = k + plane;
        out[i].stage_qparams = h.kv_format != CB_KV_PLAIN ? (float*)(k + 2 * plane) : nullptr;
        c->st.copied_bytes += 2 * code_bytes(h.kv_format, layer_elems * c->L, c->dtype) +
                              (h.kv_format != CB_KV_PLAIN ? (int64_t)c->L * 4 * c->row * 4 : 0);
    }
    return CB_OK;
}

cb_status cb_cache_commit(cb_chunk_cache* c, int32_t n, const uint64_t* keys) {
    if (!c) return set_error(CB_E_INVALID, "cache is NULL");
    if (n < 0 || (n > 0 && !keys)) return set_error(CB_E_INVALID, "bad keys");
    std::lock_guard<std::mutex> lk(c->mu);
    for (int i = 0; i < n; ++i) {
        auto it = c->entries.find(keys[i]);
        if (it == c->entries.end() || it->second.committed) continue;
        it->second.committed = true;
        ++c->st.admitted;
    }
    return CB_OK;
}

cb_status cb_cache_stats(cb_chunk_cache* c, cb_cache_stat* out) {
    if (!c || !out) return set_error(CB_E_INVALID, "NULL argument");
    std::lock_guard<std::mutex> lk(c->mu);
    *out = c->st;
    out->resident_entries = (int64_t)c->entries.size();
    out->resident_bytes = c->lru.used();
    return CB_OK;
}

}  // extern "C"
