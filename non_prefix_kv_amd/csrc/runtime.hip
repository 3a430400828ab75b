// libcacheblend runtime: argument validation, RoPE tables, workspace,
// streams/events and the per-layer schedule of the fusion path, exported
// through the C ABI declared in include/cacheblend.h.
//
// Per layer l (CacheBlend explainer (0h-n0), section "選択的再計算", Steps
// 1-4, with the token set narrowed as in section "HKVDトークン選定"):
//   side stream : [pinned host -> HBM copy of chunk K/V of layer l]
//                 rotate chunk K by its offset into fused_k[l], V into fused_v[l]
//   main stream : wait for the fetch of layer l, then
//     1 RMSNorm of the rows R (kept chunk rows of the previous layer + suffix)
//     2 QKV projection, RoPE at real positions                   (matrix cores)
//     3 deviation of the recomputed chunk rows vs the rotated cache
//     4 keep the top s[l+1] rows (exact radix select), + suffix rows
//     5 merge their K/V into fused[l]
//     6 attention of the kept rows over fused[l][0..N)           (matrix cores)
//     7 O projection + residual, 8 RMSNorm, 9 gate/up + SiLU*up, 10 down + residual
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/cacheblend.h"
#include "host.h"
#include "kernels.h"

using namespace cb;

// ---------------------------------------------------------------- errors
namespace {

thread_local std::string g_err;

cb_status vfail(cb_status st, const char* fmt, va_list ap) {
    char buf[512];
    vsnprintf(buf, sizeof buf, fmt, ap);
    g_err = buf;
    return st;
}

cb_status fail(cb_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vfail(st, fmt, ap);
    va_end(ap);
    return st;
}

#define CB_HIP(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess)                                                          \
            return fail(CB_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_));       \
    } while (0)

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------- RoPE tables
// (cos, sin)(pos * theta_i), theta_i = base^(-2i/d_head): angles in float64,
// rounded once to float32.  Tables only grow; superseded tables stay
// allocated so work already queued keeps valid pointers.
struct RopeCache {
    std::mutex mu;
    std::map<std::tuple<int, double, int>, RopeTab> cur;
    std::vector<void*> keep;
};
RopeCache& rope_cache() {
    static RopeCache c;
    return c;
}

cb_status get_rope(double base, int head_dim, int n_pos, RopeTab* out) {
    int dev = 0;
    CB_HIP(hipGetDevice(&dev));
    RopeCache& c = rope_cache();
    std::lock_guard<std::mutex> lk(c.mu);
    auto key = std::make_tuple(dev, base, head_dim);
    auto it = c.cur.find(key);
    if (it != c.cur.end() && it->second.n_pos >= n_pos) {
        *out = it->second;
        return CB_OK;
    }
    int want = std::max(n_pos, 16384);
    if (it != c.cur.end()) want = std::max(want, 2 * it->second.n_pos);
    const int half = head_dim / 2;
    std::vector<float2> host((size_t)want * half);
    for (int p = 0; p < want; ++p)
        for (int i = 0; i < half; ++i) {
            const double theta = std::pow(base, -2.0 * i / head_dim);
            const double ang = (double)p * theta;
            host[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
        }
    void* d = nullptr;
    if (hipMalloc(&d, host.size() * sizeof(float2)) != hipSuccess)
        return fail(CB_E_OOM, "RoPE table allocation (%zu bytes) failed",
                    host.size() * sizeof(float2));
    CB_HIP(hipMemcpy(d, host.data(), host.size() * sizeof(float2), hipMemcpyHostToDevice));
    c.keep.push_back(d);
    RopeTab t;
    t.tab = static_cast<const float2*>(d);
    t.n_pos = want;
    t.half = half;
    c.cur[key] = t;
    *out = t;
    return CB_OK;
}

// ---------------------------------------------------------------- schedule
cb_status make_schedule(int n, int r_bp, int kind, int L, int* s) {
    if (L <= 0 || n < 0) return fail(CB_E_INVALID, "schedule: n_layers %d, chunk tokens %d", L, n);
    if (r_bp < 0 || r_bp > 10000) return fail(CB_E_SCHEDULE, "recompute_bp %d not in 0..10000", r_bp);
    if (kind != CB_SCHED_GRADUAL && kind != CB_SCHED_FIXED)
        return fail(CB_E_INVALID, "unknown schedule kind %d", kind);
    if (r_bp == 0 || n == 0) {
        for (int l = 0; l <= L; ++l) s[l] = 0;
        return CB_OK;
    }
    s[0] = n;
    s[1] = n;
    const int64_t nn = n;
    if (kind == CB_SCHED_FIXED) {
        const int k = (int)std::max<int64_t>(1, nn * r_bp / 10000);
        for (int l = 2; l <= L; ++l) s[l] = k;
    } else {
        const int64_t r1 = std::min<int64_t>(10000, (12 * (int64_t)r_bp) / 10);
        for (int l = 1; l < L; ++l) {
            const int e = std::min(l - 1, 30);
            const int64_t p2 = (int64_t)1 << e;
            // n * (r 2^e + r1 - r) / (10000 2^e) in exact integer arithmetic
            const __int128 num = (__int128)nn * ((int64_t)r_bp * p2 + r1 - r_bp);
            const __int128 den = (__int128)10000 * p2;
            int64_t k = (int64_t)(num / den);
            if (k < 1) k = 1;
            s[l + 1] = (int)std::min<int64_t>(k, s[l]);
        }
    }
    return CB_OK;
}

bool aligned_to(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

namespace cb {

cb_status set_error(cb_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vfail(st, fmt, ap);
    va_end(ap);
    return st;
}

MemKind mem_kind(const void* p) {
    hipPointerAttribute_t at;
    memset(&at, 0, sizeof at);
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();
        return MemKind::Other;
    }
    if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) return MemKind::Device;
    if (at.type == hipMemoryTypeHost) return MemKind::Pinned;
    return MemKind::Other;
}

}  // namespace cb

// ---------------------------------------------------------------- model
struct cb_model {
    cb_model_cfg cfg;
    std::vector<cb_layer_weights> w;
    const void* final_norm = nullptr;   // gain of the final RMSNorm (cb_lm_head), or NULL
    // plan workspaces: carved from a caller's buffer (ws_user), or taken from
    // the model's pool, at most ws_limit bytes when ws_limit > 0
    void* ws_user = nullptr;
    size_t ws_user_bytes = 0;
    size_t ws_limit = 0;
    RopeTab rope;
    int device = 0;
    hipStream_t side = nullptr;   // fetch (H2D + rotation) stream, default priority
    hipMemPool_t pool = nullptr;  // plan workspaces; keeps its memory between plans
    std::mutex mu;
    std::vector<hipEvent_t> event_pool;
    // per-kernel-class timing (cb_profile_*)
    struct ProfRec {
        int cls;
        hipEvent_t a, b;
        double flops, bytes;
    };
    bool prof = false;
    std::vector<ProfRec> prof_pending;
    std::vector<hipEvent_t> timing_pool;
    cb_kernel_stat stats[CB_K_COUNT] = {};
    int es() const { return elem_size(cfg.dtype); }
    int qd() const { return cfg.n_q_heads * cfg.head_dim; }
    int kvd() const { return cfg.n_kv_heads * cfg.head_dim; }
};

// ---------------------------------------------------------------- plan
// One plan fuses a batch of requests (cb_blend: a batch of one).  Request b
// owns rows G..G+N-1 of every stacked [sum N] array; per layer its
// recomputed rows R and query rows Q are contiguous blocks of the stacked
// workspace rows (see ReqRows).
struct ReqInfo {
    int G = 0, N = 0, Nc = 0, Ns = 0;
    int C = 0;                    // first column in [L][sum N_c] outputs
    int pos0 = 0;                 // position of the request's first token
    std::vector<int> s;           // schedule s[0..L]
    std::vector<int> ids;         // pool entries in prompt order
    std::vector<int> offsets;     // chunk offsets
};

struct cb_plan {
    cb_model* m = nullptr;
    hipStream_t stream = nullptr;
    int L = 0, Ntot = 0, Nctot = 0;
    std::vector<ReqInfo> reqs;
    std::vector<cb_chunk_kv> pool;
    const void* x0 = nullptr;
    int dev_mode = CB_DEV_KV;
    const float* given = nullptr;     // CB_DEV_GIVEN scores, [sum N_c]
    int kv_pos0 = 0;              // position of key row 0 of a request
    // outputs
    void* fused_k = nullptr;
    void* fused_v = nullptr;
    int* sel_idx = nullptr;
    float* hidden_out = nullptr;
    float* deviation = nullptr;
    // workspace
    void* ws = nullptr;
    bool ws_owned = false;        // allocated from the model's pool (else the caller's)
    size_t ws_bytes = 0;
    float *X = nullptr, *Hres = nullptr, *dev = nullptr;
    void *Hn = nullptr, *Q = nullptr, *Kn = nullptr, *Vn = nullptr, *attn = nullptr,
         *act = nullptr;
    int *pos_a = nullptr, *pos_b = nullptr, *row_a = nullptr, *row_b = nullptr,
        *sel_local = nullptr;
    // layers run in place whose kept positions are asked for: sel_idx row
    // first = row second (the last layer that wrote its row), filled after
    // the last layer
    std::vector<std::pair<int, int>> sel_rows_pending;
    float* attn_dev_part = nullptr;   // CB_DEV_ATTN: per-head deviations [Hq][max rows]
    int64_t attn_dev_stride = 0;
    void* attn_ws = nullptr;      // split-attention partials
    size_t attn_ws_bytes = 0;
    // fetch: host chunks copied once per layer into their first place of use,
    // then rotation jobs that copy from a source (launched first) and jobs
    // that rotate in place (launched after, they overwrite those sources)
    struct H2D {
        const char* k;
        const char* v;
        size_t layer_bytes;       // bytes between layers of the source
        size_t bytes;             // bytes per layer
        int64_t dst_row;
    };
    std::vector<H2D> h2d;
    std::vector<RotJobs> jobs_copy, jobs_inplace;
    // quantized chunks: host ones are copied each layer (codes and that
    // layer's parameters) into a staging area of the workspace, then every
    // use is decoded from there; device ones are decoded from where they are
    struct QH2D {
        const char* k;
        const char* v;
        const char* qp;
        size_t layer_bytes;       // code bytes between layers of the source
        size_t bytes;             // code bytes per layer
        size_t qp_bytes;          // parameter bytes per layer
        size_t stage_off;         // staging offset: k codes, v codes, parameters
    };
    std::vector<QH2D> qh2d;
    // host chunks with caller-given staging buffers: each layer is copied
    // there (dense layers) and every use reads it from there
    struct StageCopy {
        const char* src_k;
        const char* src_v;
        const char* src_qp;
        size_t src_layer_bytes;   // code/value bytes between layers of the source
        size_t bytes;             // code/value bytes per layer
        size_t qp_bytes;          // parameter bytes per layer (0: plain)
        char* dst_k;
        char* dst_v;
        char* dst_qp;
    };
    std::vector<StageCopy> stage_copies;
    // quantization parameters of host chunks (all layers, one copy per
    // chunk) go to the device with the first fetch: per-layer copies of a
    // few KiB would each become a small copy kernel on the side stream
    bool params_sent = false;
    size_t stage_bytes = 0;
    char* stage = nullptr;
    std::vector<QRotJobs> qjobs[2];   // [0]: 8-bit, [1]: 4-bit codes
    // Layers the side stream may run ahead of the main stream.  Rotation
    // kernels share the compute units with the layers, so device-resident
    // chunks are fetched just ahead; host copies run on the copy engines and
    // each layer's destination is its own, so they start as early as possible.
    int lookahead = 2;

    // streams / events
    hipEvent_t ready = nullptr;                 // workspace + prior main work
    std::vector<hipEvent_t> fetched, layer_start;
    std::vector<char> fetch_done;
    int next_layer = 0;
};

namespace {

// Brackets one launch with timing events when profiling is on.
class Span {
public:
    Span(cb_model* m, int cls, hipStream_t s, double flops, double bytes)
        : m_(m), cls_(cls), s_(s), flops_(flops), bytes_(bytes) {
        if (m_->prof && (a_ = take()) != nullptr) (void)hipEventRecord(a_, s_);
    }
    ~Span() {
        if (!a_) return;
        hipEvent_t b = take();
        if (!b) return;
        (void)hipEventRecord(b, s_);
        std::lock_guard<std::mutex> lk(m_->mu);
        m_->prof_pending.push_back({cls_, a_, b, flops_, bytes_});
    }

private:
    hipEvent_t take() {
        std::lock_guard<std::mutex> lk(m_->mu);
        if (!m_->timing_pool.empty()) {
            hipEvent_t e = m_->timing_pool.back();
            m_->timing_pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
    cb_model* m_;
    int cls_;
    hipStream_t s_;
    double flops_, bytes_;
    hipEvent_t a_ = nullptr;
};

cb_status validate_cfg(const cb_model_cfg* c) {
    if (!c) return fail(CB_E_INVALID, "cfg is NULL");
    if (c->dtype != CB_F32 && c->dtype != CB_BF16) return fail(CB_E_INVALID, "dtype %d", c->dtype);
    if (c->n_layers <= 0 || c->d_model <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
        c->ffn_dim <= 0)
        return fail(CB_E_INVALID, "model sizes must be positive");
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(CB_E_UNSUPPORTED, "head_dim %d (64 or 128 supported)", c->head_dim);
    if (c->n_q_heads % c->n_kv_heads) return fail(CB_E_SHAPE, "n_kv_heads must divide n_q_heads");
    const int kmul = c->dtype == CB_BF16 ? 64 : 32;
    if (c->d_model % kmul || c->ffn_dim % kmul || (c->n_q_heads * c->head_dim) % kmul)
        return fail(CB_E_SHAPE, "d_model, ffn_dim and Hq*head_dim must be multiples of %d", kmul);
    if (!(c->rope_base > 1.0) || !(c->rms_eps >= 0.f))
        return fail(CB_E_INVALID, "rope_base must be > 1 and rms_eps >= 0");
    return CB_OK;
}

// Row blocks of every request at layer l.
struct LayerRows {
    std::vector<ReqRows> r;
    int mR = 0, mQ = 0, nC = 0;
    bool select_needed = false;   // some request keeps fewer chunk rows than it recomputes
};
LayerRows layer_rows(const cb_plan* p, int l) {
    LayerRows lr;
    lr.r.reserve(p->reqs.size());
    for (const ReqInfo& q : p->reqs) {
        ReqRows x{};
        x.r_off = lr.mR;
        x.n_c = q.s[l];
        x.n_s = q.Ns;
        x.k = q.s[l + 1];
        x.q_off = lr.mQ;
        x.c_off = lr.nC;
        x.out_col = q.C;
        lr.r.push_back(x);
        lr.mR += x.n_c + x.n_s;
        lr.mQ += x.k + x.n_s;
        lr.nC += x.n_c;
        lr.select_needed |= x.k < x.n_c;
    }
    return lr;
}

// The request table split into launches of kMaxReq requests.
std::vector<ReqTab> req_tabs(const std::vector<ReqRows>& rows) {
    std::vector<ReqTab> t;
    for (size_t i = 0; i < rows.size(); i += kMaxReq) {
        ReqTab x{};
        x.n = (int)std::min<size_t>(kMaxReq, rows.size() - i);
        for (int j = 0; j < x.n; ++j) {
            x.r[j] = rows[i + j];
            x.max_c = std::max(x.max_c, x.r[j].n_c);
        }
        t.push_back(x);
    }
    return t;
}

// Attention ranges of layer l: each request's query rows over its own keys.
std::vector<AttnRange> attn_ranges(const cb_plan* p, const LayerRows& lr) {
    std::vector<AttnRange> a;
    for (size_t b = 0; b < p->reqs.size(); ++b) {
        const int nq = lr.r[b].k + lr.r[b].n_s;
        if (nq > 0) a.push_back(AttnRange{lr.r[b].q_off, nq, p->reqs[b].G, p->reqs[b].N});
    }
    return a;
}

// Carves the workspace for up to `max_rows` stacked rows.
size_t carve(cb_plan* p, char* base, int max_rows) {
    const cb_model_cfg& c = p->m->cfg;
    const size_t es = p->m->es(), R = (size_t)std::max(1, max_rows);
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* r = base ? base + off : nullptr;
        off = align_up(off + bytes, 256);
        return r;
    };
    p->X = (float*)take(R * c.d_model * 4);
    p->Hres = (float*)take(R * c.d_model * 4);
    p->Hn = take(R * c.d_model * es);
    p->Q = take(R * p->m->qd() * es);
    p->Kn = take(R * p->m->kvd() * es);
    p->Vn = take(R * p->m->kvd() * es);
    p->attn = take(R * p->m->qd() * es);
    p->act = take(R * c.ffn_dim * es);
    p->dev = (float*)take(std::max<size_t>(1, p->Nctot) * 4);
    p->pos_a = (int*)take(R * 4);
    p->pos_b = (int*)take(R * 4);
    p->row_a = (int*)take(R * 4);
    p->row_b = (int*)take(R * 4);
    p->sel_local = (int*)take(R * 4);
    if (p->dev_mode == CB_DEV_ATTN) {
        p->attn_dev_stride = (int64_t)R;
        p->attn_dev_part = (float*)take(attention_deviation_workspace(c.n_q_heads, (int64_t)R));
    }
    p->attn_ws = p->attn_ws_bytes ? take(p->attn_ws_bytes) : nullptr;
    p->stage = p->stage_bytes ? take(p->stage_bytes) : nullptr;
    return off;
}

// Workspace bytes of a laid-out plan (most stacked rows of any layer, the
// largest attention split of any layer, staging); max_rows receives the rows.
size_t plan_bytes(cb_plan* p, int* max_rows_out) {
    const cb_model_cfg& c = p->m->cfg;
    int max_rows = 0;
    size_t aw = 0;
    for (int l = 0; l < p->L; ++l) {
        const LayerRows lr = layer_rows(p, l);
        max_rows = std::max(max_rows, lr.mR);
        const std::vector<AttnRange> ar = attn_ranges(p, lr);
        aw = std::max(aw, attention_workspace(c.dtype, ar.data(), (int)ar.size(), c.n_q_heads,
                                              c.head_dim));
    }
    p->attn_ws_bytes = aw;
    *max_rows_out = max_rows;
    return carve(p, nullptr, max_rows);
}

cb_status plan_alloc(cb_plan* p) {
    int max_rows = 0;
    const size_t bytes = plan_bytes(p, &max_rows);
    const cb_model* m = p->m;
    if (m->ws_user) {
        if (bytes > m->ws_user_bytes)
            return fail(CB_E_OOM, "workspace of %zu bytes exceeds the caller's %zu bytes", bytes,
                        m->ws_user_bytes);
        p->ws = m->ws_user;
    } else {
        if (m->ws_limit && bytes > m->ws_limit)
            return fail(CB_E_OOM, "workspace of %zu bytes exceeds the limit of %zu bytes", bytes,
                        m->ws_limit);
        if (hipMallocFromPoolAsync(&p->ws, bytes, p->m->pool, p->stream) != hipSuccess) {
            (void)hipGetLastError();
            p->ws = nullptr;
            return fail(CB_E_OOM, "workspace of %zu bytes", bytes);
        }
        p->ws_owned = true;
    }
    p->ws_bytes = bytes;
    carve(p, (char*)p->ws, max_rows);
    // decode jobs of staged chunks point into the staging area from now on
    for (auto& set : p->qjobs)
        for (QRotJobs& js : set)
            for (int i = 0; i < js.n; ++i) {
                QRotJob& j = js.j[i];
                if (!j.staged) continue;
                j.k = (const uint8_t*)(p->stage + (uintptr_t)j.k);
                j.v = (const uint8_t*)(p->stage + (uintptr_t)j.v);
                j.qp = (const float*)(p->stage + (uintptr_t)j.qp);
                j.staged = 0;
            }
    return CB_OK;
}

// Events come from a per-model pool: re-recording an event that a stream
// already waited on is safe (the wait captured the earlier recording).
cb_status plan_events(cb_plan* p) {
    std::lock_guard<std::mutex> lk(p->m->mu);
    auto get = [&](hipEvent_t* e) -> hipError_t {
        if (!p->m->event_pool.empty()) {
            *e = p->m->event_pool.back();
            p->m->event_pool.pop_back();
            return hipSuccess;
        }
        return hipEventCreateWithFlags(e, hipEventDisableTiming);
    };
    CB_HIP(get(&p->ready));
    p->fetched.assign(p->L, nullptr);
    p->layer_start.assign(p->L, nullptr);
    p->fetch_done.assign(p->L, 0);
    for (int l = 0; l < p->L; ++l) {
        CB_HIP(get(&p->fetched[l]));
        CB_HIP(get(&p->layer_start[l]));
    }
    return CB_OK;
}

// Initial rows: R_0 of request b = (all its chunk rows if s[0] = N_c) +
// suffix, positions from pos0, global rows from G.  Unmeasured deviations
// read NaN.
cb_status plan_start(cb_plan* p) {
    RowInitTab t{};
    int r_off = 0;
    for (size_t b = 0; b < p->reqs.size(); ++b) {
        const ReqInfo& q = p->reqs[b];
        const int base = q.s[0] == q.Nc ? 0 : q.Nc;
        t.r[t.n++] = RowInit{r_off, q.N - base, q.pos0 + base, q.G + base};
        r_off += q.N - base;
        if (t.n == kMaxReq || b + 1 == p->reqs.size()) {
            CB_HIP(launch_init_rows(t, p->pos_a, p->row_a, p->stream));
            t.n = 0;
        }
    }
    if (p->deviation)
        CB_HIP(launch_fill(p->deviation, (int64_t)p->L * p->Nctot, NAN, p->stream));
    CB_HIP(hipEventRecord(p->ready, p->stream));
    CB_HIP(hipStreamWaitEvent(p->m->side, p->ready, 0));
    return CB_OK;
}

void plan_free(cb_plan* p) {
    if (!p) return;
    if (p->ws) {
        // the side stream may still be rotating: main waits for its last event
        for (int l = 0; l < p->L; ++l)
            if (p->fetch_done[l]) (void)hipStreamWaitEvent(p->stream, p->fetched[l], 0);
        if (p->ws_owned) (void)hipFreeAsync(p->ws, p->stream);
    }
    {
        std::lock_guard<std::mutex> lk(p->m->mu);
        if (p->ready) p->m->event_pool.push_back(p->ready);
        for (auto e : p->fetched) if (e) p->m->event_pool.push_back(e);
        for (auto e : p->layer_start) if (e) p->m->event_pool.push_back(e);
    }
    delete p;
}

int64_t layer_elems(const cb_plan* p) { return (int64_t)p->Ntot * p->m->kvd(); }

double job_bytes(const RotJobs& js, double row_bytes) {
    double b = 0;
    for (int i = 0; i < js.n; ++i) b += js.j[i].n_tokens * row_bytes * (js.j[i].v_src ? 4 : 2);
    return b;
}

cb_status do_fetch(cb_plan* p, int l) {
    if (p->fetch_done[l]) return CB_OK;
    cb_model* m = p->m;
    const hipStream_t side = m->side;
    // keep the side stream at most `lookahead` layers ahead of the main stream
    const int behind = l - p->lookahead;
    if (behind >= 0 && behind < p->next_layer)
        CB_HIP(hipStreamWaitEvent(side, p->layer_start[behind], 0));
    const size_t es = m->es(), row_bytes = (size_t)m->kvd() * es;
    char* fk = (char*)p->fused_k + (size_t)l * layer_elems(p) * es;
    char* fv = (char*)p->fused_v + (size_t)l * layer_elems(p) * es;
    if (!p->params_sent) {
        for (const cb_plan::StageCopy& c : p->stage_copies)
            if (c.qp_bytes)
                CB_HIP(hipMemcpyAsync(c.dst_qp, c.src_qp, c.qp_bytes * p->L, hipMemcpyHostToDevice,
                                      side));
        for (const cb_plan::QH2D& h : p->qh2d)
            CB_HIP(hipMemcpyAsync(p->stage + h.stage_off + 2 * align_up(h.bytes, 256), h.qp,
                                  h.qp_bytes * p->L, hipMemcpyHostToDevice, side));
        p->params_sent = true;
    }
    for (const cb_plan::StageCopy& c : p->stage_copies) {
        const size_t src = (size_t)l * c.src_layer_bytes, dst = (size_t)l * c.bytes;
        CB_HIP(hipMemcpyAsync(c.dst_k + dst, c.src_k + src, c.bytes, hipMemcpyHostToDevice, side));
        CB_HIP(hipMemcpyAsync(c.dst_v + dst, c.src_v + src, c.bytes, hipMemcpyHostToDevice, side));
    }
    for (const cb_plan::H2D& h : p->h2d) {
        const size_t src = (size_t)l * h.layer_bytes, dst = (size_t)h.dst_row * row_bytes;
        CB_HIP(hipMemcpyAsync(fk + dst, h.k + src, h.bytes, hipMemcpyHostToDevice, side));
        CB_HIP(hipMemcpyAsync(fv + dst, h.v + src, h.bytes, hipMemcpyHostToDevice, side));
    }
    for (const std::vector<RotJobs>* set : {&p->jobs_copy, &p->jobs_inplace})
        for (const RotJobs& js : *set) {
            Span sp(m, CB_K_ROTATE, side, 0, job_bytes(js, (double)row_bytes));
            CB_HIP(launch_rerotate(m->cfg.dtype, js, l, fk, fv, m->cfg.n_kv_heads,
                                   m->cfg.head_dim, m->rope, side));
        }
    // quantized chunks; the staging area is reused every layer, which the
    // side stream's order makes safe (this layer's copies start after the
    // previous layer's decode kernels)
    for (const cb_plan::QH2D& h : p->qh2d) {
        const size_t src = (size_t)l * h.layer_bytes;
        char* st = p->stage + h.stage_off;
        CB_HIP(hipMemcpyAsync(st, h.k + src, h.bytes, hipMemcpyHostToDevice, side));
        CB_HIP(hipMemcpyAsync(st + align_up(h.bytes, 256), h.v + src, h.bytes,
                              hipMemcpyHostToDevice, side));
    }
    for (int b = 0; b < 2; ++b)
        for (const QRotJobs& js : p->qjobs[b]) {
            double bytes = 0;
            for (int i = 0; i < js.n; ++i)
                bytes += js.j[i].n_tokens * (double)m->kvd() * 2 * (es + (b == 0 ? 1.0 : 0.5));
            Span sp(m, CB_K_ROTATE, side, 0, bytes);
            CB_HIP(launch_dequant_rerotate(m->cfg.dtype, b == 0 ? 8 : 4, js, l, fk, fv,
                                           m->cfg.n_kv_heads, m->cfg.head_dim, m->rope, side));
        }
    CB_HIP(hipEventRecord(p->fetched[l], side));
    p->fetch_done[l] = 1;
    return CB_OK;
}

// Kept positions of the layers run in place (copies of the row of the last
// layer that selected), after the last layer.
cb_status flush_sel_rows(cb_plan* p) {
    if (p->sel_rows_pending.empty()) return CB_OK;
    Span sp(p->m, CB_K_SELECT, p->stream, 0, 8.0 * p->Nctot * p->sel_rows_pending.size());
    for (size_t i = 0; i < p->sel_rows_pending.size(); i += kMaxRowCopies) {
        IntRowCopies t{};
        t.n = (int)std::min<size_t>(kMaxRowCopies, p->sel_rows_pending.size() - i);
        for (int j = 0; j < t.n; ++j)
            t.c[j] = RowCopy{p->sel_rows_pending[i + j].first, p->sel_rows_pending[i + j].second};
        CB_HIP(launch_copy_int_rows(p->sel_idx, p->Nctot, t, p->stream));
    }
    p->sel_rows_pending.clear();
    return CB_OK;
}

cb_status do_layer(cb_plan* p, int l) {
    cb_model* m = p->m;
    const cb_model_cfg& c = m->cfg;
    const cb_layer_weights& w = m->w[l];
    const hipStream_t st = p->stream;
    const int dt = c.dtype, es = m->es();
    const LayerRows lr = layer_rows(p, l);
    const int mR = lr.mR, mQ = lr.mQ;
    const double d = c.d_model, F = c.ffn_dim, qd = m->qd(), kvd = m->kvd();
    CB_HIP(hipEventRecord(p->layer_start[l], st));
    if (mR == 0) {
        CB_HIP(hipStreamWaitEvent(st, p->fetched[l], 0));
        return l == p->L - 1 ? flush_sel_rows(p) : CB_OK;
    }
    void* fk = (char*)p->fused_k + (size_t)l * layer_elems(p) * es;
    void* fv = (char*)p->fused_v + (size_t)l * layer_elems(p) * es;
    const int *pos_r = p->pos_a, *row_r = p->row_a;
    int *pos_q = p->pos_b, *row_q = p->row_b;
    const std::vector<ReqTab> tabs = req_tabs(lr.r);

    // 1. RMSNorm of the input rows (layer 0 gathers them from x0 by fused row)
    {
        const double in_es = l == 0 ? es : 4;
        Span sp(m, CB_K_RMSNORM, st, 0, mR * d * (in_es + es + (l == 0 ? 4 : 0)));
        if (l == 0) {
            const bool all_rows = mR == p->Ntot;
            CB_HIP(launch_rmsnorm(dt, p->x0, all_rows ? nullptr : row_r, dt, w.attn_norm, p->Hn,
                                  p->X, mR, c.d_model, c.rms_eps, st));
        } else {
            CB_HIP(launch_rmsnorm(F32, p->X, nullptr, dt, w.attn_norm, p->Hn, nullptr, mR,
                                  c.d_model, c.rms_eps, st));
        }
    }
    // A layer where every request keeps all the rows it recomputed keeps them
    // in place: its query rows are its recomputed rows in the same order, so
    // the row maps stay as they are and no deviation or selection is
    // launched, unless the selection's outputs (kept positions, deviations by
    // position) are asked for.  (With kept positions asked for, a layer after
    // the first in place keeps the previous layer's positions: its sel_idx
    // row is copied at the end.)
    const bool measure = lr.nC > 0 && (lr.select_needed || p->deviation);
    const bool in_place =
        !lr.select_needed && !(measure && p->deviation) && (!p->sel_idx || l > 0);
    // 2. QKV projection with RoPE at the real positions.  In place, with
    // every chunk in device memory, K and V go straight to their rows of
    // fused[l] (every recomputed row is kept), after this layer's fetch has
    // written the rotated cache there (device fetches run ahead and are long
    // done).  Otherwise they go to the work rows and steps 1-2 overlap the
    // fetch: chunks copied from host memory may still be arriving.
    const bool direct_kv = in_place && p->h2d.empty() && p->qh2d.empty() && p->stage_copies.empty();
    if (direct_kv) CB_HIP(hipStreamWaitEvent(st, p->fetched[l], 0));
    {
        GemmArgs g{};
        g.a = p->Hn; g.b0 = w.wq; g.b1 = w.wk; g.b2 = w.wv;
        g.n0 = m->qd(); g.n1 = m->kvd();
        g.M = mR; g.N = m->qd() + 2 * m->kvd(); g.K = c.d_model;
        g.out0 = p->Q;
        g.out1 = direct_kv ? fk : p->Kn;
        g.out2 = direct_kv ? fv : p->Vn;
        g.kv_rows = direct_kv ? row_r : nullptr;
        g.pos = pos_r; g.rope = m->rope; g.head_dim = c.head_dim;
        const double n = g.N;
        Span sp(m, CB_K_GEMM_QKV, st, 2.0 * mR * n * d, (mR * d + n * d + mR * n) * es);
        CB_HIP(launch_gemm(dt, EPI_QKV, g, st));
    }
    // fused[l] is first read below
    if (!direct_kv) CB_HIP(hipStreamWaitEvent(st, p->fetched[l], 0));
    // 3-4. deviation of the recomputed chunk rows against the rotated cache,
    // then per request: keep the top s[l+1] chunk rows, then the suffix rows.
    const int* qmap = p->sel_local;     // query row -> recomputed row (null: identity)
    {
        int* sel_pos = p->sel_idx ? p->sel_idx + (size_t)l * p->Nctot : nullptr;
        float* dev_out = (measure && p->deviation) ? p->deviation + (size_t)l * p->Nctot : nullptr;
        if (in_place) {
            qmap = nullptr;
            pos_q = const_cast<int*>(pos_r);
            row_q = const_cast<int*>(row_r);
            if (p->sel_idx) {
                int src = l - 1;
                if (!p->sel_rows_pending.empty() && p->sel_rows_pending.back().first == l - 1)
                    src = p->sel_rows_pending.back().second;
                p->sel_rows_pending.push_back({l, src});
            }
        } else {
            if (measure && p->dev_mode == CB_DEV_GIVEN) {
                Span sp(m, CB_K_DEVIATION, st, 0, lr.nC * 12.0);
                for (const ReqTab& t : tabs)
                    CB_HIP(launch_given_scores(p->given, t, pos_r, p->dev, st));
            } else if (measure && p->dev_mode == CB_DEV_ATTN) {
                // attention deviation for the requests whose every chunk row
                // is a candidate (their chunk rows are R rows r_off.. at
                // positions 0.., cached rows G..), K and V deviation for the rest
                std::vector<AttnDevReq> ad;
                std::vector<ReqRows> kvr;
                for (size_t b = 0; b < p->reqs.size(); ++b) {
                    const ReqRows& x = lr.r[b];
                    if (x.n_c == 0) continue;
                    if (x.n_c == p->reqs[b].Nc)
                        ad.push_back(AttnDevReq{x.r_off, x.n_c, x.r_off, p->reqs[b].G, x.c_off});
                    else
                        kvr.push_back(x);
                }
                if (!ad.empty()) {
                    double fl = 0;
                    for (const AttnDevReq& x : ad) fl += 4.0 * c.n_q_heads * c.head_dim * 0.5 * x.n * (x.n + 1.0);
                    Span sp(m, CB_K_DEVIATION, st, fl, 0);
                    AttnDevArgs a{};
                    a.q = p->Q; a.k_new = p->Kn; a.k_cached = fk;
                    a.n_q_heads = c.n_q_heads; a.n_kv_heads = c.n_kv_heads; a.head_dim = c.head_dim;
                    a.part = p->attn_dev_part; a.part_stride = p->attn_dev_stride;
                    const hipError_t e = launch_attention_deviation(dt, a, ad.data(), (int)ad.size(),
                                                                    p->dev, st);
                    if (e != hipSuccess)
                        return fail(CB_E_HIP, "attention deviation launch: %s", hipGetErrorString(e));
                }
                if (!kvr.empty()) {
                    Span sp(m, CB_K_DEVIATION, st, 0, 4.0 * kvd * es * lr.nC);
                    for (const ReqTab& t : req_tabs(kvr))
                        CB_HIP(launch_deviation(dt, p->Kn, p->Vn, fk, fv, row_r, t, m->kvd(),
                                                CB_DEV_KV, p->dev, st));
                }
            } else if (measure) {
                const double parts = p->dev_mode == CB_DEV_KV ? 4 : 2;
                Span sp(m, CB_K_DEVIATION, st, 0, lr.nC * (parts * kvd * es + 8.0));
                for (const ReqTab& t : tabs)
                    CB_HIP(launch_deviation(dt, p->Kn, p->Vn, fk, fv, row_r, t, m->kvd(),
                                            p->dev_mode, p->dev, st));
            }
            Span sp(m, CB_K_SELECT, st, 0, 4.0 * lr.nC + 16.0 * mQ);
            for (const ReqTab& t : tabs)
                CB_HIP(launch_select(p->dev, t, pos_r, row_r, p->sel_local, pos_q, row_q, sel_pos,
                                     dev_out, st));
        }
    }
    // 5. merge the kept rows' K/V into the fused cache (done by step 2 if direct)
    if (!direct_kv) {
        Span sp(m, CB_K_SCATTER, st, 0, 4.0 * mQ * kvd * es);
        CB_HIP(launch_scatter_kv(dt, p->Kn, p->Vn, qmap, row_q, fk, fv, mQ, m->kvd(), st));
    }
    // 6. attention of each request's kept rows over its whole fused cache
    {
        AttnArgs a{};
        a.q = p->Q; a.qidx = qmap; a.q_pos = pos_q;
        a.k = fk; a.v = fv; a.kv_pos0 = p->kv_pos0;
        a.n_q_heads = c.n_q_heads; a.n_kv_heads = c.n_kv_heads; a.head_dim = c.head_dim;
        a.out = p->attn;
        const std::vector<AttnRange> ar = attn_ranges(p, lr);
        Span sp(m, CB_K_ATTENTION, st, 0, 0);
        const hipError_t e = launch_attention(dt, a, ar.data(), (int)ar.size(), p->attn_ws,
                                              p->attn_ws_bytes, st);
        if (e != hipSuccess) return fail(CB_E_HIP, "attention launch: %s", hipGetErrorString(e));
    }
    // 7. O projection + residual
    {
        GemmArgs go{};
        go.a = p->attn; go.b0 = w.wo; go.M = mQ; go.N = c.d_model; go.K = m->qd();
        go.out0 = p->Hres; go.resid = p->X; go.ridx = qmap;
        Span sp(m, CB_K_GEMM_O, st, 2.0 * mQ * d * qd, (mQ * qd + d * qd) * es + mQ * d * 8);
        CB_HIP(launch_gemm(dt, EPI_RESID, go, st));
    }
    // 8. RMSNorm, 9. gate/up with SiLU(gate)*up
    {
        Span sp(m, CB_K_RMSNORM, st, 0, mQ * d * (4 + es));
        CB_HIP(launch_rmsnorm(F32, p->Hres, nullptr, dt, w.mlp_norm, p->Hn, nullptr, mQ,
                              c.d_model, c.rms_eps, st));
    }
    {
        GemmArgs gu{};
        gu.a = p->Hn; gu.b0 = w.w_gate; gu.b1 = w.w_up; gu.M = mQ; gu.N = c.ffn_dim;
        gu.K = c.d_model;
        gu.out0 = p->act;
        Span sp(m, CB_K_GEMM_GATEUP, st, 4.0 * mQ * F * d, (mQ * d + 2 * F * d + mQ * F) * es);
        CB_HIP(launch_gemm(dt, EPI_SWIGLU, gu, st));
    }
    // 10. down projection + residual -> next layer input (or the caller's output)
    {
        GemmArgs gd{};
        gd.a = p->act; gd.b0 = w.w_down; gd.M = mQ; gd.N = c.d_model; gd.K = c.ffn_dim;
        const bool last = l == p->L - 1;
        gd.out0 = (last && p->hidden_out) ? p->hidden_out : p->X;
        gd.resid = p->Hres; gd.ridx = nullptr;
        Span sp(m, CB_K_GEMM_DOWN, st, 2.0 * mQ * d * F, (mQ * F + d * F) * es + mQ * d * 8);
        CB_HIP(launch_gemm(dt, EPI_RESID, gd, st));
    }
    if (!in_place) {
        std::swap(p->pos_a, p->pos_b);
        std::swap(p->row_a, p->row_b);
    }
    if (l == p->L - 1) return flush_sel_rows(p);
    return CB_OK;
}

// Checks one chunk cache descriptor.
cb_status check_chunk(cb_model* m, const cb_chunk_kv& ck, int idx) {
    if (!ck.k || !ck.v) return fail(CB_E_INVALID, "chunk %d has a NULL k/v", idx);
    if (ck.n_tokens <= 0) return fail(CB_E_INVALID, "chunk %d has %d tokens", idx, ck.n_tokens);
    if (ck.layer_stride < (int64_t)ck.n_tokens * m->kvd())
        return fail(CB_E_SHAPE, "chunk %d layer_stride %lld < n_tokens*H_kv*d_head", idx,
                    (long long)ck.layer_stride);
    const MemKind mk = mem_kind(ck.k), mv = mem_kind(ck.v);
    if (ck.on_host) {
        if (mk != MemKind::Pinned || mv != MemKind::Pinned)
            return fail(CB_E_NOT_PINNED, "chunk %d: host K/V must be pinned (hipHostMalloc)", idx);
    } else if (mk != MemKind::Device || mv != MemKind::Device) {
        return fail(CB_E_INVALID, "chunk %d: on_host = 0 but K/V are not device memory", idx);
    }
    if (ck.reserved != 0) return fail(CB_E_INVALID, "chunk %d: reserved field must be 0", idx);
    if (ck.stage_k || ck.stage_v || ck.stage_qparams) {
        const bool quant = ck.kv_format != CB_KV_PLAIN;
        if (!ck.on_host || !ck.stage_k || !ck.stage_v || quant != (ck.stage_qparams != nullptr))
            return fail(CB_E_INVALID,
                        "chunk %d: staging needs a host chunk and all of its stage buffers", idx);
        if (mem_kind(ck.stage_k) != MemKind::Device || mem_kind(ck.stage_v) != MemKind::Device ||
            (quant && mem_kind(ck.stage_qparams) != MemKind::Device))
            return fail(CB_E_INVALID, "chunk %d: stage buffers must be device memory", idx);
        if (!aligned_to(ck.stage_k, 16) || !aligned_to(ck.stage_v, 16) ||
            (quant && !aligned_to(ck.stage_qparams, 16)))
            return fail(CB_E_SHAPE, "chunk %d: stage buffers must be 16-byte aligned", idx);
    }
    if (ck.kv_format == CB_KV_PLAIN) {
        if (ck.qparams) return fail(CB_E_INVALID, "chunk %d: qparams given for a plain chunk", idx);
        if (!aligned_to(ck.k, 16) || !aligned_to(ck.v, 16) || (ck.layer_stride * m->es()) % 16)
            return fail(CB_E_SHAPE, "chunk %d: K/V and layer stride must be 16-byte aligned", idx);
        return CB_OK;
    }
    if (ck.kv_format != CB_KV_U8 && ck.kv_format != CB_KV_U4)
        return fail(CB_E_INVALID, "chunk %d: kv_format %d", idx, ck.kv_format);
    if (!ck.qparams) return fail(CB_E_INVALID, "chunk %d: quantized chunk without qparams", idx);
    const MemKind mq = mem_kind(ck.qparams);
    if (ck.on_host ? mq != MemKind::Pinned : mq != MemKind::Device)
        return fail(ck.on_host ? CB_E_NOT_PINNED : CB_E_INVALID,
                    "chunk %d: qparams must be in the same kind of memory as K/V", idx);
    const int64_t stride_bytes = ck.kv_format == CB_KV_U8 ? ck.layer_stride : ck.layer_stride / 2;
    if (!aligned_to(ck.k, 16) || !aligned_to(ck.v, 16) || !aligned_to(ck.qparams, 16) ||
        (ck.kv_format == CB_KV_U4 && ck.layer_stride % 2) || stride_bytes % 16)
        return fail(CB_E_SHAPE, "chunk %d: codes, qparams and layer stride must be 16-byte aligned",
                    idx);
    return CB_OK;
}

// Schedule of one request: explicit, or derived; min_tokens forces a full
// prefill; validated to be non-increasing with s[0] in {0, N_c}.
cb_status request_schedule(cb_plan* p, ReqInfo& q, const int32_t* sched, int r_bp, int kind,
                           int min_tokens, int b) {
    const int L = p->L;
    q.s.assign(L + 1, 0);
    if (sched) {
        q.s.assign(sched, sched + L + 1);
    } else {
        cb_status st = make_schedule(q.Nc, r_bp, kind, L, q.s.data());
        if (st != CB_OK) return st;
    }
    if (min_tokens > 0 && q.N < min_tokens) q.s.assign(L + 1, q.Nc);
    if (q.s[0] != 0 && q.s[0] != q.Nc)
        return fail(CB_E_SCHEDULE, "request %d: s[0] = %d must be 0 or the chunk token count %d",
                    b, q.s[0], q.Nc);
    for (int l = 0; l < L; ++l)
        if (q.s[l + 1] > q.s[l] || q.s[l + 1] < 0)
            return fail(CB_E_SCHEDULE,
                        "request %d: schedule must be non-increasing (s[%d]=%d, s[%d]=%d)", b, l,
                        q.s[l], l + 1, q.s[l + 1]);
    return CB_OK;
}

// Stacking offsets and the fetch program (copies and rotation jobs).
cb_status plan_layout(cb_plan* p) {
    int64_t G = 0, C = 0;
    for (ReqInfo& q : p->reqs) {
        q.G = (int)G;
        q.C = (int)C;
        G += q.N;
        C += q.Nc;
        if (G > (1 << 30)) return fail(CB_E_SHAPE, "batch too long (%lld tokens)", (long long)G);
    }
    p->Ntot = (int)G;
    p->Nctot = (int)C;
    if (p->Ntot == 0) return fail(CB_E_INVALID, "empty prompt");
    const size_t es = p->m->es(), row_elems = p->m->kvd();
    std::vector<int64_t> first_row(p->pool.size(), -1);
    std::vector<RotJob> copy, inplace;
    std::vector<QRotJob> qjobs[2];
    std::vector<int64_t> staged_at(p->pool.size(), -1);
    for (const ReqInfo& q : p->reqs)
        for (size_t c = 0; c < q.ids.size(); ++c) {
            const cb_chunk_kv& ck = p->pool[q.ids[c]];
            if (ck.kv_format != CB_KV_PLAIN) {
                const int b = ck.kv_format == CB_KV_U8 ? 0 : 1;
                const size_t code_bytes = (size_t)ck.n_tokens * row_elems / (b == 0 ? 1 : 2);
                const size_t qp_bytes = 4 * row_elems * sizeof(float);
                QRotJob j{};
                j.dst_row = q.G + q.offsets[c];
                j.n_tokens = ck.n_tokens;
                j.delta = q.offsets[c];
                if (!ck.on_host) {
                    j.k = (const uint8_t*)ck.k;
                    j.v = (const uint8_t*)ck.v;
                    j.qp = ck.qparams;
                    j.code_layer_stride = b == 0 ? ck.layer_stride : ck.layer_stride / 2;
                    j.qp_layer_stride = 4 * (int64_t)row_elems;
                } else if (ck.stage_k) {
                    if (staged_at[q.ids[c]] < 0) {
                        staged_at[q.ids[c]] = 0;
                        p->stage_copies.push_back(
                            {(const char*)ck.k, (const char*)ck.v, (const char*)ck.qparams,
                             (size_t)(b == 0 ? ck.layer_stride : ck.layer_stride / 2), code_bytes,
                             qp_bytes, (char*)ck.stage_k, (char*)ck.stage_v,
                             (char*)ck.stage_qparams});
                    }
                    j.k = (const uint8_t*)ck.stage_k;
                    j.v = (const uint8_t*)ck.stage_v;
                    j.qp = ck.stage_qparams;
                    j.code_layer_stride = (int64_t)code_bytes;
                    j.qp_layer_stride = 4 * (int64_t)row_elems;
                } else {
                    if (staged_at[q.ids[c]] < 0) {
                        staged_at[q.ids[c]] = (int64_t)p->stage_bytes;
                        p->qh2d.push_back({(const char*)ck.k, (const char*)ck.v,
                                           (const char*)ck.qparams,
                                           (size_t)(b == 0 ? ck.layer_stride : ck.layer_stride / 2),
                                           code_bytes, qp_bytes, p->stage_bytes});
                        p->stage_bytes += 2 * align_up(code_bytes, 256) +
                                          align_up(qp_bytes * p->L, 256);
                    }
                    // offsets into the staging area until the workspace exists
                    const size_t o = (size_t)staged_at[q.ids[c]];
                    j.k = (const uint8_t*)(uintptr_t)o;
                    j.v = (const uint8_t*)(uintptr_t)(o + align_up(code_bytes, 256));
                    j.qp = (const float*)(uintptr_t)(o + 2 * align_up(code_bytes, 256));
                    j.code_layer_stride = 0;                       // one layer staged at a time
                    j.qp_layer_stride = 4 * (int64_t)row_elems;    // every layer's parameters
                    j.staged = 1;
                }
                qjobs[b].push_back(j);
                continue;
            }
            RotJob j{};
            j.src_layer_stride = ck.layer_stride;
            j.dst_row = q.G + q.offsets[c];
            j.n_tokens = ck.n_tokens;
            j.delta = q.offsets[c];       // chunk-local position 0 -> real position o_c
            if (!ck.on_host) {
                j.k_src = ck.k;
                j.v_src = ck.v;
                copy.push_back(j);
            } else if (ck.stage_k) {
                const size_t bytes = (size_t)ck.n_tokens * row_elems * es;
                if (first_row[q.ids[c]] < 0) {
                    first_row[q.ids[c]] = j.dst_row;
                    p->stage_copies.push_back({(const char*)ck.k, (const char*)ck.v, nullptr,
                                               (size_t)ck.layer_stride * es, bytes, 0,
                                               (char*)ck.stage_k, (char*)ck.stage_v, nullptr});
                }
                j.k_src = ck.stage_k;
                j.v_src = ck.stage_v;
                j.src_layer_stride = (int64_t)ck.n_tokens * row_elems;
                copy.push_back(j);
            } else if (first_row[q.ids[c]] < 0) {
                first_row[q.ids[c]] = j.dst_row;
                p->h2d.push_back({(const char*)ck.k, (const char*)ck.v,
                                  (size_t)ck.layer_stride * es, ck.n_tokens * row_elems * es,
                                  j.dst_row});
                inplace.push_back(j);     // k_src = v_src = null: rotate where it landed
            } else {
                const size_t off = (size_t)first_row[q.ids[c]] * row_elems * es;
                j.k_src = (const char*)p->fused_k + off;
                j.v_src = (const char*)p->fused_v + off;
                j.src_layer_stride = layer_elems(p);
                copy.push_back(j);
            }
        }
    p->lookahead = p->h2d.empty() && p->qh2d.empty() && p->stage_copies.empty()
                       ? 2 : std::max(2, p->L);
    for (int b = 0; b < 2; ++b)
        for (size_t i = 0; i < qjobs[b].size(); ++i) {
            if (i % kMaxQRotJobs == 0) p->qjobs[b].push_back(QRotJobs{});
            QRotJobs& js = p->qjobs[b].back();
            js.j[js.n++] = qjobs[b][i];
            js.max_tokens = std::max(js.max_tokens, qjobs[b][i].n_tokens);
        }
    for (auto [src, dst] : {std::make_pair(&copy, &p->jobs_copy),
                            std::make_pair(&inplace, &p->jobs_inplace)})
        for (size_t i = 0; i < src->size(); ++i) {
            if (i % kMaxRotJobs == 0) dst->push_back(RotJobs{});
            RotJobs& js = dst->back();
            js.j[js.n++] = (*src)[i];
            js.max_tokens = std::max(js.max_tokens, (*src)[i].n_tokens);
        }
    return CB_OK;
}

// A single request as a batch of one (its chunks form the pool).
cb_status validate_request(cb_model* m, const cb_request* r, const cb_outputs* o, cb_plan* p) {
    if (!r || !o) return fail(CB_E_INVALID, "request/outputs is NULL");
    if (!o->fused_k || !o->fused_v) return fail(CB_E_INVALID, "fused_k/fused_v are required");
    if (!r->x0) return fail(CB_E_INVALID, "x0 is NULL");
    if (r->n_chunks < 0 || r->n_suffix < 0) return fail(CB_E_INVALID, "negative counts");
    if (r->n_chunks > 0 && (!r->chunks || !r->chunk_offsets))
        return fail(CB_E_INVALID, "chunks/chunk_offsets are NULL");
    if (r->dev_mode < 0 || r->dev_mode > CB_DEV_ATTN)
        return fail(CB_E_INVALID, "dev_mode %d", r->dev_mode);
    if (r->dev_mode == CB_DEV_ATTN && m->cfg.dtype != CB_BF16)
        return fail(CB_E_UNSUPPORTED, "dev_mode CB_DEV_ATTN needs a bf16 model");
    if ((r->dev_mode == CB_DEV_GIVEN) != (r->given_scores != nullptr))
        return fail(CB_E_INVALID, "given_scores goes with dev_mode CB_DEV_GIVEN, and only with it");
    if (r->given_scores && mem_kind(r->given_scores) != MemKind::Device)
        return fail(CB_E_INVALID, "given_scores must be device memory");
    p->L = m->cfg.n_layers;
    ReqInfo q;
    int64_t o_next = 0;
    for (int c = 0; c < r->n_chunks; ++c) {
        const cb_chunk_kv& ck = r->chunks[c];
        cb_status st = check_chunk(m, ck, c);
        if (st != CB_OK) return st;
        if (r->chunk_offsets[c] != o_next)
            return fail(CB_E_INVALID, "chunk %d offset %d: offsets must start at 0 and be contiguous",
                        c, r->chunk_offsets[c]);
        p->pool.push_back(ck);
        q.ids.push_back(c);
        q.offsets.push_back((int)o_next);
        o_next += ck.n_tokens;
        if (o_next > (1 << 30)) return fail(CB_E_SHAPE, "prompt too long");
    }
    if (o_next + r->n_suffix > (1 << 30)) return fail(CB_E_SHAPE, "prompt too long");
    q.Nc = (int)o_next;
    q.Ns = r->n_suffix;
    q.N = q.Nc + q.Ns;
    if (q.N == 0) return fail(CB_E_INVALID, "empty prompt");
    cb_status st = request_schedule(p, q, r->schedule, r->recompute_bp, r->schedule_kind,
                                    r->min_tokens, 0);
    if (st != CB_OK) return st;
    p->reqs.push_back(std::move(q));
    p->x0 = r->x0;
    p->dev_mode = r->dev_mode;
    p->given = r->given_scores;
    p->fused_k = o->fused_k;
    p->fused_v = o->fused_v;
    p->sel_idx = o->sel_idx;
    p->hidden_out = o->hidden_out;
    p->deviation = o->deviation;
    return plan_layout(p);
}

cb_status validate_batch(cb_model* m, const cb_batch_request* r, const cb_batch_outputs* o,
                         cb_plan* p) {
    if (!r || !o) return fail(CB_E_INVALID, "request/outputs is NULL");
    if (!o->fused_k || !o->fused_v) return fail(CB_E_INVALID, "fused_k/fused_v are required");
    if (!r->x0) return fail(CB_E_INVALID, "x0 is NULL");
    if (r->n_requests <= 0 || !r->items) return fail(CB_E_INVALID, "no requests");
    if (r->n_pool < 0 || (r->n_pool > 0 && !r->pool)) return fail(CB_E_INVALID, "pool is NULL");
    if (r->dev_mode < 0 || r->dev_mode > CB_DEV_ATTN)
        return fail(CB_E_INVALID, "dev_mode %d", r->dev_mode);
    if (r->dev_mode == CB_DEV_ATTN && m->cfg.dtype != CB_BF16)
        return fail(CB_E_UNSUPPORTED, "dev_mode CB_DEV_ATTN needs a bf16 model");
    if ((r->dev_mode == CB_DEV_GIVEN) != (r->given_scores != nullptr))
        return fail(CB_E_INVALID, "given_scores goes with dev_mode CB_DEV_GIVEN, and only with it");
    if (r->given_scores && mem_kind(r->given_scores) != MemKind::Device)
        return fail(CB_E_INVALID, "given_scores must be device memory");
    p->L = m->cfg.n_layers;
    p->pool.assign(r->pool, r->pool + r->n_pool);
    std::vector<char> checked(r->n_pool, 0);
    for (int b = 0; b < r->n_requests; ++b) {
        const cb_batch_item& it = r->items[b];
        if (it.n_chunks < 0 || it.n_suffix < 0)
            return fail(CB_E_INVALID, "request %d: negative counts", b);
        if (it.n_chunks > 0 && !it.chunk_ids)
            return fail(CB_E_INVALID, "request %d: chunk_ids is NULL", b);
        ReqInfo q;
        int64_t o_next = 0;
        for (int c = 0; c < it.n_chunks; ++c) {
            const int id = it.chunk_ids[c];
            if (id < 0 || id >= r->n_pool)
                return fail(CB_E_INVALID, "request %d: chunk id %d not in the pool", b, id);
            if (!checked[id]) {
                cb_status st = check_chunk(m, p->pool[id], id);
                if (st != CB_OK) return st;
                checked[id] = 1;
            }
            q.ids.push_back(id);
            q.offsets.push_back((int)o_next);
            o_next += p->pool[id].n_tokens;
            if (o_next > (1 << 30)) return fail(CB_E_SHAPE, "request %d too long", b);
        }
        if (o_next + it.n_suffix > (1 << 30)) return fail(CB_E_SHAPE, "request %d too long", b);
        q.Nc = (int)o_next;
        q.Ns = it.n_suffix;
        q.N = q.Nc + q.Ns;
        if (q.N == 0) return fail(CB_E_INVALID, "request %d is empty", b);
        cb_status st = request_schedule(p, q, it.schedule, r->recompute_bp, r->schedule_kind,
                                        r->min_tokens, b);
        if (st != CB_OK) return st;
        p->reqs.push_back(std::move(q));
    }
    p->x0 = r->x0;
    p->dev_mode = r->dev_mode;
    p->given = r->given_scores;
    p->fused_k = o->fused_k;
    p->fused_v = o->fused_v;
    p->sel_idx = o->sel_idx;
    p->hidden_out = o->hidden_out;
    p->deviation = o->deviation;
    return plan_layout(p);
}

cb_status ensure_rope(cb_model* m, int n_pos) {
    if (m->rope.n_pos >= n_pos) return CB_OK;
    return get_rope(m->cfg.rope_base, m->cfg.head_dim, n_pos, &m->rope);
}

int max_position(const cb_plan* p) {
    int mx = 0;
    for (const ReqInfo& q : p->reqs) mx = std::max(mx, q.pos0 + q.N);
    return mx;
}

// Workspace, events and initial rows of a validated plan.
cb_status plan_setup(cb_plan* p) {
    cb_status st = ensure_rope(p->m, max_position(p));
    if (st == CB_OK) st = plan_alloc(p);
    if (st == CB_OK) st = plan_events(p);
    if (st == CB_OK) st = plan_start(p);
    return st;
}

cb_status run_all_layers(cb_plan* p) {
    cb_status st = CB_OK;
    int fetched = 0;
    for (int l = 0; l < p->L && st == CB_OK; ++l) {
        // queue the fetch of the next layer before layer l (the side stream
        // runs it during layer l; how far it may run ahead is set by the
        // event waits in do_fetch, host-side queueing just keeps pace)
        for (; fetched < p->L && fetched <= l + 1 && st == CB_OK; ++fetched)
            st = do_fetch(p, fetched);
        if (st == CB_OK) st = do_layer(p, l);
        if (st == CB_OK) p->next_layer++;
    }
    return st;
}

}  // namespace

// ================================================================ C ABI
extern "C" {

int cb_abi_version(void) { return CB_ABI_VERSION; }

const char* cb_last_error(void) { return g_err.c_str(); }

cb_status cb_schedule(int32_t n_chunk_tokens, int32_t recompute_bp, int32_t kind,
                      int32_t n_layers, int32_t* s_out) {
    if (!s_out) return fail(CB_E_INVALID, "s_out is NULL");
    return make_schedule(n_chunk_tokens, recompute_bp, kind, n_layers, s_out);
}

cb_status cb_model_create(const cb_model_cfg* cfg, const cb_layer_weights* layers,
                          const void* final_norm, cb_model** out) {
    if (!out) return fail(CB_E_INVALID, "out is NULL");
    *out = nullptr;
    cb_status st = validate_cfg(cfg);
    if (st != CB_OK) return st;
    if (!layers) return fail(CB_E_INVALID, "layers is NULL");
    for (int l = 0; l < cfg->n_layers; ++l) {
        const cb_layer_weights& w = layers[l];
        const void* ps[] = {w.attn_norm, w.wq, w.wk, w.wv, w.wo, w.mlp_norm, w.w_gate, w.w_up, w.w_down};
        for (const void* q : ps) {
            if (!q) return fail(CB_E_INVALID, "layer %d has a NULL weight", l);
            if (!aligned_to(q, 16)) return fail(CB_E_SHAPE, "layer %d weight not 16-byte aligned", l);
        }
    }
    if (final_norm && !aligned_to(final_norm, 16))
        return fail(CB_E_SHAPE, "final_norm not 16-byte aligned");
    cb_model* m = new cb_model();
    m->cfg = *cfg;
    m->w.assign(layers, layers + cfg->n_layers);
    m->final_norm = final_norm;
    if (hipGetDevice(&m->device) != hipSuccess) {
        delete m;
        return fail(CB_E_HIP, "hipGetDevice failed");
    }
    st = get_rope(cfg->rope_base, cfg->head_dim, 16384, &m->rope);
    if (st != CB_OK) {
        delete m;
        return st;
    }
    if (hipStreamCreateWithFlags(&m->side, hipStreamNonBlocking) != hipSuccess) {
        delete m;
        return fail(CB_E_HIP, "side stream creation failed");
    }
    // Workspaces come from a pool of the model's own that keeps freed memory
    // (a plan's workspace is re-mapped on every call otherwise).
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = m->device;
    if (hipMemPoolCreate(&m->pool, &props) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipStreamDestroy(m->side);
        delete m;
        return fail(CB_E_HIP, "memory pool creation failed");
    }
    uint64_t keep = UINT64_MAX;
    (void)hipMemPoolSetAttribute(m->pool, hipMemPoolAttrReleaseThreshold, &keep);
    *out = m;
    return CB_OK;
}

void cb_model_destroy(cb_model* m) {
    if (!m) return;
    if (m->side) {
        (void)hipStreamSynchronize(m->side);
        (void)hipStreamDestroy(m->side);
    }
    if (m->pool) {
        (void)hipDeviceSynchronize();   // plans free their workspace in stream order
        (void)hipMemPoolDestroy(m->pool);
    }
    for (auto e : m->event_pool) (void)hipEventDestroy(e);
    for (auto e : m->timing_pool) (void)hipEventDestroy(e);
    for (auto& r : m->prof_pending) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    delete m;
}

cb_status cb_plan_create(cb_model* m, const cb_request* r, const cb_outputs* o, void* stream,
                         cb_plan** out) {
    if (!m || !out) return fail(CB_E_INVALID, "model/out is NULL");
    *out = nullptr;
    cb_plan* p = new cb_plan();
    p->m = m;
    p->stream = as_stream(stream);
    cb_status st = validate_request(m, r, o, p);
    if (st != CB_OK) {
        delete p;
        return st;
    }
    if (o->sel_count)
        for (int l = 0; l < p->L; ++l) o->sel_count[l] = p->reqs[0].s[l + 1];
    st = plan_setup(p);
    if (st != CB_OK) {
        plan_free(p);
        return st;
    }
    *out = p;
    return CB_OK;
}

cb_status cb_model_set_workspace(cb_model* m, void* ws, int64_t bytes) {
    if (!m) return fail(CB_E_INVALID, "model is NULL");
    if (bytes < 0) return fail(CB_E_INVALID, "negative workspace size");
    if (ws) {
        if (!aligned_to(ws, 256)) return fail(CB_E_SHAPE, "workspace must be 256-byte aligned");
        if (mem_kind(ws) != MemKind::Device)
            return fail(CB_E_INVALID, "workspace must be device memory");
    }
    m->ws_user = ws;
    m->ws_user_bytes = ws ? (size_t)bytes : 0;
    m->ws_limit = ws ? 0 : (size_t)bytes;
    return CB_OK;
}

cb_status cb_workspace_size(cb_model* m, const cb_request* r, int64_t* bytes) {
    if (!m || !r || !bytes) return fail(CB_E_INVALID, "NULL argument");
    // the request is validated as cb_plan_create would; outputs only give
    // addresses to the layout and are never touched
    cb_outputs o{};
    char probe_out[256];
    o.fused_k = o.fused_v = probe_out;
    cb_plan* p = new cb_plan();
    p->m = m;
    cb_status st = validate_request(m, r, &o, p);
    if (st == CB_OK) {
        int max_rows = 0;
        *bytes = (int64_t)plan_bytes(p, &max_rows);
    }
    delete p;
    return st;
}

cb_status cb_fetch_kv(cb_plan* p, int32_t layer) {
    if (!p) return fail(CB_E_INVALID, "plan is NULL");
    if (layer < 0 || layer >= p->L) return fail(CB_E_INVALID, "layer %d out of range", layer);
    return do_fetch(p, layer);
}

cb_status cb_prefill_layer(cb_plan* p, int32_t layer) {
    if (!p) return fail(CB_E_INVALID, "plan is NULL");
    if (layer != p->next_layer)
        return fail(CB_E_BAD_STATE, "layer %d requested, layer %d is next", layer, p->next_layer);
    cb_status st = do_fetch(p, layer);
    if (st != CB_OK) return st;
    st = do_layer(p, layer);
    if (st != CB_OK) return st;
    p->next_layer++;
    return CB_OK;
}

cb_status cb_synchronize(cb_plan* p) {
    if (!p) return fail(CB_E_INVALID, "plan is NULL");
    CB_HIP(hipStreamSynchronize(p->m->side));
    CB_HIP(hipStreamSynchronize(p->stream));
    return CB_OK;
}

void cb_plan_destroy(cb_plan* p) { plan_free(p); }

cb_status cb_blend(cb_model* m, const cb_request* r, const cb_outputs* o, void* stream) {
    cb_plan* p = nullptr;
    cb_status st = cb_plan_create(m, r, o, stream, &p);
    if (st != CB_OK) return st;
    st = run_all_layers(p);
    plan_free(p);
    return st;
}

cb_status cb_blend_batch(cb_model* m, const cb_batch_request* r, const cb_batch_outputs* o,
                         void* stream) {
    if (!m) return fail(CB_E_INVALID, "model is NULL");
    cb_plan* p = new cb_plan();
    p->m = m;
    p->stream = as_stream(stream);
    cb_status st = validate_batch(m, r, o, p);
    if (st != CB_OK) {
        delete p;
        return st;
    }
    if (o->sel_count)
        for (size_t b = 0; b < p->reqs.size(); ++b)
            for (int l = 0; l < p->L; ++l) o->sel_count[b * p->L + l] = p->reqs[b].s[l + 1];
    st = plan_setup(p);
    if (st == CB_OK) st = run_all_layers(p);
    plan_free(p);
    return st;
}

cb_status cb_prefill(cb_model* m, const void* x0, int32_t n_tokens, int32_t pos0, void* k_out,
                     void* v_out, float* hidden_out, void* stream) {
    if (!m || !x0 || !k_out || !v_out) return fail(CB_E_INVALID, "NULL argument");
    if (n_tokens <= 0 || pos0 < 0 || (int64_t)pos0 + n_tokens > (1 << 30))
        return fail(CB_E_INVALID, "n_tokens %d, pos0 %d", n_tokens, pos0);
    cb_plan* p = new cb_plan();
    p->m = m;
    p->stream = as_stream(stream);
    p->L = m->cfg.n_layers;
    ReqInfo q;
    q.Ns = n_tokens;
    q.N = n_tokens;
    q.pos0 = pos0;
    q.s.assign(p->L + 1, 0);
    p->reqs.push_back(std::move(q));
    p->kv_pos0 = pos0;
    p->x0 = x0;
    p->fused_k = k_out;
    p->fused_v = v_out;
    p->hidden_out = hidden_out;
    cb_status st = plan_layout(p);
    if (st == CB_OK) st = plan_setup(p);
    if (st == CB_OK) st = run_all_layers(p);
    plan_free(p);
    return st;
}

cb_status cb_lm_head(cb_model* m, const float* x, int32_t rows, const void* final_norm,
                     const void* w_lm, int32_t vocab, float* logits, int32_t* argmax,
                     void* stream) {
    if (m && !final_norm) final_norm = m->final_norm;
    if (!m || !x || !w_lm || !logits) return fail(CB_E_INVALID, "NULL argument");
    if (!final_norm)
        return fail(CB_E_INVALID, "no final_norm: pass one or give it to cb_model_create");
    if (rows <= 0 || vocab <= 0) return fail(CB_E_INVALID, "rows %d, vocab %d", rows, vocab);
    const cb_model_cfg& c = m->cfg;
    if (!aligned_to(x, 16) || !aligned_to(w_lm, 16) || !aligned_to(final_norm, 16))
        return fail(CB_E_SHAPE, "x, final_norm and w_lm must be 16-byte aligned");
    const hipStream_t st = as_stream(stream);
    const size_t es = m->es();
    void* hn = nullptr;
    if (hipMallocFromPoolAsync(&hn, (size_t)rows * c.d_model * es, m->pool, st) != hipSuccess) {
        (void)hipGetLastError();
        return fail(CB_E_OOM, "LM head scratch");
    }
    cb_status status = CB_OK;
    auto run = [&]() -> cb_status {
        CB_HIP(launch_rmsnorm(F32, x, nullptr, c.dtype, final_norm, hn, nullptr, rows, c.d_model,
                              c.rms_eps, st));
        for (int r = 0; r < rows; ++r) {
            GemvArgs g{};
            g.x = (const char*)hn + (size_t)r * c.d_model * es;
            g.b0 = w_lm;
            g.N = vocab;
            g.K = c.d_model;
            g.out0 = logits + (int64_t)r * vocab;
            Span sp(m, CB_K_DECODE_GEMV, st, 2.0 * vocab * c.d_model,
                    (double)vocab * c.d_model * es + vocab * 4.0);
            CB_HIP(launch_gemv(c.dtype, EPI_STORE_F32, g, st));
        }
        if (argmax) CB_HIP(launch_argmax(logits, rows, vocab, vocab, argmax, st));
        return CB_OK;
    };
    status = run();
    (void)hipFreeAsync(hn, st);
    return status;
}

cb_status cb_decode_step(cb_model* m, const void* x, int32_t n_ctx, const void* fused_k,
                         const void* fused_v, int64_t layer_rows, void* k_new, void* v_new,
                         float* hidden_out, void* stream) {
    if (!m || !x || !k_new || !v_new || !hidden_out) return fail(CB_E_INVALID, "NULL argument");
    if (n_ctx < 0 || layer_rows < n_ctx || (n_ctx > 0 && (!fused_k || !fused_v)))
        return fail(CB_E_INVALID, "n_ctx %d, layer_rows %lld", n_ctx, (long long)layer_rows);
    const cb_model_cfg& c = m->cfg;
    const int G = c.n_q_heads / c.n_kv_heads;
    if (G > 8) return fail(CB_E_UNSUPPORTED, "more than 8 query heads per KV head");
    if (!aligned_to(x, 16) || !aligned_to(fused_k, 16) || !aligned_to(fused_v, 16) ||
        !aligned_to(k_new, 16) || !aligned_to(v_new, 16) || !aligned_to(hidden_out, 16))
        return fail(CB_E_SHAPE, "buffers must be 16-byte aligned");
    cb_status st0 = ensure_rope(m, n_ctx + 1);
    if (st0 != CB_OK) return st0;
    const hipStream_t st = as_stream(stream);
    const size_t es = m->es(), d = c.d_model, qd = m->qd(), kvd = m->kvd(), F = c.ffn_dim;
    // split-attention partials: [Hq][segments][d_head] outputs, [Hq][segments][2] statistics
    const size_t nseg = (size_t)decode_attention_segments(n_ctx);
    size_t off = 0;
    auto take = [&](size_t b) { const size_t o = off; off = align_up(off + b, 256); return o; };
    const size_t oX = take(d * 4), oH = take(d * 4), oN = take(d * es), oQ = take(qd * es),
                 oA = take(qd * es), oF = take(F * es),
                 oP = take((size_t)c.n_q_heads * nseg * c.head_dim * 4),
                 oM = take((size_t)c.n_q_heads * nseg * 2 * 4);
    char* ws = nullptr;
    if (hipMallocFromPoolAsync((void**)&ws, off, m->pool, st) != hipSuccess) {
        (void)hipGetLastError();
        return fail(CB_E_OOM, "decode scratch of %zu bytes", off);
    }
    float* X = (float*)(ws + oX);
    float* Hres = (float*)(ws + oH);
    void *Hn = ws + oN, *Q = ws + oQ, *att = ws + oA, *act = ws + oF;
    const double ctx_bytes = 2.0 * (n_ctx + 1) * kvd * es;
    auto run = [&]() -> cb_status {
        for (int l = 0; l < c.n_layers; ++l) {
            const cb_layer_weights& w = m->w[l];
            const bool last = l + 1 == c.n_layers;
            char* kl = (char*)k_new + (size_t)l * kvd * es;
            char* vl = (char*)v_new + (size_t)l * kvd * es;
            CB_HIP(launch_rmsnorm(l == 0 ? c.dtype : F32, l == 0 ? x : (const void*)X, nullptr,
                                  c.dtype, w.attn_norm, Hn, l == 0 ? X : nullptr, 1, c.d_model,
                                  c.rms_eps, st));
            {
                GemvArgs g{};
                g.x = Hn; g.b0 = w.wq; g.b1 = w.wk; g.b2 = w.wv;
                g.N = (int)(qd + 2 * kvd); g.K = (int)d; g.n0 = (int)qd; g.n1 = (int)kvd;
                g.out0 = Q; g.out1 = kl; g.out2 = vl;
                g.rope = m->rope; g.pos = n_ctx; g.head_dim = c.head_dim;
                Span sp(m, CB_K_DECODE_GEMV, st, 2.0 * g.N * d, ((double)g.N * d + g.N) * es);
                CB_HIP(launch_gemv(c.dtype, EPI_QKV, g, st));
            }
            {
                DecodeAttnArgs a{};
                a.q = Q;
                a.k = (const char*)fused_k + (size_t)l * layer_rows * kvd * es;
                a.v = (const char*)fused_v + (size_t)l * layer_rows * kvd * es;
                a.k_new = kl; a.v_new = vl; a.out = att;
                a.n_ctx = n_ctx; a.n_kv_heads = c.n_kv_heads; a.group = G;
                a.head_dim = c.head_dim;
                a.scale = 1.0f / sqrtf((float)c.head_dim);
                a.part_o = (float*)(ws + oP);
                a.part_ml = (float*)(ws + oM);
                Span sp(m, CB_K_DECODE_ATTN, st, 4.0 * qd * (n_ctx + 1), ctx_bytes);
                CB_HIP(launch_decode_attention(c.dtype, a, st));
            }
            {
                GemvArgs g{};
                g.x = att; g.b0 = w.wo; g.N = (int)d; g.K = (int)qd;
                g.out0 = Hres; g.resid = X;
                Span sp(m, CB_K_DECODE_GEMV, st, 2.0 * d * qd, (double)d * qd * es + d * 8.0);
                CB_HIP(launch_gemv(c.dtype, EPI_RESID, g, st));
            }
            CB_HIP(launch_rmsnorm(F32, Hres, nullptr, c.dtype, w.mlp_norm, Hn, nullptr, 1,
                                  c.d_model, c.rms_eps, st));
            {
                GemvArgs g{};
                g.x = Hn; g.b0 = w.w_gate; g.b1 = w.w_up; g.N = (int)F; g.K = (int)d;
                g.out0 = act;
                Span sp(m, CB_K_DECODE_GEMV, st, 4.0 * F * d, 2.0 * F * d * es + F * es);
                CB_HIP(launch_gemv(c.dtype, EPI_SWIGLU, g, st));
            }
            {
                GemvArgs g{};
                g.x = act; g.b0 = w.w_down; g.N = (int)d; g.K = (int)F;
                g.out0 = last ? hidden_out : X; g.resid = Hres;
                Span sp(m, CB_K_DECODE_GEMV, st, 2.0 * d * F, (double)d * F * es + d * 8.0);
                CB_HIP(launch_gemv(c.dtype, EPI_RESID, g, st));
            }
        }
        return CB_OK;
    };
    const cb_status status = run();
    (void)hipFreeAsync(ws, st);
    return status;
}

cb_status cb_profile_enable(cb_model* m, int32_t enable) {
    if (!m) return fail(CB_E_INVALID, "model is NULL");
    if (enable) {
        cb_kernel_stat tmp[CB_K_COUNT];
        cb_status st = cb_profile_read(m, tmp);   // drain anything pending
        if (st != CB_OK) return st;
        std::lock_guard<std::mutex> lk(m->mu);
        for (auto& x : m->stats) x = cb_kernel_stat{};
    }
    m->prof = enable != 0;
    return CB_OK;
}

cb_status cb_profile_read(cb_model* m, cb_kernel_stat* stats) {
    if (!m || !stats) return fail(CB_E_INVALID, "NULL argument");
    std::vector<cb_model::ProfRec> recs;
    {
        std::lock_guard<std::mutex> lk(m->mu);
        recs.swap(m->prof_pending);
    }
    cb_status st = CB_OK;
    for (auto& r : recs) {
        float ms = 0.f;
        if (st == CB_OK) {
            hipError_t e = hipEventSynchronize(r.b);
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
            if (e != hipSuccess) st = fail(CB_E_HIP, "profile event: %s", hipGetErrorString(e));
        }
        std::lock_guard<std::mutex> lk(m->mu);
        if (st == CB_OK) {
            cb_kernel_stat& k = m->stats[r.cls];
            k.launches += 1;
            k.total_ms += ms;
            k.flops += r.flops;
            k.bytes += r.bytes;
        }
        m->timing_pool.push_back(r.a);
        m->timing_pool.push_back(r.b);
    }
    std::lock_guard<std::mutex> lk(m->mu);
    for (int i = 0; i < CB_K_COUNT; ++i) stats[i] = m->stats[i];
    return st;
}

// ------------------------------------------------------------- kernel-level
cb_status cb_rope_rerotate(int32_t dtype, const void* k_in, void* k_out, const void* v_in,
                           void* v_out, int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                           int32_t delta, double rope_base, void* stream) {
    if (dtype != CB_F32 && dtype != CB_BF16) return fail(CB_E_INVALID, "dtype %d", dtype);
    if (n_tokens > 0 && (!k_in || !k_out || (v_in && !v_out)))
        return fail(CB_E_INVALID, "NULL buffer");
    if (n_tokens < 0 || n_heads <= 0 || head_dim <= 0 || head_dim % 8)
        return fail(CB_E_SHAPE, "bad sizes (head_dim must be a multiple of 8)");
    if (!(rope_base > 1.0)) return fail(CB_E_INVALID, "rope_base must be > 1");
    if (delta == INT32_MIN) return fail(CB_E_INVALID, "delta out of range");
    RopeTab rt;
    const int ad = delta < 0 ? -delta : delta;
    cb_status st = get_rope(rope_base, head_dim, ad + 1, &rt);
    if (st != CB_OK) return st;
    RotJobs js{};
    RotJob& j = js.j[0];
    j.k_src = k_in == k_out ? nullptr : k_in;
    j.v_src = v_in;
    j.n_tokens = n_tokens;
    j.delta = delta;
    js.n = 1;
    js.max_tokens = n_tokens;
    CB_HIP(launch_rerotate(dtype, js, 0, k_out, v_out, n_heads, head_dim, rt, as_stream(stream)));
    return CB_OK;
}

cb_status cb_quantize_kv(int32_t dtype, const void* x, int32_t n_layers, int32_t n_tokens,
                         int32_t row, int64_t x_layer_stride, int32_t bits, void* codes,
                         float* scale, float* zero, int64_t param_stride, void* stream) {
    if (dtype != CB_F32 && dtype != CB_BF16) return fail(CB_E_INVALID, "dtype %d", dtype);
    if (bits != 8 && bits != 4) return fail(CB_E_INVALID, "bits must be 8 or 4, got %d", bits);
    if (n_layers < 0 || n_tokens < 0) return fail(CB_E_SHAPE, "negative sizes");
    if (n_layers == 0 || n_tokens == 0) return CB_OK;
    if (row <= 0 || row % 8) return fail(CB_E_SHAPE, "row %d must be a positive multiple of 8", row);
    if (x_layer_stride < (int64_t)n_tokens * row || param_stride < row)
        return fail(CB_E_SHAPE, "layer stride below n_tokens*row or param_stride below row");
    if (!x || !codes || !scale || !zero) return fail(CB_E_INVALID, "NULL buffer");
    if (!aligned_to(x, 16) || !aligned_to(codes, 16) || !aligned_to(scale, 16) ||
        !aligned_to(zero, 16) || (x_layer_stride * elem_size(dtype)) % 16 || param_stride % 4)
        return fail(CB_E_SHAPE, "buffers, the layer stride and param_stride must be 16-byte aligned");
    const hipStream_t st = as_stream(stream);
    const size_t wsb = quantize_workspace(n_layers, n_tokens, row);
    void* ws = nullptr;
    if (hipMallocAsync(&ws, wsb, st) != hipSuccess) {
        (void)hipGetLastError();
        return fail(CB_E_OOM, "quantization scratch of %zu bytes", wsb);
    }
    const hipError_t e = launch_quantize(dtype, x, n_layers, n_tokens, row, x_layer_stride, bits,
                                         codes, scale, zero, param_stride, ws, wsb, st);
    (void)hipFreeAsync(ws, st);
    if (e != hipSuccess) return fail(CB_E_HIP, "quantize launch: %s", hipGetErrorString(e));
    return CB_OK;
}

cb_status cb_dequant_rerotate(int32_t dtype, int32_t kv_format, const void* k_codes,
                              const void* v_codes, const float* qparams, void* k_out,
                              void* v_out, int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                              int32_t delta, double rope_base, void* stream) {
    if (dtype != CB_F32 && dtype != CB_BF16) return fail(CB_E_INVALID, "dtype %d", dtype);
    if (kv_format != CB_KV_U8 && kv_format != CB_KV_U4)
        return fail(CB_E_INVALID, "kv_format %d is not a quantized format", kv_format);
    if (n_tokens > 0 && (!k_codes || !k_out || !qparams || (v_codes && !v_out)))
        return fail(CB_E_INVALID, "NULL buffer");
    if (n_tokens < 0 || n_heads <= 0 || head_dim <= 0 || head_dim % 8)
        return fail(CB_E_SHAPE, "bad sizes (head_dim must be a multiple of 8)");
    if (!aligned_to(k_codes, 16) || !aligned_to(v_codes, 16) || !aligned_to(qparams, 16) ||
        !aligned_to(k_out, 16) || !aligned_to(v_out, 16))
        return fail(CB_E_SHAPE, "buffers must be 16-byte aligned");
    if (!(rope_base > 1.0)) return fail(CB_E_INVALID, "rope_base must be > 1");
    if (delta == INT32_MIN) return fail(CB_E_INVALID, "delta out of range");
    if (n_tokens == 0) return CB_OK;
    RopeTab rt;
    const int ad = delta < 0 ? -delta : delta;
    cb_status st = get_rope(rope_base, head_dim, ad + 1, &rt);
    if (st != CB_OK) return st;
    QRotJobs js{};
    QRotJob& j = js.j[0];
    j.k = (const uint8_t*)k_codes;
    j.v = (const uint8_t*)v_codes;
    j.qp = qparams;
    j.n_tokens = n_tokens;
    j.delta = delta;
    js.n = 1;
    js.max_tokens = n_tokens;
    CB_HIP(launch_dequant_rerotate(dtype, kv_format == CB_KV_U8 ? 8 : 4, js, 0, k_out, v_out,
                                   n_heads, head_dim, rt, as_stream(stream)));
    return CB_OK;
}

cb_status cb_deviation(int32_t dtype, const void* k_new, const void* v_new, const void* k_cached,
                       const void* v_cached, int32_t n_rows, int32_t row_elems, int32_t dev_mode,
                       float* dev_out, void* stream) {
    if (dtype != CB_F32 && dtype != CB_BF16) return fail(CB_E_INVALID, "dtype %d", dtype);
    if (dev_mode < 0 || dev_mode > 2) return fail(CB_E_INVALID, "dev_mode %d", dev_mode);
    if (!dev_out || !k_new || !k_cached || !v_new || !v_cached)
        return fail(CB_E_INVALID, "NULL buffer");
    if (n_rows < 0 || row_elems <= 0 || row_elems % 8)
        return fail(CB_E_SHAPE, "row_elems must be a positive multiple of 8");
    ReqTab t{};
    t.n = 1;
    t.max_c = n_rows;
    t.r[0].n_c = n_rows;
    CB_HIP(launch_deviation(dtype, k_new, v_new, k_cached, v_cached, nullptr, t, row_elems,
                            dev_mode, dev_out, as_stream(stream)));
    return CB_OK;
}

cb_status cb_attention_deviation(int32_t dtype, const void* q, const void* k_new,
                                 const void* k_cached, int32_t n, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim, float* dev_out,
                                 void* stream) {
    if (dtype != CB_BF16) return fail(CB_E_UNSUPPORTED, "attention deviation needs bf16 (dtype %d)", dtype);
    if (n < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads)
        return fail(CB_E_SHAPE, "bad sizes");
    if (head_dim != 64 && head_dim != 128) return fail(CB_E_UNSUPPORTED, "head_dim %d", head_dim);
    if (n == 0) return CB_OK;
    if (!q || !k_new || !k_cached || !dev_out) return fail(CB_E_INVALID, "NULL buffer");
    const hipStream_t st = as_stream(stream);
    const size_t need = attention_deviation_workspace(n_q_heads, n);
    void* ws = nullptr;
    if (hipMallocAsync(&ws, need, st) != hipSuccess) {
        (void)hipGetLastError();
        return fail(CB_E_OOM, "attention deviation workspace of %zu bytes", need);
    }
    AttnDevArgs a{};
    a.q = q; a.k_new = k_new; a.k_cached = k_cached;
    a.n_q_heads = n_q_heads; a.n_kv_heads = n_kv_heads; a.head_dim = head_dim;
    a.part = static_cast<float*>(ws); a.part_stride = n;
    const AttnDevReq r{0, n, 0, 0, 0};
    const hipError_t e = launch_attention_deviation(dtype, a, &r, 1, dev_out, st);
    (void)hipFreeAsync(ws, st);
    if (e != hipSuccess) return fail(CB_E_HIP, "attention deviation launch: %s", hipGetErrorString(e));
    return CB_OK;
}

cb_status cb_topk_select(const float* dev, int32_t n, int32_t k, int32_t* idx_out, void* stream) {
    if (n < 0 || k < 0 || k > n) return fail(CB_E_INVALID, "need 0 <= k <= n (k=%d, n=%d)", k, n);
    if (n > 0 && (!dev || (k > 0 && !idx_out))) return fail(CB_E_INVALID, "NULL buffer");
    CB_HIP(launch_topk(dev, n, k, idx_out, as_stream(stream)));
    return CB_OK;
}

cb_status cb_gather_rows(const void* src, void* dst, const int32_t* idx, int32_t n_rows,
                         int64_t row_bytes, void* stream) {
    if (n_rows < 0 || row_bytes <= 0 || row_bytes % 4) return fail(CB_E_SHAPE, "bad row size");
    if (n_rows > 0 && (!src || !dst || !idx)) return fail(CB_E_INVALID, "NULL buffer");
    CB_HIP(launch_gather_rows(src, dst, idx, n_rows, row_bytes, as_stream(stream)));
    return CB_OK;
}

cb_status cb_scatter_rows(const void* src, void* dst, const int32_t* idx, int32_t n_rows,
                          int64_t row_bytes, void* stream) {
    if (n_rows < 0 || row_bytes <= 0 || row_bytes % 4) return fail(CB_E_SHAPE, "bad row size");
    if (n_rows > 0 && (!src || !dst || !idx)) return fail(CB_E_INVALID, "NULL buffer");
    CB_HIP(launch_scatter_rows(src, dst, idx, n_rows, row_bytes, as_stream(stream)));
    return CB_OK;
}

cb_status cb_rmsnorm(int32_t x_dtype, const void* x, int32_t y_dtype, const void* g, void* y,
                     int32_t rows, int32_t d, float eps, void* stream) {
    if ((x_dtype != CB_F32 && x_dtype != CB_BF16) || (y_dtype != CB_F32 && y_dtype != CB_BF16))
        return fail(CB_E_INVALID, "dtype");
    if (rows < 0 || d <= 0) return fail(CB_E_SHAPE, "bad sizes");
    if (rows > 0 && (!x || !g || !y)) return fail(CB_E_INVALID, "NULL buffer");
    CB_HIP(launch_rmsnorm(x_dtype, x, nullptr, y_dtype, g, y, nullptr, rows, d, eps,
                          as_stream(stream)));
    return CB_OK;
}

cb_status cb_gemm(int32_t dtype, const void* a, const void* b, float* c, int32_t m, int32_t n,
                  int32_t k, void* stream) {
    if (dtype != CB_F32 && dtype != CB_BF16) return fail(CB_E_INVALID, "dtype %d", dtype);
    if (m < 0 || n < 0 || k <= 0) return fail(CB_E_SHAPE, "bad sizes");
    const int kmul = dtype == CB_BF16 ? 64 : 32;
    if (k % kmul) return fail(CB_E_SHAPE, "k = %d must be a multiple of %d", k, kmul);
    if (m > 0 && n > 0 && (!a || !b || !c)) return fail(CB_E_INVALID, "NULL buffer");
    if (!aligned_to(a, 16) || !aligned_to(b, 16)) return fail(CB_E_SHAPE, "a/b not 16-byte aligned");
    GemmArgs g{};
    g.a = a; g.b0 = b; g.M = m; g.N = n; g.K = k; g.out0 = c;
    CB_HIP(launch_gemm(dtype, EPI_STORE_F32, g, as_stream(stream)));
    return CB_OK;
}

cb_status cb_attention(int32_t dtype, const void* q, const int32_t* q_pos, int32_t n_q,
                       const void* k, const void* v, int32_t n_kv, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, void* out, void* stream) {
    if (dtype != CB_F32 && dtype != CB_BF16) return fail(CB_E_INVALID, "dtype %d", dtype);
    if (n_q < 0 || n_kv <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads)
        return fail(CB_E_SHAPE, "bad sizes");
    if (head_dim != 64 && head_dim != 128) return fail(CB_E_UNSUPPORTED, "head_dim %d", head_dim);
    if (n_q > 0 && (!q || !q_pos || !k || !v || !out)) return fail(CB_E_INVALID, "NULL buffer");
    AttnArgs a{};
    a.q = q; a.q_pos = q_pos; a.k = k; a.v = v;
    a.n_q_heads = n_q_heads; a.n_kv_heads = n_kv_heads; a.head_dim = head_dim; a.out = out;
    const hipStream_t st = as_stream(stream);
    const AttnRange range{0, n_q, 0, n_kv};
    const size_t need = attention_workspace(dtype, &range, 1, n_q_heads, head_dim);
    void* ws = nullptr;
    if (need) {
        if (hipMallocAsync(&ws, need, st) != hipSuccess) {
            (void)hipGetLastError();
            return fail(CB_E_OOM, "attention workspace of %zu bytes", need);
        }
    }
    const hipError_t e = launch_attention(dtype, a, &range, 1, ws, need, st);
    if (ws) (void)hipFreeAsync(ws, st);
    if (e != hipSuccess) return fail(CB_E_HIP, "attention launch: %s", hipGetErrorString(e));
    return CB_OK;
}

}  // extern "C"
