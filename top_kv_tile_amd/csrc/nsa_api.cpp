// C ABI of the library: validation, the host-side selection plan, workspace
// layout and kernel launches. Declarations and contracts are in include/nsa.h.
//
// The plan follows selection_plan on the page
// "automatic/modules/attention/sparse/selector.py": it depends only on the
// geometry and the pin/drop masks, never on tensor data, so it is computed on
// the host (no device readback) and uploaded with the launches.
#include "../../include/nsa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <vector>

#include "nsa_internal.h"

namespace nsa {
// Stage timing (nsa_stage_timing_begin / _end): while it is on, the
// selection and gradient calls of this thread record an event on their
// stream at the start and after every stage launch. Off, a mark costs one
// thread-local test.
struct StageTiming {
    bool on = false;
    std::vector<const char*> names;
    std::vector<hipEvent_t> marks;
};
thread_local StageTiming t_stages;

hipError_t stage_mark(const char* name, hipStream_t stream) {
    StageTiming& t = t_stages;
    if (!t.on) return hipSuccess;
    hipEvent_t ev = nullptr;
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) return e;
    t.names.push_back(name);
    t.marks.push_back(ev);
    return hipEventRecord(ev, stream);
}
}  // namespace nsa

namespace {

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
    g_last_hip = (int)e;
    return NSA_ERR_HIP;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t numel(const nsa_tensor* t) { return (int64_t)t->B * t->H * t->S * t->D; }

int check_tensor(const nsa_tensor* t) {
    if (!t) return NSA_ERR_NULL_ARG;
    if (t->dtype != NSA_F32 && t->dtype != NSA_BF16) return NSA_ERR_BAD_DTYPE;
    if (t->B < 0 || t->H <= 0 || t->S < 0 || t->D <= 0) return NSA_ERR_BAD_SHAPE;
    if (!t->data && numel(t) > 0) return NSA_ERR_NULL_ARG;
    return NSA_OK;
}

struct Geo {
    int B, Hq, Hkv, Sq, Skv, D, NQ, NK, NKW, Hsel, group;
    int bf16;
    int64_t rows;
    int64_t q_off = 0;  // absolute key position of query token 0 (decoding); 0 otherwise
};

int check_spec(const nsa_spec* s) {
    if (!s) return NSA_ERR_NULL_ARG;
    if (s->block_q <= 0 || s->block_kv <= 0) return NSA_ERR_BAD_SPEC;
    // rejects NaN, infinities and negatives
    if (!std::isfinite(s->budget) || s->budget < 0.0f) return NSA_ERR_BAD_SPEC;
    if (s->score_chunk_bytes < 0) return NSA_ERR_BAD_SPEC;
    return NSA_OK;
}

int check_mask(const nsa_mask* m, const Geo& g) {
    if (!m) return NSA_OK;
    if (m->b_dim != 1 && m->b_dim != g.B) return NSA_ERR_BAD_SHAPE;
    if (m->h_dim != 1 && m->h_dim != g.Hsel) return NSA_ERR_BAD_SHAPE;
    if (m->nq != g.NQ || m->nk != g.NK) return NSA_ERR_BAD_SHAPE;
    if (!m->data && (int64_t)m->b_dim * m->h_dim * m->nq * m->nk > 0) return NSA_ERR_NULL_ARG;
    return NSA_OK;
}

int validate_select(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec, const nsa_mask* pins,
                    const nsa_mask* drops, Geo& g) {
    int st;
    if ((st = check_tensor(q)) != NSA_OK) return st;
    if ((st = check_tensor(k)) != NSA_OK) return st;
    if ((st = check_spec(spec)) != NSA_OK) return st;
    if (q->dtype != k->dtype) return NSA_ERR_BAD_DTYPE;
    if (q->B != k->B || q->D != k->D) return NSA_ERR_BAD_SHAPE;
    if (q->H % k->H != 0) return NSA_ERR_BAD_SHAPE;
    g.B = q->B;
    g.Hq = q->H;
    g.Hkv = k->H;
    g.Sq = q->S;
    g.Skv = k->S;
    g.D = q->D;
    g.NQ = (int)ceil_div(q->S, spec->block_q);
    g.NK = (int)ceil_div(k->S, spec->block_kv);
    g.NKW = (int)ceil_div(g.NK, 64);
    g.Hsel = spec->head_shared ? 1 : q->H;
    g.group = q->H / k->H;
    g.bf16 = q->dtype == NSA_BF16;
    g.rows = (int64_t)g.B * g.Hsel * g.NQ;
    if ((st = check_mask(pins, g)) != NSA_OK) return st;
    if ((st = check_mask(drops, g)) != NSA_OK) return st;
    if (g.D != 64 && g.D != 128 && g.D != 256) return NSA_ERR_UNSUPPORTED;
    if (g.NK > 4096) return NSA_ERR_UNSUPPORTED;
    return NSA_OK;
}

// Pack an int8 mask (nonzero = set) into 64-bit words per (b, h, i) row: bit
// (j % 64) of word j / 64.
void pack_mask(const nsa_mask* m, int NKW, std::vector<uint64_t>& out) {
    const int64_t nrows = (int64_t)m->b_dim * m->h_dim * m->nq;
    out.assign((size_t)(nrows * NKW), 0ull);
    for (int64_t r = 0; r < nrows; ++r) {
        const int8_t* src = m->data + r * m->nk;
        uint64_t* dst = out.data() + r * NKW;
        int j = 0;
        for (; j + 8 <= m->nk; j += 8) {
            uint64_t x;
            std::memcpy(&x, src + j, 8);
            // any nonzero byte -> bit 0 of that byte
            x |= x >> 4;
            x |= x >> 2;
            x |= x >> 1;
            x &= 0x0101010101010101ull;
            // gather bit 0 of each byte into the low 8 bits
            const uint64_t bits = (x * 0x0102040810204080ull) >> 56;
            dst[j >> 6] |= bits << (j & 63);
        }
        for (; j < m->nk; ++j)
            if (src[j]) dst[j >> 6] |= 1ull << (j & 63);
    }
}

struct Plan {
    Geo g;
    std::vector<int32_t> row_ptr;  // rows + 1
    std::vector<uint64_t> pin_words, drop_words;
    int pb = 1, ph = 1, db = 1, dh = 1;
    bool has_pins = false, has_drops = false;
    int64_t nnz = 0;
    bool dense = true;
};

// k_r = ceil(fl32(c_r) * fl32(budget)): an integer count times the budget,
// evaluated in float32 (the type torch promotes that product to).
// A product at or above c (a budget above 1) keeps every candidate, so it is
// clamped to c before the integer conversion.
inline int64_t keep_per_row(int64_t c, float budget) {
    volatile float prod = (float)c * budget;  // one IEEE fp32 rounding, no contraction
    const float kf = std::ceil((float)prod);
    return kf >= (float)c ? c : (int64_t)kf;
}

int build_plan(const Geo& g, const nsa_spec* spec, const nsa_mask* pins, const nsa_mask* drops, Plan& p,
               bool want_row_ptr) {
    p.g = g;
    p.has_pins = pins != nullptr;
    p.has_drops = drops != nullptr;
    if (pins) {
        pack_mask(pins, g.NKW, p.pin_words);
        p.pb = pins->b_dim;
        p.ph = pins->h_dim;
    }
    if (drops) {
        pack_mask(drops, g.NKW, p.drop_words);
        p.db = drops->b_dim;
        p.dh = drops->h_dim;
    }
    // Per distinct (pin slab, drop slab) pair: kept count of each query tile.
    std::vector<int64_t> slab_key;
    std::vector<std::vector<int32_t>> slab_counts;
    std::vector<uint64_t> diag(g.NKW);
    auto counts_for = [&](int ps, int ds) -> const std::vector<int32_t>& {
        const int64_t key = (int64_t)ps * 1000003 + ds;
        for (size_t x = 0; x < slab_key.size(); ++x)
            if (slab_key[x] == key) return slab_counts[x];
        std::vector<int32_t> cnt(g.NQ);
        for (int i = 0; i < g.NQ; ++i) {
            // diagonal: kv tiles j with o + i*bq < (j+1)*bkv and j*bkv < o + (i+1)*bq (o = q_off)
            const int64_t lo = (g.q_off + (int64_t)i * spec->block_q) / spec->block_kv;
            const int64_t hi = std::min<int64_t>(
                ceil_div(g.q_off + (int64_t)(i + 1) * spec->block_q, spec->block_kv) - 1, g.NK - 1);
            std::fill(diag.begin(), diag.end(), 0ull);
            for (int64_t j = lo; j <= hi; ++j) diag[j >> 6] |= 1ull << (j & 63);
            const uint64_t* pw = pins ? p.pin_words.data() + ((int64_t)ps * g.NQ + i) * g.NKW : nullptr;
            const uint64_t* dw = drops ? p.drop_words.data() + ((int64_t)ds * g.NQ + i) * g.NKW : nullptr;
            int64_t c = 0, mk = 0;
            for (int w = 0; w < g.NKW; ++w) {
                const int rem = g.NK - 64 * w;
                const uint64_t valid = rem >= 64 ? ~0ull : ((1ull << rem) - 1);
                const uint64_t must = (diag[w] | (pw ? pw[w] : 0ull)) & valid;
                const uint64_t forb = (dw ? dw[w] : 0ull) & valid;
                c += __builtin_popcountll(valid & ~must & ~forb);
                mk += __builtin_popcountll(must & ~forb);
            }
            const int64_t kr = keep_per_row(c, spec->budget);
            if (kr < c) p.dense = false;
            cnt[i] = (int32_t)(mk + std::min(kr, c));
        }
        slab_key.push_back(key);
        slab_counts.push_back(std::move(cnt));
        return slab_counts.back();
    };
    if (want_row_ptr) p.row_ptr.resize((size_t)g.rows + 1);
    int64_t acc = 0;
    int64_t r = 0;
    if (want_row_ptr) p.row_ptr[0] = 0;
    for (int b = 0; b < g.B; ++b)
        for (int h = 0; h < g.Hsel; ++h) {
            const int ps = (b % p.pb) * p.ph + (h % p.ph);
            const int ds = (b % p.db) * p.dh + (h % p.dh);
            const std::vector<int32_t>& cnt = counts_for(ps, ds);
            for (int i = 0; i < g.NQ; ++i) {
                acc += cnt[i];
                ++r;
                if (acc > INT32_MAX) return NSA_ERR_UNSUPPORTED;
                if (want_row_ptr) p.row_ptr[r] = (int32_t)acc;
            }
        }
    p.nnz = acc;
    return NSA_OK;
}

struct WsLayout {
    size_t pq = 0, pk = 0, mq = 0, mk = 0, scores = 0, rowp = 0, pinw = 0, dropw = 0, total = 0;
    int chunk = 1;
};

WsLayout ws_layout(const Geo& g, const nsa_spec* spec, bool has_pins, int pin_slabs, bool has_drops,
                   int drop_slabs, bool external_k = false) {
    WsLayout w;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    w.pq = take((size_t)g.B * g.Hq * g.NQ * g.D * 4);
    w.pk = external_k ? 0 : take((size_t)g.B * g.Hkv * g.NK * g.D * 4);
    if (spec->head_shared) {
        w.mq = take((size_t)g.B * g.NQ * g.D * 4);
        w.mk = take((size_t)g.B * g.NK * g.D * 4);
    }
    // Head chunk of the score buffer, as score_blocks sizes it: as many heads
    // as fit in score_chunk_bytes of NQ x NK fp32 scores, at least one.
    const int64_t per_head = std::max<int64_t>((int64_t)g.NQ * g.NK * 4, 1);
    w.chunk = (int)std::max<int64_t>(1, std::min<int64_t>(g.Hsel, spec->score_chunk_bytes / per_head));
    w.scores = take((size_t)g.B * w.chunk * g.NQ * g.NK * 4);
    // Row offsets, then the mask words: uploaded together with one copy (the
    // top-k kernels write the caller's row_ptr from here).
    w.rowp = take((size_t)(g.rows + 1) * 4);
    if (has_pins) w.pinw = take((size_t)pin_slabs * g.NQ * g.NKW * 8);
    if (has_drops) w.dropw = take((size_t)drop_slabs * g.NQ * g.NKW * 8);
    w.total = off;
    return w;
}

// Pinned host staging for the plan uploads, so that hipMemcpyAsync stays
// asynchronous. A small ring per device; a slot is reused only after the copy
// that last read it has completed.
struct StagingSlot {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t done = nullptr;
    bool pending = false;
};
struct Staging {
    static constexpr int kSlots = 8;
    std::mutex mu;
    StagingSlot slot[64][kSlots];
    int next[64] = {};
};
Staging& staging() {
    static Staging* s = new Staging();  // lives until process exit
    return *s;
}

// Copies the host ranges (src[x], bytes[x]) to dst[x] on `stream` through one
// pinned staging slot.
hipError_t upload(int n, void* const* dst, const void* const* src, const size_t* bytes, hipStream_t stream) {
    size_t total = 0;
    for (int x = 0; x < n; ++x) total += align256(bytes[x]);
    if (total == 0) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    Staging& st = staging();
    std::lock_guard<std::mutex> lock(st.mu);
    StagingSlot& s = st.slot[dev][st.next[dev]];
    st.next[dev] = (st.next[dev] + 1) % Staging::kSlots;
    if (!s.done) {
        if ((e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming)) != hipSuccess) return e;
    }
    if (s.pending) {
        if ((e = hipEventSynchronize(s.done)) != hipSuccess) return e;
        s.pending = false;
    }
    if (s.cap < total) {
        if (s.host) (void)hipHostFree(s.host);
        s.host = nullptr;
        s.cap = 0;
        const size_t cap = std::max<size_t>(total, 1 << 20);
        if ((e = hipHostMalloc(&s.host, cap, hipHostMallocDefault)) != hipSuccess) return e;
        s.cap = cap;
    }
    // Buffers are staged 256-byte aligned; consecutive ones whose device
    // destinations lie at the same distances go up with one copy.
    size_t off = 0, run_off = 0, run_end = 0;
    char* run_dst = nullptr;
    for (int x = 0; x < n; ++x) {
        if (bytes[x] == 0) continue;
        std::memcpy((char*)s.host + off, src[x], bytes[x]);
        if (run_dst && (char*)dst[x] == run_dst + (off - run_off)) {
            run_end = off + bytes[x];
        } else {
            if (run_dst && (e = hipMemcpyAsync(run_dst, (char*)s.host + run_off, run_end - run_off,
                                               hipMemcpyHostToDevice, stream)) != hipSuccess)
                return e;
            run_dst = (char*)dst[x];
            run_off = off;
            run_end = off + bytes[x];
        }
        off += align256(bytes[x]);
    }
    if (run_dst && (e = hipMemcpyAsync(run_dst, (char*)s.host + run_off, run_end - run_off, hipMemcpyHostToDevice,
                                       stream)) != hipSuccess)
        return e;
    if ((e = hipEventRecord(s.done, stream)) != hipSuccess) return e;
    s.pending = true;
    return hipSuccess;
}

// Enqueues pooling (+ head means) of q and k into the workspace.
int run_pool(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec, const Geo& g, const WsLayout& w,
             char* ws, hipStream_t stream, const float** qh, const float** kh, int* Hk) {
    hipError_t e;
    float* pq = (float*)(ws + w.pq);
    float* pk = (float*)(ws + w.pk);
    if ((e = nsa::stage_mark("start", stream)) != hipSuccess) return hip_fail(e);
    if ((e = nsa::launch_pool(q->data, g.bf16, (int64_t)g.B * g.Hq, g.Sq, g.D, spec->block_q, pq, stream)) !=
        hipSuccess)
        return hip_fail(e);
    if ((e = nsa::stage_mark("pool_q", stream)) != hipSuccess) return hip_fail(e);
    if ((e = nsa::launch_pool(k->data, g.bf16, (int64_t)g.B * g.Hkv, g.Skv, g.D, spec->block_kv, pk,
                              stream)) != hipSuccess)
        return hip_fail(e);
    if ((e = nsa::stage_mark("pool_k", stream)) != hipSuccess) return hip_fail(e);
    if (spec->head_shared) {
        float* mq = (float*)(ws + w.mq);
        float* mk = (float*)(ws + w.mk);
        if ((e = nsa::launch_head_mean(pq, g.B, g.Hq, g.NQ, g.D, mq, stream)) != hipSuccess) return hip_fail(e);
        if ((e = nsa::launch_head_mean(pk, g.B, g.Hkv, g.NK, g.D, mk, stream)) != hipSuccess) return hip_fail(e);
        if ((e = nsa::stage_mark("head_mean", stream)) != hipSuccess) return hip_fail(e);
        *qh = mq;
        *kh = mk;
        *Hk = 1;
    } else {
        *qh = pq;
        *kh = pk;
        *Hk = g.Hkv;
    }
    return NSA_OK;
}


WsLayout plan_layout(const Plan& p, const nsa_spec* spec) {
    return ws_layout(p.g, spec, p.has_pins, p.pb * p.ph, p.has_drops, p.db * p.dh);
}

void fill_sizes(const Plan& p, const nsa_spec* spec, nsa_sizes* out, int32_t* row_ptr_host) {
    const WsLayout w = plan_layout(p, spec);
    out->NQ = p.g.NQ;
    out->NK = p.g.NK;
    out->sel_heads = p.g.Hsel;
    out->dense = (p.dense && !spec->force) ? 1 : 0;
    out->rows = p.g.rows;
    out->nnz = p.nnz;
    out->workspace_bytes = (int64_t)w.total;
    if (row_ptr_host) std::memcpy(row_ptr_host, p.row_ptr.data(), p.row_ptr.size() * sizeof(int32_t));
}

int score_and_topk(const Plan& p, const nsa_spec* spec, const void* qh, const float* kh, int Hk, int NKs,
                   const WsLayout& w, char* ws, nsa_selection* out, hipStream_t stream, const uint64_t* pin_words,
                   const uint64_t* drop_words, const int32_t* row_src, int32_t row_step = 0, int q_rows = 0,
                   bool inline_masks = false);

// A plan's row offsets and mask words already in device memory (the image
// nsa_plan_upload writes into a caller buffer).
struct PlanDevice {
    int32_t* row_ptr = nullptr;
    uint64_t* pin_words = nullptr;
    uint64_t* drop_words = nullptr;
};

// Enqueues the selection of a built plan (row_ptr present) for tensors q, k
// whose geometry the plan was built from; pd: the plan's device image, or null
// (then it is uploaded into the workspace).
int run_select(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec, const Plan& p, nsa_selection* out,
               void* workspace, size_t workspace_bytes, hipStream_t stream, const PlanDevice* pd = nullptr) {
    const Geo& g = p.g;
    if (p.dense && !spec->force) return NSA_DENSE;
    if (g.rows > 0 && (!out->keep || !out->row_ptr)) return NSA_ERR_NULL_ARG;
    if (!out->row_ptr) return NSA_ERR_NULL_ARG;
    if (p.nnz > 0 && !out->col_idx) return NSA_ERR_NULL_ARG;
    if (out->col_capacity < p.nnz) return NSA_ERR_CAPACITY;
    const WsLayout w = plan_layout(p, spec);
    if (workspace_bytes < w.total) return NSA_ERR_WORKSPACE;
    if (w.total > 0 && (!workspace || ((uintptr_t)workspace & 255))) return NSA_ERR_WORKSPACE;

    out->nnz = p.nnz;
    out->B = g.B;
    out->H = g.Hsel;
    out->NQ = g.NQ;
    out->NK = g.NK;
    out->block_q = spec->block_q;
    out->block_kv = spec->block_kv;
    out->seq_q = g.Sq;
    out->seq_kv = g.Skv;
    out->budget = spec->budget;

    char* ws = (char*)workspace;
    const uint64_t* pin_words = p.has_pins ? (const uint64_t*)(ws + w.pinw) : nullptr;
    const uint64_t* drop_words = p.has_drops ? (const uint64_t*)(ws + w.dropw) : nullptr;
    if (g.rows == 0 || g.NK == 0) {  // no top-k launch: the row offsets go straight to the caller
        void* dst[1] = {out->row_ptr};
        const void* src[1] = {p.row_ptr.data()};
        size_t bytes[1] = {p.row_ptr.size() * sizeof(int32_t)};
        const hipError_t e = upload(1, dst, src, bytes, stream);
        return e == hipSuccess ? NSA_OK : hip_fail(e);
    }
    const int32_t* row_src = (const int32_t*)(ws + w.rowp);
    if (pd) {  // the plan is on the device already: nothing is copied
        row_src = pd->row_ptr;
        pin_words = pd->pin_words;
        drop_words = pd->drop_words;
    } else {  // row offsets and mask words, one copy into the workspace
        void* dst[3] = {ws + w.rowp, ws + w.pinw, ws + w.dropw};
        const void* src[3] = {p.row_ptr.data(), p.pin_words.data(), p.drop_words.data()};
        size_t bytes[3] = {p.row_ptr.size() * sizeof(int32_t), p.has_pins ? p.pin_words.size() * 8 : 0,
                           p.has_drops ? p.drop_words.size() * 8 : 0};
        hipError_t e = upload(3, dst, src, bytes, stream);
        if (e != hipSuccess) return hip_fail(e);
    }

    const float* qh;
    const float* kh;
    int Hk;
    int st;
    if ((st = run_pool(q, k, spec, g, w, ws, stream, &qh, &kh, &Hk)) != NSA_OK) return st;
    return score_and_topk(p, spec, qh, kh, Hk, g.NK, w, ws, out, stream, pin_words, drop_words, row_src);
}

// Scores chunk by chunk of selection heads, each followed by its top-k and CSR.
// pin_words / drop_words: the plan's bit-packed masks on the device (or null).
int score_and_topk(const Plan& p, const nsa_spec* spec, const void* qh, const float* kh, int Hk, int NKs,
                   const WsLayout& w, char* ws, nsa_selection* out, hipStream_t stream, const uint64_t* pin_words,
                   const uint64_t* drop_words, const int32_t* row_src, int32_t row_step, int q_rows,
                   bool inline_masks) {
    const Geo& g = p.g;
    float* scores = (float*)(ws + w.scores);
    for (int h0 = 0; h0 < g.Hsel; h0 += w.chunk) {
        const int nh = std::min(w.chunk, g.Hsel - h0);
        hipError_t e = nsa::launch_scores(qh, kh, g.B, g.Hsel, Hk, g.group, h0, nh, g.NQ, g.NK, g.D, scores,
                                          stream, NKs, q_rows);
        if (e != hipSuccess) return hip_fail(e);
        if ((e = nsa::stage_mark("scores", stream)) != hipSuccess) return hip_fail(e);
        nsa::TopkArgs ta;
        ta.scores = scores;
        ta.B = g.B;
        ta.Hsel = g.Hsel;
        ta.h0 = h0;
        ta.nh = nh;
        ta.NQ = g.NQ;
        ta.NK = g.NK;
        ta.NKW = g.NKW;
        ta.block_q = spec->block_q;
        ta.block_kv = spec->block_kv;
        ta.q_off = g.q_off;
        ta.budget = spec->budget;
        ta.pin_words = pin_words;
        ta.pb = p.pb;
        ta.ph = p.ph;
        ta.drop_words = drop_words;
        ta.db = p.db;
        ta.dh = p.dh;
        ta.row_src = row_src;
        ta.row_step = row_step;
        if (inline_masks) {  // the plan's mask words ride in the launch arguments
            int n = 0;
            if (p.has_pins) {
                std::memcpy(ta.words, p.pin_words.data(), p.pin_words.size() * 8);
                ta.pin_at = 0;
                ta.pin_words = nullptr;
                n = (int)p.pin_words.size();
            }
            if (p.has_drops) {
                std::memcpy(ta.words + n, p.drop_words.data(), p.drop_words.size() * 8);
                ta.drop_at = n;
                ta.drop_words = nullptr;
            }
        }
        ta.row_ptr = out->row_ptr;
        ta.keep = out->keep;
        ta.col_idx = out->col_idx;
        if ((e = nsa::launch_topk(ta, stream)) != hipSuccess) return hip_fail(e);
        if ((e = nsa::stage_mark("topk", stream)) != hipSuccess) return hip_fail(e);
    }
    return NSA_OK;
}

// ---- decoding -------------------------------------------------------------------

// Geometry of a decode-time selection: n query tokens q (B, Hq, n, D) at
// absolute positions q_pos0 .. q_pos0 + n - 1 against the first `length`
// cached keys, whose pooled means are in pooled_k (B, Hkv, capacity, D) fp32.
int validate_decode_select(const nsa_tensor* q, const nsa_tensor* pooled_k, int32_t length, int32_t q_pos0,
                           const nsa_spec* spec, const nsa_mask* pins, const nsa_mask* drops, Geo& g) {
    int st;
    if ((st = check_tensor(q)) != NSA_OK) return st;
    if ((st = check_tensor(pooled_k)) != NSA_OK) return st;
    if ((st = check_spec(spec)) != NSA_OK) return st;
    if (pooled_k->dtype != NSA_F32) return NSA_ERR_BAD_DTYPE;
    if (q->B != pooled_k->B || q->D != pooled_k->D || q->H % pooled_k->H != 0) return NSA_ERR_BAD_SHAPE;
    if (length < 0 || q_pos0 < 0 || (int64_t)q_pos0 + q->S > length) return NSA_ERR_BAD_SHAPE;
    g.B = q->B;
    g.Hq = q->H;
    g.Hkv = pooled_k->H;
    g.Sq = q->S;
    g.Skv = length;
    g.D = q->D;
    g.NQ = (int)ceil_div(q->S, spec->block_q);
    g.NK = (int)ceil_div(length, spec->block_kv);
    g.NKW = (int)ceil_div(g.NK, 64);
    g.Hsel = spec->head_shared ? 1 : q->H;
    g.group = q->H / pooled_k->H;
    g.bf16 = q->dtype == NSA_BF16;
    g.rows = (int64_t)g.B * g.Hsel * g.NQ;
    g.q_off = q_pos0;
    if (g.NK > pooled_k->S) return NSA_ERR_BAD_SHAPE;  // the cache of pooled keys is too short
    if ((st = check_mask(pins, g)) != NSA_OK) return st;
    if ((st = check_mask(drops, g)) != NSA_OK) return st;
    if (g.D != 64 && g.D != 128 && g.D != 256) return NSA_ERR_UNSUPPORTED;
    if (g.NK > 4096) return NSA_ERR_UNSUPPORTED;
    return NSA_OK;
}

WsLayout decode_layout(const Plan& p, const nsa_spec* spec) {
    return ws_layout(p.g, spec, p.has_pins, p.pb * p.ph, p.has_drops, p.db * p.dh, true);
}

// Launch geometry of a decode attention call (everything but out / lse / partials).
// Rows whose tiles are few and many can be split over several workgroups (MFMA
// paths); the partials are merged afterwards. The decode kernel (32-row tiles)
// is used where it applies.
int decode_attn_config(const nsa_tensor* q, const nsa_tensor* k_cache, const nsa_tensor* v_cache,
                       const nsa_tensor* out, int32_t length, int32_t q_pos0, const nsa_selection* sel,
                       nsa::AttnArgs& a) {
    int st;
    if ((st = check_tensor(q)) != NSA_OK) return st;
    if ((st = check_tensor(k_cache)) != NSA_OK) return st;
    if ((st = check_tensor(v_cache)) != NSA_OK) return st;
    if ((st = check_tensor(out)) != NSA_OK) return st;
    if (q->dtype != k_cache->dtype || q->dtype != v_cache->dtype || q->dtype != out->dtype)
        return NSA_ERR_BAD_DTYPE;
    if (q->B != k_cache->B || k_cache->B != v_cache->B || k_cache->H != v_cache->H || k_cache->S != v_cache->S)
        return NSA_ERR_BAD_SHAPE;
    if (q->D != k_cache->D || q->D != v_cache->D || q->H % k_cache->H != 0) return NSA_ERR_BAD_SHAPE;
    if (out->B != q->B || out->H != q->H || out->S != q->S || out->D != q->D) return NSA_ERR_BAD_SHAPE;
    if (length < 0 || length > k_cache->S || q_pos0 < 0 || (int64_t)q_pos0 + q->S > length)
        return NSA_ERR_BAD_SHAPE;
    if (q->D != 64 && q->D != 128) return NSA_ERR_UNSUPPORTED;
    a.q = q->data;
    a.k = k_cache->data;
    a.v = v_cache->data;
    a.out = nullptr;
    a.lse = nullptr;
    a.B = q->B;
    a.Hq = q->H;
    a.Hkv = k_cache->H;
    a.S = q->S;
    a.Skv = length;
    a.kv_rows = k_cache->S;
    a.q_off = q_pos0;
    a.D = q->D;
    a.causal = 1;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)q->D));
    a.nsplit = 1;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    int64_t tiles_per_row;
    if (sel) {
        if (!sel->row_ptr) return NSA_ERR_NULL_ARG;
        if (sel->nnz > 0 && !sel->col_idx) return NSA_ERR_NULL_ARG;
        if (sel->block_q <= 0 || sel->block_kv <= 0) return NSA_ERR_BAD_SPEC;
        if ((sel->B != q->B && sel->B != 1) || (sel->H != 1 && sel->H != q->H)) return NSA_ERR_BAD_SHAPE;
        if (sel->seq_q != q->S || sel->seq_kv != length) return NSA_ERR_BAD_SHAPE;
        if (sel->NQ != ceil_div(q->S, sel->block_q) || sel->NK != ceil_div(length, sel->block_kv))
            return NSA_ERR_BAD_SHAPE;
        a.row_ptr = sel->row_ptr;
        a.col_idx = sel->col_idx;
        a.Hsel = sel->H;
        a.Bsel = sel->B;
        a.block_q = sel->block_q;
        a.block_kv = sel->block_kv;
        const int64_t rows = std::max<int64_t>((int64_t)sel->B * sel->H * sel->NQ, 1);
        tiles_per_row = ceil_div(std::max<int64_t>(sel->nnz, 0), rows);
    } else {  // every tile of the first `length` keys
        a.row_ptr = nullptr;
        a.col_idx = nullptr;
        a.Hsel = q->H;
        a.Bsel = q->B;
        a.block_q = 32;  // the decode kernel's row tile
        a.block_kv = 64;
        tiles_per_row = ceil_div(length, 64);
    }
    a.NQ = (int)ceil_div(q->S, a.block_q);
    a.NK = (int)ceil_div(length, a.block_kv);
    // One selection row shared by the heads (or none): the query heads of a GQA
    // group are packed into the rows of one workgroup, so each kept K/V tile is
    // read once per kv head instead of once per query head.
    const int G = q->H / k_cache->H;
    if (G > 1 && a.block_kv == 64 && (!sel || (sel->H == 1 && sel->NQ == 1))) {
        nsa::AttnArgs p = a;
        const int64_t rows = (int64_t)G * q->S;
        p.qpack = q->S;
        p.Hq = k_cache->H;
        p.Hsel = 1;
        p.S = (int)rows;
        p.block_q = 32;  // packed rows follow no selection tile: the decode kernel's 32-row tile
        p.NQ = (int)ceil_div(rows, p.block_q);
        if (rows < INT32_MAX && nsa::attn_mfma_supported(p, q->dtype == NSA_BF16)) a = p;
    }
    if (nsa::attn_mfma_supported(a, q->dtype == NSA_BF16)) {
        const int64_t work = std::max<int64_t>((int64_t)a.B * a.Hq * a.NQ, 1);
        // about two rounds of workgroups (five per CU for the decode kernel), at
        // least 8 tiles per split and at most 64 splits (measured at 128k)
        const int64_t want = ceil_div(nsa::attn_decode_supported(a, q->dtype == NSA_BF16) ? 2560 : 2048, work);
        const int64_t most = std::max<int64_t>(1, tiles_per_row / 8);
        a.nsplit = (int)std::max<int64_t>(1, std::min<int64_t>({want, most, 64}));
    }
    return NSA_OK;
}

size_t decode_attn_workspace(const nsa::AttnArgs& a) {
    if (a.nsplit <= 1) return 0;
    const size_t rows = (size_t)a.B * a.Hq * a.S * a.nsplit;
    return align256(rows * a.D * 4) + align256(rows * 2 * 4);
}

// ---- radial band (radial_blocks of the selection page) -------------------------

// Tiles whose query-range and kv-range centres are at most a bandwidth apart,
// the bandwidth bisected 40 times over [0, max(seq_q, seq_kv)] until the kept
// fraction reaches `density`. Arithmetic as the page's: centre distances in
// float32, the trial width rounded to float32 for the comparison, the kept
// fraction a float32 mean compared with the float64 density. The counts come
// from the sorted distances instead of a pass per trial (same result).
struct Band {
    int NQ = 0, NK = 0;
    std::vector<int32_t> row_ptr;  // NQ + 1
    std::vector<int32_t> col_idx;
    std::vector<int8_t> keep;      // NQ x NK
};
int build_band(int seq_q, int seq_kv, double density, int bq, int bkv, Band& band) {
    band.NQ = (int)ceil_div(seq_q, bq);
    band.NK = (int)ceil_div(seq_kv, bkv);
    const int64_t n = (int64_t)band.NQ * band.NK;
    if (n >= ((int64_t)1 << 31)) return NSA_ERR_UNSUPPORTED;
    std::vector<float> dist((size_t)n);
    for (int i = 0; i < band.NQ; ++i) {
        const float qc = ((float)i + 0.5f) * (float)bq;
        for (int j = 0; j < band.NK; ++j) {
            const float kc = ((float)j + 0.5f) * (float)bkv;
            dist[(size_t)i * band.NK + j] = std::fabs(qc - kc);
        }
    }
    std::vector<float> sorted(dist);
    std::sort(sorted.begin(), sorted.end());
    auto fraction = [&](double width) -> double {
        const float w32 = (float)width;
        const int64_t cnt = std::upper_bound(sorted.begin(), sorted.end(), w32) - sorted.begin();
        volatile float frac = (float)cnt / (float)std::max<int64_t>(n, 1);  // one fp32 rounding
        return (double)frac;
    };
    double low = 0.0, high = (double)std::max(seq_q, seq_kv);
    for (int it = 0; it < 40; ++it) {
        const double mid = (low + high) / 2;
        if (fraction(mid) < density) low = mid;
        else high = mid;
    }
    const float h32 = (float)high;
    band.keep.assign((size_t)n, 0);
    band.row_ptr.assign((size_t)band.NQ + 1, 0);
    band.col_idx.clear();
    for (int i = 0; i < band.NQ; ++i) {
        for (int j = 0; j < band.NK; ++j)
            if (dist[(size_t)i * band.NK + j] <= h32) {
                band.keep[(size_t)i * band.NK + j] = 1;
                band.col_idx.push_back(j);
            }
        band.row_ptr[i + 1] = (int32_t)band.col_idx.size();
    }
    return NSA_OK;
}

// ---- curve orders (token reordering) --------------------------------------------

// Morton key: bit b of axis a (a = 0 the fastest, i.e. last, axis) goes to bit
// b * n + a. Hilbert key: J. Skilling's transpose method ("Programming the
// Hilbert curve", 2004) on the enclosing 2^p cube, read level by level with
// the slowest axis giving the high bit of each level.
uint64_t morton_key(const int64_t* c, int n, int p) {
    uint64_t key = 0;
    for (int b = 0; b < p; ++b)
        for (int a = 0; a < n; ++a) key |= (uint64_t)((c[n - 1 - a] >> b) & 1) << (b * n + a);
    return key;
}
uint64_t hilbert_key(const int64_t* c, int n, int p) {
    int64_t x[8];
    for (int i = 0; i < n; ++i) x[i] = c[i];
    const int64_t top = (int64_t)1 << (p - 1);
    for (int64_t q = top; q > 1; q >>= 1) {
        const int64_t low = q - 1;
        for (int i = 0; i < n; ++i) {
            if (x[i] & q) {
                x[0] ^= low;
            } else {
                const int64_t t = (x[0] ^ x[i]) & low;
                x[0] ^= t;
                x[i] ^= t;
            }
        }
    }
    for (int i = 1; i < n; ++i) x[i] ^= x[i - 1];
    int64_t t = 0;
    for (int64_t q = top; q > 1; q >>= 1)
        if (x[n - 1] & q) t ^= q - 1;
    for (int i = 0; i < n; ++i) x[i] ^= t;
    uint64_t key = 0;
    for (int b = p - 1; b >= 0; --b)
        for (int i = 0; i < n; ++i) key = (key << 1) | (uint64_t)((x[i] >> b) & 1);
    return key;
}

}  // namespace

// Opaque host-side selection plan: the geometry, the packed pin / drop masks
// and the row offsets, built once and reused by nsa_select_planned. It holds
// host memory only; its device image lives in a buffer of the caller.
struct nsa_plan {
    nsa_spec spec;
    nsa_tensor qshape, kshape;  // shapes and dtype only
    Plan p;
};

namespace {


// Selection geometry shared by the forward and the gradients; fills the CSR
// pointers, selection heads and block sizes of a launch (dense when sel is null).
int attn_selection(const nsa_tensor* q, const nsa_tensor* k, const nsa_selection* sel, int& Hsel, int& bq,
                   int& bkv) {
    if (!sel) {
        Hsel = q->H;
        bq = 128;
        bkv = 64;
        return NSA_OK;
    }
    if (!sel->row_ptr) return NSA_ERR_NULL_ARG;
    if (sel->nnz > 0 && !sel->col_idx) return NSA_ERR_NULL_ARG;
    if (sel->nnz < 0 || sel->nnz >= ((int64_t)1 << 31)) return NSA_ERR_BAD_SHAPE;
    if (sel->block_q <= 0 || sel->block_kv <= 0) return NSA_ERR_BAD_SPEC;
    if ((sel->B != q->B && sel->B != 1) || (sel->H != 1 && sel->H != q->H)) return NSA_ERR_BAD_SHAPE;
    if (sel->seq_q != q->S || sel->seq_kv != k->S) return NSA_ERR_BAD_SHAPE;
    if (sel->NQ != ceil_div(q->S, sel->block_q) || sel->NK != ceil_div(k->S, sel->block_kv))
        return NSA_ERR_BAD_SHAPE;
    Hsel = sel->H;
    bq = sel->block_q;
    bkv = sel->block_kv;
    return NSA_OK;
}

// Gradient workspace: Delta (B*Hq*S fp32), then for a sparse selection the
// per-column counts (B*H'*NK), col_ptr (B*H'*NK + 1) and row_idx (nnz) int32.
struct BwdLayout {
    size_t delta = 0, counts = 0, col_ptr = 0, sums = 0, row_idx = 0, total = 0;
};
BwdLayout bwd_layout(const nsa_tensor* q, const nsa_selection* sel) {
    BwdLayout w;
    size_t off = 0;
    w.delta = off;
    off += align256((size_t)numel(q) / (size_t)std::max(1, q->D) * sizeof(float));
    if (sel) {
        const size_t cols = (size_t)sel->B * sel->H * sel->NK;
        w.counts = off;  // per column and quarter of the query tiles
        off += align256(cols * 4 * sizeof(int32_t));
        w.col_ptr = off;
        off += align256((cols + 1) * sizeof(int32_t));
        w.sums = off;  // per block of 2048 columns, plus the total
        off += align256((ceil_div((int64_t)cols, 2048) + 1) * sizeof(int32_t));
        w.row_idx = off;
        off += align256((size_t)std::max<int64_t>(sel->nnz, 0) * sizeof(int32_t));
    }
    w.total = off;
    return w;
}

int validate_bwd(const nsa_tensor* q, const nsa_tensor* k, const nsa_tensor* v, const nsa_tensor* out,
                 const float* lse, const nsa_tensor* dout, const nsa_selection* sel, int causal,
                 const nsa_tensor* dq, const nsa_tensor* dk, const nsa_tensor* dv) {
    const nsa_tensor* all[8] = {q, k, v, out, dout, dq, dk, dv};
    for (const nsa_tensor* t : all) {
        const int st = check_tensor(t);
        if (st != NSA_OK) return st;
    }
    for (const nsa_tensor* t : all)
        if (t->dtype != q->dtype) return NSA_ERR_BAD_DTYPE;
    auto same = [](const nsa_tensor* x, const nsa_tensor* y) {
        return x->B == y->B && x->H == y->H && x->S == y->S && x->D == y->D;
    };
    if (!same(out, q) || !same(dout, q) || !same(dq, q)) return NSA_ERR_BAD_SHAPE;
    if (!same(v, k) || !same(dk, k) || !same(dv, k)) return NSA_ERR_BAD_SHAPE;
    if (q->B != k->B || q->D != k->D || q->H % k->H != 0) return NSA_ERR_BAD_SHAPE;
    if (numel(q) > 0 && !lse) return NSA_ERR_NULL_ARG;
    if (causal && q->S != k->S) return NSA_ERR_UNSUPPORTED;
    if (q->D != 64 && q->D != 128) return NSA_ERR_UNSUPPORTED;
    if (q->S != k->S) return NSA_ERR_UNSUPPORTED;
    int Hsel, bq, bkv;
    const int st = attn_selection(q, k, sel, Hsel, bq, bkv);
    if (st != NSA_OK) return st;
    if (sel && (int64_t)sel->B * sel->H * sel->NQ * sel->NK > 0 && !sel->keep) return NSA_ERR_NULL_ARG;
    return NSA_OK;
}

// ---- plan cache of nsa_select / nsa_select_sizes ---------------------------
//
// The selection page caches its plan (must / forbidden / candidates / keep
// counts) under a caller key, the tile counts, the block sizes, the budget and
// the device (selector.py, selection_plan). The pins and drops are not part of
// that key, so a plan built for one mask set is returned for another under the
// same caller key. Here the key is the whole request: the q and k shapes and
// dtypes, every spec field, and the shape and bytes of both masks (a 64-bit
// hash rejects quickly, a byte comparison confirms). Entries hold host plans
// only, no device memory, so evicting one (least recently used) never waits
// for device work; an entry in use by a call stays alive until that call ends.
struct PlanCacheEntry {
    nsa_tensor q, k;  // data pointers cleared
    nsa_spec spec;
    int32_t pdims[4], ddims[4];  // all -1 when the mask is absent
    uint64_t phash = 0, dhash = 0;
    std::vector<int8_t> pins, drops;  // copies of the mask bytes
    std::shared_ptr<const Plan> plan;
    uint64_t stamp = 0;
};
// Requests whose masks hold more bytes than this are built per call and not
// cached (each entry keeps a copy of its masks).
constexpr size_t kMaxCachedMaskBytes = (size_t)64 << 20;
struct PlanCache {
    std::mutex mu;
    std::vector<PlanCacheEntry> entries;
    size_t capacity = 8;
    uint64_t clock = 0;
    int64_t hits = 0, misses = 0;
};
PlanCache& plan_cache() {
    static PlanCache c;
    return c;
}

size_t mask_bytes(const nsa_mask* m) {
    return m ? (size_t)m->b_dim * m->h_dim * m->nq * m->nk : 0;
}
// Four independent multiply-xor lanes over 8-byte words (a fast reject, not a
// proof of equality).
uint64_t mask_hash(const nsa_mask* m) {
    if (!m) return 0;
    const size_t n = mask_bytes(m);
    const unsigned char* p = (const unsigned char*)m->data;
    const uint64_t mul = 0xff51afd7ed558ccdull;
    uint64_t h[4] = {0x9E3779B97F4A7C15ull ^ n, 0xC2B2AE3D27D4EB4Full, 0x165667B19E3779F9ull, 0x27D4EB2F165667C5ull};
    size_t i = 0;
    for (; i + 32 <= n; i += 32)
        for (int l = 0; l < 4; ++l) {
            uint64_t w;
            std::memcpy(&w, p + i + 8 * l, 8);
            h[l] = (h[l] ^ w) * mul;
            h[l] ^= h[l] >> 29;
        }
    uint64_t r = h[0] ^ (h[1] * 3) ^ (h[2] * 5) ^ (h[3] * 7);
    for (; i < n; ++i) {
        r = (r ^ p[i]) * mul;
        r ^= r >> 29;
    }
    return r;
}
void mask_dims(const nsa_mask* m, int32_t* d) {
    if (!m) {
        d[0] = d[1] = d[2] = d[3] = -1;
        return;
    }
    d[0] = m->b_dim;
    d[1] = m->h_dim;
    d[2] = m->nq;
    d[3] = m->nk;
}
bool same_tensor_shape(const nsa_tensor& a, const nsa_tensor& b) {
    return a.dtype == b.dtype && a.B == b.B && a.H == b.H && a.S == b.S && a.D == b.D;
}
bool same_spec(const nsa_spec& a, const nsa_spec& b) {
    uint32_t ba, bb;
    std::memcpy(&ba, &a.budget, 4);
    std::memcpy(&bb, &b.budget, 4);
    return ba == bb && a.block_q == b.block_q && a.block_kv == b.block_kv && a.head_shared == b.head_shared &&
           a.force == b.force && a.score_chunk_bytes == b.score_chunk_bytes;
}
bool same_mask(const int32_t* dims, const std::vector<int8_t>& bytes, uint64_t hash, const nsa_mask* m,
               uint64_t mhash) {
    int32_t md[4];
    mask_dims(m, md);
    if (std::memcmp(dims, md, sizeof md) != 0 || hash != mhash) return false;
    const size_t n = mask_bytes(m);
    return n == bytes.size() && (n == 0 || std::memcmp(bytes.data(), m->data, n) == 0);
}

// The plan of a validated request (g from validate_select), from the cache or
// built (and cached) now.
int cached_plan(const Geo& g, const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec, const nsa_mask* pins,
                const nsa_mask* drops, std::shared_ptr<const Plan>& out) {
    PlanCache& c = plan_cache();
    size_t cap;
    {
        std::lock_guard<std::mutex> lock(c.mu);
        cap = c.capacity;
    }
    if (mask_bytes(pins) + mask_bytes(drops) > kMaxCachedMaskBytes) cap = 0;
    const uint64_t ph = cap ? mask_hash(pins) : 0, dh = cap ? mask_hash(drops) : 0;
    auto find = [&]() -> PlanCacheEntry* {  // caller holds c.mu
        for (PlanCacheEntry& e : c.entries) {
            if (!same_tensor_shape(e.q, *q) || !same_tensor_shape(e.k, *k) || !same_spec(e.spec, *spec)) continue;
            if (!same_mask(e.pdims, e.pins, e.phash, pins, ph) || !same_mask(e.ddims, e.drops, e.dhash, drops, dh))
                continue;
            return &e;
        }
        return nullptr;
    };
    if (cap) {
        std::lock_guard<std::mutex> lock(c.mu);
        if (PlanCacheEntry* e = find()) {
            e->stamp = ++c.clock;
            ++c.hits;
            out = e->plan;
            return NSA_OK;
        }
    }
    auto built = std::make_shared<Plan>();
    const int st = build_plan(g, spec, pins, drops, *built, true);
    if (st != NSA_OK) return st;
    out = built;
    std::lock_guard<std::mutex> lock(c.mu);
    ++c.misses;
    if (c.capacity == 0 || !cap) return NSA_OK;
    if (PlanCacheEntry* e = find()) {  // another caller built the same plan meanwhile
        e->stamp = ++c.clock;
        return NSA_OK;
    }
    PlanCacheEntry e;
    e.q = *q;
    e.k = *k;
    e.q.data = nullptr;
    e.k.data = nullptr;
    e.spec = *spec;
    mask_dims(pins, e.pdims);
    mask_dims(drops, e.ddims);
    e.phash = ph;
    e.dhash = dh;
    if (pins) e.pins.assign(pins->data, pins->data + mask_bytes(pins));
    if (drops) e.drops.assign(drops->data, drops->data + mask_bytes(drops));
    e.plan = built;
    e.stamp = ++c.clock;
    if (c.entries.size() >= c.capacity) {
        auto lru = std::min_element(c.entries.begin(), c.entries.end(),
                                    [](const PlanCacheEntry& a, const PlanCacheEntry& b) { return a.stamp < b.stamp; });
        *lru = std::move(e);
    } else {
        c.entries.push_back(std::move(e));
    }
    return NSA_OK;
}
}  // namespace

extern "C" {

const char* nsa_version(void) { return "0.1.0"; }

int nsa_last_hip_error(void) { return g_last_hip; }

const char* nsa_status_string(int status) {
    switch (status) {
        case NSA_OK: return "ok";
        case NSA_DENSE: return "dense: the budget covers every candidate tile, attend densely";
        case NSA_ERR_NULL_ARG: return "a required pointer is NULL";
        case NSA_ERR_BAD_SHAPE: return "inconsistent shapes (or Hq % Hkv != 0, or a mask that does not broadcast)";
        case NSA_ERR_BAD_DTYPE: return "unsupported or mismatched dtype";
        case NSA_ERR_UNSUPPORTED: return "valid request this library does not run";
        case NSA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case NSA_ERR_BAD_SPEC: return "invalid spec (block size <= 0, budget < 0 or NaN, chunk bytes < 0)";
        case NSA_ERR_HIP: return "HIP runtime error (see nsa_last_hip_error)";
        case NSA_ERR_CAPACITY: return "col_idx capacity is below the selection's nnz";
        default: return "unknown status";
    }
}

int nsa_select_sizes(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec, const nsa_mask* pins,
                     const nsa_mask* drops, nsa_sizes* out, int32_t* row_ptr_host) {
    try {
        if (!out) return NSA_ERR_NULL_ARG;
        Geo g;
        int st = validate_select(q, k, spec, pins, drops, g);
        if (st != NSA_OK) return st;
        std::shared_ptr<const Plan> p;
        st = cached_plan(g, q, k, spec, pins, drops, p);
        if (st != NSA_OK) return st;
        fill_sizes(*p, spec, out, row_ptr_host);
        return NSA_OK;
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}

int nsa_select(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec, const nsa_mask* pins,
               const nsa_mask* drops, nsa_selection* out, void* workspace, size_t workspace_bytes,
               void* stream_) {
    try {
        if (!out) return NSA_ERR_NULL_ARG;
        Geo g;
        int st = validate_select(q, k, spec, pins, drops, g);
        if (st != NSA_OK) return st;
        std::shared_ptr<const Plan> p;
        st = cached_plan(g, q, k, spec, pins, drops, p);
        if (st != NSA_OK) return st;
        return run_select(q, k, spec, *p, out, workspace, workspace_bytes, (hipStream_t)stream_);
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}

int nsa_plan_create(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec, const nsa_mask* pins,
                    const nsa_mask* drops, nsa_plan** out) {
    try {
        if (!out) return NSA_ERR_NULL_ARG;
        *out = nullptr;
        Geo g;
        int st = validate_select(q, k, spec, pins, drops, g);
        if (st != NSA_OK) return st;
        nsa_plan* plan = new nsa_plan();
        plan->spec = *spec;
        plan->qshape = *q;
        plan->kshape = *k;
        plan->qshape.data = nullptr;
        plan->kshape.data = nullptr;
        st = build_plan(g, spec, pins, drops, plan->p, true);
        if (st != NSA_OK) {
            delete plan;
            return st;
        }
        *out = plan;
        return NSA_OK;
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}

int nsa_plan_sizes(const nsa_plan* plan, nsa_sizes* out, int32_t* row_ptr_host) {
    if (!plan || !out) return NSA_ERR_NULL_ARG;
    fill_sizes(plan->p, &plan->spec, out, row_ptr_host);
    return NSA_OK;
}

namespace {
// Device image of a plan: row offsets, then pin words, then drop words, each
// section 256-byte aligned.
struct PlanImage {
    size_t rb, pb, db;
    size_t total() const { return rb + pb + db; }
};
PlanImage plan_image(const Plan& p) {
    return {align256(p.row_ptr.size() * sizeof(int32_t)), align256(p.has_pins ? p.pin_words.size() * 8 : 0),
            align256(p.has_drops ? p.drop_words.size() * 8 : 0)};
}
}  // namespace

int nsa_plan_device_bytes(const nsa_plan* plan, int64_t* bytes) {
    if (!plan || !bytes) return NSA_ERR_NULL_ARG;
    *bytes = (int64_t)plan_image(plan->p).total();
    return NSA_OK;
}

int nsa_plan_upload(const nsa_plan* plan, void* plan_dev, size_t bytes, void* stream) {
    try {
        if (!plan) return NSA_ERR_NULL_ARG;
        const Plan& p = plan->p;
        const PlanImage im = plan_image(p);
        if (!plan_dev || ((uintptr_t)plan_dev & 255) || bytes < im.total()) return NSA_ERR_WORKSPACE;
        char* c = (char*)plan_dev;
        void* dst[3] = {c, c + im.rb, c + im.rb + im.pb};
        const void* src[3] = {p.row_ptr.data(), p.pin_words.data(), p.drop_words.data()};
        size_t n[3] = {p.row_ptr.size() * sizeof(int32_t), p.has_pins ? p.pin_words.size() * 8 : 0,
                       p.has_drops ? p.drop_words.size() * 8 : 0};
        const hipError_t e = upload(3, dst, src, n, (hipStream_t)stream);
        return e == hipSuccess ? NSA_OK : hip_fail(e);
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}

int nsa_select_planned(const nsa_plan* plan, const void* plan_dev, const nsa_tensor* q, const nsa_tensor* k,
                       nsa_selection* out, void* workspace, size_t workspace_bytes, void* stream) {
    try {
        if (!plan || !out) return NSA_ERR_NULL_ARG;
        int st;
        if ((st = check_tensor(q)) != NSA_OK) return st;
        if ((st = check_tensor(k)) != NSA_OK) return st;
        const nsa_tensor &pq = plan->qshape, &pk = plan->kshape;
        if (q->dtype != pq.dtype || k->dtype != pk.dtype) return NSA_ERR_BAD_DTYPE;
        if (q->B != pq.B || q->H != pq.H || q->S != pq.S || q->D != pq.D) return NSA_ERR_BAD_SHAPE;
        if (k->B != pk.B || k->H != pk.H || k->S != pk.S || k->D != pk.D) return NSA_ERR_BAD_SHAPE;
        if (plan_dev && ((uintptr_t)plan_dev & 255)) return NSA_ERR_WORKSPACE;
        const Plan& p = plan->p;
        PlanDevice pd;
        if (plan_dev) {  // the plan's image, uploaded by nsa_plan_upload: nothing is copied here
            const PlanImage im = plan_image(p);
            const char* c = (const char*)plan_dev;
            pd.row_ptr = (int32_t*)c;
            pd.pin_words = im.pb ? (uint64_t*)(c + im.rb) : nullptr;
            pd.drop_words = im.db ? (uint64_t*)(c + im.rb + im.pb) : nullptr;
        }
        return run_select(q, k, &plan->spec, p, out, workspace, workspace_bytes, (hipStream_t)stream,
                          plan_dev ? &pd : nullptr);
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}

void nsa_plan_destroy(nsa_plan* plan) { delete plan; }

int nsa_plan_cache_config(int32_t capacity) {
    if (capacity < 0) return NSA_ERR_BAD_SPEC;
    PlanCache& c = plan_cache();
    std::lock_guard<std::mutex> lock(c.mu);
    c.capacity = (size_t)capacity;
    if (c.entries.size() > c.capacity) {  // keep the most recently used
        std::sort(c.entries.begin(), c.entries.end(),
                  [](const PlanCacheEntry& a, const PlanCacheEntry& b) { return a.stamp > b.stamp; });
        c.entries.resize(c.capacity);
    }
    return NSA_OK;
}

void nsa_plan_cache_clear(void) {
    PlanCache& c = plan_cache();
    std::lock_guard<std::mutex> lock(c.mu);
    c.entries.clear();
    c.hits = 0;
    c.misses = 0;
}

int nsa_plan_cache_stats(int64_t* hits, int64_t* misses, int32_t* entries) {
    if (!hits || !misses || !entries) return NSA_ERR_NULL_ARG;
    PlanCache& c = plan_cache();
    std::lock_guard<std::mutex> lock(c.mu);
    *hits = c.hits;
    *misses = c.misses;
    *entries = (int32_t)c.entries.size();
    return NSA_OK;
}

int nsa_schedule(int32_t steps, double budget, double bump, int32_t bump_steps, double* out) {
    if (steps > 0 && !out) return NSA_ERR_NULL_ARG;
    if (!(bump > 0) || bump_steps <= 0 || steps <= 0) {
        for (int32_t i = 0; i < steps; ++i) out[i] = budget;
        return NSA_OK;
    }
    const double raised = std::min(1.0, budget + bump);
    const int32_t edge = std::min<int32_t>(bump_steps, (int32_t)ceil_div(steps, 2));
    for (int32_t i = 0; i < steps; ++i) out[i] = (i < edge || i >= steps - edge) ? raised : budget;
    return NSA_OK;
}

int nsa_radial_sizes(int32_t seq_q, int32_t seq_kv, double density, const nsa_spec* spec, nsa_sizes* out,
                     int32_t* row_ptr_host) {
    try {
        if (!spec || !out) return NSA_ERR_NULL_ARG;
        if (spec->block_q <= 0 || spec->block_kv <= 0 || seq_q < 0 || seq_kv < 0) return NSA_ERR_BAD_SPEC;
        Band band;
        const int st = build_band(seq_q, seq_kv, density, spec->block_q, spec->block_kv, band);
        if (st != NSA_OK) return st;
        out->NQ = band.NQ;
        out->NK = band.NK;
        out->sel_heads = 1;
        out->dense = 0;
        out->rows = band.NQ;
        out->nnz = (int64_t)band.col_idx.size();
        out->workspace_bytes = 0;
        if (row_ptr_host) std::memcpy(row_ptr_host, band.row_ptr.data(), band.row_ptr.size() * sizeof(int32_t));
        return NSA_OK;
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}

int nsa_radial_blocks(int32_t seq_q, int32_t seq_kv, double density, const nsa_spec* spec, nsa_selection* out,
                      void* stream) {
    try {
        if (!spec || !out) return NSA_ERR_NULL_ARG;
        if (spec->block_q <= 0 || spec->block_kv <= 0 || seq_q < 0 || seq_kv < 0) return NSA_ERR_BAD_SPEC;
        Band band;
        const int st = build_band(seq_q, seq_kv, density, spec->block_q, spec->block_kv, band);
        if (st != NSA_OK) return st;
        const int64_t nnz = (int64_t)band.col_idx.size();
        if (!out->row_ptr || (band.keep.size() > 0 && !out->keep) || (nnz > 0 && !out->col_idx))
            return NSA_ERR_NULL_ARG;
        if (out->col_capacity < nnz) return NSA_ERR_CAPACITY;
        out->nnz = nnz;
        out->B = 1;
        out->H = 1;
        out->NQ = band.NQ;
        out->NK = band.NK;
        out->block_q = spec->block_q;
        out->block_kv = spec->block_kv;
        out->seq_q = seq_q;
        out->seq_kv = seq_kv;
        out->budget = (float)density;
        void* dst[3] = {out->keep, out->row_ptr, out->col_idx};
        const void* src[3] = {band.keep.data(), band.row_ptr.data(), band.col_idx.data()};
        size_t bytes[3] = {band.keep.size(), band.row_ptr.size() * sizeof(int32_t), (size_t)nnz * sizeof(int32_t)};
        const hipError_t e = upload(3, dst, src, bytes, (hipStream_t)stream);
        return e == hipSuccess ? NSA_OK : hip_fail(e);
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}


int nsa_curve_order(int32_t kind, int32_t ndim, const int32_t* dims, int32_t* perm) {
    try {
        if (!dims) return NSA_ERR_NULL_ARG;
        if (kind != NSA_CURVE_MORTON && kind != NSA_CURVE_HILBERT) return NSA_ERR_BAD_SPEC;
        if (ndim < 1 || ndim > 4) return NSA_ERR_UNSUPPORTED;
        int64_t n = 1, mx = 1;
        for (int a = 0; a < ndim; ++a) {
            if (dims[a] < 0) return NSA_ERR_BAD_SHAPE;
            n *= dims[a];
            mx = std::max<int64_t>(mx, dims[a]);
        }
        if (n >= ((int64_t)1 << 31)) return NSA_ERR_UNSUPPORTED;
        if (n > 0 && !perm) return NSA_ERR_NULL_ARG;
        int p = 1;
        while (((int64_t)1 << p) < mx) ++p;
        if (p * ndim > 63) return NSA_ERR_UNSUPPORTED;
        std::vector<std::pair<uint64_t, int32_t>> order((size_t)n);
        int64_t c[4];
        for (int64_t r = 0; r < n; ++r) {
            int64_t rem = r;
            for (int a = ndim - 1; a >= 0; --a) {
                c[a] = rem % dims[a];
                rem /= dims[a];
            }
            const uint64_t key = kind == NSA_CURVE_MORTON ? morton_key(c, ndim, p) : hilbert_key(c, ndim, p);
            order[(size_t)r] = {key, (int32_t)r};
        }
        std::sort(order.begin(), order.end());
        for (int64_t m = 0; m < n; ++m) perm[m] = order[(size_t)m].second;
        return NSA_OK;
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}

int nsa_permute_tokens(const nsa_tensor* x, const int32_t* perm, int32_t inverse, nsa_tensor* y, void* stream) {
    int st;
    if ((st = check_tensor(x)) != NSA_OK) return st;
    if ((st = check_tensor(y)) != NSA_OK) return st;
    if (x->dtype != y->dtype) return NSA_ERR_BAD_DTYPE;
    if (x->B != y->B || x->H != y->H || x->S != y->S || x->D != y->D) return NSA_ERR_BAD_SHAPE;
    if (numel(x) == 0) return NSA_OK;
    if (!perm) return NSA_ERR_NULL_ARG;
    if (x->data == y->data) return NSA_ERR_UNSUPPORTED;  // not in place
    const int esz = x->dtype == NSA_BF16 ? 2 : 4;
    const int row_bytes = x->D * esz;
    if (row_bytes < 64 || row_bytes > 1024 || (row_bytes & (row_bytes - 1))) return NSA_ERR_UNSUPPORTED;
    if (((uintptr_t)x->data & 15) || ((uintptr_t)y->data & 15)) return NSA_ERR_UNSUPPORTED;
    const hipError_t e = nsa::launch_permute_rows(x->data, perm, inverse ? 1 : 0, (int64_t)x->B * x->H, x->S,
                                                  row_bytes, y->data, (hipStream_t)stream);
    return e == hipSuccess ? NSA_OK : hip_fail(e);
}


int nsa_decode_pool_update(const nsa_tensor* k_cache, int32_t len_old, int32_t len_new, int32_t block_kv,
                           float* pooled, int32_t tiles_capacity, void* stream) {
    int st;
    if ((st = check_tensor(k_cache)) != NSA_OK) return st;
    if (block_kv <= 0) return NSA_ERR_BAD_SPEC;
    if (len_old < 0 || len_new < len_old || len_new > k_cache->S) return NSA_ERR_BAD_SHAPE;
    if (ceil_div(len_new, block_kv) > tiles_capacity) return NSA_ERR_BAD_SHAPE;
    if (k_cache->D != 64 && k_cache->D != 128 && k_cache->D != 256) return NSA_ERR_UNSUPPORTED;
    if (len_new == len_old || (int64_t)k_cache->B * k_cache->H == 0) return NSA_OK;
    if (!pooled) return NSA_ERR_NULL_ARG;
    // Tiles holding a new token: from the one containing len_old to the last.
    const int t0 = len_old / block_kv;
    const int t1 = (int)ceil_div(len_new, block_kv);
    const hipError_t e = nsa::launch_pool_range(k_cache->data, k_cache->dtype == NSA_BF16,
                                                (int64_t)k_cache->B * k_cache->H, len_new, k_cache->S, k_cache->D,
                                                block_kv, t0, t1 - t0, pooled, tiles_capacity, (hipStream_t)stream);
    return e == hipSuccess ? NSA_OK : hip_fail(e);
}

int nsa_decode_select_sizes(const nsa_tensor* q, const nsa_tensor* pooled_k, int32_t length, int32_t q_pos0,
                            const nsa_spec* spec, const nsa_mask* pins, const nsa_mask* drops, nsa_sizes* out,
                            int32_t* row_ptr_host) {
    try {
        if (!out) return NSA_ERR_NULL_ARG;
        Geo g;
        int st = validate_decode_select(q, pooled_k, length, q_pos0, spec, pins, drops, g);
        if (st != NSA_OK) return st;
        Plan p;
        if ((st = build_plan(g, spec, pins, drops, p, row_ptr_host != nullptr)) != NSA_OK) return st;
        fill_sizes(p, spec, out, row_ptr_host);
        out->workspace_bytes = (int64_t)decode_layout(p, spec).total;
        return NSA_OK;
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}

int nsa_decode_select(const nsa_tensor* q, const nsa_tensor* pooled_k, int32_t length, int32_t q_pos0,
                      const nsa_spec* spec, const nsa_mask* pins, const nsa_mask* drops, nsa_selection* out,
                      void* workspace, size_t workspace_bytes, void* stream_) {
    try {
        hipStream_t stream = (hipStream_t)stream_;
        if (!out) return NSA_ERR_NULL_ARG;
        Geo g;
        int st = validate_decode_select(q, pooled_k, length, q_pos0, spec, pins, drops, g);
        if (st != NSA_OK) return st;
        Plan p;
        if ((st = build_plan(g, spec, pins, drops, p, true)) != NSA_OK) return st;
        if (p.dense && !spec->force) return NSA_DENSE;
        if (g.rows > 0 && (!out->keep || !out->row_ptr)) return NSA_ERR_NULL_ARG;
        if (!out->row_ptr) return NSA_ERR_NULL_ARG;
        if (p.nnz > 0 && !out->col_idx) return NSA_ERR_NULL_ARG;
        if (out->col_capacity < p.nnz) return NSA_ERR_CAPACITY;
        const WsLayout w = decode_layout(p, spec);
        if (workspace_bytes < w.total) return NSA_ERR_WORKSPACE;
        if (w.total > 0 && (!workspace || ((uintptr_t)workspace & 255))) return NSA_ERR_WORKSPACE;
        out->nnz = p.nnz;
        out->B = g.B;
        out->H = g.Hsel;
        out->NQ = g.NQ;
        out->NK = g.NK;
        out->block_q = spec->block_q;
        out->block_kv = spec->block_kv;
        out->seq_q = g.Sq;
        out->seq_kv = g.Skv;
        out->budget = spec->budget;
        char* ws = (char*)workspace;
        if (g.rows == 0 || g.NK == 0) {  // no top-k launch: the row offsets go straight to the caller
            void* dst[1] = {out->row_ptr};
            const void* src[1] = {p.row_ptr.data()};
            size_t bytes[1] = {p.row_ptr.size() * sizeof(int32_t)};
            const hipError_t e = upload(1, dst, src, bytes, stream);
            return e == hipSuccess ? NSA_OK : hip_fail(e);
        }
        // When every row keeps the same number of tiles (always so without
        // masks: every row sees the same keys) the top-k kernel computes the
        // row offsets itself, and small masks ride in its launch arguments:
        // then nothing is copied to the device.
        const int32_t step = p.row_ptr[1] - p.row_ptr[0];
        bool uniform = true;
        for (size_t r = 1; uniform && r < p.row_ptr.size(); ++r) uniform = p.row_ptr[r] == (int64_t)r * step;
        // A mask rides in the launch arguments only as one row of words that every row shares.
        const size_t mask_words = (p.has_pins ? p.pin_words.size() : 0) + (p.has_drops ? p.drop_words.size() : 0);
        const bool one_row = (!p.has_pins || p.pin_words.size() == (size_t)g.NKW) &&
                             (!p.has_drops || p.drop_words.size() == (size_t)g.NKW);
        uniform = uniform && one_row && mask_words <= (size_t)nsa::kInlineMaskWords;
        if (!uniform) {  // row offsets and mask words, one copy into the workspace
            void* dst[3] = {ws + w.rowp, ws + w.pinw, ws + w.dropw};
            const void* src[3] = {p.row_ptr.data(), p.pin_words.data(), p.drop_words.data()};
            size_t bytes[3] = {p.row_ptr.size() * sizeof(int32_t), p.has_pins ? p.pin_words.size() * 8 : 0,
                               p.has_drops ? p.drop_words.size() * 8 : 0};
            const hipError_t e = upload(3, dst, src, bytes, stream);
            if (e != hipSuccess) return hip_fail(e);
        }
        // Pooled queries; the pooled keys are the caller's cache (capacity pooled_k->S tiles per head).
        // One new token per head (per-head selection): the score kernel pools
        // its single-row tile itself and nothing is launched for it here.
        float* pq = (float*)(ws + w.pq);
        const int q_rows = (g.Sq == 1 && !spec->head_shared) ? (g.bf16 ? 1 : 2) : 0;
        hipError_t e = nsa::stage_mark("start", stream);
        if (e != hipSuccess) return hip_fail(e);
        if (!q_rows) {
            e = nsa::launch_pool(q->data, g.bf16, (int64_t)g.B * g.Hq, g.Sq, g.D, spec->block_q, pq, stream);
            if (e != hipSuccess) return hip_fail(e);
            if ((e = nsa::stage_mark("pool_q", stream)) != hipSuccess) return hip_fail(e);
        }
        const void* qh = q_rows ? q->data : (const void*)pq;
        const float* kh = (const float*)pooled_k->data;
        int Hk = g.Hkv, NKs = pooled_k->S;
        if (spec->head_shared) {
            float* mq = (float*)(ws + w.mq);
            float* mk = (float*)(ws + w.mk);
            if ((e = nsa::launch_head_mean(pq, g.B, g.Hq, g.NQ, g.D, mq, stream)) != hipSuccess) return hip_fail(e);
            if ((e = nsa::launch_head_mean(kh, g.B, g.Hkv, g.NK, g.D, mk, stream, pooled_k->S)) != hipSuccess)
                return hip_fail(e);
            qh = mq;
            kh = mk;
            Hk = 1;
            NKs = g.NK;
        }
        return score_and_topk(p, spec, qh, kh, Hk, NKs, w, ws, out, stream,
                              p.has_pins ? (const uint64_t*)(ws + w.pinw) : nullptr,
                              p.has_drops ? (const uint64_t*)(ws + w.dropw) : nullptr,
                              uniform ? nullptr : (const int32_t*)(ws + w.rowp), uniform ? step : 0, q_rows,
                              uniform);
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}

int nsa_decode_attn_workspace_size(const nsa_tensor* q, const nsa_tensor* k_cache, int32_t length, int32_t q_pos0,
                                   const nsa_selection* sel, int64_t* bytes) {
    if (!bytes) return NSA_ERR_NULL_ARG;
    nsa::AttnArgs a;
    const int st = decode_attn_config(q, k_cache, k_cache, q, length, q_pos0, sel, a);
    if (st != NSA_OK) return st;
    *bytes = (int64_t)decode_attn_workspace(a);
    return NSA_OK;
}

int nsa_decode_attn(const nsa_tensor* q, const nsa_tensor* k_cache, const nsa_tensor* v_cache, int32_t length,
                    int32_t q_pos0, const nsa_selection* sel, nsa_tensor* out, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream_) {
    hipStream_t stream = (hipStream_t)stream_;
    nsa::AttnArgs a;
    int st = decode_attn_config(q, k_cache, v_cache, out, length, q_pos0, sel, a);
    if (st != NSA_OK) return st;
    if (numel(q) > 0 && !lse) return NSA_ERR_NULL_ARG;
    a.out = out->data;
    a.lse = lse;
    if ((int64_t)a.B * a.Hq * a.NQ == 0) return NSA_OK;
    const size_t need = decode_attn_workspace(a);
    if (workspace_bytes < need || (need > 0 && !workspace)) return NSA_ERR_WORKSPACE;
    const int bf16 = q->dtype == NSA_BF16;
    hipError_t e;
    const bool dec = nsa::attn_decode_supported(a, bf16);
    if (a.nsplit > 1) {
        a.part_o = (float*)workspace;
        a.part_ml = (float*)((char*)workspace + align256((size_t)a.B * a.Hq * a.S * a.nsplit * a.D * 4));
        if ((e = dec ? nsa::launch_attn_decode(a, stream) : nsa::launch_attn_mfma(a, stream)) != hipSuccess)
            return hip_fail(e);
        e = nsa::launch_attn_combine(a, bf16, stream);
    } else if (dec) {
        e = nsa::launch_attn_decode(a, stream);
    } else {
        e = nsa::attn_mfma_supported(a, bf16) ? nsa::launch_attn_mfma(a, stream)
                                              : nsa::launch_attn_simt(a, bf16, stream);
    }
    return e == hipSuccess ? NSA_OK : hip_fail(e);
}

int nsa_decode_attn_static(const nsa_tensor* q, const nsa_tensor* k_cache, const nsa_tensor* v_cache,
                           int32_t length, int32_t q_pos0, const nsa_selection* sel, nsa_tensor* out, float* lse,
                           void* stream) {
    nsa::AttnArgs a;
    int st = decode_attn_config(q, k_cache, v_cache, out, length, q_pos0, sel, a);
    if (st != NSA_OK) return st;
    if (numel(q) > 0 && !lse) return NSA_ERR_NULL_ARG;
    if ((int64_t)a.B * a.Hq * a.NQ == 0) return NSA_OK;
    const size_t need = decode_attn_workspace(a);
    if (need > nsa::kDecodeScratchBytes) return NSA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = nsa::decode_scratch(&ws);
        if (e != hipSuccess) return hip_fail(e);
    }
    return nsa_decode_attn(q, k_cache, v_cache, length, q_pos0, sel, out, lse, ws, need, stream);
}

int nsa_stage_timing_begin(void) {
    nsa::StageTiming& t = nsa::t_stages;
    for (hipEvent_t ev : t.marks) (void)hipEventDestroy(ev);
    t.names.clear();
    t.marks.clear();
    t.on = true;
    return NSA_OK;
}

int nsa_stage_timing_end(nsa_stage_time* out, int32_t capacity, int32_t* count) {
    nsa::StageTiming& t = nsa::t_stages;
    t.on = false;
    if (!count || (capacity > 0 && !out)) return NSA_ERR_NULL_ARG;
    int32_t n = 0;
    int st = NSA_OK;
    hipError_t e = t.marks.empty() ? hipSuccess : hipEventSynchronize(t.marks.back());
    if (e != hipSuccess) st = hip_fail(e);
    for (size_t x = 1; st == NSA_OK && x < t.marks.size(); ++x) {
        if (std::strcmp(t.names[x], "start") == 0) continue;  // a new call: no stage ends here
        float ms = 0.f;
        if ((e = hipEventElapsedTime(&ms, t.marks[x - 1], t.marks[x])) != hipSuccess) {
            st = hip_fail(e);
            break;
        }
        if (n < capacity) {
            out[n].name = t.names[x];
            out[n].ms = ms;
        }
        ++n;
    }
    for (hipEvent_t ev : t.marks) (void)hipEventDestroy(ev);
    t.names.clear();
    t.marks.clear();
    *count = n;
    return st;
}

int nsa_selection_density(const nsa_selection* sel, double* out) {
    if (!sel || !out) return NSA_ERR_NULL_ARG;
    const int64_t tiles = (int64_t)sel->B * sel->H * sel->NQ * sel->NK;
    *out = (double)sel->nnz / (double)std::max<int64_t>(tiles, 1);
    return NSA_OK;
}

int nsa_pool_blocks(const nsa_tensor* x, int32_t block, float* out, void* stream) {
    int st = check_tensor(x);
    if (st != NSA_OK) return st;
    if (block <= 0) return NSA_ERR_BAD_SPEC;
    if (x->D != 64 && x->D != 128 && x->D != 256) return NSA_ERR_UNSUPPORTED;
    const int64_t n = (int64_t)x->B * x->H * ceil_div(x->S, block) * x->D;
    if (n > 0 && !out) return NSA_ERR_NULL_ARG;
    hipError_t e = nsa::launch_pool(x->data, x->dtype == NSA_BF16, (int64_t)x->B * x->H, x->S, x->D, block, out,
                                    (hipStream_t)stream);
    return e == hipSuccess ? NSA_OK : hip_fail(e);
}

int nsa_score_blocks(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec, float* scores,
                     void* workspace, size_t workspace_bytes, void* stream_) {
    try {
        hipStream_t stream = (hipStream_t)stream_;
        Geo g;
        int st = validate_select(q, k, spec, nullptr, nullptr, g);
        if (st != NSA_OK) return st;
        const WsLayout w = ws_layout(g, spec, false, 0, false, 0);
        if (workspace_bytes < w.total) return NSA_ERR_WORKSPACE;
        if (w.total > 0 && (!workspace || ((uintptr_t)workspace & 255))) return NSA_ERR_WORKSPACE;
        if (g.rows > 0 && g.NK > 0 && !scores) return NSA_ERR_NULL_ARG;
        if (g.rows == 0 || g.NK == 0) return NSA_OK;
        const float* qh;
        const float* kh;
        int Hk;
        if ((st = run_pool(q, k, spec, g, w, (char*)workspace, stream, &qh, &kh, &Hk)) != NSA_OK) return st;
        hipError_t e = nsa::launch_scores(qh, kh, g.B, g.Hsel, Hk, g.group, 0, g.Hsel, g.NQ, g.NK, g.D, scores,
                                          stream);
        return e == hipSuccess ? NSA_OK : hip_fail(e);
    } catch (...) {
        return NSA_ERR_UNSUPPORTED;
    }
}

int nsa_block_sparse_attn(const nsa_tensor* q, const nsa_tensor* k, const nsa_tensor* v, const nsa_selection* sel,
                          int causal, nsa_tensor* out, float* lse, void* stream_) {
    hipStream_t stream = (hipStream_t)stream_;
    int st;
    if ((st = check_tensor(q)) != NSA_OK) return st;
    if ((st = check_tensor(k)) != NSA_OK) return st;
    if ((st = check_tensor(v)) != NSA_OK) return st;
    if ((st = check_tensor(out)) != NSA_OK) return st;
    if (q->dtype != k->dtype || q->dtype != v->dtype || q->dtype != out->dtype) return NSA_ERR_BAD_DTYPE;
    if (q->B != k->B || q->B != v->B || k->H != v->H || k->S != v->S) return NSA_ERR_BAD_SHAPE;
    if (q->D != k->D || q->D != v->D) return NSA_ERR_BAD_SHAPE;
    if (out->B != q->B || out->H != q->H || out->S != q->S || out->D != q->D) return NSA_ERR_BAD_SHAPE;
    if (q->H % k->H != 0) return NSA_ERR_BAD_SHAPE;
    if (numel(q) > 0 && !lse) return NSA_ERR_NULL_ARG;
    if (causal && q->S != k->S) return NSA_ERR_UNSUPPORTED;
    if (q->D != 64 && q->D != 128) return NSA_ERR_UNSUPPORTED;
    if (q->S != k->S) return NSA_ERR_UNSUPPORTED;

    nsa::AttnArgs a;
    a.q = q->data;
    a.k = k->data;
    a.v = v->data;
    a.out = out->data;
    a.lse = lse;
    a.B = q->B;
    a.Hq = q->H;
    a.Hkv = k->H;
    a.S = q->S;
    a.Skv = k->S;
    a.kv_rows = k->S;
    a.q_off = 0;
    a.nsplit = 1;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    a.D = q->D;
    a.causal = causal ? 1 : 0;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)q->D));
    if (sel) {
        if (!sel->row_ptr) return NSA_ERR_NULL_ARG;
        if (sel->nnz > 0 && !sel->col_idx) return NSA_ERR_NULL_ARG;
        if (sel->block_q <= 0 || sel->block_kv <= 0) return NSA_ERR_BAD_SPEC;
        if ((sel->B != q->B && sel->B != 1) || (sel->H != 1 && sel->H != q->H)) return NSA_ERR_BAD_SHAPE;
        if (sel->seq_q != q->S || sel->seq_kv != k->S) return NSA_ERR_BAD_SHAPE;
        if (sel->NQ != ceil_div(q->S, sel->block_q) || sel->NK != ceil_div(k->S, sel->block_kv))
            return NSA_ERR_BAD_SHAPE;
        a.row_ptr = sel->row_ptr;
        a.col_idx = sel->col_idx;
        a.Hsel = sel->H;
        a.Bsel = sel->B;
        a.block_q = sel->block_q;
        a.block_kv = sel->block_kv;
    } else {
        a.row_ptr = nullptr;
        a.col_idx = nullptr;
        a.Hsel = q->H;
        a.Bsel = q->B;
        a.block_q = 128;
        a.block_kv = 64;
    }
    a.NQ = (int)ceil_div(q->S, a.block_q);
    a.NK = (int)ceil_div(k->S, a.block_kv);
    if ((int64_t)a.B * a.Hq * a.NQ == 0) return NSA_OK;
    const int bf16 = q->dtype == NSA_BF16;
    hipError_t e = nsa::attn_mfma_supported(a, bf16) ? nsa::launch_attn_mfma(a, stream)
                                                       : nsa::launch_attn_simt(a, bf16, stream);
    return e == hipSuccess ? NSA_OK : hip_fail(e);
}


int nsa_attn_bwd_workspace_size(const nsa_tensor* q, const nsa_tensor* k, const nsa_selection* sel,
                                int64_t* bytes) {
    int st;
    if (!bytes) return NSA_ERR_NULL_ARG;
    if ((st = check_tensor(q)) != NSA_OK) return st;
    if ((st = check_tensor(k)) != NSA_OK) return st;
    int Hsel, bq, bkv;
    if ((st = attn_selection(q, k, sel, Hsel, bq, bkv)) != NSA_OK) return st;
    *bytes = (int64_t)bwd_layout(q, sel).total;
    return NSA_OK;
}

int nsa_block_sparse_attn_bwd(const nsa_tensor* q, const nsa_tensor* k, const nsa_tensor* v,
                              const nsa_tensor* out, const float* lse, const nsa_tensor* dout,
                              const nsa_selection* sel, int causal, nsa_tensor* dq, nsa_tensor* dk,
                              nsa_tensor* dv, void* workspace, size_t workspace_bytes, void* stream_) {
    hipStream_t stream = (hipStream_t)stream_;
    int st = validate_bwd(q, k, v, out, lse, dout, sel, causal, dq, dk, dv);
    if (st != NSA_OK) return st;
    const BwdLayout w = bwd_layout(q, sel);
    if (workspace_bytes < w.total || (w.total > 0 && !workspace)) return NSA_ERR_WORKSPACE;
    if (numel(q) == 0) return NSA_OK;  // S == 0 or B == 0: every output is empty

    nsa::AttnBwdArgs a;
    a.q = q->data;
    a.k = k->data;
    a.v = v->data;
    a.lse = lse;
    a.dout = dout->data;
    a.dq = dq->data;
    a.dk = dk->data;
    a.dv = dv->data;
    char* ws = (char*)workspace;
    float* delta = (float*)(ws + w.delta);
    a.delta = delta;
    a.B = q->B;
    a.Hq = q->H;
    a.Hkv = k->H;
    a.S = q->S;
    a.D = q->D;
    a.causal = causal ? 1 : 0;
    a.scale = (float)(1.0 / std::sqrt((double)q->D));
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)q->D));
    attn_selection(q, k, sel, a.Hsel, a.block_q, a.block_kv);
    a.Bsel = sel ? sel->B : q->B;
    a.NQ = (int)ceil_div(q->S, a.block_q);
    a.NK = (int)ceil_div(k->S, a.block_kv);
    const int bf16 = q->dtype == NSA_BF16;

    hipError_t e = nsa::stage_mark("start", stream);
    if (e != hipSuccess) return hip_fail(e);
    e = nsa::launch_bwd_delta(out->data, dout->data, bf16, (int64_t)q->B * q->H * q->S, q->D, delta, stream);
    if (e != hipSuccess) return hip_fail(e);
    if ((e = nsa::stage_mark("delta", stream)) != hipSuccess) return hip_fail(e);
    if (sel) {
        int32_t* counts = (int32_t*)(ws + w.counts);
        int32_t* col_ptr = (int32_t*)(ws + w.col_ptr);
        int32_t* row_idx = (int32_t*)(ws + w.row_idx);
        int32_t* sums = (int32_t*)(ws + w.sums);
        e = nsa::launch_kv_major_index(sel->keep, sel->B * sel->H, sel->NQ, sel->NK,
                                       (int32_t)std::max<int64_t>(sel->nnz, 0), counts, col_ptr, sums, row_idx,
                                       stream);
        if (e != hipSuccess) return hip_fail(e);
        if ((e = nsa::stage_mark("kv_index", stream)) != hipSuccess) return hip_fail(e);
        a.row_ptr = sel->row_ptr;
        a.col_idx = sel->col_idx;
        a.col_ptr = col_ptr;
        a.row_idx = row_idx;
    } else {
        a.row_ptr = a.col_idx = a.col_ptr = a.row_idx = nullptr;
    }
    e = nsa::attn_bwd_mfma_supported(a, bf16) ? nsa::launch_attn_bwd_mfma(a, stream)
                                               : nsa::launch_attn_bwd_simt(a, bf16, stream);
    return e == hipSuccess ? NSA_OK : hip_fail(e);
}

}  // extern "C"
