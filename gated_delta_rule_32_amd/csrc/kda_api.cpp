// libkda C ABI: argument checks, host planning, context records, launches.
//
// Contract sources (FlashInfer KDA pages): "flashinfer.kda_training.recurrent_
// kda_training_forward" (parameters), "flashinfer.kda_training" (paragraphs
// 1-4: overlap rule, context reuse on its own device and stream, head and
// layout rules, non-empty sequences, fixed scale and lower bound),
// "flashinfer.kda.recurrent_kda" (parameter cu_seqlens: host-side
// longest-first order cached per unchanged offsets).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/libkda.h"
#include "kda_kernels.h"

namespace {

constexpr int D = 128;  // head dimension

thread_local std::string g_last_error;

kda_status fail(kda_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

kda_status hip_fail(hipError_t e, const char* what) {
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kStateElems = (int64_t)D * D;
constexpr int kDefaultCk = 256;
constexpr int kChunk = 16;

// A validated problem.
struct Prob {
    int B, T, Hqk, Hv, N, G;
    bool packed;
    int route;      // resolved: 1 chunk, 2 rowsplit, 3 segment-parallel chunk, 4 column-split chunk
    int ck;         // tape interval
    int ctxmode;    // KDA_CONTEXT_TAPE or KDA_CONTEXT_RECORDS
    int precision;  // kda_precision
    int schedule;   // kda_schedule
    float scale;
    std::vector<int64_t> len;    // per sequence
    std::vector<int64_t> start;  // flattened token offset per sequence
    int64_t tokens;              // B * T
    int64_t num_tasks;
    int64_t total_ck;            // stored checkpoints (sum ceil(L/ck) - 1)
    int64_t total_chunks;        // sum ceil(L/16), each rounded up to even (record count)
    int64_t total_segs;          // sum ceil(L/ck)
    int64_t max_len;             // longest sequence
};

// Workgroups of the chunked kernel resident at once on MI355X (256 compute
// units, three each).
constexpr int64_t kChunkSlots = 768;
// Largest number of workgroups for which the column-split route is chosen:
// one per compute unit.  Measured on 8 x 1024-token sequences, the split
// forward is 9% faster than the plain one at 96 tasks and 8% slower at 192.
constexpr int64_t kSplitMax = 256;

int auto_route(const Prob& p) {
    // The chunked MFMA kernel.  With few tasks its one workgroup per task
    // leaves most compute units idle, and two other forms use them:
    //   - at most half as many tasks as compute units: two workgroups per
    //     task over half the value columns each, with producer waves that
    //     prepare four chunks ahead of the state path (about 1.6 us per
    //     chunk of the longest sequence);
    //   - when every tape segment's P and Q runs fit in one round (2 x
    //     segments x Hv <= 768): the segment-parallel form, about 2.5x the
    //     work spread over the segments, whose time grows with the segment
    //     length rather than the sequence length.  It finishes first once
    //     the longest sequence spans more than 4 segments (3 when the column
    //     split does not apply); its backward is segment-parallel as well.
    // The row-split kernel is slower per token than one chunked workgroup
    // (2 x 2048 tokens x 16 heads: 1.05 ms against 0.35 ms) and stays
    // selectable as an FP32 reference route.
    const bool split = p.ctxmode == KDA_CONTEXT_TAPE && 2 * p.num_tasks <= kSplitMax;
    if (p.ctxmode == KDA_CONTEXT_TAPE && 2 * p.total_segs * p.Hv <= kChunkSlots &&
        p.max_len > (split ? 4 : 3) * (int64_t)p.ck)
        return 3;
    if (split) return 4;
    return 1;
}

kda_status validate(const kda_problem* p, Prob& out) {
    if (p == nullptr) return fail(KDA_ERR_NULL_ARG, "problem is NULL");
    if (p->B < 1 || p->T < 1 || p->Hqk < 1 || p->Hv < 1 || p->N < 1)
        return fail(KDA_ERR_SHAPE, "B, T, Hqk, Hv and N must be >= 1 (got %d %d %d %d %d)",
                    p->B, p->T, p->Hqk, p->Hv, p->N);
    if (p->Hv % p->Hqk != 0)
        return fail(KDA_ERR_GROUPING, "Hv (%d) must be a multiple of Hqk (%d)", p->Hv, p->Hqk);
    if ((int64_t)p->N * p->Hv > (int64_t)INT32_MAX / 2)
        return fail(KDA_ERR_SHAPE, "too many (sequence, head) tasks");
    const bool packed = p->cu_seqlens != nullptr || p->cu_seqlens_host != nullptr;
    if (packed && (p->cu_seqlens == nullptr || p->cu_seqlens_host == nullptr))
        return fail(KDA_ERR_NULL_ARG, "packed layout needs both cu_seqlens and cu_seqlens_host");
    const float want_scale = 1.0f / std::sqrt(128.0f);
    float scale = p->scale;
    if (scale == 0.0f) scale = want_scale;
    if (std::fabs(scale - want_scale) > 1e-6f * want_scale)
        return fail(KDA_ERR_SCALE, "scale must be 1/sqrt(128) (got %g)", (double)p->scale);
    if (p->lower_bound != -5.0f)
        return fail(KDA_ERR_LOWER_BOUND, "lower_bound must be -5 (got %g)", (double)p->lower_bound);
    if (p->route < 0 || p->route > 4) return fail(KDA_ERR_ROUTE, "unknown route %d", p->route);
    int ck = p->checkpoint_every == 0 ? kDefaultCk : p->checkpoint_every;
    if (ck <= 0 || ck % kChunk != 0)
        return fail(KDA_ERR_ROUTE, "checkpoint_every must be a positive multiple of 16 (got %d)",
                    p->checkpoint_every);
    if (p->context != KDA_CONTEXT_TAPE && p->context != KDA_CONTEXT_RECORDS)
        return fail(KDA_ERR_ROUTE, "unknown context kind %d", p->context);
    if (p->context == KDA_CONTEXT_RECORDS && p->route >= 2)
        return fail(KDA_ERR_ROUTE, "per-chunk records need the chunked route");
    if (p->precision < KDA_PRECISION_AUTO || p->precision > KDA_PRECISION_FAST)
        return fail(KDA_ERR_ROUTE, "unknown precision %d", p->precision);
    if (p->schedule != KDA_SCHEDULE_LONGEST_FIRST && p->schedule != KDA_SCHEDULE_SEQUENCE)
        return fail(KDA_ERR_ROUTE, "unknown schedule %d", p->schedule);

    out = Prob{};
    out.B = p->B; out.T = p->T; out.Hqk = p->Hqk; out.Hv = p->Hv; out.N = p->N;
    out.G = p->Hv / p->Hqk;
    out.packed = packed;
    out.ck = ck;
    out.ctxmode = p->context;
    out.precision = p->precision;
    out.schedule = p->schedule;
    out.scale = want_scale;
    out.tokens = (int64_t)p->B * p->T;
    if (packed) {
        if (p->B != 1) return fail(KDA_ERR_SHAPE, "packed layout needs B == 1 (got %d)", p->B);
        const int64_t* cu = p->cu_seqlens_host;
        if (cu[0] != 0) return fail(KDA_ERR_SEQLENS, "cu_seqlens must start at 0");
        for (int n = 0; n < p->N; ++n) {
            if (cu[n + 1] <= cu[n])
                return fail(KDA_ERR_SEQLENS, "sequence %d is empty or offsets decrease", n);
        }
        if (cu[p->N] != p->T)
            return fail(KDA_ERR_SEQLENS, "cu_seqlens must end at T=%d (got %lld)", p->T,
                        (long long)cu[p->N]);
        out.len.resize(p->N);
        out.start.resize(p->N);
        for (int n = 0; n < p->N; ++n) {
            out.start[n] = cu[n];
            out.len[n] = cu[n + 1] - cu[n];
        }
    } else {
        if (p->N != p->B)
            return fail(KDA_ERR_SHAPE, "fixed layout needs N == B (got N=%d, B=%d)", p->N, p->B);
        out.len.assign(p->N, p->T);
        out.start.resize(p->N);
        for (int n = 0; n < p->N; ++n) out.start[n] = (int64_t)n * p->T;
    }
    out.num_tasks = (int64_t)p->N * p->Hv;
    out.total_ck = out.total_chunks = out.total_segs = out.max_len = 0;
    for (int64_t L : out.len) {
        out.max_len = std::max(out.max_len, L);
        out.total_ck += (L + ck - 1) / ck - 1;
        out.total_segs += (L + ck - 1) / ck;
        out.total_chunks += ((L + kChunk - 1) / kChunk + 1) & ~(int64_t)1;
    }
    // kernels address a sequence's rows with 32-bit element offsets
    for (int64_t L : out.len)
        if (L * (int64_t)p->Hv * D >= ((int64_t)1 << 31))
            return fail(KDA_ERR_SHAPE, "a sequence of %lld tokens x %d heads x 128 exceeds 2^31 elements",
                        (long long)L, p->Hv);
    out.route = p->route == 0 ? auto_route(out) : p->route;
    return KDA_OK;
}

// Longest sequence first; ties keep sequence order.  Within a sequence the
// value heads follow each other, so heads sharing a q/k head are adjacent.
// Sequences in dispatch order: longest first (ties in sequence order), or
// sequence order under KDA_SCHEDULE_SEQUENCE.
std::vector<int> seq_order(const Prob& p) {
    std::vector<int> seqs(p.N);
    for (int n = 0; n < p.N; ++n) seqs[n] = n;
    if (p.schedule == KDA_SCHEDULE_LONGEST_FIRST)
        std::stable_sort(seqs.begin(), seqs.end(),
                         [&](int a, int b) { return p.len[a] > p.len[b]; });
    return seqs;
}

std::vector<int32_t> lpt_order(const Prob& p) {
    const std::vector<int> seqs = seq_order(p);
    std::vector<int32_t> order;
    order.reserve((size_t)p.num_tasks);
    for (int n : seqs)
        for (int h = 0; h < p.Hv; ++h) order.push_back(n * p.Hv + h);
    return order;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Byte layout of a device schedule (one buffer): the task order, sequence
// starts and lengths, tape and chunk offsets, and the segment list.
struct PlanLayout {
    size_t off_task = 0, off_start = 0, off_len = 0, off_tape = 0, off_chunk = 0, off_seg = 0;
    size_t bytes = 0;
};

PlanLayout plan_layout(const Prob& p) {
    PlanLayout l;
    size_t off = 0;
    l.off_task = off;  off = align256(off + sizeof(int32_t) * (size_t)p.num_tasks);
    l.off_start = off; off = align256(off + sizeof(int64_t) * (size_t)p.N);
    l.off_len = off;   off = align256(off + sizeof(int32_t) * (size_t)p.N);
    l.off_tape = off;  off = align256(off + sizeof(int64_t) * (size_t)(p.N + 1));
    l.off_chunk = off; off = align256(off + sizeof(int64_t) * (size_t)(p.N + 1));
    l.off_seg = off;   off = align256(off + sizeof(int32_t) * 2 * (size_t)p.total_segs);
    l.bytes = off;
    return l;
}

// Writes the schedule of `p` into `h` (l.bytes bytes, host memory).
void fill_plan(const Prob& p, const PlanLayout& l, char* h) {
    std::memset(h, 0, l.bytes);
    std::vector<int32_t> order = lpt_order(p);
    std::memcpy(h + l.off_task, order.data(), sizeof(int32_t) * order.size());
    int64_t* st = (int64_t*)(h + l.off_start);
    int32_t* ln = (int32_t*)(h + l.off_len);
    int64_t* to = (int64_t*)(h + l.off_tape);
    int64_t* co = (int64_t*)(h + l.off_chunk);
    int32_t* sg = (int32_t*)(h + l.off_seg);
    to[0] = 0;
    co[0] = 0;
    int64_t si = 0;
    // segments in the dispatch order of their sequences
    for (int n = 0; n < p.N; ++n) {
        st[n] = p.start[n];
        ln[n] = (int32_t)p.len[n];
        to[n + 1] = to[n] + (p.len[n] + p.ck - 1) / p.ck - 1;
        co[n + 1] = co[n] + (((p.len[n] + kChunk - 1) / kChunk + 1) & ~(int64_t)1);  // even
    }
    for (int n : seq_order(p)) {
        const int64_t nseg = (p.len[n] + p.ck - 1) / p.ck;
        for (int64_t j = 0; j < nseg; ++j) {
            sg[2 * si] = n;
            sg[2 * si + 1] = (int32_t)j;
            ++si;
        }
    }
}

kda::DevPlan dev_plan_at(const void* dev, const PlanLayout& l) {
    const char* d = (const char*)dev;
    kda::DevPlan p;
    p.task = (const int32_t*)(d + l.off_task);
    p.seq_start = (const int64_t*)(d + l.off_start);
    p.seq_len = (const int32_t*)(d + l.off_len);
    p.tape_off = (const int64_t*)(d + l.off_tape);
    p.chunk_off = (const int64_t*)(d + l.off_chunk);
    return p;
}

// ---------------------------------------------------------------------------
// Device schedule cache
// ---------------------------------------------------------------------------
struct PlanEntry {
    void* dev = nullptr;
    void* host = nullptr;
    hipEvent_t ready = nullptr;
    bool settled = false;  // the upload behind `ready` was seen complete
    bool pinned = false;   // used under stream capture: a graph holds its device pointers
    int busy = 0;          // calls between get_plan and the end of their lease
    uint64_t last = 0;     // least-recently-used order
    // the last use on each stream that launched with it (events recorded
    // after the launches; all complete means no queued kernel reads it)
    std::vector<std::pair<hipStream_t, hipEvent_t>> uses;
    PlanLayout lay;
};

std::mutex g_mu;
std::map<std::vector<int64_t>, std::unique_ptr<PlanEntry>> g_plans;
uint64_t g_tick = 0;
// Distinct length sets kept at once; when full, the least recently used
// quarter of the evictable schedules is freed (variable-length training
// makes a new set almost every step).
constexpr size_t kMaxPlans = 1024;

// Frees a schedule's buffers and events (null members are skipped).
void free_plan(PlanEntry* e) {
    for (auto& u : e->uses) hipEventDestroy(u.second);
    e->uses.clear();
    if (e->ready) hipEventDestroy(e->ready);
    if (e->dev) hipFree(e->dev);
    if (e->host) hipHostFree(e->host);
    e->ready = nullptr;
    e->dev = e->host = nullptr;
}

// Called with g_mu held when the cache is full.  A schedule may be freed only
// when no call holds it, no captured graph refers to it, and its upload and
// every launch that read it have completed (waited for here).
kda_status evict_plans() {
    using It = decltype(g_plans)::iterator;
    std::vector<std::pair<uint64_t, It>> cand;
    for (It it = g_plans.begin(); it != g_plans.end(); ++it)
        if (it->second->busy == 0 && !it->second->pinned) cand.emplace_back(it->second->last, it);
    if (cand.empty())
        return fail(KDA_ERR_HIP, "schedule cache full (%zu length sets, all in use or captured)",
                    g_plans.size());
    std::sort(cand.begin(), cand.end(),
              [](const std::pair<uint64_t, It>& x, const std::pair<uint64_t, It>& y) { return x.first < y.first; });
    const size_t n = std::max<size_t>(1, cand.size() / 4);
    for (size_t i = 0; i < n; ++i) {
        PlanEntry* e = cand[i].second->second.get();
        hipError_t r = hipEventSynchronize(e->ready);
        for (size_t j = 0; r == hipSuccess && j < e->uses.size(); ++j) r = hipEventSynchronize(e->uses[j].second);
        if (r != hipSuccess) return hip_fail(r, "hipEventSynchronize(schedule eviction)");
        free_plan(e);
        g_plans.erase(cand[i].second);
    }
    return KDA_OK;
}

// One call's hold on a schedule, from get_plan to the end of the call: the
// schedule cannot be evicted meanwhile, and at the end the call's last use is
// recorded on its stream (or, for a call recorded into a graph, the schedule
// is pinned for the life of the process).
struct PlanLease {
    PlanEntry* ent = nullptr;
    hipStream_t stream = nullptr;
    bool capturing = false;
    PlanLease() = default;
    PlanLease(const PlanLease&) = delete;
    PlanLease& operator=(const PlanLease&) = delete;
    ~PlanLease() {
        if (ent == nullptr) return;
        std::lock_guard<std::mutex> lock(g_mu);
        --ent->busy;
        if (capturing) {
            ent->pinned = true;
            return;
        }
        hipEvent_t ev = nullptr;
        for (auto& u : ent->uses)
            if (u.first == stream) ev = u.second;
        if (ev == nullptr) {
            if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
                ent->pinned = true;  // no way to know when it is free: keep it
                return;
            }
            ent->uses.emplace_back(stream, ev);
        }
        if (hipEventRecord(ev, stream) != hipSuccess) ent->pinned = true;
    }
};

std::vector<int64_t> plan_key(const Prob& p, int dev) {
    std::vector<int64_t> key = {dev, p.Hv, p.ck, p.packed ? 1 : 0, p.T, p.N, p.schedule};
    key.insert(key.end(), p.len.begin(), p.len.end());
    return key;
}

// Under stream capture only a settled cached schedule is usable: the call then
// enqueues nothing but its kernels.  Outside capture a cached schedule whose
// upload is still in flight is waited for on the caller's stream.
kda_status get_plan(const Prob& p, hipStream_t stream, int dev, PlanLease& lease) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    const bool capturing = cs != hipStreamCaptureStatusNone;
    std::lock_guard<std::mutex> lock(g_mu);
    auto key = plan_key(p, dev);
    auto it = g_plans.find(key);
    if (it != g_plans.end()) {
        PlanEntry* ent = it->second.get();
        if (!ent->settled && !capturing) {
            e = hipEventQuery(ent->ready);
            if (e == hipSuccess)
                ent->settled = true;
            else if (e != hipErrorNotReady)
                return hip_fail(e, "hipEventQuery");
        }
        if (!ent->settled) {
            if (capturing)
                return fail(KDA_ERR_CAPTURE,
                            "the schedule for these lengths has not been seen on the device yet; "
                            "call again outside capture after the first call completed");
            e = hipStreamWaitEvent(stream, ent->ready, 0);
            if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
        }
        ent->last = ++g_tick;
        ++ent->busy;
        lease.ent = ent;
        lease.stream = stream;
        lease.capturing = capturing;
        return KDA_OK;
    }
    if (capturing)
        return fail(KDA_ERR_CAPTURE,
                    "no schedule cached for these lengths; make the first call outside capture");
    if (g_plans.size() >= kMaxPlans) {
        kda_status es = evict_plans();
        if (es != KDA_OK) return es;
    }
    auto ent = std::make_unique<PlanEntry>();
    // on a failure below, free what was made so far
    struct Guard {
        std::unique_ptr<PlanEntry>& e;
        ~Guard() { if (e) free_plan(e.get()); }
    } guard{ent};
    ent->lay = plan_layout(p);
    e = hipHostMalloc(&ent->host, ent->lay.bytes, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(schedule)");
    fill_plan(p, ent->lay, (char*)ent->host);
    e = hipMalloc(&ent->dev, ent->lay.bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(schedule)");
    e = hipMemcpyAsync(ent->dev, ent->host, ent->lay.bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(schedule)");
    e = hipEventCreateWithFlags(&ent->ready, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    e = hipEventRecord(ent->ready, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    ent->last = ++g_tick;
    ent->busy = 1;
    lease.ent = ent.get();
    lease.stream = stream;
    lease.capturing = false;
    g_plans.emplace(std::move(key), std::move(ent));  // leaves `ent` empty: the guard frees nothing
    return KDA_OK;
}

kda::DevPlan dev_plan(const PlanEntry* e) { return dev_plan_at(e->dev, e->lay); }

// ---------------------------------------------------------------------------
// Context records (what kda_bwd checks)
// ---------------------------------------------------------------------------
struct CtxRecord {
    std::vector<int64_t> key;   // plan key (device, Hv, ck, layout, lengths)
    int B, T, Hqk, Hv, N, route, ctxmode;
    const void* ptrs[8];
    hipStream_t stream;
    size_t ctx_bytes;
    uint64_t seq;               // fill order
};
std::map<const void*, CtxRecord> g_ctx;
uint64_t g_ctx_seq = 0;
// Context buffers remembered at once; past that, filling a new buffer forgets
// the one filled longest ago (its backward then reports a mismatch).
constexpr size_t kMaxCtx = 4096;

size_t tape_bytes(const Prob& p) {
    return (size_t)p.total_ck * (size_t)p.Hv * (size_t)kStateElems * sizeof(float);
}
// Records per (16-token chunk, value head): BF16 RF(U), FP32 T^T, Akk^T and
// scale*Aqk; and the BF16 chunk-start state frags, either per chunk or, with
// pair records, per (pair of chunks, value head) for the even chunk only,
// with its BF16 CF(U), CF(Kt) and FP32 exp(gC), which step that state to the
// odd chunk.  `recs` counts chunk records (an even number per sequence and
// head).
constexpr size_t kRecS0 = (size_t)kStateElems * 2, kRecX = (size_t)kda::REC_X_ELEMS * 2,
                 kRecU = (size_t)kChunk * D * 2, kRecTA = (size_t)3 * kChunk * kChunk * sizeof(float);
struct RecLayout {
    size_t s0, x, u, ta, end;  // byte offsets of the four record arrays
};
// Pair records (the start state of even chunks only) when the adjoint has
// tasks enough to hide forming the odd chunks' states: measured with 768
// tasks (8 x 1024 tokens, 96 heads) the backward is 2.7% faster with them
// (the rebuild writes 30% fewer bytes), 3.6% with 512 (64 heads), 1.1% with
// 384, the same with 320; with 128 tasks (4 x 4096 tokens, 32 value heads),
// where each task runs at the latency of its chain, 3.5% slower.
// (The segment-parallel route, for few tasks, keeps a start state per chunk.)
constexpr int64_t kPairMinTasks = 256;
bool rec_pairs(const Prob& p) { return p.num_tasks > kPairMinTasks && p.route != 3; }
RecLayout rec_layout(size_t recs, size_t base, bool pairs) {
    RecLayout r;
    r.s0 = base;
    r.x = align256(r.s0 + (pairs ? recs / 2 : recs) * kRecS0);
    r.u = align256(r.x + (pairs ? recs / 2 : 0) * kRecX);
    r.ta = align256(r.u + recs * kRecU);
    r.end = align256(r.ta + recs * kRecTA);
    return r;
}
// the segment-parallel route's P, Q and P^T of every segment, after the tape
size_t seg_scratch_off(const Prob& p) { return align256(256 + tape_bytes(p)); }
size_t ctx_bytes_for(const Prob& p) {
    if (p.ctxmode == KDA_CONTEXT_RECORDS)
        return rec_layout((size_t)p.total_chunks * p.Hv, 256, rec_pairs(p)).end;
    if (p.route == 3)
        return seg_scratch_off(p) + 3 * (size_t)p.total_segs * p.Hv * (size_t)kStateElems * sizeof(float);
    return 256 + tape_bytes(p);
}

struct Span {
    const void* p;
    size_t n;
    const char* name;
};

bool overlaps(const Span& a, const Span& b) {
    if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
    const char* a0 = (const char*)a.p;
    const char* b0 = (const char*)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

kda_status check_overlap(const std::vector<Span>& outs, const std::vector<Span>& ins) {
    for (size_t i = 0; i < outs.size(); ++i) {
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(KDA_ERR_OVERLAP, "outputs %s and %s overlap", outs[i].name, outs[j].name);
        for (const Span& s : ins)
            if (overlaps(outs[i], s))
                return fail(KDA_ERR_OVERLAP, "output %s overlaps %s", outs[i].name, s.name);
    }
    return KDA_OK;
}

std::vector<Span> input_spans(const Prob& p, const void* q, const void* k, const void* v,
                              const void* g, const void* beta, const float* A_log,
                              const float* dt_bias, const float* s0, const int64_t* cu) {
    const size_t tq = (size_t)p.tokens * p.Hqk * D * 2;
    const size_t tv = (size_t)p.tokens * p.Hv * D * 2;
    const size_t st = (size_t)p.N * p.Hv * kStateElems * 4;
    return {{q, tq, "q"}, {k, tq, "k"}, {v, tv, "v"}, {g, tv, "g"},
            {beta, (size_t)p.tokens * p.Hv * 2, "beta"}, {A_log, (size_t)p.Hv * 4, "A_log"},
            {dt_bias, (size_t)p.Hv * D * 4, "dt_bias"}, {s0, st, "initial_state"},
            {cu, cu ? (size_t)(p.N + 1) * 8 : 0, "cu_seqlens"}};
}

kda::FwdArgs make_fwd_args(const Prob& p, const kda::DevPlan& plan, const void* q, const void* k,
                           const void* v, const void* g, const void* beta, const float* A_log,
                           const float* dt_bias, const float* s0) {
    kda::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.A_log = A_log; a.dt_bias = dt_bias; a.s0 = s0;
    a.plan = plan;
    a.Hqk = p.Hqk; a.Hv = p.Hv; a.G = p.G;
    a.num_tasks = (int)p.num_tasks;
    a.ck_every = p.ck;
    a.scale = p.scale;
    // log2-domain decay sum above which a chunk runs precise: ln(exp(-2))
    a.rec_pairs = rec_pairs(p) ? 1 : 0;
    a.precise_log2 = p.precision == KDA_PRECISION_FULL   ? -INFINITY
                     : p.precision == KDA_PRECISION_FAST ? 1.0f
                                                         : -2.0f * 1.4426950408889634f;
    return a;
}

}  // namespace

extern "C" {

int kda_version(void) { return KDA_VERSION; }

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL_ARG: return "null argument";
        case KDA_ERR_SHAPE: return "bad shape";
        case KDA_ERR_GROUPING: return "Hv is not a multiple of Hqk";
        case KDA_ERR_SEQLENS: return "bad cu_seqlens";
        case KDA_ERR_SCALE: return "scale must be 1/sqrt(128)";
        case KDA_ERR_LOWER_BOUND: return "lower_bound must be -5";
        case KDA_ERR_OVERLAP: return "output overlaps another buffer";
        case KDA_ERR_CTX_SIZE: return "context too small";
        case KDA_ERR_CTX_MISMATCH: return "context does not match this call";
        case KDA_ERR_WORKSPACE_SIZE: return "workspace too small";
        case KDA_ERR_ROUTE: return "bad route or checkpoint interval";
        case KDA_ERR_HIP: return "HIP runtime error";
        case KDA_ERR_CAPTURE: return "schedule not ready for stream capture";
    }
    return "unknown status";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

kda_status kda_fwd_ctx_bytes(const kda_problem* pp, size_t* bytes) {
    Prob p;
    kda_status s = validate(pp, p);
    if (s != KDA_OK) return s;
    if (bytes == nullptr) return fail(KDA_ERR_NULL_ARG, "bytes is NULL");
    *bytes = ctx_bytes_for(p);
    return KDA_OK;
}

// Backward workspace: the rebuild's records (rec_layout), then BF16 dq/dk
// partials when value heads share a q/k head, then per-task parameter-gradient
// partials.
struct WsLayout {
    size_t s0, x, u, ta, dqk, par, seg_r, seg_e, total;
};
static WsLayout ws_layout(const Prob& p) {
    WsLayout w;
    // the rebuilt chunk records (none when the context already holds them)
    const size_t recs = p.ctxmode == KDA_CONTEXT_RECORDS ? 0 : (size_t)p.total_chunks * p.Hv;
    const RecLayout r = rec_layout(recs, 0, rec_pairs(p));
    w.s0 = r.s0;
    w.x = r.x;
    w.u = r.u;
    w.ta = r.ta;
    size_t off = r.end;
    w.dqk = off;
    if (p.G > 1) off = align256(off + (size_t)p.tokens * p.Hv * 2 * D * sizeof(uint16_t));
    w.par = off;
    // parameter partials per task, or per (segment, head) on the segment-parallel route
    const bool segs = p.route == 3 && p.ctxmode == KDA_CONTEXT_TAPE;
    const size_t slots = segs ? (size_t)std::max<int64_t>(p.num_tasks, p.total_segs * p.Hv) : (size_t)p.num_tasks;
    off = align256(off + slots * 2 * D * sizeof(float));
    // segment-parallel adjoint: R and the chained segment-end dS per (segment, head)
    w.seg_r = off;
    if (segs) off = align256(off + (size_t)p.total_segs * p.Hv * kStateElems * sizeof(float));
    w.seg_e = off;
    if (segs) off = align256(off + (size_t)p.total_segs * p.Hv * kStateElems * sizeof(float));
    w.total = off;
    return w;
}

kda_status kda_bwd_workspace_bytes(const kda_problem* pp, size_t* bytes) {
    Prob p;
    kda_status s = validate(pp, p);
    if (s != KDA_OK) return s;
    if (bytes == nullptr) return fail(KDA_ERR_NULL_ARG, "bytes is NULL");
    *bytes = ws_layout(p).total;
    return KDA_OK;
}

kda_status kda_plan_query(const kda_problem* pp, int32_t* route, int64_t* num_tasks,
                          int32_t* order, int64_t cap) {
    Prob p;
    kda_status s = validate(pp, p);
    if (s != KDA_OK) return s;
    if (route) *route = p.route;
    if (num_tasks) *num_tasks = p.num_tasks;
    if (order != nullptr && cap > 0) {
        std::vector<int32_t> o = lpt_order(p);
        std::memcpy(order, o.data(), sizeof(int32_t) * (size_t)std::min<int64_t>(cap, (int64_t)o.size()));
    }
    return KDA_OK;
}

}  // extern "C"

namespace {

// kda_fwd's checks, before any device access.
kda_status fwd_check(const kda_problem* pp, Prob& p, const void* q, const void* k, const void* v,
                     const void* g, const void* beta, const float* A_log, const float* dt_bias,
                     const float* initial_state, void* o, float* final_state, void* ctx,
                     size_t ctx_bytes) {
    kda_status s = validate(pp, p);
    if (s != KDA_OK) return s;
    if (!q || !k || !v || !g || !beta || !A_log || !dt_bias || !initial_state || !o || !final_state)
        return fail(KDA_ERR_NULL_ARG, "a tensor argument of kda_fwd is NULL");
    if (ctx != nullptr && ctx_bytes < ctx_bytes_for(p))
        return fail(KDA_ERR_CTX_SIZE, "context has %zu bytes, needs %zu", ctx_bytes, ctx_bytes_for(p));
    if (ctx == nullptr && ctx_bytes != 0)
        return fail(KDA_ERR_NULL_ARG, "ctx is NULL but ctx_bytes is %zu", ctx_bytes);
    std::vector<Span> ins = input_spans(p, q, k, v, g, beta, A_log, dt_bias, initial_state,
                                        pp->cu_seqlens);
    const size_t tv = (size_t)p.tokens * p.Hv * D * 2;
    const size_t st = (size_t)p.N * p.Hv * kStateElems * 4;
    std::vector<Span> outs = {{o, tv, "o"}, {final_state, st, "final_state"},
                              {ctx, ctx ? ctx_bytes : 0, "ctx"}};
    return check_overlap(outs, ins);
}

// The training forward's launches over a schedule at `plan_dev` (layout
// `lay`), and the host record of the context it fills.
kda_status fwd_launch(const Prob& p, int dev, const void* plan_dev, const PlanLayout& lay,
                      const void* q, const void* k, const void* v, const void* g,
                      const void* beta, const float* A_log, const float* dt_bias,
                      const float* initial_state, void* o, float* final_state, void* ctx,
                      size_t ctx_bytes, hipStream_t stream) {
    kda::FwdArgs a = make_fwd_args(p, dev_plan_at(plan_dev, lay), q, k, v, g, beta, A_log, dt_bias,
                                   initial_state);
    a.o = o;
    a.s_final = final_state;
    a.tape = nullptr;
    if (ctx != nullptr && p.ctxmode == KDA_CONTEXT_RECORDS) {
        const RecLayout r = rec_layout((size_t)p.total_chunks * p.Hv, 256, rec_pairs(p));
        a.rec_s0 = (kda::bf16_t*)((char*)ctx + r.s0);
        a.rec_x = (kda::bf16_t*)((char*)ctx + r.x);
        a.rec_u = (kda::bf16_t*)((char*)ctx + r.u);
        a.rec_ta = (float*)((char*)ctx + r.ta);
    } else if (ctx != nullptr) {
        a.tape = (float*)((char*)ctx + 256);
    }
    hipError_t e;
    if (p.route == 3 && ctx != nullptr) {
        // segment-parallel: segment tasks; P and Q in the context after the tape
        a.plan.task = (const int32_t*)((const char*)plan_dev + lay.off_seg);
        a.seg_out = (float*)((char*)ctx + seg_scratch_off(p));
        a.seg_items = p.total_segs * p.Hv;
        e = kda::launch_fwd_segments(a, p.N, stream);
    } else {
        // (without a context the segment-parallel route has no tape to chain
        // through: the plain chunked kernel runs)
        a.vsplit = p.route == 4;
        e = (p.route != 2) ? kda::launch_fwd_chunk(a, stream) : kda::launch_fwd_rowsplit(a, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    if (ctx != nullptr) {
        CtxRecord r;
        r.key = plan_key(p, dev);
        r.B = p.B; r.T = p.T; r.Hqk = p.Hqk; r.Hv = p.Hv; r.N = p.N; r.route = p.route;
        r.ctxmode = p.ctxmode;
        const void* ptrs[8] = {q, k, v, g, beta, A_log, dt_bias, initial_state};
        std::memcpy(r.ptrs, ptrs, sizeof(ptrs));
        r.stream = stream;
        r.ctx_bytes = ctx_bytes;
        std::lock_guard<std::mutex> lock(g_mu);
        r.seq = ++g_ctx_seq;
        if (g_ctx.size() >= kMaxCtx && g_ctx.find(ctx) == g_ctx.end()) {
            auto oldest = g_ctx.begin();
            for (auto it = g_ctx.begin(); it != g_ctx.end(); ++it)
                if (it->second.seq < oldest->second.seq) oldest = it;
            g_ctx.erase(oldest);
        }
        g_ctx[ctx] = r;
    }
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_fwd(const kda_problem* pp, const void* q, const void* k, const void* v,
                   const void* g, const void* beta, const float* A_log, const float* dt_bias,
                   const float* initial_state, void* o, float* final_state, void* ctx,
                   size_t ctx_bytes, void* stream_) {
    Prob p;
    kda_status s = fwd_check(pp, p, q, k, v, g, beta, A_log, dt_bias, initial_state, o, final_state,
                             ctx, ctx_bytes);
    if (s != KDA_OK) return s;
    hipStream_t stream = (hipStream_t)stream_;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    PlanLease lease;
    s = get_plan(p, stream, dev, lease);
    if (s != KDA_OK) return s;
    return fwd_launch(p, dev, lease.ent->dev, lease.ent->lay, q, k, v, g, beta, A_log, dt_bias,
                      initial_state, o, final_state, ctx, ctx_bytes, stream);
}

kda_status kda_fwd_noalloc(const kda_problem* pp, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, const float* A_log,
                           const float* dt_bias, const float* initial_state, void* o,
                           float* final_state, void* ctx, size_t ctx_bytes, void* stream_) {
    Prob p;
    kda_status s = fwd_check(pp, p, q, k, v, g, beta, A_log, dt_bias, initial_state, o, final_state,
                             ctx, ctx_bytes);
    if (s != KDA_OK) return s;
    const PlanLayout lay = plan_layout(p);
    if (lay.bytes > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
        return fail(KDA_ERR_WORKSPACE_SIZE,
                    "the schedule needs %zu bytes; the static scratch holds %zu "
                    "(use kda_fwd for this problem)", lay.bytes, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
    hipStream_t stream = (hipStream_t)stream_;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    void* scratch = nullptr;
    e = kda::noalloc_scratch(dev, &scratch);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    {
        // the schedule is built in a static host buffer (no heap allocation)
        // and handed over as kernel arguments, which the launch copies
        static unsigned char host[KDA_NOALLOC_SCRATCH_BYTES];
        static std::mutex host_mu;
        std::lock_guard<std::mutex> lock(host_mu);
        fill_plan(p, lay, (char*)host);
        e = kda::upload_to_scratch(scratch, host, lay.bytes, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "schedule upload launch");
    return fwd_launch(p, dev, scratch, lay, q, k, v, g, beta, A_log, dt_bias, initial_state, o,
                      final_state, ctx, ctx_bytes, stream);
}

kda_status kda_bwd(const kda_problem* pp, const void* q, const void* k, const void* v,
                   const void* g, const void* beta, const float* A_log, const float* dt_bias,
                   const float* initial_state, const void* ctx, size_t ctx_bytes,
                   const void* d_o, const float* dfinal_state, void* dq, void* dk, void* dv,
                   void* dg, void* dbeta, float* dA_log, float* ddt_bias, float* dinitial_state,
                   void* workspace, size_t workspace_bytes, void* stream_) {
    Prob p;
    kda_status s = validate(pp, p);
    if (s != KDA_OK) return s;
    if (!q || !k || !v || !g || !beta || !A_log || !dt_bias || !initial_state || !ctx || !d_o ||
        !dfinal_state || !dq || !dk || !dv || !dg || !dbeta || !dA_log || !ddt_bias ||
        !dinitial_state || !workspace)
        return fail(KDA_ERR_NULL_ARG, "a tensor argument of kda_bwd is NULL");
    if (ctx_bytes < ctx_bytes_for(p))
        return fail(KDA_ERR_CTX_SIZE, "context has %zu bytes, needs %zu", ctx_bytes, ctx_bytes_for(p));
    const WsLayout wl = ws_layout(p);
    const size_t need = wl.total;
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE_SIZE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    hipStream_t stream = (hipStream_t)stream_;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_ctx.find(ctx);
        if (it == g_ctx.end())
            return fail(KDA_ERR_CTX_MISMATCH, "context was not filled by kda_fwd");
        const CtxRecord& r = it->second;
        const void* ptrs[8] = {q, k, v, g, beta, A_log, dt_bias, initial_state};
        if (r.key != plan_key(p, dev) || r.B != p.B || r.T != p.T || r.Hqk != p.Hqk ||
            r.Hv != p.Hv || r.N != p.N || r.ctxmode != p.ctxmode)
            return fail(KDA_ERR_CTX_MISMATCH, "context was made for another shape or device");
        // every forward route leaves the same tape; the segment-parallel
        // backward also reads the transfer matrices P^T that only the
        // segment-parallel forward stores after it
        if (p.route == 3 && r.route != 3)
            return fail(KDA_ERR_CTX_MISMATCH, "context was filled on route %d, the backward resolves to %d "
                        "(segment-parallel), which needs that route's forward", r.route, p.route);
        if (std::memcmp(r.ptrs, ptrs, sizeof(ptrs)) != 0)
            return fail(KDA_ERR_CTX_MISMATCH, "inputs differ from the forward that made the context");
        if (r.stream != stream)
            return fail(KDA_ERR_CTX_MISMATCH, "context is used on another stream than its forward's");
    }
    std::vector<Span> ins = input_spans(p, q, k, v, g, beta, A_log, dt_bias, initial_state,
                                        pp->cu_seqlens);
    const size_t tq = (size_t)p.tokens * p.Hqk * D * 2;
    const size_t tv = (size_t)p.tokens * p.Hv * D * 2;
    const size_t st = (size_t)p.N * p.Hv * kStateElems * 4;
    ins.push_back({ctx, ctx_bytes, "ctx"});
    ins.push_back({d_o, tv, "do"});
    ins.push_back({dfinal_state, st, "dfinal_state"});
    std::vector<Span> outs = {{dq, tq, "dq"}, {dk, tq, "dk"}, {dv, tv, "dv"}, {dg, tv, "dg"},
                              {dbeta, (size_t)p.tokens * p.Hv * 2, "dbeta"},
                              {dA_log, (size_t)p.Hv * 4, "dA_log"},
                              {ddt_bias, (size_t)p.Hv * D * 4, "ddt_bias"},
                              {dinitial_state, st, "dinitial_state"},
                              {workspace, workspace_bytes, "workspace"}};
    s = check_overlap(outs, ins);
    if (s != KDA_OK) return s;

    PlanLease lease;
    s = get_plan(p, stream, dev, lease);
    if (s != KDA_OK) return s;
    const PlanEntry* plan = lease.ent;

    kda::BwdArgs b{};
    b.f = make_fwd_args(p, dev_plan(plan), q, k, v, g, beta, A_log, dt_bias, initial_state);
    char* ws = (char*)workspace;
    const bool records = p.ctxmode == KDA_CONTEXT_RECORDS;
    if (records) {  // the forward stored every chunk's records in the context
        const RecLayout r = rec_layout((size_t)p.total_chunks * p.Hv, 256, rec_pairs(p));
        b.f.rec_s0 = (kda::bf16_t*)((char*)ctx + r.s0);
        b.f.rec_x = (kda::bf16_t*)((char*)ctx + r.x);
        b.f.rec_u = (kda::bf16_t*)((char*)ctx + r.u);
        b.f.rec_ta = (float*)((char*)ctx + r.ta);
    } else {        // rebuilt from the tape into the workspace
        b.f.tape = (float*)((char*)ctx + 256);
        b.f.rec_s0 = (kda::bf16_t*)(ws + wl.s0);
        b.f.rec_x = (kda::bf16_t*)(ws + wl.x);
        b.f.rec_u = (kda::bf16_t*)(ws + wl.u);
        b.f.rec_ta = (float*)(ws + wl.ta);
    }
    b.d_o = d_o; b.dfinal = dfinal_state;
    b.dq = dq; b.dk = dk; b.dv = dv; b.dg = dg; b.dbeta = dbeta;
    b.dA_log = dA_log; b.ddt_bias = ddt_bias; b.dinit = dinitial_state;
    b.dqk_part = p.G > 1 ? (kda::bf16_t*)(ws + wl.dqk) : nullptr;
    b.dparam_part = (float*)(ws + wl.par);
    b.total_tokens = p.tokens;

    if (!records) {
        // segment list sits after the chunk offsets in the schedule
        kda::FwdArgs rb = b.f;
        rb.plan.task = (const int32_t*)((const char*)plan->dev + plan->lay.off_seg);
        e = kda::launch_state_rebuild(rb, p.total_segs * p.Hv, stream);
        if (e != hipSuccess) return hip_fail(e, "state rebuild launch");
    }
    int partial_rows = p.N;
    if (p.route == 3 && !records) {
        // segment-parallel adjoint over the tape segments, with the forward's P
        kda::BwdArgs bs = b;
        bs.f.plan.task = (const int32_t*)((const char*)plan->dev + plan->lay.off_seg);
        bs.f.seg_items = p.total_segs * p.Hv;
        bs.seg_p = (const float*)((const char*)ctx + seg_scratch_off(p) +
                                  2 * (size_t)p.total_segs * p.Hv * kStateElems * sizeof(float));  // P^T
        bs.seg_r = (float*)(ws + wl.seg_r);
        bs.seg_e = (float*)(ws + wl.seg_e);
        e = kda::launch_bwd_segments(bs, p.N, stream);
        partial_rows = (int)p.total_segs;  // partials per (segment, head)
    } else {
        e = kda::launch_bwd_chunk(b, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    e = kda::launch_bwd_reduce(b, partial_rows, stream);
    if (e != hipSuccess) return hip_fail(e, "backward reduction launch");
    return KDA_OK;
}

kda_status kda_infer(const kda_infer_problem* ip, const void* q, const void* k, const void* v,
                     const void* g, const void* beta, const float* A_log, const float* dt_bias,
                     void* state_pool, void* o, void* stream_) {
    if (ip == nullptr) return fail(KDA_ERR_NULL_ARG, "problem is NULL");
    // shape, grouping and sequence checks are the training forward's
    kda_problem tp{};
    tp.B = ip->B; tp.T = ip->T; tp.Hqk = ip->Hqk; tp.Hv = ip->Hv; tp.N = ip->N;
    tp.cu_seqlens = ip->cu_seqlens;
    tp.cu_seqlens_host = ip->cu_seqlens_host;
    tp.scale = 0.0f;
    tp.lower_bound = -5.0f;
    tp.route = KDA_ROUTE_ROWSPLIT;
    tp.checkpoint_every = 0;
    tp.context = KDA_CONTEXT_TAPE;
    Prob p;
    kda_status s = validate(&tp, p);
    if (s != KDA_OK) return s;
    float scale = ip->scale == 0.0f ? 1.0f / std::sqrt(128.0f) : ip->scale;
    if (!(scale > 0.0f) || !std::isfinite(scale))
        return fail(KDA_ERR_SCALE, "scale must be 0 or finite and positive (got %g)", (double)ip->scale);
    for (int32_t f : {ip->use_qk_l2norm, ip->use_gate_in_kernel, ip->beta_is_logit})
        if (f != 0 && f != 1) return fail(KDA_ERR_SHAPE, "option flags must be 0 or 1 (got %d)", f);
    if (ip->route < 0 || ip->route > 2) return fail(KDA_ERR_ROUTE, "unknown route %d", ip->route);
    // the chunk factors exp(+-gc) need every per-token log-decay >= -5: true
    // for the in-kernel gate with such a lower bound, unknown for a log-space
    // gate given as is (the host never reads g), which therefore runs token by
    // token
    const bool bounded_gate = ip->use_gate_in_kernel && ip->lower_bound >= -5.0f;
    if (ip->route == KDA_ROUTE_CHUNK && !ip->use_gate_in_kernel)
        return fail(KDA_ERR_ROUTE,
                    "the chunked route needs the in-kernel gate (a log-space gate is not bounded below)");
    if (ip->route == KDA_ROUTE_CHUNK && !bounded_gate)
        return fail(KDA_ERR_ROUTE, "the chunked route needs lower_bound >= -5 (got %g)",
                    (double)ip->lower_bound);
    if (ip->use_gate_in_kernel) {
        if (!(ip->lower_bound < 0.0f) || !std::isfinite(ip->lower_bound))
            return fail(KDA_ERR_LOWER_BOUND,
                        "the in-kernel gate needs a finite negative lower_bound (got %g); the "
                        "softplus form is not implemented", (double)ip->lower_bound);
        if (A_log == nullptr) return fail(KDA_ERR_NULL_ARG, "the in-kernel gate needs A_log");
    }
    if (!q || !k || !v || !g || !beta || !state_pool || !o)
        return fail(KDA_ERR_NULL_ARG, "a tensor argument of kda_infer is NULL");
    if (ip->pool_slots < 1 || ip->pool_slots > ((int64_t)1 << 40) / ((int64_t)p.Hv * kStateElems))
        return fail(KDA_ERR_SHAPE, "pool_slots out of range (%lld)", (long long)ip->pool_slots);
    if ((ip->state_indices == nullptr) != (ip->state_indices_host == nullptr))
        return fail(KDA_ERR_NULL_ARG, "state_indices and state_indices_host go together");
    // speculative decode: 1+S tokens and 1+S slots per sequence
    const int S = ip->num_spec_tokens;
    if (S < 0) return fail(KDA_ERR_SHAPE, "num_spec_tokens must be >= 0 (got %d)", S);
    if (S == 0 && ip->num_accepted_tokens != nullptr)
        return fail(KDA_ERR_SHAPE, "num_accepted_tokens needs num_spec_tokens > 0");
    if (S > 0) {
        if (ip->state_indices == nullptr)
            return fail(KDA_ERR_NULL_ARG, "speculative decode needs state_indices [N][1+S]");
        if (ip->checkpoint_every != 0)
            return fail(KDA_ERR_ROUTE, "speculative decode takes no state checkpoints");
        if (ip->route == KDA_ROUTE_CHUNK)
            return fail(KDA_ERR_ROUTE, "speculative decode runs on the token-serial route");
        for (int n = 0; n < p.N; ++n)
            if (p.len[n] != 1 + S)
                return fail(KDA_ERR_SEQLENS, "sequence %d has %lld tokens; speculative decode needs 1+S=%d",
                            n, (long long)p.len[n], 1 + S);
    }
    const int64_t n_idx = (int64_t)p.N * (1 + S);
    if (ip->state_indices_host != nullptr) {
        std::vector<int32_t> sorted(ip->state_indices_host, ip->state_indices_host + n_idx);
        for (int64_t i = 0; i < n_idx; ++i) {
            const int32_t slot = sorted[i];
            if (slot < 0 || slot >= ip->pool_slots)
                return fail(KDA_ERR_SHAPE, "state_indices[%lld] = %d is outside the pool", (long long)i, slot);
        }
        std::sort(sorted.begin(), sorted.end());
        for (int64_t i = 1; i < n_idx; ++i)
            if (sorted[i] == sorted[i - 1])
                return fail(KDA_ERR_SHAPE, "pool slot %d is named twice", sorted[i]);
    } else if (ip->pool_slots < p.N) {
        return fail(KDA_ERR_SHAPE, "without state_indices the pool needs N=%d slots (has %lld)", p.N,
                    (long long)ip->pool_slots);
    }
    // read-only source pool
    if ((ip->state_source == nullptr) != (ip->source_indices == nullptr) ||
        (ip->source_indices == nullptr) != (ip->source_indices_host == nullptr))
        return fail(KDA_ERR_NULL_ARG, "state_source, source_indices and its host mirror go together");
    if (ip->state_source != nullptr) {
        if (ip->source_slots < 1 ||
            ip->source_slots > ((int64_t)1 << 40) / ((int64_t)p.Hv * kStateElems))
            return fail(KDA_ERR_SHAPE, "source_slots out of range (%lld)", (long long)ip->source_slots);
        for (int n = 0; n < p.N; ++n)
            if (ip->source_indices_host[n] < 0 || ip->source_indices_host[n] >= ip->source_slots)
                return fail(KDA_ERR_SHAPE, "source_indices[%d] = %d is outside the source pool", n,
                            ip->source_indices_host[n]);
    }
    const size_t tq = (size_t)p.tokens * p.Hqk * D * 2;
    const size_t tv = (size_t)p.tokens * p.Hv * D * 2;
    std::vector<Span> ins = {{q, tq, "q"}, {k, tq, "k"}, {v, tv, "v"}, {g, tv, "g"},
                             {beta, (size_t)p.tokens * p.Hv * 2, "beta"},
                             {A_log, A_log ? (size_t)p.Hv * 4 : 0, "A_log"},
                             {dt_bias, dt_bias ? (size_t)p.Hv * D * 4 : 0, "dt_bias"},
                             {ip->cu_seqlens, ip->cu_seqlens ? (size_t)(p.N + 1) * 8 : 0, "cu_seqlens"},
                             {ip->state_indices, ip->state_indices ? (size_t)n_idx * 4 : 0,
                              "state_indices"},
                             {ip->num_accepted_tokens, ip->num_accepted_tokens ? (size_t)p.N * 4 : 0,
                              "num_accepted_tokens"},
                             {ip->state_source,
                              ip->state_source ? (size_t)ip->source_slots * p.Hv * kStateElems * 2 : 0,
                              "state_source"},
                             {ip->source_indices, ip->source_indices ? (size_t)p.N * 4 : 0,
                              "source_indices"}};
    // state checkpoints
    const int E = ip->checkpoint_every;
    if (E == 0) {
        if (ip->state_checkpoints || ip->checkpoint_rows || ip->checkpoint_cu_starts ||
            ip->checkpoint_cu_starts_host)
            return fail(KDA_ERR_ROUTE, "checkpoint fields given with checkpoint_every = 0");
    } else {
        if (E < 0 || E % kChunk != 0)
            return fail(KDA_ERR_ROUTE, "checkpoint_every must be a positive multiple of 16 (got %d)", E);
        if (!ip->state_checkpoints || !ip->checkpoint_cu_starts || !ip->checkpoint_cu_starts_host)
            return fail(KDA_ERR_NULL_ARG, "checkpoints need state_checkpoints and both start arrays");
        if (ip->checkpoint_rows < 1 ||
            ip->checkpoint_rows > ((int64_t)1 << 40) / ((int64_t)p.Hv * kStateElems))
            return fail(KDA_ERR_SHAPE, "checkpoint_rows out of range (%lld)", (long long)ip->checkpoint_rows);
        const int64_t* cs = ip->checkpoint_cu_starts_host;
        if (cs[0] != 0) return fail(KDA_ERR_SEQLENS, "checkpoint_cu_starts must start at 0");
        for (int n = 0; n < p.N; ++n)
            if (cs[n + 1] - cs[n] != (p.len[n] + E - 1) / E)
                return fail(KDA_ERR_SEQLENS, "sequence %d needs %lld checkpoint rows (starts give %lld)", n,
                            (long long)((p.len[n] + E - 1) / E), (long long)(cs[n + 1] - cs[n]));
        if (cs[p.N] > ip->checkpoint_rows)
            return fail(KDA_ERR_SHAPE, "checkpoints need %lld rows (have %lld)", (long long)cs[p.N],
                        (long long)ip->checkpoint_rows);
        ins.push_back({ip->checkpoint_cu_starts, (size_t)(p.N + 1) * 8, "checkpoint_cu_starts"});
    }
    const size_t pool_bytes = (size_t)ip->pool_slots * p.Hv * kStateElems * 2;
    const size_t ck_bytes = E ? (size_t)ip->checkpoint_rows * p.Hv * kStateElems * 2 : 0;
    std::vector<Span> outs = {{o, tv, "o"}, {state_pool, pool_bytes, "state_pool"},
                              {ip->state_checkpoints, ck_bytes, "state_checkpoints"}};
    s = check_overlap(outs, ins);
    if (s != KDA_OK) return s;

    hipStream_t stream = (hipStream_t)stream_;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    PlanLease lease;
    s = get_plan(p, stream, dev, lease);
    if (s != KDA_OK) return s;
    const PlanEntry* plan = lease.ent;
    kda::FwdArgs a = make_fwd_args(p, dev_plan(plan), q, k, v, g, beta, A_log, dt_bias, nullptr);
    const int64_t longest = *std::max_element(p.len.begin(), p.len.end());
    const int route = ip->route != KDA_ROUTE_AUTO ? ip->route
                      : (bounded_gate && longest > 1 && S == 0) ? KDA_ROUTE_CHUNK : KDA_ROUTE_ROWSPLIT;
    a.o = o;
    a.scale = scale;
    a.infer = 1;
    a.use_qk_l2norm = ip->use_qk_l2norm;
    a.use_gate_in_kernel = ip->use_gate_in_kernel;
    a.beta_is_logit = ip->beta_is_logit;
    a.lower_bound = ip->lower_bound;
    a.pool = (kda::bf16_t*)state_pool;
    a.pool_index = ip->state_indices;
    a.pool_slots = ip->pool_slots;
    a.ckpt = E ? (kda::bf16_t*)ip->state_checkpoints : nullptr;
    a.ckpt_start = ip->checkpoint_cu_starts;
    a.ckpt_rows = E ? ip->checkpoint_rows : 0;
    a.ckpt_every = E ? E : 1;
    a.spec_tokens = S;
    a.spec_accepted = ip->num_accepted_tokens;
    a.src_pool = (const kda::bf16_t*)ip->state_source;
    a.src_index = ip->source_indices;
    a.src_slots = ip->source_slots;
    e = route == KDA_ROUTE_CHUNK ? kda::launch_fwd_chunk(a, stream) : kda::launch_infer_token(a, stream);
    if (e != hipSuccess) return hip_fail(e, "inference launch");
    return KDA_OK;
}

}  // extern "C"
