// Host side of the LAGS-SGD library: argument validation, per-layer planning,
// workspace sizing, device tables, kernel launches and kernel tracing.
// The entry points are declared in include/lags.h.
#include "lags.h"
#include "lags_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

using namespace lags;

static_assert(kStaticScratchBytes == LAGS_STATIC_SCRATCH_BYTES, "one size for the static scratch");

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The aggregate's chunk plan for up to P workers: chunk widths per layer and
// the host image of its device tables (copied into a workspace by
// lags_workspace_init).
struct AggPlan {
    uint32_t NC = 0;
    uint32_t tl = kAggTableLog2;      // log2 of the aggregate's LDS hash slots
    bool dense = false;               // the layout has a layer that sends every entry
    std::vector<uint32_t> h_cbase;    // [L+1]
    size_t b_cbase = 0, b_csh = 0, b_info = 0, b_desc = 0;   // byte offsets inside the image
    std::vector<unsigned char> image; // cbase[L+1], csh[L], chunk_info[NC], sdesc[npb][2]
};

// A workspace that lags_workspace_init prepared for this layout.
struct WsRec {
    const void *ws;
    size_t bytes;
    int32_t P;
    int device;
};

struct TraceRec {
    int32_t kid;
    hipEvent_t a, b;
};

}  // namespace

struct lags_layout {
    uint64_t id = 0;               // unique per created layout
    int32_t L = 0;
    uint64_t n = 0, K = 0;
    std::vector<uint32_t> off, k, moff;
    std::vector<LayerInfo> linfo;
    std::vector<SampledInfo> sinfo;
    std::vector<MainWork> main_work;
    std::vector<LayerInfo> small_info;   // copies of the small layers' entries
    std::vector<FinWork> fin_work;
    std::vector<uint32_t> pos_layer;
    uint32_t starts_tl = 0;        // LDS table entries the start pass needs (one block per workgroup)
    uint32_t starts_tl4 = 0;       // ... four blocks per workgroup
    // per-layer prefix counts of the work lists, for layer-range launches:
    // small-layer work entries, streaming work entries, sampled layers and
    // finishing workgroups before layer l
    std::vector<uint32_t> small_pre, stream_pre, sid_pre, fin_pre;
    std::vector<uint32_t> bins_pre;   // sampled layers that need k_fin_bins (many histogram copies)
    uint32_t nseg_total = 0;
    uint64_t slots_total = 0;
    uint64_t hist_words = 0;
    // host image of the layer tables (the head of every workspace) and the
    // byte offsets of its parts
    std::vector<unsigned char> tables;
    size_t tb_linfo = 0, tb_sinfo = 0, tb_main = 0, tb_fin = 0, tb_moff = 0, tb_pos = 0,
           tb_small = 0;
    // workspace plan (byte offsets; the P-dependent part starts at ws_agg)
    size_t ws_report = 0, ws_state = 0, ws_hist = 0, ws_segcount = 0, ws_segsel = 0,
           ws_slots = 0, ws_tbin = 0, ws_fintot = 0, ws_fineq = 0, ws_fb = 0, ws_agg = 0;
    std::mutex mu;
    std::map<int32_t, AggPlan> agg;     // chunk plans by worker count
    std::vector<WsRec> wss;             // initialised workspaces
    // tracing
    bool trace = false;
    std::vector<TraceRec> recs;
    double tr_ms[kNumKernels] = {};
    int64_t tr_n[kNumKernels] = {};
};

namespace {

// Chunk widths of the aggregate for P workers: per layer, a power of two (at
// most 2^kAggMaxWidthLog2) such that a chunk holds about 2^(tl-2) message
// entries over all workers; 2^kAggDenseLog2 for a layer that sends every
// entry (k = n).
void plan_agg(const lags_layout *lo, int32_t P, uint32_t tl, std::vector<uint32_t> &cbase,
              std::vector<uint32_t> &csh, uint32_t &NC)
{
    cbase.assign(lo->L + 1, 0);
    csh.assign(lo->L, 0);
    uint64_t total = 0;
    const double target = std::ldexp(1.0, (int)tl - 2);
    for (int32_t l = 0; l < lo->L; ++l) {
        const double nl = lo->linfo[l].n, kl = lo->linfo[l].k;
        const double width = target * nl / ((double)P * kl);
        int s = 0;
        while (s < (int)kAggMaxWidthLog2 && std::ldexp(1.0, s + 1) <= width) ++s;
        // a layer that sends every entry: one index per thread of a chunk
        if (lo->linfo[l].k == lo->linfo[l].n) s = kAggDenseLog2;
        csh[l] = (uint32_t)s;
        cbase[l] = (uint32_t)total;
        total += ((uint64_t)lo->linfo[l].n + (1ull << s) - 1) >> s;
    }
    cbase[lo->L] = (uint32_t)total;
    NC = (uint32_t)total;
}

// Threshold-guess plan for a sampled layer of n entries sending k: sample s
// keys and take the j-th largest, with j = m * k * s / n and the margin m the
// smallest that keeps (1 - 1/m) * sqrt(j) >= 6 (six standard deviations of the
// sample count above the guess).  When that rank is beyond the sample (k
// close to n), j = s asks for the guess G = 0: every nonzero entry is a
// candidate.
void plan_guess(uint32_t n, uint32_t k, uint32_t s, uint32_t &j, double &m)
{
    const double lam = (double)k * (double)s / (double)n;
    m = 1.05;
    while (m < 1e6 && (1.0 - 1.0 / m) * std::sqrt(m * lam) < 6.0) m *= 1.05;
    const double jj = std::ceil(m * lam);
    j = (uint32_t)std::min<double>(std::max(1.0, jj), (double)s);
}

int build_plan(lags_layout *lo)
{
    const int32_t L = lo->L;
    lo->linfo.resize(L);
    uint32_t seg_base = 0;
    uint64_t slot_base = 0;
    std::vector<MainWork> stream_work;
    lo->small_pre.assign(L + 1, 0);
    lo->stream_pre.assign(L + 1, 0);
    lo->sid_pre.assign(L + 1, 0);
    lo->fin_pre.assign(L + 1, 0);
    lo->bins_pre.assign(L + 1, 0);
    uint32_t nbig = 0;
    auto work = [](uint32_t l, uint32_t cls, uint32_t tile) {
        MainWork w{};
        w.layer = l;
        w.cls = cls;
        w.tile = tile;
        return w;
    };
    for (int32_t l = 0; l < L; ++l) {
        lo->small_pre[l] = (uint32_t)lo->small_info.size();
        lo->stream_pre[l] = (uint32_t)stream_work.size();
        lo->sid_pre[l] = (uint32_t)lo->sinfo.size();
        lo->fin_pre[l] = (uint32_t)lo->fin_work.size();
        lo->bins_pre[l] = nbig;
        LayerInfo &li = lo->linfo[l];
        li = LayerInfo{};
        li.off = lo->off[l];
        li.n = lo->off[l + 1] - lo->off[l];
        li.k = lo->k[l];
        li.moff = lo->moff[l];
        li.sid = 0xffffffffu;
        if (li.n <= kSmallMax) {
            li.cls = kClsSmall;
            li.ntiles = 1;
            lo->small_info.push_back(li);
        } else if (li.k == li.n) {
            li.cls = kClsDense;
            li.ntiles = (li.n + kDenseTile - 1) / kDenseTile;
            for (uint32_t t = 0; t < li.ntiles; ++t) stream_work.push_back(work((uint32_t)l, kClsDense, t));
        } else {
            li.cls = kClsSampled;
            li.sid = (uint32_t)lo->sinfo.size();
            SampledInfo si{};
            si.layer = (uint32_t)l;
            si.a4 = (li.off + 3u) & ~3u;
            si.b4 = (li.off + li.n) & ~3u;
            si.nseg = (si.b4 - si.a4 + kSeg - 1) / kSeg;
            si.seg_base = seg_base;
            double m = 1.0;
            if (li.n <= kSampleMax) {
                si.full_sample = 1;
                si.j = li.k;
                si.cap = kSeg;
            } else {
                si.nchunk = kSampleMax / kSampleChunk;
                uint32_t j = 0;
                plan_guess(li.n, li.k, si.nchunk * kSampleChunk, j, m);
                si.j = j;
                // slots for the expected candidates plus eight standard
                // deviations; a segment beyond them is re-read instead
                const double mu = std::min(m * (double)li.k, (double)li.n) * kSeg / (double)li.n;
                size_t cap = (size_t)std::ceil(mu + 8.0 * std::sqrt(mu) + 32.0);
                cap = align_up(cap, 32);
                si.cap = (uint32_t)std::min<size_t>(cap, kCapMax);
            }
            si.slot_lo = (uint32_t)(slot_base & 0xffffffffu);
            si.slot_hi = (uint32_t)(slot_base >> 32);
            const uint32_t grain = fin_grain(si.nseg);
            si.fin_nblocks = (si.nseg + grain - 1) / grain;
            // every candidate the layer can store fits its threshold-bin list,
            // so a large bin (many equal keys) never forces the exact path
            si.tbin_cap = (uint32_t)std::min<uint64_t>((uint64_t)si.nseg * si.cap, 0xffffffffu);
            si.fin_first = (uint32_t)lo->fin_work.size();
            si.off = li.off;
            si.n = li.n;
            si.k = li.k;
            si.moff = li.moff;
            si.grain = grain;
            li.ntiles = (si.nseg + kTileSegs - 1) / kTileSegs;
            // histogram copies grow with the layer, so that the streaming
            // workgroups' atomics on its hottest bins stay spread
            si.hcopies = 1;
            while (si.hcopies < kHistMaxCopies && si.hcopies * kTilesPerCopy < li.ntiles) si.hcopies *= 2;
            si.hist_off = (uint32_t)lo->hist_words;
            if (si.hcopies > kSelfBinsCopies) ++nbig;
            lo->hist_words += (uint64_t)si.hcopies * kNBins;
            for (uint32_t t = 0; t < li.ntiles; ++t) {
                MainWork w = work((uint32_t)l, kClsSampled, t);
                w.sid = li.sid;
                w.off = li.off;
                w.end = li.off + li.n;
                w.a4 = si.a4;
                w.b4 = si.b4;
                w.nseg = si.nseg;
                w.seg_base = si.seg_base;
                w.cap = si.cap;
                w.slot_lo = si.slot_lo;
                w.slot_hi = si.slot_hi;
                w.hist_off = si.hist_off;
                w.hcopies = si.hcopies;
                stream_work.push_back(w);
            }
            for (uint32_t b = 0; b < si.fin_nblocks; ++b) {
                FinWork f{};
                f.sid = li.sid;
                f.seg0 = b * grain;
                f.grain = grain;
                f.nseg = si.nseg;
                f.seg_base = si.seg_base;
                f.cap = si.cap;
                f.slot_lo = si.slot_lo;
                f.slot_hi = si.slot_hi;
                f.fin_first = si.fin_first;
                f.off = li.off;
                f.n = li.n;
                f.moff = li.moff;
                f.k = li.k;
                f.tbin_cap = si.tbin_cap;
                f.a4 = si.a4;
                f.hist_off = si.hist_off;
                f.hcopies = si.hcopies;
                lo->fin_work.push_back(f);
            }
            seg_base += si.nseg;
            slot_base += (uint64_t)si.nseg * si.cap;
            lo->sinfo.push_back(si);
        }
    }
    lo->small_pre[L] = (uint32_t)lo->small_info.size();
    lo->stream_pre[L] = (uint32_t)stream_work.size();
    lo->sid_pre[L] = (uint32_t)lo->sinfo.size();
    lo->fin_pre[L] = (uint32_t)lo->fin_work.size();
    lo->bins_pre[L] = nbig;
    lo->main_work = stream_work;
    lo->nseg_total = seg_base;
    lo->slots_total = slot_base;
    // layer of every kStartsBlock-th message position (the aggregate's start pass)
    const uint64_t npb = (lo->K + 1 + kStartsBlock - 1) / kStartsBlock;
    lo->pos_layer.resize(npb);
    for (uint64_t b = 0, l = 0; b < npb; ++b) {
        const uint64_t j = b * kStartsBlock;
        while (l + 1 < (uint64_t)L && lo->moff[l + 1] <= j) ++l;
        lo->pos_layer[b] = (uint32_t)l;
    }
    // the start pass stages the layers of a block in LDS: from the layer
    // before the block's first to the layer of the next block's first
    // position, and one more moff entry
    lo->starts_tl = 0;
    lo->starts_tl4 = 0;
    for (uint64_t b = 0; b < npb; ++b) {
        const uint32_t l0 = lo->pos_layer[b];
        const uint32_t la = l0 > 0 ? l0 - 1 : 0;
        const uint32_t l1 = (b + 1 < npb) ? lo->pos_layer[b + 1] : (uint32_t)L - 1;
        const uint32_t l4 = (b + 4 < npb) ? lo->pos_layer[b + 4] : (uint32_t)L - 1;
        lo->starts_tl = std::max(lo->starts_tl, l1 - la + 2);
        lo->starts_tl4 = std::max(lo->starts_tl4, l4 - la + 2);
    }

    // the layer tables: a host image, copied to the head of a workspace by
    // lags_workspace_init
    size_t at = 0;
    auto part = [&](size_t bytes) {
        const size_t o = at;
        at = align_up(at + std::max<size_t>(bytes, 4), kAlign);
        return o;
    };
    lo->tb_linfo = part(lo->linfo.size() * sizeof(LayerInfo));
    lo->tb_sinfo = part(lo->sinfo.size() * sizeof(SampledInfo));
    lo->tb_main = part(lo->main_work.size() * sizeof(MainWork));
    lo->tb_fin = part(lo->fin_work.size() * sizeof(FinWork));
    lo->tb_moff = part(lo->moff.size() * 4);
    lo->tb_pos = part(lo->pos_layer.size() * 4);
    lo->tb_small = part(lo->small_info.size() * sizeof(LayerInfo));
    lo->tables.assign(at, 0);
    unsigned char *h = lo->tables.data();
    auto put = [&](size_t o, const void *src, size_t bytes) {
        if (bytes) std::memcpy(h + o, src, bytes);
    };
    put(lo->tb_linfo, lo->linfo.data(), lo->linfo.size() * sizeof(LayerInfo));
    put(lo->tb_sinfo, lo->sinfo.data(), lo->sinfo.size() * sizeof(SampledInfo));
    put(lo->tb_main, lo->main_work.data(), lo->main_work.size() * sizeof(MainWork));
    put(lo->tb_fin, lo->fin_work.data(), lo->fin_work.size() * sizeof(FinWork));
    put(lo->tb_moff, lo->moff.data(), lo->moff.size() * 4);
    put(lo->tb_pos, lo->pos_layer.data(), lo->pos_layer.size() * 4);
    put(lo->tb_small, lo->small_info.data(), lo->small_info.size() * sizeof(LayerInfo));

    // scratch: never read before being written in a call
    const size_t ns = lo->sinfo.size();
    lo->ws_report = at;
    at = align_up(at + kRepWords * 4, kAlign);
    lo->ws_state = at;
    at = align_up(at + ns * sizeof(SampledState), kAlign);
    lo->ws_hist = at;
    at = align_up(at + (size_t)lo->hist_words * 4, kAlign);
    lo->ws_segcount = at;
    at = align_up(at + (size_t)lo->nseg_total * 4, kAlign);
    lo->ws_segsel = at;
    at = align_up(at + (size_t)lo->nseg_total * 4, kAlign);
    lo->ws_slots = at;
    at = align_up(at + (size_t)lo->slots_total * 8, kAlign);
    lo->ws_tbin = at;
    at = align_up(at + (size_t)lo->slots_total * 8, kAlign);   // same offsets as the slots
    lo->ws_fintot = at;
    at = align_up(at + lo->fin_work.size() * 4, kAlign);
    lo->ws_fineq = at;
    at = align_up(at + lo->fin_work.size() * 4, kAlign);
    lo->ws_fb = at;
    at = align_up(at + ns * (size_t)kFbWords * 4, kAlign);
    lo->ws_agg = at;
    return LAGS_OK;
}

// The chunk plan for up to P workers (caller holds lo->mu, or the layout is
// not shared yet).  The image holds cbase, csh and, per chunk, its index range
// and its layer's message range, so that an aggregate workgroup needs one load
// to start.
const AggPlan &agg_plan(lags_layout *lo, int32_t P)
{
    auto it = lo->agg.find(P);
    if (it != lo->agg.end()) return it->second;
    AggPlan t;
    t.tl = (uint64_t)P * lo->K >= kAggWideEntries ? kAggTableLog2Wide : kAggTableLog2;
    std::vector<uint32_t> cb, cs;
    plan_agg(lo, P, t.tl, cb, cs, t.NC);
    std::vector<uint4> ci(std::max<uint32_t>(t.NC, 1), uint4{0, 0, 0, 0});
    for (int32_t l = 0; l < lo->L; ++l) {
        const uint64_t off = lo->off[l], end = lo->off[l + 1];
        const bool dense = lo->k[l] == end - off;
        t.dense = t.dense || dense;
        for (uint32_t c = cb[l]; c < cb[l + 1]; ++c) {
            const uint64_t clo = off + ((uint64_t)(c - cb[l]) << cs[l]);
            const uint64_t chi = std::min<uint64_t>(clo + ((uint64_t)1 << cs[l]), end);
            // a k = n layer's chunk: where index clo sits in every valid
            // message, and the marker kAggDenseChunk (no message range ends there)
            ci[c] = dense ? uint4{(uint32_t)clo, (uint32_t)chi, (uint32_t)(lo->moff[l] + (clo - off)), kAggDenseChunk}
                          : uint4{(uint32_t)clo, (uint32_t)chi, (uint32_t)lo->moff[l],
                                  (uint32_t)(lo->moff[l] + lo->k[l])};
        }
    }
    // per position block of the start pass: the layers of its first
    // position's predecessor and of its last position, and the first one's
    // fields (a block inside one layer needs nothing else)
    const size_t npb = lo->pos_layer.size();
    std::vector<uint4> sd(2 * npb, uint4{0, 0, 0, 0});
    auto layer_at = [&](uint64_t j) -> uint32_t {   // largest l with moff[l] <= j
        return (uint32_t)(std::upper_bound(lo->moff.begin(), lo->moff.begin() + lo->L, (uint32_t)j) -
                          lo->moff.begin()) - 1u;
    };
    for (size_t b = 0; b < npb; ++b) {
        const uint64_t jfirst = b * kStartsBlock;
        const uint64_t jlast = std::min<uint64_t>(jfirst + kStartsBlock, lo->K) - 1;
        const uint32_t l0 = layer_at(jfirst ? jfirst - 1 : 0);
        const uint32_t l1 = layer_at(std::max<uint64_t>(jlast, jfirst ? jfirst - 1 : 0));
        sd[2 * b] = uint4{l0, l1, lo->off[l0], lo->off[l0 + 1] - lo->off[l0]};
        sd[2 * b + 1] = uint4{cb[l0], cs[l0], 0, 0};
    }
    t.b_cbase = 0;
    t.b_csh = align_up(cb.size() * 4, kAlign);
    t.b_info = t.b_csh + align_up(cs.size() * 4, kAlign);
    t.b_desc = t.b_info + align_up(ci.size() * sizeof(uint4), kAlign);
    t.image.assign(t.b_desc + align_up(sd.size() * sizeof(uint4), kAlign), 0);
    std::memcpy(t.image.data() + t.b_cbase, cb.data(), cb.size() * 4);
    std::memcpy(t.image.data() + t.b_csh, cs.data(), cs.size() * 4);
    std::memcpy(t.image.data() + t.b_info, ci.data(), ci.size() * sizeof(uint4));
    std::memcpy(t.image.data() + t.b_desc, sd.data(), sd.size() * sizeof(uint4));
    t.h_cbase = std::move(cb);
    return lo->agg.emplace(P, std::move(t)).first->second;
}

// Bytes of the P-dependent tail of a workspace: the chunk-start table
// [P][NC+1], then the chunk tables.
size_t agg_tail_bytes(const AggPlan &t, int32_t P)
{
    return align_up((size_t)P * ((size_t)t.NC + 1) * 4, kAlign) + t.image.size();
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The record of an initialised workspace, or null (caller holds lo->mu).
const WsRec *find_ws(const lags_layout *lo, const void *ws)
{
    for (const WsRec &r : lo->wss)
        if (r.ws == ws) return &r;
    return nullptr;
}

// Launch with optional tracing events around it.
template <class F>
int traced(lags_layout *lo, int32_t kid, hipStream_t s, F &&launch)
{
    hipEvent_t a = nullptr, b = nullptr;
    if (lo->trace) {
        if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return LAGS_EHIP;
        if (hipEventRecord(a, s) != hipSuccess) return LAGS_EHIP;
    }
    if (launch() != hipSuccess) return LAGS_EHIP;
    if (lo->trace) {
        if (hipEventRecord(b, s) != hipSuccess) return LAGS_EHIP;
        lo->recs.push_back(TraceRec{kid, a, b});
    }
    return LAGS_OK;
}

// Exact mode: a multi-workgroup radix select of every sampled layer's
// threshold (three digit passes, each followed by a per-layer pick), the
// per-segment counts, tie cut and message offsets, then the sampled path's
// emission (from the entries >= T that k_x_count kept in the slots); every
// pass over a layer runs on the main work list (one workgroup per segment).
// Small layers as always.  k_sample has cleared the layers' state and
// histogram copies.
int sparsify_exact(lags_layout *lo, const SparsifyArgs &a, uint32_t ns, uint32_t nmain, uint32_t nfin,
                   hipStream_t s)
{
    int rc;
    if (nmain) {
        rc = traced(lo, kKXFirst, s, [&] { return launch_x_first(a, nmain, s); });
        if (rc != LAGS_OK) return rc;
    }
    for (uint32_t level = 0; ns && level < 3; ++level) {
        if (level > 0) {
            rc = traced(lo, kKXPass, s, [&] { return launch_x_pass(a, nmain, level, s); });
            if (rc != LAGS_OK) return rc;
        }
        rc = traced(lo, kKXPick, s, [&] { return launch_x_pick(a, ns, level, s); });
        if (rc != LAGS_OK) return rc;
    }
    if (ns) {
        rc = traced(lo, kKXCount, s, [&] { return launch_x_count(a, nmain, s); });
        if (rc != LAGS_OK) return rc;
        rc = traced(lo, kKXCut, s, [&] { return launch_x_cut(a, ns, s); });
        if (rc != LAGS_OK) return rc;
    }
    if (a.nsmall) {
        SparsifyArgs b = a;
        b.nsampled = 0;           // every workgroup of the launch is a small layer
        rc = traced(lo, kKFinResolve, s, [&] { return launch_fin_resolve(b, b.nsmall, s); });
        if (rc != LAGS_OK) return rc;
    }
    if (ns) {
        SparsifyArgs b = a;
        b.fix_groups = 0;         // exact mode marks no layer for the fallback
        rc = traced(lo, kKFinEmit, s, [&] { return launch_fin_emit(b, nfin, s); });
        if (rc != LAGS_OK) return rc;
    }
    return LAGS_OK;
}

// Launch the sparsify kernels for layers [l0, l1) on a workspace whose head
// holds the layout tables (caller holds lo->mu and has validated everything).
int sparsify_launch(lags_layout *lo, int32_t l0, int32_t l1, const float *grad, float *residual,
                    uint32_t *msg_idx, float *msg_val, unsigned char *w, uint32_t flags, hipStream_t s)
{
    SparsifyArgs a{};
    a.grad = grad;
    a.res = residual;
    a.msg_idx = msg_idx;
    a.msg_val = msg_val;
    a.linfo = (const LayerInfo *)(w + lo->tb_linfo);
    a.sinfo = (const SampledInfo *)(w + lo->tb_sinfo);
    a.main_work = (const MainWork *)(w + lo->tb_main);
    a.fin_work = (const FinWork *)(w + lo->tb_fin);
    a.small_info = (const LayerInfo *)(w + lo->tb_small);
    a.report = (uint32_t *)(w + lo->ws_report);
    a.state = (SampledState *)(w + lo->ws_state);
    a.hist = (uint32_t *)(w + lo->ws_hist);
    a.seg_count = (uint32_t *)(w + lo->ws_segcount);
    a.seg_sel = (uint32_t *)(w + lo->ws_segsel);
    a.slots = (uint2 *)(w + lo->ws_slots);
    a.tbin = (uint2 *)(w + lo->ws_tbin);
    a.fin_total = (uint32_t *)(w + lo->ws_fintot);
    a.fin_eq = (uint32_t *)(w + lo->ws_fineq);
    a.fb = (uint32_t *)(w + lo->ws_fb);
    a.force_exact = (flags & LAGS_SPARSIFY_EXACT) ? 1u : 0u;
    a.sample_base = lo->sid_pre[l0];
    a.nsampled = lo->sid_pre[l1] - lo->sid_pre[l0];
    a.main_base = lo->stream_pre[l0];
    a.fin_base = lo->fin_pre[l0];
    a.small_base = lo->small_pre[l0];
    a.nsmall = lo->small_pre[l1] - lo->small_pre[l0];
    const uint32_t ns = a.nsampled;
    const uint32_t nmain = lo->stream_pre[l1] - lo->stream_pre[l0];
    const uint32_t nfin = lo->fin_pre[l1] - lo->fin_pre[l0];
    // the fallback's workgroups: about one per 4 segments of the range's
    // sampled layers, at least the finishing workgroups, at most kFixGroups
    // (k_fin_emit is launched with max(nfin, fix_groups) workgroups)
    const uint32_t sid0 = lo->sid_pre[l0], sid1 = lo->sid_pre[l1];
    const uint32_t nseg_range =
        ns ? (sid1 < lo->sinfo.size() ? lo->sinfo[sid1].seg_base : lo->nseg_total) - lo->sinfo[sid0].seg_base
           : 0u;
    a.nfin = nfin;
    a.fix_groups = std::min(kFixGroups, std::max(nfin, (nseg_range + 3u) / 4u));
    int rc;
    // k_sample always runs: its first workgroup restarts the report counters
    rc = traced(lo, kKSample, s, [&] { return launch_sample(a, std::max<uint32_t>(1, ns), s); });
    if (rc != LAGS_OK) return rc;
    if (a.force_exact) return sparsify_exact(lo, a, ns, nmain, nfin, s);
    if (nmain) {
        const bool nt_store = (uint64_t)lo->off[l1] - lo->off[l0] > kCachedStreamMax;
        rc = traced(lo, kKMain, s, [&] { return launch_main(a, nmain, nt_store, s); });
        if (rc != LAGS_OK) return rc;
    }
    if (ns) {
        // layers with few histogram copies are decided inside k_fin_select
        if (lo->bins_pre[l1] > lo->bins_pre[l0]) {
            rc = traced(lo, kKFinBins, s, [&] { return launch_fin_bins(a, ns, s); });
            if (rc != LAGS_OK) return rc;
        }
        rc = traced(lo, kKFinSelect, s, [&] { return launch_fin_select(a, nfin, s); });
        if (rc != LAGS_OK) return rc;
    }
    if (ns + a.nsmall) {
        rc = traced(lo, kKFinResolve, s, [&] { return launch_fin_resolve(a, ns + a.nsmall, s); });
        if (rc != LAGS_OK) return rc;
    }
    if (ns) {
        rc = traced(lo, kKFinEmit, s, [&] { return launch_fin_emit(a, std::max(nfin, a.fix_groups), s); });
        if (rc != LAGS_OK) return rc;
    }
    return LAGS_OK;
}

// Launch the aggregate kernels for layers [l0, l1) with P workers on a
// workspace initialised for Pw >= P workers (caller holds lo->mu).
int aggregate_launch(lags_layout *lo, int32_t l0, int32_t l1, float *weights, const uint32_t *msg_idx,
                     const float *msg_val, int32_t P, int32_t Pw, float lr, unsigned char *w,
                     hipStream_t s)
{
    const AggPlan &t = agg_plan(lo, Pw);     // built when the workspace was initialised
    unsigned char *tab = w + lo->ws_agg + align_up((size_t)Pw * ((size_t)t.NC + 1) * 4, kAlign);
    AggArgs a{};
    a.w = weights;
    a.msg_idx = msg_idx;
    a.msg_val = msg_val;
    a.linfo = (const LayerInfo *)(w + lo->tb_linfo);
    a.moff = (const uint32_t *)(w + lo->tb_moff);
    a.pos_layer = (const uint32_t *)(w + lo->tb_pos);
    a.cbase = (const uint32_t *)(tab + t.b_cbase);
    a.csh = (const uint32_t *)(tab + t.b_csh);
    a.chunk_info = (const uint4 *)(tab + t.b_info);
    a.sdesc = (const uint4 *)(tab + t.b_desc);
    a.start = (uint32_t *)(w + lo->ws_agg);
    a.report = (uint32_t *)(w + lo->ws_report);
    a.L = (uint32_t)lo->L;
    a.P = (uint32_t)P;
    a.K = (uint32_t)lo->K;
    a.NC = t.NC;
    a.s = lr / (float)P;
    a.j_lo = lo->moff[l0];
    a.j_hi = lo->moff[l1];
    a.c_lo = t.h_cbase[l0];
    a.c_hi = t.h_cbase[l1];
    a.npb = (uint32_t)lo->pos_layer.size();
    // four position blocks per start-pass workgroup once the launch would
    // take several rounds of workgroups (16K or more), else one
    const uint64_t nblk = (uint64_t)(a.j_hi / kStartsBlock - a.j_lo / kStartsBlock + 1u) * (uint32_t)P;
    const bool wide = nblk >= 16384 && 5ull * lo->starts_tl4 * 4 <= 32768;
    a.bpw = wide ? 4u : 1u;
    a.tl = wide ? lo->starts_tl4 : lo->starts_tl;
    int rc = traced(lo, kKAggStarts, s, [&] { return launch_agg_starts(a, s); });
    if (rc != LAGS_OK) return rc;
    return traced(lo, kKAgg, s, [&] { return launch_agg(a, a.c_hi - a.c_lo, t.tl, t.dense, s); });
}
}  // namespace

extern "C" {

const char *lags_strerror(int status)
{
    switch (status) {
    case LAGS_OK: return "ok";
    case LAGS_EINVAL: return "invalid argument";
    case LAGS_ERANGE: return "size out of the supported range";
    case LAGS_EWORKSPACE: return "workspace missing, misaligned or too small";
    case LAGS_EHIP: return "HIP runtime error";
    case LAGS_EDEVICE: return "current device differs from the workspace's device";
    case LAGS_ENOMEM: return "out of memory";
    case LAGS_ENOTINIT: return "workspace not initialised for this layout (lags_workspace_init)";
    case LAGS_ESTATIC: return "layout needs more scratch than the static buffer of lags_sparsify_layers_static (64 MiB) holds";
    default: return "unknown status";
    }
}

int64_t lags_k_for_ratio(int64_t n, int64_t num, int64_t den)
{
    if (n < 0 || num < 1 || den < 1 || num > den) return LAGS_EINVAL;
    const __int128 p = (__int128)n * num;
    return (int64_t)((p + den - 1) / den);
}

int lags_layout_create(int32_t L, const int64_t *layer_off, const int64_t *k, lags_layout **out)
{
    if (!out) return LAGS_EINVAL;
    *out = nullptr;
    if (!layer_off || !k) return LAGS_EINVAL;
    if (L < 1 || L > LAGS_MAX_LAYERS) return LAGS_ERANGE;
    if (layer_off[0] != 0) return LAGS_EINVAL;
    uint64_t K = 0;
    for (int32_t l = 0; l < L; ++l) {
        if (layer_off[l + 1] <= layer_off[l]) return LAGS_EINVAL;
        const int64_t nl = layer_off[l + 1] - layer_off[l];
        if (k[l] < 1 || k[l] > nl) return LAGS_EINVAL;
        K += (uint64_t)k[l];
    }
    if (layer_off[L] >= (int64_t)0xffffffffLL || K >= 0xffffffffull) return LAGS_ERANGE;
    lags_layout *lo = new (std::nothrow) lags_layout();
    if (!lo) return LAGS_ENOMEM;
    static std::atomic<uint64_t> next_id{1};
    lo->id = next_id.fetch_add(1);
    lo->L = L;
    lo->n = (uint64_t)layer_off[L];
    lo->K = K;
    lo->off.resize(L + 1);
    lo->k.resize(L);
    lo->moff.resize(L + 1);
    uint64_t m = 0;
    for (int32_t l = 0; l <= L; ++l) {
        lo->off[l] = (uint32_t)layer_off[l];
        lo->moff[l] = (uint32_t)m;
        if (l < L) {
            lo->k[l] = (uint32_t)k[l];
            m += (uint64_t)k[l];
        }
    }
    try {
        build_plan(lo);
    } catch (...) {
        delete lo;
        return LAGS_ENOMEM;
    }
    *out = lo;
    return LAGS_OK;
}

void lags_layout_destroy(lags_layout *lo)
{
    if (!lo) return;
    for (auto &r : lo->recs) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    delete lo;
}

int64_t lags_layout_num_elems(const lags_layout *lo) { return lo ? (int64_t)lo->n : -1; }
int64_t lags_layout_total_k(const lags_layout *lo) { return lo ? (int64_t)lo->K : -1; }
int32_t lags_layout_num_layers(const lags_layout *lo) { return lo ? lo->L : -1; }

int64_t lags_layout_msg_offset(const lags_layout *lo, int32_t l)
{
    if (!lo || l < 0 || l > lo->L) return -1;
    return (int64_t)lo->moff[l];
}

size_t lags_workspace_bytes(const lags_layout *clo, int32_t P)
{
    lags_layout *lo = const_cast<lags_layout *>(clo);
    if (!lo || P < 1 || P > LAGS_MAX_WORKERS) return 0;
    std::lock_guard<std::mutex> g(lo->mu);
    try {
        return lo->ws_agg + agg_tail_bytes(agg_plan(lo, P), P);
    } catch (...) {
        return 0;
    }
}

int lags_workspace_init(const lags_layout *clo, void *ws, size_t ws_bytes, int32_t P, void *stream)
{
    lags_layout *lo = const_cast<lags_layout *>(clo);
    if (!lo) return LAGS_EINVAL;
    if (P < 1 || P > LAGS_MAX_WORKERS) return LAGS_ERANGE;
    std::lock_guard<std::mutex> g(lo->mu);
    const AggPlan *t;
    try {
        t = &agg_plan(lo, P);
    } catch (...) {
        return LAGS_ENOMEM;
    }
    const size_t need = lo->ws_agg + agg_tail_bytes(*t, P);
    if (!ws || !aligned16(ws) || ws_bytes < need) return LAGS_EWORKSPACE;
    WsRec rec{ws, need, P, -1};
    if (hipGetDevice(&rec.device) != hipSuccess) return LAGS_EHIP;
    hipStream_t s = (hipStream_t)stream;
    unsigned char *w = (unsigned char *)ws;
    // both images live in the layout until it is destroyed, so the copies
    // may complete after this call returns
    if (hipMemcpyAsync(w, lo->tables.data(), lo->tables.size(), hipMemcpyHostToDevice, s) != hipSuccess)
        return LAGS_EHIP;
    const size_t tail = lo->ws_agg + align_up((size_t)P * ((size_t)t->NC + 1) * 4, kAlign);
    if (hipMemcpyAsync(w + tail, t->image.data(), t->image.size(), hipMemcpyHostToDevice, s) != hipSuccess)
        return LAGS_EHIP;
    for (WsRec &r : lo->wss)
        if (r.ws == ws) {
            r = rec;
            return LAGS_OK;
        }
    try {
        lo->wss.push_back(rec);
    } catch (...) {
        return LAGS_ENOMEM;
    }
    return LAGS_OK;
}

int lags_sparsify_range(const lags_layout *clo, int32_t l0, int32_t l1, const float *grad,
                        float *residual, uint32_t *msg_idx, float *msg_val, void *ws,
                        size_t ws_bytes, uint32_t flags, void *stream)
{
    lags_layout *lo = const_cast<lags_layout *>(clo);
    if (!lo || !grad || !residual || !msg_idx || !msg_val) return LAGS_EINVAL;
    if (l0 < 0 || l1 > lo->L || l0 > l1) return LAGS_ERANGE;
    if (flags & ~LAGS_SPARSIFY_EXACT) return LAGS_EINVAL;
    if (!aligned16(grad) || !aligned16(residual) || !aligned16(msg_idx) || !aligned16(msg_val))
        return LAGS_EINVAL;
    if (!ws || !aligned16(ws) || ws_bytes < lo->ws_agg) return LAGS_EWORKSPACE;
    const size_t nb = lo->n * 4, kb = lo->K * 4;
    const void *bufs[5] = {grad, residual, msg_idx, msg_val, ws};
    const size_t lens[5] = {nb, nb, kb, kb, lo->ws_agg};
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(bufs[i], lens[i], bufs[j], lens[j])) return LAGS_EINVAL;

    std::lock_guard<std::mutex> g(lo->mu);
    const WsRec *rec = find_ws(lo, ws);
    if (!rec) return LAGS_ENOTINIT;
    if (l0 == l1) return LAGS_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return LAGS_EHIP;
    if (dev != rec->device) return LAGS_EDEVICE;
    return sparsify_launch(lo, l0, l1, grad, residual, msg_idx, msg_val, (unsigned char *)ws, flags,
                           (hipStream_t)stream);
}

int lags_sparsify_layers(const lags_layout *lo, const float *grad, float *residual,
                         uint32_t *msg_idx, float *msg_val, void *ws, size_t ws_bytes,
                         uint32_t flags, void *stream)
{
    if (!lo) return LAGS_EINVAL;
    return lags_sparsify_range(lo, 0, lo->L, grad, residual, msg_idx, msg_val, ws, ws_bytes, flags,
                               stream);
}

int lags_sparsify_layers_static(const lags_layout *clo, const float *grad, float *residual,
                                uint32_t *msg_idx, float *msg_val, uint32_t flags, void *stream)
{
    lags_layout *lo = const_cast<lags_layout *>(clo);
    if (!lo || !grad || !residual || !msg_idx || !msg_val) return LAGS_EINVAL;
    if (flags & ~LAGS_SPARSIFY_EXACT) return LAGS_EINVAL;
    if (!aligned16(grad) || !aligned16(residual) || !aligned16(msg_idx) || !aligned16(msg_val))
        return LAGS_EINVAL;
    const size_t nb = lo->n * 4, kb = lo->K * 4;
    const void *bufs[4] = {grad, residual, msg_idx, msg_val};
    const size_t lens[4] = {nb, nb, kb, kb};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(bufs[i], lens[i], bufs[j], lens[j])) return LAGS_EINVAL;
    // tables and scratch of the sparsify call (no aggregate part)
    if (lo->ws_agg > kStaticScratchBytes) return LAGS_ESTATIC;
    void *ws = nullptr;
    if (static_scratch(&ws) != hipSuccess) return LAGS_EHIP;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return LAGS_EHIP;
    hipStream_t s = (hipStream_t)stream;
    {
        // the tables of the layout last used on this device stay in the
        // buffer; another layout's are copied in first (from the layout's
        // host image, which outlives the copy as the layout outlives the call)
        static std::mutex mu;
        static std::map<int, uint64_t> loaded;     // device -> layout id
        std::lock_guard<std::mutex> g(mu);
        auto it = loaded.find(dev);
        if (it == loaded.end() || it->second != lo->id) {
            if (hipMemcpyAsync(ws, lo->tables.data(), lo->tables.size(), hipMemcpyHostToDevice, s) != hipSuccess)
                return LAGS_EHIP;
            loaded[dev] = lo->id;
        }
    }
    std::lock_guard<std::mutex> g(lo->mu);
    return sparsify_launch(lo, 0, lo->L, grad, residual, msg_idx, msg_val, (unsigned char *)ws, flags, s);
}

int lags_aggregate_range(const lags_layout *clo, int32_t l0, int32_t l1, float *weights,
                         const uint32_t *msg_idx, const float *msg_val, int32_t P, float lr,
                         void *ws, size_t ws_bytes, void *stream)
{
    lags_layout *lo = const_cast<lags_layout *>(clo);
    if (!lo || !weights || !msg_idx || !msg_val) return LAGS_EINVAL;
    if (l0 < 0 || l1 > lo->L || l0 > l1) return LAGS_ERANGE;
    if (P < 1 || P > LAGS_MAX_WORKERS) return LAGS_ERANGE;
    if ((uint64_t)P * lo->K >= (1ull << 40)) return LAGS_ERANGE;
    if (!aligned16(weights) || !aligned16(msg_idx) || !aligned16(msg_val)) return LAGS_EINVAL;
    if (!ws || !aligned16(ws)) return LAGS_EWORKSPACE;
    const size_t nb = lo->n * 4, mb = (size_t)P * lo->K * 4;
    const void *bufs[4] = {weights, msg_idx, msg_val, ws};
    size_t lens[4] = {nb, mb, mb, 0};
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(bufs[i], lens[i], bufs[j], lens[j])) return LAGS_EINVAL;

    std::lock_guard<std::mutex> g(lo->mu);
    const WsRec *rec = find_ws(lo, ws);
    if (!rec) return LAGS_ENOTINIT;
    if (P > rec->P) return LAGS_EWORKSPACE;        // initialised for fewer workers
    if (ws_bytes < rec->bytes) return LAGS_EWORKSPACE;
    lens[3] = rec->bytes;
    for (int i = 0; i < 3; ++i)
        if (overlaps(bufs[i], lens[i], bufs[3], lens[3])) return LAGS_EINVAL;
    if (l0 == l1) return LAGS_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return LAGS_EHIP;
    if (dev != rec->device) return LAGS_EDEVICE;
    return aggregate_launch(lo, l0, l1, weights, msg_idx, msg_val, P, rec->P, lr, (unsigned char *)ws,
                            (hipStream_t)stream);
}

int lags_aggregate_apply(const lags_layout *lo, float *weights, const uint32_t *msg_idx,
                         const float *msg_val, int32_t P, float lr, void *ws, size_t ws_bytes,
                         void *stream)
{
    if (!lo) return LAGS_EINVAL;
    return lags_aggregate_range(lo, 0, lo->L, weights, msg_idx, msg_val, P, lr, ws, ws_bytes,
                                stream);
}

int lags_workspace_report(const lags_layout *lo, const void *ws, size_t ws_bytes, void *stream,
                          lags_report *out)
{
    if (!lo || !ws || !out) return LAGS_EINVAL;
    if (ws_bytes < lo->ws_report + kRepWords * 4) return LAGS_EWORKSPACE;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LAGS_EHIP;
    uint32_t h[6];
    if (hipMemcpy(h, (const unsigned char *)ws + lo->ws_report, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess)
        return LAGS_EHIP;
    out->layers_sampled = (int32_t)h[kRepSampled];
    out->layers_exact = (int32_t)h[kRepExact];
    out->bad_entries = h[kRepBad];
    out->slow_chunks = h[kRepSlow];
    out->layers_wide_bin = (int32_t)h[kRepWide];
    out->fix_timeouts = h[kRepFixTimeout];
    return LAGS_OK;
}

int lags_trace_enable(lags_layout *lo, int on)
{
    if (!lo) return LAGS_EINVAL;
    std::lock_guard<std::mutex> g(lo->mu);
    lo->trace = on != 0;
    return LAGS_OK;
}

int lags_trace_read(lags_layout *lo, double *ms, int64_t *launches, int32_t nkernels)
{
    if (!lo || !ms || !launches || nkernels < 0) return LAGS_EINVAL;
    std::lock_guard<std::mutex> g(lo->mu);
    int rc = LAGS_OK;
    for (auto &r : lo->recs) {
        float t = 0.0f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
            rc = LAGS_EHIP;
        lo->tr_ms[r.kid] += t;
        lo->tr_n[r.kid] += 1;
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    lo->recs.clear();
    for (int32_t i = 0; i < nkernels; ++i) {
        ms[i] = i < kNumKernels ? lo->tr_ms[i] : 0.0;
        launches[i] = i < kNumKernels ? lo->tr_n[i] : 0;
    }
    for (int i = 0; i < kNumKernels; ++i) {
        lo->tr_ms[i] = 0.0;
        lo->tr_n[i] = 0;
    }
    return rc;
}

int32_t lags_num_kernels(void) { return kNumKernels; }

const char *lags_kernel_name(int32_t id)
{
    static const char *names[kNumKernels] = {"k_sample",     "k_main",     "k_fin_bins",   "k_fin_select",
                                             "k_fin_resolve", "k_fin_emit", "k_agg_starts", "k_agg",
                                             "k_x_first",    "k_x_pass",   "k_x_pick",     "k_x_count",
                                             "k_x_cut"};
    return (id >= 0 && id < kNumKernels) ? names[id] : "unknown";
}

}  // extern "C"
