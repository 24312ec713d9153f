// Host side of the LAGS-SGD library: argument validation, per-layer planning,
// workspace sizing, device tables, kernel launches and kernel tracing.
// The entry points are declared in include/lags.h.
#include "lags.h"
#include "lags_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

using namespace lags;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct AggTables {
    uint32_t NC = 0;
    std::vector<uint32_t> h_cbase;    // [L+1], host copy
    void *dev = nullptr;
    uint32_t *cbase = nullptr;   // [L+1]
    uint32_t *csh = nullptr;     // [L]
    uint4 *chunk_info = nullptr;      // [NC]
};

struct TraceRec {
    int32_t kid;
    hipEvent_t a, b;
};

}  // namespace

struct lags_layout {
    int32_t L = 0;
    uint64_t n = 0, K = 0;
    std::vector<uint32_t> off, k, moff;
    std::vector<LayerInfo> linfo;
    std::vector<SampledInfo> sinfo;
    std::vector<MainWork> main_work;
    std::vector<uint32_t> small_layers;
    std::vector<FinWork> fin_work;
    std::vector<uint32_t> pos_layer;
    uint32_t starts_tl = 0;        // LDS table entries the start pass needs (one block per workgroup)
    uint32_t starts_tl4 = 0;       // ... four blocks per workgroup
    // per-layer prefix counts of the work lists, for layer-range launches:
    // small-layer work entries, streaming work entries, sampled layers and
    // finishing workgroups before layer l
    std::vector<uint32_t> small_pre, stream_pre, sid_pre, fin_pre;
    uint32_t nseg_total = 0;
    uint64_t slots_total = 0;
    uint64_t hist_words = 0;
    // workspace plan (byte offsets)
    size_t ws_report = 0, ws_state = 0, ws_hist = 0, ws_segcount = 0, ws_segsel = 0,
           ws_slots = 0, ws_tbin = 0, ws_fintot = 0, ws_fineq = 0, ws_agg = 0;
    // device tables, built on first use
    std::mutex mu;
    int device = -1;
    void *dev = nullptr;
    LayerInfo *d_linfo = nullptr;
    SampledInfo *d_sinfo = nullptr;
    MainWork *d_main = nullptr;
    FinWork *d_fin = nullptr;
    uint32_t *d_moff = nullptr;
    uint32_t *d_poslayer = nullptr;
    uint32_t *d_small = nullptr;
    std::map<int32_t, AggTables> agg;
    // tracing
    bool trace = false;
    std::vector<TraceRec> recs;
    double tr_ms[kNumKernels] = {};
    int64_t tr_n[kNumKernels] = {};
};

namespace {

// Chunk widths of the aggregate for P workers: per layer, a power of two (at
// most 2^kAggMaxWidthLog2) such that a chunk holds about kAggTargetEntries
// message entries over all workers.
void plan_agg(const lags_layout *lo, int32_t P, std::vector<uint32_t> &cbase,
              std::vector<uint32_t> &csh, uint32_t &NC)
{
    cbase.assign(lo->L + 1, 0);
    csh.assign(lo->L, 0);
    uint64_t total = 0;
    for (int32_t l = 0; l < lo->L; ++l) {
        const double nl = lo->linfo[l].n, kl = lo->linfo[l].k;
        const double width = (double)kAggTargetEntries * nl / ((double)P * kl);
        int s = 0;
        while (s < (int)kAggMaxWidthLog2 && std::ldexp(1.0, s + 1) <= width) ++s;
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
    auto work = [](uint32_t l, uint32_t cls, uint32_t tile) {
        MainWork w{};
        w.layer = l;
        w.cls = cls;
        w.tile = tile;
        return w;
    };
    for (int32_t l = 0; l < L; ++l) {
        lo->small_pre[l] = (uint32_t)lo->small_layers.size();
        lo->stream_pre[l] = (uint32_t)stream_work.size();
        lo->sid_pre[l] = (uint32_t)lo->sinfo.size();
        lo->fin_pre[l] = (uint32_t)lo->fin_work.size();
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
            lo->small_layers.push_back((uint32_t)l);
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
            li.ntiles = (si.nseg + kTileSegs - 1) / kTileSegs;
            // histogram copies grow with the layer, so that the streaming
            // workgroups' atomics on its hottest bins stay spread
            si.hcopies = 1;
            while (si.hcopies < kHistMaxCopies && si.hcopies * kTilesPerCopy < li.ntiles) si.hcopies *= 2;
            si.hist_off = (uint32_t)lo->hist_words;
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
                lo->fin_work.push_back(f);
            }
            seg_base += si.nseg;
            slot_base += (uint64_t)si.nseg * si.cap;
            lo->sinfo.push_back(si);
        }
    }
    lo->small_pre[L] = (uint32_t)lo->small_layers.size();
    lo->stream_pre[L] = (uint32_t)stream_work.size();
    lo->sid_pre[L] = (uint32_t)lo->sinfo.size();
    lo->fin_pre[L] = (uint32_t)lo->fin_work.size();
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

    const size_t ns = lo->sinfo.size();
    size_t at = 0;
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
    lo->ws_agg = at;
    return LAGS_OK;
}

size_t agg_bytes(const lags_layout *lo, int32_t P)
{
    std::vector<uint32_t> cb, cs;
    uint32_t NC;
    plan_agg(lo, P, cb, cs, NC);
    return align_up((size_t)P * ((size_t)NC + 1) * 4, kAlign);
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Device tables for the layout on the current device (caller holds lo->mu).
int ensure_device(lags_layout *lo)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return LAGS_EHIP;
    if (lo->dev) return dev == lo->device ? LAGS_OK : LAGS_EDEVICE;
    const size_t b_l = align_up(lo->linfo.size() * sizeof(LayerInfo), kAlign);
    const size_t b_s = align_up(std::max<size_t>(1, lo->sinfo.size()) * sizeof(SampledInfo), kAlign);
    const size_t b_m = align_up(std::max<size_t>(1, lo->main_work.size()) * sizeof(MainWork), kAlign);
    const size_t b_f = align_up(std::max<size_t>(1, lo->fin_work.size()) * sizeof(FinWork), kAlign);
    const size_t b_o = align_up(lo->moff.size() * 4, kAlign);
    const size_t b_p = align_up(lo->pos_layer.size() * 4, kAlign);
    const size_t b_sm = align_up(std::max<size_t>(1, lo->small_layers.size()) * 4, kAlign);
    const size_t total = b_l + b_s + b_m + b_f + b_o + b_p + b_sm;
    std::vector<unsigned char> host(total, 0);
    std::memcpy(host.data(), lo->linfo.data(), lo->linfo.size() * sizeof(LayerInfo));
    if (!lo->sinfo.empty())
        std::memcpy(host.data() + b_l, lo->sinfo.data(), lo->sinfo.size() * sizeof(SampledInfo));
    std::memcpy(host.data() + b_l + b_s, lo->main_work.data(), lo->main_work.size() * sizeof(MainWork));
    if (!lo->fin_work.empty())
        std::memcpy(host.data() + b_l + b_s + b_m, lo->fin_work.data(), lo->fin_work.size() * sizeof(FinWork));
    std::memcpy(host.data() + b_l + b_s + b_m + b_f, lo->moff.data(), lo->moff.size() * 4);
    std::memcpy(host.data() + b_l + b_s + b_m + b_f + b_o, lo->pos_layer.data(), lo->pos_layer.size() * 4);
    if (!lo->small_layers.empty())
        std::memcpy(host.data() + b_l + b_s + b_m + b_f + b_o + b_p, lo->small_layers.data(),
                    lo->small_layers.size() * 4);
    void *d = nullptr;
    if (hipMalloc(&d, total) != hipSuccess) return LAGS_ENOMEM;
    if (hipMemcpy(d, host.data(), total, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(d);
        return LAGS_EHIP;
    }
    unsigned char *p = (unsigned char *)d;
    lo->dev = d;
    lo->device = dev;
    lo->d_linfo = (LayerInfo *)p;
    lo->d_sinfo = (SampledInfo *)(p + b_l);
    lo->d_main = (MainWork *)(p + b_l + b_s);
    lo->d_fin = (FinWork *)(p + b_l + b_s + b_m);
    lo->d_moff = (uint32_t *)(p + b_l + b_s + b_m + b_f);
    lo->d_poslayer = (uint32_t *)(p + b_l + b_s + b_m + b_f + b_o);
    lo->d_small = (uint32_t *)(p + b_l + b_s + b_m + b_f + b_o + b_p);
    return LAGS_OK;
}

int ensure_agg(lags_layout *lo, int32_t P, AggTables **out)
{
    auto it = lo->agg.find(P);
    if (it != lo->agg.end()) {
        *out = &it->second;
        return LAGS_OK;
    }
    std::vector<uint32_t> cb, cs;
    uint32_t NC;
    plan_agg(lo, P, cb, cs, NC);
    // per chunk: its index range inside its layer and the layer's message
    // range, so that an aggregate workgroup needs one load to start
    std::vector<uint4> ci(std::max<uint32_t>(NC, 1), uint4{0, 0, 0, 0});
    for (int32_t l = 0; l < lo->L; ++l) {
        const uint64_t off = lo->off[l], end = lo->off[l + 1];
        for (uint32_t c = cb[l]; c < cb[l + 1]; ++c) {
            const uint64_t clo = off + ((uint64_t)(c - cb[l]) << cs[l]);
            const uint64_t chi = std::min<uint64_t>(clo + ((uint64_t)1 << cs[l]), end);
            ci[c] = uint4{(uint32_t)clo, (uint32_t)chi, (uint32_t)lo->moff[l],
                          (uint32_t)(lo->moff[l] + lo->k[l])};
        }
    }
    const size_t b0 = align_up(cb.size() * 4, kAlign), b1 = align_up(cs.size() * 4, kAlign),
                 b2 = align_up(ci.size() * sizeof(uint4), kAlign);
    std::vector<unsigned char> host(b0 + b1 + b2, 0);
    std::memcpy(host.data(), cb.data(), cb.size() * 4);
    std::memcpy(host.data() + b0, cs.data(), cs.size() * 4);
    std::memcpy(host.data() + b0 + b1, ci.data(), ci.size() * sizeof(uint4));
    void *d = nullptr;
    if (hipMalloc(&d, host.size()) != hipSuccess) return LAGS_ENOMEM;
    if (hipMemcpy(d, host.data(), host.size(), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(d);
        return LAGS_EHIP;
    }
    AggTables t;
    t.NC = NC;
    t.h_cbase = cb;
    t.dev = d;
    t.cbase = (uint32_t *)d;
    t.csh = (uint32_t *)((unsigned char *)d + b0);
    t.chunk_info = (uint4 *)((unsigned char *)d + b0 + b1);
    auto res = lo->agg.emplace(P, t);
    *out = &res.first->second;
    return LAGS_OK;
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
        rc = traced(lo, kKFinEmit, s, [&] { return launch_fin_emit(a, nfin, s); });
        if (rc != LAGS_OK) return rc;
    }
    return LAGS_OK;
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
    case LAGS_EDEVICE: return "current device differs from the layout's device";
    case LAGS_ENOMEM: return "out of memory";
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
    for (auto &kv : lo->agg) (void)hipFree(kv.second.dev);
    if (lo->dev) (void)hipFree(lo->dev);
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

size_t lags_workspace_bytes(const lags_layout *lo, int32_t P)
{
    if (!lo || P < 1 || P > LAGS_MAX_WORKERS) return 0;
    return lo->ws_agg + agg_bytes(lo, P);
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
    if (l0 == l1) return LAGS_OK;

    std::lock_guard<std::mutex> g(lo->mu);
    int rc = ensure_device(lo);
    if (rc != LAGS_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    unsigned char *w = (unsigned char *)ws;
    SparsifyArgs a{};
    a.grad = grad;
    a.res = residual;
    a.msg_idx = msg_idx;
    a.msg_val = msg_val;
    a.linfo = lo->d_linfo;
    a.sinfo = lo->d_sinfo;
    a.main_work = lo->d_main;
    a.fin_work = lo->d_fin;
    a.report = (uint32_t *)(w + lo->ws_report);
    a.state = (SampledState *)(w + lo->ws_state);
    a.hist = (uint32_t *)(w + lo->ws_hist);
    a.seg_count = (uint32_t *)(w + lo->ws_segcount);
    a.seg_sel = (uint32_t *)(w + lo->ws_segsel);
    a.slots = (uint2 *)(w + lo->ws_slots);
    a.tbin = (uint2 *)(w + lo->ws_tbin);
    a.fin_total = (uint32_t *)(w + lo->ws_fintot);
    a.fin_eq = (uint32_t *)(w + lo->ws_fineq);
    a.force_exact = (flags & LAGS_SPARSIFY_EXACT) ? 1u : 0u;
    a.sample_base = lo->sid_pre[l0];
    a.nsampled = lo->sid_pre[l1] - lo->sid_pre[l0];
    a.main_base = lo->stream_pre[l0];
    a.fin_base = lo->fin_pre[l0];
    a.small_layers = lo->d_small;
    a.small_base = lo->small_pre[l0];
    a.nsmall = lo->small_pre[l1] - lo->small_pre[l0];
    const uint32_t ns = a.nsampled;
    const uint32_t nmain = lo->stream_pre[l1] - lo->stream_pre[l0];
    const uint32_t nfin = lo->fin_pre[l1] - lo->fin_pre[l0];
    // k_sample always runs: its first workgroup restarts the report counters
    rc = traced(lo, kKSample, s, [&] { return launch_sample(a, std::max<uint32_t>(1, ns), s); });
    if (rc != LAGS_OK) return rc;
    if (a.force_exact) return sparsify_exact(lo, a, ns, nmain, nfin, s);
    if (nmain) {
        rc = traced(lo, kKMain, s, [&] { return launch_main(a, nmain, s); });
        if (rc != LAGS_OK) return rc;
    }
    if (ns) {
        rc = traced(lo, kKFinBins, s, [&] { return launch_fin_bins(a, ns, s); });
        if (rc != LAGS_OK) return rc;
        rc = traced(lo, kKFinSelect, s, [&] { return launch_fin_select(a, nfin, s); });
        if (rc != LAGS_OK) return rc;
    }
    if (ns + a.nsmall) {
        rc = traced(lo, kKFinResolve, s, [&] { return launch_fin_resolve(a, ns + a.nsmall, s); });
        if (rc != LAGS_OK) return rc;
    }
    if (ns) {
        rc = traced(lo, kKFinEmit, s, [&] { return launch_fin_emit(a, nfin, s); });
        if (rc != LAGS_OK) return rc;
    }
    return LAGS_OK;
}

int lags_sparsify_layers(const lags_layout *lo, const float *grad, float *residual,
                         uint32_t *msg_idx, float *msg_val, void *ws, size_t ws_bytes,
                         uint32_t flags, void *stream)
{
    if (!lo) return LAGS_EINVAL;
    return lags_sparsify_range(lo, 0, lo->L, grad, residual, msg_idx, msg_val, ws, ws_bytes, flags,
                               stream);
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
    const size_t need = lo->ws_agg + agg_bytes(lo, P);
    if (!ws || !aligned16(ws) || ws_bytes < need) return LAGS_EWORKSPACE;
    const size_t nb = lo->n * 4, mb = (size_t)P * lo->K * 4;
    const void *bufs[4] = {weights, msg_idx, msg_val, ws};
    const size_t lens[4] = {nb, mb, mb, need};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(bufs[i], lens[i], bufs[j], lens[j])) return LAGS_EINVAL;
    if (l0 == l1) return LAGS_OK;

    std::lock_guard<std::mutex> g(lo->mu);
    int rc = ensure_device(lo);
    if (rc != LAGS_OK) return rc;
    AggTables *t = nullptr;
    rc = ensure_agg(lo, P, &t);
    if (rc != LAGS_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    unsigned char *w = (unsigned char *)ws;
    AggArgs a{};
    a.w = weights;
    a.msg_idx = msg_idx;
    a.msg_val = msg_val;
    a.linfo = lo->d_linfo;
    a.moff = lo->d_moff;
    a.pos_layer = lo->d_poslayer;
    a.cbase = t->cbase;
    a.csh = t->csh;
    a.chunk_info = t->chunk_info;
    a.start = (uint32_t *)(w + lo->ws_agg);
    a.report = (uint32_t *)(w + lo->ws_report);
    a.L = (uint32_t)lo->L;
    a.P = (uint32_t)P;
    a.K = (uint32_t)lo->K;
    a.NC = t->NC;
    a.s = lr / (float)P;
    a.j_lo = lo->moff[l0];
    a.j_hi = lo->moff[l1];
    a.c_lo = t->h_cbase[l0];
    a.c_hi = t->h_cbase[l1];
    a.npb = (uint32_t)lo->pos_layer.size();
    // four position blocks per start-pass workgroup once the launch would
    // take several rounds of workgroups (16K or more), else one
    const uint64_t nblk = (uint64_t)(a.j_hi / kStartsBlock - a.j_lo / kStartsBlock + 1u) * (uint32_t)P;
    const bool wide = nblk >= 16384 && 5ull * lo->starts_tl4 * 4 <= 32768;
    a.bpw = wide ? 4u : 1u;
    a.tl = wide ? lo->starts_tl4 : lo->starts_tl;
    rc = traced(lo, kKAggStarts, s, [&] { return launch_agg_starts(a, s); });
    if (rc != LAGS_OK) return rc;
    return traced(lo, kKAgg, s, [&] { return launch_agg(a, a.c_hi - a.c_lo, s); });
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
    if (ws_bytes < lo->ws_report + 20) return LAGS_EWORKSPACE;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LAGS_EHIP;
    uint32_t h[5];
    if (hipMemcpy(h, (const unsigned char *)ws + lo->ws_report, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess)
        return LAGS_EHIP;
    out->layers_sampled = (int32_t)h[kRepSampled];
    out->layers_exact = (int32_t)h[kRepExact];
    out->bad_entries = h[kRepBad];
    out->slow_chunks = h[kRepSlow];
    out->layers_wide_bin = (int32_t)h[kRepWide];
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
