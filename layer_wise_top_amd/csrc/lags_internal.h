// Internal tables and constants shared by the host planner (lags_host.cpp)
// and the gfx950 kernels (lags_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace lags {

// ---- launch geometry ------------------------------------------------------
constexpr int kBlock = 256;              // threads per workgroup (4 wave64)
constexpr int kWaves = kBlock / 64;
constexpr uint32_t kSeg = 4096;          // entries per segment (one streaming workgroup)
constexpr uint32_t kTileSegs = 4;        // segments per streaming work entry (one workgroup each)
constexpr uint32_t kSmallMax = 4096;     // layers up to this size: one workgroup, exact
constexpr uint32_t kDenseTile = 16384;   // entries per streaming work entry of a k == n layer
constexpr uint32_t kSampleMax = 16384;   // sampled keys per layer (LDS resident)
constexpr uint32_t kSampleChunk = 64;    // contiguous entries per sample chunk
constexpr uint32_t kCapMax = 1024;       // candidate slots per segment, at most (beyond:
                                         // the segment is re-read)
constexpr uint32_t kNBins = 2048;        // candidate histogram bins per layer
constexpr uint32_t kHistMaxCopies = 64;  // copies of a layer's histogram, at most (spread atomics)
constexpr uint32_t kTilesPerCopy = 128;  // streaming workgroups per histogram copy, about
constexpr uint32_t kSelfBinsCopies = 4;  // layers with at most this many copies are decided
                                         // by their finishing workgroups (no k_fin_bins)
// a streaming pass over at most this many entries stores the residual with
// ordinary stores (it stays in the 256 MB cache for the scattered residual
// writes that follow: ResNet-50, 25.6M entries, step 0.1525 -> 0.1499 ms);
// larger ones store non-temporally (with ordinary stores the 66M-entry LSTM
// step took 0.278 ms instead of 0.244, and the 1.31B-entry step 4.11 ms
// instead of 3.52)
constexpr uint64_t kCachedStreamMax = uint64_t(32) << 20;
constexpr uint32_t kTbinCap = 4096;      // threshold-bin entries resolved in LDS (larger: global)
constexpr uint32_t kFinSegs = 32;        // segments per finishing workgroup (at most)
constexpr uint32_t kFinSegsSmall = 16;   // ... in a layer of at most kFinSmallLayer segments
constexpr uint32_t kFinSmallLayer = 1024;
// segments per finishing workgroup of a layer of nseg segments: finer for
// smaller layers (more of them run at once; the larger layers keep fewer
// reservation atomics)
__host__ __device__ inline uint32_t fin_grain(uint32_t nseg)
{
    return nseg <= kFinSmallLayer ? kFinSegsSmall : kFinSegs;
}
// aggregate: a chunk's workgroup keeps an LDS hash table of 2^TL slots (also
// the slow path's dense window) for at most 2^(TL-1) message entries (the
// fast path) and expects 2^(TL-2); TL is kAggTableLog2 in general and
// kAggTableLog2Wide when a call reads at least kAggWideEntries message entries
// (measured: 1.31B entries, 21M entries read: 0.879 ms against 0.890 ms;
// 25.6M entries, 2.8M read: 0.056 ms against 0.046 ms)
constexpr uint32_t kAggTableLog2 = 11;
constexpr uint32_t kAggTableLog2Wide = 10;
constexpr uint64_t kAggWideEntries = uint64_t(8) << 20;
constexpr uint32_t kStartsBlock = 1024;       // message positions per start-pass block
constexpr uint32_t kAggMaxWidthLog2 = 30;     // chunk width cap (entries)
// A layer whose workers send every entry (k = n) is cut into chunks of one
// index per thread; every valid message holds index off + i at position
// moff + i, so the chunk's entries are found without the chunk-start table.
constexpr uint32_t kAggDenseLog2 = 8;
static_assert((1u << kAggDenseLog2) == (uint32_t)kBlock, "one index per thread");
constexpr uint32_t kAggDenseChunk = 0xffffffffu;   // chunk_info.w of such a chunk
// guess-failure fallback (inside k_fin_emit): the first kFixGroups workgroups
// of the launch select every failed layer together, by a radix select over all
// of its keys, meeting at barriers between the passes
constexpr uint32_t kFixGroups = 1024;
// per sampled layer: histograms of the three key digits (11, 11 and 9 bits),
// the count of keys above the range the threshold is known to lie in, the
// barrier's top counter and its kFixSubs sub-counters (one 128-byte line
// each), then per fallback workgroup its count of keys above and equal to the
// threshold.  Everything before kFbCount starts at zero.
constexpr uint32_t kFixSubs = 32;
constexpr uint32_t kFbHist0 = 0, kFbHist1 = 2048, kFbHist2 = 4096, kFbAbove = 4608, kFbBarTop = 4640,
                   kFbBarSub = 4672, kFbCount = kFbBarSub + 32 * kFixSubs;
constexpr uint32_t kFbWords = kFbCount + 2 * kFixGroups;

// ---- layer classes --------------------------------------------------------
enum : uint32_t {
    kClsSmall = 0,    // n <= kSmallMax: one workgroup does everything (LDS)
    kClsDense = 1,    // k == n: every entry is sent
    kClsSampled = 2,  // sampled threshold guess + candidate compaction
};

// ---- per-call status of a sampled layer -----------------------------------
enum : uint32_t {
    kStPending = 0,
    kStOk = 1,        // candidates hold the top k; threshold bin resolved
    kStZero = 3,      // guess G = 0 and fewer than k nonzero keys: T = 0, all nonzero
                      // entries plus the lowest-index zeros are sent
    kStFix = 4,       // the guess failed (fewer than k candidates above a nonzero G, or a
                      // threshold bin larger than its list): k_fin_emit's fallback
                      // workgroups select the layer from all of its keys
};

struct LayerInfo {        // one per layer, device table
    uint32_t off;         // first entry
    uint32_t n;           // entries
    uint32_t k;           // entries sent
    uint32_t moff;        // message offset
    uint32_t cls;
    uint32_t sid;         // sampled-layer id or 0xffffffff
    uint32_t ntiles;      // streaming workgroups of this layer in the main kernel
    uint32_t pad;
};

struct SampledInfo {      // one per sampled layer, device table
    uint32_t layer;
    uint32_t a4, b4;      // 4-aligned interior [a4, b4) of the layer
    uint32_t nseg;        // segments (kSeg entries of the interior each)
    uint32_t seg_base;    // first global segment id
    uint32_t cap;         // candidate slots per segment
    uint32_t slot_lo, slot_hi;   // first slot (64-bit, in 8-byte slots)
    uint32_t full_sample; // 1: the sample is the whole layer (guess = exact k-th key)
    uint32_t nchunk;      // sample chunks (when not full)
    uint32_t j;           // rank of the guess inside the sample (1-based, from the top)
    uint32_t spare;
    uint32_t fin_nblocks; // finishing workgroups of this layer
    uint32_t fin_first;   // index of the layer's first finishing workgroup
    uint32_t tbin_cap;    // threshold-bin entries the layer can keep: all its slots
                          // (the list sits at the layer's slot offset in its own region)
    uint32_t hist_off;    // first word of the layer's histogram copies in the workspace
    uint32_t hcopies;     // copies (a power of two), kNBins words each
    // the layer's own fields, so that one load starts a per-layer workgroup
    uint32_t off, n, k, moff;
    uint32_t grain;       // segments per finishing workgroup of the layer
    uint32_t pad[10];
};
static_assert(sizeof(SampledInfo) == 128, "two per 256-byte line");

// One entry per k_main workgroup: everything a streaming tile needs, so one
// load starts it (small and k == n layers use layer and tile only).
struct MainWork {
    uint32_t layer;
    uint32_t cls;
    uint32_t tile;        // tile index inside the layer
    uint32_t sid;         // sampled-layer id
    uint32_t off, end;    // layer range [off, end)
    uint32_t a4, b4;      // 4-aligned interior of the layer
    uint32_t nseg;        // segments of the layer
    uint32_t seg_base;    // global id of the layer's segment 0
    uint32_t cap;         // candidate slots per segment
    uint32_t slot_lo, slot_hi;   // first slot of the layer
    uint32_t hist_off, hcopies;  // the layer's histogram copies
    uint32_t pad;
};

// One entry per finishing workgroup (k_fin_select, k_fin_emit): its segments
// and the static fields of its layer, so one load starts it.
struct FinWork {
    uint32_t sid;         // sampled-layer id
    uint32_t seg0;        // first segment of the workgroup (inside the layer)
    uint32_t nseg;        // segments of the layer
    uint32_t seg_base;    // first global segment id of the layer
    uint32_t cap;         // candidate slots per segment
    uint32_t slot_lo, slot_hi;   // first slot of the layer
    uint32_t fin_first;   // first finishing workgroup of the layer
    uint32_t off, n;      // the layer's entries
    uint32_t moff, k;     // the layer's message
    uint32_t tbin_cap;
    uint32_t grain;       // segments per finishing workgroup of the layer
    uint32_t a4;          // 4-aligned start of the layer's interior
    uint32_t hist_off;    // the layer's histogram copies (first word, count)
    uint32_t hcopies;
    uint32_t pad[2];
};

struct SampledState {     // per sampled layer, per call, in the workspace
    uint32_t G;           // guess: candidates have key >= G
    uint32_t SH;          // histogram bin width 2^SH above G
    uint32_t status;
    uint32_t spare;
    uint32_t bstar;       // histogram bin holding the k-th largest candidate
    uint32_t c_above;     // candidates in bins above bstar
    uint32_t xprefix;     // exact mode: key bits found so far
    uint32_t xrank;       // exact mode: rank still to find among keys with that prefix
    uint32_t T;           // k-th largest key of the layer
    uint32_t idx_cut;     // largest global index taken among keys == T
    uint32_t spare1;
    uint32_t nfail;       // (first sampled layer of a launched range only) layers of the
                          // range that need the fallback
    uint32_t fix_klo, fix_khi;   // fallback: T is known to lie in [fix_klo, fix_khi]
    uint32_t pad0[18];
    // on a cache line of its own: every finishing workgroup of the layer
    // reads the fields above while the select pass adds to this one
    uint32_t tbin_n;      // entries of bin bstar collected
    uint32_t pad1[31];
};
static_assert(offsetof(SampledState, tbin_n) == 128 && sizeof(SampledState) == 256,
              "the collection counter sits on its own 128-byte line");

// report counters at the head of the workspace
enum : uint32_t {
    kRepSampled = 0, kRepExact = 1, kRepBad = 2, kRepSlow = 3, kRepWide = 4, kRepFixTimeout = 5,
    kRepWords = 64
};

struct SparsifyArgs {
    const float *grad;
    float *res;
    uint32_t *msg_idx;
    float *msg_val;
    const LayerInfo *linfo;
    const SampledInfo *sinfo;
    const MainWork *main_work;   // one per main workgroup
    const FinWork *fin_work;  // one per finishing workgroup
    uint32_t *report;
    SampledState *state;
    uint32_t *hist;           // candidate histograms (SampledInfo::hist_off, hcopies)
    uint32_t *seg_count;
    uint32_t *seg_sel;
    uint2 *slots;
    uint2 *tbin;
    uint32_t *fin_total;      // per finishing workgroup: count, then message offset
    uint32_t *fin_eq;         // per finishing workgroup (zero mode): zeros, then zeros before it
    uint32_t *fb;             // per sampled layer kFbWords words: the fallback's histograms, counts
    uint32_t fix_groups;      // workgroups of the k_fin_emit launch that run the fallback
    uint32_t nfin;            // finishing workgroups of the launched range (k_fin_emit may
                              // launch more: the extra ones only run the fallback)
    uint32_t nsampled;        // sampled layers in the launched range
    uint32_t force_exact;
    // the launched layer range, as offsets into the layout's work lists
    uint32_t sample_base;     // first sampled-layer id
    uint32_t main_base;       // first streaming work entry
    uint32_t fin_base;        // first finishing workgroup
    const LayerInfo *small_info;    // the small layers (n <= kSmallMax), ascending
    uint32_t small_base;      // first small layer of the range in that list
    uint32_t nsmall;          // small layers in the range
};

struct AggArgs {
    float *w;
    const uint32_t *msg_idx;
    const float *msg_val;
    const LayerInfo *linfo;
    const uint32_t *moff;       // [L+1]
    const uint32_t *pos_layer;  // [ceil((K+1)/kStartsBlock)] layer of position b*kStartsBlock
    const uint32_t *cbase;      // [L+1] first chunk of each layer
    const uint32_t *csh;        // [L] log2 chunk width
    const uint4 *chunk_info;    // [NC] per chunk: first index, end index, and the
                                // message range [moff, moff + k) of its layer; for a
                                // chunk of a k = n layer: first index, end index, the
                                // position of the first index, kAggDenseChunk
    const uint4 *sdesc;         // [npb][2] per position block b: {layer of position
                                // b*kStartsBlock - 1 (0 for b = 0), layer of the block's
                                // last position (or of position K - 1), that first
                                // layer's off and n}, {its first chunk, log2 chunk width}
    uint32_t *start;            // [P][NC+1]
    uint32_t *report;
    uint32_t L;
    uint32_t P;
    uint32_t K;
    uint32_t NC;
    float s;                    // lr / P, rounded to fp32 on the host
    // the launched layer range: message positions [j_lo, j_hi], chunks [c_lo, c_hi)
    uint32_t j_lo, j_hi;
    uint32_t c_lo, c_hi;
    uint32_t npb;               // entries of pos_layer
    uint32_t tl;                // start pass: LDS table entries (layers a workgroup spans, plus 2)
    uint32_t bpw;               // start pass: position blocks per workgroup (1 or 4)
};

// kernel ids for tracing
enum : int32_t {
    kKSample = 0, kKMain = 1, kKFinBins = 2, kKFinSelect = 3, kKFinResolve = 4,
    kKFinEmit = 5, kKAggStarts = 6, kKAgg = 7, kKXFirst = 8, kKXPass = 9, kKXPick = 10,
    kKXCount = 11, kKXCut = 12, kNumKernels = 13
};

// the allocation-free sparsify's static scratch (lags_kernels.hip): its size,
// and this device's address of it (looked up once per device)
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(void **out);

// launchers (lags_kernels.hip)
hipError_t launch_sample(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s);
hipError_t launch_main(const SparsifyArgs &a, uint32_t nblocks, bool nt_store, hipStream_t s);
hipError_t launch_fin_bins(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s);
hipError_t launch_fin_select(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s);
hipError_t launch_fin_resolve(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s);
hipError_t launch_fin_emit(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s);
hipError_t launch_x_first(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s);
hipError_t launch_x_pass(const SparsifyArgs &a, uint32_t nblocks, uint32_t level, hipStream_t s);
hipError_t launch_x_pick(const SparsifyArgs &a, uint32_t nblocks, uint32_t level, hipStream_t s);
hipError_t launch_x_count(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s);
hipError_t launch_x_cut(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s);
hipError_t launch_agg_starts(const AggArgs &a, hipStream_t s);
hipError_t launch_agg(const AggArgs &a, uint32_t nchunks, uint32_t table_log2, bool dense, hipStream_t s);

}  // namespace lags
