// gfx950 kernels of the LAGS-SGD data-parallel hot path.
//
// What is computed follows the review "Layer-wise Adaptive Gradient
// Sparsification for Distributed Deep Learning with Convergence Guarantees"
// (abstract; proposed method, bullets 1, 2 and 4): per layer, error-
// compensated top-k by magnitude, index-ordered (index, value) messages, the
// residual of what was not sent, and the S-SGD average of P workers'
// messages applied to the weights.
//
// How it is computed here (the pages give no GPU design):
//   k_sample      one workgroup per sampled layer: reads a stratified sample
//                 of acc = grad + residual, takes a rank from the top of the
//                 sample as a threshold guess G that at least k entries of the
//                 layer exceed with overwhelming probability; also clears the
//                 layer's per-call state.
//   k_main        the streaming pass, one workgroup per 4096-entry segment
//                 requesting all of it at once: acc = grad + residual is
//                 written back to the residual buffer; entries with |acc| key
//                 >= G (>= 1 when G = 0: zeros are not stored) are compacted,
//                 in index order, into per-segment candidate slots, and
//                 counted in the layer's histogram of bins above G.  k == n
//                 layers are sent whole.
//   k_fin_bins    one workgroup per sampled layer: sums the layer's
//                 histogram copies and finds the bin holding the k-th largest
//                 candidate.
//   k_fin_select  counts, per segment, candidates above the threshold bin and
//                 gathers the threshold bin's candidates.
//   k_fin_resolve one workgroup per sampled layer: resolves the exact
//                 threshold key T and the tie cut (lowest indices first) and
//                 scans segment counts into message offsets.  One more
//                 workgroup per small layer (<= 4096 entries) does that layer
//                 start to finish (exact radix select in LDS).
//   k_fin_emit    writes the selected candidates of each segment, in index
//                 order, to the message and zeroes their residual.  A layer
//                 with fewer than k nonzero keys (G = 0, "zero mode") sends
//                 every nonzero entry and its lowest-index zeros; segments
//                 that send zeros are re-read from the residual buffer.
//                 Then its first workgroups (all resident) select, by a
//                 multi-workgroup radix select over the residual buffer, any
//                 layer whose guess failed (fewer than k candidates above a
//                 nonzero G, or a threshold bin larger than the layer's list).
//   k_x_first, k_x_pass, k_x_pick, k_x_count, k_x_cut
//                 exact mode (chosen by the caller): the threshold of every
//                 sampled layer by a multi-workgroup radix select over all its
//                 keys (three digit passes, each followed by a per-layer
//                 pick), then per-segment counts, the tie cut and message
//                 offsets; k_x_count keeps each segment's keys >= T in its
//                 slots and k_fin_emit emits from them.  The passes over a
//                 layer take k_main's one-workgroup-per-segment shape.
//   k_agg_starts  for every worker, where each index chunk starts in its
//                 message (messages ascend per layer).
//   k_agg         one workgroup per index chunk: worker-ordered sums in an LDS
//                 hash table, then w -= (lr/P) * u at each touched index.
//
// Keys: key(x) = bits(x) & 0x7fffffff orders fp32 magnitudes (-0 ties +0).
// All fp32 arithmetic is IEEE round to nearest even; the product and the
// subtraction of the update are separate roundings.
#include "lags_internal.h"

#include <mutex>

namespace lags {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t key_of(float x) { return __float_as_uint(x) & 0x7fffffffu; }
__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }
__device__ __forceinline__ uint32_t mbcnt(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Memory ordering.  No kernel hands data from one workgroup to another while
// both run: every such dependency is a kernel boundary (the histogram filled
// by k_main's atomics is read by k_fin_bins, and so on).  The one ordering
// inside a workgroup that plain program order does not give is k_fin_resolve
// reading counters its own threads just incremented with device atomics: each
// thread waits for its memory operations to complete, the workgroup meets at a
// barrier, and the counters are then read with device-scope atomic loads.  No
// agent-scope fence is used: on gfx950 it writes back and invalidates the
// whole L2 of the XCD.
__device__ __forceinline__ uint32_t ld_coherent(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_mem_done()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Exclusive prefix over the wave of small counts c in [0, 7].
__device__ __forceinline__ uint32_t wave_prefix3(uint32_t c, uint32_t &tot)
{
    const uint64_t b0 = __ballot(c & 1u), b1 = __ballot(c & 2u), b2 = __ballot(c & 4u);
    tot = (uint32_t)__popcll(b0) + 2u * (uint32_t)__popcll(b1) + 4u * (uint32_t)__popcll(b2);
    return mbcnt(b0) + 2u * mbcnt(b1) + 4u * mbcnt(b2);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x)
{
    const uint32_t l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (l >= (uint32_t)d) x += y;
    }
    return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
    return x;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x = max(x, (uint32_t)__shfl_xor(x, d, 64));
    return x;
}

// Block-wide exclusive scan (all NT threads must call; tmp holds NT/64 words).
template <int NT = kBlock>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t *tmp, uint32_t &total)
{
    const uint32_t w = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_scan(v);
    if (lane_id() == 63) tmp[w] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        const uint32_t t = tmp[i];
        before += (i < (int)w) ? t : 0u;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return before + inc - v;
}

// Block-wide exclusive scan of counts in [0, 7].
__device__ uint32_t block_excl_small(uint32_t c, uint32_t *tmp, uint32_t &total)
{
    const uint32_t w = threadIdx.x >> 6;
    uint32_t wt;
    const uint32_t pre = wave_prefix3(c, wt);
    if (lane_id() == 0) tmp[w] = wt;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const uint32_t t = tmp[i];
        before += (i < (int)w) ? t : 0u;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return before + pre;
}

// Exclusive scan, in item order, of the counts of n items (n may be large):
// rounds of kBlock * E items, thread t taking the E consecutive items from
// base + t * E, all requested at once (val is called at indices clamped into
// [0, n) and must only read).  out(i, excl, count) receives each item's
// exclusive prefix; it may overwrite what val reads for the same round.
// Returns the total.  All threads of a kBlock workgroup call.
template <int E, class Val, class Out>
__device__ uint32_t block_scan_items(uint32_t n, uint32_t *tmp, const Val &val, const Out &out)
{
    uint32_t carry = 0;
    for (uint32_t base = 0; base < n; base += kBlock * E) {
        const uint32_t i0 = base + threadIdx.x * E;
        uint32_t x[E];
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = val(min(i0 + e, n - 1u));
        uint32_t sum = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (i0 + e >= n) x[e] = 0;
            sum += x[e];
        }
        uint32_t tot;
        uint32_t run = carry + block_excl_scan(sum, tmp, tot);   // its barriers end the round's reads
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (i0 + e < n) out(i0 + e, run, x[e]);
            run += x[e];
        }
        carry += tot;
    }
    return carry;
}

// Find, in an LDS histogram of nbins bins (nbins a multiple of NT), the bin
// holding the rank-th largest item (rank >= 1, counting from the top bin).
// res[0] = bin, res[1] = items in higher bins.  The caller guarantees rank <=
// total.  All NT threads call; res is valid after return.
template <int NT = kBlock>
__device__ void block_find_rank(const uint32_t *hist, uint32_t nbins, uint32_t rank,
                                uint32_t *res, uint32_t *tmp)
{
    const uint32_t per = nbins / NT;
    uint32_t s = 0;
    for (uint32_t q = 0; q < per; ++q) s += hist[nbins - 1 - (threadIdx.x * per + q)];
    uint32_t tot;
    uint32_t above = block_excl_scan<NT>(s, tmp, tot);
    for (uint32_t q = 0; q < per; ++q) {
        const uint32_t b = nbins - 1 - (threadIdx.x * per + q);
        const uint32_t h = hist[b];
        if (above < rank && rank <= above + h) {
            res[0] = b;
            res[1] = above;
        }
        above += h;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Exact selection by one workgroup: MSD radix select of the rank-th largest
// 32-bit value among the items with match(i) true, in digits of at most 11
// bits.  The caller may state that every matching value has the bits of
// `known` above bit vbits (1 <= vbits <= 32); only the bits below are then
// resolved.  Returns the value; *eq_take = how many items equal to it are
// needed to reach rank (the items strictly above it number rank - eq_take);
// *eq_count (if given) = how many matching items equal it.
template <class Val, class Match>
__device__ uint32_t block_radix_select(const Val &val, const Match &match, uint32_t n, uint32_t rank,
                                       uint32_t *hist, uint32_t *tmp, uint32_t *res, uint32_t *eq_take,
                                       uint32_t *eq_count = nullptr, uint32_t vbits = 32u,
                                       uint32_t known = 0u)
{
    uint32_t prefix = (vbits >= 32u) ? 0u : (known >> vbits) << vbits;
    for (uint32_t top = vbits; top > 0u;) {   // this digit: bits [sh, top)
        const uint32_t width = min(top, 11u);
        const uint32_t sh = top - width;
        const uint32_t nb = 1u << width;
        const uint32_t nbins = max(nb, (uint32_t)kBlock);
        for (uint32_t b = threadIdx.x; b < nbins; b += kBlock) hist[b] = 0;
        __syncthreads();
        // four items per thread per round, requested together: the reads are
        // unconditional, at indices clamped into [0, n), so that no branch
        // separates them (val and match only read)
        for (uint32_t i0 = threadIdx.x; i0 < n; i0 += 4u * kBlock) {
            uint32_t v[4];
            bool ok[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t i = i0 + (uint32_t)u * kBlock;
                const uint32_t ic = min(i, n - 1u);
                v[u] = val(ic);
                ok[u] = match(ic) && i < n;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool same = (top >= 32u) ? true : ((v[u] >> top) == (prefix >> top));
                if (ok[u] && same) atomicAdd(&hist[(v[u] >> sh) & (nb - 1)], 1u);
            }
        }
        __syncthreads();
        block_find_rank(hist, nbins, rank, res, tmp);
        prefix |= res[0] << sh;
        rank -= res[1];
        // the last digit's bin holds exactly the items equal to the result
        if (sh == 0u && eq_count) *eq_count = hist[res[0]];
        __syncthreads();
        top = sh;
    }
    *eq_take = rank;
    return prefix;
}

// Bits that resolve a value known to lie in [lo, hi]: every such value has
// lo's bits above the highest bit in which lo and hi differ.
__device__ __forceinline__ uint32_t varying_bits(uint32_t lo, uint32_t hi)
{
    return max(32u - (uint32_t)__clz(lo ^ hi), 1u);
}

// Emit the selection of one layer from a value source, in index order: entries
// with key > T, then among key == T the first e (lowest index).  Writes the
// message at msg_idx/msg_val[moff ...], residual +0.0 at sent entries, and
// (WRITE_ALL) acc at the others.
template <bool WRITE_ALL, class Src>
__device__ void exact_emit(const Src &src, uint32_t n, uint32_t k, uint32_t off, uint32_t moff, uint32_t T,
                           uint32_t e, float *res_layer, uint32_t *msg_idx, float *msg_val, uint32_t *tmp)
{
    uint32_t run_eq = 0, run_sel = 0;
    for (uint32_t base = 0; base < n; base += 4u * kBlock) {
        float a[4];
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t i = base + 4u * threadIdx.x + j;
            a[j] = 0.0f;
            if (i < n) {
                a[j] = src(i);
                const uint32_t key = key_of(a[j]);
                if (key > T) gt |= 1u << j;
                else if (key == T) eq |= 1u << j;
            }
        }
        uint32_t teq;
        const uint32_t eq_before = block_excl_small((uint32_t)__popc(eq), tmp, teq);
        uint32_t sel = gt;
        uint32_t r = run_eq + eq_before;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (eq & (1u << j)) {
                if (r < e) sel |= 1u << j;
                ++r;
            }
        }
        uint32_t tsel;
        uint32_t pos = run_sel + block_excl_small((uint32_t)__popc(sel), tmp, tsel);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t i = base + 4u * threadIdx.x + j;
            if (i < n) {
                if (sel & (1u << j)) {
                    if (pos < k) {           // the selection holds exactly k entries
                        msg_idx[moff + pos] = off + i;
                        msg_val[moff + pos] = a[j];
                    }
                    res_layer[i] = 0.0f;
                    ++pos;
                } else if (WRITE_ALL) {
                    res_layer[i] = a[j];
                }
            }
        }
        run_eq += teq;
        run_sel += tsel;
    }
}

// Whole-layer exact path: select the k-th largest key of n values, then emit.
template <bool WRITE_ALL, class Src>
__device__ void exact_layer(const Src &src, uint32_t n, uint32_t k, uint32_t off, uint32_t moff,
                            float *res_layer, uint32_t *msg_idx, float *msg_val,
                            uint32_t *hist, uint32_t *tmp, uint32_t *res)
{
    uint32_t e;
    const uint32_t T = block_radix_select([&](uint32_t i) { return key_of(src(i)); },
                                          [](uint32_t) { return true; }, n, k, hist, tmp, res, &e);
    exact_emit<WRITE_ALL>(src, n, k, off, moff, T, e, res_layer, msg_idx, msg_val, tmp);
}

// A thread's run of equal bins, added to an LDS histogram with one atomic per
// run: many equal keys would otherwise serialise on one LDS address.
struct LdsRun {
    uint32_t bin = 0, n = 0;
    __device__ void add(uint32_t *hist, uint32_t b)
    {
        if (b != bin) {
            flush(hist);
            bin = b;
        }
        ++n;
    }
    __device__ void flush(uint32_t *hist)
    {
        if (n) atomicAdd(&hist[bin], n);
        n = 0;
    }
};

// ---------------------------------------------------------------------------
// k_sample: one 1024-thread workgroup per sampled layer.  The whole sample is
// requested at once (4 float4 of grad and residual per thread), each thread
// keeps its 16 keys in registers, and two 12-bit histogram passes over them
// locate the 24-bit key prefix that holds the rank-th largest sample key.
// The guess G is that prefix's lower edge, so at least as many entries reach
// G as reach the exact sample quantile.
constexpr int kSampleThreads = 1024;
constexpr uint32_t kSampleBins = 4096;

__global__ __launch_bounds__(kSampleThreads) void k_sample(SparsifyArgs a)
{
    constexpr int NT = kSampleThreads;
    constexpr int KPT = kSampleMax / NT;       // sample keys per thread
    __shared__ uint32_t hist[kSampleBins];     // first 12 key bits below the sign
    __shared__ uint32_t hist2[kSampleBins];    // the next 12, inside the chosen bin
    __shared__ uint32_t tmp[NT / 64];
    __shared__ uint32_t wmax[NT / 64];
    __shared__ uint32_t res[2];

    if (blockIdx.x == 0 && threadIdx.x < 2) a.report[kRepSampled + threadIdx.x] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 2) a.report[kRepWide] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 3) a.report[kRepFixTimeout] = 0;
    if (blockIdx.x >= a.nsampled) return;
    const uint32_t sid = a.sample_base + blockIdx.x;
    const SampledInfo S = a.sinfo[sid];
    SampledState *st = a.state + sid;
    uint32_t *stw = reinterpret_cast<uint32_t *>(st);
    for (uint32_t t = threadIdx.x; t < sizeof(SampledState) / 4; t += NT) stw[t] = 0;
    uint32_t *lh = a.hist + S.hist_off;
    for (uint32_t t = threadIdx.x; t < S.hcopies * kNBins; t += NT) lh[t] = 0;
    for (uint32_t b = threadIdx.x; b < kSampleBins; b += NT) {
        hist[b] = 0;
        hist2[b] = 0;
    }
    __syncthreads();
    if (a.force_exact) {
        // exact mode: the radix select starts from an empty prefix at rank k
        if (threadIdx.x == 0) st->xrank = S.k;
        return;
    }
    uint32_t cnt, rank, m = 0;
    uint32_t kr[KPT];             // the thread's keys (0 past the layer's end: never counted)
    LdsRun run;
    if (S.full_sample) {
        cnt = S.n;
        rank = S.k;
        // the whole layer is requested at once (cnt <= kSampleMax entries)
        constexpr int EPT = kSampleMax / NT;
        static_assert(EPT == KPT, "one key per entry");
        float gv[EPT], rv[EPT];
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const uint32_t i = threadIdx.x + u * NT;
            gv[u] = (i < cnt) ? a.grad[S.off + i] : 0.0f;
            rv[u] = (i < cnt) ? a.res[S.off + i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const uint32_t i = threadIdx.x + u * NT;
            kr[u] = 0u;
            if (i < cnt) {
                const uint32_t key = key_of(gv[u] + rv[u]);
                kr[u] = key;
                m = max(m, key);
                run.add(hist, key >> 19);
            }
        }
    } else {
        cnt = S.nchunk * kSampleChunk;
        rank = S.j;
        constexpr int QPT = kSampleMax / 4 / NT;            // float4 per thread
        static_assert(QPT * 4 == KPT, "four keys per float4");
        constexpr uint32_t QPC = kSampleChunk / 4;          // float4 per chunk
        const uint64_t span = S.b4 - S.a4 - kSampleChunk;
        const v4f *g4 = reinterpret_cast<const v4f *>(a.grad);
        const v4f *r4 = reinterpret_cast<const v4f *>(a.res);
        v4f gv[QPT], rv[QPT];
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const uint32_t qi = threadIdx.x + u * NT;
            const uint32_t c = qi / QPC, part = qi % QPC;
            const uint32_t start = S.a4 + ((uint32_t)((uint64_t)c * span / (S.nchunk - 1)) & ~3u);
            const uint32_t q = start / 4u + part;
            gv[u] = g4[q];
            rv[u] = r4[q];
        }
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const uint32_t qi = threadIdx.x + u * NT;
            const v4f acc = gv[u] + rv[u];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = key_of(acc[j]);
                kr[u * 4 + j] = key;
                m = max(m, key);
                run.add(hist, key >> 19);
            }
        }
    }
    run.flush(hist);
    {
        const uint32_t wm = wave_max(m);
        if (lane_id() == 0) wmax[threadIdx.x >> 6] = wm;
    }
    __syncthreads();
    uint32_t M = 0;              // the largest sample key
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) M = max(M, wmax[i]);
    if (rank >= cnt) {
        // k close to n: the rank is beyond the sample, so every nonzero
        // entry is a candidate (G = 0)
        if (threadIdx.x == 0) {
            uint32_t sh = 0;
            while (sh < 31u && (uint64_t)M >= ((uint64_t)kNBins << sh)) ++sh;
            st->G = 0;
            st->SH = sh;
        }
        return;
    }
    block_find_rank<NT>(hist, kSampleBins, rank, res, tmp);   // ends at a barrier
    const uint32_t b1 = res[0];
    const uint32_t rank2 = rank - res[1];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const bool in = !S.full_sample || threadIdx.x + (uint32_t)u * NT < cnt;
        if (in && (kr[u] >> 19) == b1) run.add(hist2, (kr[u] >> 7) & (kSampleBins - 1));
    }
    run.flush(hist2);
    __syncthreads();             // also: every thread has read res
    block_find_rank<NT>(hist2, kSampleBins, rank2, res, tmp);
    if (threadIdx.x == 0) {
        const uint32_t G = (b1 << 19) | (res[0] << 7);
        uint32_t sh = 0;
        while (sh < 31u && (uint64_t)(M - G) >= ((uint64_t)kNBins << sh)) ++sh;
        st->G = G;
        st->SH = sh;
    }
}

// ---------------------------------------------------------------------------
// One segment per workgroup.  The streaming pass and the exact-mode passes
// give each 4096-entry segment of a sampled layer one 256-thread workgroup
// that requests all of the segment at once: thread t holds the float4 rows
// q0 + u * kBlock + t (u < kRows) of the segment's aligned interior, and entry
// t of the layer's unaligned head (segment 0) and tail (last segment), fewer
// than 4 each.  Measured on gfx950: workgroups that each read 16 KiB per array
// in one step stream at ~6.2 TB/s, workgroups that loop over 64 KiB at ~5.5
// TB/s (the fewer address ranges in flight at once, the more each opened DRAM
// row is reused).
constexpr int kRows = kSeg / 4u / kBlock;   // float4 rows per thread
static_assert(kRows * 4 * kBlock == (int)kSeg, "a segment is kRows rows of the workgroup");
constexpr int kParts = kRows + 2;           // head, rows, tail: index order

struct SegView {
    uint32_t q0, q1;      // float4 rows [q0, q1) of the segment's aligned interior
    uint32_t hlo, nh;     // head entries [hlo, hlo + nh)
    uint32_t tlo, ntl;    // tail entries [tlo, tlo + ntl)
    __device__ uint32_t row(int u) const { return q0 + (uint32_t)u * kBlock + threadIdx.x; }
    __device__ bool row_in(int u) const { return row(u) < q1; }
};

__device__ __forceinline__ SegView seg_view(const MainWork &w, uint32_t seg)
{
    SegView v;
    const uint32_t e0 = w.a4 + seg * kSeg;
    v.q0 = e0 / 4u;
    v.q1 = (uint32_t)min((uint64_t)e0 + kSeg, (uint64_t)w.b4) / 4u;
    v.hlo = w.off;
    v.nh = seg == 0 ? w.a4 - w.off : 0u;
    v.tlo = w.b4;
    v.ntl = seg == w.nseg - 1u ? w.end - w.b4 : 0u;
    return v;
}

// Request every row of the thread at once: the loads are unconditional, at
// rows clamped into the segment (q1 > q0), so no branch separates them.  Rows
// past the segment's end (row_in false) hold a copy of its last row and must
// not be used.
template <bool NT>
__device__ __forceinline__ void seg_rows(const float *p, const SegView &v, v4f (&x)[kRows])
{
    const v4f *p4 = reinterpret_cast<const v4f *>(p);
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
        const uint32_t q = min(v.row(u), v.q1 - 1u);
        x[u] = NT ? __builtin_nontemporal_load(p4 + q) : p4[q];
    }
}

// Positions, in index order over the workgroup, of the entries each thread
// flags: c[r] (< 8) flagged entries of the thread in part r.  On return pos[r]
// is the position of the first of them; returns the workgroup's total.  All
// threads call; one barrier; wtot (LDS) may be reused only after another.
__device__ uint32_t block_positions(const uint32_t (&c)[kParts], uint32_t (&pos)[kParts],
                                    uint32_t (*wtot)[kWaves])
{
    const uint32_t ln = lane_id(), wv = threadIdx.x >> 6;
    uint32_t any = 0;
#pragma unroll
    for (int r = 0; r < kParts; ++r) any |= c[r];
    const bool wany = __ballot(any != 0u) != 0;
#pragma unroll
    for (int r = 0; r < kParts; ++r) {
        uint32_t tot = 0;
        pos[r] = wany ? wave_prefix3(c[r], tot) : 0u;
        if (ln == 0) wtot[r][wv] = tot;
    }
    __syncthreads();
    uint32_t total = 0;
#pragma unroll
    for (int r = 0; r < kParts; ++r) {
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            const uint32_t x = wtot[r][i];
            before += i < (int)wv ? x : 0u;
            tot += x;
        }
        pos[r] += total + before;
        total += tot;
    }
    return total;
}

// ---------------------------------------------------------------------------
// k_main: the streaming pass.  One workgroup per segment of a sampled layer:
// acc = grad + residual is written back to the residual buffer, and the
// entries with key >= G are candidates.  When the guess is G = 0 (most of the
// layer may be zero), only nonzero keys are candidates; the segment's zeros
// are then its length minus its candidates.  Candidates are numbered in index
// order, staged in LDS and written to the segment's slots in one burst; every
// candidate, stored or beyond the segment's slots, is also counted in one of
// the layer's histogram copies (device atomics).

__device__ __forceinline__ uint32_t cand_bin(uint32_t key, uint32_t G, uint32_t SH)
{
    return min((key - G) >> SH, kNBins - 1u);
}

constexpr uint32_t kHeavySeg = 256;   // candidates of a segment counted in LDS beyond this

template <bool NTS>
__device__ void sampled_segment(const SparsifyArgs &a, const MainWork &w, uint32_t seg,
                                const SampledState *st, uint32_t *hist, uint2 *stage,
                                uint32_t (*wtot)[kWaves], uint32_t *lh)
{
    const uint32_t t = threadIdx.x;
    const SegView sv = seg_view(w, seg);
    v4f acc[kRows], rv[kRows];
    seg_rows<true>(a.grad, sv, acc);
    seg_rows<true>(a.res, sv, rv);
    float hv = 0.0f, tv = 0.0f;
    if (t < sv.nh) hv = a.grad[sv.hlo + t] + a.res[sv.hlo + t];
    if (t < sv.ntl) tv = a.grad[sv.tlo + t] + a.res[sv.tlo + t];
    const uint32_t G = st->G, SH = st->SH;
    const uint32_t Gs = G ? G : 1u;   // candidates: key >= Gs

    v4f *r4 = reinterpret_cast<v4f *>(a.res);
    uint32_t fl = 0;   // bit 4u + j: entry j of row u
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
        acc[u] = acc[u] + rv[u];
        if (sv.row_in(u)) {
            if (NTS) __builtin_nontemporal_store(acc[u], r4 + sv.row(u));
            else r4[sv.row(u)] = acc[u];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (key_of(acc[u][j]) >= Gs) fl |= 1u << (4 * u + j);
        }
    }
    if (t < sv.nh) a.res[sv.hlo + t] = hv;
    if (t < sv.ntl) a.res[sv.tlo + t] = tv;
    uint32_t c[kParts], pos[kParts];
    c[0] = (t < sv.nh && key_of(hv) >= Gs) ? 1u : 0u;
#pragma unroll
    for (int u = 0; u < kRows; ++u) c[1 + u] = (uint32_t)__popc((fl >> (4 * u)) & 15u);
    c[kParts - 1] = (t < sv.ntl && key_of(tv) >= Gs) ? 1u : 0u;
    const uint32_t total = block_positions(c, pos, wtot);

    const uint32_t cap = w.cap;
    const uint64_t slot0 = (((uint64_t)w.slot_hi << 32) | w.slot_lo) + (uint64_t)seg * cap;
    // a segment with many candidates (equal keys, clustered large values)
    // counts them in the workgroup's LDS histogram lh and adds its nonzero
    // bins to the layer's copy once: thousands of device atomics on one
    // address serialise
    const bool heavy = total > kHeavySeg;   // uniform over the workgroup
    if (heavy) {
        for (uint32_t b = t; b < kNBins; b += kBlock) lh[b] = 0;
        __syncthreads();
    }
    uint32_t run_b = 0, run_n = 0;      // heavy: a run of one bin among the thread's candidates
    auto put = [&](uint32_t p, uint32_t idx, float v) {
        const uint2 e = make_uint2(idx, __float_as_uint(v));
        if (p < kCapMax) stage[p] = e;
        else if (p < cap) a.slots[slot0 + p] = e;   // only layers of <= kSampleMax entries
                                                     // have more than kCapMax slots
        const uint32_t bin = cand_bin(key_of(v), G, SH);
        if (heavy) {
            if (bin != run_b) {
                if (run_n) atomicAdd(&lh[run_b], run_n);
                run_b = bin;
                run_n = 0;
            }
            ++run_n;
        } else {
            atomicAdd(&hist[bin], 1u);
        }
    };
    if (c[0]) put(pos[0], sv.hlo + t, hv);
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
        uint32_t p = pos[1 + u];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if ((fl >> (4 * u + j)) & 1u) put(p++, 4u * sv.row(u) + j, acc[u][j]);
    }
    if (c[kParts - 1]) put(pos[kParts - 1], sv.tlo + t, tv);
    if (heavy && run_n) atomicAdd(&lh[run_b], run_n);
    __syncthreads();
    // a segment with more candidates than slots keeps only the first cap
    // (the finishing kernels re-read it)
    const uint32_t ns = min(total, min(cap, kCapMax));
    for (uint32_t i = t; i < ns; i += kBlock) a.slots[slot0 + i] = stage[i];
    if (t == 0) a.seg_count[w.seg_base + seg] = total;
    if (heavy)
        for (uint32_t b = t; b < kNBins; b += kBlock)
            if (lh[b]) atomicAdd(&hist[b], lh[b]);
}

__device__ void dense_tile(const SparsifyArgs &a, const MainWork &w, uint32_t part, uint32_t nparts);

// Grid: kTileSegs workgroups per work entry.  A sampled tile's workgroup
// takes one segment; a k == n tile is split into kTileSegs equal parts.
// NTS: the residual is stored non-temporally (streams beyond the caches);
// otherwise with ordinary stores, which keep a layout small enough for the
// 256 MB cache there for the finishing kernels' scattered residual writes.
template <bool NTS>
__global__ __launch_bounds__(kBlock) void k_main(SparsifyArgs a)
{
    __shared__ uint2 stage[kCapMax];
    __shared__ uint32_t wtot[kParts][kWaves];
    extern __shared__ uint32_t lh[];     // the launch's LDS pad: kNBins words at least

    const uint32_t part = blockIdx.x % kTileSegs;
    const MainWork w = a.main_work[a.main_base + blockIdx.x / kTileSegs];

    if (w.cls == kClsSampled) {
        const uint32_t seg = w.tile * kTileSegs + part;
        // consecutive workgroups take consecutive histogram copies
        if (seg < w.nseg)
            sampled_segment<NTS>(a, w, seg, a.state + w.sid,
                            a.hist + w.hist_off + (blockIdx.x & (w.hcopies - 1u)) * kNBins, stage, wtot, lh);
        return;
    }

    dense_tile(a, w, part, kTileSegs);
}

// A k == n layer: every entry of part `part` (of nparts) of tile w.tile is sent.
__device__ void dense_tile(const SparsifyArgs &a, const MainWork &w, uint32_t part, uint32_t nparts)
{
    const LayerInfo L = a.linfo[w.layer];
    const uint32_t width = kDenseTile / nparts;
    const uint64_t end = (uint64_t)L.off + L.n;
    const uint32_t lo = (uint32_t)min((uint64_t)L.off + (uint64_t)w.tile * kDenseTile + (uint64_t)part * width, end);
    const uint32_t hi = (uint32_t)min((uint64_t)lo + width, end);
    // batches of EPT entries per thread, all loads of a batch in flight
    // before its stores (a store to the residual may alias a later load);
    // the loads are unconditional, at indices clamped into the range, so that
    // no branch separates them
    constexpr int EPT = 16;
    for (uint32_t i0 = lo + threadIdx.x; i0 < hi; i0 += EPT * kBlock) {
        float x[EPT];
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const uint32_t i = min(i0 + u * kBlock, hi - 1u);
            x[u] = a.grad[i] + a.res[i];
        }
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const uint32_t i = i0 + u * kBlock;
            if (i < hi) {
                a.res[i] = 0.0f;
                a.msg_idx[L.moff + (i - L.off)] = i;
                a.msg_val[L.moff + (i - L.off)] = x[u];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Finishing kernels.  fin_work lists, per sampled layer, workgroups of f.grain
// (at most kFinSegs) consecutive segments; each wave of a workgroup takes
// every kWaves-th.  Each entry carries everything static the workgroup needs, so
// its first load is followed directly by the per-call loads.

__device__ __forceinline__ uint32_t seg_of(const FinWork &f, uint32_t i)
{
    if (i < f.a4) return 0;
    return min((i - f.a4) / kSeg, f.nseg - 1u);
}

// Entries of segment s of the layer (segment 0 also holds the unaligned head,
// the last one the tail).
__device__ __forceinline__ uint32_t seg_len(const FinWork &f, uint32_t s)
{
    const uint32_t end = f.off + f.n, b4 = end & ~3u;
    const uint32_t lo = f.a4 + s * kSeg;
    uint32_t len = (uint32_t)min((uint64_t)lo + kSeg, (uint64_t)b4) - lo;
    if (s == 0) len += f.a4 - f.off;
    if (s == f.nseg - 1u) len += end - b4;
    return len;
}

// The static fields of sampled layer sid's finishing work (its first
// workgroup's: seg0 = 0), from the layer's own entry.
__device__ __forceinline__ FinWork layer_fin(const SampledInfo &S, uint32_t sid)
{
    FinWork f{};
    f.sid = sid;
    f.seg0 = 0;
    f.nseg = S.nseg;
    f.seg_base = S.seg_base;
    f.cap = S.cap;
    f.slot_lo = S.slot_lo;
    f.slot_hi = S.slot_hi;
    f.fin_first = S.fin_first;
    f.off = S.off;
    f.n = S.n;
    f.moff = S.moff;
    f.k = S.k;
    f.tbin_cap = S.tbin_cap;
    f.grain = S.grain;
    f.a4 = S.a4;
    f.hist_off = S.hist_off;
    f.hcopies = S.hcopies;
    return f;
}

// Hand a sampled layer whose guess failed to the fallback of k_fin_emit:
// status kStFix, one more failed layer in the range's count, the layer's
// fallback histograms cleared.  All NT threads of the workgroup call.
// [klo, khi]: the keys the layer's threshold is known to lie between (the
// whole range when nothing is known).
template <int NT>
__device__ void mark_for_fix(const SparsifyArgs &a, uint32_t sid, uint32_t klo = 0u,
                             uint32_t khi = 0x7fffffffu)
{
    uint32_t *fb = a.fb + (uint64_t)sid * kFbWords;
    for (uint32_t t = threadIdx.x; t < kFbCount; t += NT) fb[t] = 0;
    if (threadIdx.x == 0) {
        a.state[sid].fix_klo = klo;
        a.state[sid].fix_khi = khi;
        a.state[sid].status = kStFix;
        atomicAdd(&a.state[a.sample_base].nfail, 1u);
        atomicAdd(&a.report[kRepExact], 1u);
    }
}

// The threshold-bin decision for one sampled layer, after the streaming pass
// has filled the layer's histogram copies, by the NT threads of one
// workgroup: sum the copies into hist (LDS; eight loads in flight per thread),
// then the layer's status: zero mode (G = 0 and fewer than k nonzero keys),
// the fallback (too few candidates above a nonzero G, or a threshold bin
// larger than the layer's list), or Ok with the bin bstar holding the k-th
// largest candidate and the candidate count above it.  With `write` the
// workgroup records the decision in the layer's state and the report (and
// marks the layer for the fallback); every workgroup that calls it for the
// layer reaches the same decision.
struct BinsDecision {
    uint32_t status, bstar, c_above;
};

template <int NT>
__device__ BinsDecision layer_bins(const SparsifyArgs &a, uint32_t sid, uint32_t hist_off, uint32_t hcopies,
                                   uint32_t tbin_cap, uint32_t k, uint32_t G, uint32_t SH, uint32_t *hist,
                                   uint32_t *tmp, uint32_t *res, bool write)
{
    SampledState *st = a.state + sid;
    const uint32_t *lh = a.hist + hist_off;
    // thread t sums bins t + i * NT over the copies, all of a round's loads
    // in flight together: 16 per thread with 1024 threads, 8 with 256 (their
    // register budget), one copy per round
    constexpr int BPT = kNBins / NT;
    constexpr uint32_t R = (NT >= 1024 ? 16u : 8u) / BPT;   // copies per round
    static_assert(BPT * NT == (int)kNBins && R >= 1u, "bins split evenly");
    uint32_t h[BPT];
#pragma unroll
    for (int i = 0; i < BPT; ++i) h[i] = 0;
    for (uint32_t c0 = 0; c0 < hcopies; c0 += R) {
        uint32_t v[R][BPT];
#pragma unroll
        for (uint32_t u = 0; u < R; ++u)
#pragma unroll
            for (int i = 0; i < BPT; ++i)
                v[u][i] = (c0 + u < hcopies) ? lh[(c0 + u) * kNBins + threadIdx.x + i * NT] : 0u;
#pragma unroll
        for (uint32_t u = 0; u < R; ++u)
#pragma unroll
            for (int i = 0; i < BPT; ++i) h[i] += v[u][i];
    }
    uint32_t part = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        hist[threadIdx.x + i * NT] = h[i];
        part += h[i];
    }
    uint32_t C;
    block_excl_scan<NT>(part, tmp, C);    // also orders the LDS writes above
    if (C < k && G != 0) {
        if (write) {
            mark_for_fix<NT>(a, sid);
            if (threadIdx.x == 0) atomicAdd(&a.report[kRepSampled], 1u);
        }
        return {kStFix, 0u, 0u};
    }
    if (C < k) {
        // G = 0 and fewer than k nonzero keys: the k-th largest key is 0, so
        // every stored (nonzero) candidate is sent, plus the k - C zeros of
        // lowest index
        if (write && threadIdx.x == 0) {
            st->status = kStZero;
            st->c_above = C;
            atomicAdd(&a.report[kRepSampled], 1u);
        }
        return {kStZero, 0u, C};
    }
    block_find_rank<NT>(hist, kNBins, k, res, tmp);
    const uint32_t bstar = res[0], above = res[1];
    if (hist[bstar] > tbin_cap) {
        // the threshold bin holds more candidates than the layer's list (many
        // equal keys): the fallback selects the layer, knowing that the
        // threshold lies in this bin
        if (write) {
            const uint64_t blo = (uint64_t)G + ((uint64_t)bstar << SH);
            const uint32_t klo = (uint32_t)min(blo, (uint64_t)0x7fffffffu);
            const uint32_t khi = (bstar + 1u >= kNBins)
                                     ? 0x7fffffffu
                                     : (uint32_t)min(blo + (1ull << SH) - 1u, (uint64_t)0x7fffffffu);
            mark_for_fix<NT>(a, sid, klo, khi);
            if (threadIdx.x == 0) atomicAdd(&a.report[kRepSampled], 1u);
        }
        return {kStFix, 0u, 0u};
    }
    if (write && threadIdx.x == 0) {
        st->bstar = bstar;
        st->c_above = above;
        st->status = kStOk;
        atomicAdd(&a.report[kRepSampled], 1u);
    }
    return {kStOk, bstar, above};
}

// k_fin_bins: one 1024-thread workgroup per sampled layer with more than
// kSelfBinsCopies histogram copies (the finishing workgroups of a layer with
// fewer decide for themselves in k_fin_select).
constexpr int kBinsThreads = 1024;

__global__ __launch_bounds__(kBinsThreads) void k_fin_bins(SparsifyArgs a)
{
    constexpr int NT = kBinsThreads;
    __shared__ uint32_t hist[kNBins];
    __shared__ uint32_t tmp[NT / 64];
    __shared__ uint32_t res[2];
    if (blockIdx.x >= a.nsampled) return;
    const uint32_t sid = a.sample_base + blockIdx.x;
    const SampledInfo S = a.sinfo[sid];
    if (S.hcopies <= kSelfBinsCopies) return;
    const SampledState *st = a.state + sid;
    layer_bins<NT>(a, sid, S.hist_off, S.hcopies, S.tbin_cap, S.k, st->G, st->SH, hist, tmp, res, true);
}

// Walk segment seg of a sampled layer in index order, one wave: fn(valid,
// idx, v) is called wave-uniformly for the unaligned head (segment 0), each
// row of 64 float4 of the aligned interior, and the unaligned tail (last
// segment); lane entries j with (valid >> j) & 1 are real.  Values come from
// the residual buffer, which holds acc after the streaming pass.
template <class F>
__device__ void walk_segment(const SparsifyArgs &a, const FinWork &f, uint32_t seg, F &&fn)
{
    const uint32_t ln = lane_id();
    const uint32_t end = f.off + f.n, b4 = end & ~3u;
    uint32_t idx[4];
    float v[4];
    if (seg == 0 && f.off < f.a4) {
        const uint32_t i = f.off + ln;
        const bool in = i < f.a4;
        idx[0] = idx[1] = idx[2] = idx[3] = i;
        v[0] = in ? a.res[i] : 0.0f;
        v[1] = v[2] = v[3] = 0.0f;
        fn(in ? 1u : 0u, idx, v);
    }
    const uint32_t lo = f.a4 + seg * kSeg;
    const uint32_t q0 = lo / 4u;
    const uint32_t q1 = (uint32_t)min((uint64_t)lo + kSeg, (uint64_t)b4) / 4u;
    const v4f *r4 = reinterpret_cast<const v4f *>(a.res);
    for (uint32_t qb = q0; qb < q1; qb += 64u) {
        const uint32_t q = qb + ln;
        const bool in = q < q1;
        const v4f x = in ? r4[q] : (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            idx[j] = 4u * q + j;
            v[j] = x[j];
        }
        fn(in ? 0xfu : 0u, idx, v);
    }
    if (seg == f.nseg - 1u && b4 < end) {
        const uint32_t i = b4 + ln;
        const bool in = i < end;
        idx[0] = idx[1] = idx[2] = idx[3] = i;
        v[0] = in ? a.res[i] : 0.0f;
        v[1] = v[2] = v[3] = 0.0f;
        fn(in ? 1u : 0u, idx, v);
    }
}

// The segments a wave handles in a finishing workgroup, with their candidate
// counts and first 64 slots loaded up front so that one memory round trip
// serves all of them.
constexpr int kSegsPerWave = kFinSegs / kWaves;
// A workgroup of at most kFinSegs / 2 segments gives each wave at most half
// of the entries of first[]: the other half holds the next 64 slots of the
// wave's segments (layers whose segments often hold 64-128 candidates, as at
// rho = 1/100, then need no second round trip).
struct WaveSegs {
    static constexpr int H = kSegsPerWave / 2;
    uint32_t s0;                      // first segment of the workgroup
    uint32_t wave;
    uint32_t send;                    // end of the workgroup's segments
    uint32_t raw[kSegsPerWave];       // candidates of the segment (may exceed its slots)
    uint32_t cap;                     // slots per segment
    bool wide;                        // first[H + i] holds slots 64..127 of segment i
    uint2 first[kSegsPerWave];
    __device__ uint32_t seg(int i) const { return s0 + wave + (uint32_t)i * kWaves; }
    __device__ bool valid(int i) const { return seg(i) < send; }
    __device__ const uint2 *slots(const SparsifyArgs &a, const FinWork &f, int i) const
    {
        return a.slots + (((uint64_t)f.slot_hi << 32) | f.slot_lo) + (uint64_t)seg(i) * f.cap;
    }
    __device__ uint32_t cnt(int i) const { return min(raw[i], cap); }   // stored candidates
    __device__ bool full(int i) const { return raw[i] > cap; }          // re-read from acc
    // slot p (< cnt(i)) of segment i; sl = slots(a, f, i)
    __device__ uint2 at(int i, uint32_t p, const uint2 *sl) const
    {
        if (p < 64u) return first[i];
        if (wide && i < H && p < 128u) {
            uint2 r = first[0];               // (a select over constant indices: first[]
#pragma unroll                                // stays in registers)
            for (int j = H; j < kSegsPerWave; ++j)
                if (j == i + H) r = first[j];
            return r;
        }
        return sl[p];
    }
    __device__ void load(const SparsifyArgs &a, const FinWork &f, uint32_t wv, uint32_t ln)
    {
        s0 = f.seg0;
        wave = wv;
        send = min(f.seg0 + f.grain, f.nseg);
        cap = f.cap;
        wide = f.grain <= (uint32_t)(kFinSegs / 2);
#pragma unroll
        for (int i = 0; i < kSegsPerWave; ++i) raw[i] = valid(i) ? a.seg_count[f.seg_base + seg(i)] : 0u;
#pragma unroll
        for (int i = 0; i < kSegsPerWave; ++i) {
            if (i >= H && wide) {           // (segment i is past the workgroup's end)
                const int i0 = i - H;
                first[i] = (64u + ln < min(raw[i0], f.cap)) ? slots(a, f, i0)[64u + ln] : make_uint2(0, 0);
            } else {
                first[i] = (ln < min(raw[i], f.cap)) ? slots(a, f, i)[ln] : make_uint2(0, 0);
            }
        }
    }
};
static_assert(kSegsPerWave % 2 == 0 && kFinSegsSmall <= kFinSegs / 2, "the small grain uses half of first[]");

// k_fin_select: per segment, the count of candidates above the threshold bin;
// the threshold bin's candidates are gathered into the layer's list (one
// reservation per wave).  Per workgroup, the total above the bin.
// At most 64 VGPRs (8 waves per SIMD; 12 bytes spill): this latency-bound pass
// measured 62 us at 74 VGPRs, 58 at 66 and 55 at 64 on the 1.31B-entry layout.
__global__ __launch_bounds__(kBlock, 8) void k_fin_select(SparsifyArgs a)
{
    __shared__ uint32_t wtot[kWaves];
    __shared__ uint32_t wzero[kWaves];
    __shared__ uint32_t bins[kNBins];
    __shared__ uint32_t btmp[kWaves];
    __shared__ uint32_t bres[2];
    const FinWork f = a.fin_work[a.fin_base + blockIdx.x];
    SampledState *st = a.state + f.sid;
    const uint32_t ln = lane_id();
    const uint32_t wv = threadIdx.x >> 6;
    WaveSegs ws;
    ws.load(a, f, wv, ln);            // issued before the layer's status arrives
    const uint32_t G = st->G, SH = st->SH;
    uint32_t status, bstar;
    if (f.hcopies <= kSelfBinsCopies) {
        // few histogram copies: every finishing workgroup of the layer sums
        // them and decides; the layer's first records the decision
        const BinsDecision d = layer_bins<kBlock>(a, f.sid, f.hist_off, f.hcopies, f.tbin_cap, f.k, G, SH, bins,
                                                  btmp, bres, f.seg0 == 0u);
        status = d.status;
        bstar = d.bstar;
    } else {
        status = st->status;          // uniform over the workgroup
        bstar = st->bstar;
    }
    if (status == kStZero) {
        // every candidate (every nonzero entry) is sent; count the
        // workgroup's zeros
        uint32_t wsum = 0, wz = 0;
        for (int i = 0; i < kSegsPerWave; ++i) {
            if (!ws.valid(i)) continue;
            if (ln == 0) a.seg_sel[f.seg_base + ws.seg(i)] = ws.raw[i];
            wsum += ws.raw[i];
            wz += seg_len(f, ws.seg(i)) - ws.raw[i];
        }
        if (ln == 0) {
            wtot[wv] = wsum;
            wzero[wv] = wz;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t t = 0, z = 0;
            for (int i = 0; i < kWaves; ++i) {
                t += wtot[i];
                z += wzero[i];
            }
            a.fin_total[a.fin_base + blockIdx.x] = t;
            a.fin_eq[a.fin_base + blockIdx.x] = z;
        }
        return;
    }
    if (status != kStOk) return;      // the fallback takes the layer
    const uint32_t Gs = G ? G : 1u;           // candidates: key >= Gs
    // pass 1: per segment, candidates above the threshold bin; per lane,
    // candidates in it.  A segment with more candidates than slots is
    // re-read from acc.
    uint32_t wsum = 0, nt = 0;
#pragma unroll
    for (int i = 0; i < kSegsPerWave; ++i) {
        if (!ws.valid(i)) continue;
        uint32_t D = 0;
        if (ws.full(i)) {
            walk_segment(a, f, ws.seg(i), [&](uint32_t valid, const uint32_t *, const float *v) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t key = key_of(v[j]);
                    if ((valid & (1u << j)) && key >= Gs) {
                        const uint32_t bin = cand_bin(key, G, SH);
                        D += (bin > bstar) ? 1u : 0u;
                        nt += (bin == bstar) ? 1u : 0u;
                    }
                }
            });
        } else {
            const uint32_t cnt = ws.cnt(i);
            const uint2 *slots = ws.slots(a, f, i);
            for (uint32_t p = ln; p < cnt; p += 64) {
                const uint2 c = ws.at(i, p, slots);
                const uint32_t bin = cand_bin(c.y & 0x7fffffffu, G, SH);
                D += (bin > bstar) ? 1u : 0u;
                nt += (bin == bstar) ? 1u : 0u;
            }
        }
        D = wave_sum(D);
        if (ln == 0) a.seg_sel[f.seg_base + ws.seg(i)] = D;
        wsum += D;
    }
    // pass 2: one reservation per wave in the layer's threshold-bin list
    const uint32_t incl = wave_incl_scan(nt);
    const uint32_t wt = __shfl(incl, 63, 64);
    if (wt) {
        uint32_t base = 0;
        if (ln == 0) base = atomicAdd(&st->tbin_n, wt);
        uint32_t t = __shfl(base, 0, 64) + incl - nt;
        uint2 *tb = a.tbin + (((uint64_t)f.slot_hi << 32) | f.slot_lo);
#pragma unroll
        for (int i = 0; i < kSegsPerWave; ++i) {
            if (!ws.valid(i)) continue;
            if (ws.full(i)) {
                walk_segment(a, f, ws.seg(i), [&](uint32_t valid, const uint32_t *idx, const float *v) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t key = key_of(v[j]);
                        if ((valid & (1u << j)) && key >= Gs && cand_bin(key, G, SH) == bstar) {
                            if (t < f.tbin_cap) tb[t] = make_uint2(idx[j], __float_as_uint(v[j]));
                            ++t;
                        }
                    }
                });
                continue;
            }
            const uint32_t cnt = ws.cnt(i);
            const uint2 *slots = ws.slots(a, f, i);
            for (uint32_t p = ln; p < cnt; p += 64) {
                const uint2 c = ws.at(i, p, slots);
                if (cand_bin(c.y & 0x7fffffffu, G, SH) == bstar) {
                    if (t < f.tbin_cap) tb[t] = c;
                    ++t;
                }
            }
        }
    }
    if (ln == 0) wtot[wv] = wsum;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int i = 0; i < kWaves; ++i) t += wtot[i];
        a.fin_total[a.fin_base + blockIdx.x] = t;
    }
}

// Exact threshold and tie cut among the h entries of the threshold bin (the
// need-th largest key; among keys equal to it, the lowest indices first; a
// bin of at most kBlock entries by ranking every entry, a larger one by radix
// selects), and
// the per-segment and per-workgroup counts of the bin's selected entries:
// added to seg_sel, and to the finishing workgroups' counts in LDS (wcnt,
// which may alias hist) or, without wcnt, to fin_total in device memory.
// Every key of the bin lies in [klo, khi] and every index in the layer
// [f.off, f.off + f.n), so only the bits that vary there are resolved.  When
// all keys equal to the threshold are taken, the cut is the largest index.
template <class KeyF, class IdxF>
__device__ void resolve_tbin(const SparsifyArgs &a, const FinWork &f, uint32_t nfb, uint32_t h, uint32_t need,
                             uint32_t klo, uint32_t khi, const KeyF &key, const IdxF &idx,
                             uint32_t *hist, uint32_t *tmp, uint32_t *res, uint32_t *wcnt,
                             uint32_t &T_out, uint32_t &cut_out)
{
    uint32_t T, cut = 0xffffffffu;
    if (h <= (uint32_t)kBlock) {
        // a small bin: one entry per thread, ranked against all h entries in
        // (key descending, index ascending) order (the entries' indices are
        // distinct); the entry of rank need - 1 is the threshold key and,
        // unless every entry equal to it is taken, the cut
        if (threadIdx.x == 0) {
            res[0] = 0u;
            res[1] = 0xffffffffu;
        }
        __syncthreads();
        const bool in = threadIdx.x < h;
        const uint32_t km = in ? key(threadIdx.x) : 0u, im = in ? idx(threadIdx.x) : 0u;
        uint32_t rank = 0;
        for (uint32_t j = 0; j < h; ++j) {
            const uint32_t kj = key(j), ij = idx(j);
            rank += (kj > km || (kj == km && ij < im)) ? 1u : 0u;
        }
        if (in && rank == need - 1u) {
            res[0] = km;
            res[1] = im;
        }
        __syncthreads();
        T = res[0];
        if (__syncthreads_or(in && km == T && rank >= need)) cut = res[1];
    } else {
        uint32_t e, eq;
        T = block_radix_select(key, [](uint32_t) { return true; }, h, need, hist, tmp, res, &e, &eq,
                               varying_bits(klo, khi), klo);
        if (e < eq) {
            // e-th smallest index among keys == T  ==  e-th largest of ~index
            const uint32_t nlo = ~(f.off + (f.n - 1u)), nhi = ~f.off;
            uint32_t e2;
            cut = ~block_radix_select([&](uint32_t p) { return ~idx(p); },
                                      [&](uint32_t p) { return key(p) == T; }, h, e, hist, tmp, res, &e2,
                                      nullptr, varying_bits(nlo, nhi), nlo);
        }
    }
    if (wcnt) {               // the selects are done with hist (their last barrier)
        for (uint32_t b = threadIdx.x; b < nfb; b += kBlock) wcnt[b] = 0;
        __syncthreads();
    }
    for (uint32_t p = threadIdx.x; p < h; p += kBlock) {
        const uint32_t kp = key(p), ip = idx(p);
        if (kp > T || (kp == T && ip <= cut)) {
            const uint32_t sg = seg_of(f, ip);
            atomicAdd(&a.seg_sel[f.seg_base + sg], 1u);
            if (wcnt) atomicAdd(&wcnt[sg / f.grain], 1u);
            else atomicAdd(&a.fin_total[f.fin_first + sg / f.grain], 1u);
        }
    }
    if (wcnt) __syncthreads();
    T_out = T;
    cut_out = cut;
}

// k_fin_resolve: one workgroup per sampled layer.  Resolves the exact
// threshold key T and the tie cut inside the threshold bin and turns the
// per-workgroup counts into message offsets.  A layer whose guess failed
// (status not Ok, or a threshold bin above its list's capacity) is left to
// the fallback in k_fin_emit.
__global__ __launch_bounds__(kBlock) void k_fin_resolve(SparsifyArgs a)
{
    static_assert(kSmallMax <= 2 * kTbinCap, "a small layer's values fit the threshold-bin arrays");
    __shared__ uint32_t hist[kNBins];
    __shared__ uint32_t pool[2 * kTbinCap];
    __shared__ uint32_t tmp[kWaves];
    __shared__ uint32_t res[2];
    uint32_t *tk = pool, *ti = pool + kTbinCap;

    if (blockIdx.x >= a.nsampled) {
        // a small layer, start to finish: acc in LDS, exact radix select
        const LayerInfo L = a.small_info[a.small_base + (blockIdx.x - a.nsampled)];
        float *acc_s = reinterpret_cast<float *>(pool);
        {
            constexpr int EPT = kSmallMax / kBlock;   // the whole layer requested at once
            float gv[EPT], rv[EPT];
#pragma unroll
            for (int u = 0; u < EPT; ++u) {
                const uint32_t i = threadIdx.x + u * kBlock;
                gv[u] = (i < L.n) ? a.grad[L.off + i] : 0.0f;
                rv[u] = (i < L.n) ? a.res[L.off + i] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < EPT; ++u) {
                const uint32_t i = threadIdx.x + u * kBlock;
                if (i < L.n) acc_s[i] = gv[u] + rv[u];
            }
        }
        __syncthreads();
        if (L.k == L.n) {
            for (uint32_t i = threadIdx.x; i < L.n; i += kBlock) {
                a.msg_idx[L.moff + i] = L.off + i;
                a.msg_val[L.moff + i] = acc_s[i];
                a.res[L.off + i] = 0.0f;
            }
            return;
        }
        exact_layer<true>([&](uint32_t i) { return acc_s[i]; }, L.n, L.k, L.off, L.moff,
                          a.res + L.off, a.msg_idx, a.msg_val, hist, tmp, res);
        return;
    }

    const uint32_t sid = a.sample_base + blockIdx.x;
    SampledState *st = a.state + sid;
    const uint32_t status = st->status;      // requested with the layer's entry
    const uint32_t h = st->tbin_n;
    const SampledInfo S = a.sinfo[sid];
    const FinWork f = layer_fin(S, sid);
    const uint2 *tb = a.tbin + (((uint64_t)S.slot_hi << 32) | S.slot_lo);
    // requested before the status and the list's length arrive: the list's
    // first entries and the finishing workgroups' counts (all of them when
    // their LDS counts fit hist)
    constexpr int EPT = kTbinCap / kBlock;
    constexpr int FPT = kNBins / kBlock;
    const uint32_t hcap = min(S.tbin_cap, kTbinCap);      // >= 1
    uint2 c[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) c[u] = tb[min(threadIdx.x + u * kBlock, hcap - 1u)];
    const uint32_t nfb = S.fin_nblocks;
    const bool lds_counts = nfb <= kNBins;
    uint32_t ft[FPT];
#pragma unroll
    for (int e = 0; e < FPT; ++e) ft[e] = a.fin_total[S.fin_first + min(threadIdx.x * FPT + e, nfb - 1u)];

    if (status == kStZero) {
        // T = 0: the first e zeros (index order) are sent with every stored
        // candidate.  Per finishing workgroup: zeros before it, zeros it
        // sends, message offset.
        const uint32_t e = S.k - st->c_above;
        uint32_t zcarry = 0, carry = 0;
        for (uint32_t base = 0; base < S.fin_nblocks; base += kBlock) {
            const uint32_t b = base + threadIdx.x;
            const bool in = b < S.fin_nblocks;
            const uint32_t z = in ? a.fin_eq[S.fin_first + b] : 0u;
            const uint32_t t = in ? a.fin_total[S.fin_first + b] : 0u;
            uint32_t ztot, tot;
            const uint32_t zpre = zcarry + block_excl_scan(z, tmp, ztot);
            const uint32_t take = (zpre >= e) ? 0u : min(z, e - zpre);
            const uint32_t ex = block_excl_scan(t + take, tmp, tot);
            if (in) {
                a.fin_total[S.fin_first + b] = carry + ex;
                a.fin_eq[S.fin_first + b] = zpre;
            }
            zcarry += ztot;
            carry += tot;
        }
        if (threadIdx.x == 0) {
            st->T = 0;
            st->idx_cut = e;          // zero mode: the number of zeros sent
        }
        return;
    }

    if (status != kStOk) return;       // kStFix: the fallback takes the layer

    // resolve the threshold inside bin bstar: in LDS when the bin fits,
    // otherwise straight from the workspace
    const uint32_t need = S.k - st->c_above;
    // the keys of bin bstar: (key - G) >> SH == bstar, or above for the last bin
    const uint32_t bstar = st->bstar;
    const uint64_t blo = (uint64_t)st->G + ((uint64_t)bstar << st->SH);
    const uint32_t klo = (uint32_t)min(blo, (uint64_t)0x7fffffffu);
    const uint32_t khi = (bstar + 1u >= kNBins) ? 0x7fffffffu
                                                : (uint32_t)min(blo + (1ull << st->SH) - 1u, (uint64_t)0x7fffffffu);
    if (h > S.tbin_cap) {
        // more threshold-bin entries than the list holds (k_fin_bins sees this
        // from the histogram; kept as a guard): the fallback selects the layer
        mark_for_fix<kBlock>(a, sid, klo, khi);
        return;
    }
    uint32_t T, idx_cut;
    uint32_t *wcnt = lds_counts ? hist : nullptr;
    if (h <= kTbinCap) {
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const uint32_t p = threadIdx.x + u * kBlock;
            if (p < h) {
                ti[p] = c[u].x;
                tk[p] = c[u].y & 0x7fffffffu;
            }
        }
        __syncthreads();
        resolve_tbin(a, f, nfb, h, need, klo, khi, [&](uint32_t p) { return tk[p]; },
                     [&](uint32_t p) { return ti[p]; }, hist, tmp, res, wcnt, T, idx_cut);
    } else {
        if (threadIdx.x == 0) atomicAdd(&a.report[kRepWide], 1u);
        resolve_tbin(a, f, nfb, h, need, klo, khi, [&](uint32_t p) { return tb[p].y & 0x7fffffffu; },
                     [&](uint32_t p) { return tb[p].x; }, hist, tmp, res, wcnt, T, idx_cut);
    }
    // per-workgroup totals (above the bin, plus the bin's selected entries)
    // -> exclusive message offsets (in place)
    if (lds_counts) {
        uint32_t v[FPT], sum = 0;
#pragma unroll
        for (int e = 0; e < FPT; ++e) {
            const uint32_t b = threadIdx.x * FPT + e;
            v[e] = b < nfb ? ft[e] + wcnt[b] : 0u;
            sum += v[e];
        }
        uint32_t tot;
        uint32_t run = block_excl_scan(sum, tmp, tot);
#pragma unroll
        for (int e = 0; e < FPT; ++e) {
            const uint32_t b = threadIdx.x * FPT + e;
            if (b < nfb) a.fin_total[S.fin_first + b] = run;
            run += v[e];
        }
    } else {
        // the workgroup's own atomics above complete before the scan reads the totals
        wait_mem_done();
        __syncthreads();
        block_scan_items<16>(
            nfb, tmp, [&](uint32_t b) { return ld_coherent(&a.fin_total[S.fin_first + b]); },
            [&](uint32_t b, uint32_t ex, uint32_t) { a.fin_total[S.fin_first + b] = ex; });
    }
    if (threadIdx.x == 0) {
        st->T = T;
        st->idx_cut = idx_cut;
    }
}

// Re-read one segment from acc (the residual buffer) and emit its selection
// in index order from message position base on, one wave; sent entries'
// residual becomes +0.0.  Used for a segment with more candidates than slots
// and, in zero mode, for a segment that sends zeros (they are never stored).
// ZERO: every nonzero entry and the segment's first ztake zeros are sent;
// otherwise the entries with key > T, or key == T and index <= cut.
template <bool ZERO>
__device__ void emit_rescan(const SparsifyArgs &a, const FinWork &f, uint32_t seg, uint32_t base,
                            uint32_t ztake, uint32_t T, uint32_t cut)
{
    const uint32_t mend = f.moff + f.k;
    uint32_t run = 0, zrun = 0;
    walk_segment(a, f, seg, [&](uint32_t valid, const uint32_t *idx, const float *v) {
        uint32_t sel = 0, zm = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (!(valid & (1u << j))) continue;
            const uint32_t key = key_of(v[j]);
            if (ZERO) {
                if (key == 0u) zm |= 1u << j;
                else sel |= 1u << j;
            } else if (key > T || (key == T && idx[j] <= cut)) {
                sel |= 1u << j;
            }
        }
        if (ZERO) {
            uint32_t ztot;
            uint32_t zr = zrun + wave_prefix3((uint32_t)__popc(zm), ztot);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (zm & (1u << j)) {
                    if (zr < ztake) sel |= 1u << j;
                    ++zr;
                }
            }
            zrun += ztot;
        }
        uint32_t stot;
        uint32_t pos = base + run + wave_prefix3((uint32_t)__popc(sel), stot);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (sel & (1u << j)) {
                if (pos < mend) {            // the layer's selection holds exactly k entries
                    a.msg_idx[pos] = idx[j];
                    a.msg_val[pos] = v[j];
                }
                a.res[idx[j]] = 0.0f;
                ++pos;
            }
        }
        run += stot;
    });
}

// Shared memory of the guess-failure fallback (fix_layers, below).
struct FixLds {
    uint32_t hl[2048];            // this workgroup's histogram of the current digit
    uint32_t hp[2048];            // the layer's histogram of the current digit
    uint32_t flag[kBlock];        // failed layers among the next kBlock sampled layers
    uint32_t wtot[kParts][kWaves];
    uint32_t tmp[kWaves];
    uint32_t res[2];
    uint32_t run[2];
};
__device__ void fix_layers(const SparsifyArgs &a, FixLds &x);

// Emission of one finishing workgroup's segments (the body of k_fin_emit).
__device__ void emit_segments(const SparsifyArgs &a)
{
    __shared__ uint32_t sbase[kFinSegs];
    __shared__ uint32_t ztake[kFinSegs];
    __shared__ uint32_t redo[kFinSegs];
    if (blockIdx.x >= a.nfin) return;        // a workgroup launched for the fallback only
    const uint32_t fb = a.fin_base + blockIdx.x;
    const FinWork f = a.fin_work[fb];
    const SampledState *st = a.state + f.sid;
    const uint32_t ln = lane_id();
    WaveSegs ws;
    ws.load(a, f, threadIdx.x >> 6, ln);      // issued before the status arrives
    const uint32_t status = st->status;       // uniform over the workgroup
    if (status != kStOk && status != kStZero) return;
    const bool zero = status == kStZero;
    static_assert(kFinSegs <= 64, "one wave scans the segment counts");
    const uint32_t s_end = min(f.seg0 + f.grain, f.nseg);
    if (threadIdx.x < 64) {
        const uint32_t s = f.seg0 + ln;
        const bool in = s < s_end;
        uint32_t v = in ? a.seg_sel[f.seg_base + s] : 0u;
        const uint32_t raw = in ? a.seg_count[f.seg_base + s] : 0u;
        uint32_t zt = 0;
        if (zero) {
            const uint32_t e = st->idx_cut;            // zeros the layer sends
            const uint32_t z = in ? seg_len(f, s) - raw : 0u;   // every nonzero is a candidate
            const uint32_t zb = a.fin_eq[fb] + wave_incl_scan(z) - z;   // zeros before segment s
            zt = (zb >= e) ? 0u : min(z, e - zb);
            v += zt;
        }
        const uint32_t incl = wave_incl_scan(v);
        if (in) {
            sbase[ln] = f.moff + a.fin_total[fb] + incl - v;
            ztake[ln] = zt;
            redo[ln] = (raw > f.cap || zt != 0u) ? 1u : 0u;
        }
    }
    const uint32_t T = zero ? 0u : st->T, cut = zero ? 0u : st->idx_cut;
    const uint32_t mend = f.moff + f.k;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSegsPerWave; ++i) {
        if (!ws.valid(i)) continue;
        const uint32_t base = sbase[ws.seg(i) - f.seg0];
        if (redo[ws.seg(i) - f.seg0]) continue;   // re-read below
        const uint32_t cnt = ws.cnt(i);
        const uint2 *slots = ws.slots(a, f, i);
        uint32_t run = 0;
        for (uint32_t p0 = 0; p0 < cnt; p0 += 64) {
            const uint32_t p = p0 + ln;
            bool sel = false;
            uint2 c = make_uint2(0, 0);
            if (p < cnt) {
                c = ws.at(i, p, slots);
                const uint32_t key = c.y & 0x7fffffffu;
                // candidates always lie in their layer; the range test keeps a
                // damaged workspace from turning into a stray store
                sel = (c.x - f.off < f.n) && (key > T || (key == T && c.x <= cut));
            }
            const uint64_t m = __ballot(sel);
            if (sel) {
                const uint32_t pos = base + run + mbcnt(m);
                if (pos < mend) {            // the layer's selection holds exactly k entries
                    a.msg_idx[pos] = c.x;
                    a.msg_val[pos] = __uint_as_float(c.y);
                }
                a.res[c.x] = 0.0f;
            }
            run += (uint32_t)__popcll(m);
        }
    }
    for (uint32_t s = f.seg0 + (threadIdx.x >> 6); s < s_end; s += kWaves) {
        if (!redo[s - f.seg0]) continue;
        if (zero) emit_rescan<true>(a, f, s, sbase[s - f.seg0], ztake[s - f.seg0], 0u, 0u);
        else emit_rescan<false>(a, f, s, sbase[s - f.seg0], 0u, T, cut);
    }
}

// k_fin_emit: write the selected candidates of each segment, in index order,
// and zero their residual.  Segments with more candidates than slots, and in
// zero mode segments that send zeros, are re-read whole instead.  Then the
// first a.fix_groups workgroups select the layers whose guess failed, if any.
__global__ __launch_bounds__(kBlock, 8) void k_fin_emit(SparsifyArgs a)
{
    __shared__ FixLds x;
    emit_segments(a);
    if (blockIdx.x < a.fix_groups) fix_layers(a, x);
}

// ---------------------------------------------------------------------------
// Exact mode (LAGS_SPARSIFY_EXACT): the threshold of every sampled layer by a
// multi-workgroup MSD radix select over the 31-bit keys of acc, digits of
// 11, 11 and 9 bits (key bits 30..20, 19..9, 8..0).  Each digit level is one
// pass over the layer that histograms, in LDS, the digit of the keys that
// match the prefix found so far and adds the histogram to the layer's copies
// in device memory, followed by one workgroup per layer that picks the digit
// holding the remaining rank.  Then per segment the keys above and equal to
// the threshold T are counted, one workgroup per layer finds the tie cut
// (the index of the e-th key equal to T, index order) and the message
// offsets, and k_fin_emit re-reads every segment and emits its selection.

constexpr uint32_t kXShift0 = 20u, kXShift1 = 9u;   // digit k: key bits [shift_k, shift_{k-1})
__device__ __forceinline__ uint32_t x_shift(uint32_t level)
{
    return level == 0u ? kXShift0 : (level == 1u ? kXShift1 : 0u);
}
__device__ __forceinline__ uint32_t x_bins(uint32_t level) { return level < 2u ? 2048u : 512u; }

// Walk one segment like walk_segment, with R rows of 64 float4 requested at
// once.  fn must not store to the residual buffer.
template <int R, class F>
__device__ void walk_segment_rows(const SparsifyArgs &a, const FinWork &f, uint32_t seg, F &&fn)
{
    const uint32_t ln = lane_id();
    const uint32_t end = f.off + f.n, b4 = end & ~3u;
    uint32_t idx[4];
    float v[4];
    if (seg == 0 && f.off < f.a4) {
        const uint32_t i = f.off + ln;
        const bool in = i < f.a4;
        idx[0] = idx[1] = idx[2] = idx[3] = i;
        v[0] = in ? a.res[i] : 0.0f;
        v[1] = v[2] = v[3] = 0.0f;
        fn(in ? 1u : 0u, idx, v);
    }
    const uint32_t lo = f.a4 + seg * kSeg;
    const uint32_t q0 = lo / 4u;
    const uint32_t q1 = (uint32_t)min((uint64_t)lo + kSeg, (uint64_t)b4) / 4u;
    const v4f *r4 = reinterpret_cast<const v4f *>(a.res);
    for (uint32_t qb = q0; qb < q1; qb += 64u * R) {
        v4f x[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t q = qb + (uint32_t)r * 64u + ln;
            x[r] = (q < q1) ? r4[q] : (v4f){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t q = qb + (uint32_t)r * 64u + ln;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                idx[j] = 4u * q + j;
                v[j] = x[r][j];
            }
            fn(q < q1 ? 0xfu : 0u, idx, v);
        }
    }
    if (seg == f.nseg - 1u && b4 < end) {
        const uint32_t i = b4 + ln;
        const bool in = i < end;
        idx[0] = idx[1] = idx[2] = idx[3] = i;
        v[0] = in ? a.res[i] : 0.0f;
        v[1] = v[2] = v[3] = 0.0f;
        fn(in ? 1u : 0u, idx, v);
    }
}

// The workgroup's LDS histogram (2048 words) added into histogram copy gh of
// the layer in device memory, nonzero bins only; all threads call.
__device__ void x_flush(const uint32_t *hl, uint32_t *gh)
{
    __syncthreads();
    for (uint32_t b = threadIdx.x; b < 2048u; b += kBlock)
        if (hl[b]) atomicAdd(&gh[b], hl[b]);
}

__device__ __forceinline__ void x_clear(uint32_t *hl)
{
    for (uint32_t b = threadIdx.x; b < 2048u; b += kBlock) hl[b] = 0;
    __syncthreads();
}

// The exact-mode passes run, like k_main, one workgroup per segment over the
// main work list (kTileSegs workgroups per entry); a workgroup whose entry is
// not a sampled tile, or whose segment is past the layer's end, has nothing
// to do (k_x_first sends the k == n tiles whole, as k_main does).
__device__ __forceinline__ bool x_segment(const SparsifyArgs &a, MainWork &w, uint32_t &seg)
{
    w = a.main_work[a.main_base + blockIdx.x / kTileSegs];
    seg = w.tile * kTileSegs + blockIdx.x % kTileSegs;
    return w.cls == kClsSampled && seg < w.nseg;
}

// Acc of the segment from the residual buffer (after the first pass), with
// the head and tail entries of the thread.
struct XSeg {
    SegView sv;
    v4f x[kRows];
    float hv, tv;
    __device__ void load(const SparsifyArgs &a, const MainWork &w, uint32_t seg)
    {
        const uint32_t t = threadIdx.x;
        sv = seg_view(w, seg);
        seg_rows<false>(a.res, sv, x);
        hv = t < sv.nh ? a.res[sv.hlo + t] : 0.0f;
        tv = t < sv.ntl ? a.res[sv.tlo + t] : 0.0f;
    }
    // fn(index, value) for every entry the thread holds
    template <class F>
    __device__ void each(F &&fn) const
    {
        const uint32_t t = threadIdx.x;
        if (t < sv.nh) fn(sv.hlo + t, hv);
#pragma unroll
        for (int u = 0; u < kRows; ++u)
            if (sv.row_in(u)) {
#pragma unroll
                for (int j = 0; j < 4; ++j) fn(4u * sv.row(u) + j, x[u][j]);
            }
        if (t < sv.ntl) fn(sv.tlo + t, tv);
    }
};

// k_x_first: the streaming pass of exact mode.  A sampled segment computes
// acc = grad + residual, stores it, and histograms the first digit of every
// key; a k == n tile is sent whole as in k_main.
__global__ __launch_bounds__(kBlock) void k_x_first(SparsifyArgs a)
{
    __shared__ uint32_t hl[2048];
    MainWork w;
    uint32_t seg;
    if (!x_segment(a, w, seg)) {
        if (w.cls != kClsSampled) dense_tile(a, w, blockIdx.x % kTileSegs, kTileSegs);
        return;
    }
    x_clear(hl);
    const uint32_t t = threadIdx.x;
    const SegView sv = seg_view(w, seg);
    v4f acc[kRows], rv[kRows];
    seg_rows<true>(a.grad, sv, acc);
    seg_rows<true>(a.res, sv, rv);
    float hv = 0.0f, tv = 0.0f;
    if (t < sv.nh) hv = a.grad[sv.hlo + t] + a.res[sv.hlo + t];
    if (t < sv.ntl) tv = a.grad[sv.tlo + t] + a.res[sv.tlo + t];
    uint32_t *h = hl;
    v4f *r4 = reinterpret_cast<v4f *>(a.res);
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
        acc[u] = acc[u] + rv[u];
        if (sv.row_in(u)) {
            __builtin_nontemporal_store(acc[u], r4 + sv.row(u));
#pragma unroll
            for (int j = 0; j < 4; ++j) atomicAdd(&h[key_of(acc[u][j]) >> kXShift0], 1u);
        }
    }
    if (t < sv.nh) {
        a.res[sv.hlo + t] = hv;
        atomicAdd(&h[key_of(hv) >> kXShift0], 1u);
    }
    if (t < sv.ntl) {
        a.res[sv.tlo + t] = tv;
        atomicAdd(&h[key_of(tv) >> kXShift0], 1u);
    }
    x_flush(hl, a.hist + w.hist_off + (blockIdx.x & (w.hcopies - 1u)) * kNBins);
}

// k_x_pass: digit `level` (1 or 2) of the segment's keys that match the
// layer's prefix above it, from acc in the residual buffer.
__global__ __launch_bounds__(kBlock) void k_x_pass(SparsifyArgs a, uint32_t level)
{
    __shared__ uint32_t hl[2048];
    MainWork w;
    uint32_t seg;
    if (!x_segment(a, w, seg)) return;
    x_clear(hl);
    XSeg xs;
    xs.load(a, w, seg);
    const uint32_t prefix = a.state[w.sid].xprefix;
    const uint32_t top = x_shift(level - 1u), sh = x_shift(level), mask = x_bins(level) - 1u;
    uint32_t *h = hl;
    xs.each([&](uint32_t, float v) {
        const uint32_t key = key_of(v);
        if ((key >> top) == (prefix >> top)) atomicAdd(&h[(key >> sh) & mask], 1u);
    });
    x_flush(hl, a.hist + w.hist_off + (blockIdx.x & (w.hcopies - 1u)) * kNBins);
}

// k_x_pick: one 1024-thread workgroup per sampled layer sums the histogram
// copies of digit `level`, finds the digit holding the remaining rank, and
// clears the copies for the next level.  After the last digit the prefix is
// the threshold T and the remaining rank the number e of keys equal to T to
// send.
__global__ __launch_bounds__(kBinsThreads) void k_x_pick(SparsifyArgs a, uint32_t level)
{
    constexpr int NT = kBinsThreads;
    __shared__ uint32_t hist[kNBins];
    __shared__ uint32_t tmp[NT / 64];
    __shared__ uint32_t res[2];
    const uint32_t sid = a.sample_base + blockIdx.x;
    const SampledInfo S = a.sinfo[sid];
    SampledState *st = a.state + sid;
    uint32_t *lh = a.hist + S.hist_off;
    const uint32_t nb = x_bins(level);
    for (uint32_t b = threadIdx.x; b < kNBins; b += NT) {
        uint32_t h = 0;
        if (b < nb) {
            for (uint32_t c0 = 0; c0 < S.hcopies; c0 += 8) {
                uint32_t v[8];
#pragma unroll
                for (uint32_t u = 0; u < 8; ++u) v[u] = (c0 + u < S.hcopies) ? lh[(c0 + u) * kNBins + b] : 0u;
#pragma unroll
                for (uint32_t u = 0; u < 8; ++u) h += v[u];
            }
        }
        hist[b] = h;
    }
    __syncthreads();
    const uint32_t rank = st->xrank;
    block_find_rank<NT>(hist, max(nb, (uint32_t)NT), rank, res, tmp);
    for (uint32_t t = threadIdx.x; t < S.hcopies * kNBins; t += NT) lh[t] = 0;
    if (level == 2u)   // k_x_count adds into the finishing workgroups' tie counts
        for (uint32_t b = threadIdx.x; b < S.fin_nblocks; b += NT) a.fin_eq[S.fin_first + b] = 0;
    if (threadIdx.x == 0) {
        const uint32_t prefix = st->xprefix | (res[0] << x_shift(level));
        st->xprefix = prefix;
        st->xrank = rank - res[1];
        if (level == 2u) st->T = prefix;
    }
}

// k_x_count: per segment, keys above T (into seg_sel) and equal to T (into
// the layer's threshold-bin area, one word per segment); the keys equal to T
// are also added to the tie count of the segment's finishing workgroup
// (cleared by the last k_x_pick), which k_x_cut scans.  The segment's entries
// with key >= T (the only ones that can be sent) are kept, in index order, in
// its candidate slots when they fit, and their number in seg_count, which is
// what k_fin_emit reads (more than the slots: the segment is re-read).
__global__ __launch_bounds__(kBlock) void k_x_count(SparsifyArgs a)
{
    __shared__ uint32_t wtot[kParts][kWaves];
    __shared__ uint32_t wgt[kWaves];
    MainWork w;
    uint32_t seg;
    if (!x_segment(a, w, seg)) return;
    XSeg xs;
    xs.load(a, w, seg);
    const uint32_t T = a.state[w.sid].T;
    const uint32_t fin_first = a.sinfo[w.sid].fin_first;
    const uint32_t t = threadIdx.x;
    const SegView &sv = xs.sv;
    uint32_t fl = 0, gt = 0;   // fl bit 4u + j: entry j of row u has key >= T
#pragma unroll
    for (int u = 0; u < kRows; ++u)
        if (sv.row_in(u)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = key_of(xs.x[u][j]);
                if (key >= T) fl |= 1u << (4 * u + j);
                gt += key > T ? 1u : 0u;
            }
        }
    uint32_t c[kParts], pos[kParts];
    c[0] = (t < sv.nh && key_of(xs.hv) >= T) ? 1u : 0u;
    gt += (t < sv.nh && key_of(xs.hv) > T) ? 1u : 0u;
#pragma unroll
    for (int u = 0; u < kRows; ++u) c[1 + u] = (uint32_t)__popc((fl >> (4 * u)) & 15u);
    c[kParts - 1] = (t < sv.ntl && key_of(xs.tv) >= T) ? 1u : 0u;
    gt += (t < sv.ntl && key_of(xs.tv) > T) ? 1u : 0u;
    const uint32_t total = block_positions(c, pos, wtot);   // keys >= T in the segment
    gt = wave_sum(gt);
    if (lane_id() == 0) wgt[t >> 6] = gt;
    if (total <= w.cap) {
        uint2 *slots = a.slots + (((uint64_t)w.slot_hi << 32) | w.slot_lo) + (uint64_t)seg * w.cap;
        if (c[0]) slots[pos[0]] = make_uint2(sv.hlo + t, __float_as_uint(xs.hv));
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            uint32_t p = pos[1 + u];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if ((fl >> (4 * u + j)) & 1u)
                    slots[p++] = make_uint2(4u * sv.row(u) + j, __float_as_uint(xs.x[u][j]));
        }
        if (c[kParts - 1]) slots[pos[kParts - 1]] = make_uint2(sv.tlo + t, __float_as_uint(xs.tv));
    }
    __syncthreads();
    if (t == 0) {
        uint32_t g = 0;
        for (int i = 0; i < kWaves; ++i) g += wgt[i];
        const uint32_t e = total - g;
        uint32_t *segeq = reinterpret_cast<uint32_t *>(a.tbin + (((uint64_t)w.slot_hi << 32) | w.slot_lo));
        a.seg_sel[w.seg_base + seg] = g;
        a.seg_count[w.seg_base + seg] = total;
        segeq[seg] = e;
        if (e) atomicAdd(&a.fin_eq[fin_first + seg / fin_grain(w.nseg)], e);
    }
}

// k_x_cut: one workgroup per sampled layer.  Finds the segment s* holding
// the e-th key equal to T (index order) and, re-reading it, that key's index
// (the cut); then per segment the selected count (keys above T, plus its
// keys equal to T up to the cut) and per finishing workgroup the message
// offset.  k_fin_emit then emits each segment from the entries k_x_count kept
// in its slots, or re-reads a segment whose entries did not fit.
__global__ __launch_bounds__(kBlock) void k_x_cut(SparsifyArgs a)
{
    __shared__ uint32_t tmp[kWaves];
    __shared__ uint32_t res[3];
    const uint32_t sid = a.sample_base + blockIdx.x;
    const SampledInfo S = a.sinfo[sid];
    SampledState *st = a.state + sid;
    const FinWork f = layer_fin(S, sid);           // the layer's static fields
    const uint32_t *segeq =
        reinterpret_cast<const uint32_t *>(a.tbin + (((uint64_t)S.slot_hi << 32) | S.slot_lo));
    const uint32_t T = st->T, e = st->xrank;       // 1 <= e <= keys equal to T
    if (threadIdx.x == 0) {       // (kept if the counts disagreed: bounded, never out of range)
        res[0] = 0;
        res[1] = 0;
        res[2] = 0xffffffffu;
    }
    // the finishing workgroup holding the e-th tie
    block_scan_items<16>(S.fin_nblocks, tmp, [&](uint32_t b) { return a.fin_eq[S.fin_first + b]; },
                         [&](uint32_t b, uint32_t ex, uint32_t z) {
                             if (ex < e && e <= ex + z) {
                                 res[0] = b;
                                 res[1] = ex;
                             }
                         });
    __syncthreads();
    if (threadIdx.x == 0) {       // its segment holding the tie (at most kFinSegs)
        uint32_t s = res[0] * f.grain, before = res[1];
        while (s + 1u < f.nseg && before + segeq[s] < e) before += segeq[s++];
        res[0] = s;
        res[1] = before;
    }
    __syncthreads();
    const uint32_t sstar = res[0], need = e - res[1];   // the need-th tie of segment s*
    if (threadIdx.x < 64) {
        uint32_t run = 0;
        walk_segment_rows<4>(a, f, sstar, [&](uint32_t valid, const uint32_t *idx, const float *v) {
            uint32_t tm = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if ((valid & (1u << j)) && key_of(v[j]) == T) tm |= 1u << j;
            uint32_t tot;
            uint32_t r = run + wave_prefix3((uint32_t)__popc(tm), tot);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (tm & (1u << j)) {
                    ++r;
                    if (r == need) res[2] = idx[j];
                }
            }
            run += tot;
        });
    }
    __syncthreads();
    const uint32_t cut = res[2];
    // selected per segment (seg_sel) and each finishing workgroup's message
    // offset (fin_total), which k_fin_emit reads as in the sampled path
    block_scan_items<16>(
        f.nseg, tmp,
        [&](uint32_t s) {
            const uint32_t eq = segeq[s];
            return a.seg_sel[f.seg_base + s] + (s < sstar ? eq : (s == sstar ? need : 0u));
        },
        [&](uint32_t s, uint32_t ex, uint32_t v) {
            a.seg_sel[f.seg_base + s] = v;
            if (s % f.grain == 0u) a.fin_total[S.fin_first + s / f.grain] = ex;
        });
    if (threadIdx.x == 0) {
        st->idx_cut = cut;
        st->status = kStOk;
        atomicAdd(&a.report[kRepSampled], 1u);
        atomicAdd(&a.report[kRepExact], 1u);
    }
}

// ---------------------------------------------------------------------------
// Guess-failure fallback.  A sampled layer whose guess failed (fewer than k
// candidates above a nonzero G, or a threshold bin beyond its list) is marked
// kStFix and selected here from all of its keys, which the residual buffer
// holds (acc) after the streaming pass.  The first a.fix_groups workgroups of
// the k_fin_emit launch (at most kFixGroups, dispatched first and all resident
// at once) split the layer's segments into contiguous ranges and run the
// exact-mode radix select over them: three digit passes (11, 11 and 9 key
// bits), each adding the workgroup's LDS histogram of the keys that match the
// prefix found so far into the layer's histogram of that digit, then meeting
// at a barrier after which every workgroup reads that histogram and picks the
// same digit.  The last pass also counts, per workgroup, the keys whose top 22
// bits exceed the prefix; with the workgroup's own last-digit histogram that
// gives its keys above and equal to the threshold T.  After one more barrier
// every workgroup scans those counts for its ties before it (only the first e
// keys equal to T, in index order, are sent) and its message position, and
// emits its segments in index order.  Four passes of 4 bytes per entry, all
// workgroups streaming.  Every wait is bounded: a barrier that is not reached
// in time is counted in the report and passed (the layer's output is then
// wrong; stores stay inside the layer and its message range).

constexpr uint32_t kFixSpin = 1u << 21;   // sleeps of ~0.5 us: about a second

// Barrier round `round` (1, 2, ...) of the F fallback workgroups.  Arrivals
// are spread over kFixSubs counters, one cache line each: workgroup w uses
// counter w % kFixSubs, so every workgroup on a counter runs on the same XCD
// (workgroups go to the XCDs round robin, w % 8).  What crosses workgroups
// goes through device-scope atomics and is read back with device-coherent
// loads; the last arrival on a counter writes that XCD's L2 back (release)
// before it bumps the top counter, on which every workgroup waits.  One
// address thus takes at most F / kFixSubs + 1 atomics per round, and each
// XCD does kFixSubs / 8 L2 write-backs per round instead of one per
// workgroup, with no L2 invalidation while other workgroups stream.
static_assert(kFixSubs % 8 == 0, "a counter's workgroups share one XCD");

__device__ void fix_barrier(const SparsifyArgs &a, uint32_t *fb, uint32_t F, uint32_t round)
{
    wait_mem_done();          // this thread's atomics into the layer's histogram are done
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t sub = blockIdx.x % kFixSubs;
        const uint32_t nsub = (F - sub + kFixSubs - 1u) / kFixSubs;   // workgroups on this counter
        const uint32_t nact = min(F, kFixSubs);                        // counters in use
        uint32_t *top = fb + kFbBarTop;
        const uint32_t old = __hip_atomic_fetch_add(fb + kFbBarSub + 32u * sub, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old == round * nsub - 1u) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        uint32_t it = 0;
        while (__hip_atomic_load(top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < round * nact) {
            __builtin_amdgcn_s_sleep(20);
            if (++it >= kFixSpin) {
                atomicAdd(&a.report[kRepFixTimeout], 1u);
                break;
            }
        }
    }
    __syncthreads();
}

__device__ void fix_layer(const SparsifyArgs &a, uint32_t sid, FixLds &x)
{
    const uint32_t F = a.fix_groups, wg = blockIdx.x, t = threadIdx.x;
    const SampledInfo S = a.sinfo[sid];
    uint32_t *fb = a.fb + (uint64_t)sid * kFbWords;
    MainWork mw{};                        // the fields seg_view reads
    mw.off = S.off;
    mw.end = S.off + S.n;
    mw.a4 = S.a4;
    mw.b4 = S.b4;
    mw.nseg = S.nseg;
    const uint32_t s_lo = (uint32_t)((uint64_t)S.nseg * wg / F);
    const uint32_t s_hi = (uint32_t)((uint64_t)S.nseg * (wg + 1u) / F);

    // bits of T known before the passes: those above vb, shared by the ends
    // of the range it lies in; digit levels made only of known bits are
    // skipped.  The first pass also counts the keys above that range.
    const SampledState &stl = a.state[sid];
    const uint32_t klo = stl.fix_klo, khi = stl.fix_khi;
    const uint32_t vb = varying_bits(klo, khi);
    uint32_t prefix = vb >= 32u ? 0u : (klo >> vb) << vb;
    uint32_t rank = S.k, gt22 = 0, nbar = 0;
    for (uint32_t level = 0; level < 3u; ++level) {
        const uint32_t sh = x_shift(level), nb = x_bins(level);
        if (sh >= vb) continue;           // every bit of this digit is known
        const bool first = nbar == 0u;
        const uint32_t ms = first ? vb : (level == 0u ? 32u : x_shift(level - 1u));  // match shift
        uint32_t hi = 0;                  // (first pass) keys above the known range
        for (uint32_t b = t; b < 2048u; b += kBlock) x.hl[b] = 0;
        __syncthreads();
        for (uint32_t sg = s_lo; sg < s_hi; ++sg) {
            XSeg xs;
            xs.load(a, mw, sg);
            LdsRun run;
            xs.each([&](uint32_t, float v) {
                const uint32_t key = key_of(v);
                if (ms >= 32u || (key >> ms) == (prefix >> ms)) run.add(x.hl, (key >> sh) & (nb - 1u));
                if (first && ms < 32u && (key >> ms) > (prefix >> ms)) ++hi;
                if (level == 2u && (key >> kXShift1) > (prefix >> kXShift1)) ++gt22;
            });
            run.flush(x.hl);
        }
        uint32_t *gh = fb + (level == 0u ? kFbHist0 : (level == 1u ? kFbHist1 : kFbHist2));
        if (first) {
            uint32_t tot;
            block_excl_scan(hi, x.tmp, tot);     // its barriers also end the LDS histogram
            if (t == 0 && tot) atomicAdd(&fb[kFbAbove], tot);
        } else {
            __syncthreads();
        }
        for (uint32_t b = t; b < nb; b += kBlock)
            if (x.hl[b]) atomicAdd(&gh[b], x.hl[b]);
        fix_barrier(a, fb, F, ++nbar);
        if (first) rank = S.k - ld_coherent(&fb[kFbAbove]);
        for (uint32_t b = t; b < nb; b += kBlock) x.hp[b] = ld_coherent(&gh[b]);
        __syncthreads();
        block_find_rank(x.hp, nb, rank, x.res, x.tmp);
        prefix |= x.res[0] << sh;
        rank -= x.res[1];
        __syncthreads();
    }
    const uint32_t T = prefix, e = rank, d2 = T & 511u;

    // this workgroup's keys above T (top 22 bits above, or the last digit
    // above) and equal to T; x.hl still holds its last-digit histogram
    uint32_t above = gt22;
    for (uint32_t b = t; b < 512u; b += kBlock) above += b > d2 ? x.hl[b] : 0u;
    uint32_t wgt;
    block_excl_scan(above, x.tmp, wgt);
    if (t == 0) {
        __hip_atomic_store(&fb[kFbCount + wg], wgt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&fb[kFbCount + F + wg], x.hl[d2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    fix_barrier(a, fb, F, ++nbar);

    // ties and sent entries of the workgroups before this one
    uint32_t ceq = 0, csel = 0;
    for (uint32_t base = 0; base < F; base += kBlock) {
        const uint32_t v = base + t;
        const uint32_t g = v < F ? ld_coherent(&fb[kFbCount + v]) : 0u;
        const uint32_t q = v < F ? ld_coherent(&fb[kFbCount + F + v]) : 0u;
        uint32_t teq, tsel;
        const uint32_t eqx = ceq + block_excl_scan(q, x.tmp, teq);
        const uint32_t take = eqx >= e ? 0u : min(q, e - eqx);
        const uint32_t selx = csel + block_excl_scan(g + take, x.tmp, tsel);
        if (v == wg) {
            x.run[0] = eqx;
            x.run[1] = selx;
        }
        ceq += teq;
        csel += tsel;
    }
    __syncthreads();
    uint32_t run_eq = x.run[0], run_sel = x.run[1];

    // emission, segment by segment in index order; the segment's values are
    // staged in LDS (the histograms are no longer needed) so that only their
    // flags stay in registers
    float *stage = reinterpret_cast<float *>(x.hl);   // hl and hp: kSeg floats
    static_assert(sizeof(x.hl) + sizeof(x.hp) >= kSeg * sizeof(float), "a segment fits the stage");
    const uint32_t mend = S.moff + S.k;
    for (uint32_t sg = s_lo; sg < s_hi; ++sg) {
        SegView sv;
        uint32_t fgt = 0, feq = 0;        // bit 4u + j: entry j of row u
        float hv, tv;
        {
            XSeg xs;
            xs.load(a, mw, sg);
            sv = xs.sv;
            hv = xs.hv;
            tv = xs.tv;
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                reinterpret_cast<v4f *>(stage)[u * kBlock + t] = xs.x[u];
                if (sv.row_in(u)) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t key = key_of(xs.x[u][j]);
                        if (key > T) fgt |= 1u << (4 * u + j);
                        else if (key == T) feq |= 1u << (4 * u + j);
                    }
                }
            }
        }
        const bool hin = t < sv.nh, tin = t < sv.ntl;
        const uint32_t hk = key_of(hv), tk = key_of(tv);
        uint32_t c[kParts], p[kParts];
        c[0] = (hin && hk == T) ? 1u : 0u;
#pragma unroll
        for (int u = 0; u < kRows; ++u) c[1 + u] = (uint32_t)__popc((feq >> (4 * u)) & 15u);
        c[kParts - 1] = (tin && tk == T) ? 1u : 0u;
        const uint32_t neq = block_positions(c, p, x.wtot);
        __syncthreads();
        // ties are sent while fewer than e came before them
        const bool hsel = hin && (hk > T || (hk == T && run_eq + p[0] < e));
        const bool tsel = tin && (tk > T || (tk == T && run_eq + p[kParts - 1] < e));
        uint32_t fsel = fgt;
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            uint32_t r = run_eq + p[1 + u];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if ((feq >> (4 * u + j)) & 1u) {
                    if (r < e) fsel |= 1u << (4 * u + j);
                    ++r;
                }
        }
        c[0] = hsel ? 1u : 0u;
#pragma unroll
        for (int u = 0; u < kRows; ++u) c[1 + u] = (uint32_t)__popc((fsel >> (4 * u)) & 15u);
        c[kParts - 1] = tsel ? 1u : 0u;
        const uint32_t nsel = block_positions(c, p, x.wtot);
        auto put = [&](uint32_t pos, uint32_t idx, float v) {
            const uint32_t m = S.moff + run_sel + pos;
            if (m < mend) {                  // the layer's selection holds exactly k entries
                a.msg_idx[m] = idx;
                a.msg_val[m] = v;
            }
            a.res[idx] = 0.0f;
        };
        if (hsel) put(p[0], sv.hlo + t, hv);
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            uint32_t q = p[1 + u];
            for (int j = 0; j < 4; ++j)
                if ((fsel >> (4 * u + j)) & 1u) put(q++, 4u * sv.row(u) + j, stage[(u * kBlock + t) * 4 + j]);
        }
        if (tsel) put(p[kParts - 1], sv.tlo + t, tv);
        run_eq += neq;
        run_sel += nsel;
        __syncthreads();
    }
}

// Select every layer of the launched range that is marked for the fallback,
// one after another (each with its own barrier counter and histograms).
__device__ void fix_layers(const SparsifyArgs &a, FixLds &x)
{
    if (a.nsampled == 0 || a.state[a.sample_base].nfail == 0) return;   // uniform
    __syncthreads();
    for (uint32_t base = 0; base < a.nsampled; base += kBlock) {
        const uint32_t i = base + threadIdx.x;
        x.flag[threadIdx.x] = (i < a.nsampled && a.state[a.sample_base + i].status == kStFix) ? 1u : 0u;
        __syncthreads();
        for (uint32_t j = 0; j < (uint32_t)kBlock && base + j < a.nsampled; ++j)
            if (x.flag[j]) fix_layer(a, a.sample_base + base + j, x);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// aggregate

// k_agg_starts: for every worker p and message position j in [j_lo, j_hi]
// (the message range of the launched layers), the chunk of entry j; chunk
// starts are written where the chunk id changes.  The range ends count as the
// first and the one-past-last chunk of the range, so a call reads only its own
// message entries and writes only the starts of chunks [c_lo, c_hi]; the
// shared boundary start c_hi gets the same value from either neighbour.  A
// workgroup covers BPW blocks of kStartsBlock positions of one worker (4 in
// large launches, so that fewer rounds of workgroups wait on the two memory
// round trips below; 1 in small ones, which would not fill the GPU), all
// requested at once; the layers they span are staged in LDS, in five tables of
// a.tl entries (dynamic LDS, sized by the host for the layout's widest span).
template <int BPW>
__global__ __launch_bounds__(kBlock, 8) void k_agg_starts(AggArgs a)
{
    constexpr int PPT = BPW * kStartsBlock / kBlock;   // positions per thread
    extern __shared__ uint32_t tab[];
    uint32_t *t_off = tab, *t_n = tab + a.tl, *t_moff = tab + 2u * a.tl, *t_cb = tab + 3u * a.tl,
             *t_sh = tab + 4u * a.tl;
    __shared__ uint32_t lrange[2];
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 2) a.report[kRepBad + threadIdx.x] = 0;
    const uint32_t p = blockIdx.y;
    const uint32_t bb = a.j_lo / kStartsBlock + blockIdx.x * BPW;   // first absolute position block
    const uint32_t j0 = bb * kStartsBlock;
    const uint32_t *row = a.msg_idx + (uint64_t)p * a.K;
    // message entries first: they do not depend on the layer lookup.  The
    // loads are unconditional, at positions clamped into [j_lo, j_hi) (not
    // empty), so that none waits for another; positions outside it are not
    // used below.
    uint32_t x[PPT], xp[PPT];
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
        const uint32_t j = j0 + threadIdx.x + q * kBlock;
        x[q] = row[min(max(j, a.j_lo), a.j_hi - 1u)];
        xp[q] = row[min(max(j, a.j_lo + 1u), a.j_hi) - 1u];
    }
    uint32_t *srow = a.start + (uint64_t)p * (a.NC + 1);
    // The usual case: the workgroup's positions, and the one before them, lie
    // in one layer; the blocks' descriptors then hold that layer's fields and
    // are requested together with the message entries.
    const uint4 d0 = a.sdesc[2u * bb], d1 = a.sdesc[2u * bb + 1u];
    const uint32_t lhi = a.sdesc[2u * min(bb + (uint32_t)BPW - 1u, a.npb - 1u)].y;
    if (d0.x == lhi) {                      // uniform over the workgroup
        auto chunk1 = [&](uint32_t xx) -> uint32_t {
            uint32_t rel = xx - d0.z;
            if (rel >= d0.w) rel = 0;            // invalid entry: counted by k_agg
            return d1.x + (rel >> d1.y);
        };
#pragma unroll
        for (int q = 0; q < PPT; ++q) {
            const uint32_t j = j0 + threadIdx.x + q * kBlock;
            if (j < a.j_lo || j > a.j_hi) continue;
            const uint32_t c = (j == a.j_hi) ? a.c_hi : chunk1(x[q]);
            const uint32_t cp = (j == a.j_lo) ? a.c_lo - 1u : chunk1(xp[q]);
            for (uint32_t cc = cp + 1u; cc <= c && cc <= a.NC; ++cc) srow[cc] = j;
        }
        return;
    }
    // positions of several layers: stage the layers' fields in LDS
    if (threadIdx.x == 0) {
        const uint32_t l0 = a.pos_layer[bb];
        const uint32_t l1 = (bb + BPW < a.npb) ? a.pos_layer[bb + BPW] : a.L - 1;
        lrange[0] = l0 > 0 ? l0 - 1 : 0;   // the layer of position j0 - 1 may precede l0
        lrange[1] = l1;
    }
    __syncthreads();
    const uint32_t la = lrange[0], nl = lrange[1] - la + 1;
    for (uint32_t t = threadIdx.x; t < nl; t += kBlock) {
        const LayerInfo Li = a.linfo[la + t];
        t_off[t] = Li.off;
        t_n[t] = Li.n;
        t_moff[t] = Li.moff;
        t_cb[t] = a.cbase[la + t];
        t_sh[t] = a.csh[la + t];
    }
    if (threadIdx.x == 0) t_moff[nl] = a.moff[la + nl];
    __syncthreads();
    auto chunk_of = [&](uint32_t xx, uint32_t t) -> uint32_t {
        uint32_t rel = xx - t_off[t];
        if (rel >= t_n[t]) rel = 0;          // invalid entry: counted by k_agg
        return t_cb[t] + (rel >> t_sh[t]);
    };
    auto layer_of = [&](uint32_t j) -> uint32_t {   // largest t in [0, nl) with t_moff[t] <= j
        uint32_t lo = 0, hi = nl;
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) / 2;
            if (t_moff[mid] <= j) lo = mid; else hi = mid;
        }
        return lo;
    };
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
        const uint32_t j = j0 + threadIdx.x + q * kBlock;
        if (j < a.j_lo || j > a.j_hi) continue;
        const uint32_t c = (j == a.j_hi) ? a.c_hi : chunk_of(x[q], layer_of(j));
        const uint32_t cp = (j == a.j_lo) ? a.c_lo - 1u : chunk_of(xp[q], layer_of(j - 1));
        for (uint32_t cc = cp + 1u; cc <= c && cc <= a.NC; ++cc) srow[cc] = j;
    }
}

// k_agg: one workgroup per index chunk [lo, hi) of one layer, with an LDS
// hash table of 2^TL slots.  Dynamic LDS: keys[2^TL], vals[2^TL], ws0[P],
// pre[P+1] and, with more than 32 workers, minpos[2^TL].  The chunk's message
// entries are laid out worker by worker (entry e of worker p: pre[p] <= e <
// pre[p+1]), so each slot's sum must add its entries in increasing worker
// order, starting from +0.0.  With at most 32 workers every entry finds its
// rank among the entries of its slot from a bitmask of the slot's workers, and
// the sums take one barrier phase per rank; with more, each round adds every
// slot's pending entry of lowest position.  Either way the sums take as many
// phases as the fullest slot has entries, not one per worker.
template <uint32_t TL, bool DENSE>
__global__ __launch_bounds__(kBlock, 8) void k_agg(AggArgs a)
{
    constexpr uint32_t kTable = 1u << TL;
    constexpr uint32_t kCap = kTable / 2;      // fast-path entries
    extern __shared__ uint32_t dyn[];
    uint32_t *keys = dyn;
    float *vals = reinterpret_cast<float *>(dyn + kTable);
    uint32_t *vmask = dyn + kTable;           // the same words: the slots' worker masks first
    uint32_t *ws0 = dyn + 2 * kTable;
    uint32_t *pre = ws0 + a.P;
    uint32_t *minpos = pre + a.P + 1;         // with more than 32 workers: per slot
    __shared__ uint32_t tmp[kWaves];

    const uint32_t c = a.c_lo + blockIdx.x;
    const uint32_t P = a.P;
    // The chunk starts of the first kBlock workers do not depend on the
    // chunk's layer: request them together with the layer lookup.
    uint32_t s0f = 0, s1f = 0;
    if (threadIdx.x < P) {
        const uint32_t *srow = a.start + (uint64_t)threadIdx.x * (a.NC + 1);
        s0f = srow[c];
        s1f = srow[c + 1];
    }
    const uint4 ci = a.chunk_info[c];
    const uint32_t lo = ci.x, hi = ci.y;     // the chunk's indices
    // (the DENSE instances serve layouts with k = n layers; the others keep
    // the sparse path's registers free of the dense loop)
    const bool dense = DENSE && ci.w == kAggDenseChunk;   // uniform
    // its layer's message range; for a chunk of a k = n layer, the positions
    // its indices take in every valid message
    const uint32_t m0 = ci.z, m1 = dense ? ci.z + (hi - lo) : ci.w;
    const float s = a.s;

    if (dense) {
        // every worker sends every index of the layer, in order: thread t
        // sums index lo + t from position m0 + t of each message, in worker
        // order, with one coalesced load per worker, and updates its weight
        constexpr uint32_t kW = 16;           // workers whose loads are in flight together
        const bool in = threadIdx.x < hi - lo;
        // loads are unconditional, at a thread offset and worker clamped into
        // the chunk, so that none waits for another
        const uint32_t t = min((uint32_t)threadIdx.x, hi - lo - 1u);
        const uint32_t x = lo + t;
        const float wv = a.w[x];
        float u = 0.0f;
        uint32_t off_place = 0;
        for (uint32_t p0 = 0; p0 < P; p0 += kW) {
            uint32_t xi[kW];
            float xv[kW];
#pragma unroll
            for (uint32_t q = 0; q < kW; ++q) {
                // the row's start is uniform; the thread adds its own offset
                const uint64_t row = (uint64_t)min(p0 + q, P - 1u) * a.K + m0;
                xi[q] = (a.msg_idx + row)[t];
                xv[q] = (a.msg_val + row)[t];
            }
#pragma unroll
            for (uint32_t q = 0; q < kW; ++q) {
                if (p0 + q < P) {
                    u = u + xv[q];
                    off_place |= (in && xi[q] != x) ? 1u : 0u;
                }
            }
        }
        if (!__syncthreads_or((int)off_place)) {
            if (in) a.w[x] = __fsub_rn(wv, __fmul_rn(s, u));
            return;
        }
        // an entry out of place: the chunk is summed by index below, from the
        // same positions
    }

    uint32_t carry = 0;
    for (uint32_t base = 0; base < P; base += kBlock) {
        const uint32_t p = base + threadIdx.x;
        uint32_t m = 0;
        if (p < P) {
            const uint32_t *srow = a.start + (uint64_t)p * (a.NC + 1);
            uint32_t s0 = base == 0 ? s0f : srow[c], s1 = base == 0 ? s1f : srow[c + 1];
            if (dense) {
                s0 = m0;
                s1 = m1;
            }
            s0 = min(max(s0, m0), m1);
            s1 = min(max(s1, s0), m1);
            ws0[p] = s0;
            m = s1 - s0;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan(m, tmp, tot);
        if (p < P) pre[p] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) pre[P] = carry;
    __syncthreads();
    const uint32_t E = carry;
    uint32_t bad = 0;

    if (E <= kCap) {
        const bool masks = P <= 32u;          // uniform
        for (uint32_t t = threadIdx.x; t < kTable; t += kBlock) {
            keys[t] = 0xffffffffu;
            vmask[t] = 0u;                    // (and vals[t] = +0.0)
            if (!masks) minpos[t] = 0xffffffffu;
        }
        __syncthreads();
        constexpr int EPT = kCap / kBlock;
        int slot[EPT];
        uint32_t wk[EPT];
        float v[EPT];
        uint32_t xs[EPT];
#pragma unroll
        for (int q = 0; q < EPT; ++q) {       // issue every entry load first
            const uint32_t e = threadIdx.x + q * kBlock;
            slot[q] = -1;
            wk[q] = 0;
            v[q] = 0.0f;
            xs[q] = 0xffffffffu;
            if (e < E) {
                uint32_t plo = 0, phi = P;   // pre[plo] <= e < pre[phi]
                while (phi - plo > 1) {
                    const uint32_t mid = (plo + phi) / 2;
                    if (pre[mid] <= e) plo = mid; else phi = mid;
                }
                const uint64_t at = (uint64_t)plo * a.K + ws0[plo] + (e - pre[plo]);
                wk[q] = plo;
                xs[q] = a.msg_idx[at];
                v[q] = a.msg_val[at];
            }
        }
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
            const uint32_t e = threadIdx.x + q * kBlock;
            if (e >= E) continue;
            const uint32_t x = xs[q];
            if (x < lo || x >= hi) {
                ++bad;
                continue;
            }
            const uint32_t key = x - lo;
            // a chunk no wider than the table: one slot per index, in index
            // order, so that a wave's weight updates below fall in one narrow
            // index range (ResNet-50 k_agg 38.4 -> 37 us); a wider chunk: a
            // multiplicative hash (Knuth's constant), which spreads runs of
            // consecutive indices (index-ordered buckets there made a chunk
            // holding one run of 512 indices take ~0.2 ms of probing)
            uint32_t hsh = (hi - lo <= kTable) ? key : (key * 2654435761u) >> (32 - TL);
            while (true) {
                const uint32_t old = atomicCAS(&keys[hsh], 0xffffffffu, key);
                if (old == 0xffffffffu || old == key) break;
                hsh = (hsh + 1u) & (kTable - 1u);
            }
            slot[q] = (int)hsh;
            if (masks) atomicOr(&vmask[hsh], 1u << wk[q]);
        }
        __syncthreads();
        if (masks) {
            // rank of each entry among its slot's entries (workers in order)
            uint32_t rk[EPT];
#pragma unroll
            for (int q = 0; q < EPT; ++q)
                rk[q] = slot[q] >= 0 ? (uint32_t)__popc(vmask[slot[q]] & ((1u << wk[q]) - 1u)) : 0xffffffffu;
            __syncthreads();                  // every mask is read before the sums overwrite it
            uint32_t more = 0;
#pragma unroll
            for (int q = 0; q < EPT; ++q) {
                if (rk[q] == 0u) vals[slot[q]] = 0.0f + v[q];
                more |= (rk[q] != 0xffffffffu && rk[q] > 0u) ? 1u : 0u;
            }
            // phase r adds the entries of rank r; the barrier ends phase r - 1
            for (uint32_t r = 1; __syncthreads_or((int)more); ++r) {
                more = 0;
#pragma unroll
                for (int q = 0; q < EPT; ++q) {
                    if (rk[q] == r) vals[slot[q]] = vals[slot[q]] + v[q];
                    more |= (rk[q] != 0xffffffffu && rk[q] > r) ? 1u : 0u;
                }
            }
        } else {
            // more workers than mask bits: in each round every slot adds its
            // pending entry of lowest chunk position (entry e's worker is
            // nondecreasing in e, so this is worker order), found with an LDS
            // minimum; one round per entry of the fullest slot, whatever P is.
            // The winner clears the slot's minimum; a loser reading it then
            // still sees a position other than its own.
            uint32_t pend = 0, more = 0;
#pragma unroll
            for (int q = 0; q < EPT; ++q)
                if (slot[q] >= 0) pend |= 1u << q;
            more = pend;
            while (__syncthreads_or((int)more)) {
#pragma unroll
                for (int q = 0; q < EPT; ++q)
                    if (pend & (1u << q)) atomicMin(&minpos[slot[q]], threadIdx.x + q * kBlock);
                __syncthreads();
#pragma unroll
                for (int q = 0; q < EPT; ++q) {
                    if (!(pend & (1u << q))) continue;
                    if (minpos[slot[q]] == threadIdx.x + q * kBlock) {
                        vals[slot[q]] = vals[slot[q]] + v[q];
                        minpos[slot[q]] = 0xffffffffu;
                        pend &= ~(1u << q);
                    }
                }
                more = pend;
            }
        }
        // apply at every touched index: every weight load of the thread is
        // requested before the first store (a store may alias a later load as
        // far as the compiler knows, so a plain loop waits one memory round
        // trip per slot)
        constexpr int TPT = kTable / kBlock;
        uint32_t tk[TPT];
        float tu[TPT], tw[TPT];
#pragma unroll
        for (int q = 0; q < TPT; ++q) {
            tk[q] = keys[threadIdx.x + q * kBlock];
            tu[q] = vals[threadIdx.x + q * kBlock];
        }
#pragma unroll
        for (int q = 0; q < TPT; ++q)
            tw[q] = tk[q] != 0xffffffffu ? a.w[lo + tk[q]] : 0.0f;
#pragma unroll
        for (int q = 0; q < TPT; ++q)
            if (tk[q] != 0xffffffffu) a.w[lo + tk[q]] = __fsub_rn(tw[q], __fmul_rn(s, tu[q]));
    } else {
        // dense windows over the chunk's index range; every entry is visited
        // once per window, workers in order
        uint32_t *touched = keys;
        float *u = vals;
        const uint32_t nwin = (hi - lo + kTable - 1) / kTable;
        for (uint32_t win = 0; win < nwin; ++win) {
            const uint32_t wlo = lo + win * kTable;
            const uint32_t whi = min(wlo + kTable, hi);
            for (uint32_t t = threadIdx.x; t < kTable; t += kBlock) {
                touched[t] = 0;
                u[t] = 0.0f;
            }
            __syncthreads();
            for (uint32_t p = 0; p < P; ++p) {
                const uint32_t m = pre[p + 1] - pre[p];
                if (m == 0) continue;
                for (uint32_t jj = threadIdx.x; jj < m; jj += kBlock) {
                    const uint64_t at = (uint64_t)p * a.K + ws0[p] + jj;
                    const uint32_t x = a.msg_idx[at];
                    if (x >= wlo && x < whi) {
                        u[x - wlo] = u[x - wlo] + a.msg_val[at];
                        touched[x - wlo] = 1;
                    } else if (win == 0 && (x < lo || x >= hi)) {
                        ++bad;
                    }
                }
                __syncthreads();
            }
            for (uint32_t t = threadIdx.x; t < whi - wlo; t += kBlock) {
                if (touched[t]) {
                    const uint32_t x = wlo + t;
                    a.w[x] = __fsub_rn(a.w[x], __fmul_rn(s, u[t]));
                }
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) atomicAdd(&a.report[kRepSlow], 1u);
    }
    bad = wave_sum(bad);
    if (lane_id() == 0 && bad) atomicAdd(&a.report[kRepBad], bad);
}

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free sparsify (lags_sparsify_layers_static):
// a file-scope device array that each device holds from the library's first
// use on it until the process ends.  Host code never passes the array's name
// to a kernel: it looks up this device's address of it once, with the device
// current, and uses that address only.

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void **out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *ptr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// launchers

// Unused dynamic LDS that sets how many one-segment workgroups a CU holds
// (160 KiB of LDS per CU): a workgroup takes 36,000 B in launches of 12K
// workgroups and more (4 per CU), 23,000 B below (6-7 per CU).  Measured on
// the streaming pass, total LDS per workgroup: 1.31B entries (320K
// workgroups) 2.44-2.46 ms at 32,288-36,000 B, 2.56-2.58 at 32,000, 2.59 at
// 27,000, 2.65 at 23,000, 2.77 at 54,000 (3 per CU); 66M entries (16K
// workgroups) 1.4% faster at 36,000 B than at 23,000; 15M-26M entries
// (3.7K-6.2K workgroups) fastest at 23,000 B, up to 6% slower at 32,288.
// The exact-mode passes that only read the layer (k_x_pass, k_x_count) run
// 6-7 workgroups per CU at every size: their per-workgroup work (histogram,
// ordering of the keys >= T) needs more workgroups in flight than the
// streaming pass.  Same-box A/B of the exact call at 1.31B entries: 5.54 ms
// with the streaming pass's rule, 5.26 at 23,000 B, 5.30 with no pad.
constexpr size_t kReadPassLds = 23000;

size_t stream_lds_pad(uint32_t ngroups, size_t static_lds)
{
    const size_t total = ngroups >= 12288u ? 36000 : 23000;
    return total > static_lds ? total - static_lds : 0;
}

hipError_t launch_sample(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s)
{
    hipLaunchKernelGGL(k_sample, dim3(nblocks), dim3(kSampleThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_main(const SparsifyArgs &a, uint32_t nblocks, bool nt_store, hipStream_t s)
{
    const uint32_t ngroups = nblocks * kTileSegs;
    // the pad doubles as a heavy segment's LDS histogram
    const size_t pad = std::max<size_t>(stream_lds_pad(ngroups, (kCapMax * 2 + kParts * kWaves) * 4),
                                        kNBins * sizeof(uint32_t));
    if (nt_store)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_main<true>), dim3(ngroups), dim3(kBlock), pad, s, a);
    else
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_main<false>), dim3(ngroups), dim3(kBlock), pad, s, a);
    return hipGetLastError();
}

hipError_t launch_fin_bins(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s)
{
    hipLaunchKernelGGL(k_fin_bins, dim3(nblocks), dim3(kBinsThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fin_select(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s)
{
    hipLaunchKernelGGL(k_fin_select, dim3(nblocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fin_resolve(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s)
{
    hipLaunchKernelGGL(k_fin_resolve, dim3(nblocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fin_emit(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s)
{
    hipLaunchKernelGGL(k_fin_emit, dim3(nblocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_x_first(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s)
{
    const uint32_t ngroups = nblocks * kTileSegs;
    hipLaunchKernelGGL(k_x_first, dim3(ngroups), dim3(kBlock), stream_lds_pad(ngroups, 2048 * 4), s, a);
    return hipGetLastError();
}

hipError_t launch_x_pass(const SparsifyArgs &a, uint32_t nblocks, uint32_t level, hipStream_t s)
{
    const uint32_t ngroups = nblocks * kTileSegs;
    hipLaunchKernelGGL(k_x_pass, dim3(ngroups), dim3(kBlock), kReadPassLds - 2048 * 4, s, a, level);
    return hipGetLastError();
}

hipError_t launch_x_pick(const SparsifyArgs &a, uint32_t nblocks, uint32_t level, hipStream_t s)
{
    hipLaunchKernelGGL(k_x_pick, dim3(nblocks), dim3(kBinsThreads), 0, s, a, level);
    return hipGetLastError();
}

hipError_t launch_x_count(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s)
{
    const uint32_t ngroups = nblocks * kTileSegs;
    hipLaunchKernelGGL(k_x_count, dim3(ngroups), dim3(kBlock), kReadPassLds - (kParts + 1) * kWaves * 4, s, a);
    return hipGetLastError();
}

hipError_t launch_x_cut(const SparsifyArgs &a, uint32_t nblocks, hipStream_t s)
{
    hipLaunchKernelGGL(k_x_cut, dim3(nblocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_agg_starts(const AggArgs &a, hipStream_t s)
{
    const uint32_t nb = a.j_hi / kStartsBlock - a.j_lo / kStartsBlock + 1u;
    const size_t lds = 5u * a.tl * sizeof(uint32_t);
    if (a.bpw == 4)
        hipLaunchKernelGGL(k_agg_starts<4>, dim3((nb + 3u) / 4u, a.P), dim3(kBlock), lds, s, a);
    else if (a.bpw == 1)
        hipLaunchKernelGGL(k_agg_starts<1>, dim3(nb, a.P), dim3(kBlock), lds, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_agg(const AggArgs &a, uint32_t nchunks, uint32_t table_log2, bool dense, hipStream_t s)
{
    // keys and sums (or masks), the workers' starts and offsets, and with
    // more than 32 workers a per-slot minimum position
    const size_t lds =
        ((2u << table_log2) + (a.P > 32u ? (1u << table_log2) : 0u) + 2u * a.P + 1u) * sizeof(uint32_t);
    const dim3 g(nchunks), b(kBlock);
    if (table_log2 == kAggTableLog2 && dense)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_agg<kAggTableLog2, true>), g, b, lds, s, a);
    else if (table_log2 == kAggTableLog2)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_agg<kAggTableLog2, false>), g, b, lds, s, a);
    else if (table_log2 == kAggTableLog2Wide && dense)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_agg<kAggTableLog2Wide, true>), g, b, lds, s, a);
    else if (table_log2 == kAggTableLog2Wide)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_agg<kAggTableLog2Wide, false>), g, b, lds, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace lags
