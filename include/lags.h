/*
 * lags.h - C ABI of the LAGS-SGD data-parallel hot path on one MI355X (gfx950).
 *
 * What is computed (the review "Layer-wise Adaptive Gradient Sparsification
 * for Distributed Deep Learning with Convergence Guarantees", Shi et al. 2019):
 *   abstract - every worker picks a small set of "significant" gradients from
 *     each layer independently, with a per-layer size, and the workers run
 *     synchronous SGD over what was picked;
 *   proposed method, bullet 1 - per layer, the top-k gradients by magnitude;
 *   proposed method, bullet 2 - the ratio is adaptive per layer (here: an
 *     input table of exact ratios);
 *   proposed method, bullet 4 - error compensation keeps the unsent part.
 *
 * One step of worker 0, over a flat fp32 gradient buffer cut into L layers by
 * an offset table (layer l = entries [off[l], off[l+1])):
 *   lags_sparsify_layers:  acc = grad + residual (fp32);  per layer, the k_l
 *     entries of largest |acc| (ties: lower index first) are sent as
 *     (uint32 global index, fp32 acc) in ascending index order;  residual
 *     becomes +0.0 at sent entries and acc elsewhere;
 *   lags_aggregate_apply:  u = sum of the P workers' messages, in worker order
 *     0..P-1 starting from +0.0;  every touched weight becomes
 *     w - (s * u) with s = lr / P (fp32, product rounded before the subtract).
 * Results are bit-identical to a plain sequential fp32 evaluation of these
 * definitions (round to nearest even, no flush to zero, no FMA contraction).
 *
 * Conventions for every entry point:
 *   - pointers named grad, residual, weights, msg_idx, msg_val and ws are
 *     DEVICE pointers on the device that was current when the workspace was
 *     initialised; tables passed to lags_layout_create are HOST pointers and
 *     are copied;
 *   - device buffers are owned by the caller; the library never allocates
 *     device memory and keeps no pointer to the caller's buffers after a call
 *     returns, except the workspace addresses lags_workspace_init records;
 *   - the layout's device tables live at the head of the caller's workspace:
 *     lags_workspace_init copies them there once (asynchronously, on its
 *     stream); the sparsify and aggregate calls only read them;
 *   - calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream): no host synchronisation, no copy, no allocation, except where
 *     a function says so, so they can be captured into a HIP graph;
 *   - arguments are validated on the host before anything is launched; on a
 *     negative status nothing has been launched and nothing written;
 *   - device faults surface at the caller's next synchronisation (HIP rules);
 *   - one workspace must not be used by two calls that may overlap in time,
 *     except range calls on disjoint layer ranges (see lags_sparsify_range).
 */
#ifndef LAGS_H
#define LAGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (negative = error). */
#define LAGS_OK 0
#define LAGS_EINVAL (-1)     /* invalid argument: null/misaligned pointer, bad table, overlap */
#define LAGS_ERANGE (-2)     /* size outside the supported range (n or K above 2^32 - 2, P, L) */
#define LAGS_EWORKSPACE (-3) /* workspace null, misaligned or smaller than required */
#define LAGS_EHIP (-4)       /* a HIP runtime call failed (no device, launch error, ...) */
#define LAGS_EDEVICE (-5)    /* current device differs from the workspace's device */
#define LAGS_ENOMEM (-6)     /* host allocation failed */
#define LAGS_ENOTINIT (-7)   /* workspace not initialised for this layout (lags_workspace_init) */
#define LAGS_ESTATIC (-8)    /* layout too large for lags_sparsify_layers_static's buffer */

/* Limits. */
#define LAGS_MAX_LAYERS 65536
#define LAGS_MAX_WORKERS 1024

/* Flags for lags_sparsify_layers. */
#define LAGS_SPARSIFY_EXACT 1u /* skip the sampled threshold estimate: every layer
                                  above the small-layer size finds its threshold
                                  by a multi-workgroup radix select over all its
                                  keys (three digit passes, then counting and
                                  emission passes): the same results, about 24
                                  bytes of memory traffic per entry instead of
                                  about 12 */

typedef struct lags_layout lags_layout; /* opaque; host object; see below */

/* Short English description of a status code (static string). */
const char *lags_strerror(int status);

/*
 * Entry count of a layer of n entries at ratio rho = num/den (proposed
 * method, bullet 2: the ratio is a per-layer quantity):
 *   k = ceil(n * num / den), in exact integer arithmetic.
 * Returns k >= 1 for n >= 1, 0 for n == 0, or LAGS_EINVAL for n < 0,
 * num < 1, den < 1 or num > den.
 */
int64_t lags_k_for_ratio(int64_t n, int64_t num, int64_t den);

/*
 * Build a layout: L layers over a flat buffer of n = layer_off[L] entries, and
 * the per-layer count k[l] of entries each worker sends (abstract: the set's
 * size is chosen per layer).
 *   layer_off: host int64[L+1], layer_off[0] == 0, strictly increasing,
 *              layer_off[L] <= 2^32 - 2 (indices are uint32; 0xffffffff is
 *              kept free as a marker);
 *   k:         host int64[L], 1 <= k[l] <= layer_off[l+1] - layer_off[l],
 *              sum(k) <= 2^32 - 2;
 *   out:       receives the new layout (destroy with lags_layout_destroy).
 * Pure host work: no HIP call is made here; the device tables are built on
 * the host and copied into a workspace by lags_workspace_init.  The layout
 * is immutable after creation and may be shared by concurrent calls (its
 * per-worker-count chunk plans and its record of initialised workspaces are
 * guarded by a lock).
 * Returns LAGS_OK, LAGS_EINVAL (bad table / null pointer), LAGS_ERANGE
 * (L < 1 or L > LAGS_MAX_LAYERS, n or sum(k) above 2^32 - 2), LAGS_ENOMEM.
 */
int lags_layout_create(int32_t L, const int64_t *layer_off, const int64_t *k,
                       lags_layout **out);

/* Free the layout (host memory only).  NULL is accepted.  The caller must
 * make sure no call using it, and no copy issued by lags_workspace_init, is
 * still running on the device. */
void lags_layout_destroy(lags_layout *layout);

/* n (entries), K = sum(k) (message length per worker), L. -1 on NULL. */
int64_t lags_layout_num_elems(const lags_layout *layout);
int64_t lags_layout_total_k(const lags_layout *layout);
int32_t lags_layout_num_layers(const lags_layout *layout);

/* Message offset of layer l: sum_{j<l} k[j] (l = L gives K); -1 if out of range. */
int64_t lags_layout_msg_offset(const lags_layout *layout, int32_t l);

/*
 * Bytes of device workspace that lags_sparsify_layers and
 * lags_aggregate_apply (with up to P workers) need: the layout's tables, the
 * aggregate's chunk tables for P workers, and scratch space.  The scratch
 * part's contents on entry are never read before being written, so results
 * do not depend on them.  Returns 0 for a NULL layout or P outside
 * [1, LAGS_MAX_WORKERS].
 */
size_t lags_workspace_bytes(const lags_layout *layout, int32_t P);

/*
 * Prepare a workspace for a layout and up to P workers: copies the layer
 * tables and the chunk tables for P workers (host images the layout built)
 * into the head and tail of ws with hipMemcpyAsync on `stream`, and records
 * (ws, P, current device) in the layout.  The sparsify and aggregate calls
 * of this layout accept only a workspace so recorded (else LAGS_ENOTINIT),
 * read the tables from it, and allocate and copy nothing themselves.
 * Initialising the same ws again replaces its record.  The tables must stay
 * intact: anything else that writes the workspace (another layout's calls,
 * a free and reallocation at the same address) requires a new
 * lags_workspace_init before the next call.  The copies read the layout's
 * host images, so the layout must outlive them (as it must outlive every
 * call that uses it).
 *   ws:       device memory of ws_bytes >= lags_workspace_bytes(layout, P),
 *             16-byte aligned, on the current device;
 *   P:        1..LAGS_MAX_WORKERS: the largest worker count the aggregate
 *             calls will pass with this workspace;
 *   stream:   hipStream_t of the copies; calls on other streams must be
 *             ordered after them by the caller.
 * Returns LAGS_OK, LAGS_EINVAL (null layout), LAGS_ERANGE (P),
 * LAGS_EWORKSPACE (null, misaligned or small ws), LAGS_EHIP, LAGS_ENOMEM.
 */
int lags_workspace_init(const lags_layout *layout, void *ws, size_t ws_bytes, int32_t P,
                        void *stream);

/*
 * Sparsify worker 0's gradient (abstract; proposed method, bullets 1 and 4).
 *   grad:     device fp32[n], read only;
 *   residual: device fp32[n], in/out: error-compensation memory;
 *   msg_idx:  device uint32[K], out: global indices, layer by layer in table
 *             order, ascending inside each layer (layer l at
 *             lags_layout_msg_offset(l));
 *   msg_val:  device fp32[K], out: the matching acc values, bit for bit;
 *   ws:       device workspace initialised for this layout by
 *             lags_workspace_init (any P), ws_bytes its size;
 *   flags:    0 or LAGS_SPARSIFY_EXACT;
 *   stream:   hipStream_t.
 * The message buffers are exactly row 0 of the [P][K] layout that
 * lags_aggregate_apply reads.  grad, residual, msg_idx, msg_val and ws must
 * be 16-byte aligned and must not overlap.
 * Returns LAGS_OK, LAGS_EINVAL, LAGS_EWORKSPACE, LAGS_ENOTINIT, LAGS_EDEVICE
 * (current device is not the one the workspace was initialised on),
 * LAGS_EHIP.
 */
int lags_sparsify_layers(const lags_layout *layout, const float *grad,
                         float *residual, uint32_t *msg_idx, float *msg_val,
                         void *ws, size_t ws_bytes, uint32_t flags, void *stream);

/*
 * lags_sparsify_layers without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Its scratch is a static device buffer
 * of the library, LAGS_STATIC_SCRATCH_BYTES per device, which each device
 * holds from the library's first use on it until the process ends; the call
 * allocates and frees nothing.  The buffer also holds the tables of the
 * layout last used on the device: a call with another layout first copies
 * that layout's tables in (hipMemcpyAsync on `stream` from the layout's host
 * image, so the layout must outlive the call, as always).  The scratch part
 * is never read before being written in a call, so results do not depend on
 * what an earlier call left.  Every call on one device shares its buffer:
 * calls that may overlap in time on one device (other streams, other host
 * threads without ordering) race and give wrong results.
 *   grad, residual, msg_idx, msg_val, flags, stream: as lags_sparsify_layers.
 * Returns LAGS_OK, LAGS_EINVAL, LAGS_ESTATIC (the layout's tables and scratch,
 * lags_workspace_bytes(layout, 1) less the aggregate part, exceed the buffer),
 * LAGS_EHIP.
 */
#define LAGS_STATIC_SCRATCH_BYTES (64u << 20)
int lags_sparsify_layers_static(const lags_layout *layout, const float *grad, float *residual,
                                uint32_t *msg_idx, float *msg_val, uint32_t flags,
                                void *stream);

/*
 * Aggregate P workers' messages and apply the SGD step (abstract: synchronous
 * SGD over the workers' sparse gradients).
 *   weights: device fp32[n], in/out; only touched entries are written;
 *   msg_idx: device uint32[P][K], worker-major (row p = worker p's message in
 *            the layout produced by lags_sparsify_layers: per layer k[l]
 *            distinct indices of that layer, ascending);
 *   msg_val: device fp32[P][K];
 *   P:       1..LAGS_MAX_WORKERS;  lr: learning rate (s = lr / P in fp32);
 *   ws:      device workspace initialised for this layout by
 *            lags_workspace_init with at least P workers, ws_bytes its size.
 * Messages that break the layout (an index outside its layer, indices not
 * strictly ascending) never cause an out-of-bounds access and never change
 * the weights of another layer: an entry found outside the index chunk it
 * is summed in (every entry outside its layer, and out-of-order entries that
 * land outside their chunk) is skipped and counted in
 * lags_report.bad_entries; the weights of a layer with malformed entries are
 * otherwise unspecified (e.g. for a repeated index).
 * Returns LAGS_OK, LAGS_EINVAL, LAGS_ERANGE (P), LAGS_EWORKSPACE (also: P
 * above the workspace's initialised worker count), LAGS_ENOTINIT,
 * LAGS_EDEVICE, LAGS_EHIP.
 */
int lags_aggregate_apply(const lags_layout *layout, float *weights,
                         const uint32_t *msg_idx, const float *msg_val,
                         int32_t P, float lr, void *ws, size_t ws_bytes,
                         void *stream);

/*
 * Layer-range forms of the two calls above, for layer-wise pipelining: a
 * layer's messages can be produced and exchanged as soon as back-propagation
 * has finished that layer (LAGS review, proposed method, bullet 3: the
 * layer-wise selection is what lets communication overlap with the backward
 * pass), and the MG-WFBP review's merged buckets are contiguous layer ranges.
 *   l0, l1: the layers [l0, l1) of the layout, 0 <= l0 <= l1 <= L;
 *           l0 == l1 validates the arguments and launches nothing.
 * Every other argument is the same full-model buffer as in the full call (the
 * layout's global indices and message offsets are used unchanged); the call
 * reads and writes only the entries [off[l0], off[l1]) of grad / residual /
 * weights and the message positions [msg_offset(l0), msg_offset(l1)) of
 * msg_idx / msg_val (of every worker row for the aggregate).  Splitting
 * [0, L) into ranges, called in any order, gives results bit-identical to
 * the full call, since every layer's selection and every index's update
 * depend on that layer alone.
 * The workspace parts a range uses belong to its layers, so calls on
 * disjoint ranges may share one workspace, also on different streams; the
 * report counters are then shared and restarted by every call, so
 * lags_workspace_report is only meaningful after calls that do not overlap.
 * Returns as the full calls, plus LAGS_ERANGE for a bad range.
 */
int lags_sparsify_range(const lags_layout *layout, int32_t l0, int32_t l1,
                        const float *grad, float *residual, uint32_t *msg_idx,
                        float *msg_val, void *ws, size_t ws_bytes, uint32_t flags,
                        void *stream);
int lags_aggregate_range(const lags_layout *layout, int32_t l0, int32_t l1,
                         float *weights, const uint32_t *msg_idx,
                         const float *msg_val, int32_t P, float lr, void *ws,
                         size_t ws_bytes, void *stream);

/*
 * Merged-gradient message schedule (MG-WFBP review, proposed method,
 * bullets 1-3 and 5: merge the messages of consecutive layers so that fewer
 * of them pay the start-up cost; the schedule that minimises the iteration
 * time is computed once, before training, by an O(L^2) dynamic programme).
 * Host only: no HIP call, no device memory.
 * Cost model (the pages give none; this is the plain reading):
 *   - back-propagation produces layers L-1 .. 0; layer l takes
 *     backward_time[l], so it is ready at backward_time[L-1] + ... +
 *     backward_time[l] (summed in that order, in double);
 *   - a message of B bytes holds the one link for alpha + beta * B;
 *   - a run of consecutive layers is one message, sent when its lowest layer
 *     is ready and the previous message has finished;
 *   - the objective is the finish time of the last message.
 *   backward_time: host double[L], finite, >= 0 (any time unit);
 *   msg_bytes:     host int64[L], >= 0, sum <= 2^53 (for LAGS messages,
 *                  8 * k[l] per worker);
 *   alpha, beta:   finite, >= 0 (time per message, time per byte);
 *   bounds:        out, host int32[L+1]: run j (in sending order) is the
 *                  layer range [bounds[j+1], bounds[j]); bounds[0] = L,
 *                  bounds[nruns] = 0.  Each run maps to one
 *                  lags_sparsify_range / lags_aggregate_range call;
 *   nruns, finish: out, the run count and the finish time of the schedule.
 * The finish time is the minimum over all 2^(L-1) schedules, exactly (the
 * same rounded operations as evaluating the returned schedule); among equally
 * fast schedules the one with the shortest last runs is returned.  O(L^2)
 * time, O(L) memory.
 * Returns LAGS_OK, LAGS_EINVAL (null pointer, negative or non-finite input),
 * LAGS_ERANGE (L outside [1, LAGS_MAX_LAYERS], byte total above 2^53),
 * LAGS_ENOMEM.
 */
int lags_merge_schedule(int32_t L, const double *backward_time,
                        const int64_t *msg_bytes, double alpha, double beta,
                        int32_t *bounds, int32_t *nruns, double *finish);

/* Finish time of a given schedule under the same model (for comparing with
 * one message per layer, bounds = {L, L-1, ..., 0}, or one message for the
 * whole model, bounds = {L, 0}).  bounds must strictly decrease from L to 0.
 * Returns LAGS_OK, LAGS_EINVAL, LAGS_ERANGE, LAGS_ENOMEM. */
int lags_schedule_finish(int32_t L, const double *backward_time,
                         const int64_t *msg_bytes, double alpha, double beta,
                         const int32_t *bounds, int32_t nruns, double *finish);

/*
 * Adaptive per-layer message sizes (LAGS review, proposed method, bullets 2
 * and 3: each layer's sparsification ratio adapts to that layer's
 * communication-to-computation ratio so that layer-wise pipelined
 * communication hides behind back-propagation).  Host only.
 * Reading (the pages give no formula): while layer l's message is
 * exchanged, back-propagation computes layer l-1 (backward_time[l-1]); an
 * all-gather of k entries costs alpha + beta * B with B = 8 * (P - 1) * k
 * bytes; k[l] is the largest k whose exchange fits that window,
 *   floor((backward_time[l-1] - alpha) / (beta * (8 * (P - 1)))),
 * kept in [ceil(n_l * rmin_num / rmin_den), n_l] (double arithmetic in that
 * order, bounds in exact integers).  Layer 0 has no window and takes the
 * lower bound; with P == 1 or beta == 0 every layer is sent whole.
 *   layer_off:     host int64[L+1], 0 = layer_off[0] < ... < layer_off[L] < 2^40;
 *   backward_time: host double[L], finite, >= 0;
 *   P:             1..LAGS_MAX_WORKERS;  alpha, beta: finite, >= 0;
 *   rmin_num/rmin_den: lower bound of the ratio, 1 <= num <= den;
 *   k:             out, host int64[L], ready for lags_layout_create.
 * Returns LAGS_OK, LAGS_EINVAL, LAGS_ERANGE.
 */
int lags_adaptive_k(int32_t L, const int64_t *layer_off, const double *backward_time,
                    int32_t P, double alpha, double beta, int64_t rmin_num,
                    int64_t rmin_den, int64_t *k);

/* What the last calls that used a workspace did. */
typedef struct lags_report {
    int32_t layers_sampled; /* layers above the small-layer size with k < n in the last
                               sparsify (the sampled-threshold path, or exact mode) */
    int32_t layers_exact;   /* of those, layers selected exactly: all of them in exact
                               mode, otherwise those whose sampled guess fell short */
    uint32_t bad_entries;   /* message entries the last aggregate skipped as invalid */
    uint32_t slow_chunks;   /* aggregate chunks above the fast-path capacity */
    int32_t layers_wide_bin; /* sampled layers whose threshold bin was resolved from the
                                workspace rather than LDS (last sparsify) */
    uint32_t fix_timeouts;  /* barrier waits of the guess-failure fallback that gave up
                               (bounded waits; 0 unless its workgroups could not all
                               run at once, and then the layer's output is wrong) */
} lags_report;

/* Synchronise `stream` and read the report kept in the workspace.  Only
 * meaningful after a sparsify / aggregate call with this workspace. */
int lags_workspace_report(const lags_layout *layout, const void *ws,
                          size_t ws_bytes, void *stream, lags_report *out);

/*
 * Kernel tracing.  While enabled on a layout, every kernel the library
 * launches for that layout is bracketed by HIP events on the launch stream.
 * lags_trace_read synchronises on the recorded events and returns, per
 * kernel id, the summed device time in milliseconds and the launch count
 * accumulated since tracing was enabled or last read (then resets them).
 */
int lags_trace_enable(lags_layout *layout, int on);
int lags_trace_read(lags_layout *layout, double *ms, int64_t *launches,
                    int32_t nkernels);
int32_t lags_num_kernels(void);
const char *lags_kernel_name(int32_t id);

#ifdef __cplusplus
}
#endif

#endif /* LAGS_H */
