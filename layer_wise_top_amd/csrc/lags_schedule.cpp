// Host-only planning for layer-wise pipelining: the merged-gradient message
// schedule and the adaptive per-layer message sizes.
//
// Merged-gradient message schedule.
// MG-WFBP review, proposed method: the gradients of consecutive layers may be
// merged into one message so that fewer messages pay the start-up cost; the
// schedule that minimises the iteration time is found once, before training,
// by an O(L^2) dynamic programme.  Cost model (the pages print none; this is
// the plain reading): back-propagation produces layers L-1 .. 0, layer l
// taking backward_time[l], so layer l is ready at the sum of backward_time
// over l..L-1 (summed from L-1 down); a message of B bytes holds the one link
// for alpha + beta * B; a run of consecutive layers is ready when its lowest
// layer is ready and is sent when the link is also free.  The objective is
// the finish time of the last message.
//
// Recurrence over the sending order (position q = 0 is layer L-1): with
// F[0] = 0 (link free at time 0) and R[q] the ready time of position q,
//   F[q] = min over p < q of  max(F[p], R[q-1]) + (alpha + beta * B(p, q)),
// B(p, q) the bytes of positions p..q-1.  The finish of a schedule is a
// monotone function of the finish before its last run (also in rounded
// arithmetic, since max and rounding are monotone), so the minimum over
// schedules ending with run [p, q) uses the minimum F[p]: the recurrence is
// exact, not an approximation.  O(L^2) in the worst case, far less when
// start-up costs are small next to the backward pass.
#include "lags.h"

#include <cmath>
#include <cstdint>
#include <new>
#include <vector>

namespace {

bool valid_inputs(int32_t L, const double *bt, const int64_t *nb, double alpha, double beta,
                  int *status)
{
    if (!bt || !nb) {
        *status = LAGS_EINVAL;
        return false;
    }
    if (L < 1 || L > LAGS_MAX_LAYERS) {
        *status = LAGS_ERANGE;
        return false;
    }
    if (!std::isfinite(alpha) || !std::isfinite(beta) || alpha < 0.0 || beta < 0.0) {
        *status = LAGS_EINVAL;
        return false;
    }
    int64_t total = 0;
    for (int32_t l = 0; l < L; ++l) {
        if (!std::isfinite(bt[l]) || bt[l] < 0.0 || nb[l] < 0) {
            *status = LAGS_EINVAL;
            return false;
        }
        total += nb[l];
        if (total > (int64_t(1) << 53)) {   // byte counts stay exact in a double
            *status = LAGS_ERANGE;
            return false;
        }
    }
    return true;
}

// Ready time of every layer, in back-propagation order of summation.
void ready_times(int32_t L, const double *bt, std::vector<double> &r)
{
    r.assign(L, 0.0);
    double t = 0.0;
    for (int32_t l = L - 1; l >= 0; --l) {
        t = t + bt[l];
        r[l] = t;
    }
}

}  // namespace

extern "C" {

int lags_merge_schedule(int32_t L, const double *backward_time, const int64_t *msg_bytes,
                        double alpha, double beta, int32_t *bounds, int32_t *nruns,
                        double *finish)
{
    int status = LAGS_OK;
    if (!bounds || !nruns || !finish) return LAGS_EINVAL;
    if (!valid_inputs(L, backward_time, msg_bytes, alpha, beta, &status)) return status;
    try {
        std::vector<double> r;
        ready_times(L, backward_time, r);
        // positions in sending order: q -> layer L-1-q
        std::vector<int64_t> S(L + 1, 0);          // S[q] = bytes of positions < q
        for (int32_t q = 0; q < L; ++q) S[q + 1] = S[q] + msg_bytes[L - 1 - q];
        std::vector<double> F(L + 1, 0.0);
        std::vector<int32_t> from(L + 1, 0);
        for (int32_t q = 1; q <= L; ++q) {
            const double ready = r[L - q];          // position q-1 is layer L-q
            double best = 0.0;
            int32_t arg = -1;
            // scan the last run's start from the shortest run to the longest;
            // ties keep the shortest last run
            for (int32_t p = q - 1; p >= 0; --p) {
                const double start = F[p] > ready ? F[p] : ready;
                const double t = start + (alpha + beta * (double)(S[q] - S[p]));
                if (arg < 0 || t < best) {
                    best = t;
                    arg = p;
                }
                // F is nondecreasing in p (dropping the last-produced layer
                // from a schedule cannot make it finish later), so once the
                // link is free by `ready`, every longer last run starts at
                // `ready` with more bytes: none is faster
                if (F[p] <= ready) break;
            }
            F[q] = best;
            from[q] = arg;
        }
        // runs in sending order: walk back from q = L, then reverse
        std::vector<int32_t> cuts;                  // positions where runs start
        for (int32_t q = L; q > 0; q = from[q]) cuts.push_back(from[q]);
        const int32_t nr = (int32_t)cuts.size();
        // run j (sending order) covers positions [cuts[nr-1-j], next) ->
        // layers [L - next, L - start)
        bounds[0] = L;
        for (int32_t j = 0; j < nr; ++j) {
            const int32_t q_end = (j + 1 < nr) ? cuts[nr - 2 - j] : L;
            bounds[j + 1] = L - q_end;
        }
        *nruns = nr;
        *finish = F[L];
    } catch (const std::bad_alloc &) {
        return LAGS_ENOMEM;
    }
    return LAGS_OK;
}

int lags_schedule_finish(int32_t L, const double *backward_time, const int64_t *msg_bytes,
                         double alpha, double beta, const int32_t *bounds, int32_t nruns,
                         double *finish)
{
    int status = LAGS_OK;
    if (!bounds || !finish) return LAGS_EINVAL;
    if (!valid_inputs(L, backward_time, msg_bytes, alpha, beta, &status)) return status;
    if (nruns < 1 || nruns > L || bounds[0] != L || bounds[nruns] != 0) return LAGS_EINVAL;
    for (int32_t j = 0; j < nruns; ++j)
        if (bounds[j + 1] >= bounds[j]) return LAGS_EINVAL;
    try {
        std::vector<double> r;
        ready_times(L, backward_time, r);
        double link_free = 0.0;
        for (int32_t j = 0; j < nruns; ++j) {
            const int32_t l0 = bounds[j + 1], l1 = bounds[j];
            int64_t b = 0;
            for (int32_t l = l0; l < l1; ++l) b += msg_bytes[l];
            const double start = link_free > r[l0] ? link_free : r[l0];
            link_free = start + (alpha + beta * (double)b);
        }
        *finish = link_free;
    } catch (const std::bad_alloc &) {
        return LAGS_ENOMEM;
    }
    return LAGS_OK;
}

// Adaptive per-layer message sizes (LAGS review, proposed method, bullets 2
// and 3: each layer's ratio follows its communication-to-computation ratio,
// so that pipelined communication hides behind back-propagation).  Plain
// reading, the pages giving no formula: while layer l is exchanged, the
// backward pass computes layer l-1, which takes backward_time[l-1]; an
// all-gather of k entries (8 bytes each, P - 1 messages received) costs
// alpha + beta * 8 * (P - 1) * k; k[l] is the largest k that fits, kept in
// [ceil(n_l * rmin_num / rmin_den), n_l].  Layer 0 has no window and takes
// the lower bound; with P == 1 or beta == 0 nothing is exchanged and every
// layer is sent whole.
int lags_adaptive_k(int32_t L, const int64_t *layer_off, const double *backward_time, int32_t P,
                    double alpha, double beta, int64_t rmin_num, int64_t rmin_den, int64_t *k)
{
    if (!layer_off || !backward_time || !k) return LAGS_EINVAL;
    if (L < 1 || L > LAGS_MAX_LAYERS || P < 1 || P > LAGS_MAX_WORKERS) return LAGS_ERANGE;
    if (!std::isfinite(alpha) || !std::isfinite(beta) || alpha < 0.0 || beta < 0.0) return LAGS_EINVAL;
    if (rmin_num < 1 || rmin_den < 1 || rmin_num > rmin_den) return LAGS_EINVAL;
    if (layer_off[0] != 0) return LAGS_EINVAL;
    for (int32_t l = 0; l < L; ++l) {
        if (layer_off[l + 1] <= layer_off[l]) return LAGS_EINVAL;
        if (layer_off[l + 1] >= (int64_t(1) << 40)) return LAGS_ERANGE;
        if (!std::isfinite(backward_time[l]) || backward_time[l] < 0.0) return LAGS_EINVAL;
    }
    const double per_entry = beta * (double)(8 * (int64_t)(P - 1));
    for (int32_t l = 0; l < L; ++l) {
        const int64_t n = layer_off[l + 1] - layer_off[l];
        const int64_t lo = (int64_t)(((__int128)n * rmin_num + rmin_den - 1) / rmin_den);
        int64_t kl;
        if (per_entry == 0.0) {
            kl = n;
        } else if (l == 0) {
            kl = lo;
        } else {
            const double budget = backward_time[l - 1] - alpha;
            if (budget <= 0.0) {
                kl = lo;
            } else {
                const double q = budget / per_entry;
                const int64_t fit = (q >= (double)n) ? n : (int64_t)std::floor(q);
                kl = fit < lo ? lo : (fit > n ? n : fit);
            }
        }
        k[l] = kl;
    }
    return LAGS_OK;
}

}  // extern "C"
