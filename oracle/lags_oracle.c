/*
 * LAGS-SGD oracle: a plain, slow CPU statement of what one data-parallel
 * step of layer-wise adaptive gradient sparsification computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this file's library.  It shares
 * no code, header, table or helper with the GPU library; neither uses the
 * other.
 *
 * Source: the review "Layer-wise Adaptive Gradient Sparsification for
 * Distributed Deep Learning with Convergence Guarantees" (Shi, Tang, Wang,
 * Zhao, Chu, 2019):
 *   - abstract: every worker picks a small set of significant gradients from
 *     each layer independently; the set's size is adaptive per layer; the
 *     workers run synchronous SGD (S-SGD);
 *   - proposed method, bullet 1: per layer, the top-k gradients by magnitude;
 *   - proposed method, bullet 2: the ratio is set per layer;
 *   - proposed method, bullet 4: error compensation keeps what was not sent.
 *
 * Readings taken where the pages are silent:
 *   - arithmetic is IEEE binary32, round to nearest even, no flush to zero
 *     (the gradients are fp32 tensors); build with -ffp-contract=off;
 *   - acc = grad + residual (the learning rate is not folded in);
 *   - magnitude order is the order of the 31-bit key bits(acc) & 0x7fffffff,
 *     so -0.0 ties +0.0; ties are broken by the lower index;
 *   - k_l = ceil(n_l * num / den) in integer arithmetic for rho_l = num/den;
 *   - a sent entry's residual becomes +0.0, an unsent one keeps acc;
 *   - the aggregate averages over P workers: u = sum over workers in worker
 *     order 0..P-1 starting from +0.0, s = lr / P (fp32), and every touched
 *     weight becomes w - (s * u) with the product rounded before the
 *     subtraction; untouched weights are not written.
 *
 * Pins: see tests/test_oracle_pins.py (brute force on tiny layers, argmax,
 * a second library route, invariants, the dense-SGD special case, exact
 * conservation over ten steps, exact aggregation with dyadic values, a
 * hand-worked example under tests/golden/).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Entry count of a layer of n entries at ratio num/den: ceil(n*num/den).
 * Proposed method, bullet 2 (ratio per layer); the ceiling keeps k >= 1.
 * Returns -1 for a negative size or a ratio outside (0, 1]. */
int64_t oracle_k_for_ratio(int64_t n, int64_t num, int64_t den)
{
    if (n < 0 || num <= 0 || den <= 0 || num > den)
        return -1;
    __int128 p = (__int128)n * (__int128)num;
    __int128 q = (p + (den - 1)) / den;
    return (int64_t)q;
}

static uint32_t key_of(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return u & 0x7fffffffu;
}

static int desc_u64(const void *a, const void *b)
{
    uint64_t x = *(const uint64_t *)a, y = *(const uint64_t *)b;
    return (x < y) - (x > y);
}

static int asc_u32(const void *a, const void *b)
{
    uint32_t x = *(const uint32_t *)a, y = *(const uint32_t *)b;
    return (x > y) - (x < y);
}

/*
 * One worker's sparsification (abstract; proposed method, bullets 1 and 4).
 *
 * For each layer l = [off[l], off[l+1]):
 *   acc_i = grad_i + residual_i;
 *   order the layer's entries by (|acc| descending, index ascending) and take
 *   the first k[l]: the layer's significant set S_l;
 *   message: for the entries of S_l in ascending index, (global index, acc);
 *   residual_i = +0.0 for i in S_l, acc_i otherwise.
 * The message of layer l occupies positions [sum_{j<l} k[j], ... + k[l]).
 *
 * The order is realised by one library sort per layer over 64-bit words
 * (key << 32) | (0xffffffff - local index), descending, which places larger
 * keys first and, among equal keys, lower indices first.
 *
 * Returns 0, or -1 on an invalid table (offsets not increasing, k outside
 * [1, n_l], a layer of 2^32 entries or more), -2 on allocation failure.
 */
int oracle_sparsify(int32_t L, const int64_t *off, const int64_t *k,
                    const float *grad, float *residual,
                    uint32_t *msg_idx, float *msg_val)
{
    int64_t mpos = 0;
    if (L < 0 || off[0] != 0)
        return -1;
    for (int32_t l = 0; l < L; ++l) {
        int64_t a = off[l], nl = off[l + 1] - off[l], kl = k[l];
        if (nl <= 0 || nl > 0xffffffffLL || kl < 1 || kl > nl)
            return -1;
        float *acc = (float *)malloc((size_t)nl * sizeof(float));
        uint64_t *word = (uint64_t *)malloc((size_t)nl * sizeof(uint64_t));
        uint32_t *chosen = (uint32_t *)malloc((size_t)kl * sizeof(uint32_t));
        if (!acc || !word || !chosen) {
            free(acc); free(word); free(chosen);
            return -2;
        }
        for (int64_t i = 0; i < nl; ++i) {
            acc[i] = grad[a + i] + residual[a + i];
            word[i] = ((uint64_t)key_of(acc[i]) << 32)
                    | (uint64_t)(0xffffffffu - (uint32_t)i);
        }
        qsort(word, (size_t)nl, sizeof(uint64_t), desc_u64);
        for (int64_t j = 0; j < kl; ++j)
            chosen[j] = 0xffffffffu - (uint32_t)(word[j] & 0xffffffffu);
        qsort(chosen, (size_t)kl, sizeof(uint32_t), asc_u32);
        for (int64_t i = 0; i < nl; ++i)
            residual[a + i] = acc[i];
        for (int64_t j = 0; j < kl; ++j) {
            uint32_t li = chosen[j];
            msg_idx[mpos + j] = (uint32_t)(a + li);
            msg_val[mpos + j] = acc[li];
            residual[a + li] = 0.0f;
        }
        mpos += kl;
        free(acc); free(word); free(chosen);
    }
    return 0;
}

/*
 * Aggregate P workers' messages and apply the SGD step (abstract: S-SGD over
 * the workers' sparse gradients).
 *
 * msg_idx / msg_val are [P][K], worker-major.  Only entries whose index lies
 * in [lo, hi) are used, and w points at the weights of that range, so a
 * caller can restrict the check to a slice of a large model; the result on
 * the slice is the same as for the whole buffer.
 *
 *   u_i = +0.0; for p = 0..P-1, for each (i, v) of worker p: u_i = u_i + v;
 *   s = lr / P;
 *   for every touched i: w_i = w_i - (s * u_i).
 *
 * Returns 0, -1 for P < 1 or an empty range, -2 on allocation failure.
 */
int oracle_aggregate(int32_t P, int64_t K, const uint32_t *msg_idx,
                     const float *msg_val, float *w, float lr,
                     int64_t lo, int64_t hi)
{
    if (P < 1 || K < 0 || hi <= lo)
        return -1;
    int64_t m = hi - lo;
    float *u = (float *)calloc((size_t)m, sizeof(float));
    unsigned char *touched = (unsigned char *)calloc((size_t)m, 1);
    if (!u || !touched) {
        free(u); free(touched);
        return -2;
    }
    for (int32_t p = 0; p < P; ++p) {
        for (int64_t j = 0; j < K; ++j) {
            int64_t x = (int64_t)msg_idx[(int64_t)p * K + j];
            if (x < lo || x >= hi)
                continue;
            u[x - lo] = u[x - lo] + msg_val[(int64_t)p * K + j];
            touched[x - lo] = 1;
        }
    }
    float s = lr / (float)P;
    for (int64_t i = 0; i < m; ++i) {
        if (!touched[i])
            continue;
        float d = s * u[i];
        w[i] = w[i] - d;
    }
    free(u);
    free(touched);
    return 0;
}
