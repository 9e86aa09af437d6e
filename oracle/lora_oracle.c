/*
 * lora_oracle.c -- plain fp64 reference of the multi-LoRA batched adapter path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code with the HIP
 * library and includes none of its headers.
 *
 * What it computes, and where the pages define it:
 *   - LoRA replaces the update of a frozen W in R^{d x k} by Delta W = B A with
 *     A in R^{r x k}, B in R^{d x r} (DeltaServe, section 2.2), so that a layer
 *     computes h(x) = W x + B A x (MOLT, section 2.1, the displayed equation).
 *   - Multi-LoRA batching: rows of one batch that use different adapters share
 *     the base pass and each row adds the low-rank term of its own adapter
 *     (DeltaServe, section 2.2; the adapter-caching page on batching several
 *     adapters in one batch).  Here y0 = W x is the caller's base output and
 *     a per-adapter scale s_a multiplies the term (alpha = 32 at r = 16,
 *     DeltaServe section 4.1, read as s_a = alpha / r = 2).
 *   - The fine-tuning backward computes the LoRA gradients (DeltaServe,
 *     section 3.2, "Backward subprocess").  With dY = dL/dy given, the
 *     gradients of y = y0 + s B A x are
 *         g  = B^T dy,   dX += s A^T g,   dA += s g x^T,   dB += s dy (A x)^T,
 *     summed over the fine-tuning rows of each adapter.
 *
 * Every result is accumulated in double precision with straightforward loops:
 * no blocking, no reordering beyond the definition, no fused or approximate
 * arithmetic.  OpenMP only splits independent output elements across threads;
 * every individual sum runs in the order written.
 *
 * Layouts (row-major): x [T, d_in], y [T, d_out], A_a [r_a, d_in],
 * B_a [d_out, r_a], dA_a [r_a, d_in], dB_a [d_out, r_a], v and g [T, ldv].
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_version(void) { return 1; }

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Grouping of rows by adapter.  counts[a] = number of rows with id a;
 * offsets = exclusive prefix sum of counts (offsets[A] = number of rows with a
 * valid id); perm lists those rows grouped by adapter, ascending row index
 * inside each group.  Rows with id -1 carry no adapter and are left out; any
 * other id outside [0, A) is also left out and counted in *err.
 * Brute force: one pass over all rows per adapter.
 */
void oracle_segments(const int32_t* ids, int64_t T, int32_t A,
                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* err) {
    int64_t pos = 0;
    for (int32_t a = 0; a < A; ++a) {
        offsets[a] = (int32_t)pos;
        int32_t c = 0;
        for (int64_t t = 0; t < T; ++t) {
            if (ids[t] == a) {
                perm[pos++] = (int32_t)t;
                ++c;
            }
        }
        counts[a] = c;
    }
    offsets[A] = (int32_t)pos;
    int32_t bad = 0;
    for (int64_t t = 0; t < T; ++t)
        if (ids[t] != -1 && (ids[t] < 0 || ids[t] >= A)) ++bad;
    *err = bad;
}

/*
 * Forward: for every row t with adapter a = ids[t] in [0, A):
 *     v_k      = sum_i A_a[k, i] x_t[i]            (k < r_a)
 *     y_t[j]  += s_a * sum_k B_a[j, k] v_k
 * y holds y0 on entry.  Rows with any other id are left unchanged.
 * v (may be NULL) receives v_k in row t at columns k < r_a.
 */
void oracle_forward(int64_t T, int32_t d_in, int32_t d_out,
                    const double* x, const int32_t* ids,
                    int32_t A, const int32_t* ranks, const double* scales,
                    const double* const* Aw, const double* const* Bw,
                    double* y, double* v, int32_t ldv) {
    int32_t r_max = 0;
    for (int32_t a = 0; a < A; ++a) if (ranks[a] > r_max) r_max = ranks[a];
#pragma omp parallel
    {
        double* vk = (double*)malloc(sizeof(double) * (size_t)(r_max > 0 ? r_max : 1));
#pragma omp for schedule(dynamic, 8)
        for (int64_t t = 0; t < T; ++t) {
            int32_t a = ids[t];
            if (a < 0 || a >= A) continue;
            int32_t r = ranks[a];
            const double* Aa = Aw[a];
            const double* Ba = Bw[a];
            const double* xt = x + t * (int64_t)d_in;
            for (int32_t k = 0; k < r; ++k) {
                double acc = 0.0;
                for (int32_t i = 0; i < d_in; ++i) acc += Aa[(int64_t)k * d_in + i] * xt[i];
                vk[k] = acc;
                if (v) v[t * (int64_t)ldv + k] = acc;
            }
            double* yt = y + t * (int64_t)d_out;
            for (int32_t j = 0; j < d_out; ++j) {
                double acc = 0.0;
                for (int32_t k = 0; k < r; ++k) acc += Ba[(int64_t)j * r + k] * vk[k];
                yt[j] += scales[a] * acc;
            }
        }
        free(vk);
    }
}

/*
 * Backward over the fine-tuning rows t = 0..T-1 (x, dy, dx are those rows only).
 * For each row with adapter a = ids[t] in [0, A):
 *     g_k       = sum_j B_a[j, k] dy_t[j]
 *     v_k       = sum_i A_a[k, i] x_t[i]
 *     dx_t[i]  += s_a * sum_k A_a[k, i] g_k                 (dx may be NULL)
 *     dA_a[k,i]+= s_a * g_k x_t[i]        summed over the rows of a, ascending t
 *     dB_a[j,k]+= s_a * dy_t[j] v_k       summed over the rows of a, ascending t
 * dA[a] / dB[a] may be NULL for adapters that have no rows here.
 * g_out / v_out (may be NULL) receive g and v, [T, ldv].
 */
void oracle_backward(int64_t T, int32_t d_in, int32_t d_out,
                     const double* x, const double* dy, const int32_t* ids,
                     int32_t A, const int32_t* ranks, const double* scales,
                     const double* const* Aw, const double* const* Bw,
                     double* dx, double* const* dA, double* const* dB,
                     double* g_out, double* v_out, int32_t ldv) {
    int32_t r_max = 1;
    for (int32_t a = 0; a < A; ++a) if (ranks[a] > r_max) r_max = ranks[a];
    double* G = (double*)calloc((size_t)(T > 0 ? T : 1) * (size_t)r_max, sizeof(double));
    double* V = (double*)calloc((size_t)(T > 0 ? T : 1) * (size_t)r_max, sizeof(double));

#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t t = 0; t < T; ++t) {
        int32_t a = ids[t];
        if (a < 0 || a >= A) continue;
        int32_t r = ranks[a];
        const double* Aa = Aw[a];
        const double* Ba = Bw[a];
        const double* xt = x + t * (int64_t)d_in;
        const double* dyt = dy + t * (int64_t)d_out;
        for (int32_t k = 0; k < r; ++k) {
            double acc = 0.0;
            for (int32_t j = 0; j < d_out; ++j) acc += Ba[(int64_t)j * r + k] * dyt[j];
            G[t * r_max + k] = acc;
            double accv = 0.0;
            for (int32_t i = 0; i < d_in; ++i) accv += Aa[(int64_t)k * d_in + i] * xt[i];
            V[t * r_max + k] = accv;
        }
        if (dx) {
            double* dxt = dx + t * (int64_t)d_in;
            for (int32_t i = 0; i < d_in; ++i) {
                double acc = 0.0;
                for (int32_t k = 0; k < r; ++k) acc += Aa[(int64_t)k * d_in + i] * G[t * r_max + k];
                dxt[i] += scales[a] * acc;
            }
        }
    }

    for (int32_t a = 0; a < A; ++a) {
        int32_t r = ranks[a];
        double s = scales[a];
        int any = 0;
        for (int64_t t = 0; t < T; ++t) if (ids[t] == a) { any = 1; break; }
        if (!any || !dA[a] || !dB[a]) continue;
        double* dAa = dA[a];
        double* dBa = dB[a];
#pragma omp parallel for schedule(static)
        for (int32_t k = 0; k < r; ++k) {
            for (int64_t t = 0; t < T; ++t) {
                if (ids[t] != a) continue;
                double gk = G[t * r_max + k];
                const double* xt = x + t * (int64_t)d_in;
                for (int32_t i = 0; i < d_in; ++i) dAa[(int64_t)k * d_in + i] += s * gk * xt[i];
            }
        }
#pragma omp parallel for schedule(static)
        for (int32_t j = 0; j < d_out; ++j) {
            for (int64_t t = 0; t < T; ++t) {
                if (ids[t] != a) continue;
                double dyj = dy[t * (int64_t)d_out + j];
                for (int32_t k = 0; k < r; ++k) dBa[(int64_t)j * r + k] += s * dyj * V[t * r_max + k];
            }
        }
    }

    if (g_out || v_out) {
        for (int64_t t = 0; t < T; ++t) {
            int32_t a = ids[t];
            if (a < 0 || a >= A) continue;
            for (int32_t k = 0; k < ranks[a]; ++k) {
                if (g_out) g_out[t * (int64_t)ldv + k] = G[t * r_max + k];
                if (v_out) v_out[t * (int64_t)ldv + k] = V[t * r_max + k];
            }
        }
    }
    free(G);
    free(V);
}

/*
 * One AdamW step (Adam with decoupled weight decay, Loshchilov and Hutter) on
 * one tensor of adapter weights.  The fine-tuning updates the shared adapter
 * weights directly once the gradients of a backward batch have been
 * accumulated (DeltaServe, section 3.2, "Backward subprocess"); its optimizer
 * is AdamW with learning rate 1e-3 and weight decay 0.01 (DeltaServe, section
 * 4.1).  With step count t >= 1, element by element:
 *     g      = grad_scale * grad
 *     m      = beta1 m + (1 - beta1) g
 *     v      = beta2 v + (1 - beta2) g^2
 *     m_hat  = m / (1 - beta1^t)
 *     v_hat  = v / (1 - beta2^t)
 *     w      = w - lr (weight_decay w + m_hat / (sqrt(v_hat) + eps))
 * w, m, v are updated in place.
 */
void oracle_adamw(int64_t n, double* w, const double* grad, double* m, double* v,
                  double lr, double beta1, double beta2, double eps, double weight_decay,
                  double grad_scale, int32_t step) {
    double c1 = 1.0, c2 = 1.0;
    for (int32_t i = 0; i < step; ++i) {
        c1 *= beta1;
        c2 *= beta2;
    }
    const double bc1 = 1.0 - c1, bc2 = 1.0 - c2;
    for (int64_t i = 0; i < n; ++i) {
        const double g = grad_scale * grad[i];
        m[i] = beta1 * m[i] + (1.0 - beta1) * g;
        v[i] = beta2 * v[i] + (1.0 - beta2) * g * g;
        const double m_hat = m[i] / bc1;
        const double v_hat = v[i] / bc2;
        w[i] = w[i] - lr * (weight_decay * w[i] + m_hat / (sqrt(v_hat) + eps));
    }
}
