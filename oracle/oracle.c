/*
 * Plain CPU fp64 oracle for attention forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code with the HIP library.
 *
 * What it follows.  The DASH paper ("DASH: Deterministic Attention Scheduling
 * for High-throughput Reproducible LLM Training", Fig. 1 caption: tiled
 * FlashAttention backward with per-KV-tile dK/dV and a global dQ reduction)
 * states that the deterministic schedules only fix the order of the fp32 dQ
 * additions (Axiom ledger: floating-point addition is non-associative).  The
 * exact result is therefore ordinary softmax attention and its gradient, so
 * this oracle is that definition written out, loop by loop, in double:
 *
 *   forward   S_ij  = scale * <q_i, k_j>, j > i masked out under the causal mask
 *             lse_i = log sum_j exp(S_ij)          (natural log, max-shifted)
 *             P_ij  = exp(S_ij - lse_i),  O_i = sum_j P_ij v_j
 *   backward  D_i   = <dO_i, O_i>
 *             dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - D_i)
 *             dV_j  = sum_i P_ij dO_i
 *             dQ_i  = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i
 *
 * No blocking, fusion or reordering beyond the definition: the backward is
 * one pass over query rows (dQ) and one pass over key rows (dK, dV), each
 * element recomputing the P and dS entries it needs.  Parallelism is over
 * (head, row) pairs with no shared accumulators, so the oracle is itself
 * deterministic.
 *
 * Layout: every tensor is a contiguous [H][s][d] double array (H = b*h heads),
 * lse and D are [H][s].
 */
#include <math.h>
#include <stddef.h>

static int allowed(int causal, int i, int j) { return !causal || j <= i; }

static double dot(const double* a, const double* b, int d) {
    double acc = 0.0;
    for (int t = 0; t < d; ++t) acc += a[t] * b[t];
    return acc;
}

/* Forward for every head: O and lse from Q, K, V (definition above). */
void oracle_attn_fwd(int H, int s, int d, double scale, int causal,
                     const double* q, const double* k, const double* v,
                     double* o, double* lse) {
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int hh = 0; hh < H; ++hh) {
        for (int i = 0; i < s; ++i) {
            const size_t base = (size_t)hh * s * d;
            const double* qi = q + base + (size_t)i * d;
            double m = -INFINITY;
            for (int j = 0; j < s; ++j)
                if (allowed(causal, i, j)) {
                    double sij = scale * dot(qi, k + base + (size_t)j * d, d);
                    if (sij > m) m = sij;
                }
            double sum = 0.0;
            for (int j = 0; j < s; ++j)
                if (allowed(causal, i, j))
                    sum += exp(scale * dot(qi, k + base + (size_t)j * d, d) - m);
            const double l = m + log(sum);
            lse[(size_t)hh * s + i] = l;
            double* oi = o + base + (size_t)i * d;
            for (int t = 0; t < d; ++t) oi[t] = 0.0;
            for (int j = 0; j < s; ++j)
                if (allowed(causal, i, j)) {
                    const double p = exp(scale * dot(qi, k + base + (size_t)j * d, d) - l);
                    const double* vj = v + base + (size_t)j * d;
                    for (int t = 0; t < d; ++t) oi[t] += p * vj[t];
                }
        }
    }
}

/* D_i = <dO_i, O_i> for every head and row. */
void oracle_attn_delta(int H, int s, int d, const double* o, const double* dO, double* D) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int hh = 0; hh < H; ++hh)
        for (int i = 0; i < s; ++i) {
            const size_t off = ((size_t)hh * s + i) * d;
            D[(size_t)hh * s + i] = dot(dO + off, o + off, d);
        }
}

/* Backward for every head from Q, K, V, O, dO and lse (definition above).
 * dq, dk, dv are fully overwritten.  `D` is scratch of H*s doubles that
 * receives D_i. */
void oracle_attn_bwd(int H, int s, int d, double scale, int causal,
                     const double* q, const double* k, const double* v,
                     const double* o, const double* dO, const double* lse,
                     double* dq, double* dk, double* dv, double* D) {
    oracle_attn_delta(H, s, d, o, dO, D);

    /* dQ_i = scale * sum_j dS_ij k_j, one query row at a time. */
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int hh = 0; hh < H; ++hh) {
        for (int i = 0; i < s; ++i) {
            const size_t base = (size_t)hh * s * d;
            const double* qi = q + base + (size_t)i * d;
            const double* doi = dO + base + (size_t)i * d;
            const double li = lse[(size_t)hh * s + i], Di = D[(size_t)hh * s + i];
            double* dqi = dq + base + (size_t)i * d;
            for (int t = 0; t < d; ++t) dqi[t] = 0.0;
            for (int j = 0; j < s; ++j) {
                if (!allowed(causal, i, j)) continue;
                const double* kj = k + base + (size_t)j * d;
                const double p = exp(scale * dot(qi, kj, d) - li);
                const double ds = p * (dot(doi, v + base + (size_t)j * d, d) - Di);
                for (int t = 0; t < d; ++t) dqi[t] += ds * kj[t];
            }
            for (int t = 0; t < d; ++t) dqi[t] *= scale;
        }
    }

    /* dV_j = sum_i P_ij dO_i and dK_j = scale * sum_i dS_ij q_i, one key row
     * at a time. */
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int hh = 0; hh < H; ++hh) {
        for (int j = 0; j < s; ++j) {
            const size_t base = (size_t)hh * s * d;
            const double* kj = k + base + (size_t)j * d;
            const double* vj = v + base + (size_t)j * d;
            double* dkj = dk + base + (size_t)j * d;
            double* dvj = dv + base + (size_t)j * d;
            for (int t = 0; t < d; ++t) { dkj[t] = 0.0; dvj[t] = 0.0; }
            for (int i = 0; i < s; ++i) {
                if (!allowed(causal, i, j)) continue;
                const double* qi = q + base + (size_t)i * d;
                const double* doi = dO + base + (size_t)i * d;
                const double p = exp(scale * dot(qi, kj, d) - lse[(size_t)hh * s + i]);
                const double ds = p * (dot(doi, vj, d) - D[(size_t)hh * s + i]);
                for (int t = 0; t < d; ++t) {
                    dvj[t] += p * doi[t];
                    dkj[t] += ds * qi[t];
                }
            }
            for (int t = 0; t < d; ++t) dkj[t] *= scale;
        }
    }
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
