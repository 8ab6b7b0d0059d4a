/*
 * TEST INFRASTRUCTURE ONLY -- the fp64 reference ("oracle") for the gated
 * delta rule.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark may call it; the product path never links it.
 *
 * What it computes is the definition of the method, token by token:
 *
 *   S_t = S_{t-1} ( D_t (I - beta_t k_t k_t^T) ) + beta_t v_t k_t^T ,
 *   o_t = S_t (scale q_t)
 *
 * ("TileLang 实战：KDA 从零到一--Gated DeltaNet", introduction and §1.1;
 *  "Gated Delta Network（GDN）", eq. 4 and eq. 12), where D_t = alpha_t I with
 * alpha_t = exp(g_t) for the scalar gate, and D_t = Diag(exp(g_t)) for the
 * per-key-channel gate of Kimi Delta Attention ("DeltaNet 系列线性注意力变体的
 * 推导之旅", KDA section: forget first, then predict, then correct).  For the
 * scalar gate both placements of alpha_t agree because alpha_t I commutes.
 *
 * The state is kept transposed, h = S^T with shape [K][V] (key rows, value
 * columns), as the kernels on those pages store it.  Transposing the update
 * gives
 *
 *   h_t = (I - beta_t k_t k_t^T) D_t h_{t-1} + beta_t k_t v_t^T
 *       = h' + k_t (beta_t (v_t - h'^T k_t))^T ,   h' = D_t h_{t-1}
 *   o_t = h_t^T (scale q_t)            (the read follows the token's write)
 *
 * which costs O(K V) per token; no K-by-K matrix is ever formed.
 *
 * All arithmetic is IEEE double; build without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Layouts (row-major, tokens packed back to back):
 *   q, k  [T_total][H][K]      v, o  [T_total][H][V]
 *   beta  [T_total][H]         g     [T_total][H]  or  [T_total][H][K]
 *   h0,ht [n_seqs][H][K][V]    cu_seqlens [n_seqs + 1] token offsets
 * h0 == NULL means a zero initial state; ht == NULL means "do not return".
 * Returns 0 on success, -1 on bad arguments, -2 when out of memory. */
int oracle_gdn_forward(int64_t n_seqs, const int64_t *cu_seqlens,
                       int64_t H, int64_t K, int64_t V,
                       const double *q, const double *k, const double *v,
                       const double *beta, const double *g, int gate_per_key,
                       double scale, const double *h0, double *o, double *ht,
                       int n_threads)
{
    if (n_seqs < 0 || H <= 0 || K <= 0 || V <= 0 || !cu_seqlens)
        return -1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    int64_t pairs = n_seqs * H;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t p = 0; p < pairs; ++p) {
        int64_t n = p / H, hh = p % H;
        double *h = (double *)malloc(sizeof(double) * (size_t)(K * V));
        double *pred = (double *)malloc(sizeof(double) * (size_t)V);
        double *decay = (double *)malloc(sizeof(double) * (size_t)K);
        if (!h || !pred || !decay) {
            free(h); free(pred); free(decay);
            failed |= 1;
            continue;
        }
        if (h0) memcpy(h, h0 + (n * H + hh) * K * V, sizeof(double) * (size_t)(K * V));
        else memset(h, 0, sizeof(double) * (size_t)(K * V));

        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            const double *qt = q + (t * H + hh) * K;
            const double *kt = k + (t * H + hh) * K;
            const double *vt = v + (t * H + hh) * V;
            double bt = beta[t * H + hh];
            double *ot = o + (t * H + hh) * V;

            /* forget: h' = D_t h */
            if (gate_per_key) {
                const double *gt = g + (t * H + hh) * K;
                for (int64_t i = 0; i < K; ++i) decay[i] = exp(gt[i]);
            } else {
                double a = exp(g[t * H + hh]);
                for (int64_t i = 0; i < K; ++i) decay[i] = a;
            }
            for (int64_t i = 0; i < K; ++i)
                for (int64_t j = 0; j < V; ++j) h[i * V + j] *= decay[i];

            /* predict: what the decayed memory returns for k_t, h'^T k_t */
            for (int64_t j = 0; j < V; ++j) pred[j] = 0.0;
            for (int64_t i = 0; i < K; ++i)
                for (int64_t j = 0; j < V; ++j) pred[j] += h[i * V + j] * kt[i];

            /* correct: write beta_t (v_t - prediction) along k_t */
            for (int64_t j = 0; j < V; ++j) pred[j] = bt * (vt[j] - pred[j]);
            for (int64_t i = 0; i < K; ++i)
                for (int64_t j = 0; j < V; ++j) h[i * V + j] += kt[i] * pred[j];

            /* read with the updated state: o_t = h_t^T (scale q_t) */
            for (int64_t j = 0; j < V; ++j) ot[j] = 0.0;
            for (int64_t i = 0; i < K; ++i) {
                double sq = scale * qt[i];
                for (int64_t j = 0; j < V; ++j) ot[j] += h[i * V + j] * sq;
            }
        }
        if (ht) memcpy(ht + (n * H + hh) * K * V, h, sizeof(double) * (size_t)(K * V));
        free(h); free(pred); free(decay);
    }
    return failed ? -2 : 0;
}

int oracle_abi_version(void) { return 1; }
