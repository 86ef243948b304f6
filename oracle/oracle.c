/*
 * CPU oracle for the CSR graph-attention path.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It is the plain definition of every step, written as
 * per-row / per-edge loops in double precision, so that a reader can check it
 * against the definitions by eye.  It shares no code, header or helper with the
 * HIP library; neither side includes or calls the other.
 *
 * Sources of the definitions (POPCORNBENCH kernel-writing transcripts):
 *   [l1_p10] edge-only SDDMM: the reference model gathers src_feat[src_idx]
 *            and dst_feat[dst_idx] and sums their product over the feature dim.
 *   [l1_p6]  multi-head row-wise softmax over CSR edge scores: the reference
 *            loops over nodes and applies a softmax over the edge slice
 *            scores[row_ptr[i]:row_ptr[i+1], h] for every head, computed as
 *            exp(x - max) / sum(exp(x - max)).
 *   [l1_p18] multi-head sparse aggregation: out[i,h,:] is the sum over the
 *            row's edges of edge_weight[e,h] * node_feat[col_idx[e],h,:];
 *            the output starts from zeros.
 *   [l2_p37] CSR neighbourhood attention: softmax of the row's edge scores,
 *            then the weighted sum of node_value[col_idx[e]]; rows with no edges
 *            keep their zero output.
 *   [l2_p4]  dense masked attention with a relation-MLP bias: LayerNorm, q/k/v
 *            nn.Linear projections, biased masked softmax, output projection and
 *            residual; its linear projections are also the node projections on
 *            either side of the graph layer.
 * The full layer (scores from q_i . k_j, then softmax, then aggregation of v)
 * is the composition of the three steps above; no single page writes it out.
 * The backward functions at the end are the derivatives of these definitions
 * (chain rule); no page writes them out either.
 *
 * Precision: every floating-point input is widened exactly to double (bf16 is
 * decoded bit-exactly) and all arithmetic is double; results are returned as
 * double.  Outer loops over independent rows / edges may run on several
 * threads (OpenMP); that does not change any result.
 *
 * Pins (tests/test_oracle_pins.py): dense brute force with library matmul and
 * softmax on tiny graphs (with edge multiplicities), closed forms (degree-1
 * rows, constant scores, two-edge logistic), invariants (rows sum to one,
 * shift invariance, zero rows give +0.0, linearity, edge permutation within a
 * row), exact integer arithmetic, and mutation runs showing that planted
 * mistakes in this file fail at least one pin.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2

/* Element idx of a feature table stored as fp32, bf16 (raw bits) or fp64, widened exactly. */
static double load_feat(const void* base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    if (dtype == ORACLE_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double*)base)[idx];
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    return 1;
#endif
}

/* Threads for the following calls (benchmark use: the one-thread CPU figure). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

/*
 * SDDMM over an edge list [l1_p10]:
 *   out[e,h] = scale * sum_d dst_feat[dst_idx[e],h,d] * src_feat[src_idx[e],h,d]
 * Features are [n,heads,head_dim] row-major; out is [n_edges,heads].
 */
int oracle_sddmm(int64_t n_edges, const int32_t* src_idx, const int32_t* dst_idx,
                 const void* src_feat, const void* dst_feat, int dtype,
                 int heads, int head_dim, double scale, double* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n_edges; ++e) {
        for (int h = 0; h < heads; ++h) {
            int64_t a = ((int64_t)dst_idx[e] * heads + h) * head_dim;
            int64_t b = ((int64_t)src_idx[e] * heads + h) * head_dim;
            double acc = 0.0;
            for (int d = 0; d < head_dim; ++d)
                acc += load_feat(dst_feat, dtype, a + d) * load_feat(src_feat, dtype, b + d);
            out[e * heads + h] = scale * acc;
        }
    }
    return 0;
}

/*
 * Row-wise multi-head edge softmax [l1_p6]: for every row i with at least one
 * edge and every head h, over e in [row_ptr[i], row_ptr[i+1]):
 *   m = max_e s[e,h];  z = sum_e exp(s[e,h] - m);  out[e,h] = exp(s[e,h] - m) / z
 * Rows without edges have no entries.  scores/out are [n_edges,heads].
 */
int oracle_edge_softmax(int64_t n_rows, const int32_t* row_ptr, int heads,
                        const double* scores, double* out)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t start = row_ptr[i], end = row_ptr[i + 1];
        if (end <= start) continue;
        for (int h = 0; h < heads; ++h) {
            double m = -INFINITY;
            for (int64_t e = start; e < end; ++e)
                if (scores[e * heads + h] > m) m = scores[e * heads + h];
            double z = 0.0;
            for (int64_t e = start; e < end; ++e)
                z += exp(scores[e * heads + h] - m);
            for (int64_t e = start; e < end; ++e)
                out[e * heads + h] = exp(scores[e * heads + h] - m) / z;
        }
    }
    return 0;
}

/*
 * Weighted neighbour aggregation (SpMM) [l1_p18]:
 *   out[i,h,d] = sum_{e in row i} weights[e,h] * feat[col_idx[e],h,d]
 * starting from 0.0, so rows without edges are +0.0.  out is [n_rows,heads,head_dim].
 */
int oracle_aggregate(int64_t n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                     int heads, int head_dim, const double* weights,
                     const void* feat, int dtype, double* out)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t start = row_ptr[i], end = row_ptr[i + 1];
        for (int h = 0; h < heads; ++h) {
            for (int d = 0; d < head_dim; ++d) {
                double acc = 0.0;
                for (int64_t e = start; e < end; ++e)
                    acc += weights[e * heads + h] *
                           load_feat(feat, dtype, ((int64_t)col_idx[e] * heads + h) * head_dim + d);
                out[(i * heads + h) * head_dim + d] = acc;
            }
        }
    }
    return 0;
}

/*
 * Neighbourhood softmax + aggregation [l2_p37]: aggregate(softmax(scores)).
 * The edge weights are materialised in a temporary [n_edges,heads] buffer.
 */
int oracle_softmax_aggregate(int64_t n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                             int heads, int head_dim, const double* scores,
                             const void* feat, int dtype, double* out)
{
    int64_t n_edges = row_ptr[n_rows];
    double* alpha = (double*)malloc((size_t)(n_edges > 0 ? n_edges : 1) * heads * sizeof(double));
    if (!alpha) return 1;
    oracle_edge_softmax(n_rows, row_ptr, heads, scores, alpha);
    oracle_aggregate(n_rows, row_ptr, col_idx, heads, head_dim, alpha, feat, dtype, out);
    free(alpha);
    return 0;
}

/*
 * Full layer: scores[e,h] = scale * <q[i,h,:], k[col_idx[e],h,:]> for every edge
 * e of row i (the SDDMM with dst = row, src = column), then softmax +
 * aggregation of v.  q is [n_rows,heads,head_dim]; k and v are [n_src,heads,head_dim].
 */
int oracle_layer(int64_t n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                 int heads, int head_dim, const void* q, const void* k, const void* v,
                 int dtype, double scale, double* out)
{
    int64_t n_edges = row_ptr[n_rows];
    size_t ne = (size_t)(n_edges > 0 ? n_edges : 1);
    int32_t* dst = (int32_t*)malloc(ne * sizeof(int32_t));
    double* scores = (double*)malloc(ne * heads * sizeof(double));
    if (!dst || !scores) { free(dst); free(scores); return 1; }
    for (int64_t i = 0; i < n_rows; ++i)
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e)
            dst[e] = (int32_t)i;
    oracle_sddmm(n_edges, col_idx, dst, k, q, dtype, heads, head_dim, scale, scores);
    int rc = oracle_softmax_aggregate(n_rows, row_ptr, col_idx, heads, head_dim, scores, v, dtype, out);
    free(dst);
    free(scores);
    return rc;
}

/* ------------------------------------------------------------------------------------------
 * Backward.  No page writes the backward pass out; the l1_p10 page (edge-only SDDMM) notes that
 * gradients flow back to rows of the feature tables, summed over the edges that read each row.
 * Each function below is the derivative of the forward definition above it (chain rule), as
 * plain loops in double precision.  grad arguments are dL/d(output) of the forward step.
 * ------------------------------------------------------------------------------------------ */

/*
 * SDDMM backward over an edge list, g = dL/dout [n_edges,heads] of oracle_sddmm:
 *   d_dst[dst_idx[e],h,d] = sum over edges e of scale * g[e,h] * src_feat[src_idx[e],h,d]
 *   d_src[src_idx[e],h,d] = sum over edges e of scale * g[e,h] * dst_feat[dst_idx[e],h,d]
 * The l1_p10 page notes that the gradients accumulate into the rows of the two feature tables the
 * edges read.  Both outputs start at 0.0 (rows no edge reads stay +0.0); every sum visits the
 * edges in increasing edge id.  Threads split (output table, head) pairs, so no two write one
 * value.
 */
int oracle_sddmm_backward(int64_t n_edges, const int32_t* src_idx, const int32_t* dst_idx,
                          const void* src_feat, int64_t n_src, const void* dst_feat, int64_t n_dst, int dtype,
                          int heads, int head_dim, double scale, const double* grad, double* d_src,
                          double* d_dst)
{
    for (int64_t x = 0; x < n_src * heads * head_dim; ++x)
        d_src[x] = 0.0;
    for (int64_t x = 0; x < n_dst * heads * head_dim; ++x)
        d_dst[x] = 0.0;
#pragma omp parallel for schedule(static)
    for (int task = 0; task < 2 * heads; ++task) {
        int h = task / 2;
        int to_dst = task % 2;   /* 1: d_dst (reads src_feat); 0: d_src (reads dst_feat) */
        for (int64_t e = 0; e < n_edges; ++e) {
            double w = scale * grad[e * heads + h];
            int64_t out_row = to_dst ? dst_idx[e] : src_idx[e];
            int64_t in_row = to_dst ? src_idx[e] : dst_idx[e];
            const void* in = to_dst ? src_feat : dst_feat;
            double* out = to_dst ? d_dst : d_src;
            for (int d = 0; d < head_dim; ++d)
                out[(out_row * heads + h) * head_dim + d] += w * load_feat(in, dtype, (in_row * heads + h) * head_dim + d);
        }
    }
    return 0;
}

/*
 * Edge softmax backward: for every row i with edges and every head h, with a = softmax output
 * and g = dL/da over the row's edges:
 *   out[e,h] = a[e,h] * (g[e,h] - sum_{e' in row i} a[e',h] * g[e',h])
 * (the softmax Jacobian diag(a) - a a^T applied to g).
 */
int oracle_edge_softmax_backward(int64_t n_rows, const int32_t* row_ptr, int heads,
                                 const double* alpha, const double* grad, double* out)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t start = row_ptr[i], end = row_ptr[i + 1];
        for (int h = 0; h < heads; ++h) {
            double dot = 0.0;
            for (int64_t e = start; e < end; ++e)
                dot += alpha[e * heads + h] * grad[e * heads + h];
            for (int64_t e = start; e < end; ++e)
                out[e * heads + h] = alpha[e * heads + h] * (grad[e * heads + h] - dot);
        }
    }
    return 0;
}

/*
 * Aggregation backward, g = dL/dout [n_rows,heads,head_dim]:
 *   dweights[e,h] = sum_d g[i,h,d] * feat[col_idx[e],h,d]            (e in row i)
 *   dfeat[j,h,d]  = sum over edges e with col_idx[e] = j of weights[e,h] * g[row of e,h,d]
 * dfeat is [n_src,heads,head_dim] and starts at 0.0 (sources no edge reads stay +0.0); its sums
 * visit the edges in increasing edge id.  Threads split the heads, so no two write one value.
 */
int oracle_aggregate_backward(int64_t n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                              int heads, int head_dim, int64_t n_src, const double* weights,
                              const void* feat, int dtype, const double* grad,
                              double* dweights, double* dfeat)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n_rows; ++i) {
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            for (int h = 0; h < heads; ++h) {
                double acc = 0.0;
                for (int d = 0; d < head_dim; ++d)
                    acc += grad[(i * heads + h) * head_dim + d] *
                           load_feat(feat, dtype, ((int64_t)col_idx[e] * heads + h) * head_dim + d);
                dweights[e * heads + h] = acc;
            }
        }
    }
    for (int64_t x = 0; x < n_src * heads * head_dim; ++x)
        dfeat[x] = 0.0;
#pragma omp parallel for schedule(static)
    for (int h = 0; h < heads; ++h) {
        for (int64_t i = 0; i < n_rows; ++i) {
            for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
                int64_t j = col_idx[e];
                for (int d = 0; d < head_dim; ++d)
                    dfeat[(j * heads + h) * head_dim + d] += weights[e * heads + h] * grad[(i * heads + h) * head_dim + d];
            }
        }
    }
    return 0;
}

/*
 * Softmax + aggregation backward: a = softmax(scores); (g_a, dfeat) = aggregation backward of
 * a and feat; dscores = softmax backward of (a, g_a).
 */
int oracle_softmax_aggregate_backward(int64_t n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                                      int heads, int head_dim, int64_t n_src, const double* scores,
                                      const void* feat, int dtype, const double* grad,
                                      double* dscores, double* dfeat)
{
    int64_t n_edges = row_ptr[n_rows];
    size_t ne = (size_t)(n_edges > 0 ? n_edges : 1) * heads;
    double* alpha = (double*)malloc(ne * sizeof(double));
    double* ga = (double*)malloc(ne * sizeof(double));
    if (!alpha || !ga) { free(alpha); free(ga); return 1; }
    oracle_edge_softmax(n_rows, row_ptr, heads, scores, alpha);
    oracle_aggregate_backward(n_rows, row_ptr, col_idx, heads, head_dim, n_src, alpha, feat, dtype, grad, ga, dfeat);
    oracle_edge_softmax_backward(n_rows, row_ptr, heads, alpha, ga, dscores);
    free(alpha);
    free(ga);
    return 0;
}

/*
 * Full layer backward (q [n_rows,H,D]; k, v [n_src,H,D]), with s = scale * <q_i, k_j>,
 * a = softmax(s) per row, out_i = sum_e a[e] v_j:
 *   (g_a, dv) = aggregation backward of (a, v, g)
 *   g_s       = softmax backward of (a, g_a)
 *   dq[i]     = scale * sum_{e in row i} g_s[e] * k[col_idx[e]]
 *   dk[j]     = scale * sum over edges e with col_idx[e] = j of g_s[e] * q[row of e]
 * per head.  dk and dv start at 0.0.
 */
int oracle_layer_backward(int64_t n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                          int heads, int head_dim, int64_t n_src, const void* q, const void* k,
                          const void* v, int dtype, double scale, const double* grad,
                          double* dq, double* dk, double* dv)
{
    int64_t n_edges = row_ptr[n_rows];
    size_t ne = (size_t)(n_edges > 0 ? n_edges : 1);
    int32_t* row_of = (int32_t*)malloc(ne * sizeof(int32_t));
    double* s = (double*)malloc(ne * heads * sizeof(double));
    double* a = (double*)malloc(ne * heads * sizeof(double));
    double* ga = (double*)malloc(ne * heads * sizeof(double));
    double* gs = (double*)malloc(ne * heads * sizeof(double));
    if (!row_of || !s || !a || !ga || !gs) { free(row_of); free(s); free(a); free(ga); free(gs); return 1; }
    for (int64_t i = 0; i < n_rows; ++i)
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e)
            row_of[e] = (int32_t)i;
    oracle_sddmm(n_edges, col_idx, row_of, k, q, dtype, heads, head_dim, scale, s);
    oracle_edge_softmax(n_rows, row_ptr, heads, s, a);
    oracle_aggregate_backward(n_rows, row_ptr, col_idx, heads, head_dim, n_src, a, v, dtype, grad, ga, dv);
    oracle_edge_softmax_backward(n_rows, row_ptr, heads, a, ga, gs);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n_rows; ++i) {
        for (int h = 0; h < heads; ++h) {
            for (int d = 0; d < head_dim; ++d) {
                double gsum = 0.0;
                for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e)
                    gsum += gs[e * heads + h] *
                            load_feat(k, dtype, ((int64_t)col_idx[e] * heads + h) * head_dim + d);
                dq[(i * heads + h) * head_dim + d] = scale * gsum;
            }
        }
    }
    for (int64_t x = 0; x < n_src * heads * head_dim; ++x)
        dk[x] = 0.0;
#pragma omp parallel for schedule(static)
    for (int h = 0; h < heads; ++h) {
        for (int64_t e = 0; e < n_edges; ++e) {
            int64_t i = row_of[e], j = col_idx[e];
            for (int d = 0; d < head_dim; ++d)
                dk[(j * heads + h) * head_dim + d] +=
                    scale * gs[e * heads + h] * load_feat(q, dtype, (i * heads + h) * head_dim + d);
        }
    }
    free(row_of);
    free(s);
    free(a);
    free(ga);
    free(gs);
    return 0;
}

/* ------------------------------------------------------------------------------------------
 * Dense relation-biased attention block (l2_p4, the reference-model passage): for each batch
 * element b, with nodes x [N,D], pair features f [N,N,P] and an edge mask [N,N]:
 *   xn  = LayerNorm(x) over D: (x - mean) / sqrt(var + eps) * gamma + beta   (biased variance)
 *   q, k, v = xn Wq^T, xn Wk^T, xn Wv^T          (nn.Linear without bias; W is [out, in])
 *   bias[h,i,j] = (W2 silu(W1 f[i,j] + b1) + b2)[h],  silu(t) = t / (1 + exp(-t))
 *   logit[h,i,j] = <q_i, k_j>_h / sqrt(D/H) + bias[h,i,j]   over head h's D/H columns,
 *                  -inf where mask[i,j] < 0.5
 *   a[h,i,:] = softmax_j(logit[h,i,:]);  a row whose entries are all masked is all zeros
 *   o[i, h-block] = sum_j a[h,i,j] v_j[h-block]
 *   out = x + o Wo^T                              (residual on the un-normalised nodes)
 * All arrays double, row-major: nodes/out [B,N,D], pair [B,N,N,P], mask [B,N,N], gamma/beta [D],
 * wq/wk/wv/wo [D,D], w1 [P,P], b1 [P], w2 [H,P], b2 [H].
 * ------------------------------------------------------------------------------------------ */
int oracle_relation_attention(int64_t B, int64_t N, int D, int H, int P, const double* nodes,
                              const double* pair, const double* mask, const double* gamma,
                              const double* beta, double eps, const double* wq, const double* wk,
                              const double* wv, const double* wo, const double* w1, const double* b1,
                              const double* w2, const double* b2, double* out)
{
    int hd = D / H;
    double scale = 1.0 / sqrt((double)hd);
    size_t nd = (size_t)(N > 0 ? N : 1) * D;
    for (int64_t b = 0; b < B; ++b) {
        const double* x = nodes + b * N * D;
        double* xn = (double*)malloc(nd * sizeof(double));
        double* q = (double*)malloc(nd * sizeof(double));
        double* k = (double*)malloc(nd * sizeof(double));
        double* v = (double*)malloc(nd * sizeof(double));
        double* o = (double*)malloc(nd * sizeof(double));
        double* lg = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        double* hid = (double*)malloc((size_t)P * sizeof(double));
        if (!xn || !q || !k || !v || !o || !lg || !hid) {
            free(xn); free(q); free(k); free(v); free(o); free(lg); free(hid);
            return 1;
        }
        for (int64_t i = 0; i < N; ++i) {
            double mean = 0.0, var = 0.0;
            for (int d = 0; d < D; ++d) mean += x[i * D + d];
            mean /= D;
            for (int d = 0; d < D; ++d) var += (x[i * D + d] - mean) * (x[i * D + d] - mean);
            var /= D;
            for (int d = 0; d < D; ++d)
                xn[i * D + d] = (x[i * D + d] - mean) / sqrt(var + eps) * gamma[d] + beta[d];
        }
        for (int64_t i = 0; i < N; ++i) {
            for (int r = 0; r < D; ++r) {
                double sq = 0.0, sk = 0.0, sv = 0.0;
                for (int c = 0; c < D; ++c) {
                    sq += xn[i * D + c] * wq[r * D + c];
                    sk += xn[i * D + c] * wk[r * D + c];
                    sv += xn[i * D + c] * wv[r * D + c];
                }
                q[i * D + r] = sq;
                k[i * D + r] = sk;
                v[i * D + r] = sv;
            }
        }
        for (int h = 0; h < H; ++h) {
            for (int64_t i = 0; i < N; ++i) {
                int any = 0;
                double mx = -INFINITY;
                for (int64_t j = 0; j < N; ++j) {
                    lg[j] = -INFINITY;
                    if (mask[(b * N + i) * N + j] < 0.5) continue;
                    const double* f = pair + ((b * N + i) * N + j) * P;
                    double rb = b2[h];
                    for (int p = 0; p < P; ++p) {
                        double t = b1[p];
                        for (int c = 0; c < P; ++c) t += w1[p * P + c] * f[c];
                        hid[p] = t / (1.0 + exp(-t));
                    }
                    for (int p = 0; p < P; ++p) rb += w2[h * P + p] * hid[p];
                    double dot = 0.0;
                    for (int t = 0; t < hd; ++t) dot += q[i * D + h * hd + t] * k[j * D + h * hd + t];
                    lg[j] = dot * scale + rb;
                    any = 1;
                    if (lg[j] > mx) mx = lg[j];
                }
                double z = 0.0;
                if (any)
                    for (int64_t j = 0; j < N; ++j)
                        if (lg[j] != -INFINITY) z += exp(lg[j] - mx);
                for (int t = 0; t < hd; ++t) {
                    double acc = 0.0;
                    if (any)
                        for (int64_t j = 0; j < N; ++j)
                            if (lg[j] != -INFINITY) acc += exp(lg[j] - mx) / z * v[j * D + h * hd + t];
                    o[i * D + h * hd + t] = acc;
                }
            }
        }
        for (int64_t i = 0; i < N; ++i) {
            for (int r = 0; r < D; ++r) {
                double s = 0.0;
                for (int c = 0; c < D; ++c) s += o[i * D + c] * wo[r * D + c];
                out[(b * N + i) * D + r] = x[i * D + r] + s;
            }
        }
        free(xn); free(q); free(k); free(v); free(o); free(lg); free(hid);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------
 * Node projection: the nn.Linear steps on either side of the attention in the l2_p4 reference
 * model (the q/k/v projections of the node rows and the output projection):
 *   out[m, n] = bias[n] + sum_k x[m, k] * w[n, k]      (w stored [out_features, in_features])
 * x [M,K] and w [N,K] as fp32, bf16 (raw bits) or fp64, widened exactly; bias [N] double, or
 * NULL for none; out [M,N] double.
 * ------------------------------------------------------------------------------------------ */
int oracle_linear(int64_t M, int K, int N, const void* x, int x_dtype, const void* w, int w_dtype,
                  const double* bias, double* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int n = 0; n < N; ++n) {
            double s = bias ? bias[n] : 0.0;
            for (int k = 0; k < K; ++k)
                s += load_feat(x, x_dtype, m * K + k) * load_feat(w, w_dtype, (int64_t)n * K + k);
            out[m * N + n] = s;
        }
    }
    return 0;
}
