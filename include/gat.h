/*
 * gat.h -- C-ABI of libgat.so: CSR graph-attention message passing on MI355X (gfx950).
 *
 * The operations follow the POPCORNBENCH kernel-writing transcripts:
 *   [l1_p10] edge-only SDDMM, reference-model passage: out[e] is the dot product of
 *            src_feat[src_idx[e]] and dst_feat[dst_idx[e]] over the feature dim.
 *   [l1_p6]  multi-head row-wise softmax over CSR edge scores, reference-model
 *            passage: for every node and head, softmax over the node's edge slice,
 *            computed as exp(x - max) / sum(exp(x - max)).
 *   [l1_p18] multi-head sparse aggregation with per-edge, per-head weights, task
 *            statement: out[i,h,:] = sum over the row's edges of
 *            edge_weight[e,h] * node_feat[col_idx[e],h,:], starting from zeros.
 *   [l2_p37] CSR graph-attention neighbourhood softmax + aggregation, reference-model
 *            passage: softmax over the row's edge scores, then the weighted sum of
 *            node_value[col_idx[e]]; a row without edges keeps a zero output.
 * The full layer (scores q_i . k_j computed on the fly, then [l2_p37] on v) is the
 * composition of those steps.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers (memory of the current HIP device) unless the
 *    comment says host.  The caller owns every buffer; the library allocates and
 *    frees nothing and keeps no state between calls (the one exception,
 *    gat_fused_layer_noalloc, keeps its plan in a device array of its own).
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *    without waiting.  No entry point synchronises.
 *  - Layouts (row-major, contiguous):
 *      row_ptr  int32 [n_rows + 1], row_ptr[0] = 0, non-decreasing, row_ptr[n_rows] = n_edges
 *      col_idx  int32 [n_edges], 0 <= col_idx[e] < n_src; edges of row i are
 *               [row_ptr[i], row_ptr[i+1]); duplicates are allowed and each is its
 *               own softmax term; order inside a row is free
 *      scores / weights / alpha   fp32 [n_edges, heads] (edge-major)
 *      features (feat, q, k, v, src_feat, dst_feat)  [n, heads, head_dim] of
 *               dtype GAT_F32 (float) or GAT_BF16 (raw bfloat16 bits)
 *      out of aggregate / fused_layer   fp32 [n_rows, heads, head_dim]
 *    The CSR/COO preconditions above are not checked on the device.
 *  - Supported shapes: head_dim in {16, 32, 64, 128}, heads in {1, 2, 4, 8, 16},
 *    heads * head_dim <= 1024; anything else returns GAT_ERR_UNSUPPORTED.
 *    n_rows and n_src must be in [0, 2^31 - 1], n_edges in [0, 2^31 - 4097]
 *    (GAT_ERR_SIZE otherwise).
 *  - Arithmetic is fp32 (bf16 inputs are widened exactly); exp is the hardware
 *    exp2 of x*log2(e).  Outputs are fully overwritten: a row without edges gets
 *    +0.0 in every element, so outputs need no clearing.
 *  - Errors: every argument check runs on the host before anything is enqueued;
 *    a failed check returns its status and enqueues nothing.  A launch failure
 *    returns GAT_ERR_HIP.  No C++ exception crosses this interface.
 */
#ifndef GAT_H
#define GAT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gat_dtype { GAT_F32 = 0, GAT_BF16 = 1 } gat_dtype;

typedef enum gat_status {
    GAT_OK = 0,
    GAT_ERR_NULL = 1,         /* a required pointer is NULL */
    GAT_ERR_SIZE = 2,         /* a size is negative or does not fit int32 */
    GAT_ERR_UNSUPPORTED = 3,  /* (heads, head_dim, dtype) outside the supported set */
    GAT_ERR_WORKSPACE = 4,    /* plan workspace too small, or plan built for another row_ptr or sizes */
    GAT_ERR_ARGS = 5,         /* inconsistent arguments (e.g. both or neither of scores / q,k) */
    GAT_ERR_HIP = 6,          /* a HIP call or kernel launch failed */
    GAT_ERR_SCRATCH = 7       /* the graph's plan exceeds the library's fixed scratch array */
} gat_status;

/* Degree-binning defaults: rows with deg <= short_max are handled by one lane group
 * (a wave or a fraction of one); rows with short_max < deg <= seg_len by one
 * 256-thread workgroup; longer rows are split into segments of seg_len edges
 * whose partial results are merged afterwards. */
#define GAT_DEFAULT_SHORT_MAX 64
#define GAT_DEFAULT_SEG_LEN 1024

/*
 * Degree-binning plan.  Host-side POD filled by gat_plan_build; the tables it
 * points to live in the caller's device workspace `ws`.  A plan is valid for the
 * row_ptr it was built from, while `ws` is alive and unchanged.  Fields are
 * read-only for the caller (tests inspect the tables through the offsets).
 *   segment table  int32 [seg_capacity][4]: (row, e_begin, e_end, slot); every
 *                  hub segment first (slot = its index), then every long row
 *                  (slot = -1), both in increasing row id.
 *   hub table      int32 [hub_capacity][4]: (row, first segment, n segments, 0)
 *   counts         int32 [8]: n_segments, n_hub_segments, n_hubs, n_long_rows, overflow
 *                  (overflow = 1: the degrees of row_ptr sum past what n_edges allows, i.e.
 *                  row_ptr[n_rows] > n_edges; every table is then left empty, nothing is
 *                  written past the workspace, and rows above short_max get no output)
 *   partials       fp32 [hubseg_capacity][state_floats]: per hub segment
 *                  (max[heads], sum[heads], acc[heads*head_dim])
 */
typedef struct gat_plan {
    int64_t n_rows, n_edges;
    int32_t short_max, seg_len;
    int32_t heads, head_dim;         /* partial-state capacity: calls need heads*(head_dim+2) <= state_floats */
    int64_t state_floats;
    int64_t seg_capacity, hub_capacity, hubseg_capacity;
    int64_t n_blocks;                /* binner blocks */
    void* ws;
    size_t ws_bytes;
    const int32_t* row_ptr;          /* the array the plan was built from; calls must pass the same one */
    size_t off_counts, off_blocks, off_segs, off_hubs, off_partials;   /* byte offsets into ws */
    uint32_t magic;
} gat_plan;

/*
 * Bytes of device workspace gat_plan_build needs for these sizes.  heads/head_dim
 * bound the partial-state size of later calls.  short_max < 0 or seg_len <= 0
 * select the defaults.  Returns 0 for invalid sizes.  Host only; no HIP call.
 */
size_t gat_plan_workspace_bytes(int64_t n_rows, int64_t n_edges, int heads, int head_dim,
                                int short_max, int seg_len);

/*
 * Degree binning (the plan): classifies every row by degree and writes the
 * segment and hub tables into `ws` (device memory of at least
 * gat_plan_workspace_bytes(...) bytes, 256-byte aligned).  Three kernels on
 * `stream`; nothing is copied to the host, so the call does not synchronise --
 * the kernels that use the plan read the counts on the device.  `plan` is a host
 * pointer, filled before the call returns.
 * This replaces the host-side maximum-degree pass of [l2_p37] (its passages on
 * copying row_ptr to the host to size shared memory by max_degree).
 */
gat_status gat_plan_build(const int32_t* row_ptr, int64_t n_rows, int64_t n_edges,
                          int heads, int head_dim, int short_max, int seg_len,
                          void* ws, size_t ws_bytes, gat_plan* plan, hipStream_t stream);

/*
 * SDDMM over an edge list [l1_p10], multi-head:
 *   out[e,h] = scale * sum_d dst_feat[dst_idx[e],h,d] * src_feat[src_idx[e],h,d]
 * src_idx/dst_idx int32 [n_edges]; src_feat [n_src,heads,head_dim]; dst_feat
 * [n_dst,heads,head_dim]; out fp32 [n_edges,heads].  fp32 accumulation.
 */
gat_status gat_sddmm(const int32_t* src_idx, const int32_t* dst_idx, int64_t n_edges,
                     const void* src_feat, int64_t n_src, const void* dst_feat, int64_t n_dst,
                     gat_dtype dtype, int heads, int head_dim, float scale,
                     float* out, hipStream_t stream);

/*
 * Row-wise multi-head edge softmax [l1_p6]:
 *   alpha[e,h] = exp(s[e,h] - m_ih) / sum_{e' in row i} exp(s[e',h] - m_ih),  m_ih = max over the row
 * scores/out fp32 [n_edges,heads]; out may equal scores (in place).  Entries of
 * rows without edges do not exist.  plan: NULL (every row by one lane group) or a
 * plan built for this row_ptr with heads*(head_dim+2) >= 2*heads.
 */
gat_status gat_edge_softmax(const int32_t* row_ptr, int64_t n_rows, int64_t n_edges, int heads,
                            const float* scores, float* out, const gat_plan* plan, hipStream_t stream);

/*
 * Weighted aggregation / SpMM [l1_p18]:
 *   out[i,h,:] = sum_{e in row i} weights[e,h] * feat[col_idx[e],h,:]   (+0.0 for rows without edges)
 * weights fp32 [n_edges,heads]; feat [n_src,heads,head_dim] of `dtype`; out fp32
 * [n_rows,heads,head_dim].  plan: NULL or built for this row_ptr.
 */
gat_status gat_aggregate(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                         int64_t n_edges, const float* weights, const void* feat, gat_dtype dtype,
                         int heads, int head_dim, float* out, const gat_plan* plan, hipStream_t stream);

/*
 * Fused attention aggregation.  When n_edges > 0, exactly one of `scores` or the
 * pair (q, k) must be non-NULL, else GAT_ERR_ARGS (with no edges every output row
 * is +0.0 and the pointers are not read).
 *  - scores given [l2_p37]: out = aggregate(edge_softmax(scores), v) in one pass;
 *    the weights alpha never reach memory.
 *  - q, k given (full layer): s[e,h] = scale * <q[i,h,:], k[col_idx[e],h,:]> is
 *    computed on the fly (online max/sum), then the same aggregation of v; no
 *    score reaches memory.  q [n_rows,heads,head_dim], k [n_src,heads,head_dim].
 * v [n_src,heads,head_dim]; q/k/v share `dtype`; out fp32 [n_rows,heads,head_dim],
 * +0.0 for rows without edges.  plan: NULL (every row by one lane group, correct
 * for any degree) or a plan built for this row_ptr.
 */
gat_status gat_fused_layer(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                           int64_t n_edges, int heads, int head_dim, gat_dtype dtype,
                           const float* scores, const void* q, const void* k, float scale,
                           const void* v, float* out, const gat_plan* plan, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): gat_fused_layer with a degree-binning plan (default
 * thresholds) that the call builds itself, on `stream`, in a device array the library owns,
 * instead of a caller workspace.  Same arguments, modes, layouts and results as
 * gat_fused_layer given a plan from gat_plan_build with the default thresholds (the same
 * kernels on the same tables, so the outputs are bitwise equal).
 *  - The array is GAT_NOALLOC_SCRATCH_BYTES per GPU, a file-scope device array: each GPU the
 *    library runs this call on holds it from that call until the process ends.  The call
 *    itself allocates and frees nothing.  Its first call on a device looks the array up
 *    (hipGetSymbolAddress) and loads the library's code object there if needed, so make one
 *    call before capturing a graph.
 *  - A graph whose plan needs more than the array (gat_fused_layer_noalloc_bytes > the
 *    maximum: e.g. 2^20 rows and 2^24 edges at 4 x 64 need 39 MB and fit; 2^22 rows and
 *    2^26 edges at 8 x 16 need 94 MB and do not) returns GAT_ERR_SCRATCH and enqueues nothing.
 *  - Every call on one GPU uses that GPU's one array, which keeps the last call's plan.
 *    Calls that overlap on one GPU (on different streams, or from several host threads
 *    without ordering) race on it and give wrong results; calls ordered on one stream are
 *    safe.  Nothing in the array has to start at zero.
 */
#define GAT_NOALLOC_SCRATCH_BYTES (64u << 20)
gat_status gat_fused_layer_noalloc(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows,
                                   int64_t n_src, int64_t n_edges, int heads, int head_dim,
                                   gat_dtype dtype, const float* scores, const void* q, const void* k,
                                   float scale, const void* v, float* out, hipStream_t stream);

/* Bytes of the library's scratch array that gat_fused_layer_noalloc needs for these sizes
 * (0 for invalid sizes); calls above GAT_NOALLOC_SCRATCH_BYTES are refused.  Host only. */
size_t gat_fused_layer_noalloc_bytes(int64_t n_rows, int64_t n_edges, int heads, int head_dim);

/* Static description of a status code (host; never NULL). */
const char* gat_status_str(gat_status status);

/* 1 if (heads, head_dim) is in the supported set, else 0 (host; no HIP call). */
int gat_shape_supported(int heads, int head_dim);

/* sizeof(gat_plan) as compiled into the library, for bindings that mirror the struct (host). */
size_t gat_plan_sizeof(void);

/*
 * Batch of B CSR graphs as one block-diagonal CSR, assembled on the device.  The l2_p37 page
 * finds its 384-node problem too small for the launch overhead; batched, any number of such graphs
 * is one graph, every entry point above covers the batch in the launches of one call, and each
 * row's result is the same as in its own graph (bit for bit: a row only meets its own edges).
 * Inputs (device, int32): the B graphs' own arrays concatenated -- local_row_ptr [sum_b (N_b+1)]
 * (graph b's row_ptr, starting at 0) and local_col [sum_b E_b] (its source ids, < Ns_b) -- and the
 * prefix sums row_off, edge_off, src_off [B+1] of N_b, E_b, Ns_b (row_off[B] = n_rows,
 * edge_off[B] = n_edges).  Outputs (device, int32): row_ptr [n_rows+1] with
 * row_ptr[row_off[b] + i] = edge_off[b] + (graph b's row_ptr[i]), and col_idx [n_edges] with
 * col_idx[edge_off[b] + e] = src_off[b] + (graph b's col[e]).  Features of the batch are the
 * graphs' tables stacked in the same order.  Enqueued on `stream`; the offsets are not checked on
 * the device.
 */
gat_status gat_batch_csr(const int32_t* local_row_ptr, const int32_t* local_col, const int32_t* row_off,
                         const int32_t* edge_off, const int32_t* src_off, int64_t n_graphs, int64_t n_rows,
                         int64_t n_edges, int32_t* row_ptr, int32_t* col_idx, hipStream_t stream);

/*
 * Dense relation-biased attention block [l2_p4] (reference-model passage), for each of `batch`
 * elements with nodes x [n_nodes,dim], pair features f [n_nodes,n_nodes,pair_dim] and an edge
 * mask [n_nodes,n_nodes]:
 *   xn = LayerNorm(x) over dim: (x - mean) / sqrt(var + eps) * gamma + beta  (biased variance)
 *   q, k, v = xn Wq^T, xn Wk^T, xn Wv^T;  bias[h,i,j] = (W2 silu(W1 f[i,j] + b1) + b2)[h]
 *   logit[h,i,j] = <q_i, k_j>_h / sqrt(dim/heads) + bias[h,i,j], -inf where mask[i,j] < 0.5
 *   a = softmax_j(logit) (a row with every pair masked is all zeros; PyTorch would give NaN)
 *   out = x + (sum_j a[h,i,j] v_j per head, concatenated) Wo^T
 * fp32, row-major: nodes/out [batch,n_nodes,dim], pair_feats [batch,n_nodes,n_nodes,pair_dim],
 * edge_mask [batch,n_nodes,n_nodes], gamma/beta [dim], wq/wk/wv/wo [dim,dim] ([out,in], as
 * nn.Linear stores them), w1 [pair_dim,pair_dim], b1 [pair_dim], w2 [heads,pair_dim], b2 [heads].
 * nodes, the four dim x dim weights and out must be 16-byte aligned; out may equal nodes.
 * Supported: dim <= 256 and a multiple of 4 and of heads, heads <= 16, pair_dim <= 64, and the
 * per-element working set (about 4*n_nodes*dim + (heads+1)*n_nodes^2 floats, the pair MLP's
 * weights and two 16-row blocks of a weight matrix) within the 160 KB of LDS of one workgroup
 * (gat_relation_block_lds_bytes returns 0 otherwise).  One workgroup per batch element.
 */
size_t gat_relation_block_lds_bytes(int n_nodes, int dim, int heads, int pair_dim);
gat_status gat_relation_block(const float* nodes, const float* pair_feats, const float* edge_mask,
                              const float* gamma, const float* beta, float eps, const float* wq,
                              const float* wk, const float* wv, const float* wo, const float* w1,
                              const float* b1, const float* w2, const float* b2, int64_t batch,
                              int n_nodes, int dim, int heads, int pair_dim, float* out, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Node projections: the nn.Linear steps of the l2_p4 page's reference model (its q/k/v
 * projections of the node rows and its output projection), which sit on either side of the
 * graph layer above.
 *   y[m, n] = bias[n] + sum_k x[m, k] * w[n, k]     for 0 <= m < n_rows, 0 <= n < n_cols
 *   x     [n_rows, in_dim] of x_dtype, row-major.  GAT_F32 values are rounded to bfloat16
 *         (nearest, ties to even) before they are multiplied; GAT_BF16 values are used as is.
 *   w     bfloat16 bits [n_cols, in_dim], row-major (nn.Linear's [out_features, in_features])
 *   bias  fp32 [n_cols], or NULL for none
 *   out   HOST array of n_out device pointers (1 <= n_out <= 3); out[s] is
 *         [n_rows, n_cols / n_out] of y_dtype, row-major, and receives y's columns
 *         [s * n_cols / n_out, (s + 1) * n_cols / n_out).  With w = [Wq; Wk; Wv] and n_out = 3,
 *         one call writes q, k and v in the [rows, heads, head_dim] layout the layer reads,
 *         reading x once.
 * Arithmetic: bf16 x bf16 products are exact in fp32; sums are fp32, in an order fixed by the
 * tiling (independent of the launch).  y is stored as fp32, or rounded to bf16 (nearest, ties
 * to even).  in_dim = 0 gives y = bias (or zeros).
 * Requirements: in_dim in [0, 65536] and a multiple of 8, n_cols in [1, 65536] and a multiple
 * of n_out (GAT_ERR_UNSUPPORTED otherwise); n_rows in [0, 2^31 - 1] with at most 2^24 tiles of
 * 128 x 128 (GAT_ERR_SIZE); x and w 16-byte aligned (GAT_ERR_ARGS).  The output arrays must
 * not overlap each other, x, w or bias.
 * ------------------------------------------------------------------------------------------ */
gat_status gat_linear(const void* x, gat_dtype x_dtype, const uint16_t* w, const float* bias, int64_t n_rows,
                      int in_dim, int n_cols, void* const* out, int n_out, gat_dtype y_dtype,
                      hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Backward.  No page writes the backward pass out; the l1_p10 page (edge-only SDDMM, the
 * passage on the backward pass) notes that gradients sum into the feature rows that edges read.
 * Each entry point below computes the derivative of a forward entry point above, given
 * grad_out = dL/d(forward output).  Gradients with respect to gathered tables (feat, k, v) are
 * aggregations over the transposed graph (a gat_csc), so every sum runs in a fixed order and no
 * atomic additions are used.
 * ------------------------------------------------------------------------------------------ */

/*
 * Transposed view of a CSR graph, built on the device by gat_csc_build and owned by the caller
 * (its arrays live in the caller's workspace `ws`; the struct only records offsets):
 *   col_ptr  int32 [n_src+1]    entries of source j are [col_ptr[j], col_ptr[j+1])
 *   row_idx  int32 [n_edges]    destination row of each entry
 *   perm     int32 [n_edges]    CSR edge id of each entry; entries of one source are in
 *                               increasing edge id (a stable sort of the edges by column)
 *   rows     int32 [n_edges]    destination row of each CSR edge (CSR order)
 *   stage    fp32  [n_edges*heads]  per-edge values moved into CSC order during a call
 *   plan     a degree-binning plan of the transposed graph (rows = sources)
 * Calls that use one gat_csc write its stage, so they must be ordered on one stream.
 */
typedef struct gat_csc {
    int64_t n_rows, n_src, n_edges;
    int32_t heads, head_dim;
    void* ws;
    size_t ws_bytes;
    size_t off_col_ptr, off_row_idx, off_perm, off_rows, off_stage;   /* byte offsets into ws */
    gat_plan plan;
    uint32_t magic;
} gat_csc;

/* Workspace bytes for gat_csc_build (0 if the sizes or shape are unsupported). */
size_t gat_csc_workspace_bytes(int64_t n_rows, int64_t n_src, int64_t n_edges, int heads, int head_dim);

/* Size of gat_csc as compiled into the library (for bindings that mirror the struct). */
size_t gat_csc_sizeof(void);

/*
 * Builds the transposed view of (row_ptr, col_idx) into ws (device memory of at least
 * gat_csc_workspace_bytes, 256-byte aligned) and fills *csc.  heads/head_dim size the stage
 * and the plan's partial states for the calls that will use it.  Enqueued on `stream`; no
 * synchronisation.  Requires 0 <= col_idx[e] < n_src (not checked on the device).
 */
gat_status gat_csc_build(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                         int64_t n_edges, int heads, int head_dim, void* ws, size_t ws_bytes,
                         gat_csc* csc, hipStream_t stream);

/*
 * Edge softmax backward (derivative of gat_edge_softmax): with alpha its output and grad =
 * dL/dalpha, both fp32 [n_edges,heads],
 *   out[e,h] = alpha[e,h] * (grad[e,h] - sum_{e' in row i} alpha[e',h] * grad[e',h])
 * out may equal grad (in place).  plan: NULL or a plan built for this row_ptr.
 */
gat_status gat_edge_softmax_backward(const int32_t* row_ptr, int64_t n_rows, int64_t n_edges, int heads,
                                     const float* alpha, const float* grad, float* out,
                                     const gat_plan* plan, hipStream_t stream);

/*
 * Aggregation backward (derivative of gat_aggregate), grad_out fp32 [n_rows,heads,head_dim]:
 *   dweights[e,h] = <grad_out[i,h,:], feat[col_idx[e],h,:]>                 (e in row i)
 *   dfeat[j,h,:]  = sum over the edges e with col_idx[e] = j of weights[e,h] * grad_out[i,h,:]
 * dweights fp32 [n_edges,heads] and dfeat fp32 [n_src,heads,head_dim] may each be NULL (not
 * computed); dfeat is +0.0 for sources no edge reads.  csc: built for this graph with the same
 * heads and head_dim (required: it supplies the row of each edge, and the transposed graph).
 */
gat_status gat_aggregate_backward(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows,
                                  int64_t n_src, int64_t n_edges, const float* weights, const void* feat,
                                  gat_dtype dtype, int heads, int head_dim, const float* grad_out,
                                  float* dweights, float* dfeat, const gat_csc* csc, hipStream_t stream);

/* Workspace bytes for gat_fused_layer_backward (0 if the sizes are unsupported). */
size_t gat_layer_backward_workspace_bytes(int64_t n_edges, int heads);

/*
 * Fused attention backward (derivative of gat_fused_layer), grad_out fp32
 * [n_rows,heads,head_dim].  With s the scores, alpha = edge_softmax(s) and
 * g[e,h] = <grad_out[i,h,:], v[col_idx[e],h,:]> (= dL/dalpha):
 *   g_s[e,h] = alpha[e,h] * (g[e,h] - sum_{e' in row i} alpha[e',h] * g[e',h])
 *   dv[j]    = sum over the edges e with col_idx[e] = j of alpha[e] * grad_out[i]
 * Modes as in the forward (exactly one of scores or (q, k) when n_edges > 0):
 *  - scores given: dscores = g_s (fp32 [n_edges,heads]); dq, dk unused (may be NULL).
 *  - q, k given (s = scale * <q_i, k_j>, recomputed here): dq[i] = scale * sum_{e in row i}
 *    g_s[e] * k[col_idx[e]], dk[j] = scale * sum over the edges e with col_idx[e] = j of
 *    g_s[e] * q[i] (fp32 [n_rows|n_src,heads,head_dim]); dscores unused (may be NULL).
 * dv is always computed; dv, dk are +0.0 for sources no edge reads, dq for rows without edges.
 * plan: built for this row_ptr (required); csc: built for this graph with the same heads and
 * head_dim (required).  ws: device workspace of at least gat_layer_backward_workspace_bytes
 * (scores, alpha, g), 256-byte aligned.  Calls sharing ws, plan or csc must be ordered.
 */
gat_status gat_fused_layer_backward(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows,
                                    int64_t n_src, int64_t n_edges, int heads, int head_dim, gat_dtype dtype,
                                    const float* scores, const void* q, const void* k, float scale,
                                    const void* v, const float* grad_out,
                                    float* dscores, float* dq, float* dk, float* dv,
                                    const gat_plan* plan, const gat_csc* csc, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* Workspace bytes for gat_sddmm_backward (0 if the sizes or shape are unsupported). */
size_t gat_sddmm_backward_workspace_bytes(int64_t n_edges, int64_t n_src, int64_t n_dst, int heads,
                                          int head_dim);

/*
 * SDDMM backward (derivative of gat_sddmm, the edge-only SDDMM of [l1_p10]; its backward-pass
 * passage: each edge's gradient flows into the two feature rows it read).  With grad_out =
 * dL/dout fp32 [n_edges,heads]:
 *   d_src[i,h,:] = scale * sum over the edges e with src_idx[e] = i of grad_out[e,h] * dst_feat[dst_idx[e],h,:]
 *   d_dst[j,h,:] = scale * sum over the edges e with dst_idx[e] = j of grad_out[e,h] * src_feat[src_idx[e],h,:]
 * d_src fp32 [n_src,heads,head_dim] and d_dst fp32 [n_dst,heads,head_dim] may each be NULL (not
 * computed); rows that no edge reads get +0.0.  Repeated (src, dst) pairs are separate terms.
 * Each gradient is an aggregation over the edges grouped by one endpoint: the call sorts the
 * edge ids by that endpoint (stable radix passes on the device), builds the grouping's row
 * offsets and plan in `ws`, and sums each row in registers, so no atomic addition is used and
 * the result does not depend on the launch.  scale * grad_out is rounded to fp32 before it is
 * multiplied; sums are fp32.
 * ws: device workspace of at least gat_sddmm_backward_workspace_bytes(...) bytes, 256-byte
 * aligned (GAT_ERR_ARGS otherwise), owned by the caller; its contents need no clearing and are
 * scratch after the call.  Calls sharing ws must be ordered on one stream.  n_src or n_dst = 0
 * with n_edges > 0 is GAT_ERR_ARGS; src_feat must be given when d_dst is asked for and dst_feat
 * when d_src is (GAT_ERR_NULL).  Requires 0 <= src_idx[e] < n_src and 0 <= dst_idx[e] < n_dst
 * (not checked on the device).
 */
gat_status gat_sddmm_backward(const int32_t* src_idx, const int32_t* dst_idx, int64_t n_edges,
                              const void* src_feat, int64_t n_src, const void* dst_feat, int64_t n_dst,
                              gat_dtype dtype, int heads, int head_dim, float scale,
                              const float* grad_out, float* d_src, float* d_dst,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Testing hook.  The edge-parallel kernels (gat_sddmm and the edge dot products of the backward)
 * launch one wave per step of edges, up to 2^23 workgroups, and loop over the edges with a
 * grid stride past that (2^29 edges and up).  This caps their workgroups at `cap` so that the
 * loop runs at sizes a test can check; cap <= 0 or above 2^23 restores the default.  Returns the
 * previous cap.  Process-wide, host only; launches already enqueued keep their grid.  Every
 * edge's result is bitwise the same at any cap.
 * ------------------------------------------------------------------------------------------ */
int64_t gat_testing_edge_grid_cap(int64_t cap);

#ifdef __cplusplus
}
#endif

#endif /* GAT_H */
