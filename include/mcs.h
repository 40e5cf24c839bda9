/*
 * mcs.h -- C ABI of libmcs, MI355X (gfx950) token-sparse attention.
 *
 * The library implements the hot path of MC-Sparse ("MC-Sparse: Deconstructing
 * and Closing the Dense-Sparse Attention Gap in Diffusion Transformers",
 * arXiv 2610.06801), as the method is described on the ai.info summary page
 * ("Key Contributions", "Methodology in Plain English"), the wispaper.ai
 * explainer ("Token-level selection needs tile-aligned query groups",
 * "Reused exact selection beats recomputed mean pooling", "Residual
 * correction recovers the discarded tail") and the agihunt.info summary
 * (method paragraphs).
 *
 * Per layer and denoising step a caller makes these calls:
 *   anchor step:  mcs_group -> mcs_dense_attn (with lse) -> mcs_select
 *                 -> mcs_sparse_attn (no residual) -> mcs_residual_update;
 *                 the step's output is the dense output.
 *   reuse step:   mcs_sparse_attn with the cached perm, kv_idx and residual.
 *
 * Conventions shared by every call
 *   - Tensors are device pointers to contiguous row-major arrays.  bf16 values
 *     are passed as their uint16_t bit patterns.  Q, K, V, O and the residual
 *     are [B, H, N, D] (head-major, so one head's K/V is one contiguous slab).
 *   - d.B, d.H, d.N >= 1; d.D is 64 or 128; the group size C is 64 or 128.
 *   - G = ceil(N / C) query groups per head.  perm is int32 [B, H, N], a
 *     permutation of 0..N-1 per head; group g of a head is
 *     perm[g*C .. min((g+1)*C, N) - 1] (the last group may be short).
 *   - kv_idx is int32 [B, H, G, K]: the K KV token ids of each group.
 *   - lse is float32 [B, H, N], natural log.
 *   - Every pointer argument that is not documented as nullable must be
 *     non-NULL and 16-byte aligned.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it; the library never synchronises, never
 *     creates streams and never allocates or frees device memory.  Scratch
 *     memory is a caller-owned device workspace sized by the *_workspace
 *     queries.  Calls are re-entrant; concurrent calls on different streams
 *     must not share a workspace.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed check returns a non-zero status, enqueues nothing, and
 *     mcs_last_error() describes it.  A failed kernel launch returns
 *     MCS_E_HIP.  Device faults surface at the caller's next synchronisation.
 *   - Out-of-range ids cannot cause out-of-bounds accesses: perm entries are
 *     clamped into [0, N), and a kv_idx entry outside [0, N) reads as a zero
 *     key and value row; the result for such input is unspecified.  NaN/Inf
 *     inputs propagate and are not checked.
 *   - One head's K (N * D * 2 bytes) must stay below 2^31 bytes.
 */
#ifndef MCS_H
#define MCS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MCS_VERSION 200

#if defined(__GNUC__)
#define MCS_API __attribute__((visibility("default")))
#else
#define MCS_API
#endif

typedef enum {
    MCS_OK = 0,
    MCS_E_NULL = 1,        /* a required pointer is NULL                      */
    MCS_E_SHAPE = 2,       /* B, H or N < 1, or sizes overflow 32-bit indexing */
    MCS_E_HEAD_DIM = 3,    /* D is not 64 or 128                               */
    MCS_E_GROUP_SIZE = 4,  /* C is not 64 or 128                               */
    MCS_E_BUDGET = 5,      /* K is not in [1, N]                               */
    MCS_E_SCALE = 6,       /* scale is not finite and > 0                      */
    MCS_E_ALIGN = 7,       /* a pointer is not 16-byte aligned                 */
    MCS_E_WORKSPACE = 8,   /* workspace NULL or smaller than required          */
    MCS_E_HIP = 9,         /* a HIP launch failed                              */
    MCS_E_ARG = 10         /* another argument is out of range                 */
} mcs_status;

typedef struct {
    int32_t B; /* batch                      */
    int32_t H; /* heads                      */
    int32_t N; /* tokens per head            */
    int32_t D; /* head dimension (64 or 128) */
} mcs_dims;

/*
 * Dense attention with row log-sum-exp: the first pass of the two-pass exact
 * selector and the anchor step's output (ai.info, "Methodology in Plain
 * English": pass one of the selector yields the attention output together
 * with one log-sum-exp per query row).  Also the library's own dense
 * baseline.
 *   o[b,h,i,:] = sum_j softmax_j(scale * q_i.k_j) v_j   (no mask)
 *   lse[b,h,i] = ln sum_j exp(scale * q_i.k_j)          (if lse != NULL)
 * In: q, k, v bf16 [B,H,N,D].  Out: o bf16 [B,H,N,D]; lse float32 [B,H,N] or
 * NULL.  fp32 accumulation and softmax.  o must not alias q, k or v.
 */
MCS_API mcs_status mcs_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          uint16_t* o, float* lse, mcs_dims d, float scale, void* stream);

/*
 * Token-sparse attention over gathered KV ids, with the optional cached
 * residual added in the epilogue (wispaper.ai, "Token-level selection needs
 * tile-aligned query groups": each group of C similar queries shares one
 * selection of individually gathered KV tokens; "Residual correction
 * recovers the discarded tail": reuse steps add the cached dense-minus-sparse
 * residual).  For every query i of group g of head (b,h):
 *   o[b,h,i,:] = sum_{j in kv_idx[b,h,g,:]} softmax_j(scale * q_i.k_j) v_j
 *                (+ residual[b,h,i,:] when residual != NULL)
 * The softmax is renormalised over the K selected keys.  The order of the
 * ids within a group does not matter; ids should be distinct.
 * In: q, k, v bf16 [B,H,N,D]; perm int32 [B,H,N]; kv_idx int32 [B,H,G,K];
 * residual bf16 [B,H,N,D] or NULL.  Out: o bf16 [B,H,N,D] (every row written,
 * since perm is a permutation).  1 <= K <= N.  o must not alias the inputs.
 */
MCS_API mcs_status mcs_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* perm, const int32_t* kv_idx,
                           const uint16_t* residual, uint16_t* o, mcs_dims d,
                           int32_t C, int32_t K, float scale, void* stream);

/*
 * The two attention calls above with a float32 output o [B,H,N,D] instead of
 * bf16: the same kernels and arithmetic, only the final store differs (the
 * bf16 calls store the round-to-nearest-even of exactly these values).  For
 * callers that keep activations in fp32, and for verification.
 */
MCS_API mcs_status mcs_dense_attn_f32out(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 float* o, float* lse, mcs_dims d, float scale, void* stream);
MCS_API mcs_status mcs_sparse_attn_f32out(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const int32_t* perm, const int32_t* kv_idx,
                                  const uint16_t* residual, float* o, mcs_dims d, int32_t C,
                                  int32_t K, float scale, void* stream);

/*
 * mcs_sparse_attn with two extensions, for the selection diagnostics and the
 * block-sparse comparison below:
 *   kv_count: int32 [B,H,G] or NULL.  Group g attends to its first
 *             kv_count[b,h,g] ids only (a value outside [1, K] is clamped
 *             into it); the id lists stay K apart in kv_idx.  NULL: K each.
 *   lse:      float32 [B,H,N] or NULL: ln sum_{j selected} exp(scale q_i.k_j),
 *             the log-sum-exp over each query's selected keys (with the dense
 *             LSE of mcs_dense_attn, exp(lse - lse_dense) is the dense
 *             attention mass the selection keeps).  lse and residual cannot
 *             both be given.
 *   o:        float32 when o_f32 != 0, else bf16 [B,H,N,D].
 * Other arguments, layouts and checks as mcs_sparse_attn.
 */
MCS_API mcs_status mcs_sparse_attn_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* perm, const int32_t* kv_idx, const int32_t* kv_count,
                              const uint16_t* residual, void* o, int32_t o_f32, float* lse,
                              mcs_dims d, int32_t C, int32_t K, float scale, void* stream);

/*
 * Anchor-step residual (wispaper.ai, "Residual correction recovers the
 * discarded tail": at an anchor the method records dense minus sparse output).
 *   residual[e] = bf16(float(o_dense[e]) - float(o_sparse[e])),  e < n_elems
 * In: o_dense, o_sparse bf16.  Out: residual bf16 (may alias either input).
 * n_elems >= 1.
 */
MCS_API mcs_status mcs_residual_update(const uint16_t* o_dense, const uint16_t* o_sparse,
                               uint16_t* residual, int64_t n_elems, void* stream);

/*
 * Exact KV selection, the second pass of the two-pass selector (ai.info,
 * "Methodology in Plain English": recompute the QK scores, recover the
 * probabilities from the first pass's LSE, aggregate them per query group and
 * keep the top K; agihunt.info method paragraphs: the objective is the
 * largest summed attention weight of the group within a budget of K tokens).
 *   M[g, j] = sum_{i in group g} exp(scale * q_i.k_j - lse_i)   (fp32)
 *   kv_idx[b,h,g,:] = the K ids j of largest M[g, j]; equal masses go to the
 *                     smaller id; ids written in ascending order.
 * In: q, k bf16 [B,H,N,D]; lse float32 [B,H,N] (from mcs_dense_attn); perm
 * int32 [B,H,N].  Out: kv_idx int32 [B,H,G,K].  ws: device workspace of at
 * least mcs_select_workspace(d, C, K) bytes (the per-group mass rows of a
 * chunk of heads; a larger workspace processes more heads per launch).
 * Aggregation and top-K run in one kernel, as on the ai.info page: each
 * workgroup writes its group's mass row and selects from it before it ends.
 * Where that kernel's compaction counts do not fit in LDS (N > 262144 for
 * D = 128, N > 131072 for D = 64) a separate top-K kernel follows instead;
 * the ids are the same either way.
 */
MCS_API mcs_status mcs_select(const uint16_t* q, const uint16_t* k, const float* lse,
                      const int32_t* perm, int32_t* kv_idx, mcs_dims d, int32_t C,
                      int32_t K, float scale, void* ws, size_t ws_bytes, void* stream);

/*
 * mcs_select always as two kernels: the mass rows of a chunk of heads, then
 * the top-K of every row.  Same arguments, workspace, checks and results.
 */
MCS_API mcs_status mcs_select_two_pass(const uint16_t* q, const uint16_t* k, const float* lse,
                               const int32_t* perm, int32_t* kv_idx, mcs_dims d, int32_t C,
                               int32_t K, float scale, void* ws, size_t ws_bytes,
                               void* stream);

/* Minimum workspace of mcs_select (one head's mass rows: G * N * 4 bytes). */
MCS_API size_t mcs_select_workspace(mcs_dims d, int32_t C, int32_t K);

/* Workspace that lets mcs_select process every head in one launch. */
MCS_API size_t mcs_select_workspace_all_heads(mcs_dims d, int32_t C, int32_t K);

/*
 * Top-K of given non-negative float32 score rows, the selection step of
 * mcs_select on its own (same rule: larger score first, equal scores to the
 * smaller id, ids written ascending).  Scores must be >= 0 (or +0/-0).
 * In: scores float32 [rows, n].  Out: idx int32 [rows, K].  1 <= K <= n.
 */
MCS_API mcs_status mcs_topk(const float* scores, int32_t* idx, int64_t rows, int32_t n,
                    int32_t K, void* stream);

/*
 * Median-split PDDP grouping (ai.info, "Key Contributions" and "Methodology in
 * Plain English"; wispaper.ai, "Token-level selection needs tile-aligned query
 * groups": each node's queries are projected on the node's principal
 * direction and cut at the median, recursively, until every group holds
 * exactly C queries; the directions of all nodes of a tree depth are found
 * together, by batched power iteration on the pages).
 * Per head, a node of n queries forms g = ceil(n/C) groups; if g > 1 its
 * queries are ordered by (projection on the node's principal direction, query
 * id) and the first C*floor(g/2) form the left child, the rest the right
 * child.  Leaves are written left-first, so group g is perm[g*C ..].  The
 * principal direction is the top eigenvector of the node's covariance, sign
 * fixed so that its largest-magnitude component is positive.  It is computed
 * by Lanczos with full reorthogonalisation (the Krylov form of power
 * iteration: the same matrix-vector products, but it converges where power
 * steps stall on nearly equal leading eigenvalues), started from the
 * covariance column of largest diagonal, for at most lanczos_steps steps
 * (<= 0 selects the default, 32; at most 64); when that is more than 16, the
 * iteration ends after 16 steps if the top Ritz pair's residual is below
 * 1e-6 of its Ritz value.  Covariance, Lanczos and projections are fp32; the
 * small tridiagonal eigenproblem is fp64.
 * In: q bf16 [B,H,N,D].  Out: perm int32 [B,H,N].  ws: device workspace of at
 * least mcs_group_workspace(d, C) bytes.
 */
MCS_API mcs_status mcs_group(const uint16_t* q, int32_t* perm, mcs_dims d, int32_t C,
                     int32_t lanczos_steps, void* ws, size_t ws_bytes, void* stream);

/* Workspace of mcs_group in bytes (per-query projections and ids, per-node
 * directions, and partial moments of the large nodes near the root). */
MCS_API size_t mcs_group_workspace(mcs_dims d, int32_t C);

/*
 * mcs_group for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * grouping and results as mcs_group, with no workspace argument: the scratch
 * is a static device array of 64 MiB that the library holds on every device
 * its code is loaded on, until the process ends.  Heads are processed in
 * chunks whose workspace fits it (4.7 MiB per head at N = 75600, D = 128,
 * C = 128); a call whose single head needs more than 64 MiB of workspace
 * (mcs_group_workspace with B = H = 1) returns MCS_E_WORKSPACE and enqueues
 * nothing.  Runs on the calling thread's current device, whose stream must be
 * passed.  Every call on a device shares that device's scratch, which keeps
 * the last call's contents: calls on one stream are ordered and safe, but
 * calls that overlap in time on one device (other streams, other threads)
 * race and give wrong results.  The first call on a device looks up the
 * scratch's address (hipGetSymbolAddress); no call allocates or frees.
 */
MCS_API mcs_status mcs_group_noalloc(const uint16_t* q, int32_t* perm, mcs_dims d, int32_t C,
                             int32_t lanczos_steps, void* stream);

/*
 * Mean-pooled block selection, the selector of standard block-sparse
 * attention that the pages compare against (wispaper.ai, "Mean-pooled block
 * scoring misses high-mass tokens"; agihunt.info, the kernel comparison).
 * Keys form blocks of 64 consecutive tokens (the last one may be short).  For
 * each query group g (perm[g*C ..], as in mcs_select) the score of key block
 * b is scale * mean_{i in g}(q_i) . mean_{j in b}(k_j) (fp32); the K/64
 * blocks of largest score are kept, equal scores going to the smaller block
 * id.  Out: kv_idx int32 [B,H,G,K], the token ids of the kept blocks in
 * ascending order, and kv_count int32 [B,H,G], the number of real token ids
 * (K, less the missing tail when the short last block is kept; the slots past
 * it repeat id N-1).  The pair feeds mcs_sparse_attn_ex.
 * K: a multiple of 64 with 64 <= K <= 64 * ceil(N/64); ceil(N/64) <= 4096.
 * ws: device workspace of mcs_select_blocks_workspace(d) bytes (block means).
 */
MCS_API mcs_status mcs_select_blocks(const uint16_t* q, const uint16_t* k, const int32_t* perm,
                             int32_t* kv_idx, int32_t* kv_count, mcs_dims d, int32_t C,
                             int32_t K, float scale, void* ws, size_t ws_bytes, void* stream);
MCS_API size_t mcs_select_blocks_workspace(mcs_dims d);

/*
 * Per-query quality of a selection (ai.info, "Main Findings" and
 * "Methodology in Plain English": attention recall and the relative L1
 * error of the renormalised sparse output).  For every query row r of
 * [B,H,N]:
 *   recall[r] = exp(lse_sparse[r] - lse_dense[r])      (kept dense mass)
 *   l1[r]     = sum_c |o_sparse[r,c] - o_dense[r,c]|
 *   l1_ref[r] = sum_c |o_dense[r,c]|
 * In: lse_dense (mcs_dense_attn), lse_sparse (mcs_sparse_attn_ex, no
 * residual) float32 [B,H,N]; o_dense, o_sparse float32 [B,H,N,D].  Out:
 * recall, l1, l1_ref float32 [B,H,N].  The relative L1 error is
 * sum(l1) / sum(l1_ref) (mcs_row_sums).
 */
MCS_API mcs_status mcs_query_quality(const float* lse_dense, const float* lse_sparse,
                             const float* o_dense, const float* o_sparse, float* recall,
                             float* l1, float* l1_ref, mcs_dims d, void* stream);

/* out[r] = sum_i x[r*n + i] in fp64, summed in a fixed order (deterministic).
 * In: x float32 [rows, n].  Out: out float64 [rows].  1 <= rows < 2^31. */
MCS_API mcs_status mcs_row_sums(const float* x, double* out, int64_t rows, int64_t n,
                        void* stream);

/*
 * Lloyd's k-means of one head's query or key rows, the grouping the pages set
 * against exactly-C PDDP groups (ai.info, "Main Findings": k-means clusters of
 * unequal size inflate the computed interactions once padded to whole tiles;
 * wispaper.ai, "Token-level selection needs tile-aligned query groups").
 * Each of `rounds` rounds: every row goes to the nearest centre (squared
 * Euclidean distance in fp32, equal distances to the smaller centre id),
 * inertia[r] = sum of the squared distances to those centres (fp64, fixed
 * order), then every centre becomes the mean of its rows; a centre without
 * rows keeps its place.
 * In: x bf16 [n, D] (D = 64 or 128), init float32 [k, D] (initial centres;
 * 1 <= k <= n).  Out: labels int32 [n] (the last round's assignment),
 * centers float32 [k, D] (after the last update), inertia float64 [rounds],
 * sizes int32 [k] (rows per centre in the last round).  The alignment
 * inflation of tile T is sum_c ceil(sizes[c]/T)*T / n.
 * ws: device workspace of mcs_kmeans_workspace(n, k) bytes.
 */
MCS_API mcs_status mcs_kmeans(const uint16_t* x, const float* init, int32_t n, int32_t D, int32_t k,
                      int32_t rounds, int32_t* labels, float* centers, double* inertia,
                      int32_t* sizes, void* ws, size_t ws_bytes, void* stream);
MCS_API size_t mcs_kmeans_workspace(int32_t n, int32_t k);

/* Static description of a status code. */
MCS_API const char* mcs_status_string(mcs_status s);

/* Detail of the last failed call on the calling thread ("" if none). */
MCS_API const char* mcs_last_error(void);

/* MCS_VERSION of the built library. */
MCS_API int32_t mcs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MCS_H */
