/*
 * sparsepr.h -- C ABI of libsparsepr, a gfx950 (MI355X) implementation of one
 * SparsePR attention call: Response-Coupled Partitioning, block-sparse
 * attention over the group-permuted layout, and Probe-Fitted Residual
 * Reconstruction.
 *
 * Sources (page title, section):
 *   [TS] "Resumen Técnico: SparsePR – Atención Dispersa Libre de Entrenamiento
 *        para Generación de Vídeo y Modelos de Mundo" (gist.science), 2.A-2.C.
 *   [NE] news explainer reposted from 科技行者 (huashangw.com), sections
 *        "SparsePR：先把误差聚拢，再用少量“抽查”去纠正" (NE/method) and
 *        "稀疏执行怎么落地，误差怎么算才公平" (NE/exec).
 *   [DG] "Partition the Support, Reconstruct the Residual: 无训练稀疏注意力用于
 *        视频生成与世界模型" (ai-feeds.com digest), 方法 and 行业影响 sections.
 *
 * Problem statement ([DG] 方法/输入-输出): given Q, K, V of one attention call,
 * a target executed-pair density and a probe budget, return the corrected
 * attention output.  It replaces scaled-dot-product attention without state
 * kept between calls ([DG] 行业影响/与现有工作流的接口).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or keeps device memory between calls;
 *     scratch lives in a caller-provided workspace sized by
 *     sparsepr_workspace_size().
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *     is the legacy default stream).  SPARSEPR_OK means "enqueued".  Argument
 *     errors are detected on the host before anything is enqueued.  A failed
 *     kernel launch returns SPARSEPR_ERR_HIP and sparsepr_last_hip_error()
 *     holds the hipError_t (per thread).  The library never synchronises.
 *   - Tensors are [B, H, N, d] with element strides given per tensor; the
 *     d-stride must be 1 and rows must be 16-byte aligned.  Q, K, V and O
 *     must not alias each other or the workspace.
 *   - Supported: dtype bf16 or fp32, d in {64, 128}, 2 <= N <= 2^20, B*H >= 1,
 *     1 <= G_K, G_Q <= 1024 with G_Q*G_K <= 2^20 and G <= N, probe rows
 *     0..min(256, N), residual rank 0..64, T >= 1 k-means steps.
 *   - Calls on different streams with different workspaces may run
 *     concurrently; calls that share a workspace must be ordered.
 */
#ifndef SPARSEPR_H
#define SPARSEPR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARSEPR_OK = 0,
  SPARSEPR_ERR_INVALID_ARG = -1,
  SPARSEPR_ERR_UNSUPPORTED = -2,
  SPARSEPR_ERR_WORKSPACE = -3,
  SPARSEPR_ERR_HIP = -4,
  SPARSEPR_ERR_INTERNAL = -5
} sparsepr_status;

typedef enum { SPARSEPR_BF16 = 0, SPARSEPR_FP32 = 1 } sparsepr_dtype;

typedef enum {
  /* keys clustered on key-response coordinates, queries on their logits against
     the K/V-group centres ([TS] 2.A) */
  SPARSEPR_PART_RESPONSE_COUPLED = 0,
  /* comparison partition: Q and K clustered separately on raw activations
     ([NE] NE/method contrasts it with the response-coupled one) */
  SPARSEPR_PART_INDEPENDENT = 1
} sparsepr_partition_mode;

typedef enum {
  /* lambda is a fraction of the mean eigenvalue of the weighted centred Gram
     Xc^T D Xc of the probes' sparse outputs (scale free) */
  SPARSEPR_RIDGE_RELATIVE = 0,
  /* lambda is used as given */
  SPARSEPR_RIDGE_ABSOLUTE = 1
} sparsepr_ridge_mode;

typedef enum {
  /* cells by estimated per-key probability under the pair budget of
     `density` ([NE] NE/exec: the budget counts true pairs) */
  SPARSEPR_ROUTER_BUDGET = 0,
  /* per query group, its best cell and then key groups by estimated mass
     until `alpha` of the group's mass is retained ([NE] NE/method, Figure 2:
     key groups covered jointly for a target retained mass); no budget */
  SPARSEPR_ROUTER_ALPHA = 1
} sparsepr_router;

/* Method settings.  Every field is a value the pages leave open unless noted;
   sparsepr_config_default() fills the documented defaults. */
typedef struct {
  float density;          /* target executed-pair density rho in (0, 1]; probe
                             rows count toward it ([TS] 2.C).  >= 1 grants every cell */
  int probe_rows;         /* M exact rows per (b,h), 64 by default ([NE] NE/method); 0 = no fit */
  int n_kv_groups;        /* G_K paired K/V groups */
  int n_q_groups;         /* G_Q query groups */
  int residual_rank;      /* r: leading residual singular directions kept ([NE] keeps 16) */
  float ridge_lambda;     /* ridge lambda of the affine fit ([TS] 2.B); see ridge_mode */
  int kmeans_iters;       /* T Lloyd steps, no early stop */
  int n_sample_q;         /* M_s upper bound of sampled queries (min with N) */
  int key_coord_rank;     /* r_K upper bound of kept eigenvectors of M_K (min with d, M_s) */
  float scale;            /* softmax scale; 0 => 1/sqrt(d) rounded to float */
  float rank_cut;         /* relative singular-value cut of the residual subspace */
  int partition_mode;     /* sparsepr_partition_mode */
  int ridge_mode;         /* sparsepr_ridge_mode */
  unsigned long long seed;/* seed of the query sample (splitmix64) */
  int router;             /* sparsepr_router */
  float alpha;            /* target retained mass in (0, 1] of SPARSEPR_ROUTER_ALPHA */
  /* Fit and coordinate variants ([TS] 2.B "Restricción de Subespacio" and
     "Calibración Afín"; [DG] 方法/关键模块: the weighted affine fit; [TS] 2.A:
     query coordinates are pre-softmax logits): */
  float rank_cap;         /* residual rank at most floor(rank_cap * M), in (0, 1]; 1 = at most M */
  int svd_weighted;       /* 1: residual subspace from the SVD of D^(1/2) R (probe weights on the
                             rows); 0: from the SVD of R */
  int centred_query_coords; /* 1: query coordinates minus each query's mean logit over the
                               non-empty key groups; 0: raw logits */
} sparsepr_config;

/* Input/output description.  Strides are in elements, order [b, h, n, d]. */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  long long q_strides[4];
  long long k_strides[4];
  long long v_strides[4];
  long long o_strides[4];
  int B, H, N, d;
  int dtype;              /* sparsepr_dtype; q, k, v and o share it */
} sparsepr_tensors;

/* Per-(b,h) statistics written by the device when a stats pointer is given
   (device memory, B*H entries, row-major over (b,h)). */
typedef struct {
  long long routed_pairs;     /* sum over granted cells of |Q_g| * |K_h| */
  long long budget_pairs;     /* floor(rho N^2) - M N (N^2 under the alpha router: no budget) */
  long long mandatory_pairs;  /* cost of the best cell of every query group */
  long long probe_pairs;      /* M N */
  int granted_cells;
  int nonempty_q_groups;
  int nonempty_kv_groups;
  int probe_rows;
  int residual_rank;          /* r' actually used by the fit */
  int over_budget;            /* 1 when the mandatory cells alone exceed the budget */
  int q_tiles;                /* query tiles run by the sparse kernel */
  int kmeans_redecided;       /* k-means assignments re-decided in fp64 (both sides, all Lloyd
                                 steps; 0 when the partition was given) */
  int fit_fallback;           /* 1 when the ridge system of the fit was not numerically positive
                                 definite and the correction was dropped (residual_rank 0) */
  int reserved;               /* 0 (keeps the structure free of padding) */
  double rho_route;           /* routed_pairs / N^2 */
  double rho_exec;            /* (routed_pairs + probe_pairs) / N^2 */
  double sigma[4];            /* leading singular values of the probe residuals */
} sparsepr_head_stats;

/* Fill `out` with the defaults for a call of N tokens and head dim d:
   density 0.25, 64 probe rows, G_K = G_Q = clamp(N/128, 1, 256), r = 32,
   relative ridge lambda 1.0, T = 10, M_s = 256, r_K = 32, scale 0,
   rank_cut 1e-6, response-coupled partition, seed 0, budget router
   (alpha 0.9 for the alpha router), rank_cap 1, unweighted residual
   subspace, raw (uncentred) query coordinates. */
sparsepr_status sparsepr_config_default(int N, int d, sparsepr_config* out);

/* Check a config against a shape (no device work). */
sparsepr_status sparsepr_validate(const sparsepr_config* cfg, int B, int H, int N, int d, int dtype);

/* Bytes of workspace every entry point below needs for this shape (256-byte
   aligned base required). */
sparsepr_status sparsepr_workspace_size(const sparsepr_config* cfg, int B, int H, int N, int d,
                                        int dtype, size_t* bytes);

/* The full call ([NE] NE/exec latency chain: partition construction, routing,
   tensor reorder, sparse attention, exact probe rows, residual fit,
   correction, output restoration).  Writes o in the original token order.
   `stats` (device pointer, nullable) receives B*H sparsepr_head_stats.
   Every kernel of the call is enqueued on `stream`, in order, so work
   enqueued on `stream` after the call sees the whole output, and HIP graph
   capture of `stream` records the call like any other work.
   State: none.  Every intermediate lives in `workspace`, as the pages'
   per-call calibration with no persistent state requires ([DG] "Partition
   the Support, Reconstruct the Residual" digest, 行业影响/与现有工作流的接口);
   calls that share a workspace must be ordered by the caller. */
sparsepr_status sparsepr_attention(const sparsepr_config* cfg, const sparsepr_tensors* io,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   sparsepr_head_stats* stats);

/* The full call for callers that cannot allocate (code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc): the same
   computation and result as sparsepr_attention, run entirely on `stream`,
   with the intermediates in a fixed
   scratch array of sparsepr_noalloc_scratch_bytes() bytes (128 MiB) that the
   library holds on each GPU it runs on until the process ends.  No memory
   is allocated or freed by the call.  A call whose workspace would exceed
   the scratch (sparsepr_workspace_size) returns SPARSEPR_ERR_WORKSPACE
   before any device work; `stream` must belong to the current device
   (SPARSEPR_ERR_INVALID_ARG otherwise).  Every call on a GPU shares that
   GPU's scratch and it keeps the last call's contents (the call clears what
   it needs itself): calls that overlap in time on one GPU race and must be
   ordered by the caller.  `stats` as for sparsepr_attention. */
sparsepr_status sparsepr_attention_noalloc(const sparsepr_config* cfg, const sparsepr_tensors* io, void* stream,
                                           sparsepr_head_stats* stats);
size_t sparsepr_noalloc_scratch_bytes(void);

/* Stages timed by sparsepr_attention_profile(). */
enum {
  SPARSEPR_STAGE_SAMPLE_METRIC = 0,   /* a1 query sample and M_K */
  SPARSEPR_STAGE_KEY_EIGEN = 1,       /* a2 eigenvectors of M_K */
  SPARSEPR_STAGE_KEY_COORDS = 2,      /* a3 key-response coordinates */
  SPARSEPR_STAGE_KEY_KMEANS = 3,      /* a4-a5 key k-means and K/V grouping */
  SPARSEPR_STAGE_KEY_CENTRES = 4,     /* a6 K/V-group centres and the query metric */
  SPARSEPR_STAGE_QUERY_KMEANS = 5,    /* a7-a8 query k-means and grouping */
  SPARSEPR_STAGE_QUERY_CENTRES = 6,   /* query-group centres */
  SPARSEPR_STAGE_ROUTE = 7,           /* a10 router */
  SPARSEPR_STAGE_GATHER = 8,          /* a9 permuted Q, K, V */
  SPARSEPR_STAGE_PROBES = 9,          /* a11, a13 probe selection and exact probe rows */
  SPARSEPR_STAGE_FIT = 10,            /* a14 residual fit */
  SPARSEPR_STAGE_SPARSE_ATTENTION = 11, /* a12 + a15 sparse attention with fused correction */
  SPARSEPR_STAGE_RESTORE = 12,        /* probe rows written back */
  SPARSEPR_N_STAGES = 13
};

/* Measurement entry point: the same work as sparsepr_attention, with a HIP
   event recorded between stages on `stream`; it then waits for the stream
   and writes each stage's elapsed milliseconds to the HOST array stage_ms
   [SPARSEPR_N_STAGES] (stages that did not run read 0). */
sparsepr_status sparsepr_attention_profile(const sparsepr_config* cfg, const sparsepr_tensors* io,
                                           void* workspace, size_t workspace_bytes, void* stream,
                                           sparsepr_head_stats* stats, float* stage_ms);

/* The full call with the partition given instead of computed: q_labels and
   kv_labels are device int32 arrays [B*H, N] with values in [0, G_Q) and
   [0, G_K).  Used to check the stages after partitioning in isolation. */
sparsepr_status sparsepr_attention_with_partition(const sparsepr_config* cfg,
                                                  const sparsepr_tensors* io,
                                                  const int* q_labels, const int* kv_labels,
                                                  void* workspace, size_t workspace_bytes,
                                                  void* stream, sparsepr_head_stats* stats);

/* Stages a1-a2 ([TS] 2.A): the sampled query rows (device int32 [B*H, M_s],
   ascending), M_K = Q_s^T Q_s / M_s (device double [B*H, d, d]), the
   eigenvalues of M_K in descending order (device double [B*H, d]) and the key
   coordinate map (device double [B*H, d, r_K], row-major: column r is
   s sqrt(lambda_r) u_r for the r-th largest eigenpair, r_K =
   min(key_coord_rank, d, M_s); the sign of each column is unspecified).  All
   three are computed in fp64.  Any output pointer may be NULL. */
sparsepr_status sparsepr_key_metric(const sparsepr_config* cfg, const sparsepr_tensors* io,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    int* sample_idx, double* m_k, double* eigvals, double* key_map);

/* Stages a1-a8: response-coupled (or independent) partition ([TS] 2.A:
   sampled queries define the key metric, keys are grouped by k-means in its
   leading eigenvectors, queries by k-means on their logits against the key
   groups' centres, in one asymmetric pass; [NE] NE/method, which also sets
   the independent comparison partition against it).  Writes the labels of the last
   Lloyd step (device int32 [B*H, N] each): the assignment of an fp64 Lloyd
   iteration (near ties re-decided in fp64).  Errors as sparsepr_attention. */
sparsepr_status sparsepr_partition(const sparsepr_config* cfg, const sparsepr_tensors* io,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   int* q_labels, int* kv_labels);

/* Stages a5, a9-a10 from given labels ([TS] 2.C, [NE] NE/exec): stable group
   permutations perm_q/perm_k (position -> token, int32 [B*H, N]), group
   offsets off_q [B*H, G_Q+1] and off_k [B*H, G_K+1], and the granted cells as
   CSR per query group: csr_rowptr [B*H, G_Q+1], csr_cols [B*H, G_Q*G_K]
   (key-group ids ascending within a row).  NULL outputs are skipped. */
sparsepr_status sparsepr_route(const sparsepr_config* cfg, const sparsepr_tensors* io,
                               const int* q_labels, const int* kv_labels,
                               void* workspace, size_t workspace_bytes, void* stream,
                               int* perm_q, int* perm_k, int* off_q, int* off_k,
                               int* csr_rowptr, int* csr_cols, sparsepr_head_stats* stats);

/* Stage a12 alone from given labels ([TS] 2.C: attention over the granted
   blocks of the group-contiguous layout; [NE] NE/exec): the uncorrected
   ("hard-drop") sparse output, each query's softmax taken over its group's
   granted keys only, written to io->o in the original token order.  Labels
   outside [0, G) are clamped.  Errors as sparsepr_attention. */
sparsepr_status sparsepr_sparse_attention(const sparsepr_config* cfg, const sparsepr_tensors* io,
                                          const int* q_labels, const int* kv_labels,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* Stages a11, a13-a14 from given labels ([TS] 2.B, [NE] NE/method): probe
   positions in permuted order (int32 [B*H, M]), their exact dense outputs and
   sparse outputs (float [B*H, M, d]), and the fitted correction: W and Vr
   (float [B*H, d, r], zero beyond the used rank) with B = W Vr^T, the bias
   b (float [B*H, d]) and the used rank r' (int32 [B*H]).  NULL outputs are
   skipped. */
sparsepr_status sparsepr_probe_fit(const sparsepr_config* cfg, const sparsepr_tensors* io,
                                   const int* q_labels, const int* kv_labels,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   int* probe_pos, float* o_dense, float* o_sparse,
                                   float* w_mat, float* v_mat, float* bias, int* rank);

/* Dense softmax attention over all keys (the speed baseline), bf16 or fp32,
   no workspace; scale 0 => 1/sqrt(d). */
sparsepr_status sparsepr_dense_attention(const sparsepr_tensors* io, float scale, void* stream);

/* Device property the k-means assignment's error bound relies on: one bf16
   matrix-core product (32x32x16, fp32 accumulate) lands within 18 units of
   fp32 roundoff of the sum of magnitudes of its accumulator and its 16
   products.  For each of n patterns (device float
   [n, 33]: 16 values of row 0 of A, 16 of column 0 of B, all exact in bf16,
   then the accumulator) writes element (0, 0) of the product (device float
   [n]); the caller compares it with the exact sum.  Not used by the call
   itself; n in [1, 1 << 20]. */
sparsepr_status sparsepr_mfma_rounding_check(const float* patterns, int n, float* out, void* stream);

const char* sparsepr_status_string(sparsepr_status s);
int sparsepr_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSEPR_H */
