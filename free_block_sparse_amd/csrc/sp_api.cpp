// C ABI entry points: validation, workspace carve-up and stage chaining on one
// stream.  The host never synchronises and never reads device data.
#include <string.h>

#include "sp_kernels.h"

using namespace sp;

static thread_local int g_last_hip = 0;

#define HIPCHK(x)                      \
  do {                                 \
    hipError_t e_ = (x);               \
    if (e_ != hipSuccess) {            \
      g_last_hip = (int)e_;            \
      return SPARSEPR_ERR_HIP;         \
    }                                  \
  } while (0)

#define SPCHK(x)                       \
  do {                                 \
    sparsepr_status s_ = (x);          \
    if (s_ != SPARSEPR_OK) return s_;  \
  } while (0)

namespace {

// Optional per-stage events (profiling entry point only).
struct Stager {
  hipEvent_t ev[SPARSEPR_N_STAGES + 1];
  int id[SPARSEPR_N_STAGES + 1];
  int n = 0;
  hipStream_t s;
};

inline sparsepr_status mark(Stager* st, int stage) {
  if (!st) return SPARSEPR_OK;
  if (st->n > SPARSEPR_N_STAGES) return SPARSEPR_ERR_INTERNAL;
  HIPCHK(hipEventRecord(st->ev[st->n], st->s));
  st->id[st->n] = stage;
  st->n += 1;
  return SPARSEPR_OK;
}

sparsepr_status prepare(Plan& p, const sparsepr_config* cfg, const sparsepr_tensors* io, void* ws,
                        size_t ws_bytes) {
  if (!io) return SPARSEPR_ERR_INVALID_ARG;
  SPCHK(plan_init(&p, cfg, io->B, io->H, io->N, io->d, io->dtype));
  SPCHK(plan_io(&p, io));
  plan_carve(&p, nullptr);
  if (!ws) return SPARSEPR_ERR_INVALID_ARG;
  if (((uintptr_t)ws & 255u) != 0) return SPARSEPR_ERR_INVALID_ARG;
  if (ws_bytes < p.ws_bytes) return SPARSEPR_ERR_WORKSPACE;
  plan_carve(&p, static_cast<char*>(ws));
  return SPARSEPR_OK;
}

View4 contig(const void* ptr, const Plan& p, int D) {
  const long long nd = (long long)p.N * D;
  return View4{ptr, (long long)p.H * nd, nd, D, p.H};
}

// Relative error constants of the k-means assignment's approximate values
// for a point dimension D (multiple of 16).  Every accumulation chain adds
// mf MFMAs per 16 dims (hi and lo image rows, and with split points the lo
// point row) onto the fp32 bias.  One bf16 MFMA is taken to be off by at
// most 18 u (|acc| + sum |products|): its 17 terms aligned to the largest
// one with 24-bit truncation, then one rounding (the bound is checked on the
// device by sparsepr_mfma_rounding_check; it also covers 16 sequential fp32
// additions).  A chain of m MFMAs is then within gamma_K, K = 18 m, of the
// sum of magnitudes.  Split points without per-point bounds (fp32 inputs)
// add their residual (at most 2^-16 of |x|) and the dropped lo.lo product
// (2^-16 |x| |y|).
static void assign_eps(int D, bool lo, float* eps_x, float* eps_acc) {
  const double u = 0x1p-24;
  const double K = 18.0 * (lo ? 3 : 2) * (D / 16);
  *eps_acc = (float)(1.05 * K * u / (1.0 - K * u) + 4.0 * u);
  *eps_x = lo ? (float)(1.05 * (0x1p-16 + 0x1p-16 + u)) : 0.f;
}

// Lloyd k-means on one side.  side 0 = keys, 1 = queries.  Leaves the final
// labels in `labels_out`, the stable grouping in perm_out / off_out.  Each
// assignment is followed by the exact re-decision of its flagged near ties,
// so the labels are those of an fp64 assignment.
sparsepr_status kmeans_side(Plan& p, int side, int G, int* labels_out, int* perm_out, int* off_out,
                            hipStream_t s) {
  const bool rcp = p.mode == SPARSEPR_PART_RESPONSE_COUPLED;
  const bool f32 = p.dtype == SPARSEPR_FP32;
  const View4& raw = side == 0 ? p.k : p.q;
  AssignArgs aa;
  memset(&aa, 0, sizeof(aa));
  UpdateArgs ua;
  memset(&ua, 0, sizeof(ua));
  RedecideArgs ra;
  memset(&ra, 0, sizeof(ra));
  int D;
  bool lo;
  int pts_type;  // 0 bf16, 1 fp32, 2 fp64 for the update kernel
  if (side == 0 && rcp) {
    D = p.rKpad;
    lo = true;
    aa.pts = contig(p.zhi, p, D);
    aa.pts_lo = p.zlo;
    ua.pts = View4{p.z64, (long long)p.H * p.N * p.rKpad, (long long)p.N * p.rKpad, p.rKpad, p.H};
    ua.Dp = p.rK;
    ua.Dimg = p.rKpad;
    ua.metric = nullptr;
    pts_type = 2;
    ra.x64 = p.z64;
    ra.x64stride = p.rKpad;
    ra.Dx = p.rK;
  } else {
    D = p.d;
    if (f32) {
      HIPCHK(launch_split_rows(p, raw, s));
      aa.pts = contig(p.phi, p, D);
      aa.pts_lo = p.plo;
      lo = true;
    } else {
      aa.pts = raw;
      aa.pts_lo = nullptr;
      lo = false;
    }
    ua.pts = raw;
    ua.Dp = p.d;
    ua.Dimg = p.d;
    ua.metric = (side == 1 && rcp) ? p.mq : nullptr;
    pts_type = f32 ? 1 : 0;
    ra.raw = raw;
    ra.Dx = p.d;
  }
  const int Dmax = p.Dk > p.d ? p.Dk : p.d;
  aa.yhi = p.yhi;
  aa.ylo = p.ylo;
  aa.ybias = p.ybias;
  aa.ystride = Dmax;
  aa.gstride = p.Gmax;
  aa.N = p.N;
  aa.G = G;
  aa.labels = p.labels;
  aa.counts = p.counts;
  aa.nchunk = p.nchunk;
  aa.ybound = p.ybound;
  aa.xbound = (side == 0 && rcp) ? p.xbound : nullptr;
  assign_eps(D, lo, &aa.eps_x, &aa.eps_acc);
  // the assignment packs a value's 32-centre block and accumulator register
  // into its low 4 + ceil(log2(blocks)) mantissa bits
  aa.pbits = 4;
  while ((1 << (aa.pbits - 4)) * 32 < G) ++aa.pbits;
  int* fc = p.fcount + side * p.T;  // key side: steps 0..T-1, query side: T..2T-1 (full flags: + 2T)
  aa.fcstride = 4 * p.T;
  aa.fcfull = 2 * p.T;
  aa.flist = p.flist;

  ra.y64 = p.y64;
  ra.y64t = p.y64t;
  ra.c64 = p.c64;
  ra.ystride = Dmax;
  ra.gstride = p.Gmax;
  ra.N = p.N;
  ra.G = G;
  ra.fcstride = 4 * p.T;
  ra.fcfull = 2 * p.T;
  ra.flist = p.flist;
  ra.labels = p.labels;
  ra.counts = p.counts;
  ra.nchunk = p.nchunk;
  const int raw_type = f32 ? 1 : 0;

  ua.perm = p.perm_w;
  ua.off = p.off_w;
  ua.offstride = p.Gmax + 1;
  ua.cmean = p.cmean;
  ua.cstride = Dmax;
  ua.yhi = p.yhi;
  ua.ylo = p.ylo;
  ua.ybias = p.ybias;
  ua.y64 = p.y64;
  ua.y64t = p.y64t;
  ua.c64 = p.c64;
  ua.ybound = p.ybound;
  ua.ystride = Dmax;
  ua.gstride = p.Gmax;
  ua.G = G;
  ua.N = p.N;
  ua.fcount = fc;
  ua.T = p.T;
  ua.init = 1;
  HIPCHK(launch_centre_update(p, ua, pts_type, s));
  ua.init = 0;
  for (int t = 0; t < p.T; ++t) {
    const bool last = t == p.T - 1;
    aa.fcnt = fc + t;
    ra.fcnt = fc + t;
    HIPCHK(launch_assign(p, aa, D, lo, s));
    HIPCHK(launch_redecide(p, ra, raw_type, s));
    ScanArgs sa{p.counts, p.chunkoff, last ? off_out : p.off_w, last ? G + 1 : p.Gmax + 1, p.nchunk, G, p.Gmax, p.N};
    HIPCHK(launch_group_scan(p, sa, s));
    ScatterArgs sc{p.labels, p.chunkoff, last ? perm_out : p.perm_w, last ? labels_out : nullptr, p.N, p.nchunk,
                   p.Gmax};
    HIPCHK(launch_group_scatter(p, sc, s));
    if (!last) HIPCHK(launch_centre_update(p, ua, pts_type, s));
  }
  return SPARSEPR_OK;
}

// group means of raw rows over a finished grouping
sparsepr_status raw_means(Plan& p, const View4& raw, const int* perm, const int* off, int G, double* out,
                          hipStream_t s) {
  UpdateArgs ua;
  memset(&ua, 0, sizeof(ua));
  ua.pts = raw;
  ua.Dp = p.d;
  ua.Dimg = p.d;
  ua.perm = perm;
  ua.off = off;
  ua.offstride = G + 1;
  ua.G = G;
  ua.N = p.N;
  ua.means_only = 1;
  ua.means_out = out;
  ua.mo_gstride = G;
  HIPCHK(launch_centre_update(p, ua, p.dtype == SPARSEPR_FP32 ? 1 : 0, s));
  return SPARSEPR_OK;
}

sparsepr_status run_partition(Plan& p, hipStream_t s, Stager* st = nullptr) {
  const bool rcp = p.mode == SPARSEPR_PART_RESPONSE_COUPLED;
  SPCHK(mark(st, -1));
  if (rcp) {
    HIPCHK(launch_sample_metric(p, s));
    SPCHK(mark(st, SPARSEPR_STAGE_SAMPLE_METRIC));
    HIPCHK(launch_key_eig(p, s, false));
    SPCHK(mark(st, SPARSEPR_STAGE_KEY_EIGEN));
    HIPCHK(launch_key_coords(p, s));
    SPCHK(mark(st, SPARSEPR_STAGE_KEY_COORDS));
  }
  SPCHK(kmeans_side(p, 0, p.GK, p.kv_labels, p.perm_k, p.off_k, s));
  SPCHK(mark(st, SPARSEPR_STAGE_KEY_KMEANS));
  SPCHK(raw_means(p, p.k, p.perm_k, p.off_k, p.GK, p.cbar, s));
  if (rcp) HIPCHK(launch_query_metric(p, s));
  SPCHK(mark(st, SPARSEPR_STAGE_KEY_CENTRES));
  SPCHK(kmeans_side(p, 1, p.GQ, p.q_labels, p.perm_q, p.off_q, s));
  p.kmeans_ran = true;
  SPCHK(mark(st, SPARSEPR_STAGE_QUERY_KMEANS));
  SPCHK(raw_means(p, p.q, p.perm_q, p.off_q, p.GQ, p.qbar, s));
  SPCHK(mark(st, SPARSEPR_STAGE_QUERY_CENTRES));
  return SPARSEPR_OK;
}

sparsepr_status group_given(Plan& p, const int* labels, int G, int* labels_out, int* perm_out, int* off_out,
                            hipStream_t s) {
  CountArgs ca{labels, p.labels, p.counts, p.N, G, p.nchunk, p.Gmax};
  HIPCHK(launch_count_labels(p, ca, s));
  ScanArgs sa{p.counts, p.chunkoff, off_out, G + 1, p.nchunk, G, p.Gmax, p.N};
  HIPCHK(launch_group_scan(p, sa, s));
  ScatterArgs sc{p.labels, p.chunkoff, perm_out, labels_out, p.N, p.nchunk, p.Gmax};
  HIPCHK(launch_group_scatter(p, sc, s));
  return SPARSEPR_OK;
}

sparsepr_status run_given_partition(Plan& p, const int* q_labels, const int* kv_labels, hipStream_t s) {
  if (!q_labels || !kv_labels) return SPARSEPR_ERR_INVALID_ARG;
  SPCHK(group_given(p, kv_labels, p.GK, p.kv_labels, p.perm_k, p.off_k, s));
  SPCHK(raw_means(p, p.k, p.perm_k, p.off_k, p.GK, p.cbar, s));
  SPCHK(group_given(p, q_labels, p.GQ, p.q_labels, p.perm_q, p.off_q, s));
  SPCHK(raw_means(p, p.q, p.perm_q, p.off_q, p.GQ, p.qbar, s));
  return SPARSEPR_OK;
}

sparsepr_status run_after_partition(Plan& p, hipStream_t s, sparsepr_head_stats* stats, Stager* st = nullptr) {
  HIPCHK(launch_route(p, s));
  SPCHK(mark(st, SPARSEPR_STAGE_ROUTE));
  HIPCHK(launch_gather(p, s));
  SPCHK(mark(st, SPARSEPR_STAGE_GATHER));
  HIPCHK(launch_probe_select(p, s));
  HIPCHK(launch_probe_attention(p, s));
  SPCHK(mark(st, SPARSEPR_STAGE_PROBES));
  HIPCHK(launch_fit(p, s));
  SPCHK(mark(st, SPARSEPR_STAGE_FIT));
  HIPCHK(launch_sparse_attention(p, true, s));
  SPCHK(mark(st, SPARSEPR_STAGE_SPARSE_ATTENTION));
  HIPCHK(launch_probe_overwrite(p, s));
  SPCHK(mark(st, SPARSEPR_STAGE_RESTORE));
  if (stats) HIPCHK(hipMemcpyAsync(stats, p.stats, sizeof(sparsepr_head_stats) * p.BH, hipMemcpyDeviceToDevice, s));
  return SPARSEPR_OK;
}

template <typename T>
sparsepr_status copy_out(T* dst, const T* src, long long count, hipStream_t s) {
  if (!dst) return SPARSEPR_OK;
  HIPCHK(hipMemcpyAsync(dst, src, sizeof(T) * count, hipMemcpyDeviceToDevice, s));
  return SPARSEPR_OK;
}

// copy a [BH, G+1] offsets array (all the same stride) out

}  // namespace

extern "C" {

sparsepr_status sparsepr_config_default(int N, int d, sparsepr_config* out) {
  if (!out || N < 2 || (d != 64 && d != 128)) return SPARSEPR_ERR_INVALID_ARG;
  memset(out, 0, sizeof(*out));
  int g = N / 128;
  if (g < 1) g = 1;
  if (g > 256) g = 256;
  out->density = 0.25f;
  out->probe_rows = N < 64 ? N : 64;
  out->n_kv_groups = g;
  out->n_q_groups = g;
  out->residual_rank = 32;
  out->ridge_lambda = 1.0f;
  out->ridge_mode = SPARSEPR_RIDGE_RELATIVE;
  out->kmeans_iters = 10;
  out->n_sample_q = 256;
  out->key_coord_rank = 32;
  out->scale = 0.0f;
  out->rank_cut = 1e-6f;
  out->partition_mode = SPARSEPR_PART_RESPONSE_COUPLED;
  out->seed = 0;
  out->router = SPARSEPR_ROUTER_BUDGET;
  out->alpha = 0.9f;
  out->rank_cap = 1.0f;
  out->svd_weighted = 0;
  out->centred_query_coords = 0;
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_validate(const sparsepr_config* cfg, int B, int H, int N, int d, int dtype) {
  Plan p;
  return plan_init(&p, cfg, B, H, N, d, dtype);
}

sparsepr_status sparsepr_workspace_size(const sparsepr_config* cfg, int B, int H, int N, int d, int dtype,
                                        size_t* bytes) {
  if (!bytes) return SPARSEPR_ERR_INVALID_ARG;
  Plan p;
  SPCHK(plan_init(&p, cfg, B, H, N, d, dtype));
  plan_carve(&p, nullptr);
  *bytes = p.ws_bytes;
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_attention(const sparsepr_config* cfg, const sparsepr_tensors* io, void* workspace,
                                   size_t workspace_bytes, void* stream, sparsepr_head_stats* stats) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  Plan p;
  SPCHK(prepare(p, cfg, io, workspace, workspace_bytes));
  SPCHK(run_partition(p, s));
  return run_after_partition(p, s, stats);
}

sparsepr_status sparsepr_attention_noalloc(const sparsepr_config* cfg, const sparsepr_tensors* io, void* stream,
                                           sparsepr_head_stats* stats) {
  // shape and size checks first: no device call for a rejected request
  if (!io) return SPARSEPR_ERR_INVALID_ARG;
  Plan p;
  SPCHK(plan_init(&p, cfg, io->B, io->H, io->N, io->d, io->dtype));
  SPCHK(plan_io(&p, io));
  plan_carve(&p, nullptr);
  if (p.ws_bytes > kNoAllocScratchBytes) return SPARSEPR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (s) {
    // the scratch used is the current device's: the stream must live there
    int cur = 0, sdev = 0;
    HIPCHK(hipGetDevice(&cur));
    HIPCHK(hipStreamGetDevice(s, &sdev));
    if (sdev != cur) return SPARSEPR_ERR_INVALID_ARG;
  }
  void* base = nullptr;
  HIPCHK(noalloc_scratch(&base));
  SPCHK(prepare(p, cfg, io, base, kNoAllocScratchBytes));
  SPCHK(run_partition(p, s));
  return run_after_partition(p, s, stats);
}

size_t sparsepr_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

sparsepr_status sparsepr_attention_profile(const sparsepr_config* cfg, const sparsepr_tensors* io,
                                           void* workspace, size_t workspace_bytes, void* stream,
                                           sparsepr_head_stats* stats, float* stage_ms) {
  if (!stage_ms) return SPARSEPR_ERR_INVALID_ARG;
  Plan p;
  SPCHK(prepare(p, cfg, io, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  Stager st;
  st.s = s;
  int made = 0;
  sparsepr_status rc = SPARSEPR_OK;
  for (; made <= SPARSEPR_N_STAGES; ++made) {
    hipError_t e = hipEventCreate(&st.ev[made]);
    if (e != hipSuccess) {
      g_last_hip = (int)e;
      rc = SPARSEPR_ERR_HIP;
      break;
    }
  }
  if (rc == SPARSEPR_OK) rc = run_partition(p, s, &st);
  if (rc == SPARSEPR_OK) rc = run_after_partition(p, s, stats, &st);
  if (rc == SPARSEPR_OK) {
    for (int i = 0; i < SPARSEPR_N_STAGES; ++i) stage_ms[i] = 0.f;
    hipError_t e = hipEventSynchronize(st.ev[st.n - 1]);
    for (int i = 1; i < st.n && e == hipSuccess; ++i) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, st.ev[i - 1], st.ev[i]);
      if (st.id[i] >= 0) stage_ms[st.id[i]] += ms;
    }
    if (e != hipSuccess) {
      g_last_hip = (int)e;
      rc = SPARSEPR_ERR_HIP;
    }
  }
  for (int i = 0; i < made; ++i) (void)hipEventDestroy(st.ev[i]);
  return rc;
}

sparsepr_status sparsepr_attention_with_partition(const sparsepr_config* cfg, const sparsepr_tensors* io,
                                                  const int* q_labels, const int* kv_labels, void* workspace,
                                                  size_t workspace_bytes, void* stream,
                                                  sparsepr_head_stats* stats) {
  Plan p;
  SPCHK(prepare(p, cfg, io, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  SPCHK(run_given_partition(p, q_labels, kv_labels, s));
  return run_after_partition(p, s, stats);
}

sparsepr_status sparsepr_key_metric(const sparsepr_config* cfg, const sparsepr_tensors* io, void* workspace,
                                    size_t workspace_bytes, void* stream, int* sample_idx, double* m_k,
                                    double* eigvals, double* key_map) {
  Plan p;
  SPCHK(prepare(p, cfg, io, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIPCHK(launch_sample_metric(p, s));
  HIPCHK(launch_key_eig(p, s, true));
  SPCHK(copy_out(sample_idx, p.sample, (long long)p.BH * p.Ms, s));
  SPCHK(copy_out(m_k, p.mk, (long long)p.BH * p.d * p.d, s));
  SPCHK(copy_out(eigvals, p.eigval, (long long)p.BH * p.d, s));
  SPCHK(copy_out(key_map, p.kmap, (long long)p.BH * p.d * p.rK, s));
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_partition(const sparsepr_config* cfg, const sparsepr_tensors* io, void* workspace,
                                   size_t workspace_bytes, void* stream, int* q_labels, int* kv_labels) {
  Plan p;
  SPCHK(prepare(p, cfg, io, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  SPCHK(run_partition(p, s));
  SPCHK(copy_out(q_labels, p.q_labels, (long long)p.BH * p.N, s));
  SPCHK(copy_out(kv_labels, p.kv_labels, (long long)p.BH * p.N, s));
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_route(const sparsepr_config* cfg, const sparsepr_tensors* io, const int* q_labels,
                               const int* kv_labels, void* workspace, size_t workspace_bytes, void* stream,
                               int* perm_q, int* perm_k, int* off_q, int* off_k, int* csr_rowptr, int* csr_cols,
                               sparsepr_head_stats* stats) {
  Plan p;
  SPCHK(prepare(p, cfg, io, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  SPCHK(run_given_partition(p, q_labels, kv_labels, s));
  HIPCHK(launch_route(p, s));
  SPCHK(copy_out(perm_q, p.perm_q, (long long)p.BH * p.N, s));
  SPCHK(copy_out(perm_k, p.perm_k, (long long)p.BH * p.N, s));
  SPCHK(copy_out(off_q, p.off_q, (long long)p.BH * (p.GQ + 1), s));
  SPCHK(copy_out(off_k, p.off_k, (long long)p.BH * (p.GK + 1), s));
  SPCHK(copy_out(csr_rowptr, p.csr_ptr, (long long)p.BH * (p.GQ + 1), s));
  SPCHK(copy_out(csr_cols, p.csr_col, (long long)p.BH * p.GQ * p.GK, s));
  SPCHK(copy_out(stats, p.stats, p.BH, s));
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_sparse_attention(const sparsepr_config* cfg, const sparsepr_tensors* io,
                                          const int* q_labels, const int* kv_labels, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  Plan p;
  SPCHK(prepare(p, cfg, io, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  SPCHK(run_given_partition(p, q_labels, kv_labels, s));
  HIPCHK(launch_route(p, s));
  HIPCHK(launch_gather(p, s));
  HIPCHK(launch_sparse_attention(p, false, s));
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_probe_fit(const sparsepr_config* cfg, const sparsepr_tensors* io, const int* q_labels,
                                   const int* kv_labels, void* workspace, size_t workspace_bytes, void* stream,
                                   int* probe_pos, float* o_dense, float* o_sparse, float* w_mat, float* v_mat,
                                   float* bias, int* rank) {
  Plan p;
  SPCHK(prepare(p, cfg, io, workspace, workspace_bytes));
  if (p.M <= 0) return SPARSEPR_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  SPCHK(run_given_partition(p, q_labels, kv_labels, s));
  HIPCHK(launch_route(p, s));
  HIPCHK(launch_gather(p, s));
  HIPCHK(launch_probe_select(p, s));
  HIPCHK(launch_probe_attention(p, s));
  HIPCHK(launch_fit(p, s));
  const long long R = p.R > 0 ? p.R : 1;
  SPCHK(copy_out(probe_pos, p.ppos, (long long)p.BH * p.M, s));
  SPCHK(copy_out(o_dense, p.ode, (long long)p.BH * p.M * p.d, s));
  SPCHK(copy_out(o_sparse, p.osp, (long long)p.BH * p.M * p.d, s));
  SPCHK(copy_out(w_mat, p.fitW, (long long)p.BH * p.d * R, s));
  SPCHK(copy_out(v_mat, p.fitV, (long long)p.BH * p.d * R, s));
  SPCHK(copy_out(bias, p.fitb, (long long)p.BH * p.d, s));
  SPCHK(copy_out(rank, p.fitrank, (long long)p.BH, s));
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_dense_attention(const sparsepr_tensors* io, float scale, void* stream) {
  if (!io) return SPARSEPR_ERR_INVALID_ARG;
  sparsepr_config cfg;
  SPCHK(sparsepr_config_default(io->N < 2 ? 2 : io->N, io->d == 64 ? 64 : 128, &cfg));
  Plan p;
  SPCHK(plan_init(&p, &cfg, io->B, io->H, io->N, io->d, io->dtype));
  SPCHK(plan_io(&p, io));
  const float s = scale > 0.f ? scale : p.scale;
  HIPCHK(launch_dense_attention(p.q, p.k, p.v, p.o, p.BH, p.N, p.d, p.dtype, s, static_cast<hipStream_t>(stream)));
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_mfma_rounding_check(const float* patterns, int n, float* out, void* stream) {
  if (!patterns || !out || n < 1 || n > (1 << 20)) return SPARSEPR_ERR_INVALID_ARG;
  HIPCHK(launch_mfma_rounding(patterns, n, out, static_cast<hipStream_t>(stream)));
  return SPARSEPR_OK;
}

const char* sparsepr_status_string(sparsepr_status s) {
  switch (s) {
    case SPARSEPR_OK: return "ok";
    case SPARSEPR_ERR_INVALID_ARG: return "invalid argument";
    case SPARSEPR_ERR_UNSUPPORTED: return "unsupported shape, dtype or layout";
    case SPARSEPR_ERR_WORKSPACE: return "workspace too small";
    case SPARSEPR_ERR_HIP: return "HIP launch or copy failed (see sparsepr_last_hip_error)";
    case SPARSEPR_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

int sparsepr_last_hip_error(void) { return g_last_hip; }

}  // extern "C"
