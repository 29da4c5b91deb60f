// Host planner: argument validation and workspace layout (no HIP calls).
#include "sp_plan.h"

#include <math.h>
#include <string.h>

namespace sp {

static inline long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

sparsepr_status plan_init(Plan* p, const sparsepr_config* cfg, int B, int H, int N, int d,
                          int dtype) {
  if (!p || !cfg) return SPARSEPR_ERR_INVALID_ARG;
  memset(p, 0, sizeof(*p));
  if (B < 1 || H < 1 || (long long)B * H > (1 << 20)) return SPARSEPR_ERR_INVALID_ARG;
  if (N < 2 || N > (1 << 20)) return SPARSEPR_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SPARSEPR_ERR_UNSUPPORTED;
  if (dtype != SPARSEPR_BF16 && dtype != SPARSEPR_FP32) return SPARSEPR_ERR_UNSUPPORTED;
  if (!(cfg->density > 0.0f) || !isfinite(cfg->density)) return SPARSEPR_ERR_INVALID_ARG;
  if (cfg->probe_rows < 0 || cfg->probe_rows > kMaxProbe || cfg->probe_rows > N)
    return SPARSEPR_ERR_INVALID_ARG;
  if (cfg->n_kv_groups < 1 || cfg->n_q_groups < 1 || cfg->n_kv_groups > kMaxGroups ||
      cfg->n_q_groups > kMaxGroups || cfg->n_kv_groups > N || cfg->n_q_groups > N)
    return SPARSEPR_ERR_INVALID_ARG;
  if ((long long)cfg->n_kv_groups * cfg->n_q_groups > (1 << 20)) return SPARSEPR_ERR_INVALID_ARG;
  if (cfg->residual_rank < 0 || cfg->residual_rank > kMaxRank) return SPARSEPR_ERR_INVALID_ARG;
  if (!(cfg->ridge_lambda >= 0.0f) || !isfinite(cfg->ridge_lambda)) return SPARSEPR_ERR_INVALID_ARG;
  if (cfg->kmeans_iters < 1 || cfg->kmeans_iters > 100) return SPARSEPR_ERR_INVALID_ARG;
  if (cfg->n_sample_q < 1 || cfg->n_sample_q > 256) return SPARSEPR_ERR_INVALID_ARG;
  if (cfg->key_coord_rank < 1 || cfg->key_coord_rank > 64) return SPARSEPR_ERR_INVALID_ARG;
  if (!(cfg->scale >= 0.0f) || !isfinite(cfg->scale)) return SPARSEPR_ERR_INVALID_ARG;
  if (!(cfg->rank_cut >= 0.0f) || !(cfg->rank_cut < 1.0f)) return SPARSEPR_ERR_INVALID_ARG;
  if (cfg->partition_mode != SPARSEPR_PART_RESPONSE_COUPLED &&
      cfg->partition_mode != SPARSEPR_PART_INDEPENDENT)
    return SPARSEPR_ERR_INVALID_ARG;
  if (cfg->router != SPARSEPR_ROUTER_BUDGET && cfg->router != SPARSEPR_ROUTER_ALPHA) return SPARSEPR_ERR_INVALID_ARG;
  if (cfg->router == SPARSEPR_ROUTER_ALPHA && (!(cfg->alpha > 0.0f) || !(cfg->alpha <= 1.0f)))
    return SPARSEPR_ERR_INVALID_ARG;
  if (cfg->ridge_mode != SPARSEPR_RIDGE_RELATIVE && cfg->ridge_mode != SPARSEPR_RIDGE_ABSOLUTE)
    return SPARSEPR_ERR_INVALID_ARG;
  if (!(cfg->rank_cap > 0.0f) || !(cfg->rank_cap <= 1.0f)) return SPARSEPR_ERR_INVALID_ARG;
  if ((cfg->svd_weighted != 0 && cfg->svd_weighted != 1) ||
      (cfg->centred_query_coords != 0 && cfg->centred_query_coords != 1))
    return SPARSEPR_ERR_INVALID_ARG;

  p->B = B;
  p->H = H;
  p->BH = B * H;
  p->N = N;
  p->d = d;
  p->dtype = dtype;
  p->esize = dtype == SPARSEPR_BF16 ? 2 : 4;
  p->GK = cfg->n_kv_groups;
  p->GQ = cfg->n_q_groups;
  p->Gmax = p->GK > p->GQ ? p->GK : p->GQ;
  p->M = cfg->probe_rows;
  p->R = cfg->residual_rank;
  // the rank the fit may use: at most floor(rank_cap * M) (float32 cap times M, in fp64)
  p->Rfit = (int)floor((double)cfg->rank_cap * (double)p->M);
  if (p->Rfit > p->R) p->Rfit = p->R;
  p->svd_weighted = cfg->svd_weighted;
  p->centred_qc = cfg->centred_query_coords;
  p->Ms = cfg->n_sample_q < N ? cfg->n_sample_q : N;
  int rk = cfg->key_coord_rank;
  if (rk > d) rk = d;
  if (rk > p->Ms) rk = p->Ms;
  p->rK = rk;
  p->rKpad = (int)cdiv(rk, 16) * 16;
  p->T = cfg->kmeans_iters;
  p->mode = cfg->partition_mode;
  p->Dk = p->mode == SPARSEPR_PART_RESPONSE_COUPLED ? p->rKpad : d;
  p->nchunk = (int)cdiv(N, kChunk);
  p->max_tiles = (int)cdiv(N, kTileRows) + p->GQ;
  {
    // keys per probe workgroup: small calls split the keys finer, so that
    // about kProbeSlots workgroups share the chip instead of a few long ones
    const long long pblocks = cdiv(p->M > 0 ? p->M : 1, 64) * (long long)p->BH;
    long long want = cdiv(cdiv((long long)N * pblocks, kProbeSlots), 64) * 64;
    if (want < 64) want = 64;
    if (want > kProbeChunkMax) want = kProbeChunkMax;
    p->pchunk = (int)want;
  }
  p->n_pchunk = (int)cdiv(N, p->pchunk);
  p->gwords = (int)cdiv(p->GK, 32);
  float s = cfg->scale > 0.0f ? cfg->scale : (float)(1.0 / sqrt((double)d));
  p->scale = s;
  p->density = cfg->density;
  p->lambda = cfg->ridge_lambda;
  p->ridge_mode = cfg->ridge_mode;
  p->rank_cut = cfg->rank_cut;
  p->seed = cfg->seed;
  p->router = cfg->router;
  p->alpha = cfg->alpha;
  double nn = (double)N * (double)N;
  if (p->router == SPARSEPR_ROUTER_ALPHA) {
    p->dense_route = false;  // the alpha rule decides every cell; no budget
    p->budget = (long long)N * N;
  } else {
    p->dense_route = cfg->density >= 1.0f;
    p->budget = (long long)floor((double)cfg->density * nn) - (long long)p->M * N;
  }
  return SPARSEPR_OK;
}

static bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

static sparsepr_status view_ok(const void* ptr, const long long* st, int esize) {
  if (!ptr) return SPARSEPR_ERR_INVALID_ARG;
  if (st[3] != 1) return SPARSEPR_ERR_UNSUPPORTED;
  if (!aligned16(ptr)) return SPARSEPR_ERR_UNSUPPORTED;
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || (st[i] * esize) % 16 != 0) return SPARSEPR_ERR_UNSUPPORTED;
  return SPARSEPR_OK;
}

sparsepr_status plan_io(Plan* p, const sparsepr_tensors* io) {
  if (!io) return SPARSEPR_ERR_INVALID_ARG;
  if (io->B != p->B || io->H != p->H || io->N != p->N || io->d != p->d || io->dtype != p->dtype)
    return SPARSEPR_ERR_INVALID_ARG;
  sparsepr_status s;
  if ((s = view_ok(io->q, io->q_strides, p->esize)) != SPARSEPR_OK) return s;
  if ((s = view_ok(io->k, io->k_strides, p->esize)) != SPARSEPR_OK) return s;
  if ((s = view_ok(io->v, io->v_strides, p->esize)) != SPARSEPR_OK) return s;
  if ((s = view_ok(io->o, io->o_strides, p->esize)) != SPARSEPR_OK) return s;
  if (io->o == io->q || io->o == io->k || io->o == io->v) return SPARSEPR_ERR_INVALID_ARG;
  p->q = View4{io->q, io->q_strides[0], io->q_strides[1], io->q_strides[2], p->H};
  p->k = View4{io->k, io->k_strides[0], io->k_strides[1], io->k_strides[2], p->H};
  p->v = View4{io->v, io->v_strides[0], io->v_strides[1], io->v_strides[2], p->H};
  p->o = MutView4{io->o, io->o_strides[0], io->o_strides[1], io->o_strides[2], p->H};
  return SPARSEPR_OK;
}

namespace {
struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(long long count) {
    off = (off + 255) & ~(size_t)255;
    T* r = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += (size_t)count * sizeof(T);
    return r;
  }
};
}  // namespace

void plan_carve(Plan* p, char* base) {
  Carver c{base};
  const long long BH = p->BH, N = p->N, d = p->d;
  const long long Dmax = p->Dk > p->d ? p->Dk : p->d;
  p->sample = c.take<int>(BH * p->Ms);
  p->mk = c.take<double>(BH * d * d);
  p->eigval = c.take<double>(BH * d);
  p->kmap = c.take<double>(BH * d * p->rK);
  p->kmap_pad = c.take<double>(BH * d * p->rKpad);
  p->eigz = c.take<double>(BH * d * d);
  const bool rcp = p->mode == SPARSEPR_PART_RESPONSE_COUPLED;
  p->z64 = rcp ? c.take<double>(BH * N * p->rKpad) : nullptr;
  p->xbound = rcp ? c.take<float2>(BH * N) : nullptr;
  p->zhi = rcp ? c.take<bf16_t>(BH * N * p->rKpad) : nullptr;
  p->zlo = rcp ? c.take<bf16_t>(BH * N * p->rKpad) : nullptr;
  const bool f32 = p->dtype == SPARSEPR_FP32;
  p->phi = f32 ? c.take<bf16_t>(BH * N * d) : nullptr;
  p->plo = f32 ? c.take<bf16_t>(BH * N * d) : nullptr;
  p->cmean = c.take<double>(BH * p->Gmax * Dmax);
  p->yhi = c.take<bf16_t>(BH * p->Gmax * Dmax);
  p->ylo = c.take<bf16_t>(BH * p->Gmax * Dmax);
  p->ybias = c.take<float>(BH * p->Gmax);
  p->y64 = c.take<double>(BH * p->Gmax * Dmax);
  p->y64t = c.take<double>(BH * p->Gmax * Dmax);
  p->c64 = c.take<double>(BH * p->Gmax);
  p->ybound = c.take<float>(BH * p->Gmax * 4);
  p->fcount = c.take<int>(BH * 4 * p->T);
  p->flist = c.take<int4>(BH * N);
  p->labels = c.take<int>(BH * N);
  p->counts = c.take<int>(BH * p->nchunk * p->Gmax);
  p->chunkoff = c.take<int>(BH * p->nchunk * p->Gmax);
  p->perm_w = c.take<int>(BH * N);
  p->off_w = c.take<int>(BH * (p->Gmax + 1));
  p->kv_labels = c.take<int>(BH * N);
  p->q_labels = c.take<int>(BH * N);
  p->perm_k = c.take<int>(BH * N);
  p->off_k = c.take<int>(BH * (p->GK + 1));
  p->perm_q = c.take<int>(BH * N);
  p->off_q = c.take<int>(BH * (p->GQ + 1));
  p->cbar = c.take<double>(BH * p->GK * d);
  p->qbar = c.take<double>(BH * p->GQ * d);
  p->mq = c.take<double>(BH * d * d);
  p->kp = c.take<char>(BH * N * d * p->esize);
  p->vp = c.take<char>(BH * N * d * p->esize);
  p->kgroup = c.take<int>(BH * N);
  p->vmax = c.take<uint32_t>(BH);
  p->vexp = c.take<int>(BH);
  p->mu = c.take<double>(BH * (long long)p->GQ * p->GK);
  p->ckey = c.take<uint64_t>(BH * (long long)p->GQ * p->GK);
  p->rmass = p->router == SPARSEPR_ROUTER_ALPHA ? c.take<double>(BH * (long long)p->GQ * p->GK) : nullptr;
  p->mand = c.take<int>(BH * p->GQ);
  p->thr = c.take<long long>(BH * 4);
  p->csr_ptr = c.take<int>(BH * (p->GQ + 1));
  p->csr_col = c.take<int>(BH * (long long)p->GQ * p->GK);
  p->gmask = c.take<uint32_t>(BH * (long long)p->GQ * p->gwords);
  p->lg = c.take<long long>(BH * p->GQ);
  p->tiles = c.take<int>(BH * (long long)p->max_tiles * 4);
  p->ntiles = c.take<int>(BH);
  const long long M = p->M > 0 ? p->M : 1;
  p->ppos = c.take<int>(BH * M);
  p->pgroup = c.take<int>(BH * M);
  p->pw = c.take<double>(BH * M);
  p->ppart = c.take<float>(BH * p->n_pchunk * 2 * M * (d + 2));
  p->ode = c.take<float>(BH * M * d);
  p->osp = c.take<float>(BH * M * d);
  const long long R = p->R > 0 ? p->R : 1;
  p->fitW = c.take<float>(BH * d * R);
  p->fitV = c.take<float>(BH * d * R);
  p->fitb = c.take<float>(BH * d);
  p->fitrank = c.take<int>(BH);
  p->Rp = (int)((R + 31) / 32 * 32);
  p->fitpk = c.take<bf16_t>(BH * 4 * p->Rp * d);
  p->fitscratch = c.take<double>(BH * kFitScratchDoubles);
  p->stats = c.take<sparsepr_head_stats>(BH);
  p->ws_bytes = (c.off + 255) & ~(size_t)255;
}

}  // namespace sp
