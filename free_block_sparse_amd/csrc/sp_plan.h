// Host-side call plan: validated shape, method settings and the carve-up of
// the caller's workspace.  Pure host code; no HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "sp_common.h"

namespace sp {

constexpr int kChunk = 256;      // points per k-means histogram chunk
constexpr int kTileRows = 128;   // query rows per sparse-attention workgroup
constexpr int kProbeChunkMax = 1024;  // most keys per probe-attention workgroup
constexpr int kProbeSlots = 512;      // probe workgroups wanted per call (two per CU)
constexpr int kMaxProbe = 256;
constexpr int kMaxRank = 64;
constexpr int kMaxGroups = 1024;
constexpr long long kFitScratchDoubles = 7LL * 128 * 128;  // per (b,h) fit scratch
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;  // fixed scratch of sparsepr_attention_noalloc

struct Plan {
  // shape and settings
  int B, H, BH, N, d, dtype, esize;
  int bh0;  // index of this plan's first head in the caller's call (seeds the query sample)
  int GK, GQ, Gmax, M, R, Ms, rK, rKpad, T, mode;
  int Dk;            // key-side k-means point dimension (padded to 16)
  int ridge_mode;
  int Rfit;          // fit rank bound: min(R, floor(rank_cap * M))
  int svd_weighted;  // residual subspace from the SVD of D^(1/2) R
  int centred_qc;    // query coordinates centred per query
  int nchunk;        // ceil(N / kChunk)
  int max_tiles;     // per (b,h) upper bound of query tiles
  int pchunk;        // keys per probe-attention workgroup (a multiple of 64)
  int n_pchunk;      // probe key chunks per (b,h)
  int gwords;        // ceil(GK / 32)
  float scale, density, lambda, rank_cut;
  unsigned long long seed;
  long long budget;  // routed-pair budget per (b,h) (N^2 under the alpha router)
  int router;        // sparsepr_router
  float alpha;       // target retained mass of the alpha router
  bool dense_route;  // density >= 1: every cell granted

  View4 q, k, v;
  MutView4 o;

  // ---- workspace (device pointers) ----
  int* sample;            // [BH, Ms]
  double* mk;             // [BH, d, d]
  double* eigval;         // [BH, d]
  double* kmap;           // [BH, d, rK]
  double* kmap_pad;       // [BH, d, rKpad] the same, zero beyond rK
  double* eigz;           // [BH, d, d] eigensolver vectors (scratch)
  double* z64;            // [BH, N, rKpad] key coordinates (zero beyond rK)
  float2* xbound;         // [BH, N] bounds of each key's hi/lo split residual and lo part
  bf16_t* zhi;            // [BH, N, rKpad]
  bf16_t* zlo;            // [BH, N, rKpad]
  bf16_t* phi;            // [BH, N, d] raw points split (fp32 inputs only)
  bf16_t* plo;            // [BH, N, d]
  double* cmean;          // [BH, Gmax, Dmax] k-means centres (coordinate or raw space)
  bf16_t* yhi;            // [BH, Gmax, Dmax] centre images (hi part)
  bf16_t* ylo;            // [BH, Gmax, Dmax] centre images (lo part)
  float* ybias;           // [BH, Gmax]
  double* y64;            // [BH, Gmax, Dmax] centre images in fp64
  double* y64t;           // [BH, Dmax, Gmax] the same, dimension-major
  double* c64;            // [BH, Gmax] centre bias x.y of the images in fp64
  float* ybound;          // [BH, Gmax, 4] upper bounds of |y_g|, |c_g|, |y_g - hi - lo| and |lo|
  int* fcount;            // [BH, 4T] near-tie points flagged per Lloyd step: two-candidate flags (key
                          // side, then query side), then full flags (key side, then query side)
  bool kmeans_ran;        // set once this plan's partition came from its own k-means
  int4* flist;            // [BH, N] flagged points of the current step (point, two candidates, full flag)
  int* labels;            // [BH, N] working labels
  int* counts;            // [BH, nchunk, Gmax]
  int* chunkoff;          // [BH, nchunk, Gmax]
  int* perm_w;            // [BH, N] working permutation
  int* off_w;             // [BH, Gmax + 1]
  int* kv_labels;         // [BH, N]
  int* q_labels;          // [BH, N]
  int* perm_k;            // [BH, N]
  int* off_k;             // [BH, GK + 1]
  int* perm_q;            // [BH, N]
  int* off_q;             // [BH, GQ + 1]
  double* cbar;           // [BH, GK, d] raw key means
  double* qbar;           // [BH, GQ, d] raw query means
  double* mq;             // [BH, d, d] query metric s^2 Cbar^T Cbar
  void* kp;               // [BH, N, d] permuted copies of K (input dtype) and V
  void* vp;
  int* kgroup;            // [BH, N] key-group id of each permuted key position
  uint32_t* vmax;         // [BH] bit pattern of max |v| (bf16 inputs)
  int* vexp;              // [BH] power-of-two exponent k: the permuted V holds v * 2^-k in fp16
  double* mu;             // [BH, GQ, GK]
  uint64_t* ckey;         // [BH, GQ, GK] orderable descending log-probability
  double* rmass;          // [BH, GQ, GK] estimated mass shares (alpha router only, else null)
  int* mand;              // [BH, GQ] best key group per query group (-1 if empty)
  long long* thr;         // [BH, 4] selection threshold
  int* csr_ptr;           // [BH, GQ + 1]
  int* csr_col;           // [BH, GQ * GK]
  uint32_t* gmask;        // [BH, GQ, gwords] granted bitmask per query group
  long long* lg;          // [BH, GQ] granted keys per query group
  int* tiles;             // [BH, max_tiles, 4] (g, row0, nrows, 0)
  int* ntiles;            // [BH]
  int* ppos;              // [BH, M] probe positions (permuted order)
  int* pgroup;            // [BH, M] probe query group
  double* pw;             // [BH, M] probe weights
  float* ppart;           // [BH, n_pchunk, 2, M, d + 2] probe partials
  float* ode;             // [BH, M, d] exact dense probe outputs
  float* osp;             // [BH, M, d] sparse probe outputs
  float* fitW;            // [BH, d, R]
  float* fitV;            // [BH, d, R]
  float* fitb;            // [BH, d]
  int* fitrank;           // [BH]
  int Rp;                 // R rounded up to 32 (at least 32)
  bf16_t* fitpk;          // [BH, 4, Rp * d] bf16: W^T hi, W^T lo ([Rp, d]), V hi, V lo ([d, Rp])
  double* fitscratch;     // [BH, kFitScratchDoubles]
  sparsepr_head_stats* stats;  // [BH]

  size_t ws_bytes;
};

// Validate + fill the shape/settings part.  Returns SPARSEPR_OK or an error.
sparsepr_status plan_init(Plan* p, const sparsepr_config* cfg, int B, int H, int N, int d,
                          int dtype);
// Fill the io views from a tensor description (validated).
sparsepr_status plan_io(Plan* p, const sparsepr_tensors* io);
// Carve `base` (may be null to only size).  Sets ws_bytes.
void plan_carve(Plan* p, char* base);

}  // namespace sp
