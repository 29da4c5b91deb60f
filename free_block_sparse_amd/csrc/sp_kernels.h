// Kernel argument blocks and launcher declarations (internal).
#pragma once

#include "sp_plan.h"

namespace sp {

struct SampleArgs {
  View4 q;
  int N, Ms;
  int bh0;  // global index of head 0 of the launch
  unsigned long long seed;
  int* sample;
  float* mk;
};

struct EigArgs {
  const float* mk;
  float* eigval;
  float* kmap;
  int rK;
  float scale;
};

struct CoordArgs {
  View4 k;
  const float* kmap;
  int N, rK, rKpad;
  float* z32;
  bf16_t* zhi;
  bf16_t* zlo;
};

struct SplitArgs {
  View4 x;
  int N, D;
  bf16_t* hi;
  bf16_t* lo;
};

struct AssignArgs {
  View4 pts;              // hi part of the points (bf16 rows)
  const bf16_t* pts_lo;   // lo part, contiguous [BH, N, D] (fp32 points only)
  const bf16_t* yhi;      // centre images [BH, gstride, ystride]
  const bf16_t* ylo;
  const float* ybias;     // [BH, gstride]
  int ystride, gstride;
  int N, G;
  int* labels;            // [BH, N]
  int* counts;            // [BH, nchunk, gstride]
  int nchunk;
  int cpw;                // histogram chunks per workgroup (resident form; set by the launcher)
};

struct CountArgs {
  const int* in_labels;
  int* labels;
  int* counts;
  int N, G, nchunk, gstride;
};

struct ScanArgs {
  const int* counts;
  int* chunkoff;
  int* off;
  int offstride;
  int nchunk, G, gstride, N;
};

struct ScatterArgs {
  const int* labels;
  const int* chunkoff;
  int* perm;
  int* out_labels;  // nullable copy of the labels
  int N, nchunk, gstride;
};

struct UpdateArgs {
  View4 pts;            // point rows (bf16 or fp32)
  int Dp;               // point dims
  int Dimg;             // image dims (>= Dp, multiple of 16)
  const int* perm;      // [BH, N]
  const int* off;       // [BH, offstride]
  int offstride;
  const float* metric;  // [BH, Dp, Dp] or null (identity)
  double* cmean;        // [BH, gstride, cstride]
  int cstride;
  bf16_t* yhi;
  bf16_t* ylo;
  float* ybias;
  int ystride, gstride;
  int G, N;
  int init;             // centres = points at strided seed indices
  int means_only;       // only write means_out
  double* means_out;    // [BH, mo_gstride, Dp] or null; NaN for empty groups
  int mo_gstride;
};

struct QMetricArgs {
  const double* cbar;
  const int* off_k;
  int GK, d;
  float scale;
  float* mq;
};

struct GatherArgs {
  View4 k, v;
  const uint32_t* vmax;   // bf16 inputs: V is stored as fp16 scaled by 2^-vexp
  int* vexp;
  const int* perm_k;
  const int* kv_labels;
  void* kp;
  void* vp;
  int* kgroup;
  int N, d;
};

hipError_t launch_sample_metric(const Plan& p, hipStream_t s);
hipError_t launch_key_eig(const Plan& p, hipStream_t s);
hipError_t launch_key_coords(const Plan& p, hipStream_t s);
hipError_t launch_split_rows(const Plan& p, const View4& x, hipStream_t s);
hipError_t launch_assign(const Plan& p, const AssignArgs& a, int D, bool lo, hipStream_t s);
hipError_t launch_count_labels(const Plan& p, const CountArgs& a, hipStream_t s);
hipError_t launch_group_scan(const Plan& p, const ScanArgs& a, hipStream_t s);
hipError_t launch_group_scatter(const Plan& p, const ScatterArgs& a, hipStream_t s);
hipError_t launch_centre_update(const Plan& p, const UpdateArgs& a, int pts_type, hipStream_t s);
hipError_t launch_query_metric(const Plan& p, hipStream_t s);
hipError_t launch_vmax(const Plan& p, hipStream_t s);
hipError_t launch_gather(const Plan& p, hipStream_t s);

// router (k_router.hip)
hipError_t launch_route(const Plan& p, hipStream_t s);
hipError_t launch_probe_select(const Plan& p, hipStream_t s);

// attention (k_attn.hip)
hipError_t launch_probe_attention(const Plan& p, hipStream_t s);
hipError_t launch_sparse_attention(const Plan& p, bool correct, hipStream_t s);
hipError_t launch_probe_overwrite(const Plan& p, hipStream_t s);
hipError_t launch_dense_attention(const View4& q, const View4& k, const View4& v, const MutView4& o,
                                  int BH, int N, int d, int dtype, float scale, hipStream_t s);

// fit (k_fit.hip)
hipError_t launch_fit(const Plan& p, hipStream_t s);

}  // namespace sp
