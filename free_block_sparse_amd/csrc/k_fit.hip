// Probe-Fitted Residual Reconstruction: the per-call fit, fp64, one workgroup
// per (b,h).
//
// Sources (page title, section):
//   [TS] "Resumen Técnico: SparsePR ..." (gist.science) 2.B: the residual of the probe
//        rows R = O_dense - O_sparse is modelled as R ~ b + xB with x the sparse
//        output, fitted per call with ridge regularisation, and the correction is
//        confined to the span of the leading singular vectors of the probe residuals.
//   [DG] "Partition the Support, Reconstruct the Residual: ..." (ai-feeds.com digest),
//        方法/关键模块 2: the affine fit is weighted.
//   [NE] news explainer reposted from 科技行者, section "SparsePR：先把误差聚拢，再用少量
//        “抽查”去纠正": ridge regression; the 16 leading singular directions are kept.
//
// Computation (readings: unweighted uncentred SVD of R; weighted least squares
// with an unpenalised intercept; lambda relative to the mean eigenvalue of
// Xc^T D Xc unless the absolute mode is asked for):
//   Gram of R (the smaller side) -> symmetric eigensolver -> sigma, right singular
//   vectors V (r' = min(r, M, d, #{sigma > cut sigma_1}));  Y = R V;
//   weighted means xbar, ybar;  W = (Xc^T D Xc + lambda I)^-1 Xc^T D Yc, solved
//   in the M x M dual form when M <= d;  b = (ybar - xbar W) V^T.
// All matrices live in a per-(b,h) global scratch slice (L2 resident).
#include "sp_kernels.h"
#include "sp_eig.h"

namespace sp {

struct FitArgs {
  const float* ode;
  const float* osp;
  const double* pw;
  int M, d, R, Rcfg;
  int relative;
  int weighted;  // subspace from the SVD of D^(1/2) R
  double lambda, cut;
  double* scratch;  // per bh: kFitScratch doubles
  float* W;
  float* V;
  float* b;
  int* rank;
  sparsepr_head_stats* stats;
};

constexpr long long kFitScratch = kFitScratchDoubles;

__device__ inline void block_sync() { __syncthreads(); }

// Parallel cyclic Jacobi on a symmetric n x n matrix (n even) with eigenvector
// accumulation.  All threads of the block call it.
__device__ void jacobi_sym_f64(double* A, double* V, int n, double* rcs, int* rpq, int* stop, double* red) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int hp = n / 2;
  for (int e = tid; e < n * n; e += nt) V[e] = (e / n == e % n) ? 1.0 : 0.0;
  block_sync();
  for (int sweep = 0; sweep < 30; ++sweep) {
    double off = 0.0, tot = 0.0;
    for (int e = tid; e < n * n; e += nt) {
      const double x = A[e];
      tot += x * x;
      if (e / n != e % n) off += x * x;
    }
    off = wave_sum_d(off);
    tot = wave_sum_d(tot);
    if ((tid & 63) == 0) {
      red[2 * (tid >> 6)] = off;
      red[2 * (tid >> 6) + 1] = tot;
    }
    block_sync();
    if (tid == 0) {
      double o = 0.0, t = 0.0;
      for (int w = 0; w < nt / 64; ++w) {
        o += red[2 * w];
        t += red[2 * w + 1];
      }
      *stop = !(o > 1e-24 * t);
    }
    block_sync();
    if (*stop) break;
    for (int r = 0; r < n - 1; ++r) {
      for (int k = tid; k < hp; k += nt) {
        const int a0 = k, b0 = n - 1 - k;
        const int pa = a0 == 0 ? 0 : ((a0 - 1 + r) % (n - 1)) + 1;
        const int pb = b0 == 0 ? 0 : ((b0 - 1 + r) % (n - 1)) + 1;
        const int p = pa < pb ? pa : pb, q = pa < pb ? pb : pa;
        const double app = A[p * n + p], aqq = A[q * n + q], apq = A[p * n + q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double th = (aqq - app) / (2.0 * apq);
          double t;
          if (fabs(th) > 1e150) t = 0.5 / th;
          else t = (th >= 0.0 ? 1.0 : -1.0) / (fabs(th) + sqrt(1.0 + th * th));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        rcs[2 * k] = c;
        rcs[2 * k + 1] = s;
        rpq[2 * k] = p;
        rpq[2 * k + 1] = q;
      }
      block_sync();
      for (int blk = tid; blk < hp * hp; blk += nt) {
        const int ia = blk / hp, ib = blk - (blk / hp) * hp;
        const int pa = rpq[2 * ia], qa = rpq[2 * ia + 1], pb = rpq[2 * ib], qb = rpq[2 * ib + 1];
        const double ca = rcs[2 * ia], sa = rcs[2 * ia + 1], cb = rcs[2 * ib], sb = rcs[2 * ib + 1];
        const double x00 = A[pa * n + pb], x01 = A[pa * n + qb];
        const double x10 = A[qa * n + pb], x11 = A[qa * n + qb];
        const double t00 = ca * x00 - sa * x10, t01 = ca * x01 - sa * x11;
        const double t10 = sa * x00 + ca * x10, t11 = sa * x01 + ca * x11;
        A[pa * n + pb] = cb * t00 - sb * t01;
        A[pa * n + qb] = sb * t00 + cb * t01;
        A[qa * n + pb] = cb * t10 - sb * t11;
        A[qa * n + qb] = sb * t10 + cb * t11;
      }
      for (int task = tid; task < n * hp; task += nt) {
        const int i = task / hp, ib = task - (task / hp) * hp;
        const int pb = rpq[2 * ib], qb = rpq[2 * ib + 1];
        const double cb = rcs[2 * ib], sb = rcs[2 * ib + 1];
        const double v1 = V[i * n + pb], v2 = V[i * n + qb];
        V[i * n + pb] = cb * v1 - sb * v2;
        V[i * n + qb] = sb * v1 + cb * v2;
      }
      block_sync();
    }
  }
}

// Sum over the workgroup (every thread gets the result); red holds one
// double per wave.
__device__ double block_sum_d(double v, double* red) {
  const int tid = threadIdx.x, nw = blockDim.x >> 6;
  v = wave_sum_d(v);
  block_sync();
  if ((tid & 63) == 0) red[tid >> 6] = v;
  block_sync();
  double t = 0.0;
  for (int w = 0; w < nw; ++w) t += red[w];
  return t;
}

constexpr int kFitThreads = 1024;

// fp64 dot product of two strided sequences with four accumulators: in these
// small products the chain of dependent additions, not the arithmetic, sets
// the time.
template <typename TA, typename TB>
__device__ inline double dot4(const TA* x, int sx, const TB* y, int sy, int n) {
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  int k = 0;
  for (; k + 3 < n; k += 4) {
    a0 += (double)x[k * sx] * (double)y[k * sy];
    a1 += (double)x[(k + 1) * sx] * (double)y[(k + 1) * sy];
    a2 += (double)x[(k + 2) * sx] * (double)y[(k + 2) * sy];
    a3 += (double)x[(k + 3) * sx] * (double)y[(k + 3) * sy];
  }
  for (; k < n; ++k) a0 += (double)x[k * sx] * (double)y[k * sy];
  return (a0 + a1) + (a2 + a3);
}

// In-place Cholesky (lower) of an SPD n x n matrix (n <= 128, row stride
// ld, in LDS) and the solve L L^T Y = Y for the nc columns of Y (row stride
// ldy).  Wave 0 factors column by column, lanes owning rows ln and ln + 64
// (left-looking dot products); then every wave solves columns of Y, two at
// a time, lanes as rows.  No workgroup barrier inside either; all threads
// call it.  Returns false (all threads) on a non-positive pivot, with Y
// untouched.
__device__ bool chol_factor_solve128(double* K, int n, int ld, double* Y, int nc, int ldy, int* bad) {
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63, nt = blockDim.x;
  const int r0 = ln, r1 = ln + 64;
  if (n > 128) return false;  // two rows per lane at most (the callers' orders are <= 128)
  if (wv == 0) {
    bool badl = false;
    for (int k = 0; k < n; ++k) {
      double a0 = 0.0, a1 = 0.0;
      if (r0 < n && r0 >= k) a0 = K[r0 * ld + k] - dot4(K + r0 * ld, 1, K + k * ld, 1, k);
      if (r1 < n && r1 >= k) a1 = K[r1 * ld + k] - dot4(K + r1 * ld, 1, K + k * ld, 1, k);
      const double piv = __shfl(k < 64 ? a0 : a1, k & 63, 64);
      badl |= !(piv > 0.0);
      const double lkk = sqrt(piv > 0.0 ? piv : 1.0);
      // a wave's LDS accesses complete in order, and the next column's reads
      // may alias these writes, so they are not moved above them
      if (r0 == k) K[k * ld + k] = lkk;
      else if (r0 > k && r0 < n) K[r0 * ld + k] = a0 / lkk;
      if (r1 == k) K[k * ld + k] = lkk;
      else if (r1 > k && r1 < n) K[r1 * ld + k] = a1 / lkk;
    }
    if (ln == 0) *bad = badl ? 1 : 0;
  }
  block_sync();
  if (*bad) return false;
  const double dv0 = r0 < n ? 1.0 / K[r0 * ld + r0] : 0.0;
  const double dv1 = r1 < n ? 1.0 / K[r1 * ld + r1] : 0.0;
  const int nw = nt >> 6;
  for (int c0 = wv; c0 < nc; c0 += 2 * nw) {
    const int c1 = c0 + nw;
    const bool two = c1 < nc;
    // y[q][h]: column c_q, row ln + 64 h
    double y00 = r0 < n ? Y[r0 * ldy + c0] : 0.0, y01 = r1 < n ? Y[r1 * ldy + c0] : 0.0;
    double y10 = (two && r0 < n) ? Y[r0 * ldy + c1] : 0.0, y11 = (two && r1 < n) ? Y[r1 * ldy + c1] : 0.0;
    for (int j = 0; j < n; ++j) {  // L z = y
      const bool hi = j >= 64;
      const double z0 = __shfl(hi ? y01 * dv1 : y00 * dv0, j & 63, 64);
      const double z1 = __shfl(hi ? y11 * dv1 : y10 * dv0, j & 63, 64);
      const double l0 = (r0 > j && r0 < n) ? K[r0 * ld + j] : 0.0;
      const double l1 = (r1 > j && r1 < n) ? K[r1 * ld + j] : 0.0;
      y00 = r0 == j ? z0 : y00 - l0 * z0;
      y10 = r0 == j ? z1 : y10 - l0 * z1;
      y01 = r1 == j ? z0 : y01 - l1 * z0;
      y11 = r1 == j ? z1 : y11 - l1 * z1;
    }
    for (int i = n - 1; i >= 0; --i) {  // L^T x = z
      const bool hi = i >= 64;
      const double x0 = __shfl(hi ? y01 * dv1 : y00 * dv0, i & 63, 64);
      const double x1 = __shfl(hi ? y11 * dv1 : y10 * dv0, i & 63, 64);
      const double l0 = r0 < i ? K[i * ld + r0] : 0.0;
      const double l1 = r1 < i ? K[i * ld + r1] : 0.0;
      y00 = r0 == i ? x0 : y00 - l0 * x0;
      y10 = r0 == i ? x1 : y10 - l0 * x1;
      y01 = r1 == i ? x0 : y01 - l1 * x0;
      y11 = r1 == i ? x1 : y11 - l1 * x1;
    }
    if (r0 < n) {
      Y[r0 * ldy + c0] = y00;
      if (two) Y[r0 * ldy + c1] = y10;
    }
    if (r1 < n) {
      Y[r1 * ldy + c0] = y01;
      if (two) Y[r1 * ldy + c1] = y11;
    }
  }
  block_sync();
  return true;
}

// MODE 1 (ALL_LDS): M <= 64 probes and r <= 32, so every matrix lives in
// LDS; the pointers below are then known to be LDS pointers and compile to
// LDS accesses instead of generic ones.  MODE 0: M <= 64 with r > 32 (Y in
// the global slice).  MODE 2 (BIG): more than 64 probes; the Gram of order
// min(M, d) <= 128, and later the ridge system, sit in one LDS block so the
// eigensolver and the Cholesky factorisation run on LDS (in the global slice
// they took 50x longer); R, X and the eigenvectors use the global slice.
template <int MODE>
__global__ __launch_bounds__(1024) void k_fit(FitArgs a) {
  constexpr bool ALL_LDS = MODE == 1;
  constexpr bool BIG = MODE == 2;
  // LDS path for M <= 64: R and X as fp32 rows of stride d + 1, the Gram /
  // ridge system and eigenvectors as fp64 rows of stride 65 (odd strides keep
  // column walks on distinct banks).  Larger probe budgets use the
  // per-(b,h) global scratch slice with unpadded strides, except the BIG
  // block above.
  constexpr int SM = 64, SLX = 129, SLG = SM + 1;
  constexpr int EN = BIG ? 128 : 64;  // largest order of the eigen problem
  __shared__ float Rl[BIG ? 1 : SM * SLX];
  __shared__ float Xl[BIG ? 1 : SM * SLX];
  __shared__ double Gl[BIG ? 1 : SM * SLG];
  __shared__ double Ul[BIG ? 1 : SM * SLG];
  __shared__ double Gb[BIG ? 128 * 129 : 1];  // BIG: the Gram, later the ridge system
  __shared__ double rcs[2 * 64];
  __shared__ int rpq[2 * 64];
  __shared__ double red[32];
  __shared__ int stop, bad;
  __shared__ double sig_s[kMaxProbe + 1];
  __shared__ int idx_s[kMaxProbe + 1];
  __shared__ int rk_s;
  __shared__ double xb[128];
  __shared__ double yb[64];
  __shared__ double bp[64];
  __shared__ double edg[128 + 2], eeo[EN + 2], etau[EN], evb[EN], epb[EN], erot[4 * EN];
  __shared__ double Ycl[BIG ? 1 : SM * 32];  // Y (M x rk) when M <= 64 and rk <= 32
  __shared__ double wl[kMaxProbe];  // the probe weights
  __shared__ int ectl[8];
  const int bh = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int M = a.M, d = a.d, Rmax = a.R;  // Rmax: column stride of the W and V outputs
  double* S = a.scratch + (long long)bh * kFitScratch;
  const bool small = M <= d;
  const int n = small ? M : d;
  const int ne = n + (n & 1);
  const bool lds = ALL_LDS || (!BIG && M <= SM);
  const int ldx = lds ? SLX : d;
  const bool glds = ALL_LDS || (!BIG && ne <= SM);
  // BIG (more than 64 probes): the Gram / ridge block (order ne <= 128) in LDS
  // with an odd stride, the eigenvectors in the global slice
  const int ldg = BIG ? ne + 1 : (glds ? SLG : ne);
  const int ldu = BIG ? ne : ldg;
  float* Rf = lds ? Rl : reinterpret_cast<float*>(S);                        // M x d
  float* Xf = lds ? Xl : reinterpret_cast<float*>(S) + 256 * 128;            // M x d (centred below)
  double* G = BIG ? Gb : (glds ? Gl : S + 256 * 128);                      // ne x ne, later the ridge system
  double* U = glds ? Ul : S + 256 * 128 + 128 * 128;                         // ne x ne
  double* Vr = S + 256 * 128 + 2 * 128 * 128;                                // d x Rmax
  double* Wm = Vr + 128 * 64;                                                // d x rk (also the primal rhs)
  double* Yc = (ALL_LDS || (lds && a.Rcfg <= 32)) ? Ycl : Wm + 128 * 64;    // M x rk
  double* Kp = BIG ? Gb : Wm + 128 * 64 + 256 * 64;                          // primal system d x d (M > d)
  const float* ode = a.ode + (long long)bh * M * d;
  const float* osp = a.osp + (long long)bh * M * d;
  // BIG: the products over R or Xc read an LDS copy of the M x d matrix
  // (stride d + 1) held in the Gram block while that block is free; the
  // symmetric results go through the global block Gt into the Gram block.
  // (In the global slice, with one row per lane, these loops took most of
  // the fit.)
  double* const Gt = S + 256 * 128;
  float* const Ls = reinterpret_cast<float*>(Gb);
  const int lsd = d + 1;
  auto stage_rows = [&](const float* src) __attribute__((always_inline)) {
    block_sync();  // the Gram block's previous contents are no longer read
    for (int e = tid; e < M * d; e += nt) {
      const int mm = e / d, dm = e - (e / d) * d;
      Ls[mm * lsd + dm] = src[mm * ldx + dm];
    }
    block_sync();
  };
  auto gt_to_lds = [&](double* dst, int nn, int ldd) __attribute__((always_inline)) {
    block_sync();  // every product read the staged rows
    for (int e = tid; e < nn * nn; e += nt) {
      const int i = e / nn, j = e - (e / nn) * nn;
      dst[i * ldd + j] = Gt[e];
    }
    block_sync();
  };
  const double* wg = a.pw + (long long)bh * M;
  const double* w = wl;

  // staged eight elements per thread at a time, the loads in flight together
  for (int e0 = 0; e0 < M * d; e0 += 8 * nt) {
    float od[8], op[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + tid + u * nt;
      od[u] = e < M * d ? ode[e] : 0.f;
      op[u] = e < M * d ? osp[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + tid + u * nt;
      if (e < M * d) {
        const int mm = e / d, dm = e - (e / d) * d;
        Rf[mm * ldx + dm] = od[u] - op[u];
        Xf[mm * ldx + dm] = op[u];
      }
    }
  }
  double wpart = 0.0;
  for (int i = tid; i < M; i += nt) {
    const double wi = wg[i];
    wpart += wi;
    wl[i] = wi;
  }
  const double ws = block_sum_d(wpart, red);
  for (int dm = tid; dm < d; dm += nt) {
    xb[dm] = dot4(w, 1, Xf + dm, ldx, M) / ws;
  }
  block_sync();
  // Gram of the smaller side of D^(1/2) R (D = I unless the subspace is weighted):
  // sqrt(w_i w_j) r_i . r_j, or sum_m w_m r_m r_m^T
  {
    const float* Rg = BIG ? Ls : Rf;
    const int ldr = BIG ? lsd : ldx;
    if (BIG) stage_rows(Rf);
    for (int e = tid; e < ne * ne; e += nt) {
      const int i = e / ne, j = e - (e / ne) * ne;
      double acc = 0.0;
      if (i < n && j < n) {
        if (small) {
          acc = dot4(Rg + i * ldr, 1, Rg + j * ldr, 1, d);
          if (a.weighted) acc *= sqrt(w[i]) * sqrt(w[j]);
        } else if (a.weighted) {
          for (int mm = 0; mm < M; ++mm) acc += w[mm] * ((double)Rg[mm * ldr + i] * (double)Rg[mm * ldr + j]);
        } else {
          for (int mm = 0; mm < M; ++mm) acc += (double)Rg[mm * ldr + i] * (double)Rg[mm * ldr + j];
        }
      }
      if (BIG) Gt[e] = acc;
      else G[i * ldg + j] = acc;
    }
    if (BIG) gt_to_lds(G, ne, ldg);
    else block_sync();
  }
  bool fast = false;  // leading eigenpairs by multisection + twisted factorisations
  if (glds || BIG) {
    // Householder tridiagonalisation, then the leading eigenvalues by
    // multisection (the rank follows from them) and their vectors by twisted
    // factorisations; shifted QR on all of them when two leading eigenvalues
    // cannot be told apart.  Everything in LDS.
    const EigWork<double> ew{G, ldg, U, ldu, edg, eeo, etau, evb, epb, erot, ectl};
    eig_tridiagonalize<double, kFitThreads>(ew, ne);
    int nval = a.Rcfg > 4 ? a.Rcfg : 4;
    if (nval > ne) nval = ne;
    eig_bisect<double, kFitThreads>(ew, ne, nval);
    if (tid == 0) {
      const double* lam = erot + ne;
      for (int r = 0; r < nval; ++r) {
        sig_s[r] = sqrt(lam[r] > 0.0 ? lam[r] : 0.0);
        idx_s[r] = r;
      }
      const double s1 = sig_s[0];
      int cnt = 0;
      if (s1 > 0.0 && s1 < INFINITY)
        for (int r = 0; r < nval && r < n; ++r) cnt += sig_s[r] > a.cut * s1;
      int rk = a.Rcfg;
      if (M < rk) rk = M;
      if (d < rk) rk = d;
      if (cnt < rk) rk = cnt;
      rk_s = rk;
    }
    block_sync();
    if (BIG && rk_s <= 32) {
      // As in the key eigensolve: the reflectors packed column-major behind
      // an LDS block for the leading vectors (2 rk + 1 columns, the twisted
      // factorisations' scratch included), so that the vectors are formed
      // and transformed in LDS rather than in the global slice.  Element
      // (r, c), r > c, of the reflectors goes to c (ne - 1) - c (c - 1) / 2 + r - c - 1.
      constexpr int PERF = 128 * 128 / kFitThreads;
      const int zl = 2 * rk_s + 1;
      double* const Zl = Gb;
      double* const Rp = Gb + ne * (2 * 32 + 1);
      double t[PERF];
#pragma unroll
      for (int u = 0; u < PERF; ++u) {
        const int e = tid + kFitThreads * u, r = e / ne, c = e - (e / ne) * ne;
        t[u] = (e < ne * ne && r > c) ? G[r * ldg + c] : 0.0;
      }
      block_sync();
#pragma unroll
      for (int u = 0; u < PERF; ++u) {
        const int e = tid + kFitThreads * u, r = e / ne, c = e - (e / ne) * ne;
        if (e < ne * ne && r > c) Rp[c * (ne - 1) - (c * (c - 1)) / 2 + r - c - 1] = t[u];
      }
      block_sync();
      const EigWork<double> wz{nullptr, 0, Zl, zl, edg, eeo, etau, evb, epb, erot, ectl};
      fast = eig_twisted<double, kFitThreads>(wz, ne, rk_s);
      if (fast) {
        eig_back_transform_packed<double, kFitThreads, 32>(wz, Rp, ne, nullptr, rk_s);
        // the leading vectors to the global slice, where the products below read them
        for (int e = tid; e < ne * rk_s; e += nt) {
          const int i = e / rk_s, c = e - (e / rk_s) * rk_s;
          U[i * ldu + c] = Zl[i * zl + c];
        }
        block_sync();
      } else {
        const EigWork<double> wu{nullptr, 0, U, ldu, edg, eeo, etau, evb, epb, erot, ectl};
        eig_tridiagonal_qr<double, kFitThreads>(wu, ne);
        eig_back_transform_packed<double, kFitThreads, 32>(wu, Rp, ne, nullptr, ne);
      }
    } else {
      fast = eig_twisted<double, kFitThreads>(ew, ne, rk_s);
      if (fast) {
        eig_back_transform<double, kFitThreads, 16>(ew, ne, nullptr, rk_s);
      } else {
        eig_tridiagonal_qr<double, kFitThreads>(ew, ne);
        eig_back_transform<double, kFitThreads, 16>(ew, ne, nullptr, ne);
      }
    }
  } else {
    jacobi_sym_f64(G, U, ne, rcs, rpq, &stop, red);
    for (int i = tid; i < ne; i += nt) edg[i] = G[i * ne + i];
    block_sync();
  }
  if (!fast) {
    // eigenvalues, descending with ties by index
    for (int i = tid; i < ne; i += nt) {
      const double li = edg[i];
      int r = 0;
      for (int j = 0; j < ne; ++j) {
        const double lj = edg[j];
        r += (lj > li) || (lj == li && j < i);
      }
      sig_s[r] = sqrt(li > 0.0 ? li : 0.0);
      idx_s[r] = i;
    }
    block_sync();
    if (tid == 0) {
      const double s1 = sig_s[0];
      int cnt = 0;
      if (s1 > 0.0 && s1 < INFINITY)
        for (int i = 0; i < n; ++i) cnt += sig_s[i] > a.cut * s1;
      int rk = a.Rcfg;
      if (M < rk) rk = M;
      if (d < rk) rk = d;
      if (cnt < rk) rk = cnt;
      rk_s = rk;
    }
  }
  block_sync();
  int rk = rk_s;
  const float* Rv = BIG ? Ls : Rf;
  const int ldv = BIG ? lsd : ldx;
  if (BIG) stage_rows(Rf);  // the eigen work in the Gram block is done
  // right singular vectors
  for (int e = tid; e < d * rk; e += nt) {
    const int dm = e / rk, k = e - (e / rk) * rk;
    const int ci = idx_s[k];
    double v;
    if (small && a.weighted) {
      // V = (D^(1/2) R)^T U / sigma
      double acc = 0.0;
      for (int mm = 0; mm < M; ++mm) acc += (double)Rv[mm * ldv + dm] * (sqrt(w[mm]) * U[mm * ldu + ci]);
      v = acc / sig_s[k];
    } else if (small) {
      v = dot4(Rv + dm, ldv, U + ci, ldu, M) / sig_s[k];
    } else {
      v = U[dm * ldu + ci];
    }
    Vr[dm * Rmax + k] = v;
  }
  block_sync();
  // Y = R Vr (M x rk); in the dual form R Vr = R R^T U_r / sigma = U_r sigma
  for (int e = tid; e < M * rk; e += nt) {
    const int mm = e / rk, k = e - (e / rk) * rk;
    double acc = 0.0;
    if (small && !a.weighted) {
      acc = U[mm * ldu + idx_s[k]] * sig_s[k];
    } else {
      for (int dm = 0; dm < d; ++dm) acc += (double)Rv[mm * ldv + dm] * Vr[dm * Rmax + k];
    }
    Yc[mm * rk + k] = acc;
  }
  block_sync();
  for (int k = tid; k < rk; k += nt) {
    double acc = 0.0;
    for (int mm = 0; mm < M; ++mm) acc += w[mm] * Yc[mm * rk + k];
    yb[k] = acc / ws;
  }
  for (int e = tid; e < M * d; e += nt) {
    const int mm = e / d, dm = e - (e / d) * d;
    Xf[mm * ldx + dm] = (float)((double)Xf[mm * ldx + dm] - xb[dm]);
  }
  block_sync();
  for (int e = tid; e < M * rk; e += nt) Yc[e] -= yb[e % rk];
  // ridge strength (relative: lambda times the mean eigenvalue of Xc^T D Xc)
  double lam = a.lambda;
  if (a.relative) {
    double tpart = 0.0;
    for (int e = tid; e < M * d; e += nt) {
      const int mm = e / d, dm = e - (e / d) * d;
      const double t = (double)Xf[mm * ldx + dm];
      tpart += w[mm] * t * t;
    }
    lam *= block_sum_d(tpart, red) / (double)d;
  }
  block_sync();
  bool ok = rk > 0;
  if (rk > 0) {
    if (small) {
      // dual: K = D^1/2 Xc Xc^T D^1/2 + lambda I  (M x M) in the Gram buffer, rhs = D^1/2 Yc
      double* K = G;
      const float* Xk = BIG ? Ls : Xf;
      const int ldk = BIG ? lsd : ldx;
      if (BIG) stage_rows(Xf);
      for (int e = tid; e < M * M; e += nt) {
        const int i = e / M, j = e - (e / M) * M;
        const double acc = dot4(Xk + i * ldk, 1, Xk + j * ldk, 1, d);
        const double kij = sqrt(w[i] * w[j]) * acc + (i == j ? lam : 0.0);
        if (BIG) Gt[e] = kij;
        else K[i * ldg + j] = kij;
      }
      for (int e = tid; e < M * rk; e += nt) Yc[e] *= sqrt(w[e / rk]);
      if (BIG) gt_to_lds(K, M, ldg);
      else block_sync();
      if (M <= 64) {
        // one wave factors K column by column (lane i owns row i of L, left-
        // looking dot products), then every wave solves its columns of Y with
        // lanes as rows: no workgroup barrier inside either
        const int wv = tid >> 6, ln = tid & 63;
        if (wv == 0) {
          bool badl = false;
          for (int k = 0; k < M; ++k) {
            const int rl = ln < M ? ln : k;  // idle lanes shadow the pivot row
            const double acc = K[rl * ldg + k] - dot4(K + rl * ldg, 1, K + k * ldg, 1, k);
            const double piv = __shfl(acc, k, 64);
            badl |= !(piv > 0.0);
            const double lkk = sqrt(piv > 0.0 ? piv : 1.0);
            // a wave's LDS accesses complete in order, and the next column's
            // reads may alias these writes, so they are not moved above them
            if (ln == k) K[k * ldg + k] = lkk;
            else if (ln > k && ln < M) K[ln * ldg + k] = acc / lkk;
          }
          if (ln == 0) bad = badl ? 1 : 0;
        }
        block_sync();
        ok = bad == 0;
        if (ok) {
          const double dinv = ln < M ? 1.0 / K[ln * ldg + ln] : 0.0;
          // two right-hand sides per pass: independent chains
          const int nw = nt >> 6;
          for (int c0 = wv; c0 < rk; c0 += 2 * nw) {
            const int c1 = c0 + nw;
            const bool two = c1 < rk;
            double y0 = ln < M ? Yc[ln * rk + c0] : 0.0;
            double y1 = (two && ln < M) ? Yc[ln * rk + c1] : 0.0;
            for (int j = 0; j < M; ++j) {  // L z = y
              const double lj = (ln > j && ln < M) ? K[ln * ldg + j] : 0.0;
              const double z0 = __shfl(y0 * dinv, j, 64);
              const double z1 = __shfl(y1 * dinv, j, 64);
              y0 = ln == j ? z0 : y0 - lj * z0;
              y1 = ln == j ? z1 : y1 - lj * z1;
            }
            for (int i = M - 1; i >= 0; --i) {  // L^T x = z
              const double li = ln < i ? K[i * ldg + ln] : 0.0;
              const double x0 = __shfl(y0 * dinv, i, 64);
              const double x1 = __shfl(y1 * dinv, i, 64);
              y0 = ln == i ? x0 : y0 - li * x0;
              y1 = ln == i ? x1 : y1 - li * x1;
            }
            if (ln < M) {
              Yc[ln * rk + c0] = y0;
              if (two) Yc[ln * rk + c1] = y1;
            }
          }
        }
        block_sync();
      } else {
        ok = chol_factor_solve128(K, M, ldg, Yc, rk, rk, &bad);
      }
      if (ok) {
        // W = Xc^T D^1/2 Y
        for (int e = tid; e < M * rk; e += nt) Yc[e] *= sqrt(w[e / rk]);
        const float* Xw = BIG ? Ls : Xf;
        const int ldw = BIG ? lsd : ldx;
        if (BIG) stage_rows(Xf);  // the factor is no longer read
        else block_sync();
        for (int e = tid; e < d * rk; e += nt) {
          const int dm = e / rk, k = e - (e / rk) * rk;
          Wm[dm * rk + k] = dot4(Xw + dm, ldw, Yc + k, rk, M);
        }
      }
    } else {
      // primal: K = Xc^T D Xc + lambda I (d x d), rhs = Xc^T D Yc (d x rk)
      double* K = Kp;
      const float* Xp = BIG ? Ls : Xf;
      const int ldp = BIG ? lsd : ldx;
      if (BIG) stage_rows(Xf);
      for (int e = tid; e < d * d; e += nt) {
        const int i = e / d, j = e - (e / d) * d;
        double acc = 0.0;
        for (int mm = 0; mm < M; ++mm) acc += w[mm] * (double)Xp[mm * ldp + i] * (double)Xp[mm * ldp + j];
        if (BIG) Gt[e] = acc + (i == j ? lam : 0.0);
        else K[e] = acc + (i == j ? lam : 0.0);
      }
      for (int e = tid; e < d * rk; e += nt) {
        const int i = e / rk, k = e - (e / rk) * rk;
        double acc = 0.0;
        for (int mm = 0; mm < M; ++mm) acc += w[mm] * (double)Xp[mm * ldp + i] * Yc[mm * rk + k];
        Wm[e] = acc;
      }
      if (BIG) gt_to_lds(K, d, d);
      else block_sync();
      ok = chol_factor_solve128(K, d, d, Wm, rk, rk, &bad);
    }
    block_sync();
  }
  const bool fallback = rk > 0 && !ok;
  if (!ok) rk = 0;
  // outputs: W (d x R) and V (d x R) zero beyond rk, b = (ybar - xbar W) V^T
  for (int k = tid; k < rk; k += nt) {
    double acc = yb[k];
    for (int dm = 0; dm < d; ++dm) acc -= xb[dm] * Wm[dm * rk + k];
    bp[k] = acc;
  }
  block_sync();
  float* Wo = a.W + (long long)bh * d * Rmax;
  float* Vo = a.V + (long long)bh * d * Rmax;
  for (int e = tid; e < d * Rmax; e += nt) {
    const int dm = e / Rmax, k = e - (e / Rmax) * Rmax;
    Wo[e] = k < rk ? (float)Wm[dm * rk + k] : 0.f;
    Vo[e] = k < rk ? (float)Vr[dm * Rmax + k] : 0.f;
  }
  for (int dm = tid; dm < d; dm += nt) {
    double acc = 0.0;
    for (int k = 0; k < rk; ++k) acc += bp[k] * Vr[dm * Rmax + k];
    a.b[(long long)bh * d + dm] = (float)acc;
  }
  if (tid == 0) {
    a.rank[bh] = rk;
    if (a.stats) {
      a.stats[bh].residual_rank = rk;
      a.stats[bh].fit_fallback = fallback ? 1 : 0;
      for (int i = 0; i < 4; ++i) a.stats[bh].sigma[i] = i < n ? sig_s[i] : 0.0;
    }
  }
}

hipError_t launch_fit(const Plan& p, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  FitArgs a;
  a.ode = p.ode;
  a.osp = p.osp;
  a.pw = p.pw;
  a.M = p.M;
  a.d = p.d;
  a.R = p.R > 0 ? p.R : 1;
  a.Rcfg = p.Rfit;
  a.relative = p.ridge_mode == SPARSEPR_RIDGE_RELATIVE ? 1 : 0;
  a.weighted = p.svd_weighted;
  a.lambda = (double)p.lambda;
  a.cut = (double)p.rank_cut;
  a.scratch = p.fitscratch;
  a.W = p.fitW;
  a.V = p.fitV;
  a.b = p.fitb;
  a.rank = p.fitrank;
  a.stats = p.stats;
  if (a.M <= 64 && a.Rcfg <= 32) hipLaunchKernelGGL(k_fit<1>, dim3(p.BH), dim3(kFitThreads), 0, s, a);
  else if (a.M <= 64) hipLaunchKernelGGL(k_fit<0>, dim3(p.BH), dim3(kFitThreads), 0, s, a);
  else hipLaunchKernelGGL(k_fit<2>, dim3(p.BH), dim3(kFitThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sp
