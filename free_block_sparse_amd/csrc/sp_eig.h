// Symmetric eigensolver for one small matrix (n <= 128) held by one workgroup.
//
//   1. Householder reduction to tridiagonal form, A = Q T Q^T.  Each step
//      reflects the column below the diagonal onto its first entry; the
//      product with the trailing block and the rank-2 update are spread over
//      the workgroup.  The reflectors stay in the strictly lower part of A.
//   2. Implicit symmetric QR on T with Wilkinson shifts from the trailing 2x2
//      block and deflation of negligible off-diagonal entries.  One lane
//      chases the bulge of step t while the other waves apply the rotations
//      of step t-1 to the rows of Z, so the eigenvector update runs beside
//      the scalar chase.
//   3. Back-transformation of the requested columns of Z by the reflectors.
//
// When only some eigenpairs are wanted, step 2 is replaced by
//   2'. eigenvalues by multisection on Sturm counts (every eigenvalue gets a
//       group of threads that split its bracket into P+1 parts per round),
//       eigenvectors of T by one twisted factorisation each (the forward and
//       backward LDL^T pivots of T - lambda I meet at the index where the
//       twisted pivot is smallest; the vector follows from that index
//       outwards), Gram-Schmidt inside clusters of close eigenvalues, and the
//       shifted QR of step 2 as the fallback when two wanted eigenvalues are
//       too close to tell apart.
//
// Standard dense symmetric eigenvalue algorithms (reduction to tridiagonal
// form, shifted QR, Sturm-sequence bisection, inverse iteration by twisted
// factorisations); written for a single GPU workgroup.

#pragma once

#include "sp_common.h"

namespace sp {

template <typename T>
struct EigEps;
template <>
struct EigEps<float> {
  static constexpr float v = 1.1920929e-7f;
};
template <>
struct EigEps<double> {
  static constexpr double v = 2.220446049250313e-16;
};
template <typename T>
struct EigSqrtEps;
template <>
struct EigSqrtEps<float> {
  static constexpr float v = 3.4526698e-4f;
};
template <>
struct EigSqrtEps<double> {
  static constexpr double v = 1.4901161193847656e-8;
};
// smallest normal number
template <typename T>
struct EigTiny;
template <>
struct EigTiny<float> {
  static constexpr float v = 1.1754944e-38f;
};
template <>
struct EigTiny<double> {
  static constexpr double v = 2.2250738585072014e-308;
};

// 1 / sqrt(q) for q > 0: the hardware estimate, refined by one Newton step in
// fp64 (the fp32 estimate is already within about an ulp).
__device__ inline float eig_rsqrt(float q) { return __builtin_amdgcn_rsqf(q); }
__device__ inline double eig_rsqrt(double q) {
  const double y = __builtin_amdgcn_rsq(q);
  return y * (1.5 - 0.5 * q * y * y);
}

// 1 / x for the Sturm and twisted-factorisation recurrences: the hardware
// estimate (fp32, about an ulp) or the fp64 estimate refined by two Newton
// steps.  A relative error of a few ulps in a pivot is absorbed in the
// backward error of both recurrences.
__device__ inline float eig_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ inline double eig_rcp(double x) {
  double y = __builtin_amdgcn_rcp(x);
  y = fma(y, fma(-x, y, 1.0), y);
  return fma(y, fma(-x, y, 1.0), y);
}

template <typename T>
__device__ inline T eig_sum(T v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, width);
  return v;
}

template <typename T>
struct EigWork {
  T* A;
  int lda;   // n x n symmetric matrix in; reflectors out (below the subdiagonal)
  T* Z;
  int ldz;   // n x n eigenvectors out (column j belongs to dg[j])
  T* dg;     // [n + 2] eigenvalues out (unsorted)
  T* eo;     // [n + 2] off-diagonal of T
  T* tau;    // [n] reflector scales
  T* vb;     // [n] current reflector
  T* pb;     // [max(n, 2)] A22 v
  T* rot;    // [2][2n] rotation pairs (c, s), double-buffered
  int* ctl;  // [8]
};

// Reflector of the column x (x[0] and the squared norm sig of x[1..m)): the
// scalars of step k.  Returns the scale of x[1..m) in v.
template <typename T>
__device__ inline T eig_reflector(const EigWork<T>& w, int k, T x0, T sig, T diag) {
  T tau = 0, beta = x0, scale = 0;
  if (sig != T(0)) {
    const T nrm = sqrt(x0 * x0 + sig);
    beta = x0 >= T(0) ? -nrm : nrm;
    tau = (beta - x0) / beta;
    scale = T(1) / (x0 - beta);
  }
  if ((threadIdx.x & 63) == 0) {
    w.tau[k] = tau;
    w.eo[k] = beta;
    w.dg[k] = diag;
  }
  return scale;
}

// Step 1.  NT >= 256 threads; every thread calls it.  Step k: p = tau A22 v
// (all threads), then wave 0 applies the rank-2 update to the first column
// of A22 alone and forms the next step's reflector from it (in registers)
// while the other waves update the rest of A22: one workgroup barrier fewer
// per step, and the reflector's serial work runs beside the update.  The
// reflectors alternate between w.vb and w.rot (free until step 2).
template <typename T, int NT>
__device__ void eig_tridiagonalize(const EigWork<T>& w, int n) {
  static_assert(NT >= 256, "wave 0 forms the reflectors beside the other waves' update");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  T* A = w.A;
  const int lda = w.lda;
  constexpr int TPR = NT / 128;              // threads per row of the product
  constexpr int TPU = (NT - 64) / 128;       // threads per row of the update (waves 1..)
  constexpr int RGU = (NT - 64) / TPU;       // rows updated at once
  // reflector of step k from column k of A as it stands in LDS (wave 0)
  auto reflect_lds = [&](int k, T* vout) __attribute__((always_inline)) {
    const int m = n - k - 1;
    T* x = A + (k + 1) * lda + k;  // x[i * lda], i < m
    T sig = 0;
    for (int i = 1 + lane; i < m; i += 64) sig += x[i * lda] * x[i * lda];
    sig = eig_sum(sig, 64);
    const T scale = eig_reflector(w, k, x[0], sig, A[k * lda + k]);
    for (int i = lane; i < m; i += 64) {
      const T vi = i == 0 ? T(1) : x[i * lda] * scale;
      vout[i] = vi;
      x[i * lda] = vi;
    }
  };
  if (n > 2 && wv == 0) reflect_lds(0, w.vb);
  __syncthreads();
  for (int k = 0; k + 2 < n; ++k) {
    const int m = n - k - 1;
    const T* vb = (k & 1) ? w.rot : w.vb;
    T* vnext = (k & 1) ? w.vb : w.rot;
    const bool next = k + 3 < n;  // a reflector of step k + 1 follows
    const T tau = w.tau[k];
    if (tau == T(0)) {
      if (next && wv == 0) reflect_lds(k + 1, vnext);
      __syncthreads();
      continue;
    }
    {
      const int row = tid / TPR, sub = tid - row * TPR;
      T acc = 0;
      if (row < m) {
        const T* ar = A + (k + 1 + row) * lda + (k + 1);
        for (int j = sub; j < m; j += TPR) acc += ar[j] * vb[j];
      }
      acc = eig_sum(acc, TPR);
      if (row < m && sub == 0) w.pb[row] = tau * acc;
    }
    __syncthreads();
    T kk = 0;
    for (int i = lane; i < m; i += 64) kk += vb[i] * w.pb[i];
    kk = eig_sum(kk, 64) * (tau * T(0.5));
    // A22 -= v w^T + w v^T with w = p - kk v
    if (wv == 0) {
      // column 0 of A22 (rows lane and lane + 64), updated in registers
      const T v0 = vb[0], w0 = w.pb[0] - kk * v0;
      T c[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = lane + 64 * h;
        c[h] = 0;
        if (r < m) {
          const T vi = vb[r], wi = w.pb[r] - kk * vi;
          c[h] = A[(k + 1 + r) * lda + (k + 1)] - (vi * w0 + wi * v0);
        }
      }
      if (next) {
        // next column below its diagonal: x'[i] = c[i + 1], i < m - 1
        T sig = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = lane + 64 * h;
          if (r >= 2 && r < m) sig += c[h] * c[h];
        }
        sig = eig_sum(sig, 64);
        const T x0 = __shfl(c[0], 1, 64), diag = __shfl(c[0], 0, 64);
        const T scale = eig_reflector(w, k + 1, x0, sig, diag);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = lane + 64 * h;
          if (r >= 1 && r < m) {
            const T vi = r == 1 ? T(1) : c[h] * scale;
            vnext[r - 1] = vi;
            A[(k + 1 + r) * lda + (k + 1)] = vi;
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = lane + 64 * h;
          if (r < m) A[(k + 1 + r) * lda + (k + 1)] = c[h];
        }
      }
    } else {
      // rows and columns 1.. of A22 (row 0 is never read again)
      const int t = tid - 64;
      const int sub = t % TPU;
      for (int row = 1 + t / TPU; row < m; row += RGU) {
        const T vi = vb[row], wi = w.pb[row] - kk * vi;
        T* ar = A + (k + 1 + row) * lda + (k + 1);
        for (int j = 1 + sub; j < m; j += TPU) {
          const T vj = vb[j], wj = w.pb[j] - kk * vj;
          ar[j] -= vi * wj + wi * vj;
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (n >= 2) {
      w.dg[n - 2] = A[(n - 2) * lda + (n - 2)];
      w.dg[n - 1] = A[(n - 1) * lda + (n - 1)];
      w.eo[n - 2] = A[(n - 1) * lda + (n - 2)];
    } else {
      w.dg[0] = A[0];
    }
  }
  __syncthreads();
}

// Step 2.  Needs NT >= 64 + n (waves 1.. apply the rotations).
template <typename T, int NT>
__device__ void eig_tridiagonal_qr(const EigWork<T>& w, int n) {
  const int tid = threadIdx.x;
  T* Z = w.Z;
  const int ldz = w.ldz;
  for (int e = tid; e < n * n; e += NT) {
    const int i = e / n, j = e - (e / n) * n;
    Z[i * ldz + j] = i == j ? T(1) : T(0);
  }
  if (tid == 0) {
    w.ctl[0] = n - 1;  // bottom of the unreduced part
    w.ctl[1] = 0;      // steps taken
    // Gershgorin bound of T: off-diagonal entries below eps * ||T|| are at
    // the rounding level of the whole matrix and are dropped as well, so an
    // eigenvalue far below ||T|| cannot hold up convergence
    T tn = 0;
    for (int i = 0; i < n; ++i) {
      T r = fabs(w.dg[i]);
      if (i > 0) r += fabs(w.eo[i - 1]);
      if (i + 1 < n) r += fabs(w.eo[i]);
      tn = r > tn ? r : tn;
    }
    w.pb[0] = tn;
  }
  __syncthreads();
  const T eps = EigEps<T>::v;
  const T tiny = eps * w.pb[0];
  for (int t = 0;; ++t) {
    const int b = t & 1;
    if (tid < 64) {
      // Wave 0.  Negligible off-diagonal entries (relative to their diagonal
      // neighbours, or to ||T||) are found with one ballot per 64 entries:
      // the unreduced block [l, mm] ends at the last non-negligible entry
      // and starts after the negligible entry before it.
      const int lane = tid;
      T* d = w.dg;
      T* e = w.eo;
      const int mm0 = w.ctl[0];
      const int steps = w.ctl[1];
      unsigned long long neg[2] = {0ull, 0ull};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = lane + 64 * h;
        bool ng = false;
        if (i < mm0) {
          const T ei = fabs(e[i]);
          ng = ei <= eps * (fabs(d[i]) + fabs(d[i + 1])) || ei <= tiny;
          if (ng) e[i] = T(0);
        }
        neg[h] = __builtin_amdgcn_ballot_w64(ng);
      }
      // bit i of the mask (i < mm0) is set where e[i] is negligible
      int mm = 0;
      for (int h = 1; h >= 0 && mm == 0; --h) {
        const unsigned long long keep = ~neg[h] & (mm0 - 64 * h >= 64 ? ~0ull : (mm0 - 64 * h > 0 ? ((1ull << (mm0 - 64 * h)) - 1ull) : 0ull));
        if (keep) mm = 64 * h + 63 - __builtin_clzll(keep) + 1;
      }
      if (mm == 0 || steps >= 30 * n) {
        if (lane == 0) {
          w.ctl[2 + 2 * b] = -1;
          w.ctl[3 + 2 * b] = -1;
          w.ctl[0] = mm;
        }
      } else {
        int l = 0;
        for (int h = 1; h >= 0; --h) {
          const int lim = mm - 1 - 64 * h;  // entries below mm - 1 in this half
          if (lim <= 0) continue;
          const unsigned long long below = neg[h] & (lim >= 64 ? ~0ull : ((1ull << lim) - 1ull));
          if (below) {
            l = 64 * h + 63 - __builtin_clzll(below) + 1;
            break;
          }
        }
        if (lane == 0) {
          // Wilkinson shift: the eigenvalue of the trailing 2x2 block nearer d[mm]
          const T a0 = d[mm - 1], bb = e[mm - 1], c0 = d[mm];
          const T del = (a0 - c0) * T(0.5);
          const T hyp = sqrt(del * del + bb * bb);
          const T mu = c0 - bb * bb / (del + (del >= T(0) ? hyp : -hyp));
          // The chase keeps the entries it is rotating in registers: a = d[k]
          // and bq = e[k] as updated by the previous rotation; d[k+1] and
          // e[k+1] are still untouched and are read one step ahead.
          T x = d[l] - mu, z = e[l];
          T a = d[l], bq = e[l];
          T dn = d[l + 1], en = e[l + 1];
          T* rot = w.rot + b * 2 * n;
          // Branch-free body: d and e are padded by two entries, so the
          // read-ahead never leaves the arrays; the first step's "previous
          // off-diagonal" goes to a dummy slot; the block's last d and e
          // entries are written after the loop.
          T* eprev = w.pb + 1;
          for (int k = l; k < mm; ++k) {
            const T dd = dn, ek1 = en;
            dn = d[k + 2];
            en = e[k + 2];
            // rotation in the (k, k+1) plane that zeroes z against x
            const T q = x * x + z * z;
            const bool pos = q > T(0);
            const T ir = eig_rsqrt(pos ? q : T(1));
            const T c = pos ? x * ir : T(1);
            const T s = pos ? -z * ir : T(0);
            *eprev = q * ir;
            eprev = e + k;
            const T cc = c * c, ss = s * s, cs = c * s;
            const T dk = a * cc - T(2) * bq * cs + dd * ss;
            const T dk1 = a * ss + T(2) * bq * cs + dd * cc;
            const T ek = (a - dd) * cs + bq * (cc - ss);
            d[k] = dk;
            rot[2 * k] = c;
            rot[2 * k + 1] = s;
            x = ek;
            z = -s * ek1;
            bq = c * ek1;
            a = dk1;
          }
          e[mm - 1] = x;
          d[mm] = a;
          w.ctl[2 + 2 * b] = l;
          w.ctl[3 + 2 * b] = mm;
          w.ctl[1] = steps + 1;
          w.ctl[0] = mm;
        }
      }
    } else if (t > 0 && tid >= 64) {
      // rotations of the previous step, applied to the rows of Z
      const int pbuf = b ^ 1;
      const int l = w.ctl[2 + 2 * pbuf], mm = w.ctl[3 + 2 * pbuf];
      if (l >= 0) {
        const T* rot = w.rot + pbuf * 2 * n;
        for (int i = tid - 64; i < n; i += NT - 64) {
          T* zr = Z + i * ldz;
          T xk = zr[l];
          for (int k0 = l; k0 < mm; k0 += 8) {
            const int nk = mm - k0 < 8 ? mm - k0 : 8;
            T y[8], c[8], sn[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
              if (u < nk) {
                y[u] = zr[k0 + u + 1];
                c[u] = rot[2 * (k0 + u)];
                sn[u] = rot[2 * (k0 + u) + 1];
              }
#pragma unroll
            for (int u = 0; u < 8; ++u)
              if (u < nk) {
                zr[k0 + u] = c[u] * xk - sn[u] * y[u];
                xk = sn[u] * xk + c[u] * y[u];
              }
          }
          zr[mm] = xk;
        }
      }
    }
    __syncthreads();
    if (w.ctl[2 + 2 * b] < 0) break;  // converged; step t-1 was applied above
  }
}

// Number of eigenvalues of T below x (negative pivots of T - x I), with
// pivots smaller than pivmin pushed to -pivmin.  e2 holds the squared
// off-diagonal.
template <typename T>
__device__ inline int eig_sturm(const T* d, const T* e2, int n, T x, T pivmin) {
  T q = d[0] - x;
  int c = q <= pivmin;
  q = q <= pivmin ? fmin(q, -pivmin) : q;
  for (int i = 1; i < n; ++i) {
    q = (d[i] - x) - e2[i - 1] * eig_rcp(q);
    c += q <= pivmin;
    q = q <= pivmin ? fmin(q, -pivmin) : q;
  }
  return c;
}

// Step 2', eigenvalues: the nval largest eigenvalues of T (w.dg, w.eo),
// descending, into w.rot[n + r].  Leaves the squared off-diagonal in
// w.rot[0, n) and ||T|| (Gershgorin), pivmin in w.rot[2n], w.rot[2n + 1].
// Brackets shrink until they are below eps * ||T|| or two ulps of the
// eigenvalue.  Every thread calls it.
template <typename T, int NT>
__device__ void eig_bisect(const EigWork<T>& w, int n, int nval) {
  const int tid = threadIdx.x;
  T* e2 = w.rot;
  T* lam = w.rot + n;
  T* sc = w.rot + 2 * n;
  const T* d = w.dg;
  const T eps = EigEps<T>::v;
  if (tid < 64) {
    T lo = T(3.0e38), hi = T(-3.0e38), em = 0;
    for (int i = tid; i < n; i += 64) {
      const T ea = i + 1 < n ? fabs(w.eo[i]) : T(0);
      const T eb = i > 0 ? fabs(w.eo[i - 1]) : T(0);
      if (i + 1 < n) e2[i] = w.eo[i] * w.eo[i];
      lo = fmin(lo, d[i] - ea - eb);
      hi = fmax(hi, d[i] + ea + eb);
      em = fmax(em, ea * ea);
    }
    for (int o = 32; o > 0; o >>= 1) {
      lo = fmin(lo, __shfl_xor(lo, o, 64));
      hi = fmax(hi, __shfl_xor(hi, o, 64));
      em = fmax(em, __shfl_xor(em, o, 64));
    }
    if (tid == 0) {
      const T tn = fmax(fabs(lo), fabs(hi));
      const T pivmin = T(EigTiny<T>::v) * fmax(T(1), em);
      const T pad = T(2) * tn * eps * T(n) + T(2) * pivmin;
      sc[0] = tn;
      sc[1] = pivmin;
      sc[2] = lo - pad;
      sc[3] = hi + pad;
    }
  }
  __syncthreads();
  // group of P threads per eigenvalue (P a power of two, within one wave)
  int P = 64;
  while (P > 1 && P * nval > NT) P >>= 1;
  const int r = tid / P, sub = tid - (tid / P) * P;
  if (r < nval) {
    const T tn = sc[0], pivmin = sc[1];
    const T atol = eps * tn;
    const int idx = n - 1 - r;  // ascending index of the r-th largest
    T lo = sc[2], hi = sc[3];
    const int gbase = (tid & 63) - sub;
    const unsigned long long gmask = (P == 64 ? ~0ull : ((1ull << P) - 1ull)) << gbase;
    for (int it = 0; it < 256; ++it) {
      const T wd = hi - lo;
      if (!(wd > fmax(atol, T(2) * eps * fmax(fabs(lo), fabs(hi))))) break;
      const T step = wd / T(P + 1);
      const T x = lo + T(sub + 1) * step;
      const bool above = eig_sturm(d, e2, n, x, pivmin) > idx;
      const unsigned long long m = __builtin_amdgcn_ballot_w64(above) & gmask;
      const int t = m ? __builtin_ctzll(m) - gbase : P;  // first point above the eigenvalue
      const T nhi = t < P ? lo + T(t + 1) * step : hi;
      const T nlo = t > 0 ? lo + T(t) * step : lo;
      if (nhi == hi && nlo == lo) break;
      lo = nlo;
      hi = nhi;
    }
    if (sub == 0) lam[r] = (lo + hi) * T(0.5);
  }
  __syncthreads();
}

// Step 2', eigenvectors: for r < nvec, column r of Z gets the unit
// eigenvector of T for lam[r] = w.rot[n + r] (as left by eig_bisect).
// Columns [nvec, 2 nvec) of Z are scratch, so 2 nvec <= n is required.
// Returns false (all threads) when two of the wanted eigenvalues are closer
// than a few ulps of ||T|| or 2 nvec > n; Z then holds nothing useful.
template <typename T, int NT>
__device__ bool eig_twisted(const EigWork<T>& w, int n, int nvec) {
  const int tid = threadIdx.x;
  const T* e = w.eo;
  const T* d = w.dg;
  const T* lam = w.rot + n;
  const T tn = w.rot[2 * n], pivmin = w.rot[2 * n + 1];
  const T eps = EigEps<T>::v;
  T* Z = w.Z;
  const int ldz = w.ldz;
  if (2 * nvec > n) return false;
  for (int r = 1; r < nvec; ++r)
    if (lam[r - 1] - lam[r] <= T(8) * eps * tn) return false;
  if (tid < nvec) {
    const int r = tid;
    const T l = lam[r];
    T* zc = Z + r;          // l_i, later x_i
    T* uc = Z + nvec + r;   // dplus_i, later u_{i-1}
    T dp = d[0] - l;
    for (int i = 0; i + 1 < n; ++i) {
      if (fabs(dp) < pivmin) dp = dp < T(0) ? -pivmin : pivmin;
      const T li = e[i] * eig_rcp(dp);
      uc[i * ldz] = dp;
      zc[i * ldz] = li;
      dp = (d[i + 1] - l) - li * e[i];
    }
    if (fabs(dp) < pivmin) dp = dp < T(0) ? -pivmin : pivmin;
    T dm = d[n - 1] - l;
    // twisted pivot gamma_k = dplus_k + dminus_k - (d_k - lambda)
    T best = fabs(dp);
    int tw = n - 1;
    for (int i = n - 2; i >= 0; --i) {
      if (fabs(dm) < pivmin) dm = dm < T(0) ? -pivmin : pivmin;
      const T ui = e[i] * eig_rcp(dm);
      const T dpi = uc[i * ldz];
      uc[(i + 1) * ldz] = ui;
      const T g = fabs(dpi - ui * e[i]);
      if (g < best) {
        best = g;
        tw = i;
      }
      dm = (d[i] - l) - ui * e[i];
    }
    T x = T(1), ss = T(1);
    zc[tw * ldz] = x;
    for (int i = tw - 1; i >= 0; --i) {
      x = -zc[i * ldz] * x;
      zc[i * ldz] = x;
      ss += x * x;
    }
    x = T(1);
    for (int i = tw; i + 1 < n; ++i) {
      x = -uc[(i + 1) * ldz] * x;
      zc[(i + 1) * ldz] = x;
      ss += x * x;
    }
    const T inv = eig_rsqrt(ss);
    for (int i = 0; i < n; ++i) zc[i * ldz] *= inv;
  }
  __syncthreads();
  // Gram-Schmidt against the earlier members of a cluster, one wave, columns
  // in order.  A twisted-factorisation vector loses orthogonality to a
  // neighbour in proportion to eps ||T|| / gap, so clusters are gaps below
  // sqrt(eps) ||T||: the loss stays near sqrt(eps) without them.
  if (tid < 64) {
    const T ctol = T(EigSqrtEps<T>::v) * tn;
    for (int r = 1; r < nvec; ++r) {
      if (lam[r - 1] - lam[r] >= ctol) continue;
      for (int q = r - 1; q >= 0 && lam[q] - lam[r] < ctol; --q) {
        T dt = 0;
        for (int i = tid; i < n; i += 64) dt += Z[i * ldz + q] * Z[i * ldz + r];
        dt = eig_sum(dt, 64);
        for (int i = tid; i < n; i += 64) Z[i * ldz + r] -= dt * Z[i * ldz + q];
      }
      T nr = 0;
      for (int i = tid; i < n; i += 64) nr += Z[i * ldz + r] * Z[i * ldz + r];
      const T inv = eig_rsqrt(eig_sum(nr, 64));
      for (int i = tid; i < n; i += 64) Z[i * ldz + r] *= inv;
    }
  }
  __syncthreads();
  return true;
}

// Step 3 with the reflectors stored column-major and packed: column k
// (rows k+1 .. n-1) starts at refl + k (n - 1) - k (k - 1) / 2.
template <typename T, int NT, int GW>
__device__ void eig_back_transform_packed(const EigWork<T>& w, const T* refl, int n, const int* cols, int ncol) {
  const int tid = threadIdx.x, g = tid / GW, sub = tid - (tid / GW) * GW;
  constexpr int NG = NT / GW;
  for (int c = g; c < ncol; c += NG) {
    const int j = cols ? cols[c] : c;
    for (int k = n - 3; k >= 0; --k) {
      const T tau = w.tau[k];
      if (tau == T(0)) continue;
      const int m = n - k - 1;
      const T* v = refl + k * (n - 1) - (k * (k - 1)) / 2;
      T s = 0;
      for (int i = sub; i < m; i += GW) s += v[i] * w.Z[(k + 1 + i) * w.ldz + j];
      s = eig_sum(s, GW) * tau;
      for (int i = sub; i < m; i += GW) w.Z[(k + 1 + i) * w.ldz + j] -= s * v[i];
    }
  }
  __syncthreads();
}

// Step 3: Z[:, cols[c]] <- Q Z[:, cols[c]] for c < ncol (cols == nullptr: c).
// GW consecutive threads (one wave or part of one) take a column.
template <typename T, int NT, int GW>
__device__ void eig_back_transform(const EigWork<T>& w, int n, const int* cols, int ncol) {
  const int tid = threadIdx.x, g = tid / GW, sub = tid - (tid / GW) * GW;
  constexpr int NG = NT / GW;
  for (int c = g; c < ncol; c += NG) {
    const int j = cols ? cols[c] : c;
    for (int k = n - 3; k >= 0; --k) {
      const T tau = w.tau[k];
      if (tau == T(0)) continue;
      const int m = n - k - 1;
      T s = 0;
      for (int i = sub; i < m; i += GW) s += w.A[(k + 1 + i) * w.lda + k] * w.Z[(k + 1 + i) * w.ldz + j];
      s = eig_sum(s, GW) * tau;
      for (int i = sub; i < m; i += GW) w.Z[(k + 1 + i) * w.ldz + j] -= s * w.A[(k + 1 + i) * w.lda + k];
    }
  }
  __syncthreads();
}

}  // namespace sp
