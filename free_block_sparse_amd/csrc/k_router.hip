// Router and probe selection kernels for gfx950.
//
// Sources (page title, section):
//   [NE] news explainer reposted from 科技行者, section "稀疏执行怎么落地，误差怎么算才公平":
//        (query-group, key-group) cells are chosen under a budget counted in true
//        pairs, the product of the two groups' token counts; rho_route is the
//        selected fraction of the Q x K matrix; the executed density also counts
//        the exact probe rows.
//   [TS] "Resumen Técnico: SparsePR ..." (gist.science) 2.C: rho_exec includes routed
//        sparse cells and exact probe rows.
//   [NE] section "SparsePR：先把误差聚拢，再用少量“抽查”去纠正": probes are picked evenly
//        from every query group (query-group-stratified), 64 rows per head.
//
// Budget rule (a reading; the pages give no formula): mu_gh = s qbar_g . cbar_h is the
// logit of the mean query of group g against the mean key of group h;
// key_gh = mu_gh - log sum_h' n_h' exp(mu_gh') estimates the attention
// probability of one key of h for a query of g.  Every non-empty query group
// first gets its best cell; the other cells are taken in order (key desc,
// g asc, h asc) as the longest prefix that fits the budget.  mu is a
// sequential fp64 dot product without fused multiply-add, so the selection is
// reproducible bit for bit.
#include "sp_kernels.h"

namespace sp {

struct RouteArgs {
  const double* qbar;  // [BH, GQ, d]
  const double* cbar;  // [BH, GK, d]
  const int* off_q;    // [BH, GQ + 1]
  const int* off_k;    // [BH, GK + 1]
  int GQ, GK, d, N, M;
  double s;
  long long budget;
  int dense_route;
  double alpha;     // target retained mass (alpha router)
  double* mu;
  uint64_t* ckey;
  double* rmass;    // [BH, GQ, GK] estimated mass shares n_h exp(key_gh) (alpha router), else null
  int* mand;
  long long* thr;
  int* csr_ptr;
  int* csr_col;
  uint32_t* gmask;
  int gwords;
  long long* lg;
  int* tiles;
  int* ntiles;
  int max_tiles;
  sparsepr_head_stats* stats;
  const int* fcount;  // [BH, 4T] k-means flag counts (null: partition given)
  int T;
};

constexpr uint64_t kExcluded = ~0ull;

// ---------------------------------------------------------------- mu
__global__ __launch_bounds__(256) void k_route_mu(RouteArgs a) {
  constexpr int GB = 16;
  __shared__ double sq[GB][128];
  const int bh = blockIdx.y, g0 = blockIdx.x * GB, tid = threadIdx.x, d = a.d;
  const int* offq = a.off_q + (long long)bh * (a.GQ + 1);
  const int* offk = a.off_k + (long long)bh * (a.GK + 1);
  for (int e = tid; e < GB * d; e += 256) {
    const int gi = e / d, k = e - (e / d) * d;
    const int g = g0 + gi;
    double v = 0.0;
    if (g < a.GQ && offq[g + 1] > offq[g]) v = a.qbar[((long long)bh * a.GQ + g) * d + k];
    sq[gi][k] = v;
  }
  __syncthreads();
  const int ng = min(GB, a.GQ - g0);
  for (int h = tid; h < a.GK; h += 256) {
    const bool vh = offk[h + 1] > offk[h];
    const double* c = a.cbar + ((long long)bh * a.GK + h) * d;
    double acc[GB];
#pragma unroll
    for (int gi = 0; gi < GB; ++gi) acc[gi] = 0.0;
    for (int k = 0; k < d; ++k) {
      const double ck = vh ? c[k] : 0.0;
#pragma unroll
      for (int gi = 0; gi < GB; ++gi) acc[gi] = __dadd_rn(acc[gi], __dmul_rn(sq[gi][k], ck));
    }
    for (int gi = 0; gi < ng; ++gi) {
      double m = __dmul_rn(acc[gi], a.s);
      if (m != m) m = -INFINITY;
      a.mu[((long long)bh * a.GQ + g0 + gi) * a.GK + h] = m;
    }
  }
}

// ---------------------------------------------------------------- keys
// One wave per query group (four per workgroup); no workgroup barriers.
__global__ __launch_bounds__(256) void k_route_keys(RouteArgs a) {
  __shared__ double term[4][kMaxGroups];
  __shared__ int nks[kMaxGroups];  // key group sizes, staged once for the four waves
  const int bh = blockIdx.y, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int GK = a.GK;
  const int* offq = a.off_q + (long long)bh * (a.GQ + 1);
  const int* offk = a.off_k + (long long)bh * (a.GK + 1);
  for (int h = threadIdx.x; h < GK; h += 256) nks[h] = offk[h + 1] - offk[h];
  __syncthreads();
  const int g = blockIdx.x * 4 + wv;
  if (g >= a.GQ) return;
  const long long row = ((long long)bh * a.GQ + g) * GK;
  const int nq = offq[g + 1] - offq[g];
  if (nq <= 0) {
    for (int h = lane; h < GK; h += 64) {
      a.ckey[row + h] = kExcluded;
      if (a.rmass) a.rmass[row + h] = 0.0;
    }
    if (lane == 0) a.mand[(long long)bh * a.GQ + g] = -1;
    return;
  }
  // first maximum of mu over non-empty key groups
  double bm = -INFINITY;
  int bi = 0x7fffffff;
  for (int h = lane; h < GK; h += 64) {
    if (nks[h] <= 0) continue;
    const double m = a.mu[row + h];
    if (bi == 0x7fffffff || m > bm) {  // strided per-lane scan keeps the first maximum
      bm = m;
      bi = h;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const double om = __shfl_xor(bm, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    const bool take = (oi != 0x7fffffff) && (bi == 0x7fffffff || om > bm || (om == bm && oi < bi));
    if (take) {
      bm = om;
      bi = oi;
    }
  }
  const int best = bi;
  const double mx = bm;
  const bool finite = best != 0x7fffffff && mx > -INFINITY && mx < INFINITY;
  double* tm = term[wv];
  for (int h = lane; h < GK; h += 64) {
    double t = 0.0;
    if (finite && nks[h] > 0) t = __dmul_rn((double)nks[h], exp(__dsub_rn(a.mu[row + h], mx)));
    tm[h] = t;
  }
  // sequential sum in ascending h (lane 0); this wave's LDS writes above are
  // complete before its reads below, which may alias them
  double ell = 0.0;
  if (lane == 0) {
    double tot = 0.0;
    for (int h = 0; h < GK; ++h)
      if (nks[h] > 0) tot = __dadd_rn(tot, tm[h]);
    ell = finite ? __dadd_rn(mx, log(tot)) : 0.0;
    a.mand[(long long)bh * a.GQ + g] = best == 0x7fffffff ? -1 : best;
  }
  ell = __shfl(ell, 0, 64);
  for (int h = lane; h < GK; h += 64) {
    uint64_t ck = kExcluded;
    double ms = 0.0;
    if (nks[h] > 0) {
      double key = finite ? __dsub_rn(a.mu[row + h], ell) : -INFINITY;
      if (key != key) key = -INFINITY;
      if (h != best) ck = ~ord_f64(key);
      if (a.rmass) ms = __dmul_rn((double)nks[h], exp(key));
    }
    a.ckey[row + h] = ck;
    if (a.rmass) a.rmass[row + h] = ms;
  }
}

// ---------------------------------------------------------------- alpha
// Alpha router (in place of the budget selection): query group g keeps its
// best cell, then takes the other non-empty key groups in order (mass desc,
// h asc) while the retained mass -- summed one cell after another in that
// order from the best cell's -- is below alpha.  The granted cells get
// composite key 0 and the threshold "key below 1", so k_route_emit grants
// exactly them (and the best cells, as always).  One workgroup per group:
// a bitonic sort in LDS, then one thread adds up the prefix.
__global__ __launch_bounds__(256) void k_route_alpha(RouteArgs a) {
  __shared__ double sm[kMaxGroups];
  __shared__ int shh[kMaxGroups];
  const int bh = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  const int GK = a.GK;
  const int* offk = a.off_k + (long long)bh * (a.GK + 1);
  const long long row = ((long long)bh * a.GQ + g) * GK;
  if (g == 0 && tid == 0) {
    long long* thr = a.thr + (long long)bh * 4;
    thr[0] = 1;
    thr[1] = 0;
    thr[2] = 64;
    thr[3] = 2;
  }
  const int best = a.mand[(long long)bh * a.GQ + g];
  int P2 = 1;
  while (P2 < GK) P2 <<= 1;
  // candidates (masses are >= 0; padding -1 sorts last)
  for (int h = tid; h < P2; h += 256) {
    double m = -1.0;
    int hh = 0x7fffffff;
    if (h < GK && best >= 0 && h != best && offk[h + 1] > offk[h]) {
      m = a.rmass[row + h];
      hh = h;
    }
    sm[h] = m;
    shh[h] = hh;
    if (h < GK) a.ckey[row + h] = kExcluded;
  }
  __syncthreads();
  for (int k = 2; k <= P2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P2; i += 256) {
        const int l = i ^ j;
        if (l > i) {
          const double mi = sm[i], ml = sm[l];
          const int hi = shh[i], hl = shh[l];
          const bool l_first = ml > mi || (ml == mi && hl < hi);
          if (l_first == ((i & k) == 0)) {
            sm[i] = ml;
            sm[l] = mi;
            shh[i] = hl;
            shh[l] = hi;
          }
        }
      }
      __syncthreads();
    }
  if (tid == 0 && best >= 0) {
    double kept = a.rmass[row + best];
    for (int i = 0; i < P2; ++i) {
      const int h = shh[i];
      if (h == 0x7fffffff || kept >= a.alpha) break;
      a.ckey[row + h] = 0;
      kept = __dadd_rn(kept, sm[i]);
    }
  }
}

// ---------------------------------------------------------------- select
// Weighted radix select over the 88-bit composite (descending key, cell index):
// find the first cell in sorted order whose cumulative cost exceeds the budget
// left after the mandatory cells.
__device__ inline void comp_digits(uint64_t ck, uint32_t cell, int pass, int* dig) {
  *dig = pass < 8 ? (int)((ck >> (56 - 8 * pass)) & 255u) : (int)((cell >> (16 - 8 * (pass - 8))) & 255u);
}

__device__ inline bool comp_prefix_eq(uint64_t ck, uint32_t cell, int nbits, uint64_t ph, uint32_t pl) {
  if (nbits == 0) return true;
  if (nbits <= 64) {
    const int sh = 64 - nbits;
    return sh == 0 ? ck == ph : (ck >> sh) == (ph >> sh);
  }
  if (ck != ph) return false;
  const int sh = 24 - (nbits - 64);
  return (cell >> sh) == (pl >> sh);
}

// -1: below prefix, 0: equal at nbits, 1: above
__device__ inline int comp_cmp_prefix(uint64_t ck, uint32_t cell, int nbits, uint64_t ph, uint32_t pl) {
  if (nbits == 0) return 0;
  if (nbits <= 64) {
    const int sh = 64 - nbits;
    const uint64_t a = sh == 0 ? ck : (ck >> sh), b = sh == 0 ? ph : (ph >> sh);
    return a < b ? -1 : (a > b ? 1 : 0);
  }
  if (ck != ph) return ck < ph ? -1 : 1;
  const int sh = 24 - (nbits - 64);
  const uint32_t a = cell >> sh, b = pl >> sh;
  return a < b ? -1 : (a > b ? 1 : 0);
}

// thr layout: [0] prefix_hi, [1] prefix_lo, [2] nbits, [3] mode (0 none, 1 all, 2 exclusive, 3 inclusive)
__device__ inline bool thr_grants(const long long* thr, uint64_t ck, uint32_t cell) {
  const int mode = (int)thr[3];
  if (mode == 0) return false;
  if (mode == 1) return true;
  const int c = comp_cmp_prefix(ck, cell, (int)thr[2], (uint64_t)thr[0], (uint32_t)thr[1]);
  return c < 0 || (mode == 3 && c == 0);
}

// Once the cells sharing the selected prefix number at most kSelCap, they are
// gathered, sorted and scanned instead of being narrowed a byte at a time.
constexpr int kSelCap = 1024;

__global__ __launch_bounds__(1024) void k_route_select(RouteArgs a) {
  __shared__ int nq[kMaxGroups], nk[kMaxGroups];
  __shared__ unsigned long long hist[16][256];
  __shared__ int cnth[256];
  __shared__ long long red[16];
  __shared__ long long rem_s;
  __shared__ unsigned long long ph_s;
  __shared__ unsigned pl_s;
  __shared__ int nbits_s, done_s, mode_s, finish_s, ncand_s, found_s;
  __shared__ unsigned long long sk[kSelCap];
  __shared__ unsigned scell[kSelCap];
  __shared__ long long scost[kSelCap];
  const int bh = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  const int GQ = a.GQ, GK = a.GK;
  const int* offq = a.off_q + (long long)bh * (GQ + 1);
  const int* offk = a.off_k + (long long)bh * (GK + 1);
  for (int g = tid; g < GQ; g += 1024) nq[g] = offq[g + 1] - offq[g];
  for (int h = tid; h < GK; h += 1024) nk[h] = offk[h + 1] - offk[h];
  __syncthreads();
  long long* thr = a.thr + (long long)bh * 4;
  if (a.dense_route) {
    if (tid == 0) {
      thr[0] = 0;
      thr[1] = 0;
      thr[2] = 0;
      thr[3] = 1;
    }
    return;
  }
  long long cm = 0;
  const int* mand = a.mand + (long long)bh * GQ;
  for (int g = tid; g < GQ; g += 1024)
    if (mand[g] >= 0) cm += (long long)nq[g] * nk[mand[g]];
  for (int o = 32; o > 0; o >>= 1) cm += __shfl_xor(cm, o, 64);
  if ((tid & 63) == 0) red[wave] = cm;
  __syncthreads();
  if (tid == 0) {
    long long t = 0;
    for (int w = 0; w < 16; ++w) t += red[w];
    rem_s = a.budget - t;
    ph_s = 0;
    pl_s = 0;
    nbits_s = 0;
    done_s = rem_s < 0 ? 1 : 0;
    mode_s = rem_s < 0 ? 0 : 2;
  }
  __syncthreads();
  const uint64_t* ck = a.ckey + (long long)bh * GQ * GK;
  const int ncell = GQ * GK;
  if (tid == 0) finish_s = 0;
  for (int pass = 0; pass < 11 && !done_s; ++pass) {
    for (int e = tid; e < 16 * 256; e += 1024) (&hist[0][0])[e] = 0ull;
    if (tid < 256) cnth[tid] = 0;
    __syncthreads();
    const int nbits = nbits_s;
    const uint64_t ph = ph_s;
    const uint32_t pl = pl_s;
    const int lane = tid & 63;
    // four cells per thread per round, their keys loaded together
    constexpr int U = 4;
    for (int c00 = 0; c00 < ncell; c00 += U * 1024) {
      uint64_t kk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c00 + u * 1024 + tid;
        kk[u] = c < ncell ? ck[c] : kExcluded;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c00 + u * 1024 + tid;
        bool take = false;
        int dig = 0;
        unsigned long long cost = 0;
        {
          const uint64_t k = kk[u];
          if (k != kExcluded && comp_prefix_eq(k, (uint32_t)c, nbits, ph, pl)) {
            take = true;
            comp_digits(k, (uint32_t)c, pass, &dig);
            const int g = c / GK, h = c - (c / GK) * GK;
            cost = (unsigned long long)((long long)nq[g] * nk[h]);
          }
        }
        // early passes put almost every cell in one bin: when all the wave's
        // cells share a digit, one lane adds the wave's total
        const unsigned long long act = __builtin_amdgcn_ballot_w64(take);
        if (act == 0ull) continue;
        const int first = __builtin_ctzll(act);
        const int d0 = __shfl(dig, first, 64);
        if (__builtin_amdgcn_ballot_w64(take && dig == d0) == act) {
          unsigned long long t = cost;
          for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
          if (lane == first) {
            atomicAdd(&hist[wave][d0], t);
            atomicAdd(&cnth[d0], __builtin_popcountll(act));
          }
        } else if (take) {
          atomicAdd(&hist[wave][dig], cost);
          atomicAdd(&cnth[dig], 1);
        }
      }
    }
    __syncthreads();
    // bin totals and their inclusive prefix (threads 0-255, four waves); the
    // chosen bin is the first whose prefix exceeds what is left of the budget
    long long pre = 0;
    if (tid < 256) {
      unsigned long long t = 0;
      for (int w = 0; w < 16; ++w) t += hist[w][tid];
      pre = (long long)t;
      for (int o = 1; o < 64; o <<= 1) {
        const long long u = __shfl_up(pre, o, 64);
        if (lane >= o) pre += u;
      }
      if (lane == 63) red[wave] = pre;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wave; ++w) pre += red[w];
      const unsigned long long over = __builtin_amdgcn_ballot_w64(pre > rem_s);
      if (lane == 0) red[8 + wave] = over ? 64 * wave + __builtin_ctzll(over) : 256;
      hist[1][tid] = (unsigned long long)pre;  // row 1 is free after the totals above
    }
    __syncthreads();
    if (tid == 0) {
      int chosen = (int)min(min(red[8], red[9]), min(red[10], red[11]));
      long long acc = 0;
      if (chosen >= 256) chosen = -1;
      else if (chosen > 0) acc = (long long)hist[1][chosen - 1];
      if (chosen < 0) {
        mode_s = 3;  // every remaining candidate fits
        done_s = 1;
      } else {
        rem_s -= acc;
        if (pass < 8) ph_s |= (uint64_t)chosen << (56 - 8 * pass);
        else pl_s |= (uint32_t)chosen << (16 - 8 * (pass - 8));
        nbits_s = nbits + 8;
        if (cnth[chosen] <= kSelCap) {
          finish_s = 1;
          done_s = 1;
        }
      }
    }
    __syncthreads();
  }
  if (finish_s) {
    // the cells with the selected prefix, in grant order: the first whose
    // cumulative cost exceeds what is left of the budget is the threshold
    const int nbits = nbits_s;
    const uint64_t ph = ph_s;
    const uint32_t pl = pl_s;
    if (tid == 0) {
      ncand_s = 0;
      found_s = 0;
    }
    __syncthreads();
    for (int c00 = 0; c00 < ncell; c00 += 4 * 1024) {
      uint64_t kk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c00 + u * 1024 + tid;
        kk[u] = c < ncell ? ck[c] : kExcluded;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c00 + u * 1024 + tid;
        const uint64_t k = kk[u];
        if (k == kExcluded || !comp_prefix_eq(k, (uint32_t)c, nbits, ph, pl)) continue;
        const int slot = atomicAdd(&ncand_s, 1);
        const int g = c / GK, h = c - (c / GK) * GK;
        sk[slot] = k;
        scell[slot] = (unsigned)c;
        scost[slot] = (long long)nq[g] * nk[h];
      }
    }
    __syncthreads();
    const int nc = ncand_s;
    if (tid >= nc) {
      sk[tid] = ~0ull;
      scell[tid] = ~0u;
      scost[tid] = 0;
    }
    __syncthreads();
    // bitonic sort of (key, cell) ascending
    for (int kk = 2; kk <= kSelCap; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        const int ixj = tid ^ j;
        if (ixj > tid) {
          const bool up = (tid & kk) == 0;
          const bool gt = sk[tid] > sk[ixj] || (sk[tid] == sk[ixj] && scell[tid] > scell[ixj]);
          if (gt == up) {
            const unsigned long long t0 = sk[tid];
            sk[tid] = sk[ixj];
            sk[ixj] = t0;
            const unsigned t1 = scell[tid];
            scell[tid] = scell[ixj];
            scell[ixj] = t1;
            const long long t2 = scost[tid];
            scost[tid] = scost[ixj];
            scost[ixj] = t2;
          }
        }
        __syncthreads();
      }
    }
    // inclusive prefix of the costs in that order
    long long inc = scost[tid];
    for (int o = 1; o < 64; o <<= 1) {
      const long long t = __shfl_up(inc, o, 64);
      if ((tid & 63) >= o) inc += t;
    }
    if ((tid & 63) == 63) red[wave] = inc;
    __syncthreads();
    for (int w = 0; w < wave; ++w) inc += red[w];
    const long long rem = rem_s;
    // first position past the budget (positions past nc never qualify: their cost is 0
    // and their prefix equals the total of the candidates)
    const bool over = tid < nc && inc > rem && (tid == 0 || inc - scost[tid] <= rem);
    if (over) {
      found_s = 1;
      ph_s = sk[tid];
      pl_s = scell[tid];
      nbits_s = 88;
    }
    __syncthreads();
    // a threshold cell: grant everything before it; otherwise every candidate fits
    if (tid == 0) mode_s = found_s ? 2 : 3;
  }
  if (tid == 0) {
    thr[0] = (long long)ph_s;
    thr[1] = (long long)pl_s;
    thr[2] = nbits_s;
    thr[3] = mode_s;
  }
}

// ---------------------------------------------------------------- CSR, masks, tiles, stats
// Query tiles of a group of s rows: with s rounded up to a multiple of 64,
// every whole 128 rows make one tile and a last 64 (or fewer real rows) make
// one split tile, which the attention kernel runs with all four waves on half
// the rows.  The last 128-row tile may hold from 65 to 128 real rows.
__device__ inline int tiles_of_group(int s) {
  const int s64 = (s + 63) / 64;
  return (s64 >> 1) + (s64 & 1);
}
__device__ inline int tile_is_split(int s, int i) {
  const int s64 = (s + 63) / 64;
  return (s64 & 1) && i == (s64 >> 1);
}

// Exclusive scan over the block of up to 4 * 256 ints held in v[0..n) (in
// place; 4 consecutive entries per thread).  Returns the total.
__device__ inline int block_scan4(int* v, int n, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int loc[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * tid + q;
    loc[q] = i < n ? v[i] : 0;
    sum += loc[q];
  }
  int inc = sum;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  __syncthreads();
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int q = 0; q < 4; ++q) {
    if (q < w) base += tmp[q];
    tot += tmp[q];
  }
  int run = base + inc - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * tid + q;
    if (i < n) v[i] = run;
    run += loc[q];
  }
  __syncthreads();
  return tot;
}

template <typename T>
__device__ inline T block_sum256(T v, T* tmp) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  return tmp[0] + tmp[1] + tmp[2] + tmp[3];
}

__global__ __launch_bounds__(256) void k_route_emit(RouteArgs a) {
  __shared__ int nq[kMaxGroups], nk[kMaxGroups], cnt[kMaxGroups], tcnt[kMaxGroups];
  __shared__ int ord[kMaxGroups], mands[kMaxGroups];
  __shared__ long long lsh[kMaxGroups];
  __shared__ long long thr[4];
  __shared__ int tmpi[4];
  __shared__ long long tmpl[4];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int GQ = a.GQ, GK = a.GK;
  const int* offq = a.off_q + (long long)bh * (GQ + 1);
  const int* offk = a.off_k + (long long)bh * (GK + 1);
  const uint64_t* ck = a.ckey + (long long)bh * GQ * GK;
  const int* mand = a.mand + (long long)bh * GQ;
  for (int g = tid; g < GQ; g += 256) {
    nq[g] = offq[g + 1] - offq[g];
    const int mg = mand[g];
    mands[g] = mg >= 0 && mg < GK ? mg : -1;
  }
  for (int h = tid; h < GK; h += 256) nk[h] = offk[h + 1] - offk[h];
  if (tid < 4) thr[tid] = a.thr[(long long)bh * 4 + tid];
  __syncthreads();
  // grants of every cell of group g: one bit per key group
  uint32_t* gm = a.gmask + (long long)bh * GQ * a.gwords;
  for (int g = tid; g < GQ; g += 256) {
    int c = 0;
    long long L = 0;
    const uint64_t* row = ck + (long long)g * GK;
    for (int w = 0; w < a.gwords; ++w) {
      uint64_t kv[32];
#pragma unroll
      for (int b = 0; b < 32; ++b) kv[b] = 32 * w + b < GK ? row[32 * w + b] : kExcluded;
      uint32_t bits = 0;
#pragma unroll
      for (int b = 0; b < 32; ++b) {
        const int h = 32 * w + b;
        bool gr = false;
        if (h < GK && nq[g] > 0 && nk[h] > 0) {
          const uint32_t cell = (uint32_t)(g * GK + h);
          gr = (h == mands[g]) || (kv[b] != kExcluded && thr_grants(thr, kv[b], cell));
        }
        if (gr) {
          bits |= 1u << b;
          ++c;
          L += nk[h];
        }
      }
      gm[(long long)g * a.gwords + w] = bits;
    }
    cnt[g] = c;
    lsh[g] = L;
    tcnt[g] = tiles_of_group(nq[g]);
    a.lg[(long long)bh * GQ + g] = L;
  }
  // Tiles are listed by their query group's granted key groups, read as a
  // word in ascending key group (a group granted the lowest key group on
  // which two grant sets differ comes first), then by group.  A tile streams
  // its granted groups in ascending order, so neighbouring tiles -- which the
  // attention kernel runs together on one XCD -- read the same K/V rows at
  // about the same time and share the L2.  (A stable order; it only decides
  // which tiles run together, never a result.)  The comparison runs on the
  // bit-reversed mask words, most significant first: a 64-bit key of the
  // first two words, the remaining words only on ties.
  __shared__ unsigned long long lkey[kMaxGroups];
  __syncthreads();
  for (int g = tid; g < GQ; g += 256) {
    const uint32_t w0 = gm[(long long)g * a.gwords];
    const uint32_t w1 = a.gwords > 1 ? gm[(long long)g * a.gwords + 1] : 0u;
    lkey[g] = ((unsigned long long)__builtin_bitreverse32(w0) << 32) | __builtin_bitreverse32(w1);
  }
  __syncthreads();
  for (int g = tid; g < GQ; g += 256) {
    const unsigned long long kg = lkey[g];
    int pos = 0;
    for (int q = 0; q < GQ; ++q) {
      const unsigned long long kq = lkey[q];
      bool before = kq > kg;
      if (kq == kg && q != g) {
        int c = 0;  // -1: q first, 1: g first
        for (int w = 2; w < a.gwords && c == 0; ++w) {
          const uint32_t rq = __builtin_bitreverse32(gm[(long long)q * a.gwords + w]);
          const uint32_t rg = __builtin_bitreverse32(gm[(long long)g * a.gwords + w]);
          if (rq != rg) c = rq > rg ? -1 : 1;
        }
        before = c < 0 || (c == 0 && q < g);
      }
      pos += before;
    }
    ord[pos] = g;
  }
  // per-group figures for the statistics (before the scans reuse the arrays)
  long long routed = 0, mandc = 0;
  int neq = 0, nek = 0;
  for (int g = tid; g < GQ; g += 256) {
    routed += (long long)nq[g] * lsh[g];
    if (nq[g] > 0) {
      ++neq;
      if (mands[g] >= 0) mandc += (long long)nq[g] * nk[mands[g]];
    }
  }
  for (int h = tid; h < GK; h += 256) nek += nk[h] > 0;
  routed = block_sum256(routed, tmpl);
  mandc = block_sum256(mandc, tmpl);
  neq = block_sum256(neq, tmpi);
  nek = block_sum256(nek, tmpi);
  // tile offsets in that order, CSR row offsets in group order
  __shared__ int tord[kMaxGroups];
  for (int i = tid; i < GQ; i += 256) tord[i] = tcnt[ord[i]];
  __syncthreads();
  const int tacc = block_scan4(tord, GQ, tmpi);
  for (int i = tid; i < GQ; i += 256) tcnt[ord[i]] = tord[i];
  const int acc = block_scan4(cnt, GQ, tmpi);
  int* rp = a.csr_ptr + (long long)bh * (GQ + 1);
  for (int g = tid; g < GQ; g += 256) rp[g] = cnt[g];
  if (tid == 0) {
    rp[GQ] = acc;
    a.ntiles[bh] = tacc;
    sparsepr_head_stats st;
    const double nn = (double)a.N * (double)a.N;
    st.routed_pairs = routed;
    st.budget_pairs = a.budget;
    st.mandatory_pairs = mandc;
    st.probe_pairs = (long long)a.M * a.N;
    st.granted_cells = acc;
    st.nonempty_q_groups = neq;
    st.nonempty_kv_groups = nek;
    st.probe_rows = a.M;
    st.residual_rank = 0;
    st.over_budget = a.dense_route ? 0 : (routed > a.budget ? 1 : 0);
    st.q_tiles = tacc;
    int red = 0;
    if (a.fcount)
      for (int t = 0; t < 4 * a.T; ++t) red += a.fcount[(long long)bh * 4 * a.T + t];
    st.kmeans_redecided = red;
    st.fit_fallback = 0;
    st.reserved = 0;
    st.rho_route = (double)routed / nn;
    st.rho_exec = (double)(routed + (long long)a.M * a.N) / nn;
    for (int i = 0; i < 4; ++i) st.sigma[i] = 0.0;
    a.stats[bh] = st;
  }
  __syncthreads();
  int* cols = a.csr_col + (long long)bh * GQ * GK;
  int* tl = a.tiles + (long long)bh * a.max_tiles * 4;
  for (int g = tid; g < GQ; g += 256) {
    int j = cnt[g];
    for (int w = 0; w < a.gwords; ++w) {
      uint32_t bits = gm[(long long)g * a.gwords + w];
      while (bits) {
        const int b = __ffs((int)bits) - 1;
        bits &= bits - 1;
        cols[j++] = 32 * w + b;
      }
    }
    int t0 = tcnt[g];
    const int nt = tiles_of_group(nq[g]);
    for (int i = 0; i < nt; ++i) {
      int* e = tl + (long long)(t0 + i) * 4;
      const int r = kTileRows * i;
      e[0] = g;
      e[1] = offq[g] + r;
      e[2] = min(kTileRows, nq[g] - r);
      e[3] = tile_is_split(nq[g], i);
    }
  }
}

hipError_t launch_route(const Plan& p, hipStream_t s) {
  RouteArgs a;
  a.qbar = p.qbar;
  a.cbar = p.cbar;
  a.off_q = p.off_q;
  a.off_k = p.off_k;
  a.GQ = p.GQ;
  a.GK = p.GK;
  a.d = p.d;
  a.N = p.N;
  a.M = p.M;
  a.s = (double)p.scale;
  a.budget = p.budget;
  a.dense_route = p.dense_route ? 1 : 0;
  a.mu = p.mu;
  a.ckey = p.ckey;
  a.rmass = p.rmass;
  a.alpha = (double)p.alpha;
  a.mand = p.mand;
  a.thr = p.thr;
  a.csr_ptr = p.csr_ptr;
  a.csr_col = p.csr_col;
  a.gmask = p.gmask;
  a.gwords = p.gwords;
  a.lg = p.lg;
  a.tiles = p.tiles;
  a.ntiles = p.ntiles;
  a.max_tiles = p.max_tiles;
  a.stats = p.stats;
  a.fcount = p.kmeans_ran ? p.fcount : nullptr;
  a.T = p.T;
  hipLaunchKernelGGL(k_route_mu, dim3((p.GQ + 15) / 16, p.BH), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_route_keys, dim3((p.GQ + 3) / 4, p.BH), dim3(256), 0, s, a);
  if (p.router == SPARSEPR_ROUTER_ALPHA)
    hipLaunchKernelGGL(k_route_alpha, dim3(p.GQ, p.BH), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_route_select, dim3(p.BH), dim3(1024), 0, s, a);
  hipLaunchKernelGGL(k_route_emit, dim3(p.BH), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- probes
struct ProbeSelArgs {
  const int* off_q;
  int GQ, M;
  int* ppos;
  int* pgroup;
  double* pw;
};

// One wave per (b, h).  The non-empty groups are compacted in order with
// ballots, the strided allocation (M < groups) counts with LDS atomics, and
// every probe finds its group by a binary search over the allocation prefix.
__global__ __launch_bounds__(64) void k_probe_select(ProbeSelArgs a) {
  __shared__ int ne[kMaxGroups];
  __shared__ int mg[kMaxGroups];
  __shared__ int off[kMaxGroups + 1];
  __shared__ int cum[kMaxGroups + 1];
  __shared__ double wl[kMaxProbe];
  const int bh = blockIdx.x, lane = threadIdx.x;
  const int M = a.M, GQ = a.GQ;
  if (M <= 0) return;
  for (int g = lane; g <= GQ; g += 64) off[g] = a.off_q[(long long)bh * (GQ + 1) + g];
  for (int g = lane; g < GQ; g += 64) mg[g] = 0;
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
  int gp = 0;
  for (int g0 = 0; g0 < GQ; g0 += 64) {
    const int g = g0 + lane;
    const bool nz = g < GQ && off[g + 1] > off[g];
    const unsigned long long m = __builtin_amdgcn_ballot_w64(nz);
    if (nz) ne[gp + __builtin_popcountll(m & below)] = g;
    gp += __builtin_popcountll(m);
  }
  __syncthreads();
  if (gp == 0) return;
  if (M >= gp) {
    if (lane == 0) {
      const int base = M / gp, rem = M - (M / gp) * gp;
      long long carry = 0;
      for (int r = 0; r < gp; ++r) {
        const int g = ne[r];
        const long long want = base + (r < rem ? 1 : 0) + carry;
        const long long sz = off[g + 1] - off[g];
        const long long m = want < sz ? want : sz;
        mg[g] = (int)m;
        carry = want - m;
      }
      while (carry > 0) {
        for (int r = 0; r < gp && carry > 0; ++r) {
          const int g = ne[r];
          const long long room = (long long)(off[g + 1] - off[g]) - mg[g];
          const long long add = carry < room ? carry : room;
          mg[g] += (int)add;
          carry -= add;
        }
      }
    }
  } else {
    for (int j = lane; j < M; j += 64) atomicAdd(&mg[ne[(int)(((2LL * j + 1) * gp) / (2LL * M))]], 1);
  }
  __syncthreads();
  // cum[r]: probes of the groups ranked before r
  int run = 0;
  for (int r0 = 0; r0 < gp; r0 += 64) {
    const int r = r0 + lane;
    const int v = r < gp ? mg[ne[r]] : 0;
    int inc = v;
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(inc, o, 64);
      if (lane >= o) inc += t;
    }
    if (r < gp) cum[r] = run + inc - v;
    run += __shfl(inc, 63, 64);
  }
  if (lane == 0) cum[gp] = run;
  __syncthreads();
  double part = 0.0;
  for (int k = lane; k < M; k += 64) {
    int lo = 0, hi = gp - 1;  // last rank with cum[r] <= k
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cum[mid] <= k) lo = mid;
      else hi = mid - 1;
    }
    const int g = ne[lo], t = k - cum[lo];
    const long long sz = off[g + 1] - off[g];
    a.ppos[(long long)bh * M + k] = off[g] + (int)(((2LL * t + 1) * sz) / (2LL * mg[g]));
    a.pgroup[(long long)bh * M + k] = g;
    const double w = (double)sz / (double)mg[g];
    wl[k] = w;
    part += w;
  }
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  const double f = (double)M / part;
  for (int k = lane; k < M; k += 64) a.pw[(long long)bh * M + k] = wl[k] * f;
}

hipError_t launch_probe_select(const Plan& p, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  ProbeSelArgs a{p.off_q, p.GQ, p.M, p.ppos, p.pgroup, p.pw};
  hipLaunchKernelGGL(k_probe_select, dim3(p.BH), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace sp
