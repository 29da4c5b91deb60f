// Response-Coupled Partitioning kernels for gfx950.
//
// Sources (page title, section):
//   [TS] "Resumen Técnico: SparsePR – Atención Dispersa Libre de Entrenamiento ..."
//        (gist.science), 2.A: sampled queries define M_K = Q_s^T Q_s / M_s; keys are
//        grouped by k-means on the eigenvectors of M_K into paired K/V groups; the
//        group centres define query coordinates (pre-softmax logits); queries are
//        grouped by k-means on those; one asymmetric pass.
//   [NE] news explainer reposted from 科技行者, section "SparsePR：先把误差聚拢，再用少量
//        “抽查”去纠正": a random small batch of queries probes every key; a key's
//        coordinates are its logit profile under that batch.
//   2.C of [TS] and the [NE] section "稀疏执行怎么落地，误差怎么算才公平": tokens are laid
//        out group by group so every group is contiguous.
//
// Both k-means run Lloyd steps on raw bf16 rows (or split fp32 rows) against
// "centre images": for a metric M, argmin_g ||A x - mu_g||^2 equals
// argmin_g (c_g - 2 x . y_g) with y_g = M xbar_g and c_g = xbar_g . y_g, so one
// bf16 MFMA product with a fused argmin does the assignment.  Centre images
// are kept as hi + lo bf16 pairs (16 significant bits).
#include <algorithm>
#include <map>
#include <mutex>

#include "sp_kernels.h"
#include "sp_eig.h"

namespace sp {

// ============================================================================
// a1: query sample (partial Fisher-Yates on splitmix64) and M_K (fp64)
// ============================================================================
// Step j of the partial shuffle swaps slot j with slot t_j = j + (x_j mod
// (N - j)), where x_j is the generator's j-th output; the draws do not depend
// on the swaps, so thread j makes draw j.  Slot j is final after step j and
// no later step reads it, so what step j finds in a slot p >= j is what the
// latest earlier step aiming at p put there (slot i's value when step i ran),
// or p itself.  Step j's output is therefore the value found through the
// latest earlier step with the same target, and the value slot j held is
// found by following "latest earlier step aiming at slot j" links to a step
// with none; the links are followed by pointer jumping.
__global__ __launch_bounds__(256) void k_query_sample(SampleArgs a) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  __shared__ int tgt[256];
  __shared__ int held[256];  // value slot j held when step j ran
  __shared__ int lnk[256];
  __shared__ int srt[256];
  const int Ms = a.Ms, N = a.N;
  int t = 0;
  if (tid < Ms) {
    uint64_t z = (a.seed ^ ((uint64_t)(bh + a.bh0) * kGolden64)) + (uint64_t)(tid + 1) * kGolden64;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    t = tid + (int)(z % (uint64_t)(N - tid));
    tgt[tid] = t;
  }
  __syncthreads();
  int aim = -1, same = -1;  // latest earlier step aiming at slot tid / at slot t
  if (tid < Ms)
    for (int i = 0; i < tid; ++i) {
      const int ti = tgt[i];
      aim = ti == tid ? i : aim;
      same = ti == t ? i : same;
    }
  held[tid] = tid;
  lnk[tid] = aim;
  __syncthreads();
  for (int r = 1; r < 256; r <<= 1) {
    const int l = lnk[tid];
    const int hv = l >= 0 ? held[l] : held[tid];
    const int nl = l >= 0 ? lnk[l] : -1;
    __syncthreads();
    held[tid] = hv;
    lnk[tid] = nl;
    __syncthreads();
  }
  srt[tid] = tid < Ms ? (same >= 0 ? held[same] : t) : 0x7fffffff;
  __syncthreads();
  for (int k = 2; k <= 256; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int ixj = tid ^ j;
      if (ixj > tid) {
        const int a0 = srt[tid], a1 = srt[ixj];
        const bool up = (tid & k) == 0;
        if ((a0 > a1) == up) {
          srt[tid] = a1;
          srt[ixj] = a0;
        }
      }
      __syncthreads();
    }
  }
  if (tid < Ms) a.sample[(long long)bh * Ms + tid] = srt[tid];
}

// M_K = Q_s^T Q_s / M_s in fp64 (a d x d block per (b,h), 4 x 4 outputs per
// thread).  The sampled rows are staged 64 at a time as fp32 (bf16 and fp32
// inputs are exact there); products of two fp32 values are exact in fp64, so
// only the additions round.  (D/4)^2 / 256 workgroups of 256 threads per
// (b,h), each owning a band of block rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_key_metric64(SampleArgs a) {
  constexpr int LDQ = D + 4;  // 16-byte rows
  constexpr int NT = 256;
  __shared__ __align__(16) float qs[64][LDQ];
  __shared__ int smp[256];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int Ms = a.Ms;
  if (tid < Ms) smp[tid] = a.sample[(long long)bh * Ms + tid];
  constexpr int NB = D / 4;  // 4 x 4 blocks per side
  const int blk = blockIdx.x * NT + tid;
  const int bi = blk / NB, bj = blk - (blk / NB) * NB;
  const bool act = bi < NB;
  double acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.0;
  const T* qbase = static_cast<const T*>(a.q.p);
  constexpr int VEC = 16 / sizeof(T);
  for (int c0 = 0; c0 < Ms; c0 += 64) {
    const int nr = min(64, Ms - c0);
    __syncthreads();
    for (int e = tid; e < nr * (D / VEC); e += NT) {
      const int r = e / (D / VEC), c = (e - r * (D / VEC)) * VEC;
      const uint4 u = *reinterpret_cast<const uint4*>(qbase + a.q.row_off(bh, smp[c0 + r]) + c);
      const T* ev = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int j = 0; j < VEC; ++j) qs[r][c + j] = Elem<T>::load(ev + j);
    }
    __syncthreads();
    if (act)
      for (int r = 0; r < nr; ++r) {
        const float4 u = *reinterpret_cast<const float4*>(&qs[r][4 * bi]);
        const float4 v = *reinterpret_cast<const float4*>(&qs[r][4 * bj]);
        const double uu[4] = {u.x, u.y, u.z, u.w}, vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_fma(uu[x], vv[y], acc[x][y]);
      }
  }
  if (!act) return;
  double* mk = a.mk + (long long)bh * D * D;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) mk[(4 * bi + x) * D + 4 * bj + y] = acc[x][y] / (double)Ms;
}

// ============================================================================
// a2: symmetric eigensolver for M_K (one workgroup per (b,h), all in LDS)
// ============================================================================
// The metric is held in LDS in fp64 (132 KB at d = 128) for the reduction to
// tridiagonal form.  The same LDS then holds the reflectors (column-major,
// packed) behind the eigenvectors of the tridiagonal matrix (the leading rK
// and the factorisation scratch, odd row stride); the shifted-QR fallback, and
// ranks above 32, keep their eigenvector matrix in the workspace.
// NT threads per workgroup: 512 at d = 128 and 1024 at d = 64, the fastest
// of 256, 512 and 1024 at each size (the steps are short, so fewer waves meet
// at the barriers sooner, until the per-thread share of a step grows too long).
template <int D, int NT>
__global__ __launch_bounds__(NT) void k_key_eig(EigArgs a) {
  constexpr int LD = D + 1;  // odd row stride: column walks hit distinct banks
  constexpr int RKL = 32;    // largest rK whose vectors share the LDS with the reflectors
  constexpr int NPK = D * (D - 1) / 2;
  constexpr int NA = D * LD > D * (2 * RKL + 1) + NPK ? D * LD : D * (2 * RKL + 1) + NPK;
  constexpr int PER = D * D / NT;
  __shared__ double A[NA];
  __shared__ double dg[D + 2], eo[D + 2], tau[D], vb[D], pb[D];
  __shared__ double rot[4 * D];
  __shared__ int ctl[8];
  __shared__ int top[D];
  __shared__ double lamv[D];  // eigenvalue of column i of Z
  const int bh = blockIdx.x, tid = threadIdx.x;
  const double* mk = a.mk + (long long)bh * D * D;
  {
    double t[D * D / NT];
#pragma unroll
    for (int u = 0; u < D * D / NT; ++u) t[u] = mk[tid + NT * u];
#pragma unroll
    for (int u = 0; u < D * D / NT; ++u) {
      const int e = tid + NT * u, i = e / D, j = e - (e / D) * D;
      A[i * LD + j] = t[u];
    }
  }
  __syncthreads();
  const EigWork<double> w{A, LD, nullptr, 0, dg, eo, tau, vb, pb, rot, ctl};
  eig_tridiagonalize<double, NT>(w, D);
  // the largest nval eigenvalues by multisection (fewer eigenvalues: more
  // threads per bracket, fewer rounds)
  const int nval = min(max(a.nval, a.rK), D);
  eig_bisect<double, NT>(w, D, nval);
  for (int i = tid; i < D; i += NT) lamv[i] = i < nval ? rot[D + i] : 0.0;
  // reflectors: column-major packed, through registers, behind the vector block
  const bool lds_vecs = a.rK <= RKL;
  const int zl = lds_vecs ? 2 * a.rK + 1 : D;
  double* Rp = A + D * (2 * RKL + 1);
  {
    // element (r, c), r > c, goes to c (D - 1) - c (c - 1) / 2 + r - c - 1
    double t[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + NT * u, r = e / D, c = e - (e / D) * D;
      t[u] = r > c ? A[r * LD + c] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + NT * u, r = e / D, c = e - (e / D) * D;
      if (r > c) Rp[c * (D - 1) - (c * (c - 1)) / 2 + r - c - 1] = t[u];
    }
  }
  __syncthreads();
  double* Z = lds_vecs ? A : a.eigz + (long long)bh * D * D;
  EigWork<double> wz{nullptr, 0, Z, zl, dg, eo, tau, vb, pb, rot, ctl};
  if (eig_twisted<double, NT>(wz, D, a.rK)) {
    for (int i = tid; i < D; i += NT) {
      if (a.eigval && i < nval) a.eigval[(long long)bh * D + i] = lamv[i];
      if (i < a.rK) top[i] = i;
    }
  } else {
    // shifted QR over the whole tridiagonal matrix, vectors in the workspace
    Z = a.eigz + (long long)bh * D * D;
    wz.Z = Z;
    wz.ldz = D;
    eig_tridiagonal_qr<double, NT>(wz, D);
    // rank eigenvalues (descending, ties by index)
    for (int i = tid; i < D; i += NT) {
      const double li = dg[i];
      int rank = 0;
      for (int j = 0; j < D; ++j) {
        const double lj = dg[j];
        rank += (lj > li) || (lj == li && j < i);
      }
      if (a.eigval) a.eigval[(long long)bh * D + rank] = li;
      if (rank < a.rK) top[rank] = i;
      lamv[i] = li;
    }
  }
  __syncthreads();
  eig_back_transform_packed<double, NT, NT / 32>(wz, Rp, D, top, a.rK);
  // coordinate map: column k of kmap = s sqrt(lambda_k) u_k (also zero-padded
  // to rKpad columns)
  double* km = a.kmap + (long long)bh * D * a.rK;
  double* kp = a.kmap_pad + (long long)bh * D * a.rKpad;
  for (int e = tid; e < D * a.rKpad; e += NT) {
    const int k = e / a.rKpad, r = e - (e / a.rKpad) * a.rKpad;
    double v = 0.0;
    if (r < a.rK) {
      const int i = top[r];
      v = (double)a.scale * sqrt(fmax(lamv[i], 0.0)) * Z[k * wz.ldz + i];
      km[k * a.rK + r] = v;
    }
    kp[e] = v;
  }
}

// ============================================================================
// a3: key-response coordinates z = K kmap in fp64, kept also as a hi/lo bf16
// pair of its fp32 rounding (the k-means assignment's operands)
// ============================================================================
// One key per thread, 256 keys per workgroup staged through LDS with
// coalesced loads.  The map (zero-padded to RP columns) is the same for every
// lane, so its entries are wave-uniform loads that feed the fp64 FMAs as
// scalar operands.  Inputs are exact in fp32, so every product is exact in
// fp64.
template <typename T, int D, int RP>
__global__ __launch_bounds__(256) void k_key_coords64(CoordArgs a) {
  constexpr int CH = 32;                      // dims per staged chunk
  constexpr int KL = CH + 4 / (int)sizeof(T);  // row stride: an odd number of 4-byte words
  constexpr int VEC = 16 / sizeof(T), PPR = CH / VEC, NP = 256 * PPR / 256;
  __shared__ __align__(16) T kr[256 * KL];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int n0 = blockIdx.x * 256, N = a.N;
  const T* kb = static_cast<const T*>(a.k.p);
  const double* km = a.kmap_pad + (long long)bh * D * RP;
  double acc[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) acc[r] = 0.0;
  const T* row = kr + tid * KL;
  for (int c0 = 0; c0 < D; c0 += CH) {
    uint4 u[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int e = tid + 256 * q, r = e / PPR, c = (e - r * PPR) * VEC;
      u[q] = make_uint4(0, 0, 0, 0);
      if (n0 + r < N) u[q] = *reinterpret_cast<const uint4*>(kb + a.k.row_off(bh, n0 + r) + c0 + c);
    }
    __syncthreads();  // the previous chunk's readers are done
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int e = tid + 256 * q, r = e / PPR, c = (e - r * PPR) * VEC;
      uint32_t* dst = reinterpret_cast<uint32_t*>(kr + r * KL + c);
      dst[0] = u[q].x;
      dst[1] = u[q].y;
      dst[2] = u[q].z;
      dst[3] = u[q].w;
    }
    __syncthreads();
    for (int c = 0; c < CH; ++c) {
      const double x = (double)Elem<T>::load(row + c);
#pragma unroll
      for (int r = 0; r < RP; ++r) acc[r] = __builtin_fma(x, km[(c0 + c) * RP + r], acc[r]);
    }
  }
  const int n = n0 + tid;
  if (n >= N) return;
  const long long zrow = ((long long)bh * N + n) * RP;
  double res2 = 0.0, lo2 = 0.0;  // |z - hi - lo|^2 and |lo|^2 of the split pair
#pragma unroll
  for (int r = 0; r < RP; r += 8) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float f0 = (float)acc[r + j], f1 = (float)acc[r + j + 1];
      hw[j >> 1] = pack_bf16x2(f0, f1);
      lw[j >> 1] = pack_bf16x2(f0 - __uint_as_float(hw[j >> 1] << 16), f1 - __uint_as_float(hw[j >> 1] & 0xffff0000u));
      const double l0 = (double)__uint_as_float(lw[j >> 1] << 16), l1 = (double)__uint_as_float(lw[j >> 1] & 0xffff0000u);
      const double e0 = (acc[r + j] - (double)__uint_as_float(hw[j >> 1] << 16)) - l0;
      const double e1 = (acc[r + j + 1] - (double)__uint_as_float(hw[j >> 1] & 0xffff0000u)) - l1;
      res2 = __builtin_fma(e0, e0, __builtin_fma(e1, e1, res2));
      lo2 = __builtin_fma(l0, l0, __builtin_fma(l1, l1, lo2));
    }
#pragma unroll
    for (int j = 0; j < 8; j += 2)
      *reinterpret_cast<double2*>(a.z64 + zrow + r + j) = make_double2(acc[r + j], acc[r + j + 1]);
    *reinterpret_cast<uint4*>(a.zhi + zrow + r) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *reinterpret_cast<uint4*>(a.zlo + zrow + r) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  // fp32 upper bounds (the relative margin covers the fp64 roundings above)
  a.xbound[(long long)bh * N + n] = make_float2((float)(sqrt(res2) * (1.0 + 0x1p-20)), (float)(sqrt(lo2) * (1.0 + 0x1p-20)));
}

// fp64 matrix-core form for rKpad <= 32: v_mfma_f64_16x16x4f64 over 16-key
// tiles.  Lane layout (A 16x4, B 4x16, D 16x16): A[i][k] in lane i + 16k,
// B[k][j] in lane j + 16k, D[i][j] in lane 16 (i % 4) + j, register i / 4.
// Each wave keeps the whole map as B fragments in registers (d/4 k-steps x
// RP/16 column tiles) and stages 16 keys at a time in its own LDS slice.
template <typename T, int D, int RP>
__global__ __launch_bounds__(256) void k_key_coords_f64mfma(CoordArgs a) {
  typedef double f64x4_t __attribute__((ext_vector_type(4)));
  constexpr int KS = D / 4, NJ = RP / 16, KT = 4, KL = D + 4;
  constexpr int VEC = 16 / sizeof(T), PPR = D / VEC;
  __shared__ float kr[4][16 * KL];
  const int bh = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int N = a.N;
  const int li = lane & 15, lk = lane >> 4;
  const double* km = a.kmap_pad + (long long)bh * D * RP;
  double bfr[KS][NJ];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int t = 0; t < NJ; ++t) bfr[ks][t] = km[(4 * ks + lk) * RP + 16 * t + li];
  const T* kb = static_cast<const T*>(a.k.p);
  float* my = kr[w];
  // the next tile's rows are loaded into registers while the current tile is
  // multiplied (16 rows x PPR pieces, NPL pieces per lane)
  constexpr int NPL = 16 * PPR / 64;
  static_assert(16 * PPR % 64 == 0, "whole pieces per lane");
  const int kbase = (blockIdx.x * 4 + w) * (16 * KT);
  uint4 pre[NPL];
  auto load_tile = [&](int key0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int e = lane + 64 * q, r = e / PPR, c = (e - r * PPR) * VEC;
      pre[q] = key0 + r < N ? *reinterpret_cast<const uint4*>(kb + a.k.row_off(bh, key0 + r) + c)
                            : make_uint4(0, 0, 0, 0);
    }
  };
  if (kbase < N) load_tile(kbase);
  for (int kt = 0; kt < KT; ++kt) {
    const int key0 = kbase + 16 * kt;
    if (key0 >= N) break;  // uniform per wave
    // stage the tile's 16 rows (the wave's own slice: order its writes before its reads)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int e = lane + 64 * q, r = e / PPR, c = (e - r * PPR) * VEC;
      const T* ev = reinterpret_cast<const T*>(&pre[q]);
      float f[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) f[j] = Elem<T>::load(ev + j);
#pragma unroll
      for (int j = 0; j < VEC; j += 4)
        *reinterpret_cast<float4*>(&my[r * KL + c + j]) = make_float4(f[j], f[j + 1], f[j + 2], f[j + 3]);
    }
    if (kt + 1 < KT && key0 + 16 < N) load_tile(key0 + 16);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f64x4_t acc[NJ];
#pragma unroll
    for (int t = 0; t < NJ; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const double av = (double)my[li * KL + 4 * ks + lk];
#pragma unroll
      for (int t = 0; t < NJ; ++t) acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bfr[ks][t], acc[t], 0, 0, 0);
    }
    // lane holds keys key0 + 4 r + lk (r < 4), coordinate 16 t + li
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = key0 + 4 * r + lk;
      double res2 = 0.0, lo2 = 0.0;
#pragma unroll
      for (int t = 0; t < NJ; ++t) {
        const double z = acc[t][r];
        const float zf = (float)z;
        const bf16_t hi = f32_to_bf16(zf);
        const bf16_t lo = f32_to_bf16(zf - bf16_to_f32(hi));
        const double e = (z - (double)bf16_to_f32(hi)) - (double)bf16_to_f32(lo);
        res2 = __builtin_fma(e, e, res2);
        lo2 = __builtin_fma((double)bf16_to_f32(lo), (double)bf16_to_f32(lo), lo2);
        if (n < N) {
          const long long o = ((long long)bh * N + n) * RP + 16 * t + li;
          a.z64[o] = z;
          a.zhi[o] = hi;
          a.zlo[o] = lo;
        }
      }
      for (int o = 8; o > 0; o >>= 1) {
        res2 += __shfl_xor(res2, o, 16);
        lo2 += __shfl_xor(lo2, o, 16);
      }
      if (li == 0 && n < N)
        a.xbound[(long long)bh * N + n] = make_float2((float)(sqrt(res2) * (1.0 + 0x1p-20)), (float)(sqrt(lo2) * (1.0 + 0x1p-20)));
    }
  }
}

// fp32 raw rows -> hi/lo bf16 pair (fp32 inputs only)
__global__ __launch_bounds__(256) void k_split_rows(SplitArgs a) {
  const int bh = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)a.N * a.D) return;
  const int n = (int)(e / a.D), c = (int)(e - (e / a.D) * a.D);
  const float x = static_cast<const float*>(a.x.p)[a.x.row_off(bh, n) + c];
  const bf16_t hi = f32_to_bf16(x);
  const long long o = ((long long)bh * a.N + n) * a.D + c;
  a.hi[o] = hi;
  a.lo[o] = f32_to_bf16(x - bf16_to_f32(hi));
}

// ============================================================================
// a4/a8: Lloyd assignment.  One bf16 MFMA product of centre images (A, 32
// centres x 16 dims) against point rows (B, 16 dims x 32 points) per k-step,
// fused with the argmin.  256 points per workgroup, 32 or 64 per wave.
// MFMA 32x32x16 lane layout: A[m][k]: m = lane%32, k = 8*(lane/32)+j;
// B[k][n]: k = 8*(lane/32)+j, n = lane%32; D[i][j]: j = lane%32,
// i = (r%4) + 8*(r/4) + 4*(lane/32) for accumulator register r.
// ============================================================================
// Running largest three of a point's values x . y_g - c_g / 2.  Each value
// first carries the index of its 32-centre block and its accumulator register
// r in the low pbits = 4 + ceil(log2(blocks)) bits of its mantissa (a change
// below 2^(pbits - 23) of its magnitude, which the error bound includes), so
// plain max and median operations keep track of which centre a value belongs
// to: register r of block k is centre 32 k + (r & 3) + 8 (r >> 2) + 4 (lane / 32).
// Padding centres carry a large negative but finite bias, so no value is
// infinite and no packed value is a NaN.
//
// Plain min/max/median instructions: the values are finite by construction,
// so the quieting of signalling NaN inputs that the compiler puts in front of
// fminf/fmaxf (one instruction per value coming out of an integer operation)
// is not needed.
__device__ inline float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float vmed3(float a, float b, float c) {
  float r;
  asm("v_med3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
struct Seq3 {
  float b, s, t;  // b >= s >= t, packed
};
__device__ inline Seq3 seq3_init() { return Seq3{-INFINITY, -INFINITY, -INFINITY}; }
// fold in the 16 values a lane holds for 32-centre block k: with b >= s >= t,
// t' = med3(s, t, p), s' = med3(b, s, p), b' = max(b, p)
// The packing reads the matrix-core accumulators, so it is plain code: the
// compiler then places the wait states a vector instruction needs before it
// reads the result of a matrix-core instruction (it does not for inline
// assembly).  keep, the mask of the bits a value keeps, sits in a vector
// register so that the packing is one v_and_or_b32 with the index as its
// scalar operand.
// The packing adds an opaque zero z (a scalar register the compiler cannot
// see through) to the index 16 k + r: otherwise it splits the packing into
// v_and_b32 + v_or3_b32 (16 k and r as separate operands), two vector
// instructions where v_and_or_b32 with one scalar operand is one.
__device__ inline uint32_t seq3_zero() {
  uint32_t z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}
__device__ inline void seq3_add_block(Seq3& st, const f32x16& acc, uint32_t keep, int k, uint32_t z) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = __uint_as_float((__float_as_uint(acc[r]) & keep) | ((uint32_t)(16 * k + r) + z));
    st.t = vmed3(st.s, st.t, p);
    st.s = vmed3(st.b, st.s, p);
    st.b = vmax(st.b, p);
  }
}
__device__ inline uint32_t seq3_keep(int pbits) {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(~((1u << pbits) - 1u)));
  return v;
}
__device__ inline int seq3_centre(float v, int pbits, int half) {
  const uint32_t bits = __float_as_uint(v) & ((1u << pbits) - 1u);
  const int r = (int)(bits & 15u), k = (int)(bits >> 4);
  return 32 * k + (r & 3) + 8 * (r >> 2) + 4 * half;
}
// A point's result: the largest three values over all its centres and the
// centres of the first two.
struct Best3 {
  float b, s, t;
  int bi, si;
};
// merge the lane's state with that of lane ^ 32 (the other half of the same
// point's centres): the largest three of two sorted triples, the lower half
// first on equal values (its centre is the lower one)
__device__ inline Best3 seq3_finish(const Seq3& st, int pbits) {
  const int half = (threadIdx.x >> 5) & 1;
  const Seq3 o{__shfl_xor(st.b, 32, 64), __shfl_xor(st.s, 32, 64), __shfl_xor(st.t, 32, 64)};
  const Seq3 a = half ? o : st, c = half ? st : o;  // half 0, half 1
  const bool x1 = a.b >= c.b;
  const float a1 = x1 ? a.s : a.b, a2 = x1 ? a.t : a.s;
  const float c1 = x1 ? c.b : c.s, c2 = x1 ? c.s : c.t;
  const bool x2 = a1 >= c1;
  Best3 r;
  r.b = x1 ? a.b : c.b;
  r.s = x2 ? a1 : c1;
  r.t = x2 ? (a2 >= c1 ? a2 : c1) : (a1 >= c2 ? a1 : c2);
  r.bi = seq3_centre(r.b, pbits, x1 ? 0 : 1);
  r.si = seq3_centre(r.s, pbits, x2 ? 0 : 1);
  return r;
}
// the decoded centres, kept to the G real ones (a padding centre never ranks
// first or second while a point has two real centres; with G = 1 the second
// is a padding centre and never used)
__device__ inline void best3_clamp(Best3& r, int G) {
  r.bi = min(r.bi, G - 1);
  r.si = min(r.si, G - 1);
}

// Sum of squares of 8 bf16 values (exact products, fp32 sums).
__device__ inline float sumsq_bf16x8(const u32x4& v) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x2_t u = __builtin_bit_cast(bf16x2_t, v[j]);
    t = __builtin_amdgcn_fdot2_f32_bf16(u, u, t, false);
  }
  return t;
}

// Largest bound of |y_g|, |c_g| and of the split residual |y_g - hi_g - lo_g|
// over the G centres of (b,h); every lane of the calling wave gets them.
struct CentreBounds {
  float y, c, r, l;
};
__device__ inline CentreBounds centre_bounds(const AssignArgs& a, int bh) {
  const float4* yb = reinterpret_cast<const float4*>(a.ybound) + (long long)bh * a.gstride;
  float ym = 0.f, cm = 0.f, rm = 0.f, lm = 0.f;
  for (int g = threadIdx.x & 63; g < a.G; g += 64) {
    const float4 b = yb[g];
    ym = fmaxf(ym, b.x);
    cm = fmaxf(cm, b.y);
    rm = fmaxf(rm, b.z);
    lm = fmaxf(lm, b.w);
  }
  return CentreBounds{wave_max(ym), wave_max(cm), wave_max(rm), wave_max(lm)};
}

// Wave 0 of the workgroup reduces the bounds into `sb` (visible to the other
// waves after the caller's next workgroup barrier).
__device__ inline void centre_bounds_to_lds(const AssignArgs& a, int bh, CentreBounds* sb) {
  if ((threadIdx.x >> 6) != 0) return;
  const CentreBounds cb = centre_bounds(a, bh);
  if (threadIdx.x == 0) *sb = cb;
}

// Error bound of a point's approximate values x~.y~_g - c~_g/2 against the
// exact x.y_g - c_g/2, given the bound xn of |x~|:
//   |y~ - y| |x~| + |y| |x~ - x| + |y_lo| |x_lo| + accumulation error,
// with |x~ - x| and |x_lo| from the point's own split (xb) when known, else
// eps_x |x~| for both.
__device__ inline float value_bound(const AssignArgs& a, const CentreBounds& cb, float xn, float2 xb) {
  const float xs = a.xbound ? xb.x * cb.y + xb.y * cb.l : xn * a.eps_x * cb.y;
  // the block and register index packed into the low mantissa bits move a
  // value by less than 2^(pbits - 23) of its magnitude, itself at most
  // |x~||y| + |c|/2
  return 1.01f * (xn * cb.r + xs + (a.eps_acc + ldexpf(1.0f, a.pbits - 23)) * (xn * cb.y + 0.5f * cb.c));
}

// A point whose best and second values lie within twice the error bound e
// of each other is a near tie: it goes to the flag list of (b,h) with its
// two candidates.  When the third value is within 2e of the best as well,
// every centre must be re-decided: such "full" flags are counted apart and
// fill the list from its end (a point is flagged at most once per step, so
// the two parts never meet).  One counter update per wave and kind; every
// lane of the wave must call it.
__device__ inline int flag_slot(int* counter, unsigned long long m) {
  const int lane = threadIdx.x & 63;
  const int leader = __builtin_ctzll(m);
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, __builtin_popcountll(m));
  base = __shfl(base, leader, 64);
  return base + __builtin_popcountll(m & ((1ull << lane) - 1ull));
}
__device__ inline void flag_append(const AssignArgs& a, int bh, bool live, const Best3& st, float e, int n) {
  const bool flag = live && st.b - st.s <= 2.0f * e;
  const bool full = flag && st.b - st.t <= 2.0f * e;
  const bool pair = flag && !full;
  const unsigned long long mp = __builtin_amdgcn_ballot_w64(pair);
  const unsigned long long mf = __builtin_amdgcn_ballot_w64(full);
  int4* fl = a.flist + (long long)bh * a.N;
  int* cnt = a.fcnt + (long long)bh * a.fcstride;
  if (mp) {
    const int slot = flag_slot(cnt, mp);
    if (pair && slot < a.N) fl[slot] = make_int4(n, st.bi, st.si, 0);
  }
  if (mf) {
    const int slot = a.N - 1 - flag_slot(cnt + a.fcfull, mf);
    if (full && slot >= 0) fl[slot] = make_int4(n, st.bi, st.si, 1);
  }
}

template <int D>
__global__ __launch_bounds__(512) void k_kmeans_assign(AssignArgs a) {
  // Form for wide bf16 rows (d = 128) and G <= 256, where restaging the
  // centres per 256 points (the staged form below) costs twice the points'
  // own traffic.  A workgroup stages all G <= 256 centre images of one (b, h)
  // in LDS once
  // and covers a.cpw consecutive 256-point chunks of it.  Its eight waves run
  // without further barriers: each takes 64-point blocks in turn (two
  // 32-point MFMA columns held as B operands in registers, the next block's
  // rows loaded while the current one computes), runs through all centres
  // 32 at a time (A operands from LDS, one fragment feeding both columns),
  // keeps each point's nearest centre (ties keep the lower centre), and adds
  // its labels to the chunk histograms with integer atomics (the workgroup
  // clears its chunks' rows first, so the counts are exact).  The
  // accumulators start at -c_g / 2, so they end at
  // x . y_g - c_g / 2 = -(c_g - 2 x . y_g) / 2 and the nearest centre is the
  // largest value.
  constexpr int KS = D / 16, LDI = D + 8, NT = 512, NW = 8, PB = 2, BP = 32 * PB;
  __shared__ __attribute__((aligned(16))) bf16_t sh[256 * LDI];
  __shared__ __attribute__((aligned(16))) bf16_t sl[256 * LDI];
  __shared__ __attribute__((aligned(16))) float sbias[256];
  __shared__ CentreBounds sbound;
  const int bh = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int N = a.N, G = a.G, G32 = (G + 31) & ~31;
  const int c_begin = blockIdx.x * a.cpw;
  const int c_end = min(a.nchunk, c_begin + a.cpw);
  if (c_begin >= c_end) return;  // whole workgroup
  const int n_begin = c_begin * kChunk, n_end = min(N, c_end * kChunk);
  const int nblk = (n_end - n_begin + BP - 1) / BP;

  // clear this workgroup's histogram rows; stage the centre images (rows
  // past G are zero with an infinite bias)
  for (int e = tid; e < (c_end - c_begin) * G; e += NT) {
    const int cc = e / G, g = e - cc * G;
    a.counts[((long long)bh * a.nchunk + c_begin + cc) * a.gstride + g] = 0;
  }
  {
    const bf16_t* yh = a.yhi + (long long)bh * a.gstride * a.ystride;
    const bf16_t* yl = a.ylo + (long long)bh * a.gstride * a.ystride;
    constexpr int PPR = D / 8;
    for (int e0 = 0; e0 < G32 * PPR; e0 += 4 * NT) {
      u32x4 vh[4], vl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + tid + NT * u, r = e / PPR, cc = e % PPR;
        vh[u] = vl[u] = u32x4{0, 0, 0, 0};
        if (r < G) {
          vh[u] = *reinterpret_cast<const u32x4*>(yh + (long long)r * a.ystride + cc * 8);
          vl[u] = *reinterpret_cast<const u32x4*>(yl + (long long)r * a.ystride + cc * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + tid + NT * u, r = e / PPR, cc = e % PPR;
        if (r < G32) {
          *reinterpret_cast<u32x4*>(sh + r * LDI + cc * 8) = vh[u];
          *reinterpret_cast<u32x4*>(sl + r * LDI + cc * 8) = vl[u];
        }
      }
    }
    centre_bounds_to_lds(a, bh, &sbound);
    // -c_g / 2, the accumulators' start (centres past G never win)
    for (int e = tid; e < G32; e += NT) sbias[e] = e < G ? -0.5f * a.ybias[(long long)bh * a.gstride + e] : -0x1p126f;
  }
  __syncthreads();
  const CentreBounds cbd = sbound;
  const uint32_t keep = seq3_keep(a.pbits), z0 = seq3_zero();

  const bf16_t* pbase = static_cast<const bf16_t*>(a.pts.p) + a.pts.row_off(bh, 0);
  const long long psn = a.pts.sn;
  int* cnt = a.counts + (long long)bh * a.nchunk * a.gstride;
  u32x4 ph[PB][KS];
  // block b's fragments: lane (col, half) holds dims 16 ks + 8 half .. + 7 of
  // point n_begin + BP b + 32 pb + col (rows past the end repeat the last row)
#define SP_LOAD_BLOCK(b, DH)                                                                      \
  _Pragma("unroll") for (int pb = 0; pb < PB; ++pb) {                                             \
    const int n = min(n_begin + BP * (b) + 32 * pb + col, N - 1);                                 \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                           \
      DH[pb][ks] = *reinterpret_cast<const u32x4*>(pbase + n * psn + 16 * ks + 8 * half);         \
    }                                                                                             \
  }
  if (w < nblk) SP_LOAD_BLOCK(w, ph)
  for (int b = w; b < nblk; b += NW) {
    u32x4 nh[PB][KS];
    SP_LOAD_BLOCK(min(b + NW, nblk - 1), nh)
    Seq3 st[PB];
    float xsq[PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      st[pb] = seq3_init();
      xsq[pb] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) xsq[pb] += sumsq_bf16x8(ph[pb][ks]);
    }
    for (int cb = 0; cb < G32; cb += 32) {
      // -c_g / 2 of this lane's centres: four runs of four consecutive centres
      f32x16 cinit;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(sbias + cb + 8 * q + 4 * half);
        cinit[4 * q] = f.x;
        cinit[4 * q + 1] = f.y;
        cinit[4 * q + 2] = f.z;
        cinit[4 * q + 3] = f.w;
      }
      f32x16 acc[PB];
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) acc[pb] = cinit;
      // the products at raised wave priority, the top-three updates at the
      // normal one: the SIMD's other wave then fills the matrix core's
      // gaps with its VALU work rather than both waves queueing MFMAs
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int o = (cb + col) * LDI + 16 * ks + 8 * half;
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(sh + o);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(sl + o);
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
          const bf16x8 xh = __builtin_bit_cast(bf16x8, ph[pb][ks]);
          acc[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xh, acc[pb], 0, 0, 0);
          acc[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xh, acc[pb], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) seq3_add_block(st[pb], acc[pb], keep, cb >> 5, z0);
    }
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      Best3 fin = seq3_finish(st[pb], a.pbits);
      best3_clamp(fin, G);
      const float x2 = xsq[pb] + __shfl_xor(xsq[pb], 32, 64);
      const float e = value_bound(a, cbd, sqrtf(x2) * (1.0f + 0x1p-12f), make_float2(0.f, 0.f));
      const int n = n_begin + BP * b + 32 * pb + col;
      const bool live = half == 0 && n < n_end;
      flag_append(a, bh, live, fin, e, n);
      if (live) {
        a.labels[(long long)bh * N + n] = fin.bi;
        atomicAdd(cnt + (long long)(n / kChunk) * a.gstride + fin.bi, 1);
      }
    }
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ph[pb][ks] = nh[pb][ks];
  }
#undef SP_LOAD_BLOCK
}

// (second launch bound: waves per SIMD; at D <= 32 six, so that three
// workgroups share a CU, as many as the staged centres' LDS allows)
template <int D, bool LO, int CG>
__global__ __launch_bounds__(512, (LO && D >= 64) ? 2 : (D <= 32 ? 6 : 4)) void k_kmeans_assign_staged(AssignArgs a) {
  // General form (any D, any G <= kMaxGroups).  One 256-point histogram chunk per
  // workgroup (8 waves x one 32-point MFMA column, points held as B operands
  // in registers); the centre images are staged through LDS CG at a time
  // (two barriers per CG centres) and read as A operands, two 32-centre
  // blocks at a time.  The accumulators start at -c_g / 2, so they end at
  // x . y_g - c_g / 2 and the nearest centre is the largest value.
  constexpr int KS = D / 16;
  constexpr int LDI = D + 8;  // padded LDS row (bank spread)
  constexpr int NT = 512;
  __shared__ __attribute__((aligned(16))) bf16_t sh[CG * LDI];
  __shared__ __attribute__((aligned(16))) bf16_t sl[CG * LDI];
  __shared__ __attribute__((aligned(16))) float sbias[CG];
  __shared__ int hist[kMaxGroups];
  __shared__ CentreBounds sbound;
  const int bh = blockIdx.y, blk = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int N = a.N, G = a.G;
  const int half = lane >> 5, col = lane & 31;
  const int n = blk * kChunk + wave * 32 + col;

  for (int g = tid; g < G; g += NT) hist[g] = 0;

  bf16x8 ph[KS];
  bf16x8 pl[LO ? KS : 1];
  const bf16_t* hib = static_cast<const bf16_t*>(a.pts.p);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    uint4 w = make_uint4(0, 0, 0, 0);
    if (n < N) {
      v = *reinterpret_cast<const uint4*>(hib + a.pts.row_off(bh, n) + 16 * ks + 8 * half);
      if (LO) w = *reinterpret_cast<const uint4*>(a.pts_lo + ((long long)bh * N + n) * D + 16 * ks + 8 * half);
    }
    ph[ks] = __builtin_bit_cast(bf16x8, v);
    if (LO) pl[LO ? ks : 0] = __builtin_bit_cast(bf16x8, w);
  }
  Seq3 st = seq3_init();
  const uint32_t keep = seq3_keep(a.pbits), z0 = seq3_zero();
  float xsq = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) xsq += sumsq_bf16x8(__builtin_bit_cast(u32x4, ph[ks]));
  centre_bounds_to_lds(a, bh, &sbound);
  const bf16_t* yh = a.yhi + (long long)bh * a.gstride * a.ystride;
  const bf16_t* yl = a.ylo + (long long)bh * a.gstride * a.ystride;
  const float* yb = a.ybias + (long long)bh * a.gstride;
  for (int c0 = 0; c0 < G; c0 += CG) {
    __syncthreads();
    for (int e = tid; e < CG * (D / 8); e += NT) {
      const int r = e / (D / 8), cc = e - (e / (D / 8)) * (D / 8);
      const int c = c0 + r;
      uint4 vh = make_uint4(0, 0, 0, 0), vl = make_uint4(0, 0, 0, 0);
      if (c < G) {
        vh = *reinterpret_cast<const uint4*>(yh + (long long)c * a.ystride + cc * 8);
        vl = *reinterpret_cast<const uint4*>(yl + (long long)c * a.ystride + cc * 8);
      }
      *reinterpret_cast<uint4*>(sh + r * LDI + cc * 8) = vh;
      *reinterpret_cast<uint4*>(sl + r * LDI + cc * 8) = vl;
    }
    for (int e = tid; e < CG; e += NT) sbias[e] = (c0 + e < G) ? -0.5f * yb[c0 + e] : -0x1p126f;
    __syncthreads();
    const int nblk = min(CG, G - c0);
    // two 32-centre blocks at a time: independent accumulator chains
    for (int cb = 0; cb < nblk; cb += 64) {
      const bool two = cb + 32 < nblk;
      // -c_g / 2 of this lane's centres: four runs of four consecutive centres
      f32x16 acc0, acc1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f0 = *reinterpret_cast<const float4*>(sbias + cb + 8 * q + 4 * half);
        const float4 f1 = *reinterpret_cast<const float4*>(sbias + min(cb + 32, CG - 32) + 8 * q + 4 * half);
        acc0[4 * q] = f0.x;
        acc0[4 * q + 1] = f0.y;
        acc0[4 * q + 2] = f0.z;
        acc0[4 * q + 3] = f0.w;
        acc1[4 * q] = f1.x;
        acc1[4 * q + 1] = f1.y;
        acc1[4 * q + 2] = f1.z;
        acc1[4 * q + 3] = f1.w;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16_t* r0 = sh + (cb + col) * LDI + 16 * ks + 8 * half;
        const bf16_t* q0 = sl + (cb + col) * LDI + 16 * ks + 8 * half;
        const bf16x8 ah0 = *reinterpret_cast<const bf16x8*>(r0);
        const bf16x8 al0 = *reinterpret_cast<const bf16x8*>(q0);
        const bf16x8 ah1 = *reinterpret_cast<const bf16x8*>(r0 + 32 * LDI);
        const bf16x8 al1 = *reinterpret_cast<const bf16x8*>(q0 + 32 * LDI);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah0, ph[ks], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah1, ph[ks], acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al0, ph[ks], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al1, ph[ks], acc1, 0, 0, 0);
        if (LO) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah0, pl[LO ? ks : 0], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah1, pl[LO ? ks : 0], acc1, 0, 0, 0);
        }
      }
      seq3_add_block(st, acc0, keep, (c0 + cb) >> 5, z0);
      if (two) seq3_add_block(st, acc1, keep, (c0 + cb + 32) >> 5, z0);
    }
  }
  Best3 fin = seq3_finish(st, a.pbits);
  best3_clamp(fin, G);
  {
    const CentreBounds cbd = sbound;  // written before the staging barriers
    // split points: |x~| <= |x_hi| (1 + 2^-7)
    const float x2 = xsq + __shfl_xor(xsq, 32, 64);
    const float2 xb = (a.xbound && n < N) ? a.xbound[(long long)bh * N + n] : make_float2(0.f, 0.f);
    const float e = value_bound(a, cbd, sqrtf(x2) * (LO ? 1.0f + 0x1p-7f : 1.0f + 0x1p-12f), xb);
    flag_append(a, bh, half == 0 && n < N, fin, e, n);
  }
  __syncthreads();
  if (half == 0 && n < N) {
    a.labels[(long long)bh * N + n] = fin.bi;
    atomicAdd(&hist[fin.bi], 1);
  }
  __syncthreads();
  int* cnt = a.counts + ((long long)bh * a.nchunk + blk) * a.gstride;
  for (int g = tid; g < G; g += NT) cnt[g] = hist[g];
}

// Exact re-decision of the points a Lloyd step flagged as near ties.  The
// values x . y_g - c_g / 2 are computed in fp64 from the exact point row (raw
// row, or the fp64 key coordinates) and the fp64 images; the largest is kept,
// ties to the lower centre.  When only the point's two candidates are within
// twice the error bound of its best value (the front of the flag list),
// every other centre is provably below both and the two dot products decide:
// 16 lanes per such point, lanes over dimensions, row-major images.  The
// points with a third centre in range (the back of the list) are re-decided
// over every centre by a whole workgroup (one centre per thread,
// dimension-major images, 64 loads in flight).  A changed label moves the
// point between the chunk histograms with integer atomics.
template <typename T>
__device__ inline double point_value(const RedecideArgs& a, const T* row, int k) {
  return (double)Elem<T>::load(row + k);
}

__device__ inline void relabel(const RedecideArgs& a, int bh, int n, int win) {
  if (win < 0 || win >= a.G) return;
  int* lab = a.labels + (long long)bh * a.N + n;
  const int old = *lab;
  if (win != old) {
    *lab = win;
    int* cnt_row = a.counts + ((long long)bh * a.nchunk + n / kChunk) * a.gstride;
    atomicSub(cnt_row + old, 1);
    atomicAdd(cnt_row + win, 1);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_kmeans_redecide(RedecideArgs a) {
  constexpr int NW = 4, KU = 64;
  __shared__ double sv[NW];
  __shared__ int si[NW];
  __shared__ double sx[128];
  int bh, wx;
  xcd_slice(blockIdx.x, gridDim.x, a.nwg, bh, wx);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int* cntp = a.fcnt + (long long)bh * a.fcstride;
  const int cnt = min(cntp[0], a.N), cntf = min(cntp[a.fcfull], a.N - cnt);
  const int4* fl = a.flist + (long long)bh * a.N;
  const double* yr = a.y64 + (long long)bh * a.gstride * a.ystride;   // [gstride][Dimg]
  const double* yt = a.y64t + (long long)bh * a.ystride * a.gstride;  // [Dimg][gstride]
  const double* cb = a.c64 + (long long)bh * a.gstride;
  const int Dx = a.Dx, G = a.G, gs = a.gstride;
  const T* rawb = static_cast<const T*>(a.raw.p);
  // two-candidate flags (the front of the list): four points per wave at a
  // time, 16 lanes each
  const int sub = lane & 15, grp = lane >> 4;
  for (int e0 = (wx * NW + w) * 4; e0 < cnt; e0 += a.nwg * NW * 4) {
    const int e = e0 + grp;
    const bool act = e < cnt;
    const int4 ent = act ? fl[e] : make_int4(0, 0, 0, 0);
    const int n = ent.x, b = ent.y, s = ent.z;
    double db = 0.0, ds = 0.0;
    if (act) {
      // every load of the point's row and of both images first (Dx <= 128:
      // at most eight dimensions per lane), then the products in order
      constexpr int KI = 128 / 16;
      const double* x64 = a.x64 ? a.x64 + ((long long)bh * a.N + n) * a.x64stride : nullptr;
      const T* xr = a.x64 ? nullptr : rawb + a.raw.row_off(bh, n);
      const double* yb = yr + (long long)b * a.ystride;
      const double* ys = yr + (long long)s * a.ystride;
      double xv[KI], bv[KI], sv2[KI];
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int k = sub + 16 * i;
        const bool ok = k < Dx;
        xv[i] = ok ? (x64 ? x64[k] : point_value<T>(a, xr, k)) : 0.0;
        bv[i] = ok ? yb[k] : 0.0;
        sv2[i] = ok ? ys[k] : 0.0;
      }
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        db = __builtin_fma(xv[i], bv[i], db);
        ds = __builtin_fma(xv[i], sv2[i], ds);
      }
    }
    for (int o = 8; o > 0; o >>= 1) {
      db += __shfl_xor(db, o, 16);
      ds += __shfl_xor(ds, o, 16);
    }
    if (act && sub == 0) {
      db -= 0.5 * cb[b];
      ds -= 0.5 * cb[s];
      relabel(a, bh, n, (ds > db || (ds == db && s < b)) ? s : b);
    }
  }
  // full flags (the back of the list): every centre, one workgroup per
  // point, its row staged in LDS in fp64
  for (int e = wx; e < cntf; e += a.nwg) {
    const int n = fl[a.N - 1 - e].x;
    if (tid < Dx) {
      if (a.x64) sx[tid] = a.x64[((long long)bh * a.N + n) * a.x64stride + tid];
      else sx[tid] = point_value<T>(a, rawb + a.raw.row_off(bh, n), tid);
    }
    __syncthreads();
    double best = -INFINITY;
    int bi = 0x7fffffff;
    for (int g0 = 0; g0 < G; g0 += 256) {
      const int g = g0 + tid;
      double acc = 0.0;
      for (int k0 = 0; k0 < Dx; k0 += KU) {
        double y[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) y[u] = (g < G && k0 + u < Dx) ? yt[(long long)(k0 + u) * gs + g] : 0.0;
#pragma unroll
        for (int u = 0; u < KU; ++u)
          if (k0 + u < Dx) acc = __builtin_fma(sx[k0 + u], y[u], acc);
      }
      if (g < G) {
        const double v = acc - 0.5 * cb[g];
        if (v > best) {  // centres ascend per thread: ties keep the lower one
          best = v;
          bi = g;
        }
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > best || (ov == best && oi < bi)) {
        best = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      sv[w] = best;
      si[w] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int q = 1; q < NW; ++q)
        if (sv[q] > best || (sv[q] == best && si[q] < bi)) {
          best = sv[q];
          bi = si[q];
        }
      relabel(a, bh, n, bi);
    }
    __syncthreads();  // sx, sv, si are reused by the next point
  }
}

// One bf16 32x32x16 matrix-core product per pattern, restricted to output
// element (0, 0): row 0 of A and column 0 of B carry the pattern's 16 values,
// every other operand element is zero, the accumulator starts at the
// pattern's value.  One wave per pattern.
__global__ __launch_bounds__(64) void k_mfma_rounding(const float* pats, int n, float* out) {
  const int p = blockIdx.x, lane = threadIdx.x, half = lane >> 5, col = lane & 31;
  if (p >= n) return;
  const float* pa = pats + (long long)p * 33;
  bf16x8 av, bv;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = 8 * half + j;
    av[j] = (__bf16)(col == 0 ? pa[k] : 0.f);
    bv[j] = (__bf16)(col == 0 ? pa[16 + k] : 0.f);
  }
  f32x16 acc = {};
  if (lane == 0) acc[0] = pa[32];  // D[0][0]: lane 0, register 0
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  if (lane == 0) out[p] = acc[0];
}

// histogram of given labels (partition supplied by the caller); labels outside
// [0, G) are clamped
__global__ __launch_bounds__(256) void k_count_labels(CountArgs a) {
  __shared__ int hist[kMaxGroups];
  const int bh = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  for (int g = tid; g < a.G; g += 256) hist[g] = 0;
  __syncthreads();
  const int n = chunk * kChunk + tid;
  if (n < a.N) {
    int l = a.in_labels[(long long)bh * a.N + n];
    l = l < 0 ? 0 : (l >= a.G ? a.G - 1 : l);
    a.labels[(long long)bh * a.N + n] = l;
    atomicAdd(&hist[l], 1);
  }
  __syncthreads();
  int* cnt = a.counts + ((long long)bh * a.nchunk + chunk) * a.gstride;
  for (int g = tid; g < a.G; g += 256) cnt[g] = hist[g];
}

// ============================================================================
// a5: counting sort -- chunk offsets (group-major, chunk-minor) and stable scatter
// ============================================================================
__global__ __launch_bounds__(1024) void k_group_scan(ScanArgs a) {
  __shared__ int part[1024];
  __shared__ int tot[kMaxGroups];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int G = a.G, nch = a.nchunk;
  // P threads per group, each over a contiguous range of chunks
  const int P = 1024 / G;  // G <= kMaxGroups = 1024
  const int g = tid % G, pt = tid / G;
  const bool act = pt < P;
  const int c0 = act ? (int)((long long)pt * nch / P) : 0;
  const int c1 = act ? (int)((long long)(pt + 1) * nch / P) : 0;
  const int* cnt = a.counts + (long long)bh * nch * a.gstride;
  // the thread's first CV counts are loaded together and kept in registers
  // for the second pass; any further ones are loaded eight at a time
  constexpr int CV = 32;
  int cv[CV];
#pragma unroll
  for (int u = 0; u < CV; ++u) cv[u] = c0 + u < c1 ? cnt[(long long)(c0 + u) * a.gstride + g] : 0;
  int sum = 0;
#pragma unroll
  for (int u = 0; u < CV; ++u) sum += cv[u];
  int c = c0 + CV;
  for (; c + 8 <= c1; c += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = cnt[(long long)(c + u) * a.gstride + g];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  for (; c < c1; ++c) sum += cnt[(long long)c * a.gstride + g];
  if (act) part[pt * G + g] = sum;
  __syncthreads();
  if (tid < G) {
    int t = 0;
    for (int q = 0; q < P; ++q) t += part[q * G + tid];
    tot[tid] = t;
  }
  __syncthreads();
  // inclusive Hillis-Steele scan over the G group totals
  for (int o = 1; o < G; o <<= 1) {
    int v = 0;
    if (tid < G && tid >= o) v = tot[tid - o];
    __syncthreads();
    if (tid < G) tot[tid] += v;
    __syncthreads();
  }
  if (!act) return;
  int base = g == 0 ? 0 : tot[g - 1];
  int* off = a.off + (long long)bh * a.offstride;
  if (pt == 0) off[g] = base;
  if (tid == 0) off[G] = a.N;
  for (int q = 0; q < pt; ++q) base += part[q * G + g];
  int* co = a.chunkoff + (long long)bh * nch * a.gstride;
#pragma unroll
  for (int u = 0; u < CV; ++u)
    if (c0 + u < c1) {
      co[(long long)(c0 + u) * a.gstride + g] = base;
      base += cv[u];
    }
  int c2 = c0 + CV;
  for (; c2 + 8 <= c1; c2 += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = cnt[(long long)(c2 + u) * a.gstride + g];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      co[(long long)(c2 + u) * a.gstride + g] = base;
      base += v[u];
    }
  }
  for (; c2 < c1; ++c2) {
    co[(long long)c2 * a.gstride + g] = base;
    base += cnt[(long long)c2 * a.gstride + g];
  }
}

// Stable scatter of one chunk: the rank of a point among the earlier points
// of its chunk with the same label.  Inside a wave, the lanes holding a
// lane's label are the AND over the label's bits of one ballot per bit (or
// its complement): ten ballots for up to 1024 groups, whatever the number of
// distinct labels; earlier waves contribute their per-label counts.
__global__ __launch_bounds__(256) void k_group_scatter(ScatterArgs a) {
  __shared__ int hist[4][kMaxGroups];
  const int bh = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  for (int e = tid; e < 4 * a.gstride; e += 256) hist[e / a.gstride][e % a.gstride] = 0;
  __syncthreads();
  const int n = chunk * kChunk + tid;
  const int my = n < a.N ? a.labels[(long long)bh * a.N + n] : -1;
  const unsigned long long lt = (1ull << lane) - 1ull;
  unsigned long long eq = __builtin_amdgcn_ballot_w64(my >= 0);
  static_assert(kMaxGroups <= 1024, "ten label bits");
  for (int b = 0; b < 10 && (a.gstride - 1) >> b; ++b) {
    const unsigned long long bb = __builtin_amdgcn_ballot_w64(my >= 0 && ((my >> b) & 1));
    eq &= ((my >> b) & 1) ? bb : ~bb;
  }
  int rank = 0;
  if (my >= 0) {
    rank = __builtin_popcountll(eq & lt);
    if (rank == 0) hist[w][my] = __builtin_popcountll(eq);  // the label's first lane
  }
  __syncthreads();
  if (my < 0) return;
  for (int q = 0; q < w; ++q) rank += hist[q][my];
  const int pos = a.chunkoff[((long long)bh * a.nchunk + chunk) * a.gstride + my] + rank;
  a.perm[(long long)bh * a.N + pos] = n;
  if (a.out_labels) a.out_labels[(long long)bh * a.N + n] = my;
}

// ============================================================================
// centre update, step 1: fp64 mean of each group's point rows, summed one row
// after another in ascending token order (member rows are staged through LDS
// 64 at a time; each thread owns one dimension).  Empty groups keep their
// previous centre.
// ============================================================================
template <typename TP>
__global__ __launch_bounds__(256) void k_group_mean(UpdateArgs a) {
  constexpr int NT = 256;
  __shared__ double part[NT * 8];  // P subsets x (padded) dims
  const int bh = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  const int Dp = a.Dp;
  const TP* xb = static_cast<const TP*>(a.pts.p);
  double* cm = a.cmean ? a.cmean + ((long long)bh * a.gstride + g) * a.cstride : nullptr;
  if (a.init) {
    const long long sidx = ((2LL * g + 1) * a.N) / (2LL * a.G);
    for (int j = tid; j < Dp; j += NT) cm[j] = (double)Elem<TP>::load(xb + a.pts.row_off(bh, sidx) + j);
    if (g == 0 && a.fcount)
      for (int t = tid; t < a.T; t += NT) {
        a.fcount[(long long)bh * 4 * a.T + t] = 0;
        a.fcount[(long long)bh * 4 * a.T + 2 * a.T + t] = 0;
      }
    return;
  }
  const int* off = a.off + (long long)bh * a.offstride;
  const int* perm = a.perm + (long long)bh * a.N;
  const int a0 = off[g], a1 = off[g + 1];
  const int n_g = a1 - a0;
  double s = 0.0;
  if (a.means_out) {
    // Means handed to the router: rows summed one after another in ascending
    // token order, the order of the mean's plain definition (one thread per
    // dim).  The group's row indices are staged NT at a time in LDS; each
    // thread keeps 16 row loads in flight.
    __shared__ int sidx[NT];
    for (int c0 = a0; c0 < a1; c0 += NT) {
      const int nr = min(NT, a1 - c0);
      __syncthreads();  // the previous indices are consumed
      if (tid < nr) sidx[tid] = perm[c0 + tid];
      __syncthreads();
      if (tid < Dp) {
        int r = 0;
        for (; r + 15 < nr; r += 16) {
          double v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) v[u] = (double)Elem<TP>::load(xb + a.pts.row_off(bh, sidx[r + u]) + tid);
#pragma unroll
          for (int u = 0; u < 16; ++u) s = __dadd_rn(s, v[u]);
        }
        for (; r < nr; ++r) s = __dadd_rn(s, (double)Elem<TP>::load(xb + a.pts.row_off(bh, sidx[r]) + tid));
      }
    }
  } else {
    // Lloyd updates: 16-byte row pieces; thread (piece c, subset pt) sums the
    // rows r = a0 + pt (mod P) of its VEC dims; the P subset sums are added
    // in a fixed order, so the result is deterministic.
    constexpr int VEC = 16 / sizeof(TP);
    const int cpr = (Dp + VEC - 1) / VEC;  // rows are padded to a 16-byte multiple
    const int P = NT / cpr;
    const int c = tid % cpr, pt = tid / cpr;
    double acc[VEC];
#pragma unroll
    for (int q = 0; q < VEC; ++q) acc[q] = 0.0;
    if (pt < P) {
      // eight rows of the subset at a time: their indices, then their
      // pieces, all loads in flight together; summed in ascending row order
      constexpr int RB = 8;
      for (int r = a0 + pt; r < a1; r += RB * P) {
        int idx[RB];
#pragma unroll
        for (int k = 0; k < RB; ++k) idx[k] = r + k * P < a1 ? perm[r + k * P] : -1;
        uint4 u[RB];
#pragma unroll
        for (int k = 0; k < RB; ++k)
          u[k] = idx[k] >= 0 ? *reinterpret_cast<const uint4*>(xb + a.pts.row_off(bh, idx[k]) + c * VEC)
                             : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < RB; ++k) {
          if (idx[k] < 0) break;
          const TP* ev = reinterpret_cast<const TP*>(&u[k]);
#pragma unroll
          for (int q = 0; q < VEC; ++q) acc[q] = __dadd_rn(acc[q], (double)Elem<TP>::load(ev + q));
        }
      }
#pragma unroll
      for (int q = 0; q < VEC; ++q) part[pt * (cpr * VEC) + c * VEC + q] = acc[q];
    }
    __syncthreads();
    if (tid < Dp)
      for (int q = 0; q < P; ++q) s = __dadd_rn(s, part[q * (cpr * VEC) + tid]);
  }
  if (tid >= Dp) return;
  double mean;
  if (n_g > 0) {
    mean = s / (double)n_g;
    if (cm) cm[tid] = mean;
  } else {
    mean = cm ? cm[tid] : 0.0;
  }
  if (a.means_out)
    a.means_out[((long long)bh * a.mo_gstride + g) * Dp + tid] = n_g > 0 ? mean : __builtin_nan("");
}

// centre update, step 2: image y = M mean (or the mean itself) in fp64 and
// its bias c = mean . y; kept in fp64 (for the exact re-decision), as a
// hi/lo bf16 pair and an fp32 bias (the assignment's operands), with bounds
// of |y|, |c| and of the pair's residual |y - hi - lo| (its error bound).
// 16 groups per workgroup; 16 threads per group, thread jj owning the
// dimensions jj, jj + 16, ...: in the product the 16 threads of a group read
// 16 consecutive fp64 entries of a staged row of M (distinct banks) and the
// four groups of a wave read the same ones (one broadcast).  M is staged
// through LDS 32 rows at a time.
__global__ __launch_bounds__(256) void k_centre_images(UpdateArgs a) {
  constexpr int GB = 16, MR = 32, LDM = 130;
  __shared__ double smean[GB][129];
  __shared__ __attribute__((aligned(16))) double sm[MR][LDM];
  const int bh = blockIdx.y, g0 = blockIdx.x * GB, tid = threadIdx.x;
  const int Dp = a.Dp, Dimg = a.Dimg;
  const int ng = min(GB, a.G - g0);
  {
    // all eight loads of a thread in flight before the stores
    double t[GB * 128 / 256];
#pragma unroll
    for (int u = 0; u < GB * 128 / 256; ++u) {
      const int e = tid + 256 * u, gl = e >> 7, j = e & 127;
      t[u] = (gl < ng && j < Dp) ? a.cmean[((long long)bh * a.gstride + g0 + gl) * a.cstride + j] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < GB * 128 / 256; ++u) {
      const int e = tid + 256 * u;
      smean[e >> 7][e & 127] = t[u];
    }
  }
  const int gl = tid >> 4, jj = tid & 15;
  const double* M = a.metric ? a.metric + (long long)bh * Dp * Dp : nullptr;
  double y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = 0.0;
  __syncthreads();
  if (M) {
    for (int i0 = 0; i0 < Dp; i0 += MR) {
      const int nr = min(MR, Dp - i0);
      __syncthreads();
      // 16-byte pieces, four per thread in flight together
      const int np = nr * Dp / 2;
      for (int e0 = 0; e0 < np; e0 += 4 * 256) {
        double2 t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = e0 + tid + 256 * u;
          t[u] = e < np ? *reinterpret_cast<const double2*>(M + (long long)i0 * Dp + 2 * e) : make_double2(0.0, 0.0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = e0 + tid + 256 * u;
          if (e < np) {
            const int r = (2 * e) / Dp, c = 2 * e - r * Dp;
            *reinterpret_cast<double2*>(&sm[r][c]) = t[u];
          }
        }
      }
      __syncthreads();
      for (int r = 0; r < nr; ++r) {
        const double mv = smean[gl][i0 + r];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (jj + 16 * k < Dp) y[k] = __builtin_fma(sm[r][jj + 16 * k], mv, y[k]);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = jj + 16 * k;
      y[k] = j < Dp ? smean[gl][j] : 0.0;
    }
  }
  double b = 0.0, yy = 0.0, rr = 0.0, ll = 0.0;
  bf16_t hs[8], ls[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int j = jj + 16 * k;
    if (j >= Dp) y[k] = 0.0;
    if (j < Dp) b = __builtin_fma(y[k], smean[gl][j], b);
    yy = __builtin_fma(y[k], y[k], yy);
    const float yf = (float)y[k];
    hs[k] = f32_to_bf16(yf);
    ls[k] = f32_to_bf16(yf - bf16_to_f32(hs[k]));
    const double res = (y[k] - (double)bf16_to_f32(hs[k])) - (double)bf16_to_f32(ls[k]);
    rr = __builtin_fma(res, res, rr);
    ll = __builtin_fma((double)bf16_to_f32(ls[k]), (double)bf16_to_f32(ls[k]), ll);
  }
  for (int o = 8; o > 0; o >>= 1) {
    b += __shfl_xor(b, o, 16);
    yy += __shfl_xor(yy, o, 16);
    rr += __shfl_xor(rr, o, 16);
    ll += __shfl_xor(ll, o, 16);
  }
  if (gl >= ng) return;
  const long long go = (long long)bh * a.gstride + g0 + gl;
  const long long yo = go * a.ystride;
  double* yt = a.y64 ? a.y64t + (long long)bh * a.ystride * a.gstride + g0 + gl : nullptr;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int j = jj + 16 * k;
    if (j < Dimg) {
      a.yhi[yo + j] = hs[k];
      a.ylo[yo + j] = ls[k];
      if (a.y64) {
        a.y64[yo + j] = y[k];
        // and dimension-major [Dimg][gstride] per (b,h), read with lanes over centres
        yt[(long long)j * a.gstride] = y[k];
      }
    }
  }
  if (jj == 0) {
    a.ybias[go] = (float)b;
    if (a.c64) a.c64[go] = b;
    if (a.ybound) {
      // fp32 upper bounds; the relative margin covers the roundings above
      const float4 bd = make_float4((float)(sqrt(yy) * (1.0 + 0x1p-20)), (float)(fabs(b) * (1.0 + 0x1p-20)),
                                    (float)(sqrt(rr) * (1.0 + 0x1p-20)), (float)(sqrt(ll) * (1.0 + 0x1p-20)));
      reinterpret_cast<float4*>(a.ybound)[go] = bd;
    }
  }
}

// The same images when a metric is given (query side, Dimg = Dp = DP), on
// fp64 matrix cores: Y (16 centres x DP) = means (16 x DP) . M, one
// v_mfma_f64_16x16x4f64 per 16-dimension column tile and k-step of four
// (layouts as in the key coordinates: A[i][k] in lane i + 16k, B[k][j] in
// lane j + 16k, D[i][j] in lane 16 (i % 4) + j, register i / 4).  Wave w owns
// the column tiles w, w + 4, ...; B fragments come straight from M, which the
// slice mapping keeps in one XCD's L2 for all blocks of a (b,h).  The bias,
// |y|^2 and the split residuals are reduced over a group's 16 lanes, then
// over the four waves in a fixed order.
template <int DP>
__global__ __launch_bounds__(256) void k_centre_images_f64mfma(UpdateArgs a) {
  typedef double f64x4_t __attribute__((ext_vector_type(4)));
  constexpr int GB = 16, NJ = DP / 16, TPW = NJ / 4, KS = DP / 4, LDA = DP + 2, KU = 8;
  static_assert(NJ % 4 == 0, "whole column tiles per wave");
  __shared__ double smean[GB][LDA];
  __shared__ double red[4][GB][4];
  const int nb = (a.G + GB - 1) / GB;
  int bh, blk;
  xcd_slice(blockIdx.x, gridDim.x, nb, bh, blk);
  const int g0 = blk * GB, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lk = lane >> 4;
  const int ng = min(GB, a.G - g0);
  for (int e = tid; e < GB * DP; e += 256) {
    const int gl = e / DP, j = e - gl * DP;
    smean[gl][j] = gl < ng ? a.cmean[((long long)bh * a.gstride + g0 + gl) * a.cstride + j] : 0.0;
  }
  __syncthreads();
  const double* M = a.metric + (long long)bh * DP * DP;
  f64x4_t acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < KS; k0 += KU) {
    double bv[KU][TPW];
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int t = 0; t < TPW; ++t) bv[u][t] = M[(long long)(4 * (k0 + u) + lk) * DP + 16 * (w + 4 * t) + li];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const double av = smean[li][4 * (k0 + u) + lk];
#pragma unroll
      for (int t = 0; t < TPW; ++t) acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv[u][t], acc[t], 0, 0, 0);
    }
  }
  // lane holds groups 4 r + lk (r < 4), dimension 16 (w + 4 t) + li
  double* yt = a.y64t + (long long)bh * a.ystride * a.gstride;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gl = 4 * r + lk;
    const long long go = (long long)bh * a.gstride + g0 + gl;
    double b = 0.0, yy = 0.0, rr = 0.0, ll = 0.0;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int j = 16 * (w + 4 * t) + li;
      const double y = acc[t][r];
      b = __builtin_fma(y, smean[gl][j], b);
      yy = __builtin_fma(y, y, yy);
      const float yf = (float)y;
      const bf16_t hs = f32_to_bf16(yf);
      const bf16_t ls = f32_to_bf16(yf - bf16_to_f32(hs));
      const double res = (y - (double)bf16_to_f32(hs)) - (double)bf16_to_f32(ls);
      rr = __builtin_fma(res, res, rr);
      ll = __builtin_fma((double)bf16_to_f32(ls), (double)bf16_to_f32(ls), ll);
      if (gl < ng) {
        const long long yo = go * a.ystride + j;
        a.yhi[yo] = hs;
        a.ylo[yo] = ls;
        a.y64[yo] = y;
        yt[(long long)j * a.gstride + g0 + gl] = y;
      }
    }
    for (int o = 8; o > 0; o >>= 1) {
      b += __shfl_xor(b, o, 16);
      yy += __shfl_xor(yy, o, 16);
      rr += __shfl_xor(rr, o, 16);
      ll += __shfl_xor(ll, o, 16);
    }
    if (li == 0) {
      red[w][gl][0] = b;
      red[w][gl][1] = yy;
      red[w][gl][2] = rr;
      red[w][gl][3] = ll;
    }
  }
  __syncthreads();
  if (tid >= ng) return;
  double q[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) q[c] = ((red[0][tid][c] + red[1][tid][c]) + red[2][tid][c]) + red[3][tid][c];
  const long long go = (long long)bh * a.gstride + g0 + tid;
  a.ybias[go] = (float)q[0];
  a.c64[go] = q[0];
  if (a.ybound) {
    // fp32 upper bounds; the relative margin covers the roundings above
    const float4 bd = make_float4((float)(sqrt(q[1]) * (1.0 + 0x1p-20)), (float)(fabs(q[0]) * (1.0 + 0x1p-20)),
                                  (float)(sqrt(q[2]) * (1.0 + 0x1p-20)), (float)(sqrt(q[3]) * (1.0 + 0x1p-20)));
    reinterpret_cast<float4*>(a.ybound)[go] = bd;
  }
}

// M_Q = s^2 sum over non-empty key groups of cbar_h cbar_h^T (d x d per (b,h));
// 16 key groups at a time are staged in LDS, each thread owns a 4x4 block.
// Centred query coordinates u_i - mean_h(u_ih) have the metric
// s^2 sum_h (cbar_h - m)(cbar_h - m)^T with m the mean of the non-empty
// centres, so the centres are centred before the outer products.
__global__ __launch_bounds__(256) void k_query_metric(QMetricArgs a) {
  constexpr int HB = 16, NT = 256, PER = HB * 128 / NT;
  __shared__ double cs[2][HB][128];  // two stages: one barrier per stage
  __shared__ double cmean[128];
  __shared__ unsigned char ne[kMaxGroups];
  const int bh = blockIdx.y, d = a.d, tid = threadIdx.x;
  const double* cb = a.cbar + (long long)bh * a.GK * d;
  const int* off = a.off_k + (long long)bh * (a.GK + 1);
  for (int h = tid; h < a.GK; h += NT) ne[h] = off[h + 1] > off[h] ? 1 : 0;
  __syncthreads();
  if (tid < d) {
    double sm = 0.0;
    int cnt = 0;
    if (a.centred)
      for (int h = 0; h < a.GK; ++h)
        if (ne[h]) {
          sm += cb[(long long)h * d + tid];
          ++cnt;
        }
    cmean[tid] = cnt > 0 ? sm / (double)cnt : 0.0;
  }
  const int nb = d / 4;  // 4x4 blocks per row of blocks
  const int blk = blockIdx.x * NT + tid;  // (d/4)^2 / 256 workgroups per (b,h), one band of block rows each
  const int bi = blk / nb, bj = blk - (blk / nb) * nb;
  const bool act = bi < nb;
  double acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.0;
  // the next stage's centres are loaded into registers while the current
  // stage is multiplied
  double pre[PER];
  auto load = [&](int h0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + NT * u, hl = e / d, j = e - (e / d) * d;
      const int h = h0 + hl;
      pre[u] = (hl < HB && h < a.GK && ne[h]) ? cb[(long long)h * d + j] : 0.0;
    }
  };
  load(0);
  __syncthreads();  // cmean
  int buf = 0;
  for (int h0 = 0; h0 < a.GK; h0 += HB, buf ^= 1) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + NT * u, hl = e / d, j = e - (e / d) * d;
      if (hl < HB) cs[buf][hl][j] = (h0 + hl < a.GK && ne[h0 + hl]) ? pre[u] - cmean[j] : 0.0;
    }
    __syncthreads();
    if (h0 + HB < a.GK) load(h0 + HB);
    if (act) {
      for (int hl = 0; hl < HB; ++hl) {
        double u[4], v[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          u[x] = cs[buf][hl][4 * bi + x];
          v[x] = cs[buf][hl][4 * bj + x];
        }
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 4; ++y) acc[x][y] += u[x] * v[y];
      }
    }
  }
  if (!act) return;
  const double s2 = (double)a.scale * (double)a.scale;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) a.mq[(long long)bh * d * d + (4 * bi + x) * d + 4 * bj + y] = s2 * acc[x][y];
}

// ============================================================================
// a9: gather Q, K, V into group-contiguous order; key-group id per position.
// For bf16 inputs V is stored as fp16 scaled by a per-(b,h) power of two 2^-k
// (k from max |v|, so the largest value lands in [2^14, 2^15)): the P.V
// product then runs with 11-bit fp16 operands and the scale is undone exactly
// in the epilogue.
// ============================================================================
__global__ __launch_bounds__(256) void k_zero_u32(uint32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <typename T>
__global__ __launch_bounds__(256) void k_vmax(View4 v, int N, int d, uint32_t* vmax) {
  __shared__ float red[4];
  const int bh = blockIdx.y;
  constexpr int VEC = 16 / sizeof(T);
  const int cpr = d / VEC;
  const long long total = (long long)N * cpr;
  float m = 0.f;
  // four 16-byte loads in flight per thread
  const long long stride = (long long)gridDim.x * 256;
  for (long long e0 = (long long)blockIdx.x * 256 + threadIdx.x; e0 < total; e0 += 4 * stride) {
    uint4 u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const long long e = e0 + q * stride;
      u[q] = make_uint4(0, 0, 0, 0);
      if (e < total) {
        const int row = (int)(e / cpr), c = (int)(e - (e / cpr) * cpr) * VEC;
        u[q] = *reinterpret_cast<const uint4*>(static_cast<const T*>(v.p) + v.row_off(bh, row) + c);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const T* ev = reinterpret_cast<const T*>(&u[q]);
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float x = fabsf(Elem<T>::load(ev + j));
        m = (x > m || x != x) ? x : m;
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float t = __shfl_xor(m, o, 64);
    m = (t > m || t != t) ? t : m;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) m = (red[w] > m || red[w] != red[w]) ? red[w] : m;
    atomicMax(vmax + bh, __float_as_uint(m));
  }
}

__device__ inline int v_exponent(uint32_t bits) {
  const float mx = __uint_as_float(bits);
  if (!(mx > 0.f) || !(mx < INFINITY)) return 0;
  int e;
  frexpf(mx, &e);  // mx = m 2^e, m in [0.5, 1)
  return e - 15;
}

template <typename T>
__global__ __launch_bounds__(256) void k_gather(GatherArgs a) {
  const int bh = blockIdx.y;
  constexpr int VEC = 16 / sizeof(T);
  const int cpr = a.d / VEC;  // 16-byte chunks per row
  const int rows_per_blk = 256 / cpr;
  const int r = threadIdx.x / cpr, c = threadIdx.x - (threadIdx.x / cpr) * cpr;
  const int pos = blockIdx.x * rows_per_blk + r;
  const bool vf16 = a.vmax != nullptr;
  const int vk = vf16 ? v_exponent(a.vmax[bh]) : 0;
  if (vf16 && blockIdx.x == 0 && threadIdx.x == 0) a.vexp[bh] = vk;
  if (pos >= a.N) return;
  const long long dst = ((long long)bh * a.N + pos) * a.d + c * VEC;
  const int tk = a.perm_k[(long long)bh * a.N + pos];
  *reinterpret_cast<uint4*>(static_cast<T*>(a.kp) + dst) =
      *reinterpret_cast<const uint4*>(static_cast<const T*>(a.k.p) + a.k.row_off(bh, tk) + c * VEC);
  const uint4 vv = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.v.p) + a.v.row_off(bh, tk) + c * VEC);
  if (vf16) {
    const float sc = ldexpf(1.0f, -vk);
    const bf16_t* e = reinterpret_cast<const bf16_t*>(&vv);
    f16x8 h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = (_Float16)(bf16_to_f32(e[j]) * sc);
    *reinterpret_cast<f16x8*>(static_cast<bf16_t*>(a.vp) + dst) = h;
  } else {
    *reinterpret_cast<uint4*>(static_cast<T*>(a.vp) + dst) = vv;
  }
  if (c == 0) a.kgroup[(long long)bh * a.N + pos] = a.kv_labels[(long long)bh * a.N + tk];
}

// ============================================================================
// launchers
// ============================================================================
#define SP_LAUNCH(k, g, b, s, ...)                                   \
  do {                                                               \
    hipLaunchKernelGGL(k, g, b, 0, s, __VA_ARGS__);                  \
    hipError_t e_ = hipGetLastError();                               \
    if (e_ != hipSuccess) return e_;                                 \
  } while (0)

#define SP_LAUNCH_FN(fn, g, b, s, arg)                               \
  do {                                                               \
    void* args_[] = {(void*)&(arg)};                                 \
    hipError_t e_ = hipLaunchKernel(fn, g, b, args_, 0, s);          \
    if (e_ != hipSuccess) return e_;                                 \
  } while (0)

// workgroups of `fn` (with `threads` threads) resident at once on the current
// device, cached per device and kernel
static long long resident_slots(const void* fn, int threads) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, long long> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find({dev, fn});
  if (it != cache.end()) return it->second;
  int per_cu = 0, ncu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess) per_cu = 1;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) ncu = 256;
  const long long v = (long long)std::max(1, per_cu) * std::max(1, ncu);
  cache[{dev, fn}] = v;
  return v;
}

hipError_t launch_sample_metric(const Plan& p, hipStream_t s) {
  SampleArgs a{p.q, p.N, p.Ms, p.bh0, p.seed, p.sample, p.mk};
  SP_LAUNCH(k_query_sample, dim3(p.BH), dim3(256), s, a);
  if (p.dtype == SPARSEPR_BF16) {
    if (p.d == 128) SP_LAUNCH((k_key_metric64<bf16_t, 128>), dim3(4, p.BH), dim3(256), s, a);
    else SP_LAUNCH((k_key_metric64<bf16_t, 64>), dim3(1, p.BH), dim3(256), s, a);
  } else {
    if (p.d == 128) SP_LAUNCH((k_key_metric64<float, 128>), dim3(4, p.BH), dim3(256), s, a);
    else SP_LAUNCH((k_key_metric64<float, 64>), dim3(1, p.BH), dim3(256), s, a);
  }
  return hipSuccess;
}

hipError_t launch_key_eig(const Plan& p, hipStream_t s, bool all_eigenvalues) {
  // the call itself needs only the leading rK eigenpairs; the whole spectrum
  // is computed when it is reported
  EigArgs a{p.mk, p.eigval, p.kmap, p.kmap_pad, p.eigz, p.rK, p.rKpad, p.scale, all_eigenvalues ? p.d : p.rK};
  if (p.d == 128) SP_LAUNCH((k_key_eig<128, 512>), dim3(p.BH), dim3(512), s, a);
  else SP_LAUNCH((k_key_eig<64, 1024>), dim3(p.BH), dim3(1024), s, a);
  return hipSuccess;
}

template <typename T, int D>
static hipError_t launch_key_coords_t(const Plan& p, const CoordArgs& a, hipStream_t s) {
  const dim3 g((p.N + 255) / 256, p.BH);
  switch (p.rKpad) {
    case 16: SP_LAUNCH((k_key_coords_f64mfma<T, D, 16>), g, dim3(256), s, a); break;
    case 32: SP_LAUNCH((k_key_coords_f64mfma<T, D, 32>), g, dim3(256), s, a); break;
    case 48: SP_LAUNCH((k_key_coords64<T, D, 48>), g, dim3(256), s, a); break;
    case 64: SP_LAUNCH((k_key_coords64<T, D, 64>), g, dim3(256), s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

hipError_t launch_key_coords(const Plan& p, hipStream_t s) {
  CoordArgs a{p.k, p.kmap_pad, p.N, p.rK, p.rKpad, p.z64, p.zhi, p.zlo, p.xbound};
  if (p.dtype == SPARSEPR_BF16)
    return p.d == 128 ? launch_key_coords_t<bf16_t, 128>(p, a, s) : launch_key_coords_t<bf16_t, 64>(p, a, s);
  return p.d == 128 ? launch_key_coords_t<float, 128>(p, a, s) : launch_key_coords_t<float, 64>(p, a, s);
}

hipError_t launch_split_rows(const Plan& p, const View4& x, hipStream_t s) {
  SplitArgs a{x, p.N, p.d, p.phi, p.plo};
  dim3 g((unsigned)(((long long)p.N * p.d + 255) / 256), p.BH);
  SP_LAUNCH(k_split_rows, g, dim3(256), s, a);
  return hipSuccess;
}

hipError_t launch_assign(const Plan& p, const AssignArgs& args, int D, bool lo, hipStream_t s) {
  if (args.G < 1 || args.G > kMaxGroups) return hipErrorInvalidValue;
  if (D == 128 && !lo && args.G <= 256) {
    // resident centres; chunks per workgroup: the workgroups of one round
    // over the GPU's resident slots share the chunks as evenly as whole
    // chunks allow
    AssignArgs a = args;
    const void* fn = (const void*)k_kmeans_assign<128>;
    const long long slots = resident_slots(fn, 512);
    const long long per_bh = std::max(1LL, slots / p.BH);
    a.cpw = (int)std::max(1LL, (p.nchunk + per_bh - 1) / per_bh);
    const dim3 g((unsigned)((p.nchunk + a.cpw - 1) / a.cpw), p.BH);
    SP_LAUNCH_FN(fn, g, dim3(512), s, a);
    return hipSuccess;
  }
  // staged centres, one workgroup per histogram chunk
  const dim3 g(p.nchunk, p.BH), b(512);
  if (D == 16) {
    if (lo) SP_LAUNCH((k_kmeans_assign_staged<16, true, 256>), g, b, s, args);
    else SP_LAUNCH((k_kmeans_assign_staged<16, false, 256>), g, b, s, args);
  } else if (D == 32) {
    if (lo) SP_LAUNCH((k_kmeans_assign_staged<32, true, 256>), g, b, s, args);
    else SP_LAUNCH((k_kmeans_assign_staged<32, false, 256>), g, b, s, args);
  } else if (D == 48) {
    if (lo) SP_LAUNCH((k_kmeans_assign_staged<48, true, 256>), g, b, s, args);
    else SP_LAUNCH((k_kmeans_assign_staged<48, false, 256>), g, b, s, args);
  } else if (D == 64) {
    if (lo) SP_LAUNCH((k_kmeans_assign_staged<64, true, 128>), g, b, s, args);
    else SP_LAUNCH((k_kmeans_assign_staged<64, false, 128>), g, b, s, args);
  } else if (D == 128) {
    if (lo) SP_LAUNCH((k_kmeans_assign_staged<128, true, 128>), g, b, s, args);
    else SP_LAUNCH((k_kmeans_assign_staged<128, false, 128>), g, b, s, args);
  } else {
    return hipErrorInvalidValue;
  }
  return hipSuccess;
}

hipError_t launch_redecide(const Plan& p, const RedecideArgs& a, int raw_type, hipStream_t s) {
  if (a.Dx < 1 || a.Dx > 128) return hipErrorInvalidValue;
  // enough workgroups per (b,h) that a step's flagged points (typically well
  // under 2% of N) take one or two batches each
  // (the workgroups of one (b,h) on one XCD: they all read its centre images)
  RedecideArgs ra = a;
  ra.nwg = std::max(1, std::min(32, (p.N + 1023) / 1024));  // four points at a time each
  const dim3 g((unsigned)(ra.nwg * p.BH));
  if (raw_type == 0) SP_LAUNCH(k_kmeans_redecide<bf16_t>, g, dim3(256), s, ra);
  else SP_LAUNCH(k_kmeans_redecide<float>, g, dim3(256), s, ra);
  return hipSuccess;
}

hipError_t launch_mfma_rounding(const float* pats, int n, float* out, hipStream_t s) {
  SP_LAUNCH(k_mfma_rounding, dim3(n), dim3(64), s, pats, n, out);
  return hipSuccess;
}

hipError_t launch_count_labels(const Plan& p, const CountArgs& a, hipStream_t s) {
  SP_LAUNCH(k_count_labels, dim3(p.nchunk, p.BH), dim3(256), s, a);
  return hipSuccess;
}

hipError_t launch_group_scan(const Plan& p, const ScanArgs& a, hipStream_t s) {
  SP_LAUNCH(k_group_scan, dim3(p.BH), dim3(1024), s, a);
  return hipSuccess;
}

hipError_t launch_group_scatter(const Plan& p, const ScatterArgs& a, hipStream_t s) {
  SP_LAUNCH(k_group_scatter, dim3(p.nchunk, p.BH), dim3(256), s, a);
  return hipSuccess;
}

hipError_t launch_centre_update(const Plan& p, const UpdateArgs& a, int pts_type, hipStream_t s) {
  dim3 g(a.G, p.BH);
  if (pts_type == 0) SP_LAUNCH(k_group_mean<bf16_t>, g, dim3(256), s, a);
  else if (pts_type == 1) SP_LAUNCH(k_group_mean<float>, g, dim3(256), s, a);
  else SP_LAUNCH(k_group_mean<double>, g, dim3(256), s, a);
  if (a.means_only) return hipSuccess;
  const unsigned nb = (unsigned)((a.G + 15) / 16);
  if (a.metric && a.y64 && a.y64t && a.c64 && a.Dimg == a.Dp && (a.Dp == 128 || a.Dp == 64)) {
    if (a.Dp == 128) SP_LAUNCH(k_centre_images_f64mfma<128>, dim3(nb * p.BH), dim3(256), s, a);
    else SP_LAUNCH(k_centre_images_f64mfma<64>, dim3(nb * p.BH), dim3(256), s, a);
    return hipSuccess;
  }
  SP_LAUNCH(k_centre_images, dim3(nb, p.BH), dim3(256), s, a);
  return hipSuccess;
}

hipError_t launch_query_metric(const Plan& p, hipStream_t s) {
  QMetricArgs a{p.cbar, p.off_k, p.GK, p.d, p.scale, p.centred_qc, p.mq};
  SP_LAUNCH(k_query_metric, dim3((unsigned)((p.d / 4) * (p.d / 4) / 256), p.BH), dim3(256), s, a);
  return hipSuccess;
}

hipError_t launch_vmax(const Plan& p, hipStream_t s) {
  if (p.dtype != SPARSEPR_BF16) return hipSuccess;
  SP_LAUNCH(k_zero_u32, dim3((p.BH + 255) / 256), dim3(256), s, p.vmax, p.BH);
  SP_LAUNCH(k_vmax<bf16_t>, dim3(64, p.BH), dim3(256), s, p.v, p.N, p.d, p.vmax);
  return hipSuccess;
}

hipError_t launch_gather(const Plan& p, hipStream_t s) {
  const bool vf16 = p.dtype == SPARSEPR_BF16;
  if (vf16) {
    hipError_t e = launch_vmax(p, s);
    if (e != hipSuccess) return e;
  }
  GatherArgs a{p.k, p.v, vf16 ? p.vmax : nullptr, p.vexp, p.perm_k, p.kv_labels, p.kp, p.vp,
               p.kgroup, p.N, p.d};
  const int vec = 16 / p.esize;
  const int rows_per_blk = 256 / (p.d / vec);
  dim3 g((p.N + rows_per_blk - 1) / rows_per_blk, p.BH);
  if (p.dtype == SPARSEPR_BF16) SP_LAUNCH(k_gather<bf16_t>, g, dim3(256), s, a);
  else SP_LAUNCH(k_gather<float>, g, dim3(256), s, a);
  return hipSuccess;
}

}  // namespace sp
