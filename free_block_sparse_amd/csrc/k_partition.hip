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
// a1: query sample (partial Fisher-Yates on splitmix64) and M_K
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
template <typename T, int D>
__global__ __launch_bounds__(256) void k_sample_metric(SampleArgs a) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  __shared__ int tgt[256];
  __shared__ int held[256];  // value slot j held when step j ran
  __shared__ int lnk[256];
  __shared__ int srt[256];
  constexpr int QLD = 256 + 8;  // samples per dimension row (+8: 16-byte rows off the bank stride)
  __shared__ __align__(16) bf16_t qt[std::is_same<T, bf16_t>::value ? D * QLD : 8];
  __shared__ float qs[std::is_same<T, bf16_t>::value ? 1 : 64][D + 1];
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

  const float inv = 1.0f / (float)Ms;
  float* mk = a.mk + (long long)bh * D * D;
  const T* qbase = static_cast<const T*>(a.q.p);
  if constexpr (std::is_same<T, bf16_t>::value) {
    // bf16 rows: M_K on the matrix cores.  The sampled rows are staged
    // transposed (dimension-major, samples zero-padded to a multiple of 16),
    // so both MFMA operands are 16-byte LDS reads; bf16 products are exact
    // and accumulate in fp32.
    const int Mp = (Ms + 15) & ~15;
    constexpr int CPR = D / 8;  // 16-byte pieces per row
    for (int e = tid; e < Mp * CPR; e += 256) {
      const int c = (e / Mp) * 8, r = e - (e / Mp) * Mp;  // consecutive threads: consecutive samples
      uint4 u = make_uint4(0, 0, 0, 0);
      if (r < Ms) u = *reinterpret_cast<const uint4*>(qbase + a.q.row_off(bh, srt[r]) + c);
      const bf16_t* ev = reinterpret_cast<const bf16_t*>(&u);
#pragma unroll
      for (int j = 0; j < 8; ++j) qt[(c + j) * QLD + r] = ev[j];
    }
    __syncthreads();
    const int w = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
    constexpr int NB = D / 32;  // 32 x 32 output blocks per side
    for (int blk = w; blk < NB * NB; blk += 4) {
      const int bi = blk / NB, bj = blk - (blk / NB) * NB;
      f32x16 acc = {};
      for (int k0 = 0; k0 < Mp; k0 += 16) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(qt + (32 * bi + col) * QLD + k0 + 8 * half);
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(qt + (32 * bj + col) * QLD + k0 + 8 * half);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
      }
      // D[i][j]: j = lane % 32, i = (r & 3) + 8 (r >> 2) + 4 (lane / 32)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = (r & 3) + 8 * (r >> 2) + 4 * half;
        mk[(32 * bi + i) * D + 32 * bj + col] = acc[r] * inv;
      }
    }
  } else {
    constexpr int TB = D / 16;
    const int i0 = (tid >> 4) * TB, j0 = (tid & 15) * TB;
    float acc[TB][TB];
#pragma unroll
    for (int x = 0; x < TB; ++x)
#pragma unroll
      for (int y = 0; y < TB; ++y) acc[x][y] = 0.f;
    for (int c0 = 0; c0 < Ms; c0 += 64) {
      const int nr = min(64, Ms - c0);
      __syncthreads();
      for (int e = tid; e < nr * D; e += 256) {
        const int r = e / D, col = e - (e / D) * D;
        qs[r][col] = Elem<T>::load(qbase + a.q.row_off(bh, srt[c0 + r]) + col);
      }
      __syncthreads();
      for (int r = 0; r < nr; ++r) {
        float xi[TB], xj[TB];
#pragma unroll
        for (int t2 = 0; t2 < TB; ++t2) {
          xi[t2] = qs[r][i0 + t2];
          xj[t2] = qs[r][j0 + t2];
        }
#pragma unroll
        for (int x = 0; x < TB; ++x)
#pragma unroll
          for (int y = 0; y < TB; ++y) acc[x][y] += xi[x] * xj[y];
      }
    }
#pragma unroll
    for (int x = 0; x < TB; ++x)
#pragma unroll
      for (int y = 0; y < TB; ++y) mk[(i0 + x) * D + j0 + y] = acc[x][y] * inv;
  }
}

// ============================================================================
// a2: symmetric eigensolver for M_K (one workgroup per (b,h), all in LDS)
// ============================================================================
template <int D>
__global__ __launch_bounds__(1024) void k_key_eig(EigArgs a) {
  constexpr int LD = D + 1;  // odd row stride: column walks hit distinct banks
  constexpr int NT = 1024;
  __shared__ float A[D * LD];
  __shared__ float Z[D * LD];
  __shared__ float dg[D + 2], eo[D + 2], tau[D], vb[D], pb[D];
  __shared__ float rot[4 * D];
  __shared__ int ctl[8];
  __shared__ int top[D];
  __shared__ float lamv[D];  // eigenvalue of column i of Z
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* mk = a.mk + (long long)bh * D * D;
  {
    float t[D * D / NT];
#pragma unroll
    for (int u = 0; u < D * D / NT; ++u) t[u] = mk[tid + NT * u];
#pragma unroll
    for (int u = 0; u < D * D / NT; ++u) {
      const int e = tid + NT * u, i = e / D, j = e - (e / D) * D;
      A[i * LD + j] = t[u];
    }
  }
  __syncthreads();
  const EigWork<float> w{A, LD, Z, LD, dg, eo, tau, vb, pb, rot, ctl};
  eig_tridiagonalize<float, NT>(w, D);
  // every eigenvalue by multisection (all of them are reported), vectors
  // of the leading rK by twisted factorisations; shifted QR when two of the
  // leading eigenvalues cannot be told apart
  eig_bisect<float, NT>(w, D, D);
  for (int i = tid; i < D; i += NT) lamv[i] = rot[D + i];
  __syncthreads();
  if (eig_twisted<float, NT>(w, D, a.rK)) {
    for (int i = tid; i < D; i += NT) {
      if (a.eigval) a.eigval[(long long)bh * D + i] = lamv[i];
      if (i < a.rK) top[i] = i;
    }
  } else {
    eig_tridiagonal_qr<float, NT>(w, D);
    // rank eigenvalues (descending, ties by index)
    for (int i = tid; i < D; i += NT) {
      const float li = dg[i];
      int rank = 0;
      for (int j = 0; j < D; ++j) {
        const float lj = dg[j];
        rank += (lj > li) || (lj == li && j < i);
      }
      if (a.eigval) a.eigval[(long long)bh * D + rank] = li;
      if (rank < a.rK) top[rank] = i;
      lamv[i] = li;
    }
  }
  __syncthreads();
  eig_back_transform<float, NT, 32>(w, D, top, a.rK);
  // coordinate map: column k of kmap = s sqrt(lambda_k) u_k
  float* km = a.kmap + (long long)bh * D * a.rK;
  for (int e = tid; e < D * a.rK; e += NT) {
    const int r = e / D, k = e - (e / D) * D;
    const int i = top[r];
    const float f = a.scale * sqrtf(fmaxf(lamv[i], 0.f));
    km[k * a.rK + r] = f * Z[k * LD + i];
  }
}

// ============================================================================
// a3: key-response coordinates z = K kmap (fp32), stored also as hi/lo bf16
// ============================================================================
template <typename T, int D>
__global__ __launch_bounds__(256) void k_key_coords(CoordArgs a) {
  __shared__ float km[D][64];
  __shared__ float kr[64][D + 1];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int n0 = blockIdx.x * 64;
  const int rK = a.rK, rKpad = a.rKpad, N = a.N;
  const float* kmap = a.kmap + (long long)bh * D * rK;
  for (int e = tid; e < D * rK; e += 256) km[e / rK][e % rK] = kmap[e];
  const T* kb = static_cast<const T*>(a.k.p);
  constexpr int VEC = 16 / sizeof(T);
  for (int e = tid; e < 64 * (D / VEC); e += 256) {
    const int r = e / (D / VEC), c = (e - (e / (D / VEC)) * (D / VEC)) * VEC;
    const int n = n0 + r;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (n < N) u = *reinterpret_cast<const uint4*>(kb + a.k.row_off(bh, n) + c);
    const T* ev = reinterpret_cast<const T*>(&u);
#pragma unroll
    for (int j = 0; j < VEC; ++j) kr[r][c + j] = n < N ? Elem<T>::load(ev + j) : 0.f;
  }
  __syncthreads();
  const int r = tid >> 2;
  const int n = n0 + r;
  if (n >= N) return;
  const long long zrow = (long long)bh * N + n;
  for (int j = tid & 3; j < rKpad; j += 4) {
    float acc = 0.f;
    if (j < rK)
      for (int c = 0; c < D; ++c) acc += kr[r][c] * km[c][j];
    a.z32[zrow * rKpad + j] = acc;
    const bf16_t hi = f32_to_bf16(acc);
    a.zhi[zrow * rKpad + j] = hi;
    a.zlo[zrow * rKpad + j] = f32_to_bf16(acc - bf16_to_f32(hi));
  }
}

// bf16 keys on the matrix cores: z^T = kmap^T K^T with kmap split into three
// bf16 pieces (24 significant bits, like fp32); products with bf16 keys are
// exact and accumulate in fp32.  Each wave takes 32-token blocks; lanes hold
// the map as the A operand for up to two blocks of 32 coordinates.
template <int D, int NCB>
__global__ __launch_bounds__(256) void k_key_coords_mfma(CoordArgs a) {
  constexpr int KS = D / 16;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int rK = a.rK, rKpad = a.rKpad, N = a.N;
  const int ncb = (rK + 31) / 32;
  const float* kmap = a.kmap + (long long)bh * D * rK;
  bf16x8 mp[3][NCB][KS];  // NCB 32-coordinate blocks (r_K <= 32 NCB)
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16_t pv[3][8];
      const int cc = 32 * cb + col;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x = (cb < ncb && cc < rK) ? kmap[(16 * ks + 8 * half + j) * rK + cc] : 0.f;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          pv[q][j] = f32_to_bf16(x);
          x -= bf16_to_f32(pv[q][j]);
        }
      }
#pragma unroll
      for (int q = 0; q < 3; ++q) mp[q][cb][ks] = *reinterpret_cast<const bf16x8*>(pv[q]);
    }
  const bf16_t* kb = static_cast<const bf16_t*>(a.k.p);
  // each wave covers 8 consecutive 32-token blocks (the map fragments above
  // are built once per wave)
  for (int blk = 0; blk < 8; ++blk) {
    const int n0 = blockIdx.x * 1024 + 256 * w + 32 * blk;
    if (n0 >= N) break;
    const int n = n0 + col;
    bf16x8 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (n < N) u = *reinterpret_cast<const uint4*>(kb + a.k.row_off(bh, n) + 16 * ks + 8 * half);
      kf[ks] = __builtin_bit_cast(bf16x8, u);
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      if (cb >= ncb) break;
      f32x16 acc = {};
      // smallest pieces first
#pragma unroll
      for (int q = 2; q >= 0; --q)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mp[q][cb][ks], kf[ks], acc, 0, 0, 0);
      if (n >= N) continue;
      const long long zrow = ((long long)bh * N + n) * rKpad;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 32 * cb + 8 * q + 4 * half;  // coordinates c..c+3 of token n
        if (c >= rKpad) continue;
        const float4 zf = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
        uint2 hp, lp;
        hp.x = pack_bf16x2(zf.x, zf.y);
        hp.y = pack_bf16x2(zf.z, zf.w);
        lp.x = pack_bf16x2(zf.x - __uint_as_float(hp.x << 16), zf.y - __uint_as_float(hp.x & 0xffff0000u));
        lp.y = pack_bf16x2(zf.z - __uint_as_float(hp.y << 16), zf.w - __uint_as_float(hp.y & 0xffff0000u));
        *reinterpret_cast<float4*>(a.z32 + zrow + c) = zf;
        *reinterpret_cast<uint2*>(a.zhi + zrow + c) = hp;
        *reinterpret_cast<uint2*>(a.zlo + zrow + c) = lp;
      }
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
// Largest of the 16 accumulator values a lane holds for a 32-centre block
// (register r belongs to centre (r&3) + 8(r>>2) + 4*half, increasing in r).
// Pairwise tree (depth 4); on ties the lower register, i.e. the lower centre
// index, is kept.  Returns the value and writes the register index.
__device__ inline float block_argmax16(const f32x16& acc, int* ridx) {
  float v[16];
  int id[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    v[r] = acc[r];
    id[r] = r;
  }
#pragma unroll
  for (int w = 1; w < 16; w <<= 1)
#pragma unroll
    for (int r = 0; r < 16; r += 2 * w) {
      const bool right = v[r + w] > v[r];
      v[r] = right ? v[r + w] : v[r];
      id[r] = right ? id[r + w] : id[r];
    }
  *ridx = id[0];
  return v[0];
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
    // -c_g / 2, the accumulators' start (centres past G never win)
    for (int e = tid; e < G32; e += NT) sbias[e] = e < G ? -0.5f * a.ybias[(long long)bh * a.gstride + e] : -INFINITY;
  }
  __syncthreads();

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
    float best[PB];
    int bidx[PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      best[pb] = -INFINITY;
      bidx[pb] = 0;
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
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) {
        int rr;
        const float sc = block_argmax16(acc[pb], &rr);
        if (sc > best[pb]) {
          best[pb] = sc;
          bidx[pb] = cb + (rr & 3) + 8 * (rr >> 2) + 4 * half;
        }
      }
    }
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      const float ob = __shfl_xor(best[pb], 32, 64);
      const int oi = __shfl_xor(bidx[pb], 32, 64);
      if (ob > best[pb] || (ob == best[pb] && oi < bidx[pb])) bidx[pb] = oi;
      const int n = n_begin + BP * b + 32 * pb + col;
      if (half == 0 && n < n_end) {
        a.labels[(long long)bh * N + n] = bidx[pb];
        atomicAdd(cnt + (long long)(n / kChunk) * a.gstride + bidx[pb], 1);
      }
    }
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ph[pb][ks] = nh[pb][ks];
  }
#undef SP_LOAD_BLOCK
}

template <int D, bool LO, int CG>
__global__ __launch_bounds__(512, 4) void k_kmeans_assign_staged(AssignArgs a) {
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
  float best = -INFINITY;
  int bidx = 0;
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
    for (int e = tid; e < CG; e += NT) sbias[e] = (c0 + e < G) ? -0.5f * yb[c0 + e] : -INFINITY;
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
      int rr;
      float sc = block_argmax16(acc0, &rr);
      if (sc > best) {
        best = sc;
        bidx = c0 + cb + (rr & 3) + 8 * (rr >> 2) + 4 * half;
      }
      if (two) {
        sc = block_argmax16(acc1, &rr);
        if (sc > best) {
          best = sc;
          bidx = c0 + cb + 32 + (rr & 3) + 8 * (rr >> 2) + 4 * half;
        }
      }
    }
  }
  {
    const float ob = __shfl_xor(best, 32, 64);
    const int oi = __shfl_xor(bidx, 32, 64);
    if (ob > best || (ob == best && oi < bidx)) {
      best = ob;
      bidx = oi;
    }
  }
  __syncthreads();
  if (half == 0 && n < N) {
    a.labels[(long long)bh * N + n] = bidx;
    atomicAdd(&hist[bidx], 1);
  }
  __syncthreads();
  int* cnt = a.counts + ((long long)bh * a.nchunk + blk) * a.gstride;
  for (int g = tid; g < G; g += NT) cnt[g] = hist[g];
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
  // loads eight at a time, so they are in flight together
  int sum = 0;
  int c = c0;
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
  int c2 = c0;
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
// of its chunk with the same label.  Inside a wave, lanes with equal labels
// are matched with one ballot per distinct label; earlier waves contribute
// their per-label counts.
__global__ __launch_bounds__(256) void k_group_scatter(ScatterArgs a) {
  __shared__ int hist[4][kMaxGroups];
  const int bh = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  for (int e = tid; e < 4 * a.gstride; e += 256) hist[e / a.gstride][e % a.gstride] = 0;
  __syncthreads();
  const int n = chunk * kChunk + tid;
  const int my = n < a.N ? a.labels[(long long)bh * a.N + n] : -1;
  const unsigned long long lt = (1ull << lane) - 1ull;
  unsigned long long todo = __builtin_amdgcn_ballot_w64(my >= 0);
  int rank = 0;
  while (todo) {
    const int leader = __builtin_ctzll(todo);
    const int lab = __builtin_amdgcn_readlane(my, leader);
    const unsigned long long m = __builtin_amdgcn_ballot_w64(my == lab);
    if (my == lab) {
      rank = __builtin_popcountll(m & lt);
      if (lane == leader) hist[w][lab] = __builtin_popcountll(m);
    }
    todo &= ~m;
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
    return;
  }
  const int* off = a.off + (long long)bh * a.offstride;
  const int* perm = a.perm + (long long)bh * a.N;
  const int a0 = off[g], a1 = off[g + 1];
  const int n_g = a1 - a0;
  double s = 0.0;
  if (a.means_out) {
    // Means handed to the router: rows summed one after another in ascending
    // token order, as the reference computation does (one thread per dim).
    if (tid < Dp) {
      int r = a0;
      for (; r + 7 < a1; r += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = Elem<TP>::load(xb + a.pts.row_off(bh, perm[r + u]) + tid);
#pragma unroll
        for (int u = 0; u < 8; ++u) s = __dadd_rn(s, (double)v[u]);
      }
      for (; r < a1; ++r) s = __dadd_rn(s, (double)Elem<TP>::load(xb + a.pts.row_off(bh, perm[r]) + tid));
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
      int r = a0 + pt;
      for (; r + 3 * P < a1; r += 4 * P) {
        uint4 u[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          u[k] = *reinterpret_cast<const uint4*>(xb + a.pts.row_off(bh, perm[r + k * P]) + c * VEC);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const TP* ev = reinterpret_cast<const TP*>(&u[k]);
#pragma unroll
          for (int q = 0; q < VEC; ++q) acc[q] = __dadd_rn(acc[q], (double)Elem<TP>::load(ev + q));
        }
      }
      for (; r < a1; r += P) {
        const uint4 u = *reinterpret_cast<const uint4*>(xb + a.pts.row_off(bh, perm[r]) + c * VEC);
        const TP* ev = reinterpret_cast<const TP*>(&u);
#pragma unroll
        for (int q = 0; q < VEC; ++q) acc[q] = __dadd_rn(acc[q], (double)Elem<TP>::load(ev + q));
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

// centre update, step 2: image y = M mean (or the mean itself), stored as a
// hi/lo bf16 pair, and bias mean . y (fp64 accumulation).
// 16 groups per workgroup; 16 threads per group, each owning 8 consecutive
// dimensions; M is staged through LDS 32 rows at a time.
__global__ __launch_bounds__(256) void k_centre_images(UpdateArgs a) {
  constexpr int GB = 16, MR = 32;
  __shared__ double smean[GB][129];
  __shared__ __attribute__((aligned(16))) float sm[MR][132];
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
  // thread (group gl, piece jj) owns dims 8 jj .. 8 jj + 7
  const int gl = tid >> 4, jj = tid & 15;
  const float* M = a.metric ? a.metric + (long long)bh * Dp * Dp : nullptr;
  double y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = 0.0;
  __syncthreads();
  if (M) {
    for (int i0 = 0; i0 < Dp; i0 += MR) {
      const int nr = min(MR, Dp - i0);
      __syncthreads();
      if ((Dp & 3) == 0) {
        // float4 pieces, up to four per thread in flight together
        const int np = nr * Dp / 4;
        float4 t[MR * 128 / 4 / 256];
#pragma unroll
        for (int u = 0; u < MR * 128 / 4 / 256; ++u) {
          const int e = tid + 256 * u;
          if (e < np) t[u] = *reinterpret_cast<const float4*>(M + (long long)i0 * Dp + 4 * e);
        }
#pragma unroll
        for (int u = 0; u < MR * 128 / 4 / 256; ++u) {
          const int e = tid + 256 * u;
          if (e < np) {
            const int r = (4 * e) / Dp, c = 4 * e - r * Dp;
            *reinterpret_cast<float4*>(&sm[r][c]) = t[u];
          }
        }
      } else {
        for (int e = tid; e < nr * Dp; e += 256) {
          const int r = e / Dp, c = e - (e / Dp) * Dp;
          sm[r][c] = M[(long long)(i0 + r) * Dp + c];
        }
      }
      __syncthreads();
      if (8 * jj < Dp) {
        for (int r = 0; r < nr; ++r) {
          const double mv = smean[gl][i0 + r];
          const float4 m0 = *reinterpret_cast<const float4*>(&sm[r][8 * jj]);
          const float4 m1 = *reinterpret_cast<const float4*>(&sm[r][8 * jj + 4]);
          const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
          for (int k = 0; k < 8; ++k) y[k] = __builtin_fma((double)mm[k], mv, y[k]);
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = 8 * jj + k;
      y[k] = j < Dp ? smean[gl][j] : 0.0;
    }
  }
  double b = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int j = 8 * jj + k;
    if (j < Dp) b = __builtin_fma(y[k], smean[gl][j], b);
  }
  for (int o = 8; o > 0; o >>= 1) b += __shfl_xor(b, o, 16);
  if (gl >= ng) return;
  const long long yo = ((long long)bh * a.gstride + g0 + gl) * a.ystride;
  if (8 * jj < Dimg) {
    bf16_t hv[8], lv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = 8 * jj + k;
      const float yf = j < Dp ? (float)y[k] : 0.f;
      hv[k] = f32_to_bf16(yf);
      lv[k] = f32_to_bf16(yf - bf16_to_f32(hv[k]));
    }
    *reinterpret_cast<uint4*>(a.yhi + yo + 8 * jj) = *reinterpret_cast<const uint4*>(hv);
    *reinterpret_cast<uint4*>(a.ylo + yo + 8 * jj) = *reinterpret_cast<const uint4*>(lv);
  }
  if (jj == 0) a.ybias[(long long)bh * a.gstride + g0 + gl] = (float)b;
}

// M_Q = s^2 sum over non-empty key groups of cbar_h cbar_h^T (d x d per (b,h));
// 16 key groups at a time are staged in LDS, each thread owns a 4x4 block
__global__ __launch_bounds__(1024) void k_query_metric(QMetricArgs a) {
  constexpr int HB = 16;
  __shared__ double cs[HB][128];
  const int bh = blockIdx.x, d = a.d, tid = threadIdx.x;
  const double* cb = a.cbar + (long long)bh * a.GK * d;
  const int* off = a.off_k + (long long)bh * (a.GK + 1);
  const int nb = d / 4;  // 4x4 blocks per row of blocks
  const int bi = tid / nb, bj = tid - (tid / nb) * nb;
  const bool act = bi < nb;
  double acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.0;
  for (int h0 = 0; h0 < a.GK; h0 += HB) {
    __syncthreads();
    for (int e = tid; e < HB * d; e += 1024) {
      const int hl = e / d, j = e - (e / d) * d;
      const int h = h0 + hl;
      cs[hl][j] = (h < a.GK && off[h + 1] > off[h]) ? cb[(long long)h * d + j] : 0.0;
    }
    __syncthreads();
    if (act) {
      for (int hl = 0; hl < HB; ++hl) {
        double u[4], v[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          u[x] = cs[hl][4 * bi + x];
          v[x] = cs[hl][4 * bj + x];
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
    for (int y = 0; y < 4; ++y) a.mq[(long long)bh * d * d + (4 * bi + x) * d + 4 * bj + y] = (float)(s2 * acc[x][y]);
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
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
    const int row = (int)(e / cpr), c = (int)(e - (e / cpr) * cpr) * VEC;
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const T*>(v.p) + v.row_off(bh, row) + c);
    const T* ev = reinterpret_cast<const T*>(&u);
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const float x = fabsf(Elem<T>::load(ev + j));
      m = (x > m || x != x) ? x : m;
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
  if (p.dtype == SPARSEPR_BF16) {
    if (p.d == 128) SP_LAUNCH((k_sample_metric<bf16_t, 128>), dim3(p.BH), dim3(256), s, a);
    else SP_LAUNCH((k_sample_metric<bf16_t, 64>), dim3(p.BH), dim3(256), s, a);
  } else {
    if (p.d == 128) SP_LAUNCH((k_sample_metric<float, 128>), dim3(p.BH), dim3(256), s, a);
    else SP_LAUNCH((k_sample_metric<float, 64>), dim3(p.BH), dim3(256), s, a);
  }
  return hipSuccess;
}

hipError_t launch_key_eig(const Plan& p, hipStream_t s) {
  EigArgs a{p.mk, p.eigval, p.kmap, p.rK, p.scale};
  if (p.d == 128) SP_LAUNCH(k_key_eig<128>, dim3(p.BH), dim3(1024), s, a);
  else SP_LAUNCH(k_key_eig<64>, dim3(p.BH), dim3(1024), s, a);
  return hipSuccess;
}

hipError_t launch_key_coords(const Plan& p, hipStream_t s) {
  CoordArgs a{p.k, p.kmap, p.N, p.rK, p.rKpad, p.z32, p.zhi, p.zlo};
  dim3 g((p.N + 63) / 64, p.BH);
  if (p.dtype == SPARSEPR_BF16) {
    const dim3 gm((p.N + 1023) / 1024, p.BH);
    if (p.rK <= 32) {
      if (p.d == 128) SP_LAUNCH((k_key_coords_mfma<128, 1>), gm, dim3(256), s, a);
      else SP_LAUNCH((k_key_coords_mfma<64, 1>), gm, dim3(256), s, a);
    } else {
      if (p.d == 128) SP_LAUNCH((k_key_coords_mfma<128, 2>), gm, dim3(256), s, a);
      else SP_LAUNCH((k_key_coords_mfma<64, 2>), gm, dim3(256), s, a);
    }
  } else {
    if (p.d == 128) SP_LAUNCH((k_key_coords<float, 128>), g, dim3(256), s, a);
    else SP_LAUNCH((k_key_coords<float, 64>), g, dim3(256), s, a);
  }
  return hipSuccess;
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
  else SP_LAUNCH(k_group_mean<float>, g, dim3(256), s, a);
  if (a.means_only) return hipSuccess;
  SP_LAUNCH(k_centre_images, dim3((a.G + 15) / 16, p.BH), dim3(256), s, a);
  return hipSuccess;
}

hipError_t launch_query_metric(const Plan& p, hipStream_t s) {
  QMetricArgs a{p.cbar, p.off_k, p.GK, p.d, p.scale, p.mq};
  SP_LAUNCH(k_query_metric, dim3(p.BH), dim3(1024), s, a);
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
