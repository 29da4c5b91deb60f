// Attention kernels for gfx950: block-sparse flash attention over the
// group-permuted layout, exact probe rows, probe-row overwrite, dense baseline.
//
// Sources (page title, section):
//   [TS] "Resumen Técnico: SparsePR ..." (gist.science) 2.C: tokens are permuted into
//        group-contiguous order and attention runs over variable-size blocks; 2.B:
//        probe rows are evaluated exactly and R = O_dense - O_sparse; the fitted map
//        corrects the unprobed rows.
//   [NE] news explainer reposted from 科技行者, section "稀疏执行怎么落地，误差怎么算才公平":
//        the output restoration step returns rows to token order.
//
// Work decomposition: a workgroup owns up to 128 rows of one query group and
// streams the concatenation of that group's granted key groups ("virtual key
// sequence") in 64-key tiles, so only the end of the whole sequence is ragged,
// not every granted cell.  The last rows of a query group, when they fit in
// 64, form a "split" tile: its two 32-row blocks are each taken by two waves
// that split every 64-key tile between them, so the workgroup stays busy with
// half the rows instead of padding them to 128.
#include <string.h>

#include <type_traits>

#include "sp_kernels.h"

namespace sp {

struct AttnArgs {
  View4 qv, kv, vv;       // row addressing: Q in token order, K and V permuted (or all original)
  MutView4 o;
  const int* perm_q;      // position -> token (null: identity); also addresses the Q rows
  const int* off_k;
  const int* csr_ptr;
  const int* csr_col;
  const int* tiles;
  const int* ntiles;
  int max_tiles;
  const float* fitW;
  const float* fitV;
  const float* fitb;
  const int* fitrank;
  const bf16_t* fitpk;  // hi/lo bf16 W^T [Rp, D] and V [D, Rp] per head (MFMA epilogue)
  int Rp;
  int R;
  int N, GK, GQ;
  float scale;
  int correct;
  int dense;
  const int* vexp;  // V stored as fp16 * 2^-vexp (null: V in the input dtype)
  int grid_tiles;   // tile slots per head in the launch grid
  int BH;
};

// Workgroups are handed to the 8 XCDs round-robin (workgroup i runs on XCD
// i % 8), and each XCD has its own L2.  Give every XCD one contiguous range of
// (head, tile) slots so that the workgroups resident on an XCD work on the same
// head and on neighbouring query groups, whose key ranges overlap.
__device__ inline void xcd_item(const AttnArgs& a, int* bh, int* tile) {
  const int total = a.grid_tiles * a.BH;
  const int per = (total + kXcds - 1) / kXcds;
  const int i = blockIdx.x;
  const int logical = (i % kXcds) * per + i / kXcds;
  *bh = logical / a.grid_tiles;
  *tile = logical % a.grid_tiles;
}

__device__ inline int seg_find(const int* sv, int n, int v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sv[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// exclusive scan of one int per thread over the block (blockDim multiple of 64)
__device__ inline int block_excl_scan(int v, int* tmp, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  int inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < w) base += tmp[i];
    tot += tmp[i];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Resolve the work item and build the virtual key sequence of its query group.
// Returns false when the workgroup has nothing to do.
template <int PER>
__device__ inline bool setup_item(const AttnArgs& a, int bh, int tile, int* seg_v, int* seg_p, int* tmp,
                                  int* g_out, int* row0, int* nrows, int* nseg, int* L, int* split) {
  const int tid = threadIdx.x;
  *split = 0;
  if (a.dense) {
    *row0 = tile * kTileRows;
    if (*row0 >= a.N) return false;
    *nrows = min(kTileRows, a.N - *row0);
    *g_out = 0;
    if (tid == 0) {
      seg_v[0] = 0;
      seg_p[0] = 0;
      seg_v[1] = a.N;
    }
    *nseg = 1;
    *L = a.N;
    __syncthreads();
    return true;
  }
  if (tile >= a.ntiles[bh]) return false;
  const int* e = a.tiles + ((long long)bh * a.max_tiles + tile) * 4;
  const int g = e[0];
  *g_out = g;
  *row0 = e[1];
  *nrows = e[2];
  *split = e[3];
  const int* cp = a.csr_ptr + (long long)bh * (a.GQ + 1);
  const int c0 = cp[g], nc = cp[g + 1] - c0;
  const int* cols = a.csr_col + (long long)bh * a.GQ * a.GK + c0;
  const int* offk = a.off_k + (long long)bh * (a.GK + 1);
  int lens[PER];
  int lsum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = PER * tid + i;
    int l = 0;
    if (idx < nc) {
      const int h = cols[idx];
      l = offk[h + 1] - offk[h];
      seg_p[idx] = offk[h];
    }
    lens[i] = l;
    lsum += l;
  }
  int total;
  int ex = block_excl_scan(lsum, tmp, &total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = PER * tid + i;
    if (idx < nc) seg_v[idx] = ex;
    ex += lens[i];
  }
  if (tid == 0) seg_v[nc] = total;
  *nseg = nc;
  *L = total;
  __syncthreads();
  return true;
}

// Epilogue of the attention kernels: normalise, correct (b + x W V^T) on the
// matrix cores, restore token order.  o holds the wave's 32 rows in the
// S^T-accumulator layout (lane = row within the block, both lane halves carry
// partial sums l of the row).
template <int D, bool VF16>
__device__ __attribute__((always_inline)) inline void attn_epilogue(const AttnArgs& a, int bh, f32x16 (&o)[D / 32],
                                                                    float l, int lane, bool owner, bool qvalid,
                                                                    int row0, int qr) {
  constexpr int KS = D / 16, DB = D / 32;
  const int half = lane >> 5, col = lane & 31;
  const float ltot = l + __shfl_xor(l, 32, 64);
  float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (VF16) inv = ldexpf(inv, a.vexp[bh]);
  float x[DB][16];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) x[b][r] = o[b][r] * inv;
  const int rank = (a.correct && a.fitrank) ? a.fitrank[bh] : 0;
  if (rank > 0) {
    // Correction on the matrix cores, in the accumulators' own layout:
    //   T^T (rank x rows) = W^T X^T,   out^T (dims x rows) = X^T + b + V T^T,
    // so out^T lands where each lane already holds its row's dims.  X, T, W
    // and V are split into hi + lo bf16; each product adds hi.hi + lo.hi +
    // hi.lo (relative error about 2^-16).  W^T and V come from the per-head
    // packed copies (hi/lo bf16, rank columns past the head's rank zero),
    // which every workgroup of the head reads through the L2; only the
    // owner waves read them, 32 rank columns at a time.
    const int Rp = a.Rp;
    const bf16_t* Wh = a.fitpk + (long long)bh * 4 * Rp * D;  // [Rp][D]: W^T, hi
    const bf16_t* Wlo = Wh + (long long)Rp * D;               // lo
    const bf16_t* Vh = Wlo + (long long)Rp * D;               // [D][Rp]: V, hi
    const bf16_t* Vlo = Vh + (long long)Rp * D;               // lo
    // B operands take 8 consecutive dims (ranks) per lane: dims 16 c + 8 half
    // + 0..7 of the lane's row for chunk c.  The accumulator layout holds
    // dims (r & 3) + 8 (r >> 2) + 4 half, so registers 8 sub + q and
    // 8 sub + 4 + q are exchanged between lanes i and i + 32.
    auto to_b = [&](const float* v16, bf16x8* hi, bf16x8* lo) __attribute__((always_inline)) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v16[q]), __float_as_uint(v16[4 + q]), false,
                                                         false);
        v[q] = __uint_as_float(sw[0]);
        v[4 + q] = __uint_as_float(sw[1]);
      }
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ph[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        pl[j] = pack_bf16x2(v[2 * j] - __uint_as_float(ph[j] << 16), v[2 * j + 1] - __uint_as_float(ph[j] & 0xffff0000u));
      }
      *hi = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
      *lo = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
    };
    bf16x8 xh[KS], xl[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) to_b(&x[ks >> 1][8 * (ks & 1)], &xh[ks], &xl[ks]);
    // accumulators start at x + b
    f32x16 cacc[DB];
    const float* fb = a.fitb + (long long)bh * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) cacc[b][r] = x[b][r] + fb[32 * b + (r & 3) + 8 * (r >> 2) + 4 * half];
    for (int j0 = 0; j0 < rank && owner; j0 += 32) {
      {
        // T^T = W^T X^T: A = rows of W^T (rank col, dims 16 ks + 8 half ..)
        f32x16 t = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const long long wo = (long long)(j0 + col) * D + 16 * ks + 8 * half;
          const bf16x8 ah = *reinterpret_cast<const bf16x8*>(Wh + wo);
          const bf16x8 al = *reinterpret_cast<const bf16x8*>(Wlo + wo);
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xh[ks], t, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xh[ks], t, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xl[ks], t, 0, 0, 0);
        }
        bf16x8 th[2], tl[2];
        float tv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) tv[r] = t[r];
#pragma unroll
        for (int kr = 0; kr < 2; ++kr) to_b(&tv[8 * kr], &th[kr], &tl[kr]);
        // out^T += V T^T: A = rows of V (dim 32 b + col, ranks 16 kr + 8 half ..)
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int kr = 0; kr < 2; ++kr) {
            const long long vo = (long long)(32 * b + col) * Rp + j0 + 16 * kr + 8 * half;
            const bf16x8 vh = *reinterpret_cast<const bf16x8*>(Vh + vo);
            const bf16x8 vl = *reinterpret_cast<const bf16x8*>(Vlo + vo);
            cacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, th[kr], cacc[b], 0, 0, 0);
            cacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl, th[kr], cacc[b], 0, 0, 0);
            cacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, tl[kr], cacc[b], 0, 0, 0);
          }
      }
    }
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[b][r] = cacc[b][r];
  }
  if (!(owner && qvalid)) return;
  const int pos = row0 + qr;
  const int token = a.perm_q ? a.perm_q[(long long)bh * a.N + pos] : pos;
  bf16_t* orow = static_cast<bf16_t*>(a.o.p) + a.o.row_off(bh, token);
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dm = 32 * b + 8 * r4 + 4 * half;
      uint2 pk;
      pk.x = pack_bf16x2(x[b][4 * r4 + 0], x[b][4 * r4 + 1]);
      pk.y = pack_bf16x2(x[b][4 * r4 + 2], x[b][4 * r4 + 3]);
      *reinterpret_cast<uint2*>(orow + dm) = pk;
    }
}

// ============================================================================
// bf16 MFMA kernel.  Per wave: 32 query rows.  S^T = K Q^T (A = K tile from
// LDS, B = Q rows in registers) so each lane holds one query row; the online
// softmax needs one cross-half exchange.  O^T = V^T P^T with V transposed in
// LDS; the contraction order over keys inside a 16-key step follows the S^T
// register layout (keys 16s + 4h + {0..3} and 16s + 8 + 4h + {0..3}).
// ============================================================================
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define SP_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define SP_GLB(p) ((__attribute__((address_space(1))) void*)(p))

// LDS tile layout: rows of D 16-bit values, no padding; the 16-byte chunks of
// a row are permuted by an XOR swizzle so that
//   K fragment reads (16 lanes = 16 keys, one chunk)          -> distinct banks,
//   V transposing reads (ds_read_b64_tr_b16, 4 keys x 4 dims) -> distinct banks.
template <int CPR> __device__ inline int swz_k(int key) { return key & (CPR - 1); }
template <int CPR> __device__ inline int swz_v(int key) { return (4 * key) & (CPR - 1); }

template <int D, bool VF16>
__global__ __launch_bounds__(256, 2) void k_sparse_attn_mfma(AttnArgs a) {
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int CPR = D / 8;              // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;           // rows moved by one wave-wide 16-byte LDS-DMA load
  constexpr int IPW = 64 / RPI / 4;       // such loads per wave per tile (K and V each)
  // Two pipeline stages, each [K | V][64 keys][D] (V sits VOFF bytes past K).
  // They are distinct objects so that reads of one stage provably do not
  // alias the LDS-DMA writes in flight into the other: with that (and the
  // restrict-qualified tile bases below) no wait on the loads of the next
  // tile is placed in front of the current tile's LDS reads.
  constexpr int VOFF = 64 * D * 2;
  __shared__ __attribute__((aligned(1024))) bf16_t KV0[2 * 64 * D];
  __shared__ __attribute__((aligned(1024))) bf16_t KV1[2 * 64 * D];
  __shared__ long long offs0[128], offs1[128];  // element offsets of the K rows, then the V rows
  __shared__ int seg_v[kMaxGroups + 1], seg_p[kMaxGroups + 1];
  __shared__ int tmp[8];
  int bh, tile;
  xcd_item(a, &bh, &tile);
  if (bh >= a.BH) return;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  int g, row0, nrows, nseg, L, split;
  if (!setup_item<4>(a, bh, tile, seg_v, seg_p, tmp, &g, &row0, &nrows, &nseg, &L, &split)) return;
  // split tile: waves w and w + 2 take row block w & 1, key half w >> 1
  const int rw = split ? (w & 1) : w;
  const int kh = split ? (w >> 1) : 0;
  const bool wave_active = 32 * rw < nrows;
  const bool owner = wave_active && (!split || w < 2);  // holds the merged rows at the end
  const int qr = 32 * rw + col;
  const bool qvalid = qr < nrows;

  const bf16_t* qb = static_cast<const bf16_t*>(a.qv.p);
  const bf16_t* kb = static_cast<const bf16_t*>(a.kv.p);
  const bf16_t* vb = static_cast<const bf16_t*>(a.vv.p);
  const int qtok = !qvalid ? 0 : (a.perm_q ? a.perm_q[(long long)bh * a.N + row0 + qr] : row0 + qr);
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qvalid) u = *reinterpret_cast<const uint4*>(qb + a.qv.row_off(bh, qtok) + 16 * ks + 8 * half);
    qf[ks] = __builtin_bit_cast(bf16x8, u);
  }
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float c = a.scale * 1.4426950408889634f;

  // Wave 0 resolves the physical rows of one tile (virtual key -> segment);
  // lane j owns key j of every tile, so its segment cursor only moves
  // forward.  The current segment's virtual start, physical start and the
  // next segment's virtual start stay in registers: LDS is read only when a
  // key crosses into the next segment.
  int cur = 0, cv = seg_v[0], cp = seg_p[0], nv = nseg > 1 ? seg_v[1] : 0x7fffffff;
  auto rows = [&](long long* __restrict__ ofs, const int* __restrict__ sv, const int* __restrict__ sp, int tt)
                  __attribute__((always_inline)) {
    const int v = 64 * tt + lane;
    int prow = cp;  // rows past the end read a valid row; they are masked
    if (v < L) {
      while (v >= nv) {
        ++cur;
        cv = nv;
        cp = sp[cur];
        nv = cur + 1 < nseg ? sv[cur + 1] : 0x7fffffff;
      }
      prow = cp + v - cv;
    }
    ofs[lane] = a.kv.row_off(bh, prow);
    ofs[64 + lane] = a.vv.row_off(bh, prow);
  };
  // Every wave moves its share of the K and V tiles straight into LDS.
  typedef __attribute__((address_space(3))) char lds_char;
  auto issue = [&](lds_char* __restrict__ dst, const long long* __restrict__ ofs, const bf16_t* __restrict__ gk0,
                   const bf16_t* __restrict__ gv0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int rb = (w * IPW + i) * RPI;
      const int r = rb + lane / CPR, sl = lane % CPR;
      const bf16_t* gk = gk0 + ofs[r] + 8 * (sl ^ swz_k<CPR>(r));
      const bf16_t* gv = gv0 + ofs[64 + r] + 8 * (sl ^ swz_v<CPR>(r));
      __builtin_amdgcn_global_load_lds(SP_GLB(gk), dst + rb * 2 * D, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(SP_GLB(gv), dst + VOFF + rb * 2 * D, 16, 0, 0);
    }
  };

  // Per-lane LDS byte bases of the fragment reads.  The chunk swizzle only
  // flips address bits below the row bits, so every fragment address is
  // (base ^ small constant) + immediate offset.
  const int gi = lane >> 4, li = lane & 15, rr = li >> 2, qq = li & 3;
  // a key-half wave of a split tile reads keys 32..63 of every tile: the
  // offset is a whole number of 32-key blocks and leaves the swizzle bits alone
  const uint32_t khoff = (uint32_t)kh * 32 * 2 * D;
  const uint32_t kbase0 = khoff + col * 2 * D + 16 * (half ^ swz_k<CPR>(col));
  const uint32_t vbase0 = khoff + VOFF + (4 * (gi >> 1) + rr) * 2 * D + 64 * (swz_v<CPR>(rr) >> 2) +
                          16 * (2 * (gi & 1) + (qq >> 1)) + 8 * (qq & 1);

  // NKT 32-key blocks of the tile per wave: 2, or 1 (key half kh) in a split tile
  auto compute_tile = [&](auto mask_tag, auto split_tag, const lds_char* __restrict__ lds, int kt0)
                          __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int NKT = decltype(split_tag)::value ? 1 : 2;
    // opaque per tile: keeps the derived addresses from being hoisted into
    // registers for the whole loop
    uint32_t kb0 = kbase0, vb0 = vbase0;
    asm volatile("" : "+v"(kb0), "+v"(vb0));
    f32x16 sacc[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) sacc[kt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t ka = kb0 ^ (32u * ks);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const bf16x8 kf = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(lds + ka + kt * 32 * 2 * D);  // keys 32kt + col
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kt], 0, 0, 0);
      }
    }
    // row max of the raw scores (masking the ragged end of the sequence)
    float mloc = -INFINITY;
    if constexpr (MASK) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * (kt + kh) + (r & 3) + 8 * (r >> 2) + 4 * half;
          if (kt0 + key >= L) sacc[kt][r] = -INFINITY;
        }
    }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[kt][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64)) * c;
    // Lazy rescaling: the reference max only moves when a row's max grows by
    // more than 8 (log2 units), so p <= 2^8 stays exact in fp16 and fp32 sums;
    // the softmax is invariant to the reference.
    if (__builtin_amdgcn_ballot_w64(mloc > m + 8.f)) {
      const float mnew = fmaxf(m, mloc);
      float alpha = __builtin_amdgcn_exp2f(m - mnew);
      // alpha is opaque past this point, so the rescale below cannot be
      // speculated out of the (rarely taken) branch
      asm volatile("" : "+v"(alpha));
      l *= alpha;
      // in place, so the accumulators keep their registers across the branch
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("v_mul_f32 %0, %1, %0" : "+v"(o[b][i]) : "v"(alpha));
      m = mnew;
    }
    // a row that has seen no key yet (the key-half wave of a split tile whose
    // granted keys all lie in the other half) keeps m = -inf; its masked
    // scores must give p = 0, not exp2(-inf + inf)
    const float mb = m == -INFINITY ? 0.f : m;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], c, -mb));
        sacc[kt][r] = pv;
        if constexpr (!VF16) psum += pv;
      }
    // P.V: A = V^T fragment read transposed from the row-major V tile.  In a
    // 16-lane group (index gi = lane>>4, i = lane&15) lane i supplies the
    // address of key kb + (i>>2), dims 4(i&3)..+3; it receives dim (i) of keys
    // kb..kb+3 -- the keys its P values (S^T register layout) belong to.
    uint32_t va[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) va[b] = vb0 ^ (64u * b);
#pragma unroll
    for (int sp = 0; sp < 2 * NKT; ++sp) {
      const int kt = sp >> 1, rb = 8 * (sp & 1);
      uint32_t pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (VF16) {
          typedef _Float16 h2 __attribute__((ext_vector_type(2)));
          const h2 hv = {(_Float16)sacc[kt][rb + 2 * j], (_Float16)sacc[kt][rb + 2 * j + 1]};
          pw[j] = __builtin_bit_cast(uint32_t, hv);
        } else {
          pw[j] = pack_bf16x2(sacc[kt][rb + 2 * j], sacc[kt][rb + 2 * j + 1]);
        }
      }
      const uint4 pk = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      if constexpr (VF16) {
        // row sum of the fp16 probabilities the product below uses (fp32 accumulation)
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 one2 = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) psum = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, pw[j]), one2, psum, false);
      }
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        // keys 16sp + 4(gi>>1) + (0..3) and the same + 8, dims 32b + 16(gi&1) + (0..15)
        const v4i16 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<lds_char*>(lds) + va[b] + sp * 32 * D));
        const v4i16 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<lds_char*>(lds) + va[b] + sp * 32 * D + 16 * D));
        const uint2 u0 = __builtin_bit_cast(uint2, t0), u1 = __builtin_bit_cast(uint2, t1);
        const uint4 vv = make_uint4(u0.x, u0.y, u1.x, u1.y);
        if constexpr (VF16) {
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vv), __builtin_bit_cast(f16x8, pk),
                                                        o[b], 0, 0, 0);
        } else {
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv),
                                                         __builtin_bit_cast(bf16x8, pk), o[b], 0, 0, 0);
        }
      }
    }
    l += psum;
  };

  const int ntile = (L + 63) / 64;
  const int nfull = L / 64;  // tiles without a ragged end
  lds_char* const s0 = (lds_char*)KV0;
  lds_char* const s1 = (lds_char*)KV1;
  const bf16_t* const gk0 = kb;
  const bf16_t* const gv0 = vb;
  // One pipeline step: start the DMA of tile t+1 into the other stage,
  // resolve the rows of tile t+2, compute tile t, then wait for the DMA and
  // meet at the barrier.  Tile t uses offsets buffer t&1 and stage t&1.
  auto step = [&](auto mask_tag, auto split_tag, lds_char* cur_st, lds_char* nxt_st, long long* nxt_ofs,
                  long long* cur_ofs, int t) __attribute__((always_inline)) {
    if (t + 1 < ntile) issue(nxt_st, nxt_ofs, gk0, gv0);
    if (w == 0 && t + 2 < ntile) rows(cur_ofs, seg_v, seg_p, t + 2);
    if (wave_active) compute_tile(mask_tag, split_tag, cur_st, 64 * t);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  if (w == 0) rows(offs0, seg_v, seg_p, 0);
  __syncthreads();
  issue(s0, offs0, gk0, gv0);
  if (w == 0 && ntile > 1) rows(offs1, seg_v, seg_p, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // full tiles in pairs (stages fixed at compile time), then the odd one and
  // the ragged end, so the hot loop carries no masking and no path merges
  constexpr std::false_type full{};
  constexpr std::true_type ragged{};
  auto run = [&](auto split_tag) __attribute__((always_inline)) {
    int t = 0;
    for (; t + 1 < nfull; t += 2) {
      step(full, split_tag, s0, s1, offs1, offs0, t);
      step(full, split_tag, s1, s0, offs0, offs1, t + 1);
    }
    if (t < nfull) {
      step(full, split_tag, s0, s1, offs1, offs0, t);
      ++t;
    }
    if (t < ntile) {
      if (t & 1) step(ragged, split_tag, s1, s0, offs0, offs1, t);
      else step(ragged, split_tag, s0, s1, offs1, offs0, t);
    }
  };
  if (split) {
    run(std::true_type{});
    // merge the key halves: waves 2 and 3 hand (m, l, O) to waves 0 and 1
    // through the (now idle) stage buffers
    float* xo = reinterpret_cast<float*>(KV0);  // [2][DB * 16][64]
    float* xs = reinterpret_cast<float*>(KV1);  // [2][2][64]
    if (w >= 2) {
      const int ww = w - 2;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) xo[((ww * DB + b) * 16 + i) * 64 + lane] = o[b][i];
      xs[(2 * ww) * 64 + lane] = m;
      xs[(2 * ww + 1) * 64 + lane] = l;
    }
    __syncthreads();
    if (w < 2) {
      const float m2 = xs[(2 * w) * 64 + lane], l2 = xs[(2 * w + 1) * 64 + lane];
      const float mm = fmaxf(m, m2);
      const float a1 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mm);
      const float a2 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mm);
      l = a1 * l + a2 * l2;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[b][i] = a1 * o[b][i] + a2 * xo[((w * DB + b) * 16 + i) * 64 + lane];
      m = mm;
    }
  } else {
    run(std::false_type{});
  }

  attn_epilogue<D, VF16>(a, bh, o, l, lane, owner, qvalid, row0, qr);
}

// hi/lo bf16 copies of each head's fitted maps in the layouts the MFMA
// correction reads its A fragments in: W^T [Rp][D] and V [D][Rp], rank
// columns at or past the head's rank set to zero.
__global__ __launch_bounds__(256) void k_fit_pack(const float* fitW, const float* fitV, const int* fitrank, int D,
                                                  int R, int Rp, bf16_t* pk) {
  const int bh = blockIdx.x;
  const int rank = fitrank[bh];
  bf16_t* wh = pk + (long long)bh * 4 * Rp * D;
  bf16_t* wl = wh + (long long)Rp * D;
  bf16_t* vh = wl + (long long)Rp * D;
  bf16_t* vl = vh + (long long)Rp * D;
  for (int e = blockIdx.y * 256 + threadIdx.x; e < D * Rp; e += gridDim.y * 256) {
    const int dm = e / Rp, j = e - (e / Rp) * Rp;
    const bool in = j < rank && j < R;
    const float wv = in ? fitW[((long long)bh * D + dm) * R + j] : 0.f;
    const float vv = in ? fitV[((long long)bh * D + dm) * R + j] : 0.f;
    const bf16_t w0 = f32_to_bf16(wv), v0 = f32_to_bf16(vv);
    wh[(long long)j * D + dm] = w0;
    wl[(long long)j * D + dm] = f32_to_bf16(wv - bf16_to_f32(w0));
    vh[(long long)dm * Rp + j] = v0;
    vl[(long long)dm * Rp + j] = f32_to_bf16(vv - bf16_to_f32(v0));
  }
}

// ============================================================================
// Vector-ALU kernel (fp32 inputs; also usable for bf16).  128 rows x 4 threads.
// ============================================================================
template <typename T, int D>
__global__ __launch_bounds__(512) void k_sparse_attn_vec(AttnArgs a) {
  constexpr int DQ = D / 4;
  __shared__ float Kt[32][D + 1];
  __shared__ float Vs[32][D + 1];
  __shared__ int seg_v[kMaxGroups + 1], seg_p[kMaxGroups + 1];
  __shared__ int tmp[8];
  const int bh = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  int g, row0, nrows, nseg, L, split;  // a split tile is an ordinary tile here
  if (!setup_item<2>(a, bh, tile, seg_v, seg_p, tmp, &g, &row0, &nrows, &nseg, &L, &split)) return;
  const int rl = tid >> 2, sub = tid & 3;
  const bool valid = rl < nrows;
  const T* qb = static_cast<const T*>(a.qv.p);
  const T* kb = static_cast<const T*>(a.kv.p);
  const T* vb = static_cast<const T*>(a.vv.p);
  const int qtok = !valid ? 0 : (a.perm_q ? a.perm_q[(long long)bh * a.N + row0 + rl] : row0 + rl);
  float q[DQ], o[DQ];
#pragma unroll
  for (int i = 0; i < DQ; ++i) {
    q[i] = valid ? Elem<T>::load(qb + a.qv.row_off(bh, qtok) + sub + 4 * i) : 0.f;
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float c = a.scale * 1.4426950408889634f;
  for (int kt0 = 0; kt0 < L; kt0 += 32) {
    for (int e = tid; e < 32 * D; e += 512) {
      const int r = e / D, cc = e - (e / D) * D;
      const int v = kt0 + r;
      float kx = 0.f, vx = 0.f;
      if (v < L) {
        const int s = seg_find(seg_v, nseg, v);
        const int prow = seg_p[s] + v - seg_v[s];
        kx = Elem<T>::load(kb + a.kv.row_off(bh, prow) + cc);
        vx = Elem<T>::load(vb + a.vv.row_off(bh, prow) + cc);
      }
      Kt[r][cc] = kx;
      Vs[r][cc] = vx;
    }
    __syncthreads();
    float sc[32];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) p += q[i] * Kt[j][sub + 4 * i];
      p += __shfl_xor(p, 1, 64);
      p += __shfl_xor(p, 2, 64);
      sc[j] = (kt0 + j < L) ? p * c : -INFINITY;
      mloc = fmaxf(mloc, sc[j]);
    }
    const float mnew = fmaxf(m, mloc);
    const float mb = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2f(m - mb);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < DQ; ++i) o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float p = exp2f(sc[j] - mb);
      psum += p;
#pragma unroll
      for (int i = 0; i < DQ; ++i) o[i] += p * Vs[j][sub + 4 * i];
    }
    l = l * alpha + psum;
    m = mnew;
    __syncthreads();
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float x[DQ];
#pragma unroll
  for (int i = 0; i < DQ; ++i) x[i] = o[i] * inv;
  const int rank = (a.correct && a.fitrank) ? a.fitrank[bh] : 0;
  if (rank > 0) {
    const float* fw = a.fitW + (long long)bh * D * a.R;
    const float* fv = a.fitV + (long long)bh * D * a.R;
    const float* fb = a.fitb + (long long)bh * D;
    float corr[DQ];
#pragma unroll
    for (int i = 0; i < DQ; ++i) corr[i] = fb[sub + 4 * i];
    for (int j = 0; j < rank; ++j) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) t += x[i] * fw[(long long)(sub + 4 * i) * a.R + j];
      t += __shfl_xor(t, 1, 64);
      t += __shfl_xor(t, 2, 64);
#pragma unroll
      for (int i = 0; i < DQ; ++i) corr[i] += t * fv[(long long)(sub + 4 * i) * a.R + j];
    }
#pragma unroll
    for (int i = 0; i < DQ; ++i) x[i] += corr[i];
  }
  if (!valid) return;
  const int pos = row0 + rl;
  const int token = a.perm_q ? a.perm_q[(long long)bh * a.N + pos] : pos;
  T* orow = static_cast<T*>(a.o.p) + a.o.row_off(bh, token);
#pragma unroll
  for (int i = 0; i < DQ; ++i) Elem<T>::store(orow + sub + 4 * i, x[i]);
}

// ============================================================================
// Probe rows: exact dense output and the sparse output under the probe's own
// granted cells, from one pass over a key chunk (split-K), then a merge.
// ============================================================================
struct ProbeArgs {
  View4 qv, kv, vv;  // Q in token order, K and V permuted
  const int* perm_q; // position -> token, addresses the probe rows of Q
  const int* ppos;
  const int* pgroup;
  const int* kgroup;
  const uint32_t* gmask;
  int gwords;
  int N, M, GQ, n_pchunk;
  int pchunk;        // keys per workgroup (a multiple of 64)
  float scale;
  float* ppart;  // [BH, n_pchunk, 2, M, D + 2]
  float* ode;
  float* osp;
  const int* vexp;
};

template <typename T, typename VT, int D>
__global__ __launch_bounds__(256) void k_probe_attn_vec(ProbeArgs a) {
  constexpr int DQ = D / 4;
  __shared__ float Kt[32][D + 1];
  __shared__ float Vs[32][D + 1];
  __shared__ int kg[32];
  __shared__ uint32_t msk[64][33];
  const int bh = blockIdx.z, pb = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
  const int rl = tid >> 2, sub = tid & 3;
  const int p = pb * 64 + rl;
  const bool valid = p < a.M;
  for (int e = tid; e < 64 * a.gwords; e += 256) {
    const int r = e / a.gwords, wd = e - (e / a.gwords) * a.gwords;
    const int pp = pb * 64 + r;
    msk[r][wd] = pp < a.M ? a.gmask[((long long)bh * a.GQ + a.pgroup[(long long)bh * a.M + pp]) * a.gwords + wd] : 0u;
  }
  const T* qb = static_cast<const T*>(a.qv.p);
  const T* kb = static_cast<const T*>(a.kv.p);
  const VT* vb = static_cast<const VT*>(a.vv.p);
  float q[DQ], od[DQ], os[DQ];
  const int prow = valid ? a.ppos[(long long)bh * a.M + p] : 0;
  const int ptok = valid ? a.perm_q[(long long)bh * a.N + prow] : 0;
#pragma unroll
  for (int i = 0; i < DQ; ++i) {
    q[i] = valid ? Elem<T>::load(qb + a.qv.row_off(bh, ptok) + sub + 4 * i) : 0.f;
    od[i] = 0.f;
    os[i] = 0.f;
  }
  float md = -INFINITY, ld = 0.f, ms = -INFINITY, ls = 0.f;
  const float c = a.scale * 1.4426950408889634f;
  const int k0 = ch * a.pchunk, k1 = min(a.N, k0 + a.pchunk);
  for (int kt0 = k0; kt0 < k1; kt0 += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * D; e += 256) {
      const int r = e / D, cc = e - (e / D) * D;
      const int v = kt0 + r;
      float kx = 0.f, vx = 0.f;
      if (v < k1) {
        kx = Elem<T>::load(kb + a.kv.row_off(bh, v) + cc);
        vx = Elem<VT>::load(vb + a.vv.row_off(bh, v) + cc);
      }
      Kt[r][cc] = kx;
      Vs[r][cc] = vx;
    }
    if (tid < 32) kg[tid] = (kt0 + tid < k1) ? a.kgroup[(long long)bh * a.N + kt0 + tid] : 0;
    __syncthreads();
    float sc[32];
    float mld = -INFINITY, mls = -INFINITY;
    uint32_t gbits = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) s += q[i] * Kt[j][sub + 4 * i];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      const bool in = kt0 + j < k1;
      sc[j] = in ? s * c : -INFINITY;
      const int h = kg[j];
      const bool gr = in && ((msk[rl][h >> 5] >> (h & 31)) & 1u);
      gbits |= (gr ? 1u : 0u) << j;
      mld = fmaxf(mld, sc[j]);
      if (gr) mls = fmaxf(mls, sc[j]);
    }
    const float mnd = fmaxf(md, mld), mns = fmaxf(ms, mls);
    const float mbd = mnd == -INFINITY ? 0.f : mnd, mbs = mns == -INFINITY ? 0.f : mns;
    const float ad = exp2f(md - mbd), as = exp2f(ms - mbs);
#pragma unroll
    for (int i = 0; i < DQ; ++i) {
      od[i] *= ad;
      os[i] *= as;
    }
    float sd = 0.f, ss = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float pd = exp2f(sc[j] - mbd);
      const float ps = ((gbits >> j) & 1u) ? exp2f(sc[j] - mbs) : 0.f;
      sd += pd;
      ss += ps;
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
        const float vx = Vs[j][sub + 4 * i];
        od[i] += pd * vx;
        os[i] += ps * vx;
      }
    }
    ld = ld * ad + sd;
    ls = ls * as + ss;
    md = mnd;
    ms = mns;
  }
  if (!valid) return;
  const float vs = a.vexp ? ldexpf(1.0f, a.vexp[bh]) : 1.0f;
  float* base = a.ppart + (((long long)bh * a.n_pchunk + ch) * 2) * a.M * (D + 2);
  float* pd = base + (long long)p * (D + 2);
  float* ps = base + ((long long)a.M + p) * (D + 2);
#pragma unroll
  for (int i = 0; i < DQ; ++i) {
    pd[sub + 4 * i] = od[i] * vs;
    ps[sub + 4 * i] = os[i] * vs;
  }
  if (sub == 0) {
    pd[D] = md;
    pd[D + 1] = ld;
    ps[D] = ms;
    ps[D + 1] = ls;
  }
}

// Probe rows on the matrix cores (bf16 Q/K, fp16-scaled V).  One workgroup
// of four waves takes 64 probe rows against one chunk of a.pchunk keys.
// Waves 0 and 1 keep the dense online softmax (every key) of probes 0..31
// and 32..63, one per lane column; waves 2 and 3 keep the sparse one (the
// keys whose K/V group is granted to the probe's query group) of the same
// probes.  All four read the same K/V stages; each wave holds one
// accumulator set, so the kernel fits two waves per SIMD (holding both sets
// in one wave did not).  Partials (unnormalised o, reference max in log2
// units, sum) are combined across chunks by k_probe_merge.
template <int D>
__global__ __launch_bounds__(256, 2) void k_probe_attn_mfma(ProbeArgs a) {
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int CPR = D / 8, RPI = 64 / CPR, IPW = 64 / RPI / 4;
  constexpr int VOFF = 64 * D * 2;
  constexpr int MW = kMaxGroups / 32;
  constexpr int MS = MW + 1;  // odd row stride: the lanes' probes read distinct banks
  __shared__ __attribute__((aligned(1024))) bf16_t KV0[2 * 64 * D];
  __shared__ __attribute__((aligned(1024))) bf16_t KV1[2 * 64 * D];
  __shared__ int kg0[64], kg1[64];
  __shared__ uint32_t msk[64 * MS];
  const int bh = blockIdx.z, pb = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const bool sparse_role = w >= 2;
  const int k0 = ch * a.pchunk, k1 = min(a.N, k0 + a.pchunk);
  const int L = k1 - k0;
  if (L <= 0) return;
  // grant masks of the probes' query groups
  for (int e = tid; e < 64 * a.gwords; e += 256) {
    const int r = e / a.gwords, wd = e - r * a.gwords;
    const int pp = pb * 64 + r;
    msk[r * MS + wd] =
        pp < a.M ? a.gmask[((long long)bh * a.GQ + a.pgroup[(long long)bh * a.M + pp]) * a.gwords + wd] : 0u;
  }
  const int pl = 32 * (w & 1) + col;
  const int p = pb * 64 + pl;
  const bool valid = p < a.M;
  const bf16_t* qb = static_cast<const bf16_t*>(a.qv.p);
  const bf16_t* kb = static_cast<const bf16_t*>(a.kv.p);
  const bf16_t* vb = static_cast<const bf16_t*>(a.vv.p);
  const int prow = valid ? a.ppos[(long long)bh * a.M + p] : 0;
  const int ptok = valid ? a.perm_q[(long long)bh * a.N + prow] : 0;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (valid) u = *reinterpret_cast<const uint4*>(qb + a.qv.row_off(bh, ptok) + 16 * ks + 8 * half);
    qf[ks] = __builtin_bit_cast(bf16x8, u);
  }
  const float c = a.scale * 1.4426950408889634f;
  const int* kgrp = a.kgroup + (long long)bh * a.N;

  typedef __attribute__((address_space(3))) char lds_char;
  // the keys of a chunk are consecutive rows of the permuted K/V
  auto issue = [&](lds_char* __restrict__ dst, int tt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int rb = (w * IPW + i) * RPI;
      const int r = rb + lane / CPR, sl = lane % CPR;
      const int v = k0 + min(64 * tt + r, L - 1);  // rows past the end are masked
      const bf16_t* gk = kb + a.kv.row_off(bh, v) + 8 * (sl ^ swz_k<CPR>(r));
      const bf16_t* gv = vb + a.vv.row_off(bh, v) + 8 * (sl ^ swz_v<CPR>(r));
      __builtin_amdgcn_global_load_lds(SP_GLB(gk), dst + rb * 2 * D, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(SP_GLB(gv), dst + VOFF + rb * 2 * D, 16, 0, 0);
    }
  };
  const int gi = lane >> 4, li = lane & 15, rr = li >> 2, qq = li & 3;
  const uint32_t kbase0 = col * 2 * D + 16 * (half ^ swz_k<CPR>(col));
  const uint32_t vbase0 = VOFF + (4 * (gi >> 1) + rr) * 2 * D + 64 * (swz_v<CPR>(rr) >> 2) +
                          16 * (2 * (gi & 1) + (qq >> 1)) + 8 * (qq & 1);
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 one2 = {(_Float16)1.f, (_Float16)1.f};
  lds_char* const s0 = (lds_char*)KV0;
  lds_char* const s1 = (lds_char*)KV1;
  const int ntile = (L + 63) / 64;
  const uint32_t* mrow = msk + pl * MS;
  // the tile's 64 group ids travel by LDS-DMA too (wave 0, 4 bytes a lane)
  auto issue_groups = [&](int* kgn, int tt) __attribute__((always_inline)) {
    if (w == 0)
      __builtin_amdgcn_global_load_lds(SP_GLB(kgrp + k0 + min(64 * tt + lane, L - 1)), SP_LDS(kgn), 4, 0, 0);
  };
  float* const base = a.ppart + (((long long)bh * a.n_pchunk + ch) * 2) * a.M * (D + 2);

  // the whole chunk for one role: SPARSE masks the ungranted keys
  auto run = [&](auto sparse_tag) __attribute__((always_inline)) {
    constexpr bool SPARSE = decltype(sparse_tag)::value;
    f32x16 o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b] = f32x16{};
    float m = -INFINITY, l = 0.f;
    auto compute = [&](const lds_char* __restrict__ lds, const int* __restrict__ kgt, int kt0)
                       __attribute__((always_inline)) {
      uint32_t kb0 = kbase0, vb0 = vbase0;
      asm volatile("" : "+v"(kb0), "+v"(vb0));
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) sacc[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t ka = kb0 ^ (32u * ks);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8 kf = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(lds + ka + kt * 32 * 2 * D);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kt], 0, 0, 0);
        }
      }
      // which of this lane's 32 keys count: all (dense), or those granted to
      // the probe's query group (sparse)
      uint32_t amask = 0xffffffffu;
      if constexpr (SPARSE) {
        amask = 0;
        const int h0 = kgt[0];
        if (h0 == kgt[63]) {
          amask = ((mrow[h0 >> 5] >> (h0 & 31)) & 1u) ? 0xffffffffu : 0u;
        } else {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int h = kgt[32 * kt + (r & 3) + 8 * (r >> 2) + 4 * half];
              amask |= ((mrow[h >> 5] >> (h & 31)) & 1u) << (16 * kt + r);
            }
        }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kt + (r & 3) + 8 * (r >> 2) + 4 * half;
          float sv = sacc[kt][r];
          if (kt0 + key >= L || !((amask >> (16 * kt + r)) & 1u)) sv = -INFINITY;
          sacc[kt][r] = sv;
          mloc = fmaxf(mloc, sv);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64)) * c;
      // lazy rescaling of the reference max (p <= 2^8 stays exact in fp16)
      if (__builtin_amdgcn_ballot_w64(mloc > m + 8.f)) {
        const float mn = fmaxf(m, mloc);
        const float al = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        l *= al;
#pragma unroll
        for (int b = 0; b < DB; ++b) o[b] *= al;
        m = mn;
      }
      const float mb = m == -INFINITY ? 0.f : m;
      uint32_t va[DB];
#pragma unroll
      for (int b = 0; b < DB; ++b) va[b] = vb0 ^ (64u * b);
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        const int kt = sp >> 1, rb = 8 * (sp & 1);
        uint32_t pw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // excluded keys carry score -inf, i.e. probability 0
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][rb + 2 * j], c, -mb));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][rb + 2 * j + 1], c, -mb));
          const h2 hv = {(_Float16)e0, (_Float16)e1};
          pw[j] = __builtin_bit_cast(uint32_t, hv);
          l = __builtin_amdgcn_fdot2(hv, one2, l, false);
        }
        const f16x8 pk = __builtin_bit_cast(f16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const v4i16 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<lds_char*>(lds) + va[b] + sp * 32 * D));
          const v4i16 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) v4i16*>(
              const_cast<lds_char*>(lds) + va[b] + sp * 32 * D + 16 * D));
          const uint2 u0 = __builtin_bit_cast(uint2, t0), u1 = __builtin_bit_cast(uint2, t1);
          const f16x8 vv = __builtin_bit_cast(f16x8, make_uint4(u0.x, u0.y, u1.x, u1.y));
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv, pk, o[b], 0, 0, 0);
        }
      }
    };
    // one pipeline step: DMA of tile t+1 and its group ids, compute tile t
    auto step = [&](lds_char* cur, lds_char* nxt, const int* kgc, int* kgn, int t) __attribute__((always_inline)) {
      if (t + 1 < ntile) {
        issue(nxt, t + 1);
        issue_groups(kgn, t + 1);
      }
      compute(cur, kgc, 64 * t);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    issue_groups(kg0, 0);
    issue(s0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int t = 0; t < ntile; t += 2) {
      step(s0, s1, kg0, kg1, t);
      if (t + 1 < ntile) step(s1, s0, kg1, kg0, t + 1);
    }
    l += __shfl_xor(l, 32, 64);
    if (!valid) return;
    const float vs = ldexpf(1.0f, a.vexp[bh]);
    float* po = base + ((SPARSE ? (long long)a.M : 0LL) + p) * (D + 2);
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dim = 32 * b + (r & 3) + 8 * (r >> 2) + 4 * half;
        po[dim] = o[b][r] * vs;
      }
    if (half == 0) {
      po[D] = m;
      po[D + 1] = l;
    }
  };
  if (sparse_role) run(std::true_type{});
  else run(std::false_type{});
}

template <int D>
__global__ __launch_bounds__(D) void k_probe_merge(ProbeArgs a) {
  const int bh = blockIdx.z, which = blockIdx.y, p = blockIdx.x, dm = threadIdx.x;
  const long long stride_ch = 2LL * a.M * (D + 2);
  const float* pr0 = a.ppart + (((long long)bh * a.n_pchunk) * 2 + which) * a.M * (D + 2) + (long long)p * (D + 2);
  // chunk partials eight at a time, so their loads are in flight together
  float mx = -INFINITY;
  for (int c0 = 0; c0 < a.n_pchunk; c0 += 8) {
    float m8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) m8[u] = c0 + u < a.n_pchunk ? pr0[(c0 + u) * stride_ch + D] : -INFINITY;
#pragma unroll
    for (int u = 0; u < 8; ++u) mx = fmaxf(mx, m8[u]);
  }
  float num = 0.f, den = 0.f;
  if (mx > -INFINITY) {
    for (int c0 = 0; c0 < a.n_pchunk; c0 += 8) {
      float mc[8], xv[8], lv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = c0 + u < a.n_pchunk;
        const float* pr = pr0 + (c0 + u) * stride_ch;
        mc[u] = in ? pr[D] : -INFINITY;
        xv[u] = in ? pr[dm] : 0.f;
        lv[u] = in ? pr[D + 1] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (mc[u] == -INFINITY) continue;
        const float f = exp2f(mc[u] - mx);
        num += f * xv[u];
        den += f * lv[u];
      }
    }
  }
  float* out = which == 0 ? a.ode : a.osp;
  out[((long long)bh * a.M + p) * D + dm] = den > 0.f ? num / den : 0.f;
}

// probe rows keep their exact dense output
template <typename T>
__global__ __launch_bounds__(256) void k_probe_overwrite(MutView4 o, const int* perm_q, const int* ppos,
                                                         const float* ode, int N, int M, int D) {
  // one element per thread: the row lookups of every element run at once
  const int bh = blockIdx.x;
  for (int e = blockIdx.y * 256 + threadIdx.x; e < M * D; e += gridDim.y * 256) {
    const int p = e / D, dm = e - (e / D) * D;
    const int token = perm_q[(long long)bh * N + ppos[(long long)bh * M + p]];
    T* row = static_cast<T*>(o.p) + o.row_off(bh, token);
    Elem<T>::store(row + dm, ode[((long long)bh * M + p) * D + dm]);
  }
}

// ============================================================================
// launchers
// ============================================================================
static AttnArgs attn_args(const Plan& p, bool correct) {
  AttnArgs a;
  const long long nd = (long long)p.N * p.d;
  a.qv = p.q;
  a.kv = View4{p.kp, (long long)p.H * nd, nd, p.d, p.H};
  a.vv = View4{p.vp, (long long)p.H * nd, nd, p.d, p.H};
  a.o = p.o;
  a.perm_q = p.perm_q;
  a.off_k = p.off_k;
  a.csr_ptr = p.csr_ptr;
  a.csr_col = p.csr_col;
  a.tiles = p.tiles;
  a.ntiles = p.ntiles;
  a.max_tiles = p.max_tiles;
  a.fitW = p.fitW;
  a.fitV = p.fitV;
  a.fitb = p.fitb;
  a.fitrank = p.fitrank;
  a.fitpk = p.fitpk;
  a.Rp = p.Rp;
  a.R = p.R > 0 ? p.R : 1;
  a.N = p.N;
  a.GK = p.GK;
  a.GQ = p.GQ;
  a.scale = p.scale;
  a.correct = correct && p.M > 0 ? 1 : 0;
  a.dense = 0;
  a.vexp = p.dtype == SPARSEPR_BF16 ? p.vexp : nullptr;
  return a;
}

static hipError_t launch_attn(AttnArgs a, int grid_x, int BH, int d, int dtype, hipStream_t s) {
  dim3 g(grid_x, BH);
  if (dtype == SPARSEPR_BF16) {
    a.grid_tiles = grid_x;
    a.BH = BH;
    const long long total = (long long)grid_x * BH;
    const dim3 g1((unsigned)((total + kXcds - 1) / kXcds * kXcds));
    if (a.vexp) {
      if (d == 128) hipLaunchKernelGGL((k_sparse_attn_mfma<128, true>), g1, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_sparse_attn_mfma<64, true>), g1, dim3(256), 0, s, a);
    } else {
      if (d == 128) hipLaunchKernelGGL((k_sparse_attn_mfma<128, false>), g1, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_sparse_attn_mfma<64, false>), g1, dim3(256), 0, s, a);
    }
  } else {
    if (d == 128) hipLaunchKernelGGL((k_sparse_attn_vec<float, 128>), g, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((k_sparse_attn_vec<float, 64>), g, dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_sparse_attention(const Plan& p, bool correct, hipStream_t s) {
  AttnArgs a = attn_args(p, correct);
  if (a.correct && p.dtype == SPARSEPR_BF16) {
    hipLaunchKernelGGL(k_fit_pack, dim3(p.BH, (p.d * p.Rp + 255) / 256), dim3(256), 0, s, p.fitW, p.fitV, p.fitrank,
                       p.d, a.R, p.Rp, p.fitpk);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_attn(a, p.max_tiles, p.BH, p.d, p.dtype, s);
}

hipError_t launch_dense_attention(const View4& q, const View4& k, const View4& v, const MutView4& o, int BH,
                                  int N, int d, int dtype, float scale, hipStream_t s) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.qv = q;
  a.kv = k;
  a.vv = v;
  a.o = o;
  a.N = N;
  a.scale = scale;
  a.dense = 1;
  a.R = 1;
  return launch_attn(a, (N + kTileRows - 1) / kTileRows, BH, d, dtype, s);
}

hipError_t launch_probe_attention(const Plan& p, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  ProbeArgs a;
  const long long nd = (long long)p.N * p.d;
  a.qv = p.q;
  a.perm_q = p.perm_q;
  a.kv = View4{p.kp, (long long)p.H * nd, nd, p.d, p.H};
  a.vv = View4{p.vp, (long long)p.H * nd, nd, p.d, p.H};
  a.ppos = p.ppos;
  a.pgroup = p.pgroup;
  a.kgroup = p.kgroup;
  a.gmask = p.gmask;
  a.gwords = p.gwords;
  a.N = p.N;
  a.M = p.M;
  a.GQ = p.GQ;
  a.n_pchunk = p.n_pchunk;
  a.pchunk = p.pchunk;
  a.scale = p.scale;
  a.ppart = p.ppart;
  a.ode = p.ode;
  a.osp = p.osp;
  dim3 g(p.n_pchunk, (p.M + 63) / 64, p.BH);
  if (p.dtype == SPARSEPR_BF16) {
    a.vexp = p.vexp;
    if (p.d == 128) hipLaunchKernelGGL((k_probe_attn_mfma<128>), g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_probe_attn_mfma<64>), g, dim3(256), 0, s, a);
  } else {
    a.vexp = nullptr;
    if (p.d == 128) hipLaunchKernelGGL((k_probe_attn_vec<float, float, 128>), g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_probe_attn_vec<float, float, 64>), g, dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.d == 128) hipLaunchKernelGGL(k_probe_merge<128>, dim3(p.M, 2, p.BH), dim3(128), 0, s, a);
  else hipLaunchKernelGGL(k_probe_merge<64>, dim3(p.M, 2, p.BH), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_probe_overwrite(const Plan& p, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  if (p.dtype == SPARSEPR_BF16)
    hipLaunchKernelGGL(k_probe_overwrite<bf16_t>, dim3(p.BH, (p.M * p.d + 255) / 256), dim3(256), 0, s, p.o, p.perm_q,
                       p.ppos, p.ode, p.N, p.M, p.d);
  else
    hipLaunchKernelGGL(k_probe_overwrite<float>, dim3(p.BH, (p.M * p.d + 255) / 256), dim3(256), 0, s, p.o, p.perm_q,
                       p.ppos, p.ode, p.N, p.M, p.d);
  return hipGetLastError();
}

}  // namespace sp
