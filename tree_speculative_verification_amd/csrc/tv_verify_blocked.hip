// Verification of wide and deep trees: up to 512 nodes, any depth, any d_k,
// d_v in {16, 32, 64, 128}, fp32 or bf16 q/k/v.
//
// Same system as the other verification kernels (TreeWY abstract: every draft
// node's output from one triangular solve over a small pseudo-value matrix;
// Bole auto-summary, core-formula section, for the scalar-decay closed form):
//
//   (I + A) U = R,  R_n = beta_n (v_n - gamma_n S_root^T k_n),
//                   A[n, j] = beta_n D(j->n) (k_n.k_j) for j in anc(n)
//   o_n = gamma_n S_root^T q_n + sum_{j in anc*(n)} D(j->n) (q_n.k_j) u_j
//
// with anc*(n) the root-to-n path (n included), D(j->n) the product of alpha
// over the path nodes after j, gamma_n the product over all of anc*(n).  In
// scalar-decay mode u_n = v_n and only the second line is left.
//
// The solve is blocked so that any tree fits on chip.  The tree's path
// entries (node n, ancestor j) are laid out node after node with nodes sorted
// by depth, and processed in chunks of at most kBEnt entries: a chunk's
// entries get their Gram values and decays, then the chunk's nodes are solved
// one depth level at a time (a node's ancestors all sit in earlier levels, so
// they are final by then), then their outputs are gathered.  Only the chunk's
// entries and the workgroup's columns of U live in LDS, so trees of any depth
// go through the same code; a wide tree is a few chunks and one level step
// per depth.
//
// One workgroup of 512 threads per (sequence b, head h, block of up to 32
// value columns):
//   1. tree index: pointer jumping gives each node's path length and gamma;
//      nodes are then sorted by depth (counting sort) and given entry offsets;
//   2. R and gamma QS for every node into LDS: on matrix cores for bf16 with
//      d_k = d_v = 128 (32x32x16 bf16, S split into hi + lo words; the S block
//      and the first node tile are loaded before step 1, so their HBM latency
//      hides under the tree build), else fp32 FMA;
//   3. per chunk: path walk (entry nodes and decays), Gram dot products by
//      one 8-lane group per node, four of its entries in flight at a time
//      (the ancestor-masked Gram/decay builder), level solve, outputs (U and
//      o stored to HBM once).
//
// One workgroup fills most of a CU's LDS (R/U and gamma QS for 512 nodes x 32
// columns are 128 KB), so a CU runs one at a time and latency is hidden inside
// the workgroup: eight waves, loads issued ahead of use.
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {

namespace {

constexpr int kBT = 1024;   // threads per workgroup (16 waves: one node tile each)
constexpr int kBVB = 32;    // value columns per workgroup (d_v when d_v < 32)
constexpr int kBEnt = 1400; // path entries per chunk (what LDS has room for)
constexpr int kBD = 128;    // d_k = d_v of the matrix-core contraction

typedef __bf16 bbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bbf16x2 __attribute__((ext_vector_type(2)));
typedef float bf32x16 __attribute__((ext_vector_type(16)));

struct BlockedLds {
  float U[kMaxTree * kBVB];   // R rows, solved in place into U rows (row stride = columns)
  float QS[kMaxTree * kBVB];  // gamma_n QS_n rows
  float cA[kBEnt];            // decay during the walk, then beta_n D (k_n.k_j)
  float cP[kBEnt];            // D (q_n.k_j)
  uint16_t en[kBEnt];         // the entry's path node j
  int16_t par[kMaxTree];
  int16_t jmp[kMaxTree];
  int16_t len[kMaxTree];      // path length = depth + 1
  int16_t ord[kMaxTree];      // position -> node, positions sorted by depth
  int off[kMaxTree + 1];      // position -> first entry; off[N] = all entries
  int lst[kMaxTree + 1];      // depth -> first position
  int ebase[kMaxTree + 1];    // depth -> first entry
  int hist[kMaxTree];         // nodes per depth
  float alp[kMaxTree];
  float bet[kMaxTree];
  float gam[kMaxTree];
  int maxd;
};

__device__ __forceinline__ float dpp_sum8(float x) {
  // sum over the 8 lanes of a group: swap neighbours, swap pairs, then
  // mirror within the 8 (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror)
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
  return x;
}

__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
  bbf16x2 x, y;
  __builtin_memcpy(&x, &a.x, 4);
  __builtin_memcpy(&y, &b.x, 4);
  acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
  __builtin_memcpy(&x, &a.y, 4);
  __builtin_memcpy(&y, &b.y, 4);
  acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
  __builtin_memcpy(&x, &a.z, 4);
  __builtin_memcpy(&y, &b.z, 4);
  acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
  __builtin_memcpy(&x, &a.w, 4);
  __builtin_memcpy(&y, &b.w, 4);
  acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
  return acc;
}

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const bbf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  uint32_t r;
  __builtin_memcpy(&r, &v, 4);
  return r;
}

// LDS rows of R/U and gamma QS: float4 column group g of node n is stored at
// slot g ^ (n mod groups), so the lanes of a matrix-core tile (32 nodes, one
// group) and of the solve (8 nodes x 8 groups) spread over all banks.
__device__ __forceinline__ int urow(int n, int col, int vb) {
  return n * vb + ((((col >> 2) ^ n) & ((vb >> 2) - 1)) << 2);
}

// Operands of one 32-node tile for the matrix-core contraction: q and k rows
// (lane: node lane%32, 8 bf16 of each 16-wide d_k step) and v at the columns
// the accumulator lands on.
struct TileIn {
  bbf16x8 qb[8], kb[8];
  uint2 vv[4];
};

__device__ __forceinline__ void load_tile(TileIn& t, int T, int N, int H, int b, int h, int c0,
                                          bool gdn, const uint16_t* __restrict__ q,
                                          const uint16_t* __restrict__ k,
                                          const uint16_t* __restrict__ v) {
  const int lane = threadIdx.x & 63;
  const int lm = lane & 31, hi = lane >> 5;
  const int n = T * 32 + lm;
  const size_t row = ((size_t)b * N + (n < N ? n : N - 1)) * H + h;
  const uint16_t* qr = q + row * kBD + 8 * hi;
  const uint16_t* kr = k + row * kBD + 8 * hi;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    t.qb[ks] = *reinterpret_cast<const bbf16x8*>(qr + 16 * ks);
    if (gdn) t.kb[ks] = *reinterpret_cast<const bbf16x8*>(kr + 16 * ks);
  }
#pragma unroll
  for (int g = 0; g < 4; ++g)
    t.vv[g] = *reinterpret_cast<const uint2*>(v + row * kBD + c0 + 8 * g + 4 * hi);
}

// [K;Q] S_block products of one tile.  A = S block^T (value column x d_k),
// taken from the S block staged in LDS (row-major, 32 columns) and split into
// bf16 hi + lo words per 16-row step; B = [K or Q]^T (d_k x node).
__device__ __forceinline__ void mma_tile(const TileIn& t, const float* Sst, bool gdn,
                                         bf32x16& kacc, bf32x16& qacc) {
  const int lane = threadIdx.x & 63;
  const float* Sl = Sst + 8 * (lane >> 5) * kBVB + (lane & 31);  // rows 16 ks + 8 (lane/32) + i
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    kacc[r] = 0.f;
    qacc[r] = 0.f;
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = Sl[(16 * ks + 2 * i) * kBVB], x1 = Sl[(16 * ks + 2 * i + 1) * kBVB];
      wh[i] = pack2_bf16(x0, x1);
      wl[i] = pack2_bf16(x0 - __uint_as_float(wh[i] << 16), x1 - __uint_as_float(wh[i] & 0xffff0000u));
    }
    bbf16x8 shi, slo;
    __builtin_memcpy(&shi, wh, 16);
    __builtin_memcpy(&slo, wl, 16);
    qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi, t.qb[ks], qacc, 0, 0, 0);
    qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo, t.qb[ks], qacc, 0, 0, 0);
    if (gdn) {
      kacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi, t.kb[ks], kacc, 0, 0, 0);
      kacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo, t.kb[ks], kacc, 0, 0, 0);
    }
  }
}

// R and gamma QS of one tile into LDS: the accumulator puts node lane%32 and
// value columns 8 (r/4) + 4 (lane/32) + r%4 in lane `lane`.
__device__ __forceinline__ void store_tile(BlockedLds& s, const TileIn& t, int T, int N, bool gdn,
                                           const bf32x16& kacc, const bf32x16& qacc) {
  const int lane = threadIdx.x & 63;
  const int n = T * 32 + (lane & 31);
  if (n >= N) return;
  const float gn = s.gam[n], bn = s.bet[n];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint2 w = t.vv[g];
    const float4 vf = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    float4 r = vf;
    if (gdn) {
      r.x = bn * (vf.x - gn * kacc[4 * g + 0]);
      r.y = bn * (vf.y - gn * kacc[4 * g + 1]);
      r.z = bn * (vf.z - gn * kacc[4 * g + 2]);
      r.w = bn * (vf.w - gn * kacc[4 * g + 3]);
    }
    const int col = 8 * g + 4 * (lane >> 5);
    *reinterpret_cast<float4*>(&s.U[urow(n, col, kBVB)]) = r;
    *reinterpret_cast<float4*>(&s.QS[urow(n, col, kBVB)]) =
        make_float4(gn * qacc[4 * g + 0], gn * qacc[4 * g + 1], gn * qacc[4 * g + 2],
                    gn * qacc[4 * g + 3]);
  }
}

// The same with fp32 FMA, any d_k, d_v and input type; item = (node, 4 columns).
template <typename TIn>
__device__ void contract_fma(BlockedLds& s, int N, int H, int dk, int dv, int vb, int b, int h,
                             int bh, int c0, bool gdn, const TIn* __restrict__ q,
                             const TIn* __restrict__ k, const TIn* __restrict__ v,
                             const float* __restrict__ S_root) {
  const int ncg = vb / 4;
  const float* Sb = S_root + (size_t)bh * dk * dv;
  for (int it = threadIdx.x; it < N * ncg; it += kBT) {
    const int n = it / ncg;
    const int col = 4 * (it % ncg);
    const size_t row = ((size_t)b * N + n) * H + h;
    float4 ks = f4(0.f), qs = f4(0.f);
    for (int i = 0; i < dk; ++i) {
      const float4 sr = *reinterpret_cast<const float4*>(Sb + (size_t)i * dv + c0 + col);
      qs = fma4(Elem<TIn>::load(q, row * dk + i), sr, qs);
      if (gdn) ks = fma4(Elem<TIn>::load(k, row * dk + i), sr, ks);
    }
    const float gn = s.gam[n];
    float4 r = Elem<TIn>::load4(v, row * dv + c0 + col);
    if (gdn) r = mul4(s.bet[n], sub4(r, mul4(gn, ks)));
    *reinterpret_cast<float4*>(&s.U[urow(n, col, vb)]) = r;
    *reinterpret_cast<float4*>(&s.QS[urow(n, col, vb)]) = mul4(gn, qs);
  }
}

template <typename TIn, bool MFMA>
__global__ __launch_bounds__(kBT) void verify_blocked_kernel(
    int H, int N, int dk, int dv, int mode, const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ parents, const float* __restrict__ S_root, TIn* __restrict__ o,
    float* __restrict__ U, int32_t* __restrict__ status) {
  __shared__ BlockedLds s;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int vb = dv < kBVB ? dv : kBVB;
  const int nvb = dv / vb;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = bid % nvb;
  const int bh = bid / nvb;
  const int h = bh % H;
  const int b = bh / H;
  const int c0 = cb * vb;
  const bool gdn = mode == kGdn;
  const int ntiles = (N + 31) / 32;

  // small loads first (loads return in order): parents and gates
  const int pn = tid < N ? tid : N - 1;
  int p_in = parents[(size_t)b * N + pn];
  const float a_in = alpha[((size_t)b * N + pn) * H + h];
  const float b_in = gdn ? beta[((size_t)b * N + pn) * H + h] : 0.f;

  // matrix-core path: the S block (128 x 32 fp32, 16 KB) staged once in LDS by
  // coalesced loads (in the U rows, unused until the contraction's results),
  // and the wave's first node tile, both in flight during the tree build
  TileIn t0;
  if constexpr (MFMA) {
    float4* Sl = reinterpret_cast<float4*>(s.U);
    const float* Sb = S_root + (size_t)bh * kBD * kBD + c0;
    static_assert(kBT * 4 == kBD * kBVB, "one float4 of the S block per thread");
    Sl[tid] = *reinterpret_cast<const float4*>(Sb + (size_t)(tid >> 3) * kBD + 4 * (tid & 7));
    if (wave < ntiles)
      load_tile(t0, wave, N, H, b, h, c0, gdn, reinterpret_cast<const uint16_t*>(q),
                reinterpret_cast<const uint16_t*>(k), reinterpret_cast<const uint16_t*>(v));
  }

  // ---- 1. tree index ----
  if (tid == 0) s.maxd = 0;
  bool my_bad = false;
  if (tid < N) {
    s.hist[tid] = 0;
    my_bad = p_in < -1 || p_in >= tid;
    if (my_bad) p_in = -1;  // a parent outside [-1, i-1] is treated as -1 and flagged
    s.alp[tid] = a_in;
    s.bet[tid] = b_in;
    s.par[tid] = static_cast<int16_t>(p_in);
    s.jmp[tid] = static_cast<int16_t>(p_in);
    s.len[tid] = 1;
    s.gam[tid] = a_in;
  }
  const bool bad = __syncthreads_or(my_bad) != 0;
  // pointer jumping: a node's span (path nodes from it up to, not including,
  // its jump target) absorbs the target's span until the jump runs off the root
  while (true) {
    int j = -1, nj = -1, nl = 0;
    float ng = 1.f;
    if (tid < N) {
      j = s.jmp[tid];
      if (j >= 0) {
        nj = s.jmp[j];
        nl = s.len[j];
        ng = s.gam[j];
      }
    }
    if (!__syncthreads_or(j >= 0)) break;
    if (j >= 0) {
      s.jmp[tid] = static_cast<int16_t>(nj);
      s.len[tid] = static_cast<int16_t>(s.len[tid] + nl);
      s.gam[tid] *= ng;
    }
    __syncthreads();
  }
  // counting sort by depth
  int my_d = 0;
  if (tid < N) {
    my_d = s.len[tid] - 1;
    atomicAdd(&s.hist[my_d], 1);
    atomicMax(&s.maxd, my_d);
  }
  __syncthreads();
  const int maxd = s.maxd;
  for (int d = tid; d <= maxd + 1; d += kBT) {
    int c = 0, e = 0;
    for (int i = 0; i < d; ++i) {
      const int hc = s.hist[i];
      c += hc;
      e += hc * (i + 1);
    }
    s.lst[d] = c;
    s.ebase[d] = e;
  }
  __syncthreads();
  if (tid < N) {
    const int pos = s.lst[my_d] + atomicSub(&s.hist[my_d], 1) - 1;
    s.ord[pos] = static_cast<int16_t>(tid);
    s.off[pos] = s.ebase[my_d] + (pos - s.lst[my_d]) * (my_d + 1);
  }
  if (tid == 0) s.off[N] = s.ebase[maxd + 1];
  if (h == 0 && cb == 0 && tid == 0 && status) status[b] = bad ? 1 : 0;
  __syncthreads();

  // ---- 2. R and gamma QS ----
  if constexpr (MFMA) {
    // one node tile per wave (N <= 512 is at most 16 tiles); the S block sits
    // in the U rows until every wave has its products
    static_assert(kMaxTree / 32 <= kBT / 64, "a node tile per wave");
    bf32x16 kacc, qacc;
    if (wave < ntiles) mma_tile(t0, s.U, gdn, kacc, qacc);
    __syncthreads();
    if (wave < ntiles) store_tile(s, t0, wave, N, gdn, kacc, qacc);
  } else {
    contract_fma<TIn>(s, N, H, dk, dv, vb, b, h, bh, c0, gdn, q, k, v, S_root);
  }
  __syncthreads();

  // ---- 3. chunks of path entries ----
  const int ncg = vb / 4;
  const int grp = tid >> 3, lj = tid & 7;
  constexpr int kGroups = kBT / 8;
  for (int p0 = 0; p0 < N;) {
    const int e0 = s.off[p0];
    const int qpos = p0 + 1 + tid;
    const int p1 = p0 + __syncthreads_count(qpos <= N && s.off[qpos] - e0 <= kBEnt);
    const int nent = s.off[p1] - e0;

    // path walk: entry t of node n is (n, e_t) with decay D(e_t -> n)
    for (int p = p0 + tid; p < p1; p += kBT) {
      const int n = s.ord[p];
      int x = s.off[p] - e0;
      float D = 1.f;
      for (int e = n; e >= 0; e = s.par[e]) {
        s.en[x] = static_cast<uint16_t>(e);
        s.cA[x] = D;
        D *= s.alp[e];
        ++x;
      }
    }
    __syncthreads();

    // Gram values of the entries: one 8-lane group per node (its q and k rows
    // loaded once), its entries four at a time
    for (int p = p0 + grp; p < p1; p += kGroups) {
      const int n = s.ord[p];
      const int x0 = s.off[p] - e0;
      const int L = s.len[n];
      const float bn = s.bet[n];
      const size_t rn = ((size_t)b * N + n) * H + h;
      if constexpr (MFMA) {
        // bf16, d_k = 128: lane lj covers elements [16 lj, 16 lj + 16)
        const uint4* qn = reinterpret_cast<const uint4*>(q + rn * kBD) + 2 * lj;
        const uint4* kn = reinterpret_cast<const uint4*>(k + rn * kBD) + 2 * lj;
        const uint4 qa0 = qn[0], qa1 = qn[1];
        uint4 ka0 = make_uint4(0, 0, 0, 0), ka1 = ka0;
        if (gdn) {
          ka0 = kn[0];
          ka1 = kn[1];
        }
        for (int t0 = 0; t0 < L; t0 += 4) {
          uint4 ea[4][2];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int e = t0 + u < L ? s.en[x0 + t0 + u] : n;
            const uint4* ke = reinterpret_cast<const uint4*>(k + (((size_t)b * N + e) * H + h) * kBD) + 2 * lj;
            ea[u][0] = ke[0];
            ea[u][1] = ke[1];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float sq = dpp_sum8(dot8_bf16(qa1, ea[u][1], dot8_bf16(qa0, ea[u][0], 0.f)));
            const float sk =
                gdn ? dpp_sum8(dot8_bf16(ka1, ea[u][1], dot8_bf16(ka0, ea[u][0], 0.f))) : 0.f;
            const int x = x0 + t0 + u;
            if (lj == 0 && t0 + u < L) {
              const float D = s.cA[x];
              s.cP[x] = D * sq;
              s.cA[x] = t0 + u > 0 ? bn * D * sk : 0.f;
            }
          }
        }
      } else {
        for (int t = 0; t < L; ++t) {
          const int e = s.en[x0 + t];
          const size_t re = ((size_t)b * N + e) * H + h;
          float a = 0.f, c = 0.f;
          for (int i = lj; i < dk; i += 8) {
            const float ke = Elem<TIn>::load(k, re * dk + i);
            a = fmaf(Elem<TIn>::load(q, rn * dk + i), ke, a);
            if (gdn) c = fmaf(Elem<TIn>::load(k, rn * dk + i), ke, c);
          }
          const float sq = dpp_sum8(a);
          const float sk = dpp_sum8(c);
          if (lj == 0) {
            const float D = s.cA[x0 + t];
            s.cP[x0 + t] = D * sq;
            s.cA[x0 + t] = t > 0 ? bn * D * sk : 0.f;
          }
        }
      }
    }
    __syncthreads();

    // level solve: u_n = R_n - sum_{t >= 1} A[n, e_t] u_{e_t}
    if (gdn) {
      const int dlo = s.len[s.ord[p0]] - 1;
      const int dhi = s.len[s.ord[p1 - 1]] - 1;
      for (int l = dlo > 1 ? dlo : 1; l <= dhi; ++l) {
        const int a = p0 > s.lst[l] ? p0 : s.lst[l];
        const int z = p1 < s.lst[l + 1] ? p1 : s.lst[l + 1];
        for (int it = tid; it < (z - a) * ncg; it += kBT) {
          const int p = a + it / ncg;
          const int col = 4 * (it % ncg);
          const int n = s.ord[p];
          const int x = s.off[p] - e0;
          float4 u = *reinterpret_cast<const float4*>(&s.U[urow(n, col, vb)]);
#pragma unroll 4
          for (int t = 1; t <= l; ++t) {
            const float c = s.cA[x + t];
            const float4 w = *reinterpret_cast<const float4*>(&s.U[urow(s.en[x + t], col, vb)]);
            u.x = fmaf(-c, w.x, u.x);
            u.y = fmaf(-c, w.y, u.y);
            u.z = fmaf(-c, w.z, u.z);
            u.w = fmaf(-c, w.w, u.w);
          }
          *reinterpret_cast<float4*>(&s.U[urow(n, col, vb)]) = u;
        }
        __syncthreads();
      }
    }

    // outputs of the chunk's nodes
    for (int it = tid; it < (p1 - p0) * ncg; it += kBT) {
      const int p = p0 + it / ncg;
      const int col = 4 * (it % ncg);
      const int n = s.ord[p];
      const int x = s.off[p] - e0;
      const int L = s.len[n];
      float4 acc = *reinterpret_cast<const float4*>(&s.QS[urow(n, col, vb)]);
#pragma unroll 4
      for (int t = 0; t < L; ++t) {
        const float c = s.cP[x + t];
        const float4 w = *reinterpret_cast<const float4*>(&s.U[urow(s.en[x + t], col, vb)]);
        acc = fma4(c, w, acc);
      }
      Elem<TIn>::store4(o, (((size_t)b * N + n) * H + h) * dv + c0 + col, acc);
      *reinterpret_cast<float4*>(U + ((size_t)bh * N + n) * dv + c0 + col) =
          *reinterpret_cast<const float4*>(&s.U[urow(n, col, vb)]);
    }
    __syncthreads();
    p0 = p1;
  }
}

}  // namespace

int launch_verify_blocked(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                          const void* k, const void* v, const float* alpha, const float* beta,
                          const int32_t* parents, const float* S_root, void* o, float* U,
                          int32_t* status, hipStream_t stream) {
  const int vb = dv < kBVB ? dv : kBVB;
  const long long nblocks = (long long)B * H * (dv / vb);
  if (nblocks > 0x7fffffffLL) return static_cast<int>(hipErrorInvalidConfiguration);
  const dim3 grid((unsigned)nblocks), block(kBT);
  if (dtype == 1 && dk == kBD && dv == kBD) {
    hipLaunchKernelGGL((verify_blocked_kernel<uint16_t, true>), grid, block, 0, stream, H, N, dk,
                       dv, mode, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), alpha, beta, parents, S_root,
                       static_cast<uint16_t*>(o), U, status);
  } else if (dtype == 1) {
    hipLaunchKernelGGL((verify_blocked_kernel<uint16_t, false>), grid, block, 0, stream, H, N, dk,
                       dv, mode, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), alpha, beta, parents, S_root,
                       static_cast<uint16_t*>(o), U, status);
  } else {
    hipLaunchKernelGGL((verify_blocked_kernel<float, false>), grid, block, 0, stream, H, N, dk, dv,
                       mode, static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), alpha, beta, parents, S_root,
                       static_cast<float*>(o), U, status);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace tv
