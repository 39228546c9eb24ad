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
// The tree's path entries (node n, ancestor j) are laid out node after node
// with nodes sorted by depth.  One workgroup of 1024 threads handles one
// (sequence b, head h) and loops over the value columns in blocks of up to 32:
//   1. tree index: pointer jumping gives each node's path length and gamma;
//      nodes are sorted by depth (counting sort) and given entry offsets;
//   2. path walk (entry nodes and decays) and Gram values, one 8-lane group
//      per node, four of its entries in flight (the ancestor-masked
//      Gram/decay builder);
//   3. per column block: R and gamma QS (on matrix cores for bf16 with
//      d_k = d_v = 128, 32x32x16 bf16 with S split into hi + lo words; fp32
//      FMA otherwise), then the solve and the outputs, U and o stored once.
//
// Resident trees (their entries fit in LDS: up to 3040 with bf16 inputs, 1400
// with fp32) are walked and given Gram values once.  The solve is then a
// product with the inverse of I + A: it is nonzero only on root paths, like A,
// so its rows and the output weights are formed once per entry, and each
// column block is one gather over R rows.  For bf16 at d = 128 the q and k
// tiles also stay in registers for all column blocks and gamma QS stays in the
// accumulator lanes.  Deeper trees go in chunks of entries, walked again for
// every column block and solved one depth level at a time (a node's ancestors
// sit in earlier levels, so they are final by then); any depth goes through.
//
// One workgroup fills most of a CU's LDS (R for 512 nodes x 32 columns, gamma
// QS, the S block and the entries), so a CU runs one at a time and latency is
// hidden inside the workgroup: sixteen waves, loads issued a phase ahead of
// use.
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {

namespace {

constexpr int kBT = 1024;   // threads per workgroup (16 waves: one node tile each)
constexpr int kBVB = 32;    // value columns per pass (d_v when d_v < 32)
constexpr int kBD = 128;    // d_k = d_v of the matrix-core contraction

// Path entries LDS has room for: gamma QS is kept in the input type (bf16 o
// is rounded to it anyway), which leaves more room with bf16 inputs.
template <typename TIn>
constexpr int blocked_entries() { return sizeof(TIn) == 2 ? 3040 : 1400; }

typedef __bf16 bbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bbf16x2 __attribute__((ext_vector_type(2)));
typedef float bf32x16 __attribute__((ext_vector_type(16)));

template <typename TIn>
struct __align__(16) BlockedLds {  // 16-byte aligned: float4 rows read as one 128-bit access
  static constexpr int kEnt = blocked_entries<TIn>();
  float U[kMaxTree * kBVB];   // R rows, solved in place into U rows (row stride = columns);
                              // on the resident matrix-core path first half of the k rows
  union {
    TIn QS[kMaxTree * kBVB];  // gamma_n QS_n rows, in the input type
    struct {                  // resident matrix-core path (gamma QS stays in registers)
      float kk[kEnt];         // first half of k_n . k_j per entry
      float Tw[kEnt];         // T = (I + A)^-1 on the entries
      uint16_t erow[kEnt];    // first entry of the entry's path node (its row)
    } r;
  };
  float Sst[sizeof(TIn) == 2 ? kBD * kBVB : 1];  // S block of the matrix-core path, as
                                                 // bf16 hi and lo words (stage_s)
  float cA[kEnt];             // decay during the walk, then A = beta_n D (k_n.k_j) (1 on
                              // the node's own entry), then T = (I + A)^-1 if resident
  float cP[kEnt];             // D (q_n.k_j), then the output weights of R if resident
  uint16_t en[kEnt];          // the entry's path node j
  int16_t par[kMaxTree];
  int16_t jmp[kMaxTree];      // jump targets, then node -> position
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

// OR of x over the workgroup with an LDS-only barrier (no wait for this
// wave's outstanding global loads), for the tree index only: the votes sit
// at the start of the R rows, which are not in use before the contraction.
// Each wave posts its vote to its own slot of round r % 2, so no slot needs
// clearing; a round's slots are read after its barrier and written again two
// rounds later, past at least one more barrier.
template <typename TIn>
__device__ __forceinline__ bool workgroup_or(BlockedLds<TIn>& s, bool x, int r) {
  int* vote = reinterpret_cast<int*>(s.U) + (r & 1) * (kBT / 64);
  const int wave = threadIdx.x >> 6;
  const int any = __any(x) ? 1 : 0;
  if ((threadIdx.x & 63) == 0) vote[wave] = any;
  lds_barrier();
  int acc = 0;
#pragma unroll
  for (int w = 0; w < kBT / 64; ++w) acc |= vote[w];
  return acc != 0;
}

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

// Tile rows.  Lane l of a tile holds row (node) l%32 of the tile in the
// matrix-core operand layout.  The node of a lane is passed in (-1: none);
// it is made opaque so that the offsets derived from it are recomputed at
// every call instead of being hoisted out of the column block loop and held,
// or spilled, across it.  Uniform bases go in scalar registers and offsets are
// 32-bit bytes (the launch checks that a sequence's N H 128 bf16 elements fit
// in them).
//
// The loads are issued unconditionally (branches around them make the
// compiler wait for the whole batch at the join): a lane with no row, or a
// load with nothing to fetch, reads the base row, one line per wave.
__device__ __forceinline__ uint32_t tile_rowoff(int node, int H) {
  asm volatile("" : "+v"(node));
  return node >= 0 ? static_cast<uint32_t>(node * H * kBD) * 2u : 0u;
}

// Identity mapping: tile T holds nodes 32 T .. 32 T + 31.
__device__ __forceinline__ int identity_node(int T, int N) {
  const int n = T * 32 + (threadIdx.x & 31);
  return n < N ? n : -1;
}

// q and k of the lane's row: elements 8 (lane/32) + 16 ks
__device__ __forceinline__ void load_tile_qk(TileIn& t, int node, int N, int H, int b, int h,
                                             bool gdn, const uint16_t* __restrict__ q,
                                             const uint16_t* __restrict__ k) {
  const uint32_t hi = (threadIdx.x >> 5) & 1;
  const uint32_t off = tile_rowoff(node, H) + 16u * hi;
  const size_t base = ((size_t)b * N * H + h) * kBD;
  const char* qr = reinterpret_cast<const char*>(q + base) + off;
  const char* kr = reinterpret_cast<const char*>(k + base) + off;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    t.qb[ks] = *reinterpret_cast<const bbf16x8*>(qr + 32 * ks);
    t.kb[ks] = *reinterpret_cast<const bbf16x8*>(kr + 32 * ks);
  }
}

// v of the lane's row at the accumulator's columns: c0 + 8 g + 4 (lane/32) + [0, 4)
__device__ __forceinline__ void load_tile_v(TileIn& t, int node, int N, int H, int b, int h,
                                            int c0, const uint16_t* __restrict__ v) {
  const uint32_t hi = (threadIdx.x >> 5) & 1;
  const uint32_t off = tile_rowoff(node, H) + 8u * hi;
  const char* vr = reinterpret_cast<const char*>(v + ((size_t)b * N * H + h) * kBD + c0) + off;
#pragma unroll
  for (int g = 0; g < 4; ++g) t.vv[g] = *reinterpret_cast<const uint2*>(vr + 16 * g);
}

// This thread's 2 x 2 part of a 128 x 32 S block: rows r0, r0 + 1 with r0 =
// 2 (tid/16), columns c0, c0 + 1 with c0 = 2 (tid%16), as (S[r0][c0],
// S[r0][c0+1], S[r0+1][c0], S[r0+1][c0+1]); the lane offset is opaque so
// that no 64-bit address is held across the phases between two blocks.
__device__ __forceinline__ float4 load_s_part(const float* __restrict__ blk) {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  const uint32_t off = static_cast<uint32_t>((2 * (t >> 4) * kBD + 2 * (t & 15)) * 4);
  const char* p = reinterpret_cast<const char*>(blk) + off;
  const float2 a = *reinterpret_cast<const float2*>(p);
  const float2 c = *reinterpret_cast<const float2*>(p + kBD * 4);
  return make_float4(a.x, a.y, c.x, c.y);
}

// The S block (128 x 32 fp32) is staged once per block for all waves as bf16
// hi + lo words (x = hi + lo to 16 bits), transposed: value column c holds its
// 128 rows in 16 chunks of 8 (16 B), chunk j at slot j ^ (c % 16), so the 32
// columns of one operand read spread over the banks; the hi words fill the
// first 8192 elements, the lo words the next.
__device__ __forceinline__ int sst_off(int c, int j) { return c * kBD + ((j ^ (c & 15)) << 3); }

// This thread's 2 x 2 part of the block (load_s_part): per column, the two
// rows' hi words go out as one 32-bit store, and the lo words as another.
__device__ __forceinline__ void stage_s(float* Sst, float4 x) {
  uint16_t* sh = reinterpret_cast<uint16_t*>(Sst);
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));  // addresses formed at each call, not held across the blocks
  const int r0 = 2 * (t >> 4), c0 = 2 * (t & 15);
  const float v0[2] = {x.x, x.y}, v1[2] = {x.z, x.w};  // rows r0 and r0 + 1
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint16_t h0 = f32_to_bf16(v0[i]), h1 = f32_to_bf16(v1[i]);
    const uint16_t l0 = f32_to_bf16(v0[i] - __uint_as_float(static_cast<uint32_t>(h0) << 16));
    const uint16_t l1 = f32_to_bf16(v1[i] - __uint_as_float(static_cast<uint32_t>(h1) << 16));
    const int idx = sst_off(c0 + i, r0 >> 3) + (r0 & 7);  // even: a whole 32-bit word
    *reinterpret_cast<uint32_t*>(sh + idx) = h0 | (static_cast<uint32_t>(h1) << 16);
    *reinterpret_cast<uint32_t*>(sh + kBD * kBVB + idx) = l0 | (static_cast<uint32_t>(l1) << 16);
  }
}

// One [K or Q] S_block product of a tile on matrix cores: A = S block^T
// (value column x d_k) from the staged hi and lo words, B = op^T (d_k x node)
// from the tile registers.
__device__ __forceinline__ void mma_pass(const bbf16x8 (&op)[8], const float* Sst, bf32x16& acc) {
  const uint16_t* sh = reinterpret_cast<const uint16_t*>(Sst);
  // opaque, so the operand addresses are formed here at each call rather than
  // held (spilled) across the column blocks
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int c = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int o = sst_off(c, 2 * ks + hi);
    const bbf16x8 shi = *reinterpret_cast<const bbf16x8*>(sh + o);
    const bbf16x8 slo = *reinterpret_cast<const bbf16x8*>(sh + kBD * kBVB + o);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi, op[ks], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo, op[ks], acc, 0, 0, 0);
  }
  // operand reads one step ahead of their products, no further (registers)
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int ks = 0; ks < 7; ++ks) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

// R and gamma QS of one tile into LDS: the accumulator puts node lane%32 and
// value columns 8 (r/4) + 4 (lane/32) + r%4 in lane `lane`.  Q first, then K,
// one accumulator at a time.
__device__ __forceinline__ void contract_store(BlockedLds<uint16_t>& s, const TileIn& t, int T, int N,
                                               bool gdn) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // row addresses formed here, not held across the blocks
  const int n = T * 32 + (lane & 31);
  const bool live = n < N;
  const int nn = live ? n : 0;
  const float gn = s.gam[nn], bn = s.bet[nn];
  bf32x16 acc;
  mma_pass(t.qb, s.Sst, acc);
  if (live) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      Elem<uint16_t>::store4(s.QS, urow(n, 8 * g + 4 * (lane >> 5), kBVB),
                             make_float4(gn * acc[4 * g + 0], gn * acc[4 * g + 1],
                                         gn * acc[4 * g + 2], gn * acc[4 * g + 3]));
  }
  if (gdn) mma_pass(t.kb, s.Sst, acc);
  if (!live) return;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint2 w = t.vv[g];
    const float4 vf = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    float4 r = vf;
    if (gdn) {
      r.x = bn * (vf.x - gn * acc[4 * g + 0]);
      r.y = bn * (vf.y - gn * acc[4 * g + 1]);
      r.z = bn * (vf.z - gn * acc[4 * g + 2]);
      r.w = bn * (vf.w - gn * acc[4 * g + 3]);
    }
    *reinterpret_cast<float4*>(&s.U[urow(n, 8 * g + 4 * (lane >> 5), kBVB)]) = r;
  }
}

// The contraction for the register-resident path: R row of the lane's node
// n (-1: none) into LDS, gamma QS kept in the accumulator lanes as bf16 (the
// precision it has in o), four value columns 8 g + 4 (lane/32) + [0, 4) per
// group g.  The matrix instructions run in every wave (rows without a node
// hold the base row and are not stored).
__device__ __forceinline__ void contract_keep(BlockedLds<uint16_t>& s, const TileIn& t, int n,
                                              bool gdn, uint2 (&gq)[4]) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(n), "+v"(lane));  // R row addresses formed here, not held across the blocks
  const bool live = n >= 0;
  const int nn = live ? n : 0;
  const float gn = s.gam[nn], bn = s.bet[nn];
  bf32x16 acc;
  mma_pass(t.qb, s.Sst, acc);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    gq[g].x = static_cast<uint32_t>(f32_to_bf16(gn * acc[4 * g + 0])) |
              (static_cast<uint32_t>(f32_to_bf16(gn * acc[4 * g + 1])) << 16);
    gq[g].y = static_cast<uint32_t>(f32_to_bf16(gn * acc[4 * g + 2])) |
              (static_cast<uint32_t>(f32_to_bf16(gn * acc[4 * g + 3])) << 16);
  }
  if (gdn) mma_pass(t.kb, s.Sst, acc);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint2 w = t.vv[g];
    const float4 vf = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    float4 r = vf;
    if (gdn) {
      r.x = bn * (vf.x - gn * acc[4 * g + 0]);
      r.y = bn * (vf.y - gn * acc[4 * g + 1]);
      r.z = bn * (vf.z - gn * acc[4 * g + 2]);
      r.w = bn * (vf.w - gn * acc[4 * g + 3]);
    }
    if (live) *reinterpret_cast<float4*>(&s.U[urow(n, 8 * g + 4 * (lane >> 5), kBVB)]) = r;
  }
}

// Outputs of the lane's own node n (-1: none) at the columns whose gamma QS
// it holds: o_n = gamma_n QS_n + sum_s W[n, e_s] R_{e_s} and u_n =
// sum_s T[n, e_s] R_{e_s}, two column groups per pass over the entries.
__device__ __forceinline__ void gather_owner(BlockedLds<uint16_t>& s, const uint2 (&gq)[4], int n,
                                             int N, int H, int b, int h, int bh, int c0,
                                             uint16_t* __restrict__ o, float* __restrict__ U) {
  asm volatile("" : "+v"(n));  // offsets computed here, not held across the block loop
  const int hi = (threadIdx.x >> 5) & 1;
  if (n < 0) return;
  const int x = s.off[s.jmp[n]];
  const int L = s.len[n];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int ca = 16 * half + 4 * hi, cc = ca + 8;
    const uint2 g0 = gq[2 * half], g1 = gq[2 * half + 1];
    float4 a0 = make_float4(__uint_as_float(g0.x << 16), __uint_as_float(g0.x & 0xffff0000u),
                            __uint_as_float(g0.y << 16), __uint_as_float(g0.y & 0xffff0000u));
    float4 a1 = make_float4(__uint_as_float(g1.x << 16), __uint_as_float(g1.x & 0xffff0000u),
                            __uint_as_float(g1.y << 16), __uint_as_float(g1.y & 0xffff0000u));
    float4 u0 = f4(0.f), u1 = f4(0.f);
#pragma unroll 2
    for (int t = 0; t < L; ++t) {
      const int e = s.en[x + t];
      const float wt = s.r.Tw[x + t], wp = s.cP[x + t];
      const float4 r0 = *reinterpret_cast<const float4*>(&s.U[urow(e, ca, kBVB)]);
      const float4 r1 = *reinterpret_cast<const float4*>(&s.U[urow(e, cc, kBVB)]);
      a0 = fma4(wp, r0, a0);
      a1 = fma4(wp, r1, a1);
      u0 = fma4(wt, r0, u0);
      u1 = fma4(wt, r1, u1);
    }
    const size_t orow = (((size_t)b * N + n) * H + h) * kBD + c0;
    Elem<uint16_t>::store4(o, orow + ca, a0);
    Elem<uint16_t>::store4(o, orow + cc, a1);
    float* ur = U + ((size_t)bh * N + n) * kBD + c0;
    *reinterpret_cast<float4*>(ur + ca) = u0;
    *reinterpret_cast<float4*>(ur + cc) = u1;
  }
}

// The same with fp32 FMA, any d_k, d_v and input type; item = (node, 4 columns).
template <typename TIn>
__device__ void contract_fma(BlockedLds<TIn>& s, int N, int H, int dk, int dv, int vb, int b, int h,
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
    Elem<TIn>::store4(s.QS, urow(n, col, vb), mul4(gn, qs));
  }
}

// ---- per-chunk phases: positions [p0, p1) of the depth order, their path
// entries stored from entry e0 on ----

// Last position + 1 of the chunk that starts at p0: as many nodes as have all
// their entries within kEnt of e0 (a node has at most 512 entries, so at
// least one node fits).
template <typename TIn>
__device__ __forceinline__ int chunk_end(BlockedLds<TIn>& s, int p0, int N) {
  const int e0 = s.off[p0];
  const int qpos = p0 + 1 + threadIdx.x;
  return p0 + __syncthreads_count(qpos <= N && s.off[qpos] - e0 <= BlockedLds<TIn>::kEnt);
}

// Path walk: entry t of node n is (n, e_t) with decay D(e_t -> n).
template <typename TIn>
__device__ __forceinline__ void walk_entries(BlockedLds<TIn>& s, int p0, int p1, int e0) {
  for (int p = p0 + threadIdx.x; p < p1; p += kBT) {
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
}

// Gram values of the entries: cP = D (q_n.k_j), cA = beta_n D (k_n.k_j) (0 for
// the node's own entry).  One 8-lane group per node, its q and k rows loaded
// once, its entries four at a time.
template <typename TIn, bool MFMA>
__device__ __forceinline__ void gram_entries(BlockedLds<TIn>& s, int p0, int p1, int e0, int N,
                                             int H, int dk, int b, int h, bool gdn,
                                             const TIn* __restrict__ q,
                                             const TIn* __restrict__ k) {
  const int grp = threadIdx.x >> 3, lj = threadIdx.x & 7;
  constexpr int kGroups = kBT / 8;
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
            s.cA[x] = t0 + u > 0 ? bn * D * sk : 1.f;
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
          s.cA[x0 + t] = t > 0 ? bn * D * sk : 1.f;
        }
      }
    }
  }
}

// Level solve u_n = R_n - sum_{t >= 1} A[n, e_t] u_{e_t}, one depth level at a
// time (a barrier after each); the chunk's lower levels were solved before.
template <typename TIn>
__device__ __forceinline__ void level_solve(BlockedLds<TIn>& s, int p0, int p1, int e0, int vb) {
  const int ncg = vb / 4;
  const int dlo = s.len[s.ord[p0]] - 1;
  const int dhi = s.len[s.ord[p1 - 1]] - 1;
  for (int l = dlo > 1 ? dlo : 1; l <= dhi; ++l) {
    const int a = p0 > s.lst[l] ? p0 : s.lst[l];
    const int z = p1 < s.lst[l + 1] ? p1 : s.lst[l + 1];
    for (int it = threadIdx.x; it < (z - a) * ncg; it += kBT) {
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
    lds_barrier();
  }
}

// Outputs of the chunk's nodes for value columns [c0, c0 + vb): o_n =
// gamma_n QS_n + sum_t cP u_{e_t}, and the U rows, each stored to HBM once.
template <typename TIn>
__device__ __forceinline__ void chunk_outputs(BlockedLds<TIn>& s, int p0, int p1, int e0, int vb,
                                              int N, int H, int dv, int b, int h, int bh, int c0,
                                              TIn* __restrict__ o, float* __restrict__ U) {
  const int ncg = vb / 4;
  for (int it = threadIdx.x; it < (p1 - p0) * ncg; it += kBT) {
    const int p = p0 + it / ncg;
    const int col = 4 * (it % ncg);
    const int n = s.ord[p];
    const int x = s.off[p] - e0;
    const int L = s.len[n];
    float4 acc = Elem<TIn>::load4(s.QS, urow(n, col, vb));
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
}

// ---- resident trees on the matrix-core path: Gram values from the tiles ----
//
// The q and k tiles are loaded into registers once, before the Gram: each
// lane pair (lm, lm + 32) of wave w holds the node at depth-order position
// 32 w + lm (elements 16 ks + 8 (lane/32) + [0, 8)).  The k rows are staged
// in LDS one half of d_k at a time (64 bf16 a row, 64 KB for 512 nodes, over
// the R rows, which are not in use yet), and each lane pair forms its node's
// path products q_n . k_j and k_n . k_j against the staged rows: every q and
// k row is read from memory once.

// Path walk that also records, for each entry, the first entry of the
// entry's node (its row): entry t of node n is (n, e_t) with D(e_t -> n).
template <typename TIn>
__device__ __forceinline__ void walk_entries_rows(BlockedLds<TIn>& s, int N) {
  for (int p = threadIdx.x; p < N; p += kBT) {
    const int n = s.ord[p];
    int x = s.off[p];
    float D = 1.f;
    for (int e = n; e >= 0; e = s.par[e]) {
      s.en[x] = static_cast<uint16_t>(e);
      s.r.erow[x] = static_cast<uint16_t>(s.off[s.jmp[e]]);
      s.cA[x] = D;
      D *= s.alp[e];
      ++x;
    }
  }
}

// Staged half of a k row: 8 chunks of 16 B (chunk c = elements 8 c .. 8 c + 7
// of the half) at slot c ^ (row % 8), so lanes reading chunk c of different
// rows spread over the banks.
__device__ __forceinline__ int kst_off(int row, int c) { return row * 64 + ((c ^ (row & 7)) << 3); }

__device__ __forceinline__ float dot8_bf16x8(bbf16x8 a, uint4 b, float acc) {
  uint4 ua;
  __builtin_memcpy(&ua, &a, 16);
  return dot8_bf16(ua, b, acc);
}

// Sum over lanes l and l ^ 32.
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Gram values of every entry from the register tiles: cP = D (q_n.k_j),
// cA = beta_n D (k_n.k_j) (1 on the node's own entry); pos = the lane's
// depth-order position, n its node (-1: none).
__device__ __forceinline__ void gram_tiles(BlockedLds<uint16_t>& s, const TileIn& t, int pos, int n) {
  const int lane = threadIdx.x & 63;
  const int hi = lane >> 5;
  uint16_t* Kst = reinterpret_cast<uint16_t*>(s.U);
  const bool live = n >= 0;
  const int x0 = live ? s.off[pos] : 0;
  const int L = live ? s.len[n] : 0;
  const int Lw = __builtin_amdgcn_readfirstlane(__reduce_max_sync(~0ull, L));  // wave's longest path
  const float bn = live ? s.bet[n] : 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (live) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bbf16x8 w = t.kb[4 * half + j];
        *reinterpret_cast<bbf16x8*>(Kst + kst_off(n, 2 * j + hi)) = w;
      }
    }
    lds_barrier();  // the half's k rows staged
    for (int i = 0; i < Lw; ++i) {
      const int e = i < L ? s.en[x0 + i] : (live ? n : 0);
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 ke = *reinterpret_cast<const uint4*>(Kst + kst_off(e, 2 * j + hi));
        sq = dot8_bf16x8(t.qb[4 * half + j], ke, sq);
        sk = dot8_bf16x8(t.kb[4 * half + j], ke, sk);
      }
      sq = xor32_sum(sq);
      sk = xor32_sum(sk);
      if (hi == 0 && i < L) {
        const int x = x0 + i;
        if (half == 0) {
          s.cP[x] = sq;
          s.r.kk[x] = sk;
        } else {
          const float D = s.cA[x];
          s.cP[x] = D * (s.cP[x] + sq);
          s.cA[x] = i > 0 ? bn * D * (s.r.kk[x] + sk) : 1.f;  // beta is 0 without the delta rule
        }
      }
    }
    lds_barrier();  // the half's products are read (and the rows are free)
  }
}

// T = (I + A)^-1 and the output weights, node by node (no depth levels).  Row
// n of T restricted to n's path e_0 = n, e_1, ... solves x (I + A) = e_n:
//   x_0 = 1,  x_s = - sum_{t<s} x_t A[e_t, e_s],
// where A[e_t, e_s] is entry s - t of e_t's own row (e_s sits s - t steps above
// e_t).  The output weights W[n, e_s] = sum_{t<=s} Pc[n, e_t] T[e_t, e_s] need
// the ancestors' T rows, so they follow a barrier; they replace Pc in place
// (entry s reads entries t <= s of its own row only, so s runs downwards).
//
// Paths of up to kPathRegs nodes keep a row in registers and go through it
// ancestor by ancestor: after x_t is final, its products with e_t's own row
// (entries 1, 2, ... of that row, at consecutive addresses) are added to the
// later x_s.  Longer paths run the same sums through LDS.
constexpr int kPathRegs = 16;

__device__ __forceinline__ void path_inverse(BlockedLds<uint16_t>& s, int N) {
  for (int p = threadIdx.x; p < N; p += kBT) {
    const int x0 = s.off[p];
    const int L = s.len[s.ord[p]];
    if (L <= kPathRegs) {
      float acc[kPathRegs];
#pragma unroll
      for (int sp = 0; sp < kPathRegs; ++sp) acc[sp] = (sp > 0 && sp < L) ? s.cA[x0 + sp] : 0.f;
      s.r.Tw[x0] = 1.f;
#pragma unroll
      for (int t = 1; t < kPathRegs; ++t) {
        if (t < L) {
          const float xt = -acc[t];
          s.r.Tw[x0 + t] = xt;
          const float* At = s.cA + s.r.erow[x0 + t];
#pragma unroll
          for (int sp = t + 1; sp < kPathRegs; ++sp)
            if (sp < L) acc[sp] = fmaf(xt, At[sp - t], acc[sp]);
        }
      }
    } else {
      s.r.Tw[x0] = 1.f;
      for (int sp = 1; sp < L; ++sp) {
        float acc = s.cA[x0 + sp];  // t = 0: x_0 A[n, e_s] with x_0 = 1
        for (int t = 1; t < sp; ++t) acc = fmaf(s.r.Tw[x0 + t], s.cA[s.r.erow[x0 + t] + (sp - t)], acc);
        s.r.Tw[x0 + sp] = -acc;
      }
    }
  }
  lds_barrier();
  for (int p = threadIdx.x; p < N; p += kBT) {
    const int x0 = s.off[p];
    const int L = s.len[s.ord[p]];
    if (L <= kPathRegs) {
      float w[kPathRegs];
#pragma unroll
      for (int sp = 0; sp < kPathRegs; ++sp) w[sp] = 0.f;
#pragma unroll
      for (int t = 0; t < kPathRegs; ++t) {
        if (t < L) {
          const float pt = s.cP[x0 + t];
          const float* Tt = s.r.Tw + s.r.erow[x0 + t];
          w[t] += pt;  // T[e_t, e_t] = 1
#pragma unroll
          for (int sp = t + 1; sp < kPathRegs; ++sp)
            if (sp < L) w[sp] = fmaf(pt, Tt[sp - t], w[sp]);
        }
      }
#pragma unroll
      for (int sp = 0; sp < kPathRegs; ++sp)
        if (sp < L) s.cP[x0 + sp] = w[sp];
    } else {
      for (int sp = L - 1; sp >= 0; --sp) {
        float acc = s.cP[x0 + sp];  // t = s: T[e_s, e_s] = 1
        for (int t = 0; t < sp; ++t) acc = fmaf(s.cP[x0 + t], s.r.Tw[s.r.erow[x0 + t] + (sp - t)], acc);
        s.cP[x0 + sp] = acc;
      }
    }
  }
  lds_barrier();
}

// ---- resident trees: the solve as a product with the inverse ----
//
// T = (I + A)^-1 is supported on root paths like A (products of path-supported
// matrices stay path-supported), so U = T R needs, per node, only its own
// path entries: u_n = sum_s T[n, e_s] R_{e_s}.  From T = I - A T, entry s of
// node n's row is
//   T[n, e_s] = - sum_{t=1..s} A[n, e_t] T[e_t, e_s],
// where T[e_t, e_s] is entry s - t of ancestor e_t's row (1 when t = s).  Rows
// are computed one depth level at a time, in place of A: each value is held
// in a register until the level's reads are done.  The outputs then fold in T
// the same way, o_n = gamma_n QS_n + sum_s W[n, e_s] R_{e_s} with
//   W[n, e_s] = sum_{t=0..s} Pc[n, e_t] T[e_t, e_s],   Pc[n, j] = D(j->n) (q_n.k_j),
// in place of Pc.  Both are scalar work per path entry, done once for all
// column blocks; each block is then one gather over R rows with no levels.
constexpr int kItemsPerThread = 3;  // path entries per thread (kEnt <= 3 kBT)

template <typename TIn>
__device__ __forceinline__ void tree_inverse(BlockedLds<TIn>& s, int N) {
  static_assert(BlockedLds<TIn>::kEnt <= kItemsPerThread * kBT, "entries per thread");
  const int maxd = s.len[s.ord[N - 1]] - 1;
  for (int l = 1; l <= maxd; ++l) {
    const int a = s.lst[l];
    const int items = (s.lst[l + 1] - a) * l;  // entries s = 1..l of the level's nodes
    float val[kItemsPerThread];
    int dst[kItemsPerThread];
#pragma unroll
    for (int r = 0; r < kItemsPerThread; ++r) {
      const int it = threadIdx.x + r * kBT;
      dst[r] = -1;
      val[r] = 0.f;
      if (it < items) {
        const int p = a + it / l;
        const int sp = 1 + it % l;
        const int x = s.off[p];
        float acc = 0.f;
        for (int t = 1; t <= sp; ++t) {
          const int xe = s.off[s.jmp[s.en[x + t]]];  // ancestor e_t's row
          acc = fmaf(s.cA[x + t], s.cA[xe + sp - t], acc);
        }
        val[r] = -acc;
        dst[r] = x + sp;
      }
    }
    lds_barrier();
#pragma unroll
    for (int r = 0; r < kItemsPerThread; ++r)
      if (dst[r] >= 0) s.cA[dst[r]] = val[r];
    lds_barrier();
  }
  // output weights of every entry (all T rows are final)
  const int nent = s.off[N];
  float val[kItemsPerThread];
#pragma unroll
  for (int r = 0; r < kItemsPerThread; ++r) {
    const int x = threadIdx.x + r * kBT;
    val[r] = 0.f;
    if (x < nent) {
      int d = 0;
      while (s.ebase[d + 1] <= x) ++d;  // the entry's depth: rows of length d + 1
      const int sp = (x - s.ebase[d]) % (d + 1);
      const int xn = x - sp;             // node n's row
      float acc = 0.f;
      for (int t = 0; t <= sp; ++t) {
        const int xe = t == 0 ? xn : s.off[s.jmp[s.en[xn + t]]];
        acc = fmaf(s.cP[xn + t], s.cA[xe + sp - t], acc);
      }
      val[r] = acc;
    }
  }
  lds_barrier();
#pragma unroll
  for (int r = 0; r < kItemsPerThread; ++r) {
    const int x = threadIdx.x + r * kBT;
    if (x < nent) s.cP[x] = val[r];
  }
  lds_barrier();
}

// u_n and o_n of every node for value columns [c0, c0 + vb) from the R rows
// (left unchanged in LDS) and the entries' T and output weights.
template <typename TIn>
__device__ __forceinline__ void gather_outputs(BlockedLds<TIn>& s, int vb, int N, int H, int dv,
                                               int b, int h, int bh, int c0,
                                               TIn* __restrict__ o, float* __restrict__ U) {
  const int ncg = vb / 4;
  // positions are sorted by depth, so rounds alternate the lane order: each
  // wave gets shallow and deep nodes alike
  for (int r = 0; r * kBT < N * ncg; ++r) {
    const int it = r * kBT + ((r & 1) ? kBT - 1 - (int)threadIdx.x : (int)threadIdx.x);
    if (it >= N * ncg) continue;
    const int p = it / ncg;
    const int col = 4 * (it % ncg);
    const int n = s.ord[p];
    const int x = s.off[p];
    const int L = s.len[n];
    float4 acc = Elem<TIn>::load4(s.QS, urow(n, col, vb));
    float4 u = f4(0.f);
#pragma unroll 4
    for (int t = 0; t < L; ++t) {
      const float4 w = *reinterpret_cast<const float4*>(&s.U[urow(s.en[x + t], col, vb)]);
      acc = fma4(s.cP[x + t], w, acc);
      u = fma4(s.cA[x + t], w, u);
    }
    Elem<TIn>::store4(o, (((size_t)b * N + n) * H + h) * dv + c0 + col, acc);
    *reinterpret_cast<float4*>(U + ((size_t)bh * N + n) * dv + c0 + col) = u;
  }
}

template <typename TIn, bool MFMA>
__global__ __launch_bounds__(kBT) void verify_blocked_kernel(
    int H, int N, int dk, int dv, int mode, const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ parents, const float* __restrict__ S_root, TIn* __restrict__ o,
    float* __restrict__ U, int32_t* __restrict__ status) {
  __shared__ BlockedLds<TIn> s;
  constexpr int kEnt = BlockedLds<TIn>::kEnt;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vb = dv < kBVB ? dv : kBVB;
  const int nvb = dv / vb;
  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bh % H;
  const int b = bh / H;
  const bool gdn = mode == kGdn;
  const int ntiles = (N + 31) / 32;

  // small loads first (loads return in order): parents and gates
  const int pn = tid < N ? tid : N - 1;
  int p_in = parents[(size_t)b * N + pn];
  const float a_in = alpha[((size_t)b * N + pn) * H + h];
  const float b_in = gdn ? beta[((size_t)b * N + pn) * H + h] : 0.f;

  // matrix-core path: a column block's S block (128 x 32 fp32, 16 KB, one
  // float4 per thread) and the wave's node tile are loaded into registers one
  // phase ahead of their use.  The first block's S part is in flight during
  // the tree build; its tiles load after the Gram values (before the tree
  // build every workgroup would fetch them at once and the build would wait).
  static_assert(kBT * 4 == kBD * kBVB, "one float4 of the S block per thread");
  static_assert(kMaxTree / 32 <= kBT / 64, "a node tile per wave");
  TileIn t0;
  float4 snext;
// (straight-line: without a load to do, the first block's S rows or one line
// per wave are read); v, which only the contraction's last step needs, is
// loaded later
#define TV_LOAD_S(c0, load)                                                                \
  if constexpr (MFMA) snext = load_s_part(S_root + (size_t)bh * kBD * kBD + ((load) ? (c0) : 0));
#define TV_LOAD_QK(node, load)                                                             \
  if constexpr (MFMA) {                                                                    \
    load_tile_qk(t0, (load) ? (node) : -1, N, H, b, h, gdn,                                \
                 reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k)); \
  }
#define TV_LOAD_V(node, c0, load)                                                          \
  if constexpr (MFMA) {                                                                    \
    load_tile_v(t0, (load) ? (node) : -1, N, H, b, h, (load) ? (c0) : 0,                   \
                reinterpret_cast<const uint16_t*>(v));                                     \
  }
  // R and gamma QS of every node for columns [c0, c0 + vb) into LDS (the S
  // block already staged)
#define TV_CONTRACT(c0)                                                                    \
  if constexpr (MFMA) {                                                                    \
    if (wave < ntiles) {                                                                   \
      contract_store(s, t0, wave, N, gdn);                                                 \
    }                                                                                      \
  } else {                                                                                 \
    contract_fma<TIn>(s, N, H, dk, dv, vb, b, h, bh, (c0), gdn, q, k, v, S_root);          \
  }
  TV_LOAD_S(0, true)

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
  const bool bad = workgroup_or(s, my_bad, 0);
  // pointer jumping: a node's span (path nodes from it up to, not including,
  // its jump target) absorbs the target's span until the jump runs off the root
  for (int round = 1;; ++round) {
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
    if (!workgroup_or(s, j >= 0, round)) break;
    if (j >= 0) {
      s.jmp[tid] = static_cast<int16_t>(nj);
      s.len[tid] = static_cast<int16_t>(s.len[tid] + nl);
      s.gam[tid] *= ng;
    }
    lds_barrier();
  }
  // counting sort by depth
  int my_d = 0;
  if (tid < N) {
    my_d = s.len[tid] - 1;
    atomicAdd(&s.hist[my_d], 1);
    atomicMax(&s.maxd, my_d);
  }
  lds_barrier();
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
  lds_barrier();
  if (tid < N) {
    const int pos = s.lst[my_d] + atomicSub(&s.hist[my_d], 1) - 1;
    s.ord[pos] = static_cast<int16_t>(tid);
    s.jmp[tid] = static_cast<int16_t>(pos);  // pointer jumping is over
    s.off[pos] = s.ebase[my_d] + (pos - s.lst[my_d]) * (my_d + 1);
  }
  if (tid == 0) s.off[N] = s.ebase[maxd + 1];
  if (h == 0 && tid == 0 && status) status[b] = bad ? 1 : 0;
  if constexpr (MFMA) stage_s(s.Sst, snext);
  lds_barrier();

  // Chunks of path entries, as many as LDS holds.  When the whole tree's
  // entries fit (one chunk), they are walked, given their Gram values and
  // turned into T and output weights once, and each column block is one
  // gather; otherwise every block walks its chunks again and solves them
  // level by level.  The last chunk of a block is peeled out of the chunk
  // loop: the next block's S block and node tile load during its solve and
  // outputs.
  const bool resident = s.off[N] <= kEnt;
  if constexpr (MFMA) {
    if (resident) {
      // matrix-core path, entries resident: the q and k tiles are loaded once
      // and stay in registers for every column block (no re-reads), gamma QS
      // stays in the accumulator lanes, and each lane finishes the outputs of
      // its own node
      // tile T holds the nodes at depth-order positions 32 T .. 32 T + 31:
      // the lanes of a wave finish nodes of one depth, so their loops over
      // the path entries end together
      const int pj = 32 * wave + (tid & 31);
      const int myn = pj < N ? s.ord[pj] : -1;
      TV_LOAD_QK(myn, true)
      walk_entries_rows(s, N);
      lds_barrier();
      gram_tiles(s, t0, pj, myn);
      path_inverse(s, N);
      for (int cb = 0;;) {
        const int c0 = cb * vb;
        uint2 gq[4];
        TV_LOAD_V(myn, c0, true)  // needed at the end of the contraction
        contract_keep(s, t0, myn, gdn, gq);
        const bool more = cb + 1 < nvb;
        TV_LOAD_S(c0 + vb, more)
        lds_barrier();  // R rows in LDS
        gather_owner(s, gq, myn, N, H, b, h, bh, c0, o, U);
        if (more) stage_s(s.Sst, snext);  // the block's products are done
        lds_barrier();
        if (!more) break;
        ++cb;
      }
      return;
    }
  }
  const int idn = wave < ntiles ? identity_node(wave, N) : -1;  // tile rows: identity mapping
  if (resident) {
    // the first block's node tiles load during the inverse (not before: every
    // workgroup would fetch them at once and the tree build would wait)
    walk_entries(s, 0, N, 0);
    lds_barrier();
    gram_entries<TIn, MFMA>(s, 0, N, 0, N, H, dk, b, h, gdn, q, k);
    lds_barrier();
    TV_LOAD_QK(idn, true)
    TV_LOAD_V(idn, 0, true)
    if (gdn) tree_inverse(s, N);
  } else {
    TV_LOAD_QK(idn, true)
    TV_LOAD_V(idn, 0, true)
  }
  TV_CONTRACT(0)
  for (int cb = 0;;) {
    const int c0 = cb * vb;
    int p0 = 0, p1, e0;
    while (true) {
      e0 = s.off[p0];
      p1 = chunk_end(s, p0, N);  // N at once when resident
      if (!resident) {
        walk_entries(s, p0, p1, e0);
        lds_barrier();
        gram_entries<TIn, MFMA>(s, p0, p1, e0, N, H, dk, b, h, gdn, q, k);
      }
      lds_barrier();
      if (p1 == N) break;
      if (gdn) level_solve(s, p0, p1, e0, vb);
      chunk_outputs(s, p0, p1, e0, vb, N, H, dv, b, h, bh, c0, o, U);
      lds_barrier();
      p0 = p1;
    }
    const bool more = cb + 1 < nvb;
    TV_LOAD_S(c0 + vb, more)
    if (resident) {
      gather_outputs(s, vb, N, H, dv, b, h, bh, c0, o, U);
    } else {
      if (gdn) level_solve(s, p0, N, e0, vb);
      chunk_outputs(s, p0, N, e0, vb, N, H, dv, b, h, bh, c0, o, U);
    }
    if constexpr (MFMA) {
      if (more) stage_s(s.Sst, snext);  // the block's products are done
    }
    lds_barrier();
    if (!more) break;
    ++cb;
    // the next block's tiles load only now: holding them through the chunks'
    // solves would take more registers than a workgroup of 1024 has
    TV_LOAD_QK(idn, true)
    TV_LOAD_V(idn, c0 + vb, true)
    TV_CONTRACT(c0 + vb)
    lds_barrier();
  }
#undef TV_LOAD_S
#undef TV_LOAD_QK
#undef TV_LOAD_V
#undef TV_CONTRACT
}

}  // namespace

int launch_verify_blocked(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                          const void* k, const void* v, const float* alpha, const float* beta,
                          const int32_t* parents, const float* S_root, void* o, float* U,
                          int32_t* status, hipStream_t stream) {
  const long long nblocks = (long long)B * H;  // one workgroup per (sequence, head)
  if (nblocks > 0x7fffffffLL) return static_cast<int>(hipErrorInvalidConfiguration);
  const dim3 grid((unsigned)nblocks), block(kBT);
  if (dtype == 1 && dk == kBD && dv == kBD) {
    if ((long long)N * H * kBD * 2 > 0xffffffffLL) return static_cast<int>(hipErrorInvalidValue);
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
