// Tree verification on matrix cores: bf16 q/k/v, d_k = d_v = 128, fp32 state.
//
// What is computed (per sequence b, head h) is the tree-structured WY form of
// the gated delta rule that the TreeWY abstract describes (every draft node's
// output from one triangular solve, a small pseudo-value matrix U in place of
// per-node states), and in scalar-decay mode the page-4 closed form of the Bole
// auto-summary.  With anc*(n) the root-to-n path (n included),
// D(j->n) = prod of alpha over the path nodes after j, gamma_n = prod over all
// of anc*(n):
//
//   (I + A) U = R,  R_n = beta_n (v_n - gamma_n S_root^T k_n),
//                   A[n, j] = beta_n D(j->n) (k_n.k_j) for j in anc(n)
//   o_n = gamma_n S_root^T q_n + sum_{j in anc*(n)} D(j->n) (q_n.k_j) u_j
//
// The path block of (I + A) for node n is unit lower-triangular and holds
// every ancestor pair of the path, so u_n = x.R_path and
// o_n = gamma_n QS_n + w.R_path with x, w from one backward substitution of
// length len(n) (x for e_last, w for the read-out row).
//
// One workgroup per (b, h, block of VB value columns); one wave per (node
// tile, value-column tile) pair, NT * CT of them (four, or eight for the
// 128-node shape):
//   1. loads, small ones first: parents and gates, K and Q rows (staged in
//      LDS), the wave's 32 columns of S_root straight into MFMA operand
//      registers, and V at the positions the outputs land on;
//   2. tree index in registers, one copy per wave: pointer jumping over the
//      parent array with cross-lane shuffles gives each node's ancestor bitset
//      and, in the same pass, gamma (product of alpha over the path);
//   3. Gram on matrix cores (32x32x16 bf16, exact products), transposed so a
//      lane owns a node: lower-triangular blocks of K K^T and K Q^T; a lane
//      keeps the entries whose row is on its node's path, stored by distance
//      from the node (the ancestor-masked Gram/decay builder);
//   4. one lane per node (wave 0, and wave 1 when N > 64) solves the node's
//      path (x for U, w for o; decays as running products of alpha, no
//      log/exp) into LDS, while the S stream is still arriving;
//   5. Y^T = S_block^T [K;Q]^T on matrix cores with S split into bf16 hi + lo
//      (q and k are exact in bf16: ~2^-17 relative error); the accumulator
//      layout puts one node and 16 value columns in each lane;
//   6. R = beta (V - gamma KS) from the K accumulators into LDS;
//   7. U and o gathered over the node's path rows of R (float4 loads),
//      o starting from gamma_n QS_n in the Q accumulators; stored to HBM.
// Trees with a path longer than 16 take the level-scheduled solve instead
// (same kernel, same outputs).
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;       // d_k = d_v
constexpr int kMaxL = 16;     // longest root-to-node path solved in registers
// Staged K/Q rows are 256 B (16 chunks of 16 B) with chunk c of row r stored at
// slot c ^ (r & 15): the lanes of one matrix-core operand read (consecutive
// rows, one chunk) then hit 16 different 16-byte bank groups.
__device__ __forceinline__ int kq_slot(int row, int ch) { return ch ^ (row & 15); }

// Two floats to packed bf16 (round to nearest even), first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  uint32_t r;
  __builtin_memcpy(&r, &v, 4);
  return r;
}

// s_waitcnt immediate: vector-memory count 0 (expcnt, lgkmcnt left alone).
constexpr int kVmcntZero = (7 << 4) | (15 << 8);

template <int NP, int VB, bool PS>
struct MfmaLayout {
  static constexpr int RS = VB + 4;                 // fp32 row stride of R in LDS
  static constexpr int stage = 2 * NP * kD * 2;     // K, Q bf16 until the Y contraction
  static constexpr int rbytes = NP * RS * 4;        // R rows
  // R goes over the dead staging, except with one workgroup per state (PS),
  // which keeps K and Q staged for every column block and gives R its own rows
  static constexpr int roff = PS ? stage : 0;
  static constexpr int u0 = PS ? stage + rbytes : (stage > rbytes ? stage : rbytes);
  static constexpr int fb = (int)(sizeof(LevelLds) + sizeof(TreeLds));  // level-scheduled fallback
  static constexpr int bytes = u0 > fb ? u0 : fb;
};

// Accumulator element r of a 32x32 tile sits at row 8*(r/4) + 4*(lane/32) + r%4,
// column lane%32.  In Y^T and G^T the columns are nodes.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ __forceinline__ float4 bf16x4_to_f32(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

__device__ __forceinline__ uint2 f32x4_to_bf16(float a, float b, float c, float d) {
  uint2 r;
  r.x = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
  r.y = static_cast<uint32_t>(f32_to_bf16(c)) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
  return r;
}

// ---- tree index in registers (lane l holds node l, and node l + 64 when SL = 2) ----

template <int SL>
struct WaveTree {
  unsigned long long a0[SL], a1[SL];  // inclusive ancestor bitsets, nodes 0..63 and 64..127
  float g[SL];                        // gamma: product of alpha over the root path
};

// Value of a per-node register for node j (owned by lane j % 64, slot j / 64).
template <int SL, typename T>
__device__ __forceinline__ T node_val(const T (&x)[SL], int j) {
  const int src = j & 63;
  T v = __shfl(x[0], src);
  if constexpr (SL == 2) {
    const T v1 = __shfl(x[1], src);
    v = j >= 64 ? v1 : v;
  }
  return v;
}

// Pointer jumping: at each jump step a node adopts the span of the node its
// jump pointer names (ancestor set, product of alpha) and jumps past it, so
// spans double until every jump pointer runs off the root.  Spans stay
// contiguous path segments whether or not the named node already moved in the
// same step.
// Returns the tree's longest path length (same in every wave) and flags
// parents outside [-1, i-1] (treated as -1).
template <int SL>
__device__ void wave_tree(WaveTree<SL>& T, const int (&par)[SL], const float (&al)[SL], int N,
                          bool& bad, int& Lmax) {
  const int lane = threadIdx.x & 63;
  int jp[SL];
  bool badl = false;
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const int node = lane + 64 * s;
    int p = par[s];
    if (node < N && (p < -1 || p >= node)) {
      badl = true;
      p = -1;
    }
    jp[s] = node < N ? p : -1;
    T.a0[s] = node < 64 ? (1ull << node) : 0ull;
    T.a1[s] = node < 64 ? 0ull : (1ull << (node - 64));
    T.g[s] = node < N ? al[s] : 1.f;
  }
  while (true) {
    bool act = false;
#pragma unroll
    for (int s = 0; s < SL; ++s) act |= jp[s] >= 0;
    if (!__any(act)) break;
    unsigned long long x0[SL], x1[SL];
    float xg[SL];
    int xj[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int j = jp[s] >= 0 ? jp[s] : 0;
      x0[s] = node_val<SL>(T.a0, j);
      x1[s] = node_val<SL>(T.a1, j);
      xg[s] = node_val<SL>(T.g, j);
      xj[s] = node_val<SL>(jp, j);
    }
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      if (jp[s] >= 0) {
        T.a0[s] |= x0[s];
        T.a1[s] |= x1[s];
        T.g[s] *= xg[s];
        jp[s] = xj[s];
      }
    }
  }
  int L = 0;
#pragma unroll
  for (int s = 0; s < SL; ++s)
    if (lane + 64 * s < N) L = max(L, __popcll(T.a0[s]) + __popcll(T.a1[s]));
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) L = max(L, __shfl_xor(L, m));
  Lmax = L;
  bad = __any(badl);
}

// Position of node j on the root path whose set is (a0, a1) = number of path
// nodes with a smaller index = depth of j when j is on that path.
__device__ __forceinline__ int rank_below(unsigned long long a0, unsigned long long a1, int j) {
  if (j < 64) return __popcll(a0 & ((1ull << j) - 1ull));
  return __popcll(a0) + __popcll(a1 & ((1ull << (j - 64)) - 1ull));
}

// ---- helpers of the fused commit (the previous step's accepted path) ----

// Register value of node n (uniform) when lane l holds nodes l and l + 64.
__device__ __forceinline__ int node_lane_i(const int (&x)[2], int n) {
  return n < 64 ? __builtin_amdgcn_readlane(x[0], n) : __builtin_amdgcn_readlane(x[1], n - 64);
}
__device__ __forceinline__ float node_lane_f(const float (&x)[2], int n) {
  const int v = n < 64 ? __builtin_amdgcn_readlane(__float_as_int(x[0]), n)
                       : __builtin_amdgcn_readlane(__float_as_int(x[1]), n - 64);
  return __int_as_float(v);
}
__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Eight floats as three bf16 words each (x = hi + mid + lo to ~2^-26 relative).
__device__ __forceinline__ void split3_bf16(const float (&x)[8], bf16x8& h8, bf16x8& m8, bf16x8& l8) {
  uint32_t wh[4], wm[4], wl[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float x0 = x[2 * p], x1 = x[2 * p + 1];
    const uint32_t hw = pack_bf16x2(x0, x1);
    const float r0 = x0 - __uint_as_float(__builtin_amdgcn_perm(0u, hw, 0x01000c0cu));
    const float r1 = x1 - __uint_as_float(hw & 0xffff0000u);
    const uint32_t mw = pack_bf16x2(r0, r1);
    const float s0 = r0 - __uint_as_float(__builtin_amdgcn_perm(0u, mw, 0x01000c0cu));
    const float s1 = r1 - __uint_as_float(mw & 0xffff0000u);
    wh[p] = hw;
    wm[p] = mw;
    wl[p] = pack_bf16x2(s0, s1);
  }
  __builtin_memcpy(&h8, wh, 16);
  __builtin_memcpy(&m8, wm, 16);
  __builtin_memcpy(&l8, wl, 16);
}

// Waves of a workgroup: one per (node tile, value-column tile) pair.
template <int NP, int VB>
constexpr int mfma_waves() { return (NP / 32) * (VB / 32); }

template <int NP, int VB, bool FUSED, bool PS>
__global__ __launch_bounds__((64 * mfma_waves<NP, VB>()), NP > 64 ? 1 : (PS ? 2 : 3)) void verify_mfma_kernel(
    int H, int N, int mode, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const int32_t* __restrict__ parents,
    const float* S_root, uint16_t* __restrict__ o, float* __restrict__ U,
    int32_t* __restrict__ status, PrevCommit pc) {
  using Lay = MfmaLayout<NP, VB, PS>;
  constexpr int NT = NP / 32;                 // node tiles
  constexpr int CT = VB / 32;                 // value-column tiles in the block
  constexpr int NW = NT * CT;                 // waves
  constexpr int NTH = 64 * NW;                // threads
  static_assert(NW == 4 || NW == 8, "one (node tile, column tile) pair per wave");
  constexpr int NVB = kD / VB;
  constexpr int SL = NP > 64 ? 2 : 1;         // tree nodes per lane
  constexpr int NG = NT * (NT + 1);           // lower-triangular blocks of K K^T and K Q^T
  constexpr int GPW = (NG + NW - 1) / NW;
  constexpr int RS = Lay::RS;

  __shared__ __align__(16) unsigned char smem[Lay::bytes];
  // Per-node tables are stored [index][node] so lanes that touch different
  // nodes at one index hit consecutive banks.
  // Path Gram entries by distance: CkkD[d][m] = k_m . k_j, CqkD[d][m] = q_m . k_j
  // for the ancestor j of node m that sits d steps above m (d = 0: m itself).
  __shared__ __align__(16) float CkkD[kMaxL * NP];
  __shared__ __align__(16) float CqkD[kMaxL * NP];
  __shared__ float gsink[64];                          // Gram entries off every path land here
  __shared__ __align__(16) unsigned long long anc_s[NP][2];
  __shared__ __align__(16) int sdep[NP];               // depth (path length - 1)
  __shared__ __align__(16) float2 XW[kMaxL * NP];      // path coefficients [distance][node]: (x, w)
  __shared__ float sal[NP], sbe[NP], sga[NP];
  __shared__ int meta[2 + NT];                         // longest path, bad-parents flag, longest per node tile
  // each node's root path, one byte per node, in distance order (n, parent,
  // ...), padded with the node itself
  __shared__ __align__(16) uint4 sEd[NP];
  // fused commit: the previous tree's accepted path (first 16 nodes)
  struct PrevPathLds {
    float pd[16];   // D(e_t -> a), 0 past the end
    int e[16];      // e_t: node at distance t (node 0 past the end)
    float gam;      // gamma_a
    float cn;       // D at distance 16
    int next;       // node at distance 16, or -1
  };
  __shared__ __align__(16) PrevPathLds spath;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lm = lane & 31;
  const int hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: wave-uniform branches
  // One workgroup per (state, column block), or per state (PS), looping over
  // its NVB column blocks after the tree, the Gram and the path solve, which
  // then run once per state instead of once per block.
  const int bid = PS ? (int)blockIdx.x : xcd_group(blockIdx.x, gridDim.x, NVB);
  const int vb = PS ? 0 : bid % NVB;  // the (first) column block
  const int bh = PS ? bid : bid / NVB;
  const int h = bh % H;
  const int b = bh / H;
  int cbase = vb * VB;                // the current column block's first column
  const bool gdn = mode == kGdn;
  // With two node tiles (KS = 2) the two waves of a column tile split the d_k
  // contraction instead of each streaming the whole S block: wave (kh, ct)
  // loads rows 64 kh .. 64 kh + 63 and forms partial products for both node
  // tiles; the halves meet in LDS after the contraction (step 5).  It then
  // owns node tile kh for steps 4, 6 and 7.
  constexpr int KS = (NT == 2 && !PS) ? 2 : 1;  // d_k split of the S contraction
  static_assert(KS == 1 || Lay::bytes >= 4 * 8 * 64 * 16, "room for four waves' partial products");
  const int nt_w = KS == 2 ? (wave & 1) : wave / CT;    // this wave's node tile
  const int ct_w = KS == 2 ? (wave >> 1) : wave % CT;   // this wave's column tile
  const int akof = 8 * hi;
  const int col0 = ct_w * 32 + 4 * hi;         // + 8 g + j: this lane's columns in the block
  const int my_n0 = nt_w * 32 + lm;            // node this lane outputs (and solves for)
  const int my_n = min(my_n0, N - 1);

  // ---- 1-2. wave 0: gates, parents and the tree index; waves 1-3: K and Q ----
  // Row indices are clamped, not branched on: padded rows repeat row N-1 and
  // only feed outputs that are discarded.  K and Q go from HBM straight into
  // LDS (no registers): each wave instruction fills 4 rows (1 KB) and lane i
  // writes the 16 bytes at i * 16, so it fetches the chunk the swizzle puts
  // there.  Wave 0 issues none of these, so nothing delays its tree build.
  uint16_t* Ksh = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Qsh = Ksh + NP * kD;
  // Fused commit: the previous tree's parents and gates (nodes lane and
  // lane + 64).  Wave 1 (which stages no K/Q rows then) loads them, walks the
  // accepted path and stages its k rows and u columns while wave 0 builds the
  // tree.
  int ppar[2] = {-1, -1};
  float pal[2] = {1.f, 1.f};
  int pacc = 0;  // the previous accepted node
  auto load_prev_tree = [&]() {
    pacc = pc.accepted[b];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int nd = min(lane + 64 * s, pc.N - 1);
      ppar[s] = pc.parents[(size_t)b * pc.N + nd];
      pal[s] = pc.alpha[(size_t)(b * pc.N + nd) * H + h];
    }
  };
  // First node of the previous tree's accepted path (-1: none), uniform; the
  // parents must be loaded.  Invalid parents: no update (status 1); a bad
  // accepted index commits node 0's path (status 2), as tree_commit does.
  auto prev_start = [&](bool& pbad, bool& bad_acc, int& pa) {
    bool badl = false;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int nd = lane + 64 * s;
      badl |= nd < pc.N && (ppar[s] < -1 || ppar[s] >= nd);
    }
    pbad = __any(badl) != 0;
    pa = pacc;
    bad_acc = pa < 0 || pa >= pc.N;
    return pbad ? -1 : (bad_acc ? 0 : pa);
  };
  // Walks 16 steps up the previous tree from `node` (uniform), D running in c,
  // with scalar selects only; lane t < 16 keeps the node at distance t and its
  // D(node -> a) (node 0 and 0 past the end).
  auto walk16 = [&](int& node, float& c, int& my_e, float& my_d) {
    my_e = 0;
    my_d = 0.f;
    auto steps = [&](auto two) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const bool live = node >= 0;  // uniform
        const int nc = live ? node : 0;
        if (lane == t) {
          my_e = nc;
          my_d = live ? c : 0.f;
        }
        const int lo = nc & 63;
        int p = __builtin_amdgcn_readlane(ppar[0], lo);
        float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pal[0]), lo));
        if constexpr (decltype(two)::value) {
          const int p1 = __builtin_amdgcn_readlane(ppar[1], lo);
          const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pal[1]), lo));
          p = nc < 64 ? p : p1;
          a = nc < 64 ? a : a1;
        }
        const float cn = uniform_f(c * a);
        c = live ? cn : c;
        node = live ? p : -1;
      }
    };
    if (pc.N > 64)  // uniform
      steps(std::integral_constant<bool, true>{});
    else
      steps(std::integral_constant<bool, false>{});
  };
  if constexpr (FUSED) {
    if (wave == 1) load_prev_tree();
  }
  if (wave == 0) {
    int par[SL];
    float al[SL], be[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int nd = min(lane + 64 * s, N - 1);
      par[s] = parents[(size_t)b * N + nd];
      al[s] = alpha[(size_t)(b * N + nd) * H + h];
      be[s] = (gdn ? beta : alpha)[(size_t)(b * N + nd) * H + h];
    }
    WaveTree<SL> T;
    bool bad;
    int Lmax;
    wave_tree<SL>(T, par, al, N, bad, Lmax);
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int nd = lane + 64 * s;
      const int Ln = __popcll(T.a0[s]) + __popcll(T.a1[s]);
      if (nd < NP) {
        anc_s[nd][0] = T.a0[s];
        anc_s[nd][1] = T.a1[s];
        sdep[nd] = Ln - 1;
        sga[nd] = T.g[s];
        sal[nd] = al[s];
        sbe[nd] = gdn ? be[s] : 0.f;
        // Path list in distance order (n, parent, ...), padded with n, computed
        // here while K and Q are still in flight: ancestors have smaller
        // indices, so it is the ancestor set's bits from the top.  Steps past
        // the tree's longest path (uniform) only pad.
        uint32_t wd[kMaxL / 4] = {0u, 0u, 0u, 0u};
        unsigned long long h0 = T.a0[s], h1 = T.a1[s];
#pragma unroll
        for (int d = 0; d < kMaxL; ++d) {
          int jd = nd;
          if (d < Lmax) {  // uniform
            if constexpr (NP <= 64) {
              if (h0) {
                jd = 63 - __clzll(h0);
                h0 ^= 1ull << jd;
              }
            } else {
              if (h1) {
                jd = 127 - __clzll(h1);
                h1 ^= 1ull << (jd - 64);
              } else if (h0) {
                jd = 63 - __clzll(h0);
                h0 ^= 1ull << jd;
              }
            }
          }
          wd[d >> 2] |= static_cast<uint32_t>(jd) << (8 * (d & 3));
        }
        sEd[nd] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
      // longest path per node tile of 32 (the lane halves of this slot)
      int lt = nd < N ? Ln : 1;
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) lt = max(lt, __shfl_xor(lt, m));
      if ((lane & 31) == 0 && 2 * s + (lane >> 5) < NT) meta[2 + 2 * s + (lane >> 5)] = lt;
    }
    if (lane == 0) {
      meta[0] = Lmax;
      meta[1] = bad;
    }
  } else if (FUSED && wave == 1) {
    // the previous tree's accepted path (first 16 nodes) into LDS
    bool pbad, bad_acc;
    int pa;
    int node = prev_start(pbad, bad_acc, pa);
    float c = 1.f;
    int my_e;
    float my_d;
    walk16(node, c, my_e, my_d);
    const int next = node;
    const float cn = c;
    for (int n2 = node; n2 >= 0; n2 = node_lane_i(ppar, n2)) c = uniform_f(c * node_lane_f(pal, n2));
    if (lane < 16) {
      spath.pd[lane] = my_d;
      spath.e[lane] = my_e;
    }
    if (lane == 0) {
      spath.gam = c;
      spath.cn = cn;
      spath.next = next;
    }
    // The path's k rows and u columns are fetched by every wave after the
    // barrier (they are first needed by the update after the Gram), so this
    // wave's walk is not followed by a second round trip before the barrier.
    // status and root-first path of the previous step (one wave per sequence)
    if (h == 0 && vb == 0) {
      if (pc.status && lane == 0) pc.status[b] = pbad ? 1 : (bad_acc ? 2 : 0);
      if (pc.path_out) {
        int nd2 = (pbad || bad_acc) ? -1 : pa;
        int m0 = -1, m1 = -1, len = 0;  // distance of node lane (lane + 64) from a
        while (nd2 >= 0) {
          if (lane == nd2) m0 = len;
          if (lane + 64 == nd2) m1 = len;
          nd2 = node_lane_i(ppar, nd2);
          ++len;
        }
        int32_t* po = pc.path_out + (size_t)b * pc.N;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int nd = lane + 64 * s;
          const int m = s ? m1 : m0;
          if (nd < pc.N) {
            if (m >= 0) po[len - 1 - m] = nd;
            if (nd >= len) po[nd] = -1;
          }
        }
      }
    }
  } else {
    const int slot = lane & 15;
    // 4-row blocks: K, then Q (waves 2 and 3 only when wave 1 stages the commit)
    for (int blk = wave - (FUSED ? 2 : 1); blk < NP / 2; blk += NW - (FUSED ? 2 : 1)) {
      const bool isq = blk >= NP / 4;
      const int rb = isq ? blk - NP / 4 : blk;
      const int row = rb * 4 + (lane >> 4);
      const int src_row = min(row, N - 1);
      const uint16_t* src = (isq ? q : k) + ((size_t)(b * N + src_row) * H + h) * kD +
                            kq_slot(row, slot) * 8;
      __builtin_amdgcn_global_load_lds(src, (isq ? Qsh : Ksh) + rb * 4 * kD, 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(kVmcntZero);  // this wave's K/Q rows have landed
  }
  __syncthreads();  // tree, gates and K/Q staging visible

  const int Lmax = __builtin_amdgcn_readfirstlane(meta[0]);  // uniform: scalar loop bounds
  if (h == 0 && vb == 0 && tid == 0 && status) status[b] = meta[1] ? 1 : 0;

  // This wave's S block: rows srow0 + 16 ks + 8 hi + i (KSTEPS steps of 16
  // rows), column cbase + 32 ct_w + lm, straight into MFMA operand registers.
  constexpr int KSTEPS = 8 / KS;                // 16-row k steps of this wave
  constexpr int TL = KSTEPS / 2;                // 32-row tiles of those rows
  const int srow0 = KS == 2 ? nt_w * 64 : 0;
  // block base (uniform) + 32-bit lane offset in bytes: scalar-base addressing
  auto sblk_of = [&](int c) { return (size_t)bh * kD * kD + c + ct_w * 32 + (size_t)srow0 * kD; };
  const uint32_t slane = 4u * (lm + akof * kD);
  float sv[KSTEPS][8];
  auto load_S_ks = [&](int c, int ks) {
    const char* Sb = reinterpret_cast<const char*>(S_root + sblk_of(c));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sv[ks][i] = *reinterpret_cast<const float*>(Sb + slane + 4u * (ks * 16 + i) * kD);
  };
  auto load_S = [&](int c) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) load_S_ks(c, ks);
  };

  // ---- fused commit of the previous step (TreeWY abstract: only the accepted
  // state is rebuilt; Bole auto-summary, reconstruction formula) ----
  //   S = gamma_a S_in + sum_t D(e_t -> a) k_{e_t} u_{e_t}^T
  // over the previous tree's accepted path e_0 = a, e_1 = parent(a), ...  The
  // rank-16 update of a wave's S block is one matrix-core product per 32-row
  // tile (k exact in bf16, D u split into three bf16 words, accumulated onto
  // gamma_a S in the operand registers); the block is then stored as the
  // committed state and used as S below.  Path nodes j = 8 hi + i of a chunk
  // of 16 belong to lane half hi.
  // Tile (T, tau) of the update covers the wave's state rows 64 T + 2 m + tau
  // (m = matrix-core row): its accumulator element 4 s + i of lane (column c,
  // half hi) is then row 64 T + 16 s + 8 hi + 2 i + tau, i.e. sv[4 T + s][2 i + tau],
  // and one 32-bit load of k at rows (2 m, 2 m + 1) feeds both tau.
  uint32_t kpd[TL / 2][8];  // k_{e_j} at rows 64 T + 2 lm (+1), j = 8 hi + i
  float upa[8];             // u_{e_j} at this lane's column
  // The operands come straight from memory (the path's nodes are in LDS after
  // the first barrier).  They are issued before the S stream and consumed after
  // the path solve; the 32-node shape, whose registers are at their limit
  // there, issues them at the update instead.
  constexpr bool kEarlyOps = !(KS == 1 && NT == 1);
  // k of the path nodes (the same for every column block) and u at column
  // block c (with_k false: u only)
  auto load_prev_ops = [&](int c, bool with_k) {
    const int4 e0 = reinterpret_cast<const int4*>(spath.e)[2 * hi];
    const int4 e1 = reinterpret_cast<const int4*>(spath.e)[2 * hi + 1];
    const int ej[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
    const int col = c + ct_w * 32 + lm;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      upa[i] = pc.U[((size_t)bh * pc.N + ej[i]) * kD + col];
      if (with_k) {
#pragma unroll
        for (int T = 0; T < TL / 2; ++T)
          kpd[T][i] = *reinterpret_cast<const uint32_t*>(
              pc.k + ((size_t)(b * pc.N + ej[i]) * H + h) * kD + srow0 + 64 * T + 2 * lm);
      }
    }
  };
  auto prev_apply = [&](const float (&dj)[8]) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = dj[i] * upa[i];
    bf16x8 uh, um, ul;
    split3_bf16(x, uh, um, ul);
#pragma unroll
    for (int T = 0; T < TL / 2; ++T) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        uint32_t aw[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
          aw[p] = __builtin_amdgcn_perm(kpd[T][2 * p + 1], kpd[T][2 * p], tau ? 0x07060302u : 0x05040100u);
        bf16x8 a;
        __builtin_memcpy(&a, aw, 16);
        f32x16 acc;
#pragma unroll
        for (int ss = 0; ss < 4; ++ss)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[4 * ss + i] = sv[4 * T + ss][2 * i + tau];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, uh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, um, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ul, acc, 0, 0, 0);
#pragma unroll
        for (int ss = 0; ss < 4; ++ss)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[4 * T + ss][2 * i + tau] = acc[4 * ss + i];
      }
    }
  };
  auto commit_prev = [&]() {
    const float gam = spath.gam;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[ks][i] *= gam;
    {
      // first 16 path nodes
      if constexpr (!kEarlyOps) load_prev_ops(cbase, true);
      const float4 d0 = reinterpret_cast<const float4*>(spath.pd)[2 * hi];
      const float4 d1 = reinterpret_cast<const float4*>(spath.pd)[2 * hi + 1];
      const float dj[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      prev_apply(dj);
    }
    int node = __builtin_amdgcn_readfirstlane(spath.next);
    if (node >= 0) {  // uniform: a path longer than 16, one more node per round
      float c = spath.cn;
      load_prev_tree();
      const int col = cbase + ct_w * 32 + lm;
      while (node >= 0) {
        const float u = c * pc.U[((size_t)bh * pc.N + node) * kD + col];
        const uint4* kr = reinterpret_cast<const uint4*>(
            pc.k + ((size_t)(b * pc.N + node) * H + h) * kD + srow0 + akof);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const uint4 w = kr[2 * ks];  // k at rows 16 ks + 8 hi + 0..7
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sv[ks][2 * e] = fmaf(__uint_as_float(ws[e] << 16), u, sv[ks][2 * e]);
            sv[ks][2 * e + 1] = fmaf(__uint_as_float(ws[e] & 0xffff0000u), u, sv[ks][2 * e + 1]);
          }
        }
        c = uniform_f(c * node_lane_f(pal, node));
        node = node_lane_i(ppar, node);
      }
    }
  };
  // The committed block goes out during the contraction, one 16-row step at a
  // time just before that step is split (its registers are live until then
  // anyway).  With more than one node tile and no d_k split (the 128-node
  // shape) the waves of a column tile hold the same block and the one of node
  // tile 0 stores it; all waves have their S values by then (they passed the
  // barrier after the update), so S_out may be S_in.
  auto store_committed = [&](int ks) {
    if (KS == 1 && NT > 1 && nt_w != 0) return;  // uniform
    char* So = reinterpret_cast<char*>(pc.S_out + sblk_of(cbase));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<float*>(So + slane + 4u * (ks * 16 + i) * kD) = sv[ks][i];
  };

  constexpr int FBW = PS ? kD : VB;  // columns this workgroup covers
  if (Lmax > kMaxL) {
    if constexpr (FUSED) {
      // the previous step's commit of this block, plainly (rare path): the
      // whole accepted path into the Gram tables (unused here), then
      // S_out = gamma_a S_in + sum_t D_t k_t u_t^T element by element
      int* fpath = reinterpret_cast<int*>(CkkD);
      float* fd = CqkD;
      load_prev_tree();
      if (wave == 0) {
        bool pbad, bad_acc;
        int pa;
        int node = prev_start(pbad, bad_acc, pa);
        float c = 1.f;
        int t = 0;
        while (node >= 0) {  // uniform
          if (lane == 0) {
            fpath[t] = node;
            fd[t] = c;
          }
          c = uniform_f(c * node_lane_f(pal, node));
          node = node_lane_i(ppar, node);
          ++t;
        }
        if (lane == 0) {
          gsink[0] = __int_as_float(t);
          gsink[1] = c;
        }
      }
      __syncthreads();
      const int Lp = __float_as_int(gsink[0]);
      const float gam = gsink[1];
      const float* Si = S_root + (size_t)bh * kD * kD;
      float* So = pc.S_out + (size_t)bh * kD * kD;
      for (int e = tid; e < kD * (FBW / 4); e += NTH) {
        const int r = e / (FBW / 4);
        const int c = cbase + 4 * (e % (FBW / 4));
        float4 acc = mul4(gam, *reinterpret_cast<const float4*>(Si + r * kD + c));
        for (int t = 0; t < Lp; ++t) {
          const int nd = fpath[t];
          const float kr = __uint_as_float(
              static_cast<uint32_t>(pc.k[((size_t)(b * pc.N + nd) * H + h) * kD + r]) << 16);
          const float4 u = *reinterpret_cast<const float4*>(pc.U + ((size_t)bh * pc.N + nd) * kD + c);
          acc = fma4(fd[t] * kr, u, acc);
        }
        *reinterpret_cast<float4*>(So + r * kD + c) = acc;
      }
      __threadfence();  // the committed block is read back below
    }
    __syncthreads();  // the staging area becomes the fallback's tables
    TreeLds& tfb = *reinterpret_cast<TreeLds*>(smem + sizeof(LevelLds));
    build_tree(tfb, parents + (size_t)b * N, N);
    level_solve<uint16_t>(tfb, *reinterpret_cast<LevelLds*>(smem), mode, b, h, H, N, kD, kD, cbase,
                          cbase + FBW, q, k, v, alpha, beta, FUSED ? pc.S_out : S_root, o, U);
    return;
  }

  // Fused commit: this lane's operands of the update, straight from memory in
  // the matrix-core layout (k of path node 8 hi + i at rows 64 T + 2 lm and
  // + 1 of the wave's S rows, u of that node at the lane's column), issued
  // before the S stream; they are consumed after the path solve.
  if constexpr (FUSED && kEarlyOps) load_prev_ops(cbase, true);
  // S and V (at the positions the outputs land on) arrive during the Gram and
  // the path solve
  load_S(cbase);
  uint2 vv[4];
  auto load_V = [&](int c) {
    const uint16_t* vr = v + ((size_t)(b * N + my_n) * H + h) * kD + c + col0;
#pragma unroll
    for (int g = 0; g < 4; ++g) vv[g] = *reinterpret_cast<const uint2*>(vr + 8 * g);
  };
  load_V(cbase);

  // ---- 3. ancestor-masked Gram, transposed (lane = node) ----
  {
    // tile index -> (node tile nt2 in [0, 2NT): K then Q rows; ancestor tile jt <= nt2 % NT)
    int tnt[GPW], tjt[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      int rem = wave + NW * i, nt2 = -1, jt = 0;
      for (int r = 0; r < 2 * NT; ++r) {
        const int cnt = (r % NT) + 1;
        if (rem >= 0 && rem < cnt) {
          nt2 = r;
          jt = rem;
        }
        rem -= cnt;
      }
      tnt[i] = nt2;
      tjt[i] = jt;
    }
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int nt2 = tnt[i];
      if (nt2 < 0) continue;  // uniform
      const int jt = tjt[i];
      const bool kk = nt2 < NT;
      const uint16_t* Xn = (kk ? Ksh : Qsh) + ((nt2 % NT) * 32 + lm) * kD;
      const uint16_t* Kj = Ksh + (jt * 32 + lm) * kD;
      f32x16 gacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) gacc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int so = kq_slot(lm, 2 * ks + hi) * 8;  // rows of a tile start at a multiple of 16
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kj + so);
        const bf16x8 bx = *reinterpret_cast<const bf16x8*>(Xn + so);
        gacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bx, gacc, 0, 0, 0);
      }
      // Keep G[j][n] when j is on n's path, at [depth(n) - depth(j)][n]; everything
      // else goes to a sink slot, so the stores need no branches.  This lane's
      // rows are j = 32 jt + 8 g + 4 hi + i (g, i < 4): one 32-bit word of n's
      // ancestor set and four 16-byte reads of the depth table cover them.
      // (The K K^T entry j = n lands at distance 0, a slot nothing reads.)
      const int n = (nt2 % NT) * 32 + lm;  // padded lanes store to padded columns
      const int nc = min(n, N - 1);
      const unsigned long long aw = anc_s[nc][jt >> 1];
      const uint32_t word = static_cast<uint32_t>(aw >> (32 * (jt & 1))) >> (4 * hi);
      const int dn = sdep[nc];
      float* C = (kk ? CkkD : CqkD) + dn * NP + n;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int4 dj = *reinterpret_cast<const int4*>(sdep + jt * 32 + 8 * g + 4 * hi);
        const int djs[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool on = (word >> (8 * g + i)) & 1u;
          *(on ? C - djs[i] * NP : gsink + lane) = gacc[4 * g + i];
        }
      }
    }
  }
  __syncthreads();  // path Gram entries visible

  // ---- 4. path solve: lane = (node my_n, chain hi) in every wave ----
  // Distance order e_0 = n, e_1 = parent(n), ...  Chain 0 gives x (u_n = sum_t
  // x_t R_{e_t}), chain 1 gives w (o_n = gamma_n QS_n + sum_t w_t R_{e_t}); the
  // two half-waves run the same code.  The trip count is the wave's longest
  // path (uniform); lanes past their own path length compute on clamped,
  // valid addresses and keep zero coefficients.  Scalar decay needs no special
  // case: its write strengths are zero, so y = 0 and only the q.k term stays.
  uint4 ep;  // path nodes, one byte each, distance order, for the gather
  int Lw, L;
  {
    int e[kMaxL];
    L = sdep[my_n] + 1;
    {
      const uint4 ed = sEd[my_n];
      const uint32_t w4[4] = {ed.x, ed.y, ed.z, ed.w};
#pragma unroll
      for (int d = 0; d < kMaxL; ++d) e[d] = (w4[d >> 2] >> (8 * (d & 3))) & 0xff;
    }
    Lw = __builtin_amdgcn_readfirstlane(meta[2 + nt_w]);  // this wave's longest path
    // The decay between path nodes factors through the running product
    // Q_t = D(e_t -> n) = alpha(e_0) ... alpha(e_{t-1}):  D(e_t -> e_s) = Q_t / Q_s.
    // So with c_t = Q_t h_t the substitution runs on decay-free h:
    //   h_t = w_sel (q_n . k_{e_t}) - sum_{s<t} beta(e_s) h_s G(e_s, e_t)
    // (h_0 = 1 for x), one FMA per pair and no rescaling; Q_t only scales the
    // coefficient written out.
    const float wsel = hi ? 1.f : 0.f;
    // this lane's chain coefficient at distance t goes to XW[t][n].x (x) or .y (w)
    float* xwo = reinterpret_cast<float*>(XW + my_n) + hi;
    const bool owner = my_n0 < N;
    float y[kMaxL];  // beta(e_s) h_s
    const float c0 = hi ? CqkD[my_n] : 1.f;
    if (owner) xwo[0] = c0;
    y[0] = c0 * sbe[my_n];
    float qt = sal[my_n];  // Q_t at step t
    // steps in chunks under one uniform branch, so that a chunk's LDS loads
    // (static offsets from per-node bases) can all be in flight together; the
    // chunk is shorter when the whole S block is held in registers (KS = 1)
    constexpr int CHK = KS == 2 ? 4 : 2;
#pragma unroll
    for (int t0 = 1; t0 < kMaxL; t0 += CHK) {
      if (t0 < Lw) {  // uniform
#pragma unroll
        for (int tt = t0; tt < t0 + CHK && tt < kMaxL; ++tt) {
          const bool live = tt < L;
          const float cq = CqkD[tt * NP + my_n];
          const float at = sal[e[tt]];
          const float bt = sbe[e[tt]];
          float acc = wsel * cq;
#pragma unroll
          for (int ss = 0; ss < tt; ++ss) acc = fmaf(-y[ss], CkkD[(tt - ss) * NP + e[ss]], acc);
          const float hv = live ? acc : 0.f;
          y[tt] = hv * bt;
          if (owner) xwo[2 * tt * NP] = qt * hv;
          qt *= at;
        }
      }
    }
    ep = make_uint4(e[0] | (e[1] << 8) | (e[2] << 16) | (e[3] << 24),
                    e[4] | (e[5] << 8) | (e[6] << 16) | (e[7] << 24),
                    e[8] | (e[9] << 8) | (e[10] << 16) | (e[11] << 24),
                    e[12] | (e[13] << 8) | (e[14] << 16) | (e[15] << 24));
  }

  // ---- per column block (one pass, or NVB with one workgroup per state) ----
#pragma unroll
  for (int vbi = 0; vbi < (PS ? NVB : 1); ++vbi) {
  if constexpr (PS) cbase = vbi * VB;
  if constexpr (FUSED) {
    commit_prev();
    // where several waves hold the same block, every wave's S values are in
    // before one of them stores over S_in
    if constexpr (KS == 1 && NT > 1) __syncthreads();
  }

  // ---- 5. Y^T = S_block^T [K;Q]^T on matrix cores ----
  // S is split into bf16 hi and lo words, two k values per word (one packed
  // conversion each); q and k are exact in bf16.
  auto split = [&](int ks, bf16x8& shi, bf16x8& slo) {
    uint32_t whi[4], wlo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = sv[ks][2 * i], x1 = sv[ks][2 * i + 1];
      const uint32_t hw = pack_bf16x2(x0, x1);
      whi[i] = hw;
      // hi value of x0 back as a float: its 16 bits moved up by a byte permute
      // (a shift here gets rewritten as a second conversion of x0)
      const float h0 = __uint_as_float(__builtin_amdgcn_perm(0u, hw, 0x01000c0cu));
      wlo[i] = pack_bf16x2(x0 - h0, x1 - __uint_as_float(hw & 0xffff0000u));
    }
    __builtin_memcpy(&shi, whi, 16);
    __builtin_memcpy(&slo, wlo, 16);
  };
  f32x16 kacc, qacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    kacc[r] = 0.f;
    qacc[r] = 0.f;
  }
  if constexpr (KS == 1) {
    const uint16_t* Kn = Ksh + (nt_w * 32 + lm) * kD;
    const uint16_t* Qn = Qsh + (nt_w * 32 + lm) * kD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if constexpr (FUSED) store_committed(ks);
      bf16x8 shi, slo;
      split(ks, shi, slo);
      // one workgroup per state: the next column block's S rows of this step
      // go out as soon as this step's registers are split
      if constexpr (PS) {
        if (vbi + 1 < NVB) load_S_ks((vbi + 1) * VB, ks);
      }
      const int so = kq_slot(lm, 2 * ks + hi) * 8;
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Kn + so);
      const bf16x8 qb = *reinterpret_cast<const bf16x8*>(Qn + so);
      kacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi, kb, kacc, 0, 0, 0);
      kacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo, kb, kacc, 0, 0, 0);
      qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi, qb, qacc, 0, 0, 0);
      qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo, qb, qacc, 0, 0, 0);
    }
    // K/Q staging is dead (R takes its place); with one workgroup per state, K
    // and Q stay and every wave is past the previous block's gather of R
    __syncthreads();
  } else {
    // partial products over this wave's half of d_k, for both node tiles: the
    // own tile (nt_w) accumulates in kacc/qacc, the other in kx/qx
    f32x16 kx, qx;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      kx[r] = 0.f;
      qx[r] = 0.f;
    }
    const uint16_t* Kn = Ksh + (nt_w * 32 + lm) * kD;
    const uint16_t* Qn = Qsh + (nt_w * 32 + lm) * kD;
    const uint16_t* Ko = Ksh + ((1 - nt_w) * 32 + lm) * kD;
    const uint16_t* Qo = Qsh + ((1 - nt_w) * 32 + lm) * kD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if constexpr (FUSED) store_committed(ks);
      bf16x8 shi, slo;
      split(ks, shi, slo);
      const int so = kq_slot(lm, nt_w * 8 + 2 * ks + hi) * 8;
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Kn + so);
      const bf16x8 qb = *reinterpret_cast<const bf16x8*>(Qn + so);
      const bf16x8 kob = *reinterpret_cast<const bf16x8*>(Ko + so);
      const bf16x8 qob = *reinterpret_cast<const bf16x8*>(Qo + so);
      kacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi, kb, kacc, 0, 0, 0);
      kacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo, kb, kacc, 0, 0, 0);
      qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi, qb, qacc, 0, 0, 0);
      qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo, qb, qacc, 0, 0, 0);
      kx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi, kob, kx, 0, 0, 0);
      kx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo, kob, kx, 0, 0, 0);
      qx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi, qob, qx, 0, 0, 0);
      qx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo, qob, qx, 0, 0, 0);
    }
    __syncthreads();  // K/Q staging is dead: it carries the partial products now
    // wave w hands its partial for the partner's tile to the partner (w ^ 1),
    // as float4 groups [slot][group][lane] (consecutive lanes, no conflicts);
    // the staging area holds four waves' partials, so eight waves go in two
    // rounds of four (pairs never straddle a round)
    constexpr int kRounds = NW / 4;
#pragma unroll
    for (int rnd = 0; rnd < kRounds; ++rnd) {
      const bool mine = wave / 4 == rnd;  // uniform
      if (mine) {
        float4* xo = reinterpret_cast<float4*>(smem) + (wave & 3) * (8 * 64) + lane;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          xo[g * 64] = make_float4(kx[4 * g], kx[4 * g + 1], kx[4 * g + 2], kx[4 * g + 3]);
          xo[(4 + g) * 64] = make_float4(qx[4 * g], qx[4 * g + 1], qx[4 * g + 2], qx[4 * g + 3]);
        }
      }
      __syncthreads();  // partials visible
      if (mine) {
        const float4* xi = reinterpret_cast<const float4*>(smem) + ((wave ^ 1) & 3) * (8 * 64) + lane;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 pk = xi[g * 64], pq = xi[(4 + g) * 64];
          kacc[4 * g] += pk.x;
          kacc[4 * g + 1] += pk.y;
          kacc[4 * g + 2] += pk.z;
          kacc[4 * g + 3] += pk.w;
          qacc[4 * g] += pq.x;
          qacc[4 * g + 1] += pq.y;
          qacc[4 * g + 2] += pq.z;
          qacc[4 * g + 3] += pq.w;
        }
      }
      __syncthreads();  // partials consumed (the next round's, or R, take their place)
    }
  }

  // ---- 6. R = beta (V - gamma KS) into LDS rows ----
  float* Rsh = reinterpret_cast<float*>(smem + Lay::roff);
  const float my_g = sga[my_n];
  if (my_n0 < N) {
    const float bn = sbe[my_n];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 vf = bf16x4_to_f32(vv[g]);
      float4 r;
      if (gdn) {
        r.x = bn * (vf.x - my_g * kacc[4 * g + 0]);
        r.y = bn * (vf.y - my_g * kacc[4 * g + 1]);
        r.z = bn * (vf.z - my_g * kacc[4 * g + 2]);
        r.w = bn * (vf.w - my_g * kacc[4 * g + 3]);
      } else {
        r = vf;
      }
      *reinterpret_cast<float4*>(Rsh + my_n * RS + col0 + 8 * g) = r;
    }
  }
  // one workgroup per state: the next column block's S, V and u are issued
  // now (their registers are free) and arrive during this block's gather
  if constexpr (PS) {
    if (vbi + 1 < NVB) {
      const int cn = (vbi + 1) * VB;
      if constexpr (FUSED) load_prev_ops(cn, false);
      if constexpr (KS != 1) load_S(cn);  // (with KS = 1 they went out during the contraction)
      load_V(cn);
    }
  }
  // this node's path coefficients (both chains) into registers
  float2 xw[kMaxL];
#pragma unroll
  for (int tt = 0; tt < kMaxL; ++tt) xw[tt] = tt < Lw ? XW[tt * NP + my_n] : make_float2(0.f, 0.f);
  __syncthreads();  // R rows visible

  // ---- 7. U and o gathered over the node's path rows of R ----
  // Runs to the wave's longest path (shorter paths have zero coefficients);
  // the next row's loads are issued before the current row's FMAs.
  float4 u4[4], o4[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    u4[g] = f4(0.f);
    o4[g] = make_float4(my_g * qacc[4 * g + 0], my_g * qacc[4 * g + 1], my_g * qacc[4 * g + 2],
                        my_g * qacc[4 * g + 3]);
  }
  const uint32_t epw[4] = {ep.x, ep.y, ep.z, ep.w};
  auto row_of = [&](int tt) { return Rsh + ((epw[tt >> 2] >> (8 * (tt & 3))) & 0xff) * RS + col0; };
  // two row buffers in turn, so the next row's loads are in flight during the
  // current row's FMAs and no registers are copied between steps
  auto load_row = [&](float4 (&buf)[4], int tt) {
    const float* rr = row_of(tt);
#pragma unroll
    for (int g = 0; g < 4; ++g) buf[g] = *reinterpret_cast<const float4*>(rr + 8 * g);
  };
  auto accum = [&](const float4 (&buf)[4], int tt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u4[g] = fma4(xw[tt].x, buf[g], u4[g]);
      o4[g] = fma4(xw[tt].y, buf[g], o4[g]);
    }
  };
  // Steps go in pairs under one uniform branch with unconditional loads (rows
  // past a path are valid rows with zero coefficients), which keeps each
  // buffer in the same registers.
  float4 ba[4], bb[4];
  load_row(ba, 0);
#pragma unroll
  for (int tt = 0; tt < kMaxL; tt += 2) {
    if (tt < Lw) {  // uniform
      load_row(bb, tt + 1);
      accum(ba, tt);
      load_row(ba, tt + 2 < kMaxL ? tt + 2 : tt + 1);
      accum(bb, tt + 1);
    }
  }
  if (my_n0 < N) {
    float* ur = U + ((size_t)bh * N + my_n) * kD + cbase + col0;
    uint16_t* orow = o + ((size_t)(b * N + my_n) * H + h) * kD + cbase + col0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      *reinterpret_cast<float4*>(ur + 8 * g) = u4[g];
      *reinterpret_cast<uint2*>(orow + 8 * g) = f32x4_to_bf16(o4[g].x, o4[g].y, o4[g].z, o4[g].w);
    }
  }
  }  // column blocks
}

template <int NP, int VB, bool FUSED, bool PS>
static int launch_np_vb(int B, int H, int N, int mode, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const int32_t* parents,
                        const float* S_root, void* o, float* U, int32_t* status, hipStream_t stream,
                        const PrevCommit* prev) {
  const long long nblocks = (long long)B * H * (PS ? 1 : kD / VB);
  if (nblocks > 0x7fffffffLL) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL((verify_mfma_kernel<NP, VB, FUSED, PS>), dim3((unsigned)nblocks),
                     dim3((64 * mfma_waves<NP, VB>())), 0, stream, H, N, mode,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), alpha, beta, parents, S_root,
                     static_cast<uint16_t*>(o), U, status, FUSED ? *prev : PrevCommit{});
  return static_cast<int>(hipGetLastError());
}

int launch_verify_mfma(int B, int H, int N, int mode, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const int32_t* parents,
                       const float* S_root, void* o, float* U, int32_t* status,
                       hipStream_t stream, const PrevCommit* prev) {
  // Shapes (measured at the 8-, 64- and 128-node workloads):
  //  - up to 32 nodes: one workgroup per state already (a single 128-column block);
  //  - up to 64 nodes: verify with one workgroup per state (two per CU, 43-44 us
  //    against 44.5-45 us); the fused step with one per (state, 64-column block),
  //    three per CU (57.5-58.5 us against 58-59 us);
  //  - up to 128 nodes: one workgroup per state (one per CU; 640-650 us against
  //    885 us for verify, 780-795 us against 1040 us fused).
#define TV_ARGS B, H, N, mode, q, k, v, alpha, beta, parents, S_root, o, U, status, stream, prev
  if (N <= 32)
    return prev ? launch_np_vb<32, 128, true, false>(TV_ARGS) : launch_np_vb<32, 128, false, false>(TV_ARGS);
  if (N <= 64)
    return prev ? launch_np_vb<64, 64, true, false>(TV_ARGS) : launch_np_vb<64, 64, false, true>(TV_ARGS);
  return prev ? launch_np_vb<128, 64, true, true>(TV_ARGS) : launch_np_vb<128, 64, false, true>(TV_ARGS);
#undef TV_ARGS
}

}  // namespace tv
