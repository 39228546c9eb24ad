// Device helpers shared by the tree-verification kernels (gfx950, wave64).
//
// Tree conventions (Bole auto-summary, "How in Action" worked example: draft
// branches hang off their parent token, and off the root state when they have
// no parent token): parents[b][i] is -1 or an earlier node, so node order is
// topological and every ancestor has a smaller index than its descendants.
// anc*(n) is the root-to-n path including n, held as a 128-bit set: bit j%64
// of word j/64.  depth(n) = |anc*(n)| - 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tv {

constexpr int kMaxNodes = 128;   // trees the register-path and level kernels take
constexpr int kMaxTree = 512;    // trees the blocked kernel, commit and index take
constexpr int kThreads = 256;
constexpr int kGdn = 0;
constexpr int kScalar = 1;

// ------------------------------------------------------------------ numbers

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ float4 load4(const float* p, size_t i) {
    return *reinterpret_cast<const float4*>(p + i);
  }
  static __device__ __forceinline__ void store4(float* p, size_t i, float4 x) {
    *reinterpret_cast<float4*>(p + i) = x;
  }
};

template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ float4 load4(const uint16_t* p, size_t i) {
    uint2 u = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  static __device__ __forceinline__ void store4(uint16_t* p, size_t i, float4 x) {
    uint2 u;
    u.x = static_cast<uint32_t>(f32_to_bf16(x.x)) | (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
    u.y = static_cast<uint32_t>(f32_to_bf16(x.z)) | (static_cast<uint32_t>(f32_to_bf16(x.w)) << 16);
    *reinterpret_cast<uint2*>(p + i) = u;
  }
};

__device__ __forceinline__ float4 f4(float a) { return make_float4(a, a, a, a); }
__device__ __forceinline__ float4 fma4(float a, float4 x, float4 y) {
  return make_float4(fmaf(a, x.x, y.x), fmaf(a, x.y, y.y), fmaf(a, x.z, y.z), fmaf(a, x.w, y.w));
}
__device__ __forceinline__ float4 mul4(float a, float4 x) {
  return make_float4(a * x.x, a * x.y, a * x.z, a * x.w);
}
__device__ __forceinline__ float4 sub4(float4 x, float4 y) {
  return make_float4(x.x - y.x, x.y - y.y, x.z - y.z, x.w - y.w);
}

// ------------------------------------------------------------ block mapping

// Hardware hands consecutive workgroup ids to the 8 XCDs in turn, each XCD with
// its own L2.  xcd_remap gives each XCD one contiguous run of logical ids, so
// items that share inputs meet in one L2; but then the eight XCDs stream
// addresses a fixed, large power-of-two stride apart in lockstep and crowd the
// same HBM channels (a plain state copy laid out this way ran at 53-55 % of
// peak against 60-68 % in dispatch order).  Streaming kernels use xcd_group.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcds = 8;
  if (nblocks % kXcds) return bid;
  const int per = nblocks / kXcds;
  return (bid % kXcds) * per + bid / kXcds;
}

// Workgroup barrier that orders LDS only.  __syncthreads() is a release and
// acquire fence at workgroup scope over all memory, which makes every wave
// wait for all its outstanding global loads first, so a load issued for a
// later phase cannot stay in flight across it.  This one waits for the wave's
// LDS operations only.  Data moved into LDS by direct-to-LDS loads, and global
// memory shared between waves, still need their own waits.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Block id -> work item such that each run of g consecutive items (items that
// share inputs, e.g. the value-column blocks of one state) goes to one XCD and
// is dispatched together, while the chip as a whole walks the items in order.
// Within each run of 8 g blocks, block r (XCD r % 8) takes item (r % 8) g + r / 8;
// a ragged tail keeps dispatch order.  A bijection on [0, nblocks).
__device__ __forceinline__ int xcd_group(int bid, int nblocks, int g) {
  constexpr int kXcds = 8;
  if (g <= 1) return bid;
  const int span = kXcds * g;
  const int s = bid / span;
  if ((s + 1) * span > nblocks) return bid;
  const int r = bid - s * span;
  return s * span + (r % kXcds) * g + r / kXcds;
}

// --------------------------------------------------------------- tree index

struct TreeLds {
  int par[kMaxNodes];
  int jump[kMaxNodes];
  int depth[kMaxNodes];
  unsigned long long anc[kMaxNodes][2];
  int bad;       // a parent index outside [-1, i-1] was seen (clamped to -1)
  int maxdepth;
};

__device__ __forceinline__ bool anc_has(const TreeLds& t, int n, int j) {
  return (t.anc[n][j >> 6] >> (j & 63)) & 1ull;
}

// Number of ancestors of n with an index below j (= position of j on n's path
// when j is on it).
__device__ __forceinline__ int anc_rank(const TreeLds& t, int n, int j) {
  const unsigned long long a0 = t.anc[n][0], a1 = t.anc[n][1];
  if (j < 64) return __popcll(a0 & ((1ull << j) - 1ull));
  const unsigned long long m1 = (j == 64) ? 0ull : (a1 & ((1ull << (j - 64)) - 1ull));
  return __popcll(a0) + __popcll(m1);
}

// Builds par/depth/anc for one sequence by pointer jumping: after round r each
// node's set holds its 2^r nearest path nodes, so ceil(log2(depth+1)) rounds
// suffice.  Invalid parents are clamped to -1 and flagged.  Every thread of
// the block must call this; N <= kMaxNodes <= blockDim.x.  `par_tid` is
// parents_b[threadIdx.x] for threads below N (loaded by the caller, so the
// load can be issued ahead of bulk traffic), ignored above.
__device__ inline void build_tree_from(TreeLds& t, int par_tid, int N) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    t.bad = 0;
    t.maxdepth = 0;
  }
  __syncthreads();
  if (tid < N) {
    int p = par_tid;
    if (p < -1 || p >= tid) {
      atomicOr(&t.bad, 1);
      p = -1;
    }
    t.par[tid] = p;
    t.jump[tid] = p;
    t.anc[tid][0] = tid < 64 ? (1ull << tid) : 0ull;
    t.anc[tid][1] = tid < 64 ? 0ull : (1ull << (tid - 64));
  }
  __syncthreads();
  while (true) {
    int j = -1, jj = -1;
    unsigned long long a0 = 0, a1 = 0;
    if (tid < N) {
      j = t.jump[tid];
      if (j >= 0) {
        a0 = t.anc[j][0];
        a1 = t.anc[j][1];
        jj = t.jump[j];
      }
    }
    if (!__syncthreads_or(j >= 0)) break;
    if (j >= 0) {
      t.anc[tid][0] |= a0;
      t.anc[tid][1] |= a1;
      t.jump[tid] = jj;
    }
    __syncthreads();
  }
  if (tid < N) {
    const int d = __popcll(t.anc[tid][0]) + __popcll(t.anc[tid][1]) - 1;
    t.depth[tid] = d;
    atomicMax(&t.maxdepth, d);
  }
  __syncthreads();
}

__device__ inline void build_tree(TreeLds& t, const int32_t* __restrict__ parents_b, int N) {
  const int tid = threadIdx.x;
  build_tree_from(t, parents_b[tid < N ? tid : 0], N);
}

// ------------------------------------------------- level-scheduled tree solve
//
// Shared by the generic verify kernel and, for trees deeper than the register
// path supports, by the MFMA kernel.  For one (sequence b, head h) and the
// value columns [c0, c1) it computes the pseudo-values U and outputs o:
//
//   R_n = beta_n (v_n - gamma_n S_root^T k_n)              (gated delta rule)
//   u_n = R_n - beta_n sum_{j in anc(n)} D(j->n) (k_n.k_j) u_j   level by level
//   o_n = gamma_n S_root^T q_n + sum_{j in anc*(n)} D(j->n) (q_n.k_j) u_j
//
// with D(j->n) the product of alpha over the path nodes strictly below j down
// to n, and gamma_n the product over all of anc*(n).  This is forward
// substitution on the unit lower-triangular system (I + A) U = R whose
// off-diagonal entries sit only on ancestor pairs: nodes of one depth are
// independent, so each depth level is one parallel step.  In scalar-decay
// mode u_n = v_n.  U (global, fp32) holds R and then the solution.

struct LevelLds {
  float alpha[kMaxNodes];
  float beta[kMaxNodes];
  float gamma[kMaxNodes];
  int order[kMaxNodes];        // nodes sorted by (depth, index)
  int lstart[kMaxNodes + 1];   // first position of each depth in `order`
};

template <typename TIn>
__device__ void level_solve(const TreeLds& t, LevelLds& s, int mode, int b, int h, int H, int N,
                            int dk, int dv, int c0, int c1, const TIn* __restrict__ q,
                            const TIn* __restrict__ k, const TIn* __restrict__ v,
                            const float* __restrict__ alpha, const float* __restrict__ beta,
                            const float* __restrict__ S_root, TIn* __restrict__ o,
                            float* __restrict__ U) {
  const int tid = threadIdx.x;
  const int maxdepth = t.maxdepth;
  if (tid < N) {
    s.alpha[tid] = alpha[(size_t)(b * N + tid) * H + h];
    s.beta[tid] = mode == kGdn ? beta[(size_t)(b * N + tid) * H + h] : 0.f;
  }
  __syncthreads();
  if (tid < N) {
    float g = 1.f;
    for (int j = 0; j <= tid; ++j)
      if (anc_has(t, tid, j)) g *= s.alpha[j];
    s.gamma[tid] = g;
    const int d = t.depth[tid];
    int rank = 0;
    for (int m = 0; m < N; ++m) {
      const int dm = t.depth[m];
      rank += (dm < d) || (dm == d && m < tid);
    }
    s.order[rank] = tid;
  }
  if (tid <= maxdepth + 1) {
    int cnt = 0;
    for (int m = 0; m < N; ++m) cnt += t.depth[m] < tid;
    s.lstart[tid] = cnt;
  }
  __syncthreads();

  const int ncg = (c1 - c0) >> 2;
  const size_t krow_stride = (size_t)H * dk;
  const size_t vrow_stride = (size_t)H * dv;
  const TIn* kb = k + (size_t)b * N * krow_stride + (size_t)h * dk;
  const TIn* qb = q + (size_t)b * N * krow_stride + (size_t)h * dk;
  const TIn* vb = v + (size_t)b * N * vrow_stride + (size_t)h * dv;
  TIn* ob = o + (size_t)b * N * vrow_stride + (size_t)h * dv;
  const float* Sb = S_root + (size_t)(b * H + h) * dk * dv;
  float* Ub = U + (size_t)(b * H + h) * N * dv;

  // right-hand sides
  for (int item = tid; item < N * ncg; item += blockDim.x) {
    const int n = item / ncg;
    const int c = c0 + 4 * (item % ncg);
    float4 r = Elem<TIn>::load4(vb, (size_t)n * vrow_stride + c);
    if (mode == kGdn) {
      float4 ks = f4(0.f);
      for (int i = 0; i < dk; ++i)
        ks = fma4(Elem<TIn>::load(kb, (size_t)n * krow_stride + i),
                  *reinterpret_cast<const float4*>(Sb + (size_t)i * dv + c), ks);
      r = mul4(s.beta[n], sub4(r, mul4(s.gamma[n], ks)));
    }
    *reinterpret_cast<float4*>(Ub + (size_t)n * dv + c) = r;
  }
  __syncthreads();

  if (mode == kGdn) {
    for (int lev = 1; lev <= maxdepth; ++lev) {
      const int first = s.lstart[lev];
      const int cnt = s.lstart[lev + 1] - first;
      for (int item = tid; item < cnt * ncg; item += blockDim.x) {
        const int n = s.order[first + item / ncg];
        const int c = c0 + 4 * (item % ncg);
        float4 acc = f4(0.f);
        float D = s.alpha[n];
        for (int j = t.par[n]; j >= 0; j = t.par[j]) {
          float dot = 0.f;
          for (int i = 0; i < dk; ++i)
            dot = fmaf(Elem<TIn>::load(kb, (size_t)n * krow_stride + i),
                       Elem<TIn>::load(kb, (size_t)j * krow_stride + i), dot);
          acc = fma4(D * dot, *reinterpret_cast<const float4*>(Ub + (size_t)j * dv + c), acc);
          D *= s.alpha[j];
        }
        float4* un = reinterpret_cast<float4*>(Ub + (size_t)n * dv + c);
        *un = sub4(*un, mul4(s.beta[n], acc));
      }
      __syncthreads();
    }
  }

  // outputs
  for (int item = tid; item < N * ncg; item += blockDim.x) {
    const int n = item / ncg;
    const int c = c0 + 4 * (item % ncg);
    float4 qs = f4(0.f);
    for (int i = 0; i < dk; ++i)
      qs = fma4(Elem<TIn>::load(qb, (size_t)n * krow_stride + i),
                *reinterpret_cast<const float4*>(Sb + (size_t)i * dv + c), qs);
    float4 acc = mul4(s.gamma[n], qs);
    float D = 1.f;
    for (int j = n; j >= 0; j = t.par[j]) {
      float dot = 0.f;
      for (int i = 0; i < dk; ++i)
        dot = fmaf(Elem<TIn>::load(qb, (size_t)n * krow_stride + i),
                   Elem<TIn>::load(kb, (size_t)j * krow_stride + i), dot);
      acc = fma4(D * dot, *reinterpret_cast<const float4*>(Ub + (size_t)j * dv + c), acc);
      D *= s.alpha[j];
    }
    Elem<TIn>::store4(ob, (size_t)n * vrow_stride + c, acc);
  }
}

}  // namespace tv
