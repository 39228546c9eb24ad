// Tree-masked attention for the full-attention layers of a hybrid model during
// tree verification: bf16 q/k/v, head dim 128, grouped query heads.
//
// Twig abstract and Bole abstract: the model interleaves full-attention layers,
// which keep a key/value cache of the committed context, with recurrent
// linear-attention layers, and verification runs one forward over every node
// of the draft tree.  Draft node n sees what its own root path sees: the
// committed prefix (the first prefix_len[b] cache entries) and the draft nodes
// on its root path, itself included (the tree semantics of the Bole
// auto-summary worked example).  Per query row (node n, query head hq, key/value
// head hq / G):
//
//   o = sum_j softmax_j(scale q.k_j) v_j   over the visible keys j.
//
// One workgroup (4 waves) per (sequence b, key/value head, block of 128 query
// rows); a query row is (node, head in the group), rows in node-major order,
// and each wave owns 32 of them.  Keys stream through LDS 32 at a time: first
// the committed prefix, then the draft nodes up to the block's last node.  Per
// tile, on matrix cores (32x32x16 bf16):
//   S^T = K Q^T, so a lane owns one query (lane % 32) and 16 of the 32 keys:
//   the online softmax needs one cross-lane exchange per tile;
//   O += P V with P rounded to bf16: the score accumulator is already P's
//   operand layout when the k-steps take keys in the accumulator's row order,
//   and V is read in that order from a row-major tile in LDS.
// A tile's rows are loaded into registers five tiles ahead and written to one
// of four LDS buffers two tiles ahead; one barrier covers two tiles.
#include <atomic>

#include "tv_device.h"
#include "tv_launch.h"

namespace tv {

namespace {

constexpr int kAT = 256;          // threads per workgroup
constexpr int kAD = 128;          // head dim
constexpr int kARows = 128;       // query rows per workgroup
constexpr int kAKeys = 32;        // keys per tile
constexpr int kABuf = 4;          // LDS tile buffers (a barrier every second tile)
constexpr int kAMaskNodes = kARows + 1;        // nodes a row block can touch
constexpr int kAWords = kMaxTree / 32;         // ancestor words per node
constexpr int kBalSeqs = kAT;                  // sequences the work order ranks in LDS

typedef __bf16 abf16x8 __attribute__((ext_vector_type(8)));
typedef short atr4 __attribute__((ext_vector_type(4)));
typedef short atr8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) atr4 lds_tr4;
typedef float af32x16 __attribute__((ext_vector_type(16)));

// K tile rows are 256 B (16 chunks of 16 B); chunk c of row r sits at slot
// c ^ (r & 15), so the lanes of one operand read (32 rows, one chunk) spread
// over all banks.
__device__ __forceinline__ int k_slot(int row, int ch) { return ch ^ (row & 15); }

// V tile rows are 256 B too; chunk c of row r sits at slot c ^ (4 (r & 3)).  A
// transposed read covers, per 32 lanes, four consecutive rows and one 64-byte
// group of four chunks in each; the swizzle puts the four rows' groups on
// four different 16-bank quarters, so the read touches every bank once.
__device__ __forceinline__ int v_slot(int row, int ch) { return ch ^ (4 * (row & 3)); }

struct AttnLds {
  uint16_t K[kABuf][kAKeys * kAD];    // key tiles, swizzled chunks
  uint16_t V[kABuf][kAKeys * kAD];    // value tiles, swizzled chunks
  uint32_t anc[kAMaskNodes * kAWords];  // inclusive ancestor words of the block's nodes
  int par[kMaxTree];
};

// max of x over lanes l and l ^ 32 (one lane swap, no LDS round trip)
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ uint32_t bf16pair(float a, float b) {
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  const v2 x = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  uint32_t r;
  __builtin_memcpy(&r, &x, 4);
  return r;
}

// Work order.  A workgroup's work follows its sequence's prefix length, so the
// items (sequence, key/value head, query block) are ranked longest prefix
// first, and workgroup k takes the item of rank attn_rank(k).  The dispatcher
// sends workgroup k to XCD k % 8 and fills every CU's first slot before any
// second one.  When the grid is one round (at most two workgroups per CU) the
// round lasts as long as its busiest CU: on each XCD the first C workgroups
// (C = CUs per XCD) take a CU each and the next ones a second slot on the CUs
// of the first ones, so the heaviest items run alone and the rest pair the
// heavy with the light.  A longer grid goes heaviest first (each slot that
// frees takes the next heaviest).  Either way runs of consecutive ranks, the
// query blocks of one head, which read the same keys and values, stay on one
// XCD and share its L2.  A bijection on [0, G).
__device__ __forceinline__ int attn_rank(int k, int G, int ncu, int grp) {
  constexpr int kX = 8;
  const int C = ncu / kX;
  if (C > 0 && G % kX == 0 && G <= 2 * ncu) {
    const int x = k % kX, j = k / kX, J = G / kX;
    const int s0 = J < C ? J : C;   // per XCD: workgroups in first slots
    const int s1 = J - s0;          // and in second slots
    const int alone = s0 - s1;
    if (j >= C) return G - 1 - (x * s1 + (j - C));    // light, beside workgroup k - 8 C
    if (j < s1) return kX * alone + x * s1 + j;        // heavy, paired
    return x * alone + (j - s1);                       // alone on its CU: the heaviest
  }
  return xcd_group(k, G, grp);
}

__global__ __launch_bounds__(kAT, 2) void tree_attention_kernel(
    int B, int N, int Hq, int Hkv, int P_max, int nqb, int ncu, float scale_log2,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ prefix_len,
    const uint16_t* __restrict__ kt, const uint16_t* __restrict__ vt,
    const int32_t* __restrict__ parents, uint16_t* __restrict__ o, int32_t* __restrict__ status) {
  __shared__ __align__(16) AttnLds s;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lm = lane & 31, hi = lane >> 5;
  int bid;
  {
    const int per_b = Hkv * nqb;
    const int m = attn_rank(blockIdx.x, gridDim.x, ncu, nqb < 16 ? nqb : 16);
    if (B <= kBalSeqs) {
      __shared__ int sP[kBalSeqs];
      __shared__ int sel;
      if (tid < B) sP[tid] = min(max(prefix_len[tid], 0), P_max);
      __syncthreads();
      if (tid < B) {  // the sequence of rank m / per_b (longest prefix first, then by index)
        int c = 0;
        for (int t = 0; t < B; ++t) c += (sP[t] > sP[tid]) || (sP[t] == sP[tid] && t < tid);
        if (c == m / per_b) sel = tid;
      }
      __syncthreads();
      bid = sel * per_b + m % per_b;
    } else {
      bid = m;  // too many sequences to rank here: plain order
    }
  }
  // everything below that follows from the item is uniform (scalar registers,
  // scalar branches)
  bid = __builtin_amdgcn_readfirstlane(bid);
  const int qb = bid % nqb;
  const int bkv = bid / nqb;
  const int kvh = bkv % Hkv;
  const int b = bkv / Hkv;
  const int G = Hq / Hkv;
  const int R = N * G;                          // query rows of this (b, kvh)
  const int r0 = qb * kARows;
  const int n_lo = r0 / G;
  const int n_hi = min(N - 1, (min(r0 + kARows, R) - 1) / G);
  const int W = (N + 31) / 32;

  // this lane's query row and its q operand (d = 16 s + 8 hi + i)
  const int row = r0 + wave * 32 + lm;
  const int rc = min(row, R - 1);
  const int my_n = rc / G;
  const int hq = kvh * G + rc % G;
  // A negative scale is applied as its magnitude with q negated (exact in
  // bf16), so the running maximum can be taken over the unscaled scores.
  const bool negq = scale_log2 < 0.f;
  // (a zero scale runs as 1e-30: every visible score then gives exactly 1,
  // as with 0, and a hidden one, -inf, still gives 0)
  const float csc = fmaxf(fabsf(scale_log2), 1e-30f);
  abf16x8 qop[8];
  {
    const uint16_t* qr = q + (((size_t)b * N + my_n) * Hq + hq) * kAD + 8 * hi;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      uint4 w = *reinterpret_cast<const uint4*>(qr + 16 * st);
      if (negq) {
        w.x ^= 0x80008000u;
        w.y ^= 0x80008000u;
        w.z ^= 0x80008000u;
        w.w ^= 0x80008000u;
      }
      qop[st] = __builtin_bit_cast(abf16x8, w);
    }
  }

  // ---- tree: parents (validated, bad ones treated as -1), ancestor words ----
  int P = prefix_len[b];
  const bool bad_len = P < 0 || P > P_max;
  P = min(max(P, 0), P_max);
  bool my_bad = false;
  for (int i = tid; i < N; i += kAT) {
    int p = parents[(size_t)b * N + i];
    if (p < -1 || p >= i) {
      my_bad = true;
      p = -1;
    }
    s.par[i] = p;
  }
  const bool bad = __syncthreads_or(my_bad) != 0;
  if (qb == 0 && kvh == 0 && tid == 0 && status) status[b] = bad ? 1 : (bad_len ? 3 : 0);
  for (int i = tid; i <= n_hi - n_lo; i += kAT) {
    uint32_t* a = s.anc + i * kAWords;
    for (int w = 0; w < W; ++w) a[w] = 0u;
    for (int j = n_lo + i; j >= 0; j = s.par[j]) a[j >> 5] |= 1u << (j & 31);
  }

  // ---- key tiles: prefix tiles [0, TP), then tree tiles up to node n_hi ----
  const int TP = (P + kAKeys - 1) / kAKeys;
  const int T = TP + n_hi / kAKeys + 1;
  // the loop runs in steps of four tiles; tiles past T are fully masked
  // (their loads repeat tile T - 1), so the loop body has no branches and the
  // wait counts before each LDS store stay exact
  const int T4 = (T + 3) / 4 * 4;
  // Uniform row bases of this (sequence, key/value head): its committed cache
  // rows and its tree rows; a thread adds a 32-bit byte offset (the launch
  // checks that they fit).
  const size_t cache_bh = ((size_t)b * Hkv + kvh) * P_max;
  const char* kpre = reinterpret_cast<const char*>(kc + cache_bh * kAD);
  const char* vpre = reinterpret_cast<const char*>(vc + cache_bh * kAD);
  const char* ktre = reinterpret_cast<const char*>(kt + ((size_t)b * N * Hkv + kvh) * kAD);
  const char* vtre = reinterpret_cast<const char*>(vt + ((size_t)b * N * Hkv + kvh) * kAD);
  // Thread's two 16-byte chunks of a tile: chunk c = tid + 256 u, key c / 16,
  // dims 8 (c % 16) .. + 7.  Four register sets: a tile's rows are loaded
  // five iterations before the iteration that computes it, and written to
  // LDS two iterations before.
  // source rows of this thread's chunk u (0, 1) of tile t
  auto src_rows = [&](int t, int u, const uint16_t*& kp, const uint16_t*& vp) {
    t = min(t, T - 1);
    const int key = (tid >> 4) + 16 * u;
    const uint32_t chb = 16u * (tid & 15);
    if (t + 1 < TP) {  // uniform: all 32 rows are committed rows (t * 32 + key < P)
      const char* kb = kpre + static_cast<size_t>(t * kAKeys + 16 * u) * (kAD * 2);
      const char* vb = vpre + static_cast<size_t>(t * kAKeys + 16 * u) * (kAD * 2);
      uint32_t lo = 16u * tid;
      // (opaque per use: the compiler otherwise hoists 64-bit lane pointers
      // into registers; this way the load takes a scalar base and a 32-bit
      // lane offset)
      asm volatile("" : "+v"(lo));
      kp = reinterpret_cast<const uint16_t*>(kb + lo);
      vp = reinterpret_cast<const uint16_t*>(vb + lo);
    } else if (t < TP) {  // uniform
      const uint32_t off = static_cast<uint32_t>(min(t * kAKeys + key, P - 1)) * (kAD * 2) + chb;
      kp = reinterpret_cast<const uint16_t*>(kpre + off);
      vp = reinterpret_cast<const uint16_t*>(vpre + off);
    } else {
      const uint32_t off =
          static_cast<uint32_t>(min((t - TP) * kAKeys + key, N - 1) * Hkv) * (kAD * 2) + chb;
      kp = reinterpret_cast<const uint16_t*>(ktre + off);
      vp = reinterpret_cast<const uint16_t*>(vtre + off);
    }
  };
  auto store_chunk = [&](int buf, int u, uint4 kv, uint4 vv) {
    const int c = tid + kAT * u;
    const int key = c >> 4, ch = c & 15;
    *reinterpret_cast<uint4*>(&s.K[buf][key * kAD + k_slot(key, ch) * 8]) = kv;
    *reinterpret_cast<uint4*>(&s.V[buf][key * kAD + v_slot(key, ch) * 8]) = vv;
  };
  // four register sets (X = A, B, C, D) of two chunks of K and V each
  uint4 kA0, kA1, vA0, vA1, kB0, kB1, vB0, vB1, kC0, kC1, vC0, vC1, kD0, kD1, vD0, vD1;
#define TV_LOAD(X, t)                                              \
  {                                                                \
    const uint16_t *kp_, *vp_;                                     \
    src_rows((t), 0, kp_, vp_);                                    \
    k##X##0 = *reinterpret_cast<const uint4*>(kp_);                \
    v##X##0 = *reinterpret_cast<const uint4*>(vp_);                \
    src_rows((t), 1, kp_, vp_);                                    \
    k##X##1 = *reinterpret_cast<const uint4*>(kp_);                \
    v##X##1 = *reinterpret_cast<const uint4*>(vp_);                \
  }
#define TV_STORE(X, t)                                             \
  {                                                                \
    store_chunk((t) & 3, 0, k##X##0, v##X##0);                     \
    store_chunk((t) & 3, 1, k##X##1, v##X##1);                     \
  }

  af32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  // one key tile from LDS buffer t % 4 into the running softmax and O^T
  auto compute_tile = [&](int t) {
    const int buf = t & 3;
    // S^T = K Q^T: this lane holds keys 8 (r/4) + 4 hi + r%4 of the tile for query lm
    af32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    // the eight K operand reads go out four ahead of the dependent matrix
    // instructions (one read in flight left each product waiting on LDS)
    const uint16_t* Kr = s.K[buf] + lm * kAD;
    abf16x8 ka[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) ka[st] = *reinterpret_cast<const abf16x8*>(Kr + k_slot(lm, 2 * st + hi) * 8);
#pragma unroll
    for (int st = 0; st < 8; ++st) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st], qop[st], sacc, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // The running maximum m_run (per query, in scaled base-2 units) moves only
    // when some query of the wave gains more than 2^8 on it (one uniform
    // branch): until then the probabilities stay below 256, exact to fp32
    // rounding, and O^T and l need no rescaling.  mt: the tile's largest
    // visible unscaled score of this lane's query.
    auto track_max = [&](float mt) {
      mt = xor32_max(mt);
      const float ms = mt * csc;
      if (__any(ms > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, ms);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        // O's lane holds queries 8 (r/4) + 4 hi + r%4; their factors sit in
        // lanes of those queries
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float ar = __shfl(alpha, 8 * (r >> 2) + 4 * hi + (r & 3));
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) oacc[dt][r] *= ar;
        }
      }
    };
    // p = 2^(scale' s - m_run) on the transcendental unit (results below the
    // fp32 normal range flush to 0: such probabilities vanish against the
    // maximum's 1 in the sum and in bf16)
    if ((t + 1) * kAKeys > P) {  // uniform: not a prefix tile whose keys are all visible
      // visibility: prefix keys below P; tree keys on the query node's root
      // path; none past the last tile
      uint32_t vis = 0u;
      if (t < TP) {
        vis = (1u << (P - t * kAKeys)) - 1u;  // 1 .. 31 keys left
      } else if (t < T) {
        vis = s.anc[(my_n - n_lo) * kAWords + (t - TP)];
      }
      const uint32_t vh = vis >> (4 * hi);  // bit 8 (r/4) + r%4: key 8 (r/4) + 4 hi + r%4
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sacc[r] = ((vh >> (8 * (r >> 2) + (r & 3))) & 1u) ? sacc[r] : -__builtin_inff();
    }
    // (the NaN-propagating maximum takes three scores per instruction with no
    // canonicalising moves)
    float mt = __builtin_elementwise_maximum(sacc[0], sacc[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mt = __builtin_elementwise_maximum(mt, sacc[r]);
    track_max(mt);
    const float nm = -m_run;
    // l sums the probabilities in fp32 (the value product takes them rounded
    // to bf16)
    float psum = 0.f;
    uint32_t pw[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[r], csc, nm));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[r + 1], csc, nm));
      psum += p0 + p1;
      pw[r >> 1] = bf16pair(p0, p1);
    }
    l_run += psum;
    // O += P V on matrix cores.  P is already the A operand: k-step h2 of lane
    // (query lm, hi) holds keys 16 h2 + 4 hi + (0..3) and 16 h2 + 8 + 4 hi +
    // (0..3) (its accumulator rows 8 h2 .. 8 h2 + 7); the B operand takes the
    // same keys of value column 32 dt + lm from the row-major V tile.
    // The B operand comes from LDS transpose reads: within each 16-lane group
    // g, lane i receives element i % 4 of the 8-byte chunks addressed by lanes
    // i/4, i/4 + 4, i/4 + 8, i/4 + 12.  So lane (q = lane % 4, j = lane/4 % 4)
    // of group g addresses columns 16 (g % 2) + 4 q .. + 3 of key row
    // 4 (g / 2) + j (+ 16 h2, + 8 for the second half of the k-step), and lane
    // (column n, hi) gets keys 4 hi + (0..3) of its column.
    // (with the swizzle, row 4 (lane / 32) + j, j = lane / 4 % 4, holds column
    // group dt at group dt ^ j)
    const int vj = (lane >> 2) & 3;
    const uint16_t* vtr = s.V[buf] + (4 * (lane >> 5) + vj) * kAD + 4 * (lane & 1) +
                          8 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1));
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      abf16x8 pa;
      __builtin_memcpy(&pa, &pw[4 * h2], 16);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t* v0 = vtr + 16 * h2 * kAD + 32 * (dt ^ vj);
        // (C casts: the generic pointer into the LDS tile to an LDS pointer)
        const atr4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4*)(v0));
        const atr4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4*)(v0 + 8 * kAD));
        const atr8 w = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        const abf16x8 vb = __builtin_bit_cast(abf16x8, w);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vb, oacc[dt], 0, 0, 0);
      }
    }
  };

  // q (and the tree's loads) have landed before the pipeline starts, so no
  // wait inside the loop is held up by them
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
  // pipeline: tile t + 5 loaded, tile t computed from LDS buffer t % 4, tile
  // t + 2 stored, and a barrier after every second tile.  Register set
  // t % 4 holds tile t from its load until its store; buffer (t + 2) % 4 held
  // tile t - 2, whose readers have passed a barrier since.
  TV_LOAD(A, 0)
  TV_LOAD(B, 1)
  TV_LOAD(C, 2)
  TV_LOAD(D, 3)
  TV_STORE(A, 0)
  TV_STORE(B, 1)
  TV_LOAD(A, 4)
  __syncthreads();  // first two tiles and the ancestor words visible
  for (int t = 0; t < T4; t += 4) {
    TV_LOAD(B, t + 5)
    compute_tile(t);
    TV_STORE(C, t + 2)
    TV_LOAD(C, t + 6)
    compute_tile(t + 1);
    TV_STORE(D, t + 3)
    __syncthreads();
    TV_LOAD(D, t + 7)
    compute_tile(t + 2);
    TV_STORE(A, t + 4)
    TV_LOAD(A, t + 8)
    compute_tile(t + 3);
    TV_STORE(B, t + 5)
    __syncthreads();
  }
#undef TV_LOAD
#undef TV_STORE

  // ---- normalise and store: this lane holds value column 32 dt + lm of the
  // wave's queries 8 (r/4) + 4 hi + r%4 ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;  // for query lm
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qi = 8 * (r >> 2) + 4 * hi + (r & 3);
    const float iq = __shfl(inv, qi);
    const int rq = r0 + wave * 32 + qi;
    if (rq < R) {
      const int nq = rq / G;
      const int hqq = kvh * G + rq % G;
      uint16_t* orow = o + (((size_t)b * N + nq) * Hq + hqq) * kAD + lm;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) orow[32 * dt] = f32_to_bf16(oacc[dt][r] * iq);
    }
  }
}

// Compute units of the current device, asked once per device (0 if the
// runtime cannot say: the work order then goes heaviest first).
int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 0;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

int launch_tree_attention(int B, int N, int Hq, int Hkv, int P_max, float scale, const void* q,
                          const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                          const void* k_tree, const void* v_tree, const int32_t* parents, void* o,
                          int32_t* status, hipStream_t stream) {
  const int G = Hq / Hkv;
  const long long rows = (long long)N * G;
  const int nqb = (int)((rows + kARows - 1) / kARows);
  const long long nblocks = (long long)B * Hkv * nqb;
  if (nblocks > 0x7fffffffLL) return static_cast<int>(hipErrorInvalidConfiguration);
  // 32-bit byte offsets within one (sequence, key/value head): cache rows and tree rows
  if ((long long)P_max * kAD * 2 > 0xffffffffLL ||
      (long long)N * Hkv * kAD * 2 > 0xffffffffLL)
    return static_cast<int>(hipErrorInvalidValue);
  const float scale_log2 = scale * 1.4426950408889634f;  // log2(e): softmax in base 2
  hipLaunchKernelGGL(tree_attention_kernel, dim3((unsigned)nblocks), dim3(kAT), 0, stream, B, N,
                     Hq, Hkv, P_max, nqb, device_cus(), scale_log2, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                     prefix_len, static_cast<const uint16_t*>(k_tree),
                     static_cast<const uint16_t*>(v_tree), parents, static_cast<uint16_t*>(o),
                     status);
  return static_cast<int>(hipGetLastError());
}

}  // namespace tv
