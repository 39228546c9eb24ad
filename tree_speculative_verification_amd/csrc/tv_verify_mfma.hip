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
// One workgroup per (b, h, block of VB value columns), four waves:
//   1. loads, small ones first: parents and gates, K and Q rows (staged in
//      LDS), this wave's 32 columns of S_root straight into MFMA operand
//      registers, and V at the positions the outputs land on;
//   2. tree index by pointer jumping: depth and ancestor bitsets in LDS;
//   3. Gram on matrix cores (32x32x16 bf16, exact products): lower-triangular
//      blocks of K K^T and Q K^T; only ancestor-pair entries are kept,
//      stored by the ancestor's depth (the ancestor-masked Gram/decay builder);
//   4. one thread per node solves its path for x and w (decays as running
//      products of alpha, no log/exp), padded with zeros to 16 entries;
//      this overlaps the S stream;
//   5. Y^T = S_block^T [K;Q]^T on matrix cores with S split into bf16 hi + lo
//      (q and k are exact in bf16: ~2^-17 relative error); the accumulator
//      layout puts one node and 16 value columns in each lane;
//   6. R = beta (V - gamma KS) from the K accumulators into LDS;
//   7. U and o gathered over each node's path rows of R (float4), o starting
//      from gamma_n QS_n in the Q accumulators; stored straight to HBM.
// Trees with a path longer than 16 take the level-scheduled solve instead
// (same kernel, same outputs).
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;       // d_k = d_v
constexpr int kMaxL = 16;     // longest root-to-node path solved in registers
constexpr int kRow = kD + 8;  // bf16 row stride of staged K/Q (16-byte pad against bank conflicts)

template <int NP, int VB>
struct MfmaLayout {
  static constexpr int RS = VB + 4;                 // fp32 row stride of R in LDS
  static constexpr int stage = 2 * NP * kRow * 2;   // K, Q bf16 until the Y contraction
  static constexpr int rbytes = NP * RS * 4;        // R rows, over the dead staging
  static constexpr int u0 = stage > rbytes ? stage : rbytes;
  static constexpr int bytes = u0 > (int)sizeof(LevelLds) ? u0 : (int)sizeof(LevelLds);
};

// Accumulator element r of a 32x32 tile sits at row 8*(r/4) + 4*(lane/32) + r%4,
// column lane%32.  In Y^T the rows are value columns and the columns are nodes.
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

template <int NP, int VB>
__global__ __launch_bounds__(kThreads) void verify_mfma_kernel(
    int H, int N, int mode, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const int32_t* __restrict__ parents,
    const float* __restrict__ S_root, uint16_t* __restrict__ o, float* __restrict__ U,
    int32_t* __restrict__ status) {
  using Lay = MfmaLayout<NP, VB>;
  constexpr int NT = NP / 32;                 // node tiles
  constexpr int CT = VB / 32;                 // value-column tiles in the block
  constexpr int NVB = kD / VB;
  constexpr int PAIRS = NT * CT;              // (node tile, column tile) output tiles
  static_assert(PAIRS % 4 == 0, "four waves share the output tiles evenly");
  constexpr int PPW = PAIRS / 4;
  constexpr int NG = NT * (NT + 1);           // lower-triangular blocks of K K^T and Q K^T
  constexpr int GPW = (NG + 3) / 4;
  constexpr int KQPT = 2 * NP * (kD / 8) / kThreads;  // 16-byte chunks of K and Q per thread
  constexpr int RS = Lay::RS;

  __shared__ __align__(16) unsigned char smem[Lay::bytes];
  __shared__ float Ckk[NP * kMaxL], Cqk[NP * kMaxL];   // ancestor Gram entries by depth
  __shared__ __align__(8) float2 XW[NP * kMaxL];       // path coefficients (x for U, w for o)
  __shared__ uint8_t Ep[NP * kMaxL];                   // path nodes, distance order
  __shared__ TreeLds t;
  __shared__ float sal[NP], sbe[NP], sga[NP];
  __shared__ int Lsh[NP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int vb = bid % NVB;
  const int bh = bid / NVB;
  const int h = bh % H;
  const int b = bh / H;
  const int cbase = vb * VB;
  const bool gdn = mode == kGdn;
  const int ct_w = wave % CT;                 // every tile of this wave uses this column tile
  const int col0 = ct_w * 32 + 4 * (lane >> 5);   // + 8 g + j: this lane's columns in the block
  const int arow = lane & 31;
  const int akof = 8 * (lane >> 5);

  // ---- 1. loads: small ones first (loads retire in order) ----
  // Row indices are clamped, not branched on: padded rows repeat row N-1 and
  // only feed outputs that are discarded.
  const int pn = tid < N ? tid : N - 1;
  const int par_v = parents[(size_t)b * N + pn];
  const float a_n = alpha[(size_t)(b * N + pn) * H + h];
  const float b_raw = (gdn ? beta : alpha)[(size_t)(b * N + pn) * H + h];
  uint4 kq[KQPT];
#pragma unroll
  for (int i = 0; i < KQPT; ++i) {
    const int c = tid + i * kThreads;
    const int which = c / (NP * 16);
    const int row = min((c >> 4) % NP, N - 1);
    const int ch = c & 15;
    const uint16_t* src = which ? q : k;
    kq[i] = *reinterpret_cast<const uint4*>(src + ((size_t)(b * N + row) * H + h) * kD + ch * 8);
  }
  float sv[8][8];
  {
    const float* Sb = S_root + (size_t)bh * kD * kD + cbase + ct_w * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[ks][i] = Sb[(size_t)(ks * 16 + akof + i) * kD];
  }
  uint2 vv[PPW][4];
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    const int nt = (wave + 4 * pi) / CT;
    const int n = min(nt * 32 + arow, N - 1);
    const uint16_t* vr = v + ((size_t)(b * N + n) * H + h) * kD + cbase + col0;
#pragma unroll
    for (int g = 0; g < 4; ++g) vv[pi][g] = *reinterpret_cast<const uint2*>(vr + 8 * g);
  }
  const float b_n = gdn ? b_raw : 0.f;
  uint16_t* Ksh = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Qsh = Ksh + NP * kRow;
#pragma unroll
  for (int i = 0; i < KQPT; ++i) {
    const int c = tid + i * kThreads;
    const int which = c / (NP * 16);
    const int row = (c >> 4) % NP;
    const int ch = c & 15;
    *reinterpret_cast<uint4*>((which ? Qsh : Ksh) + row * kRow + ch * 8) = kq[i];
  }
  if (tid < N) {
    sal[tid] = a_n;
    sbe[tid] = b_n;
  }

  // ---- 2. tree index ----
  build_tree_from(t, par_v, N);
  if (h == 0 && vb == 0 && tid == 0 && status) status[b] = t.bad ? 1 : 0;
  if (t.maxdepth + 1 > kMaxL) {
    level_solve<uint16_t>(t, *reinterpret_cast<LevelLds*>(smem), mode, b, h, H, N, kD, kD, cbase,
                          cbase + VB, q, k, v, alpha, beta, S_root, o, U);
    return;
  }
  const int Lmax = t.maxdepth + 1;
  // gamma_n = product of alpha over anc*(n), root side first
  if (tid < N) {
    float g = 1.f;
    unsigned long long m0 = t.anc[tid][0], m1 = t.anc[tid][1];
    while (m0) {
      const int j = __ffsll((long long)m0) - 1;
      m0 &= m0 - 1;
      g *= sal[j];
    }
    while (m1) {
      const int j = 63 + __ffsll((long long)m1);
      m1 &= m1 - 1;
      g *= sal[j];
    }
    sga[tid] = g;
  }

  // ---- 3. ancestor-masked Gram on matrix cores ----
  {
    const int gw = (wave + 4 - (PAIRS * 2) % 4) % 4;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      int rem = gw + 4 * i, rt = -1, jt = 0;
      for (int r = 0; r < 2 * NT; ++r) {
        const int cnt = (r % NT) + 1;
        if (rem >= 0 && rem < cnt) {
          rt = r;
          jt = rem;
        }
        rem -= cnt;
      }
      if (rt < 0) continue;
      const uint16_t* X = rt < NT ? Ksh + rt * 32 * kRow : Qsh + (rt - NT) * 32 * kRow;
      f32x16 gacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) gacc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(X + arow * kRow + ks * 16 + akof);
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Ksh + (jt * 32 + arow) * kRow + ks * 16 + akof);
        gacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kb, gacc, 0, 0, 0);
      }
      const bool kk = rt < NT;
      const int col = jt * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (rt % NT) * 32 + acc_row(r, lane);
        if (row < N && col < N && anc_has(t, row, col)) {
          if (kk) {
            if (col != row) Ckk[row * kMaxL + t.depth[col]] = gacc[r];
          } else {
            Cqk[row * kMaxL + t.depth[col]] = gacc[r];
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- 4. per-node path solve (distance order: e_0 = n, e_1 = parent, ...) ----
  if (tid < N) {
    const int n = tid;
    const int L = t.depth[n] + 1;
    int e[kMaxL];
    float ea[kMaxL], eb[kMaxL];
    unsigned long long m0 = t.anc[n][0], m1 = t.anc[n][1];
#pragma unroll
    for (int d = 0; d < kMaxL; ++d) {
      int j;
      if (m1) {
        j = 127 - __clzll(m1);
        m1 &= ~(1ull << (j - 64));
      } else if (m0) {
        j = 63 - __clzll(m0);
        m0 &= ~(1ull << j);
      } else {
        j = n;  // past the root: zero coefficient, any valid row
      }
      e[d] = j;
      ea[d] = sal[j];
      eb[d] = sbe[j];
    }
    float y[kMaxL], z[kMaxL];
    const int rowo = n * kMaxL;
    const float w0 = Cqk[rowo + L - 1];
    XW[rowo] = make_float2(1.f, w0);
    Ep[rowo] = static_cast<uint8_t>(n);
    y[0] = eb[0] * ea[0];
    z[0] = w0 * eb[0] * ea[0];
    float pi = ea[0];  // D(e_t -> n) at step t
#pragma unroll
    for (int tt = 1; tt < kMaxL; ++tt) {
      float xt = 0.f, wt = 0.f;
      if (tt < L) {  // predicated, not a break: keeps the loop fully unrolled
        const int col = L - 1 - tt;  // depth of e_tt
        float sx = 0.f, sw = 0.f;
        if (gdn) {
#pragma unroll
          for (int ss = 0; ss < tt; ++ss) {
            const float gkk = Ckk[e[ss] * kMaxL + col];
            sx = fmaf(y[ss], gkk, sx);
            sw = fmaf(z[ss], gkk, sw);
          }
        }
        xt = -sx;
        wt = pi * Cqk[rowo + col] - sw;
        const float at = ea[tt];
#pragma unroll
        for (int ss = 0; ss < tt; ++ss) {
          y[ss] *= at;
          z[ss] *= at;
        }
        y[tt] = xt * eb[tt] * at;
        z[tt] = wt * eb[tt] * at;
        pi *= at;
      }
      XW[rowo + tt] = make_float2(xt, wt);
      Ep[rowo + tt] = static_cast<uint8_t>(e[tt]);
    }
    Lsh[n] = L;
  }

  // ---- 5. Y^T = S_block^T [K;Q]^T on matrix cores ----
  bf16x8 shi[8], slo[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = sv[ks][i];
      const __bf16 hb = static_cast<__bf16>(x);
      shi[ks][i] = hb;
      slo[ks][i] = static_cast<__bf16>(x - static_cast<float>(hb));
    }
  f32x16 kacc[PPW], qacc[PPW];
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      kacc[pi][r] = 0.f;
      qacc[pi][r] = 0.f;
    }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int pi = 0; pi < PPW; ++pi) {
      const int nt = (wave + 4 * pi) / CT;
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Ksh + (nt * 32 + arow) * kRow + ks * 16 + akof);
      const bf16x8 qb = *reinterpret_cast<const bf16x8*>(Qsh + (nt * 32 + arow) * kRow + ks * 16 + akof);
      kacc[pi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi[ks], kb, kacc[pi], 0, 0, 0);
      kacc[pi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo[ks], kb, kacc[pi], 0, 0, 0);
      qacc[pi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi[ks], qb, qacc[pi], 0, 0, 0);
      qacc[pi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo[ks], qb, qacc[pi], 0, 0, 0);
    }
  }
  __syncthreads();  // K/Q staging is dead from here on: R takes its place

  // ---- 6. R = beta (V - gamma KS) into LDS rows ----
  float* Rsh = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    const int n = ((wave + 4 * pi) / CT) * 32 + arow;
    if (n < N) {
      const float bn = sbe[n], gn = sga[n];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 vf = bf16x4_to_f32(vv[pi][g]);
        float4 r;
        if (gdn) {
          r.x = bn * (vf.x - gn * kacc[pi][4 * g + 0]);
          r.y = bn * (vf.y - gn * kacc[pi][4 * g + 1]);
          r.z = bn * (vf.z - gn * kacc[pi][4 * g + 2]);
          r.w = bn * (vf.w - gn * kacc[pi][4 * g + 3]);
        } else {
          r = vf;
        }
        *reinterpret_cast<float4*>(Rsh + n * RS + col0 + 8 * g) = r;
      }
    }
  }
  __syncthreads();

  // ---- 7. U and o gathered over path rows of R ----
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    const int n0 = ((wave + 4 * pi) / CT) * 32 + arow;
    const int n = min(n0, N - 1);
    // the wave runs to its longest path; shorter paths see zero coefficients
    int Lw = Lsh[n];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) Lw = max(Lw, __shfl_xor(Lw, m));
    Lw = min(Lw, Lmax);
    float4 u4[4], o4[4];
    const float gn = sga[n];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u4[g] = f4(0.f);
      o4[g] = make_float4(gn * qacc[pi][4 * g + 0], gn * qacc[pi][4 * g + 1],
                          gn * qacc[pi][4 * g + 2], gn * qacc[pi][4 * g + 3]);
    }
    for (int tt = 0; tt < Lw; ++tt) {
      const float2 cw = XW[n * kMaxL + tt];
      const float* rr = Rsh + Ep[n * kMaxL + tt] * RS + col0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 r4 = *reinterpret_cast<const float4*>(rr + 8 * g);
        u4[g] = fma4(cw.x, r4, u4[g]);
        o4[g] = fma4(cw.y, r4, o4[g]);
      }
    }
    if (n0 < N) {
      float* ur = U + ((size_t)bh * N + n) * kD + cbase + col0;
      uint16_t* orow = o + ((size_t)(b * N + n) * H + h) * kD + cbase + col0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        *reinterpret_cast<float4*>(ur + 8 * g) = u4[g];
        *reinterpret_cast<uint2*>(orow + 8 * g) = f32x4_to_bf16(o4[g].x, o4[g].y, o4[g].z, o4[g].w);
      }
    }
  }
}

template <int NP, int VB>
static int launch_np_vb(int B, int H, int N, int mode, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const int32_t* parents,
                        const float* S_root, void* o, float* U, int32_t* status, hipStream_t stream) {
  const long long nblocks = (long long)B * H * (kD / VB);
  if (nblocks > 0x7fffffffLL) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL((verify_mfma_kernel<NP, VB>), dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                     H, N, mode, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), alpha, beta, parents, S_root,
                     static_cast<uint16_t*>(o), U, status);
  return static_cast<int>(hipGetLastError());
}

int launch_verify_mfma(int B, int H, int N, int mode, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const int32_t* parents,
                       const float* S_root, void* o, float* U, int32_t* status, int vblock,
                       hipStream_t stream) {
#define TV_MFMA_ARGS B, H, N, mode, q, k, v, alpha, beta, parents, S_root, o, U, status, stream
  // four waves need (node tiles x column tiles) to be a multiple of four
  if (N <= 32) return launch_np_vb<32, 128>(TV_MFMA_ARGS);
  if (N <= 64) {
    if (vblock == 128) return launch_np_vb<64, 128>(TV_MFMA_ARGS);
    return launch_np_vb<64, 64>(TV_MFMA_ARGS);
  }
  if (vblock == 64 || vblock == 128) return launch_np_vb<128, 64>(TV_MFMA_ARGS);
  return launch_np_vb<128, 32>(TV_MFMA_ARGS);
#undef TV_MFMA_ARGS
}

}  // namespace tv
