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
// Work per workgroup, (b, h, block of VB value columns):
//   1. stream S_root[:, block] (fp32) from HBM straight into MFMA operand
//      registers as a hi + lo bf16 pair (q and k are exact in bf16, so
//      [K;Q] S = [K;Q] S_hi + [K;Q] S_lo keeps ~2^-17 relative error);
//      stage K, Q (bf16) and V[:, block] in LDS;
//   2. tree index by pointer jumping (depth, ancestor bitsets) in LDS;
//   3. MFMA 32x32x16 bf16: Y = [K;Q] S_block (KS and QS) and the
//      lower-triangular blocks of the Gram G = [K;Q] K^T;
//   4. keep only ancestor-pair Gram entries, indexed by the ancestor's depth
//      (the ancestor-masked Gram/decay builder);
//   5. one thread per node solves its own root path: the path block of
//      (I + A) is unit lower-triangular, so the coefficients x (U_n = x.R_path)
//      and w (o_n = gamma_n QS_n + w.R_path) come from one backward
//      substitution of length <= 16 each, decays taken as running products of
//      alpha (no log/exp);
//   6. R from the KS accumulators, then U and o gathered over each node's
//      path rows of R straight from the MFMA accumulator layout.
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
  static constexpr int stage = 2 * NP * kRow * 2;  // K, Q bf16
  static constexpr int xw = 2 * NP * kMaxL * 4;    // path coefficients x, w
  static constexpr int e = NP * kMaxL;             // path node ids, distance order
  static constexpr int c = 2 * NP * kMaxL * 4;     // ancestor Gram entries kk, qk
  static constexpr int r = NP * VB * 4;            // R rows of this column block
  static constexpr int post = xw + e + (c > r ? c : r);
  static constexpr int bytes = stage > post ? stage : post;
};

// 32x32 accumulator element r of this lane sits at row 8*(r/4) + 4*(lane/32) + r%4,
// column lane%32 of the tile.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int NP, int VB>
__global__ __launch_bounds__(kThreads) void verify_mfma_kernel(
    int H, int N, int mode, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const int32_t* __restrict__ parents,
    const float* __restrict__ S_root, uint16_t* __restrict__ o, float* __restrict__ U,
    int32_t* __restrict__ status) {
  using Lay = MfmaLayout<NP, VB>;
  constexpr int NT = NP / 32;               // node tiles
  constexpr int CT = VB / 32;               // column tiles in the block
  constexpr int NVB = kD / VB;
  constexpr int NY = 2 * NT * CT;           // [K;Q] S tiles
  constexpr int YPW = (NY + 3) / 4;
  constexpr int NG = NT * (NT + 1);         // lower-triangular blocks of K K^T and Q K^T
  constexpr int GPW = (NG + 3) / 4;
  constexpr int KQCH = 2 * NP * (kD / 8);   // 16-byte chunks of K and Q
  constexpr int KQPT = KQCH / kThreads;
  constexpr int VCH = NP * VB / 8;
  constexpr int VPT = (VCH + kThreads - 1) / kThreads;

  __shared__ __align__(16) unsigned char smem[Lay::bytes];
  __shared__ __align__(16) uint16_t vsh[NP * VB];
  __shared__ TreeLds t;
  __shared__ LevelLds s;
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

  // ---- 1. global loads: S block into operand registers, K/Q/V chunks ----
  const int ct_w = wave % CT;
  float sv[8][8];
  {
    const float* Sb = S_root + (size_t)bh * kD * kD + cbase + ct_w * 32 + (lane & 31);
    const int kofs = 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[ks][i] = Sb[(size_t)(ks * 16 + kofs + i) * kD];
  }
  uint4 kq[KQPT];
#pragma unroll
  for (int i = 0; i < KQPT; ++i) {
    const int c = tid + i * kThreads;
    const int which = c / (NP * 16);
    const int row = (c >> 4) % NP;
    const int ch = c & 15;
    const uint16_t* src = which ? q : k;
    kq[i] = row < N ? *reinterpret_cast<const uint4*>(src + ((size_t)(b * N + row) * H + h) * kD + ch * 8)
                    : make_uint4(0, 0, 0, 0);
  }
  uint4 vv[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = tid + i * kThreads;
    const int row = c / (VB / 8);
    const int ch = c % (VB / 8);
    vv[i] = (c < VCH && row < N)
                ? *reinterpret_cast<const uint4*>(v + ((size_t)(b * N + row) * H + h) * kD + cbase + ch * 8)
                : make_uint4(0, 0, 0, 0);
  }
  float a_n = 0.f, b_n = 0.f;
  if (tid < N) {
    a_n = alpha[(size_t)(b * N + tid) * H + h];
    b_n = gdn ? beta[(size_t)(b * N + tid) * H + h] : 0.f;
  }

  // ---- 2. tree index ----
  build_tree(t, parents + (size_t)b * N, N);
  if (h == 0 && vb == 0 && tid == 0 && status) status[b] = t.bad ? 1 : 0;
  if (t.maxdepth + 1 > kMaxL) {
    level_solve<uint16_t>(t, s, mode, b, h, H, N, kD, kD, cbase, cbase + VB, q, k, v, alpha, beta,
                          S_root, o, U);
    return;
  }

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
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = tid + i * kThreads;
    if (c < VCH) *reinterpret_cast<uint4*>(vsh + c * 8) = vv[i];
  }
  if (tid < N) {
    s.alpha[tid] = a_n;
    s.beta[tid] = b_n;
  }
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
  __syncthreads();

  // ---- 3. contractions on matrix cores ----
  int grt[GPW], gjt[GPW];
  const int gw = ((wave - NY) % 4 + 4) % 4;  // spread Gram tiles after the Y tiles
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    int rem = gw + 4 * i;
    grt[i] = -1;
    gjt[i] = 0;
    for (int r = 0; r < 2 * NT && rem >= 0; ++r) {
      const int cnt = (r % NT) + 1;
      if (rem < cnt) {
        grt[i] = r;
        gjt[i] = rem;
      }
      rem -= cnt;
    }
  }
  f32x16 yacc[YPW];
  f32x16 gacc[GPW];
#pragma unroll
  for (int i = 0; i < YPW; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) yacc[i][r] = 0.f;
#pragma unroll
  for (int i = 0; i < GPW; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) gacc[i][r] = 0.f;

  const int arow = lane & 31;
  const int akof = 8 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int i = 0; i < YPW; ++i) {
      const int y = wave + 4 * i;
      if (y < NY) {
        const int rt = y / CT;
        const uint16_t* X = rt < NT ? Ksh + rt * 32 * kRow : Qsh + (rt - NT) * 32 * kRow;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(X + arow * kRow + ks * 16 + akof);
        yacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, shi[ks], yacc[i], 0, 0, 0);
        yacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, slo[ks], yacc[i], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      if (grt[i] >= 0) {
        const int rt = grt[i];
        const uint16_t* X = rt < NT ? Ksh + rt * 32 * kRow : Qsh + (rt - NT) * 32 * kRow;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(X + arow * kRow + ks * 16 + akof);
        const bf16x8 kb =
            *reinterpret_cast<const bf16x8*>(Ksh + (gjt[i] * 32 + arow) * kRow + ks * 16 + akof);
        gacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kb, gacc[i], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // K/Q staging is dead from here on

  float* Xc = reinterpret_cast<float*>(smem);
  float* Wc = Xc + NP * kMaxL;
  uint8_t* Ec = reinterpret_cast<uint8_t*>(Wc + NP * kMaxL);
  float* Ckk = reinterpret_cast<float*>(Ec + NP * kMaxL);
  float* Cqk = Ckk + NP * kMaxL;
  float* Rsh = Ckk;  // replaces Ckk/Cqk once the path coefficients are built

  // ---- 4. ancestor-masked Gram entries, indexed by the ancestor's depth ----
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    if (grt[i] >= 0) {
      const int rt = grt[i];
      const bool kk = rt < NT;
      const int col = gjt[i] * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (rt % NT) * 32 + acc_row(r, lane);
        if (row < N && col < N && anc_has(t, row, col)) {
          if (kk) {
            if (col != row) Ckk[row * kMaxL + t.depth[col]] = gacc[i][r];
          } else {
            Cqk[row * kMaxL + t.depth[col]] = gacc[i][r];
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- 5. per-node path solve (distance order: e_0 = n, e_1 = parent, ...) ----
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
        j = n;  // past the root: never used
      }
      e[d] = j;
      ea[d] = s.alpha[j];
      eb[d] = s.beta[j];
    }
    float y[kMaxL], z[kMaxL];
    const int rowo = n * kMaxL;
    const float w0 = Cqk[rowo + L - 1];
    Xc[rowo] = 1.f;
    Wc[rowo] = w0;
    Ec[rowo] = static_cast<uint8_t>(n);
    y[0] = eb[0] * ea[0];
    z[0] = w0 * eb[0] * ea[0];
    float pi = ea[0];  // D(e_t -> n) at step t, gamma_n at the end
#pragma unroll
    for (int tt = 1; tt < kMaxL; ++tt) {
      if (tt >= L) break;
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
      const float xt = -sx;
      const float wt = pi * Cqk[rowo + col] - sw;
      Xc[rowo + tt] = xt;
      Wc[rowo + tt] = wt;
      Ec[rowo + tt] = static_cast<uint8_t>(e[tt]);
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
    s.gamma[n] = pi;
    Lsh[n] = L;
  }
  __syncthreads();

  // ---- 6a. R rows of this block from the KS accumulators ----
#pragma unroll
  for (int i = 0; i < YPW; ++i) {
    const int y = wave + 4 * i;
    if (y < NY && y / CT < NT) {
      const int rt = y / CT;
      const int cl = (y % CT) * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rt * 32 + acc_row(r, lane);
        if (row < N) {
          const float vval = bf16_to_f32(vsh[row * VB + cl]);
          Rsh[row * VB + cl] = gdn ? s.beta[row] * (vval - s.gamma[row] * yacc[i][r]) : vval;
        }
      }
    }
  }
  __syncthreads();

  // ---- 6b. U (K tiles) and o (Q tiles) gathered over path rows of R ----
#pragma unroll
  for (int i = 0; i < YPW; ++i) {
    const int y = wave + 4 * i;
    if (y < NY) {
      const int rt = y / CT;
      const bool ktile = rt < NT;
      const int cl = (y % CT) * 32 + (lane & 31);
      const float* cf = ktile ? Xc : Wc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (rt % NT) * 32 + acc_row(r, lane);
        if (row < N) {
          const int L = Lsh[row];
          float acc = ktile ? 0.f : s.gamma[row] * yacc[i][r];
          for (int tt = 0; tt < L; ++tt)
            acc = fmaf(cf[row * kMaxL + tt], Rsh[Ec[row * kMaxL + tt] * VB + cl], acc);
          if (ktile)
            U[((size_t)bh * N + row) * kD + cbase + cl] = acc;
          else
            o[((size_t)(b * N + row) * H + h) * kD + cbase + cl] = f32_to_bf16(acc);
        }
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

template <int NP>
static int launch_np(int B, int H, int N, int mode, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const int32_t* parents,
                     const float* S_root, void* o, float* U, int32_t* status, int vblock,
                     hipStream_t stream) {
  switch (vblock) {
    case 32: return launch_np_vb<NP, 32>(B, H, N, mode, q, k, v, alpha, beta, parents, S_root, o, U, status, stream);
    case 64: return launch_np_vb<NP, 64>(B, H, N, mode, q, k, v, alpha, beta, parents, S_root, o, U, status, stream);
    case 128: return launch_np_vb<NP, 128>(B, H, N, mode, q, k, v, alpha, beta, parents, S_root, o, U, status, stream);
  }
  return static_cast<int>(hipErrorInvalidValue);
}

int launch_verify_mfma(int B, int H, int N, int mode, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const int32_t* parents,
                       const float* S_root, void* o, float* U, int32_t* status, int vblock,
                       hipStream_t stream) {
  if (vblock == 0) vblock = 64;
  if (N <= 32) return launch_np<32>(B, H, N, mode, q, k, v, alpha, beta, parents, S_root, o, U, status, vblock, stream);
  if (N <= 64) return launch_np<64>(B, H, N, mode, q, k, v, alpha, beta, parents, S_root, o, U, status, vblock, stream);
  return launch_np<128>(B, H, N, mode, q, k, v, alpha, beta, parents, S_root, o, U, status, vblock, stream);
}

}  // namespace tv
