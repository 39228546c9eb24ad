// Tree index (debug/test entry) and the path-only commit kernel.
//
// Commit: Twig's abstract and TreeWY's abstract both say only the accepted
// state is rebuilt, from token-level factors kept at verification time; the
// Bole auto-summary writes the rebuild as a product of per-token factors
// applied to S_root ("核心公式", third formula) and spells out the c3 case in
// its worked example.  With the pseudo-values u_j from verification every
// token update is S -> alpha_j S + k_j u_j^T, so the accepted node a gets
//
//   S_new = gamma_a S_root + sum_{j on path(a)} D(j->a) k_j u_j^T,
//
// gamma_a the product of alpha over path(a) and D(j->a) the product over the
// path nodes after j.  That is a rank-len(a) update streamed over the state:
// one read and one write of d_k x d_v floats per (sequence, head).
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {

__global__ __launch_bounds__(kThreads) void index_kernel(int N, const int32_t* __restrict__ parents,
                                                         int32_t* __restrict__ depth,
                                                         unsigned long long* __restrict__ anc,
                                                         int32_t* __restrict__ status) {
  __shared__ TreeLds t;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  build_tree(t, parents + (size_t)b * N, N);
  const int W = (N + 63) / 64;
  const bool bad = t.bad != 0;
  if (tid < N) {
    depth[(size_t)b * N + tid] = bad ? 0 : t.depth[tid];
    for (int w = 0; w < W; ++w) anc[((size_t)b * N + tid) * W + w] = bad ? 0ull : t.anc[tid][w];
  }
  if (tid == 0 && status) status[b] = bad ? 1 : 0;
}

// Trees above 128 nodes: one thread per node walks its path and writes the
// ancestor words as it crosses them (indices fall along the walk, so each word
// is finished before the next lower one starts).
__global__ __launch_bounds__(kMaxTree) void index_wide_kernel(int N,
                                                             const int32_t* __restrict__ parents,
                                                             int32_t* __restrict__ depth,
                                                             unsigned long long* __restrict__ anc,
                                                             int32_t* __restrict__ status) {
  __shared__ int spar[kMaxTree];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int W = (N + 63) / 64;
  int p = -1;
  if (tid < N) {
    p = parents[(size_t)b * N + tid];
    spar[tid] = p;
  }
  const bool bad = __syncthreads_or(tid < N && (p < -1 || p >= tid)) != 0;
  if (tid == 0 && status) status[b] = bad ? 1 : 0;
  if (tid >= N) return;
  unsigned long long* a = anc + ((size_t)b * N + tid) * W;
  for (int w = 0; w < W; ++w) a[w] = 0ull;
  if (bad) {
    depth[(size_t)b * N + tid] = 0;
    return;
  }
  int d = -1, w = tid >> 6;
  unsigned long long bits = 0ull;
  for (int j = tid; j >= 0; j = spar[j]) {
    if ((j >> 6) != w) {
      a[w] = bits;
      w = j >> 6;
      bits = 0ull;
    }
    bits |= 1ull << (j & 63);
    ++d;
  }
  a[w] = bits;
  depth[(size_t)b * N + tid] = d;
}

// One workgroup per (sequence, head, tile of RT = RPP * P state rows); with
// P = DV / 8 a tile is 128 rows, i.e. the whole d_k x d_v state at d_k = 128
// (the launcher takes smaller tiles at d_v = 128).  Thread t owns float4
// column group t % CG of rows r0 + t / CG + p * RPP.
//
// Timeline of a workgroup: every state load of the tile is issued at once
// (after the few small loads the path walk needs); the first barrier lets them
// land; the path is walked from the accepted node; the path's U rows and k
// entries are staged in LDS (one dependent round trip), and the rank-len(a)
// update is applied in registers and stored.
template <typename TK, int DV, int P, int NMAX>
__global__ __launch_bounds__(kThreads, NMAX > kMaxNodes ? 4 : 1) void commit_kernel(
    int H, int N, int dk, int ntiles, const TK* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ U, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ accepted, const float* S_root, float* S_out,
    int32_t* __restrict__ path_out, int32_t* __restrict__ status) {
  constexpr int CG = DV / 4;            // float4 column groups per row
  constexpr int RPP = kThreads / CG;    // rows per pass
  constexpr int RT = RPP * P;           // rows per tile
  constexpr int CH = 16;                // path entries staged per round
  constexpr int VE = 16 / sizeof(TK);   // k elements per 16-byte load
  static_assert(RT % VE == 0, "tile rows come in whole 16-byte k chunks");
  // NMAX: largest tree of the instance (128, or 512 with a second node per thread)
  __shared__ int spar[NMAX];
  __shared__ float sal[NMAX];
  __shared__ int pidx[NMAX];            // path, accepted node first (distance order)
  __shared__ float coef[NMAX];          // D(pidx[i] -> a): product of alpha over distances < i
  __shared__ float gam;
  __shared__ int slen;
  __shared__ float4 ush[CH][CG];
  __shared__ __align__(16) float ksh[CH][RT];

  const int tid = threadIdx.x;
  // the row tiles of one state go to one XCD together (they share the path's
  // U rows through its L2), while the chip walks the states in order
  const int bid = xcd_group(blockIdx.x, gridDim.x, ntiles);
  const int tile = bid % ntiles;
  const int bh = bid / ntiles;
  const int h = bh % H;
  const int b = bh / H;
  const int r0 = tile * RT;
  const int cg = tid % CG;
  const int rsub = tid / CG;

  // small loads first (loads retire in order), then the whole state tile
  const int pn = tid < N ? tid : N - 1;
  const int par_v = parents[(size_t)b * N + pn];
  const float a_all = alpha[(size_t)(b * N + pn) * H + h];
  const int a_in = accepted[b];
  const float4* Sp = reinterpret_cast<const float4*>(S_root + (size_t)bh * dk * DV);
  float4 acc[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int r = min(r0 + rsub + p * RPP, dk - 1);
    acc[p] = Sp[(size_t)r * CG + cg];
  }
  if (tid < N) {
    spar[tid] = par_v;
    sal[tid] = a_all;
  }
  bool bad_par = __syncthreads_or(tid < N && (par_v < -1 || par_v >= tid)) != 0;
  if (NMAX > kThreads && N > kThreads) {  // uniform: a second node per thread
    // (after the first barrier, so that the load order above stays as it is)
    const int tid2 = tid + kThreads;
    const int pn2 = tid2 < N ? tid2 : N - 1;
    const int par_v2 = parents[(size_t)b * N + pn2];
    const float a_all2 = alpha[(size_t)(b * N + pn2) * H + h];
    if (tid2 < N) {
      spar[tid2] = par_v2;
      sal[tid2] = a_all2;
    }
    bad_par = (__syncthreads_or(tid2 < N && (par_v2 < -1 || par_v2 >= tid2)) != 0) || bad_par;
  }
  const bool bad_acc = a_in < 0 || a_in >= N;
  if (tid == 0) {
    // walk up from the accepted node; parents[i] < i makes it end within N steps
    int len = 0;
    float c = 1.f;
    if (!bad_par) {
      for (int n = bad_acc ? 0 : a_in; n >= 0; n = spar[n]) {
        pidx[len] = n;
        coef[len] = c;
        c *= sal[n];
        ++len;
      }
    }
    gam = c;
    slen = len;
  }
  __syncthreads();
  const int L = slen;
  if (h == 0 && tile == 0) {
    if (tid == 0 && status) status[b] = bad_par ? 1 : (bad_acc ? 2 : 0);
    if (path_out)
      for (int i = tid; i < (NMAX > kThreads ? N : min(N, kThreads)); i += kThreads)
        path_out[(size_t)b * N + i] = (!bad_par && !bad_acc && i < L) ? pidx[L - 1 - i] : -1;
  }
  const float g = gam;
#pragma unroll
  for (int p = 0; p < P; ++p) acc[p] = mul4(g, acc[p]);

  const float* Ubh = U + (size_t)bh * N * DV;
  for (int j0 = 0; j0 < L; j0 += CH) {
    const int nj = min(CH, L - j0);
    for (int i = tid; i < nj * CG; i += kThreads) {
      const int jj = i / CG;
      ush[jj][i % CG] = reinterpret_cast<const float4*>(Ubh + (size_t)pidx[j0 + jj] * DV)[i % CG];
    }
    for (int i = tid; i < nj * (RT / VE); i += kThreads) {
      const int jj = i / (RT / VE);
      const int rr = (i % (RT / VE)) * VE;
      const int node = pidx[j0 + jj];
      const float cf = coef[j0 + jj];
      float kv[VE];
      if (r0 + rr < dk) {
        const TK* kp = k + ((size_t)(b * N + node) * H + h) * dk + r0 + rr;
        if constexpr (VE == 8) {
          const uint4 w = *reinterpret_cast<const uint4*>(kp);
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv[2 * e] = __uint_as_float(ws[e] << 16);
            kv[2 * e + 1] = __uint_as_float(ws[e] & 0xffff0000u);
          }
        } else {
          const float4 w = *reinterpret_cast<const float4*>(kp);
          kv[0] = w.x;
          kv[1] = w.y;
          kv[2] = w.z;
          kv[3] = w.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) kv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < VE; e += 4)
        *reinterpret_cast<float4*>(&ksh[jj][rr + e]) =
            make_float4(cf * kv[e], cf * kv[e + 1], cf * kv[e + 2], cf * kv[e + 3]);
    }
    __syncthreads();
    for (int jj = 0; jj < nj; ++jj) {
      const float4 u = ush[jj][cg];
#pragma unroll
      for (int p = 0; p < P; ++p) acc[p] = fma4(ksh[jj][rsub + p * RPP], u, acc[p]);
    }
    __syncthreads();
  }

  float4* Op = reinterpret_cast<float4*>(S_out + (size_t)bh * dk * DV);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int r = r0 + rsub + p * RPP;
    if (r < dk) Op[(size_t)r * CG + cg] = acc[p];
  }
}

int launch_index(int B, int N, const int32_t* parents, int32_t* depth, uint64_t* anc,
                 int32_t* status, hipStream_t stream) {
  if (N > kMaxNodes)
    hipLaunchKernelGGL(index_wide_kernel, dim3(B), dim3(kMaxTree), 0, stream, N, parents, depth,
                       reinterpret_cast<unsigned long long*>(anc), status);
  else
    hipLaunchKernelGGL(index_kernel, dim3(B), dim3(kThreads), 0, stream, N, parents, depth,
                       reinterpret_cast<unsigned long long*>(anc), status);
  return static_cast<int>(hipGetLastError());
}

template <typename TK, int DV, int P>
static int commit_launch(int B, int H, int N, int dk, const void* k, const float* alpha,
                         const float* U, const int32_t* parents, const int32_t* accepted,
                         const float* S_root, float* S_out, int32_t* path_out, int32_t* status,
                         hipStream_t stream) {
  constexpr int RT = (kThreads / (DV / 4)) * P;
  const int ntiles = (dk + RT - 1) / RT;
  const long long nblocks = (long long)B * H * ntiles;
  if (nblocks > 0x7fffffffLL) return static_cast<int>(hipErrorInvalidConfiguration);
  if (N <= kMaxNodes)
    hipLaunchKernelGGL((commit_kernel<TK, DV, P, kMaxNodes>), dim3((unsigned)nblocks), dim3(kThreads),
                       0, stream, H, N, dk, ntiles, static_cast<const TK*>(k), alpha, U, parents,
                       accepted, S_root, S_out, path_out, status);
  else
    hipLaunchKernelGGL((commit_kernel<TK, DV, P, kMaxTree>), dim3((unsigned)nblocks), dim3(kThreads),
                       0, stream, H, N, dk, ntiles, static_cast<const TK*>(k), alpha, U, parents,
                       accepted, S_root, S_out, path_out, status);
  return static_cast<int>(hipGetLastError());
}

// Tiles of 128 rows (the whole state at d_k = 128); at d_v = 128, 32-row
// tiles: four workgroups per state, so the grid drains in small pieces (at
// 8192 states a launch took 194 us against 213 with whole-state tiles, and
// 1024 states are as fast either way).
template <typename TK, int DV>
static int commit_dv(int B, int H, int N, int dk, const void* k, const float* alpha, const float* U,
                     const int32_t* parents, const int32_t* accepted, const float* S_root,
                     float* S_out, int32_t* path_out, int32_t* status, hipStream_t stream) {
  if constexpr (DV == 128) {
    if (dk > 64)
      return commit_launch<TK, DV, DV / 32>(B, H, N, dk, k, alpha, U, parents, accepted, S_root,
                                            S_out, path_out, status, stream);
  }
  return commit_launch<TK, DV, DV / 8>(B, H, N, dk, k, alpha, U, parents, accepted, S_root, S_out,
                                       path_out, status, stream);
}

template <typename TK>
static int commit_t(int B, int H, int N, int dk, int dv, const void* k, const float* alpha,
                    const float* U, const int32_t* parents, const int32_t* accepted,
                    const float* S_root, float* S_out, int32_t* path_out, int32_t* status,
                    hipStream_t stream) {
  switch (dv) {
    case 16: return commit_dv<TK, 16>(B, H, N, dk, k, alpha, U, parents, accepted, S_root, S_out, path_out, status, stream);
    case 32: return commit_dv<TK, 32>(B, H, N, dk, k, alpha, U, parents, accepted, S_root, S_out, path_out, status, stream);
    case 64: return commit_dv<TK, 64>(B, H, N, dk, k, alpha, U, parents, accepted, S_root, S_out, path_out, status, stream);
    case 128: return commit_dv<TK, 128>(B, H, N, dk, k, alpha, U, parents, accepted, S_root, S_out, path_out, status, stream);
  }
  return static_cast<int>(hipErrorInvalidValue);
}

int launch_commit(int B, int H, int N, int dk, int dv, int dtype, const void* k, const float* alpha,
                  const float* U, const int32_t* parents, const int32_t* accepted,
                  const float* S_root, float* S_out, int32_t* path_out, int32_t* status,
                  hipStream_t stream) {
  if (dtype == 0)
    return commit_t<float>(B, H, N, dk, dv, k, alpha, U, parents, accepted, S_root, S_out, path_out, status, stream);
  return commit_t<uint16_t>(B, H, N, dk, dv, k, alpha, U, parents, accepted, S_root, S_out, path_out, status, stream);
}

}  // namespace tv
