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

// State rows each thread streams per tile (tile = 256 / (d_v / 4) * this rows).
#ifndef TV_COMMIT_ROWS_PER_THREAD
#define TV_COMMIT_ROWS_PER_THREAD 4
#endif

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

// One workgroup per (sequence, head, tile of RT state rows).  Each thread owns
// P float4 groups of one column group in rows r0 + rsub + p * RPP.
template <typename TK, int DV, int P>
__global__ __launch_bounds__(kThreads) void commit_kernel(
    int H, int N, int dk, int ntiles, const TK* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ U, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ accepted, const float* S_root, float* S_out,
    int32_t* __restrict__ path_out, int32_t* __restrict__ status) {
  constexpr int CG = DV / 4;            // float4 column groups per row
  constexpr int RPP = kThreads / CG;    // rows per pass
  constexpr int RT = RPP * P;           // rows per tile
  constexpr int CH = 16;                // path entries staged per round
  __shared__ TreeLds t;
  __shared__ int pidx[kMaxNodes];
  __shared__ float al[kMaxNodes];
  __shared__ float coef[kMaxNodes];
  __shared__ float gam;
  __shared__ float4 ush[CH][CG];
  __shared__ float ksh[CH][RT];

  const int tid = threadIdx.x;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = bid % ntiles;
  const int bh = bid / ntiles;
  const int h = bh % H;
  const int b = bh / H;
  const int r0 = tile * RT;
  const int cg = tid % CG;
  const int rsub = tid / CG;

  // Small loads first (parents, gates of every node, accepted index: the path
  // is not known yet), then the state stream; loads retire in order, so the
  // tree build waits only for the small ones.
  const int pn = tid < N ? tid : N - 1;
  const int par_v = parents[(size_t)b * N + pn];
  const float a_all = alpha[(size_t)(b * N + pn) * H + h];
  int a = accepted[b];
  const float4* Sp = reinterpret_cast<const float4*>(S_root + (size_t)bh * dk * DV);
  float4 s[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int r = min(r0 + rsub + p * RPP, dk - 1);
    s[p] = Sp[(size_t)r * CG + cg];
  }
  build_tree_from(t, par_v, N);
  if (tid < N) al[tid] = a_all;
  const bool bad_acc = a < 0 || a >= N;
  if (bad_acc) a = 0;
  const int L = t.depth[a] + 1;
  if (tid < N && anc_has(t, a, tid)) pidx[anc_rank(t, a, tid)] = tid;
  __syncthreads();
  if (h == 0 && tile == 0) {
    const bool badrow = t.bad || bad_acc;
    if (tid == 0 && status) status[b] = t.bad ? 1 : (bad_acc ? 2 : 0);
    if (path_out && tid < N) path_out[(size_t)b * N + tid] = (!badrow && tid < L) ? pidx[tid] : -1;
  }
  // coef[i] = D(path[i] -> a): product of alpha over the path nodes after path[i]
  if (tid < L) {
    float c = 1.f;
    for (int m = tid + 1; m < L; ++m) c *= al[pidx[m]];
    coef[tid] = c;
  }
  if (tid == 0) {
    float g = 1.f;
    for (int m = 0; m < L; ++m) g *= al[pidx[m]];
    gam = g;
  }
  __syncthreads();

  float4 acc[P];
  const float g = gam;
#pragma unroll
  for (int p = 0; p < P; ++p) acc[p] = mul4(g, s[p]);

  const float* Ubh = U + (size_t)bh * N * DV;
  for (int j0 = 0; j0 < L; j0 += CH) {
    const int nj = min(CH, L - j0);
    for (int i = tid; i < nj * CG; i += kThreads) {
      const int jj = i / CG;
      ush[jj][i % CG] = reinterpret_cast<const float4*>(Ubh + (size_t)pidx[j0 + jj] * DV)[i % CG];
    }
    for (int i = tid; i < nj * RT; i += kThreads) {
      const int jj = i / RT;
      const int r = r0 + i % RT;
      const int node = pidx[j0 + jj];
      ksh[jj][i % RT] =
          r < dk ? coef[j0 + jj] * Elem<TK>::load(k, ((size_t)(b * N + node) * H + h) * dk + r) : 0.f;
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
  hipLaunchKernelGGL(index_kernel, dim3(B), dim3(kThreads), 0, stream, N, parents, depth,
                     reinterpret_cast<unsigned long long*>(anc), status);
  return static_cast<int>(hipGetLastError());
}

template <typename TK, int DV>
static int commit_dv(int B, int H, int N, int dk, const void* k, const float* alpha, const float* U,
                     const int32_t* parents, const int32_t* accepted, const float* S_root,
                     float* S_out, int32_t* path_out, int32_t* status, hipStream_t stream) {
  constexpr int P = TV_COMMIT_ROWS_PER_THREAD;
  constexpr int RT = (kThreads / (DV / 4)) * P;
  const int ntiles = (dk + RT - 1) / RT;
  const long long nblocks = (long long)B * H * ntiles;
  if (nblocks > 0x7fffffffLL) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL((commit_kernel<TK, DV, P>), dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                     H, N, dk, ntiles, static_cast<const TK*>(k), alpha, U, parents, accepted,
                     S_root, S_out, path_out, status);
  return static_cast<int>(hipGetLastError());
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
