// Per-node-snapshot verification: the method the pages measure against.
//
// Twig's and Bole's abstracts describe what existing serving engines do with a
// draft tree on a recurrent layer: they verify it sequentially, branch by
// branch, and materialize the full state of every proposal node; the accepted
// node's snapshot then becomes the new state.  These kernels do exactly that on
// the GPU, so the tree-structured path can be compared with it on the same
// hardware and inputs:
//
//   for n in index order (parents first):  S_n = update(S_parent(n), token n)
//                                          snapshot[n] = S_n,  o_n = S_n^T q_n
//   commit: S_out = snapshot[accepted]
//
// One workgroup per (sequence, head, block of CB value columns) walks the nodes
// in order.  The parent's state is read back from its snapshot in memory (the
// same thread wrote those elements, so no synchronisation is needed for them);
// only the two column reductions (k^T S and q^T S) go through LDS.
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {

template <typename TIn, int CB>
__global__ __launch_bounds__(kThreads) void snapshot_verify_kernel(
    int H, int N, int dk, int dv, int mode, const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ parents, const float* __restrict__ S_root, float* snap,
    TIn* __restrict__ o, int32_t* __restrict__ status) {
  constexpr int RG = kThreads / CB;  // row groups: thread t owns rows t / CB + RG i
  constexpr int RPT = 128 / RG;      // rows per thread at d_k = 128 (fewer used below that)
  __shared__ float red[RG][CB];
  __shared__ float skq[2][128];
  __shared__ int spar[kMaxNodes];
  __shared__ float sal[kMaxNodes], sbe[kMaxNodes];

  const int tid = threadIdx.x;
  const int nvb = dv / CB;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int vb = bid % nvb;
  const int bh = bid / nvb;
  const int h = bh % H;
  const int b = bh / H;
  const int cl = tid % CB;
  const int c = vb * CB + cl;
  const int rg = tid / CB;
  const bool gdn = mode == kGdn;

  if (tid < N) {
    int p = parents[(size_t)b * N + tid];
    if (p < -1 || p >= tid) p = -1;  // a bad row is flagged below and computed as a forest
    spar[tid] = p;
    sal[tid] = alpha[(size_t)(b * N + tid) * H + h];
    sbe[tid] = gdn ? beta[(size_t)(b * N + tid) * H + h] : 0.f;
  }
  {
    int p = tid < N ? parents[(size_t)b * N + tid] : -1;
    const bool bad = __syncthreads_or(tid < N && (p < -1 || p >= tid)) != 0;
    if (h == 0 && vb == 0 && tid == 0 && status) status[b] = bad ? 1 : 0;
  }

  const float* Sr = S_root + (size_t)bh * dk * dv;
  float* Sb = snap + (size_t)bh * N * dk * dv;
  for (int n = 0; n < N; ++n) {
    const size_t tok = (size_t)(b * N + n) * H + h;
    if (tid < dk) skq[0][tid] = Elem<TIn>::load(k, tok * dk + tid);
    else if (tid < 2 * dk) skq[1][tid - dk] = Elem<TIn>::load(q, tok * dk + tid - dk);
    const float vc = Elem<TIn>::load(v, tok * dv + c);
    __syncthreads();
    const int p = spar[n];
    const float* src = p < 0 ? Sr : Sb + (size_t)p * dk * dv;
    float s[RPT];
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      s[i] = r < dk ? src[(size_t)r * dv + c] : 0.f;
      part = fmaf(r < dk ? skq[0][r] : 0.f, s[i], part);
    }
    const float an = sal[n], bn = sbe[n];
    float ks = 0.f;
    if (gdn) {
      red[rg][cl] = part;
      __syncthreads();
#pragma unroll
      for (int g = 0; g < RG; ++g) ks += red[g][cl];
      __syncthreads();
    }
    float* dst = Sb + (size_t)n * dk * dv;
    float po = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      if (r < dk) {
        const float kr = skq[0][r];
        const float sn = gdn ? an * (s[i] - bn * kr * ks) + bn * kr * vc : an * s[i] + kr * vc;
        dst[(size_t)r * dv + c] = sn;
        po = fmaf(skq[1][r], sn, po);
      }
    }
    red[rg][cl] = po;
    __syncthreads();
    if (rg == 0) {
      float on = 0.f;
#pragma unroll
      for (int g = 0; g < RG; ++g) on += red[g][cl];
      if constexpr (sizeof(TIn) == 2)
        o[tok * dv + c] = f32_to_bf16(on);
      else
        o[tok * dv + c] = on;
    }
    __syncthreads();  // red and skq are reused by the next node
  }
}

// One workgroup per (sequence, head): S_out = snapshot of the accepted node.
// The workgroup of head 0 also writes the path and the status, with the same
// conventions as tree_commit.
template <int DV>
__global__ __launch_bounds__(kThreads) void snapshot_commit_kernel(
    int H, int N, int dk, const float* __restrict__ snap, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ accepted, float* __restrict__ S_out,
    int32_t* __restrict__ path_out, int32_t* __restrict__ status) {
  __shared__ int spar[kMaxNodes];
  __shared__ int pidx[kMaxNodes];
  __shared__ int slen;
  const int tid = threadIdx.x;
  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bh % H;
  const int b = bh / H;
  const int a_in = accepted[b];
  const bool bad_acc = a_in < 0 || a_in >= N;
  const int a = bad_acc ? 0 : a_in;
  const float4* src = reinterpret_cast<const float4*>(snap + ((size_t)bh * N + a) * dk * DV);
  float4* dst = reinterpret_cast<float4*>(S_out + (size_t)bh * dk * DV);
  const int n4 = dk * DV / 4;
  for (int i = tid; i < n4; i += kThreads) dst[i] = src[i];
  if (h != 0) return;  // uniform per workgroup
  const int pv = tid < N ? parents[(size_t)b * N + tid] : -1;
  if (tid < N) spar[tid] = pv;
  const bool bad_par = __syncthreads_or(tid < N && (pv < -1 || pv >= tid)) != 0;
  if (tid == 0) {
    int len = 0;
    if (!bad_par && !bad_acc)
      for (int n = a; n >= 0; n = spar[n]) pidx[len++] = n;
    slen = len;
  }
  __syncthreads();
  const int L = slen;
  if (tid == 0 && status) status[b] = bad_par ? 1 : (bad_acc ? 2 : 0);
  if (path_out && tid < N) path_out[(size_t)b * N + tid] = tid < L ? pidx[L - 1 - tid] : -1;
}

template <typename TIn>
static int snapshot_verify_t(int B, int H, int N, int dk, int dv, int mode, const void* q,
                             const void* k, const void* v, const float* alpha, const float* beta,
                             const int32_t* parents, const float* S_root, float* snap, void* o,
                             int32_t* status, hipStream_t stream) {
  const long long nb = (long long)B * H * (dv >= 32 ? dv / 32 : 1);
  if (nb > 0x7fffffffLL) return static_cast<int>(hipErrorInvalidConfiguration);
  const TIn* qq = static_cast<const TIn*>(q);
  const TIn* kk = static_cast<const TIn*>(k);
  const TIn* vv = static_cast<const TIn*>(v);
  TIn* oo = static_cast<TIn*>(o);
  if (dv >= 32)
    hipLaunchKernelGGL((snapshot_verify_kernel<TIn, 32>), dim3((unsigned)nb), dim3(kThreads), 0,
                       stream, H, N, dk, dv, mode, qq, kk, vv, alpha, beta, parents, S_root, snap,
                       oo, status);
  else
    hipLaunchKernelGGL((snapshot_verify_kernel<TIn, 16>), dim3((unsigned)nb), dim3(kThreads), 0,
                       stream, H, N, dk, dv, mode, qq, kk, vv, alpha, beta, parents, S_root, snap,
                       oo, status);
  return static_cast<int>(hipGetLastError());
}

int launch_snapshot_verify(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                           const void* k, const void* v, const float* alpha, const float* beta,
                           const int32_t* parents, const float* S_root, float* snap, void* o,
                           int32_t* status, hipStream_t stream) {
  if (dtype == 0)
    return snapshot_verify_t<float>(B, H, N, dk, dv, mode, q, k, v, alpha, beta, parents, S_root,
                                    snap, o, status, stream);
  return snapshot_verify_t<uint16_t>(B, H, N, dk, dv, mode, q, k, v, alpha, beta, parents, S_root,
                                     snap, o, status, stream);
}

int launch_snapshot_commit(int B, int H, int N, int dk, int dv, const float* snap,
                           const int32_t* parents, const int32_t* accepted, float* S_out,
                           int32_t* path_out, int32_t* status, hipStream_t stream) {
  const long long nb = (long long)B * H;
  if (nb > 0x7fffffffLL) return static_cast<int>(hipErrorInvalidConfiguration);
  switch (dv) {
#define TV_SNAP_COMMIT(D)                                                                    \
  case D:                                                                                    \
    hipLaunchKernelGGL((snapshot_commit_kernel<D>), dim3((unsigned)nb), dim3(kThreads), 0,   \
                       stream, H, N, dk, snap, parents, accepted, S_out, path_out, status);  \
    break;
    TV_SNAP_COMMIT(16)
    TV_SNAP_COMMIT(32)
    TV_SNAP_COMMIT(64)
    TV_SNAP_COMMIT(128)
#undef TV_SNAP_COMMIT
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace tv
