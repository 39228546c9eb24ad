// Generic tree verification: any d_k, d_v in {16, 32, 64, 128}, fp32 or bf16
// q/k/v, any tree of up to 128 nodes.  Plain fp32 FMA, one workgroup per
// (sequence, head, block of value columns); the triangular solve runs one
// depth level per step (level_solve in tv_device.h).
#include "tv_device.h"
#include "tv_launch.h"

namespace tv {

template <typename TIn>
__global__ __launch_bounds__(kThreads) void verify_level_kernel(
    int H, int N, int dk, int dv, int mode, int cb, const TIn* __restrict__ q,
    const TIn* __restrict__ k, const TIn* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const int32_t* __restrict__ parents,
    const float* __restrict__ S_root, TIn* __restrict__ o, float* __restrict__ U,
    int32_t* __restrict__ status) {
  __shared__ TreeLds t;
  __shared__ LevelLds s;
  const int nvb = dv / cb;
  const int bid = xcd_group(blockIdx.x, gridDim.x, nvb);
  const int vb = bid % nvb;
  const int bh = bid / nvb;
  const int h = bh % H;
  const int b = bh / H;
  build_tree(t, parents + (size_t)b * N, N);
  if (h == 0 && vb == 0 && threadIdx.x == 0 && status) status[b] = t.bad ? 1 : 0;
  level_solve<TIn>(t, s, mode, b, h, H, N, dk, dv, vb * cb, vb * cb + cb, q, k, v, alpha, beta,
                   S_root, o, U);
}

int launch_verify_level(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                        const void* k, const void* v, const float* alpha, const float* beta,
                        const int32_t* parents, const float* S_root, void* o, float* U,
                        int32_t* status, hipStream_t stream) {
  const int cb = dv > 32 ? 32 : dv;
  const long long nblocks = (long long)B * H * (dv / cb);
  if (nblocks > 0x7fffffffLL) return static_cast<int>(hipErrorInvalidConfiguration);
  if (dtype == 0) {
    hipLaunchKernelGGL(verify_level_kernel<float>, dim3((unsigned)nblocks), dim3(kThreads), 0,
                       stream, H, N, dk, dv, mode, cb, static_cast<const float*>(q),
                       static_cast<const float*>(k), static_cast<const float*>(v), alpha, beta,
                       parents, S_root, static_cast<float*>(o), U, status);
  } else {
    hipLaunchKernelGGL(verify_level_kernel<uint16_t>, dim3((unsigned)nblocks), dim3(kThreads), 0,
                       stream, H, N, dk, dv, mode, cb, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), alpha,
                       beta, parents, S_root, static_cast<uint16_t*>(o), U, status);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace tv
