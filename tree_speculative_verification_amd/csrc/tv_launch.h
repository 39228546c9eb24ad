// Internal launchers behind the C ABI.  Each returns a hipError_t value (0 on
// success); argument checking happens in tv_api.cpp before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tv {

int launch_index(int B, int N, const int32_t* parents, int32_t* depth, uint64_t* anc,
                 int32_t* status, hipStream_t stream);

int launch_commit(int B, int H, int N, int dk, int dv, int dtype, const void* k, const float* alpha,
                  const float* U, const int32_t* parents, const int32_t* accepted,
                  const float* S_root, float* S_out, int32_t* path_out, int32_t* status,
                  hipStream_t stream);

int launch_verify_level(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                        const void* k, const void* v, const float* alpha, const float* beta,
                        const int32_t* parents, const float* S_root, void* o, float* U,
                        int32_t* status, hipStream_t stream);

// Blocked solve for trees of up to 512 nodes and any depth (tv_verify_blocked.hip).
int launch_verify_blocked(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                          const void* k, const void* v, const float* alpha, const float* beta,
                          const int32_t* parents, const float* S_root, void* o, float* U,
                          int32_t* status, hipStream_t stream);

// Tree-masked attention (tv_attention.hip): bf16, head dim 128.
int launch_tree_attention(int B, int N, int Hq, int Hkv, int P_max, float scale, const void* q,
                          const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                          const void* k_tree, const void* v_tree, const int32_t* parents, void* o,
                          int32_t* status, hipStream_t stream);

// The previous step's commit, applied to the state on the fly by the fused
// verification (arrays as tree_commit takes them, N = the previous tree's size).
struct PrevCommit {
  int N;
  const uint16_t* k;         // [B, N, H, 128] bf16
  const float* alpha;        // [B, N, H]
  const float* U;            // [B, H, N, 128]
  const int32_t* parents;    // [B, N]
  const int32_t* accepted;   // [B]
  float* S_out;              // [B, H, 128, 128] committed state (may be the input state)
  int32_t* path_out;         // [B, N] or null
  int32_t* status;           // [B] or null
};

// bf16 q/k/v, d_k = d_v = 128 only.  With `prev` the state read is first
// advanced by the previous step's commit, which is also written to
// prev->S_out (S_root may equal prev->S_out).
int launch_verify_mfma(int B, int H, int N, int mode, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const int32_t* parents,
                       const float* S_root, void* o, float* U, int32_t* status,
                       hipStream_t stream, const PrevCommit* prev = nullptr);

// Per-node-snapshot baseline (tv_snapshot.hip).
int launch_snapshot_verify(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                           const void* k, const void* v, const float* alpha, const float* beta,
                           const int32_t* parents, const float* S_root, float* snap, void* o,
                           int32_t* status, hipStream_t stream);
int launch_snapshot_commit(int B, int H, int N, int dk, int dv, const float* snap,
                           const int32_t* parents, const int32_t* accepted, float* S_out,
                           int32_t* path_out, int32_t* status, hipStream_t stream);

}  // namespace tv
