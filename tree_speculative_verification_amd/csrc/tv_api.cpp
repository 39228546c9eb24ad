// Host side of the C ABI: argument checks, solver choice, launch.  Nothing is
// launched unless every check passes; see include/tree_verify.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tree_verify.h"
#include "tv_launch.h"

namespace {

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Elements of the largest array stay well inside size_t and the device's
// 64-bit addressing.
bool sizes_ok(long long B, long long H, long long N, long long dk, long long dv) {
  const long long big = 1LL << 40;
  // one sequence's q, k or v rows (N H d elements of at most 4 bytes) stay
  // addressable with 32-bit byte offsets, as the kernels address them
  const long long d = dk > dv ? dk : dv;
  return B <= big / H && B * H <= big / N && B * H * N <= big / d &&
         B * H <= big / (dk * dv) && N * H * d * 4 <= 0xffffffffLL;
}

// The snapshot buffer (B H N d_k d_v floats) stays below 2^46 bytes.
bool snapshot_size_ok(long long B, long long H, long long N, long long dk, long long dv) {
  const long long big = 1LL << 44;
  return B * H <= big / N && B * H * N <= big / (dk * dv);
}

int hip_code(int err) { return err == 0 ? TV_OK : TV_ERR_HIP_BASE - err; }

// Trees the register-path (matrix-core) and level-scheduled kernels take; the
// blocked kernel takes every tree up to TV_MAX_NODES.
constexpr int kSmallTree = 128;

// Solver for tree_verify_algo's TV_ALGO_AUTO, or TV_ERR_ALGO for a choice that
// does not apply to these arguments.
int pick_algo(int algo, int N, int dk, int dv, int dtype) {
  const bool mfma_ok = dtype == TV_BF16 && dk == 128 && dv == 128 && N <= kSmallTree;
  if (algo == TV_ALGO_AUTO) return N > kSmallTree ? TV_ALGO_BLOCKED : (mfma_ok ? TV_ALGO_MFMA : TV_ALGO_LEVEL);
  if (algo == TV_ALGO_MFMA) return mfma_ok ? algo : TV_ERR_ALGO;
  if (algo == TV_ALGO_LEVEL) return N <= kSmallTree ? algo : TV_ERR_ALGO;
  if (algo == TV_ALGO_BLOCKED) return algo;
  return TV_ERR_ALGO;
}

int launch_algo(int algo, int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                const void* k, const void* v, const float* alpha, const float* beta,
                const int32_t* parents, const float* S_root, void* o, float* U, int32_t* status,
                hipStream_t st) {
  if (algo == TV_ALGO_MFMA)
    return tv::launch_verify_mfma(B, H, N, mode, q, k, v, alpha, beta, parents, S_root, o, U,
                                  status, st);
  if (algo == TV_ALGO_BLOCKED)
    return tv::launch_verify_blocked(B, H, N, dk, dv, dtype, mode, q, k, v, alpha, beta, parents,
                                     S_root, o, U, status, st);
  return tv::launch_verify_level(B, H, N, dk, dv, dtype, mode, q, k, v, alpha, beta, parents,
                                 S_root, o, U, status, st);
}

int check_common(int B, int H, int N, int dk, int dv, int dtype) {
  if (B <= 0 || H <= 0 || N <= 0 || N > TV_MAX_NODES) return TV_ERR_DIMS;
  if (!head_dim_ok(dk) || !head_dim_ok(dv)) return TV_ERR_HEAD_DIM;
  if (!sizes_ok(B, H, N, dk, dv)) return TV_ERR_DIMS;
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_MODE;
  return TV_OK;
}

}  // namespace

extern "C" {

int tree_verify_algo(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                     const void* k, const void* v, const float* alpha, const float* beta,
                     const int32_t* parents, const float* S_root, void* o, float* U,
                     int32_t* status, int algo, void* stream) {
  if (!q || !k || !v || !alpha || !parents || !S_root || !o || !U) return TV_ERR_NULL;
  int rc = check_common(B, H, N, dk, dv, dtype);
  if (rc) return rc;
  if (mode != TV_GDN && mode != TV_SCALAR_DECAY) return TV_ERR_MODE;
  if (mode == TV_GDN && !beta) return TV_ERR_MODE;
  algo = pick_algo(algo, N, dk, dv, dtype);
  if (algo < 0) return algo;
  return hip_code(launch_algo(algo, B, H, N, dk, dv, dtype, mode, q, k, v, alpha, beta, parents,
                              S_root, o, U, status, static_cast<hipStream_t>(stream)));
}

int tree_verify(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                const void* k, const void* v, const float* alpha, const float* beta,
                const int32_t* parents, const float* S_root, void* o, float* U, int32_t* status,
                void* stream) {
  return tree_verify_algo(B, H, N, dk, dv, dtype, mode, q, k, v, alpha, beta, parents, S_root, o,
                          U, status, TV_ALGO_AUTO, stream);
}

int tree_commit(int B, int H, int N, int dk, int dv, int dtype, const void* k, const float* alpha,
                const float* U, const int32_t* parents, const int32_t* accepted,
                const float* S_root, float* S_out, int32_t* path_out, int32_t* status,
                void* stream) {
  if (!k || !alpha || !U || !parents || !accepted || !S_root || !S_out) return TV_ERR_NULL;
  int rc = check_common(B, H, N, dk, dv, dtype);
  if (rc) return rc;
  const uintptr_t bytes = (uintptr_t)B * H * dk * dv * sizeof(float);
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(S_root), b0 = reinterpret_cast<uintptr_t>(S_out);
  if (a0 != b0 && a0 < b0 + bytes && b0 < a0 + bytes) return TV_ERR_ALIAS;
  return hip_code(tv::launch_commit(B, H, N, dk, dv, dtype, k, alpha, U, parents, accepted, S_root,
                                    S_out, path_out, status, static_cast<hipStream_t>(stream)));
}

int tree_index(int B, int N, const int32_t* parents, int32_t* depth, uint64_t* anc,
               int32_t* status, void* stream) {
  if (!parents || !depth || !anc) return TV_ERR_NULL;
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES || B > (1 << 30)) return TV_ERR_DIMS;
  return hip_code(tv::launch_index(B, N, parents, depth, anc, status, static_cast<hipStream_t>(stream)));
}

int tree_verify_snapshot(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta,
                         const int32_t* parents, const float* S_root, float* snapshots, void* o,
                         int32_t* status, void* stream) {
  if (!q || !k || !v || !alpha || !parents || !S_root || !snapshots || !o) return TV_ERR_NULL;
  int rc = check_common(B, H, N, dk, dv, dtype);
  if (rc) return rc;
  if (mode != TV_GDN && mode != TV_SCALAR_DECAY) return TV_ERR_MODE;
  if (mode == TV_GDN && !beta) return TV_ERR_MODE;
  if (N > kSmallTree || !snapshot_size_ok(B, H, N, dk, dv)) return TV_ERR_DIMS;
  return hip_code(tv::launch_snapshot_verify(B, H, N, dk, dv, dtype, mode, q, k, v, alpha, beta,
                                             parents, S_root, snapshots, o, status,
                                             static_cast<hipStream_t>(stream)));
}

int tree_commit_snapshot(int B, int H, int N, int dk, int dv, const float* snapshots,
                         const int32_t* parents, const int32_t* accepted, float* S_out,
                         int32_t* path_out, int32_t* status, void* stream) {
  if (!snapshots || !parents || !accepted || !S_out) return TV_ERR_NULL;
  int rc = check_common(B, H, N, dk, dv, TV_F32);
  if (rc) return rc;
  if (N > kSmallTree || !snapshot_size_ok(B, H, N, dk, dv)) return TV_ERR_DIMS;
  const uintptr_t sb = reinterpret_cast<uintptr_t>(snapshots);
  const uintptr_t se = sb + (uintptr_t)B * H * N * dk * dv * sizeof(float);
  const uintptr_t ob = reinterpret_cast<uintptr_t>(S_out);
  const uintptr_t oe = ob + (uintptr_t)B * H * dk * dv * sizeof(float);
  if (ob < se && sb < oe) return TV_ERR_ALIAS;
  return hip_code(tv::launch_snapshot_commit(B, H, N, dk, dv, snapshots, parents, accepted, S_out,
                                             path_out, status, static_cast<hipStream_t>(stream)));
}

int tree_commit_verify(int B, int H, int N_prev, int N, int dk, int dv, int dtype, int mode,
                       const void* k_prev, const float* alpha_prev, const float* U_prev,
                       const int32_t* parents_prev, const int32_t* accepted_prev,
                       const float* S_in, float* S_out, int32_t* path_out, int32_t* commit_status,
                       const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, const int32_t* parents, void* o, float* U,
                       int32_t* status, void* stream) {
  if (!k_prev || !alpha_prev || !U_prev || !parents_prev || !accepted_prev || !S_in || !S_out ||
      !q || !k || !v || !alpha || !parents || !o || !U)
    return TV_ERR_NULL;
  int rc = check_common(B, H, N, dk, dv, dtype);
  if (rc) return rc;
  rc = check_common(B, H, N_prev, dk, dv, dtype);
  if (rc) return rc;
  if (mode != TV_GDN && mode != TV_SCALAR_DECAY) return TV_ERR_MODE;
  if (mode == TV_GDN && !beta) return TV_ERR_MODE;
  const uintptr_t sbytes = (uintptr_t)B * H * dk * dv * sizeof(float);
  const uintptr_t si = reinterpret_cast<uintptr_t>(S_in), so = reinterpret_cast<uintptr_t>(S_out);
  if (si != so && si < so + sbytes && so < si + sbytes) return TV_ERR_ALIAS;
  // U_prev is read while U is written
  const uintptr_t up = reinterpret_cast<uintptr_t>(U_prev), un = reinterpret_cast<uintptr_t>(U);
  const uintptr_t upb = (uintptr_t)B * H * N_prev * dv * sizeof(float);
  const uintptr_t unb = (uintptr_t)B * H * N * dv * sizeof(float);
  if (up < un + unb && un < up + upb) return TV_ERR_ALIAS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == TV_BF16 && dk == 128 && dv == 128 && N <= kSmallTree && N_prev <= kSmallTree) {
    tv::PrevCommit pc;
    pc.N = N_prev;
    pc.k = static_cast<const uint16_t*>(k_prev);
    pc.alpha = alpha_prev;
    pc.U = U_prev;
    pc.parents = parents_prev;
    pc.accepted = accepted_prev;
    pc.S_out = S_out;
    pc.path_out = path_out;
    pc.status = commit_status;
    return hip_code(tv::launch_verify_mfma(B, H, N, mode, q, k, v, alpha, beta, parents, S_in, o, U,
                                           status, st, &pc));
  }
  // other shapes and trees: the two kernels in stream order
  int err = tv::launch_commit(B, H, N_prev, dk, dv, dtype, k_prev, alpha_prev, U_prev, parents_prev,
                              accepted_prev, S_in, S_out, path_out, commit_status, st);
  if (err) return hip_code(err);
  return hip_code(launch_algo(pick_algo(TV_ALGO_AUTO, N, dk, dv, dtype), B, H, N, dk, dv, dtype,
                              mode, q, k, v, alpha, beta, parents, S_out, o, U, status, st));
}

int tree_attention(int B, int N, int Hq, int Hkv, int D, int P_max, int dtype, const void* q,
                   const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                   const void* k_tree, const void* v_tree, const int32_t* parents, float scale,
                   void* o, int32_t* status, void* stream) {
  if (!q || !prefix_len || !k_tree || !v_tree || !parents || !o) return TV_ERR_NULL;
  if (P_max > 0 && (!k_cache || !v_cache)) return TV_ERR_NULL;
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES || Hq <= 0 || Hkv <= 0 || Hq % Hkv || P_max < 0)
    return TV_ERR_DIMS;
  if (D != 128) return TV_ERR_HEAD_DIM;
  if (dtype != TV_BF16) return TV_ERR_MODE;
  const long long big = 1LL << 40;
  if ((long long)B * N > big / ((long long)Hq * D) || (long long)B * Hkv > big / ((long long)(P_max + 1) * D))
    return TV_ERR_DIMS;
  return hip_code(tv::launch_tree_attention(B, N, Hq, Hkv, P_max, scale, q, k_cache, v_cache,
                                            prefix_len, k_tree, v_tree, parents, o, status,
                                            static_cast<hipStream_t>(stream)));
}

const char* tv_status_string(int code) {
  switch (code) {
    case TV_OK: return "ok";
    case TV_STATUS_BAD_PARENTS: return "status: a parent index is outside [-1, i-1]";
    case TV_STATUS_BAD_ACCEPTED: return "status: accepted node index is outside [0, N)";
    case TV_STATUS_BAD_PREFIX_LEN: return "status: prefix_len is outside [0, P_max] (clamped)";
    case TV_ERR_NULL: return "a required pointer is NULL";
    case TV_ERR_DIMS: return "bad sizes: B, H, N must be positive, N <= 512 (128 for the snapshot baseline), sizes must fit";
    case TV_ERR_HEAD_DIM: return "d_k and d_v must be 16, 32, 64 or 128";
    case TV_ERR_MODE: return "bad dtype or mode, or beta is NULL in gated-delta-rule mode";
    case TV_ERR_ALIAS: return "an output overlaps an input it may not overlap (S_out == S_root in place is allowed)";
    case TV_ERR_ALGO: return "bad solver choice for these arguments";
  }
  if (code <= TV_ERR_HIP_BASE) return "HIP launch failed (code = -(100 + hipError_t))";
  return "unknown code";
}

int tv_version(void) { return 100; }

}  // extern "C"
