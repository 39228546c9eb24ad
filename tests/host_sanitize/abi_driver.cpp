// Drives every C-ABI entry point of the host shim with good and bad arguments.
// Built with the stub launchers and -fsanitize=address,undefined; prints one
// line per failed expectation and exits non-zero if there was any.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tree_verify.h"

namespace tv {
extern int g_launches;
}

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      printf("FAIL line %d: %s\n", __LINE__, #cond);                   \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

// rc expected, and whether a launcher may be reached
static void check(int rc, int want, int launches_before) {
  EXPECT(rc == want);
  if (want != TV_OK) EXPECT(tv::g_launches == launches_before);
  else EXPECT(tv::g_launches > launches_before);
}

int main() {
  // fake, never dereferenced device addresses (the launchers are stubs)
  static char arena[1 << 16];
  void* P = arena;
  void* Q = arena + 4096;
  float* S = reinterpret_cast<float*>(arena + 8192);
  float* S2 = reinterpret_cast<float*>(arena + 8192 + 64);  // overlaps S partly
  int32_t* I = reinterpret_cast<int32_t*>(arena + 32768);
  int n;

  // tree_verify / tree_verify_algo
  n = tv::g_launches;
  check(tree_verify(2, 3, 7, 16, 16, TV_F32, TV_GDN, P, P, P, S, S, I, S, P, S, I, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_verify(2, 3, 7, 16, 16, TV_F32, TV_GDN, nullptr, P, P, S, S, I, S, P, S, I, nullptr), TV_ERR_NULL, n);
  n = tv::g_launches;
  check(tree_verify(0, 3, 7, 16, 16, TV_F32, TV_GDN, P, P, P, S, S, I, S, P, S, I, nullptr), TV_ERR_DIMS, n);
  n = tv::g_launches;
  check(tree_verify(1, 1, TV_MAX_NODES + 1, 16, 16, TV_F32, TV_GDN, P, P, P, S, S, I, S, P, S, I, nullptr), TV_ERR_DIMS, n);
  n = tv::g_launches;
  check(tree_verify(1, 1, 4, 24, 16, TV_F32, TV_GDN, P, P, P, S, S, I, S, P, S, I, nullptr), TV_ERR_HEAD_DIM, n);
  n = tv::g_launches;
  check(tree_verify(1, 1, 4, 16, 16, 7, TV_GDN, P, P, P, S, S, I, S, P, S, I, nullptr), TV_ERR_MODE, n);
  n = tv::g_launches;
  check(tree_verify(1, 1, 4, 16, 16, TV_F32, TV_GDN, P, P, P, S, nullptr, I, S, P, S, I, nullptr), TV_ERR_MODE, n);
  n = tv::g_launches;
  check(tree_verify(1, 1, 4, 16, 16, TV_F32, TV_SCALAR_DECAY, P, P, P, S, nullptr, I, S, P, S, I, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_verify(0x7fffffff, 0x7fffffff, 128, 128, 128, TV_BF16, TV_GDN, P, P, P, S, S, I, S, P, S, I, nullptr), TV_ERR_DIMS, n);
  n = tv::g_launches;
  check(tree_verify_algo(1, 1, 4, 16, 16, TV_F32, TV_GDN, P, P, P, S, S, I, S, P, S, I, TV_ALGO_MFMA, nullptr), TV_ERR_ALGO, n);
  n = tv::g_launches;
  check(tree_verify_algo(1, 1, 4, 128, 128, TV_BF16, TV_GDN, P, P, P, S, S, I, S, P, S, I, TV_ALGO_MFMA, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_verify_algo(1, 1, 200, 16, 16, TV_F32, TV_GDN, P, P, P, S, S, I, S, P, S, I, TV_ALGO_LEVEL, nullptr), TV_ERR_ALGO, n);
  n = tv::g_launches;
  check(tree_verify_algo(1, 1, 200, 16, 16, TV_F32, TV_GDN, P, P, P, S, S, I, S, P, S, I, TV_ALGO_AUTO, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_verify_algo(1, 1, 4, 16, 16, TV_F32, TV_GDN, P, P, P, S, S, I, S, P, S, I, 9, nullptr), TV_ERR_ALGO, n);

  // tree_commit: in place allowed, partial overlap refused
  n = tv::g_launches;
  check(tree_commit(1, 1, 4, 16, 16, TV_F32, P, S, S, I, I, S, S, I, I, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_commit(1, 1, 4, 16, 16, TV_F32, P, S, S, I, I, S, S2, I, I, nullptr), TV_ERR_ALIAS, n);
  n = tv::g_launches;
  check(tree_commit(1, 1, 4, 16, 16, TV_F32, P, S, S, I, nullptr, S, S, I, I, nullptr), TV_ERR_NULL, n);
  n = tv::g_launches;
  check(tree_commit(1, 1, 4, 16, 16, TV_F32, P, S, S, I, I, S, S, nullptr, nullptr, nullptr), TV_OK, n);

  // tree_index
  n = tv::g_launches;
  check(tree_index(3, 9, I, I, reinterpret_cast<uint64_t*>(P), nullptr, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_index(3, 0, I, I, reinterpret_cast<uint64_t*>(P), nullptr, nullptr), TV_ERR_DIMS, n);
  n = tv::g_launches;
  check(tree_index(3, 9, nullptr, I, reinterpret_cast<uint64_t*>(P), nullptr, nullptr), TV_ERR_NULL, n);

  // snapshot pair
  n = tv::g_launches;
  check(tree_verify_snapshot(1, 1, 4, 16, 16, TV_F32, TV_GDN, P, P, P, S, S, I, S, S, P, I, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_verify_snapshot(1, 1, 129, 16, 16, TV_F32, TV_GDN, P, P, P, S, S, I, S, S, P, I, nullptr), TV_ERR_DIMS, n);
  n = tv::g_launches;
  check(tree_commit_snapshot(1, 1, 4, 16, 16, S, I, I, reinterpret_cast<float*>(Q), I, I, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_commit_snapshot(1, 1, 4, 16, 16, S, I, I, S2, I, I, nullptr), TV_ERR_ALIAS, n);

  // tree_commit_verify: U overlapping U_prev refused; fused and unfused shapes launch
  float* U0 = reinterpret_cast<float*>(arena + 40960);
  float* U1 = reinterpret_cast<float*>(arena + 49152);
  n = tv::g_launches;
  check(tree_commit_verify(1, 1, 4, 4, 16, 16, TV_F32, TV_GDN, P, S, U0, I, I, S, S, I, I, P, P, P, S,
                           S, I, P, U1, I, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_commit_verify(1, 1, 4, 4, 16, 16, TV_F32, TV_GDN, P, S, U0, I, I, S, S, I, I, P, P, P, S,
                           S, I, P, U0, I, nullptr), TV_ERR_ALIAS, n);
  n = tv::g_launches;
  check(tree_commit_verify(1, 1, 4, 4, 128, 128, TV_BF16, TV_GDN, P, S, U0, I, I, S, S, I, I, P, P, P,
                           S, S, I, P, U1, I, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_commit_verify(1, 1, 4, 4, 16, 16, TV_F32, TV_GDN, P, S, U0, I, I, S, S2, I, I, P, P, P, S,
                           S, I, P, U1, I, nullptr), TV_ERR_ALIAS, n);

  // tree_attention
  n = tv::g_launches;
  check(tree_attention(2, 5, 8, 2, 128, 64, TV_BF16, P, P, P, I, P, P, I, 0.1f, P, I, nullptr), TV_OK, n);
  n = tv::g_launches;
  check(tree_attention(2, 5, 8, 3, 128, 64, TV_BF16, P, P, P, I, P, P, I, 0.1f, P, I, nullptr), TV_ERR_DIMS, n);
  n = tv::g_launches;
  check(tree_attention(2, 5, 8, 2, 64, 64, TV_BF16, P, P, P, I, P, P, I, 0.1f, P, I, nullptr), TV_ERR_HEAD_DIM, n);
  n = tv::g_launches;
  check(tree_attention(2, 5, 8, 2, 128, 64, TV_F32, P, P, P, I, P, P, I, 0.1f, P, I, nullptr), TV_ERR_MODE, n);
  n = tv::g_launches;
  check(tree_attention(2, 5, 8, 2, 128, 64, TV_BF16, P, nullptr, P, I, P, P, I, 0.1f, P, I, nullptr), TV_ERR_NULL, n);
  n = tv::g_launches;
  check(tree_attention(2, 5, 8, 2, 128, 0, TV_BF16, P, nullptr, nullptr, I, P, P, I, 0.1f, P, I, nullptr), TV_OK, n);

  // strings for every code, never NULL
  for (int c = -120; c <= 5; ++c) EXPECT(tv_status_string(c) != nullptr && strlen(tv_status_string(c)) > 0);
  EXPECT(tv_version() == 100);

  printf("%s: %d failure(s), %d launches reached\n", failures ? "FAILED" : "ok", failures, tv::g_launches);
  return failures ? 1 : 0;
}
