// Stand-ins for the kernel launchers behind the C ABI, for a CPU-only build of
// the host checks (tv_api.cpp) under AddressSanitizer and UBSan.  Each records
// that it was reached and returns success; nothing touches a device.
#include "tv_launch.h"

namespace tv {

int g_launches = 0;

int launch_index(int, int, const int32_t*, int32_t*, uint64_t*, int32_t*, hipStream_t) {
  return ++g_launches, 0;
}
int launch_commit(int, int, int, int, int, int, const void*, const float*, const float*,
                  const int32_t*, const int32_t*, const float*, float*, int32_t*, int32_t*,
                  hipStream_t) {
  return ++g_launches, 0;
}
int launch_verify_level(int, int, int, int, int, int, int, const void*, const void*, const void*,
                        const float*, const float*, const int32_t*, const float*, void*, float*,
                        int32_t*, hipStream_t) {
  return ++g_launches, 0;
}
int launch_verify_blocked(int, int, int, int, int, int, int, const void*, const void*, const void*,
                          const float*, const float*, const int32_t*, const float*, void*, float*,
                          int32_t*, hipStream_t) {
  return ++g_launches, 0;
}
int launch_tree_attention(int, int, int, int, int, float, const void*, const void*, const void*,
                          const int32_t*, const void*, const void*, const int32_t*, void*,
                          int32_t*, hipStream_t) {
  return ++g_launches, 0;
}
int launch_verify_mfma(int, int, int, int, const void*, const void*, const void*, const float*,
                       const float*, const int32_t*, const float*, void*, float*, int32_t*,
                       hipStream_t, const PrevCommit*) {
  return ++g_launches, 0;
}
int launch_snapshot_verify(int, int, int, int, int, int, int, const void*, const void*,
                           const void*, const float*, const float*, const int32_t*, const float*,
                           float*, void*, int32_t*, hipStream_t) {
  return ++g_launches, 0;
}
int launch_snapshot_commit(int, int, int, int, int, const float*, const int32_t*, const int32_t*,
                           float*, int32_t*, int32_t*, hipStream_t) {
  return ++g_launches, 0;
}

}  // namespace tv
