// Test-only program: the C-ABI used from C++ with no Python in the process.
// Plans a small group, builds and uploads its layout, packs fp32 tensors into
// a bf16 buffer, unpacks them back to fp32, takes the per-tensor squared
// norms of the fp32 tensors packed into an fp32 buffer, and checks all of it
// on the host.  Prints "capi demo ok" and exits 0 on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "rs.h"

namespace {

int fail_rs(const char* what, rs_status st) {
  std::printf("%s failed: %s (%s)\n", what, rs_status_str(st), rs_last_error());
  return 1;
}

int fail_hip(const char* what, hipError_t e) {
  std::printf("%s failed: %s\n", what, hipGetErrorString(e));
  return 1;
}

// fp32 -> bf16 -> fp32, round to nearest even (finite inputs)
float bf16_round(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  u &= 0xffff0000u;
  float r;
  std::memcpy(&r, &u, 4);
  return r;
}

}  // namespace

#define RS_CHECK(call)                          \
  do {                                          \
    const rs_status st_ = (call);               \
    if (st_ != RS_OK) return fail_rs(#call, st_); \
  } while (0)
#define HIP_CHECK(call)                            \
  do {                                             \
    const hipError_t e_ = (call);                  \
    if (e_ != hipSuccess) return fail_hip(#call, e_); \
  } while (0)

int main() {
  // rows, cols, granule rows, quantisation tile
  const rs_tensor_spec specs[] = {{64, 32, 8, 8, 32}, {1, 100, 0, 0, 0}, {40, 16, 4, 4, 16}};
  const int32_t n = 3, m = 4;
  int64_t offs[n];
  rs_plan_info plan;
  RS_CHECK(rs_plan(specs, n, m, 16, 0, offs, &plan));
  rs_layout* L = nullptr;
  RS_CHECK(rs_layout_create(specs, n, m, plan.S, offs, 0, &L));
  rs_layout_info info;
  RS_CHECK(rs_layout_get_info(L, &info));
  void* table = nullptr;
  void* ws = nullptr;
  HIP_CHECK(hipMalloc(&table, size_t(info.device_bytes)));
  HIP_CHECK(hipMalloc(&ws, size_t(info.workspace_bytes)));
  HIP_CHECK(hipMemset(ws, 0, size_t(info.workspace_bytes)));
  RS_CHECK(rs_layout_upload(L, table, nullptr));

  std::vector<std::vector<float>> host(n);
  std::vector<void*> src(n), dst(n);
  uint32_t state = 12345u;
  for (int t = 0; t < n; ++t) {
    host[t].resize(size_t(specs[t].rows * specs[t].cols));
    for (float& v : host[t]) {
      state = state * 1664525u + 1013904223u;
      v = float(int32_t(state >> 8) - (1 << 23)) / float(1 << 23);
    }
    HIP_CHECK(hipMalloc(&src[t], host[t].size() * 4));
    HIP_CHECK(hipMalloc(&dst[t], host[t].size() * 4));
    HIP_CHECK(hipMemcpy(src[t], host[t].data(), host[t].size() * 4, hipMemcpyHostToDevice));
  }
  void** dsrc = nullptr;
  void** ddst = nullptr;
  HIP_CHECK(hipMalloc(&dsrc, n * sizeof(void*)));
  HIP_CHECK(hipMalloc(&ddst, n * sizeof(void*)));
  HIP_CHECK(hipMemcpy(dsrc, src.data(), n * sizeof(void*), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(ddst, dst.data(), n * sizeof(void*), hipMemcpyHostToDevice));
  void* buf16 = nullptr;
  void* buf32 = nullptr;
  double* sq = nullptr;
  HIP_CHECK(hipMalloc(&buf16, size_t(info.total) * 2));
  HIP_CHECK(hipMalloc(&buf32, size_t(info.total) * 4));
  HIP_CHECK(hipMalloc(&sq, n * sizeof(double)));

  RS_CHECK(rs_pack(L, dsrc, RS_F32, buf16, RS_BF16, 0, m, nullptr));
  RS_CHECK(rs_unpack(L, buf16, RS_BF16, ddst, RS_F32, 0, m, nullptr));
  RS_CHECK(rs_pack(L, dsrc, RS_F32, buf32, RS_F32, 0, m, nullptr));
  RS_CHECK(rs_ragged_sqnorm(L, static_cast<const float*>(buf32), sq, nullptr, nullptr, ws, 0, m,
                            nullptr));
  HIP_CHECK(hipDeviceSynchronize());

  int bad = 0;
  for (int t = 0; t < n; ++t) {
    std::vector<float> got(host[t].size());
    HIP_CHECK(hipMemcpy(got.data(), dst[t], got.size() * 4, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < got.size(); ++i)
      if (got[i] != bf16_round(host[t][i])) ++bad;
  }
  std::vector<double> gsq(n);
  HIP_CHECK(hipMemcpy(gsq.data(), sq, n * sizeof(double), hipMemcpyDeviceToHost));
  for (int t = 0; t < n; ++t) {
    double e = 0.0;
    for (float v : host[t]) e += double(v) * double(v);
    if (std::fabs(gsq[t] - e) > 1e-9 * e) ++bad;
  }
  // an invalid call reports its error and launches nothing
  if (rs_pack(L, dsrc, RS_F32, buf16, RS_BF16, 2, 1, nullptr) != RS_ERR_RANGE) ++bad;

  for (int t = 0; t < n; ++t) {
    (void)hipFree(src[t]);
    (void)hipFree(dst[t]);
  }
  (void)hipFree(dsrc);
  (void)hipFree(ddst);
  (void)hipFree(buf16);
  (void)hipFree(buf32);
  (void)hipFree(sq);
  (void)hipFree(ws);
  (void)hipFree(table);
  rs_layout_destroy(L);
  if (bad) {
    std::printf("capi demo: %d mismatches (S=%lld)\n", bad, static_cast<long long>(plan.S));
    return 1;
  }
  std::printf("capi demo ok (S=%lld, %d tensors, %d ranks)\n", static_cast<long long>(plan.S), n, m);
  return 0;
}
