// Test-only program: the C-ABI used from C++ with no Python in the process.
// Plans a small group, builds and uploads its layout, packs fp32 tensors into
// a bf16 buffer, unpacks them back to fp32, takes the per-tensor squared
// norms of the fp32 tensors packed into an fp32 buffer, scales and adds a
// second buffer into it with found-inf, and quantises it to FP8 and back
// (every decoded value within half a code step of its input), checking all
// of it on the host.  Prints "capi demo ok" and exits 0 on success.
#include <hip/hip_runtime.h>

#include <algorithm>
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
  // y <- 0.5*y + 2*x over every fragment: fl(fl(0.5*y) + fl(2*x)), padding untouched
  std::vector<float> y(size_t(info.total)), x(size_t(info.total));
  HIP_CHECK(hipMemcpy(y.data(), buf32, y.size() * 4, hipMemcpyDeviceToHost));
  for (size_t i = 0; i < x.size(); ++i) x[i] = float(int(i % 17) - 8) * 0.125f;
  void* xdev = nullptr;
  uint32_t* found = nullptr;
  HIP_CHECK(hipMalloc(&xdev, x.size() * 4));
  HIP_CHECK(hipMalloc(&found, size_t(m) * 4));
  HIP_CHECK(hipMemcpy(xdev, x.data(), x.size() * 4, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemset(found, 0, size_t(m) * 4));
  RS_CHECK(rs_group_scale_add(L, static_cast<float*>(buf32), xdev, RS_F32, 0.5f, 2.0f, nullptr,
                              found, 0, m, nullptr));
  std::vector<float> y2(y.size());
  HIP_CHECK(hipDeviceSynchronize());
  HIP_CHECK(hipMemcpy(y2.data(), buf32, y2.size() * 4, hipMemcpyDeviceToHost));
  std::vector<char> in_tensor(y.size(), 0);
  for (int t = 0; t < n; ++t)
    for (int64_t i = 0; i < specs[t].rows * specs[t].cols; ++i) in_tensor[size_t(offs[t] + i)] = 1;
  for (size_t i = 0; i < y.size(); ++i) {
    const volatile float u = 0.5f * y[i];  // volatile: two separate fp32 roundings, no FMA
    const volatile float v = 2.0f * x[i];
    const float e = in_tensor[i] ? float(u + v) : y[i];
    if (std::memcmp(&e, &y2[i], 4) != 0) ++bad;
  }
  std::vector<uint32_t> fh(static_cast<size_t>(m));
  HIP_CHECK(hipMemcpy(fh.data(), found, fh.size() * 4, hipMemcpyDeviceToHost));
  for (uint32_t f : fh) bad += f != 0u;  // every value is finite

  // FP8 quantisation and back: each decoded value within half a code step
  uint8_t* codes = nullptr;
  float* scales = nullptr;
  float* deq = nullptr;
  HIP_CHECK(hipMalloc(&codes, size_t(info.total)));
  HIP_CHECK(hipMalloc(&scales, size_t(info.num_tiles) * 4));
  HIP_CHECK(hipMalloc(&deq, size_t(info.total) * 4));
  RS_CHECK(rs_block_quant(L, static_cast<const float*>(buf32), RS_Q_FP8_E4M3, codes, scales,
                          nullptr, 0, m, nullptr));
  RS_CHECK(rs_block_dequant(L, codes, RS_Q_FP8_E4M3, scales, deq, RS_F32, 0, m, nullptr));
  std::vector<float> d(y.size()), sc(size_t(info.num_tiles));
  HIP_CHECK(hipDeviceSynchronize());
  HIP_CHECK(hipMemcpy(d.data(), deq, d.size() * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(sc.data(), scales, sc.size() * 4, hipMemcpyDeviceToHost));
  int64_t tile = 0;
  for (int t = 0; t < n; ++t) {
    const rs_tensor_spec& s = specs[t];
    if (s.q_rows == 0) continue;
    for (int64_t r0 = 0; r0 < s.rows; r0 += s.q_rows)
      for (int64_t c0 = 0; c0 < s.cols; c0 += s.q_cols, ++tile)
        for (int64_t r = r0; r < std::min(s.rows, r0 + s.q_rows); ++r)
          for (int64_t c = c0; c < std::min(s.cols, c0 + s.q_cols); ++c) {
            const size_t p = size_t(offs[t] + r * s.cols + c);
            const double q = std::fabs(double(y2[p])) / sc[size_t(tile)];
            // E4M3 code spacing at q: 2^(floor(log2 q) - 3) for q >= 2^-6, else 2^-9
            const double step = q < 0x1p-6 ? 0x1p-9 : std::ldexp(1.0, std::ilogb(q) - 3);
            const double tol = sc[size_t(tile)] * (step / 2 + std::ldexp(1.0, std::ilogb(q) - 23)) + 1e-30;
            if (std::fabs(double(d[p]) - double(y2[p])) > tol) ++bad;
          }
  }
  if (tile != info.num_tiles) ++bad;

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
  (void)hipFree(xdev);
  (void)hipFree(found);
  (void)hipFree(codes);
  (void)hipFree(scales);
  (void)hipFree(deq);
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
