// Test-only program: random and hostile inputs to rs_plan, rs_plan_ordered
// and rs_layout_create, built with AddressSanitizer and UndefinedBehavior-
// Sanitizer on the host (no GPU call is made).  Checks that every accepted
// plan builds a layout of m*S positions and that the best order is never
// worse than the given one; prints "fuzz ok" and exits 0 on success.
#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>
#include "rs.h"

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  std::mt19937_64 rng(12345);
  auto U = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); };
  int ok = 0, rej = 0;
  for (int it = 0; it < iters; ++it) {
    const int n = int(U(1, 8));
    std::vector<rs_tensor_spec> sp(n);
    const bool hostile = U(0, 9) == 0;
    for (auto& s : sp) {
      if (hostile) {
        const int64_t big[] = {-1, 0, 1, 3, 1LL << 20, 1LL << 31, 1LL << 40, 1LL << 62, INT64_MAX};
        s.rows = big[U(0, 8)]; s.cols = big[U(0, 8)]; s.gran_rows = big[U(0, 8)];
        s.q_rows = int32_t(U(-2, 300)); s.q_cols = int32_t(U(-2, 300));
      } else {
        s.rows = U(1, 300); s.cols = U(1, 300);
        const int kind = int(U(0, 3));
        s.gran_rows = kind == 0 ? 0 : U(1, 40);
        if (kind >= 2 && s.gran_rows * s.cols <= 16384) { s.q_rows = int32_t(s.gran_rows); s.q_cols = int32_t(U(1, s.cols)); }
        else { s.q_rows = 0; s.q_cols = 0; }
        if (int64_t(s.q_rows) * s.q_cols > 16384) { s.q_rows = 0; s.q_cols = 0; }
      }
    }
    const int32_t m = hostile ? int32_t(U(-1, 300000)) : int32_t(U(1, 70));
    const int64_t align = hostile ? U(-1, 1 << 21) : (int64_t[]){1, 4, 16, 64}[U(0, 3)];
    std::vector<int64_t> offs(n);
    rs_plan_info info;
    if (rs_plan(sp.data(), n, m, align, hostile ? U(0, 100) : 0, offs.data(), &info) != RS_OK) { ++rej; continue; }
    std::vector<int32_t> perm(n);
    std::vector<int64_t> offs2(n);
    rs_plan_info info2;
    if (rs_plan_ordered(sp.data(), n, m, align, 0, RS_ORDER_BEST, perm.data(), offs2.data(), &info2) != RS_OK) {
      std::printf("ordered failed after plan ok: %s\n", rs_last_error()); return 1;
    }
    if (info2.S > info.S) { std::printf("best worse than given\n"); return 1; }
    rs_layout* L = nullptr;
    const int64_t chunk = (int64_t[]){0, 64, 128, 4096}[U(0, 3)];
    const rs_status st = rs_layout_create(sp.data(), n, m, info.S, offs.data(), chunk, &L);
    if (st == RS_OK) {
      rs_layout_info li;
      rs_layout_get_info(L, &li);
      if (li.total != int64_t(m) * info.S) { std::printf("total mismatch\n"); return 1; }
      rs_layout_destroy(L);
      ++ok;
    } else {
      ++rej;  // e.g. a tile crossing a shard boundary
    }
    // corrupt an offset: must be rejected or accepted without memory errors
    offs[U(0, n - 1)] += U(-5, 5);
    if (rs_layout_create(sp.data(), n, m, info.S, offs.data(), chunk, &L) == RS_OK) rs_layout_destroy(L);
  }
  // A layout inside the size limits whose chunk table could not be indexed
  // (2^42 positions in 2048-element chunks) is refused before any table is
  // built, with a status rather than an exception.
  {
    rs_tensor_spec one{1, 4, 0, 0, 0};
    const int64_t off = 0;
    rs_layout* L = nullptr;
    const rs_status st = rs_layout_create(&one, 1, 4, int64_t(1) << 40, &off, 0, &L);
    if (st != RS_ERR_INVALID_ARG || L != nullptr) {
      std::printf("large S: status %d (%s)\n", int(st), rs_last_error()); return 1;
    }
    if (rs_layout_create(&one, 1, 4, int64_t(1) << 40, &off, 1 << 22, &L) != RS_OK) {
      std::printf("large S with 2^22-element chunks refused: %s\n", rs_last_error()); return 1;
    }
    rs_layout_destroy(L);
  }
  std::printf("fuzz ok: %d layouts built, %d rejected\n", ok, rej);
  return 0;
}
