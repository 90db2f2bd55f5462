// Layout planner for a RaggedShard tensor group (host only).
//
// Minimises the per-rank buffer size S of m equal shards holding the group's
// tensors in order, such that no granule is cut by a shard boundary, each
// tensor's memory is contiguous and padding sits only between tensors
// (veScale-FSDP: Flexible and High-Performance FSDP at Scale, "Planning
// Algorithm", formulation under Figure 6 and Figure 6(b)).
//
// The pages solve it with a DP over three cases: a tensor inside one shard,
// across adjacent shards without containing one, or containing whole
// shards.  With the tensor order fixed the problem is exact by scanning S:
// for one S, the placement of a tensor is valid or not independently of the
// others, so placing each tensor at its earliest valid offset is optimal
// (an earlier end never removes a choice for the next tensor).  The same
// three cases appear in the per-rank step below.
#include <algorithm>
#include <chrono>
#include <cstring>
#include <numeric>

#include "rs_internal.h"

namespace rs {

namespace {
thread_local std::string g_last_error;
}

rs_status fail(rs_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

void clear_error() { g_last_error.clear(); }

namespace {

struct PItem {
  int64_t E;  // elements
  int64_t g;  // granule
};

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Earliest offset >= lo at which a tensor (E, g) is valid for shard size S,
// or -1.  Works one start rank at a time:
//  * the tensor ends before the next boundary b: valid;
//  * it crosses b and also b + S: every boundary it holds must be a whole
//    number of granules in, which needs S % g == 0; if not, nothing left in
//    this rank is valid, so move to b;
//  * otherwise (b - l) must be a multiple of lcm(g, A): take the next such l
//    below b, or move to b if there is none.
int64_t earliest(int64_t lo, const PItem& it, int64_t S, int32_t m, int64_t A) {
  const int64_t L = std::lcm(it.g, A);
  const int64_t end = S * m;
  int64_t l = round_up(lo, A);
  while (l + it.E <= end) {
    const int64_t b = (l / S + 1) * S;  // first boundary above l
    if (l + it.E <= b) return l;
    const bool holds_shard = l + it.E > b + S;
    if (holds_shard && S % it.g != 0) {
      l = b;
      continue;
    }
    const int64_t d = b - l;      // > 0
    const int64_t r = d % L;      // distance to the next position aligned to b
    if (r == 0) return l;         // aligned; with holds_shard, S % g == 0
    if (l + r >= b) {
      l = b;
      continue;
    }
    l += r;
  }
  return -1;
}

bool place_all(const std::vector<PItem>& items, int64_t S, int32_t m, int64_t A, int64_t* offs) {
  int64_t prev = 0;
  for (size_t t = 0; t < items.size(); ++t) {
    const int64_t l = earliest(prev, items[t], S, m, A);
    if (l < 0) return false;
    offs[t] = l;
    prev = l + items[t].E;
  }
  return true;
}

}  // namespace
}  // namespace rs

extern "C" rs_status rs_plan(const rs_tensor_spec* specs, int32_t n, int32_t m, int64_t align,
                             int64_t S_cap, int64_t* offsets, rs_plan_info* info) {
  using namespace rs;
  const auto t0 = std::chrono::steady_clock::now();
  if (!specs || !offsets || n <= 0 || m <= 0 || align <= 0)
    return fail(RS_ERR_INVALID_ARG, "rs_plan: null pointer or non-positive n/m/align");
  std::vector<PItem> items(n);
  int64_t total = 0, lb = 1;
  for (int32_t t = 0; t < n; ++t) {
    const rs_tensor_spec& s = specs[t];
    if (s.rows <= 0 || s.cols <= 0 || s.gran_rows < 0)
      return fail(RS_ERR_INVALID_ARG, "rs_plan: tensor " + std::to_string(t) + " has a bad shape");
    items[t].E = s.rows * s.cols;
    items[t].g = s.gran_rows > 0 ? s.gran_rows * s.cols : 1;
    total += items[t].E;
    lb = std::max(lb, std::min(items[t].g, items[t].E));
  }
  lb = std::max(lb, (total + m - 1) / m);
  lb = round_up(lb, align);
  // S large enough to hold every tensor back to back in rank 0 always works
  const int64_t hard_cap = round_up(total, align) + int64_t(n) * align;
  const int64_t cap = S_cap > 0 ? std::min(S_cap, hard_cap) : hard_cap;

  // A tensor longer than 2S holds two boundaries S apart, so S must be a
  // multiple of its granule: skip such S without placing anything.
  std::vector<PItem> by_len(items);
  std::sort(by_len.begin(), by_len.end(), [](const PItem& a, const PItem& b) { return a.E > b.E; });

  std::vector<int64_t> offs(n);
  int64_t found = -1;
  for (int64_t S = lb; S <= cap; S += align) {
    bool ok = true;
    for (const PItem& it : by_len) {
      if (it.E <= 2 * S) break;
      if (S % it.g) { ok = false; break; }
    }
    if (ok && place_all(items, S, m, align, offs.data())) {
      found = S;
      break;
    }
  }
  if (found < 0)
    return fail(RS_ERR_INFEASIBLE, "rs_plan: no layout with S <= " + std::to_string(cap));
  std::copy(offs.begin(), offs.end(), offsets);
  if (info) {
    info->S = found;
    info->total = found * m;
    info->numel = total;
    info->pad_elems = found * m - total;
    info->pad_frac = double(found * m - total) / double(total);
    info->lower_bound = lb;
    info->peak_param_bytes = 4 * found + 2 * int64_t(m) * found;
    info->seconds =
        std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  }
  clear_error();
  return RS_OK;
}

extern "C" const char* rs_status_str(rs_status st) {
  switch (st) {
    case RS_OK: return "ok";
    case RS_ERR_INVALID_ARG: return "invalid argument";
    case RS_ERR_DTYPE: return "unsupported dtype";
    case RS_ERR_ALIGN: return "misaligned pointer";
    case RS_ERR_INFEASIBLE: return "no feasible layout";
    case RS_ERR_RANGE: return "rank range out of bounds";
    case RS_ERR_HIP: return "HIP runtime error";
    case RS_ERR_STATE: return "layout not uploaded";
    default: return "unknown status";
  }
}

extern "C" const char* rs_last_error(void) { return rs::g_last_error.c_str(); }
