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
#include <cstdlib>
#include <cstring>
#include <new>
#include <numeric>
#include <system_error>
#include <thread>

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

rs_status on_exception(const char* fn) noexcept {
  rs_status st = RS_ERR_INVALID_ARG;
  const char* what = "unexpected host exception";
  try {
    throw;
  } catch (const std::bad_alloc&) {
    st = RS_ERR_NOMEM;
    what = "out of host memory";
  } catch (const std::system_error&) {
    st = RS_ERR_NOMEM;
    what = "could not start a host thread";
  } catch (...) {
  }
  try {
    g_last_error = std::string(fn) + ": " + what;
  } catch (...) {
    g_last_error.clear();
  }
  return st;
}

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

// Candidates tried in order before the scan goes parallel, and candidates
// per thread in each pass after that.
constexpr int64_t kSequentialCandidates = 4096;
constexpr int64_t kBlockCandidates = 2048;

// Host threads for a long S scan: RS_PLAN_THREADS if set (>= 1), else the
// hardware concurrency, at most 16.
int plan_threads() {
  if (const char* e = std::getenv("RS_PLAN_THREADS")) {
    const int v = std::atoi(e);
    if (v >= 1) return std::min(v, 64);
  }
  const unsigned hc = std::thread::hardware_concurrency();
  return int(std::max(1u, std::min(hc, 16u)));
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

// Minimum S for the items in the given order; offsets written to offs.
rs_status plan_items(const std::vector<PItem>& items, int32_t m, int64_t align, int64_t S_cap,
                     int64_t* offs, int64_t* S_out, int64_t* lb_out) {
  const int32_t n = int32_t(items.size());
  int64_t total = 0, lb = 1;
  for (const PItem& it : items) {
    total += it.E;
    lb = std::max(lb, std::min(it.g, it.E));
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

  *lb_out = lb;
  // First feasible S in [lo, hi] (aligned), or -1; offsets into out.
  auto scan = [&](int64_t lo, int64_t hi, int64_t* out) -> int64_t {
    for (int64_t S = lo; S <= hi;) {
      int64_t next = S + align;
      bool ok = true;
      for (const PItem& it : by_len) {
        if (it.E <= 2 * S) break;
        if (S % it.g) {
          // the aligned S that this tensor rejects run up to the next
          // multiple of lcm(g, align) or to the first S with E <= 2S
          ok = false;
          const int64_t L = std::lcm(it.g, align);
          next = std::max(next, std::min((S / L + 1) * L, round_up((it.E + 1) / 2, align)));
          break;
        }
      }
      if (ok && place_all(items, S, m, align, out)) return S;
      S = next;
    }
    return -1;
  };
  // The first candidates in order; a long scan then goes on in passes of
  // consecutive blocks, one per host thread.  The earliest block with a
  // feasible S holds the smallest one, so the result is the sequential
  // scan's.
  const int64_t head = std::min(cap, lb + kSequentialCandidates * align - align);
  int64_t S = scan(lb, head, offs);
  if (S < 0 && head < cap) {
    const int T = plan_threads();
    const int64_t block = kBlockCandidates * align;
    std::vector<std::vector<int64_t>> outs(T, std::vector<int64_t>(n));
    std::vector<int64_t> found(T);
    for (int64_t base = head + align; base <= cap && S < 0; base += T * block) {
      auto work = [&](int j) {
        const int64_t lo = base + j * block;
        found[j] = lo <= cap ? scan(lo, std::min(cap, lo + block - align), outs[j].data()) : -1;
      };
      if (T == 1) {
        work(0);
      } else {
        std::vector<std::thread> pool;
        int j = 0;
        try {
          for (; j < T; ++j) pool.emplace_back(work, j);
        } catch (const std::system_error&) {  // no more threads: finish inline
          for (; j < T; ++j) work(j);
        }
        for (std::thread& t : pool) t.join();
      }
      for (int j = 0; j < T; ++j)
        if (found[j] >= 0) {
          S = found[j];
          std::copy(outs[j].begin(), outs[j].end(), offs);
          break;
        }
    }
  }
  if (S >= 0) {
    *S_out = S;
    return RS_OK;
  }
  return fail(RS_ERR_INFEASIBLE, "rs_plan: no layout with S <= " + std::to_string(cap));
}

rs_status read_items(const char* fn, const rs_tensor_spec* specs, int32_t n,
                     std::vector<PItem>& items) {
  if (n > kMaxTensors)
    return fail(RS_ERR_INVALID_ARG, std::string(fn) + ": more than 2^20 tensors");
  items.resize(n);
  int64_t total = 0;
  for (int32_t t = 0; t < n; ++t) {
    const rs_tensor_spec& s = specs[t];
    if (!spec_sizes_ok(s))
      return fail(RS_ERR_INVALID_ARG, std::string(fn) + ": tensor " + std::to_string(t) +
                                          " has a bad shape (positive, fewer than 2^40 elements "
                                          "per tensor and granule)");
    items[t].E = s.rows * s.cols;
    items[t].g = s.gran_rows > 0 ? s.gran_rows * s.cols : 1;
    total += items[t].E;
    if (total >= kMaxElems)
      return fail(RS_ERR_INVALID_ARG, std::string(fn) + ": 2^40 or more elements in the group");
  }
  return RS_OK;
}

void fill_info(rs_plan_info* info, const std::vector<PItem>& items, int32_t m, int64_t S,
               int64_t lb, std::chrono::steady_clock::time_point t0) {
  if (!info) return;
  int64_t total = 0;
  for (const PItem& it : items) total += it.E;
  info->S = S;
  info->total = S * m;
  info->numel = total;
  info->pad_elems = S * m - total;
  info->pad_frac = double(S * m - total) / double(total);
  info->lower_bound = lb;
  info->peak_param_bytes = 4 * S + 2 * int64_t(m) * S;
  info->seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
}

// The tensor orders the pages compare (veScale-FSDP, "Planning Algorithm":
// the given order, by block size, by tensor shape).  Stable sorts, so
// tensors with equal keys keep their given order.
void order_perm(const rs_tensor_spec* specs, int32_t n, rs_order kind, int32_t* perm) {
  std::iota(perm, perm + n, 0);
  auto granule = [&](int32_t t) {
    return specs[t].gran_rows > 0 ? specs[t].gran_rows * specs[t].cols : int64_t(1);
  };
  if (kind == RS_ORDER_BLOCK)
    std::stable_sort(perm, perm + n, [&](int32_t a, int32_t b) { return granule(a) > granule(b); });
  else if (kind == RS_ORDER_SHAPE)
    std::stable_sort(perm, perm + n, [&](int32_t a, int32_t b) {
      if (specs[a].rows != specs[b].rows) return specs[a].rows > specs[b].rows;
      return specs[a].cols > specs[b].cols;
    });
}

}  // namespace
}  // namespace rs

extern "C" rs_status rs_plan(const rs_tensor_spec* specs, int32_t n, int32_t m, int64_t align,
                             int64_t S_cap, int64_t* offsets, rs_plan_info* info) try {
  using namespace rs;
  const auto t0 = std::chrono::steady_clock::now();
  if (!specs || !offsets || n <= 0 || m <= 0 || align <= 0)
    return fail(RS_ERR_INVALID_ARG, "rs_plan: null pointer or non-positive n/m/align");
  if (m > kMaxRanks || align > kMaxAlign)
    return fail(RS_ERR_INVALID_ARG, "rs_plan: more than 2^18 ranks or align above 2^20");
  std::vector<PItem> items;
  rs_status st = read_items("rs_plan", specs, n, items);
  if (st != RS_OK) return st;
  std::vector<int64_t> offs(n);
  int64_t S = 0, lb = 0;
  st = plan_items(items, m, align, S_cap, offs.data(), &S, &lb);
  if (st != RS_OK) return st;
  std::copy(offs.begin(), offs.end(), offsets);
  fill_info(info, items, m, S, lb, t0);
  clear_error();
  return RS_OK;
} catch (...) {
  return rs::on_exception("rs_plan");
}

extern "C" rs_status rs_plan_order(const rs_tensor_spec* specs, int32_t n, rs_order kind,
                                   int32_t* perm) try {
  using namespace rs;
  if (!specs || !perm || n <= 0)
    return fail(RS_ERR_INVALID_ARG, "rs_plan_order: null pointer or non-positive n");
  if (kind != RS_ORDER_GIVEN && kind != RS_ORDER_BLOCK && kind != RS_ORDER_SHAPE)
    return fail(RS_ERR_INVALID_ARG, "rs_plan_order: kind must be GIVEN, BLOCK or SHAPE");
  order_perm(specs, n, kind, perm);
  clear_error();
  return RS_OK;
} catch (...) {
  return rs::on_exception("rs_plan_order");
}

extern "C" rs_status rs_plan_ordered(const rs_tensor_spec* specs, int32_t n, int32_t m,
                                     int64_t align, int64_t S_cap, rs_order kind, int32_t* perm,
                                     int64_t* offsets, rs_plan_info* info) try {
  using namespace rs;
  const auto t0 = std::chrono::steady_clock::now();
  if (!specs || !perm || !offsets || n <= 0 || m <= 0 || align <= 0)
    return fail(RS_ERR_INVALID_ARG, "rs_plan_ordered: null pointer or non-positive n/m/align");
  if (m > kMaxRanks || align > kMaxAlign)
    return fail(RS_ERR_INVALID_ARG, "rs_plan_ordered: more than 2^18 ranks or align above 2^20");
  if (kind != RS_ORDER_GIVEN && kind != RS_ORDER_BLOCK && kind != RS_ORDER_SHAPE &&
      kind != RS_ORDER_BEST)
    return fail(RS_ERR_INVALID_ARG, "rs_plan_ordered: unknown order kind");
  std::vector<PItem> items;
  rs_status st = read_items("rs_plan_ordered", specs, n, items);
  if (st != RS_OK) return st;
  const rs_order kinds[3] = {RS_ORDER_GIVEN, RS_ORDER_BLOCK, RS_ORDER_SHAPE};
  int64_t best_S = -1, best_lb = 0;
  std::vector<int32_t> best_perm;
  std::vector<int64_t> best_offs;
  for (rs_order k : kinds) {
    if (kind != RS_ORDER_BEST && k != kind) continue;
    std::vector<int32_t> pm(n);
    order_perm(specs, n, k, pm.data());
    std::vector<PItem> ordered(n);
    for (int32_t i = 0; i < n; ++i) ordered[i] = items[pm[i]];
    std::vector<int64_t> offs(n);
    int64_t S = 0, lb = 0;
    // a later order has to beat the best S so far (ties keep the earlier)
    int64_t cap = S_cap;
    if (best_S > 0) {
      if (best_S - 1 < 1) continue;
      cap = S_cap > 0 ? std::min(S_cap, best_S - 1) : best_S - 1;
    }
    st = plan_items(ordered, m, align, cap, offs.data(), &S, &lb);
    if (st == RS_ERR_INFEASIBLE) continue;
    if (st != RS_OK) return st;
    best_S = S;
    best_lb = lb;
    best_perm = pm;
    best_offs = offs;
  }
  if (best_S < 0)
    return fail(RS_ERR_INFEASIBLE, "rs_plan_ordered: no layout within S_cap");
  for (int32_t i = 0; i < n; ++i) {
    perm[i] = best_perm[i];
    offsets[best_perm[i]] = best_offs[i];
  }
  fill_info(info, items, m, best_S, best_lb, t0);
  clear_error();
  return RS_OK;
} catch (...) {
  return rs::on_exception("rs_plan_ordered");
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
    case RS_ERR_NOMEM: return "out of host resources";
    default: return "unknown status";
  }
}

extern "C" const char* rs_last_error(void) { return rs::g_last_error.c_str(); }
