// Layout validation and descriptor tables (host side).
//
// The tables are the device-resident group description every grouped kernel
// reads, so one launch covers a whole tensor group (veScale-FSDP: Flexible
// and High-Performance FSDP at Scale, "DBuffer": group-level operators and a
// persistent mapping from each tensor to its place in the buffer).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "rs_internal.h"

using namespace rs;

namespace {

int64_t granule_of(const rs_tensor_spec& s) { return s.gran_rows > 0 ? s.gran_rows * s.cols : 1; }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Lanes per tile: a narrow tile takes the smallest power of two from 8
// lanes up that holds it at 16 elements (4 slots) per lane; a wide tile
// takes 256 lanes (up to 64 elements each).
int team_for(int64_t elems) {
  if (elems > kNarrowTileElems) return 256;
  int team = 8;
  while (team < 256 && int64_t(team) * 4 * kNarrowSlots < elems) team *= 2;
  return team;
}

// Splits the buffer into chunks of at most CH positions that never cross a
// rank, tensor or padding boundary, in buffer order.  Records each rank's
// first chunk in rank_begin and, when set_frags, creates the fragments;
// otherwise fills the fragments' coarse chunk ranges.
void build_chunks(rs_layout* L, int64_t CH, std::vector<ChunkDesc>& out,
                  std::vector<int64_t>& rank_begin, bool set_frags) {
  const int32_t n = L->n, m = L->m;
  const int64_t S = L->S;
  out.clear();
  rank_begin.assign(m + 1, 0);
  auto add = [&](int64_t lo, int64_t hi, int32_t tensor, int64_t ten_lo, int32_t rank,
                 int32_t frag) {
    for (int64_t p = lo; p < hi; p += CH) {
      ChunkDesc c;
      c.buf_off = p;
      c.ten_off = tensor >= 0 ? ten_lo + (p - lo) : -1;
      c.len = int32_t(std::min(CH, hi - p));
      c.tensor = tensor;
      c.rank = rank;
      c.frag = frag;
      out.push_back(c);
    }
  };
  int32_t t_first = 0, f = 0;
  for (int32_t k = 0; k < m; ++k) {
    const int64_t rlo = int64_t(k) * S, rhi = rlo + S;
    rank_begin[k] = int64_t(out.size());
    if (set_frags) L->rank_frag[k] = int64_t(L->frags.size());
    int64_t pos = rlo;
    while (t_first < n &&
           L->offsets[t_first] + L->specs[t_first].rows * L->specs[t_first].cols <= rlo)
      ++t_first;
    for (int32_t t = t_first; t < n; ++t) {
      const int64_t l = L->offsets[t];
      const int64_t r = l + L->specs[t].rows * L->specs[t].cols;
      if (l >= rhi) break;
      const int64_t lo = std::max(l, rlo), hi = std::min(r, rhi);
      if (lo >= hi) continue;
      if (lo > pos) add(pos, lo, -1, -1, k, -1);
      if (set_frags) {
        FragDesc fd{};
        fd.tensor = t;
        fd.rank = k;
        fd.chunk_begin = int32_t(out.size());
        add(lo, hi, t, lo - l, k, f);
        fd.chunk_end = int32_t(out.size());
        L->frags.push_back(fd);
      } else {
        L->frags[f].cchunk_begin = int32_t(out.size());
        add(lo, hi, t, lo - l, k, f);
        L->frags[f].cchunk_end = int32_t(out.size());
      }
      ++f;
      pos = hi;
    }
    if (pos < rhi) add(pos, rhi, -1, -1, k, -1);
  }
  rank_begin[m] = int64_t(out.size());
  if (set_frags) L->rank_frag[m] = int64_t(L->frags.size());
}

rs_status build(rs_layout* L) {
  const int32_t n = L->n, m = L->m;
  const int64_t S = L->S;
  L->tensors.assign(n, TensorDesc{});
  L->frags.clear();
  L->work.clear();
  L->num_tiles = 0;
  L->rank_frag.assign(m + 1, 0);
  for (int c = 0; c < 2; ++c) {
    L->rank_work[c].assign(m + 1, 0);
    L->rank_min_tile_rows[c].assign(m, INT32_MAX);
  }

  // Chunk indices are int32 in the device tables.  The fine table holds at
  // most ceil(m*S / chunk) chunks plus one partial chunk per run, and the
  // runs (fragments and padding gaps) number at most 2(n + m); refuse before
  // building rather than after.
  const int64_t max_chunks = (int64_t(m) * S + L->chunk_elems - 1) / L->chunk_elems + 2 * (int64_t(n) + m);
  if (max_chunks > int64_t(INT32_MAX))
    return fail(RS_ERR_INVALID_ARG,
                "rs_layout_create: more than 2^31 work chunks (m*S / chunk_elems); raise chunk_elems");
  build_chunks(L, L->chunk_elems, L->chunks, L->rank_chunk, true);
  build_chunks(L, L->chunk_elems * kCoarseFactor, L->cchunks, L->rank_cchunk, false);
  if (L->chunks.size() > size_t(INT32_MAX) || L->frags.size() > size_t(INT32_MAX))
    return fail(RS_ERR_INVALID_ARG, "rs_layout_create: too many chunks; raise chunk_elems");

  // tensor -> fragment range and rank range
  for (int32_t t = 0; t < n; ++t) {
    L->tensors[t].frag_begin = -1;
  }
  for (int32_t f = 0; f < int32_t(L->frags.size()); ++f) {
    TensorDesc& td = L->tensors[L->frags[f].tensor];
    if (td.frag_begin < 0) {
      td.frag_begin = f;
      td.rank_lo = L->frags[f].rank;
    }
    td.frag_end = f + 1;
    td.rank_hi = L->frags[f].rank + 1;
  }

  // quantisation tiles, tensor by tensor, row-major (ranks are
  // non-decreasing in this order because tensors and tile rows are), cut
  // into runs of consecutive tiles of one tensor and rank with the same
  // class, team size and vector flag; each class keeps its own list
  int64_t scale_idx = 0;
  bool open = false;
  int cur_cls = 0;
  QuantWork cur{};
  std::vector<QuantWork> lists[2];
  std::vector<std::pair<int64_t, int64_t>> widths[2];  // (tensor cols, tiles) per class
  for (int32_t t = 0; t < n; ++t) {
    const rs_tensor_spec& s = L->specs[t];
    if (s.q_rows <= 0) continue;
    const int64_t l = L->offsets[t];
    const int64_t ntr = (s.rows + s.q_rows - 1) / s.q_rows, ntc = (s.cols + s.q_cols - 1) / s.q_cols;
    for (int64_t tr = 0; tr < ntr; ++tr) {
      const int64_t r0 = tr * s.q_rows, rows = std::min<int64_t>(s.q_rows, s.rows - r0);
      for (int64_t tc = 0; tc < ntc; ++tc) {
        const int64_t c0 = tc * s.q_cols, cols = std::min<int64_t>(s.q_cols, s.cols - c0);
        const int64_t first = l + r0 * s.cols + c0, last = l + (r0 + rows - 1) * s.cols + c0 + cols - 1;
        if (last / S != first / S)
          return fail(RS_ERR_INVALID_ARG,
                      "rs_layout_create: a quantisation tile of tensor " + std::to_string(t) +
                          " crosses a shard boundary");
        const int32_t rank = int32_t(first / S);
        const int cls = rows * cols > kNarrowTileElems ? 1 : 0;
        const int32_t team = team_for(rows * cols);
        const int32_t vec = (cols % 4 == 0 && s.cols % 4 == 0 && first % 4 == 0) ? 1 : 0;
        const int64_t idx = tr * ntc + tc;
        if (scale_idx >= INT32_MAX)
          return fail(RS_ERR_INVALID_ARG, "rs_layout_create: more than 2^31 quantisation tiles");
        L->rank_min_tile_rows[cls][rank] =
            std::min(L->rank_min_tile_rows[cls][rank], int32_t(rows));
        if (widths[cls].empty() || widths[cls].back().first != s.cols)
          widths[cls].push_back({s.cols, 0});
        ++widths[cls].back().second;
        if (open && cur_cls == cls && cur.rank == rank && cur.team == team && cur.vec == vec &&
            cur.count < 256 / team && cur.base == l && int64_t(cur.t0) + cur.count == idx) {
          ++cur.count;
        } else {
          if (open) lists[cur_cls].push_back(cur);
          cur_cls = cls;
          cur = QuantWork{};
          cur.base = l;
          cur.t0 = int32_t(idx);
          cur.count = 1;
          cur.team = team;
          cur.vec = vec;
          cur.rows = int32_t(s.rows);
          cur.cols = int32_t(s.cols);
          cur.q_rows = s.q_rows;
          cur.q_cols = s.q_cols;
          cur.ntc = int32_t(ntc);
          cur.scale0 = int32_t(scale_idx);
          cur.rank = rank;
          open = true;
        }
        ++scale_idx;
      }
    }
  }
  if (open) lists[cur_cls].push_back(cur);
  L->num_tiles = scale_idx;
  for (int c = 0; c < 2; ++c) {  // tile-weighted median tensor width of the class
    std::sort(widths[c].begin(), widths[c].end());
    int64_t total = 0, seen = 0;
    for (const auto& w : widths[c]) total += w.second;
    L->median_tile_tensor_cols[c] = 0;
    for (const auto& w : widths[c]) {
      seen += w.second;
      if (2 * seen >= total) {
        L->median_tile_tensor_cols[c] = w.first;
        break;
      }
    }
  }
  // the narrow list, then the wide list; each rank's first item of each
  for (int c = 0; c < 2; ++c) {
    const int64_t base = int64_t(L->work.size());
    size_t i = 0;
    for (int32_t k = 0; k <= m; ++k) {
      while (i < lists[c].size() && lists[c][i].rank < k) ++i;
      L->rank_work[c][k] = base + int64_t(i);
    }
    L->work.insert(L->work.end(), lists[c].begin(), lists[c].end());
  }

  size_t off = 0;
  L->off_tensors = off;
  off = align256(off + sizeof(TensorDesc) * L->tensors.size());
  L->off_frags = off;
  off = align256(off + sizeof(FragDesc) * L->frags.size());
  L->off_chunks = off;
  off = align256(off + sizeof(ChunkDesc) * L->chunks.size());
  L->off_cchunks = off;
  off = align256(off + sizeof(ChunkDesc) * L->cchunks.size());
  L->off_work = off;
  off = align256(off + sizeof(QuantWork) * L->work.size());
  L->device_bytes = std::max<size_t>(off, 256);
  // sqnorm scratch: one fp64 partial per chunk of the finer table (small
  // rank ranges read fine chunks)
  L->workspace_bytes =
      align256(sizeof(double) * std::max<size_t>({L->chunks.size(), L->cchunks.size(), size_t(1)}));
  return RS_OK;
}

}  // namespace

extern "C" rs_status rs_layout_create(const rs_tensor_spec* specs, int32_t n, int32_t m, int64_t S,
                                      const int64_t* offsets, int64_t chunk_elems,
                                      rs_layout** out) try {
  if (!specs || !offsets || !out || n <= 0 || m <= 0 || S <= 0)
    return fail(RS_ERR_INVALID_ARG, "rs_layout_create: null pointer or non-positive n/m/S");
  if (n > kMaxTensors || m > kMaxRanks || S > 2 * kMaxElems)
    return fail(RS_ERR_INVALID_ARG,
                "rs_layout_create: more than 2^20 tensors or 2^18 ranks, or S above 2^41");
  if (chunk_elems == 0) chunk_elems = kDefaultChunk;
  if (chunk_elems < 64 || chunk_elems % 64 || chunk_elems > (int64_t(1) << 22))
    return fail(RS_ERR_INVALID_ARG, "rs_layout_create: chunk_elems must be a multiple of 64");
  int64_t prev_end = 0;
  for (int32_t t = 0; t < n; ++t) {
    const rs_tensor_spec& s = specs[t];
    const std::string name = "tensor " + std::to_string(t);
    if (!spec_sizes_ok(s))
      return fail(RS_ERR_INVALID_ARG, "rs_layout_create: " + name +
                                          " has a bad shape (positive, fewer than 2^40 elements "
                                          "per tensor and granule)");
    if ((s.q_rows > 0) != (s.q_cols > 0) || s.q_rows < 0 || s.q_cols < 0 ||
        int64_t(s.q_rows) * s.q_cols > kMaxTileElems ||
        int64_t(s.q_rows) * s.cols > int64_t(INT32_MAX) ||
        (s.q_rows > 0 && (s.rows > INT32_MAX || s.cols > INT32_MAX ||
                          ((s.rows + s.q_rows - 1) / s.q_rows) * ((s.cols + s.q_cols - 1) / s.q_cols) >
                              int64_t(INT32_MAX))))
      return fail(RS_ERR_INVALID_ARG, "rs_layout_create: " + name +
                                          " has a bad quantisation tile (at most 16384 elements, q_rows * cols < 2^31, "
                                          "fewer than 2^31 rows, columns and tiles)");
    const int64_t l = offsets[t], E = s.rows * s.cols, g = granule_of(s);
    if (l < prev_end)
      return fail(RS_ERR_INVALID_ARG, "rs_layout_create: " + name + " overlaps the previous tensor");
    if (l > S * m - E)
      return fail(RS_ERR_INVALID_ARG, "rs_layout_create: " + name + " ends past the buffer");
    for (int64_t b = (l / S + 1) * S; b < l + E; b += S)
      if ((b - l) % g)
        return fail(RS_ERR_INVALID_ARG,
                    "rs_layout_create: " + name + " has a granule cut by a shard boundary");
    prev_end = l + E;
  }
  rs_layout* L = new rs_layout;
  L->n = n;
  L->m = m;
  L->S = S;
  L->specs.assign(specs, specs + n);
  L->offsets.assign(offsets, offsets + n);
  L->chunk_elems = chunk_elems;
  rs_status st = build(L);
  if (st != RS_OK) {
    delete L;
    return st;
  }
  *out = L;
  clear_error();
  return RS_OK;
} catch (...) {
  return rs::on_exception("rs_layout_create");
}

extern "C" rs_status rs_layout_get_info(const rs_layout* L, rs_layout_info* info) try {
  if (!L || !info) return fail(RS_ERR_INVALID_ARG, "rs_layout_get_info: null pointer");
  info->n = L->n;
  info->m = L->m;
  info->S = L->S;
  info->total = L->S * L->m;
  info->num_chunks = int64_t(L->chunks.size());
  info->num_coarse_chunks = int64_t(L->cchunks.size());
  info->num_frags = int64_t(L->frags.size());
  info->num_tiles = L->num_tiles;
  info->chunk_elems = L->chunk_elems;
  info->device_bytes = int64_t(L->device_bytes);
  info->workspace_bytes = int64_t(L->workspace_bytes);
  return RS_OK;
} catch (...) {
  return rs::on_exception("rs_layout_get_info");
}

extern "C" size_t rs_layout_device_bytes(const rs_layout* L) { return L ? L->device_bytes : 0; }

extern "C" size_t rs_workspace_bytes(const rs_layout* L) { return L ? L->workspace_bytes : 0; }

extern "C" rs_status rs_layout_upload(rs_layout* L, void* dev_table, void* stream) try {
  if (!L || !dev_table) return fail(RS_ERR_INVALID_ARG, "rs_layout_upload: null pointer");
  if (reinterpret_cast<uintptr_t>(dev_table) % 256)
    return fail(RS_ERR_ALIGN, "rs_layout_upload: dev_table must be 256-byte aligned");
  std::vector<unsigned char> blob(L->device_bytes, 0);
  auto put = [&](size_t off, const void* p, size_t bytes) {
    if (bytes) std::memcpy(blob.data() + off, p, bytes);
  };
  put(L->off_tensors, L->tensors.data(), sizeof(TensorDesc) * L->tensors.size());
  put(L->off_frags, L->frags.data(), sizeof(FragDesc) * L->frags.size());
  put(L->off_chunks, L->chunks.data(), sizeof(ChunkDesc) * L->chunks.size());
  put(L->off_cchunks, L->cchunks.data(), sizeof(ChunkDesc) * L->cchunks.size());
  put(L->off_work, L->work.data(), sizeof(QuantWork) * L->work.size());
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dev_table, blob.data(), blob.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess)
    return fail(RS_ERR_HIP, std::string("rs_layout_upload: ") + hipGetErrorString(e));
  L->dev = dev_table;
  clear_error();
  return RS_OK;
} catch (...) {
  return rs::on_exception("rs_layout_upload");
}

extern "C" void rs_layout_destroy(rs_layout* L) { delete L; }
