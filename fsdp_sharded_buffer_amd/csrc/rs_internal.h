// Internal types shared by the planner, the layout builder and the kernels.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "rs.h"

namespace rs {

// One work chunk: a run of buffer positions inside one rank that is either
// part of one tensor or padding.  Chunks partition the whole buffer in
// buffer order, so a rank range maps to one contiguous run of chunks.
struct ChunkDesc {
  int64_t buf_off;  // first buffer position
  int64_t ten_off;  // first tensor element, -1 for padding
  int32_t len;      // elements
  int32_t tensor;   // -1 for padding
  int32_t rank;
  int32_t frag;     // fragment index, -1 for padding
};
static_assert(sizeof(ChunkDesc) == 32, "ChunkDesc layout");

// A tensor-rank intersection; its chunks are [chunk_begin, chunk_end) in
// the fine chunk table and [cchunk_begin, cchunk_end) in the coarse one.
struct FragDesc {
  int32_t tensor;
  int32_t rank;
  int32_t chunk_begin;
  int32_t chunk_end;
  int32_t cchunk_begin;
  int32_t cchunk_end;
  int32_t pad0, pad1;
};
static_assert(sizeof(FragDesc) == 32, "FragDesc layout");

// Per tensor: its fragments (all ranks) are [frag_begin, frag_end) and the
// ranks it touches are [rank_lo, rank_hi).
struct TensorDesc {
  int32_t frag_begin;
  int32_t frag_end;
  int32_t rank_lo;
  int32_t rank_hi;
};
static_assert(sizeof(TensorDesc) == 16, "TensorDesc layout");

// One quantisation tile: rows x cols elements at buffer position buf_off
// with row stride ld; its scale goes to scales[scale_idx].
// One workgroup of the tile kernels (quantise, dequantise, 8-bit Adam): a
// run of `count` consecutive tiles of one tensor in row-major tile order,
// all in one rank and with the same team size and vector flag.  Tile j of
// the run is tile (t0 + j) of the tensor; lanes [j*team, (j+1)*team) take
// it.  Kernels derive each tile's place and shape from these fields, so no
// per-tile table is read.
struct QuantWork {
  int64_t base;            // buffer offset of the tensor
  int32_t t0;              // first tile (row-major index within the tensor)
  int32_t count;           // tiles in the run (<= 256 / team)
  int32_t team;            // lanes per tile
  int32_t vec;             // 1: every tile of the run allows 16-byte access
  int32_t rows, cols;      // tensor shape; cols is the leading dimension
  int32_t q_rows, q_cols;  // tile shape (edge tiles are clipped)
  int32_t ntc;             // tiles per tile row
  int32_t scale0;          // scale index of tile t0
  int32_t rank;            // rank holding the run
  int32_t pad[3];
};
static_assert(sizeof(QuantWork) == 64, "QuantWork layout");

constexpr int kMaxTileElems = 16384;  // 256 lanes x 64 elements held in registers

// Tiles of at most kNarrowTileElems elements are "narrow": a team of at most
// 256 lanes holds one with at most kNarrowSlots four-element slots per lane.
// Wider tiles take 256 lanes with up to kWideSlots slots per lane.  The tile
// kernels are compiled for each class, so narrow tiles carry no registers or
// loop iterations for slots they never have.
constexpr int kNarrowTileElems = 4096;
constexpr int kNarrowSlots = 4;
constexpr int kWideSlots = kMaxTileElems / 4 / 256;

// Size limits that keep every product and sum of sizes inside int64: fewer
// than 2^40 elements per tensor, per granule and per group, at most 2^20
// tensors, 2^18 ranks and an alignment of 2^20 elements.  Then S <= 2^41
// and m*S <= 2^59.
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int32_t kMaxTensors = 1 << 20;
constexpr int32_t kMaxRanks = 1 << 18;
constexpr int64_t kMaxAlign = int64_t(1) << 20;

inline bool spec_sizes_ok(const rs_tensor_spec& s) {
  return s.rows > 0 && s.cols > 0 && s.gran_rows >= 0 && s.rows < kMaxElems / s.cols &&
         s.gran_rows < kMaxElems / s.cols;
}
#ifndef RS_DEFAULT_CHUNK
#define RS_DEFAULT_CHUNK 2048
#endif
#ifndef RS_COARSE_FACTOR
#define RS_COARSE_FACTOR 32
#endif
constexpr int64_t kDefaultChunk = RS_DEFAULT_CHUNK;   // fine chunk
constexpr int64_t kCoarseFactor = RS_COARSE_FACTOR;   // coarse chunk = factor x fine

}  // namespace rs

struct rs_layout {
  int32_t n = 0, m = 0;
  int64_t S = 0;
  std::vector<rs_tensor_spec> specs;
  std::vector<int64_t> offsets;
  int64_t chunk_elems = 0;

  std::vector<rs::TensorDesc> tensors;
  std::vector<rs::FragDesc> frags;
  std::vector<rs::ChunkDesc> chunks;   // fine chunks (copies, scale/add)
  std::vector<rs::ChunkDesc> cchunks;  // coarse chunks (norms, masked zero)
  int64_t num_tiles = 0;
  std::vector<rs::QuantWork> work;

  // per-rank begin indices, size m + 1
  std::vector<int64_t> rank_chunk, rank_cchunk, rank_frag;
  // The work table holds the narrow tiles' items (class 0), then the wide
  // tiles' items (class 1), each list in buffer order.  rank_work[c][k] is
  // rank k's first item of class c as an index into the whole table, and
  // rank_work[c][m] ends the list.
  std::vector<int64_t> rank_work[2];
  std::vector<int32_t> rank_min_tile_rows[2];  // per class and rank; INT32_MAX without tiles
  // per class: the median, over the class's tiles, of the width (columns)
  // of the tensor a tile belongs to; 0 without tiles
  int64_t median_tile_tensor_cols[2] = {0, 0};

  // byte offsets of each table inside the device blob
  size_t off_tensors = 0, off_frags = 0, off_chunks = 0, off_cchunks = 0,
         off_work = 0;
  size_t device_bytes = 0;
  size_t workspace_bytes = 0;

  // device copy (caller-owned), set by rs_layout_upload
  void* dev = nullptr;
};

namespace rs {
// Records a message for rs_last_error() and returns `st`.
rs_status fail(rs_status st, const std::string& msg);
void clear_error();
// Maps the exception in flight to a status for a C entry point (called from
// its catch block): std::bad_alloc and thread start failures give
// RS_ERR_NOMEM, anything else RS_ERR_INVALID_ARG; records the message.
rs_status on_exception(const char* fn) noexcept;
}  // namespace rs
