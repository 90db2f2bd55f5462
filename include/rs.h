/*
 * rs.h - RaggedShard flat communication buffer: planner and grouped
 * memory-bound operations for AMD Instinct MI355X (gfx950).
 *
 * Terms.  A group of n row-major tensors (one FSDP unit) is laid out in one
 * flat buffer of m*S elements split into m equal shards; virtual rank k owns
 * buffer positions [k*S, (k+1)*S).  Tensor t occupies [l_t, l_t + E_t).  A
 * fragment is the part of one tensor inside one rank.  On one GPU the m
 * ranks are slices of one device buffer; each operation takes a rank range
 * [k0, k1) and touches only positions inside [k0*S, k1*S), i.e. the shards
 * those ranks would own (veScale-FSDP: Flexible and High-Performance FSDP
 * at Scale, section "Planning Algorithm", the layout formulation under
 * Figure 6).
 *
 * Memory and streams.  The caller owns every buffer.  Pointers marked
 * "device" are HIP device pointers; "host" are host pointers.  `stream` is a
 * hipStream_t passed as void* (NULL = the null stream).  Hot calls (rs_pack
 * ... rs_block_quant) only enqueue kernels on `stream`: they never allocate,
 * copy from the host or synchronise, and return before the work is done.
 *
 * Limits.  Fewer than 2^40 elements per tensor, per granule and per group;
 * at most 2^20 tensors, 2^18 ranks and an alignment of 2^20 elements; S at
 * most 2^41.  Calls outside them return RS_ERR_INVALID_ARG.
 *
 * Launches.  A call enqueues one kernel (the norms: two; the tile
 * operations: one per tile class present).  A range with more workgroups
 * than one launch may hold (2^31 lanes) is covered by several launches of
 * the same kernel on `stream`, in order.
 *
 * Concurrency.  A call reads and writes only its rank range (and the
 * found_inf flags of those ranks), so calls over disjoint rank ranges may
 * run at the same time on different streams.  rs_ragged_sqnorm is the
 * exception: it writes sq[t] for every tensor, so calls that overlap in time
 * need separate sq arrays as well as separate workspaces.
 *
 * Aliasing.  Outputs must not overlap inputs or other outputs, except where a
 * call says so (rs_group_scale_add: x may be y).
 *
 * Errors.  Every call returns an rs_status.  On a non-zero status from
 * argument checking nothing was enqueued, no output was touched, and
 * rs_last_error() returns a message for the calling thread.  RS_ERR_HIP
 * reports a launch that failed (that launch's own hipLaunchKernel status,
 * not an error left by earlier work); launches of the same call before the
 * failed one stay enqueued.  RS_ERR_NOMEM reports a host allocation or host
 * thread that failed in a set-up call; no C++ exception leaves the library.
 *
 * Alignment.  Kernels use 128-bit accesses where a fragment's buffer and
 * tensor addresses are 16-byte aligned, and element accesses elsewhere, so
 * any element-aligned pointer is accepted; plan with align >= 16 and
 * 16-byte-aligned tensors for full speed.
 */
#ifndef RS_H
#define RS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t rs_status;
enum {
  RS_OK = 0,
  RS_ERR_INVALID_ARG = -1, /* null pointer, bad count, bad shape */
  RS_ERR_DTYPE = -2,       /* dtype not supported by this call */
  RS_ERR_ALIGN = -3,       /* pointer not aligned to its element size */
  RS_ERR_INFEASIBLE = -4,  /* no layout with S <= S_cap */
  RS_ERR_RANGE = -5,       /* rank range outside 0 <= k0 < k1 <= m */
  RS_ERR_HIP = -6,         /* HIP runtime error */
  RS_ERR_STATE = -7,       /* layout not uploaded */
  RS_ERR_NOMEM = -8        /* a host allocation or host thread failed */
};

typedef int32_t rs_dtype;
enum { RS_F32 = 0, RS_BF16 = 1, RS_U8 = 2 };

typedef int32_t rs_qfmt;
enum { RS_Q_FP8_E4M3 = 0, RS_Q_INT8 = 1 };

/* One parameter tensor, row-major rows x cols (a vector is 1 x n).
 * gran_rows: rows per granule, the unit a shard boundary may not cut
 *   (veScale-FSDP, "RaggedShard format": element-, row- or block-wise
 *   granularity); 0 means element granularity (granule = 1 element),
 *   otherwise the granule is gran_rows*cols elements.
 * q_rows, q_cols: block-quantisation tile (veScale-FSDP, section 6.3); 0,0
 *   means the tensor is not quantised.  q_rows*q_cols <= 16384 and
 *   q_rows*cols < 2^31.  The planner places granules, not tiles: make
 *   gran_rows a multiple of q_rows (usually equal) so that no tile can
 *   straddle a shard boundary; rs_layout_create refuses a layout where one
 *   does. */
typedef struct {
  int64_t rows;
  int64_t cols;
  int64_t gran_rows;
  int32_t q_rows;
  int32_t q_cols;
} rs_tensor_spec;

/* Planner result summary. */
typedef struct {
  int64_t S;                /* elements per rank */
  int64_t total;            /* m * S */
  int64_t numel;            /* sum of tensor sizes */
  int64_t pad_elems;        /* total - numel */
  double pad_frac;          /* pad_elems / numel */
  int64_t lower_bound;      /* max(ceil(numel/m), largest first block), aligned */
  int64_t peak_param_bytes; /* 4*S + 2*m*S: fp32 shard plus bf16 full unit */
  double seconds;           /* planner wall time */
} rs_plan_info;

/* rs_plan - minimum per-rank size S for the group, tensor order kept.
 * (veScale-FSDP, "Planning Algorithm": minimise S under non-split blocks,
 * contiguous tensor memory and balanced load; padding only between tensors,
 * Figure 6(b).)  The search is exact for the given order: S is scanned
 * upward from the lower bound (feasibility is not monotone in S) and each S
 * is tested by placing every tensor at its earliest valid offset, which also
 * fixes the tie-break (lexicographically smallest offsets).
 *   specs   host [n] tensor specs, in buffer order
 *   m       number of virtual ranks, >= 1
 *   align   S and every offset are multiples of align (>= 1)
 *   S_cap   largest S to try; 0 = no cap
 *   offsets host [n] out: l_t
 *   info    host out (may be NULL)
 * Host only; touches no GPU state.  RS_ERR_INFEASIBLE if no S <= S_cap. */
rs_status rs_plan(const rs_tensor_spec* specs, int32_t n, int32_t m, int64_t align,
                  int64_t S_cap, int64_t* offsets, rs_plan_info* info);

/* Tensor orders for rs_plan_ordered (veScale-FSDP, "Planning Algorithm":
 * the pages compare the given order, an order by block size and one by
 * tensor shape, and keep the given one).  Orders are stable: tensors with
 * equal keys keep their given order.
 *   RS_ORDER_GIVEN  the given order
 *   RS_ORDER_BLOCK  granule size (gran_rows*cols, or 1) descending
 *   RS_ORDER_SHAPE  (rows, cols) descending, lexicographic
 *   RS_ORDER_BEST   plan all three, keep the smallest S; ties go to the
 *                   earlier of GIVEN, BLOCK, SHAPE */
typedef enum {
  RS_ORDER_GIVEN = 0,
  RS_ORDER_BLOCK = 1,
  RS_ORDER_SHAPE = 2,
  RS_ORDER_BEST = 3
} rs_order;

/* rs_plan_order - the buffer order of one of the orders above.
 *   specs  host [n] tensor specs
 *   kind   RS_ORDER_GIVEN, RS_ORDER_BLOCK or RS_ORDER_SHAPE
 *   perm   host [n] out: perm[i] = index into specs of the i-th tensor in
 *          the buffer
 * Host only. */
rs_status rs_plan_order(const rs_tensor_spec* specs, int32_t n, rs_order kind, int32_t* perm);

/* rs_plan_ordered - rs_plan on the group taken in the order `kind` gives.
 *   perm     host [n] out: buffer order, as rs_plan_order
 *   offsets  host [n] out: offsets[t] = l_t of tensor t (indexed as specs)
 *   others   as rs_plan
 * A layout is then built from the tensors in buffer order: specs[perm[i]]
 * with offsets[perm[i]] for i = 0..n-1.  Host only.  RS_ERR_INFEASIBLE if
 * no order fits S_cap. */
rs_status rs_plan_ordered(const rs_tensor_spec* specs, int32_t n, int32_t m, int64_t align,
                          int64_t S_cap, rs_order kind, int32_t* perm, int64_t* offsets,
                          rs_plan_info* info);

/* Opaque host-side layout: tensor, fragment and chunk tables and the tile
 * work items (runs of consecutive quantisation tiles) built from a plan.
 * The device copy of the tables lives in a caller-owned device buffer (the
 * persistent descriptor table every grouped kernel reads; veScale-FSDP,
 * "DBuffer": one kernel per group instead of one per tensor). */
typedef struct rs_layout rs_layout;

/* Counts describing a layout (for sizing caller buffers). */
typedef struct {
  int32_t n, m;
  int64_t S, total;
  int64_t num_chunks;   /* work chunks over the whole buffer */
  int64_t num_coarse_chunks; /* chunks of 32*chunk_elems (norms, masked zero) */
  int64_t num_frags;    /* tensor-rank intersections */
  int64_t num_tiles;    /* quantisation tiles of all quantised tensors */
  int64_t chunk_elems;  /* maximum chunk length */
  int64_t device_bytes; /* size of the device table buffer */
  int64_t workspace_bytes; /* scratch needed by rs_ragged_sqnorm */
} rs_layout_info;

/* rs_layout_create - validate a layout and build its tables (host only).
 *   specs, n, m, S, offsets  as from rs_plan (any valid layout is accepted)
 *   chunk_elems  maximum elements per work chunk, a multiple of 64, at most
 *                2^22; 0 = 2048.  A second table of 32x larger chunks is
 *                built for the norms and the masked zero.
 *   out          receives the handle
 * RS_ERR_INVALID_ARG if a tensor overlaps the next, leaves the buffer, has a
 * granule cut by a shard boundary, or a quantisation tile crosses a shard
 * boundary (such a tile could not be quantised without communication). */
rs_status rs_layout_create(const rs_tensor_spec* specs, int32_t n, int32_t m, int64_t S,
                           const int64_t* offsets, int64_t chunk_elems, rs_layout** out);
rs_status rs_layout_get_info(const rs_layout* layout, rs_layout_info* info);

/* rs_layout_device_bytes - bytes the caller allocates on the device for the
 * layout's tables (info.device_bytes); 0 for a NULL layout.  Host only. */
size_t rs_layout_device_bytes(const rs_layout* layout);

/* rs_workspace_bytes - bytes of device scratch rs_ragged_sqnorm needs (one
 * fp64 partial per work chunk; info.workspace_bytes); 0 for a NULL layout.
 * Host only. */
size_t rs_workspace_bytes(const rs_layout* layout);

/* rs_layout_upload - copy the tables into dev_table (device, at least
 * info.device_bytes, 256-byte aligned) on `stream` and wait for the copy.
 * The layout then uses dev_table in every call; the caller keeps it alive
 * until rs_layout_destroy.  Set-up call: it synchronises `stream`. */
rs_status rs_layout_upload(rs_layout* layout, void* dev_table, void* stream);

/* rs_layout_destroy - free the host tables (not dev_table).  NULL is a no-op. */
void rs_layout_destroy(rs_layout* layout);

/* rs_pack - copy tensors into the flat buffer, with the cast fused in.
 * buf[l_t + i] = cvt(src_t[i]) for every position l_t + i in [k0*S, k1*S);
 * every other position of those ranks (padding between tensors) is set to 0.
 * This is the per-unit copy-in before a reduce-scatter / the pre-forward
 * fp32 -> bf16 cast of native mixed precision (veScale-FSDP, "DBuffer" and
 * Figure 2; PyTorch FSDP: Experiences on Scaling Fully Sharded Data
 * Parallel, native mixed precision section).
 *   src     device array [n] of device pointers, tensor t's first element
 *           (the persistent tensor -> buffer address mapping; built once)
 *   src_dt  RS_F32 or RS_BF16
 *   buf     device, m*S elements of buf_dt (RS_F32 or RS_BF16)
 * fp32 -> bf16 rounds to nearest even (overflow to +-Inf, NaN stays a quiet
 * NaN of the same sign); bf16 -> fp32 is exact. */
rs_status rs_pack(const rs_layout* layout, const void* const* src, rs_dtype src_dt, void* buf,
                  rs_dtype buf_dt, int32_t k0, int32_t k1, void* stream);

/* rs_unpack - copy the buffer back into the tensors (rebuilding tensors
 * from the flat buffer; veScale 深度技术分析, 三 / RaggedShard Placement).
 * dst_t[i] = cvt(buf[l_t + i]) for positions in [k0*S, k1*S); other tensor
 * elements are not written.
 *   dst    device array [n] of device pointers; dst_dt RS_F32 or RS_BF16 */
rs_status rs_unpack(const rs_layout* layout, const void* buf, rs_dtype buf_dt,
                    void* const* dst, rs_dtype dst_dt, int32_t k0, int32_t k1, void* stream);

/* rs_group_scale_add - one fused kernel over every fragment of the range
 * (veScale-FSDP, "DBuffer": group-level add/scale instead of per-tensor
 * kernels; gradient accumulation and the sharded gradient scaler's unscale
 * in PyTorch FSDP).
 *   y <- fl(fl(alpha*y) + fl(beta*x)), fp32, no fused multiply-add, on the
 *   tensor elements in [k0*S, k1*S) whose tensor_mask[t] != 0 (all tensors
 *   when tensor_mask is NULL); padding is never written.
 *   y          device fp32, m*S elements
 *   x          device, m*S elements of x_dt (RS_F32 or RS_BF16).  x may be
 *              y itself (x_dt RS_F32), as in the sharded gradient scaler's
 *              in-place unscale (beta = 0): then y <- fl(fl(alpha*y) +
 *              fl(beta*y)) element by element, each element read before it
 *              is written by the same lane.  Any other overlap of x and y
 *              is undefined.
 *   tensor_mask device uint8 [n] or NULL
 *   found_inf  device uint32 [m] or NULL: found_inf[k] is set to 1 when a
 *              written value in rank k is not finite; never cleared (the
 *              caller zeroes it), so it ORs across calls. */
rs_status rs_group_scale_add(const rs_layout* layout, float* y, const void* x, rs_dtype x_dt,
                             float alpha, float beta, const uint8_t* tensor_mask,
                             uint32_t* found_inf, int32_t k0, int32_t k1, void* stream);

/* rs_group_zero - y = +0 on the tensor elements in [k0*S, k1*S) with
 * tensor_mask[t] != 0; with tensor_mask NULL, on every position of those
 * ranks, padding included (veScale-FSDP, "DBuffer": group-level zero).
 *   y  device, m*S elements of dt (RS_F32 or RS_BF16) */
rs_status rs_group_zero(const rs_layout* layout, void* y, rs_dtype dt,
                        const uint8_t* tensor_mask, int32_t k0, int32_t k1, void* stream);

/* rs_ragged_sqnorm - per-tensor sum of squares over the tensor elements in
 * [k0*S, k1*S), for tensors whose fragments are ragged across ranks
 * (veScale 深度技术分析, OpDispatcher: the ragged vector-norm handler).
 * Squares and sums are fp64; chunk partials are combined in a fixed order,
 * so results are bit-identical from run to run.  A NaN input makes the sum
 * NaN, otherwise an infinite input makes it +Inf.
 *   x          device fp32, m*S elements
 *   sq         device double [n] out: written for every tensor (0 when the
 *              tensor has no element in the range), so calls that overlap
 *              in time must not share it
 *   partial    device double [m*n] or NULL: partial[k*n + t] = the sum over
 *              tensor t's fragment in rank k, written for k in [k0, k1)
 *              (0 where the rank holds none of t) - the value each rank
 *              would contribute to an all-reduce
 *   found_inf  device uint32 [m] or NULL, as in rs_group_scale_add (values
 *              read rather than written)
 *   ws         device scratch of info.workspace_bytes; calls that share ws
 *              must be ordered on one stream */
rs_status rs_ragged_sqnorm(const rs_layout* layout, const float* x, double* sq, double* partial,
                           uint32_t* found_inf, void* ws, int32_t k0, int32_t k1, void* stream);

/* rs_ragged_sqnorm_noalloc - rs_ragged_sqnorm without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same kernels, same
 * results bit for bit; the chunk partials go to a static device array of the
 * library (1 MiB per GPU, held until the process ends), so the call makes no
 * hipMalloc, hipFree or other allocating call.  The array's device address
 * is looked up once per device, on the first call with that device current.
 *   limit    the rank range may hold at most 131072 work chunks: any range
 *            of fewer than 256 coarse chunks, and up to about 8.6e9
 *            elements with the default chunk size; a larger range returns
 *            RS_ERR_INVALID_ARG before anything is enqueued
 *   others   as rs_ragged_sqnorm (x, sq, partial, found_inf, k0, k1, stream)
 * Every call on one GPU shares that GPU's array, and a call overwrites the
 * partials it reads before reading them (nothing needs clearing): calls that
 * overlap in time on one GPU race, so order them on one stream. */
rs_status rs_ragged_sqnorm_noalloc(const rs_layout* layout, const float* x, double* sq,
                                   double* partial, uint32_t* found_inf, int32_t k0, int32_t k1,
                                   void* stream);

/* rs_block_quant - absmax block quantisation of every tile of every
 * quantised tensor that lies in [k0*S, k1*S).  Tiles never cross a shard
 * boundary (rs_layout_create rejects such layouts), so each rank quantises
 * its own shard without communication (veScale-FSDP, "RaggedShard format"
 * and section 6.3, block-wise INT8/FP8).
 *   per tile: amax = max|x| (NaN if any element is NaN);
 *   scale = fp32(amax / Q), Q = 448 (RS_Q_FP8_E4M3) or 127 (RS_Q_INT8);
 *   code = encode(fp32(x / scale)) with IEEE division:
 *     FP8 E4M3FN (OCP): saturating round to nearest even, |q| > 448 and
 *     +-Inf give +-448, NaN gives 0x7F;
 *     INT8: round half to even, clip to [-127, 127], NaN gives 0;
 *   scale == 0 gives all-zero codes; a NaN scale is stored as 0x7FC00000.
 *   x       device fp32, m*S elements
 *   codes   device uint8, m*S bytes: codes[p] encodes x[p]; positions of
 *           padding and of tensors that are not quantised are not written
 *   scales  device fp32 [info.num_tiles] (may be NULL when num_tiles is 0):
 *           tiles numbered tensor by tensor
 *           (quantised tensors only, in group order), row-major inside a
 *           tensor; only tiles in the range are written
 *   found_inf device uint32 [m] or NULL: found_inf[k] is set to 1 when a
 *           quantised value read in rank k is not finite (the non-finite
 *           check of the sharded gradient scaler, for grads quantised
 *           before communication); never cleared by the call */
rs_status rs_block_quant(const rs_layout* layout, const float* x, rs_qfmt fmt, uint8_t* codes,
                         float* scales, uint32_t* found_inf, int32_t k0, int32_t k1, void* stream);

/* rs_block_dequant - the inverse: y[p] = fl(decode(codes[p]) * scale) for
 * every element of every tile in [k0*S, k1*S) (the dequantisation step of
 * an 8-bit optimizer state; veScale-FSDP, section 6.3).  decode is exact:
 * E4M3FN per OCP (codes 0x7F/0xFF give NaN), INT8 as a signed integer; the
 * fp32 product is the one rounding (bf16 output: then rounded to nearest
 * even).  Positions of padding and of tensors that are not quantised are not
 * written.
 *   codes   device uint8, m*S bytes (as written by rs_block_quant)
 *   scales  device fp32 [info.num_tiles] (may be NULL when num_tiles is 0)
 *   y       device, m*S elements of y_dt (RS_F32 or RS_BF16) */
rs_status rs_block_dequant(const rs_layout* layout, const uint8_t* codes, rs_qfmt fmt,
                           const float* scales, void* y, rs_dtype y_dt, int32_t k0, int32_t k1,
                           void* stream);

/* AdamW hyperparameters for one step (fp32).  bias_correction1/2 are
 * 1 - beta1^t and 1 - beta2^t for step t, computed by the caller. */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  float bias_correction1, bias_correction2;
  float grad_scale; /* grads are divided by it (1 = unscaled) */
} rs_adamw_params;

/* rs_adamw_step - one fused AdamW step over every fragment of the range, in
 * place (the fused optimizer the pages run on the local shard; veScale
 * 深度技术分析, OpDispatcher: fused AdamW/SGD handler).  Per element, fp32,
 * each operation rounded once, IEEE sqrt and division:
 *   g = grad / grad_scale   (as grad * fl(1/grad_scale))
 *   m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g)
 *   p = p*(1 - lr*wd) - (lr/bc1) * (m / (sqrt(v)/sqrt(bc2) + eps))
 * with 1-b1, 1-b2, 1-lr*wd, lr/bc1, sqrt(bc2), 1/grad_scale formed once in
 * fp32.  Only tensor elements in [k0*S, k1*S) with tensor_mask[t] != 0 (all
 * when NULL) change.  found_inf: device uint32 [m] or NULL; when any entry
 * is non-zero nothing is written (the step is skipped).
 *   p, g, m, v   device fp32, m*S elements each (buffer layout)
 *   hp           host; RS_ERR_INVALID_ARG unless both bias corrections are
 *                > 0 and grad_scale is non-zero */
rs_status rs_adamw_step(const rs_layout* layout, float* p, const float* g, float* m, float* v,
                        const rs_adamw_params* hp, const uint8_t* tensor_mask,
                        const uint32_t* found_inf, int32_t k0, int32_t k1, void* stream);

/* rs_adamw8_step - AdamW with block-quantised moments (8-bit Adam;
 * veScale-FSDP, section 6.3: block-wise INT8 optimizer states, quantised
 * per shard without communication).  For every tile of every quantised
 * tensor in [k0*S, k1*S):
 *   m = fl(decode(m code) * m scale), v likewise (as rs_block_dequant);
 *   the AdamW update of rs_adamw_step on (p, g, m, v);
 *   m', v' re-quantised with new absmax scales (as rs_block_quant).
 * Tensors that are not quantised are not touched (step their fp32 moments
 * with rs_adamw_step and a tensor mask).  found_inf as in rs_adamw_step.
 *   p, g               device fp32, m*S elements (buffer layout)
 *   m_codes, v_codes   device uint8, m*S bytes, in place
 *   m_scales, v_scales device fp32 [info.num_tiles], in place (may be NULL
 *                      when num_tiles is 0)
 *   fmt                RS_Q_INT8 or RS_Q_FP8_E4M3
 *   hp                 host, checked as in rs_adamw_step */
rs_status rs_adamw8_step(const rs_layout* layout, float* p, const float* g, uint8_t* m_codes,
                         float* m_scales, uint8_t* v_codes, float* v_scales, rs_qfmt fmt,
                         const rs_adamw_params* hp, const uint32_t* found_inf, int32_t k0,
                         int32_t k1, void* stream);

/* SGD hyperparameters (fp32). */
typedef struct {
  float lr, momentum, weight_decay;
  float grad_scale;
  int32_t nesterov;
} rs_sgd_params;

/* rs_sgd_step - one fused SGD-with-momentum step, in place:
 *   g = grad/grad_scale + wd*p;  b = mu*b + g;  d = nesterov ? g + mu*b : b;
 *   p = p - lr*d
 * (fp32, each operation rounded once; no dampening - a zeroed b makes the
 * first step b = g).  Masks, rank range and found_inf as in rs_adamw_step.
 *   p, g, buf    device fp32, m*S elements each
 *   hp           host; RS_ERR_INVALID_ARG when grad_scale is 0 */
rs_status rs_sgd_step(const rs_layout* layout, float* p, const float* g, float* buf,
                      const rs_sgd_params* hp, const uint8_t* tensor_mask,
                      const uint32_t* found_inf, int32_t k0, int32_t k1, void* stream);

/* Static description of a status code. */
const char* rs_status_str(rs_status status);
/* Message of the last failed call on this thread ("" if none). */
const char* rs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RS_H */
