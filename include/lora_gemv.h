/*
 * lora_gemv.h -- C ABI of the heterogeneous-adapter LoRA delta on MI355X
 * (gfx950).
 *
 * For a batch of rows in which every row b names its own adapter slot
 * a = row_adapter[b], the library adds that adapter's low-rank delta to the
 * base output of each projection:
 *
 *     v[b]  = A_a . x[b]                       (shrink, rank-r vector)
 *     y[b] += scale_a * B_a . v[b]             (expand, fused into y)
 *
 * Sources:
 *  - "m07 -- Multi-Adapter (LoRA) Serving", "2. Scale Numbers": a LoRA on a
 *    weight W of shape (d_out, d_in) is B.A with A of shape (r, d_in) and B of
 *    shape (d_out, r); r * (d_in + d_out) parameters per projection.
 *  - same page, "6. Deep Dive A: Batching Heterogeneous Adapters": the forward
 *    is y = Wx + (B.A)x(alpha/r); the base term is shared, the adapter term is
 *    per row; one batched kernel takes the batch, an index vector mapping each
 *    sequence to an adapter slot and the adapter buffer, and gathers inside
 *    the kernel (BGMV for decode, SGMV for variable-length prefill segments).
 *  - "12. Adapter Serving and Multi-Tenant Customization", "Scheduling with
 *    adapter awareness": the adapter products are a second, indexed operation
 *    after the base product, with per-request adapter pointers and a
 *    base-only group; "Interactions with other engine mechanisms", CUDA
 *    graphs: adapter addresses are read from a buffer at run time rather than
 *    baked into a captured graph; "vLLM's pre-allocated LoRA buffers" and
 *    "S-LoRA's unified paging": adapters live in fixed-size slots reached
 *    through a table.
 *  - "LoRA, quotas and noisy neighbours", "One weight read, many adapters":
 *    rows are tagged with their adapter and grouped; the update is applied in
 *    registers.
 *
 * Conventions for every call:
 *  - bf16 tensors are raw 16-bit bfloat16 values, row-major.
 *  - Every pointer argument marked "device" is device memory owned by the
 *    caller.  The library allocates no device memory, keeps no pointer after
 *    a call returns and has no global state; it is reentrant.  (The host-only
 *    lora_form_batch uses temporary host memory, freed before it returns.
 *    The one exception is lora_apply_layer_noalloc, which works in a static
 *    device array of the library and caches its address per device.)
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and returns; nothing synchronises the host.  Buffers
 *    must stay alive until the stream has passed the call.  No call
 *    allocates, frees or memsets through the runtime, so calls may be
 *    captured into a HIP graph; the table, the row ids and the segments are
 *    read from device memory when the kernels run.
 *  - Host-detectable errors (listed per call) return a status and enqueue
 *    nothing.  Errors in device data never fault: the affected rows or
 *    (segment, projection) pairs are skipped, leaving y unchanged, and the
 *    device status word `*seg.status` becomes nonzero.  lora_build_segments
 *    sets it to the number of rows whose id is >= num_slots; each delta call
 *    then adds one per segment that does not fit the batch and one per
 *    (segment, projection) whose table entry cannot be applied (rank above
 *    max_rank, a null or misaligned factor pointer).  A call made of two
 *    parts counts in its first: lora_layer_shrink and lora_linear_shrink
 *    add, lora_layer_expand and lora_linear_expand add nothing.  It is a
 *    flag and a count of problems, not a number of rows.
 *  - Dimensions d_in, d_out and leading dimensions are counted in elements;
 *    d_in, d_out, ldx and ldy must be multiples of 8 and x, y pointers
 *    16-byte aligned (16-byte vector access).
 *  - Each activation matrix (x or y: num_rows * ld * 2 bytes) must stay below
 *    4 GiB - 256 bytes; the kernels address it with 32-bit byte offsets
 *    (LORA_ERR_SHAPE otherwise).
 */
#ifndef LORA_GEMV_H
#define LORA_GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest adapter rank the kernels accept (the pages' serving ranks run from
 * 8 to 64: "12. Adapter Serving ...", "What an adapter adds"). */
#define LORA_MAX_RANK 64

/* Table columns of a transformer layer, in this order. */
#define LORA_NUM_MODULES 7

/* A flag the layer calls (lora_apply_layer and its parts, lora_decode_layer,
 * lora_apply_layer_noalloc, lora_apply_layer_stacked, lora_linear_layer and
 * its parts and their _q4 forms) accept in module_mask beside the module
 * bits: the caller's table entries are int8 (LORA_FORMAT_INT8_ROWS), so the
 * shrink's work items take more k than a bf16 item (four times, up to 4096
 * inputs: at least as many bytes per item).  Results are the same within the tolerance with or without it and
 * for entries of either format; pass the same flag to both parts of a split
 * call.  Source: "m07 -- Multi-Adapter (LoRA) Serving", "9. Bottlenecks and
 * Evolution", item 3 (int8 adapters halve the bytes). */
#define LORA_MASK_INT8_ITEMS (1u << 16)
enum {
  LORA_Q = 0, LORA_K = 1, LORA_V = 2, LORA_O = 3,
  LORA_GATE = 4, LORA_UP = 5, LORA_DOWN = 6
};

typedef enum lora_status {
  LORA_OK = 0,
  LORA_ERR_NULL = 1,       /* a required pointer is NULL                      */
  LORA_ERR_SHAPE = 2,      /* a size or leading dimension is out of range     */
  LORA_ERR_RANK = 3,       /* max_rank outside [1, LORA_MAX_RANK]             */
  LORA_ERR_ALIGN = 4,      /* a pointer or leading dimension is not 16-byte
                              aligned, or a dimension is not a multiple of 8  */
  LORA_ERR_WORKSPACE = 5,  /* ws_bytes < lora_workspace_bytes(...)            */
  LORA_ERR_MODULE = 6,     /* bad module index, n_mod or module mask          */
  LORA_ERR_LAUNCH = 7,     /* the HIP runtime refused a kernel launch, or the
                              device or its static scratch could not be found */
  LORA_ERR_SCRATCH = 8     /* the call needs more than LORA_STATIC_SCRATCH_BYTES
                              of scratch (lora_apply_layer_noalloc)           */
} lora_status_t;

/*
 * Storage format of an entry's factors.
 *   LORA_FORMAT_BF16       bf16 values (the layout described below).
 *   LORA_FORMAT_INT8_ROWS  int8 values with one fp32 scale per row, value =
 *     scale[row] * q[row][col] ("m07 ...", "9. Bottlenecks and Evolution",
 *     item 3: quantised adapters halve the bytes; symmetric per-row int8 is
 *     this library's reading).  Each factor is one block, 16-byte aligned:
 *       A block: float scale[round_up(rank, 4)], then int8 A[rank][lda8],
 *                lda8 = d_in rounded up to a multiple of 16 (bytes [d_in,
 *                lda8) of a row are padding and contribute nothing);
 *       B block: float scale[round_up(d_out, 4)], then int8 B[d_out][ldb8],
 *                ldb8 = rank rounded up to a multiple of 16 (bytes [rank,
 *                ldb8) of a row are padding and contribute nothing).
 *     Every int8 row starts 16-byte aligned.
 */
typedef enum lora_factor_format {
  LORA_FORMAT_BF16 = 0,
  LORA_FORMAT_INT8_ROWS = 1
} lora_factor_format_t;

/*
 * One entry of the device-resident adapter table: the factors of one adapter
 * for one projection ("m07 ...", "2. Scale Numbers" for the shapes).
 * A table is an array of these indexed [slot * n_mod + module].
 *   A      device, bf16 [rank][d_in], row-major, leading dimension d_in,
 *          16-byte aligned (LORA_FORMAT_BF16; see above for int8).
 *   B      device, bf16 [d_out][ldb], row-major, 16-byte aligned, with
 *          ldb = rank rounded up to a multiple of 8 (so every row is 16-byte
 *          aligned; for ranks 8, 16, 32, 64 B is compact).  Columns
 *          [rank, ldb) are padding: they must hold finite values (zero is
 *          fine) and contribute nothing.
 *   rank   0 .. max_rank; 0 means the projection is not targeted by this
 *          adapter (zero delta, A and B not read).  A rank outside
 *          [0, max_rank] is a device-data error.
 *   scale  alpha / r of the forward y = Wx + (B.A)x(alpha/r) ("m07 ...",
 *          "6. Deep Dive A"); 1.0f when the adapter gives no alpha.
 *   format a lora_factor_format_t; any other value is a device-data error.
 * Slots can live anywhere (fixed-size pages of one pool, separate buffers):
 * row ids index the table, not memory.  32 bytes.
 */
typedef struct lora_adapter_entry {
  const void *A;
  const void *B;
  int32_t rank;
  float scale;
  int32_t format;   /* lora_factor_format_t */
  int32_t reserved; /* set to 0 */
} lora_adapter_entry_t;

/*
 * Segments: the rows of the batch grouped by adapter ("LoRA, quotas and noisy
 * neighbours", "One weight read, many adapters").  All device int32 arrays,
 * written by lora_build_segments and read by the other calls.
 *   perm          [num_rows]      original row of each sorted position
 *   seg_offsets   [num_rows + 1]  segment s = sorted positions
 *                                 [seg_offsets[s], seg_offsets[s+1])
 *   seg_adapter   [num_rows]      adapter slot of segment s
 *   num_segments  [1]             number of segments
 *   tile_counts   [2]             sizes of the build's work for the other
 *                                 calls (how many of their row tiles the
 *                                 segments fill); no meaning to the caller
 *   status        [1]             0, or the number of rows with an id
 *                                 >= num_slots or in a segment past
 *                                 max_segments at the last build, plus one
 *                                 per (segment, projection) skipped since then
 * Only the first num_segments (+1) entries are meaningful.
 * One host value rides along:
 *   max_segments  0, or a bound on the segments of a build: the number of
 *                 distinct valid slot ids in the batch, which a host that
 *                 formed the batch knows ("12. Adapter Serving ...",
 *                 "Scheduling with adapter awareness": the scheduler groups
 *                 requests by adapter).  Every call sizes its tiles and grid
 *                 for min(num_rows, num_slots, max_segments) segments, so a
 *                 tight bound gives a batch of few adapters short work items
 *                 instead of items sized for one adapter per row.  A build
 *                 that finds more segments keeps the first max_segments
 *                 (lowest slots) and counts the rows of the others into
 *                 *status (those rows get no delta); the other calls apply at
 *                 most max_segments segments.  Use one value for a build and
 *                 the calls that read its segments.  Negative: LORA_ERR_SHAPE.
 */
typedef struct lora_segments {
  int32_t *perm;
  int32_t *seg_offsets;
  int32_t *seg_adapter;
  int32_t *num_segments;
  int32_t *tile_counts;
  int32_t *status;
  int32_t max_segments;
} lora_segments_t;

/* One projection of a layer for lora_apply_layer. */
typedef struct lora_module_io {
  const void *x; /* device, bf16 [num_rows][ldx]: input of the projection   */
  int64_t ldx;
  void *y;       /* device, bf16 [num_rows][ldy]: base output W.x, updated  */
  int64_t ldy;   /* in place                                                */
  int32_t d_in;
  int32_t d_out;
} lora_module_io_t;

/*
 * Workspace (device scratch) that covers every call with these sizes, in
 * bytes.  sum_d_in is the sum of d_in over the projections a
 * call processes (d_in for lora_shrink, the sum over the mask for the layer
 * calls).  One workspace of this size serves every call on the same stream.
 * A call that needs none (lora_expand; lora_build_segments on up to 1024
 * rows) accepts ws = NULL.  A workspace must be 16-byte aligned
 * (LORA_ERR_ALIGN otherwise).  Returns 0 for invalid arguments.
 */
size_t lora_workspace_bytes(int32_t num_rows, int32_t num_slots,
                            int32_t max_rank, int64_t sum_d_in);

/*
 * lora_build_segments -- group the rows of a batch by adapter.
 * Source: "m07 ...", "6. Deep Dive A" (index vector mapping each sequence to
 * an adapter slot); "LoRA, quotas and noisy neighbours", "One weight read,
 * many adapters" (tag each row with its adapter and group); "12. Adapter
 * Serving ...", "Scheduling with adapter awareness" (base-only requests form
 * their own group).
 *
 *   row_adapter  device int32 [num_rows]: slot of each row; a negative id
 *                means base only (the row joins no segment and its y is never
 *                touched); an id >= num_slots is a device-data error (the row
 *                is skipped and counted into *seg.status).
 * Result: segments in ascending slot order, rows ascending inside a segment
 * (a stable sort by id); *seg.status is reset to the number of bad ids.
 * Errors: LORA_ERR_NULL (row_adapter with num_rows > 0, any seg pointer, ws
 * when workspace is needed), LORA_ERR_SHAPE (num_rows < 0, num_slots < 1),
 * LORA_ERR_WORKSPACE, LORA_ERR_LAUNCH.
 */
lora_status_t lora_build_segments(const int32_t *row_adapter, int32_t num_rows,
                                  int32_t num_slots, lora_segments_t seg,
                                  void *ws, size_t ws_bytes, void *stream);

/*
 * lora_shrink -- v[b][j] = sum_k A_a[j][k] * x[b][k] for every row b in a
 * segment, a its adapter, j < rank (the left factor of (B.A)x, "m07 ...",
 * "6. Deep Dive A").  v is not scaled.
 *
 *   x       device bf16 [num_rows][ldx]
 *   table   device lora_adapter_entry_t [num_slots * n_mod]; this call uses
 *           column `module` (0 <= module < n_mod <= 7)
 *   v       device float [num_rows][ldv]: for rows in a segment, columns
 *           [0, rank) get the result and [rank, max_rank) get 0; other rows
 *           are not written.  ldv >= max_rank, multiple of 4.
 * Errors: LORA_ERR_NULL, LORA_ERR_SHAPE (num_rows < 0, d_in <= 0, ldx < d_in,
 * ldv < max_rank, num_slots < 1), LORA_ERR_ALIGN, LORA_ERR_RANK,
 * LORA_ERR_MODULE, LORA_ERR_WORKSPACE, LORA_ERR_LAUNCH.
 */
lora_status_t lora_shrink(const void *x, int64_t ldx, int32_t num_rows,
                          int32_t d_in, const lora_adapter_entry_t *table,
                          int32_t num_slots, int32_t n_mod, int32_t module,
                          lora_segments_t seg, int32_t max_rank, float *v,
                          int64_t ldv, void *ws, size_t ws_bytes, void *stream);

/*
 * lora_expand -- y[b][n] = bf16_rne( y[b][n] + scale_a * sum_j B_a[n][j] *
 * v[b][j] ) for every row b in a segment (the right factor of (B.A)x and the
 * sum with the shared base output, "m07 ...", "6. Deep Dive A").  The sum is
 * accumulated in fp32 and rounded to bf16 once, round-to-nearest-even.
 *
 *   v       device float [num_rows][ldv], as written by lora_shrink
 *           (columns [0, rank) are read)
 *   y       device bf16 [num_rows][ldy], base output, updated in place; rows
 *           in no segment are not touched.
 * Errors: as lora_shrink, with d_out in place of d_in.
 */
lora_status_t lora_expand(const float *v, int64_t ldv, int32_t num_rows,
                          int32_t d_out, const lora_adapter_entry_t *table,
                          int32_t num_slots, int32_t n_mod, int32_t module,
                          lora_segments_t seg, int32_t max_rank, void *y,
                          int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/*
 * lora_apply_layer -- the delta of every projection of one transformer layer
 * whose bit is set in module_mask (bit m = table column m: q, k, v, o, gate,
 * up, down), in one grouped shrink launch and one grouped expand launch.  The
 * rank-r vectors stay in the workspace and never reach the caller.
 * Projection shapes are the caller's (the 70B layer of "m07 ...",
 * "2. Scale Numbers": q, o 8192->8192; k, v 8192->1024; gate, up
 * 8192->28672; down 28672->8192).
 *
 *   io      host array lora_module_io_t[7]; entries outside the mask are
 *           ignored.  Projections may share x (q, k and v do in a layer).
 *   table   device lora_adapter_entry_t [num_slots * 7]
 * Equivalent to lora_layer_shrink followed by lora_layer_expand with the
 * same arguments.
 * Errors: LORA_ERR_NULL, LORA_ERR_SHAPE, LORA_ERR_ALIGN, LORA_ERR_RANK,
 * LORA_ERR_MODULE (mask 0 or above 0x7f), LORA_ERR_WORKSPACE,
 * LORA_ERR_LAUNCH.
 */
lora_status_t lora_apply_layer(const lora_module_io_t *io, uint32_t module_mask,
                               int32_t num_rows,
                               const lora_adapter_entry_t *table,
                               int32_t num_slots, lora_segments_t seg,
                               int32_t max_rank, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * lora_decode_layer -- lora_build_segments(row_adapter, ...) followed by
 * lora_apply_layer(...) with the same arguments: the rows grouped by adapter
 * (seg is written exactly as lora_build_segments writes it) and the delta of
 * every projection in module_mask.  Source: "m07 -- Multi-Adapter (LoRA)
 * Serving", "6. Deep Dive A" (one batched kernel takes the batch and the
 * index vector mapping each sequence to an adapter slot, and gathers inside
 * the kernel; the cost is bandwidth) and "LoRA, quotas and noisy
 * neighbours", "One weight read, many adapters" (rows tagged and grouped,
 * the update applied in registers).
 * A decode batch of at most 256 rows with max_rank <= 32 runs as ONE launch
 * when its repeated reads of A stay small (see below): every block finds its
 * row's segment from the ids itself, computes that segment's whole v and
 * applies one tile of B, so no block waits on another and nothing passes
 * through the workspace.  The blocks of one segment each read its A (served
 * from L2 after the first), so the path is taken only while those repeated
 * reads stay within about 320 MB (one pass over A per block of a segment,
 * one more per 4 further rows, segments counted by seg.max_segments when
 * given).  Any other batch runs the three launches of lora_build_segments +
 * lora_apply_layer.  lora_decode_layer_launches tells which.  Both give
 * results within the oracle tolerance; the one-launch path sums A.x in a
 * different order, so its bits may differ from lora_apply_layer's.  Results
 * are bit-reproducible.
 *
 *   row_adapter  device int32 [num_rows], as for lora_build_segments
 *   seg          written as by lora_build_segments; seg.max_segments
 *                applies as there (rows of segments past the bound get no
 *                delta); *seg.status gets the rows whose id is >= num_slots
 *                or past the bound, plus one per (segment, projection) whose
 *                entry cannot be applied
 *   ws, ws_bytes at least lora_workspace_bytes(num_rows, num_slots,
 *                max_rank, sum of the masked d_in) (the one-launch path uses
 *                none of it)
 *   other arguments as for lora_apply_layer.
 * Errors: those of lora_apply_layer and lora_build_segments.
 */
lora_status_t lora_decode_layer(const lora_module_io_t *io, uint32_t module_mask,
                                int32_t num_rows, const int32_t *row_adapter,
                                const lora_adapter_entry_t *table, int32_t num_slots,
                                lora_segments_t seg, int32_t max_rank, void *ws,
                                size_t ws_bytes, void *stream);

/*
 * lora_decode_layer_launches -- the number of kernel launches
 * lora_decode_layer makes for these arguments (host only, no device work):
 * 1 for the one-launch path, 3 otherwise, 0 for arguments it would reject.
 */
int32_t lora_decode_layer_launches(const lora_module_io_t *io, uint32_t module_mask,
                                   int32_t num_rows, int32_t num_slots,
                                   lora_segments_t seg, int32_t max_rank);

/*
 * The two launches of lora_apply_layer, for callers that interleave other
 * work or time them apart.  lora_layer_shrink leaves the rank-r partial sums
 * in the workspace; lora_layer_expand, enqueued later on the same stream with
 * the same arguments and workspace, consumes them.
 */
lora_status_t lora_layer_shrink(const lora_module_io_t *io, uint32_t module_mask,
                                int32_t num_rows,
                                const lora_adapter_entry_t *table,
                                int32_t num_slots, lora_segments_t seg,
                                int32_t max_rank, void *ws, size_t ws_bytes,
                                void *stream);
lora_status_t lora_layer_expand(const lora_module_io_t *io, uint32_t module_mask,
                                int32_t num_rows,
                                const lora_adapter_entry_t *table,
                                int32_t num_slots, lora_segments_t seg,
                                int32_t max_rank, void *ws, size_t ws_bytes,
                                void *stream);

/* One projection of a layer for lora_linear_layer: input, base weight and
 * output (which the call writes). */
typedef struct lora_linear_io {
  const void *x; /* device, bf16 [num_rows][ldx]                             */
  int64_t ldx;
  const void *W; /* device, bf16 [d_out][ldw]: the base weight, row n holds  */
  int64_t ldw;   /* the d_in weights of output n (a linear layer's weight)   */
  void *y;       /* device, bf16 [num_rows][ldy]: written, W.x + delta       */
  int64_t ldy;
  int32_t d_in;
  int32_t d_out;
} lora_linear_io_t;

/*
 * lora_linear_workspace_bytes -- workspace of lora_linear_layer for n_modules
 * projections whose d_in sum to sum_d_in (also enough for
 * lora_build_segments with the same rows and slots).  0 for bad arguments.
 */
size_t lora_linear_workspace_bytes(int32_t num_rows, int32_t num_slots,
                                   int32_t max_rank, int64_t sum_d_in,
                                   int32_t n_modules);

/*
 * lora_linear_layer -- base projection and adapter delta together:
 *     y[b] = bf16_rne( W . x[b] + scale_a * B_a . (A_a . x[b]) )
 * for every projection whose bit is set in module_mask, a = row_adapter[b]
 * (rows whose id is negative or >= num_slots get the base term only).
 * Source: "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A" (y = Wx +
 * (B.A)x(alpha/r): the base term shared by the batch, the adapter term per
 * row) and the fused base + delta on the pages' list of next steps (the
 * delta in the base product's epilogue with a wide accumulator, so y is
 * written once, never read).  Three launches on `stream`: the grouped shrink
 * of lora_layer_shrink (each distinct adapter's A read once), a sum of its
 * partials into one v per row and projection, and one fused kernel that
 * streams W once (bf16 matrix cores, fp32 accumulate) and adds each row's
 * delta before the single bf16 rounding.
 *
 *   io           array of LORA_NUM_MODULES entries, read where module_mask
 *                has a bit: x, W, y 16-byte aligned; d_in, d_out, ldx, ldw,
 *                ldy multiples of 8; W below 4 GiB
 *   row_adapter  device int32 [num_rows]: the ids the segments were built
 *                from (lora_build_segments on the same stream before)
 *   seg          those segments; *seg.status counts as for lora_apply_layer
 *   ws, ws_bytes at least lora_linear_workspace_bytes(...)
 *   other arguments as for lora_apply_layer.  Factors in either format.
 *
 * Errors: those of lora_apply_layer; LORA_ERR_NULL for a null W or
 * row_adapter, LORA_ERR_SHAPE for ldw < d_in or a W of 4 GiB or more.
 */
lora_status_t lora_linear_layer(const lora_linear_io_t *io, uint32_t module_mask,
                                int32_t num_rows, const int32_t *row_adapter,
                                const lora_adapter_entry_t *table, int32_t num_slots,
                                lora_segments_t seg, int32_t max_rank, void *ws,
                                size_t ws_bytes, void *stream);

/*
 * The two parts of lora_linear_layer, for callers that interleave other work
 * or time them apart: lora_linear_shrink leaves one v per row and projection
 * in the workspace (the grouped shrink and the sum of its partials);
 * lora_linear_expand, enqueued later on the same stream with the same
 * arguments and workspace, runs the fused kernel and writes y.
 */
lora_status_t lora_linear_shrink(const lora_linear_io_t *io, uint32_t module_mask,
                                 int32_t num_rows, const int32_t *row_adapter,
                                 const lora_adapter_entry_t *table, int32_t num_slots,
                                 lora_segments_t seg, int32_t max_rank, void *ws,
                                 size_t ws_bytes, void *stream);
lora_status_t lora_linear_expand(const lora_linear_io_t *io, uint32_t module_mask,
                                 int32_t num_rows, const int32_t *row_adapter,
                                 const lora_adapter_entry_t *table, int32_t num_slots,
                                 lora_segments_t seg, int32_t max_rank, void *ws,
                                 size_t ws_bytes, void *stream);

/* Inputs of a row of a 4-bit base weight that share one scale. */
#define LORA_Q4_GROUP 128

/* One projection of a layer with a 4-bit base weight, for
 * lora_linear_layer_q4.  W[n][k] = Ws[n][k / LORA_Q4_GROUP] * q[n][k], with
 * q[n][k] the signed 4-bit value (two's complement, -8 .. 7) in byte k / 2 of
 * row n of Wq: the low nibble for even k, the high nibble for odd k. */
typedef struct lora_linear_q4_io {
  const void *x;  /* device, bf16 [num_rows][ldx]                            */
  int64_t ldx;
  const void *Wq; /* device, uint8 [d_out][ldwq]: packed 4-bit weights      */
  int64_t ldwq;   /* bytes per row: >= d_in / 2, a multiple of 16           */
  const void *Ws; /* device, fp32 [d_out][lds]: the group scales            */
  int64_t lds;    /* floats per row: >= d_in / LORA_Q4_GROUP                */
  void *y;        /* device, bf16 [num_rows][ldy]: written, W.x + delta     */
  int64_t ldy;
  int32_t d_in;   /* a multiple of LORA_Q4_GROUP                            */
  int32_t d_out;
} lora_linear_q4_io_t;

/*
 * lora_linear_layer_q4 -- lora_linear_layer with 4-bit base weights: the
 * base dequantised in the kernel, the BF16 (or int8) adapter term added in
 * its epilogue and the sum accumulated in fp32 before the one bf16 rounding.
 * Rows with an adapter and base-only rows (id negative or >= num_slots) mix
 * in one batch.  Source: "12. Adapter Serving and Multi-Tenant
 * Customization", "Interactions with other engine mechanisms", Quantization
 * (an INT4 base with BF16 adapters: dequantise the base, add the adapter
 * contribution, accumulate wide; one batch mixes rows with and without an
 * adapter).  The matrix cores take each 4-bit value exactly (as bf16) and
 * each group's sum is scaled once, in fp32.
 *
 *   io           array of LORA_NUM_MODULES entries, read where module_mask
 *                has a bit: x, Wq, y 16-byte aligned, Ws 4-byte aligned;
 *                d_out, ldx, ldy multiples of 8; Wq and Ws below 4 GiB
 *   other arguments as for lora_linear_layer (the same workspace size).
 *
 * Errors: those of lora_linear_layer; LORA_ERR_NULL for a null Wq or Ws,
 * LORA_ERR_ALIGN for a d_in that is not a multiple of LORA_Q4_GROUP or an
 * ldwq that is not a multiple of 16, LORA_ERR_SHAPE for ldwq < d_in / 2 or
 * lds < d_in / LORA_Q4_GROUP.
 */
lora_status_t lora_linear_layer_q4(const lora_linear_q4_io_t *io, uint32_t module_mask,
                                   int32_t num_rows, const int32_t *row_adapter,
                                   const lora_adapter_entry_t *table, int32_t num_slots,
                                   lora_segments_t seg, int32_t max_rank, void *ws,
                                   size_t ws_bytes, void *stream);

/* The two parts of lora_linear_layer_q4, as for lora_linear_shrink and
 * lora_linear_expand. */
lora_status_t lora_linear_shrink_q4(const lora_linear_q4_io_t *io, uint32_t module_mask,
                                    int32_t num_rows, const int32_t *row_adapter,
                                    const lora_adapter_entry_t *table, int32_t num_slots,
                                    lora_segments_t seg, int32_t max_rank, void *ws,
                                    size_t ws_bytes, void *stream);
lora_status_t lora_linear_expand_q4(const lora_linear_q4_io_t *io, uint32_t module_mask,
                                    int32_t num_rows, const int32_t *row_adapter,
                                    const lora_adapter_entry_t *table, int32_t num_slots,
                                    lora_segments_t seg, int32_t max_rank, void *ws,
                                    size_t ws_bytes, void *stream);

/* Most adapters one row may carry in lora_apply_layer_stacked. */
#define LORA_MAX_STACK 8

/*
 * lora_apply_layer_stacked -- several adapters on one row: y += sum over the
 * row's list of scale_a * B_a . (A_a . x) for every projection in
 * module_mask.  Source: "m07 -- Multi-Adapter (LoRA) Serving", "9.
 * Bottlenecks and Evolution", item 5 (multi-adapter composition: two
 * adapters on one request, each one more read and one more kernel pass).
 * Pass t = 0 .. depth-1, in stream order: the segments of column t of
 * row_adapters (as lora_build_segments), then the shrink and the expand of
 * lora_apply_layer.  Each distinct adapter of a column is read once in its
 * pass.  y is rounded to bf16 after each pass (as by depth calls of
 * lora_apply_layer), so the delta of pass t is added to the rounded result of
 * the passes before it.
 *
 *   row_adapters  device int32 [num_rows][depth]: the adapter slots of each
 *                 row, in pass order; negative entries add nothing (a row
 *                 with fewer adapters pads its list with -1)
 *   depth         1 .. LORA_MAX_STACK
 *   pass_max_rank host int32 [depth] or NULL: the largest rank of the
 *                 adapters in each column, 1 .. max_rank (NULL: max_rank for
 *                 every pass).  Each pass is sized for its own rank class, so
 *                 a column of low-rank adapters does not run in the class of
 *                 the highest rank; an entry above its pass's rank is a
 *                 device-data error, as a rank above max_rank is.
 *   seg           device segments as for lora_build_segments; on return they
 *                 describe the last pass.  *seg.status sums the bad ids of
 *                 every pass and the delta calls' additions.
 *   ws, ws_bytes  at least lora_workspace_bytes(num_rows, num_slots,
 *                 max_rank, sum of the masked d_in); shared by the passes
 *   other arguments as for lora_apply_layer.
 *
 * Errors: those of lora_apply_layer and lora_build_segments,
 * LORA_ERR_SHAPE for a depth outside [1, LORA_MAX_STACK], and LORA_ERR_RANK
 * for a pass_max_rank entry outside [1, max_rank].
 */
lora_status_t lora_apply_layer_stacked(const lora_module_io_t *io, uint32_t module_mask,
                                       int32_t num_rows, const int32_t *row_adapters,
                                       int32_t depth, const int32_t *pass_max_rank,
                                       const lora_adapter_entry_t *table,
                                       int32_t num_slots, lora_segments_t seg,
                                       int32_t max_rank, void *ws, size_t ws_bytes,
                                       void *stream);

/*
 * lora_form_batch -- choose the requests of the next step from a waiting
 * queue so that the batch shares adapters (host code; no device work, no
 * stream).  Source: "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A",
 * "The adapter-aware scheduler" (group the queue by adapter, biggest groups
 * first and whole where possible, and admit no new adapter once the batch
 * holds max_distinct adapters and at least min_batch requests) and "The
 * fairness cost, which must be stated" (an age override); "The Revision", R1
 * (slots reserved for the long tail); "12. Adapter Serving and Multi-Tenant
 * Customization", "Batching across adapters" (base-only requests are a group
 * of their own).  The batch, in order:
 *   1. urgent: every request with waited_ms[i] > max_wait_ms, oldest first
 *      (skipped when waited_ms is NULL);
 *   2. tail: the oldest requests (at most min(reserved_tail, max_distinct))
 *      whose adapter has no other request among those not yet taken;
 *      base-only requests never take a tail slot;
 *   3. grouped fill of the rest: groups by adapter (all base-only requests
 *      form one group), in descending size, equal sizes in the order of their
 *      oldest request, members oldest first, a group cut only where the batch
 *      fills.  Before each group: stop if the batch is full, or if the fill has
 *      admitted (max_distinct - tail) adapter groups and the whole batch holds
 *      at least min_batch requests.  The base-only group counts against no
 *      budget.  Whenever min_batch <= max_distinct, steps 2 and 3 together
 *      admit at most max_distinct adapters.
 *
 *   adapters       host int32 [queue_len]: adapter slot of each waiting
 *                  request, oldest first; negative = base only
 *   queue_len      >= 0
 *   waited_ms      host float [queue_len] or NULL; max_wait_ms its deadline
 *   max_batch      >= 1: most requests chosen
 *   max_distinct   >= 0: adapter budget of steps 2 and 3
 *   min_batch      >= 0
 *   reserved_tail  >= 0
 *   out_index      host int32 [min(max_batch, queue_len)] (at least 1):
 *                  queue positions of the chosen requests, in batch order
 *   out_count      host int32 *: number chosen
 *
 * Errors: LORA_ERR_NULL (a needed pointer is NULL), LORA_ERR_SHAPE (a count
 * out of range); nothing is written then.
 */
lora_status_t lora_form_batch(const int32_t *adapters, int32_t queue_len,
                              const float *waited_ms, float max_wait_ms,
                              int32_t max_batch, int32_t max_distinct,
                              int32_t min_batch, int32_t reserved_tail,
                              int32_t *out_index, int32_t *out_count);

/* Size of the static device array that lora_apply_layer_noalloc uses as its
 * workspace (16 MiB on every device the library runs on, held until the
 * process ends). */
#define LORA_STATIC_SCRATCH_BYTES (16u << 20)

/*
 * lora_apply_layer_noalloc -- lora_apply_layer without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * k-chunk partials go to a static device array of LORA_STATIC_SCRATCH_BYTES
 * instead; the call itself allocates nothing.  Same arguments (less ws and
 * ws_bytes), same kernels, same results and the same errors as
 * lora_apply_layer, except that a call whose workspace would exceed
 * LORA_STATIC_SCRATCH_BYTES (lora_workspace_bytes with these sizes) returns
 * LORA_ERR_SCRATCH and enqueues nothing.  At 128 rows and rank 64 the array
 * holds every projection of the 70B layer (2.7 MB).
 * The array is per device and shared by every call on that device: calls
 * that may overlap on one device (other streams, other host threads) race
 * on it and must be ordered by the caller.  Nothing in it needs to start at
 * zero; a call leaves its partials there.  The first call on a device looks
 * up the array's device address (with that device current) and keeps it;
 * LORA_ERR_LAUNCH if the lookup fails.
 */
lora_status_t lora_apply_layer_noalloc(const lora_module_io_t *io, uint32_t module_mask,
                                       int32_t num_rows, const lora_adapter_entry_t *table,
                                       int32_t num_slots, lora_segments_t seg, int32_t max_rank,
                                       void *stream);

/* A static, human-readable name for a status code. */
const char *lora_status_string(lora_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* LORA_GEMV_H */
