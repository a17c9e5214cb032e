// Internal declarations of the gfx950 LoRA-delta library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_gemv.h"

namespace lora {

// Segment builder: one block handles up to kSegSmallMax rows; beyond it the
// rows are cut into chunks of kSegChunk rows and three kernels run.
constexpr int kSegSmallMax = 1024;
constexpr int kSegChunk = 256;

// Decode shrink: k-chunk per work item (the workspace is sized for the
// smallest chunk the host may pick).
constexpr int kKChunkMin = 1024;
constexpr int kMaxModules = LORA_NUM_MODULES;

// Segments of at least this many rows go to the matrix-core (SGMV) kernels;
// shorter ones to the decode kernels.
constexpr int kLongSegRows = 8;
// Rows per SGMV block: shrink 4 waves x 2 tiles of 16, expand 4 tiles of 16
// (all in every wave).  The segment builder counts the tiles of these sizes.
constexpr int kSgmvShrinkRows = 128;
constexpr int kSgmvExpandRows = 64;
// Batches of at least this many rows use a larger shrink k-chunk.
constexpr int kPrefillRows = 2048;
// Output columns per SGMV expand block (the most a block stages for): in
// batches of fewer than kPrefillRows rows, whose long segments give few row
// tiles, half of that, so the launch has more blocks (measured 13-19%
// faster on the expand of 256-row Zipf batches; the same at 256 columns).
// Prefill batches: 1024 columns measured 2-5% faster than 2048 (each block
// re-sums its rows' k-chunk partials, but more blocks per row tile keep more
// of the y read-modify-write in flight); 512 and 4096 were slower.
constexpr int kSgmvExpandCols = 1024;
constexpr int kSgmvExpandColsSmall = 512;

// Threads per block of the decode kernels: 4 waves of 64.
constexpr int kDecodeThreads = 256;
// Decode expand n-tile (outputs per item) for LPR = rank class / 8 lanes per
// output row: 2048 at rank 64, 4096 below (whole sub-tiles of 16 load passes;
// the item's sums fit in LDS).
constexpr int decode_expand_tile(int lpr) { return lpr >= 8 ? 2048 : 4096; }
// Rows staged in LDS per group by the decode expand.
constexpr int kExpandRowGroup = 16;

// One projection as the kernels see it.
struct ModuleDesc {
  const uint16_t *x;
  int64_t ldx;
  uint16_t *y;
  int64_t ldy;
  int32_t d_in;
  int32_t d_out;
  int32_t col;        // table column
  int32_t item_base;  // first work item of this module inside a segment
  int32_t n_items;    // k-chunks (shrink) or n-tiles (expand)
  int32_t part_base;  // first partial chunk of this module
  int32_t n_chunks;   // k-chunks of this module
  int32_t sg_item_base;  // first SGMV expand item (n-tile) of this module in a row tile
  int32_t sg_n_items;    // SGMV expand n-tiles of this module
  int32_t op_nt;         // one-launch decode: outputs per expand tile
  int32_t op_n_tiles;    // one-launch decode: expand tiles of this module
};

// Everything a decode kernel needs, passed by value.
struct LayerDesc {
  ModuleDesc mod[kMaxModules];
  int32_t n_active;       // modules in use (mod[0..n_active))
  int32_t items_per_seg;  // sum of n_items over modules
  int32_t table_cols;     // n_mod of the table
  int32_t kc;             // shrink k-chunk
  int32_t nt;             // expand n-tile
  int32_t rs;             // floats per row of a partial chunk
  int32_t num_rows;
  int32_t num_slots;
  int32_t max_rank;
  int32_t long_min;       // segments with at least this many rows: SGMV path
  int32_t max_seg;        // segments the grid covers: min(rows, slots, the caller's bound)
  int32_t sg_items;       // SGMV expand items (n-tiles over all modules) per row tile
  int32_t sg_nt;          // SGMV expand n-tile
  int32_t count_errors;   // whether this launch adds the segment and entry errors to the status word
  const int32_t *perm;
  const int32_t *seg_offsets;
  const int32_t *seg_adapter;
  const int32_t *num_segments;
  const int32_t *tile_counts;  // SGMV tiles of the build: [0] shrink, [1] expand
  int32_t *status;
  const lora_adapter_entry_t *table;
  float *part;            // partials [chunks][num_rows][rs]
  // expand source when v comes from the caller (lora_expand): v[b][j]
  const float *v;
  int64_t ldv;
  // shrink destination when v goes to the caller (lora_shrink reduce)
  float *v_out;
};

// Fused base projection + delta: a block computes y for kFusedRows rows and
// fused_cols(q4) output columns of one projection.
constexpr int kFusedRows = 128;
// Output columns of a block, with either base: 128 (against 64, half the x
// read from L2 per byte of W; the 4-bit kernel holds its group sums beside
// the accumulators at the cost of a few spilled registers).
constexpr int fused_cols(bool) { return 128; }

// 4-bit base weights: inputs per scale (a group of consecutive inputs of one
// output row); the fused kernel's two 64-k rounds per main-loop step make one.
constexpr int kQ4Group = LORA_Q4_GROUP;
static_assert(kQ4Group == 128, "the fused kernel scales one group per two 64-k rounds");

struct FusedModule {
  const uint16_t *x;  // [num_rows][ldx]
  int64_t ldx;
  const void *W;      // bf16 base weight [d_out][ldw] elements, or 4-bit [d_out][ldw] bytes
  int64_t ldw;
  const float *Ws;    // 4-bit base weight: fp32 group scales [d_out][ldws]
  int64_t ldws;
  uint16_t *y;        // [num_rows][ldy], written
  int64_t ldy;
  const float *v;     // [num_rows][rs]: the row's unscaled rank-r vector
  int32_t d_in;
  int32_t d_out;
  int32_t col;         // table column
  int32_t block_base;  // first block of this module
  int32_t n_tiles;     // column tiles of fused_cols(q4)
};

struct FusedDesc {
  FusedModule mod[kMaxModules];
  int32_t n_active;
  int32_t num_rows;
  int32_t num_slots;
  int32_t table_cols;
  int32_t max_rank;
  int32_t rs;          // floats per row of v
  const int32_t *ids;  // the rows' adapter slots, original order
  int32_t *status;
  const lora_adapter_entry_t *table;
  // the segments of the build: a row's delta applies only when its slot has
  // one (the builder may have dropped slots past the caller's bound)
  const int32_t *num_segments;
  const int32_t *seg_adapter;
  int32_t max_seg;
};

// q4: the base weights of every projection are 4-bit with group scales.
hipError_t launch_fused(const FusedDesc &f, bool q4, int blocks, hipStream_t stream);

// ---- One-launch decode (lora_decode_layer on batches of distinct
// adapters): the grouping of the rows, the shrink and the expand of every
// projection in one launch, with no hand-off between blocks.  Rows it takes
// at most (one row per thread of a block).
constexpr int kOnePassMaxRows = 256;
// Slot ids a block can rank against the caller's segment bound (a bitmap in
// LDS); a batch whose bound may drop segments takes the one-launch path only
// with at most this many slots.
constexpr int kOnePassMaxSlots = 8192;
// Expand tile of a block: kOnePassPasses load passes of the block over B
// (rank/8 lanes per output row, 256 lanes).  16 passes measured faster than
// 8 (the blocks of one segment each read its whole A: fewer, larger tiles
// read it fewer times): 17.1 against 24.4 us for 128 rows x 8192 at rank 16.
constexpr int kOnePassPasses = 16;

struct OnePassDesc {
  LayerDesc L;               // first member: kernel_desc() reads it from the kernel arguments
  lora_segments_t seg;       // written by the grid's last block
  const int32_t *ids;        // [num_rows] adapter slot of each row
  int32_t row_slots;         // rows per item of the grid: num_rows rounded up to a multiple of 8
  int32_t bound_check;       // the caller's segment bound may drop segments: blocks rank their slot
  int32_t tiles_per_block;   // consecutive expand tiles of one block (one shrink each)
};

hipError_t launch_onepass(const OnePassDesc &d, int grid, hipStream_t stream);

inline int round_up(int a, int b) { return (a + b - 1) / b * b; }
inline int partial_row_stride(int max_rank) { return round_up(max_rank, 8); }

size_t segments_ws_bytes(int num_rows, int num_slots);
size_t partials_ws_bytes(int num_rows, int max_rank, int64_t sum_d_in);

// Row b's id is ids[b * stride]; add_status adds the bad ids to the status
// word instead of setting it.
hipError_t launch_build_segments(const int32_t *ids, int stride, int n, int num_slots, bool add_status,
                                 const lora_segments_t &seg, void *ws, hipStream_t stream);
hipError_t launch_shrink_reduce(const LayerDesc &d, hipStream_t stream);
// Sum each row's k-chunk partials into its first chunk, for every module.
hipError_t launch_fold_partials(const LayerDesc &d, hipStream_t stream);
// One launch per phase: blocks [0, decode_blocks) take decode items, the
// rest SGMV row tiles.
hipError_t launch_shrink(const LayerDesc &d, int decode_blocks, int grid, hipStream_t stream);
hipError_t launch_expand(const LayerDesc &d, int decode_blocks, int grid, hipStream_t stream);

int long_tiles_max(int num_rows, int max_seg, int rows_per_tile);
int sgmv_shrink_rows();
int sgmv_expand_rows();

}  // namespace lora
