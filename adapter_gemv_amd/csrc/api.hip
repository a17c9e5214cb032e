// C ABI of the LoRA-delta library: argument checks, work decomposition and
// launches.  Every check runs before the first HIP call, so a rejected call
// touches neither the device nor the stream.
#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "lora_internal.h"

using namespace lora;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

lora_status_t check_segments(const lora_segments_t &seg) {
  if (!seg.perm || !seg.seg_offsets || !seg.seg_adapter || !seg.num_segments || !seg.status || !seg.tile_counts)
    return LORA_ERR_NULL;
  if (seg.max_segments < 0) return LORA_ERR_SHAPE;
  return LORA_OK;
}

// The most segments a batch can have: one per row, one per slot, and the
// caller's bound when it gives one.
int segment_bound(int num_rows, int num_slots, const lora_segments_t &seg) {
  int b = num_rows < num_slots ? num_rows : num_slots;
  if (seg.max_segments > 0 && seg.max_segments < b) b = seg.max_segments;
  return b;
}

size_t ws_need(int num_rows, int num_slots, int max_rank, int64_t sum_d_in) {  // covers every call
  const size_t a = segments_ws_bytes(num_rows, num_slots);
  const size_t b = partials_ws_bytes(num_rows, max_rank, sum_d_in);
  return a > b ? a : b;
}

// The workspace checks of a call whose own scratch is `need` bytes (0: the
// call needs no workspace and *scratch is null).
lora_status_t check_ws(void *ws, size_t ws_bytes, size_t need, void **scratch) {
  *scratch = nullptr;
  if (need == 0) return LORA_OK;
  if (!ws) return LORA_ERR_NULL;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  if (ws_bytes < need) return LORA_ERR_WORKSPACE;
  *scratch = ws;
  return LORA_OK;
}

struct ModuleArgs {
  const void *x;
  int64_t ldx;
  void *y;
  int64_t ldy;
  int32_t d_in;
  int32_t d_out;
  int32_t col;
  bool int8_items = false;  // the call's LORA_MASK_INT8_ITEMS: items sized for one-byte factors
};

// Work decomposition: the n-tile of the decode expand.  An item takes the
// largest tile the kernel stages in LDS (2048 outputs at rank class 64, 4096
// below: 256 KiB of bf16 B at the class's rank, half that in int8, where the
// fixed cost of an item weighs more); batches that would give fewer than 1024
// items take smaller tiles (down to one sub-tile of 16 load passes), so the
// work spreads over the device.  Measured on the Zipf batch of 101 adapters
// of mixed rank (q/k/v/o, rank class 64): 512-output tiles 39.7 us, 1024
// 33.9 us, 2048 40.8 us, which a threshold of 2048, 1024 and 512 items
// gives.
int pick_nt(int max_rank, int64_t max_seg, const ModuleArgs *ms, int n) {
  const int cls = max_rank <= 8 ? 8 : max_rank <= 16 ? 16 : max_rank <= 32 ? 32 : 64;
  const int lpr = cls / 8;
  const int sub = 16 * kDecodeThreads / lpr;
  int nt = decode_expand_tile(lpr);
  if (nt < sub) nt = sub;
  while (nt > sub) {
    int64_t items = 0;
    for (int i = 0; i < n; ++i) items += (ms[i].d_out + nt - 1) / nt;
    if (max_seg * items >= 1024) break;
    nt /= 2;
  }
  return nt;
}

// Fill the descriptor for a set of modules; items are k-chunks (shrink) or
// n-tiles (expand).
lora_status_t launched(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_ERR_LAUNCH; }

// Shrink k-chunk.  Prefill-sized batches: 2 * kKChunkMin (fewer partials to
// write and sum).  Decode batches: about 128 KiB of A per item at the
// launch's rank class (1024 k at rank 64, longer below; four times the k,
// at most 4 * kKChunkMin, when the caller states int8 factors,
// LORA_MASK_INT8_ITEMS), halved while the batch would give fewer than 512
// items, never below kKChunkMin (the workspace is sized for that chunk).
// Measured on the 70B layer at rank 64 with int8 factors: shrink 137 -> 109
// us with 2048 k instead of 1024, and 106 -> 102 us with 4096 (and bf16
// factors 186 -> 196 us at 2048: the hint is the caller's).
int pick_kc(int num_rows, int max_rank, int64_t max_seg, const ModuleArgs *ms, int n) {
  if (num_rows >= kPrefillRows) return 2 * kKChunkMin;
  const int cls = max_rank <= 8 ? 8 : max_rank <= 16 ? 16 : max_rank <= 32 ? 32 : 64;
  int kc = kKChunkMin * (64 / cls) * (n > 0 && ms[0].int8_items ? 4 : 1);
  if (kc > 4 * kKChunkMin) kc = 4 * kKChunkMin;
  while (kc > kKChunkMin) {
    int64_t items = 0;
    for (int i = 0; i < n; ++i) items += (ms[i].d_in + kc - 1) / kc;
    if (max_seg * items >= 512) break;
    kc /= 2;
  }
  return kc;
}

// Fill the descriptor: items per segment are k-chunks (shrink) or decode
// n-tiles (expand); sg_* give the SGMV expand n-tiles per row tile.
void fill_desc(LayerDesc &d, const ModuleArgs *ms, int n, bool shrink, int num_rows, int num_slots, int max_rank,
               int table_cols, const lora_adapter_entry_t *table, const lora_segments_t &seg, void *ws) {
  d = LayerDesc{};
  const int max_seg = segment_bound(num_rows, num_slots, seg);
  d.kc = pick_kc(num_rows, max_rank, max_seg, ms, n);
  d.nt = pick_nt(max_rank, max_seg, ms, n);
  d.sg_nt = num_rows >= kPrefillRows ? kSgmvExpandCols : kSgmvExpandColsSmall;
  int item = 0, chunk = 0, sg = 0;
  for (int i = 0; i < n; ++i) {
    ModuleDesc &m = d.mod[i];
    m.x = static_cast<const uint16_t *>(ms[i].x);
    m.ldx = ms[i].ldx;
    m.y = static_cast<uint16_t *>(ms[i].y);
    m.ldy = ms[i].ldy;
    m.d_in = ms[i].d_in;
    m.d_out = ms[i].d_out;
    m.col = ms[i].col;
    m.n_chunks = m.d_in > 0 ? (m.d_in + d.kc - 1) / d.kc : 0;
    m.part_base = chunk;
    chunk += m.n_chunks;
    m.n_items = shrink ? m.n_chunks : (m.d_out + d.nt - 1) / d.nt;
    m.item_base = item;
    item += m.n_items;
    m.sg_n_items = (m.d_out + d.sg_nt - 1) / d.sg_nt;
    m.sg_item_base = sg;
    sg += m.sg_n_items;
  }
  d.n_active = n;
  d.items_per_seg = item;
  d.sg_items = sg;
  d.table_cols = table_cols;
  d.rs = partial_row_stride(max_rank);
  d.num_rows = num_rows;
  d.num_slots = num_slots;
  d.max_rank = max_rank;
  d.long_min = num_rows >= kLongSegRows ? kLongSegRows : 0x7fffffff;
  d.max_seg = max_seg;
  d.perm = seg.perm;
  d.seg_offsets = seg.seg_offsets;
  d.seg_adapter = seg.seg_adapter;
  d.num_segments = seg.num_segments;
  d.tile_counts = seg.tile_counts;
  d.status = seg.status;
  d.table = table;
  d.part = static_cast<float *>(ws);
}

// The SGMV kernels address an activation matrix with 32-bit byte offsets.
bool fits_u32(int64_t rows, int64_t ld) { return rows * ld * 2 <= (int64_t)0xFFFFFF00; }

// A prefill batch's partials are summed once into their first chunk after
// the shrink (fold_partials_kernel): every SGMV expand tile of a row tile
// (d_out / 1024 of them per projection) would otherwise sum all the chunks
// again, and the tiles of one row tile run on different XCDs, so each
// fetches them from HBM.
bool folds_partials(const LayerDesc &d) {
  if (d.num_rows < kPrefillRows) return false;
  for (int i = 0; i < d.n_active; ++i)
    if (d.mod[i].n_chunks > 1) return true;
  return false;
}

// Launch one phase (shrink or expand) over every module: decode items for
// every possible segment and SGMV items for every row tile that segments of
// at least kLongSegRows rows can produce (the kernels put the tiles the
// build counted first and let the rest of that room exit).  fold: the
// phase's partials pass from this call's shrink to its expand (not to a
// caller's v or the fused kernel's planes), so a prefill batch folds them.
lora_status_t launch_phase(bool shrink, const ModuleArgs *ms, int n, int num_rows, int num_slots, int max_rank,
                           int table_cols, const lora_adapter_entry_t *table, const lora_segments_t &seg, void *ws,
                           const float *v_in, int64_t ldv, hipStream_t s, bool fold = false) {
  LayerDesc d;
  fill_desc(d, ms, n, shrink, num_rows, num_slots, max_rank, table_cols, table, seg, ws);
  d.v = v_in;
  d.ldv = ldv;
  const bool folded = fold && v_in == nullptr && folds_partials(d);
  if (folded && !shrink)
    for (int i = 0; i < n; ++i) d.mod[i].n_chunks = 1;  // the sums wait in each module's first chunk
  // a call counts each bad segment and entry once: the shrink of a layer call,
  // or lora_expand on the caller's v
  d.count_errors = shrink || v_in != nullptr;
  const int64_t dec = (int64_t)d.max_seg * d.items_per_seg;
  int64_t sg = 0;
  if (num_rows >= kLongSegRows)
    sg = (int64_t)long_tiles_max(num_rows, d.max_seg, shrink ? sgmv_shrink_rows() : sgmv_expand_rows()) *
         (shrink ? d.items_per_seg : d.sg_items);
  if (dec + sg > 0x7fffffff) return LORA_ERR_SHAPE;
  const hipError_t e = shrink ? launch_shrink(d, (int)dec, (int)(dec + sg), s) : launch_expand(d, (int)dec, (int)(dec + sg), s);
  const lora_status_t st = launched(e);
  if (st != LORA_OK || !(folded && shrink)) return st;
  return launched(launch_fold_partials(d, s));
}

// Common checks of the layer calls; fills the module list.
lora_status_t check_layer(const lora_module_io_t *io, uint32_t module_mask, int32_t num_rows,
                          const lora_adapter_entry_t *table, int32_t num_slots, const lora_segments_t &seg,
                          int32_t max_rank, void *ws, size_t ws_bytes, ModuleArgs *ms, int *n_out,
                          void **scratch, int64_t *sum_d_in_out = nullptr) {
  if (!io || !table) return LORA_ERR_NULL;
  lora_status_t st = check_segments(seg);
  if (st != LORA_OK) return st;
  const bool int8_items = (module_mask & LORA_MASK_INT8_ITEMS) != 0;
  module_mask &= ~LORA_MASK_INT8_ITEMS;
  if (module_mask == 0 || module_mask >= (1u << LORA_NUM_MODULES)) return LORA_ERR_MODULE;
  if (num_rows < 0 || num_slots < 1) return LORA_ERR_SHAPE;
  if (max_rank < 1 || max_rank > LORA_MAX_RANK) return LORA_ERR_RANK;
  int n = 0;
  int64_t sum_d_in = 0;
  for (int c = 0; c < LORA_NUM_MODULES; ++c) {
    if (!(module_mask & (1u << c))) continue;
    const lora_module_io_t &m = io[c];
    if (!m.x || !m.y) return LORA_ERR_NULL;
    if (m.d_in <= 0 || m.d_out <= 0 || m.ldx < m.d_in || m.ldy < m.d_out) return LORA_ERR_SHAPE;
    if ((m.d_in & 7) || (m.d_out & 7) || (m.ldx & 7) || (m.ldy & 7) || !aligned16(m.x) || !aligned16(m.y))
      return LORA_ERR_ALIGN;
    if (!fits_u32(num_rows, m.ldx) || !fits_u32(num_rows, m.ldy)) return LORA_ERR_SHAPE;
    ms[n] = ModuleArgs{m.x, m.ldx, m.y, m.ldy, m.d_in, m.d_out, c, int8_items};
    sum_d_in += m.d_in;
    ++n;
  }
  st = check_ws(ws, ws_bytes, partials_ws_bytes(num_rows, max_rank, sum_d_in), scratch);
  if (st != LORA_OK) return st;
  *n_out = n;
  if (sum_d_in_out) *sum_d_in_out = sum_d_in;
  return LORA_OK;
}

lora_status_t layer_phase(bool do_shrink, bool do_expand, const lora_module_io_t *io, uint32_t module_mask,
                          int32_t num_rows, const lora_adapter_entry_t *table, int32_t num_slots,
                          lora_segments_t seg, int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  ModuleArgs ms[LORA_NUM_MODULES];
  int n = 0;
  void *scratch = nullptr;
  lora_status_t st =
      check_layer(io, module_mask, num_rows, table, num_slots, seg, max_rank, ws, ws_bytes, ms, &n, &scratch);
  if (st != LORA_OK) return st;
  if (num_rows == 0) return LORA_OK;
  ws = scratch;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (do_shrink) {
    st = launch_phase(true, ms, n, num_rows, num_slots, max_rank, LORA_NUM_MODULES, table, seg, ws, nullptr, 0, s,
                      true);
    if (st != LORA_OK) return st;
  }
  if (do_expand)
    st = launch_phase(false, ms, n, num_rows, num_slots, max_rank, LORA_NUM_MODULES, table, seg, ws, nullptr, 0, s,
                      true);
  return st;
}

}  // namespace

extern "C" {

size_t lora_workspace_bytes(int32_t num_rows, int32_t num_slots, int32_t max_rank, int64_t sum_d_in) {
  if (num_rows < 0 || num_slots < 1 || max_rank < 1 || max_rank > LORA_MAX_RANK || sum_d_in < 0) return 0;
  return ws_need(num_rows, num_slots, max_rank, sum_d_in);
}

// The fused layer's workspace: the shrink's partials, then one v plane
// [num_rows][rs] per projection (256-byte aligned); at least the segment
// builder's.
size_t lora_linear_workspace_bytes(int32_t num_rows, int32_t num_slots, int32_t max_rank, int64_t sum_d_in,
                                   int32_t n_modules) {
  if (num_rows < 0 || num_slots < 1 || max_rank < 1 || max_rank > LORA_MAX_RANK || sum_d_in < 0 || n_modules < 1 ||
      n_modules > LORA_NUM_MODULES)
    return 0;
  const size_t part = (partials_ws_bytes(num_rows, max_rank, sum_d_in) + 255) & ~(size_t)255;
  const size_t vplanes = (size_t)n_modules * num_rows * partial_row_stride(max_rank) * 4;
  const size_t seg = segments_ws_bytes(num_rows, num_slots);
  return part + vplanes > seg ? part + vplanes : seg;
}

lora_status_t lora_build_segments(const int32_t *row_adapter, int32_t num_rows, int32_t num_slots,
                                  lora_segments_t seg, void *ws, size_t ws_bytes, void *stream) {
  lora_status_t st = check_segments(seg);
  if (st != LORA_OK) return st;
  if (num_rows < 0 || num_slots < 1) return LORA_ERR_SHAPE;
  if (num_rows > 0 && !row_adapter) return LORA_ERR_NULL;
  void *scratch = nullptr;
  st = check_ws(ws, ws_bytes, segments_ws_bytes(num_rows, num_slots), &scratch);
  if (st != LORA_OK) return st;
  return launched(launch_build_segments(row_adapter, 1, num_rows, num_slots, false, seg, scratch,
                                        static_cast<hipStream_t>(stream)));
}

lora_status_t lora_shrink(const void *x, int64_t ldx, int32_t num_rows, int32_t d_in,
                          const lora_adapter_entry_t *table, int32_t num_slots, int32_t n_mod, int32_t module,
                          lora_segments_t seg, int32_t max_rank, float *v, int64_t ldv, void *ws, size_t ws_bytes,
                          void *stream) {
  if (!x || !table || !v) return LORA_ERR_NULL;
  lora_status_t st = check_segments(seg);
  if (st != LORA_OK) return st;
  if (n_mod < 1 || n_mod > LORA_NUM_MODULES || module < 0 || module >= n_mod) return LORA_ERR_MODULE;
  if (max_rank < 1 || max_rank > LORA_MAX_RANK) return LORA_ERR_RANK;
  if (num_rows < 0 || num_slots < 1 || d_in <= 0 || ldx < d_in || ldv < max_rank) return LORA_ERR_SHAPE;
  if ((d_in & 7) || (ldx & 7) || (ldv & 3) || !aligned16(x) || !aligned16(v)) return LORA_ERR_ALIGN;
  if (!fits_u32(num_rows, ldx)) return LORA_ERR_SHAPE;
  void *scratch = nullptr;
  st = check_ws(ws, ws_bytes, partials_ws_bytes(num_rows, max_rank, d_in), &scratch);
  if (st != LORA_OK) return st;
  if (num_rows == 0) return LORA_OK;
  ws = scratch;
  ModuleArgs m{x, ldx, nullptr, 0, d_in, 0, module};
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_phase(true, &m, 1, num_rows, num_slots, max_rank, n_mod, table, seg, ws, nullptr, 0, s);
  if (st != LORA_OK) return st;
  LayerDesc d;
  fill_desc(d, &m, 1, true, num_rows, num_slots, max_rank, n_mod, table, seg, ws);
  d.v_out = v;
  d.ldv = ldv;
  return launched(launch_shrink_reduce(d, s));
}

lora_status_t lora_expand(const float *v, int64_t ldv, int32_t num_rows, int32_t d_out,
                          const lora_adapter_entry_t *table, int32_t num_slots, int32_t n_mod, int32_t module,
                          lora_segments_t seg, int32_t max_rank, void *y, int64_t ldy, void *ws, size_t ws_bytes,
                          void *stream) {
  if (!v || !table || !y) return LORA_ERR_NULL;
  lora_status_t st = check_segments(seg);
  if (st != LORA_OK) return st;
  if (n_mod < 1 || n_mod > LORA_NUM_MODULES || module < 0 || module >= n_mod) return LORA_ERR_MODULE;
  if (max_rank < 1 || max_rank > LORA_MAX_RANK) return LORA_ERR_RANK;
  if (num_rows < 0 || num_slots < 1 || d_out <= 0 || ldy < d_out || ldv < max_rank) return LORA_ERR_SHAPE;
  if ((d_out & 7) || (ldy & 7) || (ldv & 3) || !aligned16(y) || !aligned16(v)) return LORA_ERR_ALIGN;
  if (!fits_u32(num_rows, ldy)) return LORA_ERR_SHAPE;
  (void)ws;
  (void)ws_bytes;  // the expand of a caller-provided v needs no workspace
  if (num_rows == 0) return LORA_OK;
  ModuleArgs m{nullptr, 0, y, ldy, 0, d_out, module};
  return launch_phase(false, &m, 1, num_rows, num_slots, max_rank, n_mod, table, seg, ws, v, ldv,
                      static_cast<hipStream_t>(stream));
}

lora_status_t lora_layer_shrink(const lora_module_io_t *io, uint32_t module_mask, int32_t num_rows,
                                const lora_adapter_entry_t *table, int32_t num_slots, lora_segments_t seg,
                                int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  return layer_phase(true, false, io, module_mask, num_rows, table, num_slots, seg, max_rank, ws, ws_bytes, stream);
}

lora_status_t lora_layer_expand(const lora_module_io_t *io, uint32_t module_mask, int32_t num_rows,
                                const lora_adapter_entry_t *table, int32_t num_slots, lora_segments_t seg,
                                int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  return layer_phase(false, true, io, module_mask, num_rows, table, num_slots, seg, max_rank, ws, ws_bytes, stream);
}

lora_status_t lora_apply_layer(const lora_module_io_t *io, uint32_t module_mask, int32_t num_rows,
                               const lora_adapter_entry_t *table, int32_t num_slots, lora_segments_t seg,
                               int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  return layer_phase(true, true, io, module_mask, num_rows, table, num_slots, seg, max_rank, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// The one-launch plan of lora_decode_layer.  Each block of the one-launch
// kernel reads the whole A of its segment (its siblings, one per group of
// expand tiles, read the same lines through L2), so the plan bounds those
// repeated reads: at most kOnePassRepeatBytes over all projections, counting
// one pass over A per block of a segment and one more per 4 further rows
// (segments are at most the caller's bound, else one per row).  Measured on
// one MI355X (steps replayed from a HIP graph, one projection d x d, a
// distinct adapter per row, 16 to 256 rows, d 1024 to 8192, ranks 8 to 32):
// the launch beats the three launches of lora_build_segments +
// lora_apply_layer everywhere, by 2-3x up to 64 rows (4-9 us against 12-16
// us), 18.9 against 27.4 us for 128 rows x 8192 at rank 16, 39 against 42 us
// for 128 rows x 8192 at rank 32 (268 MB of repeated reads), and ties at the
// same 268 MB with 256 rows.  Batches of at most kOnePassMaxRows rows, ranks
// up to 32.  False for any other batch.
constexpr double kOnePassRepeatBytes = 320.0 * (1 << 20);
// Tiles per block grow while the blocks that work (one per row group and
// item) stay at least this many and the widest projection keeps at least
// two blocks per row group: every block of a group reads its A, so fewer
// blocks read A fewer times, until too few blocks share a row's tiles.
// Measured (graph-timed, a distinct adapter per row, 8192 x 8192): rank 32
// at 128 rows 39.5 us with 4 blocks per row, 32.0 with 2; rank 16 at 128
// rows 19.6 with 4, 19.1 with 2, 23.6 with 1 (bench); 256 rows of rank 16 at
// 4096 x 4096 14.9 with 2, 15.7 with 1; 128 rows over 32 adapters at rank 16
// 20.7 with 4 (128 working blocks), 24.7 with 2.
constexpr int64_t kOnePassMinWorking = 256;

bool onepass_plan(const ModuleArgs *ms, int n, int num_rows, const int32_t *ids, int num_slots, int max_rank,
                  const lora_adapter_entry_t *table, const lora_segments_t &seg, OnePassDesc *od, int *grid) {
  if (num_rows < 1 || num_rows > kOnePassMaxRows || max_rank > 32) return false;
  const int lpr = max_rank <= 8 ? 1 : max_rank <= 16 ? 2 : 4;
  const int nt = kOnePassPasses * (kDecodeThreads / lpr);
  const int max_seg = segment_bound(num_rows, num_slots, seg);
  // a bound below min(rows, slots) may drop segments: each block then ranks its slot in a bitmap of the slots
  const bool bound_check = max_seg < (num_rows < num_slots ? num_rows : num_slots);
  if (bound_check && num_slots > kOnePassMaxSlots) return false;
  const double passes = max_seg + (num_rows - max_seg + 3) / 4;
  // tiles per block (each block reads its segment's A once for all its tiles)
  auto items = [&](int tpb) {
    int64_t it = 0;
    for (int i = 0; i < n; ++i) it += ((ms[i].d_out + nt - 1) / nt + tpb - 1) / tpb;
    return it;
  };
  auto widest = [&](int tpb) {  // items of the projection with the most tiles
    int64_t w = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t it = ((ms[i].d_out + nt - 1) / nt + tpb - 1) / tpb;
      w = it > w ? it : w;
    }
    return w;
  };
  int tpb = 1;
  while (tpb < 64 && items(2 * tpb) < items(tpb) && widest(2 * tpb) >= 2 &&
         items(2 * tpb) * passes >= kOnePassMinWorking)
    tpb *= 2;
  double repeat = 0;
  for (int i = 0; i < n; ++i)
    repeat += (double)(((ms[i].d_out + nt - 1) / nt + tpb - 1) / tpb) * ms[i].d_in * (8 * lpr) * 2 * passes;
  if (repeat > kOnePassRepeatBytes) return false;
  *od = OnePassDesc{};
  LayerDesc &d = od->L;
  d.nt = nt;
  int item = 0;
  for (int i = 0; i < n; ++i) {
    ModuleDesc &m = d.mod[i];
    m.x = static_cast<const uint16_t *>(ms[i].x);
    m.ldx = ms[i].ldx;
    m.y = static_cast<uint16_t *>(ms[i].y);
    m.ldy = ms[i].ldy;
    m.d_in = ms[i].d_in;
    m.d_out = ms[i].d_out;
    m.col = ms[i].col;
    m.op_nt = nt;
    m.op_n_tiles = (m.d_out + nt - 1) / nt;
    m.n_items = (m.op_n_tiles + tpb - 1) / tpb;
    m.item_base = item;
    item += m.n_items;
  }
  d.n_active = n;
  d.items_per_seg = item;
  d.table_cols = LORA_NUM_MODULES;
  d.num_rows = num_rows;
  d.num_slots = num_slots;
  d.max_rank = max_rank;
  d.long_min = 0x7fffffff;
  d.max_seg = segment_bound(num_rows, num_slots, seg);
  d.status = seg.status;
  d.table = table;
  od->seg = seg;
  od->ids = ids;
  od->row_slots = (num_rows + 7) / 8 * 8;
  od->bound_check = bound_check;
  od->tiles_per_block = tpb;
  const int64_t blocks = (int64_t)item * od->row_slots + 1;
  if (blocks > 0x7fffffff) return false;
  *grid = (int)blocks;
  return true;
}

}  // namespace

extern "C" {

// Segments and the layer delta of a decode batch: one launch when the batch
// fits the one-launch kernel, else lora_build_segments + lora_apply_layer.
lora_status_t lora_decode_layer(const lora_module_io_t *io, uint32_t module_mask, int32_t num_rows,
                                const int32_t *row_adapter, const lora_adapter_entry_t *table, int32_t num_slots,
                                lora_segments_t seg, int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  ModuleArgs ms[LORA_NUM_MODULES];
  int n = 0;
  void *scratch = nullptr;
  lora_status_t st =
      check_layer(io, module_mask, num_rows, table, num_slots, seg, max_rank, ws, ws_bytes, ms, &n, &scratch);
  if (st != LORA_OK) return st;
  if (num_rows > 0 && !row_adapter) return LORA_ERR_NULL;
  void *seg_scratch = nullptr;
  st = check_ws(ws, ws_bytes, segments_ws_bytes(num_rows, num_slots), &seg_scratch);
  if (st != LORA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  OnePassDesc od;
  int grid = 0;
  if (onepass_plan(ms, n, num_rows, row_adapter, num_slots, max_rank, table, seg, &od, &grid))
    return launched(launch_onepass(od, grid, s));
  st = launched(launch_build_segments(row_adapter, 1, num_rows, num_slots, false, seg, seg_scratch, s));
  if (st != LORA_OK || num_rows == 0) return st;
  // the three-launch path
  st = launch_phase(true, ms, n, num_rows, num_slots, max_rank, LORA_NUM_MODULES, table, seg, scratch, nullptr, 0, s,
                    true);
  if (st != LORA_OK) return st;
  return launch_phase(false, ms, n, num_rows, num_slots, max_rank, LORA_NUM_MODULES, table, seg, scratch, nullptr, 0,
                      s, true);
}

int32_t lora_decode_layer_launches(const lora_module_io_t *io, uint32_t module_mask, int32_t num_rows,
                                   int32_t num_slots, lora_segments_t seg, int32_t max_rank) {
  ModuleArgs ms[LORA_NUM_MODULES];
  int n = 0;
  void *scratch = nullptr;
  // the argument checks without a workspace (an aligned stand-in of any size)
  const lora_adapter_entry_t *table = reinterpret_cast<const lora_adapter_entry_t *>(uintptr_t{256});
  if (check_layer(io, module_mask, num_rows, table, num_slots, seg, max_rank, reinterpret_cast<void *>(uintptr_t{256}),
                  ~size_t{0} >> 1, ms, &n, &scratch) != LORA_OK)
    return 0;
  OnePassDesc od;
  int grid = 0;
  const int32_t *ids = reinterpret_cast<const int32_t *>(uintptr_t{256});
  return onepass_plan(ms, n, num_rows, ids, num_slots, max_rank, table, seg, &od, &grid) ? 1 : 3;
}

// One pass per position of the rows' adapter lists: the segments of that
// column, then the layer's shrink and expand, each pass adding its delta to y
// in stream order (a row is in one segment per pass, so no two blocks of a
// launch touch the same y).
lora_status_t lora_apply_layer_stacked(const lora_module_io_t *io, uint32_t module_mask, int32_t num_rows,
                                       const int32_t *row_adapters, int32_t depth, const int32_t *pass_max_rank,
                                       const lora_adapter_entry_t *table, int32_t num_slots, lora_segments_t seg,
                                       int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  ModuleArgs ms[LORA_NUM_MODULES];
  int n = 0;
  void *scratch = nullptr;
  lora_status_t st =
      check_layer(io, module_mask, num_rows, table, num_slots, seg, max_rank, ws, ws_bytes, ms, &n, &scratch);
  if (st != LORA_OK) return st;
  if (depth < 1 || depth > LORA_MAX_STACK) return LORA_ERR_SHAPE;
  if (num_rows > 0 && !row_adapters) return LORA_ERR_NULL;
  if (pass_max_rank)
    for (int t = 0; t < depth; ++t)
      if (pass_max_rank[t] < 1 || pass_max_rank[t] > max_rank) return LORA_ERR_RANK;
  void *seg_scratch = nullptr;
  st = check_ws(ws, ws_bytes, segments_ws_bytes(num_rows, num_slots), &seg_scratch);
  if (st != LORA_OK) return st;
  ws = scratch ? scratch : seg_scratch;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int t = 0; t < depth; ++t) {
    st = launched(launch_build_segments(row_adapters + t, depth, num_rows, num_slots, t > 0, seg, ws, s));
    if (st != LORA_OK || num_rows == 0) return st;  // no rows: the first pass only resets the segments
    const int r = pass_max_rank ? pass_max_rank[t] : max_rank;  // the pass's launch class
    st = launch_phase(true, ms, n, num_rows, num_slots, r, LORA_NUM_MODULES, table, seg, ws, nullptr, 0, s, true);
    if (st != LORA_OK) return st;
    st = launch_phase(false, ms, n, num_rows, num_slots, r, LORA_NUM_MODULES, table, seg, ws, nullptr, 0, s, true);
    if (st != LORA_OK) return st;
  }
  return LORA_OK;
}

}  // extern "C"

namespace {

// One projection of a fused call, from either io struct.
struct LinearArgs {
  const void *x;
  int64_t ldx;
  const void *W;   // bf16 [d_out][ldw] elements, or 4-bit [d_out][ldw] bytes
  int64_t ldw;
  const float *Ws; // 4-bit: group scales [d_out][ldws]
  int64_t ldws;
  void *y;
  int64_t ldy;
  int32_t d_in, d_out;
};

lora_status_t check_linear(const lora_linear_io_t &m, LinearArgs *a) {
  if (!m.x || !m.y || !m.W) return LORA_ERR_NULL;
  if (m.d_in <= 0 || m.d_out <= 0 || m.ldx < m.d_in || m.ldy < m.d_out || m.ldw < m.d_in) return LORA_ERR_SHAPE;
  if ((m.d_in & 7) || (m.d_out & 7) || (m.ldx & 7) || (m.ldy & 7) || (m.ldw & 7) || !aligned16(m.x) ||
      !aligned16(m.y) || !aligned16(m.W))
    return LORA_ERR_ALIGN;
  if (!fits_u32(m.d_out, m.ldw)) return LORA_ERR_SHAPE;
  *a = LinearArgs{m.x, m.ldx, m.W, m.ldw, nullptr, 0, m.y, m.ldy, m.d_in, m.d_out};
  return LORA_OK;
}

lora_status_t check_linear(const lora_linear_q4_io_t &m, LinearArgs *a) {
  if (!m.x || !m.y || !m.Wq || !m.Ws) return LORA_ERR_NULL;
  if (m.d_in <= 0 || m.d_out <= 0 || m.ldx < m.d_in || m.ldy < m.d_out) return LORA_ERR_SHAPE;
  if ((m.d_in % LORA_Q4_GROUP) || (m.d_out & 7) || (m.ldx & 7) || (m.ldy & 7) || (m.ldwq & 15) ||
      !aligned16(m.x) || !aligned16(m.y) || !aligned16(m.Wq) || (reinterpret_cast<uintptr_t>(m.Ws) & 3))
    return LORA_ERR_ALIGN;
  if (m.ldwq < m.d_in / 2 || m.lds < m.d_in / LORA_Q4_GROUP) return LORA_ERR_SHAPE;
  if ((int64_t)m.d_out * m.ldwq > (int64_t)0xFFFFFF00 || (int64_t)m.d_out * m.lds * 4 > (int64_t)0xFFFFFF00)
    return LORA_ERR_SHAPE;
  *a = LinearArgs{m.x, m.ldx, m.Wq, m.ldwq, static_cast<const float *>(m.Ws), m.lds, m.y, m.ldy, m.d_in, m.d_out};
  return LORA_OK;
}

// Base projection + delta: the grouped shrink and the partials summed into one
// v plane per projection (original row order) (do_shrink), then the fused
// kernel (do_fused).  IO: lora_linear_io_t (bf16 base) or lora_linear_q4_io_t.
template <typename IO>
lora_status_t linear_phase(bool do_shrink, bool do_fused, const IO *io, uint32_t module_mask, int32_t num_rows,
                           const int32_t *row_adapter, const lora_adapter_entry_t *table, int32_t num_slots,
                           lora_segments_t seg, int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  constexpr bool kQ4 = std::is_same<IO, lora_linear_q4_io_t>::value;
  if (!io || !table) return LORA_ERR_NULL;
  lora_status_t st = check_segments(seg);
  if (st != LORA_OK) return st;
  const bool int8_items = (module_mask & LORA_MASK_INT8_ITEMS) != 0;
  module_mask &= ~LORA_MASK_INT8_ITEMS;
  if (module_mask == 0 || module_mask >= (1u << LORA_NUM_MODULES)) return LORA_ERR_MODULE;
  if (num_rows < 0 || num_slots < 1) return LORA_ERR_SHAPE;
  if (max_rank < 1 || max_rank > LORA_MAX_RANK) return LORA_ERR_RANK;
  if (num_rows > 0 && !row_adapter) return LORA_ERR_NULL;
  ModuleArgs ms[LORA_NUM_MODULES];
  LinearArgs la[LORA_NUM_MODULES];
  int n = 0;
  int64_t sum_d_in = 0;
  for (int c = 0; c < LORA_NUM_MODULES; ++c) {
    if (!(module_mask & (1u << c))) continue;
    st = check_linear(io[c], &la[n]);
    if (st != LORA_OK) return st;
    const LinearArgs &m = la[n];
    if (!fits_u32(num_rows, m.ldx) || !fits_u32(num_rows, m.ldy)) return LORA_ERR_SHAPE;
    ms[n] = ModuleArgs{m.x, m.ldx, m.y, m.ldy, m.d_in, m.d_out, c, int8_items};
    sum_d_in += m.d_in;
    ++n;
  }
  const size_t need = lora_linear_workspace_bytes(num_rows, num_slots, max_rank, sum_d_in, n);
  if (!ws) return LORA_ERR_NULL;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  if (ws_bytes < need) return LORA_ERR_WORKSPACE;
  const int rs = partial_row_stride(max_rank);
  if ((int64_t)num_rows * rs * 4 > (int64_t)0xFFFFFF00) return LORA_ERR_SHAPE;
  if (num_rows == 0) return LORA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *vplanes = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                             ((partials_ws_bytes(num_rows, max_rank, sum_d_in) + 255) & ~(size_t)255));
  if (do_shrink) {
    // 1. v partials of every projection (segment-grouped: each adapter's A once)
    st = launch_phase(true, ms, n, num_rows, num_slots, max_rank, LORA_NUM_MODULES, table, seg, ws, nullptr, 0, s);
    if (st != LORA_OK) return st;
    // 2. one v plane per projection, rows in their original order
    LayerDesc d;
    fill_desc(d, ms, n, true, num_rows, num_slots, max_rank, LORA_NUM_MODULES, table, seg, ws);
    d.v_out = vplanes;
    d.ldv = rs;
    st = launched(launch_shrink_reduce(d, s));
    if (st != LORA_OK) return st;
  }
  if (!do_fused) return LORA_OK;
  // 3. base projection + delta.  A block's work grows with its module's
  // d_in, and the blocks are dispatched in order, so the modules are numbered
  // longest first: a module of a long d_in (a down projection, 3.5x the
  // others) numbered last would start when the others are done and run
  // alone for most of the launch.
  FusedDesc f{};
  const int row_tiles = (num_rows + kFusedRows - 1) / kFusedRows;
  int order[LORA_NUM_MODULES];
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order, order + n, [&](int a, int b) { return la[a].d_in > la[b].d_in; });
  int64_t blocks = 0;
  for (int j = 0; j < n; ++j) {
    const int i = order[j];
    const LinearArgs &m = la[i];
    FusedModule &fm = f.mod[j];
    fm.x = static_cast<const uint16_t *>(m.x);
    fm.ldx = m.ldx;
    fm.W = m.W;
    fm.ldw = m.ldw;
    fm.Ws = m.Ws;
    fm.ldws = m.ldws;
    fm.y = static_cast<uint16_t *>(m.y);
    fm.ldy = m.ldy;
    fm.v = vplanes + (int64_t)i * num_rows * rs;
    fm.d_in = m.d_in;
    fm.d_out = m.d_out;
    fm.col = ms[i].col;
    fm.n_tiles = (m.d_out + fused_cols(kQ4) - 1) / fused_cols(kQ4);
    fm.block_base = (int)blocks;
    blocks += (int64_t)row_tiles * fm.n_tiles;
  }
  if (blocks > 0x7fffffff) return LORA_ERR_SHAPE;
  f.n_active = n;
  f.num_rows = num_rows;
  f.num_slots = num_slots;
  f.table_cols = LORA_NUM_MODULES;
  f.max_rank = max_rank;
  f.rs = rs;
  f.ids = row_adapter;
  f.status = seg.status;
  f.table = table;
  f.num_segments = seg.num_segments;
  f.seg_adapter = seg.seg_adapter;
  f.max_seg = segment_bound(num_rows, num_slots, seg);
  return launched(launch_fused(f, kQ4, (int)blocks, s));
}

}  // namespace

extern "C" {

lora_status_t lora_linear_layer(const lora_linear_io_t *io, uint32_t module_mask, int32_t num_rows,
                                const int32_t *row_adapter, const lora_adapter_entry_t *table, int32_t num_slots,
                                lora_segments_t seg, int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  return linear_phase(true, true, io, module_mask, num_rows, row_adapter, table, num_slots, seg, max_rank, ws,
                      ws_bytes, stream);
}

lora_status_t lora_linear_shrink(const lora_linear_io_t *io, uint32_t module_mask, int32_t num_rows,
                                 const int32_t *row_adapter, const lora_adapter_entry_t *table, int32_t num_slots,
                                 lora_segments_t seg, int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  return linear_phase(true, false, io, module_mask, num_rows, row_adapter, table, num_slots, seg, max_rank, ws,
                      ws_bytes, stream);
}

lora_status_t lora_linear_expand(const lora_linear_io_t *io, uint32_t module_mask, int32_t num_rows,
                                 const int32_t *row_adapter, const lora_adapter_entry_t *table, int32_t num_slots,
                                 lora_segments_t seg, int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  return linear_phase(false, true, io, module_mask, num_rows, row_adapter, table, num_slots, seg, max_rank, ws,
                      ws_bytes, stream);
}

lora_status_t lora_linear_layer_q4(const lora_linear_q4_io_t *io, uint32_t module_mask, int32_t num_rows,
                                   const int32_t *row_adapter, const lora_adapter_entry_t *table, int32_t num_slots,
                                   lora_segments_t seg, int32_t max_rank, void *ws, size_t ws_bytes, void *stream) {
  return linear_phase(true, true, io, module_mask, num_rows, row_adapter, table, num_slots, seg, max_rank, ws,
                      ws_bytes, stream);
}

lora_status_t lora_linear_shrink_q4(const lora_linear_q4_io_t *io, uint32_t module_mask, int32_t num_rows,
                                    const int32_t *row_adapter, const lora_adapter_entry_t *table,
                                    int32_t num_slots, lora_segments_t seg, int32_t max_rank, void *ws,
                                    size_t ws_bytes, void *stream) {
  return linear_phase(true, false, io, module_mask, num_rows, row_adapter, table, num_slots, seg, max_rank, ws,
                      ws_bytes, stream);
}

lora_status_t lora_linear_expand_q4(const lora_linear_q4_io_t *io, uint32_t module_mask, int32_t num_rows,
                                    const int32_t *row_adapter, const lora_adapter_entry_t *table,
                                    int32_t num_slots, lora_segments_t seg, int32_t max_rank, void *ws,
                                    size_t ws_bytes, void *stream) {
  return linear_phase(false, true, io, module_mask, num_rows, row_adapter, table, num_slots, seg, max_rank, ws,
                      ws_bytes, stream);
}

}  // extern "C"

// ---- lora_apply_layer_noalloc: the k-chunk partials in a static device
// array instead of a caller's workspace.  Each device that loads the library
// holds its own copy until the process ends; in host code `scratch` is only
// a handle, so its device address is looked up once per device and every
// launch takes that address.
static __device__ __align__(256) uint8_t scratch[LORA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device

// The address of the current device's `scratch` (looked up on the first call
// on that device, with it current).
lora_status_t scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LORA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LORA_ERR_LAUNCH;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return LORA_OK;
}

}  // namespace

extern "C" lora_status_t lora_apply_layer_noalloc(const lora_module_io_t *io, uint32_t module_mask,
                                                  int32_t num_rows, const lora_adapter_entry_t *table,
                                                  int32_t num_slots, lora_segments_t seg, int32_t max_rank,
                                                  void *stream) {
  ModuleArgs ms[LORA_NUM_MODULES];
  int n = 0;
  // the argument checks of lora_apply_layer, with the static array as an
  // aligned workspace of its full size
  void *unused = nullptr;
  lora_status_t st = check_layer(io, module_mask, num_rows, table, num_slots, seg, max_rank,
                                 reinterpret_cast<void *>(uintptr_t{256}), LORA_STATIC_SCRATCH_BYTES, ms, &n, &unused);
  if (st == LORA_ERR_WORKSPACE) return LORA_ERR_SCRATCH;
  if (st != LORA_OK) return st;
  if (num_rows == 0) return LORA_OK;
  void *ws = nullptr;
  st = scratch_address(&ws);
  if (st != LORA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_phase(true, ms, n, num_rows, num_slots, max_rank, LORA_NUM_MODULES, table, seg, ws, nullptr, 0, s, true);
  if (st != LORA_OK) return st;
  return launch_phase(false, ms, n, num_rows, num_slots, max_rank, LORA_NUM_MODULES, table, seg, ws, nullptr, 0, s,
                      true);
}
