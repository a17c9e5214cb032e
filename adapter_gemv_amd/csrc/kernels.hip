// The delta kernels: one launch per phase covers every projection of the
// call and every segment.  The SGMV row tiles (segments of at least long_min
// rows) come first, then decode_blocks blocks of decode items (shorter
// segments); the grid's remaining blocks have no work.  The
// rank class of the launch (smallest of 8, 16, 32, 64 holding max_rank) fixes
// the register tiling of both paths.
#include "decode_items.h"
#include "fused_items.h"
#include "onepass_items.h"
#include "sgmv_items.h"

namespace lora {
namespace {

// LDS of the expand kernel: the SGMV V tile and the int8 row scales of its
// n-tile, or the decode v stage plus one tile of sums and one of int8 row
// scales, whichever is larger (floats).
template <int LPR>
constexpr int expand_lds_floats() {
  constexpr int sgmv = kSgmvExpandRows * 64 + kSgmvExpandCols;
  constexpr int decode = kOneRowDeltaBase + 2 * decode_expand_tile(LPR);
  return sgmv > decode ? sgmv : decode;
}

// The shrink's LDS also caps the blocks per CU at two (the decode items
// stream fastest at that occupancy).
constexpr int kShrinkLdsAlloc = 64 * 1024;
static_assert(kShrinkLdsBytes <= kShrinkLdsAlloc, "shrink LDS");

// Blocks of the SGMV tiles the build counted (`tiles`, `items` blocks each),
// at most the room the host left for them (`room` blocks).  They come first:
// a tile of many rows is the longest work of the launch.  Then the decode
// items; the unused room ends the grid, where its blocks exit at once.
// (The order of the branches below changes the code the compiler produces
// for each path: testing the decode range first measured faster shrinks for
// batches of single-row segments, by about 2%, but slower matrix-core
// paths, by 5 to 13%; this order keeps the matrix-core code.)
__device__ __forceinline__ int sgmv_blocks(int tiles, int items, int room) {
  return items > 0 ? min(max(tiles, 0), room / items) * items : 0;
}

template <int CLS>
__global__ __launch_bounds__(256) void lora_shrink_kernel(LayerDesc d, int decode_blocks) {
  __shared__ __align__(16) uint8_t lds[kShrinkLdsAlloc];
  constexpr int JW = 2 << CLS;                          // A rows per wave (decode)
  constexpr int NT = CLS <= 1 ? 1 : CLS == 2 ? 2 : 4;   // 16-column rank tiles (SGMV)
  const int b = blockIdx.x;
  const int nseg = uniform(*d.num_segments);  // requested with the tile count: one wait for both
  const int sg = sgmv_blocks(uniform(d.tile_counts[0]), d.items_per_seg, (int)gridDim.x - decode_blocks);
  if (b < sg) sgmv_shrink_block<NT>(d, b, lds);
  else if (b < sg + decode_blocks) decode_shrink_block<JW>(d, b - sg, nseg);
}

// Waves per SIMD the expand is compiled for: every path of the kernel (bf16
// and int8, decode and SGMV) fits 4 for the rank classes up to 16 and 3 for
// ranks 32 and 64 without spilling; left to itself the compiler can give a
// class one wave less.
template <int CLS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CLS <= 1 ? 4 : 3))) void lora_expand_kernel(
    LayerDesc d, int decode_blocks) {
  constexpr int LPR = 1 << CLS;                          // lanes per output row (decode)
  __shared__ float lds[expand_lds_floats<LPR>()];
  constexpr int KT = CLS <= 2 ? 1 : 2;                   // 32-wide rank steps (SGMV)
  // k-chunk partials per round of the SGMV V staging: 4 where the register
  // bound leaves room (ranks 32 and 64), else 2
  constexpr int VU = CLS >= 2 ? 4 : 2;
  const int b = blockIdx.x;
  const int nseg = uniform(*d.num_segments);  // requested with the tile count: one wait for both
  const int sg = sgmv_blocks(uniform(d.tile_counts[1]), d.sg_items, (int)gridDim.x - decode_blocks);
  if (b < sg) sgmv_expand_block<KT, VU>(d, b, lds);
  else if (b < sg + decode_blocks) decode_expand_block<LPR>(d, b - sg, nseg, lds);
}

// Sum the k-chunk partials of each row in a segment into v[b][0..max_rank)
// (zero past the entry's rank), for module blockIdx.y into the plane
// v_out + blockIdx.y * num_rows * ldv (lora_shrink: one module, the caller's
// v; the fused layer: every module, planes in the workspace).
__global__ __launch_bounds__(256) void shrink_reduce_kernel(LayerDesc d) {
  const int nseg = min(*d.num_segments, d.max_seg);
  if (nseg <= 0) return;
  const int nvalid = min(d.seg_offsets[nseg], d.num_rows);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int p = (int)(idx / d.max_rank);
  const int j = (int)(idx - (int64_t)p * d.max_rank);
  if (p >= nvalid) return;
  int lo = 0, hi = nseg - 1;  // segment s with seg_offsets[s] <= p < seg_offsets[s+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (d.seg_offsets[mid] <= p) lo = mid;
    else hi = mid - 1;
  }
  const ModuleDesc m = kernel_desc().mod[blockIdx.y];
  float *v_out = d.v_out + (int64_t)blockIdx.y * d.num_rows * d.ldv;
  const int a = d.seg_adapter[lo];
  if ((unsigned)a >= (unsigned)d.num_slots) return;
  const lora_adapter_entry_t e = d.table[(int64_t)a * d.table_cols + m.col];  // varies per lane
  const bool ok = entry_ok(e, d.max_rank);
  float sum = 0.f;
  if (ok && j < e.rank)
    for (int c = 0; c < m.n_chunks; ++c) sum += d.part[((int64_t)(m.part_base + c) * d.num_rows + p) * d.rs + j];
  const int b = d.perm[p];
  if ((unsigned)b < (unsigned)d.num_rows) v_out[(int64_t)b * d.ldv + j] = sum;
}

// Sum the k-chunk partials of every row in a segment into its first chunk,
// for module blockIdx.y.  A prefill call runs this between its shrink and
// its expand, whose SGMV tiles (one per 1024 columns of a row tile) then
// read one chunk each instead of summing them all again.  A thread owns 4
// columns of one row: it reads them in every chunk and writes the sum over
// the first, so no two threads touch the same words.  Columns past an
// entry's rank are summed like the others and never read.
__global__ __launch_bounds__(256) void fold_partials_kernel(LayerDesc d) {
  const int nseg = min(*d.num_segments, d.max_seg);
  if (nseg <= 0) return;
  const int nvalid = min(d.seg_offsets[nseg], d.num_rows);
  const int quads = d.rs / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int p = (int)(idx / quads);
  if (p >= nvalid) return;
  const int jq = (int)(idx - (int64_t)p * quads) * 4;
  const ModuleDesc m = kernel_desc().mod[blockIdx.y];
  if (m.n_chunks < 2) return;
  const int64_t chunk_stride = (int64_t)d.num_rows * d.rs;
  float *first = d.part + ((int64_t)m.part_base * d.num_rows + p) * d.rs + jq;
  f32x4_t sum = *(const f32x4_t *)first;
  for (int c = 1; c < m.n_chunks; ++c) sum += *(const f32x4_t *)(first + c * chunk_stride);
  *(f32x4_t *)first = sum;
}

// One-launch decode (onepass_items.h): block 0 writes the segments; blocks
// 1.. are (item, row), item-major over row_slots (a multiple of 8) rows, so
// the blocks of one row share an XCD when blocks are dealt to the XCDs in
// turn.  Compiled for 3 waves per SIMD (the 16-pass B tile).
template <int CLS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void lora_onepass_kernel(
    OnePassDesc od) {
  __shared__ __align__(16) uint8_t lds[kOnePassLdsBytes];
  if (blockIdx.x == 0) {
    op_build(od, lds);
    return;
  }
  const LayerDesc &d = od.L;
  const int R = od.row_slots;
  const int b = (int)blockIdx.x - 1;
  const int it = b / R, t = b - it * R;
  if (t >= d.num_rows) return;
  const ModuleDesc m = module_of_item(d, it);
  const int c = it - m.item_base;
  // every row's id, for the ballots and the slot rank (-1: past the batch, base only or a bad id)
  const int raw_id = (int)threadIdx.x < d.num_rows ? od.ids[threadIdx.x] : -1;
  const int idu = (unsigned)raw_id < (unsigned)d.num_slots ? raw_id : -1;
  const int a = uniform(od.ids[t]);
  if ((unsigned)a >= (unsigned)d.num_slots) return;  // base only, or a bad id (the last block counts it)
  const lora_adapter_entry_t raw = d.table[(int64_t)a * d.table_cols + m.col];
  lora_adapter_entry_t e;
  e.A = uniform(raw.A);
  e.B = uniform(raw.B);
  e.rank = uniform(raw.rank);
  e.scale = uniform(raw.scale);
  e.format = uniform(raw.format);
  e.reserved = 0;
  if (!entry_ok(e, d.max_rank)) return;  // rank 0, or an entry the last block counts
  const int tpb = od.tiles_per_block;
  if (e.format == LORA_FORMAT_INT8_ROWS) op_delta<CLS, true>(m, e, c, tpb, t, a, idu, od.bound_check, d.max_seg, lds);
  else op_delta<CLS, false>(m, e, c, tpb, t, a, idu, od.bound_check, d.max_seg, lds);
}

// Base projection + delta (fused_items.h).  Two blocks per CU (their LDS
// and registers): compiled for 2 waves per SIMD, which the 128-column bf16
// tile's accumulators need without spilling.
template <bool Q4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void lora_fused_kernel(FusedDesc f) {
  __shared__ __align__(16) uint8_t lds[fused_lds_bytes(Q4)];
  fused_block<Q4>(f, blockIdx.x, lds);
}

int rank_class(int max_rank) { return max_rank <= 8 ? 0 : max_rank <= 16 ? 1 : max_rank <= 32 ? 2 : 3; }

}  // namespace

int long_tiles_max(int num_rows, int max_seg, int rows_per_tile) {
  const int long_segs = min(max_seg, num_rows / kLongSegRows);
  return num_rows / rows_per_tile + long_segs + 1;
}
int sgmv_shrink_rows() { return kSgmvShrinkRows; }
int sgmv_expand_rows() { return kSgmvExpandRows; }

hipError_t launch_shrink(const LayerDesc &d, int decode_blocks, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (rank_class(d.max_rank)) {
    case 0: lora_shrink_kernel<0><<<grid, 256, 0, stream>>>(d, decode_blocks); break;
    case 1: lora_shrink_kernel<1><<<grid, 256, 0, stream>>>(d, decode_blocks); break;
    case 2: lora_shrink_kernel<2><<<grid, 256, 0, stream>>>(d, decode_blocks); break;
    default: lora_shrink_kernel<3><<<grid, 256, 0, stream>>>(d, decode_blocks); break;
  }
  return hipGetLastError();
}

hipError_t launch_expand(const LayerDesc &d, int decode_blocks, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (rank_class(d.max_rank)) {
    case 0: lora_expand_kernel<0><<<grid, 256, 0, stream>>>(d, decode_blocks); break;
    case 1: lora_expand_kernel<1><<<grid, 256, 0, stream>>>(d, decode_blocks); break;
    case 2: lora_expand_kernel<2><<<grid, 256, 0, stream>>>(d, decode_blocks); break;
    default: lora_expand_kernel<3><<<grid, 256, 0, stream>>>(d, decode_blocks); break;
  }
  return hipGetLastError();
}

hipError_t launch_shrink_reduce(const LayerDesc &d, hipStream_t stream) {
  const int64_t total = (int64_t)d.num_rows * d.max_rank;
  if (total <= 0) return hipSuccess;
  shrink_reduce_kernel<<<dim3((unsigned)((total + 255) / 256), (unsigned)d.n_active), 256, 0, stream>>>(d);
  return hipGetLastError();
}

hipError_t launch_fold_partials(const LayerDesc &d, hipStream_t stream) {
  const int64_t total = (int64_t)d.num_rows * (d.rs / 4);
  if (total <= 0) return hipSuccess;
  fold_partials_kernel<<<dim3((unsigned)((total + 255) / 256), (unsigned)d.n_active), 256, 0, stream>>>(d);
  return hipGetLastError();
}

hipError_t launch_onepass(const OnePassDesc &d, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (rank_class(d.L.max_rank)) {
    case 0: lora_onepass_kernel<0><<<grid, 256, 0, stream>>>(d); break;
    case 1: lora_onepass_kernel<1><<<grid, 256, 0, stream>>>(d); break;
    case 2: lora_onepass_kernel<2><<<grid, 256, 0, stream>>>(d); break;
    default: return hipErrorInvalidValue;  // the host plans the one-launch path up to rank 32 only
  }
  return hipGetLastError();
}

hipError_t launch_fused(const FusedDesc &f, bool q4, int blocks, hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  if (q4) lora_fused_kernel<true><<<blocks, 256, 0, stream>>>(f);
  else lora_fused_kernel<false><<<blocks, 256, 0, stream>>>(f);
  return hipGetLastError();
}

size_t partials_ws_bytes(int num_rows, int max_rank, int64_t sum_d_in) {
  const int64_t chunks = sum_d_in / kKChunkMin + kMaxModules;
  return (size_t)((int64_t)num_rows * partial_row_stride(max_rank) * 4 * chunks);
}

}  // namespace lora
