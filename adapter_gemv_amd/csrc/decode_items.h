// Decode (BGMV-style) work items: segments shorter than kLongSegRows rows.
//
// "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A": one batched kernel
// gathers each sequence's adapter through the index vector and applies it
// without materialising per-sequence weights; the cost is bandwidth, since
// each distinct adapter in the batch is read once per step.
// "LoRA, quotas and noisy neighbours", "One weight read, many adapters": the
// update is applied in registers.
//
// Items are (segment, projection, k-chunk) for the shrink and (segment,
// projection, n-tile) for the expand; a 256-thread block takes one item, and
// a segment's rows share every load of its adapter's factors.
//
// Shrink  v = A.x: rows of A are spread over the 4 waves; each lane streams 8
//   consecutive k (16 bytes) of every A row and of each x row, so one wave
//   load covers 1 KiB of contiguous memory.  bf16 pairs meet in
//   v_dot2_f32_bf16 (exact products, fp32 sums).  The per-lane sums are
//   reduced across the wave by a reduce-scatter butterfly that leaves every
//   sum on one lane; the block writes its k-chunk's partial v to the
//   workspace (fixed order, no atomics: results are bit-reproducible).
// Expand  y += scale * B.v: the item sums the k-chunk partials of its rows
//   into LDS (times scale) and streams its tile of B, which is contiguous
//   because B is [d_out][ldb] row-major: LPR = rank/8 lanes share an output
//   row and each lane loads 16 bytes.  v (fp32) is split once per row into
//   bf16 hi + lo, so the products with B run on v_dot2_f32_bf16 without
//   converting B.  A reduce-scatter over the LPR lanes finishes the dot
//   products.  A one-row item collects its sums in LDS and updates y once,
//   16 bytes per lane, after its last B load; a multi-row item updates y
//   per row.  y + delta is rounded to bf16 (RNE); each (row, output) has one
//   writer.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace lora {

// ---------------------------------------------------------------- shrink --

// Wave w owns rows [w*jw, w*jw + jw) of A with jw = ceil(rank / 4) <= JW, so
// all waves share the stream whatever the entry's rank.  RG rows of x are
// processed together.  Q8: A is int8 with one fp32 scale per row; a lane
// takes 16 values of a row per step (one 16-byte load, widened to bf16 in
// registers) against two 16-byte pieces of x, and the row scale multiplies
// the chunk's sum.  int8 rows are padded to 16 bytes, so the load stays in
// its row; where d_in ends inside it, the second x piece lies past the row
// of x and reads zero, and the padding bytes (always finite) add nothing.
// row_of(r) gives the original row of sorted position pos0 + r.  U steps of
// loads go out together (a step past the chunk reads zeros).  The rows of A
// taken start at j_base (a pass over part of the entry's rows).
template <int JW, int RG, bool Q8, typename RowOf, int U = 1>
__device__ __forceinline__ void decode_shrink_rows(const LayerDesc &d, const ModuleDesc &m, const void *A, int rank,
                                                   int jw, int pos0, int nrows, int chunk, RowOf row_of,
                                                   int j_base = 0) {
  constexpr int VPL = Q8 ? 16 : 8;  // k per lane and step
  const int lane = threadIdx.x & 63;
  const int j0 = j_base + wave_id() * jw;
  const int k_begin = chunk * d.kc;
  const int k_end = min(k_begin + d.kc, m.d_in);
  const uint32_t row_bytes = (uint32_t)m.d_in * 2;
  const uint32_t a_row_bytes = Q8 ? lda8_of(m.d_in) : row_bytes;
  rsrc_t rx[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int b = r < nrows ? uniform(row_of(r)) : 0;
    const bool ok = (unsigned)b < (unsigned)d.num_rows;  // a stray index reads zeros
    rx[r] = make_rsrc(m.x + (int64_t)(ok ? b : 0) * m.ldx, ok ? row_bytes : 0u);
  }
  const uint8_t *a_vals = static_cast<const uint8_t *>(A) + (Q8 ? q8_values_offset(rank) : 0);
  const rsrc_t ra = make_rsrc(a_vals, (uint32_t)rank * a_row_bytes);
  float acc[JW * RG];
#pragma unroll
  for (int i = 0; i < JW * RG; ++i) acc[i] = 0.f;
  for (int k0 = k_begin + lane * VPL; k0 < k_end; k0 += U * 64 * VPL) {
#pragma unroll
   for (int u = 0; u < U; ++u) {
    const int k = k0 + u * 64 * VPL;
    const bool kin = U == 1 || k < k_end;  // a step past the chunk reads zeros
    const uint32_t voff = kin ? (uint32_t)k * 2 : kOutOfRange;
    u32x4 xv[RG], av[JW];
#pragma unroll
    for (int r = 0; r < RG; ++r) xv[r] = r < nrows ? buf_ld16(rx[r], voff, 0) : zero4();
    if constexpr (Q8) {
      u32x4 xw[RG];  // x[k + 8, k + 16)
#pragma unroll
      for (int r = 0; r < RG; ++r) xw[r] = r < nrows ? buf_ld16(rx[r], kin ? voff + 16 : kOutOfRange, 0) : zero4();
      u32x4 aq[JW];
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
        aq[jj] = (jj < jw && j0 + jj < rank)
                     ? buf_ld16_stream(ra, kin ? (uint32_t)k : kOutOfRange, (uint32_t)(j0 + jj) * a_row_bytes)
                     : zero4();
#pragma unroll
      for (int jj = 0; jj < JW; ++jj) {
        const u32x4 lo = i8x8_to_bf16x8(u32x2{aq[jj].x, aq[jj].y});
        const u32x4 hi = i8x8_to_bf16x8(u32x2{aq[jj].z, aq[jj].w});
#pragma unroll
        for (int r = 0; r < RG; ++r) acc[jj * RG + r] = dot8_bf16(hi, xw[r], dot8_bf16(lo, xv[r], acc[jj * RG + r]));
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
        av[jj] = (jj < jw && j0 + jj < rank) ? buf_ld16_stream(ra, voff, (uint32_t)(j0 + jj) * row_bytes) : zero4();
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
#pragma unroll
        for (int r = 0; r < RG; ++r) acc[jj * RG + r] = dot8_bf16(av[jj], xv[r], acc[jj * RG + r]);
    }
   }
  }
  reduce_scatter<JW * RG, 64>(acc);
  float *out = d.part + ((int64_t)(m.part_base + chunk) * d.num_rows + pos0) * d.rs;
  const float *a_scale = static_cast<const float *>(A);
  constexpr int NV = JW * RG;
  if constexpr (NV >= 64) {
#pragma unroll
    for (int i = 0; i < NV / 64; ++i) {
      const int idx = i + (NV / 64) * lane;
      const int jj = idx / RG, r = idx % RG;
      if (r < nrows && jj < jw && j0 + jj < rank)
        out[(int64_t)r * d.rs + j0 + jj] = Q8 ? acc[i] * a_scale[j0 + jj] : acc[i];
    }
  } else {
    constexpr int GS = 64 / NV;
    if (lane % GS == 0) {
      const int idx = lane / GS;
      const int jj = idx / RG, r = idx % RG;
      if (r < nrows && jj < jw && j0 + jj < rank)
        out[(int64_t)r * d.rs + j0 + jj] = Q8 ? acc[0] * a_scale[j0 + jj] : acc[0];
    }
  }
}

// Block `blk` of the decode shrink numbering (nseg: the segments built).  JW
// = rows of A per wave at the largest rank of the launch (4*JW).  An item
// runs at its entry's own rows of A per wave (rank/4, rounded up to a power
// of two), and a multi-row item with all its rows (at most kLongSegRows - 1)
// against each load of A, their count rounded up to 2, 4 or 8; where rows of
// A per wave times rows of x would pass 64 sums, the rows of A go in passes
// of 64/RG per wave.  Two steps of loads are in flight where the registers
// allow.
template <int JW>
__device__ __forceinline__ void decode_shrink_block(const LayerDesc &d, int blk, int nseg) {
  static_assert(kLongSegRows <= 8, "a decode segment's rows meet A in one pass");
  const int s = blk / d.items_per_seg;
  if (s >= nseg) return;
  const int it = blk - s * d.items_per_seg;
  const ModuleDesc m = module_of_item(d, it);
  const int chunk = it - m.item_base;
  int a, pos0, len;
  if (!load_segment(d, s, it == 0 && d.count_errors, &a, &pos0, &len)) return;
  if (len >= d.long_min) return;  // an SGMV item takes this segment
  lora_adapter_entry_t e;
  if (!load_entry(d, a, m.col, chunk == 0 && d.count_errors, &e)) return;
  const int rank = e.rank;
  const int jw = (rank + 3) >> 2;
  auto run = [&](auto q8) {
    constexpr bool Q8 = decltype(q8)::value;
    auto row = [&](int r) { return d.perm[pos0 + r]; };
    auto by_shape = [&](auto jwc, auto rgc) {
      constexpr int JWE = decltype(jwc)::value, RG = decltype(rgc)::value;
      if constexpr (JWE <= JW) {
        if constexpr (RG == 1) {
          // one row: two steps in flight below the launch's rank (at rank 64
          // the registers hold one)
          constexpr int U = JWE < JW ? 2 : 1;
          decode_shrink_rows<JWE, 1, Q8, decltype(row), U>(d, m, e.A, rank, jw, pos0, 1, chunk, row);
        } else if constexpr (JWE * RG <= 64) {
          constexpr int U = RG * (Q8 ? 2 : 1) + JWE <= 12 ? 2 : 1;
          decode_shrink_rows<JWE, RG, Q8, decltype(row), U>(d, m, e.A, rank, jw, pos0, len, chunk, row);
        } else {
          constexpr int JP = 64 / RG;  // rows of A per wave and pass
          constexpr int U = RG * (Q8 ? 2 : 1) + JP <= 12 ? 2 : 1;
          for (int jb = 0; jb < rank; jb += 4 * JP)
            decode_shrink_rows<JP, RG, Q8, decltype(row), U>(d, m, e.A, rank, JP, pos0, len, chunk, row, jb);
        }
      }
    };
    auto by_rank = [&](auto rgc) {
      if (jw <= 2) by_shape(std::integral_constant<int, 2>{}, rgc);
      else if (jw <= 4) by_shape(std::integral_constant<int, 4>{}, rgc);
      else if (jw <= 8) by_shape(std::integral_constant<int, 8>{}, rgc);
      else by_shape(std::integral_constant<int, JW>{}, rgc);
    };
    if (len == 1) by_rank(std::integral_constant<int, 1>{});
    else if (len == 2) by_rank(std::integral_constant<int, 2>{});
    else if (len <= 4) by_rank(std::integral_constant<int, 4>{});
    else by_rank(std::integral_constant<int, 8>{});
  };
  if (e.format == LORA_FORMAT_INT8_ROWS) run(std::true_type{});
  else run(std::false_type{});
}

// ---------------------------------------------------------------- expand --

// Start (floats) of two tile-sized LDS regions past the v stage and its
// reduction space: the one-row expand keeps its sums in the first and the
// int8 row scales of its tile in the second; the multi-row expand keeps the
// int8 row scales in the first.
constexpr int kOneRowDeltaBase = 64 + 1024;

// Load passes per sub-tile of the decode expand: 16, or fewer where G rows
// per pass would make a sub-tile longer than the tile capacity NTC (narrow
// lane widths in a launch of a higher rank class).
constexpr int expand_passes(int ntc, int g) { return 16 * g <= ntc ? 16 : ntc / g; }

// Row stride of B: the rank rounded up to a multiple of 8, so every row is
// 16-byte aligned.  Columns in [rank, ldb) are padding with finite values;
// they meet zeros of v and add nothing.
__device__ __forceinline__ int b_stride(int rank) { return (rank + 7) & ~7; }

// The rows [n_tile0, n_tile0 + tile_len) of an entry's B.  bf16 rows are
// b_stride(rank) * 2 bytes apart; Q8 (int8 with one fp32 scale per row)
// rows are ldb8_of(rank) bytes apart (a multiple of 16), after the d_out
// scales.  A lane reads the VPL values [jq, jq + VPL) of a row: 8 bf16 (16
// bytes), or 8 or 16 int8 (8 or 16 bytes).
template <bool Q8, int VPL = 8>
struct BTile {
  static_assert(VPL == 8 || (Q8 && VPL == 16), "values per lane");
  using raw_t = typename std::conditional<Q8 && VPL == 8, u32x2, u32x4>::type;
  rsrc_t r;
  uint32_t row_bytes;
  const float *scale;  // Q8: scale of tile row 0
  __device__ __forceinline__ BTile(const void *B, int rank, int d_out, int n_tile0, uint32_t tile_len) {
    const uint8_t *base = static_cast<const uint8_t *>(B);
    if constexpr (Q8) {
      row_bytes = (uint32_t)ldb8_of(rank);
      scale = reinterpret_cast<const float *>(base) + n_tile0;
      base += q8_values_offset(d_out);
    } else {
      row_bytes = (uint32_t)b_stride(rank) * 2;
      scale = nullptr;
    }
    r = make_rsrc(base + (int64_t)n_tile0 * row_bytes, tile_len * row_bytes);  // past the tile: zero
  }
  __device__ __forceinline__ uint32_t off(int n, int jq) const {
    return (uint32_t)n * row_bytes + (uint32_t)jq * (Q8 ? 1 : 2);
  }
  __device__ __forceinline__ raw_t load(uint32_t voff, uint32_t soff) const {
    if constexpr (sizeof(raw_t) == 8) return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNonTemporal);
    else return buf_ld16_stream(r, voff, soff);
  }
  // bf16 values for a tile that several rows use: widened once.
  static __device__ __forceinline__ u32x4 widen(const raw_t &v) {
    static_assert(VPL == 8, "widen takes 8 values");
    if constexpr (Q8) return i8x8_to_bf16x8(v);
    else return v;
  }
  // One use of a load: bf16 against the split v; int8 converted to fp32.
  static __device__ __forceinline__ float dot(const raw_t &b, const float *vv, const V8Split &vs, float c) {
    if constexpr (Q8 && VPL == 16) return dot8_i8_f32(u32x2{b.z, b.w}, vv + 8, dot8_i8_f32(u32x2{b.x, b.y}, vv, c));
    else if constexpr (Q8) return dot8_i8_f32(b, vv, c);
    else return dot8_bf16_split(b, vs, c);
  }
};

// One n-tile of one projection for every row of a multi-row segment (fewer
// than kLongSegRows rows: longer ones go to the SGMV items).  v of every row
// is staged once; the B sub-tile is loaded once into registers and used by
// all rows, and the next sub-tile is requested when the rows are done; y of
// a few rows is requested together.
template <int LPR, bool Q8, int NTC>
__device__ __forceinline__ void decode_expand_rows(const LayerDesc &d, const ModuleDesc &m, const void *B, int rank,
                                                   float scale, int pos0, int len, int tile, float *v_lds) {
  static_assert(kLongSegRows <= kExpandRowGroup, "a decode segment is staged in one group");
  constexpr int G = kDecodeThreads / LPR;  // output rows per load pass of the block
  constexpr int P = expand_passes(NTC, G);  // load passes per sub-tile
  constexpr int SUB = P * G;               // outputs per sub-tile
  constexpr int PL = P / LPR;              // outputs per lane per row after the reduce-scatter
  constexpr int YR = PL <= 4 ? 4 : 1;      // rows whose y is requested together
  const int t = threadIdx.x, g = t / LPR, q = t % LPR, jq = q * 8;
  const int nr = min(len, kExpandRowGroup);
  const int n_tile0 = tile * d.nt;
  const int n_tile1 = min(n_tile0 + d.nt, m.d_out);
  const uint32_t tile_len = (uint32_t)(n_tile1 - n_tile0);
  const BTile<Q8> bt(B, rank, m.d_out, n_tile0, tile_len);
  auto load_b = [&](int n) { return bt.load(jq < rank ? bt.off(n, jq) : kOutOfRange, 0); };
  auto y_rsrc = [&](int i) {
    const int b = i < nr ? uniform(d.perm[pos0 + i]) : -1;
    const bool ok = (unsigned)b < (unsigned)d.num_rows;  // a stray index touches nothing
    return make_rsrc(m.y + (int64_t)(ok ? b : 0) * m.ldy + n_tile0, ok ? tile_len * 2 : 0u);
  };
  VStage<kExpandRowGroup> vst;
  vst.issue(d, m, pos0, nr, rank);  // before the B stream: waiting for v does not wait for B
  typename BTile<Q8>::raw_t bv[P];
#pragma unroll
  for (int p = 0; p < P; ++p) bv[p] = load_b(p * G + g);
  float *b_scale = v_lds + kOneRowDeltaBase;  // Q8: [NT] row scales of the tile, published by finish()
  if constexpr (Q8) {
    constexpr int NT = NTC;  // the launch's tile capacity: the host tiles with the same constant
    const rsrc_t rs = make_rsrc(bt.scale, tile_len * 4);
#pragma unroll
    for (int i = 0; i < NT / (kDecodeThreads * 4); ++i) {
      const int n = (i * kDecodeThreads + t) * 4;
      *(f32x4_t *)(b_scale + n) = __builtin_bit_cast(f32x4_t, buf_ld16(rs, (uint32_t)n * 4, 0));
    }
  }
  vst.finish(d, m, scale, v_lds);
  for (int n0 = 0; n0 < (int)tile_len; n0 += SUB) {
    u32x4 wb[P];  // the sub-tile as bf16, shared by the rows
#pragma unroll
    for (int p = 0; p < P; ++p) wb[p] = BTile<Q8>::widen(bv[p]);
    for (int i0 = 0; i0 < nr; i0 += YR) {
      rsrc_t ry[YR];
      uint16_t yv[YR][PL];
#pragma unroll
      for (int u = 0; u < YR; ++u) {
        ry[u] = y_rsrc(i0 + u);
#pragma unroll
        for (int ii = 0; ii < PL; ++ii) yv[u][ii] = buf_ld_u16(ry[u], (uint32_t)(n0 + (ii + PL * q) * G + g) * 2);
      }
#pragma unroll
      for (int u = 0; u < YR; ++u) {
        const int i = i0 + u;
        if (i >= nr) break;
        float vv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) vv[k] = v_lds[i * 64 + jq + k];
        const V8Split vs = split_v8(vv);
        float acc[P];
#pragma unroll
        for (int p = 0; p < P; ++p) acc[p] = dot8_bf16_split(wb[p], vs, 0.f);
        reduce_scatter<P, LPR>(acc);
        int sn0 = n0;
        if constexpr (Q8) asm volatile("" : "+v"(sn0));  // scales read per row, not held across the rows
#pragma unroll
        for (int ii = 0; ii < PL; ++ii) {
          const uint32_t off = (uint32_t)(n0 + (ii + PL * q) * G + g) * 2;
          const float dlt = Q8 ? acc[ii] * b_scale[sn0 + (ii + PL * q) * G + g] : acc[ii];
          buf_st_u16(ry[u], off, f32_to_bf16(bf16_to_f32(yv[u][ii]) + dlt));
        }
        __builtin_amdgcn_sched_barrier(0);  // one row's sums live at a time
      }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) bv[p] = load_b(n0 + SUB + p * G + g);  // past the tile: zero
  }
}

// The same for a segment of one row (every decode row with its own adapter),
// streamed: the item covers several sub-tiles of B and each register of the
// tile is refilled with the next sub-tile's data as soon as its dot product
// is taken, so 16 loads per lane stay in flight for the whole item.  A load's
// offset is the lane's offset inside a pass plus a per-pass constant; the
// sub-tile base goes in the scalar offset.  Lanes past the rank or the tile
// get an out-of-range lane offset and read zero.
// y of the whole tile is requested with the first loads, 16 bytes per lane;
// the sums of each sub-tile go to LDS, and y is written once, after the
// last load of B.  (A store in the middle of the stream would hold up the
// loads issued after it: one counter retires loads and stores in order.)
// Q8: a lane takes 16 int8 values (16 bytes) of a row, so half as many
// lanes share a row and a load moves as many bytes as in bf16.

template <int LPR, bool Q8, int NTC>
__device__ __forceinline__ void decode_expand_one_row(const LayerDesc &d, const ModuleDesc &m, const void *B,
                                                      int rank, float scale, int pos0, int tile, int item,
                                                      float *v_lds) {
  constexpr int VPL = Q8 ? 16 : 8;                  // values per lane and load
  constexpr int L = Q8 && LPR > 1 ? LPR / 2 : LPR;  // lanes per output row
  constexpr int G = kDecodeThreads / L;
  constexpr int P = expand_passes(NTC, G);
  constexpr int SUB = P * G;
  constexpr int PL = P / L;
  constexpr int NT = NTC;
  static_assert(NT % SUB == 0 && NT % (kDecodeThreads * 8) == 0, "tile");
  constexpr int YT = NT / (kDecodeThreads * 8);  // 16-byte y pieces per thread
  using BT = BTile<Q8, VPL>;
  const int t = threadIdx.x, g = t / L, q = t % L, jq = q * VPL;
  const int n_tile0 = tile * d.nt;
  const int n_tile1 = min(n_tile0 + d.nt, m.d_out);
  const int tile_len = n_tile1 - n_tile0;  // <= NT: the host tiles with the same constant
  const int nsub = (tile_len + SUB - 1) / SUB;
  const BT bt(B, rank, m.d_out, n_tile0, (uint32_t)tile_len);
  const uint32_t lane_off = bt.off(g, jq);
  const uint32_t pass_bytes = (uint32_t)G * bt.row_bytes;
  const bool lane_on = jq < rank;
  auto b_load = [&](int n0, int p) {  // past the tile (also past the last sub-tile) reads zero
    const bool on = lane_on && n0 + p * G + g < tile_len;
    return bt.load(on ? lane_off + p * pass_bytes : kOutOfRange, (uint32_t)n0 * bt.row_bytes);
  };
  const int b = uniform(d.perm[pos0]);
  const bool row_ok = (unsigned)b < (unsigned)d.num_rows;
  const rsrc_t ry = make_rsrc(m.y + (int64_t)(row_ok ? b : 0) * m.ldy + n_tile0, row_ok ? (uint32_t)tile_len * 2 : 0u);
  auto y_col = [&](int i) { return (i * kDecodeThreads + t) * 8; };  // this thread's 8 outputs of piece i
  auto y_off = [&](int i) { return y_col(i) < tile_len ? (uint32_t)y_col(i) * 2 : kOutOfRange; };
  // Items start at different sub-tiles (by item index) and wrap around, so
  // the blocks in flight are not all at the same offset of their tiles.
  const int rot = item % nsub;
  auto sub_base = [&](int st) { return st < nsub ? ((st + rot) % nsub) * SUB : tile_len; };
  VStage<1> vst;
  vst.issue(d, m, pos0, 1, rank);  // before the B stream: waiting for v does not wait for B
  u32x4 yv[YT];
#pragma unroll
  for (int i = 0; i < YT; ++i) yv[i] = buf_ld16(ry, y_off(i), 0);
  float *b_scale = v_lds + kOneRowDeltaBase + NT;  // Q8: [NT] row scales of the tile
  if constexpr (Q8) {  // requested before B, published by the barrier that ends finish()
    const rsrc_t rs = make_rsrc(bt.scale, (uint32_t)tile_len * 4);
    f32x4_t sl[NT / (kDecodeThreads * 4)];
#pragma unroll
    for (int i = 0; i < NT / (kDecodeThreads * 4); ++i)
      sl[i] = __builtin_bit_cast(f32x4_t, buf_ld16(rs, (uint32_t)(i * kDecodeThreads + t) * 16, 0));
#pragma unroll
    for (int i = 0; i < NT / (kDecodeThreads * 4); ++i) *(f32x4_t *)(b_scale + (i * kDecodeThreads + t) * 4) = sl[i];
  }
  typename BT::raw_t bv[P];
#pragma unroll
  for (int p = 0; p < P; ++p) bv[p] = b_load(sub_base(0), p);
  vst.finish(d, m, scale, v_lds);
  float vv[VPL];  // v past the rank is zero (up to 64)
#pragma unroll
  for (int k = 0; k < VPL; ++k) vv[k] = v_lds[jq + k];
  const V8Split vs = split_v8(vv);
  float *delta = v_lds + kOneRowDeltaBase;  // [NT] sums of the tile
  for (int st = 0; st < nsub; ++st) {
    const int n0 = sub_base(st), n1 = sub_base(st + 1);  // n1 = tile_len after the last: no traffic
    float acc[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      acc[p] = BT::dot(bv[p], vv, vs, 0.f);
      bv[p] = b_load(n1, p);  // unconditional: a branch here would copy the tile registers
    }
    reduce_scatter<P, L>(acc);
#pragma unroll
    for (int ii = 0; ii < PL; ++ii) delta[n0 + (ii + PL * q) * G + g] = acc[ii];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < YT; ++i) {
    float dl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dl[e] = delta[y_col(i) + e];
    if constexpr (Q8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) dl[e] *= b_scale[y_col(i) + e];
    }
    u32x4 o;
    o.x = pack_bf16x2(bf16_to_f32(yv[i].x) + dl[0], bf16_to_f32(yv[i].x >> 16) + dl[1]);
    o.y = pack_bf16x2(bf16_to_f32(yv[i].y) + dl[2], bf16_to_f32(yv[i].y >> 16) + dl[3]);
    o.z = pack_bf16x2(bf16_to_f32(yv[i].z) + dl[4], bf16_to_f32(yv[i].z >> 16) + dl[5]);
    o.w = pack_bf16x2(bf16_to_f32(yv[i].w) + dl[6], bf16_to_f32(yv[i].w >> 16) + dl[7]);
    buf_st16<kScopeDevice>(ry, y_off(i), o);
  }
}

// Block `blk` of the decode expand numbering (nseg: the segments built).  LPR
// = lanes per output row at the largest rank of the launch (8*LPR).
// An item runs at the lane width of its entry's own rank (rank/8 lanes per
// output row, rounded up to a power of two), not at the launch's: a rank-8
// entry in a rank-64 launch streams its B tile with every lane busy and one
// eighth of the load instructions.  The tile and its LDS are the launch's.
template <int LPR>
__device__ __forceinline__ void decode_expand_block(const LayerDesc &d, int blk, int nseg, float *v_lds) {
  const int s = blk / d.items_per_seg;
  if (s >= nseg) return;
  const int it = blk - s * d.items_per_seg;
  const ModuleDesc m = module_of_item(d, it);
  const int tile = it - m.item_base;
  int a, pos0, len;
  if (!load_segment(d, s, it == 0 && d.count_errors, &a, &pos0, &len)) return;
  if (len >= d.long_min) return;  // an SGMV item takes this segment
  lora_adapter_entry_t e;
  if (!load_entry(d, a, m.col, tile == 0 && d.count_errors, &e)) return;
  constexpr int NTC = decode_expand_tile(LPR);
  auto run = [&](auto q8, auto lw) {
    constexpr bool Q8 = decltype(q8)::value;
    constexpr int LW = decltype(lw)::value;
    if constexpr (LW <= LPR) {
      if (len == 1) decode_expand_one_row<LW, Q8, NTC>(d, m, e.B, e.rank, e.scale, pos0, tile, blk, v_lds);
      else decode_expand_rows<LW, Q8, NTC>(d, m, e.B, e.rank, e.scale, pos0, len, tile, v_lds);
    }
  };
  auto by_width = [&](auto q8) {  // e.rank <= d.max_rank (load_entry), so the width is at most LPR
    if (e.rank <= 8) run(q8, std::integral_constant<int, 1>{});
    else if (e.rank <= 16) run(q8, std::integral_constant<int, 2>{});
    else if (e.rank <= 32) run(q8, std::integral_constant<int, 4>{});
    else run(q8, std::integral_constant<int, 8>{});
  };
  if (e.format == LORA_FORMAT_INT8_ROWS) by_width(std::true_type{});
  else by_width(std::false_type{});
}

}  // namespace lora
