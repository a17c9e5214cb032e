// One-launch decode: the grouping of the rows by adapter, the shrink and the
// expand of every projection in a single launch, for a small decode batch
// (lora_decode_layer).
//
// "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A": one batched
// kernel receives the batch and the index vector mapping each sequence to an
// adapter slot and gathers each sequence's adapter inside the kernel; the
// cost of the delta is bandwidth (each distinct adapter in the batch is read
// once per step), so on a small decode batch every launch and every
// dependent round trip before the factor streams counts.
// "LoRA, quotas and noisy neighbours", "One weight read, many adapters": the
// rows are tagged and grouped, and the update is applied in registers.
//
// Blocks.  Block (item it, row t) takes expand tile c of one projection for
// row t and, when t is the first, fifth, ... row of its adapter's segment,
// the next rows of that segment up to 4 (blocks of the other rows leave at
// once).  It reads the ids of the batch and its row's table entry itself, so
// no block waits for a grouping pass, and then
//   1. requests its row's tile of y;
//   2. computes v = A.x of its rows (every k of A, one pass over A for all of
//      them), times the entry's scale, into LDS;
//   3. loads its tile of B (kOnePassPasses load passes of the block, kept in
//      registers) and adds B.v to its rows' tiles of y.
// No block hands anything to another: the blocks of one (rows, projection)
// each compute the same v.  They sit on one XCD (the grid is item-major over
// a multiple of 8 rows and blocks are dealt to the XCDs in turn) and stream
// A in the same order at the same time, so the repeated reads of A are
// served by that XCD's L2 and A crosses HBM about once per group of rows.
// Block 0 writes the segments and the status word as lora_build_segments
// followed by lora_apply_layer would; it runs beside the others.
#pragma once

#include "block_sort.h"
#include "decode_items.h"

namespace lora {

// LDS of a one-launch block (bytes).
constexpr int kOpRowsOff = 0;                                 // 256 ints: the segment's rows, ascending
constexpr int kOpMiscOff = 1024;                              // 64 ints: ballots and broadcasts
constexpr int kOpRowsPerBlock = 4;                            // rows of a segment per block: one pass over A
constexpr int kOpVOff = 1280;                                 // v [kOpRowsPerBlock][64] (times scale)
constexpr int kOpMaxTile = kOnePassPasses * kDecodeThreads;   // largest tile (one lane per B row)
constexpr int kOpDeltaOff = kOpVOff + kOpRowsPerBlock * 64 * 4;  // one tile of sums
constexpr int kOnePassLdsBytes = kOpDeltaOff + kOpMaxTile * 4;
static_assert(kOpMaxTile % (kDecodeThreads * 8) == 0, "the y update takes whole steps of 8 columns per thread");

// Block-wide sum of one int per thread (256 threads); s_w holds 4 ints.
__device__ __forceinline__ int op_block_sum(int x, int *s_w) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) x += __shfl_xor(x, k, 64);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = x;
  __syncthreads();
  const int total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
  __syncthreads();  // s_w may be reused
  return total;
}

// The segment of row t: its rows, ascending, in LDS at kOpRowsOff, their
// count in *len_out and row t's place among them in *pos_out.  `id` is row
// t's slot, in [0, num_slots) (uniform); idu is row u's id in thread u (-1
// past the batch).
__device__ __forceinline__ void op_row_segment(int t, int id, int idu, uint8_t *lds, int *len_out, int *pos_out) {
  const int u = threadIdx.x, lane = u & 63, w = u >> 6;
  int *s_rows = reinterpret_cast<int *>(lds + kOpRowsOff);
  int *s_misc = reinterpret_cast<int *>(lds + kOpMiscOff);
  const uint64_t mm = __ballot(idu == id);
  const uint64_t me = __ballot(idu == id && u < t);
  if (lane == 0) {
    s_misc[w] = __popcll(mm);
    s_misc[4 + w] = __popcll(me);
  }
  __syncthreads();
  int before = 0, len = 0, earlier = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    before += k < w ? s_misc[k] : 0;
    len += s_misc[k];
    earlier += s_misc[4 + k];
  }
  if (idu == id) {
    const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(mm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mm, 0u));
    s_rows[before + in_wave] = u;
  }
  __syncthreads();
  *len_out = uniform(len);
  *pos_out = uniform(earlier);
}

// The number of distinct valid slot ids of the batch below slot a: its
// segment's index in slot order.  A bitmap of the ids (kOnePassMaxSlots
// bits) is built in LDS at `bm`; idu is row u's valid id in thread u (-1:
// none).
__device__ __forceinline__ int op_slot_rank(int a, int idu, uint32_t *bm, int *s_w) {
  const int u = threadIdx.x;
  for (int i = u; i < kOnePassMaxSlots / 32; i += kDecodeThreads) bm[i] = 0u;
  __syncthreads();
  if ((unsigned)idu < (unsigned)kOnePassMaxSlots) atomicOr(&bm[idu >> 5], 1u << (idu & 31));
  __syncthreads();
  int below = 0;
  for (int i = u; i < kOnePassMaxSlots / 32; i += kDecodeThreads) {
    const uint32_t word = bm[i];
    if (i < (a >> 5)) below += __popc(word);
    else if (i == (a >> 5)) below += __popc(word & ((1u << (a & 31)) - 1u));
  }
  return uniform(op_block_sum(below, s_w));
}

// v of rows rows[0, nr) over every k of A, times scale, into v_lds[r*64 + j]
// (zero for j in [rank, 64)).  The 4 waves split A's rows (jw = ceil(rank/4)
// each); a lane takes 16 bytes of a row per step (8 bf16 values, or 16 int8
// values widened to bf16 in registers against two 16-byte pieces of x), and
// U steps of loads are requested together.  A is read with ordinary loads:
// the other blocks of this segment read the same lines at the same time, and
// the XCD's L2 serves them.  Ends with a block barrier.
template <int JW, int RG, bool Q8>
__device__ __forceinline__ void op_shrink_rows(const ModuleDesc &m, const lora_adapter_entry_t &e, const int *rows,
                                               int nr, float *v_lds) {
  constexpr int VPL = Q8 ? 16 : 8;  // k per lane and step
  // steps in flight: at least 8 loads of A per lane for one row of x
  // (several rows of x give enough loads with one step)
  constexpr int U = RG == 1 ? (8 / JW > 2 ? 8 / JW : 2) : 1;
  constexpr int STEP = 64 * VPL;
  const int lane = threadIdx.x & 63;
  const int rank = e.rank;
  const int jw = (rank + 3) >> 2;
  const int j0 = wave_id() * jw;
  const uint32_t x_row_bytes = (uint32_t)m.d_in * 2;
  const uint32_t a_row_bytes = Q8 ? lda8_of(m.d_in) : x_row_bytes;
  rsrc_t rx[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int b = r < nr ? uniform(rows[r]) : 0;
    rx[r] = make_rsrc(m.x + (int64_t)b * m.ldx, r < nr ? x_row_bytes : 0u);
  }
  const uint8_t *a_vals = static_cast<const uint8_t *>(e.A) + (Q8 ? q8_values_offset(rank) : 0);
  const rsrc_t ra = make_rsrc(a_vals, (uint32_t)rank * a_row_bytes);
  float acc[JW * RG];
#pragma unroll
  for (int i = 0; i < JW * RG; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < m.d_in; k0 += U * STEP) {
    u32x4 av[U][JW], xv[U][RG], xw[U][RG];
#pragma unroll
    for (int s = 0; s < U; ++s) {
      const int k = k0 + s * STEP + lane * VPL;
      const bool in = k < m.d_in;  // past d_in: zero (a lane's values never straddle it: d_in % 8 == 0)
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
        av[s][jj] = __builtin_amdgcn_raw_buffer_load_b128(
            ra, in && jj < jw && j0 + jj < rank ? (uint32_t)k * (Q8 ? 1 : 2) : kOutOfRange,
            (uint32_t)(j0 + jj) * a_row_bytes, 0);
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        xv[s][r] = buf_ld16(rx[r], in ? (uint32_t)k * 2 : kOutOfRange, 0);
        if constexpr (Q8) xw[s][r] = buf_ld16(rx[r], in ? (uint32_t)k * 2 + 16 : kOutOfRange, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < U; ++s)
#pragma unroll
      for (int jj = 0; jj < JW; ++jj) {
        if constexpr (Q8) {
          const u32x4 lo = i8x8_to_bf16x8(u32x2{av[s][jj].x, av[s][jj].y});
          const u32x4 hi = i8x8_to_bf16x8(u32x2{av[s][jj].z, av[s][jj].w});
#pragma unroll
          for (int r = 0; r < RG; ++r)
            acc[jj * RG + r] = dot8_bf16(hi, xw[s][r], dot8_bf16(lo, xv[s][r], acc[jj * RG + r]));
        } else {
#pragma unroll
          for (int r = 0; r < RG; ++r) acc[jj * RG + r] = dot8_bf16(av[s][jj], xv[s][r], acc[jj * RG + r]);
        }
      }
  }
  reduce_scatter<JW * RG, 64>(acc);
  // zero the staged rows (the entries past the rank stay zero), then write the sums
  for (int i = threadIdx.x; i < RG * 64; i += kDecodeThreads) v_lds[i] = 0.f;
  __syncthreads();
  const float *a_scale = static_cast<const float *>(e.A);
  constexpr int NV = JW * RG;
  auto put = [&](int idx, float val) {
    const int jj = idx / RG, r = idx % RG;
    if (r < nr && jj < jw && j0 + jj < rank) v_lds[r * 64 + j0 + jj] = (Q8 ? val * a_scale[j0 + jj] : val) * e.scale;
  };
  if constexpr (NV >= 64) {
#pragma unroll
    for (int i = 0; i < NV / 64; ++i) put(i + (NV / 64) * lane, acc[i]);
  } else {
    constexpr int GS = 64 / NV;
    if (lane % GS == 0) put(lane / GS, acc[0]);
  }
  __syncthreads();
}

// The B tile of a block in registers: P passes, LPR lanes per output row,
// 8 values per lane (bf16: 16 bytes; Q8: 8 int8 values, 8 bytes).
template <int LPR, bool Q8>
struct OpBTile {
  static constexpr int G = kDecodeThreads / LPR;  // output rows per pass
  static constexpr int P = kOnePassPasses;
  using raw_t = typename std::conditional<Q8, u32x2, u32x4>::type;
  raw_t v[P];

  // Rows [n0, n0 + tile_len) of B for the rank `rank` entry B.
  __device__ __forceinline__ void load(const void *B, int rank, int d_out, int n0, int tile_len) {
    const int t = threadIdx.x, g = t / LPR, jq = (t % LPR) * 8;
    const uint8_t *base = static_cast<const uint8_t *>(B);
    uint32_t row_bytes;
    if constexpr (Q8) {
      row_bytes = (uint32_t)ldb8_of(rank);
      base += q8_values_offset(d_out);
    } else {
      row_bytes = (uint32_t)b_stride(rank) * 2;
    }
    const rsrc_t r = make_rsrc(base + (int64_t)n0 * row_bytes, (uint32_t)tile_len * row_bytes);
    const bool lane_on = jq < rank;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int n = p * G + g;
      const uint32_t off = lane_on && n < tile_len ? (uint32_t)n * row_bytes + (uint32_t)jq * (Q8 ? 1 : 2)
                                                   : kOutOfRange;
      if constexpr (Q8) v[p] = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNonTemporal);
      else v[p] = buf_ld16_stream(r, off, 0);
    }
  }
};

// This thread's first 16 bytes of y in row `row` of the tile at n0: the
// y update's first step, requested ahead of it.
__device__ __forceinline__ u32x4 op_load_y0(const ModuleDesc &m, int row, int n0, int tile_len) {
  const rsrc_t ry = make_rsrc(m.y + (int64_t)row * m.ldy + n0, (uint32_t)tile_len * 2);
  const int t = threadIdx.x;
  return buf_ld16(ry, t * 8 < tile_len ? (uint32_t)t * 16 : kOutOfRange, 0);
}

// y += delta for one row over one tile: the tile's sums wait in LDS; each
// thread takes 8 consecutive outputs (16 bytes of y) per step.  y0 holds the
// first step's y (op_load_y0), requested early.  Q8: the B row scales
// multiply the sums here.  Ends with a block barrier.
template <bool Q8>
__device__ __forceinline__ void op_update_y(const ModuleDesc &m, const void *B, int row, int n0, int tile_len,
                                            const float *delta, u32x4 y0) {
  const int t = threadIdx.x;
  const rsrc_t ry = make_rsrc(m.y + (int64_t)row * m.ldy + n0, (uint32_t)tile_len * 2);
  // 8 columns per thread and step: a tile of up to kOpMaxTile columns takes
  // kOpMaxTile / 2048 steps
#pragma unroll
  for (int step = 0; step < kOpMaxTile / (kDecodeThreads * 8); ++step) {
    const int col = (step * kDecodeThreads + t) * 8;
    if (col >= tile_len) break;
    const u32x4 yv = step == 0 ? y0 : buf_ld16(ry, (uint32_t)col * 2, 0);
    float dl[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) dl[k] = delta[col + k];
    if constexpr (Q8) {
      const rsrc_t rs = make_rsrc(static_cast<const float *>(B) + n0, (uint32_t)tile_len * 4);
      const f32x4_t s0 = __builtin_bit_cast(f32x4_t, buf_ld16(rs, (uint32_t)col * 4, 0));
      const f32x4_t s1 = __builtin_bit_cast(f32x4_t, buf_ld16(rs, (uint32_t)col * 4 + 16, 0));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dl[k] *= s0[k];
        dl[k + 4] *= s1[k];
      }
    }
    u32x4 o;
    o.x = pack_bf16x2(bf16_to_f32(yv.x) + dl[0], bf16_to_f32(yv.x >> 16) + dl[1]);
    o.y = pack_bf16x2(bf16_to_f32(yv.y) + dl[2], bf16_to_f32(yv.y >> 16) + dl[3]);
    o.z = pack_bf16x2(bf16_to_f32(yv.z) + dl[4], bf16_to_f32(yv.z >> 16) + dl[5]);
    o.w = pack_bf16x2(bf16_to_f32(yv.w) + dl[6], bf16_to_f32(yv.w >> 16) + dl[7]);
    buf_st16<kScopeDevice>(ry, (uint32_t)col * 2, o);
  }
  __syncthreads();  // delta is rewritten by the next row
}

// B.v for the staged rows rows[0, nr) over the block's tile (B in bt, v in
// v_lds), added to their y.  With use_pre, `pre` holds the first row's
// op_load_y0; the other rows request theirs in the update (requesting each
// one a row ahead measured no faster).
template <int LPR, bool Q8>
__device__ __forceinline__ void op_expand_rows(const ModuleDesc &m, const lora_adapter_entry_t &e,
                                               const OpBTile<LPR, Q8> &bt, int n0, int tile_len, const int *rows,
                                               int nr, const float *v_lds, float *delta, u32x4 pre, bool use_pre) {
  using BT = OpBTile<LPR, Q8>;
  constexpr int P = BT::P, G = BT::G, PL = P / LPR;
  const int t = threadIdx.x, g = t / LPR, q = t % LPR, jq = q * 8;
  for (int i = 0; i < nr; ++i) {
    float vv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) vv[k] = v_lds[i * 64 + jq + k];
    const V8Split vs = split_v8(vv);
    float acc[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if constexpr (Q8) {
        u32x2 raw = bt.v[p];
        asm volatile("" : "+v"(raw));  // widened per row: int8 B stays 8 bytes per pass in registers
        acc[p] = dot8_bf16_split(i8x8_to_bf16x8(raw), vs, 0.f);
      } else {
        acc[p] = dot8_bf16_split(bt.v[p], vs, 0.f);
      }
    }
    reduce_scatter<P, LPR>(acc);
#pragma unroll
    for (int ii = 0; ii < PL; ++ii) {
      const int n = (ii + PL * q) * G + g;
      if (n < tile_len) delta[n] = acc[ii];
    }
    __syncthreads();
    op_update_y<Q8>(m, e.B, uniform(rows[i]), n0, tile_len, delta,
                    use_pre && i == 0 ? pre : op_load_y0(m, uniform(rows[i]), n0, tile_len));
  }
}

// Tiles [c*tpb, c*tpb + tpb) of projection m for the segment of row `row` (slot a, entry e; idu:
// row u's id in thread u), unless the segment lies past the caller's bound
// (checked when bound_check: the first max_seg slots in ascending order keep
// their delta).  CLS: the launch's rank class (rows of A per wave, lanes per
// B row).
template <int CLS, bool Q8>
__device__ __forceinline__ void op_delta(const ModuleDesc &m, const lora_adapter_entry_t &e, int c, int tpb, int row,
                                         int a, int idu, bool bound_check, int max_seg, uint8_t *lds) {
  constexpr int JW = 2 << CLS;
  constexpr int LPR = 1 << CLS;
  const int *s_rows = reinterpret_cast<const int *>(lds + kOpRowsOff);
  float *v_lds = reinterpret_cast<float *>(lds + kOpVOff);
  float *delta = reinterpret_cast<float *>(lds + kOpDeltaOff);
  const int tile0 = c * tpb;
  const int tiles = min(tpb, m.op_n_tiles - tile0);  // this block's tiles: [tile0, tile0 + tiles)
  const int n0 = tile0 * m.op_nt;
  const int tile_len = min(m.op_nt, m.d_out - n0);
  // 1. the row's first tile of y, requested before anything waits
  OpBTile<LPR, Q8> bt;
  const u32x4 y_pre = op_load_y0(m, row, n0, tile_len);
  // the segment of the row, while those loads are in flight: the ballots
  // compare against a copy of the slot made here, so the wait for the ids
  // cannot be hoisted above the loads
  int a_here = a;
  asm volatile("" : "+s"(a_here));
  int len, pos;
  op_row_segment(row, a_here, idu, lds, &len, &pos);
  // the block of every kOpRowsPerBlock-th row of the segment takes that row
  // and the next ones (one pass over A for all of them); the rest leave
  if (pos % kOpRowsPerBlock != 0) return;
  if (bound_check &&  // the caller's bound on the segments: slots past it get no delta (counted by block 0)
      op_slot_rank(a_here, idu, reinterpret_cast<uint32_t *>(delta), reinterpret_cast<int *>(lds + kOpMiscOff)) >=
          max_seg)
    return;
  const int nr = min(kOpRowsPerBlock, len - pos);
  const int *my_rows = s_rows + pos;  // my_rows[0] == row
  // 2. v of the rows (every k of A), 3. their tiles of y; B follows the
  // shrink: the registers of both do not fit
  if (nr == 1) {  // a row whose adapter no other row shares: the case to be fast
    op_shrink_rows<JW, 1, Q8>(m, e, my_rows, 1, v_lds);
    for (int i = 0; i < tiles; ++i) {
      const int ni = n0 + i * m.op_nt;
      const int len_i = min(m.op_nt, m.d_out - ni);
      bt.load(e.B, e.rank, m.d_out, ni, len_i);
      op_expand_rows<LPR, Q8>(m, e, bt, ni, len_i, my_rows, 1, v_lds, delta, y_pre, i == 0);
    }
    return;
  }
  op_shrink_rows<JW, kOpRowsPerBlock, Q8>(m, e, my_rows, nr, v_lds);
  for (int i = 0; i < tiles; ++i) {
    const int ni = n0 + i * m.op_nt;
    const int len_i = min(m.op_nt, m.d_out - ni);
    bt.load(e.B, e.rank, m.d_out, ni, len_i);
    op_expand_rows<LPR, Q8>(m, e, bt, ni, len_i, my_rows, nr, v_lds, delta, y_pre, i == 0);
  }
}

// Exclusive scan of one int per thread over the 256-thread block; *total
// gets the sum.  s_w holds 4 ints.
__device__ __forceinline__ int op_block_scan(int x, int *total, int *s_w) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) {
    const int y = __shfl_up(inc, k, 64);
    if (lane >= k) inc += y;
  }
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int v = s_w[k];
    before += k < w ? v : 0;
    sum += v;
  }
  *total = sum;
  __syncthreads();  // s_w may be reused
  return before + inc - x;
}

// Block 0 of the grid: the segments and the status word as
// lora_build_segments followed by lora_apply_layer leave them.  A stable
// radix sort on the slot (block_sort.h) gives every row its place in slot
// order; a scan over the sorted ids then marks where each segment starts.
// The table entries of a kept segment's projections are requested together.
// The status word gets the rows whose
// id is >= num_slots, the rows of segments past the bound, and one per (kept
// segment, projection) whose entry cannot be applied.
__device__ __forceinline__ void op_build(const OnePassDesc &od, uint8_t *lds) {
  const LayerDesc &d = od.L;
  const int t = threadIdx.x, n = d.num_rows;
  auto s_key = reinterpret_cast<int (*)[kDecodeThreads]>(lds);         // [2][256] keys, sorted
  auto s_row = reinterpret_cast<int (*)[kDecodeThreads]>(lds + 2048);  // [2][256] their rows
  int *s_start = reinterpret_cast<int *>(lds + 4096);                  // [256] sorted start of each segment
  int *s_w = reinterpret_cast<int *>(lds + 5120);
  int key = d.num_slots, bad = 0;  // num_slots: no segment (base only, a bad id, or past the batch)
  if (t < n) {
    const int r = od.ids[t];
    if (r >= d.num_slots) bad = 1;
    else if (r >= 0) key = r;
  }
  int row = t;
  // rows in slot order, rows of one slot ascending (a stable sort on the slot)
  const int fb = block_radix_sort<kDecodeThreads>(&key, &row, key_bits(d.num_slots), s_key, s_row, s_w);
  // thread t now looks at sorted place t
  const int sid = key;
  const bool valid = sid < d.num_slots;
  const bool starts = valid && (t == 0 || s_key[fb][t - 1] != sid);
  int nseg;
  const int seg = op_block_scan(starts ? 1 : 0, &nseg, s_w);
  const int nvalid = op_block_sum(valid ? 1 : 0, s_w);
  const int nbad = op_block_sum(bad, s_w);
  if (valid) od.seg.perm[t] = row;
  if (starts) {
    od.seg.seg_offsets[seg] = t;
    od.seg.seg_adapter[seg] = sid;
    s_start[seg] = t;
  }
  __syncthreads();
  const int kept = min(nseg, d.max_seg);
  const int kept_rows = kept < nseg ? s_start[kept] : nvalid;
  const bool kept_start = starts && seg < kept;
  const int len = starts ? (seg + 1 < nseg ? s_start[seg + 1] : nvalid) - t : 0;
  int tiles = 0;  // SGMV tiles of the kept segments: expand | shrink << 16, as lora_build_segments counts them
  if (kept_start && n >= kLongSegRows && len >= kLongSegRows)
    tiles = (len + kSgmvExpandRows - 1) / kSgmvExpandRows | ((len + kSgmvShrinkRows - 1) / kSgmvShrinkRows) << 16;
  const int all_tiles = op_block_sum(tiles, s_w);
  int errs = 0;
  if (kept_start) {
    lora_adapter_entry_t es[kMaxModules];
#pragma unroll
    for (int i = 0; i < kMaxModules; ++i)
      if (i < d.n_active) es[i] = d.table[(int64_t)sid * d.table_cols + kernel_desc().mod[i].col];
#pragma unroll
    for (int i = 0; i < kMaxModules; ++i)
      if (i < d.n_active && es[i].rank != 0 && !entry_ok(es[i], d.max_rank)) ++errs;
  }
  const int nerr = op_block_sum(errs, s_w);
  if (t == 0) {
    if (kept == nseg) od.seg.seg_offsets[nseg] = nvalid;
    *od.seg.num_segments = kept;
    *od.seg.status = nbad + (nvalid - kept_rows) + nerr;
    od.seg.tile_counts[0] = all_tiles >> 16;
    od.seg.tile_counts[1] = all_tiles & 0xffff;
  }
}

}  // namespace lora
