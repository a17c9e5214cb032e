// SGMV-style work items for long segments (prefill, and decode batches where
// many rows share one adapter), on the gfx950 bf16 matrix cores.
//
// "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A": SGMV serves
// prefill, where each adapter covers a variable-length run of rows; there a
// prefill pays the adapter read once per chunk of tokens.  "LoRA, quotas and
// noisy neighbours", "One weight read, many adapters": one grouped kernel per
// layer over the row segments.
//
// A segment of L rows is a dense contraction on both sides:
//   shrink  V[L x r]  = X[L x d_in] . A^T     (K = d_in)
//   expand  Y[L x n] += V[L x r] . B^T        (K = r)
// The bytes are dominated by X and the read-modify-write of Y, so both items
// stream those once and take the adapter factors (shared by every row tile of
// a segment) from L2.
//
// Matrix-core lane layout (gfx950, checked on the device):
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) .. +8],
//     B[8*(l/16) .. +8][l%16], and C[4*(l/16) + i][l%16], i < 4.
//
// Shrink: a block takes 128 rows of one segment and one k-chunk of one
//   projection.  x and A go through LDS in rounds of 64 k, loaded as whole
//   128-byte row segments (loading the operand layout straight from memory
//   touches 16 rows per instruction and has every wave re-read A); wave w
//   then reads rows [32w, 32w+32) as two 16-row tiles and every rank column
//   from LDS.  The chunk's partial V goes to the workspace layout of the
//   decode shrink ([chunk][sorted row][rank]).
// Expand: a block takes 64 rows of one segment and an n-tile; the chunk
//   partials of its rows are summed into LDS (times scale), and every wave
//   turns all 64 rows into matrix operands, splitting each fp32 value v into
//   bf16 hi = bf16(v) and lo = bf16(v - hi) so the product keeps about fp32
//   accuracy (B is exact in bf16).  The waves split the columns (32-column
//   steps, round robin), so each B element is read once per block.  The
//   operands are swapped (C = B . V^T) and the B rows permuted so a lane's
//   results are 8 consecutive outputs of one row: y is read and written 16
//   bytes per lane, with DE column steps in flight.
#pragma once

#include "device_common.h"

namespace lora {


// Tile (segment, row tile) of a block among the segments of at least
// long_min rows, in segment order, `rows` rows per tile: one wave-wide scan
// over the segment list.  False when the block has no tile.
__device__ __forceinline__ bool find_long_tile(const LayerDesc &d, int tile, int rows, int *s_out, int *rt_out) {
  const int lane = threadIdx.x & 63;
  const int nseg = min(uniform(*d.num_segments), d.max_seg);
  int base = 0;
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    const int s = s0 + lane;
    int tl = 0;
    if (s < nseg) {
      const int len = d.seg_offsets[s + 1] - d.seg_offsets[s];
      tl = len >= d.long_min ? (len + rows - 1) / rows : 0;
    }
    int inc = tl;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
      const int y = __shfl_up(inc, k, 64);
      if (lane >= k) inc += y;
    }
    const int total = __shfl(inc, 63, 64);
    if (tile < base + total) {
      const uint64_t hit = __ballot(tile >= base + inc - tl && tile < base + inc);
      const int src = __builtin_ctzll(hit);
      *s_out = uniform(s0 + src);
      *rt_out = uniform(tile - (base + __shfl(inc - tl, src, 64)));
      return true;
    }
    base += total;
  }
  return false;
}

// ---------------------------------------------------------------- shrink --

// LDS of the SGMV shrink: two buffers of one round (kShrinkRound k) of the
// x tile [128 rows] and the A tile [64 rank rows], 16-byte pieces swizzled
// by row (piece p of row r sits at p ^ (r & 7)), so the matrix-core reads of
// 16 rows at one k do not collide in one bank.
constexpr int kShrinkRound = 64;                                  // k per round: 128 bytes of a row
constexpr int kShrinkXBytes = kSgmvShrinkRows * kShrinkRound * 2;  // 16 KiB
constexpr int kShrinkABytes = 64 * kShrinkRound * 2;               // 8 KiB
constexpr int kShrinkBufBytes = kShrinkXBytes + kShrinkABytes;
constexpr int kShrinkLdsBytes = 2 * kShrinkBufBytes;
constexpr int kShrinkStages = 4;  // rounds in flight (even)
static_assert(kShrinkStages % 2 == 0, "rounds alternate between two LDS buffers");

__device__ __forceinline__ uint32_t shrink_lds_off(int row, int piece) {
  return (uint32_t)row * (kShrinkRound * 2) + (uint32_t)((piece ^ (row & 7)) * 16);
}

// NT = 16-column tiles of the rank (1, 2 or 4).  The block streams x and A
// through LDS in rounds of 64 k: every thread loads 16-byte pieces with 8
// threads per 128-byte row segment (whole lines), two rounds ahead in
// registers; each wave then reads its matrix operands (32 rows x the whole
// rank) from LDS, so A is read once per block rather than once per wave.
// Q8: a piece of A is 8 int8 values (8 bytes), widened to bf16 (exactly) on
// the way into LDS; the partial of rank row j is multiplied by its scale.
template <int NT, bool Q8>
__device__ __forceinline__ void sgmv_shrink_tile(const LayerDesc &d, const ModuleDesc &m,
                                                 const lora_adapter_entry_t &e, int chunk, int seg0, int len, int rt,
                                                 uint8_t *lds) {
  constexpr int XL = kSgmvShrinkRows * 8 / 256;  // x pieces per thread per round (4)
  constexpr int AROWS = NT * 16;
  constexpr int AL = AROWS * 8 >= 256 ? AROWS * 8 / 256 : 1;  // A pieces per thread per round
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const int rank = e.rank;
  const int k_begin = chunk * d.kc;
  const int k_end = min(k_begin + d.kc, m.d_in);
  const int piece = t & 7;  // this thread's 16-byte piece of a row segment
  // Rows this thread loads: x rows t/8 + 32i of the tile, A rows t/8 + 32i.
  const rsrc_t rx = make_rsrc(m.x, (uint32_t)((int64_t)d.num_rows * m.ldx * 2));
  uint32_t xoff[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int r = rt * kSgmvShrinkRows + i * 32 + (t >> 3);
    const int b = r < len ? d.perm[seg0 + r] : -1;
    xoff[i] = (unsigned)b < (unsigned)d.num_rows ? (uint32_t)((int64_t)b * m.ldx * 2) : kOutOfRange;
  }
  constexpr uint32_t AE = Q8 ? 1 : 2;                                           // bytes per A value
  const uint32_t a_row = Q8 ? lda8_of(m.d_in) : (uint32_t)m.d_in * 2;          // bytes per A row
  const uint8_t *a_vals = static_cast<const uint8_t *>(e.A) + (Q8 ? q8_values_offset(rank) : 0);
  const rsrc_t ra = make_rsrc(a_vals, (uint32_t)rank * a_row);
  uint32_t aoff[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int j = i * 32 + (t >> 3);
    aoff[i] = j < rank && j < AROWS ? (uint32_t)j * a_row : kOutOfRange;
  }
  using araw_t = typename std::conditional<Q8, u32x2, u32x4>::type;
  struct Stage {
    u32x4 x[XL];
    araw_t a[AL];
  };
  auto load = [&](Stage &st, int k0) {  // one round; past the chunk: zero, no traffic
    const int k = k0 + piece * 8;
    const bool kon = k < k_end;
    const uint32_t kb = (uint32_t)k * 2;
#pragma unroll
    for (int i = 0; i < XL; ++i) st.x[i] = buf_ld16(rx, kon && xoff[i] != kOutOfRange ? xoff[i] + kb : kOutOfRange, 0);
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const uint32_t off = kon && aoff[i] != kOutOfRange ? aoff[i] + (uint32_t)k * AE : kOutOfRange;
      if constexpr (Q8) st.a[i] = buf_ld8(ra, off);
      else st.a[i] = buf_ld16(ra, off, 0);
    }
  };
  auto store = [&](const Stage &st, uint8_t *buf) {
#pragma unroll
    for (int i = 0; i < XL; ++i) *(u32x4 *)(buf + shrink_lds_off(i * 32 + (t >> 3), piece)) = st.x[i];
#pragma unroll
    for (int i = 0; i < AL; ++i)
      if (i * 32 + (t >> 3) < AROWS) {
        u32x4 v;
        if constexpr (Q8) v = i8x8_to_bf16x8(st.a[i]);
        else v = st.a[i];
        *(u32x4 *)(buf + kShrinkXBytes + shrink_lds_off(i * 32 + (t >> 3), piece)) = v;
      }
  };
  f32x4_t acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int r_in = lane & 15, g = lane >> 4;
  auto compute = [&](const uint8_t *buf) {
#pragma unroll
    for (int ks = 0; ks < kShrinkRound / 32; ++ks) {
      u32x4 xo[2], ao[NT];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) xo[mt] = *(const u32x4 *)(buf + shrink_lds_off(w * 32 + mt * 16 + r_in, ks * 4 + g));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        ao[nt] = *(const u32x4 *)(buf + kShrinkXBytes + shrink_lds_off(nt * 16 + r_in, ks * 4 + g));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xo[mt]),
                                                                __builtin_bit_cast(bf16x8_t, ao[nt]), acc[mt][nt], 0,
                                                                0, 0);
    }
  };
  // kShrinkStages rounds in flight in registers (a short segment's block
  // is a chain of rounds, each waiting one memory latency, so its time is
  // the chunk's rounds over the rounds in flight); round i is written to
  // LDS buffer i & 1, one barrier per round.  A buffer is rewritten two
  // rounds after it was read, and every wave has passed the barrier in
  // between.  Rounds past the chunk load nothing and add zeros.
  Stage st[kShrinkStages];
#pragma unroll
  for (int i = 0; i < kShrinkStages; ++i) load(st[i], k_begin + i * kShrinkRound);
  const int rounds = (k_end - k_begin + kShrinkRound - 1) / kShrinkRound;
  for (int r = 0; r < rounds; r += kShrinkStages) {
#pragma unroll
    for (int i = 0; i < kShrinkStages; ++i) {
      uint8_t *buf = lds + (i & 1) * kShrinkBufBytes;  // kShrinkStages is even: round r + i has parity i
      store(st[i], buf);
      load(st[i], k_begin + (r + i + kShrinkStages) * kShrinkRound);
      __syncthreads();
      compute(buf);
    }
  }
  // C[4*(l/16) + i][l%16] of tile (mt, nt): row 32w + 16mt + 4*(l/16) + i, column 16nt + l%16.
  float *out = d.part + ((int64_t)(m.part_base + chunk) * d.num_rows + seg0) * d.rs;
  float sa[NT];  // Q8: scales of this lane's rank columns
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int j = nt * 16 + r_in;
    sa[nt] = Q8 && j < rank ? static_cast<const float *>(e.A)[j] : 1.f;
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rt * kSgmvShrinkRows + w * 32 + mt * 16 + g * 4 + i;
      if (r < len) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int j = nt * 16 + r_in;
          if (j < rank) out[(int64_t)r * d.rs + j] = Q8 ? acc[mt][nt][i] * sa[nt] : acc[mt][nt][i];
        }
      }
    }
}

// Block `blk` of the SGMV shrink numbering (row tiles x decode items).
template <int NT>
__device__ __forceinline__ void sgmv_shrink_block(const LayerDesc &d, int blk, uint8_t *lds) {
  const int tile = blk / d.items_per_seg;
  const int it = blk - tile * d.items_per_seg;
  int s, rt;
  if (!find_long_tile(d, tile, kSgmvShrinkRows, &s, &rt)) return;
  const ModuleDesc m = module_of_item(d, it);
  const int chunk = it - m.item_base;
  int a, seg0, len;
  if (!load_segment(d, s, it == 0 && rt == 0 && d.count_errors, &a, &seg0, &len)) return;
  lora_adapter_entry_t e;
  if (!load_entry(d, a, m.col, chunk == 0 && rt == 0 && d.count_errors, &e)) return;
  if (e.format == LORA_FORMAT_INT8_ROWS) sgmv_shrink_tile<NT, true>(d, m, e, chunk, seg0, len, rt, lds);
  else sgmv_shrink_tile<NT, false>(d, m, e, chunk, seg0, len, rt, lds);
}

// ---------------------------------------------------------------- expand --

// KT = 32-wide steps over the rank (1: rank <= 32, 2: rank <= 64).  B rows
// are a multiple of 8 elements apart, so a lane's 8 values of a B row are one
// 16-byte load; past the rank they are zero (masked) or padding that meets
// zeros of V.  Q8: the 8 values are 8 int8 bytes (rows ldb8 bytes apart),
// widened to bf16 exactly; the row scales of the n-tile wait in LDS after V
// and multiply the sums in the y update.  VU = k-chunk partials summed per
// round of V staging (each round waits for the one before).
template <int KT, bool Q8, int VU>
__device__ __forceinline__ void sgmv_expand_tile(const LayerDesc &d, const ModuleDesc &m, const void *B, int rank,
                                                 float scale, int seg0, int len, int rt, int tile, float *v_lds) {
  constexpr int DE = 1;  // 32-column steps per register set (two sets in flight)
  constexpr int NQ = kSgmvExpandRows / 16;  // 16-row tiles per block, all handled by every wave
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const int r_in = lane & 15, g = lane >> 4;
  const int row0 = rt * kSgmvExpandRows;
  const int nrows = min(kSgmvExpandRows, len - row0);
  const int n_tile0 = tile * d.sg_nt;
  const int tile_len = min(n_tile0 + d.sg_nt, m.d_out) - n_tile0;
  // Output rows of this lane, one per 16-row tile (offsets of the tile's
  // first column; out of range past the segment).
  const rsrc_t ry = make_rsrc(m.y, (uint32_t)((int64_t)d.num_rows * m.ldy * 2));
  uint32_t yrow[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int r = row0 + q * 16 + r_in;
    const int b = r < len ? d.perm[seg0 + r] : -1;
    yrow[q] = (unsigned)b < (unsigned)d.num_rows ? (uint32_t)(((int64_t)b * m.ldy + n_tile0) * 2) : kOutOfRange;
  }
  const uint32_t brow = Q8 ? (uint32_t)ldb8_of(rank) : (uint32_t)((rank + 7) & ~7) * 2;  // bytes per B row
  constexpr uint32_t BE = Q8 ? 1 : 2;                                                       // bytes per B value
  const uint8_t *b_vals = static_cast<const uint8_t *>(B) + (Q8 ? q8_values_offset(m.d_out) : 0);
  const rsrc_t rb = make_rsrc(b_vals + (int64_t)n_tile0 * brow, (uint32_t)tile_len * brow);
  float *b_scale = v_lds + kSgmvExpandRows * 64;  // Q8: [kSgmvExpandCols] row scales of the tile
  // Wave w takes the 32-column steps w, w+4, w+8, ... of the tile.  Matrix
  // row i of half h stands for column n0 + 8*(i/4) + 4h + i%4, so the results
  // of the two halves give lane l the 8 consecutive columns n0 + 8*(l/16) ..
  // +8 of its row: y moves 16 bytes per lane.
  auto col0 = [&](int step) { return (4 * step + w) * 32; };
  auto y_off = [&](int q, int n0) {
    const int nc = n0 + 8 * g;
    return yrow[q] != kOutOfRange && nc < tile_len ? yrow[q] + (uint32_t)nc * 2 : kOutOfRange;
  };
  auto load_b = [&](int n0, int h, int kt) {  // B[col][32kt + 8g .. +8]; zero past the rank / tile
    const int n = n0 + 8 * (r_in >> 2) + 4 * h + (r_in & 3);
    const int k = kt * 32 + 8 * g;
    const uint32_t off = k < rank && n < tile_len ? (uint32_t)n * brow + (uint32_t)k * BE : kOutOfRange;
    if constexpr (Q8) return buf_ld8(rb, off);
    else return buf_ld16(rb, off, 0);
  };
  using braw_t = typename std::conditional<Q8, u32x2, u32x4>::type;
  struct Set {
    braw_t bop[DE][2][KT];
    u32x4 yv[DE][NQ];
  };
  auto issue = [&](Set &st, int step) {  // steps step .. step+DE; past the tile: zero, no traffic
#pragma unroll
    for (int u = 0; u < DE; ++u) {
      const int n0 = col0(step + u);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) st.bop[u][h][kt] = load_b(n0, h, kt);
#pragma unroll
      for (int q = 0; q < NQ; ++q) st.yv[u][q] = buf_ld16(ry, y_off(q, n0), 0);
    }
  };
  // V rows of the tile (times scale) into LDS, [64][64] fp32; the first
  // round of its loads goes out before the first register set.
  VStage<kSgmvExpandRows, VU> vst;
  vst.issue(d, m, seg0 + row0, nrows, rank);
  Set s0, s1;
  issue(s0, 0);
  if constexpr (Q8) {  // published by the barrier that ends finish()
    const rsrc_t rs = make_rsrc(static_cast<const float *>(B) + n_tile0, (uint32_t)tile_len * 4);
    for (int n = t * 4; n < tile_len; n += kDecodeThreads * 4)
      *(f32x4_t *)(b_scale + n) = __builtin_bit_cast(f32x4_t, buf_ld16(rs, (uint32_t)n * 4, 0));
  }
  vst.finish(d, m, scale, v_lds);
  // All 64 rows as hi/lo bf16 operands: tile q, lane l holds row 16q + l%16,
  // k = 32kt + 8*(l/16) .. +8.
  V8Split vop[NQ][KT];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) vop[q][kt] = split_v8(v_lds + (q * 16 + r_in) * 64 + kt * 32 + 8 * g);
  auto finish = [&](const Set &st, int step) {
#pragma unroll
    for (int u = 0; u < DE; ++u) {
      const int n0 = col0(step + u);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        f32x4_t acc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          acc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            u32x4 bw;
            if constexpr (Q8) bw = i8x8_to_bf16x8(st.bop[u][h][kt]);
            else bw = st.bop[u][h][kt];
            const bf16x8_t bo = __builtin_bit_cast(bf16x8_t, bw);
            acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bo, __builtin_bit_cast(bf16x8_t, vop[q][kt].hi), acc[h],
                                                             0, 0, 0);
            acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bo, __builtin_bit_cast(bf16x8_t, vop[q][kt].lo), acc[h],
                                                             0, 0, 0);
          }
        }
        if constexpr (Q8) {  // columns n0 + 8*(l/16) + 4h + i
          const int nc = min(n0 + 8 * g, kSgmvExpandCols - 8);  // past the tile: the store is dropped
          const f32x4_t s0v = *(const f32x4_t *)(b_scale + nc), s1v = *(const f32x4_t *)(b_scale + nc + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[0][i] *= s0v[i];
            acc[1][i] *= s1v[i];
          }
        }
        const u32x4 yv = st.yv[u][q];
        u32x4 o;
        o.x = pack_bf16x2(bf16_to_f32(yv.x) + acc[0][0], bf16_to_f32(yv.x >> 16) + acc[0][1]);
        o.y = pack_bf16x2(bf16_to_f32(yv.y) + acc[0][2], bf16_to_f32(yv.y >> 16) + acc[0][3]);
        o.z = pack_bf16x2(bf16_to_f32(yv.z) + acc[1][0], bf16_to_f32(yv.z >> 16) + acc[1][1]);
        o.w = pack_bf16x2(bf16_to_f32(yv.w) + acc[1][2], bf16_to_f32(yv.w >> 16) + acc[1][3]);
        buf_st16(ry, y_off(q, n0), o);
      }
    }
  };
  const int steps = (tile_len + 127) / 128;  // per wave (upper bound; extra steps are masked)
  for (int i = 0; i < steps; i += 2 * DE) {
    issue(s1, i + DE);
    __builtin_amdgcn_sched_barrier(0);  // keep the requests ahead of the math
    finish(s0, i);
    issue(s0, i + 2 * DE);
    __builtin_amdgcn_sched_barrier(0);
    finish(s1, i + DE);
  }
}

// Block `blk` of the SGMV expand numbering (row tiles x sg_items).
template <int KT, int VU>
__device__ __forceinline__ void sgmv_expand_block(const LayerDesc &d, int blk, float *v_lds) {
  const int tile_idx = blk / d.sg_items;
  const int it = blk - tile_idx * d.sg_items;
  int s, rt;
  if (!find_long_tile(d, tile_idx, kSgmvExpandRows, &s, &rt)) return;
  const ModuleDesc m = module_of_item<true>(d, it);
  const int tile = it - m.sg_item_base;
  int a, seg0, len;
  if (!load_segment(d, s, it == 0 && rt == 0 && d.count_errors, &a, &seg0, &len)) return;
  lora_adapter_entry_t e;
  if (!load_entry(d, a, m.col, tile == 0 && rt == 0 && d.count_errors, &e)) return;
  if (e.format == LORA_FORMAT_INT8_ROWS)
    sgmv_expand_tile<KT, true, VU>(d, m, e.B, e.rank, e.scale, seg0, len, rt, tile, v_lds);
  else
    sgmv_expand_tile<KT, false, VU>(d, m, e.B, e.rank, e.scale, seg0, len, rt, tile, v_lds);
}

}  // namespace lora
