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
// Matrix-core lane layouts (gfx950, checked on the device):
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) .. +8],
//     B[8*(l/16) .. +8][l%16], and C[4*(l/16) + i][l%16], i < 4.
//   v_mfma_f32_16x16x16bf16_1k: the same with 4 values of K per lane.
//
// Shrink: a block takes 128 rows of one segment and one k-chunk of one
//   projection; wave w owns rows [32w, 32w+32) as two 16-row tiles and every
//   rank column; per 32-wide k step a lane loads 16 bytes of x per row tile
//   and 16 bytes of each A row tile, with D steps in flight (a ring of
//   registers refilled as each step is consumed).  The chunk's partial V goes
//   to the workspace layout of the decode shrink ([chunk][sorted row][rank]).
// Expand: a block takes 64 rows of one segment and an n-tile; the chunk
//   partials of its rows are summed into LDS (times scale), and each wave
//   turns its 16 rows into matrix operands, splitting each fp32 value v into
//   bf16 hi = bf16(v) and lo = bf16(v - hi) so the product keeps about fp32
//   accuracy (B is exact in bf16).  The operands are swapped (C = B . V^T)
//   so a lane's four results are four consecutive outputs of one row: y is
//   read and written 8 bytes per lane, with DE column steps in flight.
#pragma once

#include "device_common.h"

namespace lora {

constexpr int kSgmvShrinkRows = 128;  // rows per shrink block: 4 waves x 2 tiles of 16
constexpr int kSgmvExpandRows = 64;   // rows per expand block: 4 waves x 16

// Tile (segment, row tile) of a block among the segments of at least
// long_min rows, in segment order, `rows` rows per tile: one wave-wide scan
// over the segment list.  False when the block has no tile.
__device__ __forceinline__ bool find_long_tile(const LayerDesc &d, int tile, int rows, int *s_out, int *rt_out) {
  const int lane = threadIdx.x & 63;
  const int nseg = min(uniform(*d.num_segments), min(d.num_rows, d.num_slots));
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

// NT = 16-column tiles of the rank per wave (1, 2 or 4).
template <int NT>
__device__ __forceinline__ void sgmv_shrink_block(const LayerDesc &d, int blk) {
  constexpr int D = NT >= 4 ? 2 : 4;  // k steps in flight
  const int lane = threadIdx.x & 63, w = wave_id();
  const int tile = blk / d.items_per_seg;
  const int it = blk - tile * d.items_per_seg;
  int s, rt;
  if (!find_long_tile(d, tile, kSgmvShrinkRows, &s, &rt)) return;
  const ModuleDesc m = module_of_item(d, it);
  const int chunk = it - m.item_base;
  int a, seg0, len;
  if (!load_segment(d, s, it == 0 && rt == 0, &a, &seg0, &len)) return;
  lora_adapter_entry_t e;
  if (!load_entry(d, a, m.col, chunk == 0 && rt == 0, &e)) return;
  const int rank = e.rank;
  const int k_begin = chunk * d.kc;
  const int k_end = min(k_begin + d.kc, m.d_in);
  const int r_in = lane & 15, kq = (lane >> 4) * 8;
  // x rows of this wave's two 16-row tiles (zero past the segment).
  const rsrc_t rx = make_rsrc(m.x, (uint32_t)((int64_t)d.num_rows * m.ldx * 2));
  uint32_t xoff[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = rt * kSgmvShrinkRows + w * 32 + mt * 16 + r_in;
    const int b = r < len ? d.perm[seg0 + r] : -1;
    xoff[mt] = (unsigned)b < (unsigned)d.num_rows ? (uint32_t)((int64_t)b * m.ldx * 2) : kOutOfRange;
  }
  const rsrc_t ra = make_rsrc(e.A, (uint32_t)rank * m.d_in * 2);
  uint32_t aoff[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int j = nt * 16 + r_in;
    aoff[nt] = j < rank ? (uint32_t)j * m.d_in * 2 : kOutOfRange;
  }
  auto load = [&](int k, u32x4(&xv)[2], u32x4(&av)[NT]) {  // past the chunk: zero, no traffic
    const bool kon = k + kq < k_end;
    const uint32_t kb = (uint32_t)(k + kq) * 2;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) xv[mt] = buf_ld16(rx, kon && xoff[mt] != kOutOfRange ? xoff[mt] + kb : kOutOfRange, 0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      av[nt] = buf_ld16(ra, kon && aoff[nt] != kOutOfRange ? aoff[nt] + kb : kOutOfRange, 0);
  };
  f32x4_t acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4 xb[D][2], ab[D][NT];
#pragma unroll
  for (int u = 0; u < D; ++u) load(k_begin + 32 * u, xb[u], ab[u]);
  for (int k = k_begin; k < k_end; k += 32 * D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xb[u][mt]),
                                                                __builtin_bit_cast(bf16x8_t, ab[u][nt]), acc[mt][nt],
                                                                0, 0, 0);
      load(k + 32 * (u + D), xb[u], ab[u]);
    }
  }
  // C[4*(l/16) + i][l%16] of tile (mt, nt): row 32w + 16mt + 4*(l/16) + i, column 16nt + l%16.
  float *out = d.part + ((int64_t)(m.part_base + chunk) * d.num_rows + seg0) * d.rs;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rt * kSgmvShrinkRows + w * 32 + mt * 16 + (lane >> 4) * 4 + i;
      if (r < len) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int j = nt * 16 + r_in;
          if (j < rank) out[(int64_t)r * d.rs + j] = acc[mt][nt][i];
        }
      }
    }
}

// ---------------------------------------------------------------- expand --

// KT = 16-wide steps over the rank (1, 2 or 4).  B rows are a multiple of 8
// elements apart, so a lane's 4 values of a B row are one 8-byte load.
template <int KT>
__device__ __forceinline__ void sgmv_expand_tile(const LayerDesc &d, const ModuleDesc &m, const uint16_t *B, int rank,
                                                 float scale, int seg0, int len, int rt, int tile, float *v_lds) {
  constexpr int DE = KT >= 4 ? 4 : 8;  // 16-column steps in flight
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const int r_in = lane & 15, kq = (lane >> 4) * 4;
  const int row0 = rt * kSgmvExpandRows;
  const int nrows = min(kSgmvExpandRows, len - row0);
  const int n_tile0 = tile * d.sg_nt;
  const int n_tile1 = min(n_tile0 + d.sg_nt, m.d_out);
  const int tile_len = n_tile1 - n_tile0;
  // This lane's output row and the B tile.
  const int r = row0 + w * 16 + r_in;
  const int b = r < len ? d.perm[seg0 + r] : -1;
  const bool yon = (unsigned)b < (unsigned)d.num_rows;
  const rsrc_t ry = make_rsrc(m.y, (uint32_t)((int64_t)d.num_rows * m.ldy * 2));
  const uint32_t yrow = yon ? (uint32_t)((int64_t)b * m.ldy * 2) : 0u;
  const int ldb = (rank + 7) & ~7;  // B row stride; columns past the rank meet zeros of V
  const rsrc_t rb = make_rsrc(B + (int64_t)n_tile0 * ldb, (uint32_t)tile_len * ldb * 2);
  auto y_off = [&](int n0) {  // this lane's 4 outputs of columns n0 + 4*(l/16) .. +4
    const int nc = n0 + kq;
    return yon && nc < tile_len ? yrow + (uint32_t)(n_tile0 + nc) * 2 : kOutOfRange;
  };
  auto load_b = [&](int n, int kt) -> s16x4_t {  // B[n][16kt + kq .. +4], zero past the rank / tile
    const int k = kt * 16 + kq;
    return __builtin_bit_cast(
        s16x4_t, buf_ld8<kNonTemporal>(rb, k < rank && n < tile_len ? ((uint32_t)n * ldb + k) * 2 : kOutOfRange));
  };
  // Requests for the first DE column steps go out before the V prologue.
  s16x4_t bop[DE][KT];
  u32x2 yv[DE];
#pragma unroll
  for (int u = 0; u < DE; ++u) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) bop[u][kt] = load_b(16 * u + r_in, kt);
    yv[u] = buf_ld8(ry, y_off(16 * u));
  }
  // V rows of the tile (times scale) into LDS: [64][64] fp32.
  for (int idx = t; idx < kSgmvExpandRows * 64; idx += 256) {
    const int i = idx >> 6, j = idx & 63;
    float sum = 0.f;
    if (i < nrows && j < rank) {
      const int p = seg0 + row0 + i;
      if (d.v != nullptr) {
        const int bb = d.perm[p];
        if ((unsigned)bb < (unsigned)d.num_rows) sum = d.v[(int64_t)bb * d.ldv + j];
      } else {
        for (int c = 0; c < m.n_chunks; ++c) sum += d.part[((int64_t)(m.part_base + c) * d.num_rows + p) * d.rs + j];
      }
    }
    v_lds[idx] = sum * scale;
  }
  __syncthreads();
  // This wave's 16 rows as hi/lo bf16 operands: row 16w + l%16, k = 16kt + 4*(l/16) .. +4.
  s16x4_t vhi[KT], vlo[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const float *src = v_lds + (w * 16 + r_in) * 64 + kt * 16 + kq;
    float hv[4], lv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      hv[c] = bf16_round(src[c]);
      lv[c] = src[c] - hv[c];
    }
    vhi[kt] = __builtin_bit_cast(s16x4_t, u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])});
    vlo[kt] = __builtin_bit_cast(s16x4_t, u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])});
  }
  // Columns in steps of 16: A-operand = B rows n0 + l%16; result lane (l, i)
  // = output column n0 + 4*(l/16) + i of row 16w + l%16.
  for (int n0 = 0; n0 < tile_len; n0 += 16 * DE) {
#pragma unroll
    for (int u = 0; u < DE; ++u) {
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bop[u][kt], vhi[kt], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bop[u][kt], vlo[kt], acc, 0, 0, 0);
      }
      const float o0 = bf16_to_f32(yv[u].x) + acc[0];
      const float o1 = bf16_to_f32(yv[u].x >> 16) + acc[1];
      const float o2 = bf16_to_f32(yv[u].y) + acc[2];
      const float o3 = bf16_to_f32(yv[u].y >> 16) + acc[3];
      buf_st8(ry, y_off(n0 + 16 * u), u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)});
      // refill this slot with the step DE ahead (past the tile: zero, no traffic)
      const int nn = n0 + 16 * (u + DE);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) bop[u][kt] = load_b(nn + r_in, kt);
      yv[u] = buf_ld8(ry, y_off(nn));
    }
  }
}

// Block `blk` of the SGMV expand numbering (row tiles x sg_items).
template <int KT>
__device__ __forceinline__ void sgmv_expand_block(const LayerDesc &d, int blk, float *v_lds) {
  const int tile_idx = blk / d.sg_items;
  const int it = blk - tile_idx * d.sg_items;
  int s, rt;
  if (!find_long_tile(d, tile_idx, kSgmvExpandRows, &s, &rt)) return;
  const ModuleDesc m = module_of_item<true>(d, it);
  const int tile = it - m.sg_item_base;
  int a, seg0, len;
  if (!load_segment(d, s, it == 0 && rt == 0, &a, &seg0, &len)) return;
  lora_adapter_entry_t e;
  if (!load_entry(d, a, m.col, tile == 0 && rt == 0, &e)) return;
  const uint16_t *B = static_cast<const uint16_t *>(e.B);
  sgmv_expand_tile<KT>(d, m, B, e.rank, e.scale, seg0, len, rt, tile, v_lds);
}

}  // namespace lora
