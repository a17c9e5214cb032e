// Base projection and adapter delta in one pass over the base weight:
//     y[b] = bf16( W . x[b] + scale_a * B_a . v[b] ),   a = the row's adapter.
//
// "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A": the forward is
// y = Wx + (B.A)x(alpha/r), the base term shared by the batch and the adapter
// term per row; "Fused mixed-precision base + delta" on the pages' list of
// next steps puts the delta into the base product's epilogue with a wide
// accumulator, so y is written once instead of written and then updated.
//
// A block takes kFusedRows rows (in their original order) and fused_cols
// (128) output columns of one projection, over the whole d_in:
//   * main loop: x and W stream through LDS in rounds of 64 k, x two rounds
//     and W four (4-bit W: two) rounds ahead in registers (x rows from L2,
//     W rows from HBM once, nontemporal, 128-byte line pieces); the waves
//     form a 2 x 2 grid over rows and columns, and each turns its 64 x 64
//     piece into 4 x 4 bf16 matrix-core tiles (16x16x32, fp32 accumulate).
//     The 128-column tile halves the x bytes read from L2 per byte of W; its
//     2 x 2 wave grid reads 8 operand fragments from LDS per step where 4
//     row bands of 32 read 10.  Loading
//     W straight into the matrix-core operand layout (16 rows x 64 bytes per
//     instruction) with each wave owning 16 or 32 columns measured slower,
//     and so did one register set for both B formats in the epilogue (a
//     branch per row around the loads makes the compiler wait for all of
//     them);
//   * epilogue: the base tile goes to LDS, then, for each 64-column half in
//     turn, each wave streams the B slice (the half's 64 rows of B_a, rank
//     values each) of one of its rows per round, one round ahead, with the
//     row's v (from the grouped shrink); 8 lanes share a B row (8 values
//     each), a reduce-scatter leaves one output column per lane, and y is
//     written once.
// The table entries of the block's rows are loaded with the first rounds of
// the main loop (one row per lane), so the epilogue starts without waiting.
#pragma once

#include "device_common.h"
#include "sgmv_items.h"

namespace lora {

// The descriptor of the fused kernel, read from its argument segment (see
// kernel_desc: indexing the by-value argument copies it to scratch memory).
__device__ __forceinline__ const FusedDesc &fused_desc() {
  return *(const FusedDesc *)(const void *)__builtin_amdgcn_kernarg_segment_ptr();
}

__device__ __forceinline__ FusedModule fused_module_of(const FusedDesc &f, int blk) {
  int mi = 0;
#pragma unroll
  for (int k = 1; k < kMaxModules; ++k)
    if (k < f.n_active && blk >= f.mod[k].block_base) mi = k;
  return fused_desc().mod[mi];
}

// LDS of a block: two round buffers of x [128 rows] and W [fused_cols rows]
// (64 k each), later the base tile [128 rows][fused_cols + 1 floats: odd, no
// bank clash].
constexpr int fused_buf_bytes(bool q4) { return kShrinkXBytes + fused_cols(q4) * kShrinkRound * 2; }
constexpr int fused_base_stride(bool q4) { return fused_cols(q4) + 1; }
constexpr int fused_lds_bytes(bool q4) {
  return 2 * fused_buf_bytes(q4) > kFusedRows * fused_base_stride(q4) * 4 ? 2 * fused_buf_bytes(q4)
                                                                          : kFusedRows * fused_base_stride(q4) * 4;
}

// One epilogue row: per lane 8 pieces of the B slice (q = 0..7: B row
// n0 + 8q + lane/8, values 8*(lane%8) .. +8; bf16 16 bytes, or int8 8 bytes
// in .x/.y) and the 8 values of v they meet.
struct FusedRowLoads {
  u32x4 b16[8];
  u32x2 b8[8];
  f32x4_t v[2];
};

// Q4: the base weight is 4-bit with group scales (lora_linear_layer_q4).
template <bool Q4>
__device__ __forceinline__ void fused_block(const FusedDesc &f, int blk, uint8_t *lds) {
  constexpr int NC = fused_cols(Q4);          // output columns of the block
  // waves: WR along the rows x 4 / WR along the columns; each takes MT x 4
  // matrix-core tiles of 16 x 16
  constexpr int WR = NC == 128 ? 2 : 4;
  constexpr int MT = kFusedRows / WR / 16;
  constexpr int NTL = 4;
  constexpr int BS = fused_base_stride(Q4);
  constexpr int XL = kFusedRows * 8 / 256;    // x pieces per thread per round (4)
  constexpr int WL = NC * 8 / 256;            // bf16 W pieces per thread per round
  constexpr int RPW = kFusedRows / 4;         // epilogue rows per wave (32)
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const int w_row = (w % WR) * (kFusedRows / WR), w_col = (w / WR) * (NC * WR / 4);
  const FusedModule m = fused_module_of(f, blk);
  const int local = blk - m.block_base;
  const int rt = local / m.n_tiles, tile = local - rt * m.n_tiles;
  const int row0 = rt * kFusedRows, n0 = tile * NC;

  // Segments come in ascending slot order, so the slots with a segment in
  // this build are the valid ones up to the last segment's.
  const int nseg = min(uniform(*f.num_segments), f.max_seg);
  const int last_slot = nseg > 0 ? uniform(f.seg_adapter[nseg - 1]) : -1;
  // Table entries of this wave's epilogue rows w + 4i, one per lane (i < 32).
  // (what the epilogue needs of it: B, rank, scale, format; rank 0 when the
  // row gets no delta: base only, a slot past the build, a malformed entry)
  const void *my_B = nullptr;
  int my_rank = 0, my_fmt = 0;
  float my_scale = 0.f;
  if (lane < RPW) {
    const int b = row0 + w + 4 * lane;
    const int a = b < f.num_rows ? f.ids[b] : -1;
    if ((unsigned)a < (unsigned)f.num_slots && a <= last_slot) {
      const lora_adapter_entry_t e = f.table[(int64_t)a * f.table_cols + m.col];
      const bool ok = entry_ok(e, f.max_rank);  // a malformed entry: counted by the shrink
      my_B = e.B;
      my_rank = ok ? e.rank : 0;
      my_fmt = e.format;
      my_scale = e.scale;
    }
  }

  const int piece = t & 7;
  const rsrc_t rx = make_rsrc(m.x, (uint32_t)((int64_t)f.num_rows * m.ldx * 2));
  uint32_t xoff[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int r = row0 + i * 32 + (t >> 3);
    xoff[i] = r < f.num_rows ? (uint32_t)((int64_t)r * m.ldx * 2) : kOutOfRange;
  }
  // W of a round: bf16, WL pieces of 8 values per thread (rows 32i + t/8);
  // 4-bit, one 16-byte piece of 32 values per thread (row t/2, values
  // 32 (t%2) .. +32 of the round), widened to bf16 on the way into LDS
  const int64_t w_row_bytes = Q4 ? m.ldw : m.ldw * 2;
  const rsrc_t rw = make_rsrc(m.W, (uint32_t)((int64_t)m.d_out * w_row_bytes));
  constexpr int WP = Q4 ? 1 : WL;
  uint32_t woff[WP];
#pragma unroll
  for (int i = 0; i < WP; ++i) {
    const int n = n0 + (Q4 ? (t >> 1) : i * 32 + (t >> 3));
    woff[i] = n < m.d_out ? (uint32_t)((int64_t)n * w_row_bytes) : kOutOfRange;
  }
  using WRaw = u32x4;
  struct XStage {
    u32x4 x[XL];
  };
  struct WStage {
    WRaw wv[WP];
  };
  auto load_x = [&](XStage &st, int k0) {  // one round; past d_in: zero, no traffic
    const int k = k0 + piece * 8;
    const bool kon = k < m.d_in;
    const uint32_t kb = (uint32_t)k * 2;
#pragma unroll
    for (int i = 0; i < XL; ++i) st.x[i] = buf_ld16(rx, kon && xoff[i] != kOutOfRange ? xoff[i] + kb : kOutOfRange, 0);
  };
  auto load_w = [&](WStage &st, int k0) {
    const int k = k0 + piece * 8;
    const bool kon = k < m.d_in;
    const uint32_t kb = (uint32_t)k * 2;
    if constexpr (Q4) {
      const int kq = k0 + 32 * (t & 1);
      st.wv[0] = __builtin_amdgcn_raw_buffer_load_b128(
          rw, kq < m.d_in && woff[0] != kOutOfRange ? woff[0] + (uint32_t)kq / 2 : kOutOfRange, 0, kNonTemporal);
    } else {
#pragma unroll
      for (int i = 0; i < WL; ++i)
        st.wv[i] = buf_ld16_stream(rw, kon && woff[i] != kOutOfRange ? woff[i] + kb : kOutOfRange, 0);
    }
  };
  auto store = [&](const XStage &xs, const WStage &ws, uint8_t *buf) {
#pragma unroll
    for (int i = 0; i < XL; ++i) *(u32x4 *)(buf + shrink_lds_off(i * 32 + (t >> 3), piece)) = xs.x[i];
    if constexpr (Q4) {
      const int row = t >> 1, p0 = 4 * (t & 1);
      *(u32x4 *)(buf + kShrinkXBytes + shrink_lds_off(row, p0)) = q4x8_to_bf16x8(ws.wv[0].x);
      *(u32x4 *)(buf + kShrinkXBytes + shrink_lds_off(row, p0 + 1)) = q4x8_to_bf16x8(ws.wv[0].y);
      *(u32x4 *)(buf + kShrinkXBytes + shrink_lds_off(row, p0 + 2)) = q4x8_to_bf16x8(ws.wv[0].z);
      *(u32x4 *)(buf + kShrinkXBytes + shrink_lds_off(row, p0 + 3)) = q4x8_to_bf16x8(ws.wv[0].w);
    } else {
#pragma unroll
      for (int i = 0; i < WL; ++i)
        *(u32x4 *)(buf + kShrinkXBytes + shrink_lds_off(i * 32 + (t >> 3), piece)) = ws.wv[i];
    }
  };
  f32x4_t acc[MT][NTL];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int r_in = lane & 15, g = lane >> 4;
  auto compute = [&](const uint8_t *buf, f32x4_t (&acc)[MT][NTL]) {
#pragma unroll
    for (int ks = 0; ks < kShrinkRound / 32; ++ks) {
      u32x4 xo[MT], wo[NTL];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xo[mt] = *(const u32x4 *)(buf + shrink_lds_off(w_row + mt * 16 + r_in, ks * 4 + g));
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt)
        wo[nt] = *(const u32x4 *)(buf + kShrinkXBytes + shrink_lds_off(w_col + nt * 16 + r_in, ks * 4 + g));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xo[mt]),
                                                                __builtin_bit_cast(bf16x8_t, wo[nt]), acc[mt][nt], 0,
                                                                0, 0);
      if constexpr (Q4) __builtin_amdgcn_sched_barrier(0);  // one k-step's operands live at a time
    }
  };
  // 4-bit: the two rounds of a main-loop step are one group of kQ4Group
  // inputs; its sums collect apart and meet the group's scale of each
  // output column (this lane's columns n0 + 16 nt + r_in), requested one
  // step ahead
  static_assert(2 * kShrinkRound == kQ4Group, "one group per main-loop step");

  f32x4_t gacc[Q4 ? MT : 1][Q4 ? 4 : 1];
  float sc_cur[4] = {0.f, 0.f, 0.f, 0.f}, sc_nxt[4] = {0.f, 0.f, 0.f, 0.f};
  const rsrc_t rs_w = make_rsrc(Q4 ? m.Ws : nullptr, Q4 ? (uint32_t)((int64_t)m.d_out * m.ldws * 4) : 0u);
  const int n_groups = Q4 ? m.d_in / kQ4Group : 0;
  auto load_scales = [&](float (&sc)[4], int grp) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = n0 + w_col + nt * 16 + r_in;
      sc[nt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rs_w, n < m.d_out && grp < n_groups ?
                                                       (uint32_t)(((int64_t)n * m.ldws + grp) * 4) : kOutOfRange,
                                             0, 0));
    }
  };
  if constexpr (Q4) load_scales(sc_cur, 0);
  // x (mostly from L2) two rounds ahead, W (from HBM) four: round r goes
  // to LDS buffer r & 1 once its loads are in, and then x of round r + 2 and
  // W of round r + 4 are requested into the registers it leaves.
  XStage x0, x1;
  WStage w0, w1, w2, w3;
  load_x(x0, 0);
  load_w(w0, 0);
  load_w(w1, kShrinkRound);
  load_x(x1, kShrinkRound);
  if constexpr (!Q4) {  // 4-bit W: two rounds ahead (its registers are few, its rounds short)
    load_w(w2, 2 * kShrinkRound);
    load_w(w3, 3 * kShrinkRound);
  }
  const int rounds = (m.d_in + kShrinkRound - 1) / kShrinkRound;
  uint8_t *b0 = lds, *b1 = lds + fused_buf_bytes(Q4);
  auto step = [&](int r, auto odd, XStage &xs, WStage &ws, uint8_t *buf) {
    constexpr bool kOdd = decltype(odd)::value;
    if constexpr (Q4 && !kOdd) {
      load_scales(sc_nxt, r / 2 + 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) gacc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    store(xs, ws, buf);
    load_x(xs, (r + 2) * kShrinkRound);
    load_w(ws, (r + (Q4 ? 2 : 4)) * kShrinkRound);
    __syncthreads();
    if constexpr (Q4) {
      compute(buf, gacc);
      if constexpr (kOdd) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][nt][i] = fmaf(sc_cur[nt], gacc[mt][nt][i], acc[mt][nt][i]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) sc_cur[nt] = sc_nxt[nt];
      }
    } else {
      compute(buf, acc);
    }
  };
  using Even = std::false_type;
  using Odd = std::true_type;
  // Four rounds per pass (one per pairing of the x and W registers); rounds
  // past d_in read zeros and add nothing.  (An exit between the rounds of a
  // pass makes the compiler spill.  The 4-bit kernel, whose W registers
  // alternate, runs the same four-round pass: in the six-round pass that W
  // three rounds ahead needed, it spilled 17 registers.)
  for (int r = 0; r < rounds; r += 4) {
    step(r, Even{}, x0, w0, b0);
    step(r + 1, Odd{}, x1, w1, b1);
    step(r + 2, Even{}, x0, Q4 ? w0 : w2, b0);
    step(r + 3, Odd{}, x1, Q4 ? w1 : w3, b1);
  }
  __syncthreads();  // every wave is done with the round buffers

  // Base tile to LDS: C[4*(l/16) + i][l%16] of tile (mt, nt) is row
  // 32w + 16mt + 4*(l/16) + i, column 16nt + l%16.
  float *base = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        base[(w_row + mt * 16 + g * 4 + i) * BS + w_col + nt * 16 + r_in] = acc[mt][nt][i];
  __syncthreads();

  // Epilogue: row rr = w + 4i of the tile in round i, over each 64-column
  // half of the block's columns in turn.
  int nh = n0, ch = 0;  // the half's first output column, and its column in the base tile
  const int bl = lane >> 3, pc = lane & 7, j0 = pc * 8;
  const int c = 8 * pc + bl;  // this lane's output column after the reduce-scatter
  const rsrc_t ry = make_rsrc(m.y, (uint32_t)((int64_t)f.num_rows * m.ldy * 2));
  const rsrc_t rv = make_rsrc(m.v, (uint32_t)((int64_t)f.num_rows * f.rs * 4));
  struct RowInfo {
    int b, rank, fmt;
    bool ok;
    float scale;
    const uint8_t *B;
  };
  auto row_info = [&](int i) {  // uniform: the entry held by lane i
    RowInfo ri;
    ri.b = row0 + w + 4 * i;
    const int rank = __builtin_amdgcn_readlane(my_rank, i);
    const void *B = (const void *)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                                                   (int)(uint32_t)(uintptr_t)my_B, i)) |
                                              ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                                                   (int)(uint32_t)((uintptr_t)my_B >> 32), i)
                                               << 32));
    ri.ok = rank > 0 && ri.b < f.num_rows;
    ri.rank = rank;
    ri.fmt = __builtin_amdgcn_readlane(my_fmt, i);
    ri.scale = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_scale), i));
    ri.B = static_cast<const uint8_t *>(B);
    return ri;
  };
  auto issue = [&](const RowInfo &ri, FusedRowLoads &L) {
    const bool on = ri.ok && j0 < ri.rank;
    const bool q8 = ri.fmt == LORA_FORMAT_INT8_ROWS;
    const uint32_t row_bytes = q8 ? (uint32_t)ldb8_of(ri.rank) : (uint32_t)((ri.rank + 7) & ~7) * 2;
    const uint8_t *vals = ri.B + (q8 ? q8_values_offset(m.d_out) : 0);
    const rsrc_t rb = make_rsrc(ri.ok ? vals : nullptr, ri.ok ? (uint32_t)m.d_out * row_bytes : 0u);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int n = nh + 8 * q + bl;
      const bool lon = on && n < m.d_out;
      const uint32_t off = (uint32_t)n * row_bytes + (uint32_t)j0 * (q8 ? 1 : 2);
      L.b16[q] = buf_ld16_stream(rb, lon && !q8 ? off : kOutOfRange, 0);
      L.b8[q] = __builtin_amdgcn_raw_buffer_load_b64(rb, lon && q8 ? off : kOutOfRange, 0, kNonTemporal);
    }
    const uint32_t voff = on ? (uint32_t)(((int64_t)ri.b * f.rs + j0) * 4) : kOutOfRange;
    L.v[0] = __builtin_bit_cast(f32x4_t, buf_ld16(rv, voff, 0));
    L.v[1] = __builtin_bit_cast(f32x4_t, buf_ld16(rv, voff == kOutOfRange ? kOutOfRange : voff + 16, 0));
  };
  auto finish = [&](const RowInfo &ri, const FusedRowLoads &L, int rr) {
    if (ri.b >= f.num_rows) return;
    float dl = 0.f;
    if (ri.ok) {
      float vv[8];  // v past the rank is not part of the row's vector: zero
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        vv[k] = j0 + k < ri.rank ? L.v[0][k] : 0.f;
        vv[4 + k] = j0 + 4 + k < ri.rank ? L.v[1][k] : 0.f;
      }
      float acc8[8];
      if (ri.fmt == LORA_FORMAT_INT8_ROWS) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc8[q] = dot8_i8_f32(L.b8[q], vv, 0.f);
      } else {
        const V8Split vs = split_v8(vv);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc8[q] = dot8_bf16_split(L.b16[q], vs, 0.f);
      }
      reduce_scatter<8, 8>(acc8);
      dl = acc8[0] * ri.scale;
      if (ri.fmt == LORA_FORMAT_INT8_ROWS && nh + c < m.d_out)
        dl *= reinterpret_cast<const float *>(ri.B)[nh + c];  // the B row's scale
    }
    const float yv = base[rr * BS + ch + c] + dl;
    buf_st_u16(ry, nh + c < m.d_out ? (uint32_t)(((int64_t)ri.b * m.ldy + nh + c) * 2) : kOutOfRange,
               f32_to_bf16(yv));
  };
  for (int h = 0; h < NC / 64; ++h) {
    nh = n0 + 64 * h;
    ch = 64 * h;
    FusedRowLoads cur, nxt;
    RowInfo ci = row_info(0);
    issue(ci, cur);
    for (int i = 0; i + 1 < RPW; ++i) {  // row i+1 is requested before row i is finished
      const RowInfo ni = row_info(i + 1);
      issue(ni, nxt);
      finish(ci, cur, w + 4 * i);
      cur = nxt;
      ci = ni;
    }
    finish(ci, cur, w + 4 * (RPW - 1));
  }
}

}  // namespace lora
