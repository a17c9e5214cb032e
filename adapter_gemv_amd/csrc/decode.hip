// Decode (BGMV-style) gather kernels for gfx950.
//
// "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A": one batched kernel
// gathers each sequence's adapter through the index vector and applies it
// without materialising per-sequence weights; the cost is bandwidth, since
// each distinct adapter in the batch is read once per step.
// "LoRA, quotas and noisy neighbours", "One weight read, many adapters": the
// update is applied in registers.
//
// Work is cut into items over (segment, projection, k-chunk) for the shrink
// and (segment, projection, n-tile) for the expand; one 256-thread block takes
// one item.  A segment's rows share every load of its adapter's factors.
//
// Shrink  v = A.x: wave w owns rows [w*JW, (w+1)*JW) of A; each lane streams
//   8 consecutive k (16 bytes) of every A row and of each x row, so one wave
//   load covers 1 KiB of contiguous memory.  bf16 pairs meet in v_dot2_f32_bf16
//   (exact products, fp32 sums).  The JW*RG per-lane sums are reduced across
//   the wave by a reduce-scatter butterfly, which leaves every sum on one
//   lane; the block writes its k-chunk's partial v to the workspace (fixed
//   order, no atomics, so results are bit-reproducible).
// Expand  y += scale * B.v: the item first sums the k-chunk partials of its
//   segment's rows into LDS (times scale), then streams its tile of B, which
//   is contiguous because B is [d_out][rank] row-major: LPR = rank/8 lanes
//   share one output row, each lane loads 16 bytes, a reduce-scatter over the
//   LPR lanes finishes the dot products, and the owning lane reads y, adds,
//   rounds to bf16 (RNE) and writes it back.  Each (row, output) is written by
//   exactly one lane.
#include "lora_internal.h"

namespace lora {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Memory access goes through raw buffer instructions: a scalar resource
// (base address and byte size) plus one 32-bit per-lane offset and an
// optional scalar offset.  The hardware returns zero for lane offsets at or
// beyond the size and drops such stores; rows are masked explicitly.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferWord3 = 0x00020000;  // 32-bit data format, no swizzle

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferWord3);
}
__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint16_t buf_ld_u16(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
}
__device__ __forceinline__ void buf_st_u16(rsrc_t r, uint32_t voff, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, 0, 0);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

__device__ __forceinline__ float dot8_bf16(const u32x4 &a, const u32x4 &b, float c) {
  c = dot2(a.x, b.x, c);
  c = dot2(a.y, b.y, c);
  c = dot2(a.z, b.z, c);
  c = dot2(a.w, b.w, c);
  return c;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Eight bf16 values (one 16-byte load) times eight floats.
__device__ __forceinline__ float dot8_bf16_f32(const u32x4 &b, const float *v, float c) {
  c = fmaf(bf16_lo(b.x), v[0], c);
  c = fmaf(bf16_hi(b.x), v[1], c);
  c = fmaf(bf16_lo(b.y), v[2], c);
  c = fmaf(bf16_hi(b.y), v[3], c);
  c = fmaf(bf16_lo(b.z), v[4], c);
  c = fmaf(bf16_hi(b.z), v[5], c);
  c = fmaf(bf16_lo(b.w), v[6], c);
  c = fmaf(bf16_hi(b.w), v[7], c);
  return c;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Reduce-scatter of NV per-lane values over aligned groups of NL lanes.
// Afterwards, if NV >= NL, lane q = lane % NL holds in v[i] (i < NV/NL) the
// group sum of value index i + (NV/NL)*q; if NV < NL, v[0] holds the sum of
// value index q / (NL/NV).  Stage MASK pairs lanes that differ in bit MASK;
// the lane with that bit set keeps the upper half of its N live values.
// Every array index is a compile-time constant.
template <int N, int MASK, int NV>
__device__ __forceinline__ void rs_stage(float (&v)[NV], int lane) {
  if constexpr (MASK >= 1) {
    if constexpr (N > 1) {
      const bool hi = (lane & MASK) != 0;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const float send = hi ? v[i] : v[i + N / 2];
        const float keep = hi ? v[i + N / 2] : v[i];
        v[i] = keep + __shfl_xor(send, MASK, 64);
      }
      rs_stage<N / 2, MASK / 2, NV>(v, lane);
    } else {
      v[0] += __shfl_xor(v[0], MASK, 64);
      rs_stage<1, MASK / 2, NV>(v, lane);
    }
  }
}

template <int NV, int NL>
__device__ __forceinline__ void reduce_scatter(float (&v)[NV]) {
  rs_stage<NV, NL / 2, NV>(v, threadIdx.x & 63);
}

// The module an item of a segment belongs to, copied out of the kernel
// argument with compile-time indices only (a runtime index into the by-value
// descriptor would copy it to scratch memory).
__device__ __forceinline__ ModuleDesc module_of_item(const LayerDesc &d, int it) {
  ModuleDesc m = d.mod[0];
#pragma unroll
  for (int k = 1; k < kMaxModules; ++k)
    if (k < d.n_active && it >= d.mod[k].item_base) m = d.mod[k];
  return m;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------- shrink --

// Rows of A are spread over the 4 waves: wave w owns rows
// [w*jw, w*jw + jw) with jw = ceil(rank / 4) <= JW, so all waves share the
// stream whatever the entry's rank.  RG rows of x are processed together.
template <int JW, int RG>
__device__ __forceinline__ void shrink_rows(const LayerDesc &d, const ModuleDesc &m, const uint16_t *__restrict__ A,
                                            int rank, int jw, int pos0, int nrows, int chunk) {
  const int lane = threadIdx.x & 63;
  const int j0 = wave_id() * jw;
  const int k_begin = chunk * d.kc;
  const int k_end = min(k_begin + d.kc, m.d_in);
  const uint32_t row_bytes = (uint32_t)m.d_in * 2;
  rsrc_t rx[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int b = r < nrows ? d.perm[pos0 + r] : 0;
    const bool ok = (unsigned)b < (unsigned)d.num_rows;  // a stray index reads zeros
    rx[r] = make_rsrc(m.x + (int64_t)(ok ? b : 0) * m.ldx, ok ? row_bytes : 0u);
  }
  const rsrc_t ra = make_rsrc(A, (uint32_t)rank * row_bytes);
  float acc[JW * RG];
#pragma unroll
  for (int i = 0; i < JW * RG; ++i) acc[i] = 0.f;
  for (int k = k_begin + lane * 8; k < k_end; k += 512) {
    const uint32_t voff = (uint32_t)k * 2;
    u32x4 xv[RG], av[JW];
#pragma unroll
    for (int r = 0; r < RG; ++r) xv[r] = r < nrows ? buf_ld16(rx[r], voff, 0) : zero4();
#pragma unroll
    for (int jj = 0; jj < JW; ++jj)
      av[jj] = (jj < jw && j0 + jj < rank) ? buf_ld16(ra, voff, (uint32_t)(j0 + jj) * row_bytes) : zero4();
#pragma unroll
    for (int jj = 0; jj < JW; ++jj)
#pragma unroll
      for (int r = 0; r < RG; ++r) acc[jj * RG + r] = dot8_bf16(av[jj], xv[r], acc[jj * RG + r]);
  }
  reduce_scatter<JW * RG, 64>(acc);
  float *out = d.part + ((int64_t)(m.part_base + chunk) * d.num_rows + pos0) * d.rs;
  constexpr int NV = JW * RG;
  if constexpr (NV >= 64) {
#pragma unroll
    for (int i = 0; i < NV / 64; ++i) {
      const int idx = i + (NV / 64) * lane;
      const int jj = idx / RG, r = idx % RG;
      if (r < nrows && jj < jw && j0 + jj < rank) out[(int64_t)r * d.rs + j0 + jj] = acc[i];
    }
  } else {
    constexpr int GS = 64 / NV;
    if (lane % GS == 0) {
      const int idx = lane / GS;
      const int jj = idx / RG, r = idx % RG;
      if (r < nrows && jj < jw && j0 + jj < rank) out[(int64_t)r * d.rs + j0 + jj] = acc[0];
    }
  }
}

// JW = rows of A per wave at the largest rank the launch allows (4*JW).
template <int JW>
__global__ __launch_bounds__(kDecodeThreads) void decode_shrink_kernel(LayerDesc d) {
  constexpr int RGM = JW >= 16 ? 2 : 4;  // rows of x per pass for multi-row segments
  const int nseg = *d.num_segments;
  const int s = blockIdx.x / d.items_per_seg;
  if (s >= nseg) return;
  const int it = blockIdx.x - s * d.items_per_seg;
  const ModuleDesc m = module_of_item(d, it);
  const int chunk = it - m.item_base;
  const int a = d.seg_adapter[s];
  const int pos0 = d.seg_offsets[s];
  const int len = d.seg_offsets[s + 1] - pos0;
  if ((unsigned)a >= (unsigned)d.num_slots || pos0 < 0 || len <= 0 || pos0 + len > d.num_rows) {
    if (threadIdx.x == 0 && it == 0) atomicAdd(d.status, 1);  // segments not built for this batch
    return;
  }
  const lora_adapter_entry_t e = d.table[(int64_t)a * d.table_cols + m.col];
  const int rank = e.rank;
  if (rank == 0) return;
  const uint16_t *A = static_cast<const uint16_t *>(e.A);
  if (rank < 0 || rank > d.max_rank || A == nullptr || ((uintptr_t)A & 15) != 0) {
    if (chunk == 0 && threadIdx.x == 0) atomicAdd(d.status, 1);
    return;
  }
  const int jw = (rank + 3) >> 2;
  if (len == 1) {
    shrink_rows<JW, 1>(d, m, A, rank, jw, pos0, 1, chunk);
  } else {
    for (int r0 = 0; r0 < len; r0 += RGM)
      shrink_rows<JW, RGM>(d, m, A, rank, jw, pos0 + r0, min(RGM, len - r0), chunk);
  }
}

// lora_shrink: sum the k-chunk partials of each valid row into v[b][0..max_rank).
__global__ __launch_bounds__(256) void shrink_reduce_kernel(LayerDesc d) {
  const int nseg = min(*d.num_segments, min(d.num_rows, d.num_slots));
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
  const ModuleDesc &m = d.mod[0];
  const int a = d.seg_adapter[lo];
  if ((unsigned)a >= (unsigned)d.num_slots) return;
  const lora_adapter_entry_t e = d.table[(int64_t)a * d.table_cols + m.col];
  const int rank = e.rank;
  const bool ok = rank > 0 && rank <= d.max_rank && e.A != nullptr && ((uintptr_t)e.A & 15) == 0;
  float sum = 0.f;
  if (ok && j < rank)
    for (int c = 0; c < m.n_chunks; ++c) sum += d.part[((int64_t)(m.part_base + c) * d.num_rows + p) * d.rs + j];
  const int b = d.perm[p];
  if ((unsigned)b < (unsigned)d.num_rows) d.v_out[(int64_t)b * d.ldv + j] = sum;
}

// ---------------------------------------------------------------- expand --

// Eight elements of row n of a B tile starting at element column jq, zero
// beyond the rank and beyond the tile.  Rows are 16-byte aligned when the
// rank is a multiple of 8; other ranks load element by element.
__device__ __forceinline__ u32x4 load_b(rsrc_t rb, int n, int rank, int jq, bool aligned) {
  const uint32_t off = ((uint32_t)n * rank + jq) * 2;
  if (aligned) return buf_ld16(rb, off, 0);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (jq + 2 * i < rank) ? buf_ld_u16(rb, off + 4 * i) : 0u;
    const uint32_t hi = (jq + 2 * i + 1 < rank) ? buf_ld_u16(rb, off + 4 * i + 2) : 0u;
    w[i] = lo | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// One n-tile of one projection for every row of a segment.
template <int LPR>
__device__ __forceinline__ void expand_item(const LayerDesc &d, const ModuleDesc &m, const uint16_t *__restrict__ B,
                                            int rank, float scale, int pos0, int len, int tile, float *v_lds) {
  constexpr int G = kDecodeThreads / LPR;  // output rows per load pass of the block
  constexpr int P = 16;                    // load passes per sub-tile
  constexpr int SUB = P * G;               // outputs per sub-tile
  constexpr int PL = P / LPR;              // outputs per lane per row after the reduce-scatter
  const int t = threadIdx.x, g = t / LPR, q = t % LPR, jq = q * 8;
  const bool aligned = (rank & 7) == 0;
  const int n_tile0 = tile * d.nt;
  const int n_tile1 = min(n_tile0 + d.nt, m.d_out);
  // B rows [n_tile0, n_tile1): loads past the tile read zero.
  const rsrc_t rb = make_rsrc(B + (int64_t)n_tile0 * rank, (uint32_t)(n_tile1 - n_tile0) * rank * 2);
  const bool lane_on = jq < rank;
  for (int r0 = 0; r0 < len; r0 += kExpandRowGroup) {
    const int nr = min(kExpandRowGroup, len - r0);
    __syncthreads();
    for (int idx = t; idx < nr * 64; idx += kDecodeThreads) {
      const int i = idx >> 6, j = idx & 63;
      float sum = 0.f;
      if (j < rank) {
        const int p = pos0 + r0 + i;
        if (d.v != nullptr) {
          const int b = d.perm[p];
          if ((unsigned)b < (unsigned)d.num_rows) sum = d.v[(int64_t)b * d.ldv + j];
        } else {
          for (int c = 0; c < m.n_chunks; ++c)
            sum += d.part[((int64_t)(m.part_base + c) * d.num_rows + p) * d.rs + j];
        }
      }
      v_lds[idx] = sum * scale;
    }
    __syncthreads();
    for (int n0 = 0; n0 < n_tile1 - n_tile0; n0 += SUB) {
      u32x4 bv[P];
#pragma unroll
      for (int p = 0; p < P; ++p) bv[p] = lane_on ? load_b(rb, n0 + p * G + g, rank, jq, aligned) : zero4();
      for (int i = 0; i < nr; ++i) {
        // Keep the bf16 tile packed across rows: without this the compiler
        // hoists its conversion to fp32 out of the row loop (2x registers).
#pragma unroll
        for (int p = 0; p < P; ++p) asm volatile("" : "+v"(bv[p]));
        float vv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) vv[k] = v_lds[i * 64 + jq + k];
        float acc[P];
#pragma unroll
        for (int p = 0; p < P; ++p) acc[p] = dot8_bf16_f32(bv[p], vv, 0.f);
        reduce_scatter<P, LPR>(acc);
        const int b = d.perm[pos0 + r0 + i];
        const bool ok = (unsigned)b < (unsigned)d.num_rows;  // a stray index writes nothing
        const rsrc_t ry =
            make_rsrc(m.y + (int64_t)(ok ? b : 0) * m.ldy + n_tile0, ok ? (uint32_t)(n_tile1 - n_tile0) * 2 : 0u);
#pragma unroll
        for (int ii = 0; ii < PL; ++ii) {
          const uint32_t off = (uint32_t)(n0 + (ii + PL * q) * G + g) * 2;
          const uint16_t y0 = buf_ld_u16(ry, off);
          buf_st_u16(ry, off, f32_to_bf16(bf16_to_f32(y0) + acc[ii]));
        }
      }
    }
  }
}

// LPR = lanes per output row at the largest rank the launch allows (8*LPR).
template <int LPR>
__global__ __launch_bounds__(kDecodeThreads) void decode_expand_kernel(LayerDesc d) {
  __shared__ float v_lds[kExpandRowGroup * 64];
  const int nseg = *d.num_segments;
  const int s = blockIdx.x / d.items_per_seg;
  if (s >= nseg) return;
  const int it = blockIdx.x - s * d.items_per_seg;
  const ModuleDesc m = module_of_item(d, it);
  const int tile = it - m.item_base;
  const int a = d.seg_adapter[s];
  const int pos0 = d.seg_offsets[s];
  const int len = d.seg_offsets[s + 1] - pos0;
  if ((unsigned)a >= (unsigned)d.num_slots || pos0 < 0 || len <= 0 || pos0 + len > d.num_rows) {
    if (threadIdx.x == 0 && it == 0) atomicAdd(d.status, 1);  // segments not built for this batch
    return;
  }
  const lora_adapter_entry_t e = d.table[(int64_t)a * d.table_cols + m.col];
  const int rank = e.rank;
  if (rank == 0) return;
  const uint16_t *B = static_cast<const uint16_t *>(e.B);
  if (rank < 0 || rank > d.max_rank || B == nullptr || ((uintptr_t)B & 15) != 0 || e.A == nullptr ||
      ((uintptr_t)e.A & 15) != 0) {
    if (tile == 0 && threadIdx.x == 0) atomicAdd(d.status, 1);
    return;
  }
  expand_item<LPR>(d, m, B, rank, e.scale, pos0, len, tile, v_lds);
}

}  // namespace

size_t partials_ws_bytes(int num_rows, int max_rank, int64_t sum_d_in) {
  const int64_t chunks = sum_d_in / kKChunkMin + kMaxModules;
  return (size_t)((int64_t)num_rows * partial_row_stride(max_rank) * 4 * chunks);
}

// Rank class of a launch: the smallest of 8, 16, 32, 64 that holds max_rank.
static int rank_class_of(int max_rank) { return max_rank <= 8 ? 0 : max_rank <= 16 ? 1 : max_rank <= 32 ? 2 : 3; }

hipError_t launch_decode_shrink(const LayerDesc &d, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (rank_class_of(d.max_rank)) {
    case 0: decode_shrink_kernel<2><<<grid, kDecodeThreads, 0, stream>>>(d); break;
    case 1: decode_shrink_kernel<4><<<grid, kDecodeThreads, 0, stream>>>(d); break;
    case 2: decode_shrink_kernel<8><<<grid, kDecodeThreads, 0, stream>>>(d); break;
    default: decode_shrink_kernel<16><<<grid, kDecodeThreads, 0, stream>>>(d); break;
  }
  return hipGetLastError();
}

hipError_t launch_shrink_reduce(const LayerDesc &d, hipStream_t stream) {
  const int64_t total = (int64_t)d.num_rows * d.max_rank;
  if (total <= 0) return hipSuccess;
  shrink_reduce_kernel<<<(int)((total + 255) / 256), 256, 0, stream>>>(d);
  return hipGetLastError();
}

hipError_t launch_decode_expand(const LayerDesc &d, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (rank_class_of(d.max_rank)) {
    case 0: decode_expand_kernel<1><<<grid, kDecodeThreads, 0, stream>>>(d); break;
    case 1: decode_expand_kernel<2><<<grid, kDecodeThreads, 0, stream>>>(d); break;
    case 2: decode_expand_kernel<4><<<grid, kDecodeThreads, 0, stream>>>(d); break;
    default: decode_expand_kernel<8><<<grid, kDecodeThreads, 0, stream>>>(d); break;
  }
  return hipGetLastError();
}

}  // namespace lora
