// Device helpers shared by the gfx950 delta kernels.
#pragma once

#include "lora_internal.h"

namespace lora {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Memory access goes through raw buffer instructions: a scalar resource
// (base address and byte size) plus one 32-bit per-lane offset and an
// optional scalar offset.  The hardware returns zero for lane offsets at or
// beyond the size and drops such stores.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferWord3 = 0x00020000;  // 32-bit data format, no swizzle
// Streaming access (nt): data read once per step should not displace reused
// lines from the caches.
constexpr int kNonTemporal = 2;
// A lane offset past every buffer this library builds (all are below 4 GiB):
// loads there return zero and stores are dropped, which masks lanes without
// a branch (a branch around each load would make the compiler wait for all
// outstanding loads where the paths join).
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferWord3);
}
__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ u32x4 buf_ld16_stream(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNonTemporal);
}
template <int AUX = 0>
__device__ __forceinline__ u32x2 buf_ld8(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void buf_st16(rsrc_t r, uint32_t voff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, AUX);
}
// Device-scope store (sc1): measured slightly faster for the y update that
// follows a long read stream.
constexpr int kScopeDevice = 16;
__device__ __forceinline__ void buf_st8(rsrc_t r, uint32_t voff, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, 0, 0);
}
__device__ __forceinline__ uint16_t buf_ld_u16(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
}
__device__ __forceinline__ void buf_st_u16(rsrc_t r, uint32_t voff, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, 0, 0);
}

// ---- bf16 arithmetic: products of bf16 values are exact in fp32.
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

// Eight fp32 values v as two bf16 vectors, v = hi + lo to about 2^-16
// relative: hi = bf16(v), lo = bf16(v - hi).  A dot product with bf16 data
// then runs on v_dot2_f32_bf16 (exact products, fp32 sums) with no
// conversion of the data to fp32.
struct V8Split {
  u32x4 hi, lo;
};
__device__ __forceinline__ V8Split split_v8(const float *v) {
  V8Split r;
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float h0 = (float)(__bf16)v[2 * i], h1 = (float)(__bf16)v[2 * i + 1];
    h[i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)h0) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)h1) << 16);
    l[i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(v[2 * i] - h0)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(v[2 * i + 1] - h1)) << 16);
  }
  r.hi = u32x4{h[0], h[1], h[2], h[3]};
  r.lo = u32x4{l[0], l[1], l[2], l[3]};
  return r;
}

// Eight bf16 values (one 16-byte load) times eight floats given as hi + lo.
__device__ __forceinline__ float dot8_bf16_split(const u32x4 &b, const V8Split &v, float c) {
  return dot8_bf16(b, v.lo, dot8_bf16(b, v.hi, c));
}

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
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float((h & 0xffffu) << 16); }
// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bf16_round(float a) { return (float)(__bf16)a; }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// ---- int8 factors (LORA_FORMAT_INT8_ROWS): a block of fp32 row scales,
// then the int8 rows.  Integers of magnitude <= 128 are exact in bf16, so
// converting the values to bf16 keeps every product exact.
__device__ __forceinline__ int round_up4(int a) { return (a + 3) & ~3; }
__device__ __forceinline__ int ldb8_of(int rank) { return (rank + 15) & ~15; }
// Row stride (bytes) of an int8 A: d_in rounded up to a multiple of 16.
__device__ __forceinline__ uint32_t lda8_of(int d_in) { return (uint32_t)(d_in + 15) & ~15u; }
// Byte offset of the int8 values after the scales of `rows` rows.
__device__ __forceinline__ uint32_t q8_values_offset(int rows) { return (uint32_t)round_up4(rows) * 4; }
// Eight int8 values (one 8-byte load) as eight bf16 values (16 bytes).
__device__ __forceinline__ u32x4 i8x8_to_bf16x8(u32x2 q) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wv = i < 2 ? q.x : q.y;
    const int sh = (i & 1) * 16;
    o[i] = pack_bf16x2((float)(int8_t)(wv >> sh), (float)(int8_t)(wv >> (sh + 8)));
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}
// Eight signed 4-bit values (one dword, value j in bits 4j .. 4j+3, two's
// complement) as eight bf16 values: each is sign-extended and converted to
// fp32, whose upper half is then the exact bf16 (|q| <= 8 needs 4 bits).
__device__ __forceinline__ u32x4 q4x8_to_bf16x8(uint32_t q) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = (float)((int32_t)(q << (28 - 8 * i)) >> 28);
    const float hi = (float)((int32_t)(q << (24 - 8 * i)) >> 28);
    o[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}
// Eight int8 values (one 8-byte load) times eight floats, in fp32: each byte
// is sign-extended and converted exactly, then multiplied and added.
__device__ __forceinline__ float dot8_i8_f32(u32x2 q, const float *v, float c) {
#pragma unroll
  for (int k = 0; k < 8; ++k) c = fmaf((float)(int8_t)((k < 4 ? q.x : q.y) >> (8 * (k & 3))), v[k], c);
  return c;
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

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// The descriptor of the running kernel, read from the kernel argument
// segment (it is the first argument of every kernel of this library).  Lets
// a non-inlined function reach it without a copy in scratch memory.
__device__ __forceinline__ const LayerDesc &kernel_desc() {
  return *(const LayerDesc *)(const void *)__builtin_amdgcn_kernarg_segment_ptr();
}

// The module of item `it` of a segment (SG: in the SGMV expand numbering).
// The index is found with scalar compares; the chosen descriptor is then read
// straight from the kernel argument segment, where the LayerDesc is the first
// argument of every kernel of this library (indexing the by-value argument
// itself makes the compiler copy the whole descriptor to scratch memory).
template <bool SG = false>
__device__ __forceinline__ ModuleDesc module_of_item(const LayerDesc &d, int it) {
  int mi = 0;
#pragma unroll
  for (int k = 1; k < kMaxModules; ++k)
    if (k < d.n_active && it >= (SG ? d.mod[k].sg_item_base : d.mod[k].item_base)) mi = k;
  return kernel_desc().mod[mi];
}

// Values that are the same for the whole block, moved to scalar registers.
// Without this a buffer resource built from a loaded pointer can be taken as
// varying per lane, and every access through it becomes a loop over lanes.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
template <typename T>
__device__ __forceinline__ const T *uniform(const T *p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const T *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Validated segment of a block: slot, first sorted row and length; false
// (and the status word counted once) when the segments do not fit this batch.
__device__ __forceinline__ bool load_segment(const LayerDesc &d, int s, bool count, int *a, int *pos0, int *len) {
  *a = uniform(d.seg_adapter[s]);
  *pos0 = uniform(d.seg_offsets[s]);
  *len = uniform(d.seg_offsets[s + 1]) - *pos0;
  if ((unsigned)*a >= (unsigned)d.num_slots || *pos0 < 0 || *len <= 0 || *pos0 + *len > d.num_rows) {
    if (count && threadIdx.x == 0) atomicAdd(d.status, 1);
    return false;
  }
  return true;
}

// Whether a table entry describes a delta this launch can apply.
__device__ __forceinline__ bool entry_ok(const lora_adapter_entry_t &e, int max_rank) {
  return e.rank > 0 && e.rank <= max_rank && (e.format == LORA_FORMAT_BF16 || e.format == LORA_FORMAT_INT8_ROWS) &&
         e.A != nullptr &&
         ((uintptr_t)e.A & 15) == 0 && e.B != nullptr && ((uintptr_t)e.B & 15) == 0;
}

// Table entry of (slot, module) for a whole block (the slot is the same for
// every lane): false for rank 0 (no delta) and for a malformed entry
// (counted once through `count`).
__device__ __forceinline__ bool load_entry(const LayerDesc &d, int a, int col, bool count, lora_adapter_entry_t *e) {
  const lora_adapter_entry_t t = d.table[(int64_t)a * d.table_cols + col];
  e->A = uniform(t.A);
  e->B = uniform(t.B);
  e->rank = uniform(t.rank);
  e->scale = uniform(t.scale);
  e->format = uniform(t.format);
  e->reserved = 0;
  if (e->rank == 0) return false;
  if (!entry_ok(*e, d.max_rank)) {
    if (count && threadIdx.x == 0) atomicAdd(d.status, 1);
    return false;
  }
  return true;
}

// Staging of v into LDS: v_lds[i*64 + j] = scale * v[i][j] for the sorted
// rows p0 + i (i < nr) of a module and j < rank, zero elsewhere in the first
// ROWS rows; v is the sum of the k-chunk partials (or the caller's v when d.v
// is set).  A thread loads 4 columns of a row at a time.  issue() sends the
// first round of loads (a round covers U chunks); the caller then issues its
// own streaming loads, and finish() adds the remaining rounds and writes
// LDS, so the wait for v does not wait for the caller's stream.  With few
// rows the chunks are also split across threads and combined in LDS (v_lds
// needs 64*ROWS + 1024 floats then).  finish() ends with a block barrier.
template <int ROWS, int UR = 0>
struct VStage {
  static constexpr int PAIRS = ROWS * 16;  // (row, 4-column group) pairs
  static constexpr int PER = PAIRS >= kDecodeThreads ? PAIRS / kDecodeThreads : 1;
  static constexpr int SPLIT = PAIRS >= kDecodeThreads ? 1 : kDecodeThreads / PAIRS;  // threads per pair
  static constexpr int U = UR > 0 ? UR : PER >= 4 ? 2 : SPLIT > 1 ? 2 : 8;             // chunks per round
  static_assert(PAIRS % kDecodeThreads == 0 || kDecodeThreads % PAIRS == 0, "rows per stage");

  int p0, nr, rank, part;
  int row[PER], jq[PER];
  bool on[PER];
  f32x4_t got[U][PER];

  __device__ __forceinline__ void load_round(const LayerDesc &d, const ModuleDesc &m, int c0) {
    const int64_t chunk_stride = (int64_t)d.num_rows * d.rs;
    const float *base = d.part + ((int64_t)m.part_base * d.num_rows + p0) * d.rs;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const bool ok = on[k] && c0 + u * SPLIT < m.n_chunks;
        got[u][k] = *(const f32x4_t *)(ok ? base + (c0 + u * SPLIT) * chunk_stride + (int64_t)row[k] * d.rs + jq[k]
                                          : d.part);
        if (!ok) got[u][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
  }

  __device__ __forceinline__ void issue(const LayerDesc &d, const ModuleDesc &m, int p0_, int nr_, int rank_) {
    p0 = p0_;
    nr = nr_;
    rank = rank_;
    const int t = threadIdx.x;
    part = t / PAIRS;  // chunk phase (0 when SPLIT == 1)
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int pair = (t % PAIRS) + k * kDecodeThreads;
      row[k] = pair >> 4;
      jq[k] = (pair & 15) * 4;
      on[k] = row[k] < nr && jq[k] < rank;
    }
    if (d.v != nullptr) {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int b = on[k] && part == 0 ? d.perm[p0 + row[k]] : -1;
        const bool ok = (unsigned)b < (unsigned)d.num_rows;
        got[0][k] = *(const f32x4_t *)(ok ? d.v + (int64_t)b * d.ldv + jq[k] : d.v);
        if (!ok) got[0][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 1; u < U; ++u) got[u][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    } else {
      load_round(d, m, part);
    }
  }

  __device__ __forceinline__ void finish(const LayerDesc &d, const ModuleDesc &m, float scale, float *v_lds) {
    f32x4_t sum[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      sum[k] = got[0][k];
#pragma unroll
      for (int u = 1; u < U; ++u) sum[k] += got[u][k];
    }
    if (d.v == nullptr) {
      for (int c0 = part + U * SPLIT; c0 < m.n_chunks; c0 += U * SPLIT) {
        load_round(d, m, c0);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int k = 0; k < PER; ++k) sum[k] += got[u][k];
      }
    }
    if constexpr (SPLIT == 1) {
#pragma unroll
      for (int k = 0; k < PER; ++k)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          v_lds[row[k] * 64 + jq[k] + c] = row[k] < nr && jq[k] + c < rank ? sum[k][c] * scale : 0.f;
      __syncthreads();
    } else {
      const int t = threadIdx.x;
      float *red = v_lds + ROWS * 64;  // [SPLIT][PAIRS][4]
      *(f32x4_t *)(red + t * 4) = sum[0];
      __syncthreads();
      if (t < PAIRS * 4) {
        const int i = t >> 6, j = t & 63;
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < SPLIT; ++q) v += red[(q * PAIRS + (t >> 2)) * 4 + (t & 3)];
        v_lds[i * 64 + j] = i < nr && j < rank ? v * scale : 0.f;
      }
      __syncthreads();
    }
  }
};

}  // namespace lora
