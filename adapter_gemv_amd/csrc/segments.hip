// Segment builder: group the rows of a batch by adapter slot.
//
// "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A": the batched kernel
// receives an index vector mapping each sequence to an adapter slot.
// "LoRA, quotas and noisy neighbours", "One weight read, many adapters": rows
// are tagged with their adapter and grouped so that each group reads its
// adapter once.  The grouping here is a stable counting sort by slot id:
// segments in ascending slot order, rows ascending inside a segment.  Negative
// ids are base-only rows and join no segment; ids >= num_slots are counted
// into the status word and skipped.
//
// A row's place inside its segment is the number of earlier rows with the same
// id.  Each thread finds it by scanning the ids of its block from LDS, and the
// last row of each id in the block writes the block's count for that id, so no
// atomics are needed and the result is deterministic.
//   * up to kSegSmallMax rows: one block does everything (decode batches);
//   * more rows: one block per chunk of kSegChunk rows writes per-chunk counts
//     and in-chunk ranks, then one block turns them into offsets and scatters.
#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kWaves = kSegThreads / 64;

// Exclusive scan of one int per thread over the block; *total gets the sum.
__device__ int block_excl_scan(int x, int *total, int *s_w) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  if (w == 0) {
    int v = lane < kWaves ? s_w[lane] : 0;
    int vi = v;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      int y = __shfl_up(vi, d, 64);
      if (lane >= d) vi += y;
    }
    if (lane < kWaves) s_w[lane] = vi - v;
    if (lane == kWaves - 1) s_w[kWaves] = vi;
  }
  __syncthreads();
  const int res = s_w[w] + inc - x;
  *total = s_w[kWaves];
  __syncthreads();
  return res;
}

__device__ int block_sum(int x, int *s_w) {
  int total;
  block_excl_scan(x, &total, s_w);
  return total;
}

// counts[a] (rows of slot a) -> exclusive row offsets in place; writes the
// segment list for every non-empty slot.
__device__ void scan_slots(int32_t *counts, int num_slots, const lora_segments_t &seg, int *s_w) {
  int carry_rows = 0, carry_segs = 0;
  for (int base = 0; base < num_slots; base += kSegThreads) {
    const int a = base + threadIdx.x;
    const int c = a < num_slots ? counts[a] : 0;
    const int f = c > 0;
    int tot_c, tot_f;
    const int ex_c = block_excl_scan(c, &tot_c, s_w);
    const int ex_f = block_excl_scan(f, &tot_f, s_w);
    if (a < num_slots) {
      const int start = carry_rows + ex_c;
      counts[a] = start;
      if (f) {
        seg.seg_offsets[carry_segs + ex_f] = start;
        seg.seg_adapter[carry_segs + ex_f] = a;
      }
    }
    carry_rows += tot_c;
    carry_segs += tot_f;
  }
  if (threadIdx.x == 0) {
    seg.seg_offsets[carry_segs] = carry_rows;
    *seg.num_segments = carry_segs;
  }
}

// Rows of this block with the same id before / after row t.  s_ids holds the
// block's ids in LDS (16-byte aligned, -1 past the end, so a valid id never
// matches padding); four ids per LDS read.
__device__ void same_id_counts(const int *s_ids, int len, int t, int id, int *before, int *after) {
  const int4 *s4 = reinterpret_cast<const int4 *>(s_ids);
  const int n4 = (len + 3) >> 2;
  int bf = 0, tot = 0;
  for (int b4 = 0; b4 < n4; ++b4) {
    const int4 v = s4[b4];
    const int b = b4 * 4;
    const int e0 = v.x == id, e1 = v.y == id, e2 = v.z == id, e3 = v.w == id;
    tot += e0 + e1 + e2 + e3;
    bf += (e0 & (b < t)) + (e1 & (b + 1 < t)) + (e2 & (b + 2 < t)) + (e3 & (b + 3 < t));
  }
  *before = bf;
  *after = tot - bf - 1;  // tot counts row t itself
}

// Slot tables up to this size keep their counts in LDS.
constexpr int kSegLdsSlots = 8192;

__global__ __launch_bounds__(kSegThreads) void seg_small_kernel(const int32_t *__restrict__ ids, int n,
                                                                int num_slots, lora_segments_t seg,
                                                                int32_t *__restrict__ ws_counts) {
  __shared__ __align__(16) int s_ids[kSegSmallMax];
  __shared__ int s_counts[kSegLdsSlots];
  __shared__ int s_w[kWaves + 1];
  int32_t *counts = num_slots <= kSegLdsSlots ? s_counts : ws_counts;
  const int t = threadIdx.x;
  int id = -1, bad = 0;
  if (t < n) {
    const int r = ids[t];
    if (r >= num_slots) bad = 1;
    else if (r >= 0) id = r;
  }
  s_ids[t] = id;
  for (int a = t; a < num_slots; a += kSegThreads) counts[a] = 0;
  const int nbad = block_sum(bad, s_w);  // also orders the LDS and count stores
  int before = 0, after = 0;
  if (id >= 0) same_id_counts(s_ids, n, t, id, &before, &after);
  if (id >= 0 && after == 0) counts[id] = before + 1;
  __syncthreads();
  scan_slots(counts, num_slots, seg, s_w);
  __syncthreads();
  if (id >= 0) seg.perm[counts[id] + before] = t;
  if (t == 0) *seg.status = nbad;
}

// Per chunk of kSegChunk rows: hist[c][a] = rows of slot a in the chunk,
// lrank[row] = earlier rows of the same slot in the chunk, bad[c].
__global__ __launch_bounds__(kSegThreads) void seg_chunk_kernel(const int32_t *__restrict__ ids, int n,
                                                                int num_slots, int32_t *__restrict__ hist,
                                                                int32_t *__restrict__ lrank,
                                                                int32_t *__restrict__ badc) {
  __shared__ __align__(16) int s_ids[kSegChunk];
  __shared__ int s_w[kWaves + 1];
  const int t = threadIdx.x;
  const int c = blockIdx.x;
  const int row = c * kSegChunk + t;
  const int len = min(kSegChunk, n - c * kSegChunk);
  int32_t *hist_c = hist + (size_t)c * num_slots;
  int id = -1, bad = 0;
  if (t < len) {
    const int r = ids[row];
    if (r >= num_slots) bad = 1;
    else if (r >= 0) id = r;
  }
  s_ids[t] = id;
  for (int a = t; a < num_slots; a += kSegThreads) hist_c[a] = 0;
  const int nbad = block_sum(bad, s_w);
  int before = 0, after = 0;
  if (id >= 0) same_id_counts(s_ids, len, t, id, &before, &after);
  if (id >= 0 && after == 0) hist_c[id] = before + 1;
  if (id >= 0) lrank[row] = before;
  if (t == 0) badc[c] = nbad;
}

// One block: chunk counts -> per-(chunk, slot) offsets, segments, scatter.
__global__ __launch_bounds__(kSegThreads) void seg_finish_kernel(const int32_t *__restrict__ ids, int n,
                                                                 int num_slots, int nchunks, lora_segments_t seg,
                                                                 int32_t *__restrict__ hist,
                                                                 const int32_t *__restrict__ lrank,
                                                                 const int32_t *__restrict__ badc,
                                                                 int32_t *__restrict__ start) {
  __shared__ int s_w[kWaves + 1];
  const int t = threadIdx.x;
  for (int a = t; a < num_slots; a += kSegThreads) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int h = hist[(size_t)c * num_slots + a];
      hist[(size_t)c * num_slots + a] = run;
      run += h;
    }
    start[a] = run;
  }
  int bad = 0;
  for (int c = t; c < nchunks; c += kSegThreads) bad += badc[c];
  const int nbad = block_sum(bad, s_w);
  scan_slots(start, num_slots, seg, s_w);
  __syncthreads();
  for (int row = t; row < n; row += kSegThreads) {
    const int id = ids[row];
    if (id >= 0 && id < num_slots)
      seg.perm[start[id] + hist[(size_t)(row / kSegChunk) * num_slots + id] + lrank[row]] = row;
  }
  if (t == 0) *seg.status = nbad;
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

size_t segments_ws_bytes(int num_rows, int num_slots) {
  if (num_rows <= kSegSmallMax) return num_slots <= kSegLdsSlots ? 0 : align256((size_t)num_slots * 4);
  const size_t nchunks = ((size_t)num_rows + kSegChunk - 1) / kSegChunk;
  return align256((size_t)num_rows * 4) + align256(nchunks * 4) + align256((size_t)num_slots * 4) +
         align256(nchunks * (size_t)num_slots * 4);
}

hipError_t launch_build_segments(const int32_t *ids, int n, int num_slots, const lora_segments_t &seg, void *ws,
                                 hipStream_t stream) {
  char *w = static_cast<char *>(ws);
  if (n <= kSegSmallMax) {
    seg_small_kernel<<<1, kSegThreads, 0, stream>>>(ids, n, num_slots, seg, reinterpret_cast<int32_t *>(w));
    return hipGetLastError();
  }
  const int nchunks = (n + kSegChunk - 1) / kSegChunk;
  int32_t *lrank = reinterpret_cast<int32_t *>(w);
  w += align256((size_t)n * 4);
  int32_t *badc = reinterpret_cast<int32_t *>(w);
  w += align256((size_t)nchunks * 4);
  int32_t *start = reinterpret_cast<int32_t *>(w);
  w += align256((size_t)num_slots * 4);
  int32_t *hist = reinterpret_cast<int32_t *>(w);
  seg_chunk_kernel<<<nchunks, kSegThreads, 0, stream>>>(ids, n, num_slots, hist, lrank, badc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  seg_finish_kernel<<<1, kSegThreads, 0, stream>>>(ids, n, num_slots, nchunks, seg, hist, lrank, badc, start);
  return hipGetLastError();
}

}  // namespace lora
