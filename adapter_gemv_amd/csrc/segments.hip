// Segment builder: group the rows of a batch by adapter slot.  Row b's id is
// ids[b * stride] (stride > 1: one column of a row's adapter list); the status
// word gets the rows with an id >= num_slots, or has them added (a later pass
// over another column of the same list).
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
// A block sorts its rows by slot id with a stable radix sort (one bit per
// pass; a ballot splits each wave's rows, the waves' counts place them), so
// rows of one slot keep their order, no atomics are needed and the result is
// deterministic.  A row's place inside its group of equal ids is then its
// sorted place minus the start of its id's run.
//   * up to kSegSmallMax rows: one block (sized to the batch) does everything;
//   * more rows: per chunk of kSegChunk rows, counts per slot and in-chunk
//     ranks; then one block scans the count table in slot-major order, which
//     gives every (slot, chunk) its first output position and every slot its
//     segment; then every chunk scatters its rows.
#include "block_sort.h"
#include "lora_internal.h"

namespace lora {
namespace {

// The end of a build, by one thread once every segment start is written:
// segs segments hold `rows` rows.  Past the caller's bound (max_segments)
// the segments of the highest slots are dropped and their rows counted as
// bad; the status word gets (or, add_status, has added) the bad rows.
__device__ void finish_segments(const lora_segments_t &seg, int segs, int rows, bool add_status, int nbad) {
  if (seg.max_segments > 0 && segs > seg.max_segments) {
    nbad += rows - seg.seg_offsets[seg.max_segments];  // the kept rows end where segment max_segments starts
    segs = seg.max_segments;
  } else {
    seg.seg_offsets[segs] = rows;
  }
  *seg.num_segments = segs;
  *seg.status = add_status ? *seg.status + nbad : nbad;
}

// Exclusive scan of one int per thread over a block of THREADS threads;
// *total gets the sum.  s_w holds THREADS/64 + 1 ints.
template <int THREADS>
__device__ int block_excl_scan(int x, int *total, int *s_w) {
  constexpr int kWaves = THREADS / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int v = lane < kWaves ? s_w[lane] : 0;
    int vi = v;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const int y = __shfl_up(vi, d, 64);
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

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Segments a build keeps: all, or the caller's bound when there are more.
__device__ __forceinline__ int kept_segments(const lora_segments_t &seg, int segs) {
  return seg.max_segments > 0 && segs > seg.max_segments ? seg.max_segments : segs;
}

// Every thread of the (scan) block, once the kept segments' offsets are
// written: the SGMV row tiles of those segments (segments of at least kLongSegRows
// rows, in batches of at least that many rows) for the other calls, in
// tiles of kSgmvShrinkRows and of kSgmvExpandRows rows.
template <int THREADS>
__device__ void count_long_tiles(const lora_segments_t &seg, int n, int segs, int *s_w) {
  int shr = 0, exp = 0;
  if (n >= kLongSegRows) {
    for (int s = threadIdx.x; s < segs; s += THREADS) {
      const int len = seg.seg_offsets[s + 1] - seg.seg_offsets[s];
      if (len >= kLongSegRows) {
        shr += ceil_div(len, kSgmvShrinkRows);
        exp += ceil_div(len, kSgmvExpandRows);
      }
    }
  }
  int tot_shr, tot_exp;
  block_excl_scan<THREADS>(shr, &tot_shr, s_w);
  block_excl_scan<THREADS>(exp, &tot_exp, s_w);
  if (threadIdx.x == 0) {
    seg.tile_counts[0] = tot_shr;
    seg.tile_counts[1] = tot_exp;
  }
}

// n <= THREADS rows in one block: the rows sorted by slot, then segment
// starts where the slot changes, one scan for their indices, and the
// outputs; the status word gets the ids >= num_slots (and, past the caller's
// bound, the rows of the dropped segments).
template <int THREADS>
__global__ __launch_bounds__(THREADS) void seg_small_kernel(const int32_t *__restrict__ ids, int stride, int n,
                                                            int num_slots, bool add_status, lora_segments_t seg) {
  __shared__ int s_key[2][THREADS];
  __shared__ int s_row[2][THREADS];
  __shared__ int s_start[THREADS];
  __shared__ int s_w[THREADS / 64 + 1];
  const int t = threadIdx.x;
  int key = num_slots, bad = 0;  // num_slots: no segment (base only, a bad id, or past the batch)
  if (t < n) {
    const int r = ids[(int64_t)t * stride];
    if (r >= num_slots) bad = 1;
    else if (r >= 0) key = r;
  }
  int row = t;
  const int fb = block_radix_sort<THREADS>(&key, &row, key_bits(num_slots), s_key, s_row, s_w);
  // thread t now holds sorted place t; rows with no segment sort last
  const bool valid = key < num_slots;
  const bool starts = valid && (t == 0 || s_key[fb][t - 1] != key);
  int nseg, nvalid, nbad;
  const int sidx = block_excl_scan<THREADS>(starts ? 1 : 0, &nseg, s_w);
  block_excl_scan<THREADS>(valid ? 1 : 0, &nvalid, s_w);
  block_excl_scan<THREADS>(bad, &nbad, s_w);
  if (valid) seg.perm[t] = row;
  if (starts) {
    seg.seg_offsets[sidx] = t;
    seg.seg_adapter[sidx] = key;
    s_start[sidx] = t;
  }
  __syncthreads();
  int tiles = 0;  // SGMV tiles of a kept segment: expand | shrink << 16 (at most 144 each)
  if (starts && (seg.max_segments <= 0 || sidx < seg.max_segments) && n >= kLongSegRows) {
    const int len = (sidx + 1 < nseg ? s_start[sidx + 1] : nvalid) - t;
    if (len >= kLongSegRows) tiles = ceil_div(len, kSgmvExpandRows) | ceil_div(len, kSgmvShrinkRows) << 16;
  }
  int all_tiles;
  block_excl_scan<THREADS>(tiles, &all_tiles, s_w);  // its barriers also publish every segment start
  if (t == 0) {
    finish_segments(seg, nseg, nvalid, add_status, nbad);
    seg.tile_counts[0] = all_tiles >> 16;
    seg.tile_counts[1] = all_tiles & 0xffff;
  }
}

// Chunk c of kSegChunk rows: hist[a * nchunks + c] = rows of slot a in the
// chunk (slot-major), lrank[row] = earlier rows of the same slot in the
// chunk, badc[c] = rows with an id >= num_slots.
__global__ __launch_bounds__(kSegChunk) void seg_chunk_kernel(const int32_t *__restrict__ ids, int stride, int n,
                                                              int num_slots, int nchunks, int32_t *__restrict__ hist,
                                                              int32_t *__restrict__ lrank,
                                                              int32_t *__restrict__ badc) {
  __shared__ int s_key[2][kSegChunk];
  __shared__ int s_row[2][kSegChunk];
  __shared__ int s_w[kSegChunk / 64 + 1];
  const int t = threadIdx.x;
  const int c = blockIdx.x;
  const int len = min(kSegChunk, n - c * kSegChunk);
  int key = num_slots, bad = 0;  // num_slots: no segment
  if (t < len) {
    const int r = ids[(int64_t)(c * kSegChunk + t) * stride];
    if (r >= num_slots) bad = 1;
    else if (r >= 0) key = r;
  }
  for (int a = t; a < num_slots; a += kSegChunk) hist[(size_t)a * nchunks + c] = 0;
  int nbad;
  block_excl_scan<kSegChunk>(bad, &nbad, s_w);  // also orders the zeroing before the counts
  int row = t;
  const int fb = block_radix_sort<kSegChunk>(&key, &row, key_bits(num_slots), s_key, s_row, s_w);
  if (key < num_slots) {
    // the run of this key in the sorted chunk: [first, last]
    int lo = 0, hi = t;  // first place with a key >= this one
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_key[fb][mid] < key) lo = mid + 1;
      else hi = mid;
    }
    lrank[c * kSegChunk + row] = t - lo;
    if (t + 1 == kSegChunk || s_key[fb][t + 1] != key) hist[(size_t)key * nchunks + c] = t - lo + 1;
  }
  if (t == 0) badc[c] = nbad;
}

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 8;  // consecutive elements per thread and pass

// One block: exclusive scan of hist in slot-major order (the first output
// position of each (slot, chunk)), then the segments: slot a opens one at
// hist[a * nchunks] when its rows are non-zero.
__global__ __launch_bounds__(kScanThreads) void seg_scan_kernel(int n, int num_slots, int nchunks, bool add_status,
                                                                lora_segments_t seg,
                                                                int32_t *__restrict__ hist,
                                                                const int32_t *__restrict__ badc) {
  __shared__ int s_w[kScanThreads / 64 + 1];
  const int t = threadIdx.x;
  const int64_t total = (int64_t)num_slots * nchunks;
  int carry = 0;
  for (int64_t base = 0; base < total; base += (int64_t)kScanThreads * kScanPer) {
    const int64_t i0 = base + (int64_t)t * kScanPer;
    int v[kScanPer];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      v[k] = i0 + k < total ? hist[i0 + k] : 0;
      sum += v[k];
    }
    int tot;
    int ex = block_excl_scan<kScanThreads>(sum, &tot, s_w) + carry;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      if (i0 + k < total) hist[i0 + k] = ex;
      ex += v[k];
    }
    carry += tot;
  }
  // hist now holds exclusive positions; slot a's rows are [hist[a*nchunks], next slot's).
  __syncthreads();
  int bad = 0;
  for (int c = t; c < nchunks; c += kScanThreads) bad += badc[c];
  int nbad;
  block_excl_scan<kScanThreads>(bad, &nbad, s_w);
  int segs = 0;
  for (int base = 0; base < num_slots; base += kScanThreads) {
    const int a = base + t;
    int first = 0, cnt = 0;
    if (a < num_slots) {
      first = hist[(size_t)a * nchunks];
      const int next = a + 1 < num_slots ? hist[(size_t)(a + 1) * nchunks] : carry;
      cnt = next - first;
    }
    int tot;
    const int ex = block_excl_scan<kScanThreads>(cnt > 0, &tot, s_w) + segs;
    if (cnt > 0) {
      seg.seg_offsets[ex] = first;
      seg.seg_adapter[ex] = a;
    }
    segs += tot;
  }
  __syncthreads();  // every segment start is written
  if (t == 0) finish_segments(seg, segs, carry, add_status, nbad);
  __syncthreads();
  count_long_tiles<kScanThreads>(seg, n, kept_segments(seg, segs), s_w);
}

// Chunk c: every valid row goes to its slot's position for this chunk plus
// its rank inside the chunk.
__global__ __launch_bounds__(kSegChunk) void seg_scatter_kernel(const int32_t *__restrict__ ids, int stride, int n,
                                                                int num_slots, int nchunks, lora_segments_t seg,
                                                                const int32_t *__restrict__ hist,
                                                                const int32_t *__restrict__ lrank) {
  const int row = blockIdx.x * kSegChunk + threadIdx.x;
  if (row >= n) return;
  const int id = ids[(int64_t)row * stride];
  if (id >= 0 && id < num_slots) seg.perm[hist[(size_t)id * nchunks + blockIdx.x] + lrank[row]] = row;
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

size_t segments_ws_bytes(int num_rows, int num_slots) {
  if (num_rows <= kSegSmallMax) return 0;
  const size_t nchunks = ((size_t)num_rows + kSegChunk - 1) / kSegChunk;
  return align256((size_t)num_rows * 4) + align256(nchunks * 4) + align256(nchunks * (size_t)num_slots * 4);
}

hipError_t launch_build_segments(const int32_t *ids, int stride, int n, int num_slots, bool add_status,
                                 const lora_segments_t &seg, void *ws, hipStream_t stream) {
  char *w = static_cast<char *>(ws);
  if (n <= 256) {
    seg_small_kernel<256><<<1, 256, 0, stream>>>(ids, stride, n, num_slots, add_status, seg);
    return hipGetLastError();
  }
  if (n <= kSegSmallMax) {
    seg_small_kernel<kSegSmallMax><<<1, kSegSmallMax, 0, stream>>>(ids, stride, n, num_slots, add_status, seg);
    return hipGetLastError();
  }
  const int nchunks = (n + kSegChunk - 1) / kSegChunk;
  int32_t *lrank = reinterpret_cast<int32_t *>(w);
  w += align256((size_t)n * 4);
  int32_t *badc = reinterpret_cast<int32_t *>(w);
  w += align256((size_t)nchunks * 4);
  int32_t *hist = reinterpret_cast<int32_t *>(w);
  seg_chunk_kernel<<<nchunks, kSegChunk, 0, stream>>>(ids, stride, n, num_slots, nchunks, hist, lrank, badc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  seg_scan_kernel<<<1, kScanThreads, 0, stream>>>(n, num_slots, nchunks, add_status, seg, hist, badc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  seg_scatter_kernel<<<nchunks, kSegChunk, 0, stream>>>(ids, stride, n, num_slots, nchunks, seg, hist, lrank);
  return hipGetLastError();
}

}  // namespace lora
