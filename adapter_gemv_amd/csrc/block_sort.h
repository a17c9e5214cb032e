// Block-wide stable sort of small integer keys, shared by the segment
// builders (segments.hip, and block 0 of the one-launch decode).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace lora {

// Stable sort of the block's rows by key, keys in [0, 2^bits): one pass per
// bit, least significant first.  In a pass a ballot splits each wave's rows
// into zeros and ones; a row goes to (zeros of earlier waves + zeros below it
// in its wave), or past every zero to (ones of earlier waves + ones below
// it), so equal keys keep their order.  In: this thread's key and value.
// Out: the key and value at sorted place threadIdx.x; the sorted keys stay in
// s_key[return value].  s_w holds THREADS/64 ints.
template <int THREADS>
__device__ int block_radix_sort(int *key, int *val, int bits, int (*s_key)[THREADS], int (*s_val)[THREADS],
                                int *s_w) {
  constexpr int kWaves = THREADS / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int buf = 0;
  for (int b = 0; b < bits; ++b) {
    const bool one = (*key >> b) & 1;
    const uint64_t zeros = __ballot(!one);
    const int zb = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(zeros >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)zeros, 0u));
    if (lane == 0) s_w[w] = __popcll(zeros);
    __syncthreads();
    int zw = 0, ztot = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const int c = s_w[k];
      zw += k < w ? c : 0;
      ztot += c;
    }
    const int dest = one ? ztot + (64 * w - zw) + (lane - zb) : zw + zb;
    s_key[buf][dest] = *key;
    s_val[buf][dest] = *val;
    __syncthreads();  // also: every wave has read s_w before the next pass writes it
    *key = s_key[buf][t];
    *val = s_val[buf][t];
    buf ^= 1;  // the next pass writes the other buffer while this one may still be read
  }
  return buf ^ 1;
}

// Bits of the keys 0 .. num_slots (num_slots: a row with no segment).
__device__ __forceinline__ int key_bits(int num_slots) { return 32 - __clz(num_slots); }

}  // namespace lora
