// Adapter-aware batch former (host code): picks the requests of the next step
// from a waiting queue so that the batch shares adapters.
//
// "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A": "The adapter-aware
// scheduler" (groups by adapter, biggest first, whole where possible; no new
// adapter once the batch holds max_distinct of them and min_batch requests)
// and "The fairness cost, which must be stated" (requests past a deadline go
// first); "The Revision", R1 (a few slots held for the oldest requests whose
// adapter no other waiting request uses).  "12. Adapter Serving and
// Multi-Tenant Customization", "Batching across adapters": base-only requests
// are a group of their own.
//
// The work is a handful of sorts over the queue: O(n log n), no device work.
// Group membership comes from one stable sort of queue positions by adapter,
// so every group lists its members oldest first and the groups can be ordered
// by (size descending, oldest member ascending).
#include <algorithm>
#include <cstdint>
#include <vector>

#include "lora_gemv.h"

namespace {

struct Group {
  int32_t first;  // queue position of the oldest member
  int32_t begin;  // members: pos[begin, begin + size)
  int32_t size;
  bool adapter;   // false: the base-only group
};

// Positions `pos` (queue order) regrouped by key with a stable sort; fills
// the groups in `out`, members oldest first.
template <class Key>
void group_by(std::vector<int32_t> &pos, Key key, std::vector<Group> &out) {
  std::stable_sort(pos.begin(), pos.end(), [&](int32_t a, int32_t b) { return key(a) < key(b); });
  out.clear();
  for (size_t i = 0; i < pos.size();) {
    size_t j = i + 1;
    while (j < pos.size() && key(pos[j]) == key(pos[i])) ++j;
    out.push_back(Group{pos[i], (int32_t)i, (int32_t)(j - i), key(pos[i]) >= 0});
    i = j;
  }
}

}  // namespace

extern "C" lora_status_t lora_form_batch(const int32_t *adapters, int32_t queue_len, const float *waited_ms,
                                         float max_wait_ms, int32_t max_batch, int32_t max_distinct,
                                         int32_t min_batch, int32_t reserved_tail, int32_t *out_index,
                                         int32_t *out_count) {
  if (out_count == nullptr || out_index == nullptr || (adapters == nullptr && queue_len > 0)) return LORA_ERR_NULL;
  if (queue_len < 0 || max_batch < 1 || max_distinct < 0 || min_batch < 0 || reserved_tail < 0) return LORA_ERR_SHAPE;
  const int32_t n = queue_len;
  std::vector<uint8_t> taken((size_t)n, 0);
  int32_t count = 0;
  auto take = [&](int32_t i) {
    out_index[count++] = i;
    taken[(size_t)i] = 1;
  };

  // Age override: every request past the deadline, oldest first.
  if (waited_ms != nullptr)
    for (int32_t i = 0; i < n && count < max_batch; ++i)
      if (waited_ms[i] > max_wait_ms) take(i);

  // Reserved tail: the oldest requests whose adapter has no other request
  // among those still waiting.
  std::vector<int32_t> pos;
  std::vector<Group> groups;
  pos.reserve((size_t)n);
  for (int32_t i = 0; i < n; ++i)
    if (!taken[(size_t)i] && adapters[i] >= 0) pos.push_back(i);
  group_by(pos, [&](int32_t i) { return adapters[i]; }, groups);
  std::vector<uint8_t> alone((size_t)n, 0);
  for (const Group &g : groups)
    if (g.size == 1) alone[(size_t)g.first] = 1;
  int32_t tail = 0;
  const int32_t tail_cap = std::min(reserved_tail, max_distinct);  // the reserved slots are part of the budget
  for (int32_t i = 0; i < n && tail < tail_cap && count < max_batch; ++i)
    if (alone[(size_t)i] && !taken[(size_t)i]) {
      take(i);
      ++tail;
    }

  // Grouped fill of the rest: base-only requests share the key -1.
  pos.clear();
  for (int32_t i = 0; i < n; ++i)
    if (!taken[(size_t)i]) pos.push_back(i);
  group_by(pos, [&](int32_t i) { return adapters[i] < 0 ? -1 : adapters[i]; }, groups);
  std::sort(groups.begin(), groups.end(), [](const Group &a, const Group &b) {
    return a.size != b.size ? a.size > b.size : a.first < b.first;
  });
  const int32_t budget = max_distinct - tail;
  int32_t distinct = 0;
  for (const Group &g : groups) {
    if (count >= max_batch) break;
    if (distinct >= budget && count >= min_batch) break;  // no new adapter: the batch is big enough
    const int32_t k = std::min(g.size, max_batch - count);
    for (int32_t m = 0; m < k; ++m) take(pos[(size_t)(g.begin + m)]);
    if (g.adapter) ++distinct;
  }
  *out_count = count;
  return LORA_OK;
}
