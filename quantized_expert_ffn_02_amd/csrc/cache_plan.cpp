// Re-selection of one layer's cached experts from usage counts (host code).
//
// The expert cache holds the most used experts and adapts to the conversation
// ("Strata Runs 125B Qwen3.8-Flash-Next on a 12GB Gaming GPU at Up to 94 Tokens/s",
// section "How a 125B model fits in 12 GB"; the aireport.net page: a cache of the few
// thousand most frequently used experts, learned while chatting).  The pages give
// no policy; this library's reading is the plainest one:
//   - wanted = the n_slots experts with the largest counts (ties: lower id first);
//   - incoming = wanted experts without a slot, largest count first (ties: lower id);
//   - targets = the layer's free slots (ascending slot id), then the slots of resident
//     experts that are not wanted, least used first (ties: lower id first);
//   - move i puts incoming[i] into targets[i], for i < min(|incoming|, |targets|,
//     max_moves).
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "moe.h"

extern "C" int moe_cache_plan(const uint32_t* counts, const int32_t* slot_row, int32_t E, const int32_t* layer_slots,
                              int32_t n_slots, int32_t max_moves, int32_t* move_experts, int32_t* move_slots,
                              int32_t* n_moves) {
  if (!counts || !slot_row || !layer_slots || !n_moves || E <= 0 || n_slots < 0 || n_slots > E || max_moves < 0)
    return MOE_EINVAL;
  if (max_moves > 0 && (!move_experts || !move_slots)) return MOE_EINVAL;
  // every resident expert must sit in one of the layer's slots, one expert per slot
  std::vector<int32_t> owner(n_slots, -1);
  for (int32_t e = 0; e < E; ++e) {
    const int32_t s = slot_row[e];
    if (s < 0) continue;
    const int32_t* at = std::find(layer_slots, layer_slots + n_slots, s);
    if (at == layer_slots + n_slots) return MOE_EINVAL;
    const int32_t j = (int32_t)(at - layer_slots);
    if (owner[j] >= 0) return MOE_EINVAL;
    owner[j] = e;
  }
  for (int32_t j = 0; j < n_slots; ++j)
    for (int32_t i = 0; i < j; ++i)
      if (layer_slots[i] == layer_slots[j]) return MOE_EINVAL;

  std::vector<int32_t> by_use(E);
  for (int32_t e = 0; e < E; ++e) by_use[e] = e;
  std::stable_sort(by_use.begin(), by_use.end(), [&](int32_t a, int32_t b) { return counts[a] > counts[b]; });
  std::vector<char> wanted(E, 0);
  for (int32_t i = 0; i < n_slots; ++i) wanted[by_use[i]] = 1;

  std::vector<int32_t> incoming;   // already in order: count descending, id ascending
  for (int32_t i = 0; i < n_slots; ++i)
    if (slot_row[by_use[i]] < 0) incoming.push_back(by_use[i]);

  std::vector<int32_t> free_slots, victims;
  for (int32_t j = 0; j < n_slots; ++j)
    if (owner[j] < 0) free_slots.push_back(layer_slots[j]);
  std::sort(free_slots.begin(), free_slots.end());
  for (int32_t j = 0; j < n_slots; ++j)
    if (owner[j] >= 0 && !wanted[owner[j]]) victims.push_back(owner[j]);
  std::sort(victims.begin(), victims.end(), [&](int32_t a, int32_t b) {
    return counts[a] != counts[b] ? counts[a] < counts[b] : a < b;
  });
  std::vector<int32_t> targets = free_slots;
  for (int32_t e : victims) targets.push_back(slot_row[e]);

  const size_t n = std::min({incoming.size(), targets.size(), (size_t)max_moves});
  for (size_t i = 0; i < n; ++i) {
    move_experts[i] = incoming[i];
    move_slots[i] = targets[i];
  }
  *n_moves = (int32_t)n;
  return MOE_OK;
}
