// expert_cache.h -- host-side bookkeeping of the HBM expert cache of the
// host-memory expert tier: which (layer, expert) blob each of n_slots device
// slots holds, and which slot to overwrite next (least recently used).
//
// The pages keep the experts on the SSD and let the operating system's page
// cache decide which stay in memory ("397B MoE en MacBook: Motor Flash-MoE a
// 4,4 t/s", section "1. Streaming de expertos desde SSD + 'Confia en el SO'";
// "Flash-MoE: Ausfuehren eines 397B-Parameter-Qwen-Modells auf dem MacBook Pro
// mit reinem C/Metal", section "SSD-Experten-Streaming"). Here the slow tier is
// host memory and the fast one HBM; the policy is least-recently-used, as a page
// cache approximates it, and deterministic: a plan for the experts of one call
// looks them up in the order given; a hit refreshes the slot's use; a miss takes
// the first empty slot, else the slot used longest ago among those the call does
// not need, ties to the lower slot.
#pragma once

#include <stdint.h>

#include <unordered_map>
#include <vector>

namespace fmoe {

class ExpertCache {
 public:
  explicit ExpertCache(int n_slots) : key_(n_slots, -1), last_(n_slots, 0), stamp_(n_slots, 0) {}

  int slots() const { return (int)key_.size(); }

  // Plans one call: slot_out[i] is the slot of experts[i] of `layer` (n distinct
  // experts), miss_out[i] 1 when that slot must be filled now. false (nothing
  // changed) if n exceeds the slots.
  bool plan(int layer, const int32_t *experts, int n, int32_t *slot_out, int32_t *miss_out) {
    if (n > slots()) return false;
    ++call_;
    // the call's experts that are resident already: kept for the call
    for (int i = 0; i < n; ++i) {
      const auto it = map_.find(key(layer, experts[i]));
      if (it != map_.end()) stamp_[it->second] = call_;
    }
    for (int i = 0; i < n; ++i) {
      const int64_t k = key(layer, experts[i]);
      const auto it = map_.find(k);
      int s;
      if (it != map_.end()) {
        s = it->second;
        ++hits_;
        miss_out[i] = 0;
      } else {
        s = victim();
        if (key_[s] >= 0) map_.erase(key_[s]);
        key_[s] = k;
        map_[k] = s;
        stamp_[s] = call_;
        ++misses_;
        miss_out[i] = 1;
      }
      last_[s] = ++clock_;
      slot_out[i] = s;
    }
    return true;
  }

  int64_t hits() const { return hits_; }
  int64_t misses() const { return misses_; }

 private:
  static int64_t key(int layer, int expert) { return ((int64_t)layer << 32) | (uint32_t)expert; }

  // the first empty slot, else the least recently used one the current call does not hold
  int victim() const {
    int best = -1;
    for (int s = 0; s < slots(); ++s) {
      if (key_[s] < 0) return s;
      if (stamp_[s] == call_) continue;
      if (best < 0 || last_[s] < last_[best]) best = s;
    }
    return best;  // (the caller checked n <= slots, so one exists)
  }

  std::vector<int64_t> key_;    // (layer, expert) held by each slot, -1: empty
  std::vector<uint64_t> last_;  // use clock of each slot
  std::vector<uint64_t> stamp_; // the call that holds each slot (call_ = the current one)
  std::unordered_map<int64_t, int> map_;
  uint64_t clock_ = 0, call_ = 0;
  int64_t hits_ = 0, misses_ = 0;
};

}  // namespace fmoe
