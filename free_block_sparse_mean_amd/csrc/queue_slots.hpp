// Pool of the fused pass's work-item queue counters (host side; no HIP here).
//
// Each fused launch takes one counter (a slot of a static device array) and
// clears it with a kernel on its own stream just before it runs. Launches in
// flight at the same time must hold different slots. Eager launches take the
// slots round-robin from the first kEagerSlots; a launch recorded into a
// graph keeps its slot for every replay, so captured launches take theirs
// round-robin from the last kCapturedSlots, which eager launches never use.
#pragma once

#include <atomic>
#include <cstdint>

namespace sol {

constexpr int kQueueSlots = 4096;                          // counters in device memory
constexpr int kCapturedSlots = 1024;                       // reserved for captured launches
constexpr int kEagerSlots = kQueueSlots - kCapturedSlots;  // shared by eager launches

class QueueSlots {
 public:
  // Slot for the next launch; `captured`: the launch is being recorded into a graph.
  int take(bool captured) {
    if (captured) return kEagerSlots + (int)(captured_.fetch_add(1, std::memory_order_relaxed) % kCapturedSlots);
    return (int)(eager_.fetch_add(1, std::memory_order_relaxed) % kEagerSlots);
  }

 private:
  std::atomic<uint64_t> eager_{0};
  std::atomic<uint64_t> captured_{0};
};

}  // namespace sol
