// Arrival counters of the balanced decode step: how many tiles of a sequence's pieces have been
// attended so far in one call, tagged with that call's generation.
//
// A counter is one 64-bit word: the generation of the call that last counted into it in the high
// 32 bits, the tiles counted by that call in the low 32 bits.  Every call of the step gets a new,
// larger generation (a per-process count of calls, taken on the host).  A piece arrives in two
// agent-scope atomic operations on its sequence's word, in this order from one thread:
//   1. max(word, generation << 32): a word left by an earlier call (smaller generation) — for
//      instance one that never reached its merge — becomes (generation, 0); a word this call has
//      already counted into is left as it is;
//   2. fetch-add(word, tiles): the returned low half is what this call counted before.
// Both operations address the same word from the same thread, so they take effect in this order
// for every observer.  The arrival that brings the count to the sequence's tile total merges the
// pieces and then writes 0, so a completed call leaves every counter it used at zero (which also
// serves a captured graph, whose replays reuse one generation).
//
// The arithmetic is kept here, apart from the atomics, so that it can be checked on the host.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define PKV_HD __host__ __device__
#else
#define PKV_HD
#endif

namespace pkv {

// The word a call's first arrival makes of a counter from an earlier call.
PKV_HD constexpr uint64_t arrival_floor(uint32_t generation) { return uint64_t(generation) << 32; }

// Tiles counted by the call that last wrote the word.
PKV_HD constexpr uint32_t arrival_count(uint64_t word) { return uint32_t(word & 0xffffffffu); }

// Generation of the call that last wrote the word.
PKV_HD constexpr uint32_t arrival_generation(uint64_t word) { return uint32_t(word >> 32); }

// The generation after `g`: generations are never 0 (the value of a fresh, zeroed word).
PKV_HD constexpr uint32_t next_generation(uint32_t g) { return g + 1 == 0 ? 1 : g + 1; }

// Host model of one arrival on `word` (the device does the same two steps atomically): returns
// the tiles this call had counted before, and leaves the word as the device leaves it.
inline uint32_t arrive_on_host(uint64_t& word, uint32_t generation, uint32_t tiles) {
  const uint64_t f = arrival_floor(generation);
  if (word < f) word = f;
  const uint64_t old = word;
  word += tiles;
  return arrival_count(old);
}

}  // namespace pkv
