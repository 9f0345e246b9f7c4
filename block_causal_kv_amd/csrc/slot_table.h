// Host bookkeeping of the bounded KV cache: which chunk sits in which slot,
// FIFO eviction of window chunks, and the list of key segments a query of the
// next chunk attends to.  Pure C++ (no HIP), so it can be tested on a CPU.
//
// The cache is the "global sink + sliding local window" of the JoyAI-Video-Edit
// tutorial (agifrontier.github.io), section "Hardware-software co-deployment",
// bullet "constant KV cache": slots [0, n_sink) hold the first chunks for good,
// slots [n_sink, n_sink + W) form a ring of the W most recent chunks.
#pragma once
#include <cstdint>
#include <deque>
#include <vector>

namespace kvc {

struct Segment {
  int32_t row0;  // first pool row (rows [0, Lc) condition, slot s at slot_row0(s, T, Lc))
  int32_t len;   // rows
  int32_t chunk; // chunk id held in the first slot of the run (-1: condition only)
};

class SlotTable {
 public:
  SlotTable(int window, int n_sink);
  int window() const { return window_; }
  int n_sink() const { return n_sink_; }
  int n_slots() const { return n_sink_ + window_; }
  int64_t next_chunk_id() const { return next_id_; }
  int occupancy() const;
  int window_count() const { return static_cast<int>(fifo_.size()); }
  int64_t slot_chunk(int s) const { return slots_[s]; }

  // Slot the next appended chunk will take, and the chunk it will evict (-1 if none).
  void plan_append(int* slot, int64_t* evicted) const;
  // Commit an append planned with plan_append.
  void commit_append(int slot);
  // Remove the n oldest window chunks (n <= window_count()); ids oldest first.
  void evict(int n, int64_t* ids);
  void reset();

  // Key segments (in pool rows) visible to a query of the next chunk: the
  // condition rows and every occupied slot.  With merge, physically adjacent
  // runs (condition rows and consecutive occupied slots) become one segment.
  // cond_rows (<= cond_len, or -1 for all) is the number of condition rows in
  // use: the layout is fixed by cond_len, a shorter condition leaves the rest
  // of its block unused.
  std::vector<Segment> segments(int chunk_tokens, int cond_len, bool merge, int cond_rows = -1) const;

  // Pool layout: the condition rows, then one slot of T rows per chunk; the
  // condition block and every slot start on a multiple of 8 rows (the rows in
  // between are padding), so 8-row pieces of a slot are 16-byte aligned in a
  // transposed bf16 pool.
  static int32_t round8(int32_t x) { return (x + 7) & ~7; }
  static int32_t slot_row0(int slot, int chunk_tokens, int cond_len) {
    return round8(cond_len) + slot * round8(chunk_tokens);
  }

 private:
  int window_, n_sink_;
  std::vector<int64_t> slots_;  // slot -> chunk id, -1 empty
  std::deque<int64_t> fifo_;    // window chunks, oldest first
  int64_t next_id_;
  int last_window_slot_;
};

}  // namespace kvc
