#include "slot_table.h"

namespace kvc {

SlotTable::SlotTable(int window, int n_sink) : window_(window), n_sink_(n_sink) { reset(); }

void SlotTable::reset() {
  slots_.assign(n_sink_ + window_, -1);
  fifo_.clear();
  next_id_ = 0;
  last_window_slot_ = n_sink_ + window_ - 1;  // so the first window chunk lands in slot n_sink
}

int SlotTable::occupancy() const {
  int n = 0;
  for (int64_t c : slots_) n += c >= 0;
  return n;
}

void SlotTable::plan_append(int* slot, int64_t* evicted) const {
  if (next_id_ < n_sink_) {  // the first chunks become the sink
    *slot = static_cast<int>(next_id_);
    *evicted = -1;
    return;
  }
  // The ring slot after the last written one holds the oldest window chunk, if any.
  int s = n_sink_ + (last_window_slot_ + 1 - n_sink_) % window_;
  *slot = s;
  *evicted = slots_[s];
}

void SlotTable::commit_append(int slot) {
  if (slot >= n_sink_) {
    if (slots_[slot] >= 0) fifo_.pop_front();  // the evicted chunk is the oldest one
    fifo_.push_back(next_id_);
    last_window_slot_ = slot;
  }
  slots_[slot] = next_id_;
  ++next_id_;
}

void SlotTable::evict(int n, int64_t* ids) {
  for (int i = 0; i < n; ++i) {
    int64_t c = fifo_.front();
    fifo_.pop_front();
    if (ids) ids[i] = c;
    for (auto& s : slots_)
      if (s == c) s = -1;
  }
}

std::vector<Segment> SlotTable::segments(int chunk_tokens, int cond_len, bool merge, int cond_rows) const {
  std::vector<Segment> out;
  if (cond_rows < 0 || cond_rows > cond_len) cond_rows = cond_len;
  if (cond_rows > 0) out.push_back({0, cond_rows, -1});
  for (int s = 0; s < n_slots(); ++s) {
    if (slots_[s] < 0) continue;
    const int32_t row0 = slot_row0(s, chunk_tokens, cond_len);
    if (merge && !out.empty() && out.back().row0 + out.back().len == row0) {
      out.back().len += chunk_tokens;
    } else {
      out.push_back({row0, chunk_tokens, static_cast<int32_t>(slots_[s])});
    }
  }
  return out;
}

}  // namespace kvc
