// Host block allocator (see allocator.h for the contract and sources).
#include "allocator.h"

#include <algorithm>
#include <utility>

#include "common.h"

namespace pkv {

namespace {
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

BlockAllocator::BlockAllocator(int32_t num_blocks, int32_t block_size,
                               const std::vector<int32_t>& order)
    : num_blocks_(num_blocks),
      block_size_(block_size),
      free_(order.rbegin(), order.rend()),
      ref_(num_blocks, 0) {}

void BlockAllocator::free_stack(int32_t* out) const {
  int32_t i = 0;
  for (auto it = free_.rbegin(); it != free_.rend(); ++it) out[i++] = *it;
}

int32_t BlockAllocator::pop() {
  int32_t b = free_.back();
  free_.pop_back();
  ref_[b] = 1;
  return b;
}

int32_t BlockAllocator::add(int64_t seq) {
  if (has(seq))
    return fail(PKV_ERR_SEQ_EXISTS, "sequence %lld already exists",
                static_cast<long long>(seq));
  seqs_.emplace(seq, Seq{});
  return ok();
}

int32_t BlockAllocator::release(int64_t seq) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end())
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld",
                static_cast<long long>(seq));
  // Logical order: a block reaching zero goes on top of the free stack.
  if (it->second.swapped) {
    for (int32_t h : it->second.table) {
      host_ref_[h] = 0;
      host_free_.push_back(h);
    }
  } else {
    for (int32_t b : it->second.table)
      if (--ref_[b] == 0) free_.push_back(b);
  }
  seqs_.erase(it);
  return ok();
}

int32_t BlockAllocator::set_host_pool(int32_t num_host_blocks) {
  if (num_host_blocks < 0) return fail(PKV_ERR_INVALID, "negative host pool size");
  for (const auto& kv : seqs_)
    if (kv.second.swapped)
      return fail(PKV_ERR_INVALID, "sequences are swapped out; the host pool is in use");
  host_ref_.assign(num_host_blocks, 0);
  host_free_.clear();
  for (int32_t h = num_host_blocks - 1; h >= 0; --h) host_free_.push_back(h);
  return ok();
}

void BlockAllocator::host_free_stack(int32_t* out) const {
  int32_t i = 0;
  for (auto it = host_free_.rbegin(); it != host_free_.rend(); ++it) out[i++] = *it;
}

int32_t BlockAllocator::swap_out(int64_t seq, std::vector<CowPair>* pairs) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end())
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", static_cast<long long>(seq));
  Seq& s = it->second;
  if (s.swapped)
    return fail(PKV_ERR_INVALID, "sequence %lld is already swapped out",
                static_cast<long long>(seq));
  if (s.table.size() > host_free_.size())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "need %zu host blocks, %zu free", s.table.size(),
                host_free_.size());
  for (int32_t& b : s.table) {
    const int32_t h = host_free_.back();
    host_free_.pop_back();
    host_ref_[h] = 1;
    pairs->push_back({b, h});
    if (--ref_[b] == 0) free_.push_back(b);
    b = h;
  }
  s.swapped = true;
  return ok();
}

int32_t BlockAllocator::swap_in(int64_t seq, std::vector<CowPair>* pairs) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end())
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", static_cast<long long>(seq));
  Seq& s = it->second;
  if (!s.swapped)
    return fail(PKV_ERR_INVALID, "sequence %lld is not swapped out",
                static_cast<long long>(seq));
  if (int64_t(s.table.size()) > num_free())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "need %zu blocks, %d free", s.table.size(), num_free());
  for (int32_t& h : s.table) {
    const int32_t b = pop();
    pairs->push_back({h, b});
    host_ref_[h] = 0;
    host_free_.push_back(h);
    h = b;
  }
  s.swapped = false;
  return ok();
}

int32_t BlockAllocator::fork(int64_t parent, int64_t child) {
  auto it = seqs_.find(parent);
  if (it == seqs_.end())
    return fail(PKV_ERR_NO_SUCH_SEQ, "no parent sequence %lld",
                static_cast<long long>(parent));
  if (has(child))
    return fail(PKV_ERR_SEQ_EXISTS, "child sequence %lld already exists",
                static_cast<long long>(child));
  if (it->second.swapped)
    return fail(PKV_ERR_INVALID, "sequence %lld is swapped out", static_cast<long long>(parent));
  Seq copy = it->second;
  for (int32_t b : copy.table) ++ref_[b];
  seqs_.emplace(child, std::move(copy));
  return ok();
}

int64_t BlockAllocator::blocks_needed(const Seq& s, int32_t n,
                                      int32_t last_ref, bool* cow) const {
  int64_t fresh = cdiv(int64_t(s.len) + n, block_size_) -
                  cdiv(s.len, block_size_);
  *cow = n > 0 && s.len % block_size_ != 0 && last_ref > 1;
  return fresh + (*cow ? 1 : 0);
}

void BlockAllocator::grow(Seq& s, int32_t n, int32_t* slots,
                          std::vector<CowPair>* cow,
                          std::vector<TableChange>* changes, int32_t row) {
  bool do_cow = false;
  if (n > 0 && s.len % block_size_ != 0) do_cow = ref_[s.table.back()] > 1;
  if (do_cow) {
    int32_t old = s.table.back();
    int32_t fresh = pop();
    --ref_[old];
    s.table.back() = fresh;
    cow->push_back({old, fresh});
    if (changes)
      changes->push_back({row, static_cast<int32_t>(s.table.size()) - 1, fresh});
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t p = s.len + i;
    if (p % block_size_ == 0) {
      s.table.push_back(pop());
      if (changes)
        changes->push_back(
            {row, static_cast<int32_t>(s.table.size()) - 1, s.table.back()});
    }
    slots[i] = s.table[p / block_size_] * block_size_ + p % block_size_;
  }
  s.len += n;
}

int64_t BlockAllocator::blocks_for_append(int64_t seq, int32_t n) const {
  auto it = seqs_.find(seq);
  if (it == seqs_.end()) return -1;
  const Seq& s = it->second;
  if (s.swapped) return -1;
  bool c = false;
  return blocks_needed(s, n, s.table.empty() ? 0 : ref_[s.table.back()], &c);
}

int32_t BlockAllocator::append(int64_t seq, int32_t n, int32_t* slots,
                               std::vector<CowPair>* cow) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end())
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld",
                static_cast<long long>(seq));
  if (n < 0) return fail(PKV_ERR_INVALID, "negative token count %d", n);
  Seq& s = it->second;
  if (s.swapped)
    return fail(PKV_ERR_INVALID, "sequence %lld is swapped out", static_cast<long long>(seq));
  bool c = false;
  int32_t last_ref = s.table.empty() ? 0 : ref_[s.table.back()];
  int64_t need = blocks_needed(s, n, last_ref, &c);
  if (need > num_free())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "need %lld blocks, %d free",
                static_cast<long long>(need), num_free());
  grow(s, n, slots, cow);
  return ok();
}

int32_t BlockAllocator::append_batch(const int64_t* seqs,
                                     const int32_t* counts, int32_t num_seqs,
                                     int32_t* slots, int64_t slots_cap,
                                     CowPair* cow, int32_t cow_cap,
                                     int32_t* n_cow, int32_t max_blocks,
                                     int32_t* tables, int32_t* lens,
                                     TableChange* changes, int32_t changes_cap,
                                     int32_t* n_changes) {
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "negative batch size");
  // One lookup per sequence; scratch reused across calls (one decode step
  // of a large batch should cost microseconds, not allocations).
  thread_local std::vector<Seq*> ptr;
  thread_local std::vector<int64_t> ids;
  thread_local std::vector<std::pair<int32_t, int32_t>> dropped;  // block, refs given up
  ptr.resize(num_seqs);
  ids.assign(seqs, seqs + num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = seqs_.find(seqs[i]);
    if (it == seqs_.end())
      return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld",
                  static_cast<long long>(seqs[i]));
    if (counts[i] < 0)
      return fail(PKV_ERR_INVALID, "negative token count %d", counts[i]);
    if (it->second.swapped)
      return fail(PKV_ERR_INVALID, "sequence %lld is swapped out",
                  static_cast<long long>(seqs[i]));
    ptr[i] = &it->second;
  }
  std::sort(ids.begin(), ids.end());
  for (int32_t i = 1; i < num_seqs; ++i)
    if (ids[i] == ids[i - 1])
      return fail(PKV_ERR_INVALID, "sequence %lld appears twice in a batch",
                  static_cast<long long>(ids[i]));
  // Count the blocks the whole batch needs in batch order: a copy-on-write
  // of one sequence lowers the count of a block other members may share.
  dropped.clear();
  int64_t total_slots = 0, need = 0;
  int32_t cows = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = *ptr[i];
    int32_t last_ref = 0;
    if (!s.table.empty()) {
      const int32_t last = s.table.back();
      last_ref = ref_[last];
      for (const auto& d : dropped)
        if (d.first == last) last_ref -= d.second;
    }
    bool c = false;
    need += blocks_needed(s, counts[i], last_ref, &c);
    if (c) {
      bool found = false;
      for (auto& d : dropped)
        if (d.first == s.table.back()) {
          ++d.second;
          found = true;
        }
      if (!found) dropped.emplace_back(s.table.back(), 1);
      ++cows;
    }
    total_slots += counts[i];
    if (tables &&
        cdiv(int64_t(s.len) + counts[i], block_size_) > int64_t(max_blocks))
      return fail(PKV_ERR_BUFFER_TOO_SMALL,
                  "sequence %lld would hold more than max_blocks %d blocks",
                  static_cast<long long>(seqs[i]), max_blocks);
  }
  if (total_slots > slots_cap)
    return fail(PKV_ERR_BUFFER_TOO_SMALL, "slots buffer holds %lld, need %lld",
                static_cast<long long>(slots_cap),
                static_cast<long long>(total_slots));
  if (cows > cow_cap)
    return fail(PKV_ERR_BUFFER_TOO_SMALL, "cow buffer holds %d, need %d",
                cow_cap, cows);
  if (changes && need > changes_cap)
    return fail(PKV_ERR_BUFFER_TOO_SMALL, "changes buffer holds %d, need %lld",
                changes_cap, static_cast<long long>(need));
  if (need > num_free())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "batch needs %lld blocks, %d free",
                static_cast<long long>(need), num_free());
  thread_local std::vector<CowPair> pairs;
  thread_local std::vector<TableChange> set;
  pairs.clear();
  set.clear();
  int64_t off = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    grow(*ptr[i], counts[i], slots + off, &pairs, changes ? &set : nullptr, i);
    off += counts[i];
  }
  for (size_t k = 0; k < pairs.size(); ++k) cow[k] = pairs[k];
  *n_cow = static_cast<int32_t>(pairs.size());
  if (changes) {
    for (size_t k = 0; k < set.size(); ++k) changes[k] = set[k];
    *n_changes = static_cast<int32_t>(set.size());
    if (lens)
      for (int32_t i = 0; i < num_seqs; ++i) lens[i] = ptr[i]->len;
  }
  if (tables) {
    for (int32_t i = 0; i < num_seqs; ++i) {
      const Seq& s = *ptr[i];
      int32_t* row = tables + int64_t(i) * max_blocks;
      const int32_t nb = static_cast<int32_t>(s.table.size());
      std::copy(s.table.begin(), s.table.end(), row);
      std::fill(row + nb, row + max_blocks, -1);
      if (lens) lens[i] = s.len;
    }
  }
  return ok();
}

}  // namespace pkv
