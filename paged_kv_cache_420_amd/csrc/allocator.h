// Host block allocator: free stack, reference counts, per-sequence tables.
//
// Mechanism: "vLLM 初探" tutorial §1.4 (fixed-size blocks in one pool,
// per-sequence logical page table, shared prefixes); explainer
// (openEuler/CSDN), PagedAttention and memory-sharing sections (blocks on
// demand, immediate release, sharing by pointing tables at the same
// blocks); KV-cache article (intelliparadigm) §2.1 (position p lives in
// table[p / block_size] at row p % block_size).  The orderings (LIFO free
// stack, copy-on-write rule, logical-order release, all-or-nothing failure)
// are the library's own contract, stated in pkv.h.
#pragma once

#include <cstdint>
#include <unordered_map>
#include <vector>

namespace pkv {

struct CowPair {
  int32_t src;
  int32_t dst;
};

// One block-table entry an append set: row of the batch, logical block
// index, physical block (a fresh block, or the copy-on-write replacement of
// the last entry).
struct TableChange {
  int32_t row;
  int32_t index;
  int32_t block;
};

class BlockAllocator {
 public:
  // `order` lists every block once; order[0] is handed out first.
  BlockAllocator(int32_t num_blocks, int32_t block_size,
                 const std::vector<int32_t>& order);

  int32_t num_blocks() const { return num_blocks_; }
  int32_t block_size() const { return block_size_; }
  int32_t num_free() const { return static_cast<int32_t>(free_.size()); }
  int32_t refcount(int32_t b) const { return ref_[b]; }
  bool has(int64_t seq) const { return seqs_.count(seq) != 0; }
  const std::vector<int32_t>& table(int64_t seq) const {
    return seqs_.at(seq).table;
  }
  int32_t length(int64_t seq) const { return seqs_.at(seq).len; }

  // Free blocks, top of the stack first.
  void free_stack(int32_t* out) const;
  const std::vector<int32_t>& refcounts() const { return ref_; }

  // Blocks an append of n tokens to `seq` would take (fresh blocks plus a
  // copy-on-write block), without changing anything; -1 if no such seq.
  int64_t blocks_for_append(int64_t seq, int32_t n) const;

  // Each returns a pkv_status; on failure nothing has changed.
  int32_t add(int64_t seq);
  int32_t release(int64_t seq);
  int32_t fork(int64_t parent, int64_t child);
  // Appends n tokens: slots (n of them) and at most one copy-on-write pair.
  int32_t append(int64_t seq, int32_t n, int32_t* slots,
                 std::vector<CowPair>* cow);
  // All-or-nothing over the batch; capacities checked before any change.
  // With `tables` (and `lens`), the batch's updated block tables are then
  // written as rows of max_blocks entries (-1 past each table's end) and
  // its lengths; a table longer than max_blocks fails up front.
  // With `changes`, every table entry the batch sets is reported instead
  // (capacity changes_cap, checked up front), plus the lengths in `lens`.
  // Host tier (swap space): num_host_blocks blocks in a second pool with
  // its own free stack (0 on top).  A swapped-out sequence keeps its
  // length and a table of host blocks; it cannot grow, fork or be read by
  // the device calls until it is swapped back in.
  int32_t set_host_pool(int32_t num_host_blocks);
  int32_t num_host_blocks() const { return static_cast<int32_t>(host_ref_.size()); }
  int32_t num_free_host() const { return static_cast<int32_t>(host_free_.size()); }
  bool swapped(int64_t seq) const {
    auto it = seqs_.find(seq);
    return it != seqs_.end() && it->second.swapped;
  }
  void host_free_stack(int32_t* out) const;
  // Moves every block of `seq` to the host tier: pairs (device block, host
  // block) in logical order; device blocks are released as by release().
  int32_t swap_out(int64_t seq, std::vector<CowPair>* pairs);
  // Back to fresh device blocks: pairs (host block, device block).
  int32_t swap_in(int64_t seq, std::vector<CowPair>* pairs);
  int32_t append_batch(const int64_t* seqs, const int32_t* counts,
                       int32_t num_seqs, int32_t* slots, int64_t slots_cap,
                       CowPair* cow, int32_t cow_cap, int32_t* n_cow,
                       int32_t max_blocks = 0, int32_t* tables = nullptr,
                       int32_t* lens = nullptr, TableChange* changes = nullptr,
                       int32_t changes_cap = 0, int32_t* n_changes = nullptr);

 private:
  struct Seq {
    std::vector<int32_t> table;  // device blocks, or host blocks when swapped
    int32_t len = 0;
    bool swapped = false;
  };
  // Blocks `seq` needs to grow by n, given `last_ref` as the current count
  // of its last block; sets *cow when a copy-on-write happens first.
  int64_t blocks_needed(const Seq& s, int32_t n, int32_t last_ref,
                        bool* cow) const;
  void grow(Seq& s, int32_t n, int32_t* slots, std::vector<CowPair>* cow,
            std::vector<TableChange>* changes = nullptr, int32_t row = 0);
  int32_t pop();

  int32_t num_blocks_;
  int32_t block_size_;
  std::vector<int32_t> free_;  // stack; top is free_.back()
  std::vector<int32_t> ref_;
  std::vector<int32_t> host_free_;  // stack; top is host_free_.back()
  std::vector<char> host_ref_;      // 1 while a swapped sequence holds it
  std::unordered_map<int64_t, Seq> seqs_;
};

}  // namespace pkv
