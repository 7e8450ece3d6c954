// Continuous-batching step scheduler over the block allocator.
//
// Mechanism: "vLLM 初探" tutorial §1.3 (requests join and leave the batch
// at any step; a finished request frees its memory at once for a waiting
// one) and §1.5 (dynamic scheduling against static batches); explainer
// (openEuler/CSDN), continuous-batching section (at every decode step the
// finished requests leave and waiting ones are pulled in) and its
// over-reservation section (a naive engine reserves the longest possible
// reply, e.g. 2000 tokens, per request); KV-cache article §3.2 (the
// max_num_seqs limit) and §4.1/§4.2 (prompts in chunks of 512 tokens).
// The pages give no policy beyond that; the one here is the library's own
// and is spelled out in pkv.h (pkv_scheduler_step).
#pragma once

#include <cstdint>
#include <deque>
#include <vector>

#include "allocator.h"

namespace pkv {

struct SchedulerConfig {
  int32_t num_blocks;
  int32_t block_size;
  int32_t max_num_seqs;
  int32_t max_num_batched_tokens;
  int32_t chunk_size;
  int32_t reserve_tokens;  // 0: admit on free blocks; > 0: reservation model
  int32_t host_blocks;     // swap space for preempted requests (0: recompute only)
};

struct Request {
  int64_t id;
  int32_t prompt;     // tokens to prefill (grows by the generated tokens on preemption)
  int32_t output;     // decode steps still to run before the request finishes
  int32_t prefilled = 0;
  int32_t generated = 0;
  bool swapped = false;  // its blocks are in the host tier
};

// One scheduled row: a decode row (1 token) or a prefill chunk.
struct PlanRow {
  int64_t id;
  int32_t query_len;
  int32_t context_len;  // cached tokens after this step's appends
};

class Scheduler {
 public:
  Scheduler(const SchedulerConfig& cfg, const std::vector<int32_t>& order);

  const SchedulerConfig& config() const { return cfg_; }
  const BlockAllocator& allocator() const { return alloc_; }

  int32_t add_request(int64_t id, int32_t prompt, int32_t output);

  // Plans one step (retire, admit, decode rows, prefill chunks) and applies
  // it to the allocator.  Results are in the accessors below until the
  // next call.
  void step();
  // Largest table length any current request can reach: the block_tables
  // width a caller needs for the next step.
  int32_t max_blocks_needed() const;

  const std::vector<PlanRow>& rows() const { return rows_; }
  int32_t num_decode() const { return num_decode_; }
  const std::vector<int32_t>& slots() const { return slots_; }
  const std::vector<int64_t>& finished() const { return finished_; }
  const std::vector<int64_t>& preempted() const { return preempted_; }
  // This step's block moves: host -> device (swap-ins at admission) and
  // device -> host (swap-outs of preempted requests).
  const std::vector<CowPair>& swap_in_pairs() const { return swap_in_; }
  const std::vector<CowPair>& swap_out_pairs() const { return swap_out_; }
  int64_t total_swapped_out() const { return total_swap_out_; }
  int64_t total_swapped_in() const { return total_swap_in_; }

  int32_t running() const { return static_cast<int32_t>(running_.size()); }
  int32_t waiting() const { return static_cast<int32_t>(waiting_.size()); }
  int64_t total_finished() const { return total_finished_; }
  int64_t total_preempted() const { return total_preempted_; }
  int64_t steps() const { return steps_; }
  int64_t cached_tokens() const;
  int64_t allocated_slots() const;
  int64_t reserved_slots() const;

 private:
  int32_t reserve_blocks() const;
  bool admissible(const Request& r) const;
  // Preempts the youngest running request at index >= min_index that has
  // no row in this step -- to the host tier if it has room (progress
  // kept), else by recompute (blocks freed, its generated tokens join its
  // prompt) -- and puts it at the front of the waiting queue; returns its
  // index in running_ or -1.
  int32_t preempt_youngest(int32_t min_index);

  SchedulerConfig cfg_;
  BlockAllocator alloc_;
  std::deque<Request> waiting_;
  std::vector<Request> running_;   // admission order, oldest first
  std::vector<bool> has_row_;      // per running_ entry, this step
  std::vector<PlanRow> rows_;
  std::vector<int32_t> slots_;
  std::vector<int64_t> finished_, preempted_;
  std::vector<CowPair> cow_;       // stays empty: requests never share blocks
  std::vector<CowPair> swap_in_, swap_out_;
  int64_t total_swap_out_ = 0, total_swap_in_ = 0;
  int32_t num_decode_ = 0;
  int64_t total_finished_ = 0, total_preempted_ = 0, steps_ = 0;
};

}  // namespace pkv
