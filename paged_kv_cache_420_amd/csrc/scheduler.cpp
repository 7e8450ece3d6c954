// Continuous-batching step scheduler (see scheduler.h for the sources and
// pkv.h, pkv_scheduler_step, for the policy).
#include "scheduler.h"

#include <algorithm>

#include "common.h"

namespace pkv {

namespace {
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

Scheduler::Scheduler(const SchedulerConfig& cfg, const std::vector<int32_t>& order)
    : cfg_(cfg), alloc_(cfg.num_blocks, cfg.block_size, order) {
  alloc_.set_host_pool(cfg.host_blocks);
}

int32_t Scheduler::reserve_blocks() const {
  return static_cast<int32_t>(cdiv(cfg_.reserve_tokens, cfg_.block_size));
}

int32_t Scheduler::add_request(int64_t id, int32_t prompt, int32_t output) {
  if (prompt < 1 || output < 1)
    return fail(PKV_ERR_INVALID, "prompt (%d) and output (%d) lengths must be positive", prompt,
                output);
  const int64_t total = int64_t(prompt) + output;
  if (cdiv(total, cfg_.block_size) > cfg_.num_blocks)
    return fail(PKV_ERR_INVALID, "a request of %lld tokens never fits the pool",
                static_cast<long long>(total));
  if (cfg_.reserve_tokens > 0 && total > cfg_.reserve_tokens)
    return fail(PKV_ERR_INVALID, "a request of %lld tokens exceeds the reservation of %d",
                static_cast<long long>(total), cfg_.reserve_tokens);
  if (alloc_.has(id)) return fail(PKV_ERR_SEQ_EXISTS, "request %lld is running",
                                  static_cast<long long>(id));
  for (const Request& r : waiting_)
    if (r.id == id)
      return fail(PKV_ERR_SEQ_EXISTS, "request %lld is waiting", static_cast<long long>(id));
  waiting_.push_back(Request{id, prompt, output});
  return ok();
}

bool Scheduler::admissible(const Request& r) const {
  const int32_t run = running();
  if (run >= cfg_.max_num_seqs) return false;
  if (cfg_.reserve_tokens > 0)
    return int64_t(run + 1) * reserve_blocks() <= cfg_.num_blocks;
  // blocks for its whole prompt, plus the prompt blocks the running
  // requests still have to take, plus one per running request (what their
  // next decode rows may take)
  // (a swapped-out request needs its blocks back instead of its prompt's)
  int64_t need = (r.swapped ? int64_t(alloc_.table(r.id).size())
                            : cdiv(r.prompt, cfg_.block_size)) + run;
  for (const Request& x : running_)
    if (x.prefilled < x.prompt)
      need += cdiv(x.prompt, cfg_.block_size) - int64_t(alloc_.table(x.id).size());
  return alloc_.num_free() >= need;
}

int32_t Scheduler::preempt_youngest(int32_t min_index) {
  for (int32_t j = running() - 1; j >= min_index; --j) {
    if (has_row_[j]) continue;
    Request v = running_[j];
    if (cfg_.host_blocks > 0 &&
        int64_t(alloc_.table(v.id).size()) <= alloc_.num_free_host()) {
      alloc_.swap_out(v.id, &swap_out_);
      v.swapped = true;
      ++total_swap_out_;
    } else {
      alloc_.release(v.id);
      // recompute: the tokens it generated become part of what it prefills
      v.prompt += v.generated;
      v.output -= v.generated;
      v.prefilled = 0;
      v.generated = 0;
    }
    running_.erase(running_.begin() + j);
    has_row_.erase(has_row_.begin() + j);
    waiting_.push_front(v);
    preempted_.push_back(v.id);
    ++total_preempted_;
    return j;
  }
  return -1;
}

int32_t Scheduler::max_blocks_needed() const {
  int64_t m = 1;
  for (const Request& r : running_)
    m = std::max(m, cdiv(int64_t(r.prompt) + r.output, cfg_.block_size));
  for (const Request& r : waiting_)
    m = std::max(m, cdiv(int64_t(r.prompt) + r.output, cfg_.block_size));
  return static_cast<int32_t>(m);
}

void Scheduler::step() {
  rows_.clear();
  slots_.clear();
  finished_.clear();
  preempted_.clear();
  swap_in_.clear();
  swap_out_.clear();
  num_decode_ = 0;
  ++steps_;

  // 1. requests that have produced all their tokens leave; their blocks go
  //    back to the pool at once
  std::vector<Request> keep;
  keep.reserve(running_.size());
  for (const Request& r : running_) {
    if (r.generated == r.output) {
      alloc_.release(r.id);
      finished_.push_back(r.id);
      ++total_finished_;
    } else {
      keep.push_back(r);
    }
  }
  running_.swap(keep);

  // 2. waiting requests join, first come first served
  while (!waiting_.empty() && admissible(waiting_.front())) {
    Request r = waiting_.front();
    waiting_.pop_front();
    if (r.swapped) {
      alloc_.swap_in(r.id, &swap_in_);
      r.swapped = false;
      ++total_swap_in_;
    } else {
      alloc_.add(r.id);
    }
    running_.push_back(r);
  }
  has_row_.assign(running_.size(), false);
  int32_t budget = cfg_.max_num_batched_tokens;

  // 3. one decode row per request past its prompt, oldest first; when the
  //    pool is out of blocks the youngest request without a row is
  //    preempted (possibly this one)
  for (int32_t i = 0; i < running() && budget > 0; ++i) {
    if (running_[i].prefilled < running_[i].prompt) continue;
    bool self = false;
    while (alloc_.blocks_for_append(running_[i].id, 1) > alloc_.num_free()) {
      const int32_t v = preempt_youngest(i);
      if (v == i) {
        self = true;
        break;
      }
    }
    if (self) break;  // it was the youngest: nothing follows it
    Request& r = running_[i];
    int32_t slot = 0;
    alloc_.append(r.id, 1, &slot, &cow_);
    ++r.generated;
    rows_.push_back(PlanRow{r.id, 1, alloc_.length(r.id)});
    slots_.push_back(slot);
    has_row_[i] = true;
    --budget;
  }
  num_decode_ = static_cast<int32_t>(rows_.size());

  // 4. prompt chunks, oldest first, within the step's token budget; a chunk
  //    may preempt younger requests without a row, never older ones
  for (int32_t i = 0; i < running() && budget > 0; ++i) {
    if (running_[i].prefilled >= running_[i].prompt) continue;
    const int32_t c = std::min({running_[i].prompt - running_[i].prefilled,
                                cfg_.chunk_size, budget});
    bool placed = true;
    while (alloc_.blocks_for_append(running_[i].id, c) > alloc_.num_free()) {
      if (preempt_youngest(i + 1) < 0) {
        placed = false;
        break;
      }
    }
    if (!placed) break;  // later requests wait for blocks too
    Request& r = running_[i];
    const size_t at = slots_.size();
    slots_.resize(at + c);
    alloc_.append(r.id, c, slots_.data() + at, &cow_);
    r.prefilled += c;
    rows_.push_back(PlanRow{r.id, c, alloc_.length(r.id)});
    has_row_[i] = true;
    budget -= c;
  }
}

int64_t Scheduler::cached_tokens() const {
  int64_t n = 0;
  for (const Request& r : running_) n += alloc_.length(r.id);
  return n;
}

int64_t Scheduler::allocated_slots() const {
  int64_t n = 0;
  for (const Request& r : running_) n += int64_t(alloc_.table(r.id).size()) * cfg_.block_size;
  return n;
}

int64_t Scheduler::reserved_slots() const {
  if (cfg_.reserve_tokens > 0) return int64_t(running()) * reserve_blocks() * cfg_.block_size;
  return allocated_slots();
}

}  // namespace pkv
