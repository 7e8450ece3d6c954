// C ABI of the continuous-batching scheduler (policy in pkv.h).
#include <algorithm>
#include <new>
#include <vector>

#include "common.h"
#include "scheduler.h"

struct pkv_scheduler {
  pkv::Scheduler impl;
};

using pkv::fail;
using pkv::ok;

extern "C" {

int32_t pkv_scheduler_create(int32_t num_blocks, int32_t block_size,
                             const int32_t* init_free_order, int32_t max_num_seqs,
                             int32_t max_num_batched_tokens, int32_t chunk_size,
                             int32_t reserve_tokens, int32_t host_blocks,
                             pkv_scheduler** out) {
  if (!out) return fail(PKV_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || max_num_seqs <= 0 || max_num_batched_tokens <= 0 ||
      chunk_size <= 0 || reserve_tokens < 0 || host_blocks < 0)
    return fail(PKV_ERR_INVALID,
                "sizes must be positive (num_blocks %d, block_size %d, max_num_seqs %d, "
                "max_num_batched_tokens %d, chunk_size %d), reserve_tokens (%d) and "
                "host_blocks (%d) >= 0",
                num_blocks, block_size, max_num_seqs, max_num_batched_tokens, chunk_size,
                reserve_tokens, host_blocks);
  if (int64_t(num_blocks) * block_size >= (int64_t(1) << 31))
    return fail(PKV_ERR_INVALID, "num_blocks * block_size must be below 2^31");
  std::vector<int32_t> order(num_blocks);
  if (init_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = init_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b])
        return fail(PKV_ERR_INVALID, "init_free_order is not a permutation of 0..%d",
                    num_blocks - 1);
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  }
  pkv::SchedulerConfig cfg{num_blocks, block_size, max_num_seqs, max_num_batched_tokens,
                           chunk_size, reserve_tokens, host_blocks};
  auto* s = new (std::nothrow) pkv_scheduler{pkv::Scheduler(cfg, order)};
  if (!s) return fail(PKV_ERR_INVALID, "out of host memory");
  *out = s;
  return ok();
}

void pkv_scheduler_destroy(pkv_scheduler* s) { delete s; }

int32_t pkv_scheduler_add_request(pkv_scheduler* s, int64_t id, int32_t prompt_len,
                                  int32_t output_len) {
  if (!s) return fail(PKV_ERR_INVALID, "scheduler is NULL");
  return s->impl.add_request(id, prompt_len, output_len);
}

int32_t pkv_scheduler_max_blocks(const pkv_scheduler* s, int32_t* out) {
  if (!s || !out) return fail(PKV_ERR_INVALID, "NULL argument");
  *out = s->impl.max_blocks_needed();
  return ok();
}

int32_t pkv_scheduler_step(pkv_scheduler* s, int32_t max_rows, int32_t max_tokens,
                           int32_t max_blocks, int64_t* seq_ids, int32_t* query_lens,
                           int32_t* context_lens, int32_t* slots, int32_t* block_tables,
                           int32_t* num_decode, int32_t* num_rows, int32_t* num_tokens) {
  if (!s) return fail(PKV_ERR_INVALID, "scheduler is NULL");
  if (!seq_ids || !query_lens || !context_lens || !slots || !block_tables || !num_decode ||
      !num_rows || !num_tokens)
    return fail(PKV_ERR_INVALID, "NULL argument");
  const pkv::SchedulerConfig& c = s->impl.config();
  const int32_t width = s->impl.max_blocks_needed();
  if (max_rows < c.max_num_seqs || max_tokens < c.max_num_batched_tokens || max_blocks < width)
    return fail(PKV_ERR_BUFFER_TOO_SMALL,
                "need max_rows >= %d, max_tokens >= %d, max_blocks >= %d (got %d, %d, %d)",
                c.max_num_seqs, c.max_num_batched_tokens, width, max_rows, max_tokens,
                max_blocks);
  s->impl.step();
  const auto& rows = s->impl.rows();
  const auto& alloc = s->impl.allocator();
  for (size_t i = 0; i < rows.size(); ++i) {
    seq_ids[i] = rows[i].id;
    query_lens[i] = rows[i].query_len;
    context_lens[i] = rows[i].context_len;
    const auto& t = alloc.table(rows[i].id);
    int32_t* row = block_tables + int64_t(i) * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j)
      row[j] = j < static_cast<int32_t>(t.size()) ? t[j] : -1;
  }
  std::copy(s->impl.slots().begin(), s->impl.slots().end(), slots);
  *num_decode = s->impl.num_decode();
  *num_rows = static_cast<int32_t>(rows.size());
  *num_tokens = static_cast<int32_t>(s->impl.slots().size());
  return ok();
}

int32_t pkv_scheduler_last_events(const pkv_scheduler* s, int64_t* finished,
                                  int32_t finished_cap, int32_t* num_finished,
                                  int64_t* preempted, int32_t preempted_cap,
                                  int32_t* num_preempted) {
  if (!s || !num_finished || !num_preempted) return fail(PKV_ERR_INVALID, "NULL argument");
  const auto& f = s->impl.finished();
  const auto& p = s->impl.preempted();
  *num_finished = static_cast<int32_t>(f.size());
  *num_preempted = static_cast<int32_t>(p.size());
  if (int64_t(f.size()) > finished_cap || int64_t(p.size()) > preempted_cap)
    return fail(PKV_ERR_BUFFER_TOO_SMALL, "%zu finished and %zu preempted requests", f.size(),
                p.size());
  if ((!f.empty() && !finished) || (!p.empty() && !preempted))
    return fail(PKV_ERR_INVALID, "NULL argument");
  std::copy(f.begin(), f.end(), finished);
  std::copy(p.begin(), p.end(), preempted);
  return ok();
}

int32_t pkv_scheduler_last_swaps(const pkv_scheduler* s, int32_t* in_host, int32_t* in_device,
                                 int32_t in_cap, int32_t* num_in, int32_t* out_device,
                                 int32_t* out_host, int32_t out_cap, int32_t* num_out) {
  if (!s || !num_in || !num_out) return fail(PKV_ERR_INVALID, "NULL argument");
  const auto& a = s->impl.swap_in_pairs();
  const auto& b = s->impl.swap_out_pairs();
  *num_in = static_cast<int32_t>(a.size());
  *num_out = static_cast<int32_t>(b.size());
  if (int64_t(a.size()) > in_cap || int64_t(b.size()) > out_cap)
    return fail(PKV_ERR_BUFFER_TOO_SMALL, "%zu swap-in and %zu swap-out pairs", a.size(),
                b.size());
  if ((!a.empty() && (!in_host || !in_device)) || (!b.empty() && (!out_device || !out_host)))
    return fail(PKV_ERR_INVALID, "NULL argument");
  for (size_t i = 0; i < a.size(); ++i) {
    in_host[i] = a[i].src;
    in_device[i] = a[i].dst;
  }
  for (size_t i = 0; i < b.size(); ++i) {
    out_device[i] = b[i].src;
    out_host[i] = b[i].dst;
  }
  return ok();
}

int32_t pkv_scheduler_stats(const pkv_scheduler* s, int64_t* out) {
  if (!s || !out) return fail(PKV_ERR_INVALID, "NULL argument");
  const pkv::Scheduler& k = s->impl;
  out[0] = k.steps();
  out[1] = k.running();
  out[2] = k.waiting();
  out[3] = k.total_finished();
  out[4] = k.total_preempted();
  out[5] = k.cached_tokens();
  out[6] = k.allocated_slots();
  out[7] = k.reserved_slots();
  out[8] = k.allocator().num_free();
  out[9] = k.total_swapped_out();
  out[10] = k.total_swapped_in();
  return ok();
}

}  // extern "C"
