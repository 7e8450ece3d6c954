// Host half of the C ABI: error text, version, allocator entry points.
#include <cstdio>
#include <new>
#include <string>
#include <vector>

#include "allocator.h"
#include "common.h"

namespace pkv {

namespace {
thread_local std::string g_last_error;
}

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return PKV_OK;
}

}  // namespace pkv

struct pkv_allocator {
  pkv::BlockAllocator impl;
};

using pkv::fail;
using pkv::ok;

#define PKV_REQUIRE(cond, ...) \
  do {                         \
    if (!(cond)) return fail(PKV_ERR_INVALID, __VA_ARGS__); \
  } while (0)

extern "C" {

const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }

const char* pkv_version(void) { return "0.1.0"; }

int32_t pkv_allocator_create(int32_t num_blocks, int32_t block_size,
                             const int32_t* init_free_order,
                             pkv_allocator** out) {
  PKV_REQUIRE(out != nullptr, "out is NULL");
  *out = nullptr;
  PKV_REQUIRE(num_blocks > 0 && block_size > 0,
              "num_blocks (%d) and block_size (%d) must be positive",
              num_blocks, block_size);
  PKV_REQUIRE(int64_t(num_blocks) * block_size < (int64_t(1) << 31),
              "num_blocks * block_size must be below 2^31");
  std::vector<int32_t> order(num_blocks);
  if (init_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = init_free_order[i];
      PKV_REQUIRE(b >= 0 && b < num_blocks && !seen[b],
                  "init_free_order is not a permutation of 0..%d",
                  num_blocks - 1);
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  }
  auto* a = new (std::nothrow) pkv_allocator{
      pkv::BlockAllocator(num_blocks, block_size, order)};
  if (!a) return fail(PKV_ERR_INVALID, "out of host memory");
  *out = a;
  return ok();
}

void pkv_allocator_destroy(pkv_allocator* alloc) { delete alloc; }

int32_t pkv_seq_add(pkv_allocator* alloc, int64_t seq) {
  PKV_REQUIRE(alloc, "allocator is NULL");
  return alloc->impl.add(seq);
}

int32_t pkv_seq_free(pkv_allocator* alloc, int64_t seq) {
  PKV_REQUIRE(alloc, "allocator is NULL");
  return alloc->impl.release(seq);
}

int32_t pkv_seq_fork(pkv_allocator* alloc, int64_t parent, int64_t child) {
  PKV_REQUIRE(alloc, "allocator is NULL");
  return alloc->impl.fork(parent, child);
}

int32_t pkv_allocator_set_host_pool(pkv_allocator* alloc, int32_t num_host_blocks) {
  PKV_REQUIRE(alloc, "allocator is NULL");
  return alloc->impl.set_host_pool(num_host_blocks);
}

int32_t pkv_num_free_host_blocks(const pkv_allocator* alloc, int32_t* out) {
  PKV_REQUIRE(alloc && out, "NULL argument");
  *out = alloc->impl.num_free_host();
  return ok();
}

int32_t pkv_seq_is_swapped(const pkv_allocator* alloc, int64_t seq, int32_t* out) {
  PKV_REQUIRE(alloc && out, "NULL argument");
  if (!alloc->impl.has(seq))
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", static_cast<long long>(seq));
  *out = alloc->impl.swapped(seq) ? 1 : 0;
  return ok();
}

static int32_t swap_call(pkv_allocator* alloc, int64_t seq, int32_t* src_blocks,
                         int32_t* dst_blocks, int32_t cap, int32_t* n, bool out) {
  PKV_REQUIRE(alloc && n, "NULL argument");
  if (!alloc->impl.has(seq))
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", static_cast<long long>(seq));
  const size_t need = alloc->impl.table(seq).size();
  if (int64_t(need) > cap)
    return fail(PKV_ERR_BUFFER_TOO_SMALL, "sequence holds %zu blocks, capacity %d", need, cap);
  PKV_REQUIRE(need == 0 || (src_blocks && dst_blocks), "NULL argument");
  thread_local std::vector<pkv::CowPair> pairs;
  pairs.clear();
  int32_t st = out ? alloc->impl.swap_out(seq, &pairs) : alloc->impl.swap_in(seq, &pairs);
  if (st != PKV_OK) return st;
  for (size_t i = 0; i < pairs.size(); ++i) {
    src_blocks[i] = pairs[i].src;
    dst_blocks[i] = pairs[i].dst;
  }
  *n = static_cast<int32_t>(pairs.size());
  return ok();
}

int32_t pkv_seq_swap_out(pkv_allocator* alloc, int64_t seq, int32_t* device_blocks,
                         int32_t* host_blocks, int32_t cap, int32_t* n) {
  return swap_call(alloc, seq, device_blocks, host_blocks, cap, n, true);
}

int32_t pkv_seq_swap_in(pkv_allocator* alloc, int64_t seq, int32_t* host_blocks,
                        int32_t* device_blocks, int32_t cap, int32_t* n) {
  return swap_call(alloc, seq, host_blocks, device_blocks, cap, n, false);
}

int32_t pkv_allocator_host_snapshot(const pkv_allocator* alloc, int32_t* host_free_stack,
                                    int32_t* n_free) {
  PKV_REQUIRE(alloc && n_free, "NULL argument");
  *n_free = alloc->impl.num_free_host();
  PKV_REQUIRE(*n_free == 0 || host_free_stack, "host_free_stack is NULL");
  alloc->impl.host_free_stack(host_free_stack);
  return ok();
}

int32_t pkv_seq_append(pkv_allocator* alloc, int64_t seq, int32_t n,
                       int32_t* slots_out, int32_t* cow_src,
                       int32_t* cow_dst, int32_t* n_cow) {
  PKV_REQUIRE(alloc, "allocator is NULL");
  PKV_REQUIRE(n == 0 || slots_out, "slots_out is NULL");
  PKV_REQUIRE(cow_src && cow_dst && n_cow, "cow outputs are NULL");
  std::vector<pkv::CowPair> pairs;
  int32_t st = alloc->impl.append(seq, n, slots_out, &pairs);
  if (st != PKV_OK) return st;
  *n_cow = static_cast<int32_t>(pairs.size());
  if (!pairs.empty()) {
    *cow_src = pairs[0].src;
    *cow_dst = pairs[0].dst;
  }
  return PKV_OK;
}

int32_t pkv_append_batch(pkv_allocator* alloc, const int64_t* seqs,
                         const int32_t* counts, int32_t num_seqs,
                         int32_t* slots_out, int64_t slots_cap,
                         int32_t* cow_src, int32_t* cow_dst, int32_t cow_cap,
                         int32_t* n_cow) {
  PKV_REQUIRE(alloc, "allocator is NULL");
  PKV_REQUIRE(num_seqs == 0 || (seqs && counts), "seqs/counts are NULL");
  PKV_REQUIRE(slots_cap == 0 || slots_out, "slots_out is NULL");
  PKV_REQUIRE(cow_cap == 0 || (cow_src && cow_dst), "cow outputs are NULL");
  PKV_REQUIRE(n_cow, "n_cow is NULL");
  PKV_REQUIRE(cow_cap >= 0 && slots_cap >= 0, "negative capacity");
  std::vector<pkv::CowPair> pairs(cow_cap > 0 ? cow_cap : 0);
  int32_t got = 0;
  int32_t st = alloc->impl.append_batch(seqs, counts, num_seqs, slots_out,
                                        slots_cap, pairs.data(), cow_cap,
                                        &got);
  if (st != PKV_OK) return st;
  for (int32_t i = 0; i < got; ++i) {
    cow_src[i] = pairs[i].src;
    cow_dst[i] = pairs[i].dst;
  }
  *n_cow = got;
  return PKV_OK;
}

int32_t pkv_append_batch_tables(pkv_allocator* alloc, const int64_t* seqs,
                                const int32_t* counts, int32_t num_seqs,
                                int32_t* slots_out, int64_t slots_cap,
                                int32_t* cow_src, int32_t* cow_dst,
                                int32_t cow_cap, int32_t* n_cow,
                                int32_t max_blocks, int32_t* block_tables,
                                int32_t* context_lens) {
  PKV_REQUIRE(alloc, "allocator is NULL");
  PKV_REQUIRE(num_seqs == 0 || (seqs && counts), "seqs/counts are NULL");
  PKV_REQUIRE(slots_cap == 0 || slots_out, "slots_out is NULL");
  PKV_REQUIRE(cow_cap == 0 || (cow_src && cow_dst), "cow outputs are NULL");
  PKV_REQUIRE(n_cow, "n_cow is NULL");
  PKV_REQUIRE(cow_cap >= 0 && slots_cap >= 0 && max_blocks >= 0, "negative capacity");
  PKV_REQUIRE(num_seqs == 0 || max_blocks == 0 || block_tables, "block_tables is NULL");
  PKV_REQUIRE(num_seqs == 0 || context_lens, "context_lens is NULL");
  thread_local std::vector<pkv::CowPair> pairs;
  pairs.resize(cow_cap > 0 ? cow_cap : 0);
  int32_t got = 0;
  thread_local int32_t dummy_row = 0;
  int32_t st = alloc->impl.append_batch(seqs, counts, num_seqs, slots_out, slots_cap,
                                        pairs.data(), cow_cap, &got, max_blocks,
                                        block_tables ? block_tables : &dummy_row,
                                        context_lens);
  if (st != PKV_OK) return st;
  for (int32_t i = 0; i < got; ++i) {
    cow_src[i] = pairs[i].src;
    cow_dst[i] = pairs[i].dst;
  }
  *n_cow = got;
  return PKV_OK;
}

int32_t pkv_append_batch_changes(pkv_allocator* alloc, const int64_t* seqs,
                                 const int32_t* counts, int32_t num_seqs,
                                 int32_t* slots_out, int64_t slots_cap,
                                 int32_t* cow_src, int32_t* cow_dst,
                                 int32_t cow_cap, int32_t* n_cow,
                                 int32_t* context_lens, int32_t* changes,
                                 int32_t changes_cap, int32_t* n_changes) {
  PKV_REQUIRE(alloc, "allocator is NULL");
  PKV_REQUIRE(num_seqs == 0 || (seqs && counts && context_lens), "NULL argument");
  PKV_REQUIRE(slots_cap == 0 || slots_out, "slots_out is NULL");
  PKV_REQUIRE(cow_cap == 0 || (cow_src && cow_dst), "cow outputs are NULL");
  PKV_REQUIRE(n_cow && n_changes, "count outputs are NULL");
  PKV_REQUIRE(changes_cap == 0 || changes, "changes is NULL");
  PKV_REQUIRE(cow_cap >= 0 && slots_cap >= 0 && changes_cap >= 0, "negative capacity");
  thread_local std::vector<pkv::CowPair> pairs;
  pairs.resize(cow_cap > 0 ? cow_cap : 0);
  static_assert(sizeof(pkv::TableChange) == 3 * sizeof(int32_t), "packed triples");
  int32_t got = 0;
  int32_t st = alloc->impl.append_batch(
      seqs, counts, num_seqs, slots_out, slots_cap, pairs.data(), cow_cap, &got, 0, nullptr,
      context_lens, reinterpret_cast<pkv::TableChange*>(changes), changes_cap, n_changes);
  if (st != PKV_OK) return st;
  for (int32_t i = 0; i < got; ++i) {
    cow_src[i] = pairs[i].src;
    cow_dst[i] = pairs[i].dst;
  }
  *n_cow = got;
  return PKV_OK;
}

int32_t pkv_seq_len(const pkv_allocator* alloc, int64_t seq, int32_t* len) {
  PKV_REQUIRE(alloc && len, "NULL argument");
  if (!alloc->impl.has(seq))
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld",
                static_cast<long long>(seq));
  *len = alloc->impl.length(seq);
  return ok();
}

int32_t pkv_seq_block_table(const pkv_allocator* alloc, int64_t seq,
                            int32_t* out, int32_t cap, int32_t* n) {
  PKV_REQUIRE(alloc && n, "NULL argument");
  if (!alloc->impl.has(seq))
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld",
                static_cast<long long>(seq));
  const auto& t = alloc->impl.table(seq);
  *n = static_cast<int32_t>(t.size());
  if (static_cast<int64_t>(t.size()) > cap)
    return fail(PKV_ERR_BUFFER_TOO_SMALL, "table has %zu entries, cap %d",
                t.size(), cap);
  PKV_REQUIRE(t.empty() || out, "out is NULL");
  for (size_t i = 0; i < t.size(); ++i) out[i] = t[i];
  return ok();
}

int32_t pkv_num_free_blocks(const pkv_allocator* alloc, int32_t* n) {
  PKV_REQUIRE(alloc && n, "NULL argument");
  *n = alloc->impl.num_free();
  return ok();
}

int32_t pkv_num_blocks(const pkv_allocator* alloc, int32_t* n) {
  PKV_REQUIRE(alloc && n, "NULL argument");
  *n = alloc->impl.num_blocks();
  return ok();
}

int32_t pkv_block_size(const pkv_allocator* alloc, int32_t* n) {
  PKV_REQUIRE(alloc && n, "NULL argument");
  *n = alloc->impl.block_size();
  return ok();
}

int32_t pkv_block_refcount(const pkv_allocator* alloc, int32_t block,
                           int32_t* count) {
  PKV_REQUIRE(alloc && count, "NULL argument");
  PKV_REQUIRE(block >= 0 && block < alloc->impl.num_blocks(),
              "block %d outside the pool", block);
  *count = alloc->impl.refcount(block);
  return ok();
}

int32_t pkv_allocator_snapshot(const pkv_allocator* alloc,
                               int32_t* free_stack, int32_t* n_free,
                               int32_t* refcounts) {
  PKV_REQUIRE(alloc && free_stack && n_free && refcounts, "NULL argument");
  alloc->impl.free_stack(free_stack);
  *n_free = alloc->impl.num_free();
  const auto& r = alloc->impl.refcounts();
  for (size_t i = 0; i < r.size(); ++i) refcounts[i] = r[i];
  return ok();
}

int32_t pkv_build_block_tables(const pkv_allocator* alloc,
                               const int64_t* seqs, int32_t num_seqs,
                               int32_t max_blocks, int32_t* block_tables,
                               int32_t* context_lens) {
  PKV_REQUIRE(alloc, "allocator is NULL");
  PKV_REQUIRE(num_seqs >= 0 && max_blocks >= 0, "negative size");
  PKV_REQUIRE(num_seqs == 0 || (seqs && context_lens), "NULL argument");
  PKV_REQUIRE(num_seqs == 0 || max_blocks == 0 || block_tables,
              "block_tables is NULL");
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (!alloc->impl.has(seqs[i]))
      return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld",
                  static_cast<long long>(seqs[i]));
    if (alloc->impl.swapped(seqs[i]))
      return fail(PKV_ERR_INVALID, "sequence %lld is swapped out",
                  static_cast<long long>(seqs[i]));
    if (static_cast<int64_t>(alloc->impl.table(seqs[i]).size()) > max_blocks)
      return fail(PKV_ERR_BUFFER_TOO_SMALL,
                  "sequence %lld holds %zu blocks, max_blocks is %d",
                  static_cast<long long>(seqs[i]),
                  alloc->impl.table(seqs[i]).size(), max_blocks);
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto& t = alloc->impl.table(seqs[i]);
    int32_t* row = block_tables + int64_t(i) * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j)
      row[j] = j < static_cast<int32_t>(t.size()) ? t[j] : -1;
    context_lens[i] = alloc->impl.length(seqs[i]);
  }
  return ok();
}

}  // extern "C"
