// Replays allocator and scheduler operations read from stdin through the C
// ABI of the library's host code (pkv.h), printing every result, so that a
// build of that code with AddressSanitizer and UndefinedBehaviorSanitizer
// can be driven by the randomized CPU tests and checked against the
// reference models.  One command per line; one result line per command.
//
//   A nb bs host order[nb]        create an allocator (host: swap tier blocks)
//   add s | free s | fork p c      sequence lifetime            -> status
//   app s n                        pkv_seq_append   -> status slots* cow*
//   batch k (s c)*k                pkv_append_batch_changes
//                                  -> status slots* cow* lens* changes*
//   btab k mb (s c)*k              pkv_append_batch_tables
//                                  -> status slots* cow* tables* lens*
//   sout s | sin s                 pkv_seq_swap_out / _in -> status pairs*
//   state k ids*                   free stack, refcounts, host free stack and
//                                  each id's (status, length, table)
//   S nb bs seqs budget chunk reserve host order[nb]   create a scheduler
//   req id p o                     pkv_scheduler_add_request    -> status
//   step                           pkv_scheduler_step -> status, rows,
//                                  slots, finished, preempted, swaps, stats
// A list prints as its length followed by its items.
#include <cstdint>
#include <iostream>
#include <string>
#include <vector>

#include "pkv.h"

namespace {

void put(const std::vector<int64_t>& v) {
  std::cout << ' ' << v.size();
  for (int64_t x : v) std::cout << ' ' << x;
}

template <class T>
std::vector<int64_t> wide(const T* p, int64_t n) {
  return std::vector<int64_t>(p, p + n);
}

std::vector<int32_t> read_i32(int64_t n) {
  std::vector<int32_t> v(n);
  for (auto& x : v) std::cin >> x;
  return v;
}

}  // namespace

int main() {
  pkv_allocator* a = nullptr;
  pkv_scheduler* s = nullptr;
  int32_t nb = 0, host = 0;
  std::string cmd;
  while (std::cin >> cmd) {
    if (cmd == "A") {
      int32_t bs;
      std::cin >> nb >> bs >> host;
      std::vector<int32_t> order = read_i32(nb);
      if (a) pkv_allocator_destroy(a);
      int32_t st = pkv_allocator_create(nb, bs, order.data(), &a);
      if (st == PKV_OK) st = pkv_allocator_set_host_pool(a, host);
      std::cout << st;
    } else if (cmd == "add" || cmd == "free") {
      int64_t q;
      std::cin >> q;
      std::cout << (cmd == "add" ? pkv_seq_add(a, q) : pkv_seq_free(a, q));
    } else if (cmd == "fork") {
      int64_t p, c;
      std::cin >> p >> c;
      std::cout << pkv_seq_fork(a, p, c);
    } else if (cmd == "app") {
      int64_t q;
      int32_t n;
      std::cin >> q >> n;
      std::vector<int32_t> slots(n > 0 ? n : 1);
      int32_t src = -1, dst = -1, ncow = 0;
      const int32_t st = pkv_seq_append(a, q, n, slots.data(), &src, &dst, &ncow);
      std::cout << st;
      if (st == PKV_OK) {
        put(wide(slots.data(), n));
        put(ncow ? std::vector<int64_t>{src, dst} : std::vector<int64_t>{});
      }
    } else if (cmd == "batch" || cmd == "btab") {
      int32_t k, mb = 0;
      std::cin >> k;
      if (cmd == "btab") std::cin >> mb;
      std::vector<int64_t> seqs(k);
      std::vector<int32_t> counts(k);
      int64_t total = 0;
      for (int32_t i = 0; i < k; ++i) {
        std::cin >> seqs[i] >> counts[i];
        total += counts[i] > 0 ? counts[i] : 0;
      }
      std::vector<int32_t> slots(total + 1), src(k + 1), dst(k + 1), lens(k + 1);
      int32_t ncow = 0;
      int32_t st;
      if (cmd == "batch") {
        const int32_t cap = int32_t(total) + k + 1;
        std::vector<int32_t> changes(3 * size_t(cap));
        int32_t nch = 0;
        st = pkv_append_batch_changes(a, seqs.data(), counts.data(), k, slots.data(), total + 1,
                                      src.data(), dst.data(), k + 1, &ncow, lens.data(),
                                      changes.data(), cap, &nch);
        std::cout << st;
        if (st == PKV_OK) {
          put(wide(slots.data(), total));
          std::vector<int64_t> cow;
          for (int32_t i = 0; i < ncow; ++i) cow.insert(cow.end(), {src[i], dst[i]});
          put(cow);
          put(wide(lens.data(), k));
          put(wide(changes.data(), 3 * int64_t(nch)));
        }
      } else {
        std::vector<int32_t> tables(size_t(k) * mb + 1);
        st = pkv_append_batch_tables(a, seqs.data(), counts.data(), k, slots.data(), total + 1,
                                     src.data(), dst.data(), k + 1, &ncow, mb, tables.data(),
                                     lens.data());
        std::cout << st;
        if (st == PKV_OK) {
          put(wide(slots.data(), total));
          std::vector<int64_t> cow;
          for (int32_t i = 0; i < ncow; ++i) cow.insert(cow.end(), {src[i], dst[i]});
          put(cow);
          put(wide(tables.data(), int64_t(k) * mb));
          put(wide(lens.data(), k));
        }
      }
    } else if (cmd == "sout" || cmd == "sin") {
      int64_t q;
      std::cin >> q;
      const int32_t cap = nb + host + 1;
      std::vector<int32_t> x(cap), y(cap);
      int32_t n = 0;
      // pairs are printed as (from, to): device -> host out, host -> device in
      const int32_t st = cmd == "sout" ? pkv_seq_swap_out(a, q, x.data(), y.data(), cap, &n)
                                       : pkv_seq_swap_in(a, q, x.data(), y.data(), cap, &n);
      std::cout << st;
      if (st == PKV_OK) {
        std::vector<int64_t> pairs;
        for (int32_t i = 0; i < n; ++i) pairs.insert(pairs.end(), {x[i], y[i]});
        put(pairs);
      }
    } else if (cmd == "state") {
      int32_t k;
      std::cin >> k;
      std::vector<int32_t> free_stack(nb + 1), refs(nb + 1), host_stack(host + 1);
      int32_t nfree = 0, nhost = 0;
      std::cout << pkv_allocator_snapshot(a, free_stack.data(), &nfree, refs.data());
      std::cout << ' ' << pkv_allocator_host_snapshot(a, host_stack.data(), &nhost);
      put(wide(free_stack.data(), nfree));
      put(wide(refs.data(), nb));
      put(wide(host_stack.data(), nhost));
      for (int32_t i = 0; i < k; ++i) {
        int64_t q;
        std::cin >> q;
        int32_t len = 0, n = 0;
        std::vector<int32_t> table(nb + host + 1);
        const int32_t st = pkv_seq_len(a, q, &len);
        std::cout << ' ' << st;
        if (st == PKV_OK) {
          pkv_seq_block_table(a, q, table.data(), int32_t(table.size()), &n);
          std::cout << ' ' << len;
          put(wide(table.data(), n));
        }
      }
    } else if (cmd == "S") {
      int32_t bs, seqs, budget, chunk, reserve;
      std::cin >> nb >> bs >> seqs >> budget >> chunk >> reserve >> host;
      std::vector<int32_t> order = read_i32(nb);
      if (s) pkv_scheduler_destroy(s);
      std::cout << pkv_scheduler_create(nb, bs, order.data(), seqs, budget, chunk, reserve,
                                        host, &s);
    } else if (cmd == "req") {
      int64_t id;
      int32_t p, o;
      std::cin >> id >> p >> o;
      std::cout << pkv_scheduler_add_request(s, id, p, o);
    } else if (cmd == "step") {
      int32_t mb = 0;
      pkv_scheduler_max_blocks(s, &mb);
      mb = mb > 0 ? mb : 1;
      const int32_t rows = 64, tokens = 4096;
      std::vector<int64_t> ids(rows);
      std::vector<int32_t> qlen(rows), ctx(rows), slots(tokens), tables(size_t(rows) * mb);
      int32_t ndec = 0, nrows = 0, ntok = 0;
      const int32_t st = pkv_scheduler_step(s, rows, tokens, mb, ids.data(), qlen.data(),
                                            ctx.data(), slots.data(), tables.data(), &ndec,
                                            &nrows, &ntok);
      std::cout << st;
      if (st == PKV_OK) {
        std::cout << ' ' << nrows << ' ' << ndec;
        for (int32_t r = 0; r < nrows; ++r) {
          std::cout << ' ' << ids[r] << ' ' << qlen[r] << ' ' << ctx[r];
          std::vector<int64_t> t;
          for (int32_t j = 0; j < mb && tables[size_t(r) * mb + j] >= 0; ++j)
            t.push_back(tables[size_t(r) * mb + j]);
          put(t);
        }
        put(wide(slots.data(), ntok));
        std::vector<int64_t> fin(rows + 1), pre(rows + 1);
        int32_t nfin = 0, npre = 0;
        pkv_scheduler_last_events(s, fin.data(), rows + 1, &nfin, pre.data(), rows + 1, &npre);
        put(std::vector<int64_t>(fin.begin(), fin.begin() + nfin));
        put(std::vector<int64_t>(pre.begin(), pre.begin() + npre));
        const int32_t cap = nb + host + 1;
        std::vector<int32_t> ih(cap), id(cap), od(cap), oh(cap);
        int32_t nin = 0, nout = 0;
        pkv_scheduler_last_swaps(s, ih.data(), id.data(), cap, &nin, od.data(), oh.data(), cap,
                                 &nout);
        std::vector<int64_t> ins, outs;
        for (int32_t i = 0; i < nin; ++i) ins.insert(ins.end(), {ih[i], id[i]});
        for (int32_t i = 0; i < nout; ++i) outs.insert(outs.end(), {od[i], oh[i]});
        put(ins);
        put(outs);
        int64_t stats[11];
        pkv_scheduler_stats(s, stats);
        put(std::vector<int64_t>(stats, stats + 11));
      }
    } else {
      std::cerr << "unknown command " << cmd << "\n";
      return 2;
    }
    std::cout << std::endl;
  }
  if (a) pkv_allocator_destroy(a);
  if (s) pkv_scheduler_destroy(s);
  return 0;
}
