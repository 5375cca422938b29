// Test driver: replays allocator commands read from stdin through the native
// allocator (allocator.cpp, built with g++ and sanitizers, no HIP) and prints
// every result, for comparison with the Python model.
//
//   create N B [perm...]   add   fork P   append S N   step K S1..SK   free S
//   table S   refs   free_count   stats
// Every command prints one line: "rc <code> ..." followed by its results.
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "pagedkv.h"
#include "status.hpp"

namespace pagedkv {
std::string& last_error() {
  static thread_local std::string msg;
  return msg;
}
}  // namespace pagedkv

int main() {
  pa_alloc* a = nullptr;
  int32_t nblocks = 0;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    in >> cmd;
    std::ostringstream out;
    if (cmd == "create") {
      int32_t n, b;
      in >> n >> b;
      std::vector<int32_t> perm;
      int32_t x;
      while (in >> x) perm.push_back(x);
      if (a) pa_alloc_destroy(a);
      a = nullptr;
      int rc = pa_alloc_create(n, b, perm.empty() ? nullptr : perm.data(), &a);
      nblocks = n;
      out << "rc " << rc;
    } else if (cmd == "add") {
      int32_t id = -1;
      int rc = pa_seq_add(a, &id);
      out << "rc " << rc << " " << id;
    } else if (cmd == "fork") {
      int32_t p, id = -1;
      in >> p;
      int rc = pa_seq_fork(a, p, &id);
      out << "rc " << rc << " " << id;
    } else if (cmd == "append") {
      int32_t s, n;
      in >> s >> n;
      std::vector<int64_t> slots(n > 0 ? n : 1);
      int32_t src = -9, dst = -9;
      int rc = pa_seq_append(a, s, n, slots.data(), &src, &dst);
      out << "rc " << rc;
      if (rc == PA_OK) {
        out << " " << src << " " << dst;
        for (int32_t i = 0; i < n; ++i) out << " " << slots[i];
      }
    } else if (cmd == "step") {
      int32_t k;
      in >> k;
      std::vector<int32_t> seqs(k);
      for (auto& s : seqs) in >> s;
      std::vector<int64_t> slots(k > 0 ? k : 1);
      std::vector<int32_t> pairs(2 * (k > 0 ? k : 1));
      int32_t np = 0, done = 0;
      int rc = pa_step_append(a, seqs.data(), k, slots.data(), pairs.data(), &np, &done);
      out << "rc " << rc << " " << done << " " << np;
      for (int32_t i = 0; i < done; ++i) out << " " << slots[i];
      for (int32_t i = 0; i < 2 * np; ++i) out << " " << pairs[i];
    } else if (cmd == "free") {
      int32_t s;
      in >> s;
      out << "rc " << pa_seq_free(a, s);
    } else if (cmd == "table") {
      int32_t s, ctx = 0, nb = 0;
      in >> s;
      int rc = pa_seq_info(a, s, &ctx, &nb);
      out << "rc " << rc;
      if (rc == PA_OK) {
        std::vector<int32_t> phys(nb + 1), filled(nb + 1);
        rc = pa_seq_block_table(a, s, phys.data(), filled.data(), nb);
        out << " " << ctx;
        for (int32_t i = 0; i < nb; ++i) out << " " << phys[i] << ":" << filled[i];
      }
    } else if (cmd == "refs") {
      out << "rc 0";
      for (int32_t b = 0; b < nblocks; ++b) {
        int32_t r = -1;
        pa_block_ref(a, b, &r);
        out << " " << r;
      }
    } else if (cmd == "free_count") {
      int32_t n = -1;
      int rc = pa_num_free(a, &n);
      out << "rc " << rc << " " << n;
    } else if (cmd == "stats") {
      int64_t used = -1, filled = -1;
      int rc = pa_alloc_stats(a, &used, &filled);
      out << "rc " << rc << " " << used << " " << filled;
    } else {
      out << "rc -100 unknown";
    }
    std::cout << out.str() << "\n";
  }
  std::cout.flush();
  if (a) pa_alloc_destroy(a);
  return 0;
}
