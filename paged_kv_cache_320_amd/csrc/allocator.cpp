// Host block allocator of the paged KV cache.
//
// «The KV Cache and PagedAttention»:
//  "Like Pages of Memory"      equal physical blocks; a text's logical blocks map anywhere.
//  "The Block Table"           per-text table of (physical block, places filled); a new
//                              block only when every earlier block is full; blocks return
//                              to the free list when the text ends.
//  "Shared, Copied on Write"   shared blocks carry reference counts; a sharer about to write
//                              into a shared block gets a copy and the original's count drops.
//  "When Memory Runs Out"      a text holds all of its blocks or none: an append that cannot
//                              get every block it needs changes nothing; texts that give way
//                              move all their blocks to a pool in host memory and back.
//  "What Came After"           prefix caching: full blocks registered under a chained hash of
//                              their tokens are reused by texts that begin the same way;
//                              registered blocks nobody holds are handed out last.
// The free-list order, id assignment and "first writer copies" choices are fixed in
// pagedkv.h so that tables are reproducible.
//
// Plain C++17, no HIP: it builds and runs on any host.
#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "status.hpp"

using pagedkv::fail;
using pagedkv::ok;

namespace {

struct Seq {
  bool live = false;
  bool swapped = false;         // blocks are host-pool blocks (pa_swap_out)
  std::vector<int32_t> blocks;  // physical block per logical block
  std::vector<int32_t> filled;  // places filled per logical block
  int64_t ctx = 0;              // tokens held
};

// The free blocks as a stack that also takes blocks at its bottom and gives up any
// block in O(1) (a doubly linked list over block ids; `down` points toward the bottom).
struct FreeStack {
  std::vector<int32_t> up, down;
  int32_t top = -1, bottom = -1, size = 0;

  void init(int32_t n) {
    up.assign(n, -1);
    down.assign(n, -1);
  }
  void push_top(int32_t b) {
    up[b] = -1;
    down[b] = top;
    if (top >= 0) up[top] = b;
    else bottom = b;
    top = b;
    ++size;
  }
  void push_bottom(int32_t b) {
    down[b] = -1;
    up[b] = bottom;
    if (bottom >= 0) down[bottom] = b;
    else top = b;
    bottom = b;
    ++size;
  }
  void remove(int32_t b) {
    const int32_t u = up[b], d = down[b];
    if (u >= 0) down[u] = d;
    else top = d;
    if (d >= 0) up[d] = u;
    else bottom = u;
    up[b] = down[b] = -1;
    --size;
  }
  int32_t pop_top() {
    const int32_t b = top;
    remove(b);
    return b;
  }
};

}  // namespace

struct pa_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  FreeStack free_stack;
  std::vector<int32_t> ref;
  std::vector<Seq> seqs;            // index = sequence id
  // prefix caching: registered blocks and their hashes
  std::unordered_map<uint64_t, int32_t> block_of;
  std::vector<uint64_t> hash_of;
  std::vector<char> registered;
  // host pool for texts that give way (pa_swap_out / pa_swap_in)
  int32_t num_host_blocks = 0;
  FreeStack host_free;
  std::vector<int32_t> host_ref;

  // Top of the free stack with count 1; a registered block loses its registration.
  int32_t take() {
    const int32_t b = free_stack.pop_top();
    if (registered[b]) {
      block_of.erase(hash_of[b]);
      registered[b] = 0;
    }
    ref[b] = 1;
    return b;
  }

  // Release device blocks whose count reached 0, in the order given: unregistered ones
  // onto the top of the free stack, registered ones below every other free block (the
  // later ones above the earlier), all above blocks freed before.
  void release(const std::vector<int32_t>& zero) {
    std::vector<int32_t> cached;
    for (int32_t b : zero) {
      if (registered[b]) cached.push_back(b);
      else free_stack.push_top(b);
    }
    for (auto it = cached.rbegin(); it != cached.rend(); ++it) free_stack.push_bottom(*it);
  }

  Seq* find(int32_t id) {
    if (id < 0 || id >= (int32_t)seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
  const Seq* find(int32_t id) const {
    if (id < 0 || id >= (int32_t)seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }

  // Blocks an append of n tokens needs, and whether it copies the last block.
  int64_t blocks_needed(const Seq& s, int64_t n, bool* copy) const {
    *copy = false;
    if (n == 0) return 0;
    int64_t room = 0;
    if (!s.blocks.empty() && s.filled.back() < block_size) {
      room = block_size - s.filled.back();
      *copy = ref[s.blocks.back()] > 1;
    }
    int64_t beyond = std::max<int64_t>(0, n - room);
    return (*copy ? 1 : 0) + (beyond + block_size - 1) / block_size;
  }

  int append(Seq& s, int32_t n, int64_t* slots, int32_t* src, int32_t* dst) {
    bool copy = false;
    int64_t need = blocks_needed(s, n, &copy);
    if (need > (int64_t)free_stack.size)
      return fail(PA_ENOBLOCKS, "append of %d tokens needs %lld blocks, %d free", n,
                  (long long)need, free_stack.size);
    *src = -1;
    *dst = -1;
    if (copy) {
      int32_t old = s.blocks.back();
      int32_t fresh = take();
      ref[old] -= 1;
      s.blocks.back() = fresh;
      *src = old;
      *dst = fresh;
    }
    for (int32_t i = 0; i < n; ++i) {
      if (s.blocks.empty() || s.filled.back() == block_size) {
        int32_t b = take();
        s.blocks.push_back(b);
        s.filled.push_back(0);
      }
      slots[i] = (int64_t)s.blocks.back() * block_size + s.filled.back();
      s.filled.back() += 1;
    }
    s.ctx += n;
    return ok();
  }
};

extern "C" {

int pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                    pa_alloc** out) {
  if (!out) return fail(PA_EINVAL, "out is null");
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1)
    return fail(PA_EINVAL, "num_blocks (%d) and block_size (%d) must be >= 1", num_blocks,
                block_size);
  if ((int64_t)num_blocks * block_size > INT64_MAX / 2)
    return fail(PA_EINVAL, "pool too large");
  pa_alloc* a = new (std::nothrow) pa_alloc();
  if (!a) return fail(PA_EINVAL, "out of host memory");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->ref.assign(num_blocks, 0);
  a->hash_of.assign(num_blocks, 0);
  a->registered.assign(num_blocks, 0);
  a->free_stack.init(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return fail(PA_EINVAL, "free_order is not a permutation of 0..%d", num_blocks - 1);
      }
      seen[b] = 1;
    }
    for (int32_t i = 0; i < num_blocks; ++i) a->free_stack.push_bottom(free_order[i]);
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->free_stack.push_bottom(i);
  }
  *out = a;
  return ok();
}

void pa_alloc_destroy(pa_alloc* a) { delete a; }

int pa_seq_add(pa_alloc* a, int32_t* seq_out) {
  if (!a || !seq_out) return fail(PA_EINVAL, "null argument");
  if (a->seqs.size() >= (size_t)INT32_MAX) return fail(PA_EINVAL, "sequence ids exhausted");
  a->seqs.emplace_back();
  a->seqs.back().live = true;
  *seq_out = (int32_t)a->seqs.size() - 1;
  return ok();
}

int pa_seq_fork(pa_alloc* a, int32_t parent, int32_t* child_out) {
  if (!a || !child_out) return fail(PA_EINVAL, "null argument");
  if (!a->find(parent)) return fail(PA_ENOSEQ, "unknown sequence %d", parent);
  if (a->find(parent)->swapped) return fail(PA_EINVAL, "sequence %d is swapped out", parent);
  if (a->seqs.size() >= (size_t)INT32_MAX) return fail(PA_EINVAL, "sequence ids exhausted");
  Seq child = *a->find(parent);  // copy before emplace_back may reallocate
  for (int32_t b : child.blocks) a->ref[b] += 1;
  a->seqs.push_back(std::move(child));
  *child_out = (int32_t)a->seqs.size() - 1;
  return ok();
}

int pa_seq_append(pa_alloc* a, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                  int32_t* cow_src, int32_t* cow_dst) {
  if (!a || !cow_src || !cow_dst || (n_tokens > 0 && !slots_out))
    return fail(PA_EINVAL, "null argument");
  if (n_tokens < 0) return fail(PA_EINVAL, "n_tokens %d < 0", n_tokens);
  Seq* s = a->find(seq);
  if (!s) return fail(PA_ENOSEQ, "unknown sequence %d", seq);
  if (s->swapped) return fail(PA_EINVAL, "sequence %d is swapped out", seq);
  return a->append(*s, n_tokens, slots_out, cow_src, cow_dst);
}

int pa_step_append(pa_alloc* a, const int32_t* seqs, int32_t n, int64_t* slots_out,
                   int32_t* pairs_out, int32_t* num_pairs_out, int32_t* done_out) {
  if (!a || !num_pairs_out || !done_out || (n > 0 && (!seqs || !slots_out || !pairs_out)))
    return fail(PA_EINVAL, "null argument");
  if (n < 0) return fail(PA_EINVAL, "n %d < 0", n);
  *num_pairs_out = 0;
  *done_out = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq* s = a->find(seqs[i]);
    if (!s) return fail(PA_ENOSEQ, "unknown sequence %d at batch index %d", seqs[i], i);
    if (s->swapped) return fail(PA_EINVAL, "sequence %d is swapped out", seqs[i]);
    int32_t src, dst;
    int rc = a->append(*s, 1, &slots_out[i], &src, &dst);
    if (rc != PA_OK) return rc;
    if (src >= 0) {
      pairs_out[2 * *num_pairs_out] = src;
      pairs_out[2 * *num_pairs_out + 1] = dst;
      *num_pairs_out += 1;
    }
    *done_out = i + 1;
  }
  return ok();
}

int pa_seq_free(pa_alloc* a, int32_t seq) {
  if (!a) return fail(PA_EINVAL, "null argument");
  Seq* s = a->find(seq);
  if (!s) return fail(PA_ENOSEQ, "unknown sequence %d", seq);
  if (s->swapped) {
    for (int32_t b : s->blocks)
      if (--a->host_ref[b] == 0) a->host_free.push_top(b);
  } else {
    std::vector<int32_t> zero;
    for (int32_t b : s->blocks)
      if (--a->ref[b] == 0) zero.push_back(b);
    a->release(zero);
  }
  *s = Seq();  // live = false, storage released
  return ok();
}

int pa_seq_info(const pa_alloc* a, int32_t seq, int32_t* ctx_len, int32_t* n_blocks) {
  if (!a || !ctx_len || !n_blocks) return fail(PA_EINVAL, "null argument");
  const Seq* s = a->find(seq);
  if (!s) return fail(PA_ENOSEQ, "unknown sequence %d", seq);
  if (s->ctx > INT32_MAX) return fail(PA_EINVAL, "context length exceeds int32");
  *ctx_len = (int32_t)s->ctx;
  *n_blocks = (int32_t)s->blocks.size();
  return ok();
}

int pa_seq_block_table(const pa_alloc* a, int32_t seq, int32_t* phys_out, int32_t* filled_out,
                       int32_t cap) {
  if (!a) return fail(PA_EINVAL, "null argument");
  const Seq* s = a->find(seq);
  if (!s) return fail(PA_ENOSEQ, "unknown sequence %d", seq);
  if ((int64_t)s->blocks.size() > cap)
    return fail(PA_EINVAL, "capacity %d < %zu blocks", cap, s->blocks.size());
  if (!s->blocks.empty() && (!phys_out || !filled_out)) return fail(PA_EINVAL, "null argument");
  std::copy(s->blocks.begin(), s->blocks.end(), phys_out);
  std::copy(s->filled.begin(), s->filled.end(), filled_out);
  return ok();
}

int pa_export_tables(const pa_alloc* a, const int32_t* seqs, int32_t n,
                     int32_t max_blocks_per_seq, int32_t* tables_out, int32_t* ctx_lens_out) {
  if (!a || (n > 0 && (!seqs || !tables_out || !ctx_lens_out)))
    return fail(PA_EINVAL, "null argument");
  if (n < 0 || max_blocks_per_seq < 0) return fail(PA_EINVAL, "negative size");
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = a->find(seqs[i]);
    if (!s) return fail(PA_ENOSEQ, "unknown sequence %d at batch index %d", seqs[i], i);
    if (s->swapped) return fail(PA_EINVAL, "sequence %d is swapped out", seqs[i]);
    if ((int64_t)s->blocks.size() > max_blocks_per_seq)
      return fail(PA_EINVAL, "sequence %d has %zu blocks > max_blocks_per_seq %d", seqs[i],
                  s->blocks.size(), max_blocks_per_seq);
    if (s->ctx > INT32_MAX) return fail(PA_EINVAL, "context length exceeds int32");
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = a->find(seqs[i]);
    int32_t* row = tables_out + (int64_t)i * max_blocks_per_seq;
    std::copy(s->blocks.begin(), s->blocks.end(), row);
    std::fill(row + s->blocks.size(), row + max_blocks_per_seq, -1);
    ctx_lens_out[i] = (int32_t)s->ctx;
  }
  return ok();
}

int pa_block_ref(const pa_alloc* a, int32_t block, int32_t* ref_out) {
  if (!a || !ref_out) return fail(PA_EINVAL, "null argument");
  if (block < 0 || block >= a->num_blocks)
    return fail(PA_EINVAL, "block %d outside [0, %d)", block, a->num_blocks);
  *ref_out = a->ref[block];
  return ok();
}

int pa_num_free(const pa_alloc* a, int32_t* n_out) {
  if (!a || !n_out) return fail(PA_EINVAL, "null argument");
  *n_out = a->free_stack.size;
  return ok();
}

int pa_alloc_stats(const pa_alloc* a, int64_t* used_blocks, int64_t* filled_slots) {
  if (!a || !used_blocks || !filled_slots) return fail(PA_EINVAL, "null argument");
  std::vector<int32_t> filled(a->num_blocks, -1);
  for (const Seq& s : a->seqs) {
    if (!s.live || s.swapped) continue;
    for (size_t j = 0; j < s.blocks.size(); ++j) filled[s.blocks[j]] = s.filled[j];
  }
  int64_t f = 0;
  for (int32_t x : filled)
    if (x > 0) f += x;
  *used_blocks = (int64_t)a->num_blocks - (int64_t)a->free_stack.size;
  *filled_slots = f;
  return ok();
}

// ---- share groups for the shared-block decode ("Shared, Copied on Write") ------

// Leading physical blocks two texts hold in common.
static int64_t common_blocks(const Seq& x, const Seq& y) {
  const size_t m = std::min(x.blocks.size(), y.blocks.size());
  size_t j = 0;
  while (j < m && x.blocks[j] == y.blocks[j]) ++j;
  return (int64_t)j;
}

// Runs of consecutive batch texts [lo, hi) whose leading blocks agree beyond `above` blocks,
// at most `members` texts each; emit (first, count, shared tokens) for runs of 2 or more.
static int emit_runs(const pa_alloc* a, const std::vector<const Seq*>& s, int32_t lo, int32_t hi,
                     int64_t above, int32_t members, int32_t cap, int32_t* first_out,
                     int32_t* count_out, int32_t* prefix_out, int32_t* num) {
  int32_t i = lo;
  while (i < hi) {
    int64_t c = INT64_MAX;
    int32_t j = i + 1;
    while (j < hi && j - i < members) {
      const int64_t cb = common_blocks(*s[i], *s[j]);
      if (cb <= above) break;
      c = std::min(c, cb);
      ++j;
    }
    if (j - i >= 2) {
      if (*num >= cap) return fail(PA_EINVAL, "more than %d share groups", cap);
      const int64_t tokens = c * a->block_size;
      first_out[*num] = i;
      count_out[*num] = j - i;
      prefix_out[*num] = (int32_t)std::min<int64_t>(tokens, INT32_MAX);
      ++*num;
      i = j;
    } else {
      ++i;
    }
  }
  return PA_OK;
}

static int batch_seqs(const pa_alloc* a, const int32_t* seqs, int32_t n,
                      std::vector<const Seq*>* out) {
  out->resize(n);
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = a->find(seqs[i]);
    if (!s) return fail(PA_ENOSEQ, "unknown sequence %d at batch index %d", seqs[i], i);
    if (s->swapped) return fail(PA_EINVAL, "sequence %d is swapped out", seqs[i]);
    (*out)[i] = s;
  }
  return PA_OK;
}

int pa_share_groups(const pa_alloc* a, const int32_t* seqs, int32_t n, int32_t max_members,
                    int32_t cap, int32_t* first_out, int32_t* count_out, int32_t* prefix_out,
                    int32_t* num_groups_out) {
  if (!a || !num_groups_out || (n > 0 && !seqs) ||
      (cap > 0 && (!first_out || !count_out || !prefix_out)))
    return fail(PA_EINVAL, "null argument");
  if (n < 0 || cap < 0 || max_members < 2)
    return fail(PA_EINVAL, "n %d and cap %d must be >= 0, max_members %d >= 2", n, cap,
                max_members);
  std::vector<const Seq*> s;
  int rc = batch_seqs(a, seqs, n, &s);
  if (rc != PA_OK) return rc;
  int32_t num = 0;
  rc = emit_runs(a, s, 0, n, 0, max_members, cap, first_out, count_out, prefix_out, &num);
  if (rc != PA_OK) return rc;
  *num_groups_out = num;
  return ok();
}

int pa_share_groups_inner(const pa_alloc* a, const int32_t* seqs, int32_t n, int32_t num_groups,
                          const int32_t* group_first, const int32_t* group_count,
                          const int32_t* group_prefix, int32_t inner_members, int32_t cap,
                          int32_t* first_out, int32_t* count_out, int32_t* prefix_out,
                          int32_t* num_inner_out) {
  if (!a || !num_inner_out || (n > 0 && !seqs) ||
      (num_groups > 0 && (!group_first || !group_count || !group_prefix)) ||
      (cap > 0 && (!first_out || !count_out || !prefix_out)))
    return fail(PA_EINVAL, "null argument");
  if (n < 0 || num_groups < 0 || cap < 0 || inner_members < 2)
    return fail(PA_EINVAL, "n %d, num_groups %d and cap %d must be >= 0, inner_members %d >= 2",
                n, num_groups, cap, inner_members);
  std::vector<const Seq*> s;
  int rc = batch_seqs(a, seqs, n, &s);
  if (rc != PA_OK) return rc;
  int32_t num = 0;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t f = group_first[g], k = group_count[g];
    if (f < 0 || k < 0 || (int64_t)f + k > n || group_prefix[g] < 0)
      return fail(PA_EINVAL, "group %d (first %d, count %d, shared %d) outside the batch", g, f,
                  k, group_prefix[g]);
    rc = emit_runs(a, s, f, f + k, group_prefix[g] / a->block_size, inner_members, cap,
                   first_out, count_out, prefix_out, &num);
    if (rc != PA_OK) return rc;
  }
  *num_inner_out = num;
  return ok();
}

// ---- prefix caching ("What Came After") ---------------------------------------

// 64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime 0x100000001b3) over `n` bytes,
// continuing from state h.
static uint64_t fnv1a64(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

int pa_hash_blocks(const int32_t* tokens, int32_t n_tokens, int32_t block_size, uint64_t parent,
                   uint64_t* hashes_out) {
  if (n_tokens < 0 || block_size < 1) return fail(PA_EINVAL, "n_tokens < 0 or block_size < 1");
  const int32_t nb = n_tokens / block_size;
  if (nb > 0 && (!tokens || !hashes_out)) return fail(PA_EINVAL, "null argument");
  uint64_t h = parent;
  for (int32_t j = 0; j < nb; ++j) {
    unsigned char le[8];
    for (int k = 0; k < 8; ++k) le[k] = (unsigned char)(h >> (8 * k));
    uint64_t x = fnv1a64(0xcbf29ce484222325ull, le, 8);
    for (int32_t t = 0; t < block_size; ++t) {
      const uint32_t tok = (uint32_t)tokens[(int64_t)j * block_size + t];
      unsigned char tb[4] = {(unsigned char)tok, (unsigned char)(tok >> 8),
                             (unsigned char)(tok >> 16), (unsigned char)(tok >> 24)};
      x = fnv1a64(x, tb, 4);
    }
    hashes_out[j] = h = x;
  }
  return ok();
}

int pa_seq_add_cached(pa_alloc* a, const uint64_t* hashes, int32_t n_hashes, int32_t* seq_out,
                      int32_t* n_cached_out) {
  if (!a || !seq_out || !n_cached_out || (n_hashes > 0 && !hashes))
    return fail(PA_EINVAL, "null argument");
  if (n_hashes < 0) return fail(PA_EINVAL, "n_hashes %d < 0", n_hashes);
  if (a->seqs.size() >= (size_t)INT32_MAX) return fail(PA_EINVAL, "sequence ids exhausted");
  Seq s;
  s.live = true;
  for (int32_t j = 0; j < n_hashes; ++j) {
    auto it = a->block_of.find(hashes[j]);
    if (it == a->block_of.end()) break;
    const int32_t b = it->second;
    if (a->ref[b] == 0) a->free_stack.remove(b);
    a->ref[b] += 1;
    s.blocks.push_back(b);
    s.filled.push_back(a->block_size);
    s.ctx += a->block_size;
  }
  *n_cached_out = (int32_t)s.blocks.size();
  a->seqs.push_back(std::move(s));
  *seq_out = (int32_t)a->seqs.size() - 1;
  return ok();
}

int pa_seq_cache_blocks(pa_alloc* a, int32_t seq, const uint64_t* hashes, int32_t n) {
  if (!a || (n > 0 && !hashes)) return fail(PA_EINVAL, "null argument");
  Seq* s = a->find(seq);
  if (!s) return fail(PA_ENOSEQ, "unknown sequence %d", seq);
  if (s->swapped) return fail(PA_EINVAL, "sequence %d is swapped out", seq);
  if (n < 0 || n > (int32_t)s->blocks.size())
    return fail(PA_EINVAL, "n %d outside [0, %zu]", n, s->blocks.size());
  for (int32_t j = 0; j < n; ++j)
    if (s->filled[j] != a->block_size)
      return fail(PA_EINVAL, "logical block %d of sequence %d is not full", j, seq);
  for (int32_t j = 0; j < n; ++j) {
    const int32_t b = s->blocks[j];
    if (a->registered[b] || a->block_of.count(hashes[j])) continue;
    a->block_of.emplace(hashes[j], b);
    a->hash_of[b] = hashes[j];
    a->registered[b] = 1;
  }
  return ok();
}

int pa_cache_stats(const pa_alloc* a, int32_t* registered_out, int32_t* registered_free_out) {
  if (!a || !registered_out || !registered_free_out) return fail(PA_EINVAL, "null argument");
  int32_t r = 0, f = 0;
  for (int32_t b = 0; b < a->num_blocks; ++b)
    if (a->registered[b]) {
      ++r;
      if (a->ref[b] == 0) ++f;
    }
  *registered_out = r;
  *registered_free_out = f;
  return ok();
}

// ---- swapping to host memory ("When Memory Runs Out") ------------------------------

int pa_alloc_host_pool(pa_alloc* a, int32_t num_host_blocks, const int32_t* free_order) {
  if (!a) return fail(PA_EINVAL, "null argument");
  if (a->num_host_blocks > 0) return fail(PA_EINVAL, "the host pool is already set up");
  if (num_host_blocks < 1) return fail(PA_EINVAL, "num_host_blocks %d < 1", num_host_blocks);
  if (free_order) {
    std::vector<char> seen(num_host_blocks, 0);
    for (int32_t i = 0; i < num_host_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_host_blocks || seen[b])
        return fail(PA_EINVAL, "free_order is not a permutation of 0..%d", num_host_blocks - 1);
      seen[b] = 1;
    }
  }
  a->num_host_blocks = num_host_blocks;
  a->host_ref.assign(num_host_blocks, 0);
  a->host_free.init(num_host_blocks);
  for (int32_t i = 0; i < num_host_blocks; ++i)
    a->host_free.push_bottom(free_order ? free_order[i] : i);
  return ok();
}

// Checks shared by pa_swap_out and pa_swap_in: every listed text live, listed once, on the
// side `swapped`; the blocks they hold in distinct first-seen order (texts in list order,
// logical order within) with how many listed texts hold each.
static int swap_plan(pa_alloc* a, const int32_t* seqs, int32_t n, bool swapped,
                     std::vector<int32_t>* order, std::unordered_map<int32_t, int32_t>* holders) {
  if (a->num_host_blocks < 1) return fail(PA_EINVAL, "no host pool (pa_alloc_host_pool)");
  if (n < 0) return fail(PA_EINVAL, "n %d < 0", n);
  if (n > 0 && !seqs) return fail(PA_EINVAL, "null argument");
  std::unordered_map<int32_t, char> listed;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = a->find(seqs[i]);
    if (!s) return fail(PA_ENOSEQ, "unknown sequence %d at list index %d", seqs[i], i);
    if (s->swapped != swapped)
      return fail(PA_EINVAL, "sequence %d is %s", seqs[i], swapped ? "not swapped out" :
                  "already swapped out");
    if (!listed.emplace(seqs[i], 1).second)
      return fail(PA_EINVAL, "sequence %d is listed twice", seqs[i]);
  }
  for (int32_t i = 0; i < n; ++i)
    for (int32_t b : a->find(seqs[i])->blocks) {
      auto it = holders->find(b);
      if (it == holders->end()) {
        holders->emplace(b, 1);
        order->push_back(b);
      } else {
        it->second += 1;
      }
    }
  return ok();
}

int pa_swap_out(pa_alloc* a, const int32_t* seqs, int32_t n, int32_t* pairs_out, int32_t cap,
                int32_t* num_pairs_out) {
  if (!a || !num_pairs_out) return fail(PA_EINVAL, "null argument");
  *num_pairs_out = 0;
  std::vector<int32_t> order;
  std::unordered_map<int32_t, int32_t> holders;
  int rc = swap_plan(a, seqs, n, false, &order, &holders);
  if (rc != PA_OK) return rc;
  const int32_t need = (int32_t)order.size();
  if (need > a->host_free.size)
    return fail(PA_ENOBLOCKS, "swapping out needs %d host blocks, %d free", need,
                a->host_free.size);
  if (need > cap || (need > 0 && !pairs_out))
    return fail(PA_EINVAL, "pairs capacity %d < %d blocks", cap, need);
  std::unordered_map<int32_t, int32_t> host_of;
  std::vector<int32_t> zero;
  for (int32_t i = 0; i < need; ++i) {
    const int32_t b = order[i], h = a->host_free.pop_top(), k = holders[b];
    a->host_ref[h] = k;
    host_of.emplace(b, h);
    pairs_out[2 * i] = b;
    pairs_out[2 * i + 1] = h;
    a->ref[b] -= k;
    if (a->ref[b] == 0) zero.push_back(b);
  }
  for (int32_t i = 0; i < n; ++i) {
    Seq* s = a->find(seqs[i]);
    for (int32_t& b : s->blocks) b = host_of[b];
    s->swapped = true;
  }
  a->release(zero);
  *num_pairs_out = need;
  return ok();
}

int pa_swap_in(pa_alloc* a, const int32_t* seqs, int32_t n, int32_t* pairs_out, int32_t cap,
               int32_t* num_pairs_out) {
  if (!a || !num_pairs_out) return fail(PA_EINVAL, "null argument");
  *num_pairs_out = 0;
  std::vector<int32_t> order;
  std::unordered_map<int32_t, int32_t> holders;
  int rc = swap_plan(a, seqs, n, true, &order, &holders);
  if (rc != PA_OK) return rc;
  const int32_t need = (int32_t)order.size();
  if (need > a->free_stack.size)
    return fail(PA_ENOBLOCKS, "swapping in needs %d blocks, %d free", need, a->free_stack.size);
  if (need > cap || (need > 0 && !pairs_out))
    return fail(PA_EINVAL, "pairs capacity %d < %d blocks", cap, need);
  std::unordered_map<int32_t, int32_t> dev_of;
  for (int32_t i = 0; i < need; ++i) {
    const int32_t h = order[i], k = holders[h];
    const int32_t b = a->take();
    a->ref[b] = k;
    dev_of.emplace(h, b);
    pairs_out[2 * i] = h;
    pairs_out[2 * i + 1] = b;
  }
  for (int32_t i = 0; i < n; ++i) {
    Seq* s = a->find(seqs[i]);
    for (int32_t& b : s->blocks) b = dev_of[b];
    s->swapped = false;
  }
  for (int32_t i = 0; i < need; ++i) {
    const int32_t h = order[i];
    a->host_ref[h] -= holders[h];
    if (a->host_ref[h] == 0) a->host_free.push_top(h);
  }
  *num_pairs_out = need;
  return ok();
}

int pa_seq_swapped(const pa_alloc* a, int32_t seq, int32_t* swapped_out) {
  if (!a || !swapped_out) return fail(PA_EINVAL, "null argument");
  const Seq* s = a->find(seq);
  if (!s) return fail(PA_ENOSEQ, "unknown sequence %d", seq);
  *swapped_out = s->swapped ? 1 : 0;
  return ok();
}

int pa_host_block_ref(const pa_alloc* a, int32_t block, int32_t* ref_out) {
  if (!a || !ref_out) return fail(PA_EINVAL, "null argument");
  if (block < 0 || block >= a->num_host_blocks)
    return fail(PA_EINVAL, "host block %d outside [0, %d)", block, a->num_host_blocks);
  *ref_out = a->host_ref[block];
  return ok();
}

int pa_host_num_free(const pa_alloc* a, int32_t* n_out) {
  if (!a || !n_out) return fail(PA_EINVAL, "null argument");
  *n_out = a->host_free.size;
  return ok();
}

}  // extern "C"
