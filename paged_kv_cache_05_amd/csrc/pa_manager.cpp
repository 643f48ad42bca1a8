// Host-side KV block manager (include/pa_manager.h): free blocks,
// per-block reference counts, per-sequence block lists and lengths.  It
// turns "sequence s gets one more token" into a slot, allocating a block
// only when the last one is full and copying a shared last block before it
// is written (the KV cache manager, reference counts and copy-on-write of
// the wywy.jp notes on PagedAttention, Keyword section and WHERE parallel
// sampling; the memory-management table of the zhaifeiyue.github.io
// summary), and the swap of a preempted group's blocks to a CPU pool and
// back (wywy.jp Keyword "Swapping" and "All-or-nothing eviction").
#include <stdint.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_manager.h"

// One pool of blocks: reference counts and the free blocks (returned ones
// first, most recent first; then never-used ones in order).
struct BlockPool {
  std::vector<int> refcount;
  std::vector<int32_t> fresh;   // never handed out; taken from the back
  std::vector<int32_t> freed;   // returned blocks; most recent at the back

  void init(int n, const int32_t *order) {
    refcount.assign(n, 0);
    fresh.resize(n);
    for (int i = 0; i < n; ++i) fresh[n - 1 - i] = order ? order[i] : i;
    freed.clear();
  }
  int free_blocks() const { return (int)(fresh.size() + freed.size()); }
  int size() const { return (int)refcount.size(); }

  int32_t take() {
    int32_t b;
    if (!freed.empty()) {
      b = freed.back();
      freed.pop_back();
    } else {
      b = fresh.back();
      fresh.pop_back();
    }
    refcount[b] = 1;
    return b;
  }

  void release(int32_t b, int times = 1) {
    refcount[b] -= times;
    if (refcount[b] == 0) freed.push_back(b);
  }

  // Every count equals the references in `count`, and the free lists hold
  // exactly the blocks at 0, once each.
  bool consistent(const std::vector<int> &count) const {
    std::vector<int> listed(refcount.size(), 0);
    for (int32_t b : fresh) ++listed[b];
    for (int32_t b : freed) ++listed[b];
    for (size_t b = 0; b < refcount.size(); ++b) {
      if (count[b] != refcount[b]) return false;
      if (listed[b] != (count[b] == 0 ? 1 : 0)) return false;
    }
    return true;
  }
};

struct pa_manager {
  struct Sequence {
    std::vector<int32_t> blocks;  // device block ids, or host block ids when swapped
    int64_t length = 0;
    bool swapped = false;
  };

  int num_blocks = 0;
  int block_size = 0;
  BlockPool dev;    // the GPU pool
  BlockPool host;   // the CPU swap space (may be empty)
  std::unordered_map<int64_t, Sequence> seqs;

  int free_blocks() const { return dev.free_blocks(); }
  int32_t take() { return dev.take(); }
  void release(int32_t b) { dev.release(b); }

  // Fresh blocks and copies the appends of seqs[0..n) need, given the
  // current state; nothing is changed.  Returns false for an unknown or a
  // swapped-out id.
  bool plan(const int64_t *ids, int n, int *need, int *copies) const {
    std::unordered_map<int64_t, int64_t> length;   // lengths as the batch goes
    std::unordered_map<int64_t, bool> owned;       // last block private to the sequence
    std::unordered_map<int32_t, int> dropped;      // count decrements made so far
    *need = *copies = 0;
    for (int i = 0; i < n; ++i) {
      const auto it = seqs.find(ids[i]);
      if (it == seqs.end() || it->second.swapped) return false;
      const auto l = length.find(ids[i]);
      const int64_t len = l == length.end() ? it->second.length : l->second;
      if (len % block_size == 0) {
        ++*need;
        owned[ids[i]] = true;
      } else if (!owned[ids[i]]) {
        const int32_t last = it->second.blocks.back();
        if (dev.refcount[last] - dropped[last] > 1) {
          ++*need;
          ++*copies;
          ++dropped[last];
        }
        owned[ids[i]] = true;
      }
      length[ids[i]] = len + 1;
    }
    return true;
  }

  // Move the listed sequences' blocks from pool `from` to pool `to`: every
  // distinct block they reference gets one block of `to` (a block shared
  // inside the group is moved once and stays shared), reported as a
  // (from, to) pair; the group's references on `from` are dropped.  All or
  // nothing.  `want_swapped` is the state the sequences must be in.
  int move(const int64_t *ids, int n, bool want_swapped, BlockPool &from, BlockPool &to,
           int64_t *pairs, int max_pairs, int *num_pairs) {
    std::unordered_map<int32_t, int> refs;   // block of `from` -> references in the group
    std::vector<int32_t> order;              // distinct blocks, first appearance first
    for (int i = 0; i < n; ++i) {
      const auto it = seqs.find(ids[i]);
      if (it == seqs.end()) return PA_ERR_NO_SEQUENCE;
      if (it->second.swapped != want_swapped) return want_swapped ? PA_ERR_SHAPE : PA_ERR_SWAPPED;
      for (int k = 0; k < i; ++k)
        if (ids[k] == ids[i]) return PA_ERR_SHAPE;  // listed twice
      for (int32_t b : it->second.blocks)
        if (refs[b]++ == 0) order.push_back(b);
    }
    if ((int)order.size() > max_pairs) return PA_ERR_SHAPE;
    if ((int)order.size() > to.free_blocks()) return PA_ERR_NO_BLOCKS;
    std::unordered_map<int32_t, int32_t> moved;
    int p = 0;
    for (int32_t b : order) {
      const int32_t t = to.take();
      to.refcount[t] = refs[b];
      from.release(b, refs[b]);
      moved[b] = t;
      pairs[2 * p] = b;
      pairs[2 * p + 1] = t;
      ++p;
    }
    for (int i = 0; i < n; ++i) {
      Sequence &q = seqs[ids[i]];
      for (int32_t &b : q.blocks) b = moved[b];
      q.swapped = !want_swapped;
    }
    *num_pairs = p;
    return PA_OK;
  }
};

extern "C" {

pa_manager *pa_manager_create(int num_blocks, int block_size, int num_host_blocks,
                              const int32_t *alloc_order) {
  if (num_blocks <= 0 || block_size <= 0 || num_host_blocks < 0) return nullptr;
  if (alloc_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      const int32_t b = alloc_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) return nullptr;
      seen[b] = 1;
    }
  }
  pa_manager *m = new (std::nothrow) pa_manager;
  if (!m) return nullptr;
  try {
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->dev.init(num_blocks, alloc_order);
    m->host.init(num_host_blocks, nullptr);
  } catch (...) {
    delete m;
    return nullptr;
  }
  return m;
}

void pa_manager_destroy(pa_manager *m) { delete m; }

int pa_manager_add(pa_manager *m, int64_t seq) {
  if (!m) return PA_ERR_NULL;
  if (m->seqs.count(seq)) return PA_ERR_EXISTS;
  m->seqs[seq];
  return PA_OK;
}

int pa_manager_fork(pa_manager *m, int64_t parent, int64_t child) {
  if (!m) return PA_ERR_NULL;
  const auto p = m->seqs.find(parent);
  if (p == m->seqs.end()) return PA_ERR_NO_SEQUENCE;
  if (p->second.swapped) return PA_ERR_SWAPPED;
  if (m->seqs.count(child)) return PA_ERR_EXISTS;
  pa_manager::Sequence copy = p->second;
  for (int32_t b : copy.blocks) ++m->dev.refcount[b];
  m->seqs.emplace(child, std::move(copy));
  return PA_OK;
}

int pa_manager_append(pa_manager *m, const int64_t *seqs, int n, int64_t *slots,
                      int64_t *copy_pairs, int max_pairs, int *num_pairs) {
  if (!m || (n > 0 && (!seqs || !slots)) || !num_pairs) return PA_ERR_NULL;
  if (n < 0 || max_pairs < 0 || (max_pairs > 0 && !copy_pairs)) return PA_ERR_SHAPE;
  int need = 0, copies = 0;
  if (!m->plan(seqs, n, &need, &copies)) {
    for (int i = 0; i < n; ++i) {
      const auto it = m->seqs.find(seqs[i]);
      if (it != m->seqs.end() && it->second.swapped) return PA_ERR_SWAPPED;
    }
    return PA_ERR_NO_SEQUENCE;
  }
  if (copies > max_pairs) return PA_ERR_SHAPE;
  if (need > m->free_blocks()) return PA_ERR_NO_BLOCKS;
  const int B = m->block_size;
  int pairs = 0;
  for (int i = 0; i < n; ++i) {
    pa_manager::Sequence &q = m->seqs[seqs[i]];
    const int offset = (int)(q.length % B);
    int32_t block;
    if (offset == 0) {
      block = m->take();
      q.blocks.push_back(block);
    } else {
      block = q.blocks.back();
      if (m->dev.refcount[block] > 1) {  // shared: copy before writing
        const int32_t fresh = m->take();
        --m->dev.refcount[block];
        copy_pairs[2 * pairs] = block;
        copy_pairs[2 * pairs + 1] = fresh;
        ++pairs;
        q.blocks.back() = fresh;
        block = fresh;
      }
    }
    slots[i] = (int64_t)block * B + offset;
    ++q.length;
  }
  *num_pairs = pairs;
  return PA_OK;
}

int pa_manager_free(pa_manager *m, int64_t seq) {
  if (!m) return PA_ERR_NULL;
  const auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_NO_SEQUENCE;
  BlockPool &pool = it->second.swapped ? m->host : m->dev;
  for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) pool.release(*b);
  m->seqs.erase(it);
  return PA_OK;
}

int pa_manager_swap_out(pa_manager *m, const int64_t *seqs, int n, int64_t *pairs,
                        int max_pairs, int *num_pairs) {
  if (!m || (n > 0 && !seqs) || !num_pairs || (max_pairs > 0 && !pairs)) return PA_ERR_NULL;
  if (n < 0 || max_pairs < 0) return PA_ERR_SHAPE;
  return m->move(seqs, n, false, m->dev, m->host, pairs, max_pairs, num_pairs);
}

int pa_manager_swap_in(pa_manager *m, const int64_t *seqs, int n, int64_t *pairs,
                       int max_pairs, int *num_pairs) {
  if (!m || (n > 0 && !seqs) || !num_pairs || (max_pairs > 0 && !pairs)) return PA_ERR_NULL;
  if (n < 0 || max_pairs < 0) return PA_ERR_SHAPE;
  return m->move(seqs, n, true, m->host, m->dev, pairs, max_pairs, num_pairs);
}

int pa_manager_num_free_host(const pa_manager *m) {
  return m ? m->host.free_blocks() : PA_ERR_NULL;
}

int pa_manager_is_swapped(const pa_manager *m, int64_t seq) {
  if (!m) return PA_ERR_NULL;
  const auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_NO_SEQUENCE;
  return it->second.swapped ? 1 : 0;
}

int pa_manager_tables(const pa_manager *m, const int64_t *seqs, int n, int32_t *tables,
                      int max_blocks, int32_t *context_lens) {
  if (!m || (n > 0 && (!seqs || !tables || !context_lens))) return PA_ERR_NULL;
  if (n < 0 || max_blocks <= 0) return PA_ERR_SHAPE;
  for (int i = 0; i < n; ++i) {
    const auto it = m->seqs.find(seqs[i]);
    if (it == m->seqs.end()) return PA_ERR_NO_SEQUENCE;
    if (it->second.swapped) return PA_ERR_SWAPPED;
    if ((int64_t)it->second.blocks.size() > max_blocks || it->second.length > INT32_MAX)
      return PA_ERR_SHAPE;
  }
  for (int i = 0; i < n; ++i) {
    const pa_manager::Sequence &q = m->seqs.find(seqs[i])->second;
    int32_t *row = tables + (int64_t)i * max_blocks;
    std::fill(row, row + max_blocks, -1);
    std::copy(q.blocks.begin(), q.blocks.end(), row);
    context_lens[i] = (int32_t)q.length;
  }
  return PA_OK;
}

int pa_manager_num_free(const pa_manager *m) { return m ? m->free_blocks() : PA_ERR_NULL; }

int pa_manager_num_sequences(const pa_manager *m) {
  return m ? (int)m->seqs.size() : PA_ERR_NULL;
}

int pa_manager_refcount(const pa_manager *m, int block) {
  if (!m) return PA_ERR_NULL;
  if (block < 0 || block >= m->num_blocks) return PA_ERR_SHAPE;
  return m->dev.refcount[block];
}

int pa_manager_length(const pa_manager *m, int64_t seq) {
  if (!m) return PA_ERR_NULL;
  const auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_NO_SEQUENCE;
  return it->second.length > INT32_MAX ? PA_ERR_SHAPE : (int)it->second.length;
}

int pa_manager_check(const pa_manager *m) {
  if (!m) return PA_ERR_NULL;
  std::vector<int> dev_count(m->dev.size(), 0), host_count(m->host.size(), 0);
  for (const auto &kv : m->seqs) {
    const pa_manager::Sequence &q = kv.second;
    const int64_t want = (q.length + m->block_size - 1) / m->block_size;
    if ((int64_t)q.blocks.size() != want) return PA_ERR_SHAPE;
    std::vector<int> &count = q.swapped ? host_count : dev_count;
    for (int32_t b : q.blocks) {
      if (b < 0 || b >= (int)count.size()) return PA_ERR_SHAPE;
      ++count[b];
    }
  }
  if (!m->dev.consistent(dev_count) || !m->host.consistent(host_count)) return PA_ERR_SHAPE;
  return PA_OK;
}

}  // extern "C"
