// Host-side KV block manager (include/pa_manager.h): free blocks,
// per-block reference counts, per-sequence block lists and lengths.  It
// turns "sequence s gets one more token" into a slot, allocating a block
// only when the last one is full and copying a shared last block before it
// is written (the KV cache manager, reference counts and copy-on-write of
// the wywy.jp notes on PagedAttention, Keyword section and WHERE parallel
// sampling; the memory-management table of the zhaifeiyue.github.io
// summary).
#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_manager.h"

struct pa_manager {
  struct Sequence {
    std::vector<int32_t> blocks;
    int64_t length = 0;
  };

  int num_blocks = 0;
  int block_size = 0;
  std::vector<int> refcount;    // per physical block
  std::vector<int32_t> fresh;   // never handed out; taken from the back
  std::vector<int32_t> freed;   // returned blocks; most recent at the back
  std::unordered_map<int64_t, Sequence> seqs;

  int free_blocks() const { return (int)(fresh.size() + freed.size()); }

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

  void release(int32_t b) {
    if (--refcount[b] == 0) freed.push_back(b);
  }

  // Fresh blocks and copies the appends of seqs[0..n) need, given the
  // current state; nothing is changed.  Returns false for an unknown id.
  bool plan(const int64_t *ids, int n, int *need, int *copies) const {
    std::unordered_map<int64_t, int64_t> length;   // lengths as the batch goes
    std::unordered_map<int64_t, bool> owned;       // last block private to the sequence
    std::unordered_map<int32_t, int> dropped;      // count decrements made so far
    *need = *copies = 0;
    for (int i = 0; i < n; ++i) {
      const auto it = seqs.find(ids[i]);
      if (it == seqs.end()) return false;
      const auto l = length.find(ids[i]);
      const int64_t len = l == length.end() ? it->second.length : l->second;
      if (len % block_size == 0) {
        ++*need;
        owned[ids[i]] = true;
      } else if (!owned[ids[i]]) {
        const int32_t last = it->second.blocks.back();
        if (refcount[last] - dropped[last] > 1) {
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
};

extern "C" {

pa_manager *pa_manager_create(int num_blocks, int block_size, const int32_t *alloc_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pa_manager *m = new (std::nothrow) pa_manager;
  if (!m) return nullptr;
  try {
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->refcount.assign(num_blocks, 0);
    m->fresh.resize(num_blocks);
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      const int32_t b = alloc_order ? alloc_order[i] : i;
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete m;
        return nullptr;
      }
      seen[b] = 1;
      m->fresh[num_blocks - 1 - i] = b;  // the back is handed out first
    }
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
  if (m->seqs.count(child)) return PA_ERR_EXISTS;
  pa_manager::Sequence copy = p->second;
  for (int32_t b : copy.blocks) ++m->refcount[b];
  m->seqs.emplace(child, std::move(copy));
  return PA_OK;
}

int pa_manager_append(pa_manager *m, const int64_t *seqs, int n, int64_t *slots,
                      int64_t *copy_pairs, int max_pairs, int *num_pairs) {
  if (!m || (n > 0 && (!seqs || !slots)) || !num_pairs) return PA_ERR_NULL;
  if (n < 0 || max_pairs < 0 || (max_pairs > 0 && !copy_pairs)) return PA_ERR_SHAPE;
  int need = 0, copies = 0;
  if (!m->plan(seqs, n, &need, &copies)) return PA_ERR_NO_SEQUENCE;
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
      if (m->refcount[block] > 1) {  // shared: copy before writing
        const int32_t fresh = m->take();
        --m->refcount[block];
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
  for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) m->release(*b);
  m->seqs.erase(it);
  return PA_OK;
}

int pa_manager_tables(const pa_manager *m, const int64_t *seqs, int n, int32_t *tables,
                      int max_blocks, int32_t *context_lens) {
  if (!m || (n > 0 && (!seqs || !tables || !context_lens))) return PA_ERR_NULL;
  if (n < 0 || max_blocks <= 0) return PA_ERR_SHAPE;
  for (int i = 0; i < n; ++i) {
    const auto it = m->seqs.find(seqs[i]);
    if (it == m->seqs.end()) return PA_ERR_NO_SEQUENCE;
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
  return m->refcount[block];
}

int pa_manager_length(const pa_manager *m, int64_t seq) {
  if (!m) return PA_ERR_NULL;
  const auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_NO_SEQUENCE;
  return it->second.length > INT32_MAX ? PA_ERR_SHAPE : (int)it->second.length;
}

int pa_manager_check(const pa_manager *m) {
  if (!m) return PA_ERR_NULL;
  std::vector<int> count(m->num_blocks, 0);
  for (const auto &kv : m->seqs) {
    const pa_manager::Sequence &q = kv.second;
    const int64_t want = (q.length + m->block_size - 1) / m->block_size;
    if ((int64_t)q.blocks.size() != want) return PA_ERR_SHAPE;
    for (int32_t b : q.blocks) {
      if (b < 0 || b >= m->num_blocks) return PA_ERR_SHAPE;
      ++count[b];
    }
  }
  std::vector<int> listed(m->num_blocks, 0);
  for (int32_t b : m->fresh) ++listed[b];
  for (int32_t b : m->freed) ++listed[b];
  for (int b = 0; b < m->num_blocks; ++b) {
    if (count[b] != m->refcount[b]) return PA_ERR_SHAPE;
    if (listed[b] != (count[b] == 0 ? 1 : 0)) return PA_ERR_SHAPE;
  }
  return PA_OK;
}

}  // extern "C"
