// block_manager.cpp — host block manager of the paged KV cache (pa_bm_* in include/pa.h).
//
// It keeps the free list of physical blocks, a reference count per block and one block table per
// sequence, and produces the per-step metadata the kernels consume:
//  * a block is taken from the free list only when a sequence's last block is full ("LLM Inference
//    Visualizer, Lesson 06", "How paging grows"; "PagedAttention" (devoured.fyi), OS-to-paging
//    table, allocate a new block on demand);
//  * finished sequences give their blocks back ("PagedAttention" (devoured.fyi), "PagedAttention in
//    one picture");
//  * fork shares every block, counts +1 ("PagedAttention, Visualized", Part 3, shared prefix
//    blocks and copy-on-write after fork);
//  * a write into a block with count > 1 clones it, decrements the original and retargets the
//    writer's table ("PagedAttention" (devoured.fyi), "Copy-on-write: when two requests share a
//    prefix").  The clone itself is pa_copy_blocks on the device.
//  * swapping a sequence out evicts its blocks to CPU memory, except the shared ones, which stay
//    because another sequence still needs them ("PagedAttention, Visualized", Part 3, the OS table's
//    swapping to disk and the paragraph after it).  The sequence keeps its reference to a shared
//    block, so the block cannot be freed while the sequence is out.  Swapping it in takes a fresh
//    device block for every host slot.  The moves themselves are pa_swap_blocks on the device.
// The free lists (device blocks and host slots) are stacks: the initial order is handed out front
// to back (host slots 0, 1, 2, ...) and a freed entry is the next one handed out.
#include <new>
#include <vector>

#include "pa.h"

struct pa_bm {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> ref;
  std::vector<std::vector<int32_t>> tables;
  std::vector<int32_t> lens;
  std::vector<char> alive;
  // swapping: the host slot stack; per sequence whether it is swapped out and, if so, which of its
  // table entries are host slots
  int32_t num_host = 0;
  std::vector<int32_t> host_free;  // top = back()
  std::vector<char> out;
  std::vector<std::vector<char>> on_host;
};

namespace {

bool valid_seq(const pa_bm *bm, int32_t s) {
  return bm && s >= 0 && (size_t)s < bm->alive.size() && bm->alive[(size_t)s];
}

int32_t new_seq(pa_bm *bm) {
  bm->tables.emplace_back();
  bm->lens.push_back(0);
  bm->alive.push_back(1);
  bm->out.push_back(0);
  bm->on_host.emplace_back();
  return (int32_t)bm->tables.size() - 1;
}

bool swapped(const pa_bm *bm, int32_t s) { return bm->out[(size_t)s] != 0; }

bool resident_seq(const pa_bm *bm, int32_t s) { return valid_seq(bm, s) && !swapped(bm, s); }

int32_t take(pa_bm *bm) {
  const int32_t b = bm->free_stack.back();
  bm->free_stack.pop_back();
  bm->ref[(size_t)b] = 1;
  return b;
}

}  // namespace

extern "C" {

pa_bm *pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t *free_order) {
  if (num_blocks < 0 || block_size < 1) return nullptr;
  pa_bm *bm = new (std::nothrow) pa_bm;
  if (!bm) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->ref.assign((size_t)num_blocks, 0);
    bm->free_stack.resize((size_t)num_blocks);
    std::vector<char> seen((size_t)num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order ? free_order[i] : i;
      if (b < 0 || b >= num_blocks || seen[(size_t)b]) {
        delete bm;
        return nullptr;  // not a permutation
      }
      seen[(size_t)b] = 1;
      bm->free_stack[(size_t)(num_blocks - 1 - i)] = b;  // free_order[0] on top
    }
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pa_bm_destroy(pa_bm *bm) { delete bm; }

pa_status pa_bm_add_seq(pa_bm *bm, int32_t *seq_id) {
  if (!bm || !seq_id) return PA_ERR_NULL;
  *seq_id = new_seq(bm);
  return PA_OK;
}

pa_status pa_bm_fork(pa_bm *bm, int32_t parent, int32_t *child) {
  if (!bm || !child) return PA_ERR_NULL;
  if (!resident_seq(bm, parent)) return PA_ERR_STATE;
  const int32_t c = new_seq(bm);
  bm->tables[(size_t)c] = bm->tables[(size_t)parent];
  bm->lens[(size_t)c] = bm->lens[(size_t)parent];
  for (int32_t b : bm->tables[(size_t)c]) bm->ref[(size_t)b] += 1;
  *child = c;
  return PA_OK;
}

pa_status pa_bm_append(pa_bm *bm, int32_t seq, int64_t *slot, int32_t *cow_src, int32_t *cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return PA_ERR_NULL;
  if (!resident_seq(bm, seq)) return PA_ERR_STATE;
  std::vector<int32_t> &t = bm->tables[(size_t)seq];
  const int32_t L = bm->lens[(size_t)seq];
  const int32_t j = L / bm->block_size, off = L % bm->block_size;
  *cow_src = *cow_dst = -1;
  if (off == 0) {
    if (bm->free_stack.empty()) return PA_ERR_NO_BLOCKS;
    t.push_back(take(bm));
  } else {
    const int32_t last = t[(size_t)j];
    if (bm->ref[(size_t)last] > 1) {
      if (bm->free_stack.empty()) return PA_ERR_NO_BLOCKS;
      const int32_t dst = take(bm);   // clone target
      bm->ref[(size_t)last] -= 1;     // the original loses this writer
      t[(size_t)j] = dst;             // the writer points at the clone
      *cow_src = last;
      *cow_dst = dst;
    }
  }
  bm->lens[(size_t)seq] = L + 1;
  *slot = (int64_t)t[(size_t)j] * bm->block_size + off;
  return PA_OK;
}

pa_status pa_bm_append_batch(pa_bm *bm, const int32_t *seqs, int32_t n, int64_t *slots,
                             int32_t *cow_pairs, int32_t *num_pairs) {
  if (!bm || !num_pairs || (n > 0 && (!seqs || !slots || !cow_pairs))) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  *num_pairs = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    const pa_status st = pa_bm_append(bm, seqs[i], &slots[i], &src, &dst);
    if (st != PA_OK) return st;
    if (src >= 0) {
      cow_pairs[2 * *num_pairs] = src;
      cow_pairs[2 * *num_pairs + 1] = dst;
      *num_pairs += 1;
    }
  }
  return PA_OK;
}

pa_status pa_bm_free_seq(pa_bm *bm, int32_t seq) {
  if (!bm) return PA_ERR_NULL;
  if (!valid_seq(bm, seq)) return PA_ERR_STATE;
  const bool is_out = swapped(bm, seq);
  const std::vector<char> &where = bm->on_host[(size_t)seq];
  const std::vector<int32_t> &t = bm->tables[(size_t)seq];
  for (size_t j = 0; j < t.size(); ++j) {
    if (is_out && where[j]) bm->host_free.push_back(t[j]);
    else if (--bm->ref[(size_t)t[j]] == 0) bm->free_stack.push_back(t[j]);
  }
  bm->out[(size_t)seq] = 0;
  bm->on_host[(size_t)seq].clear();
  bm->tables[(size_t)seq].clear();
  bm->tables[(size_t)seq].shrink_to_fit();
  bm->lens[(size_t)seq] = 0;
  bm->alive[(size_t)seq] = 0;
  return PA_OK;
}

int32_t pa_bm_refcount(const pa_bm *bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[(size_t)block];
}

int32_t pa_bm_num_free(const pa_bm *bm) { return bm ? (int32_t)bm->free_stack.size() : -1; }

int32_t pa_bm_seq_len(const pa_bm *bm, int32_t seq) {
  return valid_seq(bm, seq) ? bm->lens[(size_t)seq] : -1;
}

pa_status pa_bm_set_host_blocks(pa_bm *bm, int32_t num_host_blocks) {
  if (!bm) return PA_ERR_NULL;
  if (num_host_blocks < 0) return PA_ERR_SHAPE;
  for (size_t s = 0; s < bm->out.size(); ++s)
    if (bm->alive[s] && bm->out[s]) return PA_ERR_STATE;  // slots in use
  try {
    bm->host_free.resize((size_t)num_host_blocks);
  } catch (...) {
    return PA_ERR_SHAPE;
  }
  for (int32_t i = 0; i < num_host_blocks; ++i)
    bm->host_free[(size_t)(num_host_blocks - 1 - i)] = i;  // slot 0 on top
  bm->num_host = num_host_blocks;
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_bm *bm, int32_t seq, int32_t *pairs, int32_t cap,
                         int32_t *num_pairs) {
  if (!bm || !num_pairs || (cap > 0 && !pairs)) return PA_ERR_NULL;
  if (!resident_seq(bm, seq)) return PA_ERR_STATE;
  std::vector<int32_t> &t = bm->tables[(size_t)seq];
  int32_t need = 0;
  for (int32_t b : t) need += bm->ref[(size_t)b] == 1;
  *num_pairs = need;
  if (need > cap) return PA_ERR_SHAPE;  // nothing changed
  if ((size_t)need > bm->host_free.size()) return PA_ERR_NO_BLOCKS;
  std::vector<char> where(t.size(), 0);
  int32_t k = 0;
  for (size_t j = 0; j < t.size(); ++j) {
    const int32_t b = t[j];
    if (bm->ref[(size_t)b] != 1) continue;  // shared: stays on the device
    const int32_t h = bm->host_free.back();
    bm->host_free.pop_back();
    pairs[2 * k] = b;
    pairs[2 * k + 1] = h;
    ++k;
    bm->ref[(size_t)b] = 0;
    bm->free_stack.push_back(b);
    t[j] = h;
    where[j] = 1;
  }
  bm->on_host[(size_t)seq] = std::move(where);
  bm->out[(size_t)seq] = 1;
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_bm *bm, int32_t seq, int32_t *pairs, int32_t cap, int32_t *num_pairs) {
  if (!bm || !num_pairs || (cap > 0 && !pairs)) return PA_ERR_NULL;
  if (!valid_seq(bm, seq) || !swapped(bm, seq)) return PA_ERR_STATE;
  std::vector<int32_t> &t = bm->tables[(size_t)seq];
  const std::vector<char> &where = bm->on_host[(size_t)seq];
  int32_t need = 0;
  for (size_t j = 0; j < t.size(); ++j) need += where[j];
  *num_pairs = need;
  if (need > cap) return PA_ERR_SHAPE;  // nothing changed
  if ((size_t)need > bm->free_stack.size()) return PA_ERR_NO_BLOCKS;
  int32_t k = 0;
  for (size_t j = 0; j < t.size(); ++j) {
    if (!where[j]) continue;
    const int32_t h = t[j];
    const int32_t b = take(bm);
    pairs[2 * k] = b;
    pairs[2 * k + 1] = h;
    ++k;
    bm->host_free.push_back(h);
    t[j] = b;
  }
  bm->out[(size_t)seq] = 0;
  bm->on_host[(size_t)seq].clear();
  return PA_OK;
}

int32_t pa_bm_num_free_host(const pa_bm *bm) { return bm ? (int32_t)bm->host_free.size() : -1; }

int32_t pa_bm_is_swapped(const pa_bm *bm, int32_t seq) {
  return valid_seq(bm, seq) ? (swapped(bm, seq) ? 1 : 0) : -1;
}

pa_status pa_bm_block_table(const pa_bm *bm, int32_t seq, int32_t *out, int32_t cap,
                            int32_t *num_blocks) {
  if (!bm || !num_blocks || (cap > 0 && !out)) return PA_ERR_NULL;
  if (!valid_seq(bm, seq)) return PA_ERR_STATE;
  const std::vector<int32_t> &t = bm->tables[(size_t)seq];
  *num_blocks = (int32_t)t.size();
  for (int32_t i = 0; i < cap && (size_t)i < t.size(); ++i) out[i] = t[(size_t)i];
  return PA_OK;
}

pa_status pa_bm_export(const pa_bm *bm, const int32_t *seqs, int32_t n, int32_t *tables,
                       int32_t max_blocks_per_seq, int32_t pad_value, int32_t *context_lens) {
  if (!bm || (n > 0 && (!seqs || !tables || !context_lens))) return PA_ERR_NULL;
  if (n < 0 || max_blocks_per_seq < 0) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    if (!resident_seq(bm, seqs[i])) return PA_ERR_STATE;
    const std::vector<int32_t> &t = bm->tables[(size_t)seqs[i]];
    if ((int64_t)t.size() > max_blocks_per_seq) return PA_ERR_SHAPE;
    int32_t *row = tables + (size_t)i * max_blocks_per_seq;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j)
      row[j] = (size_t)j < t.size() ? t[(size_t)j] : pad_value;
    context_lens[i] = bm->lens[(size_t)seqs[i]];
  }
  return PA_OK;
}

}  // extern "C"
