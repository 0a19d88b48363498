// Host-side block pool: the refcounted free list behind the block tables.
//
// One layer's cache is a pool of fixed-size physical blocks shared by every session
// ("PagedAttention por dentro...", section "El pool de bloques": the pool is one global
// resource, not per session).  A block is free or allocated with a reference count:
//   * allocation takes blocks off the free list with count 1 (a request admitted or
//     grown by a block);
//   * sharing adds a reference (prefix caching, or the branches of parallel sampling /
//     beam search pointing their tables at the same block: "La despensa por
//     casilleros", section "Prefix caching: compartir casilleros con copy-on-write");
//   * release drops one; the block returns to the free list at zero (a request ends,
//     or its blocks were swapped out or evicted);
//   * copy-on-write: before a sequence writes into a block, a block shared with others
//     is replaced by a fresh private block (the caller copies the contents with
//     paged_kv_copy_blocks) and the shared one loses that reference.
// Accounting holds after every call: free + allocated == pool size, and every
// allocated block has a count >= 1 (the invariants of "Capitulo 2", section "Evals
// deterministas para esta capa").  A call that would break a rule (too few free blocks,
// an ID out of range or not allocated) changes nothing and returns an error.
#include <mutex>
#include <new>
#include <vector>

#include "pagedkv.h"

struct pkv_block_pool {
  std::mutex mu;
  std::vector<int32_t> refcount;  // 0 = free
  std::vector<int32_t> free_list;  // a stack: the most recently freed block is reused first
};

namespace {
bool valid(const pkv_block_pool* p, int32_t id) { return id >= 0 && (size_t)id < p->refcount.size(); }
}  // namespace

extern "C" {

pkv_block_pool* pkv_pool_create(int32_t num_blocks) {
  if (num_blocks <= 0) return nullptr;
  pkv_block_pool* p = new (std::nothrow) pkv_block_pool;
  if (!p) return nullptr;
  try {
    p->refcount.assign((size_t)num_blocks, 0);
    p->free_list.resize((size_t)num_blocks);
  } catch (...) {
    delete p;
    return nullptr;
  }
  for (int32_t i = 0; i < num_blocks; ++i) p->free_list[(size_t)i] = num_blocks - 1 - i;  // block 0 first
  return p;
}

void pkv_pool_destroy(pkv_block_pool* p) { delete p; }

int pkv_pool_alloc(pkv_block_pool* p, int32_t n, int32_t* ids_out) {
  if (!p || (n > 0 && !ids_out)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  std::lock_guard<std::mutex> g(p->mu);
  if ((size_t)n > p->free_list.size()) return PKV_ERR_POOL_EXHAUSTED;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = p->free_list.back();
    p->free_list.pop_back();
    p->refcount[(size_t)id] = 1;
    ids_out[i] = id;
  }
  return PKV_OK;
}

int pkv_pool_share(pkv_block_pool* p, const int32_t* ids, int32_t n) {
  if (!p || (n > 0 && !ids)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  std::lock_guard<std::mutex> g(p->mu);
  for (int32_t i = 0; i < n; ++i)
    if (!valid(p, ids[i]) || p->refcount[(size_t)ids[i]] == 0) return PKV_ERR_BLOCK_STATE;
  for (int32_t i = 0; i < n; ++i) ++p->refcount[(size_t)ids[i]];
  return PKV_OK;
}

int pkv_pool_release(pkv_block_pool* p, const int32_t* ids, int32_t n) {
  if (!p || (n > 0 && !ids)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  std::lock_guard<std::mutex> g(p->mu);
  // all or nothing: count the releases of each ID first (an ID may repeat)
  std::vector<int32_t> drop;
  try {
    drop.assign(p->refcount.size(), 0);
  } catch (...) {
    return PKV_ERR_NULL;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (!valid(p, ids[i])) return PKV_ERR_BLOCK_STATE;
    if (++drop[(size_t)ids[i]] > p->refcount[(size_t)ids[i]]) return PKV_ERR_BLOCK_STATE;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t& c = p->refcount[(size_t)ids[i]];
    if (--c == 0) p->free_list.push_back(ids[i]);
  }
  return PKV_OK;
}

int pkv_pool_cow(pkv_block_pool* p, int32_t id, int32_t* id_out) {
  if (!p || !id_out) return PKV_ERR_NULL;
  std::lock_guard<std::mutex> g(p->mu);
  if (!valid(p, id) || p->refcount[(size_t)id] == 0) return PKV_ERR_BLOCK_STATE;
  if (p->refcount[(size_t)id] == 1) {  // private already: write in place
    *id_out = id;
    return 0;
  }
  if (p->free_list.empty()) return PKV_ERR_POOL_EXHAUSTED;
  const int32_t fresh = p->free_list.back();
  p->free_list.pop_back();
  p->refcount[(size_t)fresh] = 1;
  --p->refcount[(size_t)id];
  *id_out = fresh;
  return 1;
}

int32_t pkv_pool_free_count(pkv_block_pool* p) {
  if (!p) return PKV_ERR_NULL;
  std::lock_guard<std::mutex> g(p->mu);
  return (int32_t)p->free_list.size();
}

int32_t pkv_pool_refcount(pkv_block_pool* p, int32_t id) {
  if (!p) return PKV_ERR_NULL;
  std::lock_guard<std::mutex> g(p->mu);
  if (!valid(p, id)) return PKV_ERR_BLOCK_STATE;
  return p->refcount[(size_t)id];
}

}  // extern "C"
