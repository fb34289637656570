// Host-side allocator of classical-cache blocks for the paged decode cache
// (AirCoding "deepseek-paper-analysis" section 7.6: the classical cache is
// a set of blocks allocated per request).  A pool hands out block ids
// 0 .. n_blocks-1 and takes them back; it never touches device memory, so a
// caller keeps one pool per device block array.  Free ids are kept on a
// stack (the most recently released block is reused first).  Every call is
// serialised by the pool's mutex.
#include <stdint.h>

#include <mutex>
#include <new>
#include <vector>

#include "csa.h"

struct csa_block_pool {
  std::mutex mu;
  std::vector<int32_t> free_ids;
  std::vector<uint8_t> in_use;
};

extern "C" {

csa_block_pool* csa_block_pool_create(int64_t n_blocks) {
  if (n_blocks < 1 || n_blocks > 2147483647LL) return nullptr;
  csa_block_pool* p = new (std::nothrow) csa_block_pool;
  if (!p) return nullptr;
  try {
    p->free_ids.resize((size_t)n_blocks);
    p->in_use.assign((size_t)n_blocks, 0);
  } catch (...) {
    delete p;
    return nullptr;
  }
  // lowest ids on top of the stack
  for (int64_t i = 0; i < n_blocks; ++i) p->free_ids[(size_t)i] = (int32_t)(n_blocks - 1 - i);
  return p;
}

void csa_block_pool_destroy(csa_block_pool* pool) { delete pool; }

int csa_block_pool_alloc(csa_block_pool* pool, int64_t n, int32_t* ids) {
  if (!pool || n < 0 || (n > 0 && !ids)) return CSA_EINVAL;
  std::lock_guard<std::mutex> lock(pool->mu);
  if ((size_t)n > pool->free_ids.size()) return CSA_ENOSPC;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t id = pool->free_ids.back();
    pool->free_ids.pop_back();
    pool->in_use[(size_t)id] = 1;
    ids[i] = id;
  }
  return CSA_OK;
}

int csa_block_pool_release(csa_block_pool* pool, int64_t n, const int32_t* ids) {
  if (!pool || n < 0 || (n > 0 && !ids)) return CSA_EINVAL;
  std::lock_guard<std::mutex> lock(pool->mu);
  // all or nothing: every id must be allocated, and none listed twice
  std::vector<int32_t> seen;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || (size_t)id >= pool->in_use.size() || pool->in_use[(size_t)id] != 1) {
      for (int32_t s : seen) pool->in_use[(size_t)s] = 1;
      return CSA_EINVAL;
    }
    pool->in_use[(size_t)id] = 2;   // marked for release
    seen.push_back(id);
  }
  for (int32_t id : seen) {
    pool->in_use[(size_t)id] = 0;
    pool->free_ids.push_back(id);
  }
  return CSA_OK;
}

int64_t csa_block_pool_available(csa_block_pool* pool) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  return (int64_t)pool->free_ids.size();
}

}  // extern "C"
