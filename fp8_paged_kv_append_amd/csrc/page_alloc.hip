// Host-side page allocator with the page tags of the integrity check.
//
// The pages (agentlenshq summary of the Cloudflare post, section "KV Cache 完整性检查";
// xujun.org note, section "一个不能出错的共享缓存"): every physical page of the cache carries a
// tag that changes when the page is given to a new owner; a request that still holds the old
// (page, tag) pair fails the next batched check and is aborted instead of reading someone else's
// data.  Here the tag is a uint32 generation counter bumped (mod 2^32) each time the page is
// allocated; freeing leaves it alone.  The free list is a stack: the page freed last is handed out
// first, and a fresh allocator hands out pages 0, 1, 2, ... in order.
//
// The state lives in a caller-owned host buffer (no allocation, no HIP call, not thread-safe):
//   header | tags[P] (uint32) | stack[P] (int32, free pages, top at stack[free-1]) | used[P] (uint8)
#include <stdint.h>
#include <string.h>

#include "kvfp8.h"

namespace {

struct AllocHeader {
  uint32_t magic;
  int32_t num_pages;
  int32_t free_count;
  int32_t pad;
};
constexpr uint32_t kMagic = 0x6b763870u;  // "kv8p"

size_t state_bytes(int32_t P) {
  return sizeof(AllocHeader) + (size_t)P * (sizeof(uint32_t) + sizeof(int32_t) + 1);
}

struct View {
  AllocHeader* h;
  uint32_t* tags;
  int32_t* stack;
  uint8_t* used;
};

bool view_of(void* state, View& v) {
  if (state == nullptr) return false;
  v.h = static_cast<AllocHeader*>(state);
  if (v.h->magic != kMagic || v.h->num_pages < 1) return false;
  const int32_t P = v.h->num_pages;
  uint8_t* base = static_cast<uint8_t*>(state) + sizeof(AllocHeader);
  v.tags = reinterpret_cast<uint32_t*>(base);
  v.stack = reinterpret_cast<int32_t*>(base + (size_t)P * sizeof(uint32_t));
  v.used = base + (size_t)P * (sizeof(uint32_t) + sizeof(int32_t));
  return true;
}

}  // namespace

extern "C" {

size_t kv_page_alloc_state_bytes(int32_t num_pages) { return num_pages < 1 ? 0 : state_bytes(num_pages); }

int kv_page_alloc_init(void* state, size_t state_bytes_given, int32_t num_pages, const uint32_t* initial_tags) {
  if (state == nullptr) return KVFP8_ERR_NULL;
  if (num_pages < 1) return KVFP8_ERR_SHAPE;
  if (state_bytes_given < state_bytes(num_pages)) return KVFP8_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(state) % 4 != 0) return KVFP8_ERR_ALIGN;
  AllocHeader* h = static_cast<AllocHeader*>(state);
  h->magic = kMagic;
  h->num_pages = num_pages;
  h->free_count = num_pages;
  h->pad = 0;
  View v;
  view_of(state, v);
  for (int32_t p = 0; p < num_pages; ++p) {
    v.tags[p] = initial_tags ? initial_tags[p] : 0u;
    v.stack[p] = num_pages - 1 - p;  // the top of the stack is page 0
    v.used[p] = 0;
  }
  return KVFP8_OK;
}

int32_t kv_page_alloc_free_count(const void* state) {
  View v;
  if (!view_of(const_cast<void*>(state), v)) return -1;
  return v.h->free_count;
}

int kv_page_alloc(void* state, int32_t n, int32_t* pages, uint32_t* tags) {
  View v;
  if (!view_of(state, v)) return KVFP8_ERR_NULL;
  if (n < 0) return KVFP8_ERR_SHAPE;
  if (n == 0) return KVFP8_OK;
  if (pages == nullptr) return KVFP8_ERR_NULL;
  if (n > v.h->free_count) return KVFP8_ERR_NOSPACE;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = v.stack[--v.h->free_count];
    v.used[p] = 1;
    v.tags[p] += 1u;  // a new owner: the old holders' (page, tag) pairs no longer match
    pages[i] = p;
    if (tags) tags[i] = v.tags[p];
  }
  return KVFP8_OK;
}

int kv_page_free(void* state, const int32_t* pages, int32_t n) {
  View v;
  if (!view_of(state, v)) return KVFP8_ERR_NULL;
  if (n < 0) return KVFP8_ERR_SHAPE;
  if (n == 0) return KVFP8_OK;
  if (pages == nullptr) return KVFP8_ERR_NULL;
  // validate everything first (no partial free): in range, allocated, not listed twice
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = pages[i];
    if (p < 0 || p >= v.h->num_pages || v.used[p] != 1) {
      for (int32_t j = 0; j < i; ++j) v.used[pages[j]] = 1;  // undo the marks of this scan
      return KVFP8_ERR_VALUE;
    }
    v.used[p] = 2;  // marked in this call
  }
  for (int32_t i = 0; i < n; ++i) {
    v.used[pages[i]] = 0;
    v.stack[v.h->free_count++] = pages[i];
  }
  return KVFP8_OK;
}

int kv_page_alloc_tags(const void* state, uint32_t* tags) {
  View v;
  if (!view_of(const_cast<void*>(state), v) || tags == nullptr) return KVFP8_ERR_NULL;
  memcpy(tags, v.tags, (size_t)v.h->num_pages * sizeof(uint32_t));
  return KVFP8_OK;
}

}  // extern "C"
