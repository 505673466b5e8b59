// Host page allocator of the paged KV cache (C ABI in include/mla.h).
//
// The "Flash MLA: efficient MLA decoding kernel library for variable-length
// sequences" page (developer.baidu.com, §三.1) manages the cache with two
// levels of page tables: a global one over the physical pages and one table
// per sequence, a sequence of n tokens needing ceil(n / page_size) pages, pages
// taken as the sequence grows and returned when it ends (§四, steps 2 and 5).
// Here the per-sequence tables are the rows of the decode's block_table
// [max_seqs, max_blocks] and the global table is the owner of every physical
// page plus a stack of the free ones.  All of it lives in one caller-owned
// host buffer; nothing here touches the GPU, and the block table is copied to
// the device by the caller.
//
// Policy: free pages form a stack; a new sequence takes ascending ids from a
// fresh pool, and pages a sequence returns are reused first (last freed, first
// taken), which keeps recently used pages hot.
#include <cstdint>
#include <cstring>

#include "mla.h"
#include "mla_kernels.h"

namespace {

constexpr int32_t kMagic = 0x4d4c4150;  // "MLAP"

struct Header {
  int32_t magic, num_pages, max_seqs, max_blocks, free_top, pad[3];
};
// layout after the header: free stack [num_pages], owner [num_pages],
// pages per sequence [max_seqs], block table [max_seqs * max_blocks]

int32_t* free_stack(Header* h) { return reinterpret_cast<int32_t*>(h + 1); }
int32_t* owner(Header* h) { return free_stack(h) + h->num_pages; }
int32_t* npages(Header* h) { return owner(h) + h->num_pages; }
int32_t* table(Header* h) { return npages(h) + h->max_seqs; }

Header* state_of(void* s) {
  Header* h = static_cast<Header*>(s);
  return (h && h->magic == kMagic) ? h : nullptr;
}

int pager_fail(int code, const char* msg) { return mla::set_status(code, msg); }

}  // namespace

extern "C" {

size_t mla_pager_bytes(int num_pages, int max_seqs, int max_blocks) {
  if (num_pages <= 0 || max_seqs <= 0 || max_blocks <= 0) return 0;
  return sizeof(Header) +
         4u * (2u * (size_t)num_pages + (size_t)max_seqs + (size_t)max_seqs * (size_t)max_blocks);
}

int mla_pager_init(void* state, size_t bytes, int num_pages, int max_seqs, int max_blocks) {
  if (!state) return pager_fail(MLA_ERR_INVALID, "pager: null state");
  if (reinterpret_cast<uintptr_t>(state) % alignof(int32_t))
    return pager_fail(MLA_ERR_INVALID, "pager: state must be 4-byte aligned");
  const size_t need = mla_pager_bytes(num_pages, max_seqs, max_blocks);
  if (need == 0) return pager_fail(MLA_ERR_INVALID, "pager: sizes must be positive");
  if (bytes < need) return pager_fail(MLA_ERR_WORKSPACE, "pager: state buffer smaller than mla_pager_bytes");
  Header* h = static_cast<Header*>(state);
  std::memset(h, 0, sizeof(Header));
  h->num_pages = num_pages;
  h->max_seqs = max_seqs;
  h->max_blocks = max_blocks;
  h->free_top = num_pages;
  for (int i = 0; i < num_pages; ++i) {
    free_stack(h)[i] = num_pages - 1 - i;  // top of the stack = page 0
    owner(h)[i] = -1;
  }
  for (int s = 0; s < max_seqs; ++s) npages(h)[s] = 0;
  const size_t cells = (size_t)max_seqs * (size_t)max_blocks;
  for (size_t i = 0; i < cells; ++i) table(h)[i] = -1;
  h->magic = kMagic;
  return mla::set_status(MLA_OK, "");
}

int mla_pager_reserve(void* state, int seq, int64_t new_len) {
  Header* h = state_of(state);
  if (!h) return pager_fail(MLA_ERR_INVALID, "pager: state not initialised");
  if (seq < 0 || seq >= h->max_seqs) return pager_fail(MLA_ERR_INVALID, "pager: sequence id out of range");
  if (new_len < 0) return pager_fail(MLA_ERR_INVALID, "pager: negative length");
  const int64_t need64 = (new_len + MLA_PAGE_BLOCK_SIZE - 1) / MLA_PAGE_BLOCK_SIZE;
  if (need64 > h->max_blocks) return pager_fail(MLA_ERR_CAPACITY, "pager: length exceeds max_blocks pages");
  const int need = (int)need64;
  const int have = npages(h)[seq];
  if (need <= have) return mla::set_status(MLA_OK, "");
  if (need - have > h->free_top) return pager_fail(MLA_ERR_CAPACITY, "pager: out of free pages");
  int32_t* row = table(h) + (size_t)seq * h->max_blocks;
  for (int k = have; k < need; ++k) {
    const int32_t pid = free_stack(h)[--h->free_top];
    owner(h)[pid] = seq;
    row[k] = pid;
  }
  npages(h)[seq] = need;
  return mla::set_status(MLA_OK, "");
}

int mla_pager_release(void* state, int seq) {
  Header* h = state_of(state);
  if (!h) return pager_fail(MLA_ERR_INVALID, "pager: state not initialised");
  if (seq < 0 || seq >= h->max_seqs) return pager_fail(MLA_ERR_INVALID, "pager: sequence id out of range");
  int32_t* row = table(h) + (size_t)seq * h->max_blocks;
  // push in reverse so the sequence's first page is the next one taken
  for (int k = npages(h)[seq] - 1; k >= 0; --k) {
    const int32_t pid = row[k];
    owner(h)[pid] = -1;
    free_stack(h)[h->free_top++] = pid;
    row[k] = -1;
  }
  npages(h)[seq] = 0;
  return mla::set_status(MLA_OK, "");
}

int mla_pager_free_pages(const void* state) {
  Header* h = state_of(const_cast<void*>(state));
  return h ? h->free_top : pager_fail(MLA_ERR_INVALID, "pager: state not initialised");
}

int mla_pager_seq_pages(const void* state, int seq) {
  Header* h = state_of(const_cast<void*>(state));
  if (!h) return pager_fail(MLA_ERR_INVALID, "pager: state not initialised");
  if (seq < 0 || seq >= h->max_seqs) return pager_fail(MLA_ERR_INVALID, "pager: sequence id out of range");
  return npages(h)[seq];
}

int mla_pager_page_owner(const void* state, int page) {
  Header* h = state_of(const_cast<void*>(state));
  // -1 means "free" here, so errors use a status that no owner value takes
  if (!h) return pager_fail(MLA_ERR_RANGE, "pager: state not initialised");
  if (page < 0 || page >= h->num_pages) return pager_fail(MLA_ERR_RANGE, "pager: page id out of range");
  return owner(h)[page];
}

const int32_t* mla_pager_block_table(const void* state) {
  Header* h = state_of(const_cast<void*>(state));
  return h ? table(h) : nullptr;
}

}  // extern "C"
