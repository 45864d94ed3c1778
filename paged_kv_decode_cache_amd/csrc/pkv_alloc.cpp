// Host-side block allocator and slot-mapping builder for the paged KV cache.
//
// What it follows: the KV cache is made of fixed-size blocks handed out on
// demand from a free-block queue kept on the host (Inference Engineering,
// Day 11 post on vLLM: the KV cache manager takes a free block from the queue
// when a request needs more space), and each sequence owns a block table, so
// the memory a sequence wastes is less than one block (nanoserve write-up,
// "What I built", paged KV cache item).
//
// Design: one handle holds the FIFO of free block ids, each sequence's table
// and token count.  A sequence holds exactly ceil(len / block_size) blocks
// (the waste bound holds by construction).  Freed blocks go to the back of
// the queue in table order.  Every call that can run out of blocks checks the
// whole request first and changes nothing on failure.  Plain C++ on host
// memory; no GPU call, no allocation after create.
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "pkv.h"

struct pkv_block_allocator {
  int32_t num_blocks;
  int32_t block_size;
  int32_t max_seqs;
  int32_t max_blocks_per_seq;
  // FIFO of free ids as a ring over num_blocks entries
  std::vector<int32_t> ring;
  int64_t head = 0;  // next id to hand out
  int64_t count = 0; // ids in the queue
  std::vector<int32_t> tables;  // [max_seqs, max_blocks_per_seq]
  std::vector<int32_t> nblk;    // blocks held per sequence
  std::vector<int32_t> len;     // tokens per sequence
  mutable std::vector<uint8_t> seen;  // per-call scratch: sequences of a batch

  int32_t pop() {
    const int32_t id = ring[head];
    head = (head + 1) % num_blocks;
    --count;
    return id;
  }
  void push(int32_t id) {
    ring[(head + count) % num_blocks] = id;
    ++count;
  }
  int32_t* table(int32_t s) { return tables.data() + (size_t)s * max_blocks_per_seq; }
  const int32_t* table(int32_t s) const {
    return tables.data() + (size_t)s * max_blocks_per_seq;
  }
  // blocks sequence s must newly take to hold n more tokens (-1: over its cap)
  int64_t need(int32_t s, int32_t n) const {
    const int64_t want = ((int64_t)len[s] + n + block_size - 1) / block_size;
    if (want > max_blocks_per_seq) return -1;
    return want - nblk[s];
  }
  void grow(int32_t s, int32_t n, int64_t* slots) {
    const int64_t want = ((int64_t)len[s] + n + block_size - 1) / block_size;
    int32_t* row = table(s);
    while (nblk[s] < want) row[nblk[s]++] = pop();
    for (int32_t i = 0; i < n; ++i) {
      const int32_t pos = len[s] + i;
      if (slots) slots[i] = (int64_t)row[pos / block_size] * block_size + pos % block_size;
    }
    len[s] += n;
  }
  // Table entries past a sequence's blocks hold -1 (set at create and at
  // free), so a row copies as one block of memory.
  void copy_row(int32_t s, int32_t* out, int32_t width) const {
    const int32_t n = width < max_blocks_per_seq ? width : max_blocks_per_seq;
    std::memcpy(out, table(s), sizeof(int32_t) * (size_t)n);
    for (int32_t j = n; j < width; ++j) out[j] = -1;
  }
};

namespace {

bool seq_ok(const pkv_block_allocator* a, int32_t s) { return a && s >= 0 && s < a->max_seqs; }

// Checks a batch of distinct sequences growing by n[b] tokens each (n == null:
// one each); returns PKV_OK, PKV_ERR_INVALID_ARG or PKV_ERR_NO_SPACE.
int check_batch_marked(const pkv_block_allocator* a, const int32_t* seqs, const int32_t* n,
                       int32_t B, int32_t width, int32_t& marked) {
  int64_t total = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t s = seqs[b];
    if (!seq_ok(a, s) || a->seen[s]) return PKV_ERR_INVALID_ARG;
    a->seen[s] = 1;
    marked = b + 1;
    const int32_t k = n ? n[b] : 1;
    if (k < 0) return PKV_ERR_INVALID_ARG;
    const int64_t more = a->need(s, k);
    if (more < 0) return PKV_ERR_NO_SPACE;
    if (((int64_t)a->len[s] + k + a->block_size - 1) / a->block_size > width)
      return PKV_ERR_INVALID_ARG;
    total += more;
  }
  return total > a->count ? PKV_ERR_NO_SPACE : PKV_OK;
}

int check_batch(const pkv_block_allocator* a, const int32_t* seqs, const int32_t* n, int32_t B,
                int32_t width) {
  if (!a || B < 0 || (B > 0 && !seqs) || width < 0) return PKV_ERR_INVALID_ARG;
  int32_t marked = 0;
  const int rc = check_batch_marked(a, seqs, n, B, width, marked);
  for (int32_t b = 0; b < marked; ++b) a->seen[seqs[b]] = 0;
  return rc;
}

}  // namespace

extern "C" {

pkv_block_allocator* pkv_allocator_create(int32_t num_blocks, int32_t block_size,
                                          int32_t max_seqs, int32_t max_blocks_per_seq) {
  if (num_blocks <= 0 || block_size <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0)
    return nullptr;
  if ((int64_t)num_blocks * block_size > INT64_MAX / 2) return nullptr;
  pkv_block_allocator* a = new (std::nothrow) pkv_block_allocator;
  if (!a) return nullptr;
  try {
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->max_seqs = max_seqs;
    a->max_blocks_per_seq = max_blocks_per_seq;
    a->ring.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) a->ring[i] = i;
    a->count = num_blocks;
    a->tables.assign((size_t)max_seqs * max_blocks_per_seq, -1);
    a->nblk.assign(max_seqs, 0);
    a->len.assign(max_seqs, 0);
    a->seen.assign(max_seqs, 0);
  } catch (...) {
    delete a;
    return nullptr;
  }
  return a;
}

void pkv_allocator_destroy(pkv_block_allocator* a) { delete a; }

int32_t pkv_allocator_num_free(const pkv_block_allocator* a) {
  return a ? (int32_t)a->count : PKV_ERR_INVALID_ARG;
}

int32_t pkv_allocator_context_len(const pkv_block_allocator* a, int32_t seq) {
  return seq_ok(a, seq) ? a->len[seq] : PKV_ERR_INVALID_ARG;
}

int pkv_allocator_append_slots(pkv_block_allocator* a, int32_t seq, int32_t num_tokens,
                               int64_t* slot_mapping) {
  if (!seq_ok(a, seq) || num_tokens < 0 || (num_tokens > 0 && !slot_mapping))
    return PKV_ERR_INVALID_ARG;
  const int64_t more = a->need(seq, num_tokens);
  if (more < 0 || more > a->count) return PKV_ERR_NO_SPACE;
  a->grow(seq, num_tokens, slot_mapping);
  return PKV_OK;
}

int pkv_allocator_free_seq(pkv_block_allocator* a, int32_t seq) {
  if (!seq_ok(a, seq)) return PKV_ERR_INVALID_ARG;
  const int32_t* row = a->table(seq);
  for (int32_t j = 0; j < a->nblk[seq]; ++j) a->push(row[j]);
  std::memset(a->table(seq), 0xFF, sizeof(int32_t) * a->max_blocks_per_seq);
  a->nblk[seq] = 0;
  a->len[seq] = 0;
  return PKV_OK;
}

int pkv_allocator_block_table(const pkv_block_allocator* a, int32_t seq, int32_t* row,
                              int32_t width) {
  if (!seq_ok(a, seq) || width < 0 || (width > 0 && !row)) return PKV_ERR_INVALID_ARG;
  if (width < a->nblk[seq]) return PKV_ERR_INVALID_ARG;
  a->copy_row(seq, row, width);
  return PKV_OK;
}

int pkv_allocator_build_decode_batch(pkv_block_allocator* a, const int32_t* seqs, int32_t B,
                                     int32_t width, int64_t* slot_mapping,
                                     int32_t* block_tables, int32_t* context_lens) {
  const int rc = check_batch(a, seqs, nullptr, B, width);
  if (rc != PKV_OK) return rc;
  if (B > 0 && (!slot_mapping || !block_tables || !context_lens)) return PKV_ERR_INVALID_ARG;
  for (int32_t b = 0; b < B; ++b) {
    a->grow(seqs[b], 1, slot_mapping + b);
    a->copy_row(seqs[b], block_tables + (size_t)b * width, width);
    context_lens[b] = a->len[seqs[b]];
  }
  return PKV_OK;
}

int pkv_allocator_build_prefill_batch(pkv_block_allocator* a, const int32_t* seqs,
                                      const int32_t* chunk_lens, int32_t B, int32_t width,
                                      int32_t* query_start, int64_t* slot_mapping,
                                      int32_t* block_tables, int32_t* context_lens) {
  if (B > 0 && !chunk_lens) return PKV_ERR_INVALID_ARG;
  const int rc = check_batch(a, seqs, chunk_lens, B, width);
  if (rc != PKV_OK) return rc;
  if (!query_start) return PKV_ERR_INVALID_ARG;
  int64_t total = 0;
  for (int32_t b = 0; b < B; ++b) total += chunk_lens[b];
  if (total > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (B > 0 && (!block_tables || !context_lens || (total > 0 && !slot_mapping)))
    return PKV_ERR_INVALID_ARG;
  query_start[0] = 0;
  for (int32_t b = 0; b < B; ++b) {
    a->grow(seqs[b], chunk_lens[b], slot_mapping ? slot_mapping + query_start[b] : nullptr);
    query_start[b + 1] = query_start[b] + chunk_lens[b];
    a->copy_row(seqs[b], block_tables + (size_t)b * width, width);
    context_lens[b] = a->len[seqs[b]];
  }
  return PKV_OK;
}

}  // extern "C"
