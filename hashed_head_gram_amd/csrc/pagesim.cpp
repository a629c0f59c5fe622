// Flash page-cache simulation (host C++): the 4 KiB block of every looked-up
// row in the storage order of the PageGram tech report (§2.3 row bytes, §3.3
// pages per block), and an LRU RAM page cache over the per-token block sets
// (§8 Fig. 4a; appendix D describes the report's own C simulator).
//
// The LRU keeps blocks in an intrusive doubly-linked recency list over a
// slot array, indexed by an open-addressing hash table (linear probing,
// tombstone-free deletion by backward shift), so a run of millions of
// lookups allocates once and touches no per-node heap memory.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/pagegram.h"

namespace {

constexpr int64_t kBlock = 4096;

int64_t row_bytes(int32_t dt, int r) {
  switch (dt) {
    case PG_F32: return 4LL * r;
    case PG_BF16: return 2LL * r;
    case PG_NF4: return r / 2 + 2;
    default: return -1;
  }
}

// LRU set of int64 block ids with fixed capacity.
class Lru {
 public:
  explicit Lru(int64_t cap) : cap_(cap) {
    if (cap_ <= 0) return;
    size_t n = 16;
    while (n < (size_t)cap_ * 2 + 2) n <<= 1;
    mask_ = n - 1;
    table_.assign(n, -1);
    key_.resize((size_t)cap_);
    prev_.resize((size_t)cap_);
    next_.resize((size_t)cap_);
  }

  // True on a hit; on a miss the block is inserted (evicting the least
  // recently used one when full).
  bool touch(int64_t b) {
    if (cap_ <= 0) return false;
    size_t h = find(b);
    if (table_[h] >= 0) {
      to_front(table_[h]);
      return true;
    }
    int32_t s;
    if (used_ < cap_) {
      s = (int32_t)used_++;
    } else {
      s = tail_;
      unlink(s);
      erase(key_[(size_t)s]);
      h = find(b);  // the erase may have moved entries
    }
    key_[(size_t)s] = b;
    table_[h] = s;
    push_front(s);
    return false;
  }

 private:
  static uint64_t mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  // slot of b, or the empty slot where it would go
  size_t find(int64_t b) const {
    size_t h = (size_t)mix((uint64_t)b) & mask_;
    while (table_[h] >= 0 && key_[(size_t)table_[h]] != b) h = (h + 1) & mask_;
    return h;
  }
  void erase(int64_t b) {
    size_t h = find(b);
    table_[h] = -1;
    // backward-shift the cluster after h
    size_t j = h;
    for (;;) {
      j = (j + 1) & mask_;
      if (table_[j] < 0) break;
      const size_t home = (size_t)mix((uint64_t)key_[(size_t)table_[j]]) & mask_;
      // move j to h when h lies cyclically in [home, j)
      const bool move = (j > h) ? (home <= h || home > j) : (home <= h && home > j);
      if (move) {
        table_[h] = table_[j];
        table_[j] = -1;
        h = j;
      }
    }
  }
  void unlink(int32_t s) {
    const int32_t p = prev_[(size_t)s], n = next_[(size_t)s];
    if (p >= 0) next_[(size_t)p] = n; else head_ = n;
    if (n >= 0) prev_[(size_t)n] = p; else tail_ = p;
  }
  void push_front(int32_t s) {
    prev_[(size_t)s] = -1;
    next_[(size_t)s] = head_;
    if (head_ >= 0) prev_[(size_t)head_] = s;
    head_ = s;
    if (tail_ < 0) tail_ = s;
  }
  void to_front(int32_t s) {
    if (head_ == s) return;
    unlink(s);
    push_front(s);
  }

  int64_t cap_;
  int64_t used_ = 0;
  size_t mask_ = 0;
  std::vector<int32_t> table_;
  std::vector<int64_t> key_;
  std::vector<int32_t> prev_, next_;
  int32_t head_ = -1, tail_ = -1;
};

}  // namespace

extern "C" {

PG_API int pg_flash_blocks(const pg_layout* layout, int32_t table_dtype, const int64_t* rows,
                           int64_t n, int64_t* blocks_out) {
  int64_t R = 0;
  const int st = pg_layout_rows(layout, &R);
  if (st != PG_OK) return st;
  const int64_t rb = row_bytes(table_dtype, layout->r);
  if (rb <= 0 || (table_dtype == PG_NF4 && layout->r % 2)) return PG_EINVAL;
  if (n < 0) return PG_EINVAL;
  if (n == 0) return PG_OK;
  if (!rows || !blocks_out) return PG_EINVAL;
  const int O = layout->n_max - layout->n_min + 1;
  const int K = layout->K;
  if (layout->kind == PG_PAGEGRAM) {
    const int64_t per = (int64_t)K * layout->S;
    const int64_t page_bytes = per * rb;
    for (int64_t q = 0; q < n; ++q) {
      const int64_t row = rows[q];
      if (row < 0 || row >= R) return PG_ERANGE;
      const int64_t page = row / per;
      blocks_out[q] = page_bytes <= kBlock
                          ? page / (kBlock / page_bytes)
                          : page * ((page_bytes + kBlock - 1) / kBlock) +
                                ((row - page * per) * rb) / kBlock;
    }
    return PG_OK;
  }
  // Engram-style: per-head tables in (order, head) order, each on fresh blocks.
  const int64_t rpb = kBlock / rb;
  if (rpb < 1) return PG_EINVAL;
  int64_t row_base[PG_MAX_ORDERS * PG_MAX_HEADS], blk_base[PG_MAX_ORDERS * PG_MAX_HEADS];
  int64_t acc_r = 0, acc_b = 0;
  const int H = O * K;
  for (int t = 0; t < H; ++t) {
    const int64_t P = layout->head_rows[t / K][t % K];
    row_base[t] = acc_r;
    blk_base[t] = acc_b;
    acc_r += P;
    acc_b += (P + rpb - 1) / rpb;
  }
  for (int64_t q = 0; q < n; ++q) {
    const int64_t row = rows[q];
    if (row < 0 || row >= R) return PG_ERANGE;
    int lo = 0, hi = H - 1;  // last table whose base <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (row_base[mid] <= row) lo = mid; else hi = mid - 1;
    }
    blocks_out[q] = blk_base[lo] + (row - row_base[lo]) / rpb;
  }
  return PG_OK;
}

PG_API int pg_lru_cache_sim(const int64_t* blocks, int64_t n_tok, int32_t per_token,
                            int64_t capacity_blocks, pg_cache_stats* out) {
  if (!out || per_token < 1 || capacity_blocks < 0 || n_tok < 0) return PG_EINVAL;
  if (capacity_blocks > (int64_t)INT32_MAX - 1) return PG_ERANGE;
  memset(out, 0, sizeof(*out));
  if (n_tok == 0) return PG_OK;
  if (!blocks) return PG_EINVAL;
  Lru cache(capacity_blocks);
  std::vector<int64_t> seen((size_t)per_token);
  int64_t distinct = 0, misses = 0;
  for (int64_t t = 0; t < n_tok; ++t) {
    const int64_t* b = blocks + t * per_token;
    int ns = 0;
    for (int j = 0; j < per_token; ++j) {
      bool dup = false;
      for (int q = 0; q < ns; ++q) dup |= seen[(size_t)q] == b[j];
      if (!dup) seen[(size_t)ns++] = b[j];
    }
    distinct += ns;
    for (int q = 0; q < ns; ++q)
      if (!cache.touch(seen[(size_t)q])) ++misses;
  }
  out->tokens = n_tok;
  out->lookups = n_tok * per_token;
  out->distinct = distinct;
  out->misses = misses;
  return PG_OK;
}

}  // extern "C"
