// Native host block manager of the paged KV cache (include/pa_host.h): the
// free-block queue, reference counts, the hash-keyed prefix cache and
// copy-on-write of "PagedAttention：KV cache 即虚拟内存（block manager &
// 碎片）" (section 深入原理) and the allocate-on-growth rule of "49 vLLM /
// PagedAttention" (listing "Таблица блоков"), with the same rules and the
// same block keys as the Python manager in pool.py.  Host code only.
#include "pa_host.h"

#include <cstddef>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// SHA-256 as FIPS 180-4 defines it (message schedule of 64 words, 64 rounds
// per 512-bit block, big-endian words, length padding).
// ---------------------------------------------------------------------------
constexpr uint32_t kRound[64] = {
    0x428a2f98u, 0x71374491u, 0xb5c0fbcfu, 0xe9b5dba5u, 0x3956c25bu,
    0x59f111f1u, 0x923f82a4u, 0xab1c5ed5u, 0xd807aa98u, 0x12835b01u,
    0x243185beu, 0x550c7dc3u, 0x72be5d74u, 0x80deb1feu, 0x9bdc06a7u,
    0xc19bf174u, 0xe49b69c1u, 0xefbe4786u, 0x0fc19dc6u, 0x240ca1ccu,
    0x2de92c6fu, 0x4a7484aau, 0x5cb0a9dcu, 0x76f988dau, 0x983e5152u,
    0xa831c66du, 0xb00327c8u, 0xbf597fc7u, 0xc6e00bf3u, 0xd5a79147u,
    0x06ca6351u, 0x14292967u, 0x27b70a85u, 0x2e1b2138u, 0x4d2c6dfcu,
    0x53380d13u, 0x650a7354u, 0x766a0abbu, 0x81c2c92eu, 0x92722c85u,
    0xa2bfe8a1u, 0xa81a664bu, 0xc24b8b70u, 0xc76c51a3u, 0xd192e819u,
    0xd6990624u, 0xf40e3585u, 0x106aa070u, 0x19a4c116u, 0x1e376c08u,
    0x2748774cu, 0x34b0bcb5u, 0x391c0cb3u, 0x4ed8aa4au, 0x5b9cca4fu,
    0x682e6ff3u, 0x748f82eeu, 0x78a5636fu, 0x84c87814u, 0x8cc70208u,
    0x90befffau, 0xa4506cebu, 0xbef9a3f7u, 0xc67178f2u};

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

void compress(uint32_t h[8], const uint8_t* blk) {
  uint32_t w[64];
  for (int i = 0; i < 16; ++i)
    w[i] = (uint32_t)blk[4 * i] << 24 | (uint32_t)blk[4 * i + 1] << 16 |
           (uint32_t)blk[4 * i + 2] << 8 | (uint32_t)blk[4 * i + 3];
  for (int i = 16; i < 64; ++i) {
    const uint32_t s0 =
        rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
    const uint32_t s1 =
        rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
    w[i] = w[i - 16] + s0 + w[i - 7] + s1;
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5],
           g = h[6], k = h[7];
  for (int i = 0; i < 64; ++i) {
    const uint32_t t1 = k + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) +
                        ((e & f) ^ (~e & g)) + kRound[i] + w[i];
    const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) +
                        ((a & b) ^ (a & c) ^ (b & c));
    k = g;
    g = f;
    f = e;
    e = d + t1;
    d = c;
    c = b;
    b = a;
    a = t1 + t2;
  }
  h[0] += a; h[1] += b; h[2] += c; h[3] += d;
  h[4] += e; h[5] += f; h[6] += g; h[7] += k;
}

// First 8 bytes of SHA-256(msg[0..len)), read as a little-endian uint64.
uint64_t sha256_head64(const uint8_t* msg, size_t len) {
  uint32_t h[8] = {0x6a09e667u, 0xbb67ae85u, 0x3c6ef372u, 0xa54ff53au,
                   0x510e527fu, 0x9b05688cu, 0x1f83d9abu, 0x5be0cd19u};
  size_t off = 0;
  for (; off + 64 <= len; off += 64) compress(h, msg + off);
  uint8_t tail[128] = {};
  const size_t rest = len - off;
  std::memcpy(tail, msg + off, rest);
  tail[rest] = 0x80;
  const size_t tl = rest + 9 <= 64 ? 64 : 128;
  const uint64_t bits = (uint64_t)len * 8;
  for (int i = 0; i < 8; ++i) tail[tl - 1 - i] = (uint8_t)(bits >> (8 * i));
  compress(h, tail);
  if (tl == 128) compress(h, tail + 64);
  // digest bytes 0..7 are h[0] and h[1], each big-endian
  uint8_t d[8];
  for (int i = 0; i < 4; ++i) {
    d[i] = (uint8_t)(h[0] >> (24 - 8 * i));
    d[4 + i] = (uint8_t)(h[1] >> (24 - 8 * i));
  }
  uint64_t out = 0;
  for (int i = 7; i >= 0; --i) out = out << 8 | d[i];
  return out;
}

void put_le64(uint8_t* p, uint64_t v) {
  for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

// Key of a full block: its token ids chained to the parent block's key.
uint64_t block_key(uint64_t parent, const int64_t* toks, int n,
                   std::vector<uint8_t>& buf) {
  buf.resize(8 * (size_t)(n + 1));
  put_le64(buf.data(), parent);
  for (int i = 0; i < n; ++i)
    put_le64(buf.data() + 8 * (size_t)(i + 1), (uint64_t)toks[i]);
  return sha256_head64(buf.data(), buf.size());
}

struct Seq {
  int32_t num_tokens = 0;              // tokens stored (slots in use)
  std::vector<int32_t> blocks;         // the block table, in order
  bool has_tokens = false;             // admitted with token ids
  std::vector<int64_t> tokens;
  // (block index, key) of fresh full blocks not yet registered, in order
  std::vector<std::pair<int32_t, uint64_t>> pending;
};

}  // namespace

struct pa_bm {
  int32_t nb = 0, bs = 0;
  // free queue: a doubly linked list over block ids with sentinels nb (head)
  // and nb + 1 (tail)
  std::vector<int32_t> prv, nxt, ref;
  std::vector<uint8_t> in_free, has_key;
  std::vector<uint64_t> key;
  std::unordered_map<uint64_t, int32_t> cache;
  int32_t nfree = 0;
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<int32_t> copy_src, copy_dst;
  std::vector<uint8_t> scratch;        // key input bytes
  std::vector<uint64_t> key_buf;
  mutable std::vector<int32_t> hit_buf;  // scratch of hits_of

  int32_t head() const { return nb; }
  int32_t tail() const { return nb + 1; }

  void push_tail(int32_t b) {
    const int32_t last = prv[tail()];
    nxt[last] = b;
    prv[b] = last;
    nxt[b] = tail();
    prv[tail()] = b;
    in_free[b] = 1;
    ++nfree;
  }
  void unlink(int32_t b) {
    nxt[prv[b]] = nxt[b];
    prv[nxt[b]] = prv[b];
    in_free[b] = 0;
    --nfree;
  }
  // Head of the free queue, evicted from the prefix cache; -1 when empty.
  int32_t alloc() {
    if (nfree == 0) return -1;
    const int32_t b = nxt[head()];
    unlink(b);
    if (has_key[b]) {
      auto it = cache.find(key[b]);
      if (it != cache.end() && it->second == b) cache.erase(it);
      has_key[b] = 0;
    }
    ref[b] = 1;
    return b;
  }
  void touch(int32_t b) {
    if (ref[b] == 0 && in_free[b]) unlink(b);
    ++ref[b];
  }
  void release(int32_t b) {
    if (--ref[b] == 0) push_tail(b);
  }
  // First key wins; a block keeps the first key it is given.
  void register_key(int32_t b, uint64_t k) {
    if (!has_key[b] && cache.find(k) == cache.end()) {
      has_key[b] = 1;
      key[b] = k;
      cache.emplace(k, b);
    }
  }
  // Cached blocks of the longest cached prefix (lookups stop at a miss).
  void hits_of(const uint64_t* keys, int32_t n_keys) const {
    hit_buf.clear();
    for (int32_t i = 0; i < n_keys; ++i) {
      auto it = cache.find(keys[i]);
      if (it == cache.end()) break;
      hit_buf.push_back(it->second);
    }
  }
  int32_t needed(int32_t n) const {
    return (int32_t)(((int64_t)n + bs - 1) / bs);
  }
  const uint64_t* keys_for(const int64_t* tokens, int32_t n,
                           const uint64_t* keys) {
    if (keys) return keys;
    key_buf.resize((size_t)(n / bs));
    pa_bm_prefix_keys(tokens, n, bs, key_buf.data());
    return key_buf.data();
  }
};

extern "C" {

pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size,
                    const int32_t* order) {
  // slots are int32: every slot id block * block_size + offset must fit
  if (num_blocks <= 0 || block_size <= 0 ||
      (int64_t)num_blocks * block_size > INT32_MAX)
    return nullptr;
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) return nullptr;
  const int32_t nb = num_blocks;
  bm->nb = nb;
  bm->bs = block_size;
  bm->prv.assign(nb + 2, -1);
  bm->nxt.assign(nb + 2, -1);
  bm->ref.assign(nb, 0);
  bm->in_free.assign(nb, 0);
  bm->has_key.assign(nb, 0);
  bm->key.assign(nb, 0);
  bm->nxt[bm->head()] = bm->tail();
  bm->prv[bm->tail()] = bm->head();
  std::vector<uint8_t> seen(nb, 0);
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t b = order ? order[i] : i;
    if (b < 0 || b >= nb || seen[b]) {
      delete bm;
      return nullptr;
    }
    seen[b] = 1;
    bm->push_tail(b);
  }
  return bm;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int32_t pa_bm_num_free(const pa_bm* bm) { return bm ? bm->nfree : -1; }

int32_t pa_bm_num_cached(const pa_bm* bm) {
  return bm ? (int32_t)bm->cache.size() : -1;
}

void pa_bm_prefix_keys(const int64_t* tokens, int32_t n, int32_t block_size,
                       uint64_t* keys_out) {
  if (!tokens || !keys_out || block_size <= 0 || n < block_size) return;
  std::vector<uint8_t> buf;
  uint64_t parent = 0;
  for (int32_t i = 0; i + 1 <= n / block_size; ++i) {
    parent = block_key(parent, tokens + (size_t)i * block_size, block_size,
                       buf);
    keys_out[i] = parent;
  }
}

int32_t pa_bm_blocks_to_admit(const pa_bm* bm, int32_t n,
                              const uint64_t* keys, int32_t n_keys) {
  if (!bm || n < 0 || n_keys != n / bm->bs || (n_keys && !keys)) return -1;
  bm->hits_of(keys, n_keys);
  int32_t take = bm->needed(n) - (int32_t)bm->hit_buf.size();
  for (int32_t b : bm->hit_buf) take += bm->ref[b] == 0;
  return take;
}

int32_t pa_bm_admit(pa_bm* bm, int64_t seq, int32_t n) {
  if (!bm || n < 0) return -1;
  if (bm->seqs.count(seq)) return -2;
  const int32_t fresh = bm->needed(n);
  if (fresh > bm->nfree) return 0;
  Seq s;
  s.blocks.reserve(fresh);
  for (int32_t i = 0; i < fresh; ++i) s.blocks.push_back(bm->alloc());
  s.num_tokens = n;
  bm->seqs.emplace(seq, std::move(s));
  return 1;
}

int32_t pa_bm_admit_cached(pa_bm* bm, int64_t seq, const int64_t* tokens,
                           int32_t n, const uint64_t* keys, int32_t n_keys,
                           int32_t register_now) {
  if (!bm || n < 0 || (n && !tokens)) return -1;
  if (keys && n_keys != n / bm->bs) return -1;
  if (bm->seqs.count(seq)) return -2;
  const int32_t nfull = n / bm->bs;
  const uint64_t* k = bm->keys_for(tokens, n, keys);
  bm->hits_of(k, nfull);
  const int32_t nhit = (int32_t)bm->hit_buf.size();
  const int32_t fresh = bm->needed(n) - nhit;
  int32_t free_hits = 0;
  for (int32_t b : bm->hit_buf) free_hits += bm->ref[b] == 0;
  // a hit that sits in the free queue counts as free until touched: it must
  // not be allocated for this request's fresh blocks
  if (fresh > bm->nfree - free_hits) return -3;
  Seq s;
  s.has_tokens = true;
  s.tokens.assign(tokens, tokens + n);
  s.blocks.reserve(nhit + fresh);
  for (int32_t b : bm->hit_buf) {
    bm->touch(b);
    s.blocks.push_back(b);
  }
  for (int32_t i = 0; i < fresh; ++i) {
    const int32_t b = bm->alloc();
    s.blocks.push_back(b);
    const int32_t j = nhit + i;
    if (j < nfull) {
      if (register_now)
        bm->register_key(b, k[j]);
      else
        s.pending.emplace_back(j, k[j]);
    }
  }
  s.num_tokens = n;
  bm->seqs.emplace(seq, std::move(s));
  return nhit;
}

int32_t pa_bm_fork(pa_bm* bm, int64_t src, int64_t dst) {
  if (!bm) return -1;
  auto it = bm->seqs.find(src);
  if (it == bm->seqs.end() || bm->seqs.count(dst)) return -2;
  Seq s;
  s.num_tokens = it->second.num_tokens;
  s.blocks = it->second.blocks;
  s.has_tokens = it->second.has_tokens;
  s.tokens = it->second.tokens;
  for (int32_t b : s.blocks) bm->touch(b);
  bm->seqs.emplace(dst, std::move(s));
  return 0;
}

int32_t pa_bm_cache_written(pa_bm* bm, int64_t seq, int32_t n) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -2;
  Seq& s = it->second;
  const int32_t done = n / bm->bs;
  size_t k = 0;
  while (k < s.pending.size() && s.pending[k].first < done) {
    bm->register_key(s.blocks[s.pending[k].first], s.pending[k].second);
    ++k;
  }
  s.pending.erase(s.pending.begin(), s.pending.begin() + k);
  return 0;
}

int32_t pa_bm_append_slots(pa_bm* bm, const int64_t* seqs,
                           const int64_t* tokens, int32_t count,
                           int32_t* slots_out) {
  if (!bm || count < 0 || (count && (!seqs || !slots_out))) return -1;
  const int32_t bs = bm->bs;
  for (int32_t i = 0; i < count; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return -2;
    Seq& s = it->second;
    if ((int64_t)s.blocks.size() * bs <= s.num_tokens) {
      const int32_t b = bm->alloc();
      if (b < 0) return -3;
      s.blocks.push_back(b);
    }
    const int32_t idx = s.num_tokens / bs;
    int32_t last = s.blocks[idx];
    if (bm->ref[last] > 1) {
      const int32_t copy = bm->alloc();
      if (copy < 0) return -3;
      bm->copy_src.push_back(last);
      bm->copy_dst.push_back(copy);
      bm->release(last);
      s.blocks[idx] = copy;
      last = copy;
    }
    slots_out[i] = last * bs + s.num_tokens % bs;
    ++s.num_tokens;
    if (s.has_tokens) {
      s.tokens.push_back(tokens ? tokens[i] : -1);
      if (s.num_tokens % bs == 0) {
        // a block filled by this token is registered under its key when the
        // block before it carries one (the first block's parent key is 0)
        bool has_parent = true;
        uint64_t parent = 0;
        if (idx > 0) {
          const int32_t pb = s.blocks[idx - 1];
          has_parent = bm->has_key[pb] != 0;
          parent = bm->key[pb];
        }
        if (has_parent)
          bm->register_key(last,
                           block_key(parent,
                                     s.tokens.data() + (size_t)idx * bs, bs,
                                     bm->scratch));
      }
    }
  }
  return 0;
}

int32_t pa_bm_num_copies(const pa_bm* bm) {
  return bm ? (int32_t)bm->copy_src.size() : -1;
}

int32_t pa_bm_take_copies(pa_bm* bm, int32_t* src_out, int32_t* dst_out) {
  if (!bm) return -1;
  const int32_t n = (int32_t)bm->copy_src.size();
  if (n && (!src_out || !dst_out)) return -1;
  for (int32_t i = 0; i < n; ++i) {
    src_out[i] = bm->copy_src[i];
    dst_out[i] = bm->copy_dst[i];
  }
  bm->copy_src.clear();
  bm->copy_dst.clear();
  return n;
}

int32_t pa_bm_free_seq(pa_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -2;
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  return 0;
}

int32_t pa_bm_num_tokens(const pa_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -2 : it->second.num_tokens;
}

int32_t pa_bm_num_blocks_of(const pa_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -2 : (int32_t)it->second.blocks.size();
}

int32_t pa_bm_block_ids(const pa_bm* bm, int64_t seq, int32_t* ids_out) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -2;
  const std::vector<int32_t>& b = it->second.blocks;
  if (!b.empty()) {
    if (!ids_out) return -1;
    std::memcpy(ids_out, b.data(), b.size() * sizeof(int32_t));
  }
  return (int32_t)b.size();
}

int32_t pa_bm_max_blocks(const pa_bm* bm, const int64_t* seqs,
                         int32_t count) {
  if (!bm || count < 0 || (count && !seqs)) return -1;
  int32_t w = 0;
  for (int32_t i = 0; i < count; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return -2;
    const int32_t n = (int32_t)it->second.blocks.size();
    w = n > w ? n : w;
  }
  return w;
}

int32_t pa_bm_tables(const pa_bm* bm, const int64_t* seqs, int32_t count,
                     int32_t width, int32_t pad, int32_t* table_out,
                     int32_t* lens_out) {
  if (!bm || count < 0 || width < 0 ||
      (count && (!seqs || !table_out || !lens_out)))
    return -1;
  for (int32_t i = 0; i < count; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return -2;
    const std::vector<int32_t>& b = it->second.blocks;
    if ((int32_t)b.size() > width) return -1;
    int32_t* row = table_out + (size_t)i * width;
    if (!b.empty()) std::memcpy(row, b.data(), b.size() * sizeof(int32_t));
    for (int32_t j = (int32_t)b.size(); j < width; ++j) row[j] = pad;
    lens_out[i] = it->second.num_tokens;
  }
  return 0;
}

int32_t pa_bm_ref_count(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->nb) return -1;
  return bm->ref[block];
}

int32_t pa_bm_free_queue(const pa_bm* bm, int32_t* ids_out) {
  if (!bm || (bm->nfree && !ids_out)) return -1;
  int32_t n = 0;
  for (int32_t b = bm->nxt[bm->head()]; b != bm->tail(); b = bm->nxt[b])
    ids_out[n++] = b;
  return n;
}

}  // extern "C"
