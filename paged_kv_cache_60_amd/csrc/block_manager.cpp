// Host block manager of the paged KV cache.
//
// A FIFO pool of physical block ids, per-sequence block tables and token
// counts, and per-block reference counts.
//   - Pool popped at the front, released to the back, ceil(tokens/bs) blocks
//     per sequence, check-before-pop on exhaustion:
//     "From OOM to Smooth Inference (RAG memory management)", §2.3.
//   - Reference counts, allocate / append / free / share-prefix, utilisation:
//     "Inference Engine Memory Optimisation (KV Cache to Continuous Batching)", §3.
//   - Forked sequences share blocks; copy-on-write of a shared block:
//     "vLLM Architecture and Memory Use, ch. 3", §3.2-3.3.
//   - Prefix cache: a full block's key covers its token ids and everything
//     before it; hits are mapped into the new request's table; zero-count
//     cached blocks wait for reuse; eviction is least-recently-used:
//     "Where Did the VRAM Go (KV cache tutorial)", §4.2-4.4.
//   - Preemption from the tail of the running set, by recompute (the blocks
//     are released) or by swapping the blocks to a host pool and back:
//     "Where Did the VRAM Go (KV cache tutorial)", §7.1-7.2; "From OOM to
//     Smooth Inference", §5; "vLLM Architecture and Memory Use, ch. 3", §3.4.
//     A group's shared blocks are copied once; a swapped-out sequence keeps
//     its token count and a table of host blocks and is not resident.
// The last block's fill is derived from the sequence's own token count, so two
// sequences sharing a block never update a common counter. Every call checks
// before it mutates: a failing call leaves the state as it was.
//
// A cache key is (parent block, block_size token ids); the parent's own key
// carries its parent, so equal keys mean equal token prefixes. Keys are found
// through a 64-bit hash and then compared in full, so a hash collision can
// never map a block with other content. Cached blocks reaching refcount 0 are
// appended to the evictable list deepest first; since a block never reaches 0
// after its parent, eviction (oldest first) removes children before parents,
// and no key can name a parent block that has been reused for other tokens.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <iterator>
#include <list>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pagedkv.h"

namespace {

struct Seq {
  std::vector<int32_t> table;
  int64_t count = 0;
};

// Prefix-cache key of a cached block.
struct CacheKey {
  int32_t parent = -1;
  uint64_t hash = 0;
  std::vector<int32_t> tokens;
};

// A block handed out by take(): where it came from, so that a failed batch can
// put it back exactly (an evicted block gets its key and list position back).
struct Taken {
  int32_t block;
  bool evicted;
  CacheKey key;
};

// What one append changed, so that a failed batch can be rolled back exactly.
struct AppendUndo {
  int64_t seq;
  int64_t prev_count;
  int grown;        // blocks pushed at the end of the table
  int32_t cow_src;  // -1: no copy-on-write
  int32_t cow_dst;
  std::vector<Taken> taken;  // in the order taken: the copy-on-write block, then grown ones
};

uint64_t mix64(uint64_t x) {  // splitmix64 finaliser
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

uint64_t key_hash(int32_t parent, const int32_t* tokens, int n) {
  uint64_t h = mix64(static_cast<uint64_t>(static_cast<int64_t>(parent)) + 1);
  for (int i = 0; i < n; ++i) h = mix64(h ^ static_cast<uint32_t>(tokens[i]));
  return h;
}

}  // namespace

struct pkv_bm {
  int32_t num_blocks;
  int32_t bs;
  std::deque<int32_t> free_q;
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<int32_t> ref;
  // prefix cache
  std::vector<char> cached;
  std::vector<CacheKey> key;
  std::unordered_multimap<uint64_t, int32_t> index;  // key hash -> block
  std::list<int32_t> evictable;                      // oldest first
  std::vector<std::list<int32_t>::iterator> ev_pos;
  std::vector<char> in_ev;
  int64_t prefix_query_tokens = 0;
  int64_t prefix_hit_tokens = 0;
  // host pool of swapped-out sequences
  int32_t num_host_blocks = 0;
  std::deque<int32_t> host_free;
  std::vector<int32_t> host_ref;
  std::unordered_map<int64_t, Seq> swapped;  // tables hold host block ids

  int64_t needed(int64_t tokens) const { return (tokens + bs - 1) / bs; }

  // an id that a new sequence may not take: resident or swapped out
  bool taken_id(int64_t id) const { return seqs.count(id) || swapped.count(id); }

  // Drop one reference to each block of a table, in order; uncached blocks
  // reaching 0 go to the back of the free queue, cached ones to the back of
  // the evictable list, deepest first.
  void release(const std::vector<int32_t>& table) {
    std::vector<int32_t> to_cache;
    for (int32_t b : table) {
      ref[b] -= 1;
      if (ref[b] == 0) {
        if (cached[b])
          to_cache.push_back(b);
        else
          free_q.push_back(b);
      }
    }
    for (auto r = to_cache.rbegin(); r != to_cache.rend(); ++r) ev_push_back(*r);
  }

  void release_host(const std::vector<int32_t>& table) {
    for (int32_t h : table) {
      host_ref[h] -= 1;
      if (host_ref[h] == 0) host_free.push_back(h);
    }
  }

  int64_t capacity() const { return static_cast<int64_t>(free_q.size() + evictable.size()); }

  int64_t slot(const std::vector<int32_t>& t, int64_t pos) const {
    return static_cast<int64_t>(t[pos / bs]) * bs + pos % bs;
  }

  int32_t lookup(int32_t parent, const int32_t* tokens) const {
    const uint64_t h = key_hash(parent, tokens, bs);
    auto range = index.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const CacheKey& k = key[it->second];
      if (k.parent == parent && std::equal(k.tokens.begin(), k.tokens.end(), tokens)) return it->second;
    }
    return -1;
  }

  void add_key(int32_t b, CacheKey k) {
    index.emplace(k.hash, b);
    key[b] = std::move(k);
    cached[b] = 1;
  }

  CacheKey drop_key(int32_t b) {
    auto range = index.equal_range(key[b].hash);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        index.erase(it);
        break;
      }
    cached[b] = 0;
    CacheKey k = std::move(key[b]);
    key[b] = CacheKey();
    return k;
  }

  void ev_push_back(int32_t b) {
    evictable.push_back(b);
    ev_pos[b] = std::prev(evictable.end());
    in_ev[b] = 1;
  }

  void ev_remove(int32_t b) {
    evictable.erase(ev_pos[b]);
    in_ev[b] = 0;
  }

  // One fresh block: the free queue's front, else the oldest evictable block
  // (its key is dropped). The caller has checked capacity().
  int32_t take(std::vector<Taken>* log) {
    if (!free_q.empty()) {
      int32_t b = free_q.front();
      free_q.pop_front();
      if (log) log->push_back(Taken{b, false, CacheKey()});
      return b;
    }
    int32_t b = evictable.front();
    evictable.pop_front();
    in_ev[b] = 0;
    CacheKey k = drop_key(b);
    if (log) log->push_back(Taken{b, true, std::move(k)});
    return b;
  }

  // Undo take() calls, most recent first.
  void untake(std::vector<Taken>& log) {
    for (auto it = log.rbegin(); it != log.rend(); ++it) {
      if (it->evicted) {
        add_key(it->block, std::move(it->key));
        evictable.push_front(it->block);
        ev_pos[it->block] = evictable.begin();
        in_ev[it->block] = 1;
      } else {
        free_q.push_front(it->block);
      }
    }
  }

  // Append n tokens to s; the caller has checked that s exists.
  int append_one(int64_t id, Seq& s, int n, int64_t* slots, int32_t* cow_src,
                 int32_t* cow_dst, AppendUndo* undo) {
    if (n < 0) return PKV_ERR_INVALID;
    int32_t csrc = -1, cdst = -1;
    if (n == 0) {
      if (cow_src) *cow_src = -1;
      if (cow_dst) *cow_dst = -1;
      if (undo) *undo = AppendUndo{id, s.count, 0, -1, -1, {}};
      return PKV_OK;
    }
    const bool cow = !s.table.empty() && (s.count % bs) != 0 && ref[s.table.back()] > 1;
    const int64_t grow = needed(s.count + n) - static_cast<int64_t>(s.table.size());
    const int64_t need = grow + (cow ? 1 : 0);
    if (capacity() < need) return PKV_ERR_OOM;
    std::vector<Taken> log;
    std::vector<Taken>* lp = undo ? &log : nullptr;
    if (cow) {
      csrc = s.table.back();
      cdst = take(lp);
      ref[csrc] -= 1;
      ref[cdst] += 1;
      s.table.back() = cdst;
    }
    for (int64_t i = 0; i < grow; ++i) {
      int32_t b = take(lp);
      ref[b] += 1;
      s.table.push_back(b);
    }
    const int64_t prev = s.count;
    s.count += n;
    if (slots)
      for (int64_t p = prev; p < s.count; ++p) slots[p - prev] = slot(s.table, p);
    if (cow_src) *cow_src = csrc;
    if (cow_dst) *cow_dst = cdst;
    if (undo) *undo = AppendUndo{id, prev, static_cast<int>(grow), csrc, cdst, std::move(log)};
    return PKV_OK;
  }

  void undo_append(AppendUndo& u) {
    Seq& s = seqs.at(u.seq);
    for (int i = 0; i < u.grown; ++i) {
      ref[s.table.back()] -= 1;
      s.table.pop_back();
    }
    if (u.cow_src >= 0) {
      s.table.back() = u.cow_src;
      ref[u.cow_src] += 1;
      ref[u.cow_dst] -= 1;
    }
    untake(u.taken);
    s.count = u.prev_count;
  }
};

extern "C" {

const char* pkv_status_str(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_OOM: return "block pool exhausted";
    case PKV_ERR_NO_SEQ: return "unknown sequence";
    case PKV_ERR_EXISTS: return "sequence already exists";
    case PKV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int pkv_bm_create(int num_blocks, int block_size, const int32_t* free_order, pkv_bm** out) {
  if (!out) return PKV_ERR_INVALID;
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0) return PKV_ERR_INVALID;
  std::vector<int32_t> order(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) return PKV_ERR_INVALID;
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int i = 0; i < num_blocks; ++i) order[i] = i;
  }
  pkv_bm* bm = new (std::nothrow) pkv_bm;
  if (!bm) return PKV_ERR_OOM;
  bm->num_blocks = num_blocks;
  bm->bs = block_size;
  bm->free_q.assign(order.begin(), order.end());
  bm->ref.assign(num_blocks, 0);
  bm->cached.assign(num_blocks, 0);
  bm->key.resize(num_blocks);
  bm->ev_pos.resize(num_blocks);
  bm->in_ev.assign(num_blocks, 0);
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

int pkv_bm_allocate(pkv_bm* bm, int64_t seq, int num_tokens, int64_t* slots_out) {
  if (!bm || num_tokens < 0) return PKV_ERR_INVALID;
  if (bm->taken_id(seq)) return PKV_ERR_EXISTS;
  const int64_t nb = bm->needed(num_tokens);
  if (bm->capacity() < nb) return PKV_ERR_OOM;
  Seq s;
  s.table.reserve(nb);
  for (int64_t i = 0; i < nb; ++i) {
    int32_t b = bm->take(nullptr);
    bm->ref[b] += 1;
    s.table.push_back(b);
  }
  s.count = num_tokens;
  if (slots_out)
    for (int64_t p = 0; p < num_tokens; ++p) slots_out[p] = bm->slot(s.table, p);
  bm->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

int pkv_bm_allocate_prompt(pkv_bm* bm, int64_t seq, const int32_t* tokens, int n_tokens, int* n_cached,
                           int64_t* slots_out) {
  if (!bm || n_tokens < 0 || !n_cached || (n_tokens > 0 && (!tokens || !slots_out))) return PKV_ERR_INVALID;
  if (bm->taken_id(seq)) return PKV_ERR_EXISTS;
  const int bs = bm->bs;
  const int full = n_tokens / bs;
  std::vector<int32_t> matched;
  int32_t parent = -1;
  for (int i = 0; i < full; ++i) {
    const int32_t b = bm->lookup(parent, tokens + static_cast<int64_t>(i) * bs);
    if (b < 0) break;
    matched.push_back(b);
    parent = b;
  }
  const int64_t fresh = bm->needed(n_tokens) - static_cast<int64_t>(matched.size());
  int64_t revived = 0;
  for (int32_t b : matched) revived += bm->ref[b] == 0;
  if (bm->capacity() - revived < fresh) return PKV_ERR_OOM;
  for (int32_t b : matched) {
    if (bm->ref[b] == 0) bm->ev_remove(b);
    bm->ref[b] += 1;
  }
  Seq s;
  s.table = matched;
  for (int64_t i = 0; i < fresh; ++i) {
    const int32_t b = bm->take(nullptr);
    bm->ref[b] += 1;
    s.table.push_back(b);
  }
  for (int i = static_cast<int>(matched.size()); i < full; ++i) {
    const int32_t* t = tokens + static_cast<int64_t>(i) * bs;
    CacheKey k;
    k.parent = parent;
    k.hash = key_hash(parent, t, bs);
    k.tokens.assign(t, t + bs);
    bm->add_key(s.table[i], std::move(k));
    parent = s.table[i];
  }
  s.count = n_tokens;
  const int64_t c = static_cast<int64_t>(matched.size()) * bs;
  for (int64_t p = c; p < n_tokens; ++p) slots_out[p - c] = bm->slot(s.table, p);
  bm->seqs.emplace(seq, std::move(s));
  *n_cached = static_cast<int>(c);
  bm->prefix_query_tokens += n_tokens;
  bm->prefix_hit_tokens += c;
  return PKV_OK;
}

int pkv_bm_append(pkv_bm* bm, int64_t seq, int n_tokens, int64_t* slots_out, int32_t* cow_src,
                  int32_t* cow_dst) {
  if (!bm) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_NO_SEQ;
  return bm->append_one(seq, it->second, n_tokens, slots_out, cow_src, cow_dst, nullptr);
}

}  // extern "C"

namespace {

// One token for each sequence, in order; all or nothing. cow_row (may be
// null) gets 1 for the rows whose append copied a shared block.
int append_batch_impl(pkv_bm* bm, const int64_t* seqs, int n_seqs, int64_t* slot_mapping_out,
                      int32_t* cow_pairs_out, int* n_cow, char* cow_row) {
  if (!bm || n_seqs < 0 || (n_seqs > 0 && (!seqs || !slot_mapping_out || !cow_pairs_out)) || !n_cow)
    return PKV_ERR_INVALID;
  std::unordered_set<int64_t> uniq;
  uniq.reserve(n_seqs * 2 + 1);
  for (int i = 0; i < n_seqs; ++i) {
    if (!uniq.insert(seqs[i]).second) return PKV_ERR_INVALID;
    if (!bm->seqs.count(seqs[i])) return PKV_ERR_NO_SEQ;
  }
  std::vector<AppendUndo> log;
  log.reserve(n_seqs);
  int ncow = 0;
  for (int i = 0; i < n_seqs; ++i) {
    Seq& s = bm->seqs.at(seqs[i]);
    int32_t cs, cd;
    AppendUndo u;
    int st = bm->append_one(seqs[i], s, 1, &slot_mapping_out[i], &cs, &cd, &u);
    if (st != PKV_OK) {
      for (auto r = log.rbegin(); r != log.rend(); ++r) bm->undo_append(*r);
      return st;
    }
    log.push_back(std::move(u));
    if (cow_row) cow_row[i] = cs >= 0;
    if (cs >= 0) {
      cow_pairs_out[2 * ncow] = cs;
      cow_pairs_out[2 * ncow + 1] = cd;
      ++ncow;
    }
  }
  *n_cow = ncow;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_bm_append_batch(pkv_bm* bm, const int64_t* seqs, int n_seqs, int64_t* slot_mapping_out,
                        int32_t* cow_pairs_out, int* n_cow) {
  return append_batch_impl(bm, seqs, n_seqs, slot_mapping_out, cow_pairs_out, n_cow, nullptr);
}

int pkv_bm_decode_step(pkv_bm* bm, const int64_t* seqs, int n_seqs, int64_t* slot_mapping_out,
                       int32_t* cow_pairs_out, int* n_cow, int32_t* updates_out, int* n_updates,
                       int32_t* ctx_lens_out, int max_blocks) {
  if (!bm || !n_updates || n_seqs < 0 || max_blocks < 1 ||
      (n_seqs > 0 && (!seqs || !updates_out || !ctx_lens_out)))
    return PKV_ERR_INVALID;
  // Table sizes before the step tell which entries the appends replace or add.
  // A sequence whose next token would need a table entry past the device
  // table's max_blocks columns is rejected before anything changes (the
  // device tables could not hold the entry).
  std::vector<int32_t> before(n_seqs, 0);
  for (int i = 0; i < n_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) continue;  // append_batch_impl reports NO_SEQ
    before[i] = static_cast<int32_t>(it->second.table.size());
    const int64_t need = (it->second.count + bm->bs) / bm->bs;  // ceil((count + 1) / bs)
    if (need > max_blocks) return PKV_ERR_INVALID;
  }
  std::vector<char> cow_row(n_seqs, 0);
  const int st = append_batch_impl(bm, seqs, n_seqs, slot_mapping_out, cow_pairs_out, n_cow,
                                   cow_row.data());
  if (st != PKV_OK) return st;
  int nu = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const Seq& s = bm->seqs.at(seqs[i]);
    const int32_t now = static_cast<int32_t>(s.table.size());
    const int32_t first = cow_row[i] ? before[i] - 1 : before[i];  // copy-on-write replaced the last entry
    for (int32_t j = first; j < now; ++j) {
      updates_out[3 * nu] = i;
      updates_out[3 * nu + 1] = j;
      updates_out[3 * nu + 2] = s.table[j];
      ++nu;
    }
    ctx_lens_out[i] = static_cast<int32_t>(s.count);
  }
  *n_updates = nu;
  return PKV_OK;
}

int pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return PKV_ERR_NO_SEQ;
  if (bm->taken_id(child)) return PKV_ERR_EXISTS;
  Seq c = it->second;
  for (int32_t b : c.table) bm->ref[b] += 1;
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int pkv_bm_share_prefix(pkv_bm* bm, int64_t src, int n_blocks, int64_t dst) {
  if (!bm) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(src);
  if (it == bm->seqs.end()) return PKV_ERR_NO_SEQ;
  if (bm->taken_id(dst)) return PKV_ERR_EXISTS;
  const Seq& s = it->second;
  if (n_blocks < 0 || n_blocks > static_cast<int>(s.table.size())) return PKV_ERR_INVALID;
  Seq d;
  d.table.assign(s.table.begin(), s.table.begin() + n_blocks);
  for (int32_t b : d.table) bm->ref[b] += 1;
  d.count = std::min<int64_t>(static_cast<int64_t>(n_blocks) * bm->bs, s.count);
  bm->seqs.emplace(dst, std::move(d));
  return PKV_OK;
}

int pkv_bm_free(pkv_bm* bm, int64_t seq) {
  if (!bm) return PKV_ERR_INVALID;
  auto sw = bm->swapped.find(seq);
  if (sw != bm->swapped.end()) {  // a swapped-out sequence gives back its host blocks
    bm->release_host(sw->second.table);
    bm->swapped.erase(sw);
    return PKV_OK;
  }
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_NO_SEQ;
  bm->release(it->second.table);
  bm->seqs.erase(it);
  return PKV_OK;
}

}  // extern "C"

namespace {

// The listed ids, checked: no duplicates (INVALID), each present in `where`
// (NO_SEQ).
int check_group(const std::unordered_map<int64_t, Seq>& where, const int64_t* seqs, int n) {
  if (n < 0 || (n > 0 && !seqs)) return PKV_ERR_INVALID;
  std::unordered_set<int64_t> uniq;
  for (int i = 0; i < n; ++i)
    if (!uniq.insert(seqs[i]).second) return PKV_ERR_INVALID;
  for (int i = 0; i < n; ++i)
    if (!where.count(seqs[i])) return PKV_ERR_NO_SEQ;
  return PKV_OK;
}

// Distinct block ids of the listed tables, in order of first appearance.
std::vector<int32_t> distinct_blocks(const std::unordered_map<int64_t, Seq>& where, const int64_t* seqs, int n) {
  std::vector<int32_t> out;
  std::unordered_set<int32_t> seen;
  for (int i = 0; i < n; ++i)
    for (int32_t b : where.at(seqs[i]).table)
      if (seen.insert(b).second) out.push_back(b);
  return out;
}

int swap_out_impl(pkv_bm* bm, const int64_t* seqs, int n_seqs, int32_t* pairs_out, int cap, int* n_pairs) {
  const std::vector<int32_t> blocks = distinct_blocks(bm->seqs, seqs, n_seqs);
  const int nb = static_cast<int>(blocks.size());
  if (nb > cap || (nb > 0 && !pairs_out)) return PKV_ERR_INVALID;
  if (static_cast<int>(bm->host_free.size()) < nb) return PKV_ERR_OOM;
  std::unordered_map<int32_t, int32_t> to_host;
  for (int i = 0; i < nb; ++i) {
    const int32_t h = bm->host_free.front();
    bm->host_free.pop_front();
    to_host.emplace(blocks[i], h);
    pairs_out[2 * i] = blocks[i];
    pairs_out[2 * i + 1] = h;
  }
  for (int i = 0; i < n_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    Seq host;
    host.count = it->second.count;
    host.table.reserve(it->second.table.size());
    for (int32_t b : it->second.table) {
      const int32_t h = to_host.at(b);
      host.table.push_back(h);
      bm->host_ref[h] += 1;
    }
    bm->release(it->second.table);
    bm->seqs.erase(it);
    bm->swapped.emplace(seqs[i], std::move(host));
  }
  *n_pairs = nb;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_bm_set_host_blocks(pkv_bm* bm, int num_host_blocks) {
  if (!bm || num_host_blocks < 0 || !bm->swapped.empty()) return PKV_ERR_INVALID;
  bm->num_host_blocks = num_host_blocks;
  bm->host_free.clear();
  for (int i = 0; i < num_host_blocks; ++i) bm->host_free.push_back(i);
  bm->host_ref.assign(num_host_blocks, 0);
  return PKV_OK;
}

int pkv_bm_swap_out(pkv_bm* bm, const int64_t* seqs, int n_seqs, int32_t* pairs_out, int cap, int* n_pairs) {
  if (!bm || !n_pairs || cap < 0) return PKV_ERR_INVALID;
  const int st = check_group(bm->seqs, seqs, n_seqs);
  if (st != PKV_OK) return st;
  return swap_out_impl(bm, seqs, n_seqs, pairs_out, cap, n_pairs);
}

int pkv_bm_swap_in(pkv_bm* bm, const int64_t* seqs, int n_seqs, int32_t* pairs_out, int cap, int* n_pairs) {
  if (!bm || !n_pairs || cap < 0) return PKV_ERR_INVALID;
  const int st = check_group(bm->swapped, seqs, n_seqs);
  if (st != PKV_OK) return st;
  const std::vector<int32_t> hosts = distinct_blocks(bm->swapped, seqs, n_seqs);
  const int nh = static_cast<int>(hosts.size());
  if (nh > cap || (nh > 0 && !pairs_out)) return PKV_ERR_INVALID;
  if (bm->capacity() < nh) return PKV_ERR_OOM;
  std::unordered_map<int32_t, int32_t> to_dev;
  for (int i = 0; i < nh; ++i) {
    const int32_t g = bm->take(nullptr);
    to_dev.emplace(hosts[i], g);
    pairs_out[2 * i] = hosts[i];
    pairs_out[2 * i + 1] = g;
  }
  for (int i = 0; i < n_seqs; ++i) {
    auto it = bm->swapped.find(seqs[i]);
    Seq dev;
    dev.count = it->second.count;
    dev.table.reserve(it->second.table.size());
    for (int32_t h : it->second.table) {
      const int32_t g = to_dev.at(h);
      dev.table.push_back(g);
      bm->ref[g] += 1;
    }
    bm->release_host(it->second.table);
    bm->swapped.erase(it);
    bm->seqs.emplace(seqs[i], std::move(dev));
  }
  *n_pairs = nh;
  return PKV_OK;
}

int pkv_bm_preempt_tail(pkv_bm* bm, const int64_t* running, int n_running, int blocks_needed, int mode,
                        int64_t* victims_out, int* n_victims, int32_t* pairs_out, int cap, int* n_pairs) {
  if (!bm || !n_victims || !n_pairs || blocks_needed < 0 || cap < 0 ||
      (mode != PKV_PREEMPT_RECOMPUTE && mode != PKV_PREEMPT_SWAP) || (n_running > 0 && !victims_out))
    return PKV_ERR_INVALID;
  const int st = check_group(bm->seqs, running, n_running);
  if (st != PKV_OK) return st;
  // victims from the tail until enough blocks would be available, counting
  // only the blocks each victim would actually release
  std::unordered_map<int32_t, int32_t> drop;
  int64_t avail = bm->capacity();
  int nv = 0;
  for (int i = n_running - 1; i >= 0 && avail < blocks_needed; --i) {
    victims_out[nv++] = running[i];
    for (int32_t b : bm->seqs.at(running[i]).table)
      if (bm->ref[b] - ++drop[b] == 0) ++avail;
  }
  if (avail < blocks_needed) return PKV_ERR_OOM;
  *n_pairs = 0;
  if (mode == PKV_PREEMPT_SWAP) {
    const int s2 = swap_out_impl(bm, victims_out, nv, pairs_out, cap, n_pairs);
    if (s2 != PKV_OK) return s2;
  } else {
    for (int i = 0; i < nv; ++i) pkv_bm_free(bm, victims_out[i]);
  }
  *n_victims = nv;
  return PKV_OK;
}

int pkv_bm_swapped_table(const pkv_bm* bm, int64_t seq, int32_t* out, int cap, int* n) {
  if (!bm || !n || cap < 0) return PKV_ERR_INVALID;
  auto it = bm->swapped.find(seq);
  if (it == bm->swapped.end()) return PKV_ERR_NO_SEQ;
  const auto& t = it->second.table;
  if (static_cast<int>(t.size()) > cap || (!t.empty() && !out)) return PKV_ERR_INVALID;
  std::copy(t.begin(), t.end(), out);
  *n = static_cast<int>(t.size());
  return PKV_OK;
}

int pkv_bm_swapped_tokens(const pkv_bm* bm, int64_t seq, int* n) {
  if (!bm || !n) return PKV_ERR_INVALID;
  auto it = bm->swapped.find(seq);
  if (it == bm->swapped.end()) return PKV_ERR_NO_SEQ;
  *n = static_cast<int>(it->second.count);
  return PKV_OK;
}

int pkv_bm_host_free_list(const pkv_bm* bm, int32_t* out, int cap, int* n) {
  if (!bm || !n || cap < 0) return PKV_ERR_INVALID;
  if (static_cast<int>(bm->host_free.size()) > cap || (!bm->host_free.empty() && !out)) return PKV_ERR_INVALID;
  std::copy(bm->host_free.begin(), bm->host_free.end(), out);
  *n = static_cast<int>(bm->host_free.size());
  return PKV_OK;
}

int pkv_bm_host_refcount(const pkv_bm* bm, int32_t host_block, int* rc) {
  if (!bm || !rc || host_block < 0 || host_block >= bm->num_host_blocks) return PKV_ERR_INVALID;
  *rc = bm->host_ref[host_block];
  return PKV_OK;
}

int pkv_bm_slots(const pkv_bm* bm, int64_t seq, int start, int n, int64_t* out) {
  if (!bm || start < 0 || n < 0 || (n > 0 && !out)) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_NO_SEQ;
  const Seq& s = it->second;
  if (static_cast<int64_t>(start) + n > s.count) return PKV_ERR_INVALID;
  for (int i = 0; i < n; ++i) out[i] = bm->slot(s.table, static_cast<int64_t>(start) + i);
  return PKV_OK;
}

int pkv_bm_block_table(const pkv_bm* bm, int64_t seq, int32_t* out, int cap, int* n) {
  if (!bm || !n || cap < 0) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_NO_SEQ;
  const auto& t = it->second.table;
  if (static_cast<int>(t.size()) > cap || (!t.empty() && !out)) return PKV_ERR_INVALID;
  std::copy(t.begin(), t.end(), out);
  *n = static_cast<int>(t.size());
  return PKV_OK;
}

int pkv_bm_num_tokens(const pkv_bm* bm, int64_t seq, int* n) {
  if (!bm || !n) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_NO_SEQ;
  *n = static_cast<int>(it->second.count);
  return PKV_OK;
}

int pkv_bm_refcount(const pkv_bm* bm, int32_t block, int* rc) {
  if (!bm || !rc || block < 0 || block >= bm->num_blocks) return PKV_ERR_INVALID;
  *rc = bm->ref[block];
  return PKV_OK;
}

int pkv_bm_free_list(const pkv_bm* bm, int32_t* out, int cap, int* n) {
  if (!bm || !n || cap < 0) return PKV_ERR_INVALID;
  if (static_cast<int>(bm->free_q.size()) > cap || (!bm->free_q.empty() && !out))
    return PKV_ERR_INVALID;
  std::copy(bm->free_q.begin(), bm->free_q.end(), out);
  *n = static_cast<int>(bm->free_q.size());
  return PKV_OK;
}

int pkv_bm_evictable_list(const pkv_bm* bm, int32_t* out, int cap, int* n) {
  if (!bm || !n || cap < 0) return PKV_ERR_INVALID;
  if (static_cast<int>(bm->evictable.size()) > cap || (!bm->evictable.empty() && !out))
    return PKV_ERR_INVALID;
  std::copy(bm->evictable.begin(), bm->evictable.end(), out);
  *n = static_cast<int>(bm->evictable.size());
  return PKV_OK;
}

int pkv_bm_cache_entry(const pkv_bm* bm, int32_t block, int* cached, int32_t* parent, int32_t* tokens_out) {
  if (!bm || !cached || !parent || block < 0 || block >= bm->num_blocks) return PKV_ERR_INVALID;
  *cached = bm->cached[block];
  *parent = -1;
  if (!*cached) return PKV_OK;
  if (!tokens_out) return PKV_ERR_INVALID;
  *parent = bm->key[block].parent;
  std::copy(bm->key[block].tokens.begin(), bm->key[block].tokens.end(), tokens_out);
  return PKV_OK;
}

int pkv_bm_num_free(const pkv_bm* bm) {
  return bm ? static_cast<int>(bm->free_q.size()) : PKV_ERR_INVALID;
}

int pkv_bm_stats(const pkv_bm* bm, pkv_bm_stats_t* out) {
  if (!bm || !out) return PKV_ERR_INVALID;
  std::vector<int32_t> filled(bm->num_blocks, 0);
  for (const auto& kv : bm->seqs) {
    const Seq& s = kv.second;
    for (size_t i = 0; i < s.table.size(); ++i) {
      int64_t f = s.count - static_cast<int64_t>(i) * bm->bs;
      f = std::max<int64_t>(0, std::min<int64_t>(bm->bs, f));
      filled[s.table[i]] = std::max<int32_t>(filled[s.table[i]], static_cast<int32_t>(f));
    }
  }
  int64_t total_filled = 0;
  for (int32_t f : filled) total_filled += f;
  out->total_blocks = bm->num_blocks;
  out->free_blocks = static_cast<int32_t>(bm->free_q.size());
  out->evictable_blocks = static_cast<int32_t>(bm->evictable.size());
  out->used_blocks = bm->num_blocks - out->free_blocks - out->evictable_blocks;
  out->cached_blocks = 0;
  for (char c : bm->cached) out->cached_blocks += c;
  out->prefix_query_tokens = bm->prefix_query_tokens;
  out->prefix_hit_tokens = bm->prefix_hit_tokens;
  out->live_seqs = static_cast<int32_t>(bm->seqs.size());
  out->host_blocks = bm->num_host_blocks;
  out->host_free_blocks = static_cast<int32_t>(bm->host_free.size());
  out->swapped_seqs = static_cast<int32_t>(bm->swapped.size());
  out->filled_slots = total_filled;
  out->utilization = static_cast<double>(out->used_blocks) / bm->num_blocks;
  out->slot_utilization =
      out->used_blocks ? static_cast<double>(total_filled) / (static_cast<double>(out->used_blocks) * bm->bs)
                       : 0.0;
  return PKV_OK;
}

int pkv_bm_export(const pkv_bm* bm, const int64_t* seqs, int n_seqs, int32_t* tables_out,
                  int max_blocks, int32_t* ctx_lens_out) {
  if (!bm || n_seqs < 0 || max_blocks < 0) return PKV_ERR_INVALID;
  if (n_seqs > 0 && (!seqs || !tables_out || !ctx_lens_out)) return PKV_ERR_INVALID;
  for (int i = 0; i < n_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PKV_ERR_NO_SEQ;
    if (static_cast<int>(it->second.table.size()) > max_blocks) return PKV_ERR_INVALID;
  }
  for (int i = 0; i < n_seqs; ++i) {
    const Seq& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + max_blocks, -1);
    ctx_lens_out[i] = static_cast<int32_t>(s.count);
  }
  return PKV_OK;
}

// Runs of consecutive batch entries whose tables start with the same full
// blocks. Forked sequences and prefix-cache hits hold one physical block at
// the same table position, so one read of it serves the whole run.
int pkv_bm_prefix_groups(const pkv_bm* bm, const int64_t* seqs, int n_seqs, int max_members,
                         int32_t* group_first, int32_t* group_size, int32_t* group_prefix, int cap,
                         int* num_groups) {
  if (!bm || !num_groups || n_seqs < 0 || max_members < 1 || cap < 0) return PKV_ERR_INVALID;
  if (n_seqs > 0 && !seqs) return PKV_ERR_INVALID;
  std::vector<const Seq*> s(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PKV_ERR_NO_SEQ;
    s[i] = &it->second;
  }
  const int64_t bs = bm->bs;
  // the first block if the sequence holds it in full, else -1
  auto head = [&](int i) { return s[i]->count >= bs ? s[i]->table[0] : -1; };
  struct G {
    int first, size, prefix;
  };
  std::vector<G> out;
  for (int i = 0; i < n_seqs;) {
    const int32_t h = head(i);
    int j = i + 1;
    if (h >= 0)
      while (j < n_seqs && j - i < max_members && head(j) == h) ++j;
    if (j - i >= 2) {
      int64_t n = 0;
      for (;; ++n) {
        bool same = true;
        for (int m = i; m < j && same; ++m)
          same = (n + 1) * bs <= s[m]->count && s[m]->table[n] == s[i]->table[n];
        if (!same) break;
      }
      out.push_back(G{i, j - i, static_cast<int>(n * bs)});
    }
    i = j;
  }
  if (static_cast<int>(out.size()) > cap || (!out.empty() && (!group_first || !group_size || !group_prefix)))
    return PKV_ERR_INVALID;
  for (size_t g = 0; g < out.size(); ++g) {
    group_first[g] = out[g].first;
    group_size[g] = out[g].size;
    group_prefix[g] = out[g].prefix;
  }
  *num_groups = static_cast<int>(out.size());
  return PKV_OK;
}

}  // extern "C"
