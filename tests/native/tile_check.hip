// Host-side check of the decode kernels' load addresses.  Test infrastructure: built as a
// host-only library beside the tests, never linked into libpkv.
//
// The kernels take every address of their key and value tile loads from pkv_tile_addr.h.  This
// file runs those same functions on the host, over the work items of a decode call, for every
// lane of every tile the kernels' load ring requests, and counts the loads that would leave the
// block pool or the workspace's prefetch pad.  The block ids come from the block table the way
// the kernels fetch them: entry j of an item for j below item_id_count, 0 above, lookups past
// the id registers clamped to the last one.  Table entries past a sequence's blocks are -1 in
// the tests, so a lane that takes one as a block id shows up as a load below the pool.
//
// The work items come from a host planner written with the plan kernel's cut rules (whole
// partitions, remainder chunks, shared-prefix groups; pkv_tile_addr.h); a GPU test compares its
// list with the one the plan kernel writes.
//
// A "planted" variant of each pick (the guard that sends lanes past an item's last block to
// block 0 left out) is here too, so that a test can show the check catches that mistake.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "pkv_internal.h"
#include "pkv_tile_addr.h"

namespace {

using namespace pkv;

struct Item {
  uint32_t b0, y, begin, end;
};

struct Checker {
  int64_t pool_bytes;
  int64_t bad = 0;
  char* msg;
  int msg_len;
  // one load of `size` bytes at `off` from the cache base (pool) or from the pad
  void load(bool pad, int64_t off, int size, const Item& it, int kh, int tile, int lane,
            const char* what) {
    const int64_t limit = pad ? (int64_t)kPrefetchPad : pool_bytes;
    if (off >= 0 && off + size <= limit) return;
    if (bad++ == 0 && msg && msg_len > 0)
      snprintf(msg, msg_len,
               "%s load out of %s: item (seq %u, tokens %u..%u) kv head %d tile %d lane %d "
               "offset %lld size %d limit %lld",
               what, pad ? "the pad" : "the pool", it.b0, it.begin, it.end, kh, tile, lane,
               (long long)off, size, (long long)limit);
  }
};

// The item's block id at entry j (as the kernels read it from their id registers).
struct ItemIds {
  const int32_t* row;  // table row of the item's first sequence, from entry tok0 / bs
  int nmax;
  int nregs;           // ids the registers hold: 128 (16-bit kernel) or 256 (8-bit)
  int64_t at(int j) const {
    j = std::min(j, nregs - 1);
    return j < nmax ? row[j] : 0;
  }
};

// ---- 16-bit kernel ------------------------------------------------------------------------------
template <int BS>
GqaLane planted_gqa_lane(int t0, int col, int quad, int nslots, int last, int64_t lo, int64_t hi) {
  GqaLane r = gqa_lane<BS>(t0, col, quad, nslots, last, lo, hi);
  if constexpr (BS < 16) {  // no guard: a lane past the last block takes the next table entry
    r.kblk = (col < BS) ? lo : hi;
    r.vblk = (quad * 4 < BS) ? lo : hi;
  }
  return r;
}

template <int D, int BS>
void check_gqa(Checker& ck, bool planted, const int32_t* tables, int max_blocks, int Hkv, int P,
               const Item& it) {
  constexpr int KC = D / 32, NDT = D / 16;
  const int64_t tile_bytes = (int64_t)D * BS * 2, block_bytes = tile_bytes * Hkv;
  const int tok0 = it.begin, ntok = (int)it.end - (int)it.begin;
  if (ntok <= 0) return;
  const ItemIds ids{tables + (int64_t)it.b0 * max_blocks + tok0 / BS,
                    item_id_count(P, BS, max_blocks, tok0), kMaxItemBlocks};
  const int nslots = (ntok + BS - 1) / BS * BS;
  const int ntiles = (ntok + 15) / 16, last = ntiles - 1;
  for (int kh : {0, Hkv - 1}) {
    for (int ti = 0; ti <= ring_last_tile(ntiles); ++ti) {
      const int t0 = ti * 16;
      const int64_t lo = ids.at(t0 / BS), hi = BS < 16 ? ids.at(t0 / BS + 1) : 0;
      for (int lane = 0; lane < 64; ++lane) {
        const int col = lane & 15, quad = lane >> 4;
        const GqaLane ln = planted ? planted_gqa_lane<BS>(t0, col, quad, nslots, last, lo, hi)
                                   : gqa_lane<BS>(t0, col, quad, nslots, last, lo, hi);
        const int64_t kb = (ln.pad ? 0 : kh * tile_bytes + ln.kblk * block_bytes) + ln.koff * 16;
        const int64_t vb = (ln.pad ? 0 : kh * tile_bytes + ln.vblk * block_bytes) + ln.voff * 2;
        for (int kc = 0; kc < KC; ++kc)
          ck.load(ln.pad, kb + gqa_key_chunk<BS>(kc, quad), 16, it, kh, ti, lane, "key");
        for (int i = 0; i < NDT; ++i)
          ck.load(ln.pad, vb + gqa_value_row<BS>(i, col), 8, it, kh, ti, lane, "value");
      }
    }
  }
}

// ---- 8-bit kernel -------------------------------------------------------------------------------
template <int BS>
int64_t planted_kv8_pick(int c0, int c1, int c2, int c3, int t0, int t, int nslots) {
  (void)t0;
  (void)nslots;
  return kv8_pick<BS>(c0, c1, c2, c3, 0, t, 1 << 30);  // no guard: every lane takes its entry
}

template <int D, int BS>
void check_kv8(Checker& ck, bool planted, const int32_t* tables, int max_blocks, int Hkv, int P,
               const Item& it) {
  constexpr int TT = 32, KJ = D / 64, NDT = D / 16, NBT = TT / BS;
  const int64_t tile_bytes = (int64_t)D * BS, block_bytes = tile_bytes * Hkv;
  const int tok0 = it.begin, ntok = (int)it.end - (int)it.begin;
  if (ntok <= 0) return;
  const ItemIds ids{tables + (int64_t)it.b0 * max_blocks + tok0 / BS,
                    item_id_count(P, BS, max_blocks, tok0), kMaxItemBlocks8};
  const int nslots = (ntok + BS - 1) / BS * BS;
  const int ntiles = (ntok + TT - 1) / TT, last = ntiles - 1;
  for (int kh : {0, Hkv - 1}) {
    for (int ti = 0; ti <= ring_last_tile(ntiles); ++ti) {
      const int t0 = ti * TT, j0 = t0 / BS;
      int cand[NBT];
      for (int k = 0; k < NBT; ++k) cand[k] = (int)ids.at(j0 + k);
      auto pick = [&](int t) {
        const int c0 = cand[0], c1 = cand[NBT > 1 ? 1 : 0], c2 = cand[NBT > 2 ? 2 : 0],
                  c3 = cand[NBT > 3 ? 3 : 0];
        return planted ? planted_kv8_pick<BS>(c0, c1, c2, c3, t0, t, nslots)
                       : kv8_pick<BS>(c0, c1, c2, c3, t0, t, nslots);
      };
      const bool pad = kv8_pad(t0, last);
      for (int lane = 0; lane < 64; ++lane) {
        const int col = lane & 15, quad = lane >> 4;
        const int ktok[2] = {col, 16 + col}, vtok = 8 * quad;
        for (int r = 0; r < 2; ++r) {
          const int64_t kb = (pad ? 0 : kh * tile_bytes + pick(ktok[r]) * block_bytes) +
                             kv8_key_row<BS>(ktok[r]);
          for (int j = 0; j < KJ; ++j)
            ck.load(pad, kb + kv8_key_chunk<BS>(quad + 4 * j), 16, it, kh, ti, lane, "key");
        }
        const int64_t vb = (pad ? 0 : kh * tile_bytes + pick(vtok) * block_bytes) +
                           kv8_value_run<BS>(vtok);
        for (int i = 0; i < NDT; ++i)
          ck.load(pad, vb + kv8_value_row<BS>(i * 16 + col), 8, it, kh, ti, lane, "value");
      }
    }
  }
}

template <int D, int BS>
void check_one(Checker& ck, int kernel, bool planted, const int32_t* tables, int max_blocks,
               int Hkv, int P, const Item& it) {
  if (kernel == 0)
    check_gqa<D, BS>(ck, planted, tables, max_blocks, Hkv, P, it);
  else
    check_kv8<D, BS>(ck, planted, tables, max_blocks, Hkv, P, it);
}

// Host planner: the plan kernel's items (work_plan.hip), in any order.
struct Planner {
  int P, Q;
  Item* out;
  int64_t cap, n = 0;
  void put(int b0, int nseq, int slot, int begin, int end) {
    if (n < cap) out[n] = Item{uint32_t(b0), uint32_t(nseq) | (uint32_t(slot) << 8), uint32_t(begin), uint32_t(end)};
    ++n;
  }
  int range(int b0, int nseq, int s, int e, int slot) {
    const int F = whole_parts(e - s, P);
    for (int j = 0; j < F; ++j) put(b0, nseq, slot++, s + j * P, s + (j + 1) * P);
    for (int t0 = s + F * P; t0 < e; t0 = chunk_end(t0, e, Q)) put(b0, nseq, slot++, t0, chunk_end(t0, e, Q));
    return slot;
  }
};

}  // namespace

extern "C" {

// Partition size and remainder chunk of the library's decode calls (0: auto).
int pkv_tilecheck_partition(int kv8, int block_size, int max_context_len, int partition_size) {
  return partition_size > 0 ? partition_size
                            : auto_partition(true, kv8 != 0, block_size, max_context_len);
}
int pkv_tilecheck_tail_chunk(int P, int block_size) { return tail_chunk(P, block_size); }

// Workspace offsets of the plan's item list and item count (bytes), as the library lays them out.
int64_t pkv_tilecheck_items_offset(int num_seqs, int num_heads, int head_size, int max_context_len,
                                   int partition_size) {
  const int64_t slots = layout_slots(max_context_len, partition_size);
  return (int64_t)workspace_layout(num_seqs, num_heads, head_size, slots).items_off;
}

// Workspace offset of the per-sequence item counts (bytes).
int64_t pkv_tilecheck_counts_offset(int num_seqs, int num_heads, int head_size, int max_context_len,
                                    int partition_size) {
  const int64_t slots = layout_slots(max_context_len, partition_size);
  return (int64_t)workspace_layout(num_seqs, num_heads, head_size, slots).np_off;
}

// The plan's items for the given lengths (group arrays may be null: every sequence a group of
// its own).  Writes up to `cap` items (4 x uint32 each) and each sequence's item count; returns
// the number of items.
int64_t pkv_tilecheck_plan(const int32_t* lens, int num_seqs, int len_limit, int P, int Q, int bs,
                           const int32_t* group_starts, const int32_t* prefix_lens, int num_groups,
                           int per_item, uint32_t* items, int64_t cap, int32_t* np_of) {
  Planner pl{P, Q, reinterpret_cast<Item*>(items), cap};
  auto len_of = [&](int b) { return std::min(std::max(lens[b], 0), len_limit); };
  const int ngroups = group_starts ? num_groups : num_seqs;
  for (int b = 0; b < num_seqs; ++b) np_of[b] = 0;
  for (int g = 0; g < ngroups; ++g) {
    int s0 = g, s1 = g + 1, pre = 0;
    if (group_starts) {
      s0 = std::min(std::max(group_starts[g], 0), num_seqs);
      s1 = std::min(std::max(group_starts[g + 1], s0), num_seqs);
      if (s1 - s0 >= 2) {
        int p = std::min(std::max(prefix_lens[g], 0), len_limit);
        for (int b = s0; b < s1; ++b) p = std::min(p, std::max(lens[b], 0));
        pre = p - p % bs;
      }
    }
    int npre = 0;
    for (int c0 = s0; c0 < s1; c0 += per_item) npre = pl.range(c0, std::min(per_item, s1 - c0), 0, pre, 0);
    for (int b = s0; b < s1; ++b) {
      const int L = len_of(b);
      const int n = pl.range(b, 1, pre, L, npre);
      if (L == 0) pl.put(b, 1, 0, 0, 0);
      np_of[b] = std::max(n, 1);
    }
  }
  return pl.n;
}

// Loads outside the pool or the pad over all items, for the 16-bit kernel (kernel 0) or the
// 8-bit one (kernel 1); planted = 1 runs the unguarded picks.  The first violation is described
// in msg.  Returns -1 for shapes the kernels do not build.
int64_t pkv_tilecheck_loads(int kernel, int planted, const int32_t* tables, int max_blocks,
                            int64_t num_blocks, int num_kv_heads, int head_size, int block_size,
                            int P, const uint32_t* items, int64_t n_items, char* msg, int msg_len) {
  const int64_t elem = kernel == 0 ? 2 : 1;
  Checker ck{num_blocks * num_kv_heads * head_size * block_size * elem, 0, msg, msg_len};
  if (msg && msg_len > 0) msg[0] = 0;
  const Item* it = reinterpret_cast<const Item*>(items);
  for (int64_t i = 0; i < n_items; ++i) {
#define PKV_CASE(DD, BB)                                                                        \
  if (head_size == DD && block_size == BB) {                                                   \
    check_one<DD, BB>(ck, kernel, planted != 0, tables, max_blocks, num_kv_heads, P, it[i]); \
    continue;                                                                                  \
  }
    PKV_CASE(64, 8) PKV_CASE(64, 16) PKV_CASE(64, 32)
    PKV_CASE(128, 8) PKV_CASE(128, 16) PKV_CASE(128, 32)
#undef PKV_CASE
    return -1;
  }
  return ck.bad;
}

}  // extern "C"
