// Where the decode kernels' loads go: the work-item cuts of a token range and, per lane and
// tile, the physical block and the byte offsets of the key and value loads.  The kernels
// (attention_gqa.hip, attention_fp8.hip, work_plan.hip) compute their addresses with these
// functions, and a host-side check runs the same functions over whole work lists to show that
// every load stays inside the block pool or the workspace's prefetch pad.
//
// The block a token lives in: token t of a sequence is at block_tables[b][t / bs], offset
// t % bs (the mlqm.cn explainer, "PagedAttention" block table); a (block, KV head) key tile is
// [D/x][bs][x] and a value tile [D][bs] (the "Vllm" page, "CacheEngine").  Table entries past
// a sequence's last block are not block ids, so no lane may take one as an address.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define PKV_HD __host__ __device__ __forceinline__

namespace pkv {

// ---- work-item cuts (plan kernel) -------------------------------------------------------------
// A token range [s, e) becomes whole partitions of P tokens, then remainder chunks of at most
// Q tokens (Q a multiple of the block size).
PKV_HD int whole_parts(int n, int P) { return n / P; }
// Size class of a chunk of n (1 <= n <= Q) tokens: 1 (longest) .. 8 (shortest).
PKV_HD int chunk_class(int n, int Q) { return 1 + (7 < (Q - n) * 8 / Q ? 7 : (Q - n) * 8 / Q); }
// End of the chunk that starts at t0 (< e).
PKV_HD int chunk_end(int t0, int e, int Q) { return t0 + Q < e ? t0 + Q : e; }

// ---- block ids of an item ----------------------------------------------------------------------
// An item starting at token tok0 (a multiple of bs) holds the ids of its blocks, from table
// entry tok0 / bs on: entry j for j < nmax = min(P / bs, entries left in the row), 0 past that.
// Lookups beyond the id registers (j >= kIds) read the last one.
PKV_HD int item_id_count(int P, int bs, int max_blocks, int tok0) {
  const int left = max_blocks - tok0 / bs;
  return P / bs < left ? P / bs : left;
}

// ---- 16-bit kernel: 16-token tiles ------------------------------------------------------------
// Lane (col = lane % 16, quad = lane / 16) of the tile starting at item token t0 reads
//   key chunks kc = 0 .. D/32 - 1: 16 bytes at tile_base(kblk) + koff * 16 + gqa_key_chunk(kc, quad)
//   value rows i = 0 .. D/16 - 1:  8 bytes at tile_base(vblk) + voff * 2 + gqa_value_row(i, col)
// or, for a tile past the item's last one (a prefetch of the load ring), the same offsets from
// the start of the prefetch pad.
struct GqaLane {
  int64_t kblk, vblk;
  int koff, voff;       // token offset inside the block of the lane's key row / value run
  bool kvalid, vvalid;  // false: the lane's token lies past the item's blocks (data masked)
  bool pad;
};
// lo, hi: the item's block ids at entries t0 / BS and t0 / BS + 1; nslots: tokens of the
// item's blocks (its length rounded up to whole blocks); last: index of its last tile.
template <int BS>
PKV_HD GqaLane gqa_lane(int t0, int col, int quad, int nslots, int last, int64_t lo, int64_t hi) {
  GqaLane r;
  if constexpr (BS >= 16) {
    // a 16-token tile lies inside one block, and every tile up to the last one inside the
    // item's blocks
    r.kblk = r.vblk = lo;
    r.koff = t0 % BS + col;
    r.voff = t0 % BS + quad * 4;
    r.kvalid = r.vvalid = true;
  } else {
    // a tile spans two blocks; a lane past the item's last block reads block 0
    r.kvalid = t0 + col < nslots;
    r.vvalid = t0 + quad * 4 < nslots;
    r.kblk = !r.kvalid ? 0 : (col < BS) ? lo : hi;
    r.vblk = !r.vvalid ? 0 : (quad * 4 < BS) ? lo : hi;
    r.koff = col % BS;
    r.voff = (quad * 4) % BS;
  }
  r.pad = t0 > last * 16;
  return r;
}
template <int BS>
PKV_HD int64_t gqa_key_chunk(int kc, int quad) { return (int64_t)(kc * 4 + quad) * BS * 16; }
template <int BS>
PKV_HD int64_t gqa_value_row(int i, int col) { return (int64_t)(i * 16 + col) * BS * 2; }

// ---- 8-bit kernel: 32-token tiles -------------------------------------------------------------
// Lane (col, quad) reads key rows of tile tokens col and 16 + col, and the value run of tokens
// 8 quad .. + 8.  c0 .. c3 are the item's block ids at entries t0 / BS + 0 .. 3 (only the first
// 32 / BS are used).  A lane whose token lies past the item's last block reads block 0 (its
// data is masked): a tile can reach past the item's blocks when bs < 32, and the table entries
// there are not block ids.
template <int BS>
PKV_HD int64_t kv8_pick(int c0, int c1, int c2, int c3, int t0, int t, int nslots) {
  constexpr int NBT = 32 / BS;
  int r = c0;
  if constexpr (NBT == 2) {
    r = (t >= BS) ? c1 : c0;
  } else if constexpr (NBT == 4) {
    const int j = t / BS;
    const int lo = (j & 1) ? c1 : c0, hi = (j & 1) ? c3 : c2;
    r = (j & 2) ? hi : lo;
  }
  return (t0 + t < nslots) ? int64_t(r) : int64_t(0);
}
// Bytes from the start of a (block, KV head) tile (or of the pad): the key row of tile token t
// begins at kv8_key_row(t), and its chunk c (16 bytes: dims 16 c .. + 16) kv8_key_chunk(c)
// further; the value run of token t (8 bytes: tokens t .. t + 7) begins at kv8_value_run(t),
// and its row for head dim d kv8_value_row(d) further.
template <int BS>
PKV_HD int kv8_key_row(int t) { return (t % BS) * 16; }
template <int BS>
PKV_HD int64_t kv8_key_chunk(int64_t c) { return c * BS * 16; }
template <int BS>
PKV_HD int kv8_value_run(int t) { return t % BS; }
template <int BS>
PKV_HD int64_t kv8_value_row(int d) { return (int64_t)d * BS; }
// The tile at t0 is past the item's last tile (last = index of the last tile): the pad.
PKV_HD bool kv8_pad(int t0, int last) { return t0 > last * 32; }

// ---- the load ring ----------------------------------------------------------------------------
// Both kernels load tiles 0, 1, 2 first and then, for every group of four tiles i .. i + 3
// (i = 0, 4, ..., below ntiles), tiles i + 3 .. i + 6: the last tile index loaded.
PKV_HD int ring_last_tile(int ntiles) { return (ntiles + 3) / 4 * 4 + 2; }

}  // namespace pkv
