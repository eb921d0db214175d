// Host block manager of the paged KV cache: the contract is in include/pkv_block_manager.h.
// Pure host C++ (no GPU calls): per-pool reference counts and ordered free sets, per-sequence
// block tables.  Every call checks everything it needs first and changes nothing on error.
#include "pkv_block_manager.h"

#include <cmath>
#include <cstdint>
#include <set>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

struct Pool {
  std::vector<int32_t> ref;   // references per block, 0 = free
  std::set<int32_t> free_ids;  // the lowest id is handed out first

  explicit Pool(int32_t n) : ref(size_t(n), 0) {
    for (int32_t i = 0; i < n; ++i) free_ids.insert(i);
  }
  int32_t size() const { return int32_t(ref.size()); }
  int32_t num_free() const { return int32_t(free_ids.size()); }
  int32_t take() {  // caller checked num_free() > 0
    const int32_t id = *free_ids.begin();
    free_ids.erase(free_ids.begin());
    ref[size_t(id)] = 1;
    return id;
  }
  void release(int32_t id) {
    if (--ref[size_t(id)] == 0) free_ids.insert(id);
  }
};

struct Seq {
  int64_t len = 0;
  int device = PKV_DEVICE_GPU;
  std::vector<int32_t> table;
};

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

}  // namespace

struct pkv_block_manager {
  int32_t block_size;
  Pool gpu, cpu;
  int32_t watermark_blocks;
  std::unordered_map<int64_t, Seq> seqs;

  pkv_block_manager(int32_t bs, int32_t ngpu, int32_t ncpu, int32_t wm)
      : block_size(bs), gpu(ngpu), cpu(ncpu), watermark_blocks(wm) {}
  Pool& pool(int device) { return device == PKV_DEVICE_GPU ? gpu : cpu; }
  const Pool& pool(int device) const { return device == PKV_DEVICE_GPU ? gpu : cpu; }
};

namespace {

int fail(int code, const std::string& msg) { return pkv::record_error(code, msg); }

const Seq* find(const pkv_block_manager* bm, int64_t id) {
  auto it = bm->seqs.find(id);
  return it == bm->seqs.end() ? nullptr : &it->second;
}

// Move every block of the given sequences from pool `from` to pool `to` (see the header).
int swap(pkv_block_manager* bm, const int64_t* ids, int32_t n, int from, int to, int64_t* pairs,
         int32_t cap, int32_t* num_pairs) {
  if (!bm || n < 0 || (n > 0 && !ids) || !num_pairs || cap < 0 || (cap > 0 && !pairs))
    return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  std::unordered_set<int64_t> seen;
  std::vector<int32_t> order;                   // distinct blocks, first appearance first
  std::unordered_map<int32_t, int32_t> inside;  // block -> references from these sequences
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = find(bm, ids[i]);
    if (!s) return fail(PKV_ERR_INVALID_ARG, "unknown sequence " + std::to_string(ids[i]));
    if (s->device != from) return fail(PKV_ERR_INVALID_ARG, "sequence is not in the source pool");
    if (!seen.insert(ids[i]).second) return fail(PKV_ERR_INVALID_ARG, "sequence listed twice");
    for (int32_t b : s->table)
      if (inside[b]++ == 0) order.push_back(b);
  }
  Pool& src = bm->pool(from);
  Pool& dst = bm->pool(to);
  for (int32_t b : order)
    if (inside[b] != src.ref[size_t(b)])
      return fail(PKV_ERR_INVALID_ARG, "block " + std::to_string(b) +
                                           " is shared with a sequence outside the set");
  if (int32_t(order.size()) > dst.num_free())
    return fail(PKV_ERR_WORKSPACE, "not enough free blocks in the target pool");
  if (int32_t(order.size()) > cap) return fail(PKV_ERR_WORKSPACE, "pairs buffer too small");
  std::unordered_map<int32_t, int32_t> moved;
  int32_t k = 0;
  for (int32_t b : order) {
    const int32_t nb = dst.take();
    dst.ref[size_t(nb)] = src.ref[size_t(b)];
    src.ref[size_t(b)] = 0;
    src.free_ids.insert(b);
    moved[b] = nb;
    pairs[2 * k] = b;
    pairs[2 * k + 1] = nb;
    ++k;
  }
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = bm->seqs[ids[i]];
    for (int32_t& b : s.table) b = moved[b];
    s.device = to;
  }
  *num_pairs = k;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t block_size, int32_t num_gpu_blocks, int32_t num_cpu_blocks,
                                 float watermark) {
  if (block_size <= 0 || num_gpu_blocks < 0 || num_cpu_blocks < 0 || !(watermark >= 0.f) ||
      !(watermark < 1.f)) {
    fail(PKV_ERR_INVALID_ARG, "bad block manager sizes");
    return nullptr;
  }
  try {
    return new pkv_block_manager(block_size, num_gpu_blocks, num_cpu_blocks,
                                 int32_t(watermark * float(num_gpu_blocks)));
  } catch (...) {
    fail(PKV_ERR_INVALID_ARG, "out of host memory");
    return nullptr;
  }
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_can_allocate(const pkv_block_manager* bm, int32_t num_tokens) {
  if (!bm || num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  const int64_t need = blocks_for(num_tokens, bm->block_size);
  if (int64_t(bm->gpu.size()) - need < bm->watermark_blocks) return PKV_ALLOC_NEVER;
  if (int64_t(bm->gpu.num_free()) - need >= bm->watermark_blocks) return PKV_ALLOC_OK;
  return PKV_ALLOC_LATER;
}

int pkv_bm_allocate(pkv_block_manager* bm, int64_t seq_id, int32_t num_tokens) {
  try {
    if (!bm || num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
    if (find(bm, seq_id)) return fail(PKV_ERR_INVALID_ARG, "sequence exists");
    const int64_t need = blocks_for(num_tokens, bm->block_size);
    if (need > bm->gpu.num_free()) return fail(PKV_ERR_WORKSPACE, "not enough free GPU blocks");
    Seq s;
    s.len = num_tokens;
    for (int64_t j = 0; j < need; ++j) s.table.push_back(bm->gpu.take());
    bm->seqs.emplace(seq_id, std::move(s));
    return PKV_OK;
  } catch (...) {
    return fail(PKV_ERR_INVALID_ARG, "out of host memory");
  }
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  try {
    if (!bm) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
    const Seq* p = find(bm, parent);
    if (!p) return fail(PKV_ERR_INVALID_ARG, "unknown parent");
    if (find(bm, child)) return fail(PKV_ERR_INVALID_ARG, "child exists");
    Seq c = *p;
    Pool& pool = bm->pool(c.device);
    for (int32_t b : c.table) ++pool.ref[size_t(b)];
    bm->seqs.emplace(child, std::move(c));
    return PKV_OK;
  } catch (...) {
    return fail(PKV_ERR_INVALID_ARG, "out of host memory");
  }
}

int pkv_bm_can_append(const pkv_block_manager* bm, int32_t num_seqs) {
  if (!bm || num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  return num_seqs <= bm->gpu.num_free() ? 1 : 0;
}

int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int64_t* slot, int64_t* cow_src,
                  int64_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PKV_ERR_INVALID_ARG, "unknown sequence");
  Seq& s = it->second;
  if (s.device != PKV_DEVICE_GPU) return fail(PKV_ERR_INVALID_ARG, "sequence is swapped out");
  const int32_t bs = bm->block_size;
  const int64_t t = s.len;  // index of the new token
  int64_t src = -1, dst = -1;
  if (int64_t(s.table.size()) < blocks_for(t + 1, bs)) {  // the token starts a new block
    if (bm->gpu.num_free() == 0) return fail(PKV_ERR_WORKSPACE, "no free GPU block");
    s.table.push_back(bm->gpu.take());
  } else if (bm->gpu.ref[size_t(s.table.back())] > 1) {  // shared last block: copy on write
    if (bm->gpu.num_free() == 0) return fail(PKV_ERR_WORKSPACE, "no free GPU block");
    const int32_t old = s.table.back();
    const int32_t nb = bm->gpu.take();
    --bm->gpu.ref[size_t(old)];  // still > 0: other sequences hold it
    s.table.back() = nb;
    src = old;
    dst = nb;
  }
  s.len = t + 1;
  *slot = int64_t(s.table[size_t(t / bs)]) * bs + t % bs;
  *cow_src = src;
  *cow_dst = dst;
  return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PKV_ERR_INVALID_ARG, "unknown sequence");
  Pool& pool = bm->pool(it->second.device);
  for (int32_t b : it->second.table) pool.release(b);
  bm->seqs.erase(it);
  return PKV_OK;
}

int pkv_bm_swap_out(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n, int64_t* pairs,
                    int32_t cap, int32_t* num_pairs) {
  try {
    return swap(bm, seq_ids, n, PKV_DEVICE_GPU, PKV_DEVICE_CPU, pairs, cap, num_pairs);
  } catch (...) {
    return fail(PKV_ERR_INVALID_ARG, "out of host memory");
  }
}

int pkv_bm_swap_in(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n, int64_t* pairs,
                   int32_t cap, int32_t* num_pairs) {
  try {
    return swap(bm, seq_ids, n, PKV_DEVICE_CPU, PKV_DEVICE_GPU, pairs, cap, num_pairs);
  } catch (...) {
    return fail(PKV_ERR_INVALID_ARG, "out of host memory");
  }
}

int pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* table, int32_t cap,
                       int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !table)) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  const Seq* s = find(bm, seq_id);
  if (!s) return fail(PKV_ERR_INVALID_ARG, "unknown sequence");
  if (int64_t(s->table.size()) > cap) return fail(PKV_ERR_WORKSPACE, "table buffer too small");
  for (size_t j = 0; j < s->table.size(); ++j) table[j] = s->table[j];
  *n = int32_t(s->table.size());
  return PKV_OK;
}

int64_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  const Seq* s = find(bm, seq_id);
  return s ? s->len : fail(PKV_ERR_INVALID_ARG, "unknown sequence");
}

int pkv_bm_seq_device(const pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  const Seq* s = find(bm, seq_id);
  return s ? s->device : fail(PKV_ERR_INVALID_ARG, "unknown sequence");
}

int32_t pkv_bm_num_free(const pkv_block_manager* bm, int32_t device) {
  if (!bm || (device != PKV_DEVICE_GPU && device != PKV_DEVICE_CPU))
    return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  return bm->pool(device).num_free();
}

int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t device, int32_t block) {
  if (!bm || (device != PKV_DEVICE_GPU && device != PKV_DEVICE_CPU))
    return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  const Pool& p = bm->pool(device);
  if (block < 0 || block >= p.size()) return fail(PKV_ERR_INVALID_ARG, "block out of range");
  return p.ref[size_t(block)];
}

}  // extern "C"
