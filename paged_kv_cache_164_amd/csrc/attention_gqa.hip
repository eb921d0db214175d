// Paged decode attention, phase 1, for fp16 / bf16 on the matrix cores (any group size 1..16).
//
// One wave handles one work item = (sequence, KV head, range of at most partition_size tokens),
// streaming it tile by tile (16 tokens) with an online softmax, so a wave needs no LDS and no
// barrier; the next tile's loads are in flight while a tile is computed.  Per tile:
//   S^T[t][g] = K[t][:] . Q[g][:]       v_mfma_f32_16x16x32 (bf16 / f16), G heads in N
//   online softmax per column g (base-2 logits, running max m and sum l)
//   O^T[d][g] += V^T[d][t] P^T[t][g]    v_mfma_f32_16x16x16, 16 dims x 16 heads tiles
// The QK output layout (lane = column g, four consecutive tokens per lane) is exactly the
// B-operand layout of the 16x16x16 product, so the weights never leave registers.
//
// Operands come straight from the paged layout of the "Vllm" page ("CacheEngine"):
//   key tile [D/8][bs][8]: lane (token l%16, dims 8*(l/16)..) = one 16-byte load;
//   value tile [D][bs]: lane (dim l%16, tokens 4*(l/16)..+4) = one 8-byte load, and the 64
//   lanes of one load cover 16 whole value rows (512 contiguous bytes at bs 16).
// Weights are rounded to the element type once; their sum comes from the matrix cores (a ones
// row times the same rounded weights).  The running maximum is lazy (kLazyRescale).
// Tokens past the context: logit -inf, weight 0, value entries zeroed before the product.
//
// Scheduling: workgroup t takes ticket t of the list that the plan kernel (work_plan.hip)
// filled: work item t / num_kv_heads, KV head t % num_kv_heads.  Every real item is therefore
// dispatched before any empty slot of the (upper-bound) grid, and whole partitions run before
// the short remainder chunks.  An item carries its token range, so no length has to be read
// before its first tiles can be requested.
//
// Shared-prefix decode uses the same item code with up to 16 / G sequences per item: when
// several sequences (beams, parallel samples) hold the same physical blocks for their first
// tokens, their query rows become the columns of one item over those tokens, so each shared
// block is read once per group rather than once per sequence (the memory sharing of
// PagedAttention, the mlqm.cn explainer, "PagedAttention" sharing and copy-on-write example).
// Column c is query head (c % G) of KV head kh in sequence b0 + c / G.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_tile_addr.h"

#include <algorithm>


namespace pkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma_k32(BF16, const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k32(F16, const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(BF16, const uint2& a, const uint2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(F16, const uint2& a, const uint2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                               __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Zero the 16-bit elements of an 8-byte value chunk whose token base + e is >= limit.
__device__ __forceinline__ uint2 mask4(uint2 v, int base, int limit) {
  const uint32_t m0 = ((base + 0 < limit) ? 0x0000ffffu : 0u) | ((base + 1 < limit) ? 0xffff0000u : 0u);
  const uint32_t m1 = ((base + 2 < limit) ? 0x0000ffffu : 0u) | ((base + 3 < limit) ? 0xffff0000u : 0u);
  return make_uint2(v.x & m0, v.y & m1);
}

// One item: tokens [tok0, tok_end) of the sequences b0 .. b0 + nseq - 1 (same blocks for all
// of them: table row b0 is used), KV head kh, partial slot `slot`.
template <class DT, int D, int BS>
__device__ __forceinline__ void gqa_item(const DecodeArgs& a, int G, int kh, int b0, int nseq,
                                         int tok0, int tok_end, int slot) {
  static_assert(DT::X == 8, "matrix-core path is for 16-bit element types");

  constexpr int KC = D / 32;   // 32-dim k-steps of the logit product
  constexpr int NDT = D / 16;  // 16-dim output tiles
  // Streaming (non-temporal) loads when a tile consumes whole cache lines of the value rows
  // (block_size <= 16); at block_size 32 a 16-token tile reads half of each 64-byte value row
  // and the next tile must find the other half in L2.
  constexpr bool kStream = BS <= 16;
  const int P = a.partition_size;
  const int Hkv = a.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int32_t* bt = a.block_tables + (int64_t)b0 * a.max_blocks + tok0 / BS;
  // The item's block ids (at most 128) go to two lane registers (entries past the row's end
  // are never read; entries past the context are unused).
  const int nmax = item_id_count(P, BS, a.max_blocks, tok0);
  const int ids0 = (lane < nmax) ? bt[lane] : 0;
  const int ids1 = (64 + lane < nmax) ? bt[64 + lane] : 0;
  const int h0 = kh * G;
  if (tok0 >= tok_end) {  // the sole item of an empty context
    for (int i = lane; i < G * D; i += 64)
      store_elem(DT(), a.out, ((int64_t)b0 * a.num_heads + h0) * D + i, 0.f);
    return;
  }
  const int ntok = tok_end - tok0;
  const int nslots = (ntok + BS - 1) / BS * BS;  // tokens covered by the item's blocks
  const int col = lane & 15;   // MFMA column: query head col % G of sequence b0 + col / G
  const int quad = lane >> 4;  // row group
  const int ncols = nseq * G;
  const int cseq = col / G;               // column's sequence, relative to b0
  const int chead = h0 + col - cseq * G;  // column's query head
  const int64_t crow = ((int64_t)b0 + cseq) * a.num_heads + chead;  // its row of q / out

  const int64_t tile_bytes = (int64_t)D * BS * 2;
  const int64_t block_bytes = tile_bytes * Hkv;
  const char* kbase = static_cast<const char*>(a.key_cache) + kh * tile_bytes;
  const char* vbase = static_cast<const char*>(a.value_cache) + kh * tile_bytes;
  auto block_of = [&](int j) -> int64_t {
    j = min(j, 127);  // a lookahead past the last block is never used for a load
    return (j < 64) ? __builtin_amdgcn_readlane(ids0, j) : __builtin_amdgcn_readlane(ids1, j - 64);
  };
  // One 16-token tile: KC 16-byte key chunks and NDT 8-byte value chunks per lane.  Lanes
  // whose tokens lie past the partition's blocks load nothing.
  struct Tile {
    uint4 k[KC];
    uint2 v[NDT];
  };
  const int ntiles = (ntok + 15) / 16;  // tiles holding at least one token of the partition
  const int last = ntiles - 1;
  // Loads are issued without branches (a load under a branch makes the compiler wait for every
  // outstanding load at the next use, which would serialise the double buffering).  With
  // block_size >= 16 every lane of a tile below ntok lies inside the partition's blocks; with
  // block_size 8 a lane past the last block reads block 0 and masks the data to zero
  // (gqa_lane, pkv_tile_addr.h).
  auto load_tile = [&](int t0, Tile& tl) {
    const GqaLane ln = gqa_lane<BS>(t0, col, quad, nslots, last, block_of(t0 / BS),
                                    BS < 16 ? block_of(t0 / BS + 1) : 0);
    // Tiles past the last one (the ring's prefetches at the end of the item) read the small
    // shared prefetch pad of the workspace instead, which stays in L2: no branch, no HBM re-read.
    const char* kp = (ln.pad ? a.prefetch_pad : kbase + ln.kblk * block_bytes) + ln.koff * 16;
    const char* vp = (ln.pad ? a.prefetch_pad : vbase + ln.vblk * block_bytes) + ln.voff * 2;
    const uint32_t km = ln.kvalid ? ~0u : 0u, vm = ln.vvalid ? ~0u : 0u;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      tl.k[kc] = kv_load<kStream>(reinterpret_cast<const uint4*>(kp + gqa_key_chunk<BS>(kc, quad)));
      if constexpr (BS < 16) tl.k[kc] = make_uint4(tl.k[kc].x & km, tl.k[kc].y & km, tl.k[kc].z & km, tl.k[kc].w & km);
    }
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
      tl.v[i] = kv_load<kStream>(reinterpret_cast<const uint2*>(vp + gqa_value_row<BS>(i, col)));
      if constexpr (BS < 16) tl.v[i] = make_uint2(tl.v[i].x & vm, tl.v[i].y & vm);
    }
  };

  // Q^T as the B operand of the logit product: lane holds Q[col][32 kc + 8 quad .. +8].  Unused
  // columns (col >= ncols) load the first column's row; their results are never stored.
  // These loads go out before the first tiles': the wait counter retires loads in issue order,
  // so a query load issued after the tile prologue would make the first product (and, through
  // the loop's merged wait state, every later one) wait for the tiles behind it as well.
  uint4 qop[KC];
  {
    const int64_t qrow = (col < ncols) ? crow : (int64_t)b0 * a.num_heads + h0;
    const uint4* qv = reinterpret_cast<const uint4*>(static_cast<const char*>(a.query) + qrow * D * 2);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qop[kc] = qv[kc * 4 + quad];
  }
  const int np_col = a.np_of[b0 + min(cseq, nseq - 1)];  // partial results of the column's sequence

  // The loads of the next three tiles are in flight while a tile is being computed (a ring of
  // four tile buffers); prefetches past the last tile read the prefetch pad.
  Tile T0, T1, T2, T3;
  load_tile(0, T0);
  load_tile(16, T1);
  load_tile(32, T2);

  f32x4 oacc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // reference maximum of column col (base-2 units), lazily moved
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};  // column col's sum of weights (all four rows)
  const uint2 ones = make_uint2(one_bits(DT()), one_bits(DT()));

  auto compute_tile = [&](int t0, Tile& tl) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) s = mma_k32(DT(), tl.k[kc], qop[kc], s);
    s *= a.scale_log2;
    if (t0 + 16 > ntok) {  // tokens past the item (only in its last tile): -inf
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (t0 + quad * 4 + r >= ntok) s[r] = -INFINITY;
    }
    float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // Lazy maximum: a column moves its reference (and rescales) only when the tile's maximum
    // exceeds it by more than kLazyRescale; the wave branches if any column needs it, and the
    // other columns' alpha is exactly 1.  The first tile holds a token, so every column moves
    // (alpha 0 from m = -inf); a tile past the end has only -inf logits and changes nothing.
    const bool need = tmax > m_run + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? tmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      lacc *= alpha;
#pragma unroll
      for (int i = 0; i < NDT; ++i) oacc[i] *= alpha;
    }
    // weights (at most 2^8; v_exp_f32 flushes those below 2^-126 to 0) rounded once to the
    // element type; the same values feed the sum (a ones row on the matrix cores) and P.V
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(s[r] - m_run);
    const uint2 pop = make_uint2(pack2(DT(), p[0], p[1]), pack2(DT(), p[2], p[3]));
    const int tv = t0 + quad * 4;
    if (tv + 4 > ntok) {
#pragma unroll
      for (int i = 0; i < NDT; ++i) tl.v[i] = mask4(tl.v[i], tv, ntok);
    }
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = mma_k16(DT(), tl.v[i], pop, oacc[i]);
    lacc = mma_k16(DT(), ones, pop, lacc);
  };

  // Computes of tiles past the end (at most three) are not skipped: a branch around them would
  // make the compiler's wait bookkeeping conservative; they change nothing (see above).
  for (int i = 0; i < ntiles; i += 4) {
    load_tile((i + 3) * 16, T3);
    compute_tile(i * 16, T0);
    load_tile((i + 4) * 16, T0);
    compute_tile((i + 1) * 16, T1);
    load_tile((i + 5) * 16, T1);
    compute_tile((i + 2) * 16, T2);
    load_tile((i + 6) * 16, T2);
    compute_tile((i + 3) * 16, T3);
  }

  // ---- epilogue: lane holds O[col][d = 16 i + 4 quad + r] and its column's sum of weights
  const float l_tot = lacc[0];
  if (col < ncols) {
    if (np_col <= 1) {  // the column's sequence has no other item: final output
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store_elem(DT(), a.out, crow * D + i * 16 + quad * 4 + r, oacc[i][r] * inv);
    } else {
      const int64_t sp = crow * a.slots + slot;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
        *reinterpret_cast<f32x4*>(&a.part_acc[sp * D + i * 16 + quad * 4]) = oacc[i];
      if (quad == 0) {
        a.part_m[sp] = m_run;
        a.part_l[sp] = l_tot;
      }
    }
  }
}

// One workgroup per ticket of the plan's list (the grid is an upper bound: workgroups past the
// list's end exit at once, after every real item has been dispatched).
template <class DT, int D, int BS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void gqa_grid_kernel(DecodeArgs a, int G) {
  const int Hkv = a.num_kv_heads;
  const int t = blockIdx.x;
  if (t >= int(a.queue[1]) * Hkv) return;
  const uint4 it = a.items[t / Hkv];
  if (!item_fits(a, it)) return;
  gqa_item<DT, D, BS>(a, G, t % Hkv, int(it.x), int(it.y & 255u), int(it.z), int(it.w),
                      int(it.y >> 8));
}

template <class DT, int D, int BS>
hipError_t launch_t(const DecodeArgs& a, int group, hipStream_t stream) {
  if (a.plan_mode != 2) {
    const hipError_t e = launch_plan(a, BS, 16 / group, stream);
    if (e != hipSuccess || a.plan_mode == 1) return e;
  }
  const int64_t grid = (int64_t)a.num_seqs * a.num_kv_heads * a.slots;
  hipLaunchKernelGGL((gqa_grid_kernel<DT, D, BS>), dim3((unsigned)grid), dim3(64), 0, stream, a,
                     group);
  return hipGetLastError();
}

template <class DT, int D>
hipError_t by_block(const DecodeArgs& a, int bs, int group, hipStream_t s) {
  switch (bs) {
    case 8: return launch_t<DT, D, 8>(a, group, s);
    case 16: return launch_t<DT, D, 16>(a, group, s);
    case 32: return launch_t<DT, D, 32>(a, group, s);
  }
  return hipErrorInvalidValue;
}

template <class DT>
hipError_t by_head(const DecodeArgs& a, int D, int bs, int group, hipStream_t s) {
  switch (D) {
    case 64: return by_block<DT, 64>(a, bs, group, s);
    case 128: return by_block<DT, 128>(a, bs, group, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Any group size fits: an item holds 16 / G sequences (one for G > 8).
bool gqa_supported(int dtype, int head_size, int block_size, int group) {
  return (dtype == 1 || dtype == 2) && (head_size == 64 || head_size == 128) &&
         (block_size == 8 || block_size == 16 || block_size == 32) && group >= 1 && group <= 16;
}

hipError_t launch_decode_gqa(const DecodeArgs& a, int dtype, int head_size, int block_size,
                             int group, hipStream_t stream) {
  switch (dtype) {
    case 1: return by_head<F16>(a, head_size, block_size, group, stream);
    case 2: return by_head<BF16>(a, head_size, block_size, group, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
