// Paged decode attention over an 8-bit KV cache (FP8 E4M3 or INT8 codes, one float scale per
// cache), query and output in fp16 / bf16, on the matrix cores.
//
// The cache layout is the "Vllm" page's ("CacheEngine") with x = 16 / sizeof = 16: a
// (block, KV head) key tile is [D/16][bs][16] bytes, a value tile [D][bs] bytes.  Codes are
// widened in registers to the query's type (exact: every E4M3 value and every integer code is a
// bf16 and an fp16 value); the key scale is folded into the logit scale and the value scale into the output,
// so no per-element multiply is spent on them.
//
// Same work items, scheduling, online softmax and epilogue as the 16-bit kernel
// (attention_gqa.hip), with 32-token tiles so that the P.V product is a 16x16x32 MFMA:
//   * row i of key row group r (r = 0, 1) is tile token 16 r + i, so the 16 lanes of a key
//     load read 16 consecutive tokens: whole 128-byte lines of the [D/16][bs][16] chunk (a
//     permuted order reading 4-token pieces cost 5% in a load-only probe);
//   * after the two 16x16x32 logit products lane (col, quad) holds the logits of tokens
//     4 quad .. + 4 (group 0) and 16 + 4 quad .. + 4 (group 1) of its column; two lane swaps
//     (v_permlane32_swap, then v_permlane16_swap, per dword of packed weights) regroup them so
//     that lane (col, quad) holds the weights of tokens 8 quad .. + 8 -- the B operand of the
//     16x16x32 P.V product, whose A operand (lane: one head dim, 8 consecutive tokens) is
//     one 8-byte load of a value row;
//   * a lane loads 16 dims of a key row at once (one 16-byte chunk); the two halves feed two
//     k-steps, so the query operand is loaded in the matching dim order.
#include "pkv_device.h"
#include "pkv_kv8.h"
#include "pkv_internal.h"
#include "pkv_tile_addr.h"
#include "pkv_kv8_host.h"

namespace pkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mma(BF16, const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(F16, const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Byte mask keeping the bytes of tokens base + e < limit (e = 0..3) of one dword.
__device__ __forceinline__ uint32_t keep4(int base, int limit) {
  return ((base + 0 < limit) ? 0x000000ffu : 0u) | ((base + 1 < limit) ? 0x0000ff00u : 0u) |
         ((base + 2 < limit) ? 0x00ff0000u : 0u) | ((base + 3 < limit) ? 0xff000000u : 0u);
}

template <class DT, int D, int BS, int CODE>
__device__ __forceinline__ void fp8_item(const DecodeArgs& a, int G, int kh, int b0, int nseq,
                                         int tok0, int tok_end, int slot) {
  constexpr int TT = 32;        // tokens per tile
  constexpr int KJ = D / 64;    // 16-byte key chunks per lane and row group
  constexpr int NDT = D / 16;   // 16-dim output tiles
  constexpr int NBT = TT / BS;  // blocks a tile spans (items start on block boundaries)
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  const int P = a.partition_size;
  const int Hkv = a.num_kv_heads;
  const int lane = threadIdx.x & 63;
  // The item's block ids (at most 256) go to four lane registers.
  const int32_t* bt = a.block_tables + (int64_t)b0 * a.max_blocks + tok0 / BS;
  const int nmax = item_id_count(P, BS, a.max_blocks, tok0);
  const int ids0 = (lane < nmax) ? bt[lane] : 0;
  const int ids1 = (64 + lane < nmax) ? bt[64 + lane] : 0;
  const int ids2 = (128 + lane < nmax) ? bt[128 + lane] : 0;
  const int ids3 = (192 + lane < nmax) ? bt[192 + lane] : 0;
  const int h0 = kh * G;
  if (tok0 >= tok_end) {  // the sole item of an empty context
    for (int i = lane; i < G * D; i += 64)
      store_elem(DT(), a.out, ((int64_t)b0 * a.num_heads + h0) * D + i, 0.f);
    return;
  }
  const int ntok = tok_end - tok0;
  const int nslots = (ntok + BS - 1) / BS * BS;  // tokens covered by the item's blocks
  const int col = lane & 15, quad = lane >> 4;
  const int ncols = nseq * G;
  const int cseq = col / G;
  const int chead = h0 + col - cseq * G;
  const int64_t crow = ((int64_t)b0 + cseq) * a.num_heads + chead;

  // Query operand, in the key chunks' dim order: k-step (j, h) takes dims
  // 16 * (quad + 4 j) + 8 h .. + 8 in lane group quad.  Loaded before the first tiles.
  uint4 qop[KJ][2];
  {
    const int64_t qrow = (col < ncols) ? crow : (int64_t)b0 * a.num_heads + h0;
    const uint4* qv = reinterpret_cast<const uint4*>(static_cast<const char*>(a.query) + qrow * D * 2);
#pragma unroll
    for (int j = 0; j < KJ; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) qop[j][h] = qv[2 * (quad + 4 * j) + h];
  }
  const int np_col = a.np_of[b0 + min(cseq, nseq - 1)];

  const int64_t tile_bytes = (int64_t)D * BS;  // one (block, head) tile, 1-byte elements
  const int64_t block_bytes = tile_bytes * Hkv;
  const char* kbase = static_cast<const char*>(a.key_cache) + kh * tile_bytes;
  const char* vbase = static_cast<const char*>(a.value_cache) + kh * tile_bytes;
  auto block_of = [&](int j) -> int64_t {
    j = min(j, 255);  // a lookahead past the last block is never used for a load
    const int r = j & 63;
    return (j < 128) ? ((j < 64) ? __builtin_amdgcn_readlane(ids0, r) : __builtin_amdgcn_readlane(ids1, r))
                     : ((j < 192) ? __builtin_amdgcn_readlane(ids2, r) : __builtin_amdgcn_readlane(ids3, r));
  };
  // this lane's tokens within a tile: key rows of the two row groups, the two 4-token runs of
  // its logits, and the 8 tokens of its value operand
  const int ktok0 = col, ktok1 = 16 + col;
  const int stok0 = 4 * quad, stok1 = 16 + 4 * quad;
  const int vtok = 8 * quad;
  struct Tile {
    uint4 k[2][KJ];
    uint2 v[NDT];
  };
  const int ntiles = (ntok + TT - 1) / TT;
  const int last = ntiles - 1;
  // Branch-free loads (see attention_gqa.hip): block ids by select among the tile's blocks,
  // tiles past the last one read the prefetch pad.
  auto load_tile = [&](int t0, Tile& tl) {
    const int j0 = t0 / BS;
    int cand[NBT];
#pragma unroll
    for (int k = 0; k < NBT; ++k) cand[k] = int(block_of(j0 + k));
    // A lane whose token lies past the item's last block (a tile can reach beyond it) reads
    // block 0 instead: table entries there are not block ids; its data is masked (kv8_pick,
    // pkv_tile_addr.h).  The block of tile token t is chosen by a select tree on t / BS (a
    // compare chain over four candidates was turned into an indexed scratch array).
    auto pick = [&](int t) {
      return kv8_pick<BS>(cand[0], cand[NBT > 1 ? 1 : 0], cand[NBT > 2 ? 2 : 0],
                          cand[NBT > 3 ? 3 : 0], t0, t, nslots);
    };
    const bool pad = kv8_pad(t0, last);
    const char* kp0 = (pad ? a.prefetch_pad : kbase + pick(ktok0) * block_bytes) + kv8_key_row<BS>(ktok0);
    const char* kp1 = (pad ? a.prefetch_pad : kbase + pick(ktok1) * block_bytes) + kv8_key_row<BS>(ktok1);
    const char* vp = (pad ? a.prefetch_pad : vbase + pick(vtok) * block_bytes) + kv8_value_run<BS>(vtok);
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const int64_t c = quad + 4 * j;
      tl.k[0][j] = kv_load<true>(reinterpret_cast<const uint4*>(kp0 + kv8_key_chunk<BS>(c)));
      tl.k[1][j] = kv_load<true>(reinterpret_cast<const uint4*>(kp1 + kv8_key_chunk<BS>(c)));
    }
#pragma unroll
    for (int i = 0; i < NDT; ++i)
      tl.v[i] = kv_load<true>(reinterpret_cast<const uint2*>(vp + kv8_value_row<BS>(i * 16 + col)));
  };

  Tile T0, T1, T2, T3;
  load_tile(0, T0);
  load_tile(TT, T1);
  load_tile(2 * TT, T2);

  f32x4 oacc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // reference maximum of column col (base-2 units), lazily moved
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};  // column col's sum of weights (all four rows)
  const uint32_t one2 = one_bits(DT());
  const uint4 ones = make_uint4(one2, one2, one2, one2);

  auto compute_tile = [&](int t0, Tile& tl) {
    f32x4 s[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      s[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
        s[r] = mma(DT(), widen8<DT, CODE>(tl.k[r][j].x, tl.k[r][j].y), qop[j][0], s[r]);
        s[r] = mma(DT(), widen8<DT, CODE>(tl.k[r][j].z, tl.k[r][j].w), qop[j][1], s[r]);
      }
    }
    // lane: logits of tokens t0 + 16 r + 4 quad + e (e < 4) of its column; tokens past the
    // item (only in a tile that reaches past its end) get -inf
#pragma unroll
    for (int r = 0; r < 2; ++r) s[r] *= a.scale_log2;
    if (t0 + TT > ntok) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (t0 + (r ? stok1 : stok0) + e >= ntok) s[r][e] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, s[r][e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // lazy maximum (as in attention_gqa.hip): the first tile holds a token; a tile past the end
    // leaves m, the sums and acc unchanged
    const bool need = tmax > m_run + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? tmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      lacc *= alpha;
#pragma unroll
      for (int i = 0; i < NDT; ++i) oacc[i] *= alpha;
    }
    float p[8];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) p[4 * r + e] = __builtin_amdgcn_exp2f(s[r][e] - m_run);
    // weights of tokens 4 quad .. + 4 (w0) and 16 + 4 quad .. + 4 (w1), two per dword; after
    // the swaps lane (col, quad) holds tokens 8 quad .. + 8: rows (16 lanes) 2-3 of w0 trade
    // with rows 0-1 of w1, then odd rows of the first with even rows of the second
    const uint32_t w0x = pack2(DT(), p[0], p[1]), w0y = pack2(DT(), p[2], p[3]);
    const uint32_t w1x = pack2(DT(), p[4], p[5]), w1y = pack2(DT(), p[6], p[7]);
    const auto sx = __builtin_amdgcn_permlane32_swap(w0x, w1x, false, false);
    const auto sy = __builtin_amdgcn_permlane32_swap(w0y, w1y, false, false);
    const auto tx = __builtin_amdgcn_permlane16_swap(sx[0], sx[1], false, false);
    const auto ty = __builtin_amdgcn_permlane16_swap(sy[0], sy[1], false, false);
    const uint4 pop = make_uint4(tx[0], ty[0], tx[1], ty[1]);
    const int tv = t0 + vtok;
    if (tv + 8 > ntok) {  // value codes past the context (possibly NaN) become 0 before use
      const uint32_t m0 = keep4(tv, ntok), m1 = keep4(tv + 4, ntok);
#pragma unroll
      for (int i = 0; i < NDT; ++i) tl.v[i] = make_uint2(tl.v[i].x & m0, tl.v[i].y & m1);
    }
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = mma(DT(), widen8<DT, CODE>(tl.v[i].x, tl.v[i].y), pop, oacc[i]);
    lacc = mma(DT(), ones, pop, lacc);
  };

  // Computes of tiles past the end are not skipped (see attention_gqa.hip).
  for (int i = 0; i < ntiles; i += 4) {
    load_tile((i + 3) * TT, T3);
    compute_tile(i * TT, T0);
    load_tile((i + 4) * TT, T0);
    compute_tile((i + 1) * TT, T1);
    load_tile((i + 5) * TT, T1);
    compute_tile((i + 2) * TT, T2);
    load_tile((i + 6) * TT, T2);
    compute_tile((i + 3) * TT, T3);
  }

  // ---- epilogue: lane holds O[col][d = 16 i + 4 quad + r] and its column's sum of weights; the
  // value scale is applied here
  const float l_tot = lacc[0];
  if (col < ncols) {
    if (np_col <= 1) {
      const float f = a.v_scale / l_tot;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store_elem(DT(), a.out, crow * D + i * 16 + quad * 4 + r, oacc[i][r] * f);
    } else {
      const int64_t sp = crow * a.slots + slot;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
        *reinterpret_cast<f32x4*>(&a.part_acc[sp * D + i * 16 + quad * 4]) = oacc[i] * a.v_scale;
      if (quad == 0) {
        a.part_m[sp] = m_run;
        a.part_l[sp] = l_tot;
      }
    }
  }
}

template <class DT, int D, int BS, int CODE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void fp8_grid_kernel(DecodeArgs a, int G) {
  const int Hkv = a.num_kv_heads;
  const int t = blockIdx.x;
  if (t >= int(a.queue[1]) * Hkv) return;
  const uint4 it = a.items[t / Hkv];
  if (!item_fits(a, it)) return;
  fp8_item<DT, D, BS, CODE>(a, G, t % Hkv, int(it.x), int(it.y & 255u), int(it.z), int(it.w),
                      int(it.y >> 8));
}

template <class DT, int D, int BS, int CODE>
hipError_t launch_t(const DecodeArgs& a, int group, hipStream_t stream) {
  if (a.plan_mode != 2) {
    const hipError_t e = launch_plan(a, BS, 16 / group, stream);
    if (e != hipSuccess || a.plan_mode == 1) return e;
  }
  const int64_t grid = (int64_t)a.num_seqs * a.num_kv_heads * a.slots;
  hipLaunchKernelGGL((fp8_grid_kernel<DT, D, BS, CODE>), dim3((unsigned)grid), dim3(64), 0, stream, a,
                     group);
  return hipGetLastError();
}

template <class DT, int D, int CODE>
hipError_t by_block(const DecodeArgs& a, int bs, int group, hipStream_t s) {
  switch (bs) {
    case 8: return launch_t<DT, D, 8, CODE>(a, group, s);
    case 16: return launch_t<DT, D, 16, CODE>(a, group, s);
    case 32: return launch_t<DT, D, 32, CODE>(a, group, s);
  }
  return hipErrorInvalidValue;
}

template <class DT, int CODE>
hipError_t by_head(const DecodeArgs& a, int D, int bs, int group, hipStream_t s) {
  switch (D) {
    case 64: return by_block<DT, 64, CODE>(a, bs, group, s);
    case 128: return by_block<DT, 128, CODE>(a, bs, group, s);
  }
  return hipErrorInvalidValue;
}

template <int CODE>
hipError_t by_dtype(const DecodeArgs& a, int dtype, int head_size, int block_size, int group,
                    hipStream_t stream) {
  switch (dtype) {
    case 1: return by_head<F16, CODE>(a, head_size, block_size, group, stream);
    case 2: return by_head<BF16, CODE>(a, head_size, block_size, group, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, int dtype, int head_size, int block_size,
                             int group, hipStream_t stream) {
  return by_dtype<kCodeE4M3>(a, dtype, head_size, block_size, group, stream);
}

hipError_t launch_decode_i8(const DecodeArgs& a, int dtype, int head_size, int block_size,
                            int group, hipStream_t stream) {
  return by_dtype<kCodeI8>(a, dtype, head_size, block_size, group, stream);
}

}  // namespace pkv
