// Multi-query paged attention: chunked prefill and mixed prefill / decode batches.
//
// The query rows of all requests are flattened; request b owns rows
// [query_start_loc[b], query_start_loc[b + 1]) (the attention metadata of the tiemojia.cn
// vLLM run-flow article, section 3.5).  Its n rows are the last n positions of its context of
// L tokens (the chunk that chunked prefill adds to a partly prefilled prompt, the AIGC
// interview book's scheduler note; a decode token is n = 1), and the row at position p attends
// causally to cache positions 0..p.
//
// Work decomposition.  A workgroup takes one work item = (request, query tile, key range) and
// one KV head.  Its 256 matrix columns are (query token, query head) pairs: q_tile = 256 / G
// consecutive query tokens times the G query heads that share the KV head.  The key range of a
// tile is cut at multiples of the partition size P, so every piece starts at or before the
// tile's first query position and each column sees at least one key of every piece.  Pieces
// of one tile are merged by the split-K reduce of the decode path (each query row plays the
// part of a sequence there).
//
// Per 32-key stage the workgroup copies the keys and values of its KV head from the paged
// cache (the block layout of the "Vllm" page, "CacheEngine") into LDS (six stage buffers, a
// stage stored four steps before its values are read, one barrier per two stages), and every
// wave reads them from there: the stage is fetched once for all 256 columns.  A wave computes
// the logits of the next stage while its VALU turns the current stage's logits into weights,
// and copies a later stage while its matrix core multiplies the weights by the values; the two
// waves of a SIMD run half a step apart.
//   keys:   LDS [D/8][32][8], the A operand of S^T = K Q^T (v_mfma_f32_16x16x32, tokens on
//           rows, 16 columns per product), the 32 tokens stored in the row order
//           (8q..8q+3 for q = 0..3, then 8q+4..8q+7), so that lane quad q of the two 16x16
//           logit tiles holds the logits of keys 8q..8q+7;
//   values: LDS rows of 32 tokens in their natural order (96-byte stride): a lane's 16-byte
//           read is the A operand of O^T += V^T P^T with 32 keys per product, and the lane's
//           own 8 softmax weights are its B operand without any data movement.
// Online softmax per column in base 2 with a lazy maximum: the running maximum is only moved
// (and the accumulators rescaled) when a stage's maximum exceeds it by more than 8 (weights
// stay below 2^8), so most stages skip the rescale.  The logit scale is applied to the query
// before it is rounded to the element type (one more rounding of each query element), and the
// logit products start from -m_run: the matrix cores yield the exponent of each weight, and
// the VALU only exponentiates.  Weights are rounded once to the element type, and the row sums
// come out of the matrix cores (a product with a ones row) from the same rounded weights.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_prefill.h"
#include "pkv_kv8.h"

#include <type_traits>

namespace pkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));


__device__ __forceinline__ f32x4 mma(BF16, const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(F16, const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
// pack2 / one_bits (pkv_device.h): two floats to two packed elements (RNE), and packed ones.

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one MFMA column): gfx950's lane-swap
// instructions (VALU), not an LDS permute.
__device__ __forceinline__ float column_max(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Zero the 16-bit elements of an 8-token value piece whose token base + e is >= limit.
__device__ __forceinline__ uint4 mask8(uint4 v, int base, int limit) {
  auto m = [&](int e) -> uint32_t {
    return ((base + e < limit) ? 0x0000ffffu : 0u) | ((base + e + 1 < limit) ? 0xffff0000u : 0u);
  };
  return make_uint4(v.x & m(0), v.y & m(2), v.z & m(4), v.w & m(6));
}
// The same for an 8-token piece of 8-bit codes (a zero code is the value 0 in both formats).
__device__ __forceinline__ uint2 mask8(uint2 v, int base, int limit) {
  auto m = [&](int e) -> uint32_t {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) r |= (base + e + k < limit) ? (0xffu << (8 * k)) : 0u;
    return r;
  };
  return make_uint2(v.x & m(0), v.y & m(4));
}

// ---------------------------------------------------------------------------------------
// Plan: one workgroup lists the work items.  A request's items are listed together (its
// tiles, longest first), so that the workgroups of one request and one KV head run side by
// side on one XCD (workgroup t runs on XCD t mod 8 and takes KV head t mod num_kv_heads) and
// read the request's keys and values through that XCD's L2 once, not once per tile.
// Requests go longest first (32 classes by their longest item, the longest class first; the
// order inside a class is arbitrary, which changes no result: every item writes its own
// outputs or partial slot).  Requests whose metadata is inconsistent (negative or decreasing
// offsets, rows past num_tokens, a chunk longer than its context, a context longer than
// max_context_len) get no items: their rows are left unwritten.
// ---------------------------------------------------------------------------------------
constexpr int kPlanClasses = 32;

__device__ __forceinline__ bool request_ok(const PrefillArgs& a, int b, int& qs, int& n, int& L) {
  qs = a.query_start_loc[b];
  const int qe = a.query_start_loc[b + 1];
  n = qe - qs;
  L = a.context_lens[b];
  return qs >= 0 && n >= 0 && qe <= a.num_tokens && n <= L && L <= a.max_context_len;
}

// Calls f(tile j, first key, end key, piece count) for every item of request b.
template <class F>
__device__ __forceinline__ void for_each_item(const PrefillArgs& a, int b, F&& f) {
  int qs, n, L;
  if (!request_ok(a, b, qs, n, L) || n == 0) return;
  const int QT = a.q_tile, P = a.partition_size;
  // tiles from the last to the first; the piece count floor(qpos0 / P) + 1 is carried from
  // tile to tile (qpos0 falls by QT) instead of dividing for each tile
  int j = (n + QT - 1) / QT - 1;
  int qpos0 = L - n + j * QT;
  int q = qpos0 / P, r = qpos0 - q * P;
  for (; j >= 0; --j) {
    const int end = qpos0 + min(QT, n - j * QT);
    const int np = q + 1;
    for (int p = 0; p < np; ++p) f(j, p * P, p + 1 == np ? end : (p + 1) * P);
    qpos0 -= QT;
    r -= QT;
    while (r < 0) {
      r += P;
      --q;
    }
  }
}

__global__ __launch_bounds__(1024) void prefill_plan_kernel(PrefillArgs a) {
  __shared__ int s_count[kPlanClasses];
  const int tid = threadIdx.x;
  // rows of the split-K reduce: 0 (nothing to merge) unless an item of the row's tile says
  // otherwise; rows of skipped requests stay 0
  if (a.slots > 1)
    for (int r = tid; r < a.num_tokens; r += 1024) a.np_of[r] = 0;
  if (tid < kPlanClasses) s_count[tid] = 0;
  __syncthreads();
  // an item spans at most min(P, max_context_len) + q_tile keys
  const int span = min(a.partition_size, a.max_context_len) + a.q_tile + 1;
  auto cls = [&](int len) {
    // 32-bit: len < span <= the largest partition + a tile (the class only orders the items)
    return kPlanClasses - 1 - min(kPlanClasses - 1, int(uint32_t(len) * kPlanClasses / uint32_t(span)));
  };
  // a request's item count and its longest item
  auto count = [&](int b, int& longest) {
    int n_items = 0;
    longest = 0;
    for_each_item(a, b, [&](int, int k0, int k1) {
      ++n_items;
      longest = max(longest, k1 - k0);
    });
    return n_items;
  };
  for (int b = tid; b < a.num_seqs; b += 1024) {
    int longest;
    const int n_items = count(b, longest);
    if (n_items > 0) atomicAdd(&s_count[cls(longest)], n_items);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int c = 0; c < kPlanClasses; ++c) {
      const int v = s_count[c];
      s_count[c] = run;
      run += v;
    }
    a.queue[1] = uint32_t(min<int64_t>(run, a.capacity));
  }
  __syncthreads();
  for (int b = tid; b < a.num_seqs; b += 1024) {
    int longest;
    const int n_items = count(b, longest);
    if (n_items == 0) continue;
    int idx = atomicAdd(&s_count[cls(longest)], n_items);
    for_each_item(a, b, [&](int j, int k0, int k1) {
      if (idx < a.capacity)
        a.items[idx] = make_uint4(uint32_t(b), uint32_t(j), uint32_t(k0), uint32_t(k1));
      ++idx;
    });
  }
}

// ---------------------------------------------------------------------------------------
// Attention: NW waves x CB blocks of 16 columns = 256 columns per workgroup.
// ---------------------------------------------------------------------------------------
template <class DT, int D, int BS, int NW, int CB, int KVC>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(PrefillArgs a) {
  constexpr bool KV8 = KVC != 0;  // KVC: 0 a 16-bit cache, else the 8-bit code format
  static_assert(NW * CB * 16 == kPrefillColumns, "columns per workgroup");
  static_assert(BS == 8 || BS == 16 || BS == 32, "a 32-key stage holds whole blocks");
  constexpr int NT = NW * 64;
  constexpr int KC = D / 32;        // 32-dim steps of the logit product
  constexpr int NDT = D / 16;       // 16-dim output tiles
  constexpr int KSTAGE = D * 64;    // bytes: [D/8][32 keys][16 B]
  constexpr int VRS = 96;           // value row stride: 64 B of data + 32 B of padding (fewest
                                    // bank conflicts of the layouts measured: strides 64, 80,
                                    // 96, and 64 with the 16-byte chunks XOR-swizzled by row)
  constexpr int VSTAGE = D * VRS;
  constexpr int KPIECES = D * 4;    // 16-byte pieces per stage (keys and values alike)
  constexpr int PPT = (KPIECES + NT - 1) / NT;
  // Step s reads the values of stage s and the keys of stage s + 1 and stores stage s + AHEAD;
  // a barrier follows every odd step.  Six buffers make one barrier per two steps enough (the
  // step loop below gives the reasoning).
  constexpr int NBUF = 6;
  constexpr int AHEAD = 4;
  // register sets of stage copies in flight: a stage is loaded R steps before it is stored.
  // Three (on a 16-request chunked-prefill step the loads then run about 3 us ahead of their
  // use; deeper measured no faster).
  constexpr int R = 3;
  // the loop is unrolled by U steps, so that every buffer, register set and logit set index in
  // it is a constant
  constexpr int U = 6;
  static_assert(U % NBUF == 0 && U % R == 0 && U % 2 == 0, "constant indices in the loop");
  static_assert(AHEAD >= R, "the prologue stores stages 0 .. AHEAD - 1 through the R sets");
  __shared__ __align__(16) char s_k[NBUF][KSTAGE];
  __shared__ __align__(16) char s_v[NBUF][VSTAGE];
  __shared__ int s_ids[kPrefillMaxIds];

  const int Hkv = a.num_kv_heads, Hq = a.num_heads;
  const int t = blockIdx.x;
  if (t >= int(a.queue[1]) * Hkv) return;
  const uint4 it = a.items[t / Hkv];
  const int kh = t % Hkv;
  const int b = int(it.x), j = int(it.y), k0 = int(it.z), k1 = int(it.w);
  const int G = a.group, QT = a.q_tile, P = a.partition_size;
  const int qs = a.query_start_loc[b];
  const int n = a.query_start_loc[b + 1] - qs;
  const int L = a.context_lens[b];
  const int qpos0 = L - n + j * QT;  // position of the tile's first query
  const int nqt = min(QT, n - j * QT);
  const int row0 = qs + j * QT;
  const int npieces = qpos0 / P + 1;
  const int slot = k0 / P;
  const int nst = (k1 - k0 + 31) / 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int w_uniform = __builtin_amdgcn_readfirstlane(w);
  const int col = lane & 15, quad = lane >> 4;

  if (a.slots > 1 && slot == 0 && kh == 0)  // read by the reduce, which runs after this kernel
    for (int i = tid; i < nqt; i += NT) a.np_of[row0 + i] = npieces;

  // block ids of the item's keys (ids past the context's last block: 0, a valid block whose
  // data only ever meets zero weights or zeroed values)
  const int blk0 = k0 / BS;
  const int n_ids = (k0 + nst * 32 + BS - 1) / BS - blk0;
  const int nblk = (L + BS - 1) / BS;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;
  for (int i = tid; i < n_ids; i += NT) s_ids[i] = (blk0 + i < nblk) ? bt[blk0 + i] : 0;

  // columns of this wave: c = (w CB + cb) 16 + col -> query token qi = c / G, head c % G
  int qi_c[CB], end_c[CB];
  uint4 qop[CB][KC];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c = (w * CB + cb) * 16 + col;
    const int qi = c / G;
    const int qic = min(qi, nqt - 1);  // unused columns compute a valid row; never stored
    qi_c[cb] = qi;
    end_c[cb] = min(k1, qpos0 + qic + 1);
    const int64_t qrow = (int64_t)(row0 + qic) * Hq + kh * G + (c - qi * G);
    const uint4* qv = reinterpret_cast<const uint4*>(static_cast<const char*>(a.query) + qrow * D * 2);
    // the logit scale (base 2, with the key scale of an 8-bit cache) is applied to the query
    // once, in fp32, before it is rounded back to the element type: the logit products then
    // give base-2 logits directly and no per-logit multiply is left
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      float f[8];
      unpack(DT(), qv[kc * 4 + quad], f);
      const float sl2 = a.scale_log2;
      qop[cb][kc] = make_uint4(pack2(DT(), f[0] * sl2, f[1] * sl2), pack2(DT(), f[2] * sl2, f[3] * sl2),
                               pack2(DT(), f[4] * sl2, f[5] * sl2), pack2(DT(), f[6] * sl2, f[7] * sl2));
    }
  }
  const int qi_first = (w_uniform * CB * 16) / G;  // wave-uniform, in a scalar register
  const bool active = qi_first < nqt;                       // the wave has a real column
  const int wave_full = min(k1, qpos0 + qi_first + 1);      // keys before it: seen by all

  const int64_t tile_bytes = (int64_t)D * BS * (KV8 ? 1 : 2);  // one (block, KV head) tile
  const uint32_t block_bytes = uint32_t(tile_bytes * Hkv);      // below 4 GiB (host check)
  const char* kbase = static_cast<const char*>(a.key_cache) + kh * tile_bytes;
  const char* vbase = static_cast<const char*>(a.value_cache) + kh * tile_bytes;

  // Stage s's keys and values go from HBM to registers R steps before step s - AHEAD stores them
  // to LDS (its keys are read in step s - 1, its values in step s).  Loads are never skipped (a
  // stage past the end reloads the last one, from L2): a load under a branch would make every
  // wait conservative.
  // Per-thread constants of the copies (a stage starts at a multiple of 32 >= k0, which is
  // itself a multiple of 32, so a thread's pieces sit at fixed offsets inside their blocks):
  //   key piece: dims 8 c8 .. +8 of stage token tok
  //   value piece: dim d, stage tokens t8 .. t8 + 8 (inside one block)
  // Which piece a thread copies: key piece p fills LDS row krow = p mod 32 of dim chunk
  // c8 = p / 32 (token tok of that row, in the row order above); among the value pieces, 16
  // neighbouring ones are one 8-token chunk of 16 dims, so that 16 lanes store to 16 rows in
  // the pattern the P.V operand reads use.
  auto key_piece = [](int p, int& c8, int& krow, int& tok) {
    c8 = p >> 5;
    krow = p & 31;
    tok = 8 * ((krow >> 2) & 3) + 4 * (krow >> 4) + (krow & 3);
  };
  auto value_piece = [](int p, int& d, int& t8) {
    d = ((p >> 6) << 4) + (p & 15);
    t8 = ((p >> 4) & 3) * 8;
  };
  constexpr int IDS_PER_STAGE = 32 / BS;
  int kid[PPT], vid[PPT];
  uint32_t koff[PPT], voff[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = min(tid + i * NT, KPIECES - 1);
    int c8, krow, tt, d, t8;
    key_piece(p, c8, krow, tt);
    value_piece(p, d, t8);
    kid[i] = tt / BS;
    vid[i] = t8 / BS;
    if constexpr (KV8) {  // 8-bit cache: keys [D/16][bs][16], values [D][bs], one byte each
      koff[i] = uint32_t(((c8 >> 1) * BS + tt % BS) * 16 + (c8 & 1) * 8);
      voff[i] = uint32_t(d * BS + t8 % BS);
    } else {
      koff[i] = uint32_t(c8 * BS + tt % BS) * 16u;
      voff[i] = uint32_t(d * BS + t8 % BS) * 2u;
    }
  }
  // Raw pieces as loaded (8 codes of an 8-bit cache take 8 bytes); they are widened to the
  // 16-bit type only when stored to LDS, so no load has to be waited for early.
  using Raw = typename std::conditional<KV8, uint2, uint4>::type;
  Raw kR[R][PPT], vR[R][PPT];  // register sets: stage u sits in set u mod R
  auto widen = [&](const Raw& r) -> uint4 {
    if constexpr (KV8) return widen8<DT, KVC>(r.x, r.y);
    else return r;
  };
  auto load_stage = [&](int s, Raw* kst, Raw* vst) {
    const int sid = min(s, nst - 1) * IDS_PER_STAGE;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      if (KPIECES % NT == 0 || tid + i * NT < KPIECES) {
        const uint32_t ik = uint32_t(s_ids[sid + kid[i]]), iv = uint32_t(s_ids[sid + vid[i]]);
        kst[i] = *reinterpret_cast<const Raw*>(kbase + (uint64_t)ik * block_bytes + koff[i]);
        vst[i] = *reinterpret_cast<const Raw*>(vbase + (uint64_t)iv * block_bytes + voff[i]);
      }
    }
  };
  // Values of tokens past the item's range are zeroed here (selects, no branch): the cache
  // past a context's end may hold anything, and a zero weight times NaN is NaN.
  auto store_stage = [&](int buf, int s, const Raw* kst, const Raw* vst) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * NT;
      if (KPIECES % NT == 0 || p < KPIECES) {
        int c8, krow, tok, d, t8;
        key_piece(p, c8, krow, tok);
        value_piece(p, d, t8);
        *reinterpret_cast<uint4*>(&s_k[buf][(c8 * 32 + krow) * 16]) = widen(kst[i]);
        uint4 v = widen(vst[i]);
        if (k0 + 32 * (s + 1) > k1) v = mask8(v, k0 + 32 * s + t8, k1);  // the last stage only
        *reinterpret_cast<uint4*>(&s_v[buf][d * VRS + t8 * 2]) = v;
      }
    }
  };

  f32x4 oacc[NDT][CB], lacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    lacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Per column: the running maximum m_run (base-2 units), kept as its negation in all four
  // elements of negm (the accumulator that the logit products start from, so that they yield
  // z - m_run, the exponent of the weight, with no VALU); m_run is 0 until the first maximum
  // is taken.  The lazy test's threshold on z - m_run is one value for the wave: -inf before
  // its first stage, the margin after.  Every column sees the item's first key (a piece starts
  // at or before its tile's first query), so every column takes its first maximum in the first
  // stage.
  float m_thr = -INFINITY;
  f32x4 negm[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) negm[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // A operand of the row-sum product: row 0 all ones (lanes with col == 0), other rows zero
  const uint32_t ob = (col == 0) ? one_bits(DT()) : 0u;
  const uint4 ones = make_uint4(ob, ob, ob, ob);

  // ---- the pieces of a stage's work (LDS buffer buf holds the stage)
  // S^T = K Q^T: 2 key tiles x CB column blocks, KC products each
  auto qk_read = [&](int buf, uint4 (&ka)[KC][2]) {
    const char* sk = s_k[buf];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        ka[kc][tt] = *reinterpret_cast<const uint4*>(sk + ((kc * 4 + quad) * 32 + tt * 16 + col) * 16);
  };
  // (the first product of each chain starts from -m_run instead of zero)
  auto qk_mma = [&](const uint4 (&ka)[KC][2], f32x4 (&S)[2][CB]) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          S[tt][cb] = mma(DT(), ka[kc][tt], qop[cb][kc], kc == 0 ? negm[cb] : S[tt][cb]);
  };
  auto qk = [&](int buf, f32x4 (&S)[2][CB]) {
    uint4 ka[KC][2];
    qk_read(buf, ka);
    qk_mma(ka, S);
  };
  // per column and lane: the largest of the lane's 8 values z - m_run of the stage
  auto stage_max = [&](const f32x4 (&S)[2][CB], float (&mc)[CB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      // a chain of three-input maxima (v_max3_f32): 4 instructions for 8 logits
      float m = fmaxf(fmaxf(S[0][cb][0], S[0][cb][1]), S[0][cb][2]);
      m = fmaxf(fmaxf(m, S[0][cb][3]), S[1][cb][0]);
      m = fmaxf(fmaxf(m, S[1][cb][1]), S[1][cb][2]);
      mc[cb] = fmaxf(m, S[1][cb][3]);
    }
  };
  // keys a column must not see (causal, or past the item): logit -inf.  Element r of logit
  // tile tt of lane quad q is the key 8 q + 4 tt + r of the stage.
  auto mask_stage = [&](int t0, f32x4 (&S)[2][CB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int lim = end_c[cb] - (t0 + quad * 8);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tt * 4 + r >= lim) S[tt][cb][r] = -INFINITY;
    }
  };
  // lazy maximum: move it (and rescale) only when a column's stage maximum exceeds it by more
  // than the margin (or at the first stage); the wave takes the branch if any of its
  // columns needs it.  The test runs on each lane's own maximum: some lane of a column passes it
  // exactly when the column's maximum does, and the column maximum (a cross-lane exchange) is
  // only formed inside the rare branch.  Moving m_run by d also moves the stage's values
  // z - m_run, computed against the old m_run, by -d; later stages start from the new -m_run.
  // At the first maximum the accumulators are still zero, and alpha is 0 (not exp2 of an
  // arbitrary distance, which may overflow).
  auto rescale = [&](const float (&lm)[CB], f32x4 (&Sc)[2][CB]) {
    bool any = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) any |= lm[cb] > m_thr;
    if (__builtin_amdgcn_ballot_w64(any) != 0) {
      const bool first = m_thr == -INFINITY;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float mc = column_max(lm[cb]);
        const float delta = mc > m_thr ? -mc : 0.f;
        const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(delta);
        const float nm = negm[cb][0] + delta;  // -m_run moved by delta
        negm[cb] = f32x4{nm, nm, nm, nm};
        Sc[0][cb] += delta;
        Sc[1][cb] += delta;
        lacc[cb] *= alpha;
#pragma unroll
        for (int i = 0; i < NDT; ++i) oacc[i][cb] *= alpha;
      }
      m_thr = kLazyRescale;
    }
  };
  // weights rounded to the element type (the B operand of P.V) and their sums
  auto weights = [&](const f32x4 (&S)[2][CB], uint4 (&pop)[CB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float p[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r)  // v_exp_f32: weights below 2^-126 flush to 0
          p[tt][r] = __builtin_amdgcn_exp2f(S[tt][cb][r]);
      pop[cb] = make_uint4(pack2(DT(), p[0][0], p[0][1]), pack2(DT(), p[0][2], p[0][3]),
                           pack2(DT(), p[1][0], p[1][1]), pack2(DT(), p[1][2], p[1][3]));
      lacc[cb] = mma(DT(), ones, pop[cb], lacc[cb]);
    }
  };
  // a stage with a key some column of the wave must not see
  auto needs_mask = [&](int s) { return k0 + 32 * s + 32 > wave_full; };

  // Software pipeline, one stage per step.  Step s starts from the logits of stage s (their
  // products were issued in step s - 1): it masks them where needed and tests the lazy maximum,
  // then issues the logit products of stage s + 1 -- independent work for the matrix cores
  // while the VALU turns stage s's logits into weights -- and last the P.V products of stage s.
  // Stages past a wave's last column are computed too: their keys are all masked (zero
  // weights).  The logits of stage nst, past the end, come from a block holding a copy of the
  // last stage and are never used.
  // logits: set x holds those of the stages of parity x (the unrolled loop picks constants)
  f32x4 S[2][2][CB];
  // step s with s mod U = u (a multiple of U is a multiple of NBUF, R and 2), in two parts.
  // Part a: the LDS reads of stage s + 1's keys and stage s's values (vop), the mask and lazy
  // maximum of stage s, the logit products of stage s + 1 and the weights of stage s (pop),
  // issued so that each logit product is followed by two VALU instructions of the weights and
  // every second one by a value read.
  auto step_a = [&](int s, int u, uint4 (&vop)[NDT], uint4 (&pop)[CB]) {
    f32x4 (&Sc)[2][CB] = S[u & 1];
    uint4 ka[KC][2];
    qk_read((u + 1) % NBUF, ka);  // in flight while the VALU tests the stage's maximum
    if (needs_mask(s)) mask_stage(k0 + 32 * s, Sc);
    float lm[CB];
    stage_max(Sc, lm);
    rescale(lm, Sc);  // before the stage's weights and its P.V
    const char* sv = s_v[u % NBUF];
#pragma unroll
    for (int i = 0; i < NDT; ++i)
      vop[i] = *reinterpret_cast<const uint4*>(sv + (i * 16 + col) * VRS + quad * 16);
    qk_mma(ka, S[(u + 1) & 1]);
    weights(Sc, pop);
#pragma unroll
    for (int g = 0; g < 2 * KC * CB; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
      if (g % 2 == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
  };
  // Part b: the P.V products of stage s (an active wave's; from registers only) and the copy
  // of stage s + AHEAD: its pieces stored to LDS from their register set, the next load into
  // that set.  Issued at raised wave priority, so that the SIMD's arbiter keeps feeding the
  // matrix core from this wave while the other wave on the SIMD forms weights, and interleaved
  // by hand (the copy between groups of products) so that the copy's LDS and memory traffic
  // runs in the products' shadow.  Every wave copies; only active waves multiply.
  auto step_b = [&](int s, int u, const uint4 (&vop)[NDT], const uint4 (&pop)[CB]) {
    static_assert(PPT == 1 && NDT % 4 == 0, "one piece per thread");
    const int set = (u + AHEAD) % R, buf = (u + AHEAD) % NBUF;
    auto pv = [&](int i0) {
      if (active) {
#pragma unroll
        for (int i = i0; i < i0 + NDT / 4; ++i)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) oacc[i][cb] = mma(DT(), vop[i], pop[cb], oacc[i][cb]);
      }
    };
    const bool has = KPIECES % NT == 0 || tid < KPIECES;
    int c8, krow, tok, d, t8;
    key_piece(tid, c8, krow, tok);
    value_piece(tid, d, t8);
    __builtin_amdgcn_s_setprio(1);
    if (has) *reinterpret_cast<uint4*>(&s_k[buf][(c8 * 32 + krow) * 16]) = widen(kR[set][0]);
    pv(0);
    if (has) *reinterpret_cast<uint4*>(&s_v[buf][d * VRS + t8 * 2]) = widen(vR[set][0]);
    pv(NDT / 4);
    const int sid = min(s + AHEAD + R, nst - 1) * IDS_PER_STAGE;
    uint32_t ik = 0, iv = 0;
    if (has) {
      ik = uint32_t(s_ids[sid + kid[0]]);
      iv = uint32_t(s_ids[sid + vid[0]]);
    }
    pv(NDT / 2);
    if (has) {
      kR[set][0] = *reinterpret_cast<const Raw*>(kbase + (uint64_t)ik * block_bytes + koff[0]);
      vR[set][0] = *reinterpret_cast<const Raw*>(vbase + (uint64_t)iv * block_bytes + voff[0]);
    }
    pv(3 * NDT / 4);
    __builtin_amdgcn_s_setprio(0);
  };
  // Values of the stage past the item's end zeroed in its register set before part b stores
  // them (the last stage only: a wave-uniform branch).
  auto mask_set = [&](int s, Raw* vst) {
    int d, t8;
    value_piece(tid, d, t8);
    vst[0] = mask8(vst[0], k0 + 32 * s + t8, k1);
  };
  // Waves w and w + NW/2 share a SIMD.  The later half of the waves meets the barrier of an odd
  // step between its parts a and b, the earlier half after part b, so the two waves of a SIMD
  // run half a step apart: one issues its P.V products while the other forms weights.
  // Buffers: stage X is stored in part b of step X - AHEAD; its keys are read in part a of step
  // X - 1, its values in part a of step X; the buffer step s stores into last held stage
  // s + AHEAD - NBUF = s - 2, whose values were read in part a of step s - 2.  Of steps X - 3
  // and X - 2 one is odd, and its barrier lies after the store and before the keys' read for
  // both halves of the waves; of steps s - 2 and s - 1 one is odd, and its barrier lies after
  // that last read and before the store.
  const bool late = w_uniform >= NW / 2;
  auto copy_and_step = [&](int s, int u) {
    if (k0 + 32 * (s + AHEAD + 1) > k1) mask_set(s + AHEAD, vR[(u + AHEAD) % R]);
    uint4 vop[NDT], pop[CB];
    if (active) step_a(s, u, vop, pop);
    if ((u & 1) && late) __syncthreads();
    step_b(s, u, vop, pop);
    if ((u & 1) && !late) __syncthreads();
  };

  // Prologue: stages 0 .. AHEAD - 1 stored, stages AHEAD .. AHEAD + R - 1 in their register sets
  // (stage X in set X mod R).  Stores and loads are not skipped past the end (loads of stages
  // past the last reload it; the buffers they fill are free, and unread after the loop but for
  // stage nst's discarded logits).
  __syncthreads();  // s_ids
#pragma unroll
  for (int u = 0; u < R; ++u) load_stage(u, kR[u], vR[u]);
#pragma unroll
  for (int u = 0; u < AHEAD; ++u) {
    store_stage(u, u, kR[u % R], vR[u % R]);
    load_stage(u + R, kR[u % R], vR[u % R]);
  }
  __syncthreads();
  if (active) qk(0, S[0]);

  // Steps in groups of U: the only way back to the loop head is the end of a group, so the
  // wait counters there know exactly which loads are in flight, and s is a multiple of U at
  // every step of the group (its buffer, set and parity are those of u).  The last group leaves
  // at its first step past the end.  (One loop: a second unrolled copy for the last group kept
  // more values live across the two and spilled three registers per lane.)
  for (int s = 0; s < nst; s += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u >= nst) goto stages_done;
      copy_and_step(s + u, u);
    }
  }
stages_done:
  if (!active) return;

  // ---- epilogue: lane holds O^T[d = 16 i + 4 quad + r][column]; the row sum of a column
  // sits in row 0 of its sum product (lane col, element 0)
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float l_tot = __shfl(lacc[cb][0], col, 64);
    const int c = (w * CB + cb) * 16 + col;
    if (qi_c[cb] >= nqt) continue;
    const int64_t orow = (int64_t)(row0 + qi_c[cb]) * Hq + kh * G + (c - qi_c[cb] * G);
    if (npieces == 1) {
      const float inv = (KV8 ? a.v_scale : 1.f) / l_tot;
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        const f32x4 o = oacc[i][cb] * inv;
        *reinterpret_cast<uint2*>(static_cast<char*>(a.out) + (orow * D + i * 16 + quad * 4) * 2) =
            make_uint2(pack2(DT(), o[0], o[1]), pack2(DT(), o[2], o[3]));
      }
    } else {
      const int64_t sp = orow * a.slots + slot;
#pragma unroll
      for (int i = 0; i < NDT; ++i)  // the value scale of an 8-bit cache goes into the partials
        *reinterpret_cast<f32x4*>(&a.part_acc[sp * D + i * 16 + quad * 4]) =
            KV8 ? oacc[i][cb] * a.v_scale : oacc[i][cb];
      if (quad == 0) {
        a.part_m[sp] = -negm[cb][0];
        a.part_l[sp] = l_tot;
      }
    }
  }
}

template <class DT, int D, int BS, int KVC>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  constexpr int NW = 8, CB = 2;
  const int64_t grid = a.capacity * a.num_kv_heads;
  hipLaunchKernelGGL((prefill_kernel<DT, D, BS, NW, CB, KVC>), dim3((unsigned)grid), dim3(NW * 64),
                     0, stream, a);
  return hipGetLastError();
}

template <class DT, int D, int KVC>
hipError_t by_block(const PrefillArgs& a, int bs, hipStream_t s) {
  switch (bs) {
    case 8: return launch_t<DT, D, 8, KVC>(a, s);
    case 16: return launch_t<DT, D, 16, KVC>(a, s);
    case 32: return launch_t<DT, D, 32, KVC>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class DT, int KVC>
hipError_t by_head(const PrefillArgs& a, int D, int bs, hipStream_t s) {
  switch (D) {
    case 64: return by_block<DT, 64, KVC>(a, bs, s);
    case 128: return by_block<DT, 128, KVC>(a, bs, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(int dtype, int head_size, int block_size, int group) {
  return (dtype == 1 || dtype == 2) && (head_size == 64 || head_size == 128) &&
         (block_size == 8 || block_size == 16 || block_size == 32) && group >= 1 && group <= 16;
}

hipError_t launch_prefill(const PrefillArgs& a, const DecodeArgs& red, int dtype, int head_size,
                          int block_size, int kv_code, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (kv_code) {
    case 0:
      e = (dtype == 1) ? by_head<F16, 0>(a, head_size, block_size, stream)
                       : by_head<BF16, 0>(a, head_size, block_size, stream);
      break;
    case kCodeE4M3:
      e = (dtype == 1) ? by_head<F16, kCodeE4M3>(a, head_size, block_size, stream)
                       : by_head<BF16, kCodeE4M3>(a, head_size, block_size, stream);
      break;
    case kCodeI8:
      e = (dtype == 1) ? by_head<F16, kCodeI8>(a, head_size, block_size, stream)
                       : by_head<BF16, kCodeI8>(a, head_size, block_size, stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (e != hipSuccess || a.slots <= 1) return e;
  return launch_reduce(red, dtype, head_size, stream);
}

}  // namespace pkv
