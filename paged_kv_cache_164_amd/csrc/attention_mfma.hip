// Paged decode attention, phase 1, matrix-core variant for grouped-query heads (fp16 / bf16).
//
// When G = num_heads / num_kv_heads query heads share one KV head, the
// logits of a 16-token tile are a small dense product S^T[t][g] =
// K[t][:] . Q[g][:] and the output is O^T[d][g] = sum_t V^T[d][t] P^T[t][g]:
// both run on v_mfma_f32_16x16x32_{bf16,f16} with the G query heads in the
// 16-wide N dimension (columns g >= G are zero and ignored).
//
// The cache layout of the "Vllm" page (section "CacheEngine") makes both
// operands single 16-byte loads per lane:
//  * key tile [head_size/8][block_size][8]: the A operand of 16 tokens x 32
//    dims, lane l = (token l%16, dims 8*(l/16)..+8), is chunk
//    (c = 4*kc + l/16, token) -- 256 contiguous bytes per 16 lanes;
//  * value tile [head_size][block_size]: the A operand of 16 dims x 32
//    tokens, lane l = (dim l%16, tokens 8*(l/16)..+8), is one 16-byte run of
//    a value row.
// Work split inside the workgroup (4 waves): logits by 16-token tiles
// (interleaved over waves), P.V by head-dim tiles (each wave owns
// head_size/4 dims for the whole partition, so no cross-wave reduction).
//
// Softmax weights are rounded to the element type before the P.V product
// and the running sum l adds those same rounded weights, so numerator and
// denominator use identical weights.  Tokens past the context get logit
// -inf, weight 0, and their value entries are replaced by 0 before the
// product (0 * NaN never happens).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16x16x32(BF16, const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(F16, const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Round a weight to the element type and back (the value the matrix core will see).
__device__ __forceinline__ float round_to(BF16, float v) {
  return __uint_as_float(uint32_t(f32_to_bf16_rne(v)) << 16);
}
__device__ __forceinline__ float round_to(F16, float v) {
  return static_cast<float>(static_cast<_Float16>(v));
}
// Pack two weights (already representable) into one 32-bit pair.
__device__ __forceinline__ uint32_t pack2(BF16, float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}
__device__ __forceinline__ uint32_t pack2(F16, float lo, float hi) {
  half2_t h;
  h[0] = static_cast<_Float16>(lo);
  h[1] = static_cast<_Float16>(hi);
  return __builtin_bit_cast(uint32_t, h);
}

// Zero the 16-bit elements e of a 16-byte chunk whose token index base + e is >= limit.
__device__ __forceinline__ uint4 mask_tokens(uint4 v, int base, int limit) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = (base + 2 * k < limit) ? 0x0000ffffu : 0u;
    const uint32_t hi = (base + 2 * k + 1 < limit) ? 0xffff0000u : 0u;
    w[k] &= (lo | hi);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <class DT, int D, int BS>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeArgs a, int G, int Pr) {
  static_assert(DT::X == 8, "matrix-core path is for 16-bit element types");
  constexpr int KC = D / 32;        // 32-dim k-steps of the logit product
  constexpr int DT_TILES = D / 16;  // 16-dim tiles of the output
  constexpr int DT_PER_WAVE = DT_TILES / kWaves;
  static_assert(DT_PER_WAVE >= 1, "head_size must give each wave a 16-dim tile");
  constexpr int UK = 2;             // key tiles in flight per wave
  constexpr int UV = 4;             // 32-token value steps in flight per wave
  const int P = a.partition_size;
  const int Hkv = a.num_kv_heads;
  int id = blockIdx.x;
  const int kh = id % Hkv;
  id /= Hkv;
  const int b = id % a.num_seqs;
  const int p = id / a.num_seqs;
  const int L = min(max(a.context_lens[b], 0), a.len_limit);
  const int tok0 = p * P;
  const int h0 = kh * G;
  if (tok0 >= L) {
    if (p == 0) {
      for (int i = threadIdx.x; i < G * D; i += kThreads)
        store_elem(DT(), a.out, ((int64_t)b * a.num_heads + h0) * D + i, 0.f);
    }
    return;
  }
  const int ntok = min(P, L - tok0);
  const int nblk = (ntok + BS - 1) / BS;
  const int nslots = nblk * BS;
  const int NP = (L + P - 1) / P;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_uniform(threadIdx.x / kWave);
  const int col = lane & 15;    // MFMA column: query head within the group
  const int quad = lane >> 4;   // MFMA k-group / row group

  extern __shared__ float smem[];
  float* s_p = smem;                                         // [G][Pr]
  float* s_stat = s_p + G * Pr;                              // [2][G]
  int* s_bt = reinterpret_cast<int*>(s_stat + 2 * G);        // [Pr / BS]

  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks + (int64_t)p * (P / BS);
  for (int j = threadIdx.x; j < nblk; j += kThreads) s_bt[j] = bt[j];

  // Q^T as the B operand: lane holds Q[g = col][32*kc + 8*quad .. +8], zero for col >= G.
  uint4 qop[KC];
  {
    const uint4* qv = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.query) + ((int64_t)b * a.num_heads + h0) * D * 2);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      qop[kc] = (col < G) ? qv[col * (D / 8) + kc * 4 + quad] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  const int64_t tile_bytes = (int64_t)D * BS * 2;
  const int64_t block_bytes = tile_bytes * Hkv;
  const char* kbase = static_cast<const char*>(a.key_cache) + kh * tile_bytes;
  const char* vbase = static_cast<const char*>(a.value_cache) + kh * tile_bytes;

  // ---- 1. logits, 16-token tiles
  const int nt16 = (nslots + 15) / 16;
  for (int t0 = wave; t0 < nt16; t0 += kWaves * UK) {
    uint4 kv[UK][KC];
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int tile = t0 + u * kWaves;
      const int t = tile * 16 + col;
      if (tile < nt16 && t < nslots) {
        const char* kp = kbase + (int64_t)s_bt[t / BS] * block_bytes;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          kv[u][kc] = *reinterpret_cast<const uint4*>(
              kp + ((int64_t)(kc * 4 + quad) * BS + t % BS) * 16);
      } else {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) kv[u][kc] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int tile = t0 + u * kWaves;
      if (tile < nt16) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) acc = mfma16x16x32(DT(), kv[u][kc], qop[kc], acc);
        if (col < G) {
          const int tb = tile * 16 + quad * 4;
          f32x4 s;
#pragma unroll
          for (int r = 0; r < 4; ++r) s[r] = (tb + r < ntok) ? acc[r] * a.scale_log2 : -INFINITY;
          *reinterpret_cast<f32x4*>(&s_p[col * Pr + tb]) = s;
        }
      }
    }
  }
  __syncthreads();

  // ---- 2. softmax weights per query head; positions >= ntok become exactly 0
  const int nk32 = (nslots + 31) / 32;
  const int span = nk32 * 32;
  for (int g = wave; g < G; g += kWaves) {
    float m = -INFINITY;
    for (int t = lane; t < ntok; t += kWave) m = fmaxf(m, s_p[g * Pr + t]);
    m = wave_max(m);
    float l = 0.f;
    for (int t = lane; t < span; t += kWave) {
      const float e = (t < ntok) ? round_to(DT(), exp2f(s_p[g * Pr + t] - m)) : 0.f;
      s_p[g * Pr + t] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      s_stat[g] = m;
      s_stat[G + g] = l;
    }
  }
  __syncthreads();

  // ---- 3. O^T[d][g] = sum_t V^T[d][t] P^T[t][g]; this wave owns dims [d_lo, d_lo + 16*DT_PER_WAVE)
  const int d_lo = wave * DT_PER_WAVE * 16;
  f32x4 oacc[DT_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DT_PER_WAVE; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < nk32; k0 += UV) {
    uint4 vv[UV][DT_PER_WAVE];
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int t = (k0 + u) * 32 + quad * 8;  // first of this lane's 8 tokens
      if (k0 + u < nk32 && t < nslots) {
        const char* vp = vbase + (int64_t)s_bt[t / BS] * block_bytes + (t % BS) * 2;
#pragma unroll
        for (int i = 0; i < DT_PER_WAVE; ++i) {
          const int d = d_lo + i * 16 + col;
          vv[u][i] = *reinterpret_cast<const uint4*>(vp + (int64_t)d * BS * 2);
          if (t + 8 > ntok) vv[u][i] = mask_tokens(vv[u][i], t, ntok);
        }
      } else {
#pragma unroll
        for (int i = 0; i < DT_PER_WAVE; ++i) vv[u][i] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      if (k0 + u < nk32) {
        const int t = (k0 + u) * 32 + quad * 8;
        uint4 pop = make_uint4(0, 0, 0, 0);
        if (col < G) {
          const f32x4 p0 = *reinterpret_cast<const f32x4*>(&s_p[col * Pr + t]);
          const f32x4 p1 = *reinterpret_cast<const f32x4*>(&s_p[col * Pr + t + 4]);
          pop = make_uint4(pack2(DT(), p0[0], p0[1]), pack2(DT(), p0[2], p0[3]),
                           pack2(DT(), p1[0], p1[1]), pack2(DT(), p1[2], p1[3]));
        }
#pragma unroll
        for (int i = 0; i < DT_PER_WAVE; ++i) oacc[i] = mfma16x16x32(DT(), vv[u][i], pop, oacc[i]);
      }
    }
  }

  // ---- 4. epilogue: lane holds O[g = col][d = d_lo + 16 i + 4 quad + r]
  if (col < G) {
    const int h = h0 + col;
    if (NP == 1) {
      const float inv = 1.f / s_stat[G + col];
#pragma unroll
      for (int i = 0; i < DT_PER_WAVE; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store_elem(DT(), a.out, ((int64_t)b * a.num_heads + h) * D + d_lo + i * 16 + quad * 4 + r,
                     oacc[i][r] * inv);
    } else {
      const int64_t sp = ((int64_t)b * a.num_heads + h) * a.max_partitions + p;
#pragma unroll
      for (int i = 0; i < DT_PER_WAVE; ++i)
        *reinterpret_cast<f32x4*>(&a.part_acc[sp * D + d_lo + i * 16 + quad * 4]) = oacc[i];
      if (wave == 0 && quad == 0) {
        a.part_m[sp] = s_stat[col];
        a.part_l[sp] = s_stat[G + col];
      }
    }
  }
}

template <class DT, int D, int BS>
hipError_t launch_t(const DecodeArgs& a, int group, hipStream_t stream) {
  const int Pr = (a.partition_size + 31) / 32 * 32;
  const size_t lds = mfma_lds_bytes(group, BS, a.partition_size);
  const int64_t grid = (int64_t)a.num_seqs * a.num_kv_heads * a.max_partitions;
  hipLaunchKernelGGL((decode_mfma_kernel<DT, D, BS>), dim3((unsigned)grid), dim3(kThreads), lds,
                     stream, a, group, Pr);
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

bool mfma_supported(int dtype, int head_size, int block_size, int group) {
  return (dtype == 1 || dtype == 2) && (head_size == 64 || head_size == 128) &&
         (block_size == 8 || block_size == 16 || block_size == 32) && group >= 2 && group <= 16;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_size, int block_size,
                              int group, hipStream_t stream) {
  switch (dtype) {
    case 1: return by_head<F16>(a, head_size, block_size, group, stream);
    case 2: return by_head<BF16>(a, head_size, block_size, group, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
