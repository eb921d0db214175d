// Paged decode attention, phase 1, vector-ALU variant (fp32 caches; 16-bit ones run on the
// matrix cores).
//
// One workgroup (4 wave64s) per (work item, KV head): an item is a range of
// at most partition_size tokens of one sequence, taken from the plan kernel's
// list (work_plan.hip).  The cache layout is the one of the "Vllm" page,
// section "CacheEngine": a (block, KV head) key tile is
// [head_size/x][block_size][x] and a value tile is [head_size][block_size],
// each one contiguous run of head_size * block_size elements.  A wave
// streams whole tiles with one 16-byte load per lane per 1 KiB, so every
// block-table gather becomes fully coalesced 16-byte HBM reads.
//
// Per partition:
//   1. logits s_t = scale*log2(e) * q . K_t for the partition's tokens, into
//      LDS (tokens past the context are -inf: selected out, never multiplied);
//   2. per query head: m = max_t s_t, p_t = 2^(s_t - m), l = sum_t p_t
//      (softmax in base 2; the log2(e) factor folded into the scale makes it
//      the ordinary softmax of the "Vllm" page's attention formula);
//   3. acc_d = sum_t p_t V_t,d, with value entries of masked tokens replaced
//      by 0 before the multiply (a NaN in an unused slot cannot leak);
//   4. one partition: out = acc / l; several: (m, l, acc) go to the split-K
//      workspace for the reduce kernel (FlashDecoding-style KV splitting, the
//      "Vllm" page, "Prefill vs decoding" item 5).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <class DT, int D, int BS>
struct TileShape {
  static constexpr int X = DT::X;
  static constexpr int CH = D / X;         // 16-byte chunks along the head dim (key tile)
  static constexpr int NCK = CH * BS;      // 16-byte chunks per (block, head) tile
  static constexpr int NL = NCK / kWave;   // loads per lane per tile
  static constexpr int TG = kWave / BS;    // lanes holding pieces of one token's key
  static constexpr int VCR = BS / X;       // 16-byte chunks per value row (one dim, BS tokens)
  static constexpr int DPL = kWave / VCR;  // head dims per wave-wide value load
  static_assert(NCK % kWave == 0, "a tile must be a whole number of wave-wide loads");
  static_assert(VCR >= 1 && kWave % VCR == 0, "value row must hold whole 16-byte chunks");
  static_assert(kWave % BS == 0, "block_size must divide the wave");
};

template <class DT, int D, int BS, int G>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeArgs a) {
  using S = TileShape<DT, D, BS>;
  constexpr int X = S::X, NL = S::NL, TG = S::TG, VCR = S::VCR, DPL = S::DPL;
  constexpr int U = 2;  // tiles in flight per wave
  const int P = a.partition_size;
  const int Hkv = a.num_kv_heads;
  // Workgroup t takes ticket t of the plan's list: work item t / Hkv, KV head t % Hkv.  Items
  // here hold one sequence each (shared prefixes run on the matrix-core kernel).
  const int t = blockIdx.x;
  if (t >= int(a.queue[1]) * Hkv) return;
  const uint4 it = a.items[t / Hkv];
  if (!item_fits(a, it)) return;
  const int kh = t % Hkv;
  const int b = int(it.x);
  const int slot = int(it.y >> 8);
  const int tok0 = int(it.z);
  const int h0 = kh * G;
  if (int(it.w) <= tok0) {  // the sole item of an empty context: defined as a zero output
    for (int i = threadIdx.x; i < G * D; i += kThreads)
      store_elem(DT(), a.out, ((int64_t)b * a.num_heads + h0) * D + i, 0.f);
    return;
  }
  const int ntok = int(it.w) - tok0;
  const int nblk = (ntok + BS - 1) / BS;
  const int NP = a.np_of[b];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_uniform(threadIdx.x / kWave);

  extern __shared__ float smem[];
  float* s_p = smem;                       // [G][P]: logits, then probabilities
  float* s_red = smem + G * P;             // [kWaves][G][D]: per-wave partial outputs
  float* s_stat = s_red + kWaves * G * D;  // [2][G]: max, sum

  // Query, pre-scaled.  Lane holds dims of chunks c = i*TG + lane/BS (the key chunks it loads).
  float q[G][NL][X];
  {
    const uint4* qv = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.query) + ((int64_t)b * a.num_heads + h0) * D * DT::kBytes);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        unpack(DT(), qv[g * S::CH + i * TG + lane / BS], q[g][i]);
#pragma unroll
        for (int e = 0; e < X; ++e) q[g][i][e] *= a.scale_log2;
      }
  }

  const int64_t tile_bytes = (int64_t)D * BS * DT::kBytes;
  const int64_t block_bytes = tile_bytes * Hkv;
  const char* kbase = static_cast<const char*>(a.key_cache) + kh * tile_bytes;
  const char* vbase = static_cast<const char*>(a.value_cache) + kh * tile_bytes;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks + tok0 / BS;

  // ---- 1. logits
  for (int j0 = wave; j0 < nblk; j0 += kWaves * U) {
    uint4 kv[U][NL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * kWaves;
      if (j < nblk) {
        const uint4* kp = reinterpret_cast<const uint4*>(kbase + (int64_t)bt[j] * block_bytes);
#pragma unroll
        for (int i = 0; i < NL; ++i) kv[u][i] = kv_load<true>(kp + i * kWave + lane);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * kWaves;
      if (j < nblk) {
        float dot[G];
#pragma unroll
        for (int g = 0; g < G; ++g) dot[g] = 0.f;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float kf[X];
          unpack(DT(), kv[u][i], kf);
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < X; ++e) dot[g] = fmaf(q[g][i][e], kf[e], dot[g]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) dot[g] = xor_sum_from<BS>(dot[g]);
        const int t = j * BS + lane;
        if (lane < BS) {
#pragma unroll
          for (int g = 0; g < G; ++g) s_p[g * P + t] = (t < ntok) ? dot[g] : -INFINITY;
        }
      }
    }
  }
  __syncthreads();

  // ---- 2. softmax statistics, one wave per query head
  const int nslots = nblk * BS;
  for (int g = wave; g < G; g += kWaves) {
    float m = -INFINITY;
    for (int t = lane; t < nslots; t += kWave) m = fmaxf(m, s_p[g * P + t]);
    m = wave_max(m);
    float l = 0.f;
    for (int t = lane; t < nslots; t += kWave) {
      const float e = exp2f(s_p[g * P + t] - m);
      s_p[g * P + t] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      s_stat[g] = m;
      s_stat[G + g] = l;
    }
  }
  __syncthreads();

  // ---- 3. P . V.  Lane handles value chunk tc of dims d = i*DPL + lane/VCR.
  float acc[G][NL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NL; ++i) acc[g][i] = 0.f;
  const int tc = lane % VCR;
  for (int j0 = wave; j0 < nblk; j0 += kWaves * U) {
    uint4 vv[U][NL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * kWaves;
      if (j < nblk) {
        const uint4* vp = reinterpret_cast<const uint4*>(vbase + (int64_t)bt[j] * block_bytes);
#pragma unroll
        for (int i = 0; i < NL; ++i) vv[u][i] = kv_load<true>(vp + i * kWave + lane);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * kWaves;
      if (j < nblk) {
        const int t0 = j * BS + tc * X;
        float pr[G][X];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < X; ++e) pr[g][e] = s_p[g * P + t0 + e];
        const bool tail = (j + 1) * BS > ntok;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float vf[X];
          unpack(DT(), vv[u][i], vf);
          if (tail) {
#pragma unroll
            for (int e = 0; e < X; ++e) vf[e] = (t0 + e < ntok) ? vf[e] : 0.f;
          }
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < X; ++e) acc[g][i] = fmaf(pr[g][e], vf[e], acc[g][i]);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NL; ++i) acc[g][i] = xor_sum_below<VCR>(acc[g][i]);
  if (tc == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < NL; ++i) s_red[(wave * G + g) * D + i * DPL + lane / VCR] = acc[g][i];
  }
  __syncthreads();

  // ---- 4. epilogue
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int g = i / D, d = i % D;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += s_red[(w * G + g) * D + d];
    const int h = h0 + g;
    if (NP <= 1) {
      store_elem(DT(), a.out, ((int64_t)b * a.num_heads + h) * D + d, sum / s_stat[G + g]);
    } else {
      const int64_t sp = ((int64_t)b * a.num_heads + h) * a.slots + slot;
      a.part_acc[sp * D + d] = sum;
      if (d == 0) {
        a.part_m[sp] = s_stat[g];
        a.part_l[sp] = s_stat[G + g];
      }
    }
  }
}

template <class DT, int D, int BS, int G>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const size_t lds = valu_lds_bytes(G, D, a.partition_size);
  const int64_t grid = (int64_t)a.num_seqs * a.num_kv_heads * a.slots;
  if (a.plan_mode != 2) {
    const hipError_t e = launch_plan(a, BS, 1, stream);
    if (e != hipSuccess || a.plan_mode == 1) return e;
  }
  hipLaunchKernelGGL((decode_valu_kernel<DT, D, BS, G>), dim3((unsigned)grid), dim3(kThreads), lds,
                     stream, a);
  return hipGetLastError();
}

template <class DT, int D, int BS>
hipError_t by_group(const DecodeArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_t<DT, D, BS, 1>(a, s);
    case 2: return launch_t<DT, D, BS, 2>(a, s);
    case 4: return launch_t<DT, D, BS, 4>(a, s);
    case 8: return launch_t<DT, D, BS, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class DT, int D>
hipError_t by_block(const DecodeArgs& a, int bs, int group, hipStream_t s) {
  switch (bs) {
    case 8: return by_group<DT, D, 8>(a, group, s);
    case 16: return by_group<DT, D, 16>(a, group, s);
    case 32: return by_group<DT, D, 32>(a, group, s);
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

bool valu_supported(int dtype, int head_size, int block_size, int group) {
  return dtype == 0 && (head_size == 64 || head_size == 128) &&
         (block_size == 8 || block_size == 16 || block_size == 32) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_size, int block_size,
                              int group, hipStream_t stream) {
  if (dtype != 0) return hipErrorInvalidValue;
  return by_head<F32>(a, head_size, block_size, group, stream);
}

}  // namespace pkv
