// Paged decode attention, phase 2: combine the partitions of long contexts.
//
// For one (sequence, query head) with partitions p = 0..NP-1 carrying
// (m_p, l_p, acc_p) in base-2 logit units:
//   M = max_p m_p,  w_p = 2^(m_p - M)
//   out = sum_p w_p acc_p / sum_p w_p l_p
// which equals the softmax-weighted sum over the whole context (the
// log-sum-exp identity behind split-K / FlashDecoding decoding; the "Vllm"
// page, "Prefill vs decoding" item 5).  The summation order is fixed, so
// results are run-to-run deterministic.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

__device__ __forceinline__ float block_max(float v, float* scratch) {
  v = wave_max(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, scratch[w]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* scratch) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r += scratch[w];
  return r;
}

template <class DT, int D>
__global__ __launch_bounds__(kThreads) void reduce_kernel(DecodeArgs a) {
  constexpr int SPLIT = kThreads / D;  // partition strands per head dim
  const int h = blockIdx.x % a.num_heads;
  const int b = blockIdx.x / a.num_heads;
  // the plan kernel counted each sequence's partial results
  const int NP = min(a.np_of[b], a.slots);
  if (NP <= 1) return;  // written directly by phase 1
  const int64_t base = ((int64_t)b * a.num_heads + h) * a.slots;

  extern __shared__ float smem[];
  float* s_red = smem;              // [kWaves] block-reduction scratch
  float* s_num = smem + kWaves;     // [kThreads] partial numerators
  float* s_w = s_num + kThreads;    // [slots] partition weights

  float m = -INFINITY;
  for (int q = threadIdx.x; q < NP; q += kThreads) m = fmaxf(m, a.part_m[base + q]);
  const float M = block_max(m, s_red);
  float den = 0.f;
  for (int q = threadIdx.x; q < NP; q += kThreads) {
    const float w = exp2f(a.part_m[base + q] - M);
    s_w[q] = w;
    den += w * a.part_l[base + q];
  }
  den = block_sum(den, s_red);  // contains the barrier that publishes s_w

  const int d = threadIdx.x % D, strand = threadIdx.x / D;
  float num = 0.f;
  for (int q = strand; q < NP; q += SPLIT) num = fmaf(s_w[q], a.part_acc[(base + q) * D + d], num);
  s_num[threadIdx.x] = num;
  __syncthreads();
  if (strand == 0) {
#pragma unroll
    for (int s = 1; s < SPLIT; ++s) num += s_num[s * D + d];
    store_elem(DT(), a.out, ((int64_t)b * a.num_heads + h) * D + d, num / den);
  }
}

template <class DT, int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const size_t lds = sizeof(float) * (kWaves + kThreads + size_t(a.slots));
  hipLaunchKernelGGL((reduce_kernel<DT, D>), dim3((unsigned)((int64_t)a.num_seqs * a.num_heads)),
                     dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <class DT>
hipError_t by_head(const DecodeArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_t<DT, 64>(a, s);
    case 128: return launch_t<DT, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_reduce(const DecodeArgs& a, int dtype, int head_size, hipStream_t stream) {
  switch (dtype) {
    case 0: return by_head<F32>(a, head_size, stream);
    case 1: return by_head<F16>(a, head_size, stream);
    case 2: return by_head<BF16>(a, head_size, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
