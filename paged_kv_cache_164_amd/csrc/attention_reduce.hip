// Paged decode attention, phase 2: merge each sequence's partial results.
//
// For one (sequence, query head) with items p = 0..NP-1 carrying (m_p, l_p, acc_p) in base-2
// logit units:
//   M = max_p m_p,  w_p = 2^(m_p - M)
//   out = sum_p w_p acc_p / sum_p w_p l_p
// which equals the softmax-weighted sum over the whole context (the log-sum-exp identity
// behind split-K / FlashDecoding decoding; the "Vllm" page, "Prefill vs decoding" item 5).
//
// One workgroup per (sequence, query head): one wave for many rows, else 256 threads.  Its
// threads form S strands of D/4 threads; a thread holds 4 dims of one strand, and strand s takes
// items s, s + S, ..., four loaded at a time, with its own running maximum (so its loads go out
// together, with no workgroup-wide max first).  The
// strands are then merged in LDS, always in strand order: the result is run-to-run
// deterministic.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <class DT, int D, int T>
__global__ __launch_bounds__(T) void reduce_kernel(DecodeArgs a) {
  constexpr int TPS = D / 4;           // threads per strand (4 dims each)
  constexpr int S = T / TPS;           // strands
  const int row = blockIdx.x;          // b * num_heads + h
  const int b = row / a.num_heads;
  const int NP = min(a.np_of[b], a.slots);
  if (NP <= 1) return;  // written directly by phase 1
  const int s = threadIdx.x / TPS, d0 = (threadIdx.x % TPS) * 4;
  const int64_t base = (int64_t)row * a.slots;
  const float* pm = a.part_m + base;
  const float* pl = a.part_l + base;
  const float* pacc = a.part_acc + base * D + d0;

  // strand s: online merge of its items (running max ms, sum ls, vector acc)
  float ms = -INFINITY, ls = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // U of the strand's items loaded at once, then merged in item order
  constexpr int U = 4;
  for (int q0 = s; q0 < NP; q0 += U * S) {
    float mq[U], lq[U];
    float4 aq[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = min(q0 + u * S, NP - 1);  // past the end: a valid index, its values unused
      mq[u] = pm[q];
      lq[u] = pl[q];
      aq[u] = *reinterpret_cast<const float4*>(pacc + (int64_t)q * D);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (q0 + u * S >= NP) break;
      const float mn = fmaxf(ms, mq[u]);
      const float c = exp2f(ms - mn), w = exp2f(mq[u] - mn);  // ms = -inf at first: c = 0
      ls = fmaf(ls, c, w * lq[u]);
      acc.x = fmaf(acc.x, c, w * aq[u].x);
      acc.y = fmaf(acc.y, c, w * aq[u].y);
      acc.z = fmaf(acc.z, c, w * aq[u].z);
      acc.w = fmaf(acc.w, c, w * aq[u].w);
      ms = mn;
    }
  }
  __shared__ float s_m[S], s_l[S];
  __shared__ float4 s_acc[S][TPS];
  if (threadIdx.x % TPS == 0) {
    s_m[s] = ms;
    s_l[s] = ls;
  }
  s_acc[s][threadIdx.x % TPS] = acc;
  __syncthreads();
  if (s != 0) return;
  // strand 0's threads merge all strands, in strand order (strands without items hold m = -inf)
  float M = s_m[0];
#pragma unroll
  for (int k = 1; k < S; ++k) M = fmaxf(M, s_m[k]);
  float den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const float w = exp2f(s_m[k] - M);
    const float4 v = s_acc[k][threadIdx.x];
    den = fmaf(w, s_l[k], den);
    num.x = fmaf(w, v.x, num.x);
    num.y = fmaf(w, v.y, num.y);
    num.z = fmaf(w, v.z, num.z);
    num.w = fmaf(w, v.w, num.w);
  }
  const float inv = 1.f / den;
  const int64_t o = (int64_t)row * D + d0;
  store_elem(DT(), a.out, o + 0, num.x * inv);
  store_elem(DT(), a.out, o + 1, num.y * inv);
  store_elem(DT(), a.out, o + 2, num.z * inv);
  store_elem(DT(), a.out, o + 3, num.w * inv);
}

// Workgroup shape by row count: many rows (a large batch, few items each) take one wave per
// row, so every row is resident in one round; few rows with many partials each keep 256 threads
// (more strands, more loads in flight per row).
constexpr int64_t kWaveRowsFrom = 4096;

template <class DT, int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_seqs * a.num_heads;
  if (rows >= kWaveRowsFrom)
    hipLaunchKernelGGL((reduce_kernel<DT, D, 64>), dim3((unsigned)rows), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((reduce_kernel<DT, D, kThreads>), dim3((unsigned)rows), dim3(kThreads), 0,
                       stream, a);
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
