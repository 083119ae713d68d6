// Router epilogue: top-k over each token's logits with softmax weights, per-expert counts,
// and the expert-major, token-ordered slot permutation that groups every expert's rows
// contiguously for the grouped GEMMs (grouped-nf4-gemm 0.25.0 project description, opening
// section: one launch over all active experts, a router epilogue among the glue kernels).
//
//   1. zero_counts     counts[E] = 0
//   2. topk_kernel     one wave per token: k rounds of a wave-wide arg-max under the order
//                      (higher logit, then lower expert index); softmax weights; counts[e]++
//   3. scatter_kernel  one workgroup per expert: its offset is the sum of the counts of the
//                      lower experts; tokens are scanned in order with a ballot prefix sum,
//                      so slots land expert-major and token-ascending (stable, deterministic)
#include "e4b_device.h"
#include "e4b_internal.h"

namespace e4b {

constexpr int kMaxExpertsPerLane = 16;  // E <= 1024

__global__ void zero_counts_kernel(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// a beats b: higher value, or equal value and lower index.  Invalid entries carry
// index INT_MAX and value -inf; logits are finite, so any valid entry beats them.
__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int64_t T,
                                                   int E, int k, int renorm,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ wts,
                                                   int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  const float* row = logits + t * E;
  float v[kMaxExpertsPerLane];
  const int per_lane = (E + 63) / 64;
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = (i < per_lane && e < E) ? row[e] : -INFINITY;
  }
  uint32_t taken = 0;  // bit i: my entry i already chosen
  int my_id = 0;
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i) {
      const int e = lane + 64 * i;
      if (i < per_lane && e < E && !((taken >> i) & 1u) && beats(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (beats(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      my_id = bi;
      my_v = bv;
    }
  }
  const float vmax = __shfl(my_v, 0);  // the first pick is the largest logit
  float ex = lane < k ? expf(my_v - vmax) : 0.f;
  float denom;
  if (renorm) {
    denom = ex;
  } else {
    denom = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i) {
      const int e = lane + 64 * i;
      if (i < per_lane && e < E) denom += expf(v[i] - vmax);
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) denom += __shfl_xor(denom, off);
  if (lane < k) {
    ids[t * k + lane] = my_id;
    wts[t * k + lane] = ex / denom;
    atomicAdd(&counts[my_id], 1);
  }
}

__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                      int E, int k,
                                                      const int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ slots) {
  __shared__ int32_t red[4];
  __shared__ int32_t wave_tot[4];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int part = 0;
  for (int i = tid; i < e; i += 256) part += counts[i];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) part += __shfl_xor(part, off);
  if (lane == 0) red[wave] = part;
  __syncthreads();
  const int base = red[0] + red[1] + red[2] + red[3];
  if (tid == 0) {
    offsets[e] = base;
    if (e == E - 1) offsets[E] = base + counts[e];
  }
  int running = 0;
  for (int64_t t0 = 0; t0 < T; t0 += 256) {
    const int64_t t = t0 + tid;
    int flag = 0, jsel = 0;
    if (t < T) {
      for (int j = 0; j < k; ++j) {
        if (ids[t * k + j] == e) {
          flag = 1;
          jsel = j;
        }
      }
    }
    const uint64_t b = __ballot(flag);
    const int before = __popcll(b & ((1ull << lane) - 1ull));
    __syncthreads();  // previous iteration's readers of wave_tot are done
    if (lane == 0) wave_tot[wave] = __popcll(b);
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      woff += (w < wave) ? wave_tot[w] : 0;
      tot += wave_tot[w];
    }
    if (flag) slots[base + running + woff + before] = int32_t(t * k + jsel);
    running += tot;
  }
}

hipError_t launch_route(const float* logits, int64_t T, int64_t E, int k, bool renorm,
                        int32_t* ids, float* w, int32_t* offsets, int32_t* slots, int32_t* counts,
                        hipStream_t stream) {
  hipLaunchKernelGGL(zero_counts_kernel, dim3(int((E + 255) / 256)), dim3(256), 0, stream, counts,
                     int(E));
  if (T > 0) {
    const int64_t blocks = (T + 3) / 4;
    hipLaunchKernelGGL(topk_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, logits, T,
                       int(E), k, renorm ? 1 : 0, ids, w, counts);
  }
  hipLaunchKernelGGL(scatter_kernel, dim3(unsigned(E)), dim3(256), 0, stream, ids, T, int(E), k,
                     counts, offsets, slots);
  return hipGetLastError();
}

}  // namespace e4b
