// Router epilogue: top-k over each token's logits with softmax weights, per-expert counts,
// and the expert-major, token-ordered slot permutation that groups every expert's rows
// contiguously for the grouped GEMMs (grouped-nf4-gemm 0.25.0 project description, opening
// section: one launch over all active experts, a router epilogue among the glue kernels).
// The permutation is a stable counting sort over chunks of 1024 tokens (for at most 4096
// slots, steps 2-4 are one launch, route_small_kernel):
//
//   1. topk_kernel     one wave per token: k rounds of a wave-wide arg-max (DPP lane moves)
//                      under the order (higher logit, then lower expert index); softmax
//                      weights
//   2. count_kernel    one workgroup per chunk: LDS histogram of the chunk's picks, cc[c][e]
//                      (no global atomics: per-pick atomics on a few hot counters serialised
//                      badly, 80 us at T = 4096, E = 8)
//   3. offsets_kernel  one workgroup: expert offsets (prefix sum of the totals) and the first
//                      slot of every (chunk, expert) pair
//   4. scatter_kernel  one workgroup per (chunk, expert): the chunk's tokens in order with a
//                      ballot prefix sum, so slots land expert-major and token-ascending
//                      (stable, deterministic)
#include "e4b_device.h"
#include "e4b_internal.h"
#include "e4b_topk.h"

namespace e4b {

template <int PL>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int64_t T,
                                                   int E, int k, int renorm,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  int id;
  float wt;
  topk_token<PL>(logits + t * E, E, k, renorm, lane, id, wt);
  if (lane < k) {
    ids[t * k + lane] = id;
    wts[t * k + lane] = wt;
  }
}

constexpr int kTokChunk = 1024;  // tokens per chunk of the counting sort

int route_chunks(int64_t T) { return int(T > 0 ? (T + kTokChunk - 1) / kTokChunk : 1); }

// cc[c][e] = number of picks of expert e by the tokens of chunk c (LDS histogram).
__global__ void __launch_bounds__(256) count_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                    int E, int k, int32_t* __restrict__ cc) {
  __shared__ int32_t hist[1024];
  for (int i = threadIdx.x; i < E; i += 256) hist[i] = 0;
  __syncthreads();
  const int64_t lo = int64_t(blockIdx.x) * kTokChunk * k;
  int64_t hi = lo + int64_t(kTokChunk) * k;
  if (hi > T * k) hi = T * k;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256) atomicAdd(&hist[ids[i]], 1);
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += 256) cc[int64_t(blockIdx.x) * E + i] = hist[i];
}

// One workgroup: offsets[e] = exclusive prefix sum over experts of the total counts,
// offsets[E] = T*k; then cc[c][e] becomes the first slot of (chunk c, expert e):
// offsets[e] + sum of cc[c'][e] over c' < c.
// Up to kCcLds counts are first copied into LDS by the whole workgroup (all loads in flight at
// once), so the per-expert sums over chunks read LDS instead of waiting on one global load after
// another (skewed 64-expert layer, 16 chunks: the whole routing call 56.3 -> 53.1 us).
constexpr int kCcLds = 8192;

__global__ void __launch_bounds__(256) offsets_kernel(int32_t* __restrict__ cc, int chunks, int E,
                                                      int32_t* __restrict__ offsets) {
  __shared__ int32_t wsum[4];
  __shared__ int32_t s_cc[kCcLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = int64_t(chunks) * E;
  const bool staged = n <= kCcLds;  // uniform
  if (staged) {
    for (int i = tid; i < int(n); i += 256) s_cc[i] = cc[i];
    __syncthreads();
  }
  auto count = [&](int c, int e) { return staged ? s_cc[c * E + e] : cc[int64_t(c) * E + e]; };
  constexpr int kPer = 4;  // experts per thread (E <= 1024)
  int tot[kPer];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid * kPer + i;
    int t = 0;
    if (e < E)
      for (int c = 0; c < chunks; ++c) t += count(c, e);
    tot[i] = t;
    mine += t;
  }
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - mine;
  for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid * kPer + i;
    if (e < E) {
      offsets[e] = run;
      int base = run;
      for (int c = 0; c < chunks; ++c) {
        const int v = count(c, e);
        cc[int64_t(c) * E + e] = base;
        base += v;
      }
    }
    run += tot[i];
  }
  if (tid == 255) offsets[E] = run;
}

// Slots of expert e among tokens [t_begin, t_end), in token order, written from slots[base]:
// a ballot prefix sum per 256 tokens (stable, deterministic).  Whole workgroup.
__device__ __forceinline__ void scatter_range(const int32_t* __restrict__ ids, int64_t t_begin,
                                              int64_t t_end, int k, int e, int base,
                                              int32_t* __restrict__ slots, int32_t* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int running = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 256) {
    const int64_t t = t0 + tid;
    int flag = 0, jsel = 0;
    if (t < t_end) {
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

// One workgroup per (chunk c, expert e): the chunk's tokens, from the first slot cc[c][e].
__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                      int E, int k,
                                                      const int32_t* __restrict__ cc,
                                                      int32_t* __restrict__ slots) {
  __shared__ int32_t wave_tot[4];
  const int e = int(blockIdx.x % unsigned(E));
  const int64_t c = blockIdx.x / unsigned(E);
  int64_t t_end = (c + 1) * kTokChunk;
  if (t_end > T) t_end = T;
  scatter_range(ids, c * kTokChunk, t_end, k, e, cc[c * E + e], slots, wave_tot);
}

// Few slots (T*k <= kSmallIds): one workgroup per expert counts the slots of lower experts
// and its own directly from ids (every workgroup reads all ids, a few KB from L2), writes
// its offset and scatters; one launch instead of the count / offsets / scatter passes.
constexpr int64_t kSmallIds = 4096;

__global__ void __launch_bounds__(256) route_small_kernel(const int32_t* __restrict__ ids,
                                                          int64_t T, int E, int k,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ slots) {
  __shared__ int32_t red[2][4];
  __shared__ int32_t wave_tot[4];
  const int e = int(blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = T * k;
  int below = 0, mine = 0;
  for (int64_t i = tid; i < n; i += 256) {
    const int v = ids[i];
    below += v < e;
    mine += v == e;
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    below += __shfl_xor(below, off);
    mine += __shfl_xor(mine, off);
  }
  if (lane == 0) {
    red[0][wave] = below;
    red[1][wave] = mine;
  }
  __syncthreads();
  const int base = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  if (tid == 0) {
    offsets[e] = base;
    if (e == E - 1) offsets[E] = base + red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
  scatter_range(ids, 0, T, k, e, base, slots, wave_tot);
}

// A few tokens (T <= kTinyT): route_small_kernel with the top-k folded in.  Every workgroup
// (one per expert) computes the picks of all T tokens into LDS, one wave per token; workgroup
// 0 also writes them out.  One launch for the whole router epilogue.
constexpr int64_t kTinyT = 8;

template <int PL>
__global__ void __launch_bounds__(256) route_tiny_kernel(const float* __restrict__ logits,
                                                         int64_t T, int E, int k, int renorm,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ slots) {
  __shared__ int32_t sids[kTinyT * 64];
  __shared__ int32_t red[2][4];
  __shared__ int32_t wave_tot[4];
  const int e = int(blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int t = wave; t < int(T); t += 4) {
    int id;
    float wt;
    topk_token<PL>(logits + int64_t(t) * E, E, k, renorm, lane, id, wt);
    if (lane < k) {
      sids[t * k + lane] = id;
      if (e == 0) {
        ids[t * k + lane] = id;
        wts[t * k + lane] = wt;
      }
    }
  }
  __syncthreads();
  const int n = int(T) * k;
  int below = 0, mine = 0;
  for (int i = tid; i < n; i += 256) {
    const int v = sids[i];
    below += v < e;
    mine += v == e;
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    below += __shfl_xor(below, off);
    mine += __shfl_xor(mine, off);
  }
  if (lane == 0) {
    red[0][wave] = below;
    red[1][wave] = mine;
  }
  __syncthreads();
  const int base = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  if (tid == 0) {
    offsets[e] = base;
    if (e == E - 1) offsets[E] = base + red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
  scatter_range(sids, 0, T, k, e, base, slots, wave_tot);
}

hipError_t launch_route(const float* logits, int64_t T, int64_t E, int k, bool renorm,
                        int32_t* ids, float* w, int32_t* offsets, int32_t* slots, int32_t* cc,
                        hipStream_t stream) {
  const int chunks = route_chunks(T);
  if (T > 0 && T <= kTinyT) {
    const unsigned g = unsigned(E);
    const int rn = renorm ? 1 : 0;
    if (E <= 64)
      hipLaunchKernelGGL(route_tiny_kernel<1>, dim3(g), dim3(256), 0, stream, logits, T, int(E), k, rn,
                         ids, w, offsets, slots);
    else if (E <= 128)
      hipLaunchKernelGGL(route_tiny_kernel<2>, dim3(g), dim3(256), 0, stream, logits, T, int(E), k, rn,
                         ids, w, offsets, slots);
    else if (E <= 256)
      hipLaunchKernelGGL(route_tiny_kernel<4>, dim3(g), dim3(256), 0, stream, logits, T, int(E), k, rn,
                         ids, w, offsets, slots);
    else
      hipLaunchKernelGGL(route_tiny_kernel<kMaxExpertsPerLane>, dim3(g), dim3(256), 0, stream, logits,
                         T, int(E), k, rn, ids, w, offsets, slots);
    return hipGetLastError();
  }
  if (T > 0) {
    const int64_t blocks = (T + 3) / 4;
    const unsigned g = unsigned(blocks);
    const int rn = renorm ? 1 : 0;
    if (E <= 64)
      hipLaunchKernelGGL(topk_kernel<1>, dim3(g), dim3(256), 0, stream, logits, T, int(E), k, rn, ids, w);
    else if (E <= 128)
      hipLaunchKernelGGL(topk_kernel<2>, dim3(g), dim3(256), 0, stream, logits, T, int(E), k, rn, ids, w);
    else if (E <= 256)
      hipLaunchKernelGGL(topk_kernel<4>, dim3(g), dim3(256), 0, stream, logits, T, int(E), k, rn, ids, w);
    else
      hipLaunchKernelGGL(topk_kernel<kMaxExpertsPerLane>, dim3(g), dim3(256), 0, stream, logits, T,
                         int(E), k, rn, ids, w);
  }
  if (T * k <= kSmallIds) {
    hipLaunchKernelGGL(route_small_kernel, dim3(unsigned(E)), dim3(256), 0, stream, ids, T,
                       int(E), k, offsets, slots);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(count_kernel, dim3(unsigned(chunks)), dim3(256), 0, stream, ids, T, int(E),
                     k, cc);
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(256), 0, stream, cc, chunks, int(E), offsets);
  if (T > 0)
    hipLaunchKernelGGL(scatter_kernel, dim3(unsigned(int64_t(chunks) * E)), dim3(256), 0, stream,
                       ids, T, int(E), k, cc, slots);
  return hipGetLastError();
}

}  // namespace e4b
