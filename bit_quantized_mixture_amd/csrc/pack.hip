// Packers: bf16 expert stacks -> NF4 (block 64, float32 absmax) or MXFP4 (e2m1 + e8m0
// per 32).  Each lane owns 8 consecutive weights (one 16-byte load); the 8 lanes (NF4) or
// 4 lanes (MXFP4) of a block reduce the block's absmax with cross-lane shuffles, then every
// lane quantises its own 8 weights and writes one 32-bit word of codes.
//
// NF4 follows bitsandbytes pull request #1984 (Summary, Design: per-expert blockwise
// absmax, uint8 packing, float32 absmax) and grouped-nf4-gemm 0.25.0 ("Try it on CPU right
// now", example 1: [N, K] -> [N, K/2] uint8 + [N, K/64] float32).  MXFP4 follows the same
// page's example 2 ([N, K] -> [N, K/32, 16] + [N, K/32]) with the OCP MX v1.0 conversion.
#include "e4b_device.h"
#include "e4b_internal.h"

namespace e4b {

// Each thread: 8 consecutive bf16 of one row.  Blocks never straddle rows (K % 64 == 0),
// so chunk q covers elements [8q, 8q+8) of the flattened [R, K] array.
__global__ void __launch_bounds__(256) pack_nf4_kernel(const uint16_t* __restrict__ w,
                                                       uint8_t* __restrict__ packed,
                                                       float* __restrict__ absmax,
                                                       int64_t n_chunks) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  // The loop bound is rounded up to a multiple of 8 chunks so the 8 lanes of a block stay
  // converged through the shuffles; n_chunks is itself a multiple of 8.
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < n_chunks; q += stride) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(w + 8 * q);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(raw[i] << 16);
      v[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
    a = fmaxf(a, __shfl_xor(a, 1, 8));
    a = fmaxf(a, __shfl_xor(a, 2, 8));
    a = fmaxf(a, __shfl_xor(a, 4, 8));
    uint32_t word = 0x77777777u;  // all-zero block: code 7 everywhere
    if (a > 0.f) {
      word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float n = __fdiv_rn(v[i], a);
        uint32_t code = 0;
#pragma unroll
        for (int j = 0; j < 15; ++j) code += (n >= __uint_as_float(kNf4Up[j])) ? 1u : 0u;
        // element 2b -> high nibble of byte b, element 2b+1 -> low nibble
        const int byte = i >> 1;
        const int shift = 8 * byte + ((i & 1) ? 0 : 4);
        word |= code << shift;
      }
    }
    reinterpret_cast<uint32_t*>(packed)[q] = word;
    if ((q & 7) == 0) absmax[q >> 3] = a;
  }
}

__global__ void __launch_bounds__(256) pack_mxfp4_kernel(const uint16_t* __restrict__ w,
                                                         uint8_t* __restrict__ blocks,
                                                         uint8_t* __restrict__ scales,
                                                         int64_t n_chunks) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < n_chunks; q += stride) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(w + 8 * q);
    uint32_t bits[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bits[2 * i] = raw[i] << 16;
      bits[2 * i + 1] = raw[i] & 0xFFFF0000u;
    }
    uint32_t amax_bits = 0;  // max of |v| compared as unsigned magnitudes (finite inputs)
#pragma unroll
    for (int i = 0; i < 8; ++i) amax_bits = max(amax_bits, bits[i] & 0x7FFFFFFFu);
    amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, 1, 4));
    amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, 2, 4));
    // shared exponent floor(log2 amax) - 2, clamped to [-127, 127]; zero/subnormal -> -127
    const int ef = int(amax_bits >> 23);
    const int s = ef == 0 ? -127 : max(ef - 127 - 2, -127);
    const float inv = __uint_as_float(uint32_t(127 - s) << 23);  // 2^-s, exact (s <= 126)
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float m = fabsf(__uint_as_float(bits[i])) * inv;  // exact power-of-two scaling
      uint32_t code = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) +
                      (m >= 3.5f) + (m > 5.0f);
      code |= (bits[i] >> 28) & 0x8u;
      // element 2b -> low nibble of byte b, element 2b+1 -> high nibble
      word |= code << (4 * i);
    }
    reinterpret_cast<uint32_t*>(blocks)[q] = word;
    if ((q & 3) == 0) scales[q >> 2] = uint8_t(s + 127);
  }
}

static int grid_for(int64_t n_chunks) {
  int64_t g = (n_chunks + 255) / 256;
  return int(g < 65536 ? (g < 1 ? 1 : g) : 65536);
}

hipError_t launch_pack_nf4(const uint16_t* w, int64_t n_elems, uint8_t* packed, float* absmax,
                           hipStream_t stream) {
  const int64_t n_chunks = n_elems / 8;
  hipLaunchKernelGGL(pack_nf4_kernel, dim3(grid_for(n_chunks)), dim3(256), 0, stream, w, packed,
                     absmax, n_chunks);
  return hipGetLastError();
}

hipError_t launch_pack_mxfp4(const uint16_t* w, int64_t n_elems, uint8_t* blocks, uint8_t* scales,
                             hipStream_t stream) {
  const int64_t n_chunks = n_elems / 8;
  hipLaunchKernelGGL(pack_mxfp4_kernel, dim3(grid_for(n_chunks)), dim3(256), 0, stream, w, blocks,
                     scales, n_chunks);
  return hipGetLastError();
}

}  // namespace e4b
