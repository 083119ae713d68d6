// Device-side helpers shared by the e4b kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e4b {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------
// NF4 codebook (QLoRA NormalFloat-4, ascending, code 0..15) in the two forms used here.
//
// (1) Decode table: fp16 rounding of each value, fp16 bits for codes 0..15:
//     bc00 b992 b833 b652 b48d b1ea add4 0000 2d18 3126 33e0 3568 370d 3880 39c9 3c00
//     held as a low-byte plane and a high-byte plane, 4 codes per dword (byte i of
//     kNf4LoQ = low byte of code 4Q+i), so one v_perm_b32 looks up 4 codes of one half
//     of the table at once.
constexpr uint32_t kNf4Lo0 = 0x52339200u;
constexpr uint32_t kNf4Lo1 = 0x00D4EA8Du;
constexpr uint32_t kNf4Lo2 = 0x68E02618u;
constexpr uint32_t kNf4Lo3 = 0x00C9800Du;
constexpr uint32_t kNf4Hi0 = 0xB6B8B9BCu;
constexpr uint32_t kNf4Hi1 = 0x00ADB1B4u;
constexpr uint32_t kNf4Hi2 = 0x3533312Du;
constexpr uint32_t kNf4Hi3 = 0x3C393837u;

// (2) Quantise thresholds: for the float32 codebook values C[j] (bit patterns
//     bf800000 bf3239b1 bf066b30 beca32a0 be91a24d be3d353f bdba7871 00000000
//     3da2faff 3e24cae3 3e7c04dd 3ead033a 3ee1a4b8 3f1007ab 3f3913b3 3f800000),
//     kNf4Up[j] is the smallest float32 strictly above the exact midpoint
//     (C[j] + C[j+1]) / 2.  For a float32 n, "n is nearer C[j+1], or tied and not
//     lower" reduces to n >= kNf4Up[j], so code = #{j : n >= kNf4Up[j]} is the nearest
//     code with exact ties going to the lower code.
__device__ __constant__ const uint32_t kNf4Up[15] = {
    0xBF591CD8u, 0xBF1C5270u, 0xBEEB847Fu, 0xBEADEA76u, 0xBE703CECu,
    0xBE0D38BBu, 0xBD3A7870u, 0x3D22FB00u, 0x3DF64863u, 0x3E5067E1u,
    0x3E9582D5u, 0x3EC753FAu, 0x3F006D04u, 0x3F248DB0u, 0x3F5C89DAu};

// Order in which nf4_decode8 leaves the 8 elements of a packed dword in its 4 output
// registers (two fp16 per register): slot i holds element kNf4SlotElem[i].  Activation
// operands are stored with the same order inside every aligned group of 8 elements so
// the MFMA k-slots of both operands line up.
//   slot:    0 1 2 3 4 5 6 7
//   element: 0 2 4 6 1 3 5 7
// Inverse (element e lives in slot kNf4ElemSlot[e]): 0 4 1 5 2 6 3 7.
__host__ __device__ constexpr int nf4_elem_slot(int e) { return (e >> 1) | ((e & 1) << 2); }

// Position of activation column j inside its row, in the k-slot order of the weight
// format (NF4 decodes 8 elements in slot order, MXFP4 in natural order).
template <int FMT>
__device__ __forceinline__ int64_t act_pos(int64_t j) {
  if (FMT == 0) return (j & ~int64_t(7)) | nf4_elem_slot(int(j & 7));
  return j;
}

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// (3) LDS decode table: for each packed byte value v, the fp16 pair (C[v >> 4], C[v & 15])
//     (element 2b, the high nibble, in the low half), with one private copy per lane: the
//     word for (v, lane l) sits at byte v * 256 + l * 4, so lane l always reads LDS bank l
//     and the 64 lookups of a wave never conflict.  64 KB.
constexpr int kNf4LutBytes = 256 * 64 * 4;

// Decode one packed NF4 dword (8 codes) through the LDS table to 8 fp16 codebook values in
// element order: out[b] = (element 2b, element 2b+1).  lanebase = lane * 4.  One v_perm
// builds each lookup address (byte value << 8 | lanebase).
__device__ __forceinline__ void nf4_lut_decode8(const uint8_t* lut, uint32_t lanebase, uint32_t w,
                                                uint32_t out[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t addr = perm(w, lanebase, 0x0C0C0400u + (uint32_t(b) << 8));
    out[b] = *reinterpret_cast<const uint32_t*>(lut + addr);
  }
}

// Bitfield select: bits of a where mask is 1, bits of b elsewhere (v_bfi_b32).
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) {
  return (mask & a) | (~mask & b);
}

// Decode one packed NF4 dword (8 codes, element 2b in the high nibble of byte b, 2b+1 in
// the low nibble) to 8 fp16 codebook values, in slot order (see kNf4SlotElem).
__device__ __forceinline__ void nf4_decode8(uint32_t w, uint32_t out[4]) {
  const uint32_t s_odd = w & 0x07070707u;              // low nibbles: elements 1,3,5,7
  const uint32_t s_even = (w >> 4) & 0x07070707u;      // high nibbles: elements 0,2,4,6
  // 0xFF in every byte whose code is >= 8: selector 0x0c gives 0x00, 0x0d gives 0xFF.
  const uint32_t m_odd = perm(0u, 0u, ((w >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
  const uint32_t m_even = perm(0u, 0u, ((w >> 7) & 0x01010101u) | 0x0C0C0C0Cu);
  const uint32_t lo_odd = bfi(m_odd, perm(kNf4Lo3, kNf4Lo2, s_odd), perm(kNf4Lo1, kNf4Lo0, s_odd));
  const uint32_t hi_odd = bfi(m_odd, perm(kNf4Hi3, kNf4Hi2, s_odd), perm(kNf4Hi1, kNf4Hi0, s_odd));
  const uint32_t lo_even = bfi(m_even, perm(kNf4Lo3, kNf4Lo2, s_even), perm(kNf4Lo1, kNf4Lo0, s_even));
  const uint32_t hi_even = bfi(m_even, perm(kNf4Hi3, kNf4Hi2, s_even), perm(kNf4Hi1, kNf4Hi0, s_even));
  // interleave low/high byte planes into fp16 pairs
  out[0] = perm(hi_even, lo_even, 0x05010400u);  // elements 0, 2
  out[1] = perm(hi_even, lo_even, 0x07030602u);  // elements 4, 6
  out[2] = perm(hi_odd, lo_odd, 0x05010400u);    // elements 1, 3
  out[3] = perm(hi_odd, lo_odd, 0x07030602u);    // elements 5, 7
}

// Fill the table of (3) at `lut` (kNf4LutBytes of LDS) with `nthreads` threads of the
// workgroup (nthreads divides 256 * 16); visible to other waves after the next barrier.  The
// pair of byte value v comes from the register decode of a dword whose byte 0 is v (element 0
// = high nibble in the low half of out[0], element 1 = low nibble in the low half of out[2]),
// so the fill makes no memory access and can run while a kernel's first loads are in flight.
__device__ __forceinline__ void nf4_lut_fill(uint8_t* lut, int tid, int nthreads) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  for (int c = tid; c < 256 * 16; c += nthreads) {  // 16-byte chunks: value c / 16
    uint32_t d[4];
    nf4_decode8(uint32_t(c >> 4), d);
    const uint32_t pair = (d[0] & 0xFFFFu) | (d[2] << 16);
    *reinterpret_cast<v4*>(lut + 16 * c) = v4{pair, pair, pair, pair};
  }
}

// NF4 block scales enter the fp16 decode multiplied by 2^8, and every fp32 product sum over
// such weights is multiplied by 2^-8 before it is used (both exact powers of two).  The decoded
// operand fp16(C) * fp16(absmax * 2^8) then stays an fp16 normal number for every nonzero code
// (smallest |C| = 0.0796) while 2^-18 <= absmax <= 255: the window of real weight scales, down to
// weights 2^-12 below N(0, 0.02), instead of [2^-10, 65504] without the shift.
constexpr float kNf4ScaleUp = 256.0f;
constexpr float kNf4ScaleDown = 1.0f / 256.0f;

// Multiply two packed fp16 by the same fp16 scale (v_pk_mul_f16).
__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t v, f16x2 s) {
  f16x2 r = __builtin_bit_cast(f16x2, v) * s;
  return __builtin_bit_cast(uint32_t, r);
}

// Decode one MXFP4 dword (8 e2m1 codes, element 2b in the low nibble of byte b) to 8
// fp16 values times `scale` (a power of two), natural element order.
__device__ __forceinline__ void mxfp4_decode8(uint32_t w, float scale, uint32_t out[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3));
}

// e8m0 byte -> float32 power of two 2^(b-127) (b = 0 gives 2^-127, a float32 subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(b << 23);
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane i's bytes
// land at lds_wave_base + 16 * i.  lds_wave_base must be the same for the whole wave.  The
// builtin exists only for the gfx950 device pass; the host pass never runs this body.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_wave_base, 16, 0, 0);
#endif
}

// s_waitcnt immediate: vmcnt = vm (0..63), expcnt = 7 (no wait), lgkmcnt = 0.
__host__ __device__ constexpr int waitcnt_vm_lgkm0(int vm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4);
}

// Raw buffer resource over `bytes` bytes at `base` (no stride): buffer loads take a 32-bit
// per-lane byte offset, and a load entirely past `bytes` returns zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// Direct buffer -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane i's bytes
// (from byte offset voff of the buffer) land at lds_wave_base + 16 * i.  Unlike the FLAT form
// (global_load_lds), a copy of this kind in flight leaves the compiler's LDS-read waits exact.
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t res, uint32_t voff,
                                              void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_void*)lds_wave_base, 16, int(voff), 0, 0, 0);
#endif
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// SiLU(g) * u in fp32 with the hardware exp and reciprocal (the result is stored as fp16).
// For very negative g, exp(-g) overflows to inf and the reciprocal gives 0 (SiLU -> -0).
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Clamped GLU of the MXFP4 family's expert variant: the gate clamped from above at 7, the up
// input to [-7, 7], gate * sigmoid(1.702 * gate) * (up + 1).
__device__ __forceinline__ float clamped_glu(float g, float u) {
  const float gc = fminf(g, 7.0f);
  const float uc = fminf(fmaxf(u, -7.0f), 7.0f);
  return gc * __builtin_amdgcn_rcpf(1.0f + __expf(-1.702f * gc)) * (uc + 1.0f);
}

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

}  // namespace e4b
