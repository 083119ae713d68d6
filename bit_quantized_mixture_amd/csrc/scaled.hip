// MXFP4 gate_up GEMM on gfx950's block-scaled matrix instruction
// (v_mfma_scale_f32_32x32x64_f8f6f4): the released e2m1 bytes and e8m0 scales of the weights
// go to the matrix unit as they are, with no decode (grouped-nf4-gemm 0.25.0 project
// description, opening section: MXFP4 on a checkpoint's exact released bytes;
// experts4bit-qlora 0.35.0 project description, Scope: MXFP4 experts).
//
// The instruction multiplies fp8/fp6/fp4 operands.  The bf16 activations are carried exactly
// as two fp8 e4m3 parts under one e8m0 scale per 32 elements: with the scale 2^s chosen so the
// block's largest magnitude lies in [128, 256), hi = e4m3(x / 2^s) keeps the top 4 of bf16's 8
// significant bits and lo = e4m3(x / 2^s - hi) the rest (exact while lo is at least e4m3's
// smallest subnormal 2^-9; smaller remainders, of elements below 2^-9 of the block's maximum,
// are rounded to 2^-10 * 2^s).  Each product then takes two instructions (hi, lo) whose
// products are exact and accumulate in fp32.
//
// Operand layout of the 32x32x64 instruction (checked on the device): for lane l, row / column
// l % 32 and lane half h = l / 32, the fp4 operand holds K [32h, 32h + 32) (16 bytes, low
// nibble first: one released MXFP4 block) and the fp8 operand holds K [16h, 16h + 16) in its
// bytes 0-15 and K [32 + 16h, 32 + 16h + 16) in bytes 16-31; the scale of K block b is taken
// from lane row + 32b.  The activation rows are therefore stored per 64-wide K step as 128
// bytes: hi for half 0 (K 0-15, 32-47), hi for half 1 (K 16-31, 48-63), then lo likewise.
#include <type_traits>

#include "e4b_device.h"
#include "e4b_internal.h"

namespace e4b {

__host__ __device__ int64_t scale_pitch(int64_t K) { return (K / 32 + 7) / 8 * 8; }

namespace {

// e4m3 (OCP, bias 7, no infinities, largest 448) code of a float32 v with |v| <= 448,
// round to nearest even; subnormals below 2^-6 in steps of 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sgn = (b >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a < 0.015625f) {  // 2^-6: subnormal e4m3 m * 2^-9, m in 0..8
    const uint32_t m = uint32_t(__builtin_rintf(a * 512.0f));  // rint: ties to even
    return sgn | (m == 8 ? 0x08u : m);                         // 8 * 2^-9 = 2^-6, exponent field 1
  }
  uint32_t u = __float_as_uint(a);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // round the mantissa to 3 bits
  const uint32_t e = (u >> 23) - 127 + 7;
  return sgn | (e << 3) | ((u >> 20) & 7u);
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const float s = (c & 0x80u) ? -1.0f : 1.0f;
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return s * float(m) * 0.001953125f;  // 2^-9
  return s * __uint_as_float(((e - 7 + 127) << 23) | (m << 20));
}

}  // namespace

// x bf16 [T, K] -> a8 [T, 2K] bytes (per 64-wide K step: hi half 0, hi half 1, lo half 0, lo
// half 1, 32 bytes each, in the operand order above) and asc [T, scale_pitch(K)] e8m0 scale
// bytes (rows padded to a multiple of 8 bytes).  One thread per 32-element block.
__global__ void __launch_bounds__(256) convert_x_scaled_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                               int64_t K, uint8_t* __restrict__ a8,
                                                               uint8_t* __restrict__ asc) {
  const int64_t nblk = T * (K / 32);
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < nblk; q += stride) {
    const int64_t t = q / (K / 32), b = q - t * (K / 32);
    const u32x4* src = reinterpret_cast<const u32x4*>(x + t * K + 32 * b);
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 raw = src[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * c + 2 * i] = __uint_as_float(raw[i] << 16);
        v[8 * c + 2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
        amax = fmaxf(amax, fmaxf(fabsf(v[8 * c + 2 * i]), fabsf(v[8 * c + 2 * i + 1])));
      }
    }
    // 2^s with amax / 2^s in [128, 256): s = floor(log2 amax) - 7, in the e8m0 range
    int s = amax > 0.0f ? int((__float_as_uint(amax) >> 23) & 255u) - 127 - 7 : -127;
    if (amax > 0.0f && ((__float_as_uint(amax) >> 23) & 255u) == 0) s = -127;  // subnormal block
    s = s < -127 ? -127 : (s > 127 ? 127 : s);
    const float inv = __builtin_ldexpf(1.0f, -s);
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) hi[w] = lo[w] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float qv = v[i] * inv;  // exact: a power of two
      const uint32_t ch = e4m3_rne(qv);
      const uint32_t cl = e4m3_rne(qv - e4m3_value(ch));
      hi[i >> 2] |= ch << (8 * (i & 3));
      lo[i >> 2] |= cl << (8 * (i & 3));
    }
    // block b covers K [32b, 32b + 32) of its step (b & 1): its first 16 elements belong to
    // lane half 0 if b is even (K 0-15 of the step) else half 1's second part, and so on
    uint8_t* row = a8 + t * (2 * K) + 128 * (b >> 1);
    const int p = int(b & 1);  // 0: K 0-31 of the step, 1: K 32-63
    // elements 0-15 of the block: K 32p + [0,16) -> half 0, bytes 16p + [0,16)
    // elements 16-31:             K 32p + [16,32) -> half 1, bytes 32 + 16p + [0,16)
    *reinterpret_cast<u32x4*>(row + 16 * p) = u32x4{hi[0], hi[1], hi[2], hi[3]};
    *reinterpret_cast<u32x4*>(row + 32 + 16 * p) = u32x4{hi[4], hi[5], hi[6], hi[7]};
    *reinterpret_cast<u32x4*>(row + 64 + 16 * p) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *reinterpret_cast<u32x4*>(row + 96 + 16 * p) = u32x4{lo[4], lo[5], lo[6], lo[7]};
    asc[t * scale_pitch(K) + b] = uint8_t(s + 127);
  }
}

namespace {

struct ScaledArgs {
  const uint8_t* a8;       // [T, 2K] activation parts (see convert_x_scaled_kernel)
  const uint8_t* asc;      // [T, K/32] activation scales
  const uint8_t* wq;       // [E, N, K/32, 16] e2m1 blocks
  const uint8_t* wsc;      // [E, N, K/32] e8m0
  const int32_t* tiles;    // [max_mtiles, 4]: expert, first sorted row, rows, 0
  const int32_t* n_mtiles;
  const int32_t* slots;    // sorted slots [S]
  _Float16* h;             // [S, I] out
  int64_t K, N, I, T;
  int32_t k_top, n_ntiles;
  const float* bias;       // nullable [E, N]
  int32_t clamped_glu, interleaved;
};

constexpr int kRowBytes = 128;  // activation bytes per row per 64-wide K step

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i cat8(u32x4 a, u32x4 b) {
  return v8i{int(a[0]), int(a[1]), int(a[2]), int(a[3]), int(b[0]), int(b[1]), int(b[2]), int(b[3])};
}

// One workgroup: BM routed rows of one expert x WAVES * 32 gate columns and the matching up
// columns.  Each wave owns all BM rows x (32 gate + 32 up) weight rows; accumulators in
// registers.  Activations come through a 4-stage LDS ring filled by direct buffer->LDS copies
// (a row's 16-byte chunk c sits at position c ^ ((row >> 1) & 7): the 16 rows of a read phase
// then cover all 64 banks); weights and scales come straight into registers, two steps ahead.
template <int BM, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) moe_gemm_scaled_kernel(ScaledArgs p) {
  constexpr int ST = 4;
  constexpr int RB = BM / 32;
  constexpr int ROWS_W = BM / WAVES;  // tile rows copied by this wave each step
  constexpr int NLD = ROWS_W / 8;     // copy instructions per wave per step (8 rows each)
  static_assert(ROWS_W % 8 == 0, "copy row groups");
  __shared__ __attribute__((aligned(16))) uint8_t ring[ST * BM * kRowBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int nt = blockIdx.x % p.n_ntiles;
  const int mt = blockIdx.x / p.n_ntiles;
  if (mt >= *p.n_mtiles) return;
  const int e = p.tiles[4 * mt], row0 = p.tiles[4 * mt + 1], rows = p.tiles[4 * mt + 2];
  const int nk = int(p.K / 64);
  const uint32_t rowb = uint32_t(p.K / 2);   // packed bytes per weight row
  const uint32_t rows_c = uint32_t(p.K / 32);  // scale bytes per row

  // ---- this lane's weight rows: fragment 0 = gate column j, 1 = its up column
  const int64_t j = int64_t(nt) * (WAVES * 32) + wave * 32 + col;
  const bool jvalid = j < p.I;
  const int64_t jc = jvalid ? j : p.I - 1;
  const int64_t nrow[2] = {p.interleaved ? 2 * jc : jc, p.interleaved ? 2 * jc + 1 : p.I + jc};
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(p.wq + int64_t(e) * p.N * rowb, uint32_t(p.N * rowb));
  const __amdgpu_buffer_rsrc_t sres = buffer_rsrc(p.wsc + int64_t(e) * p.N * rows_c, uint32_t(p.N * rows_c));
  uint32_t woff[2], soff[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    woff[f] = uint32_t(nrow[f]) * rowb + 16 * half;
    soff[f] = uint32_t(nrow[f]) * rows_c + half;
  }
  // ---- activation rows: scale offsets of this lane's row in each row block, and the copy
  // sources (lane i of a copy fills position i & 7 of tile row 8jj + i / 8 of this wave)
  const uint32_t apitch = uint32_t(scale_pitch(p.K));
  const __amdgpu_buffer_rsrc_t asres = buffer_rsrc(p.asc, uint32_t(p.T * apitch));
  const __amdgpu_buffer_rsrc_t ares = buffer_rsrc(p.a8, uint32_t(p.T * 2 * p.K));
  uint32_t asoff[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int m = 32 * rb + col;
    const int mm = m < rows ? m : rows - 1;
    asoff[rb] = uint32_t(p.slots[row0 + mm] / p.k_top) * apitch + half;
  }
  uint32_t aoff[NLD];
#pragma unroll
  for (int jj = 0; jj < NLD; ++jj) {
    const int m = wave * ROWS_W + 8 * jj + (lane >> 3);
    const int mm = m < rows ? m : rows - 1;
    const int c = (lane & 7) ^ ((m >> 1) & 7);
    aoff[jj] = uint32_t(p.slots[row0 + mm] / p.k_top) * uint32_t(2 * p.K) + 16 * c;
  }

  auto stage_a = [&](int kb) {
    const int kc = kb < nk ? kb : nk - 1;
    uint8_t* dst = ring + (kb % ST) * (BM * kRowBytes) + wave * ROWS_W * kRowBytes;
#pragma unroll
    for (int jj = 0; jj < NLD; ++jj)
      lds_dma16_buf(ares, aoff[jj] + uint32_t(kRowBytes * kc), dst + 8 * jj * kRowBytes);
  };
  // loads of step kb: the weights (16 bytes: block 2 kb + half of this lane's row) and the
  // scale bytes of that block for the weight rows and the activation rows (byte loads: the
  // packed scale rows are only 2-byte aligned)
  struct StepRegs {
    u32x4 w[2];
    uint32_t ws[2];
    uint32_t as[RB];
  };
  auto issue = [&](int kb, StepRegs& R) {
    const int kc = kb < nk ? kb : nk - 1;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      R.w[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, woff[f], 32 * kc, 0));
      R.ws[f] = __builtin_amdgcn_raw_buffer_load_b8(sres, soff[f], 2 * kc, 0);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) R.as[rb] = __builtin_amdgcn_raw_buffer_load_b8(asres, asoff[rb], 2 * kc, 0);
  };
  constexpr int OPS = 4 + RB;  // register loads per step

  f32x16 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb][0] = acc[rb][1] = f32x16{};

  // the fp8 operand of row block rb, part (0 hi, 1 lo), from ring buffer `buf`
  auto afrag = [&](const uint8_t* buf, int rb, int part) {
    const int m = 32 * rb + col;
    const uint8_t* rowp = buf + m * kRowBytes;
    const int c0 = 4 * part + 2 * half;
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(rowp + 16 * (c0 ^ ((m >> 1) & 7)));
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(rowp + 16 * ((c0 + 1) ^ ((m >> 1) & 7)));
    return cat8(x0, x1);
  };
  auto compute = [&](int kb, const StepRegs& R) {
    const uint8_t* buf = ring + (kb % ST) * (BM * kRowBytes);
    v8i bw[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) bw[f] = cat8(R.w[f], u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int part = 0; part < 2; ++part)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const v8i a = afrag(buf, rb, part);
#pragma unroll
        for (int f = 0; f < 2; ++f)
          acc[rb][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bw[f], acc[rb][f], 0, 4, 0,
                                                                       int(R.as[rb]), 0, int(R.ws[f]));
      }
  };

  // ---- pipeline.  Step kb: wait for its copies (issued ST - 1 steps earlier) and for every
  // wave to be done with the buffer of step kb - 1, copy step kb + ST - 1 into that buffer,
  // load the registers of step kb + 2, then compute step kb.  After the copies of step kb at
  // least (ST - 2) steps of copies and register loads were issued, so waiting until at most
  // that many loads are in flight covers them.
  constexpr int kWait = (ST - 2) * (NLD + OPS);
  static_assert(kWait < 64, "vmcnt range");
  StepRegs R0, R1, R2;
  stage_a(0);
  issue(0, R0);
  stage_a(1);
  issue(1, R1);
  stage_a(2);
  auto step = [&](int kb, const StepRegs& cur, StepRegs& ahead) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kWait));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    stage_a(kb + ST - 1);
    issue(kb + 2, ahead);
    compute(kb, cur);
  };
  for (int kb = 0; kb < nk; kb += 3) {
    step(kb, R0, R2);
    if (kb + 1 >= nk) break;
    step(kb + 1, R1, R0);
    if (kb + 2 >= nk) break;
    step(kb + 2, R2, R1);
  }
  // the copies issued past the last step must land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  if (!jvalid) return;

  // ---- epilogue: element r of a 32x32 block is row 8 (r / 4) + 4 half + r % 4, column col
  const float bg = p.bias ? p.bias[int64_t(e) * p.N + nrow[0]] : 0.0f;
  const float bu = p.bias ? p.bias[int64_t(e) * p.N + nrow[1]] : 0.0f;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
      if (row < rows) {
        const float g = acc[rb][0][r] + bg;
        const float u = acc[rb][1][r] + bu;
        const float hv = p.clamped_glu ? clamped_glu(g, u) : swiglu(g, u);
        p.h[int64_t(row0 + row) * p.I + j] = (_Float16)hv;
      }
    }
  }
}

}  // namespace

// MXFP4 gate_up on the scaled instruction: activation parts, then the main tiles (128 rows),
// then the streaming kernel over the tail tiles (with the fp16 activations convert_x wrote).
hipError_t launch_gate_up_scaled(const MoeLaunch& L, hipStream_t stream) {
  const int64_t nblk = L.T * (L.H / 32);
  int64_t g = (nblk + 255) / 256;
  if (g > 1 << 20) g = 1 << 20;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(convert_x_scaled_kernel, dim3(unsigned(g)), dim3(256), 0, stream, L.x, L.T, L.H,
                     L.x8, L.xsc);
  ScaledArgs a{};
  a.a8 = L.x8;
  a.asc = L.xsc;
  a.wq = L.w_gu;
  a.wsc = reinterpret_cast<const uint8_t*>(L.s_gu);
  a.tiles = L.tiles;
  a.n_mtiles = L.n_mtiles + 2;  // gate_up main tiles (regular + absorbed tails)
  a.slots = L.slots;
  a.h = L.h;
  a.K = L.H;
  a.N = 2 * L.I;
  a.I = L.I;
  a.T = L.T;
  a.k_top = L.k;
  a.bias = L.b_gu;
  a.clamped_glu = L.clamped_glu;
  a.interleaved = L.interleaved;
  constexpr int kWavesS = 4;
  a.n_ntiles = int((L.I + kWavesS * 32 - 1) / (kWavesS * 32));
  // 128-row tiles: with 256 rows the accumulators and the operand registers do not fit
  if (L.cfg.bm != 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL((moe_gemm_scaled_kernel<128, kWavesS>), dim3(unsigned(L.max_mtiles * a.n_ntiles)),
                     dim3(kWavesS * 64), 0, stream, a);
  if (L.max_stiles > 0) return launch_gemv_tails(L, stream, 0);
  return hipGetLastError();
}

}  // namespace e4b
