// int4-b32 decode GEMV over routed experts with exact integer accumulation, its round-to-nearest
// packer and the per-token int8 activation quantiser.
//
// grouped-nf4-gemm 0.25.0 project description, opening section: the package carries an int4-b32
// decode GEMV and a packer for it.  Cerin Amroth "ML systems" index, Solutions: a single-token
// int4-b32 decode GEMV over routed MoE experts with exact integer accumulation.  The pages fix
// nothing else; the format read here: signed 4-bit codes (two's complement, even element in the
// low nibble), one fp16 scale s = fp16(absmax / 7) per 32 weights of a row; activations
// quantised per token to int8 with s_x = absmax / 127; y[n] = s_x * sum_b s[n, b] * I_b with
// I_b the exact int32 dot product of block b's codes and the token's int8 codes.
//
// GEMV layout (both kernels): a workgroup of 8 waves owns one tile of <= 16 routed rows of one
// expert (their tokens' int8 rows staged in LDS) and 128 / ksplit weight rows; the K axis is
// cut into ksplit parts, one per wave of a row group, summed through LDS at the end in a fixed
// order.
//
// int4_gemv_mfma_kernel (tiles of 4 or more routed rows).  Lane (r = lane % 16, g = lane / 16) of a wave streams the 16 bytes (one 32-weight block) of block
// 4c + g of chunk c of row r, so a wave's load covers 64 contiguous bytes of each of 16 rows.
// A 4 x 4 transpose across the four 16-lane groups (two permlane32 and two permlane16 swaps)
// then leaves register j of lane (r, g) with dword g of block 4c + j: the codes of row r at
// elements 8g .. 8g + 7 of that block, which is how the int8 MFMA 16 x 16 x 32 takes one
// 32-wide block from 64 lanes.  Each code enters the MFMA as an int8 holding 16 q (the nibble
// at the top of its byte: one shift and one mask per 4 codes), each token's activations in
// their stored order, every group of 8 as 0,2,4,6,1,3,5,7 (the low nibbles of a dword, then
// the high ones), so one MFMA per block gives
//   D[t][r] = 16 * I_b(row r, token t)   exactly (|D| <= 16 * 8 * 127 * 32 < 2^24),
// and the block adds D * (s[r, b] / 16) (both factors exact in fp32, one rounding in the FMA,
// as s * I_b) into lane (r, g)'s fp32 sums of tokens 4g .. 4g + 3.
//
// int4_gemv_dot4_kernel (a batch of 1 to 3 tokens, where most of the MFMA's 16 token rows would
// be padding).  Lane (r = lane / 4, g = lane % 4) streams block 4c + g of row r and takes, for
// each token of the tile, v_dot4 products of its codes read as u = q + 8 (the nibble XOR 8, a
// byte-wise mask gives the operand); the block sum of the token's codes times 8 is subtracted
// back (exact):  I_b = sum u * x - 8 * sum x.  The 4 block lanes of a row are added at the end.
#include "e4b_device.h"
#include "e4b_internal.h"

namespace e4b {

namespace {

constexpr int kI4Block = 32;
constexpr int kGvWaves = 8;
constexpr int kGvTok = 16;  // routed rows per tile

// ---- packer: lane per 8 weights (one 16-byte load), 4 lanes per block.
__global__ void __launch_bounds__(256) pack_int4_kernel(const uint16_t* __restrict__ w,
                                                        uint8_t* __restrict__ packed,
                                                        uint16_t* __restrict__ scales,
                                                        int64_t n_chunks) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  // n_chunks and the stride are multiples of 4, so the 4 lanes of a block stay together
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
    a = fmaxf(a, __shfl_xor(a, 1, 4));
    a = fmaxf(a, __shfl_xor(a, 2, 4));
    const _Float16 s16 = (_Float16)__fdiv_rn(a, 7.0f);  // correctly rounded, then RNE to fp16
    const float s = (float)s16;
    uint32_t word = 0;
    if (s > 0.f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r = fminf(fmaxf(rintf(__fdiv_rn(v[i], s)), -8.f), 7.f);
        word |= (uint32_t(int(r)) & 0xFu) << (4 * i);  // element 2p: low nibble of byte p
      }
    }
    reinterpret_cast<uint32_t*>(packed)[q] = word;
    if ((q & 3) == 0) scales[q >> 2] = __builtin_bit_cast(uint16_t, s16);
  }
}

// Tile list for the GEMV (run by one extra workgroup of the quantiser launch): for each expert
// e, tiles of <= bm consecutive sorted rows: (e, first row, rows, 0), experts in order; the
// count goes to n_tiles[0].
__device__ void int4_build_tiles(const int32_t* __restrict__ offsets, int E, int bm,
                                 int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ int32_t scan[256];
  const int tid = threadIdx.x;
  int run = 0;
  for (int base = 0; base < E; base += 256) {
    const int e = base + tid;
    const int start = e < E ? offsets[e] : 0;
    const int cnt = e < E ? offsets[e + 1] - start : 0;
    const int nt = (cnt + bm - 1) / bm;
    scan[tid] = nt;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {  // inclusive scan (Hillis-Steele)
      const int v = tid >= d ? scan[tid - d] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int first = run + scan[tid] - nt;
    const int total = scan[255];
    for (int i = 0; i < nt; ++i) {
      int32_t* t = tiles + 4 * int64_t(first + i);
      t[0] = e;
      t[1] = start + i * bm;
      t[2] = min(bm, cnt - i * bm);
      t[3] = 0;
    }
    run += total;
    __syncthreads();  // scan[] is rewritten by the next pass
  }
  if (tid == 0) n_tiles[0] = run;
}

// Quantise one activation row xr[0..K) with the NT threads of a workgroup: s = absmax / 127
// (correctly rounded), code = clamp(rint(v / s), -127, 127) (0 for an all-zero row), written to
// q[0..K); PERM stores each group of 8 codes in the order 0,2,4,6,1,3,5,7 and writes the block
// sums of the codes to xs[0..K/32).  Returns s in every thread.  red: NT/64 floats of LDS; the
// leading barrier keeps a second call from overwriting them before every thread has read them.
template <int NT, bool PERM>
__device__ float quant_row(const uint16_t* __restrict__ xr, int64_t K, int tid, float* red,
                           int8_t* q, int32_t* xs) {
  constexpr int NW = NT / 64;
  const int ngroups = int(K >> 3);
  float a = 0.f;
  for (int g = tid; g < ngroups; g += NT) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(xr + 8 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a = fmaxf(a, fmaxf(fabsf(__uint_as_float(raw[i] << 16)),
                         fabsf(__uint_as_float(raw[i] & 0xFFFF0000u))));
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) a = fmaxf(a, __shfl_xor(a, m));
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = a;
  __syncthreads();
  a = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) a = fmaxf(a, red[w]);
  const float s = __fdiv_rn(a, 127.0f);
  // ngroups is a multiple of 4 and the stride NT, so the 4 lanes of a block stay together
  for (int g = tid; g < ngroups; g += NT) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(xr + 8 * g);
    int c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = __uint_as_float(i & 1 ? raw[i >> 1] & 0xFFFF0000u : raw[i >> 1] << 16);
      const float r = s > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(v, s)), -127.f), 127.f) : 0.f;
      c[i] = int(r);
    }
    uint32_t lo, hi;
    if (PERM) {
      lo = (c[0] & 0xFF) | ((c[2] & 0xFF) << 8) | ((c[4] & 0xFF) << 16) | (uint32_t(c[6] & 0xFF) << 24);
      hi = (c[1] & 0xFF) | ((c[3] & 0xFF) << 8) | ((c[5] & 0xFF) << 16) | (uint32_t(c[7] & 0xFF) << 24);
    } else {
      lo = (c[0] & 0xFF) | ((c[1] & 0xFF) << 8) | ((c[2] & 0xFF) << 16) | (uint32_t(c[3] & 0xFF) << 24);
      hi = (c[4] & 0xFF) | ((c[5] & 0xFF) << 8) | ((c[6] & 0xFF) << 16) | (uint32_t(c[7] & 0xFF) << 24);
    }
    *reinterpret_cast<u32x2*>(q + 8 * g) = u32x2{lo, hi};
    if (PERM) {
      int sum = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += c[i];
      sum += __shfl_xor(sum, 1, 4);
      sum += __shfl_xor(sum, 2, 4);
      if ((g & 3) == 0) xs[g >> 2] = sum;
    }
  }
  return s;
}

// ---- activation quantiser: one workgroup per token (quant_row), and, with PERM, one more
// workgroup (blockIdx.x == T) that builds the GEMV's tile list.
template <bool PERM>
__global__ void __launch_bounds__(256) quant_act_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                        int8_t* __restrict__ q,
                                                        float* __restrict__ s_out,
                                                        int32_t* __restrict__ xs, int64_t T,
                                                        const int32_t* __restrict__ offsets, int E,
                                                        int bm, int32_t* __restrict__ tiles,
                                                        int32_t* __restrict__ n_tiles) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  if (PERM && t == T) {  // uniform
    int4_build_tiles(offsets, E, bm, tiles, n_tiles);
    return;
  }
  const float s = quant_row<256, PERM>(x + t * K, K, tid, red, q + t * K, PERM ? xs + t * (K >> 5) : nullptr);
  if (tid == 0) s_out[t] = s;
}

struct I4Args {
  const uint8_t* wq;        // [E, N, K/2]
  const uint16_t* sc;       // [E, N, K/32] fp16 bits
  const int8_t* qx;         // [T, K] int8, permuted groups
  const int32_t* xs;        // [T, K/32] block sums of qx (dot4 kernel)
  const float* sx;          // [T]
  const int32_t* slots;     // [S] sorted slots
  const int32_t* tiles;     // [max_tiles, 4]: expert, first sorted row, rows, 0
  const int32_t* n_tiles;
  float* out;               // [S, N] float32, sorted rows
  int64_t N, K;
  int32_t k, n_rblocks, tile_rows, ksplit;
  // fused dot4 launch only: bf16 activations [T, K] and the routing offsets [E + 1]
  const uint16_t* x;
  const int32_t* offsets;
  int32_t E;
};

// Activation rows in LDS are K + 16 bytes apart, so the 16 token rows of one MFMA operand
// read (same block, same lane group) fall in 16 different 16-byte bank groups.
constexpr int kActPad = 16;

__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

__global__ void __launch_bounds__(512) int4_gemv_mfma_kernel(I4Args p) {
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = int(blockIdx.x) % p.n_rblocks;
  const int it = int(blockIdx.x) / p.n_rblocks;
  if (it >= *p.n_tiles) return;  // uniform
  const int e = p.tiles[4 * it], row0 = p.tiles[4 * it + 1], ntok = p.tiles[4 * it + 2];
  const int64_t K = p.K;
  const int64_t pitch = K + kActPad;
  const int nb = int(K >> 5);  // blocks per row
  const int ks = p.ksplit, rows_wg = 16 * (kGvWaves / ks);
  int8_t* act = reinterpret_cast<int8_t*>(lds);                                  // [tile_rows][pitch]
  float* part = reinterpret_cast<float*>(lds + int64_t(p.tile_rows) * pitch);   // [rows_wg * ks][16]

  const int kq = wave % ks, rg = wave / ks;
  const int r = lane & 15, g = lane >> 4;
  const int rl = 16 * rg + r;                       // row inside the workgroup's block
  const int64_t n = int64_t(rb) * rows_wg + rl;
  const int nch = int(K >> 7);                      // 128-weight chunks per row
  const int c0 = (kq * nch) / ks, c1 = ((kq + 1) * nch) / ks;
  const uint32_t kb = uint32_t(K >> 1);
  const __amdgpu_buffer_rsrc_t wres =
      buffer_rsrc(p.wq + int64_t(e) * p.N * kb, uint32_t(p.N * kb));
  const __amdgpu_buffer_rsrc_t sres =
      buffer_rsrc(p.sc + int64_t(e) * p.N * nb, uint32_t(p.N * nb * 2));
  const uint32_t woff = uint32_t(n) * kb + 16u * g;
  const uint32_t soff = uint32_t(n) * uint32_t(nb) * 2u;
  // MFMA A operand: token row r of the tile (rows past the tile's count repeat its last row;
  // their sums are never stored), the 8 activation bytes of lane group g in a block
  const int8_t* arow = act + int64_t(r < ntok ? r : ntok - 1) * pitch + 8 * g;

  float acc[4] = {0.f, 0.f, 0.f, 0.f};  // tokens 4g .. 4g + 3 of row r

  // Chunks in groups of 4 with the next group's loads in flight (two register sets); loads
  // past the wave's last chunk repeat it (in bounds, never used).
  u32x4 wA[4], wB[4];
  u32x2 sA[4], sB[4];
  auto load4 = [&](int cb, u32x4 (&w)[4], u32x2 (&sv)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = cb + j < c1 ? cb + j : c1 - 1;
      w[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, woff, 64u * c, 0));
      sv[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(sres, soff, 8u * c, 0));
    }
  };
  auto compute = [&](const u32x4& wv, const u32x2& sv, int c) {
    uint32_t d[4] = {wv[0], wv[1], wv[2], wv[3]};
    swap32(d[0], d[2]);
    swap32(d[1], d[3]);
    swap16(d[0], d[1]);
    swap16(d[2], d[3]);
    i32x4 D[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = (d[j] << 4) & 0xF0F0F0F0u;  // elements 0,2,4,6 of the 8, times 16
      const uint32_t hi = d[j] & 0xF0F0F0F0u;         // elements 1,3,5,7, times 16
      const int64_t wop = int64_t((uint64_t(hi) << 32) | lo);
      const int64_t aop = *reinterpret_cast<const int64_t*>(arow + 32 * (4 * c + j));
      D[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, wop, i32x4{0, 0, 0, 0}, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t sh = uint16_t(j & 1 ? sv[j >> 1] >> 16 : sv[j >> 1] & 0xFFFFu);
      const float s16 = float(__builtin_bit_cast(_Float16, sh)) * 0.0625f;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(s16, float(D[j][i]), acc[i]);
    }
  };
  // the first weight loads go out before the activations are staged, so the two latencies
  // overlap
  if (c0 < c1) load4(c0, wA, sA);  // uniform
  // stage the tile's token rows (int8 codes)
  const int pieces = int(K >> 4);
  for (int i = tid; i < ntok * pieces; i += 512) {
    const int tt = i / pieces, c = i - tt * pieces;
    const int64_t tok = p.slots[row0 + tt] / p.k;
    *reinterpret_cast<u32x4*>(act + tt * pitch + 16 * c) =
        *reinterpret_cast<const u32x4*>(p.qx + tok * K + 16 * c);
  }
  __syncthreads();
  if (c0 < c1) {  // uniform
    for (int c = c0; c < c1; c += 8) {
      load4(c + 4, wB, sB);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c + j < c1) compute(wA[j], sA[j], c + j);
      load4(c + 8, wA, sA);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c + 4 + j < c1) compute(wB[j], sB[j], c + 4 + j);
    }
  }
  // the ksplit waves of a row group through LDS, in wave order
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (4 * g + i < ntok) part[(rl * ks + kq) * kGvTok + 4 * g + i] = acc[i];
  __syncthreads();
  for (int i = tid; i < rows_wg * ntok; i += 512) {
    const int tt = i / rows_wg, row = i - tt * rows_wg;
    float sum = 0.f;
    for (int q = 0; q < ks; ++q) sum += part[(row * ks + q) * kGvTok + tt];
    const int64_t tok = p.slots[row0 + tt] / p.k;
    p.out[int64_t(row0 + tt) * p.N + int64_t(rb) * rows_wg + row] = sum * p.sx[tok];
  }
}

// FUSED (batches of 1-3 tokens, E <= kFuseMaxE): no quantiser launch before the GEMV; each
// workgroup finds its tile from the routing offsets (the tiles int4_build_tiles would list, in
// the same order) and quantises its tile's token rows into LDS itself (quant_row, the
// quantiser's own arithmetic, so the codes are the same bits).
template <bool FUSED>
__global__ void __launch_bounds__(512) int4_gemv_dot4_kernel(I4Args p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ float red[kGvWaves];
  __shared__ int32_t s_cnt[kGvWaves];
  __shared__ int32_t s_tile[3];
  __shared__ float s_sx[kGvTok];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = int(blockIdx.x) % p.n_rblocks;
  const int it = int(blockIdx.x) / p.n_rblocks;
  int e, row0, ntok;
  if (FUSED) {
    // tile `it` of the expert-ordered list: expert e owns ceil(count_e / bm) tiles
    const int bm = p.tile_rows;
    if (tid == 0) s_tile[0] = -1;
    int run = 0;
    for (int base = 0; base < p.E; base += 512) {
      const int ee = base + tid;
      const int start = ee < p.E ? p.offsets[ee] : 0;
      const int cnt = ee < p.E ? p.offsets[ee + 1] - start : 0;
      const int nt = (cnt + bm - 1) / bm;
      int incl = nt;  // inclusive scan of nt over the wave
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (lane == 63) s_cnt[wave] = incl;
      __syncthreads();
      int pre = run, tot = 0;
#pragma unroll
      for (int w = 0; w < kGvWaves; ++w) {
        pre += w < wave ? s_cnt[w] : 0;
        tot += s_cnt[w];
      }
      const int first = pre + incl - nt;
      if (nt > 0 && it >= first && it < first + nt) {
        const int i = it - first;
        s_tile[0] = ee;
        s_tile[1] = start + i * bm;
        s_tile[2] = min(bm, cnt - i * bm);
      }
      run += tot;
      __syncthreads();  // s_cnt is rewritten by the next pass; s_tile is complete
      if (run > it) break;  // uniform
    }
    if (s_tile[0] < 0) return;  // uniform: past the tile count
    e = s_tile[0];
    row0 = s_tile[1];
    ntok = s_tile[2];
  } else {
    if (it >= *p.n_tiles) return;  // uniform
    e = p.tiles[4 * it];
    row0 = p.tiles[4 * it + 1];
    ntok = p.tiles[4 * it + 2];
  }
  const int64_t K = p.K;
  const int nb = int(K >> 5);  // blocks per row
  const int ks = p.ksplit, rows_wg = 16 * (kGvWaves / ks);
  int8_t* act = reinterpret_cast<int8_t*>(lds);                                // [tile_rows][K]
  int32_t* xsl = reinterpret_cast<int32_t*>(lds + int64_t(p.tile_rows) * K);   // [tile_rows][nb]
  float* part = reinterpret_cast<float*>(lds + int64_t(p.tile_rows) * K + int64_t(p.tile_rows) * nb * 4);

  const int kq = wave % ks, rg = wave / ks;
  const int r = lane >> 2, g = lane & 3;
  const int rl = 16 * rg + r;                       // row inside the workgroup's block
  const int64_t n = int64_t(rb) * rows_wg + rl;
  const int nch = int(K >> 7);                      // 128-weight chunks per row
  const int c0 = (kq * nch) / ks, c1 = ((kq + 1) * nch) / ks;
  const uint32_t kb = uint32_t(K >> 1);
  const __amdgpu_buffer_rsrc_t wres =
      buffer_rsrc(p.wq + int64_t(e) * p.N * kb, uint32_t(p.N * kb));
  const __amdgpu_buffer_rsrc_t sres =
      buffer_rsrc(p.sc + int64_t(e) * p.N * nb, uint32_t(p.N * nb * 2));
  const uint32_t woff = uint32_t(n) * kb + 16u * g;
  const uint32_t soff = (uint32_t(n) * uint32_t(nb) + g) * 2u;

  float acc[kGvTok];
#pragma unroll
  for (int tt = 0; tt < kGvTok; ++tt) acc[tt] = 0.f;

  // Chunks in groups of 4 with the next group's loads in flight (two register sets); loads
  // past the wave's last chunk repeat it (in bounds, never used).
  u32x4 wA[4], wB[4];
  uint32_t sA[4], sB[4];
  auto load4 = [&](int cb, u32x4 (&w)[4], uint32_t (&s)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = cb + j < c1 ? cb + j : c1 - 1;
      w[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, woff, 64u * c, 0));
      s[j] = __builtin_amdgcn_raw_buffer_load_b16(sres, soff, 8u * c, 0);
    }
  };
  auto compute = [&](const u32x4& wv, uint32_t sv, int c) {
    const int b = 4 * c + g;
    const float sf = float(__builtin_bit_cast(_Float16, uint16_t(sv)));
    uint32_t u[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      u[2 * d] = (wv[d] & 0x0F0F0F0Fu) ^ 0x08080808u;
      u[2 * d + 1] = ((wv[d] >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
    }
    const int8_t* ab = act + 32 * b;
#pragma unroll
    for (int tt = 0; tt < kGvTok; ++tt) {
      if (tt < ntok) {  // uniform
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(ab + tt * K);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(ab + tt * K + 16);
        int isum = -8 * xsl[tt * nb + b];
#pragma unroll
        for (int i = 0; i < 4; ++i) isum = __builtin_amdgcn_sdot4(int(u[i]), int(a0[i]), isum, false);
#pragma unroll
        for (int i = 0; i < 4; ++i) isum = __builtin_amdgcn_sdot4(int(u[4 + i]), int(a1[i]), isum, false);
        acc[tt] = fmaf(sf, float(isum), acc[tt]);
      }
    }
  };
  // the first weight loads go out before the activations are staged, so the two latencies
  // overlap
  if (c0 < c1) load4(c0, wA, sA);  // uniform
  // stage the tile's token rows (int8 codes and block sums)
  if (FUSED) {
    for (int tt = 0; tt < ntok; ++tt) {  // uniform
      const int64_t tok = p.slots[row0 + tt] / p.k;
      const float sv = quant_row<512, true>(p.x + tok * K, K, tid, red, act + tt * K, xsl + tt * nb);
      if (tid == 0) s_sx[tt] = sv;
    }
  } else {
    const int pieces = int(K >> 4);
    for (int i = tid; i < ntok * pieces; i += 512) {
      const int tt = i / pieces, c = i - tt * pieces;
      const int64_t tok = p.slots[row0 + tt] / p.k;
      *reinterpret_cast<u32x4*>(act + tt * K + 16 * c) =
          *reinterpret_cast<const u32x4*>(p.qx + tok * K + 16 * c);
    }
    for (int i = tid; i < ntok * nb; i += 512) {
      const int tt = i / nb, b = i - tt * nb;
      const int64_t tok = p.slots[row0 + tt] / p.k;
      xsl[tt * nb + b] = p.xs[tok * nb + b];
    }
  }
  __syncthreads();
  if (c0 < c1) {  // uniform
    for (int c = c0; c < c1; c += 8) {
      load4(c + 4, wB, sB);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c + j < c1) compute(wA[j], sA[j], c + j);
      load4(c + 8, wA, sA);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c + 4 + j < c1) compute(wB[j], sB[j], c + 4 + j);
    }
  }
  // the 4 block lanes of a row, then the ksplit waves of a row group through LDS
#pragma unroll
  for (int tt = 0; tt < kGvTok; ++tt) {
    acc[tt] += __shfl_xor(acc[tt], 1);
    acc[tt] += __shfl_xor(acc[tt], 2);
  }
  if (g == 0) {
#pragma unroll
    for (int tt = 0; tt < kGvTok; ++tt)
      if (tt < ntok) part[(rl * ks + kq) * kGvTok + tt] = acc[tt];
  }
  __syncthreads();
  for (int i = tid; i < rows_wg * ntok; i += 512) {
    const int tt = i / rows_wg, row = i - tt * rows_wg;
    float sum = 0.f;
    for (int q = 0; q < ks; ++q) sum += part[(row * ks + q) * kGvTok + tt];
    const float sx = FUSED ? s_sx[tt] : p.sx[p.slots[row0 + tt] / p.k];
    p.out[int64_t(row0 + tt) * p.N + int64_t(rb) * rows_wg + row] = sum * sx;
  }
}

}  // namespace

hipError_t launch_pack_int4(const uint16_t* w, int64_t n_elems, uint8_t* packed, uint16_t* scales,
                            hipStream_t stream) {
  const int64_t n_chunks = n_elems / 8;
  const int64_t want = (n_chunks + 255) / 256;
  const unsigned grid = unsigned(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_int4_kernel, dim3(grid), dim3(256), 0, stream, w, packed, scales, n_chunks);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, int64_t T, int64_t K, int8_t* q, float* s,
                            hipStream_t stream) {
  hipLaunchKernelGGL(quant_act_kernel<false>, dim3(unsigned(T)), dim3(256), 0, stream, x, K, q, s,
                     nullptr, T, nullptr, 0, 1, nullptr, nullptr);
  return hipGetLastError();
}

int int4_gemv_tile_rows(int64_t T) { return int(T < kGvTok ? T : kGvTok); }

int int4_gemv_ksplit(int64_t max_tiles, int64_t N, int64_t K) {
  // The smallest K split (with whole row blocks) that gives the chip at least 6 waves per CU
  // (the tile count is the host's upper bound), short of a split that would leave a wave fewer
  // than 4 chunks of 128 weights.  Measured per call against the earlier target of 8192 waves
  // (alternating runs on one box): one dense [14336, 4096] matrix at M = 1 16.3 against 20.0
  // us (split 2 instead of 8), the 128-expert gate_up stack at 4 tokens 24.5 against 38.9 us
  // (1 instead of 4); 1 and 64 tokens within noise.  Larger splits leave each wave one round
  // of loads and spend the time in the workgroup's cross-wave sum.
  const int64_t want = 6 * int64_t(cu_count());
  for (int ks = 1; ks <= 8; ks <<= 1) {
    const int64_t rows_wg = 16 * (kGvWaves / ks);
    if (N % rows_wg) continue;
    const int64_t waves = max_tiles * (N / rows_wg) * kGvWaves;
    if (waves >= want || ks == 8 || (K >> 7) < 4 * 2 * ks) return ks;
  }
  return 8;
}

// The MFMA kernel for tiles of at least kI4MfmaRows routed rows (a batch of that many tokens),
// the dot4 kernel below it.  Measured on the 128-expert decode layer's gate_up stack: at 64
// tokens (tiles of about 4 rows) 67 us against 76 us; at one token the MFMA kernel was no
// faster on the routed layer and 42 % slower on one dense matrix.
constexpr int kI4MfmaRows = 4;

bool int4_use_mfma(int64_t T) { return int4_gemv_tile_rows(T) >= kI4MfmaRows; }

size_t int4_gemv_lds_bytes(int64_t T, int64_t K) {
  const int64_t tr = int4_gemv_tile_rows(T);
  if (int4_use_mfma(T)) return size_t(tr * (K + kActPad) + 128 * kGvTok * 4);
  return size_t(tr * K + tr * (K >> 5) * 4 + 128 * kGvTok * 4);
}

// Batches the dot4 kernel takes (1-3 tokens) skip the quantiser launch when the expert count
// is small enough for every workgroup to scan the offsets itself.  Measured per call on one box
// (quantiser + GEMV launches against the fused launch, alternating runs): one dense [14336,
// 4096] matrix at M = 1 16.3 -> 14.3 us; the 128-expert gate_up stack at 1 / 2 / 3 tokens
// 15.9 / 16.1 / 19.6 -> 13.4 / 15.6 / 18.0 us.
constexpr int64_t kFuseMaxE = 4096;

hipError_t launch_int4_gemv(const Int4GemvLaunch& L, hipStream_t stream) {
  const int tr = int4_gemv_tile_rows(L.T);
  const bool fused = !int4_use_mfma(L.T) && L.E <= kFuseMaxE;
  hipError_t err = hipSuccess;
  if (!fused) {
    // one launch quantises the activations (T workgroups) and builds the tile list (one more)
    hipLaunchKernelGGL(quant_act_kernel<true>, dim3(unsigned(L.T + 1)), dim3(256), 0, stream, L.x, L.K,
                       L.qx, L.sx, L.xs, L.T, L.offsets, int(L.E), tr, L.tiles, L.n_tiles);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  I4Args a{};
  a.wq = L.wq;
  a.sc = L.sc;
  a.qx = L.qx;
  a.xs = L.xs;
  a.sx = L.sx;
  a.slots = L.slots;
  a.tiles = L.tiles;
  a.n_tiles = L.n_tiles;
  a.out = L.out;
  a.N = L.N;
  a.K = L.K;
  a.k = L.k;
  a.ksplit = int4_gemv_ksplit(L.max_tiles, L.N, L.K);
  a.n_rblocks = int(L.N / (16 * (kGvWaves / a.ksplit)));
  a.tile_rows = tr;
  a.x = L.x;
  a.offsets = L.offsets;
  a.E = int32_t(L.E);
  const size_t lds = int4_gemv_lds_bytes(L.T, L.K);
  const void* kern = int4_use_mfma(L.T) ? reinterpret_cast<const void*>(int4_gemv_mfma_kernel)
                     : fused            ? reinterpret_cast<const void*>(int4_gemv_dot4_kernel<true>)
                                        : reinterpret_cast<const void*>(int4_gemv_dot4_kernel<false>);
  if (lds > 64 * 1024) {
    err = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (err != hipSuccess) return err;
  }
  const unsigned grid = unsigned(L.max_tiles * a.n_rblocks);
  if (int4_use_mfma(L.T))
    hipLaunchKernelGGL(int4_gemv_mfma_kernel, dim3(grid), dim3(512), lds, stream, a);
  else if (fused)
    hipLaunchKernelGGL(int4_gemv_dot4_kernel<true>, dim3(grid), dim3(512), lds, stream, a);
  else
    hipLaunchKernelGGL(int4_gemv_dot4_kernel<false>, dim3(grid), dim3(512), lds, stream, a);
  return hipGetLastError();
}

}  // namespace e4b
