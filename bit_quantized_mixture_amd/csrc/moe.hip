// Grouped expert GEMMs of the MoE forward, computed on 4-bit packed weights.
//
// grouped-nf4-gemm 0.25.0 project description, opening section: one launch covers every
// active expert; codes are decoded through a table in registers, scaled per block,
// accumulated in fp32, and only the output is rounded to bf16; no dequantised weight copy
// exists.  bitsandbytes pull request #1984, Design: the expert is a SwiGLU MLP on the fused
// gate_up / down stacks.
//
// Pipeline (all on the caller's stream, no device->host read-back):
//   convert_x     x bf16 [T,H] -> fp16 (exact in fp16 range), k-slot order of the format
//   build_tiles   per expert, ceil(rows/BM) row tiles of the expert-major slot order
//   gemm<GU>      h[p, j] = silu(x_t . Wg[e,j]) * (x_t . Wu[e,j]) for the rows p of a tile
//   gemm<DN>      y[s, n] = topk_w[s] * (h[p] . Wd[e,n])   (s = slot of sorted row p)
//   combine       out[t] = sum_j y[t*k+j]  (fixed order)  -> fp32 and bf16 (RNE)
//
// Tile structure of gemm: a workgroup owns BM rows of one expert and WAVES*64 weight rows
// (GU: 32 gate + 32 matching up rows per wave, so SwiGLU is formed in registers).  Each
// wave owns all BM rows x 64 weight rows and keeps its accumulators in registers
// (v_mfma_f32_32x32x16_f16).  The activation tile (BM x 64 fp16) is staged through LDS,
// double-buffered, and shared by the waves; each lane streams its own weight row's packed
// bytes straight from HBM (16 bytes per 64-wide K step) and decodes them in registers.
#include "e4b_device.h"
#include "e4b_internal.h"

namespace e4b {

constexpr int kBK = 64;            // K per main-loop step: one NF4 block, two MXFP4 blocks
constexpr int kPitch = kBK + 8;    // LDS row pitch in fp16 (144 B): conflict-free 16 B reads

struct GemmArgs {
  const _Float16* a;       // GU: x16 [T, K]; DN: h [S, K]
  const uint8_t* wq;       // packed weights [E, N, K/2]
  const void* sc;          // NF4 float [E, N, K/64] | MXFP4 uint8 [E, N, K/32]
  const int32_t* tiles;    // [max_mtiles, 4]: expert, first sorted row, rows, 0
  const int32_t* n_mtiles;
  const int32_t* slots;    // sorted slots [S]
  const float* topk_w;     // [S]
  void* out;               // GU: h fp16 [S, I]; DN: y float [S, N]
  int64_t K;
  int64_t N;               // weight rows per expert (2I for GU, H for DN)
  int64_t I;
  int32_t k_top;
  int32_t n_ntiles;
};

// Position of h column j inside its row, in the k-slot order the down GEMM reads.
template <int FMT>
__device__ __forceinline__ int64_t act_pos(int64_t j) {
  if (FMT == 0) return (j & ~int64_t(7)) | nf4_elem_slot(int(j & 7));
  return j;
}

template <int FMT, bool GU, int BM, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) moe_gemm_kernel(GemmArgs p) {
  constexpr int NT = WAVES * 64;
  constexpr int RB = BM / 32;
  constexpr int CHUNKS = BM * (kBK / 8) / NT;
  static_assert(CHUNKS >= 1 && (BM * (kBK / 8)) % NT == 0, "A staging split");
  __shared__ __attribute__((aligned(16))) _Float16 lds[2][BM][kPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int nt = blockIdx.x % p.n_ntiles;
  const int mt = blockIdx.x / p.n_ntiles;
  if (mt >= *p.n_mtiles) return;
  const int e = p.tiles[4 * mt], row0 = p.tiles[4 * mt + 1], rows = p.tiles[4 * mt + 2];

  // ---- this lane's two weight rows (fragment f = 0, 1)
  int64_t nrow[2];
  bool nvalid[2];
  if (GU) {
    const int64_t j = int64_t(nt) * (WAVES * 32) + wave * 32 + col;
    nvalid[0] = nvalid[1] = j < p.I;
    const int64_t jc = j < p.I ? j : p.I - 1;
    nrow[0] = jc;
    nrow[1] = p.I + jc;
  } else {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int64_t n = int64_t(nt) * (WAVES * 64) + wave * 64 + f * 32 + col;
      nvalid[f] = n < p.N;
      nrow[f] = n < p.N ? n : p.N - 1;
    }
  }
  const int64_t kbytes = p.K >> 1;
  const uint8_t* wrow[2];
  const float* srow_nf4[2];
  const uint8_t* srow_mx[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int64_t r = int64_t(e) * p.N + nrow[f];
    wrow[f] = p.wq + r * kbytes + 16 * half;
    srow_nf4[f] = reinterpret_cast<const float*>(p.sc) + r * (p.K >> 6);
    srow_mx[f] = reinterpret_cast<const uint8_t*>(p.sc) + r * (p.K >> 5) + half;
  }

  // ---- activation rows this thread stages (16-byte chunks)
  const _Float16* arow[CHUNKS];
  int lrow[CHUNKS], lcol[CHUNKS];
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const int q = tid + c * NT;
    const int r = q >> 3;
    const int rr = r < rows ? r : rows - 1;
    int64_t src;
    if (GU) {
      src = int64_t(p.slots[row0 + rr] / p.k_top);
    } else {
      src = int64_t(row0 + rr);
    }
    arow[c] = p.a + src * p.K + (q & 7) * 8;
    lrow[c] = r;
    lcol[c] = (q & 7) * 8;
  }

  f32x16 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    acc[rb][0] = f32x16{};
    acc[rb][1] = f32x16{};
  }

  const int nk = int(p.K / kBK);
  u32x4 areg[CHUNKS];
  u32x4 breg[2];
  float sreg[2];

  auto load_a = [&](int kb) {
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) areg[c] = *reinterpret_cast<const u32x4*>(arow[c] + kb * kBK);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
      *reinterpret_cast<u32x4*>(&lds[buf][lrow[c]][lcol[c]]) = areg[c];
  };
  auto load_b = [&](int kb) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      breg[f] = *reinterpret_cast<const u32x4*>(wrow[f] + int64_t(kb) * 32);
      if (FMT == 0)
        sreg[f] = srow_nf4[f][kb];
      else
        sreg[f] = e8m0_to_f32(srow_mx[f][2 * kb]);
    }
  };

  load_a(0);
  load_b(0);
  store_a(0);
  __syncthreads();

  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    u32x4 bcur[2] = {breg[0], breg[1]};
    float scur[2] = {sreg[0], sreg[1]};
    if (kb + 1 < nk) {
      load_a(kb + 1);
      load_b(kb + 1);
    }
    f16x2 s16[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) s16[f] = f16x2{(_Float16)scur[f], (_Float16)scur[f]};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f16x8 bfrag[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        uint32_t d[4];
        if (FMT == 0) {
          nf4_decode8(bcur[f][s], d);
#pragma unroll
          for (int i = 0; i < 4; ++i) d[i] = pk_mul_f16(d[i], s16[f]);
        } else {
          mxfp4_decode8(bcur[f][s], scur[f], d);
        }
        bfrag[f] = __builtin_bit_cast(f16x8, u32x4{d[0], d[1], d[2], d[3]});
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const f16x8 afrag =
            *reinterpret_cast<const f16x8*>(&lds[cur][32 * rb + col][32 * half + 8 * s]);
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afrag, bfrag[0], acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afrag, bfrag[1], acc[rb][1], 0, 0, 0);
      }
    }
    if (kb + 1 < nk) store_a(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Accumulator element r of a 32x32 block: row 8*(r/4) + 4*half + r%4,
  // column = col.
  if (GU) {
    if (!nvalid[0]) return;
    const int64_t j = int64_t(nt) * (WAVES * 32) + wave * 32 + col;
    _Float16* hout = reinterpret_cast<_Float16*>(p.out);
    const int64_t pos = act_pos<FMT>(j);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < rows) {
          const float g = acc[rb][0][r];
          const float u = acc[rb][1][r];
          const float hv = g / (1.0f + __expf(-g)) * u;
          hout[int64_t(row0 + row) * p.I + pos] = (_Float16)hv;
        }
      }
    }
  } else {
    float* y = reinterpret_cast<float*>(p.out);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < rows) {
          const int32_t slot = p.slots[row0 + row];
          const float wgt = p.topk_w[slot];
#pragma unroll
          for (int f = 0; f < 2; ++f)
            if (nvalid[f]) y[int64_t(slot) * p.N + nrow[f]] = wgt * acc[rb][f][r];
        }
      }
    }
  }
}

// x bf16 -> fp16 (exact for |x| in fp16's normal range), stored in the k-slot order of the
// weight format inside each aligned group of 8.
template <int FMT>
__global__ void __launch_bounds__(256) convert_x_kernel(const uint16_t* __restrict__ x,
                                                        _Float16* __restrict__ x16,
                                                        int64_t n_chunks) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < n_chunks; q += stride) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(x + 8 * q);
    _Float16 v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (_Float16)__uint_as_float(raw[i] << 16);
      v[2 * i + 1] = (_Float16)__uint_as_float(raw[i] & 0xFFFF0000u);
    }
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[FMT == 0 ? nf4_elem_slot(i) : i] = v[i];
    *reinterpret_cast<f16x8*>(x16 + 8 * q) = o;
  }
}

// One workgroup: walk the experts in order, cut each expert's rows into BM-row tiles.
__global__ void __launch_bounds__(256) build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                          int E, int bm,
                                                          int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ n_mtiles) {
  __shared__ int32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int run = 0;
  for (int base = 0; base < E; base += 256) {
    const int e = base + tid;
    const int start = e < E ? offsets[e] : 0;
    const int cnt = e < E ? offsets[e + 1] - start : 0;
    const int nt = (cnt + bm - 1) / bm;
    // inclusive scan inside the wave
    int incl = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    __syncthreads();
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      woff += w < wave ? wsum[w] : 0;
      tot += wsum[w];
    }
    const int first = run + woff + incl - nt;
    for (int i = 0; i < nt; ++i) {
      int32_t* t = tiles + 4 * int64_t(first + i);
      t[0] = e;
      t[1] = start + i * bm;
      t[2] = min(bm, cnt - i * bm);
      t[3] = 0;
    }
    run += tot;
  }
  if (tid == 0) *n_mtiles = run;
}

// out[t, :] = sum_{j<k} y[t*k + j, :], fixed order; fp32 and bf16 (RNE) outputs.
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y, int64_t T,
                                                      int64_t H, int k,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ out_f32) {
  const int64_t n4 = T * (H / 4);
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < n4; q += stride) {
    const int64_t t = q / (H / 4);
    const int64_t c = (q - t * (H / 4)) * 4;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) s += *reinterpret_cast<const f32x4*>(y + (t * k + j) * H + c);
    if (out_f32) *reinterpret_cast<f32x4*>(out_f32 + t * H + c) = s;
    u32x2 o;
    o[0] = uint32_t(f32_to_bf16_rne(s[0])) | (uint32_t(f32_to_bf16_rne(s[1])) << 16);
    o[1] = uint32_t(f32_to_bf16_rne(s[2])) | (uint32_t(f32_to_bf16_rne(s[3])) << 16);
    *reinterpret_cast<u32x2*>(out + t * H + c) = o;
  }
}

static unsigned grid_1d(int64_t work, int per_block = 256) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > 1 << 20) g = 1 << 20;
  return unsigned(g);
}

static void record(const MoeLaunch& L, int i, hipStream_t stream) {
  if (L.events) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(L.events[i]), stream);
}

template <int FMT, int BM, int WAVES>
static hipError_t launch_gemms(const MoeLaunch& L, hipStream_t stream) {
  GemmArgs g{};
  g.tiles = L.tiles;
  g.n_mtiles = L.n_mtiles;
  g.slots = L.slots;
  g.topk_w = L.topk_w;
  g.k_top = L.k;
  g.I = L.I;
  // gate_up + SwiGLU
  g.a = L.x16;
  g.wq = L.w_gu;
  g.sc = L.s_gu;
  g.out = L.h;
  g.K = L.H;
  g.N = 2 * L.I;
  g.n_ntiles = int((L.I + WAVES * 32 - 1) / (WAVES * 32));
  hipLaunchKernelGGL((moe_gemm_kernel<FMT, true, BM, WAVES>),
                     dim3(unsigned(L.max_mtiles * g.n_ntiles)), dim3(WAVES * 64), 0, stream, g);
  record(L, 3, stream);
  // down + routing weight
  g.a = L.h;
  g.wq = L.w_dn;
  g.sc = L.s_dn;
  g.out = L.y;
  g.K = L.I;
  g.N = L.H;
  g.n_ntiles = int((L.H + WAVES * 64 - 1) / (WAVES * 64));
  hipLaunchKernelGGL((moe_gemm_kernel<FMT, false, BM, WAVES>),
                     dim3(unsigned(L.max_mtiles * g.n_ntiles)), dim3(WAVES * 64), 0, stream, g);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(const MoeLaunch& L, hipStream_t stream) {
  record(L, 0, stream);
  hipLaunchKernelGGL(convert_x_kernel<FMT>, dim3(grid_1d(L.T * L.H / 8)), dim3(256), 0, stream,
                     L.x, L.x16, L.T * L.H / 8);
  record(L, 1, stream);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, stream, L.offsets, int(L.E),
                     L.cfg.bm, L.tiles, L.n_mtiles);
  record(L, 2, stream);
  hipError_t err;
  if (L.cfg.bm == 256)
    err = launch_gemms<FMT, 256, 4>(L, stream);
  else if (L.cfg.bm == 128)
    err = launch_gemms<FMT, 128, 4>(L, stream);
  else
    err = launch_gemms<FMT, 32, 1>(L, stream);
  if (err != hipSuccess) return err;
  record(L, 4, stream);
  hipLaunchKernelGGL(combine_kernel, dim3(grid_1d(L.T * L.H / 4)), dim3(256), 0, stream, L.y, L.T,
                     L.H, L.k, L.out, L.out_f32);
  record(L, 5, stream);
  return hipGetLastError();
}

hipError_t launch_moe_forward(const MoeLaunch& L, hipStream_t stream) {
  return L.fmt == 0 ? launch_fmt<0>(L, stream) : launch_fmt<1>(L, stream);
}

}  // namespace e4b
