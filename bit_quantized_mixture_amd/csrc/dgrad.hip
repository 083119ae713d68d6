// Grouped input gradient on the packed expert stacks: for the rows p of expert e (grouped by
// expert, offsets from the router), out[p, k] = sum_n g[p, n] * W_e[n, k], i.e. the forward
// product y = x W_e^T transposed (Cerin Amroth "ML systems" index, Ownership: the grouped
// packed GEMM and its dgrad).  The weights stay packed; they are decoded tile by tile.
//
// The contraction now runs over the weight rows n, while a packed row is contiguous along k,
// so the MFMA operand that needs 8 consecutive n for one k cannot be read from a row.  Each
// K step (32 weight rows) is decoded cooperatively and written to LDS transposed, [k][n]
// fp16, with a padded row pitch; the gradient tile goes to LDS as [row][n] fp16.  Both are
// double-buffered with one workgroup barrier per step.
//
// Workgroup: 4 waves, a tile of <= 128 grouped rows of one expert x 256 columns k; wave w owns
// columns 64w .. 64w + 63 (two 32-column fragments) for all 128 rows, fp32 accumulators in
// registers (v_mfma_f32_32x32x16_f16, four row blocks x two fragments).
#include "e4b_device.h"
#include "e4b_internal.h"

namespace e4b {

namespace {

constexpr int kRows = 128;           // grouped rows per tile
constexpr int kCols = 256;           // output columns k per workgroup
constexpr int kStepN = 32;           // weight rows n per step
constexpr int kPitch = 80;           // LDS row pitch in bytes (64 data + 16 pad: 16-lane
                                     // groups of 16-byte reads hit distinct banks)
constexpr int kGBytes = kRows * kPitch;   // gradient tile [128][32] fp16
constexpr int kWBytes = kCols * kPitch;   // transposed weight tile [256][32] fp16
constexpr int kBufBytes = kGBytes + kWBytes;

struct DgradArgs {
  const uint16_t* g;        // [S, N] bf16, grouped rows
  const uint8_t* wq;        // [E, N, K/2] packed codes
  const void* sc;           // NF4 float [E, N, K/64] | MXFP4 uint8 [E, N, K/32]
  const int32_t* tiles;     // [max_tiles, 4]: expert, first row, rows, 0
  const int32_t* n_tiles;
  float* out_f32;           // [S, K]
  uint16_t* out;            // nullable [S, K] bf16
  int64_t N, K;
  int32_t n_ktiles;
};

// Element e (0..7) of a decoded dword sits in output register kReg[e], half kHi[e]: NF4's
// register decode leaves slot order (0,2) (4,6) (1,3) (5,7), MXFP4 natural order.
template <int FMT>
__device__ __forceinline__ int elem_reg(int e) { return FMT == 0 ? ((e & 1) ? 2 + (e >> 2) : (e >> 2)) : (e >> 1); }
template <int FMT>
__device__ __forceinline__ int elem_hi(int e) { return FMT == 0 ? ((e >> 1) & 1) : (e & 1); }

template <int FMT>
__global__ void __launch_bounds__(256) dgrad_kernel(DgradArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kBufBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int kt = int(blockIdx.x) % p.n_ktiles;
  const int mt = int(blockIdx.x) / p.n_ktiles;
  if (mt >= *p.n_tiles) return;  // uniform
  const int e = p.tiles[4 * mt], row0 = p.tiles[4 * mt + 1], rows = p.tiles[4 * mt + 2];
  const int64_t kbytes = p.K >> 1;
  const int nsteps = int(p.N / kStepN);

  // ---- staging roles.  Gradient: thread t loads row t/2, n half (t&1)*16 (two 16-byte
  // loads of 8 bf16).  Weights: thread t decodes rows 4q..4q+3 (q = t/32) of the step at
  // column chunk c = t%32 (8 columns = one packed dword per row).
  const int grow = tid >> 1, gh = tid & 1;
  const int grow_c = grow < rows ? grow : rows - 1;
  const uint16_t* gsrc = p.g + int64_t(row0 + grow_c) * p.N + 16 * gh;
  const int wq4 = tid >> 5, wc = tid & 31;
  const int64_t kcol0 = int64_t(kt) * kCols + 8 * wc;       // first column of the chunk
  const bool wvalid = kcol0 < p.K;
  const uint32_t wbyte = uint32_t(wvalid ? (kcol0 >> 1) : 0);
  const __amdgpu_buffer_rsrc_t wres =
      buffer_rsrc(p.wq + int64_t(e) * p.N * kbytes, uint32_t(p.N * kbytes));
  const int64_t nblk = FMT == 0 ? (p.K >> 6) : (p.K >> 5);  // scale blocks per row
  const int64_t sblk = wvalid ? (FMT == 0 ? (kcol0 >> 6) : (kcol0 >> 5)) : 0;

  u32x4 gv[2];
  uint32_t wv[4], sv[4];
  auto load_step = [&](int s) {
    const int n0 = s * kStepN;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      gv[i] = *reinterpret_cast<const u32x4*>(gsrc + n0 + 8 * i);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t n = n0 + 4 * wq4 + r;
      wv[r] = __builtin_amdgcn_raw_buffer_load_b32(wres, uint32_t(n * kbytes) + wbyte, 0, 0);
      if (FMT == 0)
        sv[r] = __float_as_uint(reinterpret_cast<const float*>(p.sc)[(int64_t(e) * p.N + n) * nblk + sblk]);
      else
        sv[r] = reinterpret_cast<const uint8_t*>(p.sc)[(int64_t(e) * p.N + n) * nblk + sblk];
    }
  };
  auto stage_step = [&](int buf) {
    uint8_t* gb = smem + buf * kBufBytes;
    uint8_t* wb = gb + kGBytes;
    // gradient: bf16 -> fp16 (exact in fp16's normal range)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f16x8 h;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[2 * j] = (_Float16)__uint_as_float(gv[i][j] << 16);
        h[2 * j + 1] = (_Float16)__uint_as_float(gv[i][j] & 0xFFFF0000u);
      }
      *reinterpret_cast<f16x8*>(gb + grow * kPitch + 32 * gh + 16 * i) = h;
    }
    // weights: decode 4 rows x 8 columns, write each column's 4 rows as one 8-byte word
    uint32_t d[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (FMT == 0) {
        nf4_decode8(wv[r], d[r]);
        const float scf = __uint_as_float(sv[r]);
        const f16x2 s16 = f16x2{(_Float16)scf, (_Float16)scf};
#pragma unroll
        for (int i = 0; i < 4; ++i) d[r][i] = pk_mul_f16(d[r][i], s16);
      } else {
        mxfp4_decode8(wv[r], e8m0_to_f32(sv[r]), d[r]);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int reg = elem_reg<FMT>(c), hi = elem_hi<FMT>(c);
      const uint32_t sel = hi ? 0x07060302u : 0x05040100u;
      const uint32_t lo01 = perm(d[1][reg], d[0][reg], sel);
      const uint32_t lo23 = perm(d[3][reg], d[2][reg], sel);
      *reinterpret_cast<u32x2*>(wb + (8 * wc + c) * kPitch + 8 * wq4) = u32x2{lo01, lo23};
    }
  };
  // A fragment: rows 32rb + col, n 16sub + 8half .. +7; B fragment: column 64wave + 32f + col.
  auto afrag = [&](int buf, int rb, int sub) {
    return *reinterpret_cast<const f16x8*>(smem + buf * kBufBytes + (32 * rb + col) * kPitch +
                                           32 * sub + 16 * half);
  };
  auto bfrag = [&](int buf, int f, int sub) {
    return *reinterpret_cast<const f16x8*>(smem + buf * kBufBytes + kGBytes +
                                           (64 * wave + 32 * f + col) * kPitch + 32 * sub + 16 * half);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb][0] = acc[rb][1] = f32x16{};

  load_step(0);
  stage_step(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nsteps;  // uniform
    if (more) load_step(s + 1);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const f16x8 b0 = bfrag(buf, 0, sub), b1 = bfrag(buf, 1, sub);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const f16x8 a = afrag(buf, rb, sub);
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b0, acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b1, acc[rb][1], 0, 0, 0);
      }
    }
    // the other buffer was last read in step s - 1, before the previous barrier
    if (more) stage_step(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Accumulator element r of a 32x32 block: row 8(r/4) + 4half + r%4.
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int64_t k = int64_t(kt) * kCols + 64 * wave + 32 * f + col;
    if (k >= p.K) continue;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < rows) {
          const int64_t o = int64_t(row0 + row) * p.K + k;
          const float v = acc[rb][f][r];
          p.out_f32[o] = v;
          if (p.out) p.out[o] = f32_to_bf16_rne(v);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_dgrad(const DgradLaunch& L, hipStream_t stream) {
  hipError_t err = launch_build_tiles(L.offsets, int(L.E), kRows, L.tiles, L.n_tiles, stream);
  if (err != hipSuccess) return err;
  DgradArgs a{};
  a.g = L.g;
  a.wq = L.wq;
  a.sc = L.sc;
  a.tiles = L.tiles;
  a.n_tiles = L.n_tiles;
  a.out_f32 = L.out_f32;
  a.out = L.out;
  a.N = L.N;
  a.K = L.K;
  a.n_ktiles = int((L.K + kCols - 1) / kCols);
  const unsigned grid = unsigned(L.max_tiles * a.n_ktiles);
  if (L.fmt == 0)
    hipLaunchKernelGGL(dgrad_kernel<0>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(dgrad_kernel<1>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

int dgrad_tile_rows() { return kRows; }

}  // namespace e4b
