// Grouped input gradient on the packed expert stacks: for the rows p of expert e (grouped by
// expert, offsets from the router), out[p, k] = sum_n g[p, n] * W_e[n, k], i.e. the forward
// product y = x W_e^T transposed (Cerin Amroth "ML systems" index, Ownership: the grouped
// packed GEMM and its dgrad).  The weights stay packed; they are decoded tile by tile.
//
// The contraction now runs over the weight rows n, while a packed row is contiguous along k,
// so the MFMA operand that needs 8 consecutive n for one k cannot be read from a row.  Each
// K step (32 weight rows) is decoded cooperatively and written to LDS transposed, [k][n]
// fp16, in a padded, swizzled layout; the gradient tile goes to LDS as [row][n] fp16.  Both are
// double-buffered with one workgroup barrier per step.
//
// Workgroup: 8 waves (two per SIMD), a tile of <= 256 grouped rows of one expert x 256
// columns k; wave w owns rows 128(w/4) .. +127 and columns 64(w%4) .. +63 (four 32-row blocks x
// two 32-column fragments, fp32 accumulators in registers, v_mfma_f32_32x32x16_f16), so each
// decoded weight feeds 256 rows.  The global loads of a step are issued two steps ahead of its
// staging (two register sets) with per-step offsets in scalar registers.
#include "e4b_device.h"
#include "e4b_internal.h"

namespace e4b {

namespace {

constexpr int kThreads = 512;
constexpr int kRows = 256;           // grouped rows per tile
constexpr int kCols = 256;           // output columns k per workgroup
constexpr int kStepN = 32;           // weight rows n per step

// LDS tile layout: a tile row (a grouped row of the gradient, or a column k of the weights)
// holds the step's 32 n values in fp16 as four 16-byte chunks.  Rows are 64 bytes apart plus
// 64 bytes after every 8 rows, and chunk j of row r sits in slot j ^ ((r >> 2) & 3) (gradient)
// or j ^ (((r >> 2) ^ (r >> 5)) & 3) (weights).  Then the 16-byte fragment reads (16
// consecutive rows, one chunk), the 16-byte gradient writes (whole rows) and the 4-byte
// transposed weight writes (4 n-pairs x 16 columns 8 apart) each spread over all 64 banks
// without conflicts.
__device__ __forceinline__ int lds_off(int r, int j) {
  return 64 * r + 64 * (r >> 3) + 16 * (j ^ ((r >> 2) & 3));
}
__device__ __forceinline__ int lds_off_w(int r, int j) {
  return 64 * r + 64 * (r >> 3) + 16 * (j ^ (((r >> 2) ^ (r >> 5)) & 3));
}
constexpr int tile_bytes(int rows) { return 64 * rows + 64 * (rows / 8); }
constexpr int kGBytes = tile_bytes(kRows);   // gradient tile [256][32] fp16
constexpr int kWBytes = tile_bytes(kCols);   // transposed weight tile [256][32] fp16
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

// Element e (0..7) of a decoded dword sits in output register elem_reg(e), half elem_hi(e):
// NF4's register decode leaves slot order (0,2) (4,6) (1,3) (5,7), MXFP4 natural order.
template <int FMT>
__device__ __forceinline__ int elem_reg(int e) { return FMT == 0 ? ((e & 1) ? 2 + (e >> 2) : (e >> 2)) : (e >> 1); }
template <int FMT>
__device__ __forceinline__ int elem_hi(int e) { return FMT == 0 ? ((e >> 1) & 1) : (e & 1); }

// Global loads of one step for one thread: two 16-byte gradient pieces, two packed dwords and
// their two scales.
struct StepRegs {
  u32x4 g[2];
  uint32_t w[2], s[2];
};

template <int FMT>
__global__ void __launch_bounds__(kThreads) dgrad_kernel(DgradArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kBufBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int rh = wave >> 2, wcol = wave & 3;
  const int kt = int(blockIdx.x) % p.n_ktiles;
  const int mt = int(blockIdx.x) / p.n_ktiles;
  if (mt >= *p.n_tiles) return;  // uniform
  const int e = p.tiles[4 * mt], row0 = p.tiles[4 * mt + 1], rows = p.tiles[4 * mt + 2];
  const int64_t kbytes = p.K >> 1;
  const int nsteps = int(p.N / kStepN);  // even: N is a multiple of 64

  // ---- staging roles.  Gradient: thread t loads chunk t%4 (8 n values) of rows t/4 and
  // t/4 + 128, so 16 consecutive lanes fill 4 whole tile rows (256 contiguous LDS bytes).
  // Weights: lane l of wave w decodes rows 2q, 2q + 1 (q = 4(w%4) + l/16) of the step at
  // column chunk c = 16(w/4) + l%16 (8 columns = one packed dword per row), so one load covers
  // 64 contiguous bytes of each of 4 rows.
  const int grow = tid >> 2, gj = tid & 3;
  const int grow0_c = grow < rows ? grow : rows - 1;
  const int grow1_c = grow + kThreads / 4 < rows ? grow + kThreads / 4 : rows - 1;
  const __amdgpu_buffer_rsrc_t gres =
      buffer_rsrc(p.g + int64_t(row0) * p.N, uint32_t(int64_t(rows) * p.N * 2));
  const uint32_t goff0 = uint32_t(grow0_c) * uint32_t(p.N) * 2u + 16u * gj;
  const uint32_t goff1 = uint32_t(grow1_c) * uint32_t(p.N) * 2u + 16u * gj;
  const int wq2 = 4 * (wave & 3) + (lane >> 4), wc = 16 * (wave >> 2) + (lane & 15);
  const int64_t kcol0 = int64_t(kt) * kCols + 8 * wc;       // first column of the chunk
  const bool wvalid = kcol0 < p.K;
  const uint32_t nblk = uint32_t(FMT == 0 ? (p.K >> 6) : (p.K >> 5));  // scale blocks per row
  const uint32_t sblk = wvalid ? uint32_t(FMT == 0 ? (kcol0 >> 6) : (kcol0 >> 5)) : 0u;
  const __amdgpu_buffer_rsrc_t wres =
      buffer_rsrc(p.wq + int64_t(e) * p.N * kbytes, uint32_t(p.N * kbytes));
  const uint32_t woff = uint32_t(2 * wq2) * uint32_t(kbytes) + uint32_t(wvalid ? (kcol0 >> 1) : 0);
  constexpr uint32_t kScaleBytes = FMT == 0 ? 4u : 1u;
  const __amdgpu_buffer_rsrc_t sres =
      buffer_rsrc(static_cast<const uint8_t*>(p.sc) + int64_t(e) * p.N * nblk * kScaleBytes,
                  uint32_t(p.N * nblk * kScaleBytes));
  const uint32_t soff = (uint32_t(2 * wq2) * nblk + sblk) * kScaleBytes;

  // The loads of a step are issued in one fixed order everywhere (scheduling barriers between
  // them): the wait-count pass merges the prologue's and the loop's states at the loop header
  // and can only keep its counts tight if both issued the loads in the same order.
  auto load_step = [&](int s, StepRegs& R) {
    const uint32_t n0 = uint32_t(s * kStepN);  // uniform: the step's offsets go in SGPRs
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      R.g[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(gres, i ? goff1 : goff0, 2u * n0, 0));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      R.w[r] = __builtin_amdgcn_raw_buffer_load_b32(wres, woff + uint32_t(r) * uint32_t(kbytes),
                                                     n0 * uint32_t(kbytes), 0);
      __builtin_amdgcn_sched_barrier(0);
      if (FMT == 0)
        R.s[r] = __builtin_amdgcn_raw_buffer_load_b32(sres, soff + uint32_t(r) * nblk * 4u, n0 * nblk * 4u, 0);
      else
        R.s[r] = __builtin_amdgcn_raw_buffer_load_b8(sres, soff + uint32_t(r) * nblk, n0 * nblk, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto stage_step = [&](const StepRegs& R, int buf) {
    uint8_t* gb = smem + buf * kBufBytes;
    uint8_t* wb = gb + kGBytes;
    // gradient: bf16 -> fp16 (exact in fp16's normal range)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f16x8 h;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[2 * j] = (_Float16)__uint_as_float(R.g[i][j] << 16);
        h[2 * j + 1] = (_Float16)__uint_as_float(R.g[i][j] & 0xFFFF0000u);
      }
      *reinterpret_cast<f16x8*>(gb + lds_off(grow + i * (kThreads / 4), gj)) = h;
    }
    // weights: decode 2 rows x 8 columns, write each column's 2 rows as one 4-byte word
    uint32_t d[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (FMT == 0) {
        nf4_decode8(R.w[r], d[r]);
        const _Float16 sh = (_Float16)(__uint_as_float(R.s[r]) * kNf4ScaleUp);
        const f16x2 s16 = f16x2{sh, sh};
#pragma unroll
        for (int i = 0; i < 4; ++i) d[r][i] = pk_mul_f16(d[r][i], s16);
      } else {
        mxfp4_decode8(R.w[r], e8m0_to_f32(R.s[r]), d[r]);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int reg = elem_reg<FMT>(c), hi = elem_hi<FMT>(c);
      const uint32_t v = perm(d[1][reg], d[0][reg], hi ? 0x07060302u : 0x05040100u);
      *reinterpret_cast<uint32_t*>(wb + lds_off_w(8 * wc + c, wq2 >> 2) + 4 * (wq2 & 3)) = v;
    }
  };
  // A fragment: rows 128rh + 32rb + col, n 16sub + 8half .. +7; B fragment: column
  // 64wcol + 32f + col.
  auto afrag = [&](int buf, int rb, int sub) {
    return *reinterpret_cast<const f16x8*>(smem + buf * kBufBytes +
                                           lds_off(128 * rh + 32 * rb + col, 2 * sub + half));
  };
  auto bfrag = [&](int buf, int f, int sub) {
    return *reinterpret_cast<const f16x8*>(smem + buf * kBufBytes + kGBytes +
                                           lds_off_w(64 * wcol + 32 * f + col, 2 * sub + half));
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb][0] = acc[rb][1] = f32x16{};
  auto read_sub = [&](int buf, int sub, f16x8 (&a)[4], f16x8 (&b)[2]) {
    b[0] = bfrag(buf, 0, sub);
    b[1] = bfrag(buf, 1, sub);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) a[rb] = afrag(buf, rb, sub);
  };
  auto mma = [&](const f16x8 (&a)[4], const f16x8 (&b)[2]) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[rb], b[0], acc[rb][0], 0, 0, 0);
      acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[rb], b[1], acc[rb][1], 0, 0, 0);
    }
  };
  // One step: all twelve fragment reads of the step go out first, into distinct registers, so
  // the LDS latency is paid once per step; the staging of the next step into the other buffer
  // is woven between the MFMAs (both waves of a SIMD leave the barrier together, so the MFMA
  // pipe and the VALU only overlap if each wave interleaves them itself).
  auto step = [&](int buf, const StepRegs& R) {
    f16x8 a0[4], b0[2], a1[4], b1[2];
    __builtin_amdgcn_sched_barrier(0);
    read_sub(buf, 0, a0, b0);
    read_sub(buf, 1, a1, b1);
    mma(a0, b0);
    mma(a1, b1);
    stage_step(R, buf ^ 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // DS read: all fragments
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
      if (i >= 6) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Register set A holds the even steps' loads, B the odd ones'.  Loads past the last step
  // repeat the last step and the last staging writes a buffer nobody reads any more: both keep
  // the loop body branch-free and the wait counts the same every pass.
  StepRegs A, B;
  load_step(0, A);
  load_step(1, B);
  stage_step(A, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_step(nsteps > 2 ? 2 : nsteps - 1, A);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    // step s in buffer 0; B holds step s + 1, A step s + 2
    step(0, B);  // buffer 1 was last read in step s - 1, before the previous barrier
    load_step(s + 3 < nsteps ? s + 3 : nsteps - 1, B);
    __syncthreads();
    // step s + 1 in buffer 1; A holds step s + 2, B step s + 3
    step(1, A);
    load_step(s + 4 < nsteps ? s + 4 : nsteps - 1, A);
    __syncthreads();
  }

  // ---- epilogue.  Accumulator element r of a 32x32 block: row 8(r/4) + 4half + r%4.
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int64_t k = int64_t(kt) * kCols + 64 * wcol + 32 * f + col;
    if (k >= p.K) continue;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 128 * rh + 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < rows) {
          const int64_t o = int64_t(row0 + row) * p.K + k;
          const float v = FMT == 0 ? acc[rb][f][r] * kNf4ScaleDown : acc[rb][f][r];
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
    hipLaunchKernelGGL(dgrad_kernel<0>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(dgrad_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

int dgrad_tile_rows() { return kRows; }

}  // namespace e4b
