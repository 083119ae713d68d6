// Small-M expert path (decode): the same grouped gate_up + SwiGLU and down products as
// moe.hip, shaped for experts that receive only a few routed rows.  There the work is
// streaming the packed weights once (grouped-nf4-gemm 0.25.0 project description: the decode
// GEMV beside the grouped GEMM), so this kernel is built around HBM throughput:
//
// * Persistent workgroups of 8 waves, two per CU (16 waves per CU, four per SIMD, so one
//   wave's compute overlaps the others' loads).  A work item is (tile of <= 16 routed rows of
//   one expert, block of 128 * RB weight rows); each wave owns RB row blocks of 16 rows (the
//   launches use RB = 1, which measured faster than 2).  A
//   workgroup walks its items and, inside each item, K in steps of 256, as one flat sequence.
// * 16x16x32 f16 MFMA with the weights as the A operand and the routed activations as B (16
//   columns): D[row, token] += sum_k W[row, k] * X[token, k].  One activation fragment read
//   from LDS feeds the RB row blocks of the wave.
// * Software pipeline: while step s is computed, the weights, scales and activations of step
//   s + 1 are in flight in registers.  Every wave issues the same number of memory operations
//   in every step, with no branch around them (past the last step the loads repeat it and are
//   not used), so one s_waitcnt per step covers it and the compiler's own counting agrees.
//   The activations of step s go to LDS (double buffer) with ordinary ds_write once they have
//   landed: a direct global->LDS copy in flight during the compute would make the compiler
//   wait for every LDS read to drain (lgkmcnt(0)).
// * NF4 decode through a 256-entry LDS table of fp16 pairs, one per packed byte value, with a
//   private copy for each lane: lane l's copy sits entirely in LDS bank l, so the 64 lookups of
//   a wave never conflict, and one v_perm builds each lookup address (byte value * 256 + lane
//   * 4).  A packed dword costs 4 v_perm + 4 ds_read_b32 + 4 v_pk_mul_f16 (the scale), against
//   ~28 VALU operations for an in-register table.  MXFP4 uses the hardware e2m1 conversion
//   with the e8m0 scale.
// * With fewer work items than a third of the resident workgroups (about one token), a second
//   kernel, moe_gemv_ks_kernel, splits K over the waves of a workgroup instead, so that every
//   CU gets work.
//
// K order.  A step covers 256 K = 128 bytes of a weight row.  Load i (0, 1) of lane
// (r = lane % 16, g = lane / 16) reads the 16 bytes at 32*g + 16*i of its row's step, so the
// four lanes of a row fill the 128-byte line, and lane group g's NF4 pieces lie in 64-block g.
// MFMA (i, q) takes dword q of load i: K = 64*g + 32*i + 8*q + [0, 8) inside the step; the
// activation chunk with the same K is read from LDS for token r.  Activations and h are in
// natural K order on this path (the table yields the two elements of a byte in order).
#include <atomic>

#include "e4b_device.h"
#include "e4b_internal.h"
#include "e4b_topk.h"

namespace e4b {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStepK = 256;                        // K per pipeline step
constexpr int kTok = kGemvTileRows;                 // routed rows per tile (MFMA N)
constexpr int kActRowBytes = kStepK * 2;            // fp16 activations of one row per step
constexpr int kActBufBytes = kTok * kActRowBytes;   // 8 KB per buffer
constexpr int kLutBytes = kNf4LutBytes;            // 64 KB: 256 pairs x 64 lane copies
constexpr int kWgPerCu = 2;                         // LDS: 80 KB per workgroup with the table
constexpr int kStages = 2;                          // register sets in the load ring
constexpr int kActLoads = kTok / (2 * kWaves);      // activation loads (two rows each) per wave

static_assert(kTok == 16, "one MFMA pass of 16 routed rows per tile");
static_assert(kActLoads >= 1 && kTok == 2 * kWaves * kActLoads, "activation rows per wave");

// vector-memory operations per lane per step: 2 weight loads and 1 scale load per row block,
// and the activation loads
template <int RB>
constexpr int ops_per_step() { return 3 * RB + kActLoads; }

struct GemvArgs {
  const _Float16* a;       // gate_up: x16 [T, K]; down: h [S, K] (natural K order)
  const uint8_t* wq;       // packed weights [E, N, K/2]
  const void* sc;          // NF4 float [E, N, K/64] | MXFP4 uint8 [E, N, K/32]
  int64_t K;
  int64_t N;               // weight rows per expert (2I for gate_up, H for down)
  int64_t I;
  int64_t T, S;            // tokens, routed rows (rows of x16 and of h)
  int32_t n_rblocks;       // weight-row blocks per expert
  int32_t clamped_glu;     // gate_up activation: 0 silu(G) * U, 1 clamped GLU
  int32_t interleaved;     // gate_up rows: 0 halves (gate j, up I + j), 1 interleaved
  const float* bias;       // nullable [E, N], added to the products
  int32_t ks_waves;        // K-split kernel: waves per 16-row block (1, 2, 4 or 8)
  // down, MFMA path's tail tiles only: nullable [T, N] float32 accumulator; when set,
  // topk_w[slots[p]] * y of sorted row p is added to row tok[p] atomically instead of stored
  float* comb;
  const int32_t* slots;
  const float* topk_w;
};

// Index arrays read with uniform addresses inside the persistent loop are separate
// __restrict__ kernel arguments, so the compiler reads them with scalar loads, which do not
// count against the vector-memory counter the pipeline waits on.
struct Ptrs {
  const int32_t* __restrict__ tiles;  // [n, 4]: expert, first sorted row, rows (<= 16), 0
  const int32_t* __restrict__ tok;    // token of each sorted row [S]
  void* __restrict__ out;             // gate_up: h fp16 [S, I]; down: y float [S, N] (sorted)
};

// Where a step's data come from; every field is uniform across the workgroup.
struct StepInfo {
  int32_t e, row0, rows, rb;
  int32_t kstep;  // first K of the step
  bool last;      // last step of its item
};

// Position of the next step a workgroup issues: flat step s (held at the workgroup's last
// step once reached), K segment seg of item (tile mt, row block rb).  Items of a workgroup
// are blockIdx + i * gridDim, so moving to the next item adds fixed amounts to (mt, rb) and
// no division runs per step.
struct Cursor {
  int32_t s, seg, mt, rb;
};

struct CursorStride {
  int32_t last, nseg, n_rblocks, d_mt, d_rb;
};

__device__ __forceinline__ void advance(Cursor& c, const CursorStride& d) {
  if (c.s < d.last) {
    ++c.s;
    if (++c.seg == d.nseg) {
      c.seg = 0;
      c.mt += d.d_mt;
      c.rb += d.d_rb;
      if (c.rb >= d.n_rblocks) {
        c.rb -= d.n_rblocks;
        ++c.mt;
      }
    }
  }
}

__device__ __forceinline__ StepInfo step_at(const Ptrs& q, const Cursor& c, int nseg) {
  StepInfo st;
  st.rb = c.rb;
  st.e = q.tiles[4 * c.mt];
  st.row0 = q.tiles[4 * c.mt + 1];
  st.rows = q.tiles[4 * c.mt + 2];
  st.kstep = c.seg * kStepK;
  st.last = c.seg == nseg - 1;
  return st;
}

// Weight row of lane row r in row block b of this wave, for item row block rb (clamped;
// results of clamped rows are never stored).  gate_up: a row block is 8 gate rows j..j+7 and
// the 8 matching up rows.
template <bool GU, int RB>
__device__ __forceinline__ int32_t lane_row(const GemvArgs& p, int rb, int wave, int b, int r) {
  if (GU) {
    const int32_t I = int32_t(p.I);
    int32_t j = rb * (kWaves * RB * 8) + (wave * RB + b) * 8 + (r & 7);
    j = j < I ? j : I - 1;
    if (p.interleaved) return r < 8 ? 2 * j : 2 * j + 1;
    return r < 8 ? j : I + j;
  }
  const int32_t N = int32_t(p.N);
  const int32_t n = rb * (kWaves * RB * 16) + (wave * RB + b) * 16 + r;
  return n < N ? n : N - 1;
}

// Activation chunk (8 fp16) L of row c sits at chunk position L ^ (c % 16) of the row, so the
// 16 lanes of one B-operand read (16 rows, same L) hit 16 different 4-bank groups.
__device__ __forceinline__ int xpos(int c, int L) { return L ^ (c & 15); }

template <int RB>
struct StepRegs {
  u32x4 w[RB][2];   // packed weights
  uint32_t sv[RB];  // NF4 absmax bits | MXFP4 two e8m0 bytes
  u32x4 av[kActLoads];  // activations for LDS
};

// Buffer resource over `bytes` bytes at `base` (raw buffer, no stride).  Buffer loads take a
// 32-bit per-lane offset plus a wave-uniform offset, so no 64-bit address arithmetic runs per
// load, and a load entirely past `bytes` returns zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// Issue every memory operation of one step, all unconditional, so the count per step is the
// same for every wave.  The activations go first: the workgroup barrier of a step waits only
// for them, and each wave waits for its own weights where it first uses them.  Pieces past K read the next row (or zeros past the buffer); their
// scale is forced to 0 where the data are used, and activation columns past K meet zero
// weights.
template <int FMT, bool GU, int RB>
__device__ __forceinline__ void issue_step(const GemvArgs& p, const Ptrs& pt,
                                           const StepInfo& st, int wave, int lane,
                                           StepRegs<RB>& R) {
  const int r = lane & 15, g = lane >> 4;
  const uint32_t kb = uint32_t(p.K >> 1);               // packed bytes per row
  const uint32_t nbs = uint32_t(FMT == 0 ? (p.K >> 6) * 4 : (p.K >> 5));  // scale bytes per row
  const __amdgpu_buffer_rsrc_t wres =
      rsrc(p.wq + int64_t(st.e) * p.N * kb, uint32_t(p.N) * kb);
  const __amdgpu_buffer_rsrc_t sres =
      rsrc(reinterpret_cast<const uint8_t*>(p.sc) + int64_t(st.e) * p.N * nbs, uint32_t(p.N) * nbs);
  const int wso = st.kstep >> 1;                               // uniform byte offsets of the step
  const int sso = FMT == 0 ? (st.kstep >> 6) * 4 : (st.kstep >> 5);
  // activations: 16 rows x 512 B; wave w loads rows 2Aw .. 2Aw + 2A - 1 (A = kActLoads), lane
  // l the 16 bytes of chunk position l % 32 of row 2Aw + 2h + l / 32.  Rows at or past the
  // tile's row count repeat its last row (their MFMA columns are discarded).
  const int64_t arows = GU ? p.T : p.S;
  const __amdgpu_buffer_rsrc_t ares = rsrc(p.a, uint32_t(arows * p.K * 2));
#pragma unroll
  for (int h = 0; h < kActLoads; ++h) {
    // the two rows of this load are wave-uniform, so their sources come from scalar loads
    const int c0 = 2 * kActLoads * wave + 2 * h, c1 = c0 + 1;
    const int cs0 = c0 < st.rows ? c0 : st.rows - 1, cs1 = c1 < st.rows ? c1 : st.rows - 1;
    const int32_t src0 = GU ? pt.tok[st.row0 + cs0] : st.row0 + cs0;
    const int32_t src1 = GU ? pt.tok[st.row0 + cs1] : st.row0 + cs1;
    const int c = (lane >> 5) ? c1 : c0;
    const uint32_t src = uint32_t((lane >> 5) ? src1 : src0);
    const uint32_t ao = src * uint32_t(p.K * 2) + 16 * uint32_t(xpos(c, lane & 31));
    R.av[h] = __builtin_bit_cast(u32x4,
                                 __builtin_amdgcn_raw_buffer_load_b128(ares, ao, st.kstep * 2, 0));
  }
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const uint32_t row = uint32_t(lane_row<GU, RB>(p, st.rb, wave, b, r));
    const uint32_t wo = row * kb + 32 * g;
    R.w[b][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, wo, wso, 0));
    R.w[b][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, wo + 16, wso, 0));
    if (FMT == 0)
      R.sv[b] = __builtin_amdgcn_raw_buffer_load_b32(sres, row * nbs + 4 * g, sso, 0);
    else
      R.sv[b] = __builtin_amdgcn_raw_buffer_load_b16(sres, row * nbs + 2 * g, sso, 0);
  }
}

__device__ __forceinline__ void stage_acts(const u32x4 (&av)[kActLoads], int wave, int lane,
                                           uint8_t* xbuf) {
#pragma unroll
  for (int h = 0; h < kActLoads; ++h) {
    const int c = 2 * kActLoads * wave + 2 * h + (lane >> 5);
    *reinterpret_cast<u32x4*>(xbuf + c * kActRowBytes + 16 * (lane & 31)) = av[h];
  }
}

// MFMAs of one step as one straight-line block.  Group n = ((i * 4 + q) * RB + b): dword q of
// load i of row block b.  The table lookups (and, for the first row block, the activation
// fragment) of group n + 2 are issued before group n is formed.
template <int FMT, int RB, int NA, bool SLOT>
__device__ __forceinline__ void compute_step(int64_t krem, int lane, const StepRegs<RB>& R,
                                             const uint8_t* xbuf, const uint8_t* lut,
                                             f32x4 (&acc)[NA]) {
  constexpr int NG = 8 * RB;
  constexpr int D = 2;
  const int r = lane & 15, g = lane >> 4;
  const uint32_t lanebase = uint32_t(lane) << 2;
  const uint8_t* xrow = xbuf + r * kActRowBytes;
  // pieces past K contribute nothing (scale 0)
  const bool valid = int64_t(64 * g) < krem;
  f16x2 s16[RB];
  float smx[RB][2];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if (FMT == 0) {
      const _Float16 sh = (_Float16)(valid ? __uint_as_float(R.sv[b]) * kNf4ScaleUp : 0.0f);
      s16[b] = f16x2{sh, sh};
    } else {
      smx[b][0] = valid ? e8m0_to_f32(R.sv[b] & 0xFFu) : 0.0f;
      smx[b][1] = valid ? e8m0_to_f32((R.sv[b] >> 8) & 0xFFu) : 0.0f;
    }
  }
  uint32_t lk[NG][4];
  f16x8 xb[8];
  auto fetch = [&](int n) {
    const int b = n % RB, iq = n / RB, i = iq >> 2, q = iq & 3;
    if (b == 0) {
      const int L = 8 * g + 4 * i + q;
      xb[iq] = *reinterpret_cast<const f16x8*>(xrow + 16 * xpos(r, L));
    }
    if (FMT == 0) {
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        // byte bt of the dword -> table address (value << 8) | (lane << 2)
        const uint32_t addr = perm(R.w[b][i][q], lanebase, 0x0C0C0400u + (uint32_t(bt) << 8));
        lk[n][bt] = *reinterpret_cast<const uint32_t*>(lut + addr);
      }
    }
  };
#pragma unroll
  for (int n = 0; n < D; ++n) fetch(n);
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    if (n + D < NG) fetch(n + D);
    const int b = n % RB, iq = n / RB, i = iq >> 2, q = iq & 3;
    uint32_t d[4];
    if (FMT == 0) {
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) d[bt] = pk_mul_f16(lk[n][bt], s16[b]);
      if (SLOT) {
        // natural pairs (0,1) (2,3) (4,5) (6,7) -> the slot order of the MFMA-tile path's
        // activations: (0,2) (4,6) (1,3) (5,7)
        const uint32_t p0 = d[0], p1 = d[1], p2 = d[2], p3 = d[3];
        d[0] = perm(p1, p0, 0x05040100u);
        d[1] = perm(p3, p2, 0x05040100u);
        d[2] = perm(p1, p0, 0x07060302u);
        d[3] = perm(p3, p2, 0x07060302u);
      }
    } else {
      mxfp4_decode8(R.w[b][i][q], smx[b][i], d);
    }
    const f16x8 a = __builtin_bit_cast(f16x8, u32x4{d[0], d[1], d[2], d[3]});
    const int ai = RB == 1 ? (n & 1) : b;
    acc[ai] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, xb[iq], acc[ai], 0, 0, 0);
    // keep the written order (lookahead loads before their use) through scheduling
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Results of 16-row block `blk` of the expert's output rows (gate_up: 8 gate rows and the 8
// matching up rows).  acc: element i = D[row 4g + i of the block, token r].
template <int FMT, bool GU, bool SLOT>
__device__ __forceinline__ void store_block(const GemvArgs& p, const Ptrs& pt,
                                            const StepInfo& st, int32_t blk, int lane,
                                            f32x4 acc) {
  const int r = lane & 15, g = lane >> 4;
  if (FMT == 0) acc *= kNf4ScaleDown;  // NF4 sums carry the 2^8 of the scale shift
  if (GU) {
    // rows 0-7 are gate rows, 8-15 the matching up rows: lane groups 0/1 hold gate values,
    // 2/3 the up values of the same (j, token)
    float up[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc[i], 32);
    if (g < 2 && r < st.rows) {
      _Float16* h = reinterpret_cast<_Float16*>(pt.out) + int64_t(st.row0 + r) * p.I;
      const int32_t j0 = blk * 8 + 4 * g;
      const float* bias = p.bias ? p.bias + int64_t(st.e) * p.N : nullptr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t j = j0 + i;
        if (j < int32_t(p.I)) {
          float gv = acc[i], uv = up[i];
          if (bias) {
            gv += bias[p.interleaved ? 2 * j : j];
            uv += bias[p.interleaved ? 2 * j + 1 : int32_t(p.I) + j];
          }
          h[act_pos<SLOT ? 0 : 1>(j)] = (_Float16)(p.clamped_glu ? clamped_glu(gv, uv) : swiglu(gv, uv));
        }
      }
    }
  } else if (r < st.rows) {
    const int32_t n0 = blk * 16 + 4 * g;
    if (n0 < int32_t(p.N)) {  // N % 64 == 0
      f32x4 v = acc;
      if (p.bias) v += *reinterpret_cast<const f32x4*>(p.bias + int64_t(st.e) * p.N + n0);
      if (p.comb) {
        const float w = p.topk_w[p.slots[st.row0 + r]];
        float* dst = p.comb + int64_t(pt.tok[st.row0 + r]) * p.N + n0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          (void)__hip_atomic_fetch_add(dst + i, w * v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        float* y = reinterpret_cast<float*>(pt.out) + int64_t(st.row0 + r) * p.N;
        *reinterpret_cast<f32x4*>(y + n0) = v;
      }
    }
  }
}

template <int FMT, bool GU, int RB, bool SLOT>
__global__ void __launch_bounds__(kThreads)
    moe_gemv_kernel(GemvArgs p, const int32_t* __restrict__ tiles,
                    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ tok,
                    void* __restrict__ out) {
  // n_tiles: the list's tile count, then the index of its first tile in `tiles`
  const Ptrs pt{tiles + 4 * n_tiles[1], tok, out};
  constexpr int kLut = FMT == 0 ? kLutBytes : 0;
  constexpr int kOps = ops_per_step<RB>();
  constexpr int kActWait = (kStages - 1) * kOps + 3 * RB;  // loads issued after a step's acts
  static_assert(kActWait < 64, "vmcnt range");
  constexpr int NA = RB < 2 ? 2 : RB;  // accumulators (two alternating chains when RB == 1)
  // one allocation: the table, then two activation buffers
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLut + 2 * kActBufBytes];
  uint8_t* const lut = smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_items = *n_tiles * p.n_rblocks;
  if (int(blockIdx.x) >= n_items) return;  // uniform over the workgroup
  const int nseg = int((p.K + kStepK - 1) / kStepK);
  const int my_items = (n_items - int(blockIdx.x) + int(gridDim.x) - 1) / int(gridDim.x);
  const int nsteps = my_items * nseg;
  const int last = nsteps - 1;


  // Ring of kStages register sets: step s uses set s % kStages and LDS buffer s % 2; the loads
  // of steps s + 1 .. s + kStages - 1 (and step s's own weights, until first used) are in
  // flight while step s is computed.  Past the last
  // step the loads repeat it and are never used.  Step s's activations are written to LDS
  // right before its barrier, and the barrier of step s + 1 also tells that every wave is done
  // reading buffer s % 2, so one barrier per step suffices.  The loop has a single exit so the
  // compiler's memory-counter bookkeeping stays exact (a mid-loop exit made it fall back to
  // waiting for everything).
  StepRegs<RB> R[kStages];
  StepInfo ci[kStages];
  f32x4 acc[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int first = int(blockIdx.x);
  Cursor cur{0, 0, first / p.n_rblocks, first % p.n_rblocks};
  const CursorStride cst{last, nseg, p.n_rblocks, int(gridDim.x) / p.n_rblocks,
                         int(gridDim.x) % p.n_rblocks};
#pragma unroll
  for (int b = 0; b < kStages - 1; ++b) {
    ci[b] = step_at(pt, cur, nseg);
    issue_step<FMT, GU, RB>(p, pt, ci[b], wave, lane, R[b]);
    advance(cur, cst);
  }
  // the table is filled while the first loads are in flight (the fill makes no memory
  // access, so the loop's memory-counter waits are unchanged); the first step's barrier
  // publishes it to every wave
  if (FMT == 0) nf4_lut_fill(lut, tid, kThreads);
  constexpr int kPeriod = kStages % 2 ? 2 * kStages : kStages;  // (register set, LDS buffer)
  for (int s = 0; s < nsteps; s += kPeriod) {
#pragma unroll
    for (int b2 = 0; b2 < kPeriod; ++b2) {
      const int rs = b2 % kStages, nxt = (b2 + kStages - 1) % kStages;
      uint8_t* const xbuf = smem + kLut + (b2 & 1) * kActBufBytes;
      // step min(s + b2 + kStages - 1, last)
      ci[nxt] = step_at(pt, cur, nseg);
      issue_step<FMT, GU, RB>(p, pt, ci[nxt], wave, lane, R[nxt]);
      advance(cur, cst);
      // the activations of step s + b2 have landed for this wave (its weights and the later
      // steps' loads may stay in flight) ...
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kActWait));
      stage_acts(R[rs].av, wave, lane, xbuf);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kActWait));
      // ... and for every wave, with its activations (and the table) in LDS
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (b2 == 0 || s + b2 < nsteps) {
        compute_step<FMT, RB, NA, SLOT>(p.K - ci[rs].kstep, lane, R[rs], xbuf, lut, acc);
        if (ci[rs].last) {
          const int32_t blk0 = ci[rs].rb * (kWaves * RB) + wave * RB;
          if (RB == 1) {
            store_block<FMT, GU, SLOT>(p, pt, ci[rs], blk0, lane, acc[0] + acc[1]);
          } else {
#pragma unroll
            for (int b = 0; b < RB; ++b) store_block<FMT, GU, SLOT>(p, pt, ci[rs], blk0 + b, lane, acc[b]);
          }
#pragma unroll
          for (int a = 0; a < NA; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
}

// Few routed rows (fewer items than resident workgroups, e.g. one token): a workgroup takes
// 8 / W 16-row blocks of one tile and splits K over W waves per block (wave w of a block takes
// the 256-wide K steps w, w + W, ...); the W partial sums are added in LDS in wave order.  The
// streaming kernel above would leave most CUs idle there and run each item's K steps one after
// another on one CU.  The K order inside a step is that of compute_step; the activation
// fragments come straight from global memory (L2) and NF4 is decoded in registers, so a
// workgroup neither fills a table nor waits for other waves before the final sum.  The
// register decode leaves the 8 elements of a dword in slot order; each activation fragment
// is put in the same order.
template <int FMT, bool GU>
__global__ void __launch_bounds__(kThreads)
    moe_gemv_ks_kernel(GemvArgs p, const int32_t* __restrict__ tiles,
                       const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ tok,
                       void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) f32x4 part[kThreads];  // partial sums
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = p.ks_waves;
  const int mt = int(blockIdx.x) / p.n_rblocks;
  if (mt >= *n_tiles) return;  // uniform over the workgroup
  tiles += 4 * n_tiles[1];     // n_tiles: count, then the index of the list's first tile
  const int32_t n_blocks = int32_t(GU ? (p.I + 7) / 8 : (p.N + 15) / 16);
  const int32_t blk = (int(blockIdx.x) % p.n_rblocks) * (kWaves / W) + wave / W;
  const int wi = wave % W;

  StepInfo st;
  st.e = tiles[4 * mt];
  st.row0 = tiles[4 * mt + 1];
  st.rows = tiles[4 * mt + 2];
  st.rb = blk;
  st.kstep = 0;
  st.last = true;
  const int r = lane & 15, g = lane >> 4;
  // weight row of lane row r (clamped; results of clamped rows are never stored)
  uint32_t row;
  if (GU) {
    const int32_t I = int32_t(p.I);
    int32_t j = blk * 8 + (r & 7);
    j = j < I ? j : I - 1;
    row = uint32_t(p.interleaved ? (r < 8 ? 2 * j : 2 * j + 1) : (r < 8 ? j : I + j));
  } else {
    const int32_t N = int32_t(p.N);
    const int32_t n = blk * 16 + r;
    row = uint32_t(n < N ? n : N - 1);
  }
  // activation row of token column r; columns past the tile's row count repeat its last row
  // (their results are discarded)
  const int c = r < st.rows ? r : st.rows - 1;
  const uint32_t src = uint32_t(GU ? tok[st.row0 + c] : st.row0 + c);
  const uint32_t kb = uint32_t(p.K >> 1);
  const uint32_t nbs = uint32_t(FMT == 0 ? (p.K >> 6) * 4 : (p.K >> 5));
  const __amdgpu_buffer_rsrc_t wres = rsrc(p.wq + int64_t(st.e) * p.N * kb, uint32_t(p.N) * kb);
  const __amdgpu_buffer_rsrc_t sres =
      rsrc(reinterpret_cast<const uint8_t*>(p.sc) + int64_t(st.e) * p.N * nbs, uint32_t(p.N) * nbs);
  const int64_t arows = GU ? p.T : p.S;
  const __amdgpu_buffer_rsrc_t ares = rsrc(p.a, uint32_t(arows * p.K * 2));
  const uint32_t wo = row * kb + 32 * g;
  const uint32_t so = row * nbs + (FMT == 0 ? 4 * g : 2 * g);
  const uint32_t ao = src * uint32_t(p.K * 2) + 128 * g;  // chunk 8g of the step
  // a block past the expert's rows (last workgroup of a tile) computes nothing
  const int nseg = blk < n_blocks ? int((p.K + kStepK - 1) / kStepK) : 0;

  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int seg = wi; seg < nseg; seg += W) {
    const int kstep = seg * kStepK;
    u32x4 w[2];
    w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, wo, kstep >> 1, 0));
    w[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, wo + 16, kstep >> 1, 0));
    const uint32_t sv = FMT == 0 ? __builtin_amdgcn_raw_buffer_load_b32(sres, so, (kstep >> 6) * 4, 0)
                                 : uint32_t(__builtin_amdgcn_raw_buffer_load_b16(sres, so, kstep >> 5, 0));
    // B fragments: chunk 8g + 4i + q of the step for token column r (pieces past K read the
    // next row or zeros past the buffer; they meet zero-scaled weights)
    u32x4 xa[8];
#pragma unroll
    for (int iq = 0; iq < 8; ++iq)
      xa[iq] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ares, ao + 16 * iq, 2 * kstep, 0));
    const bool valid = int64_t(64 * g) < p.K - kstep;
    f16x2 s16{};
    float smx[2] = {0.f, 0.f};
    if (FMT == 0) {
      const _Float16 sh = (_Float16)(valid ? __uint_as_float(sv) * kNf4ScaleUp : 0.0f);
      s16 = f16x2{sh, sh};
    } else {
      smx[0] = valid ? e8m0_to_f32(sv & 0xFFu) : 0.0f;
      smx[1] = valid ? e8m0_to_f32((sv >> 8) & 0xFFu) : 0.0f;
    }
#pragma unroll
    for (int iq = 0; iq < 8; ++iq) {
      const int i = iq >> 2, q = iq & 3;
      uint32_t d[4];
      u32x4 x = xa[iq];
      if (FMT == 0) {
        nf4_decode8(w[i][q], d);
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) d[bt] = pk_mul_f16(d[bt], s16);
        // natural pairs (0,1) (2,3) (4,5) (6,7) -> slot order (0,2) (4,6) (1,3) (5,7)
        x = u32x4{perm(x[1], x[0], 0x05040100u), perm(x[3], x[2], 0x05040100u),
                  perm(x[1], x[0], 0x07060302u), perm(x[3], x[2], 0x07060302u)};
      } else {
        mxfp4_decode8(w[i][q], smx[i], d);
      }
      const f16x8 a = __builtin_bit_cast(f16x8, u32x4{d[0], d[1], d[2], d[3]});
      acc[iq & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, x),
                                                          acc[iq & 1], 0, 0, 0);
    }
  }
  part[tid] = acc[0] + acc[1];
  __syncthreads();
  if (wi == 0 && blk < n_blocks) {
    f32x4 sum = part[64 * wave + lane];
    for (int w = 1; w < W; ++w) sum += part[64 * (wave + w) + lane];
    store_block<FMT, GU, false>(p, Ptrs{tiles, tok, out}, st, blk, lane, sum);
  }
}

// ---------------------------------------------------------------------------------------
// Single-launch decode step for a few tokens (T <= 8, T*k <= 64): the router epilogue, the
// gate_up products with the activation, the down products and the weighted combine in one
// kernel (grouped-nf4-gemm 0.25.0 project description, "What is measured", limit 1: at
// decode the launches, not the bytes, set the time).
//
// * Routing: every workgroup computes the top-k of the T tokens itself (one wave per token,
//   the router's own per-token routine, so ids and weights are bit-identical to
//   e4b_route_permute), sorts the T*k slots expert-major (token-ascending inside an expert)
//   and lists the active experts as tiles of <= T rows.  Workgroup 0 writes the routing out.
// * gate_up: a work item is (tile, 8 gate + 8 up rows); its K steps are split over the 8
//   waves and added in LDS in wave order; the activation goes to h (fp16, sorted-row order)
//   in the workspace with device-coherent stores (written through to memory, so no cache
//   write-back is needed before other workgroups read it).  x is converted from bf16 to fp16
//   as it is loaded.
// * One grid barrier: workgroups arrive on 8 group counters (blockIdx % 8, one cache line
//   each); the last of a group arrives on a top counter, the last of all raises the 8 group
//   flags that the workgroups poll.  Polls are bounded: a wait that gives up sets a flag
//   reported through `status`, and every workgroup still runs to the end.  The first down
//   weights of each wave are loaded while the barrier is pending.
// * down + combine: a work item is (16 output columns, a group of tiles); its (tile, K step)
//   units are spread over the 8 waves, each weighting its product rows by the slot's routing
//   weight into per-token sums, added over lanes and waves in a fixed order.  Items of the
//   same columns store their sums (device-coherent) and count themselves on a per-column
//   counter; the last adds the groups' sums in group order and writes the output.  No y
//   buffer, no second grid barrier, deterministic.
// * Exit: the last workgroup to finish resets the barrier words (the column counters are
//   reset by their last users), so the next call on the same workspace starts from zero.

constexpr int kDecMaxT = 8;    // tokens
constexpr int kDecMaxS = 64;   // routed slots (one wave holds them)
constexpr int kDecGroups = 8;  // barrier groups
constexpr int kDecXChunks = 8; // 16-byte chunks of x per thread: T * H <= 8 * 8 * 512
constexpr int kDecMaxTG = 8;   // tile groups per column block in the down phase
// control words (uint32 offsets): group counters and flags one 64-byte line apart
constexpr int kCtlGrp = 0, kCtlGo = 128, kCtlTop = 256, kCtlDepart = 272, kCtlGaveUp = 288,
              kCtlCols = 512;

struct DecodeStepArgs {
  int32_t E, H, I, T, k, renorm;
  int32_t clamped_glu, interleaved;
  int32_t spin_limit;          // barrier polls before giving up (negative: do not wait)
  const float* logits;         // [T, E]
  const uint16_t* x;           // [T, H] bf16
  const uint8_t* w_gu;
  const void* s_gu;
  const uint8_t* w_dn;
  const void* s_dn;
  const float* b_gu;           // nullable [E, 2I]
  const float* b_dn;           // nullable [E, H]
  int32_t* ids_out;            // nullable [T, k]
  float* w_out;                // nullable [T, k]
  int32_t* offsets_out;        // nullable [E + 1]
  int32_t* slots_out;          // nullable [T * k]
  uint16_t* out;               // [T, H] bf16
  float* out_f32;              // nullable [T, H]
  _Float16* h;                 // workspace [T * k, I], sorted-row order
  float* part;                 // workspace [H / 16][kDecMaxTG][kDecMaxT][16] column-block sums
  uint32_t* ctl;               // workspace control words (zero between calls)
  int32_t* status;             // nullable: 0, or 1 when a barrier wait gave up
};

constexpr int kCohere = 16;  // buffer cache policy: device-coherent (sc1) load / store

// 8 bf16 (one 16-byte load) -> 8 fp16, round to nearest even (exact in fp16's normal range).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 raw) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 lo = (_Float16)__uint_as_float(raw[i] << 16);
    const _Float16 hi = (_Float16)__uint_as_float(raw[i] & 0xFFFF0000u);
    o[i] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
  }
  return o;
}

// One 256-wide K step of a 16-row weight block against <= 16 activation rows (the MFMA
// layout of moe_gemv_ks_kernel): acc[q & 1] += W[16 rows, kstep..] . A[cols, kstep..].
// `act` holds the lane's 8 activation chunks of the step in natural order (fp16).
template <int FMT>
__device__ __forceinline__ void decode_step_mfma(const u32x4 (&w)[2], uint32_t sv, const u32x4 (&act)[8],
                                                 bool valid, f32x4 (&acc)[2]) {
  f16x2 s16{};
  float smx[2] = {0.f, 0.f};
  if (FMT == 0) {
    const _Float16 sh = (_Float16)(valid ? __uint_as_float(sv) * kNf4ScaleUp : 0.0f);
    s16 = f16x2{sh, sh};
  } else {
    smx[0] = valid ? e8m0_to_f32(sv & 0xFFu) : 0.0f;
    smx[1] = valid ? e8m0_to_f32((sv >> 8) & 0xFFu) : 0.0f;
  }
#pragma unroll
  for (int iq = 0; iq < 8; ++iq) {
    const int i = iq >> 2, q = iq & 3;
    uint32_t d[4];
    u32x4 xv = act[iq];
    if (FMT == 0) {
      nf4_decode8(w[i][q], d);
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) d[bt] = pk_mul_f16(d[bt], s16);
      // natural pairs (0,1) (2,3) (4,5) (6,7) -> slot order (0,2) (4,6) (1,3) (5,7)
      xv = u32x4{perm(xv[1], xv[0], 0x05040100u), perm(xv[3], xv[2], 0x05040100u),
                 perm(xv[1], xv[0], 0x07060302u), perm(xv[3], xv[2], 0x07060302u)};
    } else {
      mxfp4_decode8(w[i][q], smx[i], d);
    }
    const f16x8 a = __builtin_bit_cast(f16x8, u32x4{d[0], d[1], d[2], d[3]});
    acc[iq & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, xv), acc[iq & 1], 0, 0, 0);
  }
}

// Weight registers of one down-phase unit.
struct DnUnit {
  u32x4 w[2];
  uint32_t sv;
};

template <int FMT, int PL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
    moe_decode_step_kernel(DecodeStepArgs p) {
  __shared__ int32_t s_ids[kDecMaxS];
  __shared__ float s_w[kDecMaxS];
  __shared__ int32_t s_sorted[kDecMaxS];     // sorted row -> slot
  __shared__ int32_t s_tile[3][kDecMaxS];    // expert, first sorted row, rows
  __shared__ int32_t s_ntiles;
  __shared__ int32_t s_last;
  __shared__ __attribute__((aligned(16))) f32x4 part[kThreads];
  __shared__ float red[kWaves][4][kDecMaxT][4];
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // x as fp16, T rows of 2H + 16 bytes

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, k = p.k, S = T * k, E = p.E;
  const int G = int(gridDim.x);
  const int r = lane & 15, g = lane >> 4;
  const uint32_t xrow = uint32_t(2 * p.H + 16);  // LDS row pitch of x (16 bytes of padding)

  // ---- x -> LDS as fp16, natural order
  // x chunks are spread over the waves that do not route (T < 8), which load them while the
  // routing waves work; with 8 tokens every wave loads its share after the routing
  const int nchunk = T * (p.H / 8);
  const int xw0 = T < kWaves ? T : 0;                    // first loading wave
  const int xthreads = (kWaves - xw0) * 64;
  const int xt = tid - xw0 * 64;                         // index among the loading threads
  const __amdgpu_buffer_rsrc_t xres = rsrc(p.x, uint32_t(int64_t(T) * p.H * 2));
  auto x_to_lds = [&]() {
    for (int c = xt; c < nchunk; c += xthreads) {
      const int t = c / (p.H / 8), k8 = c - t * (p.H / 8);
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, uint32_t(c) * 16, 0, 0));
      *reinterpret_cast<u32x4*>(xs + uint32_t(t) * xrow + 16 * k8) = bf16x8_to_f16x8(v);
    }
  };
  if (T < kWaves && wave >= T) x_to_lds();

  // ---- routing, in every workgroup
  if (wave < T) {
    int id;
    float wt;
    topk_token<PL>(p.logits + int64_t(wave) * E, E, k, p.renorm, lane, id, wt);
    if (lane < k) {
      s_ids[wave * k + lane] = id;
      s_w[wave * k + lane] = wt;
      if (blockIdx.x == 0 && p.ids_out) {
        p.ids_out[wave * k + lane] = id;
        p.w_out[wave * k + lane] = wt;
      }
    }
  }
  __syncthreads();
  if (wave == 0 && lane < S) {  // rank of slot `lane`: expert-major, then slot (= token) order
    const int e = s_ids[lane];
    int rank = 0;
    for (int q = 0; q < S; ++q) {
      const int eq = s_ids[q];
      rank += (eq < e) || (eq == e && q < lane);
    }
    s_sorted[rank] = lane;
  }
  __syncthreads();
  if (wave == 0) {
    const bool v = lane < S;
    const int e = v ? s_ids[s_sorted[lane]] : -1;
    const bool first = v && (lane == 0 || s_ids[s_sorted[lane - 1]] != e);
    const uint64_t m = __ballot(first);
    if (first) {
      const int ti = __popcll(m & ((uint64_t(1) << lane) - 1));
      const uint64_t after = lane == 63 ? 0 : (m >> (lane + 1));
      const int next = after ? lane + 1 + int(__builtin_ctzll(after)) : S;
      s_tile[0][ti] = e;
      s_tile[1][ti] = lane;
      s_tile[2][ti] = next - lane;
    }
    if (lane == 0) s_ntiles = __popcll(m);
    if (blockIdx.x == 0 && v && p.slots_out) p.slots_out[lane] = s_sorted[lane];
  }
  if (blockIdx.x == 0 && p.offsets_out) {
    for (int e = tid; e <= E; e += kThreads) {
      int c = 0;
      for (int q = 0; q < S; ++q) c += s_ids[q] < e;
      p.offsets_out[e] = c;
    }
  }
  if (T >= kWaves) x_to_lds();
  __syncthreads();
  const int ntiles = s_ntiles;

  // ---- gate_up + activation -> h (device-coherent stores).  An item (tile, 8 gate + 8 up
  // rows) is taken by W waves that split its K steps (W = 8, 4, 2 or 1: the largest that still
  // gives every item its waves in one pass over the grid, so few items get split and many do
  // not); a wave runs its K steps of its items as one sequence with the next step's weights in
  // flight (two register sets); the activations come from x in LDS.  With W > 1 an item's last
  // step adds its waves' sums in LDS.
  {
    const int njb = (p.I + 7) / 8;
    const int items = ntiles * njb;
    const int nseg = (p.H + kStepK - 1) / kStepK;
    int W = kWaves;
    while (W > 1 && int64_t(items) * W > int64_t(G) * kWaves) W >>= 1;
    const int ipp = kWaves / W;              // items per workgroup pass
    const int slot = wave / W, kp = wave - slot * W;
    const int spw = (nseg + W - 1) / W;      // K steps per wave per item
    const int64_t N = 2 * int64_t(p.I);
    const uint32_t kb = uint32_t(p.H >> 1);
    const uint32_t nbs = FMT == 0 ? uint32_t(p.H >> 6) * 4 : uint32_t(p.H >> 5);
    const __amdgpu_buffer_rsrc_t hres = rsrc(p.h, uint32_t(int64_t(S) * p.I * 2));
    struct GuLoad {
      u32x4 w[2];
      uint32_t sv;
    };
    // weights of K step st of item it (clamped item past the end; steps past K read zeros or
    // the next row, and their scale is 0)
    auto issue = [&](int it, int st, GuLoad& L) {
      const int itc = it < items ? it : items - 1;
      const int a = itc / njb, jb = itc - a * njb;
      const int e = s_tile[0][a];
      int32_t j = jb * 8 + (r & 7);
      j = j < p.I ? j : p.I - 1;
      const uint32_t row = uint32_t(p.interleaved ? (r < 8 ? 2 * j : 2 * j + 1) : (r < 8 ? j : p.I + j));
      const __amdgpu_buffer_rsrc_t wres = rsrc(p.w_gu + int64_t(e) * N * kb, uint32_t(N) * kb);
      const __amdgpu_buffer_rsrc_t sres =
          rsrc(reinterpret_cast<const uint8_t*>(p.s_gu) + int64_t(e) * N * nbs, uint32_t(N) * nbs);
      const uint32_t wo = row * kb + 32 * g;
      const uint32_t so = row * nbs + (FMT == 0 ? 4 * g : 2 * g);
      const int kstep = (kp + W * st) * kStepK;
      L.w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, wo, kstep >> 1, 0));
      L.w[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, wo + 16, kstep >> 1, 0));
      L.sv = FMT == 0 ? __builtin_amdgcn_raw_buffer_load_b32(sres, so, (kstep >> 6) * 4, 0)
                      : uint32_t(__builtin_amdgcn_raw_buffer_load_b16(sres, so, kstep >> 5, 0));
    };
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    // h of item it from the full sums `sum` (held by one wave)
    auto epilogue = [&](int it, f32x4 sum) {
      const int a = it / njb, jb = it - a * njb;
      const int e = s_tile[0][a], row0 = s_tile[1][a], rows = s_tile[2][a];
      if (FMT == 0) sum *= kNf4ScaleDown;
      // rows 0-7 of the block are gate rows, 8-15 the matching up rows: lane groups 0/1
      // hold gate values of (j0 + i, token column r), 2/3 the up values
      float up[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(sum[i], 32);
      if (g < 2 && r < rows) {
        const int32_t j0 = jb * 8 + 4 * g;
        uint32_t hv[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t jj = j0 + i;
          float gv = sum[i], uv = up[i];
          if (p.b_gu) {
            gv += p.b_gu[int64_t(e) * N + (p.interleaved ? 2 * jj : jj)];
            uv += p.b_gu[int64_t(e) * N + (p.interleaved ? 2 * jj + 1 : p.I + jj)];
          }
          const _Float16 hh = (_Float16)(p.clamped_glu ? clamped_glu(gv, uv) : swiglu(gv, uv));
          hv[i >> 1] |= uint32_t(__builtin_bit_cast(uint16_t, hh)) << (16 * (i & 1));
        }
        // I % 64 == 0: the 4 columns j0..j0+3 are in range and 8-byte aligned
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{hv[0], hv[1]}, hres,
                                              uint32_t(row0 + r) * uint32_t(p.I * 2) + 2 * j0, 0, kCohere);
      }
    };
    auto consume = [&](int it, int st, GuLoad& L) {
      const int kstep = (kp + W * st) * kStepK;
      if (it < items) {
        const int a = it / njb;
        const int row0 = s_tile[1][a], rows = s_tile[2][a];
        const int c = r < rows ? r : rows - 1;
        const int t = s_sorted[row0 + c] / k;
        const uint8_t* xr = xs + uint32_t(t) * xrow + 2 * uint32_t(kstep + 64 * g);
        u32x4 xa[8];
        const bool inK = kstep + 64 * g < p.H;  // past K: the scale is 0; read row 0 in range
#pragma unroll
        for (int iq = 0; iq < 8; ++iq)
          xa[iq] = inK ? *reinterpret_cast<const u32x4*>(xr + 16 * iq) : u32x4{0u, 0u, 0u, 0u};
        decode_step_mfma<FMT>(L.w, L.sv, xa, inK, acc);
      }
      if (st != spw - 1) return;
      if (W == 1) {
        if (it < items) epilogue(it, acc[0] + acc[1]);
      } else {
        part[tid] = acc[0] + acc[1];
        __syncthreads();
        if (kp == 0 && it < items) {
          f32x4 sum = part[tid];
          for (int w = 1; w < W; ++w) sum += part[tid + 64 * w];
          epilogue(it, sum);
        }
        __syncthreads();
      }
      acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // step sequence of this wave: items it = blockIdx.x * ipp + slot + m * G * ipp, each with
    // steps st = 0 .. spw-1; the loop runs over whole passes so every wave of the workgroup
    // reaches the same LDS barriers
    const int npass = (items - int(blockIdx.x) * ipp + G * ipp - 1) / (G * ipp);
    const int nsteps = npass > 0 ? npass * spw : 0;
    auto item_of = [&](int q) { return int(blockIdx.x) * ipp + slot + (q / spw) * G * ipp; };
    // ring of 4 register sets: the loads of steps q + 1 .. q + 3 are in flight while step q
    // is computed
    GuLoad R0, R1, R2, R3;
    auto issue_q = [&](int q, GuLoad& L) {
      if (q < nsteps) issue(item_of(q), q % spw, L);
    };
    issue_q(0, R0);
    issue_q(1, R1);
    issue_q(2, R2);
    for (int q = 0; q < nsteps; q += 4) {
      issue_q(q + 3, R3);
      consume(item_of(q), q % spw, R0);
      if (q + 1 >= nsteps) break;
      issue_q(q + 4, R0);
      consume(item_of(q + 1), (q + 1) % spw, R1);
      if (q + 2 >= nsteps) break;
      issue_q(q + 5, R1);
      consume(item_of(q + 2), (q + 2) % spw, R2);
      if (q + 3 >= nsteps) break;
      issue_q(q + 6, R2);
      consume(item_of(q + 3), (q + 3) % spw, R3);
    }
  }

  // ---- down phase layout (the same in every workgroup): column blocks of 16 outputs, the
  // tiles cut into ntg groups so that there are about as many items as workgroups
  const int nseg2 = (p.I + kStepK - 1) / kStepK;
  const int nblk = (p.H + 15) / 16;
  int tpg = (ntiles * nblk + G - 1) / G;  // tiles per group
  tpg = tpg < 1 ? 1 : tpg;
  int ntg = (ntiles + tpg - 1) / tpg;
  if (ntg > kDecMaxTG) {
    ntg = kDecMaxTG;
    tpg = (ntiles + ntg - 1) / ntg;
  }
  const int items2 = nblk * ntg;
  const uint32_t kb2 = uint32_t(p.I >> 1);
  const uint32_t nbs2 = FMT == 0 ? uint32_t(p.I >> 6) * 4 : uint32_t(p.I >> 5);
  // unit u of item (cb, grp): tile grp * tpg + u / nseg2, K step u % nseg2
  auto unit_count = [&](int grp) {
    const int t0 = grp * tpg;
    const int nt = ntiles - t0 < tpg ? ntiles - t0 : tpg;
    return nt * nseg2;
  };
  auto load_unit = [&](int cb, int grp, int u, DnUnit& U) {
    const int a = grp * tpg + u / nseg2, seg = u % nseg2;
    const int e = s_tile[0][a];
    const int n0 = cb * 16;
    const uint32_t row = uint32_t(n0 + r < p.H ? n0 + r : p.H - 1);
    const __amdgpu_buffer_rsrc_t wres = rsrc(p.w_dn + int64_t(e) * p.H * kb2, uint32_t(p.H) * kb2);
    const __amdgpu_buffer_rsrc_t sres =
        rsrc(reinterpret_cast<const uint8_t*>(p.s_dn) + int64_t(e) * p.H * nbs2, uint32_t(p.H) * nbs2);
    const uint32_t wo = row * kb2 + 32 * g;
    const uint32_t so = row * nbs2 + (FMT == 0 ? 4 * g : 2 * g);
    const int kstep = seg * kStepK;
    U.w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, wo, kstep >> 1, 0));
    U.w[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, wo + 16, kstep >> 1, 0));
    U.sv = FMT == 0 ? __builtin_amdgcn_raw_buffer_load_b32(sres, so, (kstep >> 6) * 4, 0)
                    : uint32_t(__builtin_amdgcn_raw_buffer_load_b16(sres, so, kstep >> 5, 0));
  };

  // ---- grid barrier.  h is stored device-coherently; its stores are complete (vmcnt 0) in
  // every wave before the workgroup arrives.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __builtin_amdgcn_s_barrier();
  const int q = int(blockIdx.x) % kDecGroups;
  const int ngrp = G < kDecGroups ? G : kDecGroups;
  if (tid == 0) {
    const uint32_t gsize = uint32_t((G - 1 - q) / kDecGroups + 1);  // workgroups with this residue
    const uint32_t o = __hip_atomic_fetch_add(&p.ctl[kCtlGrp + 16 * q], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (o == gsize - 1) {
      const uint32_t o2 = __hip_atomic_fetch_add(&p.ctl[kCtlTop], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (o2 == uint32_t(ngrp) - 1)
        for (int qq = 0; qq < ngrp; ++qq)
          __hip_atomic_store(&p.ctl[kCtlGo + 16 * qq], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // the first down unit's weights do not depend on h: load them while the barrier is pending
  DnUnit pre;
  const int it0 = int(blockIdx.x);
  const bool have_pre = it0 < items2 && wave < unit_count(it0 % ntg);
  if (have_pre) load_unit(it0 / ntg, it0 % ntg, wave, pre);
  if (tid == 0) {
    int spins = 0;
    while (__hip_atomic_load(&p.ctl[kCtlGo + 16 * q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      if (spins >= p.spin_limit) {
        __hip_atomic_fetch_or(&p.ctl[kCtlGaveUp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      ++spins;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __builtin_amdgcn_s_barrier();

  // ---- down + weighted combine -> column-block sums -> out
  {
    const __amdgpu_buffer_rsrc_t hres = rsrc(p.h, uint32_t(int64_t(S) * p.I * 2));
    const __amdgpu_buffer_rsrc_t pres = rsrc(p.part, uint32_t(nblk) * kDecMaxTG * kDecMaxT * 16 * 4);
    for (int it = int(blockIdx.x); it < items2; it += G) {
      const int cb = it / ntg, grp = it - cb * ntg;
      const int n0 = cb * 16;
      const int nu = unit_count(grp);
      float acc_t[kDecMaxT][4];
#pragma unroll
      for (int t = 0; t < kDecMaxT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_t[t][i] = 0.f;
      for (int u = wave; u < nu; u += kWaves) {
        DnUnit U;
        if (it == it0 && u == wave) {
          U = pre;
        } else {
          load_unit(cb, grp, u, U);
        }
        const int a = grp * tpg + u / nseg2, seg = u % nseg2;
        const int e = s_tile[0][a], row0 = s_tile[1][a], rows = s_tile[2][a];
        const int c = r < rows ? r : rows - 1;
        const int kstep = seg * kStepK;
        const uint32_t ao = uint32_t(row0 + c) * uint32_t(p.I * 2) + 128 * g;
        u32x4 ha[8];
#pragma unroll
        for (int iq = 0; iq < 8; ++iq)
          ha[iq] = __builtin_bit_cast(u32x4,
                                      __builtin_amdgcn_raw_buffer_load_b128(hres, ao + 16 * iq, 2 * kstep, kCohere));
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        decode_step_mfma<FMT>(U.w, U.sv, ha, int64_t(64 * g) < int64_t(p.I) - kstep, acc);
        f32x4 d = acc[0] + acc[1];
        if (FMT == 0) d *= kNf4ScaleDown;
        if (seg == 0 && p.b_dn) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = n0 + 4 * g + i;
            d[i] += n < p.H ? p.b_dn[int64_t(e) * p.H + n] : 0.0f;
          }
        }
        if (r < rows) {
          const int slot = s_sorted[row0 + r];
          const int t = slot / k;
          const float wt = s_w[slot];
#pragma unroll
          for (int tt = 0; tt < kDecMaxT; ++tt)
            if (tt == t) {
#pragma unroll
              for (int i = 0; i < 4; ++i) acc_t[tt][i] += wt * d[i];
            }
        }
      }
      // per token: the 16 lanes of a row group hold different slots; add them (fixed order)
#pragma unroll
      for (int tt = 0; tt < kDecMaxT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = acc_t[tt][i];
          v += __shfl_xor(v, 1);
          v += __shfl_xor(v, 2);
          v += __shfl_xor(v, 4);
          v += __shfl_xor(v, 8);
          if (r == 0 && tt < T) red[wave][g][tt][i] = v;
        }
      __syncthreads();
      // this item's sums over its tiles -> part[cb][grp] (device-coherent stores)
      if (tid < T * 16) {
        const int t = tid >> 4, rr = tid & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) sum += red[w][rr >> 2][t][rr & 3];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), pres,
                                              uint32_t(((cb * kDecMaxTG + grp) * kDecMaxT + t) * 16 + rr) * 4, 0,
                                              kCohere);
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      __syncthreads();
      if (tid == 0) {
        const uint32_t o = __hip_atomic_fetch_add(&p.ctl[kCtlCols + cb], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        s_last = o == uint32_t(ntg) - 1;
        if (s_last) __hip_atomic_store(&p.ctl[kCtlCols + cb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (s_last && tid < T * 16) {  // every group of these columns is stored: add them in order
        const int t = tid >> 4, rr = tid & 15;
        float sum = 0.f;
        for (int gg = 0; gg < ntg; ++gg)
          sum += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              pres, uint32_t(((cb * kDecMaxTG + gg) * kDecMaxT + t) * 16 + rr) * 4, 0, kCohere));
        const int n = n0 + rr;
        if (n < p.H) {
          if (p.out_f32) p.out_f32[int64_t(t) * p.H + n] = sum;
          p.out[int64_t(t) * p.H + n] = f32_to_bf16_rne(sum);
        }
      }
      __syncthreads();
    }
  }

  // ---- exit: the last workgroup resets the barrier words for the next call
  __syncthreads();
  if (tid == 0) {
    const uint32_t d = __hip_atomic_fetch_add(&p.ctl[kCtlDepart], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == uint32_t(G) - 1) {
      const uint32_t gave_up = __hip_atomic_load(&p.ctl[kCtlGaveUp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p.status) *p.status = gave_up ? 1 : 0;
      for (int qq = 0; qq < kDecGroups; ++qq) {
        __hip_atomic_store(&p.ctl[kCtlGrp + 16 * qq], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&p.ctl[kCtlGo + 16 * qq], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(&p.ctl[kCtlTop], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.ctl[kCtlGaveUp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.ctl[kCtlDepart], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}


// A list of 16-row tiles: the tile array, its device-side count, a host-side bound, and
// whether these are the tail tiles of the MFMA-tile path.
struct TileList {
  const int32_t* tiles;
  const int32_t* n;
  int64_t max_tiles;
  bool tails;
};

template <int FMT, bool GU, int RB, bool SLOT>
hipError_t launch_rb(const GemvArgs& g, const TileList& tl, const MoeLaunch& L, void* out,
                     int64_t n_out, int64_t wgs, hipStream_t stream) {
  constexpr int64_t kPerItem = kWaves * RB * (GU ? 8 : 16);  // output rows (gate_up: j) per item
  GemvArgs a = g;
  a.n_rblocks = int((n_out + kPerItem - 1) / kPerItem);
  const int64_t max_items = tl.max_tiles * a.n_rblocks;
  int64_t grid = wgs < max_items ? wgs : max_items;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((moe_gemv_kernel<FMT, GU, RB, SLOT>), dim3(unsigned(grid)), dim3(kThreads),
                     0, stream, a, tl.tiles, tl.n, L.tok, out);
  return hipGetLastError();
}

// One row block per wave.  Two (one activation fragment feeding two row blocks) were measured
// slower on every decode layer tried, by 2-20 % for gate_up: 128 experts of 1536 x 2048 at 16
// and 64 tokens, 8 experts of 28672 x 4096 at 4 to 32 tokens.  The item count uses the
// host-side upper bound of the tile count (a device value).
template <int FMT, bool GU, bool SLOT>
hipError_t launch_stage(const GemvArgs& g, const TileList& tl, const MoeLaunch& L, void* out,
                        int64_t n_out, hipStream_t stream) {
  const int64_t wgs = int64_t(kWgPerCu) * cu_count();
  // tail tiles are few and their bound loose: one row block per wave gives the most items
  if (tl.tails) return launch_rb<FMT, GU, 1, SLOT>(g, tl, L, out, n_out, wgs, stream);
  const int64_t per_block = GU ? 8 : 16;
  auto items = [&](int64_t rb) {
    const int64_t per_item = kWaves * rb * per_block;
    return tl.max_tiles * ((n_out + per_item - 1) / per_item);
  };
  if (SLOT || 3 * items(1) >= wgs)
    return launch_rb<FMT, GU, 1, SLOT>(g, tl, L, out, n_out, wgs, stream);
  // fewer items than a third of the resident workgroups (measured on a 128-expert layer,
  // 512 resident workgroups: 96 and 128 items 15-20 % faster than the streaming kernel, 192
  // items 10 % slower): K split over W waves per 16-row block, W the smallest power of two
  // >= the K steps (at most the 8 waves)
  GemvArgs a = g;
  const int64_t nseg = (g.K + kStepK - 1) / kStepK;
  a.ks_waves = nseg > 4 ? 8 : nseg > 2 ? 4 : nseg > 1 ? 2 : 1;
  const int64_t blocks_per_wg = kWaves / a.ks_waves;
  a.n_rblocks = int(((n_out + per_block - 1) / per_block + blocks_per_wg - 1) / blocks_per_wg);
  const int64_t grid = tl.max_tiles * a.n_rblocks;
  if (grid < 1 || grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((moe_gemv_ks_kernel<FMT, GU>), dim3(unsigned(grid)), dim3(kThreads), 0, stream,
                     a, tl.tiles, tl.n, L.tok, out);
  return hipGetLastError();
}

}  // namespace

int cu_count() {
  static std::atomic<int> cached[64];  // 0 = not read yet; the value read is idempotent
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// SLOT: activations and h in the slot order of the NF4 MFMA-tile path (tail tiles of that
// path); otherwise natural order.
template <int FMT, bool SLOT>
static hipError_t launch_gemv_fmt(const MoeLaunch& L, const TileList& tl, hipStream_t stream,
                                  int stage) {
  GemvArgs g{};
  g.I = L.I;
  g.T = L.T;
  g.S = L.T * L.k;
  g.clamped_glu = L.clamped_glu;
  g.interleaved = L.interleaved;
  g.bias = stage == 0 ? L.b_gu : L.b_dn;
  if (stage == 0) {
    g.a = L.x16;
    g.wq = L.w_gu;
    g.sc = L.s_gu;
    g.K = L.H;
    g.N = 2 * L.I;
    return launch_stage<FMT, true, SLOT>(g, tl, L, L.h, L.I, stream);
  }
  g.a = L.h;
  g.wq = L.w_dn;
  g.sc = L.s_dn;
  g.K = L.I;
  g.N = L.H;
  if (L.atomic_combine && tl.tails) {  // the MFMA path's accumulator (see launch_fmt)
    g.comb = L.out_f32 ? L.out_f32 : L.y;
    g.slots = L.slots;
    g.topk_w = L.topk_w;
  }
  return launch_stage<FMT, false, SLOT>(g, tl, L, L.y, L.H, stream);
}

// Single-launch decode step: a grid of co-resident workgroups (at most what the device holds at
// once, so the grid barrier cannot wait on a workgroup that is not running).
template <int FMT, int PL>
static hipError_t launch_decode_pl(const DecodeStepArgs& a, int64_t items, hipStream_t stream) {
  // x in LDS: T rows of 2H + 16 bytes (at most 64 KB + padding); the occupancy is taken at the
  // largest size, once per device, with the dynamic-LDS limit raised for it
  constexpr size_t kMaxXs = size_t(kDecXChunks) * kThreads * 16 + kDecMaxT * 16;
  const size_t lds = size_t(a.T) * size_t(2 * a.H + 16);
  static std::atomic<int> occ_cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int occ = occ_cache[dev].load(std::memory_order_relaxed);
  if (occ == 0) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(moe_decode_step_kernel<FMT, PL>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxXs)) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, moe_decode_step_kernel<FMT, PL>, kThreads, kMaxXs) !=
            hipSuccess || occ <= 0)
      return hipErrorInvalidValue;
    occ_cache[dev].store(occ, std::memory_order_relaxed);
  }
  int64_t grid = int64_t(occ < 2 ? occ : 2) * cu_count();
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((moe_decode_step_kernel<FMT, PL>), dim3(unsigned(grid)), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

size_t decode_ctl_bytes(int64_t H) {
  const size_t words = size_t(kCtlCols) + size_t((H + 15) / 16);
  return (words * 4 + 255) / 256 * 256;
}

hipError_t launch_decode_step(const DecodeLaunch& L, hipStream_t stream) {
  DecodeStepArgs a{};
  a.E = int32_t(L.E);
  a.H = int32_t(L.H);
  a.I = int32_t(L.I);
  a.T = int32_t(L.T);
  a.k = L.k;
  a.renorm = L.renorm;
  a.clamped_glu = L.clamped_glu;
  a.interleaved = L.interleaved;
  a.spin_limit = L.spin_limit;
  a.logits = L.logits;
  a.x = L.x;
  a.w_gu = L.w_gu;
  a.s_gu = L.s_gu;
  a.w_dn = L.w_dn;
  a.s_dn = L.s_dn;
  a.b_gu = L.b_gu;
  a.b_dn = L.b_dn;
  a.ids_out = L.ids;
  a.w_out = L.w;
  a.offsets_out = L.offsets;
  a.slots_out = L.slots;
  a.out = L.out;
  a.out_f32 = L.out_f32;
  a.h = L.h;
  a.part = L.part;
  a.ctl = L.ctl;
  a.status = L.status;
  const int64_t S = L.T * L.k;
  const int64_t active = L.E < S ? L.E : S;
  const int64_t items1 = active * ((L.I + 7) / 8), items2 = (L.H + 15) / 16;
  const int64_t items = items1 > items2 ? items1 : items2;
  const bool nf4 = L.fmt == 0;
  if (L.E <= 64) return nf4 ? launch_decode_pl<0, 1>(a, items, stream) : launch_decode_pl<1, 1>(a, items, stream);
  if (L.E <= 128) return nf4 ? launch_decode_pl<0, 2>(a, items, stream) : launch_decode_pl<1, 2>(a, items, stream);
  if (L.E <= 256) return nf4 ? launch_decode_pl<0, 4>(a, items, stream) : launch_decode_pl<1, 4>(a, items, stream);
  return nf4 ? launch_decode_pl<0, kMaxExpertsPerLane>(a, items, stream)
             : launch_decode_pl<1, kMaxExpertsPerLane>(a, items, stream);
}

hipError_t launch_gemv(const MoeLaunch& L, hipStream_t stream, int stage) {
  const TileList tl{L.tiles, L.n_mtiles, L.max_mtiles, false};
  return L.fmt == 0 ? launch_gemv_fmt<0, false>(L, tl, stream, stage)
                    : launch_gemv_fmt<1, false>(L, tl, stream, stage);
}

hipError_t launch_gemv_tails(const MoeLaunch& L, hipStream_t stream, int stage) {
  // this GEMM's tail tiles: count and first index at n_mtiles[4 + 2 * stage]
  const TileList tl{L.tiles + 4 * L.max_mtiles, L.n_mtiles + 4 + 2 * stage, L.max_stiles, true};
  return L.fmt == 0 ? launch_gemv_fmt<0, true>(L, tl, stream, stage)
                    : launch_gemv_fmt<1, false>(L, tl, stream, stage);
}

}  // namespace e4b
