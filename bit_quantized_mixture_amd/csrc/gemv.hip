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
    float* y = reinterpret_cast<float*>(pt.out) + int64_t(st.row0 + r) * p.N;
    const int32_t n0 = blk * 16 + 4 * g;
    if (n0 < int32_t(p.N)) {  // N % 64 == 0
      f32x4 v = acc;
      if (p.bias) v += *reinterpret_cast<const f32x4*>(p.bias + int64_t(st.e) * p.N + n0);
      *reinterpret_cast<f32x4*>(y + n0) = v;
    }
  }
}

template <int FMT, bool GU, int RB, bool SLOT>
__global__ void __launch_bounds__(kThreads)
    moe_gemv_kernel(GemvArgs p, const int32_t* __restrict__ tiles,
                    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ tok,
                    void* __restrict__ out) {
  const Ptrs pt{tiles, tok, out};
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

  if (FMT == 0) nf4_lut_fill(lut, tid, kThreads);

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
  return launch_stage<FMT, false, SLOT>(g, tl, L, L.y, L.H, stream);
}

hipError_t launch_gemv(const MoeLaunch& L, hipStream_t stream, int stage) {
  const TileList tl{L.tiles, L.n_mtiles, L.max_mtiles, false};
  return L.fmt == 0 ? launch_gemv_fmt<0, false>(L, tl, stream, stage)
                    : launch_gemv_fmt<1, false>(L, tl, stream, stage);
}

hipError_t launch_gemv_tails(const MoeLaunch& L, hipStream_t stream, int stage) {
  const TileList tl{L.tiles + 4 * L.max_mtiles, L.n_mtiles + 1, L.max_stiles, true};
  return L.fmt == 0 ? launch_gemv_fmt<0, true>(L, tl, stream, stage)
                    : launch_gemv_fmt<1, false>(L, tl, stream, stage);
}

}  // namespace e4b
