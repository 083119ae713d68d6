// Grouped expert GEMMs of the MoE forward, computed on 4-bit packed weights.
//
// grouped-nf4-gemm 0.25.0 project description, opening section: one launch covers every
// active expert; codes are decoded through a table in registers, scaled per block,
// accumulated in fp32, and only the output is rounded to bf16; no dequantised weight copy
// exists.  bitsandbytes pull request #1984, Design: the expert is a SwiGLU MLP on the fused
// gate_up / down stacks.
//
// Pipeline (all on the caller's stream, no device->host read-back):
//   convert_x     x bf16 [T,H] -> fp16 (exact in fp16 range), k-slot order of the format;
//                 its last workgroup also runs build_tiles: per expert, BM-row tiles of the
//                 expert-major slot order, and 16-row tail tiles for a short last piece
//   gemm<GU>      h[p, j] = silu(x_t . Wg[e,j]) * (x_t . Wu[e,j]) for the rows p of a tile
//                 (tail tiles: the streaming kernel of gemv.hip, same operand order)
//   gemm<DN>      y[p, n] = h[p] . Wd[e,n]   (sorted row p)
//   combine       out[t] = sum_j topk_w[s] * y[inv[s]], s = t*k+j  (fixed order) -> fp32, bf16
//                 (RNE); inv (slot -> sorted row) is written by convert_x
//   (atomic combine: gemm<DN> adds topk_w[s] * y straight into a [T, H] fp32 accumulator that
//   convert_x cleared, and the last pass only rounds it to bf16)
//
// Tile structure of gemm: a workgroup owns BM rows of one expert and WAVES*64 weight rows
// (GU: 32 gate + 32 matching up rows per wave, so SwiGLU is formed in registers).  Each
// wave owns all BM rows x 64 weight rows and keeps its accumulators in registers
// (v_mfma_f32_32x32x16_f16).  The activation tile (BM x 64 fp16 per K step) comes through a
// 4-stage LDS ring filled by direct buffer->LDS loads and is shared by the waves.  The
// packed weight rows of each wave come through a wave-private LDS tile, one 256-wide K group
// at a time (also by direct buffer->LDS copies); each lane reads its 64-byte span of its rows
// from there into registers and decodes it in registers.
#include <type_traits>

#include "e4b_device.h"
#include "e4b_internal.h"

namespace e4b {

constexpr int kBK = 64;  // K per main-loop step: one NF4 block, two MXFP4 blocks

// LDS activation tile: BM rows x 64 fp16 (128 B), no padding.  The 16-byte chunk holding
// elements [8c, 8c+8) of row r sits at chunk position c ^ (r & 7) ^ ((r >> 3) & 1).  An MFMA
// operand read touches one chunk index c in consecutive rows; with 64 four-byte banks a
// 16-lane phase covers rows r0..r0+15, whose bank groups 8*(r&1) + position are then all
// distinct (the (r >> 3) term separates rows r and r+8, which share r & 7).
__device__ __forceinline__ int lds_chunk(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

struct GemmArgs {
  const _Float16* a;       // GU: x16 [T, K]; DN: h [S, K]
  const uint8_t* wq;       // packed weights [E, N, K/2]
  const void* sc;          // NF4 float [E, N, K/64] | MXFP4 uint8 [E, N, K/32]
  const int32_t* tiles;    // [max_mtiles, 4]: expert, first sorted row, rows, 0
  const int32_t* n_mtiles;
  const int32_t* slots;    // sorted slots [S]
  void* out;               // GU: h fp16 [S, I]; DN: y float [S, N]
  int64_t K;
  int64_t N;               // weight rows per expert (2I for GU, H for DN)
  int64_t I;
  int64_t T;               // tokens (rows of x16; h has T * k_top rows)
  int32_t k_top;
  int32_t n_ntiles;
  const float* bias;       // nullable [E, N]: added to the products (GU before the activation)
  int32_t clamped_glu;     // GU activation: 0 silu(G) * U, 1 clamped GLU
  int32_t interleaved;     // GU rows: 0 halves (gate j, up I + j), 1 interleaved (2j, 2j + 1)
  int32_t xcd_order;       // 1: workgroup ids dealt to the 8 XCDs in contiguous chunks
  const float* topk_w;     // DN with comb: routing weight of each slot [T * k_top]
  float* comb;             // DN: nullable [T, N] float32; when set, topk_w[slot] * y is added
                           // there atomically instead of y being stored
};


template <int FMT, bool GU, int BM, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) moe_gemm_kernel(GemmArgs p) {
  constexpr int ST = 4;  // pipeline depth
  constexpr int RB = BM / 32;
  // One LDS object holds the activation ring lds[ST][BM][kBK] and, after it, the weight rows
  // of one 256-wide K group (128 packed bytes per row; wave w's 64 rows at w * 8 KB).
  constexpr int kWRowBytes = 128;
  constexpr int kRingBytes = ST * BM * kBK * 2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRingBytes + WAVES * 64 * kWRowBytes];
  auto lds = reinterpret_cast<_Float16(*)[BM][kBK]>(smem);
  uint8_t* const wl = smem + kRingBytes;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  // Workgroups go to the XCDs round robin (id % 8).  With xcd_order, XCD x takes a
  // contiguous chunk of the real (row tile, column tile) ids, in order, instead.
  int bid = int(blockIdx.x);
  if (p.xcd_order) {
    const int G = *p.n_mtiles * p.n_ntiles;
    if (bid >= G) return;
    const int q = G >> 3, r = G & 7, x = bid & 7;
    bid = x * q + (x < r ? x : r) + (bid >> 3);
  }
  const int nt = bid % p.n_ntiles;
  const int mt = bid / p.n_ntiles;
  if (mt >= *p.n_mtiles) return;
  const int e = p.tiles[4 * mt], row0 = p.tiles[4 * mt + 1], rows = p.tiles[4 * mt + 2];

  // ---- this lane's two weight rows (fragment f = 0, 1)
  int64_t nrow[2];
  bool nvalid[2];
  if (GU) {
    const int64_t j = int64_t(nt) * (WAVES * 32) + wave * 32 + col;
    nvalid[0] = nvalid[1] = j < p.I;
    const int64_t jc = j < p.I ? j : p.I - 1;
    nrow[0] = p.interleaved ? 2 * jc : jc;
    nrow[1] = p.interleaved ? 2 * jc + 1 : p.I + jc;
  } else {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int64_t n = int64_t(nt) * (WAVES * 64) + wave * 64 + f * 32 + col;
      nvalid[f] = n < p.N;
      nrow[f] = n < p.N ? n : p.N - 1;
    }
  }
  // ---- K order.  K is cut into groups of 256 (4 steps of 64).  Inside group G, step j,
  // lane half h supplies K elements [256G + 128h + 32j, +32): half h owns a contiguous
  // 64-byte span of its weight row per group, so a group needs one pair of scale loads.  The
  // activation tile of step j is staged in the same order (chunk c of a row holds K
  // 256G + 128(c>>2) + 32j + 8(c&3)), so the MFMA k-slots of both operands agree.  The last
  // group may be partial: out-of-range pieces are loaded from a clamped address and get a
  // zero scale, so they contribute exactly 0.
  const int64_t kbytes = p.K >> 1;
  const int nk = int(p.K / kBK);          // real 64-wide steps (= NF4 blocks per row)
  const int ng = (nk + 3) >> 2;           // 256-wide groups
  const float* srow_nf4[2];
  const uint16_t* srow_mx[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int64_t r = int64_t(e) * p.N + nrow[f];
    srow_nf4[f] = reinterpret_cast<const float*>(p.sc) + r * nk;
    srow_mx[f] = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(p.sc) + r * (2 * nk));
  }
  // ---- weight staging: a group's rows come into LDS by direct buffer->LDS copies, 8 rows x
  // 128 contiguous bytes per wave instruction (instead of 16-byte register loads that each
  // touch 32 rows).  Copy i of wave w fills wave-local tile rows 8i .. 8i+7; lane l lands in
  // row 8i + l/8, slot l%8, and brings the 16-byte piece (l%8) ^ ((row >> 1) & 7) of that
  // row.  A fragment read (16 lanes, 16 consecutive rows, one piece) then meets 16 distinct
  // (row parity, slot) pairs: with 128-byte rows on 64 four-byte banks, 16 distinct bank
  // groups.  Tile row rr = 32f + c holds the weight row of lane c, fragment f.
  const __amdgpu_buffer_rsrc_t wres =
      buffer_rsrc(p.wq + int64_t(e) * p.N * kbytes, uint32_t(p.N * kbytes));
  uint32_t wrow_off[8];   // row start (bytes from the expert's stack)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = 8 * i + (lane >> 3), f = rr >> 5, c = rr & 31;
    int64_t row;
    if (GU) {
      const int64_t j = int64_t(nt) * (WAVES * 32) + wave * 32 + c;
      const int64_t jc = j < p.I ? j : p.I - 1;
      row = f == 0 ? (p.interleaved ? 2 * jc : jc) : (p.interleaved ? 2 * jc + 1 : p.I + jc);
    } else {
      const int64_t n = int64_t(nt) * (WAVES * 64) + wave * 64 + f * 32 + c;
      row = n < p.N ? n : p.N - 1;
    }
    wrow_off[i] = uint32_t(row) * uint32_t(kbytes);
  }
  // (rr >> 1) & 7 = (4i + lane / 16) & 7: the piece depends on i only through its parity
  uint32_t wpiece[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) wpiece[par] = 16u * uint32_t((lane & 7) ^ ((4 * par + (lane >> 4)) & 7));
  const uint32_t wlast = uint32_t(kbytes - 16);
  uint8_t* wl_wave = wl + wave * (64 * kWRowBytes);

  // ---- activation staging: global -> LDS directly (global_load_lds_dwordx4).  One
  // instruction of a wave fills 8 consecutive tile rows (64 lanes x 16 B); lane i writes
  // LDS chunk position i & 7 of row i >> 3, so it fetches the logical chunk that belongs
  // there.  Offsets are in fp16 elements from p.a (the ABI keeps them below 2^31).
  constexpr int ROWS_W = BM / WAVES;      // tile rows staged by this wave
  constexpr int NLD = ROWS_W / 8;         // DMA instructions per wave per K-step
  static_assert(ROWS_W % 8 == 0, "DMA row groups");
  uint32_t arow_off[NLD];                 // row start (elements)
  uint32_t apart = 0;                     // this lane's chunk offset inside a step (elements)
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int r = wave * ROWS_W + 8 * j + (lane >> 3);
    const int rr = r < rows ? r : rows - 1;
    const int64_t src = GU ? int64_t(p.slots[row0 + rr] / p.k_top) : int64_t(row0 + rr);
    arow_off[j] = uint32_t(src * p.K);
  }
  // the logical chunk differs per row only through lds_chunk's row terms; rows of one DMA
  // instruction are 8*j + (lane >> 3), so (r & 7) = lane >> 3 and (r >> 3) & 1 = parity of
  // (wave*ROWS_W/8 + j): two variants of the chunk offset per lane.
  uint32_t apart2[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int c = (lane & 7) ^ (lane >> 3) ^ par;
    apart2[par] = uint32_t(128 * (c >> 2) + 8 * (c & 3));
  }
  (void)apart;
  const uint32_t kmax_a = uint32_t(p.K - 8);

  f32x16 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    acc[rb][0] = f32x16{};
    acc[rb][1] = f32x16{};
  }

  // ---- software pipeline.  Step kb (= 4G + j) reads LDS buffer j; the activation DMA of
  // step kb + ST - 1 is issued at the top of step kb.  At the top of group G the scales of
  // group G + 1 are loaded into the "next" registers and its weight rows copied into the
  // weight tile, which step 3 of group G reads into the "next" registers.  The step count
  // is padded to whole groups.
  u32x4 bg[2][2][4];   // [cur/next][fragment][step in group]
  // Raw scale words of a half's span (loaded values are only combined where they are used,
  // so no wait is forced at load time).  NF4: absmax of blocks b0, b0+1 (float bits);
  // MXFP4: the two 16-bit words holding the e8m0 bytes of 32-blocks b0..b0+3.
  uint32_t sraw[2][2][2];
  int gld[2];          // group index loaded into each slot (for validity)

  const __amdgpu_buffer_rsrc_t ares =
      buffer_rsrc(p.a, uint32_t((GU ? int64_t(p.T) : int64_t(p.T) * p.k_top) * p.K * 2));
  auto stage_a = [&](int kb, int buf) {
    const uint32_t kg = uint32_t(256 * (kb >> 2) + 32 * (kb & 3));
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int par = ((wave * ROWS_W) / 8 + j) & 1;
      uint32_t ko = kg + apart2[par];
      ko = ko < kmax_a ? ko : kmax_a;
      lds_dma16_buf(ares, 2 * (arow_off[j] + ko), &lds[buf][wave * ROWS_W + 8 * j][0]);
    }
  };
  // The weight rows of group G into this wave's LDS tile (8 copies).  A piece past the end
  // of its row (only in a partial last group) is fetched from the row's last 16 bytes
  // instead; its scale is 0, so it contributes exactly 0.
  auto dma_weights = [&](int G) {
    const uint32_t go = 128u * uint32_t(G);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      typedef __attribute__((address_space(3))) void lds_void;
      uint32_t o = go + wpiece[i & 1];
      o = o < wlast ? o : wlast;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void*)(wl_wave + 1024 * i), 16,
                                               int(wrow_off[i] + o), 0, 0, 0);
    }
  };
  auto read_weights = [&](int slot) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int rr = 32 * f + col;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bg[slot][f][j] = *reinterpret_cast<const u32x4*>(
            wl_wave + rr * kWRowBytes + 16 * ((4 * half + j) ^ ((rr >> 1) & 7)));
    }
  };
  // Scales of group G into register slot `slot`.
  auto load_group = [&](int G, int slot) {
    gld[slot] = G;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (FMT == 0) {
        const int b0 = 4 * G + 2 * half;
        sraw[slot][f][0] = __float_as_uint(srow_nf4[f][b0 < nk ? b0 : nk - 1]);
        sraw[slot][f][1] = __float_as_uint(srow_nf4[f][b0 + 1 < nk ? b0 + 1 : nk - 1]);
      } else {
        const int b0 = 8 * G + 4 * half;  // a row has 2*nk 32-blocks
        const int i0 = b0 < 2 * nk - 2 ? b0 : 2 * nk - 2;
        const int i1 = b0 + 2 < 2 * nk - 2 ? b0 + 2 : 2 * nk - 2;
        sraw[slot][f][0] = srow_mx[f][i0 >> 1];
        sraw[slot][f][1] = srow_mx[f][i1 >> 1];
      }
    }
  };
  // Scale of step j of the group in `slot`, fragment f; zero where the step's K range of
  // this lane's half lies past the end of K.
  auto step_scale = [&](int slot, int f, int j) -> float {
    const int G = gld[slot];
    if (FMT == 0) {
      const int b = 4 * G + 2 * half + (j >> 1);
      return b < nk ? __uint_as_float(sraw[slot][f][j >> 1]) : 0.0f;
    }
    const int b = 8 * G + 4 * half + j;
    const uint32_t byte = (sraw[slot][f][j >> 1] >> (8 * (j & 1))) & 0xFFu;
    return b < 2 * nk ? e8m0_to_f32(byte) : 0.0f;
  };
  // Loads per wave: a group issues 2 x 2 scale loads and 8 weight copies; a step NLD DMA.
  constexpr int kGroupOps = 12;
  auto afrag = [&](int buf, int rb, int s) {
    const int m = 32 * rb + col;
    return *reinterpret_cast<const f16x8*>(&lds[buf][m][8 * lds_chunk(m, 4 * half + s)]);
  };

  // Decoded weight fragments of one 16-wide substep, one substep ahead of their MFMAs.
  auto decode = [&](const u32x4 (*bsl)[4], int j, int s, float sc0, float sc1, f16x8* out) {
    const float scs[2] = {sc0, sc1};
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      uint32_t d[4];
      if (FMT == 0) {
        nf4_decode8(bsl[f][j][s], d);
        const _Float16 sh = (_Float16)(scs[f] * kNf4ScaleUp);
        const f16x2 s16 = f16x2{sh, sh};
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = pk_mul_f16(d[i], s16);
      } else {
        mxfp4_decode8(bsl[f][j][s], scs[f], d);
      }
      out[f] = __builtin_bit_cast(f16x8, u32x4{d[0], d[1], d[2], d[3]});
    }
  };
  constexpr int kMfmaPerSub = 2 * RB;
  constexpr int kDecodeValu = FMT == 0 ? 58 : 12;
  constexpr int kValuPerMfma = (kDecodeValu + kMfmaPerSub - 1) / kMfmaPerSub;

  f16x8 afr[RB];
  f16x8 bcur[2], bnxt[2];
  // One step: J = position in the group (compile time) = LDS buffer.
  auto kstep = [&](int G, auto j_c) {
    constexpr int J = decltype(j_c)::value;
    constexpr int NXT = (J + ST - 1) % ST;  // buffer freed by the previous step
    const int kb = 4 * G + J;
    stage_a(kb + ST - 1, NXT);
    if (J == 0) {  // the weight tile was read into registers in step 3 of the previous group
      const int Gn = G + 1 < ng ? G + 1 : ng - 1;
      load_group(Gn, 1);
      dma_weights(Gn);
    }
    if (J == 3) read_weights(1);  // copied in step 0, landed before the barrier of step 2
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
        decode(bg[0], J, s + 1, step_scale(0, 0, J), step_scale(0, 1, J), bnxt);
      } else if (J < 3) {
        decode(bg[0], J + 1, 0, step_scale(0, 0, J + 1), step_scale(0, 1, J + 1), bnxt);
      } else {
        decode(bg[1], 0, 0, step_scale(1, 0, 0), step_scale(1, 1, 0), bnxt);
      }
      // A fragment rb is reloaded with the next substep's data right after its two MFMAs.
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afr[rb], bcur[0], acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afr[rb], bcur[1], acc[rb][1], 0, 0, 0);
        if (s < 3) afr[rb] = afrag(J, rb, s + 1);
      }
#pragma unroll
      for (int i = 0; i < kMfmaPerSub; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // VALU
        if (s < 3 && (i & 1)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      bcur[0] = bnxt[0];
      bcur[1] = bnxt[1];
    }
    // Step kb+1's DMA (every wave's) has landed; this wave's reads of buffer J are done.
    // Loads issued after DMA(kb+1): the DMA of steps kb-1 and kb, plus the group ops of
    // step 0 (issued after its DMA) while step 0 is one of those two.  In step 2 this also
    // covers the group's weight copies, read at the top of step 3.
    constexpr int kWait = 2 * NLD + (J < 2 ? kGroupOps : 0);
    static_assert(kWait < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kWait));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) afr[rb] = afrag((J + 1) % ST, rb, 0);
    if (J == 3) {
      gld[0] = gld[1];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) bg[0][f][q] = bg[1][f][q];
        sraw[0][f][0] = sraw[1][f][0];
        sraw[0][f][1] = sraw[1][f][1];
      }
    }
  };

  load_group(0, 0);
  dma_weights(0);
#pragma unroll
  for (int i = 0; i < ST - 1; ++i) stage_a(i, i);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * NLD));  // weights and DMA of step 0 landed
  __builtin_amdgcn_s_barrier();
  read_weights(0);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) afr[rb] = afrag(0, rb, 0);
  decode(bg[0], 0, 0, step_scale(0, 0, 0), step_scale(0, 1, 0), bcur);
  // the weight tile's reads are complete before step 0 refills it
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
  // A last group holding a single 64-wide step keeps its K in half 0's steps 0 and 1 (steps 2
  // and 3 would only add zero-scaled products): it runs two steps (K = 2880: 46 steps, not 48).
  const bool short_last = nk - 4 * (ng - 1) == 1;
  const int nfull = ng - (short_last ? 1 : 0);
  for (int G = 0; G < nfull; ++G) {
    kstep(G, std::integral_constant<int, 0>{});
    kstep(G, std::integral_constant<int, 1>{});
    kstep(G, std::integral_constant<int, 2>{});
    kstep(G, std::integral_constant<int, 3>{});
  }
  if (short_last) {
    kstep(nfull, std::integral_constant<int, 0>{});
    kstep(nfull, std::integral_constant<int, 1>{});
  }
  // drain the DMA issued past the last step before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

  // ---- epilogue.  Accumulator element r of a 32x32 block: row 8*(r/4) + 4*half + r%4,
  // column = col.  The plain SwiGLU / unbiased forms are kept as their own branches: the
  // stores then take their data straight from the accumulators.  NF4 sums carry the 2^8 of
  // the scale shift (kNf4ScaleUp), taken out here.
  if (FMT == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      acc[rb][0] *= kNf4ScaleDown;
      acc[rb][1] *= kNf4ScaleDown;
    }
  }
  if (GU) {
    if (!nvalid[0]) return;
    const int64_t j = int64_t(nt) * (WAVES * 32) + wave * 32 + col;
    _Float16* hout = reinterpret_cast<_Float16*>(p.out);
    const int64_t pos = act_pos<FMT>(j);
    if (rows == BM && (RB <= 4 || (!p.bias && !p.clamped_glu))) {
      // a full tile: buffer stores with a per-lane offset fixed for the whole epilogue and a
      // wave-uniform offset per accumulator row, so no per-store address arithmetic runs.
      // One copy of the store loop per activation form keeps the selection out of the loop;
      // 256-row tiles keep the guarded loop below for the bias and clamped-GLU forms, since
      // further copies there take the kernel past its 256 VGPRs.
      const uint32_t vo = uint32_t(4 * half * p.I + pos) * 2u;
      auto store_full = [&](auto act) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const __amdgpu_buffer_rsrc_t hres =
              buffer_rsrc(hout + (int64_t(row0) + 32 * rb) * p.I, uint32_t(32 * p.I * 2));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t so = uint32_t((8 * (r >> 2) + (r & 3)) * p.I) * 2u;
            const _Float16 hv = (_Float16)act(acc[rb][0][r], acc[rb][1][r]);
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, hv), hres, int(vo), int(so), 0);
          }
        }
      };
      if (!p.bias && !p.clamped_glu) {
        store_full([](float g, float u) { return swiglu(g, u); });
      } else if constexpr (RB <= 4) {
        const float bg = p.bias ? p.bias[int64_t(e) * p.N + nrow[0]] : 0.0f;
        const float bu = p.bias ? p.bias[int64_t(e) * p.N + nrow[1]] : 0.0f;
        if (p.clamped_glu)
          store_full([=](float g, float u) { return clamped_glu(g + bg, u + bu); });
        else
          store_full([=](float g, float u) { return swiglu(g + bg, u + bu); });
      }
    } else if (!p.bias && !p.clamped_glu) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (row < rows) {
            const float g = acc[rb][0][r];
            const float u = acc[rb][1][r];
            hout[int64_t(row0 + row) * p.I + pos] = (_Float16)swiglu(g, u);
          }
        }
      }
    } else {
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
            hout[int64_t(row0 + row) * p.I + pos] = (_Float16)hv;
          }
        }
      }
    }
  } else if (p.comb) {
    // weighted scatter-combine: row p of the tile belongs to slot s = slots[row0 + p], token
    // s / k; its products go to comb[token] scaled by topk_w[s].  The token offsets and
    // weights of the tile's rows are staged in LDS (the activation ring is free once every
    // wave has left the main loop), then read back with one address per lane half.
    int32_t* s_toff = reinterpret_cast<int32_t*>(smem);
    float* s_w = reinterpret_cast<float*>(smem + BM * 4);
    __syncthreads();
    for (int i = tid; i < BM; i += WAVES * 64) {
      int32_t toff = 0;
      float w = 0.0f;
      if (i < rows) {
        const int32_t sl = p.slots[row0 + i];
        toff = (sl / p.k_top) * int32_t(p.N);  // T * N < 2^31
        w = p.topk_w[sl];
      }
      s_toff[i] = toff;
      s_w[i] = w;
    }
    __syncthreads();
    float bn[2] = {0.0f, 0.0f};
    if (p.bias) {
#pragma unroll
      for (int f = 0; f < 2; ++f) bn[f] = p.bias[int64_t(e) * p.N + nrow[f]];
    }
    const bool full = rows == BM && int64_t(nt + 1) * (WAVES * 64) <= p.N;  // uniform
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (full || row < rows) {
          float* dst = p.comb + s_toff[row];
          const float w = s_w[row];
#pragma unroll
          for (int f = 0; f < 2; ++f)
            if (full || nvalid[f])
              (void)__hip_atomic_fetch_add(dst + nrow[f], w * (acc[rb][f][r] + bn[f]),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  } else {
    float* y = reinterpret_cast<float*>(p.out);
    const bool full = rows == BM && int64_t(nt + 1) * (WAVES * 64) <= p.N;  // uniform
    if (!p.bias && full) {
      // a full tile: no per-element guards, so the stores issue back to back.  y is read
      // once, by the combine, long after this launch: non-temporal stores keep it from
      // displacing the weights and activations in the caches (down stage -1 %, combine -3 %
      // on the skewed 64-expert layer, A/B on one box)
      float* yb = y + int64_t(row0) * p.N;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
#pragma unroll
          for (int f = 0; f < 2; ++f)
            __builtin_nontemporal_store(acc[rb][f][r], &yb[int64_t(row) * p.N + nrow[f]]);
        }
      }
    } else if (!p.bias) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (row < rows) {
#pragma unroll
            for (int f = 0; f < 2; ++f)
              if (nvalid[f]) y[int64_t(row0 + row) * p.N + nrow[f]] = acc[rb][f][r];
          }
        }
      }
    } else {
      float bn[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) bn[f] = p.bias[int64_t(e) * p.N + nrow[f]];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (row < rows) {
#pragma unroll
            for (int f = 0; f < 2; ++f)
              if (nvalid[f]) y[int64_t(row0 + row) * p.N + nrow[f]] = acc[rb][f][r] + bn[f];
          }
        }
      }
    }
  }
}

// Explicit instantiations: the host pass does not emit launch stubs for these templates
// implicitly (their bodies use generic lambdas).
#define E4B_GEMM_INST(FMT, GU, BM, W) \
  template __global__ void moe_gemm_kernel<FMT, GU, BM, W>(GemmArgs);
#define E4B_GEMM_INST_ALL(FMT)                                                           \
  E4B_GEMM_INST(FMT, true, 256, 4) E4B_GEMM_INST(FMT, false, 256, 4)                     \
  E4B_GEMM_INST(FMT, true, 128, 4) E4B_GEMM_INST(FMT, false, 128, 4)                     \
  E4B_GEMM_INST(FMT, true, 32, 1) E4B_GEMM_INST(FMT, false, 32, 1)
E4B_GEMM_INST_ALL(0)
E4B_GEMM_INST_ALL(1)


// Exclusive prefix sum of v over the 256 threads of the workgroup; *total = the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int32_t* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
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
  *total = tot;
  return woff + incl - v;
}

// One workgroup walks the experts in order and cuts each expert's rows into bm-row tiles.  If
// the last piece of an expert has at most `tail` rows (tail > 0), it becomes a "tail": it is
// cut into 16-row tiles for the streaming kernel, listed in tails[], so a full-size tile is
// not spent on a few rows -- unless a long GEMM launch's last round of workgroups has room
// for it.  The main list holds the regular tiles, then one entry per tail (its rows as a
// single tile, in expert order; t[3] = index of its first 16-row tile).  For a GEMM whose
// column sweep has nt tiles, the workgroups of the regular tiles fill
// R = ceil(regular * nt / n_cu) rounds of the n_cu compute units; when R >= kAbsorbRounds the
// first j tails, j = (free slots of the last round) / nt, run as main tiles in that round, and
// only the others go to the streaming kernel.  (In a launch of a few rounds a filled last
// round costs more than it saves: its workgroups then share the memory system with many
// more others.)  Counts written to n_mtiles (kTileCounts ints):
//   [0] regular tiles, [1] 0              (count and first index, the streaming path's list)
//   [2] gate_up main tiles, [3] down main tiles
//   [4], [5] gate_up 16-row tail tiles: count, first index in tails[]
//   [6], [7] the same for down
constexpr int kAbsorbRounds = 4;

struct TileArgs {
  const int32_t* offsets;
  int E, bm, tail;
  int32_t* tiles;
  int32_t* tails;
  int32_t* n_mtiles;
  int nt_gu, nt_dn, n_cu;  // column tiles of the two GEMMs, compute units (tails only)
};

__device__ void build_tiles(const TileArgs& ta) {
  const int32_t* __restrict__ offsets = ta.offsets;
  const int E = ta.E, bm = ta.bm, tail = ta.tail;
  int32_t* __restrict__ tiles = ta.tiles;
  int32_t* __restrict__ tails = ta.tails;
  int32_t* __restrict__ n_mtiles = ta.n_mtiles;
  __shared__ int32_t wsum[4];
  const int tid = threadIdx.x;
  int run = 0, run_s = 0;
  // regular tiles and 16-row tail tiles
  for (int base = 0; base < E; base += 256) {
    const int e = base + tid;
    const int start = e < E ? offsets[e] : 0;
    const int cnt = e < E ? offsets[e + 1] - start : 0;
    const int nfull = cnt / bm, rem = cnt - nfull * bm;
    const bool split = rem > 0 && rem <= tail;
    const int nt = split ? nfull : (cnt + bm - 1) / bm;
    const int ns = split ? (rem + kGemvTileRows - 1) / kGemvTileRows : 0;
    int tot, tot_s;
    const int first = run + block_exclusive_scan(nt, wsum, &tot);
    const int first_s = run_s + block_exclusive_scan(ns, wsum, &tot_s);
    for (int i = 0; i < nt; ++i) {
      int32_t* t = tiles + 4 * int64_t(first + i);
      t[0] = e;
      t[1] = start + i * bm;
      t[2] = min(bm, cnt - i * bm);
      t[3] = 0;
    }
    for (int i = 0; i < ns; ++i) {
      int32_t* t = tails + 4 * int64_t(first_s + i);
      t[0] = e;
      t[1] = start + nfull * bm + kGemvTileRows * i;
      t[2] = min(kGemvTileRows, rem - kGemvTileRows * i);
      t[3] = 0;
    }
    run += tot;
    run_s += tot_s;
  }
  // one main entry per tail, after the regular tiles
  int run_t = 0, run_s2 = 0;
  for (int base = 0; base < E; base += 256) {
    const int e = base + tid;
    const int start = e < E ? offsets[e] : 0;
    const int cnt = e < E ? offsets[e + 1] - start : 0;
    const int nfull = cnt / bm, rem = cnt - nfull * bm;
    const bool split = rem > 0 && rem <= tail;
    const int ns = split ? (rem + kGemvTileRows - 1) / kGemvTileRows : 0;
    int tot_t, tot_s;
    const int ord = run_t + block_exclusive_scan(split ? 1 : 0, wsum, &tot_t);
    const int first_s = run_s2 + block_exclusive_scan(ns, wsum, &tot_s);
    if (split) {
      int32_t* t = tiles + 4 * int64_t(run + ord);
      t[0] = e;
      t[1] = start + nfull * bm;
      t[2] = rem;
      t[3] = first_s;
    }
    run_t += tot_t;
    run_s2 += tot_s;
  }
  __syncthreads();  // the tail entries' first indices are read back below
  if (tid == 0) {
    n_mtiles[0] = run;
    n_mtiles[1] = 0;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int64_t nt = g == 0 ? ta.nt_gu : ta.nt_dn;
      int j = 0;
      if (run_t > 0 && nt > 0 && ta.n_cu > 0) {
        const int64_t wgs = int64_t(run) * nt;
        const int64_t rounds = (wgs + ta.n_cu - 1) / ta.n_cu;
        if (rounds >= kAbsorbRounds) j = int(min(int64_t(run_t), (rounds * ta.n_cu - wgs) / nt));
      }
      const int s0 = j < run_t ? tiles[4 * int64_t(run + j) + 3] : run_s;
      n_mtiles[2 + g] = run + j;
      n_mtiles[4 + 2 * g] = run_s - s0;
      n_mtiles[5 + 2 * g] = s0;
    }
  }
}

__global__ void __launch_bounds__(256) build_tiles_kernel(TileArgs ta) { build_tiles(ta); }

hipError_t launch_build_tiles(const int32_t* offsets, int E, int bm, int32_t* tiles,
                              int32_t* n_tiles, hipStream_t stream) {
  const TileArgs ta{offsets, E, bm, 0, tiles, tiles, n_tiles, 0, 0, 0};
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, stream, ta);
  return hipGetLastError();
}

// x bf16 -> fp16 (exact for |x| in fp16's normal range), stored in the k-slot order of the
// weight format inside each aligned group of 8.  Also inverts the routing permutation,
// inv[slots[p]] = p for the S sorted rows p, and records each sorted row's token,
// tok[p] = slots[p] / k.  The last workgroup first builds the tile list (build_tiles).  With
// `zero` set it also clears that [T, H] float32 accumulator of the atomic combine (kernel
// stores, not a memset, so the sequence can be captured in a graph).
template <int FMT>
__global__ void __launch_bounds__(256) convert_x_kernel(const uint16_t* __restrict__ x,
                                                        _Float16* __restrict__ x16,
                                                        int64_t n_chunks,
                                                        const int32_t* __restrict__ slots,
                                                        int64_t S, int32_t k,
                                                        int32_t* __restrict__ inv,
                                                        int32_t* __restrict__ tok,
                                                        float* __restrict__ zero,
                                                        TileArgs ta) {
  if (blockIdx.x == gridDim.x - 1) build_tiles(ta);  // uniform over the workgroup
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t n = n_chunks > S ? n_chunks : S;
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < n; q += stride) {
    if (q < S) {
      const int32_t sl = slots[q];
      inv[sl] = int32_t(q);
      tok[q] = sl / k;
    }
    if (q >= n_chunks) continue;
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
    if (zero) {
      reinterpret_cast<f32x4*>(zero + 8 * q)[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      reinterpret_cast<f32x4*>(zero + 8 * q)[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// out[t, :] = sum_{j<k} topk_w[s] * y[inv[s], :] with s = t*k + j, fixed order; fp32 and
// bf16 (RNE).
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ inv, int64_t T,
                                                      int64_t H, int k,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ out_f32) {
  const int64_t n4 = T * (H / 4);
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < n4; q += stride) {
    const int64_t t = q / (H / 4);
    const int64_t c = (q - t * (H / 4)) * 4;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j)
      s += topk_w[t * k + j] *
           *reinterpret_cast<const f32x4*>(y + int64_t(inv[t * k + j]) * H + c);
    if (out_f32) *reinterpret_cast<f32x4*>(out_f32 + t * H + c) = s;
    u32x2 o;
    o[0] = uint32_t(f32_to_bf16_rne(s[0])) | (uint32_t(f32_to_bf16_rne(s[1])) << 16);
    o[1] = uint32_t(f32_to_bf16_rne(s[2])) | (uint32_t(f32_to_bf16_rne(s[3])) << 16);
    *reinterpret_cast<u32x2*>(out + t * H + c) = o;
  }
}

// out[t, :] = bf16 RNE of the atomic combine's accumulator acc [T, H] (n4 = T * H / 4).
__global__ void __launch_bounds__(256) round_out_kernel(const float* __restrict__ acc, int64_t n4,
                                                        uint16_t* __restrict__ out) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < n4; q += stride) {
    const f32x4 s = reinterpret_cast<const f32x4*>(acc)[q];
    u32x2 o;
    o[0] = uint32_t(f32_to_bf16_rne(s[0])) | (uint32_t(f32_to_bf16_rne(s[1])) << 16);
    o[1] = uint32_t(f32_to_bf16_rne(s[2])) | (uint32_t(f32_to_bf16_rne(s[3])) << 16);
    reinterpret_cast<u32x2*>(out)[q] = o;
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

// The [T, H] float32 accumulator of the atomic combine.
static float* combine_target(const MoeLaunch& L) { return L.out_f32 ? L.out_f32 : L.y; }

// One grouped GEMM stage over the main tiles, then the streaming kernel over the 16-row tail
// tiles if any (an expert's last few rows: streaming its weights once per 16 rows beats
// running them as a mostly empty MFMA tile).
template <int FMT, bool GU, int BM, int WAVES>
static hipError_t launch_stage_tiles(const MoeLaunch& L, GemmArgs g, hipStream_t stream) {
  const int64_t n_out = GU ? L.I : L.H;
  const int per_wave = GU ? 32 : 64;
  g.tiles = L.tiles;
  g.n_mtiles = L.n_mtiles + (GU ? 2 : 3);  // main tiles of this GEMM (regular + absorbed tails)

  g.n_ntiles = int((n_out + WAVES * per_wave - 1) / (WAVES * per_wave));
  // XCD-local order when a row tile's column sweep fits one XCD's 32 CUs (one round): its
  // workgroups then share the activation tile in that XCD's L2.  Measured on one box: the
  // skewed 64-expert layer 6.12 -> 6.03 ms/step, the MXFP4 layer 0.679 -> 0.665 ms; with 112
  // column tiles (the Mixtral-shaped layer) the same order was 3 % slower.
  g.xcd_order = g.n_ntiles <= 32;
  hipLaunchKernelGGL((moe_gemm_kernel<FMT, GU, BM, WAVES>),
                     dim3(unsigned(L.max_mtiles * g.n_ntiles)), dim3(WAVES * 64), 0, stream, g);
  if (L.max_stiles > 0) return launch_gemv_tails(L, stream, GU ? 0 : 1);
  return hipGetLastError();
}

template <int FMT, int BM, int WAVES>
static hipError_t launch_gemms(const MoeLaunch& L, hipStream_t stream) {
  GemmArgs g{};
  g.slots = L.slots;
  g.clamped_glu = L.clamped_glu;
  g.interleaved = L.interleaved;
  g.k_top = L.k;
  g.I = L.I;
  g.T = L.T;
  // gate_up + SwiGLU
  g.a = L.x16;
  g.wq = L.w_gu;
  g.sc = L.s_gu;
  g.out = L.h;
  g.bias = L.b_gu;
  g.K = L.H;
  g.N = 2 * L.I;
  hipError_t err = (FMT == 1 && L.scaled && BM >= 128) ? launch_gate_up_scaled(L, stream)
                                                       : launch_stage_tiles<FMT, true, BM, WAVES>(L, g, stream);
  if (err != hipSuccess) return err;
  record(L, 3, stream);
  // down + routing weight
  g.a = L.h;
  g.bias = L.b_dn;
  g.wq = L.w_dn;
  g.sc = L.s_dn;
  g.out = L.y;
  g.K = L.I;
  g.N = L.H;
  g.topk_w = L.topk_w;
  g.comb = L.atomic_combine ? combine_target(L) : nullptr;
  return launch_stage_tiles<FMT, false, BM, WAVES>(L, g, stream);
}

template <int FMT>
static hipError_t launch_fmt(const MoeLaunch& L, hipStream_t stream) {
  record(L, 0, stream);
  // the streaming path takes activations in natural order for both formats
  const int64_t S = L.T * L.k, nchunks = L.T * L.H / 8;
  const unsigned gx = grid_1d(nchunks > S ? nchunks : S);
  // one launch converts x and builds the tile list (the "build_tiles" stage stays empty)
  const int wv = L.cfg.waves;
  const TileArgs ta{L.offsets, int(L.E), L.cfg.bm, L.tail_rows, L.tiles,
                    L.tiles + 4 * L.max_mtiles, L.n_mtiles,
                    int((L.I + 32 * wv - 1) / (32 * wv)), int((L.H + 64 * wv - 1) / (64 * wv)), cu_count()};
  float* zero = L.atomic_combine ? combine_target(L) : nullptr;
  if (FMT == 0 && !L.cfg.gemv)
    hipLaunchKernelGGL(convert_x_kernel<0>, dim3(gx), dim3(256), 0, stream, L.x, L.x16, nchunks,
                       L.slots, S, L.k, L.inv, L.tok, zero, ta);
  else
    hipLaunchKernelGGL(convert_x_kernel<1>, dim3(gx), dim3(256), 0, stream, L.x, L.x16, nchunks,
                       L.slots, S, L.k, L.inv, L.tok, zero, ta);
  record(L, 1, stream);
  record(L, 2, stream);
  hipError_t err;
  if (L.cfg.gemv) {
    err = launch_gemv(L, stream, 0);
    record(L, 3, stream);
    if (err == hipSuccess) err = launch_gemv(L, stream, 1);
  } else if (L.cfg.bm == 256)
    err = launch_gemms<FMT, 256, 4>(L, stream);
  else if (L.cfg.bm == 128)
    err = launch_gemms<FMT, 128, 4>(L, stream);
  else
    err = launch_gemms<FMT, 32, 1>(L, stream);
  if (err != hipSuccess) return err;
  record(L, 4, stream);
  if (L.atomic_combine)
    hipLaunchKernelGGL(round_out_kernel, dim3(grid_1d(L.T * L.H / 4)), dim3(256), 0, stream,
                       combine_target(L), L.T * L.H / 4, L.out);
  else
    hipLaunchKernelGGL(combine_kernel, dim3(grid_1d(L.T * L.H / 4)), dim3(256), 0, stream, L.y,
                       L.topk_w, L.inv, L.T, L.H, L.k, L.out, L.out_f32);
  record(L, 5, stream);
  return hipGetLastError();
}

hipError_t launch_moe_forward(const MoeLaunch& L, hipStream_t stream) {
  return L.fmt == 0 ? launch_fmt<0>(L, stream) : launch_fmt<1>(L, stream);
}

}  // namespace e4b
