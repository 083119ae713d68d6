// Host-side launchers shared between the kernel translation units and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e4b {

// Tile shapes of the grouped expert GEMM.  BM = rows (routed slots) per tile; the N extent
// per workgroup is 32 h-columns per wave for gate_up (a 32-wide gate fragment and the
// matching 32-wide up fragment) and 64 output columns per wave for down.
// gemv = 1 selects the small-M streaming kernels (gemv.hip) instead, with tiles of at most
// kGemvTileRows rows.
struct TileCfg {
  int bm;
  int waves;
  int gemv;
};

constexpr int kGemvTileRows = 16;
constexpr int kTileCounts = 8;  // ints of tile counts written by the tile-list builder

// Compute units of the current device (cached per device).
int cu_count();

hipError_t launch_pack_nf4(const uint16_t* w, int64_t n_elems, uint8_t* packed, float* absmax,
                           hipStream_t stream);
hipError_t launch_pack_mxfp4(const uint16_t* w, int64_t n_elems, uint8_t* blocks, uint8_t* scales,
                             hipStream_t stream);

// Routing: per-(chunk, expert) counts, [route_chunks(T), E] int32, live in the workspace.
int route_chunks(int64_t T);
hipError_t launch_route(const float* logits, int64_t T, int64_t E, int k, bool renorm,
                        int32_t* ids, float* w, int32_t* offsets, int32_t* slots, int32_t* cc,
                        hipStream_t stream);

struct MoeLaunch {
  int fmt;
  int64_t E, H, I, T;
  int k;
  TileCfg cfg;
  int64_t max_mtiles;
  int64_t max_stiles;  // bound on 16-row tail tiles (0: not used)
  int tail_rows;       // an expert's last rows go to tail tiles if at most this many
  const uint16_t* x;
  const uint8_t* w_gu;
  const void* s_gu;
  const uint8_t* w_dn;
  const void* s_dn;
  const float* topk_w;
  const int32_t* offsets;
  const int32_t* slots;
  uint16_t* out;
  float* out_f32;
  const float* b_gu;  // nullable [E, 2I]
  const float* b_dn;  // nullable [E, H]
  int clamped_glu;    // activation: 0 silu(G) * U, 1 clamped GLU
  int interleaved;    // gate_up rows: 0 halves, 1 interleaved
  int scaled;         // MXFP4 gate_up on the block-scaled fp8 x fp4 instruction (MFMA tiles)
  int atomic_combine; // MFMA tile path: the down GEMM adds topk_w * y into a [T, H] float32
                      // accumulator (out_f32, else the y region) with atomic adds
  // workspace carve-outs
  _Float16* x16;   // [T, H]
  _Float16* h;     // [S, I]
  float* y;        // [S, H], sorted-row order (atomic combine: the [T, H] accumulator when
                   // out_f32 is NULL)
  int32_t* inv;    // [S]: slot -> sorted row
  int32_t* tok;    // [S]: sorted row -> token (slot / k)
  int32_t* tiles;  // [max_mtiles + max_stiles, 4]: main tiles, then tail tiles
  int32_t* n_mtiles;  // [kTileCounts]: tile counts and first indices (build_tiles in moe.hip)
  uint8_t* x8;        // [T, 2H] activation fp8 parts (scaled route)
  uint8_t* xsc;       // [T, scale_pitch(H)] activation e8m0 scales (scaled route)
  void* const* events;  // nullable: 6 hipEvent_t around the 5 stages
};

hipError_t launch_moe_forward(const MoeLaunch& L, hipStream_t stream);
// MXFP4 gate_up on the block-scaled instruction (128-row MFMA tiles, then tails); its activation
// scale rows hold scale_pitch(K) bytes.
hipError_t launch_gate_up_scaled(const MoeLaunch& L, hipStream_t stream);
__host__ __device__ int64_t scale_pitch(int64_t K);

// The tile list of build_tiles as its own launch (bm-row tiles, no tail tiles).
hipError_t launch_build_tiles(const int32_t* offsets, int E, int bm, int32_t* tiles,
                              int32_t* n_tiles, hipStream_t stream);

// Grouped dgrad: out[p] = g[p] @ W_e for the grouped rows p of expert e.
struct DgradLaunch {
  int fmt;
  int64_t E, N, K, S;
  const uint16_t* g;
  const uint8_t* wq;
  const void* sc;
  const int32_t* offsets;
  float* out_f32;
  uint16_t* out;        // nullable
  int32_t* tiles;       // workspace [max_tiles, 4]
  int32_t* n_tiles;     // workspace [2]
  int64_t max_tiles;
};
hipError_t launch_dgrad(const DgradLaunch& L, hipStream_t stream);
int dgrad_tile_rows();

// int4-b32: packer, per-token int8 activations in natural order, and the routed decode GEMV
// (which quantises into its own permuted layout).
hipError_t launch_pack_int4(const uint16_t* w, int64_t n_elems, uint8_t* packed, uint16_t* scales,
                            hipStream_t stream);
hipError_t launch_quant_act(const uint16_t* x, int64_t T, int64_t K, int8_t* q, float* s,
                            hipStream_t stream);
struct Int4GemvLaunch {
  int64_t E, N, K, T;
  int k;
  const uint16_t* x;
  const uint8_t* wq;
  const uint16_t* sc;
  const int32_t* offsets;
  const int32_t* slots;
  float* out;
  int8_t* qx;          // workspace [T, K]
  int32_t* xs;         // workspace [T, K/32]
  float* sx;           // workspace [T]
  int32_t* tiles;      // workspace [max_tiles, 4]
  int32_t* n_tiles;    // workspace [2]
  int64_t max_tiles;
};
hipError_t launch_int4_gemv(const Int4GemvLaunch& L, hipStream_t stream);
int int4_gemv_tile_rows(int64_t T);
size_t int4_gemv_lds_bytes(int64_t T, int64_t K);

// Small-M streaming kernels: stage 0 = gate_up + SwiGLU (x16 -> h), 1 = down (h -> y).
hipError_t launch_gemv(const MoeLaunch& L, hipStream_t stream, int stage);
// The same kernels over the tail tiles of the MFMA-tile path (its activation order).
hipError_t launch_gemv_tails(const MoeLaunch& L, hipStream_t stream, int stage);

// Single-launch decode step (T <= 8, T*k <= 64): routing, gate_up + activation, down and the
// weighted combine in one kernel with one grid barrier.
struct DecodeLaunch {
  int fmt;
  int64_t E, H, I, T;
  int k;
  int renorm, clamped_glu, interleaved;
  int spin_limit;
  const float* logits;
  const uint16_t* x;
  const uint8_t* w_gu;
  const void* s_gu;
  const uint8_t* w_dn;
  const void* s_dn;
  const float* b_gu;
  const float* b_dn;
  int32_t* ids;       // nullable outputs
  float* w;
  int32_t* offsets;
  int32_t* slots;
  uint16_t* out;
  float* out_f32;     // nullable
  _Float16* h;        // workspace [T*k, I]
  float* part;        // workspace [ceil(H/16)][8][8][16] column-block sums
  uint32_t* ctl;      // workspace control words (decode_ctl_bytes), zero between calls
  int32_t* status;    // nullable
};
size_t decode_ctl_bytes(int64_t H);
hipError_t launch_decode_step(const DecodeLaunch& L, hipStream_t stream);

// Streaming read (mode 0; dst: NULL or a 4-byte sink that is never written in practice) or
// copy (mode 1) of `bytes` (a multiple of 16) with cus * 8 workgroups.
hipError_t launch_stream_probe(const void* src, void* dst, int64_t bytes, int mode, int cus,
                               hipStream_t stream);

}  // namespace e4b
