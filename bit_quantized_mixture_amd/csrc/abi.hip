// C ABI of the e4b library: host-side validation, workspace carving and kernel launches.
// Every check runs before anything is enqueued; a failed check enqueues nothing.  There is
// no alternative code path: on a device other than gfx950 every compute entry point fails.
#include <string.h>

#include <atomic>

#include "e4b.h"
#include "e4b_internal.h"

namespace {

constexpr size_t kAlign = 256;
// MXFP4 gate_up on the block-scaled instruction unless E4B_MXFP4_FP16 is given
constexpr bool kScaledByDefault = false;
constexpr int kMaxDevices = 64;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 1 = gfx950, -1 = other arch, 0 = not yet probed.
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return E4B_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return E4B_ERR_UNSUPPORTED;
  if (g_arch_ok[dev].load(std::memory_order_relaxed) == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return E4B_ERR_HIP;
    g_arch_ok[dev].store(strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1,
                         std::memory_order_relaxed);
  }
  return g_arch_ok[dev].load(std::memory_order_relaxed) == 1 ? E4B_OK : E4B_ERR_UNSUPPORTED;
}

int launched(hipError_t e) { return e == hipSuccess ? E4B_OK : E4B_ERR_HIP; }

// Workspace of e4b_moe_forward_noalloc: a file-scope device array, one copy per GPU the library
// runs on, held until the process ends.  Host code never uses the array's name as an address
// (on the host it is only a stand-in for the symbol): the device address of the current GPU's
// copy comes from hipGetSymbolAddress, once per device, and is kept in g_scratch.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];

int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return E4B_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return E4B_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // the address of this device's copy (the symbol lookup is idempotent, so two threads
    // racing here store the same value)
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return E4B_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return E4B_OK;
}

int check_pack(const void* w, int64_t E, int64_t N, int64_t K, const void* o1, const void* o2,
               int64_t block) {
  if (!w || !o1 || !o2) return E4B_ERR_ARG;
  if (E <= 0 || N <= 0 || K <= 0) return E4B_ERR_ARG;
  if (K % block) return E4B_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(o1) || !aligned16(o2)) return E4B_ERR_ALIGN;
  if (E > (int64_t(1) << 40) / N / K) return E4B_ERR_OVERFLOW;
  return E4B_OK;
}

// Tile (rows, waves) for the sizes of a forward call (host-known only).
struct Tile {
  int bm, waves, gemv;
};
Tile pick_tile(const e4b_moe_args* a) {
  const int64_t S = a->T * a->k;
  const int path = a->flags & E4B_PATH_MASK;
  switch (a->flags & E4B_TILE_MASK) {
    case E4B_TILE_32: return {32, 1, 0};
    case E4B_TILE_128: return {128, 4, 0};
    case E4B_TILE_256: return {256, 4, 0};
    default: break;
  }
  const double mean_rows = double(S) / double(a->E);
  if (path == E4B_PATH_GEMV || (path == E4B_PATH_AUTO && mean_rows < 16.0))
    return {e4b::kGemvTileRows, 4, 1};
  // 256-row tiles once an expert averages two of them: below that most experts end in a
  // partly filled 256-row tile, and the launch has too few workgroups for even rounds
  return mean_rows >= 512.0 ? Tile{256, 4, 0} : Tile{128, 4, 0};
}

struct FwdLayout {
  int bm, waves, gemv, scaled;
  int64_t max_mtiles, max_stiles;
  int tail_rows;
  size_t off_x16, off_h, off_y, off_inv, off_tok, off_tiles, off_n, off_x8, off_xsc, total;
};

// Route of an MXFP4 gate_up on MFMA tiles: the block-scaled fp8 x fp4 instruction or fp16
// operands decoded in registers.
bool use_scaled(const e4b_moe_args* a, const Tile& t) {
  if (a->fmt != E4B_FMT_MXFP4 || t.gemv || t.bm < 128) return false;
  const int r = a->flags & E4B_MXFP4_ROUTE_MASK;
  if (r == E4B_MXFP4_SCALED) return true;
  if (r == E4B_MXFP4_FP16) return false;
  return kScaledByDefault;
}

// The tile, with the scaled route's 128-row tiles where it applies.
Tile pick_route_tile(const e4b_moe_args* a) {
  Tile t = pick_tile(a);
  if (use_scaled(a, t)) t = Tile{128, 4, 0};
  return t;
}

int layout_forward(const e4b_moe_args* a, FwdLayout* L) {
  const int64_t S = a->T * a->k;
  const Tile t = pick_route_tile(a);
  L->bm = t.bm;
  L->waves = t.waves;
  L->gemv = t.gemv;
  const int64_t n_active_max = a->E < S ? a->E : S;
  L->max_mtiles = (S + n_active_max * (L->bm - 1)) / L->bm;
  // MFMA tiles of 128 or 256 rows: an expert's remainder of at most bm / 4 rows goes to
  // 16-row tiles of the streaming kernel instead of a mostly empty full tile
  L->tail_rows = (!L->gemv && L->bm >= 128) ? L->bm / 4 : 0;
  L->max_stiles = n_active_max * int64_t((L->tail_rows + e4b::kGemvTileRows - 1) / e4b::kGemvTileRows);
  size_t off = 0;
  L->off_x16 = off;
  off += align_up(size_t(a->T) * size_t(a->H) * 2);
  L->off_h = off;
  off += align_up(size_t(S) * size_t(a->I) * 2);
  L->off_y = off;
  off += align_up(size_t(S) * size_t(a->H) * 4);
  L->off_inv = off;
  off += align_up(size_t(S) * 4);
  L->off_tok = off;
  off += align_up(size_t(S) * 4);
  L->off_tiles = off;
  off += align_up(size_t(L->max_mtiles + L->max_stiles) * 16);
  L->off_n = off;
  off += kAlign;
  L->scaled = use_scaled(a, t) ? 1 : 0;
  L->off_x8 = off;
  L->off_xsc = off;
  if (L->scaled) {
    off += align_up(size_t(a->T) * size_t(a->H) * 2);
    L->off_xsc = off;
    off += align_up(size_t(a->T) * size_t(e4b::scale_pitch(a->H)));
  }
  L->total = off;
  return E4B_OK;
}

int check_forward_shape(const e4b_moe_args* a) {
  if (!a) return E4B_ERR_ARG;
  if (a->fmt != E4B_FMT_NF4 && a->fmt != E4B_FMT_MXFP4) return E4B_ERR_ARG;
  if (a->E <= 0 || a->H <= 0 || a->I <= 0 || a->T < 0 || a->k < 1) return E4B_ERR_ARG;
  if (a->k > a->E) return E4B_ERR_ARG;
  if ((a->flags & ~(E4B_PATH_MASK | E4B_TILE_MASK | E4B_ACT_CLAMPED_GLU | E4B_GU_INTERLEAVED |
                    E4B_MXFP4_ROUTE_MASK | E4B_COMBINE_ATOMIC)) != 0 ||
      (a->flags & E4B_MXFP4_ROUTE_MASK) == E4B_MXFP4_ROUTE_MASK ||
      (a->flags & E4B_PATH_MASK) == 3)
    return E4B_ERR_ARG;
  // a row-tile override names an MFMA tile; it cannot go with the streaming path
  if ((a->flags & E4B_PATH_MASK) == E4B_PATH_GEMV && (a->flags & E4B_TILE_MASK) != 0)
    return E4B_ERR_ARG;
  if (a->reserved != 0) return E4B_ERR_ARG;
  if (a->H % 64 || a->I % 64) return E4B_ERR_SHAPE;
  if (a->T * a->k >= (int64_t(1) << 31)) return E4B_ERR_OVERFLOW;
  if (a->E >= (int64_t(1) << 31) || a->H >= (int64_t(1) << 31) || a->I >= (int64_t(1) << 30))
    return E4B_ERR_OVERFLOW;
  // activation offsets inside the GEMMs are 32-bit element indices, weight offsets 32-bit
  // byte offsets inside one expert's stack (I * H bytes for gate_up)
  if (a->T * a->H >= (int64_t(1) << 31) || a->T * a->k * a->I >= (int64_t(1) << 31))
    return E4B_ERR_OVERFLOW;
  if (a->I * a->H >= (int64_t(1) << 31)) return E4B_ERR_OVERFLOW;
  return E4B_OK;
}

int check_decode(const e4b_decode_args* a) {
  if (!a) return E4B_ERR_ARG;
  if (a->fmt != E4B_FMT_NF4 && a->fmt != E4B_FMT_MXFP4) return E4B_ERR_ARG;
  if (a->reserved != 0) return E4B_ERR_ARG;
  if ((a->route_flags & ~E4B_ROUTE_RENORMALIZE) != 0) return E4B_ERR_ARG;
  if ((a->flags & ~(E4B_ACT_CLAMPED_GLU | E4B_GU_INTERLEAVED)) != 0) return E4B_ERR_ARG;
  if (a->E <= 0 || a->H <= 0 || a->I <= 0 || a->k < 1 || a->k > a->E) return E4B_ERR_ARG;
  if (a->T < 1 || a->T > 8 || a->T * a->k > 64 || a->E > 1024) return E4B_ERR_SHAPE;
  if (a->T * a->H > 32768) return E4B_ERR_SHAPE;  // x is held in LDS: at most 64 KB
  if (a->H % 64 || a->I % 64) return E4B_ERR_SHAPE;
  if (a->I * a->H >= (int64_t(1) << 31) || a->H >= (int64_t(1) << 24) || a->I >= (int64_t(1) << 24))
    return E4B_ERR_OVERFLOW;
  return E4B_OK;
}

int dgrad_check(const e4b_dgrad_args* a, int64_t* max_tiles) {
  if (!a) return E4B_ERR_ARG;
  if (a->fmt != E4B_FMT_NF4 && a->fmt != E4B_FMT_MXFP4) return E4B_ERR_ARG;
  if (a->reserved != 0) return E4B_ERR_ARG;
  if (a->E <= 0 || a->N <= 0 || a->K <= 0 || a->S < 0) return E4B_ERR_ARG;
  if (a->N % 64 || a->K % 64) return E4B_ERR_SHAPE;
  if (a->E > 1024 * 1024 || a->S * a->N >= (int64_t(1) << 31) || a->S * a->K >= (int64_t(1) << 31) ||
      a->N * (a->K / 2) >= (int64_t(1) << 31))
    return E4B_ERR_OVERFLOW;
  const int64_t bm = e4b::dgrad_tile_rows();
  const int64_t active = a->E < a->S ? a->E : a->S;
  *max_tiles = (a->S + active * (bm - 1)) / bm;
  return E4B_OK;
}

int int4_check(const e4b_int4_gemv_args* a, int64_t* max_tiles) {
  if (!a) return E4B_ERR_ARG;
  if (a->reserved != 0) return E4B_ERR_ARG;
  if (a->E <= 0 || a->N <= 0 || a->K <= 0 || a->T < 0 || a->k < 1 || a->k > 64 || a->k > a->E)
    return E4B_ERR_ARG;
  if (a->N % 16 || a->K % 128 || a->K > 8192) return E4B_ERR_SHAPE;
  const int64_t S = a->T * a->k;
  if (a->E > 1024 * 1024 || a->T >= (int64_t(1) << 31) || S >= (int64_t(1) << 31) ||
      S * a->N >= (int64_t(1) << 40) || a->N * (a->K / 2) >= (int64_t(1) << 31))
    return E4B_ERR_OVERFLOW;
  const int64_t bm = a->T > 0 ? e4b::int4_gemv_tile_rows(a->T) : 1;
  const int64_t active = a->E < S ? a->E : S;
  *max_tiles = (S + active * (bm - 1)) / bm;
  if (*max_tiles * (a->N / 16) >= (int64_t(1) << 31)) return E4B_ERR_OVERFLOW;  // grid size
  return E4B_OK;
}

}  // namespace

extern "C" {

int e4b_pack_int4_b32(const uint16_t* w, int64_t E, int64_t N, int64_t K, uint8_t* packed,
                      uint16_t* scales, void* stream) {
  if (!w || !packed || !scales || E <= 0 || N <= 0 || K <= 0) return E4B_ERR_ARG;
  if (K % 32) return E4B_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(scales)) return E4B_ERR_ALIGN;
  if (E > (int64_t(1) << 40) / N / K) return E4B_ERR_OVERFLOW;
  const int st = check_device();
  if (st != E4B_OK) return st;
  return launched(e4b::launch_pack_int4(w, E * N * K, packed, scales, (hipStream_t)stream));
}

int e4b_quantize_act_int8(const uint16_t* x, int64_t T, int64_t K, int8_t* q, float* s,
                          void* stream) {
  if (!x || !q || !s || T < 0 || K <= 0) return E4B_ERR_ARG;
  if (K % 32) return E4B_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return E4B_ERR_ALIGN;
  if (T >= (int64_t(1) << 31) || K >= (int64_t(1) << 31)) return E4B_ERR_OVERFLOW;
  const int st = check_device();
  if (st != E4B_OK || T == 0) return st;
  return launched(e4b::launch_quant_act(x, T, K, q, s, (hipStream_t)stream));
}

int e4b_int4_gemv_workspace_bytes(const e4b_int4_gemv_args* a, size_t* bytes) {
  if (!bytes) return E4B_ERR_ARG;
  int64_t mt = 0;
  const int st = int4_check(a, &mt);
  if (st != E4B_OK) return st;
  *bytes = align_up(size_t(a->T * a->K)) + align_up(size_t(a->T * (a->K / 32) * 4)) +
           align_up(size_t(a->T * 4)) + align_up(size_t(mt) * 16) + kAlign;
  return E4B_OK;
}

int e4b_gemv_int4_b32(const e4b_int4_gemv_args* a, void* stream) {
  int64_t mt = 0;
  int st = int4_check(a, &mt);
  if (st != E4B_OK) return st;
  if (a->T == 0) return check_device();
  if (!a->x || !a->w || !a->s || !a->expert_offsets || !a->sorted_slots || !a->out_f32 || !a->ws)
    return E4B_ERR_ARG;
  const void* ptrs[] = {a->x, a->w, a->s, a->expert_offsets, a->sorted_slots, a->out_f32, a->ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return E4B_ERR_ALIGN;
  size_t need = 0;
  e4b_int4_gemv_workspace_bytes(a, &need);
  if (a->ws_bytes < need) return E4B_ERR_WORKSPACE;
  if ((st = check_device()) != E4B_OK) return st;
  char* ws = reinterpret_cast<char*>(a->ws);
  e4b::Int4GemvLaunch L{};
  L.E = a->E;
  L.N = a->N;
  L.K = a->K;
  L.T = a->T;
  L.k = a->k;
  L.x = a->x;
  L.wq = a->w;
  L.sc = a->s;
  L.offsets = a->expert_offsets;
  L.slots = a->sorted_slots;
  L.out = a->out_f32;
  size_t off = 0;
  L.qx = reinterpret_cast<int8_t*>(ws + off);
  off += align_up(size_t(a->T * a->K));
  L.xs = reinterpret_cast<int32_t*>(ws + off);
  off += align_up(size_t(a->T * (a->K / 32) * 4));
  L.sx = reinterpret_cast<float*>(ws + off);
  off += align_up(size_t(a->T * 4));
  L.tiles = reinterpret_cast<int32_t*>(ws + off);
  off += align_up(size_t(mt) * 16);
  L.n_tiles = reinterpret_cast<int32_t*>(ws + off);
  L.max_tiles = mt;
  return launched(e4b::launch_int4_gemv(L, (hipStream_t)stream));
}

int e4b_version(void) { return 400; }


int e4b_dgrad_workspace_bytes(const e4b_dgrad_args* a, size_t* bytes) {
  if (!bytes) return E4B_ERR_ARG;
  int64_t mt = 0;
  const int st = dgrad_check(a, &mt);
  if (st != E4B_OK) return st;
  *bytes = align_up(size_t(mt) * 16) + kAlign;
  return E4B_OK;
}

int e4b_grouped_dgrad(const e4b_dgrad_args* a, void* stream) {
  int64_t mt = 0;
  int st = dgrad_check(a, &mt);
  if (st != E4B_OK) return st;
  if (a->S == 0) return check_device();
  if (!a->g || !a->w || !a->s || !a->expert_offsets || !a->out_f32 || !a->ws) return E4B_ERR_ARG;
  const void* ptrs[] = {a->g, a->w, a->s, a->expert_offsets, a->out_f32, a->out, a->ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return E4B_ERR_ALIGN;
  size_t need = 0;
  e4b_dgrad_workspace_bytes(a, &need);
  if (a->ws_bytes < need) return E4B_ERR_WORKSPACE;
  if ((st = check_device()) != E4B_OK) return st;
  char* ws = reinterpret_cast<char*>(a->ws);
  e4b::DgradLaunch L{};
  L.fmt = a->fmt;
  L.E = a->E;
  L.N = a->N;
  L.K = a->K;
  L.S = a->S;
  L.g = a->g;
  L.wq = a->w;
  L.sc = a->s;
  L.offsets = a->expert_offsets;
  L.out_f32 = a->out_f32;
  L.out = a->out;
  L.tiles = reinterpret_cast<int32_t*>(ws);
  L.n_tiles = reinterpret_cast<int32_t*>(ws + align_up(size_t(mt) * 16));
  L.max_tiles = mt;
  return launched(e4b::launch_dgrad(L, (hipStream_t)stream));
}

const char* e4b_status_string(int status) {
  switch (status) {
    case E4B_OK: return "ok";
    case E4B_ERR_ARG: return "invalid argument (null pointer, bad size, flag or format)";
    case E4B_ERR_SHAPE: return "shape breaks a block or tiling constraint";
    case E4B_ERR_ALIGN: return "pointer not 16-byte aligned";
    case E4B_ERR_WORKSPACE: return "workspace missing or too small";
    case E4B_ERR_UNSUPPORTED: return "current device is not gfx950";
    case E4B_ERR_OVERFLOW: return "size overflows the index types";
    case E4B_ERR_HIP: return "HIP runtime or launch failure";
    case E4B_ERR_TOO_LARGE:
      return "the call needs more workspace than the allocation-free entry point's fixed scratch";
    default: return "unknown status";
  }
}

int e4b_pack_nf4(const uint16_t* w, int64_t E, int64_t N, int64_t K, uint8_t* packed,
                 float* absmax, void* stream) {
  int st = check_pack(w, E, N, K, packed, absmax, 64);
  if (st != E4B_OK) return st;
  if ((st = check_device()) != E4B_OK) return st;
  return launched(e4b::launch_pack_nf4(w, E * N * K, packed, absmax, (hipStream_t)stream));
}

int e4b_pack_mxfp4(const uint16_t* w, int64_t E, int64_t N, int64_t K, uint8_t* blocks,
                   uint8_t* scales, void* stream) {
  int st = check_pack(w, E, N, K, blocks, scales, 32);
  if (st != E4B_OK) return st;
  if ((st = check_device()) != E4B_OK) return st;
  return launched(e4b::launch_pack_mxfp4(w, E * N * K, blocks, scales, (hipStream_t)stream));
}

int e4b_route_workspace_bytes(int64_t T, int64_t E, int32_t k, size_t* bytes) {
  if (!bytes) return E4B_ERR_ARG;
  if (T < 0 || E <= 0 || k < 1) return E4B_ERR_ARG;
  *bytes = align_up(size_t(e4b::route_chunks(T)) * size_t(E) * 4);
  return E4B_OK;
}

int e4b_route_permute(const float* logits, int64_t T, int64_t E, int32_t k, int32_t flags,
                      int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                      int32_t* sorted_slots, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || E <= 0 || k < 1 || k > E) return E4B_ERR_ARG;
  if (E > 1024 || k > 64) return E4B_ERR_SHAPE;
  if (flags & ~E4B_ROUTE_RENORMALIZE) return E4B_ERR_ARG;
  if (!expert_offsets || !ws) return E4B_ERR_ARG;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_slots)) return E4B_ERR_ARG;
  if (T * k >= (int64_t(1) << 31)) return E4B_ERR_OVERFLOW;
  const void* ptrs[] = {logits, topk_ids, topk_w, expert_offsets, sorted_slots, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return E4B_ERR_ALIGN;
  size_t need = 0;
  e4b_route_workspace_bytes(T, E, k, &need);
  if (ws_bytes < need) return E4B_ERR_WORKSPACE;
  int st = check_device();
  if (st != E4B_OK) return st;
  return launched(e4b::launch_route(logits, T, E, k, (flags & E4B_ROUTE_RENORMALIZE) != 0,
                                    topk_ids, topk_w, expert_offsets, sorted_slots,
                                    reinterpret_cast<int32_t*>(ws), (hipStream_t)stream));
}

int e4b_moe_workspace_bytes(const e4b_moe_args* a, size_t* bytes) {
  if (!bytes) return E4B_ERR_ARG;
  int st = check_forward_shape(a);
  if (st != E4B_OK) return st;
  FwdLayout L;
  layout_forward(a, &L);
  *bytes = L.total;
  return E4B_OK;
}

}  // extern "C"

namespace {

// The forward once the workspace is known: `ws` holds at least layout_forward's total.
int forward_impl(const e4b_moe_args* a, char* ws, hipStream_t stream) {
  FwdLayout L;
  layout_forward(a, &L);
  e4b::MoeLaunch M{};
  M.fmt = a->fmt;
  M.E = a->E;
  M.H = a->H;
  M.I = a->I;
  M.T = a->T;
  M.k = a->k;
  M.cfg.bm = L.bm;
  M.cfg.waves = L.waves;
  M.cfg.gemv = L.gemv;
  M.max_mtiles = L.max_mtiles;
  M.max_stiles = L.max_stiles;
  M.tail_rows = L.tail_rows;
  M.x = a->x;
  M.w_gu = a->w_gu;
  M.s_gu = a->s_gu;
  M.w_dn = a->w_dn;
  M.s_dn = a->s_dn;
  M.topk_w = a->topk_w;
  M.offsets = a->expert_offsets;
  M.slots = a->sorted_slots;
  M.out = a->out;
  M.out_f32 = a->out_f32;
  M.b_gu = a->b_gu;
  M.b_dn = a->b_dn;
  M.clamped_glu = (a->flags & E4B_ACT_CLAMPED_GLU) ? 1 : 0;
  M.interleaved = (a->flags & E4B_GU_INTERLEAVED) ? 1 : 0;
  M.atomic_combine = ((a->flags & E4B_COMBINE_ATOMIC) && !L.gemv) ? 1 : 0;
  M.x16 = reinterpret_cast<_Float16*>(ws + L.off_x16);
  M.h = reinterpret_cast<_Float16*>(ws + L.off_h);
  M.y = reinterpret_cast<float*>(ws + L.off_y);
  M.inv = reinterpret_cast<int32_t*>(ws + L.off_inv);
  M.tok = reinterpret_cast<int32_t*>(ws + L.off_tok);
  M.tiles = reinterpret_cast<int32_t*>(ws + L.off_tiles);
  M.n_mtiles = reinterpret_cast<int32_t*>(ws + L.off_n);
  M.scaled = L.scaled;
  M.x8 = reinterpret_cast<uint8_t*>(ws + L.off_x8);
  M.xsc = reinterpret_cast<uint8_t*>(ws + L.off_xsc);
  M.events = a->stage_events;
  return launched(e4b::launch_moe_forward(M, stream));
}

// Checks shared by both forward entry points, up to (not including) the workspace.
int check_forward_call(const e4b_moe_args* a) {
  if (!a->x || !a->w_gu || !a->s_gu || !a->w_dn || !a->s_dn || !a->topk_w ||
      !a->expert_offsets || !a->sorted_slots || !a->out)
    return E4B_ERR_ARG;
  const void* ptrs[] = {a->x, a->w_gu, a->s_gu, a->w_dn, a->s_dn, a->topk_w,
                        a->expert_offsets, a->sorted_slots, a->out, a->out_f32, a->ws,
                        a->b_gu, a->b_dn};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return E4B_ERR_ALIGN;
  return E4B_OK;
}

}  // namespace

extern "C" {

int e4b_moe_forward(const e4b_moe_args* a, void* stream) {
  int st = check_forward_shape(a);
  if (st != E4B_OK) return st;
  if (a->T == 0) return check_device();  // nothing to compute; no buffer is touched
  if ((st = check_forward_call(a)) != E4B_OK) return st;
  if (!a->ws) return E4B_ERR_ARG;
  FwdLayout L;
  layout_forward(a, &L);
  if (a->ws_bytes < L.total) return E4B_ERR_WORKSPACE;
  if ((st = check_device()) != E4B_OK) return st;
  return forward_impl(a, reinterpret_cast<char*>(a->ws), (hipStream_t)stream);
}

int e4b_decode_workspace_bytes(const e4b_decode_args* a, size_t* bytes) {
  if (!bytes) return E4B_ERR_ARG;
  const int st = check_decode(a);
  if (st != E4B_OK) return st;
  *bytes = e4b::decode_ctl_bytes(a->H) + align_up(size_t(a->T * a->k) * size_t(a->I) * 2) +
           align_up(size_t((a->H + 15) / 16) * 8 * 8 * 16 * 4);
  return E4B_OK;
}

int e4b_moe_decode_step(const e4b_decode_args* a, void* stream) {
  int st = check_decode(a);
  if (st != E4B_OK) return st;
  if (!a->logits || !a->x || !a->w_gu || !a->s_gu || !a->w_dn || !a->s_dn || !a->out || !a->ws)
    return E4B_ERR_ARG;
  if ((a->topk_ids == nullptr) != (a->topk_w == nullptr)) return E4B_ERR_ARG;
  const void* ptrs[] = {a->logits, a->x, a->w_gu, a->s_gu, a->w_dn, a->s_dn, a->b_gu, a->b_dn,
                        a->topk_ids, a->topk_w, a->expert_offsets, a->sorted_slots, a->out,
                        a->out_f32, a->ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return E4B_ERR_ALIGN;
  size_t need = 0;
  e4b_decode_workspace_bytes(a, &need);
  if (a->ws_bytes < need) return E4B_ERR_WORKSPACE;
  if ((st = check_device()) != E4B_OK) return st;
  char* ws = reinterpret_cast<char*>(a->ws);
  e4b::DecodeLaunch L{};
  L.fmt = a->fmt;
  L.E = a->E;
  L.H = a->H;
  L.I = a->I;
  L.T = a->T;
  L.k = a->k;
  L.renorm = (a->route_flags & E4B_ROUTE_RENORMALIZE) ? 1 : 0;
  L.clamped_glu = (a->flags & E4B_ACT_CLAMPED_GLU) ? 1 : 0;
  L.interleaved = (a->flags & E4B_GU_INTERLEAVED) ? 1 : 0;
  L.spin_limit = a->spin_limit == 0 ? (1 << 20) : a->spin_limit;
  L.logits = a->logits;
  L.x = a->x;
  L.w_gu = a->w_gu;
  L.s_gu = a->s_gu;
  L.w_dn = a->w_dn;
  L.s_dn = a->s_dn;
  L.b_gu = a->b_gu;
  L.b_dn = a->b_dn;
  L.ids = a->topk_ids;
  L.w = a->topk_w;
  L.offsets = a->expert_offsets;
  L.slots = a->sorted_slots;
  L.out = a->out;
  L.out_f32 = a->out_f32;
  L.status = a->status;
  const size_t ctl = e4b::decode_ctl_bytes(a->H);
  L.ctl = reinterpret_cast<uint32_t*>(ws);
  L.h = reinterpret_cast<_Float16*>(ws + ctl);
  L.part = reinterpret_cast<float*>(ws + ctl + align_up(size_t(a->T * a->k) * size_t(a->I) * 2));
  return launched(e4b::launch_decode_step(L, (hipStream_t)stream));
}

size_t e4b_noalloc_scratch_bytes(void) { return kScratchBytes; }

int e4b_stream_probe(const void* src, void* dst, int64_t bytes, int32_t mode, void* stream) {
  if (!src || bytes <= 0 || (mode != 0 && mode != 1) || (mode == 1 && !dst)) return E4B_ERR_ARG;
  if (bytes % 16) return E4B_ERR_SHAPE;
  if (!aligned16(src) || (dst && !aligned16(dst))) return E4B_ERR_ALIGN;
  int st = check_device();
  if (st != E4B_OK) return st;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return E4B_ERR_HIP;
  return launched(e4b::launch_stream_probe(src, dst, bytes, mode, cus, (hipStream_t)stream));
}

int e4b_moe_forward_noalloc(const e4b_moe_args* a, void* stream) {
  int st = check_forward_shape(a);
  if (st != E4B_OK) return st;
  if (a->ws || a->ws_bytes) return E4B_ERR_ARG;  // the workspace is the library's own
  if (a->T == 0) return check_device();
  if ((st = check_forward_call(a)) != E4B_OK) return st;
  FwdLayout L;
  layout_forward(a, &L);
  if (L.total > kScratchBytes) return E4B_ERR_TOO_LARGE;
  if ((st = check_device()) != E4B_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws)) != E4B_OK) return st;
  // Every buffer carved from the scratch is written before it is read within the call (x16,
  // inv and tok by the conversion, the tile list and its counts by the tile builder, h and y
  // by the two products), so nothing is cleared and the previous call's contents are harmless.
  return forward_impl(a, reinterpret_cast<char*>(ws), (hipStream_t)stream);
}

}  // extern "C"
