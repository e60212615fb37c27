// C ABI of libqmoe: validation, workspace layout and dispatch.
//
// Validation happens once, on the host, before any device work: the pages
// record admission paths that disagreed about a normalized field and a
// division by zero on an expert count of zero, fixed by validating positive,
// representable dimensions up front ("[CUDA] Add INT4 and INT3 QMoE CPU/GPU
// offload support", review-fix commits: weights_prepacked=-1 normalization
// and E=0 rejection). Environment overrides are read once, at create.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "device.h"
#include "internal.h"

struct qmoe_handle {
  qmoe::Layer L;
  int device;
  int force;              // QMOE_FORCE_PATH: one of the kForce* values below
  bool split_decode;      // use the two-kernel decode even where the fused one applies
  bool fused_ok;          // fused single-launch decode applies to this layer
  bool small_ok;          // the small-batch path applies to this layer
  int fused_grid;         // resident workgroups for the fused decode
  uint32_t spin_limit;    // fused decode wait bound in polls (0: the library default)
  uint32_t calls;         // epoch of the last fused decode call launched (0: none yet)
  void* xbuf;             // device: fused decode exchange buffer (error bits, tagged h and y)
};

namespace qmoe {

static int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

GemvShape gemv_shape(int64_t K, int min_rows_block) {
  GemvShape s;
  s.units = static_cast<int>(K / 32);
  int p = 1;
  while (p < s.units && p < 64) p <<= 1;
  s.lpr = p;
  int upl = (s.units + s.lpr - 1) / s.lpr;
  s.upl = upl <= 1 ? 1 : upl <= 2 ? 2 : 4;
  s.rows_wave = kWave / s.lpr;
  int steps = (min_rows_block + 4 * s.rows_wave - 1) / (4 * s.rows_wave);
  if (steps < 1) steps = 1;
  s.rows_block = 4 * s.rows_wave * steps;
  return s;
}

// Paths forced from the environment (QMOE_FORCE_PATH, read at create).
constexpr int kForceNone = 0, kForcePrefill = 1, kForceSmall = 2, kForceGrouped = 3;

// Batches above the decode's four tokens. On layers the fused decode serves,
// up to kGroupedDecodeMaxTokens run it once per group of four tokens (each
// launch streams only its group's experts). Up to kSmallMaxTokens run the
// small-batch path, which streams each active expert's weights once per
// call; larger batches run the grouped GEMMs on 256-row tiles. Measured on
// the Qwen3-30B-A3B-shaped INT4 layer (us per call, cold weights):
//   tokens          5     8     9    12    16    24    32    64   128   256   384
//   grouped decode 45    55    71    81   107   158
//   small path     55    71    72    81    84   101   106   121   144   211   263
//   grouped GEMMs 100   135   136   152   154   204   207   213   224   231   232
// QMOE_FORCE_PATH=grouped extends the grouped decode to 24 tokens.
constexpr int64_t kGroupedDecodeMaxTokens = 8;
constexpr int64_t kGroupedDecodeForcedMax = 24;
constexpr int64_t kSmallMaxTokens = 256;

Path choose_path(const Layer& L, int force, bool small_ok, bool fused, int64_t T) {
  (void)L;
  if (force == kForcePrefill) return Path::kPrefill;
  if (force == kForceSmall && small_ok) return Path::kSmall;
  if (T <= kDecodeMaxTokens) return Path::kDecode;
  const int64_t grouped_max = force == kForceGrouped ? kGroupedDecodeForcedMax : kGroupedDecodeMaxTokens;
  if (fused && T <= grouped_max) return Path::kDecode;
  if (small_ok && T <= kSmallMaxTokens) return Path::kSmall;
  return Path::kPrefill;
}

static Workspace layout(const Layer& L, int64_t T, Path path) {
  Workspace W;
  memset(&W, 0, sizeof W);
  const int64_t R = T * L.k;
  W.R = R;
  W.decode = path == Path::kDecode;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = static_cast<size_t>(round_up(static_cast<int64_t>(off + bytes), 256));
    return at;
  };
  W.topk_id = take(R * 4);
  W.topk_w = take(R * 4);
  if (path == Path::kDecode) {
    const GemvShape s2 = gemv_shape(L.I, 64);
    W.fc2_row_blocks = static_cast<int>((L.H + s2.rows_block - 1) / s2.rows_block);
    W.h32 = take(static_cast<size_t>(R * L.I * 4));
    W.y32 = take(static_cast<size_t>(R * L.H * 4));
  } else {
    W.tile_m = path == Path::kSmall ? kSmallRows : kTileM;
    W.nchunks = (T + kChunkTokens - 1) / kChunkTokens;
    W.max_tiles = (R + W.tile_m - 1) / W.tile_m + L.E;
    W.hist = take(static_cast<size_t>(W.nchunks * L.E * 4));
    W.chunk_base = take(static_cast<size_t>(W.nchunks * L.E * 4));
    W.counts = take(static_cast<size_t>(L.E * 4));
    W.offsets = take(static_cast<size_t>((L.E + 1) * 4));
    W.sorted_routes = take(static_cast<size_t>(R * 4));
    W.inv_pos = take(static_cast<size_t>(R * 4));
    W.tiles = take(static_cast<size_t>(W.max_tiles * 16));
    W.num_tiles = take(4);
    // fp16 activations are staged only to put them in operand order
    const bool staged = L.act != kActF16 || operand_perm(L.bits) != 0;
    W.x16 = staged ? take(static_cast<size_t>(T * L.H * 2)) : 0;
    W.xexp = L.act == kActF16 ? 0 : take(static_cast<size_t>(T));
    if (path == Path::kSmall) {
      W.h32 = take(static_cast<size_t>(R * L.I * 4));
    } else {
      W.h16 = take(static_cast<size_t>(R * L.I * 2));
      W.hexp = take(static_cast<size_t>(R * h_exp_stride(L.I)));
      W.rexp = take(static_cast<size_t>(R));
    }
    W.yf32 = take(static_cast<size_t>(R * L.H * 4));
  }
  W.total = off;
  return W;
}

}  // namespace qmoe

using namespace qmoe;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

class DeviceGuard {
 public:
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev_) != hipSuccess) prev_ = -1;
    ok_ = true;
    if (prev_ != dev) ok_ = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev_ >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev_) (void)hipSetDevice(prev_);
  }
  bool ok() const { return ok_; }

 private:
  int prev_ = -1;
  bool ok_ = false;
};

// Workspace for a forward call on T tokens: enough for the path it takes,
// with or without the fused decode (a call under graph capture does without
// it), and for qmoe_route, which runs the grouped GEMMs' routing.
size_t required_bytes(const qmoe_handle* h, int64_t T) {
  size_t need = layout(h->L, T, Path::kPrefill).total;
  for (bool fused : {false, true}) {
    const Path p = choose_path(h->L, h->force, h->small_ok, fused && h->fused_ok && !h->split_decode, T);
    const size_t b = layout(h->L, T, p).total;
    need = b > need ? b : need;
  }
  return need;
}

// Workspace of qmoe_forward_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends. In host code the
// symbol's name is no device address: qmoe_create resolves each device's
// copy once (with that device current) and every use goes through the
// pointer kept here.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[QMOE_NOALLOC_WORKSPACE_BYTES];
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// Resolve the calling thread's current device's copy of `scratch`, once.
hipError_t resolve_scratch(int device) {
  if (device >= kMaxDevices) return hipSuccess;   // qmoe_forward_noalloc refuses such devices
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[device]) return hipSuccess;
  void* p = nullptr;
  const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (err == hipSuccess) g_scratch[device] = p;
  return err;
}

void* scratch_for(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch[device];
}

// The dispatch shared by qmoe_forward and qmoe_forward_noalloc; the caller
// has validated the arguments, checked that `ws` holds required_bytes(h, T)
// bytes and made the handle's device current.
qmoe_status forward_impl(qmoe_handle* h, const void* x, const void* logits, void* out, int64_t T,
                         void* ws, hipStream_t s);

}  // namespace

extern "C" {

const char* qmoe_status_string(int st) {
  // an int, not the enum: callers may pass any value, and a C++ enum object
  // holding a value outside its enumerators' range is undefined behaviour
  switch (st) {
    case QMOE_OK: return "ok";
    case QMOE_ERR_INVALID_ARG: return "invalid argument";
    case QMOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case QMOE_ERR_WORKSPACE: return "workspace missing or too small";
    case QMOE_ERR_HIP: return "HIP runtime error";
    case QMOE_ERR_OOM: return "out of host memory";
  }
  return "unknown status";
}

qmoe_status qmoe_create(const qmoe_config* c, const qmoe_weights* w, int device, qmoe_handle** out) {
  if (!out) return QMOE_ERR_INVALID_ARG;
  *out = nullptr;
  if (!c || !w) return QMOE_ERR_INVALID_ARG;
  if (c->struct_size != sizeof(qmoe_config)) return QMOE_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->inter <= 0 || c->num_experts <= 0) return QMOE_ERR_INVALID_ARG;
  if (c->top_k < 1 || c->top_k > c->num_experts) return QMOE_ERR_INVALID_ARG;
  if (c->bits != 2 && c->bits != 3 && c->bits != 4) return QMOE_ERR_INVALID_ARG;
  if (c->block_size != 32 && c->block_size != 64 && c->block_size != 128) return QMOE_ERR_INVALID_ARG;
  if (c->hidden % c->block_size != 0 || c->inter % c->block_size != 0) return QMOE_ERR_INVALID_ARG;
  if (c->zero_point < -1 || c->zero_point >= (1 << c->bits)) return QMOE_ERR_INVALID_ARG;
  if (c->act_dtype != QMOE_F32 && c->act_dtype != QMOE_BF16 && c->act_dtype != QMOE_F16)
    return QMOE_ERR_INVALID_ARG;
  if ((c->flags & ~QMOE_FLAG_FC1_INTERLEAVED) != 0 || c->max_tokens < 0) return QMOE_ERR_INVALID_ARG;
  if (c->normalize_routing != 0 && c->normalize_routing != 1) return QMOE_ERR_INVALID_ARG;
  if (!w->fc1_codes || !w->fc1_scales || !w->fc2_codes || !w->fc2_scales) return QMOE_ERR_INVALID_ARG;
  if (!aligned16(w->fc1_codes) || !aligned16(w->fc1_scales) || !aligned16(w->fc2_codes) ||
      !aligned16(w->fc2_scales))
    return QMOE_ERR_INVALID_ARG;
  if ((w->fc1_bias && !aligned16(w->fc1_bias)) || (w->fc2_bias && !aligned16(w->fc2_bias)))
    return QMOE_ERR_INVALID_ARG;
  // limits of this implementation
  if (c->num_experts > kMaxExperts || c->top_k > kMaxTopK) return QMOE_ERR_UNSUPPORTED;
  if (c->hidden > 8192 || c->inter > 8192) return QMOE_ERR_UNSUPPORTED;
  if (c->max_tokens > (int64_t{1} << 31) / (c->top_k * int64_t{kTileN})) return QMOE_ERR_UNSUPPORTED;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return QMOE_ERR_HIP;
  if (device < 0 || device >= ndev) return QMOE_ERR_INVALID_ARG;

  qmoe_handle* h = new (std::nothrow) qmoe_handle;
  if (!h) return QMOE_ERR_OOM;
  Layer& L = h->L;
  L.H = c->hidden;
  L.I = c->inter;
  L.E = c->num_experts;
  L.k = c->top_k;
  L.bits = c->bits;
  L.bs = c->block_size;
  L.zp = c->zero_point < 0 ? (1 << (c->bits - 1)) : c->zero_point;
  L.act = c->act_dtype == QMOE_BF16 ? kActBF16 : c->act_dtype == QMOE_F16 ? kActF16 : kActF32;
  L.act_bf16 = L.act == kActBF16;
  L.normalize = c->normalize_routing == 1;
  L.fc1_interleaved = (c->flags & QMOE_FLAG_FC1_INTERLEAVED) != 0;
  L.max_tokens = c->max_tokens;
  L.fc1_codes = static_cast<const uint8_t*>(w->fc1_codes);
  L.fc1_scales = static_cast<const uint16_t*>(w->fc1_scales);
  L.fc2_codes = static_cast<const uint8_t*>(w->fc2_codes);
  L.fc2_scales = static_cast<const uint16_t*>(w->fc2_scales);
  L.fc1_bias = w->fc1_bias;
  L.fc2_bias = w->fc2_bias;
  L.fc1_zp = static_cast<const uint8_t*>(w->fc1_zero_points);
  L.fc2_zp = static_cast<const uint8_t*>(w->fc2_zero_points);
  L.fc1_row_bytes = L.H * L.bits / 8;
  L.fc2_row_bytes = L.I * L.bits / 8;
  L.fc1_nblk = L.H / L.bs;
  L.fc2_nblk = L.I / L.bs;
  L.hook = nullptr;
  L.hook_user = nullptr;
  h->device = device;
  const char* force = getenv("QMOE_FORCE_PATH");
  h->force = !force                           ? kForceNone
             : strcmp(force, "prefill") == 0  ? kForcePrefill
             : strcmp(force, "small") == 0    ? kForceSmall
             : strcmp(force, "grouped") == 0  ? kForceGrouped
                                              : kForceNone;
  h->split_decode = force && strcmp(force, "decode_split") == 0;
  h->small_ok = small_path_supported(L);
  h->xbuf = nullptr;
  h->calls = 0;
  h->fused_ok = false;
  h->fused_grid = 0;
  h->spin_limit = 0;
  {
    DeviceGuard guard(device);
    if (!guard.ok() || resolve_scratch(device) != hipSuccess ||
        (h->small_ok && prepare_small(L) != hipSuccess)) {
      delete h;
      return QMOE_ERR_HIP;
    }
    if (fused_decode_supported(L)) {
      const size_t xb = fused_exchange_bytes(L);
      if (hipMalloc(&h->xbuf, xb) != hipSuccess || hipMemset(h->xbuf, 0, xb) != hipSuccess) {
        if (h->xbuf) (void)hipFree(h->xbuf);
        delete h;
        return QMOE_ERR_HIP;
      }
      h->fused_grid = fused_decode_grid(L, device);
      // QMOE_FUSED_GRID=n caps the fused decode grid at n workgroups (n >= 1),
      // e.g. to exercise its many-experts-per-workgroup schedule
      const char* cap = getenv("QMOE_FUSED_GRID");
      if (cap) {
        const long n = strtol(cap, nullptr, 10);
        if (n >= 1 && n < h->fused_grid) h->fused_grid = static_cast<int>(n);
      }
      h->fused_ok = h->fused_grid > 0;
      // QMOE_FUSED_EPOCH_START=n makes the first fused call use epoch n + 1
      // (with n = 4294967295 the first call takes the wrap path)
      const char* e0 = getenv("QMOE_FUSED_EPOCH_START");
      if (e0) h->calls = static_cast<uint32_t>(strtoul(e0, nullptr, 10));
      // QMOE_FUSED_SPIN_LIMIT=n (n >= 1) bounds each wait at n polls, so a
      // test can make waits run out and check that the error bits report it
      const char* sl = getenv("QMOE_FUSED_SPIN_LIMIT");
      if (sl) {
        const long n = strtol(sl, nullptr, 10);
        if (n >= 1) h->spin_limit = static_cast<uint32_t>(n);
      }
    }
  }
  *out = h;
  return QMOE_OK;
}

qmoe_status qmoe_workspace_size(const qmoe_handle* h, int64_t T, size_t* bytes) {
  if (!h || !bytes || T < 0 || T > h->L.max_tokens) return QMOE_ERR_INVALID_ARG;
  *bytes = required_bytes(h, T);
  return QMOE_OK;
}

qmoe_status qmoe_workspace_routing(const qmoe_handle* h, int64_t T, size_t* id_off, size_t* w_off) {
  if (!h || !id_off || !w_off || T < 0 || T > h->L.max_tokens) return QMOE_ERR_INVALID_ARG;
  const Workspace W =
      layout(h->L, T, choose_path(h->L, h->force, h->small_ok, h->fused_ok && !h->split_decode, T));
  *id_off = W.topk_id;
  *w_off = W.topk_w;
  return QMOE_OK;
}

qmoe_status qmoe_forward(qmoe_handle* h, const void* x, const void* logits, void* out, int64_t T,
                         void* ws, size_t ws_bytes, void* stream) {
  if (!h || T < 0 || T > h->L.max_tokens) return QMOE_ERR_INVALID_ARG;
  if (T == 0) return QMOE_OK;
  if (!x || !logits || !out || !aligned16(x) || !aligned16(logits) || !aligned16(out))
    return QMOE_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < required_bytes(h, T)) return QMOE_ERR_WORKSPACE;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return QMOE_ERR_HIP;
  return forward_impl(h, x, logits, out, T, ws, static_cast<hipStream_t>(stream));
}

qmoe_status qmoe_forward_noalloc(qmoe_handle* h, const void* x, const void* logits, void* out,
                                 int64_t T, void* stream) {
  if (!h || T < 0 || T > h->L.max_tokens) return QMOE_ERR_INVALID_ARG;
  if (T == 0) return QMOE_OK;
  if (!x || !logits || !out || !aligned16(x) || !aligned16(logits) || !aligned16(out))
    return QMOE_ERR_INVALID_ARG;
  if (required_bytes(h, T) > QMOE_NOALLOC_WORKSPACE_BYTES) return QMOE_ERR_WORKSPACE;
  void* ws = scratch_for(h->device);
  if (!ws) return QMOE_ERR_UNSUPPORTED;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return QMOE_ERR_HIP;
  return forward_impl(h, x, logits, out, T, ws, static_cast<hipStream_t>(stream));
}

qmoe_status qmoe_route(qmoe_handle* h, const void* logits, int64_t T, int32_t* topk_id, float* topk_w,
                       int32_t* expert_offsets, int32_t* sorted_routes, int32_t* inv_pos, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!h || T < 1 || T > h->L.max_tokens) return QMOE_ERR_INVALID_ARG;
  if (!logits || !aligned16(logits)) return QMOE_ERR_INVALID_ARG;
  // the routing a forward of T tokens runs on the batched paths
  const Path path = choose_path(h->L, h->force, h->small_ok, h->fused_ok && !h->split_decode, T);
  const bool small = path == Path::kSmall && route_small_fits(h->L, T);
  const Workspace W = layout(h->L, T, small ? Path::kSmall : Path::kPrefill);
  if (!ws || !aligned16(ws) || ws_bytes < W.total) return QMOE_ERR_WORKSPACE;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return QMOE_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  hipError_t err = small ? launch_route_small(h->L, logits, nullptr, T, base, W, s, nullptr, nullptr)
                         : launch_route(h->L, logits, T, base, W, s);
  const size_t R = static_cast<size_t>(W.R);
  auto copy = [&](void* dst, size_t off, size_t bytes) {
    if (dst && err == hipSuccess) err = hipMemcpyAsync(dst, base + off, bytes, hipMemcpyDeviceToDevice, s);
  };
  copy(topk_id, W.topk_id, R * 4);
  copy(topk_w, W.topk_w, R * 4);
  copy(expert_offsets, W.offsets, static_cast<size_t>(h->L.E + 1) * 4);
  copy(sorted_routes, W.sorted_routes, R * 4);
  copy(inv_pos, W.inv_pos, R * 4);
  return err == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

qmoe_status qmoe_dequant(qmoe_handle* h, int fc, int64_t expert, float* out_f32, uint16_t* out_f16,
                         void* stream) {
  if (!h || (fc != 1 && fc != 2) || expert < 0 || expert >= h->L.E) return QMOE_ERR_INVALID_ARG;
  if (!out_f32 && !out_f16) return QMOE_OK;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return QMOE_ERR_HIP;
  hipError_t err = launch_dequant(h->L, fc, expert, out_f32, out_f16, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

qmoe_status qmoe_set_stage_hook(qmoe_handle* h, qmoe_stage_fn fn, void* user) {
  if (!h) return QMOE_ERR_INVALID_ARG;
  h->L.hook = fn;
  h->L.hook_user = user;
  return QMOE_OK;
}

qmoe_status qmoe_decode_errors(qmoe_handle* h, void* stream, uint32_t* bits) {
  if (!h || !bits) return QMOE_ERR_INVALID_ARG;
  *bits = 0;
  if (!h->xbuf) return QMOE_OK;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return QMOE_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  // the error word is the first word of the exchange buffer's header
  if (hipStreamSynchronize(s) != hipSuccess ||
      hipMemcpy(&v, h->xbuf, sizeof v, hipMemcpyDeviceToHost) != hipSuccess)
    return QMOE_ERR_HIP;
  if (v != 0) {
    const uint32_t zero = 0;
    if (hipMemcpy(h->xbuf, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return QMOE_ERR_HIP;
  }
  *bits = v;
  return QMOE_OK;
}

qmoe_status qmoe_destroy(qmoe_handle* h) {
  if (!h) return QMOE_OK;
  if (h->xbuf) {
    DeviceGuard guard(h->device);
    (void)hipFree(h->xbuf);
  }
  delete h;
  return QMOE_OK;
}

}  // extern "C"

namespace {

qmoe_status forward_impl(qmoe_handle* h, const void* x, const void* logits, void* out, int64_t T,
                         void* ws, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  hipError_t err;
  bool fused = h->fused_ok && !h->split_decode;
  if (fused) {
    // The fused decode tags its exchange entries with an epoch the host
    // picks per call; a captured graph would replay one epoch forever, so a
    // call under stream capture takes the paths without cross-workgroup
    // exchange (split decode up to four tokens, grouped GEMMs above).
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return QMOE_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) fused = false;
  }
  stage_done(h->L, 0, "start");
  const Path path = choose_path(h->L, h->force, h->small_ok, fused, T);
  if (path == Path::kDecode) {
    const Workspace W = layout(h->L, T, Path::kDecode);
    if (fused) {
      // one launch per group of up to four tokens (bf16 rows), each with its
      // own epoch: 1, 2, ...; when the counter wraps the exchange buffer is
      // zeroed again first, so no entry can carry a reused epoch. A launch
      // that did not happen does not use up its epoch.
      err = hipSuccess;
      const int64_t H = h->L.H, E = h->L.E, k = h->L.k;
      for (int64_t t0 = 0; t0 < T && err == hipSuccess; t0 += kDecodeMaxTokens) {
        const int64_t tg = T - t0 < kDecodeMaxTokens ? T - t0 : kDecodeMaxTokens;
        uint32_t epoch = h->calls + 1u;
        if (epoch == 0u) {
          epoch = 1u;
          err = clear_exchange(h->L, h->xbuf, s);
          if (err != hipSuccess) break;
        }
        Workspace Wg = W;   // this group's routing slots
        Wg.topk_id += static_cast<size_t>(t0 * k * 4);
        Wg.topk_w += static_cast<size_t>(t0 * k * 4);
        err = launch_decode_fused(h->L, static_cast<const uint16_t*>(x) + t0 * H,
                                  static_cast<const uint16_t*>(logits) + t0 * E,
                                  static_cast<uint16_t*>(out) + t0 * H, tg, base, Wg, h->xbuf, epoch,
                                  h->fused_grid, h->spin_limit, s);
        if (err == hipSuccess) h->calls = epoch;
      }
    } else {
      err = launch_decode(h->L, x, logits, out, T, base, W, s);
    }
  } else {
    const Workspace W = layout(h->L, T, path);
    if (path == Path::kSmall) {
      err = launch_small(h->L, x, logits, out, T, base, W, s);
    } else {
      err = launch_route(h->L, logits, T, base, W, s);
      if (err == hipSuccess) err = launch_prefill(h->L, x, out, T, base, W, s);
    }
  }
  return err == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

}  // namespace

