// Host-side internals of libqmoe: the validated layer description, the
// workspace layout, and the kernel launchers each .hip file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qmoe.h"

namespace qmoe {

// Everything a launcher needs, resolved once at create time.
struct Layer {
  int64_t H, I, E;
  int k, bits, bs, zp;
  int act;        // kActF32, kActBF16 or kActF16 (x, logits, out and biases)
  bool act_bf16;  // act == kActBF16
  bool normalize;   // routing weights: softmax over the selected k (else over all experts)
  bool fc1_interleaved;   // FC1 row 2n = gate n, row 2n+1 = up n (else gate rows, then up rows)
  int64_t max_tokens;
  const uint8_t* fc1_codes;
  const uint16_t* fc1_scales;
  const uint8_t* fc2_codes;
  const uint16_t* fc2_scales;
  const void* fc1_bias;   // [E, 2I] in the activation dtype, or null
  const void* fc2_bias;   // [E, H] in the activation dtype, or null
  const uint8_t* fc1_zp;  // [E, 2I, H/bs] zero-point codes, or null (scalar zp)
  const uint8_t* fc2_zp;  // [E, H, I/bs] zero-point codes, or null (scalar zp)
  int64_t fc1_row_bytes, fc2_row_bytes;   // H*bits/8, I*bits/8
  int64_t fc1_nblk, fc2_nblk;             // H/bs, I/bs
  qmoe_stage_fn hook;                     // profiling hook (may be null)
  void* hook_user;
};

// Report a finished launch to the profiling hook, if any.
inline void stage_done(const Layer& L, int stage, const char* name) {
  if (L.hook) L.hook(L.hook_user, stage, name);
}

// Prefill GEMM tiling (rows = routes of one expert, cols = output features).
constexpr int kTileM = 256;
// Small-batch path: routes of one expert per tile (one MFMA row block).
constexpr int kSmallRows = 16;
constexpr int kTileN = 128;
constexpr int kChunkTokens = 32;           // tokens per histogram/scatter chunk

// Bytes per route of the prefill's h exponents (one per 32 columns of h),
// padded to whole 16-byte rows.
__host__ __device__ constexpr int h_exp_stride(int64_t I) {
  return static_cast<int>((I / 32 + 15) / 16 * 16);
}

// Decode GEMV row blocking.
struct GemvShape {
  int units;       // K / 32
  int lpr;         // lanes per row (power of two, <= 64)
  int upl;         // units per lane (1, 2 or 4)
  int rows_wave;   // rows one wave covers per step = 64 / lpr
  int rows_block;  // rows one workgroup covers
};
GemvShape gemv_shape(int64_t K, int min_rows_block);

// Workspace layout for one forward call on T tokens (byte offsets).
struct Workspace {
  size_t topk_id, topk_w;             // int32 / fp32 [R]
  size_t h32, y32;                    // decode: fp32 [R, I], fp32 [R, H]
  size_t hist, chunk_base;            // prefill: int32 [nchunks, E] each
  size_t counts, offsets;             // int32 [E], [E + 1]
  size_t sorted_routes, inv_pos;      // int32 [R]
  size_t tiles, num_tiles;            // int4 [max_tiles], int32 [1]
  size_t x16, xexp;                   // prefill, bf16/fp32 activations: fp16 [T, H], int8 [T]
  size_t h16, hexp, rexp, yf32;       // prefill: fp16 [R, I], int8 [R, h_exp_stride(I)], int8 [R],
                                      // fp32 [R, H]
  size_t total;
  int64_t R, nchunks, max_tiles;
  int tile_m;                         // routes per tile of the grouped paths
  int fc2_row_blocks;                 // decode: FC2 workgroups per route
  bool decode;
};

// The path a forward call takes.
enum class Path { kDecode, kSmall, kPrefill };

// ---- launchers (each returns hipSuccess or the launch error)
hipError_t launch_route(const Layer& L, const void* logits, int64_t T, char* ws, const Workspace& W,
                        hipStream_t s);
// One-launch routing of a small batch (with the activation staging when x is
// not null; *xa and *xexp, when not null, receive FC1's operand rows and
// exponents), usable while route_small_fits.
bool route_small_fits(const Layer& L, int64_t T);
hipError_t launch_route_small(const Layer& L, const void* logits, const void* x, int64_t T, char* ws,
                              const Workspace& W, hipStream_t s, const uint16_t** xa,
                              const int8_t** xexp);
hipError_t launch_prefill(const Layer& L, const void* x, void* out, int64_t T, char* ws,
                          const Workspace& W, hipStream_t s);
// Staging of FC1's activations (fp16 in operand order, with a per-token
// exponent for bf16/fp32 inputs) and the routing-weighted combine, shared by
// the grouped paths.
hipError_t launch_stage_x(const Layer& L, const void* x, int64_t T, char* ws, const Workspace& W,
                          hipStream_t s, const uint16_t** xa, const int8_t** xexp);
hipError_t launch_combine(const Layer& L, void* out, int64_t T, char* ws, const Workspace& W,
                          hipStream_t s);
// Small-batch path (routing included): grouped GEMMs streaming each
// expert's weights once.
bool small_path_supported(const Layer& L);
hipError_t prepare_small(const Layer& L);
hipError_t launch_small(const Layer& L, const void* x, const void* logits, void* out, int64_t T,
                        char* ws, const Workspace& W, hipStream_t s);
hipError_t launch_decode(const Layer& L, const void* x, const void* logits, void* out, int64_t T,
                         char* ws, const Workspace& W, hipStream_t s);
// Fused single-launch decode (bf16 or fp16 activations, H <= 2048,
// I <= 1024, or I <= 768 with fp16, biases or zero-point tensors; E <= 256).
// Its workgroups exchange h and y through a per-handle device
// buffer of epoch-tagged entries (fused_exchange_bytes, zeroed at create and
// by clear_exchange whenever the epoch counter wraps); every call passes a
// new nonzero epoch.
constexpr int kFusedMaxWorkgroups = 1024;
constexpr int kFusedMaxExperts = 256;
constexpr size_t kExchangeHeader = 256;                 // error bits, then the h and y entries
bool fused_decode_supported(const Layer& L);
int fused_decode_grid(const Layer& L, int device);
size_t fused_exchange_bytes(const Layer& L);
hipError_t clear_exchange(const Layer& L, void* xbuf, hipStream_t s);
hipError_t launch_decode_fused(const Layer& L, const void* x, const void* logits, void* out,
                               int64_t T, char* ws, const Workspace& W, void* xbuf,
                               uint32_t epoch, int grid, uint32_t spin_limit, hipStream_t s);
hipError_t launch_dequant(const Layer& L, int fc, int64_t expert, float* out_f32,
                          uint16_t* out_f16, hipStream_t s);

}  // namespace qmoe
