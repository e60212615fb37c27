// Decode path (1..4 tokens): memory-bound dequant-GEMVs.
//
// Every active expert's weights are streamed from HBM once and applied to
// all (at most four) tokens that selected it. Three launches:
//   1. decode_fc1: each workgroup recomputes the top-k routing of the <= 4
//      tokens in its prologue (a few hundred logits), owns one (expert, block
//      of gate rows) pair, and writes h = silu(gate) * up in fp32 per route;
//   2. decode_fc2: each workgroup owns one (expert, block of output rows)
//      pair and writes the per-route fp32 FC2 rows;
//   3. decode_combine: sums the k slots of every token in slot order and
//      rounds once. (A separate launch: having the last FC2 workgroup of a
//      row block combine needed a device-scope fence in every workgroup,
//      which cost more than the launch.)
//
// Semantics: SwiGLU experts with fc1 rows = 2 * inter ("[CUDA/CPU] Add AVX2
// INT4 cold-expert kernel and zero-cold doorbell short-circuit for QMoE
// offload", Motivation & Summary item 3); fp32 partial sums rounded once by
// the combine ("[CUDA] Add MoEPacked CPU/GPU hybrid offload and consolidate
// QMoE/GGUF offload optimizations", Key Changes item 4).
//
// Arithmetic: codes are turned into bf16 pairs 128 + q (exact) and dotted
// with bf16 activations by v_dot2_f32_bf16 into an fp32 accumulator that
// starts at -(128 + zp) * sum(x); the block result is then
// sum((q - zp) * x), scaled by s. fp32 activations (and the fp32 FC2 input
// h) use plain fp32 FMAs on the integer codes instead.
#include "device.h"
#include "internal.h"

namespace qmoe {

namespace {

template <int BITS, int UPL>
struct XPairs {
  uint32_t p[UPL][16];
  float sum[UPL];   // sum of the unit's 32 x values
};

template <int UPL>
struct XFloats {
  float v[UPL][32];
  float sum[UPL];
};

// sum((q - zp) * x) over one unit, bf16 activations.
template <int BITS>
__device__ __forceinline__ float unit_dot_pairs(const uint32_t (&wp)[16], const uint32_t (&xp)[16],
                                                float corr) {
  float acc = corr;
#pragma unroll
  for (int p = 0; p < 16; ++p) acc = dot2_bf16(wp[p], xp[p], acc);
  return acc;
}

// sum(q * v) over one unit, fp32 values (natural code order).
template <int BITS>
__device__ __forceinline__ float unit_dot_f32(const UnitWords<BITS>& u, const float (&v)[32]) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) acc = fmaf(static_cast<float>(unit_code<BITS>(u, i)), v[i], acc);
  return acc;
}

struct RoutingLds {
  int32_t ids[kDecodeMaxTokens * kMaxTopK];
  float w[kDecodeMaxTokens * kMaxTopK];
};

// slot[t] = the slot of expert e in token t's selection, or -1.
__device__ __forceinline__ void token_slots(const RoutingLds& R, int T, int k, int e,
                                            int (&slot)[kDecodeMaxTokens]) {
#pragma unroll
  for (int t = 0; t < kDecodeMaxTokens; ++t) {
    slot[t] = -1;
    if (t < T)
      for (int j = 0; j < k; ++j)
        if (R.ids[t * k + j] == e) slot[t] = j;
  }
}

}  // namespace

// grid = (ceil(I / rows_block), T * k), block = 256 (4 waves)
template <int BITS, int UPL, int ACT>
__global__ __launch_bounds__(256) void decode_fc1_kernel(
    const void* __restrict__ xv, const void* __restrict__ logitsv, int T, int E, int k, bool normalize,
    bool fc1_il, const void* __restrict__ fc1_bias, const uint8_t* __restrict__ fc1_zp,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int H, int I, int bs,
    int zp, int64_t row_bytes, int64_t nblk, int lpr, int rows_block,
    int32_t* __restrict__ ws_ids, float* __restrict__ ws_w, float* __restrict__ h32) {
  __shared__ RoutingLds R;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  if (wave < T) {
    if constexpr (ACT == kActBF16)
      topk_softmax_wave(static_cast<const uint16_t*>(logitsv) + static_cast<int64_t>(wave) * E, E, k,
                        normalize, lane, R.ids + wave * k, R.w + wave * k);
    else if constexpr (ACT == kActF16)
      topk_softmax_wave(static_cast<const _Float16*>(logitsv) + static_cast<int64_t>(wave) * E, E, k,
                        normalize, lane, R.ids + wave * k, R.w + wave * k);
    else
      topk_softmax_wave(static_cast<const float*>(logitsv) + static_cast<int64_t>(wave) * E, E, k,
                        normalize, lane, R.ids + wave * k, R.w + wave * k);
  }
  __syncthreads();
  const int nroutes = T * k;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = threadIdx.x; i < nroutes; i += 256) {
      ws_ids[i] = R.ids[i];
      ws_w[i] = R.w[i];
    }
  }
  const int r = blockIdx.y;
  const int e = R.ids[r];
  for (int q = 0; q < r; ++q)
    if (R.ids[q] == e) return;  // the first slot that chose e owns it
  int slot[kDecodeMaxTokens];
  token_slots(R, T, k, e, slot);

  const int units = H / 32;
  const int row_in_wave = lane / lpr, lane_in_row = lane % lpr;
  const int rows_wave = kWave / lpr;
  const uint8_t* ebase = codes + static_cast<int64_t>(e) * (2 * I) * row_bytes;
  const uint16_t* sbase = scales + static_cast<int64_t>(e) * (2 * I) * nblk;
  const uint8_t* zbase = fc1_zp ? fc1_zp + static_cast<int64_t>(e) * (2 * I) * nblk : nullptr;

  // activations of the tokens that use e, for this lane's units
  XPairs<BITS, UPL> xp[kDecodeMaxTokens];
  XFloats<UPL> xf[kDecodeMaxTokens];
#pragma unroll
  for (int t = 0; t < kDecodeMaxTokens; ++t) {
    if (slot[t] < 0) continue;
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      const int u = lane_in_row + lpr * i;
      if (u >= units) continue;
      if constexpr (ACT == kActBF16) {
        load_x_pairs<BITS>(static_cast<const uint16_t*>(xv) + static_cast<int64_t>(t) * H + 32 * u,
                           xp[t].p[i], xp[t].sum[i]);
      } else {
        // fp32 or fp16 activations, widened to fp32 (exact)
        const int64_t x0 = static_cast<int64_t>(t) * H + 32 * u;
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < 32; ++c) {
          xf[t].v[i][c] = load_act(xv, ACT, x0 + c);
          s += xf[t].v[i][c];
        }
        xf[t].sum[i] = s;
      }
    }
  }

  const int rows_per_wave = rows_block / 4;
  const int nsteps = rows_per_wave / rows_wave;
  const int n_wave0 = blockIdx.x * rows_block + wave * rows_per_wave + row_in_wave;
  for (int step = 0; step < nsteps; ++step) {
    const int n = n_wave0 + step * rows_wave;
    const bool valid = n < I;
    float g[kDecodeMaxTokens], up[kDecodeMaxTokens];
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) g[t] = up[t] = 0.0f;
    // gate and up rows of n (interleaved FC1: rows 2n and 2n+1)
    const int64_t gr = fc1_il ? 2 * static_cast<int64_t>(n) : n;
    const int64_t ur = fc1_il ? gr + 1 : static_cast<int64_t>(I) + n;
    if (valid) {
      UnitWords<BITS> gw[UPL], uw[UPL];
      float gs[UPL], us[UPL];
      int gz[UPL], uz[UPL];   // zero points of the gate and up rows' blocks
#pragma unroll
      for (int i = 0; i < UPL; ++i) {
        const int u = lane_in_row + lpr * i;
        if (u >= units) continue;
        gw[i] = load_unit<BITS>(ebase + gr * row_bytes + u * (4 * BITS));
        uw[i] = load_unit<BITS>(ebase + ur * row_bytes + u * (4 * BITS));
        gs[i] = half_to_f32(sbase[gr * nblk + (32 * u) / bs]);
        us[i] = half_to_f32(sbase[ur * nblk + (32 * u) / bs]);
        gz[i] = zbase ? static_cast<int>(zbase[gr * nblk + (32 * u) / bs]) : zp;
        uz[i] = zbase ? static_cast<int>(zbase[ur * nblk + (32 * u) / bs]) : zp;
      }
#pragma unroll
      for (int i = 0; i < UPL; ++i) {
        const int u = lane_in_row + lpr * i;
        if (u >= units) continue;
        if constexpr (ACT == kActBF16) {
          uint32_t gp[16], upp[16];
#pragma unroll
          for (int p = 0; p < 16; ++p) {
            gp[p] = unit_pair<BITS>(gw[i], p);
            upp[p] = unit_pair<BITS>(uw[i], p);
          }
#pragma unroll
          for (int t = 0; t < kDecodeMaxTokens; ++t) {
            if (slot[t] < 0) continue;
            const float gc = -(128.0f + static_cast<float>(gz[i])) * xp[t].sum[i];
            const float uc = -(128.0f + static_cast<float>(uz[i])) * xp[t].sum[i];
            g[t] = fmaf(gs[i], unit_dot_pairs<BITS>(gp, xp[t].p[i], gc), g[t]);
            up[t] = fmaf(us[i], unit_dot_pairs<BITS>(upp, xp[t].p[i], uc), up[t]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < kDecodeMaxTokens; ++t) {
            if (slot[t] < 0) continue;
            const float gzs = static_cast<float>(gz[i]) * xf[t].sum[i];
            const float uzs = static_cast<float>(uz[i]) * xf[t].sum[i];
            g[t] = fmaf(gs[i], unit_dot_f32<BITS>(gw[i], xf[t].v[i]) - gzs, g[t]);
            up[t] = fmaf(us[i], unit_dot_f32<BITS>(uw[i], xf[t].v[i]) - uzs, up[t]);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) {
      if (slot[t] < 0) continue;
      const float gt = group_sum(g[t], lpr) + (valid ? bias_at(fc1_bias, ACT, e * 2LL * I + gr) : 0.0f);
      const float ut = group_sum(up[t], lpr) + (valid ? bias_at(fc1_bias, ACT, e * 2LL * I + ur) : 0.0f);
      if (valid && lane_in_row == 0)
        h32[static_cast<int64_t>(t * k + slot[t]) * I + n] = silu_mul(gt, ut);
    }
  }
}

// grid = (fc2_row_blocks = ceil(H / rows_block), T * k), block = 256
template <int BITS, int UPL, int ACT>
__global__ __launch_bounds__(256) void decode_fc2_kernel(
    const float* __restrict__ h32, const int32_t* __restrict__ ws_ids,
    const float* __restrict__ ws_w, int T, int k, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, int H, int I, int bs, int zp, int64_t row_bytes,
    int64_t nblk, int lpr, int rows_block, const void* __restrict__ fc2_bias,
    const uint8_t* __restrict__ fc2_zp,
    float* __restrict__ y32) {
  __shared__ RoutingLds R;
  const int nroutes = T * k;
  for (int i = threadIdx.x; i < nroutes; i += 256) {
    R.ids[i] = ws_ids[i];
    R.w[i] = ws_w[i];
  }
  __syncthreads();

  const int r = blockIdx.y;
  const int e = R.ids[r];
  for (int q = 0; q < r; ++q)
    if (R.ids[q] == e) return;
  int slot[kDecodeMaxTokens];
  token_slots(R, T, k, e, slot);

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int units = I / 32;
  const int row_in_wave = lane / lpr, lane_in_row = lane % lpr;
  const int rows_wave = kWave / lpr;
  const uint8_t* ebase = codes + static_cast<int64_t>(e) * H * row_bytes;
  const uint16_t* sbase = scales + static_cast<int64_t>(e) * H * nblk;
  const uint8_t* zbase = fc2_zp ? fc2_zp + static_cast<int64_t>(e) * H * nblk : nullptr;

  XFloats<UPL> hf[kDecodeMaxTokens];
#pragma unroll
  for (int t = 0; t < kDecodeMaxTokens; ++t) {
    if (slot[t] < 0) continue;
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      const int u = lane_in_row + lpr * i;
      if (u >= units) continue;
      const float4* src =
          reinterpret_cast<const float4*>(h32 + static_cast<int64_t>(t * k + slot[t]) * I + 32 * u);
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float4 v = src[q];
        hf[t].v[i][4 * q + 0] = v.x; hf[t].v[i][4 * q + 1] = v.y;
        hf[t].v[i][4 * q + 2] = v.z; hf[t].v[i][4 * q + 3] = v.w;
        s += (v.x + v.y) + (v.z + v.w);
      }
      hf[t].sum[i] = s;
    }
  }

  const int rows_per_wave = rows_block / 4;
  const int nsteps = rows_per_wave / rows_wave;
  const int m0 = blockIdx.x * rows_block;
  const int m_wave0 = m0 + wave * rows_per_wave + row_in_wave;
  // Rows are taken in batches whose weight loads are all issued before any
  // of them is used, so their HBM latencies overlap instead of adding up
  // (with four units per lane the registers allow no batching).
  constexpr int kBatch = UPL == 1 ? 8 : UPL == 2 ? 4 : 1;
  for (int s0 = 0; s0 < nsteps; s0 += kBatch) {
    UnitWords<BITS> w[kBatch][UPL];
    float sc[kBatch][UPL];
    int zz[kBatch][UPL];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int m = m_wave0 + (s0 + b) * rows_wave;
      if (s0 + b >= nsteps || m >= H) continue;
#pragma unroll
      for (int i = 0; i < UPL; ++i) {
        const int u = lane_in_row + lpr * i;
        if (u >= units) continue;
        w[b][i] = load_unit<BITS>(ebase + static_cast<int64_t>(m) * row_bytes + u * (4 * BITS));
        sc[b][i] = half_to_f32(sbase[static_cast<int64_t>(m) * nblk + (32 * u) / bs]);
        zz[b][i] = zbase ? static_cast<int>(zbase[static_cast<int64_t>(m) * nblk + (32 * u) / bs]) : zp;
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (s0 + b >= nsteps) break;
      const int m = m_wave0 + (s0 + b) * rows_wave;
      const bool valid = m < H;
      float y[kDecodeMaxTokens];
#pragma unroll
      for (int t = 0; t < kDecodeMaxTokens; ++t) y[t] = 0.0f;
      if (valid) {
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
          const int u = lane_in_row + lpr * i;
          if (u >= units) continue;
#pragma unroll
          for (int t = 0; t < kDecodeMaxTokens; ++t) {
            if (slot[t] < 0) continue;
            const float d =
                unit_dot_f32<BITS>(w[b][i], hf[t].v[i]) - static_cast<float>(zz[b][i]) * hf[t].sum[i];
            y[t] = fmaf(sc[b][i], d, y[t]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < kDecodeMaxTokens; ++t) {
        if (slot[t] < 0) continue;
        const float yt = group_sum(y[t], lpr) + (valid ? bias_at(fc2_bias, ACT, e * static_cast<int64_t>(H) + m) : 0.0f);
        if (valid && lane_in_row == 0) y32[static_cast<int64_t>(t * k + slot[t]) * H + m] = yt;
      }
    }
  }

}

// out[t][m] = round(sum_j w[t][j] * y32[t*k + j][m]), slot order j = 0..k-1,
// one fp32 accumulator rounded once. grid = (ceil(H / 256), T), block = 256.
template <int ACT>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ y32,
                                                             const float* __restrict__ ws_w, int k,
                                                             int H, void* __restrict__ out) {
  const int t = blockIdx.y;
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= H) return;
  float acc = 0.0f;
  for (int j = 0; j < k; ++j)
    acc = fmaf(ws_w[t * k + j], __builtin_nontemporal_load(y32 + static_cast<int64_t>(t * k + j) * H + m), acc);
  store_act(out, ACT, static_cast<int64_t>(t) * H + m, acc);
}

namespace {

template <int BITS, int UPL>
hipError_t launch_decode_t(const Layer& L, const void* x, const void* logits, void* out, int64_t T,
                           char* ws, const Workspace& W, hipStream_t s, const GemvShape& s1,
                           const GemvShape& s2) {
  const int Ti = static_cast<int>(T), k = L.k, E = static_cast<int>(L.E);
  const int H = static_cast<int>(L.H), I = static_cast<int>(L.I);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + W.topk_id);
  float* w = reinterpret_cast<float*>(ws + W.topk_w);
  float* h32 = reinterpret_cast<float*>(ws + W.h32);
  dim3 g1((I + s1.rows_block - 1) / s1.rows_block, Ti * k);
  auto fc1 = L.act == kActBF16 ? decode_fc1_kernel<BITS, UPL, kActBF16>
             : L.act == kActF16 ? decode_fc1_kernel<BITS, UPL, kActF16>
                                : decode_fc1_kernel<BITS, UPL, kActF32>;
  fc1<<<g1, 256, 0, s>>>(x, logits, Ti, E, k, L.normalize, L.fc1_interleaved, L.fc1_bias, L.fc1_zp,
                         L.fc1_codes, L.fc1_scales, H, I, L.bs, L.zp, L.fc1_row_bytes, L.fc1_nblk,
                         s1.lpr, s1.rows_block, ids, w, h32);
  stage_done(L, 1, "decode_fc1_swiglu");
  return hipGetLastError();
}

template <int BITS, int UPL>
hipError_t launch_fc2_t(const Layer& L, void* out, int64_t T, char* ws, const Workspace& W,
                        hipStream_t s, const GemvShape& s2) {
  const int Ti = static_cast<int>(T), k = L.k;
  const int H = static_cast<int>(L.H), I = static_cast<int>(L.I);
  const int32_t* ids = reinterpret_cast<const int32_t*>(ws + W.topk_id);
  const float* w = reinterpret_cast<const float*>(ws + W.topk_w);
  const float* h32 = reinterpret_cast<const float*>(ws + W.h32);
  float* y32 = reinterpret_cast<float*>(ws + W.y32);
  dim3 g2(W.fc2_row_blocks, Ti * k);
  auto fc2 = L.act == kActBF16 ? decode_fc2_kernel<BITS, UPL, kActBF16>
             : L.act == kActF16 ? decode_fc2_kernel<BITS, UPL, kActF16>
                                : decode_fc2_kernel<BITS, UPL, kActF32>;
  fc2<<<g2, 256, 0, s>>>(h32, ids, w, Ti, k, L.fc2_codes, L.fc2_scales, H, I, L.bs, L.zp,
                         L.fc2_row_bytes, L.fc2_nblk, s2.lpr, s2.rows_block, L.fc2_bias, L.fc2_zp,
                         y32);
  stage_done(L, 2, "decode_fc2");
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 g3((H + 255) / 256, Ti);
  auto comb = L.act == kActBF16 ? decode_combine_kernel<kActBF16>
              : L.act == kActF16 ? decode_combine_kernel<kActF16>
                                 : decode_combine_kernel<kActF32>;
  comb<<<g3, 256, 0, s>>>(y32, w, k, H, out);
  stage_done(L, 3, "decode_combine");
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_decode_bits(const Layer& L, const void* x, const void* logits, void* out,
                              int64_t T, char* ws, const Workspace& W, hipStream_t s) {
  // FC1 workgroups cover 32 gate rows each when that still leaves at least
  // two workgroups per CU of a 256-CU part (ceil(I / 32) * T * k >= 512), else
  // 16: larger blocks recompute the routing prologue in fewer workgroups
  // (4 tokens: FC1 52 -> 41 us), smaller ones fill the chip when few routes
  // are active (1 token: 22 us at 16 rows, 28 us at 32).
  const int64_t wg32 = (L.I + 31) / 32 * T * L.k;
  const GemvShape s1 = gemv_shape(L.H, wg32 >= 512 ? 32 : 16);
  const GemvShape s2 = gemv_shape(L.I, 64);
  hipError_t err;
  switch (s1.upl) {
    case 1: err = launch_decode_t<BITS, 1>(L, x, logits, out, T, ws, W, s, s1, s2); break;
    case 2: err = launch_decode_t<BITS, 2>(L, x, logits, out, T, ws, W, s, s1, s2); break;
    default: err = launch_decode_t<BITS, 4>(L, x, logits, out, T, ws, W, s, s1, s2); break;
  }
  if (err != hipSuccess) return err;
  switch (s2.upl) {
    case 1: return launch_fc2_t<BITS, 1>(L, out, T, ws, W, s, s2);
    case 2: return launch_fc2_t<BITS, 2>(L, out, T, ws, W, s, s2);
    default: return launch_fc2_t<BITS, 4>(L, out, T, ws, W, s, s2);
  }
}

}  // namespace

hipError_t launch_decode(const Layer& L, const void* x, const void* logits, void* out, int64_t T,
                         char* ws, const Workspace& W, hipStream_t s) {
  switch (L.bits) {
    case 4: return launch_decode_bits<4>(L, x, logits, out, T, ws, W, s);
    case 3: return launch_decode_bits<3>(L, x, logits, out, T, ws, W, s);
    default: return launch_decode_bits<2>(L, x, logits, out, T, ws, W, s);
  }
}

}  // namespace qmoe
