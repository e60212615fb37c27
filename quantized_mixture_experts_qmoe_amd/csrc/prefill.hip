// Prefill path (5+ tokens): expert-grouped GEMMs on the CDNA4 matrix cores.
//
// The routing stage leaves the routes sorted by expert and a tile list
// (expert, first sorted row, rows). Each workgroup computes one 128 x 128
// output tile of one expert:
//   FC1: A = x rows gathered through sorted_routes (bf16), B = the expert's
//        gate rows [n0, n0+64) and up rows [I+n0, I+n0+64), dequantized into
//        LDS as bf16; the epilogue applies h = silu(gate) * up and stores h
//        as bf16 [R, I] in sorted order.
//   FC2: A = h rows of the tile (bf16), B = the expert's FC2 rows
//        [n0, n0+128) dequantized into LDS; the epilogue stores fp32 y
//        [R, H] in sorted order.
// A combine kernel then sums each token's k slots in slot order and rounds
// once.
//
// Semantics: grouped prefill over expert-sorted routes with tile descriptors
// ("[CUDA] Add INT4 and INT3 QMoE CPU/GPU offload support", description of
// the tensor-core INT3/INT4 prefill in the stacked PR); SwiGLU contract
// ("[CUDA/CPU] Add AVX2 INT4 cold-expert kernel and zero-cold doorbell
// short-circuit for QMoE offload", Motivation & Summary item 3); fp32
// combine rounded once ("[CUDA] Add MoEPacked CPU/GPU hybrid offload and
// consolidate QMoE/GGUF offload optimizations", Key Changes item 4).
#include "device.h"
#include "internal.h"

namespace qmoe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

namespace {

constexpr int kKT = 64;              // K per LDS stage (two 16x16x32 MFMA steps)
constexpr int kLdsStride = kKT + 8;  // bf16 elements per LDS row (padding against bank conflicts)

// Logical tile index of this workgroup. Workgroups are dealt to the 8 XCDs
// round-robin; consecutive logical tiles are kept on one XCD so the n-tiles
// of one m-tile (which share their A rows) meet in the same L2.
__device__ __forceinline__ int logical_tile(int active) {
  const int b = blockIdx.x;
  const int per_xcd = (active + 7) / 8;
  const int j = b / 8;
  if (j >= per_xcd) return -1;
  const int L = (b % 8) * per_xcd + j;
  return L < active ? L : -1;
}

}  // namespace

// grid = 8 * ceil(max_tiles * n_tiles_n / 8), block = 256 (2 x 2 waves of 64 x 64)
template <int BITS, bool FC1>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(
    const uint16_t* __restrict__ a_src, const int32_t* __restrict__ sorted_routes, int k,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int K, int H, int I,
    int bs, int zp, int64_t row_bytes, int64_t nblk, const int4* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int n_tiles_n, uint16_t* __restrict__ h_out,
    float* __restrict__ y_out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kTileM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kTileN * kLdsStride];

  const int active = num_tiles[0] * n_tiles_n;
  const int L = logical_tile(active);
  if (L < 0) return;
  const int m_tile = L / n_tiles_n, n_tile = L % n_tiles_n;
  const int4 td = tiles[m_tile];
  const int e = td.x, row0 = td.y, nrows = td.z;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_rows_total = FC1 ? 2 * I : H;                    // rows of W
  const uint8_t* ebase = codes + static_cast<int64_t>(e) * n_rows_total * row_bytes;
  const uint16_t* sbase = scales + static_cast<int64_t>(e) * n_rows_total * nblk;

  // this thread's B row (one 32-code unit per K stage)
  const int b_row = tid >> 1, b_half = tid & 1;
  int w_row;
  bool b_valid;
  if (FC1) {
    const int n0 = n_tile * 64;
    const int c = n0 + (b_row & 63);
    b_valid = c < I;
    w_row = (b_row < 64) ? c : I + c;
  } else {
    const int c = n_tile * kTileN + b_row;
    b_valid = c < H;
    w_row = c;
  }

  // this thread's A rows: 4 chunks of 8 bf16 per stage
  const int64_t a_ld = FC1 ? H : I;
  const uint16_t* a_ptr[4];
  int a_row[4], a_col[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + 256 * q;
    a_row[q] = c >> 3;
    a_col[q] = (c & 7) * 8;
    if (a_row[q] < nrows) {
      const int64_t src_row = FC1 ? (sorted_routes[row0 + a_row[q]] / k) : (row0 + a_row[q]);
      a_ptr[q] = a_src + src_row * a_ld;
    } else {
      a_ptr[q] = nullptr;
    }
  }

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int quad = lane >> 4, l16 = lane & 15;
  for (int k0 = 0; k0 < K; k0 += kKT) {
    // ---- stage A
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (a_ptr[q] && k0 + a_col[q] < K) v = *reinterpret_cast<const uint4*>(a_ptr[q] + k0 + a_col[q]);
      *reinterpret_cast<uint4*>(&As[a_row[q] * kLdsStride + a_col[q]]) = v;
    }
    // ---- stage B: dequantize one unit
    {
      uint32_t pairs[16];
      const int kk = k0 + 32 * b_half;
      if (b_valid && kk < K) {
        const UnitWords<BITS> u =
            load_unit<BITS>(ebase + static_cast<int64_t>(w_row) * row_bytes + (kk / 32) * (4 * BITS));
        const float s = half_to_f32(sbase[static_cast<int64_t>(w_row) * nblk + kk / bs]);
        dequant_unit_bf16<BITS>(u, s, zp, pairs);
      } else {
#pragma unroll
        for (int p = 0; p < 16; ++p) pairs[p] = 0u;
      }
      uint4* dst = reinterpret_cast<uint4*>(&Bs[b_row * kLdsStride + 32 * b_half]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dst[q] = make_uint4(pairs[4 * q], pairs[4 * q + 1], pairs[4 * q + 2], pairs[4 * q + 3]);
    }
    __syncthreads();
    // ---- MFMA
#pragma unroll
    for (int ks = 0; ks < kKT / 32; ++ks) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) {
        const int r = wm * 64 + tm * 16 + l16;
        af[tm] = *reinterpret_cast<const bf16x8_t*>(&As[r * kLdsStride + ks * 32 + quad * 8]);
      }
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        int r;
        if (FC1) r = (tn < 2 ? 0 : 64) + wn * 32 + (tn & 1) * 16 + l16;
        else r = wn * 64 + tn * 16 + l16;
        bfr[tn] = *reinterpret_cast<const bf16x8_t*>(&Bs[r * kLdsStride + ks * 32 + quad * 8]);
      }
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], bfr[tn], acc[tm][tn], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*quad + i, column l16 of each 16x16 tile
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = wm * 64 + tm * 16 + quad * 4 + i;
      if (p >= nrows) continue;
      const int64_t orow = row0 + p;
      if (FC1) {
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
          const int c = n_tile * 64 + wn * 32 + tn * 16 + l16;
          if (c < I) {
            const float hv = silu_mul(acc[tm][tn][i], acc[tm][tn + 2][i]);
            h_out[orow * I + c] = static_cast<uint16_t>(f32_to_bf16(hv));
          }
        }
      } else {
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
          const int c = n_tile * kTileN + wn * 64 + tn * 16 + l16;
          if (c < H) y_out[orow * H + c] = acc[tm][tn][i];
        }
      }
    }
  }
}

// out[t][m] = round(sum_j w[t][j] * y[inv_pos[t*k + j]][m]), slot order j = 0..k-1.
// grid = (ceil(H / 1024), T), block = 256, 4 columns per thread.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ topk_w, int k,
                                                      int H, void* __restrict__ out) {
  const int64_t t = blockIdx.y;
  const int m = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (m >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int64_t p = inv_pos[t * k + j];
    const float w = topk_w[t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + p * H + m);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  if constexpr (OUT_BF16) {
    uint2 o;
    o.x = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
    o.y = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + t * H + m) = o;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + t * H + m) = acc;
  }
}

// fp32 activations are staged for the matrix cores as bf16 (round to nearest
// even) once per call.
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ in, int64_t n,
                                                          uint16_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) out[i] = static_cast<uint16_t>(f32_to_bf16(in[i]));
}

namespace {

template <int BITS>
hipError_t launch_gemms(const Layer& L, const uint16_t* xb, char* ws, const Workspace& W,
                        hipStream_t s) {
  const int H = static_cast<int>(L.H), I = static_cast<int>(L.I);
  const int32_t* sorted = reinterpret_cast<const int32_t*>(ws + W.sorted_routes);
  const int4* tiles = reinterpret_cast<const int4*>(ws + W.tiles);
  const int32_t* ntiles = reinterpret_cast<const int32_t*>(ws + W.num_tiles);
  uint16_t* hb = reinterpret_cast<uint16_t*>(ws + W.hbf16);
  float* yf = reinterpret_cast<float*>(ws + W.yf32);
  const int nt1 = (I + 63) / 64;
  const int nt2 = (H + kTileN - 1) / kTileN;
  const int64_t g1 = 8 * ((W.max_tiles * nt1 + 7) / 8);
  const int64_t g2 = 8 * ((W.max_tiles * nt2 + 7) / 8);
  grouped_gemm_kernel<BITS, true><<<static_cast<unsigned>(g1), 256, 0, s>>>(
      xb, sorted, L.k, L.fc1_codes, L.fc1_scales, H, H, I, L.bs, L.zp, L.fc1_row_bytes, L.fc1_nblk,
      tiles, ntiles, nt1, hb, nullptr);
  stage_done(L, 6, "gemm_fc1_swiglu");
  grouped_gemm_kernel<BITS, false><<<static_cast<unsigned>(g2), 256, 0, s>>>(
      hb, sorted, L.k, L.fc2_codes, L.fc2_scales, I, H, I, L.bs, L.zp, L.fc2_row_bytes, L.fc2_nblk,
      tiles, ntiles, nt2, nullptr, yf);
  stage_done(L, 7, "gemm_fc2");
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const Layer& L, const void* x, void* out, int64_t T, char* ws,
                          const Workspace& W, hipStream_t s) {
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (!L.act_bf16) {
    uint16_t* staged = reinterpret_cast<uint16_t*>(ws + W.xbf16);
    const int64_t n = T * L.H;
    f32_to_bf16_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
        static_cast<const float*>(x), n, staged);
    stage_done(L, 5, "stage_x_bf16");
    xb = staged;
  }
  hipError_t err;
  switch (L.bits) {
    case 4: err = launch_gemms<4>(L, xb, ws, W, s); break;
    case 3: err = launch_gemms<3>(L, xb, ws, W, s); break;
    default: err = launch_gemms<2>(L, xb, ws, W, s); break;
  }
  if (err != hipSuccess) return err;
  const int H = static_cast<int>(L.H);
  dim3 gc((H / 4 + 255) / 256, static_cast<unsigned>(T));
  const float* yf = reinterpret_cast<const float*>(ws + W.yf32);
  const int32_t* inv = reinterpret_cast<const int32_t*>(ws + W.inv_pos);
  const float* w = reinterpret_cast<const float*>(ws + W.topk_w);
  if (L.act_bf16)
    combine_kernel<true><<<gc, 256, 0, s>>>(yf, inv, w, L.k, H, out);
  else
    combine_kernel<false><<<gc, 256, 0, s>>>(yf, inv, w, L.k, H, out);
  stage_done(L, 8, "combine");
  return hipGetLastError();
}

}  // namespace qmoe
