// Test export: materialize one expert matrix with the kernels' own unpacking.
//
//   out_f32[n][k]  = (q - zp) * s as the decode GEMV reads it (zp the scalar
//                    zero point or the row's per-block code): the code comes
//                    back out of the bf16 pair 128 + q that unit_pair builds
//                    (exact), placed at the code index pair_a/pair_b name;
//   out_f16[n][k]  = the fp16 operand fp16((q - zp) * s) the batched paths
//                    feed the matrix cores, from the same routine
//                    (dequant_unit_f16), moved from operand order to K order.
//
// Dequantization W = (q - zp) * s[n][k / block] ("[CUDA] Add INT4 and INT3
// QMoE CPU/GPU offload support", Description: raw integer experts, block
// sizes 32/64/128, scales [N, K/block]).
#include "device.h"
#include "internal.h"

namespace qmoe {

// one thread per 32-code unit; grid = ceil(N * K/32 / 256)
template <int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint8_t* __restrict__ zps, int64_t N,
                                                      int64_t K, int bs, int zp, int64_t row_bytes,
                                                      int64_t nblk, float* __restrict__ out_f32,
                                                      uint16_t* __restrict__ out_f16) {
  const int64_t units = K / 32;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= N * units) return;
  const int64_t n = gid / units, u = gid % units;
  const UnitWords<BITS> w = load_unit<BITS>(codes + n * row_bytes + u * (4 * BITS));
  const uint16_t sbits = scales[n * nblk + (32 * u) / bs];
  const float s = half_to_f32(sbits);
  if (zps) zp = zps[n * nblk + (32 * u) / bs];   // per-block zero point
  const int64_t base = n * K + 32 * u;
  if (out_f32) {
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const uint32_t pr = unit_pair<BITS>(w, p);
      const float qa = bf16_to_f32(pr & 0xFFFFu) - 128.0f;
      const float qb = bf16_to_f32(pr >> 16) - 128.0f;
      out_f32[base + pair_a(BITS, p)] = (qa - static_cast<float>(zp)) * s;
      out_f32[base + pair_b(BITS, p)] = (qb - static_cast<float>(zp)) * s;
    }
  }
  if (out_f16) {
    // pairs in operand order, written back to their K positions
    uint32_t pairs[16];
    dequant_unit_f16<BITS>(w, sbits, zp, pairs);
    constexpr int P = operand_perm(BITS);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      out_f16[base + operand_k(P, 2 * p)] = static_cast<uint16_t>(pairs[p] & 0xFFFFu);
      out_f16[base + operand_k(P, 2 * p + 1)] = static_cast<uint16_t>(pairs[p] >> 16);
    }
  }
}

hipError_t launch_dequant(const Layer& L, int fc, int64_t expert, float* out_f32,
                          uint16_t* out_f16, hipStream_t s) {
  const int64_t N = fc == 1 ? 2 * L.I : L.H;
  const int64_t K = fc == 1 ? L.H : L.I;
  const int64_t rb = fc == 1 ? L.fc1_row_bytes : L.fc2_row_bytes;
  const int64_t nb = fc == 1 ? L.fc1_nblk : L.fc2_nblk;
  const uint8_t* c = (fc == 1 ? L.fc1_codes : L.fc2_codes) + expert * N * rb;
  const uint16_t* sc = (fc == 1 ? L.fc1_scales : L.fc2_scales) + expert * N * nb;
  const uint8_t* zb = fc == 1 ? L.fc1_zp : L.fc2_zp;
  const uint8_t* z = zb ? zb + expert * N * nb : nullptr;
  const int64_t threads = N * (K / 32);
  const unsigned grid = static_cast<unsigned>((threads + 255) / 256);
  switch (L.bits) {
    case 4: dequant_kernel<4><<<grid, 256, 0, s>>>(c, sc, z, N, K, L.bs, L.zp, rb, nb, out_f32, out_f16); break;
    case 3: dequant_kernel<3><<<grid, 256, 0, s>>>(c, sc, z, N, K, L.bs, L.zp, rb, nb, out_f32, out_f16); break;
    default: dequant_kernel<2><<<grid, 256, 0, s>>>(c, sc, z, N, K, L.bs, L.zp, rb, nb, out_f32, out_f16); break;
  }
  return hipGetLastError();
}

}  // namespace qmoe
