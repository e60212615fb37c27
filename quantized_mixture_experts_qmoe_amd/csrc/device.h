// Device helpers for the gfx950 QMoE kernels: number formats, packed-code
// unpacking and wavefront reductions. Wave64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

constexpr int kWave = 64;
constexpr int kMaxTopK = 32;       // routing slots per token
constexpr int kMaxExperts = 1024;  // 16 logits per lane in the top-k wave
constexpr int kDecodeMaxTokens = 4;

// ---------------------------------------------------------------- formats

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet bit set).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 -> packed bf16 pair (low half = a) with the hardware conversion
// (v_cvt_pk_bf16_f32, round to nearest even).
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
typedef float f32x2_hw_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const f32x2_hw_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw_t));
}

__device__ __forceinline__ float half_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ float act_to_f32(float v) { return v; }
__device__ __forceinline__ float act_to_f32(uint16_t b) { return bf16_to_f32(b); }
__device__ __forceinline__ float act_to_f32(_Float16 h) { return static_cast<float>(h); }

// Activation dtypes of x, logits, out and the biases.
constexpr int kActF32 = 0, kActBF16 = 1, kActF16 = 2;

// Store v into element i of an activation-dtype array, rounding once (round
// to nearest even; NaN stays NaN).
__device__ __forceinline__ void store_act(void* p, int act, int64_t i, float v) {
  if (act == kActBF16)
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_bf16(v));
  else if (act == kActF16)
    static_cast<_Float16*>(p)[i] = static_cast<_Float16>(v);
  else
    static_cast<float*>(p)[i] = v;
}

// Element i of an activation-dtype array as fp32 (exact).
__device__ __forceinline__ float load_act(const void* p, int act, int64_t i) {
  if (act == kActBF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  if (act == kActF16) return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  return static_cast<const float*>(p)[i];
}

// ---------------------------------------------------------------- packed codes
//
// A "unit" is 32 consecutive codes of one row. Every supported block size is
// a multiple of 32, so a unit never straddles a scale block, and a unit is
// exactly BITS dwords: INT4 16 B, INT3 12 B, INT2 8 B.

template <int BITS>
struct UnitWords {
  uint32_t w[BITS];
};

template <int BITS>
__device__ __forceinline__ UnitWords<BITS> load_unit(const uint8_t* p) {
  UnitWords<BITS> u;
  if constexpr (BITS == 4) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    u.w[0] = v.x; u.w[1] = v.y; u.w[2] = v.z; u.w[3] = v.w;
  } else if constexpr (BITS == 2) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    u.w[0] = v.x; u.w[1] = v.y;
  } else {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    u.w[0] = q[0]; u.w[1] = q[1]; u.w[2] = q[2];
  }
  return u;
}

// Code i (0..31) of a unit, natural order. The packed stream is little-endian:
// code i occupies bits [BITS*i, BITS*i + BITS) of the unit's 32*BITS bits.
template <int BITS>
__device__ __forceinline__ uint32_t unit_code(const UnitWords<BITS>& u, int i) {
  const int bit = BITS * i;
  const int d = bit >> 5, o = bit & 31;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  if (o + BITS <= 32) return (u.w[d] >> o) & mask;
  return ((u.w[d] >> o) | (u.w[d + 1] << (32 - o))) & mask;
}

// Pair p (0..15) of a unit, as two bf16 values 128 + q_a (low half) and
// 128 + q_b (high half): the code is the low mantissa byte of bf16 128.0
// (0x4300), which is exact for q < 128 (the ulp at 128 is 1). pair_a/pair_b
// name the code indices so the activations can be paired the same way. INT4
// and INT2 pair codes 16 bits apart, i.e. two bytes apart once each byte
// holds one code: a mask (and a shift) per word puts one code in each byte,
// and one byte permute per pair inserts the 0x43 exponent bytes.
__host__ __device__ constexpr int pair_a(int bits, int p) {
  return bits == 4 ? 8 * (p / 4) + (p % 4) : bits == 2 ? 16 * (p / 8) + (p % 8) : 2 * p;
}
__host__ __device__ constexpr int pair_b(int bits, int p) {
  return bits == 4 ? 8 * (p / 4) + (p % 4) + 4 : bits == 2 ? 16 * (p / 8) + (p % 8) + 8 : 2 * p + 1;
}

template <int BITS>
__device__ __forceinline__ uint32_t unit_pair(const UnitWords<BITS>& u, int p) {
  // v_perm_b32 picks bytes of {0x43434343 (bytes 4-7), codes (bytes 0-3)}:
  // selector 0x04020400 makes (0x4300 | byte 0, 0x4300 | byte 2), 0x04030401
  // the same from bytes 1 and 3
  constexpr uint32_t kExp = 0x43434343u, kSel02 = 0x04020400u, kSel13 = 0x04030401u;
  if constexpr (BITS == 4) {
    // nibbles j and j + 4 of word p / 4 (j = p % 4): the even nibbles are the
    // bytes of w & 0x0F0F0F0F, the odd ones those of (w >> 4) & 0x0F0F0F0F
    const uint32_t w = u.w[p >> 2];
    const uint32_t f = (p & 1) ? ((w >> 4) & 0x0F0F0F0Fu) : (w & 0x0F0F0F0Fu);
    return __builtin_amdgcn_perm(kExp, f, (p & 2) ? kSel13 : kSel02);
  } else if constexpr (BITS == 2) {
    // fields j and j + 8 of word p / 8 (j = p % 8): field 4b + i is byte b of
    // (w >> 2i) & 0x03030303
    const uint32_t w = u.w[p >> 3];
    const uint32_t f = (w >> (2 * (p & 3))) & 0x03030303u;
    return __builtin_amdgcn_perm(kExp, f, (p & 4) ? kSel13 : kSel02);
  } else {
    return unit_code<3>(u, 2 * p) | (unit_code<3>(u, 2 * p + 1) << 16) | 0x43004300u;
  }
}

// ---------------------------------------------------------------- fp16 operands
//
// The grouped (prefill) GEMMs feed the matrix cores fp16 operands. A weight
// enters as fp16((q - zp) * s): round to nearest even of the exact product,
// with gradual underflow. dequant_unit_f16 forms it for the 32 codes of a
// unit, as 16 packed pairs in operand order (defined with it below):
//   1. each pair of codes becomes the fp16 pair (1024 + q_a, 1024 + q_b): the
//      code is OR-ed into the mantissa of 1024.0 (0x6400), exact for q < 1024;
//   2. adding -(1024 + zp) gives q - zp exactly (small integers);
//   3. one packed fp16 multiply by (s, s) rounds the exact product once.
// Step 3 is an IEEE product, so the result is fp16((q - zp) * s) for every
// scale pattern, infinities and NaN included (q = zp and s = inf gives NaN,
// as (q - zp) * s does).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f16_pair_scale(uint32_t biased_pair, f16x2_t off, f16x2_t sv) {
  const f16x2_t v = __builtin_bit_cast(f16x2_t, biased_pair);
  return __builtin_bit_cast(uint32_t, (v + off) * sv);
}

// Range exponents. A row or chunk of values with largest magnitude m is
// stored as fp16(v * 2^-e): e = 0 while m lies in [lo, 2^15] (or m is 0 or
// not finite), else the e that puts m in [2^14, 2^15), clamped to
// [-120, 120]. Activations use lo = 2^-3 (so every value at least 2^-14 of
// the row's largest stays a normal fp16 number), h chunks lo = 2^-14 (the
// smallest normal fp16 number; a chunk's values below it carry less than
// 2^-14 of the row's weight), which keeps ordinary chunks unscaled.
template <int LO_EXP>
__device__ __forceinline__ int range_exponent_lo(float m) {
  const bool out = (m > 32768.0f || (m > 0.0f && m < __builtin_ldexpf(1.0f, LO_EXP))) && m <= 3.4028235e38f;
  int ex = 0;
  (void)frexpf(m, &ex);
  return out ? min(max(ex - 15, -120), 120) : 0;
}
__device__ __forceinline__ int range_exponent(float m) { return range_exponent_lo<-3>(m); }
__device__ __forceinline__ int h_chunk_exponent(float m) { return range_exponent_lo<-14>(m); }

// The fp16 matrix operands of the batched paths hold their K values in an
// order of their own ("operand order") that lets the dequantization build a
// pair of codes with one shift and one mask: within each group of 8 (INT4)
// or 16 (INT2) K values, position 2j holds K value j and position 2j + 1 K
// value j + 4 (INT4) or j + 8 (INT2); INT3 keeps K order. Every operand of a
// dot product uses the same order (the activation rows and h are written in
// it), so the products are unchanged; only the order of the additions inside
// a matrix-core step differs.
__host__ __device__ constexpr int operand_perm(int bits) { return bits == 4 ? 8 : bits == 2 ? 16 : 0; }
// K value held at operand position pos
__host__ __device__ constexpr int operand_k(int perm, int pos) {
  return perm == 8    ? (pos & ~7) + ((pos & 7) >> 1) + 4 * (pos & 1)
         : perm == 16 ? (pos & ~15) + ((pos & 15) >> 1) + 8 * (pos & 1)
                      : pos;
}
// operand position of K value k
__host__ __device__ constexpr int operand_pos(int perm, int k) {
  return perm == 8    ? (k & ~7) + 2 * (k & 3) + ((k >> 2) & 1)
         : perm == 16 ? (k & ~15) + 2 * (k & 7) + ((k >> 3) & 1)
                      : k;
}

// One 32-code unit dequantized to the fp16 operand fp16((q - zp) * s), as
// 16 pairs in operand order (pair p = operand positions 2p, 2p + 1). Each
// pair is built exactly as the fp16 numbers 1024 + q (the code OR-ed into
// the mantissa of 1024.0), then a packed add of -(1024 + zp) (exact: small
// integers) and a packed multiply by the scale, the only rounding. Shared by
// both batched paths and the export of qmoe_dequant.
template <int BITS>
__device__ __forceinline__ void dequant_unit_f16(const UnitWords<BITS>& u, uint32_t scale_bits, int zp,
                                                 uint32_t (&out)[16]) {
  const _Float16 s = __builtin_bit_cast(_Float16, static_cast<uint16_t>(scale_bits));
  const f16x2_t sv = {s, s};
  const _Float16 o = static_cast<_Float16>(-(1024 + zp));
  const f16x2_t off = {o, o};
  // v_perm_b32 picks bytes of {0x64646464 (bytes 4-7), codes (bytes 0-3)}:
  // selector kSelEven builds (0x64 | byte 0, 0x64 | byte 2) as the fp16
  // pair (1024 + byte 0, 1024 + byte 2), kSelOdd the same from bytes 1, 3
  constexpr uint32_t kHigh = 0x64646464u, kSelEven = 0x04020400u, kSelOdd = 0x04030401u;
  if constexpr (BITS == 4) {
    // dword d holds codes 8d..8d+7 as nibbles; the low nibbles of its bytes
    // are codes 8d + {0, 2, 4, 6}, the high ones 8d + {1, 3, 5, 7}: pair
    // 4d + j = codes (8d + j, 8d + j + 4)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = u.w[d] & 0x0F0F0F0Fu, hi = (u.w[d] >> 4) & 0x0F0F0F0Fu;
      out[4 * d + 0] = f16_pair_scale(__builtin_amdgcn_perm(kHigh, lo, kSelEven), off, sv);
      out[4 * d + 1] = f16_pair_scale(__builtin_amdgcn_perm(kHigh, hi, kSelEven), off, sv);
      out[4 * d + 2] = f16_pair_scale(__builtin_amdgcn_perm(kHigh, lo, kSelOdd), off, sv);
      out[4 * d + 3] = f16_pair_scale(__builtin_amdgcn_perm(kHigh, hi, kSelOdd), off, sv);
    }
  } else if constexpr (BITS == 2) {
    // dword d holds codes 16d..16d+15, two bits each; bits [2i, 2i+2) of
    // its bytes are codes 16d + i + {0, 4, 8, 12}: pair 8d + j = codes
    // (16d + j, 16d + j + 8)
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t c = (u.w[d] >> (2 * i)) & 0x03030303u;
        out[8 * d + i] = f16_pair_scale(__builtin_amdgcn_perm(kHigh, c, kSelEven), off, sv);
        out[8 * d + 4 + i] = f16_pair_scale(__builtin_amdgcn_perm(kHigh, c, kSelOdd), off, sv);
      }
    }
  } else {
    // pair p = codes (2p, 2p + 1), the six bits [6p, 6p + 6) of the 96-bit unit
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int bit = 6 * p, d = bit >> 5, o6 = bit & 31;
      const uint32_t f = (o6 <= 26) ? (u.w[d] >> o6) & 63u
                                    : __builtin_amdgcn_alignbit(u.w[d + 1], u.w[d], o6) & 63u;
      const uint32_t pr = (f & 7u) | ((f >> 3) << 16);
      out[p] = f16_pair_scale(pr | 0x64006400u, off, sv);
    }
  }
}

// ---------------------------------------------------------------- activation staging

// The batched paths' activations, in operand order (P = operand_perm of the
// layer's bits), for token t, by one wave: bf16 and fp32 rows scaled by
// 2^-e_t and rounded once to fp16, e_t = range_exponent of the row's largest
// magnitude (0 for a row with a non-finite value), e_t to xexp[t]; fp16 rows
// copied as they are (no exponent). bf16 rows come through exactly (8
// significant bits), fp32 rows are rounded to 11. 16 consecutive values per
// lane.
template <int ACT, int P>
__device__ __forceinline__ void stage_x_row(const void* __restrict__ x, int64_t t, int H,
                                            uint16_t* __restrict__ x16, int8_t* __restrict__ xexp,
                                            int lane) {
  auto load16 = [&](int i, float (&v)[16]) {
    if constexpr (ACT == kActF32) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + t * H + i);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a = p[q];
        v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
      }
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + t * H + i);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 u = p[q];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t lo = static_cast<uint16_t>(w[j] & 0xFFFFu), hi = static_cast<uint16_t>(w[j] >> 16);
          v[8 * q + 2 * j] = ACT == kActBF16 ? bf16_to_f32(lo) : half_to_f32(lo);
          v[8 * q + 2 * j + 1] = ACT == kActBF16 ? bf16_to_f32(hi) : half_to_f32(hi);
        }
      }
    }
  };
  int e = 0;
  if constexpr (ACT != kActF16) {
    float m = 0.0f;
    bool finite = true;
    for (int i = lane * 16; i < H; i += kWave * 16) {
      float v[16];
      load16(i, v);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        finite = finite && (fabsf(v[j]) <= 3.4028235e38f);
        m = fmaxf(m, fabsf(v[j]));
      }
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    finite = __all(finite);
    e = finite ? range_exponent(m) : 0;
  }
  for (int i = lane * 16; i < H; i += kWave * 16) {
    float v[16];
    load16(i, v);
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float lo = v[operand_k(P, 2 * j)], hi = v[operand_k(P, 2 * j + 1)];
      const _Float16 a = static_cast<_Float16>(ACT == kActF16 ? lo : ldexpf(lo, -e));
      const _Float16 b = static_cast<_Float16>(ACT == kActF16 ? hi : ldexpf(hi, -e));
      o[j] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(x16 + t * H + i);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
  if (ACT != kActF16 && lane == 0) xexp[t] = static_cast<int8_t>(e);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// acc + a.lo*b.lo + a.hi*b.hi with bf16 inputs and fp32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Activation unit (32 bf16 values at x) -> pairs matching unit_pair<BITS>.
template <int BITS>
__device__ __forceinline__ void load_x_pairs(const uint16_t* x, uint32_t (&pairs)[16],
                                             float& sum) {
  uint32_t v[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 c = reinterpret_cast<const uint4*>(x)[q];
    v[4 * q + 0] = c.x; v[4 * q + 1] = c.y; v[4 * q + 2] = c.z; v[4 * q + 3] = c.w;
  }
  sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) sum += bf16_to_f32((v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int a = pair_a(BITS, p), b = pair_b(BITS, p);
    const uint32_t xa = (v[a >> 1] >> (16 * (a & 1))) & 0xFFFFu;
    const uint32_t xb = (v[b >> 1] >> (16 * (b & 1))) & 0xFFFFu;
    pairs[p] = xa | (xb << 16);
  }
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, kWave); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl_xor(lo, off, kWave);
  hi = __shfl_xor(hi, off, kWave);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// ---------------------------------------------------------------- routing

// Sortable key: larger key = larger logit, then lower expert index. -0 and +0
// compare equal (both map to the +0 key) so ties between them go to the lower
// index, as for any other equal logits.
__device__ __forceinline__ uint64_t route_key(float v, uint32_t e) {
  uint32_t u = __float_as_uint(v);
  if (v == 0.0f) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | (0xFFFFFFFFu - e);
}

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t u = static_cast<uint32_t>(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}

__device__ __forceinline__ int key_expert(uint64_t key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

// Routing key of a bf16 logit: the order-preserving 16-bit image of the value
// (-0 folded into +0) above the inverted expert index, so the largest key is
// the largest logit and, among equal logits, the lowest expert index.
__device__ __forceinline__ uint32_t logit_key(uint32_t b, int e) {
  b = (b == 0x8000u) ? 0u : b;
  const uint32_t ord = (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
  return (ord << 16) | (0xFFFFu - static_cast<uint32_t>(e));
}
__device__ __forceinline__ float key_logit(uint32_t key) {
  const uint32_t ord = key >> 16;
  return bf16_to_f32((ord & 0x8000u) ? (ord & 0x7FFFu) : (~ord & 0xFFFFu));
}
__device__ __forceinline__ int key_to_expert(uint32_t key) {
  return 0xFFFF - static_cast<int>(key & 0xFFFFu);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  const uint32_t p = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(v), static_cast<int>(v), CTRL, ROWS, 0xF, false));
  return p > v ? p : v;
}

// Maximum over the wavefront, returned uniformly.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = dpp_umax<0x128, 0xF>(v);   // row_ror:8
  v = dpp_umax<0x124, 0xF>(v);   // row_ror:4
  v = dpp_umax<0x122, 0xF>(v);   // row_ror:2
  v = dpp_umax<0x121, 0xF>(v);   // row_ror:1
  v = dpp_umax<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_umax<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// One wavefront selects the top-k experts of one token and computes their
// routing weights: the softmax over the k selected logits (normalize), or each
// selected expert's softmax probability over all E logits. Slot j holds the
// j-th largest logit (ties to the lower expert index). Lanes j < k write
// ids[j] and w[j].
template <typename ACT>
__device__ __forceinline__ void topk_softmax_wave_r(const ACT* logits, int E, int k, bool normalize,
                                                    int lane, int& id, float& wt) {
  uint64_t keys[kMaxExperts / kWave];
#pragma unroll
  for (int i = 0; i < kMaxExperts / kWave; ++i) {
    const int e = lane + kWave * i;
    keys[i] = (e < E) ? route_key(act_to_f32(logits[e]), static_cast<uint32_t>(e)) : 0ull;
  }
  const int epl = (E + kWave - 1) / kWave;
  int my_id = 0;
  float my_v = 0.0f, v0 = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < kMaxExperts / kWave; ++i)
      if (i < epl && keys[i] > best) best = keys[i];
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
      uint64_t o = shfl_xor_u64(best, off);
      best = o > best ? o : best;
    }
    const int e = key_expert(best);
    const float v = key_value(best);
    if (j == 0) v0 = v;
    if (lane == j) { my_id = e; my_v = v; }
#pragma unroll
    for (int i = 0; i < kMaxExperts / kWave; ++i)
      if (lane == (e & (kWave - 1)) && i == (e / kWave)) keys[i] = 0ull;
  }
  const float ex = (lane < k) ? expf(my_v - v0) : 0.0f;
  float all = 0.0f;   // sum over all experts (weights without normalization)
  if (!normalize)
    for (int e = lane; e < E; e += kWave) all += expf(act_to_f32(logits[e]) - v0);
  const float sum = wave_sum(normalize ? ex : all);
  id = my_id;
  wt = ex / sum;
}
template <typename ACT>
__device__ __forceinline__ void topk_softmax_wave(const ACT* logits, int E, int k, bool normalize,
                                                  int lane, int32_t* ids, float* w) {
  int id;
  float wt;
  topk_softmax_wave_r(logits, E, k, normalize, lane, id, wt);
  if (lane < k) {
    ids[lane] = id;
    w[lane] = wt;
  }
}

// The same selection for bf16 logits with 32-bit keys (logit_key) and DPP
// reductions; SLOTS logits per lane (E <= 64 * SLOTS). Lanes j < k receive
// slot j's expert and weight.
template <int SLOTS>
__device__ __forceinline__ void topk_softmax_bf16_wave(const uint16_t (&lg)[SLOTS], int E, int k,
                                                       bool normalize, int lane, int& id, float& wt) {
  uint32_t keys[SLOTS];
#pragma unroll
  for (int c = 0; c < SLOTS; ++c) {
    const int e = lane + kWave * c;
    keys[c] = (e < E) ? logit_key(lg[c], e) : 0u;
  }
  uint32_t mine = 0u, first = 0u;
  for (int j = 0; j < k; ++j) {
    uint32_t b = keys[0];
#pragma unroll
    for (int c = 1; c < SLOTS; ++c) b = keys[c] > b ? keys[c] : b;
    b = wave_umax(b);
    if (j == 0) first = b;
    if (lane == j) mine = b;
#pragma unroll
    for (int c = 0; c < SLOTS; ++c) keys[c] = (keys[c] == b) ? 0u : keys[c];
  }
  const float ex = (lane < k) ? expf(key_logit(mine) - key_logit(first)) : 0.0f;
  float all = 0.0f;   // sum over all experts (weights without normalization)
  if (!normalize)
#pragma unroll
    for (int c = 0; c < SLOTS; ++c)
      if (lane + kWave * c < E) all += expf(bf16_to_f32(lg[c]) - key_logit(first));
  const float sum = wave_sum(normalize ? ex : all);
  id = key_to_expert(mine);
  wt = ex / sum;
}

// Element i of an optional bias in the activation dtype (0 when absent).
__device__ __forceinline__ float bias_at(const void* b, int act, int64_t i) {
  return b ? load_act(b, act, i) : 0.0f;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// silu(g) * u with the hardware exp2 and reciprocal (a few ulp in fp32), for
// epilogues that round h to bf16 right after.
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

}  // namespace qmoe
