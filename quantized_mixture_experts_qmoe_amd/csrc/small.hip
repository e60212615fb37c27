// Small-batch path (5 to a few hundred tokens): expert-grouped GEMMs whose
// weights stream from HBM straight into the matrix cores.
//
// Between four tokens and a few hundred, each active expert serves only a
// handful of routes. The grouped GEMMs of the prefill path stage every
// weight tile through LDS for 256-row tiles that are nearly empty; here each
// expert's weights are read once per call and go from registers to the
// matrix cores.
//
// Routing (top-k, histogram, scan, stable scatter) and the activation
// staging run in one launch while the route list fits in LDS (else the
// prefill path's launches), with tiles of at most 16 routes of one expert. Each workgroup (8 waves)
// takes one tile and a block of output columns:
//   FC1: the tile's activation rows (fp16, staged per token as for the
//        prefill GEMMs) go to LDS once; each wave owns 16 h columns, streams
//        the matching 16 gate and 16 up weight rows, dequantizes each
//        32-code unit to fp16((q - zp) * s) in registers (the routine the
//        prefill GEMMs and the export use) and feeds
//        v_mfma_f32_16x16x32_f16; the epilogue applies SwiGLU and stores h
//        in fp32 [R, I] in sorted order;
//   FC2: the tile's h rows go to LDS as fp16 with a per-route exponent (the
//        range exponent of the row, so no value leaves fp16 range); each
//        wave owns 32 output columns; the epilogue stores y in fp32 [R, H],
//        which the prefill path's combine sums per token in slot order and
//        rounds once.
// Lane (q, n) of a wave (q = lane / 16, n = lane % 16) feeds the matrix
// cores, for each 128-K sub-block, unit 4s + q (32 codes) of weight row n:
// its 32 values are the B operand of the sub-block's four MFMA steps, K
// values 32(4s + q) + 8t + 0..7 at step t, and the A operand of step t is
// read from the same K range of the staged rows. The weights are loaded in
// whole row segments (StreamLanes, RowGroup) and handed to that layout across
// lanes, so every weight byte is loaded once per call, by one lane.
//
// Semantics: grouped experts over expert-sorted routes ("[CUDA] Add INT4 and
// INT3 QMoE CPU/GPU offload support", Description of the grouped prefill
// path); SwiGLU contract ("[CUDA/CPU] Add AVX2 INT4 cold-expert kernel and
// zero-cold doorbell short-circuit for QMoE offload", Motivation & Summary
// item 3); fp32 partial sums rounded once ("[CUDA] Add MoEPacked CPU/GPU
// hybrid offload and consolidate QMoE/GGUF offload optimizations", Key
// Changes item 4).
#include "device.h"
#include "internal.h"

namespace qmoe {

namespace {

typedef _Float16 sf16x8_t __attribute__((ext_vector_type(8)));
typedef float sf32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSmallWaves = 8;
constexpr int kSmallThreads = kSmallWaves * kWave;
constexpr int kFc1Groups = 1;                        // 16-column groups of h per FC1 wave
constexpr int kFc2Groups = 4;                        // 16-row groups of outputs per FC2 wave
constexpr int kFc1Depth = 2;                         // row blocks in flight per FC1 row group
constexpr int kFc2Depth = 1;                         // and per FC2 row group
constexpr int kTransBytes = 2048;                    // per-wave LDS slice for a block's units
constexpr int kFc1Cols = kSmallWaves * 16 * kFc1Groups;   // h columns per FC1 workgroup
constexpr int kFc2Cols = kSmallWaves * 16 * kFc2Groups;   // output columns per FC2 workgroup

// Logical index of this workgroup: the column blocks of one tile (which
// share its staged rows) are dealt to one XCD.
__device__ __forceinline__ int small_logical(int active) {
  const int b = blockIdx.x;
  const int per_xcd = (active + 7) / 8;
  const int j = b / 8;
  if (j >= per_xcd) return -1;
  const int L = (b % 8) * per_xcd + j;
  return L < active ? L : -1;
}

// Weight rows stream in groups of sixteen (row n of a group is the MFMA
// column of the lanes with l16 = n), in blocks of UB units per row. Each
// load instruction reads UB consecutive units (128 bytes for INT4 and INT2,
// 96 for INT3) of each of RPI rows: lane l loads unit (l mod UB) of row
// RPI * m + l / UB in instruction m. Rows read in such whole segments keep
// HBM streaming at full rate, where 64-byte pieces of 16 rows at a time
// fall to about two thirds of it. ds_bpermute then hands lane (q, n) the
// unit 4s + q of its own row n for each 128-K sub-block s, the layout the
// matrix cores' B operand takes. Units past K get a zero scale (their
// addresses are clamped to the row's first unit).
template <int BITS>
struct StreamLanes {
  static constexpr int UB = BITS == 2 ? 16 : 8;   // units per row per block
  static constexpr int RPI = kWave / UB;          // rows per load instruction
  static constexpr int NI = 16 / RPI;             // load instructions per block
  static constexpr int SB = UB / 4;               // 128-K sub-blocks per block
  int lu, q, msel;
  int64_t cofs[NI];   // byte offset (from the group's first row) of the row this lane
                      // loads in instruction m
  int64_t sofs;       // element offset of this lane's own row's scales
  static constexpr int SLOT = BITS == 2 ? 8 : 16;   // bytes per unit in the LDS slice
  int tofs[SB];       // byte offset, in the wave's LDS slice, of the unit this lane takes
  // rows of every group a wave streams lie rstride bytes apart (their
  // scales and zero points sstride elements apart)
  __device__ __forceinline__ StreamLanes(int lane, int64_t rstride, int64_t sstride) {
    lu = lane % UB;
    q = lane >> 4;
    const int n = lane & 15;
    msel = n / RPI;
#pragma unroll
    for (int m = 0; m < NI; ++m) cofs[m] = (RPI * m + lane / UB) * rstride;
    sofs = n * sstride;
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) tofs[sb] = (msel * kWave + (n % RPI) * UB + 4 * sb + q) * SLOT;
  }
};

// Sixteen rows: the codes, scales and zero points of the group's first row
// (the same pointers for every lane of a wave).
struct RowGroup {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint8_t* zps;
};

template <int BITS>
struct RowBlock {
  UnitWords<BITS> raw[StreamLanes<BITS>::NI];
  uint32_t s[StreamLanes<BITS>::SB];
  int z[StreamLanes<BITS>::SB];
};

template <int BITS, bool HAS_ZP>
__device__ __forceinline__ void load_block(const StreamLanes<BITS>& ln, const RowGroup& g, int b, int nunits,
                                           int ushift, int zp, RowBlock<BITS>& blk) {
  using SL = StreamLanes<BITS>;
  // a unit past K reads the row's first unit (unused: its scale is zero)
  const int u = b * SL::UB + ln.lu;
  const int uc = u < nunits ? u : 0;
#pragma unroll
  for (int m = 0; m < SL::NI; ++m) blk.raw[m] = load_unit<BITS>(g.codes + ln.cofs[m] + uc * (4 * BITS));
#pragma unroll
  for (int sb = 0; sb < SL::SB; ++sb) {
    const int v = b * SL::UB + 4 * sb + ln.q;
    const int vc = v < nunits ? v : 0;
    blk.s[sb] = v < nunits ? g.scales[ln.sofs + (vc >> ushift)] : 0u;   // past K weighs zero
    blk.z[sb] = HAS_ZP ? g.zps[ln.sofs + (vc >> ushift)] : zp;
  }
}

// A block's units go through the wave's LDS slice (kTransBytes): each lane
// stores the units it loaded (instruction m at slot m * 64 + lane), then
// reads back unit 4 * sb + q of its own row for each sub-block. The slice
// is the wave's own and LDS accesses of a wave complete in order, so no
// barrier is needed.
template <int BITS>
__device__ __forceinline__ void stash_block(const RowBlock<BITS>& blk, uint8_t* tb, int lane) {
  using SL = StreamLanes<BITS>;
#pragma unroll
  for (int m = 0; m < SL::NI; ++m) {
    uint8_t* p = tb + (m * kWave + lane) * SL::SLOT;
    if constexpr (BITS == 2) {
      *reinterpret_cast<uint2*>(p) = make_uint2(blk.raw[m].w[0], blk.raw[m].w[1]);
    } else if constexpr (BITS == 4) {
      *reinterpret_cast<uint4*>(p) = make_uint4(blk.raw[m].w[0], blk.raw[m].w[1], blk.raw[m].w[2], blk.raw[m].w[3]);
    } else {
      *reinterpret_cast<uint4*>(p) = make_uint4(blk.raw[m].w[0], blk.raw[m].w[1], blk.raw[m].w[2], 0u);
    }
  }
}

template <int BITS>
__device__ __forceinline__ UnitWords<BITS> fetch_unit(const StreamLanes<BITS>& ln, const uint8_t* tb, int sb) {
  UnitWords<BITS> w;
  const uint8_t* p = tb + ln.tofs[sb];
  if constexpr (BITS == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w.w[0] = v.x; w.w[1] = v.y;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w.w[0] = v.x; w.w[1] = v.y; w.w[2] = v.z;
    if constexpr (BITS == 4) w.w[3] = v.w;
  }
  return w;
}

// Staged rows are K fp16 values each, in 16-byte pieces: piece c of row r
// sits at piece c ^ (r mod 16) of the row (K is a multiple of 128, so the
// swizzle stays inside the row), so the 16 rows an MFMA step reads at one
// column fall in 16 different pieces of LDS.
__device__ __forceinline__ int swz(int r, int piece) { return 8 * (piece ^ (r & 15)); }

// acc += A(rows of the block) x B(one unit of one weight row), four steps;
// arow is this lane's row (l16), col0 the unit's first column.
__device__ __forceinline__ sf32x4_t mfma_unit(const uint16_t* arow, int l16, int col0,
                                              const uint32_t (&pairs)[16], sf32x4_t acc) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const sf16x8_t a = *reinterpret_cast<const sf16x8_t*>(arow + swz(l16, (col0 >> 3) + t));
    const uint4 b4 = make_uint4(pairs[4 * t], pairs[4 * t + 1], pairs[4 * t + 2], pairs[4 * t + 3]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(sf16x8_t, b4), acc, 0, 0, 0);
  }
  return acc;
}

}  // namespace

// FC1 + SwiGLU over one tile (<= 16 routes of expert e) and kFc1Cols h columns.
// grid = 8 * ceil(max_tiles * n_blocks / 8), block = 512, dynamic LDS =
// 16 * H * 2 bytes of staged rows + one kTransBytes slice per wave.
template <int BITS, bool HAS_ZP>
__global__ __launch_bounds__(kSmallThreads) void small_fc1_kernel(
    const uint16_t* __restrict__ xa, const int8_t* __restrict__ xexp,
    const int32_t* __restrict__ sorted_routes, int k, const int4* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zps, int zp, int ushift,
    int64_t row_bytes, int64_t nblk, int H, int I, bool fc1_il, const void* __restrict__ bias,
    int act, int n_blocks, float* __restrict__ h32) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int active = num_tiles[0] * n_blocks;
  const int L = small_logical(active);
  if (L < 0) return;
  const int4 td = tiles[L / n_blocks];
  const int e = td.x, row0 = td.y, nrows = td.z, nb = L % n_blocks;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int ld = H;
  uint8_t* tb = reinterpret_cast<uint8_t*>(smem + kSmallRows * H) + wave * kTransBytes;

  // the wave's h columns: kFc1Groups groups of 16, each streaming its 16
  // gate rows (group 2c) and 16 up rows (group 2c + 1)
  constexpr int NG = 2 * kFc1Groups;
  using SL = StreamLanes<BITS>;
  const int64_t step = fc1_il ? 2 : 1;   // interleaved FC1: gate and up rows alternate
  const SL ln(lane, step * row_bytes, step * nblk);
  const int64_t ebase = static_cast<int64_t>(e) * 2 * I;
  const int nunits = H / 32;
  const int col_w = nb * kFc1Cols + __builtin_amdgcn_readfirstlane(wave) * 16 * kFc1Groups;
  RowGroup grp[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int c0 = col_w + 16 * (g >> 1), up = g & 1;
    const int cc = c0 < I ? c0 : 0;
    const int64_t row = ebase + (fc1_il ? 2 * cc + up : (up ? I + cc : cc));
    grp[g] = RowGroup{codes + row * row_bytes, scales + row * nblk, HAS_ZP ? zps + row * nblk : nullptr};
  }
  const int nbk = (nunits + SL::UB - 1) / SL::UB;
  constexpr int D = kFc1Depth;
  RowBlock<BITS> blk[NG][D];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int g = 0; g < NG; ++g)
      load_block<BITS, HAS_ZP>(ln, grp[g], d < nbk ? d : nbk - 1, nunits, ushift, zp, blk[g][d]);

  // stage the tile's activation rows while the first blocks' loads are in
  // flight
  const int upr = H / 8;   // 16-byte pieces per row
  for (int i = threadIdx.x; i < nrows * upr; i += kSmallThreads) {
    const int r = i / upr, c = i % upr;
    const int64_t tok = sorted_routes[row0 + r] / k;
    *reinterpret_cast<uint4*>(smem + r * ld + swz(r, c)) =
        *reinterpret_cast<const uint4*>(xa + tok * H + 8 * c);
  }
  __syncthreads();

  sf32x4_t acc[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = sf32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint16_t* arow = smem + l16 * ld;
  int bk = 0;
  for (; bk + D <= nbk; bk += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int bb = bk + d;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        // (a group past I computes on clamped rows; its results are not stored)
        stash_block<BITS>(blk[g][d], tb, lane);
        uint32_t sc[SL::SB];
        int zc[SL::SB];
#pragma unroll
        for (int sb = 0; sb < SL::SB; ++sb) {
          sc[sb] = blk[g][d].s[sb];
          zc[sb] = blk[g][d].z[sb];
        }
        // the next load goes out as soon as the block is in LDS; the loads
        // are unconditional, so the compiler's waits count them exactly
        // (past the last block they read the last block again, still in L2)
        load_block<BITS, HAS_ZP>(ln, grp[g], bb + D < nbk ? bb + D : nbk - 1, nunits, ushift, zp, blk[g][d]);
#pragma unroll
        for (int sb = 0; sb < SL::SB; ++sb) {
          // K is a multiple of 128, so a sub-block lies wholly inside or
          // wholly past it; one past it has no staged A columns to read
          if (bb * SL::UB + 4 * sb >= nunits) break;
          uint32_t p[16];
          dequant_unit_f16<BITS>(fetch_unit<BITS>(ln, tb, sb), sc[sb], zc[sb], p);
          acc[g] = mfma_unit(arow, l16, 32 * (bb * SL::UB + 4 * sb + q), p, acc[g]);
        }
      }
    }
  }
  // the last nbk % D blocks (already loaded)
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (bk + d >= nbk) break;
    const int bb = bk + d;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        stash_block<BITS>(blk[g][d], tb, lane);
#pragma unroll
        for (int sb = 0; sb < SL::SB; ++sb) {
          if (bb * SL::UB + 4 * sb >= nunits) break;
          uint32_t p[16];
          dequant_unit_f16<BITS>(fetch_unit<BITS>(ln, tb, sb), blk[g][d].s[sb], blk[g][d].z[sb], p);
          acc[g] = mfma_unit(arow, l16, 32 * (bb * SL::UB + 4 * sb + q), p, acc[g]);
        }
      }
  }

  // epilogue: lane holds rows 4q + i, column n of each group pair
#pragma unroll
  for (int c = 0; c < kFc1Groups; ++c) {
    const int n = col_w + 16 * c + l16;
    if (n >= I) continue;
    const float bg = bias_at(bias, act, ebase + (fc1_il ? 2 * n : n));
    const float bu = bias_at(bias, act, ebase + (fc1_il ? 2 * n + 1 : I + n));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * q + i;
      if (r < nrows) {
        const int ex = xexp != nullptr ? xexp[sorted_routes[row0 + r] / k] : 0;
        const float gv = ldexpf(acc[2 * c][i], ex) + bg, uv = ldexpf(acc[2 * c + 1][i], ex) + bu;
        h32[static_cast<int64_t>(row0 + r) * I + n] = silu_mul(gv, uv);
      }
    }
  }
}

// FC2 over one tile and kFc2Cols output columns. grid as FC1, block = 512,
// dynamic LDS = 16 * I * 2 + 8 * kTransBytes bytes.
template <int BITS, bool HAS_ZP>
__global__ __launch_bounds__(kSmallThreads) void small_fc2_kernel(
    const float* __restrict__ h32, const int4* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zps, int zp, int ushift,
    int64_t row_bytes, int64_t nblk, int H, int I, const void* __restrict__ bias, int act,
    int n_blocks, float* __restrict__ y32) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ int s_exp[kSmallRows];
  const int active = num_tiles[0] * n_blocks;
  const int L = small_logical(active);
  if (L < 0) return;
  const int4 td = tiles[L / n_blocks];
  const int e = td.x, row0 = td.y, nrows = td.z, nb = L % n_blocks;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int ld = I;
  uint8_t* tb = reinterpret_cast<uint8_t*>(smem + kSmallRows * I) + wave * kTransBytes;

  // the wave's output rows: kFc2Groups groups of 16
  using SL = StreamLanes<BITS>;
  const SL ln(lane, row_bytes, nblk);
  const int nunits = I / 32;
  const int64_t ebase = static_cast<int64_t>(e) * H;
  const int row_w = nb * kFc2Cols + __builtin_amdgcn_readfirstlane(wave) * 16 * kFc2Groups;
  RowGroup grp[kFc2Groups];
#pragma unroll
  for (int g = 0; g < kFc2Groups; ++g) {
    const int m0 = row_w + 16 * g;
    const int64_t row = ebase + (m0 < H ? m0 : 0);
    grp[g] = RowGroup{codes + row * row_bytes, scales + row * nblk, HAS_ZP ? zps + row * nblk : nullptr};
  }
  const int nbk = (nunits + SL::UB - 1) / SL::UB;
  constexpr int D = kFc2Depth;
  RowBlock<BITS> blk[kFc2Groups][D];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int g = 0; g < kFc2Groups; ++g)
      load_block<BITS, HAS_ZP>(ln, grp[g], d < nbk ? d : nbk - 1, nunits, ushift, zp, blk[g][d]);

  // stage h rows as fp16 with the row's range exponent (while the first
  // blocks' loads are in flight); wave w takes rows
  // w and w + 8 (rows past the tile are left unset: no stored output reads
  // them, since row m of a product depends on row m of A only)
  for (int r = wave; r < nrows; r += kSmallWaves) {
    const float* hr = h32 + static_cast<int64_t>(row0 + r) * I;
    float m = 0.0f;
    bool finite = true;
    for (int c = lane; c < I; c += kWave) {
      const float v = hr[c];
      finite = finite && fabsf(v) <= 3.4028235e38f;
      m = fmaxf(m, fabsf(v));
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    const int ex = __all(finite) ? range_exponent(m) : 0;
    // 16 values per lane, placed in operand order
    constexpr int P = operand_perm(BITS);
    for (int c = 16 * lane; c < I; c += 16 * kWave) {
      float v[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 f = *reinterpret_cast<const float4*>(hr + c + 4 * q4);
        v[4 * q4] = f.x; v[4 * q4 + 1] = f.y; v[4 * q4 + 2] = f.z; v[4 * q4 + 3] = f.w;
      }
      uint32_t o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16x2_t hv = {static_cast<_Float16>(ldexpf(v[operand_k(P, 2 * j)], -ex)),
                            static_cast<_Float16>(ldexpf(v[operand_k(P, 2 * j + 1)], -ex))};
        o[j] = __builtin_bit_cast(uint32_t, hv);
      }
      *reinterpret_cast<uint4*>(smem + r * ld + swz(r, c >> 3)) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(smem + r * ld + swz(r, (c >> 3) + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
    if (lane == 0) s_exp[r] = ex;
  }

  __syncthreads();

  sf32x4_t acc[kFc2Groups];
#pragma unroll
  for (int g = 0; g < kFc2Groups; ++g) acc[g] = sf32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint16_t* arow = smem + l16 * ld;
  int bk = 0;
  for (; bk + D <= nbk; bk += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int bb = bk + d;
#pragma unroll
      for (int g = 0; g < kFc2Groups; ++g) {
        // (a group past H computes on clamped rows; its results are not stored)
        stash_block<BITS>(blk[g][d], tb, lane);
        uint32_t sc[SL::SB];
        int zc[SL::SB];
#pragma unroll
        for (int sb = 0; sb < SL::SB; ++sb) {
          sc[sb] = blk[g][d].s[sb];
          zc[sb] = blk[g][d].z[sb];
        }
        load_block<BITS, HAS_ZP>(ln, grp[g], bb + D < nbk ? bb + D : nbk - 1, nunits, ushift, zp, blk[g][d]);
#pragma unroll
        for (int sb = 0; sb < SL::SB; ++sb) {
          if (bb * SL::UB + 4 * sb >= nunits) break;   // past K (K % 128 == 0)
          uint32_t p[16];
          dequant_unit_f16<BITS>(fetch_unit<BITS>(ln, tb, sb), sc[sb], zc[sb], p);
          acc[g] = mfma_unit(arow, l16, 32 * (bb * SL::UB + 4 * sb + q), p, acc[g]);
        }
      }
    }
  }
  // the last nbk % D blocks (already loaded)
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (bk + d >= nbk) break;
    const int bb = bk + d;
#pragma unroll
      for (int g = 0; g < kFc2Groups; ++g) {
        stash_block<BITS>(blk[g][d], tb, lane);
#pragma unroll
        for (int sb = 0; sb < SL::SB; ++sb) {
          if (bb * SL::UB + 4 * sb >= nunits) break;
          uint32_t p[16];
          dequant_unit_f16<BITS>(fetch_unit<BITS>(ln, tb, sb), blk[g][d].s[sb], blk[g][d].z[sb], p);
          acc[g] = mfma_unit(arow, l16, 32 * (bb * SL::UB + 4 * sb + q), p, acc[g]);
        }
      }
  }

#pragma unroll
  for (int g = 0; g < kFc2Groups; ++g) {
    const int m = row_w + 16 * g + l16;
    if (m >= H) continue;
    const float b = bias_at(bias, act, ebase + m);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * q + i;
      if (r < nrows)
        __builtin_nontemporal_store(ldexpf(acc[g][i], s_exp[r]) + b,
                                    &y32[static_cast<int64_t>(row0 + r) * H + m]);
    }
  }
}

namespace {

template <int BITS>
hipError_t launch_small_gemms(const Layer& L, const uint16_t* xa, const int8_t* xexp, char* ws,
                              const Workspace& W, hipStream_t s) {
  const int H = static_cast<int>(L.H), I = static_cast<int>(L.I);
  const int32_t* sorted = reinterpret_cast<const int32_t*>(ws + W.sorted_routes);
  const int4* tiles = reinterpret_cast<const int4*>(ws + W.tiles);
  const int32_t* ntiles = reinterpret_cast<const int32_t*>(ws + W.num_tiles);
  float* h32 = reinterpret_cast<float*>(ws + W.h32);
  float* y32 = reinterpret_cast<float*>(ws + W.yf32);
  const int ushift = L.bs == 32 ? 0 : L.bs == 64 ? 1 : 2;
  const int nb1 = (I + kFc1Cols - 1) / kFc1Cols, nb2 = (H + kFc2Cols - 1) / kFc2Cols;
  const int64_t g1 = 8 * ((W.max_tiles * nb1 + 7) / 8), g2 = 8 * ((W.max_tiles * nb2 + 7) / 8);
  const size_t lds1 = static_cast<size_t>(kSmallRows) * H * 2 + kSmallWaves * kTransBytes;
  const size_t lds2 = static_cast<size_t>(kSmallRows) * I * 2 + kSmallWaves * kTransBytes;
  auto fc1 = L.fc1_zp ? small_fc1_kernel<BITS, true> : small_fc1_kernel<BITS, false>;
  auto fc2 = L.fc2_zp ? small_fc2_kernel<BITS, true> : small_fc2_kernel<BITS, false>;
  fc1<<<static_cast<unsigned>(g1), kSmallThreads, lds1, s>>>(
      xa, xexp, sorted, L.k, tiles, ntiles, L.fc1_codes, L.fc1_scales, L.fc1_zp, L.zp, ushift,
      L.fc1_row_bytes, L.fc1_nblk, H, I, L.fc1_interleaved, L.fc1_bias, L.act, nb1, h32);
  stage_done(L, 6, "small_fc1_swiglu");
  fc2<<<static_cast<unsigned>(g2), kSmallThreads, lds2, s>>>(
      h32, tiles, ntiles, L.fc2_codes, L.fc2_scales, L.fc2_zp, L.zp, ushift, L.fc2_row_bytes,
      L.fc2_nblk, H, I, L.fc2_bias, L.act, nb2, y32);
  stage_done(L, 7, "small_fc2");
  return hipGetLastError();
}

}  // namespace

bool small_path_supported(const Layer& L) {
  // K values in whole 128-wide sub-blocks, and a tile's staged rows (16 x K
  // fp16, at most 128 KB) plus the waves' 16 KB of slices within the 160 KB
  // of LDS
  return L.H % 128 == 0 && L.I % 128 == 0 && L.H <= 4096 && L.I <= 4096;
}

// Allow each instance the dynamic LDS its largest layer needs (beyond the
// 64 KB default of a launch).
hipError_t prepare_small(const Layer& L) {
  const int b1 = static_cast<int>(kSmallRows * L.H * 2 + kSmallWaves * kTransBytes);
  const int b2 = static_cast<int>(kSmallRows * L.I * 2 + kSmallWaves * kTransBytes);
  const void* f1[] = {reinterpret_cast<const void*>(&small_fc1_kernel<4, false>),
                      reinterpret_cast<const void*>(&small_fc1_kernel<4, true>),
                      reinterpret_cast<const void*>(&small_fc1_kernel<3, false>),
                      reinterpret_cast<const void*>(&small_fc1_kernel<3, true>),
                      reinterpret_cast<const void*>(&small_fc1_kernel<2, false>),
                      reinterpret_cast<const void*>(&small_fc1_kernel<2, true>)};
  const void* f2[] = {reinterpret_cast<const void*>(&small_fc2_kernel<4, false>),
                      reinterpret_cast<const void*>(&small_fc2_kernel<4, true>),
                      reinterpret_cast<const void*>(&small_fc2_kernel<3, false>),
                      reinterpret_cast<const void*>(&small_fc2_kernel<3, true>),
                      reinterpret_cast<const void*>(&small_fc2_kernel<2, false>),
                      reinterpret_cast<const void*>(&small_fc2_kernel<2, true>)};
  for (const void* f : f1) {
    const hipError_t err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, b1);
    if (err != hipSuccess) return err;
  }
  for (const void* f : f2) {
    const hipError_t err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, b2);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_small(const Layer& L, const void* x, const void* logits, void* out, int64_t T,
                        char* ws, const Workspace& W, hipStream_t s) {
  const uint16_t* xa = nullptr;
  const int8_t* xexp = nullptr;
  hipError_t err;
  if (route_small_fits(L, T)) {
    err = launch_route_small(L, logits, x, T, ws, W, s, &xa, &xexp);
  } else {
    err = launch_route(L, logits, T, ws, W, s);
    if (err == hipSuccess) err = launch_stage_x(L, x, T, ws, W, s, &xa, &xexp);
  }
  if (err != hipSuccess) return err;
  switch (L.bits) {
    case 4: err = launch_small_gemms<4>(L, xa, xexp, ws, W, s); break;
    case 3: err = launch_small_gemms<3>(L, xa, xexp, ws, W, s); break;
    default: err = launch_small_gemms<2>(L, xa, xexp, ws, W, s); break;
  }
  if (err != hipSuccess) return err;
  return launch_combine(L, out, T, ws, W, s);
}

}  // namespace qmoe
