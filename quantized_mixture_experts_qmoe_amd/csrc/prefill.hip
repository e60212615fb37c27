// Prefill path (5+ tokens): expert-grouped GEMMs on the CDNA4 matrix cores
// with fp16 operands.
//
// The routing stage leaves the routes sorted by expert and a tile list
// (expert, first sorted row, rows <= 256). Each workgroup (8 waves, 4 x 2 of
// 64 x 128) computes one 256 x 256 tile of one expert:
//   FC1: A = x rows gathered through sorted_routes (fp16, each token scaled
//        by its power of two), B = the expert's gate rows [n0, n0+128) and up
//        rows [I+n0, I+n0+128), dequantized to fp16((q - zp) * s) into LDS;
//        each wave holds 64 gate and the 64 matching up columns, so the
//        epilogue applies h = silu(gate) * up and stores h as fp16 [R, I] in
//        sorted order (with per-chunk exponents, see below).
//   FC2: A = h rows of the tile (fp16), B = the expert's FC2 rows
//        [n0, n0+256) dequantized into LDS; the epilogue stores fp32 y
//        [R, H] in sorted order (non-temporal: the combine reads it once).
// Both epilogues stage each wave's results in LDS, 16 rows at a time, and
// write whole 16-byte row segments.
// The tall tile shares each dequantized weight among 256 rows; a wave whose
// 64 rows all lie past the expert's last route skips its matrix work, and a
// wave whose 32 rows of the A share all lie past it neither loads nor stores
// them. A tile
// of at most 128 rows runs in half mode: both wave groups compute rows
// 0-127, each for half of the columns.
// The K loop runs in stages of 64 with two LDS buffers, ping-pong style: the
// waves form two groups of four (rows 0-127 and 128-255 of the tile) that
// run half a stage apart. In each phase between two barriers one group runs
// the MFMAs of stage s while the other dequantizes and stores its share of
// stage s+1 (its own A rows and half of B) and issues its global loads for
// stage s+2; each SIMD holds one wave of each group, so its matrix and vector
// work overlap. The MFMA wave raises its issue priority for its phase.
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
#include <utility>

#include "device.h"
#include "internal.h"

namespace qmoe {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

namespace {

constexpr int kKT = 64;                 // K per stage (two 16x16x32 MFMA steps)
constexpr int kLdsStride = kKT + 16;    // bf16 per LDS row (padding against bank conflicts)
constexpr int kBM = kTileM;             // A rows per tile (256)
constexpr int kBN = 256;                // B rows per tile
constexpr int kGemmThreads = 512;       // 8 waves: 2 groups of 2 x 2 waves of 64 x 128
static_assert(kBM == 256, "the staging below assumes 256-row tiles");
static_assert(2 * (kBM + kBN) * kLdsStride * 2 <= 160 * 1024, "LDS of one workgroup");
// epilogue staging: per wave, 16 output rows of its 64 x 128 block at a time,
// in a private slice of the A buffers (fp32 y: 128 + 4 columns; bf16 h: 64 + 8)
constexpr int kStgY = 16 * (128 + 4);
constexpr int kStgH = 16 * (64 + 8);
static_assert(8 * kStgY * 4 <= 2 * kBM * kLdsStride * 2, "epilogue staging fits in the A buffers");

// Logical tile index of this workgroup. Workgroups are dealt to the 8 XCDs
// round-robin; consecutive logical tiles are kept on one XCD so the n-tiles
// of one m-tile (which share their A rows) and the m-tiles of one expert
// (which share B) meet in the same L2.
__device__ __forceinline__ int logical_tile(int active) {
  const int b = blockIdx.x;
  const int per_xcd = (active + 7) / 8;
  const int j = b / 8;
  if (j >= per_xcd) return -1;
  const int L = (b % 8) * per_xcd + j;
  return L < active ? L : -1;
}

// v of lane (l + N) mod 16 within this lane's row of 16 (DPP row_ror).
template <int N>
__device__ __forceinline__ float row_rotate(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}

// Calls f(std::integral_constant<int, J>) for J = 0..N-1, so that each step's
// counts are compile-time constants (the scheduling hints below need them).
template <typename F, int... J>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

int gemm_n_tiles(const Layer& L, bool fc1) {
  return fc1 ? static_cast<int>((L.I + kBN / 2 - 1) / (kBN / 2))
             : static_cast<int>((L.H + kBN - 1) / kBN);
}

}  // namespace

// grid = 8 * ceil(max_tiles * n_tiles_n / 8), block = 512
// (one workgroup per CU: its LDS use limits each SIMD to two waves, so the
// compiler may use the whole register file to keep fragments in flight)
//
// Operand ranges: FC1's A rows are a token's activations scaled by 2^-e_t
// (a per-token exponent from the staging pass, or none for fp16 inputs),
// undone on the accumulators in the epilogue. FC1 stores h as fp16 in chunks
// of 32 columns with an exponent per (route, chunk), nonzero only for chunks
// whose largest magnitude lies outside [2^-14, 2^15]; a pass between the two
// GEMMs brings each route's chunks to the route's largest exponent E, and
// FC2 scales its accumulators by 2^E. A row's exponent sits in the unused
// padding of its row in the first B buffer from the prologue to the
// epilogue.
template <int BITS, bool FC1, bool HAS_ZP>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_kernel(
    const uint16_t* __restrict__ a_src, const int32_t* __restrict__ sorted_routes, int k,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int K, int H, int I,
    int bs_shift, int zp, const uint8_t* __restrict__ zps, bool fc1_il,
    const void* __restrict__ bias, int act,
    int64_t row_bytes, int64_t nblk, const int4* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int n_tiles_n, uint16_t* __restrict__ h_out,
    float* __restrict__ y_out, const int8_t* __restrict__ a_exp, int8_t* __restrict__ h_exp) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLdsStride];

  const int active = num_tiles[0] * n_tiles_n;
  const int L = logical_tile(active);
  if (L < 0) return;
  const int m_tile = L / n_tiles_n, n_tile = L % n_tiles_n;
  const int4 td = tiles[m_tile];
  const int e = td.x, row0 = td.y, nrows = td.z;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // two groups of four waves, half a stage apart: group g owns rows
  // [128 g, 128 g + 128) of the tile; in each phase one group runs its MFMAs
  // while the other stores its share of the next stage
  const int grp = wave >> 2, gw = wave & 3, gt = tid & 255;
  // A tile of at most 128 rows runs in half mode: both groups compute rows
  // 0-127 (stored by group 0), each for half of the tile's columns, so the
  // matrix cores stay busy in both phases; each wave then holds 64 x 64.
  const bool half = nrows <= kBM / 2;
  const int wm = half ? (gw >> 1) : 2 * grp + (gw >> 1), wn = gw & 1;
  const int cg = half ? grp : 0;   // column half of this group in half mode
  const bool wave_live = wm * 64 < nrows;
  const int n_rows_total = FC1 ? 2 * I : H;
  const uint8_t* ebase = codes + static_cast<int64_t>(e) * n_rows_total * row_bytes;
  const uint16_t* sbase = scales + static_cast<int64_t>(e) * n_rows_total * nblk;
  const int n0 = n_tile * (FC1 ? kBN / 2 : kBN);

  // this thread's B share: unit 256 grp + gt of the stage's 512 (row u >> 1,
  // K offset 32 * (u & 1))
  const int b_unit = 256 * grp + gt, b_row = b_unit >> 1, b_kq = b_unit & 1;
  int w_row;
  if (FC1) {
    const int c = n0 + (b_row & (kBN / 2 - 1));
    const int up = b_row >= kBN / 2;   // gate rows of the tile first, then the matching up rows
    w_row = c < I ? (fc1_il ? 2 * c + up : (up ? I + c : c)) : 0;
  } else {
    const int c = n0 + b_row;
    w_row = c < H ? c : 0;
  }
  const uint8_t* b_ptr = ebase + static_cast<int64_t>(w_row) * row_bytes;
  const uint16_t* s_ptr = sbase + static_cast<int64_t>(w_row) * nblk;
  // per-block zero points of this thread's B row (when the layer has them)
  const uint8_t* z_ptr =
      HAS_ZP ? zps + (static_cast<int64_t>(e) * n_rows_total + w_row) * nblk : nullptr;

  // this thread's A share: the 16-byte chunk (lane & 7) of rows
  // 128 grp + 32 gw + 8 q + (lane >> 3), q = 0..3, so each load instruction
  // reads whole 128-byte row segments (eight rows per instruction)
  const int64_t a_ld = FC1 ? H : I;
  const int a_chunk = (lane & 7) * 8;
  const int a_row0 = 128 * grp + 32 * gw + (lane >> 3);
  const uint16_t* a_ptr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = a_row0 + 8 * q;
    const int rr = r < nrows ? r : 0;
    const int64_t src_row = FC1 ? (sorted_routes[row0 + rr] / k) : (row0 + rr);
    a_ptr[q] = a_src + src_row * a_ld + a_chunk;
  }

  // a wave whose 32 A rows all lie past the tile's routes neither loads nor
  // stores them: no stored output row reads them (row m of a product depends
  // on row m of A only)
  const bool a_live = 128 * grp + 32 * gw < nrows;
  // this thread's rows' exponents (FC1: the token's activation exponent;
  // FC2: the route's h exponent), issued now and stored to LDS after the
  // first stage's loads are on their way
  int row_e[4] = {0, 0, 0, 0};
  if (a_exp != nullptr && a_live) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = a_row0 + 8 * q;
      const int rr = r < nrows ? r : 0;
      row_e[q] = FC1 ? a_exp[sorted_routes[row0 + rr] / k] : a_exp[row0 + rr];
    }
  }
  auto store_row_exponents = [&]() {
    if ((lane & 7) == 0 && a_live) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        Bs[0][(a_row0 + 8 * q) * kLdsStride + kKT] = static_cast<uint16_t>(static_cast<int16_t>(row_e[q]));
    }
  };
  const int hstride = h_exp_stride(I);

  uint4 ra0, ra1, ra2, ra3;
  UnitWords<BITS> rb;
  uint16_t rs;      // raw fp16 scale of this stage's B unit
  bool rpast;       // the unit lies past K (its scale is taken as zero)
  int rz = zp;   // this stage's zero point (the scalar one without a tensor)
  auto load_stage = [&](int st) {
    const int k0 = st * kKT;
    // (a chunk past K reads its row's first columns instead: always inside
    // the row; the zero scales of the B units past K cancel it)
    const int ka = (k0 + a_chunk < K) ? k0 : -a_chunk;
    if (a_live) {
      ra0 = *reinterpret_cast<const uint4*>(a_ptr[0] + ka);
      ra1 = *reinterpret_cast<const uint4*>(a_ptr[1] + ka);
      ra2 = *reinterpret_cast<const uint4*>(a_ptr[2] + ka);
      ra3 = *reinterpret_cast<const uint4*>(a_ptr[3] + ka);
    }
    const int kk = k0 + 32 * b_kq;
    const int kb = (kk < K) ? kk : 0;
    rb = load_unit<BITS>(b_ptr + (kb / 32) * (4 * BITS));
    // (the flag is kept apart from the loaded value, so nothing waits for
    // the load before the store phase that consumes it)
    rs = s_ptr[kb >> bs_shift];
    rpast = kk >= K;
    if constexpr (HAS_ZP) rz = z_ptr[kb >> bs_shift];
  };
  auto store_stage = [&](int buf) {
    if (a_live) {
      uint16_t* ad = &As[buf][a_row0 * kLdsStride + a_chunk];
      *reinterpret_cast<uint4*>(ad) = ra0;
      *reinterpret_cast<uint4*>(ad + 8 * kLdsStride) = ra1;
      *reinterpret_cast<uint4*>(ad + 16 * kLdsStride) = ra2;
      *reinterpret_cast<uint4*>(ad + 24 * kLdsStride) = ra3;
    }
    // the fp16 operand fp16((q - zp) * s) (a unit past K gets a zero scale)
    uint32_t pairs[16];
    dequant_unit_f16<BITS>(rb, rpast ? 0u : static_cast<uint32_t>(rs), rz, pairs);
    uint4* bd = reinterpret_cast<uint4*>(&Bs[buf][b_row * kLdsStride + 32 * b_kq]);
#pragma unroll
    for (int q = 0; q < 4; ++q) bd[q] = make_uint4(pairs[4 * q], pairs[4 * q + 1], pairs[4 * q + 2], pairs[4 * q + 3]);
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int quad = lane >> 4, l16 = lane & 15;
  // B rows (output columns) of fragment tn: FC1 pairs gate fragment tn with
  // up fragment tn + NT/2 (NT = 8 fragments per wave, 4 in half mode)
  int b_frag_row[8];
#pragma unroll
  for (int tn = 0; tn < 8; ++tn) {
    if (half)
      b_frag_row[tn] = FC1 ? ((tn & 2) ? kBN / 2 : 0) + cg * 64 + wn * 32 + (tn & 1) * 16 + l16
                           : cg * 128 + wn * 64 + (tn & 3) * 16 + l16;
    else
      b_frag_row[tn] = FC1 ? (tn < 4 ? 0 : kBN / 2) + wn * 64 + (tn & 3) * 16 + l16
                           : wn * 128 + tn * 16 + l16;
  }
  auto frag_a = [&](int buf, int ks, int tm) {
    const int r = wm * 64 + tm * 16 + l16;
    return *reinterpret_cast<const f16x8_t*>(&As[buf][r * kLdsStride + ks * 32 + quad * 8]);
  };
  auto frag_b = [&](int buf, int ks, int tn) {
    return *reinterpret_cast<const f16x8_t*>(&Bs[buf][b_frag_row[tn] * kLdsStride + ks * 32 + quad * 8]);
  };
  // A stage is 2 K halves x NT B fragments (NT = 8, or 4 in half mode); each
  // step runs 4 MFMAs that share one B fragment. Fragment reads run ahead of
  // their use: B two steps ahead through a ring of three registers, the
  // second K half's A fragments during the first half's last four steps, so
  // the LDS latency hides behind the matrix work instead of stalling it.
  auto mfma_steps = [&](int buf, auto ntc) {
    constexpr int NT = decltype(ntc)::value, NS = 2 * NT;
    f16x8_t af[2][4], bfr[3];
#pragma unroll
    for (int t = 0; t < 4; ++t) af[0][t] = frag_a(buf, 0, t);
    bfr[0] = frag_b(buf, 0, 0);
    bfr[1] = frag_b(buf, 0, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    static_for<NS>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int ks = j / NT, tn = j % NT;
      constexpr bool rd_a = ks == 0 && tn >= NT - 4;
      constexpr int nreads = (j + 2 < NS ? 1 : 0) + (rd_a ? 1 : 0);
      if constexpr (j + 2 < NS) bfr[(j + 2) % 3] = frag_b(buf, (j + 2) / NT, (j + 2) % NT);
      if constexpr (rd_a) af[1][tn - (NT - 4)] = frag_a(buf, 1, tn - (NT - 4));
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[ks][tm], bfr[j % 3], acc[tm][tn], 0, 0, 0);
      // keep the issue order: this step's reads, then its four MFMAs
      if constexpr (nreads > 0) __builtin_amdgcn_sched_group_barrier(0x100, nreads, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    });
  };
  const int ns = (K + kKT - 1) / kKT;
  auto clampst = [&](int st) { return st < ns ? st : ns - 1; };
  // prologue: stage 0 complete in buffer 0; registers hold stage 1
  load_stage(0);
  store_stage(0);
  load_stage(clampst(1));
  store_row_exponents();
  __syncthreads();
  // The K loop, instantiated once per fragment count (the mode is uniform
  // over the tile, so each instance keeps its own register allocation); one
  // loop per group (same barrier sequence), so each keeps only its own live
  // registers.
  auto kloop = [&](auto ntc) {
    // (the MFMA wave of each SIMD runs at a raised issue priority, so its
    // matrix instructions go first and the other group's dequantization
    // fills the remaining issue slots)
    auto mfma_stage = [&](int buf) {
      if (wave_live) {
        __builtin_amdgcn_s_setprio(1);
        mfma_steps(buf, ntc);
        __builtin_amdgcn_s_setprio(0);
      }
    };
    if (grp == 0) {
      for (int st = 0; st < ns; ++st) {
        const int buf = st & 1;
        mfma_stage(buf);             // phase X
        __syncthreads();
        store_stage(buf ^ 1);        // phase Y
        load_stage(clampst(st + 2));
        __syncthreads();
      }
    } else {
      for (int st = 0; st < ns; ++st) {
        const int buf = st & 1;
        store_stage(buf ^ 1);        // phase X
        load_stage(clampst(st + 2));
        __syncthreads();
        mfma_stage(buf);             // phase Y
        __syncthreads();
      }
    }
  };
  if (half)
    kloop(std::integral_constant<int, 4>{});
  else
    kloop(std::integral_constant<int, 8>{});
  if (!wave_live) return;

  // ---- epilogue: lane holds rows 4*quad + i, column l16 of each 16x16
  // fragment. Results go out through a private LDS slice of this wave, 16
  // rows at a time, so that each row segment is written with whole 16-byte
  // stores (the loop's last barrier has retired every LDS access of the K
  // loop). The optional bias is per column (FC1: the gate and up rows').
  float* stg_y = reinterpret_cast<float*>(&As[0][0]) + wave * kStgY;
  uint16_t* stg_h = &As[0][0] + wave * kStgH;
  auto epilogue = [&](auto ntc) {
    constexpr int NT = decltype(ntc)::value, NH = NT / 2;
    // first output column of this wave (FC1: h columns, NH * 16 of them;
    // FC2: y columns, NT * 16 of them)
    const int cb = FC1 ? n0 + (half ? cg * 64 + wn * 32 : wn * 64)
                       : n0 + (half ? cg * 128 + wn * 64 : wn * 128);
    float bcol[NT];
#pragma unroll
    for (int tn = 0; tn < NT; ++tn) {
      if (FC1) {
        const int c = cb + (tn % NH) * 16 + l16, up = tn >= NH;
        const int64_t r = fc1_il ? 2 * c + up : (up ? I + c : c);
        bcol[tn] = c < I ? bias_at(bias, act, static_cast<int64_t>(e) * 2 * I + r) : 0.0f;
      } else {
        const int c = cb + tn * 16 + l16;
        bcol[tn] = c < H ? bias_at(bias, act, static_cast<int64_t>(e) * H + c) : 0.0f;
      }
    }
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
      const int prow = wm * 64 + tm * 16;   // first tile row of this block
      // this lane's rows' exponents (prologue, padding of the first B buffer)
      int re[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        re[i] = static_cast<int16_t>(Bs[0][(prow + quad * 4 + i) * kLdsStride + kKT]);
      // the row exponents, then the bias, in place; both branches are
      // wave-uniform, so the common case (no exponent, no bias) skips them
      if (__ballot((re[0] | re[1] | re[2] | re[3]) != 0) != 0) {
#pragma unroll
        for (int tn = 0; tn < NT; ++tn)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tm][tn][i] = ldexpf(acc[tm][tn][i], re[i]);
      }
      if (bias != nullptr) {
#pragma unroll
        for (int tn = 0; tn < NT; ++tn)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tm][tn][i] += bcol[tn];
      }
      if (FC1) {
        // h of this lane's 4 rows x NH columns, then per (row, 32-column
        // chunk of fragments 2c, 2c+1) the exponent that keeps the chunk in
        // fp16 range (0 unless its largest magnitude lies outside
        // [2^-10, 2^15]); the 16 lanes of a DPP row hold one row's columns
        float hv[4][NH];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int tn = 0; tn < NH; ++tn) hv[i][tn] = silu_mul_fast(acc[tm][tn][i], acc[tm][tn + NH][i]);
        constexpr int NC = NH / 2;
        int ce[4][NC];
        // a chunk needs an exponent only if its maximum leaves [2^-14, 2^15]:
        // a lane whose own values of the chunk are all inside that range (or
        // hold one at least 2^-14 and none above 2^15) settles it for its
        // row, so the chunk maxima are formed only in the rare waves where
        // some lane cannot tell
        float lm[4][NC];
        bool unsure = false;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            lm[i][c] = fmaxf(fabsf(hv[i][2 * c]), fabsf(hv[i][2 * c + 1]));
            unsure = unsure || !(lm[i][c] >= 0x1p-14f && lm[i][c] <= 32768.0f);
            ce[i][c] = 0;
          }
        if (__ballot(unsure) != 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              float m = lm[i][c];
              m = fmaxf(m, row_rotate<8>(m));
              m = fmaxf(m, row_rotate<4>(m));
              m = fmaxf(m, row_rotate<2>(m));
              m = fmaxf(m, row_rotate<1>(m));
              ce[i][c] = h_chunk_exponent(m);
            }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int tn = 0; tn < NH; ++tn) hv[i][tn] = ldexpf(hv[i][tn], -ce[i][tn / 2]);
        }
        // h goes out in operand order, the order FC2's A rows need
        const int hpos = operand_pos(operand_perm(BITS), l16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int tn = 0; tn < NH; ++tn)
            stg_h[(quad * 4 + i) * 72 + tn * 16 + hpos] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(hv[i][tn]));
        if (l16 == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p = prow + quad * 4 + i;
            if (p < nrows)
#pragma unroll
              for (int c = 0; c < NC; ++c)
                if (cb + 32 * c < I)
                  h_exp[static_cast<int64_t>(row0 + p) * hstride + (cb >> 5) + c] = static_cast<int8_t>(ce[i][c]);
          }
        }
        // 16 rows x NH*16 columns: NT 16-byte chunks per row
#pragma unroll
        for (int j = 0; j < NT / 4; ++j) {
          const int idx = lane + 64 * j, row = idx / NT, c8 = idx % NT;
          const int p = prow + row, c = cb + c8 * 8;
          const uint4 v = *reinterpret_cast<const uint4*>(&stg_h[row * 72 + c8 * 8]);
          if (p < nrows && c < I) *reinterpret_cast<uint4*>(&h_out[static_cast<int64_t>(row0 + p) * I + c]) = v;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int tn = 0; tn < NT; ++tn)
            stg_y[(quad * 4 + i) * 132 + tn * 16 + l16] = acc[tm][tn][i];
        // 16 rows x NT*16 columns: NT*4 float4 per row
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int idx = lane + 64 * j, row = idx / (NT * 4), c4 = idx % (NT * 4);
          const int p = prow + row, c = cb + c4 * 4;
          const float4 v = *reinterpret_cast<const float4*>(&stg_y[row * 132 + c4 * 4]);
          // y is written once and read once, by the combine: non-temporal stores
        if (p < nrows && c < H)
          __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w},
                                      reinterpret_cast<f32x4_t*>(&y_out[static_cast<int64_t>(row0 + p) * H + c]));
        }
      }
    }
  };
  if (half)
    epilogue(std::integral_constant<int, 4>{});
  else
    epilogue(std::integral_constant<int, 8>{});
}

// out[t][m] = round(sum_j w[t][j] * y[inv_pos[t*k + j]][m]), slot order j = 0..k-1.
// grid = (ceil(H / 1024), T), block = 256, 4 columns per thread.
template <int ACT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ topk_w, int k,
                                                      int H, void* __restrict__ out) {
  const int64_t t = blockIdx.y;
  const int m = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (m >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // (each y value is read exactly once: non-temporal loads, 27% faster than
  // cached ones at 8K tokens)
  auto add = [&](float w, const f32x4_t& v) {
    acc.x = fmaf(w, v[0], acc.x);
    acc.y = fmaf(w, v[1], acc.y);
    acc.z = fmaf(w, v[2], acc.z);
    acc.w = fmaf(w, v[3], acc.w);
  };
  // slots in groups of eight: a group's loads all go out before its sums,
  // which still run in slot order
  int j = 0;
  for (; j + 8 <= k; j += 8) {
    int64_t p[8];
    float w[8];
    f32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      p[u] = inv_pos[t * k + j + u];
      w[u] = topk_w[t * k + j + u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(y + p[u] * H + m));
#pragma unroll
    for (int u = 0; u < 8; ++u) add(w[u], v[u]);
  }
  for (; j < k; ++j) {
    const int64_t p = inv_pos[t * k + j];
    add(topk_w[t * k + j], __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(y + p * H + m)));
  }
  if constexpr (ACT == kActBF16) {
    uint2 o;
    o.x = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
    o.y = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + t * H + m) = o;
  } else if constexpr (ACT == kActF16) {
    const int64_t o = t * H + m;
    store_act(out, kActF16, o, acc.x);
    store_act(out, kActF16, o + 1, acc.y);
    store_act(out, kActF16, o + 2, acc.z);
    store_act(out, kActF16, o + 3, acc.w);
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + t * H + m) = acc;
  }
}

// FC1's activations in operand order (stage_x_row), one wave per token.
template <int ACT, int P>
__global__ __launch_bounds__(256) void stage_x_f16_kernel(const void* __restrict__ x, int64_t T, int H,
                                                          uint16_t* __restrict__ x16,
                                                          int8_t* __restrict__ xexp) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  stage_x_row<ACT, P>(x, t, H, x16, xexp, threadIdx.x & (kWave - 1));
}

// Between the GEMMs: each route's h chunks brought to the route's largest
// chunk exponent E (a chunk stored at e < E is multiplied by 2^(e - E), one
// more fp16 rounding), and E written to rexp[route] for FC2. Chunks are
// rewritten only in the rare routes whose exponents differ. One thread per
// route: it reads the route's exponent row (h_exp_stride bytes, 16-byte
// aligned) 16 bytes at a time.
__global__ __launch_bounds__(256) void h_common_exponent_kernel(uint16_t* __restrict__ h16,
                                                               const int8_t* __restrict__ hexp,
                                                               int8_t* __restrict__ rexp, int64_t R,
                                                               int I) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (r >= R) return;
  const int nchk = I / 32, hs = h_exp_stride(I);
  const int8_t* er = hexp + r * hs;
  int emax = -128, emin = 127;
  for (int c0 = 0; c0 < nchk; c0 += 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(er + c0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      if (c0 + b < nchk) {
        const int e = static_cast<int8_t>(w[b >> 2] >> (8 * (b & 3)));
        emax = max(emax, e);
        emin = min(emin, e);
      }
    }
  }
  rexp[r] = static_cast<int8_t>(emax);
  if (emin == emax) return;
  // rare: rescale the chunks below E (8 fp16 values per step)
  for (int i = 0; i < I; i += 8) {
    const int d = er[i >> 5] - emax;
    if (d == 0) continue;
    const uint16_t fb = d >= -14 ? static_cast<uint16_t>((d + 15) << 10)
                        : d >= -24 ? static_cast<uint16_t>(1u << (d + 24)) : uint16_t{0};
    const _Float16 f = __builtin_bit_cast(_Float16, fb);
    const f16x2_t fv = {f, f};
    uint4* p = reinterpret_cast<uint4*>(h16 + r * I + i);
    uint4 v = *p;
    v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.x) * fv);
    v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.y) * fv);
    v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.z) * fv);
    v.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.w) * fv);
    *p = v;
  }
}

namespace {

template <int BITS>
hipError_t launch_gemms(const Layer& L, const uint16_t* xa, const int8_t* xexp, char* ws,
                        const Workspace& W, hipStream_t s) {
  const int H = static_cast<int>(L.H), I = static_cast<int>(L.I);
  const int32_t* sorted = reinterpret_cast<const int32_t*>(ws + W.sorted_routes);
  const int4* tiles = reinterpret_cast<const int4*>(ws + W.tiles);
  const int32_t* ntiles = reinterpret_cast<const int32_t*>(ws + W.num_tiles);
  uint16_t* hb = reinterpret_cast<uint16_t*>(ws + W.h16);
  int8_t* hexp = reinterpret_cast<int8_t*>(ws + W.hexp);
  int8_t* rexp = reinterpret_cast<int8_t*>(ws + W.rexp);
  float* yf = reinterpret_cast<float*>(ws + W.yf32);
  const int bs_shift = L.bs == 32 ? 5 : L.bs == 64 ? 6 : 7;   // block sizes are 32/64/128
  const int nt1 = gemm_n_tiles(L, true);
  const int nt2 = gemm_n_tiles(L, false);
  const int64_t g1 = 8 * ((W.max_tiles * nt1 + 7) / 8);
  const int64_t g2 = 8 * ((W.max_tiles * nt2 + 7) / 8);
  auto fc1 = L.fc1_zp ? grouped_gemm_kernel<BITS, true, true> : grouped_gemm_kernel<BITS, true, false>;
  auto fc2 = L.fc2_zp ? grouped_gemm_kernel<BITS, false, true> : grouped_gemm_kernel<BITS, false, false>;
  fc1<<<static_cast<unsigned>(g1), kGemmThreads, 0, s>>>(
      xa, sorted, L.k, L.fc1_codes, L.fc1_scales, H, H, I, bs_shift, L.zp, L.fc1_zp, L.fc1_interleaved,
      L.fc1_bias, L.act,
      L.fc1_row_bytes, L.fc1_nblk,
      tiles, ntiles, nt1, hb, nullptr, xexp, hexp);
  stage_done(L, 6, "gemm_fc1_swiglu");
  h_common_exponent_kernel<<<static_cast<unsigned>((W.R + 255) / 256), 256, 0, s>>>(hb, hexp, rexp, W.R, I);
  stage_done(L, 9, "h_common_exponent");
  fc2<<<static_cast<unsigned>(g2), kGemmThreads, 0, s>>>(
      hb, sorted, L.k, L.fc2_codes, L.fc2_scales, I, H, I, bs_shift, L.zp, L.fc2_zp, false, L.fc2_bias,
      L.act,
      L.fc2_row_bytes, L.fc2_nblk,
      tiles, ntiles, nt2, nullptr, yf, rexp, nullptr);
  stage_done(L, 7, "gemm_fc2");
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stage_x(const Layer& L, const void* x, int64_t T, char* ws, const Workspace& W,
                          hipStream_t s, const uint16_t** xa, const int8_t** xexp) {
  // the matrix operands hold K values in operand order; fp16 activations of
  // a layer whose order is K order go to the matrix cores as they are
  const int P = operand_perm(L.bits);
  *xa = static_cast<const uint16_t*>(x);
  *xexp = nullptr;
  if (L.act == kActF16 && P == 0) return hipSuccess;
  uint16_t* staged = reinterpret_cast<uint16_t*>(ws + W.x16);
  int8_t* e = L.act == kActF16 ? nullptr : reinterpret_cast<int8_t*>(ws + W.xexp);
  const unsigned grid = static_cast<unsigned>((T + 3) / 4);
  const int H = static_cast<int>(L.H);
  auto go = [&](auto pc) {
    constexpr int PP = decltype(pc)::value;
    if (L.act == kActBF16)
      stage_x_f16_kernel<kActBF16, PP><<<grid, 256, 0, s>>>(x, T, H, staged, e);
    else if (L.act == kActF16)
      stage_x_f16_kernel<kActF16, PP><<<grid, 256, 0, s>>>(x, T, H, staged, e);
    else
      stage_x_f16_kernel<kActF32, PP><<<grid, 256, 0, s>>>(x, T, H, staged, e);
  };
  if (P == 8)
    go(std::integral_constant<int, 8>{});
  else if (P == 16)
    go(std::integral_constant<int, 16>{});
  else
    go(std::integral_constant<int, 0>{});
  stage_done(L, 5, "stage_x_f16");
  *xa = staged;
  *xexp = e;
  return hipGetLastError();
}

hipError_t launch_combine(const Layer& L, void* out, int64_t T, char* ws, const Workspace& W,
                          hipStream_t s) {
  const int H = static_cast<int>(L.H);
  dim3 gc((H / 4 + 255) / 256, static_cast<unsigned>(T));
  const float* yf = reinterpret_cast<const float*>(ws + W.yf32);
  const int32_t* inv = reinterpret_cast<const int32_t*>(ws + W.inv_pos);
  const float* w = reinterpret_cast<const float*>(ws + W.topk_w);
  if (L.act == kActBF16)
    combine_kernel<kActBF16><<<gc, 256, 0, s>>>(yf, inv, w, L.k, H, out);
  else if (L.act == kActF16)
    combine_kernel<kActF16><<<gc, 256, 0, s>>>(yf, inv, w, L.k, H, out);
  else
    combine_kernel<kActF32><<<gc, 256, 0, s>>>(yf, inv, w, L.k, H, out);
  stage_done(L, 8, "combine");
  return hipGetLastError();
}

hipError_t launch_prefill(const Layer& L, const void* x, void* out, int64_t T, char* ws,
                          const Workspace& W, hipStream_t s) {
  const uint16_t* xa = nullptr;
  const int8_t* xexp = nullptr;
  hipError_t err = launch_stage_x(L, x, T, ws, W, s, &xa, &xexp);
  if (err != hipSuccess) return err;
  switch (L.bits) {
    case 4: err = launch_gemms<4>(L, xa, xexp, ws, W, s); break;
    case 3: err = launch_gemms<3>(L, xa, xexp, ws, W, s); break;
    default: err = launch_gemms<2>(L, xa, xexp, ws, W, s); break;
  }
  if (err != hipSuccess) return err;
  return launch_combine(L, out, T, ws, W, s);
}

}  // namespace qmoe
