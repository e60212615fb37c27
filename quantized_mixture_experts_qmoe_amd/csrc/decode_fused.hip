// Fused decode path (1..4 tokens, bf16 or fp16 activations): one kernel launch with
// no grid-wide barrier.
//
// Layers with FC1/FC2 biases or per-block zero-point tensors run an instance
// that also loads, per weight row, the row's bias and its blocks' zero points
// (EX below).
//
// Phases (one workgroup of 8 waves per CU; the grid is the number of
// workgroups that fit on the device at once, so all are resident):
//   0. routing of the <= 4 tokens, recomputed by every workgroup: wave t
//      takes token t's logits straight into registers as 32-bit keys
//      (ordered bf16 logit, then the inverted expert index) and selects the
//      k largest with DPP max reductions, then the routing weights (softmax
//      over the selected, or without normalization over all experts);
//      the distinct experts, in ascending expert order, come from an LDS
//      bitmask;
//   1. FC1 + SwiGLU: items of two gate rows and the two matching up rows of
//      one expert, dealt to the workgroups in contiguous ranges; inside a
//      workgroup each wave starts with two items and then claims the next
//      unclaimed one from an LDS counter whenever it finishes one, so waves
//      that the memory system serves sooner take more items. Each wave issues
//      the loads of its first two FC1 items before computing anything, those
//      of its first two FC2 items after its first FC1 item, keeps two FC1
//      items in flight, buffers its h values in LDS and writes them out in
//      batches; the loads of its third and fourth FC2 items follow once the
//      expert's h is staged;
//   2. FC2: a workgroup works on one expert (or, with more experts than
//      workgroups, on whole experts in turn). It stages the expert's h in LDS
//      as bf16 hi/lo pairs, waiting for each value to arrive, and its waves
//      compute items of eight output rows, buffered in LDS and written once;
//   3. combine: each group of eight output rows has one combining wave, which
//      waits for the group's y values of every token slot, sums each token's
//      k slots in slot order in fp32 and rounds once.
//
// Cross-workgroup data (h, y) lives in a buffer the handle owns, as 64-bit
// entries {fp32 value, epoch} written and read with single agent-scope atomic
// stores and loads (global_store/load_dwordx2 with sc1), which are coherent
// per location at device scope across the XCDs' separate L2 caches. A
// consumer spins on the entries themselves until every one it needs carries
// this call's epoch, so a value becomes usable one memory round trip after it
// is stored: no flag, no fence, no read-modify-write atomic. Each call has a
// new nonzero epoch; the buffer is zeroed at create and again when the epoch
// counter wraps, so no entry can hold a matching epoch before this call's
// producer writes it. Waits are bounded: a wait that runs out sets an error
// bit and goes on.
//
// Matrix cores: v_mfma_f32_4x4x4_16b_bf16 works on 16 independent 4x4 blocks;
// block b (lanes 4b..4b+3) multiplies A_b (lane 4b+i holds token i's four
// k-values) by B_b (lane 4b+j holds four k-values of weight row j) and lane
// 4b+j receives D_b[token i][row j] in element i, so with four tokens every
// lane does useful work. FC1 gives the 16 blocks 16 different quant blocks of
// four rows; FC2 gives them 8 quant blocks x 2 sets of four rows. One unit of
// 32 codes feeds eight consecutive MFMAs of one block.
//
// Weight codes and scales are read through buffer resources. Every load of an
// item is issued unconditionally, so the compiler's wait counts stay static; a
// load for an item the wave has no use for (past the end of its range) gets a
// resource with no records, which returns zeros without touching memory.
//
// Exactness: each code enters as the bf16 value 128 + q (the code is the low
// mantissa byte of 128.0); the block sum is then
// sum((q - zp) * v) = D - (128 + zp) * sum(v), scaled by the fp16 block scale
// in fp32. x is bf16 and exact; the fp32 h of FC2 enters as bf16 hi + lo
// (16 significant bits) through two MFMAs into the same accumulator. With
// fp16 activations FC1's codes enter as fp16 1 + q/128 instead, and the
// block sum is 128 * D - (128 + zp) * sum(v).
//
// Semantics: SwiGLU experts, fc1 rows = 2 * inter ("[CUDA/CPU] Add AVX2 INT4
// cold-expert kernel and zero-cold doorbell short-circuit for QMoE offload",
// Motivation & Summary item 3); top-k over raw logits with a softmax over the
// selected ("Document and test packed token inputs for MoE and QMoE", review
// of the test harness); fp32 partial sums rounded once ("[CUDA] Add MoEPacked
// CPU/GPU hybrid offload and consolidate QMoE/GGUF offload optimizations",
// Key Changes item 4).
#include "device.h"
#include "internal.h"

namespace qmoe {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * kWave;
constexpr int kKeySlots = kFusedMaxExperts / kWave;   // logits per lane in the top-k
constexpr int kMaxRoutes = kDecodeMaxTokens * kMaxTopK;
constexpr int kMaxGroups = 256;                       // output row groups of 8 (H <= 2048)
constexpr int kXRow = 2048 / 8 + 1;                   // 16-byte vectors per token row of x in LDS
                                                      // (H <= 2048, padded by one vector)
static_assert(kDecodeMaxTokens * (kXRow - 1) <= 2 * kFusedThreads, "x staging: two vectors per thread");
constexpr int kMaxI32 = 32;                           // FC2 quant blocks staged (I <= 1024)
constexpr int kCap1 = 32;                             // FC1 items buffered per wave (even)
constexpr int kCap2 = 16;                             // FC2 items buffered per wave (multiple of 4)
constexpr uint32_t kSpinLimit = 1u << 20;             // default bound of a wait for an exchange entry

__device__ __forceinline__ f32x4_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                         f32x4_t c) {
  const short4_t a = __builtin_bit_cast(short4_t, u32x2_t{a0, a1});
  const short4_t b = __builtin_bit_cast(short4_t, u32x2_t{b0, b1});
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}

// fp16 activations: the same 4x4x4 block product on fp16 operands (x is exact
// in fp16, and so is 1 + q/128 for q < 128).
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t mfma4_f16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                             f32x4_t c) {
  const half4_t a = __builtin_bit_cast(half4_t, u32x2_t{a0, a1});
  const half4_t b = __builtin_bit_cast(half4_t, u32x2_t{b0, b1});
  return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 0, 0, 0);
}

// A 16-bit activation value (bf16, or fp16 when F16) as fp32, exactly.
template <bool F16>
__device__ __forceinline__ float act16(uint32_t bits) {
  return F16 ? half_to_f32(static_cast<uint16_t>(bits)) : bf16_to_f32(bits);
}
// The logit a routing key was made from (logit_key orders the 16-bit
// patterns of bf16 and fp16 alike: both are sign-magnitude).
template <bool F16>
__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t ord = key >> 16;
  return act16<F16>((ord & 0x8000u) ? (ord & 0x7FFFu) : (~ord & 0xFFFFu));
}

// Pair p of a unit as two fp16 values 1 + q/128: the code sits at bit 3 of
// the fp16 mantissa of 1.0 (0x3C00); same pairing as unit_pair.
template <int BITS>
__device__ __forceinline__ uint32_t unit_pair_f16(const UnitWords<BITS>& u, int p) {
  if constexpr (BITS == 4) {
    const uint32_t w = u.w[p >> 2];
    const int sh = 4 * (p & 3);
    const uint32_t v = sh >= 3 ? (w >> (sh - 3)) : (w << (3 - sh));
    return (v & 0x00780078u) | 0x3C003C00u;
  } else if constexpr (BITS == 2) {
    const uint32_t w = u.w[p >> 3];
    const int sh = 2 * (p & 7);
    const uint32_t v = sh >= 3 ? (w >> (sh - 3)) : (w << (3 - sh));
    return (v & 0x00180018u) | 0x3C003C00u;
  } else {
    return ((unit_code<3>(u, 2 * p) | (unit_code<3>(u, 2 * p + 1) << 16)) << 3) | 0x3C003C00u;
  }
}

// Exchange entries: {fp32 value (low word), epoch (high word)}.
__device__ __forceinline__ void put_tagged(uint64_t* p, float v, uint32_t epoch) {
  const uint64_t e = (static_cast<uint64_t>(epoch) << 32) | __float_as_uint(v);
  __hip_atomic_store(p, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_tagged(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(uint64_t e, uint32_t epoch) {
  return static_cast<uint32_t>(e >> 32) == epoch;
}
__device__ __forceinline__ float tag_value(uint64_t e) {
  return __uint_as_float(static_cast<uint32_t>(e));
}

struct FusedLds {
  int32_t ids[kMaxRoutes];                            // route r = t*k + j -> expert
  float w[kMaxRoutes];                                // routing weight of route r
  uint32_t emask[kFusedMaxExperts / 32];              // experts selected by any token
  int8_t slot[kDecodeMaxTokens][kFusedMaxExperts];    // (token, expert) -> slot, or -1
  int32_t dlist[kFusedWaves][kMaxRoutes];             // distinct index -> expert (ascending),
                                                      // one copy per wave
  int next1;                                          // FC1 items claimed past the static ones
  int32_t hitem[kFusedWaves][kCap1];                  // FC1 item of each buffered h pair
  // FC2 A operand of one expert, in register order: unit c, 16-byte chunk j
  // (pairs 4j..4j+3), lane l (token l & 3, quant block (l >> 2) + 8c; lanes
  // l and l + 32 use the same slot), so a wave's ds_read_b128 are bank-conflict
  // free; bf16 hi and lo pairs, and the sum of the represented values per
  // (token, quant block)
  uint4 ahi[kMaxI32 / 8][4][32];
  uint4 alo[kMaxI32 / 8][4][32];
  float hsum[kDecodeMaxTokens][kMaxI32];
  // x (FC1 A operand source), token rows padded so the four tokens of a quad
  // fall in different banks
  uint4 xs[kDecodeMaxTokens][kXRow];
  // per-wave result buffers: h [token][2 * item + row], y [token][8 * item + row]
  float hbuf[kFusedWaves][kDecodeMaxTokens][2 * kCap1];
  float ybuf[kFusedWaves][kDecodeMaxTokens][8 * kCap2];
};

// Cross-lane moves without the LDS crossbar (DPP and v_permlane*_swap).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over lanes l, l-4, l-8, l-12 of each row of 16 (one residue class mod 4)
__device__ __forceinline__ float row_class_sum(float v) {
  v += dpp_f<0x124>(v);   // row_ror:4
  v += dpp_f<0x128>(v);   // row_ror:8
  return v;
}
// v of this lane plus v of the same lane in the paired row (rows 0+1, 2+3)
__device__ __forceinline__ float row_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// v of this lane plus v of the same lane in the other half of the wave
__device__ __forceinline__ float half_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// value of lane t of this lane's quad (DPP quad_perm [t, t, t, t])
template <int T>
__device__ __forceinline__ float quad_get(float v) {
  return dpp_f<T * 0x55>(v);
}

// A raw buffer resource over `bytes` bytes at p (stride 0: offsets are byte
// offsets, range-checked against `bytes`; 0x00020000 is the gfx9 data-format
// word for raw dword access). bytes = 0 makes every load return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
// One unit (32 codes) at byte offset off of a resource.
template <int BITS>
__device__ __forceinline__ UnitWords<BITS> load_unit_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  UnitWords<BITS> u;
  if constexpr (BITS == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    u.w[0] = v[0]; u.w[1] = v[1]; u.w[2] = v[2]; u.w[3] = v[3];
  } else if constexpr (BITS == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    u.w[0] = v[0]; u.w[1] = v[1];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
    u.w[0] = v[0]; u.w[1] = v[1]; u.w[2] = v[2];
  }
  return u;
}
__device__ __forceinline__ uint32_t load_u16_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

}  // namespace

struct FusedArgs {
  const uint16_t* x;
  const uint16_t* logits;
  uint16_t* out;
  const uint8_t* c1;
  const uint16_t* s1;
  const uint8_t* c2;
  const uint16_t* s2;
  int T, E, k, H, I, bs, zp;
  int normalize;     // routing weights over the selected k (1) or over all experts (0)
  int fc1_il;        // FC1 rows interleaved: 2n gate n, 2n+1 up n
  int64_t rb1, rb2, nb1, nb2;
  uint32_t c1_bytes, s1_bytes, c2_bytes, s2_bytes;   // sizes of c1, s1, c2, s2 (< 2^31)
  int32_t* ws_ids;
  float* ws_w;
  uint64_t* hx;      // exchange: h [route][inter]
  uint64_t* yx;      // exchange: y [route][hidden]
  uint32_t* err;     // error bits (bounded waits that ran out)
  uint32_t epoch;    // nonzero; no exchange entry holds it before this call writes it
  // optional: FC1/FC2 biases (bf16, [E][2I] / [E][H]) and per-block
  // zero-point codes (uint8, laid out like the scales); read only by the
  // instance built for layers that have any of them
  const uint16_t* b1;
  const uint16_t* b2;
  const uint8_t* z1;
  const uint8_t* z2;
  uint32_t spin_limit;   // polls before a wait for an exchange entry gives up
};

// U1: FC1 quant blocks per lane (ceil(H/32 / 16)); U2: FC2 quant blocks per lane (ceil(I/32 / 8)).
// EX: the layer has biases or zero-point tensors. Each lane then also loads,
// with an item's codes and scales, the bias of its weight row and the zero
// point of each of its quant blocks; the block correction becomes
// (128 + zp) * sum(x) per block, and the bias is added to the row's sum
// before SwiGLU (FC1) or before the combine (FC2).
// F16: fp16 x, logits, biases and out (with EX): FC1 runs on fp16 operands;
// FC2's operands are built from the fp32 h as in the bf16 case.
template <int BITS, int U1, int U2, bool EX, bool F16>
__global__ __launch_bounds__(kFusedThreads) void decode_fused_kernel(FusedArgs a) {
  __shared__ FusedLds S;
  // wave-uniform values go through readfirstlane so the compiler keeps them
  // (and the loops over them) scalar
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * kFusedWaves + wave, NW = gridDim.x * kFusedWaves;
  const int T = a.T, k = a.k, H = a.H, I = a.I, E = a.E, zp = a.zp, bs = a.bs;
  const int R = T * k;
  const int blk = lane >> 2, q4 = lane & 3;   // MFMA block and lane-in-block
  const float zc = 128.0f + static_cast<float>(zp);

  // ---- loads that need no routing: token `wave`'s logits, then x (FC1 A
  // operand), two 16-byte vectors per thread, staged in LDS once per
  // workgroup; all addresses clamped in range, values masked afterwards
  uint16_t lg[kKeySlots];
  if (wave < T) {
#pragma unroll
    for (int c = 0; c < kKeySlots; ++c) {
      const int e = lane + kWave * c;
      lg[c] = a.logits[static_cast<int64_t>(wave) * E + (e < E ? e : 0)];
    }
  }
  const int nkb1 = H / 32;
  // (a thread past the end re-reads a vector other threads also read, so no
  // single line gets every spare thread's request)
  const int xrow = H / 8, nx = T * xrow;   // vectors per token row, in all
  const int xi0 = static_cast<int>(threadIdx.x), xi1 = xi0 + kFusedThreads;
  const uint4 xv0 = reinterpret_cast<const uint4*>(a.x)[xi0 % nx];
  const uint4 xv1 = reinterpret_cast<const uint4*>(a.x)[xi1 % nx];
  if (threadIdx.x < kDecodeMaxTokens * kFusedMaxExperts / 4)
    reinterpret_cast<uint32_t*>(&S.slot[0][0])[threadIdx.x] = 0xFFFFFFFFu;
  if (threadIdx.x < kFusedMaxExperts / 32) S.emask[threadIdx.x] = 0u;
  if (threadIdx.x == 0) S.next1 = 0;
  __syncthreads();

  // ---- routing: wave t selects token t's experts
  if (wave < T) {
    uint32_t keys[kKeySlots];
#pragma unroll
    for (int c = 0; c < kKeySlots; ++c) {
      const int e = lane + kWave * c;
      keys[c] = (e < E) ? logit_key(lg[c], e) : 0u;
    }
    uint32_t mine = 0u, first = 0u;
    for (int j = 0; j < k; ++j) {
      uint32_t b = keys[0];
#pragma unroll
      for (int c = 1; c < kKeySlots; ++c) b = keys[c] > b ? keys[c] : b;
      b = wave_umax(b);
      if (j == 0) first = b;
      if (lane == j) mine = b;
#pragma unroll
      for (int c = 0; c < kKeySlots; ++c) keys[c] = (keys[c] == b) ? 0u : keys[c];
    }
    const float ex = (lane < k) ? expf(key_value<F16>(mine) - key_value<F16>(first)) : 0.0f;
    float all = 0.0f;   // sum over all experts (weights without normalization)
    if (!a.normalize)
#pragma unroll
      for (int c = 0; c < kKeySlots; ++c)
        if (lane + kWave * c < E) all += expf(act16<F16>(lg[c]) - key_value<F16>(first));
    const float sum = wave_sum(a.normalize ? ex : all);
    if (lane < k) {
      const int e = key_to_expert(mine);
      S.ids[wave * k + lane] = e;
      S.w[wave * k + lane] = ex / sum;
      S.slot[wave][e] = static_cast<int8_t>(lane);
      atomicOr(&S.emask[e >> 5], 1u << (e & 31));
    }
  }
  if (xi0 < nx) S.xs[xi0 / xrow][xi0 % xrow] = xv0;
  if (xi1 < nx) S.xs[xi1 / xrow][xi1 % xrow] = xv1;
  __syncthreads();
  // distinct experts in ascending order (prefix of the mask words'
  // popcounts), built by every wave into its own copy, so no barrier waits
  // for one wave to build it; LDS accesses of a wave complete in order
  int D;
  {
    uint32_t m = (lane < (E + 31) / 32) ? S.emask[lane] : 0u;
    const int pc = __popc(m);
    int incl = pc;
#pragma unroll
    for (int off = 1; off < kFusedMaxExperts / 32; off <<= 1) {
      const int o = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += o;
    }
    int pos = incl - pc;
    while (m) {
      S.dlist[wave][pos++] = lane * 32 + (__ffs(m) - 1);
      m &= m - 1u;
    }
    D = __builtin_amdgcn_readlane(incl, kFusedMaxExperts / 32 - 1);
  }
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < R; i += kFusedThreads) {
      a.ws_ids[i] = S.ids[i];
      a.ws_w[i] = S.w[i];
    }

  // ---- work ranges
  // FC1: items (expert d, row pair p), contiguous per workgroup over the grid
  const int g1 = I / 2;
  const int n1 = D * g1;
  // (unsigned 32-bit range arithmetic: n1 <= 32 * 512 and blockIdx.x < 1024,
  // so every product fits, and the divisions stay short scalar sequences)
  const uint32_t un1 = static_cast<uint32_t>(n1), uNG = static_cast<uint32_t>(gridDim.x);
  const int w1_0 = static_cast<int>(un1 * blockIdx.x / uNG);
  const int w1_1 = static_cast<int>(un1 * (blockIdx.x + 1) / uNG);
  // FC2: items (expert d, group q of 8 output rows); a workgroup owns a slice
  // of one expert when there are at least as many workgroups as experts,
  // otherwise whole experts [dA, dB)
  const int NG = gridDim.x;
  const int g2 = H / 8;
  int dA, dB, q0, q1;
  if (D <= NG) {
    dA = static_cast<int>(blockIdx.x * static_cast<uint32_t>(D) / static_cast<uint32_t>(NG));
    dB = dA + 1;
    const int w_lo = static_cast<int>(static_cast<uint32_t>(dA * NG + D - 1) / static_cast<uint32_t>(D));
    const int w_hi = static_cast<int>(static_cast<uint32_t>((dA + 1) * NG + D - 1) / static_cast<uint32_t>(D));
    const int nq = (w_hi - w_lo) * kFusedWaves, qw = (blockIdx.x - w_lo) * kFusedWaves + wave;
    q0 = static_cast<int>(static_cast<uint32_t>(g2 * qw) / static_cast<uint32_t>(nq));
    q1 = static_cast<int>(static_cast<uint32_t>(g2 * (qw + 1)) / static_cast<uint32_t>(nq));
  } else {
    dA = static_cast<int>(blockIdx.x * static_cast<uint32_t>(D) / static_cast<uint32_t>(NG));
    dB = static_cast<int>((blockIdx.x + 1) * static_cast<uint32_t>(D) / static_cast<uint32_t>(NG));
    q0 = g2 * wave / kFusedWaves;
    q1 = g2 * (wave + 1) / kFusedWaves;
  }
  const int nkb2 = I / 32;

  const int bsh = (bs == 32) ? 0 : (bs == 64) ? 1 : 2;   // bs = 32 << bsh: block of unit kb
  // Loads of one item: branch-free (out-of-range quant blocks read unit 0 and
  // get a zero scale when used); scales stay raw fp16 until used.
  // (live: the wave uses the item; otherwise its loads read nothing. it and
  // live are wave-uniform, so the resources stay in scalar registers.)
  auto load_fc1 = [&](int it, bool live, UnitWords<BITS> (&wv)[U1], uint32_t (&sc)[U1], uint32_t& bv,
                      uint32_t (&zv)[U1]) {
    const int e = S.dlist[wave][it / g1];
    const int n = 2 * (it % g1) + (q4 & 1);
    const int row = a.fc1_il ? 2 * n + (q4 >> 1) : ((q4 < 2) ? n : I + n);
    const uint32_t grow = static_cast<uint32_t>(e * 2 * I + row);
    const __amdgpu_buffer_rsrc_t rc = raw_rsrc(a.c1, live ? a.c1_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(a.s1, live ? a.s1_bytes : 0u);
    const uint32_t cofs = grow * static_cast<uint32_t>(a.rb1);
    const uint32_t sofs = grow * static_cast<uint32_t>(a.nb1);
#pragma unroll
    for (int c = 0; c < U1; ++c) {
      const int kb = blk + 16 * c;
      const int kbc = kb < nkb1 ? kb : 0;
      wv[c] = load_unit_rsrc<BITS>(rc, cofs + kbc * (4 * BITS));
      sc[c] = load_u16_rsrc(rs, 2 * (sofs + (kbc >> bsh)));
    }
    if constexpr (EX) {
      (void)live;
      bv = a.b1 ? a.b1[static_cast<int64_t>(e) * 2 * I + row] : 0u;
      const uint8_t* zrow = a.z1 ? a.z1 + (static_cast<int64_t>(e) * 2 * I + row) * a.nb1 : nullptr;
#pragma unroll
      for (int c = 0; c < U1; ++c) {
        const int kb = blk + 16 * c;
        zv[c] = zrow ? zrow[(kb < nkb1 ? kb : 0) >> bsh] : static_cast<uint32_t>(zp);
      }
    }
  };
  auto load_fc2 = [&](int d, int q, bool live, UnitWords<BITS> (&wv)[U2], uint32_t (&sc)[U2],
                      uint32_t& bv, uint32_t (&zv)[U2]) {
    const int e = S.dlist[wave][d];
    const int m = q * 8 + (blk >= 8 ? 4 : 0) + q4;
    const uint32_t grow = static_cast<uint32_t>(e * H + m);
    const __amdgpu_buffer_rsrc_t rc = raw_rsrc(a.c2, live ? a.c2_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(a.s2, live ? a.s2_bytes : 0u);
    const uint32_t cofs = grow * static_cast<uint32_t>(a.rb2);
    const uint32_t sofs = grow * static_cast<uint32_t>(a.nb2);
#pragma unroll
    for (int c = 0; c < U2; ++c) {
      const int kb = (blk & 7) + 8 * c;
      const int kbc = kb < nkb2 ? kb : 0;
      wv[c] = load_unit_rsrc<BITS>(rc, cofs + kbc * (4 * BITS));
      sc[c] = load_u16_rsrc(rs, 2 * (sofs + (kbc >> bsh)));
    }
    if constexpr (EX) {
      bv = a.b2 ? a.b2[static_cast<int64_t>(e) * H + m] : 0u;
      const uint8_t* zrow = a.z2 ? a.z2 + (static_cast<int64_t>(e) * H + m) * a.nb2 : nullptr;
#pragma unroll
      for (int c = 0; c < U2; ++c) {
        const int kb = (blk & 7) + 8 * c;
        zv[c] = zrow ? zrow[(kb < nkb2 ? kb : 0) >> bsh] : static_cast<uint32_t>(zp);
      }
    }
  };

  // ---- issue: the first two FC1 items, then the first two FC2 items. The
  // loads are unconditional (an item past the wave's range is a valid index
  // whose loads read nothing), so the compiler's wait counts stay exact.
  UnitWords<BITS> w1A[U1], w1B[U1];
  uint32_t s1A[U1], s1B[U1];   // raw fp16 scales, one per register
  uint32_t b1A = 0u, b1B = 0u, z1A[U1], z1B[U1];   // raw bias and zero points (EX)
  // (sched_barrier keeps the issue order A, B that the waits below count
  // on; the first FC2 items follow the wave's first FC1 item)
  const int last1 = max(w1_1 - 1, 0);
  int itA = w1_0 + wave, itB = w1_0 + kFusedWaves + wave;   // (itA past the end => itB too)
  load_fc1(min(itA, last1), itA < w1_1, w1A, s1A, b1A, z1A);
  __builtin_amdgcn_sched_barrier(0);
  load_fc1(min(itB, last1), itB < w1_1, w1B, s1B, b1B, z1B);
  __builtin_amdgcn_sched_barrier(0);
  UnitWords<BITS> w2A[U2], w2B[U2];
  uint32_t s2A[U2], s2B[U2];
  uint32_t b2A = 0u, b2B = 0u, z2A[U2], z2B[U2];
  const int last2 = max(q1 - 1, 0);
  // FC2's first two items load once the wave's first FC1 item is computed,
  // so the FC1 loads go out first; FC2 needs its weights only after h is
  // staged. (A wave with a single FC2 item, as every wave has at M=1, loads
  // no second one.)
  auto load_fc2_first = [&]() {
    load_fc2(dA, min(q0, last2), q0 < q1, w2A, s2A, b2A, z2A);
    if (q0 + 1 < q1) load_fc2(dA, q0 + 1, true, w2B, s2B, b2B, z2B);
  };

  // x pairs and their sums (x was staged in LDS before the routing's last barrier)
  uint32_t xp[U1][16];
  float sx[U1];
#pragma unroll
  for (int c = 0; c < U1; ++c) {
    const int kb = blk + 16 * c;
    const bool ok = kb < nkb1 && q4 < T;
    const int kbc = kb < nkb1 ? kb : 0, tc = q4 < T ? q4 : 0;
    uint32_t v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 xq = S.xs[tc][4 * kbc + q];
      v[4 * q] = ok ? xq.x : 0u; v[4 * q + 1] = ok ? xq.y : 0u;
      v[4 * q + 2] = ok ? xq.z : 0u; v[4 * q + 3] = ok ? xq.w : 0u;
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += act16<F16>((v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int pa = pair_a(BITS, p), pb = pair_b(BITS, p);
      xp[c][p] = ((v[pa >> 1] >> (16 * (pa & 1))) & 0xFFFFu) | (((v[pb >> 1] >> (16 * (pb & 1))) & 0xFFFFu) << 16);
    }
    sx[c] = sum;
  }
  float corr1[U1][kDecodeMaxTokens];
#pragma unroll
  for (int c = 0; c < U1; ++c) {
    // (with EX the zero point varies per block: the sums stay raw here and
    // the item scales them by 128 + zp)
    const float zcc = EX ? 1.0f : zc;
    corr1[c][0] = zcc * quad_get<0>(sx[c]);
    corr1[c][1] = zcc * quad_get<1>(sx[c]);
    corr1[c][2] = zcc * quad_get<2>(sx[c]);
    corr1[c][3] = zcc * quad_get<3>(sx[c]);
  }

  // one FC1 item: gate/up sums of two rows for every token, SwiGLU, into hbuf
  auto fc1_item = [&](const UnitWords<BITS> (&wv)[U1], const uint32_t (&sc)[U1], uint32_t bv,
                      const uint32_t (&zv)[U1], int li) {
    float acc[kDecodeMaxTokens] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < U1; ++c) {
      uint32_t wp[16];
#pragma unroll
      for (int p = 0; p < 16; ++p) wp[p] = F16 ? unit_pair_f16<BITS>(wv[c], p) : unit_pair<BITS>(wv[c], p);
      f32x4_t dv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 8; ++m)
        dv = F16 ? mfma4_f16(xp[c][2 * m], xp[c][2 * m + 1], wp[2 * m], wp[2 * m + 1], dv)
                 : mfma4(xp[c][2 * m], xp[c][2 * m + 1], wp[2 * m], wp[2 * m + 1], dv);
      const float s = (blk + 16 * c) < nkb1 ? half_to_f32(static_cast<uint16_t>(sc[c])) : 0.0f;
      // (bf16 codes enter as 128 + q, fp16 codes as 1 + q/128)
      const float sw = F16 ? 128.0f * s : s;
      // (with EX: the same product (128 + zp) * sum(x) as the scalar path
      // forms once, so a tensor holding the scalar gives identical bits)
      const float zcl = 128.0f + static_cast<float>(zv[c]);
#pragma unroll
      for (int t = 0; t < kDecodeMaxTokens; ++t)
        acc[t] = fmaf(sw, dv[t], fmaf(-s, EX ? zcl * corr1[c][t] : corr1[c][t], acc[t]));
    }
    // sum over the 16 blocks: lanes 0..3 end with rows 0..3 (gate n, gate
    // n+1, up n, up n+1); lanes 0 and 1 then take the up sums of lanes 2, 3
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) acc[t] = half_pair_sum(row_pair_sum(row_class_sum(acc[t])));
    if (EX && a.b1) {
      // every lane now holds the total of its row: add that row's bias
      const float b = act16<F16>(bv);
#pragma unroll
      for (int t = 0; t < kDecodeMaxTokens; ++t) acc[t] += b;
    }
    float up[kDecodeMaxTokens];
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) up[t] = dpp_f<0xEE>(acc[t]);   // quad_perm [2, 3, 2, 3]
    if (lane < 2)
#pragma unroll
      for (int t = 0; t < kDecodeMaxTokens; ++t) S.hbuf[wave][t][2 * li + lane] = silu_mul(acc[t], up[t]);
  };

  // ---- phase 1: FC1 + SwiGLU, two items in flight, claimed one at a time;
  // results buffered per wave and written out in batches
  auto claim = [&]() -> int {   // the workgroup's next FC1 item (wave-uniform)
    int v = 0;
    if (lane == 0) v = atomicAdd(&S.next1, 1);
    return w1_0 + 2 * kFusedWaves + __builtin_amdgcn_readfirstlane(v);
  };
  auto flush_h = [&](int nb) {  // write the nb buffered items' h (pairs contiguous)
    const int ni2 = 2 * nb;
    for (int i = lane; i < T * ni2; i += kWave) {
      const int t = i / ni2, nl = i % ni2;
      const int it = S.hitem[wave][nl >> 1], d = it / g1;
      const int slot = S.slot[t][S.dlist[wave][d]];
      if (slot >= 0)
        put_tagged(a.hx + static_cast<int64_t>(t * k + slot) * I + 2 * (it % g1) + (nl & 1),
                   S.hbuf[wave][t][nl], a.epoch);
    }
  };
  int nbuf = 0;   // items in this wave's h buffer
  // (the loop's first pass, with FC2's first loads after the first item)
  if (itA < w1_1) {
    fc1_item(w1A, s1A, b1A, z1A, nbuf);
    if (lane == 0) S.hitem[wave][nbuf] = itA;
    ++nbuf;
    const int nA = claim();
    load_fc1(min(nA, last1), nA < w1_1, w1A, s1A, b1A, z1A);
    load_fc2_first();
    if (itB < w1_1) {
      fc1_item(w1B, s1B, b1B, z1B, nbuf);
      if (lane == 0) S.hitem[wave][nbuf] = itB;
      ++nbuf;
    }
    const int nB = claim();
    load_fc1(min(nB, last1), nB < w1_1, w1B, s1B, b1B, z1B);
    itA = nA;
    itB = nB;
  } else {
    load_fc2_first();
  }
  while (itA < w1_1) {
    fc1_item(w1A, s1A, b1A, z1A, nbuf);
    if (lane == 0) S.hitem[wave][nbuf] = itA;
    ++nbuf;
    const int nA = claim();
    load_fc1(min(nA, last1), nA < w1_1, w1A, s1A, b1A, z1A);
    if (itB < w1_1) {
      fc1_item(w1B, s1B, b1B, z1B, nbuf);
      if (lane == 0) S.hitem[wave][nbuf] = itB;
      ++nbuf;
    }
    const int nB = claim();   // (claimed after nA: nA past the end => nB too)
    load_fc1(min(nB, last1), nB < w1_1, w1B, s1B, b1B, z1B);
    itA = nA;
    itB = nB;
    if (nbuf + 2 > kCap1) {
      flush_h(nbuf);
      nbuf = 0;
    }
  }
  flush_h(nbuf);
  // the third and fourth FC2 items of this wave, loaded once h is staged
  // (the waits on h's entries would otherwise also wait for them: loads
  // complete in order). Loads past the wave's range are not issued at all
  // from here on: nothing later is timed on them, and a wave that skips
  // them leaves the memory pipeline to the waves still streaming.
  UnitWords<BITS> w2C[U2], w2D[U2];
  uint32_t s2C[U2], s2D[U2];
  uint32_t b2C = 0u, b2D = 0u, z2C[U2], z2D[U2];

  // ---- phase 2: FC2 of this workgroup's expert(s)
  for (int d = dA; d < dB; ++d) {
    __syncthreads();   // previous expert's staging area is free
    const int e = S.dlist[wave][d];
    // stage h of expert d in register order (see FusedLds)
    for (int i = threadIdx.x; i < U2 * 4 * 32; i += kFusedThreads) {
      const int c = i / 128, j = (i / 32) % 4, l = i % 32;
      const int t = l & 3, kb = (l >> 2) + 8 * c;
      const int slot = (t < T) ? S.slot[t][e] : -1;
      uint32_t hi[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
      if (slot >= 0 && kb < nkb2) {
        // the h values of this (token, quant block, chunk), each waited for
        // until it carries this call's epoch
        const uint64_t* hr = a.hx + static_cast<int64_t>(t * k + slot) * I + 32 * kb;
        uint64_t ea[4], eb[4];
        uint32_t spins = 0;
        bool ready;
        do {
          ready = true;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            ea[q] = get_tagged(hr + pair_a(BITS, 4 * j + q));
            eb[q] = get_tagged(hr + pair_b(BITS, 4 * j + q));
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) ready = ready && tag_is(ea[q], a.epoch) && tag_is(eb[q], a.epoch);
          if (!ready) {
            if (++spins > a.spin_limit) {
              atomicOr(a.err, 1u);
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        } while (!ready);
        float va[4], vb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          va[q] = tag_value(ea[q]);
          vb[q] = tag_value(eb[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hi[q] = f32x2_to_bf16x2(va[q], vb[q]);
          lo[q] = f32x2_to_bf16x2(va[q] - bf16_to_f32(hi[q] & 0xFFFFu), vb[q] - bf16_to_f32(hi[q] >> 16));
        }
      }
      S.ahi[c][j][l] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      S.alo[c][j][l] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kDecodeMaxTokens * nkb2; i += kFusedThreads) {
      const int t = i / nkb2, kb = i % nkb2;
      const int c = kb / 8, l = ((kb % 8) << 2) | t;
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 h4 = S.ahi[c][j][l], l4 = S.alo[c][j][l];
        const uint32_t hv[4] = {h4.x, h4.y, h4.z, h4.w}, lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          s += (bf16_to_f32(hv[q] & 0xFFFFu) + bf16_to_f32(lv[q] & 0xFFFFu)) +
               (bf16_to_f32(hv[q] >> 16) + bf16_to_f32(lv[q] >> 16));
      }
      S.hsum[t][kb] = s;
    }
    __syncthreads();
    if (q0 >= q1) continue;
    if (d == dA) {
      if (q0 + 2 < q1) load_fc2(dA, q0 + 2, true, w2C, s2C, b2C, z2C);
      if (q0 + 3 < q1) load_fc2(dA, q0 + 3, true, w2D, s2D, b2D, z2D);
    }
    // this wave's A operand for expert d
    uint32_t hhi[U2][16], hlo[U2][16];
    float corr2[U2][kDecodeMaxTokens];
#pragma unroll
    for (int c = 0; c < U2; ++c) {
      const int kb = (blk & 7) + 8 * c;
      const bool ok = kb < nkb2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 h4 = S.ahi[c][j][lane & 31], l4 = S.alo[c][j][lane & 31];
        hhi[c][4 * j] = h4.x; hhi[c][4 * j + 1] = h4.y; hhi[c][4 * j + 2] = h4.z; hhi[c][4 * j + 3] = h4.w;
        hlo[c][4 * j] = l4.x; hlo[c][4 * j + 1] = l4.y; hlo[c][4 * j + 2] = l4.z; hlo[c][4 * j + 3] = l4.w;
      }
#pragma unroll
      for (int t = 0; t < kDecodeMaxTokens; ++t) corr2[c][t] = ok ? (EX ? 1.0f : zc) * S.hsum[t][kb] : 0.0f;
    }
    if (d != dA) {
      load_fc2(d, q0, true, w2A, s2A, b2A, z2A);
      if (q0 + 1 < q1) load_fc2(d, q0 + 1, true, w2B, s2B, b2B, z2B);
      if (q0 + 2 < q1) load_fc2(d, q0 + 2, true, w2C, s2C, b2C, z2C);
      if (q0 + 3 < q1) load_fc2(d, q0 + 3, true, w2D, s2D, b2D, z2D);
    }
    auto fc2_item = [&](const UnitWords<BITS> (&wv)[U2], const uint32_t (&sc)[U2], uint32_t bv,
                        const uint32_t (&zv)[U2], int li) {
      float acc[kDecodeMaxTokens] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < U2; ++c) {
        uint32_t wp[16];
#pragma unroll
        for (int p = 0; p < 16; ++p) wp[p] = unit_pair<BITS>(wv[c], p);
        f32x4_t dv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          dv = mfma4(hhi[c][2 * m], hhi[c][2 * m + 1], wp[2 * m], wp[2 * m + 1], dv);
          dv = mfma4(hlo[c][2 * m], hlo[c][2 * m + 1], wp[2 * m], wp[2 * m + 1], dv);
        }
        const float s = ((blk & 7) + 8 * c) < nkb2 ? half_to_f32(static_cast<uint16_t>(sc[c])) : 0.0f;
        const float zcl = 128.0f + static_cast<float>(zv[c]);
#pragma unroll
        for (int t = 0; t < kDecodeMaxTokens; ++t)
          acc[t] = fmaf(s, dv[t], fmaf(-s, EX ? zcl * corr2[c][t] : corr2[c][t], acc[t]));
      }
      // sum over the 8 quant blocks of each half wave: lanes 0..3 end with
      // rows 0..3 of the item, lanes 32..35 with rows 4..7
#pragma unroll
      for (int t = 0; t < kDecodeMaxTokens; ++t) acc[t] = row_pair_sum(row_class_sum(acc[t]));
      if (EX && a.b2) {
        // lanes holding a row's total add that row's bias
        const float b = act16<F16>(bv);
#pragma unroll
        for (int t = 0; t < kDecodeMaxTokens; ++t) acc[t] += b;
      }
      if ((lane & ~32) < 4)
#pragma unroll
        for (int t = 0; t < kDecodeMaxTokens; ++t)
          S.ybuf[wave][t][8 * li + (lane >= 32 ? 4 : 0) + q4] = acc[t];
    };
    for (int c0 = q0; c0 < q1; c0 += kCap2) {
      const int c1 = min(c0 + kCap2, q1);
      for (int q = c0; q < c1; q += 4) {
        fc2_item(w2A, s2A, b2A, z2A, q - c0);
        if (q + 4 < q1) load_fc2(d, q + 4, true, w2A, s2A, b2A, z2A);
        if (q + 1 < c1) fc2_item(w2B, s2B, b2B, z2B, q + 1 - c0);
        if (q + 5 < q1) load_fc2(d, q + 5, true, w2B, s2B, b2B, z2B);
        if (q + 2 < c1) fc2_item(w2C, s2C, b2C, z2C, q + 2 - c0);
        if (q + 6 < q1) load_fc2(d, q + 6, true, w2C, s2C, b2C, z2C);
        if (q + 3 < c1) fc2_item(w2D, s2D, b2D, z2D, q + 3 - c0);
        if (q + 7 < q1) load_fc2(d, q + 7, true, w2D, s2D, b2D, z2D);
      }
      // write this chunk's y (coalesced along m per token)
      const int nm = 8 * (c1 - c0);
      for (int i = lane; i < T * nm; i += kWave) {
        const int t = i / nm, ml = i % nm;
        const int slot = S.slot[t][e];
        if (slot >= 0)
          put_tagged(a.yx + static_cast<int64_t>(t * k + slot) * H + 8 * c0 + ml, S.ybuf[wave][t][ml],
                     a.epoch);
      }
    }
  }

  // ---- phase 3: combine the row groups this wave owns
  const int gc0 = static_cast<int>(static_cast<uint32_t>(g2 * gw) / static_cast<uint32_t>(NW));
  const int gc1 = static_cast<int>(static_cast<uint32_t>(g2 * (gw + 1)) / static_cast<uint32_t>(NW));
  for (int grp = gc0; grp < gc1; ++grp) {
    if (lane < 8 * T) {
      const int t = lane >> 3, m = 8 * grp + (lane & 7);
      const uint64_t* yr = a.yx + static_cast<int64_t>(t * k) * H + m;
      float o = 0.0f;
      for (int j0 = 0; j0 < k; j0 += 8) {
        // slots j0..j0+7 of token t at row m, each waited for until it
        // carries this call's epoch
        uint64_t v[8];
        uint32_t spins = 0;
        bool ready;
        do {
          ready = true;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            v[j] = (j0 + j < k) ? get_tagged(yr + static_cast<int64_t>(j0 + j) * H) : 0ull;
#pragma unroll
          for (int j = 0; j < 8; ++j) ready = ready && (j0 + j >= k || tag_is(v[j], a.epoch));
          if (!ready) {
            if (++spins > a.spin_limit) {
              atomicOr(a.err, 2u);
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        } while (!ready);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j0 + j < k) o = fmaf(S.w[t * k + j0 + j], tag_value(v[j]), o);
      }
      a.out[static_cast<int64_t>(t) * H + m] =
          F16 ? __builtin_bit_cast(uint16_t, static_cast<_Float16>(o)) : static_cast<uint16_t>(f32_to_bf16(o));
    }
  }
}

namespace {

// variant 0: bf16; 1: bf16 with biases or zero-point tensors; 2: fp16 (with
// the same extras machinery, which costs nothing when a layer has none)
template <int BITS, int U1, int U2>
const void* fused_fn(int variant) {
  if (variant == 2) return reinterpret_cast<const void*>(&decode_fused_kernel<BITS, U1, U2, true, true>);
  if (variant == 1) return reinterpret_cast<const void*>(&decode_fused_kernel<BITS, U1, U2, true, false>);
  return reinterpret_cast<const void*>(&decode_fused_kernel<BITS, U1, U2, false, false>);
}

template <int BITS>
const void* fused_fn_bits(int u1, int u2, int ex) {
#define QMOE_FUSED_CASE(A, B) \
  if (u1 == A && u2 == B) return fused_fn<BITS, A, B>(ex);
  QMOE_FUSED_CASE(1, 1)
  QMOE_FUSED_CASE(1, 2)
  QMOE_FUSED_CASE(2, 1)
  QMOE_FUSED_CASE(2, 2)
  QMOE_FUSED_CASE(4, 1)
  QMOE_FUSED_CASE(4, 2)
  QMOE_FUSED_CASE(4, 3)
  QMOE_FUSED_CASE(4, 4)
#undef QMOE_FUSED_CASE
  return nullptr;
}

int fused_u1(const Layer& L) {
  const int64_t nkb = L.H / 32;
  return nkb <= 16 ? 1 : nkb <= 32 ? 2 : nkb <= 64 ? 4 : 0;
}
int fused_u2(const Layer& L) {
  const int64_t nkb = L.I / 32;
  return nkb <= 8 ? 1 : nkb <= 16 ? 2 : nkb <= 24 ? 3 : nkb <= 32 ? 4 : 0;
}

bool fused_extras(const Layer& L) {
  return L.fc1_bias || L.fc2_bias || L.fc1_zp || L.fc2_zp;
}

const void* fused_kernel_for(const Layer& L) {
  const int u1 = fused_u1(L), u2 = fused_u2(L);
  const int ex = L.act == kActF16 ? 2 : fused_extras(L) ? 1 : 0;
  switch (L.bits) {
    case 4: return fused_fn_bits<4>(u1, u2, ex);
    case 3: return fused_fn_bits<3>(u1, u2, ex);
    default: return fused_fn_bits<2>(u1, u2, ex);
  }
}

}  // namespace

bool fused_decode_supported(const Layer& L) {
  // (with biases or zero-point tensors, I > 768 runs the split decode: that
  // instance would keep its extra operands in scratch memory)
  const bool ex = fused_extras(L) || L.act == kActF16;
  return (L.act_bf16 || L.act == kActF16) && fused_u1(L) > 0 && (!ex || fused_u2(L) <= 3) &&
         fused_u2(L) > 0 &&
         L.H % 8 == 0 && L.I % 2 == 0 &&
         L.E <= kFusedMaxExperts && L.k <= kMaxTopK && fused_kernel_for(L) != nullptr &&
         // buffer resources take byte sizes below 2^31
         L.E * 2 * L.I * L.fc1_row_bytes < (int64_t{1} << 31) &&
         L.E * L.H * L.fc2_row_bytes < (int64_t{1} << 31);
}

int fused_decode_grid(const Layer& L, int device) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    return 0;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fused_kernel_for(L), kFusedThreads, 0) !=
      hipSuccess)
    return 0;
  if (nb > 1) nb = 1;   // one workgroup per CU
  const int grid = cus * nb;
  return grid <= kFusedMaxWorkgroups ? grid : kFusedMaxWorkgroups;
}

size_t fused_exchange_bytes(const Layer& L) {
  const size_t routes = static_cast<size_t>(kDecodeMaxTokens) * static_cast<size_t>(L.k);
  return kExchangeHeader + routes * static_cast<size_t>(L.I + L.H) * sizeof(uint64_t);
}

namespace {
__global__ void exchange_clear_kernel(uint4* p, size_t n16) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}
}  // namespace

hipError_t clear_exchange(const Layer& L, void* xbuf, hipStream_t s) {
  const size_t n16 = fused_exchange_bytes(L) / 16;
  hipLaunchKernelGGL(exchange_clear_kernel, dim3(256), dim3(256), 0, s, static_cast<uint4*>(xbuf), n16);
  return hipGetLastError();
}

hipError_t launch_decode_fused(const Layer& L, const void* x, const void* logits, void* out,
                               int64_t T, char* ws, const Workspace& W, void* xbuf,
                               uint32_t epoch, int grid, uint32_t spin_limit, hipStream_t s) {
  FusedArgs fa;
  fa.x = static_cast<const uint16_t*>(x);
  fa.logits = static_cast<const uint16_t*>(logits);
  fa.out = static_cast<uint16_t*>(out);
  fa.c1 = L.fc1_codes;
  fa.s1 = L.fc1_scales;
  fa.c2 = L.fc2_codes;
  fa.s2 = L.fc2_scales;
  fa.T = static_cast<int>(T);
  fa.E = static_cast<int>(L.E);
  fa.k = L.k;
  fa.H = static_cast<int>(L.H);
  fa.I = static_cast<int>(L.I);
  fa.bs = L.bs;
  fa.zp = L.zp;
  fa.normalize = L.normalize ? 1 : 0;
  fa.fc1_il = L.fc1_interleaved ? 1 : 0;
  fa.rb1 = L.fc1_row_bytes;
  fa.rb2 = L.fc2_row_bytes;
  fa.nb1 = L.fc1_nblk;
  fa.nb2 = L.fc2_nblk;
  fa.c1_bytes = static_cast<uint32_t>(L.E * 2 * L.I * L.fc1_row_bytes);
  fa.s1_bytes = static_cast<uint32_t>(L.E * 2 * L.I * L.fc1_nblk * 2);
  fa.c2_bytes = static_cast<uint32_t>(L.E * L.H * L.fc2_row_bytes);
  fa.s2_bytes = static_cast<uint32_t>(L.E * L.H * L.fc2_nblk * 2);
  fa.b1 = static_cast<const uint16_t*>(L.fc1_bias);
  fa.b2 = static_cast<const uint16_t*>(L.fc2_bias);
  fa.z1 = L.fc1_zp;
  fa.z2 = L.fc2_zp;
  fa.ws_ids = reinterpret_cast<int32_t*>(ws + W.topk_id);
  fa.ws_w = reinterpret_cast<float*>(ws + W.topk_w);
  char* xb = static_cast<char*>(xbuf);
  const size_t routes = static_cast<size_t>(kDecodeMaxTokens) * static_cast<size_t>(L.k);
  fa.err = reinterpret_cast<uint32_t*>(xb);
  fa.hx = reinterpret_cast<uint64_t*>(xb + kExchangeHeader);
  fa.yx = fa.hx + routes * static_cast<size_t>(L.I);
  fa.epoch = epoch;
  fa.spin_limit = spin_limit ? spin_limit : kSpinLimit;
  void* args[] = {&fa};
  const hipError_t err =
      hipLaunchKernel(fused_kernel_for(L), dim3(grid), dim3(kFusedThreads), args, 0, s);
  if (err == hipSuccess) stage_done(L, 1, "decode_fused");
  return err;
}

}  // namespace qmoe
