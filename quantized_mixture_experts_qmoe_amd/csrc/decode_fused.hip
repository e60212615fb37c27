// Fused decode path (1..4 tokens, bf16 activations): one kernel launch.
//
// Phases (one workgroup of 8 waves per CU; the grid is the number of
// workgroups that fit on the device at once, so all are resident):
//   0. routing of the <= 4 tokens, recomputed by every workgroup: a parallel
//      rank-based top-k over raw logits and the softmax over the selected k;
//      the list of distinct experts and, per expert, each token's slot;
//   1. FC1 + SwiGLU: items of two gate rows and the two matching up rows of
//      one expert, dealt to the waves in contiguous ranges. Before computing,
//      each wave issues the loads of its first two FC2 items;
//   2. grid barrier;
//   3. FC2: items of eight output rows of one expert, contiguous per wave.
//      Each workgroup stages the h of the expert(s) its waves need in LDS as
//      bf16 hi/lo pairs (converted once per workgroup);
//   4. grid barrier;
//   5. combine: every token's k slots summed in slot order (fp32), rounded
//      once, spread over all threads of the grid.
//
// Cross-workgroup data (h, y) moves only through agent-scope atomic loads and
// stores (global_load/store with sc1), which are coherent per location at
// device scope across the XCDs' separate L2 caches. A barrier arrival waits
// for the workgroup's own stores to complete (s_waitcnt) before it publishes
// its flag, so no cache write-back or invalidate is needed. Barriers are one
// flag per workgroup plus a release word, tagged with a per-call epoch.
//
// Matrix cores: v_mfma_f32_4x4x4_16b_bf16 works on 16 independent 4x4 blocks;
// block b (lanes 4b..4b+3) multiplies A_b (lane 4b+i holds token i's four
// k-values) by B_b (lane 4b+j holds four k-values of weight row j) and lane
// 4b+j receives D_b[token i][row j] in element i, so with four tokens every
// lane does useful work. FC1 gives the 16 blocks 16 different quant blocks of
// four rows; FC2 gives them 8 quant blocks x 2 sets of four rows. One 16-byte
// unit of 32 INT4 codes feeds eight consecutive MFMAs of one block.
//
// Exactness: each code enters as the bf16 value 1 + q/128 (its bits OR-ed
// into the mantissa of 1.0); the block sum is then
// sum((q - zp) * v) = 128 * D - (128 + zp) * sum(v), scaled by the fp16 block
// scale in fp32. x is bf16 and exact; the fp32 h of FC2 enters as bf16 hi + lo
// (16 significant bits) through two MFMAs into the same accumulator.
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
constexpr uint32_t kSpinLimit = 1u << 24;   // bounded barrier wait (then flag and go on)
constexpr int kMaxI32 = 32;                  // FC2 quant blocks staged (I <= 1024)

// sync buffer words
constexpr int kSyncError = 0;
constexpr int kSyncRelease = 32;
constexpr int kSyncFlags = 64;

__device__ __forceinline__ f32x4_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                         f32x4_t c) {
  const short4_t a = __builtin_bit_cast(short4_t, u32x2_t{a0, a1});
  const short4_t b = __builtin_bit_cast(short4_t, u32x2_t{b0, b1});
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_flag(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct FusedLds {
  float logits[kDecodeMaxTokens][kMaxExperts + 4];
  float selv[kDecodeMaxTokens][kMaxTopK];
  int32_t ids[kDecodeMaxTokens * kMaxTopK];
  float w[kDecodeMaxTokens * kMaxTopK];
  int32_t firstr[kMaxExperts];                  // expert -> its first route
  int nfirst[2];
  int32_t dindex[kDecodeMaxTokens * kMaxTopK];  // first route -> distinct index
  int32_t dlist[kDecodeMaxTokens * kMaxTopK];   // distinct index -> expert
  int32_t dslot[kDecodeMaxTokens * kMaxTopK][kDecodeMaxTokens];
  int nd;
  // FC2 A operand of one expert, in register order: unit c, 16-byte chunk j
  // (pairs 4j..4j+3), lane l (token l & 3, quant block (l >> 2) + 8c; lanes
  // l and l + 32 use the same slot), so a wave's ds_read_b128 are bank-conflict
  // free; bf16 hi and lo pairs, and the sum of the represented values per
  // (token, quant block)
  uint4 ahi[kMaxI32 / 8][4][32];
  uint4 alo[kMaxI32 / 8][4][32];
  float hsum[kDecodeMaxTokens][kMaxI32];
};

// Grid barrier: every workgroup publishes `epoch` in its flag after its own
// coherent stores have completed; workgroup 0 waits for all flags and then
// publishes `epoch` in the release word, which the others wait for.
__device__ void flag_barrier(uint32_t* sync, uint32_t epoch) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(sync + kSyncFlags + blockIdx.x, epoch, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (blockIdx.x == 0) {
    if (threadIdx.x < kWave) {
      for (int i = threadIdx.x; i < static_cast<int>(gridDim.x); i += kWave) {
        uint32_t spins = 0;
        while (load_flag(sync + kSyncFlags + i) != epoch) {
          if (++spins > kSpinLimit) {
            atomicOr(sync + kSyncError, 1u);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(sync + kSyncRelease, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (load_flag(sync + kSyncRelease) != epoch) {
      if (++spins > kSpinLimit) {
        atomicOr(sync + kSyncError, 2u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Share value v of lane (lane & ~3) | t with the four lanes of each block.
__device__ __forceinline__ float quad_get(float v, int lane, int t) {
  return __shfl(v, (lane & ~3) | t, kWave);
}

}  // namespace

struct FusedArgs {
  const uint16_t* x;
  const uint16_t* logits;
  void* out;
  const uint8_t* c1;
  const uint16_t* s1;
  const uint8_t* c2;
  const uint16_t* s2;
  int T, E, k, H, I, bs, zp;
  int64_t rb1, rb2, nb1, nb2;
  int32_t* ws_ids;
  float* ws_w;
  float* h32;
  float* y32;
  uint32_t* sync;
  uint32_t epoch;   // this call uses epoch + 1 and epoch + 2
};

// U1: FC1 quant blocks per lane (ceil(H/32 / 16)); U2: FC2 quant blocks per lane (ceil(I/32 / 8)).
template <int BITS, int U1, int U2>
__global__ __launch_bounds__(kFusedThreads) void decode_fused_kernel(FusedArgs a) {
  __shared__ FusedLds S;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int gw = blockIdx.x * kFusedWaves + wave, NW = gridDim.x * kFusedWaves;
  const int T = a.T, k = a.k, H = a.H, I = a.I, E = a.E, zp = a.zp, bs = a.bs;
  const int R = T * k;
  const int blk = lane >> 2, q4 = lane & 3;   // MFMA block and lane-in-block
  const float zc = 128.0f + static_cast<float>(zp);

  // ---- logits to LDS and x for the FC1 A operand (neither needs routing)
  // logits: loaded into registers first, written to LDS after the x loads are issued
  const int E4 = (E + 3) & ~3;
  constexpr int kLg = (kDecodeMaxTokens * (kMaxExperts + 4) + kFusedThreads - 1) / kFusedThreads;
  uint16_t lg[kLg];
#pragma unroll
  for (int q = 0; q < kLg; ++q) {
    const int i = threadIdx.x + q * kFusedThreads;
    const int t = i / E4, e = i % E4;
    const bool ok = i < T * E4 && e < E;
    lg[q] = a.logits[ok ? static_cast<int64_t>(t) * E + e : 0];
  }
  // x: every lane issues all of its loads before consuming any (clamped
  // addresses, zeroed afterwards when out of range)
  const int nkb1 = H / 32;
  uint4 xraw[U1][4];
#pragma unroll
  for (int c = 0; c < U1; ++c) {
    const int kb = blk + 16 * c;
    const int kbc = kb < nkb1 ? kb : 0, tc = q4 < T ? q4 : 0;
    const uint4* src = reinterpret_cast<const uint4*>(a.x + static_cast<int64_t>(tc) * H + 32 * kbc);
#pragma unroll
    for (int q = 0; q < 4; ++q) xraw[c][q] = src[q];
  }
#pragma unroll
  for (int q = 0; q < kLg; ++q) {
    const int i = threadIdx.x + q * kFusedThreads;
    const int t = i / E4, e = i % E4;
    if (i < T * E4) S.logits[t][e] = (e < E) ? canon_logit(bf16_to_f32(lg[q])) : -__builtin_inff();
  }
  for (int i = threadIdx.x; i < R; i += kFusedThreads)
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) S.dslot[i][t] = -1;
  __syncthreads();

  // ---- routing: wave t selects token t's experts
  if (wave < T) topk_softmax_dpp(S.logits[wave], E, k, lane, S.ids + wave * k, S.w + wave * k);
  __syncthreads();
  // distinct experts in first-occurrence order: the first route of each
  // expert from an LDS min table, its index from ballots over the (<= 128) routes
  {
    const int r = threadIdx.x;
    const int e = (r < R) ? S.ids[r] : 0;
    if (r < R) S.firstr[e] = R;
    __syncthreads();
    if (r < R) atomicMin(&S.firstr[e], r);
    __syncthreads();
    const bool is_first = (r < R) && (S.firstr[e] == r);
    const uint64_t mask = __ballot(is_first);
    if (lane == 0 && wave < 2) S.nfirst[wave] = __popcll(mask);
    __syncthreads();
    if (is_first) {
      const int d = __popcll(mask & ((1ull << lane) - 1ull)) + (wave == 1 ? S.nfirst[0] : 0);
      S.dindex[r] = d;
      S.dlist[d] = e;
    }
    __syncthreads();
    if (r < R) S.dslot[S.dindex[S.firstr[e]]][r / k] = r % k;
    if (threadIdx.x == 0) S.nd = S.nfirst[0] + (R > kWave ? S.nfirst[1] : 0);
  }
  __syncthreads();
  const int D = S.nd;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < R; i += kFusedThreads) {
      a.ws_ids[i] = S.ids[i];
      a.ws_w[i] = S.w[i];
    }

  uint32_t xp[U1][16];
  float sx[U1];
#pragma unroll
  for (int c = 0; c < U1; ++c) {
    const bool ok = (blk + 16 * c) < nkb1 && q4 < T;
    uint32_t v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[4 * q] = ok ? xraw[c][q].x : 0u; v[4 * q + 1] = ok ? xraw[c][q].y : 0u;
      v[4 * q + 2] = ok ? xraw[c][q].z : 0u; v[4 * q + 3] = ok ? xraw[c][q].w : 0u;
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += bf16_to_f32((v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int pa = pair_a(BITS, p), pb = pair_b(BITS, p);
      xp[c][p] = ((v[pa >> 1] >> (16 * (pa & 1))) & 0xFFFFu) | (((v[pb >> 1] >> (16 * (pb & 1))) & 0xFFFFu) << 16);
    }
    sx[c] = sum;
  }
  float corr1[U1][kDecodeMaxTokens];
#pragma unroll
  for (int c = 0; c < U1; ++c)
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) corr1[c][t] = zc * quad_get(sx[c], lane, t);

  // ---- work ranges (contiguous per wave)
  const int g1 = I / 2;
  const int n1 = D * g1;
  const int i1_0 = static_cast<int>(static_cast<int64_t>(n1) * gw / NW);
  const int i1_1 = static_cast<int>(static_cast<int64_t>(n1) * (gw + 1) / NW);
  const int g2 = H / 8;
  const int n2 = D * g2;
  const int i2_0 = static_cast<int>(static_cast<int64_t>(n2) * gw / NW);
  const int i2_1 = static_cast<int>(static_cast<int64_t>(n2) * (gw + 1) / NW);
  const int nkb2 = I / 32;

  auto load_fc2 = [&](int it, UnitWords<BITS> (&wv)[U2], float (&sc)[U2]) {
    const int e = S.dlist[it / g2];
    const int m = (it % g2) * 8 + (blk >= 8 ? 4 : 0) + q4;
    const uint8_t* rowp = a.c2 + (static_cast<int64_t>(e) * H + m) * a.rb2;
    const uint16_t* srow = a.s2 + (static_cast<int64_t>(e) * H + m) * a.nb2;
#pragma unroll
    for (int c = 0; c < U2; ++c) {
      const int kb = (blk & 7) + 8 * c;
      if (kb < nkb2) {
        wv[c] = load_unit<BITS>(rowp + kb * (4 * BITS));
        sc[c] = half_to_f32(srow[(32 * kb) / bs]);
      } else {
#pragma unroll
        for (int w = 0; w < BITS; ++w) wv[c].w[w] = 0u;
        sc[c] = 0.0f;
      }
    }
  };
  auto load_fc1 = [&](int it, UnitWords<BITS> (&wv)[U1], float (&sc)[U1]) {
    const int e = S.dlist[it / g1];
    const int n = 2 * (it % g1) + (q4 & 1);
    const int row = (q4 < 2) ? n : I + n;
    const uint8_t* rowp = a.c1 + (static_cast<int64_t>(e) * 2 * I + row) * a.rb1;
    const uint16_t* srow = a.s1 + (static_cast<int64_t>(e) * 2 * I + row) * a.nb1;
#pragma unroll
    for (int c = 0; c < U1; ++c) {
      const int kb = blk + 16 * c;
      if (kb < nkb1) {
        wv[c] = load_unit<BITS>(rowp + kb * (4 * BITS));
        sc[c] = half_to_f32(srow[(32 * kb) / bs]);
      } else {
#pragma unroll
        for (int w = 0; w < BITS; ++w) wv[c].w[w] = 0u;
        sc[c] = 0.0f;
      }
    }
  };

  // ---- loads: the first two FC1 items, then the first two FC2 items of this wave
  UnitWords<BITS> w1a[U1], w1b[U1];
  float s1a[U1], s1b[U1];
  if (i1_0 < i1_1) load_fc1(i1_0, w1a, s1a);
  if (i1_0 + 1 < i1_1) load_fc1(i1_0 + 1, w1b, s1b);
  UnitWords<BITS> w2a[U2], w2b[U2];
  float s2a[U2], s2b[U2];
  if (i2_0 < i2_1) load_fc2(i2_0, w2a, s2a);
  if (i2_0 + 1 < i2_1) load_fc2(i2_0 + 1, w2b, s2b);

  // ---- phase 1: FC1 + SwiGLU
  for (int it = i1_0; it < i1_1; ++it) {
    float acc[kDecodeMaxTokens] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < U1; ++c) {
      uint32_t wp[16];
#pragma unroll
      for (int p = 0; p < 16; ++p) wp[p] = unit_pair<BITS>(w1a[c], p);
      f32x4_t dv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 8; ++m) dv = mfma4(xp[c][2 * m], xp[c][2 * m + 1], wp[2 * m], wp[2 * m + 1], dv);
      const float s = s1a[c], s128 = 128.0f * s1a[c];
#pragma unroll
      for (int t = 0; t < kDecodeMaxTokens; ++t)
        acc[t] = fmaf(s128, dv[t], fmaf(-s, corr1[c][t], acc[t]));
    }
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) {
      acc[t] += __shfl_xor(acc[t], 4, kWave);
      acc[t] += __shfl_xor(acc[t], 8, kWave);
      acc[t] += __shfl_xor(acc[t], 16, kWave);
      acc[t] += __shfl_xor(acc[t], 32, kWave);
    }
    float up[kDecodeMaxTokens];
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) up[t] = __shfl_down(acc[t], 2, kWave);
    if (lane < 2) {
      const int d = it / g1;
      const int n = 2 * (it % g1) + lane;
#pragma unroll
      for (int t = 0; t < kDecodeMaxTokens; ++t) {
        const int slot = (t < T) ? S.dslot[d][t] : -1;
        if (slot >= 0)
          store_coherent(a.h32 + static_cast<int64_t>(t * k + slot) * I + n, silu_mul(acc[t], up[t]));
      }
    }
#pragma unroll
    for (int c = 0; c < U1; ++c) {
      w1a[c] = w1b[c];
      s1a[c] = s1b[c];
    }
    if (it + 2 < i1_1) load_fc1(it + 2, w1b, s1b);
  }

  // ---- phase 2
  flag_barrier(a.sync, a.epoch + 1);

  // ---- phase 3: FC2, one staged expert at a time
  const int wg0 = static_cast<int>(static_cast<int64_t>(n2) * (blockIdx.x * kFusedWaves) / NW);
  const int wg1 = static_cast<int>(static_cast<int64_t>(n2) * ((blockIdx.x + 1) * kFusedWaves) / NW);
  const int d_lo = wg0 / g2, d_hi = (wg1 - 1) / g2;
  int it = i2_0;
  for (int d = d_lo; wg0 < wg1 && d <= d_hi; ++d) {
    // stage h of expert d in register order (see FusedLds)
    __syncthreads();
    for (int i = threadIdx.x; i < U2 * 4 * 32; i += kFusedThreads) {
      const int c = i / 128, j = (i / 32) % 4, l = i % 32;
      const int t = l & 3, kb = (l >> 2) + 8 * c;
      const int slot = (t < T) ? S.dslot[d][t] : -1;
      uint32_t hi[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
      if (slot >= 0 && kb < nkb2) {
        const float* hr = a.h32 + static_cast<int64_t>(t * k + slot) * I + 32 * kb;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int p = 4 * j + q;
          const float va = load_coherent(hr + pair_a(BITS, p)), vb = load_coherent(hr + pair_b(BITS, p));
          hi[q] = f32x2_to_bf16x2(va, vb);
          lo[q] = f32x2_to_bf16x2(va - bf16_to_f32(hi[q] & 0xFFFFu), vb - bf16_to_f32(hi[q] >> 16));
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
    if (it >= i2_1 || it / g2 != d) continue;
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
      for (int t = 0; t < kDecodeMaxTokens; ++t) corr2[c][t] = ok ? zc * S.hsum[t][kb] : 0.0f;
    }
    for (; it < i2_1 && it / g2 == d; ++it) {
      float acc[kDecodeMaxTokens] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < U2; ++c) {
        uint32_t wp[16];
#pragma unroll
        for (int p = 0; p < 16; ++p) wp[p] = unit_pair<BITS>(w2a[c], p);
        f32x4_t dv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          dv = mfma4(hhi[c][2 * m], hhi[c][2 * m + 1], wp[2 * m], wp[2 * m + 1], dv);
          dv = mfma4(hlo[c][2 * m], hlo[c][2 * m + 1], wp[2 * m], wp[2 * m + 1], dv);
        }
        const float s = s2a[c], s128 = 128.0f * s2a[c];
#pragma unroll
        for (int t = 0; t < kDecodeMaxTokens; ++t)
          acc[t] = fmaf(s128, dv[t], fmaf(-s, corr2[c][t], acc[t]));
      }
#pragma unroll
      for (int c = 0; c < U2; ++c) {
        w2a[c] = w2b[c];
        s2a[c] = s2b[c];
      }
      if (it + 2 < i2_1) load_fc2(it + 2, w2b, s2b);
#pragma unroll
      for (int t = 0; t < kDecodeMaxTokens; ++t) {
        acc[t] += __shfl_xor(acc[t], 4, kWave);
        acc[t] += __shfl_xor(acc[t], 8, kWave);
        acc[t] += __shfl_xor(acc[t], 16, kWave);
      }
      if ((lane & ~32) < 4) {
        const int m = (it % g2) * 8 + (lane >= 32 ? 4 : 0) + q4;
#pragma unroll
        for (int t = 0; t < kDecodeMaxTokens; ++t) {
          const int slot = (t < T) ? S.dslot[d][t] : -1;
          if (slot >= 0) store_coherent(a.y32 + static_cast<int64_t>(t * k + slot) * H + m, acc[t]);
        }
      }
    }
  }

  // ---- phase 4
  flag_barrier(a.sync, a.epoch + 2);

  // ---- phase 5: out[t][m] = round(sum_j w[t][j] * y[t*k + j][m]), slot order
  for (int idx = blockIdx.x * kFusedThreads + threadIdx.x; idx < T * H;
       idx += gridDim.x * kFusedThreads) {
    const int t = idx / H, m = idx % H;
    float o = 0.0f;
    for (int j = 0; j < k; ++j)
      o = fmaf(S.w[t * k + j], load_coherent(a.y32 + static_cast<int64_t>(t * k + j) * H + m), o);
    static_cast<uint16_t*>(a.out)[idx] = static_cast<uint16_t>(f32_to_bf16(o));
  }
}

namespace {

template <int BITS, int U1, int U2>
const void* fused_fn() {
  return reinterpret_cast<const void*>(&decode_fused_kernel<BITS, U1, U2>);
}

template <int BITS>
const void* fused_fn_bits(int u1, int u2) {
#define QMOE_FUSED_CASE(A, B) \
  if (u1 == A && u2 == B) return fused_fn<BITS, A, B>();
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

const void* fused_kernel_for(const Layer& L) {
  const int u1 = fused_u1(L), u2 = fused_u2(L);
  switch (L.bits) {
    case 4: return fused_fn_bits<4>(u1, u2);
    case 3: return fused_fn_bits<3>(u1, u2);
    default: return fused_fn_bits<2>(u1, u2);
  }
}

}  // namespace

bool fused_decode_supported(const Layer& L) {
  return L.act_bf16 && fused_u1(L) > 0 && fused_u2(L) > 0 && L.H % 8 == 0 && L.I % 2 == 0 &&
         L.E <= kMaxExperts && fused_kernel_for(L) != nullptr;
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

hipError_t launch_decode_fused(const Layer& L, const void* x, const void* logits, void* out,
                               int64_t T, char* ws, const Workspace& W, uint32_t* sync,
                               uint32_t epoch, int grid, hipStream_t s) {
  FusedArgs fa;
  fa.x = static_cast<const uint16_t*>(x);
  fa.logits = static_cast<const uint16_t*>(logits);
  fa.out = out;
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
  fa.rb1 = L.fc1_row_bytes;
  fa.rb2 = L.fc2_row_bytes;
  fa.nb1 = L.fc1_nblk;
  fa.nb2 = L.fc2_nblk;
  fa.ws_ids = reinterpret_cast<int32_t*>(ws + W.topk_id);
  fa.ws_w = reinterpret_cast<float*>(ws + W.topk_w);
  fa.h32 = reinterpret_cast<float*>(ws + W.h32);
  fa.y32 = reinterpret_cast<float*>(ws + W.y32);
  fa.sync = sync;
  fa.epoch = epoch;
  void* args[] = {&fa};
  const hipError_t err =
      hipLaunchKernel(fused_kernel_for(L), dim3(grid), dim3(kFusedThreads), args, 0, s);
  if (err == hipSuccess) stage_done(L, 1, "decode_fused");
  return err;
}

}  // namespace qmoe
