// Routing for the grouped (prefill) path: top-k + softmax over the selected
// logits fused with a per-chunk expert histogram (chunks of 32 tokens), one
// scan that yields expert offsets, per-chunk scatter bases and the GEMM tile
// list, and a stable scatter of the route ids into expert-sorted order.
//
// Semantics: top-k on the raw router logits with a softmax over the selected
// k ("Document and test packed token inputs for MoE and QMoE", review of the
// test harness); the expert-sorted route map with per-expert first offsets is
// the grouped-GEMM input the tensor-core prefill path consumes ("[CUDA] Add
// INT4 and INT3 QMoE CPU/GPU offload support", Description of #33731:
// sorted_routes, tile descriptors, expert_first_token_offset).
#include <utility>

#include "device.h"
#include "internal.h"

namespace qmoe {

// Top-k + softmax of the chunk's tokens (chunk c = tokens [32c, 32c + 32);
// wave w of eight takes four of them in turn, loading the next token's logits while
// it selects the current one) and the chunk's expert histogram:
// hist[c][e] = number of the chunk's routes sent to e.
template <int SLOTS>
__global__ __launch_bounds__(512) void route_topk_hist_bf16_kernel(
    const uint16_t* __restrict__ logits, int64_t T, int E, int k, bool normalize,
    int32_t* __restrict__ topk_id, float* __restrict__ topk_w, int32_t* __restrict__ hist) {
  __shared__ int32_t s_hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 512) s_hist[e] = 0;
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  constexpr int kPerWave = kChunkTokens / 8;
  const int64_t tw = static_cast<int64_t>(blockIdx.x) * kChunkTokens + wave * kPerWave;
  auto load = [&](int64_t t, uint16_t (&lg)[SLOTS]) {
    const int64_t tc = t < T ? t : T - 1;
#pragma unroll
    for (int c = 0; c < SLOTS; ++c) {
      const int e = lane + kWave * c;
      lg[c] = logits[tc * E + (e < E ? e : 0)];
    }
  };
  uint16_t cur[SLOTS], nxt[SLOTS];
  load(tw, cur);
  for (int i = 0; i < kPerWave; ++i) {
    const int64_t t = tw + i;
    if (t >= T) break;
    load(t + 1, nxt);
    int id;
    float wt;
    topk_softmax_bf16_wave<SLOTS>(cur, E, k, normalize, lane, id, wt);
    if (lane < k) {
      topk_id[t * k + lane] = id;
      topk_w[t * k + lane] = wt;
      atomicAdd(&s_hist[id], 1);
    }
#pragma unroll
    for (int c = 0; c < SLOTS; ++c) cur[c] = nxt[c];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 512) hist[static_cast<int64_t>(blockIdx.x) * E + e] = s_hist[e];
}

// The same for fp32 or fp16 logits (64-bit keys: the value widened to fp32,
// then the inverted index).
template <typename ACT>
__global__ __launch_bounds__(512) void route_topk_hist_wide_kernel(
    const ACT* __restrict__ logits, int64_t T, int E, int k, bool normalize,
    int32_t* __restrict__ topk_id, float* __restrict__ topk_w, int32_t* __restrict__ hist) {
  __shared__ int32_t s_hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 512) s_hist[e] = 0;
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  constexpr int kPerWave = kChunkTokens / 8;
  const int64_t tw = static_cast<int64_t>(blockIdx.x) * kChunkTokens + wave * kPerWave;
  for (int i = 0; i < kPerWave; ++i) {
    const int64_t t = tw + i;
    if (t >= T) break;
    int id;
    float wt;
    topk_softmax_wave_r(logits + t * E, E, k, normalize, lane, id, wt);
    if (lane < k) {
      topk_id[t * k + lane] = id;
      topk_w[t * k + lane] = wt;
      atomicAdd(&s_hist[id], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 512) hist[static_cast<int64_t>(blockIdx.x) * E + e] = s_hist[e];
}

// Inclusive scans of a[0..n) and b[0..n) in place (n <= 1024, blockDim.x ==
// 1024, each thread tid < n having written a[tid] and b[tid]): a shuffle
// scan per wave, then the preceding waves' totals; two barriers in all.
__device__ void block_scan2_inclusive(int32_t* a, int32_t* b, int n) {
  __shared__ int32_t s_wa[16], s_wb[16];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
  int32_t va = tid < n ? a[tid] : 0, vb = tid < n ? b[tid] : 0;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t ta = __shfl_up(va, off, kWave), tb = __shfl_up(vb, off, kWave);
    if (lane >= off) {
      va += ta;
      vb += tb;
    }
  }
  if (lane == kWave - 1) {
    s_wa[w] = va;
    s_wb[w] = vb;
  }
  __syncthreads();
  for (int i = 0; i < w; ++i) {
    va += s_wa[i];
    vb += s_wb[i];
  }
  if (tid < n) {
    a[tid] = va;
    b[tid] = vb;
  }
  __syncthreads();
}

// One workgroup of 1024 threads. Thread (e, p) owns expert e and the p-th
// slice of the chunks.
__global__ __launch_bounds__(1024) void route_scan_kernel(const int32_t* __restrict__ hist,
                                                          int64_t nchunks, int E, int tile_m,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ chunk_base,
                                                          int4* __restrict__ tiles,
                                                          int32_t* __restrict__ num_tiles) {
  __shared__ int32_t s_part[1024];
  __shared__ int32_t s_scan[1024];
  __shared__ int32_t s_tiles[1024];
  const int P = 1024 / E;  // E <= 1024
  const int tid = threadIdx.x;
  const int e = tid % E, p = tid / E;
  const bool active = p < P;
  int64_t c0 = 0, c1 = 0;
  if (active) {
    c0 = nchunks * p / P;
    c1 = nchunks * (p + 1) / P;
    // (batches of 32, then 8, independent loads)
    int32_t sum = 0;
    int64_t c = c0;
    for (; c + 32 <= c1; c += 32) {
      int32_t v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) v[u] = hist[(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < 32; ++u) sum += v[u];
    }
    for (; c + 8 <= c1; c += 8) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hist[(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; c < c1; ++c) sum += hist[c * E + e];
    s_part[p * E + e] = sum;
  }
  __syncthreads();
  // per-expert totals and exclusive bases of each slice
  if (tid < E) {
    int32_t run = 0;
    for (int q = 0; q < P; ++q) {
      int32_t v = s_part[q * E + tid];
      s_part[q * E + tid] = run;
      run += v;
    }
    counts[tid] = run;
    s_scan[tid] = run;
    s_tiles[tid] = (run + tile_m - 1) / tile_m;
  }
  block_scan2_inclusive(s_scan, s_tiles, E);
  if (tid < E) {
    offsets[tid + 1] = s_scan[tid];
    if (tid == 0) offsets[0] = 0;
  }
  if (tid == 0) num_tiles[0] = s_tiles[E - 1];
  __syncthreads();
  if (active) {
    const int32_t expert_start = (e == 0) ? 0 : s_scan[e - 1];
    int32_t run = expert_start + s_part[p * E + e];
    int64_t c = c0;
    for (; c + 8 <= c1; c += 8) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hist[(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        chunk_base[(c + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; c < c1; ++c) {
      chunk_base[c * E + e] = run;
      run += hist[c * E + e];
    }
  }
  if (tid < E) {
    const int32_t expert_start = (tid == 0) ? 0 : s_scan[tid - 1];
    const int32_t cnt = s_scan[tid] - expert_start;
    const int32_t t0 = (tid == 0) ? 0 : s_tiles[tid - 1];
    for (int32_t i = 0; i * tile_m < cnt; ++i) {
      const int32_t rows = min(tile_m, cnt - i * tile_m);
      tiles[t0 + i] = make_int4(tid, expert_start + i * tile_m, rows, 0);
    }
  }
}

// Stable scatter: a route's rank among the earlier routes of its chunk that
// chose the same expert, added to the chunk's base for that expert.
__global__ __launch_bounds__(256) void route_scatter_kernel(const int32_t* __restrict__ topk_id,
                                                            int64_t R, int k, int E,
                                                            const int32_t* __restrict__ chunk_base,
                                                            int32_t* __restrict__ sorted_routes,
                                                            int32_t* __restrict__ inv_pos) {
  __shared__ int32_t s_e[kChunkTokens * kMaxTopK];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kChunkTokens * k;
  const int n = static_cast<int>(min(static_cast<int64_t>(kChunkTokens) * k, R - r0));
  for (int i = threadIdx.x; i < n; i += 256) s_e[i] = topk_id[r0 + i];
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 256) {
    const int32_t e = s_e[i];
    int32_t rank = 0;
    for (int j = 0; j < i; ++j) rank += (s_e[j] == e);
    const int32_t pos = chunk_base[static_cast<int64_t>(blockIdx.x) * E + e] + rank;
    sorted_routes[pos] = static_cast<int32_t>(r0 + i);
    inv_pos[r0 + i] = pos;
  }
}

// Routing of a small batch in one launch, together with the activation
// staging. Workgroup 0 (16 waves) routes every token: top-k + softmax (wave
// w takes tokens w, w + 16, ...), then, over the route list in chunks of 64
// routes, each route's rank among the earlier routes of its chunk with the
// same expert and the per-(chunk, expert) counts, a per-expert scan over the
// chunks, the expert offsets and the tile list (tiles of tile_m routes), and
// the stable scatter. Workgroups 1.. stage the activations, one token per
// wave (stage_x_row). Used while the route list and the (chunk, expert)
// table fit in LDS (route_small_fits).
constexpr int kSmallRouteMax = 4096;        // routes of one call
constexpr int kSmallRouteTable = 8192;      // (64-route chunk, expert) counters

bool route_small_fits(const Layer& L, int64_t T) {
  const int64_t R = T * L.k;
  return R <= kSmallRouteMax && ((R + 63) / 64) * L.E <= kSmallRouteTable;
}

template <int SLOTS, typename LG, int ACT, int P>
__global__ __launch_bounds__(1024) void route_small_kernel(
    const LG* __restrict__ logits, int64_t T, int E, int k, bool normalize, int tile_m,
    int32_t* __restrict__ topk_id, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_routes, int32_t* __restrict__ inv_pos,
    int4* __restrict__ tiles, int32_t* __restrict__ num_tiles, const void* __restrict__ x, int H,
    uint16_t* __restrict__ x16, int8_t* __restrict__ xexp) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6, tid = threadIdx.x;
  if (blockIdx.x > 0) {
    const int64_t t = static_cast<int64_t>(blockIdx.x - 1) * 16 + wave;
    if (t < T) stage_x_row<ACT, P>(x, t, H, x16, xexp, lane);
    return;
  }
  __shared__ int32_t s_id[kSmallRouteMax];
  __shared__ uint8_t s_rank[kSmallRouteMax];
  __shared__ int32_t s_tab[kSmallRouteTable];
  __shared__ int32_t s_scan[1024];
  __shared__ int32_t s_tiles[1024];
  const int R = static_cast<int>(T) * k;
  const int nch = (R + 63) / 64;
  for (int i = tid; i < nch * E; i += 1024) s_tab[i] = 0;
  // top-k + softmax, one token per wave at a time (bf16 logits: the next
  // token's logits load while the current one is selected)
  if constexpr (SLOTS > 0) {
    auto load = [&](int64_t t, uint16_t (&lg)[SLOTS]) {
      const int64_t tc = t < T ? t : T - 1;
#pragma unroll
      for (int c = 0; c < SLOTS; ++c) {
        const int e = lane + kWave * c;
        lg[c] = reinterpret_cast<const uint16_t*>(logits)[tc * E + (e < E ? e : 0)];
      }
    };
    uint16_t cur[SLOTS], nxt[SLOTS];
    load(wave, cur);
    for (int64_t t = wave; t < T; t += 16) {
      load(t + 16, nxt);
      int id;
      float wt;
      topk_softmax_bf16_wave<SLOTS>(cur, E, k, normalize, lane, id, wt);
      if (lane < k) {
        topk_id[t * k + lane] = id;
        topk_w[t * k + lane] = wt;
        s_id[t * k + lane] = id;
      }
#pragma unroll
      for (int c = 0; c < SLOTS; ++c) cur[c] = nxt[c];
    }
  } else {
    for (int64_t t = wave; t < T; t += 16) {
      int id;
      float wt;
      topk_softmax_wave_r(logits + t * E, E, k, normalize, lane, id, wt);
      if (lane < k) {
        topk_id[t * k + lane] = id;
        topk_w[t * k + lane] = wt;
        s_id[t * k + lane] = id;
      }
    }
  }
  __syncthreads();
  // per chunk of 64 routes: each route's rank among the chunk's earlier
  // routes with its expert, and the chunk's count per expert (written by
  // the expert's last route in the chunk)
  // (the lanes holding the same expert: the AND over the expert's bits of
  // each bit's ballot or its complement)
  for (int c = wave; c < nch; c += 16) {
    const int r = 64 * c + lane;
    const int e = r < R ? s_id[r] : -1;
    uint64_t same = __ballot(r < R);
    for (int b = 0; (1 << b) < E; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      same &= bit ? bb : ~bb;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    const bool later = lane < kWave - 1 && (same >> (lane + 1)) != 0;
    if (r < R) {
      s_rank[r] = static_cast<uint8_t>(rank);
      if (!later) s_tab[c * E + e] = rank + 1;
    }
  }
  __syncthreads();
  // per expert: exclusive bases of the chunks, the total, its tile count
  if (tid < E) {
    int32_t run = 0;
    for (int c = 0; c < nch; ++c) {
      const int32_t v = s_tab[c * E + tid];
      s_tab[c * E + tid] = run;
      run += v;
    }
    counts[tid] = run;
    s_scan[tid] = run;
    s_tiles[tid] = (run + tile_m - 1) / tile_m;
  }
  block_scan2_inclusive(s_scan, s_tiles, E);
  if (tid < E) {
    offsets[tid + 1] = s_scan[tid];
    if (tid == 0) offsets[0] = 0;
    const int32_t start = tid == 0 ? 0 : s_scan[tid - 1];
    const int32_t cnt = s_scan[tid] - start;
    const int32_t t0 = tid == 0 ? 0 : s_tiles[tid - 1];
    for (int32_t i = 0; i * tile_m < cnt; ++i)
      tiles[t0 + i] = make_int4(tid, start + i * tile_m, min(tile_m, cnt - i * tile_m), 0);
  }
  if (tid == 0) num_tiles[0] = s_tiles[E - 1];
  // stable scatter
  for (int r = tid; r < R; r += 1024) {
    const int e = s_id[r];
    const int32_t pos = (e == 0 ? 0 : s_scan[e - 1]) + s_tab[(r >> 6) * E + e] + s_rank[r];
    sorted_routes[pos] = r;
    inv_pos[r] = pos;
  }
}

hipError_t launch_route_small(const Layer& L, const void* logits, const void* x, int64_t T, char* ws,
                              const Workspace& W, hipStream_t s, const uint16_t** xa,
                              const int8_t** xexp) {
  const int E = static_cast<int>(L.E), k = L.k, H = static_cast<int>(L.H);
  const int P = operand_perm(L.bits);
  const bool stage = x != nullptr && (L.act != kActF16 || P != 0);
  uint16_t* x16 = stage ? reinterpret_cast<uint16_t*>(ws + W.x16) : nullptr;
  int8_t* xe = L.act != kActF16 ? reinterpret_cast<int8_t*>(ws + W.xexp) : nullptr;
  if (xa) *xa = stage ? x16 : static_cast<const uint16_t*>(x);
  if (xexp) *xexp = stage ? xe : nullptr;
  const unsigned grid = 1 + (stage ? static_cast<unsigned>((T + 15) / 16) : 0u);
  int32_t* topk_id = reinterpret_cast<int32_t*>(ws + W.topk_id);
  float* topk_w = reinterpret_cast<float*>(ws + W.topk_w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + W.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + W.offsets);
  int32_t* srt = reinterpret_cast<int32_t*>(ws + W.sorted_routes);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + W.inv_pos);
  int4* tiles = reinterpret_cast<int4*>(ws + W.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(ws + W.num_tiles);
  auto go = [&](auto slots, auto lgt, auto actc, auto pc) {
    constexpr int SL = decltype(slots)::value, AC = decltype(actc)::value, PP = decltype(pc)::value;
    using LT = typename decltype(lgt)::type;
    route_small_kernel<SL, LT, AC, PP><<<grid, 1024, 0, s>>>(
        static_cast<const LT*>(logits), T, E, k, L.normalize, W.tile_m, topk_id, topk_w, counts, offsets,
        srt, inv, tiles, ntiles, x, H, x16, xe);
  };
  auto with_perm = [&](auto slots, auto lgt, auto actc) {
    if (P == 8)
      go(slots, lgt, actc, std::integral_constant<int, 8>{});
    else if (P == 16)
      go(slots, lgt, actc, std::integral_constant<int, 16>{});
    else
      go(slots, lgt, actc, std::integral_constant<int, 0>{});
  };
  using I0 = std::integral_constant<int, 0>;
  if (L.act_bf16) {
    using A = std::integral_constant<int, kActBF16>;
    struct U16 { using type = uint16_t; };
    if (E <= 64) with_perm(std::integral_constant<int, 1>{}, U16{}, A{});
    else if (E <= 128) with_perm(std::integral_constant<int, 2>{}, U16{}, A{});
    else if (E <= 256) with_perm(std::integral_constant<int, 4>{}, U16{}, A{});
    else if (E <= 512) with_perm(std::integral_constant<int, 8>{}, U16{}, A{});
    else with_perm(std::integral_constant<int, 16>{}, U16{}, A{});
  } else if (L.act == kActF16) {
    struct F16 { using type = _Float16; };
    with_perm(I0{}, F16{}, std::integral_constant<int, kActF16>{});
  } else {
    struct F32 { using type = float; };
    with_perm(I0{}, F32{}, std::integral_constant<int, kActF32>{});
  }
  stage_done(L, 1, "route_small");
  return hipGetLastError();
}

hipError_t launch_route(const Layer& L, const void* logits, int64_t T, char* ws, const Workspace& W,
                        hipStream_t s) {
  const int E = static_cast<int>(L.E), k = L.k;
  int32_t* topk_id = reinterpret_cast<int32_t*>(ws + W.topk_id);
  float* topk_w = reinterpret_cast<float*>(ws + W.topk_w);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + W.hist);
  const unsigned nc = static_cast<unsigned>(W.nchunks);
  if (L.act_bf16) {
    const uint16_t* lg = static_cast<const uint16_t*>(logits);
    if (E <= 64)
      route_topk_hist_bf16_kernel<1><<<nc, 512, 0, s>>>(lg, T, E, k, L.normalize, topk_id, topk_w, hist);
    else if (E <= 128)
      route_topk_hist_bf16_kernel<2><<<nc, 512, 0, s>>>(lg, T, E, k, L.normalize, topk_id, topk_w, hist);
    else if (E <= 256)
      route_topk_hist_bf16_kernel<4><<<nc, 512, 0, s>>>(lg, T, E, k, L.normalize, topk_id, topk_w, hist);
    else if (E <= 512)
      route_topk_hist_bf16_kernel<8><<<nc, 512, 0, s>>>(lg, T, E, k, L.normalize, topk_id, topk_w, hist);
    else
      route_topk_hist_bf16_kernel<16><<<nc, 512, 0, s>>>(lg, T, E, k, L.normalize, topk_id, topk_w, hist);
  } else if (L.act == kActF16) {
    route_topk_hist_wide_kernel<_Float16><<<nc, 512, 0, s>>>(static_cast<const _Float16*>(logits), T,
                                                              E, k, L.normalize, topk_id, topk_w, hist);
  } else {
    route_topk_hist_wide_kernel<float><<<nc, 512, 0, s>>>(static_cast<const float*>(logits), T, E, k,
                                                           L.normalize, topk_id, topk_w, hist);
  }
  stage_done(L, 1, "route_topk_hist");
  route_scan_kernel<<<1, 1024, 0, s>>>(hist, W.nchunks, E, W.tile_m,
                                       reinterpret_cast<int32_t*>(ws + W.counts),
                                       reinterpret_cast<int32_t*>(ws + W.offsets),
                                       reinterpret_cast<int32_t*>(ws + W.chunk_base),
                                       reinterpret_cast<int4*>(ws + W.tiles),
                                       reinterpret_cast<int32_t*>(ws + W.num_tiles));
  stage_done(L, 3, "route_scan");
  route_scatter_kernel<<<nc, 256, 0, s>>>(topk_id, W.R, k, E,
                                          reinterpret_cast<const int32_t*>(ws + W.chunk_base),
                                          reinterpret_cast<int32_t*>(ws + W.sorted_routes),
                                          reinterpret_cast<int32_t*>(ws + W.inv_pos));
  stage_done(L, 4, "route_scatter");
  return hipGetLastError();
}

}  // namespace qmoe
