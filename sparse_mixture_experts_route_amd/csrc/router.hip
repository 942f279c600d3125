// Router kernel: fp32 logits, scores, selection key, wavefront top-k,
// weight normalisation, shared-expert gate.
//
// Follows the router contract of "mstar.model.components.moe" (Router
// contract; TopKRouter: softmax top-k router, norm_topk_prob) and the MoEGate
// of "Sparse MoE FFN for DFlash-family drafters" (What's here: sqrtsoftplus
// scores, fp32 aux-loss-free balancing bias used for selection).
//
// One workgroup (4 waves) routes a tile of TM tokens:
//   1. logits tile [TM x (E + gate)] = x_tile . [w_router; w_shared_gate]^T.
//      bf16 with H % 64 == 0 (route_dma_kernel): x rows and router rows
//      stream through an LDS ring by global_load_lds, v_mfma_f32_16x16x32_bf16
//      on fragments read from it (16 tokens per tile up to 144 columns, 32
//      beyond).  Other bf16 H (route_kernel): the H loop split across the
//      four waves (interleaved 64-wide k chunks read as whole 128-byte lines
//      into registers), partials summed in LDS in the fixed order
//      w0 + w1 + w2 + w3.  fp32: plain FMA loops, 32 tokens per tile.
//   2. each wave selects for its tokens: lane L holds experts L, L+64,
//      L+128, L+192; k rounds of a wave-wide (key desc, index asc) arg-max,
//      the maximum found with DPP row reductions and four lane reads.  Up
//      to 64 experts (one a lane), four tokens go at once, their chains of
//      reductions interleaved.
// This file is compiled with -ffp-contract=off (the score recipe needs it).
#include <algorithm>
#include <cstring>

#include "common.h"
#include "kernels.h"
#include "score32.h"

namespace moe {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kMaxCols = 272;  // 256 experts + gate column, padded to 16
constexpr int kMaxPairs = 32 * 8;  // (token, slot) pairs of one route tile: 32 tokens, top-8

struct RouteArgs {
  const void* x;
  const void* w_router;
  const void* w_gate;  // shared gate weight [H] or null
  const float* bias;   // [E] or null
  float* logits;       // [T,E] out (or in with logits_in) or null
  float* weights;      // [T,k]
  int64_t* ids;        // [T,k]
  float* gate;         // [T] or null
  float* score_part;   // [gridDim.x, E] per-tile column sums of the scores, or null
  int32_t* tile_counts;  // [gridDim.x, E] per-tile expert loads (selections per expert), or null
  float* kpart;        // partial logits of a split reduction: split s, token t, column c at
                       // kpart[s kstride + t kld + c] (c below the tile's 16-padded columns), or null
  int32_t *d_counts, *d_offsets, *d_perm, *d_pos;  // the counting sort of a one-tile batch, or null
  int64_t kstride;     // floats from one split's partials to the next
  int kld;             // floats from one token's partial row to the next
  int T, H, E, k, score, renorm, logits_in;
  int ksplit;          // partial sums per logit (1: none)
};

// Wave-wide maximum of an unsigned value, in every lane: DPP within each row
// of 16 lanes (quad xor 1, quad xor 2, half-row mirror, row mirror), then the
// four row results read into scalars.  The whole wave must be active.
MOE_DEV uint32_t dpp_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Sortable image of a float key: larger key -> larger unsigned value.
MOE_DEV uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 and +0 are one key
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Selection for one token whose logits row (E values, then the gate logit)
// sits in LDS at `row`.  Called by a whole wave.  ssum[r] accumulates the
// token's unbiased fp32 score of expert lane + 64 r (zero past E).
MOE_DEV void select_token(const RouteArgs& a, const float* row, int t, float (&ssum)[4], int* hist,
                          int* ids_lds = nullptr) {
  const int lane = threadIdx.x & 63;
  const int E = a.E;
  float lg[4], s[4];
  uint32_t ok[4];
  bool valid[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane + 64 * r;
    valid[r] = e < E;
    lg[r] = valid[r] ? row[e] : 0.0f;
  }
  if (a.score == 0) {
    float m = -__int_as_float(0x7f800000);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (valid[r]) m = fmaxf(m, lg[r]);
    m = wave_max(m);
    float v[4];
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = (64 * r < E && valid[r]) ? score32::exp32(lg[r] - m) : 0.0f;
      part = part + v[r];
    }
    // fixed xor-butterfly over the lanes; every lane ends with the same bits
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) part = part + shfl_xor_f(part, d);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = v[r] / part;
  } else if (a.score == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = 64 * r < E ? score32::sigmoid32(lg[r]) : 0.0f;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = 64 * r < E ? score32::sqrtsoftplus32(lg[r]) : 0.0f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) ssum[r] += valid[r] ? s[r] : 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float key = lg[r];
    if (a.bias) key = s[r] + (valid[r] ? a.bias[lane + 64 * r] : 0.0f);
    ok[r] = valid[r] ? order_key(key) : 0u;  // 0: below every real key
  }
  int my_id = 0;
  float my_w = 0.0f;
  for (int j = 0; j < a.k; ++j) {
    // local best: largest key, then lowest expert index (r ascending)
    uint32_t bk = 0u, bi = 0u;
    float bs = 0.0f;
    int br = -1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t idx = 0xffffffffu - (uint32_t)(lane + 64 * r);
      if (ok[r] > bk || (ok[r] == bk && ok[r] != 0u && idx > bi)) {
        bk = ok[r];
        bi = idx;
        bs = s[r];
        br = r;
      }
    }
    // winner: the largest key; among lanes holding it, the lowest expert
    // index (largest bi).  One lane holds the maximum unless keys tie.
    const uint32_t wk = dpp_max_u32(bk);
    const unsigned long long cand = __ballot(bk == wk);
    uint32_t wi;
    if (__popcll(cand) == 1) {
      wi = (uint32_t)__builtin_amdgcn_readlane((int)bi, (int)(__ffsll((long long)cand) - 1));
    } else {
      wi = dpp_max_u32(bk == wk ? bi : 0u);
    }
    const int e_win = (int)(0xffffffffu - wi);
    const int owner = e_win & 63;
    const float w_win = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bs), owner));
    if (lane == owner) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r == br) ok[r] = 0u;  // taken
    }
    if (lane == j) {
      my_id = e_win;
      my_w = w_win;
    }
  }
  if (a.renorm) {
    float sum = 0.0f;
    for (int j = 0; j < a.k; ++j) sum = sum + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
    my_w = sum > 0.0f ? my_w / sum : 0.0f;
  }
  if (lane < a.k) {
    a.ids[(int64_t)t * a.k + lane] = (int64_t)my_id;
    a.weights[(int64_t)t * a.k + lane] = my_w;
    if (hist) atomicAdd(&hist[my_id], 1);  // the tile's expert loads (integer: order-free)
    if (ids_lds) ids_lds[t * a.k + lane] = my_id;
  }
  if (a.logits && !a.logits_in) {
    for (int e = lane; e < E; e += 64) a.logits[(int64_t)t * E + e] = row[e];
  }
  if (a.gate && lane == 0) a.gate[t] = score32::sigmoid32(row[E]);
}

// Selection for up to four tokens at once when E <= 64 (lane = expert):
// token q < nq has its logits row at rows[q] (LDS) and index t[q].  Each
// token takes the same operations in the same order as in select_token, so
// the results are the same bits, and ssum (expert lane's score sum) adds the
// tokens in the order q = 0, 1, ...; the four tokens' chains of wave
// reductions are independent and interleave, where select_token waits out
// one chain at a time.  A round whose remaining keys are all 0 (NaN logits)
// gives expert -1 at weight 0, as select_token does.
MOE_DEV void select_narrow4(const RouteArgs& a, const float* const (&rows)[4], const int (&t)[4], int nq,
                            float& ssum, int* hist, int* ids_lds) {
  const int lane = threadIdx.x & 63;
  const int E = a.E;
  const bool valid = lane < E;
  float lg[4], s[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) lg[q] = (q < nq && valid) ? rows[q][lane] : 0.0f;
  if (a.score == 0) {
    float m[4], v[4], part[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = valid ? lg[q] : -__int_as_float(0x7f800000);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
#pragma unroll
      for (int q = 0; q < 4; ++q) m[q] = fmaxf(m[q], shfl_xor_f(m[q], d));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = valid ? score32::exp32(lg[q] - m[q]) : 0.0f;
      part[q] = 0.0f + v[q];
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
#pragma unroll
      for (int q = 0; q < 4; ++q) part[q] = part[q] + shfl_xor_f(part[q], d);
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] = v[q] / part[q];
  } else if (a.score == 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] = score32::sigmoid32(lg[q]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] = score32::sqrtsoftplus32(lg[q]);
  }
  const float b = (a.bias && valid) ? a.bias[lane] : 0.0f;
  uint32_t key[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < nq) ssum += valid ? s[q] : 0.0f;
    key[q] = valid ? order_key(a.bias ? s[q] + b : lg[q]) : 0u;
  }
  int id[4] = {0, 0, 0, 0};
  float w[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < a.k; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wk = dpp_max_u32(key[q]);
      const int first = (int)__ffsll((long long)__ballot(key[q] == wk)) - 1;
      const float w_win = wk ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s[q]), first)) : 0.0f;
      if (lane == first) key[q] = 0u;  // taken
      if (lane == j) {
        id[q] = wk ? first : -1;
        w[q] = w_win;
      }
    }
  }
  if (a.renorm) {
    float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < a.k; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) sum[q] = sum[q] + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[q]), j));
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = sum[q] > 0.0f ? w[q] / sum[q] : 0.0f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q >= nq) break;
    if (lane < a.k) {
      a.ids[(int64_t)t[q] * a.k + lane] = (int64_t)id[q];
      a.weights[(int64_t)t[q] * a.k + lane] = w[q];
      if (hist) atomicAdd(&hist[id[q]], 1);
      if (ids_lds) ids_lds[t[q] * a.k + lane] = id[q];
    }
    if (a.logits && !a.logits_in && valid) a.logits[(int64_t)t[q] * E + lane] = lg[q];
    if (a.gate && lane == 0) a.gate[t[q]] = score32::sigmoid32(rows[q][E]);
  }
}

// The selections of a wave's tokens m = m0, m0 + step, ... (m < TM, t0 + m
// < T) in that order: four at a time when E <= 64 and a wave has several,
// else one at a time.  ids_lds (or null): a copy of the ids at [t k + j]
// (a one-tile batch's, for its sort).
MOE_DEV void select_tokens(const RouteArgs& a, const float* tile, int ld, int TM, int t0, int m0, int step,
                           float (&ssum)[4], int* hist, int* ids_lds = nullptr) {
  if (a.E <= 64 && step < TM) {
    for (int m = m0; m < TM && t0 + m < a.T; m += 4 * step) {
      const float* rows[4];
      int t[4], nq = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int mq = m + q * step;
        rows[q] = tile + (int64_t)mq * ld;
        t[q] = t0 + mq;
        if (mq < TM && t0 + mq < a.T) nq = q + 1;
      }
      select_narrow4(a, rows, t, nq, ssum[0], hist, ids_lds);
    }
    return;
  }
  for (int m = m0; m < TM; m += step) {
    const int t = t0 + m;
    if (t < a.T) select_token(a, tile + m * ld, t, ssum, hist, ids_lds);
  }
}

// Logits of a 16 * MB-token tile with bf16 MFMA.  Output row-major in LDS:
// tile[m * ld + col], col < ncols (E, then the gate column).
template <int NB, int MB>
MOE_DEV void logits_tile_bf16(const RouteArgs& a, int t0, int ncols, float* tile, int ld) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const bf16_t* x = (const bf16_t*)a.x;
  const bf16_t* wr = (const bf16_t*)a.w_router;
  const bf16_t* wg = (const bf16_t*)a.w_gate;
  const int nb_used = (ncols + 15) >> 4;
  constexpr int U = NB > 8 ? 1 : 2;  // 64-wide chunks whose loads are in flight together
  f32x4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Each wave takes 64-wide K chunks c = wave, wave + 4, ...; lane (lr, lq)
  // loads 16 consecutive k of its row at 16 lq (so a row's four lanes read
  // one whole 128-byte line) and feeds the first 8 to MFMA substep 0 and the
  // last 8 to substep 1.  Both operands use the same order of k, so each
  // substep still sums matching products.
  const int lr = lane & 15;         // row inside a 16-block
  const int lk = (lane >> 4) * 16;  // first of 16 k values held by this lane
  const bf16_t* xrow[MB];
  bool xok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t = t0 + mb * 16 + lr;
    xok[mb] = t < a.T;
    xrow[mb] = x + (int64_t)(xok[mb] ? t : 0) * a.H;
  }
  const bf16_t* wrow[NB];
  bool wok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + lr;
    if (n < a.E) {
      wrow[nb] = wr + (int64_t)n * a.H;
      wok[nb] = true;
    } else if (n == a.E && wg) {
      wrow[nb] = wg;
      wok[nb] = true;
    } else {
      wrow[nb] = wr;
      wok[nb] = false;
    }
  }
  const int nchunks = (a.H + 63) >> 6;
  for (int c0 = wave; c0 < nchunks; c0 += 4 * U) {
    u32x4_t xv[U][MB][2], wv[U][NB][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = (c0 + 4 * u) * 64 + lk;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool kok = kk + 8 * h < a.H;  // H % 8 == 0: 8 values are all in or all out
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          xv[u][mb][h] = u32x4_t{0u, 0u, 0u, 0u};
          if (xok[mb] && kok) xv[u][mb][h] = *(const u32x4_t*)(xrow[mb] + kk + 8 * h);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          wv[u][nb][h] = u32x4_t{0u, 0u, 0u, 0u};
          if (nb < nb_used && wok[nb] && kok) wv[u][nb][h] = *(const u32x4_t*)(wrow[nb] + kk + 8 * h);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if (nb < nb_used) {
            const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, wv[u][nb][h]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv[u][mb][h]), bfr,
                                                                    acc[mb][nb], 0, 0, 0);
          }
        }
  }
  // Sum the four wave partials in LDS in the order w0, w1, w2, w3.
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if (nb < nb_used) {
            const int col = nb * 16 + lr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = mb * 16 + (lane >> 4) * 4 + i;
              float* p = tile + m * ld + col;
              *p = (w == 0) ? acc[mb][nb][i] : (*p + acc[mb][nb][i]);
            }
          }
        }
    }
    __syncthreads();
  }
}

template <typename T, int TM>
MOE_DEV void logits_tile_simt(const RouteArgs& a, int t0, int ncols, float* tile, int ld) {
  const T* x = (const T*)a.x;
  const T* wr = (const T*)a.w_router;
  const T* wg = (const T*)a.w_gate;
  for (int p = threadIdx.x; p < TM * ncols; p += kThreads) {
    const int m = p / ncols, col = p % ncols;
    const int t = t0 + m;
    float acc = 0.0f;
    if (t < a.T) {
      const T* xr = x + (int64_t)t * a.H;
      const T* wrow = col < a.E ? wr + (int64_t)col * a.H : wg;
      for (int h = 0; h < a.H; ++h) acc += Elem<T>::load(xr + h) * Elem<T>::load(wrow + h);
    }
    tile[m * ld + col] = acc;
  }
  __syncthreads();
}

// Writes this tile's expert loads (hist, in LDS) to tile_counts; called by
// the whole workgroup after its selections.
MOE_DEV void write_tile_counts(const RouteArgs& a, const int* hist) {
  if (!a.tile_counts) return;
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.tile_counts[(int64_t)blockIdx.x * a.E + e] = hist[e];
}

template <typename T, int NB, int TM>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  __shared__ float tile[TM * kMaxCols];
  __shared__ int hist[256];
  hist[threadIdx.x] = 0;  // 256 threads; ordered before the selections by the barriers below
  const int t0 = blockIdx.x * TM;
  const int ncols = a.E + (a.w_gate ? 1 : 0);
  const int ld = kMaxCols;
  if (a.logits_in) {
    for (int p = threadIdx.x; p < TM * a.E; p += kThreads) {
      const int m = p / a.E, e = p % a.E;
      const int t = t0 + m;
      tile[m * ld + e] = t < a.T ? a.logits[(int64_t)t * a.E + e] : 0.0f;
    }
    __syncthreads();
  } else if constexpr (sizeof(T) == 2 && NB > 0) {
    logits_tile_bf16<NB, TM / 16>(a, t0, ncols, tile, ld);
  } else {
    logits_tile_simt<T, TM>(a, t0, ncols, tile, ld);
  }
  const int wave = threadIdx.x >> 6;
  float ssum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  select_tokens(a, tile, ld, TM, t0, wave, 4, ssum, a.tile_counts ? hist : nullptr);
  write_tile_counts(a, hist);
  if (a.score_part) {
    // this tile's score column sums: wave partials (tokens wave, wave + 4,
    // ... in increasing order) added in the order w0 + w1 + w2 + w3
    const int lane = threadIdx.x & 63;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) tile[wave * 256 + lane + 64 * r] = ssum[r];
    __syncthreads();
    for (int e = threadIdx.x; e < a.E; e += kThreads)
      a.score_part[(int64_t)blockIdx.x * a.E + e] = ((tile[e] + tile[256 + e]) + tile[512 + e]) + tile[768 + e];
  }
}

// score_sums[e] = sum over route tiles of score_part[b][e]: wave w of a
// 1024-thread workgroup adds tiles w, w + 16, ... in fp64, and the sixteen
// wave sums are added in the order w0 + w1 + ... + w15.  Workgroup g covers
// experts 64 g .. 64 g + 63.
__global__ __launch_bounds__(1024) void score_sum_kernel(const float* part, int nb, int E, float* sums) {
  __shared__ double red[16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  double acc = 0.0;
  if (e < E)
    for (int b = wave; b < nb; b += 16) acc += (double)part[(int64_t)b * E + e];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && e < E) {
    double tot = red[0][lane];
    for (int w = 1; w < 16; ++w) tot += red[w][lane];
    sums[e] = (float)tot;
  }
}

// Switch-style aux loss from the score column sums and the expert loads:
// coef[e] = alpha * E * counts[e] / (T * k * T) is d loss / d score[t,e] for
// every token; loss = sum_e coef[e] * sums[e] (fp64, fixed tree order).
__global__ __launch_bounds__(256) void aux_loss_kernel(const float* sums, const int32_t* counts, int E, double scale,
                                                       float* loss, float* coef) {
  __shared__ double red[256];
  const int e = threadIdx.x;
  double term = 0.0;
  if (e < E) {
    const double c = scale * (double)counts[e];
    if (coef) coef[e] = (float)c;
    term = c * (double)sums[e];
  }
  red[e] = term;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (e < w) red[e] = red[e] + red[e + w];
    __syncthreads();
  }
  if (e == 0 && loss) loss[0] = (float)red[0];
}

// bf16 router with H % 64 == 0: the logits of a TM-token tile stream
// through an LDS ring of 64-wide K chunks.  A chunk holds the tile's TM x
// rows and the 16 NB router rows (w_router, then the shared-gate row, then
// clamped filler rows whose results are never read), each row segment one
// whole 128-byte line brought in by global_load_lds_dwordx4 (no register
// staging), with the eight 16-byte pieces of row r stored at position
// piece ^ (r & 7) so the fragment reads of 16 rows spread over the banks.
// One barrier per chunk: wait for this wave's DMA of chunk c, barrier (every
// wave's DMA of c landed and chunk c - 1 consumed), refill the slot of c - 1
// with chunk c + S - 1 (past the end: a re-read of the last chunk into a slot
// nobody reads again, so the wait count stays constant), then the MFMAs of c.
// The four waves split the (token block, expert block) pairs of the tile.
// Short token counts leave most CUs idle with one workgroup per tile, and
// each workgroup's chunk loop is bound by memory latency: below kSplitTiles
// tiles the reduction over H is split over up to kSplitWgs / tiles
// workgroups (each at least two 64-wide chunks).
constexpr int kSplitTiles = 64, kSplitWgs = 128;
int route_ksplit(int64_t T, int64_t H, int tm) {
  const int64_t tiles = (T + tm - 1) / tm, nk = H / 64;
  if (tiles >= kSplitTiles) return 1;
  const int64_t ks = std::min<int64_t>(nk / 2, kSplitWgs / tiles);
  return ks >= 2 ? (int)ks : 1;
}

template <int NB, int TM, int SMAX>
struct RouteDma {
  static constexpr int MB = TM / 16;
  static constexpr int IW = (TM + 16 * NB + 31) / 32;   // DMA instructions per wave per chunk
  static constexpr int CHUNK = IW * 4 * 1024;             // bytes per ring slot
  static constexpr int S0 = (160 * 1024 - TM * 16 * NB * 4) / CHUNK;
  static constexpr int S = S0 < SMAX ? S0 : SMAX;          // ring slots
  static constexpr int TILE = TM * 16 * NB * 4;           // logits tile (fp32) before the ring
  static constexpr int LDS = TILE + S * CHUNK;
  static_assert(S >= 3, "ring depth");
  static_assert((S - 2) * IW < 64, "vmcnt range");
};

MOE_DEV void route_finish(const RouteArgs& a, float* tile, int TM, int ld, int t0);

template <int NB, int TM, int SMAX>
__global__ __launch_bounds__(kThreads) void route_dma_kernel(RouteArgs a) {
  using C = RouteDma<NB, TM, SMAX>;
  constexpr int MB = C::MB;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* tile = (float*)smem;
  char* ring = smem + C::TILE;
  constexpr int ld = 16 * NB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * TM;
  const int ncols = a.E + (a.w_gate ? 1 : 0);
  const int nb_used = (ncols + 15) >> 4;
  const bf16_t* x = (const bf16_t*)a.x;
  const bf16_t* wr = (const bf16_t*)a.w_router;
  const bf16_t* wg = (const bf16_t*)a.w_gate;

  // this lane's DMA source rows (byte pointers at k = 0, logical piece applied)
  const char* src[C::IW];
#pragma unroll
  for (int i = 0; i < C::IW; ++i) {
    const int rr = (wave * C::IW + i) * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ (rr & 7);
    const bf16_t* row;
    if (rr < TM) {
      row = x + (int64_t)min(t0 + rr, a.T - 1) * a.H;
    } else {
      const int e = rr - TM;
      row = e < a.E ? wr + (int64_t)e * a.H : ((e == a.E && wg) ? wg : wr);
    }
    src[i] = (const char*)(row + piece * 8);
  }
  // 64-wide chunks [c0, c0 + nk) of H: all of them, or this workgroup's
  // share of a reduction split over blockIdx.y
  const int nk_all = a.H >> 6;
  const int c0 = (int)((int64_t)blockIdx.y * nk_all / a.ksplit);
  const int nk = (int)((int64_t)(blockIdx.y + 1) * nk_all / a.ksplit) - c0;
  int issued = 0;
  auto issue = [&]() {
    const int c = c0 + min(issued, nk - 1);
    char* dst = ring + (issued % C::S) * C::CHUNK + wave * (C::IW * 1024);
#pragma unroll
    for (int i = 0; i < C::IW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + (int64_t)c * 128),
                                       (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
    ++issued;
  };

  // (token block, expert block) pairs of this wave
  constexpr int NP = (MB * NB + 3) / 4;
  f32x4_t acc[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int lr = lane & 15, lg = lane >> 4;

#pragma unroll
  for (int c = 0; c < C::S - 1; ++c) issue();
  for (int c = 0; c < nk; ++c) {
    wait_vmcnt<(C::S - 2) * C::IW>();
    ring_barrier();
    issue();
    const char* slot = ring + (c % C::S) * C::CHUNK;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int pr = wave + 4 * q;
      const int mb = pr % MB, nb = pr / MB;
      if (pr < MB * NB && nb < nb_used) {
        const int ra = mb * 16 + lr, rb = TM + nb * 16 + lr;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int piece = 4 * h + lg;
          const bf16x8_t fa = *(const bf16x8_t*)(slot + ra * 128 + ((piece ^ (ra & 7)) << 4));
          const bf16x8_t fb = *(const bf16x8_t*)(slot + rb * 128 + ((piece ^ (rb & 7)) << 4));
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc[q], 0, 0, 0);
        }
      }
    }
  }
  wait_vmcnt<0>();
  // split reduction: the partial tile goes to scratch and route_select_kernel
  // adds the splits; otherwise it goes to LDS for the selection below
  float* out = a.kpart ? a.kpart + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * (TM * ld) : tile;
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int pr = wave + 4 * q;
    const int mb = pr % MB, nb = pr / MB;
    if (pr < MB * NB && nb < nb_used) {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[(mb * 16 + lg * 4 + i) * ld + nb * 16 + lr] = acc[q][i];
    }
  }
  if (a.kpart) return;
  __syncthreads();
  route_finish(a, tile, TM, ld, t0);
}

// Selection of a tile of TM tokens whose logits rows (stride ld) are in LDS
// at `tile` (at least 1 KB per wave): wave w selects tokens w, w + NW, ...
// (the selection of one token is a chain of dependent wave reductions, so
// tokens spread over as many waves as the workgroup has), then this tile's
// score column sums when they are asked for, added over the waves in order.
// Called by the whole workgroup.
// The counting sort of a batch that is this workgroup's one tile (called by
// the whole workgroup after its selections, hist holding the batch's expert
// loads and sid its ids at [t k + j], in LDS): counts, offsets (exclusive
// scan of the loads), and for every pair
// i = t k + j its position offsets[e] + #{i' < i : ids[i'] == e}, stable in
// i as moe_dispatch's.
MOE_DEV void tile_dispatch(const RouteArgs& a, const int* hist, const int* sid) {
  __shared__ int off[257];
  __syncthreads();  // every selection's ids in sid
  const int P = a.T * a.k;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int c[4], local = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane * 4 + r;
      c[r] = e < a.E ? hist[e] : 0;
      local += c[r];
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    int run = incl - local;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane * 4 + r;
      if (e < a.E) {
        off[e] = run;
        a.d_counts[e] = c[r];
        a.d_offsets[e] = run;
      }
      run += c[r];
    }
    if (lane == 63) a.d_offsets[a.E] = incl;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    const int e = sid[i];
    int rank = 0;
    for (int j = 0; j < i; ++j) rank += (sid[j] == e) ? 1 : 0;
    const int ps = off[e] + rank;
    a.d_pos[i] = ps;
    a.d_perm[ps] = i;
  }
}

MOE_DEV void route_finish(const RouteArgs& a, float* tile, int TM, int ld, int t0) {
  __shared__ int hist[256];
  __shared__ int sid[kMaxPairs];  // the ids of a one-tile batch, for its sort
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  if (a.tile_counts) {
    for (int e = threadIdx.x; e < 256; e += blockDim.x) hist[e] = 0;
    __syncthreads();
  }
  float ssum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  select_tokens(a, tile, ld, TM, t0, wave, nw, ssum, a.tile_counts ? hist : nullptr, a.d_counts ? sid : nullptr);
  write_tile_counts(a, hist);
  if (a.d_counts) tile_dispatch(a, hist, sid);
  if (a.score_part) {
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) tile[wave * 256 + lane + 64 * r] = ssum[r];
    __syncthreads();
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
      float v = tile[e];
      for (int w = 1; w < nw; ++w) v = v + tile[w * 256 + e];
      a.score_part[(int64_t)blockIdx.x * a.E + e] = v;
    }
  }
}

// Second half of a split reduction: tile blockIdx.x's logits are the sum of
// its ksplit partial tiles taken in split order (fixed, so two calls give
// identical bits), then the selection of route_finish by 16 waves.
constexpr int kSelectThreads = 1024;
template <int NB, int TM>
__global__ __launch_bounds__(kSelectThreads) void route_select_kernel(RouteArgs a) {
  constexpr int ld = 16 * NB;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* tile = (float*)smem;
  const int cols = ((a.E + (a.w_gate ? 1 : 0) + 15) >> 4) << 4;  // columns the partials hold
  const int64_t stride = a.kstride;
  const float* part = a.kpart + (int64_t)blockIdx.x * TM * a.kld;
  // four columns per thread (ld, kld and cols are multiples of 16); the
  // loads of eight splits are issued together, then added in split order;
  // the rows of the last tile past T are read (inside the buffer) and not used
  for (int i = 4 * threadIdx.x; i < TM * ld; i += 4 * kSelectThreads) {
    const int m = i / ld, c = i % ld;
    if (c >= cols) continue;
    const int64_t o = (int64_t)m * a.kld + c;
    f32x4_t v = *(const f32x4_t*)(part + o);
    for (int s = 1; s < a.ksplit; s += 8) {
      f32x4_t t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s + j < a.ksplit) t[j] = *(const f32x4_t*)(part + (s + j) * stride + o);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s + j < a.ksplit) v += t[j];
    }
    *(f32x4_t*)(tile + i) = v;
  }
  __syncthreads();
  route_finish(a, tile, TM, ld, blockIdx.x * TM);
}

__global__ __launch_bounds__(256) void score_kernel(int score, const float* l, float* s, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = l[i];
    s[i] = score == 1 ? score32::sigmoid32(v) : (score == 2 ? score32::sqrtsoftplus32(v) : score32::exp32(v));
  }
}

// Router rows for the GEMM form: out[r] = w_router row r (r < E), the shared
// gate row (r == E, when given), else w_router row E - 1 (filler columns whose
// logits are never read); 16 bytes a thread.
__global__ __launch_bounds__(256) void router_rows_kernel(const bf16_t* wr, const bf16_t* wg, bf16_t* out, int E,
                                                          int H, int N) {
  const int64_t per = H / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)N * per) return;
  const int r = (int)(i / per);
  const int64_t c = i % per;
  const bf16_t* src = r < E ? wr + (int64_t)r * H : ((r == E && wg) ? wg : wr + (int64_t)(E - 1) * H);
  ((u32x4_t*)(out + (int64_t)r * H))[c] = ((const u32x4_t*)src)[c];
}

}  // namespace

// Prefill-sized bf16 batches take the logits as a GEMM on the 256x256 engine:
// x [T, H] times the router rows [N, H] (N = the columns, E and the gate,
// padded to 16), the reduction over H split over enough workgroup sets to
// give one 256x256 tile to each of 256 CUs, the fp32 partials [splits][T][N]
// left in the workspace; route_select_kernel adds them in split order and
// selects.  The router rows are read in place when they are exactly the N
// rows (no gate, E % 16 == 0), else copied with the gate row and filler rows
// into the workspace first.  Smaller batches take route_dma_kernel.
constexpr int64_t kGemmRouteMinT = 2048;
constexpr int kGemmRouteMaxSplits = 8;

int64_t gemm_route_cols(int64_t ncols) { return (ncols + 15) / 16 * 16; }

int gemm_route_splits(int64_t T, int64_t H, int64_t N) {
  const int64_t tiles = ((T + 255) / 256) * ((N + 255) / 256);
  int64_t sp = 256 / tiles;
  sp = std::min<int64_t>(sp, kGemmRouteMaxSplits);
  sp = std::min<int64_t>(sp, H / 64 / 8);
  return (int)std::max<int64_t>(sp, 1);
}

// Measured (DSV4-Flash shape, 64 columns: 32 -> 36 us; Qwen2-MoE, 61: 20 -> 26
// us; DeepSeek-V3, 256 columns: 334 -> 109 us): below 256 columns the tile
// computes columns nobody reads, and route_dma_kernel's re-reads of the
// router rows are still cheap; the GEMM form is taken above 80 columns.
constexpr int64_t kGemmRouteMinCols = 81;
bool gemm_route_fits(int64_t T, int64_t H, int64_t ncols) {
  return T >= kGemmRouteMinT && ncols >= kGemmRouteMinCols && T * H * 2 < (1LL << 32);
}

// workspace of the GEMM form: router rows (N x H bf16, 256-byte aligned),
// then the partials with room for the last selection tile's rows past T
size_t gemm_route_ws_bytes(int64_t T, int64_t H, int64_t N, int splits) {
  const size_t rows = (size_t)((N * H * 2 + 255) / 256 * 256);
  return rows + (size_t)splits * T * N * 4 + (size_t)32 * N * 4;
}

template <int NB, int TM>
int launch_route_gemm(RouteArgs a, int64_t N, void* ws, hipStream_t stream) {
  const int ncols = a.E + (a.w_gate ? 1 : 0);
  const int sp = gemm_route_splits(a.T, a.H, N);
  const bf16_t* rows = (const bf16_t*)a.w_router;
  char* w = (char*)ws;
  if (a.w_gate || ncols != N) {
    const int64_t chunks = N * (a.H / 8);
    hipLaunchKernelGGL(router_rows_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                       (const bf16_t*)a.w_router, (const bf16_t*)a.w_gate, (bf16_t*)w, a.E, a.H, (int)N);
    rows = (const bf16_t*)w;
  }
  float* part = (float*)(w + (N * a.H * 2 + 255) / 256 * 256);
  GemmProblem q;
  memset(&q, 0, sizeof(q));
  q.sched = SCHED_GROUP_M;
  q.epi = EPI_STORE_F32;
  q.A = a.x;
  q.lda = a.H;
  q.a_kmajor = 1;
  q.a_div = 1;
  q.B = rows;
  q.ldb = a.H;
  q.b_kmajor = 1;
  q.C = part;
  q.ldc = N;
  q.G = 1;
  q.M = a.T;
  q.N = N;
  q.K = a.H;
  q.split_ws = part;
  q.splits = sp;
  q.partials_only = 1;
  if (gemm_q64_splits(q, 1) != sp) return -2;  // not the 256x256 kernel: the caller's checks failed
  if (launch_gemm(q, 1, stream)) return -4;
  a.kpart = part;
  a.ksplit = sp;
  a.kld = (int)N;
  a.kstride = a.T * N;
  const int tiles = (a.T + TM - 1) / TM;
  using C = RouteDma<NB, TM, 4>;
  constexpr int per_wave = 256 * sizeof(float);  // the score-sum exchange of route_finish
  constexpr int lds = C::TILE > kSelectThreads / 64 * per_wave ? C::TILE : kSelectThreads / 64 * per_wave;
  hipLaunchKernelGGL((route_select_kernel<NB, TM>), dim3((unsigned)tiles), dim3(kSelectThreads), lds, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_score(int score, const float* l, float* s, int64_t n, hipStream_t stream) {
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(score_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, score, l, s, n);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

template <int NB, int TM, int SMAX>
int launch_route_dma(RouteArgs a, void* split_ws, size_t split_bytes, hipStream_t stream) {
  using C = RouteDma<NB, TM, SMAX>;
  auto kern = route_dma_kernel<NB, TM, SMAX>;
  static std::atomic<unsigned long long> lds_set{0};
  if (set_lds_limit((const void*)kern, C::LDS, lds_set)) return -4;
  const int tiles = (a.T + TM - 1) / TM;
  const int ks = route_ksplit(a.T, a.H, TM);
  const size_t need = (size_t)ks * tiles * TM * 16 * NB * sizeof(float);
  a.ksplit = 1;
  a.kpart = nullptr;
  if (ks > 1 && split_ws && split_bytes >= need) {
    a.ksplit = ks;
    a.kpart = (float*)split_ws;
    a.kld = 16 * NB;
    a.kstride = (int64_t)tiles * TM * 16 * NB;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles, (unsigned)a.ksplit), dim3(kThreads), C::LDS, stream, a);
  if (a.ksplit > 1) {
    constexpr int per_wave = 256 * sizeof(float);  // the score-sum exchange of route_finish
    constexpr int lds = C::TILE > kSelectThreads / 64 * per_wave ? C::TILE : kSelectThreads / 64 * per_wave;
    hipLaunchKernelGGL((route_select_kernel<NB, TM>), dim3((unsigned)tiles), dim3(kSelectThreads), lds, stream, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

size_t route_part_bytes(int64_t T, int64_t E, int bf16);

// Tokens per route tile (workgroup) of the kernel launch_route picks.
// Measured at the DSV4 shape (8192 tokens, 64 columns): 32-token tiles (half
// the router-row re-reads, a 10-slot ring, one workgroup a CU) took 50 us
// against 32 us for 16-token tiles: with one workgroup a CU nothing overlaps
// a tile's selection (8 tokens a wave, each a chain of wave reductions).
int route_tile_tokens(int64_t T, int64_t H, int64_t ncols, int bf16, int logits_in) {
  (void)T;
  if (!bf16) return 32;
  if (logits_in || H % 64) return 16;
  return ncols <= 144 ? 16 : 32;
}

int launch_route(const RouteLaunch& p, hipStream_t stream) {
  RouteArgs a;
  a.x = p.x;
  a.w_router = p.w_router;
  a.w_gate = p.w_gate;
  a.bias = p.bias;
  a.logits = p.logits;
  a.weights = p.weights;
  a.ids = p.ids;
  a.gate = p.gate;
  a.T = (int)p.T;
  a.H = (int)p.H;
  a.E = (int)p.E;
  a.k = (int)p.k;
  a.score = p.score;
  a.renorm = p.renorm;
  a.logits_in = p.logits_in;
  a.score_part = p.score_sums ? (float*)p.ws : nullptr;
  a.tile_counts = p.tile_counts;
  a.kpart = nullptr;
  a.ksplit = 1;
  a.kld = 0;
  a.kstride = 0;
  a.d_counts = a.d_offsets = a.d_perm = a.d_pos = nullptr;
  if (p.dispatched) *p.dispatched = 0;
  const int ncols = a.E + (a.w_gate ? 1 : 0);
  // the split partial tiles follow the score partials in ws
  const size_t part_bytes = route_part_bytes(p.T, p.E, p.bf16);
  void* split_ws = (p.ws && p.ws_bytes > part_bytes) ? (char*)p.ws + part_bytes : nullptr;
  const size_t split_bytes = split_ws ? p.ws_bytes - part_bytes : 0;
  const dim3 block(kThreads);
  const int tm = route_tile_tokens(p.T, p.H, ncols, p.bf16, p.logits_in);  // tokens per workgroup
  int st = 0;
  if (p.T == 0) {
    // nothing to route; score_sums (if asked for) become zeros
  } else if (!p.bf16) {
    hipLaunchKernelGGL((route_kernel<float, 0, 32>), dim3((unsigned)((p.T + 31) / 32)), block, 0, stream, a);
  } else if (!p.logits_in && p.H % 64 == 0 && gemm_route_fits(p.T, p.H, ncols) && split_ws &&
             split_bytes >= gemm_route_ws_bytes(p.T, p.H, gemm_route_cols(ncols),
                                                gemm_route_splits(p.T, p.H, gemm_route_cols(ncols)))) {
    const int64_t N = gemm_route_cols(ncols);
    if (ncols <= 144) st = launch_route_gemm<9, 16>(a, N, split_ws, stream);
    else st = launch_route_gemm<17, 32>(a, N, split_ws, stream);
  } else if (!p.logits_in && p.H % 64 == 0) {
    // a batch of one tile (decode): its workgroup also sorts
    if (p.tile_counts && p.d_counts && p.dispatched && p.T <= tm && p.T * p.k <= kMaxPairs) {
      a.d_counts = p.d_counts;
      a.d_offsets = p.d_offsets;
      a.d_perm = p.d_perm;
      a.d_pos = p.d_pos;
      *p.dispatched = 1;
    }
    // 16-token tiles and a 4-slot ring (under 80 KB of LDS, so several
    // workgroups share a CU and one's selection overlaps another's
    // streaming; a 7-slot ring measured 62 against 32 us at the DSV4 shape)
    if (ncols <= 64) st = launch_route_dma<4, 16, 4>(a, split_ws, split_bytes, stream);
    else if (ncols <= 80) st = launch_route_dma<5, 16, 4>(a, split_ws, split_bytes, stream);
    else if (ncols <= 144) st = launch_route_dma<9, 16, 4>(a, split_ws, split_bytes, stream);
    else st = launch_route_dma<17, 32, 8>(a, split_ws, split_bytes, stream);
  } else if (ncols <= 80) {
    hipLaunchKernelGGL((route_kernel<bf16_t, 5, 16>), dim3((unsigned)((p.T + 15) / 16)), block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((route_kernel<bf16_t, 17, 16>), dim3((unsigned)((p.T + 15) / 16)), block, 0, stream, a);
  }
  if (st) return st;
  if (p.score_sums) {
    const int nb = (int)((p.T + tm - 1) / tm);
    hipLaunchKernelGGL(score_sum_kernel, dim3((unsigned)((p.E + 63) / 64)), dim3(1024), 0, stream, (float*)p.ws, nb,
                       (int)p.E, p.score_sums);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int route_tile(int bf16) { return bf16 ? 16 : 32; }

// score partials: one row of E per tile, rounded up to 256 bytes
size_t route_part_bytes(int64_t T, int64_t E, int bf16) {
  const int64_t tm = route_tile(bf16);
  return (size_t)((((T + tm - 1) / tm) * E * 4 + 256 + 255) / 256 * 256);
}

// the score partials, then room for the split partial tiles of the widest
// tile shape E routed columns (plus a gate column) can take
size_t route_ws_bytes(int64_t T, int64_t H, int64_t E, int bf16) {
  size_t split = 0;
  if (bf16 && H % 64 == 0 && gemm_route_fits(T, H, E + 1)) {
    // the GEMM form, sized for a gate column and the largest split count
    split = gemm_route_ws_bytes(T, H, gemm_route_cols(E + 1), gemm_route_splits(T, H, 16));
  } else if (bf16 && T > 0) {
    const int64_t ncols = E + 1;
    const int64_t nb = ncols <= 64 ? 4 : ncols <= 80 ? 5 : ncols <= 144 ? 9 : 17;
    const int64_t tm = ncols <= 144 ? 16 : 32;
    const int64_t tiles = (T + tm - 1) / tm;
    if (tiles < kSplitTiles) split = (size_t)((kSplitWgs / tiles) * tiles * tm * 16 * nb * 4);
  }
  return route_part_bytes(T, E, bf16) + split;
}

int launch_aux_loss(const float* sums, const int32_t* counts, int64_t T, int64_t k, int64_t E, float alpha, float* loss,
                    float* coef, hipStream_t stream) {
  const double scale = (double)alpha * (double)E / ((double)T * (double)k * (double)T);
  hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(256), 0, stream, sums, counts, (int)E, scale, loss, coef);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace moe
