// Per-token kernels: combine, its backward, router backward, the dx sum, the
// weight-gradient row reduction, and the balance controller.
//
// Combine: "feat: Phase 43 — Sparse/Grouped MoE Dispatch" scatters each
// expert's weighted output back with index_add; "mstar.model.components.moe"
// (SparseMoeBlockWithSharedExpert) adds sigmoid(shared_gate(x)) *
// shared_expert(x).  Here every token gathers its k expert rows and sums
// w[t,j] * y in the fixed order j = 0..k-1 in fp32 (no atomics), then adds the
// shared term.  y and S arrive in fp32, or in binary16 (the forward of a bf16
// layer stores them so).  Balance: "Sparse MoE FFN for DFlash-family drafters" (What's
// here: sign controller on expert loads, fp32 bias).  Every reduction here runs
// in a fixed order, so results are bitwise reproducible.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// fixed xor-butterfly wave sum for float or double
template <typename Acc>
MOE_DEV Acc wave_sum_t(Acc v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// 16-byte chunk <-> 8 (bf16) or 4 (fp32) floats
template <typename T> struct Vec;
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  static MOE_DEV void load(const bf16_t* p, float* v) {
    const u32x4_t w = *(const u32x4_t*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static MOE_DEV void store(bf16_t* p, const float* v) {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *(u32x4_t*)p = w;
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  static MOE_DEV void load(const float* p, float* v) {
    const f32x4_t w = *(const f32x4_t*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = w[i];
  }
  static MOE_DEV void store(float* p, const float* v) { *(f32x4_t*)p = f32x4_t{v[0], v[1], v[2], v[3]}; }
};

// Four consecutive y / S values as floats (fp32 or binary16 storage).
MOE_DEV void ld4(const float* p, float* v) { Vec<float>::load(p, v); }
MOE_DEV void ld4(const f16_t* p, float* v) {
  const f16x4_t h = *(const f16x4_t*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (float)h[i];
}

// One workgroup (4 waves) per token.  Lanes j < k hold the slot's sorted row
// and weight; each column chunk of V outputs loads all k rows before
// accumulating (KMAX > 0), then acc = sum_j w[t,j] * y[row_j] in increasing
// j, plus gate * S.  The four waves take interleaved 64 V-column blocks, so
// at any time they read 4 consecutive KB of each gathered row (one wave per
// token, 1 KB pieces of 6-8 scattered rows, measured 125 against 107 us at
// the DSV4-Flash shape).
template <typename T, int KMAX, typename YT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* y, const int32_t* pos, const float* w,
                                                      const YT* s, const float* gate, T* out, int T_, int k,
                                                      int H) {
  constexpr int V = Vec<T>::N;  // outputs per 16-byte store
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  const int wv = threadIdx.x >> 6;
  if (t >= T_) return;
  int my_r = 0;
  float my_w = 0.0f;
  if (KMAX > 0 && lane < k) {
    my_r = pos[(int64_t)t * k + lane];
    my_w = w[(int64_t)t * k + lane];
  }
  const float g = gate ? gate[t] : 1.0f;
  // one token a workgroup: wave w takes column blocks w, w + 4, ..., so the
  // four waves read 4 consecutive KB of each row together
  for (int c = ((blockIdx.y * 4 + wv) * 64 + lane) * V; c < H; c += gridDim.y * 4 * 64 * V) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
    if constexpr (KMAX > 0) {
      float v[KMAX][V];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) {
          const YT* yr = y + (int64_t)__builtin_amdgcn_readlane(my_r, j) * H + c;
#pragma unroll
          for (int i = 0; i < V; i += 4) ld4(yr + i, &v[j][i]);
        }
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) {
          const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j));
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] += wj * v[j][i];
        }
    } else {
      for (int j = 0; j < k; ++j) {
        const float wj = w[(int64_t)t * k + j];
        const YT* yr = y + (int64_t)pos[(int64_t)t * k + j] * H + c;
        float v[V];
#pragma unroll
        for (int i = 0; i < V; i += 4) ld4(yr + i, &v[i]);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += wj * v[i];
      }
    }
    if (s) {
      float v[V];
#pragma unroll
      for (int i = 0; i < V; i += 4) ld4(s + (int64_t)t * H + c + i, &v[i]);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += g * v[i];
    }
    Vec<T>::store(out + (int64_t)t * H + c, acc);
  }
}

// dy[pos[t,j]] = w[t,j] * dout[t];  dweights[t,j] = dout[t] . y[pos[t,j]];
// ds[t] = gate[t] * dout[t];  dz[t] = gate (1 - gate) dout[t] . s[t]
template <typename T, typename Acc, typename YT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* dout, const YT* y, const int32_t* pos,
                                                          const float* w, const YT* s, const float* gate, T* dy,
                                                          float* dweights, T* ds, float* dz, int T_, int k, int H) {
  constexpr int V = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const float g = gate ? gate[t] : 1.0f;
  Acc part[9];
  const int kk = k < 8 ? k : 8;
#pragma unroll
  for (int j = 0; j < 9; ++j) part[j] = 0.0f;
  for (int c = lane * V; c < H; c += 64 * V) {
    float d[V];
    Vec<T>::load(dout + (int64_t)t * H + c, d);
    for (int j = 0; j < kk; ++j) {
      const int r = pos[(int64_t)t * k + j];
      const float wj = w[(int64_t)t * k + j];
      float v[V], o[V];
#pragma unroll
      for (int i = 0; i < V; i += 4) ld4(y + (int64_t)r * H + c + i, &v[i]);
      Acc dot = 0;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        dot += (Acc)d[i] * (Acc)v[i];
        o[i] = wj * d[i];
      }
      part[j] += dot;
      Vec<T>::store(dy + (int64_t)r * H + c, o);
    }
    if (s) {
      float v[V], o[V];
#pragma unroll
      for (int i = 0; i < V; i += 4) ld4(s + (int64_t)t * H + c + i, &v[i]);
      Acc dot = 0;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        dot += (Acc)d[i] * (Acc)v[i];
        o[i] = g * d[i];
      }
      part[8] += dot;
      Vec<T>::store(ds + (int64_t)t * H + c, o);
    }
  }
  for (int j = 0; j < kk; ++j) {
    const Acc tot = wave_sum_t(part[j]);
    if (lane == 0) dweights[(int64_t)t * k + j] = (float)tot;
  }
  if (s && dz) {
    const Acc tot = wave_sum_t(part[8]);
    if (lane == 0) dz[t] = (float)(tot * (Acc)g * ((Acc)1 - (Acc)g));
  }
}

// dlogits of one token: weights -> selected scores (renorm) -> scores -> logits.
// aux_coef (or null): the aux loss's score gradient, the same for every token.
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* logits, const int64_t* ids, const float* w,
                                                         const float* dw, const float* aux_coef, float* dl, int T_,
                                                         int E, int k, int score, int renorm) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  // selected-score gradients, identical on every lane
  float wdw = 0.0f, den = 0.0f;
  for (int j = 0; j < k; ++j) wdw += w[(int64_t)t * k + j] * dw[(int64_t)t * k + j];
  float lg[4], s[4], ds[4];
  float m = -__int_as_float(0x7f800000);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane + 64 * r;
    lg[r] = e < E ? logits[(int64_t)t * E + e] : -__int_as_float(0x7f800000);
    m = fmaxf(m, lg[r]);
  }
  if (score == 0) {
    m = wave_max(m);
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = (lane + 64 * r < E) ? expf(lg[r] - m) : 0.0f;
      part += s[r];
    }
    const float tot = wave_sum(part);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = s[r] / tot;
  } else if (score == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = 1.0f / (1.0f + expf(-lg[r]));
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = sqrtf(fmaxf(lg[r], 0.0f) + log1pf(expf(-fabsf(lg[r]))));
  }
  // denominator of the renormalisation: sum of selected scores (j order)
  for (int j = 0; j < k; ++j) {
    const int e = (int)ids[(int64_t)t * k + j];
    const int r = e >> 6;  // uniform across the wave
    const float mine = r == 0 ? s[0] : (r == 1 ? s[1] : (r == 2 ? s[2] : s[3]));
    den += __shfl(mine, e & 63, 64);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) ds[r] = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int e = (int)ids[(int64_t)t * k + j];
    const float g = renorm ? (dw[(int64_t)t * k + j] - wdw) / den : dw[(int64_t)t * k + j];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (e == lane + 64 * r) ds[r] += g;
  }
  if (aux_coef) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (lane + 64 * r < E) ds[r] += aux_coef[lane + 64 * r];
  }
  if (score == 0) {
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) part += s[r] * ds[r];
    const float sd = wave_sum(part);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + 64 * r;
      if (e < E) dl[(int64_t)t * E + e] = s[r] * (ds[r] - sd);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + 64 * r;
      if (e >= E) continue;
      float v;
      if (score == 1) {
        v = ds[r] * s[r] * (1.0f - s[r]);
      } else {
        const float sig = 1.0f / (1.0f + expf(-lg[r]));
        v = ds[r] * sig / (2.0f * s[r]);
      }
      dl[(int64_t)t * E + e] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Parallel dense + MoE block (the DeepSpec issue "Feat: Compatible with Gamme4 MoE structure":
// Decoder layer forward pass).  One wave per token; every sum of squares is a per-lane partial over
// the lane's columns (increasing), then the fixed xor butterfly; Acc is fp32 for a bf16 layer, fp64
// for an fp32 one.

// out[t] = x[t] / sqrt(mean(x[t]^2) + eps) * g
template <typename T, typename Acc>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* x, const T* g, float eps, T* out, int T_, int H) {
  constexpr int V = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  Acc ss = 0;
  for (int c = lane * V; c < H; c += 64 * V) {
    float v[V];
    Vec<T>::load(x + (int64_t)t * H + c, v);
#pragma unroll
    for (int i = 0; i < V; ++i) ss += (Acc)v[i] * (Acc)v[i];
  }
  ss = wave_sum_t(ss);
  const float r = (float)((Acc)1 / sqrt(ss / (Acc)H + (Acc)eps));
  for (int c = lane * V; c < H; c += 64 * V) {
    float v[V], gv[V], o[V];
    Vec<T>::load(x + (int64_t)t * H + c, v);
    Vec<T>::load(g + c, gv);
#pragma unroll
    for (int i = 0; i < V; ++i) o[i] = v[i] * r * gv[i];
    Vec<T>::store(out + (int64_t)t * H + c, o);
  }
}

// Block output of one token: h2 = sum_j w[t,j] y[pos[t,j]] (j increasing),
// h1 = s[t] (the dense MLP), a = N(h1; g1) + N(h2; g2), out = (residual +
// N(a; g)) * scalar with N(v; g) = v / sqrt(mean(v^2) + eps) * g.  The wave
// keeps h1 and h2 (then a) of its token in LDS between the passes.
template <typename T, typename Acc, typename YT, int KMAX>
__global__ __launch_bounds__(64) void block_out_kernel(const YT* y, const int32_t* pos, const float* w,
                                                       const YT* s, const T* residual, const T* g1, const T* g2,
                                                       const T* g, float eps, float scalar, T* out, int T_, int k,
                                                       int H) {
  extern __shared__ float rows[];  // [2][H]: h1, h2
  constexpr int V = Vec<T>::N;
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  float* h1 = rows;
  float* h2 = rows + H;
  int my_r = 0;
  float my_w = 0.0f;
  if (lane < k) {
    my_r = pos[(int64_t)t * k + lane];
    my_w = w[(int64_t)t * k + lane];
  }
  Acc s1 = 0, s2 = 0;
  for (int c = lane * V; c < H; c += 64 * V) {
    float acc[V], v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k && j < KMAX; ++j) {
      const YT* yr = y + (int64_t)__builtin_amdgcn_readlane(my_r, j) * H + c;
      const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j));
#pragma unroll
      for (int i = 0; i < V; i += 4) ld4(yr + i, &v[i]);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += wj * v[i];
    }
#pragma unroll
    for (int i = 0; i < V; i += 4) ld4(s + (int64_t)t * H + c + i, &v[i]);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      h1[c + i] = v[i];
      h2[c + i] = acc[i];
      s1 += (Acc)v[i] * (Acc)v[i];
      s2 += (Acc)acc[i] * (Acc)acc[i];
    }
  }
  s1 = wave_sum_t(s1);
  s2 = wave_sum_t(s2);
  const float r1 = (float)((Acc)1 / sqrt(s1 / (Acc)H + (Acc)eps));
  const float r2 = (float)((Acc)1 / sqrt(s2 / (Acc)H + (Acc)eps));
  Acc s3 = 0;
  for (int c = lane * V; c < H; c += 64 * V) {
    float a1[V], a2[V];
    Vec<T>::load(g1 + c, a1);
    Vec<T>::load(g2 + c, a2);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float a = h1[c + i] * r1 * a1[i] + h2[c + i] * r2 * a2[i];
      h1[c + i] = a;
      s3 += (Acc)a * (Acc)a;
    }
  }
  s3 = wave_sum_t(s3);
  const float r3 = (float)((Acc)1 / sqrt(s3 / (Acc)H + (Acc)eps));
  for (int c = lane * V; c < H; c += 64 * V) {
    float res[V], gv[V], o[V];
    Vec<T>::load(residual + (int64_t)t * H + c, res);
    Vec<T>::load(g + c, gv);
#pragma unroll
    for (int i = 0; i < V; ++i) o[i] = (res[i] + h1[c + i] * r3 * gv[i]) * scalar;
    Vec<T>::store(out + (int64_t)t * H + c, o);
  }
}

// tokens per row-reduction chunk: 128 gives the 16-column kernel 64 chunks
// at 8192 tokens, enough workgroups to hide its load latency (256: 0.131 ms,
// 128: 0.094 ms for the router-weight gradient of the Qwen2-MoE training shape)
constexpr int kRowChunk = 128;

// partial[c][e][h] = sum_{t in chunk c} a[t,e] b[t,h]  (t ascending).
// Acc is fp32 for a bf16 layer, fp64 for an fp32 layer.
// partial[c][e][h] = sum over t in chunk c (increasing t) of a[t][e] * b[t][h].
// Thread: one column h and 64 experts e0 .. e0 + 63 (blockIdx.y); each b
// element is loaded once; the a rows go through LDS 32 tokens at a time and
// are read back as broadcasts.
template <typename T, typename Acc>
__global__ __launch_bounds__(256) void rowreduce_partial_kernel(const float* __restrict__ a,
                                                                const T* __restrict__ b, Acc* __restrict__ partial,
                                                                int T_, int E, int H) {
  constexpr int EG = 64, TB = 32;
  __shared__ __attribute__((aligned(16))) float at[TB][EG];
  const int h = blockIdx.x * 256 + threadIdx.x;
  const int e0 = blockIdx.y * EG;
  const int c = blockIdx.z;
  const int t0 = c * kRowChunk, t1 = min(T_, t0 + kRowChunk);
  const int ne = min(EG, E - e0);
  Acc acc[EG];
#pragma unroll
  for (int j = 0; j < EG; ++j) acc[j] = 0;
  const bool hok = h < H;
  for (int tb = t0; tb < t1; tb += TB) {
    __syncthreads();
    for (int i = threadIdx.x; i < TB * EG; i += 256) {
      const int tt = tb + i / EG, j = i % EG;
      at[i / EG][j] = (tt < t1 && j < ne) ? a[(int64_t)tt * E + e0 + j] : 0.0f;
    }
    __syncthreads();
    const int nt = min(TB, t1 - tb);
    for (int u = 0; u < nt; ++u) {
      const Acc xv = hok ? (Acc)Elem<T>::load(b + (int64_t)(tb + u) * H + h) : (Acc)0;
#pragma unroll
      for (int j = 0; j < EG; j += 4) {
        const f32x4_t av = *(const f32x4_t*)&at[u][j];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[j + q] += (Acc)av[q] * xv;
      }
    }
  }
  if (!hok) return;
#pragma unroll
  for (int j = 0; j < EG; ++j)
    if (j < ne) partial[((int64_t)c * E + e0 + j) * H + h] = acc[j];
}

// bf16 operand b: partial[c][e][h] as above, a thread owning 8 consecutive
// columns (one 16-byte load of b per token) and EG experts e0 .. e0 + EG - 1;
// the a rows go through LDS 32 tokens at a time and are read as broadcasts.
// Each accumulator still sums its chunk's tokens in increasing order.
// a2 (optional, [T]) is one more column after the E columns of a: the
// partial rows are [nchunks][Et][H] with Et = E + (a2 != null).
template <int EG>
__global__ __launch_bounds__(128) void rowreduce8_kernel(const float* __restrict__ a, const float* __restrict__ a2,
                                                         const bf16_t* __restrict__ b, float* __restrict__ partial,
                                                         int T_, int E, int H) {
  constexpr int TB = 32;
  __shared__ __attribute__((aligned(16))) float at[TB][EG < 4 ? 4 : EG];
  const int h0 = (blockIdx.x * 128 + threadIdx.x) * 8;
  const int Et = E + (a2 ? 1 : 0);
  const int e0 = blockIdx.y * EG;
  const int c = blockIdx.z;
  const int t0 = c * kRowChunk, t1 = min(T_, t0 + kRowChunk);
  const int ne = min(EG, Et - e0);
  float acc[EG][8];
#pragma unroll
  for (int j = 0; j < EG; ++j)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[j][q] = 0.0f;
  const bool hok = h0 < H;
  for (int tb = t0; tb < t1; tb += TB) {
    __syncthreads();
    for (int i = threadIdx.x; i < TB * EG; i += 128) {
      const int tt = tb + i / EG, j = i % EG;
      at[i / EG][j] = (tt < t1 && j < ne) ? (e0 + j < E ? a[(int64_t)tt * E + e0 + j] : a2[tt]) : 0.0f;
    }
    __syncthreads();
    const int nt = min(TB, t1 - tb);
    // 8 tokens at a time: their 8 row loads are in flight together
    for (int u0 = 0; u0 < nt; u0 += 8) {
      u32x4_t xr[8];
#pragma unroll
      for (int v = 0; v < 8; ++v)
        xr[v] = (hok && u0 + v < nt) ? *(const u32x4_t*)(b + (int64_t)(tb + u0 + v) * H + h0) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        if (u0 + v >= nt) break;
        float xv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xv[2 * i] = __uint_as_float(xr[v][i] << 16);
          xv[2 * i + 1] = __uint_as_float(xr[v][i] & 0xffff0000u);
        }
        if constexpr (EG % 4 == 0) {
#pragma unroll
          for (int j = 0; j < EG; j += 4) {
            const f32x4_t a4 = *(const f32x4_t*)&at[u0 + v][j];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
              for (int q = 0; q < 8; ++q) acc[j + jj][q] += a4[jj] * xv[q];
          }
        } else {
#pragma unroll
          for (int j = 0; j < EG; ++j) {
            const float av = at[u0 + v][j];
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[j][q] += av * xv[q];
          }
        }
      }
    }
  }
  if (!hok) return;
#pragma unroll
  for (int j = 0; j < EG; ++j)
    if (j < ne) {
      float* dst = partial + ((int64_t)c * Et + e0 + j) * H + h0;
      *(f32x4_t*)dst = f32x4_t{acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
      *(f32x4_t*)(dst + 4) = f32x4_t{acc[j][4], acc[j][5], acc[j][6], acc[j][7]};
    }
}

// out = rows [0, E) of the chunk sum, out2 = row E when Et = E + 1
template <typename Acc>
__global__ __launch_bounds__(256) void rowreduce_final_kernel(const Acc* partial, float* out, float* out2, int nchunks,
                                                              int Et, int E, int H) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)Et * H) return;
  Acc acc = 0;
  for (int c = 0; c < nchunks; ++c) acc += partial[(int64_t)c * Et * H + i];
  if (i < (int64_t)E * H)
    out[i] = (float)acc;
  else
    out2[i - (int64_t)E * H] = (float)acc;
}

// dx for a block of TB tokens x 256 V columns: V consecutive columns per
// thread (4 in a bf16 layer, whose dxs / dxsh rows are binary16; 1 in an fp32
// layer, fp32 rows, fp64 accumulation).  The router term of the block's
// tokens shares each w_router load; the slot rows are loaded slot by slot for
// all the block's tokens at once (their row indices staged in LDS), so a
// wave keeps TB independent loads in flight.  Per token the slot rows (in
// slot order), the shared row, the router term and the gate term are added
// in that order.
template <typename DT, int V> MOE_DEV void ldv(const DT* p, float* v);
template <> MOE_DEV void ldv<f16_t, 4>(const f16_t* p, float* v) {
  const f16x4_t h = *(const f16x4_t*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (float)h[i];
}
template <> MOE_DEV void ldv<float, 1>(const float* p, float* v) { v[0] = *p; }
template <> MOE_DEV void ldv<bf16_t, 4>(const bf16_t* p, float* v) {
  const u32x2_t w = *(const u32x2_t*)p;
  v[0] = __uint_as_float(w[0] << 16);
  v[1] = __uint_as_float(w[0] & 0xffff0000u);
  v[2] = __uint_as_float(w[1] << 16);
  v[3] = __uint_as_float(w[1] & 0xffff0000u);
}
template <typename T, int V> MOE_DEV void stv(T* p, const float* v);
template <> MOE_DEV void stv<bf16_t, 4>(bf16_t* p, const float* v) {
  *(u32x2_t*)p = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
template <> MOE_DEV void stv<float, 1>(float* p, const float* v) { *p = v[0]; }

constexpr int kDxTok = 8;  // tokens per dx_sum block
template <typename T, typename Acc, typename DT, int V>
__global__ __launch_bounds__(256) void dx_sum_kernel(const DT* dxs, const int32_t* pos, const DT* dxsh,
                                                     const float* dl, const T* wr, const float* dz, const T* wg, T* dx,
                                                     int T_, int k, int E, int H) {
  constexpr int TB = kDxTok;
  __shared__ float sdl[TB][256];
  __shared__ int spos[TB * 64];
  const int t0 = blockIdx.y * TB;
  const int nt = min(TB, T_ - t0);
  const int h = (blockIdx.x * 256 + threadIdx.x) * V;
  for (int i = threadIdx.x; i < TB * E; i += 256) {
    const int tt = i / E, e = i % E;
    sdl[tt][e] = tt < nt ? dl[(int64_t)(t0 + tt) * E + e] : 0.0f;
  }
  for (int i = threadIdx.x; i < nt * k; i += 256) spos[i] = pos[(int64_t)t0 * k + i];
  __syncthreads();
  if (h >= H) return;
  Acc v[TB][V];
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int c = 0; c < V; ++c) v[i][c] = 0;
  for (int j = 0; j < k; ++j) {
    float d[TB][V];
#pragma unroll
    for (int i = 0; i < TB; ++i)
      if (i < nt) ldv<DT, V>(dxs + (int64_t)spos[i * k + j] * H + h, d[i]);
#pragma unroll
    for (int i = 0; i < TB; ++i)
      if (i < nt)
#pragma unroll
        for (int c = 0; c < V; ++c) v[i][c] += (Acc)d[i][c];
  }
  if (dxsh) {
    float d[TB][V];
#pragma unroll
    for (int i = 0; i < TB; ++i)
      if (i < nt) ldv<DT, V>(dxsh + (int64_t)(t0 + i) * H + h, d[i]);
#pragma unroll
    for (int i = 0; i < TB; ++i)
      if (i < nt)
#pragma unroll
        for (int c = 0; c < V; ++c) v[i][c] += (Acc)d[i][c];
  }
  Acc acc[TB][V];
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int c = 0; c < V; ++c) acc[i][c] = 0;
  for (int e = 0; e < E; ++e) {
    float wv[V];
    ldv<T, V>(wr + (int64_t)e * H + h, wv);
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int c = 0; c < V; ++c) acc[i][c] += (Acc)sdl[i][e] * (Acc)wv[c];
  }
  float wgv[V];
#pragma unroll
  for (int c = 0; c < V; ++c) wgv[c] = 0.0f;
  if (wg) ldv<T, V>(wg + h, wgv);
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    if (i < nt) {
      float o[V];
#pragma unroll
      for (int c = 0; c < V; ++c) {
        Acc u = v[i][c] + acc[i][c];
        if (wg && dz) u += (Acc)dz[t0 + i] * (Acc)wgv[c];
        o[c] = (float)u;
      }
      stv<T, V>(dx + (int64_t)(t0 + i) * H + h, o);
    }
  }
}

__global__ __launch_bounds__(1024) void balance_kernel(const int64_t* ids, int32_t* counts, float* bias, float rate,
                                                       int P, int E) {
  __shared__ int h[256];
  for (int e = threadIdx.x; e < E; e += 1024) h[e] = ids ? 0 : counts[e];
  __syncthreads();
  if (ids) {
    for (int i = threadIdx.x; i < P; i += 1024) atomicAdd(&h[(int)ids[i]], 1);
    __syncthreads();
  }
  for (int e = threadIdx.x; e < E; e += 1024) {
    if (ids) counts[e] = h[e];
    if (bias) {
      // sign(T*k/E - c) in exact integer arithmetic: sign(T*k - c*E)
      const int64_t d = (int64_t)P - (int64_t)h[e] * E;
      const float step = d > 0 ? 1.0f : (d < 0 ? -1.0f : 0.0f);
      bias[e] = bias[e] + rate * step;
    }
  }
}

}  // namespace

template <typename OT, typename YT>
void combine_launch(const YT* y, const int32_t* pos, const float* weights, const YT* s, const float* gate, void* out,
                    int64_t T, int64_t k, int64_t H, hipStream_t stream) {
  // short batches: the column blocks of a token spread over gridDim.y
  // workgroups (up to about 1024 in all), so each wave's loop has fewer
  // dependent load rounds
  const int64_t tb = T, cb = (H + 4 * 64 * Vec<OT>::N - 1) / (4 * 64 * Vec<OT>::N);
  const int64_t hs = std::max<int64_t>(1, std::min<int64_t>(cb, 1024 / tb));
  dim3 grid((unsigned)tb, (unsigned)hs), block(256);
  if (k <= 8)
    hipLaunchKernelGGL((combine_kernel<OT, 8, YT>), grid, block, 0, stream, y, pos, weights, s, gate, (OT*)out,
                       (int)T, (int)k, (int)H);
  else
    hipLaunchKernelGGL((combine_kernel<OT, 0, YT>), grid, block, 0, stream, y, pos, weights, s, gate, (OT*)out,
                       (int)T, (int)k, (int)H);
}

int launch_combine(const void* y, int y_f16, const int32_t* pos, const float* weights, const void* s,
                   const float* gate, void* out, int64_t T, int64_t k, int64_t H, int bf16, hipStream_t stream) {
  if (T == 0) return 0;
  if (bf16 && y_f16)
    combine_launch<bf16_t>((const f16_t*)y, pos, weights, (const f16_t*)s, gate, out, T, k, H, stream);
  else if (bf16)
    combine_launch<bf16_t>((const float*)y, pos, weights, (const float*)s, gate, out, T, k, H, stream);
  else if (y_f16)
    combine_launch<float>((const f16_t*)y, pos, weights, (const f16_t*)s, gate, out, T, k, H, stream);
  else
    combine_launch<float>((const float*)y, pos, weights, (const float*)s, gate, out, T, k, H, stream);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_combine_bwd(const void* dout, const void* y, int y_f16, const int32_t* pos, const float* weights,
                       const void* s, const float* gate, void* dy, float* dweights, void* ds, float* dz, int64_t T,
                       int64_t k, int64_t H, int bf16, hipStream_t stream) {
  if (T == 0) return 0;
  if (k > 8) return -2;
  dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (bf16 && y_f16)
    hipLaunchKernelGGL((combine_bwd_kernel<bf16_t, float, f16_t>), grid, block, 0, stream, (const bf16_t*)dout,
                       (const f16_t*)y, pos, weights, (const f16_t*)s, gate, (bf16_t*)dy, dweights, (bf16_t*)ds, dz,
                       (int)T, (int)k, (int)H);
  else if (bf16)
    hipLaunchKernelGGL((combine_bwd_kernel<bf16_t, float, float>), grid, block, 0, stream, (const bf16_t*)dout,
                       (const float*)y, pos, weights, (const float*)s, gate, (bf16_t*)dy, dweights, (bf16_t*)ds, dz,
                       (int)T, (int)k, (int)H);
  else
    hipLaunchKernelGGL((combine_bwd_kernel<float, double, float>), grid, block, 0, stream, (const float*)dout,
                       (const float*)y, pos, weights, (const float*)s, gate, (float*)dy, dweights, (float*)ds, dz,
                       (int)T, (int)k, (int)H);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_router_bwd(const float* logits, const int64_t* ids, const float* weights, const float* dweights,
                      const float* aux_coef, float* dlogits, int64_t T, int64_t E, int64_t k, int score, int renorm,
                      hipStream_t stream) {
  if (T == 0) return 0;
  dim3 grid((unsigned)((T + 3) / 4)), block(256);
  hipLaunchKernelGGL(router_bwd_kernel, grid, block, 0, stream, logits, ids, weights, dweights, aux_coef, dlogits,
                     (int)T, (int)E, (int)k, score, renorm);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_rmsnorm(const void* x, const void* g, float eps, void* out, int64_t T, int64_t H, int bf16,
                   hipStream_t stream) {
  if (T == 0) return 0;
  dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (bf16)
    hipLaunchKernelGGL((rmsnorm_kernel<bf16_t, float>), grid, block, 0, stream, (const bf16_t*)x, (const bf16_t*)g, eps,
                       (bf16_t*)out, (int)T, (int)H);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<float, double>), grid, block, 0, stream, (const float*)x, (const float*)g, eps,
                       (float*)out, (int)T, (int)H);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_block_out(const void* y, int y_f16, const int32_t* pos, const float* weights, const void* s,
                     const void* residual, const void* g1, const void* g2, const void* g, float eps, float scalar,
                     void* out, int64_t T, int64_t k, int64_t H, int bf16, hipStream_t stream) {
  if (T == 0) return 0;
  if (k > 8 || H * 8 > 64 * 1024) return -2;
  const size_t lds = (size_t)H * 2 * 4;
  if (bf16 && y_f16)
    hipLaunchKernelGGL((block_out_kernel<bf16_t, float, f16_t, 8>), dim3((unsigned)T), dim3(64), lds, stream,
                       (const f16_t*)y, pos, weights, (const f16_t*)s, (const bf16_t*)residual, (const bf16_t*)g1,
                       (const bf16_t*)g2, (const bf16_t*)g, eps, scalar, (bf16_t*)out, (int)T, (int)k, (int)H);
  else if (!bf16 && !y_f16)
    hipLaunchKernelGGL((block_out_kernel<float, double, float, 8>), dim3((unsigned)T), dim3(64), lds, stream,
                       (const float*)y, pos, weights, (const float*)s, (const float*)residual, (const float*)g1,
                       (const float*)g2, (const float*)g, eps, scalar, (float*)out, (int)T, (int)k, (int)H);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

int launch_zero_f32(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

size_t rowreduce_ws_bytes(int64_t T, int64_t E, int64_t H) {
  const int64_t nch = (T + kRowChunk - 1) / kRowChunk;
  return (size_t)((nch > 0 ? nch : 1) * E * H * 8);
}

int launch_rowreduce(const float* a, const float* a2, const void* b, void* out, void* out2, int64_t T, int64_t E,
                     int64_t H, int bf16, void* ws, hipStream_t stream) {
  const int nch = (int)((T + kRowChunk - 1) / kRowChunk);
  const bool fused = a2 && bf16 && nch > 0 && H % 8 == 0;
  if (a2 && !fused) {  // the extra column as a reduction of its own
    const int st = launch_rowreduce(a, nullptr, b, out, nullptr, T, E, H, bf16, ws, stream);
    return st ? st : launch_rowreduce(a2, nullptr, b, out2, nullptr, T, 1, H, bf16, ws, stream);
  }
  const int64_t Et = E + (fused ? 1 : 0);
  dim3 grid((unsigned)((H + 255) / 256), (unsigned)((E + 63) / 64), (unsigned)nch);
  dim3 g2((unsigned)((Et * H + 255) / 256));
  if (bf16) {
    float* partial = (float*)ws;
    if (nch > 0 && H % 8 == 0) {
      // 16 (8, or 1 for a single column) columns of a a thread: each x row
      // load serves them all, and there are enough workgroups for every SIMD
      // at the usual sizes
      const dim3 gx((unsigned)((H / 8 + 127) / 128), 1, (unsigned)nch);
      if (Et == 1)
        hipLaunchKernelGGL((rowreduce8_kernel<1>), gx, dim3(128), 0, stream, a, a2, (const bf16_t*)b, partial,
                           (int)T, (int)E, (int)H);
      else if (Et <= 8)
        hipLaunchKernelGGL((rowreduce8_kernel<8>), gx, dim3(128), 0, stream, a, a2, (const bf16_t*)b, partial,
                           (int)T, (int)E, (int)H);
      else
        hipLaunchKernelGGL((rowreduce8_kernel<16>), dim3(gx.x, (unsigned)((Et + 15) / 16), gx.z), dim3(128), 0,
                           stream, a, a2, (const bf16_t*)b, partial, (int)T, (int)E, (int)H);
    } else if (nch > 0) {
      hipLaunchKernelGGL((rowreduce_partial_kernel<bf16_t, float>), grid, dim3(256), 0, stream, a, (const bf16_t*)b,
                         partial, (int)T, (int)E, (int)H);
    }
    hipLaunchKernelGGL((rowreduce_final_kernel<float>), g2, dim3(256), 0, stream, partial, (float*)out, (float*)out2,
                       nch, (int)Et, (int)E, (int)H);
  } else {
    double* partial = (double*)ws;
    if (nch > 0)
      hipLaunchKernelGGL((rowreduce_partial_kernel<float, double>), grid, dim3(256), 0, stream, a, (const float*)b,
                         partial, (int)T, (int)E, (int)H);
    hipLaunchKernelGGL((rowreduce_final_kernel<double>), g2, dim3(256), 0, stream, partial, (float*)out, nullptr,
                       nch, (int)Et, (int)E, (int)H);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_dx_sum(const void* dxs, const int32_t* pos, const void* dxsh, const float* dl, const void* w_router,
                  const float* dz, const void* w_gate, void* dx, int64_t T, int64_t k, int64_t E, int64_t H, int bf16,
                  hipStream_t stream) {
  if (T == 0) return 0;
  if (bf16) {  // H % 8 == 0: four columns a thread
    dim3 grid((unsigned)((H / 4 + 255) / 256), (unsigned)((T + kDxTok - 1) / kDxTok));
    hipLaunchKernelGGL((dx_sum_kernel<bf16_t, float, f16_t, 4>), grid, dim3(256), 0, stream, (const f16_t*)dxs, pos,
                       (const f16_t*)dxsh, dl, (const bf16_t*)w_router, dz, (const bf16_t*)w_gate, (bf16_t*)dx,
                       (int)T, (int)k, (int)E, (int)H);
  } else {
    dim3 grid((unsigned)((H + 255) / 256), (unsigned)((T + kDxTok - 1) / kDxTok));
    hipLaunchKernelGGL((dx_sum_kernel<float, double, float, 1>), grid, dim3(256), 0, stream, (const float*)dxs, pos,
                       (const float*)dxsh, dl, (const float*)w_router, dz, (const float*)w_gate, (float*)dx, (int)T,
                       (int)k, (int)E, (int)H);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_balance(const int64_t* ids, int32_t* counts, float* bias, float rate, int64_t T, int64_t k, int64_t E,
                   hipStream_t stream) {
  hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(1024), 0, stream, ids, counts, bias, rate, (int)(T * k), (int)E);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace moe
