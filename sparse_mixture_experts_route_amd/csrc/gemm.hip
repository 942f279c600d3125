// Grouped GEMM over contiguous per-expert segments (bf16 MFMA, fp32 acc).
//
// "Sparse MoE FFN for DFlash-family drafters" (What's here: routed experts
// as stacked [E, out, in] parameters, grouped-GEMM-ready; sorted-segment
// dispatch with no host syncs) and "mstar.model.components.moe"
// (SparseMoeBlock: gate_up_proj (E, 2I, H), down_proj (E, H, I);
// dispatch_experts_fused runs SwiGLU per expert) define the product:
// for every expert segment, rows of the sorted activations times that
// expert's weight slice.
//
// One engine serves every GEMM of the layer:
//   C[m, n] = sum_k A(m, k) * B(n, k)
// with each operand either K-contiguous (loaded as 16-byte vectors along K)
// or MN-contiguous (loaded as 8x8 blocks and transposed in registers), and
// two tile schedulers that read segment offsets from device memory:
//   GROUP_M: segments split the M rows (forward GEMMs, data gradients);
//            tile slots are launched for the bound sum ceil(c_e/BM) <=
//            ceil(rows/BM) + G, surplus workgroups exit, empty experts get
//            no tiles and their weights are never read.
//   GROUP_K: segments split the reduction rows (weight gradients); every
//            expert's output is written, exact zeros for an empty segment.
// Epilogues: bf16 store; fp32 store; SwiGLU (gate and up columns of one tile
// land in the same lane: h = silu(g) * u, optional fp32 save of g, u);
// SwiGLU backward (dg = dh * u * silu'(g), du = dh * silu(g) from the saved
// fp32 g, u).
//
// Tile: BM x BN x BK with WM x WN waves; LDS holds both operands K-major with
// a 16-byte-chunk XOR swizzle, double buffered with one barrier per K step.
// v_mfma_f32_16x16x32_bf16 takes the weight-side fragment as its A operand,
// so each lane's four accumulators are four consecutive output columns.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

struct Args {
  const bf16_t* A;
  int64_t lda;
  const int32_t* a_idx;
  int a_div;
  const bf16_t* B;
  int64_t ldb, strideB;
  bf16_t* C;
  int64_t ldc, strideC;
  bf16_t* aux;
  bf16_t* aux_out;
  int64_t ld_aux;
  const int32_t* offsets;
  int G;
  int M, N, K;
  int n_half;
  int NTn;  // n tiles
  int MTk;  // GROUP_K: m tiles per group
};

// Tile slot -> (group, first row, row limit) for GROUP_M.  Wave 0 scans the
// per-group tile counts; result broadcast through LDS.  Returns false when
// the slot has no tile.
template <int BM>
MOE_DEV bool find_group_m(const Args& p, int mt, int* s_info, int& g, int& row0, int& row_end) {
  if (p.offsets == nullptr) {
    g = 0;
    row0 = mt * BM;
    row_end = p.M;
    return row0 < p.M;
  }
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int c[4];
    int local = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gi = lane * 4 + r;
      c[r] = 0;
      if (gi < p.G) {
        const int rows = p.offsets[gi + 1] - p.offsets[gi];
        c[r] = (rows + BM - 1) / BM;
      }
      local += c[r];
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const int excl = incl - local;
    if (lane == 63 && mt >= incl) s_info[0] = -1;
    if (mt >= excl && mt < incl) {
      int acc = excl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (mt >= acc && mt < acc + c[r]) {
          const int gi = lane * 4 + r;
          s_info[0] = gi;
          s_info[1] = p.offsets[gi] + (mt - acc) * BM;
          s_info[2] = p.offsets[gi + 1];
        }
        acc += c[r];
      }
    }
  }
  __syncthreads();
  g = s_info[0];
  row0 = s_info[1];
  row_end = s_info[2];
  return g >= 0;
}

MOE_DEV void transpose8x8(const u32x4_t (&v)[8], u32x4_t (&o)[8]) {
  // v[kk] holds 8 bf16 along mn at k = kk; o[mn] holds 8 bf16 along k.
#pragma unroll
  for (int mn = 0; mn < 8; ++mn) {
    const int w = mn >> 1;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t a = v[2 * d][w], b = v[2 * d + 1][w];
      o[mn][d] = (mn & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}

template <int BM, int BN, int BK, int WM, int WN, bool AK, bool BKM, int SCHED, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(Args p) {
  constexpr int NTH = WM * WN * 64;
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int CPR = BK / 8;  // 16-byte chunks per LDS row
  constexpr int ROWS = BM + BN;
  static_assert(FM >= 1 && FN >= 1 && (EPI != EPI_SWIGLU || FN % 2 == 0), "tile");
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];  // [2][ROWS*BK]
  __shared__ int s_info[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---------------- schedule
  int g, row0, row_end, n0, kbeg, kend;
  const int slot = blockIdx.x;
  if constexpr (SCHED == SCHED_GROUP_M) {
    const int nt = slot % p.NTn;
    const int mt = slot / p.NTn;
    if (!find_group_m<BM>(p, mt, s_info, g, row0, row_end)) return;
    n0 = nt * ((EPI == EPI_SWIGLU) ? BN / 2 : BN);
    kbeg = 0;
    kend = p.K;
  } else {
    g = slot / (p.MTk * p.NTn);
    const int rem = slot % (p.MTk * p.NTn);
    row0 = (rem / p.NTn) * BM;
    row_end = p.M;
    n0 = (rem % p.NTn) * BN;
    kbeg = p.offsets ? p.offsets[g] : 0;
    kend = p.offsets ? p.offsets[g + 1] : p.K;
  }
  const bf16_t* Bg = p.B + (SCHED == SCHED_GROUP_M ? (int64_t)g * p.strideB : 0);

  // ---------------- per-thread load descriptors
  // K-major operand: chunk q -> (row r = q / CPR, chunk c = q % CPR)
  // MN-major operand: 8x8 block q -> (row block q % (R/8), k block q / (R/8))
  constexpr int A_UNITS = AK ? BM * CPR : (BM / 8) * (BK / 8);
  constexpr int B_UNITS = BKM ? BN * CPR : (BN / 8) * (BK / 8);
  constexpr int A_IT = (A_UNITS + NTH - 1) / NTH;
  constexpr int B_IT = (B_UNITS + NTH - 1) / NTH;
  constexpr int A_REG = AK ? A_IT : A_IT * 8;
  constexpr int B_REG = BKM ? B_IT : B_IT * 8;
  u32x4_t ra[A_REG], rb[B_REG];
  const bf16_t* a_base[AK ? A_IT : 1];
  bool a_ok[AK ? A_IT : 1];
  const bf16_t* b_base[BKM ? B_IT : 1];
  bool b_ok[BKM ? B_IT : 1];

  // B tile row j -> weight row (SwiGLU: gate rows then the matching up rows)
  auto b_row = [&](int j, bool& ok) -> int {
    if constexpr (EPI == EPI_SWIGLU) {
      const int half = BN / 2;
      const int c = n0 + (j % half);
      ok = c < p.n_half;
      return (j < half) ? c : p.n_half + c;
    } else {
      const int n = n0 + j;
      ok = n < p.N;
      return n;
    }
  };

  if constexpr (AK) {
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
      const int q = tid + it * NTH;
      const int r = q / CPR;
      const int m = row0 + r;
      const bool ok = (q < A_UNITS) && (m < row_end);
      int64_t src = ok ? m : 0;
      if (ok && p.a_idx) src = p.a_idx[m] / p.a_div;
      a_base[it] = p.A + src * p.lda;
      a_ok[it] = ok;
    }
  }
  if constexpr (BKM) {
#pragma unroll
    for (int it = 0; it < B_IT; ++it) {
      const int q = tid + it * NTH;
      const int r = q / CPR;
      bool ok = false;
      int n = 0;
      if (q < B_UNITS) n = b_row(r, ok);
      b_base[it] = Bg + (int64_t)(ok ? n : 0) * p.ldb;
      b_ok[it] = ok;
    }
  }

  auto load_tiles = [&](int k0) {
    if constexpr (AK) {
#pragma unroll
      for (int it = 0; it < A_IT; ++it) {
        const int q = tid + it * NTH;
        const int kk = k0 + (q % CPR) * 8;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (a_ok[it] && kk < kend) v = *(const u32x4_t*)(a_base[it] + kk);
        ra[it] = v;
      }
    } else {
#pragma unroll
      for (int it = 0; it < A_IT; ++it) {
        const int q = tid + it * NTH;
        const int rbk = q % (BM / 8), kb = q / (BM / 8);
        const int m = row0 + rbk * 8;
        const bool ok = (q < A_UNITS) && (m < row_end);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int k = k0 + kb * 8 + kk;
          u32x4_t v = {0u, 0u, 0u, 0u};
          if (ok && k < kend) v = *(const u32x4_t*)(p.A + (int64_t)k * p.lda + m);
          ra[it * 8 + kk] = v;
        }
      }
    }
    if constexpr (BKM) {
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int q = tid + it * NTH;
        const int kk = k0 + (q % CPR) * 8;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (b_ok[it] && kk < kend) v = *(const u32x4_t*)(b_base[it] + kk);
        rb[it] = v;
      }
    } else {
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int q = tid + it * NTH;
        const int rbk = q % (BN / 8), kb = q / (BN / 8);
        const int n = n0 + rbk * 8;
        const bool ok = (q < B_UNITS) && (n < p.N);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int k = k0 + kb * 8 + kk;
          u32x4_t v = {0u, 0u, 0u, 0u};
          if (ok && k < kend) v = *(const u32x4_t*)(Bg + (int64_t)k * p.ldb + n);
          rb[it * 8 + kk] = v;
        }
      }
    }
  };

  auto lds_off = [](int row, int chunk) { return row * BK + ((chunk ^ (row & (CPR - 1))) * 8); };

  auto store_tiles = [&](int buf) {
    bf16_t* la = lds + buf * ROWS * BK;
    bf16_t* lb = la + BM * BK;
    if constexpr (AK) {
#pragma unroll
      for (int it = 0; it < A_IT; ++it) {
        const int q = tid + it * NTH;
        if (q < A_UNITS) *(u32x4_t*)(la + lds_off(q / CPR, q % CPR)) = ra[it];
      }
    } else {
#pragma unroll
      for (int it = 0; it < A_IT; ++it) {
        const int q = tid + it * NTH;
        if (q < A_UNITS) {
          const int rbk = q % (BM / 8), kb = q / (BM / 8);
          u32x4_t v[8], o[8];
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) v[kk] = ra[it * 8 + kk];
          transpose8x8(v, o);
#pragma unroll
          for (int mn = 0; mn < 8; ++mn) *(u32x4_t*)(la + lds_off(rbk * 8 + mn, kb)) = o[mn];
        }
      }
    }
    if constexpr (BKM) {
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int q = tid + it * NTH;
        if (q < B_UNITS) *(u32x4_t*)(lb + lds_off(q / CPR, q % CPR)) = rb[it];
      }
    } else {
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int q = tid + it * NTH;
        if (q < B_UNITS) {
          const int rbk = q % (BN / 8), kb = q / (BN / 8);
          u32x4_t v[8], o[8];
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) v[kk] = rb[it * 8 + kk];
          transpose8x8(v, o);
#pragma unroll
          for (int mn = 0; mn < 8; ++mn) *(u32x4_t*)(lb + lds_off(rbk * 8 + mn, kb)) = o[mn];
        }
      }
    }
  };

  // LDS row of the wave's fn-th 16-row block of the B tile
  auto b_lds_block = [&](int fn) -> int {
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int H2 = FN / 2;
      return (fn < H2) ? (wn * H2 + fn) : (BN / 32 + wn * H2 + (fn - H2));
    } else {
      return wn * FN + fn;
    }
  };

  f32x4_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (kend - kbeg + BK - 1) / BK;
  if (nk > 0) {
    load_tiles(kbeg);
    store_tiles(0);
  }
  __syncthreads();
  const int lr = lane & 15, lq = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_tiles(kbeg + (kt + 1) * BK);
    const bf16_t* la = lds + (kt & 1) * ROWS * BK;
    const bf16_t* lb = la + BM * BK;
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int row = wm * (BM / WM) + fm * 16 + lr;
        af[fm] = *(const bf16x8_t*)(la + lds_off(row, s * 4 + lq));
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int row = b_lds_block(fn) * 16 + lr;
        bfr[fn] = *(const bf16x8_t*)(lb + lds_off(row, s * 4 + lq));
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[fn][fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[fn], af[fm], acc[fn][fm], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles((kt + 1) & 1);
    __syncthreads();
  }

  // ---------------- epilogue: lane holds rows m = ... + lr, cols n = ... + 4*lq + i
  bf16_t* Cg = p.C + (SCHED == SCHED_GROUP_K ? (int64_t)g * p.strideC : 0);
  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int H2 = FN / 2;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = row0 + wm * (BM / WM) + fm * 16 + lr;
      if (m >= row_end) continue;
#pragma unroll
      for (int fn = 0; fn < H2; ++fn) {
        const int col = n0 + (wn * H2 + fn) * 16 + lq * 4;
        if (col >= p.n_half) continue;
        const f32x4_t gv = acc[fn][fm], uv = acc[fn + H2][fm];
        float h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = gv[i] * fast_sigmoid(gv[i]) * uv[i];
        u32x2_t hv = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        *(u32x2_t*)(Cg + (int64_t)m * p.ldc + col) = hv;
        if (p.aux) {  // fp32 pre-activations for the backward
          float* ga = (float*)p.aux + (int64_t)m * p.ld_aux + col;
          *(f32x4_t*)ga = gv;
          *(f32x4_t*)(ga + p.n_half) = uv;
        }
      }
    }
  } else if constexpr (EPI == EPI_DSWIGLU) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = row0 + wm * (BM / WM) + fm * 16 + lr;
      if (m >= row_end) continue;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = n0 + (wn * FN + fn) * 16 + lq * 4;
        if (col >= p.N) continue;
        const float* ga = (const float*)p.aux + (int64_t)m * p.ld_aux + col;
        const f32x4_t g4 = *(const f32x4_t*)ga;
        const f32x4_t u4 = *(const f32x4_t*)(ga + p.n_half);
        float dg[4], du[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gval = g4[i], uval = u4[i];
          const float sg = fast_sigmoid(gval);
          const float dh = acc[fn][fm][i];
          du[i] = dh * gval * sg;
          dg[i] = dh * uval * (sg * (1.0f + gval * (1.0f - sg)));
        }
        u32x2_t dg2 = {pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
        u32x2_t du2 = {pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
        *(u32x2_t*)(p.aux_out + (int64_t)m * p.ld_aux + col) = dg2;
        *(u32x2_t*)(p.aux_out + (int64_t)m * p.ld_aux + p.n_half + col) = du2;
      }
    }
  } else if constexpr (EPI == EPI_STORE_F32) {
    float* Cf = (float*)p.C + (SCHED == SCHED_GROUP_K ? (int64_t)g * p.strideC : 0);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = row0 + wm * (BM / WM) + fm * 16 + lr;
      if (m >= row_end) continue;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = n0 + (wn * FN + fn) * 16 + lq * 4;
        if (col >= p.N) continue;
        *(f32x4_t*)(Cf + (int64_t)m * p.ldc + col) = acc[fn][fm];
      }
    }
  } else {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = row0 + wm * (BM / WM) + fm * 16 + lr;
      if (m >= row_end) continue;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = n0 + (wn * FN + fn) * 16 + lq * 4;
        if (col >= p.N) continue;
        const f32x4_t v = acc[fn][fm];
        u32x2_t o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *(u32x2_t*)(Cg + (int64_t)m * p.ldc + col) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 engine (the fp32 layer dtype): one thread per output element, a plain
// loop over k in increasing order accumulated in fp64 (the fp32 layer's
// gradients sum over thousands of rows; fp64 keeps them within 1e-5).  Same operand, scheduler and
// epilogue semantics as the bf16 engine.
constexpr int kSB = 16;  // 16 x 16 outputs per workgroup

template <int SCHED, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(Args pa, const float* A, const float* B, float* C,
                                                        float* aux, float* aux_out, int a_kmajor, int b_kmajor) {
  __shared__ int s_info[4];
  int g, row0, row_end, n0, kbeg, kend;
  const int slot = blockIdx.x;
  if constexpr (SCHED == SCHED_GROUP_M) {
    const int nt = slot % pa.NTn;
    const int mt = slot / pa.NTn;
    if (!find_group_m<kSB>(pa, mt, s_info, g, row0, row_end)) return;
    n0 = nt * kSB;
    kbeg = 0;
    kend = pa.K;
  } else {
    g = slot / (pa.MTk * pa.NTn);
    const int rem = slot % (pa.MTk * pa.NTn);
    row0 = (rem / pa.NTn) * kSB;
    row_end = pa.M;
    n0 = (rem % pa.NTn) * kSB;
    kbeg = pa.offsets ? pa.offsets[g] : 0;
    kend = pa.offsets ? pa.offsets[g + 1] : pa.K;
  }
  const int m = row0 + (threadIdx.x >> 4);
  const int n = n0 + (threadIdx.x & 15);
  const int ncols = (EPI == EPI_SWIGLU) ? pa.n_half : pa.N;
  if (m >= row_end || n >= ncols) return;
  const float* Bg = B + (SCHED == SCHED_GROUP_M ? (int64_t)g * pa.strideB : 0);
  int64_t arow = m;
  if (pa.a_idx) arow = pa.a_idx[m] / pa.a_div;
  auto a_at = [&](int k) { return a_kmajor ? A[arow * pa.lda + k] : A[(int64_t)k * pa.lda + m]; };
  auto b_at = [&](int nn, int k) { return b_kmajor ? Bg[(int64_t)nn * pa.ldb + k] : Bg[(int64_t)k * pa.ldb + nn]; };
  if constexpr (EPI == EPI_SWIGLU) {
    double gd = 0.0, ud = 0.0;
    for (int k = kbeg; k < kend; ++k) {
      const double av = a_at(k);
      gd += av * (double)b_at(n, k);
      ud += av * (double)b_at(pa.n_half + n, k);
    }
    const float gs = (float)gd, us = (float)ud;
    const float sg = 1.0f / (1.0f + expf(-gs));
    C[(int64_t)m * pa.ldc + n] = gs * sg * us;
    if (aux) {
      aux[(int64_t)m * pa.ld_aux + n] = gs;
      aux[(int64_t)m * pa.ld_aux + pa.n_half + n] = us;
    }
  } else {
    double accd = 0.0;
    for (int k = kbeg; k < kend; ++k) accd += (double)a_at(k) * (double)b_at(n, k);
    const float acc = (float)accd;
    if constexpr (EPI == EPI_DSWIGLU) {
      const float gv = aux[(int64_t)m * pa.ld_aux + n];
      const float uv = aux[(int64_t)m * pa.ld_aux + pa.n_half + n];
      const float sg = 1.0f / (1.0f + expf(-gv));
      aux_out[(int64_t)m * pa.ld_aux + n] = acc * uv * (sg * (1.0f + gv * (1.0f - sg)));
      aux_out[(int64_t)m * pa.ld_aux + pa.n_half + n] = acc * gv * sg;
    } else {
      float* Cg = C + (SCHED == SCHED_GROUP_K ? (int64_t)g * pa.strideC : 0);
      Cg[(int64_t)m * pa.ldc + n] = acc;
    }
  }
}

Args make_args(const GemmProblem& q) {
  Args a;
  a.A = (const bf16_t*)q.A;
  a.lda = q.lda;
  a.a_idx = q.a_idx;
  a.a_div = q.a_div > 0 ? q.a_div : 1;
  a.B = (const bf16_t*)q.B;
  a.ldb = q.ldb;
  a.strideB = q.strideB;
  a.C = (bf16_t*)q.C;
  a.ldc = q.ldc;
  a.strideC = q.strideC;
  a.aux = (bf16_t*)q.aux;
  a.aux_out = (bf16_t*)q.aux_out;
  a.ld_aux = q.ld_aux;
  a.offsets = q.offsets;
  a.G = q.G;
  a.M = (int)q.M;
  a.N = (int)q.N;
  a.K = (int)q.K;
  a.n_half = (int)q.n_half;
  return a;
}

template <int BM, int BN, int BK, int WM, int WN, bool AK, bool BKM, int SCHED, int EPI>
int run_bf16(const GemmProblem& q, hipStream_t stream) {
  Args a = make_args(q);
  const int ncols = (EPI == EPI_SWIGLU) ? (int)q.n_half : (int)q.N;
  const int tn = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  a.NTn = (ncols + tn - 1) / tn;
  int64_t slots;
  if (SCHED == SCHED_GROUP_M) {
    const int64_t mt = q.offsets ? (q.rows_bound + BM - 1) / BM + q.G : (q.M + BM - 1) / BM;
    slots = mt * a.NTn;
    a.MTk = 0;
  } else {
    a.MTk = (int)((q.M + BM - 1) / BM);
    slots = (int64_t)q.G * a.MTk * a.NTn;
  }
  if (slots <= 0) return 0;
  const size_t lds_bytes = (size_t)2 * (BM + BN) * BK * sizeof(bf16_t);
  auto kern = gemm_bf16_kernel<BM, BN, BK, WM, WN, AK, BKM, SCHED, EPI>;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)slots), dim3(WM * WN * 64), lds_bytes, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

template <int SCHED, int EPI>
int run_f32(const GemmProblem& q, hipStream_t stream) {
  Args a = make_args(q);
  const int ncols = (EPI == EPI_SWIGLU) ? (int)q.n_half : (int)q.N;
  a.NTn = (ncols + kSB - 1) / kSB;
  int64_t slots;
  if (SCHED == SCHED_GROUP_M) {
    const int64_t mt = q.offsets ? (q.rows_bound + kSB - 1) / kSB + q.G : (q.M + kSB - 1) / kSB;
    slots = mt * a.NTn;
    a.MTk = 0;
  } else {
    a.MTk = (int)((q.M + kSB - 1) / kSB);
    slots = (int64_t)q.G * a.MTk * a.NTn;
  }
  if (slots <= 0) return 0;
  hipLaunchKernelGGL((gemm_f32_kernel<SCHED, EPI>), dim3((unsigned)slots), dim3(256), 0, stream, a,
                     (const float*)q.A, (const float*)q.B, (float*)q.C, (float*)q.aux, (float*)q.aux_out,
                     q.a_kmajor, q.b_kmajor);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace

int launch_gemm(const GemmProblem& q, int bf16, hipStream_t stream) {
  if (!bf16) {
    if (q.sched == SCHED_GROUP_M) {
      if (q.epi == EPI_SWIGLU) return run_f32<SCHED_GROUP_M, EPI_SWIGLU>(q, stream);
      if (q.epi == EPI_DSWIGLU) return run_f32<SCHED_GROUP_M, EPI_DSWIGLU>(q, stream);
      return run_f32<SCHED_GROUP_M, EPI_STORE>(q, stream);  // EPI_STORE_F32: same for fp32
    }
    return run_f32<SCHED_GROUP_K, EPI_STORE>(q, stream);
  }
  // bf16 MFMA engine; the operand layouts each GEMM of the layer uses:
  if (q.sched == SCHED_GROUP_M && q.a_kmajor && q.b_kmajor) {
    if (q.epi == EPI_SWIGLU) return run_bf16<128, 128, 64, 2, 2, true, true, SCHED_GROUP_M, EPI_SWIGLU>(q, stream);
    if (q.epi == EPI_STORE_F32)
      return run_bf16<128, 128, 64, 2, 2, true, true, SCHED_GROUP_M, EPI_STORE_F32>(q, stream);
    return run_bf16<128, 128, 64, 2, 2, true, true, SCHED_GROUP_M, EPI_STORE>(q, stream);
  }
  if (q.sched == SCHED_GROUP_M && q.a_kmajor && !q.b_kmajor) {
    if (q.epi == EPI_DSWIGLU) return run_bf16<128, 128, 64, 2, 2, true, false, SCHED_GROUP_M, EPI_DSWIGLU>(q, stream);
    if (q.epi == EPI_STORE_F32)
      return run_bf16<128, 128, 64, 2, 2, true, false, SCHED_GROUP_M, EPI_STORE_F32>(q, stream);
    return run_bf16<128, 128, 64, 2, 2, true, false, SCHED_GROUP_M, EPI_STORE>(q, stream);
  }
  if (q.sched == SCHED_GROUP_K && !q.a_kmajor && !q.b_kmajor) {
    if (q.epi == EPI_STORE_F32)
      return run_bf16<128, 128, 64, 2, 2, false, false, SCHED_GROUP_K, EPI_STORE_F32>(q, stream);
    return run_bf16<128, 128, 64, 2, 2, false, false, SCHED_GROUP_K, EPI_STORE>(q, stream);
  }
  return -2;
}

}  // namespace moe
