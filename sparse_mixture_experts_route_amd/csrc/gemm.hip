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
// Kernels:
//   gemm_fwd_q64_kernel  forward GROUP_M GEMMs with K % 64 == 0: 256x256
//                        tiles, 64-wide K slices streamed global -> LDS by
//                        DMA in whole cache lines, 32x32x16 MFMAs; with an
//                        N-contiguous B (transposing fragment reads) it runs
//                        the data gradients on the weights as stored;
//   gemm_stream_kernel   forward GROUP_M GEMMs over few rows per group (decode
//                        sizes): 32-row tiles, a weight stream through LDS;
//   gemm_fwd_dma_kernel  forward GROUP_M GEMMs with K % 32 == 0 otherwise;
//   gemm_bf16_kernel     everything else (backward, ragged K): BM x BN x BK
//                        tiles with WM x WN waves, register-staged LDS
//                        double buffer, K- or MN-contiguous operands;
//   gemm_f32_kernel      the fp32 layer dtype (fp64 accumulation).
// The 16x16x32 kernels take the weight-side fragment as the MFMA A operand,
// so each lane's four accumulators are four consecutive output columns.
#include <type_traits>

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
  int c_f16;  // EPI_STORE_F32: binary16 C
  int splits;        // streaming kernel: K split over this many workgroup sets
  int slots;         // forward 256x256 kernel: tile slots to walk
  float* split_ws;   // [splits, M, N] fp32 partials when splits > 1 (SwiGLU: N = 2 n_half, gate | up)
  const bf16_t* A_lo;  // streaming kernel: the lo rows of a split operand A + A_lo (A's layout), or null
  bf16_t* C_lo;        // streaming SwiGLU epilogue: h - bf16(h) rounded to bf16 (C's layout), or null
  int fixed_stores;    // 256x256 LDS epilogues: buffer stores, a fixed count per wave (see store_tile32_lds)
  uint32_t out_bytes;  // with fixed_stores: bytes of C (M ldc 16-bit values), and of aux (M ld_aux fp32)
  uint32_t aux_bytes;
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

constexpr int kXcdGroupM = 2;  // m-tiles per XCD group (1 and 4 measured no different)

// Tile slot -> (m tile, n tile) for GROUP_M grids.  Workgroups reach the 8
// XCDs round-robin (slot b runs on XCD b % 8), and each XCD has its own L2.
// Slots are grouped as GM m-tiles x all NT n-tiles; XCD x takes groups x,
// x + 8, x + 16, ... and walks each group m-fastest, so the ~32 tiles an XCD
// runs at once form a GM x (32 / GM) block that shares A and B panels in its
// L2.  The m-tile order inside a group rotates from group to group: a
// persistent workgroup takes every 32nd slot of its XCD, and with a fixed
// order it could meet the same row of every group (at the Qwen2-MoE shape,
// 22 slots a group: half the workgroups took only the full first m-tiles of
// the experts, the other half only their mostly empty last ones).  The launch
// pads the slot count to a multiple of 8 * GM * NT.
MOE_DEV void slot_to_tile(int b, int NT, int GM, int& mt, int& nt) {
  const int x = b & 7, i = b >> 3;
  const int gt = GM * NT;
  const int q = i / gt;
  const int group = q * 8 + x;
  const int r = i % gt;
  mt = group * GM + (r % GM + q) % GM;
  nt = r / GM;
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

// Epilogue of one output tile.  Lane (lr = lane % 16, lq = lane / 16) of wave
// (wm, wn) holds, for MFMA block (fn, fm), rows m = ... + lr and the four
// consecutive columns n = ... + 4 lq + i.
template <int BM, int BN, int WM, int WN, int SCHED, int EPI, int FN, int FM>
MOE_DEV void store_tile(const Args& p, const f32x4_t (&acc)[FN][FM], int g, int row0, int row_end, int n0) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lq = lane >> 4;
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
      // the row's g, u loads first (see store_tile32)
      f32x4_t g4[FN], u4[FN];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = n0 + (wn * FN + fn) * 16 + lq * 4;
        if (col >= p.N) continue;
        const float* ga = (const float*)p.aux + (int64_t)m * p.ld_aux + col;
        g4[fn] = *(const f32x4_t*)ga;
        u4[fn] = *(const f32x4_t*)(ga + p.n_half);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = n0 + (wn * FN + fn) * 16 + lq * 4;
        if (col >= p.N) continue;
        float dg[4], du[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gval = g4[fn][i], uval = u4[fn][i];
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
        if (p.c_f16) {
          const f32x4_t v = acc[fn][fm];
          *(u32x2_t*)((f16_t*)p.C + (SCHED == SCHED_GROUP_K ? (int64_t)g * p.strideC : 0) + (int64_t)m * p.ldc +
                      col) = u32x2_t{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
        } else {
          *(f32x4_t*)(Cf + (int64_t)m * p.ldc + col) = acc[fn][fm];
        }
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

  store_tile<BM, BN, WM, WN, SCHED, EPI>(p, acc, g, row0, row_end, n0);
}

// ---------------------------------------------------------------------------
// Pipelined forward GEMM (GROUP_M, both operands K-contiguous, K % 32 == 0).
//
// Tile BM x BN x 32 with WM x WN waves.  Each K step's tile ((BM + BN) rows of
// 64 bytes) is brought into a ring of NS LDS stages by global_load_lds_dwordx4
// (lane l of a wave's DMA instruction fills bytes [16 l, 16 l + 16) of a 1 KB
// LDS block), so NS - 1 K steps are in flight without staging registers.  A
// row's four 16-byte chunks are stored XOR-swizzled (chunk ^ swz(row)) so the
// MFMA fragment reads (16 rows x one chunk per quarter-wave) spread over the
// banks; the swizzle is applied on the global-address side of the DMA.
// Per K step: wait for this wave's DMA of the step (s_waitcnt vmcnt), one
// barrier (all waves' DMA landed, previous stage free), issue the DMA of step
// kt + NS - 1 into the freed stage, then the MFMAs of step kt.
// Rows past a segment's end (and columns past N) load a clamped valid row;
// their results are never stored.
//

template <int SHIFT>
MOE_DEV int swz4(int row) {
  return SHIFT < 0 ? 0 : ((row >> (SHIFT < 0 ? 0 : SHIFT)) & 3);
}

template <int BM, int BN, int WM, int WN, int NS, int SWZ, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_fwd_dma_kernel(Args p) {
  constexpr int BK = 32;
  constexpr int NW = WM * WN;
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * BK * 2;  // bytes per ring stage
  constexpr int BLOCKS = ROWS / 16;     // 1 KB DMA blocks per stage
  constexpr int BPW = BLOCKS / NW;      // DMA instructions per wave per stage
  static_assert(BLOCKS % NW == 0 && FM >= 1 && FN >= 1 && (EPI != EPI_SWIGLU || FN % 2 == 0), "tile");
  static_assert(NS >= 2 && (NS - 2) * BPW < 64, "ring");
  extern __shared__ __attribute__((aligned(16))) char ring[];  // [NS][STAGE]
  __shared__ int s_info[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  int g, row0, row_end;
  const int nt = blockIdx.x % p.NTn;
  const int mt = blockIdx.x / p.NTn;
  if (!find_group_m<BM>(p, mt, s_info, g, row0, row_end)) return;
  const int n0 = nt * ((EPI == EPI_SWIGLU) ? BN / 2 : BN);
  const bf16_t* Bg = p.B + (int64_t)g * p.strideB;

  // DMA source of each of this wave's BPW blocks: tile row rr = 16 b + lane / 4,
  // logical chunk (lane % 4) ^ swz(rr).
  const bf16_t* src[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int rr = (wave * BPW + i) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ swz4<SWZ>(rr);
    if (rr < BM) {
      const int m = min(row0 + rr, row_end - 1);
      const int64_t srow = p.a_idx ? (int64_t)(p.a_idx[m] / p.a_div) : (int64_t)m;
      src[i] = p.A + srow * p.lda + chunk * 8;
    } else {
      const int j = rr - BM;
      int n;
      if constexpr (EPI == EPI_SWIGLU) {
        constexpr int half = BN / 2;
        const int c = min(n0 + (j % half), p.n_half - 1);
        n = (j < half) ? c : p.n_half + c;
      } else {
        n = min(n0 + j, p.N - 1);
      }
      src[i] = Bg + (int64_t)n * p.ldb + chunk * 8;
    }
  }
  auto issue = [&](int kstep, int stage) {
    char* base = ring + stage * STAGE + wave * BPW * 1024;
#pragma unroll
    for (int i = 0; i < BPW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + kstep * BK),
                                       (__attribute__((address_space(3))) void*)(base + i * 1024), 16, 0, 0);
  };

  f32x4_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15, lq = lane >> 4;
  int a_off[FM], b_off[FN];  // byte offsets of this lane's fragments inside a stage
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int rr = wm * (BM / WM) + fm * 16 + lr;
    a_off[fm] = rr * 64 + ((lq ^ swz4<SWZ>(rr)) * 16);
  }
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    int blk;
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int H2 = FN / 2;
      blk = (fn < H2) ? (wn * H2 + fn) : (BN / 32 + wn * H2 + (fn - H2));
    } else {
      blk = wn * FN + fn;
    }
    const int rr = BM + blk * 16 + lr;
    b_off[fn] = rr * 64 + ((lq ^ swz4<SWZ>(rr)) * 16);
  }

  const int nk = p.K / BK;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    const int ahead = nk - 1 - kt;  // steps already issued after kt: min(NS - 2, ahead)
    if (ahead >= NS - 2) {
      wait_vmcnt<(NS - 2) * BPW>();
    } else if constexpr (NS >= 4) {
      if (ahead == 2) wait_vmcnt<2 * BPW>();
      else if (ahead == 1) wait_vmcnt<BPW>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    ring_barrier();
    if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);
    const char* st = ring + (kt % NS) * STAGE;
    bf16x8_t af[FM], bfr[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) af[fm] = *(const bf16x8_t*)(st + a_off[fm]);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) bfr[fn] = *(const bf16x8_t*)(st + b_off[fn]);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        acc[fn][fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[fn], af[fm], acc[fn][fm], 0, 0, 0);
    // issue every fragment read of the step before its MFMAs, so the reads
    // stream in while the first MFMAs run
    __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
  }
  store_tile<BM, BN, WM, WN, SCHED_GROUP_M, EPI>(p, acc, g, row0, row_end, n0);
}

template <int BM, int BN, int WM, int WN, int NS, int SWZ, int EPI>
int run_fwd_dma(const GemmProblem& q, hipStream_t stream);

// ---------------------------------------------------------------------------
// 32x32 variant of the pipelined forward GEMM: v_mfma_f32_32x32x16_bf16 (one
// instruction does twice the work of 16x16x32, so a single wave per SIMD can
// keep the matrix core busy).  A lane holds 8 consecutive k of row (lane % 32)
// at k offset 8 * (lane / 32) of a 16-wide k substep; the 32x32 result holds,
// for r = 0..15, row 8 (r / 4) + 4 (lane / 32) + r % 4 and column lane % 32.
// With the weight fragment as the MFMA A operand, each lane therefore owns
// four runs of four consecutive output columns of one output row.
template <int BM, int BN, int WM, int WN, int SCHED, int EPI, int FN, int FM>
MOE_DEV void store_tile32(const Args& p, const f32x16_t (&acc)[FN][FM], int g, int row0, int row_end, int n0,
                          int sp = 0) {
  static_assert(EPI != EPI_DSWIGLU, "the SwiGLU-backward epilogue of the 32x32 tiles is dswiglu_tile_lds");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lm = lane & 31, lh = lane >> 5;
  bf16_t* Cg = p.C + (SCHED == SCHED_GROUP_K ? (int64_t)g * p.strideC : 0);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = row0 + wm * (BM / WM) + fm * 32 + lm;
    if (m >= row_end) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int H2 = FN / 2;
#pragma unroll
      for (int fn = 0; fn < H2; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + (wn * H2 + fn) * 32 + q * 8 + lh * 4;
          if (col >= p.n_half) continue;
          f32x4_t gv, uv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            gv[i] = acc[fn][fm][q * 4 + i];
            uv[i] = acc[fn + H2][fm][q * 4 + i];
          }
          float h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = gv[i] * fast_sigmoid(gv[i]) * uv[i];
          u32x2_t hv = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
          *(u32x2_t*)(Cg + (int64_t)m * p.ldc + col) = hv;
          if (p.aux) {
            float* ga = (float*)p.aux + (int64_t)m * p.ld_aux + col;
            *(f32x4_t*)ga = gv;
            *(f32x4_t*)(ga + p.n_half) = uv;
          }
        }
    } else {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + (wn * FN + fn) * 32 + q * 8 + lh * 4;
          if (col >= p.N) continue;
          f32x4_t v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[fn][fm][q * 4 + i];
          if constexpr (EPI == EPI_STORE_F32) {
            const int64_t off = (SCHED == SCHED_GROUP_K ? (int64_t)g * p.strideC : 0) + (int64_t)m * p.ldc + col;
            if (p.splits > 1)  // K-split partial of split sp (split_reduce_kernel stores C)
              *(f32x4_t*)(p.split_ws + ((int64_t)sp * p.M + m) * p.N + col) = v;
            else if (p.c_f16)
              *(u32x2_t*)((f16_t*)p.C + off) = u32x2_t{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
            else
              *(f32x4_t*)((float*)p.C + off) = v;
          } else {
            u32x2_t o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *(u32x2_t*)(Cg + (int64_t)m * p.ldc + col) = o;
          }
        }
    }
  }
}

// Tile slot -> (group, first row, row limit) for GROUP_M, computed by every
// wave on its own (no LDS, no barrier): the same scan over per-group tile
// counts as find_group_m, with the owning lane found by a ballot.
template <int BM>
MOE_DEV bool find_group_m_wave(const Args& p, int mt, int& g, int& row0, int& row_end) {
  if (p.offsets == nullptr) {
    g = 0;
    row0 = mt * BM;
    row_end = p.M;
    return row0 < p.M;
  }
  const int lane = threadIdx.x & 63;
  int c[4];
  int local = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gi = lane * 4 + r;
    c[r] = 0;
    if (gi < p.G) c[r] = (p.offsets[gi + 1] - p.offsets[gi] + BM - 1) / BM;
    local += c[r];
  }
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  const int excl = incl - local;
  const bool mine = mt >= excl && mt < incl;
  const unsigned long long own = __ballot(mine);
  if (own == 0) return false;
  int gs = 0, r0 = 0, re = 0;
  if (mine) {
    int acc = excl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (mt >= acc && mt < acc + c[r]) {
        gs = lane * 4 + r;
        r0 = p.offsets[gs] + (mt - acc) * BM;
        re = p.offsets[gs + 1];
      }
      acc += c[r];
    }
  }
  const int src = __ffsll(own) - 1;
  g = __builtin_amdgcn_readfirstlane(__shfl(gs, src, 64));
  row0 = __builtin_amdgcn_readfirstlane(__shfl(r0, src, 64));
  row_end = __builtin_amdgcn_readfirstlane(__shfl(re, src, 64));
  return true;
}

// ---------------------------------------------------------------------------
// Forward GEMM with 64-wide K slices: a 256x256 output tile per workgroup,
// 2 x WN waves each owning a 128 x (256 / WN) block as 32x32 blocks of
// v_mfma_f32_32x32x16_bf16 accumulators (WN = 4: 8 waves, two per SIMD, so
// one wave's MFMAs run while the other waits on a DMA issue or an LDS read).
// Operands stream into LDS by global_load_lds_dwordx4 with every row segment
// a full 128-byte line (64 bf16 of K): the L2 serves whole-line requests at a
// markedly higher rate than half-line ones.  A slice is two 32 KB units (A
// rows, then B rows); the ring holds 5 units (160 KB), so while slice kt is
// consumed, slice kt + 1 and half of slice kt + 2 are resident or in flight.
// Unit u = 2 kt + (0 for A, 1 for B) lives in slot u % 5.  Unit row r keeps
// its eight 16-byte chunks at r * 128 + (c ^ sw(r)) * 16 with
// sw(r) = ((r >> 1) ^ ((r & 1) << 2)) & 7, so a fragment read (32 rows, one
// chunk each) hits distinct banks in every 8- or 16-lane phase.  Each lane's
// DMA source is a fixed 32-bit offset from a wave-uniform base that advances
// along K.  Step kt runs four 16-wide substeps; each substep's MFMAs overlap
// the fragment reads of the next substep:
//   substeps 0-1: MFMAs of (kt, s), read (kt, s + 2);
//   wait for units 2 kt + 2, 2 kt + 3 (this wave's DMA count), barrier;
//   DMA units 2 kt + 5, 2 kt + 6 into the slots of units 2 kt, 2 kt + 1;
//   substeps 2-3: MFMAs of (kt, s), read (kt + 1, s - 2).
// Fragments are read two substeps ahead (three fragment sets rotate, so the
// slice loop is unrolled by three).
// Units past the last slice re-read the last slice into slots nobody reads.
MOE_DEV int swz8(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

// The lo parts of four values: v - bf16(v), each rounded to bf16 (0 where v
// is not finite), packed as the hi parts are by pack_bf16x2.
MOE_DEV u32x2_t lo_pair(const float (&v)[4]) {
  float lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float hi = bf16_to_f32(f32_to_bf16(v[i]));
    lo[i] = __builtin_isfinite(v[i]) ? v[i] - hi : 0.0f;
  }
  return u32x2_t{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])};
}

// GROUPED: tiles come from per-group segment offsets (routed experts);
// otherwise one group of M rows (the shared expert).
// 16-bit epilogue of the 256x256 tile through LDS.  A lane's accumulators
// cover four columns of one row per 32x32 block, so direct stores touch 32
// rows (32 cache lines) per instruction with 16 bytes each; here every wave
// first writes its converted block into a row-major copy of the tile in the
// (then idle) part of the ring at `lds`, and after one barrier the
// workgroup stores whole rows: 8 lanes per 128-byte line, full lines only.
// Rows of the copy are OW * 2 bytes, 16-byte chunk c of row r sits at chunk
// c ^ (r % CH) (the 32 rows one write instruction covers spread over
// distinct chunks).  A pass stages at most 64 KB (the caller's DMA of the
// next tile may fill the rest of the ring): the 256 rows of h at once, 256
// 16-bit columns and the saved fp32 g, u rows one wave row (128 rows) at a
// time.  Applies to EPI_STORE, binary16 EPI_STORE_F32 without K split, and
// the h output of EPI_SWIGLU (and its fp32 g, u copy, when requested).
// On entry every wave is past the barrier that ends the tile's ring reads;
// the caller's barrier after it keeps the next tile's later DMA out.
template <int BM, int BN, int WM, int WN, int EPI, int FN, int FM>
MOE_DEV void store_tile32_lds(const Args& p, const f32x16_t (&acc)[FN][FM], int row0, int row_end, int n0,
                              char* lds) {
  constexpr int OW = (EPI == EPI_SWIGLU) ? BN / 2 : BN;  // output columns of the tile
  constexpr int RB = OW * 2, CH = RB / 16;
  constexpr int HR = BM / WM;  // rows of one wave row (wm) of the tile
  // opaque copy of the thread index: keeps the address arithmetic below from
  // being hoisted out of the tile loop, where it would hold registers
  // through the main loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lm = lane & 31, lh = lane >> 5;
  const bool f16 = (EPI == EPI_STORE_F32);
  constexpr int NT = 64 * WM * WN;
  const int nout = (EPI == EPI_SWIGLU) ? p.n_half : p.N;
  char* C = (char*)p.C;
  // with fixed_stores: C's range is its out_bytes (under 2^31, checked on
  // the host); a chunk outside the output goes to offset out_bytes, past the
  // range, and the hardware drops it
  const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(C, (short)0, (int)p.out_bytes, 0x00020000);
  // every pass stages at most 64 KB: the h tile (256 rows x 256 bytes) at
  // once, 256 16-bit columns (512 bytes a row) and the saved fp32 rows (512
  // bytes of gate or up a row) one wave row (128 rows) at a time
  constexpr int PASSES = (EPI == EPI_SWIGLU) ? 1 : WM;
#pragma unroll
  for (int h = 0; h < PASSES; ++h) {
    if (PASSES == 1 || wm == h) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = (PASSES == 1 ? wm * HR : 0) + fm * 32 + lm;  // staging row
        char* row = lds + r * RB + lh * 8;
        const int rs = r & (CH - 1);
        if constexpr (EPI == EPI_SWIGLU) {
          constexpr int H2 = FN / 2;
#pragma unroll
          for (int fn = 0; fn < H2; ++fn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c8 = (wn * H2 + fn) * 4 + q;  // 8-column chunk within the tile
              f32x4_t gv, uv;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                gv[i] = acc[fn][fm][q * 4 + i];
                uv[i] = acc[fn + H2][fm][q * 4 + i];
              }
              float hv[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) hv[i] = gv[i] * fast_sigmoid(gv[i]) * uv[i];
              *(u32x2_t*)(row + ((c8 ^ rs) << 4)) = u32x2_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
            }
        } else {
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c8 = (wn * FN + fn) * 4 + q;
              const f32x16_t& a = acc[fn][fm];
              const u32x2_t o = f16 ? u32x2_t{pack_f16x2(a[q * 4], a[q * 4 + 1]), pack_f16x2(a[q * 4 + 2], a[q * 4 + 3])}
                                    : u32x2_t{pack_bf16x2(a[q * 4], a[q * 4 + 1]), pack_bf16x2(a[q * 4 + 2], a[q * 4 + 3])};
              *(u32x2_t*)(row + ((c8 ^ rs) << 4)) = o;
            }
        }
      }
    }
    // LDS writes of every wave complete (vmcnt and expcnt left alone)
    __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));
    ring_barrier();
    constexpr int ROWS = BM / PASSES;
    if (p.fixed_stores) {
      // every lane stores each of its chunks, those outside the output at an
      // offset past the buffer's range (dropped): a fixed count of vector
      // memory instructions per wave, which the next tile's first wait counts
#pragma unroll 4
      for (int id = tid; id < ROWS * CH; id += NT) {
        const int r = id / CH, c = id % CH;
        const int m = row0 + h * ROWS + r;
        const int col = n0 + c * 8;
        const u32x4_t v = *(const u32x4_t*)(lds + r * RB + ((c ^ (r & (CH - 1))) << 4));
        const bool in = m < row_end && col < nout;
        const uint32_t off = in ? (uint32_t)(((int64_t)m * p.ldc + col) * 2) : p.out_bytes;
        __builtin_amdgcn_raw_buffer_store_b128(v, out_rsrc, (int)off, 0, 2);
      }
    } else {
#pragma unroll 4
      for (int id = tid; id < ROWS * CH; id += NT) {
        const int r = id / CH, c = id % CH;
        const int m = row0 + h * ROWS + r;
        const int col = n0 + c * 8;
        const u32x4_t v = *(const u32x4_t*)(lds + r * RB + ((c ^ (r & (CH - 1))) << 4));
        if (m >= row_end || col >= nout) continue;
        char* dst = C + ((int64_t)m * p.ldc + col) * 2;
        if (col + 8 <= nout) {
          __builtin_nontemporal_store(v, (u32x4_t*)dst);
        } else {
          *(u32x2_t*)dst = u32x2_t{v[0], v[1]};
        }
      }
    }
    if (h + 1 < PASSES) {
      __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));  // LDS reads done
      ring_barrier();
    }
  }
  if constexpr (EPI == EPI_SWIGLU) {
    if (p.aux) {
      // the saved fp32 gate rows, then the up rows: per part, one wave row
      // (128 rows of 128 columns, 512 bytes, 32 chunks at c ^ (r % 32)) a pass
      constexpr int H2 = FN / 2, GB = (BN / 2) * 4, GC = GB / 16;
#pragma unroll
      for (int part = 0; part < 2; ++part) {
#pragma unroll
        for (int h = 0; h < WM; ++h) {
          __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));  // earlier LDS reads done
          ring_barrier();
          if (wm == h) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
              const int r = fm * 32 + lm;
              char* row = lds + r * GB;
#pragma unroll
              for (int fn = 0; fn < H2; ++fn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const int c = ((wn * H2 + fn) * 4 + q) * 2 + lh;  // 4-column chunk within the 128
                  const f32x16_t& a = acc[fn + part * H2][fm];
                  *(f32x4_t*)(row + ((c ^ (r & (GC - 1))) << 4)) =
                      f32x4_t{a[q * 4], a[q * 4 + 1], a[q * 4 + 2], a[q * 4 + 3]};
                }
            }
          }
          __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));  // LDS writes done
          ring_barrier();
          float* aux = (float*)p.aux + part * p.n_half;
          if (p.fixed_stores) {
            const uint32_t part_bytes = p.aux_bytes - (uint32_t)(part * p.n_half * 4);  // from this part's base
            const __amdgpu_buffer_rsrc_t aux_rsrc =
                __builtin_amdgcn_make_buffer_rsrc(aux, (short)0, (int)part_bytes, 0x00020000);
#pragma unroll 4
            for (int id = tid; id < HR * GC; id += NT) {
              const int r = id / GC, c = id % GC;
              const int m = row0 + h * HR + r, col = n0 + c * 4;
              const f32x4_t v = *(const f32x4_t*)(lds + r * GB + ((c ^ (r & (GC - 1))) << 4));
              const bool in = m < row_end && col < p.n_half;
              const uint32_t off = in ? (uint32_t)(((int64_t)m * p.ld_aux + col) * 4) : part_bytes;
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), aux_rsrc, (int)off, 0, 2);
            }
          } else {
#pragma unroll 4
            for (int id = tid; id < HR * GC; id += NT) {
              const int r = id / GC, c = id % GC;
              const int m = row0 + h * HR + r, col = n0 + c * 4;
              const f32x4_t v = *(const f32x4_t*)(lds + r * GB + ((c ^ (r & (GC - 1))) << 4));
              if (m >= row_end || col >= p.n_half) continue;
              __builtin_nontemporal_store(v, (f32x4_t*)(aux + (int64_t)m * p.ld_aux + col));
            }
          }
        }
      }
    }
  }
}

// SwiGLU-backward epilogue of the 256x256 tile through LDS.  The direct
// form loads the saved fp32 g, u in the accumulator layout: every load
// instruction touches 32 rows with 32 bytes each, and every store 32 rows
// with 16 bytes.  Here the tile's rows go in four passes of 64 (rows
// wm 128 + fm 32 + lm for both wave rows wm, so all eight waves work in each
// pass): the g and u rows of the pass (the tile's 256 columns, 1 KB each)
// come by DMA of whole rows into the ring (16-byte chunk c of staging row s
// at chunk c ^ (s % 16), so the 32 rows one fragment read covers spread over
// the banks), every lane computes its dg, du from them and its accumulators
// with the direct form's arithmetic, and as soon as those reads are done the
// DMA of the next pass's g, u is issued; meanwhile dg and then du are
// written as bf16 into a row-major copy (chunk c ^ (s % 32)) and stored as
// whole 16-byte chunks of whole rows.  The stores are buffer stores of a
// fixed count per lane (chunks outside the output go to the offset equal to
// the output's range and are dropped), so the wait for the next pass's DMA,
// which was issued before them, can leave them in flight.  Rows past the
// segment and columns past the output are loaded out of range (nothing is
// read: the descriptors, based at the tile's first row, carry the byte range
// of the rows from there to M) and never stored.  The DMA is the asm form, which the kernels with
// transposing fragment reads need.  On entry the ring is free (every wave
// past the barrier that ends the tile's ring reads; no early DMA of the
// next tile); on exit every staging read is done.
template <int BM, int BN, int WM, int WN, int FN, int FM>
MOE_DEV void dswiglu_tile_lds(const Args& p, const f32x16_t (&acc)[FN][FM], int row0, int row_end, int n0,
                              char* lds) {
  static_assert(BN == 256 && FN * WN * 32 == BN && FM * 32 * WM == BM, "tile shape");
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int PR = 32 * WM;             // staging rows a pass
  constexpr int RB = BN * 4;              // one fp32 row of g (or u) over the tile's columns: 1 KB
  constexpr int OB = BN * 2;              // one bf16 row of dg (or du): 512 bytes, 32 chunks
  constexpr int HR = BM / WM;
  constexpr int SPL = PR * 32 / NT;       // stores a lane per part and pass
  static_assert(PR * 32 % NT == 0 && 32 % (PR / NW) == 0, "store count, DMA rows a wave");
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // keeps the address arithmetic inside the tile loop
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lm = lane & 31, lh = lane >> 5;
  char* const G = lds;                 // g rows of the pass
  char* const U = lds + PR * RB;       // u rows of the pass
  char* const S = lds + 2 * PR * RB;   // dg (then du) rows of the pass, bf16
  // descriptors based at the tile's first row, their range the rows from
  // there to M (at most 2^31 bytes; a tile's 256 rows lie well inside)
  // wave-uniform tile bounds, held in scalar registers
  const int r0s = __builtin_amdgcn_readfirstlane(row0);
  const int nrs = __builtin_amdgcn_readfirstlane(row_end - row0);  // rows of the segment in the tile
  const int64_t rows_left = (int64_t)p.M - r0s;
  const uint32_t g_range = (uint32_t)min(rows_left * p.ld_aux * 4, (int64_t)1 << 31);
  const uint32_t u_range = g_range - (uint32_t)p.n_half * 4;
  const uint32_t o_range = (uint32_t)min(rows_left * p.ld_aux * 2, (int64_t)1 << 31);
  const char* gbase = (const char*)p.aux + (int64_t)r0s * p.ld_aux * 4;
  const i32x4_t gr = dma_rsrc_words(gbase, g_range);
  const i32x4_t ur = dma_rsrc_words(gbase + (int64_t)p.n_half * 4, u_range);
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      p.aux_out + (int64_t)r0s * p.ld_aux, (short)0, (int)o_range, 0x00020000);
  // wave w loads staging rows w PR / NW .. + PR / NW - 1 of g and of u: the
  // row's byte offset (wave-uniform) in the scalar offset, the lane's column
  // in the vector offset; a row past the segment or a column past n_half
  // takes the range as its vector offset (out of range: nothing is read)
  // rows relative to the tile's first row
  const int wrow = __builtin_amdgcn_readfirstlane((wave * (PR / NW) / 32) * HR + (wave * (PR / NW)) % 32);
  const int wend = nrs;
  auto dma_pass = [&](int fm) {
#pragma unroll
    for (int i = 0; i < PR / NW; ++i) {
      const int s = wave * (PR / NW) + i;
      const int m = wrow + fm * 32 + i;  // PR / NW rows of one wave stay inside one 32-row block
      const bool in = m < wend;
      const int col = n0 + 4 * (lane ^ (s & 15));  // the source chunk this lane's 16 bytes hold
      const bool cin = in && col < p.n_half;
      const uint32_t so = in ? (uint32_t)m * (uint32_t)p.ld_aux * 4u : 0u;
      dma16_hidden_so(gr, cin ? (uint32_t)col * 4u : g_range, so, G + s * RB);
      dma16_hidden_so(ur, cin ? (uint32_t)col * 4u : u_range, so, U + s * RB);
    }
  };
  // one part (0: dg, 1: du) of the pass from S: SPL chunks a lane
  auto store_part = [&](int fm, int part) {
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const int id = tid + j * NT;
      const int r = id / 32, c = id % 32;
      const int m = (r / 32) * HR + fm * 32 + (r % 32);  // from the tile's first row
      const int col = n0 + c * 8;
      const u32x4_t v = *(const u32x4_t*)(S + r * OB + ((c ^ (r & 31)) << 4));
      const bool in = m < nrs && col < p.n_half;  // n_half % 8 == 0: whole chunks
      const uint32_t off = in ? (uint32_t)((m * p.ld_aux + part * p.n_half + col) * 2) : o_range;
      __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, (int)off, 0, 2);
    }
  };
  dma_pass(0);
#pragma unroll  // acc[.][fm] needs a compile-time fm
  for (int fm = 0; fm < FM; ++fm) {
    // this pass's g, u landed (the previous pass's 2 SPL stores, issued after
    // that DMA, may still be in flight)
    if (fm == 0)
      wait_vmcnt<0>();
    else
      wait_vmcnt<2 * SPL>();
    ring_barrier();
    const int s = wm * 32 + lm;  // this lane's staging row
    u32x2_t dg2[FN][4], du2[FN][4];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = (wn * FN + fn) * 8 + q * 2 + lh;  // 16-byte chunk: columns 4 c .. 4 c + 3
        const f32x4_t gv = *(const f32x4_t*)(G + s * RB + ((c ^ (s & 15)) << 4));
        const f32x4_t uv = *(const f32x4_t*)(U + s * RB + ((c ^ (s & 15)) << 4));
        float dg[4], du[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gval = gv[i], uval = uv[i];
          const float sg = fast_sigmoid(gval);
          const float dh = acc[fn][fm][q * 4 + i];
          du[i] = dh * gval * sg;
          dg[i] = dh * uval * (sg * (1.0f + gval * (1.0f - sg)));
        }
        dg2[fn][q] = u32x2_t{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
        du2[fn][q] = u32x2_t{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
      }
    __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));  // reads of g, u done
    ring_barrier();
    if (fm + 1 < FM) dma_pass(fm + 1);
#pragma unroll
    for (int part = 0; part < 2; ++part) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c8 = (wn * FN + fn) * 4 + q;  // 8-column chunk of the output row
          *(u32x2_t*)(S + s * OB + ((c8 ^ (s & 31)) << 4) + lh * 8) = part ? du2[fn][q] : dg2[fn][q];
        }
      __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));  // staging writes done
      ring_barrier();
      store_part(fm, part);
      __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));  // staging reads done
      ring_barrier();
    }
  }
}

// An operand tile held k-row-major in LDS: row k of 256 16-bit values (512
// bytes), its 16-byte chunk c stored at c ^ 4 (k % 4), so that one transposing
// read (16 lanes, 4 columns of a row each) hits distinct bank windows; the
// value (k, col) sits at byte
//   kmaj_off(k, col) = 512 k + 16 ((col / 8) ^ 4 (k % 4)) + 2 (col % 8).

// The 32x32x16 MFMA fragment of columns c0 .. c0 + 31 at k-rows k0 .. k0 + 15
// of a k-row-major LDS tile, by two ds_read_b64_tr_b16 per lane: lane group
// G = lane / 16 covers k half G / 2 and column half G % 2; within a group,
// lane s addresses 4 columns of row k0 + 8 (G / 2) + s / 4 (+ 4 for the
// second read) and lane l receives rows .. + 3 of one column, so lane l ends
// up with the 8 consecutive k of column l % 32 at k offset 8 (l / 32).
// `unit` + kmaj_off(kq, cq) with kq = k0 + 8 (G / 2) + (lane % 16) / 4 and
// cq = c0 + 16 (G % 2) + 4 (lane % 4) is this lane's first address, the
// second 4 k-rows (2048 bytes) further.  With k0 a multiple of 16 and c0 of
// 32 that first address is
//   unit + 512 k0 + frag_lane_off(kl, cl) + 64 ((c0 / 32) ^ (kl % 4))
// for kl = kq - k0, cl = cq - c0, since the swizzle only flips the low two
// bits of the 32-column block: one per-lane base per column block, the k
// offset an immediate of the read.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
MOE_DEV int frag_lane_off(int kl, int cl) { return kl * 512 + (cl >> 3) * 16 + (cl & 7) * 2; }
MOE_DEV bf16x8_t tr_frag32_at(const char* a) {
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)a);
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(a + 2048));
  const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// LDS_EPI: 16-bit output through store_tile32_lds (chosen on the host).
// BT: B is N-contiguous in memory (B(n, k) at B[k ldb + n]: the data-gradient
// GEMMs reading the expert weights as stored); its units hold 64 k-rows of
// the tile's 256 columns and its fragments come from transposing LDS reads.
// The DMA is then the hidden (asm) form, which the transposing reads need.
template <int WN, bool GROUPED, int EPI, bool LDS_EPI, bool BT>
__global__ __launch_bounds__(128 * WN) __attribute__((amdgpu_waves_per_eu(WN / 2, WN / 2))) void gemm_fwd_q64_kernel(Args p) {
  constexpr int BM = 256, BN = 256, BK = 64, WM = 2;
  constexpr int NW = WM * WN;                 // 4 (one wave per SIMD) or 8 (two)
  constexpr int FM = 4, FN = BN / WN / 32;    // 32x32 blocks per wave
  constexpr int UNIT = 256 * BK * 2;          // 32 KB
  constexpr int NU = 5;                       // ring slots
  constexpr int IPW = UNIT / 1024 / NW;       // DMA instructions per wave per unit
  static_assert(WN == 2 || WN == 4, "wave grid");
  static_assert(!BT || EPI != EPI_SWIGLU, "N-contiguous B: data-gradient epilogues only");
  extern __shared__ __attribute__((aligned(16))) char ring[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // tile slots slot = blockIdx.x, blockIdx.x + gridDim.x, ... (one slot per
  // workgroup when the grid covers every slot; a persistent grid of one
  // workgroup per CU walks them, the next tile's DMA issued right after
  // this tile's epilogue stores); gridDim.x is a multiple of 8, so a slot's
  // XCD is that of its workgroup
  // with a K split (one group, too few tiles for the CUs), slot = sp * base
  // + tile slot, and split sp covers slices [sp nk / splits, (sp + 1) nk /
  // splits); base is a multiple of 8, so a tile slot keeps its XCD
  const int base_slots = p.slots / p.splits;
  // The DMA of a tile: operand bases and this lane's 32-bit source offsets.
  struct TileDma {
    const char* abase;
    const char* bbase;
    uint32_t aoff[IPW], boff[IPW];
    int nk;
  };
  // Tile of slot `slot`: false when the slot has no tile (a padding slot of
  // the grouped bound); else its rows, first output column and DMA.
  auto tile_of = [&](int slot, int& g, int& row0, int& row_end, int& n0, int& sp, TileDma& d) -> bool {
    sp = slot / base_slots;
    int mt, nt;
    slot_to_tile(slot - sp * base_slots, p.NTn, kXcdGroupM, mt, nt);
    if constexpr (GROUPED) {
      if (!find_group_m_wave<BM>(p, mt, g, row0, row_end)) return false;
    } else {
      g = 0;
      row0 = mt * BM;
      row_end = p.M;
      if (row0 >= p.M) return false;
    }
    n0 = nt * ((EPI == EPI_SWIGLU) ? BN / 2 : BN);
    // DMA: instruction i of this wave covers unit rows 8 (IPW wave + i) .. + 7;
    // lane reads row 8 (IPW wave + i) + lane / 8, logical chunk (lane % 8) ^ sw.
    const int nk_all = p.K / BK;
    const int kb = sp * nk_all / p.splits;
    d.abase = (const char*)p.A + (int64_t)kb * (BK * 2);
    d.bbase = (const char*)(p.B + (int64_t)g * p.strideB) + (int64_t)kb * BK * (BT ? p.ldb * 2 : 2);
  #pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int rr = (wave * IPW + i) * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ swz8(rr);
      const int m = min(row0 + rr, row_end - 1);
      const int64_t arow = p.a_idx ? (int64_t)(p.a_idx[m] / p.a_div) : (int64_t)m;
      d.aoff[i] = (uint32_t)((arow * p.lda + chunk * 8) * 2);
      if constexpr (BT) {
        // instruction i covers k-rows 2 (IPW wave + i) + {0, 1} of the unit;
        // lane: k-row + lane / 32, physical chunk lane % 32 holding logical
        // 8-column chunk (lane % 32) ^ 4 (k % 4); columns clamped inside N
        const int kr = 2 * (IPW * wave + i) + (lane >> 5);
        const int n = min(n0 + (((lane & 31) ^ (4 * (kr & 3))) << 3), p.N - 8);
        d.boff[i] = (uint32_t)(((int64_t)kr * p.ldb + n) * 2);
      } else {
        int n;
        if constexpr (EPI == EPI_SWIGLU) {
          const int c = min(n0 + (rr & 127), p.n_half - 1);
          n = (rr < 128) ? c : p.n_half + c;
        } else {
          n = min(n0 + rr, p.N - 1);
        }
        d.boff[i] = (uint32_t)(((int64_t)n * p.ldb + chunk * 8) * 2);
      }
    }
    d.nk = (sp + 1) * nk_all / p.splits - kb;
    return true;
  };
  const int bstep = BT ? BK * (int)p.ldb * 2 : BK * 2;  // bytes from one B slice to the next
  // unit u of a tile (A rows of slice u / 2 for even u, B rows for odd) into ring slot u % NU
  auto issue_unit = [&](const TileDma& d, int u) {
    const int slice = min(u >> 1, d.nk - 1);
    char* dst = ring + (u % NU) * UNIT + wave * (IPW * 1024);
    const bool is_b = u & 1;
    if constexpr (BT) {
      const i32x4_t r = dma_rsrc_words(is_b ? d.bbase : d.abase);
      const uint32_t so = (uint32_t)slice * (uint32_t)(is_b ? bstep : BK * 2);
  #pragma unroll
      for (int i = 0; i < IPW; ++i) dma16_hidden(r, (is_b ? d.boff[i] : d.aoff[i]) + so, dst + i * 1024);
    } else {
      const __amdgpu_buffer_rsrc_t r = dma_rsrc(is_b ? d.bbase : d.abase);
      const int soff = slice * (BK * 2);
  #pragma unroll
      for (int i = 0; i < IPW; ++i) dma16(r, is_b ? d.boff[i] : d.aoff[i], soff, dst + i * 1024);
    }
  };
  // Ring units of the next tile whose DMA is issued before this tile's
  // epilogue: three before an LDS epilogue (its passes stage at most 64 KB,
  // in the top two units), all five before one that stores from registers,
  // none before the SwiGLU-backward epilogue, whose loads of the saved g, u
  // would queue behind that DMA (vector memory completes in issue order).
  const int early = EPI == EPI_DSWIGLU ? 0 : !LDS_EPI ? NU : NU - 2;
  // this workgroup's tiles: slots blockIdx.x, blockIdx.x + gridDim.x, ...
  // (those without a tile skipped); the next tile's mapping and DMA offsets
  // are found before the current tile's epilogue (the row-index loads of a
  // gathered A wait for every vector memory operation before them) and kept
  int slot = blockIdx.x;
  int g, row0, row_end, n0, sp;
  TileDma dm;
  while (slot < p.slots && !tile_of(slot, g, row0, row_end, n0, sp, dm)) slot += gridDim.x;
  int pend = 0;  // units of this tile issued by the previous one
  while (slot < p.slots) {
    const int nk = dm.nk;
    int issued = 0;  // units issued so far
    auto issue = [&]() {
      issue_unit(dm, issued);
      ++issued;
    };

    const int lm = lane & 31, lh = lane >> 5;
    const int sw = swz8(lm);
    const int a_row = (wm * (BM / WM) + lm) * 128;
    // transposing reads (BT): this lane's k-row and column offsets
    const int tr_k = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto b_blk = [&](int fn) -> int {
      if constexpr (EPI == EPI_SWIGLU) {
        constexpr int H2 = FN / 2;
        return (fn < H2) ? (wn * H2 + fn) : (BN / 64 + wn * H2 + (fn - H2));
      } else {
        return wn * FN + fn;
      }
    };
    // transposing reads (BT): this lane's first address in a B unit for
    // fragment fn, less the substep's 16 k-rows (8192 bytes each)
    int tr_base[FN];
    if constexpr (BT) {
  #pragma unroll
      for (int fn = 0; fn < FN; ++fn) tr_base[fn] = frag_lane_off(tr_k, tr_c) + 64 * (b_blk(fn) ^ (tr_k & 3));
    }
    struct Frags {
      bf16x8_t a[FM], b[FN];
    };
    f32x16_t acc[FN][FM];
  #pragma unroll
    for (int i = 0; i < FN; ++i)
  #pragma unroll
      for (int j = 0; j < FM; ++j)
  #pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // 32-row blocks of this wave that hold rows of the segment: a segment's
    // last tile is mostly padding, and there a wave skips the MFMAs and A
    // fragment reads of empty blocks (its SIMD partner's MFMAs then run back
    // to back).  Full tiles take the loop compiled with every block active.
    const int fa = min(FM, max(0, (row_end - row0 - wm * (BM / WM) + 31) / 32));
    auto main_loop = [&](auto all_blocks) {
      constexpr bool FULL = decltype(all_blocks)::value;
      // substep s of slice kt: logical chunk 2 s + lh
      auto read_sub = [&](int kt, int s, Frags& f) {
        const int ua = (2 * kt) % NU;
        const int ub = ua + 1 == NU ? 0 : ua + 1;
        const int ch = ((2 * s + lh) ^ sw) * 16;
        const char* sa = ring + ua * UNIT + a_row + ch;
        const char* sb = ring + ub * UNIT + lm * 128 + ch;
        if (!FULL && fa == 0) return;
  #pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          if (FULL || fm < fa) f.a[fm] = *(const bf16x8_t*)(sa + fm * 32 * 128);
        if constexpr (BT) {
          const char* ubp = ring + ub * UNIT;
  #pragma unroll
          for (int fn = 0; fn < FN; ++fn) f.b[fn] = tr_frag32_at(ubp + tr_base[fn] + 8192 * s);
        } else {
  #pragma unroll
          for (int fn = 0; fn < FN; ++fn) f.b[fn] = *(const bf16x8_t*)(sb + b_blk(fn) * 32 * 128);
        }
      };
      auto mfmas = [&](const Frags& f) {
  #pragma unroll
        for (int fn = 0; fn < FN; ++fn)
  #pragma unroll
          for (int fm = 0; fm < FM; ++fm)
            if (FULL || fm < fa)
              acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[fn], f.a[fm], acc[fn][fm], 0, 0, 0);
      };
      auto interleave_reads = [&]() {
        if constexpr (FULL) {
  #pragma unroll
          for (int i = 0; i < FM + FN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
        }
      };
      // fragments two substeps ahead: on entry to slice kt, a = (kt, 0) and
      // b = (kt, 1) are read or in flight; the barrier (slice kt + 1 landed,
      // every read of slice kt done) comes after substep 1
      auto slice = [&](int kt, Frags& a, Frags& b, Frags& c) {
        read_sub(kt, 2, c);
        mfmas(a);
        interleave_reads();
        read_sub(kt, 3, a);
        mfmas(b);
        interleave_reads();
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<IPW>();  // units 2 kt + 2, 2 kt + 3 landed (2 kt + 4 may be in flight)
        ring_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue();
        issue();
        read_sub(kt + 1, 0, b);
        mfmas(c);
        // the refill DMA one instruction per MFMA of this substep (two per
        // MFMA over its first half measured 2 % slower: the issue of a
        // burst of DMA instructions stalls the wave's MFMA stream)
        if constexpr (FULL) {
  #pragma unroll
          for (int i = 0; i < FM + FN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
  #pragma unroll
          for (int i = 0; i < FM * FN - (FM + FN); ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        }
        read_sub(kt + 1, 1, c);
        mfmas(a);
        interleave_reads();
      };
      Frags x, y, z;
      read_sub(0, 0, x);
      read_sub(0, 1, y);
      int kt = 0;
      for (; kt + 3 <= nk; kt += 3) {
        slice(kt, x, y, z);
        slice(kt + 1, y, z, x);
        slice(kt + 2, z, x, y);
      }
      if (kt < nk) slice(kt, x, y, z);
      if (kt + 1 < nk) slice(kt + 1, y, z, x);
    };

    // units 0 .. pend - 1 were issued before the previous tile's epilogue;
    // in-order completion then makes the wait below cover that epilogue's
    // stores too (issued after them), as when all five follow the stores
    issued = pend;
    while (issued < NU) issue();
    // units 0, 1 landed.  After early units, the previous tile's epilogue
    // stores sit between units 2 and 3 in issue order; with a fixed store
    // count the wait lets them drain behind this tile's first slices
    constexpr int EPI_STORES = (EPI == EPI_SWIGLU) ? 8 : 16;  // per wave, one LDS epilogue (h, or 16-bit)
    if (LDS_EPI && pend > 0 && p.fixed_stores) {
      if (EPI == EPI_SWIGLU && p.aux)
        wait_vmcnt<3 * IPW + EPI_STORES + 32>();  // and the saved g, u rows: 2 parts x 2 passes x 8
      else
        wait_vmcnt<3 * IPW + EPI_STORES>();
    } else {
      wait_vmcnt<3 * IPW>();
    }
    ring_barrier();
    if (fa == FM)
      main_loop(std::true_type{});
    else
      main_loop(std::false_type{});
    wait_vmcnt<0>();
    ring_barrier();  // every wave's ring reads and DMA done: the ring is free
    // the next tile of this workgroup and the first units of its DMA (for
    // the SwiGLU-backward epilogue, which takes none early, found after it:
    // its registers are the scarcer)
    constexpr bool NEXT_FIRST = EPI != EPI_DSWIGLU;
    int ns = slot + gridDim.x;
    int g2 = 0, r02 = 0, re2 = 0, n02 = 0, sp2 = 0;
    TileDma d2;
    auto find_next = [&]() {
      while (ns < p.slots && !tile_of(ns, g2, r02, re2, n02, sp2, d2)) ns += gridDim.x;
    };
    pend = 0;
    if constexpr (NEXT_FIRST) {
      find_next();
      if (ns < p.slots) {
        for (int u = 0; u < early; ++u) issue_unit(d2, u);
        pend = early;
      }
    }
    if constexpr (LDS_EPI && EPI == EPI_DSWIGLU) {
      dswiglu_tile_lds<BM, BN, WM, WN, FN, FM>(p, acc, row0, row_end, n0, ring);
    } else if constexpr (LDS_EPI) {
      store_tile32_lds<BM, BN, WM, WN, EPI, FN, FM>(p, acc, row0, row_end, n0, ring + early * UNIT);
    } else {
      store_tile32<BM, BN, WM, WN, SCHED_GROUP_M, EPI>(p, acc, g, row0, row_end, n0, sp);
    }
    ring_barrier();  // every wave done with the staging units before the next tile's DMA
    if constexpr (!NEXT_FIRST) find_next();
    slot = ns;
    g = g2;
    row0 = r02;
    row_end = re2;
    n0 = n02;
    sp = sp2;
    dm = d2;
  }
}

template <int WN, bool GROUPED, int EPI, bool BT = false>
int run_fwd_q64(const GemmProblem& q, hipStream_t stream);

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
  a.c_f16 = q.c_f16;
  a.splits = 1;
  a.split_ws = nullptr;
  a.slots = 0;
  a.A_lo = (const bf16_t*)q.A_lo;
  a.C_lo = (bf16_t*)q.C_lo;
  a.fixed_stores = 0;
  a.out_bytes = a.aux_bytes = 0;
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
  static std::atomic<unsigned long long> lds_set{0};
  if (set_lds_limit((const void*)kern, (int)lds_bytes, lds_set)) return -4;
  hipLaunchKernelGGL(kern, dim3((unsigned)slots), dim3(WM * WN * 64), lds_bytes, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

template <int BM, int BN, int WM, int WN, int NS, int SWZ, int EPI>
int run_fwd_dma(const GemmProblem& q, hipStream_t stream) {
  Args a = make_args(q);
  const int ncols = (EPI == EPI_SWIGLU) ? (int)q.n_half : (int)q.N;
  const int tn = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  a.NTn = (ncols + tn - 1) / tn;
  a.MTk = 0;
  const int64_t mt = q.offsets ? (q.rows_bound + BM - 1) / BM + q.G : (q.M + BM - 1) / BM;
  const int64_t slots = mt * a.NTn;
  if (slots <= 0) return 0;
  const size_t lds_bytes = (size_t)NS * (BM + BN) * 32 * 2;
  auto kern = gemm_fwd_dma_kernel<BM, BN, WM, WN, NS, SWZ, EPI>;
  static std::atomic<unsigned long long> lds_set{0};
  if (set_lds_limit((const void*)kern, (int)lds_bytes, lds_set)) return -4;
  hipLaunchKernelGGL(kern, dim3((unsigned)slots), dim3(WM * WN * 64), lds_bytes, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

__global__ __launch_bounds__(256) void split_reduce_kernel(const float* ws, int splits, int M, int N, void* C,
                                                           int64_t ldc, int kind, float* aux, int64_t ld_aux,
                                                           bf16_t* c_lo);

// K split of a one-group STORE_F32 GEMM on the 256x256 kernel whose tiles
// are fewer than the CUs (e.g. the shared down projection of a 4096-token
// batch: 16 x 8 tiles): splits = CUs / tiles (at most 8, each keeping at
// least 8 slices), fp32 partials into the caller's scratch, summed in split
// order by split_reduce_kernel.
int q64_splits(const GemmProblem& q) {
  if (q.offsets || !q.split_ws || q.epi != EPI_STORE_F32) return 1;
  const int64_t tiles = ((q.M + 255) / 256) * ((q.N + 255) / 256);
  const int cus = device_cu_count();
  if (tiles == 0 || cus <= 0 || tiles >= cus) return 1;
  int64_t sp = cus / tiles;
  if (sp > 8) sp = 8;
  if (sp > q.K / 64 / 8) sp = q.K / 64 / 8;
  return sp > 1 ? (int)sp : 1;
}

template <int WN, bool GROUPED, int EPI, bool BT>
int run_fwd_q64(const GemmProblem& q, hipStream_t stream) {
  Args a = make_args(q);
  const int ncols = (EPI == EPI_SWIGLU) ? (int)q.n_half : (int)q.N;
  const int tn = (EPI == EPI_SWIGLU) ? 128 : 256;
  a.NTn = (ncols + tn - 1) / tn;
  a.MTk = 0;
  int64_t mt = q.offsets ? (q.rows_bound + 255) / 256 + q.G : (q.M + 255) / 256;
  if (mt <= 0) return 0;
  const int64_t per = 8LL * kXcdGroupM;
  mt = (mt + per - 1) / per * per;
  const int64_t slots = mt * a.NTn;
  const size_t lds_bytes = 5 * 256 * 64 * 2;
  const int sp = GROUPED ? 1 : (q.splits > 0 ? q.splits : q64_splits(q));
  // 16-bit outputs without K split go through the LDS epilogue, which
  // stores 16-byte chunks: C and its row pitch must keep them aligned
  // the SwiGLU-backward epilogue through LDS: 16-byte chunks of the saved
  // fp32 rows and of the bf16 dg | du rows, 32-bit offsets into the saved rows
  // (the SwiGLU-backward epilogue always goes through LDS: launch_gemm
  // takes this kernel for it only when dswiglu_lds_ok)
  const bool lds_epi = EPI == EPI_DSWIGLU || ((EPI != EPI_STORE_F32 || (q.c_f16 && sp == 1)) &&
                                              (reinterpret_cast<uintptr_t>(q.C) & 15) == 0 && q.ldc % 8 == 0);
  // buffer stores of a fixed count: every output byte offset (and the saved
  // rows') below 0xFFFFFFF0, whole 16-byte chunks (the column count a multiple of 8)
  if (lds_epi && EPI != EPI_DSWIGLU) {
    const int64_t out_cols = EPI == EPI_SWIGLU ? q.n_half : q.N;
    const int64_t out_bytes = q.M * q.ldc * 2;
    const int64_t aux_bytes = q.aux ? q.M * q.ld_aux * 4 : 0;
    if (out_cols % 8 == 0 && out_bytes < (1LL << 31) && aux_bytes < (1LL << 31) &&
        (!q.aux || q.ld_aux >= 2 * q.n_half)) {
      a.fixed_stores = 1;
      a.out_bytes = (uint32_t)out_bytes;
      a.aux_bytes = (uint32_t)aux_bytes;
    }
  }
  void (*kern)(Args) = gemm_fwd_q64_kernel<WN, GROUPED, EPI, true, BT>;
  static std::atomic<unsigned long long> lds_set{0}, lds_set_epi{0};
  if constexpr (EPI != EPI_DSWIGLU) {
    if (!lds_epi) kern = gemm_fwd_q64_kernel<WN, GROUPED, EPI, false, BT>;
  }
  if (set_lds_limit((const void*)kern, (int)lds_bytes, lds_epi ? lds_set_epi : lds_set)) return -4;
  if (sp > 1) {
    a.splits = sp;
    a.split_ws = (float*)q.split_ws;
  }
  a.slots = (int)(slots * sp);
  int64_t grid = a.slots;
  {
    const int n_cu = device_cu_count() / 8 * 8;
    if (n_cu >= 8 && grid > n_cu) grid = n_cu;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(128 * WN), lds_bytes, stream, a);
  if (sp > 1 && !q.partials_only) {
    const int64_t nthreads = q.M * (q.N / 4);
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, stream,
                       (const float*)q.split_ws, sp, (int)q.M, (int)q.N, q.C, (int64_t)q.ldc, q.c_f16 ? 2 : 1,
                       nullptr, (int64_t)0, nullptr);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// ---------------------------------------------------------------------------
// Skinny forward GEMM for segments of few rows (decode-sized token counts,
// small shared-expert batches): every weight element is used by at most a
// few dozen rows, so the GEMM is a weight stream and wants whole-line reads
// with many bytes in flight.  A workgroup of 4 waves computes BM (32, or 64
// for one group of at least 256 rows) rows x 128 B-rows (SwiGLU: 64 gate rows
// and the matching 64 up rows); wave w owns BM / 16 16-row m-blocks and two
// 16-wide n-blocks (SwiGLU: gate block w and up block
// w, so the epilogue has gate and up of one column in one lane).  64-wide K
// slices (BM A rows + 128 B rows, 20 or 24 KB, every row segment one 128-byte
// line) stream into an NS-slot LDS ring (4 slots, 3 for BM = 64: two
// workgroups a CU) by global_load_lds_dwordx4; step kt reads
// its fragments and runs its 8 v_mfma_f32_16x16x32_bf16, waits until slice
// kt + 1 has landed (own DMA count, then a barrier for everyone's), and
// refills the slot of slice kt with slice kt + NS.  Slices past the end
// re-read the last one into slots nobody reads again.  Rows keep the swizzle
// of the 256x256 kernel.  Slots: XCD x = slot % 8 takes the n-tiles congruent
// to x and, for each, every m-tile in turn, so the m-tiles that share a
// weight panel run on one XCD and share its L2.
// SPLIT: the A operand is a pair of bf16 tensors A + A_lo (an activation
// kept as its bf16 rounding and the bf16 rounding of the remainder): a slice
// holds BM rows of each, and every B fragment meets both, in two MFMA passes
// into the same accumulators (3 ring slots; the MFMAs of a weight stream have
// time to spare).  The SwiGLU epilogue writes that pair for h when C_lo is
// set.
template <int EPI, bool GROUPED, int BM, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_stream_kernel(Args p) {
  constexpr int BR = 128, BK = 64;
  constexpr int NS = (BM == 32 && !SPLIT) ? 4 : 3;  // ring slots (two workgroups a CU up to 80 KB)
  constexpr int MB = BM / 16;  // 16-row m-blocks of a wave
  constexpr int AR = SPLIT ? 2 * BM : BM;  // A rows of a slice (hi, then lo)
  constexpr int ROWS = AR + BR;
  constexpr int SLICE = ROWS * BK * 2;  // 20 KB (BM 32), 24 KB (BM 64 or split BM 32), 32 KB (split BM 64)
  constexpr int IPW = SLICE / 1024 / 4;  // DMA instructions per wave per slice
  static_assert(SLICE % 4096 == 0 && (NS - 1) * IPW < 64, "slice");
  __shared__ __attribute__((aligned(16))) char ring[NS * SLICE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // with a split K, workgroup set sp = slot / slots covers slices
  // [sp nk / splits, (sp + 1) nk / splits); slots is a multiple of 8, so the
  // XCD of a tile does not depend on sp
  const int slots = p.MTk * ((p.NTn + 7) / 8) * 8;
  const int sp = blockIdx.x / slots, b = blockIdx.x - sp * slots;
  const int x = b & 7, i = b >> 3;
  const int mt = i % p.MTk;
  const int nt = (i / p.MTk) * 8 + x;
  if (nt >= p.NTn) return;
  int g, row0, row_end;
  if constexpr (GROUPED) {
    if (!find_group_m_wave<BM>(p, mt, g, row0, row_end)) return;
  } else {
    g = 0;
    row0 = mt * BM;
    row_end = p.M;
    if (row0 >= p.M) return;
  }
  const int n0 = nt * ((EPI == EPI_SWIGLU) ? BR / 2 : BR);
  const bf16_t* Bg = p.B + (int64_t)g * p.strideB;
  // DMA: instruction j of this wave covers slice rows 8 (IPW wave + j) .. + 7;
  // lane reads row 8 (IPW wave + j) + lane / 8, logical chunk (lane % 8) ^ sw.
  const bf16_t* src[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int rr = (wave * IPW + j) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz8(rr);
    if (rr < AR) {
      const int m = min(row0 + (rr % BM), row_end - 1);
      const int64_t r = p.a_idx ? (int64_t)(p.a_idx[m] / p.a_div) : (int64_t)m;
      src[j] = (SPLIT && rr >= BM ? p.A_lo : p.A) + r * p.lda + chunk * 8;
    } else {
      const int b = rr - AR;
      int n;
      if constexpr (EPI == EPI_SWIGLU) {
        const int c = min(n0 + (b & 63), p.n_half - 1);
        n = b < 64 ? c : p.n_half + c;
      } else {
        n = min(n0 + b, p.N - 1);
      }
      src[j] = Bg + (int64_t)n * p.ldb + chunk * 8;
    }
  }
  const int nk_all = p.K / BK;
  const int kb = sp * nk_all / p.splits;
  const int nk = (sp + 1) * nk_all / p.splits - kb;
  int issued = 0;
  auto issue = [&](int slot) {
    char* dst = ring + slot * SLICE + wave * (IPW * 1024);
    const int64_t koff = (int64_t)(kb + min(issued, nk - 1)) * BK;
#pragma unroll
    for (int j = 0; j < IPW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + koff),
                                       (__attribute__((address_space(3))) void*)(dst + j * 1024), 16, 0, 0);
    ++issued;
  };
  const int lr = lane & 15, lq = lane >> 4;
  // B rows of this wave's n-blocks inside the slice (after the A rows)
  int brow[2];
  if constexpr (EPI == EPI_SWIGLU) {
    brow[0] = AR + wave * 16;       // gate block
    brow[1] = AR + 64 + wave * 16;  // the matching up block
  } else {
    brow[0] = AR + wave * 32;
    brow[1] = AR + wave * 32 + 16;
  }
  f32x4_t acc[2][MB];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto frag = [&](const char* st, int row, int s) -> bf16x8_t {
    return *(const bf16x8_t*)(st + row * 128 + (((4 * s + lq) ^ swz8(row)) * 16));
  };
#pragma unroll
  for (int s = 0; s < NS; ++s) issue(s);
  wait_vmcnt<(NS - 1) * IPW>();  // slice 0 landed
  ring_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const char* st = ring + (kt % NS) * SLICE;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8_t af[MB], al[SPLIT ? MB : 1], bfr[2];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) af[mb] = frag(st, mb * 16 + lr, s);
      if constexpr (SPLIT) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) al[mb] = frag(st, BM + mb * 16 + lr, s);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bfr[nb] = frag(st, brow[nb] + lr, s);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[nb], af[mb], acc[nb][mb], 0, 0, 0);
          if constexpr (SPLIT)
            acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[nb], al[mb], acc[nb][mb], 0, 0, 0);
        }
    }
    wait_vmcnt<(NS - 2) * IPW>();  // slice kt + 1 landed; this wave's reads of slice kt done
    ring_barrier();
    issue(kt % NS);
  }
  wait_vmcnt<0>();
  // lane (lr, lq) holds rows mb * 16 + lr, columns 4 lq + 0..3 of n-block nb
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = row0 + mb * 16 + lr;
    if (m >= row_end) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      const int col = n0 + wave * 16 + lq * 4;
      if (col >= p.n_half) continue;  // n_half % 8 == 0: a run of 4 is all in or all out
      const f32x4_t gv = acc[0][mb], uv = acc[1][mb];
      if (p.splits > 1) {  // partial gate | up sums; split_reduce_kernel applies SwiGLU
        float* part = p.split_ws + ((int64_t)sp * p.M + m) * (2 * p.n_half) + col;
        *(f32x4_t*)part = gv;
        *(f32x4_t*)(part + p.n_half) = uv;
        continue;
      }
      float h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = gv[q] * fast_sigmoid(gv[q]) * uv[q];
      const u32x2_t hv = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
      *(u32x2_t*)(p.C + (int64_t)m * p.ldc + col) = hv;
      if (p.C_lo) *(u32x2_t*)(p.C_lo + (int64_t)m * p.ldc + col) = lo_pair(h);
      if (p.aux) {
        float* ga = (float*)p.aux + (int64_t)m * p.ld_aux + col;
        *(f32x4_t*)ga = gv;
        *(f32x4_t*)(ga + p.n_half) = uv;
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = n0 + wave * 32 + nb * 16 + lq * 4;
        if (col >= p.N) continue;
        const f32x4_t v = acc[nb][mb];
        if (p.splits > 1) {
          *(f32x4_t*)(p.split_ws + ((int64_t)sp * p.M + m) * p.N + col) = v;
        } else if constexpr (EPI == EPI_STORE_F32) {
          if (p.c_f16)
            *(u32x2_t*)((f16_t*)p.C + (int64_t)m * p.ldc + col) = u32x2_t{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
          else
            *(f32x4_t*)((float*)p.C + (int64_t)m * p.ldc + col) = v;
        } else {
          const u32x2_t o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(u32x2_t*)(p.C + (int64_t)m * p.ldc + col) = o;
        }
      }
    }
  }
}

// Sum over sp = 0 .. splits - 1 (in this order) of the fp32 partials
// ws[sp][m][n], four columns from `col`: the loads of eight splits are
// issued together, then added in split order.
MOE_DEV f32x4_t sum_splits(const float* ws, int splits, int64_t stride, int64_t off) {
  f32x4_t acc = *(const f32x4_t*)(ws + off);
  for (int sp = 1; sp < splits; sp += 8) {
    f32x4_t t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (sp + j < splits) t[j] = *(const f32x4_t*)(ws + (sp + j) * stride + off);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (sp + j < splits) acc += t[j];
  }
  return acc;
}

// C[m, n] = the split sum of ws[.][m][n], stored as bf16 (kind 0), fp32 (1)
// or binary16 (2); 4 columns a thread.  Kind 3 (SwiGLU, N = 2 n_half):
// g, u = the split sums of columns n and n_half + n, C[m, n] = bf16 of
// silu(g) u (its lo part in c_lo[m, n] when c_lo is set), and g, u stored
// to aux[m, n] and aux[m, n_half + n] when aux is set.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* ws, int splits, int M, int N, void* C,
                                                           int64_t ldc, int kind, float* aux, int64_t ld_aux,
                                                           bf16_t* c_lo) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)M * N;
  if (kind == 3) {
    const int nh = N / 2;
    const int64_t n4 = nh / 4;
    if (q >= (int64_t)M * n4) return;
    const int m = (int)(q / n4), col = (int)(q % n4) * 4;
    const f32x4_t gv = sum_splits(ws, splits, stride, (int64_t)m * N + col);
    const f32x4_t uv = sum_splits(ws, splits, stride, (int64_t)m * N + nh + col);
    float h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = gv[i] * fast_sigmoid(gv[i]) * uv[i];
    *(u32x2_t*)((bf16_t*)C + (int64_t)m * ldc + col) = u32x2_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
    if (c_lo) *(u32x2_t*)(c_lo + (int64_t)m * ldc + col) = lo_pair(h);
    if (aux) {
      *(f32x4_t*)(aux + (int64_t)m * ld_aux + col) = gv;
      *(f32x4_t*)(aux + (int64_t)m * ld_aux + nh + col) = uv;
    }
    return;
  }
  const int64_t n4 = N / 4;
  if (q >= (int64_t)M * n4) return;
  const int m = (int)(q / n4), col = (int)(q % n4) * 4;
  const f32x4_t acc = sum_splits(ws, splits, stride, (int64_t)m * N + col);
  if (kind == 1) {
    *(f32x4_t*)((float*)C + (int64_t)m * ldc + col) = acc;
  } else if (kind == 2) {
    *(u32x2_t*)((f16_t*)C + (int64_t)m * ldc + col) = u32x2_t{pack_f16x2(acc[0], acc[1]), pack_f16x2(acc[2], acc[3])};
  } else {
    *(u32x2_t*)((bf16_t*)C + (int64_t)m * ldc + col) = u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  }
}

// K split of the one-group streaming GEMM: a weight stream needs about one
// workgroup's ring of slices in flight per CU to cover the memory latency,
// so when the caller gave scratch and the tiles alone are fewer than the
// CUs, K splits over up to 16 workgroup sets (about 256 workgroups), each
// keeping at least 4 slices.  The partials cost a reduce kernel (a few us,
// mostly launch and latency): STORE epilogues split below 256 tiles, the
// SwiGLU epilogue only below 64 (measured: at 88 and 176 tiles the reduce
// costs more than the split saves).
// Rows per tile of the streaming GEMM: 32; 64 for a one-group problem of at
// least 256 rows (the shared expert of a 256-token decode batch), whose
// weight panels are then read by half as many tiles (measured at T = 256:
// shared gate_up 38.5 -> 35.1 us, down 26.0 -> 22.4 us; at T = 64 the halved
// tile count made it slower).
int stream_bm(const GemmProblem& q) { return (!q.offsets && q.M >= 256) ? 64 : 32; }

int stream_splits(const GemmProblem& q) {
  if (q.offsets || !q.split_ws || (q.epi != EPI_STORE && q.epi != EPI_STORE_F32 && q.epi != EPI_SWIGLU)) return 1;
  const int64_t mts = (q.M + stream_bm(q) - 1) / stream_bm(q);
  const int64_t tiles = q.epi == EPI_SWIGLU ? mts * ((q.n_half + 63) / 64) : mts * ((q.N + 127) / 128);
  const int64_t nk = q.K / 64;
  if (tiles == 0 || tiles >= (q.epi == EPI_SWIGLU ? 64 : 256)) return 1;
  int64_t sp = 256 / tiles;
  if (sp > 16) sp = 16;
  if (sp > nk / 4) sp = nk / 4;
  return sp > 1 ? (int)sp : 1;
}

template <int EPI, bool GROUPED, int BM, bool SPLIT = false>
int run_fwd_stream(const GemmProblem& q, hipStream_t stream) {
  Args a = make_args(q);
  const int ncols = (EPI == EPI_SWIGLU) ? (int)q.n_half : (int)q.N;
  const int tn = (EPI == EPI_SWIGLU) ? 64 : 128;
  a.NTn = (ncols + tn - 1) / tn;
  const int64_t mt = GROUPED ? (q.rows_bound + BM - 1) / BM + q.G : (q.M + BM - 1) / BM;
  if (mt <= 0 || a.NTn <= 0) return 0;
  a.MTk = (int)mt;
  const int64_t slots = mt * ((a.NTn + 7) / 8) * 8;
  const int sp = GROUPED ? 1 : stream_splits(q);
  if (sp > 1) {
    a.splits = sp;
    a.split_ws = (float*)q.split_ws;
  }
  hipLaunchKernelGGL((gemm_stream_kernel<EPI, GROUPED, BM, SPLIT>), dim3((unsigned)(slots * sp)), dim3(256), 0, stream,
                     a);
  if (sp > 1) {
    const int64_t ncols = EPI == EPI_SWIGLU ? 2 * q.n_half : q.N;  // columns of the partials
    const int64_t nthreads = q.M * ((EPI == EPI_SWIGLU ? q.n_half : q.N) / 4);
    const int kind = EPI == EPI_SWIGLU ? 3 : EPI == EPI_STORE_F32 ? (q.c_f16 ? 2 : 1) : 0;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, stream,
                       (const float*)q.split_ws, sp, (int)q.M, (int)ncols, q.C, (int64_t)q.ldc, kind,
                       EPI == EPI_SWIGLU ? (float*)q.aux : nullptr, (int64_t)q.ld_aux,
                       EPI == EPI_SWIGLU ? (bf16_t*)q.C_lo : nullptr);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}


// fp32 epilogue of a 256x256 weight-gradient tile through LDS, in two
// 128-row halves (a half is 128 KB of the idle ring): the waves of that half
// write their f32x4 pieces (four columns of one row per lane and 32x32
// block) into a row-major copy, 16-byte chunk c of row r at c ^ (r % 64),
// and after a barrier the workgroup stores whole 1 KB rows, one row per
// store instruction, instead of 16 bytes into each of 32 rows.  On entry
// every wave's DMA has landed; the first barrier ends the ring's reads.
template <int BM, int BN, int WM, int WN, int FN, int FM>
MOE_DEV void store_wgrad_lds(const Args& p, const f32x16_t (&acc)[FN][FM], int g, int m0, int n0, char* lds) {
  constexpr int HR = BM / WM, RB = BN * 4, CH = RB / 16, NT = 64 * WM * WN;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lm = lane & 31, lh = lane >> 5;
  float* Cg = (float*)p.C + (int64_t)g * p.strideC;
  ring_barrier();
#pragma unroll
  for (int h = 0; h < WM; ++h) {
    if (wm == h) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = fm * 32 + lm;
        char* row = lds + r * RB;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = (wn * FN + fn) * 8 + q * 2 + lh;
            const f32x16_t& a = acc[fn][fm];
            *(f32x4_t*)(row + ((c ^ (r & (CH - 1))) << 4)) = f32x4_t{a[q * 4], a[q * 4 + 1], a[q * 4 + 2], a[q * 4 + 3]};
          }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));  // LDS writes done
    ring_barrier();
#pragma unroll 4
    for (int i = 0; i < HR * CH / NT; ++i) {
      const int id = tid + i * NT;
      const int r = id / CH, c = id % CH;
      const f32x4_t v = *(const f32x4_t*)(lds + r * RB + ((c ^ (r & (CH - 1))) << 4));
      const int m = m0 + h * HR + r, col = n0 + c * 4;
      if (m < p.M && col < p.N) __builtin_nontemporal_store(v, (f32x4_t*)(Cg + (int64_t)m * p.ldc + col));
    }
    if (h + 1 < WM) {
      __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));  // LDS reads done
      ring_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// Weight-gradient GEMM (GROUP_K): C_g[m][n] = sum over the rows r of segment
// g of A[r][m] * B[r][n], both operands row-major over the segment's rows
// (dw_down = dy^T h, dw_gate_up = dgu^T x, and the shared-expert pair).
// 256x256 output tiles over 8 waves (128 x 64 each, 32x32x16 MFMAs); 64-row
// K slices of each operand (64 rows x 512 bytes of columns, whole lines) go
// global -> LDS by DMA (the asm form, dma16_hidden) into the same 5-unit ring
// as the forward kernel, in the k-row-major unit layout of kmaj_off, and
// every MFMA fragment is read by tr_frag32_at (two ds_read_b64_tr_b16).  Rows past the
// segment are clamped for the DMA and zeroed in the A fragments of the last
// slice.  Every group gets all its tiles: an empty segment writes zeros.
template <int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_wgrad_kernel(Args p) {
  constexpr int BM = 256, BN = 256, BK = 64, WM = 2, WN = 4;
  constexpr int FM = BM / WM / 32, FN = BN / WN / 32;  // 4, 2
  constexpr int UNIT = BK * 512;                       // 32 KB
  constexpr int NU = 5;
  constexpr int IPW = UNIT / 1024 / 8;  // 4
  static_assert(EPI == EPI_STORE_F32, "weight gradients are fp32");
  extern __shared__ __attribute__((aligned(16))) char ring[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int ntiles = p.G * p.MTk * p.NTn;
  const int per = (ntiles + 7) / 8;
  const int j = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (j >= ntiles) return;
  const int g = j / (p.MTk * p.NTn), rem = j % (p.MTk * p.NTn);
  const int m0 = (rem / p.NTn) * BM, n0 = (rem % p.NTn) * BN;
  const int o0 = p.offsets ? p.offsets[g] : 0;
  const int L = p.offsets ? p.offsets[g + 1] - o0 : p.K;
  const int nk = (L + BK - 1) / BK;

  // DMA: instruction i of this wave covers unit rows 2 (IPW wave + i) + {0, 1};
  // lane: row 2 (IPW wave + i) + lane / 32, physical chunk lane % 32, logical
  // chunk (lane % 32) ^ (4 (row % 4)); columns clamped to the matrix (those
  // outputs are not stored).
  int krow[IPW], acol[IPW], bcol[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    krow[i] = 2 * (IPW * wave + i) + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (krow[i] & 3));
    acol[i] = min(m0 + c * 8, p.M - 8);
    bcol[i] = min(n0 + c * 8, p.N - 8);
  }
  int issued = 0;
  auto issue = [&]() {
    const int u = issued;
    const int slice = min(u >> 1, nk - 1);
    char* dst = ring + (u % NU) * UNIT + wave * (IPW * 1024);
    const bool is_b = u & 1;
    // rows of the slice relative to its first row (the clamped rows past the
    // segment stay inside the slice), so every offset fits 32 bits
    const int64_t r0 = o0 + (int64_t)slice * BK;
    const int64_t ld = is_b ? p.ldb : p.lda;
    const i32x4_t rs = dma_rsrc_words(is_b ? p.B + r0 * p.ldb : p.A + r0 * p.lda);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int rr = min(slice * BK + krow[i], L - 1) - slice * BK;
      dma16_hidden(rs, (uint32_t)((rr * ld + (is_b ? bcol[i] : acol[i])) * 2), dst + i * 1024);
    }
    ++issued;
  };
  // this lane's k-row and column offsets of the transposing fragment reads
  const int G = lane >> 4;
  const int fr_k = 8 * (G >> 1) + ((lane & 15) >> 2);
  const int fr_c = 16 * (G & 1) + 4 * (lane & 3);
  // first addresses of the A and B fragments in their units, less the
  // substep's 16 k-rows
  int fa_base[FM], fb_base[FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
    fa_base[fm] = frag_lane_off(fr_k, fr_c) + 64 * ((wm * (BM / WM / 32) + fm) ^ (fr_k & 3));
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) fb_base[fn] = frag_lane_off(fr_k, fr_c) + 64 * ((wn * FN + fn) ^ (fr_k & 3));
  struct Frags {
    bf16x8_t a[FM], b[FN];
  };
  auto read_sub = [&](int kt, int s, Frags& f) {
    const char* ua = ring + ((2 * kt) % NU) * UNIT;
    const char* ub = ring + ((2 * kt + 1) % NU) * UNIT;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) f.a[fm] = tr_frag32_at(ua + fa_base[fm] + 8192 * s);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) f.b[fn] = tr_frag32_at(ub + fb_base[fn] + 8192 * s);
    if (kt == nk - 1) {  // rows past the segment contribute nothing
      const int valid = L - kt * BK;
      const int kl = 16 * s + 8 * (G >> 1);  // this lane's 8 k values: kl .. kl + 7
      if (kl + 8 > valid) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          short __attribute__((ext_vector_type(8))) v = __builtin_bit_cast(short __attribute__((ext_vector_type(8))), f.a[fm]);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (kl + e >= valid) v[e] = 0;
          f.a[fm] = __builtin_bit_cast(bf16x8_t, v);
        }
      }
    }
  };

  f32x16_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int jj = 0; jj < FM; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[fn], f.a[fm], acc[fn][fm], 0, 0, 0);
  };
  // each substep's 12 transposing reads between its 8 MFMAs
  auto interleave_reads = [&]() {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < FM * FN - FM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  // fragments two substeps ahead, as in the forward kernel: on entry to
  // slice kt, a = (kt, 0) and b = (kt, 1) are read or in flight; the barrier
  // (slice kt + 1 landed, every read of slice kt done) comes after substep 1
  auto slice = [&](int kt, Frags& a, Frags& b, Frags& c) {
    read_sub(kt, 2, c);
    mfmas(a);
    interleave_reads();
    read_sub(kt, 3, a);
    mfmas(b);
    interleave_reads();
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<IPW>();  // units 2 kt + 2, 2 kt + 3 landed
    ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue();
    issue();
    read_sub(kt + 1, 0, b);
    mfmas(c);
    interleave_reads();
    read_sub(kt + 1, 1, c);
    mfmas(a);
    interleave_reads();
  };
  if (nk > 0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) issue();
    wait_vmcnt<3 * IPW>();  // units 0, 1 landed
    ring_barrier();
    Frags x, y, z;
    read_sub(0, 0, x);
    read_sub(0, 1, y);
    int kt = 0;
    for (; kt + 3 <= nk; kt += 3) {
      slice(kt, x, y, z);
      slice(kt + 1, y, z, x);
      slice(kt + 2, z, x, y);
    }
    if (kt < nk) slice(kt, x, y, z);
    if (kt + 1 < nk) slice(kt + 1, y, z, x);
    wait_vmcnt<0>();
  }
  store_wgrad_lds<BM, BN, WM, WN, FN, FM>(p, acc, g, m0, n0, ring);
}

template <int EPI>
int run_wgrad(const GemmProblem& q, hipStream_t stream) {
  Args a = make_args(q);
  a.MTk = (int)((q.M + 255) / 256);
  a.NTn = (int)((q.N + 255) / 256);
  a.G = q.offsets ? q.G : 1;
  const int64_t ntiles = (int64_t)a.G * a.MTk * a.NTn;
  if (ntiles <= 0) return 0;
  const int64_t slots = (ntiles + 7) / 8 * 8;
  const size_t lds_bytes = 5 * 64 * 512;
  auto kern = gemm_wgrad_kernel<EPI>;
  static std::atomic<unsigned long long> lds_set{0};
  if (set_lds_limit((const void*)kern, (int)lds_bytes, lds_set)) return -4;
  hipLaunchKernelGGL(kern, dim3((unsigned)slots), dim3(512), lds_bytes, stream, a);
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


// The streaming kernel takes forward GEMMs whose tiles of 256 rows would be
// mostly padding or too few to fill the GPU.
bool use_stream(const GemmProblem& q) {
  const bool fwd_epi = q.epi == EPI_SWIGLU || q.epi == EPI_STORE || q.epi == EPI_STORE_F32;
  if (!(fwd_epi && q.sched == SCHED_GROUP_M && q.a_kmajor && q.b_kmajor && q.K % 64 == 0 &&
        !(q.epi == EPI_SWIGLU && q.n_half % 8) && !(q.epi != EPI_SWIGLU && q.N % 4)))
    return false;
  const int64_t groups = q.offsets ? q.G : 1;
  const int64_t rows = q.offsets ? q.rows_bound : q.M;
  const int64_t ncols = q.epi == EPI_SWIGLU ? q.n_half : q.N;
  const int64_t tn = q.epi == EPI_SWIGLU ? 128 : 256;
  const int64_t big_tiles = ((rows + 255) / 256 + (q.offsets ? groups : 0)) * ((ncols + tn - 1) / tn);
  return rows <= 64 * groups || (rows <= 256 * groups && big_tiles < 256);
}

bool gemm_uses_stream(const GemmProblem& q, int bf16) { return bf16 && use_stream(q); }

bool gemm_split_operand_ok(const GemmProblem& q, int bf16) {
  return bf16 && use_stream(q) && (q.epi == EPI_SWIGLU || (!q.a_idx && q.epi != EPI_SWIGLU));
}

// launch_gemm's choice of the 256x256 kernel for a bf16 problem
// the 256x256 kernel with an N-contiguous B (transposing fragment reads):
// the data-gradient GEMMs (SwiGLU-backward or binary16 / fp32 store
// epilogue) straight on the stored expert weights
// The SwiGLU-backward epilogue of the 256x256 kernel (dswiglu_tile_lds)
// moves 16-byte chunks of the saved fp32 rows and of the bf16 dg | du rows.
bool dswiglu_lds_ok(const GemmProblem& q) {
  return ((reinterpret_cast<uintptr_t>(q.aux) | reinterpret_cast<uintptr_t>(q.aux_out)) & 15) == 0 &&
         q.n_half % 8 == 0 && q.ld_aux % 8 == 0 && q.ld_aux >= 2 * q.n_half;
}

bool use_q64_bt(const GemmProblem& q) {
  if (!((q.epi == EPI_DSWIGLU || q.epi == EPI_STORE_F32) && q.sched == SCHED_GROUP_M && q.a_kmajor && !q.b_kmajor &&
        q.K % 64 == 0 && q.N % 8 == 0 && q.N >= 8 && q.ldb % 8 == 0 && !(q.epi == EPI_DSWIGLU && !dswiglu_lds_ok(q))))
    return false;
  const int64_t a_rows = q.a_idx ? (q.M + q.a_div - 1) / q.a_div : q.M;
  return a_rows * q.lda * 2 < (1LL << 32) && q.K * q.ldb * 2 < (1LL << 31);
}

bool use_q64(const GemmProblem& q) {
  const bool fwd_epi = q.epi == EPI_SWIGLU || q.epi == EPI_STORE || q.epi == EPI_STORE_F32;
  if (fwd_epi && use_stream(q)) return false;
  if (!((fwd_epi || q.epi == EPI_DSWIGLU) && q.sched == SCHED_GROUP_M && q.a_kmajor && q.b_kmajor &&
        q.K % 32 == 0 && !((q.epi == EPI_SWIGLU || q.epi == EPI_DSWIGLU) && q.n_half % 8) &&
        !(q.epi == EPI_DSWIGLU && !dswiglu_lds_ok(q))))
    return false;
  const int64_t a_rows = q.a_idx ? (q.M + q.a_div - 1) / q.a_div : q.M;
  const bool off32 = a_rows * q.lda * 2 < (1LL << 32) && q.N * q.ldb * 2 < (1LL << 32);
  return off32 && q.K % 64 == 0;
}

int gemm_q64_splits(const GemmProblem& q, int bf16) {
  if (!bf16 || q.offsets || q.epi != EPI_STORE_F32 || use_stream(q) || !use_q64(q)) return 0;
  return q.splits > 0 ? q.splits : q64_splits(q);
}

size_t gemm_split_ws_bytes(const GemmProblem& q, int bf16) {
  if (!bf16) return 0;
  GemmProblem t = q;
  t.split_ws = (void*)16;  // as if scratch were given
  if (use_q64(t)) {
    const int sp = q64_splits(t);
    return sp > 1 ? (size_t)sp * (size_t)q.M * (size_t)q.N * 4 : 0;
  }
  if (!use_stream(q)) return 0;
  const int sp = stream_splits(t);
  const int64_t ncols = q.epi == EPI_SWIGLU ? 2 * q.n_half : q.N;
  return sp > 1 ? (size_t)sp * (size_t)q.M * (size_t)ncols * 4 : 0;
}

int launch_gemm(const GemmProblem& q, int bf16, hipStream_t stream) {
  // the epilogue's outputs must exist: C, or (dgate | dup) and the saved (gate | up)
  if (q.epi == EPI_DSWIGLU ? (!q.aux || !q.aux_out) : !q.C) return -1;
  if (!bf16) {
    if (q.sched == SCHED_GROUP_M) {
      if (q.epi == EPI_SWIGLU) return run_f32<SCHED_GROUP_M, EPI_SWIGLU>(q, stream);
      if (q.epi == EPI_DSWIGLU) return run_f32<SCHED_GROUP_M, EPI_DSWIGLU>(q, stream);
      return run_f32<SCHED_GROUP_M, EPI_STORE>(q, stream);  // EPI_STORE_F32: same for fp32
    }
    return run_f32<SCHED_GROUP_K, EPI_STORE>(q, stream);
  }
  // bf16 MFMA engine; the operand layouts each GEMM of the layer uses:
  // few rows per group: the streaming kernel, when the 256x256 tiles would
  // be mostly padding or too few to fill the GPU
  const bool fwd_epi = q.epi == EPI_SWIGLU || q.epi == EPI_STORE || q.epi == EPI_STORE_F32;
  // a split operand (A_lo in, C_lo out) exists only on the streaming kernel
  if ((q.A_lo || q.C_lo) && !gemm_split_operand_ok(q, bf16)) return -2;
  if (q.C_lo && q.epi != EPI_SWIGLU) return -2;
  if (q.A_lo && fwd_epi && q.epi != EPI_SWIGLU) {
    if (q.offsets) {
      if (q.epi == EPI_STORE_F32) return run_fwd_stream<EPI_STORE_F32, true, 32, true>(q, stream);
      return run_fwd_stream<EPI_STORE, true, 32, true>(q, stream);
    }
    if (stream_bm(q) == 64) {
      if (q.epi == EPI_STORE_F32) return run_fwd_stream<EPI_STORE_F32, false, 64, true>(q, stream);
      return run_fwd_stream<EPI_STORE, false, 64, true>(q, stream);
    }
    if (q.epi == EPI_STORE_F32) return run_fwd_stream<EPI_STORE_F32, false, 32, true>(q, stream);
    return run_fwd_stream<EPI_STORE, false, 32, true>(q, stream);
  }
  if (fwd_epi) {
    if (use_stream(q)) {
      if (q.offsets) {
        if (q.epi == EPI_SWIGLU) return run_fwd_stream<EPI_SWIGLU, true, 32>(q, stream);
        if (q.epi == EPI_STORE_F32) return run_fwd_stream<EPI_STORE_F32, true, 32>(q, stream);
        return run_fwd_stream<EPI_STORE, true, 32>(q, stream);
      }
      if (stream_bm(q) == 64) {
        if (q.epi == EPI_SWIGLU) return run_fwd_stream<EPI_SWIGLU, false, 64>(q, stream);
        if (q.epi == EPI_STORE_F32) return run_fwd_stream<EPI_STORE_F32, false, 64>(q, stream);
        return run_fwd_stream<EPI_STORE, false, 64>(q, stream);
      }
      if (q.epi == EPI_SWIGLU) return run_fwd_stream<EPI_SWIGLU, false, 32>(q, stream);
      if (q.epi == EPI_STORE_F32) return run_fwd_stream<EPI_STORE_F32, false, 32>(q, stream);
      return run_fwd_stream<EPI_STORE, false, 32>(q, stream);
    }
  }
  if ((fwd_epi || q.epi == EPI_DSWIGLU) && q.sched == SCHED_GROUP_M && q.a_kmajor && q.b_kmajor && q.K % 32 == 0 &&
      !((q.epi == EPI_SWIGLU || q.epi == EPI_DSWIGLU) && q.n_half % 8)) {
// the 32-wide-slice kernel: 256 x 256 tiles, 2 x 4 waves, a 4-stage ring, chunk swizzle (row >> 1) & 3
#define DMA_CFG 256, 256, 2, 4, 4, 1
    // the 256x256 kernel addresses each operand with 32-bit byte offsets
    if (use_q64(q)) {
      if (q.epi == EPI_DSWIGLU) {
        if (q.offsets) return run_fwd_q64<4, true, EPI_DSWIGLU>(q, stream);
        return run_fwd_q64<4, false, EPI_DSWIGLU>(q, stream);
      }
      if (q.offsets) {
        if (q.epi == EPI_SWIGLU) return run_fwd_q64<4, true, EPI_SWIGLU>(q, stream);
        if (q.epi == EPI_STORE_F32) return run_fwd_q64<4, true, EPI_STORE_F32>(q, stream);
        return run_fwd_q64<4, true, EPI_STORE>(q, stream);
      }
      if (q.epi == EPI_SWIGLU) return run_fwd_q64<4, false, EPI_SWIGLU>(q, stream);
      if (q.epi == EPI_STORE_F32) return run_fwd_q64<4, false, EPI_STORE_F32>(q, stream);
      return run_fwd_q64<4, false, EPI_STORE>(q, stream);
    }
    if (q.epi == EPI_SWIGLU) return run_fwd_dma<DMA_CFG, EPI_SWIGLU>(q, stream);
    if (q.epi == EPI_DSWIGLU) return run_fwd_dma<DMA_CFG, EPI_DSWIGLU>(q, stream);
    if (q.epi == EPI_STORE_F32) return run_fwd_dma<DMA_CFG, EPI_STORE_F32>(q, stream);
    return run_fwd_dma<DMA_CFG, EPI_STORE>(q, stream);
#undef DMA_CFG
  }
  if (q.sched == SCHED_GROUP_M && q.a_kmajor && q.b_kmajor) {
#define FWD_CFG 128, 128, 64, 2, 2, true, true, SCHED_GROUP_M
    if (q.epi == EPI_SWIGLU) return run_bf16<FWD_CFG, EPI_SWIGLU>(q, stream);
    if (q.epi == EPI_DSWIGLU) return run_bf16<FWD_CFG, EPI_DSWIGLU>(q, stream);
    if (q.epi == EPI_STORE_F32) return run_bf16<FWD_CFG, EPI_STORE_F32>(q, stream);
    if (q.epi == EPI_STORE) return run_bf16<FWD_CFG, EPI_STORE>(q, stream);
    return -2;
#undef FWD_CFG
  }
  if (use_q64_bt(q)) {
    if (q.epi == EPI_DSWIGLU) {
      if (q.offsets) return run_fwd_q64<4, true, EPI_DSWIGLU, true>(q, stream);
      return run_fwd_q64<4, false, EPI_DSWIGLU, true>(q, stream);
    }
    if (q.offsets) return run_fwd_q64<4, true, EPI_STORE_F32, true>(q, stream);
    return run_fwd_q64<4, false, EPI_STORE_F32, true>(q, stream);
  }
  if (q.sched == SCHED_GROUP_M && q.a_kmajor && !q.b_kmajor) {
    if (q.epi == EPI_DSWIGLU) return run_bf16<128, 128, 64, 2, 2, true, false, SCHED_GROUP_M, EPI_DSWIGLU>(q, stream);
    if (q.epi == EPI_STORE_F32)
      return run_bf16<128, 128, 64, 2, 2, true, false, SCHED_GROUP_M, EPI_STORE_F32>(q, stream);
    return run_bf16<128, 128, 64, 2, 2, true, false, SCHED_GROUP_M, EPI_STORE>(q, stream);
  }
  if (q.sched == SCHED_GROUP_K && !q.a_kmajor && !q.b_kmajor && q.epi == EPI_STORE_F32 && q.M % 8 == 0 &&
      q.N % 8 == 0 && q.M >= 8 && q.N >= 8)
    return run_wgrad<EPI_STORE_F32>(q, stream);
  if (q.sched == SCHED_GROUP_K && !q.a_kmajor && !q.b_kmajor) {
    if (q.epi == EPI_STORE_F32)
      return run_bf16<128, 128, 64, 2, 2, false, false, SCHED_GROUP_K, EPI_STORE_F32>(q, stream);
    return run_bf16<128, 128, 64, 2, 2, false, false, SCHED_GROUP_K, EPI_STORE>(q, stream);
  }
  return -2;
}


}  // namespace moe
