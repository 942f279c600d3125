// Host-side launchers of the MoE kernels (internal to libmoe_mi355x.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct RouteLaunch {
  const void* x;
  const void* w_router;
  const void* w_gate;
  const float* bias;
  float* logits;
  float* weights;
  int64_t* ids;
  float* gate;
  float* score_sums;  // [E] column sums of the scores, or null
  void* ws;           // scratch (route_ws_bytes), required with score_sums; null: no split reduction
  size_t ws_bytes;
  int32_t* tile_counts;  // [tiles, E] per-tile expert loads (tiles of route_tile_tokens tokens), or null
  // with tile_counts, when the whole batch is one tile of the LDS-ring router: the counting sort
  // (moe_dispatch's counts, offsets, perm, pos) done by the selecting workgroup; *dispatched is set to
  // 1 when it was (else 0, and the caller sorts from tile_counts)
  int32_t *d_counts, *d_offsets, *d_perm, *d_pos;
  int* dispatched;
  int64_t T, H, E, k;
  int score, renorm, logits_in, bf16;
};
int launch_route(const RouteLaunch& p, hipStream_t stream);
int route_tile(int bf16);
// tokens per tile of the router launch for these sizes (ncols = E + 1 with a shared gate, else E)
int route_tile_tokens(int64_t T, int64_t H, int64_t ncols, int bf16, int logits_in);
size_t route_ws_bytes(int64_t T, int64_t H, int64_t E, int bf16);
int launch_aux_loss(const float* sums, const int32_t* counts, int64_t T, int64_t k, int64_t E, float alpha, float* loss,
                    float* coef, hipStream_t stream);
int launch_score(int score, const float* l, float* s, int64_t n, hipStream_t stream);

size_t dispatch_ws_bytes(int64_t P, int64_t E);
int launch_dispatch(const int64_t* ids, int64_t T, int64_t k, int64_t E, int32_t* counts, int32_t* offsets,
                    int32_t* perm, int32_t* pos, void* ws, hipStream_t stream);
int launch_gather(const void* x, int64_t T, int64_t k, int64_t row_bytes, const int32_t* pos, void* x_sorted,
                  hipStream_t stream);
// The dispatch from the router's per-tile expert loads (tile_counts [ntiles, E], tiles of tm tokens):
// counts, offsets, perm, pos in one launch.  ws: dispatch_tiles_ws_bytes.
int launch_dispatch_tiles(const int64_t* ids, int64_t T, int64_t k, int64_t E, int tm, const int32_t* tile_counts,
                          int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos, hipStream_t stream);

// ---- grouped GEMM engine:  C[m, n] = sum_k A(m, k) * B(n, k)
enum GemmSched { SCHED_GROUP_M = 0, SCHED_GROUP_K = 1 };
enum GemmEpi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2, EPI_STORE_F32 = 3 };

struct GemmProblem {
  int sched;  // SCHED_GROUP_M: group g owns rows [off[g], off[g+1]) of A and C, B_g = B + g*strideB.
              // SCHED_GROUP_K: group g owns reduction rows [off[g], off[g+1]), C_g = C + g*strideC.
  int epi;
  // A(m,k): a_kmajor ? A[row(m)*lda + k] : A[k*lda + m];  row(m) = a_idx ? a_idx[m] / a_div : m
  const void* A;
  int64_t lda;
  int a_kmajor;
  const int32_t* a_idx;
  int a_div;
  // B(n,k): b_kmajor ? B[n*ldb + k] : B[k*ldb + n]
  const void* B;
  int64_t ldb, strideB;
  int b_kmajor;
  void* C;
  int64_t ldc, strideC;
  // EPI_SWIGLU: aux = optional fp32 [rows, 2*n_half] save of (gate | up);
  // EPI_DSWIGLU: aux = saved fp32 (gate | up) input, aux_out = (dgate | dup) output (dtype).
  void* aux;
  void* aux_out;
  int64_t ld_aux;
  const int32_t* offsets;  // [G+1] device, or null for one group
  int G;
  int64_t M, N, K;  // GROUP_M: M = rows bound (total rows when offsets is null), N, K
                    // GROUP_K: M x N per group; K = rows when offsets is null
  int64_t n_half;   // SWIGLU / DSWIGLU: I
  int64_t rows_bound;  // GROUP_M with offsets: total rows (T*k), for the tile-slot bound
  int c_f16;           // EPI_STORE_F32: write C as binary16 instead of fp32
  void* split_ws;      // optional fp32 scratch: lets a one-group streaming GEMM with few tiles split K
  // Split bf16 operand (streaming kernel only): with A_lo, A(m, k) is the pair A + A_lo, both bf16 with
  // A's layout (no a_idx), multiplied as two MFMA passes into the same fp32 accumulators; with C_lo, an
  // EPI_SWIGLU epilogue also writes h - bf16(h) rounded to bf16 there (C's layout), the lo part of h.
  const void* A_lo;
  void* C_lo;
  // EPI_STORE_F32, one group, 256x256 kernel: splits > 0 fixes the K split (else the kernel picks it from
  // the CU count); with partials_only and a K split the fp32 partials [splits][M][N] stay in split_ws
  // (no reduce kernel), for a consumer that adds them itself
  int splits;
  int partials_only;
};
// K splits the 256x256 kernel will take for q (an EPI_STORE_F32 problem without offsets), or 0 when
// launch_gemm runs q on another kernel
int gemm_q64_splits(const GemmProblem& q, int bf16);
// bytes of split_ws the GEMM would use for q (0: it does not split K)
size_t gemm_split_ws_bytes(const GemmProblem& q, int bf16);
// true when launch_gemm runs q on the streaming kernel (few rows per group)
bool gemm_uses_stream(const GemmProblem& q, int bf16);
// true when the streaming kernel can take q with a split operand (A_lo / C_lo)
bool gemm_split_operand_ok(const GemmProblem& q, int bf16);
int launch_gemm(const GemmProblem& p, int bf16, hipStream_t stream);

// ---- combine / backward helpers (expert outputs y and shared output s are fp32)
// y and s: fp32, or binary16 when y_f16
int launch_combine(const void* y, int y_f16, const int32_t* pos, const float* weights, const void* s, const float* gate,
                   void* out, int64_t T, int64_t k, int64_t H, int bf16, hipStream_t stream);
int launch_combine_bwd(const void* dout, const void* y, int y_f16, const int32_t* pos, const float* weights, const void* s,
                       const float* gate, void* dy, float* dweights, void* ds, float* dz, int64_t T, int64_t k,
                       int64_t H, int bf16, hipStream_t stream);
int launch_router_bwd(const float* logits, const int64_t* ids, const float* weights, const float* dweights,
                      const float* aux_coef, float* dlogits, int64_t T, int64_t E, int64_t k, int score, int renorm,
                      hipStream_t stream);
// p[0 .. n) = 0 (a fill kernel: no memset node in a captured graph)
int launch_zero_f32(float* p, int64_t n, hipStream_t stream);
// out = x / sqrt(mean(x^2) + eps) * g per row (x, g, out in the layer dtype)
int launch_rmsnorm(const void* x, const void* g, float eps, void* out, int64_t T, int64_t H, int bf16,
                   hipStream_t stream);
// parallel dense + MoE block output: routed sum of y (binary16 when y_f16), dense output s, three norms,
// residual and layer scalar; H <= 8192, k <= 8
int launch_block_out(const void* y, int y_f16, const int32_t* pos, const float* weights, const void* s,
                     const void* residual, const void* g1, const void* g2, const void* g, float eps, float scalar,
                     void* out, int64_t T, int64_t k, int64_t H, int bf16, hipStream_t stream);
// out[e, h] = sum_t a[t, e] * b[t, h]  (a fp32 [T,E], b dtype [T,H], out fp32); fixed order.
// With a2 ([T] fp32), also out2[h] = sum_t a2[t] b[t, h] (in the same pass when it can);
// ws: rowreduce_ws_bytes(T, E + 1, H) then.
size_t rowreduce_ws_bytes(int64_t T, int64_t E, int64_t H);
int launch_rowreduce(const float* a, const float* a2, const void* b, void* out, void* out2, int64_t T, int64_t E,
                     int64_t H, int bf16, void* ws, hipStream_t stream);
// dx[t] = sum_j dxs[pos[t,j]] + dxsh[t] + sum_e dl[t,e] w_router[e] + dz[t] w_gate
// (dxs, dxsh: binary16 in a bf16 layer, fp32 in an fp32 layer)
int launch_dx_sum(const void* dxs, const int32_t* pos, const void* dxsh, const float* dl, const void* w_router,
                  const float* dz, const void* w_gate, void* dx, int64_t T, int64_t k, int64_t E, int64_t H, int bf16,
                  hipStream_t stream);
int launch_balance(const int64_t* ids, int32_t* counts, float* bias, float rate, int64_t T, int64_t k, int64_t E,
                   hipStream_t stream);
// plain HBM streams (kind 0 read, 1 write, 2 copy) of `bytes` bytes over wgs workgroups of 256 threads
int launch_probe(int kind, const void* src, void* dst, int64_t bytes, int wgs, hipStream_t stream);

}  // namespace moe
