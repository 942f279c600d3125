// Counting-sort dispatch and token gather.
//
// "Sparse MoE FFN for DFlash-family drafters" (What's here, SparseMoE) sorts
// the (token, slot) pairs once into contiguous per-expert segments; "feat:
// Phase 43 — Sparse/Grouped MoE Dispatch" (sparse_grouped_dispatch) groups
// tokens by a no-grad arg_sort then index_selects them.  Here the sort is a
// stable counting sort over the flat index i = t*k + j, in three kernels:
//   hist : one wave per chunk of kChunk pairs -> per-chunk expert histogram
//   scan : one workgroup per expert: exclusive scan of that expert's column
//          of chunk counts (the chunk's base inside the expert's segment)
//          and the expert's total
//   rank : one wave per chunk: expert offsets = exclusive scan of the totals
//          (the first chunk also writes counts and offsets); then it walks
//          its pairs in order, 64 at a time; a pair's rank among equal
//          experts in the 64-pair step comes from a ballot match over the
//          expert id bits.  pos[i] and perm[pos[i]].
// Up to 512 pairs (decode-sized batches) one wave does all three steps in a
// single launch (dispatch_small_kernel): histogram in LDS, offsets, then the
// same in-order ranking over every pair.
// With the router's per-tile expert loads at hand (moe_route_dispatch), the
// whole sort is one launch, dispatch_tiles_kernel.
// Integer work only: results are bit-exact and order independent.
// The gather copies each token row once per slot into its sorted row with
// 16-byte loads and stores (one wave per token).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kChunk = 256;

__global__ __launch_bounds__(64) void hist_kernel(const int64_t* ids, int P, int E, int32_t* chunk_hist) {
  __shared__ int h[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) h[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  const int end = min(P, base + kChunk);
  for (int i = base + lane; i < end; i += 64) atomicAdd(&h[(int)ids[i]], 1);
  __syncthreads();
  for (int e = lane; e < E; e += 64) chunk_hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// Workgroup e: chunk_hist[b][e] -> exclusive prefix over b (in place) and
// total[e].  Thread i owns chunks [i * per, (i + 1) * per).
__global__ __launch_bounds__(256) void scan_kernel(int32_t* chunk_hist, int nchunks, int E, int32_t* total) {
  __shared__ int part[256];
  const int e = blockIdx.x, i = threadIdx.x;
  const int per = (nchunks + 255) / 256;
  const int b0 = i * per, b1 = min(nchunks, b0 + per);
  int sum = 0;
  for (int b = b0; b < b1; ++b) sum += chunk_hist[(int64_t)b * E + e];
  part[i] = sum;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {  // inclusive Hillis-Steele scan
    const int v = i >= d ? part[i - d] : 0;
    __syncthreads();
    part[i] += v;
    __syncthreads();
  }
  int run = part[i] - sum;
  for (int b = b0; b < b1; ++b) {
    const int c = chunk_hist[(int64_t)b * E + e];
    chunk_hist[(int64_t)b * E + e] = run;  // base of chunk b inside expert e's segment
    run += c;
  }
  if (i == 255) total[e] = part[255];
}

// Walks pairs [base, end) in order, 64 at a time, one wave: a pair's rank among
// equal experts in its 64-pair step comes from a ballot match over the expert
// id bits; the pair goes to next[e] + rank and the step's highest lane of each
// expert advances next[e].  Writes pos[i] and perm[pos[i]].
MOE_DEV void rank_pairs(const int64_t* ids, int base, int end, int E, int* next, int32_t* perm, int32_t* pos) {
  const int lane = threadIdx.x;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s = base; s < end; s += 64) {
    const int i = s + lane;
    const bool act = i < end;
    const int e = act ? (int)ids[i] : 0;
    uint64_t same = __ballot(act);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t m = __ballot(act && ((e >> b) & 1));
      same &= ((e >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(same & lt_mask);
    const int cnt = __popcll(same);
    int p = 0;
    if (act) p = next[e] + rank;
    __syncthreads();
    // the highest lane of each group advances its expert's cursor
    if (act && rank == cnt - 1) next[e] += cnt;
    __syncthreads();
    if (act) {
      pos[i] = p;
      perm[p] = i;
    }
  }
}

__global__ __launch_bounds__(64) void rank_kernel(const int64_t* ids, int P, int E, const int32_t* chunk_base,
                                                  const int32_t* total, int32_t* counts, int32_t* offsets,
                                                  int32_t* perm, int32_t* pos) {
  __shared__ int next[256];
  const int lane = threadIdx.x;
  // expert offsets: exclusive scan of the totals; lane L holds experts 4 L .. 4 L + 3
  int tv[4], loc = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane * 4 + r;
    tv[r] = e < E ? total[e] : 0;
    loc += tv[r];
  }
  int incl = loc;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  int off = incl - loc;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane * 4 + r;
    if (e < E) {
      next[e] = off + chunk_base[(int64_t)blockIdx.x * E + e];
      if (blockIdx.x == 0) {
        counts[e] = tv[r];
        offsets[e] = off;
      }
    }
    off += tv[r];
  }
  if (blockIdx.x == 0 && lane == 63) offsets[E] = P;
  __syncthreads();
  rank_pairs(ids, blockIdx.x * kChunk, min(P, blockIdx.x * kChunk + kChunk), E, next, perm, pos);
}

__global__ __launch_bounds__(64) void dispatch_small_kernel(const int64_t* ids, int P, int E, int32_t* counts,
                                                            int32_t* offsets, int32_t* perm, int32_t* pos) {
  __shared__ int next[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) next[e] = 0;
  __syncthreads();
  for (int i = lane; i < P; i += 64) atomicAdd(&next[(int)ids[i]], 1);
  __syncthreads();
  int tv[4], loc = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane * 4 + r;
    tv[r] = e < E ? next[e] : 0;
    loc += tv[r];
  }
  int incl = loc;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  int off = incl - loc;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane * 4 + r;
    if (e < E) {
      next[e] = off;
      counts[e] = tv[r];
      offsets[e] = off;
    }
    off += tv[r];
  }
  if (lane == 63) offsets[E] = P;
  __syncthreads();
  rank_pairs(ids, 0, P, E, next, perm, pos);
}


// Dispatch from the router's per-tile expert loads, in one launch.  Route
// tile b holds the tokens [b tm, (b + 1) tm), so the pairs [b tm k,
// (b + 1) tm k) of the flat order, and cnt[b][e] of them went to expert e.
// A pair's sorted row is offsets[e] + (pairs of e in earlier tiles) + (its
// rank among the pairs of e in its own tile).  Workgroup g takes the G tiles
// [g G, (g + 1) G), its wave w (of four ranking waves) the tiles from
// g G + w R on, R = ceil(G / 4).  Sums without atomics: thread (q, e) of the
// Q = floor(1024 / E) threads of expert column e reads the rows q, q + Q, ...
// of the [ntiles, E] table (a row is E consecutive ints: the loads of a wave
// are contiguous) and keeps in registers the column's total and, for each
// ranking wave, its sum over the tiles before that wave's first tile; one
// pass through LDS adds the Q partials of a column in q order.  Wave 0 forms
// the offsets (exclusive scan of the totals; workgroup 0 also writes counts
// and offsets); then each ranking wave walks its pairs in order, 64 at a
// time, a pair's rank among equal experts from a ballot match over the
// expert id bits, its cursor per expert in LDS.
// a thread's table loads are all issued before any is used: 32 rows (the
// DSV4 shape's 512 tiles of 64 experts in one batch)
constexpr int kTileThreads = 1024, kRankWaves = 4, kRowsInFlight = 32, kIdsAhead = 8;

__global__ __launch_bounds__(kTileThreads) void dispatch_tiles_kernel(const int64_t* ids, int P, int E,
                                                                      int tile_pairs, int ntiles, int G,
                                                                      const int32_t* cnt, int32_t* counts,
                                                                      int32_t* offsets, int32_t* perm,
                                                                      int32_t* pos) {
  __shared__ int part[kTileThreads][1 + kRankWaves];  // per thread: total, then the ranking waves' prefixes
  __shared__ int cur[kRankWaves][256];
  __shared__ int tot[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b0 = blockIdx.x * G;
  const int R = (G + kRankWaves - 1) / kRankWaves;
  // a ranking wave's pairs, [p_begin, p_end); their first kIdsAhead * 64
  // expert ids are loaded now, so the loads overlap the table sums below
  const int g_end = min(b0 + G, ntiles);
  const int p_begin = min(b0 + wave * R, g_end) * tile_pairs;
  const int p_end = min(P, min(b0 + (wave + 1) * R, g_end) * tile_pairs);
  int ahead[kIdsAhead];
#pragma unroll
  for (int u = 0; u < kIdsAhead; ++u) {
    const int i = p_begin + u * 64 + lane;
    ahead[u] = (wave < kRankWaves && i < p_end) ? (int)ids[i] : 0;
  }
  const int Q = kTileThreads / E;
  const int q = tid / E, e = tid - q * E;
  int acc[1 + kRankWaves] = {0, 0, 0, 0, 0};
  if (q < Q) {
    for (int t0 = q; t0 < ntiles; t0 += kRowsInFlight * Q) {
      int v[kRowsInFlight];
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const int t = t0 + u * Q;
        v[u] = t < ntiles ? cnt[(int64_t)t * E + e] : 0;
      }
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const int t = t0 + u * Q;
        acc[0] += v[u];
#pragma unroll
        for (int w = 0; w < kRankWaves; ++w) acc[1 + w] += t < b0 + w * R ? v[u] : 0;
      }
    }
  }
#pragma unroll
  for (int j = 0; j <= kRankWaves; ++j) part[tid][j] = acc[j];
  __syncthreads();
  if (tid < E) {  // column e = tid: its Q partials in q order
    int s[1 + kRankWaves] = {0, 0, 0, 0, 0};
    for (int qq = 0; qq < Q; ++qq)
#pragma unroll
      for (int j = 0; j <= kRankWaves; ++j) s[j] += part[qq * E + tid][j];
    tot[tid] = s[0];
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) cur[w][tid] = s[1 + w];
  }
  __syncthreads();
  if (wave == 0) {  // offsets: exclusive scan of the totals; lane L holds experts 4 L .. 4 L + 3
    int tv[4], loc = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ee = lane * 4 + r;
      tv[r] = ee < E ? tot[ee] : 0;
      loc += tv[r];
    }
    int incl = loc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int x = __shfl_up(incl, d, 64);
      if (lane >= d) incl += x;
    }
    int off = incl - loc;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ee = lane * 4 + r;
      if (ee < E) {
#pragma unroll
        for (int w = 0; w < kRankWaves; ++w) cur[w][ee] += off;
        if (blockIdx.x == 0) {
          counts[ee] = tv[r];
          offsets[ee] = off;
        }
      }
      off += tv[r];
    }
    if (blockIdx.x == 0 && lane == 63) offsets[E] = P;
  }
  __syncthreads();
  if (wave >= kRankWaves) return;
  int* next = cur[wave];
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s0 = p_begin, u = 0; s0 < p_end; s0 += 64, ++u) {
    const int i = s0 + lane;
    const bool act = i < p_end;
    int ei = 0;
    if (u < kIdsAhead) {
#pragma unroll
      for (int j = 0; j < kIdsAhead; ++j)
        if (j == u) ei = ahead[j];
    } else if (act) {
      ei = (int)ids[i];
    }
    uint64_t same = __ballot(act);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t m = __ballot(act && ((ei >> b) & 1));
      same &= ((ei >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(same & lt_mask);
    const int n_e = __popcll(same);
    const int p = act ? next[ei] + rank : 0;
    // one wave: its LDS operations complete in issue order, so every lane
    // has read its cursor before the group's highest lane advances it
    __builtin_amdgcn_wave_barrier();
    if (act && rank == n_e - 1) next[ei] += n_e;
    __builtin_amdgcn_wave_barrier();
    if (act) {
      pos[i] = p;
      perm[p] = i;
    }
  }
}

__global__ __launch_bounds__(256) void zero_kernel(int E, int32_t* counts, int32_t* offsets) {
  for (int e = threadIdx.x; e <= E; e += 256) {
    if (e < E) counts[e] = 0;
    offsets[e] = 0;
  }
}

// One wave per token; 16-byte chunks; each x row read once, written k times.
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* x, int T, int k, int row_bytes,
                                                     const int32_t* pos, uint8_t* xs) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nvec = row_bytes >> 4;
  const u32x4_t* src = (const u32x4_t*)(x + (int64_t)t * row_bytes);
  int dst_row[8];
  const int kk = k < 8 ? k : 8;
  for (int j = 0; j < kk; ++j) dst_row[j] = pos[(int64_t)t * k + j];
  for (int c = lane; c < nvec; c += 64) {
    const u32x4_t v = src[c];
    for (int j = 0; j < kk; ++j) ((u32x4_t*)(xs + (int64_t)dst_row[j] * row_bytes))[c] = v;
    for (int j = 8; j < k; ++j) ((u32x4_t*)(xs + (int64_t)pos[(int64_t)t * k + j] * row_bytes))[c] = v;
  }
}

}  // namespace

size_t dispatch_ws_bytes(int64_t P, int64_t E) {
  const int64_t nchunks = (P + kChunk - 1) / kChunk;
  return (size_t)((nchunks > 0 ? nchunks : 1) * E * 4 + E * 4 + 256);
}

int launch_dispatch(const int64_t* ids, int64_t T, int64_t k, int64_t E, int32_t* counts, int32_t* offsets,
                    int32_t* perm, int32_t* pos, void* ws, hipStream_t stream) {
  const int P = (int)(T * k);
  const int nchunks = (P + kChunk - 1) / kChunk;
  int32_t* chunk_hist = (int32_t*)ws;
  int32_t* total = chunk_hist + (int64_t)(nchunks > 0 ? nchunks : 1) * E;
  if (nchunks == 0) {  // no pairs: every count and offset is zero
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(256), 0, stream, (int)E, counts, offsets);
    return hipGetLastError() == hipSuccess ? 0 : -4;
  }
  if (P <= 512) {  // one wave does the whole sort: one launch instead of three
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(64), 0, stream, ids, P, (int)E, counts, offsets, perm,
                       pos);
    return hipGetLastError() == hipSuccess ? 0 : -4;
  }
  hipLaunchKernelGGL(hist_kernel, dim3(nchunks), dim3(64), 0, stream, ids, P, (int)E, chunk_hist);
  hipLaunchKernelGGL(scan_kernel, dim3((unsigned)E), dim3(256), 0, stream, chunk_hist, nchunks, (int)E, total);
  hipLaunchKernelGGL(rank_kernel, dim3(nchunks), dim3(64), 0, stream, ids, P, (int)E, chunk_hist, total, counts,
                     offsets, perm, pos);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Tiles per workgroup of dispatch_tiles_kernel: at most 64 workgroups (each
// reads all tile loads, ntiles * E ints: 128 KB at the DSV4 shape).
int launch_dispatch_tiles(const int64_t* ids, int64_t T, int64_t k, int64_t E, int tm, const int32_t* tile_counts,
                          int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos, hipStream_t stream) {
  const int64_t P = T * k;
  if (P == 0) {
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(256), 0, stream, (int)E, counts, offsets);
    return hipGetLastError() == hipSuccess ? 0 : -4;
  }
  const int ntiles = (int)((T + tm - 1) / tm);
  const int G = (ntiles + 63) / 64;
  const int wgs = (ntiles + G - 1) / G;
  hipLaunchKernelGGL(dispatch_tiles_kernel, dim3((unsigned)wgs), dim3(kTileThreads), 0, stream, ids, (int)P,
                     (int)E, (int)(tm * k), ntiles, G, tile_counts, counts, offsets, perm, pos);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_gather(const void* x, int64_t T, int64_t k, int64_t row_bytes, const int32_t* pos, void* x_sorted,
                  hipStream_t stream) {
  if (T == 0) return 0;
  dim3 grid((unsigned)((T + 3) / 4)), block(256);
  hipLaunchKernelGGL(gather_kernel, grid, block, 0, stream, (const uint8_t*)x, (int)T, (int)k, (int)row_bytes, pos,
                     (uint8_t*)x_sorted);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace moe
