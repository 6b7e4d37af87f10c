// kernels.hpp -- device kernels of the fused LM-head + cross-entropy path.
//
//   target_logit_kernel z_y = H_n . W[y_n] per row (CCE, arXiv 2411.09009,
//                       Sec. 4.1 / Alg. 1, the indexed matrix multiplication).
//   fwd_lse_kernel      Z tile = W_v H_n^T on MFMA; online max / sum-exp per
//                       token row over this workgroup's vocabulary range
//                       (Sec. 4.2 / Alg. 2 for the blockwise log-sum-exp;
//                       online normaliser of Sec. 2).
//   lse_combine_kernel  merges the per-split (max, sum) partials of a row in a
//                       fixed order into LSE and the row loss (replaces the
//                       paper's spin-locked log-add-exp), plus per-block sums.
//   finalize_kernel     fixed-order scalar loss, valid-row count, row scale.
//   bwd_prep_kernel     the same count / scale for a standalone backward.
//   bwd_band_kernel     one backward launch of two tile kinds:
//     dz_tile           recomputes a logits tile and writes
//                       dZ = g_n (softmax - onehot) for one band into the
//                       workspace, with 64x64 filter flags (CCE Alg. 4, first
//                       half; gradient filtering of Sec. 4.3);
//     grad_tile         the band contractions dH[band rows] (+)= dZ W[band
//                       vocab] and dW[band vocab] (+)= dZ^T H[band rows]
//                       (Alg. 4, second half, done as two ordinary MFMA GEMMs
//                       without locks), float or bf16 outputs.
//   compact_*, zero_ignored_rows_kernel   ignored-row compaction (CCE App. B).
//   fill / scale / clear kernels          small helpers.
// vocab_sort.hpp holds the kernels of the sorted vocabulary (CCE Sec. 4.3).
#pragma once

#include "tile_dma.hpp"
#include "tile_mma.hpp"

namespace flce {

struct Header {           // first 256 bytes of the workspace
  int status;             // bit 0: target outside [0, V) and != ignore_index
  int count;              // non-ignored rows
  float gscale;           // g for mean / sum: dloss / max(count, 1) or dloss
  int nvalid;             // with row compaction: rows whose target is not ignore_index
  // gradient filter: 64-wide K blocks of the filtered gradient contractions
  // that ran / that exist, summed over the tiles of the last backward
  unsigned long long kblk[2];
  float pad[56];
};
static_assert(sizeof(Header) == 256, "the header is the first 256 bytes of the workspace");

// The LDS row table of a compacted dW^T contraction holds NS / 2 entries per
// parity, i.e. 32 per 64-row filter block of the band.
constexpr int kFilterHalfPerBlock = 32;

// The bf16 core: four fragment sets and the barrier after a stage's second
// sub-step (gemm_tile_dma2), except with a gathered A, whose row table and
// per-lane indices leave no room for the two extra fragment sets (they
// spill): two sets and the barrier before the last sub-step (gemm_tile_dma).
template <bool AT, bool BT, class Active, bool GATHER_A>
__device__ __forceinline__ void gemm_tile_dma_any(const Operand& A, const Operand& B, int m0,
                                                  int n0, int nsteps, Active active,
                                                  f32x16 (&acc)[4][4], char* lds, L2Split sa,
                                                  L2Split sb) {
  if constexpr (GATHER_A)
    gemm_tile_dma<AT, BT, Active, GATHER_A>(A, B, m0, n0, nsteps, active, acc, lds, sa, sb);
  else
    gemm_tile_dma2<AT, BT, Active, GATHER_A>(A, B, m0, n0, nsteps, active, acc, lds, sa, sb);
}

// K elements of one pass of a tile contraction: 64 for bf16 (LDS-DMA core,
// whole 128-byte lines per operand row), 32 for fp32 (register-staged core).
template <typename T>
constexpr int step_k() { return sizeof(T) == 2 ? kDmaKStep : 32; }

// A 256x256 tile contraction over K = [0, K): bf16 through the LDS-DMA core,
// fp32 through the register-staged core.  active(s) covers K
// [s step_k, (s + 1) step_k).
template <typename T, bool AT, bool BT, class Active, bool GATHER_A = false>
__device__ __forceinline__ void tile_contract(const Operand& A, const Operand& B, int m0, int n0,
                                              int K, const Active& active, f32x16 (&acc)[4][4],
                                              char* lds) {
  const int nsteps = (K + step_k<T>() - 1) / step_k<T>();
  // Every contraction here visits its tiles in the grouped order of
  // grouped_tile with 4 tile rows (A side) per group, so the ~32 workgroups
  // that run together on one XCD form about 4 A blocks x 8 B blocks: an A
  // block is shared by 8 consecutive B tiles, a B block by 4 consecutive A
  // tiles, and consecutive tiles have distinct residues.
  if constexpr (sizeof(T) == 2)
    gemm_tile_dma_any<AT, BT, Active, GATHER_A>(A, B, m0, n0, nsteps, active, acc, lds,
                                             L2Split{(n0 / kTile) & 7, 8},
                                             L2Split{(m0 / kTile) & 3, 4});
  else gemm_tile<T, AT, BT>(A, B, m0, n0, nsteps, active, acc, lds);
}

// The rescaled merges of (max, sum-exp) pairs below are written with explicit
// fmaf: left to the compiler, a * b + c * d contracts to either fma(a, b, c d)
// or fma(c, d, a b) depending on the surrounding code, which moved the last
// bit of a sum between builds of the same source.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Max and sum-exp of one 32-column block (token rows) over this lane's 64
// logits of the tile; MASKED: rows of the wave block at or past `lim`
// (V - first row of the block) are left out (last vocabulary tile).
template <int J, bool MASKED>
__device__ __forceinline__ void fwd_column(const f32x16 (&acc)[4][4], float& m, float& s, int lim,
                                           int lane) {
  auto val = [&](int i, int r) {
    return !MASKED || acc_row(i, r, lane) < lim ? acc[i][J][r] : -INFINITY;
  };
  float tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, val(i, r));
  m = tmax;
  if (tmax == -INFINITY) {
    s = 0.f;
    return;
  }
  const float ml = tmax * kLog2e;
  float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s4[i] += fast_exp2(fmaf(val(i, r), kLog2e, -ml));
  s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
}

// ------------------------------------------------------------- forward ----
// One 256 (vocabulary) x 256 (token rows) logits tile per workgroup, for the
// token rows [nb0, nb0 + ns) of a band: Z = W_v H_n^T stays in registers; the
// tile's per-row max m and sum s = sum_v exp(Z - m) go to
// part_m / part_s [vocab tile][row of the band].  (The target logits come
// from target_logit_kernel.)
template <typename T>
__global__ void __launch_bounds__(kThreads, 1)
fwd_lse_kernel(const T* __restrict__ H, const T* __restrict__ W,
               int N, int D, int V, int nb0, int ns, int TMv, int TNn,
               float* __restrict__ part_m, float* __restrict__ part_s,
               Header* __restrict__ hdr, const int* __restrict__ rowmap) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  if (nb0 == 0 && blockIdx.x == 0 && threadIdx.x == 0) hdr->status = 0;   // start of a forward
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  int tm, tn;
  grouped_tile(t, TMv, TNn, 4, tm, tn);
  const int v0 = tm * kTile, n0 = nb0 + tn * kTile;
  // rows are compacted positions when rowmap is given (the row itself is
  // rowmap[c]); tiles past the non-ignored rows have nothing to do
  const int nval = rowmap ? hdr->nvalid : N;
  if (n0 >= nval) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const Operand A{reinterpret_cast<const char*>(W), D, V, D};
  const Operand B{reinterpret_cast<const char*>(H), D, nval, D, rowmap};
  f32x16 acc[4][4];
  tile_contract<T, false, false>(A, B, v0, n0, D, AllActive{}, acc, lds);

  const int vw = v0 + wm * 128;  // first vocabulary row of this wave's block
  float m[4], s[4];
  if (vw + 128 > V) {   // last vocabulary tile: rows past V are left out
    const int lim = V - vw;
    fwd_column<0, true>(acc, m[0], s[0], lim, lane);
    fwd_column<1, true>(acc, m[1], s[1], lim, lane);
    fwd_column<2, true>(acc, m[2], s[2], lim, lane);
    fwd_column<3, true>(acc, m[3], s[3], lim, lane);
  } else {
    fwd_column<0, false>(acc, m[0], s[0], 0, lane);
    fwd_column<1, false>(acc, m[1], s[1], 0, lane);
    fwd_column<2, false>(acc, m[2], s[2], 0, lane);
    fwd_column<3, false>(acc, m[3], s[3], 0, lane);
  }

  // merge the two lanes holding one token column, then the two waves
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float mo = __shfl_xor(m[j], 32), so = __shfl_xor(s[j], 32);
    const float M = fmaxf(m[j], mo);
    s[j] = (M == -INFINITY) ? 0.f
                            : fmaf(s[j], fast_exp2((m[j] - M) * kLog2e),
                                   so * fast_exp2((mo - M) * kLog2e));
    m[j] = M;
  }
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      red[(wn * 128 + j * 32 + lane) * 2 + 0] = m[j];
      red[(wn * 128 + j * 32 + lane) * 2 + 1] = s[j];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = wn * 128 + j * 32 + lane;
      const float mo = red[c * 2 + 0], so = red[c * 2 + 1];
      const float M = fmaxf(m[j], mo);
      const float S = (M == -INFINITY) ? 0.f
                                       : fmaf(s[j], fast_exp2((m[j] - M) * kLog2e),
                                              so * fast_exp2((mo - M) * kLog2e));
      const int nl = tn * kTile + c;   // row within the band
      if (nl < ns) {
        part_m[(int64_t)tm * ns + nl] = M;
        part_s[(int64_t)tm * ns + nl] = S;
      }
    }
  }
}

// Target logits z_y of positions [0, npos): z[pos] = H[n] . W[y_n] for row n
// = pos (rowmap[pos] with compaction) when y_n is a vocabulary row (CCE
// Sec. 4.1, Alg. 1: the indexed matrix multiplication as its own pass).  One
// wave per position, 4 per block: lane L takes d = E L + 64 E i (E = 8 bf16
// or 4 float per 16-byte load), fp32 products summed in a fixed order, then
// a fixed xor butterfly over the lanes.  D % 8 == 0, rows 16-byte aligned.
template <typename T>
__global__ void __launch_bounds__(256)
target_logit_kernel(const T* __restrict__ H, const T* __restrict__ W, const int64_t* __restrict__ y,
                    int npos, int D, int V, const int* __restrict__ rowmap, float* __restrict__ zy) {
  constexpr int E = 16 / sizeof(T);
  const int pos = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (pos >= npos) return;
  const int n = rowmap ? rowmap[pos] : pos;
  const int64_t yy = y[n];
  if (yy < 0 || yy >= V) return;   // ignored or invalid target: z is not used
  const T* h = H + (int64_t)n * D;
  const T* w = W + yy * D;
  float acc = 0.f;
  for (int d = lane * E; d < D; d += 64 * E) {
    if constexpr (sizeof(T) == 2) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(h + d);
      const u32x4 b = *reinterpret_cast<const u32x4*>(w + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(__builtin_bit_cast(float, a[e] << 16), __builtin_bit_cast(float, b[e] << 16), acc);
        acc = fmaf(__builtin_bit_cast(float, a[e] & 0xffff0000u),
                   __builtin_bit_cast(float, b[e] & 0xffff0000u), acc);
      }
    } else {
      // float rows are loaded as float vectors (an integer-vector load
      // reinterpreted element by element was miscompiled with packed fp32
      // codegen disabled: overlapping load registers, one product repeated)
      const f32x4 a = *reinterpret_cast<const f32x4*>(h + d);
      const f32x4 b = *reinterpret_cast<const f32x4*>(w + d);
      acc = fmaf(a[0], b[0], acc);
      acc = fmaf(a[1], b[1], acc);
      acc = fmaf(a[2], b[2], acc);
      acc = fmaf(a[3], b[3], acc);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) zy[pos] = acc;
}

// Fixed-order block reduction of (double sum, int count) over 256 threads.
__device__ __forceinline__ void block_reduce_256(double& s, int& c, double* sh_s, int* sh_c) {
  const int tid = threadIdx.x;
  sh_s[tid] = s;
  sh_c[tid] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      sh_s[tid] += sh_s[tid + w];
      sh_c[tid] += sh_c[tid + w];
    }
    __syncthreads();
  }
  s = sh_s[0];
  c = sh_c[0];
}

// One block = 16 token rows x 16 slices of the vocabulary tiles: slice sl
// merges partials sl, sl + 16, ... of its row (online, rescaling only when the
// max grows), then the 16 slice results of a row merge in slice order.
constexpr int kCombineRows = 16;

__global__ void __launch_bounds__(256)
lse_combine_kernel(const float* __restrict__ part_m, const float* __restrict__ part_s,
                   const float* __restrict__ zy, const int64_t* __restrict__ y, int N, int V,
                   int Tv, int nb0, int ns, int64_t ignore, float* __restrict__ lse,
                   float* __restrict__ loss_rows, double* __restrict__ blk_sum,
                   int* __restrict__ blk_cnt, Header* __restrict__ hdr,
                   const int* __restrict__ rowmap) {
  __shared__ float sh_m[16][kCombineRows], sh_sum[16][kCombineRows];
  __shared__ double sh_s[256];
  __shared__ int sh_c[256];
  const int r = threadIdx.x % kCombineRows, sl = threadIdx.x / kCombineRows;
  const int nl = blockIdx.x * kCombineRows + r;   // row within the band
  // with compaction, positions past the non-ignored rows hold the ignored
  // rows: no partials were made for them, their outputs are 0
  const bool live = nl < ns && (!rowmap || nb0 + nl < hdr->nvalid);
  float M = -INFINITY, S = 0.f;
  if (live) {
    // partials k = sl, sl + 16, ... in increasing order; the loads of eight
    // of them go out together, ahead of the dependent merges
    constexpr int kBatch = 8;
    for (int k0 = sl; k0 < Tv; k0 += 16 * kBatch) {
      float mb[kBatch], sb[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int k = k0 + 16 * u;
        mb[u] = k < Tv ? part_m[(int64_t)k * ns + nl] : -INFINITY;
        sb[u] = k < Tv ? part_s[(int64_t)k * ns + nl] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float m = mb[u], sk = sb[u];
        if (m == -INFINITY) continue;
        if (m <= M) {
          S = fmaf(sk, fast_exp2((m - M) * kLog2e), S);
        } else {
          S = fmaf(S, fast_exp2((M - m) * kLog2e), sk);   // M = -inf: S = 0 * 0 + sk
          M = m;
        }
      }
    }
  }
  sh_m[sl][r] = M;
  sh_sum[sl][r] = S;
  __syncthreads();
  double s = 0.0;
  int c = 0;
  if (sl == 0 && nl < ns && !live) {
    const int n = rowmap[nb0 + nl];
    lse[n] = 0.f;
    loss_rows[n] = 0.f;
  }
  if (sl == 0 && live) {
    float Mx = -INFINITY;
    for (int q = 0; q < 16; ++q) Mx = fmaxf(Mx, sh_m[q][r]);
    float St = 0.f;
    for (int q = 0; q < 16; ++q)
      St = fmaf(sh_sum[q][r], fast_exp2((sh_m[q][r] - Mx) * kLog2e), St);
    const float l = Mx + fast_log2(St) * kLn2;
    const int pos = nb0 + nl;                   // position (zy is by position)
    const int n = rowmap ? rowmap[pos] : pos;   // row
    lse[n] = l;
    const int64_t yy = y[n];
    float lr = 0.f;
    if (yy != ignore) {
      c = 1;
      if (yy < 0 || yy >= V) {
        lr = __builtin_nanf("");
        atomicOr(&hdr->status, 1);
      } else {
        lr = l - zy[pos];
      }
    }
    loss_rows[n] = lr;
    s = (double)lr;
  }
  block_reduce_256(s, c, sh_s, sh_c);
  if (threadIdx.x == 0) {
    blk_sum[nb0 / kCombineRows + blockIdx.x] = s;
    blk_cnt[nb0 / kCombineRows + blockIdx.x] = c;
  }
}

// reduction: 0 mean, 1 sum, 2 none.  One block of 256 threads.
__global__ void __launch_bounds__(256)
finalize_kernel(const double* __restrict__ blk_sum, const int* __restrict__ blk_cnt, int nblk,
                int reduction, float* __restrict__ loss, const float* __restrict__ dloss,
                Header* __restrict__ hdr) {
  __shared__ double sh_s[256];
  __shared__ int sh_c[256];
  double s = 0.0;
  int c = 0;
  for (int k = threadIdx.x; k < nblk; k += 256) {
    s += blk_sum[k];
    c += blk_cnt[k];
  }
  block_reduce_256(s, c, sh_s, sh_c);
  if (threadIdx.x == 0) {
    const int cl = c > 1 ? c : 1;
    if (loss != nullptr && reduction != 2) *loss = (float)(reduction == 0 ? s / cl : s);
    const float up = dloss ? dloss[0] : 1.f;
    hdr->count = c;
    hdr->gscale = reduction == 0 ? up / (float)cl : up;
    hdr->kblk[0] = hdr->kblk[1] = 0ull;
  }
}

// Standalone backward: clear status, count rows, flag bad targets, row scale.
__global__ void __launch_bounds__(256)
bwd_prep_kernel(const int64_t* __restrict__ y, int N, int V, int64_t ignore, int reduction,
                const float* __restrict__ dloss, Header* __restrict__ hdr) {
  __shared__ double sh_s[256];
  __shared__ int sh_c[256];
  int c = 0, bad = 0;
  for (int n = threadIdx.x; n < N; n += 256) {
    const int64_t yy = y[n];
    if (yy != ignore) {
      ++c;
      bad |= (yy < 0 || yy >= V);
    }
  }
  double s = (double)bad;
  block_reduce_256(s, c, sh_s, sh_c);
  if (threadIdx.x == 0) {
    const int cl = c > 1 ? c : 1;
    const float up = (dloss && reduction != 2) ? dloss[0] : 1.f;
    hdr->status = s > 0.0 ? 1 : 0;
    hdr->count = c;
    hdr->gscale = reduction == 0 ? up / (float)cl : up;
    hdr->kblk[0] = hdr->kblk[1] = 0ull;
  }
}

// ------------------------------------------------- ignored-row compaction ----
// rowmap lists the rows whose target is not ignore_index, in order, then the
// ignored rows, in order; hdr->nvalid counts the former.  Blocks of
// kCompactRows rows: count, one-block exclusive scan of the counts, scatter.
constexpr int kCompactRows = 1024;

__device__ __forceinline__ int block_sum_256(int v, int* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  const int r = sh[0];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(256)
compact_count_kernel(const int64_t* __restrict__ y, int N, int64_t ignore, int* __restrict__ blk) {
  __shared__ int sh[256];
  int c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = blockIdx.x * kCompactRows + threadIdx.x * 4 + i;
    c += (n < N && y[n] != ignore) ? 1 : 0;
  }
  const int tot = block_sum_256(c, sh);
  if (threadIdx.x == 0) blk[blockIdx.x] = tot;
}

// blk[b] <- valid rows in blocks before b; hdr->nvalid <- all valid rows
__global__ void __launch_bounds__(1024)
compact_scan_kernel(int* __restrict__ blk, int nblk, Header* __restrict__ hdr) {
  __shared__ int sh[1024];
  int carry = 0;
  for (int base = 0; base < nblk; base += 1024) {
    const int i = base + (int)threadIdx.x;
    const int v = i < nblk ? blk[i] : 0;
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {   // inclusive scan (Hillis-Steele)
      const int a = (int)threadIdx.x >= o ? sh[threadIdx.x - o] : 0;
      __syncthreads();
      sh[threadIdx.x] += a;
      __syncthreads();
    }
    if (i < nblk) blk[i] = carry + sh[threadIdx.x] - v;
    carry += sh[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) hdr->nvalid = carry;
}

__global__ void __launch_bounds__(256)
compact_scatter_kernel(const int64_t* __restrict__ y, int N, int64_t ignore,
                       const int* __restrict__ blk, const Header* __restrict__ hdr,
                       int* __restrict__ rowmap) {
  __shared__ int sh[256];
  const int b = blockIdx.x, t = threadIdx.x;
  bool f[4];
  int c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = b * kCompactRows + t * 4 + i;
    f[i] = n < N && y[n] != ignore;
    c += f[i] ? 1 : 0;
  }
  sh[t] = c;   // exclusive scan of the per-thread counts
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int a = t >= o ? sh[t - o] : 0;
    __syncthreads();
    sh[t] += a;
    __syncthreads();
  }
  const int before = sh[t] - c;                    // valid rows of this block before thread t
  int pv = blk[b] + before;                        // next position of a valid row
  int pi = hdr->nvalid + (b * kCompactRows - blk[b]) + (t * 4 - before);   // of an ignored row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = b * kCompactRows + t * 4 + i;
    if (n < N) rowmap[f[i] ? pv++ : pi++] = n;
  }
}

// dH rows of the ignored rows (positions nvalid .. N of rowmap) <- 0; a row
// is row_bytes long (a multiple of 16: D % 8 == 0).
__global__ void __launch_bounds__(256)
zero_ignored_rows_kernel(const int* __restrict__ rowmap, const Header* __restrict__ hdr, int N,
                         int row_bytes, char* __restrict__ dH) {
  const int c0 = blockIdx.x * 16;
  const int nval = hdr->nvalid;
  for (int c = c0 > nval ? c0 : nval; c < c0 + 16 && c < N; ++c) {
    u32x4* row = reinterpret_cast<u32x4*>(dH + (int64_t)rowmap[c] * row_bytes);
    for (int i = threadIdx.x; i < row_bytes / 16; i += 256) row[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// p[i] *= s[0] over n floats (p 16-byte aligned): the upstream scalar applied
// to gradients computed with an upstream gradient of 1.
__global__ void scale_f32_kernel(float* __restrict__ p, int64_t n, const float* __restrict__ s) {
  const float g = s[0];
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  f32x4* __restrict__ p4 = reinterpret_cast<f32x4*>(p);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    p4[i] = p4[i] * g;
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] *= g;
}

// The same for bf16 values: p[i] = bf16(p[i] * s[0]) (round to nearest even),
// n a multiple of 8, p 16-byte aligned.
__global__ void scale_bf16_kernel(uint16_t* __restrict__ p, int64_t n, const float* __restrict__ s) {
  const float g = s[0];
  const int64_t n8 = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  u32x4* __restrict__ p8 = reinterpret_cast<u32x4*>(p);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const u32x4 v = p8[i];
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = pack_bf16x2(__builtin_bit_cast(float, v[e] << 16) * g,
                         __builtin_bit_cast(float, v[e] & 0xffff0000u) * g);
    p8[i] = o;
  }
}

__global__ void clear_status_kernel(Header* __restrict__ hdr, float* __restrict__ loss) {
  if (threadIdx.x == 0) {
    hdr->status = 0;
    hdr->count = 0;
    hdr->kblk[0] = hdr->kblk[1] = 0ull;
    if (loss) *loss = 0.f;
  }
}

// ------------------------------------------------------------ backward ----
struct BandArgs {
  int nb0, ns_cur;   // first token row of the band, rows in it
  int vb0, vs_cur;   // first vocabulary row of the band, rows in it
  int ldz;           // row stride of the dZ band (elements) == VS, a multiple of 64
  int frows, fcols;  // filter-flag grid of the band (64x64 blocks)
  int fstride;       // row stride of the flags: fcols rounded up to a multiple of 4
};

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Arguments of the dZ tiles of one band.
template <typename T>
struct DzArgs {
  const T* H;
  const T* W;
  const int64_t* y;
  const float* lse;
  const float* dloss_rows;
  const Header* hdr;
  int N, D, V;
  int64_t ignore;
  int reduction;
  float eps;
  BandArgs band;
  int TMv, TNn;          // vocabulary and token-row tiles of the band
  T* dz;                 // the band's dZ buffer [ns][ldz]
  uint8_t* flags;        // [frows][fstride]
  uint8_t* flagsT;       // [fcols][frows]
  const int* rowmap;     // row compaction: band rows are positions of rowmap (else rows)
  int keep_dropped;      // store dropped blocks' dZ too (filter on one product only)
  const int* vperm;      // sorted vocabulary: band position p is vocabulary row vperm[p]
  const int* vinv;       // and row v sits at position vinv[v] (null: natural order)
};

// dZ tile t of a band: Z = W_v H_n^T recomputed, G = softmax(Z) - onehot(y),
// dZ = g G (bf16 for bf16 inputs), plus the 64x64 filter flags.
// FILTER false: no block decision is needed (a block would be dropped only
// if all of it is zero, which changes no value), so the softmax goes out one
// 32-row block at a time and no flags are written.
template <typename T, bool FILTER = true>
__device__ __forceinline__ void dz_tile(const DzArgs<T>& a, int t, char* lds) {
  const T* __restrict__ H = a.H;
  const T* __restrict__ W = a.W;
  const int64_t* __restrict__ y = a.y;
  const float* __restrict__ lse = a.lse;
  const float* __restrict__ dloss_rows = a.dloss_rows;
  const int N = a.N, D = a.D, V = a.V, reduction = a.reduction;
  const int64_t ignore = a.ignore;
  const float eps = a.eps;
  const BandArgs& band = a.band;
  const int TMv = a.TMv, TNn = a.TNn;
  T* __restrict__ dz = a.dz;
  uint8_t* __restrict__ flags = a.flags;
  uint8_t* __restrict__ flagsT = a.flagsT;
  const int* __restrict__ rowmap = a.rowmap;
  int tm, tn;
  grouped_tile(t, TMv, TNn, 4, tm, tn);
  const int v0 = band.vb0 + tm * kTile, n0 = band.nb0 + tn * kTile;
  const int nval = rowmap ? a.hdr->nvalid : N;
  if (n0 >= nval) return;   // only ignored rows: the contractions do not read them
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // vocabulary positions are rows of W, or rows vperm[p] with a sorted vocabulary
  const Operand A{reinterpret_cast<const char*>(W), D, V, D, a.vperm};
  const Operand B{reinterpret_cast<const char*>(H), D, nval, D, rowmap};
  f32x16 acc[4][4];
  tile_contract<T, false, false>(A, B, v0, n0, D, AllActive{}, acc, lds);

  float g[4], ml[4];
  int rel[4];
  bool bad[4];
  const float gs = a.hdr->gscale;
  const int vw = v0 + wm * 128;  // first vocabulary row of this wave's block
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = n0 + wn * 128 + j * 32 + (lane & 31);
    const bool in = c < nval;
    const int n = in ? (rowmap ? rowmap[c] : c) : 0;
    const int64_t yy = in ? y[n] : ignore;
    const bool valid = in && yy != ignore;
    bad[j] = valid && (yy < 0 || yy >= V);
    const float gj = reduction == 2 ? (dloss_rows ? dloss_rows[in ? n : 0] : 1.f) : gs;
    g[j] = bad[j] ? __builtin_nanf("") : (valid ? gj : 0.f);
    ml[j] = valid ? lse[n] * kLog2e : INFINITY;       // rows outside the loss get p = 0
    rel[j] = (valid && !bad[j]) ? (a.vinv ? a.vinv[yy] : (int)yy) - vw : -1;   // target's position
  }
  const int fr0 = (n0 - band.nb0 + wn * 128) >> 6;   // flag row of this wave's first 64 rows
  const int fc0 = (v0 - band.vb0 + wm * 128) >> 6;   // flag column of its first 64 vocab rows
  // dZ = g (p - onehot).  bf16: into the LDS copy of the tile ([256 token
  // rows][512 B], 16-byte chunk c of row r at chunk c ^ (r % 32), so the 32
  // rows one instruction writes spread over all banks), stored to the band
  // below in whole rows.  fp32: straight to the band.  Column block j of the
  // wave (32 token rows), scale gg(i) for row block i.
  auto store_block = [&](int j, const float (&pj)[4][16], float gA, float gB) {
    const int r = wn * 128 + j * 32 + (lane & 31);   // tile row
    T* row = dz + (int64_t)(n0 - band.nb0 + r) * band.ldz + (vw - band.vb0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gg = i < 2 ? gA : gB;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = i * 32 + 8 * q + 4 * (lane >> 5);        // column within the wave's 128
        if constexpr (sizeof(T) == 2) {
          const int col = wm * 128 + c;                          // tile column
          *reinterpret_cast<u32x2*>(lds + r * 512 + (((col >> 3) ^ (r & 31)) * 16) +
                                    ((col >> 2) & 1) * 8) =
              u32x2{pack_bf16x2(gg * pj[i][4 * q + 0], gg * pj[i][4 * q + 1]),
                    pack_bf16x2(gg * pj[i][4 * q + 2], gg * pj[i][4 * q + 3])};
        } else {
          store4<T>(row + c, gg * pj[i][4 * q + 0], gg * pj[i][4 * q + 1],
                    gg * pj[i][4 * q + 2], gg * pj[i][4 * q + 3]);
        }
      }
    }
  };
  if constexpr (!FILTER) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float pj[4][16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) pj[i][r] = fast_exp2(fmaf(acc[i][j][r], kLog2e, -ml[j]));
      if (vw + 128 > V) {   // vocabulary rows past V (last tile)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vw + acc_row(i, r, lane) >= V) pj[i][r] = 0.f;
      }
      const int rl = rel[j];
      const bool hit = (unsigned)rl < 128u;
      if (__any(hit)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (hit && rl == acc_row(i, r, lane)) pj[i][r] -= 1.f;
      }
      store_block(j, pj, g[j], g[j]);
    }
  } else {
  // One pair of 32-column blocks (64 token rows) at a time, so at most 128
  // softmax values sit in VGPRs while the accumulators stay where they are.
#pragma unroll
  for (int bj = 0; bj < 2; ++bj) {
    float p[2][4][16];
    float kmax[2] = {0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[jj][i][r] = fast_exp2(fmaf(acc[i][2 * bj + jj][r], kLog2e, -ml[2 * bj + jj]));
          kmax[i >> 1] = fmaxf(kmax[i >> 1], p[jj][i][r]);
        }
    // rare: vocabulary rows past V (last tile) and targets (G = p - 1) change
    // the block maxima, which are then recomputed over |G|
    bool redo = false;
    if (vw + 128 > V) {
      redo = true;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (vw + acc_row(i, r, lane) >= V) p[0][i][r] = p[1][i][r] = 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int rl = rel[2 * bj + jj];
      const bool hit = (unsigned)rl < 128u;
      if (__any(hit)) {
        redo = true;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (hit && rl == acc_row(i, r, lane)) p[jj][i][r] -= 1.f;
      }
    }
    if (redo) {
      kmax[0] = kmax[1] = 0.f;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) kmax[i >> 1] = fmaxf(kmax[i >> 1], fabsf(p[jj][i][r]));
    }
    // CCE Alg. 4 filter on 64x64 blocks: dropped iff every |G| < eps (an
    // all-zero block is dropped too, which changes nothing).  Dropped blocks
    // are written as zeros and flagged so the contractions can skip them;
    // with keep_dropped (filter on one product only) their values are kept
    // and only the filtered product skips.
    float gk[2][2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const bool kp = __any((kmax[bi] > 0.f && kmax[bi] >= eps) || bad[2 * bj] || bad[2 * bj + 1]);
      gk[bi][0] = kp || a.keep_dropped ? g[2 * bj] : 0.f;
      gk[bi][1] = kp || a.keep_dropped ? g[2 * bj + 1] : 0.f;
      if (lane == 0) {
        const int fr = fr0 + bj, fc = fc0 + bi;
        if (fc < band.fcols) {
          flags[fr * band.fstride + fc] = kp ? 0 : 1;
          flagsT[fc * band.frows + fr] = kp ? 0 : 1;
        } else {
          // past the band (its last tile is partial): a padding column, never
          // the reason a K step runs
          flags[fr * band.fstride + fc] = 1;
        }
      }
    }
    store_block(2 * bj, p[0], gk[0][0], gk[1][0]);
    store_block(2 * bj + 1, p[1], gk[0][1], gk[1][1]);
  }
  }
  if constexpr (sizeof(T) == 2) {
    // The tile's 128 KiB of bf16 dZ from LDS to the band: wave w stores rows
    // 64 w .. 64 w + 63, two whole 512-byte rows per instruction.  The band's
    // row stride is a multiple of 64 columns, not necessarily of the tile:
    // 16-byte chunks past it belong to the next row and are not written
    // (their offset is out of range).  The stores are system-scope (sc0 sc1:
    // written through rather than held dirty in this XCD's L2); the band is
    // read in the next launch, after the launch boundary's cache write-back
    // anyway, and the fused step is ~0.5% faster (17.56 -> 17.47 ms, same-box
    // A/B at 8192 x 2048 x 151552).
    __syncthreads();
    const int half = lane >> 5, ch = lane & 31;
    T* base = dz + (int64_t)(n0 - band.nb0) * band.ldz + (v0 - band.vb0);
    const bool cin = (v0 - band.vb0) + ch * 8 < band.ldz;
    const auto rsz = make_rsrc(reinterpret_cast<const char*>(base));
    constexpr int kSc0Sc1 = 17;   // cache-policy bits of the buffer store: sc0 | sc1
#pragma unroll 8
    for (int s2 = 0; s2 < 32; ++s2) {
      const int r = 64 * wave + 2 * s2 + half;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * 512 + ((ch ^ (r & 31)) * 16));
      __builtin_amdgcn_raw_buffer_store_b128(
          v, rsz, cin ? (uint32_t)(((int64_t)r * band.ldz + ch * 8) * 2) : kOob, 0, kSc0Sc1);
    }
  }
}

// Active K steps of a contraction whose K runs over 64-wide filter blocks: a
// step is skipped when all four flags of its 64-block (one per 64 output
// rows of the tile) are set.  The flags are read once, before the K loop,
// into a 64-bit mask: scalar loads inside the loop would share the LDS wait
// counter with the fragment reads and stall them.  STEP is the K width of a
// step (64 or 32).
template <int STEP>
struct SkipRowsOfFlags {
  static_assert(STEP == 64 || STEP == 32, "step width");
  static constexpr int kShift = STEP == 64 ? 0 : 1;   // log2(steps per 64-block)
  static constexpr int kMaxBlocks = 128;              // K <= 8192
  const uint8_t* base;     // first of the four flags of 64-block 0
  int step_stride;         // bytes between consecutive 64-blocks
  int all = 0;             // every step active (the product is not filtered)
  uint64_t lo = 0, hi = 0; // bit b of (hi:lo): 64-block b is active
  unsigned long long* ctr = nullptr;   // optional: += active and total 64-blocks
  // Lane L of every wave reads the flags of 64-blocks L and 64 + L (indices
  // clamped to the last block, so every read is inside the tile's flags) and
  // two ballots give the masks: one round trip for the whole K range.
  __device__ __forceinline__ void prepare(int nsteps) {
    const int nb = min((nsteps + (1 << kShift) - 1) >> kShift, kMaxBlocks);
    const int lane = threadIdx.x & 63, last = nb > 0 ? nb - 1 : 0;
    const uint32_t f0 = *reinterpret_cast<const uint32_t*>(base + min(lane, last) * step_stride);
    const uint32_t f1 =
        *reinterpret_cast<const uint32_t*>(base + min(lane + 64, last) * step_stride);
    const uint64_t m0 = __ballot(lane < nb && f0 != 0x01010101u);
    const uint64_t m1 = __ballot(lane + 64 < nb && f1 != 0x01010101u);
    // (a select, not a branch: a branch here makes the compiler treat the
    // tile's operand descriptors as divergent)
    const uint64_t every = all ? ~0ull : 0ull;
    lo = m0 | every;
    hi = m1 | every;
    if (ctr != nullptr && !all && threadIdx.x == 0) {
      atomicAdd(ctr, (unsigned long long)(__popcll(m0) + __popcll(m1)));
      atomicAdd(ctr + 1, (unsigned long long)nb);
    }
  }
  __device__ __forceinline__ bool operator()(int s) const {
    const int b = s >> kShift;
    return ((b < 64 ? lo >> b : hi >> (b - 64)) & 1) != 0;
  }
  // first active step >= s (nsteps if none)
  __device__ __forceinline__ int next(int s, int nsteps) const {
    const int b = s >> kShift;
    int nb;
    if (b < 64 && (lo >> b) != 0) {
      nb = b + __builtin_ctzll(lo >> b);
    } else {
      const int c = b < 64 ? 0 : b - 64;
      if (c >= 64) return nsteps;
      const uint64_t rest = hi >> c;
      if (rest == 0) return nsteps;
      nb = 64 + c + __builtin_ctzll(rest);
    }
    const int ns = nb == b ? s : (nb << kShift);
    return ns < nsteps ? ns : nsteps;
  }
};


// dH[band rows] (+)= dZ W[band vocab] and dW[band vocab] (+)= dZ^T H[band rows]
// in one launch.  Both products are computed transposed, C[d][row], so that
// each lane's accumulator column holds 4 consecutive d values of one output
// row: the fp32 read-modify-write is one 16-byte access per 4 values.
//   dH^T tile: A = W_band^T (stored [v][d]), B = dZ (stored [n][v]), K = v
//   dW^T tile: A = H_band^T (stored [n][d]), B = dZ^T (stored [n][v]), K = n
// Arguments of the gradient tiles of one band.
template <typename T>
struct GradArgs {
  const T* H;
  const T* W;
  const T* dz;             // the band's dZ buffer
  const uint8_t* flags;
  const uint8_t* flagsT;
  float* dH;
  float* dW;
  int N, D, V;
  BandArgs band;
  int T3n, T2n, Td;        // token-row tiles, vocabulary tiles, d tiles of the band
  int beta_h, beta_w;      // accumulate into dH / dW (else overwrite)
  int skip_h, skip_w;      // FILTER: the product skips dropped K steps (else exact)
  const int* rowmap;       // row compaction (COMPACT): band rows are positions of rowmap
  const Header* hdr;       // nvalid with row compaction
  // bf16 gradients (BF16G): dH, dW are bf16; dH of the token band is summed in
  // `stage` [NS][D] floats.  h_mode: 0 stage = acc, 1 stage += acc,
  // 2 dH = bf16(stage + acc), 3 dH = bf16(acc); dW = bf16(acc) or, with beta_w,
  // bf16(dW + acc).
  uint16_t* dHb;
  uint16_t* dWb;
  float* stage;
  int h_mode;
  uint16_t* dWc;           // KAHAN: bf16 compensation of dWb, same layout
  const int* vperm;        // SORT: band vocabulary position p is row vperm[p] of W and dW
  unsigned long long* kblk;   // FILTER: Header::kblk (active, total K blocks), else null
};

// Epilogue of a gradient tile for bf16 inputs: out[r][d] = acc + src[r][d]
// (src optional) for the tile rows r < rvalid - row0 and d < D.  src rows are
// the tile's rows (SRC_MAPPED: map[r], like the out rows); out rows are the
// same or, with `map`, map[r].  The rows go through LDS half a tile (128
// rows) at a time: the waves holding the half write their accumulators
// row-major (16-byte chunk c of row r at chunk c ^ (r % 32), which spreads a
// column of chunks over all banks), then every wave adds and stores 32 whole
// rows, so one load or store instruction covers a whole row of the tile (1 KiB
// of floats, 512 B of bf16) instead of 16 or 32 bytes of 64 rows.  A wave
// handles its rows in four batches of 16 (two per half); the old values of a
// batch are loaded one batch ahead (those of the first batch before the
// accumulators are staged), so their latency overlaps the staging and the
// previous batch's adds and stores.  bf16 values are widened exactly and
// rounded to nearest even once.  Both contraction cores end with a barrier,
// so the staging slots are free here.
//
// KAHAN (bf16 source and destination only): the destination is a running
// bf16 sum s with a bf16 compensation c of the same layout at rsC (Kahan's
// compensated summation, CCE Sec. 5.1): with the tile's float partial p,
// y = p - c, t = s + y, s' = bf16(t), c' = bf16((s' - s) - y), all in float,
// so that s' - c' carries what the rounding of s' lost.  With src_on false
// (first contribution) s = c = 0.
template <bool SRC_BF16, bool DST_BF16, bool SRC_MAPPED = false, bool KAHAN = false>
__device__ __forceinline__ void grad_epilogue_rows(const f32x16 (&acc)[4][4], bool src_on,
                                                   __amdgpu_buffer_rsrc_t rsS,
                                                   __amdgpu_buffer_rsrc_t rsD, const int* map,
                                                   int row0, int rvalid, int D, int td,
                                                   char* lds, __amdgpu_buffer_rsrc_t rsC) {
  static_assert(!KAHAN || (SRC_BF16 && DST_BF16), "compensation of a bf16 running sum");
  constexpr int SES = SRC_BF16 ? 2 : 4, DES = DST_BF16 ? 2 : 4;
  constexpr int R = KAHAN ? 8 : 16;   // rows of one batch
  constexpr int NB = 64 / R;          // batches per wave (half a tile: 32 rows per wave)
  using Old = std::conditional_t<SRC_BF16, u32x2, f32x4>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int wm = wave >> 1, wn = wave & 1;
  const int dcol = td * kTile + lane * 4;   // this lane's 4 columns
  const bool dok = dcol < D;
  // The map entries of the wave's 64 rows, one per lane (lane L: row
  // (L / 32) 128 + 32 wave + L % 32), in one load; each row's entry is then
  // read from its lane, not loaded on its own.
  int mapv = 0;
  if (map) {
    const int r = (lane >> 5) * 128 + wave * 32 + (lane & 31);
    mapv = row0 + r < rvalid ? map[r] : 0;
  }
  auto widen = [](u32x2 b) {   // four bf16 (element d in the low half of a dword)
    return f32x4{__builtin_bit_cast(float, b[0] << 16), __builtin_bit_cast(float, b[0] & 0xffff0000u),
                 __builtin_bit_cast(float, b[1] << 16), __builtin_bit_cast(float, b[1] & 0xffff0000u)};
  };
  // batch n: tile rows (n / (NB / 2)) * 128 + wave * 32 + (n % (NB / 2)) * R + k
  auto issue = [&](int n, uint32_t (&od)[R], Old (&old)[R], u32x2 (&oc)[R]) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int h = n / (NB / 2), b = n % (NB / 2);
      const int trow = h * 128 + wave * 32 + b * R + k;   // row within the tile
      const bool rok = row0 + trow < rvalid, ok = rok && dok;
      const int64_t orow =
          map ? (rok ? (int64_t)__builtin_amdgcn_readlane(mapv, h * 32 + b * R + k) : 0)
              : trow;   // uniform per wave
      // without a source every load is out of range and reads zeros: the loads
      // are issued either way, so no branch sits between them and their uses
      // (a branch per load made the wait before the first add cover the next
      // batch's loads too)
      const uint32_t os = ok && src_on
                              ? (uint32_t)(((SRC_MAPPED ? orow : (int64_t)trow) * D + dcol) * SES)
                              : kOob;
      od[k] = ok ? (uint32_t)((orow * D + dcol) * DES) : kOob;
      if constexpr (SRC_BF16)
        old[k] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsS, os, 0, 0));
      else
        old[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsS, os, 0, 0));
      if constexpr (KAHAN)   // the compensation has the destination's layout
        oc[k] = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsC, src_on ? od[k] : kOob, 0, 0));
    }
  };
  auto finish = [&](int n, const uint32_t (&od)[R], const Old (&old)[R], const u32x2 (&oc)[R]) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int rl = wave * 32 + (n % (NB / 2)) * R + k;   // row within the half
      const f32x4 p = *reinterpret_cast<const f32x4*>(lds + rl * 1024 + ((lane ^ (rl & 31)) * 16));
      if constexpr (KAHAN) {
        const f32x4 s = widen(old[k]), c = widen(oc[k]);
        u32x2 sb, cb;
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const float y0 = p[e] - c[e], y1 = p[e + 1] - c[e + 1];
          const uint32_t t = pack_bf16x2(s[e] + y0, s[e + 1] + y1);
          const float t0 = __builtin_bit_cast(float, t << 16);
          const float t1 = __builtin_bit_cast(float, t & 0xffff0000u);
          sb[e >> 1] = t;
          cb[e >> 1] = pack_bf16x2((t0 - s[e]) - y0, (t1 - s[e + 1]) - y1);
        }
        __builtin_amdgcn_raw_buffer_store_b64(sb, rsD, od[k], 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(cb, rsC, od[k], 0, 0);
        continue;
      }
      f32x4 o;
      if constexpr (SRC_BF16)
        o = widen(old[k]);
      else
        o = old[k];
      const f32x4 v = p + o;
      if constexpr (DST_BF16)
        __builtin_amdgcn_raw_buffer_store_b64(
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}, rsD, od[k], 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsD, od[k], 0, 0);
    }
  };
  auto stage = [&](int half) {
    if (wn == half) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 32 * j + (lane & 31);
            const int c = wm * 32 + 8 * i + 2 * q + (lane >> 5);
            *reinterpret_cast<f32x4*>(lds + r * 1024 + ((c ^ (r & 31)) * 16)) =
                f32x4{acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
          }
    }
    __syncthreads();
  };
  uint32_t odA[R], odB[R];
  Old oldA[R], oldB[R];
  u32x2 ocA[R], ocB[R];   // compensation (KAHAN only; unused otherwise)
  // batches 0 .. NB-1 with two in flight: the old values of batch n + 1 load
  // while batch n is added and stored.  The first half's rows are staged
  // after batch 0's loads are issued, the second half's once every wave has
  // finished the first half (their loads already out).
  issue(0, odA, oldA, ocA);
  stage(0);
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    if (n + 1 < NB) {
      if (n & 1) issue(n + 1, odA, oldA, ocA);
      else issue(n + 1, odB, oldB, ocB);
    }
    if (n & 1) finish(n, odB, oldB, ocB);
    else finish(n, odA, oldA, ocA);
    if (n + 1 == NB / 2) {
      __syncthreads();
      stage(1);
    }
  }
  __syncthreads();
}

// Gradient tile `local` of one of the band's two contractions (is_h: dH^T).
// COMPACT: the band's rows are positions of a.rowmap; only the first
// nvalid - nb0 of them are rows (the rest are ignored rows, whose dZ rows are
// not made): dH^T tiles past them exit, their rows are scattered through the
// map, and dW^T contracts over them only, gathering H's rows through an LDS
// copy of the map.
// SORT: the band's vocabulary positions are rows vperm[p]: dH^T gathers W's
// k rows through an LDS copy of the band's part of vperm, dW^T rows are
// scattered through it.
template <typename T, bool FILTER, bool COMPACT = false, bool BF16G = false, bool SORT = false,
          bool KAHAN = false>
__device__ __forceinline__ void grad_tile(const GradArgs<T>& a, bool is_h, int local, char* lds) {
  static_assert(!KAHAN || BF16G, "the compensation is of bf16 gradients");
  const T* __restrict__ H = a.H;
  const T* __restrict__ W = a.W;
  const T* __restrict__ dz = a.dz;
  const uint8_t* __restrict__ flags = a.flags;
  const uint8_t* __restrict__ flagsT = a.flagsT;
  float* __restrict__ dH = a.dH;
  float* __restrict__ dW = a.dW;
  const int D = a.D;
  const BandArgs& band = a.band;
  const int T3n = a.T3n, T2n = a.T2n, Td = a.Td, beta_h = a.beta_h, beta_w = a.beta_w;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[4][4];
  float* out;
  int rvalid, beta, td, tr;
  // rows of the band that are rows (all of them without compaction)
  const int nrows = COMPACT ? min(band.ns_cur, a.hdr->nvalid - band.nb0) : band.ns_cur;
  if (is_h) {
    grouped_tile(local, Td, T3n, 4, td, tr);   // d tile, band row tile
    if (COMPACT && tr * kTile >= nrows) return;   // ignored rows only: zeroed separately
    out = dH + (int64_t)band.nb0 * D;
    rvalid = COMPACT ? nrows : band.ns_cur;
    beta = beta_h;
    // K read up to the tile multiple (zeros past V in the last band), but
    // never past the band's row stride
    const int kpad = min((band.vs_cur + kTile - 1) / kTile * kTile, band.ldz);
    const Operand B{reinterpret_cast<const char*>(dz), band.ldz, (int64_t)T3n * kTile, kpad};
    if constexpr (SORT) {
      static_assert(FILTER, "the vocabulary order only serves the filter");
      char* table = lds + kDmaLdsBytes + 256;
      const int half = band.fcols * kFilterHalfPerBlock;   // VS / 2 entries per parity
      gather_table(table, a.vperm + band.vb0, band.vs_cur, half);
      const Operand A{reinterpret_cast<const char*>(W), D, D, band.vs_cur,
                      reinterpret_cast<const int*>(table), half};
      const SkipRowsOfFlags<step_k<T>()> act{flagsT + tr * 4, band.frows, !a.skip_h, 0, 0, a.kblk};
      tile_contract<T, true, false, SkipRowsOfFlags<step_k<T>()>, true>(
          A, B, td * kTile, tr * kTile, band.vs_cur, act, acc, lds);
    } else if constexpr (FILTER) {
      const Operand A{reinterpret_cast<const char*>(W + (int64_t)band.vb0 * D), D, D, band.vs_cur};
      const SkipRowsOfFlags<step_k<T>()> act{flagsT + tr * 4, band.frows, !a.skip_h, 0, 0, a.kblk};
      tile_contract<T, true, false>(A, B, td * kTile, tr * kTile, band.vs_cur, act, acc, lds);
    } else {
      const Operand A{reinterpret_cast<const char*>(W + (int64_t)band.vb0 * D), D, D, band.vs_cur};
      tile_contract<T, true, false>(A, B, td * kTile, tr * kTile, band.vs_cur, AllActive{}, acc,
                                    lds);
    }
  } else {
    grouped_tile(local, Td, T2n, 4, td, tr);   // d tile, band vocabulary tile
    out = dW + (int64_t)band.vb0 * D;
    rvalid = band.vs_cur;
    beta = beta_w;
    const int K = nrows > 0 ? nrows : 0;
    if constexpr (COMPACT) {
      char* table = lds + kDmaLdsBytes + 256;
      const int half = band.frows * kFilterHalfPerBlock;   // NS / 2 entries per parity
      gather_table(table, a.rowmap + band.nb0, K, half);
      const Operand A{reinterpret_cast<const char*>(H), D, D, K,
                      reinterpret_cast<const int*>(table), half};
      const Operand B{reinterpret_cast<const char*>(dz), band.ldz,
                      min((int64_t)T2n * kTile, (int64_t)band.ldz), K};
      if constexpr (FILTER) {
        const SkipRowsOfFlags<step_k<T>()> act{flags + tr * 4, band.fstride, !a.skip_w, 0, 0, a.kblk};
        tile_contract<T, true, true, SkipRowsOfFlags<step_k<T>()>, true>(A, B, td * kTile,
                                                                        tr * kTile, K, act, acc,
                                                                        lds);
      } else {
        tile_contract<T, true, true, AllActive, true>(A, B, td * kTile, tr * kTile, K, AllActive{},
                                                      acc, lds);
      }
    } else {
      const Operand A{reinterpret_cast<const char*>(H + (int64_t)band.nb0 * D), D, D, band.ns_cur};
      const Operand B{reinterpret_cast<const char*>(dz), band.ldz,
                      min((int64_t)T2n * kTile, (int64_t)band.ldz), band.ns_cur};
      if constexpr (FILTER) {
        const SkipRowsOfFlags<step_k<T>()> act{flags + tr * 4, band.fstride, !a.skip_w, 0, 0, a.kblk};
        tile_contract<T, true, true>(A, B, td * kTile, tr * kTile, band.ns_cur, act, acc, lds);
      } else {
        tile_contract<T, true, true>(A, B, td * kTile, tr * kTile, band.ns_cur, AllActive{}, acc,
                                     lds);
      }
    }
  }
  // acc[i][j][4q + e]: d = dw + 32 i + 8 q + 4 (lane / 32) + e, row = rw + 32 j + lane % 32.
  // Buffer accesses relative to the tile's first output row: an offset past
  // the output (row >= rvalid or d >= D) reads zeros and drops the store, so
  // the 16 loads of a row group go out together, with no branches between
  // them.
  const int row0 = tr * kTile;
  const int dw = td * kTile + wm * 128 + 4 * (lane >> 5);
  const int lw = wn * 128 + (lane & 31);
  if constexpr (BF16G) {
    if (is_h) {
      const int hm = a.h_mode;
      const auto rsS = make_rsrc(reinterpret_cast<const char*>(a.stage + (int64_t)row0 * D));
      if (hm <= 1) {
        grad_epilogue_rows<false, false>(acc, hm == 1, rsS, rsS, nullptr, row0, rvalid, D, td,
                                         lds, rsS);
      } else {
        // scattered rows: offsets from the start of dH (N D 4 < 2^31 with compaction)
        const auto rsD = make_rsrc(reinterpret_cast<const char*>(
            COMPACT ? a.dHb : a.dHb + ((int64_t)band.nb0 + row0) * D));
        grad_epilogue_rows<false, true>(acc, hm == 2, rsS, rsD,
                                        COMPACT ? a.rowmap + band.nb0 + row0 : nullptr, row0,
                                        rvalid, D, td, lds, rsD);
      }
    } else {
      if constexpr (SORT) {   // rows scattered: offsets from the start of dW (V D 4 < 2^31)
        const auto rs = make_rsrc(reinterpret_cast<const char*>(a.dWb));
        const auto rc = make_rsrc(reinterpret_cast<const char*>(KAHAN ? a.dWc : a.dWb));
        grad_epilogue_rows<true, true, true, KAHAN>(acc, beta_w != 0, rs, rs,
                                                    a.vperm + band.vb0 + row0, row0, rvalid, D,
                                                    td, lds, rc);
      } else {
        const int64_t o = ((int64_t)band.vb0 + row0) * D;
        const auto rs = make_rsrc(reinterpret_cast<const char*>(a.dWb + o));
        const auto rc = make_rsrc(reinterpret_cast<const char*>((KAHAN ? a.dWc : a.dWb) + o));
        grad_epilogue_rows<true, true, false, KAHAN>(acc, beta_w != 0, rs, rs, nullptr, row0,
                                                     rvalid, D, td, lds, rc);
      }
    }
    return;
  }
  // with compaction the dH^T tile's rows are scattered through the row map,
  // with a sorted vocabulary the dW^T tile's rows through vperm: offsets from
  // the start of dH / dW (below 2^31 by the planner's checks)
  const int* smap = is_h ? (COMPACT ? a.rowmap + band.nb0 + row0 : nullptr)
                         : (SORT ? a.vperm + band.vb0 + row0 : nullptr);
  const bool scatter = (COMPACT && is_h) || (SORT && !is_h);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const char*>(
      scatter ? (is_h ? dH : dW) : out + (int64_t)row0 * D));
  if constexpr (std::is_same_v<T, float>) {
    // Float inputs keep their accumulators in VGPRs, where staging through
    // LDS spills: the epilogue goes straight from the accumulators, two row
    // groups in flight (the loads of group j + 1 and j + 2 are out while
    // group j is added and stored).
    auto offsets = [&](int j, uint32_t (&off)[4][4]) {
      const int lr = lw + 32 * j;
      const bool rok = row0 + lr < rvalid;
      const int64_t orow = scatter ? (rok ? (int64_t)smap[lr] : 0) : lr;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int d = dw + 32 * i + 8 * q;
          off[i][q] = rok && d < D ? (uint32_t)((orow * D + d) * 4) : kOob;
        }
    };
    auto load = [&](const uint32_t (&off)[4][4], f32x4 (&old)[4][4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          old[i][q] = __builtin_bit_cast(   // out of range (zeros) without beta
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, beta ? off[i][q] : kOob, 0, 0));
    };
    auto store = [&](int j, const uint32_t (&off)[4][4], const f32x4 (&old)[4][4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = f32x4{acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                acc[i][j][4 * q + 3]} + old[i][q];
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off[i][q], 0,
                                                 0);
        }
    };
    uint32_t offA[4][4], offB[4][4];
    f32x4 oldA[4][4], oldB[4][4];
    offsets(0, offA);
    load(offA, oldA);
    offsets(1, offB);
    load(offB, oldB);
    store(0, offA, oldA);
    offsets(2, offA);
    load(offA, oldA);
    store(1, offB, oldB);
    offsets(3, offB);
    load(offB, oldB);
    store(2, offA, oldA);
    store(3, offB, oldB);
    return;
  }
  // bf16 inputs: whole rows through LDS (old values at the out rows)
  grad_epilogue_rows<false, false, true>(acc, beta != 0, rs, rs, smap, row0, rvalid, D, td, lds,
                                         rs);
}

// Epilogue of a 128 (d) x 256 (rows) gradient tile, float output:
// out[r][d] = acc + out[r][d] (the old value only with src_on) for the tile
// rows r < rvalid - row0 and d < D.  The whole tile goes through LDS as
// [256 rows][512 B] (16-byte chunk c of row r at c ^ (r % 32)); then wave w
// adds and stores rows 64 w .. 64 w + 63, a pair of whole rows per
// instruction (lanes 0-31 the first, 32-63 the second), in four batches of
// 16 rows whose old values load one batch ahead (the first batch's before
// the accumulators are staged).
__device__ __forceinline__ void grad_epilogue_narrow(const f32x16 (&acc)[2][4], bool src_on,
                                                     __amdgpu_buffer_rsrc_t rs, int row0,
                                                     int rvalid, int D, int td, char* lds) {
  constexpr int R = 8;    // row pairs of one batch
  constexpr int NB = 4;   // batches per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int ch = lane & 31, hr = lane >> 5;   // chunk of the row, row of the pair
  const int dcol = td * 128 + ch * 4;
  const bool dok = dcol < D;
  auto issue = [&](int n, uint32_t (&od)[R], f32x4 (&old)[R]) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int r = 64 * wave + 2 * (n * R + k) + hr;
      od[k] = row0 + r < rvalid && dok ? (uint32_t)(((int64_t)r * D + dcol) * 4) : kOob;
      // branch-free: without a source the load is out of range and reads zeros
      old[k] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, src_on ? od[k] : kOob, 0, 0));
    }
  };
  auto finish = [&](int n, const uint32_t (&od)[R], const f32x4 (&old)[R]) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int r = 64 * wave + 2 * (n * R + k) + hr;
      const f32x4 p = *reinterpret_cast<const f32x4*>(lds + r * 512 + ((ch ^ (r & 31)) * 16));
      const f32x4 v = p + old[k];
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, od[k], 0, 0);
    }
  };
  uint32_t odA[R], odB[R];
  f32x4 oldA[R], oldB[R];
  issue(0, odA, oldA);
  // acc[i][j][4q + e]: d = 64 wm + 32 i + 8 q + 4 (lane / 32) + e, row 128 wn + 32 j + lane % 32
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wn * 128 + 32 * j + (lane & 31);
        const int c = wm * 16 + 8 * i + 2 * q + (lane >> 5);
        *reinterpret_cast<f32x4*>(lds + r * 512 + ((c ^ (r & 31)) * 16)) =
            f32x4{acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                  acc[i][j][4 * q + 3]};
      }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    if (n + 1 < NB) {
      if (n & 1) issue(n + 1, odA, oldA);
      else issue(n + 1, odB, oldB);
    }
    if (n & 1) finish(n, odB, oldB);
    else finish(n, odA, oldA);
  }
  __syncthreads();
}

// Gradient tile `local` of a band's contraction (is_h: dH^T) as a 128 (d) x
// 256 (rows) tile, bf16 inputs, float gradients, no compaction or vocabulary
// order: the same products and K order as grad_tile, with d tiles of 128
// (a.Td of them), for a launch that only contracts and would leave half the
// CUs idle with 256-wide tiles.  FILTER: K steps skipped as in grad_tile.
template <bool FILTER>
__device__ __forceinline__ void grad_tile_narrow(const GradArgs<uint16_t>& a, bool is_h, int local,
                                                 char* lds) {
  const int D = a.D;
  const BandArgs& band = a.band;
  const int T3n = a.T3n, T2n = a.T2n, Td = a.Td;
  f32x16 acc[2][4];
  float* out;
  int rvalid, beta, td, tr;
  // The filter's K-block counters count per 256-wide d range, as the wide
  // tiles do: only the first of each pair of narrow tiles adds to them.
  auto counters = [&](int t) { return (t & 1) ? nullptr : a.kblk; };
  if (is_h) {
    grouped_tile(local, Td, T3n, 4, td, tr);   // d tile, band row tile
    unsigned long long* kblk = counters(td);
    out = a.dH + (int64_t)band.nb0 * D;
    rvalid = band.ns_cur;
    beta = a.beta_h;
    const int kpad = min((band.vs_cur + kTile - 1) / kTile * kTile, band.ldz);
    const Operand A{reinterpret_cast<const char*>(a.W + (int64_t)band.vb0 * D), D, D, band.vs_cur};
    const Operand B{reinterpret_cast<const char*>(a.dz), band.ldz, (int64_t)T3n * kTile, kpad};
    const int nsteps = (band.vs_cur + kDmaKStep - 1) / kDmaKStep;
    if constexpr (FILTER) {
      const SkipRowsOfFlags<kDmaKStep> act{a.flagsT + tr * 4, band.frows, !a.skip_h, 0, 0, kblk};
      gemm_tile_dma2n<false>(A, B, td * 128, tr * kTile, nsteps, act, acc, lds,
                             L2Split{tr & 7, 8}, L2Split{td & 3, 4});
    } else {
      gemm_tile_dma2n<false>(A, B, td * 128, tr * kTile, nsteps, AllActive{}, acc, lds,
                             L2Split{tr & 7, 8}, L2Split{td & 3, 4});
    }
  } else {
    grouped_tile(local, Td, T2n, 4, td, tr);   // d tile, band vocabulary tile
    unsigned long long* kblk = counters(td);
    out = a.dW + (int64_t)band.vb0 * D;
    rvalid = band.vs_cur;
    beta = a.beta_w;
    const Operand A{reinterpret_cast<const char*>(a.H + (int64_t)band.nb0 * D), D, D, band.ns_cur};
    const Operand B{reinterpret_cast<const char*>(a.dz), band.ldz,
                    min((int64_t)T2n * kTile, (int64_t)band.ldz), band.ns_cur};
    const int nsteps = (band.ns_cur + kDmaKStep - 1) / kDmaKStep;
    if constexpr (FILTER) {
      const SkipRowsOfFlags<kDmaKStep> act{a.flags + tr * 4, band.fstride, !a.skip_w, 0, 0, kblk};
      gemm_tile_dma2n<true>(A, B, td * 128, tr * kTile, nsteps, act, acc, lds,
                            L2Split{tr & 7, 8}, L2Split{td & 3, 4});
    } else {
      gemm_tile_dma2n<true>(A, B, td * 128, tr * kTile, nsteps, AllActive{}, acc, lds,
                            L2Split{tr & 7, 8}, L2Split{td & 3, 4});
    }
  }
  const int row0 = tr * kTile;
  grad_epilogue_narrow(acc, beta != 0,
                       make_rsrc(reinterpret_cast<const char*>(out + (int64_t)row0 * D)), row0,
                       rvalid, D, td, lds);
}

// One launch of the backward pipeline: the gradient tiles of band k - 1
// (reading dZ buffer (k - 1) % 2) together with the dZ tiles of band k
// (writing buffer k % 2), so that the tiles' memory-heavy epilogues do not
// all fall at the same moment and no launch boundary sits between the two.
// Tile kinds, longest first on every XCD: [0, g_long) gradient tiles of the
// contraction with the longer K, [g_long, g_grad) the other gradient tiles,
// [g_grad, G) dZ tiles.
constexpr int kBandLdsCompact = kDmaLdsBytes + 256 + kGatherTableBytes;   // slots, line touch, map

template <typename T, bool FILTER, bool COMPACT, bool BF16G = false, bool SORT = false,
          bool KAHAN = false, bool NARROW = false>
__global__ void __launch_bounds__(kThreads, 1)
bwd_band_kernel(GradArgs<T> ga, DzArgs<T> da, int g_long, int g_grad, int h_first) {
  __shared__ __attribute__((aligned(1024))) char
      lds[(COMPACT || SORT) && kBandLdsCompact > kLdsBytes ? kBandLdsCompact : kLdsBytes];
  const int t = xcd_remap_kinds(blockIdx.x, gridDim.x, g_long, g_grad);
  if (t >= g_grad) {
    dz_tile<T, FILTER>(da, t - g_grad, lds);
    return;
  }
  const int T3 = ga.Td * ga.T3n;   // dH^T tiles
  const bool is_h = h_first ? t < T3 : t >= g_long;
  const int local = h_first ? (is_h ? t : t - T3) : (is_h ? t - g_long : t);
  if constexpr (NARROW) {
    static_assert(sizeof(T) == 2 && !COMPACT && !BF16G && !SORT, "128-wide gradient tiles");
    grad_tile_narrow<FILTER>(ga, is_h, local, lds);
  } else {
    grad_tile<T, FILTER, COMPACT, BF16G, SORT, KAHAN>(ga, is_h, local, lds);
  }
}

}  // namespace flce
