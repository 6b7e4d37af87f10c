// vocab_sort.hpp -- the vocabulary ordered by average logit, for the blocks
// of the gradient filter (Cut Cross-Entropy, arXiv 2411.09009, Sec. 4.3,
// "Vocabulary sorting": blocks of entries with similar average logit keep the
// entries with non-trivial gradients together).
//
// The key of vocabulary entry v is the sum of its logits over the
// non-ignored rows, which orders the entries as their average does:
//     key_v = sum_n Z[n, v] = W_v . (sum_n H_n)
// so it is a column sum of H (colsum_*) and one matrix-vector product with W
// (vocab_key_kernel) instead of a reduction in every forward tile.  A stable
// LSD radix sort (four 8-bit passes of histogram / scan / scatter) orders the
// indices by decreasing key, ties by increasing index.  Every sum has a fixed
// order: the result is deterministic.
#pragma once

#include "tile_mma.hpp"

namespace flce {

constexpr int kColSplits = 64;        // row splits of the column sum
constexpr int kSortItems = 8;         // elements per thread of a sort block
constexpr int kSortTile = 256 * kSortItems;

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) {
  return __builtin_bit_cast(float, x & 0xffff0000u);
}

// part[s][d] = sum over rows n of split s whose target is not `ignore` of
// H[n][d] (float, increasing n).  grid (ceil(D / 256), kColSplits).
__global__ void __launch_bounds__(256)
colsum_partial_kernel(const uint16_t* __restrict__ H, const int64_t* __restrict__ y, int N, int D,
                      int64_t ignore, float* __restrict__ part) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  const int per = (N + kColSplits - 1) / kColSplits;
  const int n0 = blockIdx.y * per, n1 = min(N, n0 + per);
  if (d >= D) return;
  float acc = 0.f;
  for (int n = n0; n < n1; ++n)
    if (y[n] != ignore) acc += __builtin_bit_cast(float, (uint32_t)H[(int64_t)n * D + d] << 16);
  part[(int64_t)blockIdx.y * D + d] = acc;
}

// hbar[d] = sum_s part[s][d] (increasing s).  grid ceil(D / 256).
__global__ void __launch_bounds__(256)
colsum_final_kernel(const float* __restrict__ part, int D, float* __restrict__ hbar) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  float acc = 0.f;
  for (int s = 0; s < kColSplits; ++s) acc += part[(int64_t)s * D + d];
  hbar[d] = acc;
}

// keys[v] = the key of W_v . hbar for an ascending sort that puts large
// values first (float order reversed; -0 taken as +0).  One wave per
// vocabulary row (4 per block): lane L takes d = 8 L + 512 i, then a fixed
// xor-butterfly sums the lanes.  D % 8 == 0, W and hbar 16-byte aligned.
__global__ void __launch_bounds__(256)
vocab_key_kernel(const uint16_t* __restrict__ W, const float* __restrict__ hbar, int V, int D,
                 uint32_t* __restrict__ keys) {
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (v >= V) return;
  const uint16_t* w = W + (int64_t)v * D;
  float acc = 0.f;
  for (int d = lane * 8; d < D; d += 512) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(w + d);
    const f32x4 h0 = *reinterpret_cast<const f32x4*>(hbar + d);
    const f32x4 h1 = *reinterpret_cast<const f32x4*>(hbar + d + 4);
    acc = fmaf(bf16_lo(q[0]), h0[0], acc);
    acc = fmaf(bf16_hi(q[0]), h0[1], acc);
    acc = fmaf(bf16_lo(q[1]), h0[2], acc);
    acc = fmaf(bf16_hi(q[1]), h0[3], acc);
    acc = fmaf(bf16_lo(q[2]), h1[0], acc);
    acc = fmaf(bf16_hi(q[2]), h1[1], acc);
    acc = fmaf(bf16_lo(q[3]), h1[2], acc);
    acc = fmaf(bf16_hi(q[3]), h1[3], acc);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) {
    const uint32_t u = __builtin_bit_cast(uint32_t, acc == 0.f ? 0.f : acc);
    const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // float order as uint
    keys[v] = ~asc;                                                        // large first
  }
}

// Radix pass, step 1: hist[d * nblk + b] = number of keys of block b (kSortTile
// keys from b * kSortTile) whose digit (key >> shift) & 255 is d.
__global__ void __launch_bounds__(256)
sort_hist_kernel(const uint32_t* __restrict__ keys, int V, int shift, int nblk,
                 uint32_t* __restrict__ hist) {
  __shared__ uint32_t cnt[256];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int e0 = blockIdx.x * kSortTile;
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const int e = e0 + i * 256 + threadIdx.x;
    if (e < V) atomicAdd(&cnt[(keys[e] >> shift) & 255u], 1u);
  }
  __syncthreads();
  hist[threadIdx.x * nblk + blockIdx.x] = cnt[threadIdx.x];
}

// Step 2: exclusive prefix sum of hist[0 .. n) in place (digit-major order:
// the output position of each block's first key of each digit).  One block
// of 1024 threads, each summing a contiguous chunk.
__global__ void __launch_bounds__(1024)
sort_scan_kernel(uint32_t* __restrict__ hist, int n) {
  __shared__ uint32_t part[1024];
  const int t = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int a = min(n, t * per), b = min(n, a + per);
  uint32_t s = 0;
  for (int i = a; i < b; ++i) s += hist[i];
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive scan of the chunk sums
    const uint32_t x = t >= o ? part[t - o] : 0u;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
  uint32_t run = part[t] - s;
  for (int i = a; i < b; ++i) {
    const uint32_t h = hist[i];
    hist[i] = run;
    run += h;
  }
}

// Step 3: stable scatter.  Block b walks its keys in index order, 256 at a
// time; a key goes to offs[digit] of its block plus the keys of the same
// digit before it (earlier rounds, earlier waves, lower lanes).  idx_in ==
// nullptr means the identity (first pass).
__global__ void __launch_bounds__(256)
sort_scatter_kernel(const uint32_t* __restrict__ keys_in, const int* __restrict__ idx_in, int V,
                    int shift, int nblk, const uint32_t* __restrict__ offs,
                    uint32_t* __restrict__ keys_out, int* __restrict__ idx_out) {
  __shared__ uint32_t run[256];
  __shared__ uint32_t wc[4][256];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  run[t] = offs[t * nblk + blockIdx.x];
#pragma unroll
  for (int w = 0; w < 4; ++w) wc[w][t] = 0;
  __syncthreads();
  const int e0 = blockIdx.x * kSortTile;
  for (int i = 0; i < kSortItems; ++i) {
    const int e = e0 + i * 256 + t;
    const bool ok = e < V;
    const uint32_t key = ok ? keys_in[e] : 0u;
    const int idx = ok ? (idx_in ? idx_in[e] : e) : 0;
    const uint32_t dig = (key >> shift) & 255u;
    // lanes of this wave holding the same digit
    uint64_t m = __ballot(ok);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (dig >> bit) & 1u;
      const uint64_t bb = __ballot(ok && on);
      m &= on ? bb : ~bb;
    }
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    if (ok && rank == 0) wc[wave][dig] = (uint32_t)__popcll(m);
    __syncthreads();
    if (ok) {
      uint32_t pos = run[dig] + rank;
      for (int w = 0; w < wave; ++w) pos += wc[w][dig];
      keys_out[pos] = key;
      idx_out[pos] = idx;
    }
    __syncthreads();
    run[t] += wc[0][t] + wc[1][t] + wc[2][t] + wc[3][t];
#pragma unroll
    for (int w = 0; w < 4; ++w) wc[w][t] = 0;
    __syncthreads();
  }
}

// inv[perm[i]] = i
__global__ void __launch_bounds__(256)
invert_perm_kernel(const int* __restrict__ perm, int V, int* __restrict__ inv) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < V) inv[perm[i]] = i;
}

}  // namespace flce
