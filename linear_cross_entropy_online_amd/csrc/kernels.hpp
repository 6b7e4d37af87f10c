// kernels.hpp -- device kernels of the fused LM-head + cross-entropy path.
//
//   fwd_lse_kernel      Z tile = W_v H_n^T on MFMA; online max / sum-exp per
//                       token row over this workgroup's vocabulary range; the
//                       target logit is picked from the same accumulators.
//                       (CCE, arXiv 2411.09009, Sec. 4.2 / Alg. 2 for the
//                       blockwise log-sum-exp, Sec. 4.1 / Alg. 1 for the
//                       indexed logit; online normaliser of Sec. 2.)
//   lse_combine_kernel  merges the per-split (max, sum) partials of a row in a
//                       fixed order into LSE and the row loss (replaces the
//                       paper's spin-locked log-add-exp), plus per-block sums.
//   finalize_kernel     fixed-order scalar loss, valid-row count, row scale.
//   bwd_prep_kernel     the same count / scale for a standalone backward.
//   bwd_dz_kernel       recomputes a logits tile and writes
//                       dZ = g_n (softmax - onehot) for one band into the
//                       workspace, with 64x64 filter flags (CCE Alg. 4, first
//                       half; gradient filtering of Sec. 4.3).
//   bwd_grad_kernel     one launch holding both band contractions:
//                       dH[band rows] (+)= dZ W[band vocab] and
//                       dW[band vocab] (+)= dZ^T H[band rows] (Alg. 4, second
//                       half, done as two ordinary MFMA GEMMs without locks).
#pragma once

#include "tile_mma.hpp"

namespace flce {

struct Header {           // first 256 bytes of the workspace
  int status;             // bit 0: target outside [0, V) and != ignore_index
  int count;              // non-ignored rows
  float gscale;           // g for mean / sum: dloss / max(count, 1) or dloss
  float pad[61];
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ------------------------------------------------------------- forward ----
template <typename T>
__global__ void __launch_bounds__(kThreads, 1)
fwd_lse_kernel(const T* __restrict__ H, const T* __restrict__ W, const int64_t* __restrict__ y,
               int N, int D, int V, int64_t ignore, int Sv, int Tv, float* __restrict__ part_m,
               float* __restrict__ part_s, float* __restrict__ zy, Header* __restrict__ hdr) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int nt = t / Sv, split = t - nt * Sv;
  const int n0 = nt * kTile;
  const int vt0 = (int)((int64_t)split * Tv / Sv);
  const int vt1 = (int)((int64_t)(split + 1) * Tv / Sv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if (blockIdx.x == 0 && tid == 0) hdr->status = 0;

  int ytg[4];
  float mrun[4], srun[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 128 + j * 32 + (lane & 31);
    const int64_t yy = n < N ? y[n] : ignore;
    ytg[j] = (yy >= 0 && yy < V) ? (int)yy : -1;
    mrun[j] = -INFINITY;
    srun[j] = 0.f;
  }
  const Operand A{reinterpret_cast<const char*>(W), D, V, D};
  const Operand B{reinterpret_cast<const char*>(H), D, N, D};
  const int nk = (D + kKStep<T> - 1) / kKStep<T>;
  f32x16 acc[4][4];

  for (int vt = vt0; vt < vt1; ++vt) {
    const int v0 = vt * kTile;
    gemm_tile<T, false, false>(A, B, v0, n0, nk, AllActive{}, acc, lds);
    const int vw = v0 + wm * 128;  // first vocabulary row of this wave's block
    if (vw + 128 > V) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (vw + acc_row(i, r, lane) >= V)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j][r] = -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, acc[i][j][r]);
      const float mnew = fmaxf(mrun[j], tmax);
      if (mnew != -INFINITY) {
        const float ml = mnew * kLog2e;
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) s4[i] += fast_exp2(fmaf(acc[i][j][r], kLog2e, -ml));
        srun[j] = srun[j] * fast_exp2((mrun[j] - mnew) * kLog2e) + ((s4[0] + s4[1]) + (s4[2] + s4[3]));
        mrun[j] = mnew;
      }
      const int rel = ytg[j] - vw;
      const bool hit = (unsigned)rel < 128u;
      if (__any(hit)) {
        float z = 0.f;
        bool own = false;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (rel == acc_row(i, r, lane)) {
              z = acc[i][j][r];
              own = true;
            }
        if (hit && own) zy[n0 + wn * 128 + j * 32 + (lane & 31)] = z;
      }
    }
  }

  // merge the two lanes holding one token column, then the two waves
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float mo = __shfl_xor(mrun[j], 32), so = __shfl_xor(srun[j], 32);
    const float M = fmaxf(mrun[j], mo);
    srun[j] = (M == -INFINITY) ? 0.f
                               : srun[j] * fast_exp2((mrun[j] - M) * kLog2e) +
                                     so * fast_exp2((mo - M) * kLog2e);
    mrun[j] = M;
  }
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      red[(wn * 128 + j * 32 + lane) * 2 + 0] = mrun[j];
      red[(wn * 128 + j * 32 + lane) * 2 + 1] = srun[j];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = wn * 128 + j * 32 + lane;
      const float mo = red[c * 2 + 0], so = red[c * 2 + 1];
      const float M = fmaxf(mrun[j], mo);
      const float S = (M == -INFINITY) ? 0.f
                                       : srun[j] * fast_exp2((mrun[j] - M) * kLog2e) +
                                             so * fast_exp2((mo - M) * kLog2e);
      const int n = n0 + c;
      if (n < N) {
        part_m[(int64_t)split * N + n] = M;
        part_s[(int64_t)split * N + n] = S;
      }
    }
  }
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

__global__ void __launch_bounds__(256)
lse_combine_kernel(const float* __restrict__ part_m, const float* __restrict__ part_s,
                   const float* __restrict__ zy, const int64_t* __restrict__ y, int N, int V,
                   int Sv, int64_t ignore, float* __restrict__ lse, float* __restrict__ loss_rows,
                   double* __restrict__ blk_sum, int* __restrict__ blk_cnt,
                   Header* __restrict__ hdr) {
  __shared__ double sh_s[256];
  __shared__ int sh_c[256];
  const int n = blockIdx.x * 256 + threadIdx.x;
  double s = 0.0;
  int c = 0;
  if (n < N) {
    float M = -INFINITY;
    for (int k = 0; k < Sv; ++k) M = fmaxf(M, part_m[(int64_t)k * N + n]);
    float S = 0.f;
    for (int k = 0; k < Sv; ++k) {
      const float m = part_m[(int64_t)k * N + n];
      S += part_s[(int64_t)k * N + n] * fast_exp2((m - M) * kLog2e);
    }
    const float l = M + fast_log2(S) * kLn2;
    lse[n] = l;
    const int64_t yy = y[n];
    float lr = 0.f;
    if (yy != ignore) {
      c = 1;
      if (yy < 0 || yy >= V) {
        lr = __builtin_nanf("");
        atomicOr(&hdr->status, 1);
      } else {
        lr = l - zy[n];
      }
    }
    loss_rows[n] = lr;
    s = (double)lr;
  }
  block_reduce_256(s, c, sh_s, sh_c);
  if (threadIdx.x == 0) {
    blk_sum[blockIdx.x] = s;
    blk_cnt[blockIdx.x] = c;
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
  }
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

__global__ void clear_status_kernel(Header* __restrict__ hdr, float* __restrict__ loss) {
  if (threadIdx.x == 0) {
    hdr->status = 0;
    hdr->count = 0;
    if (loss) *loss = 0.f;
  }
}

// ------------------------------------------------------------ backward ----
struct BandArgs {
  int nb0, ns_cur;   // first token row of the band, rows in it
  int vb0, vs_cur;   // first vocabulary row of the band, rows in it
  int ldz;           // row stride of the dZ band (elements) == VS
  int frows, fcols;  // filter-flag grid of the band (64x64 blocks)
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

template <typename T>
__global__ void __launch_bounds__(kThreads, 1)
bwd_dz_kernel(const T* __restrict__ H, const T* __restrict__ W, const int64_t* __restrict__ y,
              const float* __restrict__ lse, const float* __restrict__ dloss_rows,
              const Header* __restrict__ hdr, int N, int D, int V, int64_t ignore, int reduction,
              float eps, BandArgs band, int TMv, int TNn, T* __restrict__ dz,
              uint8_t* __restrict__ flags, uint8_t* __restrict__ flagsT) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  int tm, tn;
  grouped_tile(t, TMv, TNn, 4, tm, tn);
  const int v0 = band.vb0 + tm * kTile, n0 = band.nb0 + tn * kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const Operand A{reinterpret_cast<const char*>(W), D, V, D};
  const Operand B{reinterpret_cast<const char*>(H), D, N, D};
  const int nk = (D + kKStep<T> - 1) / kKStep<T>;
  f32x16 acc[4][4];
  gemm_tile<T, false, false>(A, B, v0, n0, nk, AllActive{}, acc, lds);

  float g[4], ml[4];
  int yt[4];
  bool valid[4], bad[4];
  const float gs = hdr->gscale;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 128 + j * 32 + (lane & 31);
    const bool in = n < N;
    const int64_t yy = in ? y[n] : ignore;
    valid[j] = in && yy != ignore;
    bad[j] = valid[j] && (yy < 0 || yy >= V);
    float gj = reduction == 2 ? (dloss_rows ? (in ? dloss_rows[n] : 0.f) : 1.f) : gs;
    gj = valid[j] ? gj : 0.f;
    g[j] = bad[j] ? __builtin_nanf("") : gj;
    ml[j] = in ? lse[n] * kLog2e : 0.f;
    yt[j] = (valid[j] && !bad[j]) ? (int)yy : -1;
  }
  const int vw = v0 + wm * 128;
  bool keep[2][2] = {{false, false}, {false, false}};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = vw + acc_row(i, r, lane);
      const bool vin = v < V;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = fast_exp2(fmaf(acc[i][j][r], kLog2e, -ml[j]));
        float G = p - (v == yt[j] ? 1.f : 0.f);
        const bool ok = valid[j] && vin;
        G = ok ? G : 0.f;
        keep[i >> 1][j >> 1] |= ok && (fabsf(G) >= eps || bad[j]);
        acc[i][j][r] = g[j] * G;
      }
    }
  const int fr0 = (n0 - band.nb0 + wn * 128) >> 6;   // flag row of this wave's first 64 rows
  const int fc0 = (v0 - band.vb0 + wm * 128) >> 6;   // flag column of its first 64 vocab rows
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const bool kp = __any(keep[bi][bj]);
      if (!kp) {
#pragma unroll
        for (int i = 2 * bi; i < 2 * bi + 2; ++i)
#pragma unroll
          for (int j = 2 * bj; j < 2 * bj + 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
      }
      if (lane == 0) {
        const int fr = fr0 + bj, fc = fc0 + bi;
        flags[fr * band.fcols + fc] = kp ? 0 : 1;
        flagsT[fc * band.frows + fr] = kp ? 0 : 1;
      }
    }
  // dZ band is [rows of the band][vocab of the band], row stride ldz
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nl = n0 - band.nb0 + wn * 128 + j * 32 + (lane & 31);
    T* row = dz + (int64_t)nl * band.ldz + (vw - band.vb0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = i * 32 + 8 * q + 4 * (lane >> 5);
        store4<T>(row + c, acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                  acc[i][j][4 * q + 3]);
      }
  }
}

struct SkipRowsOfFlags {   // active unless all four flags of this K step are set
  const uint8_t* base;     // first of the four flags of K step 0
  int step_stride;         // bytes between consecutive 64-wide K blocks
  int kshift;              // log2(64 / K elements per stage)
  __device__ __forceinline__ bool operator()(int kb) const {
    const uint32_t f = *reinterpret_cast<const uint32_t*>(base + (kb >> kshift) * step_stride);
    return f != 0x01010101u;
  }
};

template <typename T>
__global__ void __launch_bounds__(kThreads, 1)
bwd_grad_kernel(const T* __restrict__ H, const T* __restrict__ W, const T* __restrict__ dz,
                const uint8_t* __restrict__ flags, const uint8_t* __restrict__ flagsT,
                float* __restrict__ dH, float* __restrict__ dW, int N, int D, int V,
                BandArgs band, int T3m, int T2m, int Td, int beta_h, int beta_w) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int KS = kKStep<T>;
  constexpr int kshift = (KS == 64) ? 0 : 1;
  f32x16 acc[4][4];
  float* out;
  int mvalid, beta, tm, tn;
  const int T3 = T3m * Td;
  if (t < T3) {
    // dH[band rows, :] (+)= dZ[band rows, band vocab] . W[band vocab, :]
    grouped_tile(t, T3m, Td, 4, tm, tn);
    const int kpad = (band.vs_cur + kTile - 1) / kTile * kTile;
    const Operand A{reinterpret_cast<const char*>(dz), band.ldz, (int64_t)T3m * kTile, kpad};
    const Operand B{reinterpret_cast<const char*>(W + (int64_t)band.vb0 * D), D, D, band.vs_cur};
    const SkipRowsOfFlags act{flagsT + tm * 4, band.frows, kshift};
    gemm_tile<T, false, true>(A, B, tm * kTile, tn * kTile, (band.vs_cur + KS - 1) / KS, act, acc,
                              lds);
    out = dH + (int64_t)band.nb0 * D;
    mvalid = band.ns_cur;
    beta = beta_h;
  } else {
    // dW[band vocab, :] (+)= dZ[band rows, band vocab]^T . H[band rows, :]
    grouped_tile(t - T3, T2m, Td, 4, tm, tn);
    const Operand A{reinterpret_cast<const char*>(dz), band.ldz, (int64_t)T2m * kTile,
                    band.ns_cur};
    const Operand B{reinterpret_cast<const char*>(H + (int64_t)band.nb0 * D), D, D, band.ns_cur};
    const SkipRowsOfFlags act{flags + tm * 4, band.fcols, kshift};
    gemm_tile<T, true, true>(A, B, tm * kTile, tn * kTile, (band.ns_cur + KS - 1) / KS, act, acc,
                             lds);
    out = dW + (int64_t)band.vb0 * D;
    mvalid = band.vs_cur;
    beta = beta_w;
  }
  const int mw = tm * kTile + wm * 128, dw0 = tn * kTile + wn * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mw + acc_row(i, r, lane);
      if (m >= mvalid) continue;
      float* row = out + (int64_t)m * D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = dw0 + j * 32 + (lane & 31);
        if (d < D) row[d] = beta ? row[d] + acc[i][j][r] : acc[i][j][r];
      }
    }
  (void)V;
}

}  // namespace flce
