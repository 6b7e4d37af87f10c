// tile_mma.hpp -- the 256x256 MFMA tile core shared by every contraction of
// the fused LM-head + cross-entropy path on gfx950 (CDNA4).
//
// One workgroup = 256 threads = 4 wave64s arranged 2x2; each wave owns a
// 128x128 block of the 256x256 fp32 accumulator tile, i.e. 4x4 MFMA blocks of
// 32x32 (v_mfma_f32_32x32x16_bf16 for bf16 inputs, v_mfma_f32_32x32x2_f32 for
// fp32 inputs).  Operands are staged through LDS 128 bytes of K at a time per
// tile row, double buffered (2 stages x (A + B) x 32 KiB = 128 KiB of the
// 160 KiB LDS), with one barrier per K step.  Global loads of step k+1 are in
// flight while step k is multiplied.
//
// LDS layout: each operand tile is [256 rows][128 bytes], row r holding the K
// slice of tile row r.  The 16-byte chunk c of row r sits at chunk position
// c ^ swz(r), swz(r) = (r ^ (r >> 3)) & 7, so that 8 consecutive rows read at
// one chunk index (the MFMA fragment read) and rows {8i + j} written at one
// chunk index (the transposing store) both spread over all banks.
//
// Operands come in two storage orders:
//   natural    : element (m, k) at base[m * ld + k]  (K contiguous)
//   transposed : element (m, k) at base[k * ld + m]  (M contiguous)
// A transposed operand is read as E x E blocks (E = elements per 16 bytes),
// transposed in registers and written to LDS in the natural layout, so the
// fragment reads are identical for both orders.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 256;                        // output tile edge
constexpr int kThreads = 256;                     // 4 waves
constexpr int kRowBytes = 128;                    // K bytes per LDS row per stage
constexpr int kOperandBytes = kTile * kRowBytes;  // 32 KiB
constexpr int kStageBytes = 2 * kOperandBytes;    // A + B
constexpr int kLdsBytes = 2 * kStageBytes;        // two stages: 128 KiB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 values are carried as uint16_t bit patterns on the host side of the
// templates; the MFMA sees them as __bf16.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int kPerChunk = 8; };
template <> struct Elem<float> { static constexpr int kPerChunk = 4; };
template <typename T> constexpr int kKStep = 8 * Elem<T>::kPerChunk;  // K per stage

struct Operand {
  const char* base;  // address of element (0, 0)
  int64_t ld;        // elements between consecutive stored rows
  int64_t mext;      // M (natural: stored rows; transposed: stored columns) readable
  int64_t kext;      // K readable
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * kRowBytes + ((c ^ swz(r)) << 4); }

// ---------------------------------------------------------------- loads ----
template <typename T>
__device__ __forceinline__ void load_natural(u32x4 (&r)[8], const Operand& op, int m0, int k0,
                                             int tid) {
  constexpr int E = Elem<T>::kPerChunk;
  const int64_t k = k0 + (tid & 7) * E;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + (tid >> 3) + 32 * i;
    if (m < op.mext && k < op.kext)
      r[i] = *reinterpret_cast<const u32x4*>(op.base + (m * op.ld + k) * (int64_t)sizeof(T));
    else
      r[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_natural(char* s, const u32x4 (&r)[8], int tid) {
  const int c = tid & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(s + lds_off((tid >> 3) + 32 * i, c)) = r[i];
}

template <typename T>
__device__ __forceinline__ void load_transposed(u32x4 (&r)[8], const Operand& op, int m0, int k0,
                                                int tid);

// bf16: 8x8 blocks, one per thread: 32 blocks along M x 8 along K.
template <>
__device__ __forceinline__ void load_transposed<uint16_t>(u32x4 (&r)[8], const Operand& op,
                                                          int m0, int k0, int tid) {
  const int64_t m = m0 + (tid & 31) * 8;
  const int64_t kb = k0 + (tid >> 5) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t k = kb + i;
    if (k < op.kext && m < op.mext)
      r[i] = *reinterpret_cast<const u32x4*>(op.base + (k * op.ld + m) * 2);
    else
      r[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

// fp32: 4x4 blocks, two per thread: 64 blocks along M x 8 along K.
template <>
__device__ __forceinline__ void load_transposed<float>(u32x4 (&r)[8], const Operand& op, int m0,
                                                       int k0, int tid) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int blk = tid + 256 * h;
    const int64_t m = m0 + (blk & 63) * 4;
    const int64_t kb = k0 + (blk >> 6) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t k = kb + i;
      if (k < op.kext && m < op.mext)
        r[h * 4 + i] = *reinterpret_cast<const u32x4*>(op.base + (k * op.ld + m) * 4);
      else
        r[h * 4 + i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <typename T>
__device__ __forceinline__ void store_transposed(char* s, const u32x4 (&r)[8], int tid);

template <>
__device__ __forceinline__ void store_transposed<uint16_t>(char* s, const u32x4 (&r)[8], int tid) {
  const int mb = tid & 31, kb = tid >> 5;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = r[2 * w][j >> 1], y = r[2 * w + 1][j >> 1];
      o[w] = (j & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
    }
    *reinterpret_cast<u32x4*>(s + lds_off(mb * 8 + j, kb)) = o;
  }
}

template <>
__device__ __forceinline__ void store_transposed<float>(char* s, const u32x4 (&r)[8], int tid) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int blk = tid + 256 * h;
    const int mb = blk & 63, kb = blk >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 o{r[h * 4 + 0][j], r[h * 4 + 1][j], r[h * 4 + 2][j], r[h * 4 + 3][j]};
      *reinterpret_cast<u32x4*>(s + lds_off(mb * 4 + j, kb)) = o;
    }
  }
}

template <typename T, bool TRANS>
__device__ __forceinline__ void load_op(u32x4 (&r)[8], const Operand& op, int m0, int k0, int tid) {
  if constexpr (TRANS) load_transposed<T>(r, op, m0, k0, tid);
  else load_natural<T>(r, op, m0, k0, tid);
}

template <typename T, bool TRANS>
__device__ __forceinline__ void store_op(char* s, const u32x4 (&r)[8], int tid) {
  if constexpr (TRANS) store_transposed<T>(s, r, tid);
  else store_natural(s, r, tid);
}

// ------------------------------------------------------------ multiply ----
// Lane l of a wave reads, for tile row (wave base + 32 i + l % 32), chunk
// (2 ks + l / 32): 8 consecutive K values for bf16, 4 for fp32.  A and B use
// the same lane -> K mapping, so every MFMA pairs equal K indices.
template <typename T>
__device__ __forceinline__ void mma_stage(const char* sA, const char* sB, f32x16 (&acc)[4][4],
                                          int wm, int wn, int lane);

template <>
__device__ __forceinline__ void mma_stage<uint16_t>(const char* sA, const char* sB,
                                                    f32x16 (&acc)[4][4], int wm, int wn,
                                                    int lane) {
  const int lr = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(sA + lds_off(wm * 128 + i * 32 + lr, ks * 2 + hf));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(sB + lds_off(wn * 128 + j * 32 + lr, ks * 2 + hf));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

template <>
__device__ __forceinline__ void mma_stage<float>(const char* sA, const char* sB,
                                                 f32x16 (&acc)[4][4], int wm, int wn, int lane) {
  const int lr = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    f32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const f32x4*>(sA + lds_off(wm * 128 + i * 32 + lr, ks * 2 + hf));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const f32x4*>(sB + lds_off(wn * 128 + j * 32 + lr, ks * 2 + hf));
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][t], b[j][t], acc[i][j], 0, 0, 0);
  }
}

struct AllActive {
  __device__ __forceinline__ bool operator()(int) const { return true; }
};

// acc[i][j] (wave (wm, wn)) receives C[m0 + 128 wm + 32 i + row][n0 + 128 wn + 32 j + col]
// with C = sum over active K steps of A[m][k] B[n][k]; in register r of lane
// l: row = 8 (r / 4) + 4 (l / 32) + r % 4, col = l % 32.
// `active(kb)` must give the same answer in every thread of the workgroup.
template <typename T, bool AT, bool BT, class Active>
__device__ __forceinline__ void gemm_tile(const Operand& A, const Operand& B, int m0, int n0,
                                          int nk, const Active& active, f32x16 (&acc)[4][4],
                                          char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int KS = kKStep<T>;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  int kb = 0;
  while (kb < nk && !active(kb)) ++kb;
  if (kb >= nk) return;
  u32x4 ra[8], rb[8];
  load_op<T, AT>(ra, A, m0, kb * KS, tid);
  load_op<T, BT>(rb, B, n0, kb * KS, tid);
  store_op<T, AT>(lds, ra, tid);
  store_op<T, BT>(lds + kOperandBytes, rb, tid);
  __syncthreads();
  int buf = 0;
  for (;;) {
    int nxt = kb + 1;
    while (nxt < nk && !active(nxt)) ++nxt;
    const bool more = nxt < nk;
    if (more) {
      load_op<T, AT>(ra, A, m0, nxt * KS, tid);
      load_op<T, BT>(rb, B, n0, nxt * KS, tid);
    }
    const char* s = lds + buf * kStageBytes;
    mma_stage<T>(s, s + kOperandBytes, acc, wm, wn, lane);
    if (!more) break;
    buf ^= 1;
    char* w = lds + buf * kStageBytes;
    store_op<T, AT>(w, ra, tid);
    store_op<T, BT>(w + kOperandBytes, rb, tid);
    __syncthreads();
    kb = nxt;
  }
  __syncthreads();  // LDS may be reused by the caller
}

// Row (within the wave's 128-row block) held by register r of `lane` in
// MFMA block i.
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// The hardware sends workgroup b to XCD b % 8.  Give XCD x a contiguous range
// of tile ids so tiles that share operands share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int q = G >> 3, rem = G & 7;
  const int x = b & 7, idx = b >> 3;
  return x * q + (x < rem ? x : rem) + idx;
}

// Tile id t -> (tm, tn) in a TM x TN grid, visiting GM tile rows at a time.
__device__ __forceinline__ void grouped_tile(int t, int TM, int TN, int GM, int& tm, int& tn) {
  const int per = GM * TN;
  const int g = t / per, first = g * GM;
  const int gm = (TM - first) < GM ? (TM - first) : GM;
  const int in = t - g * per;
  tm = first + in % gm;
  tn = in / gm;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v{(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace flce
