// tile_mma.hpp -- the 256x256 MFMA tile core shared by every contraction of
// the fused LM-head + cross-entropy path on gfx950 (CDNA4).
//
// One workgroup = 256 threads = 4 wave64s arranged 2x2; each wave owns a
// 128x128 block of the 256x256 fp32 accumulator tile, i.e. 4x4 MFMA blocks of
// 32x32 (v_mfma_f32_32x32x16_bf16 for bf16 inputs, v_mfma_f32_32x32x2_f32 for
// fp32 inputs).  Operands are staged through LDS 128 bytes of K at a time per
// tile row, double buffered, with one barrier per K step; the global loads of
// step k+1 are in flight while step k is multiplied.
//
// LDS layout: each operand tile is [256 rows][144 bytes]: row r holds the
// 128-byte K slice of tile row r followed by 16 bytes of padding.  With the
// 144-byte stride, 8 (or 16) consecutive rows read at one 16-byte chunk index
// fall in distinct banks, and every fragment address is one per-lane base
// plus a compile-time offset.  2 stages x 2 operands x 36 KiB = 144 KiB of
// the 160 KiB LDS.
//
// Global loads are raw buffer loads: one 32-bit offset per lane and load,
// fixed for the whole K loop, against a buffer descriptor whose base moves
// with the K step.  Lanes with nothing to load use an offset beyond the
// descriptor's range, which the hardware answers with zeros, so there are
// no branches around loads.
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

constexpr int kTile = 256;                         // output tile edge
constexpr int kThreads = 256;                      // 4 waves
constexpr int kRowBytes = 128;                     // K bytes per LDS row per stage
constexpr int kRowStride = 144;                    // LDS bytes per row (padded)
constexpr int kOperandBytes = kTile * kRowStride;  // 36 KiB
constexpr int kStageBytes = 2 * kOperandBytes;     // A + B
constexpr int kLdsBytes = 2 * kStageBytes;         // two stages: 144 KiB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr uint32_t kOob = 0x80000000u;             // offset past every descriptor range
constexpr int kRsrcFlags = 0x00020000;             // raw 32-bit buffer, no swizzle

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
  // Optional (bf16 LDS-DMA core only), rows gathered through a map; byte
  // offsets of mapped rows must stay below 2^31.
  //  natural operand: stored row r (M) is row rowmap[r] of `base` (global map);
  //  transposed operand: k row k is row table[k % 2][k / 2] of `base`, where
  //  rowmap points at an LDS table with rowmap_half entries per parity.
  const int* rowmap = nullptr;
  int rowmap_half = 0;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, 0x7fffffff, kRsrcFlags);
}

// -------------------------------------------------------------- loaders ----
// A loader owns the per-lane offsets of its 8 loads (fixed over the K loop)
// and moves a descriptor base along K.
template <typename T, bool TRANS> struct Loader;

// natural: thread t loads chunk (t & 7) of tile rows (t >> 3) + 32 i.
template <typename T> struct Loader<T, false> {
  static constexpr int E = Elem<T>::kPerChunk;
  uint32_t off[8];
  int c;
  const char* base;   // element (m0, 0)
  int64_t kext;
  __device__ __forceinline__ void init(const Operand& op, int m0, int tid) {
    c = tid & 7;
    base = op.base + (int64_t)m0 * op.ld * (int64_t)sizeof(T);
    kext = op.kext;
    const int r0 = tid >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = (int64_t)m0 + r0 + 32 * i;
      off[i] = m < op.mext ? (uint32_t)(((int64_t)(r0 + 32 * i) * op.ld + c * E) * (int64_t)sizeof(T))
                           : kOob;
    }
  }
  __device__ __forceinline__ void load(u32x4 (&r)[8], int k0) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)k0 * sizeof(T));
    const bool kin = k0 + c * E < kext;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, kin ? off[i] : kOob, 0, 0));
  }
  // LDS: row (t >> 3) + 32 i, chunk t & 7
  __device__ __forceinline__ static int store_base(int tid) {
    return (tid >> 3) * kRowStride + (tid & 7) * 16;
  }
  __device__ __forceinline__ static void store(char* s, const u32x4 (&r)[8], int tid) {
    char* p = s + store_base(tid);
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(p + i * 32 * kRowStride) = r[i];
  }
};

// transposed bf16: thread t owns the 8x8 block (k block t & 7, m block t >> 3):
// 8 loads of 16 bytes (8 m values of one k row); lanes 0..7 cover 8 k rows of
// one 64-column span, so each load instruction reads whole 128-byte rows.
template <> struct Loader<uint16_t, true> {
  uint32_t off[8];
  int kb;
  bool min;
  const char* base;   // element (0, m0) of the stored [k][m] matrix
  int64_t ld, kext;
  __device__ __forceinline__ void init(const Operand& op, int m0, int tid) {
    kb = tid & 7;
    const int mb = tid >> 3;
    base = op.base + (int64_t)m0 * 2;
    ld = op.ld;
    kext = op.kext;
    min = (int64_t)m0 + mb * 8 < op.mext;
#pragma unroll
    for (int i = 0; i < 8; ++i) off[i] = (uint32_t)(((int64_t)(kb * 8 + i) * op.ld + mb * 8) * 2);
  }
  __device__ __forceinline__ void load(u32x4 (&r)[8], int k0) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)k0 * ld * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = min && (k0 + kb * 8 + i < kext);
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off[i] : kOob, 0, 0));
    }
  }
  // LDS: rows (t >> 3) * 8 + j, chunk t & 7; 8x8 transpose in registers.
  __device__ __forceinline__ static void store(char* s, const u32x4 (&r)[8], int tid) {
    char* p = s + (tid >> 3) * 8 * kRowStride + (tid & 7) * 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = r[2 * w][j >> 1], y = r[2 * w + 1][j >> 1];
        o[w] = (j & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
      }
      *reinterpret_cast<u32x4*>(p + j * kRowStride) = o;
    }
  }
};

// transposed fp32: 4x4 blocks, two per thread: block b = t + 256 h has
// k block b & 7 and m block b >> 3 (64 m blocks of 4).
template <> struct Loader<float, true> {
  uint32_t off[8];
  int kb;
  bool min[2];
  const char* base;
  int64_t ld, kext;
  __device__ __forceinline__ void init(const Operand& op, int m0, int tid) {
    kb = tid & 7;
    base = op.base + (int64_t)m0 * 4;
    ld = op.ld;
    kext = op.kext;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mb = (tid + 256 * h) >> 3;
      min[h] = (int64_t)m0 + mb * 4 < op.mext;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        off[h * 4 + i] = (uint32_t)(((int64_t)(kb * 4 + i) * op.ld + mb * 4) * 4);
    }
  }
  __device__ __forceinline__ void load(u32x4 (&r)[8], int k0) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)k0 * ld * 4);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = min[h] && (k0 + kb * 4 + i < kext);
        r[h * 4 + i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off[h * 4 + i] : kOob, 0, 0));
      }
  }
  __device__ __forceinline__ static void store(char* s, const u32x4 (&r)[8], int tid) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mb = (tid + 256 * h) >> 3;
      char* p = s + mb * 4 * kRowStride + (tid & 7) * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 o{r[h * 4 + 0][j], r[h * 4 + 1][j], r[h * 4 + 2][j], r[h * 4 + 3][j]};
        *reinterpret_cast<u32x4*>(p + j * kRowStride) = o;
      }
    }
  }
};

// ------------------------------------------------------------ multiply ----
// Lane l of a wave reads, for tile row (wave base + 32 i + l % 32), chunk
// (2 ks + l / 32): 8 consecutive K values for bf16, 4 for fp32.  A and B use
// the same lane -> K mapping, so every MFMA pairs equal K indices.
__device__ __forceinline__ int frag_base(int wrow, int lane) {
  return (wrow + (lane & 31)) * kRowStride + (lane >> 5) * 16;
}

// fresh: the first MFMA of every accumulator takes C = 0 (start of a tile).
template <typename T>
__device__ __forceinline__ void mma_stage(const char* sA, const char* sB, f32x16 (&acc)[4][4],
                                          bool fresh);

template <>
__device__ __forceinline__ void mma_stage<uint16_t>(const char* sA, const char* sB,
                                                    f32x16 (&acc)[4][4], bool fresh) {
  const f32x16 zero = {};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(sA + i * 32 * kRowStride + ks * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(sB + j * 32 * kRowStride + ks * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j],
                                                            (ks == 0 && fresh) ? zero : acc[i][j],
                                                            0, 0, 0);
  }
}

template <>
__device__ __forceinline__ void mma_stage<float>(const char* sA, const char* sB,
                                                 f32x16 (&acc)[4][4], bool fresh) {
  const f32x16 zero = {};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    f32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const f32x4*>(sA + i * 32 * kRowStride + ks * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const f32x4*>(sB + j * 32 * kRowStride + ks * 32);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
              a[i][t], b[j][t], (ks == 0 && t == 0 && fresh) ? zero : acc[i][j], 0, 0, 0);
  }
}

// Pins the accumulators to AGPRs at a tile's end and waits out the MFMA
// result latency before VALU code reads them (an 8-pass 32x32 MFMA needs 11
// wait states before a VALU read of its result; this gives 34).  Passing every
// block as an "+a" operand orders the fence after all MFMAs of the tile and
// before every read, and keeps the register allocator from moving the
// accumulators into VGPRs around an epilogue.
__device__ __forceinline__ void acc_fence(f32x16 (&acc)[4][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 1"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                 "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]),
                 "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[2][2]), "+a"(acc[2][3]),
                 "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]));
}
__device__ __forceinline__ void acc_fence(f32x16 (&acc)[2][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 1"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                 "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]));
}

struct AllActive {
  __device__ __forceinline__ void prepare(int) {}
  __device__ __forceinline__ bool operator()(int) const { return true; }
  __device__ __forceinline__ int next(int s, int nsteps) const { return s < nsteps ? s : nsteps; }
};

// acc[i][j] (wave (wm, wn)) receives C[m0 + 128 wm + 32 i + row][n0 + 128 wn + 32 j + col]
// with C = sum over active K steps of A[m][k] B[n][k]; in register r of lane
// l: row = 8 (r / 4) + 4 (l / 32) + r % 4, col = l % 32.
// `active(kb)` must give the same answer in every thread of the workgroup.
template <typename T, bool AT, bool BT, class Active>
__device__ __forceinline__ void gemm_tile(const Operand& A, const Operand& B, int m0, int n0,
                                          int nk, Active active, f32x16 (&acc)[4][4],
                                          char* lds) {
  active.prepare(nk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int KS = kKStep<T>;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  int kb = active.next(0, nk);
  if (kb >= nk) return;
  Loader<T, AT> la;
  Loader<T, BT> lb;
  la.init(A, m0, tid);
  lb.init(B, n0, tid);
  const int fa = frag_base(wm * 128, lane), fb = frag_base(wn * 128, lane);
  u32x4 ra[8], rb[8];
  la.load(ra, kb * KS);
  lb.load(rb, kb * KS);
  Loader<T, AT>::store(lds, ra, tid);
  Loader<T, BT>::store(lds + kOperandBytes, rb, tid);
  __syncthreads();
  int buf = 0;
  // single-exit loop: the accumulators have one loop-carried definition
  while (kb < nk) {
    const int nxt = active.next(kb + 1, nk);
    const bool more = nxt < nk;
    if (more) {
      la.load(ra, nxt * KS);
      lb.load(rb, nxt * KS);
    }
    const char* s = lds + buf * kStageBytes;
    mma_stage<T>(s + fa, s + kOperandBytes + fb, acc, false);
    if (more) {
      char* w = lds + (buf ^ 1) * kStageBytes;
      Loader<T, AT>::store(w, ra, tid);
      Loader<T, BT>::store(w + kOperandBytes, rb, tid);
      __syncthreads();
    }
    buf ^= 1;
    kb = nxt;
  }
  acc_fence(acc);
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

// As xcd_remap, for a grid of three consecutive kinds of tiles [0, c1),
// [c1, c2), [c2, G), longest first: XCD x gets an even share of every kind
// as a contiguous range and is sent them kind by kind, so that no XCD is left
// holding most of the long work.  The tiles of a kind that do not divide
// evenly go one each to the XCDs that follow those given the previous
// kind's, which keeps every XCD's total equal to the number of workgroups
// the hardware sends it.
__device__ __forceinline__ int xcd_remap_kinds(int b, int G, int c1, int c2) {
  const int x = b & 7;
  int idx = b >> 3, j0 = 0, lo = 0;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int hi = k == 0 ? c1 : (k == 1 ? c2 : G);
    const int n = hi - lo, q = n >> 3, r = n & 7;
    int before = 0;
    for (int xx = 0; xx < x; ++xx) before += ((xx - j0) & 7) < r ? 1 : 0;
    const int cnt = q + (((x - j0) & 7) < r ? 1 : 0);
    if (idx < cnt) return lo + x * q + before + idx;
    idx -= cnt;
    j0 += r;
    lo = hi;
  }
  return G;   // not reached for b < G
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
