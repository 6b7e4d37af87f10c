// tile_dma.hpp -- bf16 256x256 MFMA tile core fed by LDS DMA (gfx950).
//
// Same output contract as gemm_tile in tile_mma.hpp (acc layout, Operand,
// natural / transposed storage), for bf16 operands only:
//
//  * Operands go from global memory straight into LDS with
//    `buffer_load_dwordx4 ... lds` (16 bytes per lane, lane-linear in LDS):
//    no staging registers, no LDS store instructions, no register
//    transposes.  Each lane loads whichever global chunk belongs at its LDS
//    slot, which is how the layouts below get their swizzles.
//  * Stages of 64 K values, so that every DMA instruction reads whole
//    128-byte lines (8 rows of a natural operand, 2 k rows of a transposed
//    one): measured on MI355X, loads of half lines reach about half the
//    L2-to-CU rate of whole lines.  Two stage slots of 64 KiB (A + B).
//  * The LDS serves 256 bytes per clock (64 banks of 4 bytes; measured: 16
//    lanes of a ds_read_b128 go in one clock), so each swizzle below spreads
//    the lanes served together over all 64 banks.
//  * Natural operands ([m][k], K contiguous) sit in LDS as [256 rows][128 B]:
//    16-byte chunk c of row r at chunk c ^ ((r >> 1) & 7).  An MFMA fragment
//    (8 K values of one row per lane) is one ds_read_b128.
//  * Transposed operands ([k][m], M contiguous) sit in LDS as
//    [64 k rows][512 B]: 32-byte segment s of row k at segment
//    s ^ (2 (k & 3)).
//    A fragment is two ds_read_b64_tr_b16: within each 16-lane group the
//    hardware hands lane i the element (row kbase + e, column mbase + i),
//    e = 0..3, when source lane j points at row kbase + j / 4, columns
//    mbase + 4 (j % 4) .. +3 (measured lane layout of the instruction).
//  * One barrier per stage.  gemm_tile_dma2 (the default) reads all four
//    sub-steps' fragments of a stage before its barrier, which sits after the
//    second sub-step: the slot just read then takes the DMAs of the stage
//    after next over the last two sub-steps, one instruction per MFMA pair,
//    which is the rate the address unit drains them at (measured on MI355X:
//    issuing them all in one sub-step stalls the MFMA issue; 8192^2 x 4096
//    GEMM 1294 -> 1348 TFLOP/s).  gemm_tile_dma keeps two fragment sets and
//    the barrier before the last sub-step, for callers with less register
//    room.
//  * Each workgroup also touches, one dword per 128-byte line, its share of
//    the lines of the stage two ahead of the one being loaded, so those
//    lines are in L2 when their DMAs are issued.
//
// The DMA instructions are inline assembly so that the compiler does not
// wait for every outstanding DMA before each LDS read; the code below waits
// exactly for the stage it is about to read.
#pragma once

#include <type_traits>

#include "tile_mma.hpp"

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

namespace flce {

constexpr int kDmaSlots = 2;
constexpr int kDmaKStep = 64;                    // bf16 K values per stage
constexpr int kDmaKs = kDmaKStep / 16;           // MFMA K sub-steps per stage
constexpr int kDmaOpBytes = 256 * 128;           // one operand of one stage: 32 KiB
constexpr int kDmaStageBytes = 2 * kDmaOpBytes;  // A + B
constexpr int kDmaLdsBytes = kDmaSlots * kDmaStageBytes;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)p;   // generic -> LDS offset (low 32 bits of the aperture address)
}

// One lane's 16 bytes into LDS slot m0 + 16 * lane.
__device__ __forceinline__ void dma16(uint32_t lds_base, uint32_t voff, __amdgpu_buffer_rsrc_t rs) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rs)
               : "memory", "m0");
}

// One lane's 4 bytes into LDS at m0 + 4 * lane: pulls the line holding them
// into L2 ahead of the stage that loads it (the LDS target is a dummy area).
__device__ __forceinline__ void dma4(uint32_t lds_base, uint32_t voff, __amdgpu_buffer_rsrc_t rs) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rs)
               : "memory", "m0");
}

// The workgroups that run at the same time on one XCD and share an operand
// block split the block's lines of a future stage `nshare` ways (a power of
// two); this workgroup touches part `share`.
struct L2Split {
  int share, nshare;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void barrier_raw() { asm volatile("s_barrier" ::: "memory"); }

// ------------------------------------------------------------- loaders ----
// Each wave issues 8 DMA instructions per operand per stage (32 per
// workgroup = 32 KiB), every instruction reading whole 128-byte lines.
// Offsets are fixed per lane; the descriptor base moves along K.  Rows or
// columns outside the operand get an out-of-range offset, so the hardware
// writes zeros into their LDS slots.

// natural [m][k]: instruction q of wave w covers tile rows 8 (8 w + q) .. +7
// (128 bytes = 64 K values each); lane L -> row 8 (8 w + q) + L / 8, LDS
// chunk L % 8, global chunk (L % 8) ^ ((row / 2) % 8), where
// (row / 2) % 8 = 4 (q % 2) + L / 16.
struct DmaNatural {
  uint32_t off[8];
  int kc[2];              // K element offset of this lane's chunk, by q parity
  const char* base;       // element (m0, 0)
  int64_t ld, kext, mrem;
  bool gather;            // rows through op.rowmap (no line prefetch then)
  __device__ __forceinline__ void init(const Operand& op, int m0, int wave, int lane) {
    gather = op.rowmap != nullptr;
    base = gather ? op.base : op.base + (int64_t)m0 * op.ld * 2;
    ld = op.ld;
    kext = op.kext;
    mrem = op.mext - m0;
#pragma unroll
    for (int par = 0; par < 2; ++par) kc[par] = ((lane & 7) ^ (4 * par + (lane >> 4))) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 8 * (8 * wave + q) + (lane >> 3);
      const bool in = (int64_t)m0 + row < op.mext;
      const int64_t r = gather ? (in ? (int64_t)op.rowmap[m0 + row] : 0) : row;
      off[q] = in ? (uint32_t)((r * op.ld + kc[q & 1]) * 2) : kOob;
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds_op, int k0, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)k0 * 2);
    const bool kin0 = k0 + kc[0] < kext, kin1 = k0 + kc[1] < kext;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      dma16(lds_op + (8 * wave + q) * 1024, ((q & 1) ? kin1 : kin0) ? off[q] : kOob, rs);
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int k0) const {
    return make_rsrc(base + (int64_t)k0 * 2);
  }
  // instruction Q alone (`more` false: every lane out of range, no memory access)
  template <int Q>
  __device__ __forceinline__ void issue_q(uint32_t lds_op, int k0, int wave, bool more,
                                          __amdgpu_buffer_rsrc_t rs) const {
    const bool kin = more && k0 + kc[Q & 1] < kext;
    dma16(lds_op + (8 * wave + Q) * 1024, kin ? off[Q] : kOob, rs);
  }
  // one 128-byte line per tile row: lane L touches row share * per + L % per
  __device__ __forceinline__ void prefetch(uint32_t lds_dummy, int k0, L2Split sp, int lane,
                                           bool on) const {
    const int per = kTile / sp.nshare;
    const int row = sp.share * per + (lane & (per - 1));
    const bool ok = on && !gather && row < mrem && k0 < kext;
    dma4(lds_dummy, ok ? (uint32_t)((int64_t)row * ld * 2) : kOob,
         make_rsrc(base + (int64_t)k0 * 2));
  }
};

// transposed [k][m]: instruction q of wave w covers k rows 2 (8 w + q), +1
// (512 bytes = 256 M values each); lane L -> k row 2 (8 w + q) + L / 32, LDS
// segment (L % 32) / 2, half L % 2, global segment
// ((L % 32) / 2) ^ (2 (krow % 4)).
struct DmaTransposed {
  uint32_t off[8];
  bool colok[8];
  const char* base;       // element (0, m0) of the stored [k][m] matrix
  int64_t ld, kext, mrem;
  int krow0;              // k row of instruction 0 for this lane
  __device__ __forceinline__ void init(const Operand& op, int m0, int wave, int lane) {
    base = op.base + (int64_t)m0 * 2;
    ld = op.ld;
    kext = op.kext;
    mrem = op.mext - m0;
    krow0 = 16 * wave + (lane >> 5);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int krow = krow0 + 2 * q;
      const int seg = ((lane & 31) >> 1) ^ (2 * (krow & 3));
      const int m = seg * 16 + (lane & 1) * 8;
      colok[q] = (int64_t)m0 + m < op.mext;
      off[q] = (uint32_t)(((int64_t)krow * op.ld + m) * 2);
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds_op, int k0, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)k0 * ld * 2);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool ok = colok[q] && (k0 + krow0 + 2 * q < kext);
      dma16(lds_op + (8 * wave + q) * 1024, ok ? off[q] : kOob, rs);
    }
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int k0) const {
    return make_rsrc(base + (int64_t)k0 * ld * 2);
  }
  template <int Q>
  __device__ __forceinline__ void issue_q(uint32_t lds_op, int k0, int wave, bool more,
                                          __amdgpu_buffer_rsrc_t rs) const {
    const bool ok = more && colok[Q] && (k0 + krow0 + 2 * Q < kext);
    dma16(lds_op + (8 * wave + Q) * 1024, ok ? off[Q] : kOob, rs);
  }
  // four 128-byte lines per k row: lane L touches line li = share * per + L % per,
  // k row li / 4, quarter li % 4
  __device__ __forceinline__ void prefetch(uint32_t lds_dummy, int k0, L2Split sp, int lane,
                                           bool on) const {
    const int per = kTile / sp.nshare;
    const int li = sp.share * per + (lane & (per - 1));
    const int krow = li >> 2, quarter = li & 3;
    const bool ok = on && k0 + krow < kext && quarter * 64 < mrem;
    dma4(lds_dummy, ok ? (uint32_t)((int64_t)krow * ld * 2 + quarter * 128) : kOob,
         make_rsrc(base + (int64_t)k0 * ld * 2));
  }
};

template <bool TRANS> struct DmaLoader;
template <> struct DmaLoader<false> : DmaNatural {};
template <> struct DmaLoader<true> : DmaTransposed {};

// transposed [k][m] operand whose k rows are gathered: op.rowmap points at
// an LDS table (built by the caller before the contraction) that holds the
// operand's row indices split by parity, table[h][j] = row of k = 2 j + h,
// `table_half` entries per parity.  A lane loads k rows k0 + 16 w + 2 q + h
// (h = lane / 32, q = 0..7), so its eight indices of a stage are eight
// consecutive entries of table[h]: two 16-byte LDS reads, issued by rows()
// before the barrier that precedes the stage's DMAs.
constexpr int kGatherTableBytes = 16384;   // 4096 rows
struct DmaTransposedGather {
  uint32_t col[8];        // this lane's byte column (m) for instruction q
  bool colok[8];
  const char* base;       // element (0, m0)
  const char* table;      // LDS table (generic pointer into LDS)
  int table_half;
  int64_t ld, kext, mrem;
  int krow0;              // 16 w + L / 32
  int wave16;             // 16 w
  int idx[8];             // row of k0 + 16 w + 2 q + h, per q
  bool gather = true;
  __device__ __forceinline__ void init(const Operand& op, int m0, int wave, int lane) {
    base = op.base + (int64_t)m0 * 2;
    table = reinterpret_cast<const char*>(op.rowmap);
    table_half = op.rowmap_half;
    ld = op.ld;
    kext = op.kext;
    mrem = op.mext - m0;
    wave16 = 16 * wave;
    krow0 = wave16 + (lane >> 5);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int krow = krow0 + 2 * q;
      const int seg = ((lane & 31) >> 1) ^ (2 * (krow & 3));
      const int m = seg * 16 + (lane & 1) * 8;
      colok[q] = (int64_t)m0 + m < op.mext;
      col[q] = (uint32_t)(m * 2);
    }
  }
  __device__ __forceinline__ void rows(int k0) {
    typedef __attribute__((address_space(3))) const i32x4 lds_i32x4;
    const int h = (threadIdx.x >> 5) & 1;
    lds_i32x4* p = (lds_i32x4*)(lds_char*)(table + (h * table_half + ((k0 + wave16) >> 1)) * 4);
    const i32x4 lo = p[0], hi = p[1];
    idx[0] = lo.x; idx[1] = lo.y; idx[2] = lo.z; idx[3] = lo.w;
    idx[4] = hi.x; idx[5] = hi.y; idx[6] = hi.z; idx[7] = hi.w;
  }
  __device__ __forceinline__ void rows_wait() {}
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int) const { return make_rsrc(base); }
  template <int Q>
  __device__ __forceinline__ void issue_q(uint32_t lds_op, int k0, int wave, bool more,
                                          __amdgpu_buffer_rsrc_t rs) const {
    const bool ok = more && colok[Q] && (k0 + krow0 + 2 * Q < kext);
    const uint32_t o = (uint32_t)idx[Q] * (uint32_t)(ld * 2) + col[Q];   // < 2^31
    dma16(lds_op + (8 * wave + Q) * 1024, ok ? o : kOob, rs);
  }
  __device__ __forceinline__ void issue(uint32_t lds_op, int k0, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = rsrc(k0);
    issue_q<0>(lds_op, k0, wave, true, rs);
    issue_q<1>(lds_op, k0, wave, true, rs);
    issue_q<2>(lds_op, k0, wave, true, rs);
    issue_q<3>(lds_op, k0, wave, true, rs);
    issue_q<4>(lds_op, k0, wave, true, rs);
    issue_q<5>(lds_op, k0, wave, true, rs);
    issue_q<6>(lds_op, k0, wave, true, rs);
    issue_q<7>(lds_op, k0, wave, true, rs);
  }
  __device__ __forceinline__ void prefetch(uint32_t lds_dummy, int, L2Split, int, bool) const {
    dma4(lds_dummy, kOob, make_rsrc(base));   // keeps the per-wave load count; touches nothing
  }
};

// Fills the LDS gather table of a transposed gathered operand from the global
// row indices rowmap[0 .. rows) (zeros after them, up to `half` entries per
// parity); every thread of the workgroup takes part, and a barrier follows.
__device__ __forceinline__ void gather_table(char* lds_table, const int* rowmap, int rows,
                                             int half) {
  int* t = reinterpret_cast<int*>(lds_table);
  for (int k = threadIdx.x; k < 2 * half; k += blockDim.x)
    t[(k & 1) * half + (k >> 1)] = k < rows ? rowmap[k] : 0;
  __syncthreads();
}

// ----------------------------------------------------------- fragments ----
// Fragments of MFMA K sub-step KS (0..3) of a stage for the wave's 4 blocks.
template <bool TRANS> struct FragReader;

// natural: row r = wbase + 32 i + lane % 32, chunk 2 KS + lane / 32 stored at
// chunk ^ ((r / 2) % 8) = chunk ^ ((lane / 2) % 8).
template <> struct FragReader<false> {
  int off[kDmaKs];   // per KS: byte offset of this lane's fragment in block i = 0
  __device__ __forceinline__ void init(int wbase, int lane) {
    const int r = wbase + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < kDmaKs; ++ks)
      off[ks] = r * 128 + (((2 * ks + (lane >> 5)) ^ ((lane >> 1) & 7)) * 16);
  }
  template <int KS>
  __device__ __forceinline__ void read(const char* s, bf16x8 (&f)[4]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f[i] = *reinterpret_cast<const bf16x8*>(s + off[KS] + i * 32 * 128);
  }
  template <int KS, int I>
  __device__ __forceinline__ void read_blk(const char* s, bf16x8 (&f)[4]) const {
    f[I] = *reinterpret_cast<const bf16x8*>(s + off[KS] + I * 32 * 128);
  }
};

// transposed: lane l of 16-lane group g4 = l / 16 (k half h = l / 32, column
// half g = g4 % 2, j = l % 16) points at k row 16 KS + 8 h + 4 e + j / 4,
// columns wbase + 32 i + 16 g + 4 (j % 4) .. +3 (segment swizzled by
// 2 (k % 4)); the transposing read hands it (k = 16 KS + 8 h + 4 e + 0..3,
// column wbase + 32 i + l % 32).
template <> struct FragReader<true> {
  int addr[4];  // per block i: byte address for KS 0, e 0
  __device__ __forceinline__ void init(int wbase, int lane) {
    const int h = lane >> 5, g = (lane >> 4) & 1, j = lane & 15;
    const int krow = 8 * h + (j >> 2);          // + 16 KS + 4 e (same k % 4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int seg = (wbase >> 4) + 2 * i + g;  // 16 columns per 32-byte segment
      addr[i] = krow * 512 + ((seg ^ (2 * (krow & 3))) * 32) + (j & 3) * 8;
    }
  }
  template <int KS, int I>
  __device__ __forceinline__ void read_blk(const char* s, bf16x8 (&f)[4]) const {
    lds_char* p = (lds_char*)(s + addr[I] + KS * 16 * 512);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 512));
    f[I] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  template <int KS>
  __device__ __forceinline__ void read(const char* s, bf16x8 (&f)[4]) const {
    read_blk<KS, 0>(s, f);
    read_blk<KS, 1>(s, f);
    read_blk<KS, 2>(s, f);
    read_blk<KS, 3>(s, f);
  }
};

// Fragments of sub-step KS of both operands, read in the order the MFMA
// group uses them (A0 with B0..B3 first, then A1..A3).
template <int KS, bool AT, bool BT>
__device__ __forceinline__ void read_frags(const FragReader<AT>& fa, const FragReader<BT>& fb,
                                           const char* s, bf16x8 (&a)[4], bf16x8 (&b)[4]) {
  fa.template read_blk<KS, 0>(s, a);
  fb.template read_blk<KS, 0>(s + kDmaOpBytes, b);
  fb.template read_blk<KS, 1>(s + kDmaOpBytes, b);
  fb.template read_blk<KS, 2>(s + kDmaOpBytes, b);
  fb.template read_blk<KS, 3>(s + kDmaOpBytes, b);
  fa.template read_blk<KS, 1>(s, a);
  fa.template read_blk<KS, 2>(s, a);
  fa.template read_blk<KS, 3>(s, a);
}

// Scheduling pattern for a 16-MFMA group that hides the R fragment reads of
// the next group: 8 x {R/8 LDS reads, 2 MFMA} (R = 8, 12 or 16: one read per
// natural fragment, two per transposed one).
template <int R, int Q = 0>
__device__ __forceinline__ void interleave_reads_mfma() {
  if constexpr (Q < 8) {
    constexpr int n = (R * (Q + 1)) / 8 - (R * Q) / 8;
    __builtin_amdgcn_sched_group_barrier(0x100, n, 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
    interleave_reads_mfma<R, Q + 1>();
  }
}

template <bool FRESH>
__device__ __forceinline__ void mfma_group(f32x16 (&acc)[4][4], const bf16x8 (&a)[4],
                                           const bf16x8 (&b)[4]) {
  const f32x16 zero = {};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], FRESH ? zero : acc[i][j],
                                                          0, 0, 0);
}

// The last MFMA sub-step of a stage, right after the barrier that frees the
// stage's slot: eight steps of {one DMA instruction of each operand for the
// stage after next, one fragment read of the next stage's first sub-step (in
// the order its MFMAs use them: A0, B0..B3, A1..A3), the two MFMAs of blocks
// (P / 2, 2 (P % 2)) and (P / 2, 2 (P % 2) + 1)}, pinned in that order so
// that a DMA instruction that has to wait for the address unit does not hold
// back more than the MFMAs already issued.
template <int P, bool AT, bool BT, class LA, class LB>
__device__ __forceinline__ void last_substep(f32x16 (&acc)[4][4], const bf16x8 (&a)[4],
                                             const bf16x8 (&b)[4], const LA& la,
                                             const LB& lb, uint32_t la_op,
                                             uint32_t lb_op, int k0, bool more, int wave,
                                             __amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb,
                                             const FragReader<AT>& fa, const FragReader<BT>& fb,
                                             const char* sn, bf16x8 (&an)[4], bf16x8 (&bn)[4]) {
  if constexpr (P < 8) {
    la.template issue_q<P>(la_op, k0, wave, more, rsa);
    lb.template issue_q<P>(lb_op, k0, wave, more, rsb);
    // A0, B0..B3, A1..A3: the order the next sub-step's MFMAs use them
    if constexpr (P == 0) fa.template read_blk<0, 0>(sn, an);
    else if constexpr (P <= 4) fb.template read_blk<0, P - 1>(sn + kDmaOpBytes, bn);
    else fa.template read_blk<0, P - 4>(sn, an);
    constexpr int i = P / 2, j = 2 * (P % 2);
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    acc[i][j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j + 1], acc[i][j + 1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    last_substep<P + 1, AT, BT, LA, LB>(acc, a, b, la, lb, la_op, lb_op, k0, more, wave, rsa, rsb,
                                        fa, fb, sn, an, bn);
  }
}

// acc = sum over active K steps (64 wide) of A[m][k] B[n][k] for the
// 256 x 256 tile at (m0, n0); `active(s)` must agree across the workgroup.
//
// A stage (K = 64, four MFMA sub-steps ks0..ks3 of 16 MFMAs per wave) sits
// in one of two LDS slots.  While sub-step k's MFMAs run, the fragments of
// the sub-step after it are read.  Between ks2 and ks3 of a stage every wave
// waits for its own DMAs of the next stage and for its reads of this slot,
// then one barrier makes the next stage visible to all and frees this slot,
// which immediately takes the DMAs of the stage after next.  The loop body
// runs from ks1 of one stage to ks0 of the next, so the first MFMA group
// (which starts from zero instead of the accumulators) sits before the loop.
template <bool AT, bool BT, class Active, bool GATHER_A = false>
__device__ __forceinline__ void gemm_tile_dma(const Operand& A, const Operand& B, int m0, int n0,
                                              int nsteps, Active active,
                                              f32x16 (&acc)[4][4], char* lds,
                                              L2Split sa = {0, 8}, L2Split sb = {0, 4}) {
  static_assert(!GATHER_A || AT, "the gathered transposed loader is for a transposed A");
  using LoaderA = std::conditional_t<GATHER_A, DmaTransposedGather, DmaLoader<AT>>;
  active.prepare(nsteps);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int wm = wave >> 1, wn = wave & 1;

  int cur = active.next(0, nsteps);
  if (cur >= nsteps) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    __syncthreads();
    return;
  }
  int nxt = active.next(cur + 1, nsteps);

  LoaderA la;
  DmaLoader<BT> lb;
  la.init(A, m0, wave, lane);
  lb.init(B, n0, wave, lane);
  FragReader<AT> fa;
  FragReader<BT> fb;
  fa.init(wm * 128, lane);
  fb.init(wn * 128, lane);
  const uint32_t lbase = lds_addr(lds);
  auto issue = [&](int slot, int step) {
    if constexpr (GATHER_A) la.rows(step * kDmaKStep);
    la.issue(lbase + slot * kDmaStageBytes, step * kDmaKStep, wave);
    lb.issue(lbase + slot * kDmaStageBytes + kDmaOpBytes, step * kDmaKStep, wave);
  };
  // Wave 0 touches this workgroup's share of A's lines of a future step,
  // wave 1 that of B; waves 2 and 3 issue the same instruction with every
  // lane out of range (no memory access), so that every wave has the same
  // number of loads in flight and the wait counts below hold for all.
  const uint32_t ldummy = lbase + kDmaLdsBytes;
  auto prefetch = [&](int step) {
    const bool on = step < nsteps;
    if (wave == 1) lb.prefetch(ldummy, step * kDmaKStep, sb, lane, on);
    else la.prefetch(ldummy, step * kDmaKStep, sa, lane, on && wave == 0);
  };
  constexpr int kReads = 4 * (AT ? 2 : 1) + 4 * (BT ? 2 : 1);
  issue(0, cur);
  if (nxt < nsteps) {
    issue(1, nxt);
    prefetch(nxt + 1);
    prefetch(nxt + 2);
    wait_vmcnt<18>();      // the first stage (16 DMAs per wave per stage)
  } else {
    wait_vmcnt<0>();
  }
  barrier_raw();
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  read_frags<0, AT, BT>(fa, fb, lds, a0, b0);
  read_frags<1, AT, BT>(fa, fb, lds, a1, b1);
  mfma_group<true>(acc, a0, b0);
  interleave_reads_mfma<kReads>();

  int slot = 0;
  // Stages with a successor run the straight-line body; the last stage is
  // peeled so no control-flow merge sits between the next stage's fragment
  // reads and this stage's MFMAs (a merge would make the LDS wait count
  // conservative and stall on those reads).
  while (nxt < nsteps) {
    const char* s = lds + slot * kDmaStageBytes;
    read_frags<2, AT, BT>(fa, fb, s, a0, b0);
    mfma_group<false>(acc, a1, b1);
    interleave_reads_mfma<kReads>();
    read_frags<3, AT, BT>(fa, fb, s, a1, b1);
    mfma_group<false>(acc, a0, b0);
    interleave_reads_mfma<kReads>();
    const int nn = active.next(nxt + 1, nsteps);   // the stage after next
    if constexpr (GATHER_A) la.rows((nn < nsteps ? nn : 0) * kDmaKStep);
    // own DMAs of the next stage; only the latest line touch may still fly
    // (loads complete in order, so every older one has landed too)
    wait_vmcnt<1>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // own reads of this slot
    barrier_raw();
    // every wave is done with this slot: it takes the stage after next
    {
      const bool more = nn < nsteps;
      const int k0n = (more ? nn : 0) * kDmaKStep;
      const uint32_t la_op = lbase + slot * kDmaStageBytes;
      const char* sn = lds + (slot ^ 1) * kDmaStageBytes;
      last_substep<0, AT, BT, LoaderA, DmaLoader<BT>>(acc, a1, b1, la, lb, la_op,
                                                      la_op + kDmaOpBytes, k0n, more, wave,
                                                      la.rsrc(k0n), lb.rsrc(k0n), fa, fb, sn, a0,
                                                      b0);
    }
    prefetch(nn + 2);   // after the DMAs: the wait above leaves only this one in flight
    {
      const char* sn = lds + (slot ^ 1) * kDmaStageBytes;
      read_frags<1, AT, BT>(fa, fb, sn, a1, b1);
    }
    mfma_group<false>(acc, a0, b0);
    interleave_reads_mfma<kReads>();
    nxt = nn;
    slot ^= 1;
  }
  {
    const char* s = lds + slot * kDmaStageBytes;
    read_frags<2, AT, BT>(fa, fb, s, a0, b0);
    mfma_group<false>(acc, a1, b1);
    read_frags<3, AT, BT>(fa, fb, s, a1, b1);
    mfma_group<false>(acc, a0, b0);
    mfma_group<false>(acc, a1, b1);
  }
  acc_fence(acc);
  wait_vmcnt<0>();   // DMAs past the last stage (out of range: zeros) and line touches
  __syncthreads();   // LDS may be reused by the caller
}

// One MFMA sub-step after a stage's barrier: eight steps of {DMA instruction
// P of loader `ld` (the stage after next, into the slot just freed), one
// fragment read of sub-step NKS of the next stage (A0, B0..B3, A1..A3), the
// two MFMAs of blocks (P / 2, 2 (P % 2)) and (P / 2, 2 (P % 2) + 1)}.
template <int P, int NKS, bool AT, bool BT, class LD>
__device__ __forceinline__ void dma_substep(f32x16 (&acc)[4][4], const bf16x8 (&a)[4],
                                            const bf16x8 (&b)[4], const LD& ld, uint32_t ld_op,
                                            int k0, bool more, int wave,
                                            __amdgpu_buffer_rsrc_t rs, const FragReader<AT>& fa,
                                            const FragReader<BT>& fb, const char* sn,
                                            bf16x8 (&an)[4], bf16x8 (&bn)[4]) {
  if constexpr (P < 8) {
    ld.template issue_q<P>(ld_op, k0, wave, more, rs);
    if constexpr (P == 0) fa.template read_blk<NKS, 0>(sn, an);
    else if constexpr (P <= 4) fb.template read_blk<NKS, P - 1>(sn + kDmaOpBytes, bn);
    else fa.template read_blk<NKS, P - 4>(sn, an);
    constexpr int i = P / 2, j = 2 * (P % 2);
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    acc[i][j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j + 1], acc[i][j + 1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    dma_substep<P + 1, NKS, AT, BT, LD>(acc, a, b, ld, ld_op, k0, more, wave, rs, fa, fb, sn, an,
                                        bn);
  }
}

// As gemm_tile_dma, with the stage's barrier after its second sub-step: the
// fragments of all four sub-steps are read before it (four fragment sets,
// one per sub-step), so the slot is free half a stage earlier and the DMAs of
// the stage after next go out over two sub-steps (A's during the third, B's
// during the fourth: one instruction per MFMA pair) instead of one.
template <bool AT, bool BT, class Active, bool GATHER_A = false>
__device__ __forceinline__ void gemm_tile_dma2(const Operand& A, const Operand& B, int m0, int n0,
                                               int nsteps, Active active,
                                               f32x16 (&acc)[4][4], char* lds,
                                               L2Split sa = {0, 8}, L2Split sb = {0, 4}) {
  static_assert(!GATHER_A || AT, "the gathered transposed loader is for a transposed A");
  using LoaderA = std::conditional_t<GATHER_A, DmaTransposedGather, DmaLoader<AT>>;
  active.prepare(nsteps);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int cur = active.next(0, nsteps);
  if (cur >= nsteps) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    __syncthreads();
    return;
  }
  int nxt = active.next(cur + 1, nsteps);
  LoaderA la;
  DmaLoader<BT> lb;
  la.init(A, m0, wave, lane);
  lb.init(B, n0, wave, lane);
  FragReader<AT> fa;
  FragReader<BT> fb;
  fa.init(wm * 128, lane);
  fb.init(wn * 128, lane);
  const uint32_t lbase = lds_addr(lds);
  auto issue = [&](int slot, int step) {
    if constexpr (GATHER_A) la.rows(step * kDmaKStep);
    la.issue(lbase + slot * kDmaStageBytes, step * kDmaKStep, wave);
    lb.issue(lbase + slot * kDmaStageBytes + kDmaOpBytes, step * kDmaKStep, wave);
  };
  const uint32_t ldummy = lbase + kDmaLdsBytes;
  auto prefetch = [&](int step) {
    const bool on = step < nsteps;
    if (wave == 1) lb.prefetch(ldummy, step * kDmaKStep, sb, lane, on);
    else la.prefetch(ldummy, step * kDmaKStep, sa, lane, on && wave == 0);
  };
  constexpr int kReads = 4 * (AT ? 2 : 1) + 4 * (BT ? 2 : 1);
  issue(0, cur);
  if (nxt < nsteps) {
    issue(1, nxt);
    prefetch(nxt + 1);
    prefetch(nxt + 2);
    wait_vmcnt<18>();
  } else {
    wait_vmcnt<0>();
  }
  barrier_raw();
  bf16x8 a0[4], b0[4], a1[4], b1[4], a2[4], b2[4], a3[4], b3[4];
  read_frags<0, AT, BT>(fa, fb, lds, a0, b0);
  read_frags<1, AT, BT>(fa, fb, lds, a1, b1);
  int slot = 0;
  // one stage: ks0 and ks1 while ks2 / ks3 fragments load; barrier (this
  // slot is then free); ks2 and ks3 while the DMAs of the stage after next
  // fill this slot and the next stage's ks0 / ks1 fragments load
  auto body = [&](auto fresh, bool& last) {
    const char* s = lds + slot * kDmaStageBytes;
    read_frags<2, AT, BT>(fa, fb, s, a2, b2);
    mfma_group<decltype(fresh)::value>(acc, a0, b0);
    interleave_reads_mfma<kReads>();
    read_frags<3, AT, BT>(fa, fb, s, a3, b3);
    mfma_group<false>(acc, a1, b1);
    interleave_reads_mfma<kReads>();
    last = nxt >= nsteps;
    const int nn = last ? nsteps : active.next(nxt + 1, nsteps);
    if constexpr (GATHER_A) la.rows((nn < nsteps ? nn : 0) * kDmaKStep);
    wait_vmcnt<1>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_raw();
    if (last) return;
    const bool more = nn < nsteps;
    const int k0n = (more ? nn : 0) * kDmaKStep;
    const uint32_t la_op = lbase + slot * kDmaStageBytes;
    const char* sn = lds + (slot ^ 1) * kDmaStageBytes;
    dma_substep<0, 0, AT, BT, LoaderA>(acc, a2, b2, la, la_op, k0n, more, wave, la.rsrc(k0n), fa,
                                       fb, sn, a0, b0);
    dma_substep<0, 1, AT, BT, DmaLoader<BT>>(acc, a3, b3, lb, la_op + kDmaOpBytes, k0n, more, wave,
                                             lb.rsrc(k0n), fa, fb, sn, a1, b1);
    prefetch(nn + 2);
    nxt = nn;
    slot ^= 1;
  };
  bool last = false;
  body(std::true_type{}, last);
  while (!last) body(std::false_type{}, last);
  mfma_group<false>(acc, a2, b2);
  mfma_group<false>(acc, a3, b3);
  acc_fence(acc);
  wait_vmcnt<0>();
  __syncthreads();
}

// ------------------------------------------------- 128 x 256 tiles ----
// A 128 (m) x 256 (n) output tile whose A operand is transposed ([k][m], M
// contiguous) and 128 wide: the gradient contractions of a launch that only
// contracts use it when 256 x 256 tiles would fill at most half the CUs (per
// MFMA it loads 1.5 times the operand bytes, so it pays only where it puts
// idle CUs to work).  Waves 2 x 2 as in the
// 256 x 256 core, each holding 64 x 128 (acc[2][4]); the B side, the stage
// slots and the schedule are those of gemm_tile_dma2.

// The narrow A operand in LDS: [64 k rows][256 B], 32-byte segment s of row k
// at s ^ (2 (k % 4)) (the wide layout's swizzle on a half-width row).  DMA
// instruction q of wave w covers k rows 4 (4 w + q) .. +3 (1 KiB, two whole
// 128-byte lines per row); lane L -> k row 4 (4 w + q) + L / 16, LDS 16-byte
// chunk L % 16 of the row (segment (L % 16) / 2, half L % 2), global segment
// ((L % 16) / 2) ^ (2 (L / 16)).
struct DmaTransposedNarrow {
  uint32_t off[4];
  bool colok;             // this lane's 8 columns are inside the operand
  const char* base;       // element (0, m0) of the stored [k][m] matrix
  int64_t ld, kext, mrem;
  int krow0;              // k row of instruction 0: 16 w + L / 16
  __device__ __forceinline__ void init(const Operand& op, int m0, int wave, int lane) {
    base = op.base + (int64_t)m0 * 2;
    ld = op.ld;
    kext = op.kext;
    mrem = op.mext - m0;
    krow0 = 16 * wave + (lane >> 4);
    const int seg = ((lane & 15) >> 1) ^ (2 * (lane >> 4));   // k row % 4 = L / 16
    const int m = seg * 16 + (lane & 1) * 8;
    colok = (int64_t)m0 + m < op.mext;
#pragma unroll
    for (int q = 0; q < 4; ++q) off[q] = (uint32_t)(((int64_t)(krow0 + 4 * q) * op.ld + m) * 2);
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int k0) const {
    return make_rsrc(base + (int64_t)k0 * ld * 2);
  }
  template <int Q>
  __device__ __forceinline__ void issue_q(uint32_t lds_op, int k0, int wave, bool more,
                                          __amdgpu_buffer_rsrc_t rs) const {
    const bool ok = more && colok && (k0 + krow0 + 4 * Q < kext);
    dma16(lds_op + (4 * wave + Q) * 1024, ok ? off[Q] : kOob, rs);
  }
  __device__ __forceinline__ void issue(uint32_t lds_op, int k0, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = rsrc(k0);
    issue_q<0>(lds_op, k0, wave, true, rs);
    issue_q<1>(lds_op, k0, wave, true, rs);
    issue_q<2>(lds_op, k0, wave, true, rs);
    issue_q<3>(lds_op, k0, wave, true, rs);
  }
  // two 128-byte lines per k row: lane L touches line li = share * per + L % per,
  // k row li / 2, half li % 2
  __device__ __forceinline__ void prefetch(uint32_t lds_dummy, int k0, L2Split sp, int lane,
                                           bool on) const {
    const int per = 128 / sp.nshare;
    const int li = sp.share * per + (lane & (per - 1));
    const int krow = li >> 1, half = li & 1;
    const bool ok = on && k0 + krow < kext && half * 64 < mrem;
    dma4(lds_dummy, ok ? (uint32_t)((int64_t)krow * ld * 2 + half * 128) : kOob, rsrc(k0));
  }
};

// Fragments of the narrow A operand: as FragReader<true> on 256-byte rows,
// two 32-column blocks per wave (wbase = 64 wm).
struct FragReaderNarrow {
  int addr[2];
  __device__ __forceinline__ void init(int wbase, int lane) {
    const int h = lane >> 5, g = (lane >> 4) & 1, j = lane & 15;
    const int krow = 8 * h + (j >> 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int seg = (wbase >> 4) + 2 * i + g;
      addr[i] = krow * 256 + ((seg ^ (2 * (krow & 3))) * 32) + (j & 3) * 8;
    }
  }
  template <int KS, int I>
  __device__ __forceinline__ void read_blk(const char* s, bf16x8 (&f)[2]) const {
    lds_char* p = (lds_char*)(s + addr[I] + KS * 16 * 256);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 256));
    f[I] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// Fragments of sub-step KS in the order the MFMA group uses them: A0, B0..B3, A1.
template <int KS, bool BT>
__device__ __forceinline__ void read_frags_n(const FragReaderNarrow& fa, const FragReader<BT>& fb,
                                             const char* s, bf16x8 (&a)[2], bf16x8 (&b)[4]) {
  fa.template read_blk<KS, 0>(s, a);
  fb.template read_blk<KS, 0>(s + kDmaOpBytes, b);
  fb.template read_blk<KS, 1>(s + kDmaOpBytes, b);
  fb.template read_blk<KS, 2>(s + kDmaOpBytes, b);
  fb.template read_blk<KS, 3>(s + kDmaOpBytes, b);
  fa.template read_blk<KS, 1>(s, a);
}

// 4 x {R/4 LDS reads, 2 MFMA} for an 8-MFMA group.
template <int R, int Q = 0>
__device__ __forceinline__ void interleave_reads_mfma_n() {
  if constexpr (Q < 4) {
    constexpr int n = (R * (Q + 1)) / 4 - (R * Q) / 4;
    __builtin_amdgcn_sched_group_barrier(0x100, n, 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
    interleave_reads_mfma_n<R, Q + 1>();
  }
}

template <bool FRESH>
__device__ __forceinline__ void mfma_group_n(f32x16 (&acc)[2][4], const bf16x8 (&a)[2],
                                             const bf16x8 (&b)[4]) {
  const f32x16 zero = {};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], FRESH ? zero : acc[i][j],
                                                          0, 0, 0);
}

// One MFMA sub-step after a stage's barrier (four pairs of MFMAs), with the
// DMAs of the stage after next: NKS 0 issues A's four and B's first two,
// NKS 1 B's other six (one or two per pair), and the fragment reads of
// sub-step NKS of the next stage (A0 B0 | B1 | B2 | B3 A1).
template <int P, int NKS, bool BT>
__device__ __forceinline__ void dma_substep_n(f32x16 (&acc)[2][4], const bf16x8 (&a)[2],
                                              const bf16x8 (&b)[4], const DmaTransposedNarrow& la,
                                              const DmaLoader<BT>& lb, uint32_t la_op,
                                              uint32_t lb_op, int k0, bool more, int wave,
                                              __amdgpu_buffer_rsrc_t rsa,
                                              __amdgpu_buffer_rsrc_t rsb,
                                              const FragReaderNarrow& fa,
                                              const FragReader<BT>& fb, const char* sn,
                                              bf16x8 (&an)[2], bf16x8 (&bn)[4]) {
  if constexpr (P < 4) {
    if constexpr (NKS == 0) {
      la.template issue_q<P>(la_op, k0, wave, more, rsa);
      if constexpr (P < 2) lb.template issue_q<P>(lb_op, k0, wave, more, rsb);
    } else {
      lb.template issue_q<2 + P>(lb_op, k0, wave, more, rsb);
      if constexpr (P < 2) lb.template issue_q<6 + P>(lb_op, k0, wave, more, rsb);
    }
    if constexpr (P == 0) {
      fa.template read_blk<NKS, 0>(sn, an);
      fb.template read_blk<NKS, 0>(sn + kDmaOpBytes, bn);
    } else if constexpr (P < 3) {
      fb.template read_blk<NKS, P>(sn + kDmaOpBytes, bn);
    } else {
      fb.template read_blk<NKS, 3>(sn + kDmaOpBytes, bn);
      fa.template read_blk<NKS, 1>(sn, an);
    }
    constexpr int i = P / 2, j = 2 * (P % 2);
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    acc[i][j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j + 1], acc[i][j + 1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    dma_substep_n<P + 1, NKS, BT>(acc, a, b, la, lb, la_op, lb_op, k0, more, wave, rsa, rsb, fa,
                                  fb, sn, an, bn);
  }
}

// acc = sum over active K steps (64 wide) of A[m][k] B[n][k] for the
// 128 x 256 tile at (m0, n0), A transposed and 128 wide; the stage schedule
// of gemm_tile_dma2 (barrier after a stage's second sub-step, four fragment
// sets, the DMAs of the stage after next over the last two sub-steps), with
// 12 DMA instructions per wave and stage instead of 16.
template <bool BT, class Active>
__device__ __forceinline__ void gemm_tile_dma2n(const Operand& A, const Operand& B, int m0, int n0,
                                                int nsteps, Active active, f32x16 (&acc)[2][4],
                                                char* lds, L2Split sa, L2Split sb) {
  active.prepare(nsteps);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int cur = active.next(0, nsteps);
  if (cur >= nsteps) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    __syncthreads();
    return;
  }
  int nxt = active.next(cur + 1, nsteps);
  DmaTransposedNarrow la;
  DmaLoader<BT> lb;
  la.init(A, m0, wave, lane);
  lb.init(B, n0, wave, lane);
  FragReaderNarrow fa;
  FragReader<BT> fb;
  fa.init(wm * 64, lane);
  fb.init(wn * 128, lane);
  const uint32_t lbase = lds_addr(lds);
  auto issue = [&](int slot, int step) {
    la.issue(lbase + slot * kDmaStageBytes, step * kDmaKStep, wave);
    lb.issue(lbase + slot * kDmaStageBytes + kDmaOpBytes, step * kDmaKStep, wave);
  };
  const uint32_t ldummy = lbase + kDmaLdsBytes;
  auto prefetch = [&](int step) {
    const bool on = step < nsteps;
    if (wave == 1) lb.prefetch(ldummy, step * kDmaKStep, sb, lane, on);
    else la.prefetch(ldummy, step * kDmaKStep, sa, lane, on && wave == 0);
  };
  constexpr int kReads = 2 * 2 + 4 * (BT ? 2 : 1);
  issue(0, cur);
  if (nxt < nsteps) {
    issue(1, nxt);
    prefetch(nxt + 1);
    prefetch(nxt + 2);
    wait_vmcnt<14>();      // the first stage (12 DMAs per wave per stage)
  } else {
    wait_vmcnt<0>();
  }
  barrier_raw();
  bf16x8 a0[2], b0[4], a1[2], b1[4], a2[2], b2[4], a3[2], b3[4];
  read_frags_n<0, BT>(fa, fb, lds, a0, b0);
  read_frags_n<1, BT>(fa, fb, lds, a1, b1);
  int slot = 0;
  auto body = [&](auto fresh, bool& last) {
    const char* s = lds + slot * kDmaStageBytes;
    read_frags_n<2, BT>(fa, fb, s, a2, b2);
    mfma_group_n<decltype(fresh)::value>(acc, a0, b0);
    interleave_reads_mfma_n<kReads>();
    read_frags_n<3, BT>(fa, fb, s, a3, b3);
    mfma_group_n<false>(acc, a1, b1);
    interleave_reads_mfma_n<kReads>();
    last = nxt >= nsteps;
    const int nn = last ? nsteps : active.next(nxt + 1, nsteps);
    wait_vmcnt<1>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_raw();
    if (last) return;
    const bool more = nn < nsteps;
    const int k0n = (more ? nn : 0) * kDmaKStep;
    const uint32_t la_op = lbase + slot * kDmaStageBytes;
    const char* sn = lds + (slot ^ 1) * kDmaStageBytes;
    const __amdgpu_buffer_rsrc_t rsa = la.rsrc(k0n), rsb = lb.rsrc(k0n);
    dma_substep_n<0, 0, BT>(acc, a2, b2, la, lb, la_op, la_op + kDmaOpBytes, k0n, more, wave, rsa,
                            rsb, fa, fb, sn, a0, b0);
    dma_substep_n<0, 1, BT>(acc, a3, b3, la, lb, la_op, la_op + kDmaOpBytes, k0n, more, wave, rsa,
                            rsb, fa, fb, sn, a1, b1);
    prefetch(nn + 2);
    nxt = nn;
    slot ^= 1;
  };
  bool last = false;
  body(std::true_type{}, last);
  while (!last) body(std::false_type{}, last);
  mfma_group_n<false>(acc, a2, b2);
  mfma_group_n<false>(acc, a3, b3);
  acc_fence(acc);
  wait_vmcnt<0>();
  __syncthreads();
}

}  // namespace flce

#pragma clang diagnostic pop
