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
//  * 4 LDS stages of 32 K values each (32 KiB per stage, 128 KiB total),
//    loaded 3 stages ahead; completion is tracked with explicit vmcnt waits.
//  * Natural operands ([m][k], K contiguous) sit in LDS as [256 rows][64 B]:
//    16-byte chunk c of row r at chunk c ^ ((r >> 1) & 3).  An MFMA fragment
//    (8 K values of one row per lane) is one ds_read_b128.
//  * Transposed operands ([k][m], M contiguous) sit in LDS as
//    [32 k rows][512 B]: 32-byte segment s of row k at segment s ^ (k & 3).
//    A fragment is two ds_read_b64_tr_b16: within each 16-lane group the
//    hardware hands lane i the element (row kbase + e, column mbase + i),
//    e = 0..3, when source lane j points at row kbase + j / 4, columns
//    mbase + 4 (j % 4) .. +3 (measured lane layout of the instruction).
//  * One barrier per stage, in the middle: the next stage's first fragments
//    load while the current stage's second half of MFMAs runs.
//
// The DMA instructions are inline assembly so that the compiler does not
// wait for every outstanding DMA before each LDS read; the code below waits
// exactly for the stage it is about to read.
#pragma once

#include "tile_mma.hpp"

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

namespace flce {

constexpr int kDmaStages = 4;
constexpr int kDmaKStep = 32;                    // bf16 K values per stage
constexpr int kDmaOpBytes = 256 * 64;            // one operand of one stage: 16 KiB
constexpr int kDmaStageBytes = 2 * kDmaOpBytes;  // A + B
constexpr int kDmaLdsBytes = kDmaStages * kDmaStageBytes;

typedef short s16x4 __attribute__((ext_vector_type(4)));
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

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void barrier_raw() { asm volatile("s_barrier" ::: "memory"); }

// ------------------------------------------------------------- loaders ----
// Each wave issues 4 DMA instructions per operand per stage (16 per
// workgroup = 16 KiB).  Offsets are fixed per lane; the descriptor base moves
// along K.  Rows/columns outside the operand get an out-of-range offset, so
// the hardware writes zeros into their LDS slots.

// natural [m][k]: instruction q of wave w covers tile rows 16 (4 w + q) .. +15;
// lane L -> row 16 (4 w + q) + L / 4, LDS chunk L % 4, global chunk
// (L % 4) ^ ((row >> 1) & 3).
struct DmaNatural {
  uint32_t off[4];
  bool rowok[4];
  int kc;                 // K element offset of this lane's chunk
  const char* base;       // element (m0, 0)
  int64_t kext;
  __device__ __forceinline__ void init(const Operand& op, int m0, int wave, int lane) {
    base = op.base + (int64_t)m0 * op.ld * 2;
    kext = op.kext;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 16 * (4 * wave + q) + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 1) & 3);
      if (q == 0) kc = c * 8;
      rowok[q] = (int64_t)m0 + row < op.mext;
      off[q] = (uint32_t)(((int64_t)row * op.ld + c * 8) * 2);
    }
  }
  // chunk index depends on the row only through (row >> 1) & 3, which is the
  // same for all q (row differs by multiples of 16) -> one kc for all q.
  __device__ __forceinline__ void issue(uint32_t lds_op, int k0, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)k0 * 2);
    const bool kin = k0 + kc < kext;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dma16(lds_op + (4 * wave + q) * 1024, (kin && rowok[q]) ? off[q] : kOob, rs);
  }
};

// transposed [k][m]: instruction q of wave w covers k rows 2 (4 w + q), +1;
// lane L -> k row 2 (4 w + q) + L / 32, LDS segment (L % 32) / 2, half L % 2,
// global segment ((L % 32) / 2) ^ (krow & 3).
struct DmaTransposed {
  uint32_t off[4];
  bool colok[4];
  const char* base;       // element (0, m0) of the stored [k][m] matrix
  int64_t ld, kext;
  int krow0;              // k row of instruction 0 for this lane
  __device__ __forceinline__ void init(const Operand& op, int m0, int wave, int lane) {
    base = op.base + (int64_t)m0 * 2;
    ld = op.ld;
    kext = op.kext;
    krow0 = 8 * wave + (lane >> 5);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int krow = krow0 + 2 * q;
      const int seg = ((lane & 31) >> 1) ^ (krow & 3);
      const int m = seg * 16 + (lane & 1) * 8;
      colok[q] = (int64_t)m0 + m < op.mext;
      off[q] = (uint32_t)(((int64_t)krow * op.ld + m) * 2);
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds_op, int k0, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)k0 * ld * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = colok[q] && (k0 + krow0 + 2 * q < kext);
      dma16(lds_op + (4 * wave + q) * 1024, ok ? off[q] : kOob, rs);
    }
  }
};

template <bool TRANS> struct DmaLoader;
template <> struct DmaLoader<false> : DmaNatural {};
template <> struct DmaLoader<true> : DmaTransposed {};

// ----------------------------------------------------------- fragments ----
// Fragments of MFMA K sub-step ks (0 or 1) of a stage for the wave's 4 blocks.
template <bool TRANS> struct FragReader;

template <> struct FragReader<false> {
  int off[2];   // per ks: byte offset of this lane's chunk in its row
  int row0;     // byte offset of row (wbase + lane % 32)
  __device__ __forceinline__ void init(int wbase, int lane) {
    const int r = wbase + (lane & 31);
    row0 = r * 64;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) off[ks] = ((2 * ks + (lane >> 5)) ^ ((r >> 1) & 3)) * 16;
  }
  template <int KS>
  __device__ __forceinline__ void read(const char* s, bf16x8 (&f)[4]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f[i] = *reinterpret_cast<const bf16x8*>(s + row0 + i * 32 * 64 + off[KS]);
  }
};

template <> struct FragReader<true> {
  int addr[2];  // per (i & 1): byte address of this lane's 8 bytes for ks 0, e 0, i 0/1
  __device__ __forceinline__ void init(int wbase, int lane) {
    const int h = lane >> 5, g = (lane >> 4) & 1, j = lane & 15;
    const int krow = 8 * h + (j >> 2);          // + 16 ks + 4 e
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int seg = (wbase >> 4) + 2 * ii + g;  // 16 m values per 32-byte segment
      addr[ii] = krow * 512 + ((seg ^ (krow & 3)) * 32) + (j & 3) * 8;
    }
  }
  template <int KS>
  __device__ __forceinline__ void read(const char* s, bf16x8 (&f)[4]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // blocks i and i + 2 differ by 4 segments (128 bytes): an immediate
      lds_char* p = (lds_char*)(s + addr[i & 1] + (i >> 1) * 128 + KS * 16 * 512);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 512));
      f[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
};

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

template <int KS>
__device__ __forceinline__ void mfma_ks(f32x16 (&acc)[4][4], const bf16x8 (&a)[4],
                                        const bf16x8 (&b)[4], bool fresh) {
  const f32x16 zero = {};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j],
                                                          (KS == 0 && fresh) ? zero : acc[i][j], 0, 0, 0);
}

// acc = sum over active K steps (32 wide) of A[m][k] B[n][k] for the
// 256 x 256 tile at (m0, n0); `active(s)` must agree across the workgroup.
template <bool AT, bool BT, class Active>
__device__ __forceinline__ void gemm_tile_dma(const Operand& A, const Operand& B, int m0, int n0,
                                              int nsteps, Active active,
                                              f32x16 (&acc)[4][4], char* lds) {
  active.prepare(nsteps);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto next_active = [&](int s) { return active.next(s, nsteps); };
  int st[4];                         // the next 4 active steps (nsteps = none)
  st[0] = next_active(0);
  if (st[0] >= nsteps) {
    __syncthreads();
    return;
  }
  st[1] = next_active(st[0] + 1);
  st[2] = next_active(st[1] + 1);
  st[3] = next_active(st[2] + 1);

  DmaLoader<AT> la;
  DmaLoader<BT> lb;
  la.init(A, m0, wave, lane);
  lb.init(B, n0, wave, lane);
  FragReader<AT> fa;
  FragReader<BT> fb;
  fa.init(wm * 128, lane);
  fb.init(wn * 128, lane);
  const uint32_t lbase = lds_addr(lds);
  auto issue = [&](int slot, int step) {
    la.issue(lbase + slot * kDmaStageBytes, step * kDmaKStep, wave);
    lb.issue(lbase + slot * kDmaStageBytes + kDmaOpBytes, step * kDmaKStep, wave);
  };
  // prologue: up to 3 stages in flight
  issue(0, st[0]);
  if (st[1] < nsteps) issue(1, st[1]);
  if (st[2] < nsteps) issue(2, st[2]);
  // stage 0 landed (allow the 16 DMAs of stages 1, 2 to fly)
  if (st[2] < nsteps) wait_vmcnt<16>();
  else if (st[1] < nsteps) wait_vmcnt<8>();
  else wait_vmcnt<0>();
  barrier_raw();
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  fa.template read<0>(lds, a0);
  fb.template read<0>(lds + kDmaOpBytes, b0);

  constexpr int kReads = 4 * (AT ? 2 : 1) + 4 * (BT ? 2 : 1);
  bool fresh = true;
  int slot = 0;
  // Steps with a successor run the straight-line body; the last step is
  // peeled so no control-flow merge sits between the next stage's fragment
  // reads and this stage's second MFMA group (a merge would make the LDS
  // wait count conservative and stall on those reads).
  while (st[1] < nsteps) {
    const char* s = lds + slot * kDmaStageBytes;
    fa.template read<1>(s, a1);
    fb.template read<1>(s + kDmaOpBytes, b1);
    mfma_ks<0>(acc, a0, b0, fresh);
    interleave_reads_mfma<kReads>();
    fresh = false;
    // the next stage landed: its DMAs were issued before those of the (up
    // to) one stage behind it
    if (st[2] < nsteps) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    barrier_raw();
    // every wave is past stage slot-1: its buffer takes the step 3 ahead
    if (st[3] < nsteps) issue((slot + 3) & 3, st[3]);
    const char* sn = lds + ((slot + 1) & 3) * kDmaStageBytes;
    fa.template read<0>(sn, a0);
    fb.template read<0>(sn + kDmaOpBytes, b0);
    mfma_ks<1>(acc, a1, b1, false);
    interleave_reads_mfma<kReads>();
    st[1] = st[2];
    st[2] = st[3];
    st[3] = st[3] < nsteps ? next_active(st[3] + 1) : nsteps;
    slot = (slot + 1) & 3;
  }
  {
    const char* s = lds + slot * kDmaStageBytes;
    fa.template read<1>(s, a1);
    fb.template read<1>(s + kDmaOpBytes, b1);
    mfma_ks<0>(acc, a0, b0, fresh);
    mfma_ks<1>(acc, a1, b1, false);
  }
  acc_fence(acc);
  __syncthreads();   // LDS may be reused by the caller
}

}  // namespace flce

#pragma clang diagnostic pop
