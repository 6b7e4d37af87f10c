// flce.hip -- C ABI, planner and launch sequence of the fused LM-head +
// cross-entropy library (declared in include/flce.h).
//
// Launch sequence of one fused call on the caller's stream:
//   target_logit_kernel  z_y of every row (one wave per row)
//   for each band of NF token rows:
//     fwd_lse_kernel     grid = ceil(V/256) x ceil(NF/256) logits tiles
//     lse_combine_kernel grid = ceil(NF/256)
//   finalize_kernel      1 block
//   bands k = 0 .. nb-1 of NS token rows x VS vocabulary rows (rows outer):
//     bwd_band_kernel    launch k: the gradient tiles of band k - 1
//                        (ceil(D/256) x ceil(NS/256) for dH^T + ceil(D/256) x
//                        ceil(VS/256) for dW^T, reading dZ buffer (k-1) % 2)
//                        and the dZ tiles of band k (ceil(VS/256) x
//                        ceil(NS/256), writing buffer k % 2); nb + 1 launches
//     (bf16 gradients: one dZ buffer, and per band a dZ launch then a
//     gradient launch; dH of the token band summed in a float stage)
//   (sorted vocabulary, before the bands: colsum_partial/final_kernel,
//    vocab_key_kernel, 4 x sort_hist/scan/scatter_kernel, invert_perm_kernel)
// dH of a token band accumulates over the vocabulary bands and dW of a
// vocabulary band over the token bands; the first contribution stores, the
// rest add, all in stream order, so the result is deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/flce.h"
#include "kernels.hpp"
#include "vocab_sort.hpp"

// Device scratch of flce_fused_fwd_bwd_noalloc (64 MiB per GPU; see
// scratch_of_current_device below for how host code reaches it).
constexpr size_t kScratchBytes = 64ull << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr uint64_t kDefaultBudget = 64ull << 20;
constexpr int kFilterBlock = 64;
constexpr int kMaxBandRows = 4096;    // NS: token rows of a backward band
constexpr int kMaxBandVocab = 8192;   // VS: the filter's K-skip masks cover K <= 8192
constexpr int kMaxBandVocabSorted = 4096;   // VS with a sorted vocabulary: LDS row table
constexpr int kCUs = 256;             // compute units of an MI355X (gfx950)
constexpr int kNarrowTile = 128;      // d width of a narrow gradient tile

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  int64_t N, D, V;
  int dtype, es;
  int Tv;              // vocabulary tiles of 256
  int NF, nbf;         // forward band rows (multiple of 256) and band count
  int NS, VS;          // backward band sizes (multiples of 256)
  int nbn, nbv;        // backward band counts
  int frows, fcols;    // flag grid of a backward band
  int fstride;         // its row stride: fcols rounded up to a multiple of 4
  int nblk;            // combine blocks (16 rows each)
  size_t big;          // bytes shared by the forward partials and the dZ buffers
  size_t dz_bytes;     // one dZ band buffer
  size_t flag_bytes;   // one flag grid
  bool compact;        // ignored rows compacted away (row map in the workspace)
  bool bf16g;          // bf16 gradients: one dZ buffer + a float dH stage
  bool sort;           // sorted vocabulary (with the filter)
  bool narrow;         // the last (gradient-only) launch runs tiles 128 wide in d
  int nsblk;           // radix-sort blocks
  size_t off_vperm, off_vinv, sort_bytes;
  int ncblk;           // compaction blocks
  size_t stage_bytes;  // the dH stage of one token band (bf16 gradients)
  size_t off_rowmap, off_cblk;
  size_t off_zy, off_bsum, off_bcnt, off_flags, off_flagsT, off_big, total;
};

int validate(const flce_desc* d) {
  if (!d) return FLCE_E_NULL;
  if (d->n_rows < 0 || d->n_rows >= (int64_t(1) << 31)) return FLCE_E_SHAPE;
  if (d->vocab < 1 || d->vocab >= (int64_t(1) << 31)) return FLCE_E_SHAPE;
  if (d->hidden < 8 || d->hidden % 8 != 0 || d->hidden >= (int64_t(1) << 20)) return FLCE_E_SHAPE;
  if (d->in_dtype != FLCE_BF16 && d->in_dtype != FLCE_F32) return FLCE_E_DTYPE;
  if (d->reduction < FLCE_MEAN || d->reduction > FLCE_NONE) return FLCE_E_UNSUPPORTED;
  constexpr uint32_t full = FLCE_FLAG_FILTER_FULL_C | FLCE_FLAG_FILTER_FULL_E;
  if (d->flags & ~uint32_t(FLCE_FLAG_PROFILE | FLCE_FLAG_COMPACT_IGNORED | FLCE_FLAG_BF16_GRADS |
                           FLCE_FLAG_SORT_VOCAB | FLCE_FLAG_WIDE_GRAD_TILES | full))
    return FLCE_E_UNSUPPORTED;
  if ((d->flags & full) == full) return FLCE_E_UNSUPPORTED;
  if ((d->flags & FLCE_FLAG_BF16_GRADS) && d->in_dtype != FLCE_BF16) return FLCE_E_UNSUPPORTED;
  if (d->flags & FLCE_FLAG_SORT_VOCAB) {
    // bf16 core only; gathered W rows and scattered dW rows use 32-bit byte offsets
    if (d->in_dtype != FLCE_BF16) return FLCE_E_UNSUPPORTED;
    if (d->vocab * d->hidden * 4 >= (int64_t(1) << 31)) return FLCE_E_UNSUPPORTED;
  }
  if (d->flags & FLCE_FLAG_COMPACT_IGNORED) {
    // bf16 core only; gathered H rows and scattered dH rows use 32-bit byte offsets
    if (d->in_dtype != FLCE_BF16) return FLCE_E_UNSUPPORTED;
    if (d->n_rows * d->hidden * 4 >= (int64_t(1) << 31)) return FLCE_E_UNSUPPORTED;
  }
  if (!(d->filter_eps >= 0.f) || !std::isfinite(d->filter_eps)) return FLCE_E_UNSUPPORTED;
  return FLCE_OK;
}

// Workspace: Header | zy [N] | block sums | block counts | flags x 2 |
// flagsT x 2 | big, where `big` holds either the forward partials of one band
// (2 x Tv x NF floats) or two backward dZ band buffers (NS x VS elements
// each; one is written while the other is contracted): the forward's
// partials are consumed before the first dZ band is written.  With bf16
// gradients the backward part of `big` is one dZ buffer and the float dH
// stage of a token band (NS x D).
size_t backward_bytes(const Plan& p) {
  return p.bf16g ? p.dz_bytes + p.stage_bytes : 2 * p.dz_bytes;
}

// Scratch of the vocabulary sort, at the start of `big` (used before the first
// dZ band): keys x 2, indices, histograms, column-sum partials, column sums.
size_t sort_scratch(const Plan& p) {
  if (!p.sort) return 0;
  const size_t V = size_t(p.V);
  return align256(V * 4) * 3 + align256(size_t(256) * p.nsblk * 4) +
         align256(size_t(flce::kColSplits) * p.D * 4) + align256(size_t(p.D) * 4);
}

// Forward band rows: as many as the backward part of `big` holds partials
// for (2 Tv floats per row), a multiple of 256, at least 256.
int forward_rows(const Plan& p, int64_t Npad) {
  const size_t dz = size_t(p.NS) * p.VS * p.es;
  const size_t bytes = p.bf16g ? dz + size_t(p.NS) * p.D * 4 : 2 * dz;
  const int64_t fit = int64_t(bytes / (size_t(8) * p.Tv)) / 256 * 256;
  return int(std::max<int64_t>(256, std::min<int64_t>(Npad, fit)));
}

size_t layout(Plan& p) {
  size_t o = 256;  // Header
  const size_t N = size_t(p.N);
  p.off_zy = o;
  o = align256(o + N * 4);
  p.off_bsum = o;
  o = align256(o + size_t(p.nblk) * 8);
  p.off_bcnt = o;
  o = align256(o + size_t(p.nblk) * 4);
  p.fstride = (p.fcols + 3) / 4 * 4;
  p.flag_bytes = align256(size_t(p.frows) * p.fstride);
  p.off_flags = o;
  o += 2 * p.flag_bytes;
  p.off_flagsT = o;
  o += 2 * p.flag_bytes;
  p.off_rowmap = o;
  p.off_cblk = o;
  if (p.compact) {
    o = align256(o + N * 4);
    p.off_cblk = o;
    o = align256(o + size_t(p.ncblk) * 4);
  }
  p.off_vperm = p.off_vinv = o;
  if (p.sort) {
    p.off_vperm = o;
    o = align256(o + size_t(p.V) * 4);
    p.off_vinv = o;
    o = align256(o + size_t(p.V) * 4);
  }
  p.off_big = o;
  p.dz_bytes = align256(size_t(p.NS) * p.VS * p.es);
  p.stage_bytes = p.bf16g ? align256(size_t(p.NS) * p.D * 4) : 0;
  p.sort_bytes = sort_scratch(p);
  p.big = std::max({backward_bytes(p), size_t(2) * p.Tv * p.NF * 4, p.sort_bytes});
  o = align256(o + p.big);
  p.total = o;
  return o;
}

// Smallest multiple of g that splits n into as few parts as parts of at
// most `cap` (a multiple of g) would.
int64_t even_split(int64_t n, int64_t cap, int64_t g = 256) {
  for (int64_t parts = cdiv(n, cap);; ++parts) {
    const int64_t sz = cdiv(cdiv(n, parts), g) * g;
    if (sz <= cap) return sz;
  }
}

int make_plan(const flce_desc* d, Plan& p) {
  const int rc = validate(d);
  if (rc) return rc;
  p.N = d->n_rows;
  p.D = d->hidden;
  p.V = d->vocab;
  p.dtype = d->in_dtype;
  p.es = d->in_dtype == FLCE_BF16 ? 2 : 4;
  p.compact = (d->flags & FLCE_FLAG_COMPACT_IGNORED) != 0;
  p.bf16g = (d->flags & FLCE_FLAG_BF16_GRADS) != 0;
  p.sort = (d->flags & FLCE_FLAG_SORT_VOCAB) != 0 && d->filter_eps > 0.f;
  p.nsblk = int(cdiv(p.V, flce::kSortTile));
  p.ncblk = int(cdiv(std::max<int64_t>(p.N, 1), flce::kCompactRows));
  p.Tv = int(cdiv(p.V, flce::kTile));
  const int64_t Npad = cdiv(std::max<int64_t>(p.N, 1), 256) * 256;
  p.nblk = int(cdiv(std::max<int64_t>(p.N, 1), flce::kCombineRows));   // one per combine block
  // The band is as large as the budget allows: every band costs a launch,
  // and the fp32 read-modify-write of dH and dW per step scales with
  // 1 / NS + 1 / VS.  For NS from its cap (its tiles fill the machine at 4096
  // rows) down by halves, VS is the widest multiple of g (below) that fits; the
  // first NS whose VS is at least NS / 2 is taken.
  const uint64_t budget = d->ws_budget_bytes ? d->ws_budget_bytes : kDefaultBudget;
  // VS granularity: 64 vocabulary rows for bf16 inputs (a band's last
  // vocabulary tile may then be partial: its dZ stores and the contractions'
  // reads stop at the band's row stride, and its flag columns past the band
  // are padding that is always dropped), so that the dZ buffers can use the
  // budget to within 64 rows -- at 8192 x 2048 x 151552 this makes the band
  // 4096 x 4032 and gives every CU one gradient tile and one dZ tile per
  // launch.  256 (whole tiles) for the filter on one product, which drops a K
  // step for 256-wide groups of 64 x 64 blocks anchored at vocabulary row 0
  // (with the filter on both products the dropped blocks are zeros and the
  // grouping changes no value), with a sorted vocabulary, and for fp32.
  const bool one_product = (d->flags & (FLCE_FLAG_FILTER_FULL_C | FLCE_FLAG_FILTER_FULL_E)) != 0;
  const bool filt = d->filter_eps > 0.f;
  const bool fine = p.dtype == FLCE_BF16 && !(filt && (one_product || p.sort));
  const int g = fine ? kFilterBlock : flce::kTile;
  const int vs_cap = int(std::min<int64_t>(p.sort ? kMaxBandVocabSorted : kMaxBandVocab,
                                           cdiv(p.V, g) * g));
  auto fits = [&](int ns, int vs) {
    p.NS = ns;
    p.VS = vs;
    p.frows = p.NS / kFilterBlock;
    p.fcols = p.VS / kFilterBlock;
    p.NF = forward_rows(p, Npad);
    return layout(p) <= budget;
  };
  int ns_best = 0, vs_best = 0;
  for (int ns = int(std::min<int64_t>(kMaxBandRows, Npad));; ns = std::max(256, ns / 2 / 256 * 256)) {
    int vs = vs_cap;
    while (vs > 256 && !fits(ns, vs)) vs -= g;
    if (fits(ns, vs) && (vs >= ns / 2 || vs == vs_cap || ns == 256)) {
      ns_best = ns;
      vs_best = vs;
      break;
    }
    if (ns == 256) break;
  }
  if (ns_best == 0) return FLCE_E_WORKSPACE;
  p.NS = ns_best;
  p.VS = vs_best;
  // Band sizes spread evenly over the fewest bands whose rounded size still
  // fits (no thin last band); never larger than what was fitted.
  p.NS = int(even_split(std::max<int64_t>(p.N, 1), p.NS));
  p.VS = int(even_split(p.V, p.VS, g));
  p.frows = p.NS / kFilterBlock;
  p.fcols = p.VS / kFilterBlock;
  p.NF = forward_rows(p, Npad);
  layout(p);
  p.nbf = int(cdiv(std::max<int64_t>(p.N, 1), p.NF));
  p.nbn = int(cdiv(std::max<int64_t>(p.N, 1), p.NS));
  p.nbv = int(cdiv(p.V, p.VS));
  // The last launch only contracts (the gradient tiles of the last band).
  // When a band's 256 x 256 gradient tiles would fill at most half the CUs
  // (small hidden sizes: 128 tiles at 4096 x 1024 x 32000), that launch runs
  // tiles 128 wide in d instead: twice the tiles, each with half the MFMA
  // work, the same K order and sums (81 instead of 108 us there on MI355X).
  // The pipelined launches keep 256 x 256: a 128-wide tile loads 3/4 of the
  // operand bytes for 1/2 of the MFMAs, and the core's speed follows the LDS
  // DMA bytes, so a narrow gradient tile beside a dZ tile ends later than a
  // wide one (125 vs 115 us per launch).  bf16 inputs with float gradients,
  // without compaction or a sorted vocabulary (their gathered loaders and
  // scattered epilogues are 256 wide).
  const int64_t wide_tiles =
      cdiv(p.D, flce::kTile) * (cdiv(p.NS, flce::kTile) + cdiv(p.VS, flce::kTile));
  p.narrow = p.dtype == FLCE_BF16 && !p.bf16g && !p.compact && !p.sort &&
             !(d->flags & FLCE_FLAG_WIDE_GRAD_TILES) && 2 * wide_tiles <= kCUs;
  return FLCE_OK;
}

// ------------------------------------------------------------ profiling ----
struct ProfRec {
  int cls;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof_pending;
int64_t g_prof_count[FLCE_K_COUNT];
double g_prof_ms[FLCE_K_COUNT];

template <class F>
int launch(int cls, bool prof, hipStream_t s, F&& f) {
  hipEvent_t a = nullptr, b = nullptr;
  if (prof) {
    if (hipEventCreate(&a) != hipSuccess) return FLCE_E_DEVICE;
    if (hipEventCreate(&b) != hipSuccess || hipEventRecord(a, s) != hipSuccess) {
      (void)hipEventDestroy(a);
      if (b) (void)hipEventDestroy(b);
      return FLCE_E_DEVICE;
    }
  }
  f();
  const hipError_t e = hipGetLastError();
  if (prof) {
    if (hipEventRecord(b, s) != hipSuccess) {
      (void)hipEventDestroy(a);
      (void)hipEventDestroy(b);
      return FLCE_E_DEVICE;
    }
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof_pending.push_back({cls, a, b});
  }
  return e == hipSuccess ? FLCE_OK : FLCE_E_LAUNCH;
}

#define FLCE_TRY(x)            \
  do {                         \
    const int _rc = (x);       \
    if (_rc != FLCE_OK) return _rc; \
  } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Ws {
  flce::Header* hdr;
  float *pm, *zy;        // pm: forward partials, aliasing the dZ band
  double* bsum;
  int* bcnt;
  uint8_t *flags[2], *flagsT[2];
  char* dz[2];    // the same buffer twice with bf16 gradients
  float* stage;  // dH stage of a token band (bf16 gradients)
  int *vperm, *vinv;   // sorted vocabulary (null otherwise)
  uint32_t *keys[2], *hist;
  int* idx;            // sort ping-pong indices (the other half is vperm)
  float *part, *hbar;
  int* rowmap;   // null without compaction
  int* cblk;
};

Ws carve(const Plan& p, void* ws) {
  char* b = static_cast<char*>(ws);
  Ws w;
  w.hdr = reinterpret_cast<flce::Header*>(b);
  w.pm = reinterpret_cast<float*>(b + p.off_big);
  w.zy = reinterpret_cast<float*>(b + p.off_zy);
  w.bsum = reinterpret_cast<double*>(b + p.off_bsum);
  w.bcnt = reinterpret_cast<int*>(b + p.off_bcnt);
  w.rowmap = p.compact ? reinterpret_cast<int*>(b + p.off_rowmap) : nullptr;
  w.cblk = reinterpret_cast<int*>(b + p.off_cblk);
  for (int k = 0; k < 2; ++k) {
    w.flags[k] = reinterpret_cast<uint8_t*>(b + p.off_flags + k * p.flag_bytes);
    w.flagsT[k] = reinterpret_cast<uint8_t*>(b + p.off_flagsT + k * p.flag_bytes);
    w.dz[k] = b + p.off_big + (p.bf16g ? 0 : k * p.dz_bytes);
  }
  w.stage = p.bf16g ? reinterpret_cast<float*>(b + p.off_big + p.dz_bytes) : nullptr;
  w.vperm = p.sort ? reinterpret_cast<int*>(b + p.off_vperm) : nullptr;
  w.vinv = p.sort ? reinterpret_cast<int*>(b + p.off_vinv) : nullptr;
  {
    char* q = b + p.off_big;
    const size_t kv = align256(size_t(p.V) * 4);
    w.keys[0] = reinterpret_cast<uint32_t*>(q);
    w.keys[1] = reinterpret_cast<uint32_t*>(q + kv);
    w.idx = reinterpret_cast<int*>(q + 2 * kv);
    w.hist = reinterpret_cast<uint32_t*>(q + 3 * kv);
    w.part = reinterpret_cast<float*>(q + 3 * kv + align256(size_t(256) * p.nsblk * 4));
    w.hbar = w.part + size_t(flce::kColSplits) * p.D;
  }
  return w;
}

// Row map of the non-ignored rows, then the ignored ones (CCE App. B: ignored
// tokens removed before any contraction); hdr->nvalid counts the former.
int run_compact(const flce_desc* d, const Plan& p, const int64_t* y, const Ws& w, bool prof,
                hipStream_t s) {
  const int N = int(p.N);
  FLCE_TRY(launch(FLCE_K_AUX, prof, s, [&] {
    flce::compact_count_kernel<<<dim3(p.ncblk), dim3(256), 0, s>>>(y, N, d->ignore_index, w.cblk);
  }));
  FLCE_TRY(launch(FLCE_K_AUX, prof, s, [&] {
    flce::compact_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(w.cblk, p.ncblk, w.hdr);
  }));
  return launch(FLCE_K_AUX, prof, s, [&] {
    flce::compact_scatter_kernel<<<dim3(p.ncblk), dim3(256), 0, s>>>(y, N, d->ignore_index, w.cblk,
                                                                    w.hdr, w.rowmap);
  });
}

template <typename T>
int run_forward(const flce_desc* d, const Plan& p, const void* H, const void* W, const int64_t* y,
                float* loss_rows, float* lse, float* loss, const Ws& w, bool prof, hipStream_t s) {
  const int N = int(p.N), D = int(p.D), V = int(p.V);
  FLCE_TRY(launch(FLCE_K_AUX, prof, s, [&] {
    flce::target_logit_kernel<T><<<dim3(int(cdiv(N, 4))), dim3(256), 0, s>>>(
        static_cast<const T*>(H), static_cast<const T*>(W), y, N, D, V, w.rowmap, w.zy);
  }));
  for (int bf = 0; bf < p.nbf; ++bf) {
    const int nb0 = bf * p.NF;
    const int ns = int(std::min<int64_t>(p.NF, p.N - nb0));
    const int TNn = int(cdiv(ns, flce::kTile));
    float* pm = w.pm;
    float* ps = w.pm + size_t(p.Tv) * ns;
    FLCE_TRY(launch(FLCE_K_FWD_LSE, prof, s, [&] {
      flce::fwd_lse_kernel<T><<<dim3(p.Tv * TNn), dim3(flce::kThreads), 0, s>>>(
          static_cast<const T*>(H), static_cast<const T*>(W), N, D, V, nb0, ns, p.Tv, TNn, pm, ps,
          w.hdr, w.rowmap);
    }));
    FLCE_TRY(launch(FLCE_K_LSE_COMBINE, prof, s, [&] {
      flce::lse_combine_kernel<<<dim3(int(cdiv(ns, flce::kCombineRows))), dim3(256), 0, s>>>(
          pm, ps, w.zy, y, N, V, p.Tv, nb0, ns, d->ignore_index, lse, loss_rows, w.bsum, w.bcnt,
          w.hdr, w.rowmap);
    }));
  }
  FLCE_TRY(launch(FLCE_K_FINALIZE, prof, s, [&] {
    flce::finalize_kernel<<<dim3(1), dim3(256), 0, s>>>(w.bsum, w.bcnt, p.nblk, d->reduction,
                                                         loss, nullptr, w.hdr);
  }));
  return FLCE_OK;
}

flce::BandArgs band_args(const Plan& p, int k) {
  const int bn = k / p.nbv, bv = k % p.nbv;
  flce::BandArgs band;
  band.nb0 = bn * p.NS;
  band.ns_cur = int(std::min<int64_t>(p.NS, p.N - band.nb0));
  band.vb0 = bv * p.VS;
  band.vs_cur = int(std::min<int64_t>(p.VS, p.V - band.vb0));
  band.ldz = p.VS;
  band.frows = p.frows;
  band.fcols = p.fcols;
  band.fstride = p.fstride;
  return band;
}

// The sorted vocabulary (CCE Sec. 4.3): key_v = W_v . sum of the kept rows
// of H, then a stable LSD radix sort by decreasing key (4 passes of 8 bits;
// indices ping-pong between the scratch and vperm, ending in vperm), then
// its inverse.
int run_sort(const flce_desc* d, const Plan& p, const void* H, const void* W, const int64_t* y,
             const Ws& w, bool prof, hipStream_t s) {
  const int N = int(p.N), D = int(p.D), V = int(p.V);
  const auto* Hb = static_cast<const uint16_t*>(H);
  FLCE_TRY(launch(FLCE_K_AUX, prof, s, [&] {
    flce::colsum_partial_kernel<<<dim3(int(cdiv(D, 256)), flce::kColSplits), dim3(256), 0, s>>>(
        Hb, y, N, D, d->ignore_index, w.part);
  }));
  FLCE_TRY(launch(FLCE_K_AUX, prof, s, [&] {
    flce::colsum_final_kernel<<<dim3(int(cdiv(D, 256))), dim3(256), 0, s>>>(w.part, D, w.hbar);
  }));
  FLCE_TRY(launch(FLCE_K_AUX, prof, s, [&] {
    flce::vocab_key_kernel<<<dim3(int(cdiv(V, 4))), dim3(256), 0, s>>>(
        static_cast<const uint16_t*>(W), w.hbar, V, D, w.keys[0]);
  }));
  const int* idx_in = nullptr;
  for (int pass = 0; pass < 4; ++pass) {
    uint32_t* kin = w.keys[pass & 1];
    uint32_t* kout = w.keys[(pass + 1) & 1];
    int* iout = (pass & 1) ? w.vperm : w.idx;
    FLCE_TRY(launch(FLCE_K_AUX, prof, s, [&] {
      flce::sort_hist_kernel<<<dim3(p.nsblk), dim3(256), 0, s>>>(kin, V, 8 * pass, p.nsblk, w.hist);
    }));
    FLCE_TRY(launch(FLCE_K_AUX, prof, s, [&] {
      flce::sort_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(w.hist, 256 * p.nsblk);
    }));
    FLCE_TRY(launch(FLCE_K_AUX, prof, s, [&] {
      flce::sort_scatter_kernel<<<dim3(p.nsblk), dim3(256), 0, s>>>(kin, idx_in, V, 8 * pass,
                                                                     p.nsblk, w.hist, kout, iout);
    }));
    idx_in = iout;
  }
  return launch(FLCE_K_AUX, prof, s, [&] {
    flce::invert_perm_kernel<<<dim3(int(cdiv(V, 256))), dim3(256), 0, s>>>(w.vperm, V, w.vinv);
  });
}

// One backward launch: grid = g_grad gradient tiles (the first g_long of the
// contraction with the longer K) + the dZ tiles of `da`.  KAHAN: bf16 dW with
// its compensation (bf16 gradients only).
template <typename T, bool BF16G, bool KAHAN = false>
void band_kernel(bool filt, bool compact, bool sort, bool narrow, dim3 grid, hipStream_t s,
                 const flce::GradArgs<T>& ga, const flce::DzArgs<T>& da, int g_long, int g_grad,
                 int h_first) {
  const dim3 block(flce::kThreads);
  if constexpr (sizeof(T) == 2 && !BF16G && !KAHAN) {
    if (narrow) {   // 128-wide gradient tiles (no compaction or sorted vocabulary)
      if (filt)
        flce::bwd_band_kernel<T, true, false, false, false, false, true><<<grid, block, 0, s>>>(
            ga, da, g_long, g_grad, h_first);
      else
        flce::bwd_band_kernel<T, false, false, false, false, false, true><<<grid, block, 0, s>>>(
            ga, da, g_long, g_grad, h_first);
      return;
    }
  }
  if constexpr (sizeof(T) == 2) {
    if (sort) {   // only with the filter
      if (compact)
        flce::bwd_band_kernel<T, true, true, BF16G, true, KAHAN><<<grid, block, 0, s>>>(
            ga, da, g_long, g_grad, h_first);
      else
        flce::bwd_band_kernel<T, true, false, BF16G, true, KAHAN><<<grid, block, 0, s>>>(
            ga, da, g_long, g_grad, h_first);
      return;
    }
    if (compact) {
      if (filt)
        flce::bwd_band_kernel<T, true, true, BF16G, false, KAHAN><<<grid, block, 0, s>>>(
            ga, da, g_long, g_grad, h_first);
      else
        flce::bwd_band_kernel<T, false, true, BF16G, false, KAHAN><<<grid, block, 0, s>>>(
            ga, da, g_long, g_grad, h_first);
      return;
    }
  }
  if constexpr (!KAHAN) {
    if (filt)
      flce::bwd_band_kernel<T, true, false, BF16G><<<grid, block, 0, s>>>(ga, da, g_long, g_grad,
                                                                          h_first);
    else
      flce::bwd_band_kernel<T, false, false, BF16G><<<grid, block, 0, s>>>(ga, da, g_long, g_grad,
                                                                           h_first);
  } else {
    if (filt)
      flce::bwd_band_kernel<T, true, false, BF16G, false, true><<<grid, block, 0, s>>>(
          ga, da, g_long, g_grad, h_first);
    else
      flce::bwd_band_kernel<T, false, false, BF16G, false, true><<<grid, block, 0, s>>>(
          ga, da, g_long, g_grad, h_first);
  }
}

// The gradient filter's K-block counters in the workspace header.
unsigned long long* kblk_counters(const Ws& w) {
  return reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(w.hdr) +
                                               offsetof(flce::Header, kblk));
}

// Bands k = 0 .. nb-1 (token-row band outer, vocabulary band inner).  Launch
// k runs the gradient tiles of band k - 1 and the dZ tiles of band k, with
// band k's dZ in buffer k % 2: the first launch only makes dZ, the last only
// contracts.  Launches on one stream run in order, so band k - 1's dZ is
// complete before its gradient tiles start, and buffer k % 2 is no longer
// read (band k - 2's gradients ran in launch k - 1) when band k writes it.
// bf16 gradients: one dZ buffer, and band k is a dZ launch followed by its
// gradient launch; dH of a token band goes through the float stage (stored at
// its first vocabulary band, added to at the middle ones, added, rounded and
// written to dH at the last), dW is rounded once per token band.
template <typename T>
int run_bands(const flce_desc* d, const Plan& p, const void* H, const void* W, const int64_t* y,
              const float* lse, const float* dloss_rows, void* dH, void* dW, const Ws& w,
              bool prof, hipStream_t s, void* dWc = nullptr) {
  const int N = int(p.N), D = int(p.D), V = int(p.V);
  const int nb = p.nbn * p.nbv;
  const bool filt = d->filter_eps > 0.f;
  // filter on one product only (CCE FullC / FullE): dZ keeps every value
  const int skip_h = (d->flags & FLCE_FLAG_FILTER_FULL_E) ? 0 : 1;
  const int skip_w = (d->flags & FLCE_FLAG_FILTER_FULL_C) ? 0 : 1;
  const int keep_dropped = skip_h && skip_w ? 0 : 1;
  if (p.sort) FLCE_TRY(run_sort(d, p, H, W, y, w, prof, s));
  if (w.rowmap)   // dH rows of ignored rows: no tile writes them
    FLCE_TRY(launch(FLCE_K_AUX, prof, s, [&] {
      flce::zero_ignored_rows_kernel<<<dim3(int(cdiv(N, 16))), dim3(256), 0, s>>>(
          w.rowmap, w.hdr, N, D * (p.bf16g ? 2 : 4), static_cast<char*>(dH));
    }));
  auto dz_args = [&](int k, int buf) {
    const flce::BandArgs band = band_args(p, k);
    const int TMv = int(cdiv(band.vs_cur, flce::kTile));
    const int TNn = int(cdiv(band.ns_cur, flce::kTile));
    return flce::DzArgs<T>{static_cast<const T*>(H), static_cast<const T*>(W), y, lse, dloss_rows,
                           w.hdr, N, D, V, d->ignore_index, d->reduction, d->filter_eps, band,
                           TMv, TNn, reinterpret_cast<T*>(w.dz[buf]), w.flags[buf],
                           w.flagsT[buf], w.rowmap, keep_dropped, w.vperm, w.vinv};
  };
  // gradient tiles of band k reading buffer `buf`; g_long, g_grad, h_first out
  auto grad_args = [&](int k, int buf, int& g_long, int& g_grad, int& h_first, bool narrow) {
    const flce::BandArgs band = band_args(p, k);
    const int Td = int(cdiv(D, narrow ? kNarrowTile : flce::kTile));   // d tiles
    const int T2n = int(cdiv(band.vs_cur, flce::kTile));
    const int T3n = int(cdiv(band.ns_cur, flce::kTile));
    const int bn = k / p.nbv, bv = k % p.nbv;
    const int h_mode = p.nbv == 1 ? 3 : (bv == 0 ? 0 : (bv == p.nbv - 1 ? 2 : 1));
    // the contraction with the longer K (dH^T: band vocabulary, dW^T: band rows) first
    h_first = band.vs_cur >= band.ns_cur ? 1 : 0;
    g_long = Td * (h_first ? T3n : T2n);
    g_grad = Td * (T3n + T2n);
    return flce::GradArgs<T>{static_cast<const T*>(H), static_cast<const T*>(W),
                             reinterpret_cast<const T*>(w.dz[buf]), w.flags[buf], w.flagsT[buf],
                             p.bf16g ? nullptr : static_cast<float*>(dH),
                             p.bf16g ? nullptr : static_cast<float*>(dW), N, D, V, band, T3n, T2n,
                             Td, bv > 0 ? 1 : 0, bn > 0 ? 1 : 0, skip_h, skip_w, w.rowmap, w.hdr,
                             p.bf16g ? static_cast<uint16_t*>(dH) : nullptr,
                             p.bf16g ? static_cast<uint16_t*>(dW) : nullptr, w.stage, h_mode,
                             static_cast<uint16_t*>(dWc), w.vperm,
                             filt ? kblk_counters(w) : nullptr};
  };
  if (p.bf16g) {
    if constexpr (sizeof(T) == 2) {
      for (int k = 0; k < nb; ++k) {
        const flce::DzArgs<T> da = dz_args(k, 0);
        FLCE_TRY(launch(FLCE_K_BWD_DZ, prof, s, [&] {
          band_kernel<T, true>(filt, p.compact, p.sort, false, dim3(da.TMv * da.TNn), s,
                               flce::GradArgs<T>{}, da, 0, 0, 1);
        }));
        int g_long = 0, g_grad = 0, h_first = 1;
        const flce::GradArgs<T> ga = grad_args(k, 0, g_long, g_grad, h_first, false);
        FLCE_TRY(launch(FLCE_K_BWD_GRAD, prof, s, [&] {
          if (dWc)
            band_kernel<T, true, true>(filt, p.compact, p.sort, false, dim3(g_grad), s, ga,
                                       flce::DzArgs<T>{}, g_long, g_grad, h_first);
          else
            band_kernel<T, true>(filt, p.compact, p.sort, false, dim3(g_grad), s, ga,
                                 flce::DzArgs<T>{},
                                 g_long, g_grad, h_first);
        }));
      }
      return FLCE_OK;
    }
    return FLCE_E_UNSUPPORTED;   // bf16 gradients need bf16 inputs (validated)
  }
  for (int k = 0; k <= nb; ++k) {
    flce::DzArgs<T> da{};
    flce::GradArgs<T> ga{};
    int g_long = 0, g_grad = 0, g_dz = 0, h_first = 1;
    if (k < nb) {
      da = dz_args(k, k & 1);
      g_dz = da.TMv * da.TNn;
    }
    const bool narrow = p.narrow && k == nb;   // the launch that only contracts
    if (k > 0) ga = grad_args(k - 1, (k - 1) & 1, g_long, g_grad, h_first, narrow);
    const int cls = k == 0 ? FLCE_K_BWD_DZ : (k == nb ? FLCE_K_BWD_GRAD : FLCE_K_BWD_BAND);
    FLCE_TRY(launch(cls, prof, s, [&] {
      band_kernel<T, false>(filt, p.compact, p.sort, narrow, dim3(g_grad + g_dz), s, ga, da,
                            g_long, g_grad, h_first);
    }));
  }
  return FLCE_OK;
}

int check_ws(const Plan& p, const void* ws, size_t ws_bytes) {
  if (!ws) return FLCE_E_NULL;
  if (!aligned(ws, 256)) return FLCE_E_ALIGN;
  if (ws_bytes < p.total) return FLCE_E_WORKSPACE;
  return FLCE_OK;
}

int check_inputs(const Plan& p, const void* H, const void* W, const int64_t* y) {
  if (!W) return FLCE_E_NULL;
  if (p.N > 0 && (!H || !y)) return FLCE_E_NULL;
  if (!aligned(W, 16) || (H && !aligned(H, 16)) || (y && !aligned(y, 8))) return FLCE_E_ALIGN;
  return FLCE_OK;
}

// dW <- 0 (float or bf16: zero bits either way)
int zero_dW(const Plan& p, void* dW, bool prof, hipStream_t s) {
  return launch(FLCE_K_AUX, prof, s, [&] {
    flce::fill_f32_kernel<<<dim3(1024), dim3(256), 0, s>>>(static_cast<float*>(dW),
                                                           p.V * p.D / (p.bf16g ? 2 : 1), 0.f);
  });
}

// Checks of a Kahan compensation buffer (bf16, dW's layout): only with bf16
// gradients.
int check_comp(const flce_desc* d, const void* dWc) {
  if (!(d->flags & FLCE_FLAG_BF16_GRADS)) return FLCE_E_UNSUPPORTED;
  if (!dWc) return FLCE_E_NULL;
  if (!aligned(dWc, 16)) return FLCE_E_ALIGN;
  return FLCE_OK;
}

// Forward then backward on the plan p for *d (argument checks, then the
// launches); shared by the caller-workspace, static-scratch and compensated
// entry points.  dWc: the bf16 compensation of dW, or null.
int fused_with_plan(const flce_desc* d, const Plan& p, const void* H, const void* W,
                    const int64_t* y, float* loss_rows, float* lse, float* loss, void* dH,
                    void* dW, void* ws, size_t ws_bytes, hipStream_t stream,
                    void* dWc = nullptr) {
  FLCE_TRY(check_inputs(p, H, W, y));
  if (p.N > 0 && (!loss_rows || !lse || !dH)) return FLCE_E_NULL;
  if (!dW) return FLCE_E_NULL;
  if (d->reduction != FLCE_NONE && !loss) return FLCE_E_NULL;
  if (!aligned(dW, 16) || (dH && !aligned(dH, 16))) return FLCE_E_ALIGN;
  FLCE_TRY(check_ws(p, ws, ws_bytes));
  const bool prof = d->flags & FLCE_FLAG_PROFILE;
  const Ws w = carve(p, ws);
  if (p.N == 0) {
    FLCE_TRY(launch(FLCE_K_AUX, prof, stream, [&] {
      flce::clear_status_kernel<<<1, 64, 0, stream>>>(w.hdr, d->reduction != FLCE_NONE ? loss : nullptr);
    }));
    if (dWc) FLCE_TRY(zero_dW(p, dWc, prof, stream));
    return zero_dW(p, dW, prof, stream);
  }
  if (p.compact) FLCE_TRY(run_compact(d, p, y, w, prof, stream));
  if (p.dtype == FLCE_BF16) {
    FLCE_TRY(run_forward<uint16_t>(d, p, H, W, y, loss_rows, lse, loss, w, prof, stream));
    return run_bands<uint16_t>(d, p, H, W, y, lse, nullptr, dH, dW, w, prof, stream, dWc);
  }
  FLCE_TRY(run_forward<float>(d, p, H, W, y, loss_rows, lse, loss, w, prof, stream));
  return run_bands<float>(d, p, H, W, y, lse, nullptr, dH, dW, w, prof, stream);
}

// Backward on the plan for *d; dWc as above.
int backward_impl(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                  const float* lse, const float* dloss, void* dH, void* dW, void* ws,
                  size_t ws_bytes, hipStream_t stream, void* dWc) {
  Plan p;
  FLCE_TRY(make_plan(d, p));
  FLCE_TRY(check_inputs(p, H, W, y));
  if (!dW || (p.N > 0 && (!dH || !lse))) return FLCE_E_NULL;
  if (!aligned(dW, 16) || (dH && !aligned(dH, 16))) return FLCE_E_ALIGN;
  FLCE_TRY(check_ws(p, ws, ws_bytes));
  const bool prof = d->flags & FLCE_FLAG_PROFILE;
  const Ws w = carve(p, ws);
  if (p.N == 0) {
    FLCE_TRY(launch(FLCE_K_AUX, prof, stream, [&] {
      flce::clear_status_kernel<<<1, 64, 0, stream>>>(w.hdr, nullptr);
    }));
    if (dWc) FLCE_TRY(zero_dW(p, dWc, prof, stream));
    return zero_dW(p, dW, prof, stream);
  }
  FLCE_TRY(launch(FLCE_K_FINALIZE, prof, stream, [&] {
    flce::bwd_prep_kernel<<<dim3(1), dim3(256), 0, stream>>>(y, int(p.N), int(p.V), d->ignore_index,
                                                             d->reduction, dloss, w.hdr);
  }));
  if (p.compact) FLCE_TRY(run_compact(d, p, y, w, prof, stream));
  const float* drows = d->reduction == FLCE_NONE ? dloss : nullptr;
  if (p.dtype == FLCE_BF16)
    return run_bands<uint16_t>(d, p, H, W, y, lse, drows, dH, dW, w, prof, stream, dWc);
  return run_bands<float>(d, p, H, W, y, lse, drows, dH, dW, w, prof, stream);
}

// ------------------------------------------------ static scratch memory ----
// The workspace of flce_fused_fwd_bwd_noalloc: a device array of the library
// itself, one copy per GPU, held until the process ends.  Host code never
// uses the array's name as an address (on the host it is a stand-in, not the
// device copy): the device address is looked up once per device with that
// device current and kept in g_scratch_ptr.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FLCE_E_DEVICE;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return FLCE_E_DEVICE;
    if (!aligned(p, 256)) return FLCE_E_ALIGN;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLCE_OK;
}

}  // namespace

extern "C" {

size_t flce_workspace_bytes(const flce_desc* d) {
  Plan p;
  if (make_plan(d, p) != FLCE_OK) return 0;
  return p.total;
}

int flce_plan(const flce_desc* d, flce_plan_info* out) {
  if (!out) return FLCE_E_NULL;
  Plan p;
  FLCE_TRY(make_plan(d, p));
  out->ws_bytes = int64_t(p.total);
  out->band_rows = p.NS;
  out->band_vocab = p.VS;
  out->n_bands_rows = p.nbn;
  out->n_bands_vocab = p.nbv;
  out->fwd_band_rows = p.NF;
  out->fwd_workgroups = p.Tv * int(cdiv(std::min<int64_t>(p.NF, std::max<int64_t>(p.N, 1)), 256));
  out->tile = flce::kTile;
  out->filter_block = kFilterBlock;
  out->dz_bytes = int64_t(p.NS) * p.VS * p.es;   // one dZ buffer
  out->vocab_order_offset = p.sort ? int64_t(p.off_vperm) : -1;
  out->grad_tile_d = p.narrow ? kNarrowTile : flce::kTile;
  out->reserved = 0;
  return FLCE_OK;
}

int flce_forward(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                 float* loss_rows, float* lse, float* loss, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  Plan p;
  FLCE_TRY(make_plan(d, p));
  FLCE_TRY(check_inputs(p, H, W, y));
  if (p.N > 0 && (!loss_rows || !lse)) return FLCE_E_NULL;
  if (d->reduction != FLCE_NONE && !loss) return FLCE_E_NULL;
  FLCE_TRY(check_ws(p, ws, ws_bytes));
  const bool prof = d->flags & FLCE_FLAG_PROFILE;
  const Ws w = carve(p, ws);
  if (p.N == 0) {
    return launch(FLCE_K_AUX, prof, stream, [&] {
      flce::clear_status_kernel<<<1, 64, 0, stream>>>(w.hdr, d->reduction != FLCE_NONE ? loss : nullptr);
    });
  }
  if (p.compact) FLCE_TRY(run_compact(d, p, y, w, prof, stream));
  if (p.dtype == FLCE_BF16)
    return run_forward<uint16_t>(d, p, H, W, y, loss_rows, lse, loss, w, prof, stream);
  return run_forward<float>(d, p, H, W, y, loss_rows, lse, loss, w, prof, stream);
}

int flce_backward(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                  const float* lse, const float* dloss, void* dH, void* dW, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
  return backward_impl(d, H, W, y, lse, dloss, dH, dW, ws, ws_bytes, stream, nullptr);
}

int flce_backward_kahan(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                        const float* lse, const float* dloss, void* dH, void* dW, void* dW_comp,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  FLCE_TRY(validate(d));
  FLCE_TRY(check_comp(d, dW_comp));
  return backward_impl(d, H, W, y, lse, dloss, dH, dW, ws, ws_bytes, stream, dW_comp);
}

int flce_fused_fwd_bwd(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                       float* loss_rows, float* lse, float* loss, void* dH, void* dW, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  Plan p;
  FLCE_TRY(make_plan(d, p));
  return fused_with_plan(d, p, H, W, y, loss_rows, lse, loss, dH, dW, ws, ws_bytes, stream);
}

int flce_fused_fwd_bwd_kahan(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                             float* loss_rows, float* lse, float* loss, void* dH, void* dW,
                             void* dW_comp, void* ws, size_t ws_bytes, hipStream_t stream) {
  Plan p;
  FLCE_TRY(make_plan(d, p));
  FLCE_TRY(check_comp(d, dW_comp));
  return fused_with_plan(d, p, H, W, y, loss_rows, lse, loss, dH, dW, ws, ws_bytes, stream,
                         dW_comp);
}

int flce_fused_fwd_bwd_noalloc(const flce_desc* d, const void* H, const void* W,
                               const int64_t* y, float* loss_rows, float* lse, float* loss,
                               void* dH, void* dW, hipStream_t stream) {
  FLCE_TRY(validate(d));
  // profiling creates HIP events: not for callers that cannot allocate
  if (d->flags & FLCE_FLAG_PROFILE) return FLCE_E_UNSUPPORTED;
  // the plan the caller's budget gives, held to the static scratch array
  flce_desc dd = *d;
  const uint64_t budget = d->ws_budget_bytes ? d->ws_budget_bytes : kDefaultBudget;
  dd.ws_budget_bytes = std::min<uint64_t>(budget, kScratchBytes);
  Plan p;
  FLCE_TRY(make_plan(&dd, p));
  if (p.total > kScratchBytes) return FLCE_E_WORKSPACE;
  void* ws = nullptr;
  FLCE_TRY(scratch_of_current_device(&ws));
  return fused_with_plan(&dd, p, H, W, y, loss_rows, lse, loss, dH, dW, ws, kScratchBytes, stream);
}

int flce_scale_gradients(const flce_desc* d, const float* dloss, void* dH, void* dW,
                         hipStream_t stream) {
  // only the descriptor's arguments are checked: the scaling needs no
  // workspace, so no band plan is made
  FLCE_TRY(validate(d));
  if (d->reduction == FLCE_NONE) return FLCE_E_UNSUPPORTED;
  const int64_t N = d->n_rows, D = d->hidden, V = d->vocab;
  const bool bf16g = (d->flags & FLCE_FLAG_BF16_GRADS) != 0;
  if (!dW || (N > 0 && !dH)) return FLCE_E_NULL;
  if (!aligned(dW, 16) || (dH && !aligned(dH, 16)) || (dloss && !aligned(dloss, 4)))
    return FLCE_E_ALIGN;
  if (!dloss) return FLCE_OK;   // an upstream gradient of 1
  const bool prof = d->flags & FLCE_FLAG_PROFILE;
  auto scale = [&](void* g, int64_t n) {
    return launch(FLCE_K_AUX, prof, stream, [&] {
      if (bf16g)
        flce::scale_bf16_kernel<<<dim3(2048), dim3(256), 0, stream>>>(static_cast<uint16_t*>(g), n,
                                                                      dloss);
      else
        flce::scale_f32_kernel<<<dim3(2048), dim3(256), 0, stream>>>(static_cast<float*>(g), n,
                                                                     dloss);
    });
  };
  if (N > 0) FLCE_TRY(scale(dH, N * D));
  return scale(dW, V * D);
}

int flce_filter_stats(const void* ws, hipStream_t stream, int64_t* active, int64_t* total) {
  if (!ws || !active || !total) return FLCE_E_NULL;
  if (hipStreamSynchronize(stream) != hipSuccess) return FLCE_E_DEVICE;
  unsigned long long v[2] = {0, 0};
  if (hipMemcpy(v, static_cast<const char*>(ws) + offsetof(flce::Header, kblk), sizeof(v),
                hipMemcpyDeviceToHost) != hipSuccess)
    return FLCE_E_DEVICE;
  *active = int64_t(v[0]);
  *total = int64_t(v[1]);
  return FLCE_OK;
}

int flce_device_status(const void* ws, hipStream_t stream, int32_t* out) {
  if (!ws || !out) return FLCE_E_NULL;
  if (hipStreamSynchronize(stream) != hipSuccess) return FLCE_E_DEVICE;
  int32_t v = 0;
  if (hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return FLCE_E_DEVICE;
  *out = v;
  return FLCE_OK;
}

const char* flce_strerror(int code) {
  switch (code) {
    case FLCE_OK: return "ok";
    case FLCE_E_NULL: return "a required pointer is NULL";
    case FLCE_E_SHAPE: return "invalid shape (need N >= 0, V >= 1, D >= 8, D % 8 == 0)";
    case FLCE_E_DTYPE: return "unsupported element type";
    case FLCE_E_ALIGN: return "misaligned pointer (tensors 16 B, workspace 256 B)";
    case FLCE_E_WORKSPACE: return "workspace too small for this problem";
    case FLCE_E_UNSUPPORTED: return "unsupported reduction, flag or filter threshold";
    case FLCE_E_LAUNCH: return "kernel launch failed";
    case FLCE_E_DEVICE: return "HIP runtime call failed";
    default: return "unknown error code";
  }
}

int flce_profile_reset(void) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (auto& r : g_prof_pending) {
    (void)hipEventSynchronize(r.b);
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof_pending.clear();
  for (int k = 0; k < FLCE_K_COUNT; ++k) {
    g_prof_count[k] = 0;
    g_prof_ms[k] = 0.0;
  }
  return FLCE_OK;
}

int flce_profile_read(int kernel_class, int64_t* launches, double* total_ms) {
  if (kernel_class < 0 || kernel_class >= FLCE_K_COUNT) return FLCE_E_UNSUPPORTED;
  if (!launches || !total_ms) return FLCE_E_NULL;
  std::lock_guard<std::mutex> g(g_prof_mu);
  // records are consumed in order; on an error the ones not yet read stay
  // pending (and are read or released by a later call)
  size_t done = 0;
  int rc = FLCE_OK;
  for (; done < g_prof_pending.size(); ++done) {
    const ProfRec& r = g_prof_pending[done];
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      rc = FLCE_E_DEVICE;
      break;
    }
    g_prof_count[r.cls] += 1;
    g_prof_ms[r.cls] += ms;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof_pending.erase(g_prof_pending.begin(), g_prof_pending.begin() + done);
  if (rc != FLCE_OK) return rc;
  *launches = g_prof_count[kernel_class];
  *total_ms = g_prof_ms[kernel_class];
  return FLCE_OK;
}

const char* flce_version(void) { return "flce 0.1.0 gfx950"; }

}  // extern "C"
