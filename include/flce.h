/*
 * flce.h -- C ABI of the fused LM-head projection + cross-entropy library
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (for H [N,D], W [V,D], targets y [N]):
 *   Z      = H W^T                      (never stored in device memory)
 *   lse_n  = log sum_v exp(Z_nv)
 *   loss_n = lse_n - Z_{n, y_n}         (0 on rows with y_n == ignore_index)
 *   dZ     = g_n (softmax(Z)_n - onehot(y_n))
 *   dH     = dZ W,   dW = dZ^T H
 * Definitions: Trillion Labs "Fused Linear Cross-Entropy" reading notes,
 * section "Cross Entropy를 다시 보면" (loss and dL/dz = softmax - onehot);
 * PyTorch 2.13 LinearCrossEntropyLoss chapter, section "먼저 수식에서 없앨 수
 * 있는 tensor를 찾는다" (dZ, dH = dZ W, dW = dZ^T H); Cut Cross-Entropy
 * (arXiv 2411.09009) Sec. 4, Eq. 4 (indexed matmul minus linear-log-sum-exp)
 * and Algorithm 4 (merged backward with the optional gradient filter).
 * ignore_index and the mean over non-ignored rows clamped to >= 1 follow the
 * notes' section "1. Chunked Cross-Entropy".
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates device memory: the only scratch is the caller's
 *     workspace `ws` of at least flce_workspace_bytes() bytes (256-byte
 *     aligned).  Extra device memory of a call is therefore exactly ws_bytes.
 *   - Layouts are row-major and contiguous: H [N,D], W [V,D], dH [N,D],
 *     dW [V,D]; y is int64 [N]; loss_rows, lse are float [N]; loss is float [1].
 *     H and W share one element type (desc->in_dtype); gradients dH, dW are
 *     float, or bf16 under FLCE_FLAG_BF16_GRADS.  H, W, dH, dW must be
 *     16-byte aligned.
 *   - Work is enqueued on `stream` (0 = the null stream) and runs
 *     asynchronously; no entry point synchronises except
 *     flce_device_status() and flce_filter_stats().  Outputs are overwritten, never accumulated.
 *   - Argument errors are reported synchronously by the return code, before
 *     anything is enqueued; outputs are then untouched.
 *   - A target outside [0, V) that is not ignore_index is detected on the
 *     device: its row's loss_rows entry becomes NaN, its dZ row becomes NaN
 *     (so dH/dW carry NaN) and bit 0 of the workspace status word is set.
 *     Every entry point clears the status word when it starts.
 *   - Results are deterministic: no floating-point atomics, fixed reduction
 *     orders; two calls with the same inputs give the same bits.
 *   - The library keeps no state between calls other than the profiling
 *     record (guarded by a mutex), so calls from several host threads are
 *     safe; two calls whose work overlaps on the device must not share a
 *     workspace (the workspace carries each call's intermediate data).
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

/* Return codes. */
enum {
  FLCE_OK = 0,
  FLCE_E_NULL = 1,        /* a required pointer is NULL                      */
  FLCE_E_SHAPE = 2,       /* N < 0, V < 1, D < 8, D % 8 != 0 or a size too big */
  FLCE_E_DTYPE = 3,       /* in_dtype is not FLCE_BF16 / FLCE_F32              */
  FLCE_E_ALIGN = 4,       /* pointer misaligned (16 B tensors, 256 B ws)       */
  FLCE_E_WORKSPACE = 5,   /* ws_bytes < flce_workspace_bytes(), or the budget
                             cannot hold the smallest plan                     */
  FLCE_E_UNSUPPORTED = 6, /* reduction/flags value not supported               */
  FLCE_E_LAUNCH = 7,      /* a kernel launch failed (HIP error)                */
  FLCE_E_DEVICE = 8       /* a HIP runtime call other than a launch failed     */
};

enum { FLCE_BF16 = 0, FLCE_F32 = 1 };             /* element type of H and W   */
enum { FLCE_MEAN = 0, FLCE_SUM = 1, FLCE_NONE = 2 }; /* loss reduction           */

/* Bits of flce_desc.flags. */
enum {
  FLCE_FLAG_PROFILE = 1u,          /* record HIP events around every launch (see
                                      flce_profile_read); costs a little time  */
  FLCE_FLAG_COMPACT_IGNORED = 2u,  /* remove the rows whose target is ignore_index
                                      before every contraction (CCE App. B):
                                      the tiles cover only the other rows.  Their
                                      loss_rows entry, dH row and dW contribution
                                      are 0 as without the flag, but their lse
                                      entry is 0 (not computed).  bf16 inputs
                                      only, and N * D * 4 < 2^31; otherwise
                                      FLCE_E_UNSUPPORTED.  Adds N int32 and
                                      ceil(N/1024) int32 to the workspace.    */
  FLCE_FLAG_BF16_GRADS = 4u,       /* dH and dW are bf16 (the parameters' type)
                                      instead of float: the gradient type a
                                      bf16 training loop keeps (CCE Sec. 5.1 with
                                      Table 1 rows 8-10 sums gradients in the
                                      final type, Kahan optional;
                                      p2 section "precision policy는 속도 옵션이
                                      아니라 gradient 계약이다" makes the
                                      accumulator a choice).  bf16 inputs only,
                                      else FLCE_E_UNSUPPORTED.  Accumulation:
                                      dH of a token band is summed over the
                                      vocabulary bands in a float stage in the
                                      workspace (NS x D floats) and rounded to
                                      bf16 once; dW of a vocabulary band is
                                      rounded once per token band
                                      (n_bands_rows roundings to nearest even).
                                      The backward then stages one dZ band and
                                      runs each band as a dZ launch followed by
                                      a gradient launch.                     */
  FLCE_FLAG_FILTER_FULL_C = 8u,    /* with filter_eps > 0: dW (the classifier's
                                      gradient, CCE's C) is exact and only dH
                                      is filtered ("FullC", CCE Sec. 5.1 and
                                      Table 1 row 9).  The dZ band then keeps
                                      the dropped blocks' values and dH skips
                                      a 64-wide vocabulary step when the 256
                                      token rows of its tile are all dropped
                                      there: dH's filter block is 256 x 64
                                      (rows x vocabulary, anchored at 0).    */
  FLCE_FLAG_FILTER_FULL_E = 16u,   /* with filter_eps > 0: dH (the embeddings'
                                      gradient, CCE's E) is exact and only dW
                                      is filtered ("FullE", Table 1 row 10),
                                      with a 64 x 256 filter block.  Setting
                                      both FULL flags is FLCE_E_UNSUPPORTED. */
  FLCE_FLAG_SORT_VOCAB = 32u,      /* with filter_eps > 0: the filter's
                                      vocabulary blocks are taken over the
                                      vocabulary ordered by decreasing average
                                      logit over the non-ignored rows (ties by
                                      increasing index) instead of the natural
                                      order (CCE Sec. 4.3, "Vocabulary
                                      sorting").  The backward first computes
                                      the order (sum of the kept rows of H,
                                      one product with W, a stable radix
                                      sort); its bands then hold sorted
                                      positions.  bf16 inputs and V * D * 4 <
                                      2^31 only, else FLCE_E_UNSUPPORTED; the
                                      bands' vocabulary width is capped at
                                      4096.  Adds 2 V int32 to the workspace
                                      (the order, at
                                      flce_plan_info.vocab_order_offset, and
                                      its inverse).  No effect without the
                                      filter.                                */
  FLCE_FLAG_WIDE_GRAD_TILES = 64u  /* keep every gradient contraction on
                                      256 x 256 output tiles.  By default the
                                      backward's last launch, which only
                                      contracts, runs tiles 128 wide in d
                                      when the band's 256 x 256 tiles would
                                      fill at most half the CUs (small hidden
                                      sizes; bf16 inputs with float gradients,
                                      no compaction or sorted vocabulary;
                                      flce_plan_info.grad_tile_d): the same
                                      sums in the same order, so the results
                                      are identical bit for bit; the flag
                                      exists for comparison runs.  The
                                      library's own option, not the pages'.  */
};

typedef struct flce_desc {
  int64_t n_rows;          /* N >= 0 token rows                                */
  int64_t hidden;          /* D >= 8, D % 8 == 0, D < 2^20                     */
  int64_t vocab;           /* V >= 1, V < 2^31                                 */
  int32_t in_dtype;        /* FLCE_BF16 or FLCE_F32                            */
  int32_t reduction;       /* FLCE_MEAN, FLCE_SUM or FLCE_NONE                 */
  int64_t ignore_index;    /* rows with this target are ignored (-100 usual)   */
  float filter_eps;        /* 0 = gradient filter off; CCE Sec. 4.3 uses 2^-12.
                              A 64x64 (rows x vocab) block of softmax - onehot
                              whose every entry (non-ignored rows) has
                              |.| < filter_eps is dropped from dH and dW.       */
  uint32_t flags;          /* FLCE_FLAG_* bits, others must be 0               */
  uint64_t ws_budget_bytes;/* 0 = 64 MiB; the planner sizes its backward
                              blocks to fit                                    */
} flce_desc;

/* Planner decisions (for reporting and host tests; no device work). */
typedef struct flce_plan_info {
  int64_t ws_bytes;        /* == flce_workspace_bytes()                        */
  int32_t band_rows;       /* NS: token rows per backward band                 */
  int32_t band_vocab;      /* VS: vocabulary rows per backward band            */
  int32_t n_bands_rows;    /* ceil(N / NS)                                     */
  int32_t n_bands_vocab;   /* ceil(V / VS)                                     */
  int32_t fwd_band_rows;   /* NF: token rows per forward band                  */
  int32_t fwd_workgroups;  /* forward grid of one band (256 x 256 logits tiles) */
  int32_t tile;            /* output tile edge of every contraction (256; the
                              gradient tiles' d width is grad_tile_d)         */
  int32_t filter_block;    /* edge of a filter block (64)                      */
  int64_t dz_bytes;        /* bytes of one staged dZ band buffer (two of them,
                              or one with FLCE_FLAG_BF16_GRADS)                */
  int64_t vocab_order_offset; /* FLCE_FLAG_SORT_VOCAB with the filter: byte
                              offset in ws of the int32 [V] sorted vocabulary
                              (position -> vocabulary row) a backward leaves
                              there; else -1                                 */
  int32_t grad_tile_d;     /* d width of the gradient tiles of the last
                              backward launch: 256, or 128 (see
                              FLCE_FLAG_WIDE_GRAD_TILES); the other launches
                              use 256                                         */
  int32_t reserved;        /* 0                                               */
} flce_plan_info;

/* Exact workspace size for *d (the maximum over the three compute entry
 * points); 0 if *d is invalid.  The library's own call, no passage of the
 * pages behind it: it states the O(N + band) scratch the path needs in place
 * of the [N, V] logits that the pages' chunked and SRAM-tiled designs avoid
 * materialising (Trillion Labs notes, section "1. Chunked Cross-Entropy";
 * CCE Sec. 4, the logits never stored in global memory).  Pure host
 * arithmetic: touches no device. */
size_t flce_workspace_bytes(const flce_desc* d);

/* Fills *out with the plan for *d (the library's own call: the band sizes
 * behind flce_workspace_bytes).  Returns FLCE_OK or an argument error
 * (FLCE_E_NULL for a NULL out).  Pure host arithmetic: touches no device. */
int flce_plan(const flce_desc* d, flce_plan_info* out);

/* Forward: loss_rows [N], lse [N] (every row, ignored ones included) and,
 * unless reduction == FLCE_NONE, loss [1] (mean or sum of loss_rows).
 * loss may be NULL iff reduction == FLCE_NONE.  The logits are produced one
 * 256 x 256 tile per workgroup in registers and reduced to a per-(row,
 * vocabulary tile) max and sum-exp; a second pass merges a row's partials in
 * a fixed order (CCE Alg. 2 without the lock).  The target logit of each row
 * is its own pass, a dot product of the row with W's target row (CCE Alg. 1). */
int flce_forward(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                 float* loss_rows, float* lse, float* loss,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward: dH [N,D] and dW [V,D] (float, or bf16 under FLCE_FLAG_BF16_GRADS;
 * overwritten) from the forward's lse.
 * dloss is a device pointer: [1] for FLCE_MEAN / FLCE_SUM, [N] for FLCE_NONE;
 * NULL means an upstream gradient of 1.  The logits are recomputed block by
 * block, dZ is staged in ws one band at a time (bf16 for bf16 inputs, float
 * for float inputs; two band buffers, one written while the other is
 * contracted) and contracted into dH and dW (CCE Alg. 4 structure). */
int flce_backward(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                  const float* lse, const float* dloss,
                  void* dH, void* dW,
                  void* ws, size_t ws_bytes, hipStream_t stream);

/* Forward then backward with an upstream gradient of 1, in one call: the
 * loss and both gradients of the same definitions as flce_forward and
 * flce_backward (Trillion Labs notes, section "Cross Entropy를 다시 보면";
 * PyTorch 2.13 chapter, section "먼저 수식에서 없앨 수 있는 tensor를
 * 찾는다"; CCE Alg. 2 then Alg. 4).  Arguments as in those two; loss may be
 * NULL iff reduction == FLCE_NONE; dH may be NULL only when N == 0.  With
 * N == 0 the call sets loss to 0 and dW to 0.  Errors as in those two. */
int flce_fused_fwd_bwd(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                       float* loss_rows, float* lse, float* loss,
                       void* dH, void* dW,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* bf16 gradients with Kahan-compensated dW (CCE Sec. 5.1 and Table 1 rows
 * 8-10, "CCE-Kahan": the gradient is summed in its final type with a
 * compensation term of the same type).  Same arguments and results as
 * flce_fused_fwd_bwd / flce_backward, plus dW_comp: a caller-owned device
 * buffer of bf16 [V,D] (dW's layout, 16-byte aligned, outside the workspace,
 * so the workspace bound is unchanged; CCE counts it in its memory column).
 * desc->flags must hold FLCE_FLAG_BF16_GRADS, else FLCE_E_UNSUPPORTED; a NULL
 * dW_comp is FLCE_E_NULL.  dH needs no compensation: it is summed in a float
 * stage and rounded once.  dW of a vocabulary band is updated once per token
 * band, each update in float: y = p - c, t = s + y, s <- bf16(t),
 * c <- bf16((s_new - s) - y), with p the band's float partial and (s, c) the
 * stored bf16 sum and compensation (the first band stores bf16(p) and the
 * rounding it lost).  On return dW_comp holds the last compensation, with
 * dW - dW_comp the closer estimate of the float sum; its contents on entry
 * are ignored.  With one token band dW is bitwise the uncompensated result. */
int flce_fused_fwd_bwd_kahan(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                             float* loss_rows, float* lse, float* loss, void* dH, void* dW,
                             void* dW_comp, void* ws, size_t ws_bytes, hipStream_t stream);
int flce_backward_kahan(const flce_desc* d, const void* H, const void* W, const int64_t* y,
                        const float* lse, const float* dloss, void* dH, void* dW, void* dW_comp,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * forward + backward as flce_fused_fwd_bwd, with the same arguments minus the
 * workspace.  The scratch is a 64 MiB device array inside the library, one
 * per GPU, held until the process ends; its device address is looked up on
 * the first call on each device (with that device current: it must be the
 * stream's device), and no call allocates or frees anything.  The plan is
 * made for a budget of min(desc->ws_budget_bytes or 64 MiB, 64 MiB), so at
 * the default budget the launches and results are those of
 * flce_fused_fwd_bwd bit for bit; a problem whose plan does not fit in 64 MiB
 * returns FLCE_E_WORKSPACE (checked on the host before anything else).
 * FLCE_FLAG_PROFILE is FLCE_E_UNSUPPORTED here (it creates events).  Every
 * call on one GPU shares that GPU's array and leaves its contents behind
 * (the next call needs no cleared scratch): two calls whose work overlaps on
 * one GPU (other streams, other host threads) race and give wrong results;
 * serialise them.  Other errors as flce_fused_fwd_bwd; FLCE_E_DEVICE if the
 * array's address cannot be obtained. */
int flce_fused_fwd_bwd_noalloc(const flce_desc* d, const void* H, const void* W,
                               const int64_t* y, float* loss_rows, float* lse, float* loss,
                               void* dH, void* dW, hipStream_t stream);

/* Multiplies dH [N,D] and dW [V,D] (in place, 16-byte aligned; float, or
 * bf16 under FLCE_FLAG_BF16_GRADS, rounded to nearest even) by the
 * upstream gradient dloss[0] (device pointer; NULL means 1: nothing to do).
 * Together with flce_fused_fwd_bwd this is the contract in which the forward
 * already computes the gradients: p1 (Trillion Labs FLCE notes) section
 * "6. Backward는 새 logits를 만들지 않음" and p2 (PyTorch 2.13
 * LinearCrossEntropyLoss chapter) section "scalar reduction에서는 forward가
 * gradient까지 계산한다": for mean and sum the forward produces dH and dW with
 * an upstream gradient of 1 and the backward only scales them by the upstream
 * scalar.  reduction == FLCE_NONE returns FLCE_E_UNSUPPORTED: a per-row
 * upstream gradient cannot be applied after the contraction, so that path
 * recomputes (flce_backward).  No workspace is used. */
int flce_scale_gradients(const flce_desc* d, const float* dloss, void* dH, void* dW,
                         hipStream_t stream);

/* Synchronises `stream`, then reads the status word of `ws` into *out
 * (bit 0: a target outside [0, V) that is not ignore_index).  The library's
 * own call: the pages define no error channel; it reports the reading that
 * only ignore_index may fall outside [0, V) (Trillion Labs notes, section
 * "1. Chunked Cross-Entropy", where ignored rows are masked out).  Returns
 * FLCE_E_NULL for a NULL argument, FLCE_E_DEVICE if a HIP call fails. */
int flce_device_status(const void* ws, hipStream_t stream, int32_t* out);

/* Work the gradient filter left out (CCE Sec. 4.3, "Gradient filtering",
 * and Algorithm 4: a K step of a gradient contraction is skipped when every
 * block of softmax - onehot it covers is below filter_eps).  Synchronises
 * `stream`, then reads from `ws` the 64-wide K blocks of the filtered
 * gradient contractions of the last flce_backward or flce_fused_fwd_bwd call
 * on this workspace (a later flce_forward on it clears them): *active =
 * blocks that ran, *total = blocks that exist,
 * summed over the tiles (each block of a tile is 256 x 256 x 64
 * multiply-adds).  Only the products the filter acts on are counted (both,
 * or the one FLCE_FLAG_FILTER_FULL_C / _FULL_E leaves filtered); with the
 * filter off both are 0.  The skip fraction is 1 - active / total.  Returns
 * FLCE_E_NULL for a NULL argument, FLCE_E_DEVICE if a HIP call fails. */
int flce_filter_stats(const void* ws, hipStream_t stream, int64_t* active, int64_t* total);

/* Static description of a return code (the library's own call); never NULL. */
const char* flce_strerror(int code);

/* Kernel classes reported by flce_profile_read. */
enum {
  FLCE_K_FWD_LSE = 0,     /* forward contraction + online max/sum-exp        */
  FLCE_K_LSE_COMBINE = 1, /* per-row merge of partials, loss rows            */
  FLCE_K_FINALIZE = 2,    /* scalar loss / row scale                         */
  FLCE_K_BWD_DZ = 3,      /* backward launches of dZ tiles only (the first
                             one; every band's first under BF16_GRADS)        */
  FLCE_K_BWD_GRAD = 4,    /* backward launches of dH, dW tiles only (the last
                             one; every band's second under BF16_GRADS)      */
  FLCE_K_AUX = 5,         /* small fills                                     */
  FLCE_K_BWD_BAND = 6,    /* other backward launches: dH += dZ W_band and
                             dW_band (+)= dZ^T H_band of band k - 1 together
                             with the logits recompute + dZ of band k        */
  FLCE_K_COUNT = 7
};

/* The library's own calls, for measurement (no passage of the pages).
 * Launch timing recorded while desc->flags has FLCE_FLAG_PROFILE.  Each
 * launch made under the flag is bracketed by two HIP events on the launch
 * stream.  flce_profile_read synchronises those events and returns, for
 * kernel class k, the number of launches and their summed duration in ms
 * since the last flce_profile_reset. */
int flce_profile_reset(void);
int flce_profile_read(int kernel_class, int64_t* launches, double* total_ms);
/* flce_profile_read returns FLCE_E_UNSUPPORTED for an unknown class,
 * FLCE_E_NULL for a NULL output and FLCE_E_DEVICE if an event read fails
 * (the unread records stay pending). */

/* Library version, e.g. "flce 0.1.0 gfx950" (the library's own call). */
const char* flce_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FLCE_H */
