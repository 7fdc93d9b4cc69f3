/*
 * radial.h -- C ABI of the radial block-sparse attention library (libradial.so).
 *
 * The library computes multi-head softmax attention under the static
 * "radial" mask of Radial Attention (O(n log n) sparse attention with energy
 * decay for long video generation), on AMD Instinct MI355X (gfx950) GPUs.
 *
 * Sources (abbreviations used below):
 *   review   -- jaehun.me paper review "Radial Attention: O(n log n) Sparse
 *               Attention with Energy Decay for Long Video Generation",
 *               Prompt 1.3.1 (method steps and the f=4, s=9 toy example);
 *               bracketed names (§3, §4.2, Eq.4, Fig.5) are the paper's own
 *               numbering as the review quotes it.
 *   rebuttal -- paperhub.cn author responses for the same paper (ablations
 *               of the sink, the central band and the band width scale).
 *
 * Conventions for every call:
 *   - Return value: RADIAL_OK (0) or a negative RADIAL_E_* code.  No call
 *     aborts or throws across the ABI.  radial_last_error() gives a
 *     human-readable detail string for the calling thread's last failure.
 *   - Tensors are dense row-major [B, H, N, D] (bf16: the raw 16-bit
 *     bfloat16 pattern) or [B, H, N] (fp32), owned by the caller, in device
 *     memory of the current HIP device, 16-byte aligned.  Element (b,h,n,d)
 *     sits at ((b*H + h)*N + n)*D + d.  Offsets are computed in 64 bits.
 *   - Compute calls are asynchronous on the given HIP stream (hipStream_t
 *     passed as void*; NULL = the default stream).  The caller synchronises.
 *     They never allocate device memory and never synchronise the device.
 *   - A layout is immutable once built and uploaded; it may be shared by
 *     any number of streams and threads.  Only radial_layout_upload and
 *     radial_layout_destroy modify it and must not race with its use.
 */
#ifndef RADIAL_H
#define RADIAL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  RADIAL_OK = 0,
  RADIAL_E_INVALID = -1,     /* null / misaligned pointer, bad scalar value   */
  RADIAL_E_UNSUPPORTED = -2, /* (D, block_size) without a kernel, or a size  */
                             /* beyond a stated limit (a slice of 2^31 bytes */
                             /* or more, rows beyond the allocation-free     */
                             /* backward's scratch)                          */
  RADIAL_E_SHAPE = -3,       /* N differs from frames * tokens_per_frame       */
  RADIAL_E_NOMEM = -4,       /* host or device allocation failed               */
  RADIAL_E_HIP = -5,         /* a HIP runtime call or kernel launch failed     */
  RADIAL_E_STATE = -6        /* layout not uploaded to the current device      */
};

/* ---- layout flags ------------------------------------------------------ */
enum {
  /* Attention sink: every query may attend every key of frame 0
     (review Step 4; paper §4.2, Appx A.1 Eq.8).  On in the paper's runs. */
  RADIAL_SINK = 1u << 0,
  /* Keep every tile: plain dense attention through the same kernels, the
     in-library dense baseline. */
  RADIAL_DENSE = 1u << 1,
  /* Token-exact semantics: inside kept tiles only the allowed token pairs
     take part (the mask of paper Eq.4 at token granularity, review Step 3),
     instead of every pair of a kept tile.  The tile lists are the same; the
     kernels apply the token predicate inside the tiles the layout marks
     partial.  No effect together with RADIAL_DENSE (every tile is full). */
  RADIAL_TOKEN_EXACT = 1u << 2
};

typedef struct radial_layout radial_layout; /* opaque */

/* ---- mask variants ------------------------------------------------------
   Knobs of the rebuttal's ablations and the review's harmonic-series
   comparison (review 1.3.2, Appx C.3).  The pages name them but not where
   they enter the formulas; the readings below are used.  With the frame
   distance delta = |i - j|, the shifted distance is
     e = max(delta - central_band + 1, 1)
   (rebuttal "Width of Central Band": frame pairs with delta <= d attend in
   full), the band index is r = floor(log2(e)) and the half width w and the
   sampling period p (used when w == 0) are
     RADIAL_DECAY_RADIAL:   w = floor(s / c^r), p = ceil(c^r / s), where
                            c = scale_num / scale_den is the ratio between
                            consecutive bands' widths (rebuttal "Width Scale
                            Between Consecutive Bands"); bands keep their
                            doubling extent;
     RADIAL_DECAY_HARMONIC: w = floor(s / e), p = ceil(e / s) (width
                            inversely proportional to the distance); the
                            scale is ignored.
   The defaults (radial, d = 1, c = 2/1) give the mask described at
   radial_mask_build. */
enum { RADIAL_DECAY_RADIAL = 0, RADIAL_DECAY_HARMONIC = 1 };

typedef struct radial_mask_params {
  int32_t decay;        /* RADIAL_DECAY_RADIAL or RADIAL_DECAY_HARMONIC           */
  int32_t central_band; /* d >= 0                                                  */
  int32_t scale_num;    /* c = scale_num / scale_den; 1 <= scale_den <= 4,         */
  int32_t scale_den;    /*   scale_den < scale_num <= 16 (checked for radial only) */
} radial_mask_params;

/* Fills *p with the defaults (radial decay, d = 1, c = 2/1). */
void radial_mask_params_default(radial_mask_params *p);

/*
 * radial_mask_build -- compile the radial mask of a video with `frames`
 * frames of `tokens_per_frame` tokens (n = frames * tokens_per_frame) into
 * a block-sparse layout of block_size x block_size tiles.  Host only; no
 * HIP call is made.
 *
 * Token q = i*s + a is position a (row-major in-frame index) of frame i
 * (review "Terms and variables"; the 4-D mask is flattened as in paper
 * Eq.4 / §4.2).  Query (i, a) may attend key (j, b) iff
 *   - RADIAL_SINK is set and j == 0, or
 *   - with delta = |i - j|, r = floor(log2(max(delta, 1))) (temporal band,
 *     review Step 2-A, paper §4.2 Fig.5a) and w = floor(s / 2^r) (spatial
 *     half width, review Step 2-B, paper Fig.5b):
 *       w >= 1: |a - b| < w (strict, as the review's toy example fixes);
 *       w == 0: a == b and delta is a multiple of ceil(2^r / s) (diagonal
 *               subsampling below unit width, review Step 2-C, paper Fig.5
 *               caption).
 * A tile (u, v) is kept iff at least one allowed token pair lies in it, and
 * kept tiles are computed in full (review Step 5, paper §4.2: block-wise
 * computation in 128 x 128 blocks); with RADIAL_TOKEN_EXACT only the
 * allowed pairs inside them take part.  The last tile row/column is partial
 * when block_size does not divide n.
 *
 * frames >= 1, tokens_per_frame >= 1, n < 2^31, 1 <= block_size <= 4096.
 * flags: RADIAL_SINK | RADIAL_DENSE | RADIAL_TOKEN_EXACT.  On success *out owns a new layout
 * (free with radial_layout_destroy); on failure *out is set to NULL.
 */
int radial_mask_build(int64_t frames, int64_t tokens_per_frame, int32_t block_size,
                      uint32_t flags, radial_layout **out);

/* radial_mask_build for a mask variant (see radial_mask_params); params ==
   NULL means the defaults, i.e. radial_mask_build.  RADIAL_E_INVALID for
   parameters outside the stated ranges.  Every other call works on the
   resulting layout unchanged, token-exact semantics included. */
int radial_mask_build_ex(int64_t frames, int64_t tokens_per_frame, int32_t block_size,
                         uint32_t flags, const radial_mask_params *params,
                         radial_layout **out);

/* Sizes of a layout.  n_tokens = frames * tokens_per_frame; n_blocks =
   ceil(n / block_size); nnz_tiles = kept tiles; nnz_pairs = token pairs
   inside kept tiles, counting only rows and columns < n (the work the
   kernels do per batch and head).  Any output pointer may be NULL. */
int radial_layout_info(const radial_layout *L, int64_t *n_tokens, int32_t *n_blocks,
                       int64_t *nnz_tiles, int64_t *nnz_pairs);

/* Host copies of the tile lists.  CSR: row_ptr[n_blocks + 1] and
   col_idx[nnz_tiles], key tiles ascending per query tile.  CSC:
   col_ptr[n_blocks + 1] and row_idx[nnz_tiles], query tiles ascending per
   key tile.  Any pointer may be NULL (that array is skipped). */
int radial_layout_export(const radial_layout *L, int32_t *row_ptr, int32_t *col_idx,
                         int32_t *col_ptr, int32_t *row_idx);

/* Full/partial marks of the kept tiles: csr_full[t] (CSR order) and
   csc_full[t] (CSC order) are 1 when every token pair of tile t with row and
   column < n is allowed, else 0 (the tiles token-exact semantics must mask
   inside).  Filled for every layout; with RADIAL_DENSE every tile is full.
   Any pointer may be NULL. */
int radial_layout_tile_flags(const radial_layout *L, uint8_t *csr_full, uint8_t *csc_full);

/* ---- layer / step schedule ---------------------------------------------
   radial_schedule_dense -- whether layer `layer` at denoising step `step`
   should attend in full, i.e. be called with a RADIAL_DENSE layout instead
   of the radial one (rebuttal "Capability of Capturing Long-Range
   Dependencies" and "Ablations on Initial Full-Attention Layers and
   Steps": the first two layers stay dense in training and inference, and
   the first 12 of 50 steps (default-length videos) or 2 steps (4x longer
   videos) are a dense warm-up at inference).  Returns 1 (dense) when
   layer < dense_layers or step < warmup_steps, else 0 (radial);
   RADIAL_E_INVALID when any argument is negative.  Training has no
   warm-up: pass warmup_steps = 0.  Host only. */
int radial_schedule_dense(int32_t layer, int32_t step, int32_t dense_layers,
                          int32_t warmup_steps);

/* Band table, one entry per frame distance delta in [0, frames):
   band[delta] = r, width[delta] = w, period[delta] = sampling period
   (1 when w >= 1; capped at 2^31 - 1, beyond every frame distance).  Any
   pointer may be NULL. */
int radial_layout_band_table(const radial_layout *L, int32_t *band, int64_t *width,
                             int64_t *period);

/* Token-level mask for testing: out[q * n + k] = 1 if query q may attend
   key k, else 0.  Needs cap >= n * n bytes; returns RADIAL_E_INVALID if
   n * n > cap. */
int radial_layout_token_mask(const radial_layout *L, uint8_t *out, int64_t cap);

/* Copy the tile lists to the current HIP device (blocking; allocates device
   memory owned by the layout).  Must be called once before any compute call
   on that device; a second call on another device moves the layout there. */
int radial_layout_upload(radial_layout *L);

/* Free a layout and its device copy.  NULL is ignored. */
void radial_layout_destroy(radial_layout *L);

/*
 * radial_attn_fwd -- O = softmax(scale * Q K^T + M) V under the layout's
 * mask M (review Step 0, paper §3 Eq.1/Eq.2), for every batch b and head h.
 * M is 0 on every pair of a kept tile and -inf elsewhere; with
 * RADIAL_TOKEN_EXACT it is 0 exactly on the allowed token pairs.
 *
 *   q, k, v : bf16 [B, H, N, D] inputs.
 *   o       : bf16 [B, H, N, D] output (rounded to nearest even).
 *   lse     : fp32 [B, H, N] output, natural-log log-sum-exp of the scaled,
 *             masked logits of each query row (used by the backward pass).
 * N must equal the layout's n; (D, block_size) must be (64, 64),
 * (64, 128) or (128, 128); B, H >= 1; scale finite and > 0 (usually 1/sqrt(D)).
 * One (batch, head) slice must hold fewer than 2^31 bytes (N * D * 2 < 2^31,
 * i.e. N < 8,388,608 at D = 128): larger N returns RADIAL_E_UNSUPPORTED
 * (checked before N is compared with the layout).
 * Products run on bf16 MFMA with fp32 accumulation and an fp32 online
 * softmax; the probabilities are rounded to bf16 before the P V product.
 */
int radial_attn_fwd(const radial_layout *L, int32_t B, int32_t H, int64_t N, int32_t D,
                    float scale, const void *q, const void *k, const void *v, void *o,
                    float *lse, void *hip_stream);

/* Workspace bytes radial_attn_bwd needs for these sizes: two fp32 row
   arrays, -Delta and -LSE * log2(e) (2 * B * H * N floats, rounded up). */
size_t radial_attn_bwd_workspace_bytes(const radial_layout *L, int32_t B, int32_t H,
                                       int64_t N, int32_t D);

/*
 * radial_attn_bwd -- gradients of the forward above for an upstream
 * gradient dout = dL/dO: dq, dk, dv (bf16 [B, H, N, D], fully overwritten).
 * o and lse must be the forward's outputs for the same q, k, v, scale and
 * layout.  Shapes, limits and errors as radial_attn_fwd.  The probabilities are recomputed from lse; Delta = rowsum(dO*O)
 * and the exponent's row term are formed first in `workspace` (caller-owned
 * device memory of at least radial_attn_bwd_workspace_bytes bytes, 16-byte
 * aligned).  Deterministic:
 * no atomics, fixed summation order.
 */
int radial_attn_bwd(const radial_layout *L, int32_t B, int32_t H, int64_t N, int32_t D,
                    float scale, const void *q, const void *k, const void *v, const void *o,
                    const float *lse, const void *dout, void *dq, void *dk, void *dv,
                    void *workspace, size_t workspace_bytes, void *hip_stream);

/* Bytes of the static device scratch radial_attn_bwd_noalloc uses (per
   device, held until the process ends): room for the two row arrays at
   B * H * N up to 8,388,544. */
#define RADIAL_BWD_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * radial_attn_bwd_noalloc -- radial_attn_bwd without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid
 * hipMalloc).  The two row arrays live in a static device array of
 * RADIAL_BWD_SCRATCH_BYTES bytes that the library holds on every device it
 * runs on; the call allocates nothing (the array's address is looked up on
 * the first call on each device).  Same arguments, kernels and results as
 * radial_attn_bwd (bit for bit).  RADIAL_E_UNSUPPORTED when
 * radial_attn_bwd_workspace_bytes(L, B, H, N, D) > RADIAL_BWD_SCRATCH_BYTES.
 * Every call on a device shares that device's scratch: calls that overlap
 * in time on one device (different streams, threads) race and must be
 * serialised by the caller.  Nothing in the scratch needs to start at zero:
 * each call writes every row before reading it.
 */
int radial_attn_bwd_noalloc(const radial_layout *L, int32_t B, int32_t H, int64_t N, int32_t D,
                            float scale, const void *q, const void *k, const void *v,
                            const void *o, const float *lse, const void *dout, void *dq,
                            void *dk, void *dv, void *hip_stream);

/* Test hook: caps the query-tile grouping of every later radial_attn_fwd
   call in the process at max_group tiles per workgroup (1 single tiles, 2
   pairs, 3 triples, the default); the three forms give identical bits, and
   tests compare them.  Returns the previous cap, or RADIAL_E_INVALID for a
   value outside 1..3.  Not for concurrent use with forward calls. */
int radial_test_set_fwd_group(int32_t max_group);

/* Test hook: while on = 1, radial_mask_build[_ex] and radial_layout_upload
   fail with RADIAL_E_NOMEM before allocating anything (0 restores normal
   behaviour), so tests can reach the allocation-failure paths.  Returns the
   previous setting, or RADIAL_E_INVALID for a value other than 0 or 1.  Not
   for concurrent use with layout calls. */
int radial_test_set_fail_alloc(int32_t on);

/* Static text for a status code. */
const char *radial_status_string(int status);

/* Detail of the calling thread's last failed call ("" if none). */
const char *radial_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RADIAL_H */
