/*
 * gsa.h -- C ABI of libgsa: one rank's fused GEMV + one-shot AllReduce over
 * a symmetric buffer, on one MI355X (gfx950).
 *
 * The operation (restated from the sources):
 *   - "Overlapping Collective Communication with Dependent Computation ...
 *     GPU-Initiated Intra-Kernel Networking" (summary of "Optimizing
 *     Distributed ML Communication with Fused Computation-Collective
 *     Operations"), Abstract: a GEMV fused with its AllReduce in one kernel;
 *     each workgroup hands its finished share to the collective at once, and
 *     scale-up results are written straight into peer memory.
 *   - "Bay.Area.AI: Tensor and 2D Parallelism", Megatron MLP segment: the
 *     row-parallel layer leaves a partial sum on every rank and one
 *     all-reduce finishes it.  Rank r holds A_r, the input-dimension slice
 *     (N x K/W) of the weight, and x_r, the matching activation slice.
 *   - "PyTorch Symmetric Memory" documentation, writing-your-own-kernel
 *     section: buffers of every rank are visible to the kernel, a signal pad
 *     comes with every symmetric allocation, and the one-shot all-reduce sums
 *     the buffers of ranks 0..W-1 in order from a zero accumulator.
 *
 * One call of gsa_gemv_allreduce on rank `rank`:
 *   1. y_r[n][b] = sum_k A_r[n][k] x_r[b][k]   (bf16 in, fp32 accumulate)
 *   2. slot[rank][n][b] = y_r[n][b]            (publish)
 *   3. flag[rank][t] = e_t                     (release, per flag tile t of 4 rows)
 *   4. wait flag[p][t] >= e_t for every p      (acquire, per flag tile, bounded)
 *   5. out[n][b] = ((0 + s_0) + s_1) ... + s_{W-1}, s_r = slot[r][n][b],
 *      fp32 round-to-nearest, s_rank being the value published in step 2.
 * On one GPU the W-1 peer slots are ordinary device memory filled by the
 * caller, and simulated peers are marked "published" in the signal pad.
 *
 * Conventions for every entry point:
 *   - Pointers marked [device] are device addresses on the current HIP
 *     device; [host] are host addresses.  Sizes are element counts.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Return value: GSA_OK or a negative GSA_E* code; no exceptions escape.
 *   - Nothing here allocates on the call path except gsa_symm_alloc.
 */
#ifndef GSA_H
#define GSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GSA_OK        0
#define GSA_EINVAL   (-1)  /* bad argument; nothing was launched            */
#define GSA_ENOMEM   (-2)  /* device allocation failed                      */
#define GSA_EHIP     (-3)  /* a HIP runtime call or a launch failed         */
#define GSA_ETIMEOUT (-4)  /* a device-side flag wait expired (asynchronous) */
#define GSA_ESTATE   (-5)  /* the caller's own flag row was marked published
                              for every call, or its epoch is exhausted
                              (asynchronous)                               */
#define GSA_ESPLIT   (-6)  /* a split or offset read on the device was out of
                              range, or an expert got more tokens than
                              GSA_MOE_MAX_TOKENS (asynchronous)            */

/* Flag value of a simulated peer: "published for every epoch". */
#define GSA_FLAG_PUBLISHED 0xFFFFFFFFu
/* Signal-pad protocol: one flag per rank per flag tile of 4 output rows (all
 * batch columns).  T = ceil(N / 4) flag tiles.  A workgroup computes 4 or 16
 * rows (chosen from K/W and B), so it raises and waits on 1 or 4 flags. */
#define GSA_FLAG_TILE_ROWS 4
/* Within a rank's row the flags come in groups of GSA_FLAG_GROUP_TILES
 * consecutive flag tiles (16 rows), one group per GSA_FLAG_GROUP_WORDS words
 * (128 bytes): flag tile t sits at word (t / 4) * 32 + t % 4.  A 16-row
 * workgroup's flags share one line, and neighbouring workgroups' flags do
 * not. */
#define GSA_FLAG_GROUP_TILES 4
#define GSA_FLAG_GROUP_WORDS 32
/* The MoE combine's flags cover tiles of 16 output features. */
#define GSA_MOE_TILE_ROWS 16
/* The pad starts with GSA_PAD_HEADER_WORDS status words, then 2W rows of
 * flags, row r at word GSA_PAD_HEADER_WORDS + r * gsa_signal_pad_row_stride(N)
 * (flag tile t of the row at word (t / 4) * 32 + t % 4 of it):
 * rows 0..W-1 hold each rank's slot flags, rows W..2W-1 each rank's
 * reduced-chunk flags of the two-shot variant. */
#define GSA_PAD_HEADER_WORDS 16
#define GSA_MAX_W 8
#define GSA_MAX_B 16
/* For B <= 8 every workgroup stages x in LDS: B*K/W*2 bytes may not exceed
 * this.  For B > 8 x is staged in LDS (16 batch rows of K/W*2 + 16 bytes)
 * when that fits under this bound and read from memory otherwise. */
#define GSA_MAX_X_LDS_BYTES (128 * 1024)

/* Element types: of a buffer's slots (gsa_symm_alloc_dtype), of out
 * (gsa_gemv_allreduce_dtype) and of the fused epilogue's y. */
#define GSA_DTYPE_F32 0
#define GSA_DTYPE_BF16 1

typedef struct gsa_symm gsa_symm; /* opaque host-side handle */

/* Allocate one symmetric buffer: W fp32 slots of N x B (n-major) followed by
 * the signal pad, as one device allocation on the current device, zeroed,
 * every flag 0.  Host-blocking; meant for init time, not the call path (the
 * PyTorch Symmetric Memory docs, API reference of empty(): allocate once and
 * reuse).  1 <= W <= GSA_MAX_W, N >= 1, 1 <= B <= GSA_MAX_B.
 * *out [host] receives the handle.  Errors: GSA_EINVAL, GSA_ENOMEM, GSA_EHIP. */
int gsa_symm_alloc(int W, int64_t N, int B, gsa_symm **out);

/* gsa_symm_alloc with the slots' element type: GSA_DTYPE_F32 (the slots of
 * gsa_symm_alloc) or GSA_DTYPE_BF16, W bf16 slots of N x B (n-major, half
 * the bytes).  A buffer with bf16 slots is used through
 * gsa_gemv_allreduce_dtype only (the other calls take fp32 slots and reject
 * it with GSA_EINVAL).  Errors as gsa_symm_alloc; an unknown type is
 * GSA_EINVAL. */
int gsa_symm_alloc_dtype(int W, int64_t N, int B, int slot_dtype, gsa_symm **out);

/* Free a handle and its device memory (host-blocking: synchronizes the
 * device first).  NULL is a no-op.  Errors: GSA_EINVAL (unknown handle). */
int gsa_symm_free(gsa_symm *h);

/* [device] slot 0 of the buffer; slot r starts r*N*B elements later (fp32,
 * or the 16 bits of each bf16 value for a buffer whose slots are bf16).
 * NULL for an unknown handle.  The library owns this memory. */
float *gsa_symm_slots(const gsa_symm *h);

/* [device] signal pad of the buffer (header + flags).  NULL if unknown. */
uint32_t *gsa_symm_signal_pad(const gsa_symm *h);

/* [device] the two-shot variant's gathered chunks: N x B fp32 (n-major), the
 * rows of rank p's chunk holding what rank p published as its reduced chunk
 * (on one GPU the caller fills the other ranks' rows).  NULL if unknown. */
float *gsa_symm_gathered(const gsa_symm *h);

/* Words between consecutive rank rows of the pad for N rows
 * (ceil(ceil(N / 4) / 4) groups of 32 words, rounded up to a multiple of 64).
 * Returns -1 for N < 1. */
int64_t gsa_signal_pad_row_stride(int64_t N);

/* Reset a pad: flag rows p and W + p := GSA_FLAG_PUBLISHED if bit p of
 * published_mask is set, else 0; status words and the fused epilogue's counts cleared (and
 * its library-held scratch made ready for them).  Stream-ordered (a small kernel), no
 * host sync, no allocation.  `pad` [device] must come from
 * gsa_symm_signal_pad of a buffer allocated with the same W and N.  The
 * calling rank's bit must be clear before it calls gsa_gemv_allreduce.
 * Errors: GSA_EINVAL, GSA_EHIP. */
int gsa_signal_pad_reset(uint32_t *pad, int W, int64_t N, uint32_t published_mask,
                         void *stream);

/* One fused call on rank `rank` (steps 1-5 above), enqueued on `stream`.
 *   A_r   [device] bf16 bits, N x Ks row-major (Ks = K/W, leading dim Ks)
 *   x     [device] bf16 bits, this rank's activation slice, B x Ks row-major
 *   slots [device] gsa_symm_slots of a buffer allocated with (W, N, B)
 *   pad   [device] gsa_symm_signal_pad of the same buffer
 *   out   [device] fp32 N x B (n-major); any device memory, written only
 * Requires 1 <= W <= 8, 0 <= rank < W, K % W == 0, Ks % 8 == 0, N >= 1,
 * 1 <= B <= 16, N * Ks * 2 < 2^31 (A_r is addressed with 32-bit offsets),
 * every pointer non-null and 16-byte aligned, and, for B <= 8 (x staged in
 * LDS), B * Ks * 2 <= GSA_MAX_X_LDS_BYTES; otherwise GSA_EINVAL and nothing
 * is launched.
 * A_r must hold finite values (chunks past a row's end are paired with zeros).
 * No host sync, no allocation.  All calls on one buffer must use one stream
 * (flags are indexed by tile, not by stream).  Each flag tile's epoch is its
 * own previous flag + 1, so at most 2^32 - 2 calls fit between resets.
 * Device-side failures leave `out` rows unwritten and are reported by
 * gsa_signal_pad_status: a wait that exceeded the timeout, the rows of that
 * flag tile; an unusable own flag, every row of its workgroup (which then
 * raises none of its flags).  Errors: GSA_EINVAL, GSA_EHIP (launch failed). */
int gsa_gemv_allreduce(const uint16_t *A_r, const uint16_t *x, float *slots,
                       uint32_t *pad, float *out, int W, int rank, int64_t N,
                       int64_t K, int B, void *stream);

/* gsa_gemv_allreduce with element types: the "PyTorch Symmetric Memory"
 * documentation, higher-precision reduction section, takes bf16 values,
 * accumulates them in fp32 and hands the result back in bf16.  Here:
 *   - slots [device]: a buffer from gsa_symm_alloc_dtype; if its slots are
 *     bf16, step 2 publishes y_r rounded to bf16 (to nearest, ties to even)
 *     and step 5 widens every slot value exactly and sums in fp32 -- the own
 *     term being the value as published, so out is the fold of the slots as
 *     they stand after the call;
 *   - out [device]: N x B of out_dtype (GSA_DTYPE_F32, or GSA_DTYPE_BF16:
 *     the fp32 sum rounded to nearest, ties to even), 16-byte aligned.
 * Step 1 accumulates in fp32 in every case.  Everything else (arguments,
 * limits, protocol, errors) as gsa_gemv_allreduce; GSA_EINVAL also for an
 * unknown out_dtype.  With fp32 slots and an fp32 out the result is the
 * same as gsa_gemv_allreduce's, bit for bit. */
int gsa_gemv_allreduce_dtype(const uint16_t *A_r, const uint16_t *x, void *slots,
                             uint32_t *pad, void *out, int out_dtype, int W, int rank,
                             int64_t N, int64_t K, int B, void *stream);

/* The two-stage variant of the same operator: the documentation's op
 * reference lists a two-stage all-reduce (two_shot_all_reduce_) beside the
 * one-shot one, read here as reduce-scatter then all-gather.  Each rank owns
 * one chunk of ceil(ceil(N / W) / 16) * 16 rows (whole 16-row workgroup
 * tiles; rank p owns rows [p * chunk, (p + 1) * chunk)).  A call computes and publishes y_r and
 * the slot flags as gsa_gemv_allreduce does; for the rows of its own chunk it
 * waits for every rank's slot flag, writes out = the rank-order sum from zero
 * (the one-shot rule, same bits) and publishes it into `gathered` with its
 * reduced-chunk flag (pad row W + rank); for every other row it waits for
 * the owner's reduced-chunk flag and copies the owner's `gathered` rows into
 * out.  Per rank this reads (W - 1) chunks of peer slots plus W - 1 peer
 * chunks, instead of W - 1 whole slots.  `gathered` [device] must be
 * gsa_symm_gathered of the same buffer; everything else as gsa_gemv_allreduce.
 * Errors: GSA_EINVAL, GSA_EHIP. */
int gsa_gemv_allreduce_two_shot(const uint16_t *A_r, const uint16_t *x, float *slots,
                                uint32_t *pad, float *gathered, float *out, int W, int rank,
                                int64_t N, int64_t K, int B, void *stream);

/* What gsa_gemv_allreduce_rmsnorm does after the one-shot sum.  The
 * "PyTorch Symmetric Memory" talk's real-model example follows the
 * all-reduce with a bias addition (elementwise, so it joins the reduction
 * loop) and an RMSNorm, all in one kernel; RMSNorm is taken by its textbook
 * definition over the hidden dimension, i.e. the N output rows of a token:
 *   z[n][b]  = out[n][b] + bias[n]                     (fp32)
 *   inv[b]   = 1 / sqrtf(sum_n z[n][b]^2 / N + eps)     (fp32)
 *   y[n][b]  = (z[n][b] * inv[b]) * rms_weight[n]       (fp32, then y_dtype)
 * A bf16 y is rounded to nearest, ties to even (an fp32 accumulation handed
 * back in bf16, as in the documentation's higher-precision reduction). */
typedef struct gsa_epilogue {
  const float *bias;       /* [device] N fp32, or NULL: no bias */
  const float *rms_weight; /* [device] N fp32, or NULL: weight 1 */
  float eps;               /* finite, >= 0 (eps = 0 and an all-zero column give NaN) */
  int y_dtype;             /* GSA_DTYPE_F32 or GSA_DTYPE_BF16 */
  void *y;                 /* [device] N x B (n-major), naturally aligned, written */
  float *inv_rms;          /* [device] B fp32 written with inv[b], or NULL */
} gsa_epilogue;

/* gsa_gemv_allreduce (same arguments, same contract, `out` written as
 * there), followed in the same kernel by the epilogue `ep` [host, read
 * before return].  The sum over n crosses tiles: each tile publishes its
 * partial sums of squares in the buffer's epilogue scratch, each value
 * tagged with the call's index (taken from counts that only grow, cleared
 * with the scratch by gsa_signal_pad_reset); one workgroup folds them in
 * one fixed order as they arrive, so repeated calls are bit-identical, and
 * publishes 1/rms.  A tile that finds every tile of the call started once
 * its own rows are done waits for 1/rms and normalises its own rows
 * (started tiles always finish, so that wait cannot deadlock); on calls of
 * at most 64 partial sums (16-row tiles x B) such a tile folds them itself,
 * in the same order, instead of waiting for 1/rms.  The rows of every other
 * tile are normalised by the folding workgroup.  All give the same bits.
 * The waits are bounded (a fold's by twice, a tile's wait for 1/rms by four
 * times the timeout of gsa_set_wait_timeout_us); if one
 * expires, gsa_signal_pad_status reports GSA_ETIMEOUT with that tile's first
 * flag tile and peer -1.  If any tile of the call failed, y and inv_rms are
 * NaN.
 * Requires N <= 2^24 in addition.  Errors: GSA_EINVAL (also: ep or y NULL,
 * unknown y_dtype, misaligned pointer, eps negative or not finite),
 * GSA_EHIP. */
int gsa_gemv_allreduce_rmsnorm(const uint16_t *A_r, const uint16_t *x, float *slots,
                               uint32_t *pad, float *out, int W, int rank, int64_t N,
                               int64_t K, int B, const gsa_epilogue *ep, void *stream);

/* The epilogue of gsa_gemv_allreduce_rmsnorm as a kernel of its own, over
 * an `out` [device] (N x B fp32, n-major) already written, e.g. by a
 * gsa_gemv_allreduce call earlier on the same stream: the unfused form of the
 * talk's real-model example ("PyTorch Symmetric Memory: A New Programming
 * Paradigm for Distributed AI"), where the reduction, a bias addition and an
 * RMSNorm run in one kernel.  Same definition as there (bias, rms_weight,
 * eps, y, inv_rms of `ep` [host, read before return]); one kernel of B
 * workgroups, no host sync, no allocation.  inv_rms is the fold of the
 * squares in one fixed order (its bits may differ from the fused call's, which
 * sums in another order); y is computed from it exactly as there.
 * Errors: GSA_EINVAL (out, ep or y NULL, N < 1, N > 2^24, B outside
 * 1..GSA_MAX_B, unknown y_dtype, misaligned pointer, eps negative or not
 * finite), GSA_EHIP. */
int gsa_bias_rmsnorm(const float *out, int64_t N, int B, const gsa_epilogue *ep, void *stream);

/* One-GPU stand-in for a peer's zero-copy push, for tests of the signal-pad
 * protocol.  The fused-operators page has each rank write its finished
 * results straight into the peers' memory and signal them; the
 * documentation's custom-kernel section asks that a peer's writes be visible
 * before it signals.  On `stream`, one workgroup spins for delay_us
 * microseconds of device wall-clock time (0 <= delay_us <= 1000000), stores
 * `values` [device] (N x B, n-major, of the buffer's slot element type: fp32,
 * or bf16 bits) into slot `peer` with device-coherent stores, waits until
 * they are complete, and then stores `epoch` into every flag of pad row
 * `peer` (flag tiles 0..ceil(N/4)-1).  Run on a second stream it publishes
 * while a fused call on another stream is already waiting.  slots, pad [device]:
 * one buffer of (W, N, B); `values` must stay valid until the kernel ran.
 * The kernel always ends.  Errors: GSA_EINVAL (unknown buffer, sizes, peer
 * out of range, misaligned values, delay too long), GSA_EHIP. */
int gsa_peer_publish(void *slots, uint32_t *pad, const void *values, int W, int peer,
                     int64_t N, int B, uint32_t epoch, uint32_t delay_us, void *stream);

/* gsa_gemv_allreduce_rmsnorm for callers that cannot allocate device memory
 * or have the library hold any per buffer for them: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, contract and results (bit for bit) as
 * gsa_gemv_allreduce_rmsnorm; the difference is the epilogue's scratch (the
 * partial sums of squares per 16-row tile, the published 1/rms and the
 * started counts).  It lives in one file-scope device array of the
 * library, at most 2048 tiles' worth (N <= 32768; larger N: GSA_EINVAL),
 * 272 KiB, which every GPU the library runs on holds until the process
 * ends.  Every call first clears the part of the array it uses with a small
 * kernel (so a call is two kernels on `stream`) and allocates nothing.  All
 * calls on
 * one GPU share the array, which keeps the last call's contents: calls that
 * overlap on one GPU (other streams) race and must not be issued. */
int gsa_gemv_allreduce_rmsnorm_noalloc(const uint16_t *A_r, const uint16_t *x, float *slots,
                                       uint32_t *pad, float *out, int W, int rank, int64_t N,
                                       int64_t K, int B, const gsa_epilogue *ep, void *stream);

/* Read the pad's status words after the work queued on `stream` has finished
 * (synchronizes `stream`).  *code [host] := GSA_ESTATE if any call found its
 * own flag row unusable (then *tile := the smallest such flag tile, *peer :=
 * -1), else GSA_ETIMEOUT if any wait expired (then *tile, *peer := the
 * smallest (flag tile, peer) pair whose wait expired), else GSA_OK (*tile =
 * *peer = -1).
 * Words stay set until the next gsa_signal_pad_reset.
 * Errors: GSA_EINVAL (unknown pad), GSA_EHIP. */
int gsa_signal_pad_status(const uint32_t *pad, void *stream, int *code,
                          int64_t *tile, int *peer);

/* Device-side wait bound for later calls, in microseconds (default 100000).
 * 0 is rejected with GSA_EINVAL. */
int gsa_set_wait_timeout_us(uint32_t us);

/* Static text for a GSA_* code. */
const char *gsa_strerror(int code);

/* ------------------------------------------------------------------------
 * Mixture of experts: an expert's down-projection GEMM fused with the
 * combine all-to-all, at one rank's share.
 *
 * The fused-operators page names GEMM + All-to-All for mixture-of-experts
 * models beside GEMV + AllReduce; the symmetric-memory documentation's op
 * reference (all_to_all_vdev_2d, all_to_all_vdev_2d_offset) fixes the data
 * movement: the dispatch leaves each rank's tokens expert-major (for local
 * expert e, the segments of source ranks 0..W-1), splits and offsets live on
 * the device, and the combine sends every segment back to its source rank at
 * an offset that rank chose.  Here rank `rank` holds ne experts (global
 * expert rank * ne + e); for each local expert e and each 16-feature tile t
 * one workgroup multiplies the expert's dispatched rows by the tile's 16
 * weight rows (bf16 in, fp32 accumulation), stores each result row straight
 * into its source rank's combine buffer, raises flag (rank, e, t) in that
 * rank's signal pad, and then waits (bounded) for flag (p, e, t) of every
 * other rank p in its own pad: when the call's work has finished, this
 * rank's combine buffer holds every expert's rows for its tokens.
 *
 * On one GPU the W combine buffers and W pads of a gsa_a2a allocation stand
 * for the W ranks' symmetric buffers: this rank writes its rows into all of
 * them, and the other ranks' rows in its own buffer are filled by the
 * caller, their flags marked published by gsa_a2a_reset.
 * ---------------------------------------------------------------------- */

/* Tokens one local expert may take per call: the kernel runs them in tiles of
 * 16 tokens (one MFMA operand of 16 columns each); a split table that gives
 * an expert more is reported as GSA_ESPLIT for that expert. */
#define GSA_MOE_MAX_TOKENS 256
/* Largest input width F of the expert GEMM (the dispatched rows of one
 * expert are staged in LDS). */
#define GSA_MOE_MAX_F 4088

typedef struct gsa_a2a gsa_a2a;

/* Words of one signal pad: GSA_PAD_HEADER_WORDS status words, then W * ne
 * flag rows of S = (pad words - GSA_PAD_HEADER_WORDS) / (W * ne) words
 * (ceil(H / GSA_MOE_TILE_ROWS) rounded up to a multiple of 64); row
 * p * ne + e holds the flags of source rank p's local expert e, one per
 * 16-feature tile.  -1 on a bad argument. */
int64_t gsa_a2a_pad_words(int W, int ne, int64_t H);

/* Allocate (zeroed, host-blocking, init time) W combine buffers of
 * rows_out x H fp32 (rank s's buffer at s * rows_out * H, row-major) and W
 * signal pads.  1 <= W <= GSA_MAX_W, 1 <= ne <= 256, H >= 1,
 * 1 <= rows_out, W * rows_out * H < 2^40.  *out [host] := the handle.
 * Errors: GSA_EINVAL, GSA_ENOMEM, GSA_EHIP. */
int gsa_a2a_alloc(int W, int ne, int64_t H, int64_t rows_out, gsa_a2a **out);
/* Free a handle (synchronizes its device first).  NULL is a no-op. */
int gsa_a2a_free(gsa_a2a *h);
/* [device] the W combine buffers, or NULL for an unknown handle. */
float *gsa_a2a_buffers(const gsa_a2a *h);
/* [device] the W signal pads (pad s at s * gsa_a2a_pad_words(W, ne, H)). */
uint32_t *gsa_a2a_signal_pads(const gsa_a2a *h);

/* Reset every pad of the allocation on `stream`: status words cleared; flag
 * row p * ne + e := GSA_FLAG_PUBLISHED if bit p of published_mask is set,
 * else 0.  Errors: GSA_EINVAL (unknown pads or mismatched sizes), GSA_EHIP. */
int gsa_a2a_reset(uint32_t *pads, int W, int ne, int64_t H, uint32_t published_mask,
                  void *stream);

/* One call of rank `rank` (asynchronous on `stream`, one kernel, no
 * allocation, no host sync):
 *   X      [device] bf16 bits, rows_in x F: the dispatched rows
 *   Wd     [device] bf16 bits, ne x H x F: expert e's weight, H output
 *          features of F inputs, row-major
 *   splits [device] int32, 2 x ne x W: splits[e * W + s] = rows of source
 *          rank s for local expert e, splits[ne * W + e * W + s] = the first
 *          of them in X (gaps between segments are allowed)
 *   dst_off [device] int32, W x ne: dst_off[s * ne + e] = the first row of
 *          that segment in rank s's combine buffer
 *   bufs, pads: gsa_a2a_buffers / gsa_a2a_signal_pads of one allocation of
 *          (W, ne, H, rows_out)
 * Row i of segment (e, s) of the result, sum_k X[row][k] * Wd[e][n][k] in
 * fp32, goes to row dst_off[s * ne + e] + i of buffer s.  Each local expert
 * may take at most GSA_MOE_MAX_TOKENS rows per call; experts with none skip
 * their weights.  Host-checked: sizes (F % 8 == 0, F <= GSA_MOE_MAX_F,
 * H * F * 2 < 2^31), 16-byte alignment of X, Wd, bufs, pads, 4-byte
 * alignment of splits and dst_off.  Device-checked: every split and offset
 * (a bad table sets GSA_ESPLIT for that expert, which then writes nothing
 * and raises no flag).  Flags carry epochs like gsa_gemv_allreduce (own row
 * of the own pad + 1).  Errors: GSA_EINVAL, GSA_EHIP; GSA_ETIMEOUT,
 * GSA_ESTATE and GSA_ESPLIT later through gsa_a2a_status. */
int gsa_moe_gemm_all_to_all(const uint16_t *X, const uint16_t *Wd, const int32_t *splits,
                            const int32_t *dst_off, float *bufs, uint32_t *pads, int W,
                            int rank, int ne, int64_t H, int64_t F, int64_t rows_in,
                            int64_t rows_out, void *stream);

/* Status of rank `rank`'s pad after the work queued on `stream` (synchronizes
 * it): *code := GSA_ESPLIT (then *tile := the smallest bad local expert),
 * else GSA_ESTATE (*tile := smallest e * tiles + t with an unusable own
 * row), else GSA_ETIMEOUT (*tile, *peer := smallest expired (e * tiles + t,
 * peer)), else GSA_OK (*tile = *peer = -1).  Errors: GSA_EINVAL, GSA_EHIP. */
int gsa_a2a_status(const uint32_t *pads, int rank, void *stream, int *code, int64_t *tile,
                   int *peer);

#ifdef __cplusplus
}
#endif

#endif /* GSA_H */
