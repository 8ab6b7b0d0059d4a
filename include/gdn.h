/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule library: the
 * chunked forward, the single-token decode step and the chunked backward.
 *
 * The operation (the "gated delta rule"):
 *
 *   S_t = S_{t-1} ( D_t (I - beta_t k_t k_t^T) ) + beta_t v_t k_t^T ,
 *   o_t = S_t (scale * q_t)
 *
 * with D_t = exp(g_t) I for the scalar gate (Gated DeltaNet: page
 * "TileLang 实战：KDA 从零到一--Gated DeltaNet", introduction and §2.3;
 * page "Gated Delta Network（GDN）", eq. 4) or D_t = Diag(exp(g_t)) for the
 * per-key-channel gate (Kimi Delta Attention: page "DeltaNet 系列线性注意力
 * 变体的推导之旅", KDA section).  g is the natural log of the gate
 * (g <= 0 for a decaying state).  The state is stored transposed,
 * h = S^T with shape [K, V], as the pages' kernels store it ("TileLang 实战"
 * §3.0; "Gated Delta Network（GDN）" §4.1(d): [B, H, K, V]).
 *
 * The output of step t reads the state after token t's own write.  q and k are
 * used as given: L2 normalisation is the caller's precondition ("TileLang
 * 实战" §0 and §1.2), unless the *_act entry points are asked to normalise
 * them (GDN_ACT_QK_L2NORM below).  beta is used as given (normally in (0, 1);
 * any value in (0, 2) gives the write a negative eigenvalue 1 - beta), unless
 * the *_act entry points are asked to activate it (gdn_activation below).
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is device memory owned by the caller (any memory
 *    a gfx950 kernel can read or write).  The library never allocates,
 *    never keeps a pointer after returning and never synchronises.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *    Outputs are valid once that stream has reached the enqueued work;
 *    inputs must stay unchanged until then.  Outputs must not alias inputs,
 *    except where an entry point says so.
 *  - All shape and pointer checks happen before the first launch, so a call
 *    that returns an error status has enqueued nothing and written nothing.
 *  - Non-finite input values propagate; they are not checked.
 *  - All entry points are reentrant and thread-safe.
 *  - Layouts are dense row-major with the shapes given.  Alignment: q, k, v,
 *    o of the chunked forward and the decode state need 16 bytes (they are
 *    moved in 16-byte vectors); cu_seqlens needs 8; every other tensor its
 *    element size; the workspace 256.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 9

typedef int32_t gdn_status;
enum {
    GDN_OK = 0,
    GDN_ERR_NULL_ARG = 1,        /* a required pointer is NULL */
    GDN_ERR_BAD_SHAPE = 2,       /* negative/zero sizes, B != 1 with cu_seqlens, ... */
    GDN_ERR_BAD_DTYPE = 3,       /* unknown dtype or gate code */
    GDN_ERR_UNSUPPORTED = 4,     /* chunk != 64; K, V not in {64,128} */
    GDN_ERR_WORKSPACE_TOO_SMALL = 5,
    GDN_ERR_MISALIGNED = 6,      /* a pointer lacks the alignment stated below */
    GDN_ERR_HIP = 7,             /* a kernel launch failed; see gdn_last_error() */
    GDN_ERR_BAD_SEQLENS = 8      /* packed offsets invalid: found on the device, read
                                    through gdn_seqlens_status_offset (never returned
                                    by a compute call, which does not wait for it) */
};

/* element type of q, k, v and o */
enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 };
/* gate shape: one log-gate per (token, head), or one per (token, head, key) */
enum { GDN_GATE_SCALAR = 0, GDN_GATE_PER_KEY = 1 };

/* Shape of a chunked (prefill) forward call. */
typedef struct gdn_fwd_desc {
    int64_t batch;      /* B; must be 1 when cu_seqlens is given */
    int64_t seq_len;    /* T: tokens per sequence, or all packed tokens */
    int64_t num_heads;  /* H */
    int64_t key_dim;    /* K, in {64, 128} */
    int64_t value_dim;  /* V, in {64, 128} */
    int64_t num_seqs;   /* N packed sequences when cu_seqlens is given, else 0 */
    int32_t chunk;      /* C: 64; see "Chunk size" below */
    int32_t qkv_dtype;  /* GDN_DTYPE_* of q, k, v, o */
    int32_t gate;       /* GDN_GATE_* */
    float scale;        /* multiplies q (usually 1/sqrt(K)) */
    int64_t num_v_heads;  /* H_V value heads (0: H_V = H); see GVA below */
} gdn_fwd_desc;

/*
 * Chunk size.  Only the 64-token tiling is built.  The pages allow 16, 32 and
 * 64 ("Gated Delta Network（GDN）" §4.1(d)); every entry point returns
 * GDN_ERR_UNSUPPORTED for any chunk other than 64, before launching anything.
 * (The chunked form reaches the recurrence's result whatever the chunk size,
 * "TileLang 实战" §2.3, so a caller asking for 16 or 32 loses nothing but
 * rounding order by passing 64.)
 */

/* Shape of a single-token (decode) step over N independent sequences. */
typedef struct gdn_step_desc {
    int64_t num_seqs;   /* N */
    int64_t num_heads;  /* H */
    int64_t key_dim;    /* K, in {64, 128} */
    int64_t value_dim;  /* V, in {64, 128} */
    int32_t qkv_dtype;  /* GDN_DTYPE_* of q, k, v, o */
    int32_t gate;       /* GDN_GATE_* */
    float scale;
    int64_t num_v_heads;  /* H_V value heads (0: H_V = H); see GVA below */
} gdn_step_desc;

/*
 * GVA, grouped value heads ("Gated Delta Network（GDN）" §5): q and k have H
 * heads, v has H_V = m H heads (m a positive integer) and the state is kept
 * per value head.  Value head hv reads q/k head hv / m (integer division),
 * like grouped-query attention.  Everything that belongs to a state -- v, o,
 * beta, g, h0, ht, A_log, dt_bias -- has H_V heads; the shapes below then read
 * H_V wherever the head count of those tensors appears.
 */

/*
 * Optional in-kernel input activation ("Gated Delta Network（GDN）" §3.1,
 * eq. 5: log alpha = -e^{A_log} softplus(W_alpha x + b_alpha), beta =
 * sigmoid(W_beta x); §5: the activation fused into the chunk kernel, and
 * beta in (0, 2) for negative eigenvalues).  With a flag set, the matching
 * input holds the raw logits instead of the activated values:
 *   GDN_ACT_GATE          g = a (raw):  log alpha = -exp(A_log[h]) * softplus(a + dt_bias)
 *                         with dt_bias[h] for the scalar gate and
 *                         dt_bias[h][kc] (key channel kc) for the per-key gate
 *   GDN_ACT_BETA_SIGMOID  beta = sigmoid(b)
 *   GDN_ACT_BETA_NEG_EIG  with GDN_ACT_BETA_SIGMOID: beta = 2 sigmoid(b), in
 *                         (0, 2), so the eigenvalue 1 - beta of the write
 *                         ranges over (-1, 1)
 *   GDN_ACT_QK_L2NORM     q and k are L2-normalised per token and head as
 *                         they are read: x / sqrt(sum_K x^2 + 1e-6) ("TileLang
 *                         实战" §1.2: unit-norm keys keep the write's
 *                         eigenvalues in [-1, 1]; the pages fix no epsilon)
 * A_log [H] and dt_bias ([H] or [H, K]) are float device arrays, required
 * with GDN_ACT_GATE and otherwise ignored.  Unknown bits, or NEG_EIG without
 * BETA_SIGMOID, give GDN_ERR_UNSUPPORTED.  Every flag runs on both prefill
 * routes; the workspace does not depend on the activation.
 */
enum { GDN_ACT_GATE = 1, GDN_ACT_BETA_SIGMOID = 2, GDN_ACT_BETA_NEG_EIG = 4, GDN_ACT_QK_L2NORM = 8 };
typedef struct gdn_activation {
    int32_t flags;           /* GDN_ACT_* */
    const float *A_log;      /* [H] */
    const float *dt_bias;    /* [H] (scalar gate) or [H, K] (per-key gate) */
} gdn_activation;

/*
 * Where a packed call leaves its check of cu_seqlens in the workspace (byte
 * offset from the workspace start, written to *offset): an int32 that the
 * call's chunk-table kernel sets to 0 when the offsets start at 0, never
 * decrease and end at seq_len, and to 1 otherwise (invalid offsets are also
 * clamped into [0, seq_len], so they never cause an access out of bounds;
 * the results are then undefined).  backward = 0: gdn_chunk_fwd[_act] with
 * *act (NULL allowed), gdn_chunk_intra and gdn_chunk_scan use the
 * two-stage layout's word, which is the same unless the call ran as the
 * single-pass kernel; backward = 1: gdn_chunk_bwd[_act].  The word is valid
 * once the call's stream has reached it; reading it is the caller's (a
 * debugging aid: it needs a wait on the stream).  d must describe packed
 * input (num_seqs > 0).
 */
gdn_status gdn_seqlens_status_offset(const gdn_fwd_desc *d, const gdn_activation *act,
                                     int32_t backward, size_t *offset);

/*
 * Where the single-pass kernel of gdn_chunk_fwd[_act] reports a failed
 * hand-off between its waves (byte offset from the workspace start, written
 * to *offset).  The waves of one workgroup pass each chunk's products to
 * each other through flags in local memory; every wait for a flag polls a
 * bounded number of times (about 2^16 polls, several milliseconds, against a
 * chunk step of a few microseconds), so a wave never waits forever.  A wait
 * that gives up sets this int32 to 1 (the call's results are then wrong) and
 * leaves it at 1: the library never clears it.  A caller that wants to know
 * clears it before the call (e.g. allocates the workspace zeroed) and reads
 * it once the stream has reached the call.  d (with *act, NULL allowed) must
 * describe a shape that runs the single-pass kernel (bf16, scalar gate,
 * K and V each 64 or 128, chunk 64); other shapes run the two-stage route,
 * which has no such waits, and give GDN_ERR_UNSUPPORTED.
 */
gdn_status gdn_sync_status_offset(const gdn_fwd_desc *d, const gdn_activation *act,
                                  size_t *offset);

/* Integer version of this ABI (GDN_ABI_VERSION), for binding checks. */
int gdn_abi_version(void);

/* Static name of a status code (never NULL). */
const char *gdn_status_str(gdn_status s);

/* Detail of the last failing call on this thread (never NULL, may be ""). */
const char *gdn_last_error(void);

/*
 * Bytes of device workspace gdn_chunk_fwd needs for the shape *d (written to
 * *bytes).  A descriptor with num_seqs > 0 describes packed input.
 *   - bf16 inputs, scalar gate, K and V each 64 or 128, chunk 64 (the
 *     single-pass kernel): the per-sequence table of packed input, 16 bytes per
 *     sequence and one more record rounded up to 256 (256 bytes without
 *     cu_seqlens), then 256 bytes that hold the synchronisation status word
 *     of gdn_sync_status_offset.
 *   - every other shape (two stages): the per-chunk products of the
 *     intra-chunk stage and the chunk table, gdn_workspace_layout_of().total.
 * gdn_chunk_intra and gdn_chunk_scan always need
 * gdn_workspace_layout_of().total.
 */
gdn_status gdn_chunk_fwd_workspace(const gdn_fwd_desc *d, size_t *bytes);

/* The same for gdn_chunk_fwd_act with the activation *act (NULL: exactly
 * gdn_chunk_fwd_workspace; no flag changes the size at present). */
gdn_status gdn_chunk_fwd_workspace_act(const gdn_fwd_desc *d, const gdn_activation *act,
                                       size_t *bytes);

/*
 * Chunked forward pass ("TileLang 实战" §2.2.4-2.3: UT transform and gated
 * chunk equations 11-12; "阅读笔记：DeltaNet 在 FLA 中的代码实现笔记",
 * forward Steps 1-5; signature of its chunk_delta_rule_fwd: q, k, v, beta,
 * scale, initial_state, output_final_state, cu_seqlens).
 *
 * bf16 inputs with the scalar gate, K and V each 64 or 128, chunk 64 run as
 * one kernel that builds each chunk's intra-chunk products on chip while it
 * carries the state; every other shape runs gdn_chunk_intra then
 * gdn_chunk_scan.  The two routes compute the same quantities in a
 * different order: they agree to rounding, not bit for bit.
 *
 *   q, k   [B, T, H, K]   qkv_dtype
 *   v      [B, T, H, V]   qkv_dtype
 *   beta   [B, T, H]      float
 *   g      [B, T, H] (GDN_GATE_SCALAR) or [B, T, H, K] (GDN_GATE_PER_KEY),
 *          float, natural-log gate
 *   h0     [N, H, K, V]   float, initial state; NULL means zeros
 *   cu_seqlens  NULL, or int64 [num_seqs + 1] on the device: packed sequence
 *          offsets, starting at 0, nondecreasing, ending at T (B must be 1).
 *          Chunks restart at every sequence start and every sequence starts
 *          from its own h0 ("Gated Delta Network（GDN）", terminology note:
 *          a chunk boundary is not a sequence boundary).  Offsets are
 *          checked on the device without stopping the call: bad offsets
 *          give undefined results (never an access out of bounds) and set
 *          the word of gdn_seqlens_status_offset.
 *   o      [B, T, H, V]   qkv_dtype, output
 *   ht     [N, H, K, V]   float, final state; NULL means not returned.
 *          ht may equal h0 (in-place carry); no other aliasing is allowed.
 *   N = B without cu_seqlens, num_seqs with it.
 *   workspace, workspace_bytes: device scratch of at least
 *          gdn_chunk_fwd_workspace() bytes, 256-byte aligned.
 */
gdn_status gdn_chunk_fwd(const gdn_fwd_desc *d,
                         const void *q, const void *k, const void *v,
                         const float *beta, const float *g, const float *h0,
                         const int64_t *cu_seqlens,
                         void *o, float *ht,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * gdn_chunk_fwd with the input activation applied inside the kernels (act
 * may be NULL: then exactly gdn_chunk_fwd).  Rows past the end of a
 * sequence are never activated: they stay outside every result.
 */
gdn_status gdn_chunk_fwd_act(const gdn_fwd_desc *d, const gdn_activation *act,
                             const void *q, const void *k, const void *v,
                             const float *beta, const float *g, const float *h0,
                             const int64_t *cu_seqlens,
                             void *o, float *ht,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * gdn_chunk_fwd_act without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It runs the single-pass kernel only:
 * d must describe bf16 q/k/v, the scalar gate, K and V each 64 or 128,
 * chunk 64, and at most GDN_NOALLOC_MAX_SEQS packed sequences; other shapes
 * give GDN_ERR_UNSUPPORTED before anything is launched.  Arguments, layouts and
 * results are those of gdn_chunk_fwd_act (act may be NULL).
 * Its scratch (the per-sequence records of packed input) is a device array
 * inside the library, about 66 KB, one per GPU, held until the process
 * ends; its address on the current device is looked up on the first call on
 * that device.  The call itself allocates nothing.  Every call on one GPU
 * uses the same scratch: calls that may overlap on one GPU (on different
 * streams, or from several threads without ordering) race and give wrong
 * results; calls ordered on one stream do not.  The device-side check of
 * cu_seqlens and the synchronisation status word of gdn_chunk_fwd are not
 * reported by this entry point.
 */
#define GDN_NOALLOC_MAX_SEQS 4096
gdn_status gdn_chunk_fwd_noalloc(const gdn_fwd_desc *d, const gdn_activation *act,
                                 const void *q, const void *k, const void *v,
                                 const float *beta, const float *g, const float *h0,
                                 const int64_t *cu_seqlens,
                                 void *o, float *ht, void *stream);

/*
 * Where gdn_chunk_intra / gdn_chunk_scan (and the two-stage route of
 * gdn_chunk_fwd) keep each intermediate inside the
 * workspace (byte offsets from its start).  Every per-chunk array is indexed
 * [head][chunk][...] with max_chunks chunk slots per head; chunk j of
 * sequence b is slot b * ceil(T / C) + j without cu_seqlens, and slot
 * (first chunk of the sequence) + j with it.  With G the inclusive cumulative
 * log2 gate inside the chunk and gamma = 2^G:
 *   gcum  float [H][mc][C]  (scalar gate) or [H][mc][C][K] (per-key gate): G;
 *         with the per-key gate only row C-1 (G at the chunk's last token,
 *         the decay of the carried state) is written
 *   w     [H][mc] x (C x K)  W = (I+A)^{-1} diag(beta) diag(gamma) K      F
 *   u     [H][mc] x (C x V)  U = (I+A)^{-1} diag(beta) V                  A
 *   qs    [H][mc] x (C x K)  scale * diag(gamma) Q                        F
 *   ks    [H][mc] x (K x C)  (diag(gamma_C / gamma) K)^T                  F
 *   aqk   [H][mc] x (C x C)  scale * (Q K^T masked by Gamma, diagonal kept)  F
 *   ainv  float [H][mc][C][C]  (I+A)^{-1}, row-major; written only by
 *                           gdn_chunk_intra
 *   chunks int32 [mc][4]    (first token, token count, sequence, 0) per chunk
 *                           slot (packed input only)
 *   seqs  int32 [N][4]      (first token, length, first chunk slot, order[n])
 *                           (packed input only); order[r] = the sequence of
 *                           rank r by length, longest first (ties by index;
 *                           order[r] = r above 1024 sequences): the serial
 *                           passes take their workgroups in that order
 * A = strictLower(diag(beta) (Gamma * K K^T)), Gamma_ij = 2^(G_i - G_j) for
 * j <= i.  w, u, qs, ks and aqk have the element type qkv_dtype.  For the
 * per-key gate gamma is per channel and every Gamma factor sits inside the
 * sum over the key channel.  A descriptor with num_seqs > 0 describes packed
 * input.
 *
 * Element order of an R x D block X (the orders the MFMA instructions of the
 * state pass read without rearranging):
 *   F (fragment order): 16-byte groups of 64 lanes; group (rt, sg), rt <
 *     R/16, sg < D/KG, lane l, element e < VE holds X[16 rt + l%16][KG sg + c]
 *     at element ((rt * D/KG + sg) * 64 + l) * VE + e, with c = 8 (l/16) + e,
 *     KG = 32, VE = 8 for bf16 and c = 4 e + l/16, KG = 16, VE = 4 for fp32.
 *   A (accumulator order): tile (rt, ct), rt < R/16, ct < D/16, lane l,
 *     element e < 4 holds X[16 rt + 4 (l/16) + e][16 ct + l%16] at element
 *     ((rt * D/16 + ct) * 64 + l) * 4 + e.
 * Rows of W and U past the end of a ragged last chunk are zero; there the
 * rows of qs and aqk and the columns of ks repeat the chunk's last token and
 * never reach an output.
 */
typedef struct gdn_workspace_layout {
    size_t gcum, w, u, qs, ks, aqk, ainv, chunks, seqs;
    size_t total;        /* bytes the two stages need */
    int64_t max_chunks;  /* chunk slots per head (mc) */
} gdn_workspace_layout;

gdn_status gdn_workspace_layout_of(const gdn_fwd_desc *d, gdn_workspace_layout *out);

/*
 * The two stages of the forward pass, callable one at a time, for every
 * supported shape (for shapes without the single-pass kernel gdn_chunk_fwd
 * is exactly gdn_chunk_intra(flags = 0) followed by gdn_chunk_scan on the
 * same workspace and stream).  The workspace holds
 * gdn_workspace_layout_of().total bytes.
 *
 * gdn_chunk_intra: the intra-chunk stage ("TileLang 实战" §2.2.4, §2.3 and
 * §4.1-4.2; "阅读笔记：DeltaNet 在 FLA 中的代码实现笔记", forward Steps 1-3):
 * cumulative gates, the beta-scaled decay-masked strictly-lower K K^T, its
 * unit-lower inverse, W, U, Qs, Ks and the causal Q K^T block, left in the
 * workspace as gdn_workspace_layout_of describes.  With
 * flags & GDN_INTRA_STORE_AINV the inverse (I+A)^{-1} is written too (for
 * checking the stage; gdn_chunk_fwd does not write it).  Arguments as for
 * gdn_chunk_fwd.
 */
#define GDN_INTRA_STORE_AINV 1
gdn_status gdn_chunk_intra(const gdn_fwd_desc *d,
                           const void *q, const void *k, const void *v,
                           const float *beta, const float *g,
                           const int64_t *cu_seqlens,
                           void *workspace, size_t workspace_bytes,
                           int32_t flags, void *stream);

/*
 * gdn_chunk_scan: the inter-chunk state pass with the chunk output ("TileLang
 * 实战" §2.3 eqs. 11-12; "Gated Delta Network（GDN）" §4.1(d); "阅读笔记"
 * forward Steps 4-5), serial over the chunks of each sequence:
 *   V_new = U - W h,  o = Qs h + Aqk V_new,  h <- gamma_C h + Ks^T V_new.
 * The workspace must hold what gdn_chunk_intra left there for the same
 * descriptor, inputs and cu_seqlens (which is only used to know the number
 * of sequences; the chunk table comes from the workspace).  h0, o, ht as for
 * gdn_chunk_fwd.
 */
gdn_status gdn_chunk_scan(const gdn_fwd_desc *d, const float *h0,
                          const int64_t *cu_seqlens, void *o, float *ht,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode token for N independent sequences: the recurrent form used
 * when a single new token arrives ("Gated Delta Network（GDN）" §4.4,
 * eq. 12; "DeltaNet 系列线性注意力变体的推导之旅", fused recurrent kernel:
 * forget, predict, correct, read).
 *
 *   q, k   [N, H, K]   qkv_dtype
 *   v      [N, H, V]   qkv_dtype
 *   beta   [N, H]      float
 *   g      [N, H] or [N, H, K]   float, natural-log gate
 *   state  [N, H, K, V]  float, read and updated in place
 *   o      [N, H, V]   qkv_dtype, output
 */
gdn_status gdn_recurrent_step(const gdn_step_desc *d,
                              const void *q, const void *k, const void *v,
                              const float *beta, const float *g,
                              float *state, void *o, void *stream);

/* gdn_recurrent_step with the input activation (act may be NULL). */
gdn_status gdn_recurrent_step_act(const gdn_step_desc *d, const gdn_activation *act,
                                  const void *q, const void *k, const void *v,
                                  const float *beta, const float *g,
                                  float *state, void *o, void *stream);

/*
 * Backward pass of the chunked forward ("阅读笔记：DeltaNet 在 FLA 中的代码实现
 * 笔记", 二、反向传播, Steps 1-6, written there for the ungated DeltaNet; the
 * gate enters by the chain rule through the same chunked forward).  Given
 * the gradient dout of o and dht of ht, it writes the gradients of
 * L = <dout, o> + <dht, ht> with respect to q, k, v, beta, g and h0.  The
 * forward quantities (U, W, the chunk entry states) are recomputed from the
 * inputs, as the pages' Steps 1-2 do; nothing is kept from a forward call.
 * With the per-key-channel gate (GDN_GATE_PER_KEY) every decay ratio of those
 * steps sits inside the sum over the key channel, as in the chunkwise KDA
 * section of "DeltaNet 系列线性注意力变体的推导之旅"; the carried state
 * gradient then decays row by row and dg is per channel.
 *
 *   q, k, v, beta, g, h0, cu_seqlens, scale: as for gdn_chunk_fwd
 *   dout       [B, T, H, V]  qkv_dtype
 *   dht        [N, H, K, V]  float, or NULL: no final-state gradient
 *   dq, dk     [B, T, H, K]  qkv_dtype, written
 *   dv         [B, T, H, V]  qkv_dtype, written
 *   dbeta      [B, T, H]     float, written
 *   dg         [B, T, H] or [B, T, H, K] (the shape of g)  float, written: the
 *              gradient of the natural-log gate
 *   dh0        [N, H, K, V]  float, written, or NULL: not computed
 *
 * Supported: chunk 64, grouped value heads (see GVA above: v, dv, beta,
 * dbeta, g, dg, h0, dht, dh0 have H_V heads; q, k, dq, dk have H, and dq, dk
 * of a q/k head sum the terms of its H_V/H value heads); bf16 q/k/v with K, V
 * in {64, 128} for either gate; fp32 with K = V = 64 for the scalar gate.
 * Other shapes give GDN_ERR_UNSUPPORTED.  dout, dq, dk, dv need 16-byte alignment.
 * The workspace (gdn_chunk_bwd_workspace bytes, 256-byte aligned) holds the
 * recomputed per-chunk quantities, the chunk entry states and the state
 * gradients; its contents on return are unspecified.  No output may alias an
 * input or another output.
 */
gdn_status gdn_chunk_bwd_workspace(const gdn_fwd_desc *d, size_t *bytes);
gdn_status gdn_chunk_bwd(const gdn_fwd_desc *d,
                         const void *q, const void *k, const void *v,
                         const float *beta, const float *g, const float *h0,
                         const int64_t *cu_seqlens,
                         const void *dout, const float *dht,
                         void *dq, void *dk, void *dv, float *dbeta, float *dg, float *dh0,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_chunk_bwd with the input activation applied inside the kernels, as
 * gdn_chunk_fwd_act does it (act may be NULL: then exactly gdn_chunk_bwd).
 * The gradients of the activated inputs are carried to the raw ones by the
 * chain rule of "Gated Delta Network（GDN）" §3.1 eq. 5 (x = a + dt_bias[h]):
 *   dg     d/da = dlog_alpha * (-exp(A_log[h]) * sigmoid(x))   with GDN_ACT_GATE
 *   dbeta  d/db = dbeta_act * m sigmoid(b) sigmoid(-b)          with GDN_ACT_BETA_SIGMOID
 *          (m = 2 with GDN_ACT_BETA_NEG_EIG, else 1)
 *   dA_log   [H_V] float, written with GDN_ACT_GATE (required then):
 *            sum over the tokens (and, per-key gate, the channels) of
 *            dlog_alpha * log_alpha
 *   ddt_bias [H_V] ([H_V, K] for the per-key gate) float, written with
 *            GDN_ACT_GATE (required then): sum over the tokens of d/da
 * Both are ignored without GDN_ACT_GATE.  With GDN_ACT_QK_L2NORM, dq and dk
 * are the gradients of the raw q and k: the normalisation's chain rule
 * dx = (dy - x (x.dy) / n2) / sqrt(n2), n2 = sum_K x^2 + 1e-6, is applied to
 * the gradients of the normalised rows.  The per-key gate takes dt_bias
 * [H_V, K] and applies the chain rule per channel; the rest is as for
 * gdn_chunk_bwd, with the same workspace.
 */
gdn_status gdn_chunk_bwd_act(const gdn_fwd_desc *d, const gdn_activation *act,
                             const void *q, const void *k, const void *v,
                             const float *beta, const float *g, const float *h0,
                             const int64_t *cu_seqlens,
                             const void *dout, const float *dht,
                             void *dq, void *dk, void *dv, float *dbeta, float *dg, float *dh0,
                             float *dA_log, float *ddt_bias,
                             void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
