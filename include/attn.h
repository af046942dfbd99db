/*
 * attn.h -- C ABI of the blockwise online-softmax attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Scaled dot-product attention forward,
 *     out = softmax(Q K^T / sqrt(d) + mask) V,
 * ("Transformers and Attention" digest, reference #22 Attention Is All You
 * Need and #24 PyTorch scaled_dot_product_attention) one key/value tile at a
 * time with online softmax: a running row max, a running denominator and a
 * rescaled weighted sum per query row (brunomaga.github.io
 * sequence-context-parallelism post, sections "Ring Attention" and "Improving
 * numerical stability").  Partial results over disjoint key blocks are
 * carried as (out, lse) and merged, which is the per-device work of Ring
 * Attention ("CP: Split Long Contexts Across GPUs", section "Circulate K/V
 * blocks with Ring").
 *
 * Conventions shared by every entry point.
 *  - Layout: q and out are (B, Tq, H, d); k and v are (B, Tkv, H, d); all
 *    contiguous, row-major, the layout the pages' ring code hands to its
 *    attention kernel.  lse is (B, H, Tq) float32, natural log.
 *  - Positions: query row i has absolute position q_off + i, key j has
 *    kv_off + j.  They drive the causal test and the rotary embedding.
 *  - Masks: nonzero = excluded.  kpm is (B, Tkv) uint8 (ignored source
 *    entries per batch item), attn_mask is (Tq, Tkv) uint8 (forbidden
 *    (query, key) pairs, shared over B and H).  Exclusions combine with each
 *    other and with causal order ("Transformers and Attention" #2).
 *  - A row with no allowed key yields out = 0 and lse = -inf, so that
 *    (0, -inf) is the identity of attn_merge.
 *  - Ownership: every pointer is caller-owned device memory (except where a
 *    host pointer is stated).  Some calls need device scratch.  Each entry
 *    point below states it in bytes as a formula of its sizes ("Scratch:");
 *    every term is rounded up to a multiple of 256 bytes.  Entry points
 *    without a "Scratch:" line use none.  The scratch comes from a buffer the
 *    library keeps per (device, stream) and reuses from call to call: it is
 *    allocated stream-ordered (hipMallocAsync) by the first call that needs
 *    it, replaced by a larger one (the old one freed in stream order) when a
 *    call needs more, rounded up to 2 MiB, and kept until
 *    attn_release_scratch.  A call holds its stream's buffer while it
 *    enqueues, so calls on one stream from several host threads take turns.
 *    Under stream capture (graph allocation nodes) and on the per-thread
 *    default stream (hipStreamPerThread) a call allocates its scratch
 *    stream-ordered and frees it after its last launch instead, and leaves
 *    the kept buffers alone.
 *  - Streams: every call only enqueues work on `stream` (NULL = the null
 *    stream) and returns; there is no host synchronisation inside, except
 *    that a call which must replace its stream's scratch buffer by a larger
 *    one frees the old buffer in stream order, which can wait for the
 *    stream's earlier work (once per growth), a call with scratch on the
 *    per-thread default stream can wait likewise when it frees it, and
 *    attn_release_scratch waits for the device.
 *  - Errors: arguments are validated on the host before any HIP call; a call
 *    that fails validation returns ATTN_ERR_INVALID_ARG or
 *    ATTN_ERR_UNSUPPORTED, enqueues nothing, and attn_last_error() describes
 *    the problem (thread-local string).  A failed scratch allocation (device
 *    memory exhausted) or kernel launch returns ATTN_ERR_HIP; an allocation
 *    failure happens before the call's first launch, a launch failure may
 *    leave the call's earlier launches enqueued.  Faults during execution
 *    surface at the caller's next synchronisation.
 */
#ifndef BOSA_ATTN_H
#define BOSA_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* attn_stream_t; /* the same type as hipStream_t */

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad flag combination */
    ATTN_ERR_UNSUPPORTED = 2, /* head dim other than 64/128, unknown dtype */
    ATTN_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

enum {
    /* out/lse already hold a partial result (float32 out); merge this call's
     * result into them in place instead of overwriting.  Requires OUT_F32. */
    ATTN_ACCUMULATE = 1u,
    /* out is float32 (a partial kept for merging) rather than the input dtype. */
    ATTN_OUT_F32 = 2u,
    /* debugging aid: visit every key tile, also the fully masked ones; the
     * results are bit-identical to the default. */
    ATTN_NO_TILE_SKIP = 4u
};

/*
 * attn_fwd -- one attention forward call over one key/value block.
 *
 * Follows: "Transformers and Attention" #22/#24 (definition, 1/sqrt(d)
 * scale, causal triangle with the diagonal), #2 (key-padding and attention
 * masks, exclusions combined), #4 (rotary embedding of q and k);
 * brunomaga.github.io post, "Improving numerical stability" (running max,
 * rescale of both accumulators by exp of the max difference, LogSumExp) and
 * "Implementation" (each ring step produces block_out and block_lse).
 *
 *  q, k, v    device, dtype `dtype`, layouts above.  k and v must not alias out.
 *  out        device, (B, Tq, H, d): dtype `dtype`, or float32 with ATTN_OUT_F32.
 *  lse        device float32 (B, H, Tq); may be NULL unless ATTN_ACCUMULATE.
 *  B, H, Tq, Tkv  sizes >= 0 (B, H or Tq = 0: nothing to do; Tkv = 0: every
 *             row is empty).  d: 64 or 128.
 *  q_off, kv_off  absolute position of row 0 of q and of k/v; |q_off|,
 *             |kv_off| <= 2^52 (ATTN_ERR_INVALID_ARG otherwise).
 *  causal     nonzero: key j is allowed for query i only if kv_off+j <= q_off+i.
 *  kpm        device uint8 (B, Tkv) or NULL.  attn_mask: device uint8 (Tq, Tkv) or NULL.
 *  rope_base  > 0: rotate adjacent coordinate pairs (2t, 2t+1) of q and k by
 *             pos * rope_base^(-2t/d) (angle, cos, sin and rotation in
 *             float64) and round the rotated values once, to nearest even,
 *             to `dtype` before the dot product.  0: no rotary embedding.  A
 *             float64 angle carries an absolute error that grows with the
 *             position: about 1e-4 rad near position 2^40, tenths of a
 *             radian near 2^52.
 *  dtype      ATTN_BF16 (bf16 MFMA, float32 accumulation and softmax) or
 *             ATTN_F32 (float32 throughout).
 *  flags      ATTN_ACCUMULATE | ATTN_OUT_F32 | ATTN_NO_TILE_SKIP.
 * Scratch:    with rope_base > 0 and Tkv > 0: in bf16 the rotated copies of k
 *             and q, 2 * B * (Tkv + Tq) * H * d (the kernel streams
 *             rotated operands; the rotation computes its own cos and sin);
 *             in float32 the float64 (cos, sin) tables (Tq + Tkv) * (d/2) * 16.
 *             In bf16 with kpm (without ATTN_NO_TILE_SKIP) the live key-tile
 *             list, 4 * B * (ceil(Tkv / 64) + 2).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int H, int Tq, int Tkv, int d,
             long long q_off, long long kv_off, int causal,
             const uint8_t* kpm, const uint8_t* attn_mask,
             double rope_base, int dtype, unsigned flags, attn_stream_t stream);

/*
 * Variants of an attention call ("Transformers and Attention" #55 Longformer:
 * sliding-window attention connects each token to nearby positions; #58
 * ALiBi: a penalty proportional to the query-key distance, with a fixed
 * slope per head, added to the scores before the softmax).  The pages' ring
 * step passes the same two knobs to its attention kernel as a (left, right)
 * window and per-head slopes (brunomaga.github.io post, "Implementation").
 *
 *  window_left   a key is allowed only if pos_k >= pos_q - window_left;
 *                -1 = no limit.  Combines with causal order and the masks.
 *  window_right  a key is allowed only if pos_k <= pos_q + window_right;
 *                -1 = no limit.
 *  alibi_slopes  device float32 [H], or NULL: the score of every allowed pair
 *                becomes q.k / sqrt(d) - slope_h * |pos_q - pos_k| (absolute
 *                positions); lse includes the penalty.
 */
typedef struct attn_variant {
    long long window_left;
    long long window_right;
    const float* alibi_slopes;
} attn_variant;

/*
 * attn_fwd_ex -- attn_fwd with a sliding window and/or ALiBi slopes.
 *
 * Same arguments and conventions as attn_fwd, plus `var` (host pointer,
 * read during the call; NULL = attn_fwd).  Windows must be >= -1.  Tiles
 * outside every row's window are skipped like fully masked tiles.
 * Scratch: as attn_fwd.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                int B, int H, int Tq, int Tkv, int d,
                long long q_off, long long kv_off, int causal,
                const uint8_t* kpm, const uint8_t* attn_mask,
                double rope_base, int dtype, unsigned flags,
                const attn_variant* var, attn_stream_t stream);

/*
 * attn_kv_append -- one decoding step's cache update: append the new token's
 * key and value to a static key/value cache.
 *
 * "Transformers and Attention" #53 (causal key/value caching: each step
 * computes the new token's key and value and appends them to the layer's
 * cache) and #57 (a static cache preallocates its slots; unused slots are
 * masked).
 *
 *  k_new, v_new  device (B, H, d) of dtype `dtype` (4-byte aligned for bf16,
 *                8-byte for float32).
 *  k_cache, v_cache  device (B, Tcap, H, d), same dtype and alignment; slot j
 *                of row b holds the token at position j.
 *  cache_len     device int32 [B], read and written: slot L = cache_len[b]
 *                receives the token, then cache_len[b] = L + 1.  A row with
 *                L >= Tcap (full) or L < 0 is left unchanged -- nothing is
 *                written past the last slot; the caller keeps L < Tcap.
 *  rope_base     > 0: the key is stored rotated to position L (the rotation
 *                and rounding of attn_fwd), so cached keys are rotated once.
 *  d             64 or 128.
 */
int attn_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, int* cache_len,
                   int B, int H, int Tcap, int d, double rope_base, int dtype, attn_stream_t stream);

/*
 * attn_decode -- attention of each row's newest token over its cache.
 *
 * "Transformers and Attention" #53: the new query attends over the retained
 * and the current keys and values (work proportional to the cached length);
 * #57: windowed layers retain a bounded history.  The keys are split into
 * chunks folded in parallel into partial (out, lse) results, merged as
 * attn_merge does.
 *
 *  q            device (B, H, d), the query of the token at position
 *               cache_len[b] - 1 (its key and value already appended), not
 *               rotated: with rope_base > 0 it is rotated here.  16-byte aligned.
 *  k_cache, v_cache  device (B, Tcap, H, d) as filled by attn_kv_append
 *               (keys stored rotated); 16-byte aligned.
 *  cache_len    device int32 [B], values clamped to [0, Tcap]; slots
 *               [0, cache_len[b]) are visible.  Causal order holds by
 *               construction (no slot after the query is filled).
 *  out          device (B, H, d): dtype `dtype`, or float32 with ATTN_OUT_F32.
 *  lse          device float32 (B, H), or NULL.  A row with no visible slot
 *               gives out = 0, lse = -inf.
 *  var          NULL, or window_left (only the slots at most that many
 *               positions before the query) and alibi_slopes as for
 *               attn_fwd_ex; window_right has no effect (nothing after the
 *               query is filled).
 *  flags        0 or ATTN_OUT_F32.
 * Scratch: the chunks' partial results, 4 * B * H * n * d + 4 * B * H * n
 * with n = the number of chunks, at most ceil(8192 / (B * H)): below
 * 4 * (d + 1) * (8192 + B * H) in all.
 */
int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int* cache_len,
                void* out, float* lse, int B, int H, int Tcap, int d, double rope_base, int dtype,
                unsigned flags, const attn_variant* var, attn_stream_t stream);

/*
 * attn_decode_noalloc -- attn_decode that allocates nothing, for callers that
 * cannot allocate device memory during the call: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results and kernels as attn_decode (bit for bit).  The
 * chunk partials go to a static workspace of 16 MiB that the library holds on
 * every device it runs on until the process ends (its address is looked up on
 * the first call on a device).  A call whose partials need more
 * (4 * B * H * n * (d + 1) bytes with n chunks as for attn_decode; about
 * B * H > 24000 at d = 128) returns ATTN_ERR_UNSUPPORTED and enqueues
 * nothing.  Every call on one device shares that device's workspace: calls
 * that may overlap on one device (different streams without ordering, or
 * several host threads) race and must be serialised by the caller.
 */
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* cache_len,
                        void* out, float* lse, int B, int H, int Tcap, int d, double rope_base, int dtype,
                        unsigned flags, const attn_variant* var, attn_stream_t stream);

/*
 * attn_merge -- (out_a, lse_a) <- (out_a, lse_a) (+) (out_b, lse_b), in place.
 *
 * The pages call an accumulate step after every ring step without defining
 * it (brunomaga.github.io post, "Implementation"); this is the combination
 * the fraction form and LogSumExp carry imply ("Ring Attention", "Improving
 * numerical stability"): lse = logaddexp(lse_a, lse_b),
 * out = e^(lse_a - lse) out_a + e^(lse_b - lse) out_b.  Never a plain sum or
 * average ("CP: Split Long Contexts Across GPUs", "Circulate K/V blocks with
 * Ring").  (0, -inf) is the identity; the operation is commutative bit for bit.
 *
 *  out_a      device float32 (B, Tq, H, d), read and written.
 *  lse_a      device float32 (B, H, Tq), read and written.
 *  out_b      device (B, Tq, H, d) of dtype b_dtype.  lse_b: device float32 (B, H, Tq).
 *  d          any positive multiple of 4.
 */
int attn_merge(float* out_a, float* lse_a, const void* out_b, const float* lse_b,
               int B, int H, int Tq, int d, int b_dtype, attn_stream_t stream);

/*
 * rope_apply -- rotary position embedding of x in place.
 *
 * "Transformers and Attention" #4 (RoFormer): an even-dimensional vector is
 * split into coordinate pairs, each rotated by a positional angle, so that a
 * rotated query and key interact through their position difference only.
 * Pair (2t, 2t+1) of token i is rotated by pos[i] * base^(-2t/d):
 * (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a), computed in float64
 * and rounded once, to nearest even, to `dtype`.
 *
 *  x          device (B, T, H, d) of dtype `dtype`, rotated in place.
 *  pos        device int64 [T]: absolute position of each token (shared over B and H).
 *  base       > 0.  d: even, <= 256.
 */
int rope_apply(void* x, const long long* pos, double base, int B, int T, int H, int d,
               int dtype, attn_stream_t stream);

/*
 * attn_cast -- dst[i] = (dst_dtype) src[i] for i < n, round-to-nearest-even.
 * The last step of a ring share: the float32 accumulator becomes the
 * output in the input dtype (brunomaga.github.io post, "Implementation":
 * the accumulated output is cast to the dtype of q at the end).
 */
int attn_cast(const float* src, void* dst, long long n, int dst_dtype, attn_stream_t stream);

/*
 * Ring-attention share on one device.
 *
 * One rank of a P-rank ring keeps its query rows and meets every key/value
 * block in ring order: its own block first, then the block of rank-1,
 * rank-2, ... mod P ("CP: Split Long Contexts Across GPUs", "Circulate K/V
 * blocks with Ring"; brunomaga.github.io post, "Distributed algorithm").
 * Placement is contiguous (rank r owns tokens [r T/P, (r+1) T/P)) or zigzag
 * (rank r owns chunks r and 2P-1-r of size T/(2P), "Balance the workload in
 * causal attention").  Under zigzag, each (query chunk, key chunk) pair of a
 * step is one attn_fwd sub-call; pairs that causal order masks completely
 * are not issued.
 *
 * attn_ring_plan -- host-only bookkeeping (no HIP call).  Fills up to `cap`
 * entries of `plan` (host memory) in issue order and returns the number of
 * sub-calls, or a negative attn_status on bad arguments.
 */
typedef struct {
    int step;          /* ring step 0..P-1 */
    int block;         /* rank whose K/V block is used at this step */
    int q_row0;        /* first local query row of the sub-call */
    int q_rows;        /* number of local query rows */
    long long q_pos0;  /* absolute position of local row q_row0 */
    long long kv_pos0; /* absolute position (= row in the full K/V) of the first key */
    int kv_rows;       /* number of keys */
    int accumulate;    /* 1: merge into the partial already held for these rows */
} attn_ring_call;

int attn_ring_plan(int T, int P, int rank, int zigzag, int causal, attn_ring_call* plan, int cap);

/*
 * attn_ring_fwd -- execute a rank's ring share.
 *
 *  q          device (B, Tq_local, H, d) local query rows, Tq_local = T/P,
 *             in local order (zigzag: chunk r then chunk 2P-1-r).
 *  k, v       device (B, T, H, d): every block, at its absolute position (one
 *             device emulates the arriving blocks; nothing is copied).
 *  out        device (B, Tq_local, H, d) of `dtype`: the final output.
 *  lse        device float32 (B, H, Tq_local): the final log-sum-exp.
 *  acc        device float32 (B, Tq_local, H, d) scratch for the running partial
 *             (may equal out when dtype is ATTN_F32).
 *  kpm        device uint8 (B, T) or NULL, over absolute key positions.
 *  Other arguments as attn_fwd.  The work is the sub-calls of attn_ring_plan,
 *  issued in order on `stream`, each writing or merging its partial into acc,
 *  then one attn_cast of acc into out.  In bf16 (without window or ALiBi) up
 *  to sixteen consecutive sub-calls of one query block run in one kernel launch
 *  that carries each row's softmax state across them (so they act as one key
 *  sequence in ring order) and writes or merges one partial per launch; the
 *  last launch of a query block writes out directly.  out and lse then equal
 *  one attn_fwd call per launch over that launch's keys in ring order, and
 *  one attn_fwd call per sub-call up to rounding.  With RoPE the call rotates
 *  every key block and the local queries once into scratch copies.
 * Scratch:    with rope_base > 0: in bf16 the rotated keys and local queries,
 *             2 * B * (T + T/P) * H * d; in float32 the float64 (cos, sin)
 *             table over the T positions, T * (d/2) * 16.  In bf16 with kpm
 *             (without ATTN_NO_TILE_SKIP) one live key-tile list per
 *             sub-call, 4 * B * (ceil(c / 64) + 2) each, c = the sub-call's
 *             key rows (T/P, or T/(2P) under zigzag).  The 128K zigzag share
 *             (B = 1, H = 32, d = 128, T = 131072, P = 8) with RoPE:
 *             1 GiB + 128 MiB.
 */
int attn_ring_fwd(const void* q, const void* k, const void* v, void* out, float* lse, float* acc,
                  int B, int H, int T, int d, int P, int rank, int zigzag, int causal,
                  const uint8_t* kpm, double rope_base, int dtype, unsigned flags,
                  attn_stream_t stream);

/*
 * attn_ring_fwd_ex -- attn_ring_fwd with a sliding window and/or ALiBi slopes
 * (`var` as for attn_fwd_ex, host pointer read during the call; NULL =
 * attn_ring_fwd).  Sub-calls whose key block lies outside the window of
 * every query of their block are not issued: with a window the share needs
 * only the blocks near its queries ("Transformers and Attention" #55: with a
 * fixed window the number of interactions grows linearly with length).
 */
int attn_ring_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse, float* acc,
                     int B, int H, int T, int d, int P, int rank, int zigzag, int causal,
                     const uint8_t* kpm, double rope_base, int dtype, unsigned flags,
                     const attn_variant* var, attn_stream_t stream);

/*
 * attn_bwd -- attention backward: gradients of L = sum(dout * out) for the
 * attn_fwd call with the same q, k, v, positions, masks and rotary base.
 *
 * Follows the backward pass of the brunomaga.github.io post ("Ring Attention",
 * item 3: gradients computed blockwise, never storing the attention matrix;
 * "Implementation": each ring step computes the block gradients of the local
 * queries against the current K/V block from dout, q, k, v, the final out and
 * the saved log-sum-exp; dq accumulates locally, dk and dv accumulate with
 * their block).  With P = exp(s - lse) on allowed pairs and
 * delta_i = sum_c dout_ic out_ic:  dv_j = sum_i P_ij dout_i,
 * dS_ij = P_ij (dout_i . v_j - delta_i),  dq_i = sum_j dS_ij k_j / sqrt(d),
 * dk_j = sum_i dS_ij q_i / sqrt(d), with q, k rotated when rope_base > 0 and
 * dq, dk rotated back (the rotation is orthogonal).
 *
 *  q, dout, out  device (B, Tq, H, d) bf16; out is the final forward output.
 *  k, v          device (B, Tkv, H, d) bf16.
 *  lse           device float32 (B, H, Tq): the forward's log-sum-exp over
 *                every key the rows see (not a block partial).
 *  dq            device (B, Tq, H, d); dk, dv device (B, Tkv, H, d): bf16,
 *                or float32 with ATTN_OUT_F32.  ATTN_ACCUMULATE (needs
 *                ATTN_OUT_F32) adds the gradients into dq, dk and dv instead
 *                of overwriting them, as a ring step does with its
 *                accumulators.
 *  dtype         ATTN_BF16 only (ATTN_ERR_UNSUPPORTED otherwise).
 *  flags         ATTN_ACCUMULATE | ATTN_OUT_F32 | ATTN_NO_TILE_SKIP.
 *  Rows with no allowed key contribute nothing; keys with kpm set get zero
 *  gradients.  Results are deterministic (every output element is written by
 *  one workgroup).
 * Scratch:       the per-row (lse, delta) pairs, 8 * B * H * Tq; with
 *                rope_base > 0 the float64 (cos, sin) tables
 *                (Tq + Tkv) * (d/2) * 16 and the rotated q and k,
 *                2 * B * (Tq + Tkv) * H * d; the float32 dq,
 *                4 * B * H * d * Tq, unless the call writes float32
 *                gradients without RoPE (then the kernels write dq, dk, dv
 *                directly); the float32 dk and dv, 8 * B * H * d * Tkv, only
 *                when it writes float32 gradients with RoPE (bf16 dk and dv
 *                are written by the dK/dV kernel itself); with kpm (without
 *                ATTN_NO_TILE_SKIP) the live key-tile list,
 *                4 * B * (ceil(Tkv / 64) + 2).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv,
             int B, int H, int Tq, int Tkv, int d, long long q_off, long long kv_off, int causal,
             const uint8_t* kpm, const uint8_t* attn_mask, double rope_base, int dtype, unsigned flags,
             attn_stream_t stream);

/*
 * attn_bwd_ex -- attn_bwd for a call made with attn_fwd_ex: the same window
 * and ALiBi slopes (`var`, host pointer read during the call; NULL =
 * attn_bwd).  The penalty enters P only (it does not depend on q or k) and
 * the window removes pairs like a mask, so the gradients are those of the
 * forward definition with the variant ("Transformers and Attention" #55, #58).
 */
int attn_bwd_ex(const void* q, const void* k, const void* v, const void* out, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int B, int H, int Tq, int Tkv, int d,
                long long q_off, long long kv_off, int causal, const uint8_t* kpm,
                const uint8_t* attn_mask, double rope_base, int dtype, unsigned flags,
                const attn_variant* var, attn_stream_t stream);

/*
 * attn_ring_bwd -- backward of a rank's ring share (the inverse of
 * attn_ring_fwd): the sub-calls of attn_ring_plan, each computing the block
 * gradients of the local rows against one K/V block, with dq accumulated over
 * the blocks and dk, dv accumulated at the block's absolute positions (the
 * pages rotate these accumulators with their block; one device holds them in
 * place).  The rotation back and the cast happen once at the end.
 *
 *  q, out, dout  device (B, T/P, H, d) bf16, local rows in local order.
 *  lse           device float32 (B, H, T/P) from attn_ring_fwd.
 *  k, v          device (B, T, H, d) bf16, every block at its position.
 *  dq            device (B, T/P, H, d); dk, dv device (B, T, H, d): bf16, or
 *                float32 with ATTN_OUT_F32.  dk and dv receive this rank's
 *                contributions only (keys no local row sees get 0).
 *  flags         ATTN_OUT_F32 | ATTN_NO_TILE_SKIP.  Other arguments as
 *                attn_ring_fwd.
 * Scratch:       the per-row (lse, delta) pairs, 8 * B * H * (T/P); the
 *                float32 gradients of the share, 4 * B * H * d * (T/P + 2 T);
 *                with rope_base > 0 the float64 (cos, sin) tables
 *                (T/P + T) * (d/2) * 16 and the rotated q and k,
 *                2 * B * (T/P + T) * H * d; with kpm (without
 *                ATTN_NO_TILE_SKIP) one live key-tile list per sub-call as
 *                for attn_ring_fwd.
 */
int attn_ring_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv,
                  int B, int H, int T, int d, int P, int rank, int zigzag, int causal,
                  const uint8_t* kpm, double rope_base, int dtype, unsigned flags,
                  attn_stream_t stream);

/*
 * attn_ring_bwd_ex -- attn_ring_bwd for a share computed by attn_ring_fwd_ex
 * with the same `var` (the same sub-calls are skipped).
 */
int attn_ring_bwd_ex(const void* q, const void* k, const void* v, const void* out, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int T, int d, int P,
                     int rank, int zigzag, int causal, const uint8_t* kpm, double rope_base, int dtype,
                     unsigned flags, const attn_variant* var, attn_stream_t stream);

/*
 * Kernel timing for measurement tools.  Between attn_profile_start and
 * attn_profile_stop, every attention-kernel launch made by attn_fwd,
 * attn_ring_fwd, attn_bwd or attn_ring_bwd on the calling thread (for the
 * backward: the dQ and the dK/dV kernel) is bracketed by a pair of HIP events
 * recorded on the launch's own stream (at most max_launches launches; later
 * ones are not timed).  attn_profile_stop waits for those events, writes the
 * duration of each timed launch in milliseconds to ms[0 .. min(n, cap)) (host
 * memory; may be NULL) and returns n, the number of timed launches, or a
 * negative attn_status.  The events are created by start and destroyed by stop.
 */
int attn_profile_start(int max_launches);
int attn_profile_stop(float* ms, int cap);

/*
 * Free the scratch buffers the library keeps for the current device (see
 * Ownership above): waits for all work on the device first, since the
 * buffers' streams may have been destroyed, then frees each buffer.  Calls
 * made afterwards allocate again.  Returns ATTN_OK or ATTN_ERR_HIP.
 */
int attn_release_scratch(void);

/* Thread-local description of the last failure ("" if none). */
const char* attn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BOSA_ATTN_H */
