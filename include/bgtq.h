/*
 * bgtq.h -- C ABI of the Block-GTQ packed-cache decode path for AMD MI355X (gfx950).
 *
 * Method: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (Liang, Zhang,
 * Jia; arXiv 2606.24033), abstract.  Per layer and KV head the method scores
 * the energy of every 2-D RoPE frequency block, hands out integer bit widths
 * greedily by marginal gain under a matched K bit budget, quantizes keys with
 * TurboQuant-MSE at those widths and values at a uniform width, and serves
 * decode attention from the packed cache.  The four calls below are those
 * steps.  Where the abstract leaves a detail open, the reading is stated at
 * the call.
 *
 * Conventions for every call
 *   - All tensors are device memory owned by the caller; the library never
 *     allocates or frees device memory and keeps no per-call state.  The one
 *     device memory it owns is the static scratch array of
 *     bgtq_decode_step_noalloc (part of the code object, one per GPU).
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     null stream) and the call returns without waiting.
 *   - Arguments are validated on the host before anything is enqueued; a bad
 *     argument returns an error status and enqueues nothing.  A failed launch
 *     returns BGTQ_ERR_HIP.  bgtq_last_error() gives a message for the last
 *     failure on the calling thread.  No call aborts or throws.
 *   - Strides are in elements.  fp16 data is IEEE binary16 stored as uint16.
 *   - Call bgtq_init() once per device before capturing calls in a HIP graph;
 *     otherwise the first call on a device initialises it (a synchronous copy
 *     of the codebook tables to device constant memory).
 *   - Two process-wide options exist for tests and diagnosis (bgtq_set_option);
 *     the first initialisation reads their defaults from the environment once.
 */
#ifndef BGTQ_H
#define BGTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BGTQ_OK = 0,
  BGTQ_ERR_INVALID_ARG = 1,   /* null pointer, bad size, stride or enum */
  BGTQ_ERR_BUDGET = 2,        /* k_width_sum outside [n*b_min, n*b_max], or b_max > 8 */
  BGTQ_ERR_CAPACITY = 3,      /* capacity too small for the request */
  BGTQ_ERR_WORKSPACE = 4,     /* workspace missing or smaller than required */
  BGTQ_ERR_UNSUPPORTED = 5,   /* valid but not built: head_dim, GQA group size */
  BGTQ_ERR_HIP = 6            /* the HIP runtime reported an error */
} bgtq_status;

typedef enum { BGTQ_F32 = 0, BGTQ_BF16 = 1 } bgtq_dtype;

/* Which two coordinates form RoPE block j (the abstract speaks of 2-D
 * frequency blocks but fixes no coordinate layout): HALF pairs (j, j + d/2) as Llama/Qwen checkpoints do,
 * INTERLEAVED pairs (2j, 2j + 1). */
typedef enum { BGTQ_PAIR_HALF = 0, BGTQ_PAIR_INTERLEAVED = 1 } bgtq_pairing;

typedef void* bgtq_stream;

/* Library limits. */
#define BGTQ_MAX_HEAD_DIM 256
#define BGTQ_MAX_BITS 8
#define BGTQ_MAX_GROUP 16        /* query heads per KV head */
#define BGTQ_TILE 64             /* token slots per cache tile */
#define BGTQ_LAYOUT_BYTES 4096   /* size of one per-head layout descriptor */
#define BGTQ_MAX_WINDOW 4096     /* tokens in the fp16 recent-key window */

/* Rotation kinds.  The abstract builds on TQ-MSE, which rotates before scalar coding, and
 * fixes no rotation type.  DENSE: one Haar matrix per size (m x m multiply-adds per
 * vector).  GIVENS: a structured rotation per size m, a product of layers that each rotate
 * the pairs of a perfect matching of the m coordinates by their own angle, O(m log m) per
 * vector.  The two give different codes; a cache is written and read with one kind. */
typedef enum { BGTQ_ROT_DENSE = 0, BGTQ_ROT_GIVENS = 1 } bgtq_rotation;

/* Random rotations the quantizer draws (TQ-MSE rotates before scalar coding).
 * Device memory, caller-owned, read-only, shared by all layers and heads.
 *   rot_bank:   Haar matrices for the key width groups, m = 2, 4, ..., head_dim,
 *               each m x m row-major (y = R x), concatenated in that order
 *               (bgtq_rotation_bank_floats(head_dim) floats).
 *   rot_v:      head_dim x head_dim row-major rotation for values.
 *   rot_bank_t, rot_v_t: the same matrices transposed (each block column-major),
 *               written by bgtq_transpose_rotations; kernels that form one
 *               output row per lane read these so that a wavefront's loads are
 *               contiguous.
 *   (the four matrices are read with rotation = BGTQ_ROT_DENSE and may be NULL otherwise)
 *   givens      with rotation = BGTQ_ROT_GIVENS: uint32 rows of 4.  Rows 0..127 are a
 *               header, row m/2 - 1 = (first record row of size m, layer count L_m, 0, 0)
 *               for every even m <= head_dim; a record row is (a | b << 16, fp32 bits of
 *               c, fp32 bits of s, 0), and size m has L_m layers of m/2 records, layer by
 *               layer.  Layer l maps y_a = c x_a - s x_b, y_b = s x_a + c x_b for each of
 *               its pairs (a, b), which must form a perfect matching of 0..m-1; every
 *               product, difference and sum is rounded to fp32 (no fused multiply-add), so
 *               codes are reproducible bit for bit.  Values use size head_dim.  Keys are
 *               rotated per width group in storage order. */
typedef struct {
  const float* rot_bank;
  const float* rot_v;
  const float* rot_bank_t;
  const float* rot_v_t;
  int head_dim;
  bgtq_rotation rotation;
  const uint32_t* givens;
} bgtq_quantizer;

/* Floats in a rotation bank for head_dim (sum of m*m over even m <= head_dim), 0 if
 * head_dim is not a supported even size. */
size_t bgtq_rotation_bank_floats(int head_dim);

/* Writes the transposed copies a bgtq_quantizer carries: every m x m block of
 * rot_bank transposed into rot_bank_t (same offsets), rot_v into rot_v_t.
 * All device pointers, caller-owned; rot_bank_t and rot_v_t must not overlap the
 * inputs.  Enqueued on `stream`.  Errors: INVALID_ARG, HIP. */
bgtq_status bgtq_transpose_rotations(const float* rot_bank, const float* rot_v, int head_dim,
                                     float* rot_bank_t, float* rot_v_t, bgtq_stream stream);

/* Packed K/V cache of one layer for a batch of sequences.  All pointers are
 * device memory the caller allocates (sizes from bgtq_cache_bytes) and owns.
 * Region of sequence s, KV head h = [s * n_kv_heads + h] of each array.
 * With tiles = capacity / 64 and chunks = ceil(2 * k_width_sum / 128):
 *   k_codes  uint8  [batch][n_kv_heads][tiles][chunks][64][16]
 *            slot j of a tile holds the token's K record: its codes in storage
 *            order, LSB first, code p at record bits [offset_p, offset_p+w_p).
 *   k_norms  fp16   [batch][n_kv_heads][tiles][8][64]  width-group norms.
 *   v_codes  uint8  [batch][n_kv_heads][tiles][head_dim][8*v_bits]
 *            rotated coordinate r of a tile is a 64*v_bits-bit segment; slot j
 *            holds its code at bits [j*v_bits, (j+1)*v_bits).
 *   v_norms  fp16   [batch][n_kv_heads][tiles][64].
 *   lengths  int32  [batch]  tokens cached per sequence; advanced by
 *            bgtq_quantize_append.  The caller sets it (normally 0) at start.
 *   widths   uint8  [batch][n_kv_heads][head_dim/2], layouts
 *            [batch][n_kv_heads][BGTQ_LAYOUT_BYTES]: written by
 *            bgtq_allocate_bits at prefill and read by the other calls.
 *   status   int32  [1], nullable: a kernel sets bit 0 when an append would
 *            pass capacity (that append is then skipped for that sequence), and
 *            bit 1 when a decode step's attention pass gave up waiting for its
 *            own append (a bounded wait; that step's output is not to be trusted).
 *   window, k_window  the fp16 recent-key window (abstract: the AIME run is stated to be
 *            without an fp16 recent-key buffer, so the serving path has one as an option).
 *            Reading: the keys of the newest `window` tokens of a sequence, t in
 *            [lengths[s] - window, lengths[s]), are also kept as fp16 (nearest-even,
 *            saturated at +-65504) and attention uses them in place of their quantized
 *            reconstruction; their values stay quantized.  window = 0 turns it off
 *            (k_window may then be NULL); otherwise 1 <= window <= BGTQ_MAX_WINDOW and
 *            k_window is fp16 [batch][n_kv_heads][window][head_dim], token t of a sequence
 *            at slot t mod window.  Every token is still quantized into the packed arrays.
 * Unused slots may hold anything; only slots below lengths[s] are read. */
typedef struct {
  int batch;
  int n_kv_heads;
  int head_dim;
  int k_width_sum;      /* B = sum of block widths = (K bits per coordinate) * head_dim/2 */
  int v_bits;           /* 1..8 */
  int64_t capacity;     /* token slots per sequence, multiple of 64 */
  bgtq_pairing pairing;
  uint8_t* k_codes;
  uint16_t* k_norms;
  uint8_t* v_codes;
  uint16_t* v_norms;
  int32_t* lengths;
  uint8_t* widths;
  void* layouts;
  int32_t* status;
  int32_t window;       /* fp16 recent-key window in tokens; 0 = none */
  uint16_t* k_window;
} bgtq_cache;

/* Energy score of every RoPE block, computed from keys alone (abstract: one
 * score per block, per layer and KV head, with no labels needed).
 * Reading: E_j = (1/T) * sum_t (k[t,a_j]^2 + k[t,b_j]^2) over the given keys,
 * in fp64, summed in ascending t inside chunks of 256 tokens and then over the
 * chunks in ascending order (a fixed order, so the result is reproducible).
 *   keys        [n_heads] x [n_tokens] x [head_dim] of `dtype` with strides
 *               (stride_head, stride_token, 1); post-RoPE keys are fine, RoPE
 *               does not change block norms.
 *   energy_out  fp64 [n_heads][head_dim/2].
 *   workspace   >= bgtq_energy_workspace_bytes(n_heads, n_tokens, head_dim).
 * Errors: INVALID_ARG (null, n_tokens < 1, odd or oversized head_dim),
 * WORKSPACE, HIP. */
bgtq_status bgtq_block_energy(const void* keys, bgtq_dtype dtype, int n_heads, int64_t n_tokens,
                              int head_dim, int64_t stride_head, int64_t stride_token,
                              bgtq_pairing pairing, double* energy_out, void* workspace,
                              size_t workspace_bytes, bgtq_stream stream);
size_t bgtq_energy_workspace_bytes(int n_heads, int64_t n_tokens, int head_dim);

/* Greedy integer bit widths by marginal gain (abstract: integer widths are
 * handed out one bit at a time to the block that gains most, so blocks with
 * more energy end up with more bits; the K budget equals that of uniform
 * TQ-MSE).
 * Reading: all blocks start at b_min; k_width_sum - n*b_min times, one bit goes
 * to the block with the largest gain E_j * (D(b_j) - D(b_j + 1)) among blocks
 * below b_max, ties to the lowest j, where D(b) = fl32(MSE of the b-bit
 * Lloyd-Max quantizer of N(0,1)) and D(0) = 1; gains are fp64.
 *   energy       fp64 [n_heads][head_dim/2] (device), e.g. from bgtq_block_energy.
 *   widths_out   uint8 [n_heads][head_dim/2].
 *   layouts_out  [n_heads][BGTQ_LAYOUT_BYTES]: width groups (descending width,
 *                blocks ascending), storage order and bit offsets.
 * Errors: INVALID_ARG, BUDGET (k_width_sum infeasible or 0 > b_min > b_max > 8),
 * HIP. */
bgtq_status bgtq_allocate_bits(const double* energy, int n_heads, int head_dim, int k_width_sum,
                               int b_min, int b_max, bgtq_pairing pairing, uint8_t* widths_out,
                               void* layouts_out, bgtq_stream stream);

/* TQ-MSE quantize-and-pack of new tokens (abstract: the method uses
 * TurboQuant-MSE as its base quantizer, and its serving path keeps the cache
 * packed).
 * Reading (width-group TQ-MSE): blocks of equal width w >= 1 form one vector of
 * m = 2*|group| coordinates coded at w bits: fp32 norm n (sequential sum of
 * squares, sqrt), y = R_m x (sequential, no fused multiply-add), z = (y/n)*fl32(sqrt(m)),
 * code = #{k : z > T_w[k]} with the fp32 Lloyd-Max thresholds of N(0,1);
 * norm stored fp16 (nearest-even, saturated).  Values: one group of m =
 * head_dim with rot_v at v_bits.  Codes, norms and packed bytes are
 * reproducible bit for bit.
 * Appends n_new tokens to each sequence s in [seq_begin, seq_begin + n_seqs):
 * token i of s goes to slot lengths[s] + i, then lengths[s] += n_new.  With a window,
 * the appended tokens that end up among the newest `window` also get their fp16 key
 * written to the window.
 *   keys, values  [n_seqs][n_kv_heads][n_new][head_dim] of `dtype` with strides
 *                 (stride_seq, stride_head, stride_token, 1); keys post-RoPE.
 * The sequence's widths/layouts must already be written by bgtq_allocate_bits.
 * Errors: INVALID_ARG, CAPACITY (n_new > capacity; an overflow that depends on
 * the device lengths is reported through cache->status instead), HIP. */
bgtq_status bgtq_quantize_append(const bgtq_quantizer* qz, const bgtq_cache* cache, int seq_begin,
                                 int n_seqs, const void* keys, const void* values, bgtq_dtype dtype,
                                 int64_t n_new, int64_t stride_seq, int64_t stride_head,
                                 int64_t stride_token, bgtq_stream stream);

/* Prefill of one sequence: the method's three steps in one call (abstract: per layer and
 * KV head, block energies from the keys, greedy integer widths under the K budget, TQ-MSE
 * quantization into the packed cache).  The result equals bgtq_block_energy over the given
 * keys, bgtq_allocate_bits with the cache's k_width_sum (widths and layouts of sequence
 * `seq`), then bgtq_quantize_append of the tokens to `seq`, bit for bit; the energies' final
 * reduction and the allocation run in one kernel.  Keys are read twice (energy, then
 * quantization): no width is known before every key has been scored.
 *   keys, values  [n_kv_heads][n_tokens][head_dim] of dtype with strides
 *                 (stride_head, stride_token, 1); keys post-RoPE.
 *   energy_out    nullable fp64 [n_kv_heads][head_dim/2].
 *   workspace     >= bgtq_prefill_workspace_bytes(n_kv_heads, n_tokens, head_dim).
 * Errors: those of the three calls. */
bgtq_status bgtq_prefill(const bgtq_quantizer* qz, const bgtq_cache* cache, int seq, const void* keys,
                         const void* values, bgtq_dtype dtype, int64_t n_tokens, int64_t stride_head,
                         int64_t stride_token, int b_min, int b_max, double* energy_out, void* workspace,
                         size_t workspace_bytes, bgtq_stream stream);
size_t bgtq_prefill_workspace_bytes(int n_kv_heads, int64_t n_tokens, int head_dim);

/* Decode attention straight from the packed cache (abstract: RoPE query-key
 * logits; the serving path attends over a packed K3V3 cache at 128K context).
 * For every sequence s and query head h (KV head h / (n_q_heads/n_kv_heads)):
 * q' = RoPE(q[s][h], pos) with angles pos*rope_theta^(-2j/d) formed and reduced
 * modulo 2*pi in fp64;
 * logits l_t = softmax_scale * q' . k_hat_t over the cached slots t <
 * lengths[s]; out = sum_t softmax(l)_t * v_hat_t, with k_hat, v_hat the TQ-MSE
 * reconstructions (width-0 blocks are zero).  The packed codes are decoded in
 * registers; the query is rotated into each width group's frame instead of
 * un-rotating every key, and the value rotation is undone once per head.
 *   q           [batch][n_q_heads][head_dim] of q_dtype, pre-RoPE (contiguous).
 *   q_pos       int64 [batch] (device) query positions, or NULL for
 *               lengths[s] - 1 (the newest cached token).
 *   rope_theta  RoPE base; <= 0 means q is already rotated.
 *   out         fp32 [batch][n_q_heads][head_dim]; must not overlap q (the attention
 *               pass clears it before the merge adds the heads' halves into it).
 *   logits_out  nullable fp32 [batch][n_q_heads][capacity]; slots >= lengths[s]
 *               are left untouched.
 *   workspace   >= bgtq_decode_workspace_bytes(...); must be zero-filled before
 *               its first use; every call leaves it ready for the next.
 * With a window, the logits of the newest min(window, lengths[s]) tokens use their fp16
 * keys, q' . k16_t, instead of k_hat_t; the softmax runs over all tokens at once.
 * A sequence with lengths[s] == 0 gets out = 0.
 * Errors: INVALID_ARG, UNSUPPORTED (group size > 16, head_dim not 64/128/256; with a
 * window, group size > 8), WORKSPACE, HIP. */
bgtq_status bgtq_decode_attention(const bgtq_quantizer* qz, const bgtq_cache* cache, int n_q_heads,
                                  const void* q, bgtq_dtype q_dtype, const int64_t* q_pos,
                                  double rope_theta, float softmax_scale, float* out,
                                  float* logits_out, void* workspace, size_t workspace_bytes,
                                  bgtq_stream stream);
size_t bgtq_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                   int64_t capacity);

/* One decode step (abstract: the serving path decodes token by token from the packed
 * cache): for every sequence s of the cache, quantize and append one new key/value
 * token, then attend with q at that token's position.  The result equals
 * bgtq_quantize_append(n_new = 1, all sequences) followed by
 * bgtq_decode_attention(q_pos = NULL), cache contents, lengths, status and out
 * included.  The append runs beside the attention pass, in the same launch; only the
 * part of the pass that reads the new token's tile waits for it (a flag in the workspace,
 * zero between calls).
 *   keys, values  [batch][n_kv_heads][head_dim] of kv_dtype, element (s, h, c) at
 *                 s * stride_seq + h * stride_head + c.
 *   q, out, logits_out, workspace: as for bgtq_decode_attention (the same workspace
 *   size serves both calls).
 * A sequence whose append would exceed the capacity sets cache->status, keeps its
 * length and is attended without the new token.
 * Errors: those of the two calls it stands for. */
bgtq_status bgtq_decode_step(const bgtq_quantizer* qz, const bgtq_cache* cache, int n_q_heads,
                             const void* q, bgtq_dtype q_dtype, const void* keys, const void* values,
                             bgtq_dtype kv_dtype, int64_t stride_seq, int64_t stride_head,
                             double rope_theta, float softmax_scale, float* out, float* logits_out,
                             void* workspace, size_t workspace_bytes, bgtq_stream stream);

/* bgtq_decode_step for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It takes no workspace:
 * the split partials and the step flags live in a library-owned device array of
 * BGTQ_NOALLOC_SCRATCH_BYTES per GPU (held until the process ends).  The call allocates
 * nothing; it clears the step flags with a small kernel, then runs the same kernels as
 * bgtq_decode_step, so the results are the same bit for bit.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (different streams, or different host
 * threads without ordering) race and give undefined results.  Arguments as for
 * bgtq_decode_step, minus the workspace.
 * Errors: those of bgtq_decode_step; WORKSPACE when bgtq_decode_workspace_bytes for the
 * cache exceeds BGTQ_NOALLOC_SCRATCH_BYTES. */
#define BGTQ_NOALLOC_SCRATCH_BYTES (32u << 20)
bgtq_status bgtq_decode_step_noalloc(const bgtq_quantizer* qz, const bgtq_cache* cache, int n_q_heads,
                                     const void* q, bgtq_dtype q_dtype, const void* keys,
                                     const void* values, bgtq_dtype kv_dtype, int64_t stride_seq,
                                     int64_t stride_head, double rope_theta, float softmax_scale,
                                     float* out, float* logits_out, bgtq_stream stream);

/* Key-only logit error (abstract: Block-GTQ is judged on how well it keeps the RoPE
 * query-key logits, as the per-layer mean absolute logit error when only keys are quantized,
 * at 2 and 3 bits per coordinate, against uniform TQ-MSE at the same budget).
 * For every sequence s and query head h (KV head h / (n_q_heads/n_kv_heads)), with
 * T_s = min(lengths[s], capacity): q' = RoPE(q[s][h], pos) as in bgtq_decode_attention (fp64
 * angles reduced modulo 2*pi), exact logits e_t = softmax_scale * q' . k_t from the unquantized
 * post-RoPE keys, and
 *     mae_out[s][h] = (1/T_s) * sum_{t < T_s} |logits[s][h][t] - e_t|   (0 when T_s == 0),
 * where `logits` is what bgtq_decode_attention wrote to logits_out for the same q, q_pos,
 * rope_theta and softmax_scale over the quantized cache.  The exact logits are fp32 products
 * and sums; the absolute errors are summed in fp64 in a fixed order (reproducible).
 *   q           [batch][n_q_heads][head_dim] of q_dtype, pre-RoPE (contiguous).
 *   q_pos       int64 [batch] (device) or NULL for lengths[s] - 1.
 *   keys        post-RoPE keys of k_dtype, element (s, h, t, c) at
 *               s * stride_seq + h * stride_head + t * stride_token + c; tokens t < T_s are read.
 *               Strides must be multiples of 4 and the pointer 16-byte aligned (8 for bf16).
 *   lengths     int32 [batch] (device), e.g. the cache's lengths.
 *   logits      fp32 [batch][n_q_heads][capacity], 16-byte aligned.
 *   mae_out     fp64 [batch][n_q_heads].
 *   workspace   >= bgtq_logit_error_workspace_bytes(batch, n_q_heads, capacity); no
 *               initial contents needed.
 * Errors: INVALID_ARG, UNSUPPORTED (head_dim not 64/128/256, group size > 16), WORKSPACE, HIP. */
bgtq_status bgtq_logit_error(const void* q, bgtq_dtype q_dtype, const int64_t* q_pos, const void* keys,
                             bgtq_dtype k_dtype, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                             int64_t stride_seq, int64_t stride_head, int64_t stride_token,
                             const int32_t* lengths, int64_t capacity, bgtq_pairing pairing,
                             double rope_theta, float softmax_scale, const float* logits, double* mae_out,
                             void* workspace, size_t workspace_bytes, bgtq_stream stream);
size_t bgtq_logit_error_workspace_bytes(int batch, int n_q_heads, int64_t capacity);

/* Bytes of each cache array for the given geometry (k_codes, k_norms, v_codes,
 * v_norms, in that order, written to out4); returns the total, 0 if invalid. */
size_t bgtq_cache_bytes(int batch, int n_kv_heads, int head_dim, int k_width_sum, int v_bits,
                        int64_t capacity, size_t* out4);

/* The frozen fp32 Lloyd-Max tables and fl32(D(b)) the kernels use, copied to host
 * memory: thresholds[2^bits - 1], centroids[2^bits], *distortion (bits 0..8;
 * bits 0 has no tables).  Host-only, enqueues nothing. */
bgtq_status bgtq_codebook(int bits, float* thresholds, float* centroids, double* distortion);

/* Copy the frozen tables to the current device's constant memory (synchronous) and
 * look up the device's allocation-free scratch (bgtq_decode_step_noalloc).  The first
 * call in the process also reads the options' defaults from the environment:
 * BGTQ_DECODE_KERNEL=valu (tiled) sets BGTQ_OPT_DECODE_KERNEL to 1 (2), BGTQ_STEP_SPIN_LIMIT=n sets
 * BGTQ_OPT_STEP_WAIT_LIMIT to n.  Nothing reads the environment afterwards. */
bgtq_status bgtq_init(void);

/* Process-wide options, for tests and diagnosis; every later call reads the value set
 * last.  Not meant to change while calls are in flight on other threads.
 *   BGTQ_OPT_DECODE_KERNEL    0 (default): the decode runs on the matrix cores when the
 *                             group size is <= 8 (the streamed pass where it serves the
 *                             cache geometry, the tiled one otherwise), on the vector ALU
 *                             otherwise; 1: always on the vector ALU (then a cache with a
 *                             window is refused: UNSUPPORTED); 2: matrix cores, always
 *                             the tiled pass.
 *   BGTQ_OPT_STEP_WAIT_LIMIT  bound of a decode step's wait for its own append, in polls
 *                             of a few hundred cycles (default 1 << 22, about 0.2 s;
 *                             0: no wait, so the step reports through cache->status that
 *                             it gave up, which is how that report is tested).
 * Errors: INVALID_ARG (unknown option or value out of range). */
typedef enum { BGTQ_OPT_DECODE_KERNEL = 0, BGTQ_OPT_STEP_WAIT_LIMIT = 1 } bgtq_option;
bgtq_status bgtq_set_option(bgtq_option option, int64_t value);
int64_t bgtq_get_option(bgtq_option option);

const char* bgtq_status_string(bgtq_status s);
const char* bgtq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BGTQ_H */
