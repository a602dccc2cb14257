/*
 * libllmdec: the KV-cached forward step of a LLaMA-style decoder over a paged
 * KV cache, for AMD Instinct MI355X (gfx950).
 *
 * Pages the operations follow (cited by tag):
 *   [W] "企业官网建设流程全解析" (www.dpshk.com/news/4990443), the weights
 *       article: §1.1 forward skeleton, §1.2 where parameters live, §2.x
 *       weight layout [out][in], §4.2 group-quantized weights.
 *   [F] "大模型推理全流程解析：从权重加载到文本生成的工程实践"
 *       (www.stapisi.com/news/4049481): §2.2.1 embedding, §2.2.2 attention
 *       and KV cache, §2.2.3 lm_head and greedy choice, §4 cached greedy loop.
 *   [E] "为什么要自己动手写一个LLM推理引擎" (www.wzjinhao.cn/news/61427):
 *       §3.4 KV cache sizing and paging, §4.2 RMSNorm, §4.3 attention forward
 *       with the cache, §4.4 generate loop, §5.3 preallocated cache pool and
 *       sampling on the device.
 *
 * Conventions for every function below.
 *  - Pointers marked "dev" are device pointers; "host" are host pointers.
 *  - The caller owns all memory (weights, packed weights, hidden states, the
 *    KV pool's device buffer, workspaces, ids, tables).  The library never
 *    allocates device memory; it only keeps the host-side pool handle.
 *  - Device work is enqueued on the caller's stream (a hipStream_t passed as
 *    llmdec_stream; NULL is the default stream) and the call returns after
 *    enqueueing, without synchronising.  Buffers must stay alive until the
 *    work completes.
 *  - Every call checks what the host can check before it launches anything,
 *    so a rejected call has done no work.  Status codes are returned; a
 *    thread-local message is available from llmdec_last_error().  Nothing
 *    prints, throws or aborts across this interface.
 *  - Values that only the device knows (token ids, positions, block-table
 *    entries) are range-checked inside the kernels: an out-of-range page id
 *    or position makes the kernel skip that access and set a sticky error
 *    word in the workspace, read back by llmdec_workspace_error().
 *  - bf16 means IEEE-754 binary32 truncated to its top 16 bits; rounding into
 *    bf16 is to nearest, ties to even.
 *  - Precision: weights and cached K/V are bf16 (the K/V values rounded to
 *    nearest-even when appended).  Activations entering a weight product on
 *    the matrix cores are fp16 (nearest-even; magnitudes beyond 65504 clipped
 *    to it), the compute precision of [E] §4.1's minimal engine, and multiply
 *    the weights in fp16 with fp32 accumulation: the packing carries each bf16
 *    weight exactly as an fp16 value times a power of two (see
 *    llmdec_pack_matrix).  The q|k|v product, and every product of a step of
 *    at most 64 new tokens (decode), take the activation as an fp16 pair
 *    hi + lo (about 22 bits); the o, gate/up and down products of a longer
 *    step (prefill) take one fp16 value.  The residual stream, attention
 *    (scores, softmax, weighted sum) and logits are fp32.  The products of a
 *    single-sequence decode step (one row) and those with group-quantized
 *    weights take the unrounded fp32 activation instead.
 *  - Not thread-safe per pool handle; distinct handles are independent.
 */
#ifndef LLMDEC_H
#define LLMDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LLMDEC_OK = 0,
  LLMDEC_E_INVALID = -1,     /* bad argument: null pointer, inconsistent sizes, out of range */
  LLMDEC_E_UNSUPPORTED = -2, /* valid but not built: head_dim not 64/128, page_size not 16 */
  LLMDEC_E_NO_PAGES = -3,    /* the pool cannot cover a request; nothing was changed */
  LLMDEC_E_WORKSPACE = -4,   /* workspace pointer missing or smaller than required */
  LLMDEC_E_HIP = -5          /* a HIP runtime call or kernel launch failed */
} llmdec_status;

typedef void *llmdec_stream; /* hipStream_t */

/* Model shape.  [W] §1.2 gives the 7B values: hidden 4096, 32 layers,
 * intermediate 11008, vocab 32000; [E] §3.4 gives 32 heads of 128.
 * page_size must be 16 ([E] §3.4 recommends 16 or 32 tokens per page).
 * head_dim must be 64 or 128; hidden == n_heads * head_dim; hidden and
 * intermediate must be multiples of 16.  n_kv_heads must divide n_heads:
 * with fewer K/V heads than query heads (grouped-query attention, whose
 * smaller k/v projections [W] §5.1 and the per-head K/V reshape of [E] §4.3
 * describe), query head h attends with K/V head h / (n_heads / n_kv_heads). */
typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab, page_size;
  float rms_eps;    /* added to the mean square inside the root ([E] §4.2) */
  float rope_theta; /* rotary base: pair i turns by pos * theta^(-2i/head_dim) */
} llmdec_config;

/* One layer's parameters as loaded: bf16, each matrix [out][in] row-major
 * (the nn.Linear layout of [W] §1.2).  attn_norm, mlp_norm: [hidden];
 * wq, wo: [hidden][hidden]; wk, wv: [n_kv_heads*head_dim][hidden];
 * w_gate, w_up: [intermediate][hidden]; w_down: [hidden][intermediate]. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} llmdec_layer_weights;

/* One layer re-laid out for the kernels by llmdec_pack_layer (pointers into
 * the caller's packed buffer).  Matrices are packed as llmdec_pack_matrix
 * describes; q/k/v are fused into one [hidden + 2*n_kv_heads*head_dim][hidden]
 * matrix (wq rows, then wk, then wv) and gate/up into one matrix whose 16-row
 * blocks alternate gate and up, each fused matrix with one power-of-two
 * scale. */
typedef struct {
  const void *attn_norm, *mlp_norm; /* bf16 [hidden], copied */
  const void *w_qkv, *w_o, *w_gu, *w_down;
} llmdec_packed_layer;

/* Whole model for llmdec_model_step_greedy.  embed: dev bf16 [vocab][hidden]
 * as loaded; layers: host array [n_layers] of packed layers; final_norm: dev
 * bf16 [hidden]; lm_head: dev, packed with llmdec_pack_matrix from the
 * [vocab][hidden] matrix (untied from embed). */
typedef struct {
  const void *embed;
  const llmdec_packed_layer *layers;
  const void *final_norm;
  const void *lm_head;
} llmdec_model_weights;

/* ------------------------------------------------------------------ errors */
/* Message for the last failing call on this thread ("" if none). */
const char *llmdec_last_error(void);

/* ------------------------------------------------------------------ weights */
/* Bytes of a packed rows x cols matrix (rows a multiple of 16; cols padded up
 * to a multiple of 32 with zeros): rows * round_up(cols, 32) fp16 values, then
 * a 256-byte trailer. */
size_t llmdec_packed_matrix_bytes(int32_t rows, int32_t cols);
/* Re-lay a dev bf16 [rows][cols] matrix into dev dst (>= packed_matrix_bytes).
 * The tiles hold fp16(w * 2^s) in the tile order of "Packed activations"
 * below; the trailer's first 32-bit word is the largest finite |w| (its fp32
 * bits), from which s = 14 - floor(log2 max|w|) (clamped to [-100, 100]).
 * That puts the largest magnitude in [2^14, 2^15), so every weight within a
 * factor 2^31 of the largest is carried exactly (a bf16 significand has 8
 * bits, fp16 holds 11 and reaches 2^-24 with its subnormals); smaller ones
 * round to the nearest multiple of 2^(-24-s).  Products multiply their fp32
 * result by 2^-s.  Errors: E_INVALID for null pointers, rows % 16 != 0,
 * dst_bytes too small. */
llmdec_status llmdec_pack_matrix(int32_t rows, int32_t cols, const void *src, void *dst, size_t dst_bytes,
                                 llmdec_stream stream);
/* Bytes of one packed layer for cfg. */
size_t llmdec_packed_layer_bytes(const llmdec_config *cfg);
/* Pack one layer ([W] §2 keeps weights [out][in] and lets the operator side
 * pick the layout its kernels want) into dev buffer dst; fills *out with
 * pointers into dst.  The input weights may be freed once the stream has run. */
llmdec_status llmdec_pack_layer(const llmdec_config *cfg, const llmdec_layer_weights *in, void *dst,
                                size_t dst_bytes, llmdec_packed_layer *out, llmdec_stream stream);

/* ------------------------------------------------------------------ KV pool */
/* [E] §3.4: the cache is split into fixed-size pages handed out from a free
 * list on demand and returned when a request ends; attention reaches a
 * token's cache block through a per-sequence page index.  Each sequence owns a
 * block-table row of page ids; position p lives in page row[p / 16] at in-page
 * offset o = p % 16.  Device layout per layer (element = bf16):
 *   K: [num_pages][n_kv_heads][16][head_dim]   (K[page][h][o][d])
 *   V: [num_pages][n_kv_heads][4][head_dim][4] (V[page][h][o/4][d][o%4]: per
 *      quarter of the page, each dim's 4 tokens are adjacent, so one
 *      contiguous read gives every lane all tokens of its dims),
 * K block then V block, layer after layer; so pool_bytes = n_layers * 2 *
 * num_pages * n_kv_heads * 16 * head_dim * 2 (for 7B and 128 pages: 1 GiB,
 * the [E] §3.4 example). */
typedef struct llmdec_kv_pool llmdec_kv_pool;

size_t llmdec_kv_pool_bytes(const llmdec_config *cfg, int32_t num_pages);
/* Create a host handle over the caller's dev buffer (>= kv_pool_bytes).
 * free_order (host, may be NULL = 0,1,2,...) is a permutation of page ids:
 * the order in which pages are handed out.  Errors: E_INVALID for a bad
 * config, null pointers, short buffer, or a free_order that is not a
 * permutation. */
llmdec_status llmdec_kv_pool_create(const llmdec_config *cfg, void *dev_base, size_t bytes, int32_t num_pages,
                                    const int32_t *free_order, llmdec_kv_pool **out);
/* Grow a sequence so that it covers tokens_needed tokens: appends
 * ceil(tokens_needed/16) - *n_pages_inout pages (popped from the free list) to
 * the host row block_table_row[0..max_pages) and updates *n_pages_inout.
 * Atomic: on E_NO_PAGES neither the row nor the pool changes.  E_INVALID if
 * ceil(tokens_needed/16) > max_pages or *n_pages_inout is out of range. */
llmdec_status llmdec_kv_pool_alloc(llmdec_kv_pool *pool, int32_t tokens_needed, int32_t *block_table_row,
                                   int32_t *n_pages_inout, int32_t max_pages);
/* Return pages (host array) to the free list, pushed in the given order (the
 * last one returned is handed out first).  E_INVALID, with no change, for an
 * id out of range, an id already free, or a repeated id. */
llmdec_status llmdec_kv_pool_free(llmdec_kv_pool *pool, const int32_t *pages, int32_t n);
int32_t llmdec_kv_pool_free_count(const llmdec_kv_pool *pool);
void *llmdec_kv_pool_device_base(const llmdec_kv_pool *pool);
void llmdec_kv_pool_destroy(llmdec_kv_pool *pool);

/* Test support: copy positions 0..n_tokens-1 of one sequence's K and V for
 * one layer into dev k_out, v_out ([n_tokens][n_kv_heads][head_dim] bf16),
 * walking the dev block-table row. */
llmdec_status llmdec_debug_gather_kv(const llmdec_kv_pool *pool, int32_t layer, const int32_t *block_table_row,
                                    int32_t n_tokens, void *k_out, void *v_out, llmdec_stream stream);

/* ------------------------------------------------------------------ workspace */
/* Bytes of device scratch needed for steps of up to max_tokens new tokens over
 * up to max_seqs sequences whose block-table rows are max_pages wide.  The
 * first 256 bytes hold the sticky device error word.  A workspace serves one
 * stream at a time: calls that overlap on one workspace race. */
size_t llmdec_workspace_bytes(const llmdec_config *cfg, int32_t max_tokens, int32_t max_seqs, int32_t max_pages);
/* Clear the device error word (enqueued on stream). */
llmdec_status llmdec_workspace_reset(void *ws, size_t ws_bytes, llmdec_stream stream);
/* Synchronise stream and read the device error word: 0 = none; otherwise a
 * bit mask (1: page id out of range, 2: position beyond the block-table row or
 * negative context length, 4: token id out of range, 8: sequence index,
 * cu_seqlens entry or start position out of range).  A kernel that finds such
 * a value skips the access it would have made. */
llmdec_status llmdec_workspace_error(const void *ws, llmdec_stream stream, uint32_t *error_bits);

/* ------------------------------------------------------------------ layer steps */
/* Prefill (or chunked prefill) of one layer.  hidden: dev fp32 [n_tokens][hidden],
 * the residual stream, updated in place.  Sequence s owns tokens
 * cu_seqlens[s]..cu_seqlens[s+1]-1 (dev int32 [n_seqs+1], starting at 0 and
 * strictly increasing: every sequence carries at least one new token; a
 * segment with none sets error bit 8); its first new token sits at position
 * start_pos[s] (dev int32 [n_seqs]).  block_tables: dev int32
 * [n_seqs][max_pages], rows already covering start_pos+len tokens.  n_tokens
 * (= cu_seqlens[n_seqs]) and max_q_len (>= every sequence's new-token count)
 * are host copies used to size the launch.  Computes ([W] §1.1, [E] §4.2-4.3):
 *   y = RMSNorm(x); q,k,v = y Wq^T, y Wk^T, y Wv^T; rotate q, k by position;
 *   store bf16 k, v into the pool; causal attention over positions 0..p;
 *   x += o Wo^T; y = RMSNorm(x); x += (silu(y Wg^T) * (y Wu^T)) Wd^T. */
llmdec_status llmdec_layer_prefill(const llmdec_config *cfg, const llmdec_packed_layer *w, int32_t layer,
                                   float *hidden, int32_t n_seqs, int32_t n_tokens, int32_t max_q_len,
                                   const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *block_tables,
                                   int32_t max_pages, llmdec_kv_pool *pool, void *ws, size_t ws_bytes,
                                   llmdec_stream stream);

/* One decode token per sequence for one layer ([F] §2.2.2: only the new
 * token's q, k, v are computed; cached K/V are reused).  hidden: dev fp32
 * [n_seqs][hidden], updated in place.  ctx_lens: dev int32 [n_seqs], the
 * number of tokens already cached = the new token's position; its K/V go to
 * that position and attention covers positions 0..ctx_lens[s]. */
llmdec_status llmdec_layer_decode(const llmdec_config *cfg, const llmdec_packed_layer *w, int32_t layer,
                                  float *hidden, int32_t n_seqs, const int32_t *ctx_lens, const int32_t *block_tables,
                                  int32_t max_pages, llmdec_kv_pool *pool, void *ws, size_t ws_bytes,
                                  llmdec_stream stream);

/* One greedy step of the whole model ([F] §4, [E] §4.4): embed the new
 * tokens, run every layer, take each sequence's last new token, final
 * RMSNorm, lm_head, argmax with the lowest index winning ties, and write
 * next_tokens (dev int32 [n_seqs]) without a host synchronisation ([E] §5.3).
 * tokens: dev int32 [n_tokens].  cu_seqlens == NULL means one token per
 * sequence (decode; n_tokens == n_seqs, max_q_len == 1) at position
 * start_pos[s]; otherwise as in llmdec_layer_prefill.  logits: optional dev
 * fp32 [n_seqs][vocab]. */
llmdec_status llmdec_model_step_greedy(const llmdec_config *cfg, const llmdec_model_weights *w, int32_t n_seqs,
                                       int32_t n_tokens, int32_t max_q_len, const int32_t *tokens,
                                       const int32_t *cu_seqlens, const int32_t *start_pos,
                                       const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool,
                                       int32_t *next_tokens, float *logits, void *ws, size_t ws_bytes,
                                       llmdec_stream stream);

/* ------------------------------------------------------------------ single operations
 * The kernels the layer steps are built from, exposed one by one so each can
 * be checked on its own.  Same conventions as above.
 *
 * Packed activations: an fp16 [R][C] matrix (R a multiple of 16, C of 32) is
 * stored as 16 x 32 tiles, tile (R/16 index i, C/32 index t) at element
 * offset (i * C/32 + t) * 512; inside a tile, lane l = (r % 16) + 16 * ((c %
 * 32) / 8) holds elements c % 8 = 0..7 at l * 8 + c % 8.  This is the operand
 * order of one 16x16x32 matrix-core instruction, so every operand fetch is
 * one contiguous 16-byte load.  Packed weight matrices use the same order. */

/* y = x * (mean(x^2) + eps)^(-1/2) * gamma per row ([E] §4.2).  x: dev fp32
 * [rows][n], n a multiple of 32 and at most 8192; gamma: dev bf16 [n].
 * out_f32 (fp32 [rows][n]) and out_act (fp16(y), rounded to nearest-even and
 * clipped to +-65504, in the packed tile layout of a
 * [round_up(rows,16)][ld_packed] matrix, ld_packed a multiple of 32 from n
 * to 8192: see "Packed activations" above; columns n..ld_packed-1 zeroed)
 * may each be NULL but not both.  out_lo
 * (NULL, or the same layout as out_act, which must then be given) receives
 * fp16(y - out_act): the pair the q|k|v product reads. */
llmdec_status llmdec_op_rmsnorm(const float *x, const void *gamma, int32_t rows, int32_t n, float eps,
                                float *out_f32, void *out_act, void *out_lo, int32_t ld_packed, llmdec_stream stream);

/* out[m][n] (+)= sum_k a[m][k] * W[n][k], fp32 accumulation, for a dev fp32
 * a [rows][k_dim] and a packed W (llmdec_pack_matrix of [n_dim][k_dim]).
 * act_parts = 1: a enters the matrix cores rounded to fp16 (as the o,
 * gate/up, down and lm_head products of the layer steps take theirs);
 * act_parts = 2: as the fp16 pair hi + lo (as the q|k|v product takes its
 * input).  accumulate = 0 stores, 1 adds into out (the residual add of [W]
 * §1.1).  ws: scratch for the fp16 activation and split-k partial sums (>=
 * llmdec_op_linear_ws_bytes).  rows == 1 takes the one-row kernel (fp32
 * activation whatever act_parts, k_dim <= 14336), rows <= 64 the
 * weight-streaming kernel, rows > 64 the tiled one.  E_INVALID for act_parts
 * other than 1 or 2. */
size_t llmdec_op_linear_ws_bytes(int32_t rows, int32_t k_dim, int32_t n_dim);
llmdec_status llmdec_op_linear(const float *a, int32_t rows, int32_t k_dim, const void *w_packed, int32_t n_dim,
                               float *out, int32_t accumulate, int32_t act_parts, void *ws, size_t ws_bytes,
                               llmdec_stream stream);

/* The gate/up product with the SwiGLU epilogue, as the layer steps run it
 * ([W] §1.2, [E] §4.2): for a fused gate/up matrix as llmdec_pack_layer lays
 * it out (16-row blocks alternating gate and up, 2*inter rows), writes
 * u[m][j] = silu(g[m][j]) * up[m][j], g and up the fp32 products, in fp16
 * into out_act, in the packed layout of a [round_up(rows,16)][ld_packed]
 * matrix (inter <= ld_packed <= inter + 16, ld_packed a multiple of 32;
 * columns inter.. zeroed).  act_parts = 1: the input a enters rounded to fp16
 * (a prefill's gate/up product); act_parts = 2: a enters as the fp16 pair and
 * u is written as the pair out_act + out_lo (out_lo in the same layout), as a
 * decode step's gate/up product runs.  ws as for llmdec_op_linear with n_dim =
 * 2*inter.  E_INVALID for act_parts other than 1 or 2, or 2 without out_lo. */
llmdec_status llmdec_op_swiglu_linear(const float *a, int32_t rows, int32_t k_dim, const void *w_gu_packed,
                                      int32_t inter, void *out_act, void *out_lo, int32_t ld_packed, int32_t act_parts,
                                      void *ws, size_t ws_bytes, llmdec_stream stream);

/* Rotate q and k of each new token by its position and store bf16 k, v into
 * the pool ([E] §4.3: rotation first, then the cache update).  qkv: dev fp32
 * [n_tokens][hidden + 2*n_kv_heads*head_dim] (q | k | v: n_heads query
 * heads, then n_kv_heads key and n_kv_heads value heads); q is rotated in
 * place.  Token t belongs
 * to sequence seq_of_token[t] (dev int32, in [0, n_seqs): the row of
 * block_tables [n_seqs][max_pages]) at position pos_of_token[t]. */
llmdec_status llmdec_op_rope_append(const llmdec_config *cfg, float *qkv, int32_t n_tokens, int32_t n_seqs,
                                    const int32_t *seq_of_token, const int32_t *pos_of_token,
                                    const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool,
                                    int32_t layer, void *ws, size_t ws_bytes, llmdec_stream stream);

/* Decode attention: for each sequence s and head h, o = softmax(q K^T /
 * sqrt(head_dim)) V over positions 0..ctx_lens[s] read through the pages
 * ([E] §4.3).  q: dev fp32 [n_seqs][hidden]; out: dev fp32 [n_seqs][hidden]. */
llmdec_status llmdec_op_decode_attention(const llmdec_config *cfg, const float *q, int32_t n_seqs,
                                         const int32_t *ctx_lens, const int32_t *block_tables, int32_t max_pages,
                                         const llmdec_kv_pool *pool, int32_t layer, float *out, void *ws,
                                         size_t ws_bytes, llmdec_stream stream);

/* Causal prefill attention: new token i of sequence s (position start_pos[s]+i)
 * attends positions 0..start_pos[s]+i read through the pages.  q: dev fp32
 * [n_tokens][hidden] (already rotated); out: dev fp32 [n_tokens][hidden]. */
llmdec_status llmdec_op_prefill_attention(const llmdec_config *cfg, const float *q, int32_t n_seqs,
                                          int32_t n_tokens, int32_t max_q_len, const int32_t *cu_seqlens,
                                          const int32_t *start_pos, const int32_t *block_tables, int32_t max_pages,
                                          const llmdec_kv_pool *pool, int32_t layer, float *out, void *ws,
                                          size_t ws_bytes, llmdec_stream stream);

/* u = silu(gate) * up, silu(z) = z / (1 + e^-z) ([W] §1.2, [E] §4.2).  gate,
 * up: dev fp32 [rows][n]; out: dev fp32 [rows][n]. */
llmdec_status llmdec_op_silu_mul(const float *gate, const float *up, int32_t rows, int32_t n, float *out,
                                 llmdec_stream stream);

/* Greedy choice ([F] §2.2.3): logits = x lm_head^T for dev fp32 x [rows][hidden]
 * (already normalised) and a packed lm_head [vocab][hidden]; next[r] = argmax,
 * lowest index on ties.  logits_out: optional dev fp32 [rows][vocab]. */
llmdec_status llmdec_op_lm_head_argmax(const float *x, int32_t rows, int32_t hidden, const void *lm_head_packed,
                                       int32_t vocab, int32_t *next, float *logits_out, void *ws, size_t ws_bytes,
                                       llmdec_stream stream);

/* ------------------------------------------------------------------ sampling
 * [E] §3.5 and [F] §2.2.3: temperature divides the logits before the
 * softmax; top-k keeps the k most probable tokens; top-p keeps the smallest
 * set of most probable tokens whose probability sum reaches p; combined, the
 * temperature comes first, then the truncations, then the draw.  Here top-k
 * is applied before top-p (which works on the distribution renormalised over
 * the top-k set); a token tied with the last one a truncation keeps is kept
 * too; the token drawn is the first kept one, in increasing id, whose
 * cumulative renormalised probability exceeds u.  The draw for row r of a
 * call is u = (w >> 8) * 2^-24 with w word 0 of Philox4x32-10 (Salmon et al.,
 * SC 2011) at counter (r, step & 0xffffffff, step >> 32, 0) and key
 * (seed & 0xffffffff, seed >> 32), so results are reproducible and need no
 * generator state on the device; every sum the decision depends on is taken
 * in a fixed order, so the same inputs give the same tokens on every call.
 *   temperature <= 0: greedy (argmax, lowest index on ties);
 *   top_k <= 0 or >= vocab: no top-k;  top_p in (0, 1], 1: no top-p. */
typedef struct {
  float temperature;
  int32_t top_k;
  float top_p;
  uint64_t seed;
  uint64_t step;
} llmdec_sampling;

/* next[r] for dev fp32 logits [rows][vocab] (vocab <= 32768), dev int32
 * next [rows].  Errors: E_INVALID for null pointers, sizes out of range,
 * top_p outside (0, 1] or a non-finite temperature. */
llmdec_status llmdec_op_sample(const float *logits, int32_t rows, int32_t vocab, const llmdec_sampling *params,
                               int32_t *next, llmdec_stream stream);

/* llmdec_model_step_greedy with the next tokens sampled on the device
 * ([E] §5.3: no host synchronisation) instead of the argmax; row r of the
 * draw is sequence r.  Same arguments otherwise; vocab <= 32768. */
llmdec_status llmdec_model_step_sample(const llmdec_config *cfg, const llmdec_model_weights *w, int32_t n_seqs,
                                       int32_t n_tokens, int32_t max_q_len, const int32_t *tokens,
                                       const int32_t *cu_seqlens, const int32_t *start_pos,
                                       const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool,
                                       const llmdec_sampling *params, int32_t *next_tokens, float *logits, void *ws,
                                       size_t ws_bytes, llmdec_stream stream);

/* For callers that cannot allocate device memory, not even a workspace (code
 * under HIP graph capture, serving loops and harnesses that forbid
 * allocation): llmdec_model_step_greedy with its workspace in a device array
 * of the library, 48 MiB per GPU (enough for 7B-shaped decode steps of up to
 * 64 sequences), held from the first call on that GPU until the process
 * ends.  Same arguments as llmdec_model_step_greedy without ws / ws_bytes;
 * error_bits (dev uint32, nullable) receives this call's device error word
 * (the bits llmdec_workspace_error reports).  E_WORKSPACE when the step needs
 * more workspace than the array holds.  The call allocates nothing.  Every
 * call on a GPU uses that GPU's one array: calls that overlap on one GPU
 * (two streams, two threads) race.  The first call on a GPU looks up the
 * array's address; make it outside graph capture. */
llmdec_status llmdec_model_step_greedy_noalloc(const llmdec_config *cfg, const llmdec_model_weights *w, int32_t n_seqs,
                                               int32_t n_tokens, int32_t max_q_len, const int32_t *tokens,
                                               const int32_t *cu_seqlens, const int32_t *start_pos,
                                               const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool,
                                               int32_t *next_tokens, float *logits, uint32_t *error_bits,
                                               llmdec_stream stream);


/* ------------------------------------------------------------------ group-quantized weights
 * [W] §4.2: a matrix stored as integers in groups of 128 consecutive elements,
 * each group with one scale and one zero point, turned back into floating
 * point for the product.  Here the codes are 8-bit unsigned, the groups run
 * along each row (the input dimension of an [out][in] matrix; a row's last
 * group may be shorter), and
 *   W[r][c] = (codes[r][c] - zeros[r][c/128]) * scales[r][c/128]
 * with the scale a bf16 value.  Device pointers: codes uint8 [rows][cols],
 * scales bf16 [rows][ceil(cols/128)], zeros uint8 [rows][ceil(cols/128)]. */
typedef struct {
  const void *codes, *scales, *zeros;
} llmdec_q8_matrix;

/* One layer with quantized matrices (norm gains stay bf16 [hidden]). */
typedef struct {
  const void *attn_norm;
  llmdec_q8_matrix wq, wk, wv, wo;
  const void *mlp_norm;
  llmdec_q8_matrix w_gate, w_up, w_down;
} llmdec_q8_layer_weights;

/* A quantized layer packed by llmdec_q8_pack_layer (pointers into the
 * caller's buffer): q|k|v fused into one matrix (wq rows, then wk, wv), gate
 * and up into one ([w_gate; w_up], 2*intermediate rows). */
typedef struct {
  const void *attn_norm, *mlp_norm;
  const void *w_qkv, *w_o, *w_gu, *w_down;
} llmdec_q8_packed_layer;

/* Bytes of a packed quantized rows x cols matrix: the codes as given
 * (rows*cols bytes), then one 32-bit word per (row, group) holding the bf16
 * scale and the zero point, ordered for the kernel's lanes and padded per
 * row to a multiple of 32 words (the padding words are zero).  0 when the
 * shape is unsupported: cols must be a multiple of 16 and at most 14336,
 * rows a multiple of 4 (and at most about 120000 rows). */
size_t llmdec_q8_matrix_bytes(int32_t rows, int32_t cols);
/* Pack one quantized matrix into dev dst (>= q8_matrix_bytes).  The source
 * may be freed once the stream has run.  Errors: E_INVALID for null
 * pointers, an unsupported shape or dst_bytes too small. */
llmdec_status llmdec_q8_pack_matrix(int32_t rows, int32_t cols, const llmdec_q8_matrix *src, void *dst,
                                    size_t dst_bytes, llmdec_stream stream);
/* Bytes of one packed quantized layer for cfg (0 if cfg is invalid or its
 * matrices have an unsupported shape). */
size_t llmdec_q8_packed_layer_bytes(const llmdec_config *cfg);
llmdec_status llmdec_q8_pack_layer(const llmdec_config *cfg, const llmdec_q8_layer_weights *in, void *dst,
                                   size_t dst_bytes, llmdec_q8_packed_layer *out, llmdec_stream stream);

/* out[n] (+)= sum_k a[k] * W[n][k] for one dev fp32 row a [k_dim] and a
 * packed quantized W [n_dim][k_dim], fp32 arithmetic throughout (the
 * activation is not rounded; partial sums are added in a fixed order, so
 * repeated calls give identical results).  accumulate = 0 stores, 1 adds into out.  No
 * workspace.  Errors: E_INVALID for null pointers or a shape q8_matrix_bytes
 * rejects. */
llmdec_status llmdec_op_linear_q8(const float *a, int32_t k_dim, const void *w_q8_packed, int32_t n_dim, float *out,
                                  int32_t accumulate, llmdec_stream stream);

/* llmdec_layer_decode with quantized matrices, for a single sequence
 * (n_seqs must be 1: the quantized products are matrix-vector products;
 * more sequences return E_UNSUPPORTED).  Same arguments, workspace size
 * (llmdec_workspace_bytes) and results otherwise. */
llmdec_status llmdec_layer_decode_q8(const llmdec_config *cfg, const llmdec_q8_packed_layer *w, int32_t layer,
                                     float *hidden, int32_t n_seqs, const int32_t *ctx_lens,
                                     const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool, void *ws,
                                     size_t ws_bytes, llmdec_stream stream);

/* ------------------------------------------------------------------ 4-bit codes
 * The same scheme with 4-bit codes and zero points (0..15), two codes to a
 * byte: byte j of a row holds column 2j in its low nibble and 2j+1 in its
 * high nibble, so a row of `cols` codes is cols/2 bytes in the caller's
 * codes array ([rows][cols/2]); scales and zeros as for 8-bit codes.  The
 * packed matrix pads each row's codes with zero codes to a multiple of 16
 * bytes; its metadata words are ordered for 4 lanes per group.  The entry
 * points below mirror the 8-bit ones (same errors, same limits). */
typedef llmdec_q8_matrix llmdec_q4_matrix;
typedef llmdec_q8_layer_weights llmdec_q4_layer_weights;
typedef llmdec_q8_packed_layer llmdec_q4_packed_layer;
size_t llmdec_q4_matrix_bytes(int32_t rows, int32_t cols);
llmdec_status llmdec_q4_pack_matrix(int32_t rows, int32_t cols, const llmdec_q4_matrix *src, void *dst,
                                    size_t dst_bytes, llmdec_stream stream);
size_t llmdec_q4_packed_layer_bytes(const llmdec_config *cfg);
llmdec_status llmdec_q4_pack_layer(const llmdec_config *cfg, const llmdec_q4_layer_weights *in, void *dst,
                                   size_t dst_bytes, llmdec_q4_packed_layer *out, llmdec_stream stream);
llmdec_status llmdec_op_linear_q4(const float *a, int32_t k_dim, const void *w_q4_packed, int32_t n_dim, float *out,
                                  int32_t accumulate, llmdec_stream stream);
llmdec_status llmdec_layer_decode_q4(const llmdec_config *cfg, const llmdec_q4_packed_layer *w, int32_t layer,
                                     float *hidden, int32_t n_seqs, const int32_t *ctx_lens,
                                     const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool, void *ws,
                                     size_t ws_bytes, llmdec_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* LLMDEC_H */
