// Internal declarations: error reporting, argument checks, workspace layout and
// the host-side launchers of every kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "llmdec.h"

namespace llmdec {

llmdec_status set_error(llmdec_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
llmdec_status clear_error();
llmdec_status check_config(const llmdec_config *cfg, const char *who);
llmdec_status check_launch(const char *who);

// How an activation matrix is handed to a linear kernel.
//  - rows == 1: fp32 vector `f32` (GEMV path, no rounding of the activation);
//  - rows > 1: `hi`/`lo` bf16 matrices in the packed tile layout (rows padded
//    to 16, columns to kpad) holding bf16(a) and bf16(a - bf16(a)).
struct Act {
  const float *f32 = nullptr;
  const uint16_t *hi = nullptr;
  const uint16_t *lo = nullptr;
  int rows = 0;
  int kpad = 0;  // padded column count of hi/lo (multiple of 32)
};

enum Epilogue { kStore = 0, kAccumulate = 1 };

// Workspace layout for steps of up to max_tokens tokens and max_seqs sequences.
struct WsLayout {
  size_t err, tok_seq, tok_pos, x, act_f32, act_hi, act_lo, qkv, attn, gu, part, attn_part, logits, amax, total;
  int max_tokens, max_seqs, max_pages, kpad_max, attn_slots, ksplit_max;
};
WsLayout ws_layout(const llmdec_config &cfg, int max_tokens, int max_seqs, int max_pages);

// Decode-attention partitioning: pages per partition and partitions per row.
void decode_partition(int n_seqs, int n_heads, int max_pages, int *pages_per_part, int *n_parts);

// ---------------------------------------------------------------- launchers (kernels_*.hip)
void launch_pack_matrix(int rows, int cols, const uint16_t *src, uint16_t *dst, hipStream_t s, int nb_stride = 1);
void launch_embed(const uint16_t *embed, const int32_t *tokens, int n_tokens, int hidden, int vocab, float *x,
                  uint32_t *err, hipStream_t s);
// y = rmsnorm(x) * gamma on the given rows; outputs: f32 [rows][n] and/or tiled hi/lo with kpad columns.
void launch_rmsnorm(const float *x, int ld_x, const int32_t *row_index, int n_src_rows, const uint16_t *gamma, int rows, int n,
                    float eps, uint32_t *err, float *out_f32, uint16_t *out_hi, uint16_t *out_lo, int kpad, hipStream_t s);
// fp32 [rows][ld] -> tiled hi/lo [rows_pad16][kpad] (zero padding).
void launch_split(const float *a, int ld, int rows, int cols, uint16_t *hi, uint16_t *lo, int kpad, hipStream_t s);
void launch_linear(const Act &a, const uint16_t *w_packed, int n, int k, float *out, int ld_out, Epilogue epi,
                   float *partials, size_t partial_floats, hipStream_t s);
size_t linear_partial_floats(int rows, int n, int k);
void launch_token_map(const int32_t *cu_seqlens, const int32_t *start_pos, int n_seqs, int n_tokens, uint32_t *err, int32_t *tok_seq,
                      int32_t *tok_pos, hipStream_t s);
void launch_rope_append(const llmdec_config &cfg, float *qkv, int ld_qkv, int n_tokens, int n_seqs, const int32_t *tok_seq,
                        const int32_t *tok_pos, const int32_t *block_tables, int max_pages, uint16_t *pool_layer_k,
                        uint16_t *pool_layer_v, int num_pages, uint32_t *err, hipStream_t s);
void launch_decode_attention(const llmdec_config &cfg, const float *q, int ld_q, int n_seqs, const int32_t *ctx_lens,
                             const int32_t *block_tables, int max_pages, const uint16_t *pool_layer_k,
                             const uint16_t *pool_layer_v, int num_pages, float *partials, float *out_f32,
                             uint16_t *out_hi, uint16_t *out_lo, int kpad, uint32_t *err, hipStream_t s);
void launch_prefill_attention(const llmdec_config &cfg, const float *q, int ld_q, int n_seqs, int n_tokens, int max_q_len,
                              const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *block_tables,
                              int max_pages, const uint16_t *pool_layer_k, const uint16_t *pool_layer_v,
                              int num_pages, float *out_f32, uint16_t *out_hi, uint16_t *out_lo, int kpad,
                              uint32_t *err, hipStream_t s);
// u = silu(g) * up.  g at g[r*ld_in + (j/16)*blk + j%16], up likewise from u_ptr.
void launch_silu_mul(const float *g, const float *u, int ld_in, int blk, int rows, int n, float *out_f32,
                     uint16_t *out_hi, uint16_t *out_lo, int kpad, hipStream_t s);
void launch_argmax(const float *logits, int rows, int vocab, int32_t *next, hipStream_t s);
void launch_gather_kv(const uint16_t *pool_layer_k, const uint16_t *pool_layer_v, int num_pages, int n_heads,
                      int head_dim, const int32_t *row, int n_tokens, uint16_t *k_out, uint16_t *v_out,
                      hipStream_t s);
void launch_fill_u32(uint32_t *p, uint32_t value, size_t n, hipStream_t s);

}  // namespace llmdec
