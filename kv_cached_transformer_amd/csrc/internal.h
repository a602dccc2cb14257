// Internal declarations: error reporting, argument checks, workspace layout and
// the host-side launchers of every kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "host.h"
#include "llmdec.h"

namespace llmdec {

llmdec_status check_launch(const char *who);

// An activation matrix as a weight product reads it: fp16 values (rounded to nearest-even from the
// fp32 producer, clipped to +-65504) in the packed tile layout, rows padded to 16 (row_blocks 16-row
// blocks exist in the buffer), columns padded to kpad (a multiple of 32) with zeros.  With lo set, the
// activation is the pair hi + lo (hi = fp16(a), lo = fp16(a - hi), about 22 significant bits) and the
// product takes both parts.
struct Act {
  const uint16_t *a = nullptr;
  const uint16_t *lo = nullptr;
  int rows = 0;
  int kpad = 0;
  int row_blocks = 0;
};

enum Epilogue { kStore = 0, kAccumulate = 1, kSiluMul = 2, kRope = 3 };

struct RopeFreq {
  double inv_freq[64];
};
RopeFreq rope_freq(const llmdec_config &cfg);

// The kRope epilogue of a prefill q|k|v product (tiled products only, more than 64 rows).  Row r is
// token r: its sequence and position come from tok_seq / tok_pos; pair i turns by pos * fr.inv_freq[i],
// as in the RoPE/append kernel.  The product's column c is column col0 + c of the q|k|v row: q
// columns are rotated and stored to f32[r*ld + c]; k columns are rotated, v columns left as they are,
// and both rounded to bf16 and written to the page slot block_tables[seq][pos / 16], offset pos % 16,
// as the RoPE/append kernel stores them (a bad sequence, position or page sets err, and that row's K/V
// are not written).
struct RopeRows {
  RopeFreq fr;
  const int32_t *tok_seq = nullptr, *tok_pos = nullptr, *block_tables = nullptr;
  uint16_t *pool_k = nullptr, *pool_v = nullptr;
  uint32_t *err = nullptr;
  int col0 = 0, n_seqs = 0, max_pages = 0, num_pages = 0, n_heads = 0, n_kv_heads = 0, head_dim = 0;
};

// Where a weight product's result goes.  kStore / kAccumulate: fp32 f32[r*ld + c]
// (= or +=).  kSiluMul: the product's row blocks alternate gate and up; the
// result silu(gate) * up goes, in fp16, to the packed activation act (with
// act_lo: as the fp16 pair act + act_lo) with act_kt k-tiles per row block and
// act_cols real columns (the rest of the row is zeroed).
struct LinearOut {
  int kind = kStore;
  float *f32 = nullptr;
  int ld = 0;
  uint16_t *act = nullptr;
  uint16_t *act_lo = nullptr;
  int act_kt = 0;
  int act_cols = 0;
  RopeRows rope;  // kRope only
};


// How a streaming weight product left its result (a stream-K split).  Its work is the units
// (column group, k-tile) -- groups of group_cols columns with kt k-tiles each, `units` in all, in
// group-major order -- and block b of `blocks` takes units [b*units/blocks, (b+1)*units/blocks), so
// every block gets the same amount whatever the shape.  Each (block, group) segment leaves one fp32
// [rows][n] plane of partial sums: for a group's columns, plane j holds the j-th block covering the
// group, and the planes are added in that order.  blocks == 0: no partials, the epilogue was applied.
struct Splits {
  int blocks = 0, units = 0, kt = 0, group_cols = 0;
  __host__ __device__ bool any() const { return blocks > 0; }
  // the block whose range holds unit u: the least b with floor((b+1)*units/blocks) > u
  __host__ __device__ int first_block(long u) const {
    return (int)(((u + 1) * (long)blocks + units - 1) / units) - 1;
  }
  // number of partial planes of the group holding column c
  __host__ __device__ int slots(int c) const {
    const long g = c / group_cols;
    return first_block((g + 1) * (long)kt - 1) - first_block(g * (long)kt) + 1;
  }
};

// Columns of the fused q|k|v product: n_heads query heads, then n_kv_heads key heads, then n_kv_heads
// value heads, head_dim each (grouped-query attention shares one K/V head among n_heads / n_kv_heads
// query heads).
inline int qkv_cols(const llmdec_config &c) { return (c.n_heads + 2 * c.n_kv_heads) * c.head_dim; }
inline int kv_cols(const llmdec_config &c) { return c.n_kv_heads * c.head_dim; }

// Workspace layout for steps of up to max_tokens tokens and max_seqs sequences.
struct WsLayout {
  size_t err, tok_seq, tok_pos, x, act_h, act_hl, act_i, act_il, qkv, part, attn_part, logits, total;
  size_t part_floats;
  int max_tokens, max_seqs, max_pages, row_blocks, kpad_h, kpad_i, attn_slots;
};
WsLayout ws_layout(const llmdec_config &cfg, int max_tokens, int max_seqs, int max_pages);

// Decode-attention partitioning: pages per partition and partitions per (sequence, wave of heads) row.
void decode_partition(const llmdec_config &cfg, int n_seqs, int max_pages, int *pages_per_part, int *n_parts);
// Query heads one decode-attention wave serves (they share a K/V head): 1, 2 or 4.
int decode_heads_per_wave(const llmdec_config &cfg);
// Partial results per (sequence, head) of a decode with n_parts partitions: one per block of waves.
int decode_blocks_per_seq(int n_parts);

// ---------------------------------------------------------------- launchers (kernels_*.hip)
// Packed weight matrices: bytes of the tiles of a rows x cols matrix (the trailer follows them).
size_t packed_tiles_bytes(int rows, int cols);
// Clear a packed matrix's trailer, then fold the largest |w| of each source matrix it will hold into
// it (launch_weight_absmax), then pack each source (launch_pack_matrix: bf16 [rows][cols] -> fp16 tiles
// scaled by the shift the trailer gives).  Source 16-row block nb lands at destination block
// nb * nb_stride of the matrix at dst (nb_stride 2 interleaves two matrices block by block).
void launch_weight_trailer_clear(uint16_t *dst, size_t tiles_bytes, hipStream_t s);
void launch_weight_absmax(int rows, int cols, const uint16_t *src, uint16_t *dst, size_t tiles_bytes, hipStream_t s);
void launch_pack_matrix(int rows, int cols, const uint16_t *src, uint16_t *dst, size_t tiles_bytes, hipStream_t s,
                        int nb_stride = 1);
void launch_embed(const uint16_t *embed, const int32_t *tokens, int n_tokens, int hidden, int vocab, float *x,
                  uint32_t *err, hipStream_t s);
// y = rmsnorm(x) * gamma on the given rows; outputs: f32 [rows][n] and/or the packed fp16 activation with
// kpad columns (out_lo != NULL: as the pair out_act = fp16(y), out_lo = fp16(y - out_act)).  add_partials (may be NULL): the partial sums [plane][rows][n] of a split output projection
// (described by sp), first added into x (its residual add), x being written back.
void launch_rmsnorm(float *x, int ld_x, const int32_t *row_index, int n_src_rows, const uint16_t *gamma, int rows,
                    int n, float eps, uint32_t *err, float *out_f32, uint16_t *out_act, uint16_t *out_lo, int kpad,
                    const float *add_partials, const Splits &sp, hipStream_t s);
// fp32 [rows][ld] -> packed fp16 activation [rows_pad16][kpad] (lo != NULL: the pair), zero padding.
void launch_split(const float *a, int ld, int rows, int cols, uint16_t *act, uint16_t *lo, int kpad, hipStream_t s);
// Weight product.  When the product is split (the returned Splits has any()), the result is left as fp32
// partial sums [plane][rows][n] in partials and the epilogue is NOT applied: the caller reduces them, either
// with launch_reduce or inside the next kernel.  Otherwise the epilogue is applied.
// kSplitBalanced: every CU gets the same work, so split boundaries differ between column groups (and so,
// in the last bits, does the summation order).  kSplitUniform: every column group is cut at the same k
// boundaries, so equal weight rows give bit-equal outputs (what an argmax over the outputs needs for its
// ties).  kSplitNone: one block per column group, epilogue applied.
enum SplitPolicy { kSplitBalanced = 0, kSplitUniform = 1, kSplitNone = 2 };
Splits launch_linear(const Act &a, const uint16_t *w_packed, int n, int k, const LinearOut &o, float *partials,
                     size_t partial_floats, SplitPolicy policy, hipStream_t s);
// The product over columns [col0, col0 + n) of a packed matrix of n_total columns (col0 and n multiples of
// 16), unsplit, the epilogue o applied with the range's first column as column 0 (kRope: more than 64
// rows).
void launch_linear_cols(const Act &a, const uint16_t *w_packed, int n_total, int col0, int n, int k,
                        const LinearOut &o, hipStream_t s);
// Sum the partial products of a split product and apply the epilogue o.
void launch_reduce(const float *partials, const Splits &sp, int rows, int n, const LinearOut &o, hipStream_t s);


size_t linear_partial_floats(int rows, int n, int k, SplitPolicy policy = kSplitBalanced);
void launch_token_map(const int32_t *cu_seqlens, const int32_t *start_pos, int n_seqs, int n_tokens, uint32_t *err, int32_t *tok_seq,
                      int32_t *tok_pos, hipStream_t s);
// qkv_partials / sp: when the q|k|v product was split, its partial sums [plane][n_tokens][3*hidden] are
// added first (and the sum written to qkv); NULL otherwise.
void launch_rope_append(const llmdec_config &cfg, float *qkv, const float *qkv_partials, const Splits &sp, int ld_qkv,
                        int n_tokens, int n_seqs, const int32_t *tok_seq,
                        const int32_t *tok_pos, const int32_t *block_tables, int max_pages, uint16_t *pool_layer_k,
                        uint16_t *pool_layer_v, int num_pages, uint32_t *err, hipStream_t s);
// Attention outputs go to fp32 out_f32 [rows][hidden] and/or the packed fp16 activation with kpad columns
// (out_lo != NULL: as the fp16 pair out_act + out_lo).
void launch_decode_attention(const llmdec_config &cfg, const float *q, int ld_q, int n_seqs, const int32_t *ctx_lens,
                             const int32_t *block_tables, int max_pages, const uint16_t *pool_layer_k,
                             const uint16_t *pool_layer_v, int num_pages, float *partials, float *out_f32,
                             uint16_t *out_act, uint16_t *out_lo, int kpad, uint32_t *err, hipStream_t s);
void launch_prefill_attention(const llmdec_config &cfg, const float *q, int ld_q, int n_seqs, int n_tokens, int max_q_len,
                              const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *block_tables,
                              int max_pages, const uint16_t *pool_layer_k, const uint16_t *pool_layer_v,
                              int num_pages, float *out_f32, uint16_t *out_act, uint16_t *out_lo, int kpad,
                              uint32_t *err, hipStream_t s);
// u = silu(g) * up elementwise, fp32 [rows][n] (the stand-alone operation; the layer steps fuse it
// into the gate/up product's epilogue).
void launch_silu_mul(const float *g, const float *u, int rows, int n, float *out, hipStream_t s);
// Row-wise argmax of fp32 [rows][vocab], lowest index on ties; vocab a multiple of 4 (the API requires 16).
void launch_argmax(const float *logits, int rows, int vocab, int32_t *next, hipStream_t s);
void launch_gather_kv(const uint16_t *pool_layer_k, const uint16_t *pool_layer_v, int num_pages, int n_heads,
                      int head_dim, const int32_t *row, int n_tokens, uint16_t *k_out, uint16_t *v_out,
                      hipStream_t s);
void launch_fill_u32(uint32_t *p, uint32_t value, size_t n, hipStream_t s);
// *dst = *src (one word, device to device)
void launch_copy_u32(const uint32_t *src, uint32_t *dst, hipStream_t s);

// Rotary frequencies inv_freq[i] = theta^(-2i/D), i < D/2 (zero past), computed in double on the host.

// Where the one-row q|k|v product sends its result when it also applies RoPE and the paged append (a
// single decode token of sequence 0 at position *pos): rotated q to its output, rotated bf16 k and bf16
// v to the pool slot block_row[pos/16], offset pos%16, as the RoPE/append kernel stores them; a bad
// position or page sets err and skips the K/V stores, as that kernel does.
struct RopeAppend {
  RopeFreq fr;
  const int32_t *pos;
  const int32_t *block_row;
  int max_pages, num_pages, n_heads, n_kv_heads, head_dim;
  uint16_t *pool_k, *pool_v;
  uint32_t *err;
};

// One-row products with a packed bf16 matrix (kernels_gemv.hip): x fp32 [k], n a multiple of 16 (of 32
// for kSiluMul, whose matrix is the fused gate/up one: 16-row blocks alternating gate and up, out[j] =
// silu(gate_j) * up_j for j < n / 2).  kStore / kAccumulate write or add out[0..n).  gamma != NULL: the
// product reads rmsnorm(x) * gamma (eps inside the root).  gemv_shape_ok: k a multiple of 16, <= 14336.
bool gemv_shape_ok(int k);
void launch_gemv(const float *x, const uint16_t *gamma, float eps, const uint16_t *w_packed, int n, int k, int mode,
                 float *out, hipStream_t s);
// The q|k|v product of a single decode token with RoPE and the paged K/V append in its epilogue.
void launch_gemv_qkv_rope(const float *x, const uint16_t *gamma, float eps, const uint16_t *w_packed, int n, int k,
                          float *qkv, const RopeAppend &ra, hipStream_t s);

// Temperature / top-k / top-p sampling of fp32 logits [rows][vocab] (kernels_sample.hip); vocab <= 32768.
bool sample_shape_ok(int vocab);
void launch_sample(const float *logits, int rows, int vocab, float temperature, int top_k, float top_p,
                   uint64_t seed, uint64_t step, int32_t *next, hipStream_t s);

// Group-quantized matrices (kernels_quant.hip), codes of `bits` = 8 or 4 bits.  q_shape_ok: cols a
// multiple of 16, at most 14336.
bool q_shape_ok(int bits, int cols);
size_t q_matrix_bytes(int bits, int rows, int cols);
// Pack a source matrix's rows into rows dst_row0.. of a packed matrix with dst_rows rows in all.
void launch_q_pack(int bits, const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros, int rows, int cols,
                   uint8_t *dst, int dst_rows, int dst_row0, hipStream_t s);
// One-row product with a packed quantized matrix of `rows` rows: mode kStore / kAccumulate write
// out[0..rows); kSiluMul reads the matrix as [gate; up] and writes out[j] = silu(gate_j) * up_j for
// j < rows / 2.  rows % 4 == 0.  gamma != NULL: the product reads rmsnorm(x) * gamma (eps inside the root)
// instead of x.
void launch_q_gemv(int bits, const float *x, const uint16_t *gamma, float eps, const uint8_t *w, int rows, int k,
                   int mode, float *out, hipStream_t s);

}  // namespace llmdec
