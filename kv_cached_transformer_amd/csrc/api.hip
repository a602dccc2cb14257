// C ABI of libllmdec: argument checks, workspace layout and the order of the
// kernels in a layer step and a model step.
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace llmdec {

llmdec_status check_launch(const char *who) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(LLMDEC_E_HIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
  return clear_error();
}

static size_t al(size_t x) { return round_up_sz(x, 256); }

WsLayout ws_layout(const llmdec_config &c, int max_tokens, int max_seqs, int max_pages) {
  WsLayout L{};
  const int T = std::max(1, max_tokens), S = std::max(1, max_seqs), P = std::max(1, max_pages);
  const int h = c.hidden, I = c.intermediate;
  const int rows = std::max(T, S);
  L.max_tokens = T;
  L.max_seqs = S;
  L.max_pages = P;
  L.row_blocks = (rows + 15) / 16;
  L.kpad_h = round_up(h, kTileK);
  L.kpad_i = round_up(I, kTileK);
  // decode-attention partial slots: the worst case over every batch size up to S
  size_t slots = 0;
  for (int n = 1; n <= S; ++n) {
    int ppp, parts;
    decode_partition(c, n, P, &ppp, &parts);
    slots = std::max(slots, (size_t)n * c.n_heads * decode_blocks_per_seq(parts));
  }
  L.attn_slots = (int)slots;
  // split-k partial sums: the worst case over every streamed product (rows <= 64) this workspace can see
  size_t part = 0;
  const int shapes[4][2] = {{qkv_cols(c), h}, {h, h}, {2 * I, h}, {h, I}};
  for (int m = 1; m <= std::min(rows, 64); ++m) {
    for (auto &sh : shapes) part = std::max(part, linear_partial_floats(m, sh[0], sh[1], kSplitBalanced));
    part = std::max(part, linear_partial_floats(m, c.vocab, h, kSplitUniform));  // lm_head
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += al(bytes);
    return o;
  };
  L.err = take(kWsHeader);
  L.tok_seq = take(sizeof(int32_t) * T);
  L.tok_pos = take(sizeof(int32_t) * T);
  L.x = take(sizeof(float) * (size_t)rows * h);
  L.act_h = take(sizeof(uint16_t) * (size_t)L.row_blocks * 16 * L.kpad_h);
  L.act_hl = take(sizeof(uint16_t) * (size_t)L.row_blocks * 16 * L.kpad_h);
  L.act_i = take(sizeof(uint16_t) * (size_t)L.row_blocks * 16 * L.kpad_i);
  L.act_il = take(sizeof(uint16_t) * (size_t)L.row_blocks * 16 * L.kpad_i);
  L.qkv = take(sizeof(float) * (size_t)rows * qkv_cols(c));
  L.part = take(sizeof(float) * part);
  L.part_floats = part;
  L.attn_part = take(sizeof(float) * slots * (c.head_dim + 2));
  L.logits = take(sizeof(float) * (size_t)S * c.vocab);
  L.total = off;
  return L;
}

template <typename T>
static T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off);
}

static size_t layer_stride_elems(const llmdec_config &c, int num_pages) {
  return (size_t)2 * num_pages * c.n_kv_heads * kPage * c.head_dim;
}

static void pool_layer(const llmdec_kv_pool *p, int layer, uint16_t **k, uint16_t **v) {
  uint16_t *base = reinterpret_cast<uint16_t *>(p->base) + (size_t)layer * layer_stride_elems(p->cfg, p->num_pages);
  *k = base;
  *v = base + (size_t)p->num_pages * p->cfg.n_kv_heads * kPage * p->cfg.head_dim;
}

static bool same_shape(const llmdec_config &a, const llmdec_config &b) {
  return a.n_layers == b.n_layers && a.hidden == b.hidden && a.n_heads == b.n_heads && a.n_kv_heads == b.n_kv_heads &&
         a.head_dim == b.head_dim;
}

static llmdec_status check_packed(const llmdec_packed_layer *w, const char *who) {
  if (!w || !w->attn_norm || !w->mlp_norm || !w->w_qkv || !w->w_o || !w->w_gu || !w->w_down)
    return set_error(LLMDEC_E_INVALID, "%s: packed layer weights missing", who);
  return LLMDEC_OK;
}

static llmdec_status check_pool(const llmdec_kv_pool *pool, const llmdec_config &c, int layer, const char *who) {
  if (!pool) return set_error(LLMDEC_E_INVALID, "%s: pool is NULL", who);
  if (!same_shape(pool->cfg, c)) return set_error(LLMDEC_E_INVALID, "%s: pool was created for another shape", who);
  if (layer < 0 || layer >= c.n_layers)
    return set_error(LLMDEC_E_INVALID, "%s: layer %d out of range [0,%d)", who, layer, c.n_layers);
  return LLMDEC_OK;
}

static llmdec_status check_ws(const void *ws, size_t ws_bytes, size_t need, const char *who) {
  if (!ws) return set_error(LLMDEC_E_WORKSPACE, "%s: workspace is NULL", who);
  if (ws_bytes < need)
    return set_error(LLMDEC_E_WORKSPACE, "%s: workspace holds %zu bytes, %zu needed", who, ws_bytes, need);
  return LLMDEC_OK;
}

// The body of one layer once every argument has been checked.  rows == number
// of new tokens; decode passes tok_seq = NULL (token t is sequence t) and
// positions = ctx_lens.
struct LayerArgs {
  const llmdec_config *cfg;
  const llmdec_packed_layer *w;
  int layer;
  float *hidden;
  int rows;
  bool decode;
  int n_seqs, max_q_len;
  const int32_t *cu, *start, *ctx;
  const int32_t *bt;
  int max_pages;
  const llmdec_kv_pool *pool;
  void *ws;
  WsLayout L;
  hipStream_t s;
  Splits pending;  // split-k partial sums of the previous layer's down projection, not yet in hidden
};

// Decode of a single sequence: every product is a matrix-vector product (one-row kernels with the
// RMSNorms folded into the q|k|v and gate/up launches, epilogues applied in the kernels, no split-k
// partial sums); activations between kernels are fp32.
static void run_layer_one_row(const LayerArgs &a) {
  const llmdec_config &c = *a.cfg;
  const int h = c.hidden, I = c.intermediate, nqkv = qkv_cols(c);
  const WsLayout &L = a.L;
  uint32_t *err = at<uint32_t>(a.ws, L.err);
  // one row: the fp32 activations fit in the packed activations' space (16 fp16 rows)
  float *y = at<float>(a.ws, L.act_h), *u = at<float>(a.ws, L.act_i), *qkv = at<float>(a.ws, L.qkv);
  uint16_t *pk, *pv;
  pool_layer(a.pool, a.layer, &pk, &pv);
  // q|k|v with the attention RMSNorm before it and RoPE + the paged K/V append after it, in one launch
  RopeAppend ra;
  ra.fr = rope_freq(c);
  ra.pos = a.ctx, ra.block_row = a.bt, ra.max_pages = a.max_pages, ra.num_pages = a.pool->num_pages;
  ra.n_heads = c.n_heads, ra.n_kv_heads = c.n_kv_heads, ra.head_dim = c.head_dim;
  ra.pool_k = pk, ra.pool_v = pv, ra.err = err;
  launch_gemv_qkv_rope(a.hidden, (const uint16_t *)a.w->attn_norm, c.rms_eps, (const uint16_t *)a.w->w_qkv, nqkv, h,
                       qkv, ra, a.s);
  launch_decode_attention(c, qkv, nqkv, 1, a.ctx, a.bt, a.max_pages, pk, pv, a.pool->num_pages,
                          at<float>(a.ws, L.attn_part), y, nullptr, nullptr, 0, err, a.s);
  launch_gemv(y, nullptr, 0.f, (const uint16_t *)a.w->w_o, h, h, kAccumulate, a.hidden, a.s);
  launch_gemv(a.hidden, (const uint16_t *)a.w->mlp_norm, c.rms_eps, (const uint16_t *)a.w->w_gu, 2 * I, h, kSiluMul,
              u, a.s);
  launch_gemv(u, nullptr, 0.f, (const uint16_t *)a.w->w_down, h, I, kAccumulate, a.hidden, a.s);
}

// Returns the split of the down projection whose partial sums are left in the workspace instead of added
// into hidden (none when it was not split); the caller adds them (finish_layer) or hands them to the next
// layer, whose attention RMSNorm adds them into hidden before normalising.
static Splits run_layer(const LayerArgs &a) {
  const llmdec_config &c = *a.cfg;
  const int h = c.hidden, I = c.intermediate, M = a.rows;
  const WsLayout &L = a.L;
  if (a.decode && M == 1 && gemv_shape_ok(h) && gemv_shape_ok(I)) {
    run_layer_one_row(a);
    return Splits{};
  }
  uint32_t *err = at<uint32_t>(a.ws, L.err);
  uint16_t *act_h = at<uint16_t>(a.ws, L.act_h), *act_hl = at<uint16_t>(a.ws, L.act_hl);
  uint16_t *act_i = at<uint16_t>(a.ws, L.act_i), *act_il = at<uint16_t>(a.ws, L.act_il);
  float *qkv = at<float>(a.ws, L.qkv), *part = at<float>(a.ws, L.part);
  // The k|v columns of the q|k|v product read their input as an fp16 pair (k and v are rounded to bf16
  // for the cache, so their error must stay far below a bf16 step).  The other products read the pair in
  // a decode step (at most 64 rows: the products stream the weights, a second activation plane costs
  // little, and single fp16 inputs would compound over a model's layers) and one fp16 plane in a prefill
  // (matrix-core bound), the q columns included.
  const bool pairs = M <= 64;
  uint16_t *lo_h = pairs ? act_hl : nullptr, *lo_i = pairs ? act_il : nullptr;
  const Act ah2{act_h, act_hl, M, L.kpad_h, L.row_blocks}, ah{act_h, lo_h, M, L.kpad_h, L.row_blocks};
  const Act ai{act_i, lo_i, M, L.kpad_i, L.row_blocks};
  uint16_t *pk, *pv;
  pool_layer(a.pool, a.layer, &pk, &pv);

  // attention block: x += Wo . attn(rope(Wq y), rope(Wk y), Wv y),  y = RMSNorm(x)
  launch_rmsnorm(a.hidden, h, nullptr, M, (const uint16_t *)a.w->attn_norm, M, h, c.rms_eps, err, nullptr, act_h,
                 act_hl, L.kpad_h, a.pending.any() ? part : nullptr, a.pending, a.s);
  LinearOut o_qkv;
  o_qkv.kind = kStore;
  o_qkv.f32 = qkv;
  const int nqkv = qkv_cols(c);
  o_qkv.ld = nqkv;
  int32_t *ts = at<int32_t>(a.ws, L.tok_seq), *tp = at<int32_t>(a.ws, L.tok_pos);
  if (!a.decode) launch_token_map(a.cu, a.start, a.n_seqs, M, err, ts, tp, a.s);
  // A split q|k|v product leaves partial sums that the rotary/append kernel adds up.  A tiled prefill
  // product applies RoPE and the K/V append in its own epilogue (kRope), so no rotary/append pass
  // follows it.
  const bool fused_rope = !pairs && !a.decode;
  Splits sp_qkv;
  if (pairs) {
    sp_qkv = launch_linear(ah2, (const uint16_t *)a.w->w_qkv, nqkv, h, o_qkv, part, L.part_floats, kSplitBalanced, a.s);
  } else {
    const int nq = c.n_heads * c.head_dim;
    LinearOut o_q = o_qkv, o_kv = o_qkv;
    o_kv.f32 = qkv + nq;
    if (fused_rope) {
      RopeRows rr;
      rr.fr = rope_freq(c);
      rr.tok_seq = ts, rr.tok_pos = tp, rr.block_tables = a.bt;
      rr.pool_k = pk, rr.pool_v = pv, rr.err = err;
      rr.n_seqs = a.n_seqs, rr.max_pages = a.max_pages, rr.num_pages = a.pool->num_pages;
      rr.n_heads = c.n_heads, rr.n_kv_heads = c.n_kv_heads, rr.head_dim = c.head_dim;
      o_q.kind = o_kv.kind = kRope;
      o_q.rope = o_kv.rope = rr;
      o_kv.rope.col0 = nq;
    }
    launch_linear_cols(ah, (const uint16_t *)a.w->w_qkv, nqkv, 0, nq, h, o_q, a.s);
    launch_linear_cols(ah2, (const uint16_t *)a.w->w_qkv, nqkv, nq, nqkv - nq, h, o_kv, a.s);
  }
  const float *qkv_part = sp_qkv.any() ? part : nullptr;
  if (a.decode) {
    launch_rope_append(c, qkv, qkv_part, sp_qkv, nqkv, M, a.n_seqs, nullptr, a.ctx, a.bt, a.max_pages, pk, pv,
                       a.pool->num_pages, err, a.s);
    launch_decode_attention(c, qkv, nqkv, M, a.ctx, a.bt, a.max_pages, pk, pv, a.pool->num_pages,
                            at<float>(a.ws, L.attn_part), nullptr, act_h, lo_h, L.kpad_h, err, a.s);
  } else {
    if (!fused_rope)
      launch_rope_append(c, qkv, qkv_part, sp_qkv, nqkv, M, a.n_seqs, ts, tp, a.bt, a.max_pages, pk, pv,
                         a.pool->num_pages, err, a.s);
    launch_prefill_attention(c, qkv, nqkv, a.n_seqs, M, a.max_q_len, a.cu, a.start, a.bt, a.max_pages, pk, pv,
                             a.pool->num_pages, nullptr, act_h, lo_h, L.kpad_h, err, a.s);
  }
  LinearOut o_res;
  o_res.kind = kAccumulate;
  o_res.f32 = a.hidden;
  o_res.ld = h;
  // a split output projection leaves partial sums that the MLP's RMSNorm adds into x before normalising
  const Splits sp_o = launch_linear(ah, (const uint16_t *)a.w->w_o, h, h, o_res, part, L.part_floats, kSplitBalanced, a.s);

  // MLP block: x += Wd (silu(Wg y) * (Wu y)),  y = RMSNorm(x); the gate/up product's epilogue forms the
  // SwiGLU activation directly
  launch_rmsnorm(a.hidden, h, nullptr, M, (const uint16_t *)a.w->mlp_norm, M, h, c.rms_eps, err, nullptr, act_h,
                 lo_h, L.kpad_h, sp_o.any() ? part : nullptr, sp_o, a.s);
  LinearOut o_gu;
  o_gu.kind = kSiluMul;
  o_gu.act = act_i;
  o_gu.act_lo = lo_i;
  o_gu.act_kt = L.kpad_i / kTileK;
  o_gu.act_cols = I;
  const Splits sp_gu = launch_linear(ah, (const uint16_t *)a.w->w_gu, 2 * I, h, o_gu, part, L.part_floats, kSplitBalanced, a.s);
  if (sp_gu.any()) launch_reduce(part, sp_gu, M, 2 * I, o_gu, a.s);
  return launch_linear(ai, (const uint16_t *)a.w->w_down, h, I, o_res, part, L.part_floats, kSplitBalanced, a.s);
}

// Adds a layer's pending down-projection partial sums into hidden.
static void finish_layer(const LayerArgs &a, const Splits &pending) {
  if (!pending.any()) return;
  LinearOut o_res;
  o_res.kind = kAccumulate;
  o_res.f32 = a.hidden;
  o_res.ld = a.cfg->hidden;
  launch_reduce(at<float>(a.ws, a.L.part), pending, a.rows, a.cfg->hidden, o_res, a.s);
}

}  // namespace llmdec

using namespace llmdec;


// ------------------------------------------------------------------ weights
extern "C" size_t llmdec_packed_matrix_bytes(int32_t rows, int32_t cols) {
  if (rows <= 0 || cols <= 0 || rows % 16) return 0;
  return packed_tiles_bytes(rows, cols) + kWTrailer;
}

extern "C" llmdec_status llmdec_pack_matrix(int32_t rows, int32_t cols, const void *src, void *dst, size_t dst_bytes,
                                           llmdec_stream stream) {
  if (!src || !dst) return set_error(LLMDEC_E_INVALID, "pack_matrix: NULL pointer");
  if (rows <= 0 || cols <= 0 || rows % 16)
    return set_error(LLMDEC_E_INVALID, "pack_matrix: rows (%d) must be a positive multiple of 16, cols (%d) > 0", rows,
                     cols);
  const size_t need = llmdec_packed_matrix_bytes(rows, cols);
  if (dst_bytes < need) return set_error(LLMDEC_E_INVALID, "pack_matrix: dst holds %zu bytes, %zu needed", dst_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  const size_t tb = packed_tiles_bytes(rows, cols);
  uint16_t *d = (uint16_t *)dst;
  launch_weight_trailer_clear(d, tb, s);
  launch_weight_absmax(rows, cols, (const uint16_t *)src, d, tb, s);
  launch_pack_matrix(rows, cols, (const uint16_t *)src, d, tb, s);
  return check_launch("pack_matrix");
}

static size_t packed_layer_parts(const llmdec_config &c, size_t off[6]) {
  const int h = c.hidden, I = c.intermediate;
  size_t o = 0;
  off[0] = o;  // attn_norm
  o += al((size_t)h * 2);
  off[1] = o;  // mlp_norm
  o += al((size_t)h * 2);
  off[2] = o;  // qkv
  o += al(llmdec_packed_matrix_bytes(qkv_cols(c), h));
  off[3] = o;  // o
  o += al(llmdec_packed_matrix_bytes(h, h));
  off[4] = o;  // gate/up
  o += al(llmdec_packed_matrix_bytes(2 * I, h));
  off[5] = o;  // down
  o += al(llmdec_packed_matrix_bytes(h, I));
  return o;
}

extern "C" size_t llmdec_packed_layer_bytes(const llmdec_config *cfg) {
  if (check_config(cfg, "packed_layer_bytes") != LLMDEC_OK) return 0;
  size_t off[6];
  return packed_layer_parts(*cfg, off);
}

extern "C" llmdec_status llmdec_pack_layer(const llmdec_config *cfg, const llmdec_layer_weights *in, void *dst,
                                          size_t dst_bytes, llmdec_packed_layer *out, llmdec_stream stream) {
  llmdec_status st = check_config(cfg, "pack_layer");
  if (st != LLMDEC_OK) return st;
  if (!in || !dst || !out || !in->attn_norm || !in->wq || !in->wk || !in->wv || !in->wo || !in->mlp_norm ||
      !in->w_gate || !in->w_up || !in->w_down)
    return set_error(LLMDEC_E_INVALID, "pack_layer: NULL pointer");
  size_t off[6];
  const size_t need = packed_layer_parts(*cfg, off);
  if (dst_bytes < need) return set_error(LLMDEC_E_INVALID, "pack_layer: dst holds %zu bytes, %zu needed", dst_bytes, need);
  const int h = cfg->hidden, I = cfg->intermediate;
  hipStream_t s = (hipStream_t)stream;
  char *d = (char *)dst;
  if (hipMemcpyAsync(d + off[0], in->attn_norm, (size_t)h * 2, hipMemcpyDeviceToDevice, s) != hipSuccess ||
      hipMemcpyAsync(d + off[1], in->mlp_norm, (size_t)h * 2, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return set_error(LLMDEC_E_HIP, "pack_layer: copy of the norm gains failed");
  // One packed matrix from one or more sources: each source's rows land at 16-row block row0/16 (times
  // nb_stride when two sources interleave block by block).  The trailer takes the largest magnitude of
  // all of them before any is packed, so the fused matrix has one shift.
  struct Src {
    const void *p;
    int rows, cols, row0, nb_stride;
  };
  auto pack = [&](uint16_t *dm, int rows_total, int cols, std::initializer_list<Src> srcs) {
    const size_t tb = packed_tiles_bytes(rows_total, cols);
    const int ktc = round_up(cols, kTileK);
    launch_weight_trailer_clear(dm, tb, s);
    for (const Src &x : srcs) launch_weight_absmax(x.rows, x.cols, (const uint16_t *)x.p, dm, tb, s);
    for (const Src &x : srcs)
      launch_pack_matrix(x.rows, x.cols, (const uint16_t *)x.p, dm + (size_t)x.row0 * ktc, tb - (size_t)x.row0 * ktc * 2,
                         s, x.nb_stride);
  };
  const int kv = kv_cols(*cfg), nqkv = qkv_cols(*cfg);
  // fused q|k|v: row blocks of wq ([h][h]), then wk and wv ([kv][h] each; every part whole 16-row blocks)
  pack((uint16_t *)(d + off[2]), nqkv, h,
       {{in->wq, h, h, 0, 1}, {in->wk, kv, h, h, 1}, {in->wv, kv, h, h + kv, 1}});
  pack((uint16_t *)(d + off[3]), h, h, {{in->wo, h, h, 0, 1}});
  // gate/up interleaved by 16-row block: block 2j = gate rows 16j.., block 2j+1 = up rows 16j..
  pack((uint16_t *)(d + off[4]), 2 * I, h, {{in->w_gate, I, h, 0, 2}, {in->w_up, I, h, 16, 2}});
  pack((uint16_t *)(d + off[5]), h, I, {{in->w_down, h, I, 0, 1}});
  st = check_launch("pack_layer");
  if (st != LLMDEC_OK) return st;
  out->attn_norm = d + off[0];
  out->mlp_norm = d + off[1];
  out->w_qkv = d + off[2];
  out->w_o = d + off[3];
  out->w_gu = d + off[4];
  out->w_down = d + off[5];
  return LLMDEC_OK;
}

// ------------------------------------------------------------------ workspace
extern "C" size_t llmdec_workspace_bytes(const llmdec_config *cfg, int32_t max_tokens, int32_t max_seqs,
                                         int32_t max_pages) {
  if (check_config(cfg, "workspace_bytes") != LLMDEC_OK || max_tokens < 0 || max_seqs < 0 || max_pages < 0) return 0;
  return ws_layout(*cfg, max_tokens, max_seqs, max_pages).total;
}

extern "C" llmdec_status llmdec_workspace_reset(void *ws, size_t ws_bytes, llmdec_stream stream) {
  if (!ws || ws_bytes < kWsHeader) return set_error(LLMDEC_E_WORKSPACE, "workspace_reset: workspace missing or too small");
  launch_fill_u32((uint32_t *)ws, 0u, kWsHeader / 4, (hipStream_t)stream);
  return check_launch("workspace_reset");
}

extern "C" llmdec_status llmdec_workspace_error(const void *ws, llmdec_stream stream, uint32_t *bits) {
  if (!ws || !bits) return set_error(LLMDEC_E_INVALID, "workspace_error: NULL pointer");
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(bits, ws, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return set_error(LLMDEC_E_HIP, "workspace_error: read-back failed");
  return clear_error();
}

extern "C" llmdec_status llmdec_debug_gather_kv(const llmdec_kv_pool *pool, int32_t layer, const int32_t *row,
                                               int32_t n_tokens, void *k_out, void *v_out, llmdec_stream stream) {
  if (!pool || !row || !k_out || !v_out) return set_error(LLMDEC_E_INVALID, "debug_gather_kv: NULL pointer");
  if (layer < 0 || layer >= pool->cfg.n_layers || n_tokens < 0)
    return set_error(LLMDEC_E_INVALID, "debug_gather_kv: layer %d / n_tokens %d out of range", layer, n_tokens);
  uint16_t *pk, *pv;
  pool_layer(pool, layer, &pk, &pv);
  launch_gather_kv(pk, pv, pool->num_pages, pool->cfg.n_kv_heads, pool->cfg.head_dim, row, n_tokens,
                   (uint16_t *)k_out, (uint16_t *)v_out, (hipStream_t)stream);
  return check_launch("debug_gather_kv");
}

// ------------------------------------------------------------------ layer steps
extern "C" llmdec_status llmdec_layer_prefill(const llmdec_config *cfg, const llmdec_packed_layer *w, int32_t layer,
                                             float *hidden, int32_t n_seqs, int32_t n_tokens, int32_t max_q_len,
                                             const int32_t *cu_seqlens, const int32_t *start_pos,
                                             const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool,
                                             void *ws, size_t ws_bytes, llmdec_stream stream) {
  const char *who = "layer_prefill";
  llmdec_status st = check_config(cfg, who);
  if (st == LLMDEC_OK) st = check_packed(w, who);
  if (st == LLMDEC_OK) st = check_pool(pool, *cfg, layer, who);
  if (st != LLMDEC_OK) return st;
  if (!hidden || !cu_seqlens || !start_pos || !block_tables)
    return set_error(LLMDEC_E_INVALID, "%s: NULL device pointer", who);
  if (n_seqs <= 0 || n_tokens <= 0 || max_q_len <= 0 || max_q_len > n_tokens || max_pages <= 0)
    return set_error(LLMDEC_E_INVALID, "%s: n_seqs=%d n_tokens=%d max_q_len=%d max_pages=%d out of range", who, n_seqs,
                     n_tokens, max_q_len, max_pages);
  WsLayout L = ws_layout(*cfg, n_tokens, n_seqs, max_pages);
  st = check_ws(ws, ws_bytes, L.total, who);
  if (st != LLMDEC_OK) return st;
  LayerArgs a{cfg, w, layer, hidden, n_tokens, false, n_seqs, max_q_len, cu_seqlens, start_pos, nullptr,
              block_tables, max_pages, pool, ws, L, (hipStream_t)stream, Splits{}};
  finish_layer(a, run_layer(a));
  return check_launch(who);
}

extern "C" llmdec_status llmdec_layer_decode(const llmdec_config *cfg, const llmdec_packed_layer *w, int32_t layer,
                                            float *hidden, int32_t n_seqs, const int32_t *ctx_lens,
                                            const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool,
                                            void *ws, size_t ws_bytes, llmdec_stream stream) {
  const char *who = "layer_decode";
  llmdec_status st = check_config(cfg, who);
  if (st == LLMDEC_OK) st = check_packed(w, who);
  if (st == LLMDEC_OK) st = check_pool(pool, *cfg, layer, who);
  if (st != LLMDEC_OK) return st;
  if (!hidden || !ctx_lens || !block_tables) return set_error(LLMDEC_E_INVALID, "%s: NULL device pointer", who);
  if (n_seqs <= 0 || max_pages <= 0)
    return set_error(LLMDEC_E_INVALID, "%s: n_seqs=%d max_pages=%d out of range", who, n_seqs, max_pages);
  WsLayout L = ws_layout(*cfg, n_seqs, n_seqs, max_pages);
  st = check_ws(ws, ws_bytes, L.total, who);
  if (st != LLMDEC_OK) return st;
  LayerArgs a{cfg, w, layer, hidden, n_seqs, true, n_seqs, 1, nullptr, nullptr, ctx_lens, block_tables, max_pages,
              pool, ws, L, (hipStream_t)stream, Splits{}};
  finish_layer(a, run_layer(a));
  return check_launch(who);
}

static llmdec_status check_sampling(const llmdec_sampling *p, int vocab, const char *who) {
  if (!p) return set_error(LLMDEC_E_INVALID, "%s: sampling parameters are NULL", who);
  if (!(p->top_p > 0.f && p->top_p <= 1.f))
    return set_error(LLMDEC_E_INVALID, "%s: top_p=%g outside (0, 1]", who, (double)p->top_p);
  if (!__builtin_isfinite(p->temperature))
    return set_error(LLMDEC_E_INVALID, "%s: temperature is not finite", who);
  if (!sample_shape_ok(vocab)) return set_error(LLMDEC_E_INVALID, "%s: vocab=%d outside [1, 32768]", who, vocab);
  return LLMDEC_OK;
}

// One model step; smp == NULL: the greedy choice, else sampling.
static llmdec_status model_step(const char *who, const llmdec_config *cfg, const llmdec_model_weights *w,
                                int32_t n_seqs, int32_t n_tokens, int32_t max_q_len, const int32_t *tokens,
                                const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *block_tables,
                                int32_t max_pages, llmdec_kv_pool *pool, const llmdec_sampling *smp,
                                int32_t *next_tokens, float *logits, void *ws, size_t ws_bytes, llmdec_stream stream) {
  llmdec_status st = check_config(cfg, who);
  if (st != LLMDEC_OK) return st;
  if (!w || !w->embed || !w->layers || !w->final_norm || !w->lm_head)
    return set_error(LLMDEC_E_INVALID, "%s: model weights missing", who);
  for (int l = 0; l < cfg->n_layers; ++l) {
    st = check_packed(&w->layers[l], who);
    if (st != LLMDEC_OK) return st;
  }
  st = check_pool(pool, *cfg, 0, who);
  if (st != LLMDEC_OK) return st;
  if (!tokens || !start_pos || !block_tables || !next_tokens)
    return set_error(LLMDEC_E_INVALID, "%s: NULL device pointer", who);
  const bool decode = cu_seqlens == nullptr;
  if (n_seqs <= 0 || max_pages <= 0 || n_tokens <= 0 || max_q_len <= 0 || max_q_len > n_tokens)
    return set_error(LLMDEC_E_INVALID, "%s: n_seqs=%d n_tokens=%d max_q_len=%d max_pages=%d out of range", who, n_seqs,
                     n_tokens, max_q_len, max_pages);
  if (decode && (n_tokens != n_seqs || max_q_len != 1))
    return set_error(LLMDEC_E_INVALID, "%s: without cu_seqlens each sequence takes one token (n_tokens=%d, n_seqs=%d)",
                     who, n_tokens, n_seqs);
  WsLayout L = ws_layout(*cfg, n_tokens, n_seqs, max_pages);
  st = check_ws(ws, ws_bytes, L.total, who);
  if (st != LLMDEC_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  float *x = at<float>(ws, L.x);
  launch_embed((const uint16_t *)w->embed, tokens, n_tokens, cfg->hidden, cfg->vocab, x, at<uint32_t>(ws, L.err), s);
  Splits pending{};  // each layer's down-projection partial sums go into the next layer's RMSNorm
  for (int l = 0; l < cfg->n_layers; ++l) {
    LayerArgs a{cfg, &w->layers[l], l, x, n_tokens, decode, n_seqs, max_q_len, cu_seqlens, start_pos,
                decode ? start_pos : nullptr, block_tables, max_pages, pool, ws, L, s, pending};
    pending = run_layer(a);
    if (l + 1 == cfg->n_layers) finish_layer(a, pending);
  }
  // final norm on each sequence's last new token, lm_head, argmax ([W] §1.1, [F] §2.2.3)
  const int h = cfg->hidden;
  uint16_t *act_h = at<uint16_t>(ws, L.act_h);
  launch_rmsnorm(x, h, decode ? nullptr : cu_seqlens, n_tokens, (const uint16_t *)w->final_norm, n_seqs, h,
                 cfg->rms_eps, at<uint32_t>(ws, L.err), nullptr, act_h, nullptr, L.kpad_h, nullptr, Splits{}, s);
  float *lg = logits ? logits : at<float>(ws, L.logits);
  LinearOut o;
  o.kind = kStore;
  o.f32 = lg;
  o.ld = cfg->vocab;
  float *part = at<float>(ws, L.part);
  const Splits sp = launch_linear(Act{act_h, nullptr, n_seqs, L.kpad_h, L.row_blocks}, (const uint16_t *)w->lm_head,
                                  cfg->vocab, h, o, part, L.part_floats, kSplitUniform, s);  // argmax ties
  if (sp.any()) launch_reduce(part, sp, n_seqs, cfg->vocab, o, s);
  if (smp)
    launch_sample(lg, n_seqs, cfg->vocab, smp->temperature, smp->top_k, smp->top_p, smp->seed, smp->step,
                  next_tokens, s);
  else
    launch_argmax(lg, n_seqs, cfg->vocab, next_tokens, s);
  return check_launch(who);
}

extern "C" llmdec_status llmdec_model_step_greedy(const llmdec_config *cfg, const llmdec_model_weights *w,
                                                 int32_t n_seqs, int32_t n_tokens, int32_t max_q_len,
                                                 const int32_t *tokens, const int32_t *cu_seqlens,
                                                 const int32_t *start_pos, const int32_t *block_tables,
                                                 int32_t max_pages, llmdec_kv_pool *pool, int32_t *next_tokens,
                                                 float *logits, void *ws, size_t ws_bytes, llmdec_stream stream) {
  return model_step("model_step_greedy", cfg, w, n_seqs, n_tokens, max_q_len, tokens, cu_seqlens, start_pos,
                    block_tables, max_pages, pool, nullptr, next_tokens, logits, ws, ws_bytes, stream);
}

extern "C" llmdec_status llmdec_model_step_sample(const llmdec_config *cfg, const llmdec_model_weights *w,
                                                 int32_t n_seqs, int32_t n_tokens, int32_t max_q_len,
                                                 const int32_t *tokens, const int32_t *cu_seqlens,
                                                 const int32_t *start_pos, const int32_t *block_tables,
                                                 int32_t max_pages, llmdec_kv_pool *pool, const llmdec_sampling *params,
                                                 int32_t *next_tokens, float *logits, void *ws, size_t ws_bytes,
                                                 llmdec_stream stream) {
  const char *who = "model_step_sample";
  if (!cfg) return set_error(LLMDEC_E_INVALID, "%s: config is NULL", who);
  llmdec_status st = check_sampling(params, cfg->vocab, who);
  if (st != LLMDEC_OK) return st;
  return model_step(who, cfg, w, n_seqs, n_tokens, max_q_len, tokens, cu_seqlens, start_pos, block_tables, max_pages,
                    pool, params, next_tokens, logits, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ the step without a workspace
// For callers that cannot allocate (code under graph capture, serving loops that forbid allocation): the
// greedy model step with its workspace in a device array of this library (48 MiB, enough for 7B-shaped
// decode steps of up to 64 sequences), one copy per GPU, held until the process ends.  Its address on
// each device is looked up once, with that device current, and the kernels only ever get that address.
constexpr size_t kScratchBytes = (size_t)48 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch[kMaxDevices];

static llmdec_status scratch_address(const char *who, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(LLMDEC_E_HIP, "%s: no current device (or device id %d beyond %d)", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(LLMDEC_E_HIP, "%s: address of the static workspace on device %d: %s", who, dev,
                       hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return LLMDEC_OK;
}

extern "C" llmdec_status llmdec_model_step_greedy_noalloc(const llmdec_config *cfg, const llmdec_model_weights *w,
                                                         int32_t n_seqs, int32_t n_tokens, int32_t max_q_len,
                                                         const int32_t *tokens, const int32_t *cu_seqlens,
                                                         const int32_t *start_pos, const int32_t *block_tables,
                                                         int32_t max_pages, llmdec_kv_pool *pool, int32_t *next_tokens,
                                                         float *logits, uint32_t *error_bits, llmdec_stream stream) {
  const char *who = "model_step_greedy_noalloc";
  llmdec_status st = check_config(cfg, who);
  if (st != LLMDEC_OK) return st;
  if (n_seqs <= 0 || n_tokens <= 0 || max_pages <= 0)
    return set_error(LLMDEC_E_INVALID, "%s: n_seqs=%d n_tokens=%d max_pages=%d out of range", who, n_seqs, n_tokens,
                     max_pages);
  const size_t need = ws_layout(*cfg, n_tokens, n_seqs, max_pages).total;
  if (need > kScratchBytes)
    return set_error(LLMDEC_E_WORKSPACE, "%s: the step needs %zu bytes of workspace, the static one holds %zu", who, need,
                     kScratchBytes);
  void *ws = nullptr;
  st = scratch_address(who, &ws);
  if (st != LLMDEC_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // the array keeps the previous call's contents: only the error word must start at zero (every other
  // region is written before it is read)
  launch_fill_u32((uint32_t *)ws, 0u, kWsHeader / 4, s);
  st = model_step(who, cfg, w, n_seqs, n_tokens, max_q_len, tokens, cu_seqlens, start_pos, block_tables, max_pages,
                  pool, nullptr, next_tokens, logits, ws, kScratchBytes, stream);
  if (st != LLMDEC_OK) return st;
  if (error_bits) launch_copy_u32((const uint32_t *)ws, error_bits, s);
  return check_launch(who);
}


extern "C" llmdec_status llmdec_op_sample(const float *logits, int32_t rows, int32_t vocab,
                                         const llmdec_sampling *params, int32_t *next, llmdec_stream stream) {
  const char *who = "op_sample";
  if (!logits || !next) return set_error(LLMDEC_E_INVALID, "%s: NULL pointer", who);
  if (rows <= 0) return set_error(LLMDEC_E_INVALID, "%s: rows=%d out of range", who, rows);
  llmdec_status st = check_sampling(params, vocab, who);
  if (st != LLMDEC_OK) return st;
  launch_sample(logits, rows, vocab, params->temperature, params->top_k, params->top_p, params->seed, params->step,
                next, (hipStream_t)stream);
  return check_launch(who);
}

// ------------------------------------------------------------------ single operations
extern "C" llmdec_status llmdec_op_rmsnorm(const float *x, const void *gamma, int32_t rows, int32_t n, float eps,
                                          float *out_f32, void *out_act, void *out_lo, int32_t ld_packed,
                                          llmdec_stream stream) {
  if (!x || !gamma || (!out_f32 && !out_act) || (out_lo && !out_act))
    return set_error(LLMDEC_E_INVALID, "op_rmsnorm: NULL pointer");
  // the row kernel writes (and zero-pads) at most 8192 columns of a row
  if (rows <= 0 || n <= 0 || n % 32 || n > 8192 || (out_act && (ld_packed < n || ld_packed % 32 || ld_packed > 8192)))
    return set_error(LLMDEC_E_INVALID,
                     "op_rmsnorm: rows=%d n=%d (a multiple of 32, <= 8192) ld_packed=%d (a multiple of 32, n..8192) "
                     "out of range", rows, n, ld_packed);
  launch_rmsnorm(const_cast<float *>(x), n, nullptr, rows, (const uint16_t *)gamma, rows, n, eps, nullptr, out_f32,
                 (uint16_t *)out_act, (uint16_t *)out_lo, ld_packed, nullptr, Splits{}, (hipStream_t)stream);
  return check_launch("op_rmsnorm");
}

// Workspace of the stand-alone products: error word, the packed fp16 activation, partial sums.
static size_t op_linear_parts(int rows, int k, int n, size_t *act_off, size_t *part_off) {
  const int kp = round_up(k, kTileK);
  const size_t act = al((size_t)round_up(rows, 16) * kp * 2);
  *act_off = kWsHeader;
  *part_off = *act_off + 2 * act;  // room for an fp16 pair
  return *part_off + al(std::max(linear_partial_floats(rows, n, k, kSplitBalanced),
                                 linear_partial_floats(rows, n, k, kSplitUniform)) * sizeof(float));
}

extern "C" size_t llmdec_op_linear_ws_bytes(int32_t rows, int32_t k_dim, int32_t n_dim) {
  size_t a, b;
  if (rows <= 0 || k_dim <= 0 || n_dim <= 0) return 0;
  return op_linear_parts(rows, k_dim, n_dim, &a, &b);
}

static llmdec_status run_op_linear(const char *who, const float *a, int32_t rows, int32_t k_dim, const void *w_packed,
                                   int32_t n_dim, int parts, const LinearOut &o, void *ws, size_t ws_bytes,
                                   size_t extra, SplitPolicy policy, hipStream_t s) {
  size_t act_off, part_off;
  const size_t need = op_linear_parts(rows, k_dim, n_dim, &act_off, &part_off) + extra;
  llmdec_status st = check_ws(ws, ws_bytes, need, who);
  if (st != LLMDEC_OK) return st;
  const int kp = round_up(k_dim, kTileK);
  uint16_t *act = at<uint16_t>(ws, act_off);
  uint16_t *lo = parts == 2 ? act + (size_t)round_up(rows, 16) * kp : nullptr;
  launch_split(a, k_dim, rows, k_dim, act, lo, kp, s);
  float *part = at<float>(ws, part_off);
  const Splits sp = launch_linear(Act{act, lo, rows, kp, (rows + 15) / 16}, (const uint16_t *)w_packed, n_dim,
                                  k_dim, o, part, linear_partial_floats(rows, n_dim, k_dim, policy), policy, s);
  if (sp.any()) launch_reduce(part, sp, rows, n_dim, o, s);
  return LLMDEC_OK;
}

extern "C" llmdec_status llmdec_op_linear(const float *a, int32_t rows, int32_t k_dim, const void *w_packed,
                                         int32_t n_dim, float *out, int32_t accumulate, int32_t act_parts, void *ws,
                                         size_t ws_bytes, llmdec_stream stream) {
  if (!a || !w_packed || !out) return set_error(LLMDEC_E_INVALID, "op_linear: NULL pointer");
  if (rows <= 0 || k_dim <= 0 || n_dim <= 0 || n_dim % 16)
    return set_error(LLMDEC_E_INVALID, "op_linear: rows=%d k=%d n=%d out of range (n a multiple of 16)", rows, k_dim,
                     n_dim);
  if (act_parts != 1 && act_parts != 2)
    return set_error(LLMDEC_E_INVALID, "op_linear: act_parts=%d must be 1 or 2", act_parts);
  LinearOut o;
  o.kind = accumulate ? kAccumulate : kStore;
  o.f32 = out;
  o.ld = n_dim;
  if (rows == 1 && gemv_shape_ok(k_dim)) {  // the one-row kernel, as a single-sequence decode step runs it
    size_t act_off, part_off;
    llmdec_status st = check_ws(ws, ws_bytes, op_linear_parts(rows, k_dim, n_dim, &act_off, &part_off), "op_linear");
    if (st != LLMDEC_OK) return st;
    launch_gemv(a, nullptr, 0.f, (const uint16_t *)w_packed, n_dim, k_dim, o.kind, out, (hipStream_t)stream);
    return check_launch("op_linear");
  }
  llmdec_status st = run_op_linear("op_linear", a, rows, k_dim, w_packed, n_dim, act_parts, o, ws, ws_bytes, 0,
                                   kSplitBalanced, (hipStream_t)stream);
  return st != LLMDEC_OK ? st : check_launch("op_linear");
}

extern "C" llmdec_status llmdec_op_swiglu_linear(const float *a, int32_t rows, int32_t k_dim, const void *w_gu_packed,
                                                int32_t inter, void *out_act, void *out_lo, int32_t ld_packed,
                                                int32_t act_parts, void *ws, size_t ws_bytes, llmdec_stream stream) {
  if (!a || !w_gu_packed || !out_act || (act_parts == 2 && !out_lo))
    return set_error(LLMDEC_E_INVALID, "op_swiglu_linear: NULL pointer");
  if (act_parts != 1 && act_parts != 2)
    return set_error(LLMDEC_E_INVALID, "op_swiglu_linear: act_parts=%d must be 1 or 2", act_parts);
  if (rows <= 0 || k_dim <= 0 || inter <= 0 || inter % 16 || ld_packed < inter || ld_packed % 32 ||
      ld_packed - inter > 16)
    return set_error(LLMDEC_E_INVALID, "op_swiglu_linear: rows=%d k=%d inter=%d ld_packed=%d out of range", rows, k_dim,
                     inter, ld_packed);
  LinearOut o;
  o.kind = kSiluMul;
  o.act = (uint16_t *)out_act;
  o.act_lo = act_parts == 2 ? (uint16_t *)out_lo : nullptr;
  o.act_kt = ld_packed / kTileK;
  o.act_cols = inter;
  llmdec_status st = run_op_linear("op_swiglu_linear", a, rows, k_dim, w_gu_packed, 2 * inter, act_parts, o, ws,
                                   ws_bytes, 0, kSplitBalanced, (hipStream_t)stream);
  return st != LLMDEC_OK ? st : check_launch("op_swiglu_linear");
}

extern "C" llmdec_status llmdec_op_rope_append(const llmdec_config *cfg, float *qkv, int32_t n_tokens,
                                              int32_t n_seqs, const int32_t *seq_of_token, const int32_t *pos_of_token,
                                              const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool,
                                              int32_t layer, void *ws, size_t ws_bytes, llmdec_stream stream) {
  const char *who = "op_rope_append";
  llmdec_status st = check_config(cfg, who);
  if (st == LLMDEC_OK) st = check_pool(pool, *cfg, layer, who);
  if (st == LLMDEC_OK) st = check_ws(ws, ws_bytes, kWsHeader, who);
  if (st != LLMDEC_OK) return st;
  if (!qkv || !seq_of_token || !pos_of_token || !block_tables) return set_error(LLMDEC_E_INVALID, "%s: NULL pointer", who);
  if (n_tokens <= 0 || n_seqs <= 0 || max_pages <= 0)
    return set_error(LLMDEC_E_INVALID, "%s: n_tokens/n_seqs/max_pages out of range", who);
  uint16_t *pk, *pv;
  pool_layer(pool, layer, &pk, &pv);
  launch_rope_append(*cfg, qkv, nullptr, Splits{}, qkv_cols(*cfg), n_tokens, n_seqs, seq_of_token, pos_of_token, block_tables, max_pages, pk, pv,
                     pool->num_pages, (uint32_t *)ws, (hipStream_t)stream);
  return check_launch(who);
}

extern "C" llmdec_status llmdec_op_decode_attention(const llmdec_config *cfg, const float *q, int32_t n_seqs,
                                                   const int32_t *ctx_lens, const int32_t *block_tables,
                                                   int32_t max_pages, const llmdec_kv_pool *pool, int32_t layer,
                                                   float *out, void *ws, size_t ws_bytes, llmdec_stream stream) {
  const char *who = "op_decode_attention";
  llmdec_status st = check_config(cfg, who);
  if (st == LLMDEC_OK) st = check_pool(pool, *cfg, layer, who);
  if (st != LLMDEC_OK) return st;
  if (!q || !ctx_lens || !block_tables || !out) return set_error(LLMDEC_E_INVALID, "%s: NULL pointer", who);
  if (n_seqs <= 0 || max_pages <= 0) return set_error(LLMDEC_E_INVALID, "%s: n_seqs/max_pages out of range", who);
  WsLayout L = ws_layout(*cfg, n_seqs, n_seqs, max_pages);
  st = check_ws(ws, ws_bytes, L.total, who);
  if (st != LLMDEC_OK) return st;
  uint16_t *pk, *pv;
  pool_layer(pool, layer, &pk, &pv);
  launch_decode_attention(*cfg, q, cfg->hidden, n_seqs, ctx_lens, block_tables, max_pages, pk, pv, pool->num_pages,
                          at<float>(ws, L.attn_part), out, nullptr, nullptr, 0, at<uint32_t>(ws, L.err),
                          (hipStream_t)stream);
  return check_launch(who);
}

extern "C" llmdec_status llmdec_op_prefill_attention(const llmdec_config *cfg, const float *q, int32_t n_seqs,
                                                    int32_t n_tokens, int32_t max_q_len, const int32_t *cu_seqlens,
                                                    const int32_t *start_pos, const int32_t *block_tables,
                                                    int32_t max_pages, const llmdec_kv_pool *pool, int32_t layer,
                                                    float *out, void *ws, size_t ws_bytes, llmdec_stream stream) {
  const char *who = "op_prefill_attention";
  llmdec_status st = check_config(cfg, who);
  if (st == LLMDEC_OK) st = check_pool(pool, *cfg, layer, who);
  if (st == LLMDEC_OK) st = check_ws(ws, ws_bytes, kWsHeader, who);
  if (st != LLMDEC_OK) return st;
  if (!q || !cu_seqlens || !start_pos || !block_tables || !out)
    return set_error(LLMDEC_E_INVALID, "%s: NULL pointer", who);
  if (n_seqs <= 0 || n_tokens <= 0 || max_q_len <= 0 || max_pages <= 0)
    return set_error(LLMDEC_E_INVALID, "%s: sizes out of range", who);
  uint16_t *pk, *pv;
  pool_layer(pool, layer, &pk, &pv);
  launch_prefill_attention(*cfg, q, cfg->hidden, n_seqs, n_tokens, max_q_len, cu_seqlens, start_pos, block_tables, max_pages,
                           pk, pv, pool->num_pages, out, nullptr, nullptr, 0, (uint32_t *)ws, (hipStream_t)stream);
  return check_launch(who);
}

extern "C" llmdec_status llmdec_op_silu_mul(const float *gate, const float *up, int32_t rows, int32_t n, float *out,
                                           llmdec_stream stream) {
  if (!gate || !up || !out) return set_error(LLMDEC_E_INVALID, "op_silu_mul: NULL pointer");
  if (rows <= 0 || n <= 0) return set_error(LLMDEC_E_INVALID, "op_silu_mul: rows=%d n=%d out of range", rows, n);
  launch_silu_mul(gate, up, rows, n, out, (hipStream_t)stream);
  return check_launch("op_silu_mul");
}

extern "C" llmdec_status llmdec_op_lm_head_argmax(const float *x, int32_t rows, int32_t hidden,
                                                 const void *lm_head_packed, int32_t vocab, int32_t *next,
                                                 float *logits_out, void *ws, size_t ws_bytes, llmdec_stream stream) {
  if (!x || !lm_head_packed || !next) return set_error(LLMDEC_E_INVALID, "op_lm_head_argmax: NULL pointer");
  if (rows <= 0 || hidden <= 0 || vocab <= 0 || vocab % 16)
    return set_error(LLMDEC_E_INVALID, "op_lm_head_argmax: rows=%d hidden=%d vocab=%d out of range", rows, hidden, vocab);
  size_t act_off, part_off;
  const size_t logit_off = op_linear_parts(rows, hidden, vocab, &act_off, &part_off);
  const size_t extra = logits_out ? 0 : al((size_t)rows * vocab * sizeof(float));
  float *lg = logits_out ? logits_out : (ws ? at<float>(ws, logit_off) : nullptr);
  LinearOut o;
  o.kind = kStore;
  o.f32 = lg;
  o.ld = vocab;
  hipStream_t s = (hipStream_t)stream;
  llmdec_status st = run_op_linear("op_lm_head_argmax", x, rows, hidden, lm_head_packed, vocab, 1, o, ws, ws_bytes, extra,
                                   kSplitUniform, s);
  if (st != LLMDEC_OK) return st;
  launch_argmax(lg, rows, vocab, next, s);
  return check_launch("op_lm_head_argmax");
}

// ------------------------------------------------------------------ group-quantized weights
// A quantized matrix is supported when its rows split into the four-row tasks of the matrix-vector
// kernel and its columns into whole 16-byte lane chunks that fit the kernel's LDS staging of x.
static bool q_ok(int bits, int rows, int cols) {
  // byte offsets inside the packed matrix stay below 2^31 (the kernel's buffer offsets)
  return rows > 0 && rows % 4 == 0 && q_shape_ok(bits, cols) && q_matrix_bytes(bits, rows, cols) < (size_t)1 << 31;
}

static bool q_src_ok(const llmdec_q8_matrix *m) { return m && m->codes && m->scales && m->zeros; }

static size_t q_layer_parts(int bits, const llmdec_config &c, size_t off[6]) {
  const int h = c.hidden, I = c.intermediate;
  size_t o = 0;
  off[0] = o;  // attn_norm
  o += al((size_t)h * 2);
  off[1] = o;  // mlp_norm
  o += al((size_t)h * 2);
  off[2] = o;  // q|k|v
  o += al(q_matrix_bytes(bits, qkv_cols(c), h));
  off[3] = o;  // o
  o += al(q_matrix_bytes(bits, h, h));
  off[4] = o;  // [gate; up]
  o += al(q_matrix_bytes(bits, 2 * I, h));
  off[5] = o;  // down
  o += al(q_matrix_bytes(bits, h, I));
  return o;
}

static bool q_layer_ok(int bits, const llmdec_config &c) {
  return q_ok(bits, qkv_cols(c), c.hidden) && q_ok(bits, c.hidden, c.hidden) && q_ok(bits, 2 * c.intermediate, c.hidden) &&
         q_ok(bits, c.hidden, c.intermediate) && c.intermediate % 2 == 0;
}

static size_t q_matrix_bytes_api(int bits, int32_t rows, int32_t cols) {
  return q_ok(bits, rows, cols) ? q_matrix_bytes(bits, rows, cols) : 0;
}

static llmdec_status q_pack_matrix(int bits, const char *who, int32_t rows, int32_t cols, const llmdec_q8_matrix *src,
                                   void *dst, size_t dst_bytes, llmdec_stream stream) {
  if (!q_src_ok(src) || !dst) return set_error(LLMDEC_E_INVALID, "%s: NULL pointer", who);
  if (!q_ok(bits, rows, cols))
    return set_error(LLMDEC_E_INVALID,
                     "%s: rows (%d) must be a positive multiple of 4, cols (%d) a positive multiple of 16 and at most "
                     "14336", who, rows, cols);
  const size_t need = q_matrix_bytes(bits, rows, cols);
  if (dst_bytes < need) return set_error(LLMDEC_E_INVALID, "%s: dst holds %zu bytes, %zu needed", who, dst_bytes, need);
  launch_q_pack(bits, (const uint8_t *)src->codes, (const uint16_t *)src->scales, (const uint8_t *)src->zeros, rows,
                cols, (uint8_t *)dst, rows, 0, (hipStream_t)stream);
  return check_launch(who);
}

static size_t q_packed_layer_bytes(int bits, const char *who, const llmdec_config *cfg) {
  if (check_config(cfg, who) != LLMDEC_OK || !q_layer_ok(bits, *cfg)) return 0;
  size_t off[6];
  return q_layer_parts(bits, *cfg, off);
}

static llmdec_status q_pack_layer(int bits, const char *who, const llmdec_config *cfg, const llmdec_q8_layer_weights *in,
                                  void *dst, size_t dst_bytes, llmdec_q8_packed_layer *out, llmdec_stream stream) {
  llmdec_status st = check_config(cfg, who);
  if (st != LLMDEC_OK) return st;
  if (!in || !dst || !out || !in->attn_norm || !in->mlp_norm || !q_src_ok(&in->wq) || !q_src_ok(&in->wk) ||
      !q_src_ok(&in->wv) || !q_src_ok(&in->wo) || !q_src_ok(&in->w_gate) || !q_src_ok(&in->w_up) ||
      !q_src_ok(&in->w_down))
    return set_error(LLMDEC_E_INVALID, "%s: NULL pointer", who);
  if (!q_layer_ok(bits, *cfg))
    return set_error(LLMDEC_E_UNSUPPORTED, "%s: hidden %d / intermediate %d: quantized matrices need row counts that are "
                     "multiples of 4 and input widths that are multiples of 16, at most 14336", who, cfg->hidden,
                     cfg->intermediate);
  size_t off[6];
  const size_t need = q_layer_parts(bits, *cfg, off);
  if (dst_bytes < need) return set_error(LLMDEC_E_INVALID, "%s: dst holds %zu bytes, %zu needed", who, dst_bytes, need);
  const int h = cfg->hidden, I = cfg->intermediate, kv = kv_cols(*cfg), nqkv = qkv_cols(*cfg);
  hipStream_t s = (hipStream_t)stream;
  char *d = (char *)dst;
  if (hipMemcpyAsync(d + off[0], in->attn_norm, (size_t)h * 2, hipMemcpyDeviceToDevice, s) != hipSuccess ||
      hipMemcpyAsync(d + off[1], in->mlp_norm, (size_t)h * 2, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return set_error(LLMDEC_E_HIP, "%s: copy of the norm gains failed", who);
  auto pack = [&](const llmdec_q8_matrix &m, int rows, int cols, size_t at_off, int dst_rows, int row0) {
    launch_q_pack(bits, (const uint8_t *)m.codes, (const uint16_t *)m.scales, (const uint8_t *)m.zeros, rows, cols,
                  (uint8_t *)(d + at_off), dst_rows, row0, s);
  };
  pack(in->wq, h, h, off[2], nqkv, 0);
  pack(in->wk, kv, h, off[2], nqkv, h);
  pack(in->wv, kv, h, off[2], nqkv, h + kv);
  pack(in->wo, h, h, off[3], h, 0);
  pack(in->w_gate, I, h, off[4], 2 * I, 0);
  pack(in->w_up, I, h, off[4], 2 * I, I);
  pack(in->w_down, h, I, off[5], h, 0);
  st = check_launch(who);
  if (st != LLMDEC_OK) return st;
  out->attn_norm = d + off[0];
  out->mlp_norm = d + off[1];
  out->w_qkv = d + off[2];
  out->w_o = d + off[3];
  out->w_gu = d + off[4];
  out->w_down = d + off[5];
  return LLMDEC_OK;
}

static llmdec_status q_op_linear(int bits, const char *who, const float *a, int32_t k_dim, const void *w_packed,
                                 int32_t n_dim, float *out, int32_t accumulate, llmdec_stream stream) {
  if (!a || !w_packed || !out) return set_error(LLMDEC_E_INVALID, "%s: NULL pointer", who);
  if (!q_ok(bits, n_dim, k_dim))
    return set_error(LLMDEC_E_INVALID, "%s: n=%d k=%d unsupported (n a multiple of 4, k of 16, k <= 14336)", who,
                     n_dim, k_dim);
  launch_q_gemv(bits, a, nullptr, 0.f, (const uint8_t *)w_packed, n_dim, k_dim, accumulate ? kAccumulate : kStore,
                out, (hipStream_t)stream);
  return check_launch(who);
}

static llmdec_status q_layer_decode(int bits, const char *who, const llmdec_config *cfg,
                                    const llmdec_q8_packed_layer *w, int32_t layer, float *hidden, int32_t n_seqs,
                                    const int32_t *ctx_lens, const int32_t *block_tables, int32_t max_pages,
                                    llmdec_kv_pool *pool, void *ws, size_t ws_bytes, llmdec_stream stream) {
  llmdec_status st = check_config(cfg, who);
  if (st != LLMDEC_OK) return st;
  if (!w || !w->attn_norm || !w->mlp_norm || !w->w_qkv || !w->w_o || !w->w_gu || !w->w_down)
    return set_error(LLMDEC_E_INVALID, "%s: packed layer weights missing", who);
  if (!q_layer_ok(bits, *cfg)) return set_error(LLMDEC_E_UNSUPPORTED, "%s: shape unsupported for quantized matrices", who);
  st = check_pool(pool, *cfg, layer, who);
  if (st != LLMDEC_OK) return st;
  if (!hidden || !ctx_lens || !block_tables) return set_error(LLMDEC_E_INVALID, "%s: NULL device pointer", who);
  if (n_seqs != 1)
    return set_error(LLMDEC_E_UNSUPPORTED, "%s: n_seqs=%d; the quantized products serve one sequence", who, n_seqs);
  if (max_pages <= 0) return set_error(LLMDEC_E_INVALID, "%s: max_pages=%d out of range", who, max_pages);
  const WsLayout L = ws_layout(*cfg, 1, 1, max_pages);
  st = check_ws(ws, ws_bytes, L.total, who);
  if (st != LLMDEC_OK) return st;

  const llmdec_config &c = *cfg;
  const int h = c.hidden, I = c.intermediate, nqkv = qkv_cols(c);
  hipStream_t s = (hipStream_t)stream;
  uint32_t *err = at<uint32_t>(ws, L.err);
  // one row: the fp32 activations fit in the packed activation planes' space
  float *y = at<float>(ws, L.act_h), *u = at<float>(ws, L.act_i), *qkv = at<float>(ws, L.qkv);
  uint16_t *pk, *pv;
  pool_layer(pool, layer, &pk, &pv);
  // x += Wo . attn(rope(Wq y), rope(Wk y), Wv y),  y = RMSNorm(x): the product stages y itself
  launch_q_gemv(bits, hidden, (const uint16_t *)w->attn_norm, c.rms_eps, (const uint8_t *)w->w_qkv, nqkv, h, kStore,
                qkv, s);
  launch_rope_append(c, qkv, nullptr, Splits{}, nqkv, 1, 1, nullptr, ctx_lens, block_tables, max_pages, pk, pv,
                     pool->num_pages, err, s);
  launch_decode_attention(c, qkv, nqkv, 1, ctx_lens, block_tables, max_pages, pk, pv, pool->num_pages,
                          at<float>(ws, L.attn_part), y, nullptr, nullptr, 0, err, s);
  launch_q_gemv(bits, y, nullptr, 0.f, (const uint8_t *)w->w_o, h, h, kAccumulate, hidden, s);
  // x += Wd (silu(Wg y) * (Wu y)),  y = RMSNorm(x)
  launch_q_gemv(bits, hidden, (const uint16_t *)w->mlp_norm, c.rms_eps, (const uint8_t *)w->w_gu, 2 * I, h, kSiluMul,
                u, s);
  launch_q_gemv(bits, u, nullptr, 0.f, (const uint8_t *)w->w_down, h, I, kAccumulate, hidden, s);
  return check_launch(who);
}

// 8-bit codes
extern "C" size_t llmdec_q8_matrix_bytes(int32_t rows, int32_t cols) { return q_matrix_bytes_api(8, rows, cols); }
extern "C" llmdec_status llmdec_q8_pack_matrix(int32_t rows, int32_t cols, const llmdec_q8_matrix *src, void *dst,
                                              size_t dst_bytes, llmdec_stream stream) {
  return q_pack_matrix(8, "q8_pack_matrix", rows, cols, src, dst, dst_bytes, stream);
}
extern "C" size_t llmdec_q8_packed_layer_bytes(const llmdec_config *cfg) {
  return q_packed_layer_bytes(8, "q8_packed_layer_bytes", cfg);
}
extern "C" llmdec_status llmdec_q8_pack_layer(const llmdec_config *cfg, const llmdec_q8_layer_weights *in, void *dst,
                                             size_t dst_bytes, llmdec_q8_packed_layer *out, llmdec_stream stream) {
  return q_pack_layer(8, "q8_pack_layer", cfg, in, dst, dst_bytes, out, stream);
}
extern "C" llmdec_status llmdec_op_linear_q8(const float *a, int32_t k_dim, const void *w_q8_packed, int32_t n_dim,
                                            float *out, int32_t accumulate, llmdec_stream stream) {
  return q_op_linear(8, "op_linear_q8", a, k_dim, w_q8_packed, n_dim, out, accumulate, stream);
}
extern "C" llmdec_status llmdec_layer_decode_q8(const llmdec_config *cfg, const llmdec_q8_packed_layer *w,
                                               int32_t layer, float *hidden, int32_t n_seqs, const int32_t *ctx_lens,
                                               const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool,
                                               void *ws, size_t ws_bytes, llmdec_stream stream) {
  return q_layer_decode(8, "layer_decode_q8", cfg, w, layer, hidden, n_seqs, ctx_lens, block_tables, max_pages, pool,
                        ws, ws_bytes, stream);
}

// 4-bit codes
extern "C" size_t llmdec_q4_matrix_bytes(int32_t rows, int32_t cols) { return q_matrix_bytes_api(4, rows, cols); }
extern "C" llmdec_status llmdec_q4_pack_matrix(int32_t rows, int32_t cols, const llmdec_q4_matrix *src, void *dst,
                                              size_t dst_bytes, llmdec_stream stream) {
  return q_pack_matrix(4, "q4_pack_matrix", rows, cols, src, dst, dst_bytes, stream);
}
extern "C" size_t llmdec_q4_packed_layer_bytes(const llmdec_config *cfg) {
  return q_packed_layer_bytes(4, "q4_packed_layer_bytes", cfg);
}
extern "C" llmdec_status llmdec_q4_pack_layer(const llmdec_config *cfg, const llmdec_q4_layer_weights *in, void *dst,
                                             size_t dst_bytes, llmdec_q4_packed_layer *out, llmdec_stream stream) {
  return q_pack_layer(4, "q4_pack_layer", cfg, in, dst, dst_bytes, out, stream);
}
extern "C" llmdec_status llmdec_op_linear_q4(const float *a, int32_t k_dim, const void *w_q4_packed, int32_t n_dim,
                                            float *out, int32_t accumulate, llmdec_stream stream) {
  return q_op_linear(4, "op_linear_q4", a, k_dim, w_q4_packed, n_dim, out, accumulate, stream);
}
extern "C" llmdec_status llmdec_layer_decode_q4(const llmdec_config *cfg, const llmdec_q4_packed_layer *w,
                                               int32_t layer, float *hidden, int32_t n_seqs, const int32_t *ctx_lens,
                                               const int32_t *block_tables, int32_t max_pages, llmdec_kv_pool *pool,
                                               void *ws, size_t ws_bytes, llmdec_stream stream) {
  return q_layer_decode(4, "layer_decode_q4", cfg, w, layer, hidden, n_seqs, ctx_lens, block_tables, max_pages, pool,
                        ws, ws_bytes, stream);
}
