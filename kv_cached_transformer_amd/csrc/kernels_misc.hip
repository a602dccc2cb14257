// Small bandwidth-bound kernels: weight packing, embedding lookup, RMSNorm,
// fp32 -> packed fp16 activation, rotary embedding + paged KV append, SwiGLU gate,
// argmax, and the test-only cache gather.
#include <math.h>

#include <algorithm>

#include "bodies.h"

namespace llmdec {

// ---------------------------------------------------------------- packing
// A packed matrix holds fp16(w * 2^s) in the tile layout, then a trailer whose first word is the largest
// |w| of every source it holds (fp32 bits); s = weight_shift(that word).  The trailer is cleared, every
// source's largest magnitude folded in, and only then are the sources packed.
size_t packed_tiles_bytes(int rows, int cols) { return (size_t)rows * round_up(cols, kTileK) * sizeof(uint16_t); }

void launch_weight_trailer_clear(uint16_t *dst, size_t tiles_bytes, hipStream_t s) {
  launch_fill_u32(reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(dst) + tiles_bytes), 0u, kWTrailer / 4, s);
}

// Largest finite |w| of a bf16 matrix, as the fp32 bits of |w| (non-negative floats order as integers),
// folded into the trailer word with an atomic maximum.  Infinities and NaNs are left out.
__global__ __launch_bounds__(256) void weight_absmax_kernel(const uint16_t *__restrict__ src, size_t n,
                                                            uint32_t *__restrict__ out) {
  uint32_t m = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const uint32_t b = src[i] & 0x7fffu;
    if (b < 0x7f80u) m = b > m ? b : m;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t v = (uint32_t)__shfl_xor((int)m, o, 64);
    m = v > m ? v : m;
  }
  if ((threadIdx.x & 63) == 0 && m) atomicMax(out, m << 16);
}

void launch_weight_absmax(int rows, int cols, const uint16_t *src, uint16_t *dst, size_t tiles_bytes, hipStream_t s) {
  const size_t n = (size_t)rows * cols;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 2048);
  if (n)
    weight_absmax_kernel<<<blocks, 256, 0, s>>>(
        src, n, reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(dst) + tiles_bytes));
}

// One thread moves the 8 elements one lane owns in one tile: bf16 w -> fp16(w * 2^s), exact for every
// weight within 2^31 of the matrix's largest (see weight_shift).
__global__ void pack_matrix_kernel(int rows, int cols, int kt_count, int nb_stride, const uint16_t *__restrict__ src,
                                   uint16_t *__restrict__ dst, const uint32_t *__restrict__ trailer) {
  const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t n_slots = (size_t)(rows / 16) * kt_count * 64;
  if (g >= n_slots) return;
  const float scale = __builtin_ldexpf(1.0f, weight_shift(*trailer));
  const int lane = (int)(g & 63);
  const size_t tile = g >> 6;
  const int nb = (int)(tile / kt_count), kt = (int)(tile % kt_count);
  const int r = nb * 16 + (lane & 15);
  const int c0 = kt * 32 + (lane >> 4) * 8;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (c0 + j < cols) ? bf16_to_f32(src[(size_t)r * cols + c0 + j]) * scale : 0.f;
  const size_t dtile = (size_t)nb * nb_stride * kt_count + kt;
  *reinterpret_cast<uint4 *>(dst + (dtile * 64 + lane) * 8) = pack8_f16(v);
}

void launch_pack_matrix(int rows, int cols, const uint16_t *src, uint16_t *dst, size_t tiles_bytes, hipStream_t s,
                        int nb_stride) {
  const int kt = round_up(cols, kTileK) / kTileK;
  const size_t n = (size_t)(rows / 16) * kt * 64;
  const uint32_t *trailer = reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(dst) + tiles_bytes);
  if (n) pack_matrix_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(rows, cols, kt, nb_stride, src, dst, trailer);
}

// ---------------------------------------------------------------- embedding ([F] §2.2.1: row lookup)
__global__ void embed_kernel(const uint16_t *__restrict__ embed, const int32_t *__restrict__ tokens, int hidden,
                             int vocab, float *__restrict__ x, uint32_t *err) {
  const int t = blockIdx.x;
  const int tok = tokens[t];
  const bool ok = tok >= 0 && tok < vocab;
  if (!ok && threadIdx.x == 0) raise_error(err, kErrToken);
  const uint16_t *row = embed + (size_t)(ok ? tok : 0) * hidden;
  for (int i = threadIdx.x; i < hidden; i += blockDim.x) x[(size_t)t * hidden + i] = ok ? bf16_to_f32(row[i]) : 0.f;
}

void launch_embed(const uint16_t *embed, const int32_t *tokens, int n_tokens, int hidden, int vocab, float *x,
                  uint32_t *err, hipStream_t s) {
  if (n_tokens > 0) embed_kernel<<<n_tokens, 256, 0, s>>>(embed, tokens, hidden, vocab, x, err);
}

// ---------------------------------------------------------------- RMSNorm ([E] §4.2)
// y = x * (mean(x^2) + eps)^(-1/2) * gamma, eps inside the root.  One block of
// 512 threads per row; each thread owns runs of 8 consecutive columns (up to
// two runs: n <= 8192), kept in registers between the two passes, and each run
// is one 16-byte chunk of the packed fp16 output.  Columns n..kpad-1 of the packed
// output are zeroed.  With add_partials, the ks partial sums of a split-k
// residual product are first added into x (and x written back): the residual
// add of the output projection fused into the norm that follows it.
constexpr int kNormThreads = 512;
constexpr int kNormRuns = 2;

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(float *__restrict__ x, int ld_x,
                                                      const int32_t *__restrict__ cu_last, int n_src_rows,
                                                      const uint16_t *__restrict__ gamma, int n, float eps,
                                                      uint32_t *err, float *out_f32, uint16_t *out_act,
                                                      uint16_t *out_lo, int kpad, const float *__restrict__ add,
                                                      Splits sp, int rows) {
  __shared__ float red[kNormThreads / 64];
  norm_row<kNormThreads, kNormRuns>(blockIdx.x, red, x, ld_x, cu_last, n_src_rows, gamma, n, eps, err, out_f32,
                                    out_act, out_lo, kpad, add, sp, rows);
}

// Many-row form (a prefill's rows, packed output only): a block of 16 waves takes 8 rows, so that its
// stores fill whole 128-byte runs of the packed tiles (a tile holds 16 rows, each row 16 bytes of every
// 256-byte quarter) instead of one 16-byte piece per row.  Lane l holds row l % 8 and, of each 64-column
// group, columns 8 (l / 8) .. + 7; wave w takes groups w*CG .. w*CG + CG - 1.  The 8 lanes of a row add
// their squares with shuffles, the waves through LDS.  With one block per CU (2048 rows: 256 blocks),
// 16 waves keep more loads in flight than 4 (7B prefill norm: 17.3 -> 12.3 us; 8 waves: 13.8 us).
constexpr int kRows8Waves = 16;
template <int CG>
__global__ __launch_bounds__(64 * kRows8Waves) void rmsnorm_rows8_kernel(const float *__restrict__ x, int ld_x,
                                                            const uint16_t *__restrict__ gamma, int n, float eps,
                                                            uint16_t *out_act, uint16_t *out_lo, int kpad, int rows) {
  __shared__ float red[kRows8Waves][8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane & 7, piece = lane >> 3;
  const int r = blockIdx.x * 8 + rl;
  const bool row_ok = r < rows;
  const float *xr = x + (size_t)(row_ok ? r : 0) * ld_x;
  float v[CG][8];
  uint4 gw[CG];
  float ss = 0.f;
#pragma unroll
  for (int g = 0; g < CG; ++g) {
    const int c0 = (wave * CG + g) * 64 + piece * 8;
    if (row_ok && c0 < n) {
      const float4 a = *reinterpret_cast<const float4 *>(xr + c0), b = *reinterpret_cast<const float4 *>(xr + c0 + 4);
      gw[g] = *reinterpret_cast<const uint4 *>(gamma + c0);
      v[g][0] = a.x, v[g][1] = a.y, v[g][2] = a.z, v[g][3] = a.w;
      v[g][4] = b.x, v[g][5] = b.y, v[g][6] = b.z, v[g][7] = b.w;
    } else {
      gw[g] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[g][j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[g][j], v[g][j], ss);
  }
  ss += __shfl_xor(ss, 8, 64);
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  if (lane < 8) red[wave][lane] = ss;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kRows8Waves; ++w) total += red[w][rl];
  const float inv = 1.0f / sqrtf(total / (float)n + eps);
  if (!row_ok) return;
  const int kt = kpad >> 5;
#pragma unroll
  for (int g = 0; g < CG; ++g) {
    const int c0 = (wave * CG + g) * 64 + piece * 8;
    if (c0 >= kpad) continue;
    const uint32_t gg[4] = {gw[g].x, gw[g].y, gw[g].z, gw[g].w};
    float y[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // past n: zeros (x and gamma were read as zeros)
      y[2 * j] = v[g][2 * j] * inv * bf16lo(gg[j]);
      y[2 * j + 1] = v[g][2 * j + 1] * inv * bf16hi(gg[j]);
    }
    const size_t off = packed_offset(r, c0, kt);
    if (out_lo) {
      uint4 h, l;
      pack8_f16x2(y, h, l);
      *reinterpret_cast<uint4 *>(out_act + off) = h;
      *reinterpret_cast<uint4 *>(out_lo + off) = l;
    } else {
      *reinterpret_cast<uint4 *>(out_act + off) = pack8_f16(y);
    }
  }
}

template <int CG>
static void launch_rows8(const float *x, int ld_x, const uint16_t *gamma, int rows, int n, float eps,
                         uint16_t *out_act, uint16_t *out_lo, int kpad, hipStream_t s) {
  rmsnorm_rows8_kernel<CG><<<(rows + 7) / 8, 64 * kRows8Waves, 0, s>>>(x, ld_x, gamma, n, eps, out_act, out_lo, kpad,
                                                                       rows);
}

void launch_rmsnorm(float *x, int ld_x, const int32_t *cu_last, int n_src_rows, const uint16_t *gamma, int rows, int n,
                    float eps, uint32_t *err, float *out_f32, uint16_t *out_act, uint16_t *out_lo, int kpad,
                    const float *add_partials, const Splits &sp, hipStream_t s) {
  if (rows <= 0) return;
  const int groups = (kpad + 63) / 64;  // 64-column groups, 4 waves share them
  if (rows > 64 && out_act && !out_f32 && !add_partials && !cu_last && groups <= kRows8Waves * 8) {
    if (groups <= kRows8Waves) launch_rows8<1>(x, ld_x, gamma, rows, n, eps, out_act, out_lo, kpad, s);
    else if (groups <= kRows8Waves * 2) launch_rows8<2>(x, ld_x, gamma, rows, n, eps, out_act, out_lo, kpad, s);
    else if (groups <= kRows8Waves * 4) launch_rows8<4>(x, ld_x, gamma, rows, n, eps, out_act, out_lo, kpad, s);
    else launch_rows8<8>(x, ld_x, gamma, rows, n, eps, out_act, out_lo, kpad, s);
    return;
  }
  rmsnorm_kernel<<<rows, kNormThreads, 0, s>>>(x, ld_x, cu_last, n_src_rows, gamma, n, eps, err, out_f32, out_act,
                                               out_lo, kpad, add_partials, sp, rows);
}

// ---------------------------------------------------------------- fp32 -> packed fp16 activation
__global__ void split_kernel(const float *__restrict__ a, int ld, int rows, int cols, uint16_t *act, uint16_t *lo,
                             int kpad) {
  const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = kpad / 8;
  if (g >= (size_t)rows * per_row) return;
  const int r = (int)(g / per_row), c0 = (int)(g % per_row) * 8;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = c0 + j < cols ? a[(size_t)r * ld + c0 + j] : 0.f;
  const size_t off = packed_offset(r, c0, kpad >> 5);
  if (lo) {
    uint4 h, l;
    pack8_f16x2(v, h, l);
    *reinterpret_cast<uint4 *>(act + off) = h;
    *reinterpret_cast<uint4 *>(lo + off) = l;
  } else {
    *reinterpret_cast<uint4 *>(act + off) = pack8_f16(v);
  }
}

void launch_split(const float *a, int ld, int rows, int cols, uint16_t *act, uint16_t *lo, int kpad, hipStream_t s) {
  const size_t n = (size_t)rows * (kpad / 8);
  if (n) split_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a, ld, rows, cols, act, lo, kpad);
}

// ---------------------------------------------------------------- token -> (sequence, position)
// Sequence s owns tokens cu[s]..cu[s+1]-1; a table that is not increasing
// within [0, n_tokens] (every sequence carries at least one new token), does
// not end at n_tokens, or a negative start is flagged and that sequence's
// tokens are not written.
__global__ void token_map_kernel(const int32_t *__restrict__ cu, const int32_t *__restrict__ start, int n_seqs,
                                 int n_tokens, uint32_t *err, int32_t *tok_seq, int32_t *tok_pos) {
  const int s = blockIdx.x;
  const int b = cu[s], e = cu[s + 1], p0 = start[s];
  const bool bad = b < 0 || e <= b || e > n_tokens || p0 < 0 || (s == n_seqs - 1 && e != n_tokens) || (s == 0 && b != 0);
  if (bad) {
    if (threadIdx.x == 0) raise_error(err, kErrSeq);
    return;
  }
  for (int i = b + threadIdx.x; i < e; i += blockDim.x) {
    tok_seq[i] = s;
    tok_pos[i] = p0 + (i - b);
  }
}

void launch_token_map(const int32_t *cu, const int32_t *start, int n_seqs, int n_tokens, uint32_t *err,
                      int32_t *tok_seq, int32_t *tok_pos, hipStream_t s) {
  if (n_seqs > 0) token_map_kernel<<<n_seqs, 256, 0, s>>>(cu, start, n_seqs, n_tokens, err, tok_seq, tok_pos);
}

// ---------------------------------------------------------------- RoPE + paged append ([E] §4.3)
// One block per (new token, chunk of heads holding 256 rotation pairs).  Pair i
// of every head turns by pos * inv_freq[i],
// inv_freq[i] = theta^(-2i/D) computed in double on the host; the angle is
// formed and reduced to a fraction of a turn in double, then its sine and
// cosine taken in fp32, so positions in the thousands lose no accuracy.  q is rotated in
// place; rotated k and plain v are rounded to bf16 and written to the page
// slot bt[seq][pos/16], offset pos%16 (K as [h][o][d], V as [h][o/4][d][o%4]).
__global__ __launch_bounds__(256) void rope_append_kernel(float *__restrict__ qkv, const float *__restrict__ part,
                                                          Splits sp, int ld_qkv, int n_tokens, int n_heads,
                                                          int n_kv_heads, int head_dim, RopeFreq fr, int n_seqs,
                                                          const int32_t *__restrict__ tok_seq,
                                                          const int32_t *__restrict__ tok_pos,
                                                          const int32_t *__restrict__ block_tables, int max_pages,
                                                          uint16_t *__restrict__ pool_k, uint16_t *__restrict__ pool_v,
                                                          int num_pages, uint32_t *err) {
  __shared__ float cs[64], sn[64];
  rope_item(blockIdx.x, blockIdx.y, cs, sn, qkv, part, sp, ld_qkv, n_tokens, n_heads, n_kv_heads, head_dim, fr,
            n_seqs, tok_seq, tok_pos, block_tables, max_pages, pool_k, pool_v, num_pages, err);
}

RopeFreq rope_freq(const llmdec_config &cfg) {
  RopeFreq fr;
  for (int i = 0; i < 64; ++i)
    fr.inv_freq[i] = i < cfg.head_dim / 2 ? pow((double)cfg.rope_theta, -2.0 * i / (double)cfg.head_dim) : 0.0;
  return fr;
}

void launch_rope_append(const llmdec_config &cfg, float *qkv, const float *qkv_partials, const Splits &sp, int ld_qkv,
                        int n_tokens, int n_seqs, const int32_t *tok_seq, const int32_t *tok_pos,
                        const int32_t *block_tables, int max_pages, uint16_t *pool_k, uint16_t *pool_v, int num_pages,
                        uint32_t *err, hipStream_t s) {
  if (n_tokens <= 0) return;
  const RopeFreq fr = rope_freq(cfg);
  dim3 grid(n_tokens, (cfg.n_heads * (cfg.head_dim / 2) + 255) / 256);
  rope_append_kernel<<<grid, 256, 0, s>>>(qkv, qkv_partials, sp, ld_qkv, n_tokens, cfg.n_heads, cfg.n_kv_heads,
                                              cfg.head_dim, fr, n_seqs, tok_seq, tok_pos, block_tables, max_pages,
                                              pool_k, pool_v, num_pages, err);
}

// ---------------------------------------------------------------- SwiGLU gate ([W] §1.2, [E] §4.2)
// Stand-alone form: u = silu(g) * up, silu(z) = z / (1 + e^-z).
__global__ void silu_mul_kernel(const float *__restrict__ g, const float *__restrict__ u, size_t n,
                                float *__restrict__ out) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float gv = g[i];
  out[i] = gv / (1.0f + expf(-gv)) * u[i];
}

void launch_silu_mul(const float *g, const float *u, int rows, int n, float *out, hipStream_t s) {
  const size_t total = (size_t)rows * n;
  if (total) silu_mul_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(g, u, total, out);
}

// ---------------------------------------------------------------- greedy argmax ([F] §2.2.3)
// Largest logit per row; among equal values the lowest index wins.  One 1024-thread block per row:
// every thread has its four 16-byte loads per pass in flight at once, so a 32000-logit row is read
// in one or two memory latencies.  vocab is a multiple of 16 (the lm_head is tiled by 16 rows), so
// rows are 16-byte aligned.
constexpr int kArgmaxThreads = 1024;
__global__ __launch_bounds__(kArgmaxThreads) void argmax_kernel(const float *__restrict__ logits, int vocab,
                                                                int32_t *next) {
  const int r = blockIdx.x;
  const float4 *x4 = reinterpret_cast<const float4 *>(logits + (size_t)r * vocab);
  const int n4 = vocab >> 2;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  // indices visited per thread are ascending, so a strict > keeps the first of equal values
  for (int i0 = threadIdx.x; i0 < n4; i0 += 4 * kArgmaxThreads) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = x4[min(i0 + u * kArgmaxThreads, n4 - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kArgmaxThreads;
      if (i >= n4) break;
      const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (e[j] > best) {
          best = e[j];
          bi = 4 * i + j;
        }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > best || (ov == best && oi < bi)) {
      best = ov;
      bi = oi;
    }
  }
  constexpr int NW = kArgmaxThreads / 64;
  __shared__ float bv[NW];
  __shared__ int bix[NW];
  if ((threadIdx.x & 63) == 0) {
    bv[threadIdx.x >> 6] = best;
    bix[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < NW; ++w)
      if (bv[w] > best || (bv[w] == best && bix[w] < bi)) {
        best = bv[w];
        bi = bix[w];
      }
    next[r] = (bi == 0x7fffffff) ? 0 : bi;
  }
}

void launch_argmax(const float *logits, int rows, int vocab, int32_t *next, hipStream_t s) {
  if (rows > 0 && vocab > 0 && vocab % 4 == 0) argmax_kernel<<<rows, kArgmaxThreads, 0, s>>>(logits, vocab, next);
}

// ---------------------------------------------------------------- test-only gather
__global__ void gather_kv_kernel(const uint16_t *__restrict__ pk, const uint16_t *__restrict__ pv, int num_pages,
                                 int n_heads, int head_dim, const int32_t *__restrict__ row, uint16_t *k_out,
                                 uint16_t *v_out) {
  const int p = blockIdx.x;
  const int page = row[p >> 4], off = p & 15;
  const bool ok = page >= 0 && page < num_pages;
  for (int e = threadIdx.x; e < n_heads * head_dim; e += blockDim.x) {
    const int h = e / head_dim, d = e % head_dim;
    const size_t o = (size_t)p * n_heads * head_dim + e;
    k_out[o] = ok ? pk[(((size_t)page * n_heads + h) * 16 + off) * head_dim + d] : (uint16_t)0xffff;
    v_out[o] = ok ? pv[((((size_t)page * n_heads + h) * 4 + (off >> 2)) * head_dim + d) * 4 + (off & 3)] : (uint16_t)0xffff;
  }
}

void launch_gather_kv(const uint16_t *pk, const uint16_t *pv, int num_pages, int n_heads, int head_dim,
                      const int32_t *row, int n_tokens, uint16_t *k_out, uint16_t *v_out, hipStream_t s) {
  if (n_tokens > 0) gather_kv_kernel<<<n_tokens, 256, 0, s>>>(pk, pv, num_pages, n_heads, head_dim, row, k_out, v_out);
}

__global__ void fill_u32_kernel(uint32_t *p, uint32_t value, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

__global__ void copy_u32_kernel(const uint32_t *src, uint32_t *dst) { *dst = *src; }

void launch_copy_u32(const uint32_t *src, uint32_t *dst, hipStream_t s) { copy_u32_kernel<<<1, 1, 0, s>>>(src, dst); }

void launch_fill_u32(uint32_t *p, uint32_t value, size_t n, hipStream_t s) {
  if (n) fill_u32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, value, n);
}

}  // namespace llmdec
