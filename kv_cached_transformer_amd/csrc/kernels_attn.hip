// Attention over the paged KV cache ([E] §4.3: softmax(q K^T / sqrt(D)) V with
// the causal mask; [E] §3.4: keys found through the page index).
//
// Pool layout per layer: K[page][h][16][D], V[page][h][D][16].
//
// Decode: one wave per (sequence, head, partition of pages).  Lane l takes
// token l/4 of each page and a quarter of the head dimension of its key, so a
// page's K block (4 KiB at D = 128) is one coalesced read; the 16 scores are
// reduced in-wave, the running max is wave-uniform per page (one rescale per
// page), and for P.V lane l owns dims 2l, 2l+1, whose 16 values per page are
// contiguous in the transposed V block.  Partitions are merged by a
// log-sum-exp combine kernel.
//
// Prefill: MFMA.  Scores are formed transposed, S^T = K Q^T (keys as rows),
// so a lane's accumulator holds 4 keys of one query: exactly the operand
// slots the P.V product O^T = V^T P^T needs, with no shuffle through LDS.  q
// and p are split into three bf16 parts each (hi + mid + lo carries fp32's
// 24 bits; three MFMAs per product), K and V are the stored bf16 values, so
// the scores and the weighted sum keep fp32-level accuracy.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace llmdec {

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline f32x4 mfma16(const uint4 &a, const uint4 &b, f32x4 c) {
  bf16x8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

// A 32-bit word holding the bf16 values of tokens t and t+1: keep only those below n_valid.
__device__ inline uint32_t mask_pair(uint32_t w, int t, int n_valid) {
  return t + 1 < n_valid ? w : (t < n_valid ? (w & 0xffffu) : 0u);
}

// The attention output feeds the o projection as a packed hi/lo activation pair; the stand-alone
// operation also (or only) writes fp32.
__device__ inline void store_out(float v, int r, int c, int ld, float *out_f32, uint16_t *out_hi, uint16_t *out_lo,
                                 int kpad) {
  if (out_f32) out_f32[(size_t)r * ld + c] = v;
  if (out_hi) {
    uint16_t h, l;
    split_bf16(v, h, l);
    const size_t o = packed_offset(r, c, kpad >> 5);
    out_hi[o] = h;
    out_lo[o] = l;
  }
}

// ---------------------------------------------------------------- decode
template <int D>
__global__ __launch_bounds__(64) void decode_attn_kernel(const float *__restrict__ q, int ld_q, int n_heads,
                                                         const int32_t *__restrict__ ctx_lens,
                                                         const int32_t *__restrict__ block_tables, int max_pages,
                                                         const uint16_t *__restrict__ pool_k,
                                                         const uint16_t *__restrict__ pool_v, int num_pages, int ppp,
                                                         int n_parts, float *__restrict__ partials, float *out_f32,
                                                         uint16_t *out_hi, uint16_t *out_lo, int kpad, uint32_t *err) {
  constexpr int DK = D / 4;   // key dims per lane
  constexpr int DV = D / 64;  // value dims per lane
  const int part = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x;
  const int n_tok = ctx_lens[s] + 1;
  const int n_pages = (n_tok + 15) >> 4;
  const int p0 = part * ppp;
  if (n_tok <= 0) {
    if (lane == 0 && part == 0) raise_error(err, kErrPos);
    return;
  }
  if (p0 >= n_pages) return;
  if (n_pages > max_pages) {
    if (lane == 0) raise_error(err, kErrPos);
    return;
  }
  const int p1 = min(n_pages, p0 + ppp);
  const float scale = kLog2e * rsqrtf((float)D);
  float qr[DK];
  {
    const float *qp = q + (size_t)s * ld_q + h * D + (lane & 3) * DK;
#pragma unroll
    for (int i = 0; i < DK; i += 4) {
      const float4 v = *reinterpret_cast<const float4 *>(qp + i);
      qr[i] = v.x * scale;
      qr[i + 1] = v.y * scale;
      qr[i + 2] = v.z * scale;
      qr[i + 3] = v.w * scale;
    }
  }
  float m = -1e30f, l = 0.f, o[DV];
#pragma unroll
  for (int i = 0; i < DV; ++i) o[i] = 0.f;
  const int tok = lane >> 2;
  const int32_t *bt = block_tables + (size_t)s * max_pages;
  for (int pi = p0; pi < p1; ++pi) {
    int pg = bt[pi];
    if (pg < 0 || pg >= num_pages) {
      if (lane == 0) raise_error(err, kErrPage);
      pg = -1;
    }
    const bool valid = pg >= 0 && pi * 16 + tok < n_tok;
    float sc = -INFINITY;
    uint4 vv[DV * 2];
    if (pg >= 0) {
      const uint4 *kp = reinterpret_cast<const uint4 *>(pool_k + (((size_t)pg * n_heads + h) * 16 + tok) * D + (lane & 3) * DK);
      uint4 kk[DK / 8];
#pragma unroll
      for (int i = 0; i < DK / 8; ++i) kk[i] = kp[i];
      const uint4 *vp = reinterpret_cast<const uint4 *>(pool_v + (((size_t)pg * n_heads + h) * D + lane * DV) * 16);
#pragma unroll
      for (int i = 0; i < DV * 2; ++i) vv[i] = vp[i];
      // slots past the last token hold whatever the pool held (possibly NaN): their weight is 0,
      // and 0 * NaN would poison the sum, so their values are cleared
      const int n_valid = n_tok - pi * 16;
      if (n_valid < 16) {
#pragma unroll
        for (int i = 0; i < DV * 2; ++i) {
          vv[i].x = mask_pair(vv[i].x, (i & 1) * 8 + 0, n_valid);
          vv[i].y = mask_pair(vv[i].y, (i & 1) * 8 + 2, n_valid);
          vv[i].z = mask_pair(vv[i].z, (i & 1) * 8 + 4, n_valid);
          vv[i].w = mask_pair(vv[i].w, (i & 1) * 8 + 6, n_valid);
        }
      }
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DK / 8; ++i) {
        const uint32_t w[4] = {kk[i].x, kk[i].y, kk[i].z, kk[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc = fmaf(bf16lo(w[j]), qr[i * 8 + 2 * j], acc);
          acc = fmaf(bf16hi(w[j]), qr[i * 8 + 2 * j + 1], acc);
        }
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      if (valid) sc = acc;
    } else {
#pragma unroll
      for (int i = 0; i < DV * 2; ++i) vv[i] = make_uint4(0, 0, 0, 0);
    }
    const float pm = wave_max(sc);
    const float m_new = fmaxf(m, pm);
    const float alpha = exp2f(m - m_new);
    const float p = valid ? exp2f(sc - m_new) : 0.f;
    l = l * alpha + wave_sum((lane & 3) == 0 ? p : 0.f);
#pragma unroll
    for (int i = 0; i < DV; ++i) o[i] *= alpha;
    m = m_new;
    float pts[16];  // p of token t sits in lanes 4t..4t+3
#pragma unroll
    for (int t = 0; t < 16; ++t) pts[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 4 * t));
#pragma unroll
    for (int i = 0; i < DV; ++i) {
      const uint32_t w[8] = {vv[2 * i].x, vv[2 * i].y, vv[2 * i].z, vv[2 * i].w,
                             vv[2 * i + 1].x, vv[2 * i + 1].y, vv[2 * i + 1].z, vv[2 * i + 1].w};
      float acc = o[i];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc = fmaf(pts[2 * j], bf16lo(w[j]), acc);
        acc = fmaf(pts[2 * j + 1], bf16hi(w[j]), acc);
      }
      o[i] = acc;
    }
  }
  const int parts_here = (n_pages + ppp - 1) / ppp;
  if (parts_here == 1) {
    const float inv = 1.f / l;
#pragma unroll
    for (int i = 0; i < DV; ++i) store_out(o[i] * inv, s, h * D + lane * DV + i, n_heads * D, out_f32, out_hi, out_lo, kpad);
  } else {
    float *pp = partials + (((size_t)s * n_heads + h) * n_parts + part) * (D + 2);
    if (lane == 0) {
      pp[0] = m;
      pp[1] = l;
    }
#pragma unroll
    for (int i = 0; i < DV; ++i) pp[2 + lane * DV + i] = o[i];
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(int n_heads, const int32_t *__restrict__ ctx_lens,
                                                           int max_pages, int ppp, int n_parts,
                                                           const float *__restrict__ partials, float *out_f32,
                                                           uint16_t *out_hi, uint16_t *out_lo, int kpad) {
  const int s = blockIdx.x / n_heads, h = blockIdx.x % n_heads;
  const int n_pages = (ctx_lens[s] + 1 + 15) >> 4;
  if (n_pages > max_pages || n_pages <= 0) return;
  const int parts = (n_pages + ppp - 1) / ppp;
  if (parts <= 1) return;
  const float *pp = partials + ((size_t)s * n_heads + h) * n_parts * (D + 2);
  float mx = -1e30f;
  for (int i = 0; i < parts; ++i) mx = fmaxf(mx, pp[i * (D + 2)]);
  float L = 0.f, acc = 0.f;
  const int d = threadIdx.x;
  for (int i = 0; i < parts; ++i) {
    const float w = exp2f(pp[i * (D + 2)] - mx);
    L = fmaf(pp[i * (D + 2) + 1], w, L);
    acc = fmaf(pp[i * (D + 2) + 2 + d], w, acc);
  }
  store_out(acc / L, s, h * D + d, n_heads * D, out_f32, out_hi, out_lo, kpad);
}

void decode_partition(int n_seqs, int n_heads, int max_pages, int *pages_per_part, int *n_parts) {
  // Aim for ~8 waves per CU over 256 CUs counting every (sequence, head) row
  // at full width; never split finer than one page, never coarser than 32.
  const long rows = (long)n_seqs * n_heads;
  int parts = (int)((2048 + rows - 1) / rows);
  parts = parts < 1 ? 1 : parts;
  int ppp = (max_pages + parts - 1) / parts;
  ppp = ppp < 1 ? 1 : (ppp > 32 ? 32 : ppp);
  *pages_per_part = ppp;
  *n_parts = (max_pages + ppp - 1) / ppp;
}

void launch_decode_attention(const llmdec_config &cfg, const float *q, int ld_q, int n_seqs, const int32_t *ctx_lens,
                             const int32_t *block_tables, int max_pages, const uint16_t *pk, const uint16_t *pv,
                             int num_pages, float *partials, float *out_f32, uint16_t *out_hi, uint16_t *out_lo,
                             int kpad, uint32_t *err, hipStream_t s) {
  if (n_seqs <= 0) return;
  int ppp, n_parts;
  decode_partition(n_seqs, cfg.n_heads, max_pages, &ppp, &n_parts);
  dim3 grid(n_parts, cfg.n_heads, n_seqs);
  if (cfg.head_dim == 128) {
    decode_attn_kernel<128><<<grid, 64, 0, s>>>(q, ld_q, cfg.n_heads, ctx_lens, block_tables, max_pages, pk, pv,
                                                num_pages, ppp, n_parts, partials, out_f32, out_hi, out_lo, kpad, err);
    if (n_parts > 1)
      decode_combine_kernel<128><<<n_seqs * cfg.n_heads, 128, 0, s>>>(cfg.n_heads, ctx_lens, max_pages, ppp, n_parts,
                                                                     partials, out_f32, out_hi, out_lo, kpad);
  } else {
    decode_attn_kernel<64><<<grid, 64, 0, s>>>(q, ld_q, cfg.n_heads, ctx_lens, block_tables, max_pages, pk, pv,
                                               num_pages, ppp, n_parts, partials, out_f32, out_hi, out_lo, kpad, err);
    if (n_parts > 1)
      decode_combine_kernel<64><<<n_seqs * cfg.n_heads, 64, 0, s>>>(cfg.n_heads, ctx_lens, max_pages, ppp, n_parts,
                                                                   partials, out_f32, out_hi, out_lo, kpad);
  }
}

// ---------------------------------------------------------------- prefill (causal, MFMA)
// One wave per (sequence, head, block of 16 new tokens).  Keys are taken two
// pages (32 keys) at a time: S^T blocks for both pages, mask, online softmax
// per query, then O^T += V^T P^T over the 32 keys.
template <int D>
__global__ __launch_bounds__(64) void prefill_attn_kernel(const float *__restrict__ q, int ld_q, int n_heads,
                                                          int n_tokens, int max_q_len,
                                                          const int32_t *__restrict__ cu,
                                                          const int32_t *__restrict__ start_pos,
                                                          const int32_t *__restrict__ block_tables, int max_pages,
                                                          const uint16_t *__restrict__ pool_k,
                                                          const uint16_t *__restrict__ pool_v, int num_pages,
                                                          float *out_f32, uint16_t *out_hi, uint16_t *out_lo, int kpad,
                                                          uint32_t *err) {
  constexpr int KT = D / 32;  // k-tiles of the head dimension
  constexpr int DB = D / 16;  // 16-dim blocks of the output
  const int qb = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
  const int t0 = cu[s], len = cu[s + 1] - t0;
  if (t0 < 0 || len < 0 || len > max_q_len || t0 + len > n_tokens || start_pos[s] < 0) {
    if (lane == 0 && qb == 0 && h == 0) raise_error(err, kErrSeq);
    return;
  }
  if (qb * 16 >= len) return;
  const int n_q = min(16, len - qb * 16);
  const int pos0 = start_pos[s] + qb * 16;  // position of query 0 of this block
  const int my_pos = pos0 + c;               // position of this lane's query
  const bool q_ok = c < n_q;
  const float scale = kLog2e * rsqrtf((float)D);

  // Q^T operand: lane (g, c) holds dims 32kt + 8g .. +7 of query c as three bf16 parts
  // (q = hi + mid + lo to fp32 precision).
  uint4 qs[3][KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    float qv[8];
    if (q_ok) {
      const float *qp = q + (size_t)(t0 + qb * 16 + c) * ld_q + h * D + kt * 32 + g * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[j] = qp[j] * scale;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[j] = 0.f;
    }
    split3_pack8(qv, qs[0][kt], qs[1][kt], qs[2][kt]);
  }
  const int last_pos = pos0 + n_q - 1;
  const int n_kpages = (last_pos >> 4) + 1;
  if (n_kpages > max_pages) {
    if (lane == 0) raise_error(err, kErrPos);
    return;
  }
  const int32_t *bt = block_tables + (size_t)s * max_pages;
  f32x4 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -1e30f, l = 0.f;

  for (int pa = 0; pa < n_kpages; pa += 2) {
    int pgs[2];
    float sc[2][4];
    uint2 vt[DB][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pi = pa + u;
      int pg = -1;
      if (pi < n_kpages) {
        pg = bt[pi];
        if (pg < 0 || pg >= num_pages) {
          if (lane == 0) raise_error(err, kErrPage);
          pg = -1;
        }
      }
      pgs[u] = pg;
      f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
      if (pg >= 0) {
        const uint4 *kp = reinterpret_cast<const uint4 *>(pool_k + (((size_t)pg * n_heads + h) * 16 + c) * D + g * 8);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const uint4 kk = kp[kt * 4];  // dims 32kt + 8g .. +7 of key c
          st = mfma16(kk, qs[2][kt], st);  // smallest parts first
          st = mfma16(kk, qs[1][kt], st);
          st = mfma16(kk, qs[0][kt], st);
        }
        const uint16_t *vp = pool_v + ((size_t)pg * n_heads + h) * D * 16 + g * 4;
        // keys after the block's last query are not written yet (possibly NaN): clear their values
        const int n_valid = last_pos + 1 - (pi * 16 + g * 4);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          uint2 w = *reinterpret_cast<const uint2 *>(vp + (db * 16 + c) * 16);
          w.x = mask_pair(w.x, 0, n_valid);
          w.y = mask_pair(w.y, 2, n_valid);
          vt[db][u] = w;
        }
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db) vt[db][u] = make_uint2(0, 0);
      }
      // accumulator element e: key 4g+e of page pi, query c
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kpos = pi * 16 + g * 4 + e;
        sc[u][e] = (pg >= 0 && q_ok && kpos <= my_pos) ? st[e] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2f(m - m_new);
    m = m_new;
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pr[u * 4 + e] = exp2f(sc[u][e] - m_new);
        psum += pr[u * 4 + e];
      }
    l = l * alpha + psum;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[i][e] *= alpha;
    // P^T operand: slots 8g+e -> key 4g+e of page pa (e < 4) or of page pa+1 (e >= 4)
    uint4 ps[3];
    split3_pack8(pr, ps[0], ps[1], ps[2]);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint4 va = make_uint4(vt[db][0].x, vt[db][0].y, vt[db][1].x, vt[db][1].y);
      oacc[db] = mfma16(va, ps[2], oacc[db]);
      oacc[db] = mfma16(va, ps[1], oacc[db]);
      oacc[db] = mfma16(va, ps[0], oacc[db]);
    }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (!q_ok) return;
  const float inv = 1.f / l;
  const int tok = t0 + qb * 16 + c;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      store_out(oacc[db][e] * inv, tok, h * D + db * 16 + g * 4 + e, n_heads * D, out_f32, out_hi, out_lo, kpad);
}

void launch_prefill_attention(const llmdec_config &cfg, const float *q, int ld_q, int n_seqs, int n_tokens, int max_q_len,
                              const int32_t *cu, const int32_t *start_pos, const int32_t *block_tables, int max_pages,
                              const uint16_t *pk, const uint16_t *pv, int num_pages, float *out_f32, uint16_t *out_hi, uint16_t *out_lo,
                              int kpad, uint32_t *err, hipStream_t s) {
  if (n_seqs <= 0 || max_q_len <= 0) return;
  dim3 grid((max_q_len + 15) / 16, cfg.n_heads, n_seqs);
  if (cfg.head_dim == 128)
    prefill_attn_kernel<128><<<grid, 64, 0, s>>>(q, ld_q, cfg.n_heads, n_tokens, max_q_len, cu, start_pos, block_tables, max_pages, pk, pv,
                                                 num_pages, out_f32, out_hi, out_lo, kpad, err);
  else
    prefill_attn_kernel<64><<<grid, 64, 0, s>>>(q, ld_q, cfg.n_heads, n_tokens, max_q_len, cu, start_pos, block_tables, max_pages, pk, pv,
                                                num_pages, out_f32, out_hi, out_lo, kpad, err);
}

}  // namespace llmdec
