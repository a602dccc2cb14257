// Device bodies shared by stand-alone kernels and the fused decode programs: one row of RMSNorm and one
// item of RoPE + paged K/V append.  The comments at their kernels (kernels_misc.hip) describe them.
#pragma once

#include "common.h"
#include "internal.h"

namespace llmdec {

// One row of RMSNorm by a block of NT threads (see rmsnorm_kernel); red: NT / 64 floats of LDS.  The
// caller synchronises the block before red is used again.
template <int NT, int RUNS>
__device__ __forceinline__ void norm_row(int r, float *red, float *__restrict__ x, int ld_x,
                                         const int32_t *__restrict__ cu_last, int n_src_rows,
                                         const uint16_t *__restrict__ gamma, int n, float eps, uint32_t *err,
                                         float *out_f32, uint16_t *out_act, uint16_t *out_lo, int kpad,
                                         const float *__restrict__ add, const Splits &sp, int rows) {
  int src_row = cu_last ? cu_last[r + 1] - 1 : r;
  // a bad cu_seqlens entry, or a sequence without new tokens (it has no last row): flag it, read row 0
  if (src_row < 0 || src_row >= n_src_rows || (cu_last && cu_last[r + 1] <= cu_last[r])) {
    if (threadIdx.x == 0) raise_error(err, kErrSeq);
    src_row = 0;
  }
  float *xr = x + (size_t)src_row * ld_x;
  float xv[RUNS][8];
  float ss = 0.f;
#pragma unroll
  for (int it = 0; it < RUNS; ++it) {
    const int c0 = threadIdx.x * 8 + it * NT * 8;
    if (c0 < n) {
      const float4 v0 = *reinterpret_cast<const float4 *>(xr + c0);
      const float4 v1 = *reinterpret_cast<const float4 *>(xr + c0 + 4);
      float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      if (add) {
        float4 a[2] = {make_float4(v[0], v[1], v[2], v[3]), make_float4(v[4], v[5], v[6], v[7])};
        const int ks = sp.slots(c0);  // c0..c0+7 lie in one column group
        const float *src[2] = {add + (size_t)r * n + c0, add + (size_t)r * n + c0 + 4};
        const int kss[2] = {ks, ks};
        add_splits_n<2>(a, src, (size_t)rows * n, kss);
        v[0] = a[0].x, v[1] = a[0].y, v[2] = a[0].z, v[3] = a[0].w;
        v[4] = a[1].x, v[5] = a[1].y, v[6] = a[1].z, v[7] = a[1].w;
        *reinterpret_cast<float4 *>(xr + c0) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(xr + c0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xv[it][j] = v[j];
        ss = fmaf(v[j], v[j], ss);
      }
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) total += red[w];
  const float inv = 1.0f / sqrtf(total / (float)n + eps);
  const int kt = kpad >> 5;
#pragma unroll
  for (int it = 0; it < RUNS; ++it) {
    const int c0 = threadIdx.x * 8 + it * NT * 8;
    if (c0 >= (out_act ? kpad : n)) continue;
    float y[8];
    if (c0 < n) {
      const uint4 gw = *reinterpret_cast<const uint4 *>(gamma + c0);
      const uint32_t gg[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[2 * j] = xv[it][2 * j] * inv * bf16lo(gg[j]);
        y[2 * j + 1] = xv[it][2 * j + 1] * inv * bf16hi(gg[j]);
      }
      if (out_f32) {
        float *o = out_f32 + (size_t)r * n + c0;
        *reinterpret_cast<float4 *>(o) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4 *>(o + 4) = make_float4(y[4], y[5], y[6], y[7]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = 0.f;
    }
    if (out_act) {
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
}

// One (token t, chunk of 256 rotation pairs) item of RoPE + paged append by a block of 256 threads (see
// rope_append_kernel); cs, sn: 64 floats of LDS each.  The caller synchronises the block before they are
// used again.
__device__ __forceinline__ void rope_item(int t, int chunk, float *cs, float *sn, float *__restrict__ qkv,
                                          const float *__restrict__ part, const Splits &sp, int ld_qkv,
                                          int n_tokens, int n_heads, int n_kv_heads, int head_dim,
                                          const RopeFreq &fr, int n_seqs, const int32_t *__restrict__ tok_seq,
                                          const int32_t *__restrict__ tok_pos,
                                          const int32_t *__restrict__ block_tables, int max_pages,
                                          uint16_t *__restrict__ pool_k, uint16_t *__restrict__ pool_v,
                                          int num_pages, uint32_t *err) {
  const int half = head_dim / 2;
  const int hidden = n_heads * head_dim, kv = n_kv_heads * head_dim;
  const int g0 = chunk * 256;  // first (head, pair) index of this item's chunk
  const int seq = tok_seq ? tok_seq[t] : t;
  const int pos = tok_pos[t];
  if ((int)threadIdx.x < half) {
    const int i = threadIdx.x;
    rope_cos_sin(pos, fr.inv_freq[i], cs[i], sn[i]);
  }
  __syncthreads();
  int page = -1;
  const int blk = pos >> 4, off = pos & 15;
  if (seq < 0 || seq >= n_seqs) {
    if (threadIdx.x == 0) raise_error(err, kErrSeq);
  } else if (pos < 0 || blk >= max_pages) {
    if (threadIdx.x == 0) raise_error(err, kErrPos);
  } else {
    page = block_tables[(size_t)seq * max_pages + blk];
    if (page < 0 || page >= num_pages) {
      if (threadIdx.x == 0) raise_error(err, kErrPage);
      page = -1;
    }
  }
  float *q = qkv + (size_t)t * ld_qkv;
  // the token's q|k|v row: from qkv, or the sum of the split-k partial products
  auto row2 = [&](int col) -> float2 {
    if (!part) return *reinterpret_cast<const float2 *>(q + col);
    float2 acc = make_float2(0.f, 0.f);
    add_splits(acc, part + (size_t)t * ld_qkv + col, (size_t)n_tokens * ld_qkv, sp.slots(col));
    return acc;
  };
  for (int g = g0 + threadIdx.x; g < min(n_heads * half, g0 + 256); g += 256) {
    const int h = g / half, i = g % half;
    const float c = cs[i], s = sn[i];
    const int d = h * head_dim + 2 * i;
    const float2 qq = row2(d);
    *reinterpret_cast<float2 *>(q + d) = make_float2(qq.x * c - qq.y * s, qq.x * s + qq.y * c);
    if (page >= 0 && h < n_kv_heads) {  // K/V head h (its columns follow the query heads')
      const float2 kk = row2(hidden + d);
      const uint32_t kb = f32_to_bf16(kk.x * c - kk.y * s) | ((uint32_t)f32_to_bf16(kk.x * s + kk.y * c) << 16);
      const size_t kbase = (((size_t)page * n_kv_heads + h) * 16 + off) * head_dim + 2 * i;
      *reinterpret_cast<uint32_t *>(pool_k + kbase) = kb;
      const float2 vv = row2(hidden + kv + d);
      // V block [4 quarters][D][4 tokens]: dim d of token off at ((off/4) * D + d) * 4 + off % 4
      const size_t vbase = (((size_t)page * n_kv_heads + h) * 4 + (off >> 2)) * head_dim * 4 + (size_t)(2 * i) * 4 + (off & 3);
      pool_v[vbase] = f32_to_bf16(vv.x);
      pool_v[vbase + 4] = f32_to_bf16(vv.y);
    }
  }
}

}  // namespace llmdec
