// Attention over the paged KV cache ([E] §4.3: softmax(q K^T / sqrt(D)) V with
// the causal mask; [E] §3.4: keys found through the page index).
//
// Pool layout per layer: K[page][h][16][D], V[page][h][4][D][4] (token
// quarter, dim, token within the quarter).
//
// Decode: one wave per (sequence, head, partition of pages), every load a
// contiguous 1 KiB of a K or V block (details at the kernel); the running max
// is wave-uniform per page (one rescale per page).  The eight waves of a block
// merge their partitions in LDS; where a sequence spans several blocks, a
// log-sum-exp combine kernel merges the blocks' results.
//
// Prefill: MFMA.  Scores are formed transposed, S^T = K Q^T (keys as rows),
// so a lane's accumulator holds 4 keys of one query: exactly the operand
// slots the P.V product O^T = V^T P^T needs, with no shuffle through LDS.  q
// and p are split into three bf16 parts each (hi + mid + lo carries fp32's
// 24 bits; three MFMAs per product), K and V are the stored bf16 values, so
// the scores and the weighted sum keep fp32-level accuracy.
#include <math.h>

#include <type_traits>

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

// The attention output feeds the o projection as a packed fp16 activation (with out_lo: the fp16 pair);
// the stand-alone operation also (or only) writes fp32.
__device__ inline void store_out(float v, int r, int c, int ld, float *out_f32, uint16_t *out_act, uint16_t *out_lo,
                                 int kpad) {
  if (out_f32) out_f32[(size_t)r * ld + c] = v;
  if (out_act) {
    const size_t o = packed_offset(r, c, kpad >> 5);
    const uint16_t h = f32_to_f16(v);
    out_act[o] = h;
    if (out_lo) out_lo[o] = f32_to_f16(v - f16_to_f32(h));
  }
}

// ---------------------------------------------------------------- decode
// One wave per (sequence, head, partition of at most 64 pages).  Every load
// instruction reads one contiguous run of a page's K or V block (lane l takes
// bytes 16l..16l+15 of a 1 KiB run): random 4 KiB blocks read this way run at
// about 6.8 TB/s on MI355X, where a lane reading a 64-byte run of its own gets
// about 3.9.
//   K block [16 tokens][D]: instruction i, lane l -> token G*i + l/LPT, dims
//     8(l%LPT)..+7 (LPT = D/8 lanes per token); a score is the sum over the
//     lanes of its group, formed with DPP lane swizzles (no LDS round trips).
//   V block [4 quarters][D][4 tokens]: instruction i reads quarter i, lane l ->
//     dims D/64*l..+D/64-1, its 4 tokens.  Over the four instructions every
//     lane holds all 16 tokens of its dims, so the softmax weights of a page
//     are wave-uniform: they live in scalar registers and feed the FMAs
//     directly.
// q enters the K products (v_dot2_f32_bf16) as a bf16 pair hi + lo (about 17
// bits).  The partition's page ids are read once, one per lane, and picked
// out with a lane shuffle; K/V of the next DA_RING - 1 pages are in flight
// while a page is computed (32 KiB per wave at D = 128).  Partitions are the
// slowest grid dimension,
// so every sequence's full first partitions are dispatched before the short
// last ones, which fill in the tail.
constexpr int DA_RING = 3;
constexpr int DA_WAVES = 8;        // decode waves per block: consecutive partitions of one (sequence, heads)
constexpr int kMaxPartPages = 18;  // pages per decode partition, at most
static_assert(DA_WAVES * kMaxPartPages <= 192, "a block's page ids fit three per lane");

__device__ inline uint32_t vword(const uint4 &v, int k) { return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w; }
__device__ inline uint32_t vword(const uint2 &v, int k) { return k == 0 ? v.x : v.y; }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  bf16x2_t x, y;
  __builtin_memcpy(&x, &a, 4);
  __builtin_memcpy(&y, &b, 4);
  return __builtin_amdgcn_fdot2_f32_bf16(x, y, c, false);
}

// x + (the value of another lane), for the DPP lane patterns used below
template <int CTRL>
__device__ inline float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Sum over aligned groups of N lanes (N = 8 or 16), result in every lane of the group.
template <int N>
__device__ inline float group_sum(float x) {
  x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x = dpp_add<0x141>(x);  // row_half_mirror: the other quad of the 8
  if (N == 16) x = dpp_add<0x140>(x);  // row_mirror: the other 8 of the 16
  return x;
}

__device__ inline float uniform_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

template <int D, int QH, bool SHARED_KV>
__global__ __launch_bounds__(64 * DA_WAVES) void decode_attn_kernel(const float *__restrict__ q, int ld_q, int n_heads,
                                                         int n_kv_heads, const int32_t *__restrict__ ctx_lens,
                                                         const int32_t *__restrict__ block_tables, int max_pages,
                                                         const uint16_t *__restrict__ pool_k,
                                                         const uint16_t *__restrict__ pool_v, int num_pages, int ppp,
                                                         int n_parts, float *__restrict__ partials, float *out_f32,
                                                         uint16_t *out_act, uint16_t *out_lo, int kpad, uint32_t *err) {
  constexpr int NI = D / 32;      // 1 KiB K load instructions per page
  constexpr int LPT = D / 8;      // lanes per token in K (each holds 8 dims)
  constexpr int G = 64 / LPT;     // token groups per K instruction
  constexpr int VE = D / 64;      // V dims per lane
  // Grouped-query attention: query head h reads K/V head h / group.  A wave serves QH consecutive query
  // heads h0..h0+QH-1 of one K/V head (QH = the group, at most 4), so each page it reads feeds QH score
  // and value sums.  Where a group is larger than QH, its waves are launched n_kv_heads blocks apart:
  // blocks go round-robin to the 8 XCDs, so with n_kv_heads a multiple of 8 they share one L2.
  const int group = n_heads / n_kv_heads;
  const int kvh = blockIdx.x % n_kv_heads, h0 = kvh * group + (blockIdx.x / n_kv_heads) * QH;
  const int s = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Block z covers pages [z DA_WAVES ppp, (z + 1) DA_WAVES ppp) of its sequence (ppp pages per wave);
  // a block holding fewer pages (a sequence's last or only block) spreads them evenly over its waves,
  // so it lasts as long as its share, not as long as a full partition.
  const int blk0 = blockIdx.z * DA_WAVES * ppp;
  // Three independent reads leave together: the context length, the block's block-table entries
  // (every wave reads all of them, up to three per lane; each picks its own once the length is known)
  // and q.
  const int32_t *bt = block_tables + (size_t)s * max_pages;
  int ent[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int i = 64 * j + lane;
    ent[j] = (64 * j < DA_WAVES * ppp && i < DA_WAVES * ppp && blk0 + i < max_pages) ? bt[blk0 + i] : -1;
  }
  float4 qv0[QH], qv1[QH];
#pragma unroll
  for (int j = 0; j < QH; ++j) {
    const float *qp = q + (size_t)s * ld_q + (h0 + j) * D + (lane % (D / 8)) * 8;
    qv0[j] = *reinterpret_cast<const float4 *>(qp);
    qv1[j] = *reinterpret_cast<const float4 *>(qp + 4);
  }
  const int n_tok = ctx_lens[s] + 1;
  const int n_pages = (n_tok + 15) >> 4;
  // the returns below are block-uniform (they depend on the sequence and the block only); a wave whose
  // partition lies past the context still takes part in the block's combine with an empty result
  if (n_tok <= 0) {
    if (threadIdx.x == 0 && blockIdx.z == 0) raise_error(err, kErrPos);
    return;
  }
  if (blk0 >= n_pages) return;
  if (n_pages > max_pages) {
    if (threadIdx.x == 0) raise_error(err, kErrPos);
    return;
  }
  const int nb = min(DA_WAVES * ppp, n_pages - blk0);  // the block's pages
  const int per = (nb + DA_WAVES - 1) / DA_WAVES;       // pages per wave (at most ppp)
  const int p0 = blk0 + wave * per;
  const int p1 = max(p0, min(blk0 + nb, p0 + per));
  // lane i's entry: block page wave * per + i, held by lane (that & 63) in ent[that >> 6]
  const int bi = wave * per + lane;
  const int from = (bi & 63) * 4;
  const int e0 = __builtin_amdgcn_ds_bpermute(from, ent[0]), e1 = __builtin_amdgcn_ds_bpermute(from, ent[1]),
            e2 = __builtin_amdgcn_ds_bpermute(from, ent[2]);
  const int raw_pg = bi < 64 ? e0 : (bi < 128 ? e1 : e2);
  int my_pg = -1;  // lane i: page id of page p0 + i
  if (lane < p1 - p0) {
    my_pg = raw_pg;
    if (my_pg < 0 || my_pg >= num_pages) {
      raise_error(err, kErrPage);
      my_pg = -1;
    }
  }
  uint32_t qh[QH][4], ql[QH][4];  // q * log2(e)/sqrt(D), dims 8(lane % LPT)..+7, as bf16 hi/lo pairs
#pragma unroll
  for (int jh = 0; jh < QH; ++jh) {
    const float scale = kLog2e * rsqrtf((float)D);
    const float qv[8] = {qv0[jh].x * scale, qv0[jh].y * scale, qv0[jh].z * scale, qv0[jh].w * scale,
                         qv1[jh].x * scale, qv1[jh].y * scale, qv1[jh].z * scale, qv1[jh].w * scale};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint16_t a0, b0, a1, b1;
      split_bf16(qv[2 * j], a0, b0);
      split_bf16(qv[2 * j + 1], a1, b1);
      qh[jh][j] = a0 | ((uint32_t)a1 << 16);
      ql[jh][j] = b0 | ((uint32_t)b1 << 16);
    }
  }
  float m[QH], l[QH], o[QH][VE];
#pragma unroll
  for (int jh = 0; jh < QH; ++jh) {
    m[jh] = -1e30f;
    l[jh] = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) o[jh][e] = 0.f;
  }

  uint4 kb[DA_RING][NI];
  // V quarter i of a page: VW words (2 bf16 each), kept as one vector so the ring stays in fixed registers
  using VVec = std::conditional_t<VE == 2, uint4, uint2>;
  VVec vb[DA_RING][4];
  auto page_id = [&](int pi) { return __builtin_amdgcn_readlane(my_pg, pi - p0); };  // wave-uniform
  // Each page-head block (16 tokens x D bf16 of K, the same of V) is read through a buffer resource
  // of its own; an absent page (past the partition, or a rejected id) gets an empty resource, whose
  // loads read zeros without touching memory, so the ring below needs no branches.  Without grouping
  // every page is read once per step: the non-temporal policy keeps it from displacing anything in the
  // caches (measured: 12% less time for the same bytes).  A K/V head whose group spans several waves
  // is read by each of them, so there the pages are cached normally for the others to hit.
  constexpr int policy = SHARED_KV ? 0 : kLoadStream;
  const uint32_t lane_bytes = (uint32_t)lane * 16u;
  auto load = [&](int pi, int b) {
    const int pg = page_id(pi);
    const bool ok = pg >= 0;
    const size_t blk = ((size_t)(ok ? pg : 0) * n_kv_heads + kvh) * 16 * D;  // element offset of the block
    const size_t bytes = ok ? (size_t)16 * D * 2 : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(pool_k + blk, bytes), vr = make_rsrc(pool_v + blk, bytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) kb[b][i] = buffer_load16(kr, lane_bytes, i * 1024, policy);
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // token quarter i: D x 4 bf16, lane holds VE dims x 4 tokens
      if constexpr (VE == 2) {
        vb[b][i] = buffer_load16(vr, lane_bytes, i * D * 8, policy);
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(vr, (int)(lane * 8u), i * D * 8, policy);
        vb[b][i] = make_uint2(v[0], v[1]);
      }
    }
  };
  // One page with n_valid (wave-uniform) live tokens: 16, fewer on a sequence's last page, 0 for a
  // rejected page id.
  auto compute = [&](int b, int n_valid) {
    // scores of the QH query heads for the page's 16 tokens (lane = token group, 8 dims)
    float sc[QH][NI], lm[QH];
#pragma unroll
    for (int jh = 0; jh < QH; ++jh) lm[jh] = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t w[4] = {kb[b][i].x, kb[b][i].y, kb[b][i].z, kb[b][i].w};
      const bool valid = G * i + lane / LPT < n_valid;
#pragma unroll
      for (int jh = 0; jh < QH; ++jh) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) a = dot2_bf16(w[j], qh[jh][j], dot2_bf16(w[j], ql[jh][j], a));
        a = group_sum<LPT>(a);
        sc[jh][i] = valid ? a : -INFINITY;
        lm[jh] = fmaxf(lm[jh], sc[jh][i]);
      }
    }
    // per head: page max and weight sum over the G groups (one value per group, read from its first
    // lane), then the 16 weights made wave-uniform: token t's weight sits in group t % G, slot t / G
    float alpha[QH], pt[QH][16];
#pragma unroll
    for (int jh = 0; jh < QH; ++jh) {
      float pm = -INFINITY;
#pragma unroll
      for (int g = 0; g < G; ++g) pm = fmaxf(pm, uniform_f(lm[jh], g * LPT));
      const float m_new = fmaxf(m[jh], pm);
      alpha[jh] = __builtin_amdgcn_exp2f(m[jh] - m_new);
      float pr[NI], ps = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(sc[jh][i] - m_new);  // 0 for masked tokens
        ps += pr[i];
      }
      float gs = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) gs += uniform_f(ps, g * LPT);
      l[jh] = l[jh] * alpha[jh] + gs;
      m[jh] = m_new;
#pragma unroll
      for (int t = 0; t < 16; ++t) pt[jh][t] = uniform_f(pr[t / G], (t % G) * LPT);
    }
    // slots past the last token hold whatever the pool held (possibly NaN): their weight is 0, and
    // 0 * NaN would poison the sum, so their values are cleared through per-token mask words; each
    // V value is unpacked once for all QH heads
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float a[QH];
#pragma unroll
      for (int jh = 0; jh < QH; ++jh) a[jh] = o[jh][e] * alpha[jh];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t m0 = (4 * i < n_valid ? 0xffffu : 0u) | (4 * i + 1 < n_valid ? 0xffff0000u : 0u);
        const uint32_t m1 = (4 * i + 2 < n_valid ? 0xffffu : 0u) | (4 * i + 3 < n_valid ? 0xffff0000u : 0u);
        const uint32_t w0 = vword(vb[b][i], 2 * e) & m0, w1 = vword(vb[b][i], 2 * e + 1) & m1;  // tokens 4i, 4i+1 | 4i+2, 4i+3
        const float v0 = bf16lo(w0), v1 = bf16hi(w0), v2 = bf16lo(w1), v3 = bf16hi(w1);
#pragma unroll
        for (int jh = 0; jh < QH; ++jh) {
          a[jh] = fmaf(pt[jh][4 * i], v0, a[jh]);
          a[jh] = fmaf(pt[jh][4 * i + 1], v1, a[jh]);
          a[jh] = fmaf(pt[jh][4 * i + 2], v2, a[jh]);
          a[jh] = fmaf(pt[jh][4 * i + 3], v3, a[jh]);
        }
      }
#pragma unroll
      for (int jh = 0; jh < QH; ++jh) o[jh][e] = a[jh];
    }
  };
  // Ring of DA_RING pages: DA_RING - 1 in flight while one is consumed.  The page count is padded to
  // a multiple of DA_RING with absent pages (zero loads, no live tokens); scheduling barriers keep the
  // loads in ring order so the compiler's wait counts stay partial.
  auto live = [&](int pi) { return (pi < p1 && page_id(pi) >= 0) ? min(16, n_tok - pi * 16) : 0; };
#pragma unroll
  for (int b = 0; b < DA_RING - 1; ++b) {
    load(p0 + b, b);
    __builtin_amdgcn_sched_barrier(0);
  }
  // A partition holds at most kMaxPartPages pages, so the page loop unrolls completely; leaving it
  // early is a forward branch, and with no back edge the ring never has to be copied between registers.
#pragma unroll
  for (int it = 0; it < (kMaxPartPages + DA_RING - 1) / DA_RING; ++it) {
    const int pi = p0 + it * DA_RING;
    if (pi >= p1) break;
#pragma unroll
    for (int b = 0; b < DA_RING; ++b) {
      load(pi + b + DA_RING - 1, (b + DA_RING - 1) % DA_RING);  // refill the slot freed one page ago
      compute(b, live(pi + b));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // The block's waves hold consecutive partitions: merge their (max, sum, output) in LDS, so only one
  // result per block leaves the CU.  Writes among the page reads cost more than their bytes (a probe
  // of this kernel's read pattern lost 6 % to one 520-byte partial per wave).
  __shared__ float cm[DA_WAVES][QH][2];
  __shared__ float co[DA_WAVES][QH][D];
#pragma unroll
  for (int jh = 0; jh < QH; ++jh) {
    if (lane == 0) {
      cm[wave][jh][0] = m[jh];
      cm[wave][jh][1] = l[jh];
    }
#pragma unroll
    for (int e = 0; e < VE; ++e) co[wave][jh][lane * VE + e] = o[jh][e];
  }
  __syncthreads();
  const int blocks_here = (n_pages + DA_WAVES * ppp - 1) / (DA_WAVES * ppp);  // blocks covering the sequence
  for (int idx = threadIdx.x; idx < QH * D; idx += 64 * DA_WAVES) {
    const int jh = idx / D, d = idx % D, h = h0 + jh;
    float mx = cm[0][jh][0];
#pragma unroll
    for (int w = 1; w < DA_WAVES; ++w) mx = fmaxf(mx, cm[w][jh][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < DA_WAVES; ++w) {  // in partition order
      const float wt = exp2f(cm[w][jh][0] - mx);
      L = fmaf(cm[w][jh][1], wt, L);
      O = fmaf(co[w][jh][d], wt, O);
    }
    if (blocks_here == 1) {
      store_out(O / L, s, h * D + d, n_heads * D, out_f32, out_act, out_lo, kpad);
    } else {
      float *pp = partials + (((size_t)s * n_heads + h) * n_parts + blockIdx.z) * (D + 2);
      if (d == 0) {
        pp[0] = mx;
        pp[1] = L;
      }
      pp[2 + d] = O;
    }
  }
}

// Up to NP partitions of one (sequence, head): every partial is loaded at once (one memory round trip),
// then the same arithmetic as the general path below, in the same order.
template <int D, int NP>
__device__ inline void combine_few(const float *__restrict__ pp, int parts, int s, int h, int n_heads, float *out_f32,
                                   uint16_t *out_act, uint16_t *out_lo, int kpad) {
  const int d = threadIdx.x;
  float m[NP], l[NP], o[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {  // indexes past the last partition repeat it; their terms are skipped
    const float *pj = pp + (size_t)min(j, parts - 1) * (D + 2);
    m[j] = pj[0];
    l[j] = pj[1];
    o[j] = pj[2 + d];
  }
  float mx = m[0];
#pragma unroll
  for (int j = 1; j < NP; ++j) mx = j < parts ? fmaxf(mx, m[j]) : mx;
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int j = 0; j < NP; ++j)
    if (j < parts) {
      const float w = exp2f(m[j] - mx);
      L = fmaf(l[j], w, L);
      acc = fmaf(o[j], w, acc);
    }
  store_out(acc / L, s, h * D + d, n_heads * D, out_f32, out_act, out_lo, kpad);
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(int n_heads, const int32_t *__restrict__ ctx_lens,
                                                           int max_pages, int ppp, int n_parts,
                                                           const float *__restrict__ partials, float *out_f32,
                                                           uint16_t *out_act, uint16_t *out_lo, int kpad) {
  const int s = blockIdx.x / n_heads, h = blockIdx.x % n_heads;
  const int n_pages = (ctx_lens[s] + 1 + 15) >> 4;
  if (n_pages > max_pages || n_pages <= 0) return;
  const int parts = (n_pages + ppp - 1) / ppp;
  if (parts <= 1) return;
  const float *pp = partials + ((size_t)s * n_heads + h) * n_parts * (D + 2);
  if (parts <= 4) return combine_few<D, 4>(pp, parts, s, h, n_heads, out_f32, out_act, out_lo, kpad);
  if (parts <= 16) return combine_few<D, 16>(pp, parts, s, h, n_heads, out_f32, out_act, out_lo, kpad);
  const int d = threadIdx.x;
  // maximum of the partitions' running maxima: one partition per thread, then a block reduction
  __shared__ float red[D / 64], wl[2][D];
  float mx = -1e30f;
  for (int i = d; i < parts; i += D) mx = fmaxf(mx, pp[(size_t)i * (D + 2)]);
  mx = wave_max(mx);
  if ((d & 63) == 0) red[d >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < D / 64; ++w) mx = fmaxf(mx, red[w]);
  // partitions in chunks of D: each thread forms one partition's weight, then every thread adds the
  // chunk's contributions to its dimension in partition order (loads batched 8 at a time)
  float L = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < parts; c0 += D) {
    const int nc = min(D, parts - c0);
    __syncthreads();  // the previous chunk's weights are no longer read
    if (d < nc) {
      const float *pi = pp + (size_t)(c0 + d) * (D + 2);
      const float w = exp2f(pi[0] - mx);
      wl[0][d] = w;
      wl[1][d] = pi[1];
    }
    __syncthreads();
    for (int i = 0; i < nc; i += 8) {
      float ov[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (i + j < nc) ov[j] = pp[(size_t)(c0 + i + j) * (D + 2) + 2 + d];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (i + j < nc) {
          const float w = wl[0][i + j];
          L = fmaf(wl[1][i + j], w, L);
          acc = fmaf(ov[j], w, acc);
        }
    }
  }
  store_out(acc / L, s, h * D + d, n_heads * D, out_f32, out_act, out_lo, kpad);
}

void decode_partition(const llmdec_config &cfg, int n_seqs, int max_pages, int *pages_per_part, int *n_parts) {
  // Aim for ~16 waves per CU over 256 CUs counting every (sequence, wave of heads) row at full width,
  // QH times that where a wave serves QH query heads (its pages cost QH times the arithmetic, so shorter
  // partitions keep the waves' lengths even); never split finer than one page.  Where that asks for
  // partitions longer than kMaxPartPages, a sequence takes as few blocks as hold its pages at up to
  // kMaxPartPages a wave, the pages spread evenly over the blocks' waves: at 2049 tokens (129 pages) one
  // block of eight 17-page partitions instead of two blocks of 16-page ones, so no combine launch follows.
  const int qh = decode_heads_per_wave(cfg);
  const long rows = (long)n_seqs * (cfg.n_heads / qh);
  const long target = 4096L * qh;
  int parts = (int)((target + rows - 1) / rows);
  parts = parts < 1 ? 1 : parts;
  int ppp = (max_pages + parts - 1) / parts;
  ppp = ppp < 1 ? 1 : ppp;
  if (ppp > kMaxPartPages) {
    const int blocks = (max_pages + DA_WAVES * kMaxPartPages - 1) / (DA_WAVES * kMaxPartPages);
    ppp = (max_pages + blocks * DA_WAVES - 1) / (blocks * DA_WAVES);
  }
  *pages_per_part = ppp;
  *n_parts = (max_pages + ppp - 1) / ppp;
}

int decode_blocks_per_seq(int n_parts) { return (n_parts + DA_WAVES - 1) / DA_WAVES; }

int decode_heads_per_wave(const llmdec_config &cfg) {
  const int g = cfg.n_heads / cfg.n_kv_heads;
  return g % 4 == 0 ? 4 : (g % 2 == 0 ? 2 : 1);
}

template <int D, int QH>
static void launch_decode_qh(const llmdec_config &cfg, dim3 grid, hipStream_t s, const float *q, int ld_q,
                             const int32_t *ctx_lens, const int32_t *block_tables, int max_pages, const uint16_t *pk,
                             const uint16_t *pv, int num_pages, int ppp, int n_parts, float *partials, float *out_f32,
                             uint16_t *out_act, uint16_t *out_lo, int kpad, uint32_t *err) {
  if (cfg.n_heads / cfg.n_kv_heads > QH)  // a K/V head read by several waves
    decode_attn_kernel<D, QH, true><<<grid, 64 * DA_WAVES, 0, s>>>(q, ld_q, cfg.n_heads, cfg.n_kv_heads, ctx_lens, block_tables,
                                                        max_pages, pk, pv, num_pages, ppp, n_parts, partials, out_f32,
                                                        out_act, out_lo, kpad, err);
  else
    decode_attn_kernel<D, QH, false><<<grid, 64 * DA_WAVES, 0, s>>>(q, ld_q, cfg.n_heads, cfg.n_kv_heads, ctx_lens, block_tables,
                                                         max_pages, pk, pv, num_pages, ppp, n_parts, partials, out_f32,
                                                         out_act, out_lo, kpad, err);
}

template <int D>
static void launch_decode_d(const llmdec_config &cfg, int qh, dim3 grid, hipStream_t s, const float *q, int ld_q,
                            const int32_t *ctx_lens, const int32_t *block_tables, int max_pages, const uint16_t *pk,
                            const uint16_t *pv, int num_pages, int ppp, int n_parts, float *partials, float *out_f32,
                            uint16_t *out_act, uint16_t *out_lo, int kpad, uint32_t *err) {
  if (qh == 4)
    launch_decode_qh<D, 4>(cfg, grid, s, q, ld_q, ctx_lens, block_tables, max_pages, pk, pv, num_pages, ppp, n_parts,
                           partials, out_f32, out_act, out_lo, kpad, err);
  else if (qh == 2)
    launch_decode_qh<D, 2>(cfg, grid, s, q, ld_q, ctx_lens, block_tables, max_pages, pk, pv, num_pages, ppp, n_parts,
                           partials, out_f32, out_act, out_lo, kpad, err);
  else
    launch_decode_qh<D, 1>(cfg, grid, s, q, ld_q, ctx_lens, block_tables, max_pages, pk, pv, num_pages, ppp, n_parts,
                           partials, out_f32, out_act, out_lo, kpad, err);
  const int n_seqs = (int)grid.y;
  if (n_parts > 1)  // here: partial results per (sequence, head), one per block of DA_WAVES partitions
    decode_combine_kernel<D><<<n_seqs * cfg.n_heads, D, 0, s>>>(cfg.n_heads, ctx_lens, max_pages, ppp * DA_WAVES,
                                                                n_parts, partials, out_f32, out_act, out_lo, kpad);
}

void launch_decode_attention(const llmdec_config &cfg, const float *q, int ld_q, int n_seqs, const int32_t *ctx_lens,
                             const int32_t *block_tables, int max_pages, const uint16_t *pk, const uint16_t *pv,
                             int num_pages, float *partials, float *out_f32, uint16_t *out_act, uint16_t *out_lo,
                             int kpad, uint32_t *err, hipStream_t s) {
  if (n_seqs <= 0) return;
  const int qh = decode_heads_per_wave(cfg);
  int ppp, n_parts;
  decode_partition(cfg, n_seqs, max_pages, &ppp, &n_parts);
  const int n_blocks_z = decode_blocks_per_seq(n_parts);  // partial results per (sequence, head)
  dim3 grid(cfg.n_heads / qh, n_seqs, n_blocks_z);
  if (cfg.head_dim == 128)
    launch_decode_d<128>(cfg, qh, grid, s, q, ld_q, ctx_lens, block_tables, max_pages, pk, pv, num_pages, ppp,
                         n_blocks_z, partials, out_f32, out_act, out_lo, kpad, err);
  else
    launch_decode_d<64>(cfg, qh, grid, s, q, ld_q, ctx_lens, block_tables, max_pages, pk, pv, num_pages, ppp,
                        n_blocks_z, partials, out_f32, out_act, out_lo, kpad, err);
}

// ---------------------------------------------------------------- prefill (causal, MFMA)
// One wave per (sequence, head, block of 16 new tokens).  Keys are taken two
// pages (32 keys) at a time: S^T blocks for both pages, mask, online softmax
// per query, then O^T += V^T P^T over the 32 keys.
template <int D>
__global__ __launch_bounds__(64) void prefill_attn_kernel(const float *__restrict__ q, int ld_q, int n_heads, int n_kv_heads,
                                                          int n_tokens, int max_q_len,
                                                          const int32_t *__restrict__ cu,
                                                          const int32_t *__restrict__ start_pos,
                                                          const int32_t *__restrict__ block_tables, int max_pages,
                                                          const uint16_t *__restrict__ pool_k,
                                                          const uint16_t *__restrict__ pool_v, int num_pages,
                                                          float *out_f32, uint16_t *out_act, uint16_t *out_lo, int kpad,
                                                          uint32_t *err) {
  constexpr int KT = D / 32;  // k-tiles of the head dimension
  constexpr int DB = D / 16;  // 16-dim blocks of the output
  // the query block is the slowest index, counted down: the blocks with the most keys start first
  const int qb = (int)gridDim.z - 1 - (int)blockIdx.z, h = blockIdx.x, s = blockIdx.y;
  const int kvh = h / (n_heads / n_kv_heads);  // the K/V head this query head reads
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
        const uint4 *kp = reinterpret_cast<const uint4 *>(pool_k + (((size_t)pg * n_kv_heads + kvh) * 16 + c) * D + g * 8);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const uint4 kk = kp[kt * 4];  // dims 32kt + 8g .. +7 of key c
          st = mfma16(kk, qs[2][kt], st);  // smallest parts first
          st = mfma16(kk, qs[1][kt], st);
          st = mfma16(kk, qs[0][kt], st);
        }
        // V block [4 quarters][D][4 tokens]: tokens 4g..4g+3 of dim d at (g * D + d) * 4
        const uint16_t *vp = pool_v + ((size_t)pg * n_kv_heads + kvh) * D * 16 + (size_t)g * D * 4;
        // keys after the block's last query are not written yet (possibly NaN): clear their values
        const int n_valid = last_pos + 1 - (pi * 16 + g * 4);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          uint2 w = *reinterpret_cast<const uint2 *>(vp + (db * 16 + c) * 4);
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
      store_out(oacc[db][e] * inv, tok, h * D + db * 16 + g * 4 + e, n_heads * D, out_f32, out_act, out_lo, kpad);
}

// Maximum and sum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (in an MFMA accumulator: the four key groups of
// one query column), with gfx950's row swaps (no trip through the LDS crossbar).  A swap returns the
// operand with rows exchanged in both orders, so op(r[0], r[1]) pairs every lane with its partner; the
// sums associate as (x_l + x_l^16) + (x_l^32 + x_l^48) in every lane, so all four get the same bits.
__device__ inline float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Head dimension 128: four waves per block, one block per (sequence, head, 64 queries); wave w takes the
// 16 queries of block 4 x + w.  The block walks the keys its last query sees two pages (32 keys) at a
// time; each chunk's K and V pages go from the pool straight into LDS (16 loads of 1 KiB, four per
// wave), through three stages, and every wave reads its operands from there, so a page is fetched once
// per 64 queries instead of once per 16.  Step: wait for the chunk's loads, barrier, issue the loads of
// the chunk two ahead (into the stage the previous step read), then the same scores / online softmax /
// P.V arithmetic as the one-wave kernel; a wave past its own last key only takes part in the loads and
// barriers.  Every load lands on a 1 KiB boundary of LDS and writes its 1 KiB in lane order, so the
// bank-conflict-free layouts come from the choice of source bytes per lane: K rows hold their 16-byte
// units XOR-swizzled by the row (the 16 keys a wave's lanes read at one column land in 16 different bank
// groups), and odd V quarters hold theirs with bit 3 of the unit index flipped (a 128-byte shift, so the
// two quarters one half-wave reads use different banks).
constexpr int kPfKPage = 16 * 128 * 2;         // one page of one K head: 16 keys x 128 dims, bf16
constexpr int kPfVQuarter = 4 * 128 * 2;       // one quarter of a V page: 128 dims x 4 keys
constexpr int kPfVPage = 4 * kPfVQuarter;
constexpr int kPfStage = 2 * kPfKPage + 2 * kPfVPage;
constexpr int kPfStages = 3;

// Three blocks per CU (one wave per SIMD each, 48 KiB of LDS each): at most 168 registers a lane.
__global__ __launch_bounds__(256, 3) void prefill_attn4_kernel(const float *__restrict__ q, int ld_q, int n_heads,
                                                            int n_kv_heads, int n_tokens, int max_q_len,
                                                            const int32_t *__restrict__ cu,
                                                            const int32_t *__restrict__ start_pos,
                                                            const int32_t *__restrict__ block_tables, int max_pages,
                                                            const uint16_t *__restrict__ pool_k,
                                                            const uint16_t *__restrict__ pool_v, int num_pages,
                                                            float *out_f32, uint16_t *out_act, uint16_t *out_lo,
                                                            int kpad, uint32_t *err) {
  constexpr int D = 128, KT = D / 32, DB = D / 16;
  __shared__ uint4 lds[kPfStages * kPfStage / 16];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4 *)lds;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  // Blocks start roughly in index order and the query group is the slowest index, counted down: every
  // (head, sequence)'s group with the most keys starts first, and the short ones fill in at the end.
  const int qg = (int)gridDim.z - 1 - (int)blockIdx.z, h = blockIdx.x, s = blockIdx.y;
  const int kvh = h / (n_heads / n_kv_heads);
  const int t0 = cu[s], len = cu[s + 1] - t0;
  if (t0 < 0 || len < 0 || len > max_q_len || t0 + len > n_tokens || start_pos[s] < 0) {
    if (threadIdx.x == 0 && qg == 0 && h == 0) raise_error(err, kErrSeq);
    return;
  }
  if (qg * 64 >= len) return;  // block-uniform
  const int qb = qg * 4 + wave;
  const int n_q = max(0, min(16, len - qb * 16));
  const int pos0 = start_pos[s] + qb * 16, my_pos = pos0 + c;
  const bool q_ok = c < n_q;
  const float scale = kLog2e * rsqrtf((float)D);
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
  const int blk_last = start_pos[s] + min(len, qg * 64 + 64) - 1;  // the block's last query position
  const int n_kpages = (blk_last >> 4) + 1;
  if (n_kpages > max_pages) {
    if (threadIdx.x == 0) raise_error(err, kErrPos);
    return;
  }
  const int last_pos = pos0 + n_q - 1;  // this wave's (below pos0 when it has no queries)
  const int32_t *bt = block_tables + (size_t)s * max_pages;
  const int n_chunks = (n_kpages + 1) / 2;

  // page pi of the sequence, or -1 (past the block's keys, or a bad entry: its loads read zeros)
  auto page_of = [&](int pi) -> int {
    if (pi >= n_kpages) return -1;
    const int pg = bt[pi];
    return pg >= 0 && pg < num_pages ? pg : -1;
  };
  // wave w loads page u = w / 2 of the chunk: its K (w even) or V (w odd) block, 4 x 1 KiB
  const int u_ld = wave >> 1;
  const bool ld_v = wave & 1;
  auto issue = [&](int st, int ch) {
    const int pg = page_of(2 * ch + u_ld);
    const size_t blk = ((size_t)(pg < 0 ? 0 : pg) * n_kv_heads + kvh) * (16 * D);
    const u32x4 d = buffer_desc((ld_v ? pool_v : pool_k) + blk, pg < 0 ? 0u : (uint32_t)kPfKPage);
    const uint32_t stage = lds_base + (uint32_t)(st * kPfStage);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (ld_v) {  // quarter j: LDS unit l holds the quarter's unit l ^ (8 (j % 2))
        load_to_lds16((uint32_t)(j * 1024 + ((lane ^ ((j & 1) * 8)) * 16)), d, 0u,
                      stage + 2 * kPfKPage + u_ld * kPfVPage + j * 1024);
      } else {  // rows 4j..4j+3; LDS unit l % 16 of row r holds the row's unit (l % 16) ^ (r % 16)
        const int r = 4 * j + (lane >> 4), unit = (lane & 15) ^ (r & 15);
        load_to_lds16((uint32_t)(r * 256 + unit * 16), d, 0u, stage + u_ld * kPfKPage + j * 1024);
      }
    }
  };

  f32x4 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -1e30f, l = 0.f;
  if (threadIdx.x == 0)
    for (int pi = 0; pi < n_kpages; ++pi)
      if (bt[pi] < 0 || bt[pi] >= num_pages) raise_error(err, kErrPage);

  issue(0, 0);
  issue(1, 1);
  for (int ch = 0; ch < n_chunks; ++ch) {
    const int st = ch % kPfStages;
    wait_loads_barrier<4>();  // this wave's loads of chunk ch have landed (chunk ch + 1's may be in flight)
    issue((ch + 2) % kPfStages, ch + 2);
    if (ch * 32 > last_pos) continue;  // wave-uniform: no key of this chunk is visible to this wave
    const char *stg = reinterpret_cast<const char *>(lds) + st * kPfStage;
    int pgs[2];
    float sc[2][4];
    uint2 vt[DB][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pi = 2 * ch + u;
      const int pg = page_of(pi);
      pgs[u] = pg;
      // one accumulator per 32 dims (independent MFMA chains), added up afterwards
      f32x4 sk[KT];
      const char *kp = stg + u * kPfKPage + c * 256;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const uint4 kk = *reinterpret_cast<const uint4 *>(kp + (((kt * 4 + g) ^ c) * 16));
        sk[kt] = mfma16(kk, qs[2][kt], f32x4{0.f, 0.f, 0.f, 0.f});  // smallest parts first
        sk[kt] = mfma16(kk, qs[1][kt], sk[kt]);
        sk[kt] = mfma16(kk, qs[0][kt], sk[kt]);
      }
      f32x4 sacc;
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[e] = (sk[0][e] + sk[1][e]) + (sk[2][e] + sk[3][e]);
      // V quarter g (keys 4g..4g+3 of the page), dim db * 16 + c; keys after this wave's last query are
      // not written yet (possibly NaN): clear them
      const char *vp = stg + 2 * kPfKPage + u * kPfVPage + g * 1024;
      const bool tail = pi * 16 + 15 > last_pos;  // wave-uniform: the page holds keys past this wave's queries
      const int n_valid = last_pos + 1 - (pi * 16 + g * 4);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int unit = ((db * 16 + c) >> 1) ^ ((g & 1) * 8);  // 8 bytes: half c % 2 of a 16-byte unit
        uint2 w = *reinterpret_cast<const uint2 *>(vp + unit * 16 + (c & 1) * 8);
        if (tail) {
          w.x = mask_pair(w.x, 0, n_valid);
          w.y = mask_pair(w.y, 2, n_valid);
        }
        vt[db][u] = w;
      }
      if (pg >= 0 && pi * 16 + 15 <= pos0) {  // every key of the page is visible to every query of the wave
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[u][e] = sacc[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kpos = pi * 16 + g * 4 + e;
          sc[u][e] = (pg >= 0 && q_ok && kpos <= my_pos) ? sacc[e] : -INFINITY;
        }
      }
    }
    (void)pgs;
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = rows4_max(mx);
    const float m_new = fmaxf(m, mx);
    // the accumulators are rescaled only when some query's maximum grew (otherwise the factor is 1)
    const bool grow = __any(m_new > m);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pr[u * 4 + e] = __builtin_amdgcn_exp2f(sc[u][e] - m_new);  // 0 for masked keys
        psum += pr[u * 4 + e];
      }
    if (grow) {
      l = l * alpha + psum;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[i][e] *= alpha;
    } else {
      l += psum;
    }
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
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // the loads issued past the last chunk land before exit
  l = rows4_sum(l);
  if (!q_ok) return;
  const float inv = 1.f / l;
  const int tok = t0 + qb * 16 + c;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      store_out(oacc[db][e] * inv, tok, h * D + db * 16 + g * 4 + e, n_heads * D, out_f32, out_act, out_lo, kpad);
}

void launch_prefill_attention(const llmdec_config &cfg, const float *q, int ld_q, int n_seqs, int n_tokens, int max_q_len,
                              const int32_t *cu, const int32_t *start_pos, const int32_t *block_tables, int max_pages,
                              const uint16_t *pk, const uint16_t *pv, int num_pages, float *out_f32, uint16_t *out_act,
                              uint16_t *out_lo, int kpad, uint32_t *err, hipStream_t s) {
  if (n_seqs <= 0 || max_q_len <= 0) return;
  if (cfg.head_dim == 128) {
    dim3 grid4(cfg.n_heads, n_seqs, (max_q_len + 63) / 64);
    prefill_attn4_kernel<<<grid4, 256, 0, s>>>(q, ld_q, cfg.n_heads, cfg.n_kv_heads, n_tokens, max_q_len, cu, start_pos,
                                               block_tables, max_pages, pk, pv, num_pages, out_f32, out_act, out_lo,
                                               kpad, err);
    return;
  }
  dim3 grid(cfg.n_heads, n_seqs, (max_q_len + 15) / 16);
  prefill_attn_kernel<64><<<grid, 64, 0, s>>>(q, ld_q, cfg.n_heads, cfg.n_kv_heads, n_tokens, max_q_len, cu, start_pos,
                                              block_tables, max_pages, pk, pv, num_pages, out_f32, out_act, out_lo,
                                              kpad, err);
}

}  // namespace llmdec
