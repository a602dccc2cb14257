// Weight products: out[m][n] = sum_k a[m][k] * W[n][k] on the matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// The activation enters as a bf16 pair a = hi + lo (hi = bf16(a), lo =
// bf16(a - hi), about 17 significant bits), so every product is two MFMAs,
// hi * W + lo * W.  A single bf16 rounding of the activation would put the
// 7B-layer output outside a 2e-2 max-abs bound against an unrounded
// reference: a chain of four such roundings per layer turns any relative
// difference e into an output difference of order sqrt(512 e) * 2^-9 at each
// stage.  The pair keeps the weight product within fp32-level agreement.
//
// Both operands are in the packed tile layout (see packed_offset): a 16-row x
// 32-column tile is 1 KiB, and lane l of a wave holds row l%16, columns
// 8(l/16)..+7 -- exactly one MFMA operand.  Activations are packed the same
// way by their producers (RMSNorm, attention, the SwiGLU epilogue), so every
// operand fetch is one contiguous 16-byte load per lane.
//
// Two kernels:
//   * stream_gemm (rows <= 64, decode): the weight matrix is read once from
//     HBM and that read bounds the kernel.  A block owns 64 output columns
//     (4 row blocks of W); its 4 waves take interleaved k-tiles of the block's
//     k-range and keep a ring of SG_DEPTH k-tiles of weights in flight (16 KiB
//     per wave).  Wave sums meet in LDS.  Narrow matrices also split k across
//     blocks: each block then stores its fp32 partial sums and the caller adds
//     them (launch_reduce, or the next kernel that reads the result anyway).
//   * tiled_gemm (rows > 64, prefill): 128 x 128 output tile per block, one
//     32-wide k-tile per LDS stage (A hi, A lo, W: 24 tiles, 24 KiB), two
//     stages; 4 waves in 2 x 2, each 64 x 64 = 4 x 4 MFMA blocks.  Tiles are
//     handed to the 8 XCDs in contiguous runs, row tiles innermost, so a
//     weight tile is fetched into one XCD's L2 and reused by every row tile.
//
// Epilogues: store fp32; add into fp32 (the residual stream); SwiGLU, where
// W's row blocks alternate gate / up (block 2j: gate rows 16j.., block 2j+1:
// up rows 16j..) and the kernel writes silu(g) * u straight into the packed
// hi/lo activation of the down projection.
#include "common.h"
#include "internal.h"

namespace llmdec {

__device__ inline f32x4 mfma16(const uint4 &a, const uint4 &b, f32x4 c) {
  bf16x8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

__device__ inline float silu_f(float g) { return g / (1.0f + expf(-g)); }

// One output element through the epilogue.  c is the column of the product;
// for kSiluMul only gate columns call this, with u the matching up value.
__device__ inline void epi_store(const LinearOut &o, int r, int c, float v, float u) {
  if (o.kind == kSiluMul) {
    const int j = ((c >> 5) << 4) | (c & 15);  // gate column -> activation column
    uint16_t h, l;
    split_bf16(silu_f(v) * u, h, l);
    const size_t off = packed_offset(r, j, o.act_kt);
    o.act_hi[off] = h;
    o.act_lo[off] = l;
    // the row's padding columns (act_cols .. 32*act_kt-1, fewer than 16 since act_cols % 16 == 0)
    // follow the last real 16-column block, whose writers clear them
    if (j + 16 >= o.act_cols && j + 16 < o.act_kt * 32) {
      const size_t pad = packed_offset(r, j + 16, o.act_kt);
      o.act_hi[pad] = 0;
      o.act_lo[pad] = 0;
    }
  } else {
    float *p = o.f32 + (size_t)r * o.ld + c;
    *p = o.kind == kAccumulate ? *p + v : v;
  }
}

// ---------------------------------------------------------------- stream_gemm (rows <= 64)
constexpr int SG_NB = 4;     // W row blocks per block: 64 output columns
constexpr int SG_DEPTH = 4;  // k-tiles of weights in flight per wave

// Activation tiles are L2 hits but still a round trip: they ride a ring of
// their own, AD deep (AD divides SG_DEPTH; fewer slots for wide MB keep the
// registers of a wave within one SIMD's share at two waves per SIMD).
template <int MB, int AD = (MB <= 2 ? 4 : 2)>
__global__ __launch_bounds__(256) void stream_gemm_kernel(const uint4 *__restrict__ a_hi,
                                                          const uint4 *__restrict__ a_lo, int a_kt, int rows,
                                                          const uint4 *__restrict__ w, int kt_count, int n_blocks,
                                                          LinearOut o, float *__restrict__ partials) {
  __shared__ float red[3][MB * 16][SG_NB * 16 + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x, split = blockIdx.y, ks = gridDim.y;
  const int nb0 = g * SG_NB;
  const int nbs = min(SG_NB, n_blocks - nb0);
  const int kt0 = (int)((long)kt_count * split / ks), kt1 = (int)((long)kt_count * (split + 1) / ks);
  const int n_it = kt1 - kt0 > wave ? (kt1 - kt0 - wave + 3) >> 2 : 0;  // k-tiles kt0 + wave + 4i

  f32x4 acc[MB][SG_NB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < SG_NB; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint4 *wl = w + (size_t)nb0 * kt_count * 64 + lane;  // row block nb0, tile 0, this lane
  auto a_tile = [&](const uint4 *base, int m, int i) { return base[((size_t)m * a_kt + kt0 + wave + 4 * i) * 64 + lane]; };
  uint4 wb[SG_DEPTH][SG_NB];
  uint4 ahb[AD][MB], alb[AD][MB];
#pragma unroll
  for (int d = 0; d < SG_DEPTH; ++d)
#pragma unroll
    for (int j = 0; j < SG_NB; ++j)
      wb[d][j] = (d < n_it && j < nbs) ? load_stream(wl + ((size_t)j * kt_count + kt0 + wave + 4 * d) * 64)
                                       : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int d = 0; d < AD; ++d)
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      ahb[d][m] = d < n_it ? a_tile(a_hi, m, d) : make_uint4(0, 0, 0, 0);
      alb[d][m] = d < n_it ? a_tile(a_lo, m, d) : make_uint4(0, 0, 0, 0);
    }
  for (int it = 0; it < n_it; it += SG_DEPTH) {
#pragma unroll
    for (int d = 0; d < SG_DEPTH; ++d) {
      const int i = it + d;
      if (i < n_it) {
        const int da = d % AD;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int j = 0; j < SG_NB; ++j) {
            acc[m][j] = mfma16(alb[da][m], wb[d][j], acc[m][j]);
            acc[m][j] = mfma16(ahb[da][m], wb[d][j], acc[m][j]);
          }
        if (i + AD < n_it) {
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            ahb[da][m] = a_tile(a_hi, m, i + AD);
            alb[da][m] = a_tile(a_lo, m, i + AD);
          }
        }
        const int i2 = i + SG_DEPTH;
        if (i2 < n_it) {
          const int kt2 = kt0 + wave + 4 * i2;
#pragma unroll
          for (int j = 0; j < SG_NB; ++j)
            if (j < nbs) wb[d][j] = load_stream(wl + ((size_t)j * kt_count + kt2) * 64);
        }
      }
    }
  }
  // accumulator layout: lane l, element e -> row 4(l/16)+e, column l%16 of each 16 x 16 block
  const int rq = (lane >> 4) * 4, cq = lane & 15;
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int j = 0; j < SG_NB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave - 1][m * 16 + rq + e][j * 16 + cq] = acc[m][j][e];
  }
  __syncthreads();
  if (wave != 0) return;
  const int n = n_blocks * 16;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < SG_NB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = m * 16 + rq + e, c = j * 16 + cq;
        const float v = acc[m][j][e] + red[0][r][c] + red[1][r][c] + red[2][r][c];
        acc[m][j][e] = v;
        if (ks > 1 && r < rows && j < nbs) partials[((size_t)split * rows + r) * n + (nb0 + j) * 16 + cq] = v;
      }
  if (ks > 1) return;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < SG_NB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = m * 16 + rq + e, c = (nb0 + j) * 16 + cq;
        if (r >= rows || j >= nbs) continue;
        if (o.kind == kSiluMul) {
          if ((j & 1) == 0) epi_store(o, r, c, acc[m][j][e], acc[m][j + 1][e]);
        } else {
          epi_store(o, r, c, acc[m][j][e], 0.f);
        }
      }
}

// ---------------------------------------------------------------- split-k reduction
// One thread per (row, 4 consecutive columns): sums the ks partials in split
// order (deterministic) and applies the epilogue.  For SwiGLU the threads of
// gate columns also read the matching up columns (16 further on).
__global__ void reduce_kernel(const float *__restrict__ partials, int ks, int rows, int n, LinearOut o) {
  const int n4 = n >> 2;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)rows * n4) return;
  const int r = (int)(idx / n4), c = (int)(idx % n4) * 4;
  if (o.kind == kSiluMul && ((c >> 4) & 1)) return;
  const size_t plane = (size_t)rows * n;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f), u = s;
  for (int q = 0; q < ks; ++q) {
    const float4 v = *reinterpret_cast<const float4 *>(partials + q * plane + (size_t)r * n + c);
    s.x += v.x, s.y += v.y, s.z += v.z, s.w += v.w;
    if (o.kind == kSiluMul) {
      const float4 w = *reinterpret_cast<const float4 *>(partials + q * plane + (size_t)r * n + c + 16);
      u.x += w.x, u.y += w.y, u.z += w.z, u.w += w.w;
    }
  }
  epi_store(o, r, c, s.x, u.x);
  epi_store(o, r, c + 1, s.y, u.y);
  epi_store(o, r, c + 2, s.z, u.z);
  epi_store(o, r, c + 3, s.w, u.w);
}

void launch_reduce(const float *partials, int ks, int rows, int n, const LinearOut &o, hipStream_t s) {
  const size_t total = (size_t)rows * (n / 4);
  if (total) reduce_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(partials, ks, rows, n, o);
}

// ---------------------------------------------------------------- tiled_gemm (rows > 64)
constexpr int TG_MB = 8;                               // 16-row blocks of A per block (128 rows)
constexpr int TG_NB = 8;                               // 16-row blocks of W per block (128 columns)
constexpr int TG_STAGE_TILES = TG_MB * 2 + TG_NB;      // A hi, A lo, W tiles of one k-tile: 24 KiB
constexpr size_t TG_LDS = (size_t)2 * TG_STAGE_TILES * 1024;

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Global source of tile q (0..23) of k-tile kt, or NULL when it lies outside the operands.
__device__ inline const uint4 *tg_src(int q, int kt, int mb0, int nb0, int a_blocks, int n_blocks, int a_kt,
                                      int kt_count, const uint4 *a_hi, const uint4 *a_lo, const uint4 *w) {
  if (q < TG_MB) {
    const int rb = mb0 + q;
    return rb < a_blocks ? a_hi + ((size_t)rb * a_kt + kt) * 64 : nullptr;
  }
  if (q < 2 * TG_MB) {
    const int rb = mb0 + q - TG_MB;
    return rb < a_blocks ? a_lo + ((size_t)rb * a_kt + kt) * 64 : nullptr;
  }
  const int nb = nb0 + q - 2 * TG_MB;
  return nb < n_blocks ? w + ((size_t)nb * kt_count + kt) * 64 : nullptr;
}

template <bool DIRECT>
__global__ __launch_bounds__(256) void tiled_gemm_kernel(const uint4 *__restrict__ a_hi,
                                                         const uint4 *__restrict__ a_lo, int a_kt, int a_blocks,
                                                         int rows, const uint4 *__restrict__ w, int kt_count,
                                                         int n_blocks, int tiles_m, LinearOut o) {
  extern __shared__ uint4 lds[];  // [2 stages][24 tiles][64 lanes]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // XCD-aware order: block b runs on XCD b % 8; each XCD gets a contiguous run of tiles, row tiles innermost
  const int nblk = gridDim.x;
  int t = blockIdx.x;
  if ((nblk & 7) == 0) t = (t & 7) * (nblk >> 3) + (t >> 3);
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int mb0 = tm * TG_MB, nb0 = tn * TG_NB;
  constexpr int PER_WAVE = TG_STAGE_TILES / 4;  // 6 tiles per wave per stage

  uint4 stage_regs[PER_WAVE];
  auto fetch = [&](int kt) {  // global -> registers (staged variant)
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const uint4 *src = tg_src(wave + 4 * i, kt, mb0, nb0, a_blocks, n_blocks, a_kt, kt_count, a_hi, a_lo, w);
      stage_regs[i] = src ? src[lane] : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {  // registers -> LDS
    uint4 *base = lds + (size_t)buf * TG_STAGE_TILES * 64;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) base[(size_t)(wave + 4 * i) * 64 + lane] = stage_regs[i];
  };
  auto direct = [&](int kt, int buf) {  // global -> LDS without registers
    uint4 *base = lds + (size_t)buf * TG_STAGE_TILES * 64;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave + 4 * i;
      const uint4 *src = tg_src(q, kt, mb0, nb0, a_blocks, n_blocks, a_kt, kt_count, a_hi, a_lo, w);
      if (src)
        __builtin_amdgcn_global_load_lds((const void *)(src + lane), (lds_ptr_t)(base + (size_t)q * 64), 16, 0, 0);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;  // wave owns A row blocks wm*4.. and W row blocks wn*4..
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (DIRECT) {
    direct(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    fetch(0);
    store(0);
  }
  __syncthreads();
  int buf = 0;
  for (int kt = 0; kt < kt_count; ++kt) {
    const bool more = kt + 1 < kt_count;
    if (more) {
      if (DIRECT) direct(kt + 1, buf ^ 1);
      else fetch(kt + 1);
    }
    const uint4 *st = lds + (size_t)buf * TG_STAGE_TILES * 64;
    uint4 ah[4], al[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ah[i] = st[(size_t)(wm * 4 + i) * 64 + lane];
      al[i] = st[(size_t)(TG_MB + wm * 4 + i) * 64 + lane];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = st[(size_t)(2 * TG_MB + wn * 4 + j) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = mfma16(al[i], bv[j], acc[i][j]);
        acc[i][j] = mfma16(ah[i], bv[j], acc[i][j]);
      }
    if (more) {
      if (DIRECT) __builtin_amdgcn_s_waitcnt(0);
      else store(buf ^ 1);
    }
    __syncthreads();
    buf ^= 1;
  }

  const int rq = (lane >> 4) * 4, cq = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nb = nb0 + wn * 4 + j;
      if (nb >= n_blocks) continue;
      if (o.kind == kSiluMul && (j & 1)) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = (mb0 + wm * 4 + i) * 16 + rq + e;
        if (r < rows) epi_store(o, r, nb * 16 + cq, acc[i][j][e], o.kind == kSiluMul ? acc[i][j + 1][e] : 0.f);
      }
    }
}

// ---------------------------------------------------------------- dispatch
// Splits of k across blocks for the streaming kernel: enough blocks to keep
// every CU streaming, while the partial sums (written once and read back
// once) stay at most a quarter of the weight bytes and every wave keeps at
// least four k-tiles to pipeline.
int stream_ksplit(int rows, int n, int k) {
  const int groups = (n / 16 + SG_NB - 1) / SG_NB;
  const int kt = round_up(k, kTileK) / kTileK;
  int ks = 1;
  while (groups * ks < 512 && kt / (ks * 2) >= 16 && (long)(ks * 2) * rows * 16 <= (long)k) ks *= 2;
  return ks;
}

size_t linear_partial_floats(int rows, int n, int k) {
  if (rows > 64) return 0;
  const int ks = stream_ksplit(rows, n, k);
  return ks > 1 ? (size_t)ks * rows * n : 0;
}

#ifndef LLMDEC_TILED_DIRECT
#define LLMDEC_TILED_DIRECT 0
#endif

int launch_linear(const Act &a, const uint16_t *w_packed, int n, int k, const LinearOut &o, float *partials,
                  size_t partial_floats, bool allow_split, hipStream_t s) {
  const int kt_count = round_up(k, kTileK) / kTileK;
  const int n_blocks = n / 16;
  const uint4 *w = reinterpret_cast<const uint4 *>(w_packed);
  const uint4 *ah = reinterpret_cast<const uint4 *>(a.hi), *al = reinterpret_cast<const uint4 *>(a.lo);
  const int a_kt = a.kpad / kTileK;
  if (a.rows <= 64) {
    int ks = allow_split ? stream_ksplit(a.rows, n, k) : 1;
    if (ks > 1 && (!partials || partial_floats < (size_t)ks * a.rows * n)) ks = 1;
    dim3 grid((n_blocks + SG_NB - 1) / SG_NB, ks);
    switch ((a.rows + 15) / 16) {
      case 1: stream_gemm_kernel<1><<<grid, 256, 0, s>>>(ah, al, a_kt, a.rows, w, kt_count, n_blocks, o, partials); break;
      case 2: stream_gemm_kernel<2><<<grid, 256, 0, s>>>(ah, al, a_kt, a.rows, w, kt_count, n_blocks, o, partials); break;
      case 3: stream_gemm_kernel<3><<<grid, 256, 0, s>>>(ah, al, a_kt, a.rows, w, kt_count, n_blocks, o, partials); break;
      default: stream_gemm_kernel<4><<<grid, 256, 0, s>>>(ah, al, a_kt, a.rows, w, kt_count, n_blocks, o, partials); break;
    }
    return ks;
  }
  const int tiles_m = (a.rows + TG_MB * 16 - 1) / (TG_MB * 16);
  const int tiles_n = (n_blocks + TG_NB - 1) / TG_NB;
  tiled_gemm_kernel<LLMDEC_TILED_DIRECT><<<tiles_m * tiles_n, 256, TG_LDS, s>>>(ah, al, a_kt, a.row_blocks, a.rows, w,
                                                                               kt_count, n_blocks, tiles_m, o);
  return 1;
}

}  // namespace llmdec
