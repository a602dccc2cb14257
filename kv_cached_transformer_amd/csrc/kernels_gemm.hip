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
//     k-range and keep a ring of 3 to 8 k-steps (weights and activations) in
//     flight, 12 to 32 KiB of weights per wave.  Wave sums meet in LDS.  Narrow matrices also split k across
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
// A block is 4 waves: WN column waves, each owning SG_NB row blocks of W (64
// output columns), times WK = 4 / WN k-waves that take interleaved k-tiles, so
// one step of the block covers WK k-tiles.  A k-tile's 2*MB activation tiles
// (hi and lo of every row block) are needed by all WN column waves of its
// k-wave: with WN > 1 those waves fetch a share each and pass them on through
// LDS, which divides the activation requests per weight byte by WN.  (The
// activation tiles are L2 hits, but vector loads retire in issue order, so
// each one holds a request slot for as long as the weight loads ahead of it.)
// k-wave sums meet in LDS at the end; k-splits across blocks store fp32
// partials that the consumer adds.
constexpr int SG_NB = 4;

template <int MB, int WN> struct SgShape {
  static constexpr int WK = 4 / WN;
  static constexpr int NA = 2 * MB;                             // activation tiles per k-tile
  static constexpr int APW = WN > 1 ? (NA + WN - 1) / WN : NA;  // of them fetched by one wave
  // k-steps in flight per wave: as deep as about 230 registers allow (two waves per SIMD),
  // counting the ring, the activation operands read back from LDS and the accumulators
  static constexpr int RAW = (230 - (WN > 1 ? 8 * MB : 0) - 16 * MB) / (4 * (SG_NB + APW)) - 2;
  static constexpr int D = RAW < 2 ? 2 : (RAW > 8 ? 8 : RAW);
  static constexpr int R = D + 1;  // ring slots: D in flight + the one being computed
  static constexpr int NSLOT = APW * WN;  // staged tiles per k-tile: slots past NA hold unread copies
  static constexpr int STAGE_U4 = WN > 1 ? 2 * WK * NSLOT * 64 : 0;               // two stages of tiles
  static constexpr int RED_F = WK > 1 ? (WK - 1) * MB * 16 * (WN * 64 + 1) : 0;  // k-wave sums
  static constexpr int LDS_U4 = STAGE_U4 > (RED_F + 3) / 4 ? STAGE_U4 : ((RED_F + 3) / 4 > 0 ? (RED_F + 3) / 4 : 1);
};

// The steady-state loop issues only unconditional loads (row blocks past the
// matrix and k-tiles past the range are clamped to the last one and their
// products skipped or dropped), and scheduling barriers keep the ring order,
// so the compiler's wait counts follow the ring instead of draining it.
//
// Work is split stream-K (see Splits): block b walks its share of the
// (column group, k-tile) units group by group; each group segment runs the
// ring over its k-tiles and leaves either the finished result (no split) or
// one plane of partial sums.
template <int MB, int WN>
__global__ __launch_bounds__(256, 2) void stream_gemm_kernel(const uint4 *__restrict__ a_hi,
                                                             const uint4 *__restrict__ a_lo, int a_kt, int rows,
                                                             const uint4 *__restrict__ w, int kt_count, int n_blocks,
                                                             LinearOut o, float *__restrict__ partials, Splits sp) {
  using S = SgShape<MB, WN>;
  constexpr int WK = S::WK, NA = S::NA, APW = S::APW, D = S::D, R = S::R;
  constexpr bool SHARE = WN > 1;
  __shared__ uint4 lds[S::LDS_U4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar control
  const int cw = wave % WN, kw = wave / WN;
  const int n = n_blocks * 16;
  const int rq = (lane >> 4) * 4, cq = lane & 15;  // accumulator: lane l, element e -> row 4(l/16)+e, column l%16

  // Scalar resources and offsets; the lane adds its own 16 bytes of a 1 KiB tile.  Each resource spans
  // only what the wave reads (its own row blocks; the MB row blocks of the activations), far below 2^31
  // bytes, so the out-of-range marker below is always past its end.
  const uint32_t lane_bytes = (uint32_t)lane * 16u;
  const size_t a_bytes = (size_t)MB * a_kt * 1024;
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(a_hi, a_bytes), lr = make_rsrc(a_lo, a_bytes);
  // activation tiles this wave fetches: q = cw + WN*s (hi row block q, or lo row block q - MB)
  __amdgpu_buffer_rsrc_t ar[APW];
  uint32_t a_off[APW];
#pragma unroll
  for (int s = 0; s < APW; ++s) {
    const int q = min(SHARE ? cw + WN * s : s, NA - 1);
    ar[s] = q < MB ? hr : lr;
    a_off[s] = (uint32_t)(q < MB ? q : q - MB) * (uint32_t)a_kt * 1024u;
  }

  // this block's units; without a split every block is one whole column group
  long u = sp.any() ? (long)blockIdx.x * sp.units / sp.blocks : (long)blockIdx.x * kt_count;
  const long u_end = sp.any() ? (long)(blockIdx.x + 1) * sp.units / sp.blocks : u + kt_count;
  while (u < u_end) {  // one segment per column group touched (block-uniform)
    const int g = (int)(u / kt_count);
    const int kt0 = (int)(u - (long)g * kt_count);
    const int kt1 = (int)min((long)kt_count, u_end - (long)g * kt_count);
    u = (long)g * kt_count + kt1;
    const int nb0 = (g * WN + cw) * SG_NB;       // this wave's first row block of W
    const int nbs = min(SG_NB, n_blocks - nb0);  // <= 0 for a wave past the matrix
    const int n_it = (kt1 - kt0 + WK - 1) / WK;  // block-uniform; step i is k-tile kt0 + kw + WK*i

    f32x4 acc[MB][SG_NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int j = 0; j < SG_NB; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nbb = min(nb0, n_blocks - 1);
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(w + (size_t)nbb * kt_count * 64, (size_t)(min(nb0 + SG_NB, n_blocks) - nbb) * kt_count * 1024);
    uint32_t w_off[SG_NB];
#pragma unroll
    for (int j = 0; j < SG_NB; ++j) w_off[j] = (uint32_t)(min(nb0 + j, n_blocks - 1) - nbb) * (uint32_t)kt_count * 1024u;

    // A step past the segment's k-range (the k-waves' last steps, and the padding of the step count to
    // a multiple of R) moves the lane offset past every resource's size: such loads read zeros without
    // touching memory and their products add nothing, so the ring needs no branches.
    uint4 wb[R][SG_NB], ab[R][APW];
    auto issue = [&](int slot, int i) {
      const int kt = kt0 + kw + WK * i;
      const uint32_t voff = lane_bytes | (kt < kt1 ? 0u : 0x80000000u);
      const uint32_t koff = (uint32_t)min(kt, kt1 - 1) * 1024u;
#pragma unroll
      for (int s = 0; s < APW; ++s) ab[slot][s] = buffer_load16(ar[s], voff, a_off[s] + koff, 0);
#pragma unroll
      for (int j = 0; j < SG_NB; ++j) wb[slot][j] = buffer_load16(wr, voff, w_off[j] + koff, kLoadStream);
    };
    auto compute = [&](int slot, int i) {
      uint4 av[NA];  // hi of row block m at m, lo at MB + m
      if constexpr (SHARE) {
        // every wave writes all its slots (a skipped write would be a branch in the ring)
        uint4 *st = lds + (size_t)((i & 1) * WK + kw) * S::NSLOT * 64;
#pragma unroll
        for (int s = 0; s < APW; ++s) st[(cw + WN * s) * 64 + lane] = ab[slot][s];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NA; ++q) av[q] = st[q * 64 + lane];
      } else {
#pragma unroll
        for (int q = 0; q < NA; ++q) av[q] = ab[slot][q];
      }
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < SG_NB; ++j) {
          acc[m][j] = mfma16(av[MB + m], wb[slot][j], acc[m][j]);
          acc[m][j] = mfma16(av[m], wb[slot][j], acc[m][j]);
        }
    };
    // R = D + 1 slots: each step first refills the slot freed by the previous step, then computes, so
    // D steps stay in flight while one is computed
#pragma unroll
    for (int d = 0; d < D; ++d) {
      issue(d, d);
      __builtin_amdgcn_sched_barrier(0);  // slots leave in ring order, so the waits stay partial
    }
    for (int it = 0; it < n_it; it += R) {  // block-uniform trip count; the final refills read nothing
#pragma unroll
      for (int d = 0; d < R; ++d) {
        issue((d + D) % R, it + d + D);
        compute(d, it + d);
        __builtin_amdgcn_sched_barrier(0);  // the scheduler would otherwise sink every refill to the end
      }
    }

    if constexpr (WK > 1) {  // k-waves 1.. hand their sums to k-wave 0, which adds them in order
      constexpr int RW = WN * 64 + 1;
      float *red = reinterpret_cast<float *>(lds);  // [WK-1][MB*16][RW], over the dead staging buffers
      __syncthreads();
      if (kw > 0) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int j = 0; j < SG_NB; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              red[((kw - 1) * MB * 16 + m * 16 + rq + e) * RW + cw * 64 + j * 16 + cq] = acc[m][j][e];
      }
      __syncthreads();
      if (kw == 0) {
#pragma unroll
        for (int q = 0; q < WK - 1; ++q)
#pragma unroll
          for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int j = 0; j < SG_NB; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[m][j][e] += red[(q * MB * 16 + m * 16 + rq + e) * RW + cw * 64 + j * 16 + cq];
      }
    }
    if (kw == 0 && nbs > 0) {
      if (sp.any()) {  // plane = this block's place among the blocks covering group g
        float *plane = partials + (size_t)(blockIdx.x - sp.first_block((long)g * kt_count)) * rows * n;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int j = 0; j < SG_NB; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = m * 16 + rq + e;
              if (r < rows && j < nbs) plane[(size_t)r * n + (nb0 + j) * 16 + cq] = acc[m][j][e];
            }
      } else {
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
    }
    if constexpr (SHARE || WK > 1) __syncthreads();  // the next segment reuses the LDS
  }
}

// ---------------------------------------------------------------- split-k reduction
// One thread per (row, 4 consecutive columns): sums the ks partials in split
// order (deterministic) and applies the epilogue.  For SwiGLU the threads of
// gate columns also read the matching up columns (16 further on).
// One thread per 8 consecutive columns of a row for the SwiGLU epilogue, so every store is a lane's
// 16-byte chunk of the packed hi/lo activation; one thread per 4 columns (one float4) for fp32 outputs.
__global__ void reduce_kernel(const float *__restrict__ partials, Splits sp, int rows, int n, LinearOut o) {
  const int cpt = o.kind == kSiluMul ? 8 : 4;  // columns per thread
  const int nt = n / cpt;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)rows * nt) return;
  const int r = (int)(idx / nt), c = (int)(idx % nt) * cpt;
  if (o.kind == kSiluMul && ((c >> 4) & 1)) return;  // up columns: read by their gate's thread
  const size_t plane = (size_t)rows * n;
  const int ks = sp.slots(c);  // c..c+cpt-1 (and the up columns c+16..) lie in one column group
  const float *p = partials + (size_t)r * n + c;
  float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
  add_splits(s0, p, plane, ks);
  if (o.kind == kSiluMul) {
    add_splits(s1, p + 4, plane, ks);
    float4 u0 = make_float4(0.f, 0.f, 0.f, 0.f), u1 = u0;
    add_splits(u0, p + 16, plane, ks);
    add_splits(u1, p + 20, plane, ks);
    const float y[8] = {silu_f(s0.x) * u0.x, silu_f(s0.y) * u0.y, silu_f(s0.z) * u0.z, silu_f(s0.w) * u0.w,
                        silu_f(s1.x) * u1.x, silu_f(s1.y) * u1.y, silu_f(s1.z) * u1.z, silu_f(s1.w) * u1.w};
    const int j = ((c >> 5) << 4) | (c & 15);  // gate column -> activation column (a multiple of 8)
    uint4 h, l;
    split_pack8(y, h, l);
    const size_t off = packed_offset(r, j, o.act_kt);
    *reinterpret_cast<uint4 *>(o.act_hi + off) = h;
    *reinterpret_cast<uint4 *>(o.act_lo + off) = l;
    // the row's padding columns (act_cols .. 32*act_kt-1: none or one 16-column block) follow the last
    // real 16-column block, whose writers clear them
    if (j + 16 >= o.act_cols && j + 16 < o.act_kt * 32) {
      const size_t pad = packed_offset(r, j + 16, o.act_kt);
      *reinterpret_cast<uint4 *>(o.act_hi + pad) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4 *>(o.act_lo + pad) = make_uint4(0, 0, 0, 0);
    }
  } else {
    float4 *q = reinterpret_cast<float4 *>(o.f32 + (size_t)r * o.ld + c);
    if (o.kind == kAccumulate) vadd(s0, *q);
    *q = s0;
  }
}

void launch_reduce(const float *partials, const Splits &sp, int rows, int n, const LinearOut &o, hipStream_t s) {
  const size_t total = (size_t)rows * (n / (o.kind == kSiluMul ? 8 : 4));
  if (total) reduce_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(partials, sp, rows, n, o);
}

// ---------------------------------------------------------------- tiled_gemm (rows > 64)
// Block tile MB x 16 rows by 256 columns.  The four waves sit side by side along the columns: wave w
// owns all MB row blocks and column blocks 4w..4w+3 (4 MB accumulators of 16 x 16).  Per k-tile the
// block needs 2 MB activation tiles (hi and lo of each row block), which every wave uses, and 16
// weight tiles, each used by one wave only.  So activations are shared through LDS (each wave fetches
// a quarter of them and writes them to one of two LDS stages a k-tile before they are used), while
// weights go from memory straight into the registers of the wave that uses them.  Both sit in a
// register ring PgShape::D k-tiles deep.  Latency is hidden by occupancy rather than ring depth: at
// 64 rows and a 2-deep ring a wave needs under 128 registers, so four blocks share a CU and one
// block's MFMAs run while the others wait at their barriers or on memory (measured on the 7B prefill
// products: 5 % faster than 128-row tiles at two blocks per CU, whose 4 KiB more activation reuse per
// k-tile does not make up for the lost occupancy).  Every tile is read through a buffer resource: a
// row block past the operand gets an empty one, k-tiles past the end move the lane offset out of
// range, so those loads read zeros without branches and the padded steps add nothing.
constexpr int PG_NBW = 4;          // 16-row blocks of W per wave
constexpr int PG_NB = 4 * PG_NBW;  // per block (256 columns)
template <int MB> struct PgShape {
  static constexpr int AT = 2 * MB;                  // activation tiles per k-tile (hi and lo)
  static constexpr int APW = AT / 4;                 // of them fetched by one wave
  static constexpr int D = 2;                        // k-tiles in flight
  static constexpr int GM = 32 / MB;                 // row tiles per group of the block order (512 rows)
  static constexpr size_t LDS = (size_t)2 * AT * 1024;
};

template <int MB>
__global__ __launch_bounds__(256, 4) void tiled_gemm_kernel(const uint4 *__restrict__ a_hi,
                                                            const uint4 *__restrict__ a_lo, int a_kt, int a_blocks,
                                                            int rows, const uint4 *__restrict__ w, int kt_count,
                                                            int n_blocks, int tiles_m, LinearOut o) {
  using S = PgShape<MB>;
  constexpr int AT = S::AT, APW = S::APW, D = S::D;
  extern __shared__ uint4 lds[];  // [2 stages][AT tiles][64 lanes]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar control
  // Block order: blocks go round-robin to the 8 XCDs, so each XCD takes a contiguous range of tile ids;
  // ids run through groups of GM row tiles, row tiles innermost, so the blocks one XCD runs together
  // share a few activation and weight slabs in its L2.
  const int nblk = gridDim.x;
  int t = blockIdx.x;
  if ((nblk & 7) == 0) t = (t & 7) * (nblk >> 3) + (t >> 3);
  const int tiles_n = nblk / tiles_m;  // the grid is exactly tiles_m * tiles_n
  const int group = t / (S::GM * tiles_n), first_m = group * S::GM;
  const int gm = min(S::GM, tiles_m - first_m);
  const int r_in = t - group * S::GM * tiles_n;
  const int tm = first_m + r_in % gm, tn = r_in / gm;
  const int mb0 = tm * MB, nbw0 = tn * PG_NB + wave * PG_NBW;

  // activation tiles this wave fetches: q = wave + 4i is the hi tile of row block q (q < MB) or the lo
  // tile of row block q - MB; LDS holds tile q at index q
  const uint32_t lane_bytes = (uint32_t)lane * 16u;
  __amdgpu_buffer_rsrc_t asrc[APW];
#pragma unroll
  for (int i = 0; i < APW; ++i) {
    const int q = wave + 4 * i;
    const int rb = mb0 + (q % MB);
    const bool ok = rb < a_blocks;
    const uint4 *base = (q < MB ? a_hi : a_lo) + (size_t)(ok ? rb : 0) * a_kt * 64;
    asrc[i] = make_rsrc(base, ok ? (size_t)a_kt * 1024 : 0);
  }
  // this wave's weight row blocks nbw0.. through one resource (empty past the matrix; a block past the
  // last one re-reads the last, and its columns are not stored)
  const int nbv = min(PG_NBW, n_blocks - nbw0);
  const __amdgpu_buffer_rsrc_t wsrc =
      make_rsrc(w + (size_t)(nbv > 0 ? nbw0 : 0) * kt_count * 64, nbv > 0 ? (size_t)nbv * kt_count * 1024 : 0);
  uint32_t w_off[PG_NBW];
#pragma unroll
  for (int j = 0; j < PG_NBW; ++j) w_off[j] = (uint32_t)min(j, max(nbv - 1, 0)) * (uint32_t)kt_count * 1024u;

  uint4 ar[D][APW], wr[D][PG_NBW];
  auto fetch = [&](int slot, int kt) {
    const uint32_t voff = lane_bytes | (kt < kt_count ? 0u : 0x80000000u);
    const uint32_t koff = (uint32_t)min(kt, kt_count - 1) * 1024u;
#pragma unroll
    for (int i = 0; i < APW; ++i) ar[slot][i] = buffer_load16(asrc[i], voff, koff, 0);  // reused through L2
#pragma unroll
    for (int j = 0; j < PG_NBW; ++j) wr[slot][j] = buffer_load16(wsrc, voff, w_off[j] + koff, 0);
  };
  auto stage = [&](int slot, int buf) {
    uint4 *st = lds + (size_t)buf * AT * 64;
#pragma unroll
    for (int i = 0; i < APW; ++i) st[(size_t)(wave + 4 * i) * 64 + lane] = ar[slot][i];
  };

  f32x4 acc[MB][PG_NBW];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < PG_NBW; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, int slot) {
    const uint4 *st = lds + (size_t)buf * AT * 64;
    uint4 ah[MB], al[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      ah[m] = st[(size_t)m * 64 + lane];
      al[m] = st[(size_t)(MB + m) * 64 + lane];
    }
    // the lo and hi products of one accumulator are four instructions apart
#pragma unroll
    for (int m = 0; m < MB; ++m) {
#pragma unroll
      for (int j = 0; j < PG_NBW; ++j) acc[m][j] = mfma16(al[m], wr[slot][j], acc[m][j]);
#pragma unroll
      for (int j = 0; j < PG_NBW; ++j) acc[m][j] = mfma16(ah[m], wr[slot][j], acc[m][j]);
    }
  };

  // prologue: k-tiles 0..D-1 in flight (k-tile j always lives in slot j % D), k-tile 0's
  // activations staged
#pragma unroll
  for (int p = 0; p < D; ++p) {
    fetch(p, p);
    __builtin_amdgcn_sched_barrier(0);
  }
  stage(0, 0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  // step kt: compute k-tile kt (activations from LDS stage kt & 1, weights from slot kt % D), stage
  // k-tile kt+1's activations into the other stage, refill the consumed slot with k-tile kt + D
  for (int k0 = 0; k0 < kt_count; k0 += D) {  // block-uniform; steps past kt_count compute zeros
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kt = k0 + d;
      compute(kt & 1, d);
      stage((d + 1) % D, (kt + 1) & 1);
      fetch(d, kt + D);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  const int rq = (lane >> 4) * 4, cq = lane & 15;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < PG_NBW; ++j) {
      const int nb = nbw0 + j;
      if (nb >= n_blocks) continue;
      if (o.kind == kSiluMul && (j & 1)) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = (mb0 + m) * 16 + rq + e;
        if (r < rows) epi_store(o, r, nb * 16 + cq, acc[m][j][e], o.kind == kSiluMul ? acc[m][j + 1][e] : 0.f);
      }
    }
}

// ---------------------------------------------------------------- dispatch
// Shape of a streaming launch: column waves WN and the stream-K split.  Every
// CU gets exactly one block, so all carry the same work whatever the shape
// (with 257..511 blocks some CUs would run two and set the time).  Preferred
// (above 16 rows): more column waves (fewer activation requests per weight
// byte), as long as every wave keeps at least 8 k-steps to pipeline and the
// partial sums (written and read back once) stay below the weight bytes.  Measured on the
// 7B decode shapes, one block per CU beats two: a second block doubles the
// partial sums for little gain in bandwidth.  A product too small to split
// runs unsplit, one block per column group.
constexpr int kCUs = 256;

struct StreamPlan {
  int wn, grid;
  Splits sp;
};

static StreamPlan stream_plan(int rows, int n, int k, SplitPolicy policy) {
  const int nb = n / 16, kt = round_up(k, kTileK) / kTileK;
  const double w_bytes = 2.0 * n * k;
  // Wide column groups first (fewer activation requests per weight byte).  With 16 rows or fewer the
  // activations are a small share of the bytes, and narrow groups mean fewer partial planes per column
  // for the consumers to add up (measured on the batch-1 7B layer: 124.7 -> 120.1 us).
  const int order[2][3] = {{4, 2, 1}, {1, 2, 4}};
  for (int wn : order[rows <= 16 ? 1 : 0]) {
    if (policy == kSplitNone) break;
    const int wk = 4 / wn, cols = SG_NB * 16 * wn;
    const int groups = (nb + SG_NB * wn - 1) / (SG_NB * wn);
    if (policy == kSplitBalanced) {
      const long units = (long)groups * kt;
      if (units / kCUs / wk < 8) continue;
      if (8.0 * rows * cols * (kCUs + groups) > w_bytes) continue;
      return {wn, kCUs, Splits{kCUs, (int)units, kt, cols}};
    }
    // uniform: ks equal cuts per group, groups * ks <= one block per CU
    if (groups > kCUs) continue;
    int ks = kCUs / groups;
    while (ks > 1 && kt / ks / wk < 8) --ks;
    if (ks < 2 || 8.0 * rows * cols * groups * ks > w_bytes) continue;
    return {wn, groups * ks, Splits{groups * ks, groups * kt, kt, cols}};
  }
  // unsplit: the layout with the most blocks
  return {1, (nb + SG_NB - 1) / SG_NB, Splits{}};
}

size_t linear_partial_floats(int rows, int n, int k, SplitPolicy policy) {
  if (rows > 64) return 0;
  const StreamPlan p = stream_plan(rows, n, k, policy);
  if (!p.sp.any()) return 0;
  int max_slots = 1;
  for (int c = 0; c < n; c += p.sp.group_cols) max_slots = std::max(max_slots, p.sp.slots(c));
  return (size_t)max_slots * rows * n;
}

template <int MB>
static void launch_stream(int wn, int grid, hipStream_t s, const uint4 *ah, const uint4 *al, int a_kt, int rows,
                          const uint4 *w, int kt_count, int n_blocks, const LinearOut &o, float *partials,
                          const Splits &sp) {
  if (wn == 4)
    stream_gemm_kernel<MB, 4><<<grid, 256, 0, s>>>(ah, al, a_kt, rows, w, kt_count, n_blocks, o, partials, sp);
  else if (wn == 2)
    stream_gemm_kernel<MB, 2><<<grid, 256, 0, s>>>(ah, al, a_kt, rows, w, kt_count, n_blocks, o, partials, sp);
  else
    stream_gemm_kernel<MB, 1><<<grid, 256, 0, s>>>(ah, al, a_kt, rows, w, kt_count, n_blocks, o, partials, sp);
}

Splits launch_linear(const Act &a, const uint16_t *w_packed, int n, int k, const LinearOut &o, float *partials,
                     size_t partial_floats, SplitPolicy policy, hipStream_t s) {
  const int kt_count = round_up(k, kTileK) / kTileK;
  const int n_blocks = n / 16;
  const uint4 *w = reinterpret_cast<const uint4 *>(w_packed);
  const uint4 *ah = reinterpret_cast<const uint4 *>(a.hi), *al = reinterpret_cast<const uint4 *>(a.lo);
  const int a_kt = a.kpad / kTileK;
  if (a.rows <= 64) {
    StreamPlan p = stream_plan(a.rows, n, k, policy);
    if (p.sp.any() && (!partials || partial_floats < linear_partial_floats(a.rows, n, k, policy)))
      p = stream_plan(a.rows, n, k, kSplitNone);
    switch ((a.rows + 15) / 16) {
      case 1: launch_stream<1>(p.wn, p.grid, s, ah, al, a_kt, a.rows, w, kt_count, n_blocks, o, partials, p.sp); break;
      case 2: launch_stream<2>(p.wn, p.grid, s, ah, al, a_kt, a.rows, w, kt_count, n_blocks, o, partials, p.sp); break;
      case 3: launch_stream<3>(p.wn, p.grid, s, ah, al, a_kt, a.rows, w, kt_count, n_blocks, o, partials, p.sp); break;
      default: launch_stream<4>(p.wn, p.grid, s, ah, al, a_kt, a.rows, w, kt_count, n_blocks, o, partials, p.sp); break;
    }
    return p.sp;
  }
  constexpr int MB = 4;  // 64-row block tiles
  const int tiles_n = (n_blocks + PG_NB - 1) / PG_NB;
  const int tiles_m = (a.rows + MB * 16 - 1) / (MB * 16);
  tiled_gemm_kernel<MB><<<tiles_m * tiles_n, 256, PgShape<MB>::LDS, s>>>(ah, al, a_kt, a.row_blocks, a.rows, w,
                                                                         kt_count, n_blocks, tiles_m, o);
  return Splits{};
}

}  // namespace llmdec
