// Weight products: out[m][n] = sum_k a[m][k] * W[n][k] on the matrix cores
// (v_mfma_f32_16x16x32_f16, fp32 accumulation).
//
// Both operands are fp16: the activation rounded to nearest-even by its
// producer (the pages' minimal engine computes in fp16), the weight carried
// exactly as fp16(w * 2^s) with one shift per matrix (see weight_shift), so a
// product is one MFMA per tile pair and its fp32 result is multiplied by 2^-s.
// An fp16 activation keeps 11 significant bits, eight times bf16's 8: one
// bf16 rounding at each product input would put the 7B-layer output beyond a
// 2e-2 max-abs bound against an unrounded reference, fp16 stays well inside.
// Where more precision is needed the activation comes as an fp16 pair hi + lo
// (NP = 2 planes, two MFMAs per tile pair, about 22 bits): always for the
// q|k|v product (k and v are rounded to bf16 when they enter the cache, and
// with single fp16 inputs about one in ten of them would land on the other
// side of a bf16 rounding boundary than an exact product's, a full bf16 step
// that every later token attends to), and for every product of a decode step
// (its rounding errors compound over the layers of a model: 32 layers of
// single fp16 inputs bring the logits to 1.6e-2 of the exact ones, pairs to
// 1.2e-3; the second plane costs a decode step little, its time is the weights').
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
//     per column wave (4 row blocks of W); its 4 waves take interleaved
//     k-tiles of the block's k-range and keep a ring of 3 to 8 k-steps
//     (weights and activations) in flight.  Wave sums meet in LDS.  Narrow
//     matrices also split k across blocks: each block then stores its fp32
//     partial sums and the caller adds them (launch_reduce, or the next kernel
//     that reads the result anyway).
//   * tiled_gemm (rows > 64, prefill): see its own comment.
//
// Epilogues: store fp32; add into fp32 (the residual stream); SwiGLU, where
// W's row blocks alternate gate / up (block 2j: gate rows 16j.., block 2j+1:
// up rows 16j..) and the kernel writes silu(g) * u straight into the packed
// fp16 activation of the down projection.
#include "bodies.h"

namespace llmdec {

__device__ inline f32x4 mfma16(const uint4 &a, const uint4 &b, f32x4 c) {
  f16x8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
}

__device__ inline float silu_f(float g) { return g / (1.0f + expf(-g)); }

// One output element through the epilogue.  c is the column of the product;
// for kSiluMul only gate columns call this, with u the matching up value.
__device__ inline void epi_store(const LinearOut &o, int r, int c, float v, float u) {
  if (o.kind == kSiluMul) {
    const int j = ((c >> 5) << 4) | (c & 15);  // gate column -> activation column
    const float y = silu_f(v) * u;
    const size_t off = packed_offset(r, j, o.act_kt);
    const uint16_t h = f32_to_f16(y);
    o.act[off] = h;
    if (o.act_lo) o.act_lo[off] = f32_to_f16(y - f16_to_f32(h));
    // the row's padding columns (act_cols .. 32*act_kt-1, fewer than 16 since act_cols % 16 == 0)
    // follow the last real 16-column block, whose writers clear them
    if (j + 16 >= o.act_cols && j + 16 < o.act_kt * 32) {
      const size_t pad = packed_offset(r, j + 16, o.act_kt);
      o.act[pad] = 0;
      if (o.act_lo) o.act_lo[pad] = 0;
    }
  } else {
    float *p = o.f32 + (size_t)r * o.ld + c;
    *p = o.kind == kAccumulate ? *p + v : v;
  }
}

// ---------------------------------------------------------------- stream_gemm (rows <= 64)
// A block is 4 waves: WN column waves, each owning SG_NB row blocks of W (64
// output columns), times WK = 4 / WN k-waves that take interleaved k-tiles, so
// one step of the block covers WK k-tiles.  A k-tile's MB activation tiles
// (one per row block) are needed by all WN column waves of its
// k-wave: with WN > 1 those waves fetch a share each and pass them on through
// LDS, which divides the activation requests per weight byte by WN.  (The
// activation tiles are L2 hits, but vector loads retire in issue order, so
// each one holds a request slot for as long as the weight loads ahead of it.)
// k-wave sums meet in LDS at the end; k-splits across blocks store fp32
// partials that the consumer adds.
constexpr int SG_NB = 4;

template <int MB, int WN, int NP> struct SgShape {
  static constexpr int WK = 4 / WN;
  static constexpr int NA = NP * MB;                            // activation tiles per k-tile
  static constexpr int APW = WN > 1 ? (NA + WN - 1) / WN : NA;  // of them fetched by one wave
  // k-steps in flight per wave: as deep as about 230 registers allow (two waves per SIMD), counting the
  // ring, the activation operands read back from LDS and the accumulators; one plane's shallower steps
  // make deeper rings, whose addressing needs 15 registers more headroom to compile without spills
  static constexpr int RAW = ((NP > 1 ? 230 : 215) - (WN > 1 ? 4 * NA : 0) - 16 * MB) / (4 * (SG_NB + APW)) - 2;
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
//
// w points at the first of the n_blocks column blocks the product covers; w_end at the packed matrix's
// trailer (its scale), which follows the matrix's last column block, so that a product can cover a
// range of a matrix's columns.
template <int MB, int WN, int NP>
__device__ __forceinline__ void stream_gemm_body(uint4 *lds, int bid, const uint4 *__restrict__ a_act,
                                                 const uint4 *__restrict__ a_lo, int a_kt, int rows,
                                                 const uint4 *__restrict__ w, const uint4 *__restrict__ w_end,
                                                 int kt_count, int n_blocks, const LinearOut &o,
                                                 float *__restrict__ partials, const Splits &sp) {
  using S = SgShape<MB, WN, NP>;
  constexpr int WK = S::WK, NA = S::NA, APW = S::APW, D = S::D, R = S::R;
  constexpr bool SHARE = WN > 1;
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
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(a_act, a_bytes), lr = make_rsrc(NP > 1 ? a_lo : a_act, a_bytes);
  // activation tiles this wave fetches: q = cw + WN*s (row block q of the first plane, or row block q - MB
  // of the lo plane)
  __amdgpu_buffer_rsrc_t ar[APW];
  uint32_t a_off[APW];
#pragma unroll
  for (int s = 0; s < APW; ++s) {
    const int q = min(SHARE ? cw + WN * s : s, NA - 1);
    ar[s] = q < MB ? hr : lr;
    a_off[s] = (uint32_t)(q < MB ? q : q - MB) * (uint32_t)a_kt * 1024u;
  }

  // this block's units; without a split every block is one whole column group
  long u = sp.any() ? (long)bid * sp.units / sp.blocks : (long)bid * kt_count;
  const long u_end = sp.any() ? (long)(bid + 1) * sp.units / sp.blocks : u + kt_count;
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
      uint4 av[NA];  // row block m at m, its lo part (NP = 2) at MB + m
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
          if constexpr (NP > 1) acc[m][j] = mfma16(av[MB + m], wb[slot][j], acc[m][j]);  // smaller part first
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
      const float wunscale = weight_unscale(w_end);
      if (sp.any()) {  // plane = this block's place among the blocks covering group g
        float *plane = partials + (size_t)(bid - sp.first_block((long)g * kt_count)) * rows * n;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int j = 0; j < SG_NB; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = m * 16 + rq + e;
              if (r < rows && j < nbs) plane[(size_t)r * n + (nb0 + j) * 16 + cq] = acc[m][j][e] * wunscale;
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
                if ((j & 1) == 0) epi_store(o, r, c, acc[m][j][e] * wunscale, acc[m][j + 1][e] * wunscale);
              } else {
                epi_store(o, r, c, acc[m][j][e] * wunscale, 0.f);
              }
            }
      }
    }
    if constexpr (SHARE || WK > 1) __syncthreads();  // the next segment reuses the LDS
  }
}

template <int MB, int WN, int NP>
__global__ __launch_bounds__(256, 2) void stream_gemm_kernel(const uint4 *__restrict__ a_act,
                                                             const uint4 *__restrict__ a_lo, int a_kt, int rows,
                                                             const uint4 *__restrict__ w,
                                                             const uint4 *__restrict__ w_end, int kt_count,
                                                             int n_blocks, LinearOut o, float *__restrict__ partials,
                                                             Splits sp) {
  __shared__ uint4 lds[SgShape<MB, WN, NP>::LDS_U4];
  stream_gemm_body<MB, WN, NP>(lds, blockIdx.x, a_act, a_lo, a_kt, rows, w, w_end, kt_count, n_blocks, o, partials,
                               sp);
}

// ---------------------------------------------------------------- split-k reduction
// Sums the ks partials of each output in split order (deterministic) and applies the epilogue.  One
// thread per 8 consecutive columns of a row for the SwiGLU epilogue, so every store is a lane's
// 16-byte chunk of the packed fp16 activation (the threads of gate columns also read the matching up
// columns, 16 further on); one thread per 4 columns (one float4) for fp32 outputs.
__device__ __forceinline__ void reduce_item(size_t idx, const float *__restrict__ partials, const Splits &sp,
                                            int rows, int n, const LinearOut &o) {
  const int cpt = o.kind == kSiluMul ? 8 : 4;  // columns per thread
  const int nt = n / cpt;
  if (idx >= (size_t)rows * nt) return;
  const int r = (int)(idx / nt), c = (int)(idx % nt) * cpt;
  if (o.kind == kSiluMul && ((c >> 4) & 1)) return;  // up columns: read by their gate's thread
  const size_t plane = (size_t)rows * n;
  const int ks = sp.slots(c);  // c..c+cpt-1 (and the up columns c+16..) lie in one column group
  const float *p = partials + (size_t)r * n + c;
  float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (o.kind == kSiluMul) {
    float4 acc[4] = {s0, s0, s0, s0};  // gate columns c..c+7, then the matching up columns c+16..c+23
    const float *src[4] = {p, p + 4, p + 16, p + 20};
    const int kss[4] = {ks, ks, ks, ks};
    add_splits_n<4>(acc, src, plane, kss);
    s0 = acc[0];
    const float4 s1 = acc[1], u0 = acc[2], u1 = acc[3];
    const float y[8] = {silu_f(s0.x) * u0.x, silu_f(s0.y) * u0.y, silu_f(s0.z) * u0.z, silu_f(s0.w) * u0.w,
                        silu_f(s1.x) * u1.x, silu_f(s1.y) * u1.y, silu_f(s1.z) * u1.z, silu_f(s1.w) * u1.w};
    const int j = ((c >> 5) << 4) | (c & 15);  // gate column -> activation column (a multiple of 8)
    const size_t off = packed_offset(r, j, o.act_kt);
    if (o.act_lo) {
      uint4 h, l;
      pack8_f16x2(y, h, l);
      *reinterpret_cast<uint4 *>(o.act + off) = h;
      *reinterpret_cast<uint4 *>(o.act_lo + off) = l;
    } else {
      *reinterpret_cast<uint4 *>(o.act + off) = pack8_f16(y);
    }
    // the row's padding columns (act_cols .. 32*act_kt-1: none or one 16-column block) follow the last
    // real 16-column block, whose writers clear them
    if (j + 16 >= o.act_cols && j + 16 < o.act_kt * 32) {
      const size_t pad = packed_offset(r, j + 16, o.act_kt);
      *reinterpret_cast<uint4 *>(o.act + pad) = make_uint4(0, 0, 0, 0);
      if (o.act_lo) *reinterpret_cast<uint4 *>(o.act_lo + pad) = make_uint4(0, 0, 0, 0);
    }
  } else {
    add_splits(s0, p, plane, ks);
    float4 *q = reinterpret_cast<float4 *>(o.f32 + (size_t)r * o.ld + c);
    if (o.kind == kAccumulate) vadd(s0, *q);
    *q = s0;
  }
}

__global__ __launch_bounds__(256) void reduce_kernel(const float *__restrict__ partials, Splits sp, int rows, int n,
                                                     LinearOut o) {
  reduce_item((size_t)blockIdx.x * blockDim.x + threadIdx.x, partials, sp, rows, n, o);
}

void launch_reduce(const float *partials, const Splits &sp, int rows, int n, const LinearOut &o, hipStream_t s) {
  const size_t total = (size_t)rows * (n / (o.kind == kSiluMul ? 8 : 4));
  if (total) reduce_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(partials, sp, rows, n, o);
}

// ---------------------------------------------------------------- tile_gemm (rows > 64)
// A block is WR x WC waves (2 x 2, or 2 x 4 with two waves per SIMD); wave (wr, wc) computes WM row
// blocks by WNT column blocks of the output, so the block tile is BM = WR WM row blocks by BN = WC WNT
// column blocks (16 x 16 each).  Per k-tile (32 deep) the block needs NP * BM activation tiles (each
// used by the WC waves of its row group) and BN weight tiles (each used by the WR waves of its column
// group).  All of them go from memory straight into LDS (buffer_load ... lds: lane l's 16 bytes land at
// l * 16 of the tile's 1 KiB slot, which is the packed tile itself), every wave issuing an equal share,
// through R stages.
// Step t:
//   * wait until k-tile t + 1 has landed (the loads of R - 2 later k-tiles may still be in flight) and
//     for this wave's LDS reads of stage t, then a barrier: every wave's share of k-tile t + 1 is in
//     LDS, and every wave has finished reading stage t;
//   * read stage t + 1 into the second register set (the fragments of k-tile t + 1);
//   * issue the loads of k-tile t + R into stage t, which no wave reads any more;
//   * run the WM * WNT * NP MFMAs of k-tile t from the first register set (read during step t - 1), so
//     the LDS reads of the next k-tile overlap them.
// With WM = WNT = 8 a wave keeps 256 accumulators and one wave per SIMD runs; the R - 1 k-tiles in
// flight (3000+ clocks of MFMA work) cover the memory latency instead of other waves.  A 256 x 256
// block tile loads 32 KiB per k-tile for 64 MFMAs per SIMD, a third less per MFMA than two waves
// side by side with weights in registers.
//
// Blocks go round-robin to the 8 XCDs, so block b takes tile (b % 8) * G/8 + b / 8 of G (a multiple of
// 8, spare blocks exit), with tiles numbered column-major (row tiles innermost): the blocks one XCD runs
// together cover every row tile of a few column groups, so each weight tile is fetched into that
// XCD's L2 once and each activation k-slab serves all of them.
// PCU: blocks per CU (1, or 2 with half the LDS each; the registers are then also halved).  WR x WC
// waves per block (2 x 2, or 2 x 4: two waves per SIMD sharing one block tile).
template <int WM, int WNT, int NP, int PCU = 1, int WR = 2, int WC = 2> struct TgShape {
  static constexpr int NW = WR * WC;                 // waves per block
  static constexpr int BM = WR * WM, BN = WC * WNT;  // row / column blocks of the block tile
  static constexpr int AT = NP * BM;                 // activation tiles per k-tile (all planes)
  static constexpr int TILES = AT + BN;              // 1 KiB tiles per stage
  static constexpr int G = TILES / NW;               // loads per wave per k-tile
  static constexpr int R = 160 / PCU / TILES < 4 ? 160 / PCU / TILES : 4;  // stages (160 KiB of LDS per CU)
  static_assert(AT % NW == 0 && BN % NW == 0, "load i of wave w is tile NW i + w: a whole number per kind");
  static_assert(NP == 1 || BM % NW == 0, "a load's plane is the same for every wave");
  static_assert(WNT % 2 == 0, "gate/up column pairs");
  static_assert(R >= 3 && (R - 1) * G <= 63, "at least one k-tile of lookahead; the loads fit vmcnt");
};

// The kRope epilogue (see RopeRows).  Each wave passes its results through its own share of the LDS
// (free once the k-loop has ended), one 16-row block at a time: its accumulators go to a row-major
// staging area, and the wave then walks the staged rows pair by pair, lane l taking pair l of a row (two
// rows a step when a row holds 32 pairs), so a q row leaves as contiguous fp32 pairs and a k row as
// contiguous bf16 pairs.  The walk is a short loop, not one unrolled copy per accumulator (an epilogue
// that large runs from outside the instruction cache).  Each pair's rotation is formed where it is used
// (the angle reduced in double, then sine and cosine in fp32, as the RoPE/append kernel does): a load
// from memory in the walk would make the wave wait for its earlier stores too.  The rows' positions
// and page slots are looked up once, lane l holding rows l and l + 64 of the wave, and read in the walk
// with scalar lane reads.
// A wave whose columns are all v columns skips the walk: it works on the accumulators' own layout (lane
// l of a 16 x 16 block holds column l % 16 of rows 4 (l / 16) .. + 3), and where a lane's four rows are
// the token slots 4i..4i+3 of one page (consecutive positions of one sequence), its four values are
// the four adjacent bf16 of the V layout and leave as one 8-byte store (else one value at a time).  It
// parks its blocks of one 16-row band in its LDS share and takes them in a short loop (one copy of the
// per-block code), each lane reading back its own 16 bytes.
template <int WM, int WNT>
__device__ __forceinline__ void tile_v_epilogue(f32x4 *fr, const f32x4 (&acc)[WM][WNT], float wunscale,
                                                const RopeRows &rp, int rows, int n_blocks, int mw, int nw,
                                                const int (&slot_r)[2], int lane) {
  const int D = rp.head_dim;
  const int v0 = rp.n_heads * D + rp.n_kv_heads * D;  // the first v column of the q|k|v row
  const int g = lane >> 4, cq = lane & 15;
  StaticFor<0, WM>::run([&](auto mc) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value;
#pragma unroll
    for (int j = 0; j < WNT; ++j) fr[j * 64 + lane] = acc[m][j] * wunscale;
    int slt[4];  // page * 16 + offset of this lane's rows m*16 + 4g + e (-1: none)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      slt[e] = __builtin_amdgcn_ds_bpermute(((m * 16 + 4 * g + e) & 63) * 4, slot_r[(m * 16) >> 6]);
    const int r0 = (mw + m) * 16 + 4 * g;
    const bool quad = r0 + 3 < rows && slt[0] >= 0 && (slt[0] & 3) == 0 && slt[1] == slt[0] + 1 &&
                      slt[2] == slt[0] + 2 && slt[3] == slt[0] + 3;
#pragma unroll 2
    for (int j = 0; j < WNT; ++j) {
      if (nw + j >= n_blocks) break;  // no columns past the matrix (wave-uniform)
      const f32x4 v = fr[j * 64 + lane];
      const int d = rp.col0 + (nw + j) * 16 + cq - v0;
      const size_t head_d = (size_t)(d / D);
      if (quad) {  // V [h][o/4][d][o%4]
        const size_t head = (size_t)(slt[0] >> 4) * rp.n_kv_heads + head_d;
        const uint2 w = make_uint2(f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                                   f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
        *reinterpret_cast<uint2 *>(rp.pool_v + (head * 4 + ((slt[0] & 15) >> 2)) * D * 4 + (size_t)(d % D) * 4) = w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (r0 + e < rows && slt[e] >= 0) {
            const size_t head = (size_t)(slt[e] >> 4) * rp.n_kv_heads + head_d;
            const int of = slt[e] & 15;
            rp.pool_v[(head * 4 + (of >> 2)) * D * 4 + (size_t)(d % D) * 4 + (of & 3)] = f32_to_bf16(v[e]);
          }
      }
    }
  });
}

template <int WM, int WNT>
__device__ __forceinline__ void tile_rope_epilogue(uint4 *lds, const f32x4 (&acc)[WM][WNT], float wunscale,
                                                   const LinearOut &o, int rows, int n_blocks, int mw, int nw,
                                                   int wave, int lane) {
  constexpr int P = WNT * 8;            // pairs per row of the wave's columns
  constexpr int PITCH = WNT * 16 + 4;   // floats per staged row (the 4-float skew spreads the rows' banks)
  constexpr int STEPS = 16 * P / 64;    // walk steps per 16-row block
  static_assert(WM * 16 <= 128, "two rows per lane");
  const RopeRows &rp = o.rope;
  const int D = rp.head_dim;
  const int hid = rp.n_heads * D, kvc = rp.n_kv_heads * D;
  const bool kv = rp.col0 > 0;
  const int c0 = nw * 16;                                  // the wave's first column of the product
  const int ncols = min(WNT * 16, (n_blocks - nw) * 16);  // its real columns (none past the matrix)
  const int rq = (lane >> 4) * 4, cq = lane & 15;
  float *st = reinterpret_cast<float *>(lds) + wave * (16 * PITCH + 2 * 64);
  double *fq = reinterpret_cast<double *>(st + 16 * PITCH);  // [64] rotation frequencies

  // positions and page slots (K/V products; page -1 = no store, flagged) of rows mw*16 + lane and + 64
  int pos_r[2] = {0, 0};
  int2 slot[2] = {make_int2(-1, 0), make_int2(-1, 0)};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = mw * 16 + lane + 64 * h;
    if (lane + 64 * h >= WM * 16 || r >= rows) continue;
    const int pos = rp.tok_pos[r];
    pos_r[h] = pos;
    if (!kv) continue;
    const int seq = rp.tok_seq[r];
    if (seq < 0 || seq >= rp.n_seqs) {
      raise_error(rp.err, kErrSeq);
    } else if (pos < 0 || (pos >> 4) >= rp.max_pages) {
      raise_error(rp.err, kErrPos);
    } else {
      const int page = rp.block_tables[(size_t)seq * rp.max_pages + (pos >> 4)];
      if (page < 0 || page >= rp.num_pages) raise_error(rp.err, kErrPage);
      else slot[h] = make_int2(page, pos & 15);
    }
  }
  const double f_lane = rp.fr.inv_freq[lane];
  __syncthreads();  // every wave's k-loop reads of the LDS are done
  if (kv && rp.col0 + c0 >= hid + kvc) {  // every column of the wave is a v column (wave-uniform)
    const int slot_r[2] = {slot[0].x >= 0 ? slot[0].x * 16 + slot[0].y : -1,
                           slot[1].x >= 0 ? slot[1].x * 16 + slot[1].y : -1};
    tile_v_epilogue<WM, WNT>(reinterpret_cast<f32x4 *>(st), acc, wunscale, rp, rows, n_blocks, mw, nw, slot_r, lane);
    return;
  }
  fq[lane] = f_lane;
  double f_pair = 0.0;  // 64 % P == 0: the frequency of this lane's pair (q or k columns)
  if constexpr (64 % P == 0) {
    const int col = rp.col0 + c0 + 2 * (lane % P);
    const int d = col < hid ? col : col - hid;
    f_pair = fq[(d % D) >> 1];
  }

  StaticFor<0, WM>::run([&](auto mc) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value;
    const int r0 = (mw + m) * 16;  // the block's first row
#pragma unroll
    for (int j = 0; j < WNT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[(rq + e) * PITCH + j * 16 + cq] = acc[m][j][e] * wunscale;
    // A step covers at most two rows (P >= 32); their positions and slots are read from the lanes that
    // hold them with scalar reads.  With 64 % P == 0 a lane keeps the same pair in every step, so its
    // frequency is read once.
#pragma unroll 4
    for (int it = 0; it < STEPS; ++it) {
      const int idx = it * 64 + lane, rl = idx / P, p = idx - rl * P;
      const int rla = (it * 64) / P, rlb = min(rla + 1, 15);  // the step's rows (wave-uniform)
      const int rwa = m * 16 + rla, rwb = m * 16 + rlb;
      const int pos_a = __builtin_amdgcn_readlane(pos_r[rwa >> 6], rwa & 63);
      const int pos_b = __builtin_amdgcn_readlane(pos_r[rwb >> 6], rwb & 63);
      const int pg_a = __builtin_amdgcn_readlane(slot[rwa >> 6].x, rwa & 63);
      const int pg_b = __builtin_amdgcn_readlane(slot[rwb >> 6].x, rwb & 63);
      const int of_a = __builtin_amdgcn_readlane(slot[rwa >> 6].y, rwa & 63);
      const int of_b = __builtin_amdgcn_readlane(slot[rwb >> 6].y, rwb & 63);
      const bool on_a = rl == rla;
      const int pos = on_a ? pos_a : pos_b;
      const int2 ps = make_int2(on_a ? pg_a : pg_b, on_a ? of_a : of_b);
      const int r = r0 + rl;  // row of the product
      if (r >= rows || 2 * p >= ncols) continue;
      const float2 xv = *reinterpret_cast<const float2 *>(st + rl * PITCH + 2 * p);
      const int col = rp.col0 + c0 + 2 * p;
      if (col < hid + kvc) {  // q or k: rotate the pair
        const int d = col < hid ? col : col - hid;
        float c, sn;
        rope_cos_sin(pos, 64 % P == 0 ? f_pair : fq[(d % D) >> 1], c, sn);
        const float re = xv.x * c - xv.y * sn, ro = xv.x * sn + xv.y * c;
        if (col < hid) {
          *reinterpret_cast<float2 *>(o.f32 + (size_t)r * o.ld + c0 + 2 * p) = make_float2(re, ro);
        } else if (ps.x >= 0) {  // K [h][o][d]
          const size_t head = (size_t)ps.x * rp.n_kv_heads + d / D;
          *reinterpret_cast<uint32_t *>(rp.pool_k + (head * 16 + ps.y) * D + (d % D)) =
              f32_to_bf16(re) | ((uint32_t)f32_to_bf16(ro) << 16);
        }
      } else if (ps.x >= 0) {  // V [h][o/4][d][o%4]
        const int d = col - hid - kvc;
        const size_t head = (size_t)ps.x * rp.n_kv_heads + d / D;
        uint16_t *vp = rp.pool_v + (head * 4 + (ps.y >> 2)) * D * 4 + (size_t)(d % D) * 4 + (ps.y & 3);
        vp[0] = f32_to_bf16(xv.x);
        vp[4] = f32_to_bf16(xv.y);
      }
    }
  });
}

// ROPE: the kRope epilogue (its own instantiation, so that the others carry none of its registers).
template <int WM, int WNT, int NP, int PCU, bool ROPE, int WR = 2, int WC = 2>
__global__ __launch_bounds__(64 * WR * WC, PCU) void tile_gemm_kernel(const uint4 *__restrict__ a_act,
                                                           const uint4 *__restrict__ a_lo, int a_kt, int a_blocks,
                                                           int rows, const uint4 *__restrict__ w,
                                                           const uint4 *__restrict__ w_end, int kt_count,
                                                           int n_blocks, int tiles_m, int n_tiles, LinearOut o) {
  using S = TgShape<WM, WNT, NP, PCU, WR, WC>;
  constexpr int BM = S::BM, BN = S::BN, AT = S::AT, TILES = S::TILES, G = S::G, R = S::R, NW = S::NW;
  __shared__ uint4 lds[R * TILES * 64];  // [R stages][TILES tiles][64 lanes]
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4 *)lds;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave % WR, wc = wave / WR;
  const int per_xcd = (int)(gridDim.x >> 3);
  const int t = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (t >= n_tiles) return;  // block-uniform: a spare block of the rounded-up grid
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int mb0 = tm * BM, nb0 = tn * BN;

  // Load i of this wave is stage tile q = NW i + wave: activation tiles first (plane q / BM, row block
  // mb0 + q % BM), then weight tiles (column block nb0 + q - AT).  A row block past the operand reads
  // zeros (its lane offsets leave the resource); a column block past the matrix re-reads the last one
  // (its columns are not stored).  Offsets are bytes from the operand's base, without the k-tile.
  const u32x4 dhi = buffer_desc(a_act, (uint32_t)a_blocks * (uint32_t)a_kt * 1024u);
  const u32x4 dlo = buffer_desc(NP > 1 ? a_lo : a_act, (uint32_t)a_blocks * (uint32_t)a_kt * 1024u);
  const u32x4 dw = buffer_desc(w, (uint32_t)n_blocks * (uint32_t)kt_count * 1024u);
  uint32_t base[G], oob[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int q = NW * i + wave;
    if (NW * i < AT) {
      const int rb = mb0 + q % BM;
      base[i] = (uint32_t)min(rb, a_blocks - 1) * (uint32_t)a_kt * 1024u;
      oob[i] = rb < a_blocks ? 0u : 0x80000000u;
    } else {
      base[i] = (uint32_t)min(nb0 + q - AT, n_blocks - 1) * (uint32_t)kt_count * 1024u;
      oob[i] = 0u;
    }
  }
  const uint32_t lane_bytes = (uint32_t)lane * 16u;
  // load i of k-tile kt into stage st (past the last k-tile: zeros, through the lane offset)
  auto issue = [&](int st, int kt, int i) {
    const uint32_t kflag = kt < kt_count ? 0u : 0x80000000u;
    const uint32_t koff = (uint32_t)min(kt, kt_count - 1) * 1024u;
    const u32x4 d = NW * i < AT ? ((NW * i) / BM == 0 ? dhi : dlo) : dw;
    load_to_lds16(lane_bytes | oob[i] | kflag, d, base[i] + koff,
                  lds_base + (uint32_t)(st * TILES * 1024) + (uint32_t)((NW * i + wave) * 1024));
  };

  // Register set b holds this wave's fragments of one k-tile: its row half's activation tiles of each
  // plane (fa) and its column half's weight tiles (fb).  Fragment f of a stage (activation tiles
  // first, then weight tiles) is one 16-byte LDS read per lane.
  constexpr int NF = NP * WM + WNT;
  uint4 fa[2][NP * WM], fb[2][WNT];
  auto read_frag = [&](int b, int st, int f) {
    const uint4 *sa = lds + (size_t)(st * TILES + wr * WM) * 64 + lane;
    const uint4 *sw = lds + (size_t)(st * TILES + AT + wc * WNT) * 64 + lane;
    if (f < NP * WM) fa[b][f] = sa[((f / WM) * BM + f % WM) * 64];
    else fb[b][f - NP * WM] = sw[(f - NP * WM) * 64];
  };

  f32x4 acc[WM][WNT];
#pragma unroll
  for (int m = 0; m < WM; ++m)
#pragma unroll
    for (int j = 0; j < WNT; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < R; ++st)
#pragma unroll
    for (int i = 0; i < G; ++i) issue(st, st, i);
  wait_loads_barrier<(R - 1) * G>();
#pragma unroll
  for (int f = 0; f < NF; ++f) read_frag(0, 0, f);
  // Two steps per trip (the register sets alternate; an odd k-tile count runs one step on zeros).  A
  // step runs row by row, each row's MFMAs in a scheduling region of their own together with a share
  // of the next k-tile's LDS reads and of the loads into the freed stage, so that both are issued
  // while the matrix cores work.
  constexpr int RF = (NF + WM - 1) / WM, RG = (G + WM - 1) / WM;  // reads, loads per row
  for (int k0 = 0; k0 < kt_count; k0 += 2) {
    int st = k0 % R;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int nst = st + 1 == R ? 0 : st + 1;
      wait_loads_barrier<(R - 2) * G>();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < WM; ++m) {
#pragma unroll
        for (int f = m * RF; f < (m + 1) * RF; ++f)
          if (f < NF) read_frag(b ^ 1, nst, f);
#pragma unroll
        for (int i = m * RG; i < (m + 1) * RG; ++i)
          if (i < G) issue(st, k0 + b + R, i);
#pragma unroll
        for (int j = 0; j < WNT; ++j) {
          if constexpr (NP > 1) acc[m][j] = mfma16(fa[b][WM + m], fb[b][j], acc[m][j]);  // the smaller part first
          acc[m][j] = mfma16(fa[b][m], fb[b][j], acc[m][j]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      st = nst;
    }
  }
  // the loads issued past the last k-tile (zeros) land before the block's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");

  // epilogue, one fully unrolled loop per kind (the accumulators stay in registers only if every index
  // is a constant)
  const float wunscale = weight_unscale(w_end);
  const int rq = (lane >> 4) * 4, cq = lane & 15;
  const int mw = mb0 + wr * WM, nw = nb0 + wc * WNT;
  if constexpr (ROPE) {
    static_assert(NW * (16 * (WNT * 16 + 4) + 2 * 64) * 4 <= R * TILES * 1024, "the waves' staging fits the LDS");
    static_assert(16 * (WNT * 16 + 4) + 2 * 64 >= WNT * 64 * 4, "a wave's share holds its blocks of one band");
    tile_rope_epilogue<WM, WNT>(lds, acc, wunscale, o, rows, n_blocks, mw, nw, wave, lane);
  } else if (o.kind == kSiluMul) {
#pragma unroll
    for (int m = 0; m < WM; ++m)
#pragma unroll
      for (int j = 0; j < WNT; j += 2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = (mw + m) * 16 + rq + e;
          if (r < rows && nw + j < n_blocks)
            epi_store(o, r, (nw + j) * 16 + cq, acc[m][j][e] * wunscale, acc[m][j + 1][e] * wunscale);
        }
  } else {
    const bool add = o.kind == kAccumulate;
#pragma unroll
    for (int m = 0; m < WM; ++m)
#pragma unroll
      for (int j = 0; j < WNT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = (mw + m) * 16 + rq + e;
          if (r < rows && nw + j < n_blocks) {
            float *p = o.f32 + (size_t)r * o.ld + (nw + j) * 16 + cq;
            const float v = acc[m][j][e] * wunscale;
            *p = add ? *p + v : v;
          }
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
  // for the consumers to add up (measured on the batch-1 7B layer: 124.7 -> 120.1 us).  At 32 rows the
  // middle width balances the two (7B layer at 32 sequences: 328 -> 317 us); at 64, 4 column waves win
  // (64-sequence 32-layer step: 11.06 ms against 11.23 with 2 and 12.40 with 1).
  const int order[3][3] = {{4, 2, 1}, {2, 4, 1}, {1, 2, 4}};
  for (int wn : order[rows <= 16 ? 2 : (rows <= 32 ? 1 : 0)]) {
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

// Prefill tile shape (WM row blocks x WNT column blocks per wave, 2 x WC waves per block).  Blocks with more
// than 80 KiB of LDS stages run one per CU, smaller ones two, so a launch runs in rounds of 256 or 512
// blocks; a round's time scales with the MFMAs a SIMD runs in it, and smaller tiles load more bytes per
// MFMA (relative speeds below are estimates, but for the measured two-per-CU 4 x 8).  Two blocks per CU
// also let one block's matrix cores run while the other waits at its barrier, and their rounds of 512
// cut the idle tail of a launch whose tile count is not a multiple of 256.  The shape with the least
// estimated time wins, larger tiles on ties.
struct TileChoice {
  int wm, wnt, pcu, tiles_m, tiles_n, wc = 2;  // wc: column waves (2, or 4: eight waves per block)
};
static TileChoice choose_tiles(int rows, int n_blocks, int planes) {
  // pcu 2: two blocks per CU, each with half the LDS (3 stages of 24 KiB); measured on the 7B gate/up
  // product (2048 rows, 1376 tiles of 4 x 8) at 0.95 of the 8 x 8 tiles' time for the same MFMAs per SIMD.
  // wc 4: eight waves of 4 x 4 on a 128 x 256 tile, or of 8 x 4 on a 256 x 256 one, two per SIMD, so one
  // wave's MFMAs run while the other waits; measured on the 7B o and down products (256 tiles at 2048
  // rows) at 0.9 of the four-wave 4 x 8 tile's time, and on gate/up (688 tiles of 256 x 256) at 0.96 of
  // the two-per-CU 4 x 8 tiles' time.
  static const struct {
    int wm, wnt, pcu, wc;
    double speed;
  } shapes[] = {{8, 8, 1, 2, 1.0},  {8, 6, 1, 2, 0.95}, {4, 8, 1, 2, 0.85}, {8, 4, 1, 2, 0.85},
                {4, 4, 1, 2, 0.7},  {4, 8, 2, 2, 1.05}, {4, 4, 1, 4, 0.95}, {8, 4, 1, 4, 1.1}};
  const int row_blocks = (rows + 15) / 16;
  TileChoice best{0, 0, 1, 0, 0};
  double best_cost = 1e300;
  for (const auto &sh : shapes) {
    // (as 512 tiles of 4 x 4 on the pair, the 7B k|v product measured 234 against 229 us for 256 of 8 x 8)
    if (sh.wc > 2 && planes > 1) continue;
    const double speed = sh.speed;
    const int bm = 2 * sh.wm, bn = sh.wc * sh.wnt;  // the block tile in 16-row / 16-column blocks
    const int tiles_kib = planes * bm + bn;
    const int stages = std::min(4, 160 / sh.pcu / tiles_kib);
    if (sh.pcu > 1 && stages < 3) continue;
    // blocks of at most 80 KiB run two per CU whatever their bounds say (4 x 4)
    const int per_cu = sh.pcu > 1 || stages * tiles_kib <= 80 ? 2 : 1;
    const int tm = (row_blocks + bm - 1) / bm, tn = (n_blocks + bn - 1) / bn;
    const long tiles = (long)tm * tn;
    // two blocks per CU only pay when the launch fills the second slots
    if (sh.pcu > 1 && tiles <= (long)kCUs) continue;
    // a round's time: the MFMAs of the waves a SIMD runs in it
    const double cost = (double)((tiles + per_cu * kCUs - 1) / (per_cu * kCUs)) * per_cu * (sh.wc / 2) * sh.wm *
                        sh.wnt / speed;
    if (cost < best_cost * 0.999) best_cost = cost, best = TileChoice{sh.wm, sh.wnt, sh.pcu, tm, tn, sh.wc};
  }
  return best;
}

template <int WM, int WNT, int NP, int PCU, int WC = 2>
static void launch_tile(hipStream_t s, const TileChoice &tc, const uint4 *act, const uint4 *lo, int a_kt,
                        int a_blocks, int rows, const uint4 *w, const uint4 *w_end, int kt_count, int n_blocks,
                        const LinearOut &o) {
  const int n_tiles = tc.tiles_m * tc.tiles_n;
  const int grid = (n_tiles + 7) / 8 * 8;
  constexpr int threads = 64 * 2 * WC;
  if (o.kind == kRope)
    tile_gemm_kernel<WM, WNT, NP, PCU, true, 2, WC><<<grid, threads, 0, s>>>(
        act, lo, a_kt, a_blocks, rows, w, w_end, kt_count, n_blocks, tc.tiles_m, n_tiles, o);
  else
    tile_gemm_kernel<WM, WNT, NP, PCU, false, 2, WC><<<grid, threads, 0, s>>>(
        act, lo, a_kt, a_blocks, rows, w, w_end, kt_count, n_blocks, tc.tiles_m, n_tiles, o);
}

template <int NP>
static void launch_tiles(const TileChoice &tc, hipStream_t s, const uint4 *act, const uint4 *lo, int a_kt,
                         int a_blocks, int rows, const uint4 *w, const uint4 *w_end, int kt_count, int n_blocks,
                         const LinearOut &o) {
#define LLMDEC_TILE(WM_, WNT_, PCU_) \
  launch_tile<WM_, WNT_, NP, PCU_>(s, tc, act, lo, a_kt, a_blocks, rows, w, w_end, kt_count, n_blocks, o)
  if (tc.wc == 4 && tc.wm == 8) {
    if constexpr (NP == 1) launch_tile<8, 4, 1, 1, 4>(s, tc, act, lo, a_kt, a_blocks, rows, w, w_end, kt_count, n_blocks, o);
  } else if (tc.wc == 4) {
    launch_tile<4, 4, NP, 1, 4>(s, tc, act, lo, a_kt, a_blocks, rows, w, w_end, kt_count, n_blocks, o);
  } else if (tc.pcu == 2) {
    if constexpr (NP == 1) LLMDEC_TILE(4, 8, 2);  // the only two-per-CU shape (3 stages fit one plane only)
  } else if (tc.wm == 8 && tc.wnt == 8) {
    LLMDEC_TILE(8, 8, 1);
  } else if (tc.wm == 8 && tc.wnt == 6) {
    LLMDEC_TILE(8, 6, 1);
  } else if (tc.wm == 4 && tc.wnt == 8) {
    LLMDEC_TILE(4, 8, 1);
  } else if (tc.wm == 8 && tc.wnt == 4) {
    LLMDEC_TILE(8, 4, 1);
  } else {
    LLMDEC_TILE(4, 4, 1);
  }
#undef LLMDEC_TILE
}

template <int MB, int NP>
static void launch_stream(int wn, int grid, hipStream_t s, const uint4 *act, const uint4 *lo, int a_kt, int rows,
                          const uint4 *w, const uint4 *w_end, int kt_count, int n_blocks, const LinearOut &o,
                          float *partials,
                          const Splits &sp) {
  if (wn == 4)
    stream_gemm_kernel<MB, 4, NP><<<grid, 256, 0, s>>>(act, lo, a_kt, rows, w, w_end, kt_count, n_blocks, o, partials,
                                                       sp);
  else if (wn == 2)
    stream_gemm_kernel<MB, 2, NP><<<grid, 256, 0, s>>>(act, lo, a_kt, rows, w, w_end, kt_count, n_blocks, o, partials,
                                                       sp);
  else
    stream_gemm_kernel<MB, 1, NP><<<grid, 256, 0, s>>>(act, lo, a_kt, rows, w, w_end, kt_count, n_blocks, o, partials,
                                                       sp);
}

// The product over n columns of the packed matrix (n_total columns) that start at column block nb0.
template <int NP>
static Splits launch_linear_np(const Act &a, const uint16_t *w_packed, int n_total, int nb0, int n, int k,
                               const LinearOut &o, float *partials, size_t partial_floats, SplitPolicy policy,
                               hipStream_t s) {
  const int kt_count = round_up(k, kTileK) / kTileK;
  const int n_blocks = n / 16;
  const uint4 *w = reinterpret_cast<const uint4 *>(w_packed) + (size_t)nb0 * kt_count * 64;
  const uint4 *w_end = reinterpret_cast<const uint4 *>(w_packed) + (size_t)(n_total / 16) * kt_count * 64;
  const uint4 *act = reinterpret_cast<const uint4 *>(a.a), *lo = reinterpret_cast<const uint4 *>(a.lo);
  const int a_kt = a.kpad / kTileK;
  if (a.rows <= 64) {
    StreamPlan p = stream_plan(a.rows, n, k, policy);
    if (p.sp.any() && (!partials || partial_floats < linear_partial_floats(a.rows, n, k, policy)))
      p = stream_plan(a.rows, n, k, kSplitNone);
    switch ((a.rows + 15) / 16) {
      case 1: launch_stream<1, NP>(p.wn, p.grid, s, act, lo, a_kt, a.rows, w, w_end, kt_count, n_blocks, o, partials, p.sp); break;
      case 2: launch_stream<2, NP>(p.wn, p.grid, s, act, lo, a_kt, a.rows, w, w_end, kt_count, n_blocks, o, partials, p.sp); break;
      case 3: launch_stream<3, NP>(p.wn, p.grid, s, act, lo, a_kt, a.rows, w, w_end, kt_count, n_blocks, o, partials, p.sp); break;
      default: launch_stream<4, NP>(p.wn, p.grid, s, act, lo, a_kt, a.rows, w, w_end, kt_count, n_blocks, o, partials, p.sp); break;
    }
    return p.sp;
  }
  // tile shape: the largest tiles that still give every CU work in whole rounds where possible
  const TileChoice tc = choose_tiles(a.rows, n_blocks, NP);
  launch_tiles<NP>(tc, s, act, lo, a_kt, a.row_blocks, a.rows, w, w_end, kt_count, n_blocks, o);
  return Splits{};
}

Splits launch_linear(const Act &a, const uint16_t *w_packed, int n, int k, const LinearOut &o, float *partials,
                     size_t partial_floats, SplitPolicy policy, hipStream_t s) {
  if (a.lo) return launch_linear_np<2>(a, w_packed, n, 0, n, k, o, partials, partial_floats, policy, s);
  return launch_linear_np<1>(a, w_packed, n, 0, n, k, o, partials, partial_floats, policy, s);
}

void launch_linear_cols(const Act &a, const uint16_t *w_packed, int n_total, int col0, int n, int k,
                        const LinearOut &o, hipStream_t s) {
  if (a.lo) launch_linear_np<2>(a, w_packed, n_total, col0 / 16, n, k, o, nullptr, 0, kSplitNone, s);
  else launch_linear_np<1>(a, w_packed, n_total, col0 / 16, n, k, o, nullptr, 0, kSplitNone, s);
}


}  // namespace llmdec
