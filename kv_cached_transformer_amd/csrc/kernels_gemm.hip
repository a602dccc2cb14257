// Weight-streaming linear layers: out[m][n] (+)= sum_k a[m][k] * W[n][k].
//
// W is bf16 in the packed tile layout (see packed_offset): each 16-row block
// is a run of 1 KiB tiles along k, so a wave streaming one block reads
// contiguous memory.  Three shapes:
//   * rows == 1 (batch-1 decode): a VALU GEMV with the activation kept in
//     fp32; HBM-bound on the weight stream.
//   * rows <= 64 (batched decode, short prompts): MFMA 16x16x32 bf16 with the
//     activation split into hi/lo bf16 halves (two MFMAs per tile), weights
//     read once; split over k across the waves of a block and, for narrow
//     matrices, across blocks (partials reduced by a second kernel).
//   * rows > 64 (prefill): MFMA tiles of 128 x 128 per block.
// The hi/lo split keeps the activation at ~16 significant bits: plain bf16
// activations put the layer output about 3x outside a 2e-2 max-abs bound at
// 7B sizes, while hi/lo stays about 5x inside it.
#include "common.h"
#include "internal.h"

namespace llmdec {

__device__ inline f32x4 mfma16(const uint4 &a, const uint4 &b, f32x4 c) {
  bf16x8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

__device__ inline float dot8(const uint4 &w, const float *x) {
  float s = bf16lo(w.x) * x[0];
  s = fmaf(bf16hi(w.x), x[1], s);
  s = fmaf(bf16lo(w.y), x[2], s);
  s = fmaf(bf16hi(w.y), x[3], s);
  s = fmaf(bf16lo(w.z), x[4], s);
  s = fmaf(bf16hi(w.z), x[5], s);
  s = fmaf(bf16lo(w.w), x[6], s);
  s = fmaf(bf16hi(w.w), x[7], s);
  return s;
}

// ---------------------------------------------------------------- GEMV (rows == 1)
// Block = one 16-row block of W, GEMV_WAVES waves splitting its tiles.  The
// fp32 activation is staged in LDS; lane l of a wave multiplies its 8 weights
// of row l%16 by x[32kt + 8(l/16) .. +7].
constexpr int GEMV_WAVES = 8;
constexpr int GEMV_UNROLL = 8;

__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_kernel(const float *__restrict__ x, int k, int kt_count,
                                                               const uint4 *__restrict__ w, float *__restrict__ out,
                                                               int epi) {
  extern __shared__ float smem[];
  float *xs = smem;                          // [kt_count * 32]
  float *red = smem + kt_count * 32;         // [GEMV_WAVES][16]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kt_count * 32; i += 64 * GEMV_WAVES) xs[i] = i < k ? x[i] : 0.f;
  __syncthreads();
  const uint4 *wb = w + (size_t)blockIdx.x * kt_count * 64 + lane;
  const float *xl = xs + (lane >> 4) * 8;
  float acc = 0.f;
  int kt = wave;
  for (; kt + (GEMV_UNROLL - 1) * GEMV_WAVES < kt_count; kt += GEMV_UNROLL * GEMV_WAVES) {
    uint4 t[GEMV_UNROLL];
#pragma unroll
    for (int u = 0; u < GEMV_UNROLL; ++u) t[u] = load_stream(wb + (size_t)(kt + u * GEMV_WAVES) * 64);
#pragma unroll
    for (int u = 0; u < GEMV_UNROLL; ++u) acc += dot8(t[u], xl + (kt + u * GEMV_WAVES) * 32);
  }
  for (; kt < kt_count; kt += GEMV_WAVES) acc += dot8(load_stream(wb + (size_t)kt * 64), xl + kt * 32);
  acc += __shfl_xor(acc, 16, 64);
  acc += __shfl_xor(acc, 32, 64);
  if (lane < 16) red[wave * 16 + lane] = acc;
  __syncthreads();
  if (tid < 16) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < GEMV_WAVES; ++i) s += red[i * 16 + tid];
    float *o = out + (size_t)blockIdx.x * 16 + tid;
    *o = epi == kAccumulate ? *o + s : s;
  }
}

// ---------------------------------------------------------------- skinny MFMA (rows <= 64)
// Block = 64 output columns (4 row-blocks of W) x one k-range; its 4 waves
// interleave over the k-tiles of that range, each wave holding all MB x 4
// accumulators; the waves are summed through LDS.  With ksplit > 1 the
// block writes a partial sum and reduce_kernel applies the epilogue.
template <int MB>
__global__ __launch_bounds__(256) void skinny_kernel(const uint4 *__restrict__ a_hi, const uint4 *__restrict__ a_lo,
                                                     int a_kt, int rows, const uint4 *__restrict__ w, int kt_count,
                                                     int n, float *__restrict__ out, int ld_out, int epi,
                                                     float *__restrict__ partials) {
  __shared__ float red[3][MB * 16][64 + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 64;  // first output column
  const int ks = blockIdx.y, nks = gridDim.y;
  const int kt0 = (int)((long)kt_count * ks / nks), kt1 = (int)((long)kt_count * (ks + 1) / nks);
  f32x4 acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nb0 = n0 >> 4;
  const int nbs = min(4, (n - n0) >> 4);
  for (int kt = kt0 + wave; kt < kt1; kt += 4) {
    uint4 wt[4], ah[MB], al[MB];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wt[j] = j < nbs ? load_stream(w + ((size_t)(nb0 + j) * kt_count + kt) * 64 + lane) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      ah[i] = a_hi[((size_t)i * a_kt + kt) * 64 + lane];
      al[i] = a_lo[((size_t)i * a_kt + kt) * 64 + lane];
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = mfma16(ah[i], wt[j], acc[i][j]);
        acc[i][j] = mfma16(al[i], wt[j], acc[i][j]);
      }
  }
  // C layout: lane l, element e holds row 4*(l/16)+e, column l%16 of each 16x16 block.
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave - 1][i * 16 + (lane >> 4) * 4 + e][j * 16 + (lane & 15)] = acc[i][j][e];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = i * 16 + (lane >> 4) * 4 + e, c = j * 16 + (lane & 15);
          const float v = acc[i][j][e] + red[0][r][c] + red[1][r][c] + red[2][r][c];
          if (r < rows && j < nbs) {
            if (partials) {
              partials[((size_t)ks * rows + r) * n + n0 + c] = v;
            } else {
              float *o = out + (size_t)r * ld_out + n0 + c;
              *o = epi == kAccumulate ? *o + v : v;
            }
          }
        }
  }
}

__global__ void reduce_kernel(const float *__restrict__ partials, int ksplit, int rows, int n, float *__restrict__ out,
                              int ld_out, int epi) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)rows * n) return;
  const int r = (int)(idx / n), c = (int)(idx % n);
  float s = 0.f;
  for (int k = 0; k < ksplit; ++k) s += partials[((size_t)k * rows + r) * n + c];
  float *o = out + (size_t)r * ld_out + c;
  *o = epi == kAccumulate ? *o + s : s;
}

// ---------------------------------------------------------------- tiled MFMA (rows > 64)
// Block = 128 x 128 outputs, 4 waves in 2 x 2, each wave 64 x 64 (4 x 4 MFMA blocks).
__global__ __launch_bounds__(256) void tiled_kernel(const uint4 *__restrict__ a_hi, const uint4 *__restrict__ a_lo,
                                                    int a_kt, int rows, const uint4 *__restrict__ w, int kt_count,
                                                    int n, float *__restrict__ out, int ld_out, int epi) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mb0 = blockIdx.y * 8 + (wave >> 1) * 4;  // first 16-row block of activations
  const int nb0 = blockIdx.x * 8 + (wave & 1) * 4;   // first 16-row block of W
  const int m_blocks = (rows + 15) >> 4, n_blocks = n >> 4;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kt = 0; kt < kt_count; ++kt) {
    uint4 wt[4], ah[4], al[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wt[j] = (nb0 + j < n_blocks) ? w[((size_t)(nb0 + j) * kt_count + kt) * 64 + lane] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = mb0 + i < m_blocks;
      ah[i] = ok ? a_hi[((size_t)(mb0 + i) * a_kt + kt) * 64 + lane] : make_uint4(0, 0, 0, 0);
      al[i] = ok ? a_lo[((size_t)(mb0 + i) * a_kt + kt) * 64 + lane] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = mfma16(ah[i], wt[j], acc[i][j]);
        acc[i][j] = mfma16(al[i], wt[j], acc[i][j]);
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = (mb0 + i) * 16 + (lane >> 4) * 4 + e, c = (nb0 + j) * 16 + (lane & 15);
        if (r < rows && nb0 + j < n_blocks) {
          float *o = out + (size_t)r * ld_out + c;
          *o = epi == kAccumulate ? *o + acc[i][j][e] : acc[i][j][e];
        }
      }
}

// ---------------------------------------------------------------- dispatch
static int skinny_ksplit(int n, int kt_count) {
  const int col_blocks = (n + 63) / 64;
  int ks = 1;
  while (col_blocks * ks < 512 && kt_count / (ks * 2) >= 8) ks *= 2;
  return ks;
}

size_t linear_partial_floats(int rows, int n, int k) {
  if (rows <= 1 || rows > 64) return 0;
  const int ks = skinny_ksplit(n, round_up(k, kTileK) / kTileK);
  return ks > 1 ? (size_t)ks * rows * n : 0;
}

void launch_linear(const Act &a, const uint16_t *w_packed, int n, int k, float *out, int ld_out, Epilogue epi,
                   float *partials, size_t partial_floats, hipStream_t s) {
  const int kt_count = round_up(k, kTileK) / kTileK;
  const uint4 *w = reinterpret_cast<const uint4 *>(w_packed);
  if (a.rows == 1 && a.f32) {
    static bool lds_raised = false;  // allow K up to 16384 (64 KiB of fp32 activation in LDS)
    if (!lds_raised) {
      (void)hipFuncSetAttribute((const void *)gemv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
      lds_raised = true;
    }
    const size_t lds = ((size_t)kt_count * 32 + GEMV_WAVES * 16) * sizeof(float);
    gemv_kernel<<<n / 16, 64 * GEMV_WAVES, lds, s>>>(a.f32, k, kt_count, w, out, epi);
    return;
  }
  const uint4 *ah = reinterpret_cast<const uint4 *>(a.hi), *al = reinterpret_cast<const uint4 *>(a.lo);
  const int a_kt = a.kpad / kTileK;
  if (a.rows <= 64) {
    int ks = skinny_ksplit(n, kt_count);
    if (ks > 1 && (!partials || partial_floats < (size_t)ks * a.rows * n)) ks = 1;
    dim3 grid((n + 63) / 64, ks);
    float *p = ks > 1 ? partials : nullptr;
    switch ((a.rows + 15) / 16) {
      case 1: skinny_kernel<1><<<grid, 256, 0, s>>>(ah, al, a_kt, a.rows, w, kt_count, n, out, ld_out, epi, p); break;
      case 2: skinny_kernel<2><<<grid, 256, 0, s>>>(ah, al, a_kt, a.rows, w, kt_count, n, out, ld_out, epi, p); break;
      case 3: skinny_kernel<3><<<grid, 256, 0, s>>>(ah, al, a_kt, a.rows, w, kt_count, n, out, ld_out, epi, p); break;
      default: skinny_kernel<4><<<grid, 256, 0, s>>>(ah, al, a_kt, a.rows, w, kt_count, n, out, ld_out, epi, p); break;
    }
    if (ks > 1) {
      const size_t total = (size_t)a.rows * n;
      reduce_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(partials, ks, a.rows, n, out, ld_out, epi);
    }
    return;
  }
  dim3 grid((n + 127) / 128, (a.rows + 127) / 128);
  tiled_kernel<<<grid, 256, 0, s>>>(ah, al, a_kt, a.rows, w, kt_count, n, out, ld_out, epi);
}

}  // namespace llmdec
