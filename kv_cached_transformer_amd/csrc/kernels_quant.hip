// Group-quantized weight products for single-token decode: out[n] = sum_k x[k] * W[n][k] with
// W[n][k] = (codes[n][k] - zero[n][g]) * scale[n][g], g = k / 128 ("企业官网建设流程全解析" §4.2:
// integer weights, int8 or int4, in groups of 128 elements, one scale and one zero point per group,
// turned back into floating point before the product).  Codes are 8-bit, or 4-bit two to a byte
// (the low nibble is the even column).
//
// One row of activations makes this a matrix-vector product: every code is used once, so the
// kernel is bound by the HBM read of the codes (1 or 1/2 byte per weight, plus 4 bytes of scale and
// zero point per group of 128).  No matrix cores: a code becomes fp32 in one conversion (4-bit codes
// are first spread to bytes by two masks per 8 codes) and meets its activation in one fma, and the
// zero point and scale are applied once per lane chunk:
//   sum_k x_k (c_k - z) s = s * (sum_k x_k c_k - z * sum_k x_k)
// over the columns a lane's 16-byte chunk holds (16 or 32; they always lie in one group), with the
// chunk sums of x formed once per block.
//
// Work: a wave owns four output rows and streams them over the whole k range, one 16-byte chunk per
// lane per row per step (a step covers 1024 columns with 8-bit codes, 2048 with 4-bit), with the
// steps of a row kept in flight ahead of the arithmetic.  x lives in LDS as fp32, stored by
// quarter-chunks (float4 j of chunk c at [j][c]) so that the lanes of one ds_read_b128 read
// consecutive 16-byte words.  When the product follows an RMSNorm, each block stages
// rmsnorm(x) * gamma itself ("为什么要自己动手写一个LLM推理引擎" §4.2: x (mean(x^2) + eps)^-1/2 gamma),
// so the norm costs no launch of its own.
//
// Packed layout of a quantized matrix (llmdec_q8_pack_matrix, llmdec_q4_pack_matrix): the codes,
// [rows][row_bytes] (8-bit: row_bytes = cols; 4-bit: the row's cols/2 bytes padded with zero codes to
// a multiple of 16), followed by the group metadata, one 32-bit word per (row, group): bf16 scale bits
// in the high half, zero point in the low byte.  Within a row the words are ordered for the lanes:
// for steps 4t..4t+3, the lanes that share a group in every step (8 of them with 8-bit codes, 4 with
// 4-bit) find their four words (one per step) as one 16-byte run, so one load every four steps
// brings a lane all the metadata it needs.  Rows are padded with zero words (scale 0).
#include "common.h"
#include "internal.h"

namespace llmdec {

constexpr int kQGroup = 128;       // elements per quantization group
constexpr int kQMaxK = 14336;      // x (fp32), its chunk sums and the norm's sums fit 64 KiB of LDS

// Geometry for codes of BITS bits: columns per 16-byte lane chunk, per wave step, groups per step,
// lanes per group, metadata bytes per four steps.
template <int BITS> struct QGeom {
  static constexpr int CPL = 128 / BITS;
  static constexpr int STEP = 64 * CPL;
  static constexpr int GPS = STEP / kQGroup;
  static constexpr int LPG = 64 / GPS;
  static constexpr int QUAD = GPS * 16;
};

__host__ __device__ inline int q_steps(int bits, int k) { return (k + 64 * (128 / bits) - 1) / (64 * (128 / bits)); }
__host__ __device__ inline size_t q_row_bytes(int bits, int k) {
  return bits == 8 ? (size_t)k : (size_t)(k + 31) / 32 * 16;
}
// bytes of metadata per row: one quad (16 bytes per lane group) per four steps
__host__ __device__ inline size_t q_meta_row_bytes(int bits, int k) {
  return (size_t)((q_steps(bits, k) + 3) / 4) * (64 * (128 / bits) / kQGroup) * 16;
}

size_t q_matrix_bytes(int bits, int rows, int cols) {
  return (size_t)rows * q_row_bytes(bits, cols) + (size_t)rows * q_meta_row_bytes(bits, cols);
}

// ---------------------------------------------------------------- packing
// One block per source row: copy the row's codes to row dst_row0 + r of the destination (4-bit rows
// padded with zero bytes), and write its metadata words in lane order.  cols % 16 == 0.
template <int BITS>
__global__ void q_pack_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                              const uint8_t *__restrict__ zeros, int cols, uint8_t *__restrict__ dst, int dst_rows,
                              int dst_row0) {
  using G = QGeom<BITS>;
  const int r = blockIdx.x;
  const int groups = (cols + kQGroup - 1) / kQGroup;
  const size_t src_bytes = BITS == 8 ? (size_t)cols : (size_t)cols / 2;  // cols % 16 == 0: whole bytes
  const size_t rb = q_row_bytes(BITS, cols);
  const uint8_t *src = codes + (size_t)r * src_bytes;
  uint8_t *out = dst + (size_t)(dst_row0 + r) * rb;
  for (size_t i = threadIdx.x; i < rb; i += blockDim.x) out[i] = i < src_bytes ? src[i] : 0;
  const int nq = (q_steps(BITS, cols) + 3) / 4;
  const int words = nq * G::GPS * 4;
  uint32_t *meta = reinterpret_cast<uint32_t *>(dst + (size_t)dst_rows * rb +
                                                (size_t)(dst_row0 + r) * q_meta_row_bytes(BITS, cols));
  for (int w = threadIdx.x; w < words; w += blockDim.x) {
    const int t = w / (G::GPS * 4), h = (w / 4) % G::GPS, i = w % 4;
    const int g = G::GPS * (4 * t + i) + h;  // step 4t+i, lane group h
    uint32_t v = 0;
    if (g < groups) v = ((uint32_t)scales[(size_t)r * groups + g] << 16) | zeros[(size_t)r * groups + g];
    meta[w] = v;
  }
}

void launch_q_pack(int bits, const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros, int rows, int cols,
                   uint8_t *dst, int dst_rows, int dst_row0, hipStream_t s) {
  if (rows <= 0) return;
  if (bits == 4) q_pack_kernel<4><<<rows, 256, 0, s>>>(codes, scales, zeros, cols, dst, dst_rows, dst_row0);
  else q_pack_kernel<8><<<rows, 256, 0, s>>>(codes, scales, zeros, cols, dst, dst_rows, dst_row0);
}

// ---------------------------------------------------------------- matrix-vector product
// Output modes: kStore out[n] = v; kAccumulate out[n] += v (the residual stream); kSiluMul: the
// matrix is [gate; up] (2 n_out rows), a wave owns gate rows 2t, 2t+1 and up rows 2t, 2t+1, and
// writes out[n] = silu(gate_n) * up_n.
struct Q8Args {
  const float *x;         // [k] fp32
  const uint16_t *gamma;  // NULL, or the RMSNorm gain [k] (bf16): the product then reads rmsnorm(x) * gamma
  float eps;
  const uint8_t *w;       // packed matrix (codes, then metadata)
  int rows;               // rows of the packed matrix
  int k;
  int n_tasks;            // waves with work: rows / 4
  int n_out;              // SwiGLU: rows / 2
  float *out;
};

__device__ inline float q8_silu(float g) { return g / (1.0f + expf(-g)); }

// Steps of a row kept in flight ahead of the arithmetic.
template <int NSTEP> struct Q8Ring {
  static constexpr int D = NSTEP < 6 ? NSTEP : 6;
};

template <int BITS, int NSTEP, int MODE>
__global__ __launch_bounds__(512) void q_gemv_kernel(Q8Args a) {
  using G = QGeom<BITS>;
  constexpr int CPL = G::CPL, NJ = CPL / 4;  // columns and float4 quarters per lane chunk
  constexpr int NCH = NSTEP * 64;           // lane chunks of x held in LDS (columns past k are zero)
  constexpr int D = Q8Ring<NSTEP>::D;
  constexpr int NQ = (NSTEP + 3) / 4;
  extern __shared__ float4 smem[];
  float4 *xq = smem;                                           // [NJ][NCH]: quarter j of chunk c
  float *xsum = reinterpret_cast<float *>(smem + NJ * NCH);   // [NCH]: sum of the chunk's values
  float *red = xsum + NCH;                                     // [waves]: the norm's sums of squares

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int task = blockIdx.x * (blockDim.x >> 6) + wave;
  const bool active = task < a.n_tasks;  // wave-uniform
  const int k = a.k;

  // the wave's four rows (scalar)
  int row[4];
  if (MODE == kSiluMul) {
    row[0] = 2 * task, row[1] = 2 * task + 1, row[2] = a.n_out + 2 * task, row[3] = a.n_out + 2 * task + 1;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) row[r] = 4 * task + r;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) row[r] = active ? row[r] : 0;

  // Codes: one resource over the whole matrix; a lane past the row's end gets an offset past the
  // resource (reads zeros, touches nothing), so every load is unconditional.
  const uint32_t rb = (uint32_t)q_row_bytes(BITS, k);
  const size_t code_bytes = (size_t)a.rows * rb;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.w, code_bytes);
  const uint32_t mrow = (uint32_t)q_meta_row_bytes(BITS, k);
  const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.w + code_bytes, (size_t)a.rows * mrow);

  uint4 cb[NSTEP][4];  // fully unrolled: only D steps are live at a time
  uint4 mb[NQ][4];
  auto issue = [&](int s) {
    const int col = s * G::STEP + lane * CPL;
    const uint32_t voff = col < k ? (uint32_t)(s * 1024 + lane * 16) : 0x80000000u;  // 1 KiB of a row per step
    if (s % 4 == 0) {
      const uint32_t moff = (uint32_t)(s / 4) * G::QUAD + (uint32_t)(lane / G::LPG) * 16u;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mb[s / 4][r] = buffer_load16(rm, moff, __builtin_amdgcn_readfirstlane((uint32_t)row[r] * mrow), 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      cb[s][r] = buffer_load16(rc, voff, __builtin_amdgcn_readfirstlane((uint32_t)row[r] * rb), kLoadStream);
  };
  // the codes do not depend on x: start them before x is staged (an idle wave issues nothing)
  if (active) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      issue(s);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // stage x (or rmsnorm(x) * gamma): thread i takes columns 8i..8i+7 (two quarters of a chunk)
  float ss = 0.f;
  for (int i = threadIdx.x; i < NCH * NJ / 2; i += blockDim.x) {
    const int c0 = 8 * i;
    float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
    if (c0 < k) {  // k % 16 == 0, so 8 columns are either all in or all out
      const float4 *p = reinterpret_cast<const float4 *>(a.x + c0);
      v0 = p[0];
      v1 = p[1];
      if (a.gamma) {  // block-uniform: stage x * gamma now, scale by the norm's factor once it is known
        const uint4 gw = *reinterpret_cast<const uint4 *>(a.gamma + c0);
        ss = fmaf(v0.x, v0.x, ss), ss = fmaf(v0.y, v0.y, ss), ss = fmaf(v0.z, v0.z, ss), ss = fmaf(v0.w, v0.w, ss);
        ss = fmaf(v1.x, v1.x, ss), ss = fmaf(v1.y, v1.y, ss), ss = fmaf(v1.z, v1.z, ss), ss = fmaf(v1.w, v1.w, ss);
        v0 = make_float4(v0.x * bf16lo(gw.x), v0.y * bf16hi(gw.x), v0.z * bf16lo(gw.y), v0.w * bf16hi(gw.y));
        v1 = make_float4(v1.x * bf16lo(gw.z), v1.y * bf16hi(gw.z), v1.z * bf16lo(gw.w), v1.w * bf16hi(gw.w));
      }
    }
    const int ch = c0 / CPL, j = (c0 % CPL) / 4;  // j is even
    xq[j * NCH + ch] = v0;
    xq[(j + 1) * NCH + ch] = v1;
  }
  if (a.gamma) {  // block-uniform
    const int nw = blockDim.x >> 6;
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float total = 0.f;
    for (int w = 0; w < nw; ++w) total += red[w];
    const float inv = 1.0f / sqrtf(total / (float)k + a.eps);
    for (int i = threadIdx.x; i < NCH * NJ / 2; i += blockDim.x) {  // the values this thread staged
      const int c0 = 8 * i;
      if (c0 >= k) continue;
      const int ch = c0 / CPL, j = (c0 % CPL) / 4;
      const float4 v0 = xq[j * NCH + ch], v1 = xq[(j + 1) * NCH + ch];
      xq[j * NCH + ch] = make_float4(v0.x * inv, v0.y * inv, v0.z * inv, v0.w * inv);
      xq[(j + 1) * NCH + ch] = make_float4(v1.x * inv, v1.y * inv, v1.z * inv, v1.w * inv);
    }
  }
  __syncthreads();
  for (int ch = threadIdx.x; ch < NCH; ch += blockDim.x) {
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float4 v = xq[j * NCH + ch];
      t += v.x + v.y + v.z + v.w;
    }
    xsum[ch] = t;
  }
  __syncthreads();
  if (!active) return;  // no barrier follows

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    if (s + D < NSTEP) issue(s + D);
    __builtin_amdgcn_sched_barrier(0);
    const int ch = s * 64 + lane;
    float xv[CPL];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float4 v = xq[j * NCH + ch];
      xv[4 * j] = v.x, xv[4 * j + 1] = v.y, xv[4 * j + 2] = v.z, xv[4 * j + 3] = v.w;
    }
    const float xs = xsum[ch];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t cw[4] = {cb[s][r].x, cb[s][r].y, cb[s][r].z, cb[s][r].w};
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (BITS == 8) {  // bytes 0..3 of word j: columns 4j..4j+3
          d = fmaf(xv[4 * j], (float)(cw[j] & 0xffu), d);
          d = fmaf(xv[4 * j + 1], (float)((cw[j] >> 8) & 0xffu), d);
          d = fmaf(xv[4 * j + 2], (float)((cw[j] >> 16) & 0xffu), d);
          d = fmaf(xv[4 * j + 3], (float)(cw[j] >> 24), d);
        } else {  // byte b of word j holds columns 8j+2b (low nibble) and 8j+2b+1 (high nibble)
          const uint32_t lo = cw[j] & 0x0f0f0f0fu, hi = (cw[j] >> 4) & 0x0f0f0f0fu;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            d = fmaf(xv[8 * j + 2 * b], (float)((lo >> (8 * b)) & 0xffu), d);
            d = fmaf(xv[8 * j + 2 * b + 1], (float)((hi >> (8 * b)) & 0xffu), d);
          }
        }
      }
      const uint4 mq = mb[s / 4][r];
      const uint32_t m = (s & 3) == 0 ? mq.x : (s & 3) == 1 ? mq.y : (s & 3) == 2 ? mq.z : mq.w;
      const float scale = __uint_as_float(m & 0xffff0000u), zero = (float)(m & 0xffu);
      acc[r] = fmaf(scale, fmaf(-zero, xs, d), acc[r]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
    if (MODE == kSiluMul) {
      *reinterpret_cast<float2 *>(a.out + 2 * task) =
          make_float2(q8_silu(acc[0]) * acc[2], q8_silu(acc[1]) * acc[3]);
    } else {
      float4 *o = reinterpret_cast<float4 *>(a.out + 4 * task);
      float4 v = make_float4(acc[0], acc[1], acc[2], acc[3]);
      if (MODE == kAccumulate) vadd(v, *o);
      *o = v;
    }
  }
}

template <int BITS, int MODE> static void q_dispatch(int nstep, const Q8Args &a, int wpb, hipStream_t s) {
  const size_t lds = (size_t)nstep * 64 * ((128 / BITS / 4) * sizeof(float4) + sizeof(float)) + 16 * sizeof(float);
  const int blocks = (a.n_tasks + wpb - 1) / wpb;
  switch (nstep) {
#define Q_CASE(N) \
  case N: q_gemv_kernel<BITS, N, MODE><<<blocks, wpb * 64, lds, s>>>(a); break;
    Q_CASE(1) Q_CASE(2) Q_CASE(3) Q_CASE(4) Q_CASE(5) Q_CASE(6) Q_CASE(7)
#undef Q_CASE
    default:
      if constexpr (BITS == 8) {
        switch (nstep) {
#define Q_CASE8(N) \
  case N: q_gemv_kernel<8, N, MODE><<<blocks, wpb * 64, lds, s>>>(a); break;
          Q_CASE8(8) Q_CASE8(9) Q_CASE8(10) Q_CASE8(11) Q_CASE8(12) Q_CASE8(13) Q_CASE8(14)
#undef Q_CASE8
          default: break;
        }
      }
      break;
  }
}

bool q_shape_ok(int bits, int k) { return (bits == 8 || bits == 4) && k > 0 && k % 16 == 0 && k <= kQMaxK; }

void launch_q_gemv(int bits, const float *x, const uint16_t *gamma, float eps, const uint8_t *w, int rows, int k,
                   int mode, float *out, hipStream_t s) {
  Q8Args a;
  a.x = x, a.gamma = gamma, a.eps = eps, a.w = w, a.rows = rows, a.k = k, a.out = out;
  a.n_out = mode == kSiluMul ? rows / 2 : rows;
  a.n_tasks = rows / 4;  // four matrix rows per wave in every mode
  if (a.n_tasks <= 0) return;
  const int nstep = q_steps(bits, k);
  // 8 waves per block share one staging of x, unless that would leave CUs without two blocks each
  const int wpb = a.n_tasks >= 8 * 512 ? 8 : 4;
  if (bits == 4) {
    if (mode == kSiluMul) q_dispatch<4, kSiluMul>(nstep, a, wpb, s);
    else if (mode == kAccumulate) q_dispatch<4, kAccumulate>(nstep, a, wpb, s);
    else q_dispatch<4, kStore>(nstep, a, wpb, s);
  } else {
    if (mode == kSiluMul) q_dispatch<8, kSiluMul>(nstep, a, wpb, s);
    else if (mode == kAccumulate) q_dispatch<8, kAccumulate>(nstep, a, wpb, s);
    else q_dispatch<8, kStore>(nstep, a, wpb, s);
  }
}

}  // namespace llmdec
