// One-row weight products on the packed matrices: out[n] = sum_k x[k] * W[n][k] for a single
// token (decode of one sequence, "大模型推理全流程解析：从权重加载到文本生成的工程实践" §2.2.2: only
// the new token's projections are computed).
//
// With one row, every weight is used once, so the read of W bounds the product; the matrix cores would
// run 15 of 16 operand rows on padding.  Here a packed weight (fp16(w * 2^s), see weight_shift) becomes
// fp32 in one conversion and meets x in one fma; x stays fp32 (it is not rounded to fp16), staged in
// LDS, and the sum is multiplied by 2^-s at the end.
//
// The matrix is read in its packed tile layout (16 rows x 32 columns per 1 KiB tile, lane l holding
// row l%16, columns 8(l/16)..+7; a 16-row block's tiles contiguous along k).  A block owns TB whole
// row blocks (SwiGLU: a gate block and its up block) and its 8 waves split the k-tiles evenly; each
// wave streams its tiles through a ring of loads, and at the end the 4 lanes that share a row add
// their sums, the waves' sums meet in LDS in wave order, and the block applies the epilogue itself.
// No partial sums leave the block, so no reduction launch follows.  When the product follows an
// RMSNorm, the block stages rmsnorm(x) * gamma itself ("为什么要自己动手写一个LLM推理引擎" §4.2), so the
// norm needs no launch of its own either.
#include "common.h"
#include "internal.h"

namespace llmdec {

constexpr int kGvWaves = 8;         // waves per block, splitting the k-tiles
constexpr int kGvMaxK = 14336;      // x (fp32) in LDS
constexpr int kGvRope = 3;          // epilogue: RoPE and the paged K/V append of a q|k|v product

struct GemvArgs {
  const float *x;         // [k] fp32
  const uint16_t *gamma;  // NULL, or the RMSNorm gain [k]: the product reads rmsnorm(x) * gamma
  float eps;
  const uint16_t *w;      // packed matrix, n_blocks 16-row blocks of kt k-tiles
  int k, kt, n_blocks;
  float *out;
  RopeAppend ra;          // kGvRope only
};

__device__ inline float gv_silu(float g) { return g / (1.0f + expf(-g)); }

// TB row blocks per block: 1, or 2 for SwiGLU (blocks 2j = gate rows 16j.., 2j+1 = up rows 16j..).
// Three blocks per CU (6 waves per SIMD, at most 80 registers) keep a 7B matrix's 768 (q|k|v) or 688
// (gate/up) blocks resident in one round instead of a round and a half.
template <int MODE, int TB>
__global__ __launch_bounds__(kGvWaves * 64, 6) void gemv_kernel(GemvArgs a) {
  constexpr int D = TB == 1 ? 8 : 6;  // k-tile steps in flight per wave
  constexpr int R = D + 1;             // ring slots
  constexpr uint32_t kOut = 0x80000000u;
  extern __shared__ float smem[];
  const int k = a.k, kt = a.kt, kx = kt * 32;
  float *xs = smem;                     // [kx] fp32, zero past k
  float *part = smem + kx;              // [waves][TB][16]
  float *red = part + kGvWaves * TB * 16;  // [waves] norm sums

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb0 = blockIdx.x * TB;  // first row block of this block
  // this wave's k-tiles
  const int kt0 = wave * kt / kGvWaves, kt1 = (wave + 1) * kt / kGvWaves;
  const int n = kt1 - kt0;

  // one resource per row block: its tiles are contiguous; a step past the wave's range reads zeros
  const size_t blk_bytes = (size_t)kt * 1024;
  __amdgpu_buffer_rsrc_t rw[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) rw[t] = make_rsrc(a.w + (size_t)(nb0 + t) * kt * 512, blk_bytes);
  const uint32_t lane_bytes = (uint32_t)lane * 16u;

  uint4 wb[R][TB];
  auto issue = [&](int slot, int i) {
    const int t = kt0 + i;
    const uint32_t voff = i < n ? (uint32_t)t * 1024u + lane_bytes : kOut;
#pragma unroll
    for (int b = 0; b < TB; ++b) wb[slot][b] = buffer_load16(rw[b], voff, 0, kLoadStream);
  };
  // the weights do not depend on x: start them before x is staged
#pragma unroll
  for (int d = 0; d < D; ++d) {
    issue(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  // RoPE epilogue: the position, its page and the rotation depend only on the inputs, so the threads
  // that apply it (0..15) look them up now, while the weights stream
  int rp_page = -1, rp_off = 0;
  float rp_c = 1.f, rp_s = 0.f;
  if (MODE == kGvRope && threadIdx.x < 16) {
    const RopeAppend &ra = a.ra;
    const int n = nb0 * 16 + threadIdx.x, D = ra.head_dim;
    const int hidden = ra.n_heads * D, kvc = ra.n_kv_heads * D;
    const int pos = ra.pos[0];
    if (n < hidden + kvc) {
      const int dd = n < hidden ? n : n - hidden;
      rope_cos_sin(pos, ra.fr.inv_freq[(dd % D) >> 1], rp_c, rp_s);
    }
    if (n >= hidden) {
      const int blk = pos >> 4;
      rp_off = pos & 15;
      if (pos < 0 || blk >= ra.max_pages) {
        if (threadIdx.x == 0) raise_error(ra.err, kErrPos);
      } else {
        rp_page = ra.block_row[blk];
        if (rp_page < 0 || rp_page >= ra.num_pages) {
          if (threadIdx.x == 0) raise_error(ra.err, kErrPage);
          rp_page = -1;
        }
      }
    }
  }

  // stage x (or x * gamma, scaled by the norm's factor below): thread i takes columns 8i..8i+7
  float ss = 0.f;
  for (int i = threadIdx.x; i < kx / 8; i += blockDim.x) {
    const int c0 = 8 * i;
    float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
    if (c0 < k) {  // k % 16 == 0: 8 columns are all in or all out
      const float4 *p = reinterpret_cast<const float4 *>(a.x + c0);
      v0 = p[0];
      v1 = p[1];
      if (a.gamma) {
        const uint4 gw = *reinterpret_cast<const uint4 *>(a.gamma + c0);
        ss = fmaf(v0.x, v0.x, ss), ss = fmaf(v0.y, v0.y, ss), ss = fmaf(v0.z, v0.z, ss), ss = fmaf(v0.w, v0.w, ss);
        ss = fmaf(v1.x, v1.x, ss), ss = fmaf(v1.y, v1.y, ss), ss = fmaf(v1.z, v1.z, ss), ss = fmaf(v1.w, v1.w, ss);
        v0 = make_float4(v0.x * bf16lo(gw.x), v0.y * bf16hi(gw.x), v0.z * bf16lo(gw.y), v0.w * bf16hi(gw.y));
        v1 = make_float4(v1.x * bf16lo(gw.z), v1.y * bf16hi(gw.z), v1.z * bf16lo(gw.w), v1.w * bf16hi(gw.w));
      }
    }
    reinterpret_cast<float4 *>(xs)[2 * i] = v0;
    reinterpret_cast<float4 *>(xs)[2 * i + 1] = v1;
  }
  if (a.gamma) {  // block-uniform
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float total = 0.f;
    for (int w = 0; w < kGvWaves; ++w) total += red[w];
    const float inv = 1.0f / sqrtf(total / (float)k + a.eps);
    for (int i = threadIdx.x; i < kx / 8; i += blockDim.x) {  // the values this thread staged
      float4 *p = reinterpret_cast<float4 *>(xs) + 2 * i;
      const float4 v0 = p[0], v1 = p[1];
      p[0] = make_float4(v0.x * inv, v0.y * inv, v0.z * inv, v0.w * inv);
      p[1] = make_float4(v1.x * inv, v1.y * inv, v1.z * inv, v1.w * inv);
    }
  }
  __syncthreads();

  float acc[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) acc[b] = 0.f;
  const int xoff = (lane >> 4) * 8;  // the lane's 8 columns inside a k-tile
  auto compute = [&](int slot, int i) {
    const int t = min(kt0 + i, kt - 1);  // a step past the range multiplies zeros
    const float4 *xp = reinterpret_cast<const float4 *>(xs + t * 32 + xoff);
    const float4 x0 = xp[0], x1 = xp[1];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const uint4 w = wb[slot][b];
      float s = acc[b];
      s = fmaf(x0.x, f16lo(w.x), s);
      s = fmaf(x0.y, f16hi(w.x), s);
      s = fmaf(x0.z, f16lo(w.y), s);
      s = fmaf(x0.w, f16hi(w.y), s);
      s = fmaf(x1.x, f16lo(w.z), s);
      s = fmaf(x1.y, f16hi(w.z), s);
      s = fmaf(x1.z, f16lo(w.w), s);
      s = fmaf(x1.w, f16hi(w.w), s);
      acc[b] = s;
    }
  };
  for (int it = 0; it < n; it += R) {  // wave-uniform trip count; steps past n read and add nothing
#pragma unroll
    for (int d = 0; d < R; ++d) {
      issue((d + D) % R, it + d + D);
      compute(d, it + d);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the 4 lanes of a row (l, l+16, l+32, l+48) add their sums; lanes 0..15 hold the wave's 16 rows
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    float v = acc[b];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (lane < 16) part[(wave * TB + b) * 16 + lane] = v;
  }
  __syncthreads();
  if (threadIdx.x < 16) {  // row r of each of the block's row blocks
    const int r = threadIdx.x;
    const float unscale = weight_unscale(a.w + (size_t)a.n_blocks * kt * 512);
    float v[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      v[b] = 0.f;
      for (int w = 0; w < kGvWaves; ++w) v[b] += part[(w * TB + b) * 16 + r];
      v[b] *= unscale;
    }
    if (MODE == kSiluMul) {  // row block 0 holds the gate rows, row block 1 the matching up rows
      a.out[blockIdx.x * 16 + r] = gv_silu(v[0]) * v[TB - 1];
    } else if (MODE == kGvRope) {
      // column n of q|k|v; a rotation pair (2i, 2i+1) is two adjacent threads of this wave
      const RopeAppend &ra = a.ra;
      const int n = nb0 * 16 + r, D = ra.head_dim;
      const int hidden = ra.n_heads * D, kvc = ra.n_kv_heads * D;
      const float partner = __shfl_xor(v[0], 1, 64);
      const float xe = (r & 1) ? partner : v[0], xo = (r & 1) ? v[0] : partner;
      const int d = n < hidden ? n : (n < hidden + kvc ? n - hidden : n - hidden - kvc);
      const int h = d / D, i = (d % D) >> 1;
      const float c = rp_c, sn = rp_s;
      const float re = xe * c - xo * sn, ro = xe * sn + xo * c;  // the rotated pair
      if (n < hidden) {
        a.out[n] = (r & 1) ? ro : re;
      } else {
        const int page = rp_page, off = rp_off;
        if (page >= 0) {
          const size_t head = (size_t)page * ra.n_kv_heads + h;
          if (n < hidden + kvc) {
            if (!(r & 1))  // K [h][o][d]: the pair as one 32-bit store
              *reinterpret_cast<uint32_t *>(ra.pool_k + (head * 16 + off) * D + 2 * i) =
                  f32_to_bf16(re) | ((uint32_t)f32_to_bf16(ro) << 16);
          } else {  // V [h][o/4][d][o%4]
            ra.pool_v[(head * 4 + (off >> 2)) * D * 4 + (size_t)(d % D) * 4 + (off & 3)] = f32_to_bf16(v[0]);
          }
        }
      }
    } else {
      float *o = a.out + (size_t)nb0 * 16 + r;
      *o = MODE == kAccumulate ? *o + v[0] : v[0];
    }
  }
}

void launch_gemv_qkv_rope(const float *x, const uint16_t *gamma, float eps, const uint16_t *w_packed, int n, int k,
                          float *qkv, const RopeAppend &ra, hipStream_t s) {
  GemvArgs a;
  a.x = x, a.gamma = gamma, a.eps = eps, a.w = w_packed, a.out = qkv, a.ra = ra;
  a.k = k, a.kt = (k + 31) / 32, a.n_blocks = n / 16;
  if (a.n_blocks <= 0) return;
  const size_t lds = ((size_t)a.kt * 32 + kGvWaves * 16 + kGvWaves) * sizeof(float);
  gemv_kernel<kGvRope, 1><<<a.n_blocks, kGvWaves * 64, lds, s>>>(a);
}

bool gemv_shape_ok(int k) { return k > 0 && k % 16 == 0 && k <= kGvMaxK; }

void launch_gemv(const float *x, const uint16_t *gamma, float eps, const uint16_t *w_packed, int n, int k, int mode,
                 float *out, hipStream_t s) {
  GemvArgs a;
  a.x = x, a.gamma = gamma, a.eps = eps, a.w = w_packed, a.out = out;
  a.k = k, a.kt = (k + 31) / 32, a.n_blocks = n / 16;
  const int tb = mode == kSiluMul ? 2 : 1;
  const int blocks = a.n_blocks / tb;
  if (blocks <= 0) return;
  const size_t lds = ((size_t)a.kt * 32 + kGvWaves * tb * 16 + kGvWaves) * sizeof(float);
  if (mode == kSiluMul) gemv_kernel<kSiluMul, 2><<<blocks, kGvWaves * 64, lds, s>>>(a);
  else if (mode == kAccumulate) gemv_kernel<kAccumulate, 1><<<blocks, kGvWaves * 64, lds, s>>>(a);
  else gemv_kernel<kStore, 1><<<blocks, kGvWaves * 64, lds, s>>>(a);
}

}  // namespace llmdec
