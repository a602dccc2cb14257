// Shared helpers for the libllmdec kernels and host code (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "host.h"
#include "llmdec.h"

namespace llmdec {

constexpr int kTileRows = 16;   // packed-matrix tile: 16 rows ...
constexpr int kTileK = 32;      // ... x 32 columns = one 16x16x32 MFMA operand
constexpr int kTileElems = 512; // bf16 elements per tile (1 KiB)

// Device error bits (sticky word at the start of every workspace).
constexpr uint32_t kErrPage = 1u;   // block-table page id out of range
constexpr uint32_t kErrPos = 2u;    // position beyond the block-table row
constexpr uint32_t kErrToken = 4u;  // token id out of range
constexpr uint32_t kErrSeq = 8u;    // sequence index, cu_seqlens entry or position out of range
constexpr size_t kWsHeader = 256;   // bytes reserved for the error word

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load (weights and cache pages are read once per step).
__device__ inline uint4 load_stream(const uint4 *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw buffer access: a scalar resource (base, byte size) plus a per-lane and a
// scalar byte offset.  A load at or past the size reads zeros and touches no
// memory, so an empty resource turns a load off without a branch.
constexpr int kLoadStream = 2;  // cache policy: non-temporal (read once)
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, size_t bytes) {
  const int n = bytes >= 0xffffffffull ? (int)0xffffffffu : (int)(uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
__device__ inline uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, int policy) {
  u32x4 v;
  if (policy == kLoadStream) v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kLoadStream);
  else v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 8-byte streaming (non-temporal) load.
__device__ inline uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kLoadStream);
  return make_uint2(v[0], v[1]);
}

// acc += p[0] + p[stride] + ... + p[(ks-1)*stride], added in that order (the result does not depend
// on the batching).  Loads leave 8 at a time, so a long list of split-k partials costs a few memory
// round trips rather than one per split.
__device__ inline void vadd(float4 &a, const float4 &b) { a.x += b.x, a.y += b.y, a.z += b.z, a.w += b.w; }
__device__ inline void vadd(float2 &a, const float2 &b) { a.x += b.x, a.y += b.y; }
template <typename V>
__device__ inline void add_splits(V &acc, const float *p, size_t stride, int ks) {
  for (int q = 0; q < ks; q += 8) {
    V v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (q + j < ks) v[j] = *reinterpret_cast<const V *>(p + (size_t)(q + j) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (q + j < ks) vadd(acc, v[j]);
  }
}
// N independent sums at once (acc[i] += the partials at p[i]): every batch issues the loads of all N
// before the first add, so N sums cost the memory round trips of one.  Each sum is added in plane order,
// exactly as add_splits adds it.
template <int N, typename V>
__device__ inline void add_splits_n(V (&acc)[N], const float *const (&p)[N], size_t stride, const int (&ks)[N]) {
  constexpr int B = N <= 2 ? 16 : 8;  // planes per batch
  int kmax = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) kmax = ks[i] > kmax ? ks[i] : kmax;
  for (int q = 0; q < kmax; q += B) {
    V v[N][B];
#pragma unroll
    for (int j = 0; j < B; ++j)
#pragma unroll
      for (int i = 0; i < N; ++i)
        if (q + j < ks[i]) v[i][j] = *reinterpret_cast<const V *>(p[i] + (size_t)(q + j) * stride);
#pragma unroll
    for (int j = 0; j < B; ++j)
#pragma unroll
      for (int i = 0; i < N; ++i)
        if (q + j < ks[i]) vadd(acc[i], v[i][j]);
  }
}

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }
__host__ __device__ inline size_t round_up_sz(size_t x, size_t m) { return (x + m - 1) / m * m; }

// Element offset of (row, col) inside a packed matrix with kt_count tiles per
// 16-row block.  Tile (nb, kt) holds rows 16nb..16nb+15 and columns
// 32kt..32kt+31; inside it, lane l (0..63) owns 8 consecutive elements: row
// l%16, columns 8*(l/16)..8*(l/16)+7.  That is exactly the operand a wave feeds
// one 16x16x32 bf16 MFMA, so a wave loads a whole tile as one contiguous 1 KiB.
__host__ __device__ inline size_t packed_offset(int row, int col, int kt_count) {
  const int nb = row >> 4, kt = col >> 5;
  const int lane = (row & 15) | (((col >> 3) & 3) << 4);
  return ((((size_t)nb * kt_count + kt) << 6) + lane) * 8 + (col & 7);
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ inline float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest bf16, ties to even (inputs are finite here).
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// hi = bf16(x), lo = bf16(x - hi): x == hi + lo to about 2^-17 relative.
__device__ inline void split_bf16(float x, uint16_t &hi, uint16_t &lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// ---------------------------------------------------------------- fp16 activations and weights
// Activations enter the weight products in fp16, the compute precision of the pages' minimal engine
// ("为什么要自己动手写一个LLM推理引擎" §4.1).  Rounding is to nearest, ties to even; a magnitude beyond
// fp16's largest finite value (65504) is clipped to it instead of overflowing to infinity, the remedy
// "企业官网建设流程全解析" recommends for values outside fp16's range.  NaN stays NaN.
constexpr float kF16Max = 65504.f;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ inline uint16_t f32_to_f16(float f) {
  if (__builtin_fabsf(f) > kF16Max) f = __builtin_copysignf(kF16Max, f);
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ inline float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ inline float f16lo(uint32_t w) { return f16_to_f32((uint16_t)(w & 0xffffu)); }
__device__ inline float f16hi(uint32_t w) { return f16_to_f32((uint16_t)(w >> 16)); }

// Packs 8 values as one 16-byte run of fp16 (one lane's share of a packed activation tile).
__device__ inline uint4 pack8_f16(const float *x) {
  uint32_t h[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) h[j / 2] = f32_to_f16(x[j]) | ((uint32_t)f32_to_f16(x[j + 1]) << 16);
  return make_uint4(h[0], h[1], h[2], h[3]);
}
// The same 8 values as an fp16 pair: hi = fp16(x), lo = fp16(x - hi) (the difference is exact in fp32),
// x == hi + lo to about 2^-22 relative.
__device__ inline void pack8_f16x2(const float *x, uint4 &hi, uint4 &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const uint16_t h0 = f32_to_f16(x[j]), h1 = f32_to_f16(x[j + 1]);
    h[j / 2] = h0 | ((uint32_t)h1 << 16);
    l[j / 2] = f32_to_f16(x[j] - f16_to_f32(h0)) | ((uint32_t)f32_to_f16(x[j + 1] - f16_to_f32(h1)) << 16);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// A packed weight matrix holds w * 2^s in fp16, one shift s per matrix, and ends in a trailer whose
// first word is the largest |w| as fp32 bits.  s puts that largest magnitude in [2^14, 2^15), so every
// bf16 weight within a factor 2^31 of it is an fp16 value exactly (a bf16 significand has 8 bits, fp16
// keeps 11, and its subnormals reach 2^-24); smaller ones round to a multiple of 2^(-24-s).  Products
// take the fp16 values and multiply the fp32 result by 2^-s, an exact rescaling.
constexpr size_t kWTrailer = 256;  // bytes after the tiles of a packed matrix
__host__ __device__ inline int weight_shift(uint32_t max_abs_bits) {
  if (max_abs_bits == 0) return 0;
  const int e = (int)((max_abs_bits >> 23) & 0xff) - 127;  // exponent of the largest magnitude
  const int s = 14 - e;
  return s < -100 ? -100 : (s > 100 ? 100 : s);
}
// 2^-s for the packed matrix whose tiles end at w_end (its trailer), built from its exponent bits
// (s lies in [-100, 100], so 2^-s is a normal fp32 value)
__device__ inline float weight_unscale(const void *w_end) {
  const uint32_t bits = *reinterpret_cast<const uint32_t *>(w_end);
  return __uint_as_float((uint32_t)(127 - weight_shift(bits)) << 23);
}

// Two fp32 values rounded to bf16 (nearest-even) in one packed conversion: a in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
// x = hi + mid + lo with hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid):
// the differences are exact in fp32 and the three parts carry fp32's precision.
// Packs 8 values into the three operand registers of a 16x16x32 bf16 MFMA.
__device__ inline void split3_pack8(const float *x, uint4 &hi, uint4 &mid, uint4 &lo) {
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    h[j / 2] = pack_bf16x2(x[j], x[j + 1]);
    const float r0 = x[j] - bf16lo(h[j / 2]), r1 = x[j + 1] - bf16hi(h[j / 2]);
    m[j / 2] = pack_bf16x2(r0, r1);
    l[j / 2] = pack_bf16x2(r0 - bf16lo(m[j / 2]), r1 - bf16hi(m[j / 2]));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  mid = make_uint4(m[0], m[1], m[2], m[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// f(std::integral_constant<int, I>{}) for I = 0 .. N-1 in order: indices that are constants whatever
// the size of the body (a loop the unroller finds too large keeps a variable index, and an array such
// as a tile's accumulators indexed by it moves to scratch memory).
template <int I, int N>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F &&f) {
    if constexpr (I < N) {
      f(std::integral_constant<int, I>{});
      StaticFor<I + 1, N>::run(f);
    }
  }
};

// The value of lane l ^ 1 (DPP quad permutation 1, 0, 3, 2); every lane of the wave must be active.
__device__ inline float swap_pair_lanes(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// Rotation of pair i at position pos ("为什么要自己动手写一个LLM推理引擎" §4.3 rotates q and k by position):
// the angle pos * inv_freq (inv_freq = theta^(-2i/D), computed in double on the host) is formed in
// double and reduced there to a fraction of a turn in [-1/2, 1/2], so positions in the thousands lose no
// accuracy; the sine and cosine of that fraction come from the hardware's fp32 instructions, which take
// their argument in turns.  Over every (position < 4096, pair) of a 128-wide head their largest error
// against double is 1.8e-7 (the library's fp32 sincosf: 1.5e-7), at a few instructions instead of the
// library's range reduction and polynomials.
__device__ inline void rope_cos_sin(int pos, double inv_freq, float &c, float &s) {
  const double turns = (double)pos * inv_freq * 0.15915494309189535;
  const float r = (float)(turns - rint(turns));
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
}

__device__ inline void raise_error(uint32_t *err, uint32_t bits) {
  if (err) atomicOr(err, bits);
}

// A 16-byte-per-lane load from a buffer straight into LDS (lane l's bytes land at lds_addr + 16 l).
// Issued from asm: the compiler neither counts it nor treats it as a write to LDS, so it adds no waits
// for it before LDS reads (it would wait for every such load in flight, into any stage, before each
// read).  The callers wait for these loads themselves and synchronise the block before reading a
// stage.  The descriptor is built by hand: base address, stride 0, num_records bytes, raw-buffer flags.
__device__ inline u32x4 buffer_desc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
// M0 carries the LDS address; nothing else in these kernels uses it, so the compiler's note that a
// clobbered M0 is not preserved does not apply.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// soff and lds_addr are wave-uniform; readfirstlane hands them to the asm in scalar registers even where
// the compiler keeps them in vector ones.
__device__ inline void load_to_lds16(uint32_t voff, u32x4 desc, uint32_t soff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(desc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                 "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory loads of this wave are in flight and all its LDS reads are done,
// then the block barrier.  The wait is the builtin, so the compiler knows the LDS reads have completed
// (and adds no waits for them later); the barrier is asm with a memory clobber, so the compiler moves
// no memory access across it.
template <int N>
__device__ inline void wait_loads_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // lgkmcnt field (bits 8-11) 0
  asm volatile("s_barrier" : : : "memory");
}

}  // namespace llmdec
