// Sampling the next token on the device ("为什么要自己动手写一个LLM推理引擎" §3.5 and §5.3: temperature,
// top-k and top-p, combined as temperature first, then the truncations, then the draw, with no host
// synchronisation; "大模型推理全流程解析" §2.2.3).
//
// One 1024-thread block per row; thread t holds logits t*per .. t*per+per-1 (per <= 32, so the
// vocabulary is at most 32768) in registers for the whole kernel.
//   1. m = max logit; e_i = exp((z_i - m) / T).
//   2. top-k: the k-th largest logit by a 4-pass radix select (8 bits a pass, counts in LDS) on an
//      order-preserving integer image of the logits, so the kept set is exactly the tokens whose
//      logit is >= the k-th largest (ties stay).
//   3. top-p: over the kept tokens, the largest probability tau such that the kept mass at or above
//      tau reaches p times the kept total, by the same radix select with masses instead of counts
//      (e >= 0, so its bits order like its values); tokens with e >= tau stay.
//   4. u = Philox4x32-10 draw for (seed, step, row): 24 bits times 2^-24.  The token is the first
//      kept one in increasing id whose cumulative mass exceeds u times the kept total; thread sums
//      are combined by a block scan in thread order, so the result does not depend on timing.
// Temperature <= 0 is the greedy choice (largest logit, lowest index on ties).
#include "common.h"
#include "internal.h"

namespace llmdec {

constexpr int kSmpThreads = 1024;
constexpr int kSmpWaves = kSmpThreads / 64;
constexpr int kSmpPer = 32;  // values per thread

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011): ten rounds; each multiplies counter words 0
// and 2 by fixed odd constants into 64-bit products and mixes their halves with words 1 and 3 and
// the key, which is bumped by two Weyl constants between rounds.
__device__ inline uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                        uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) k0 += 0x9E3779B9u, k1 += 0xBB67AE85u;
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1, c3 = (uint32_t)p0, c0 = n0, c2 = n2;
  }
  return c0;
}

// order-preserving integer image of a float: larger float, larger key
__device__ inline uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct SampleArgs {
  const float *logits;
  int vocab, per;
  float temperature, top_p;
  int top_k;
  uint32_t seed_lo, seed_hi, step_lo, step_hi;
  int32_t *next;
};

// Block-wide reductions through LDS: every thread gets the result; waves are combined in wave order.
__device__ inline float block_sum(float v, float *scratch) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < kSmpWaves; ++w) t += scratch[w];
  return t;
}
__device__ inline float block_max(float v, float *scratch) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = scratch[0];
  for (int w = 1; w < kSmpWaves; ++w) t = fmaxf(t, scratch[w]);
  return t;
}

// Run by the 64 lanes of one wave: walking the 256 bins down from 255, find the first bin at which
// start + (everything in higher bins) + (this bin) reaches target; bins with nothing in them are passed
// over.  Lane l holds bins 255-4l .. 252-4l, and the lanes' totals meet in a prefix scan.  Writes the
// bin and the running total before it; if no bin reaches the target (rounding), bin 0 and the total
// of the higher bins.
template <typename T>
__device__ inline void find_bin_desc(const T *h, T start, T target, uint32_t *bin_out, T *before_out) {
  const int lane = threadIdx.x & 63;
  T c[4], t = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c[q] = h[255 - (4 * lane + q)];
    t += c[q];
  }
  T incl = t;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  T excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0;
  T cum = start + excl, before = 0;
  int hit = -1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (hit < 0 && c[q] > 0 && cum + c[q] >= target) hit = q, before = cum;
    cum += c[q];
  }
  const uint64_t m = __ballot(hit >= 0);
  if (m) {
    if (lane == __ffsll((unsigned long long)m) - 1) *bin_out = (uint32_t)(255 - (4 * lane + hit)), *before_out = before;
  } else {
    const T total = __shfl(incl, 63, 64);
    if (lane == 0) *bin_out = 0u, *before_out = start + total - h[0];
  }
}

__global__ __launch_bounds__(kSmpThreads) void sample_kernel(SampleArgs a) {
  __shared__ float red[kSmpWaves];
  __shared__ uint32_t hist[256];
  __shared__ float histf[256];
  __shared__ float whist[kSmpWaves][256];  // top-p: each wave's own mass histogram
  __shared__ uint32_t sel[2];  // chosen digit; remaining count
  __shared__ float self[2];    // mass above the chosen bin
  __shared__ float wtot[kSmpWaves];
  __shared__ int32_t pick, pick_last;

  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.vocab, per = a.per, i0 = tid * per;
  const float *z = a.logits + (size_t)row * V;
  float v[kSmpPer];
#pragma unroll
  for (int j = 0; j < kSmpPer; ++j) v[j] = (j < per && i0 + j < V) ? z[i0 + j] : -INFINITY;
  auto in_range = [&](int j) { return j < per && i0 + j < V; };

  // greedy: largest logit, lowest index on ties
  if (a.temperature <= 0.f) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kSmpPer; ++j)
      if (in_range(j) && (v[j] > bv || bi == 0x7fffffff)) bv = v[j], bi = i0 + j;
    const float m = block_max(bv, red);
    if (tid == 0) pick = 0x7fffffff;
    __syncthreads();
    if (bv == m) atomicMin(&pick, bi);
    __syncthreads();
    if (tid == 0) a.next[row] = pick;
    return;
  }

  float lm = -INFINITY;
#pragma unroll
  for (int j = 0; j < kSmpPer; ++j) lm = fmaxf(lm, v[j]);
  const float m = block_max(lm, red);
  // e_j for the thread's tokens (with the logits: 64 values, a few of them spilled at 128 registers)
  float ev[kSmpPer];
  uint32_t kept = 0;  // bit j: token i0 + j is kept
#pragma unroll
  for (int j = 0; j < kSmpPer; ++j) {
    ev[j] = in_range(j) ? expf((v[j] - m) / a.temperature) : 0.f;
    if (in_range(j)) kept |= 1u << j;
  }
  auto e = [&](int j) { return ev[j]; };

  // top-k: the k-th largest logit's key
  if (a.top_k > 0 && a.top_k < V) {
    uint32_t prefix = 0, pmask = 0;
    int remaining = a.top_k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kSmpPer; ++j) {
        const uint32_t key = order_key(v[j]);
        if ((kept >> j & 1) && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) find_bin_desc<uint32_t>(hist, 0u, (uint32_t)remaining, &sel[0], &sel[1]);
      __syncthreads();
      if (tid == 0) sel[1] = (uint32_t)remaining - sel[1];  // the rank left inside the chosen bin
      __syncthreads();
      prefix |= sel[0] << shift;
      pmask |= 255u << shift;
      remaining = (int)sel[1];
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < kSmpPer; ++j)
      if (order_key(v[j]) < prefix) kept &= ~(1u << j);
  }

  // top-p over the kept tokens
  if (a.top_p < 1.f) {
    float ts = 0.f;
#pragma unroll
    for (int j = 0; j < kSmpPer; ++j)
      if (kept >> j & 1) ts += e(j);
    const float target = a.top_p * block_sum(ts, red);
    uint32_t prefix = 0, pmask = 0;
    float above = 0.f;  // kept mass strictly above the current prefix range
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      // masses go to the wave's own histogram (no other wave adds to it, so the waves do not contend
      // and each bin's sum does not depend on how the waves interleave), then bin by bin in wave order
#pragma unroll
      for (int q = 0; q < 4; ++q) whist[wave][lane + 64 * q] = 0.f;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kSmpPer; ++j) {
        const float ev = e(j);
        const uint32_t key = __float_as_uint(ev);
        if ((kept >> j & 1) && (key & pmask) == prefix) atomicAdd(&whist[wave][(key >> shift) & 255u], ev);
      }
      __syncthreads();
      if (tid < 256) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < kSmpWaves; ++w) t += whist[w][tid];
        histf[tid] = t;
      }
      __syncthreads();
      // (if rounding leaves the target out of reach, the whole range stays: bin 0)
      if (wave == 0) find_bin_desc<float>(histf, above, target, &sel[0], &self[0]);
      __syncthreads();
      prefix |= sel[0] << shift;
      pmask |= 255u << shift;
      above = self[0];
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < kSmpPer; ++j)
      if (__float_as_uint(e(j)) < prefix) kept &= ~(1u << j);
  }

  // the draw: first kept token in increasing id whose cumulative mass exceeds u times the kept total
  float ts = 0.f;
#pragma unroll
  for (int j = 0; j < kSmpPer; ++j)
    if (kept >> j & 1) ts += e(j);
  // exclusive scan of the thread sums in thread order
  float incl = ts;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  float excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.f;
  if (lane == 63) wtot[wave] = incl;
  if (tid == 0) pick = 0x7fffffff, pick_last = -1;
  __syncthreads();
  float base = 0.f, total = 0.f;
  for (int w = 0; w < kSmpWaves; ++w) {
    if (w < wave) base += wtot[w];
    total += wtot[w];
  }
  const uint32_t wd = philox_word0((uint32_t)row, a.step_lo, a.step_hi, 0u, a.seed_lo, a.seed_hi);
  const float u = (float)(wd >> 8) * 5.9604644775390625e-8f;  // 2^-24
  const float target = u * total;
  float c = base + excl;  // mass before this thread's tokens
  int found = -1, last = -1;
#pragma unroll
  for (int j = 0; j < kSmpPer; ++j) {
    if (kept >> j & 1) {
      last = i0 + j;
      c += e(j);
      if (found < 0 && c > target) found = i0 + j;
    }
  }
  if (found >= 0) atomicMin(&pick, found);
  if (last >= 0) atomicMax(&pick_last, last);
  __syncthreads();
  // rounding may put the target past the last cumulative value: then the last kept token
  if (tid == 0) a.next[row] = pick != 0x7fffffff ? pick : pick_last;
}

bool sample_shape_ok(int vocab) { return vocab > 0 && vocab <= kSmpThreads * kSmpPer; }

void launch_sample(const float *logits, int rows, int vocab, float temperature, int top_k, float top_p,
                   uint64_t seed, uint64_t step, int32_t *next, hipStream_t s) {
  SampleArgs a;
  a.logits = logits, a.vocab = vocab, a.per = (vocab + kSmpThreads - 1) / kSmpThreads;
  a.temperature = temperature, a.top_p = top_p, a.top_k = top_k;
  a.seed_lo = (uint32_t)seed, a.seed_hi = (uint32_t)(seed >> 32);
  a.step_lo = (uint32_t)step, a.step_hi = (uint32_t)(step >> 32);
  a.next = next;
  if (rows > 0) sample_kernel<<<rows, kSmpThreads, 0, s>>>(a);
}

}  // namespace llmdec
