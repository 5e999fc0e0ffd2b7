// FP8 (OCP e4m3) quantisation of a [B, L, H, d] bf16 block for gfx950.
//
// One scale per (batch, head), a power of two: with y = float32(x * c) (c a
// float32 pre-multiplier: 1 for keys and values, the softmax scale times
// log2(e) for the query), amax = max |y| over the block's tokens and head
// dim and scale = 2^e, e the smallest integer >= -126 with
// amax <= 448 * 2^e (0 when amax = 0); code(x) = e4m3 nearest to y * 2^-e,
// ties to even (v_cvt_pk_fp8_f32, which rounds to nearest even; the clamp
// to +-448 only guards it, since |y * 2^-e| <= 448 by the choice of e).
// Powers of two are what the FP8 matrix core's e8m0 block-scale operands
// apply exactly.  The compassingai.com context-parallelism page notes that
// the bytes CP moves depend on FP8 transfer (section "通訊量分析"); the format
// and scaling are this library's choice.
//
// Four launches, all HBM-bound streaming except the last: fill the amax slots
// with 0, the per-workgroup maxima merged with a vector atomicMax on the
// float bits (order-preserving for non-negative floats), the codes, then the
// scales.  Each thread handles 8 consecutive elements of one token row of one
// head; a workgroup covers kRowsPerWg rows of one (b, h).
#include "launch.h"

#include <stdint.h>

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWg = 256;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// e of an amax (amax = m 2^k with 0.5 <= m < 1, and 448 = 0.875 * 2^9: the
// smallest e with m 2^k <= 0.875 * 2^(9+e) is k - 9, or k - 8 when m > 0.875)
__device__ __forceinline__ int scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int k;
  const float m = frexpf(amax, &k);
  const int e = k - 9 + (m > 0.875f ? 1 : 0);
  return e < -126 ? -126 : e;
}

// 2^e for -126 <= e <= 127, from its bits
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

__global__ __launch_bounds__(kThreads) void fill_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = v;
}

// grid: x = row chunk of kRowsPerWg rows, y = b * H + h
template <int D>
__global__ __launch_bounds__(kThreads) void amax_kernel(QuantArgs a, float prescale) {
  constexpr int TPR = D / 8;                        // threads per row
  constexpr int RPP = kThreads / TPR;               // rows per pass
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int64_t r0 = (int64_t)blockIdx.x * kRowsPerWg;
  const int c = threadIdx.x % TPR;
  float m = 0.f;
  for (int rr = threadIdx.x / TPR; rr < kRowsPerWg; rr += RPP) {
    const int64_t t = r0 + rr;
    if (t < a.L) {
      const bf16x8 x = *(const bf16x8*)((const bf16*)a.x + (((int64_t)b * a.L + t) * a.H + h) * D + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)x[e] * prescale));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float wm[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = wm[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) mm = fmaxf(mm, wm[i]);
    atomicMax((unsigned int*)&a.scales[bh], __float_as_uint(mm));
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a, float prescale) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const float amax = a.scales[bh];                  // still the amax here
  const float inv = pow2f(-scale_exp(amax));       // exact: 2^-e, -120 <= -e <= 126
  const int64_t r0 = (int64_t)blockIdx.x * kRowsPerWg;
  const int c = threadIdx.x % TPR;
  for (int rr = threadIdx.x / TPR; rr < kRowsPerWg; rr += RPP) {
    const int64_t t = r0 + rr;
    if (t >= a.L) break;
    const int64_t off = (((int64_t)b * a.L + t) * a.H + h) * D + 8 * c;
    const bf16x8 x = *(const bf16x8*)((const bf16*)a.x + off);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xc = (float)x[e] * prescale;     // the float32 product, rounded once
      y[e] = __builtin_amdgcn_fmed3f(xc * inv, -448.f, 448.f);
    }
    uint32_t w0 = 0, w1 = 0;
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], w0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], w1, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
    *(uint2*)((uint8_t*)a.codes + off) = uint2{w0, w1};
  }
}

__global__ __launch_bounds__(kThreads) void scale_kernel(float* s, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) s[i] = pow2f(scale_exp(s[i]));
}

}  // namespace

hipError_t launch_quantize_fp8(const QuantArgs& a, int d, float prescale, hipStream_t s) {
  const int n = a.B * a.H;
  const dim3 grid((unsigned)((a.L + kRowsPerWg - 1) / kRowsPerWg), (unsigned)n);
  fill_kernel<<<(n + kThreads - 1) / kThreads, kThreads, 0, s>>>(a.scales, n, 0.f);
  if (d == 128) {
    amax_kernel<128><<<grid, kThreads, 0, s>>>(a, prescale);
    quantize_kernel<128><<<grid, kThreads, 0, s>>>(a, prescale);
  } else {
    amax_kernel<64><<<grid, kThreads, 0, s>>>(a, prescale);
    quantize_kernel<64><<<grid, kThreads, 0, s>>>(a, prescale);
  }
  scale_kernel<<<(n + kThreads - 1) / kThreads, kThreads, 0, s>>>(a.scales, n);
  return hipGetLastError();
}

}  // namespace cpattn
