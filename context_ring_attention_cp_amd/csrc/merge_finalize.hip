// HBM-bound epilogue kernels.
//
// merge: the log-sum-exp form of the online-softmax merge (compassingai.com
// context-parallelism page, section "線上 Softmax", rewritten for normalised
// partials): lse = ln sum_j exp(lse_j), O = sum_j exp(lse_j - lse) O_j, the
// terms summed in the caller's order.
// finalize: out = O / l, lse = m + ln l (same section, last line).
//
// Both are streaming kernels: each thread owns 4 consecutive head-dim
// elements of one (batch, row, head), so a wave reads/writes whole 512-byte
// rows of float32 with 16-byte accesses.
#include "kernels.h"

#include <math.h>

namespace cpattn {
namespace {

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;
constexpr int kThreads = 256;

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store4(void* out, int64_t off, bool bf, float4 v) {
  if (bf) {
    const bf16x2 lo = __builtin_convertvector(float2v{v.x, v.y}, bf16x2);
    const bf16x2 hi = __builtin_convertvector(float2v{v.z, v.w}, bf16x2);
    *(bf16x4*)((bf16*)out + off) = bf16x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    *(float4*)((float*)out + off) = v;
  }
}

// Parts whose lse values are held in registers in one pass; longer merges
// reread them.
constexpr int kRegParts = 16;
// Partials loaded back to back before their multiply-adds.
constexpr int kBatch = 8;

__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  const int d4 = a.d / 4;
  const int64_t total = (int64_t)a.B * a.L * a.H * d4;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const int x4 = (int)(idx % d4);
  const int64_t rowhead = idx / d4;               // (b * L + row) * H + h
  const int h = (int)(rowhead % a.H);
  const int64_t br = rowhead / a.H;               // b * L + row
  const int64_t row = br % a.L;
  const int b = (int)(br / a.L);
  const int64_t ml = ((int64_t)b * a.H + h) * a.L + row;
  const int n = a.n;

  // lse = ln sum exp(lse_j), in base 2 with the max factored out
  float l2[kRegParts];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kRegParts; ++j) {
    l2[j] = j < n ? a.lse[j][ml] * kLog2e : -INFINITY;
    mx = fmaxf(mx, l2[j]);
  }
  for (int j = kRegParts; j < n; ++j) mx = fmaxf(mx, a.lse[j][ml] * kLog2e);
  float4 o = float4{0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float tot = 0.f;
#pragma unroll
    for (int j = 0; j < kRegParts; ++j) tot += __builtin_amdgcn_exp2f(l2[j] - mx);
    for (int j = kRegParts; j < n; ++j) tot += __builtin_amdgcn_exp2f(__builtin_fmaf(a.lse[j][ml], kLog2e, -mx));
    const float lse2 = mx + __builtin_amdgcn_logf(tot);   // v_log_f32 is log2
    lse = lse2 * kLn2;
    const int64_t off = rowhead * a.d + 4 * x4;
    // terms in the given order, kBatch partial loads in flight at a time
    for (int j0 = 0; j0 < n; j0 += kBatch) {
      float4 v[kBatch];
      float wj[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int j = j0 + t;
        v[t] = j < n ? *(const float4*)(a.o[j] + off) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int j = j0 + t;
        const float lj = j < kRegParts ? l2[j < kRegParts ? j : 0] : (j < n ? a.lse[j][ml] * kLog2e : -INFINITY);
        wj[t] = j < n ? __builtin_amdgcn_exp2f(lj - lse2) : 0.f;
      }
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        o.x = __builtin_fmaf(wj[t], v[t].x, o.x);
        o.y = __builtin_fmaf(wj[t], v[t].y, o.y);
        o.z = __builtin_fmaf(wj[t], v[t].z, o.z);
        o.w = __builtin_fmaf(wj[t], v[t].w, o.w);
      }
    }
  }
  store4(a.out, rowhead * a.d + 4 * x4, a.out_bf16, o);
  if (x4 == 0 && a.lse_out) a.lse_out[ml] = lse;
}

__global__ __launch_bounds__(kThreads) void finalize_kernel(FinalizeArgs a) {
  const int d4 = a.d / 4;
  const int64_t total = (int64_t)a.B * a.L * a.H * d4;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const int x4 = (int)(idx % d4);
  const int64_t rowhead = idx / d4;
  const int h = (int)(rowhead % a.H);
  const int64_t br = rowhead / a.H;
  const int64_t row = br % a.L;
  const int b = (int)(br / a.L);
  const int64_t ml = ((int64_t)b * a.H + h) * a.L + row;
  const float l = a.st_l[ml];
  const float m = a.st_m[ml];
  const bool has = l > 0.f;
  const float inv = has ? 1.f / l : 0.f;
  const float4 v = *(const float4*)(a.st_o + rowhead * a.d + 4 * x4);
  store4(a.out, rowhead * a.d + 4 * x4, a.out_bf16, float4{v.x * inv, v.y * inv, v.z * inv, v.w * inv});
  if (x4 == 0) {
    if (a.m_out) a.m_out[ml] = m;
    if (a.l_out) a.l_out[ml] = l;
    if (a.lse_out) a.lse_out[ml] = has ? m + __builtin_amdgcn_logf(l) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.L * a.H * (a.d / 4);
  merge_kernel<<<dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.L * a.H * (a.d / 4);
  finalize_kernel<<<dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace cpattn
