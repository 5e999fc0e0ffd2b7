// HBM-bound epilogue kernels.
//
// merge: the log-sum-exp form of the online-softmax merge (compassingai.com
// context-parallelism page, section "線上 Softmax", rewritten for normalised
// partials): lse = ln sum_j exp(lse_j), O = sum_j exp(lse_j - lse) O_j, the
// terms summed in the caller's order.
// finalize: out = O / l, lse = m + ln l (same section, last line).
//
// Both are streaming kernels: each thread owns 8 (merge) or 4 (finalize)
// consecutive head-dim elements of one (batch, row, head), so a wave
// reads/writes whole 512-byte rows of float32 with 16-byte accesses.  A
// workgroup covers consecutive (batch, row, head) triples in memory order
// (a 1-D grid), so its partial and state reads are one contiguous run; the
// small lse / m / l loads ([B, H, L]) are the scattered ones, and they stay
// in the caches (a cache line of them serves 32 rows).  Measured at the
// merge stress case: 0.112 ms against 0.123 ms with workgroups of rows of
// one (batch, head).
#include "launch.h"

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

// grid: one workgroup per kThreads / (D / 8) consecutive (batch, row, head)
// triples.  Each thread owns 8 consecutive head-dim elements (two 16-byte
// loads per part), so a thread keeps 2 kBatch partial loads in flight.
template <int D, bool I32>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  constexpr int D8 = D / 8;                       // threads per row-head
  constexpr int RPW = kThreads / D8;              // row-heads per workgroup
  const int64_t rowhead = (int64_t)blockIdx.x * RPW + threadIdx.x / D8;   // ((b L) + row) H + h
  if (rowhead >= (int64_t)a.B * a.L * a.H) return;
  int64_t h, row, b;
  if constexpr (I32) {        // 32-bit divisions when B L H fits (the usual case)
    const uint32_t rh = (uint32_t)rowhead, bl = rh / (uint32_t)a.H;
    h = rh - bl * (uint32_t)a.H;
    b = bl / (uint32_t)a.L;
    row = bl - (uint32_t)b * (uint32_t)a.L;
  } else {
    h = rowhead % a.H;
    const int64_t bl = rowhead / a.H;
    row = bl % a.L;
    b = bl / a.L;
  }
  const int x8 = threadIdx.x % D8;
  const int64_t ml = (b * a.H + h) * a.L + row;
  const int64_t off = rowhead * D + 8 * x8;
  const int n = a.n;

  // The partials of the first kBatch parts are requested before the lse
  // values, so the two memory latencies of a thread overlap.
  float4 v0[kBatch], v1[kBatch];
#pragma unroll
  for (int t = 0; t < kBatch; ++t) {
    v0[t] = t < n ? *(const float4*)(a.o[t] + off) : float4{0.f, 0.f, 0.f, 0.f};
    v1[t] = t < n ? *(const float4*)(a.o[t] + off + 4) : float4{0.f, 0.f, 0.f, 0.f};
  }
  // lse = ln sum exp(lse_j), in base 2 with the max factored out.  The lse
  // values held in registers are loaded without a branch (slots from n on
  // alias part 0, so every load is valid) and the unused ones masked after.
  float l2[kRegParts];
#pragma unroll
  for (int j = 0; j < kRegParts; ++j) l2[j] = a.lse[j][ml];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kRegParts; ++j) {
    l2[j] = j < n ? l2[j] * kLog2e : -INFINITY;
    mx = fmaxf(mx, l2[j]);
  }
  for (int j = kRegParts; j < n; ++j) mx = fmaxf(mx, a.lse[j][ml] * kLog2e);
  float4 o0 = float4{0.f, 0.f, 0.f, 0.f}, o1 = o0;
  float lse = -INFINITY;
  auto fma_batch = [&](const float (&wj)[kBatch]) {
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      o0.x = __builtin_fmaf(wj[t], v0[t].x, o0.x);
      o0.y = __builtin_fmaf(wj[t], v0[t].y, o0.y);
      o0.z = __builtin_fmaf(wj[t], v0[t].z, o0.z);
      o0.w = __builtin_fmaf(wj[t], v0[t].w, o0.w);
      o1.x = __builtin_fmaf(wj[t], v1[t].x, o1.x);
      o1.y = __builtin_fmaf(wj[t], v1[t].y, o1.y);
      o1.z = __builtin_fmaf(wj[t], v1[t].z, o1.z);
      o1.w = __builtin_fmaf(wj[t], v1[t].w, o1.w);
    }
  };
  if (mx != -INFINITY) {
    float tot = 0.f;
#pragma unroll
    for (int j = 0; j < kRegParts; ++j) tot += __builtin_amdgcn_exp2f(l2[j] - mx);
    for (int j = kRegParts; j < n; ++j) tot += __builtin_amdgcn_exp2f(__builtin_fmaf(a.lse[j][ml], kLog2e, -mx));
    const float lse2 = mx + __builtin_amdgcn_logf(tot);   // v_log_f32 is log2
    lse = lse2 * kLn2;
    // terms in the given order; the weights of the parts held in registers
    // are indexed at compile time
    float wj[kBatch];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) wj[t] = t < n ? __builtin_amdgcn_exp2f(l2[t] - lse2) : 0.f;
    fma_batch(wj);
    static_assert(kRegParts == 2 * kBatch, "two batches held in registers");
    if (n > kBatch) {
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int j = kBatch + t;
        v0[t] = j < n ? *(const float4*)(a.o[j] + off) : float4{0.f, 0.f, 0.f, 0.f};
        v1[t] = j < n ? *(const float4*)(a.o[j] + off + 4) : float4{0.f, 0.f, 0.f, 0.f};
        wj[t] = j < n ? __builtin_amdgcn_exp2f(l2[j] - lse2) : 0.f;
      }
      fma_batch(wj);
    }
    // parts from kRegParts on: their lse values are read again
    for (int j0 = kRegParts; j0 < n; j0 += kBatch) {
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int j = j0 + t;
        v0[t] = j < n ? *(const float4*)(a.o[j] + off) : float4{0.f, 0.f, 0.f, 0.f};
        v1[t] = j < n ? *(const float4*)(a.o[j] + off + 4) : float4{0.f, 0.f, 0.f, 0.f};
        wj[t] = j < n ? __builtin_amdgcn_exp2f(__builtin_fmaf(a.lse[j][ml], kLog2e, -lse2)) : 0.f;
      }
      fma_batch(wj);
    }
  }
  store4(a.out, off, a.out_bf16, o0);
  store4(a.out, off + 4, a.out_bf16, o1);
  if (x8 == 0 && a.lse_out) a.lse_out[ml] = lse;
}

// grid: one workgroup per kThreads / (D / 4) consecutive (batch, row, head)
// triples; each thread owns 4 consecutive head-dim elements.
template <int D>
__global__ __launch_bounds__(kThreads) void finalize_kernel(FinalizeArgs a) {
  constexpr int D4 = D / 4;
  constexpr int RPW = kThreads / D4;
  const int64_t rowhead = (int64_t)blockIdx.x * RPW + threadIdx.x / D4;   // ((b L) + row) H + h
  if (rowhead >= (int64_t)a.B * a.L * a.H) return;
  const int h = (int)(rowhead % a.H);
  const int64_t bl = rowhead / a.H;
  const int64_t row = bl % a.L, b = bl / a.L;
  const int x4 = threadIdx.x % D4;
  const int64_t ml = (b * a.H + h) * a.L + row;
  const float l = a.st_l[ml];
  const float m = a.st_m[ml];
  const bool has = l > 0.f;
  const float inv = has ? 1.f / l : 0.f;
  const float4 v = *(const float4*)(a.st_o + rowhead * D + 4 * x4);
  store4(a.out, rowhead * D + 4 * x4, a.out_bf16, float4{v.x * inv, v.y * inv, v.z * inv, v.w * inv});
  if (x4 == 0) {
    if (a.m_out) a.m_out[ml] = m;
    if (a.l_out) a.l_out[ml] = l;
    if (a.lse_out) a.lse_out[ml] = has ? m + __builtin_amdgcn_logf(l) * kLn2 : -INFINITY;
  }
}

}  // namespace

// The grids (B L H / 16 or / 32 workgroups) stay below 2^31: the caller
// bounds B L H d / 1024.
hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int rpw = kThreads / (a.d / 8);
  const dim3 grid((unsigned)(((int64_t)a.B * a.L * a.H + rpw - 1) / rpw));
  const bool i32 = (int64_t)a.B * a.L * a.H < ((int64_t)1 << 31);
  if (a.d == 128) {
    if (i32) merge_kernel<128, true><<<grid, dim3(kThreads), 0, s>>>(a);
    else merge_kernel<128, false><<<grid, dim3(kThreads), 0, s>>>(a);
  } else {
    if (i32) merge_kernel<64, true><<<grid, dim3(kThreads), 0, s>>>(a);
    else merge_kernel<64, false><<<grid, dim3(kThreads), 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s) {
  const int rpw = kThreads / (a.d / 4);
  const dim3 grid((unsigned)(((int64_t)a.B * a.L * a.H + rpw - 1) / rpw));
  if (a.d == 128) finalize_kernel<128><<<grid, dim3(kThreads), 0, s>>>(a);
  else finalize_kernel<64><<<grid, dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace cpattn
