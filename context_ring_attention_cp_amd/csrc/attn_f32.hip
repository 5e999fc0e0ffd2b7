// float32 block kernel: one rank's query shard against one K/V block with the
// online-softmax recurrence of the compassingai.com context-parallelism page
// (section "線上 Softmax"), computed entirely in fp32 on the vector ALUs so that
// fp32 inputs are never rounded to a narrower type.
//
// Four consecutive lanes own one query row; lane quarter x4 holds head-dim
// elements x4, x4+4, x4+8, ... of q and of the running O (so a row's state
// fits in registers for d = 128), and a score is the sum of the four lanes'
// partial dot products.  A workgroup of 256 lanes covers 64 rows and stages
// key tiles of 16 keys of K and V in LDS.
#include "launch.h"

#include <math.h>

namespace cpattn {
namespace {

constexpr int kRows = 64;
constexpr int kLanesPerRow = 4;
constexpr int kThreads = kRows * kLanesPerRow;
constexpr int kKeys = 16;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;

__device__ __forceinline__ int64_t doc_start_of(const int32_t* __restrict__ cu, int ndocs, int64_t p) {
  int lo = 0, hi = ndocs;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)cu[mid] <= p) lo = mid; else hi = mid;
  }
  return cu[lo];
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_block_f32_kernel(BlockArgs a) {
  constexpr int DQ = D / kLanesPerRow;      // head-dim elements per lane
  __shared__ __attribute__((aligned(16))) float Ks[kKeys][D];
  __shared__ __attribute__((aligned(16))) float Vs[kKeys][D];

  const int tid = threadIdx.x;
  const int x4 = tid & (kLanesPerRow - 1);
  const int64_t L = a.L;
  const int H = a.H;
  const int64_t rows_end = a.rows_end;                     // rows taking part in this launch
  const int nqt = (int)((rows_end + kRows - 1) / kRows);
  const int64_t hb = blockIdx.x / nqt;
  const int qt = nqt - 1 - (int)(blockIdx.x % nqt);
  const int h = (int)(hb % H), b = (int)(hb / H);
  const int64_t rs = (int64_t)H * D;
  const int64_t base = (int64_t)b * L * rs + (int64_t)h * D;
  const float* __restrict__ qg = (const float*)a.q + base;
  const float* __restrict__ kg = (const float*)a.k + base;
  const float* __restrict__ vg = (const float*)a.v + base;

  const int64_t q0 = (int64_t)qt * kRows;
  const int64_t row = q0 + tid / kLanesPerRow;
  const bool row_ok = row < L;
  const int64_t p = a.q_pos0 + row;
  const int mask = a.mask;
  const bool doc = mask == MASK_DOC_CAUSAL;
  const int64_t last = (q0 + kRows < rows_end ? q0 + kRows : rows_end) - 1;

  const int nkt = (int)((L + kKeys - 1) / kKeys);
  int kt_begin = 0, kt_end = nkt;
  if (mask != MASK_NONE) {
    const int64_t hi = a.q_pos0 + last - a.k_pos0;
    kt_end = hi < 0 ? 0 : (int)(hi / kKeys + 1 < nkt ? hi / kKeys + 1 : nkt);
    if (doc) {
      const int64_t lo = doc_start_of(a.cu, a.ndocs, a.q_pos0 + q0) - a.k_pos0;
      if (lo > 0) kt_begin = (int)(lo / kKeys < nkt ? lo / kKeys : nkt);
    }
  }
  const bool rd = a.flags & F_READ_STATE;
  // nothing to compute and nothing to store: the state of these rows stays as it is
  if (kt_begin >= kt_end && rd && !writes_final(a.flags, last, a.final_from) && !(a.flags & F_WRITE_PARTIAL)) return;
  const int64_t dstart = doc ? doc_start_of(a.cu, a.ndocs, row_ok ? p : a.q_pos0 + last) : 0;

  float q[DQ], o[DQ];
  float m_run = -INFINITY, l_run = 0.f;   // m in base-2 units
  const int64_t st_row = ((int64_t)b * L + row) * rs + (int64_t)h * D;
  const int64_t ml_idx = ((int64_t)b * H + h) * L + row;
#pragma unroll
  for (int x = 0; x < DQ; ++x) {
    q[x] = row_ok ? qg[row * rs + kLanesPerRow * x + x4] : 0.f;
    o[x] = 0.f;
  }
  if (rd && row_ok) {
    m_run = a.st_m[ml_idx] * kLog2e;
    l_run = a.st_l[ml_idx];
#pragma unroll
    for (int x = 0; x < DQ; ++x) o[x] = a.st_o[st_row + kLanesPerRow * x + x4];
  }
  const float c2 = a.scale_log2;

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int64_t k0 = (int64_t)kt * kKeys;
    __syncthreads();
    for (int e = tid; e < kKeys * D / 4; e += kThreads) {
      const int kk = e / (D / 4), c4 = e % (D / 4);
      float4 kv = float4{0.f, 0.f, 0.f, 0.f}, vv = float4{0.f, 0.f, 0.f, 0.f};
      if (k0 + kk < L) {
        kv = *(const float4*)(kg + (k0 + kk) * rs + 4 * c4);
        vv = *(const float4*)(vg + (k0 + kk) * rs + 4 * c4);
      }
      *(float4*)&Ks[kk][4 * c4] = kv;
      *(float4*)&Vs[kk][4 * c4] = vv;
    }
    __syncthreads();
    float s[kKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kKeys; ++kk) {
      float acc = 0.f;
#pragma unroll
      for (int x = 0; x < DQ; ++x) acc = __builtin_fmaf(q[x], Ks[kk][kLanesPerRow * x + x4], acc);
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      const int64_t c = a.k_pos0 + k0 + kk;
      const bool vis = (k0 + kk < L) && (mask == MASK_NONE || (c <= p && (!doc || c >= dstart)));
      s[kk] = vis ? acc * c2 : -INFINITY;
      mx = fmaxf(mx, s[kk]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int x = 0; x < DQ; ++x) o[x] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kKeys; ++kk) {
      const float pk = __builtin_amdgcn_exp2f(s[kk] - m_use);
      l_run += pk;
#pragma unroll
      for (int x = 0; x < DQ; ++x) o[x] = __builtin_fmaf(pk, Vs[kk][kLanesPerRow * x + x4], o[x]);
    }
  }

  if (!row_ok || row >= rows_end) return;
  const bool has = l_run > 0.f;
  if (writes_state(a.flags, row, a.final_from)) {
#pragma unroll
    for (int x = 0; x < DQ; ++x) a.st_o[st_row + kLanesPerRow * x + x4] = o[x];
    if (x4 == 0) {
      a.st_m[ml_idx] = m_run * kLn2;
      a.st_l[ml_idx] = l_run;
    }
  }
  const float inv = has ? 1.f / l_run : 0.f;
  // v_log_f32 is the base-2 logarithm
  const float lse = has ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
  if (writes_final(a.flags, row, a.final_from)) {
    float* outp = (float*)a.out + st_row;
#pragma unroll
    for (int x = 0; x < DQ; ++x) outp[kLanesPerRow * x + x4] = o[x] * inv;
    if (x4 == 0) {
      if (a.m_out) a.m_out[ml_idx] = m_run * kLn2;
      if (a.l_out) a.l_out[ml_idx] = l_run;
      if (a.lse_out) a.lse_out[ml_idx] = lse;
    }
  }
  if (a.flags & F_WRITE_PARTIAL) {
#pragma unroll
    for (int x = 0; x < DQ; ++x) a.o_part[st_row + kLanesPerRow * x + x4] = o[x] * inv;
    if (x4 == 0) a.lse_part[ml_idx] = lse;
  }
}

}  // namespace

hipError_t launch_block_f32(const BlockArgs& a, int d, hipStream_t s, const LaunchEvents& ev) {
  if (a.flags & (F_SPLIT | F_READ_SIDE)) return hipErrorInvalidValue;   // bf16 kernel only
  const int64_t nqt = (a.rows_end + kRows - 1) / kRows;
  const dim3 grid((unsigned)(nqt * a.H * a.B)), block(kThreads);
  return d == 128 ? launch_bound(attn_block_f32_kernel<128>, grid, block, s, ev, a)
                  : launch_bound(attn_block_f32_kernel<64>, grid, block, s, ev, a);
}

}  // namespace cpattn
