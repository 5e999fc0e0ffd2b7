// Regrouping kernels of all-to-all (Ulysses) context parallelism for gfx950.
//
// The ranks hold sequence shards [B, L, H, d]; a first all-to-all regroups
// Q, K and V so that each rank holds the whole sequence of its heads, and a
// second one returns the attention outputs to the sequence shards
// (compassingai.com context-parallelism page, section
// "方案二：All-to-All（全交換）").  On one GPU the exchanges are these copies:
//   gather:  full[b, i L + t, h', :] = shard_i[b, t, h0 + h', :]
//   scatter: shard_i[b, t, h0 + h', :] = full[b, i L + t, h', :]
// for the head group [h0, h0 + Hn) of one rank.  A (batch, token) row of the
// group is one contiguous run of Hn d elements in both layouts; each thread
// moves 16 bytes, consecutive threads consecutive bytes of a run.  The
// second grid dimension is the shard, so the shard pointer is a uniform load.
#include "kernels.h"

#include <stdint.h>

namespace cpattn {
namespace {

constexpr int kThreads = 256;

template <bool GATHER, typename I>
__global__ __launch_bounds__(kThreads) void a2a_kernel(RegroupArgs a) {
  const int i = blockIdx.y;                                   // shard (rank) of these rows
  const I cpr = (I)((int64_t)a.Hn * a.d * a.elt / 16);        // 16-byte chunks per row of the group
  const I total = (I)(a.B * a.L) * cpr;                       // chunks of this shard's rows
  char* __restrict__ sh = (char*)a.shards[i];
  char* __restrict__ fu = (char*)a.full;
  const int64_t row_bytes = (int64_t)a.H * a.d * a.elt;       // shard row: all H heads
  const int64_t grp_bytes = (int64_t)a.h0 * a.d * a.elt;      // start of the group in a shard row
  for (I idx = (I)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += (I)gridDim.x * kThreads) {
    const I rl = idx / cpr;                                   // b L + t
    const I c = idx - rl * cpr;
    const I b = rl / (I)a.L;
    const I t = rl - b * (I)a.L;
    const int64_t s_off = (int64_t)rl * row_bytes + grp_bytes + 16 * (int64_t)c;
    const int64_t f_off = (((int64_t)b * a.S + (int64_t)i * a.L + t) * cpr + c) * 16;
    if (GATHER) *(uint4*)(fu + f_off) = *(const uint4*)(sh + s_off);
    else *(uint4*)(sh + s_off) = *(const uint4*)(fu + f_off);
  }
}

template <bool GATHER>
hipError_t launch_a2a(const RegroupArgs& a, hipStream_t s) {
  const int64_t total = a.B * a.L * ((int64_t)a.Hn * a.d * a.elt / 16);
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;                          // grid-stride beyond this
  const dim3 grid((unsigned)blocks, (unsigned)a.N);
  if (total < ((int64_t)1 << 31) - (int64_t)65536 * kThreads) a2a_kernel<GATHER, uint32_t><<<grid, kThreads, 0, s>>>(a);
  else a2a_kernel<GATHER, int64_t><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_a2a_gather(const RegroupArgs& a, hipStream_t s) { return launch_a2a<true>(a, s); }
hipError_t launch_a2a_scatter(const RegroupArgs& a, hipStream_t s) { return launch_a2a<false>(a, s); }

}  // namespace cpattn
