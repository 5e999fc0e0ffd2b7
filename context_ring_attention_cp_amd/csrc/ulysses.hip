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
//
// For bf16 V over a sequence of whole 64-key tiles the gather writes the
// tiled layout the attention kernel reads best instead ([B, Hn, S / 64, d,
// 64]: each 64-key tile head-dim-major and contiguous), taking each key row
// from whichever shard holds it.
#include "launch.h"
#include "gfx950_util.h"

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

// One workgroup per (batch, head of the group, 64-key tile of the whole
// sequence): the tile's rows go through LDS (rows padded by 16 bytes), then
// every lane writes 16-byte runs of 8 consecutive keys of one head-dim row.
template <int D>
__global__ __launch_bounds__(kThreads) void a2a_gather_v_tiles_kernel(RegroupArgs a) {
  using dev::bf16;
  using dev::bf16x8;
  constexpr int kT = 64;
  constexpr int CH = D / 8;
  constexpr int RS = D + 8;
  __shared__ __attribute__((aligned(16))) bf16 t[kT * RS];
  const int64_t ntile = a.S / kT;
  const int64_t bid = blockIdx.x;
  const int64_t kt = bid % ntile;
  const int64_t hb = bid / ntile;
  const int h = (int)(hb % a.Hn);
  const int64_t b = hb / a.Hn;
  const int tid = threadIdx.x;
#pragma unroll
  for (int s = tid; s < kT * CH; s += kThreads) {
    const int r = s / CH, c = s % CH;
    const int64_t key = kt * kT + r;                          // position in the whole sequence
    const int64_t i = key / a.L, tt = key - i * a.L;          // its shard and row there
    const bf16* src = (const bf16*)a.shards[i] + ((b * a.L + tt) * a.H + a.h0 + h) * D + 8 * c;
    *(bf16x8*)(t + r * RS + 8 * c) = *(const bf16x8*)src;
  }
  __syncthreads();
  bf16* dst = (bf16*)a.full + ((b * a.Hn + h) * ntile + kt) * (int64_t)(D * kT);
#pragma unroll
  for (int s = tid; s < D * (kT / 8); s += kThreads) {
    const int dr = s / (kT / 8), c = s % (kT / 8);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = t[(8 * c + e) * RS + dr];
    *(bf16x8*)(dst + dr * kT + 8 * c) = o;
  }
}

}  // namespace

hipError_t launch_a2a_gather_v_tiles(const RegroupArgs& a, hipStream_t s) {
  const int64_t nwg = a.B * a.Hn * (a.S / 64);
  if (a.d == 128) a2a_gather_v_tiles_kernel<128><<<dim3((unsigned)nwg), dim3(kThreads), 0, s>>>(a);
  else a2a_gather_v_tiles_kernel<64><<<dim3((unsigned)nwg), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_a2a_gather(const RegroupArgs& a, hipStream_t s) { return launch_a2a<true>(a, s); }
hipError_t launch_a2a_scatter(const RegroupArgs& a, hipStream_t s) { return launch_a2a<false>(a, s); }

}  // namespace cpattn
