// Tiled copy of a bf16 V block, written by the simulated ring receive:
// [B, L, H, d] -> [B, H, T, d, 64] with T = ceil(L / 64) tiles of 64 keys,
// each tile head-dim-major (d rows of 64 consecutive keys), zeros for keys
// from L on.  A key tile of V^T is then one contiguous run (16 KiB at
// d = 128) that the attention kernel fetches into LDS as it is, and the A
// operand of O^T = V^T P^T (8 consecutive keys of one head dim) is one 16-byte
// LDS read per lane.  In a real ring the owner of a block would write this
// layout once and the block would travel in it; here the layout change is
// fused into the receive copy.  HBM-bound: 2 d bytes read and written per key
// and head.
//
// e4m3 codes (the FP8 ring): [B, L, H, d] bytes -> [B, H, T8, d, 128], T8 =
// ceil(L / 128) tiles of 128 keys, each head-dim-major, zero codes from L on,
// and within each 64-key half key 16 q + 8 g + e stored at position
// 32 g + 8 q + e: the order in which the FP8 MFMA's A operand consumes keys
// (byte e of lane half g stands for key 16 (e / 8) + 8 g + e % 8), so the 32
// bytes of a lane half are contiguous.
#include "launch.h"
#include "gfx950_util.h"

namespace cpattn {
namespace {

using namespace dev;

constexpr int kTile = 64;        // keys per workgroup
constexpr int kThreadsT = 256;

// One workgroup per (batch, head, 64-key tile): the tile's 64 rows of d
// elements go through LDS (rows padded by 16 bytes), then every lane writes
// 16-byte runs of 8 consecutive keys of one head-dim row.
template <int D>
__global__ __launch_bounds__(kThreadsT) void v_tiles_kernel(const bf16* __restrict__ v, bf16* __restrict__ vt,
                                                           int64_t L, int H) {
  constexpr int CH = D / 8;                 // 16-byte chunks of a key row
  constexpr int RS = D + 8;                 // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) bf16 t[kTile * RS];
  const int64_t ntile = v_tiled_keys(L) / kTile;
  const int64_t bid = blockIdx.x;
  const int64_t kt = bid % ntile;
  const int64_t hb = bid / ntile;
  const int h = (int)(hb % H);
  const int64_t b = hb / H;
  const int tid = threadIdx.x;
#pragma unroll
  for (int s = tid; s < kTile * CH; s += kThreadsT) {
    const int r = s / CH, c = s % CH;
    const int64_t key = kt * kTile + r;
    bf16x8 x = {};
    if (key < L) x = *(const bf16x8*)(v + ((b * L + key) * H + h) * D + 8 * c);
    *(bf16x8*)(t + r * RS + 8 * c) = x;
  }
  __syncthreads();
  bf16* dst = vt + ((b * H + h) * ntile + kt) * (int64_t)(D * kTile);
#pragma unroll
  for (int s = tid; s < D * (kTile / 8); s += kThreadsT) {
    const int dr = s / (kTile / 8), c = s % (kTile / 8);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = t[(8 * c + e) * RS + dr];
    *(bf16x8*)(dst + dr * kTile + 8 * c) = o;
  }
}

// One workgroup per (batch, head, 128-key tile) of e4m3 codes: the tile's 128
// rows of d bytes go through LDS (rows padded by 16 bytes), then every lane
// writes 16 bytes (positions 16 c .. 16 c + 15) of one head-dim row.
template <int D>
__global__ __launch_bounds__(kThreadsT) void v_tiles_fp8_kernel(const uint8_t* __restrict__ v,
                                                               uint8_t* __restrict__ vt, int64_t L, int H) {
  constexpr int kT8 = 128;                  // keys per tile
  constexpr int CH = D / 16;                // 16-byte chunks of a key row
  constexpr int RS = D + 16;                // padded LDS row (bytes)
  __shared__ __attribute__((aligned(16))) uint8_t t[kT8 * RS];
  const int64_t ntile = (L + kT8 - 1) / kT8;
  const int64_t bid = blockIdx.x;
  const int64_t kt = bid % ntile;
  const int64_t hb = bid / ntile;
  const int h = (int)(hb % H);
  const int64_t b = hb / H;
  const int tid = threadIdx.x;
#pragma unroll
  for (int s = tid; s < kT8 * CH; s += kThreadsT) {
    const int r = s / CH, c = s % CH;
    const int64_t key = kt * kT8 + r;
    uint4 x = {0u, 0u, 0u, 0u};
    if (key < L) x = *(const uint4*)(v + ((b * L + key) * H + h) * D + 16 * c);
    *(uint4*)(t + r * RS + 16 * c) = x;
  }
  __syncthreads();
  uint8_t* dst = vt + ((b * H + h) * ntile + kt) * (int64_t)(D * kT8);
#pragma unroll
  for (int s = tid; s < D * (kT8 / 16); s += kThreadsT) {
    const int dr = s / (kT8 / 16), c = s % (kT8 / 16);
    uint32_t wd[4];
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      uint32_t acc = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int j = 4 * w4 + bb;                      // byte of the 16
        const int pos = 16 * c + j;                     // position in the tile row
        const int kh = pos >> 6, within = pos & 63;
        const int g = within >> 5, q = (within & 31) >> 3, e = within & 7;
        const int key = 64 * kh + 16 * q + 8 * g + e;
        acc |= (uint32_t)t[key * RS + dr] << (8 * bb);
      }
      wd[w4] = acc;
    }
    *(uint4*)(dst + dr * kT8 + 16 * c) = uint4{wd[0], wd[1], wd[2], wd[3]};
  }
}

}  // namespace

hipError_t launch_v_tiles(const void* v, void* v_tiled, int64_t L, int32_t B, int32_t H, int d, hipStream_t s,
                          const LaunchEvents& ev) {
  const dim3 grid((unsigned)(v_tiled_keys(L) / kTile * H * B)), block(kThreadsT);
  const bf16* src = (const bf16*)v;
  bf16* dst = (bf16*)v_tiled;
  return d == 128 ? launch_bound(v_tiles_kernel<128>, grid, block, s, ev, src, dst, L, H)
                  : launch_bound(v_tiles_kernel<64>, grid, block, s, ev, src, dst, L, H);
}

hipError_t launch_v_tiles_fp8(const void* v, void* v_tiled, int64_t L, int32_t B, int32_t H, int d, hipStream_t s,
                              const LaunchEvents& ev) {
  const dim3 grid((unsigned)((L + 127) / 128 * H * B)), block(kThreadsT);
  const uint8_t* src = (const uint8_t*)v;
  uint8_t* dst = (uint8_t*)v_tiled;
  return d == 128 ? launch_bound(v_tiles_fp8_kernel<128>, grid, block, s, ev, src, dst, L, H)
                  : launch_bound(v_tiles_fp8_kernel<64>, grid, block, s, ev, src, dst, L, H);
}

}  // namespace cpattn
