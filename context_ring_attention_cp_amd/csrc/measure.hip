// Measurement helper: a read-only stream through the global -> LDS fetch
// (global_load_lds_dwordx4, 16 bytes per lane) that the attention kernels use
// for their K/V tiles.  It reads a given number of bytes once and discards
// them in a small LDS ring, so a hardware counter of HBM bytes fetched
// (rocprofv3 FETCH_SIZE) read for this kernel calibrates the same counter
// read for the attention kernels.
#include "launch.h"
#include "gfx950_util.h"

namespace cpattn {
namespace {

using namespace dev;

constexpr int kThreadsS = 256;
constexpr int kChunk = kThreadsS * 16;        // bytes of one fetch of the workgroup
constexpr int kRing = 4;                      // LDS chunks the fetches rotate over

__global__ __launch_bounds__(kThreadsS) void lds_stream_kernel(const uint8_t* __restrict__ src, int64_t chunks) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing][kChunk];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t off = (uint32_t)(threadIdx.x * 16);           // lane n of wave w reads bytes 16 (64 w + n)
  const uint32_t lds0 = lds_addr(&ring[0][0]) + (uint32_t)(w * 64 * 16);
  int slot = 0;
  for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    fetch16(src + c * kChunk, off, lds0 + (uint32_t)(slot * kChunk));
    slot = (slot + 1) & (kRing - 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);                        // vmcnt(0): no fetch outlives the workgroup
}

}  // namespace

hipError_t launch_lds_stream(const void* src, int64_t bytes, hipStream_t s) {
  const int64_t chunks = bytes / kChunk;
  const int64_t wgs = chunks < 4096 ? chunks : 4096;
  lds_stream_kernel<<<dim3((unsigned)wgs), dim3(kThreadsS), 0, s>>>((const uint8_t*)src, chunks);
  return hipGetLastError();
}

}  // namespace cpattn
