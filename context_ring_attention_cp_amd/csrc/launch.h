// Launchers of the HIP kernels, called by the host API (api.cpp).  Each
// returns the hipError_t of its launch(es).  Not part of the public ABI.
#pragma once
#include "kernels.h"

#include <hip/hip_ext.h>

#include <tuple>

namespace cpattn {

// Events bound to one kernel dispatch (hipExtLaunchKernel): `start` and `stop`
// take that dispatch's own begin and end, so timing a kernel, or making another
// stream wait for it, adds no marker packet to the stream (each marker between
// two dependent kernels costs several microseconds of idle time).  Either may
// be null.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launch kernel<<<grid, block, 0, s>>>(args...) with the events of `ev` bound;
// each argument is converted to the kernel's parameter type first.
template <typename... P, typename... A>
inline hipError_t launch_bound(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, const LaunchEvents& ev,
                               const A&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  std::tuple<P...> vals{static_cast<P>(args)...};
  return std::apply(
      [&](auto&... v) {
        void* argv[] = {(void*)&v...};
        return hipExtLaunchKernel((const void*)kernel, grid, block, argv, 0, s, ev.start, ev.stop, 0);
      },
      vals);
}

hipError_t launch_block_bf16(const BlockArgs& a, int d, hipStream_t s, const LaunchEvents& ev = {});
hipError_t launch_block_f32(const BlockArgs& a, int d, hipStream_t s, const LaunchEvents& ev = {});
// bf16 V block [B, L, H, d] -> the tiled layout F_V_TILED reads, keys L..
// filled with zeros.
hipError_t launch_v_tiles(const void* v, void* v_tiled, int64_t L, int32_t B, int32_t H, int d, hipStream_t s,
                          const LaunchEvents& ev = {});
// e4m3 V codes [B, L, H, d] -> [B, H, T8, d, 128] (T8 = ceil(L / 128)), each
// 64-key half in the order the FP8 MFMA's A operand consumes keys, zero codes
// from L on.
hipError_t launch_v_tiles_fp8(const void* v, void* v_tiled, int64_t L, int32_t B, int32_t H, int d, hipStream_t s,
                              const LaunchEvents& ev = {});
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);
hipError_t launch_bwd_delta(const DeltaArgs& a, int d, hipStream_t s);
hipError_t launch_bwd_blocks(const BwdArgs& a, int d, hipStream_t s);   // dq kernel, then dk/dv kernel
hipError_t launch_zero(float* p, int64_t n, hipStream_t s);            // n a multiple of 4
hipError_t launch_a2a_gather(const RegroupArgs& a, hipStream_t s);
hipError_t launch_a2a_scatter(const RegroupArgs& a, hipStream_t s);
// The gather of bf16 V straight into the tiled layout F_V_TILED reads, over the
// whole sequence: full = [B, Hn, S / 64, d, 64]; S a multiple of 64.
hipError_t launch_a2a_gather_v_tiles(const RegroupArgs& a, hipStream_t s);
// x is multiplied by prescale (float32) before it is quantised.
hipError_t launch_quantize_fp8(const QuantArgs& a, int d, float prescale, hipStream_t s);
// FP8 (e4m3) inputs, bf16 output; the same flags and state as the bf16 kernel.
hipError_t launch_block_fp8(const BlockArgs& a, int d, hipStream_t s, const LaunchEvents& ev = {});
// Measurement: read `bytes` (a multiple of 4096) from src through the
// global -> LDS fetch once, discarding them (measure.hip).
hipError_t launch_lds_stream(const void* src, int64_t bytes, hipStream_t s);
// Device address and size of the static scratch on the current device
// (looked up once per device; scratch.hip).
hipError_t static_scratch(void** addr, size_t* bytes);

}  // namespace cpattn
