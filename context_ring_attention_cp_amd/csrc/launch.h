// Launchers of the HIP kernels, called by the host API (api.cpp).  Each
// returns the hipError_t of its launch(es).  Not part of the public ABI.
#pragma once
#include "kernels.h"

namespace cpattn {

hipError_t launch_block_bf16(const BlockArgs& a, int d, hipStream_t s);
hipError_t launch_block_f32(const BlockArgs& a, int d, hipStream_t s);
// bf16 V block [B, L, H, d] -> the tiled layout F_V_TILED reads, keys L..
// filled with zeros.
hipError_t launch_v_tiles(const void* v, void* v_tiled, int64_t L, int32_t B, int32_t H, int d, hipStream_t s);
// e4m3 V codes [B, L, H, d] -> [B, H, T8, d, 128] (T8 = ceil(L / 128)), each
// 64-key half in the order the FP8 MFMA's A operand consumes keys, zero codes
// from L on.
hipError_t launch_v_tiles_fp8(const void* v, void* v_tiled, int64_t L, int32_t B, int32_t H, int d, hipStream_t s);
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
hipError_t launch_quantize_fp8(const QuantArgs& a, int d, hipStream_t s);
// FP8 (e4m3) inputs, bf16 output; the same flags and state as the bf16 kernel.
hipError_t launch_block_fp8(const BlockArgs& a, int d, hipStream_t s);
// Measurement: read `bytes` (a multiple of 4096) from src through the
// global -> LDS fetch once, discarding them (measure.hip).
hipError_t launch_lds_stream(const void* src, int64_t bytes, hipStream_t s);
// Device address and size of the static scratch on the current device
// (looked up once per device; scratch.hip).
hipError_t static_scratch(void** addr, size_t* bytes);

}  // namespace cpattn
