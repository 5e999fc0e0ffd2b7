// Device helpers shared by the gfx950 attention kernels (forward and
// backward): bf16 vector types, LDS tile swizzles, the MFMA row permutation,
// document lookup, the half-wave exchange, LDS barriers and the global->LDS
// fetch.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {
namespace dev {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;

// 16-byte chunk swizzles of a bf16 tile row of D elements in LDS (XOR on the
// chunk index within the row).  swz_k suits reads of MFMA operand rows (16
// lanes at 16 different rows, one logical chunk); swz_v suits the transpose
// loads (4 rows x 4 chunks per 32 lanes).  Any tile may use either: the
// writer and the readers only have to agree.
template <int D> __device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128) return row & 15;          // 256-B rows: chunk alone picks the bank
  else return (row >> 1) & 7;                       // 128-B rows: row parity picks the half
}
template <int D> __device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 128) return 4 * (row & 3);
  else return 4 * ((row >> 1) & 1);
}

__device__ __forceinline__ int pi32(int r) {      // swap bits 2 and 3
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ int64_t doc_start_of(const int32_t* __restrict__ cu, int ndocs, int64_t p) {
  int lo = 0, hi = ndocs;                           // cu[lo] <= p < cu[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)cu[mid] <= p) lo = mid; else hi = mid;
  }
  return cu[lo];
}

// Value of lane ^ 32 (v_permlane32_swap exchanges the two 32-lane halves).
__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  // r[0]: lanes 0-31 keep x, lanes 32-63 get lanes 0-31 of x; r[1]: lanes 0-31
  // get lanes 32-63 of x, lanes 32-63 keep x.  The half that moved is the partner's.
  const unsigned lo_half_kept = r[0], hi_half_moved = r[1];
  const bool upper = (__lane_id() & 32) != 0;
  return __builtin_bit_cast(float, upper ? lo_half_kept : hi_half_moved);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Workgroup barrier that waits only for this wave's LDS reads (lgkmcnt(0)),
// not for its in-flight global->LDS fetches: used where the fetched stage is
// not read in the next phase.  The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_read_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt and expcnt at their maximum, lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// One 16-byte global -> LDS fetch per lane (global_load_lds_dwordx4): lane n's
// data lands at lds + 16 n (lds wave-uniform, through M0), read from
// base + off (base wave-uniform, off per lane).  Written as inline assembly so
// that the compiler does not track it: the kernel itself waits for the fetches
// (vmcnt) before the barrier that publishes a stage, and the compiler
// therefore never places a full vmcnt(0) wait in front of LDS reads of other
// stages.
__device__ __forceinline__ void fetch16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
// One 4-byte global -> LDS fetch per active lane (global_load_lds_dword):
// lane n's data lands at lds + 4 n; otherwise as fetch16.
__device__ __forceinline__ void fetch4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base),
               "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace dev
}  // namespace cpattn
