// bf16 backward kernels for gfx950: one rank's query shard against one K/V
// block, P recomputed from the forward's log-sum-exp.
//
// The backward walks the ring's blocks again and recomputes what the forward
// did not keep (compassingai.com context-parallelism page, section
// "反向傳播"); the gradients are the chain rule of the forward definition
// (same page, section "數學基礎"), per block j:
//   S = Q K_j^T * scale (masked),  P = exp(S - lse),  dP = dO V_j^T,
//   dS = P * (dP - delta) with delta = rowsum(dO * O),
//   dQ += scale dS K_j,  dK_j = scale dS^T Q,  dV_j = P^T dO.
// In base 2: P = exp2(s * scale * log2(e) - lse * log2(e)).
//
// Two kernels share the work without atomics, so results are deterministic:
//   dq   - a workgroup owns 128 query rows (4 waves x 32) and streams the key
//          tiles of the block through LDS: S^T = K Q^T and dP^T = V dO^T with
//          Q^T and dO^T held in registers (each lane one query column, as in
//          the forward kernel), dS^T from them, then dQ^T += K^T dS^T with K^T
//          read from the same LDS tile by the transpose loads;
//   dkdv - a workgroup owns 128 keys (4 waves x 32) with K and V held in
//          registers and streams the query tiles that can see them: S = Q K^T
//          and dP = dO V^T (each lane one key column), then dV^T += dO^T P and
//          dK^T += Q^T dS with dO^T and Q^T read by the transpose loads.
// Rows of Q (dkdv) or of K and V (dq) are fed to the MFMA through pi(r) (bits
// 2 and 3 swapped): accumulator elements 8h .. 8h+7 of a lane half are then 8
// consecutive rows, exactly the B operand of the next product's k-step h.
#include "kernels.h"
#include "gfx950_util.h"

#include <math.h>

namespace cpattn {
namespace {

using namespace dev;

constexpr int kThreads = 256;   // 4 waves

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(DeltaArgs a) {
  constexpr int TPR = D / 8;                       // threads per (row, head): 8 bf16 each
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.L * a.H * TPR;
  const bool ok = idx < total;                     // whole row groups are in or out together
  const int64_t rowhead = idx / TPR;               // (b * L + row) * H + h
  const int x = (int)(idx % TPR);
  float acc = 0.f;
  if (ok) {
    const bf16x8 o = *(const bf16x8*)((const bf16*)a.o + rowhead * D + 8 * x);
    const bf16x8 g = *(const bf16x8*)((const bf16*)a.d_o + rowhead * D + 8 * x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (ok && x == 0) {
    const int h = (int)(rowhead % a.H);
    const int64_t br = rowhead / a.H;
    const int64_t row = br % a.L;
    const int b = (int)(br / a.L);
    a.delta[((int64_t)b * a.H + h) * a.L + row] = acc;
  }
}

__global__ __launch_bounds__(kThreads) void zero_kernel(float* p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n4) ((float4*)p)[i] = float4{0.f, 0.f, 0.f, 0.f};
}

// base-2 log-sum-exp of a row; +inf for rows that see no key (P = 0 there)
__device__ __forceinline__ float lse2_of(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BMQ = 128;           // query rows per workgroup
  constexpr int BN = 64;             // keys per LDS tile
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int NS = D / 16;         // k-steps over the head dim
  constexpr int NDT = D / 32;        // 32-row tiles of dQ^T
  constexpr int NT = BN / 32;        // 32-key sub-tiles
  constexpr int NPV = BN / 16;       // k-steps of dQ^T = K^T dS^T
  constexpr int TILE = BN * D;

  __shared__ __attribute__((aligned(16))) bf16 smem[2][2][TILE];   // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int r32 = lane & 31;
  const int64_t L = a.L;
  const int H = a.H;

  // workgroup -> (batch, head, query tile): XCD-contiguous runs, heaviest first
  const int nqt = (int)((L + BMQ - 1) / BMQ);
  const int64_t nwg = (int64_t)nqt * H * a.B;
  const int64_t bid = blockIdx.x;
  const int64_t logical = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int64_t hb = logical / nqt;
  const int qt = nqt - 1 - (int)(logical % nqt);
  const int h = (int)(hb % H);
  const int b = (int)(hb / H);

  const int64_t rs = (int64_t)H * D;
  const int64_t base = (int64_t)b * L * rs + (int64_t)h * D;
  const bf16* __restrict__ qg = (const bf16*)a.q + base;
  const bf16* __restrict__ kg = (const bf16*)a.k + base;
  const bf16* __restrict__ vg = (const bf16*)a.v + base;
  const bf16* __restrict__ dog = (const bf16*)a.d_o + base;

  const int64_t q0 = (int64_t)qt * BMQ;
  const int64_t qrow = q0 + 32 * w + r32;
  const bool row_ok = qrow < L;
  const int64_t p = a.q_pos0 + qrow;
  const int mask = a.mask;
  const bool doc = mask == MASK_DOC_CAUSAL;
  const int64_t ml_idx = ((int64_t)b * H + h) * L + qrow;
  const int64_t st_row = ((int64_t)b * L + qrow) * rs + (int64_t)h * D;

  // key tiles the workgroup needs
  const int nkt = (int)((L + BN - 1) / BN);
  int kt_begin = 0, kt_end = nkt;
  {
    const int64_t wg_last = (q0 + BMQ < L ? q0 + BMQ : L) - 1;
    if (mask != MASK_NONE) {
      const int64_t hi = a.q_pos0 + wg_last - a.k_pos0;
      kt_end = hi < 0 ? 0 : (int)(hi / BN + 1 < nkt ? hi / BN + 1 : nkt);
      if (doc) {
        const int64_t lo = doc_start_of(a.cu, a.ndocs, a.q_pos0 + q0) - a.k_pos0;
        if (lo > 0) kt_begin = (int)(lo / BN < nkt ? lo / BN : nkt);
      }
    }
  }

  // per-wave mask thresholds (as in the forward kernel)
  const int64_t w_first = q0 + 32 * w;
  const bool wave_ok = w_first < L;
  const int64_t w_last = (w_first + 31 < L ? w_first + 31 : L - 1);
  const int64_t pw_first = a.q_pos0 + w_first, pw_last = a.q_pos0 + w_last;
  int64_t ds_last = 0, dstart = 0;
  if (doc && wave_ok) {
    ds_last = doc_start_of(a.cu, a.ndocs, pw_last);
    dstart = doc_start_of(a.cu, a.ndocs, row_ok ? p : pw_last);
  }
  const int ragged_kt = (L % BN != 0) ? nkt - 1 : -1;
  int causal_from = nkt, doc_below = 0;
  if (mask != MASK_NONE) {
    const int64_t x = pw_first - a.k_pos0 - (BN - 1);
    causal_from = x < 0 ? 0 : (int)(x / BN + 1 < nkt ? x / BN + 1 : nkt);
    if (doc) {
      const int64_t y = ds_last - a.k_pos0;
      doc_below = y <= 0 ? 0 : (int)((y + BN - 1) / BN < nkt ? (y + BN - 1) / BN : nkt);
    }
  }
  auto need_mask = [&](int kt) -> bool { return kt == ragged_kt || kt >= causal_from || kt < doc_below; };

  // Q^T and dO^T operands of this wave's 32 queries; the row's lse and delta
  bf16x8 qreg[NS], doreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (row_ok) {
      qreg[s] = *(const bf16x8*)(qg + qrow * rs + 16 * s + 8 * g);
      doreg[s] = *(const bf16x8*)(dog + qrow * rs + 16 * s + 8 * g);
    } else {
      qreg[s] = bf16x8{};
      doreg[s] = bf16x8{};
    }
  }
  const float lse2 = row_ok ? lse2_of(a.lse[ml_idx]) : INFINITY;
  const float dlt = row_ok ? a.delta[ml_idx] : 0.f;
  const float c2 = a.scale_log2;

  floatx16 dqacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dqacc[dt] = floatx16{};

  // tile fetch by all 256 threads, both tiles with the row-read swizzle
  constexpr int DMA = BN * CH / kThreads;
  constexpr int RPS = kThreads / CH;
  static_assert(DMA >= 1 && (BN * CH) % kThreads == 0 && RPS % 16 == 0, "tile fetch split");
  const int f_row = tid / CH;
  const int f_ph = tid % CH;
  const uint32_t f_off = (uint32_t)(((int64_t)f_row * rs + 8 * (f_ph ^ swz_k<D>(f_row))) * 2);
  const uint32_t smem_base = lds_addr(&smem[0][0][0]);
  auto lds_of = [&](int st, int tensor, int e) { return smem_base + (uint32_t)(((st * 2 + tensor) * TILE + e) * 2); };
  auto fetch = [&](int kt, int st) {
    if ((int64_t)(kt + 1) * BN <= L) {
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const int64_t rowoff = ((int64_t)kt * BN + i * RPS) * rs;
        const int wbase = (i * kThreads + 64 * w) * 8;
        fetch16(kg + rowoff, f_off, lds_of(st, 0, wbase));
        fetch16(vg + rowoff, f_off, lds_of(st, 1, wbase));
      }
    } else {
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        int64_t key = (int64_t)kt * BN + i * RPS + f_row;
        if (key > L - 1) key = L - 1;
        const uint32_t off = (uint32_t)((key * rs + 8 * (f_ph ^ swz_k<D>(f_row))) * 2);
        const int wbase = (i * kThreads + 64 * w) * 8;
        fetch16(kg, off, lds_of(st, 0, wbase));
        fetch16(vg, off, lds_of(st, 1, wbase));
      }
    }
  };

  const int krow_l = pi32(r32);
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // rows pi(r) of a tile as MFMA A operands, k-step s, sub-tile t
  auto rd_row = [&](const bf16* __restrict__ T, int s, int t) {
    const int row = 32 * t + krow_l;
    return *(const bf16x8*)(T + row * D + 8 * ((2 * s + g) ^ swz_k<D>(row)));
  };
  // K^T operand for key step ks, head-dim tile dt (transpose loads)
  auto rd_tr = [&](const bf16* __restrict__ T, int ks, int dt) {
    const int col = 32 * dt + tr_col;
    const int row0 = 16 * ks + 8 * g + tr_row;
    const int row1 = row0 + 4;
    const short4v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(T + row0 * D + 8 * ((col >> 3) ^ swz_k<D>(row0)) + (col & 7)));
    const short4v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(T + row1 * D + 8 * ((col >> 3) ^ swz_k<D>(row1)) + (col & 7)));
    return __builtin_bit_cast(bf16x8, short8v{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
  };

  if (kt_begin < kt_end) {
    fetch(kt_begin, 0);
    __builtin_amdgcn_s_waitcnt(0x0070);            // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    for (int u = kt_begin; u < kt_end; ++u) {
      const int st = (u - kt_begin) & 1;
      const bool more = u + 1 < kt_end;
      if (more) fetch(u + 1, st ^ 1);               // that stage was last read before the previous barrier
      const bf16* __restrict__ Ks = smem[st][0];
      const bf16* __restrict__ Vs = smem[st][1];
      floatx16 sacc[NT], pacc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        sacc[t] = floatx16{};
        pacc[t] = floatx16{};
      }
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row(Ks, s, t), qreg[s], sacc[t], 0, 0, 0);
          pacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row(Vs, s, t), doreg[s], pacc[t], 0, 0, 0);
        }
      if (need_mask(u)) {
        const int64_t kbase = (int64_t)u * BN;
        const int64_t c_lo = a.k_pos0 + kbase;
        int64_t hi64 = (L - kbase < BN ? L - kbase : BN) - 1;
        if (mask != MASK_NONE && p - c_lo < hi64) hi64 = p - c_lo;
        const int64_t lo64 = doc ? dstart - c_lo : 0;
        const int hi = (int)(hi64 < -1 ? -1 : hi64) - 8 * g;
        const int lo = (int)(lo64 < 0 ? 0 : (lo64 > BN ? BN : lo64)) - 8 * g;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ko = 32 * t + 16 * (i >> 3) + (i & 7);
            sacc[t][i] = (ko >= lo && ko <= hi) ? sacc[t][i] : -INFINITY;
          }
      }
      // dS^T = P^T (dP^T - delta), packed as the B operands of dQ^T += K^T dS^T
      bf16x8 dsb[NPV];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int i = 8 * hh + e;
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i], c2, -lse2));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i + 1], c2, -lse2));
            const bf16x2 two = __builtin_convertvector(float2v{p0 * (pacc[t][i] - dlt), p1 * (pacc[t][i + 1] - dlt)}, bf16x2);
            dsb[2 * t + hh][e] = two[0];
            dsb[2 * t + hh][e + 1] = two[1];
          }
#pragma unroll
      for (int ks = 0; ks < NPV; ++ks)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          dqacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_tr(Ks, ks, dt), dsb[ks], dqacc[dt], 0, 0, 0);
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0070);          // the next tile landed; this tile's reads are done
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    }
  }

  if (!row_ok) return;
  const float sc = a.scale;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float4* dst = (float4*)(a.dq + st_row + 32 * dt + 8 * i4 + 4 * g);
      float4 v = float4{dqacc[dt][4 * i4] * sc, dqacc[dt][4 * i4 + 1] * sc, dqacc[dt][4 * i4 + 2] * sc,
                        dqacc[dt][4 * i4 + 3] * sc};
      if (a.accumulate) {
        const float4 old = *dst;
        v = float4{old.x + v.x, old.y + v.y, old.z + v.z, old.w + v.w};
      }
      *dst = v;
    }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BK = 128;            // keys per workgroup (4 waves x 32)
  constexpr int BQ = 32;             // query rows per LDS tile
  constexpr int CH = D / 8;
  constexpr int NS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int TILE = BQ * D;

  __shared__ __attribute__((aligned(16))) bf16 smem[2][2][TILE];   // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float s_row[2][2][BQ];    // [stage][lse, delta] of the tile's rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int r32 = lane & 31;
  const int64_t L = a.L;
  const int H = a.H;

  // workgroup -> (batch, head, key tile): XCD-contiguous runs, the key tiles
  // that see the most queries first (ascending keys for the causal masks)
  const int nkt = (int)((L + BK - 1) / BK);
  const int64_t nwg = (int64_t)nkt * H * a.B;
  const int64_t bid = blockIdx.x;
  const int64_t logical = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int64_t hb = logical / nkt;
  const int kt = (int)(logical % nkt);
  const int h = (int)(hb % H);
  const int b = (int)(hb / H);

  const int64_t rs = (int64_t)H * D;
  const int64_t base = (int64_t)b * L * rs + (int64_t)h * D;
  const bf16* __restrict__ qg = (const bf16*)a.q + base;
  const bf16* __restrict__ kg = (const bf16*)a.k + base;
  const bf16* __restrict__ vg = (const bf16*)a.v + base;
  const bf16* __restrict__ dog = (const bf16*)a.d_o + base;

  const int64_t k0 = (int64_t)kt * BK;
  const int64_t key = k0 + 32 * w + r32;
  const bool key_ok = key < L;
  const int64_t c = a.k_pos0 + key;                 // this lane's global key position
  const int mask = a.mask;
  const bool doc = mask == MASK_DOC_CAUSAL;
  const int64_t st_row = ((int64_t)b * L + key) * rs + (int64_t)h * D;
  const float* __restrict__ lse_row = a.lse + ((int64_t)b * H + h) * L;
  const float* __restrict__ dl_row = a.delta + ((int64_t)b * H + h) * L;

  // K and V rows of this lane's key as B operands (K^T, V^T columns)
  bf16x8 kreg[NS], vreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (key_ok) {
      kreg[s] = *(const bf16x8*)(kg + key * rs + 16 * s + 8 * g);
      vreg[s] = *(const bf16x8*)(vg + key * rs + 16 * s + 8 * g);
    } else {
      kreg[s] = bf16x8{};
      vreg[s] = bf16x8{};
    }
  }

  // End of the document holding global position x: the first boundary
  // above x.  A query p >= c sees key c under the document mask iff
  // doc_start(p) <= c, i.e. iff p < doc_end(c).
  auto doc_end = [&](int64_t x) -> int64_t {
    int lo = 0, hi = a.ndocs;                      // cu[lo] <= x < cu[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)a.cu[mid] <= x) lo = mid; else hi = mid;
    }
    return a.cu[lo + 1];
  };
  // query rows that can see some key of the workgroup: causal from the first
  // key on, documents up to the end of the last key's document
  const int64_t c_lo = a.k_pos0 + k0;
  const int64_t c_hi = a.k_pos0 + (k0 + BK < L ? k0 + BK : L) - 1;
  int64_t q_begin = 0, q_end = L;
  if (mask != MASK_NONE) {
    q_begin = c_lo - a.q_pos0;
    if (q_begin < 0) q_begin = 0;
    if (doc) {
      const int64_t end = doc_end(c_hi) - a.q_pos0;   // first query of the next document
      if (end < q_end) q_end = end;
    }
  }
  // this lane's key: end of its document (documents only)
  const int64_t c_end = doc ? doc_end(key_ok ? c : c_hi) : 0;
  const int qt_begin = (int)(q_begin / BQ);
  const int qt_end = q_end <= q_begin ? qt_begin : (int)((q_end + BQ - 1) / BQ);

  floatx16 dkacc[NDT], dvacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    dkacc[dt] = floatx16{};
    dvacc[dt] = floatx16{};
  }
  const float c2 = a.scale_log2;

  // stage fetch, all through global->LDS loads (waited for by the kernel's own
  // vmcnt waits, never by the compiler's): the Q and dO tiles, and the rows'
  // lse and delta (4 bytes per lane, lanes 0-31 of wave 0)
  constexpr int DMA = BQ * CH / kThreads;
  constexpr int RPS = kThreads / CH;
  static_assert(DMA >= 1 && (BQ * CH) % kThreads == 0 && RPS % 16 == 0, "tile fetch split");
  const int f_row = tid / CH;
  const int f_ph = tid % CH;
  const uint32_t smem_base = lds_addr(&smem[0][0][0]);
  auto lds_of = [&](int st, int tensor, int e) { return smem_base + (uint32_t)(((st * 2 + tensor) * TILE + e) * 2); };
  auto fetch = [&](int qt, int st) {
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      int64_t row = (int64_t)qt * BQ + i * RPS + f_row;
      if (row > L - 1) row = L - 1;                 // rows past the end re-read the last row (P = 0 there)
      const uint32_t off = (uint32_t)((row * rs + 8 * (f_ph ^ swz_k<D>(f_row))) * 2);
      const int wbase = (i * kThreads + 64 * w) * 8;
      fetch16(qg, off, lds_of(st, 0, wbase));
      fetch16(dog, off, lds_of(st, 1, wbase));
    }
    if (tid < BQ) {
      int64_t qr = (int64_t)qt * BQ + tid;
      if (qr > L - 1) qr = L - 1;                   // masked below
      fetch4(lse_row, (uint32_t)(qr * 4), lds_addr(&s_row[st][0][0]));
      fetch4(dl_row, (uint32_t)(qr * 4), lds_addr(&s_row[st][1][0]));
    }
  };

  const int qrow_l = pi32(r32);
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto rd_row = [&](const bf16* __restrict__ T, int s) {
    const int row = qrow_l;
    return *(const bf16x8*)(T + row * D + 8 * ((2 * s + g) ^ swz_k<D>(row)));
  };
  auto rd_tr = [&](const bf16* __restrict__ T, int ks, int dt) {
    const int col = 32 * dt + tr_col;
    const int row0 = 16 * ks + 8 * g + tr_row;
    const int row1 = row0 + 4;
    const short4v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(T + row0 * D + 8 * ((col >> 3) ^ swz_k<D>(row0)) + (col & 7)));
    const short4v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(T + row1 * D + 8 * ((col >> 3) ^ swz_k<D>(row1)) + (col & 7)));
    return __builtin_bit_cast(bf16x8, short8v{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
  };

  // this wave's keys (uniform): the per-tile mask test
  const int64_t cw_first = a.k_pos0 + k0 + 32 * w;
  const int64_t cw_last = cw_first + 31;
  const int64_t cw_end = doc ? doc_end(cw_first) : 0;   // smallest doc_end over the wave's keys

  if (qt_begin < qt_end) {
    fetch(qt_begin, 0);
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    for (int u = qt_begin; u < qt_end; ++u) {
      const int st = (u - qt_begin) & 1;
      if (u + 1 < qt_end) fetch(u + 1, st ^ 1);
      const bf16* __restrict__ Qs = smem[st][0];
      const bf16* __restrict__ Ds = smem[st][1];
      // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys
      floatx16 sacc = floatx16{}, pacc = floatx16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row(Qs, s), kreg[s], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row(Ds, s), vreg[s], pacc, 0, 0, 0);
      }
      // Element i of lane half g is row 16 (i / 8) + 8 g + i % 8 of the tile,
      // global query p = p0 + that row.  Masked when the tile passes the end
      // of the shard, or a key of this wave comes after the tile's first
      // query (causal), or the tile reaches past the end of the document of
      // this wave's first key (documents).
      const int64_t p0 = a.q_pos0 + (int64_t)u * BQ;
      const bool ragged = (int64_t)u * BQ + BQ > L;
      const bool masked = ragged || (mask != MASK_NONE && (cw_last > p0 || (doc && p0 + BQ - 1 >= cw_end)));
      float lq[16], dq[16];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int q8 = 16 * hh + 8 * g;
        const float4 l0 = *(const float4*)&s_row[st][0][q8], l1 = *(const float4*)&s_row[st][0][q8 + 4];
        const float4 d0 = *(const float4*)&s_row[st][1][q8], d1 = *(const float4*)&s_row[st][1][q8 + 4];
        lq[8 * hh + 0] = l0.x; lq[8 * hh + 1] = l0.y; lq[8 * hh + 2] = l0.z; lq[8 * hh + 3] = l0.w;
        lq[8 * hh + 4] = l1.x; lq[8 * hh + 5] = l1.y; lq[8 * hh + 6] = l1.z; lq[8 * hh + 7] = l1.w;
        dq[8 * hh + 0] = d0.x; dq[8 * hh + 1] = d0.y; dq[8 * hh + 2] = d0.z; dq[8 * hh + 3] = d0.w;
        dq[8 * hh + 4] = d1.x; dq[8 * hh + 5] = d1.y; dq[8 * hh + 6] = d1.z; dq[8 * hh + 7] = d1.w;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) lq[i] = lse2_of(lq[i]);
      if (masked) {
        // row offset o_i = 16 (i / 8) + i % 8 from p0 + 8 g; visible iff the
        // row is inside the shard, c <= p (causal) and p < doc_end(c)
        const int64_t pg = p0 + 8 * g;
        auto clamp64 = [](int64_t x) { return (int)(x < -1 ? -1 : (x > 64 ? 64 : x)); };
        const int lim_row = clamp64(L - ((int64_t)u * BQ + 8 * g));   // o_i < lim_row
        const int lim_c = mask != MASK_NONE ? clamp64(c - pg) : -1;    // o_i >= lim_c
        const int lim_doc = doc ? clamp64(c_end - pg) : 64;            // o_i < lim_doc
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int o = 16 * (i >> 3) + (i & 7);
          const bool vis = o < lim_row && o >= lim_c && o < lim_doc;
          sacc[i] = vis ? sacc[i] : -INFINITY;
        }
      }
      bf16x8 pbp[2], pbs[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int i = 8 * hh + e;
          const float p0v = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c2, -lq[i]));
          const float p1v = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i + 1], c2, -lq[i + 1]));
          const bf16x2 pp = __builtin_convertvector(float2v{p0v, p1v}, bf16x2);
          const bf16x2 ss = __builtin_convertvector(float2v{p0v * (pacc[i] - dq[i]), p1v * (pacc[i + 1] - dq[i + 1])}, bf16x2);
          pbp[hh][e] = pp[0];
          pbp[hh][e + 1] = pp[1];
          pbs[hh][e] = ss[0];
          pbs[hh][e + 1] = ss[1];
        }
      // dV^T += dO^T P and dK^T += Q^T dS over the tile's 32 queries (2 k-steps)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_tr(Ds, hh, dt), pbp[hh], dvacc[dt], 0, 0, 0);
          dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_tr(Qs, hh, dt), pbs[hh], dkacc[dt], 0, 0, 0);
        }
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0070);          // next stage landed (loads and stores); reads done
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    }
  }

  if (!key_ok) return;
  const float sc = a.scale;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      *(float4*)(a.dk + st_row + 32 * dt + 8 * i4 + 4 * g) =
          float4{dkacc[dt][4 * i4] * sc, dkacc[dt][4 * i4 + 1] * sc, dkacc[dt][4 * i4 + 2] * sc, dkacc[dt][4 * i4 + 3] * sc};
      *(float4*)(a.dv + st_row + 32 * dt + 8 * i4 + 4 * g) =
          float4{dvacc[dt][4 * i4], dvacc[dt][4 * i4 + 1], dvacc[dt][4 * i4 + 2], dvacc[dt][4 * i4 + 3]};
    }
}

}  // namespace

hipError_t launch_bwd_delta(const DeltaArgs& a, int d, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.L * a.H * (d / 8);
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  if (d == 128) bwd_delta_kernel<128><<<grid, dim3(kThreads), 0, s>>>(a);
  else bwd_delta_kernel<64><<<grid, dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_bwd_blocks(const BwdArgs& a, int d, hipStream_t s) {
  const int64_t nq = (a.L + 127) / 128, nk = (a.L + 127) / 128;
  const dim3 gq((unsigned)(nq * a.H * a.B)), gk((unsigned)(nk * a.H * a.B));
  if (d == 128) {
    bwd_dq_kernel<128><<<gq, dim3(kThreads), 0, s>>>(a);
    bwd_dkdv_kernel<128><<<gk, dim3(kThreads), 0, s>>>(a);
  } else {
    bwd_dq_kernel<64><<<gq, dim3(kThreads), 0, s>>>(a);
    bwd_dkdv_kernel<64><<<gk, dim3(kThreads), 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  zero_kernel<<<dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(p, n4);
  return hipGetLastError();
}

}  // namespace cpattn
