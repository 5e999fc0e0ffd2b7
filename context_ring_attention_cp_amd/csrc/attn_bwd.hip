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
//   dkdv - a workgroup owns 128 keys in 4 pairs of waves, 32 keys per pair,
//          and streams the query tiles that can see them.  In a pair, one
//          wave holds the keys' K rows, computes S = Q K^T and P, hands P to
//          the other through LDS and accumulates dV^T += dO^T P; the other
//          holds their V rows, computes dP = dO V^T, forms dS = P (dP - delta)
//          and accumulates dK^T += Q^T dS (each lane one key column; dO^T and
//          Q^T come from the transpose loads).  Splitting the two gradients
//          over the pair halves the accumulators of a wave, so two waves
//          share a SIMD.
// Rows of Q (dkdv) or of K and V (dq) are fed to the MFMA through pi(r) (bits
// 2 and 3 swapped): accumulator elements 8h .. 8h+7 of a lane half are then 8
// consecutive rows, exactly the B operand of the next product's k-step h.
// The LDS tiles of both kernels are read both as MFMA operand rows and by the
// transpose loads; swz_kv below keeps both patterns free of bank conflicts.
#include "launch.h"
#include "gfx950_util.h"

#include <math.h>

namespace cpattn {
namespace {

using namespace dev;

template <int V> struct IntTag { static constexpr int value = V; };

constexpr int kThreads = 256;       // 4 waves: delta, dq, zero fill
constexpr int kPairThreads = 512;   // 8 waves: dkdv

// XOR swizzle of the 16-byte chunks of a bf16 tile row of D elements.  Rows
// pi(0..15) at one chunk (operand-row reads, 16 lanes) and 4 consecutive rows
// x 4 consecutive chunks (transpose loads, 32 lanes) each land on 16
// different 16-byte bank groups (64 banks of 4 bytes; a 128-element row fills
// all of them, a 64-element row half).
template <int D> __device__ __forceinline__ int swz_kv(int row) {
  if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);
  else return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

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
  const uint32_t smem_base = lds_addr(&smem[0][0][0]);
  auto lds_of = [&](int st, int tensor, int e) { return smem_base + (uint32_t)(((st * 2 + tensor) * TILE + e) * 2); };
  // byte offsets are relative to the first row a fetch step covers (32 bits suffice there)
  const uint32_t f_off = (uint32_t)(((int64_t)f_row * rs + 8 * (f_ph ^ swz_kv<D>(f_row))) * 2);
  auto fetch = [&](int kt, int st) {
    const int64_t key0 = (int64_t)kt * BN;
    if (key0 + BN <= L) {
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const int64_t rowoff = (key0 + i * RPS) * rs;
        const int wbase = (i * kThreads + 64 * w) * 8;
        fetch16(kg + rowoff, f_off, lds_of(st, 0, wbase));
        fetch16(vg + rowoff, f_off, lds_of(st, 1, wbase));
      }
    } else {
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const int row = i * RPS + f_row;
        const int rrow = key0 + row < L ? row : (int)(L - 1 - key0);   // keys past the end re-read the last key
        const uint32_t off = (uint32_t)(((int64_t)rrow * rs + 8 * (f_ph ^ swz_kv<D>(row))) * 2);
        const int wbase = (i * kThreads + 64 * w) * 8;
        fetch16(kg + key0 * rs, off, lds_of(st, 0, wbase));
        fetch16(vg + key0 * rs, off, lds_of(st, 1, wbase));
      }
    }
  };

  const int krow_l = pi32(r32);
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // rows pi(r) of a tile as MFMA A operands, k-step s, sub-tile t
  auto rd_row = [&](const bf16* __restrict__ T, int s, int t) {
    const int row = 32 * t + krow_l;
    return *(const bf16x8*)(T + row * D + 8 * ((2 * s + g) ^ swz_kv<D>(row)));
  };
  // K^T operand for key step ks, head-dim tile dt (transpose loads)
  auto rd_tr = [&](const bf16* __restrict__ T, int ks, int dt) {
    const int col = 32 * dt + tr_col;
    const int row0 = 16 * ks + 8 * g + tr_row;
    const int row1 = row0 + 4;
    const short4v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(T + row0 * D + 8 * ((col >> 3) ^ swz_kv<D>(row0)) + (col & 7)));
    const short4v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(T + row1 * D + 8 * ((col >> 3) ^ swz_kv<D>(row1)) + (col & 7)));
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
__global__ __launch_bounds__(kPairThreads) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BK = 128;            // keys per workgroup (4 pairs x 32)
  constexpr int BQ = 32;             // query rows per LDS tile
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int NS = D / 16;         // k-steps of S and dP over the head dim
  constexpr int NDT = D / 32;        // 32-row tiles of dV^T or dK^T
  constexpr int NP = 2 * NDT;        // product MFMAs per tile (2 query steps x NDT)
  constexpr int TILE = BQ * D;
  constexpr int NSTG = 4;            // LDS ring of query tiles (fetched three tiles ahead)
  constexpr int XS = 16 * 64;        // floats of one pair's exchange slot
  constexpr int NB = 4;              // block operands in flight
  constexpr int NT = 3;              // product operands in flight
  static_assert(NB <= NS && NT <= NB && NT <= NP, "read-ahead split");

  __shared__ __attribute__((aligned(16))) bf16 smem[NSTG][2][TILE];   // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float s_row[NSTG][2][BQ];   // [stage][lse (base 2), delta] of the rows
  __shared__ __attribute__((aligned(16))) float xbuf[2][4][XS];       // [tile % 2][pair]: P

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = w & 3;              // key pair: keys 32 pr .. 32 pr + 31 of the workgroup
  const int role = w >> 2;           // 0: K rows, S, P and dV; 1: V rows, dP, dS and dK
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
  const bf16* __restrict__ dog = (const bf16*)a.d_o + base;

  const int64_t k0 = (int64_t)kt * BK;
  const int64_t key = k0 + 32 * pr + r32;
  const bool key_ok = key < L;
  const int64_t c = a.k_pos0 + key;                 // this lane's global key position
  const int mask = a.mask;
  const bool doc = mask == MASK_DOC_CAUSAL;
  const int64_t st_row = ((int64_t)b * L + key) * rs + (int64_t)h * D;
  const float* __restrict__ lse_row = a.lse + ((int64_t)b * H + h) * L;
  const float* __restrict__ dl_row = a.delta + ((int64_t)b * H + h) * L;

  // this lane's key row of K (role 0) or V (role 1) as the B operands (columns of K^T, V^T)
  const bf16* __restrict__ kvg = (const bf16*)(role == 0 ? a.k : a.v) + base;
  bf16x8 kv[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    kv[s] = key_ok ? *(const bf16x8*)(kvg + key * rs + 16 * s + 8 * g) : bf16x8{};

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
  const int nq = qt_end - qt_begin;

  floatx16 acc2[NDT];                               // dV^T (role 0) or dK^T (role 1), this pair's keys
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc2[dt] = floatx16{};
  const float c2 = a.scale_log2;

  // stage fetch, all through global->LDS loads (waited for by the kernel's own
  // vmcnt waits, never by the compiler's): the Q and dO tiles (each thread NF
  // chunks of the two tiles together), and the rows' lse and delta (4 bytes
  // per lane, lanes 0-31 of wave 0).  Byte offsets are relative to the tile's
  // first row.
  constexpr int NCH = BQ * CH;                     // 16-byte chunks of one tile
  constexpr int NF = 2 * NCH / kPairThreads;
  static_assert(NF >= 1 && (2 * NCH) % kPairThreads == 0 && NCH % 64 == 0, "tile fetch split");
  const uint32_t smem_base = lds_addr(&smem[0][0][0]);
  const uint32_t srow_base = lds_addr(&s_row[0][0][0]);
  auto fetch = [&](int qt, int st) {
    const int64_t row0 = (int64_t)qt * BQ;
    const bf16* __restrict__ q_t = qg + row0 * rs;
    const bf16* __restrict__ do_t = dog + row0 * rs;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int wc = i * kPairThreads + 64 * w;      // first chunk of this wave's 64 (wave-uniform)
      const int tensor = wc / NCH;                   // 0: Q, 1: dO
      const int e = wc - tensor * NCH + lane;        // chunk within that tile
      const int row = e / CH, ph = e % CH;
      const int rrow = row0 + row < L ? row : (int)(L - 1 - row0);   // rows past the end re-read the last row
      const uint32_t off = (uint32_t)(((int64_t)rrow * rs + 8 * (ph ^ swz_kv<D>(row))) * 2);
      fetch16(tensor == 0 ? q_t : do_t, off,
              smem_base + (uint32_t)(((st * 2 + tensor) * TILE + 8 * (wc - tensor * NCH)) * 2));
    }
    if (tid < BQ) {
      const int rr = row0 + tid < L ? tid : (int)(L - 1 - row0);      // masked below
      fetch4(lse_row + row0, (uint32_t)(rr * 4), srow_base + (uint32_t)((st * 2 + 0) * BQ * 4));
      fetch4(dl_row + row0, (uint32_t)(rr * 4), srow_base + (uint32_t)((st * 2 + 1) * BQ * 4));
    }
  };
  // Wave 0 turns the lse of a freshly fetched stage into base 2 in place
  // (+inf for rows that see no key, so that P = 0 there), once per tile,
  // after its own fetch of that stage has landed.
  auto lse_to_base2 = [&](int st) {
    if (tid < BQ) s_row[st][0][tid] = lse2_of(s_row[st][0][tid]);
  };
  auto sync = [&]() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);            // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  };
  // Wait for all but the latest stage fetch of this wave (NF tile chunks,
  // and in wave 0 the two row fetches) and for its LDS accesses.
  auto wait_but_last_fetch = [&]() {
    __asm__ volatile("" ::: "memory");
    if (w == 0) __builtin_amdgcn_s_waitcnt(0x0070 + NF + 2);   // vmcnt(NF + 2) lgkmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0x0070 + NF);              // vmcnt(NF) lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
  };
  auto barrier = [&]() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  };

  const int qrow_l = pi32(r32);
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // rows pi(r) of a query tile as MFMA A operands, k-step s
  auto rd_row = [&](const bf16* __restrict__ T, int s) {
    return *(const bf16x8*)(T + qrow_l * D + 8 * ((2 * s + g) ^ swz_kv<D>(qrow_l)));
  };
  // T^T operand for query step ks (16 rows), head-dim tile dt (transpose loads)
  auto rd_tr = [&](const bf16* __restrict__ T, int ks, int dt) {
    const int col = 32 * dt + tr_col;
    const int row0 = 16 * ks + 8 * g + tr_row;
    const int row1 = row0 + 4;
    const short4v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(T + row0 * D + 8 * ((col >> 3) ^ swz_kv<D>(row0)) + (col & 7)));
    const short4v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(T + row1 * D + 8 * ((col >> 3) ^ swz_kv<D>(row1)) + (col & 7)));
    return __builtin_bit_cast(bf16x8, short8v{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
  };

  // this pair's keys (uniform): the per-tile mask test
  const int64_t cw_first = a.k_pos0 + k0 + 32 * pr;
  const int64_t cw_last = cw_first + 31;
  const int64_t cw_end = doc ? doc_end(cw_first) : 0;   // smallest doc_end over the pair's keys

  // Tile t (query tile qt_begin + t) uses stage t % 4 and exchange slot
  // t % 2.  The loop is software-pipelined: iteration t, between the
  // barriers that end tiles t and t+1, forms the pair block of tile t+1 (S
  // then P, handed to the partner, or dP then dP - delta) while it finishes
  // tile t (dV^T from P, or dS = P (dP - delta) and dK^T).  After the barrier
  // that ends tile t, tile t+3 is fetched into the stage of tile t-1, whose
  // readers have all passed that barrier; before the next barrier every wave
  // has written its exchange values and waited for its part of the fetch of
  // tile t+2 (issued one iteration earlier), which that barrier publishes.
  auto run = [&](auto role_tag) {
    constexpr int ROLE = decltype(role_tag)::value;
    // the pair block of the tile in stage st: S = Q K^T (role 0) or dP = dO V^T (role 1)
    auto block = [&](int st) {
      const bf16* __restrict__ Xs = smem[st][ROLE];
      floatx16 acc = floatx16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row(Xs, s), kv[s], acc, 0, 0, 0);
      return acc;
    };
    // base-2 lse (role 0) or delta (role 1) of the rows of the tile in stage
    // st: element i of lane half g is row 16 (i / 8) + 8 g + i % 8
    auto rows = [&](int st, float* rv) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float4 v = *(const float4*)&s_row[st][ROLE][16 * (x >> 1) + 8 * g + 4 * (x & 1)];
        rv[4 * x] = v.x; rv[4 * x + 1] = v.y; rv[4 * x + 2] = v.z; rv[4 * x + 3] = v.w;
      }
    };
    auto own_elem = [&](const floatx16& acc, const float* rv, int i) {
      return ROLE == 0 ? __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], c2, -rv[i])) : acc[i] - rv[i];
    };
    // role 0: zero P outside the mask for query tile u.  Masked when the tile
    // passes the end of the shard, or a key of this pair comes after the
    // tile's first query (causal), or the tile reaches past the end of the
    // document of the pair's first key.
    auto mask_own = [&](int u, float* own) {
      if constexpr (ROLE == 0) {
        const int64_t p0 = a.q_pos0 + (int64_t)u * BQ;
        const bool ragged = (int64_t)u * BQ + BQ > L;
        if (ragged || (mask != MASK_NONE && (cw_last > p0 || (doc && p0 + BQ - 1 >= cw_end)))) {
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
            own[i] = (o < lim_row && o >= lim_c && o < lim_doc) ? own[i] : 0.f;
          }
        }
      }
    };
    auto put = [&](int slot, const float* own) {     // role 0: P to the other wave of the pair
      if constexpr (ROLE == 0) {
        float* __restrict__ xo = xbuf[slot][pr];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(float4*)(xo + 4 * (64 * q4 + lane)) = float4{own[4 * q4], own[4 * q4 + 1], own[4 * q4 + 2], own[4 * q4 + 3]};
      }
    };
    auto take = [&](int slot, float* pv) {            // role 1: the partner's P of a tile
      if constexpr (ROLE == 1) {
        const float* __restrict__ xi = xbuf[slot][pr];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 x = *(const float4*)(xi + 4 * (64 * q4 + lane));
          pv[4 * q4] = x.x; pv[4 * q4 + 1] = x.y; pv[4 * q4 + 2] = x.z; pv[4 * q4 + 3] = x.w;
        }
      }
    };
    // the B operands of the tile's products: P (role 0) or dS = P (dP - delta) (role 1)
    auto pack = [&](int hh, const float* own, const float* pv, bf16x8& pb) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int i = 8 * hh + e;
        const float x0 = ROLE == 0 ? own[i] : pv[i] * own[i];
        const float x1 = ROLE == 0 ? own[i + 1] : pv[i + 1] * own[i + 1];
        const bf16x2 two = __builtin_convertvector(float2v{x0, x1}, bf16x2);
        pb[e] = two[0];
        pb[e + 1] = two[1];
      }
    };
    // product f of tile t: query step f / NDT, head-dim tile f % NDT, from
    // dO^T (role 0) or Q^T (role 1)
    auto product = [&](const bf16x8& at, const bf16x8 (&pb)[2], int f) {
      acc2[f % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at, pb[f / NDT], acc2[f % NDT], 0, 0, 0);
    };

    const int q_last = qt_end - 1;
    float own[16];                                    // P (role 0) or dP - delta (role 1) of the current tile
    // Iteration t of the pipelined loop, issued in the order written: the
    // segments between scheduling fences hold one MFMA each, with the LDS
    // reads it needs issued several MFMAs earlier (LDS returns in order, so
    // reads are issued in the order they are consumed) and a share of the
    // VALU work.
    auto iter = [&](int t) {
      const int st = t % NSTG, st1 = (t + 1) % NSTG, st2 = (t + 2) % NSTG, st3 = (t + 3) % NSTG;
      const int u = qt_begin + t;
      fetch(u + 3 <= q_last ? u + 3 : q_last, st3);  // past the last tile: a harmless re-fetch into a free stage
      const bf16* __restrict__ Xs = smem[st1][ROLE];
      const bf16* __restrict__ Ts = smem[st][ROLE ^ 1];   // dO (role 0) or Q (role 1) of tile t
      bf16x8 ab[NB], tb[NT], pb[2];
      float pv[16], rv[16];
#pragma unroll
      for (int s = 0; s < NB; ++s) ab[s] = rd_row(Xs, s);
      take(t & 1, pv);
      __builtin_amdgcn_sched_barrier(0);
      // the block of tile t+1; its last steps issue the first transpose reads
      // and pack the products' B operands of tile t
      floatx16 acc = floatx16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[s % NB], kv[s], acc, 0, 0, 0);
        if (s + NB < NS) ab[s % NB] = rd_row(Xs, s + NB);
        else if (s + NB - NS < NT) tb[s + NB - NS] = rd_tr(Ts, (s + NB - NS) / NDT, (s + NB - NS) % NDT);
        if (s >= NS - 2) pack(s - (NS - 2), own, pv, pb[s - (NS - 2)]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the products of tile t; the rows of tile t+1 are read after the
      // first, and its P or dP - delta is formed a few elements per product
#pragma unroll
      for (int f = 0; f < NP; ++f) {
        product(tb[f % NT], pb, f);
        if (f + NT < NP) tb[f % NT] = rd_tr(Ts, (f + NT) / NDT, (f + NT) % NDT);
        if (f == 0) rows(st1, rv);
        constexpr int per = (16 + NP - 3) / (NP - 2);
        if (f >= 2) {
#pragma unroll
          for (int i = per * (f - 2); i < per * (f - 1) && i < 16; ++i) {
            own[i] = own_elem(acc, rv, i);
            __asm__ volatile("" : "+v"(own[i]));    // keeps the arithmetic in this segment
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mask_own(u + 1, own);
      put((t + 1) & 1, own);
      wait_but_last_fetch();
      lse_to_base2(st2);
      barrier();
    };

    fetch(qt_begin, 0);
    if (nq > 1) fetch(qt_begin + 1, 1);
    if (nq > 2) fetch(qt_begin + 2, 2);
    __builtin_amdgcn_s_waitcnt(0x0070);
    lse_to_base2(0);                                 // (stage 1 unused when nq == 1; tile 2 is
    lse_to_base2(1);                                 // converted at the end of iteration 0)
    sync();
    {
      float rv[16];
      rows(0, rv);
      const floatx16 acc = block(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) own[i] = own_elem(acc, rv, i);
      mask_own(qt_begin, own);
      put(0, own);
    }
    sync();
    for (int t = 0; t + 1 < nq; ++t) iter(t);
    // the last tile's products
    {
      const int st = (nq - 1) % NSTG;
      const bf16* __restrict__ Ts = smem[st][ROLE ^ 1];
      float pv[16];
      bf16x8 pb[2];
      take((nq - 1) & 1, pv);
      pack(0, own, pv, pb[0]);
      pack(1, own, pv, pb[1]);
#pragma unroll
      for (int f = 0; f < NP; ++f) product(rd_tr(Ts, f / NDT, f % NDT), pb, f);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);              // no fetch may still write this workgroup's LDS at exit
  };
  if (nq > 0) {
    if (role == 0) run(IntTag<0>{});
    else run(IntTag<1>{});
  }

  if (!key_ok) return;
  // role 0 holds dV^T, role 1 dK^T (scaled here): lane element i of tile dt is
  // head dim 32 dt + 8 (i / 4) + 4 g + i % 4 of this lane's key
  float* __restrict__ out = (role == 0 ? a.dv : a.dk) + st_row;
  const float sc = role == 0 ? 1.f : a.scale;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      *(float4*)(out + 32 * dt + 8 * i4 + 4 * g) =
          float4{acc2[dt][4 * i4] * sc, acc2[dt][4 * i4 + 1] * sc, acc2[dt][4 * i4 + 2] * sc, acc2[dt][4 * i4 + 3] * sc};
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
    bwd_dkdv_kernel<128><<<gk, dim3(kPairThreads), 0, s>>>(a);
  } else {
    bwd_dq_kernel<64><<<gq, dim3(kThreads), 0, s>>>(a);
    bwd_dkdv_kernel<64><<<gk, dim3(kPairThreads), 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  zero_kernel<<<dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(p, n4);
  return hipGetLastError();
}

}  // namespace cpattn
