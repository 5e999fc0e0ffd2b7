// bf16 block kernel for gfx950: one rank's query shard against one K/V block,
// online softmax in registers, QK^T and PV on bf16 MFMA (fp32 accumulate).
//
// The recurrence is the one of the compassingai.com context-parallelism page,
// section "線上 Softmax": per block S = Q K^T * scale, masked; row max; P =
// exp(S - max); row sum; merge into the running (O, m, l) with the factor
// exp(m_old - m_new).  Here it also runs over key tiles of BN keys inside the
// block, in base 2: scores are taken as x = s * scale * log2(e), and
// exp(s*scale - m) = exp2(x - m*log2(e)).
//
// Work split: a workgroup of 8 waves (two per SIMD) owns BM = 256 query rows
// of one (batch, head); each wave owns 32 rows.  Key tiles of BN = 64 keys of
// K and V are fetched straight into LDS (global_load_lds, 16 B per lane) in a
// ring of 4 stages and shared by the 8 waves.
//
// MFMA orientation (v_mfma_f32_32x32x16_bf16, D = A x B + C, A 32x16, B 16x32):
//   S^T = K Q^T : A = K tile (rows = keys, k = head dim), B = Q^T (k = head
//                 dim, columns = this wave's 32 queries).
//   O^T = V^T P^T: A = V^T (rows = head dim, k = keys), B = P^T.
// Every lane therefore holds one query column (lane % 32) of S^T and O^T: the
// row max / row sum of the softmax are reductions over the lane's own
// registers plus one exchange with lane ^ 32, and rescaling O is per lane.
//
// Operand layouts (lane l, g = l / 32, r = l % 32):
//   A: lane holds A[r][8g .. 8g+7];  B: lane holds B[8g .. 8g+7][r];
//   C/D: lane holds D[8(i/4) + 4g + i%4][r] for i = 0..15.
// K rows are fed to A through pi(r) = r with bits 2 and 3 swapped, so that
// accumulator element i of lane-half g belongs to key 16(i/8) + 8g + i%8 of
// the 32-key sub-tile: elements 8h..8h+7 are then exactly the 8 consecutive
// keys the B operand of the PV step with k-step 2t+h needs - P^T goes from
// the S^T accumulator to the PV MFMA without any data movement.
//
// V^T comes from the row-major V tile in LDS through ds_read_b64_tr_b16:
// within each group of 16 lanes, lane lam supplies the address of 4
// consecutive elements of row base + lam/4 at column base + 4(lam%4) and
// receives the elements at column base + lam of rows base .. base+3 -
// 4 consecutive keys of one head-dim column.
//
// Tiled V (F_V_TILED, the layout the ring's receive writes): V arrives as
// [B, H, T, d, 64] (T tiles of 64 keys, each head-dim-major, zero past L), so
// a key tile of V^T is one contiguous run, fetched whole, and the A operand of
// O^T = V^T P^T (8 consecutive keys of one head-dim row) is one 16-byte LDS
// read per lane instead of two transpose loads.
//
// Overlap: the two waves of a SIMD belong to two groups that alternate MFMA
// phases and softmax phases one phase apart (see the main loop).
//
// Lazy rescaling: the exponentials use a reference max m_ref that is only
// raised (and O, l rescaled) when a tile's max exceeds it by more than 2^8;
// P <= 256 in between.  O / l is unchanged by the choice of reference; at the
// end O and l are rescaled once to the true running max, which is what the
// state and the outputs hold.
#include "launch.h"
#include "gfx950_util.h"

#include <math.h>

namespace cpattn {
namespace {

template <int V> struct IntTag { static constexpr int value = V; };

using namespace dev;


constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 32 * kWaves;   // query rows per workgroup
constexpr int BN = 64;            // keys per LDS tile
static_assert(BM == kBf16Rows && BN == kBf16Keys, "host tile constants");
constexpr int kStages = 4;        // LDS ring depth
constexpr float kLazy = 8.0f;     // log2 headroom before a rescale

// Code placement.  The main loop runs up to 3.5 % slower when it starts in the
// first half of a 32-byte instruction block (offsets 0-12 mod 32 against
// 16-28, measured on the full-block form).  The build counts where each form's
// main loop lands and sets CP_LOOP_PAD_<D>_<VT>: that many 4-byte no-ops at the
// kernel entry (run once per wave) move the loop to the offset it aims for.
#ifndef CP_LOOP_PAD_128_1
#define CP_LOOP_PAD_128_1 0
#endif
#ifndef CP_LOOP_PAD_128_0
#define CP_LOOP_PAD_128_0 0
#endif
#ifndef CP_LOOP_PAD_64_1
#define CP_LOOP_PAD_64_1 0
#endif
#ifndef CP_LOOP_PAD_64_0
#define CP_LOOP_PAD_64_0 0
#endif
#define CP_STR2(x) #x
#define CP_STR(x) CP_STR2(x)
#define CP_NOPS(n) asm volatile(".rept " CP_STR(n) "\n s_nop 0\n .endr")

template <int D, bool VT>
__device__ __forceinline__ void loop_placement() {
  if constexpr (D == 128 && VT) CP_NOPS(CP_LOOP_PAD_128_1);
  else if constexpr (D == 128) CP_NOPS(CP_LOOP_PAD_128_0);
  else if constexpr (VT) CP_NOPS(CP_LOOP_PAD_64_1);
  else CP_NOPS(CP_LOOP_PAD_64_0);
}

template <int D, bool VT>
__global__ __launch_bounds__(kThreads) void attn_block_bf16_kernel(BlockArgs a) {
  loop_placement<D, VT>();
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int NS = D / 16;         // k-steps of S^T = K Q^T
  constexpr int NDT = D / 32;        // 32-row tiles of O^T
  constexpr int NT = BN / 32;        // 32-key sub-tiles of S^T
  constexpr int NPV = BN / 16;       // k-steps of O^T = V^T P^T
  constexpr int TILE = BN * D;       // elements of one K or V tile

  __shared__ __attribute__((aligned(16))) bf16 smem[kStages][2][TILE];   // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index, uniform across the wave: everything derived from it (the
  // wave's rows, its group, its tile thresholds) stays in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int r32 = lane & 31;
  const int64_t L = a.L;
  const int H = a.H;

  // Workgroup -> (batch, head, work item).  Workgroups are dispatched to the
  // 8 XCDs round robin; the remap gives each XCD a contiguous run of logical
  // ids (one head's query tiles share its K/V in that XCD's L2).  Within a
  // head, the items with the most keys start first.  An item is a query tile,
  // or with F_SPLIT one of the two key ranges of a split tile: the nsp tiles
  // from nlo on are split, first the nsp lower key ranges (nlo tiles' worth of
  // keys each), then the unsplit tiles above the pairs, then for m = nsp .. 1
  // the upper key range of tile nlo + m - 1 and the unsplit tile m - 1 (m
  // tiles' worth of keys each, for a causal diagonal block).  With a host-given
  // order (document masks), the tiles of an XCD's heads run rank by rank
  // instead: the heaviest tile of each head first.
  const int64_t rows_end = a.rows_end;                     // rows taking part in this launch
  const int nqt = (int)((rows_end + BM - 1) / BM);
  const bool split = a.flags & F_SPLIT;
  const int nlo = split ? a.split_from : nqt;              // tiles below the split ones
  const int nsp = nqt - nlo;
  const int items = nqt + nsp;
  const int64_t nwg = (int64_t)items * H * a.B;
  const int64_t bid = blockIdx.x;
  const int64_t logical = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  int64_t hb = logical / items;
  const int it = (int)(logical % items);
  int qt = nqt - 1 - it;
  int part = 0;                                            // 1: lower key range of a split tile, 2: upper
  if (!split && a.order_n == nqt) {
    // host-given order by decreasing work; rank-major over the whole heads of an XCD
    const int64_t per = nwg / 8;
    if (nwg % 8 == 0 && per % nqt == 0) {
      const int64_t hpx = per / nqt, j = logical % per;
      hb = (logical / per) * hpx + j % hpx;
      qt = a.order[j / hpx];
    } else {
      qt = a.order[it];
    }
  }
  if (split) {
    const int extra = nlo - nsp;
    if (it < nsp) {
      part = 1;
    } else if (it - nsp < extra) {
      qt = nlo - 1 - (it - nsp);
    } else {
      const int pp = it - nsp - extra, m = nsp - pp / 2;
      qt = (pp & 1) ? m - 1 : nlo + m - 1;
      part = (pp & 1) ? 0 : 2;
    }
  }
  const int h = (int)(hb % H);
  const int b = (int)(hb / H);

  const int64_t rs = (int64_t)H * D;                        // row stride (elements)
  const int64_t base = (int64_t)b * L * rs + (int64_t)h * D;
  const bf16* __restrict__ qg = (const bf16*)a.q + base;
  const bf16* __restrict__ kg = (const bf16*)a.k + base;
  // tiled V: this head's tiles of D x BN elements, one after another
  const bf16* __restrict__ vg = (const bf16*)a.v + (VT ? ((int64_t)b * H + h) * D * v_tiled_keys(L) : base);

  const int64_t q0 = (int64_t)qt * BM;
  const int64_t qrow = q0 + 32 * w + r32;                   // this lane's query row
  const bool row_ok = qrow < L;
  const int64_t p = a.q_pos0 + qrow;                        // its global position
  const int mask = a.mask;
  const bool doc = mask == MASK_DOC_CAUSAL;

  // Key tiles this workgroup needs.
  const int nkt = (int)((L + BN - 1) / BN);
  int kt_begin = 0, kt_end = nkt;
  {
    const int64_t wg_last = (q0 + BM < rows_end ? q0 + BM : rows_end) - 1;
    if (mask != MASK_NONE) {
      const int64_t hi = a.q_pos0 + wg_last - a.k_pos0;   // last visible key (local)
      kt_end = hi < 0 ? 0 : (int)(hi / BN + 1 < nkt ? hi / BN + 1 : nkt);
      if (doc) {
        const int64_t lo = doc_start_of(a.cu, a.ndocs, a.q_pos0 + q0) - a.k_pos0;
        if (lo > 0) kt_begin = (int)(lo / BN < nkt ? lo / BN : nkt);
      }
    }
    const int split_kt = nlo * (BM / BN);
    if (part == 1 && kt_end > split_kt) kt_end = split_kt;
    if (part == 2 && kt_begin < split_kt) kt_begin = split_kt;
  }
  const bool rd = a.flags & F_READ_STATE;
  // nothing to compute and nothing to store: the state of these rows stays as
  // it is (unless a side state waits to be merged into it)
  const bool wg_final = writes_final(a.flags, (q0 + BM < rows_end ? q0 + BM : rows_end) - 1, a.final_from);
  const bool wg_side = (a.flags & F_READ_SIDE) && qt >= a.split_from;
  if (kt_begin >= kt_end && rd && !wg_final && !wg_side && !(a.flags & F_WRITE_PARTIAL)) return;

  // This wave's rows.  Every wave runs every key tile of the workgroup; tiles
  // a wave cannot see are fully masked (only the few tiles of a causal
  // diagonal band or a document edge).
  const int64_t w_first = q0 + 32 * w;
  const bool wave_ok = w_first < L;
  const int64_t w_last = (w_first + 31 < L ? w_first + 31 : L - 1);
  const int64_t pw_first = a.q_pos0 + w_first, pw_last = a.q_pos0 + w_last;
  int64_t ds_last = 0, dstart = 0;
  if (doc && wave_ok) {
    ds_last = doc_start_of(a.cu, a.ndocs, pw_last);
    dstart = doc_start_of(a.cu, a.ndocs, row_ok ? p : pw_last);
  }

  // Q^T operand for this wave's 32 queries.
  bf16x8 qreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (row_ok) qreg[s] = *(const bf16x8*)(qg + qrow * rs + 16 * s + 8 * g);
    else qreg[s] = bf16x8{};
  }

  // Running state of this lane's query (base-2 units; l is this lane half's
  // partial sum, combined with lane ^ 32 at the end).
  floatx16 oacc[NDT];
  float m_true = -INFINITY, m_ref = -INFINITY, l_run = 0.f;
  const int64_t st_row = ((int64_t)b * L + qrow) * rs + (int64_t)h * D;   // element offset of [b][qrow][h][0]
  const int64_t ml_idx = ((int64_t)b * H + h) * L + qrow;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = floatx16{};
  if (rd && row_ok) {
    m_true = m_ref = a.st_m[ml_idx] * kLog2e;
    l_run = g == 0 ? a.st_l[ml_idx] : 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 v4 = *(const float4*)(a.st_o + st_row + 32 * dt + 8 * i4 + 4 * g);
        oacc[dt][4 * i4 + 0] = v4.x;
        oacc[dt][4 * i4 + 1] = v4.y;
        oacc[dt][4 * i4 + 2] = v4.z;
        oacc[dt][4 * i4 + 3] = v4.w;
      }
  }

  const float c2 = a.scale_log2;

  // Fetch key tile kt into LDS stage st: lane n of wave w's i-th fetch fills
  // 16-byte slot (i * kThreads + 64 w + n) of the tile, i.e. row slot/CH,
  // physical chunk slot%CH, which holds logical chunk phys ^ swizzle(row).
  // Rows past the ragged end re-read row L-1 (finite data the mask drops).
  // Tiles are fetched by the 256 lanes of waves 0-3 (the first wave group).
  // Fetch i of a lane fills 16-byte slot (i * 256 + tid) of the tile: row
  // i * RPS + tid / CH, physical chunk tid % CH.  The swizzles only use row
  // bits below RPS, so every fetch of a lane reads the same logical chunk
  // offset: one 32-bit byte offset per tensor and lane, plus a uniform tile and
  // fetch offset.  Rows past the ragged end (last tile only) re-read row L-1
  // (finite data the mask drops).
  constexpr int kFetchThreads = kThreads / 2;
  constexpr int DMA = BN * CH / kFetchThreads;   // 16-byte fetches per lane per tensor per tile
  constexpr int RPS = kFetchThreads / CH;        // rows covered by one fetch of the 256 lanes
  static_assert(DMA >= 1 && (BN * CH) % kFetchThreads == 0, "tile fetch split");
  static_assert((D == 128 && RPS % 16 == 0) || (D == 64 && RPS % 16 == 0), "swizzle bits below RPS");
  // lane index within the fetching group of kFetchThreads threads (and its
  // wave within the group): the slot of a fetch never depends on which group
  // issues it
  const int f_tid = tid & (kFetchThreads - 1);
  const int f_w = w & (kFetchThreads / 64 - 1);
  const int f_row = f_tid / CH;
  const int f_ph = f_tid % CH;
  const uint32_t fk_off = (uint32_t)(((int64_t)f_row * rs + 8 * (f_ph ^ swz_k<D>(f_row))) * 2);
  const uint32_t fv_off = (uint32_t)(((int64_t)f_row * rs + 8 * (f_ph ^ swz_v<D>(f_row))) * 2);
  // LDS byte address of smem[st][tensor][e]: the stage, tensor and wave terms
  // are uniform, so the fetch destinations are scalar arithmetic.
  const uint32_t smem_base = lds_addr(&smem[0][0][0]);
  auto lds_of = [&](int st, int tensor, int e) { return smem_base + (uint32_t)(((st * 2 + tensor) * TILE + e) * 2); };
  // Tiled V: a V^T tile is D rows of BN keys (128 bytes, CHT chunks), stored
  // contiguously.  Fetch i of a lane fills V^T row i * RPST + f_tid / CHT,
  // physical chunk f_tid % CHT, with the swizzle of 128-byte rows (row bits
  // 1-3, below RPST).  Keys past L are zeros in the block itself, so every
  // tile is read whole.
  constexpr int CHT = BN / 8;
  constexpr int RPST = kFetchThreads / CHT;
  static_assert(D * CHT == BN * CH && RPST % 16 == 0, "tiled V fetch split");
  const int ft_row = f_tid / CHT;
  const uint32_t fvt_off = (uint32_t)((ft_row * BN + 8 * ((f_tid % CHT) ^ swz_k<BN>(ft_row))) * 2);
  auto fetch_vt = [&](int kt, int i, uint32_t lds) { fetch16(vg + ((int64_t)kt * D + i * RPST) * BN, fvt_off, lds); };
  auto fetch = [&](int kt, int st) {
    if ((int64_t)(kt + 1) * BN <= L) {
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const int64_t rowoff = ((int64_t)kt * BN + i * RPS) * rs;          // uniform
        const int wbase = (i * kFetchThreads + 64 * f_w) * 8;
        fetch16(kg + rowoff, fk_off, lds_of(st, 0, wbase));
        if constexpr (VT) fetch_vt(kt, i, lds_of(st, 1, wbase));
        else fetch16(vg + rowoff, fv_off, lds_of(st, 1, wbase));
      }
    } else {
      // the ragged last tile: byte offsets relative to its first row (32 bits suffice there)
      const int64_t key0 = (int64_t)kt * BN;
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const int row = i * RPS + f_row;
        const int64_t rrow = key0 + row < L ? row : L - 1 - key0;
        const int wbase = (i * kFetchThreads + 64 * f_w) * 8;
        fetch16(kg + key0 * rs, (uint32_t)((rrow * rs + 8 * (f_ph ^ swz_k<D>(f_row))) * 2), lds_of(st, 0, wbase));
        if constexpr (VT) fetch_vt(kt, i, lds_of(st, 1, wbase));
        else fetch16(vg + key0 * rs, (uint32_t)((rrow * rs + 8 * (f_ph ^ swz_v<D>(f_row))) * 2), lds_of(st, 1, wbase));
      }
    }
  };

  // Lane constants of the LDS reads.
  const int krow_l = pi32(r32);
  const int tr_row = (lane & 15) >> 2;                         // + 16 kstep + 8 g + 4 h
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32 dt

  // LDS operands of the compute phase, in the order the MFMAs consume them:
  // slots 0 .. NQK-1 are the K rows of S^T = K Q^T (head-dim step j / NT,
  // key sub-tile j % NT), slots NQK .. NQK+NPM-1 the V^T operands of
  // O^T += V^T P^T (key step k / NDT, head-dim tile k % NDT, from the
  // transpose loads).
  constexpr int NQK = NS * NT;
  constexpr int NPM = NPV * NDT;
  constexpr int RA = 6;                                        // operands read ahead of their MFMA
  auto rd_k = [&](const bf16* __restrict__ Ks, int j) {
    const int row = 32 * (j % NT) + krow_l;
    return *(const bf16x8*)(Ks + row * D + 8 * ((2 * (j / NT) + g) ^ swz_k<D>(row)));
  };
  auto rd_v = [&](const bf16* __restrict__ Vs, int k) {
    if constexpr (VT) {
      // row 32 dt + r32 of V^T (a head dim), keys 16 kstep + 8 g .. + 7: logical chunk 2 kstep + g
      const int row = 32 * (k % NDT) + r32;
      return *(const bf16x8*)(Vs + row * BN + 8 * ((2 * (k / NDT) + g) ^ swz_k<BN>(row)));
    }
    const int col = 32 * (k % NDT) + tr_col;
    const int row0 = 16 * (k / NDT) + 8 * g + tr_row;
    const int row1 = row0 + 4;
    const short4v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(Vs + row0 * D + 8 * ((col >> 3) ^ swz_v<D>(row0)) + (col & 7)));
    const short4v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v*)(Vs + row1 * D + 8 * ((col >> 3) ^ swz_v<D>(row1)) + (col & 7)));
    return __builtin_bit_cast(bf16x8, short8v{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
  };
  // The compute phase: S^T = K Q^T of one tile (QK) and O^T += V^T P^T of the
  // previous one (PV), as one stream of MFMAs.  Each MFMA's operand is read
  // RA MFMAs earlier (LDS returns in order, so the reads go out in the order
  // they are consumed, and the V reads start under the last QK MFMAs); the
  // scheduling fences keep that order.
  auto compute = [&](const bf16* __restrict__ Ks, const bf16* __restrict__ Vs, floatx16 (&sacc)[NT],
                     const bf16x8 (&pb)[NPV], auto qk_tag, auto pv_tag) {
    constexpr bool QK = decltype(qk_tag)::value != 0, PV = decltype(pv_tag)::value != 0;
    constexpr int J0 = QK ? 0 : NQK, J1 = PV ? NQK + NPM : NQK;
    auto rd = [&](int j) { return j < NQK ? rd_k(Ks, j) : rd_v(Vs, j - NQK); };
    if constexpr (QK) {
#pragma unroll
      for (int t = 0; t < NT; ++t) sacc[t] = floatx16{};
    }
    bf16x8 ring[RA];
#pragma unroll
    for (int j = J0; j < J0 + RA && j < J1; ++j) ring[j - J0] = rd(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const bf16x8 op = ring[(j - J0) % RA];
      if (j < NQK) sacc[j % NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qreg[j / NT], sacc[j % NT], 0, 0, 0);
      else oacc[(j - NQK) % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pb[(j - NQK) / NDT],
                                                                          oacc[(j - NQK) % NDT], 0, 0, 0);
      if (j + RA < J1) ring[(j - J0) % RA] = rd(j + RA);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tiles of this wave that need a mask: the ragged last tile; with a causal
  // mask the tiles from the first one holding a key after the wave's first
  // query (key k_pos0 + kt BN + BN - 1 > pw_first); with documents also the
  // tiles holding a key before the document start of the wave's last query
  // (k_pos0 + kt BN < ds_last).  Thresholds in tiles, computed once.
  const int ragged_kt = (L % BN != 0) ? nkt - 1 : -1;
  int causal_from = nkt, doc_below = 0;
  if (mask != MASK_NONE) {
    const int64_t x = pw_first - a.k_pos0 - (BN - 1);       // tile needs it when kt BN > x
    causal_from = x < 0 ? 0 : (int)(x / BN + 1 < nkt ? x / BN + 1 : nkt);
    if (doc) {
      const int64_t y = ds_last - a.k_pos0;                  // tile needs it when kt BN < y
      doc_below = y <= 0 ? 0 : (int)((y + BN - 1) / BN < nkt ? (y + BN - 1) / BN : nkt);
    }
  }
  auto need_mask = [&](int kt) -> bool { return kt == ragged_kt || kt >= causal_from || kt < doc_below; };
  auto apply_mask = [&](int kt, floatx16 (&sacc)[NT]) {
    // This lane's visible keys of the tile are the tile offsets [lo, hi]:
    // below the ragged end, not after its query (causal), not before its
    // document's first token.  Offsets are clamped to [-1, BN] before the
    // narrowing so the comparisons stay in int32; the select is branch-free.
    const int64_t kbase = (int64_t)kt * BN;
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
        const int ko = 32 * t + 16 * (i >> 3) + (i & 7);   // tile offset of element i, minus 8 g
        sacc[t][i] = (ko >= lo && ko <= hi) ? sacc[t][i] : -INFINITY;
      }
  };
  // Row max of a tile (this lane's keys; both lane halves combined).
  // Four independent chains, each folding two new values per step (v_max3).
  auto row_max = [&](floatx16 (&sacc)[NT]) -> float {
    float m[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) m[c] = sacc[0][c];
#pragma unroll
    for (int k = 4; k < 16 * NT; k += 8)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i0 = k + 2 * c, i1 = i0 + 1;
        if (i1 < 16 * NT) m[c] = fmaxf(fmaxf(m[c], sacc[i0 / 16][i0 % 16]), sacc[i1 / 16][i1 % 16]);
        else if (i0 < 16 * NT) m[c] = fmaxf(m[c], sacc[i0 / 16][i0 % 16]);
      }
    const float mx = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
    return fmaxf(mx, xor32(mx));
  };
  // Lazy rescale for a tile with row max mx (raw score units): raise the
  // reference max, and rescale O and l, only when the tile's max exceeds it
  // by more than kLazy (wave-uniform branch, rarely taken).
  auto rescale = [&](float mx) {
    const float mt = mx * c2;
    m_true = fmaxf(m_true, mt);
    const bool need = mt > m_ref + kLazy;
    if (__any(need)) {
      const float nref = need ? m_true : m_ref;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - nref) : 1.f;
      m_ref = nref;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
    }
  };
  // P = exp2(x - m_ref) of a tile, in place, summed into l; returns P packed
  // to bf16 as the four PV B operands.
  auto exp_sum = [&](floatx16 (&sacc)[NT], bf16x8 (&pb)[NPV]) {
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i], c2, -m_use));
    float part[NT * 4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        part[4 * t + q] = (sacc[t][4 * q] + sacc[t][4 * q + 1]) + (sacc[t][4 * q + 2] + sacc[t][4 * q + 3]);
#pragma unroll
    for (int n = NT * 4; n > 1; n /= 2)
#pragma unroll
      for (int q = 0; q < n / 2; ++q) part[q] = part[2 * q] + part[2 * q + 1];
    l_run += part[0];
#pragma unroll
    for (int ks = 0; ks < NPV; ++ks) {
      const int t = ks >> 1, hh = ks & 1;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const bf16x2 two = __builtin_convertvector(float2v{sacc[t][8 * hh + j], sacc[t][8 * hh + j + 1]}, bf16x2);
        pb[ks][j] = two[0];
        pb[ks][j + 1] = two[1];
      }
    }
  };
  if (kt_begin < kt_end) {
    const int grp = w >> 2;
    auto stage = [&](int u) { return (u - kt_begin) & (kStages - 1); };
    if (grp == 0) {
      fetch(kt_begin, 0);
      if (kt_begin + 1 < kt_end) fetch(kt_begin + 1, 1);
    }
    // every wave: the first two tiles (group 0) and the Q / state loads are done
    __builtin_amdgcn_s_waitcnt(0x0070);              // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    if (grp == 1) __syncthreads();                   // group 1 runs one phase behind
    floatx16 sacc[NT];
    bf16x8 pb[NPV];
    // One step u: the compute phase (QK of tile u unless u == kt_end, PV of
    // tile u-1 unless u == kt_begin), then the softmax phase of tile u.  The
    // first and last steps are peeled off the loop, so that the loop body
    // holds one form of the compute phase.
    auto step = [&](int u, auto qk_tag, auto pv_tag) {
      constexpr bool QK = decltype(qk_tag)::value != 0;
      compute(smem[stage(u)][0], smem[stage(u - 1)][1], sacc, pb, qk_tag, pv_tag);
      lds_read_barrier();
      // softmax phase; group 0 first starts the fetch of tile u+2
      const bool more = u + 2 < kt_end;
      if (grp == 0 && more) {
        fetch(u + 2, stage(u + 2));
      }
      if constexpr (QK) {
        if (need_mask(u)) apply_mask(u, sacc);
        rescale(row_max(sacc));
        exp_sum(sacc, pb);
      }
      // tile u+1 must have landed: at most the fetch of tile u+2 outstanding
      __asm__ volatile("" ::: "memory");
      if (more) __builtin_amdgcn_s_waitcnt(D == 128 ? 0x0078 : 0x0074);   // vmcnt(8 or 4) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(0x0070);                             // vmcnt(0) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    };
    step(kt_begin, IntTag<1>{}, IntTag<0>{});
    for (int u = kt_begin + 1; u < kt_end; ++u) step(u, IntTag<1>{}, IntTag<1>{});
    step(kt_end, IntTag<0>{}, IntTag<1>{});
    if (grp == 0) __syncthreads();                   // same barrier count for both groups
  }

  // Rescale O and l from the reference max to the true running max.
  if (m_true != -INFINITY && m_true != m_ref) {
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_true);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
  }

  if (!row_ok || qrow >= rows_end) return;
  if (wg_side) {
    // the other key range of a split tile: merge the two states at their common max
    const float m2 = a.side_m[ml_idx] * kLog2e;
    const float mt = fmaxf(m_true, m2);
    const float c1 = m_true == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_true - mt);
    const float c2s = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mt);
    l_run = g == 0 ? c1 * l_run + c2s * a.side_l[ml_idx] : c1 * l_run;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 v4 = *(const float4*)(a.side_o + st_row + 32 * dt + 8 * i4 + 4 * g);
        oacc[dt][4 * i4 + 0] = c1 * oacc[dt][4 * i4 + 0] + c2s * v4.x;
        oacc[dt][4 * i4 + 1] = c1 * oacc[dt][4 * i4 + 1] + c2s * v4.y;
        oacc[dt][4 * i4 + 2] = c1 * oacc[dt][4 * i4 + 2] + c2s * v4.z;
        oacc[dt][4 * i4 + 3] = c1 * oacc[dt][4 * i4 + 3] + c2s * v4.w;
      }
    m_true = mt;
  }
  const float l_tot = l_run + xor32(l_run);
  const bool has = l_tot > 0.f;
  const float m_run = m_true;

  if (writes_state(a.flags, qrow, a.final_from)) {
    // the lower key range of a split tile keeps its state on the side
    float* const so = part == 1 ? a.side_o : a.st_o;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *(float4*)(so + st_row + 32 * dt + 8 * i4 + 4 * g) =
            float4{oacc[dt][4 * i4], oacc[dt][4 * i4 + 1], oacc[dt][4 * i4 + 2], oacc[dt][4 * i4 + 3]};
    if (g == 0) {
      (part == 1 ? a.side_m : a.st_m)[ml_idx] = m_run * kLn2;
      (part == 1 ? a.side_l : a.st_l)[ml_idx] = l_tot;
    }
  }
  const float inv = has ? 1.f / l_tot : 0.f;
  // v_log_f32 is the base-2 logarithm
  const float lse = has ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  if (writes_final(a.flags, qrow, a.final_from)) {
    bf16* outp = (bf16*)a.out + st_row;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const bf16x2 lo2 = __builtin_convertvector(float2v{oacc[dt][4 * i4] * inv, oacc[dt][4 * i4 + 1] * inv}, bf16x2);
        const bf16x2 hi2 = __builtin_convertvector(float2v{oacc[dt][4 * i4 + 2] * inv, oacc[dt][4 * i4 + 3] * inv}, bf16x2);
        *(bf16x4*)(outp + 32 * dt + 8 * i4 + 4 * g) = bf16x4{lo2[0], lo2[1], hi2[0], hi2[1]};
      }
    if (g == 0) {
      if (a.m_out) a.m_out[ml_idx] = m_run * kLn2;
      if (a.l_out) a.l_out[ml_idx] = l_tot;
      if (a.lse_out) a.lse_out[ml_idx] = lse;
    }
  }
  if (a.flags & F_WRITE_PARTIAL) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *(float4*)(a.o_part + st_row + 32 * dt + 8 * i4 + 4 * g) =
            float4{oacc[dt][4 * i4] * inv, oacc[dt][4 * i4 + 1] * inv, oacc[dt][4 * i4 + 2] * inv,
                   oacc[dt][4 * i4 + 3] * inv};
    if (g == 0) a.lse_part[ml_idx] = lse;
  }
}

}  // namespace

hipError_t launch_block_bf16(const BlockArgs& a, int d, hipStream_t s, const LaunchEvents& ev) {
  const int64_t nqt = (a.rows_end + BM - 1) / BM;
  // a key split covers the upper tiles of the launch, at most half of them
  if ((a.flags & F_SPLIT) && (a.split_from >= nqt || 2 * (int64_t)a.split_from < nqt)) return hipErrorInvalidValue;
  const int64_t items = (a.flags & F_SPLIT) ? 2 * nqt - a.split_from : nqt;
  const dim3 grid((unsigned)(items * a.H * a.B)), block(kThreads);
  const bool vt = (a.flags & F_V_TILED) != 0;
  if (d == 128)
    return vt ? launch_bound(attn_block_bf16_kernel<128, true>, grid, block, s, ev, a)
              : launch_bound(attn_block_bf16_kernel<128, false>, grid, block, s, ev, a);
  return vt ? launch_bound(attn_block_bf16_kernel<64, true>, grid, block, s, ev, a)
            : launch_bound(attn_block_bf16_kernel<64, false>, grid, block, s, ev, a);
}

}  // namespace cpattn
