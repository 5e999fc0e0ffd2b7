// FP8 (OCP e4m3) block kernel for gfx950: one rank's query shard against one
// K/V block, Q, K and V given as e4m3 codes with one power-of-two float32
// scale per (batch, head) each (value = decode(code) * scale; the query's
// codes also carry the softmax scale times log2(e)), the output in bf16.
//
// The recurrence, work split, wave ping-pong, LDS ring, fetch schedule, masks
// and lazy rescaling are those of the bf16 kernel (attn_mfma.hip); the online
// softmax follows the compassingai.com context-parallelism page, section
// "線上 Softmax".  That page also notes that the bytes CP moves depend on FP8
// transfer (section "通訊量分析") and that FlashAttention-3 computes in FP8
// (section "技術演進史").  What differs:
//
// Products on v_mfma_f32_32x32x64_f8f6f4 (both operands e4m3): A 32 x 64,
// B 64 x 32, each lane holding 32 bytes (8 VGPRs).  The instruction pairs
// byte e of lane half g of A with byte e of lane half g of B (one k each), and
// its accumulator layout is the bf16 one: lane holds D[8(i/4) + 4g + i%4][r].
//   S^T = K Q^T: A = K rows (through pi, as in bf16), bytes e of half g = head
//     dims 64 s + 32 g + e; B = Q^T from registers with the same head dims.
//     The two sub-tiles' accumulators hold keys 32 t + 16(i/8) + 8g + i%8.
//   O^T += V^T P^T (64 keys per MFMA, one per head-dim tile and key half):
//     byte e of half g stands for key 16(e/8) + 8g + e%8 of the 64-key half.
//     B = P^T is then simply two S^T accumulators converted to e4m3 in order
//     (bytes 0-15 from sub-tile 2h, 16-31 from sub-tile 2h+1); A = V^T comes
//     from four ds_read_b64_tr_b8 of the row-major V tile: within 16 lanes,
//     lane s addresses row base + s/2 at column base + 8(s%2), and lane l
//     receives column base + l of the 8 rows base .. base+7 (measured on the
//     device with an index-filled LDS probe).
// Tiled V (F_V_TILED, the layout the ring's receive writes): V arrives as
//   [B, H, T, d, 128] (T tiles of 128 keys, each tile head-dim-major, zero
//   past L), with the keys of each 64-key half stored in the order the A
//   operand consumes them (key 16 q + 8 g + e at position 32 g + 8 q + e), so
//   the 32 bytes of lane half g are contiguous: two 16-byte LDS reads per
//   operand instead of four transpose loads.
// Scales: the S^T products run as v_mfma_scale_f32_32x32x64_f8f6f4 with the
//   key block's and the query's exponents as the e8m0 block scales (powers
//   of two, applied exactly), and the query's codes already hold the softmax
//   scale times log2(e): the accumulators are the base-2 logits x.  The O
//   accumulator holds sum P V_codes, so the running state is divided by s_v
//   on load and O multiplied by s_v before it is stored.
// P = exp2(x - m_ref) with an integer reference m_ref: v_exp_f32 of x itself,
//   and the e4m3 conversion v_cvt_scalef32_pk_fp8_f32 divides by 2^m_ref
//   (it uses the exponent of its scale operand; both steps exact as powers of
//   two), so the softmax issues no multiply-add per score.  That needs
//   2^(m_ref + 8) and 2^(m_ref - 10) to be normal float32 values (P below
//   2^-10 rounds to code 0 either way): for -116 <= m_ref <= 119 in every
//   lane of the wave; otherwise the wave subtracts m_ref first and converts
//   with scale 1.
// P is rounded to e4m3 for the PV product (P <= 256 under the lazy rescale, so
//   it never reaches the 448 limit); l sums the same rounded values, so O / l
//   stays a convex combination of V rows.  The row sums come from the matrix
//   core as well: one more MFMA per tile with an all-ones A operand
//   (1.0 = code 0x38) and a P^T operand leaves sum_k P[q][k] in every
//   accumulator element of query q's lanes.  That MFMA falls in the compute
//   phase and saves the softmax the decode and the adds of 32 values per lane
//   per tile.
// Tiles are 128 keys x d bytes (16 KiB at d = 128), 4 stages, 128 KiB of LDS:
//   with FP8 products a 64-key tile is too little work per phase to carry the
//   phase's fixed costs (barriers, waits, the row max exchange); 128-key tiles
//   were 5 % faster on the same device.  The operands are read 2 MFMAs ahead,
//   which keeps the kernel within 256 VGPRs.
#include "launch.h"
#include "gfx950_util.h"

#include <math.h>

namespace cpattn {
namespace {

using namespace dev;

template <int V> struct Tag { static constexpr int value = V; };

typedef int int8v __attribute__((ext_vector_type(8)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef short short2v __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 32 * kWaves;   // query rows per workgroup
constexpr int BN = 128;           // keys per LDS tile
constexpr int kStages = 4;        // LDS ring depth
constexpr float kLazy = 8.0f;     // log2 headroom before a rescale

// XOR swizzle of the 16-byte chunks of an e4m3 tile row of D bytes.  Operand
// rows (16 lanes at rows pi(0..15), one chunk) and the 8-bit transpose loads
// (8 consecutive rows x 2 consecutive chunks per 32 lanes) each touch 16
// different 16-byte bank groups.
template <int D> __device__ __forceinline__ int swz8(int row) {
  if constexpr (D == 128) return (row >> 1) & 7;    // 2 rows per 256 bytes
  else return (row >> 2) & 3;                       // 4 rows per 256 bytes
}

__device__ __forceinline__ floatx16 mfma8(const int8v& a, const int8v& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same product scaled by 2^(byte 0 of sc - 127) for A and 2^(byte 1 of
// sc - 127) for B (e8m0 block scales, one register for both).
__device__ __forceinline__ floatx16 mfma8_scaled(const int8v& a, const int8v& b, const floatx16& c, int sc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sc, 1, sc);
}

// e8m0 code of a power-of-two float32 (its biased exponent)
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xFF); }

// Code placement, as for the bf16 kernel: the build sets
// CP_F8_LOOP_PAD_<D>_<VT>, the number of 4-byte no-ops at the kernel entry
// that put the main loop at the offset within a 32-byte instruction block it
// aims for (the full-block form ran 8.65 ms per launch at offset 28 against
// 8.78-8.89 ms at the seven other offsets on one machine, two rounds; on a
// faster machine offsets 4 and 28 were within 0.5 % of each other).
#ifndef CP_F8_LOOP_PAD_128_1
#define CP_F8_LOOP_PAD_128_1 0
#endif
#ifndef CP_F8_LOOP_PAD_128_0
#define CP_F8_LOOP_PAD_128_0 0
#endif
#ifndef CP_F8_LOOP_PAD_64_1
#define CP_F8_LOOP_PAD_64_1 0
#endif
#ifndef CP_F8_LOOP_PAD_64_0
#define CP_F8_LOOP_PAD_64_0 0
#endif
#define CP_F8_STR2(x) #x
#define CP_F8_STR(x) CP_F8_STR2(x)
#define CP_F8_NOPS(n) asm volatile(".rept " CP_F8_STR(n) "\n s_nop 0\n .endr")

template <int D, bool VT>
__device__ __forceinline__ void loop_placement_fp8() {
  if constexpr (D == 128 && VT) CP_F8_NOPS(CP_F8_LOOP_PAD_128_1);
  else if constexpr (D == 128) CP_F8_NOPS(CP_F8_LOOP_PAD_128_0);
  else if constexpr (VT) CP_F8_NOPS(CP_F8_LOOP_PAD_64_1);
  else CP_F8_NOPS(CP_F8_LOOP_PAD_64_0);
}

template <int D, bool VT>
__global__ __launch_bounds__(kThreads) void attn_block_fp8_kernel(BlockArgs a) {
  loop_placement_fp8<D, VT>();
  constexpr int CH = D / 16;         // 16-byte chunks per row
  constexpr int NS = D / 64;         // k-steps of S^T = K Q^T
  constexpr int NDT = D / 32;        // 32-row tiles of O^T
  constexpr int NT = BN / 32;        // 32-key sub-tiles of S^T
  constexpr int NH = BN / 64;        // 64-key halves: one P^T operand each (two sub-tiles)
  constexpr int TILE = BN * D;       // bytes of one K or V tile
  static_assert(NT == 2 * NH, "P^T operands built from pairs of 32-key sub-tiles");

  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages][2][TILE];   // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int r32 = lane & 31;
  const int64_t L = a.L;
  const int H = a.H;

  const int64_t rows_end = a.rows_end;                     // rows taking part in this launch
  const int nqt = (int)((rows_end + BM - 1) / BM);
  const int64_t nwg = (int64_t)nqt * H * a.B;
  const int64_t bid = blockIdx.x;
  const int64_t logical = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int64_t hb = logical / nqt;
  const int qt = nqt - 1 - (int)(logical % nqt);
  const int h = (int)(hb % H);
  const int b = (int)(hb / H);

  const int64_t rs = (int64_t)H * D;                        // row stride (bytes = elements)
  const int64_t base = (int64_t)b * L * rs + (int64_t)h * D;
  const uint8_t* __restrict__ qg = (const uint8_t*)a.q + base;
  const uint8_t* __restrict__ kg = (const uint8_t*)a.k + base;
  // tiled V: this head's tiles of D x BN bytes, one after another
  const int64_t nkt_all = (L + BN - 1) / BN;
  const uint8_t* __restrict__ vg = (const uint8_t*)a.v + (VT ? ((int64_t)b * H + h) * D * nkt_all * BN : base);
  const int bh = b * H + h;
  const int sc_kq = e8m0_of(a.k_scale[bh]) | (e8m0_of(a.q_scale[bh]) << 8);
  const float s_v = a.v_scale[bh];

  const int64_t q0 = (int64_t)qt * BM;
  const int64_t qrow = q0 + 32 * w + r32;
  const bool row_ok = qrow < L;
  const int64_t p = a.q_pos0 + qrow;
  const int mask = a.mask;
  const bool doc = mask == MASK_DOC_CAUSAL;

  const int nkt = (int)((L + BN - 1) / BN);
  int kt_begin = 0, kt_end = nkt;
  {
    const int64_t wg_last = (q0 + BM < rows_end ? q0 + BM : rows_end) - 1;
    if (mask != MASK_NONE) {
      const int64_t hi = a.q_pos0 + wg_last - a.k_pos0;
      kt_end = hi < 0 ? 0 : (int)(hi / BN + 1 < nkt ? hi / BN + 1 : nkt);
      if (doc) {
        const int64_t lo = doc_start_of(a.cu, a.ndocs, a.q_pos0 + q0) - a.k_pos0;
        if (lo > 0) kt_begin = (int)(lo / BN < nkt ? lo / BN : nkt);
      }
    }
  }
  const bool rd = a.flags & F_READ_STATE;
  // nothing to compute and nothing to store: the state of these rows stays as it is
  const bool wg_final = writes_final(a.flags, (q0 + BM < rows_end ? q0 + BM : rows_end) - 1, a.final_from);
  if (kt_begin >= kt_end && rd && !wg_final && !(a.flags & F_WRITE_PARTIAL)) return;

  const int64_t w_first = q0 + 32 * w;
  const bool wave_ok = w_first < L;
  const int64_t w_last = (w_first + 31 < L ? w_first + 31 : L - 1);
  const int64_t pw_first = a.q_pos0 + w_first, pw_last = a.q_pos0 + w_last;
  int64_t ds_last = 0, dstart = 0;
  if (doc && wave_ok) {
    ds_last = doc_start_of(a.cu, a.ndocs, pw_last);
    dstart = doc_start_of(a.cu, a.ndocs, row_ok ? p : pw_last);
  }

  // Q^T operand: head dims 64 s + 32 g .. +31 of this lane's query
  int8v qreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (row_ok) {
      const uint4 lo = *(const uint4*)(qg + qrow * rs + 64 * s + 32 * g);
      const uint4 hi = *(const uint4*)(qg + qrow * rs + 64 * s + 32 * g + 16);
      qreg[s] = int8v{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      qreg[s] = int8v{};
    }
  }

  // Running state (base-2 units; the O accumulator in units of s_v; every
  // element of lacc holds the row sum l of this lane's query).  O and l are
  // relative to m_ref, an integer (or -inf) at least as large as m_true.
  floatx16 oacc[NDT];
  floatx16 lacc = floatx16{};
  float m_true = -INFINITY, m_ref = -INFINITY;
  const int64_t st_row = ((int64_t)b * L + qrow) * ((int64_t)H * D) + (int64_t)h * D;
  const int64_t ml_idx = ((int64_t)b * H + h) * L + qrow;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = floatx16{};
  if (rd && row_ok) {
    // the stored state is relative to the true running max: move it to the
    // integer reference above it
    m_true = a.st_m[ml_idx] * kLog2e;
    m_ref = ceilf(m_true);
    const float f = m_true == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_true - m_ref);
    const float fv = f / s_v;
    const float l0 = a.st_l[ml_idx] * f;
#pragma unroll
    for (int i = 0; i < 16; ++i) lacc[i] = l0;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 v4 = *(const float4*)(a.st_o + st_row + 32 * dt + 8 * i4 + 4 * g);
        oacc[dt][4 * i4 + 0] = v4.x * fv;
        oacc[dt][4 * i4 + 1] = v4.y * fv;
        oacc[dt][4 * i4 + 2] = v4.z * fv;
        oacc[dt][4 * i4 + 3] = v4.w * fv;
      }
  }

  // Tile fetch by the 256 lanes of waves 0-3: fetch i of a lane fills 16-byte
  // slot (i * 256 + tid) of the tile, row i * RPS + tid / CH, physical chunk
  // tid % CH, holding logical chunk phys ^ swz8(row).  K and V share the
  // swizzle, so one byte offset per lane serves both.
  constexpr int kFetchThreads = kThreads / 2;
  constexpr int DMA = BN * CH / kFetchThreads;
  constexpr int RPS = kFetchThreads / CH;
  static_assert(DMA >= 1 && (BN * CH) % kFetchThreads == 0 && RPS % 16 == 0, "tile fetch split");
  const int f_tid = tid & (kFetchThreads - 1);
  const int f_w = w & (kFetchThreads / 64 - 1);
  const int f_row = f_tid / CH;
  const int f_ph = f_tid % CH;
  const uint32_t f_off = (uint32_t)((int64_t)f_row * rs + 16 * (f_ph ^ swz8<D>(f_row)));
  const uint32_t smem_base = lds_addr(&smem[0][0][0]);
  auto lds_of = [&](int st, int tensor, int byte) { return smem_base + (uint32_t)((st * 2 + tensor) * TILE + byte); };
  // Tiled V: a tile is D rows of BN bytes (CHT chunks), stored contiguously;
  // fetch i of a lane fills row i * RPST + f_tid / CHT, physical chunk
  // f_tid % CHT, with the swizzle of 128-byte rows.  Keys past L are zero
  // codes in the block itself, so every tile is read whole.
  constexpr int CHT = BN / 16;
  constexpr int RPST = kFetchThreads / CHT;
  static_assert(D * CHT == BN * CH && RPST % 16 == 0, "tiled V fetch split");
  const int ft_row = f_tid / CHT;
  const uint32_t fvt_off = (uint32_t)(ft_row * BN + 16 * ((f_tid % CHT) ^ swz8<BN>(ft_row)));
  auto fetch_vt = [&](int kt, int i, uint32_t lds) { fetch16(vg + ((int64_t)kt * D + i * RPST) * BN, fvt_off, lds); };
  auto fetch = [&](int kt, int st) {
    const int64_t key0 = (int64_t)kt * BN;
    if (key0 + BN <= L) {
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const int64_t rowoff = (key0 + i * RPS) * rs;
        const int wbase = (i * kFetchThreads + 64 * f_w) * 16;
        fetch16(kg + rowoff, f_off, lds_of(st, 0, wbase));
        if constexpr (VT) fetch_vt(kt, i, lds_of(st, 1, wbase));
        else fetch16(vg + rowoff, f_off, lds_of(st, 1, wbase));
      }
    } else {
      // the ragged last tile: offsets relative to its first row; rows past the
      // end re-read row L-1 (finite data the mask drops)
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const int row = i * RPS + f_row;
        const int64_t rrow = key0 + row < L ? row : L - 1 - key0;
        const uint32_t off = (uint32_t)(rrow * rs + 16 * (f_ph ^ swz8<D>(f_row)));
        const int wbase = (i * kFetchThreads + 64 * f_w) * 16;
        fetch16(kg + key0 * rs, off, lds_of(st, 0, wbase));
        if constexpr (VT) fetch_vt(kt, i, lds_of(st, 1, wbase));
        else fetch16(vg + key0 * rs, off, lds_of(st, 1, wbase));
      }
    }
  };

  // LDS operands.  K rows through pi (as in bf16): 32 bytes = logical chunks
  // 4 s + 2 g and +1 of row 32 t + pi(r32).  V^T of head-dim tile dt: four
  // 8-bit transpose loads, load x covering keys 8 (2x + g) .. +7.
  const int krow_l = pi32(r32);
  const int lam = lane & 15;
  const int tr_col = 16 * ((lane >> 4) & 1) + 8 * (lam & 1);   // + 32 dt
  const int tr_row = lam >> 1;                                  // + 8 (2 x + g)
  auto rd_k = [&](const uint8_t* __restrict__ Ks, int j) {     // j = s * NT + t
    const int s = j / NT, t = j % NT;
    const int row = 32 * t + krow_l;
    const uint8_t* rp = Ks + row * D;
    const uint4 lo = *(const uint4*)(rp + 16 * ((4 * s + 2 * g) ^ swz8<D>(row)));
    const uint4 hi = *(const uint4*)(rp + 16 * ((4 * s + 2 * g + 1) ^ swz8<D>(row)));
    return int8v{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto rd_v = [&](const uint8_t* __restrict__ Vs, int kh, int dt) {
    if constexpr (VT) {
      // row 32 dt + r32 of V^T, the 32 bytes of half g of key half kh: logical chunks 4 kh + 2 g and + 1
      const int row = 32 * dt + r32;
      const uint8_t* rp = Vs + row * BN;
      const uint4 lo = *(const uint4*)(rp + 16 * ((4 * kh + 2 * g) ^ swz8<BN>(row)));
      const uint4 hi = *(const uint4*)(rp + 16 * ((4 * kh + 2 * g + 1) ^ swz8<BN>(row)));
      return int8v{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    const int col = 32 * dt + tr_col;
    int2v x[4];
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) {
      const int row = 64 * kh + 8 * (2 * xx + g) + tr_row;
      x[xx] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) int2v*)(Vs + row * D + 16 * ((col >> 4) ^ swz8<D>(row)) + (col & 15)));
    }
    return int8v{x[0][0], x[0][1], x[1][0], x[1][1], x[2][0], x[2][1], x[3][0], x[3][1]};
  };
  // The compute phase as one stream of MFMAs (NQK of S^T = K Q^T, then NH NDT
  // of O^T += V^T P^T and NH of the row sums), each operand read RA MFMAs
  // ahead in consumption order.
  constexpr int NQK = NS * NT;
  constexpr int RA = 2;
  auto compute = [&](const uint8_t* __restrict__ Ks, const uint8_t* __restrict__ Vs, floatx16 (&sacc)[NT],
                     const int8v (&pb)[NH], auto qk_tag, auto pv_tag) {
    constexpr bool QK = decltype(qk_tag)::value != 0, PV = decltype(pv_tag)::value != 0;
    constexpr int J0 = QK ? 0 : NQK, J1 = PV ? NQK + NH * NDT : NQK;
    auto rd = [&](int j) { return j < NQK ? rd_k(Ks, j) : rd_v(Vs, (j - NQK) / NDT, (j - NQK) % NDT); };
    if constexpr (QK) {
#pragma unroll
      for (int t = 0; t < NT; ++t) sacc[t] = floatx16{};
    }
    int8v ring[RA];
#pragma unroll
    for (int j = J0; j < J0 + RA && j < J1; ++j) ring[j - J0] = rd(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const int8v op = ring[(j - J0) % RA];
      if (j < NQK) sacc[j % NT] = mfma8_scaled(op, qreg[j / NT], sacc[j % NT], sc_kq);
      else oacc[(j - NQK) % NDT] = mfma8(op, pb[(j - NQK) / NDT], oacc[(j - NQK) % NDT]);
      if (j + RA < J1) ring[(j - J0) % RA] = rd(j + RA);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (PV) {
      constexpr int kOne = 0x38383838;   // four e4m3 codes of 1.0
#pragma unroll
      for (int kh = 0; kh < NH; ++kh) {
        lacc = mfma8(int8v{kOne, kOne, kOne, kOne, kOne, kOne, kOne, kOne}, pb[kh], lacc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (QK) {
      // The scaled products are otherwise sunk past the phase's end to their
      // first use; an (empty) use here keeps them in the compute phase.
#pragma unroll
      for (int t = 0; t < NT; ++t) asm volatile("" ::"v"(sacc[t]));
    }
  };

  // Masks, row max and the lazy rescale: as in the bf16 kernel.
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
  auto apply_mask = [&](int kt, floatx16 (&sacc)[NT]) {
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
        const int ko = 32 * t + 16 * (i >> 3) + (i & 7);
        sacc[t][i] = (ko >= lo && ko <= hi) ? sacc[t][i] : -INFINITY;
      }
  };
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
  // The lazy rescale, and the reference the exponentials use.  Returns the
  // scale operand of the e4m3 conversions: 2^m_ref when every lane's
  // reference is in the range where exp2(x) and 2^m_ref are normal floats;
  // otherwise the wave subtracts m_ref from the logits here and converts with
  // scale 1.  Both rare cases share one branch.
  auto rescale = [&](float mx, floatx16 (&sacc)[NT]) -> float {
    m_true = fmaxf(m_true, mx);
    const bool need = mx > m_ref + kLazy;
    const float nref = need ? ceilf(m_true) : m_ref;
    const float m_use = nref == -INFINITY ? 0.f : nref;
    const bool fast = __all(m_use >= -116.f && m_use <= 119.f);
    if (__any(need) || !fast) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - nref) : 1.f;
      lacc *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
      if (!fast) {
#pragma unroll
        for (int t = 0; t < NT; ++t) sacc[t] -= m_use;
      }
    }
    m_ref = nref;
    return fast ? __uint_as_float((uint32_t)((int)m_use + 127) << 23) : 1.f;
  };
  // P = exp2(x - m_ref), rounded to e4m3 as the PV B operands (operand h:
  // bytes 0-15 from sub-tile 2h, 16-31 from sub-tile 2h+1).  The first
  // conversion of a word keeps bytes 2-3 of its old value, which the second
  // one overwrites.  Passing the previous tile's word (already consumed by the
  // P V products of this step's compute phase) keeps the conversions in place
  // in the operand registers.
  auto exp_sum = [&](floatx16 (&sacc)[NT], int8v (&pb)[NH], float pscale) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[t][i] = __builtin_amdgcn_exp2f(sacc[t][i]);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        short2v w2 = __builtin_bit_cast(short2v, pb[t / 2][4 * (t % 2) + q]);
        w2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w2, sacc[t][4 * q], sacc[t][4 * q + 1], pscale, false);
        w2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w2, sacc[t][4 * q + 2], sacc[t][4 * q + 3], pscale, true);
        pb[t / 2][4 * (t % 2) + q] = __builtin_bit_cast(int, w2);
      }
  };

  if (kt_begin < kt_end) {
    const int grp = w >> 2;
    auto stage = [&](int u) { return (u - kt_begin) & (kStages - 1); };
    if (grp == 0) {
      fetch(kt_begin, 0);
      if (kt_begin + 1 < kt_end) fetch(kt_begin + 1, 1);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);              // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    if (grp == 1) __syncthreads();                   // group 1 runs one phase behind
    floatx16 sacc[NT];
    int8v pb[NH];
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) pb[kh] = int8v{};
    auto step = [&](int u, auto qk_tag, auto pv_tag) {
      constexpr bool QK = decltype(qk_tag)::value != 0;
      compute(smem[stage(u)][0], smem[stage(u - 1)][1], sacc, pb, qk_tag, pv_tag);
      lds_read_barrier();
      const bool more = u + 2 < kt_end;
      if (grp == 0 && more) {
        fetch(u + 2, stage(u + 2));
      }
      if constexpr (QK) {
        if (need_mask(u)) apply_mask(u, sacc);
        const float pscale = rescale(row_max(sacc), sacc);
        exp_sum(sacc, pb, pscale);
      }
      // tile u+1 must have landed: at most the fetch of tile u+2 (2 DMA tensors) outstanding
      __asm__ volatile("" ::: "memory");
      if (more) __builtin_amdgcn_s_waitcnt(0x0070 + 2 * DMA);   // vmcnt(2 DMA) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(0x0070);
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    };
    step(kt_begin, Tag<1>{}, Tag<0>{});
    for (int u = kt_begin + 1; u < kt_end; ++u) step(u, Tag<1>{}, Tag<1>{});
    step(kt_end, Tag<0>{}, Tag<1>{});
    if (grp == 0) __syncthreads();
  }

  // O back to true units, then to the true running max.
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= s_v;
  if (m_true != -INFINITY && m_true != m_ref) {
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_true);
    lacc *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
  }

  if (!row_ok || qrow >= rows_end) return;
  const float l_tot = lacc[0];
  const bool has = l_tot > 0.f;
  const float m_run = m_true;
  // m in natural-log units of the true scores (x is the base-2 logit)
  if (writes_state(a.flags, qrow, a.final_from)) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *(float4*)(a.st_o + st_row + 32 * dt + 8 * i4 + 4 * g) =
            float4{oacc[dt][4 * i4], oacc[dt][4 * i4 + 1], oacc[dt][4 * i4 + 2], oacc[dt][4 * i4 + 3]};
    if (g == 0) {
      a.st_m[ml_idx] = m_run * kLn2;
      a.st_l[ml_idx] = l_tot;
    }
  }
  const float inv = has ? 1.f / l_tot : 0.f;
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

hipError_t launch_block_fp8(const BlockArgs& a, int d, hipStream_t s, const LaunchEvents& ev) {
  if (a.flags & (F_SPLIT | F_READ_SIDE)) return hipErrorInvalidValue;   // bf16 kernel only
  const int64_t nqt = (a.rows_end + BM - 1) / BM;
  const dim3 grid((unsigned)(nqt * a.H * a.B)), block(kThreads);
  const bool vt = (a.flags & F_V_TILED) != 0;
  if (d == 128)
    return vt ? launch_bound(attn_block_fp8_kernel<128, true>, grid, block, s, ev, a)
              : launch_bound(attn_block_fp8_kernel<128, false>, grid, block, s, ev, a);
  return vt ? launch_bound(attn_block_fp8_kernel<64, true>, grid, block, s, ev, a)
            : launch_bound(attn_block_fp8_kernel<64, false>, grid, block, s, ev, a);
}

}  // namespace cpattn
