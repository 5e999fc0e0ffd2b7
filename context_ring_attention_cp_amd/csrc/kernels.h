// Internal interface between the host API (api.cpp) and the HIP kernels:
// the flags, layouts and argument structs the kernels are compiled against.
// The launcher declarations are in launch.h.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

// What a block kernel reads and writes.
enum : int32_t {
  F_READ_STATE = 1,     // start from the running state (O, m, l) instead of empty
  F_WRITE_STATE = 2,    // store the running state
  F_WRITE_FINAL = 4,    // store out = O / l (input dtype) and m, l, lse
  F_WRITE_PARTIAL = 8,  // store normalised O (float32) and lse of this block alone
  F_V_TILED = 16,       // v in head-dim-major key tiles, zero past L: bf16 [B, H, T, d, 64],
                        // e4m3 [B, H, T8, d, 128] with the operand key order (launch_v_tiles_fp8)
  F_SPLIT = 32,         // bf16 kernel: split the keys of the query tiles from split_from on
  F_READ_SIDE = 64,     // bf16 kernel: merge the side state of those tiles into the state read
};

// Query rows per workgroup of the bf16 block kernel, and keys per LDS tile.
constexpr int kBf16Rows = 256;
constexpr int kBf16Keys = 64;
// Longest query-tile dispatch order a launch carries in its arguments.
constexpr int kOrderMax = 512;

// Per-row store decisions of a block launch (see BlockArgs::final_from).
__host__ __device__ inline bool writes_final(int32_t flags, int64_t row, int64_t final_from) {
  return (flags & F_WRITE_FINAL) && (!(flags & F_WRITE_STATE) || row >= final_from);
}
__host__ __device__ inline bool writes_state(int32_t flags, int64_t row, int64_t final_from) {
  return (flags & F_WRITE_STATE) && (!(flags & F_WRITE_FINAL) || row < final_from);
}
// Keys of a tiled V block: L rounded up to whole 64-key tiles (T = that / 64).
__host__ __device__ inline int64_t v_tiled_keys(int64_t L) { return (L + 63) / 64 * 64; }

enum : int32_t { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_DOC_CAUSAL = 2 };

// One launch: the rank's query shard against one key/value block.
struct BlockArgs {
  const void* q;         // [B, L, H, d]
  const void* k;         // [B, L, H, d] block j
  const void* v;         // [B, L, H, d] block j (F_V_TILED: [B, H, T, d, 64])
  int64_t L;             // shard length (rows of q, rows of k/v)
  int32_t B, H;
  int64_t q_pos0;        // global position of query row 0 (rank * L)
  int64_t k_pos0;        // global position of key row 0 (j * L)
  int32_t mask;
  int32_t ndocs;
  const int32_t* cu;     // device cu_seqlens (DOC_CAUSAL)
  float scale_log2;      // softmax scale * log2(e)
  int32_t flags;
  // Rows of this launch: query rows [0, rows_end) take part (the grid covers
  // their tiles only).  When both F_WRITE_STATE and F_WRITE_FINAL are set,
  // rows [final_from, rows_end) store the final output and the rows before
  // them the running state; with one of the two flags every row stores that.
  int64_t rows_end;
  int64_t final_from;
  // Key split of a causal diagonal block (bf16 kernel).  With F_SPLIT, each
  // query tile qt >= split_from (of kBf16Rows rows) runs as two workgroups:
  // one takes the key tiles [0, split_from * kBf16Rows / kBf16Keys), which
  // those rows all see, and stores its running state in side_*; the other
  // takes the rest of the block and stores into st_*.  With F_READ_SIDE the
  // rows of those tiles merge side_* into their state at the end of the launch
  // (the merge of running states is associative: the launch may add its block
  // to either part first).
  // split_from >= (number of query tiles) / 2.
  int32_t split_from;
  float* side_o;         // [B, L, H, d]
  float* side_m;         // [B, H, L] natural-log units
  float* side_l;         // [B, H, L]
  // running state
  float* st_o;           // [B, L, H, d]
  float* st_m;           // [B, H, L] natural-log units
  float* st_l;           // [B, H, L]
  // final outputs
  void* out;             // [B, L, H, d] input dtype
  float* m_out;          // [B, H, L] or null
  float* l_out;
  float* lse_out;
  // partial outputs
  float* o_part;         // [B, L, H, d]
  float* lse_part;       // [B, H, L]
  // FP8 (e4m3) inputs only: q, k, v hold codes; value = decode(code) * scale
  const float* q_scale;  // [B, H] of the query shard
  const float* k_scale;  // [B, H] of block j
  const float* v_scale;  // [B, H] of block j
  // Dispatch order of the query tiles (bf16 kernel, without F_SPLIT): when
  // order_n equals the launch's number of query tiles, order[r] is the tile
  // of rank r by decreasing work (the host computes it from the document
  // boundaries), and an XCD that holds whole heads runs their tiles rank by
  // rank; otherwise the tiles run in decreasing index.
  int32_t order_n;
  uint16_t order[kOrderMax];
};

// Largest merge count handled by one kernel launch.
constexpr int kMaxParts = 64;

struct MergeArgs {
  const float* o[kMaxParts];    // already in merge order
  const float* lse[kMaxParts];
  int32_t n;
  int64_t L;
  int32_t B, H, d;
  int32_t out_bf16;
  void* out;
  float* lse_out;
};

struct FinalizeArgs {
  const float* st_o;
  const float* st_m;
  const float* st_l;
  int64_t L;
  int32_t B, H, d;
  int32_t out_bf16;
  void* out;
  float* m_out;
  float* l_out;
  float* lse_out;
};

// Backward of one block (bf16 inputs, fp32 gradients).
struct BwdArgs {
  const void* q;         // [B, L, H, d] the rank's queries
  const void* k;         // [B, L, H, d] block j
  const void* v;         // [B, L, H, d] block j
  const void* d_o;       // [B, L, H, d] gradient of the rank's output
  const float* lse;      // [B, H, L] log-sum-exp of the rank's forward (natural log)
  const float* delta;    // [B, H, L] rowsum(dO * O)
  int64_t L;
  int32_t B, H;
  int64_t q_pos0, k_pos0;
  int32_t mask;
  int32_t ndocs;
  const int32_t* cu;     // device cu_seqlens (DOC_CAUSAL)
  float scale;           // softmax scale
  float scale_log2;      // scale * log2(e)
  int32_t accumulate;    // dq += (1) or dq = (0)
  float* dq;             // [B, L, H, d]
  float* dk;             // [B, L, H, d] of block j
  float* dv;             // [B, L, H, d] of block j
};

struct DeltaArgs {
  const void* o;         // [B, L, H, d] bf16
  const void* d_o;       // [B, L, H, d] bf16
  int64_t L;
  int32_t B, H;
  float* delta;          // [B, H, L]
};

// Regrouping of all-to-all (Ulysses) context parallelism between the N
// sequence shards [B, L, H, d] and the whole sequence of one rank's head
// group [h0, h0 + Hn), stored [B, S, Hn, d] (S = N L).  Element bytes elt; Hn d
// elt a multiple of 16 and every pointer 16-byte aligned.
constexpr int kMaxShards = 64;
struct RegroupArgs {
  void* shards[kMaxShards];   // gather: read; scatter: written (only the group's heads)
  void* full;                 // gather: written; scatter: read
  int64_t B, L, S;
  int32_t N, H, Hn, h0, d, elt;
};

// FP8 (e4m3) quantisation of a bf16 block [B, L, H, d] with one scale per
// (b, h): codes [B, L, H, d] bytes, scales [B, H] float32 (amax / 448).
struct QuantArgs {
  const void* x;
  void* codes;
  float* scales;
  int64_t L;
  int32_t B, H;
};

}  // namespace cpattn
