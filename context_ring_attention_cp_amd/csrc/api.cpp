// Host side of libcpattn: argument validation, the ring schedule with
// mask-aware block skipping, workspace layout, and the one-GPU ring driver
// (two receive slots, a copy stream, events).  Every public entry point
// validates all of its arguments before it makes any HIP call, so invalid
// calls fail without touching a device.
#include "cpattn.h"
#include "launch.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

using namespace cpattn;

namespace {

thread_local std::string g_last_error;

cp_status fail(cp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

cp_status hip_fail(hipError_t e, const char* what) {
  return fail(CP_ERR_HIP, "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elt_bytes(int32_t dtype) { return dtype == CP_BF16 ? 2 : 4; }

// Validation of the description alone (no pointers of tensors).
cp_status check_desc(const cp_attn_desc* d) {
  if (!d) return fail(CP_ERR_INVALID_ARG, "desc is NULL");
  if (d->B < 1 || d->H < 1) return fail(CP_ERR_INVALID_ARG, "B=%d and H=%d must be >= 1", d->B, d->H);
  if (d->L < 1) return fail(CP_ERR_INVALID_ARG, "L=%lld must be >= 1", (long long)d->L);
  if (d->N < 1 || d->N > CP_MAX_RING)
    return fail(CP_ERR_INVALID_ARG, "ring size N=%d outside [1, %d]", d->N, CP_MAX_RING);
  if (d->rank < 0 || d->rank >= d->N)
    return fail(CP_ERR_INVALID_ARG, "rank=%d outside [0, N=%d)", d->rank, d->N);
  if (d->dtype != CP_F32 && d->dtype != CP_BF16) return fail(CP_ERR_INVALID_ARG, "dtype=%d unknown", d->dtype);
  if (d->mask != CP_MASK_NONE && d->mask != CP_MASK_CAUSAL && d->mask != CP_MASK_DOC_CAUSAL)
    return fail(CP_ERR_INVALID_ARG, "mask=%d unknown", d->mask);
  if (!(std::isfinite(d->scale) && d->scale >= 0.f))
    return fail(CP_ERR_INVALID_ARG, "scale=%g must be finite and >= 0", (double)d->scale);
  if (d->d != 64 && d->d != 128) return fail(CP_ERR_UNSUPPORTED, "head dim d=%d not in {64, 128}", d->d);
  // sizes: total sequence and element counts must stay well inside int64 and
  // the sequence positions inside int32 (cu_seqlens are int32)
  const long double S = (long double)d->N * (long double)d->L;
  if (S > 2147483647.0L) return fail(CP_ERR_UNSUPPORTED, "sequence N*L=%.0Lf exceeds int32 positions", S);
  const long double elems = (long double)d->B * d->L * d->H * d->d;
  if (elems * 4 > 4.0e18L) return fail(CP_ERR_UNSUPPORTED, "tensor of %.0Lf elements too large", elems);
  // the bf16 kernel addresses the rows of one 64-key tile with 32-bit byte offsets
  if ((long double)d->H * d->d * 4 * 64 > 4294967295.0L)
    return fail(CP_ERR_UNSUPPORTED, "row stride H*d=%lld too large", (long long)d->H * d->d);
  // launch grid of the widest kernel (one workgroup per 64 rows of a head)
  const long double wgs = (long double)d->B * d->H * ((d->L + 63) / 64);
  if (wgs > 2147483647.0L) return fail(CP_ERR_UNSUPPORTED, "launch grid of %.0Lf workgroups too large", wgs);
  const long double thr = elems / 4;
  if (thr / 256 > 2147483647.0L) return fail(CP_ERR_UNSUPPORTED, "elementwise grid too large");
  if (d->mask == CP_MASK_DOC_CAUSAL) {
    if (!d->cu_seqlens || !d->cu_seqlens_dev)
      return fail(CP_ERR_INVALID_ARG, "DOC_CAUSAL needs cu_seqlens (host) and cu_seqlens_dev (device)");
    if (d->ndocs < 1) return fail(CP_ERR_INVALID_ARG, "ndocs=%d must be >= 1", d->ndocs);
    if (!aligned(d->cu_seqlens_dev, 4)) return fail(CP_ERR_INVALID_ARG, "cu_seqlens_dev not 4-byte aligned");
    const int32_t* cu = d->cu_seqlens;
    if (cu[0] != 0) return fail(CP_ERR_INVALID_ARG, "cu_seqlens[0]=%d must be 0", cu[0]);
    for (int32_t k = 0; k < d->ndocs; ++k)
      if (cu[k + 1] <= cu[k])
        return fail(CP_ERR_INVALID_ARG, "cu_seqlens not strictly increasing at %d (%d, %d)", k, cu[k], cu[k + 1]);
    if ((int64_t)cu[d->ndocs] != (int64_t)d->N * d->L)
      return fail(CP_ERR_INVALID_ARG, "cu_seqlens[ndocs]=%d must equal N*L=%lld", cu[d->ndocs],
                  (long long)d->N * d->L);
  }
  return CP_OK;
}

cp_status check_tensor(const void* p, const char* name) {
  if (!p) return fail(CP_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(CP_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return CP_OK;
}

cp_status check_vec(const void* p, const char* name, bool optional) {
  if (!p) return optional ? CP_OK : fail(CP_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, 4)) return fail(CP_ERR_INVALID_ARG, "%s is not 4-byte aligned", name);
  return CP_OK;
}

// First position of the document holding global position p (host cu).
int64_t doc_start_host(const cp_attn_desc* d, int64_t p) {
  int lo = 0, hi = d->ndocs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if ((int64_t)d->cu_seqlens[mid] <= p) lo = mid; else hi = mid;
  }
  return d->cu_seqlens[lo];
}

// Does any row of the rank see any key of block j?  Causal forms: row p sees
// keys up to p, so block j > rank is invisible and block rank always visible;
// for an earlier block the rows with the earliest first key is the shard's
// first row (doc_start is non-decreasing in p).
bool block_visible(const cp_attn_desc* d, int32_t j) {
  if (d->mask == CP_MASK_NONE) return true;
  if (j > d->rank) return false;
  if (j == d->rank || d->mask == CP_MASK_CAUSAL) return true;
  const int64_t first = doc_start_host(d, (int64_t)d->rank * d->L);
  return first <= (int64_t)(j + 1) * d->L - 1;
}

// Rows of the shard that see block j.  Every row sees the rank's own block
// and, under the causal or no mask, every visible block.  Under the document
// mask, row p sees an earlier block j when its document starts at or before
// the block's last key; the document start is non-decreasing in p, so those
// rows are a prefix: the rows before the first document that starts after
// the block (cu[ndocs] = N L always does).
int64_t rows_seeing(const cp_attn_desc* d, int32_t j) {
  if (d->mask != CP_MASK_DOC_CAUSAL || j >= d->rank) return d->L;
  const int64_t last_key = (int64_t)(j + 1) * d->L - 1;
  int lo = 0, hi = d->ndocs;
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if ((int64_t)d->cu_seqlens[mid] > last_key) hi = mid; else lo = mid + 1;
  }
  const int64_t r = (int64_t)d->cu_seqlens[lo] - (int64_t)d->rank * d->L;
  return r < 0 ? 0 : (r > d->L ? d->L : r);
}

// Dispatch order of the bf16 kernel's query tiles for block j under the
// document mask: the tiles of the launch's rows by decreasing number of key
// tiles they run (the key range a workgroup covers, from the document start
// of its first row to the causal end of its last), so that the longest
// workgroups start first.  Other masks keep the kernel's own order (the
// causal work falls with the tile index already).
void fill_order(const cp_attn_desc* d, int32_t j, BlockArgs& a) {
  a.order_n = 0;
  if (d->mask != CP_MASK_DOC_CAUSAL) return;
  const int64_t nqt = (a.rows_end + kBf16Rows - 1) / kBf16Rows;
  if (nqt < 2 || nqt > kOrderMax) return;
  const int64_t L = d->L, nkt = (L + kBf16Keys - 1) / kBf16Keys;
  const int64_t q_pos0 = (int64_t)d->rank * L, k_pos0 = (int64_t)j * L;
  auto doc_start = [&](int64_t p) {   // start of the document holding global position p
    int lo = 0, hi = d->ndocs;
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if ((int64_t)d->cu_seqlens[mid + 1] > p) hi = mid; else lo = mid + 1;
    }
    return (int64_t)d->cu_seqlens[lo < d->ndocs ? lo : d->ndocs - 1];
  };
  std::vector<std::pair<int64_t, int32_t>> w((size_t)nqt);
  for (int64_t qt = 0; qt < nqt; ++qt) {
    const int64_t q0 = qt * kBf16Rows, q_last = std::min(q0 + kBf16Rows, a.rows_end) - 1;
    const int64_t hi = q_pos0 + q_last - k_pos0;
    const int64_t kt_end = hi < 0 ? 0 : std::min(hi / kBf16Keys + 1, nkt);
    const int64_t lo = doc_start(q_pos0 + q0) - k_pos0;
    const int64_t kt_begin = lo > 0 ? std::min(lo / kBf16Keys, nkt) : 0;
    w[(size_t)qt] = {std::max<int64_t>(kt_end - kt_begin, 0), (int32_t)qt};
  }
  // decreasing work; among equals the higher tile first (the kernel's own order)
  std::sort(w.begin(), w.end(), [](const auto& x, const auto& y) {
    return x.first != y.first ? x.first > y.first : x.second > y.second;
  });
  for (int64_t r = 0; r < nqt; ++r) a.order[r] = (uint16_t)w[(size_t)r].second;
  a.order_n = (int32_t)nqt;
}

std::vector<int32_t> schedule(const cp_attn_desc* d, int32_t flags) {
  std::vector<int32_t> out;
  const int step = (flags & CP_RING_REVERSE) ? 1 : -1;
  for (int32_t t = 0; t < d->N; ++t) {
    const int32_t j = (int32_t)((((int64_t)d->rank + step * t) % d->N + d->N) % d->N);
    if (block_visible(d, j)) out.push_back(j);
  }
  return out;
}

float scale_log2(const cp_attn_desc* d) {
  const float sc = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->d);
  return sc * 1.442695040888963407360f;
}

BlockArgs block_args(const cp_attn_desc* d, int32_t j, const void* q, const void* k, const void* v) {
  BlockArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.L = d->L;
  a.B = d->B;
  a.H = d->H;
  a.q_pos0 = (int64_t)d->rank * d->L;
  a.k_pos0 = (int64_t)j * d->L;
  a.mask = d->mask;
  a.ndocs = d->ndocs;
  a.cu = d->mask == CP_MASK_DOC_CAUSAL ? d->cu_seqlens_dev : nullptr;
  a.scale_log2 = scale_log2(d);
  a.rows_end = d->L;
  a.final_from = 0;
  return a;
}

hipError_t launch_block(const cp_attn_desc* d, const BlockArgs& a, hipStream_t s, const LaunchEvents& ev = {}) {
  return d->dtype == CP_BF16 ? launch_block_bf16(a, d->d, s, ev) : launch_block_f32(a, d->d, s, ev);
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Key split of the causal diagonal block (the first ring step) when its launch
// would fill the chip's 256 compute units at most once: the heaviest query
// tiles then set the launch's length alone, and splitting the keys of the upper
// half of the tiles between two workgroups halves it.  The next step (a full
// block, seen by every row) merges the two states.  bf16 only.
constexpr int64_t kSplitMaxWorkgroups = 256;

bool split_eligible(const cp_attn_desc* d) {
  const int64_t nqt = (d->L + kBf16Rows - 1) / kBf16Rows;
  return d->dtype == CP_BF16 && d->mask == CP_MASK_CAUSAL && d->rank >= 1 && nqt >= 2 &&
         nqt * d->H * d->B <= kSplitMaxWorkgroups;
}

// First split query tile: the upper half of the tiles.
int32_t split_from_of(const cp_attn_desc* d) {
  const int64_t nqt = (d->L + kBf16Rows - 1) / kBf16Rows;
  return (int32_t)(nqt - nqt / 2);
}

struct WorkspaceLayout {
  size_t slot_k[2], slot_v[2], st_o, st_m, st_l, side_o, side_m, side_l, total;
  bool side;
};

// With room for the side state of a key-split diagonal block where
// split_eligible holds.
WorkspaceLayout layout_of(const cp_attn_desc* d) {
  WorkspaceLayout w;
  const size_t blk = round_up((size_t)d->B * d->L * d->H * d->d * elt_bytes(d->dtype), 256);
  // a bf16 V slot holds the tiled copy, whose keys are padded to whole 64-key tiles
  const size_t blk_v = round_up((size_t)d->B * v_tiled_keys(d->L) * d->H * d->d * elt_bytes(d->dtype), 256);
  const size_t ost = round_up((size_t)d->B * d->L * d->H * d->d * 4, 256);
  const size_t vec = round_up((size_t)d->B * d->H * d->L * 4, 256);
  size_t off = 0;
  for (int s = 0; s < 2; ++s) {
    w.slot_k[s] = off;
    off += blk;
    w.slot_v[s] = off;
    off += blk_v;
  }
  w.st_o = off;
  off += ost;
  w.st_m = off;
  off += vec;
  w.st_l = off;
  off += vec;
  w.side = split_eligible(d);
  w.side_o = w.side_m = w.side_l = 0;
  if (w.side) {
    w.side_o = off;
    off += ost;
    w.side_m = off;
    off += vec;
    w.side_l = off;
    off += vec;
  }
  w.total = off;
  return w;
}

}  // namespace

struct cp_attn_profiler {
  std::vector<hipEvent_t> start, stop;            // attention launches
  std::vector<hipEvent_t> copy_start, copy_stop;  // ring receives
  int32_t used = 0, copies = 0;
};

extern "C" {

const char* cp_attn_status_string(int32_t status) {
  switch (status) {
    case CP_OK: return "CP_OK";
    case CP_ERR_INVALID_ARG: return "CP_ERR_INVALID_ARG";
    case CP_ERR_UNSUPPORTED: return "CP_ERR_UNSUPPORTED";
    case CP_ERR_WORKSPACE: return "CP_ERR_WORKSPACE";
    case CP_ERR_HIP: return "CP_ERR_HIP";
    default: return "CP_ERR_UNKNOWN";
  }
}

const char* cp_attn_last_error(void) { return g_last_error.c_str(); }

cp_status cp_attn_ring_schedule(const cp_attn_desc* desc, int32_t flags, int32_t* blocks_out,
                                int32_t capacity, int32_t* count_out) {
  g_last_error.clear();
  cp_status st = check_desc(desc);
  if (st != CP_OK) return st;
  if (!count_out) return fail(CP_ERR_INVALID_ARG, "count_out is NULL");
  if (flags & ~(CP_RING_PREFETCH | CP_RING_REVERSE)) return fail(CP_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const std::vector<int32_t> s = schedule(desc, flags);
  if (capacity < (int32_t)s.size() || (!blocks_out && !s.empty()))
    return fail(CP_ERR_INVALID_ARG, "capacity %d < %zu scheduled blocks", capacity, s.size());
  for (size_t i = 0; i < s.size(); ++i) blocks_out[i] = s[i];
  *count_out = (int32_t)s.size();
  return CP_OK;
}

cp_status cp_attn_visible_pairs(const cp_attn_desc* desc, int64_t* pairs_out) {
  g_last_error.clear();
  cp_status st = check_desc(desc);
  if (st != CP_OK) return st;
  if (!pairs_out) return fail(CP_ERR_INVALID_ARG, "pairs_out is NULL");
  const int64_t L = desc->L, r = desc->rank;
  const int64_t s0 = r * L, s1 = (r + 1) * L;     // rows [s0, s1)
  int64_t pairs = 0;
  if (desc->mask == CP_MASK_NONE) {
    pairs = (int64_t)desc->N * L * L;
  } else if (desc->mask == CP_MASK_CAUSAL) {
    pairs = s0 * L + L * (L + 1) / 2;             // sum over p of (p + 1)
  } else {
    // sum over rows p of (p - doc_start(p) + 1), one document at a time
    for (int32_t k = 0; k < desc->ndocs; ++k) {
      const int64_t a = desc->cu_seqlens[k], e = desc->cu_seqlens[k + 1];
      const int64_t lo = a > s0 ? a : s0, hi = e < s1 ? e : s1;   // rows [lo, hi)
      if (lo >= hi) continue;
      const int64_t n = hi - lo, first = lo - a + 1;              // first + (first+1) + ... n terms
      pairs += n * first + n * (n - 1) / 2;
    }
  }
  *pairs_out = pairs;
  return CP_OK;
}

size_t cp_attn_workspace_bytes(const cp_attn_desc* desc) {
  g_last_error.clear();
  if (check_desc(desc) != CP_OK) return 0;
  return layout_of(desc).total;
}

cp_status cp_attn_block_partial(const cp_attn_desc* desc, int32_t j, int32_t mode, const void* q,
                                const void* k_j, const void* v_j, const cp_state* state, float* o_part,
                                float* lse_part, void* stream) {
  g_last_error.clear();
  cp_status st = check_desc(desc);
  if (st != CP_OK) return st;
  if (j < 0 || j >= desc->N) return fail(CP_ERR_INVALID_ARG, "block j=%d outside [0, N=%d)", j, desc->N);
  if ((st = check_tensor(q, "q")) != CP_OK || (st = check_tensor(k_j, "k_j")) != CP_OK ||
      (st = check_tensor(v_j, "v_j")) != CP_OK)
    return st;
  BlockArgs a = block_args(desc, j, q, k_j, v_j);
  if (mode == CP_MODE_INIT || mode == CP_MODE_ACCUMULATE) {
    if (!state) return fail(CP_ERR_INVALID_ARG, "state is NULL for mode %d", mode);
    if (o_part || lse_part) return fail(CP_ERR_INVALID_ARG, "o_part/lse_part must be NULL for mode %d", mode);
    if ((st = check_tensor(state->o, "state->o")) != CP_OK || (st = check_vec(state->m, "state->m", false)) != CP_OK ||
        (st = check_vec(state->l, "state->l", false)) != CP_OK)
      return st;
    a.st_o = state->o;
    a.st_m = state->m;
    a.st_l = state->l;
    a.flags = F_WRITE_STATE | (mode == CP_MODE_ACCUMULATE ? F_READ_STATE : 0);
  } else if (mode == CP_MODE_PARTIAL_LSE) {
    if (state) return fail(CP_ERR_INVALID_ARG, "state must be NULL for PARTIAL_LSE");
    if ((st = check_tensor(o_part, "o_part")) != CP_OK || (st = check_vec(lse_part, "lse_part", false)) != CP_OK)
      return st;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.flags = F_WRITE_PARTIAL;
  } else {
    return fail(CP_ERR_INVALID_ARG, "mode=%d unknown", mode);
  }
  const hipError_t e = launch_block(desc, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "block kernel launch");
  return CP_OK;
}

cp_status cp_attn_merge_lse(const cp_attn_desc* desc, int32_t n, const float* const* o_parts,
                            const float* const* lse_parts, const int32_t* order, void* out, float* lse_out,
                            void* stream) {
  g_last_error.clear();
  cp_status st = check_desc(desc);
  if (st != CP_OK) return st;
  if (n < 1 || n > CP_MAX_RING || n > kMaxParts) return fail(CP_ERR_INVALID_ARG, "n=%d outside [1, %d]", n, CP_MAX_RING);
  if (!o_parts || !lse_parts) return fail(CP_ERR_INVALID_ARG, "o_parts/lse_parts is NULL");
  if ((st = check_tensor(out, "out")) != CP_OK || (st = check_vec(lse_out, "lse_out", true)) != CP_OK) return st;
  MergeArgs a;
  std::memset(&a, 0, sizeof(a));
  std::vector<char> seen(n, 0);
  for (int32_t t = 0; t < n; ++t) {
    const int32_t j = order ? order[t] : t;
    if (j < 0 || j >= n || seen[j]) return fail(CP_ERR_INVALID_ARG, "order is not a permutation of 0..%d", n - 1);
    seen[j] = 1;
    if ((st = check_tensor(o_parts[j], "o_parts[j]")) != CP_OK || (st = check_vec(lse_parts[j], "lse_parts[j]", false)) != CP_OK)
      return st;
    a.o[t] = o_parts[j];
    a.lse[t] = lse_parts[j];
  }
  // unused slots point at part 0, so no load the kernel guards by j < n can
  // ever see a null address
  for (int32_t t = n; t < kMaxParts; ++t) {
    a.o[t] = a.o[0];
    a.lse[t] = a.lse[0];
  }
  a.n = n;
  a.L = desc->L;
  a.B = desc->B;
  a.H = desc->H;
  a.d = desc->d;
  a.out_bf16 = desc->dtype == CP_BF16;
  a.out = out;
  a.lse_out = lse_out;
  const hipError_t e = launch_merge(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return CP_OK;
}

cp_status cp_attn_finalize(const cp_attn_desc* desc, const cp_state* state, void* out, float* m_out,
                           float* l_out, float* lse_out, void* stream) {
  g_last_error.clear();
  cp_status st = check_desc(desc);
  if (st != CP_OK) return st;
  if (!state) return fail(CP_ERR_INVALID_ARG, "state is NULL");
  if ((st = check_tensor(state->o, "state->o")) != CP_OK || (st = check_vec(state->m, "state->m", false)) != CP_OK ||
      (st = check_vec(state->l, "state->l", false)) != CP_OK || (st = check_tensor(out, "out")) != CP_OK ||
      (st = check_vec(m_out, "m_out", true)) != CP_OK || (st = check_vec(l_out, "l_out", true)) != CP_OK ||
      (st = check_vec(lse_out, "lse_out", true)) != CP_OK)
    return st;
  FinalizeArgs a;
  a.st_o = state->o;
  a.st_m = state->m;
  a.st_l = state->l;
  a.L = desc->L;
  a.B = desc->B;
  a.H = desc->H;
  a.d = desc->d;
  a.out_bf16 = desc->dtype == CP_BF16;
  a.out = out;
  a.m_out = m_out;
  a.l_out = l_out;
  a.lse_out = lse_out;
  const hipError_t e = launch_finalize(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "finalize kernel launch");
  return CP_OK;
}

namespace {

cp_status check_bwd_desc(const cp_attn_desc* d) {
  const cp_status st = check_desc(d);
  if (st != CP_OK) return st;
  if (d->dtype != CP_BF16) return fail(CP_ERR_UNSUPPORTED, "the backward takes bf16 inputs (dtype=%d)", d->dtype);
  return CP_OK;
}

int64_t tensor_elems(const cp_attn_desc* d) { return (int64_t)d->B * d->L * d->H * d->d; }

BwdArgs bwd_args(const cp_attn_desc* d, int32_t j, const void* q, const void* k, const void* v, const void* d_o,
                 const float* lse, const float* delta, float* dq, float* dk, float* dv, bool accumulate) {
  BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.d_o = d_o;
  a.lse = lse;
  a.delta = delta;
  a.L = d->L;
  a.B = d->B;
  a.H = d->H;
  a.q_pos0 = (int64_t)d->rank * d->L;
  a.k_pos0 = (int64_t)j * d->L;
  a.mask = d->mask;
  a.ndocs = d->ndocs;
  a.cu = d->mask == CP_MASK_DOC_CAUSAL ? d->cu_seqlens_dev : nullptr;
  a.scale_log2 = scale_log2(d);
  a.scale = a.scale_log2 / 1.442695040888963407360f;
  a.accumulate = accumulate ? 1 : 0;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  return a;
}

// One block's backward after validation: kernels for a visible block, zeros
// for an invisible one (dq only with INIT).
cp_status run_block_backward(const cp_attn_desc* d, int32_t j, bool accumulate, const void* q, const void* k,
                             const void* v, const void* d_o, const float* lse, const float* delta, float* dq,
                             float* dk, float* dv, hipStream_t s) {
  hipError_t e;
  if (!block_visible(d, j)) {
    const int64_t n = tensor_elems(d);
    if ((e = launch_zero(dk, n, s)) != hipSuccess) return hip_fail(e, "zero fill");
    if ((e = launch_zero(dv, n, s)) != hipSuccess) return hip_fail(e, "zero fill");
    if (!accumulate && (e = launch_zero(dq, n, s)) != hipSuccess) return hip_fail(e, "zero fill");
    return CP_OK;
  }
  const BwdArgs a = bwd_args(d, j, q, k, v, d_o, lse, delta, dq, dk, dv, accumulate);
  if ((e = launch_bwd_blocks(a, d->d, s)) != hipSuccess) return hip_fail(e, "backward kernel launch");
  return CP_OK;
}

}  // namespace

cp_status cp_attn_bwd_delta(const cp_attn_desc* desc, const void* o, const void* d_o, float* delta, void* stream) {
  g_last_error.clear();
  cp_status st = check_bwd_desc(desc);
  if (st != CP_OK) return st;
  if ((st = check_tensor(o, "o")) != CP_OK || (st = check_tensor(d_o, "d_o")) != CP_OK ||
      (st = check_vec(delta, "delta", false)) != CP_OK)
    return st;
  DeltaArgs a;
  a.o = o;
  a.d_o = d_o;
  a.L = desc->L;
  a.B = desc->B;
  a.H = desc->H;
  a.delta = delta;
  const hipError_t e = launch_bwd_delta(a, desc->d, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "delta kernel launch");
  return CP_OK;
}

cp_status cp_attn_block_backward(const cp_attn_desc* desc, int32_t j, int32_t mode, const void* q, const void* k_j,
                                 const void* v_j, const void* d_o, const float* lse, const float* delta, float* dq,
                                 float* dk_j, float* dv_j, void* stream) {
  g_last_error.clear();
  cp_status st = check_bwd_desc(desc);
  if (st != CP_OK) return st;
  if (j < 0 || j >= desc->N) return fail(CP_ERR_INVALID_ARG, "block j=%d outside [0, N=%d)", j, desc->N);
  if (mode != CP_MODE_INIT && mode != CP_MODE_ACCUMULATE)
    return fail(CP_ERR_INVALID_ARG, "mode=%d: the backward takes INIT or ACCUMULATE", mode);
  if ((st = check_tensor(q, "q")) != CP_OK || (st = check_tensor(k_j, "k_j")) != CP_OK ||
      (st = check_tensor(v_j, "v_j")) != CP_OK || (st = check_tensor(d_o, "d_o")) != CP_OK ||
      (st = check_vec(lse, "lse", false)) != CP_OK || (st = check_vec(delta, "delta", false)) != CP_OK ||
      (st = check_tensor(dq, "dq")) != CP_OK || (st = check_tensor(dk_j, "dk_j")) != CP_OK ||
      (st = check_tensor(dv_j, "dv_j")) != CP_OK)
    return st;
  return run_block_backward(desc, j, mode == CP_MODE_ACCUMULATE, q, k_j, v_j, d_o, lse, delta, dq, dk_j, dv_j,
                            (hipStream_t)stream);
}

cp_status cp_attn_rank_backward(const cp_attn_desc* desc, const void* q, const void* const* k_blocks,
                                const void* const* v_blocks, const void* o, const void* d_o, const float* lse,
                                float* delta, float* dq, float* const* dk_blocks, float* const* dv_blocks,
                                int32_t flags, void* stream) {
  g_last_error.clear();
  cp_status st = check_bwd_desc(desc);
  if (st != CP_OK) return st;
  if (flags & ~CP_RING_REVERSE) return fail(CP_ERR_INVALID_ARG, "unknown flags 0x%x (only CP_RING_REVERSE)", flags);
  if ((st = check_tensor(q, "q")) != CP_OK || (st = check_tensor(o, "o")) != CP_OK ||
      (st = check_tensor(d_o, "d_o")) != CP_OK || (st = check_vec(lse, "lse", false)) != CP_OK ||
      (st = check_vec(delta, "delta", false)) != CP_OK || (st = check_tensor(dq, "dq")) != CP_OK)
    return st;
  if (!k_blocks || !v_blocks || !dk_blocks || !dv_blocks)
    return fail(CP_ERR_INVALID_ARG, "k_blocks/v_blocks/dk_blocks/dv_blocks is NULL");
  const std::vector<int32_t> sched = schedule(desc, flags);
  for (int32_t j = 0; j < desc->N; ++j) {
    if ((st = check_tensor(dk_blocks[j], "dk_blocks[j]")) != CP_OK ||
        (st = check_tensor(dv_blocks[j], "dv_blocks[j]")) != CP_OK)
      return st;
  }
  for (int32_t j : sched) {
    if ((st = check_tensor(k_blocks[j], "k_blocks[j]")) != CP_OK || (st = check_tensor(v_blocks[j], "v_blocks[j]")) != CP_OK)
      return st;
  }
  if (sched.empty()) return fail(CP_ERR_INVALID_ARG, "no visible block");   // unreachable: the diagonal is visible
  hipStream_t s = (hipStream_t)stream;
  if ((st = cp_attn_bwd_delta(desc, o, d_o, delta, stream)) != CP_OK) return st;
  std::vector<char> seen(desc->N, 0);
  bool first = true;
  for (int32_t j : sched) {
    if ((st = run_block_backward(desc, j, !first, q, k_blocks[j], v_blocks[j], d_o, lse, delta, dq, dk_blocks[j],
                                 dv_blocks[j], s)) != CP_OK)
      return st;
    seen[j] = 1;
    first = false;
  }
  const int64_t n = tensor_elems(desc);
  for (int32_t j = 0; j < desc->N; ++j) {
    if (seen[j]) continue;
    hipError_t e;
    if ((e = launch_zero(dk_blocks[j], n, s)) != hipSuccess || (e = launch_zero(dv_blocks[j], n, s)) != hipSuccess)
      return hip_fail(e, "zero fill");
  }
  return CP_OK;
}

// The ring forward of one rank; with fp8 set, q and the blocks hold e4m3
// codes with the given per-(b, h) scales and the output is bf16.
static cp_status rank_forward_impl(const cp_attn_desc* desc, const void* q, const void* const* k_blocks,
                                   const void* const* v_blocks, void* out, float* m_out, float* l_out, float* lse_out,
                                   void* workspace, size_t workspace_bytes, void* compute_stream, void* copy_stream,
                                   int32_t flags, cp_attn_profiler* prof, bool fp8, const float* q_scale,
                                   const float* const* k_scales, const float* const* v_scales,
                                   bool static_ws = false) {
  g_last_error.clear();
  cp_status st = check_desc(desc);
  if (st != CP_OK) return st;
  if (fp8) {
    if (desc->dtype != CP_BF16)
      return fail(CP_ERR_UNSUPPORTED, "the FP8 forward writes a bf16 output: desc->dtype must be bf16 (dtype=%d)", desc->dtype);
    if ((st = check_vec(q_scale, "q_scale", false)) != CP_OK) return st;
    if (!k_scales || !v_scales) return fail(CP_ERR_INVALID_ARG, "k_scales/v_scales is NULL");
  }
  if (flags & ~(CP_RING_PREFETCH | CP_RING_REVERSE)) return fail(CP_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((st = check_tensor(q, "q")) != CP_OK || (st = check_tensor(out, "out")) != CP_OK ||
      (st = check_vec(m_out, "m_out", true)) != CP_OK || (st = check_vec(l_out, "l_out", true)) != CP_OK ||
      (st = check_vec(lse_out, "lse_out", true)) != CP_OK)
    return st;
  if (!k_blocks || !v_blocks) return fail(CP_ERR_INVALID_ARG, "k_blocks/v_blocks is NULL");
  const std::vector<int32_t> sched = schedule(desc, flags);
  for (int32_t j : sched) {
    if ((st = check_tensor(k_blocks[j], "k_blocks[j]")) != CP_OK || (st = check_tensor(v_blocks[j], "v_blocks[j]")) != CP_OK)
      return st;
    if (fp8 && ((st = check_vec(k_scales[j], "k_scales[j]", false)) != CP_OK ||
                (st = check_vec(v_scales[j], "v_scales[j]", false)) != CP_OK))
      return st;
  }
  const WorkspaceLayout wl = layout_of(desc);
  if (static_ws) {
    if (wl.total > CP_STATIC_SCRATCH_BYTES)
      return fail(CP_ERR_WORKSPACE,
                  "this shard needs %zu bytes of scratch, more than the %zu of the static scratch "
                  "(CP_STATIC_SCRATCH_BYTES): use cp_attn_rank_forward with a workspace",
                  wl.total, (size_t)CP_STATIC_SCRATCH_BYTES);
  } else {
    if (!workspace) return fail(CP_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(CP_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < wl.total)
      return fail(CP_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, wl.total);
  }
  const bool prefetch = flags & CP_RING_PREFETCH;
  if (prefetch && (copy_stream == compute_stream))
    return fail(CP_ERR_INVALID_ARG, "CP_RING_PREFETCH needs a copy_stream distinct from compute_stream");
  if (sched.empty()) return fail(CP_ERR_INVALID_ARG, "no visible block");   // unreachable: the diagonal is visible
  if (static_ws) {
    // every argument is valid: the first HIP call looks up this device's array
    const hipError_t se = static_scratch(&workspace, &workspace_bytes);
    if (se != hipSuccess) return hip_fail(se, "static scratch lookup");
  }

  hipStream_t cs = (hipStream_t)compute_stream;
  hipStream_t xs = (hipStream_t)copy_stream;
  char* ws = (char*)workspace;
  const size_t blk_bytes = (size_t)desc->B * desc->L * desc->H * desc->d * (fp8 ? 1 : elt_bytes(desc->dtype));
  const int32_t nsteps = (int32_t)sched.size();
  // bf16 and e4m3 V blocks are received in head-dim-major key tiles (the
  // receive writes that layout; the attention kernel fetches each tile as one
  // contiguous run and reads V^T operands as whole 16-byte rows)
  const bool v_tiled = fp8 || desc->dtype == CP_BF16;

  // ready[t]: block of step t is in its slot; done[t]: step t's kernel
  // finished with its slot.  Both are bound to the dispatch they follow (the
  // receive's last kernel, the attention kernel), so that the cross-stream
  // dependencies add no marker packets between dependent kernels; with a
  // profiler its events take those places.
  std::vector<hipEvent_t> ready(nsteps, nullptr), done(nsteps, nullptr);
  std::vector<hipEvent_t> ready_at(nsteps, nullptr), done_at(nsteps, nullptr);   // the events to wait for
  hipError_t e = hipSuccess;
  hipEvent_t start_ev = nullptr;   // the copy stream's start (inputs ready), with prefetch
  auto cleanup = [&]() {
    for (auto ev : ready) if (ev) (void)hipEventDestroy(ev);
    for (auto ev : done) if (ev) (void)hipEventDestroy(ev);
    if (start_ev) (void)hipEventDestroy(start_ev);
  };
  if (prefetch) {
    for (int32_t t = 0; t < nsteps; ++t) {
      if ((e = hipEventCreate(&ready[t])) != hipSuccess || (e = hipEventCreate(&done[t])) != hipSuccess) {
        cleanup();
        return hip_fail(e, "hipEventCreate");
      }
    }
  }
  auto slot_k = [&](int32_t t) { return (void*)(ws + wl.slot_k[t & 1]); };
  auto slot_v = [&](int32_t t) { return (void*)(ws + wl.slot_v[t & 1]); };
  // The receive of step t into its slots; with prefetch, ready_at[t] is set to
  // the event that completes with it.
  auto enqueue_copy = [&](int32_t t, hipStream_t s) -> hipError_t {
    const int32_t j = sched[t];
    const bool timed = prof && prof->copies < (int32_t)prof->copy_start.size();
    hipError_t r;
    if (timed && (r = hipEventRecord(prof->copy_start[prof->copies], s)) != hipSuccess) return r;
    r = hipMemcpyAsync(slot_k(t), k_blocks[j], blk_bytes, hipMemcpyDeviceToDevice, s);
    if (r != hipSuccess) return r;
    hipEvent_t fin = timed ? prof->copy_stop[prof->copies] : (prefetch ? ready[t] : nullptr);
    if (v_tiled) {
      const LaunchEvents ev{nullptr, fin};
      r = fp8 ? launch_v_tiles_fp8(v_blocks[j], slot_v(t), desc->L, desc->B, desc->H, desc->d, s, ev)
              : launch_v_tiles(v_blocks[j], slot_v(t), desc->L, desc->B, desc->H, desc->d, s, ev);
    } else {
      r = hipMemcpyAsync(slot_v(t), v_blocks[j], blk_bytes, hipMemcpyDeviceToDevice, s);
      if (r == hipSuccess && fin) r = hipEventRecord(fin, s);
    }
    if (r != hipSuccess) return r;
    if (timed) prof->copies++;
    if (prefetch) ready_at[t] = fin;
    return hipSuccess;
  };
  // The copy stream starts after everything already queued on the compute
  // stream (the inputs are ready), but not after the first attention kernel,
  // which reads the rank's own block; that kernel is enqueued before the
  // first receive, so the compute stream does not wait on the host's
  // enqueueing of the copy.
  if (prefetch && nsteps > 1) {
    if ((e = hipEventCreateWithFlags(&start_ev, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventRecord(start_ev, cs)) != hipSuccess) {
      cleanup();
      return hip_fail(e, "copy stream start");
    }
  }
  auto start_copies = [&]() -> hipError_t {
    hipError_t r = hipStreamWaitEvent(xs, start_ev, 0);
    (void)hipEventDestroy(start_ev);
    start_ev = nullptr;
    if (r != hipSuccess) return r;
    return enqueue_copy(1, xs);
  };

  for (int32_t t = 0; t < nsteps; ++t) {
    const int32_t j = sched[t];
    const void* kp = t == 0 ? k_blocks[j] : slot_k(t);
    const void* vp = t == 0 ? v_blocks[j] : slot_v(t);
    if (t > 0) {
      if (prefetch) e = hipStreamWaitEvent(cs, ready_at[t], 0);
      else e = enqueue_copy(t, cs);
      if (e != hipSuccess) { cleanup(); return hip_fail(e, "ring receive"); }
    }
    BlockArgs a = block_args(desc, j, q, kp, vp);
    if (fp8) {
      a.q_scale = q_scale;
      a.k_scale = k_scales[j];
      a.v_scale = v_scales[j];
    }
    // Mask-aware rows: this step runs the rows that see block j only, and a
    // row that sees no later block of the schedule stores its final output
    // here (those are the rows from final_from on; the others keep the state)
    a.rows_end = rows_seeing(desc, j);
    int64_t later = 0;
    for (int32_t u = t + 1; u < nsteps; ++u) {
      const int64_t r = rows_seeing(desc, sched[u]);
      if (r > later) later = r;
    }
    a.final_from = later;
    a.flags = (t > 0 ? F_READ_STATE : 0) | F_WRITE_STATE | F_WRITE_FINAL | (t > 0 && v_tiled ? F_V_TILED : 0);
    a.st_o = (float*)(ws + wl.st_o);
    a.st_m = (float*)(ws + wl.st_m);
    a.st_l = (float*)(ws + wl.st_l);
    if (!fp8) fill_order(desc, j, a);
    if (wl.side && !fp8 && t < 2) {
      // key split of the diagonal block (step 0, the rank's own block), merged
      // by step 1 (a full block: every row reads its state there)
      a.flags |= t == 0 ? F_SPLIT : F_READ_SIDE;
      a.split_from = split_from_of(desc);
      a.side_o = (float*)(ws + wl.side_o);
      a.side_m = (float*)(ws + wl.side_m);
      a.side_l = (float*)(ws + wl.side_l);
    }
    a.out = out;
    a.m_out = m_out;
    a.l_out = l_out;
    a.lse_out = lse_out;
    // the receive for step t+2 reuses the slot of step t: it waits for this kernel
    const bool reuse = prefetch && t + 1 < nsteps - 1;
    const bool timed = prof && prof->used < (int32_t)prof->start.size();
    LaunchEvents ev;
    if (timed) ev = LaunchEvents{prof->start[prof->used], prof->stop[prof->used]};
    else if (reuse) ev.stop = done[t];
    e = fp8 ? launch_block_fp8(a, desc->d, cs, ev) : launch_block(desc, a, cs, ev);
    if (e != hipSuccess) { cleanup(); return hip_fail(e, "block kernel launch"); }
    if (timed) prof->used++;
    done_at[t] = ev.stop;
    if (t == 0 && start_ev && (e = start_copies()) != hipSuccess) { cleanup(); return hip_fail(e, "ring receive copy"); }
    if (reuse) {
      if ((e = hipStreamWaitEvent(xs, done_at[t], 0)) != hipSuccess || (e = enqueue_copy(t + 2, xs)) != hipSuccess) {
        cleanup();
        return hip_fail(e, "ring receive copy");
      }
    }
  }
  cleanup();
  return CP_OK;
}

cp_status cp_attn_rank_forward(const cp_attn_desc* desc, const void* q, const void* const* k_blocks,
                               const void* const* v_blocks, void* out, float* m_out, float* l_out, float* lse_out,
                               void* workspace, size_t workspace_bytes, void* compute_stream, void* copy_stream,
                               int32_t flags, cp_attn_profiler* prof) {
  return rank_forward_impl(desc, q, k_blocks, v_blocks, out, m_out, l_out, lse_out, workspace, workspace_bytes,
                           compute_stream, copy_stream, flags, prof, false, nullptr, nullptr, nullptr);
}

cp_status cp_attn_rank_forward_static(const cp_attn_desc* desc, const void* q, const void* const* k_blocks,
                                      const void* const* v_blocks, void* out, float* m_out, float* l_out,
                                      float* lse_out, void* compute_stream, void* copy_stream, int32_t flags,
                                      cp_attn_profiler* prof) {
  return rank_forward_impl(desc, q, k_blocks, v_blocks, out, m_out, l_out, lse_out, nullptr, 0, compute_stream,
                           copy_stream, flags, prof, false, nullptr, nullptr, nullptr, true);
}

cp_status cp_attn_rank_forward_fp8(const cp_attn_desc* desc, const void* q, const float* q_scale,
                                   const void* const* k_blocks, const float* const* k_scales,
                                   const void* const* v_blocks, const float* const* v_scales, void* out,
                                   float* m_out, float* l_out, float* lse_out, void* workspace,
                                   size_t workspace_bytes, void* compute_stream, void* copy_stream, int32_t flags,
                                   cp_attn_profiler* prof) {
  return rank_forward_impl(desc, q, k_blocks, v_blocks, out, m_out, l_out, lse_out, workspace, workspace_bytes,
                           compute_stream, copy_stream, flags, prof, true, q_scale, k_scales, v_scales);
}

cp_status cp_attn_measure_lds_stream(const void* src, size_t bytes, void* stream) {
  g_last_error.clear();
  cp_status st = check_tensor(src, "src");
  if (st != CP_OK) return st;
  if (bytes == 0 || bytes % 4096 != 0 || bytes > ((size_t)1 << 46))
    return fail(CP_ERR_INVALID_ARG, "bytes=%zu must be a positive multiple of 4096", bytes);
  const hipError_t e = launch_lds_stream(src, (int64_t)bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "measurement kernel launch");
  return CP_OK;
}

cp_status cp_attn_profiler_create(int32_t capacity, cp_attn_profiler** out) {
  g_last_error.clear();
  if (!out) return fail(CP_ERR_INVALID_ARG, "out is NULL");
  if (capacity < 1 || capacity > (1 << 20)) return fail(CP_ERR_INVALID_ARG, "capacity=%d outside [1, 2^20]", capacity);
  cp_attn_profiler* p = new (std::nothrow) cp_attn_profiler;
  if (!p) return fail(CP_ERR_INVALID_ARG, "out of host memory");
  p->start.assign(capacity, nullptr);
  p->stop.assign(capacity, nullptr);
  p->copy_start.assign(capacity, nullptr);
  p->copy_stop.assign(capacity, nullptr);
  for (int32_t i = 0; i < capacity; ++i) {
    hipError_t e = hipEventCreate(&p->start[i]);
    if (e == hipSuccess) e = hipEventCreate(&p->stop[i]);
    if (e == hipSuccess) e = hipEventCreate(&p->copy_start[i]);
    if (e == hipSuccess) e = hipEventCreate(&p->copy_stop[i]);
    if (e != hipSuccess) {
      cp_attn_profiler_destroy(p);
      return hip_fail(e, "hipEventCreate");
    }
  }
  *out = p;
  return CP_OK;
}

cp_status cp_attn_profiler_reset(cp_attn_profiler* prof) {
  g_last_error.clear();
  if (!prof) return fail(CP_ERR_INVALID_ARG, "prof is NULL");
  prof->used = 0;
  prof->copies = 0;
  return CP_OK;
}

cp_status cp_attn_profiler_read(cp_attn_profiler* prof, float* ms_out, int32_t capacity, int32_t* count_out) {
  g_last_error.clear();
  if (!prof || !count_out) return fail(CP_ERR_INVALID_ARG, "prof/count_out is NULL");
  if (capacity < prof->used || (!ms_out && prof->used > 0))
    return fail(CP_ERR_INVALID_ARG, "capacity %d < %d recorded launches", capacity, prof->used);
  for (int32_t i = 0; i < prof->used; ++i) {
    hipError_t e = hipEventSynchronize(prof->stop[i]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms_out[i], prof->start[i], prof->stop[i]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
  }
  *count_out = prof->used;
  return CP_OK;
}

cp_status cp_attn_profiler_read_copies(cp_attn_profiler* prof, float* ms_out, int32_t capacity, int32_t* count_out) {
  g_last_error.clear();
  if (!prof || !count_out) return fail(CP_ERR_INVALID_ARG, "prof/count_out is NULL");
  if (capacity < prof->copies || (!ms_out && prof->copies > 0))
    return fail(CP_ERR_INVALID_ARG, "capacity %d < %d recorded receives", capacity, prof->copies);
  for (int32_t i = 0; i < prof->copies; ++i) {
    hipError_t e = hipEventSynchronize(prof->copy_stop[i]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms_out[i], prof->copy_start[i], prof->copy_stop[i]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
  }
  *count_out = prof->copies;
  return CP_OK;
}

void cp_attn_profiler_destroy(cp_attn_profiler* prof) {
  if (!prof) return;
  for (auto ev : prof->start) if (ev) (void)hipEventDestroy(ev);
  for (auto ev : prof->stop) if (ev) (void)hipEventDestroy(ev);
  for (auto ev : prof->copy_start) if (ev) (void)hipEventDestroy(ev);
  for (auto ev : prof->copy_stop) if (ev) (void)hipEventDestroy(ev);
  delete prof;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// all-to-all (Ulysses) context parallelism, one rank's share
// ---------------------------------------------------------------------------
namespace {

static_assert(kMaxShards == CP_MAX_RING, "regroup pointer table sized to the ring limit");

// The description of the attention a rank runs after the first all-to-all:
// one block of the whole sequence (N = 1, L = S) on H/N heads.
cp_status ulysses_full_desc(const cp_attn_desc* d, cp_attn_desc* full) {
  cp_status st = check_desc(d);
  if (st != CP_OK) return st;
  if (d->H % d->N != 0)
    return fail(CP_ERR_INVALID_ARG, "H=%d is not a multiple of N=%d (each rank takes H/N heads)", d->H, d->N);
  *full = *d;
  full->N = 1;
  full->rank = 0;
  full->L = d->L * d->N;
  full->H = d->H / d->N;
  return check_desc(full);
}

size_t ulysses_full_bytes(const cp_attn_desc* full) {
  return round_up((size_t)full->B * full->L * full->H * full->d * elt_bytes(full->dtype), 256);
}

}  // namespace

extern "C" {

size_t cp_attn_ulysses_workspace_bytes(const cp_attn_desc* desc) {
  g_last_error.clear();
  cp_attn_desc full;
  if (ulysses_full_desc(desc, &full) != CP_OK) return 0;
  return 4 * ulysses_full_bytes(&full);
}

cp_status cp_attn_ulysses_forward(const cp_attn_desc* desc, const void* const* q_shards,
                                  const void* const* k_shards, const void* const* v_shards,
                                  void* const* o_shards, float* m_out, float* l_out, float* lse_out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  cp_attn_desc full;
  cp_status st = ulysses_full_desc(desc, &full);
  if (st != CP_OK) return st;
  if (!q_shards || !k_shards || !v_shards || !o_shards)
    return fail(CP_ERR_INVALID_ARG, "q_shards/k_shards/v_shards/o_shards is NULL");
  for (int32_t i = 0; i < desc->N; ++i) {
    if ((st = check_tensor(q_shards[i], "q_shards[i]")) != CP_OK || (st = check_tensor(k_shards[i], "k_shards[i]")) != CP_OK ||
        (st = check_tensor(v_shards[i], "v_shards[i]")) != CP_OK || (st = check_tensor(o_shards[i], "o_shards[i]")) != CP_OK)
      return st;
  }
  if ((st = check_vec(m_out, "m_out", true)) != CP_OK || (st = check_vec(l_out, "l_out", true)) != CP_OK ||
      (st = check_vec(lse_out, "lse_out", true)) != CP_OK)
    return st;
  const size_t fb = ulysses_full_bytes(&full);
  if (!workspace) return fail(CP_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(CP_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < 4 * fb) return fail(CP_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, 4 * fb);

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  void* qf = ws;
  void* kf = ws + fb;
  void* vf = ws + 2 * fb;
  void* of = ws + 3 * fb;
  RegroupArgs ra;
  std::memset(&ra, 0, sizeof(ra));
  ra.B = desc->B;
  ra.L = desc->L;
  ra.S = full.L;
  ra.N = desc->N;
  ra.H = desc->H;
  ra.Hn = full.H;
  ra.h0 = desc->rank * full.H;
  ra.d = desc->d;
  ra.elt = (int32_t)elt_bytes(desc->dtype);
  hipError_t e = hipSuccess;
  // bf16 V over whole 64-key tiles is gathered straight into the tiled layout
  // (the same bytes; the attention kernel reads V^T operands as 16-byte rows)
  const bool v_tiled = desc->dtype == CP_BF16 && full.L % 64 == 0;
  // step 1: the first all-to-all, as seen by this rank (its heads of every shard)
  const void* const* srcs[3] = {q_shards, k_shards, v_shards};
  void* dsts[3] = {qf, kf, vf};
  for (int x = 0; x < 3; ++x) {
    for (int32_t i = 0; i < desc->N; ++i) ra.shards[i] = const_cast<void*>(srcs[x][i]);
    ra.full = dsts[x];
    e = (x == 2 && v_tiled) ? launch_a2a_gather_v_tiles(ra, s) : launch_a2a_gather(ra, s);
    if (e != hipSuccess) return hip_fail(e, "all-to-all gather launch");
  }
  // step 2: attention over the whole sequence for this rank's heads
  BlockArgs a = block_args(&full, 0, qf, kf, vf);
  a.flags = F_WRITE_FINAL | (v_tiled ? F_V_TILED : 0);
  a.out = of;
  a.m_out = m_out;
  a.l_out = l_out;
  a.lse_out = lse_out;
  if ((e = launch_block(&full, a, s)) != hipSuccess) return hip_fail(e, "block kernel launch");
  // step 3: the second all-to-all, as sent by this rank (its heads of every shard)
  for (int32_t i = 0; i < desc->N; ++i) ra.shards[i] = o_shards[i];
  ra.full = of;
  if ((e = launch_a2a_scatter(ra, s)) != hipSuccess) return hip_fail(e, "all-to-all scatter launch");
  return CP_OK;
}

cp_status cp_attn_quantize_fp8(const cp_attn_desc* desc, const void* x, int32_t role, void* codes, float* scales,
                               void* stream) {
  g_last_error.clear();
  cp_status st = check_desc(desc);
  if (st != CP_OK) return st;
  if (desc->dtype != CP_BF16) return fail(CP_ERR_UNSUPPORTED, "cp_attn_quantize_fp8 takes bf16 input (dtype=%d)", desc->dtype);
  if (role != CP_FP8_KV && role != CP_FP8_QUERY) return fail(CP_ERR_INVALID_ARG, "unknown FP8 role %d", role);
  if ((st = check_tensor(x, "x")) != CP_OK) return st;
  if (!codes) return fail(CP_ERR_INVALID_ARG, "codes is NULL");
  if (!aligned(codes, 8)) return fail(CP_ERR_INVALID_ARG, "codes is not 8-byte aligned");
  if ((st = check_vec(scales, "scales", false)) != CP_OK) return st;
  if ((long double)desc->L / 256 + 1 > 2147483647.0L || (long double)desc->B * desc->H > 65535.0L)
    return fail(CP_ERR_UNSUPPORTED, "grid of the quantisation too large (B*H=%lld)", (long long)desc->B * desc->H);
  QuantArgs a;
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.L = desc->L;
  a.B = desc->B;
  a.H = desc->H;
  const float prescale = role == CP_FP8_QUERY ? scale_log2(desc) : 1.0f;
  const hipError_t e = launch_quantize_fp8(a, desc->d, prescale, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quantisation launch");
  return CP_OK;
}

}  // extern "C"
