// Host side of the C ABI declared in include/paged_gqa.h: argument checks,
// split-KV planning and kernel launches.  Every host-checkable condition is
// checked before the first launch, so a rejected call launches nothing.
#include "paged_gqa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <climits>
#include <cmath>
#include <cstdint>
#include <random>

#include "pga_args.h"

namespace {

using pga::KvArgs;

constexpr int kBF16 = PGA_DTYPE_BF16;
constexpr int kFP8 = PGA_DTYPE_FP8_E4M3;
constexpr int kHeadDim = PGA_HEAD_DIM;
constexpr int kMaxRowsPerGroup = 64;   // query rows of one kv group a verify workgroup holds
constexpr int kTileKeys = 64;          // keys per LDS tile of the causal kernels
constexpr int kMinTilesPerWg = pga::kVerifyMinTilesPerWg;  // verify: shortest run one workgroup takes
constexpr int kMaxVerifyWgs = pga::kVerifyMaxWgs;          // verify: cap of the persistent grid
constexpr int kMaxGridYZ = 65535;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int64_t x) {
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}
int elt_bytes(int dt) { return dt == kFP8 ? 1 : 2; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Checks of the KV descriptor shared by all calls.  `pages_per_seq` is the
// number of block-table columns the call may read (-1: not host-checkable).
int check_kv(const pga_paged_kv* kv, int32_t num_q_heads, int64_t pages_per_seq) {
  if (!kv) return PGA_ERR_NULL;
  if (!kv->k_cache || !kv->v_cache || !kv->block_table) return PGA_ERR_NULL;
  if (kv->dtype != kBF16 && kv->dtype != kFP8) return PGA_ERR_DTYPE;
  if (kv->head_dim != kHeadDim) return PGA_ERR_SHAPE;
  if (kv->num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % kv->num_kv_heads != 0) return PGA_ERR_SHAPE;
  if (kv->num_kv_heads > kMaxGridYZ) return PGA_ERR_UNSUPPORTED;
  if (kv->num_pages <= 0) return PGA_ERR_SHAPE;
  if (!pow2(kv->page_size) || kv->page_size < 16 || kv->page_size > 1024) return PGA_ERR_UNSUPPORTED;
  const int64_t per16 = 16 / elt_bytes(kv->dtype);  // elements in 16 bytes
  const int64_t st[6] = {kv->k_stride_page, kv->k_stride_token, kv->k_stride_head,
                         kv->v_stride_page, kv->v_stride_token, kv->v_stride_head};
  for (int64_t s : st)
    if (s < 0 || s % per16 != 0) return PGA_ERR_UNSUPPORTED;
  // Within a page, token rows are addressed by 32-bit byte offsets.
  const int64_t tok_bytes = std::max(kv->k_stride_token, kv->v_stride_token) * elt_bytes(kv->dtype);
  if (tok_bytes * kv->page_size + kHeadDim * elt_bytes(kv->dtype) > INT32_MAX) return PGA_ERR_UNSUPPORTED;
  if (!aligned(kv->k_cache, 16) || !aligned(kv->v_cache, 16)) return PGA_ERR_UNSUPPORTED;
  if (kv->block_table_stride < 0 || (pages_per_seq > 0 && kv->block_table_stride < pages_per_seq))
    return PGA_ERR_SHAPE;
  return PGA_OK;
}

KvArgs make_kv(const pga_paged_kv* kv) {
  const int64_t e = elt_bytes(kv->dtype);
  KvArgs a;
  a.k = static_cast<const uint8_t*>(kv->k_cache);
  a.v = static_cast<const uint8_t*>(kv->v_cache);
  a.k_sp = kv->k_stride_page * e;
  a.k_st = kv->k_stride_token * e;
  a.k_sh = kv->k_stride_head * e;
  a.v_sp = kv->v_stride_page * e;
  a.v_st = kv->v_stride_token * e;
  a.v_sh = kv->v_stride_head * e;
  a.bt = kv->block_table;
  a.bt_stride = kv->block_table_stride;
  a.page_size = kv->page_size;
  a.page_shift = ilog2(kv->page_size);
  a.num_pages = kv->num_pages;
  a.num_kv_heads = kv->num_kv_heads;
  a.k_ds = kv->k_descale;
  a.v_ds = kv->v_descale;
  return a;
}

struct VerifyPlan {
  int32_t seg_tiles = 0;   // 64-key tiles per segment
  int32_t max_segs = 0;    // segments per (sequence, kv head), host bound
  int32_t rows_cap = 0;    // r * max_q_len
  int32_t wg_cap = 0;      // bound of the persistent grid (device independent)
  size_t ws_o_bytes = 0, ws_lse_bytes = 0, ws_bytes = 0;
};

// Verify work plan from the host bounds.  The workspace holds one slot per
// (segment, workgroup) piece -- at most #segments + #workgroups of them -- of
// partial rows and their lse values, then the plan the merge reads: per
// (sequence, kv head) unit its first tile and first segment in the flattened
// order, and the tiles per workgroup.
// Returns PGA_OK, PGA_ERR_SHAPE (invalid arguments) or PGA_ERR_UNSUPPORTED (the
// flattened work list or the slot indices would not fit the kernels' int32
// positions).
int plan_verify(int32_t hq, int32_t hkv, int32_t num_seqs, int32_t max_q_len, int32_t max_kv_len,
                int32_t kv_split_tokens, VerifyPlan& p) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || num_seqs < 0 || max_q_len < 1 || max_kv_len < 0) return PGA_ERR_SHAPE;
  if (kv_split_tokens < 0 || kv_split_tokens % kTileKeys != 0) return PGA_ERR_SHAPE;
  const int64_t tiles_bound = cdiv(max_kv_len, kTileKeys);
  p.seg_tiles = kv_split_tokens > 0 ? kv_split_tokens / kTileKeys
                                    : static_cast<int32_t>(std::max<int64_t>(1, tiles_bound));
  p.max_segs = static_cast<int32_t>(std::max<int64_t>(1, cdiv(tiles_bound, p.seg_tiles)));
  p.rows_cap = (hq / hkv) * max_q_len;
  const int64_t units = int64_t(num_seqs) * hkv;
  // Every list position (tiles plus the start cost of each segment, over all
  // units, and a workgroup's run end wg * tpw past the total) and every slot
  // index (segments plus workgroups) is an int32 in the kernels; the per-unit
  // plan entries are addressed as 2 * units.  Half the int32 range leaves the
  // run ends their margin.
  if (units * (tiles_bound + int64_t(pga::kVerifySegStartCost) * p.max_segs) > INT32_MAX / 2 ||
      units * p.max_segs + kMaxVerifyWgs > INT32_MAX / 2 || 2 * units + 4 > INT32_MAX / 2)
    return PGA_ERR_UNSUPPORTED;
  // Enough workgroups for runs of kMinTilesPerWg positions over the whole
  // list, start positions included (the kernel's run length is the list
  // length over the grid, at least kMinTilesPerWg).
  const int64_t list_bound = units * (tiles_bound + int64_t(pga::kVerifySegStartCost) * p.max_segs);
  p.wg_cap = static_cast<int32_t>(std::min<int64_t>(kMaxVerifyWgs, std::max<int64_t>(1, cdiv(list_bound, kMinTilesPerWg))));
  if (units > 0 && tiles_bound > 0) {
    const size_t slots = size_t(units) * p.max_segs + p.wg_cap;
    p.ws_o_bytes = slots * p.rows_cap * kHeadDim * sizeof(float);
    p.ws_o_bytes = (p.ws_o_bytes + 255) & ~size_t(255);
    p.ws_lse_bytes = (slots * p.rows_cap * sizeof(float) + 15) & ~size_t(15);
    p.ws_bytes = p.ws_o_bytes + p.ws_lse_bytes + (size_t(units) * 2 + 4) * sizeof(int32_t);
  }
  return PGA_OK;
}

// Compute units of the current device (cached per device; 256 if unknown).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

int launch_status(hipError_t e) { return e == hipSuccess ? PGA_OK : PGA_ERR_LAUNCH; }

// A 48-bit odd tag unique to each quantisation call of this process: a
// random start drawn once plus twice the call count (the barrier of the
// single-read path recognises this call's slots by it, whatever the
// workspace held before).
uint64_t next_quant_tag() {
  static const uint64_t start = [] {
    uint64_t r = static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count());
    r ^= reinterpret_cast<uintptr_t>(&r) << 16;
    try {
      std::random_device rd;
      r ^= (uint64_t(rd()) << 32) ^ rd();
    } catch (...) {
    }
    return r;
  }();
  static std::atomic<uint64_t> calls{0};
  return ((start + 2 * calls.fetch_add(1, std::memory_order_relaxed)) | 1u) & ((uint64_t(1) << 48) - 1);
}

}  // namespace

// Sparse split plan from the host arguments alone.  When the rows' jobs
// (query token x kv head x 16-row block) would not fill the GPU, each row's
// index list is cut into pieces (multiples of 32 entries, at least 256 per
// piece, at most kMaxSparseSplits), processed by separate waves and merged by
// log-sum-exp.  The piece count minimises a round count times a piece
// length: the sparse kernels hold one workgroup per CU, so on a 256-CU part
// the waves run in rounds of 2,048 (FP8, eight waves per workgroup) or 1,024
// (BF16, four); a call's time is its rounds times one piece's tiles plus the
// cost of starting a piece (kSparsePieceStartTiles).  A few jobs past a round
// boundary cost a whole extra round, which the job count alone does not see.
constexpr int64_t kSparseTargetJobs = 4096;  // jobs at or past this fill the GPU: no split
constexpr int32_t kMaxSparseSplits = 32;
constexpr int64_t kSparseRoundWavesFp8 = 2048, kSparseRoundWavesBf16 = 1024;
constexpr int64_t kSparsePieceStartTiles = 3;  // query load, table translation, pipeline fill
struct SparsePlan {
  int32_t splits = 1, split_len = 1;
  size_t ws_o_bytes = 0, ws_bytes = 0;
};
bool plan_sparse(int32_t hq, int32_t hkv, int32_t num_q_tokens, int32_t num_selected, SparsePlan& p) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || num_q_tokens < 0 || num_selected < 0) return false;
  const int64_t jobs = int64_t(num_q_tokens) * hkv * cdiv(hq / hkv, 16);
  auto piece_len = [&](int64_t s) { return std::max<int64_t>(32, (cdiv(num_selected, s) + 31) / 32 * 32); };
  int64_t len = piece_len(1);
  if (jobs > 0 && jobs < kSparseTargetJobs && num_selected > 0) {
    const int64_t s_max = std::max<int64_t>(1, std::min<int64_t>(kMaxSparseSplits, cdiv(num_selected, 256)));
    int64_t best = -1;
    for (int64_t s = 1; s <= s_max; ++s) {
      const int64_t l = piece_len(s), pieces = cdiv(num_selected, l);
      const int64_t rounds = cdiv(jobs * pieces, kSparseRoundWavesFp8) + cdiv(jobs * pieces, kSparseRoundWavesBf16);
      const int64_t cost = rounds * (cdiv(l, 16) + kSparsePieceStartTiles);
      if (best < 0 || cost < best) {
        best = cost;
        len = l;
      }
    }
  }
  p.splits = num_selected > 0 ? static_cast<int32_t>(cdiv(num_selected, len)) : 1;
  p.split_len = static_cast<int32_t>(len);
  p.ws_o_bytes = p.ws_bytes = 0;
  if (p.splits > 1) {
    const size_t slots = size_t(num_q_tokens) * hq * p.splits;
    p.ws_o_bytes = (slots * kHeadDim * sizeof(float) + 255) & ~size_t(255);
    p.ws_bytes = p.ws_o_bytes + slots * sizeof(float);
  }
  return true;
}

extern "C" {

int pga_abi_version(void) { return PGA_ABI_VERSION; }

const char* pga_status_string(int status) {
  switch (status) {
    case PGA_OK: return "ok";
    case PGA_ERR_NULL: return "a required pointer is NULL";
    case PGA_ERR_SHAPE: return "invalid shape or length bound";
    case PGA_ERR_DTYPE: return "unsupported dtype or dtype pair";
    case PGA_ERR_UNSUPPORTED: return "outside the kernel envelope (page size, alignment, rows per kv group)";
    case PGA_ERR_WORKSPACE: return "workspace too small";
    case PGA_ERR_LAUNCH: return "kernel launch failed";
    case PGA_ERR_INVALID_DATA: return "device data break a precondition (see the counts)";
    case PGA_ERR_SCRATCH: return "the call needs more than the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

size_t paged_attn_verify_workspace_bytes(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                         int32_t max_q_len, int32_t max_kv_len, int32_t kv_split_tokens) {
  VerifyPlan p;
  if (plan_verify(num_q_heads, num_kv_heads, num_seqs, max_q_len, max_kv_len, kv_split_tokens, p) != PGA_OK) return 0;
  return p.ws_bytes;
}

int32_t paged_attn_verify_split_tokens(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                       int32_t max_q_len, int32_t max_kv_len, int32_t kv_split_tokens) {
  VerifyPlan p;
  if (plan_verify(num_q_heads, num_kv_heads, num_seqs, max_q_len, max_kv_len, kv_split_tokens, p) != PGA_OK) return 0;
  return p.seg_tiles * kTileKeys;
}

// Validates a verify call and fills the launch arguments; returns a status.
// With use_scratch the caller's workspace arguments are ignored and the
// partials go to the library's fixed per-device scratch, laid out for this
// call exactly (partial rows in their stored width, slots for the actual
// grid) and refused with PGA_ERR_SCRATCH when they do not fit.
//
// The grid of a verify call (and of its page-gather roof): the stream-K plan's
// persistent grid, or for small calls one workgroup per tile of each unit with
// no plan (at most as many slots as the plan's workspace holds, wg_cap >=
// units * tiles).  Returns the plan-free mode's tiles per unit, 0 under the plan.
static int32_t verify_grid(int32_t num_seqs, const pga_paged_kv* kv, int32_t max_kv_len, const VerifyPlan& p,
                           int& num_wg) {
  const int occupancy = kv->dtype == kFP8 ? 2 : 1;  // workgroups per CU the LDS allows
  num_wg = std::max(1, std::min(p.wg_cap, device_cus() * occupancy));
  const int64_t tiles_bound = cdiv(max_kv_len, kTileKeys);
  const int64_t static_tiles = int64_t(num_seqs) * kv->num_kv_heads * tiles_bound;
  if (tiles_bound > 0 && tiles_bound <= 64 && static_tiles <= pga::kVerifyStaticMaxTiles) {
    num_wg = static_cast<int>(static_tiles);
    return static_cast<int32_t>(tiles_bound);
  }
  return 0;
}
static int prepare_verify(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                          int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k, int32_t max_q_len,
                          int32_t max_kv_len, const pga_paged_kv* kv, float softmax_scale, int32_t kv_split_tokens,
                          void* workspace, size_t workspace_bytes, void* out, float* lse, VerifyPlan& p,
                          pga::VerifyArgs& a, int& num_wg, bool& nothing, bool use_scratch = false) {
  nothing = false;
  if (!q || !cu_seqlens_q || !seq_lens_k || !out || !kv) return PGA_ERR_NULL;
  if (num_seqs < 0 || num_q_heads <= 0 || max_kv_len < 0) return PGA_ERR_SHAPE;
  if (max_q_len < 1 || max_q_len > 4) return PGA_ERR_SHAPE;
  if (q_dtype != kBF16) return PGA_ERR_DTYPE;
  if (!std::isfinite(softmax_scale)) return PGA_ERR_SHAPE;
  if (int e = check_kv(kv, num_q_heads, cdiv(max_kv_len, kv->page_size > 0 ? kv->page_size : 1))) return e;
  const int32_t r = num_q_heads / kv->num_kv_heads;
  if (int64_t(r) * max_q_len > kMaxRowsPerGroup) return PGA_ERR_UNSUPPORTED;
  if (kv_split_tokens < 0 || kv_split_tokens % kTileKeys != 0) return PGA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(out, 8) || (lse && !aligned(lse, 4))) return PGA_ERR_UNSUPPORTED;
  if (int e = plan_verify(num_q_heads, kv->num_kv_heads, num_seqs, max_q_len, max_kv_len, kv_split_tokens, p))
    return e;
  const int32_t plan_free_tiles = verify_grid(num_seqs, kv, max_kv_len, p, num_wg);
  size_t ws_o_bytes = p.ws_o_bytes, ws_lse_bytes = p.ws_lse_bytes;
  if (use_scratch) {
    if (p.ws_bytes > 0) {
      const int64_t units = int64_t(num_seqs) * kv->num_kv_heads;
      const size_t slots = size_t(units) * p.max_segs + size_t(num_wg);
      const size_t part = kv->dtype == kFP8 ? sizeof(uint16_t) : sizeof(float);  // stored partial width
      ws_o_bytes = (slots * p.rows_cap * kHeadDim * part + 255) & ~size_t(255);
      ws_lse_bytes = (slots * p.rows_cap * sizeof(float) + 15) & ~size_t(15);
      const size_t need = ws_o_bytes + ws_lse_bytes + (size_t(units) * 2 + 4) * sizeof(int32_t);
      if (need > pga::kVerifyScratchBytes) return PGA_ERR_SCRATCH;
    }
    workspace = nullptr;
  } else {
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return PGA_ERR_WORKSPACE;
    if (p.ws_bytes > 0 && !aligned(workspace, 256)) return PGA_ERR_UNSUPPORTED;
  }
  if (num_seqs == 0 || max_kv_len == 0) {
    nothing = true;
    return PGA_OK;
  }
  if (use_scratch && pga::verify_scratch(&workspace) != hipSuccess) return PGA_ERR_LAUNCH;
  a = pga::VerifyArgs{};
  a.q = static_cast<const uint16_t*>(q);
  a.q_ds = q_descale;
  a.hq = num_q_heads;
  a.r = r;
  a.num_seqs = num_seqs;
  a.cu_q = cu_seqlens_q;
  a.lens_k = seq_lens_k;
  a.kv = make_kv(kv);
  a.c2_base = softmax_scale * 1.4426950408889634f;
  a.max_q_len = max_q_len;
  a.max_kv_len = max_kv_len;
  a.seg_tiles = p.seg_tiles;
  a.rows_cap = p.rows_cap;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.ws_o = workspace;
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws_o_bytes);
  a.ws_plan = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + ws_o_bytes + ws_lse_bytes);
  a.static_tiles = plan_free_tiles;
  return PGA_OK;
}

#define PGA_VERIFY_ARGS                                                                                       \
  q, q_dtype, q_descale, num_q_heads, num_seqs, cu_seqlens_q, seq_lens_k, max_q_len, max_kv_len, kv,          \
      softmax_scale, kv_split_tokens, workspace, workspace_bytes, out, lse

int paged_attn_verify_partials(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                               int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                               int32_t max_q_len, int32_t max_kv_len, const pga_paged_kv* kv, float softmax_scale,
                               int32_t kv_split_tokens, void* workspace, size_t workspace_bytes, void* out,
                               float* lse, void* stream) {
  VerifyPlan p;
  pga::VerifyArgs a;
  int num_wg = 0;
  bool nothing;
  if (int e = prepare_verify(PGA_VERIFY_ARGS, p, a, num_wg, nothing)) return e;
  if (nothing) return PGA_OK;
  return launch_status(pga::launch_verify(a, kv->dtype, num_wg, static_cast<hipStream_t>(stream)));
}

int paged_attn_verify_merge(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                            int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                            int32_t max_q_len, int32_t max_kv_len, const pga_paged_kv* kv, float softmax_scale,
                            int32_t kv_split_tokens, void* workspace, size_t workspace_bytes, void* out, float* lse,
                            void* stream) {
  VerifyPlan p;
  pga::VerifyArgs a;
  int num_wg = 0;
  bool nothing;
  if (int e = prepare_verify(PGA_VERIFY_ARGS, p, a, num_wg, nothing)) return e;
  if (nothing) return PGA_OK;
  return launch_status(pga::launch_verify_merge(a, kv->dtype, num_wg, static_cast<hipStream_t>(stream)));
}

int paged_attn_verify(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads, int32_t num_seqs,
                      const int32_t* cu_seqlens_q, const int32_t* seq_lens_k, int32_t max_q_len, int32_t max_kv_len,
                      const pga_paged_kv* kv, float softmax_scale, int32_t kv_split_tokens, void* workspace,
                      size_t workspace_bytes, void* out, float* lse, void* stream) {
  VerifyPlan p;
  pga::VerifyArgs a;
  int num_wg = 0;
  bool nothing;
  if (int e = prepare_verify(PGA_VERIFY_ARGS, p, a, num_wg, nothing)) return e;
  if (nothing) return PGA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int e = launch_status(pga::launch_verify(a, kv->dtype, num_wg, s))) return e;
  if (a.static_tiles == 1) return PGA_OK;  // every unit fits one tile: all written directly
  return launch_status(pga::launch_verify_merge(a, kv->dtype, num_wg, s));
}

int paged_attn_verify_noalloc(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                              int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                              int32_t max_q_len, int32_t max_kv_len, const pga_paged_kv* kv, float softmax_scale,
                              int32_t kv_split_tokens, void* out, float* lse, void* stream) {
  VerifyPlan p;
  pga::VerifyArgs a;
  int num_wg = 0;
  bool nothing;
  if (int e = prepare_verify(q, q_dtype, q_descale, num_q_heads, num_seqs, cu_seqlens_q, seq_lens_k, max_q_len,
                             max_kv_len, kv, softmax_scale, kv_split_tokens, nullptr, 0, out, lse, p, a, num_wg,
                             nothing, /*use_scratch=*/true))
    return e;
  if (nothing) return PGA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int e = launch_status(pga::launch_verify(a, kv->dtype, num_wg, s))) return e;
  if (a.static_tiles == 1) return PGA_OK;  // every unit fits one tile: all written directly
  return launch_status(pga::launch_verify_merge(a, kv->dtype, num_wg, s));
}

int paged_attn_verify_gather_sum(int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                 int32_t max_q_len, int32_t max_kv_len, const pga_paged_kv* kv,
                                 int32_t kv_split_tokens, uint32_t* out, void* stream) {
  if (!cu_seqlens_q || !seq_lens_k || !out || !kv) return PGA_ERR_NULL;
  if (num_seqs < 0 || max_kv_len < 0 || max_q_len < 1 || max_q_len > 4) return PGA_ERR_SHAPE;
  if (int e = check_kv(kv, kv->num_kv_heads > 0 ? kv->num_kv_heads : 1,
                       cdiv(max_kv_len, kv->page_size > 0 ? kv->page_size : 1)))
    return e;
  if (kv_split_tokens < 0 || kv_split_tokens % kTileKeys != 0) return PGA_ERR_SHAPE;
  if (!aligned(out, 4)) return PGA_ERR_UNSUPPORTED;
  // The work split does not depend on the query heads: plan as for one per kv head.
  VerifyPlan p;
  if (int e = plan_verify(kv->num_kv_heads, kv->num_kv_heads, num_seqs, max_q_len, max_kv_len, kv_split_tokens, p))
    return e;
  if (num_seqs == 0) return PGA_OK;
  int num_wg = 0;
  pga::VerifyArgs a{};
  a.static_tiles = verify_grid(num_seqs, kv, max_kv_len, p, num_wg);
  a.hq = kv->num_kv_heads;
  a.r = 1;
  a.num_seqs = num_seqs;
  a.cu_q = cu_seqlens_q;
  a.lens_k = seq_lens_k;
  a.kv = make_kv(kv);
  a.max_q_len = max_q_len;
  a.max_kv_len = max_kv_len;
  a.seg_tiles = p.seg_tiles;
  a.rows_cap = p.rows_cap;
  a.sum_out = out;
  return launch_status(pga::launch_verify_gather(a, kv->dtype, num_wg, static_cast<hipStream_t>(stream)));
}

int paged_attn_prefill_prefix(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                              int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t max_seqlen_q, int32_t max_seqlen_k, const pga_paged_kv* kv,
                              float softmax_scale, void* out, float* lse, void* stream) {
  if (!q || !cu_seqlens_q || !cu_seqlens_k || !out || !kv) return PGA_ERR_NULL;
  if (num_seqs < 0 || num_q_heads <= 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return PGA_ERR_SHAPE;
  if (q_dtype != kBF16 && q_dtype != kFP8) return PGA_ERR_DTYPE;
  if (!std::isfinite(softmax_scale)) return PGA_ERR_SHAPE;
  if (int e = check_kv(kv, num_q_heads, cdiv(max_seqlen_k, kv->page_size > 0 ? kv->page_size : 1))) return e;
  if (q_dtype == kFP8 && kv->dtype != kFP8) return PGA_ERR_DTYPE;
  const int32_t r = num_q_heads / kv->num_kv_heads;
  if (r > kMaxRowsPerGroup) return PGA_ERR_UNSUPPORTED;
  if (num_seqs > kMaxGridYZ) return PGA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(out, 8) || (lse && !aligned(lse, 4))) return PGA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_seqlen_q == 0) return PGA_OK;

  const int32_t tile_tokens = pga::prefill_tile_tokens(q_dtype, kv->dtype, r);
  const int64_t q_tiles = cdiv(max_seqlen_q, tile_tokens);
  if (q_tiles > INT32_MAX) return PGA_ERR_UNSUPPORTED;
  pga::PrefillArgs a{};
  a.q = q;
  a.q_ds = q_descale;
  a.hq = num_q_heads;
  a.r = r;
  a.num_seqs = num_seqs;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.kv = make_kv(kv);
  a.c2_base = softmax_scale * 1.4426950408889634f;
  a.max_q_len = max_seqlen_q;
  a.max_kv_len = max_seqlen_k;
  a.tile_tokens = tile_tokens;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  return launch_status(pga::launch_prefill(a, q_dtype, kv->dtype, static_cast<int>(q_tiles),
                                           static_cast<hipStream_t>(stream)));
}

int sparse_paged_attn(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                      int32_t num_q_tokens, int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                      const int32_t* indices, int64_t index_stride, int32_t num_selected, const pga_paged_kv* kv,
                      float softmax_scale, void* workspace, size_t workspace_bytes, void* out, float* lse,
                      void* stream) {
  if (!q || !cu_seqlens_q || !seq_lens_k || !out || !kv) return PGA_ERR_NULL;
  if (num_selected > 0 && !indices) return PGA_ERR_NULL;
  if (num_seqs < 0 || num_q_heads <= 0 || num_q_tokens < 0 || num_selected < 0 || index_stride < num_selected)
    return PGA_ERR_SHAPE;
  if (num_q_tokens > 0 && num_seqs == 0) return PGA_ERR_SHAPE;
  if (q_dtype != kBF16) return PGA_ERR_DTYPE;
  if (!std::isfinite(softmax_scale)) return PGA_ERR_SHAPE;
  if (int e = check_kv(kv, num_q_heads, -1)) return e;
  if (int64_t(kv->num_pages) * kv->page_size > INT32_MAX) return PGA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(out, 8) || (lse && !aligned(lse, 4))) return PGA_ERR_UNSUPPORTED;
  if (num_selected > 0 && !aligned(indices, 4)) return PGA_ERR_UNSUPPORTED;
  SparsePlan plan;
  if (!plan_sparse(num_q_heads, kv->num_kv_heads, num_q_tokens, num_selected, plan)) return PGA_ERR_SHAPE;
  if (plan.splits > 1) {
    if (!workspace && workspace_bytes == 0) {
      plan.splits = 1;  // the caller asked for the unsplit launch
      plan.split_len = std::max(num_selected, 1);
    } else if (!workspace || workspace_bytes < plan.ws_bytes) {
      return PGA_ERR_WORKSPACE;
    } else if (!aligned(workspace, 256)) {
      return PGA_ERR_UNSUPPORTED;
    }
  }
  if (num_q_tokens == 0) return PGA_OK;

  pga::SparseArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.q_ds = q_descale;
  a.hq = num_q_heads;
  a.r = num_q_heads / kv->num_kv_heads;
  a.num_seqs = num_seqs;
  a.num_tokens = num_q_tokens;
  a.cu_q = cu_seqlens_q;
  a.lens_k = seq_lens_k;
  a.idx = indices;
  a.idx_stride = index_stride;
  a.num_selected = num_selected;
  a.kv = make_kv(kv);
  a.c2_base = softmax_scale * 1.4426950408889634f;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.splits = plan.splits;
  a.split_len = plan.split_len;
  if (plan.splits > 1) {
    a.ws_o = workspace;
    a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ws_o_bytes);
  }
  return launch_status(pga::launch_sparse(a, kv->dtype, static_cast<hipStream_t>(stream)));
}

int sparse_gather_sum(int32_t num_q_tokens, int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                      const int32_t* indices, int64_t index_stride, int32_t num_selected, const pga_paged_kv* kv,
                      uint32_t* out, void* stream) {
  if (!cu_seqlens_q || !seq_lens_k || !out || !kv) return PGA_ERR_NULL;
  if (num_selected > 0 && !indices) return PGA_ERR_NULL;
  if (num_seqs < 0 || num_q_tokens < 0 || num_selected < 0 || index_stride < num_selected) return PGA_ERR_SHAPE;
  if (num_q_tokens > 0 && num_seqs == 0) return PGA_ERR_SHAPE;
  if (int e = check_kv(kv, kv->num_kv_heads > 0 ? kv->num_kv_heads : 1, -1)) return e;
  // Evenly spaced token rows, addressed by 32-bit byte offsets from each
  // head's base formed by 24-bit multiplies: at most 2^24 rows, token strides
  // below 2^24 bytes, every row within 4 GiB of its head's base.
  if (kv->k_stride_page != int64_t(kv->page_size) * kv->k_stride_token ||
      kv->v_stride_page != int64_t(kv->page_size) * kv->v_stride_token)
    return PGA_ERR_UNSUPPORTED;
  const int64_t rows = int64_t(kv->num_pages) * kv->page_size;
  const int64_t st = std::max(kv->k_stride_token, kv->v_stride_token) * elt_bytes(kv->dtype);
  if (std::min(kv->k_stride_token, kv->v_stride_token) <= 0 || st >= (int64_t(1) << 24) ||
      rows > (int64_t(1) << 24) || (rows - 1) * st + kHeadDim * elt_bytes(kv->dtype) > (int64_t(1) << 32))
    return PGA_ERR_UNSUPPORTED;
  if (!aligned(out, 16) || (num_selected > 0 && !aligned(indices, 4))) return PGA_ERR_UNSUPPORTED;
  if (num_q_tokens == 0) return PGA_OK;
  pga::GatherArgs a{};
  a.num_tokens = num_q_tokens;
  a.num_seqs = num_seqs;
  a.cu_q = cu_seqlens_q;
  a.lens_k = seq_lens_k;
  a.idx = indices;
  a.idx_stride = index_stride;
  a.num_selected = num_selected;
  a.kv = make_kv(kv);
  a.out = out;
  // The list pieces sparse_paged_attn takes for this many rows (up to 16 query
  // heads per kv head: one row block per kv head, as the workloads have).
  SparsePlan plan;
  if (!plan_sparse(16 * a.kv.num_kv_heads, a.kv.num_kv_heads, num_q_tokens, num_selected, plan)) return PGA_ERR_SHAPE;
  a.splits = plan.splits;
  a.split_len = plan.split_len;
  return launch_status(pga::launch_gather_sum(a, kv->dtype, static_cast<hipStream_t>(stream)));
}

size_t sparse_paged_attn_workspace_bytes(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_q_tokens,
                                         int32_t num_selected) {
  SparsePlan p;
  return plan_sparse(num_q_heads, num_kv_heads, num_q_tokens, num_selected, p) ? p.ws_bytes : 0;
}

int32_t sparse_paged_attn_splits(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_q_tokens,
                                 int32_t num_selected) {
  SparsePlan p;
  return plan_sparse(num_q_heads, num_kv_heads, num_q_tokens, num_selected, p) ? p.splits : 0;
}

size_t prefill_quantize_fp8_workspace_bytes(void) { return pga::kQuantWorkspaceBytes; }

int prefill_quantize_fp8(const void* q, int32_t num_q_heads, int32_t num_q_tokens, const float* q_descale_in,
                         void* q_fp8, float* q_descale_out, const void* k_new, const void* v_new, int32_t num_seqs,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const pga_paged_kv* kv,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if ((!q || !q_fp8) && num_q_tokens > 0) return PGA_ERR_NULL;
  if (!q_descale_in && !q_descale_out) return PGA_ERR_NULL;
  if (!k_new != !v_new) return PGA_ERR_NULL;
  if (num_q_heads <= 0 || num_q_tokens < 0 || num_seqs < 0) return PGA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(q_fp8, 8) || (q_descale_out && !aligned(q_descale_out, 4)))
    return PGA_ERR_UNSUPPORTED;
  const bool with_kv = k_new != nullptr;
  if (with_kv) {
    if (!cu_seqlens_q || !cu_seqlens_k || !kv) return PGA_ERR_NULL;
    if (int e = check_kv(kv, num_q_heads, -1)) return e;
    if (kv->dtype != kFP8) return PGA_ERR_DTYPE;
    if (num_q_tokens > 0 && num_seqs == 0) return PGA_ERR_SHAPE;
    if (!aligned(k_new, 16) || !aligned(v_new, 16)) return PGA_ERR_UNSUPPORTED;
    if (int64_t(num_q_tokens) * kv->num_kv_heads * (kHeadDim / 8) > INT32_MAX) return PGA_ERR_UNSUPPORTED;
  }
  const bool dynamic = q_descale_in == nullptr;
  if (dynamic) {
    if (!workspace || workspace_bytes < prefill_quantize_fp8_workspace_bytes()) return PGA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return PGA_ERR_UNSUPPORTED;
  }

  pga::QuantArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.q_chunks = int64_t(num_q_tokens) * num_q_heads * (kHeadDim / 8);
  a.q_ds_in = q_descale_in;
  a.q_ds_out = q_descale_out;
  a.q_out = static_cast<uint8_t*>(q_fp8);
  a.partial = static_cast<uint32_t*>(workspace);
  a.num_partial = dynamic ? pga::quant_amax_blocks(a.q_chunks) : 0;
  if (with_kv) {
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.kv_rows = int64_t(num_q_tokens) * kv->num_kv_heads;
    a.num_seqs = num_seqs;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.kv = make_kv(kv);
  }
  a.max_blocks = int64_t(device_cus()) * 8;
  a.num_cus = device_cus();
  a.tag = next_quant_tag();
  return launch_status(pga::launch_quantize(a, static_cast<hipStream_t>(stream)));
}

int pga_validate_inputs(int32_t num_seqs, int32_t num_q_tokens, const int32_t* cu_seqlens_q,
                        const int32_t* seq_lens_k, const int32_t* cu_seqlens_k, int32_t max_q_len,
                        int32_t max_kv_len, const pga_paged_kv* kv, const int32_t* indices, int64_t index_stride,
                        int32_t num_selected, int32_t* counts_device, int32_t* counts_host, void* stream) {
  if (!cu_seqlens_q || !kv || !kv->block_table || !counts_device) return PGA_ERR_NULL;
  if (!seq_lens_k == !cu_seqlens_k) return PGA_ERR_NULL;  // exactly one of them
  if (num_seqs < 0) return PGA_ERR_SHAPE;
  if (!pow2(kv->page_size) || kv->num_pages <= 0 || kv->block_table_stride < 0) return PGA_ERR_SHAPE;
  if (indices && (num_q_tokens < 0 || num_selected < 0 || index_stride < num_selected)) return PGA_ERR_SHAPE;
  if (!aligned(counts_device, 4)) return PGA_ERR_UNSUPPORTED;
  pga::ValidateArgs a{};
  a.num_seqs = num_seqs;
  a.num_q_tokens = num_q_tokens;
  a.cu_q = cu_seqlens_q;
  a.lens_k = seq_lens_k;
  a.cu_k = cu_seqlens_k;
  a.max_q_len = max_q_len;
  a.max_kv_len = max_kv_len;
  a.bt = kv->block_table;
  a.bt_stride = kv->block_table_stride;
  a.page_size = kv->page_size;
  a.num_pages = kv->num_pages;
  a.idx = indices;
  a.idx_stride = index_stride;
  a.num_selected = num_selected;
  a.counts = counts_device;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (int e = launch_status(pga::launch_validate(a, s))) return e;
  int32_t c[pga::kValidateCounts] = {0, 0, 0, 0};
  if (hipMemcpyAsync(c, counts_device, sizeof c, hipMemcpyDeviceToHost, s) != hipSuccess) return PGA_ERR_LAUNCH;
  if (hipStreamSynchronize(s) != hipSuccess) return PGA_ERR_LAUNCH;
  if (counts_host)
    for (int i = 0; i < pga::kValidateCounts; ++i) counts_host[i] = c[i];
  return (c[0] | c[1] | c[2]) ? PGA_ERR_INVALID_DATA : PGA_OK;
}

}  // extern "C"
