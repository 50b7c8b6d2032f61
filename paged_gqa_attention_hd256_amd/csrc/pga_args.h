// Kernel argument blocks and launch entry points shared by the host API and
// the kernel translation units.  Host-compilable: no device code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "paged_gqa.h"

namespace pga {

// Paged KV description with byte strides, as the kernels consume it.
struct KvArgs {
  const uint8_t* k;
  const uint8_t* v;
  int64_t k_sp, k_st, k_sh;
  int64_t v_sp, v_st, v_sh;
  const int32_t* bt;
  int64_t bt_stride;
  int32_t page_size;
  int32_t page_shift;
  int32_t num_pages;
  int32_t num_kv_heads;
  const float* k_ds;
  const float* v_ds;
};

// Speculative verify plan constants, shared by the host plan and the kernels.
// The work list is every unit's 64-key tiles, each segment preceded by
// kVerifySegStartCost empty positions (the cost of starting a piece: query
// reload, pipeline refill, partial write); a workgroup takes a run of at
// least kVerifyMinTilesPerWg positions.  Positions and slot indices are int32.
// Both values are measured: a start costs about five tiles' time on this part,
// and with runs of one position the grid reaches 1,024 workgroups also on
// small batches, where longer minimum runs left most of the chip idle.
constexpr int kVerifySegStartCost = 5;
constexpr int kVerifyMinTilesPerWg = 1;
constexpr int kVerifyMaxWgs = 1024;  // cap of the persistent grid
// Calls whose host bounds give at most this many tiles over all units (and
// at most 64 per unit) run one workgroup per tile without the plan.
constexpr int kVerifyStaticMaxTiles = 256;

// Speculative verify: persistent stream-K grid over the key tiles of every
// (sequence, kv head) unit; see verify.hip.
struct VerifyArgs {
  const uint16_t* q;       // [T, hq, 256] bf16
  const float* q_ds;
  int32_t hq, r, num_seqs;
  const int32_t* cu_q;
  const int32_t* lens_k;
  KvArgs kv;
  float c2_base;           // softmax_scale * log2(e)
  int32_t max_q_len;       // host bounds: per-sequence lengths are clamped to them, so a
  int32_t max_kv_len;      //   caller that exceeds them cannot push an access out of bounds
  int32_t seg_tiles;       // 64-key tiles per segment (a partial never spans two segments)
  int32_t rows_cap;        // r * max_q_len: row slots per workspace slot
  uint16_t* out;           // [T, hq, 256] bf16
  float* lse;              // [T, hq] or null
  void* ws_o;              // [slots, rows_cap, 256] partial outputs divided by their row sums, in V code
                           // units (v_descale not applied): fp16 for FP8 V (|x| <= 448), fp32 for BF16 V
  float* ws_lse;           // [slots, rows_cap] fp32 natural-log lse of the partials
  int32_t* ws_plan;        // [units][2]: first tile, first segment of each unit; then tiles per workgroup
  int32_t static_tiles;    // > 0: plan-free mode, workgroup w takes tile w % static_tiles of unit
                           //   w / static_tiles and writes slot w (0: the stream-K plan)
  uint32_t* sum_out;       // [units] checksums the page-gather roof adds into (verify_gather_kernel only)
};

// Prefill against a cached prefix: one workgroup per (tile of query tokens,
// kv head, sequence), all keys up to the tile's last diagonal position.
struct PrefillArgs {
  const void* q;           // [T, hq, 256] bf16 or FP8 codes
  const float* q_ds;
  int32_t hq, r, num_seqs;
  const int32_t* cu_q;
  const int32_t* cu_k;     // [B + 1] key prefix sums
  KvArgs kv;
  float c2_base;
  int32_t max_q_len, max_kv_len;
  int32_t tile_tokens;     // query tokens per workgroup
  uint16_t* out;
  float* lse;
};

struct SparseArgs {
  const uint16_t* q;       // [T, hq, 256] bf16
  const float* q_ds;
  int32_t hq, r, num_seqs, num_tokens;
  const int32_t* cu_q;
  const int32_t* lens_k;
  const int32_t* idx;      // [T, idx_stride]
  int64_t idx_stride;
  int32_t num_selected;
  KvArgs kv;
  float c2_base;
  uint16_t* out;
  float* lse;
  int32_t splits;          // pieces each row's list is cut into (1: no split, output written directly)
  int32_t split_len;       // list entries per piece (a multiple of 32)
  void* ws_o;              // [T * hq * splits, 256] partial rows over their row sums, V code units:
                           // fp16 for FP8 V, fp32 for BF16 V
  float* ws_lse;           // [T * hq * splits] natural-log lse of the pieces
};

// Same-index gather of a selected-token call's K and V rows (gather.hip).
struct GatherArgs {
  int32_t num_tokens, num_seqs;
  const int32_t* cu_q;
  const int32_t* lens_k;
  const int32_t* idx;      // [T, idx_stride]
  int64_t idx_stride;
  int32_t num_selected;
  KvArgs kv;               // evenly spaced pool; row byte offsets below 2^32
  uint32_t* out;           // [T, hkv, row bytes / 4] word sums
  int32_t splits;          // pieces of each row's list (the sparse call's plan); > 1: added atomically
  int32_t split_len;       // entries per piece
};

// FP8 quantisation of a prefill's inputs (quantize.hip).
constexpr int kQuantMaxPartials = 1024;  // partial maxima of the reduction pass
constexpr int kQuantResidentChunks = 16;  // Q chunks per thread held by the resident path (64 VGPRs)
// Workspace: the two-launch path's partial maxima (4 KB), then the resident
// path's grid barrier: one 128-byte line per workgroup for its tagged
// partial, then the expired-wait flag word.
constexpr size_t kQuantWorkspaceBytes = kQuantMaxPartials * sizeof(uint32_t) + 128 * kQuantMaxPartials + 256;
struct QuantArgs {
  const uint16_t* q;       // [T, hq, 256] bf16
  int64_t q_chunks;        // 16-byte chunks of q: T * hq * 32
  const float* q_ds_in;    // given descale, or null for the dynamic one (amax / 448)
  float* q_ds_out;         // the descale used, or null
  uint8_t* q_out;          // [T, hq, 256] E4M3FN codes
  uint32_t* partial;       // [num_partial] per-workgroup max |q| as bf16 magnitude patterns
  int32_t num_partial;
  const uint16_t* k_new;   // [T, hkv, 256] bf16, or null (then kv_rows is 0)
  const uint16_t* v_new;
  int64_t kv_rows;         // T * hkv
  int32_t num_seqs;
  const int32_t* cu_q;
  const int32_t* cu_k;
  KvArgs kv;               // the FP8 pool the new keys and values are written into
  int64_t max_blocks;      // grid cap of the coding pass
  int32_t num_cus;         // CUs of the device (the resident path's grid follows from it), 0 = that path off
  uint64_t tag;            // the resident path's barrier tag, unique to the call (48 bits, odd)
};

// Device check of the data-dependent preconditions (validate.hip).
constexpr int kValidateCounts = 4;
struct ValidateArgs {
  int32_t num_seqs;
  int64_t num_q_tokens;    // host copy of cu_q[num_seqs], or -1 when unknown
  const int32_t* cu_q;
  const int32_t* lens_k;   // exactly one of lens_k / cu_k is set
  const int32_t* cu_k;
  int32_t max_q_len, max_kv_len;  // host bounds to check against (<= 0: not checked)
  const int32_t* bt;
  int64_t bt_stride;
  int32_t page_size, num_pages;
  const int32_t* idx;      // [num_q_tokens, idx_stride] or null
  int64_t idx_stride;
  int32_t num_selected;
  int32_t* counts;         // [kValidateCounts] device counters
};

// Allocation-free verify (noalloc.hip): bytes of the fixed per-device scratch,
// and its device address on the current device (looked up once per device).
constexpr size_t kVerifyScratchBytes = PGA_VERIFY_NOALLOC_SCRATCH_BYTES;
hipError_t verify_scratch(void** ptr);

// Launchers (defined next to their kernels).  They return the launch status.
hipError_t launch_verify(const VerifyArgs& a, int kv_dtype, int num_wg, hipStream_t s);
hipError_t launch_verify_merge(const VerifyArgs& a, int kv_dtype, int num_wg, hipStream_t s);
hipError_t launch_verify_gather(const VerifyArgs& a, int kv_dtype, int num_wg, hipStream_t s);
// Query tokens per prefill workgroup for this dtype pair and group size r.
int prefill_tile_tokens(int q_dtype, int kv_dtype, int r);
hipError_t launch_prefill(const PrefillArgs& a, int q_dtype, int kv_dtype, int q_tiles, hipStream_t s);
hipError_t launch_sparse(const SparseArgs& a, int kv_dtype, hipStream_t s);
hipError_t launch_gather_sum(const GatherArgs& a, int kv_dtype, hipStream_t s);
// Workgroups of the reduction pass for q_chunks 16-byte chunks (1 .. kQuantMaxPartials).
int quant_amax_blocks(int64_t q_chunks);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
hipError_t launch_validate(const ValidateArgs& a, hipStream_t s);

}  // namespace pga
