// Kernel argument blocks and launch entry points shared by the host API and
// the kernel translation units.  Host-compilable: no device code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Bottom-right causal attention over a paged cache: speculative verify (one
// workgroup per key segment, all query tokens of the sequence) or prefill (one
// workgroup per tile of query tokens, all keys up to the tile's diagonal).
struct CausalArgs {
  const void* q;           // [T, hq, 256] bf16 or FP8 codes
  const float* q_ds;
  int32_t hq, r, num_seqs;
  const int32_t* cu_q;
  const int32_t* lens_k;   // verify: [B] key lengths
  const int32_t* cu_k;     // prefill: [B + 1] key prefix sums
  KvArgs kv;
  float c2_base;           // softmax_scale * log2(e)
  int32_t max_q_len;       // host bounds: per-sequence lengths are clamped to them, so a
  int32_t max_kv_len;      //   caller that exceeds them cannot push an access out of bounds
  int32_t tile_tokens;     // prefill: query tokens per workgroup
  int32_t seg_len;         // verify: keys per segment (multiple of 64)
  int32_t max_segs;        // verify: segment slots per (sequence, kv head) in the workspace
  int32_t rows_cap;        // verify: r * max_q_len row slots per unit in the workspace
  uint16_t* out;           // [T, hq, 256] bf16
  float* lse;              // [T, hq] or null
  float* ws_o;             // [B, hkv, max_segs, rows_cap, 256] fp32, normalised and v-descaled
  float* ws_lse;           // [B, hkv, max_segs, rows_cap] fp32 natural-log lse
};

struct MergeArgs {
  int32_t hq, r, hkv, num_seqs, max_kv_len;
  const int32_t* cu_q;
  const int32_t* lens_k;
  int32_t seg_len, max_segs, rows_cap;
  const float* ws_o;
  const float* ws_lse;
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
};

// Launchers (defined next to their kernels).  They return the launch status.
hipError_t launch_causal(const CausalArgs& a, bool prefill, int q_dtype, int kv_dtype, int grid_x, int grid_y,
                         int grid_z, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, int max_q_len, hipStream_t s);
hipError_t launch_sparse(const SparseArgs& a, int kv_dtype, hipStream_t s);

}  // namespace pga
