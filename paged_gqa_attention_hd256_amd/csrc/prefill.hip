// Prefill of new tokens against a cached prefix, bottom-right causal.
//
// One workgroup per (tile of query tokens, kv head, sequence): the tile packs
// 64 / r tokens x r heads of one kv group (token-major rows), and streams all
// keys from 0 to the tile's last diagonal position, with the mask of ROCm/ATOM
// PR #2534 (FMHA commit message: the cached + new keys are longer than the
// queries and the causal mask is bottom-right aligned).  Pages are read in the
// kernel, with no gather to contiguous memory first (ROCm/ATOM PR #2830, recipe
// commit).  Workgroups are ordered longest first.
#include "causal_stream.h"



namespace pga {

// NW waves per workgroup (16 NW rows).  Four waves for every dtype pair: eight
// (128 rows, one ~81 KB workgroup per CU) halve the K/V bytes streamed from L2
// per row but measured slower, the barriers of a tile then waiting on eight
// waves.
template <int QDT, int KV, int NW>
__global__ __launch_bounds__(64 * NW, (KV == kFP8 && NW == 4) ? 2 : 1) void prefill_kernel(PrefillArgs a) {
  __shared__ CausalSmem<KV, NW> sm;
  const int g = blockIdx.y, b = blockIdx.z;
  const int tok0 = a.cu_q[b];
  const int lq = min(a.cu_q[b + 1] - tok0, a.max_q_len);
  const int lk = min(a.cu_k[b + 1] - a.cu_k[b], a.max_kv_len);
  // Longest first: block 0 takes the last query tile, which sees the most keys.
  const int t_lo = (gridDim.x - 1 - blockIdx.x) * a.tile_tokens;
  if (t_lo >= lq) return;
  const int t_hi = min(t_lo + a.tile_tokens, lq);
  const int k_hi = lk - lq + t_hi;  // one past the last visible key of the tile
  const int rows = a.r * (t_hi - t_lo);

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int n = lane & 15;
  const int rho = 16 * w + n;  // this lane's softmax row
  const bool row_ok = rho < rows;
  const int tq = row_ok ? rho / a.r : 0;
  const int head = g * a.r + (row_ok ? rho - tq * a.r : 0);
  const int64_t tok = tok0 + t_lo + tq;
  const int32_t* bt_row = a.kv.bt + (int64_t)b * a.kv.bt_stride;
  const int2 first = first_pages<NW>(a.kv, bt_row, 0, k_hi);
  QFragT<KV> qf;
  load_q<QDT, KV>(qf, a.q, tok, a.hq, head, row_ok);
  const float c2 = a.c2_base * load_scale(a.q_ds) * load_scale(a.kv.k_ds);
  const int klim = row_ok ? min(lk - lq + t_lo + tq, k_hi - 1) : -1;
  const int min_lim = min(lk - lq + t_lo, k_hi - 1);
  const bool live = 16 * w < rows;
  RowStat rs;
  rs.init();
  f32x4 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
  stream_keys(sm, a.kv, bt_row, g, 0, k_hi, first,
              SplitTile<QDT, KV, NW>{qf, c2 * qf.rscale, klim, min_lim, live, rs, o, lsum, sm.x});
  const float lrow = finish_rows(lsum, live, sm.x);
  if (row_ok && (lane >> 4) == 0 && a.lse)
    a.lse[tok * a.hq + head] = lrow > 0.f ? (rs.m + log2f(lrow)) * kLn2 : kNegInf;
  const float vds = load_scale(a.kv.v_ds);
#pragma unroll
  for (int rb = 0; rb < NW; ++rb) {
    const int rr = 16 * rb + n;
    if (rr < rows) {
      const int t2 = rr / a.r;
      const float l = sm.x.row[rr];
      store_share_bf16<NW>(o, rb, l > 0.f ? vds / l : 0.f,
                           a.out + ((tok0 + t_lo + t2) * (int64_t)a.hq + g * a.r + rr - t2 * a.r) * kHeadDim);
    }
  }
}

constexpr int kFp8PrefillWaves = 4;

int prefill_tile_tokens(int q_dtype, int kv_dtype, int r) {
  if (r <= 0) return 0;
  return (q_dtype == kFP8 && kv_dtype == kFP8) ? 16 * kFp8PrefillWaves / r : 64 / r;
}

hipError_t launch_prefill(const PrefillArgs& a, int q_dtype, int kv_dtype, int q_tiles, hipStream_t s) {
  dim3 grid(q_tiles, a.kv.num_kv_heads, a.num_seqs);
  if (q_dtype == kFP8 && kv_dtype == kFP8)
    hipLaunchKernelGGL((prefill_kernel<kFP8, kFP8, kFp8PrefillWaves>), grid, dim3(64 * kFp8PrefillWaves), 0, s, a);
  else if (q_dtype == kBF16 && kv_dtype == kFP8)
    hipLaunchKernelGGL((prefill_kernel<kBF16, kFP8, 4>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_kernel<kBF16, kBF16, 4>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pga
