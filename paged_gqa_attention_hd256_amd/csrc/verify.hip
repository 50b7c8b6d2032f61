// Bottom-right causal attention over the paged cache (speculative verify and
// prefix prefill) and the split-KV log-sum-exp merge.
//
// Verify: one workgroup per (key segment, kv head, sequence).  All r * Lq_b
// query rows of the kv group (token-major: row = t * r + h) are packed into
// the workgroup, 16 rows per wave, so every KV page of the segment is fetched
// from HBM once for all speculative tokens -- the reuse SGLang PR #36330 adds
// (Motivation; Modifications: BLOCK_M = 16 x BLOCK_Q).  A sequence whose keys
// fit one segment writes bf16 output directly; longer ones write fp32 partial
// outputs (already divided by their row sums) and natural-log lse values that
// lse_merge_kernel combines (Modifications: segments chosen from CU
// parallelism and per-segment KV work).
//
// Prefill: one workgroup per (tile of query tokens, kv head, sequence), all
// keys from 0 to the tile's last diagonal position, with the bottom-right rule
// of ROCm/ATOM PR #2534 (FMHA commit message: keys longer than queries).
// Pages are read in the kernel, no gather first (ROCm/ATOM PR #2830, recipe
// commit).
//
// Keys stream through LDS in 64-key tiles by 16-byte global->LDS DMA,
// double-buffered; block-table entries are read with scalar loads, so the only
// vector-memory traffic in the loop is the DMA and its counter can be waited
// on exactly.
#include "attn_core.h"
#include "pga_args.h"

namespace pga {

template <bool PREFILL, int QDT, int KV>
__global__ __launch_bounds__(256, (KV == kFP8) ? 2 : 1) void causal_kernel(CausalArgs a) {
  using G = TileGeom<KV>;
  constexpr int kRowsPerDma = 1024 / G::kRowBytes;  // rows one 1 KB DMA instruction fills
  constexpr int kDmaPerWave = 16 / kRowsPerDma;     // instructions per wave for its 16 rows of K (or V)
  __shared__ __attribute__((aligned(16))) char smem[2][2][G::template tile_bytes<64>()];  // [buffer][K, V]

  const int g = blockIdx.y, b = blockIdx.z;
  const int tok0 = a.cu_q[b];
  const int lq = min(a.cu_q[b + 1] - tok0, a.max_q_len);
  const int lk = min(PREFILL ? a.cu_k[b + 1] - a.cu_k[b] : a.lens_k[b], a.max_kv_len);
  // Query tokens [t_lo, t_hi) of the sequence and keys [k_lo, k_hi) this workgroup covers.
  int t_lo, t_hi, k_lo, k_hi, seg = 0, nseg_b = 1;
  if constexpr (PREFILL) {
    // Longest-first: block 0 takes the last query tile, which sees the most keys.
    t_lo = (gridDim.x - 1 - blockIdx.x) * a.tile_tokens;
    t_hi = min(t_lo + a.tile_tokens, lq);
    if (t_lo >= lq) return;
    k_lo = 0;
    k_hi = lk - lq + t_hi;  // one past the last token's last visible key
  } else {
    seg = blockIdx.x;
    t_lo = 0;
    t_hi = lq;
    k_lo = seg * a.seg_len;
    if (lq <= 0 || k_lo >= lk) return;
    k_hi = min(k_lo + a.seg_len, lk);
    nseg_b = (lk + a.seg_len - 1) / a.seg_len;
  }
  const int rows = a.r * (t_hi - t_lo);

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int n = lane & 15, gq = lane >> 4;
  const int rho = 16 * w + n;
  const bool row_ok = rho < rows;
  const int tq = row_ok ? rho / a.r : 0;
  const int hh = row_ok ? rho - tq * a.r : 0;
  const int t = t_lo + tq;
  const int64_t tok = tok0 + t;
  const int head = g * a.r + hh;
  const bool wave_active = 16 * w < rows;

  QFrag qf;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf.q[ks] = bf16x8{};
  if (row_ok) {
    if constexpr (QDT == kFP8) {
      const i32x2* qp = reinterpret_cast<const i32x2*>(static_cast<const uint8_t*>(a.q) + (tok * a.hq + head) * kHeadDim);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf.q[ks] = fp8x8_to_bf16(qp[4 * ks + gq]);
    } else {
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(a.q) + (tok * a.hq + head) * kHeadDim);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf.q[ks] = qp[4 * ks + gq];
    }
  }
  const float c2 = a.c2_base * load_scale(a.q_ds) * load_scale(a.kv.k_ds);
  // Largest visible key of this lane's row, and the smallest such limit over
  // the workgroup's rows (bottom-right causal, clipped to the key range).
  const int klim = row_ok ? min(lk - lq + t, k_hi - 1) : -1;
  const int min_lim = min(lk - lq + t_lo, k_hi - 1);

  const int ntiles = (k_hi - k_lo + 63) >> 6;
  const uint8_t* kbase = a.kv.k + g * a.kv.k_sh;
  const uint8_t* vbase = a.kv.v + g * a.kv.v_sh;
  const int32_t* bt_row = a.kv.bt + (int64_t)b * a.kv.bt_stride;

  // Issue the DMA of tile `it` into buffer `buf`: this wave fetches tile rows
  // 16w .. 16w + 15, which lie in one page (pages hold >= 16 tokens and tiles
  // start at multiples of 64).
  auto issue = [&](int it, int buf) {
    const int tb = k_lo + it * 64;
    const int key0 = tb + 16 * w;
    int page = -1;
    if (key0 < k_hi) page = bt_row[key0 >> a.kv.page_shift];
    page = __builtin_amdgcn_readfirstlane(page);
    const bool page_ok = page >= 0 && page < a.kv.num_pages;
    const int64_t kpage = (int64_t)page * a.kv.k_sp;
    const int64_t vpage = (int64_t)page * a.kv.v_sp;
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
      const int row0 = 16 * w + u * kRowsPerDma;
      const int row = row0 + lane / G::kChunks;
      const int chunk = (lane % G::kChunks) ^ (row & (G::kChunks - 1));
      const int key = tb + row;
      const bool ok = page_ok && key < k_hi;
      const int slot = key & (a.kv.page_size - 1);
      const uint8_t* ks = ok ? kbase + kpage + slot * a.kv.k_st + chunk * 16 : reinterpret_cast<const uint8_t*>(g_zero16);
      const uint8_t* vs = ok ? vbase + vpage + slot * a.kv.v_st + chunk * 16 : reinterpret_cast<const uint8_t*>(g_zero16);
      dma16(ks, (lds_t*)&smem[buf][0][row0 * G::kRowBytes]);
      dma16(vs, (lds_t*)&smem[buf][1][row0 * G::kRowBytes]);
    }
  };

  WaveState st;
  st.init();
  issue(0, 0);
  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) {
      issue(it + 1, (it + 1) & 1);
      wait_vmcnt<2 * kDmaPerWave>();
    } else {
      wait_vmcnt<0>();
    }
    barrier();
    if (wave_active) {
      const lds_t* kt = (const lds_t*)&smem[it & 1][0][0];
      const lds_t* vt = (const lds_t*)&smem[it & 1][1][0];
      const int tb = k_lo + it * 64;
      f32x4 sc[4];
      tile_scores<KV, 4>(kt, qf, sc);
      const int lim = klim - tb;
      tile_softmax<4>(st, sc, c2, tb + 63 > min_lim, [lim](int key) { return key <= lim; });
      tile_pv<KV, 4>(st, vt, sc);
    }
    barrier();
  }

  if (!wave_active) return;
  const float lrow = group4_sum(st.l);
  if (!row_ok) return;
  const float vds = load_scale(a.kv.v_ds);
  const float inv = lrow > 0.f ? vds / lrow : 0.f;
  const float lse = lrow > 0.f ? (st.m + log2f(lrow)) * kLn2 : kNegInf;
  if (nseg_b == 1) {
    uint16_t* op = a.out + (tok * a.hq + head) * kHeadDim + 4 * gq;
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) {
      const uint32_t lo = pack_bf16x2(st.o[mb][0] * inv, st.o[mb][1] * inv);
      const uint32_t hi = pack_bf16x2(st.o[mb][2] * inv, st.o[mb][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * mb) = make_uint2(lo, hi);
    }
    if (gq == 0 && a.lse) a.lse[tok * a.hq + head] = lse;
  } else {
    const int64_t unit = ((int64_t)b * a.kv.num_kv_heads + g) * a.max_segs + seg;
    float* wp = a.ws_o + (unit * a.rows_cap + rho) * kHeadDim + 4 * gq;
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) *reinterpret_cast<f32x4*>(wp + 16 * mb) = st.o[mb] * inv;
    if (gq == 0) a.ws_lse[unit * a.rows_cap + rho] = lse;
  }
}

// Combine the segments of one (token, head): weights exp(lse_s - max lse),
// segments with lse = -inf (no visible key) contribute nothing.  One wave per
// (token, head); each lane owns four consecutive output elements.
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
  const int b = blockIdx.y;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  const int t = pair / a.hq, h = pair - (pair / a.hq) * a.hq;
  const int tok0 = a.cu_q[b];
  const int lq = a.cu_q[b + 1] - tok0;
  if (t >= lq) return;
  const int lk = min(a.lens_k[b], a.max_kv_len);
  const int nseg = min((lk + a.seg_len - 1) / a.seg_len, a.max_segs);
  if (nseg <= 1) return;
  const int g = h / a.r;
  const int rho = t * a.r + (h - g * a.r);
  if (rho >= a.rows_cap) return;
  const int64_t unit0 = ((int64_t)b * a.hkv + g) * a.max_segs;
  float mx = kNegInf;
  for (int s = 0; s < nseg; ++s) mx = fmaxf(mx, a.ws_lse[(unit0 + s) * a.rows_cap + rho]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != kNegInf) {
    for (int s = 0; s < nseg; ++s) {
      const float ls = a.ws_lse[(unit0 + s) * a.rows_cap + rho];
      if (ls == kNegInf) continue;
      const float wgt = __expf(ls - mx);
      wsum += wgt;
      const f32x4 o = *reinterpret_cast<const f32x4*>(a.ws_o + ((unit0 + s) * a.rows_cap + rho) * kHeadDim + 4 * lane);
      acc += wgt * o;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t tok = tok0 + t;
  uint16_t* op = a.out + (tok * a.hq + h) * kHeadDim + 4 * lane;
  *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
  if (lane == 0 && a.lse) a.lse[tok * a.hq + h] = wsum > 0.f ? mx + logf(wsum) : kNegInf;
}

hipError_t launch_causal(const CausalArgs& a, bool prefill, int q_dtype, int kv_dtype, int gx, int gy, int gz,
                         hipStream_t s) {
  dim3 grid(gx, gy, gz), block(256);
  if (prefill) {
    if (q_dtype == kFP8 && kv_dtype == kFP8)
      hipLaunchKernelGGL((causal_kernel<true, kFP8, kFP8>), grid, block, 0, s, a);
    else if (q_dtype == kBF16 && kv_dtype == kFP8)
      hipLaunchKernelGGL((causal_kernel<true, kBF16, kFP8>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((causal_kernel<true, kBF16, kBF16>), grid, block, 0, s, a);
  } else {
    if (kv_dtype == kFP8)
      hipLaunchKernelGGL((causal_kernel<false, kBF16, kFP8>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((causal_kernel<false, kBF16, kBF16>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, int max_q_len, hipStream_t s) {
  dim3 grid((max_q_len * a.hq + 3) / 4, a.num_seqs), block(256);
  hipLaunchKernelGGL(lse_merge_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace pga
