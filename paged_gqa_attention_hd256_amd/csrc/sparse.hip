// Selected-token paged attention (vLLM PR #62590, "Tune sparse GQA prefill
// profile on gfx942 and gfx950": Overview; Earlier results: 2,051 selected
// tokens per row at head size 256, BF16 or FP8 K/V).
//
// Work unit: one wave per (query token, kv head, block of 16 query heads of
// that kv group).  The waves of a workgroup are independent -- each owns its
// LDS region and never waits for another -- so the gather of one wave overlaps
// the arithmetic of the others without workgroup barriers.
//
// Per wave, the selected entries are processed in chunks: the wave first
// translates a chunk of the row's index list into physical token rows of the
// pool (index -> block-table page -> page * page_size + slot, or -1 for
// padding) and keeps that table in LDS; then it streams 32-key tiles of K and
// V through a double-buffered LDS region by 16-byte DMA whose per-lane source
// comes from the table, and runs the shared attention core on each tile.
// Because the table is read from LDS, no vector-memory load sits between the
// DMA instructions and their counter can be waited on exactly.
#include "causal_stream.h"

namespace pga {

constexpr int kSparseTableEntries = 1024;  // index-list chunk held in LDS per wave

template <int KV>
struct SparseCfg {
  using G = TileGeom<KV>;
  // Four independent waves per CU: 32-key tiles of FP8 K and V, 16-key tiles
  // of BF16 (two stages of K and V plus the index table fit 4 x 36 KB of LDS).
  static constexpr int kWaves = 4;
  static constexpr int kTileKeys = (KV == kFP8) ? 32 : 16;
  static constexpr int kBlocks = kTileKeys / 16;  // 16-key MFMA blocks per tile
  static constexpr int kTileBytes = G::template tile_bytes<kTileKeys>();         // K or V of one tile
  static constexpr int kWaveBytes = 4 * kTileBytes + 4 * kSparseTableEntries;    // 2 buffers x (K, V) + table
  static constexpr int kRowsPerDma = 1024 / G::kRowBytes;
  static constexpr int kDmaPerTile = kTileKeys / kRowsPerDma;                     // per K (or V)
};

// Sequence of a query token: the last b with cu_q[b] <= tok.
__device__ __forceinline__ int seq_of(const int32_t* cu_q, int num_seqs, int tok) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int KV>
__global__ __launch_bounds__(SparseCfg<KV>::kWaves * 64) void sparse_kernel(SparseArgs a) {
  using C = SparseCfg<KV>;
  using G = typename C::G;
  __shared__ __attribute__((aligned(16))) char smem[C::kWaves][C::kWaveBytes];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int n = lane & 15, gq = lane >> 4;
  const int nrb = (a.r + 15) >> 4;                  // 16-row blocks per kv group
  const int64_t job = (int64_t)blockIdx.x * C::kWaves + w;
  const int64_t njobs = (int64_t)a.num_tokens * a.kv.num_kv_heads * nrb;
  if (job >= njobs) return;
  const int tok = (int)(job / (a.kv.num_kv_heads * nrb));
  const int rem = (int)(job - (int64_t)tok * a.kv.num_kv_heads * nrb);
  const int g = rem / nrb, rb = rem - (rem / nrb) * nrb;
  const int b = seq_of(a.cu_q, a.num_seqs, tok);
  const int lk = a.lens_k[b];

  char* wbase = smem[w];
  lds_t* tiles = (lds_t*)wbase;                                         // [buf][K, V][tile]
  lds_t* table = (lds_t*)(wbase + 4 * C::kTileBytes);                   // int32 [kSparseTableEntries]

  const int hh = 16 * rb + n;
  const bool row_ok = hh < a.r;
  const int head = g * a.r + hh;
  QFragT<KV> qf;
  load_q<kBF16, KV>(qf, a.q, tok, a.hq, head, row_ok);
  const float c2 = a.c2_base * load_scale(a.q_ds) * load_scale(a.kv.k_ds) * qf.rscale;
  const uint8_t* kbase = a.kv.k + g * a.kv.k_sh;
  const uint8_t* vbase = a.kv.v + g * a.kv.v_sh;
  const int32_t* bt_row = a.kv.bt + (int64_t)b * a.kv.bt_stride;
  const int32_t* idx_row = a.idx + (int64_t)tok * a.idx_stride;
  const int pmask = a.kv.page_size - 1;

  WaveState st;
  st.init();

  for (int c0 = 0; c0 < a.num_selected; c0 += kSparseTableEntries) {
    const int cnt = min(kSparseTableEntries, a.num_selected - c0);
    const int ntiles = (cnt + C::kTileKeys - 1) / C::kTileKeys;
    // Translate this chunk's entries (and pad the last tile) into physical rows.
    for (int e = lane; e < ntiles * C::kTileKeys; e += 64) {
      int phys = -1;
      if (e < cnt) {
        const int j = idx_row[c0 + e];
        if (j >= 0 && j < lk) {
          const int page = bt_row[j >> a.kv.page_shift];
          if (page >= 0 && page < a.kv.num_pages) phys = page * a.kv.page_size + (j & pmask);
        }
      }
      lds_store<int>(table + 4 * e, phys);
    }

    auto issue = [&](int it, int buf) {
#pragma unroll
      for (int u = 0; u < C::kDmaPerTile; ++u) {
        const int row0 = u * C::kRowsPerDma;
        const int row = row0 + lane / G::kChunks;
        const int chunk = (lane % G::kChunks) ^ (row & (G::kChunks - 1));
        const int phys = lds_load<int>(table + 4 * (it * C::kTileKeys + row));
        const int64_t page = phys >> a.kv.page_shift;
        const int slot = phys & pmask;
        const uint8_t* ks = phys >= 0 ? kbase + page * a.kv.k_sp + slot * a.kv.k_st + chunk * 16
                                      : reinterpret_cast<const uint8_t*>(g_zero16);
        const uint8_t* vs = phys >= 0 ? vbase + page * a.kv.v_sp + slot * a.kv.v_st + chunk * 16
                                      : reinterpret_cast<const uint8_t*>(g_zero16);
        dma16(ks, tiles + (2 * buf + 0) * C::kTileBytes + row0 * G::kRowBytes);
        dma16(vs, tiles + (2 * buf + 1) * C::kTileBytes + row0 * G::kRowBytes);
      }
    };

    issue(0, 0);
    for (int it = 0; it < ntiles; ++it) {
      if (it + 1 < ntiles) {
        issue(it + 1, (it + 1) & 1);
        wait_vmcnt<2 * C::kDmaPerTile>();
      } else {
        wait_vmcnt<0>();
      }
      const lds_t* kt = tiles + (2 * (it & 1) + 0) * C::kTileBytes;
      const lds_t* vt = tiles + (2 * (it & 1) + 1) * C::kTileBytes;
      f32x4 sc[C::kBlocks];
      tile_scores<KV, C::kBlocks, true>(kt, qf, sc);
      const lds_t* tt = table + 4 * (it * C::kTileKeys);
      const i32x4 v0 = lds_load<i32x4>(tt + 4 * (4 * gq));
      i32x4 v1 = v0;
      if constexpr (C::kBlocks == 2) v1 = lds_load<i32x4>(tt + 4 * (16 + 4 * gq));
      tile_softmax<true>(st, sc, c2, [&](int key) {
        const int q = key - 4 * gq;  // 0..3 in block 0, 16..19 in block 1
        const int e = q & 3;
        const int v = (q < 16) ? v0[e] : v1[e];
        return v >= 0;
      });
      tile_pv<KV, C::kBlocks>(st, vt, sc);
    }
  }

  const float lrow = group4_sum(st.l);
  if (!row_ok) return;
  const float vds = load_scale(a.kv.v_ds);
  const float inv = lrow > 0.f ? vds / lrow : 0.f;
  uint16_t* op = a.out + ((int64_t)tok * a.hq + head) * kHeadDim + 4 * gq;
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) {
    const uint32_t lo = pack_bf16x2(st.o[mb][0] * inv, st.o[mb][1] * inv);
    const uint32_t hi = pack_bf16x2(st.o[mb][2] * inv, st.o[mb][3] * inv);
    *reinterpret_cast<uint2*>(op + 16 * mb) = make_uint2(lo, hi);
  }
  if (gq == 0 && a.lse) a.lse[(int64_t)tok * a.hq + head] = lrow > 0.f ? (st.m + log2f(lrow)) * kLn2 : kNegInf;
}

hipError_t launch_sparse(const SparseArgs& a, int kv_dtype, hipStream_t s) {
  const int nrb = (a.r + 15) / 16;
  const int64_t jobs = (int64_t)a.num_tokens * a.kv.num_kv_heads * nrb;
  if (kv_dtype == kFP8) {
    constexpr int W = SparseCfg<kFP8>::kWaves;
    hipLaunchKernelGGL(sparse_kernel<kFP8>, dim3((unsigned)((jobs + W - 1) / W)), dim3(W * 64), 0, s, a);
  } else {
    constexpr int W = SparseCfg<kBF16>::kWaves;
    hipLaunchKernelGGL(sparse_kernel<kBF16>, dim3((unsigned)((jobs + W - 1) / W)), dim3(W * 64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pga
