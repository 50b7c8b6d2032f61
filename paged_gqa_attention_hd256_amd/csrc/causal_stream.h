// Streaming of a contiguous key range of one (sequence, kv head) through LDS,
// shared by the verify and prefill kernels.
//
// A workgroup of four waves walks keys [k_lo, k_hi) in 64-key tiles.  Each
// wave fetches 16 rows of every tile (K and V) by 16-byte global->LDS DMA into
// a double buffer, then each wave whose 16 query rows are live runs the
// attention core on the tile.  The page of a wave's 16 rows is read with a
// scalar load, so the only vector-memory instructions in flight are the DMA
// and the wait for tile i can let tile i + 1 stay in flight.
#pragma once

#include "attn_core.h"
#include "pga_args.h"

namespace pga {

template <int KV>
struct CausalSmem {
  static constexpr int kTileBytes = TileGeom<KV>::template tile_bytes<64>();
  char buf[2][2][kTileBytes];  // [buffer][K, V]
};

// Uniform load through the scalar data cache (read-only data, uniform address).
template <class T>
__device__ __forceinline__ T scalar_load(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Attend keys [k_lo, k_hi) of kv head g of the sequence whose block-table row
// is bt_row.  c2: this row's log2-domain score multiplier (including the Q
// fragment's rscale).  klim: largest visible key of this lane's query row; min_lim: the
// smallest such limit over the workgroup's rows (tiles entirely at or below it
// skip the mask).  Every wave of the workgroup must call this (it contains
// barriers); `compute` is false for waves without live query rows.
template <int QDT, int KV>
__device__ __forceinline__ void stream_keys(CausalSmem<KV>& sm, const KvArgs& kv, const int32_t* bt_row, int g,
                                            int k_lo, int k_hi, const QFragT<KV>& qf, float c2, int klim,
                                            int min_lim, bool compute, WaveState& st) {
  using G = TileGeom<KV>;
  constexpr int kRowsPerDma = 1024 / G::kRowBytes;  // rows one 1 KB DMA instruction fills
  constexpr int kDmaPerWave = 16 / kRowsPerDma;     // per wave, for its 16 rows of K (or V)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const uint8_t* kbase = kv.k + g * kv.k_sh;
  const uint8_t* vbase = kv.v + g * kv.v_sh;
  const int ntiles = (k_hi - k_lo + 63) >> 6;

  // This wave's rows of a tile (16w .. 16w + 15) lie in one page: pages hold
  // at least 16 tokens and tiles start at multiples of 64.  The page id of tile
  // it + 2 is requested while tile it is being computed, so the scalar read
  // (often a cache miss: block-table rows are long) never delays a DMA issue.
  auto page_of = [&](int it) {
    const int key0 = k_lo + it * 64 + 16 * w;
    const int pidx = __builtin_amdgcn_readfirstlane(min(key0, k_hi - 1) >> kv.page_shift);
    return scalar_load(bt_row + pidx);
  };
  auto issue = [&](int it, int buf, int page) {
    const int tb = k_lo + it * 64;
    const bool page_ok = page >= 0 && page < kv.num_pages;
    const int64_t kpage = (int64_t)page * kv.k_sp;
    const int64_t vpage = (int64_t)page * kv.v_sp;
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
      const int row0 = 16 * w + u * kRowsPerDma;
      const int row = row0 + lane / G::kChunks;
      const int chunk = (lane % G::kChunks) ^ (row & (G::kChunks - 1));
      const int key = tb + row;
      const bool ok = page_ok && key < k_hi;
      const int slot = key & (kv.page_size - 1);
      const uint8_t* ks = ok ? kbase + kpage + slot * kv.k_st + chunk * 16 : reinterpret_cast<const uint8_t*>(g_zero16);
      const uint8_t* vs = ok ? vbase + vpage + slot * kv.v_st + chunk * 16 : reinterpret_cast<const uint8_t*>(g_zero16);
      dma16(ks, (lds_t*)&sm.buf[buf][0][row0 * G::kRowBytes]);
      dma16(vs, (lds_t*)&sm.buf[buf][1][row0 * G::kRowBytes]);
    }
  };

  if (ntiles <= 0) return;
  issue(0, 0, page_of(0));
  int next_page = ntiles > 1 ? page_of(1) : 0;
  for (int it = 0; it < ntiles; ++it) {
    const int after_page = it + 2 < ntiles ? page_of(it + 2) : 0;
    if (it + 1 < ntiles) {
      issue(it + 1, (it + 1) & 1, next_page);
      wait_vmcnt<2 * kDmaPerWave>();
    } else {
      wait_vmcnt<0>();
    }
    next_page = after_page;
    barrier();
    if (compute) {
      const lds_t* kt = (const lds_t*)&sm.buf[it & 1][0][0];
      const lds_t* vt = (const lds_t*)&sm.buf[it & 1][1][0];
      const int tb = k_lo + it * 64;
      f32x4 sc[4];
      tile_scores<KV, 4, QDT == kBF16>(kt, qf, sc);
      const int lim = klim - tb;
      if (tb + 63 > min_lim)  // workgroup-uniform: only tiles past the first row's diagonal or the range end
        tile_softmax<true>(st, sc, c2, [lim](int key) { return key <= lim; });
      else
        tile_softmax<false>(st, sc, c2, [](int) { return true; });
      tile_pv<KV, 4>(st, vt, sc);
    }
    barrier();
  }
}

// Q^T fragment of this lane's query row (lane % 16 of the wave), complete on
// return: a wait left to the compiler would land inside the key loop, where it
// would also drain the LDS copies in flight.  Rows that are not live get zeros.
//   BF16 keys: bf16 queries as they are.
//   FP8 keys:  FP8 queries as they are; bf16 queries scaled by a power of two
//              that puts the row maximum in [128, 256) and split exactly into
//              two FP8 parts (rscale undoes the scaling).
template <int QDT, int KV>
__device__ __forceinline__ void load_q(QFragT<KV>& qf, const void* q, int64_t tok, int hq, int head, bool live) {
  const int gq = lane_id() >> 4;
  qf.rscale = 1.f;
  if constexpr (KV == kBF16) {
    static_assert(QDT == kBF16, "BF16 keys take bf16 queries");
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf.q[ks] = bf16x8{};
    if (live) {
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(q) + (tok * hq + head) * kHeadDim);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf.q[ks] = qp[4 * ks + gq];
    }
  } else if constexpr (QDT == kFP8) {
    qf.has_lo = false;
#pragma unroll
    for (int h = 0; h < 2; ++h) qf.hi[h] = qf.lo[h] = i32x8{};
    if (live) {
      const i32x8* qp = reinterpret_cast<const i32x8*>(static_cast<const uint8_t*>(q) + (tok * hq + head) * kHeadDim);
#pragma unroll
      for (int h = 0; h < 2; ++h) qf.hi[h] = qp[4 * h + gq];
    }
  } else {
    qf.has_lo = true;
    bf16x8 v[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c) v[h][c] = bf16x8{};
    if (live) {
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(q) + (tok * hq + head) * kHeadDim);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[h][c] = qp[16 * h + 4 * gq + c];
    }
    wait_vmcnt<0>();
    float amax = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)v[h][c][j]));
    amax = group4_max(amax);
    int e = 0;
    frexpf(amax, &e);  // amax = m * 2^e, m in [0.5, 1)
    const int sh = amax > 0.f ? min(max(8 - e, -120), 120) : 0;
    const float sc = ldexpf(1.f, sh);
    qf.rscale = ldexpf(1.f, -sh);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (float)v[h][c][j] * sc;
        int h0, h1, l0, l1;
        split_q8(x, h0, h1, l0, l1);
        qf.hi[h][2 * c] = h0;
        qf.hi[h][2 * c + 1] = h1;
        qf.lo[h][2 * c] = l0;
        qf.lo[h][2 * c + 1] = l1;
      }
    }
  }
  wait_vmcnt<0>();
}

// Final bf16 output row (and lse) of one wave's query row from its state.
__device__ __forceinline__ void store_out(const WaveState& st, float lrow, float vds, uint16_t* out, float* lse,
                                          int64_t tok, int hq, int head) {
  const int gq = lane_id() >> 4;
  const float inv = lrow > 0.f ? vds / lrow : 0.f;
  uint16_t* op = out + (tok * hq + head) * kHeadDim + 4 * gq;
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) {
    const uint32_t lo = pack_bf16x2(st.o[mb][0] * inv, st.o[mb][1] * inv);
    const uint32_t hi = pack_bf16x2(st.o[mb][2] * inv, st.o[mb][3] * inv);
    *reinterpret_cast<uint2*>(op + 16 * mb) = make_uint2(lo, hi);
  }
  if (gq == 0 && lse) lse[tok * hq + head] = lrow > 0.f ? (st.m + log2f(lrow)) * kLn2 : kNegInf;
}

}  // namespace pga
