// Streaming of a contiguous key range of one (sequence, kv head) through LDS
// for the verify kernels, and the attention of the workgroup's 16 * NW query
// rows on each streamed tile (NW = 4 waves).
//
// A workgroup of NW waves walks keys [k_lo, k_hi) in 64-key tiles.  Each wave
// fetches 64 / NW rows of every tile (K and V) by 16-byte global->LDS DMA into
// a double buffer.  The page of a wave's rows is read with a scalar load, so
// the only vector-memory instructions in flight are the DMA and the wait for
// tile i can let tile i + 1 stay in flight.
//
// On a tile the work is split two ways.  For QK^T and the softmax, wave w owns
// query rows 16w .. 16w + 15 (its scores and running maximum); it publishes
// the probabilities, already in the B-operand layout of the PV MFMA, and its
// rows' rescale factors to LDS.  For PV, wave w owns head dimensions
// (256 / NW) w .. (256 / NW)(w + 1) - 1 of all rows, so each wave reads and
// widens a 1/NW share of the V tile instead of all of it.
#pragma once

#include "attn_core.h"
#include "pga_args.h"

namespace pga {

// Exchange area between the softmax of a tile and its PV product.
template <int KV, int NW>
struct Exchange {
  static constexpr int kPVec = (KV == kFP8) ? 1 : 2;  // 16-byte P fragments per lane: fp16, or bf16 high + low
  i32x4 p[NW][2][kPVec][64];                          // [row block][32-key step][part][lane]
  float row[16 * NW];  // per row: rescale factor of the current tile; at the end, the row sum
  int grow[NW];        // per softmax wave: whether any of its rows was rescaled on this tile
};

template <int KV, int NW>
struct CausalSmem {
  static constexpr int kWaves = NW;
  static constexpr int kTileBytes = TileGeom<KV>::template tile_bytes<64>();
  char buf[2][2][kTileBytes];  // [buffer][K, V]
  Exchange<KV, NW> x;
};

// Running maximum (log2 domain) of one softmax row.
struct RowStat {
  float m;
  __device__ __forceinline__ void init() { m = kNegInf; }
};

// Uniform load through the scalar data cache (read-only data, uniform address).
template <class T>
__device__ __forceinline__ T scalar_load(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Stream keys [k_lo, k_hi) of kv head g of the sequence whose block-table row
// is bt_row through LDS (`first`: first_pages() of the same range), calling
// tile.front(kt, tb) and then tile.back(vt, tb)
// on every 64-key tile in every wave (kt / vt: the tile's K and V in LDS; tb:
// its first key).  front may read only K and back only V and the exchange
// area; a barrier separates them.  Every wave of the workgroup must call this.
//
// K and V have separate double buffers: K of tile i + 2 is requested as soon
// as front(i) is done with K of tile i (about 1.5 tiles ahead), V of tile i + 1
// as soon as back(i - 1) is done with V of tile i - 1 (one tile ahead), so two
// barriers per tile suffice and more of the gather is in flight.
// Page ids of this wave's rows of the first two tiles of [k_lo, k_hi) (see
// stream_keys).  Reading them before the queries load lets both reads overlap.
template <int NW>
__device__ __forceinline__ int2 first_pages(const KvArgs& kv, const int32_t* bt_row, int k_lo, int k_hi) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p0 = __builtin_amdgcn_readfirstlane(min(k_lo + (64 / NW) * w, k_hi - 1) >> kv.page_shift);
  const int p1 = __builtin_amdgcn_readfirstlane(min(k_lo + 64 + (64 / NW) * w, k_hi - 1) >> kv.page_shift);
  return int2{k_hi > k_lo ? scalar_load(bt_row + p0) : 0, k_hi > k_lo + 64 ? scalar_load(bt_row + p1) : 0};
}

// The keys are read exactly once (each piece of each history belongs to one
// workgroup), so their copies use the non-temporal cache policy.
template <int KV, int NW, class Tile>
__device__ __forceinline__ void stream_keys(CausalSmem<KV, NW>& sm, const KvArgs& kv, const int32_t* bt_row, int g,
                                            int k_lo, int k_hi, int2 first, const Tile& tile) {
  using G = TileGeom<KV>;
  constexpr int kRowsPerWave = 64 / NW;                   // rows of a tile each wave fetches
  constexpr int kRowsPerDma = 1024 / G::kRowBytes;        // rows one 1 KB DMA instruction fills
  constexpr int kDma = kRowsPerWave / kRowsPerDma;        // per wave, for its rows of K (or V)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int ntiles = (k_hi - k_lo + 63) >> 6;

  // This wave's rows of a tile lie in one page: pages hold at least 16 tokens
  // and tiles start at multiples of 64.  Page ids are read
  // with scalar loads two tiles ahead, so the read (often a cache miss:
  // block-table rows are long) never delays a DMA issue.
  auto page_of = [&](int it) {
    const int key0 = k_lo + it * 64 + kRowsPerWave * w;
    const int pidx = __builtin_amdgcn_readfirstlane(min(key0, k_hi - 1) >> kv.page_shift);
    return scalar_load(bt_row + pidx);
  };
  // kDma DMA instructions per call, from the wave's page (a uniform base) plus
  // a 32-bit offset per lane.  Tiles start at multiples of 64 keys, so a row's
  // slot in its page is (tb mod page_size) + (row mod page_size): the lane
  // part is fixed for the whole stream and the rest joins the uniform base.
  // In the range's last tile, keys at or past k_hi read key k_hi - 1 instead
  // (finite data that the mask gives probability 0).  A page id outside the
  // pool reads zeros.
  const unsigned pmask = kv.page_size - 1;
  unsigned lane_k[kDma], lane_v[kDma];
#pragma unroll
  for (int u = 0; u < kDma; ++u) {
    const int row = kRowsPerWave * w + u * kRowsPerDma + lane / G::kChunks;
    const unsigned chunk = (lane % G::kChunks) ^ (row & (G::kChunks - 1));
    lane_k[u] = (row & pmask) * (unsigned)kv.k_st + chunk * 16;
    lane_v[u] = (row & pmask) * (unsigned)kv.v_st + chunk * 16;
  }
  // LDS byte address of the tile buffers (a constant: sm is a static LDS object).
  const unsigned lds_buf = (unsigned)(uintptr_t)(lds_t*)&sm.buf[0][0][0];
  auto issue = [&](int it, int page, const uint8_t* base, int64_t sh, int64_t sp, int64_t st,
                   const unsigned (&lane_off)[kDma], unsigned dst) {
    const int tb = k_lo + it * 64;
    const bool page_ok = page >= 0 && page < kv.num_pages;
    const uint64_t pbase = page_ok ? (uint64_t)(uintptr_t)(base + g * sh + (int64_t)page * sp)
                                   : (uint64_t)(uintptr_t)g_zero16;
    if (!page_ok) {
#pragma unroll
      for (int u = 0; u < kDma; ++u) dma16_off<true>(pbase, 0u, dst + (kRowsPerWave * w + u * kRowsPerDma) * G::kRowBytes);
    } else if (tb + 64 <= k_hi) {  // every key of the tile exists
      const uint64_t tbase = pbase + (uint64_t)((tb & pmask) * (unsigned)st);
#pragma unroll
      for (int u = 0; u < kDma; ++u)
        dma16_off<true>(tbase, lane_off[u], dst + (kRowsPerWave * w + u * kRowsPerDma) * G::kRowBytes);
    } else {
#pragma unroll
      for (int u = 0; u < kDma; ++u) {
        const int row0 = kRowsPerWave * w + u * kRowsPerDma;
        const int row = row0 + lane / G::kChunks;
        const unsigned chunk = (lane % G::kChunks) ^ (row & (G::kChunks - 1));
        const unsigned key = (unsigned)min(tb + row, k_hi - 1);
        dma16_off<true>(pbase, (key & pmask) * (unsigned)st + chunk * 16, dst + row0 * G::kRowBytes);
      }
    }
  };
  constexpr unsigned kTile = CausalSmem<KV, NW>::kTileBytes;
  auto issue_k = [&](int it, int page) {
    issue(it, page, kv.k, kv.k_sh, kv.k_sp, kv.k_st, lane_k, lds_buf + (2 * (it & 1) + 0) * kTile);
  };
  auto issue_v = [&](int it, int page) {
    issue(it, page, kv.v, kv.v_sh, kv.v_sp, kv.v_st, lane_v, lds_buf + (2 * (it & 1) + 1) * kTile);
  };

  if (ntiles <= 0) return;
  const int pg0 = first.x;
  issue_k(0, pg0);
  issue_v(0, pg0);
  int pg1 = first.y;  // page of tile it + 1
  if (ntiles > 1) {
    issue_k(1, pg1);
    issue_v(1, pg1);
  }
  for (int it = 0; it < ntiles; ++it) {
    const int pg2 = it + 2 < ntiles ? page_of(it + 2) : 0;
    // DMA issue order: ..., K(it) V(it) | then K(it + 1) (and, at it = 0, V(1)).
    if (it == 0) {
      if (ntiles > 1) wait_vmcnt<2 * kDma>(); else wait_vmcnt<0>();
    } else {
      if (it + 1 < ntiles) wait_vmcnt<kDma>(); else wait_vmcnt<0>();
    }
    barrier();  // tile it is in LDS; every wave is done with back(it - 1)
    if (it >= 1 && it + 1 < ntiles) issue_v(it + 1, pg1);
    const int tb = k_lo + it * 64;
    tile.front((const lds_t*)&sm.buf[it & 1][0][0], tb);
    barrier_publish();  // every wave is done with K of tile it; the exchange area is complete
    if (it + 2 < ntiles) issue_k(it + 2, pg2);
    tile.back((const lds_t*)&sm.buf[it & 1][1][0], tb);
    pg1 = pg2;
  }
}

// Online softmax of this wave's 16 rows on a tile (scores s from tile_scores;
// reference maximum raised only past kRescaleLog2): the rescale factor is
// published for the PV waves instead of being applied, the probabilities go
// to LDS as PV operands, and the row sums are left to the PV step (see
// pv_quarter).
template <int KV, bool MASKED, class Vis, int NW>
__device__ __forceinline__ void softmax_publish(RowStat& rs, f32x4 (&s)[4], float c2, Vis visible,
                                                Exchange<KV, NW>& x, int w) {
  const int lane = lane_id();
  const int gq = lane >> 4, n = lane & 15;
  float mt = kNegInf;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = s[mb][i] * c2;
      if constexpr (MASKED) v = visible(mb * 16 + 4 * gq + i) ? v : kNegInf;
      s[mb][i] = v;
      mt = fmaxf(mt, v);
    }
  }
  mt = group4_max(mt);
  const uint64_t grow = __builtin_amdgcn_ballot_w64(mt > rs.m + kRescaleLog2);
  float alpha = 1.f;
  if (grow != 0) {  // wave-uniform
    const float m_new = fmaxf(rs.m, mt);
    alpha = m_new == rs.m ? 1.f : fast_exp2(rs.m - m_new);
    rs.m = m_new;
  }
  const float m_use = (rs.m == kNegInf) ? 0.f : rs.m;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) s[mb][i] = fast_exp2(s[mb][i] - m_use);
  if (gq == 0) x.row[16 * w + n] = alpha;
  if (lane == 0) x.grow[w] = grow != 0;
  // B operand of the 32-key step t: keys 32t + 4gq + i and 32t + 16 + 4gq + i.
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if constexpr (KV == kFP8) {
      const f16x8 pb = {(_Float16)s[2 * t][0],     (_Float16)s[2 * t][1],     (_Float16)s[2 * t][2],
                        (_Float16)s[2 * t][3],     (_Float16)s[2 * t + 1][0], (_Float16)s[2 * t + 1][1],
                        (_Float16)s[2 * t + 1][2], (_Float16)s[2 * t + 1][3]};
      x.p[w][t][0][lane] = __builtin_bit_cast(i32x4, pb);
    } else {
      bf16x8 ph, pl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = s[2 * t + (j >> 2)][j & 3];
        const __bf16 h = (__bf16)v;
        ph[j] = h;
        pl[j] = (__bf16)(v - (float)h);
      }
      x.p[w][t][0][lane] = __builtin_bit_cast(i32x4, ph);
      x.p[w][t][1][lane] = __builtin_bit_cast(i32x4, pl);
    }
  }
}

// A wave without live query rows: zero probabilities and no rescale.
template <int KV, int NW>
__device__ __forceinline__ void publish_nothing(Exchange<KV, NW>& x, int w) {
  const int lane = lane_id();
  if (lane < 16) x.row[16 * w + lane] = 1.f;
  if (lane == 0) x.grow[w] = 0;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c = 0; c < Exchange<KV, NW>::kPVec; ++c) x.p[w][t][c][lane] = i32x4{0, 0, 0, 0};
}

// O^T += V^T P^T for head dimensions (256 / NW) w .. of all 16 NW rows, after
// applying the published rescale factors: with DB = 16 / NW d-blocks per wave,
// o[DB * rb + db] holds rows 16rb + lane % 16 and dims
// (256 / NW) w + 16db + 4 (lane / 16) + i.
//
// The row sums of the wave's own softmax rows (row block w) come from the same
// MFMAs with an all-ones A operand: lsum[i] = sum of this tile's P of row
// 16w + lane % 16 (as rounded for PV), accumulated and rescaled like O.
template <int KV, int NW>
__device__ __forceinline__ void pv_quarter(f32x4 (&o)[16], f32x4& lsum, const lds_t* vt, const Exchange<KV, NW>& x,
                                           int w) {
  using G = TileGeom<KV>;
  constexpr int DB = 16 / NW;
  const int lane = lane_id();
  const int gq = lane >> 4, sl = lane & 15;
  int any = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) any |= x.grow[i];
  if (__builtin_amdgcn_readfirstlane(any) != 0) {
#pragma unroll
    for (int rb = 0; rb < NW; ++rb) {
      const float al = x.row[16 * rb + sl];
#pragma unroll
      for (int db = 0; db < DB; ++db) o[DB * rb + db] *= al;
    }
    lsum *= x.row[16 * w + sl];
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if constexpr (KV == kFP8) {
      f16x8 pb[NW];
#pragma unroll
      for (int rb = 0; rb < NW; ++rb) pb[rb] = __builtin_bit_cast(f16x8, x.p[rb][t][0][lane]);
      // transpose-read source: lane sl = 2e + q points at key(e), bytes 8q..8q+7 of the d-block
      const int e = sl >> 1, q = sl & 1;
      const int key = 32 * t + 16 * (e >> 2) + 4 * gq + (e & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f16x8 a = fp8x8_to_f16(lds_tr8(vt + G::off(key, DB * w + db) + 8 * q));
#pragma unroll
        for (int rb = 0; rb < NW; ++rb) o[DB * rb + db] = mfma_f16(a, pb[rb], o[DB * rb + db]);
      }
      constexpr f16x8 ones = {(_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f,
                              (_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f};
      lsum = mfma_f16(ones, __builtin_bit_cast(f16x8, x.p[w][t][0][lane]), lsum);
    } else {
      bf16x8 ph[NW], pl[NW];
#pragma unroll
      for (int rb = 0; rb < NW; ++rb) {
        ph[rb] = __builtin_bit_cast(bf16x8, x.p[rb][t][0][lane]);
        pl[rb] = __builtin_bit_cast(bf16x8, x.p[rb][t][1][lane]);
      }
      // transpose-read source: lane sl = 4e + q points at key(e), columns 4q..4q+3
      const int e = sl >> 2, q = sl & 3;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int chunk = 2 * (DB * w + db) + (q >> 1);
        const int key0 = 32 * t + 4 * gq + e;
        const i32x2 lo = __builtin_bit_cast(i32x2, lds_tr16(vt + G::off(key0, chunk) + 8 * (q & 1)));
        const i32x2 hi = __builtin_bit_cast(i32x2, lds_tr16(vt + G::off(key0 + 16, chunk) + 8 * (q & 1)));
        const bf16x8 a = __builtin_bit_cast(bf16x8, i32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int rb = 0; rb < NW; ++rb) {
          o[DB * rb + db] = mfma_bf16(a, ph[rb], o[DB * rb + db]);
          o[DB * rb + db] = mfma_bf16(a, pl[rb], o[DB * rb + db]);
        }
      }
      const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                           (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
      lsum = mfma_bf16(ones, __builtin_bit_cast(bf16x8, x.p[w][t][0][lane]), lsum);
      lsum = mfma_bf16(ones, __builtin_bit_cast(bf16x8, x.p[w][t][1][lane]), lsum);
    }
  }
}

// The workgroup's 16 NW rows on one streamed tile.  qf, c2, klim, rs: this
// wave's softmax rows (c2 includes the Q fragment's rscale; klim is the largest
// visible key of this lane's row); min_lim: the smallest such limit over the
// workgroup's rows (tiles entirely at or below it skip the mask); live: this
// wave has live softmax rows; o, lsum: this wave's PV share.
template <int QDT, int KV, int NW>
struct SplitTile {
  const QFragT<KV>& qf;
  float c2;
  int klim, min_lim;
  bool live;
  RowStat& rs;
  f32x4 (&o)[16];
  f32x4& lsum;
  Exchange<KV, NW>& x;
  __device__ __forceinline__ void front(const lds_t* kt, int tb) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (live) {
      f32x4 sc[4];
      tile_scores<KV, 4, QDT == kBF16>(kt, qf, sc);
      const int lim = klim - tb;
      if (tb + 63 > min_lim)  // workgroup-uniform: only tiles past the first row's diagonal or the range end
        softmax_publish<KV, true>(rs, sc, c2, [lim](int key) { return key <= lim; }, x, w);
      else
        softmax_publish<KV, false>(rs, sc, c2, [](int) { return true; }, x, w);
    } else {
      publish_nothing(x, w);
    }
  }
  __device__ __forceinline__ void back(const lds_t* vt, int) const {
    pv_quarter<KV, NW>(o, lsum, vt, x, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
  }
};

// After the last tile: each wave publishes the sums of its softmax rows (0 for
// a wave without live rows) so that every wave can normalise its PV share;
// returns this lane's row sum.  Contains a barrier.
template <int KV, int NW>
__device__ __forceinline__ float finish_rows(const f32x4& lsum, bool live, Exchange<KV, NW>& x) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const float lrow = live ? lsum[0] : 0.f;
  if (lane < 16) x.row[16 * w + lane] = lrow;
  barrier_publish();
  return lrow;
}

// Row block rb of this wave's PV share times `scale`, written to a row of 256
// head dimensions: bf16 (output), fp16 or fp32 (partials).
template <int NW>
__device__ __forceinline__ void store_share_bf16(const f32x4 (&o)[16], int rb, float scale, uint16_t* row_base) {
  constexpr int DB = 16 / NW;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gq = lane_id() >> 4;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const f32x4 v = o[DB * rb + db];
    *reinterpret_cast<uint2*>(row_base + (256 / NW) * w + 16 * db + 4 * gq) =
        make_uint2(pack_bf16x2(v[0] * scale, v[1] * scale), pack_bf16x2(v[2] * scale, v[3] * scale));
  }
}
template <int NW>
__device__ __forceinline__ void store_share_f16(const f32x4 (&o)[16], int rb, float scale, uint16_t* row_base) {
  constexpr int DB = 16 / NW;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gq = lane_id() >> 4;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const f32x4 v = o[DB * rb + db] * scale;
    const f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<f16x4*>(row_base + (256 / NW) * w + 16 * db + 4 * gq) = h;
  }
}
template <int NW>
__device__ __forceinline__ void store_share_f32(const f32x4 (&o)[16], int rb, float scale, float* row_base) {
  constexpr int DB = 16 / NW;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gq = lane_id() >> 4;
#pragma unroll
  for (int db = 0; db < DB; ++db)
    *reinterpret_cast<f32x4*>(row_base + (256 / NW) * w + 16 * db + 4 * gq) = o[DB * rb + db] * scale;
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

}  // namespace pga
