// Prefill of new tokens against a cached prefix, bottom-right causal.
//
// One workgroup per (tile of query tokens, kv head, sequence): the tile packs
// rows / r tokens x r heads of one kv group (token-major rows), and streams all
// keys from 0 to the tile's last diagonal position, with the mask of ROCm/ATOM
// PR #2534 (FMHA commit message: the cached + new keys are longer than the
// queries and the causal mask is bottom-right aligned).  Pages are read in the
// kernel, with no gather to contiguous memory first (ROCm/ATOM PR #2830, recipe
// commit).  Workgroups are ordered longest first.
//
// One warp-specialised kernel serves FP8 queries with FP8 keys (the pages'
// FP8 FMHA), bf16 queries with bf16 keys, and bf16 queries against FP8 keys.
#include <type_traits>

#include "causal_stream.h"

namespace pga {

// ---------------------------------------------------------------------------
// A warp-specialised, software-pipelined tile loop.  Tiles hold 64 FP8 or 32
// bf16 keys (16 KB of K and of V either way).
//
// The verify kernel's tile step runs a tile's QK^T, softmax and PV back to
// back in every wave, so a wave's vector work (scaling, maxima, exponentials,
// conversions) and its matrix work follow each other.  Here the eight waves
// of a workgroup (128 rows, one workgroup per CU) split by kind of work:
//  - waves 0 .. 3 compute scores and softmax, wave w for rows 32 w .. 32 w + 31
//    (two 16-row blocks sharing every K fragment read from LDS), and issue
//    every tile copy (a quarter of the rows of each K and V tile per wave);
//  - waves 4 .. 7 compute the PV product, wave 4 + d for head dims
//    64 d .. 64 d + 63 of all 128 rows.
// Each SIMD holds one wave of each kind, so the softmax's vector work runs
// beside the PV matrix work, and every K tile and every tile of probabilities
// is read from LDS by four waves.  Iteration i: the softmax waves process tile
// i + 1 while the PV waves multiply tile i.  Probabilities are double buffered
// (tile i's are read while tile i + 1's are written), K and V tiles triple
// buffered (copies run two iterations ahead), and one barrier per iteration
// publishes tile i's probabilities and retires every read of the buffers the
// next copies fill.
constexpr int kPipeStages = 3;
constexpr int kPipeRows = 128;  // query rows per workgroup
// Keys per tile: 64 FP8 keys, 32 bf16 keys -- the same 16 KB of K (and of V)
// per stage, so three stages of both fit LDS with the probabilities.
template <int KV>
constexpr int kWsKeys = KV == kFP8 ? 64 : 32;

// Probabilities of one tile for the PV waves: per row block, 32-key step and
// part (fp16 P; bf16 P as a high and a low part), the B operand of each lane;
// the rows' rescale factors, and per row block whether any row was rescaled.
template <int KV, int NRB>
struct WsExchange {
  static constexpr int kSteps = kWsKeys<KV> / 32;
  static constexpr int kPVec = KV == kFP8 ? 1 : 2;
  i32x4 p[NRB][kSteps][kPVec][64];
  float row[16 * NRB];
  int grow[NRB];
};

template <int KV, int NRB>
struct PipeSmem {
  static constexpr int kTile = TileGeom<KV>::template tile_bytes<kWsKeys<KV>>();
  char k[kPipeStages][kTile];
  char v[kPipeStages][kTile];
  WsExchange<KV, NRB> x[2];
};

// Copies of this wave's rows of one tile of K or V (global -> LDS).
template <int KV, int NW>
struct TileCopy {
  using G = TileGeom<KV, KV == kBF16>;  // bf16 tiles use the spread swizzle
  static constexpr int kKeys = kWsKeys<KV>;
  static constexpr int kRowsPerWave = kKeys / NW;
  static constexpr int kRowsPerDma = 1024 / G::kRowBytes;
  static constexpr int kDma = kRowsPerWave / kRowsPerDma;
  static_assert(kDma * kRowsPerDma == kRowsPerWave, "whole DMA instructions per wave");
  const KvArgs& kv;
  const int32_t* bt_row;
  int g, k_hi, w;
  unsigned lane_k[kDma], lane_v[kDma];

  __device__ __forceinline__ TileCopy(const KvArgs& kv_, const int32_t* bt, int g_, int k_hi_)
      : kv(kv_), bt_row(bt), g(g_), k_hi(k_hi_), w(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    const int lane = lane_id();
    const unsigned pmask = kv.page_size - 1;
#pragma unroll
    for (int u = 0; u < kDma; ++u) {
      const int row = kRowsPerWave * w + u * kRowsPerDma + lane / G::kChunks;
      const unsigned chunk = (lane % G::kChunks) ^ ((KV == kFP8 ? row : 2 * row) & (G::kChunks - 1));
      lane_k[u] = (row & pmask) * (unsigned)kv.k_st + chunk * 16;
      lane_v[u] = (row & pmask) * (unsigned)kv.v_st + chunk * 16;
    }
  }
  // Page holding this wave's rows of tile `it` (keys from 0), read through the
  // scalar cache; all of them lie in one page (pages hold at least 16 keys).
  __device__ __forceinline__ int page(int it) const {
    const int key0 = it * kKeys + kRowsPerWave * w;
    const int pidx = __builtin_amdgcn_readfirstlane(min(key0, k_hi - 1) >> kv.page_shift);
    return scalar_load(bt_row + pidx);
  }
  // Keys at or past k_hi read key k_hi - 1 (masked later); a page id outside
  // the pool reads zeros.
  __device__ __forceinline__ void issue(int it, int page, bool is_v, unsigned dst) const {
    const uint8_t* base = is_v ? kv.v : kv.k;
    const int64_t sh = is_v ? kv.v_sh : kv.k_sh, sp = is_v ? kv.v_sp : kv.k_sp, st = is_v ? kv.v_st : kv.k_st;
    const int tb = it * kKeys;
    const unsigned pmask = kv.page_size - 1;
    const bool page_ok = page >= 0 && page < kv.num_pages;
    const uint64_t pbase = page_ok ? (uint64_t)(uintptr_t)(base + g * sh + (int64_t)page * sp)
                                   : (uint64_t)(uintptr_t)g_zero16;
    if (!page_ok) {
#pragma unroll
      for (int u = 0; u < kDma; ++u) dma16_off(pbase, 0u, dst + (kRowsPerWave * w + u * kRowsPerDma) * G::kRowBytes);
    } else if (tb + kKeys <= k_hi) {
      const uint64_t tbase = pbase + (uint64_t)((tb & pmask) * (unsigned)st);
#pragma unroll
      for (int u = 0; u < kDma; ++u)
        dma16_off(tbase, is_v ? lane_v[u] : lane_k[u], dst + (kRowsPerWave * w + u * kRowsPerDma) * G::kRowBytes);
    } else {
      const int lane = lane_id();
#pragma unroll
      for (int u = 0; u < kDma; ++u) {
        const int row0 = kRowsPerWave * w + u * kRowsPerDma;
        const int row = row0 + lane / G::kChunks;
        const unsigned chunk = (lane % G::kChunks) ^ ((KV == kFP8 ? row : 2 * row) & (G::kChunks - 1));
        const unsigned key = (unsigned)min(tb + row, k_hi - 1);
        dma16_off(pbase, (key & pmask) * (unsigned)st + chunk * 16, dst + row0 * G::kRowBytes);
      }
    }
  }
};

// Softmax of one 16-row block (global block rb) on one tile, straight-line:
// raw scores s (scaled by c2 > 0 here: max(c2 s) = c2 max(s)), optional mask
// (key relative to the tile start visible iff <= lim), lazy reference maximum
// as in softmax_publish, probabilities published as the fp16 B operand with
// the row rescale factors and the block's rescale flag next to them, and the
// block's running row sums from an all-ones A operand.
template <bool MASKED, int NRB>
__device__ __forceinline__ void softmax_ws(RowStat& rs, f32x4& lsum, f32x4 (&s)[4], float c2, int lim,
                                           WsExchange<kFP8, NRB>& x, int rb) {
  const int lane = lane_id();
  const int gq = lane >> 4, n = lane & 15;
  float mt = kNegInf;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (MASKED) s[mb][i] = (mb * 16 + 4 * gq + i <= lim) ? s[mb][i] : kNegInf;
      mt = fmaxf(mt, s[mb][i]);
    }
  mt = group4_max(mt);
  mt = mt == kNegInf ? kNegInf : mt * c2;
  const bool grow = __builtin_amdgcn_ballot_w64(mt > rs.m + kRescaleLog2) != 0;  // wave-uniform
  const float m_new = grow ? fmaxf(rs.m, mt) : rs.m;
  const float alpha = m_new == rs.m ? 1.f : fast_exp2(rs.m - m_new);
  rs.m = m_new;
  const float nm = m_new == kNegInf ? 0.f : -m_new;
  x.row[16 * rb + n] = alpha;
  x.grow[rb] = grow;
  lsum *= alpha;
  constexpr f16x8 ones = {(_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f,
                          (_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f16x8 pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[j] = (_Float16)fast_exp2(__builtin_fmaf(s[2 * t + (j >> 2)][j & 3], c2, nm));
    x.p[rb][t][0][lane] = __builtin_bit_cast(i32x4, pb);
    lsum = mfma_f16(ones, pb, lsum);
  }
}

// PV of one tile for head dims 64 d .. 64 d + 63 of all NRB row blocks, after
// rescaling the rows whose maximum moved.
template <int NRB>
__device__ __forceinline__ void pv_ws(f32x4 (&o)[4 * NRB], const lds_t* vt, const WsExchange<kFP8, NRB>& x, int d) {
  using G = TileGeom<kFP8>;
  const int lane = lane_id();
  const int gq = lane >> 4, sl = lane & 15;
  int any = 0;
#pragma unroll
  for (int i = 0; i < NRB; ++i) any |= x.grow[i];
  // Every fragment of the tile is requested before the first product, so the
  // LDS latency is paid once per tile rather than once per row block.
  const int e = sl >> 1, q = sl & 1;
  i32x2 vr[2][4];
  i32x4 pr[2][NRB];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = 32 * t + 16 * (e >> 2) + 4 * gq + (e & 3);
#pragma unroll
    for (int db = 0; db < 4; ++db) vr[t][db] = lds_tr8(vt + G::off(key, 4 * d + db) + 8 * q);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) pr[t][rb] = x.p[rb][t][0][lane];
  }
  asm volatile("" ::: "memory");
  if (__builtin_amdgcn_readfirstlane(any) != 0) {
#pragma unroll
    for (int i = 0; i < 4 * NRB; ++i) asm volatile("" : "+v"(o[i]));
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float al = x.row[16 * rb + sl];
#pragma unroll
      for (int db = 0; db < 4; ++db) o[4 * rb + db] *= al;
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f16x8 av[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) av[db] = fp8x8_to_f16(vr[t][db]);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const f16x8 pb = __builtin_bit_cast(f16x8, pr[t][rb]);
#pragma unroll
      for (int db = 0; db < 4; ++db) o[4 * rb + db] = mfma_f16(av[db], pb, o[4 * rb + db]);
    }
  }
}

// bf16 queries and keys, 32-key tiles.  Scores of the wave's NRB row blocks:
// each K fragment read from LDS feeds one bf16 MFMA per row block.
template <int NRB, int NMB>
__device__ __forceinline__ void tile_scores_rows_bf16(const lds_t* kt, const QFragT<kBF16> (&qf)[NRB],
                                                      f32x4 (&s)[NRB][NMB]) {
  using G = TileGeom<kBF16, true>;
  const int lane = lane_id();
  const int n = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) s[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const bf16x8 k8 = lds_load<bf16x8>(kt + G::off(mb * 16 + n, 4 * ks + gq));
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) s[rb][mb] = mfma_bf16(k8, qf[rb].q[ks], s[rb][mb]);
    }
  }
}

// softmax_ws on a 32-key tile of bf16 keys: the probabilities are published as
// a bf16 high and low part (keys 4 (lane / 16) + i and 16 + 4 (lane / 16) + i,
// the B-operand order of the 32-key step), and the row sums count both parts.
template <bool MASKED, int NRB>
__device__ __forceinline__ void softmax_ws_bf16(RowStat& rs, f32x4& lsum, f32x4 (&s)[2], float c2, int lim,
                                                WsExchange<kBF16, NRB>& x, int rb) {
  const int lane = lane_id();
  const int gq = lane >> 4, n = lane & 15;
  float mt = kNegInf;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (MASKED) s[mb][i] = (mb * 16 + 4 * gq + i <= lim) ? s[mb][i] : kNegInf;
      mt = fmaxf(mt, s[mb][i]);
    }
  mt = group4_max(mt);
  mt = mt == kNegInf ? kNegInf : mt * c2;
  const bool grow = __builtin_amdgcn_ballot_w64(mt > rs.m + kRescaleLog2) != 0;  // wave-uniform
  const float m_new = grow ? fmaxf(rs.m, mt) : rs.m;
  const float alpha = m_new == rs.m ? 1.f : fast_exp2(rs.m - m_new);
  rs.m = m_new;
  const float nm = m_new == kNegInf ? 0.f : -m_new;
  x.row[16 * rb + n] = alpha;
  x.grow[rb] = grow;
  lsum *= alpha;
  bf16x8 ph, pl;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float v = fast_exp2(__builtin_fmaf(s[j >> 2][j & 3], c2, nm));
    const __bf16 h = (__bf16)v;
    ph[j] = h;
    pl[j] = (__bf16)(v - (float)h);
  }
  x.p[rb][0][0][lane] = __builtin_bit_cast(i32x4, ph);
  x.p[rb][0][1][lane] = __builtin_bit_cast(i32x4, pl);
  const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                       (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
  lsum = mfma_bf16(ones, ph, lsum);
  lsum = mfma_bf16(ones, pl, lsum);
}

// pv_ws on a 32-key tile of bf16 values: V^T by 16-bit transpose reads (lane
// sl = 4e + q points at key 4 (lane / 16) + e, or 16 more, columns 4q .. 4q + 3
// of the d-block), two bf16 products per block (high and low part of P).
template <int NRB>
__device__ __forceinline__ void pv_ws_bf16(f32x4 (&o)[4 * NRB], const lds_t* vt, const WsExchange<kBF16, NRB>& x,
                                           int d) {
  using G = TileGeom<kBF16, true>;
  const int lane = lane_id();
  const int gq = lane >> 4, sl = lane & 15;
  int any = 0;
#pragma unroll
  for (int i = 0; i < NRB; ++i) any |= x.grow[i];
  const int e = sl >> 2, q = sl & 3;
  bf16x8 av[4];
  i32x4 ph[NRB], pl[NRB];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int chunk = 2 * (4 * d + db) + (q >> 1);
    const i32x2 k0 = __builtin_bit_cast(i32x2, lds_tr16(vt + G::off(4 * gq + e, chunk) + 8 * (q & 1)));
    const i32x2 k1 = __builtin_bit_cast(i32x2, lds_tr16(vt + G::off(16 + 4 * gq + e, chunk) + 8 * (q & 1)));
    av[db] = __builtin_bit_cast(bf16x8, i32x4{k0[0], k0[1], k1[0], k1[1]});
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    ph[rb] = x.p[rb][0][0][lane];
    pl[rb] = x.p[rb][0][1][lane];
  }
  asm volatile("" ::: "memory");
  if (__builtin_amdgcn_readfirstlane(any) != 0) {
#pragma unroll
    for (int i = 0; i < 4 * NRB; ++i) asm volatile("" : "+v"(o[i]));
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float al = x.row[16 * rb + sl];
#pragma unroll
      for (int db = 0; db < 4; ++db) o[4 * rb + db] *= al;
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const bf16x8 h = __builtin_bit_cast(bf16x8, ph[rb]), l = __builtin_bit_cast(bf16x8, pl[rb]);
#pragma unroll
    for (int db = 0; db < 4; ++db) o[4 * rb + db] = mfma_bf16(av[db], h, o[4 * rb + db]);
#pragma unroll
    for (int db = 0; db < 4; ++db) o[4 * rb + db] = mfma_bf16(av[db], l, o[4 * rb + db]);
  }
}

template <int QDT, int KV>
__global__ __launch_bounds__(512, 1) void prefill_ws_kernel(PrefillArgs a) {
  // bf16 queries against FP8 keys: each row split exactly into two FP8 parts
  // (its own power-of-two scale), two products per K fragment.
  constexpr bool QSPLIT = QDT == kBF16 && KV == kFP8;
  constexpr int NRB = kPipeRows / 16;  // row blocks of the workgroup
  constexpr int TK = kWsKeys<KV>;      // keys per tile
  __shared__ PipeSmem<KV, NRB> sm;
  const int g = blockIdx.y, b = blockIdx.z;
  const int tok0 = a.cu_q[b];
  const int lq = min(a.cu_q[b + 1] - tok0, a.max_q_len);
  const int lk = min(a.cu_k[b + 1] - a.cu_k[b], a.max_kv_len);
  const int t_lo = (gridDim.x - 1 - blockIdx.x) * a.tile_tokens;  // longest tiles first
  if (t_lo >= lq) return;
  const int t_hi = min(t_lo + a.tile_tokens, lq);
  const int k_hi = lk - lq + t_hi;
  const int rows = a.r * (t_hi - t_lo);
  if (k_hi <= 0) {
    // No key is visible to any row of the tile (a sequence with fewer keys than
    // queries breaks the caller contract): zero rows and lse = -inf, as the
    // bf16-query kernel gives, without reading the block table.  Uniform exit,
    // before any barrier.
    for (int i = threadIdx.x; i < rows * (kHeadDim / 4); i += blockDim.x) {
      const int rr = i / (kHeadDim / 4), c = i - rr * (kHeadDim / 4);
      const int t2 = rr / a.r;
      const int64_t row = (tok0 + t_lo + t2) * (int64_t)a.hq + g * a.r + rr - t2 * a.r;
      *reinterpret_cast<uint2*>(a.out + row * kHeadDim + 4 * c) = make_uint2(0u, 0u);
      if (c == 0 && a.lse) a.lse[row] = kNegInf;
    }
    return;
  }

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int n = lane & 15;
  const int32_t* bt_row = a.kv.bt + (int64_t)b * a.kv.bt_stride;
  const int T = (k_hi + TK - 1) / TK;
  constexpr unsigned kTile = PipeSmem<KV, NRB>::kTile;

  if (w < 4) {
    // ---- scores and softmax of row blocks 2w, 2w + 1; all tile copies ----
    // The four softmax waves copy 16 rows each of every K and V tile, so the
    // PV waves carry no copies, scalar loads or copy waits.
    TileCopy<KV, 4> cp(a.kv, bt_row, g, k_hi);
    int pg0 = cp.page(0), pg1 = T > 1 ? cp.page(1) : 0, pg2 = T > 2 ? cp.page(2) : 0;
    const unsigned kbuf = (unsigned)(uintptr_t)(lds_t*)&sm.k[0][0];
    const unsigned vbuf = (unsigned)(uintptr_t)(lds_t*)&sm.v[0][0];
    constexpr int kDma = TileCopy<KV, 4>::kDma;
    // Prologue copies: K and V of tiles 0 and 1, K of tile 2.
    cp.issue(0, pg0, false, kbuf);
    cp.issue(0, pg0, true, vbuf);
    if (T > 1) {
      cp.issue(1, pg1, false, kbuf + kTile);
      cp.issue(1, pg1, true, vbuf + kTile);
    }
    if (T > 2) cp.issue(2, pg2, false, kbuf + 2 * kTile);
    int pg3 = T > 3 ? cp.page(3) : 0;
    // Iteration i's wait, barrier and copies (K of tile i + 3, V of tile i + 2).
    auto open_step = [&](int i) {
      if (i + 2 < T)
        wait_vmcnt<2 * kDma>();
      else if (i + 1 < T)
        wait_vmcnt<kDma>();
      else
        wait_vmcnt<0>();
      barrier_publish();  // tile i's probabilities are visible; iteration i - 1's reads are done
      if (i + 3 < T) cp.issue(i + 3, pg3, false, kbuf + ((i + 3) % kPipeStages) * kTile);
      if (i + 2 < T) cp.issue(i + 2, pg2, true, vbuf + ((i + 2) % kPipeStages) * kTile);
      pg2 = pg3;
      pg3 = i + 4 < T ? cp.page(i + 4) : 0;
    };
    QFragT<KV> qf[2];
    int klim[2];
    float c2 = a.c2_base * load_scale(a.q_ds) * load_scale(a.kv.k_ds);
    const bool flip = c2 < 0.f;  // keep c2 positive: negate the queries instead (the sign bit of every element)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rr = 16 * (2 * w + j) + n;
      const bool ok = rr < rows;
      const int t2 = ok ? rr / a.r : 0;
      load_q<QDT, KV>(qf[j], a.q, tok0 + t_lo + t2, a.hq, g * a.r + (ok ? rr - t2 * a.r : 0), ok);
      klim[j] = ok ? min(lk - lq + t_lo + t2, k_hi - 1) : -1;
      if (flip) {
        if constexpr (KV == kFP8) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              qf[j].hi[h][i] ^= (int)0x80808080u;
              if constexpr (QSPLIT) qf[j].lo[h][i] ^= (int)0x80808080u;
            }
        } else {
#pragma unroll
          for (int ks = 0; ks < 8; ++ks)
            qf[j].q[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(i32x4, qf[j].q[ks]) ^ (int)0x80008000u);
        }
      }
    }
    c2 = fmaxf(fabsf(c2), 1e-30f);  // a zero scale: every score counts the same
    float c2row[2] = {c2, c2};       // per row block: times the split's row scale (this lane's row)
    if constexpr (QSPLIT) {
#pragma unroll
      for (int j = 0; j < 2; ++j) c2row[j] *= qf[j].rscale;
    }
    const int min_lim = min(lk - lq + t_lo, k_hi - 1);  // tiles ending at or below it need no mask
    RowStat rs[2];
    f32x4 lsum[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      rs[j].init();
      lsum[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto tile = [&](int j, auto masked) {
      f32x4 s[2][TK / 16];
      const lds_t* kt = (const lds_t*)&sm.k[0][0] + (j % kPipeStages) * kTile;
      WsExchange<KV, NRB>& x = sm.x[j & 1];
      if constexpr (KV == kFP8) {
        tile_scores_rows<2, 4, QSPLIT>(kt, qf, s);
#pragma unroll
        for (int r = 0; r < 2; ++r)
          softmax_ws<decltype(masked)::value>(rs[r], lsum[r], s[r], c2row[r], klim[r] - TK * j, x, 2 * w + r);
      } else {
        tile_scores_rows_bf16<2, 2>(kt, qf, s);
#pragma unroll
        for (int r = 0; r < 2; ++r)
          softmax_ws_bf16<decltype(masked)::value>(rs[r], lsum[r], s[r], c2row[r], klim[r] - TK * j, x, 2 * w + r);
      }
    };
    wait_vmcnt<0>();
    barrier();
    if (TK - 1 > min_lim)
      tile(0, std::true_type{});
    else
      tile(0, std::false_type{});
    // Tiles needing the mask form a suffix, so two loops with one body each.
    int i = 0;
    for (; i + 1 < T && TK * (i + 1) + TK - 1 <= min_lim; ++i) {
      open_step(i);
      tile(i + 1, std::false_type{});
    }
    for (; i + 1 < T; ++i) {
      open_step(i);
      tile(i + 1, std::true_type{});
    }
    open_step(T - 1);
    // Row sums for the PV waves, through the buffer nobody reads in the last
    // iteration, and the rows' log-sum-exp.
    WsExchange<KV, NRB>& xe = sm.x[T & 1];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (lane < 16) xe.row[16 * (2 * w + j) + lane] = lsum[j][0];
      const int rr = 16 * (2 * w + j) + n;
      if (rr < rows && (lane >> 4) == 0 && a.lse) {
        const int t2 = rr / a.r;
        const float lrow = lsum[j][0];
        a.lse[(tok0 + t_lo + t2) * (int64_t)a.hq + g * a.r + rr - t2 * a.r] =
            lrow > 0.f ? (rs[j].m + log2f(lrow)) * kLn2 : kNegInf;
      }
    }
    barrier_publish();
  } else {
    // ---- PV of head dims 64 (w - 4) .. of all rows ----
    const int d = w - 4;
    f32x4 o[4 * NRB];
#pragma unroll
    for (int k = 0; k < 4 * NRB; ++k) o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    barrier();
    for (int i = 0; i < T; ++i) {
      barrier_publish();  // V of tile i has landed (the copying waves waited for it); P(i) is visible
      const lds_t* vt = (const lds_t*)&sm.v[0][0] + (i % kPipeStages) * kTile;
      if constexpr (KV == kFP8)
        pv_ws<NRB>(o, vt, sm.x[i & 1], d);
      else
        pv_ws_bf16<NRB>(o, vt, sm.x[i & 1], d);
    }
    barrier_publish();
    const WsExchange<KV, NRB>& xe = sm.x[T & 1];
    const float vds = load_scale(a.kv.v_ds);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int rr = 16 * rb + n;
      if (rr < rows) {
        const int t2 = rr / a.r;
        const float l = xe.row[rr];
        const float scale = l > 0.f ? vds / l : 0.f;
        uint16_t* row_base = a.out + ((tok0 + t_lo + t2) * (int64_t)a.hq + g * a.r + rr - t2 * a.r) * kHeadDim;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const f32x4 v = o[4 * rb + db];
          *reinterpret_cast<uint2*>(row_base + 64 * d + 16 * db + 4 * (lane >> 4)) =
              make_uint2(pack_bf16x2(v[0] * scale, v[1] * scale), pack_bf16x2(v[2] * scale, v[3] * scale));
        }
      }
    }
  }
}

// Every pair of encodings runs the 128-row kernel.
int prefill_tile_tokens(int, int, int r) { return r > 0 ? kPipeRows / r : 0; }

hipError_t launch_prefill(const PrefillArgs& a, int q_dtype, int kv_dtype, int q_tiles, hipStream_t s) {
  dim3 grid(q_tiles, a.kv.num_kv_heads, a.num_seqs);
  if (q_dtype == kFP8 && kv_dtype == kFP8)
    hipLaunchKernelGGL((prefill_ws_kernel<kFP8, kFP8>), grid, dim3(512), 0, s, a);
  else if (q_dtype == kBF16 && kv_dtype == kBF16)
    hipLaunchKernelGGL((prefill_ws_kernel<kBF16, kBF16>), grid, dim3(512), 0, s, a);
  else if (q_dtype == kBF16 && kv_dtype == kFP8)
    hipLaunchKernelGGL((prefill_ws_kernel<kBF16, kFP8>), grid, dim3(512), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pga
