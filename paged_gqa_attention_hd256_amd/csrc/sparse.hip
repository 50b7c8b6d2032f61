// Selected-token paged attention (vLLM PR #62590, "Tune sparse GQA prefill
// profile on gfx942 and gfx950": Overview; Earlier results: 2,051 selected
// tokens per row at head size 256, BF16 or FP8 K/V).
//
// Work unit: one wave per (query token, kv head, block of 16 query heads of
// that kv group).  The waves of a workgroup are independent -- each owns its
// LDS region and never waits for another -- so the gather of one wave overlaps
// the arithmetic of the others without workgroup barriers.  When the kv head
// count divides the XCD count, every workgroup of an XCD works on one kv head
// (head_job), so an XCD's L2 holds one head's rows.
//
// Per wave, the selected entries are processed in chunks: the wave first
// translates a chunk of the row's index list into physical token rows of the
// pool (index -> block-table page -> page * page_size + slot; negative for an
// entry that selects nothing) and keeps that table in LDS (the chunk's indices
// were requested before the previous chunk's copies); then it streams 16-key
// tiles of K and V through two LDS stages each by 16-byte DMA whose per-lane
// source comes from the table, software pipelined: the scores and softmax of
// tile i + 1 run between the requests and the products of tile i's PV.
// Because the table is read from LDS, no vector-memory load sits between the
// DMA instructions and their counter can be waited on exactly.
#include <algorithm>
#include <type_traits>

#include "causal_stream.h"

namespace pga {

template <int KV>
struct SparseCfg {
  using G = TileGeom<KV>;
  // Independent waves, 16-key tiles of K and V in two stages each plus the
  // index table per wave: FP8 runs two waves per SIMD (8 x 18 KB of LDS: a
  // 512-entry table), BF16 one (4 x 36 KB: a 1,024-entry table).  Measured
  // on the same-index gather: two waves per SIMD gather FP8 rows about 30 %
  // faster than one, and BF16 rows (twice the bytes per tile) slower.
  static constexpr int kWaves = (KV == kFP8) ? 8 : 4;
  static constexpr int kWavesPerSimd = kWaves / 4;
  static constexpr int kTileKeys = 16;
  static constexpr int kBlocks = kTileKeys / 16;  // 16-key MFMA blocks per tile
  static constexpr int kTable = (KV == kFP8) ? 512 : 1024;                       // index-list chunk per wave
  static constexpr int kTileBytes = G::template tile_bytes<kTileKeys>();         // K or V of one tile
  static constexpr int kWaveBytes = 4 * kTileBytes + 4 * kTable;                 // 2 buffers x (K, V) + table
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

// Online-softmax step of one tile that leaves the accumulators alone: the
// scores become probabilities in place and the row maximum and sum move on;
// the returned factor is what the accumulators must be multiplied by before
// this tile's product is added (1 unless the reference maximum moved; `grow`
// is set, wave-uniformly, when some row's did).  No branch, so it can run
// between the products of the previous tile.  The reference maximum moves
// only when a tile's maximum exceeds it by more than kRescaleLog2.
template <int NMB, class Vis>
__device__ __forceinline__ float softmax_deferred(float& m, float& l, f32x4 (&s)[NMB], float c2, Vis visible,
                                                  bool& grow) {
  const int gq = lane_id() >> 4;
  float mt = kNegInf;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = visible(mb * 16 + 4 * gq + i) ? s[mb][i] * c2 : kNegInf;
      s[mb][i] = x;
      mt = fmaxf(mt, x);
    }
  mt = group4_max(mt);
  grow = __builtin_amdgcn_ballot_w64(mt > m + kRescaleLog2) != 0;
  const float m_new = grow ? fmaxf(m, mt) : m;
  // 0 when m is -inf and the row now has a key; 1 when its maximum did not move.
  const float alpha = m_new == m ? 1.f : fast_exp2(m - m_new);
  l *= alpha;
  m = m_new;
  const float m_use = m == kNegInf ? 0.f : m;
  float sum = 0.f;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = fast_exp2(s[mb][i] - m_use);
      s[mb][i] = pv;
      sum += pv;
    }
  l += sum;
  return alpha;
}

// DENSE: the pool's token rows are evenly spaced (page stride = page_size x
// token stride, for K and for V; the "NHD" layout), there are at most 2^24
// physical rows, the token strides are below 2^24 bytes and every row of a kv
// head lies within 4 GiB of that head's base.  Then a copy's source is the
// head's base (wave-uniform) plus a 32-bit byte offset formed by one 24-bit
// multiply-add of the table entry (whose bits 24..31, the mask flag among
// them, the multiply ignores) onto the lane's chunk offset, instead of
// splitting the index into page and slot and forming 64-bit products (address
// arithmetic is most of this kernel's vector work).  Other pools take the
// general form.  Waves per SIMD as SparseCfg sets them (two for FP8, one for
// BF16: the LDS holds that many waves' buffers), which also bounds their
// registers.
template <int KV, bool DENSE>
__global__ __launch_bounds__(SparseCfg<KV>::kWaves * 64)
__attribute__((amdgpu_waves_per_eu(SparseCfg<KV>::kWavesPerSimd, SparseCfg<KV>::kWavesPerSimd)))
void sparse_kernel(SparseArgs a) {
  using C = SparseCfg<KV>;
  using G = typename C::G;
  __shared__ __attribute__((aligned(16))) char smem[C::kWaves][C::kWaveBytes];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int n = lane & 15, gq = lane >> 4;
  const int nrb = (a.r + 15) >> 4;                  // 16-row blocks per kv group
  const int S = a.splits;
  // Jobs of one kv head: (token, row block, piece), pieces fastest.
  const HeadJob hj = head_job(blockIdx.x, w, C::kWaves, a.kv.num_kv_heads);
  if (hj.j >= (int64_t)a.num_tokens * nrb * S) return;
  const int g = hj.g;
  const int64_t rowjob = hj.j / S;
  const int sp = (int)(hj.j - rowjob * S);  // piece of the row's index list
  const int tok = (int)(rowjob / nrb);
  const int rb = (int)(rowjob - (int64_t)tok * nrb);
  const int b = seq_of(a.cu_q, a.num_seqs, tok);
  const int lk = a.lens_k[b];

  char* wbase = smem[w];
  lds_t* tiles = (lds_t*)wbase;                                         // [buf][K, V][tile]
  lds_t* table = (lds_t*)(wbase + 4 * C::kTileBytes);                   // int32 [C::kTable]

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
  // Per-lane parts of the DMA source addresses that do not change from tile
  // to tile: the byte offset of the 16-byte chunk this lane copies of its row
  // (swizzled by the row's place in the tile).
  const uint64_t zaddr = (uint64_t)(uintptr_t)g_zero16;
  const uint64_t kb = (uint64_t)(uintptr_t)kbase, vb = (uint64_t)(uintptr_t)vbase;
  const uint32_t kst = (uint32_t)a.kv.k_st, vst = (uint32_t)a.kv.v_st;
  uint32_t co[C::kDmaPerTile];
#pragma unroll
  for (int u = 0; u < C::kDmaPerTile; ++u) {
    const int row = u * C::kRowsPerDma + lane / G::kChunks;
    co[u] = (uint32_t)((lane % G::kChunks) ^ (row & (G::kChunks - 1))) * 16u;
  }

  const int e_end = min((sp + 1) * a.split_len, a.num_selected);
  constexpr int kPer = C::kTable / 64;  // entries per lane
  // The index entries of the chunk at c0 (-1 past the piece).  Each row's
  // list is read exactly once: non-temporal, so it does not displace the K/V
  // rows that other rows of the sequence reuse from L2.
  auto load_indices = [&](int c0, int (&jv)[kPer]) {
    const int cnt = min(C::kTable, e_end - c0);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = lane + 64 * k;
      jv[k] = e < cnt ? __builtin_nontemporal_load(idx_row + c0 + e) : -1;
    }
  };
  int jnext[kPer];
  load_indices(sp * a.split_len, jnext);
  for (int c0 = sp * a.split_len; c0 < e_end; c0 += C::kTable) {
    const int cnt = min(C::kTable, e_end - c0);
    const int ntiles = (cnt + C::kTileKeys - 1) / C::kTileKeys;
    // Translate this chunk's entries (and pad the last tile) into physical
    // rows: its indices were requested a chunk ahead; every block-table entry
    // they need is requested at once, so the chunk's translation waits for one
    // memory round trip rather than two per entry.
    const int nent = ntiles * C::kTileKeys;
    int jv[kPer], pgv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) jv[k] = jnext[k];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = jv[k];
      pgv[k] = (j >= 0 && j < lk) ? bt_row[j >> a.kv.page_shift] : -1;
    }
    // An entry that selects nothing (padding, out of range, the last tile's
    // tail) is stored negative, which masks its key.  On an evenly spaced pool
    // it also carries, in its low 31 bits, the row of the chunk's first valid
    // entry, so its copy reads finite data of the same list (the mask gives it
    // probability 0 exactly) and the copies need no per-lane fallback address;
    // a chunk without any valid entry is skipped.
    int physv[kPer];
    uint64_t anyv = 0;
    int first_valid = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = jv[k], page = pgv[k];
      const bool ok = j >= 0 && j < lk && page >= 0 && page < a.kv.num_pages;
      physv[k] = ok ? page * a.kv.page_size + (j & pmask) : -1;
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
      if (anyv == 0 && m != 0) first_valid = __builtin_amdgcn_readlane(physv[k], __builtin_ctzll(m));
      anyv |= m;
    }
    // The next chunk's indices travel while this chunk's tiles stream: they
    // are requested before the first copy, and first used after the last.
    if (c0 + C::kTable < e_end) load_indices(c0 + C::kTable, jnext);
    if (anyv == 0) continue;  // nothing selected in this chunk (wave-uniform)
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = lane + 64 * k;
      const int ph = physv[k] >= 0 ? physv[k] : (DENSE ? (int)(0x80000000u | (unsigned)first_valid) : -1);
      if (e < nent) lds_store<int>(table + 4 * e, ph);
    }

    // Copies of one operand (K or V) of tile it into stage BUF (a compile-time
    // constant, so the stage's LDS offsets are immediates).
    auto issue = [&](int it, auto buf_c, bool is_v) {
      constexpr int buf = decltype(buf_c)::value;
      // Every table read of the tile first, so their LDS latency is paid once
      // (the copies below are ordered memory operations: no load moves past them).
      int physv[C::kDmaPerTile];
#pragma unroll
      for (int u = 0; u < C::kDmaPerTile; ++u)
        physv[u] = lds_load<int>(table + 4 * (it * C::kTileKeys + u * C::kRowsPerDma + lane / G::kChunks));
#pragma unroll
      for (int u = 0; u < C::kDmaPerTile; ++u) {
        const int row0 = u * C::kRowsPerDma;
        const int phys = physv[u];
        lds_t* dst = tiles + (2 * buf + (is_v ? 1 : 0)) * C::kTileBytes + row0 * G::kRowBytes;
        if constexpr (DENSE) {
          const uint32_t off = __umul24((uint32_t)phys, is_v ? vst : kst) + co[u];
          dma16_off(is_v ? vb : kb, off, (unsigned)(uintptr_t)dst);
        } else {
          const int row = row0 + lane / G::kChunks;
          const int chunk = (lane % G::kChunks) ^ (row & (G::kChunks - 1));
          const int64_t page = phys >> a.kv.page_shift;
          const int slot = phys & pmask;
          const uint64_t src = phys >= 0 ? (uint64_t)(uintptr_t)((is_v ? vbase : kbase) + page * (is_v ? a.kv.v_sp : a.kv.k_sp) +
                                                                 slot * (is_v ? a.kv.v_st : a.kv.k_st) + chunk * 16)
                                         : zaddr;
          dma16((const void*)(uintptr_t)src, dst);
        }
      }
    };
    // Scores and softmax of tile it (K in stage PAR = it & 1); the
    // accumulators are left for the caller to rescale after the previous
    // tile's product.
    auto scores_softmax = [&](int it, auto par_c, f32x4 (&sc)[C::kBlocks], bool& grow) -> float {
      constexpr int par = decltype(par_c)::value;
      tile_scores<KV, C::kBlocks, true>(tiles + (2 * par + 0) * C::kTileBytes, qf, sc);
      const lds_t* tt = table + 4 * (it * C::kTileKeys);
      const i32x4 v0 = lds_load<i32x4>(tt + 4 * (4 * gq));
      i32x4 v1 = v0;
      if constexpr (C::kBlocks == 2) v1 = lds_load<i32x4>(tt + 4 * (16 + 4 * gq));
      return softmax_deferred(st.m, st.l, sc, c2, [&](int key) {
        const int q = key - 4 * gq;  // 0..3 in block 0, 16..19 in block 1
        const int e = q & 3;
        const int v = (q < 16) ? v0[e] : v1[e];
        return v >= 0;
      }, grow);
    };

    // Software pipeline: iteration it computes the scores and softmax of tile
    // it + 1 and the product of tile it, so neither waits on the other's
    // latencies.  K runs two tiles ahead of the product, V one: K(it + 2) goes
    // into the K stage of tile it (its scores were computed an iteration
    // earlier), V(it + 1) into the V stage of tile it - 1.  The loop is
    // unrolled by two so each stage index is a compile-time constant.
    constexpr int D = C::kDmaPerTile;
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    issue(0, Even{}, false);
    issue(0, Even{}, true);
    if (ntiles > 1) {
      issue(1, Odd{}, false);
      wait_vmcnt<2 * D>();  // K(0)
    } else {
      wait_vmcnt<D>();
    }
    f32x4 p[C::kBlocks];
    bool grow;
    scores_softmax(0, Even{}, p, grow);  // the accumulators are still zero
    // One iteration; PAR = it & 1.
    auto step = [&](int it, auto par_c) {
      constexpr int par = decltype(par_c)::value;
      using Same = std::integral_constant<int, par>;
      using Other = std::integral_constant<int, par ^ 1>;
      if (it + 2 < ntiles) {
        issue(it + 2, Same{}, false);
        issue(it + 1, Other{}, true);
        wait_vmcnt<2 * D>();  // K(it + 1) and V(it) have landed
      } else {
        issue(it + 1, Other{}, true);
        wait_vmcnt<D>();
      }
      TilePV<KV, C::kBlocks> pv;
      pv.fetch(tiles + (2 * par + 1) * C::kTileBytes);
      f32x4 pn[C::kBlocks];
      bool gn;
      const float an = scores_softmax(it + 1, Other{}, pn, gn);
      pv.multiply(st, p);
      if (gn) {
#pragma unroll
        for (int d = 0; d < 16; ++d) st.o[d] *= an;
      }
#pragma unroll
      for (int mb = 0; mb < C::kBlocks; ++mb) p[mb] = pn[mb];
    };
    for (int it = 0; it + 1 < ntiles; it += 2) {
      step(it, Even{});
      if (it + 2 < ntiles) step(it + 1, Odd{});
    }
    wait_vmcnt<0>();
    TilePV<KV, C::kBlocks> pv;
    pv.fetch(tiles + (2 * ((ntiles - 1) & 1) + 1) * C::kTileBytes);
    pv.multiply(st, p);
  }

  const float lrow = group4_sum(st.l);
  if (!row_ok) return;
  if (S > 1) {  // a piece of the row: rows over their sums (V code units) and lse, merged later
    const int64_t slot = ((int64_t)tok * a.hq + head) * S + sp;
    const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) {
      const f32x4 v = st.o[mb] * inv;
      if constexpr (KV == kFP8) {
        const f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        *reinterpret_cast<f16x4*>(static_cast<uint16_t*>(a.ws_o) + slot * kHeadDim + 16 * mb + 4 * gq) = h;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.ws_o) + slot * kHeadDim + 16 * mb + 4 * gq) = v;
      }
    }
    if (gq == 0) a.ws_lse[slot] = lrow > 0.f ? (st.m + log2f(lrow)) * kLn2 : kNegInf;
    return;
  }
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

// Log-sum-exp merge of the pieces of each (query token, head) row: one wave
// per row, the lse of up to 64 pieces read one per lane, the rows of 8 pieces
// in flight at a time; pieces with lse = -inf (no visible entry) get weight 0.
template <int KV>
__global__ __launch_bounds__(256) void sparse_merge_kernel(SparseArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // token * hq + head
  if (row >= (int64_t)a.num_tokens * a.hq) return;
  const int lane = lane_id();
  const int S = a.splits;
  const float ls = lane < S ? a.ws_lse[row * S + lane] : kNegInf;
  const float mx = wave_max(ls);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != kNegInf) {
    const float wgt = ls == kNegInf ? 0.f : __expf(ls - mx);
    wsum = wave_sum(wgt);
    auto part = [&](int sl) -> f32x4 {
      const int64_t off = (row * S + sl) * kHeadDim + 4 * lane;
      if constexpr (KV == kFP8) {
        const f16x4 h = *reinterpret_cast<const f16x4*>(static_cast<const uint16_t*>(a.ws_o) + off);
        return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
      } else {
        return *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.ws_o) + off);
      }
    };
    for (int s0 = 0; s0 < S; s0 += 8) {
      f32x4 v[8];
      float wq[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int sk = min(s0 + k, S - 1);
        wq[k] = s0 + k < S ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), min(s0 + k, 63))) : 0.f;
        v[k] = part(sk);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (wq[k] != 0.f) acc += wq[k] * v[k];
    }
  }
  const float inv = wsum > 0.f ? load_scale(a.kv.v_ds) / wsum : 0.f;
  uint16_t* op = a.out + row * kHeadDim + 4 * lane;
  *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
  if (lane == 0 && a.lse) a.lse[row] = wsum > 0.f ? mx + logf(wsum) : kNegInf;
}

hipError_t launch_sparse(const SparseArgs& a, int kv_dtype, hipStream_t s) {
  const int nrb = (a.r + 15) / 16;
  const int W = kv_dtype == kFP8 ? SparseCfg<kFP8>::kWaves : SparseCfg<kBF16>::kWaves;  // waves per workgroup
  const dim3 grid((unsigned)head_job_grid((int64_t)a.num_tokens * nrb * a.splits, W, a.kv.num_kv_heads));
  const KvArgs& kv = a.kv;
  const int64_t rows = (int64_t)kv.num_pages * kv.page_size;
  const int64_t row_bytes = kv_dtype == kFP8 ? 256 : 512;
  const bool dense = kv.k_sp == (int64_t)kv.page_size * kv.k_st && kv.v_sp == (int64_t)kv.page_size * kv.v_st &&
                     kv.k_st > 0 && kv.v_st > 0 && kv.k_st < (int64_t(1) << 24) && kv.v_st < (int64_t(1) << 24) &&
                     rows <= (int64_t(1) << 24) &&
                     (rows - 1) * std::max(kv.k_st, kv.v_st) + row_bytes <= (int64_t(1) << 32);
  if (kv_dtype == kFP8) {
    if (dense)
      hipLaunchKernelGGL((sparse_kernel<kFP8, true>), grid, dim3(W * 64), 0, s, a);
    else
      hipLaunchKernelGGL((sparse_kernel<kFP8, false>), grid, dim3(W * 64), 0, s, a);
  } else {
    if (dense)
      hipLaunchKernelGGL((sparse_kernel<kBF16, true>), grid, dim3(W * 64), 0, s, a);
    else
      hipLaunchKernelGGL((sparse_kernel<kBF16, false>), grid, dim3(W * 64), 0, s, a);
  }
  if (a.splits > 1) {
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const dim3 mgrid((unsigned)(((int64_t)a.num_tokens * a.hq + 3) / 4));
    if (kv_dtype == kFP8)
      hipLaunchKernelGGL(sparse_merge_kernel<kFP8>, mgrid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(sparse_merge_kernel<kBF16>, mgrid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pga
