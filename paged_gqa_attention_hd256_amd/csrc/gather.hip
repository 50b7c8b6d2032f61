// Same-index gather of the selected-token call's K and V rows: the practical
// bandwidth roof of sparse_paged_attn on a given selection (measurement only).
//
// The sparse kernel's cost on the pages' workload (vLLM PR #62590, "Tune sparse
// GQA prefill profile on gfx942 and gfx950": Overview, Measured results -- 2,051
// selected rows per query row gathered from a pool that the caches hold) is
// the gather, not the arithmetic.  This kernel moves exactly the rows that
// call attends, through the same translation (index -> block-table page ->
// physical row) and the same 16-byte global->LDS copies into the same per-wave
// tiles, and does nothing with them but sum their 32-bit words, so its rate is
// what the gather alone reaches on this part.
//
// Work unit: one wave per (query row, kv head, piece of the row's list) -- the
// rows that every 16-head block of that kv group reads once each in the
// attention kernel, in the pieces that kernel splits a short batch's lists
// into (the pieces' sums are added atomically into a zeroed output).  Waves are
// independent (no barriers).  Per chunk of up to 1,024 list entries the wave
// translates the entries into a table of physical rows in LDS (negative for an
// entry that selects nothing, carrying the chunk's first valid row so its copy
// stays in bounds), then streams tiles of K and V rows through two LDS stages
// each on the attention kernel's schedule (K two tiles ahead of V's use, V
// one).  Only the pool's evenly spaced layout is handled (page stride = page
// size x token stride for K and for V), the one the benchmarked selections
// use.
//
// Output: out[row][kv head][w] = sum over the row's valid entries j of the
// 32-bit words w of K_j and of V_j of that head (row bytes / 4 words), mod
// 2^32 -- an exact, order-independent checksum.
#include <type_traits>

#include "causal_stream.h"

namespace pga {

// The sparse kernel's shape: waves per CU, rows per stage, table entries.
template <int KV>
struct GatherCfg {
  using G = TileGeom<KV>;
  static constexpr int kWaves = (KV == kFP8) ? 8 : 4;
  static constexpr int kWavesPerSimd = kWaves / 4;
  static constexpr int kTileKeys = 16;                                       // rows of one stage
  static constexpr int kTileBytes = G::template tile_bytes<kTileKeys>();     // 4 KB (FP8) / 8 KB (BF16)
  static constexpr int kTable = (KV == kFP8) ? 512 : 1024;                   // list entries translated at a time
  static constexpr int kWaveBytes = 4 * kTileBytes + 4 * kTable;              // 2 stages x (K, V) + table
  static constexpr int kRowsPerDma = 1024 / G::kRowBytes;                    // 4 (FP8) or 2 (BF16)
  static constexpr int kDma = kTileKeys / kRowsPerDma;                       // copies per operand and tile: 8
};

// Sequence of a query row: the last b with cu_q[b] <= tok.
__device__ __forceinline__ int gather_seq_of(const int32_t* cu_q, int num_seqs, int tok) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int KV>
__global__ __launch_bounds__(GatherCfg<KV>::kWaves * 64)
__attribute__((amdgpu_waves_per_eu(GatherCfg<KV>::kWavesPerSimd, GatherCfg<KV>::kWavesPerSimd)))
void gather_sum_kernel(GatherArgs a) {
  using C = GatherCfg<KV>;
  using G = typename C::G;
  __shared__ __attribute__((aligned(16))) char smem[C::kWaves][C::kWaveBytes];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int hkv = a.kv.num_kv_heads;
  const int S = a.splits;
  // Jobs of one kv head: (row, piece), pieces fastest; the heads spread over
  // the XCDs as in the sparse kernel.
  const HeadJob hj = head_job(blockIdx.x, w, C::kWaves, hkv);
  if (hj.j >= (int64_t)a.num_tokens * S) return;
  const int g = hj.g;
  const int tok = (int)(hj.j / S);
  const int sp = (int)(hj.j - (int64_t)tok * S);
  const int64_t rowjob = (int64_t)tok * hkv + g;
  const int b = gather_seq_of(a.cu_q, a.num_seqs, tok);
  const int lk = a.lens_k[b];
  const int32_t* bt_row = a.kv.bt + (int64_t)b * a.kv.bt_stride;
  const int32_t* idx_row = a.idx + (int64_t)tok * a.idx_stride;
  const int pmask = a.kv.page_size - 1;

  lds_t* tiles = (lds_t*)smem[w];                          // [stage][K, V][tile]
  lds_t* table = (lds_t*)(smem[w] + 4 * C::kTileBytes);   // int32 [kTable]
  const unsigned tiles_addr = (unsigned)(uintptr_t)tiles;
  // Per-wave uniform bases (this kv head) and the lane's fixed chunk offset.
  const uint64_t kbase = (uint64_t)(uintptr_t)(a.kv.k + g * a.kv.k_sh);
  const uint64_t vbase = (uint64_t)(uintptr_t)(a.kv.v + g * a.kv.v_sh);
  const unsigned kst = (unsigned)a.kv.k_st, vst = (unsigned)a.kv.v_st;
  const unsigned chunk_off = (unsigned)(lane % G::kChunks) * 16u;
  const int row_in_dma = lane / G::kChunks;

  u32x4 acc = {0u, 0u, 0u, 0u};
  const int e_end = min((sp + 1) * a.split_len, a.num_selected);
  for (int c0 = sp * a.split_len; c0 < e_end; c0 += C::kTable) {
    const int cnt = min(C::kTable, e_end - c0);
    const int ntiles = (cnt + C::kTileKeys - 1) / C::kTileKeys;
    // Translate: every index of the lane, then every block-table entry.
    constexpr int kPer = C::kTable / 64;
    int jv[kPer], pv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = lane + 64 * k;
      jv[k] = e < cnt ? __builtin_nontemporal_load(idx_row + c0 + e) : -1;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = jv[k];
      pv[k] = (j >= 0 && j < lk) ? bt_row[j >> a.kv.page_shift] : -1;
    }
    uint64_t any = 0;
    int first_valid = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = jv[k], page = pv[k];
      const bool ok = j >= 0 && j < lk && page >= 0 && page < a.kv.num_pages;
      pv[k] = ok ? page * a.kv.page_size + (j & pmask) : -1;
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
      if (any == 0 && m != 0) first_valid = __builtin_amdgcn_readlane(pv[k], __builtin_ctzll(m));
      any |= m;
    }
    if (any == 0) continue;  // nothing selected in this chunk (wave-uniform)
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = lane + 64 * k;
      const int ph = pv[k] >= 0 ? pv[k] : (int)(0x80000000u | (unsigned)first_valid);
      if (e < ntiles * C::kTileKeys) lds_store<int>(table + 4 * e, ph);
    }
    // Copies of one operand (K or V) of tile `it` into stage ST (a
    // compile-time constant).  A row's source offset is one 24-bit
    // multiply-add of the table entry (bits 24..31, the mask flag among them,
    // are ignored by the multiply).
    auto issue = [&](int it, auto st_c, bool is_v) {
      constexpr int st = decltype(st_c)::value;
      int ph[C::kDma];
#pragma unroll
      for (int u = 0; u < C::kDma; ++u)
        ph[u] = lds_load<int>(table + 4 * (it * C::kTileKeys + u * C::kRowsPerDma + row_in_dma));
#pragma unroll
      for (int u = 0; u < C::kDma; ++u) {
        const unsigned dst = tiles_addr + (2 * st + (is_v ? 1 : 0)) * C::kTileBytes + u * 1024;
        dma16_off(is_v ? vbase : kbase, __umul24((unsigned)ph[u], is_v ? vst : kst) + chunk_off, dst);
      }
    };
    // Add this lane's chunk of its valid rows of one operand of tile `it`
    // (stage ST): every DMA lane wrote its 16 bytes at 16 * lane of its 1 KB
    // block, so each lane reads back exactly what it copied.
    // Every read is issued before any sum, and the mask is applied by an AND,
    // so no read waits behind a branch on the previous one.
    auto sum = [&](int it, auto st_c, bool is_v) {
      constexpr int st = decltype(st_c)::value;
      int ph[C::kDma];
      u32x4 x[C::kDma];
#pragma unroll
      for (int u = 0; u < C::kDma; ++u) {
        ph[u] = lds_load<int>(table + 4 * (it * C::kTileKeys + u * C::kRowsPerDma + row_in_dma));
        x[u] = lds_load<u32x4>(tiles + (2 * st + (is_v ? 1 : 0)) * C::kTileBytes + u * 1024 + 16 * lane);
      }
#pragma unroll
      for (int u = 0; u < C::kDma; ++u) {
        const unsigned m = ph[u] >= 0 ? ~0u : 0u;
        acc += x[u] & u32x4{m, m, m, m};
      }
    };
    // The stage's LDS reads are complete before a later copy refills it.
    auto reads_done = [] {
      __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
      asm volatile("" ::: "memory");
    };
    // The attention kernel's copy schedule: K two tiles ahead of V's use, V
    // one; iteration it takes K(it + 1) and V(it) (where that kernel computes
    // the scores of tile it + 1 and the product of tile it).  Unrolled by two
    // so each stage is a compile-time constant.
    constexpr int D = C::kDma;  // copies per operand and tile
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
    sum(0, Even{}, false);
    reads_done();
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
      sum(it, Same{}, true);
      sum(it + 1, Other{}, false);
      reads_done();
    };
    for (int it = 0; it + 1 < ntiles; it += 2) {
      step(it, Even{});
      if (it + 2 < ntiles) step(it + 1, Odd{});
    }
    wait_vmcnt<0>();
    if ((ntiles - 1) & 1)
      sum(ntiles - 1, Odd{}, true);
    else
      sum(ntiles - 1, Even{}, true);
    reads_done();
  }
  // Lanes with the same chunk hold the same words of different rows.
#pragma unroll
  for (int off = G::kChunks; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += (unsigned)__shfl_xor((int)acc[i], off);
  }
  if (lane < G::kChunks) {
    uint32_t* o = a.out + rowjob * (G::kRowBytes / 4) + 4 * lane;
    if (S == 1) {
      *reinterpret_cast<u32x4*>(o) = acc;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(o + i, acc[i]);
    }
  }
}

__global__ __launch_bounds__(256) void gather_zero_kernel(uint32_t* out, int64_t words) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < words) out[i] = 0u;
}

hipError_t launch_gather_sum(const GatherArgs& a, int kv_dtype, hipStream_t s) {
  const int W = kv_dtype == kFP8 ? GatherCfg<kFP8>::kWaves : GatherCfg<kBF16>::kWaves;
  if (a.splits > 1) {
    const int64_t words = (int64_t)a.num_tokens * a.kv.num_kv_heads * ((kv_dtype == kFP8 ? 256 : 512) / 4);
    hipLaunchKernelGGL(gather_zero_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, a.out, words);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)head_job_grid((int64_t)a.num_tokens * a.splits, W, a.kv.num_kv_heads));
  if (kv_dtype == kFP8)
    hipLaunchKernelGGL(gather_sum_kernel<kFP8>, grid, dim3(W * 64), 0, s, a);
  else
    hipLaunchKernelGGL(gather_sum_kernel<kBF16>, grid, dim3(W * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pga
