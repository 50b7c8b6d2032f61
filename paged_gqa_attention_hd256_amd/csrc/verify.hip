// Speculative-verify attention with balanced split-KV and a separate
// log-sum-exp merge kernel.
//
// All r * Lq_b query rows of a kv group (token-major: row = t * r + h) sit in
// one workgroup, so every KV page is fetched from HBM once for all
// speculative tokens of the group -- the reuse SGLang PR #36330 adds
// (Motivation; Modifications: BLOCK_M = 16 x BLOCK_Q).
//
// Work split.  The 64-key tiles of every (sequence, kv head) unit, each unit
// optionally cut into segments of at most kv_split_tokens keys, are laid end to
// end, each segment preceded by a few empty positions that stand for the cost
// of starting it; a persistent grid of P workgroups takes equal contiguous runs
// of that list (stream-K).  A run that covers a whole single-segment unit
// writes the bf16 output directly; any other piece (segment sigma, workgroup w)
// writes its partial output, already divided by its row sums, and
// natural-log lse to workspace slot sigma + w.  Pieces are ordered in both
// sigma and w, so that slot is unique, and there are at most (#segments + P)
// of them.  The merge kernel combines each row's pieces with weights
// exp(lse - max lse).  This replaces a fixed segment count, which on a batch
// of uneven lengths leaves a nearly empty second round of workgroups
// (Modifications: segments chosen from CU parallelism and per-segment work).
//
// Small calls (static_tiles > 0: at most kVerifyStaticMaxTiles tiles over all
// units by the host bounds) skip the plan: workgroup w takes tile w % P of
// unit w / P (P = static_tiles, the host bound of a unit's tiles) and writes
// its piece to slot w, or the output when it is the unit's only tile.  Its
// first reads (the lengths and each wave's block-table entry, taken at the
// host bound) then go out together, one memory round trip before the copies
// instead of a plan scan before them.
#include <type_traits>

#include "causal_stream.h"

namespace pga {

constexpr int kMinTilesPerWg = kVerifyMinTilesPerWg;  // shortest run a workgroup takes (in plan units)
// Plan units charged for starting a piece of work: a workgroup that begins a
// second piece reloads its queries, refills its pipeline and writes a partial
// result, which costs about as much as streaming this many tiles.  Each
// segment is preceded by this many units without keys in the flattened list.
constexpr int kSegStartCost = kVerifySegStartCost;

// Per-sequence work of the plan, per kv head: 64-key tiles, segments, and the
// length in the flattened list (tiles plus the start cost of each segment).
struct SeqWork {
  int tiles, segs, span;
};
__device__ __forceinline__ SeqWork seq_work_of(const VerifyArgs& a, int lq, int lk) {
  lq = min(lq, a.max_q_len);
  lk = min(lk, a.max_kv_len);
  SeqWork s;
  s.tiles = (lq > 0 && lk > 0) ? (lk + 63) >> 6 : 0;
  s.segs = s.tiles > 0 ? (s.tiles + a.seg_tiles - 1) / a.seg_tiles : 0;
  s.span = s.tiles + kSegStartCost * s.segs;
  return s;
}
// Uniform b: scalar loads.
__device__ __forceinline__ SeqWork seq_work(const VerifyArgs& a, int b) {
  return seq_work_of(a, scalar_load(a.cu_q + b + 1) - scalar_load(a.cu_q + b), scalar_load(a.lens_k + b));
}
// Per-lane b (out of range gives no work).
__device__ __forceinline__ SeqWork seq_work_lane(const VerifyArgs& a, int b) {
  if (b >= a.num_seqs) return SeqWork{0, 0, 0};
  return seq_work_of(a, a.cu_q[b + 1] - a.cu_q[b], a.lens_k[b]);
}

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Plan of one call, identical in every workgroup: the total length of the
// flattened list, its length per workgroup, and the list / segment prefix (per
// kv head) of sequence `target_b`, or of the sequence holding list position
// `target_t` when target_b < 0.
// Called by a whole wave.
struct PlanPos {
  int total, tpw, b, tile_prefix, seg_prefix;
};
__device__ PlanPos plan_scan(const VerifyArgs& a, int num_wg, int target_t, int target_b) {
  const int lane = lane_id();
  const int hkv = a.kv.num_kv_heads;
  int tot = 0;
  for (int c = 0; c < a.num_seqs; c += 64) tot += __shfl(wave_incl_scan(seq_work_lane(a, c + lane).span), 63);
  PlanPos p;
  p.total = tot * hkv;
  p.tpw = max(kMinTilesPerWg, (p.total + num_wg - 1) / num_wg);
  p.b = -1;
  p.tile_prefix = p.seg_prefix = 0;
  int ts = 0, ss = 0;
  for (int c = 0; c < a.num_seqs; c += 64) {
    const int b = c + lane;
    const SeqWork s = seq_work_lane(a, b);
    const int it = wave_incl_scan(s.span), is = wave_incl_scan(s.segs);
    bool hit;
    if (target_b >= 0)
      hit = (b == target_b);
    else
      hit = s.span > 0 && (ts + it - s.span) * hkv <= target_t && target_t < (ts + it) * hkv;
    const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
    if (m) {
      const int src = __builtin_ctzll(m);
      p.b = c + src;
      p.tile_prefix = ts + __shfl(it - s.span, src);
      p.seg_prefix = ss + __shfl(is - s.segs, src);
      break;
    }
    ts += __shfl(it, 63);
    ss += __shfl(is, 63);
  }
  return p;
}

// One piece: keys [k_lo, k_hi) of kv head g of sequence b (tok0 = its first
// query token, lq / lk its clamped lengths; `first`: the page ids of the
// range's first two tiles for this wave).  A direct piece writes the bf16
// output and lse; any other writes its rows divided by their sums (V code
// units) and their natural-log lse to workspace slot `slot`.
template <int KV>
__device__ __forceinline__ void verify_piece(const VerifyArgs& a, CausalSmem<KV, 4>& sm, int b, int g, int tok0,
                                             int lq, int lk, int k_lo, int k_hi, int2 first, bool direct,
                                             int64_t slot) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int n = lane & 15, gq = lane >> 4;
  const float c2 = a.c2_base * load_scale(a.q_ds) * load_scale(a.kv.k_ds);
  const float vds = load_scale(a.kv.v_ds);
  const int rows = min(a.r * lq, a.rows_cap);
  const int rho = 16 * w + n;  // this lane's softmax row
  const bool row_ok = rho < rows;
  const int t = row_ok ? rho / a.r : 0;
  const int head = g * a.r + (row_ok ? rho - t * a.r : 0);
  const int64_t tok = tok0 + t;
  const bool live = 16 * w < rows;
  const int32_t* bt_row = a.kv.bt + (int64_t)b * a.kv.bt_stride;
  QFragT<KV> qf;
  load_q<kBF16, KV>(qf, a.q, tok, a.hq, head, row_ok);
  const int klim = row_ok ? min(lk - lq + t, k_hi - 1) : -1;
  const int min_lim = min(lk - lq, k_hi - 1);
  RowStat rs;
  rs.init();
  f32x4 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
  stream_keys(sm, a.kv, bt_row, g, k_lo, k_hi, first,
              SplitTile<kBF16, KV, 4>{qf, c2 * qf.rscale, klim, min_lim, live, rs, o, lsum, sm.x});
  const float lrow = finish_rows(lsum, live, sm.x);
  if (row_ok && gq == 0) {
    const float lse = lrow > 0.f ? (rs.m + log2f(lrow)) * kLn2 : kNegInf;
    if (!direct)
      a.ws_lse[slot * a.rows_cap + rho] = lse;
    else if (a.lse)
      a.lse[tok * a.hq + head] = lse;
  }
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int rr = 16 * rb + n;
    if (rr < rows) {
      const float l = sm.x.row[rr];
      const float inv = l > 0.f ? vds / l : 0.f;
      if (direct) {
        const int t2 = rr / a.r;
        store_share_bf16<4>(o, rb, inv, a.out + ((tok0 + t2) * (int64_t)a.hq + g * a.r + rr - t2 * a.r) * kHeadDim);
      } else if constexpr (KV == kFP8) {
        store_share_f16<4>(o, rb, l > 0.f ? 1.f / l : 0.f,
                          static_cast<uint16_t*>(a.ws_o) + (slot * a.rows_cap + rr) * kHeadDim);
      } else {
        store_share_f32<4>(o, rb, l > 0.f ? 1.f / l : 0.f,
                          static_cast<float*>(a.ws_o) + (slot * a.rows_cap + rr) * kHeadDim);
      }
    }
  }
}

// The page-gather roof (verify_gather_kernel): the copies of one piece, on
// the same pipeline, only summed.  Each lane adds the 32-bit words of the
// 16-byte chunks it copied itself, of rows holding keys below k_hi (the last
// tile's rows past it repeat key k_hi - 1).
template <int KV>
struct SumTile {
  using G = TileGeom<KV>;
  static constexpr int kRowsPerWave = 16;                       // 64 keys over 4 waves
  static constexpr int kRowsPerDma = 1024 / G::kRowBytes;
  static constexpr int kDma = kRowsPerWave / kRowsPerDma;
  u32x4* acc;
  int k_hi;
  __device__ __forceinline__ void add(const lds_t* t, int tb) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = lane_id();
    u32x4 x[kDma];
#pragma unroll
    for (int u = 0; u < kDma; ++u)
      x[u] = lds_load<u32x4>(t + (kRowsPerWave * w + u * kRowsPerDma) * G::kRowBytes + 16 * lane);
#pragma unroll
    for (int u = 0; u < kDma; ++u) {
      const int row = kRowsPerWave * w + u * kRowsPerDma + lane / G::kChunks;
      const unsigned m = tb + row < k_hi ? ~0u : 0u;
      *acc += x[u] & u32x4{m, m, m, m};
    }
  }
  __device__ __forceinline__ void front(const lds_t* kt, int tb) const { add(kt, tb); }
  __device__ __forceinline__ void back(const lds_t* vt, int tb) const { add(vt, tb); }
};

// One piece of the roof: keys [k_lo, k_hi) of kv head g of sequence b, added
// into sum_out[unit] (every word of every copied K and V row, mod 2^32).
template <int KV>
__device__ __forceinline__ void gather_piece(const VerifyArgs& a, CausalSmem<KV, 4>& sm, int b, int g, int k_lo,
                                             int k_hi, int2 first) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  stream_keys(sm, a.kv, a.kv.bt + (int64_t)b * a.kv.bt_stride, g, k_lo, k_hi, first, SumTile<KV>{&acc, k_hi});
  uint32_t t = acc[0] + acc[1] + acc[2] + acc[3];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) t += (uint32_t)__shfl_xor((int)t, off);
  if (lane_id() == 0) atomicAdd(a.sum_out + (int64_t)b * a.kv.num_kv_heads + g, t);
}

// The work split and piece loop shared by the attention kernel and its
// page-gather roof (SUM: the roof, which writes no workspace).
template <int KV, bool SUM>
__device__ __forceinline__ void verify_body(const VerifyArgs& a, CausalSmem<KV, 4>& sm, int* plan_lds) {
  const int wg = blockIdx.x, num_wg = gridDim.x;
  const int hkv = a.kv.num_kv_heads;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();

  if (a.static_tiles > 0) {
    // Tile k of unit u; the wave's block-table entry is read at the host
    // bound of the keys (in the row), with the lengths, and kept only if the
    // wave's first key exists (a wave past the end copies zeros, which its
    // mask gives probability 0).
    const int P = a.static_tiles;
    const int u = wg / P, k = wg - (wg / P) * P;
    const int b = u / hkv, g = u - (u / hkv) * hkv;
    const int32_t* bt_row = a.kv.bt + (int64_t)b * a.kv.bt_stride;
    const int key0 = 64 * k + 16 * w;
    const int pidx = __builtin_amdgcn_readfirstlane(min(key0, a.max_kv_len - 1) >> a.kv.page_shift);
    const int tok0 = scalar_load(a.cu_q + b);
    const int tq1 = scalar_load(a.cu_q + b + 1);
    const int lk_raw = scalar_load(a.lens_k + b);
    const int page = scalar_load(bt_row + pidx);
    const int lq = min(tq1 - tok0, a.max_q_len);
    const int lk = min(lk_raw, a.max_kv_len);
    const int tiles = (lq > 0 && lk > 0) ? (lk + 63) >> 6 : 0;
    if (k >= tiles) return;  // workgroup-uniform
    const int k_hi = min(64 * k + 64, lk);
    if constexpr (SUM)
      gather_piece<KV>(a, sm, b, g, 64 * k, k_hi, int2{key0 < k_hi ? page : -1, 0});
    else
      verify_piece<KV>(a, sm, b, g, tok0, lq, lk, 64 * k, k_hi, int2{key0 < k_hi ? page : -1, 0}, tiles == 1,
                       (int64_t)wg);
    return;
  }

  if (w == 0) {
    // This workgroup's run starts at tile wg * tpw; tpw needs the total first.
    const PlanPos p0 = plan_scan(a, num_wg, 0, 0);
    const int t0 = wg * p0.tpw;
    const PlanPos p = t0 < p0.total ? plan_scan(a, num_wg, t0, -1) : p0;
    if (lane == 0) {
      plan_lds[0] = t0 < p0.total ? p.b : -1;
      plan_lds[1] = p0.tpw;
      plan_lds[2] = p0.total;
      plan_lds[3] = p.tile_prefix;
      plan_lds[4] = p.seg_prefix;
    }
  }
  __syncthreads();
  int b = __builtin_amdgcn_readfirstlane(plan_lds[0]);
  const int tpw = __builtin_amdgcn_readfirstlane(plan_lds[1]);
  const int total = __builtin_amdgcn_readfirstlane(plan_lds[2]);
  const int tprefix = __builtin_amdgcn_readfirstlane(plan_lds[3]);
  const int sprefix = __builtin_amdgcn_readfirstlane(plan_lds[4]);
  const int t0 = wg * tpw;
  if (b < 0 || t0 >= total) return;
  const int t1 = min(t0 + tpw, total);
  SeqWork sw = seq_work(a, b);
  int g = (t0 - tprefix * hkv) / sw.span;
  int tu = tprefix * hkv + g * sw.span;   // start of unit (b, g) in the flattened list
  int su = sprefix * hkv + g * sw.segs;   // first segment of unit (b, g)

  if (!SUM && wg == 0 && threadIdx.x == 0) a.ws_plan[2 * a.num_seqs * hkv] = tpw;
  int cur = t0;
  while (cur < t1) {
    // Segment s of the unit occupies [s * S, s * S + kSegStartCost + its tiles)
    // of the unit's span; the first kSegStartCost units hold no keys.
    const int S = kSegStartCost + a.seg_tiles;
    const int x = cur - tu;
    const int s = min(x / S, sw.segs - 1);
    const int seg_tiles = s == sw.segs - 1 ? sw.tiles - s * a.seg_tiles : a.seg_tiles;
    const int xr = max(x, s * S + kSegStartCost);           // first key-holding position of the piece
    const int xe = min(s * S + kSegStartCost + seg_tiles, t1 - tu);
    if (xe <= xr) {  // the run ends before the segment's first tile
      cur = tu + xe;
      continue;
    }
    const int lt0 = s * a.seg_tiles + (xr - s * S - kSegStartCost);
    const int lt1 = s * a.seg_tiles + (xe - s * S - kSegStartCost);
    const int lts1 = s * a.seg_tiles + seg_tiles;
    if (!SUM && lt0 == 0 && threadIdx.x == 0) {  // this workgroup holds the unit's first tile: record where it lies
      a.ws_plan[2 * (b * hkv + g)] = tu;
      a.ws_plan[2 * (b * hkv + g) + 1] = su;
    }
    const int tok0 = scalar_load(a.cu_q + b);
    const int lq = min(scalar_load(a.cu_q + b + 1) - tok0, a.max_q_len);
    const int lk = min(scalar_load(a.lens_k + b), a.max_kv_len);
    const int k_lo = lt0 * 64, k_hi = min(lt1 * 64, lk);
    const int32_t* bt_row = a.kv.bt + (int64_t)b * a.kv.bt_stride;
    // A run that covers a whole uncut unit writes the output; any other piece
    // writes its partial rows to its workspace slot.
    const bool direct = lt0 == s * a.seg_tiles && lt1 == lts1 && sw.segs == 1;
    if constexpr (SUM)
      gather_piece<KV>(a, sm, b, g, k_lo, k_hi, first_pages<4>(a.kv, bt_row, k_lo, k_hi));
    else
      verify_piece<KV>(a, sm, b, g, tok0, lq, lk, k_lo, k_hi, first_pages<4>(a.kv, bt_row, k_lo, k_hi), direct,
                       (int64_t)su + s + wg);
    cur = tu + xe;
    if (xe == sw.span) {  // next unit: next kv head, or the next sequence with work
      tu += sw.span;
      su += sw.segs;
      if (++g == hkv) {
        g = 0;
        do {
          if (++b >= a.num_seqs) break;
          sw = seq_work(a, b);
        } while (sw.tiles == 0);
        if (b >= a.num_seqs) break;
      }
    }
  }
}

template <int KV>
__global__ __launch_bounds__(256, (KV == kFP8) ? 2 : 1) void verify_kernel(VerifyArgs a) {
  __shared__ CausalSmem<KV, 4> sm;
  __shared__ int plan_lds[5];
  verify_body<KV, false>(a, sm, plan_lds);
}

// The same work split, grid and copies as verify_kernel, with the arithmetic
// replaced by a checksum of the copied rows: the rate the page gather alone
// reaches on a call's pages (measurement only).
template <int KV>
__global__ __launch_bounds__(256, (KV == kFP8) ? 2 : 1) void verify_gather_kernel(VerifyArgs a) {
  __shared__ CausalSmem<KV, 4> sm;
  __shared__ int plan_lds[5];
  verify_body<KV, true>(a, sm, plan_lds);
}

// Log-sum-exp merge of the partial rows of every (sequence, kv head) unit that
// verify_kernel did not write directly.  One wave per pair of query rows, one
// row per half-wave (16 bytes of stored partial per lane and piece): the
// lanes take one piece each (the lse values of up to 64 pieces for both rows
// in one load each, their maxima and weight sums by wave reductions), then
// every half-wave reads its row of the pieces with the loads of several
// pieces in flight at once; batches of 64 pieces are combined online.  Pieces
// with lse = -inf (no visible key) get weight 0.
template <int KV>
__global__ __launch_bounds__(256) void verify_merge_kernel(VerifyArgs a) {
  const int hkv = a.kv.num_kv_heads;
  const int u = blockIdx.x;
  const int b = u / hkv, g = u - (u / hkv) * hkv;
  const int rho_a = blockIdx.y * 8 + 2 * (threadIdx.x >> 6);  // this wave's rows: rho_a, rho_a + 1
  const int lane = lane_id();
  const int half = lane >> 5, hl = lane & 31;
  // Where the unit lies in the flattened order, as verify_kernel recorded it:
  // loaded together with the sequence's lengths so the two latencies overlap
  // (the addresses are in bounds for every unit; the values are used only
  // when the unit has work).
  const int tu = scalar_load(a.ws_plan + 2 * u);
  const int su = scalar_load(a.ws_plan + 2 * u + 1);
  const int tpw = scalar_load(a.ws_plan + 2 * a.num_seqs * hkv);
  const SeqWork sw = seq_work(a, b);
  if (sw.tiles == 0) return;
  const int tok0 = scalar_load(a.cu_q + b);
  const int lq = min(scalar_load(a.cu_q + b + 1) - tok0, a.max_q_len);
  const int rows = min(a.r * lq, a.rows_cap);
  if (rho_a >= rows) return;
  const bool b_ok = rho_a + 1 < rows;
  const int rho_b = b_ok ? rho_a + 1 : rho_a;    // a missing second row reads the first (in bounds)
  const int rho = half ? rho_b : rho_a;          // this lane's row
  const int S = kSegStartCost + a.seg_tiles;
  if (sw.segs == 1 && (tu + kSegStartCost) / tpw == (tu + kSegStartCost + sw.tiles - 1) / tpw)
    return;  // written directly
  constexpr int kBatch = (KV == kFP8) ? 16 : 8;  // pieces whose rows are in flight at once
  // This lane's 8 head dimensions of its row in piece slot sl, as stored (fp16
  // for FP8 V, fp32 for BF16 V), and widened to fp32.
  using Raw = std::conditional_t<KV == kFP8, i32x4, f32x8>;
  auto load_part = [&](int sl) -> Raw {
    const int64_t off = ((int64_t)sl * a.rows_cap + rho) * kHeadDim + 8 * hl;
    if constexpr (KV == kFP8)
      return *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(a.ws_o) + off);
    else
      return *reinterpret_cast<const f32x8*>(static_cast<const float*>(a.ws_o) + off);
  };
  auto widen = [](Raw r) -> f32x8 {
    if constexpr (KV == kFP8) {
      const f16x8 h = __builtin_bit_cast(f16x8, r);
      f32x8 x;
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
      return x;
    } else {
      return r;
    }
  };
  // Pieces per segment: lane s takes segment s (up to 64 segments at once),
  // so piece j's segment is found by comparisons against a prefix sum instead
  // of a division per segment per piece.
  f32x8 acc;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float mx_a = kNegInf, ws_a = 0.f, mx_b = kNegInf, ws_b = 0.f;
  for (int s0 = 0; s0 < sw.segs; s0 += 64) {
    const int sl = s0 + lane;
    int first = 0, cnt = 0;
    if (sl < sw.segs) {
      const int x0 = tu + sl * S + kSegStartCost;  // first tile of segment sl in the flattened list
      first = x0 / tpw;
      cnt = (x0 + min(a.seg_tiles, sw.tiles - sl * a.seg_tiles) - 1) / tpw - first + 1;
    }
    const int incl = wave_incl_scan(cnt);
    const int excl = incl - cnt;
    const int nseg = min(64, sw.segs - s0);
    const int np = __builtin_amdgcn_readfirstlane(__shfl(incl, nseg - 1));  // pieces of these segments
    for (int c = 0; c < np; c += 64) {
      // Piece j's segment and that segment's first piece and slot, taken with
      // scalar reads of lane k's values: a lane shuffle here would sit under
      // the j < np condition, and a shuffle reads 0 from a lane that is off.
      const int j = c + lane;
      int sj = 0, fj = __builtin_amdgcn_readlane(first, 0), ej = 0;
      for (int k = 1; k < nseg; ++k) {
        const int ek = __builtin_amdgcn_readlane(excl, k);
        const int fk = __builtin_amdgcn_readlane(first, k);
        if (j >= ek) { sj = k; fj = fk; ej = ek; }
      }
      const int slot = j < np ? su + s0 + sj + fj + (j - ej) : -1;
      const float ls_a = slot >= 0 ? a.ws_lse[(int64_t)slot * a.rows_cap + rho_a] : kNegInf;
      const float ls_b = slot >= 0 ? a.ws_lse[(int64_t)slot * a.rows_cap + rho_b] : kNegInf;
      // The rows of the first pieces are requested with their lse values (one
      // round trip for the usual piece counts); no load past the last piece.
      const int n = min(64, np - c);
      Raw v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        v[k] = Raw{};
        if (k < n) v[k] = load_part(__builtin_amdgcn_readlane(slot, k));  // wave-uniform slot
      }
      // Online merge of this batch of pieces into each row's (mx, ws) and acc.
      const float mb_a = wave_max(ls_a), mb_b = wave_max(ls_b);
      if (mb_a == kNegInf && mb_b == kNegInf) continue;
      float sc_a = 1.f, sc_b = 1.f;
      if (mb_a != kNegInf) {
        const float m_new = fmaxf(mx_a, mb_a);
        sc_a = mx_a == kNegInf ? 0.f : __expf(mx_a - m_new);
        ws_a *= sc_a;
        mx_a = m_new;
      }
      if (mb_b != kNegInf) {
        const float m_new = fmaxf(mx_b, mb_b);
        sc_b = mx_b == kNegInf ? 0.f : __expf(mx_b - m_new);
        ws_b *= sc_b;
        mx_b = m_new;
      }
      acc *= half ? sc_b : sc_a;
      const float wg_a = (ls_a == kNegInf || mx_a == kNegInf) ? 0.f : __expf(ls_a - mx_a);
      const float wg_b = (ls_b == kNegInf || mx_b == kNegInf) ? 0.f : __expf(ls_b - mx_b);
      ws_a += wave_sum(wg_a);
      ws_b += wave_sum(wg_b);
      for (int q = 0; q < n; q += kBatch) {
        if (q > 0) {
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            v[k] = Raw{};
            if (q + k < n) v[k] = load_part(__builtin_amdgcn_readlane(slot, q + k));  // wave-uniform slot
          }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          float wq = 0.f;
          if (q + k < n) {
            const float wa = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wg_a), q + k));
            const float wb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wg_b), q + k));
            wq = half ? wb : wa;
          }
          if (wq != 0.f) acc += wq * widen(v[k]);  // a zero weight never touches the slot's data
        }
      }
    }
  }
  if (half && !b_ok) return;
  const float ws = half ? ws_b : ws_a, mx = half ? mx_b : mx_a;
  const float inv = ws > 0.f ? load_scale(a.kv.v_ds) / ws : 0.f;
  const int t = rho / a.r;
  const int head = g * a.r + (rho - t * a.r);
  const int64_t tok = tok0 + t;
  uint16_t* op = a.out + (tok * a.hq + head) * kHeadDim + 8 * hl;  // out is 8-byte aligned: two 8-byte stores
  reinterpret_cast<uint2*>(op)[0] = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
  reinterpret_cast<uint2*>(op)[1] = make_uint2(pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
  if (hl == 0 && a.lse) a.lse[tok * a.hq + head] = ws > 0.f ? mx + logf(ws) : kNegInf;
}

// The merge of the plan-free mode: unit u's pieces are slots u * P + k for
// its tiles k (P = static_tiles <= 64).  One wave per query row; the lse of
// every slot of the unit (one per lane) and the rows of the first 16 are read
// together with the lengths, before it is known how many of them the unit
// has (the reads stay in the workspace; slots past its tiles hold stale
// values and get weight 0).
template <int KV>
__global__ __launch_bounds__(256) void verify_merge_tiles_kernel(VerifyArgs a) {
  const int hkv = a.kv.num_kv_heads;
  const int u = blockIdx.x;
  const int b = u / hkv, g = u - (u / hkv) * hkv;
  const int rho = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (rho >= a.rows_cap) return;
  using Raw = std::conditional_t<KV == kFP8, uint2, f32x4>;
  auto load_part = [&](int64_t sl) -> Raw {
    const int64_t off = (sl * a.rows_cap + rho) * kHeadDim + 4 * lane;
    if constexpr (KV == kFP8)
      return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.ws_o) + off);
    else
      return *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.ws_o) + off);
  };
  auto widen = [](Raw r) -> f32x4 {
    if constexpr (KV == kFP8) {
      const f16x4 h = __builtin_bit_cast(f16x4, r);
      return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    } else {
      return r;
    }
  };
  const int P = a.static_tiles;
  const int64_t base = (int64_t)u * P;
  const float ls_all = lane < P ? a.ws_lse[(base + lane) * a.rows_cap + rho] : kNegInf;
  Raw v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = k < P ? load_part(base + k) : Raw{};
  const SeqWork sw = seq_work(a, b);
  const int tok0 = scalar_load(a.cu_q + b);
  const int lq = min(scalar_load(a.cu_q + b + 1) - tok0, a.max_q_len);
  if (sw.tiles <= 1 || rho >= min(a.r * lq, a.rows_cap)) return;  // written directly / no such row
  const float ls = lane < sw.tiles ? ls_all : kNegInf;
  const float mx = wave_max(ls);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != kNegInf) {
    const float wgt = ls == kNegInf ? 0.f : __expf(ls - mx);
    wsum = wave_sum(wgt);
    for (int q = 0; q < sw.tiles; q += 16) {
      if (q > 0) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          v[k] = Raw{};
          if (q + k < sw.tiles) v[k] = load_part(base + q + k);
        }
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float wq = q + k < sw.tiles ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), q + k)) : 0.f;
        if (wq != 0.f) acc += wq * widen(v[k]);
      }
    }
  }
  const float inv = wsum > 0.f ? load_scale(a.kv.v_ds) / wsum : 0.f;
  const int t = rho / a.r;
  const int head = g * a.r + (rho - t * a.r);
  const int64_t tok = tok0 + t;
  uint16_t* op = a.out + (tok * a.hq + head) * kHeadDim + 4 * lane;
  *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
  if (lane == 0 && a.lse) a.lse[tok * a.hq + head] = wsum > 0.f ? mx + logf(wsum) : kNegInf;
}

hipError_t launch_verify(const VerifyArgs& a, int kv_dtype, int num_wg, hipStream_t s) {
  if (kv_dtype == kFP8)
    hipLaunchKernelGGL(verify_kernel<kFP8>, dim3(num_wg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(verify_kernel<kBF16>, dim3(num_wg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_verify_gather(const VerifyArgs& a, int kv_dtype, int num_wg, hipStream_t s) {
  if (kv_dtype == kFP8)
    hipLaunchKernelGGL(verify_gather_kernel<kFP8>, dim3(num_wg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(verify_gather_kernel<kBF16>, dim3(num_wg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_verify_merge(const VerifyArgs& a, int kv_dtype, int num_wg, hipStream_t s) {
  const unsigned units = (unsigned)(a.num_seqs * a.kv.num_kv_heads);
  if (a.static_tiles > 0) {
    const dim3 grid(units, (a.rows_cap + 3) / 4);  // one row per wave
    if (kv_dtype == kFP8)
      hipLaunchKernelGGL(verify_merge_tiles_kernel<kFP8>, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(verify_merge_tiles_kernel<kBF16>, grid, dim3(256), 0, s, a);
  } else {
    const dim3 grid(units, (a.rows_cap + 7) / 8);  // two rows per wave
    if (kv_dtype == kFP8)
      hipLaunchKernelGGL(verify_merge_kernel<kFP8>, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(verify_merge_kernel<kBF16>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pga
