// Wave-level attention core for 16 query rows against a 32- or 64-key tile in LDS.
//
// The scores are formed transposed, S^T = K * Q^T, with the keys as the MFMA M
// dimension and the wave's 16 query rows as N.  A lane then owns one query row
// (n = lane % 16) and 4 * NMB of the tile's keys
// (key = 16 * mb + 4 * (lane / 16) + i), so the row maximum and sum need only
// in-lane work plus one reduction over the four 16-lane groups, and the
// probabilities already sit in the B-operand layout of the P * V product:
// O^T = V^T * P^T, with V^T read from LDS by transpose loads.
//
// Arithmetic (fixed by the 2e-3 rel-L2 bar; see the rounding emulator test):
//   QK^T  BF16 keys: bf16 x bf16 MFMA, fp32 accumulate.
//         FP8 keys: scaled FP8 MFMA, keys used as stored; a bf16 query row is
//         split exactly into two FP8 parts (hi + lo / 16, row scaled by a power
//         of two) -- the same products as bf16 arithmetic without widening the
//         keys; an FP8 query row is used as it is.
//   softmax in fp32, base 2, scale folded into one multiplier per row.
//   PV    FP8 V: fp16 P x fp16 V (exact widening);  BF16 V: P split into a
//         bf16 high and low part, two bf16 MFMAs.
//
// LDS tile layout: row = key, row bytes RB = 256 * elt, stored in 16-byte
// chunks whose position is XOR-swizzled by the key: logical chunk c of key k
// sits at chunk c ^ (k & (RB / 16 - 1)).  SPREAD (bf16 rows, 32 chunks): at
// c ^ (2 k mod 32) instead, which keeps the two chunks of one 16-column block
// (2d, 2d + 1) apart for neighbouring keys, so the 16-bit transpose reads of
// V (keys 4 (lane / 16) + e, both chunks of a block) and the row reads of K
// (16 keys, one chunk each) hit distinct banks.
#pragma once

#include "pga_device.h"

namespace pga {

template <int KV, bool SPREAD = false>
struct TileGeom {
  static constexpr int kElt = (KV == kFP8) ? 1 : 2;
  static constexpr int kRowBytes = kHeadDim * kElt;  // 256 or 512
  static constexpr int kChunks = kRowBytes / 16;     // 16 or 32
  template <int TK>
  static constexpr int tile_bytes() { return TK * kRowBytes; }  // one of K or V
  // The key's part of the swizzle: logical chunk c of key k sits at c ^ xor_of(k).
  // The tile copies compute the same term in place.
  __device__ static __forceinline__ int xor_of(int key) {
    if constexpr (SPREAD)
      return (2 * key) & (kChunks - 1);
    else
      return key & (kChunks - 1);
  }
  __device__ static __forceinline__ int swz(int key, int chunk) { return chunk ^ xor_of(key); }
  __device__ static __forceinline__ int off(int key, int chunk) { return key * kRowBytes + (swz(key, chunk) << 4); }
};

// Running state of one wave: 16 rows, full head dimension.
struct WaveState {
  f32x4 o[16];  // O^T: o[mb][i] = O[row = lane % 16][d = 16 * mb + 4 * (lane / 16) + i]
  float m;      // reference maximum of the scaled scores (log2 domain), per row
  float l;      // this lane's partial sum of probabilities (reduced over groups at the end)
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = kNegInf;
    l = 0.f;
  }
};

// Q^T operand of the wave's 16 rows, by key encoding.
//   BF16 keys: q[ks] holds Q[row][32 * ks + 8 * (lane / 16) + j] (bf16 MFMA B operand).
//   FP8 keys:  hi[h] / lo[h] hold 32 FP8 codes of Q[row][128 * h + 32 * (lane / 16) + j]
//     (B operand of the scaled 16x16x128 FP8 MFMA).
// rscale multiplies the scores computed from the fragment (1 unless the row
// was scaled before its FP8 split).
template <int KV>
struct QFragT;
template <>
struct QFragT<kBF16> {
  bf16x8 q[8];
  float rscale;
};
template <>
struct QFragT<kFP8> {
  i32x8 hi[2];
  i32x8 lo[2];
  bool has_lo;
  float rscale;
};

// E8M0 scale codes of the scaled FP8 MFMA: 2^0 and 2^-4.
constexpr int kScaleOne = 127;
constexpr int kScaleLo = 123;

__device__ __forceinline__ f32x4 mfma_fp8_scaled(i32x8 a, i32x8 b, f32x4 c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kScaleOne, 0, scale_b);
}

// Split 8 query values (already multiplied by the row scale) into FP8 codes,
// two dwords each: x = hi + lo / 16 exactly whenever |x| >= 2^-6.
__device__ __forceinline__ void split_q8(const float (&x)[8], int& hi0, int& hi1, int& lo0, int& lo1) {
  int h[2] = {0, 0}, l[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const int w = j >> 2;
    const bool up = (j & 2) != 0;
    const int hp = __builtin_amdgcn_cvt_pk_fp8_f32(x[j], x[j + 1], 0, false);
    const auto back = __builtin_amdgcn_cvt_pk_f32_fp8(hp, false);
    const int lp = __builtin_amdgcn_cvt_pk_fp8_f32((x[j] - back[0]) * 16.f, (x[j + 1] - back[1]) * 16.f, 0, false);
    h[w] |= up ? (hp & 0xFFFF) << 16 : (hp & 0xFFFF);
    l[w] |= up ? (lp & 0xFFFF) << 16 : (lp & 0xFFFF);
  }
  hi0 = h[0];
  hi1 = h[1];
  lo0 = l[0];
  lo1 = l[1];
}

// Scores of a tile of 16 * NMB keys: s[mb][i] for key 16 * mb + 4 * (lane / 16) + i,
// before the softmax scale and the fragment's rscale.  QSPLIT: the FP8 query
// fragment has a low part (bf16 queries).
template <int KV, int NMB, bool QSPLIT>
__device__ __forceinline__ void tile_scores(const lds_t* kt, const QFragT<KV>& qf, f32x4 (&s)[NMB]) {
  using G = TileGeom<KV>;
  const int lane = lane_id();
  const int n = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (KV == kFP8) {
    // A operand: 32 FP8 codes of key 16 * mb + n, bytes 128 * h + 32 * gq .. + 31
    // (logical chunks 8h + 2gq and 8h + 2gq + 1 of the key row).
    // The low-part MFMA of a block depends on its high-part result, so all
    // high parts of a half are issued before the low parts.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x8 a[NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int key = mb * 16 + n;
        const i32x4 a0 = lds_load<i32x4>(kt + G::off(key, 8 * h + 2 * gq));
        const i32x4 a1 = lds_load<i32x4>(kt + G::off(key, 8 * h + 2 * gq + 1));
        a[mb] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) s[mb] = mfma_fp8_scaled(a[mb], qf.hi[h], s[mb], kScaleOne);
      if constexpr (QSPLIT) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) s[mb] = mfma_fp8_scaled(a[mb], qf.lo[h], s[mb], kScaleLo);
      }
    }
  } else if constexpr (NMB == 1) {
    // One 16-key block: every K fragment is requested first, and the head
    // dimension is summed in two chains (even and odd 32-element steps) so
    // that consecutive MFMAs do not wait on each other's results.
    bf16x8 a[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) a[ks] = lds_load<bf16x8>(kt + G::off(n, 4 * ks + gq));
    __builtin_amdgcn_sched_barrier(0);  // keep the requests ahead of the products
    f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ks += 2) {
      s[0] = mfma_bf16(a[ks], qf.q[ks], s[0]);
      s1 = mfma_bf16(a[ks + 1], qf.q[ks + 1], s1);
    }
    s[0] += s1;
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int key = mb * 16 + n;
        const bf16x8 a = lds_load<bf16x8>(kt + G::off(key, 4 * ks + gq));
        s[mb] = mfma_bf16(a, qf.q[ks], s[mb]);
      }
    }
  }
}

// Online softmax (every kernel): the probabilities are taken relative to a
// reference maximum m that is only raised when some row's tile maximum exceeds
// it by more than kRescaleLog2, so the accumulators are rescaled a handful of
// times per row instead of once per tile; p stays below 2^kRescaleLog2, well
// inside fp16 and bf16 range, and the row sum l is kept relative to the same
// reference.
constexpr float kRescaleLog2 = 8.0f;

// O^T += V^T * P^T over one tile, in two steps: fetch() requests every V
// fragment of the tile from LDS, multiply() runs the products, so a caller can
// place other work (the next tile's scores and softmax) between the requests
// and the products.  Three tile shapes: 16 BF16 keys (one 16-key step, P as a
// bf16 high and low part), 32 FP8 keys (one 32-key step, fp16 P, V widened
// exactly to fp16) and 16 FP8 keys (one 16-key step, the same precisions).
template <int KV, int NMB>
struct TilePV;

template <>
struct TilePV<kBF16, 1> {
  i16x4 a[16];
  // V^T: transpose-read source lane sl = 4e + q points at key 4 (lane / 16) + e,
  // columns 4q .. 4q + 3 of the d-block.
  __device__ __forceinline__ void fetch(const lds_t* vt) {
    using G = TileGeom<kBF16>;
    const int lane = lane_id();
    const int gq = lane >> 4, sl = lane & 15;
    const int e = sl >> 2, q = sl & 3;
#pragma unroll
    for (int mb = 0; mb < 16; ++mb)
      a[mb] = __builtin_bit_cast(i16x4, lds_tr16(vt + G::off(4 * gq + e, 2 * mb + (q >> 1)) + 8 * (q & 1)));
  }
  // P^T as the B operand: lane holds keys 4 (lane / 16) + j of its row, as the
  // scores lie.  The high parts of all 16 blocks, then the low parts (the same
  // sums per block as high-then-low, without a product waiting on the one just
  // before it).
  __device__ __forceinline__ void multiply(WaveState& st, const f32x4 (&p)[1]) const {
    i16x4 ph, pl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = p[0][j];
      const __bf16 h = (__bf16)x;
      ph[j] = __builtin_bit_cast(short, h);
      pl[j] = __builtin_bit_cast(short, (__bf16)(x - (float)h));
    }
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) st.o[mb] = mfma_bf16_k16(a[mb], ph, st.o[mb]);
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) st.o[mb] = mfma_bf16_k16(a[mb], pl, st.o[mb]);
  }
};

template <>
struct TilePV<kFP8, 2> {
  i32x2 raw[16];
  // Transpose-read source: lane sl = 2e + q points at key(e), bytes 8q .. 8q + 7 of the d-block.
  __device__ __forceinline__ void fetch(const lds_t* vt) {
    using G = TileGeom<kFP8>;
    const int lane = lane_id();
    const int gq = lane >> 4, sl = lane & 15;
    const int e = sl >> 1, q = sl & 1;
    const int key = 16 * (e >> 2) + 4 * gq + (e & 3);
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) raw[mb] = lds_tr8(vt + G::off(key, mb) + 8 * q);
  }
  __device__ __forceinline__ void multiply(WaveState& st, const f32x4 (&p)[2]) const {
    const f16x8 pb = {(_Float16)p[0][0], (_Float16)p[0][1], (_Float16)p[0][2], (_Float16)p[0][3],
                      (_Float16)p[1][0], (_Float16)p[1][1], (_Float16)p[1][2], (_Float16)p[1][3]};
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) st.o[mb] = mfma_f16(fp8x8_to_f16(raw[mb]), pb, st.o[mb]);
  }
};

template <>
struct TilePV<kFP8, 1> {
  int32_t raw[16];
  // The 32-key transpose read of TilePV<kFP8, 2>, whose bytes 0..3 in lane l
  // are V at keys 4 (l / 16) + j, column l % 16 of the d-block: exactly the
  // 16x16x16 operand.  Its sources for keys 16..31 point at keys 0..15 here
  // (in bounds); those bytes (4..7) are not used.
  __device__ __forceinline__ void fetch(const lds_t* vt) {
    using G = TileGeom<kFP8>;
    const int lane = lane_id();
    const int gq = lane >> 4, sl = lane & 15;
    const int e = sl >> 1, q = sl & 1;
    const int key = 4 * gq + (e & 3);
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) raw[mb] = lds_tr8(vt + G::off(key, mb) + 8 * q)[0];
  }
  __device__ __forceinline__ void multiply(WaveState& st, const f32x4 (&p)[1]) const {
    const f16x4 pb = {(_Float16)p[0][0], (_Float16)p[0][1], (_Float16)p[0][2], (_Float16)p[0][3]};
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) st.o[mb] = mfma_f16_k16(fp8x4_to_f16((unsigned)raw[mb]), pb, st.o[mb]);
  }
};

// Scores of several 16-row blocks of one wave on the same tile (FP8 keys):
// each K fragment read from LDS feeds one MFMA per row block (two with a
// split bf16 query, QSPLIT: the high and the low part), so the LDS reads of a
// tile are shared by NRB * 16 query rows.
template <int NRB, int NMB, bool QSPLIT = false>
__device__ __forceinline__ void tile_scores_rows(const lds_t* kt, const QFragT<kFP8> (&qf)[NRB],
                                                 f32x4 (&s)[NRB][NMB]) {
  using G = TileGeom<kFP8>;
  const int lane = lane_id();
  const int n = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) s[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (!QSPLIT) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int key = mb * 16 + n;
        const i32x4 a0 = lds_load<i32x4>(kt + G::off(key, 8 * h + 2 * gq));
        const i32x4 a1 = lds_load<i32x4>(kt + G::off(key, 8 * h + 2 * gq + 1));
        const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) s[rb][mb] = mfma_fp8_scaled(a, qf[rb].hi[h], s[rb][mb], kScaleOne);
      }
    } else {
      // Every high-part product of the half before the low parts, so no
      // product waits on the one just issued into the same accumulator.
      i32x8 a[NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int key = mb * 16 + n;
        const i32x4 a0 = lds_load<i32x4>(kt + G::off(key, 8 * h + 2 * gq));
        const i32x4 a1 = lds_load<i32x4>(kt + G::off(key, 8 * h + 2 * gq + 1));
        a[mb] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) s[rb][mb] = mfma_fp8_scaled(a[mb], qf[rb].hi[h], s[rb][mb], kScaleOne);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) s[rb][mb] = mfma_fp8_scaled(a[mb], qf[rb].lo[h], s[rb][mb], kScaleLo);
    }
  }
}

}  // namespace pga
