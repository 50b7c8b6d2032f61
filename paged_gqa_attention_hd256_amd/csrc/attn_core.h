// Wave-level attention core for 16 query rows against a 32- or 64-key tile in LDS.
//
// The scores are formed transposed, S^T = K * Q^T, on 16x16x32 bf16 MFMAs with
// the keys as the M dimension and the wave's 16 query rows as N.  A lane then
// owns one query row (n = lane % 16) and 16 of the tile's keys
// (key = 16 * mb + 4 * (lane / 16) + i), so the row maximum and sum need only
// in-lane work plus one reduction over the four 16-lane groups, and the
// probabilities already sit in the B-operand layout of the P * V product:
// O^T = V^T * P^T, with V^T read from LDS by transpose loads.
//
// Arithmetic (fixed by the 2e-3 rel-L2 bar; see the rounding emulator test):
//   QK^T  bf16 x bf16 -> fp32 (FP8 keys are widened to bf16 exactly)
//   softmax in fp32, base 2, scale folded into one multiplier
//   PV    FP8 V: fp16 P x fp16 V (exact widening);  BF16 V: P split into a
//         bf16 high and low part, two bf16 MFMAs.
//
// LDS tile layout: row = key, row bytes RB = 256 * elt, stored in
// 16-byte chunks whose position is XOR-swizzled by the key: logical chunk c of
// key k sits at chunk c ^ (k & (RB / 16 - 1)).
#pragma once

#include "pga_device.h"

namespace pga {

template <int KV>
struct TileGeom {
  static constexpr int kElt = (KV == kFP8) ? 1 : 2;
  static constexpr int kRowBytes = kHeadDim * kElt;  // 256 or 512
  static constexpr int kChunks = kRowBytes / 16;     // 16 or 32
  template <int TK>
  static constexpr int tile_bytes() { return TK * kRowBytes; }  // one of K or V
  __device__ static __forceinline__ int swz(int key, int chunk) { return chunk ^ (key & (kChunks - 1)); }
  __device__ static __forceinline__ int off(int key, int chunk) { return key * kRowBytes + (swz(key, chunk) << 4); }
};

// Running state of one wave: 16 rows, full head dimension.
struct WaveState {
  f32x4 o[16];  // O^T: o[mb][i] = O[row = lane % 16][d = 16 * mb + 4 * (lane / 16) + i]
  float m;      // running max of the scaled scores (log2 domain), per row
  float l;      // this lane's partial sum of probabilities (reduced over groups at the end)
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = kNegInf;
    l = 0.f;
  }
};

// Q^T operand of the 16 rows: qf[ks] holds Q[row][32 * ks + 8 * (lane / 16) + j].
struct QFrag {
  bf16x8 q[8];
};

// Scores of a tile of 16 * NMB keys: s[mb][i] for key 16 * mb + 4 * (lane / 16) + i.
template <int KV, int NMB>
__device__ __forceinline__ void tile_scores(const lds_t* kt, const QFrag& qf, f32x4 (&s)[NMB]) {
  using G = TileGeom<KV>;
  const int lane = lane_id();
  const int n = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const int key = mb * 16 + n;
      bf16x8 a;
      if constexpr (KV == kFP8) {
        const int byte = 32 * ks + 8 * gq;
        a = fp8x8_to_bf16(lds_load<i32x2>(kt + G::off(key, byte >> 4) + (byte & 15)));
      } else {
        a = lds_load<bf16x8>(kt + G::off(key, 4 * ks + gq));
      }
      s[mb] = mfma_bf16(a, qf.q[ks], s[mb]);
    }
  }
}

// Online-softmax update with the tile's scores; returns the probabilities in
// s (in place) and rescales the accumulators.  `c2` is the log2-domain score
// multiplier.  When `masked` is true, `visible(key)` (key relative to the tile
// start) decides which of this lane's keys count.
template <int NMB, class Vis>
__device__ __forceinline__ void tile_softmax(WaveState& st, f32x4 (&s)[NMB], float c2, bool masked, Vis visible) {
  const int gq = lane_id() >> 4;
  float mt = kNegInf;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = s[mb][i] * c2;
      if (masked && !visible(mb * 16 + 4 * gq + i)) x = kNegInf;
      s[mb][i] = x;
      mt = fmaxf(mt, x);
    }
  }
  mt = group4_max(mt);
  const float m_new = fmaxf(st.m, mt);
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = fast_exp2(st.m - m_use);
  float sum = 0.f;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(s[mb][i] - m_use);
      s[mb][i] = p;
      sum += p;
    }
  }
  st.l = st.l * alpha + sum;
  st.m = m_new;
#pragma unroll
  for (int d = 0; d < 16; ++d) st.o[d] *= alpha;
}

// O^T += V^T * P^T over the tile's 16 * NMB keys (32-key MFMA steps).
template <int KV, int NMB>
__device__ __forceinline__ void tile_pv(WaveState& st, const lds_t* vt, const f32x4 (&p)[NMB]) {
  static_assert(NMB % 2 == 0, "tiles hold a multiple of 32 keys");
  using G = TileGeom<KV>;
  const int lane = lane_id();
  const int gq = lane >> 4, sl = lane & 15;
#pragma unroll
  for (int t = 0; t < NMB / 2; ++t) {
    if constexpr (KV == kFP8) {
      const f16x8 pb = {(_Float16)p[2 * t][0], (_Float16)p[2 * t][1], (_Float16)p[2 * t][2], (_Float16)p[2 * t][3],
                        (_Float16)p[2 * t + 1][0], (_Float16)p[2 * t + 1][1], (_Float16)p[2 * t + 1][2],
                        (_Float16)p[2 * t + 1][3]};
      // transpose-read source: lane sl = 2e + q points at key(e), bytes 8q..8q+7 of the d-block
      const int e = sl >> 1, q = sl & 1;
      const int key = 32 * t + 16 * (e >> 2) + 4 * gq + (e & 3);
#pragma unroll
      for (int mb = 0; mb < 16; ++mb) {
        const f16x8 a = fp8x8_to_f16(lds_tr8(vt + G::off(key, mb) + 8 * q));
        st.o[mb] = mfma_f16(a, pb, st.o[mb]);
      }
    } else {
      bf16x8 ph, pl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = p[2 * t + (j >> 2)][j & 3];
        const __bf16 h = (__bf16)x;
        ph[j] = h;
        pl[j] = (__bf16)(x - (float)h);
      }
      // transpose-read source: lane sl = 4e + q points at key(e), columns 4q..4q+3
      const int e = sl >> 2, q = sl & 3;
#pragma unroll
      for (int mb = 0; mb < 16; ++mb) {
        const int chunk = 2 * mb + (q >> 1);
        const int key0 = 32 * t + 4 * gq + e;
        const int key1 = key0 + 16;
        const i32x2 lo = __builtin_bit_cast(i32x2, lds_tr16(vt + G::off(key0, chunk) + 8 * (q & 1)));
        const i32x2 hi = __builtin_bit_cast(i32x2, lds_tr16(vt + G::off(key1, chunk) + 8 * (q & 1)));
        const bf16x8 a = __builtin_bit_cast(bf16x8, i32x4{lo[0], lo[1], hi[0], hi[1]});
        st.o[mb] = mfma_bf16(a, ph, st.o[mb]);
        st.o[mb] = mfma_bf16(a, pl, st.o[mb]);
      }
    }
  }
}

}  // namespace pga
