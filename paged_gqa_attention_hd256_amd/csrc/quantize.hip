// Per-tensor FP8 E4M3FN quantisation of a prefix-hit prefill's inputs: Q to a
// contiguous FP8 tensor under a dynamic (or given) descale, and the new tokens'
// keys and values straight into the FP8 page pool under the pool's own
// descales.  These are the casts to FP8 that ROCm/ATOM PR #2534 counts inside
// its prefill timings (FMHA commit message; Results, per-layer trace), done
// here in two launches over all three tensors:
//   quant_amax_kernel   max |q| over the non-NaN elements, one partial per
//                       workgroup (bf16 magnitudes compare as integers);
//   quant_apply_kernel  every workgroup folds the partials into the descale
//                       (amax / 448 in fp32, or 1 when amax is 0), then codes
//                       its share of Q and of the new key / value rows.
// Both are HBM streams (2 bytes in per element, 1 byte out); every lane moves
// 16-byte chunks.
//
// The code of x is the E4M3FN value nearest to fp32(x / descale), ties to the
// even code, saturated at +-448.  The division is an exact-rounding
// reciprocal scheme: with r = 1/d rounded, q0 = x * r is within one ulp of
// x/d, and one correction y = q0 + (x - q0 d) r, with the remainder formed
// exactly by an fma, is the correctly rounded quotient (Markstein's theorem;
// the remainder must not underflow, hence the range guard on d, outside of
// which the plain IEEE division runs).  The rounding to E4M3 is the
// hardware's round-to-nearest-even conversion after an explicit clamp.
#include <algorithm>

#include "pga_args.h"
#include "pga_device.h"

namespace pga {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kChunksPerThread = 4;          // 16-byte chunks in flight per lane
constexpr int kChunksPerRow = kHeadDim / 8;  // 32 chunks of 8 bf16 elements per head row

// Largest non-NaN magnitude of two bf16 values packed in a word, folded into
// m.  For non-negative floats the bit patterns order like the values; patterns
// above 0x7F80 (after dropping the sign) are NaNs and are left out.
__device__ __forceinline__ uint32_t fold_absmax(uint32_t m, uint32_t w) {
  const uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
  m = lo <= 0x7F80u ? max(m, lo) : m;
  m = hi <= 0x7F80u ? max(m, hi) : m;
  return m;
}

__device__ __forceinline__ uint32_t fold_absmax(uint32_t m, uint4 v) {
  m = fold_absmax(m, v.x);
  m = fold_absmax(m, v.y);
  m = fold_absmax(m, v.z);
  return fold_absmax(m, v.w);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), off)));
  return x;
}

// Block-wide maximum; every thread gets the result.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t x, uint32_t* red) {
  x = wave_max_u32(x);
  if (lane_id() == 0) red[wave_id()] = x;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; ++w) m = max(m, red[w]);
  return m;
}

__global__ __launch_bounds__(kQuantThreads) void quant_amax_kernel(const uint4* __restrict__ q, int64_t chunks,
                                                                   uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kQuantThreads / 64];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kQuantThreads;
  uint32_t m = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kQuantThreads + threadIdx.x; i < chunks;
       i += stride * kChunksPerThread) {
    uint4 v[kChunksPerThread];
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u)
      v[u] = i + u * stride < chunks ? q[i + u * stride] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) m = fold_absmax(m, v[u]);
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// Quotient x / d rounded as IEEE fp32 division would round it (see the file
// comment).  FAST is the reciprocal scheme, valid for d in [2^-64, 2^64]; it
// is exact up to the saturation point, beyond which only |y| > 448 matters,
// and q0 is clamped so that no infinity meets a zero.
template <bool FAST>
struct Divider {
  float d, r;
  __device__ __forceinline__ explicit Divider(float descale) : d(descale), r(1.0f / descale) {}
  __device__ __forceinline__ float operator()(float x) const {
    if constexpr (!FAST) {
      return x / d;
    } else {
      float q0 = __fmul_rn(x, r);
      q0 = __builtin_fminf(__builtin_fmaxf(q0, -1024.0f), 1024.0f);
      const float e = __builtin_fmaf(-q0, d, x);
      // The correction never changes the sign of a nonzero q0; copying q0's
      // sign keeps the sign of a zero quotient (-0 / d is -0, but e is +0).
      return __builtin_copysignf(__builtin_fmaf(e, r, q0), q0);
    }
  }
};

__device__ __forceinline__ bool reciprocal_ok(float d) { return d >= 0x1p-64f && d <= 0x1p64f; }

__device__ __forceinline__ float clamp448(float y) {
  return y != y ? y : __builtin_fminf(__builtin_fmaxf(y, -448.0f), 448.0f);
}

// Eight bf16 values -> eight E4M3FN codes (little-endian in the result).
template <class Div>
__device__ __forceinline__ uint2 quant8(uint4 v, const Div& div) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = clamp448(div(__builtin_bit_cast(float, w[i] << 16)));
    y[2 * i + 1] = clamp448(div(__builtin_bit_cast(float, w[i] & 0xFFFF0000u)));
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  return make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
}

// Sequence of query token `tok`: the largest b with cu_q[b] <= tok.
__device__ __forceinline__ int seq_of(const int32_t* cu_q, int num_seqs, int64_t tok) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The coding pass proper.  Work items are Q's 16-byte chunks, then one item
// per 16-byte chunk of a new token's key row together with the same chunk of
// its value row (they share the destination page and slot).
template <bool FAST>
__device__ __forceinline__ void apply_chunks(const QuantArgs& a, float qd, float kd, float vd) {
  const Divider<FAST> qdiv(qd), kdiv(kd), vdiv(vd);
  const int64_t q_chunks = a.q_chunks;
  const int64_t total = q_chunks + a.kv_rows * kChunksPerRow;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kQuantThreads;
  const uint4* q = reinterpret_cast<const uint4*>(a.q);
  const uint4* kn = reinterpret_cast<const uint4*>(a.k_new);
  const uint4* vn = reinterpret_cast<const uint4*>(a.v_new);
  uint2* qo = reinterpret_cast<uint2*>(a.q_out);
  const int hkv = a.kv.num_kv_heads;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * kQuantThreads + threadIdx.x; i0 < total;
       i0 += stride * kChunksPerThread) {
    uint4 x[kChunksPerThread], y[kChunksPerThread];
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      const int64_t i = i0 + u * stride;
      x[u] = y[u] = make_uint4(0, 0, 0, 0);
      if (i < q_chunks) {
        x[u] = q[i];
      } else if (i < total) {
        x[u] = kn[i - q_chunks];
        y[u] = vn[i - q_chunks];
      }
    }
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < q_chunks) {
        qo[i] = quant8(x[u], qdiv);
      } else if (i < total) {
        const int32_t j = static_cast<int32_t>(i - q_chunks);  // < 2^31 (host check)
        const int32_t row = j / kChunksPerRow;                  // token * hkv + head
        const int c = j % kChunksPerRow;
        const int32_t tok = row / hkv;
        const int g = row - tok * hkv;
        const int b = seq_of(a.cu_q, a.num_seqs, tok);
        const int32_t lq = a.cu_q[b + 1] - a.cu_q[b];
        const int32_t lk = a.cu_k[b + 1] - a.cu_k[b];
        const int32_t t = tok - a.cu_q[b];
        const int32_t pos = lk - lq + t;
        if (pos < 0 || t >= lq) continue;  // before the sequence start / past cu_seqlens_q's last token
        const int32_t page = a.kv.bt[b * a.kv.bt_stride + (pos >> a.kv.page_shift)];
        if (page < 0 || page >= a.kv.num_pages) continue;
        const int64_t slot = pos & (a.kv.page_size - 1);
        uint8_t* kdst = const_cast<uint8_t*>(a.kv.k) + page * a.kv.k_sp + slot * a.kv.k_st + g * a.kv.k_sh;
        uint8_t* vdst = const_cast<uint8_t*>(a.kv.v) + page * a.kv.v_sp + slot * a.kv.v_st + g * a.kv.v_sh;
        *reinterpret_cast<uint2*>(kdst + 8 * c) = quant8(x[u], kdiv);
        *reinterpret_cast<uint2*>(vdst + 8 * c) = quant8(y[u], vdiv);
      }
    }
  }
}

__global__ __launch_bounds__(kQuantThreads) void quant_apply_kernel(QuantArgs a) {
  __shared__ uint32_t red[kQuantThreads / 64];
  float qd;
  if (a.q_ds_in) {
    qd = *a.q_ds_in;
  } else {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < a.num_partial; i += kQuantThreads) m = max(m, a.partial[i]);
    m = block_max_u32(m, red);
    const float amax = __builtin_bit_cast(float, m << 16);
    qd = amax > 0.0f ? amax / 448.0f : 1.0f;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && a.q_ds_out) *a.q_ds_out = qd;
  const float kd = load_scale(a.kv.k_ds), vd = load_scale(a.kv.v_ds);
  if (reciprocal_ok(qd) && reciprocal_ok(kd) && reciprocal_ok(vd))
    apply_chunks<true>(a, qd, kd, vd);
  else
    apply_chunks<false>(a, qd, kd, vd);
}

}  // namespace

int quant_amax_blocks(int64_t q_chunks) {
  const int64_t per_block = int64_t(kQuantThreads) * kChunksPerThread;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(kQuantMaxPartials, (q_chunks + per_block - 1) / per_block)));
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (!a.q_ds_in) {
    hipLaunchKernelGGL(quant_amax_kernel, dim3(a.num_partial), dim3(kQuantThreads), 0, s,
                       reinterpret_cast<const uint4*>(a.q), a.q_chunks, a.partial);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  const int64_t total = a.q_chunks + a.kv_rows * kChunksPerRow;
  const int64_t per_block = int64_t(kQuantThreads) * kChunksPerThread;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(a.max_blocks, (total + per_block - 1) / per_block));
  hipLaunchKernelGGL(quant_apply_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kQuantThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pga
