// Per-tensor FP8 E4M3FN quantisation of a prefix-hit prefill's inputs: Q to a
// contiguous FP8 tensor under a dynamic (or given) descale, and the new tokens'
// keys and values straight into the FP8 page pool under the pool's own
// descales.  These are the casts to FP8 that ROCm/ATOM PR #2534 counts inside
// its prefill timings (FMHA commit message; Results, per-layer trace).  All
// of it is an HBM stream (2 bytes in per element, 1 byte out; every lane moves
// 16-byte chunks), and Q's descale needs all of Q before any of Q is coded.
//
// Resident path (dynamic descale, Q up to kQuantResidentChunks chunks per
// thread over one workgroup per CU: 64 MiB of Q at 256 CUs with 16 chunks per
// thread, which the register file holds):
//   quant_resident_kernel    one launch, one workgroup per CU.  Each loads its
//                            share of Q into registers, codes its
//                            share of the new key / value rows (their
//                            descales are static), folds max |q| over the
//                            non-NaN elements (bf16 magnitudes compare as
//                            integers) and publishes it; after a grid barrier
//                            every workgroup folds the partials into the
//                            descale (amax / 448 in fp32, or 1 when amax is 0)
//                            and codes the Q it holds.  Q is read from HBM
//                            once.
// Otherwise two launches:
//   quant_amax_kernel   the partial maxima of Q, one per workgroup;
//   quant_apply_kernel  every workgroup folds the partials into the descale,
//                       then codes its share of Q (read a second time) and of
//                       the new key / value rows.
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
constexpr int kResidentThreads = 1024;  // threads of a resident workgroup
constexpr int kResidentWgPerCu = 1024 / kResidentThreads;  // 16 waves per CU
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
// One correction of the estimate q0 of x / d: y = q0 - e r with the remainder
// e = q0 d - x formed exactly by an fma (the negation of x - q0 d, so y is
// the usual q0 + (x - q0 d) r bit for bit).  Written this way round, a zero
// quotient keeps its sign without a copysign: for x = -0, q0 = -0, e = +0 and
// y = -0 - (+0) r = -0.  The correction never changes the sign of a nonzero q0.
__device__ __forceinline__ float correct_quotient(float x, float q0, float d, float r) {
  const float e = __builtin_fmaf(q0, d, -x);
  return __builtin_fmaf(-e, r, q0);
}

template <bool FAST>
struct Divider {
  float d, r;
  __device__ __forceinline__ explicit Divider(float descale) : d(descale), r(1.0f / descale) {}
  __device__ __forceinline__ float correct(float x, float q0) const { return correct_quotient(x, q0, d, r); }
  __device__ __forceinline__ float operator()(float x) const {
    if constexpr (!FAST) {
      return x / d;
    } else {
      float q0 = __fmul_rn(x, r);
      q0 = __builtin_fminf(__builtin_fmaxf(q0, -1024.0f), 1024.0f);
      return correct(x, q0);
    }
  }
};

__device__ __forceinline__ bool reciprocal_ok(float d) { return d >= 0x1p-64f && d <= 0x1p64f; }

__device__ __forceinline__ float clamp448(float y) {
  return y != y ? y : __builtin_fminf(__builtin_fmaxf(y, -448.0f), 448.0f);
}

// Q's quotient under its own dynamic descale on the reciprocal's range: with
// d = fp32(amax / 448) and |x| <= amax (NaN x are left out of amax; an
// infinite x makes d infinite, outside the range), |x / d| stays within
// 448 (1 + 2^-23) and x * r cannot overflow, so neither clamp of the general
// scheme can act: the unclamped estimate and correction give the same
// correctly rounded quotient, a NaN x gives NaN, and the conversion rounds
// anything up to 464 to 448 by itself.
struct DynamicDivider {
  float d, r;
  __device__ __forceinline__ explicit DynamicDivider(float descale) : d(descale), r(1.0f / descale) {}
  __device__ __forceinline__ float operator()(float x) const { return correct_quotient(x, __fmul_rn(x, r), d, r); }
};

// Eight bf16 values -> eight E4M3FN codes (little-endian in the result).
// CLAMP: saturate finite quotients at +-448 (NaN kept); off only for the
// DynamicDivider, whose quotients never need it.
template <class Div, bool CLAMP = true>
__device__ __forceinline__ uint2 quant8(uint4 v, const Div& div) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = div(__builtin_bit_cast(float, w[i] << 16));
    y[2 * i + 1] = div(__builtin_bit_cast(float, w[i] & 0xFFFF0000u));
    if constexpr (CLAMP) {
      y[2 * i] = clamp448(y[2 * i]);
      y[2 * i + 1] = clamp448(y[2 * i + 1]);
    }
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

// One key/value work item: the j-th 16-byte chunk of the new key rows and the
// same chunk of the new value rows (they share the destination page and
// slot), coded under the pool's descales and written into the pool.
template <class Div>
__device__ __forceinline__ void code_kv_item(const QuantArgs& a, int32_t j, uint4 x, uint4 y, const Div& kdiv,
                                             const Div& vdiv) {
  const int32_t row = j / kChunksPerRow;  // token * hkv + head
  const int c = j % kChunksPerRow;
  const int hkv = a.kv.num_kv_heads;
  const int32_t tok = row / hkv;
  const int g = row - tok * hkv;
  const int b = seq_of(a.cu_q, a.num_seqs, tok);
  const int32_t lq = a.cu_q[b + 1] - a.cu_q[b];
  const int32_t lk = a.cu_k[b + 1] - a.cu_k[b];
  const int32_t t = tok - a.cu_q[b];
  const int32_t pos = lk - lq + t;
  if (pos < 0 || t >= lq) return;  // before the sequence start / past cu_seqlens_q's last token
  const int32_t page = a.kv.bt[b * a.kv.bt_stride + (pos >> a.kv.page_shift)];
  if (page < 0 || page >= a.kv.num_pages) return;
  const int64_t slot = pos & (a.kv.page_size - 1);
  uint8_t* kdst = const_cast<uint8_t*>(a.kv.k) + page * a.kv.k_sp + slot * a.kv.k_st + g * a.kv.k_sh;
  uint8_t* vdst = const_cast<uint8_t*>(a.kv.v) + page * a.kv.v_sp + slot * a.kv.v_st + g * a.kv.v_sh;
  *reinterpret_cast<uint2*>(kdst + 8 * c) = quant8(x, kdiv);
  *reinterpret_cast<uint2*>(vdst + 8 * c) = quant8(y, vdiv);
}

// The coding pass of the two-launch path.  Work items are Q's 16-byte chunks,
// then the key/value items.
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
        code_kv_item(a, static_cast<int32_t>(i - q_chunks), x[u], y[u], kdiv, vdiv);  // < 2^31 (host check)
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

// Grid barrier of the resident path, with no counter to clear: workgroup b
// publishes its partial maximum in slot b (one 64-bit word per 128-byte line,
// after the two-launch path's partials), tagged with a 48-bit value that the
// host makes unique to the call (a per-process random start plus twice a
// call count, odd, so never a zero-filled or earlier call's slot).  Every
// workgroup then polls all slots, one lane per slot, until each carries the
// call's tag, and folds their maxima itself.  The wait is bounded: a lane
// whose wait expires writes the call's tag to the flag word after the slots
// and the workgroup codes its Q with a NaN descale (NaN codes, loud), so
// every wave exits whatever happens.  One workgroup per CU keeps the grid
// co-resident on an otherwise idle part; the launch is an ordinary one (a
// cooperative launch, which would guarantee it, cost about 17 us more per
// call on this part).
constexpr unsigned kSpinLimit = 1u << 22;  // polls of >= 128 cycles each: > 0.2 s
constexpr int kSlotStride = 16;            // 64-bit words between slots (128 bytes)
constexpr uint64_t kTagMask = (uint64_t(1) << 48) - 1;
static_assert(kQuantWorkspaceBytes >= kQuantMaxPartials * sizeof(uint32_t) + (kQuantMaxPartials * kSlotStride + 1) * 8,
              "workspace holds the barrier slots and the flag word");

// Q's chunk pairs in the resident path: pair p = v * (grid threads) + gt is
// chunks 2p and 2p + 1, held in x[2v] and x[2v + 1].  Each load step of the
// grid covers one contiguous stretch of Q, and each lane stores the 16 code
// bytes of its pair at once.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_q_chunk(const uint4* q, int64_t i, int64_t n) {
  if (i >= n) return make_uint4(0, 0, 0, 0);
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(q + i));  // read once
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int R, bool CLAMP, class Div>
__device__ __forceinline__ void code_resident_q(const QuantArgs& a, const uint4 (&x)[R], int64_t gt, int64_t gthreads,
                                                const Div& div) {
#pragma unroll
  for (int v = 0; v < R / 2; ++v) {
    const int64_t i = 2 * (v * gthreads + gt);
    if (i + 1 < a.q_chunks) {
      const uint2 c0 = quant8<Div, CLAMP>(x[2 * v], div), c1 = quant8<Div, CLAMP>(x[2 * v + 1], div);
      *reinterpret_cast<uint4*>(a.q_out + 8 * i) = make_uint4(c0.x, c0.y, c1.x, c1.y);
    } else if (i < a.q_chunks) {
      *reinterpret_cast<uint2*>(a.q_out + 8 * i) = quant8<Div, CLAMP>(x[2 * v], div);
    }
  }
}

template <int R>
__global__ __launch_bounds__(kResidentThreads) void quant_resident_kernel(QuantArgs a) {
  static_assert(R % 2 == 0, "chunk pairs");
  __shared__ uint32_t red[kResidentThreads / 64];
  __shared__ float qd_sh;
  const int64_t gthreads = static_cast<int64_t>(gridDim.x) * kResidentThreads;
  const int64_t gt = static_cast<int64_t>(blockIdx.x) * kResidentThreads + threadIdx.x;
  // The new keys and values: the thread's first two items are requested
  // ahead of Q and coded during the grid barrier's wait (the pool's
  // descales are static).
  const float kd = load_scale(a.kv.k_ds), vd = load_scale(a.kv.v_ds);
  const bool kv_fast = reciprocal_ok(kd) && reciprocal_ok(vd);
  const int32_t items = static_cast<int32_t>(a.kv_rows * kChunksPerRow);  // < 2^31 (host check)
  const uint4* kn = reinterpret_cast<const uint4*>(a.k_new);
  const uint4* vn = reinterpret_cast<const uint4*>(a.v_new);
  const int32_t j0 = static_cast<int32_t>(gt), j1 = static_cast<int32_t>(gt + gthreads);  // < 2^31: grid <= 1024
  uint4 kx0 = make_uint4(0, 0, 0, 0), vx0 = kx0, kx1 = kx0, vx1 = kx0;
  if (j0 < items) { kx0 = kn[j0]; vx0 = vn[j0]; }
  if (j1 < items) { kx1 = kn[j1]; vx1 = vn[j1]; }
  const uint4* q = reinterpret_cast<const uint4*>(a.q);
  uint4 x[R];
#pragma unroll
  for (int v = 0; v < R / 2; ++v) {
    const int64_t i = 2 * (v * gthreads + gt);
    x[2 * v] = load_q_chunk(q, i, a.q_chunks);
    x[2 * v + 1] = load_q_chunk(q, i + 1, a.q_chunks);
  }
  uint32_t m = 0;
#pragma unroll
  for (int u = 0; u < R; ++u) m = fold_absmax(m, x[u]);
  m = wave_max_u32(m);
  if (lane_id() == 0) red[wave_id()] = m;
  __syncthreads();
  uint64_t* slots = reinterpret_cast<uint64_t*>(a.partial + kQuantMaxPartials);
  const uint64_t tag = a.tag & kTagMask;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 0; w < kResidentThreads / 64; ++w) m = max(m, red[w]);
    __hip_atomic_store(slots + kSlotStride * blockIdx.x, (tag << 16) | m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The keys and values while the other workgroups publish.
  if (kv_fast) {
    const Divider<true> kdiv(kd), vdiv(vd);
    if (j0 < items) code_kv_item(a, j0, kx0, vx0, kdiv, vdiv);
    if (j1 < items) code_kv_item(a, j1, kx1, vx1, kdiv, vdiv);
    for (int64_t j = gt + 2 * gthreads; j < items; j += gthreads)
      code_kv_item(a, static_cast<int32_t>(j), kn[j], vn[j], kdiv, vdiv);
  }
  __syncthreads();  // red is free again (thread 0 has read it)
  // Every slot, one lane each, until it carries this call's tag.
  uint32_t all = 0;
  bool expired = false;
  for (unsigned b = threadIdx.x; b < gridDim.x; b += kResidentThreads) {
    const uint64_t* sp = slots + kSlotStride * b;
    uint64_t v = __hip_atomic_load(sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned polls = 0;
    while ((v >> 16) != tag) {
      __builtin_amdgcn_s_sleep(2);
      if (++polls == kSpinLimit) {
        expired = true;
        break;
      }
      v = __hip_atomic_load(sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    all = max(all, static_cast<uint32_t>(v & 0xFFFFu));
  }
  if (expired)
    __hip_atomic_store(slots + kSlotStride * kQuantMaxPartials, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  all = wave_max_u32(all);
  const bool wave_expired = __builtin_amdgcn_ballot_w64(expired) != 0;
  if (lane_id() == 0) red[wave_id()] = wave_expired ? 0xFFFFFFFFu : all;
  __syncthreads();
  all = 0;
  bool any_expired = false;
#pragma unroll
  for (int w = 0; w < kResidentThreads / 64; ++w) {
    any_expired |= red[w] == 0xFFFFFFFFu;
    all = max(all, red[w]);
  }
  const float amax = __builtin_bit_cast(float, all << 16);
  const float qd_fold = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (threadIdx.x == 0) qd_sh = any_expired ? __builtin_nanf("") : qd_fold;  // NaN descale: NaN codes
  __syncthreads();
  const float qd = qd_sh;
  if (blockIdx.x == 0 && threadIdx.x == 0 && a.q_ds_out) *a.q_ds_out = qd;
  if (reciprocal_ok(qd))
    code_resident_q<R, false>(a, x, gt, gthreads, DynamicDivider(qd));
  else
    code_resident_q<R, true>(a, x, gt, gthreads, Divider<false>(qd));  // also a NaN descale
  if (!kv_fast) {
    // Descales outside the reciprocal's range: the keys and values are coded
    // by the plain division, after Q, when its registers are free.
    const Divider<false> kdiv(kd), vdiv(vd);
    for (int64_t j = gt; j < items; j += gthreads) code_kv_item(a, static_cast<int32_t>(j), kn[j], vn[j], kdiv, vdiv);
  }
}

// Whether Q's chunks fit the resident path at R chunks per thread on `grid`
// workgroups, and the kernel's co-residency on this device.
template <int R>
bool resident_fits(int64_t q_chunks, int grid) {
  return q_chunks <= static_cast<int64_t>(grid) * R * kResidentThreads;
}

template <int R>
hipError_t launch_resident(const QuantArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(quant_resident_kernel<R>, dim3(grid), dim3(kResidentThreads), 0, s, a);
  return hipGetLastError();
}

// kResidentWgPerCu workgroups of every resident instance fit on a CU
// (checked once per device), so the grid is resident at once.
bool resident_supported() {
  static int cache[64] = {0};  // 0 unknown, 1 yes, -1 no
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (cache[dev] == 0) {
    int n4 = 0, n8 = 0, n16 = 0;
    bool ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n4, quant_resident_kernel<4>, kResidentThreads, 0) == hipSuccess;
    ok = ok && hipOccupancyMaxActiveBlocksPerMultiprocessor(&n8, quant_resident_kernel<8>, kResidentThreads, 0) == hipSuccess;
    ok = ok && hipOccupancyMaxActiveBlocksPerMultiprocessor(&n16, quant_resident_kernel<16>, kResidentThreads, 0) == hipSuccess;
    cache[dev] = ok && n4 >= kResidentWgPerCu && n8 >= kResidentWgPerCu && n16 >= kResidentWgPerCu ? 1 : -1;
  }
  return cache[dev] == 1;
}

}  // namespace

int quant_amax_blocks(int64_t q_chunks) {
  const int64_t per_block = int64_t(kQuantThreads) * kChunksPerThread;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(kQuantMaxPartials, (q_chunks + per_block - 1) / per_block)));
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  // The resident path stores 16 code bytes per lane: q_out 16-byte aligned.
  const bool out16 = (reinterpret_cast<uintptr_t>(a.q_out) & 15) == 0;
  if (!a.q_ds_in && out16 && a.num_cus > 0 && a.num_cus * kResidentWgPerCu <= kQuantMaxPartials &&
      resident_supported()) {
    const int g = a.num_cus * kResidentWgPerCu;
    int r = 0;
    if (resident_fits<4>(a.q_chunks, g)) r = 4;
    else if (resident_fits<8>(a.q_chunks, g)) r = 8;
    else if (resident_fits<kQuantResidentChunks>(a.q_chunks, g)) r = kQuantResidentChunks;
    if (r > 0) {
      if (r == 4) return launch_resident<4>(a, g, s);
      if (r == 8) return launch_resident<8>(a, g, s);
      return launch_resident<kQuantResidentChunks>(a, g, s);
    }
  }
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
