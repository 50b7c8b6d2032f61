// Device-side building blocks for the gfx950 (CDNA4) attention kernels.
//
// Lane layouts used throughout (wave64, verified on gfx950):
//   mfma 16x16x32 (bf16 / f16):  A lane l holds A[l % 16][8 * (l / 16) + j],
//     B lane l holds B[8 * (l / 16) + j][l % 16], C register i of lane l holds
//     C[4 * (l / 16) + i][l % 16].
//   ds_read_b64_tr_b8:  within each 16-lane group, lane i receives byte i % 8
//     of source lane 2e + i / 8 as its element e (e = 0..7): if source lane
//     2e + q points at row e, bytes 8q..8q+7, lane i gets column i of rows 0..7.
//   ds_read_b64_tr_b16: lane i receives element i % 4 of source lane 4e + i / 4
//     (e = 0..3): if source lane 4e + q points at row e, columns 4q..4q+3, lane i
//     gets column i of rows 0..3.
//   global_load_lds (16 B): lane l's bytes land at the wave-uniform LDS base
//     plus 16 * l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pga {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((address_space(3))) char lds_t;

constexpr int kHeadDim = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

enum KvKind { kBF16 = 1, kFP8 = 2 };

// Sixteen zero bytes: the load source of every lane whose key is masked, so
// each DMA instruction is issued by every lane and stays finite in LDS.
__device__ __attribute__((aligned(16))) static const uint32_t g_zero16[4] = {0, 0, 0, 0};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// MI355X dispatches workgroup b of a launch to XCD b % 8, and each XCD has an
// L2 of its own.
constexpr int kXcds = 8;

// Jobs of independent waves that each belong to one of hkv kv heads: job j of
// head g is wave j % W of the j / W-th workgroup of that head.  When hkv
// divides the XCD count, every workgroup of an XCD works on one head (the
// XCDs take the heads in turn), so an XCD's L2 holds the rows of one head
// instead of all of them; the launch then needs kXcds * ceil(ceil(L / W) /
// (kXcds / hkv)) workgroups for L jobs per head.  Otherwise the heads take
// consecutive jobs in turn (ceil(hkv * L / W) workgroups).
struct HeadJob {
  int g;      // kv head
  int64_t j;  // job index among that head's jobs
};
__device__ __forceinline__ HeadJob head_job(int b, int w, int W, int hkv) {
  if (kXcds % hkv == 0) {
    const int per = kXcds / hkv, xcd = b % kXcds;
    return HeadJob{xcd % hkv, ((int64_t)(b / kXcds) * per + xcd / hkv) * W + w};
  }
  const int64_t job = (int64_t)b * W + w;
  return HeadJob{(int)(job % hkv), job / hkv};
}
inline int64_t head_job_grid(int64_t jobs_per_head, int W, int hkv) {
  const int64_t wgs = (jobs_per_head + W - 1) / W;
  if (kXcds % hkv == 0) {
    const int per = kXcds / hkv;
    return kXcds * ((wgs + per - 1) / per);
  }
  return (hkv * jobs_per_head + W - 1) / W;
}
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Wait until at most N vector-memory loads of this wave are outstanding (loads
// complete in issue order for this counter).  Other counters are not waited on.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without a memory fence (a fence would also wait for every
// in-flight LDS-DMA load).  The empty asm keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier after which this wave's LDS writes are visible to the other waves:
// waits for its LDS (and scalar-memory) operations, not for vector memory.
__device__ __forceinline__ void barrier_publish() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte global -> LDS copy; `lds_wave_base` must be the same for the whole
// wave (lane l writes lds_wave_base + 16 * l).  Issued from inline assembly so
// the compiler does not treat every later LDS read as possibly aliasing the
// copy in flight (it would wait for all of them); the kernels wait on this
// wave's copies explicitly with wait_vmcnt.  Compiler-generated waits for its
// own loads stay correct, only more conservative, because the counter retires
// loads in issue order.
//
// The LDS destination travels in M0.  M0 is an input operand of the asm
// ("{m0}"): the compiler writes it before the statement and knows it is
// unchanged after, so no reserved register is clobbered behind its back.  On
// GFX9 an LDS DMA must not issue in the cycle right after an SALU write of
// M0; the compiler's hazard check cannot see inside the asm, hence the s_nop.
__device__ __forceinline__ void dma16(const void* src, lds_t* lds_wave_base) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_wave_base);
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "{m0}"(base)
      : "memory");
}
// The same copy from a wave-uniform 64-bit base plus a 32-bit per-lane byte
// offset (the scalar-base form: no 64-bit address arithmetic per lane).
// `lds_addr` is the wave-uniform LDS byte address lane 0 writes.  NT: the load
// carries the non-temporal cache policy, for data read exactly once (a
// speculative-verify KV stream): its lines do not displace reused ones.
template <bool NT = false>
__device__ __forceinline__ void dma16_off(uint64_t uniform_base, unsigned offset, unsigned lds_addr) {
  const unsigned lds = __builtin_amdgcn_readfirstlane(lds_addr);
  if constexpr (NT) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(offset), "s"(uniform_base), "{m0}"(lds)
        : "memory");
  } else {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(offset), "s"(uniform_base), "{m0}"(lds)
        : "memory");
  }
}

template <class T>
__device__ __forceinline__ T lds_load(const lds_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <class T>
__device__ __forceinline__ void lds_store(lds_t* p, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}

__device__ __forceinline__ i32x2 lds_tr8(const lds_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)p);
}
__device__ __forceinline__ i16x4 lds_tr16(const lds_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}

// Eight FP8 E4M3FN codes (two dwords) -> eight bf16 / f16 values (exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(i32x2 w) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ f16x8 fp8x8_to_f16(i32x2 w) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w[0], 1.0f, false);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w[0], 1.0f, true);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w[1], 1.0f, false);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w[1], 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Four FP8 E4M3FN codes (one dword) -> four f16 values (exact).
__device__ __forceinline__ f16x4 fp8x4_to_f16(unsigned w) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return f16x4{a[0], a[1], b[0], b[1]};
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x16 bf16: A lane l holds A[l % 16][4 * (l / 16) + j], B lane l holds
// B[4 * (l / 16) + j][l % 16], j = 0..3 (bf16 bit patterns in shorts).
__device__ __forceinline__ f32x4 mfma_bf16_k16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 16x16x16 f16, the lane layout of mfma_bf16_k16.
__device__ __forceinline__ f32x4 mfma_f16_k16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Reductions over the four 16-lane groups of a wave (lanes n, n+16, n+32, n+48).
__device__ __forceinline__ float group4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)b[0]), __builtin_bit_cast(float, (int)b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  return __builtin_bit_cast(float, (int)b[0]) + __builtin_bit_cast(float, (int)b[1]);
}

// Reductions over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float load_scale(const float* p) { return p ? *p : 1.0f; }

}  // namespace pga
