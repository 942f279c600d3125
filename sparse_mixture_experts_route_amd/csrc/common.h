// Shared device helpers for the gfx950 MoE kernels: bf16 <-> fp32, vector
// types, wavefront shuffles.  Wavefronts are 64 lanes wide.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#define MOE_DEV __device__ __forceinline__

typedef uint16_t bf16_t;  // storage type: raw bfloat16 bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace moe {

constexpr int kWave = 64;

MOE_DEV float bf16_to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
MOE_DEV bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Element load/store through the storage type of the layer dtype.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static MOE_DEV float load(const float* p) { return *p; }
  static MOE_DEV void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static MOE_DEV float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static MOE_DEV void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

MOE_DEV float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }
MOE_DEV uint32_t shfl_xor_u(uint32_t v, int m) { return (uint32_t)__shfl_xor((int)v, m, kWave); }

MOE_DEV float wave_sum(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
  return v;
}
MOE_DEV float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}

// Wait until at most N of this wave's vector-memory operations (the DMA
// instructions) are outstanding and every LDS operation has completed.
template <int N>
MOE_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  // gfx9 s_waitcnt: vmcnt[3:0] bits 3:0, vmcnt[5:4] bits 15:14, expcnt bits
  // 6:4 left at its maximum (no wait), lgkmcnt bits 11:8 = 0.
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Whole-line DMA global -> LDS through a buffer descriptor: one
// buffer_load_dwordx4 ... lds per wave moves 16 bytes per lane from
// base + voff + soff into byte 16 l of the 1 KB LDS block `lds` (lane l).
// The descriptor form rather than global_load_lds: the compiler takes a
// FLAT-encoded LDS DMA in flight as an LDS event of unknown completion order
// and then makes every later fragment read wait for all outstanding LDS reads
// (lgkmcnt 0), which undoes any read-ahead; with the buffer form its waits
// keep exact counts.  Descriptor: raw (stride 0), 0xFFFFFFFF bytes of range
// (the offsets are 32-bit), dword 3 = 0x00020000 (32-bit data format).
MOE_DEV __amdgpu_buffer_rsrc_t dma_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
MOE_DEV void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, soff, 0,
                                           0);
}

// The same DMA written as inline asm, for kernels whose fragment reads use
// the transposing LDS read builtin: the compiler cannot tell such a read from
// an LDS DMA it can see in flight and makes it wait for every outstanding
// DMA (vmcnt 0), the prefetch of the next slices included.  Hidden from the
// compiler, the DMA is ordered against the reads by the kernel's own vmcnt
// waits and barriers only.  No register outputs; M0, the instruction's LDS
// base, is set in the same block (a kernel using this must leave M0 to it:
// no other LDS DMA and nothing else that reads M0).  `r`: the 4 descriptor
// words of dma_rsrc, wave-uniform.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
// range: bytes from base a load may read; a load at or past it reads no
// memory (the default covers every 32-bit offset)
MOE_DEV i32x4_t dma_rsrc_words(const void* base, uint32_t range = 0xffffffffu) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)range);
  r[3] = 0x00020000;
  return r;
}
// The same with a wave-uniform byte offset in the scalar offset operand.
MOE_DEV void dma16_hidden_so(i32x4_t r, uint32_t voff, uint32_t soff, void* lds) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(r),
               "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}
MOE_DEV void dma16_hidden(i32x4_t r, uint32_t voff, void* lds) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for every outstanding DMA): LDS visibility is established by the
// explicit waits above.  The empty asm statements keep the compiler from
// moving memory operations across the barrier.
MOE_DEV void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// binary16 storage of fp32 GEMM outputs (expert outputs of a bf16 layer):
// round to nearest even; beyond the binary16 range the value becomes inf.
typedef _Float16 f16_t;
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
MOE_DEV uint32_t pack_f16x2(float a, float b) {
  const f16x2_t h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Fast SiLU pieces for GEMM epilogues (hardware exp2 and reciprocal).
MOE_DEV float fast_sigmoid(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// ---- host helpers.  Kernel attributes and device properties belong to a
// device, so both caches are per device (the device current at the call).

// Raises kern's dynamic-LDS limit to `bytes` once per device; `done` is the
// caller's per-kernel bitmask of the devices already set.  0 or -4.
inline int set_lds_limit(const void* kern, int bytes, std::atomic<unsigned long long>& done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -4;
  const unsigned long long bit = 1ull << dev;
  if (done.load(std::memory_order_acquire) & bit) return 0;
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) return -4;
  done.fetch_or(bit, std::memory_order_acq_rel);
  return 0;
}

// Compute units of the current device (cached per device), 0 on error.
inline int device_cu_count() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cus[dev].load(std::memory_order_acquire);
  if (v) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cus[dev].store(v, std::memory_order_release);
  return v;
}

}  // namespace moe
