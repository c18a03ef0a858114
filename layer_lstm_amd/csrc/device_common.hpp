// device_common.hpp -- element types, bf16 rounding, activations, MFMA
// wrappers and the tagged-word exchange used by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lstm {

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory

typedef _Float16 f16_t;   // IEEE binary16 storage
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
// operand types of the buffer load / store builtins
typedef uint32_t v2u32_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32_t __attribute__((ext_vector_type(4)));

// Round fp32 to the nearest bf16, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Storage element <-> fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float to_f(float v) { return v; }
  __device__ __forceinline__ static float from_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static float to_f(bf16_t v) { return bf2f(v); }
  __device__ __forceinline__ static bf16_t from_f(float v) { return f2bf(v); }
};

template <> struct Elem<f16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const f16_t* p) { return (float)*p; }
  __device__ __forceinline__ static float to_f(f16_t v) { return (float)v; }
  // v_cvt_f16_f32: round to nearest even (the default mode); beyond the
  // range, +-inf
  __device__ __forceinline__ static f16_t from_f(float v) { return (f16_t)v; }
};
// A 16-bit storage element from the low 16 bits of a word.
template <typename T>
__device__ __forceinline__ float f_of_bits16(uint32_t bits) {
  return Elem<T>::to_f(__builtin_bit_cast(T, (uint16_t)bits));
}

// Logistic sigmoid s(u) = 1/(1+e^-u) from its definition on the hardware
// base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32; about 1 ulp
// each): e^-u = 2^(-u*log2(e)).  For u -> -inf, 2^(..) -> +inf and the
// reciprocal gives 0; for u -> +inf it gives 1; never NaN for finite u.
// tanh(u) = 2 s(2u) - 1 (absolute error about 1e-7, saturates to +-1).
__device__ __forceinline__ float sigmoidf(float u) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u * -1.4426950408889634f));
}
__device__ __forceinline__ float tanh_f(float u) { return 2.0f * sigmoidf(2.0f * u) - 1.0f; }

// One MFMA k-block: 16 bytes per lane of each operand.
//  fp32: 4 k-values per lane -> four v_mfma_f32_16x16x4f32 (k-slot s of the
//        lane group q holds k = 4q + s of a 16-wide k-block);
//  bf16: 8 k-values per lane -> one v_mfma_f32_16x16x32_bf16;
// Lane layout of both operands: row (A) / column (B) = lane % 16, k-group =
// lane / 16.  Result: lane holds C[4*(lane/16)+i][lane%16], i = 0..3.
template <typename T> struct Mfma;
template <> struct Mfma<float> {
  static constexpr int kBlock = 16;  // k elements per 16-byte fragment group
  __device__ __forceinline__ static f32x4_t mac(u32x4_t a, u32x4_t b, f32x4_t c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[1]), __uint_as_float(b[1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[2]), __uint_as_float(b[2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[3]), __uint_as_float(b[3]), c, 0, 0, 0);
    return c;
  }
};
template <> struct Mfma<bf16_t> {
  static constexpr int kBlock = 32;
  __device__ __forceinline__ static f32x4_t mac(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
//  fp16: 8 k-values per lane -> one v_mfma_f32_16x16x32_f16.
template <> struct Mfma<f16_t> {
  static constexpr int kBlock = 32;
  __device__ __forceinline__ static f32x4_t mac(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

// Element type of a storage dtype code (0 fp32, 1 bf16, 2 fp16).
__host__ __device__ __forceinline__ int dtype_bytes(int dtype) { return dtype == 0 ? 4 : 2; }
// fp32 value of element i of a buffer of storage dtype `dtype`.
__device__ __forceinline__ float load_as_f(const void* p, int64_t i, int dtype) {
  if (dtype == 1) return bf2f(((const bf16_t*)p)[i]);
  if (dtype == 2) return (float)((const f16_t*)p)[i];
  return ((const float*)p)[i];
}
// Store fp32 v as element i of a buffer of storage dtype `dtype`.
__device__ __forceinline__ void store_from_f(void* p, int64_t i, float v, int dtype) {
  if (dtype == 1) ((bf16_t*)p)[i] = f2bf(v);
  else if (dtype == 2) ((f16_t*)p)[i] = (f16_t)v;
  else ((float*)p)[i] = v;
}

// ---------------------------------------------------------------------------
// Tagged-word exchange between the work-groups of a persistent kernel.
// A word is 8 bytes: low 32 bits = an fp32 value, high 32 bits = the step
// tag.  Words are written and read with relaxed agent-scope 64-bit atomics,
// so a reader that sees the expected tag sees the value written with it: no
// fence and no separate barrier are needed.  Exchange buffers are cleared
// (tag 0) before every launch and tags are 1-based.
//
// XCD-local groups (all readers of a word on the writer's XCD): the word is
// stored with a plain (work-group scope) store, which stays in that XCD's
// L2, and the device-coherent load of a reader on the same XCD finds it
// there; this saves the write-through to memory on every step.  Readers on
// other XCDs would not see such a word, so callers use it only after
// checking that the work-group runs where the layout assumes (xcc_id()).
// (The plain store is one aligned 8-byte global store, so a reader sees
// either the old or the new word whole.)
__device__ __forceinline__ void xstore_word(uint64_t* p, uint64_t w, bool local) {
  if (local)
    *p = w;
  else
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xstore(uint64_t* p, float v, uint32_t tag, bool local) {
  xstore_word(p, ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v), local);
}
// Index of the XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 15u;
}
__device__ __forceinline__ uint64_t xload(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t xtag(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float xval(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Wait until every vector memory operation of this wave has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left alone).  Used on the rare
// paths of a step (the first step, a dead wait) so that every path reaching
// the next step has no loads or stores outstanding; otherwise the compiler
// must assume some are and waits for all stores before reusing their
// registers on the common path.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// 16 bytes per lane from a buffer straight into LDS, to (wave-uniform) lds +
// 16 * lane; SC1 selects a device-coherent read.  Issued through inline asm
// so that the compiler does not see an LDS write: for a direct-to-LDS
// builtin it inserts waits of its own before LDS reads it cannot tell
// apart from the destination, which empties every pipeline built on these
// loads.  The caller therefore waits (vmcnt, then a barrier for the other
// waves) before the data is read.  The instruction writes no register (the
// hazard of asm loads with register outputs does not arise); M0 carries the
// LDS address and is declared clobbered.
typedef __attribute__((address_space(3))) void lds_void_t;

// Row block of gate g (0..3 = i, f, g, o) in W, b, dW and db: the gate order
// "ifjo" (i, f, g, o), or with ijfo "ijfo" (i, g, f, o) -- the two values of
// the gate_order attribute of the SingleLayerLstmGrad page (参数说明).
__host__ __device__ __forceinline__ int gate_block(int g, int ijfo) { return (ijfo && (g == 1 || g == 2)) ? 3 - g : g; }
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// (lds_addr: the LDS byte address the wave's 1 KB goes to)
template <bool SC1>
__device__ __forceinline__ void lds_dma16_at(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  if constexpr (SC1)
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, %3 offen sc1 lds"
                 :
                 : "v"(voff), "s"(m0v), "s"(r), "s"(soff)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
                 :
                 : "v"(voff), "s"(m0v), "s"(r), "s"(soff)
                 : "memory", "m0");
}
template <bool SC1>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  lds_dma16_at<SC1>(r, (uint32_t)(uintptr_t)(lds_void_t*)lds, voff, soff);
}
#pragma clang diagnostic pop

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; a field at its maximum does not wait):
// vmcnt(n) alone, and lgkmcnt(0) alone
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }
constexpr int kLgkm0 = 0xC07F;

// Time bound of one wait: s_memrealtime runs at 100 MHz.
constexpr uint64_t kWaitTicks = 200000000ull;  // 2 s
__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

}  // namespace lstm
