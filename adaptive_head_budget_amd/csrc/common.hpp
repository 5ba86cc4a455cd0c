// Device helpers shared by the gfx950 kernels of libadakv.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace adakv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Raw 16-byte global / LDS moves (callers guarantee 16-byte alignment).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming (nontemporal) forms for data read or written once.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }

// One 16x16 MFMA step per element type.  Lane l supplies A[m = l%16][KPL*(l/16) .. +KPL)
// and B[KPL*(l/16) .. +KPL)[n = l%16]; the result D[m = 4*(l/16)+j][n = l%16], j < 4,
// stays in the lane.  Any consistent K ordering of A and B gives the same product.
template <typename T> struct Mma;

template <> struct Mma<uint16_t> {   // bf16 storage
  static constexpr int KSTEP = 32;   // K per instruction
  static constexpr int KPL = 8;      // K elements per lane
  typedef bf16x8 op_t;
  __device__ __forceinline__ static op_t load(const uint16_t* p) { return *reinterpret_cast<const op_t*>(p); }
  __device__ __forceinline__ static op_t load_nt(const uint16_t* p) { return __builtin_bit_cast(op_t, ld16_nt(p)); }
  __device__ __forceinline__ static op_t zero() { u32x4 z = {0u, 0u, 0u, 0u}; return __builtin_bit_cast(op_t, z); }
  __device__ __forceinline__ static f32x4 mma(op_t a, op_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  typedef float op_t;
  __device__ __forceinline__ static op_t load(const float* p) { return *p; }
  __device__ __forceinline__ static op_t load_nt(const float* p) { return __builtin_nontemporal_load(p); }
  __device__ __forceinline__ static op_t zero() { return 0.f; }
  __device__ __forceinline__ static f32x4 mma(op_t a, op_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// Lane shuffles through the LDS permute network (no LDS storage used).
__device__ __forceinline__ float shfl_lane(float x, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(x)));
}
__device__ __forceinline__ int shfl_lane_i(int x, int src_lane) {
  return __builtin_amdgcn_ds_bpermute(src_lane << 2, x);
}
__device__ __forceinline__ float shfl_xor(float x, int mask) {
  return shfl_lane(x, (int)(__lane_id() ^ mask));
}

// Lane moves inside rows of 16 lanes on the vector unit (DPP), no LDS traffic:
// DPP_MIRROR: lane i <- lane 15 - i; DPP_HALF_MIRROR: i <- 7 - i within each 8;
// DPP_XOR2 / DPP_XOR1: i <- i ^ 2 / i ^ 1 within each 4.  All four are
// involutions, so they pair lanes like a butterfly.
enum { DPP_MIRROR = 0x140, DPP_HALF_MIRROR = 0x141, DPP_XOR2 = 0x4E, DPP_XOR1 = 0xB1 };
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// exp2 on the hardware transcendental unit (results below 2^-126 flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Score keys are non-negative floats: their bit patterns order like the values,
// once -0.0 is mapped to +0.0.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  return u == 0x80000000u ? 0u : u;
}

}  // namespace adakv
