// Device helpers shared by the gfx950 kernels: 16-byte vector loads, bf16 /
// fp16 <-> fp32 conversion, DPP lane reductions inside a row of 16 lanes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace duo {

constexpr float kLog2e = 1.4426950408889634f;

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8) that waits for all vector memory loads only.
constexpr int kWaitVmcnt0 = 0x0F70;

struct alignas(16) u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
// Streamed (read-once) 16-byte load: one global_load_dwordx4 with the
// non-temporal hint, so that the KV sweep does not evict data that is reused.
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  v4u32 r = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
  return u32x4{r.x, r.y, r.z, r.w};
}

// A wave-uniform pointer to global memory moved to scalar registers
// explicitly; it is rebuilt as a global-address-space pointer, so loads
// through it stay global (not flat) loads.
template <typename T>
__device__ __forceinline__ T* wave_ptr(T* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  typedef __attribute__((address_space(1))) T global_t;
  global_t* g = (global_t*)(((uint64_t)hi << 32) | lo);
  return (T*)g;
}

// Buffer resource for a wave-uniform byte range [p, p + bytes): the base is
// moved to scalar registers explicitly (it is uniform by construction), the
// stride is 0 (raw addressing) and the third dword is the gfx9 default format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
// 16-byte buffer load at byte offset voff (per lane) + soff (scalar), with
// the non-temporal hint (aux bit 1).
__device__ __forceinline__ u32x4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
  typedef uint32_t v4u32b __attribute__((ext_vector_type(4)));
  const v4u32b x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2);
  return u32x4{x.x, x.y, x.z, x.w};
}

// 16-byte buffer load with default caching.
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t v4u32b __attribute__((ext_vector_type(4)));
  const v4u32b x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return u32x4{x.x, x.y, x.z, x.w};
}

// 8-byte variant (two words).
__device__ __forceinline__ void buf_ld8_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                           uint32_t& w0, uint32_t& w1) {
  typedef uint32_t v2u32b __attribute__((ext_vector_type(2)));
  const v2u32b x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 2);
  w0 = x.x;
  w1 = x.y;
}

// Word i (0..3) and 16-bit half i (0..7) of a 16-byte vector, by value (no
// pointer reinterpretation of the struct).
__device__ __forceinline__ uint32_t word_of(const u32x4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint16_t half_of(const u32x4& v, int i) {
  const uint32_t w = word_of(v, i >> 1);
  return (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu));
}

// ---- element types ---------------------------------------------------------
struct Bf16Tag {
  static constexpr bool is_bf16 = true;
};
struct Fp16Tag {
  static constexpr bool is_bf16 = false;
};

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16lo(uint32_t w) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  return (float)h;
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  return (float)h;
}

template <typename Tag>
__device__ __forceinline__ void unpack8(const u32x4& v, float* f);

template <>
__device__ __forceinline__ void unpack8<Bf16Tag>(const u32x4& v, float* f) {
  f[0] = bf16lo(v.x); f[1] = bf16hi(v.x);
  f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
  f[4] = bf16lo(v.z); f[5] = bf16hi(v.z);
  f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
}
template <>
__device__ __forceinline__ void unpack8<Fp16Tag>(const u32x4& v, float* f) {
  f[0] = f16lo(v.x); f[1] = f16hi(v.x);
  f[2] = f16lo(v.y); f[3] = f16hi(v.y);
  f[4] = f16lo(v.z); f[5] = f16hi(v.z);
  f[6] = f16lo(v.w); f[7] = f16hi(v.w);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f2bf(a) | (f2bf(b) << 16);
}

// ---- DPP reductions --------------------------------------------------------
// dpp_ctrl values (GCN/CDNA DPP): quad_perm [1,0,3,2] = 0xB1, quad_perm
// [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 2, 4, 8, 16); every lane of the
// group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
  if constexpr (N >= 2) v += dpp<0xB1>(v);
  if constexpr (N >= 4) v += dpp<0x4E>(v);
  if constexpr (N >= 8) v += dpp<0x141>(v);
  if constexpr (N >= 16) v += dpp<0x140>(v);
  return v;
}

// Butterfly across lane groups with xor distances >= 16 (ds_bpermute).
__device__ __forceinline__ float xor_lane(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace duo
