// Device helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16;
typedef unsigned int u32;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf2f(u16 x) { return __uint_as_float((u32)x << 16); }

__device__ __forceinline__ int frame_hi(int i, int P, int E) {
  return i < P ? P : (i < E ? i + 1 : E);
}

// SiLU(x) = x * sigmoid(x) with the hardware exp2 and reciprocal.
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// SiLU'(z) = s (1 + z (1 - s)) with s = 1 / (1 + e^-z) (the layer's phi1).
__device__ __forceinline__ float silu_grad(float z) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
  return sg * (1.0f + z * (1.0f - sg));
}

// floor(log2(max(1, |dt|))) clamped to n_tb - 1.
__device__ __forceinline__ int time_bucket(long long dt, int n_tb) {
  unsigned long long m = dt < 0 ? 0ull - (unsigned long long)dt : (unsigned long long)dt;
  int b = m <= 1ull ? 0 : 63 - __clzll((long long)m);
  return b < n_tb - 1 ? b : n_tb - 1;
}

__device__ __forceinline__ int pos_bucket(int dp, int n_pos) {
  dp = dp < 0 ? -dp : dp;
  return dp < n_pos - 1 ? dp : n_pos - 1;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// gfx950 transposing LDS read: within each group of 16 lanes, output lane j,
// element e is the 16-bit value at (address of source lane 4e + j/4) + j%4.
__device__ __forceinline__ s16x4 lds_read_tr16(const u16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
}

// |a - b| of two unsigned values (one instruction).
__device__ __forceinline__ unsigned absdiff_u32(unsigned a, unsigned b) {
  unsigned d;
  asm("v_sad_u32 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// Index of the highest set bit counted from the top (0..31), -1 for 0.
__device__ __forceinline__ int ffbh_u32(unsigned x) {
  int c;
  asm("v_ffbh_u32 %0, %1" : "=v"(c) : "v"(x));
  return c;
}

__device__ __forceinline__ int bucket_u32(unsigned x, int n_tb) {
  const int b = x <= 1u ? 0 : 31 - __builtin_clz(x);
  return b < n_tb - 1 ? b : n_tb - 1;
}

// Wave-wide unsigned min / max, returned in every lane: DPP moves reduce each
// row of 16 lanes (quad swaps, then rotations by 4 and 8), four lane reads
// combine the rows. No LDS traffic; every lane of the wave must be active.
template <bool MAX>
__device__ __forceinline__ unsigned wave_ext_u32(unsigned v) {
  auto f = [](unsigned a, unsigned b) { return MAX ? max(a, b) : min(a, b); };
  v = f(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = f(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = f(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror 4
  v = f(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror 8
  const unsigned a = f((unsigned)__builtin_amdgcn_readlane((int)v, 0), (unsigned)__builtin_amdgcn_readlane((int)v, 16));
  const unsigned b = f((unsigned)__builtin_amdgcn_readlane((int)v, 32), (unsigned)__builtin_amdgcn_readlane((int)v, 48));
  return f(a, b);
}
__device__ __forceinline__ unsigned wave_min_u32(unsigned v) { return wave_ext_u32<false>(v); }
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) { return wave_ext_u32<true>(v); }

// A DPP lane move of an fp32 value; a lane whose source lies outside its row
// (row shifts) reads 0 (bound_ctrl), so no zeroed destination is needed.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Wave-wide fp32 sum by the same DPP pattern (every lane active).
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x124>(v);
  v += dpp_f32<0x128>(v);
  auto at = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  return (at(0) + at(16)) + (at(32) + at(48));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(u32, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Eight bf16 gradients g times SiLU'(z) of eight bf16 pre-activations, each
// product rounded once to bf16.
__device__ __forceinline__ u32x4 dsilu_bf16x8(u32x4 g, u32x4 z) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float g0 = __uint_as_float(g[i] << 16), g1 = __uint_as_float(g[i] & 0xffff0000u);
    const float z0 = __uint_as_float(z[i] << 16), z1 = __uint_as_float(z[i] & 0xffff0000u);
    r[i] = pack_bf16x2(g0 * silu_grad(z0), g1 * silu_grad(z1));
  }
  return r;
}

// A raw buffer resource over [p, p + bytes) (bytes clamped to [0, 2^32 - 1];
// word 3 is the gfx9 raw-dword format). A load whose 32-bit byte offset runs
// past the end returns zeros without touching memory, so a tile's rows past
// the end of a sequence need no branch, no zero fill and no clamped index, and
// the per-lane offsets inside a tile stay fixed while the base moves.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_view(const void *p, long long bytes) {
  const long long n = bytes < 0 ? 0 : (bytes > 0xffffffffLL ? 0xffffffffLL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)(unsigned)n, 0x00020000);
}

// 16 bytes at byte offset off (all of it in the vector offset, which is the
// part the range check sees).
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}


}  // namespace dev
}  // namespace hstu
