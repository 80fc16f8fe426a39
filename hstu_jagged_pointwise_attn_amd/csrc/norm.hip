// Per-token epilogue Y = Norm(X) * U over the full width D = H*d of a token
// (HSTU blog, section 3 layer formula: Norm(A(X)V(X)) * U(X)); Norm is none,
// LayerNorm (population variance, eps), or MTGR's Group LayerNorm (MTGR deep
// read, section 2: normalisation grouped by token source), read as per-token
// statistics with an affine (gamma_g, beta_g) chosen by the token's group.
// One wave per token; the row sits in registers, the mean and the variance are
// two wave reductions (the variance from the centred values).
#include "hstu_internal.h"
#include "device_common.h"
#include "../../include/hstu.h"

namespace hstu {
namespace {

typedef unsigned short u16;
typedef unsigned int u32;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the wave, returned in every lane: DPP moves add within each row of
// 16 lanes (quad swaps, then rotations by 4 and 8) and four lane reads add
// the rows, with no LDS round trips. Every lane of the wave must be active.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm 1,0,3,2
  v += dpp_mov<0x4E>(v);   // quad_perm 2,3,0,1
  v += dpp_mov<0x124>(v);  // row_ror 4
  v += dpp_mov<0x128>(v);  // row_ror 8
  auto lane = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  return (lane(0) + lane(16)) + (lane(32) + lane(48));
}

template <bool BF16>
struct Vec;
template <>
struct Vec<true> {
  static constexpr int N = 8;
  __device__ static void load(const void *p, long long off, float *x) {
    const uint4 v = *(const uint4 *)((const u16 *)p + off);
    const u32 *w = (const u32 *)&v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  __device__ static void unpack(const uint4 &v, float *x) {
    const u32 *w = (const u32 *)&v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  __device__ static void store(void *p, long long off, const float *x) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint4 v;
    u32 *w = (u32 *)&v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16x2 t;
      t[0] = (__bf16)x[2 * e];
      t[1] = (__bf16)x[2 * e + 1];
      w[e] = __builtin_bit_cast(u32, t);
    }
    *(uint4 *)((u16 *)p + off) = v;
  }
};
template <>
struct Vec<false> {
  static constexpr int N = 4;
  __device__ static void load(const void *p, long long off, float *x) {
    const float4 v = *(const float4 *)((const float *)p + off);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  __device__ static void unpack(const uint4 &v, float *x) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
  __device__ static void store(void *p, long long off, const float *x) {
    *(float4 *)((float *)p + off) = float4{x[0], x[1], x[2], x[3]};
  }
};

// N consecutive fp32 values of an affine row (gamma or beta), as 16-byte loads.
template <int N>
__device__ __forceinline__ void load_affine(const float *p, int c, float *x) {
#pragma unroll
  for (int e = 0; e < N; e += 4) {
    const float4 v = *(const float4 *)(p + c + e);
    x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
  }
}

// The token's group and its X and U rows are all requested before the first
// reduction, so one wave has its whole row in flight at once; gamma and beta
// (fp32, a few KB per group, L2-resident) are read as 16-byte vectors.
template <bool BF16, int MAXCH>
__global__ __launch_bounds__(256) void norm_fwd_kernel(NormArgs a) {
  using V = Vec<BF16>;
  constexpr int N = V::N;
  if (a.merge_ts && blockIdx.x == 0 && threadIdx.x == 0) {
    if ((unsigned)a.hdr[kHdrInlineTs] == a.epoch) atomicOr(&a.hdr[kHdrStatus], HSTU_DEV_BAD_TIMESTAMPS);
    a.hdr[kHdrInlineTs] = (int)~a.epoch;
  }
  const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63;
  const int D = a.D, nch = D / N;
  const long long row = t * D;
  int g = a.mode == HSTU_NORM_GLN ? (int)a.group[t] : 0;
  float x[MAXCH][N], u[MAXCH][N];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < MAXCH; ++k) {
    const int ch = lane + 64 * k;
    if (ch < nch) {
      V::load(a.X, row + ch * N, x[k]);
      V::load(a.U, row + ch * N, u[k]);
#pragma unroll
      for (int e = 0; e < N; ++e) s += x[k][e];
    }
  }
  float mean = 0.f, rstd = 1.f;
  if (a.mode != HSTU_NORM_NONE) {
    mean = wave_sum(s) / (float)D;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < MAXCH; ++k) {
      const int ch = lane + 64 * k;
      if (ch < nch) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const float c = x[k][e] - mean;
          v += c * c;
        }
      }
    }
    const float var = wave_sum(v) / (float)D;
    rstd = 1.0f / sqrtf(var + a.eps);
    if (g >= a.n_groups) {
      if (lane == 0) atomicOr(&a.hdr[kHdrStatus], HSTU_DEV_BAD_GROUP);
      g = -1;
    }
  }
  const bool norm = a.mode != HSTU_NORM_NONE;
  const float *gm = (norm && g >= 0 && a.gamma) ? a.gamma + (long long)g * D : nullptr;
  const float *bt = (norm && g >= 0 && a.beta) ? a.beta + (long long)g * D : nullptr;
#pragma unroll
  for (int k = 0; k < MAXCH; ++k) {
    const int ch = lane + 64 * k;
    if (ch < nch) {
      float gam[N], bet[N], y[N];
#pragma unroll
      for (int e = 0; e < N; ++e) gam[e] = 1.f, bet[e] = 0.f;
      if (gm) load_affine<N>(gm, ch * N, gam);
      if (bt) load_affine<N>(bt, ch * N, bet);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float n = norm ? (x[k][e] - mean) * rstd * gam[e] + bet[e] : x[k][e];
        y[e] = n * u[k][e];
      }
      V::store(a.Y, row + ch * N, y);
    }
  }
  if (lane == 0 && a.mean) {
    a.mean[t] = mean;
    a.rstd[t] = rstd;
  }
}

template <bool BF16>
hipError_t norm_fwd_dispatch(const NormArgs &a, hipStream_t s) {
  const int nch = a.D / Vec<BF16>::N;
  const dim3 grid((unsigned)((a.T + 3) / 4));
  if (nch <= 64) hipLaunchKernelGGL((norm_fwd_kernel<BF16, 1>), grid, dim3(256), 0, s, a);
  else if (nch <= 128) hipLaunchKernelGGL((norm_fwd_kernel<BF16, 2>), grid, dim3(256), 0, s, a);
  else if (nch <= 256) hipLaunchKernelGGL((norm_fwd_kernel<BF16, 4>), grid, dim3(256), 0, s, a);
  else if (nch <= 512) hipLaunchKernelGGL((norm_fwd_kernel<BF16, 8>), grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Backward of Y = Norm(X) * U for one token per wave:
//   dU = n * dY, dN = dY * u,
//   LN/GLN: xhat = (x - mean) * rstd, g = dN * gamma,
//           dX = rstd * (g - mean(g) - xhat * mean(g * xhat)),
//           dgamma += dN * xhat, dbeta += dN   (row of the token's group)
//   NONE:   dX = dN.
// Each wave walks a contiguous run of tokens and keeps the affine gradients
// of the current group in registers, flushing them only when the group
// changes and at the end of its run: with `partial` into the workgroup's
// [2][G][D] rows in LDS (written out per workgroup and reduced by a second
// kernel), else with global atomics.
template <bool BF16, int MAXCH, bool ZU>
__global__ __launch_bounds__(256) void norm_bwd_kernel(NormBwdArgs a) {
  using V = Vec<BF16>;
  constexpr int N = V::N;
  extern __shared__ float s_aff[];  // [2][G][D] with `partial`
  const int lane = threadIdx.x & 63;
  const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long t0 = wave * a.tokens_per_wave;
  const bool lds_acc = a.partial != nullptr;
  const int GD = a.n_groups * a.D;
  if (lds_acc) {
    for (int i = threadIdx.x; i < 2 * GD; i += 256) s_aff[i] = 0.f;
    __syncthreads();
  } else if (t0 >= a.T) {
    return;
  }
  const long long t1 = min(a.T, t0 + a.tokens_per_wave);
  const int D = a.D, nch = D / N;
  const bool affine = a.mode != HSTU_NORM_NONE && (a.dgamma || a.dbeta);
  float dg[MAXCH][N], db[MAXCH][N];
#pragma unroll
  for (int k = 0; k < MAXCH; ++k)
#pragma unroll
    for (int e = 0; e < N; ++e) dg[k][e] = db[k][e] = 0.f;
  int gcur = -1;
  auto flush = [&](int g) __attribute__((always_inline)) {
    if (g < 0) return;
#pragma unroll
    for (int k = 0; k < MAXCH; ++k) {
      const int ch = lane + 64 * k;
      if (ch < nch) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const long long c = (long long)g * D + ch * N + e;
          if (lds_acc) {
            atomicAdd(&s_aff[c], dg[k][e]);
            atomicAdd(&s_aff[GD + c], db[k][e]);
          } else {
            if (a.dgamma) atomicAdd(a.dgamma + c, dg[k][e]);
            if (a.dbeta) atomicAdd(a.dbeta + c, db[k][e]);
          }
          dg[k][e] = db[k][e] = 0.f;
        }
      }
    }
  };
  // The next token's rows (16-byte chunks) and statistics are requested
  // before the current one is computed, so a wave keeps one token in flight
  // (rows of up to 16 chunks per lane; wider rows would spill).
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr bool PREFETCH = MAXCH <= 2;
  constexpr int RC = PREFETCH ? MAXCH : 1;
  constexpr bool fz = BF16 && ZU;  // a layer's fused SiLU' on dU
  uint4 rx[RC], rdy[RC], ru[RC], rz[fz ? RC : 1];
  float nmean = 0.f, nrstd = 1.f;
  int ngrp = 0;
  auto fetch = [&](long long t) __attribute__((always_inline)) {
    const long long row = t * D;
#pragma unroll
    for (int k = 0; k < RC; ++k) {
      const int ch = lane + 64 * k;
      if (ch < nch) {
        const long long off = (row + ch * N) * ESZ;
        rx[k] = *(const uint4 *)((const char *)a.X + off);
        rdy[k] = *(const uint4 *)((const char *)a.dY + off);
        ru[k] = *(const uint4 *)((const char *)a.U + off);
        if constexpr (fz) rz[k] = *(const uint4 *)((const char *)a.zu + (t * a.ldu + ch * N) * ESZ);
      }
    }
    if (a.mode != HSTU_NORM_NONE) {
      nmean = a.mean[t];
      nrstd = a.rstd[t];
      if (a.mode == HSTU_NORM_GLN) ngrp = a.group[t];
    }
  };
  if constexpr (PREFETCH) {
    if (t0 < t1) fetch(t0);
  }
  for (long long t = t0; t < t1; ++t) {
    const long long row = t * D;
    float x[MAXCH][N], dy[MAXCH][N], u[MAXCH][N];
    float mean = 1.f, rstd = 1.f;
    int grp_t = 0;
    if constexpr (PREFETCH) {
#pragma unroll
      for (int k = 0; k < RC; ++k) {
        const int ch = lane + 64 * k;
        if (ch < nch) {
          V::unpack(rx[k], x[k]);
          V::unpack(rdy[k], dy[k]);
          V::unpack(ru[k], u[k]);
        }
      }
      mean = nmean;
      rstd = nrstd;
      grp_t = ngrp;
    } else {
#pragma unroll
      for (int k = 0; k < MAXCH; ++k) {
        const int ch = lane + 64 * k;
        if (ch < nch) {
          V::load(a.X, row + ch * N, x[k]);
          V::load(a.dY, row + ch * N, dy[k]);
          V::load(a.U, row + ch * N, u[k]);
        }
      }
      if (a.mode != HSTU_NORM_NONE) {
        mean = a.mean[t];
        rstd = a.rstd[t];
        if (a.mode == HSTU_NORM_GLN) grp_t = a.group[t];
      }
    }
    // A layer's fused SiLU': this token's pre-activation of the U block
    // (requested with the token's rows when they are prefetched).
    float zz[MAXCH][N];
    if constexpr (fz) {
#pragma unroll
      for (int k = 0; k < MAXCH; ++k) {
        const int ch = lane + 64 * k;
        if (ch < nch) {
          if constexpr (PREFETCH) V::unpack(rz[k], zz[k]);
          else V::load(a.zu, t * a.ldu + ch * N, zz[k]);
        }
      }
    }
    auto store_du = [&](int k, int ch, float *du) __attribute__((always_inline)) {
      if constexpr (fz) {
#pragma unroll
        for (int e = 0; e < N; ++e) du[e] *= dev::silu_grad(zz[k][e]);
        V::store(a.dU, t * a.ldu + ch * N, du);
      } else {
        V::store(a.dU, t * D + ch * N, du);
      }
    };
    if constexpr (PREFETCH) {
      if (t + 1 < t1) fetch(t + 1);
    }
    if (a.mode == HSTU_NORM_NONE) {
#pragma unroll
      for (int k = 0; k < MAXCH; ++k) {
        const int ch = lane + 64 * k;
        if (ch < nch) {
          float du[N], dx[N];
#pragma unroll
          for (int e = 0; e < N; ++e) {
            du[e] = x[k][e] * dy[k][e];
            dx[e] = dy[k][e] * u[k][e];
          }
          store_du(k, ch, du);
          V::store(a.dX, row + ch * N, dx);
        }
      }
      continue;
    }
    int g = 0;
    if (a.mode == HSTU_NORM_GLN) {
      g = grp_t;
      if (g >= a.n_groups) g = -1;
    }
    const float *gm = (g >= 0 && a.gamma) ? a.gamma + (long long)g * D : nullptr;
    const float *bt = (g >= 0 && a.beta) ? a.beta + (long long)g * D : nullptr;
    if (affine && g != gcur) {
      flush(gcur);
      gcur = g;
    }
    float s1 = 0.f, s2 = 0.f;
    float xh[MAXCH][N], gh[MAXCH][N];
#pragma unroll
    for (int k = 0; k < MAXCH; ++k) {
      const int ch = lane + 64 * k;
      if (ch < nch) {
        float du[N], gam[N], bet[N];
#pragma unroll
        for (int e = 0; e < N; ++e) gam[e] = 1.f, bet[e] = 0.f;
        if (gm) load_affine<N>(gm, ch * N, gam);
        if (bt) load_affine<N>(bt, ch * N, bet);
#pragma unroll
        for (int e = 0; e < N; ++e) {
          xh[k][e] = (x[k][e] - mean) * rstd;
          const float n = xh[k][e] * gam[e] + bet[e];
          du[e] = n * dy[k][e];
          const float dn = dy[k][e] * u[k][e];
          if (affine && g >= 0) {
            dg[k][e] += dn * xh[k][e];
            db[k][e] += dn;
          }
          gh[k][e] = dn * gam[e];
          s1 += gh[k][e];
          s2 += gh[k][e] * xh[k][e];
        }
        store_du(k, ch, du);
      }
    }
    const float m1 = wave_sum(s1) / (float)D, m2 = wave_sum(s2) / (float)D;
#pragma unroll
    for (int k = 0; k < MAXCH; ++k) {
      const int ch = lane + 64 * k;
      if (ch < nch) {
        float dx[N];
#pragma unroll
        for (int e = 0; e < N; ++e) dx[e] = rstd * (gh[k][e] - m1 - xh[k][e] * m2);
        V::store(a.dX, row + ch * N, dx);
      }
    }
  }
  if (affine) flush(gcur);
  if (lds_acc) {
    __syncthreads();
    float *out = a.partial + (long long)blockIdx.x * 2 * GD;
    for (int i = threadIdx.x; i < 2 * GD; i += 256) out[i] = s_aff[i];
  }
}

template <bool BF16, bool ZU>
hipError_t norm_bwd_dispatch(const NormBwdArgs &a, hipStream_t s) {
  const int nch = a.D / Vec<BF16>::N;
  const dim3 grid((unsigned)norm_bwd_blocks(a.T, a.tokens_per_wave));
  const size_t lds = a.partial ? 2 * sizeof(float) * a.n_groups * a.D : 0;
  if (nch <= 64) hipLaunchKernelGGL((norm_bwd_kernel<BF16, 1, ZU>), grid, dim3(256), lds, s, a);
  else if (nch <= 128) hipLaunchKernelGGL((norm_bwd_kernel<BF16, 2, ZU>), grid, dim3(256), lds, s, a);
  else if (nch <= 256) hipLaunchKernelGGL((norm_bwd_kernel<BF16, 4, ZU>), grid, dim3(256), lds, s, a);
  else if (nch <= 512) hipLaunchKernelGGL((norm_bwd_kernel<BF16, 8, ZU>), grid, dim3(256), lds, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Column sums of partial [blocks][2 GD]: a workgroup takes 64 columns, its
// sixteen waves every sixteenth block row (eight loads in flight each), and
// LDS adds the sixteen.
__global__ __launch_bounds__(1024) void norm_affine_reduce_kernel(const float *partial, long long blocks, int GD,
                                                                  float *dgamma, float *dbeta) {
  __shared__ float s_sum[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  float acc = 0.f;
  if (col < 2 * GD) {
#pragma unroll 8
    for (long long b = w; b < blocks; b += 16) acc += partial[b * 2 * GD + col];
  }
  s_sum[w][lane] = acc;
  __syncthreads();
  if (w == 0 && col < 2 * GD) {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v += s_sum[i][lane];
    if (col < GD) {
      if (dgamma) dgamma[col] = v;
    } else if (dbeta) {
      dbeta[col - GD] = v;
    }
  }
}

__global__ void fill_f32_kernel(float *p, long long n, float v) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_norm_fwd(const NormArgs &a, bool bf16, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return bf16 ? norm_fwd_dispatch<true>(a, s) : norm_fwd_dispatch<false>(a, s);
}

}  // namespace hstu

namespace hstu {

long long norm_bwd_blocks(long long T, int tokens_per_wave) {
  const long long waves = (T + tokens_per_wave - 1) / tokens_per_wave;
  return (waves + 3) / 4;
}

hipError_t launch_norm_bwd(const NormBwdArgs &a, bool bf16, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (bf16) return a.zu ? norm_bwd_dispatch<true, true>(a, s) : norm_bwd_dispatch<true, false>(a, s);
  return norm_bwd_dispatch<false, false>(a, s);
}

hipError_t launch_norm_affine_reduce(const float *partial, long long blocks, int GD, float *dgamma, float *dbeta,
                                     hipStream_t s) {
  if (GD <= 0 || blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_affine_reduce_kernel, dim3((unsigned)((2 * GD + 63) / 64)), dim3(1024), 0, s, partial,
                     blocks, GD, dgamma, dbeta);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float *p, long long n, float v, hipStream_t s) {
  if (n <= 0 || !p) return hipSuccess;
  const long long blocks = min((n + 255) / 256, 4096LL);
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace hstu
