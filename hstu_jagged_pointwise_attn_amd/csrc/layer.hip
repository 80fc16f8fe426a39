// Elementwise steps of a full HSTU layer around the attention core (HSTU
// blog, section 3, the layer formula: U, V, Q, K from phi1(f1(X)) with
// phi1 = SiLU, and O = f2(Norm(A V) * U)). The projections f1 and f2 are
// library GEMMs (gemm.cpp); these kernels are the HBM-bound passes between
// them:
//   silu_split   Z [T, 4D] -> U, V, Q, K [T, D] (SiLU of the four column
//                blocks, in that order)
//   dsilu        dZ = [dU | dV | dQ | dK] * SiLU'(Z), and optionally the
//                column sums of dZ (the bias gradient of f1)
//   colsum       column sums of a [T, n] matrix (the bias gradient of f2)
// Every wave load is 1 KiB of one row (64 lanes x 16 bytes, coalesced).
#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr int kThreads = 256;  // 4 waves

typedef unsigned short u16;

// VW elements of one 16-byte vector (bf16: 8, fp32: 4), widened to fp32.
template <bool BF16>
struct Vec {
  static constexpr int VW = BF16 ? 8 : 4;
  float v[VW];
  __device__ __forceinline__ void load(const void *p, long long elem) {
    const uint4 r = *reinterpret_cast<const uint4 *>(static_cast<const char *>(p) + elem * (BF16 ? 2 : 4));
    const unsigned w[4] = {r.x, r.y, r.z, r.w};
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
    }
  }
  __device__ __forceinline__ void store(void *p, long long elem) const {
    uint4 r;
    if constexpr (BF16) {
      unsigned w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned lo = __builtin_bit_cast(u16, (__bf16)v[2 * i]);
        const unsigned hi = __builtin_bit_cast(u16, (__bf16)v[2 * i + 1]);
        w[i] = lo | (hi << 16);
      }
      r = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      r = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    }
    *reinterpret_cast<uint4 *>(static_cast<char *>(p) + elem * (BF16 ? 2 : 4)) = r;
  }
};

// 1 / (1 + e^-z) with the hardware reciprocal (1 ulp): SiLU and its
// derivative need no IEEE-exact division at bf16 or fp32 tolerance.
__device__ __forceinline__ float sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Work split shared by the kernels. A block is 4 waves over 64 consecutive
// column vectors (a chunk) of a 16-row strip: wave w takes kRPT consecutive
// rows, all of whose loads are issued before any use. Block b covers chunk
// b % nchunk, so consecutive blocks read whole rows. Without column sums,
// block b does strip b / nchunk. With column sums, the blocks of row group
// g = b / nchunk (G groups) loop over strips g, g + G, ... and write the
// group's column sums to partial[g][...]; a second kernel adds the G rows of
// partial. (One atomic per column and block would serialise thousands of
// updates on each address.)
constexpr int kRPT = 4;
constexpr int kStripRows = 4 * kRPT;

struct Work {
  long long strip0, stride, nstrips;  // strips this block visits: strip0, strip0 + stride, ...
  long long grp;                      // row group (sums) / strip (no sums)
  int cv;                             // column vector of this lane
  bool live;                          // cv inside the matrix
};

__device__ __forceinline__ Work work_of(long long T, int nvec, bool sums) {
  const int nchunk = (nvec + 63) / 64;
  Work w;
  w.grp = blockIdx.x / nchunk;
  const int chunk = blockIdx.x - (int)(w.grp * nchunk);
  w.cv = chunk * 64 + (threadIdx.x & 63);
  w.live = w.cv < nvec;
  w.nstrips = (T + kStripRows - 1) / kStripRows;
  w.strip0 = w.grp;
  w.stride = sums ? gridDim.x / nchunk : w.nstrips;
  return w;
}

// Sums acc[VW] over the block's 4 waves and stores it as partial row `grp`
// (columns cv * VW ...; n columns per row).
template <int VW>
__device__ __forceinline__ void block_colsum_store(float (&acc)[VW], float *partial, long long grp, int n, int cv,
                                                   bool live) {
  __shared__ float red[4][64][VW + 1];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < VW; ++i) red[w][lane][i] = acc[i];
  __syncthreads();
  if (w == 0 && live) {
#pragma unroll
    for (int i = 0; i < VW; ++i)
      partial[grp * n + (long long)cv * VW + i] = red[0][lane][i] + red[1][lane][i] + red[2][lane][i] + red[3][lane][i];
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) silu_split_kernel(const void *__restrict__ Z, long long T, int D,
                                                              void *U, void *V, void *Q, void *K) {
  using Vt = Vec<BF16>;
  const int nvec = 4 * D / Vt::VW, bvec = D / Vt::VW;
  const Work wk = work_of(T, nvec, false);
  if (!wk.live) return;
  const int blk = wk.cv / bvec, col = (wk.cv - blk * bvec) * Vt::VW;
  void *out = blk == 0 ? U : blk == 1 ? V : blk == 2 ? Q : K;
  const long long rb = wk.strip0 * kStripRows + (threadIdx.x >> 6) * kRPT;
  Vt z[kRPT];
#pragma unroll
  for (int i = 0; i < kRPT; ++i)
    if (rb + i < T) z[i].load(Z, (rb + i) * 4 * D + (long long)wk.cv * Vt::VW);
#pragma unroll
  for (int i = 0; i < kRPT; ++i) {
    if (rb + i < T) {
#pragma unroll
      for (int e = 0; e < Vt::VW; ++e) z[i].v[e] = z[i].v[e] * sigmoid(z[i].v[e]);
      z[i].store(out, (rb + i) * D + col);
    }
  }
}

template <bool BF16, bool SUM>
__global__ void __launch_bounds__(kThreads) dsilu_kernel(const void *__restrict__ Z, const void *dU, const void *dV,
                                                         const void *dQ, const void *dK, long long T, int D,
                                                         void *dZ, float *partial) {
  using Vt = Vec<BF16>;
  const int nvec = 4 * D / Vt::VW, bvec = D / Vt::VW;
  const Work wk = work_of(T, nvec, SUM);
  float acc[Vt::VW];
#pragma unroll
  for (int e = 0; e < Vt::VW; ++e) acc[e] = 0.f;
  if (wk.live) {
    const int blk = wk.cv / bvec, col = (wk.cv - blk * bvec) * Vt::VW;
    const void *g = blk == 0 ? dU : blk == 1 ? dV : blk == 2 ? dQ : dK;
    for (long long st = wk.strip0; st < wk.nstrips; st += wk.stride) {
      const long long rb = st * kStripRows + (threadIdx.x >> 6) * kRPT;
      Vt z[kRPT], dy[kRPT];
#pragma unroll
      for (int i = 0; i < kRPT; ++i) {
        if (rb + i < T) {
          z[i].load(Z, (rb + i) * 4 * D + (long long)wk.cv * Vt::VW);
          dy[i].load(g, (rb + i) * D + col);
        }
      }
#pragma unroll
      for (int i = 0; i < kRPT; ++i) {
        if (rb + i < T) {
#pragma unroll
          for (int e = 0; e < Vt::VW; ++e) {
            const float zz = z[i].v[e], s = sigmoid(zz);
            float v = dy[i].v[e] * s * (1.0f + zz * (1.0f - s));
            // the bias gradient sums the stored dZ (rounded to bf16), as the
            // weight-gradient GEMM sees it
            if constexpr (BF16) v = (float)(__bf16)v;
            dy[i].v[e] = v;
            if constexpr (SUM) acc[e] += v;
          }
          dy[i].store(dZ, (rb + i) * 4 * D + (long long)wk.cv * Vt::VW);
        }
      }
    }
  }
  if constexpr (SUM) block_colsum_store<Vt::VW>(acc, partial, wk.grp, 4 * D, wk.cv, wk.live);
}

// Row-group column sums of M [T, n] into partial [G, n]: 16-byte vectors when
// n is a multiple of the vector width, one element per lane otherwise.
template <bool BF16, bool VEC>
__global__ void __launch_bounds__(kThreads) colsum_kernel(const void *__restrict__ M, long long T, int n,
                                                          float *partial) {
  constexpr int VW = VEC ? Vec<BF16>::VW : 1;
  const int nvec = n / VW;
  const Work wk = work_of(T, nvec, true);
  float acc[VW];
#pragma unroll
  for (int i = 0; i < VW; ++i) acc[i] = 0.f;
  if (wk.live) {
    for (long long st = wk.strip0; st < wk.nstrips; st += wk.stride) {
      const long long rb = st * kStripRows + (threadIdx.x >> 6) * kRPT;
      if constexpr (VEC) {
        Vec<BF16> x[kRPT];
#pragma unroll
        for (int i = 0; i < kRPT; ++i)
          if (rb + i < T) x[i].load(M, (rb + i) * n + (long long)wk.cv * VW);
#pragma unroll
        for (int i = 0; i < kRPT; ++i)
          if (rb + i < T) {
#pragma unroll
            for (int e = 0; e < VW; ++e) acc[e] += x[i].v[e];
          }
      } else {
        float x[kRPT];
#pragma unroll
        for (int i = 0; i < kRPT; ++i) {
          const long long e = (rb + i) * n + wk.cv;
          x[i] = rb + i >= T ? 0.f
                 : BF16     ? __uint_as_float((unsigned)static_cast<const u16 *>(M)[e] << 16)
                            : static_cast<const float *>(M)[e];
        }
#pragma unroll
        for (int i = 0; i < kRPT; ++i) acc[0] += x[i];
      }
    }
  }
  block_colsum_store<VW>(acc, partial, wk.grp, n, wk.cv, wk.live);
}

// out[c] = sum over g < G of partial[g][c] (overwrites out); 16 waves per
// block each add G/16 rows of a 64-column slab.
constexpr int kReduceThreads = 1024;
__global__ void __launch_bounds__(kReduceThreads) colsum_reduce_kernel(const float *__restrict__ partial, int G,
                                                                       int n, float *out) {
  __shared__ float red[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (c < n) {
#pragma unroll 8
    for (int g = w; g < G; g += 16) s += partial[(long long)g * n + c];
  }
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && c < n) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += red[i][lane];
    out[c] = t;
  }
}

// out[i] = sum over s < ns of slices[s * n + i], four consecutive floats per
// thread (n is a multiple of 4 and the pointers 16-byte aligned).
__global__ void __launch_bounds__(kThreads) sum_slices_kernel(const float *__restrict__ slices, int ns, long long n4,
                                                              float *out) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n4) return;
  const float4 *src = reinterpret_cast<const float4 *>(slices);
  float4 acc = src[i];
  for (int k = 1; k < ns; ++k) {
    const float4 v = src[(long long)k * n4 + i];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  reinterpret_cast<float4 *>(out)[i] = acc;
}

// Row groups of a column-sum launch: enough blocks to fill the chip (about
// 2048 with the column chunks), at most kColsumGroups, at most one per strip.
int groups_for(long long T, int nvec) {
  const long long nstrips = (T + kStripRows - 1) / kStripRows;
  const int nchunk = (nvec + 63) / 64;
  long long g = 2048 / nchunk;
  g = g < 64 ? 64 : g > kColsumGroups ? kColsumGroups : g;
  return (int)(g < nstrips ? g : nstrips);
}

// Blocks of a launch: (strips, or the row groups when summing) x (column
// chunks of 64 vectors); 0 when the grid would exceed 2^32 work-items (the
// launchers then refuse).
unsigned grid_for(long long T, int nvec, bool sums) {
  const long long groups = sums ? groups_for(T, nvec) : (T + kStripRows - 1) / kStripRows;
  const long long blocks = groups * ((nvec + 63) / 64);
  return blocks * kThreads >= (1LL << 32) ? 0u : (unsigned)blocks;
}

}  // namespace

hipError_t launch_silu_split(const void *Z, long long T, int D, bool bf16, void *U, void *V, void *Q, void *K,
                             hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int vw = bf16 ? 8 : 4;
  const unsigned g = grid_for(T, 4 * D / vw, false);
  if (!g) return hipErrorInvalidConfiguration;
  if (bf16) hipLaunchKernelGGL(silu_split_kernel<true>, dim3(g), dim3(kThreads), 0, s, Z, T, D, U, V, Q, K);
  else hipLaunchKernelGGL(silu_split_kernel<false>, dim3(g), dim3(kThreads), 0, s, Z, T, D, U, V, Q, K);
  return hipGetLastError();
}

hipError_t launch_dsilu(const void *Z, const void *dU, const void *dV, const void *dQ, const void *dK, long long T,
                        int D, bool bf16, void *dZ, float *partial, float *db, hipStream_t s) {
  if (T <= 0) return db ? launch_fill_f32(db, 4LL * D, 0.f, s) : hipSuccess;
  const int vw = bf16 ? 8 : 4;
  const unsigned g = grid_for(T, 4 * D / vw, db != nullptr);
  if (!g) return hipErrorInvalidConfiguration;
#define HSTU_DSILU(B, S) \
  hipLaunchKernelGGL((dsilu_kernel<B, S>), dim3(g), dim3(kThreads), 0, s, Z, dU, dV, dQ, dK, T, D, dZ, partial)
  if (bf16) {
    if (db) HSTU_DSILU(true, true);
    else HSTU_DSILU(true, false);
  } else {
    if (db) HSTU_DSILU(false, true);
    else HSTU_DSILU(false, false);
  }
#undef HSTU_DSILU
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !db) return e;
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((4 * D + 63) / 64), dim3(kReduceThreads), 0, s, partial,
                     groups_for(T, 4 * D / vw), 4 * D, db);
  return hipGetLastError();
}

hipError_t launch_sum_slices(const float *slices, int nslices, long long n, float *out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 4 || reinterpret_cast<uintptr_t>(slices) % 16 || reinterpret_cast<uintptr_t>(out) % 16 || nslices < 1)
    return hipErrorInvalidValue;
  const long long n4 = n / 4;
  hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, slices,
                     nslices, n4, out);
  return hipGetLastError();
}

hipError_t launch_colsum(const void *M, long long T, int n, bool bf16, float *partial, float *out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (T <= 0) return launch_fill_f32(out, n, 0.f, s);
  const int vw = bf16 ? 8 : 4;
  const bool vec = n % vw == 0 && reinterpret_cast<uintptr_t>(M) % 16 == 0;
  const unsigned g = grid_for(T, vec ? n / vw : n, true);
  if (!g) return hipErrorInvalidConfiguration;
  if (bf16) {
    if (vec) hipLaunchKernelGGL((colsum_kernel<true, true>), dim3(g), dim3(kThreads), 0, s, M, T, n, partial);
    else hipLaunchKernelGGL((colsum_kernel<true, false>), dim3(g), dim3(kThreads), 0, s, M, T, n, partial);
  } else {
    if (vec) hipLaunchKernelGGL((colsum_kernel<false, true>), dim3(g), dim3(kThreads), 0, s, M, T, n, partial);
    else hipLaunchKernelGGL((colsum_kernel<false, false>), dim3(g), dim3(kThreads), 0, s, M, T, n, partial);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((n + 63) / 64), dim3(kReduceThreads), 0, s, partial,
                     groups_for(T, vec ? n / vw : n), n, out);
  return hipGetLastError();
}

}  // namespace hstu
