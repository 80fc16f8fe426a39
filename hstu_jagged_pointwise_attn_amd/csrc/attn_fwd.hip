// Forward of the HSTU pointwise-attention core (HSTU blog, section 3 layer
// formula and 3.1: phi2 = SiLU in place of softmax; 3.2: rab^p and rab^t):
//   o_i = (1/N_max) * sum_{j visible} SiLU(q_i.k_j + rab_p[..] + rab_t[..]) v_j
// over the work list of the jagged tile scheduler. There is no row max and no
// normaliser, so key tiles contribute independently and nothing is rescaled.
//
// bf16 kernel (gfx950 MFMA, v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   workgroup = 4 waves = one (query tile of 128 rows, head); each wave owns
//   32 query rows whose Q fragments stay in registers for the whole key loop.
//   Per key tile of 64 keys: K is staged row-major in LDS and V transposed
//   (V^T, so that the A.V operand holds consecutive keys per lane); the wave
//   computes S^T = K Q^T, whose accumulator layout (lane = query row, 4
//   consecutive keys per register group) is directly the A operand of
//   O += P V once the keys of the contraction are taken in the matching
//   permuted order. The bias gather, SiLU and mask stay in registers; FULL
//   tiles skip the mask. A candidate's pair with itself is added per row after
//   the key loop.
// fp32 kernel (vector ALU, fp32 throughout) for the fp32 problems.
#include "hstu_internal.h"

namespace hstu {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef unsigned int u32;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(u16 x) { return __uint_as_float((u32)x << 16); }

__device__ __forceinline__ int frame_hi(int i, int P, int E) {
  return i < P ? P : (i < E ? i + 1 : E);
}

// SiLU(x) = x * sigmoid(x) with the hardware exp2 and reciprocal.
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
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

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int BM = kFwdBM, BN = kFwdBN;
  constexpr int KS = D / 32;     // k-steps of the K Q^T contraction
  constexpr int ND = D / 16;     // 16-column blocks of O
  constexpr int KPAD = D + 8;    // LDS row stride of K (elements)
  constexpr int VPAD = BN + 4;   // LDS row stride of V^T (elements)
  static_assert(BM == 128 && BN == 64, "wave layout assumes 4 waves x 32 rows, 64 keys");
  __shared__ __attribute__((aligned(16))) u16 Ks[BN * KPAD];
  __shared__ __attribute__((aligned(16))) u16 Vt[D * VPAD];
  __shared__ long long tsk[BN];

  const int H = a.H;
  const int unit = blockIdx.x;
  const int r = unit / H, h = unit % H;
  if (r >= a.hdr[kHdrNQ]) return;
  const QTile tile = a.tiles[r];
  const SeqDesc sd = a.desc[tile.b];
  const int nk = tile.nk, nf = tile.nf_nrows & 0xffff, nrows = tile.nf_nrows >> 16;
  const int row0 = tile.row0;
  const long long ld = (long long)H * D;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;

  const u16 *Q = (const u16 *)a.Q, *K = (const u16 *)a.K, *V = (const u16 *)a.V;
  const bool use_p = a.rab_p != nullptr;
  const bool use_t = a.rab_t != nullptr;

  // Rows of this lane in the S^T layout: local rows w*32 + nq*16 + lr.
  int hi_r[2], pos_r[2];
  long long ts_r[2];
  bool ok_r[2];
  bf16x8 qf[2][KS];
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int lrow = w * 32 + nq * 16 + lr;
    ok_r[nq] = lrow < nrows;
    const int fi = sd.q_frame0 + row0 + lrow;
    hi_r[nq] = ok_r[nq] ? frame_hi(fi, sd.P, sd.E) : 0;
    pos_r[nq] = fi < sd.E ? fi : sd.E;
    ts_r[nq] = (use_t && ok_r[nq]) ? a.ts_q[sd.q_base + row0 + lrow] : 0;
    const u16 *qp = Q + (long long)(sd.q_base + row0 + lrow) * ld + h * D + lg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = {0u, 0u, 0u, 0u};
      if (ok_r[nq]) v = *(const uint4 *)(qp + ks * 32);
      qf[nq][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 acc[2][ND];
#pragma unroll
  for (int nq = 0; nq < 2; ++nq)
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) acc[nq][nd] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Keys at or beyond kv_limit are never visible to any row of this tile and
  // are zero-filled instead of loaded.
  const int kv_limit = frame_hi(sd.q_frame0 + row0 + nrows - 1, sd.P, sd.E);

  for (int kt = 0; kt < nk; ++kt) {
    const int c0 = kt * BN;
    __syncthreads();
    for (int c = tid; c < BN * (D / 8); c += 256) {
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      uint4 v = {0u, 0u, 0u, 0u};
      if (c0 + row < kv_limit)
        v = *(const uint4 *)(K + (long long)(sd.kv_base + c0 + row) * ld + h * D + col);
      *(uint4 *)(Ks + row * KPAD + col) = v;
    }
    for (int c = tid; c < (BN / 4) * (D / 8); c += 256) {
      const int kq = c % (BN / 4), dc = c / (BN / 4);
      uint4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int row = kq * 4 + k;
        v[k] = uint4{0u, 0u, 0u, 0u};
        if (c0 + row < kv_limit)
          v[k] = *(const uint4 *)(V + (long long)(sd.kv_base + c0 + row) * ld + h * D + dc * 8);
      }
      const u32 *w0 = (const u32 *)&v[0], *w1 = (const u32 *)&v[1];
      const u32 *w2 = (const u32 *)&v[2], *w3 = (const u32 *)&v[3];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        const u32 x0 = (w0[e >> 1] >> sh) & 0xffffu, x1 = (w1[e >> 1] >> sh) & 0xffffu;
        const u32 x2 = (w2[e >> 1] >> sh) & 0xffffu, x3 = (w3[e >> 1] >> sh) & 0xffffu;
        uint2 o = {x0 | (x1 << 16), x2 | (x3 << 16)};
        *(uint2 *)(Vt + (dc * 8 + e) * VPAD + kq * 4) = o;
      }
    }
    if (tid < BN) tsk[tid] = (use_t && c0 + tid < kv_limit) ? a.ts_kv[sd.kv_base + c0 + tid] : 0;
    __syncthreads();

    // S^T = K Q^T : st[mk][nq] lane holds S(row nq*16+lr, key c0+mk*16+lg*4+i)
    f32x4 st[4][2];
#pragma unroll
    for (int mk = 0; mk < 4; ++mk)
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) st[mk][nq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mk = 0; mk < 4; ++mk) {
        const bf16x8 kf = *(const bf16x8 *)(Ks + (mk * 16 + lr) * KPAD + ks * 32 + lg * 8);
#pragma unroll
        for (int nq = 0; nq < 2; ++nq)
          st[mk][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[nq][ks], st[mk][nq], 0, 0, 0);
      }
    }

    // Bias, SiLU, mask, and the bf16 A operands of P V.
    const bool full = kt < nf;
    bf16x8 pa[2][2];
#pragma unroll
    for (int mk = 0; mk < 4; ++mk) {
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int jl = mk * 16 + lg * 4 + i;
          const int j = c0 + jl;
          float x = st[mk][nq][i];
          if (use_p) x += a.rab_p[pos_bucket(pos_r[nq] - j, a.n_pos)];
          if (use_t) x += a.rab_t[time_bucket(ts_r[nq] - tsk[jl], a.n_tb)];
          float p = silu_fast(x);
          if (!full && j >= hi_r[nq]) p = 0.f;
          pa[nq][mk >> 1][(mk & 1) * 4 + i] = (__bf16)p;
        }
      }
    }

    // O += P V with the contraction keys in the order of the S^T layout.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const u16 *vp = Vt + (nd * 16 + lr) * VPAD + kk * 32 + lg * 4;
        const uint2 v0 = *(const uint2 *)vp, v1 = *(const uint2 *)(vp + 16);
        const bf16x8 vb = __builtin_bit_cast(bf16x8, uint4{v0.x, v0.y, v1.x, v1.y});
#pragma unroll
        for (int nq = 0; nq < 2; ++nq)
          acc[nq][nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[nq][kk], vb, acc[nq][nd], 0, 0, 0);
      }
    }
  }

  // A candidate's pair with itself: o_i += SiLU(q_i.k_i + rab_p[0] + rab_t[0]) v_i.
  const bool any_cand = sd.q_frame0 + row0 + nrows - 1 >= sd.E;
  if (any_cand) {
    const u16 *Ksf = (const u16 *)a.Kself, *Vsf = (const u16 *)a.Vself;
    const float bias0 = (use_p ? a.rab_p[0] : 0.f) + (use_t ? a.rab_t[0] : 0.f);
    float as[2];
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
      const int lrow = w * 32 + nq * 16 + lr;
      const int fi = sd.q_frame0 + row0 + lrow;
      const bool cand = ok_r[nq] && fi >= sd.E;
      float part = 0.f;
      if (cand) {
        const u16 *kp = Ksf + (long long)(sd.self_base + fi - sd.E) * ld + h * D + lg * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 kv = *(const uint4 *)(kp + ks * 32);
          const u16 *ke = (const u16 *)&kv;
#pragma unroll
          for (int e = 0; e < 8; ++e) part += (float)qf[nq][ks][e] * bf2f(ke[e]);
        }
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      as[nq] = cand ? silu_fast(part + bias0) : 0.f;
    }
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float av = __shfl(as[nq], lg * 4 + i, 64);
        const int lrow = w * 32 + nq * 16 + lg * 4 + i;
        const int fi = sd.q_frame0 + row0 + lrow;
        if (lrow < nrows && fi >= sd.E) {
          const u16 *vp = Vsf + (long long)(sd.self_base + fi - sd.E) * ld + h * D + lr;
#pragma unroll
          for (int nd = 0; nd < ND; ++nd) acc[nq][nd][i] += av * bf2f(vp[nd * 16]);
        }
      }
    }
  }

  u16 *O = (u16 *)a.O;
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lrow = w * 32 + nq * 16 + lg * 4 + i;
      if (lrow < nrows) {
        u16 *op = O + (long long)(sd.q_base + row0 + lrow) * ld + h * D + lr;
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const __bf16 v = (__bf16)(acc[nq][nd][i] * a.inv_nmax);
          op[nd * 16] = __builtin_bit_cast(u16, v);
        }
      }
    }
  }
}

// fp32: 256 threads = 64 rows x 4 column slices of D/4; keys staged in LDS.
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(FwdArgs a) {
  constexpr int BN = kF32BN, DP = D / 4;
  static_assert(kF32BM == 64, "64 rows x 4 slices");
  __shared__ float Ks[BN][D];
  __shared__ float Vs[BN][D];
  __shared__ long long tsk[BN];

  const int H = a.H;
  const int unit = blockIdx.x;
  const int r = unit / H, h = unit % H;
  if (r >= a.hdr[kHdrNQ]) return;
  const QTile tile = a.tiles[r];
  const SeqDesc sd = a.desc[tile.b];
  const int nk = tile.nk, nrows = tile.nf_nrows >> 16, row0 = tile.row0;
  const long long ld = (long long)H * D;
  const int tid = threadIdx.x, lrow = tid >> 2, part = tid & 3;
  const float *Q = (const float *)a.Q, *K = (const float *)a.K, *V = (const float *)a.V;
  const bool use_p = a.rab_p != nullptr, use_t = a.rab_t != nullptr;

  const bool ok = lrow < nrows;
  const int fi = sd.q_frame0 + row0 + lrow;
  const int hi = ok ? frame_hi(fi, sd.P, sd.E) : 0;
  const int pos = fi < sd.E ? fi : sd.E;
  const long long tq = (use_t && ok) ? a.ts_q[sd.q_base + row0 + lrow] : 0;
  float q[DP], o[DP];
#pragma unroll
  for (int c = 0; c < DP; ++c) {
    q[c] = ok ? Q[(long long)(sd.q_base + row0 + lrow) * ld + h * D + part * DP + c] : 0.f;
    o[c] = 0.f;
  }
  const int kv_limit = frame_hi(sd.q_frame0 + row0 + nrows - 1, sd.P, sd.E);

  for (int kt = 0; kt < nk; ++kt) {
    const int c0 = kt * BN;
    __syncthreads();
    for (int c = tid; c < BN * D; c += 256) {
      const int row = c / D, col = c % D;
      const bool in = c0 + row < kv_limit;
      const long long g = (long long)(sd.kv_base + c0 + row) * ld + h * D + col;
      Ks[row][col] = in ? K[g] : 0.f;
      Vs[row][col] = in ? V[g] : 0.f;
    }
    if (tid < BN) tsk[tid] = (use_t && c0 + tid < kv_limit) ? a.ts_kv[sd.kv_base + c0 + tid] : 0;
    __syncthreads();
    const int jend = min(BN, kv_limit - c0);
    for (int jl = 0; jl < jend; ++jl) {
      const int j = c0 + jl;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) s = fmaf(q[c], Ks[jl][part * DP + c], s);
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      if (use_p) s += a.rab_p[pos_bucket(pos - j, a.n_pos)];
      if (use_t) s += a.rab_t[time_bucket(tq - tsk[jl], a.n_tb)];
      const float p = j < hi ? s / (1.0f + expf(-s)) : 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) o[c] = fmaf(p, Vs[jl][part * DP + c], o[c]);
    }
  }

  if (ok && fi >= sd.E) {
    const float *Ksf = (const float *)a.Kself, *Vsf = (const float *)a.Vself;
    const long long srow = (long long)(sd.self_base + fi - sd.E) * ld + h * D + part * DP;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < DP; ++c) s = fmaf(q[c], Ksf[srow + c], s);
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += (use_p ? a.rab_p[0] : 0.f) + (use_t ? a.rab_t[0] : 0.f);
    const float p = s / (1.0f + expf(-s));
#pragma unroll
    for (int c = 0; c < DP; ++c) o[c] = fmaf(p, Vsf[srow + c], o[c]);
  } else {
    // keep the shuffles above uniform across the four lanes of a row
  }
  if (ok) {
    float *O = (float *)a.O;
    const long long orow = (long long)(sd.q_base + row0 + lrow) * ld + h * D + part * DP;
#pragma unroll
    for (int c = 0; c < DP; ++c) O[orow + c] = o[c] * a.inv_nmax;
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdArgs &a, hipStream_t s) {
  if (a.units <= 0) return hipSuccess;
  switch (a.d) {
    case 32: hipLaunchKernelGGL(attn_fwd_bf16_kernel<32>, dim3(a.units), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, dim3(a.units), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, dim3(a.units), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const FwdArgs &a, hipStream_t s) {
  if (a.units <= 0) return hipSuccess;
  switch (a.d) {
    case 32: hipLaunchKernelGGL(attn_fwd_f32_kernel<32>, dim3(a.units), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3(a.units), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3(a.units), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hstu
