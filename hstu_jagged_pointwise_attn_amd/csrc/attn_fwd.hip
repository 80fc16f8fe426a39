// Forward of the HSTU pointwise-attention core (HSTU blog, section 3 layer
// formula and 3.1: phi2 = SiLU in place of softmax; 3.2: rab^p and rab^t):
//   o_i = (1/N_max) * sum_{j visible} SiLU(q_i.k_j + rab_p[..] + rab_t[..]) v_j
// over the work list of the jagged tile scheduler. There is no row max and no
// normaliser, so key tiles contribute independently and nothing is rescaled.
//
// bf16 kernel (gfx950 MFMA, v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   workgroup = 4 waves = one (query tile of 128 rows, head); each wave owns
//   32 query rows whose Q fragments stay in registers for the whole key loop.
//   Key tiles of 64 keys are double-buffered in LDS (row-major K and V, the
//   next tile prefetched into registers while the current one is computed,
//   one barrier per tile). The wave computes S^T = bias + K Q^T with the
//   accumulator initialised from an LDS window of rab_p; that accumulator
//   layout (lane = query row, 4 consecutive keys per register group) is
//   directly the A operand of O += P V once the keys of the contraction are
//   taken in the matching permuted order, and the V operand comes from the
//   row-major tile through gfx950's transposing LDS read. SiLU, rab_t and the
//   mask stay in registers; FULL tiles skip the mask. A candidate's pair with
//   itself is added per row after the key loop; O leaves through LDS as
//   16-byte rows.
// fp32 kernel (vector ALU, fp32 throughout) for the fp32 problems.
#include "hstu_internal.h"
#include "../../include/hstu.h"
#include "device_common.h"
#include "sched_common.h"

namespace hstu {
namespace {

using namespace dev;

// One key tile of K and V (and its rab_p window entry and key timestamp)
// held in registers between its global load and its LDS store.
template <int NCH>
struct TilePrefetch {
  u32x4 k[NCH], v[NCH];
  float r;
  long long t;
  unsigned off[NCH];  // byte offset of this thread's chunks inside a tile (fixed)
};

// Per-workgroup constants of the key loop.
struct FwdTileCtx {
  const u16 *K, *V;
  const float *rab_p;
  const int64_t *ts_kv;
  long long ld;
  int kv_base, kv_limit, pos_max, n_pos, tid;
};

template <int D, int BN, bool USE_P, bool USE_T, int NCH>
__device__ __forceinline__ void fwd_load_tile(TilePrefetch<NCH> &pf, const FwdTileCtx &c, int t) {
  constexpr int WIN = kFwdBM + BN;
  const int c0 = t * BN;
  // keys past kv_limit (seen by no row here) fall outside the buffers and load as zeros
  const long long rb = (long long)(c.kv_base + c0) * c.ld;
  const long long nb = (long long)(c.kv_limit - c0) * c.ld * 2;
  const __amdgpu_buffer_rsrc_t kr = buf_view(c.K + rb, nb), vr = buf_view(c.V + rb, nb);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    pf.k[i] = buf_load16(kr, pf.off[i]);
    pf.v[i] = buf_load16(vr, pf.off[i]);
  }
  if (USE_P && c.tid < WIN) pf.r = c.rab_p[pos_bucket(c.pos_max - c0 - c.tid, c.n_pos)];
  // key times by the last wave (waves 0-2 stage the rab_p window)
  if (USE_T && c.tid >= 256 - BN) pf.t = c.ts_kv[c.kv_base + min(c0 + c.tid - (256 - BN), c.kv_limit - 1)];
}

template <int D, int BN, bool USE_P, bool USE_T, int NCH>
__device__ __forceinline__ void fwd_store_tile(const TilePrefetch<NCH> &pf, int tid, u16 *Kb, u16 *Vb,
                                               float *rw, unsigned *tk, unsigned *tst, long long t_ref,
                                               bool &bad_t) {
  constexpr int CH = D / 8, WIN = kFwdBM + BN, KST = D + 16, VST = D + 16;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int chunk = tid + c * 256;
    const int row = chunk / CH, col = (chunk % CH) * 8;
    *(u32x4 *)(Kb + row * KST + col) = pf.k[c];
    *(u32x4 *)(Vb + row * VST + col) = pf.v[c];
  }
  if (USE_P && tid < WIN) rw[tid] = pf.r;
  if (USE_T && tid >= 256 - BN) {  // exactly the last wave
    const int j = tid - (256 - BN);
    const long long dk = pf.t - t_ref;
    bad_t |= dk < -2147483648LL || dk > 2147483647LL;
    const unsigned u = (unsigned)(dk + 2147483648LL);
    tk[j] = u;
    const unsigned mn = wave_min_u32(u), mx = wave_max_u32(u);
    if (j == 0) {
      tst[0] = mn;
      tst[1] = mx;
    }
  }
}

// P = SiLU(S + rab_t) (masked on PARTIAL tiles) as the bf16 A operands of
// P V: pa[nq][kk] holds keys kk*32 + {lg*4 + 0..3, 16 + lg*4 + 0..3}.
// FULL: every pair of the tile is visible. TCONST: rab_t is the scalar tcv
// for the whole block; T2: the block spans two buckets, tcv below |dt| = thr
// and tcv_hi from there on; else rab_t is gathered per element.
// TF (timestamp filter, partial tiles with the gathered rab_t path only): a
// row flagged in tfr also needs its key inside the prefix (prel = P - first
// key of this lane's group) or strictly earlier in time.
template <bool FULL, bool USE_T, bool TCONST, bool TF = false, bool T2 = false>
__device__ __forceinline__ void fwd_epilogue(const f32x4 (&st)[4][2], bf16x8 (&pa)[2][2],
                                             const int (&hirel)[2], const unsigned (&tq)[2],
                                             const unsigned *tkb, const float *t2tab, float tcv,
                                             int lg, const bool (&tfr)[2] = {false, false},
                                             int prel = 0, unsigned thr = 0u, float tcv_hi = 0.f) {
  static_assert(!TF || (USE_T && !FULL && !TCONST && !T2), "the filter runs on partial gathered tiles");
  static_assert(!T2 || !TCONST, "two buckets is a per-element path");
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    u32x4 w[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int mk = kk * 2 + h2;
      u32x4 tk4 = {0u, 0u, 0u, 0u};
      if (USE_T && !TCONST) tk4 = *(const u32x4 *)(tkb + mk * 16 + lg * 4);
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // t = -log2(e) (S + rab_t) (t2tab and tcv hold -log2(e) rab_t), and
          // t / (1 + 2^t) = -log2(e) SiLU(S + rab_t); the output scale undoes
          // the factor.
          float t;
          if (USE_T && T2) t = fmaf(st[mk][nq][i], -kLog2e, absdiff_u32(tq[nq], tk4[i]) >= thr ? tcv_hi : tcv);
          else if (USE_T) t = fmaf(st[mk][nq][i], -kLog2e, TCONST ? tcv : t2tab[ffbh_u32(absdiff_u32(tq[nq], tk4[i])) + 1]);
          else t = st[mk][nq][i] * -kLog2e;
          p[i] = t * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
          bool vis = hirel[nq] > mk * 16 + i;
          if (TF) vis = vis && (!tfr[nq] || prel > mk * 16 + i || tk4[i] < tq[nq]);
          if (!FULL) p[i] = vis ? p[i] : 0.f;
        }
        w[nq][h2 * 2] = pack_bf16x2(p[0], p[1]);
        w[nq][h2 * 2 + 1] = pack_bf16x2(p[2], p[3]);
      }
    }
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) pa[nq][kk] = __builtin_bit_cast(bf16x8, w[nq]);
  }
}

// Timestamps enter the kernel as int64 and are used as 32-bit values biased
// by 2^31 around a per-tile reference t_ref (the first query row's time):
// u = (t - t_ref) + 2^31. For any two tokens of a sequence whose times are
// within 2^31 s of each other, |u_i - u_j| is exactly |t_i - t_j|; a larger
// span is flagged in the status word.
//
// Per key tile and wave the time bucket of all (row, key) pairs is checked
// for being one constant (times usually grow along a sequence, so the bucket
// of a distant key tile rarely changes); then rab_t is one scalar for the
// whole block, else it is gathered per element from a 33-entry LDS table
// indexed by ffbh(|dt|) + 1.
// INL: the workgroup builds its own tile (small batches, no scheduler launch).
template <int D, bool USE_P, bool USE_T, bool TF, bool INL>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(FwdArgs a) {
  static_assert(!TF || USE_T, "the timestamp filter needs the timestamps");
  constexpr int BM = kFwdBM, BN = kFwdBN;
  constexpr int KS = D / 32;          // k-steps of the K Q^T contraction
  constexpr int ND = D / 16;          // 16-column blocks of O
  constexpr int KST = D + 16;         // LDS row stride of K (elements)
  constexpr int VST = D + 16;         // LDS row stride of V (elements)
  constexpr int OST = D + 8;          // LDS row stride of the staged output
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int NCH = BN * CH / 256;  // chunks per thread per matrix and tile
  constexpr int WIN = BM + BN;        // rab_p window entries per key tile
  static_assert(BM == 128 && BN == 64, "4 waves x 32 rows, 64 keys");
  static_assert(BM * OST <= 2 * BN * KST, "output staging reuses the K buffers");
  __shared__ __attribute__((aligned(16))) u16 Ks[2 * BN * KST];
  __shared__ __attribute__((aligned(16))) u16 Vs[2 * BN * VST];
  __shared__ float rabw[USE_P ? 2 * WIN : 1];
  __shared__ __attribute__((aligned(16))) unsigned tkey[USE_T ? 2 * BN : 4];
  __shared__ unsigned tkst[4];
  __shared__ float t2tab[33];
  __shared__ int s_bad;

  const int H = a.H;
  const int unit = blockIdx.x;
  const int r = unit / H, h = unit % H;
  QTile tile;
  SeqDesc sd;
  if constexpr (INL) {
    // the K buffers are free until the first tile is staged
    if (!sched_dev::inline_tile<256>(a.sched, r, unit == 0, (int *)Ks, &tile, &sd)) return;
  } else {
    if (r >= a.hdr[kHdrNQ]) return;
    tile = a.tiles[r];
    sd = a.desc[tile.b];
  }
  const int nk = tile.nk, nf = tile.nf_nrows & 0xffff, nrows = tile.nf_nrows >> 16;
  const int row0 = tile.row0;
  const long long ld = (long long)H * D;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const u16 *Q = (const u16 *)a.Q, *K = (const u16 *)a.K, *V = (const u16 *)a.V;

  const int fi0 = sd.q_frame0 + row0;
  const int fil = fi0 + nrows - 1;
  const int kv_limit = frame_hi(fil, sd.P, sd.E);  // keys >= kv_limit are seen by no row here
  const int pos_max = fil < sd.E ? fil : sd.E;
  const long long t_ref = USE_T ? a.ts_q[sd.q_base + row0] : 0;

  // Global -> register prefetch of one key tile, and register -> LDS store.
  TilePrefetch<NCH> pf;
  pf.r = 0.f;
  pf.t = 0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int chunk = tid + i * 256;
    pf.off[i] = (unsigned)(((chunk / (D / 8)) * ld + h * D + (chunk % (D / 8)) * 8) * 2);
  }
  FwdTileCtx cx;
  cx.K = K; cx.V = V; cx.rab_p = a.rab_p; cx.ts_kv = a.ts_kv; cx.ld = ld;
  cx.kv_base = sd.kv_base; cx.kv_limit = kv_limit; cx.pos_max = pos_max;
  cx.n_pos = a.n_pos; cx.tid = tid;
  // The first key tile is requested before the query rows, so that the two
  // loads overlap instead of waiting one after the other.
  if (nk > 0) fwd_load_tile<D, BN, USE_P, USE_T>(pf, cx, 0);

  // With USE_T the kernel has timestamps; the rab_t table may still be
  // absent when they serve only the timestamp filter (then it adds zero).
  const bool has_rt = a.rab_t != nullptr;

  // This lane's query rows in the S^T layout: local rows w*32 + nq*16 + lr.
  int hi_r[2], vb_r[2];
  unsigned tq_r[2] = {0u, 0u};
  bool ok_r[2], tfr[2];
  bf16x8 qf[2][KS];
  bool bad_t = false;
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int lrow = w * 32 + nq * 16 + lr;
    ok_r[nq] = lrow < nrows;
    const int crow = ok_r[nq] ? lrow : nrows - 1;
    const int fi = fi0 + crow;
    hi_r[nq] = ok_r[nq] ? frame_hi(fi, sd.P, sd.E) : 0;
    vb_r[nq] = pos_max - (fi < sd.E ? fi : sd.E) + lg * 4;
    tfr[nq] = TF && ok_r[nq] && fi >= sd.E;
    if (USE_T) {
      const long long dq = a.ts_q[sd.q_base + row0 + crow] - t_ref;
      bad_t |= dq < -2147483648LL || dq > 2147483647LL;
      tq_r[nq] = (unsigned)(dq + 2147483648LL);
    }
    const u16 *qp = Q + (long long)(sd.q_base + row0 + lrow) * ld + h * D + lg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = {0u, 0u, 0u, 0u};
      if (ok_r[nq]) v = *(const uint4 *)(qp + ks * 32);
      qf[nq][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // The t2tab entries in a register too (lane c holds entry c); the table
  // is read after the rows are requested, so its wait covers those loads.
  float t2v = 0.f;
  if (USE_T && has_rt && lane < 33) {
    const int bkt = lane == 0 ? 0 : 32 - lane;
    t2v = -kLog2e * a.rab_t[bkt < a.n_tb - 1 ? bkt : a.n_tb - 1];
  }
  if (tid == 0) s_bad = 0;
  if (USE_T && tid < 33) t2tab[tid] = t2v;  // the same entries, for the per-element reads
  __syncthreads();
  unsigned qmin = 0, qmax = 0;
  if (USE_T) {
    qmin = __builtin_amdgcn_readfirstlane(wave_min_u32(min(tq_r[0], tq_r[1])));
    qmax = __builtin_amdgcn_readfirstlane(wave_max_u32(max(tq_r[0], tq_r[1])));
  }
  // Keys [0, wave_hi) are the ones this wave's rows see: a key tile at or
  // beyond it (the upper half of a diagonal block, or a wave past the last
  // row) is skipped by this wave; its pairs are all masked.
  const int wave_hi = __builtin_amdgcn_readfirstlane(
      (int)wave_max_u32((unsigned)max(hi_r[0], hi_r[1])));
  // Whether some row of this wave is a candidate under the timestamp filter.
  const bool wave_tf = TF && __builtin_amdgcn_readfirstlane(
      (int)wave_max_u32((tfr[0] || tfr[1]) ? 1u : 0u)) != 0;

  f32x4 acc[2][ND];
#pragma unroll
  for (int nq = 0; nq < 2; ++nq)
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) acc[nq][nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 st[4][2];
  bf16x8 pa[2][2];

  // S^T = bias + K Q^T for the key tile in buffer buf.
  auto qk = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int mk = 0; mk < 4; ++mk)
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        if (USE_P) {
          const float *rw = rabw + buf * WIN + vb_r[nq] + mk * 16;
          st[mk][nq] = f32x4{rw[0], rw[1], rw[2], rw[3]};
        } else {
          st[mk][nq] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    const u16 *kb = Ks + buf * BN * KST;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mk = 0; mk < 4; ++mk) {
        const bf16x8 kf = *(const bf16x8 *)(kb + (mk * 16 + lr) * KST + ks * 32 + lg * 8);
#pragma unroll
        for (int nq = 0; nq < 2; ++nq)
          st[mk][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[nq][ks], st[mk][nq], 0, 0, 0);
      }
    }
  };

  // O += P V with V read transposed from its row-major LDS tile. The 2 x ND
  // fragment reads run PVD steps ahead of their MFMAs in a ring, so that no
  // step waits for a whole batch of reads to drain (not with the timestamp
  // filter, whose extra state leaves no registers for it).
  auto pv = [&](int buf) __attribute__((always_inline)) {
    const u16 *vb = Vs + buf * BN * VST + (lg * 4 + (lr >> 2)) * VST + (lr & 3) * 4;
    if constexpr (TF) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const u16 *p0 = vb + kk * 32 * VST + nd * 16;
          const s16x4 lo = lds_read_tr16(p0), hi = lds_read_tr16(p0 + 16 * VST);
          const bf16x8 vbf = __builtin_bit_cast(
              bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
          for (int nq = 0; nq < 2; ++nq)
            acc[nq][nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[nq][kk], vbf, acc[nq][nd], 0, 0, 0);
        }
      }
    } else {
      constexpr int NI = 2 * ND, PVD = 2;
      s16x4 rlo[PVD], rhi[PVD];
      auto rd = [&](int i) __attribute__((always_inline)) {
        const u16 *p0 = vb + (i / ND) * 32 * VST + (i % ND) * 16;
        rlo[i % PVD] = lds_read_tr16(p0);
        rhi[i % PVD] = lds_read_tr16(p0 + 16 * VST);
      };
#pragma unroll
      for (int i = 0; i < PVD; ++i) rd(i);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const s16x4 lo = rlo[i % PVD], hi = rhi[i % PVD];
        const bf16x8 vbf = __builtin_bit_cast(
            bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        if (i + PVD < NI) rd(i + PVD);
        const int kk = i / ND, nd = i % ND;
#pragma unroll
        for (int nq = 0; nq < 2; ++nq)
          acc[nq][nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[nq][kk], vbf, acc[nq][nd], 0, 0, 0);
      }
    }
  };

  if (nk > 0) {
    fwd_store_tile<D, BN, USE_P, USE_T>(pf, tid, Ks, Vs, rabw, tkey, tkst, t_ref, bad_t);
    if (nk > 1) fwd_load_tile<D, BN, USE_P, USE_T>(pf, cx, 1);
    __syncthreads();
    if (wave_hi > 0) qk(0);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int b = kt & 1;
    const int c0 = kt * BN;
    const bool full = kt < nf;
    int hirel[2];
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) hirel[nq] = hi_r[nq] - (c0 + lg * 4);

    // rab_t: one constant for the block when all its pairs share a bucket.
    bool tconst = true, two = false;
    float tcv = 0.f, tcv_hi = 0.f;
    unsigned thr = 0u;
    if (USE_T) {
      const unsigned kmin = __builtin_amdgcn_readfirstlane(tkst[b * 2]);
      const unsigned kmax = __builtin_amdgcn_readfirstlane(tkst[b * 2 + 1]);
      unsigned dlo, dhi;
      if (qmin >= kmax) {
        dlo = qmin - kmax;
        dhi = qmax - kmin;
      } else if (kmin >= qmax) {
        dlo = kmin - qmax;
        dhi = kmax - qmin;
      } else {
        dlo = 0u;
        dhi = max(qmax - kmin, kmax - qmin);
      }
      const int blo = bucket_u32(dlo, a.n_tb), bhi = bucket_u32(dhi, a.n_tb);
      tconst = blo == bhi;
      // t2tab entry ffbh(dlo) + 1 as a lane read (scalar index, no LDS round trip)
      tcv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t2v), dlo ? __builtin_clz(dlo) + 1 : 0));
      // Two buckets: |dt| >= 2^bhi is bucket bhi, the rest blo (bhi may be
      // the clamped last bucket; blo is then below the clamp).
      two = bhi == blo + 1;
      if (two) {
        thr = 1u << bhi;
        tcv_hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t2v), 32 - bhi));
      }
    }

    const unsigned *tkb = tkey + b * (USE_T ? BN : 0);
    if (wave_hi > c0) {
      if constexpr (TF) {
        if (wave_tf && !full) {
          fwd_epilogue<false, USE_T, false, true>(st, pa, hirel, tq_r, tkb, t2tab, tcv, lg, tfr,
                                                  sd.P - (c0 + lg * 4));
          pv(b);
          goto tile_done;
        }
      }
      if (USE_T && !tconst && two) {
        if (full) fwd_epilogue<true, USE_T, false, false, true>(st, pa, hirel, tq_r, tkb, t2tab, tcv, lg, tfr, 0, thr, tcv_hi);
        else fwd_epilogue<false, USE_T, false, false, true>(st, pa, hirel, tq_r, tkb, t2tab, tcv, lg, tfr, 0, thr, tcv_hi);
      } else if (USE_T && !tconst) {
        if (full) fwd_epilogue<true, USE_T, false>(st, pa, hirel, tq_r, tkb, t2tab, tcv, lg);
        else fwd_epilogue<false, USE_T, false>(st, pa, hirel, tq_r, tkb, t2tab, tcv, lg);
      } else {
        if (full) fwd_epilogue<true, USE_T, true>(st, pa, hirel, tq_r, tkb, t2tab, tcv, lg);
        else fwd_epilogue<false, USE_T, true>(st, pa, hirel, tq_r, tkb, t2tab, tcv, lg);
      }
      pv(b);
    }
  tile_done:
    if (kt + 1 < nk) {
      fwd_store_tile<D, BN, USE_P, USE_T>(pf, tid, Ks + (b ^ 1) * BN * KST, Vs + (b ^ 1) * BN * VST,
                                          rabw + (b ^ 1) * (USE_P ? WIN : 0), tkey + (b ^ 1) * (USE_T ? BN : 0),
                                          tkst + (b ^ 1) * 2, t_ref, bad_t);
      if (kt + 2 < nk) fwd_load_tile<D, BN, USE_P, USE_T>(pf, cx, kt + 2);
      __syncthreads();
      if (wave_hi > c0 + BN) qk(b ^ 1);
    }
  }

  // A candidate's pair with itself: o_i += SiLU(q_i.k_i + rab_p[0] + rab_t[0]) v_i.
  const bool any_cand = fil >= sd.E;
  if (any_cand) {
    const u16 *Ksf = (const u16 *)a.Kself, *Vsf = (const u16 *)a.Vself;
    const float bias0 = (USE_P ? a.rab_p[0] : 0.f) + (USE_T && has_rt ? a.rab_t[0] : 0.f);
    float as[2];
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
      const int lrow = w * 32 + nq * 16 + lr;
      const int fi = fi0 + lrow;
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
      as[nq] = cand ? -kLog2e * silu_fast(part + bias0) : 0.f;
    }
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float av = __shfl(as[nq], lg * 4 + i, 64);
        const int lrow = w * 32 + nq * 16 + lg * 4 + i;
        const int fi = fi0 + lrow;
        if (lrow < nrows && fi >= sd.E) {
          const u16 *vp = Vsf + (long long)(sd.self_base + fi - sd.E) * ld + h * D + lr;
#pragma unroll
          for (int nd = 0; nd < ND; ++nd) acc[nq][nd][i] += av * bf2f(vp[nd * 16]);
        }
      }
    }
  }

  if (USE_T && bad_t) atomicOr(&s_bad, 1);
  // The key loop summed -log2(e) SiLU(.) v; -ln(2) / N_max restores the scale.
  const float oscale = a.inv_nmax * -0.69314718055994531f;
  // Stage O through LDS (the K buffers) so that global stores are 16-byte rows.
  __syncthreads();
  u16 *os = Ks;
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lrow = w * 32 + nq * 16 + lg * 4 + i;
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const __bf16 v = (__bf16)(acc[nq][nd][i] * oscale);
        os[lrow * OST + nd * 16 + lr] = __builtin_bit_cast(u16, v);
      }
    }
  }
  __syncthreads();
  u16 *O = (u16 *)a.O;
  for (int c = tid; c < BM * CH; c += 256) {
    const int row = c / CH, col = (c % CH) * 8;
    if (row < nrows)
      *(uint4 *)(O + (long long)(sd.q_base + row0 + row) * ld + h * D + col) =
          *(const uint4 *)(os + row * OST + col);
  }
  if (USE_T && tid == 0 && s_bad) {
    if constexpr (INL) a.hdr[kHdrInlineTs] = (int)a.epoch;
    else atomicOr(&a.hdr[kHdrStatus], HSTU_DEV_BAD_TIMESTAMPS);
  }
}

// fp32: 256 threads = 64 rows x 4 column slices of D/4; keys staged in LDS.
// Key groups of the fp32 kernel: the keys of a tile are dealt round-robin to
// KSPLIT groups of 256 threads, whose partial outputs are summed in LDS at the
// end, so that a thread's dependent chain is 64 / KSPLIT keys long.
template <int D>
constexpr int f32_ksplit() { return D <= 64 ? 4 : 2; }

template <int D, bool INL>
__global__ __launch_bounds__(256 * f32_ksplit<D>()) void attn_fwd_f32_kernel(FwdArgs a) {
  constexpr int BN = kF32BN, DP = D / 4;
  constexpr int KSPLIT = f32_ksplit<D>(), NT = 256 * KSPLIT;
  static_assert(kF32BM == 64, "64 rows x 4 slices per key group");
  __shared__ float Ks[BN][D];
  __shared__ float Vs[BN][D];
  __shared__ long long tsk[BN];
  // rab_p window of a key tile (entry x: rab_p[|pos_max - c0 - x|]) and the
  // rab_t table by bucket (|dt| < 2^63, so buckets stop at 62), in LDS so
  // that the key loop does no dependent global loads.
  constexpr int PWIN = kF32BM + BN;
  __shared__ float rabw[PWIN];
  __shared__ float rabt[64];
  __shared__ float red[(KSPLIT - 1) * kF32BM * D];  // partial outputs of key groups 1..

  const int H = a.H;
  const int unit = blockIdx.x;
  const int r = unit / H, h = unit % H;
  QTile tile;
  SeqDesc sd;
  if constexpr (INL) {
    static_assert(sizeof(Ks) >= (NT + NT / 64 + 3) * sizeof(int), "scan space in the K tile");
    if (!sched_dev::inline_tile<NT>(a.sched, r, unit == 0, (int *)&Ks[0][0], &tile, &sd)) return;
  } else {
    if (r >= a.hdr[kHdrNQ]) return;
    tile = a.tiles[r];
    sd = a.desc[tile.b];
  }
  const int nk = tile.nk, nrows = tile.nf_nrows >> 16, row0 = tile.row0;
  const long long ld = (long long)H * D;
  const int tid = threadIdx.x, kgrp = tid >> 8, lrow = (tid & 255) >> 2, part = tid & 3;
  const float *Q = (const float *)a.Q, *K = (const float *)a.K, *V = (const float *)a.V;
  const bool use_p = a.rab_p != nullptr, use_t = a.ts_q != nullptr, has_rt = a.rab_t != nullptr;

  const bool ok = lrow < nrows;
  const int fi = sd.q_frame0 + row0 + lrow;
  const int hi = ok ? frame_hi(fi, sd.P, sd.E) : 0;
  const int pos = fi < sd.E ? fi : sd.E;
  const long long tq = (use_t && ok) ? a.ts_q[sd.q_base + row0 + lrow] : 0;
  const bool tfr = use_t && a.tfilt && ok && fi >= sd.E;  // candidate under the timestamp filter
  float q[DP], o[DP];
#pragma unroll
  for (int c = 0; c < DP; ++c) {
    q[c] = ok ? Q[(long long)(sd.q_base + row0 + lrow) * ld + h * D + part * DP + c] : 0.f;
    o[c] = 0.f;
  }
  const int kv_limit = frame_hi(sd.q_frame0 + row0 + nrows - 1, sd.P, sd.E);
  const int fil = sd.q_frame0 + row0 + nrows - 1;
  const int pos_max = fil < sd.E ? fil : sd.E;
  if (use_t && has_rt && tid < 64) rabt[tid] = a.rab_t[min(tid, a.n_tb - 1)];

  for (int kt = 0; kt < nk; ++kt) {
    const int c0 = kt * BN;
    __syncthreads();
    for (int c = tid; c < BN * D; c += NT) {
      const int row = c / D, col = c % D;
      const bool in = c0 + row < kv_limit;
      const long long g = (long long)(sd.kv_base + c0 + row) * ld + h * D + col;
      Ks[row][col] = in ? K[g] : 0.f;
      Vs[row][col] = in ? V[g] : 0.f;
    }
    if (tid < BN) tsk[tid] = (use_t && c0 + tid < kv_limit) ? a.ts_kv[sd.kv_base + c0 + tid] : 0;
    if (use_p && tid < PWIN) rabw[tid] = a.rab_p[pos_bucket(pos_max - c0 - tid, a.n_pos)];
    __syncthreads();
    const int jend = min(BN, kv_limit - c0);
    // The four lanes of a row hold a quarter of q each; their partial dot
    // products are summed with two quad DPP moves (no LDS round trip).
    // A fixed trip count (the body holds DPP moves, which keep a loop with
    // a run-time count from being unrolled); keys past jend are skipped by a
    // branch that is uniform in the wave.
#pragma unroll 4
    for (int jj = 0; jj < BN / KSPLIT; ++jj) {
      const int jl = kgrp + jj * KSPLIT;
      if (jl >= jend) continue;
      const int j = c0 + jl;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) s = fmaf(q[c], Ks[jl][part * DP + c], s);
      s += dpp_f32<0xB1>(s);
      s += dpp_f32<0x4E>(s);
      // pos - j = pos_max - c0 - x with x = pos_max - pos + jl in [0, 126]
      // (rows past the tile end read x = jl; their pairs are masked)
      if (use_p) s += rabw[(ok ? pos_max - pos : 0) + jl];
      if (use_t && has_rt) s += rabt[time_bucket(tq - tsk[jl], 64)];
      const bool vis = j < hi && (!tfr || j < sd.P || tsk[jl] < tq);
      const float p = vis ? s / (1.0f + expf(-s)) : 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) o[c] = fmaf(p, Vs[jl][part * DP + c], o[c]);
    }
  }

  // Sum the key groups' partial outputs (group 0 keeps the total).
  if (kgrp > 0) {
#pragma unroll
    for (int c = 0; c < DP; ++c) red[((kgrp - 1) * kF32BM + lrow) * D + part * DP + c] = o[c];
  }
  __syncthreads();
  if (kgrp > 0) return;
#pragma unroll
  for (int g = 0; g < KSPLIT - 1; ++g)
#pragma unroll
    for (int c = 0; c < DP; ++c) o[c] += red[(g * kF32BM + lrow) * D + part * DP + c];

  if (ok && fi >= sd.E) {
    const float *Ksf = (const float *)a.Kself, *Vsf = (const float *)a.Vself;
    const long long srow = (long long)(sd.self_base + fi - sd.E) * ld + h * D + part * DP;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < DP; ++c) s = fmaf(q[c], Ksf[srow + c], s);
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += (use_p ? a.rab_p[0] : 0.f) + (use_t && has_rt ? a.rab_t[0] : 0.f);
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

template <int D, bool INL>
hipError_t launch_bf16_di(const FwdArgs &a, hipStream_t s) {
  const bool p = a.rab_p != nullptr, t = a.ts_q != nullptr;
  const dim3 g(a.units), b(256);
  if (a.tfilt) {
    if (p) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, true, true, INL>), g, b, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, true, true, INL>), g, b, 0, s, a);
  } else if (p && t) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, true, false, INL>), g, b, 0, s, a);
  } else if (p) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, false, false, INL>), g, b, 0, s, a);
  } else if (t) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, true, false, INL>), g, b, 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, false, false, INL>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(const FwdArgs &a, hipStream_t s) {
  return a.inline_sched ? launch_bf16_di<D, true>(a, s) : launch_bf16_di<D, false>(a, s);
}

hipError_t launch_attn_fwd_bf16(const FwdArgs &a, hipStream_t s) {
  if (a.units <= 0) return hipSuccess;
  switch (a.d) {
    case 32: return launch_bf16_d<32>(a, s);
    case 64: return launch_bf16_d<64>(a, s);
    case 128: return launch_bf16_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_f32_d(const FwdArgs &a, hipStream_t s) {
  const dim3 g(a.units), b(256 * f32_ksplit<D>());
  if (a.inline_sched) hipLaunchKernelGGL((attn_fwd_f32_kernel<D, true>), g, b, 0, s, a);
  else hipLaunchKernelGGL((attn_fwd_f32_kernel<D, false>), g, b, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const FwdArgs &a, hipStream_t s) {
  if (a.units <= 0) return hipSuccess;
  switch (a.d) {
    case 32: return launch_f32_d<32>(a, s);
    case 64: return launch_f32_d<64>(a, s);
    case 128: return launch_f32_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hstu
