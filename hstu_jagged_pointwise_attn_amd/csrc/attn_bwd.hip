// Backward of the HSTU pointwise-attention core. With s_ij the logit,
// a_ij = SiLU(s_ij)/N_max on visible pairs and dO the gradient of the
// pre-norm output (HSTU blog, section 3 layer formula; SiLU from 3.1):
//   dV_j += a_ij dO_i,   dA_ij = <dO_i, v_j>,
//   dS_ij = dA_ij * SiLU'(s_ij) / N_max,   SiLU'(x) = sig(x) (1 + x (1 - sig(x))),
//   dQ_i += dS_ij k_j,   dK_j += dS_ij q_i,
//   d rab_p[min(|pos_i - pos_j|, n_pos-1)] += dS_ij,  d rab_t[bucket(t_i - t_j)] += dS_ij.
// Nothing of size O(n^2) is kept from the forward: S is recomputed (the
// activation-memory design of the HSTU blog, section 3.3).
//
// Two passes, no atomics on dQ/dK/dV:
//  * query-major (dq kernel): the forward's loop with dO next to Q in
//    registers; per key tile S^T = bias + K Q^T and dP^T = V dO^T, then
//    dS and dQ += dS K (K read transposed from LDS). It also sums d rab
//    (rab_p by signed diagonal pos_i - j, reduced per wave in registers or
//    through a skewed LDS block and kept in rings that slide with the key
//    tiles; rab_t by bucket) and handles a candidate's pair with itself,
//    including the candidate rows of dK and dV, which no other row sees.
//  * key-major (dkdv kernel): per tile of 64 non-candidate keys, K and V in
//    registers, the rows that see them streamed from LDS; S = Q K^T and
//    dP = dO V^T, then dV += P^T dO and dK += dS^T Q with dO and Q read
//    transposed from LDS.
#include "hstu_internal.h"
#include "../../include/hstu.h"
#include "device_common.h"

#include <type_traits>

namespace hstu {
namespace {

using namespace dev;

template <bool B>
using bc = std::integral_constant<bool, B>;

__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

template <int NCH>
struct PairPrefetch {
  u32x4 a[NCH], b[NCH];
  float r;
  long long t;
};

// ---------------------------------------------------------------------------
// dQ kernel (query-major): the forward's 128-row query tiles, 4 waves x 32
// rows (Q and dO of a lane's two rows stay in registers), key tiles of 32.
//
// d rab_p: without candidates (every row at its own position) a wave's
// 32 x 32 block of dS is reduced to diagonal sums in registers by DPP row
// shifts (DIAG_DPP, below). With candidates (positions repeat) each wave
// writes the block into a private LDS area with row r shifted left by its
// position offset s_r (so column c holds the diagonal
// pos_i - j = pos_w0 - c0 + 31 - c), and one column sum per lane gives the
// diagonal sums; cells outside a row's 32 written columns stay zero for the
// whole query tile, because the shifts do not change between key tiles.
// The sums go into rings indexed by the signed diagonal; diagonals that no
// later key tile can touch are flushed to global memory after every tile.
// ---------------------------------------------------------------------------
template <int D, bool USE_P, bool USE_T, bool TF, bool DIAG_DPP, bool ZO>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  static_assert(!DIAG_DPP || USE_P, "register diagonal sums are for rab_p");
  static_assert(!TF || USE_T, "the timestamp filter needs the timestamps");
  constexpr int BM = kFwdBM, BN = 32, NWV = 4;
  constexpr int KS = D / 32, ND = D / 16;
  constexpr int ST = D + 16;           // LDS row stride of K, V and the staged dQ
  constexpr int CH = D / 8;
  constexpr int NT = NWV * 64;
  constexpr int NCHUNK = BN * CH;
  constexpr int NCH = (NCHUNK + NT - 1) / NT;
  constexpr int WIN = BM + BN;         // 159 window entries used
  constexpr int RING = 256;              // > the 159 diagonals live at once
  constexpr int SKW = 64;              // skewed row: 32 keys + 31 shifts (+1 pad)
  static_assert(BM == 128 && NCH >= 1, "4 waves x 32 rows");
  static_assert(BM * ST <= 4 * BN * ST, "dQ staging reuses the K/V buffers");
  __shared__ __attribute__((aligned(16))) u16 KV[4 * BN * ST];  // K[2 stages], V[2 stages]
  __shared__ float rabw[USE_P ? 2 * WIN : 1];
  __shared__ __attribute__((aligned(16))) unsigned tkey[USE_T ? 2 * BN : 4];
  __shared__ unsigned tkst[4];
  __shared__ float t2tab[33];
  // Diagonal rings, each updated by plain read-add-write (LDS float atomics
  // are slow): with DIAG_DPP one per (wave, lane group) (no two lanes of a
  // wave share an address; rings 20 words apart put a wave's 64 lanes in 64
  // banks), otherwise one per wave for the skewed block's column sums.
  constexpr int RSTR = RING + 20;
  constexpr int NRING = DIAG_DPP ? NWV * 4 : NWV;
  __shared__ float ring[USE_P ? NRING * RSTR : 1];
  __shared__ float skew[USE_P && !DIAG_DPP ? NWV * 32 * SKW : 1];
  // per-element path: by ffbh(|dt|) + 1, one copy per lane row (lr), so that
  // the sixteen rows of a lane group, which usually share a bucket, add into
  // different words instead of queueing on one (summed at the end)
  constexpr int HSN = 16, HSS = 33;
  constexpr bool HIST_AFTER = D < 128;
  __shared__ float hts[USE_T ? HSN * HSS : 1];
  __shared__ float htb[USE_T ? 32 : 1];   // constant blocks: by bucket
  __shared__ float self_acc;
  __shared__ int s_bad;
  u16 *const Ks = KV, *const Vs = KV + 2 * BN * ST;

  const int H = a.H;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  if (r >= a.hdr[kHdrNQ]) return;
  const QTile tile = a.tiles[r];
  const SeqDesc sd = a.desc[tile.b];
  const int nrows = tile.nf_nrows >> 16;
  const int row0 = tile.row0;
  const long long ld = (long long)H * D;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const u16 *Q = (const u16 *)a.Q, *K = (const u16 *)a.K, *V = (const u16 *)a.V;

  const int fi0 = sd.q_frame0 + row0;
  const int fil = fi0 + nrows - 1;
  const int kv_limit = frame_hi(fil, sd.P, sd.E);
  const int nk = (kv_limit + BN - 1) / BN;       // key tiles of 32
  // the first nf are fully visible (a candidate under the timestamp filter is
  // sure to see only the prefix)
  const int nf = (TF && fil >= sd.E) ? min(frame_hi(fi0, sd.P, sd.E), sd.P) / BN
                                     : frame_hi(fi0, sd.P, sd.E) / BN;
  const int pos_max = fil < sd.E ? fil : sd.E;
  const long long t_ref = USE_T ? a.ts[sd.q_base + row0] : 0;

  PairPrefetch<NCH> pf;
  pf.r = 0.f;
  pf.t = 0;
  auto load = [&](int t) __attribute__((always_inline)) {
    const int c0 = t * BN;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int chunk = tid + c * NT;
      if (NCHUNK % NT != 0 && chunk >= NCHUNK) break;
      const int row = chunk / CH, col = (chunk % CH) * 8;
      const int key = min(c0 + row, kv_limit - 1);
      const long long g = (long long)(sd.kv_base + key) * ld + h * D + col;
      pf.a[c] = *(const u32x4 *)(K + g);
      pf.b[c] = *(const u32x4 *)(V + g);
    }
    if (USE_P && tid < WIN) pf.r = a.rab_p[pos_bucket(pos_max - c0 - tid, a.n_pos)];
    if (USE_T && tid < BN) pf.t = a.ts[sd.kv_base + min(c0 + tid, kv_limit - 1)];
  };
  // The first key tile is requested before the query rows, so that the two
  // loads overlap instead of waiting one after the other.
  if (nk > 0) load(0);
  const bool has_rt = a.rab_t != nullptr;  // USE_T without a table: times for the filter only

  // This lane's query rows (S^T layout): local rows w*32 + nq*16 + lr.
  const int wrow0 = min(w * 32, nrows - 1);
  const int pos_w0 = min(fi0 + wrow0, sd.E);
  int hi_r[2], vb_r[2], sh_r[2];
  bool ok_r[2], tfr[2];
  unsigned tq[2] = {0u, 0u};
  bool bad_t = false;
  bf16x8 qf[2][KS], dof[2][KS];
  const u16 *dO = (const u16 *)a.dO;
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int lrow = w * 32 + nq * 16 + lr;
    ok_r[nq] = lrow < nrows;
    const int crow = ok_r[nq] ? lrow : nrows - 1;
    const int fi = fi0 + crow;
    const int pos_r = fi < sd.E ? fi : sd.E;
    hi_r[nq] = ok_r[nq] ? frame_hi(fi, sd.P, sd.E) : 0;
    vb_r[nq] = pos_max - pos_r + lg * 4;
    sh_r[nq] = pos_r - pos_w0;  // 0..31 for the rows of this wave
    tfr[nq] = TF && ok_r[nq] && fi >= sd.E;
    if (USE_T) {
      const long long dq = a.ts[sd.q_base + row0 + crow] - t_ref;
      bad_t |= dq < -2147483648LL || dq > 2147483647LL;
      tq[nq] = (unsigned)(dq + 2147483648LL);
    }
    const long long off = (long long)(sd.q_base + row0 + lrow) * ld + h * D + lg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u};
      if (ok_r[nq]) {
        v = *(const u32x4 *)(Q + off + ks * 32);
        g = *(const u32x4 *)(dO + off + ks * 32);
      }
      qf[nq][ks] = __builtin_bit_cast(bf16x8, v);
      dof[nq][ks] = __builtin_bit_cast(bf16x8, g);
    }
  }
  // (tables and accumulators are set up after the rows are requested: the
  // table's wait covers those loads)
  if (tid == 0) {
    s_bad = 0;
    self_acc = 0.f;
  }
  if (USE_T && tid < 33) {
    const int c = tid - 1;
    const int bkt = c < 0 ? 0 : 31 - c;
    t2tab[tid] = has_rt ? -kLog2e * a.rab_t[bkt < a.n_tb - 1 ? bkt : a.n_tb - 1] : 0.f;
    if (tid < 32) htb[tid] = 0.f;
  }
  if (USE_T)
    for (int c = tid; c < HSN * HSS; c += NT) hts[c] = 0.f;
  if (USE_P) {
    for (int c = tid; c < NRING * RSTR; c += NT) ring[c] = 0.f;
    if (!DIAG_DPP)
      for (int c = tid; c < NWV * 32 * SKW; c += NT) skew[c] = 0.f;
  }
  __syncthreads();
  unsigned qmin = 0, qmax = 0;
  if (USE_T) {
    qmin = __builtin_amdgcn_readfirstlane(wave_min_u32(min(tq[0], tq[1])));
    qmax = __builtin_amdgcn_readfirstlane(wave_max_u32(max(tq[0], tq[1])));
  }
  // Keys [0, wave_hi) are the ones this wave's rows see: a key tile at or
  // beyond it (the upper part of the diagonal block, or a wave past the last
  // row) has only masked pairs for this wave, which skips its work on it
  // (the tiles come in increasing order, so once skipped always skipped).
  const int wave_hi = __builtin_amdgcn_readfirstlane(
      (int)wave_max_u32((unsigned)max(hi_r[0], hi_r[1])));
  // Whether some row of this wave is a candidate under the timestamp filter.
  const bool wave_tf = TF && __builtin_amdgcn_readfirstlane(
      (int)wave_max_u32((tfr[0] || tfr[1]) ? 1u : 0u)) != 0;

  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int chunk = tid + c * NT;
      if (NCHUNK % NT != 0 && chunk >= NCHUNK) break;
      const int row = chunk / CH, col = (chunk % CH) * 8;
      *(u32x4 *)(Ks + buf * BN * ST + row * ST + col) = pf.a[c];
      *(u32x4 *)(Vs + buf * BN * ST + row * ST + col) = pf.b[c];
    }
    if (USE_P && tid < WIN) rabw[buf * WIN + tid] = pf.r;
    if (USE_T && tid < 64) {  // wave 0; keys are lanes 0..31
      unsigned u = 0u;
      if (tid < BN) {
        const long long dk = pf.t - t_ref;
        bad_t |= dk < -2147483648LL || dk > 2147483647LL;
        u = (unsigned)(dk + 2147483648LL);
        tkey[buf * BN + tid] = u;
      }
      const unsigned mn = wave_min_u32(tid < BN ? u : 0xffffffffu);
      const unsigned mx = wave_max_u32(tid < BN ? u : 0u);
      if (tid == 0) {
        tkst[buf * 2] = mn;
        tkst[buf * 2 + 1] = mx;
      }
    }
  };

  f32x4 acc[2][ND];
#pragma unroll
  for (int nq = 0; nq < 2; ++nq)
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) acc[nq][nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 st[2][2], dpt[2][2];
  bf16x8 dsa[2];

  // S^T = bias + K Q^T and dP^T = V dO^T for the key tile in buffer buf.
  auto gemms = [&](int buf) __attribute__((always_inline)) {
    const u16 *kb = Ks + buf * BN * ST, *vbuf = Vs + buf * BN * ST;
#pragma unroll
    for (int mk = 0; mk < 2; ++mk)
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        if (USE_P) {
          const float *rw = rabw + buf * WIN + vb_r[nq] + mk * 16;
          st[mk][nq] = f32x4{rw[0], rw[1], rw[2], rw[3]};
        } else {
          st[mk][nq] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        dpt[mk][nq] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mk = 0; mk < 2; ++mk) {
        const bf16x8 kf = *(const bf16x8 *)(kb + (mk * 16 + lr) * ST + ks * 32 + lg * 8);
        const bf16x8 vf = *(const bf16x8 *)(vbuf + (mk * 16 + lr) * ST + ks * 32 + lg * 8);
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) {
          st[mk][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[nq][ks], st[mk][nq], 0, 0, 0);
          dpt[mk][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, dof[nq][ks], dpt[mk][nq], 0, 0, 0);
        }
      }
    }
  };

  float *skw = skew + w * 32 * SKW;
  // DIAG_DPP (launches without candidates, so every row sits at its own
  // position): the diagonal sums of a wave's 32 x 32 dS block of d rab_p are
  // formed in registers. In the S^T layout lane (lg, lr) holds keys
  // 16 mk + 4 lg + i of row 16 nq + lr, so element i sits on diagonal
  // base + 16 (nq - mk) + lr - 4 lg - i. Shifting element i of every lane down
  // by i lanes within its row of 16 (DPP row_shl) lines all four up on
  // diagonal base + 16 (nq - mk) + lr - 4 lg; the elements that would leave
  // the row land, shifted up by 16 - i (row_shr), on the diagonal 16 lower.
  // dacc[s] holds diagonal base + 16 - 16 s + lr - 4 lg; the four are added
  // into the ring of this wave and lane group. With candidates (positions
  // repeat) the skewed LDS block is used instead.
  constexpr bool wave_dpp = DIAG_DPP;
  // rab_t sums of constant / two-bucket tiles, carried across key tiles while
  // the bucket stays: per-lane partial sums of buckets tcur and tcur + 1
  // (tcur < 0: none yet; -2 so that bucket 0 does not match tcur + 1).
  int tcur = -2;
  float tacc_lo = 0.f, tacc_hi = 0.f;
  auto tflush = [&]() __attribute__((always_inline)) {
    if (tcur >= 0) {
      const float lo = wave_sum_f32(tacc_lo), hi = wave_sum_f32(tacc_hi);
      if (lane == 0) {
        if (lo != 0.f) atomicAdd(&htb[tcur], lo);
        if (hi != 0.f) atomicAdd(&htb[tcur + 1], hi);
      }
    }
    tacc_lo = tacc_hi = 0.f;
  };
  if (nk > 0) {
    store(0);
    if (nk > 1) load(1);
    __syncthreads();
    if (wave_hi > 0) gemms(0);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int b = kt & 1;
    const int c0 = kt * BN;
    const bool full = __builtin_amdgcn_readfirstlane(kt < nf ? 1 : 0) != 0;
    int hirel[2];
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) hirel[nq] = hi_r[nq] - (c0 + lg * 4);

    bool tconst = true, two = false;
    float tcv = 0.f, tcv_hi = 0.f;
    int tcidx = 0;
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
      tconst = __builtin_amdgcn_readfirstlane(blo == bhi ? 1 : 0) != 0;
      tcv = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t2tab[ffbh_u32(dlo) + 1])));
      tcidx = blo;
      // Two buckets: |dt| >= 2^bhi is bucket bhi, the rest blo (bhi may be
      // the clamped last bucket; blo is then below the clamp).
      two = __builtin_amdgcn_readfirstlane(bhi == blo + 1 ? 1 : 0) != 0;
      if (two) {
        thr = 1u << bhi;
        tcv_hi = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t2tab[32 - bhi])));
      }
    }

    // dS of this wave's 32 rows x 32 keys (fp32, masked), its bf16 copy as the
    // A operand of dQ += dS K, and its rab contributions. FULL: every pair is
    // visible; TC: one rab_t bucket for the whole block. On the per-element
    // rab_t path a lane's keys ascend along (mk, i) for each row, so equal
    // buckets come in runs that are merged before they go to the histogram.
    // TFV: a candidate row under the timestamp filter also needs its key in
    // the prefix or strictly earlier in time (partial, gathered tiles only).
    auto epilogue = [&](auto fullc, auto tconstc, auto tfc, auto twoc) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(fullc)::value, TC = decltype(tconstc)::value;
      constexpr bool TFV = decltype(tfc)::value, T2 = decltype(twoc)::value;
      static_assert(!TFV || (USE_T && !FULL && !TC && !T2), "the filter runs on partial gathered tiles");
      static_assert(!T2 || !TC, "two buckets is a per-element path");
      const int prel = sd.P - (c0 + lg * 4);
      float tsum = 0.f, tsum_hi = 0.f, run_s = 0.f;
      int run_b = -1;
      auto merge = [&](int tix, float ds) __attribute__((always_inline)) {
        if (tix != run_b) {
          if (run_b >= 0) atomicAdd(&hts[lr * HSS + run_b], run_s);
          run_b = tix;
          run_s = 0.f;
        }
        run_s += ds;
      };
      float dacc[4] = {-0.f, -0.f, -0.f, -0.f};  // -0: the first add is exact and folds away
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        u32x4 wds;
        // HIST_AFTER: the row's buckets and dS are kept and merged into the
        // histogram after its scores, so no branch sits inside the score
        // chain (d = 128 has no registers to spare for them)
        int tixs[2][4];
        float dsn[2][4];
#pragma unroll
        for (int mk = 0; mk < 2; ++mk) {
          u32x4 tk4 = {0u, 0u, 0u, 0u};
          if (USE_T && !TC) tk4 = *(const u32x4 *)(tkey + b * BN + mk * 16 + lg * 4);
          float dsv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // t = -log2(e) x with x = S + rab_t (t2tab and tcv hold
            // -log2(e) rab_t); sig(x) = 1 / (1 + 2^t) and
            // SiLU'(x) = sig + x sig (1 - sig) = sig + (t sig) (-ln 2) (1 - sig).
            int tix = 0;
            bool hi = false;
            float t;
            if (USE_T) {
              if (T2) {
                hi = absdiff_u32(tq[nq], tk4[i]) >= thr;
                t = fmaf(st[mk][nq][i], -kLog2e, hi ? tcv_hi : tcv);
              } else {
                if (!TC) tix = ffbh_u32(absdiff_u32(tq[nq], tk4[i])) + 1;
                t = fmaf(st[mk][nq][i], -kLog2e, TC ? tcv : t2tab[tix]);
              }
            } else {
              t = st[mk][nq][i] * -kLog2e;
            }
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
            float ds = dpt[mk][nq][i] * fmaf(t * sg, fmaf(sg, kLn2, -kLn2), sg);
            bool vis = hirel[nq] > mk * 16 + i;
            if (TFV) vis = vis && (!tfr[nq] || prel > mk * 16 + i || tk4[i] < tq[nq]);
            if (!FULL) ds = vis ? ds : 0.f;
            dsv[i] = ds;
            if (USE_P && !wave_dpp) skw[(nq * 16 + lr) * SKW + mk * 16 + lg * 4 + i + 31 - sh_r[nq]] = ds;
            if (USE_T) {
              if (TC || T2) {
                if (!(USE_P && wave_dpp)) tsum += ds;  // else from the diagonal sums below
                if (T2) tsum_hi += hi ? ds : 0.f;
              } else if (HIST_AFTER) {
                tixs[mk][i] = tix;
                dsn[mk][i] = ds;
              } else {
                merge(tix, ds);
              }
            }
          }
          wds[mk * 2] = pack_bf16x2(dsv[0], dsv[1]);
          wds[mk * 2 + 1] = pack_bf16x2(dsv[2], dsv[3]);
          if (USE_P && wave_dpp) {
            const int sa = 1 - nq + mk;  // offset 16 (nq - mk) -> slot
            dacc[sa] += dsv[0] + dpp_f32<0x101>(dsv[1]) + dpp_f32<0x102>(dsv[2]) + dpp_f32<0x103>(dsv[3]);
            dacc[sa + 1] += dpp_f32<0x11F>(dsv[1]) + dpp_f32<0x11E>(dsv[2]) + dpp_f32<0x11D>(dsv[3]);
          }
        }
        dsa[nq] = __builtin_bit_cast(bf16x8, wds);
        if (USE_T && !TC && !T2 && HIST_AFTER) {
#pragma unroll
          for (int mk = 0; mk < 2; ++mk)
#pragma unroll
            for (int i = 0; i < 4; ++i) merge(tixs[mk][i], dsn[mk][i]);
        }
      }
      if (USE_P && wave_dpp) {
        // every dS of the block sits in exactly one lane's four diagonal sums,
        // so their total is the block's sum for a one- or two-bucket rab_t
        if (USE_T && (TC || T2)) tsum = (dacc[0] + dacc[1]) + (dacc[2] + dacc[3]);
        const int dbase = pos_w0 - c0 + lr - 4 * lg + 16;
        float *rg = ring + (w * 4 + lg) * RSTR;
        float old[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) old[k] = rg[(dbase - 16 * k) & (RING - 1)];
#pragma unroll
        for (int k = 0; k < 4; ++k) rg[(dbase - 16 * k) & (RING - 1)] = old[k] + dacc[k];
      }
      if (USE_T && TC) {
        if (tcidx == tcur) {
          tacc_lo += tsum;
        } else if (tcidx == tcur + 1) {
          tacc_hi += tsum;
        } else {
          tflush();
          tcur = tcidx;
          tacc_lo = tsum;
        }
      }
      if (USE_T && T2) {
        if (tcidx != tcur) {
          tflush();
          tcur = tcidx;
        }
        tacc_lo += tsum - tsum_hi;
        tacc_hi += tsum_hi;
      }
      if (USE_T && !TC && !T2 && run_b >= 0) atomicAdd(&hts[lr * HSS + run_b], run_s);
    };
    bool done = c0 >= wave_hi;  // nothing this wave sees
    if constexpr (TF) {
      if (!done && wave_tf && !full) {
        epilogue(bc<false>(), bc<false>(), bc<true>(), bc<false>());
        done = true;
      }
    }
    if (!done) {
      if (USE_T && !tconst && two) {
        if (full) epilogue(bc<true>(), bc<false>(), bc<false>(), bc<true>());
        else epilogue(bc<false>(), bc<false>(), bc<false>(), bc<true>());
      } else if (USE_T && !tconst) {
        if (full) epilogue(bc<true>(), bc<false>(), bc<false>(), bc<false>());
        else epilogue(bc<false>(), bc<false>(), bc<false>(), bc<false>());
      } else {
        if (full) epilogue(bc<true>(), bc<true>(), bc<false>(), bc<false>());
        else epilogue(bc<false>(), bc<true>(), bc<false>(), bc<false>());
      }
    }
    if (USE_P && !wave_dpp && c0 < wave_hi) {
      // column sums of the skewed block = this wave's diagonal sums
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane < 2 * BN - 1) {
        float c1 = 0.f;
#pragma unroll
        for (int rr = 0; rr < 32; ++rr) c1 += skw[rr * SKW + lane];
        const int tbase = pos_w0 - c0 + 31;  // diagonal of column c is tbase - c
        float *slot = &ring[w * RSTR + ((tbase - lane) & (RING - 1))];
        *slot += c1;
      }
      __builtin_amdgcn_wave_barrier();
    }
    // dQ += dS K with K read transposed from its row-major tile; the
    // fragment reads run QD steps ahead of their MFMAs in a ring.
    if (c0 < wave_hi) {
      const u16 *kbuf = Ks + b * BN * ST + (lg * 4 + (lr >> 2)) * ST + (lr & 3) * 4;
      constexpr int QD = ND < 2 ? ND : 2;
      s16x4 rlo[QD], rhi[QD];
      auto rd = [&](int nd) __attribute__((always_inline)) {
        rlo[nd % QD] = lds_read_tr16(kbuf + nd * 16);
        rhi[nd % QD] = lds_read_tr16(kbuf + nd * 16 + 16 * ST);
      };
#pragma unroll
      for (int nd = 0; nd < QD; ++nd) rd(nd);
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const s16x4 lo = rlo[nd % QD], hi = rhi[nd % QD];
        const bf16x8 kb = __builtin_bit_cast(
            bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        if (nd + QD < ND) rd(nd + QD);
#pragma unroll
        for (int nq = 0; nq < 2; ++nq)
          acc[nq][nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsa[nq], kb, acc[nq][nd], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) {
      store(b ^ 1);
      if (kt + 2 < nk) load(kt + 2);
    }
    __syncthreads();
    // Diagonals above the next tile's window are complete: flush them.
    // (by the last wave: wave 0 stages the key times)
    if (USE_P && tid >= NT - BN) {
      const int t = (pos_max - c0) - (tid - (NT - BN));
      float *slot = &ring[t & (RING - 1)];
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < NRING; ++q) {
        v += slot[q * RSTR];
        slot[q * RSTR] = 0.f;
      }
      if (v != 0.f) atomicAdd(a.drab_p + pos_bucket(t, a.n_pos), v * a.inv_nmax);
    }
    if (kt + 1 < nk && c0 + BN < wave_hi) gemms(b ^ 1);
  }
  if (USE_P && nk > 0 && tid < WIN - BN) {
    // the rest of the last window: diagonals [pos_max - c_last - 159, pos_max - c_last - 32]
    const int t = (pos_max - (nk - 1) * BN) - BN - tid;
    const float *slot = &ring[t & (RING - 1)];
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < NRING; ++q) v += slot[q * RSTR];
    if (v != 0.f) atomicAdd(a.drab_p + pos_bucket(t, a.n_pos), v * a.inv_nmax);
  }

  if (USE_T) tflush();

  // A candidate's pair with itself (|pos| and |dt| are 0).
  const bool any_cand = fil >= sd.E;
  if (any_cand) {
    const float bias0 = (USE_P ? a.rab_p[0] : 0.f) + (USE_T && has_rt ? a.rab_t[0] : 0.f);
    u16 *dK = (u16 *)a.dK, *dV = (u16 *)a.dV;
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
      const int lrow = w * 32 + nq * 16 + lr;
      const bool cand = ok_r[nq] && fi0 + lrow >= sd.E;
      float qk = 0.f, dov = 0.f;
      const long long srow = (long long)(sd.self_base + fi0 + lrow - sd.E) * ld + h * D + lg * 8;
      // the same row of dK / dV (row stride ldo: a layer's dZ blocks)
      const long long sout = ZO ? (long long)(sd.self_base + fi0 + lrow - sd.E) * a.ldo + h * D + lg * 8 : srow;
      if (cand) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 kv = *(const u32x4 *)(K + srow + ks * 32);
          const u32x4 vv = *(const u32x4 *)(V + srow + ks * 32);
          const u16 *ke = (const u16 *)&kv, *ve = (const u16 *)&vv;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            qk += (float)qf[nq][ks][e] * bf2f(ke[e]);
            dov += (float)dof[nq][ks][e] * bf2f(ve[e]);
          }
        }
      }
      qk += __shfl_xor(qk, 16, 64);
      qk += __shfl_xor(qk, 32, 64);
      dov += __shfl_xor(dov, 16, 64);
      dov += __shfl_xor(dov, 32, 64);
      const float x = qk + bias0;
      const float sg = sigmoid_fast(x);
      const float dss = cand ? dov * sg * (1.0f + x * (1.0f - sg)) : 0.f;  // unscaled
      const float as = cand ? x * sg : 0.f;
      if (cand) {
        // dK_i = dS_ii q_i / N_max and dV_i = a_ii dO_i / N_max (rows no other row sees)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 wk, wv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            wk[e] = pack_bf16x2((float)qf[nq][ks][2 * e] * dss * a.inv_nmax,
                                (float)qf[nq][ks][2 * e + 1] * dss * a.inv_nmax);
            wv[e] = pack_bf16x2((float)dof[nq][ks][2 * e] * as * a.inv_nmax,
                                (float)dof[nq][ks][2 * e + 1] * as * a.inv_nmax);
          }
          if constexpr (ZO) {  // a layer's dZ blocks: times SiLU'(Z), as the dK/dV kernel's own rows
            wk = dsilu_bf16x8(wk, *(const u32x4 *)((const u16 *)a.zk + sout + ks * 32));
            wv = dsilu_bf16x8(wv, *(const u32x4 *)((const u16 *)a.zv + sout + ks * 32));
          }
          *(u32x4 *)(dK + sout + ks * 32) = wk;
          *(u32x4 *)(dV + sout + ks * 32) = wv;
        }
        if (lg == 0) atomicAdd(&self_acc, dss);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dv = __shfl(dss, lg * 4 + i, 64);
        const int orow = w * 32 + nq * 16 + lg * 4 + i;
        if (orow < nrows && fi0 + orow >= sd.E) {
          const u16 *kp = K + (long long)(sd.self_base + fi0 + orow - sd.E) * ld + h * D + lr;
#pragma unroll
          for (int nd = 0; nd < ND; ++nd) acc[nq][nd][i] += dv * bf2f(kp[nd * 16]);
        }
      }
    }
  }
  if (USE_T && bad_t) atomicOr(&s_bad, 1);
  __syncthreads();
  if (tid == 0 && any_cand) {
    if (USE_P) atomicAdd(a.drab_p, self_acc * a.inv_nmax);
    if (USE_T && has_rt) atomicAdd(a.drab_t, self_acc * a.inv_nmax);
  }
  if (USE_T && has_rt && tid < 33) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < HSN; ++k) v += hts[k * HSS + tid];
    if (v != 0.f) {
      const int c = tid - 1;
      const int bkt = c < 0 ? 0 : 31 - c;
      atomicAdd(a.drab_t + (bkt < a.n_tb - 1 ? bkt : a.n_tb - 1), v * a.inv_nmax);
    }
    if (tid < 32 && htb[tid] != 0.f) atomicAdd(a.drab_t + tid, htb[tid] * a.inv_nmax);
  }
  // A layer's pre-activation rows for the fused SiLU', requested before the
  // staging below so that their latency overlaps it.
  constexpr int NCO = BM * CH / NT;  // 16-byte chunks of dQ per thread
  static_assert(BM * CH % NT == 0, "whole chunks per thread");
  const u16 *zq = (const u16 *)a.zq;
  u32x4 zpre[NCO];
  if constexpr (ZO) {
#pragma unroll
    for (int j = 0; j < NCO; ++j) {
      const int c = tid + j * NT, row = c / CH, col = (c % CH) * 8;
      if (row < nrows) zpre[j] = *(const u32x4 *)(zq + (long long)(sd.q_base + row0 + row) * a.ldo + h * D + col);
    }
  }
  // Stage dQ through LDS for 16-byte row stores.
  u16 *os = KV;
#pragma unroll
  for (int nq = 0; nq < 2; ++nq)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int orow = w * 32 + nq * 16 + lg * 4 + i;
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const __bf16 v = (__bf16)(acc[nq][nd][i] * a.inv_nmax);
        os[orow * ST + nd * 16 + lr] = __builtin_bit_cast(u16, v);
      }
    }
  __syncthreads();
  u16 *dQ = (u16 *)a.dQ;
  if constexpr (ZO) {
#pragma unroll
    for (int j = 0; j < NCO; ++j) {
      const int c = tid + j * NT, row = c / CH, col = (c % CH) * 8;
      if (row < nrows) {
        const long long g = (long long)(sd.q_base + row0 + row) * a.ldo + h * D + col;
        *(u32x4 *)(dQ + g) = dsilu_bf16x8(*(const u32x4 *)(os + row * ST + col), zpre[j]);  // a layer's dZ block
      }
    }
  } else {
    for (int c = tid; c < BM * CH; c += NT) {
      const int row = c / CH, col = (c % CH) * 8;
      if (row < nrows)
        *(u32x4 *)(dQ + (long long)(sd.q_base + row0 + row) * ld + h * D + col) =
            *(const u32x4 *)(os + row * ST + col);
    }
  }
  if (USE_T && tid == 0 && s_bad) atomicOr(a.status, HSTU_DEV_BAD_TIMESTAMPS);
}

// ---------------------------------------------------------------------------
// dK/dV kernel (key-major): 4 waves x 16 keys, query steps of 64 rows.
// ---------------------------------------------------------------------------
template <int D, bool USE_P, bool USE_T, bool TF, bool ZO>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
  static_assert(!TF || USE_T, "the timestamp filter needs the timestamps");
  constexpr int BN = kBwdKBN, BM = kBwdKBM;
  constexpr int KS = D / 32, ND = D / 16;
  constexpr int ST = D + 16;           // LDS row stride of the Q and dO tiles
  constexpr int CH = D / 8;
  constexpr int NCH = BM * CH / 256;
  constexpr int WIN = BM + BN;
  static_assert(BN == 64 && BM == 64, "4 waves x 16 keys, 64 rows");
  __shared__ __attribute__((aligned(16))) u16 Qs[2 * BM * ST];
  __shared__ __attribute__((aligned(16))) u16 Os[2 * BM * ST];
  __shared__ float rabw[USE_P ? 2 * WIN : 1];
  __shared__ __attribute__((aligned(16))) unsigned trow[USE_T ? 2 * BM : 4];
  __shared__ unsigned trst[4];
  __shared__ float t2tab[33];

  const int H = a.H;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  if (r >= a.hdr[kHdrNQ]) return;
  const QTile tile = a.tiles[r];
  const SeqDesc sd = a.desc[tile.b];
  const int k0 = tile.row0;
  const int qt_lo = tile.nf_nrows & 0xffff, nkeys = tile.nf_nrows >> 16;
  const int nq = tile.nk;
  const int L = sd.qcount;
  const long long ld = (long long)H * D;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const u16 *Q = (const u16 *)a.Q, *K = (const u16 *)a.K, *V = (const u16 *)a.V;
  const u16 *dO = (const u16 *)a.dO;

  PairPrefetch<NCH> pf;
  pf.r = 0.f;
  pf.t = 0;
  // Byte offset of this thread's chunk c inside a step's rows: the same in
  // every step (the buffer base moves instead).
  unsigned coff[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int chunk = tid + c * 256;
    coff[c] = (unsigned)(((chunk / CH) * ld + h * D + (chunk % CH) * 8) * 2);
  }
  // rows [fr0, fr0 + 64) of the frame; rows past the end load as zeros
  // (they fall outside the buffer, which ends at the sequence's last row).
  auto load = [&](int qt) __attribute__((always_inline)) {
    const int fr0 = qt * BM;
    const long long rb = (long long)(sd.q_base + fr0) * ld;
    const long long nb = (long long)(L - fr0) * ld * 2;
    const __amdgpu_buffer_rsrc_t qr = buf_view(Q + rb, nb), gr = buf_view(dO + rb, nb);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      pf.a[c] = buf_load16(qr, coff[c]);
      pf.b[c] = buf_load16(gr, coff[c]);
    }
    if (USE_P && tid < WIN) {
      // window of t = pos(row) - key: t_lo = pos(fr0) - (k0 + 63)
      const int p0 = fr0 < sd.E ? fr0 : sd.E;
      pf.r = a.rab_p[pos_bucket(p0 - (k0 + BN - 1) + tid, a.n_pos)];
    }
    // row times by the last wave (waves 0-1 stage the rab_p window)
    if (USE_T && tid >= 256 - BM) pf.t = a.ts[sd.q_base + min(fr0 + tid - (256 - BM), L - 1)];
  };
  // The first query step is requested before the keys, so that the loads
  // overlap instead of waiting one after the other.
  if (nq > 0) load(qt_lo);
  const bool has_rt = a.rab_t != nullptr;  // USE_T without a table: times for the filter only

  // This lane's key (B-operand and C-column layout): k0 + w*16 + lr.
  const int lkey = w * 16 + lr;
  const bool kok = lkey < nkeys;
  const int key = k0 + (kok ? lkey : nkeys - 1);
  const int rmin = kok ? (key < sd.P ? 0 : key) : 0x7fffffff;  // first row that sees the key
  const int kmax_valid = k0 + nkeys - 1;
  const int rmin_tile = kmax_valid < sd.P ? 0 : kmax_valid;      // rows >= it see every key

  bf16x8 kf[KS], vf[KS];
  {
    const long long off = (long long)(sd.kv_base + key) * ld + h * D + lg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(K + off + ks * 32));
      vf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(V + off + ks * 32));
    }
  }
  const long long t_ref = USE_T ? a.ts[sd.kv_base + k0] : 0;
  const long long t_key = USE_T ? a.ts[sd.kv_base + key] : 0;
  float t2raw = 0.f;
  if (USE_T && has_rt) {
    const int bkt = (lane == 0 || lane > 32) ? 0 : 32 - lane;
    t2raw = a.rab_t[bkt < a.n_tb - 1 ? bkt : a.n_tb - 1];
  }
  __shared__ int s_bad;
  if (tid == 0) s_bad = 0;
  // Times are kept as u = t - t_ref + 2^31; a row or key 2^31 s or more
  // away from t_ref would wrap, so it raises the status bit.
  bool bad_t = false;
  unsigned tk = 0u;
  if (USE_T) {
    const long long dk = t_key - t_ref;
    bad_t = dk < -2147483648LL || dk > 2147483647LL;
    tk = (unsigned)(dk + 2147483648LL);
  }
  unsigned kmin = 0, kmax = 0;
  if (USE_T) {
    kmin = __builtin_amdgcn_readfirstlane(wave_min_u32(tk));
    kmax = __builtin_amdgcn_readfirstlane(wave_max_u32(tk));
  }
  // The t2tab entries in a register (lane c holds entry c): a step's
  // constant rab_t term is a lane read, with no LDS round trip. (The table
  // was requested with the key rows; lanes past 32 read entry 0 and drop it.)
  const float t2v = (USE_T && lane < 33) ? -kLog2e * t2raw : 0.f;
  if (USE_T && tid < 33) t2tab[tid] = t2v;  // the same entries, for the per-element reads

  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int chunk = tid + c * 256;
      const int row = chunk / CH, col = (chunk % CH) * 8;
      *(u32x4 *)(Qs + buf * BM * ST + row * ST + col) = pf.a[c];
      *(u32x4 *)(Os + buf * BM * ST + row * ST + col) = pf.b[c];
    }
    if (USE_P && tid < WIN) rabw[buf * WIN + tid] = pf.r;
    if (USE_T && tid >= 256 - BM) {  // exactly the last wave
      const int j = tid - (256 - BM);
      const long long dr = pf.t - t_ref;
      bad_t |= dr < -2147483648LL || dr > 2147483647LL;
      const unsigned u = (unsigned)(dr + 2147483648LL);
      trow[buf * BM + j] = u;
      const unsigned mn = wave_min_u32(u), mx = wave_max_u32(u);
      if (j == 0) {
        trst[buf * 2] = mn;
        trst[buf * 2 + 1] = mx;
      }
    }
  };

  f32x4 dk[ND], dv[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) dk[nd] = dv[nd] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nq > 0) {
    store(0);
    if (nq > 1) load(qt_lo + 1);
  }
  __syncthreads();
  for (int it = 0; it < nq; ++it) {
    const int b = it & 1;
    const int fr0 = (qt_lo + it) * BM;
    const u16 *qb = Qs + b * BM * ST, *ob = Os + b * BM * ST;
    f32x4 s[4], dp[4];
#pragma unroll
    for (int mr = 0; mr < 4; ++mr) s[mr] = dp[mr] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (USE_P) {
      // bias of element (mr, i): rabw[min(A + 16 mr + i, Bc)]
      const int tlo = (fr0 < sd.E ? fr0 : sd.E) - (k0 + BN - 1);
      const int A = fr0 + lg * 4 - key - tlo, Bc = sd.E - key - tlo;
      if (fr0 + BM <= sd.E) {
        // every row of the step sits at its own position: no clamp, so the
        // sixteen reads share one address and take immediate offsets
        const float *rw = rabw + b * WIN + A;
#pragma unroll
        for (int mr = 0; mr < 4; ++mr)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[mr][i] = rw[mr * 16 + i];
      } else {
#pragma unroll
        for (int mr = 0; mr < 4; ++mr)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[mr][i] = rabw[b * WIN + min(A + mr * 16 + i, Bc)];
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mr = 0; mr < 4; ++mr) {
        const bf16x8 qa = *(const bf16x8 *)(qb + (mr * 16 + lr) * ST + ks * 32 + lg * 8);
        s[mr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[ks], s[mr], 0, 0, 0);
        const bf16x8 oa = *(const bf16x8 *)(ob + (mr * 16 + lr) * ST + ks * 32 + lg * 8);
        dp[mr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vf[ks], dp[mr], 0, 0, 0);
      }
    }
    bool tconst = true;
    float tcv = 0.f;
    if (USE_T) {
      const unsigned rmn = __builtin_amdgcn_readfirstlane(trst[b * 2]);
      const unsigned rmx = __builtin_amdgcn_readfirstlane(trst[b * 2 + 1]);
      unsigned dlo, dhi;
      if (rmn >= kmax) {
        dlo = rmn - kmax;
        dhi = rmx - kmin;
      } else if (kmin >= rmx) {
        dlo = kmin - rmx;
        dhi = kmax - rmn;
      } else {
        dlo = 0u;
        dhi = max(rmx - kmin, kmax - rmn);
      }
      const int blo = bucket_u32(dlo, a.n_tb), bhi = bucket_u32(dhi, a.n_tb);
      tconst = blo == bhi;
      // t2tab index ffbh(dlo) + 1, in scalar registers
      tcv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t2v), dlo ? __builtin_clz(dlo) + 1 : 0));
    }
    // Under the timestamp filter, candidate rows of this step see the tile's
    // causal keys by time: such a step is partial and takes the gathered path.
    const bool tf_step = TF && fr0 + BM > sd.E && k0 + nkeys > sd.P;
    if (tf_step) tconst = false;
    const bool full = fr0 >= rmin_tile && !tf_step;
    const int rrel = rmin - (fr0 + lg * 4);  // element (mr, i) visible iff 16 mr + i >= rrel
    bf16x8 pa[2], da[2];
    // FULL (every pair visible) and TC (one rab_t value for the step) are
    // compile-time in each copy of the epilogue, so that the per-element
    // bucket reads of the other steps are straight-line code (issued
    // together, one wait) rather than a branch and a wait per element.
    auto epilogue = [&](auto fullc, auto tconstc) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(fullc)::value, TC = decltype(tconstc)::value;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 wp, wd;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int mr = kk * 2 + h2;
          u32x4 tr4 = {0u, 0u, 0u, 0u};
          if (USE_T && !TC) tr4 = *(const u32x4 *)(trow + b * BM + mr * 16 + lg * 4);
          float pv[4], dv4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // t = -log2(e) x with x = S + rab_t (t2tab and tcv hold
            // -log2(e) rab_t); p = t sig(x) = -log2(e) SiLU(x), which the dV
            // scale undoes, and SiLU'(x) = sig + p (-ln 2) (1 - sig).
            float t;
            if (USE_T) t = fmaf(s[mr][i], -kLog2e, TC ? tcv : t2tab[ffbh_u32(absdiff_u32(tr4[i], tk)) + 1]);
            else t = s[mr][i] * -kLog2e;
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
            float p = t * sg;
            float d = dp[mr][i] * fmaf(p, fmaf(sg, kLn2, -kLn2), sg);
            if (!FULL) {
              bool vis = mr * 16 + i >= rrel;
              if (TF && !TC && tf_step) {
                const int row = fr0 + lg * 4 + mr * 16 + i;
                vis = vis && (row < sd.E || key < sd.P || tk < tr4[i]);
              }
              if (!vis) {
                p = 0.f;
                d = 0.f;
              }
            }
            pv[i] = p;
            dv4[i] = d;
          }
          wp[h2 * 2] = pack_bf16x2(pv[0], pv[1]);
          wp[h2 * 2 + 1] = pack_bf16x2(pv[2], pv[3]);
          wd[h2 * 2] = pack_bf16x2(dv4[0], dv4[1]);
          wd[h2 * 2 + 1] = pack_bf16x2(dv4[2], dv4[3]);
        }
        pa[kk] = __builtin_bit_cast(bf16x8, wp);
        da[kk] = __builtin_bit_cast(bf16x8, wd);
      }
    };
    // (a timestamp-filter step is never FULL and never TC)
    if (!USE_T || tconst) {
      if (full) epilogue(bc<true>(), bc<true>());
      else epilogue(bc<false>(), bc<true>());
    } else {
      if (full) epilogue(bc<true>(), bc<false>());
      else epilogue(bc<false>(), bc<false>());
    }
    // dV += P^T dO and dK += dS^T Q with dO and Q read transposed; the
    // fragment reads run GD steps ahead of their MFMAs in a ring.
    {
      constexpr int NI = 2 * ND, GD = 1;
      const int base = (lg * 4 + (lr >> 2)) * ST + (lr & 3) * 4;
      s16x4 ro0[GD], ro1[GD], rq0[GD], rq1[GD];
      auto rd = [&](int i) __attribute__((always_inline)) {
        const int off = base + (i / ND) * 32 * ST + (i % ND) * 16;
        ro0[i % GD] = lds_read_tr16(ob + off);
        ro1[i % GD] = lds_read_tr16(ob + off + 16 * ST);
        rq0[i % GD] = lds_read_tr16(qb + off);
        rq1[i % GD] = lds_read_tr16(qb + off + 16 * ST);
      };
#pragma unroll
      for (int i = 0; i < GD; ++i) rd(i);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const s16x4 o0 = ro0[i % GD], o1 = ro1[i % GD], q0 = rq0[i % GD], q1 = rq1[i % GD];
        const bf16x8 ot = __builtin_bit_cast(bf16x8, s16x8{o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]});
        const bf16x8 qt = __builtin_bit_cast(bf16x8, s16x8{q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]});
        if (i + GD < NI) rd(i + GD);
        const int kk = i / ND, nd = i % ND;
        dv[nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[kk], ot, dv[nd], 0, 0, 0);
        dk[nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da[kk], qt, dk[nd], 0, 0, 0);
      }
    }
    if (it + 1 < nq) {
      store(b ^ 1);
      if (it + 2 < nq) load(qt_lo + it + 2);
    }
    __syncthreads();
  }

  if (USE_T && bad_t) atomicOr(&s_bad, 1);
  // A layer's pre-activation rows for the fused SiLU', requested before the
  // staging below so that their latency overlaps it.
  constexpr int NCO = BN * CH / 256;  // 16-byte chunks of dK (and dV) per thread
  static_assert(BN * CH % 256 == 0, "whole chunks per thread");
  const u16 *zk = (const u16 *)a.zk, *zv = (const u16 *)a.zv;
  u32x4 zkp[NCO], zvp[NCO];
  if constexpr (ZO) {
#pragma unroll
    for (int j = 0; j < NCO; ++j) {
      const int c = tid + j * 256, row = c / CH, col = (c % CH) * 8;
      if (row < nkeys) {
        const long long g = (long long)(sd.kv_base + k0 + row) * a.ldo + h * D + col;
        zkp[j] = *(const u32x4 *)(zk + g);
        zvp[j] = *(const u32x4 *)(zv + g);
      }
    }
  }
  // Stage dK and dV (C layout: key 4 lg + i, column 16 nd + lr) through LDS;
  // dV summed -log2(e) SiLU(.) dO, which -ln(2) / N_max restores.
  const float vscale = a.inv_nmax * -kLn2;
  u16 *sk = Qs, *sv = Os;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kr = w * 16 + lg * 4 + i;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      sk[kr * ST + nd * 16 + lr] = __builtin_bit_cast(u16, (__bf16)(dk[nd][i] * a.inv_nmax));
      sv[kr * ST + nd * 16 + lr] = __builtin_bit_cast(u16, (__bf16)(dv[nd][i] * vscale));
    }
  }
  __syncthreads();
  u16 *dK = (u16 *)a.dK, *dV = (u16 *)a.dV;
  if constexpr (ZO) {  // a layer's dZ blocks
#pragma unroll
    for (int j = 0; j < NCO; ++j) {
      const int c = tid + j * 256, row = c / CH, col = (c % CH) * 8;
      if (row < nkeys) {
        const long long g = (long long)(sd.kv_base + k0 + row) * a.ldo + h * D + col;
        *(u32x4 *)(dK + g) = dsilu_bf16x8(*(const u32x4 *)(sk + row * ST + col), zkp[j]);
        *(u32x4 *)(dV + g) = dsilu_bf16x8(*(const u32x4 *)(sv + row * ST + col), zvp[j]);
      }
    }
  } else {
    for (int c = tid; c < BN * CH; c += 256) {
      const int row = c / CH, col = (c % CH) * 8;
      if (row < nkeys) {
        const long long g = (long long)(sd.kv_base + k0 + row) * ld + h * D + col;
        *(u32x4 *)(dK + g) = *(const u32x4 *)(sk + row * ST + col);
        *(u32x4 *)(dV + g) = *(const u32x4 *)(sv + row * ST + col);
      }
    }
  }
  if (USE_T && tid == 0 && s_bad) atomicOr(a.status, HSTU_DEV_BAD_TIMESTAMPS);
}

// ---------------------------------------------------------------------------
// fp32 kernels (vector ALU): 4 threads per row (dQ) or per key (dK/dV).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(BwdArgs a) {
  constexpr int BN = 64, DP = D / 4;
  __shared__ float Ks[BN][D];
  __shared__ float Vs[BN][D];
  __shared__ long long tsk[BN];
  const int H = a.H;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  if (r >= a.hdr[kHdrNQ]) return;
  const QTile tile = a.tiles[r];
  const SeqDesc sd = a.desc[tile.b];
  const int nk = tile.nk, nrows = tile.nf_nrows >> 16, row0 = tile.row0;
  const long long ld = (long long)H * D;
  const int tid = threadIdx.x, lrow = tid >> 2, part = tid & 3;
  const float *Q = (const float *)a.Q, *K = (const float *)a.K, *V = (const float *)a.V;
  const float *dO = (const float *)a.dO;
  const bool use_p = a.rab_p != nullptr, use_t = a.ts != nullptr, has_rt = a.rab_t != nullptr;
  const bool ok = lrow < nrows;
  const int fi = sd.q_frame0 + row0 + lrow;
  const int hi = ok ? frame_hi(fi, sd.P, sd.E) : 0;
  const int pos = fi < sd.E ? fi : sd.E;
  const long long tq = (use_t && ok) ? a.ts[sd.q_base + row0 + lrow] : 0;
  const bool tfr = use_t && a.tfilt && ok && fi >= sd.E;  // candidate under the timestamp filter
  const long long roff = (long long)(sd.q_base + row0 + lrow) * ld + h * D + part * DP;
  float q[DP], g[DP], dq[DP];
#pragma unroll
  for (int c = 0; c < DP; ++c) {
    q[c] = ok ? Q[roff + c] : 0.f;
    g[c] = ok ? dO[roff + c] : 0.f;
    dq[c] = 0.f;
  }
  const int kv_limit = frame_hi(sd.q_frame0 + row0 + nrows - 1, sd.P, sd.E);
  for (int kt = 0; kt < nk; ++kt) {
    const int c0 = kt * BN;
    __syncthreads();
    for (int c = tid; c < BN * D; c += 256) {
      const int row = c / D, col = c % D;
      const bool in = c0 + row < kv_limit;
      const long long gi = (long long)(sd.kv_base + c0 + row) * ld + h * D + col;
      Ks[row][col] = in ? K[gi] : 0.f;
      Vs[row][col] = in ? V[gi] : 0.f;
    }
    if (tid < BN) tsk[tid] = (use_t && c0 + tid < kv_limit) ? a.ts[sd.kv_base + c0 + tid] : 0;
    __syncthreads();
    const int jend = min(BN, kv_limit - c0);
    for (int jl = 0; jl < jend; ++jl) {
      const int j = c0 + jl;
      float s = 0.f, da = 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) {
        s = fmaf(q[c], Ks[jl][part * DP + c], s);
        da = fmaf(g[c], Vs[jl][part * DP + c], da);
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      da += __shfl_xor(da, 1, 64);
      da += __shfl_xor(da, 2, 64);
      int pidx = 0, tidx = 0;
      if (use_p) {
        pidx = pos_bucket(pos - j, a.n_pos);
        s += a.rab_p[pidx];
      }
      if (use_t && has_rt) {
        tidx = time_bucket(tq - tsk[jl], a.n_tb);
        s += a.rab_t[tidx];
      }
      if (j < hi && (!tfr || j < sd.P || tsk[jl] < tq)) {
        const float sg = 1.0f / (1.0f + expf(-s));
        const float ds = da * sg * (1.0f + s * (1.0f - sg));
#pragma unroll
        for (int c = 0; c < DP; ++c) dq[c] = fmaf(ds, Ks[jl][part * DP + c], dq[c]);
        if (part == 0) {
          if (use_p) atomicAdd(a.drab_p64 + pidx, (double)ds);
          if (use_t && has_rt) atomicAdd(a.drab_t64 + tidx, (double)ds);
        }
      }
    }
  }
  if (ok && fi >= sd.E) {
    const long long srow = (long long)(sd.self_base + fi - sd.E) * ld + h * D + part * DP;
    float s = 0.f, da = 0.f;
#pragma unroll
    for (int c = 0; c < DP; ++c) {
      s = fmaf(q[c], K[srow + c], s);
      da = fmaf(g[c], V[srow + c], da);
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    da += __shfl_xor(da, 1, 64);
    da += __shfl_xor(da, 2, 64);
    s += (use_p ? a.rab_p[0] : 0.f) + (use_t && has_rt ? a.rab_t[0] : 0.f);
    const float sg = 1.0f / (1.0f + expf(-s));
    const float ds = da * sg * (1.0f + s * (1.0f - sg));
    float *dK = (float *)a.dK, *dV = (float *)a.dV;
#pragma unroll
    for (int c = 0; c < DP; ++c) {
      dq[c] = fmaf(ds, K[srow + c], dq[c]);
      dK[srow + c] = ds * q[c] * a.inv_nmax;
      dV[srow + c] = s * sg * g[c] * a.inv_nmax;
    }
    if (part == 0) {
      if (use_p) atomicAdd(a.drab_p64, (double)ds);
      if (use_t && has_rt) atomicAdd(a.drab_t64, (double)ds);
    }
  }
  if (ok) {
    float *dQ = (float *)a.dQ;
#pragma unroll
    for (int c = 0; c < DP; ++c) dQ[roff + c] = dq[c] * a.inv_nmax;
  }
}

__global__ __launch_bounds__(256) void rab64_finalize_kernel(const double *acc_p, int n_pos, const double *acc_t,
                                                             int n_tb, float inv_nmax, float *drab_p, float *drab_t) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (acc_p && i < n_pos) drab_p[i] = (float)(acc_p[i] * (double)inv_nmax);
  if (acc_t && i < n_tb) drab_t[i] = (float)(acc_t[i] * (double)inv_nmax);
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(BwdArgs a) {
  constexpr int BM = 64, DP = D / 4;
  __shared__ float Qs[BM][D];
  __shared__ float Gs[BM][D];
  __shared__ long long tsr[BM];
  const int H = a.H;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  if (r >= a.hdr[kHdrNQ]) return;
  const QTile tile = a.tiles[r];
  const SeqDesc sd = a.desc[tile.b];
  const int k0 = tile.row0, qt_lo = tile.nf_nrows & 0xffff, nkeys = tile.nf_nrows >> 16;
  const int nq = tile.nk, L = sd.qcount;
  const long long ld = (long long)H * D;
  const int tid = threadIdx.x, lkey = tid >> 2, part = tid & 3;
  const float *Q = (const float *)a.Q, *K = (const float *)a.K, *V = (const float *)a.V;
  const float *dO = (const float *)a.dO;
  const bool use_p = a.rab_p != nullptr, use_t = a.ts != nullptr, has_rt = a.rab_t != nullptr;
  const bool kok = lkey < nkeys;
  const int key = k0 + (kok ? lkey : 0);
  const int rmin = kok ? (key < sd.P ? 0 : key) : 0x7fffffff;
  const long long koff = (long long)(sd.kv_base + key) * ld + h * D + part * DP;
  const long long tk = use_t ? a.ts[sd.kv_base + key] : 0;
  float k[DP], v[DP], dk[DP], dv[DP];
#pragma unroll
  for (int c = 0; c < DP; ++c) {
    k[c] = K[koff + c];
    v[c] = V[koff + c];
    dk[c] = dv[c] = 0.f;
  }
  for (int it = 0; it < nq; ++it) {
    const int fr0 = (qt_lo + it) * BM;
    __syncthreads();
    for (int c = tid; c < BM * D; c += 256) {
      const int row = c / D, col = c % D;
      const bool in = fr0 + row < L;
      const long long gi = (long long)(sd.q_base + fr0 + row) * ld + h * D + col;
      Qs[row][col] = in ? Q[gi] : 0.f;
      Gs[row][col] = in ? dO[gi] : 0.f;
    }
    if (tid < BM) tsr[tid] = (use_t && fr0 + tid < L) ? a.ts[sd.q_base + fr0 + tid] : 0;
    __syncthreads();
    const int rend = min(BM, L - fr0);
    for (int rl = 0; rl < rend; ++rl) {
      const int i = fr0 + rl;
      float s = 0.f, da = 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) {
        s = fmaf(Qs[rl][part * DP + c], k[c], s);
        da = fmaf(Gs[rl][part * DP + c], v[c], da);
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      da += __shfl_xor(da, 1, 64);
      da += __shfl_xor(da, 2, 64);
      if (use_p) s += a.rab_p[pos_bucket((i < sd.E ? i : sd.E) - key, a.n_pos)];
      if (use_t && has_rt) s += a.rab_t[time_bucket(tsr[rl] - tk, a.n_tb)];
      // under the timestamp filter a candidate row sees a causal key only if later
      const bool tf_ok = !(use_t && a.tfilt && i >= sd.E && key >= sd.P) || tk < tsr[rl];
      if (i >= rmin && tf_ok) {
        const float sg = 1.0f / (1.0f + expf(-s));
        const float p = s * sg;
        const float ds = da * sg * (1.0f + s * (1.0f - sg));
#pragma unroll
        for (int c = 0; c < DP; ++c) {
          dv[c] = fmaf(p, Gs[rl][part * DP + c], dv[c]);
          dk[c] = fmaf(ds, Qs[rl][part * DP + c], dk[c]);
        }
      }
    }
  }
  if (kok) {
    float *dK = (float *)a.dK, *dV = (float *)a.dV;
#pragma unroll
    for (int c = 0; c < DP; ++c) {
      dK[koff + c] = dk[c] * a.inv_nmax;
      dV[koff + c] = dv[c] * a.inv_nmax;
    }
  }
}

}  // namespace

#define HSTU_BWD_BF16_LAUNCH(KERNEL, NTHR)                                                      \
  template <int D, bool ZO>                                                                     \
  hipError_t launch_##KERNEL##_d(const BwdArgs &a, hipStream_t s) {                             \
    const bool p = a.rab_p != nullptr, t = a.ts != nullptr;                                     \
    const dim3 g(a.units), b(NTHR);                                                             \
    if (a.tfilt) {                                                                              \
      if (p) hipLaunchKernelGGL((KERNEL<D, true, true, true, ZO>), g, b, 0, s, a);                  \
      else hipLaunchKernelGGL((KERNEL<D, false, true, true, ZO>), g, b, 0, s, a);                   \
    } else if (p && t) {                                                                        \
      hipLaunchKernelGGL((KERNEL<D, true, true, false, ZO>), g, b, 0, s, a);                        \
    } else if (p) {                                                                             \
      hipLaunchKernelGGL((KERNEL<D, true, false, false, ZO>), g, b, 0, s, a);                       \
    } else if (t) {                                                                             \
      hipLaunchKernelGGL((KERNEL<D, false, true, false, ZO>), g, b, 0, s, a);                       \
    } else {                                                                                    \
      hipLaunchKernelGGL((KERNEL<D, false, false, false, ZO>), g, b, 0, s, a);                      \
    }                                                                                           \
    return hipGetLastError();                                                                   \
  }

template <int D, bool ZO>
hipError_t launch_bwd_dq_kernel_d(const BwdArgs &a, hipStream_t s) {
  const bool p = a.rab_p != nullptr, t = a.ts != nullptr;
  const dim3 g(a.units), b(256);
  if (a.tfilt) {
    if (p) hipLaunchKernelGGL((bwd_dq_kernel<D, true, true, true, false, ZO>), g, b, 0, s, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<D, false, true, true, false, ZO>), g, b, 0, s, a);
  } else if (p && a.no_cand) {
    if (t) hipLaunchKernelGGL((bwd_dq_kernel<D, true, true, false, true, ZO>), g, b, 0, s, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<D, true, false, false, true, ZO>), g, b, 0, s, a);
  } else if (p && t) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, true, true, false, false, ZO>), g, b, 0, s, a);
  } else if (p) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, true, false, false, false, ZO>), g, b, 0, s, a);
  } else if (t) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, false, true, false, false, ZO>), g, b, 0, s, a);
  } else {
    hipLaunchKernelGGL((bwd_dq_kernel<D, false, false, false, false, ZO>), g, b, 0, s, a);
  }
  return hipGetLastError();
}
HSTU_BWD_BF16_LAUNCH(bwd_dkdv_kernel, 256)

hipError_t launch_attn_bwd_dq_bf16(const BwdArgs &a, hipStream_t s) {
  if (a.units <= 0) return hipSuccess;
  switch (a.d) {
    case 32: return a.zq ? launch_bwd_dq_kernel_d<32, true>(a, s) : launch_bwd_dq_kernel_d<32, false>(a, s);
    case 64: return a.zq ? launch_bwd_dq_kernel_d<64, true>(a, s) : launch_bwd_dq_kernel_d<64, false>(a, s);
    case 128: return a.zq ? launch_bwd_dq_kernel_d<128, true>(a, s) : launch_bwd_dq_kernel_d<128, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bwd_dkdv_bf16(const BwdArgs &a, hipStream_t s) {
  if (a.units <= 0) return hipSuccess;
  switch (a.d) {
    case 32: return a.zq ? launch_bwd_dkdv_kernel_d<32, true>(a, s) : launch_bwd_dkdv_kernel_d<32, false>(a, s);
    case 64: return a.zq ? launch_bwd_dkdv_kernel_d<64, true>(a, s) : launch_bwd_dkdv_kernel_d<64, false>(a, s);
    case 128: return a.zq ? launch_bwd_dkdv_kernel_d<128, true>(a, s) : launch_bwd_dkdv_kernel_d<128, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bwd_dq_f32(const BwdArgs &a, hipStream_t s) {
  if (a.units <= 0) return hipSuccess;
  switch (a.d) {
    case 32: hipLaunchKernelGGL(bwd_dq_f32_kernel<32>, dim3(a.units), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, dim3(a.units), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, dim3(a.units), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rab64_finalize(const double *acc_p, int n_pos, const double *acc_t, int n_tb, float inv_nmax,
                                 float *drab_p, float *drab_t, hipStream_t s) {
  const int n = max(acc_p ? n_pos : 0, acc_t ? n_tb : 0);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rab64_finalize_kernel, dim3((n + 255) / 256), dim3(256), 0, s, acc_p, n_pos, acc_t, n_tb,
                     inv_nmax, drab_p, drab_t);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv_f32(const BwdArgs &a, hipStream_t s) {
  if (a.units <= 0) return hipSuccess;
  switch (a.d) {
    case 32: hipLaunchKernelGGL(bwd_dkdv_f32_kernel<32>, dim3(a.units), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, dim3(a.units), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(bwd_dkdv_f32_kernel<128>, dim3(a.units), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hstu
