// Jagged tile scheduler: one workgroup turns the offsets of a jagged batch
// into the list of query tiles the attention kernels run, with no padding and
// no host round trip.
//
// The masks of the method (causal; MTGR's static / real-time / candidate
// mask, MTGR deep read section 2 "动态混合掩码"; M-FALCON's candidate mask,
// HSTU blog section 4.2) all give every query row a visible key set that is a
// prefix [0, hi(i)) of its sequence, once a candidate's pair with itself is
// taken out (that pair is added per row by the attention kernel):
//   hi(i) = P for i < P,  i + 1 for P <= i < E,  E for i >= E,
// and hi is non-decreasing in i. So the key tiles a query tile [i0, i1]
// touches are [0, ceil(hi(i1)/BN)), the first floor(hi(i0)/BN) of them fully
// visible. Tiles with no visible pair are never listed. Under MTGR's
// timestamp filter a candidate sees a causal key only if the key is earlier;
// the schedule does not read timestamps, so for a query tile with candidate
// rows only the prefix tiles count as fully visible and the kernels test the
// remaining pairs one by one.
//
// Steps: per-sequence validation and query-tile counts -> exclusive scan ->
// one record per query tile -> longest-first order (bitonic sort in LDS on
// the unique key (nk descending, canonical index ascending)).
//
// Key-major mode (the dK/dV backward): one record per key tile [k0, k0+BN)
// of the non-candidate keys [0, E) (a candidate key is seen only by itself);
// the rows that see key j form the suffix i >= (j < P ? 0 : j), so the
// record lists the query tiles [qt_lo, qt_hi) of BM rows from
// (k0 < P ? 0 : k0) to the end of the sequence.
#include "hstu_internal.h"
#include "../../include/hstu.h"
#include "sched_common.h"

namespace hstu {
namespace {

using namespace sched_dev;

// Exclusive scan of one value per thread across the workgroup.
__device__ int block_exclusive_scan(int v, int *s_wsum, int *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int NW = kSchedThreads / 64;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    int ws = lane < NW ? s_wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      int y = __shfl_up(ws, o, 64);
      if (lane >= o) ws += y;
    }
    if (lane < NW) s_wsum[lane] = ws;
  }
  __syncthreads();
  int excl = (w > 0 ? s_wsum[w - 1] : 0) + x - v;
  *total = s_wsum[NW - 1];
  __syncthreads();
  return excl;
}

template <int CTRL>
__device__ __forceinline__ unsigned dpp_u32(unsigned x) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// The value of lane (lane ^ J), J < 64. J = 1, 2: quad permutes; J = 8: a
// rotation by 8 within the row of 16; J = 4: one of the rotations by 4 and
// by 12, whichever reaches lane ^ 4 (fwd4, found once from the lane ids);
// J = 16, 32: a lane permute through the LDS crossbar. All lanes active.
template <int J>
__device__ __forceinline__ unsigned lane_xor(unsigned x, bool fwd4) {
  if constexpr (J == 1) return dpp_u32<0xB1>(x);  // quad_perm 1,0,3,2
  else if constexpr (J == 2) return dpp_u32<0x4E>(x);  // quad_perm 2,3,0,1
  else if constexpr (J == 4) {
    const unsigned a = dpp_u32<0x124>(x), b = dpp_u32<0x12C>(x);  // row_ror 4, 12
    return fwd4 ? a : b;
  } else if constexpr (J == 8) return dpp_u32<0x128>(x);  // row_ror 8
  else return (unsigned)__shfl_xor((int)x, J, 64);
}

// One compare-exchange stage of distance J < 64 on the E keys of a thread
// (index tid + e * kSchedThreads), partners in the same wave.
template <int J, int E>
__device__ __forceinline__ void wave_stage(unsigned (&x)[E], int k, bool fwd4) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid + e * kSchedThreads;
    const unsigned y = lane_xor<J>(x[e], fwd4);
    const bool up = (i & k) == 0, lower = (i & J) == 0;
    x[e] = (lower == up) ? min(x[e], y) : max(x[e], y);
  }
}

// Bitonic sort of n2 keys (a power of two, at most E * kSchedThreads), E per
// thread at indices tid + e * kSchedThreads, kept in registers. Per merge
// size k, the stages run from distance k/2 down to 1: partners in the same
// thread (distance >= kSchedThreads), through two LDS buffers used in turn
// with one barrier each (64 .. kSchedThreads/2), then within the wave as
// straight-line code (32 .. 1), so that a stage costs a few vector
// instructions and no scalar branching. keys holds the input and receives
// the output; tmp is the second buffer. Every thread of the block calls it.
template <int E>
__device__ void sort_keys(unsigned *keys, unsigned *tmp, int n2) {
  const int tid = threadIdx.x, lane = tid & 63;
  const bool fwd4 = dpp_u32<0x124>((unsigned)lane) == (unsigned)(lane ^ 4);
  unsigned x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid + e * kSchedThreads;
    x[e] = i < n2 ? keys[i] : 0xffffffffu;
  }
  int pb = 0;
  for (int k = 2; k <= n2; k <<= 1) {
    int j = k >> 1;
    if constexpr (E > 1) {
      for (; j >= kSchedThreads; j >>= 1) {
        const int d = j / kSchedThreads;
#pragma unroll
        for (int e = 0; e < E; ++e) {
#pragma unroll
          for (int f = e + 1; f < E; ++f) {
            if (f != (e | d) || (e & d)) continue;
            const bool up = ((tid + e * kSchedThreads) & k) == 0;
            const unsigned lo = min(x[e], x[f]), hi = max(x[e], x[f]);
            x[e] = up ? lo : hi;
            x[f] = up ? hi : lo;
          }
        }
      }
    }
    for (; j >= 64; j >>= 1) {
      unsigned *bb = pb ? tmp : keys;
      pb ^= 1;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = tid + e * kSchedThreads;
        if (i < n2) bb[i] = x[e];
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = tid + e * kSchedThreads;
        const unsigned y = i < n2 ? bb[i ^ j] : 0xffffffffu;
        const bool up = (i & k) == 0, lower = (i & j) == 0;
        x[e] = (lower == up) ? min(x[e], y) : max(x[e], y);
      }
    }
    switch (j) {
      case 32: wave_stage<32>(x, k, fwd4); [[fallthrough]];
      case 16: wave_stage<16>(x, k, fwd4); [[fallthrough]];
      case 8: wave_stage<8>(x, k, fwd4); [[fallthrough]];
      case 4: wave_stage<4>(x, k, fwd4); [[fallthrough]];
      case 2: wave_stage<2>(x, k, fwd4); [[fallthrough]];
      case 1: wave_stage<1>(x, k, fwd4); break;
      default: break;
    }
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid + e * kSchedThreads;
    if (i < n2) keys[i] = x[e];
  }
  __syncthreads();
}

// Sort key of record g (ascending = run first). Longest first: (record
// length descending, g). By sequence: (sequence length descending, then the
// sequence's records longest first: g descending for query tiles, whose
// length grows with the row, g ascending for key tiles, whose length shrinks
// with the key). Lengths are in key (or query) tiles, below kMaxKeyTiles;
// g < 2^18 (kSortCap).
__device__ __forceinline__ unsigned sort_key(const SchedArgs &a, const SeqDesc &s, const QTile &r, int g) {
  if (a.order != kOrderBySequence || a.mode == kSchedMFalcon)
    return ((unsigned)(kMaxKeyTiles - r.nk) << 18) | (unsigned)g;
  int len;
  unsigned low;
  if (a.mode == kSchedKeys) {
    len = (s.qcount + a.BM - 1) / a.BM;  // the first key tile sees every query tile
    low = (unsigned)g;
  } else {
    len = (frame_hi(s.q_frame0 + s.qcount - 1, s.P, s.E) + a.BN - 1) / a.BN;  // the last query tile's
    low = 0x3ffffu - (unsigned)g;
  }
  len = min(len, kMaxKeyTiles);
  return ((unsigned)(kMaxKeyTiles - len) << 18) | low;
}

__device__ __forceinline__ int key_index(const SchedArgs &a, unsigned key) {
  const int low = (int)(key & 0x3ffffu);
  return (a.order == kOrderBySequence && a.mode == kSchedAttn) ? 0x3ffff - low : low;
}

__device__ __forceinline__ void sched_body(const SchedArgs &a) {
  constexpr int kRecCache = kSchedThreads;  // records kept in LDS for short lists
  __shared__ int s_qoff[kMaxSeqs + 1];
  __shared__ unsigned s_keys[kSortCap];
  __shared__ unsigned s_tmp[kSortCap];
  __shared__ QTile s_rec[kRecCache];
  __shared__ int s_wsum[kSchedThreads / 64];
  __shared__ int s_bits, s_first;
  const int tid = threadIdx.x;

  // Status: accumulated in LDS, written once at the end.
  if (tid == 0) {
    s_bits = 0;
    s_first = 0x7fffffff;
  }
  __syncthreads();
  if (tid == 0) {
    bool bad;
    if (a.mode != kSchedMFalcon)
      bad = a.offsets[0] != 0 || (long long)a.offsets[a.B] != a.Tq;
    else
      bad = a.cand_offsets[0] != 0 || (long long)a.cand_offsets[a.B] != a.Tq ||
            a.hist_offsets[0] != 0 || (long long)a.hist_offsets[a.B] != a.Tkv;
    if (bad) {
      atomicOr(&s_bits, HSTU_DEV_BAD_OFFSETS);
      atomicMin(&s_first, -1);
    }
  }

  // Per-sequence validation, descriptors and query-tile counts; scan.
  int carry = 0;
  for (int base = 0; base < a.B; base += kSchedThreads) {
    int b = base + tid, nq = 0;
    if (b < a.B) {
      int bits;
      SeqDesc s = seq_info(a, b, &bits);
      if (bits) {
        atomicOr(&s_bits, bits);
        atomicMin(&s_first, b);
      }
      a.desc[b] = s;
      nq = qtile_count(a, s);
    }
    int total;
    int excl = block_exclusive_scan(nq, s_wsum, &total);  // contains barriers
    if (b < a.B) s_qoff[b] = carry + excl;
    carry += total;
  }
  if (tid == 0) s_qoff[a.B] = carry;
  __syncthreads();
  // Sequences that overlap (possible only with inconsistent offsets) could
  // exceed the capacity sized from the token count: then nothing runs.
  const int NQ = carry <= a.max_tiles ? carry : 0;
  for (int b = tid; b <= a.B; b += kSchedThreads) a.qoff[b] = s_qoff[b];

  const bool sorted = NQ <= kSortCap;
  const bool cached = NQ <= kRecCache;
  int n2 = 1;
  while (n2 < NQ) n2 <<= 1;

  // One record per query tile; sort keys when the list fits in LDS.
  for (int g = tid; g < (sorted ? n2 : NQ); g += kSchedThreads) {
    if (g >= NQ) {
      s_keys[g] = 0xffffffffu;
      continue;
    }
    int lo = 0, hi = a.B;  // largest b with s_qoff[b] <= g
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (s_qoff[mid] <= g) lo = mid; else hi = mid;
    }
    int bits;
    SeqDesc s = seq_info(a, lo, &bits);
    QTile r = make_tile(a, s, lo, g - s_qoff[lo]);
    if (cached) s_rec[g] = r;
    if (sorted) s_keys[g] = sort_key(a, s, r, g);
    else a.tiles[g] = r;
  }
  __syncthreads();
  if (tid == 0) {
    int bits = s_bits, first = s_first;
    if (carry > a.max_tiles) {
      bits |= HSTU_DEV_BAD_OFFSETS;
      first = -1;
    }
    a.hdr[kHdrStatus] = bits;
    a.hdr[kHdrFirstBad] = first;
    a.hdr[kHdrNQ] = NQ;
  }
  if (!sorted) return;

  static_assert(kSortCap <= 8 * kSchedThreads, "at most 8 keys per thread");
  if (n2 <= kSchedThreads) sort_keys<1>(s_keys, s_tmp, n2);
  else if (n2 <= 2 * kSchedThreads) sort_keys<2>(s_keys, s_tmp, n2);
  else if (n2 <= 4 * kSchedThreads) sort_keys<4>(s_keys, s_tmp, n2);
  else sort_keys<8>(s_keys, s_tmp, n2);

  for (int r = tid; r < NQ; r += kSchedThreads) {
    const int g = key_index(a, s_keys[r]);
    if (cached) {
      a.tiles[r] = s_rec[g];
      continue;
    }
    int lo = 0, hi = a.B;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (s_qoff[mid] <= g) lo = mid; else hi = mid;
    }
    int bits;
    SeqDesc s = seq_info(a, lo, &bits);
    a.tiles[r] = make_tile(a, s, lo, g - s_qoff[lo]);
  }
}

__global__ __launch_bounds__(kSchedThreads) void sched_kernel(SchedArgs a) { sched_body(a); }

// Two independent schedules in one launch (workgroup 0 builds a, 1 builds b).
__global__ __launch_bounds__(kSchedThreads) void sched_pair_kernel(SchedArgs a, SchedArgs b) {
  if (blockIdx.x == 0) sched_body(a);
  else sched_body(b);
}

}  // namespace

hipError_t launch_sched(const SchedArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kSchedThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sched_pair(const SchedArgs &a, const SchedArgs &b, hipStream_t s) {
  hipLaunchKernelGGL(sched_pair_kernel, dim3(2), dim3(kSchedThreads), 0, s, a, b);
  return hipGetLastError();
}

}  // namespace hstu
