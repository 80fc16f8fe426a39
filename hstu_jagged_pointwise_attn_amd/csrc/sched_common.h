// Per-sequence steps of the jagged tile schedule, shared by the scheduler
// kernel and by the attention forward, which can build its own tile for
// small batches instead of waiting for a scheduler launch.
//
// The masks of the method (causal; MTGR's static / real-time / candidate
// mask, MTGR deep read section 2; M-FALCON's candidate mask, HSTU blog
// section 4.2) give every query row i a visible key set that is a prefix
// [0, hi(i)) of its sequence once a candidate's pair with itself is taken
// out; hi is non-decreasing (frame_hi).
#pragma once

#include "hstu_internal.h"
#include "../../include/hstu.h"
#include "device_common.h"

namespace hstu {
namespace sched_dev {

using dev::frame_hi;

// Validated frame of sequence b (see SeqDesc). Offending sequences come back
// with valid = 0 and qcount = 0, and their status bits in *bits.
__device__ inline SeqDesc seq_info(const SchedArgs &a, int b, int *bits) {
  SeqDesc s{};
  *bits = 0;
  if (a.mode != kSchedMFalcon) {
    long long beg = a.offsets[b], end = a.offsets[b + 1];
    int P = a.prefix ? a.prefix[b] : 0;
    int C = a.cand ? a.cand[b] : 0;
    long long L = end - beg;
    if (beg < 0 || end < beg || end > a.Tq) *bits |= HSTU_DEV_BAD_OFFSETS;
    else if (L > a.max_len) *bits |= HSTU_DEV_TOO_LONG;
    else if (P < 0 || C < 0 || (long long)P + C > L) *bits |= HSTU_DEV_BAD_SEGMENTS;
    if (*bits) return s;
    s.q_base = (int)beg;
    s.kv_base = (int)beg;
    s.E = (int)L - C;
    s.P = P;
    s.self_base = (int)beg + s.E;
    s.q_frame0 = 0;
    s.qcount = (int)L;
    s.valid = 1;
  } else {
    long long hb = a.hist_offsets[b], he = a.hist_offsets[b + 1];
    long long cb = a.cand_offsets[b], ce = a.cand_offsets[b + 1];
    if (hb < 0 || he < hb || he > a.Tkv || cb < 0 || ce < cb || ce > a.Tq)
      *bits |= HSTU_DEV_BAD_OFFSETS;
    else if (he - hb > a.hist_max_len || ce - cb > a.max_len)
      *bits |= HSTU_DEV_TOO_LONG;
    if (*bits) return s;
    int n = (int)(he - hb);
    s.q_base = (int)cb;
    s.kv_base = (int)hb;
    s.self_base = (int)cb;
    s.q_frame0 = n;
    s.P = 0;
    s.E = n;
    s.qcount = (int)(ce - cb);
    s.valid = 1;
  }
  return s;
}

__device__ __forceinline__ int div_up(int x, int y) { return (x + y - 1) / y; }

// Number of work records (query tiles, or key tiles in key-major mode) of a sequence.
__device__ inline int qtile_count(const SchedArgs &a, const SeqDesc &s) {
  const int q = s.qcount;
  if (q <= 0) return 0;
  if (a.mode == kSchedKeys) return div_up(s.E, a.BN);
  if (a.mode == kSchedAttn || a.microbatch <= 0 || a.microbatch >= q) return div_up(q, a.BM);
  int bm = a.microbatch, tpm = div_up(bm, a.BM);
  return (q / bm) * tpm + div_up(q % bm, a.BM);
}

// Record of the t-th query tile (canonical order) of sequence s.
__device__ inline QTile make_tile(const SchedArgs &a, const SeqDesc &s, int b, int t) {
  int row0, nrows;
  if (a.mode == kSchedKeys) {
    const int k0 = t * a.BN;
    const int nkeys = min(a.BN, s.E - k0);
    const int qt_lo = (k0 < s.P ? 0 : k0) / a.BM;
    const int qt_hi = div_up(s.qcount, a.BM);
    QTile r;
    r.b = b;
    r.row0 = k0;
    r.nk = qt_hi - qt_lo;
    r.nf_nrows = qt_lo | (nkeys << 16);
    return r;
  }
  if (a.mode == kSchedAttn || a.microbatch <= 0 || a.microbatch >= s.qcount) {
    row0 = t * a.BM;
    nrows = min(a.BM, s.qcount - row0);
  } else {
    int bm = a.microbatch, tpm = div_up(bm, a.BM);
    int mb = t / tpm, ti = t % tpm;
    row0 = mb * bm + ti * a.BM;
    int end = min(s.qcount, (mb + 1) * bm);
    nrows = min(a.BM, end - row0);
  }
  int i0 = s.q_frame0 + row0, i1 = i0 + nrows - 1;
  int nk = div_up(frame_hi(i1, s.P, s.E), a.BN);
  int nf = frame_hi(i0, s.P, s.E) / a.BN;
  // Under the timestamp filter a candidate row is sure to see only the prefix.
  if (a.time_filter && i1 >= s.E) nf = min(nf, s.P / a.BN);
  QTile r;
  r.b = b;
  r.row0 = row0;
  r.nk = nk;
  r.nf_nrows = nf | (nrows << 16);
  return r;
}

// Query tile r of an attention-mode schedule (kSchedAttn), found by the
// calling workgroup itself, for batches of at most NT sequences (NT = the
// workgroup's thread count). Thread b validates sequence b and counts its
// query tiles, a workgroup scan gives each sequence's first tile, and every
// thread then searches those offsets for r. Tiles come in canonical order
// (sequence, then rows); the records are the scheduler kernel's. With
// `report` the workgroup also writes the header words the scheduler kernel
// writes (status bits, first offending sequence, tile count). `lds` is
// NT + NT / 64 + 3 ints of LDS, free again when the function returns.
// Returns false (uniformly) when r is past the end of the list.
template <int NT>
__device__ inline bool inline_tile(const SchedArgs &a, int r, bool report, int *lds, QTile *tile, SeqDesc *sd) {
  static_assert(NT % 64 == 0 && NT <= 1024, "whole waves");
  constexpr int NW = NT / 64;
  int *s_off = lds, *s_w = lds + NT + 1, *s_bits = s_w + NW, *s_first = s_bits + 1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int bits = 0, nq = 0;
  if (tid < a.B) {
    const SeqDesc s = seq_info(a, tid, &bits);
    nq = qtile_count(a, s);
  }
  int first = bits ? tid : 0x7fffffff;
  if (tid == 0 && (a.offsets[0] != 0 || (long long)a.offsets[a.B] != a.Tq)) {
    bits |= HSTU_DEV_BAD_OFFSETS;
    first = -1;
  }
  int x = nq;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[w] = x;
  if (tid == 0) {
    *s_bits = 0;
    *s_first = 0x7fffffff;
  }
  __syncthreads();
  if (report && bits) {
    atomicOr(s_bits, bits);
    atomicMin(s_first, first);
  }
  int pre = 0, total = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const int v = s_w[k];
    pre += k < w ? v : 0;
    total += v;
  }
  if (tid < a.B) s_off[tid] = pre + x - nq;
  __syncthreads();
  // A list longer than the capacity (possible only with inconsistent
  // offsets) runs nothing, as in the scheduler kernel.
  const int NQ = total <= a.max_tiles ? total : 0;
  if (report && tid == 0) {
    int b = *s_bits, f = *s_first;
    if (total > a.max_tiles) {
      b |= HSTU_DEV_BAD_OFFSETS;
      f = -1;
    }
    a.hdr[kHdrStatus] = b;
    a.hdr[kHdrFirstBad] = f;
    a.hdr[kHdrNQ] = NQ;
  }
  bool found = false;
  if (r < NQ) {
    int lo = 0, hi = a.B;  // largest b with s_off[b] <= r
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= r) lo = mid; else hi = mid;
    }
    int bb;
    const SeqDesc s = seq_info(a, lo, &bb);
    const QTile t = make_tile(a, s, lo, r - s_off[lo]);
    // The values are the same in every lane: keep them in scalar registers.
    const auto u = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    tile->b = u(t.b);
    tile->row0 = u(t.row0);
    tile->nk = u(t.nk);
    tile->nf_nrows = u(t.nf_nrows);
    sd->q_base = u(s.q_base);
    sd->kv_base = u(s.kv_base);
    sd->self_base = u(s.self_base);
    sd->q_frame0 = u(s.q_frame0);
    sd->P = u(s.P);
    sd->E = u(s.E);
    sd->qcount = u(s.qcount);
    sd->valid = u(s.valid);
    found = true;
  }
  __syncthreads();
  return found;
}

}  // namespace sched_dev
}  // namespace hstu
