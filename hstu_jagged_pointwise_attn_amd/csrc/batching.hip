// Batch preparation on the device, ahead of the attention layers.
//
// Stochastic Length (HSTU blog, section 3.4): a training sequence longer
// than a budget `cap` is cut down to a random subset of cap of its tokens
// (the budget the page gives is 4096^(alpha/2), about 776 at alpha = 1.6);
// shorter sequences are kept whole. The subset is uniform and keeps the
// tokens' order: with one random 32-bit key per token (an input, so that the
// result is reproducible), a long sequence keeps the cap tokens with the
// smallest (key, index). The output is the new offsets and, for every kept
// token, its index in the input batch, with which the caller gathers Q, K,
// V, U, timestamps (hstu_gather_rows).
//
// Work-balanced batching (MTGR deep read, section 2: batch sizes adapted so
// that every GPU holds the same number of tokens): sequences go to n_bins
// bins longest-first, each to the bin with the smallest cost so far (ties to
// the lowest bin); the cost of a sequence is its length, or its length
// squared for attention work.
#include "hstu_internal.h"
#include "../../include/hstu.h"

namespace hstu {
namespace {

constexpr int kBatchThreads = 1024;
constexpr int kSelThreads = 256;

__device__ int block_scan_excl(int v, int *s_w, int *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[w] = x;
  __syncthreads();
  if (w == 0) {
    int s = lane < nw ? s_w[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < nw) s_w[lane] = s;
  }
  __syncthreads();
  const int excl = (w > 0 ? s_w[w - 1] : 0) + x - v;
  *total = s_w[nw - 1];
  __syncthreads();
  return excl;
}

// New offsets (exclusive scan of min(L_b, cap)) and input validation. Any
// violation keeps nothing at all, so that the output stays within T rows.
__global__ __launch_bounds__(kBatchThreads) void sl_offsets_kernel(const int *offsets, int B, long long T,
                                                                   int max_len, int cap, int *new_offsets,
                                                                   int *status) {
  __shared__ int s_w[kBatchThreads / 64];
  __shared__ int s_bits;
  if (threadIdx.x == 0) s_bits = (offsets[0] != 0 || (long long)offsets[B] != T) ? HSTU_DEV_BAD_OFFSETS : 0;
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += kBatchThreads) {
    const long long L = (long long)offsets[b + 1] - offsets[b];
    if (L < 0 || offsets[b] < 0 || offsets[b + 1] > T) atomicOr(&s_bits, HSTU_DEV_BAD_OFFSETS);
    else if (L > max_len) atomicOr(&s_bits, HSTU_DEV_TOO_LONG);
  }
  __syncthreads();
  const bool bad = s_bits != 0;
  int carry = 0;
  for (int base = 0; base < B; base += kBatchThreads) {
    const int b = base + threadIdx.x;
    int k = 0;
    if (b < B && !bad) k = (int)min((long long)offsets[b + 1] - offsets[b], (long long)cap);
    int total;
    const int excl = block_scan_excl(k, s_w, &total);
    if (b < B) new_offsets[b] = carry + excl;
    carry += total;
  }
  if (threadIdx.x == 0) {
    new_offsets[B] = carry;
    *status = s_bits;
  }
}

// One workgroup per sequence: the indices of its kept tokens, in order.
__global__ __launch_bounds__(kSelThreads) void sl_select_kernel(const int *offsets, const int *new_offsets,
                                                                const unsigned *keys, int cap,
                                                                int *gather_idx) {
  __shared__ int hist[256];
  __shared__ int s_w[kSelThreads / 64];
  __shared__ unsigned s_prefix;
  __shared__ int s_need;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int beg = offsets[b], out = new_offsets[b];
  const int k = new_offsets[b + 1] - out;   // 0 for sequences the offsets kernel rejected
  const int L = offsets[b + 1] - beg;
  if (k <= 0) return;
  if (k == L) {
    for (int j = tid; j < L; j += kSelThreads) gather_idx[out + j] = beg + j;
    return;
  }
  // Radix select, most significant byte first: the k-th smallest key T and
  // how many keys equal to T are taken (need), keys below T all are.
  if (tid == 0) {
    s_prefix = 0u;
    s_need = k;
  }
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;  // kSelThreads == 256 bins
    __syncthreads();
    const unsigned prefix = s_prefix;
    const unsigned hmask = shift == 24 ? 0u : ~0u << (shift + 8);
    for (int j = tid; j < L; j += kSelThreads) {
      const unsigned key = keys[beg + j];
      if ((key & hmask) == (prefix & hmask)) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int need = s_need, d = 0;
      while (hist[d] < need) {
        need -= hist[d];
        ++d;
      }
      s_need = need;
      s_prefix = prefix | ((unsigned)d << shift);
    }
    __syncthreads();
  }
  const unsigned thr = s_prefix;
  const int need = s_need;
  // Ordered compaction: keep key < thr, and the first `need` keys == thr.
  int ties = 0, kept = 0;
  for (int base = 0; base < L; base += kSelThreads) {
    const int j = base + tid;
    unsigned key = 0xffffffffu;
    if (j < L) key = keys[beg + j];
    const bool tie = j < L && key == thr;
    int ttot;
    const int trank = ties + block_scan_excl(tie ? 1 : 0, s_w, &ttot);
    const bool keep = j < L && (key < thr || (tie && trank < need));
    int ktot;
    const int pos = kept + block_scan_excl(keep ? 1 : 0, s_w, &ktot);
    if (keep) gather_idx[out + pos] = beg + j;
    ties += ttot;
    kept += ktot;
  }
}

// Row gather: dst[r] = src[idx[r]] for rows of `words` elements of W (4 or
// 16 bytes), consecutive threads on consecutive elements of a row.
template <typename W>
__global__ void gather_rows_kernel(const W *src, const int *idx, long long n, long long words, W *dst) {
  const long long total = n * words;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long r = e / words, c = e % words;
    dst[e] = src[(long long)idx[r] * words + c];
  }
}

// Longest-first greedy assignment of sequences to bins (one workgroup).
constexpr int kBalCap = 8192;
// One step of a wave prefix minimum of (v, w) ordered by v then w: each
// lane takes its DPP source lane's pair when that is smaller; lanes without
// a source keep their own (the old value is the lane's own).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_min_step(long long &v, int &w) {
  const int lo = (int)(unsigned)(unsigned long long)v, hi = (int)((unsigned long long)v >> 32);
  const int olo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false);
  const int ohi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false);
  const int ow = __builtin_amdgcn_update_dpp(w, w, CTRL, ROW_MASK, 0xf, false);
  const long long ov = (long long)(((unsigned long long)(unsigned)ohi << 32) | (unsigned)olo);
  const bool take = ov < v || (ov == v && ow < w);
  v = take ? ov : v;
  w = take ? ow : w;
}

// The greedy assignment of the sorted items (wave 0, lane = bin): STEPS
// prefix-minimum steps cover 2^STEPS lanes.
template <int STEPS>
__device__ __forceinline__ void greedy(long long &load, int B, const long long *s_cost, const int *s_idx, int *bin) {
  const int tid = threadIdx.x;
  constexpr int kLast = (1 << STEPS) - 1;
  for (int r = 0; r < B; ++r) {
    const long long c = s_cost[r];  // same address in every lane: read early, off the critical path
    const int item = s_idx[r];
    long long best = load;
    int who = tid;
    dpp_min_step<0x111, 0xf>(best, who);                    // row_shr:1
    dpp_min_step<0x112, 0xf>(best, who);                    // row_shr:2
    dpp_min_step<0x114, 0xf>(best, who);                    // row_shr:4
    if constexpr (STEPS >= 4) dpp_min_step<0x118, 0xf>(best, who);  // row_shr:8
    if constexpr (STEPS >= 5) dpp_min_step<0x142, 0xa>(best, who);  // row_bcast:15
    if constexpr (STEPS >= 6) dpp_min_step<0x143, 0xc>(best, who);  // row_bcast:31
    const int winner = __builtin_amdgcn_readlane(who, kLast);
    if (tid == winner) load += c;
    if (tid == 0) bin[item] = winner;
  }
}

__global__ __launch_bounds__(kBatchThreads) void balance_kernel(const int *offsets, int B, int n_bins,
                                                                int cost_kind, int *bin, long long *bin_cost) {
  __shared__ long long s_cost[kBalCap];
  __shared__ int s_idx[kBalCap];
  const int tid = threadIdx.x;
  int n2 = 1;
  while (n2 < B) n2 <<= 1;
  for (int i = tid; i < n2; i += kBatchThreads) {
    if (i < B) {
      const long long L = max(0, offsets[i + 1] - offsets[i]);
      s_cost[i] = cost_kind == HSTU_COST_ATTENTION ? L * L : L;
      s_idx[i] = i;
    } else {
      s_cost[i] = -1;  // sorts last
      s_idx[i] = 0x7fffffff;
    }
  }
  __syncthreads();
  // Bitonic sort into (cost descending, index ascending).
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += kBatchThreads) {
        const int p = i ^ j;
        if (p > i) {
          const long long ci = s_cost[i], cp = s_cost[p];
          const int ii = s_idx[i], ip = s_idx[p];
          const bool i_first = ci > cp || (ci == cp && ii < ip);  // i precedes p in the order
          const bool up = (i & k) == 0;
          if (i_first != up) {
            s_cost[i] = cp;
            s_cost[p] = ci;
            s_idx[i] = ip;
            s_idx[p] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
  if (tid >= 64) return;
  // Wave 0: lane = bin. Each step takes the least loaded bin (lowest on ties):
  // an inclusive prefix minimum of (load, lane) with DPP row shifts (and row
  // broadcasts beyond 16 bins) leaves the winner in the last lane that holds
  // a bin's prefix; only as many steps as the bin count needs are taken.
  const long long kInf = 0x7fffffffffffffffLL;
  long long load = tid < n_bins ? 0 : kInf;
  if (n_bins <= 8) greedy<3>(load, B, s_cost, s_idx, bin);
  else if (n_bins <= 16) greedy<4>(load, B, s_cost, s_idx, bin);
  else if (n_bins <= 32) greedy<5>(load, B, s_cost, s_idx, bin);
  else greedy<6>(load, B, s_cost, s_idx, bin);
  if (tid < n_bins) bin_cost[tid] = load;
}

}  // namespace

hipError_t launch_stochastic_length(const int *offsets, int B, long long T, int max_len, int cap,
                                    const unsigned *keys, int *new_offsets, int *gather_idx, int *status,
                                    hipStream_t s) {
  hipLaunchKernelGGL(sl_offsets_kernel, dim3(1), dim3(kBatchThreads), 0, s, offsets, B, T, max_len, cap,
                     new_offsets, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || B == 0) return e;
  hipLaunchKernelGGL(sl_select_kernel, dim3(B), dim3(kSelThreads), 0, s, offsets, new_offsets, keys, cap,
                     gather_idx);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void *src, const int *idx, long long n, long long row_bytes, void *dst,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool v16 = row_bytes % 16 == 0 && (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0;
  const long long words = row_bytes / (v16 ? 16 : 4);
  const long long total = n * words;
  const unsigned blocks = (unsigned)min((total + 255) / 256, 65536LL);
  if (v16)
    hipLaunchKernelGGL(gather_rows_kernel<uint4>, dim3(blocks), dim3(256), 0, s, (const uint4 *)src, idx, n, words,
                       (uint4 *)dst);
  else
    hipLaunchKernelGGL(gather_rows_kernel<unsigned>, dim3(blocks), dim3(256), 0, s, (const unsigned *)src, idx, n,
                       words, (unsigned *)dst);
  return hipGetLastError();
}

hipError_t launch_balance(const int *offsets, int B, int n_bins, int cost_kind, int *bin, long long *bin_cost,
                          hipStream_t s) {
  hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(kBatchThreads), 0, s, offsets, B, n_bins, cost_kind, bin,
                     bin_cost);
  return hipGetLastError();
}

}  // namespace hstu
