// Internal declarations shared by the HIP kernels and the C-ABI layer of
// libhstu.so. Device code targets gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hstu.h"

namespace hstu {

// Per-sequence frame of the attention core. A "frame" is the sequence as the
// mask sees it: frame indices [0, P) are the bidirectional prefix, [P, E) the
// causal part, and indices >= E candidates. For the plain forward the query
// rows are frame rows [0, L); for M-FALCON scoring the query rows are the
// candidates, frame rows [n, n + m), and the keys are the cached history.
struct SeqDesc {
  int q_base;     // first query row of the sequence in Q/U/O/Y (and query timestamps)
  int kv_base;    // first key row in K/V (and key timestamps)
  int self_base;  // row of the first candidate in the self-term K/V arrays
  int q_frame0;   // frame index of the first query row
  int P, E;       // prefix end and candidate start, in frame indices
  int qcount;     // number of query rows
  int valid;      // 0 when the sequence failed a device-side check (treated as empty)
};

// One query tile of the work list: key tiles [0, nf) are FULL (every pair
// visible, no mask), [nf, nk) PARTIAL (mask applied), rows [row0, row0+nrows)
// are local query rows of sequence b.
struct QTile {
  int b, row0, nk, nf_nrows;  // nf | nrows << 16
};

// Workspace header words.
constexpr int kHdrStatus = 0;    // OR of HSTU_DEV_* bits
constexpr int kHdrFirstBad = 1;  // smallest offending sequence index
constexpr int kHdrNQ = 2;        // number of query tiles
// Timestamp flag of a forward whose workgroups built their own tiles: the
// attention kernel stores the call's epoch there when it meets a timestamp
// out of range, and the norm kernel that follows moves that into
// kHdrStatus and overwrites the word (so no flag outlives its call).
constexpr int kHdrInlineTs = 3;
constexpr int kHdrWords = 64;    // 256 bytes

constexpr int kSchedThreads = 1024;
constexpr int kSortCap = 8192;   // longest-first order up to this many query tiles
constexpr int kMaxSeqs = 8192;   // sequences per call (query-tile offsets live in LDS)
constexpr int kMaxKeyTiles = 16383;

enum SchedMode { kSchedAttn = 0, kSchedMFalcon = 1, kSchedKeys = 2 };

// Work-list orders (hstu_set_tile_order): longest record first, or whole
// sequences longest first with each sequence's records together (its
// longest first), which keeps a sequence's K/V (Q/dO for the key-major
// pass) in one L2 while its records run. M-FALCON lists are always
// longest first.
enum TileOrder { kOrderLongest = 0, kOrderBySequence = 1 };

// A forward of at most this many sequences and work units (query tiles x
// heads, as bounded on the host) skips the scheduler launch: every attention
// workgroup finds its own tile (sched_dev::inline_tile). At this size all
// units run at once or nearly, so the longest-first order has nothing to win.
constexpr int kInlineSchedMaxSeqs = 256;
constexpr long long kInlineSchedMaxUnits = 1024;

struct SchedArgs {
  int mode;
  // attention forward: one jagged batch
  const int *offsets, *prefix, *cand;
  // M-FALCON: candidate offsets (query rows) and history offsets (keys)
  const int *cand_offsets, *hist_offsets;
  int B;
  long long Tq, Tkv;
  int max_len, hist_max_len;
  int BM, BN, microbatch;
  int time_filter; // candidates see causal keys by timestamp: their causal tiles are never full
  int order;       // kOrderLongest or kOrderBySequence (attention and key-major modes)
  int max_tiles;   // capacity of `tiles`; a larger count marks the offsets bad and runs nothing
  int *hdr;
  SeqDesc *desc;
  int *qoff;
  QTile *tiles;
};

hipError_t launch_sched(const SchedArgs &a, hipStream_t s);
// Builds two independent schedules in one launch (one workgroup each).
hipError_t launch_sched_pair(const SchedArgs &a, const SchedArgs &b, hipStream_t s);

// Forward attention kernels. Arrays are token-major with row stride H*d.
struct FwdArgs {
  const void *Q, *K, *V;          // query rows / key rows
  const void *Kself, *Vself;      // rows used by a candidate's pair with itself
  void *O;                        // [Tq, H*d] output, scaled by 1/N_max
  const int64_t *ts_q, *ts_kv;    // timestamps of query / key rows (rab_t or the filter), or NULL
  const float *rab_p, *rab_t;
  int n_pos, n_tb;
  float inv_nmax;
  int H, d;
  int tfilt;                      // candidates see causal-segment keys only if strictly earlier
  int *hdr;                       // header words (tile count in, status bits out)
  const SeqDesc *desc;
  const QTile *tiles;
  int units;                      // grid size bound: max query tiles * H
  // Small batches: each workgroup builds its own tile from `sched`
  // (kSchedAttn) instead of reading desc / tiles, and a timestamp out of
  // range is flagged by storing `epoch` into hdr[kHdrInlineTs].
  int inline_sched;
  unsigned epoch;
  SchedArgs sched;
};

// bf16 inputs, MFMA, tile 128 x 64
constexpr int kFwdBM = 128, kFwdBN = 64;
// fp32 inputs, vector ALU, tile 64 x 64
constexpr int kF32BM = 64, kF32BN = 64;

hipError_t launch_attn_fwd_bf16(const FwdArgs &a, hipStream_t s);
hipError_t launch_attn_fwd_f32(const FwdArgs &a, hipStream_t s);

// Per-token Norm(x) * u (forward) and its backward.
struct NormArgs {
  const void *X;        // [T, D] pre-norm attention output
  const void *U;        // [T, D]
  void *Y;              // [T, D]
  float *mean, *rstd;   // [T] or NULL (norm NONE)
  const uint8_t *group; // [T] or NULL
  const float *gamma, *beta;  // [G, D] or NULL
  int n_groups;
  int mode;             // 0 none, 1 LN, 2 GLN
  float eps;
  long long T;
  int D;
  int *hdr;             // status word (group id violations)
  // After an attention forward with inline_sched: fold hdr[kHdrInlineTs] ==
  // epoch into the status word, then overwrite it.
  int merge_ts;
  unsigned epoch;
};
hipError_t launch_norm_fwd(const NormArgs &a, bool bf16, hipStream_t s);

struct NormBwdArgs {
  const void *X, *U, *dY;         // [T, D] pre-norm output, gate, output gradient
  const float *mean, *rstd;       // [T]
  const uint8_t *group;           // [T] or NULL
  const float *gamma, *beta;      // [G, D] or NULL
  int n_groups, mode;
  long long T;
  int D;
  int tokens_per_wave;            // contiguous tokens handled by one wave
  void *dU;                       // [T, D], row stride ldu
  long long ldu;                  // D, or 4 D when dU is a column block of a layer's dZ
  const void *zu;                 // with it (bf16 only), dU is multiplied by SiLU'(zu) (row stride ldu)
  void *dX;                       // [T, D] gradient w.r.t. the pre-norm output
  float *dgamma, *dbeta;          // [G, D] accumulated with atomics (zeroed by the caller), or NULL
  // When set, dgamma / dbeta are instead summed per workgroup in LDS into
  // partial [workgroups][2][G][D] (fp32) and reduced by launch_norm_affine_reduce.
  float *partial;
};
hipError_t launch_norm_bwd(const NormBwdArgs &a, bool bf16, hipStream_t s);
// Workgroups of the norm backward launch for these sizes.
long long norm_bwd_blocks(long long T, int tokens_per_wave);
// dgamma / dbeta (each [G, D], overwritten; either may be NULL) = the sum over
// `blocks` rows of partial [blocks][2][G][D].
hipError_t launch_norm_affine_reduce(const float *partial, long long blocks, int GD, float *dgamma, float *dbeta,
                                     hipStream_t s);
// Largest G * D whose two affine rows fit the norm backward's LDS accumulator.
constexpr int kNormAffineLdsMax = 8192;

// Backward attention kernels. dO is the gradient w.r.t. the pre-norm output
// (computed by the norm backward into the workspace).
struct BwdArgs {
  const void *Q, *K, *V, *dO;
  void *dQ, *dK, *dV;
  const int64_t *ts;               // timestamps (rab_t or the filter) or NULL
  const float *rab_p, *rab_t;      // tables or NULL
  float *drab_p, *drab_t;          // fp32 accumulators (zeroed by the caller)
  double *drab_p64, *drab_t64;     // fp32 path: fp64 accumulators of the unscaled sums (zeroed by the caller)
  int n_pos, n_tb;
  float inv_nmax;
  int H, d;
  int tfilt;                       // candidates see causal-segment keys only if strictly earlier
  int no_cand;                     // no sequence has candidates (cand_len is NULL)
  int *hdr;                        // header of the schedule this kernel runs
  int *status;                     // the call's status word (HSTU_DEV_* bits)
  const SeqDesc *desc;
  const QTile *tiles;
  int units;                       // grid bound: records * H
  // Row stride (elements) of dQ, dK, dV: H * d, or 4 H d when they are
  // column blocks of a layer's dZ. With zq / zk / zv set (bf16 only), each
  // is multiplied by SiLU' of the matching column block of the layer's
  // pre-activation Z (same row stride) before it is stored.
  long long ldo;
  const void *zq, *zk, *zv;
};
// bf16: the query-major dQ kernel runs the forward's query tiles (kFwdBM x
// kFwdBN); the key-major dK/dV kernel runs 64-key tiles x 64-row query steps.
constexpr int kBwdKBN = 64, kBwdKBM = 64;
hipError_t launch_attn_bwd_dq_bf16(const BwdArgs &a, hipStream_t s);
hipError_t launch_attn_bwd_dkdv_bf16(const BwdArgs &a, hipStream_t s);
hipError_t launch_attn_bwd_dq_f32(const BwdArgs &a, hipStream_t s);
hipError_t launch_attn_bwd_dkdv_f32(const BwdArgs &a, hipStream_t s);
// d rab_p[i] = acc_p[i] * inv_nmax and d rab_t[i] = acc_t[i] * inv_nmax,
// rounded once from fp64 (either table may be NULL).
hipError_t launch_rab64_finalize(const double *acc_p, int n_pos, const double *acc_t, int n_tb, float inv_nmax,
                                 float *drab_p, float *drab_t, hipStream_t s);

hipError_t launch_fill_f32(float *p, long long n, float v, hipStream_t s);

// Records `msg` as this thread's hstu_last_error text and returns st.
hstu_status_t set_last_error(hstu_status_t st, const char *msg);

// Batch preparation (Stochastic Length, row gather, work-balanced bins).
hipError_t launch_stochastic_length(const int *offsets, int B, long long T, int max_len, int cap,
                                    const unsigned *keys, int *new_offsets, int *gather_idx, int *status,
                                    hipStream_t s);
hipError_t launch_gather_rows(const void *src, const int *idx, long long n, long long row_bytes, void *dst,
                              hipStream_t s);
hipError_t launch_balance(const int *offsets, int B, int n_bins, int cost_kind, int *bin, long long *bin_cost,
                          hipStream_t s);

// Full layer (projections around the core). Row-major GEMM on hipBLASLt:
// C[M, N] = op(A) op(B) (+ bias over N) (+ C when accumulating); returns a
// hipblasStatus_t (0 = success).
enum GemmType { kGemmBF16 = 0, kGemmF32 = 1 };
struct GemmRM {
  bool ta, tb;              // op(A) = A^T, op(B) = B^T
  long long M, N, K;
  const void *A;            // stored [M, K] (ta false) or [K, M] (ta true), row stride lda
  long long lda;
  const void *B;            // stored [K, N] (tb false) or [N, K] (tb true), row stride ldb
  long long ldb;
  void *C;                  // [M, N], row stride ldc
  long long ldc;
  GemmType ab, c;           // element type of A and B, and of C
  const float *bias;        // fp32 [N] or NULL
  bool silu;                // C = SiLU(op(A) op(B) + bias) (the epilogue applies it before rounding)
  bool accumulate;
  int batch;                // > 1: a strided batch of GEMMs of these sizes
  long long sA, sB, sC;     // element offsets between consecutive batch entries
};
int gemm_rm(const GemmRM &g, void *ws, size_t ws_bytes, hipStream_t s);
// Creates the current device's hipBLASLt handle if needed (before a stream capture).
int gemm_init();
const char *gemm_status_text(int st);
bool gemm_unsupported(int st);  // no algorithm for the problem

hipError_t launch_silu_split(const void *Z, long long T, int D, bool bf16, void *U, void *V, void *Q, void *K,
                             hipStream_t s);
// Column sums run in two passes through a scratch `partial` of
// kColsumGroups * n floats (n = columns).
constexpr int kColsumGroups = 1024;
// db (fp32 [4D], overwritten with the column sums of dZ) may be NULL
hipError_t launch_dsilu(const void *Z, const void *dU, const void *dV, const void *dQ, const void *dK, long long T,
                        int D, bool bf16, void *dZ, float *partial, float *db, hipStream_t s);
// out[i] = sum over s < nslices of slices[s * n + i] (fp32, n elements)
hipError_t launch_sum_slices(const float *slices, int nslices, long long n, float *out, hipStream_t s);
// out (fp32 [n]) = column sums of M [T, n]
hipError_t launch_colsum(const void *M, long long T, int n, bool bf16, float *partial, float *out, hipStream_t s);

}  // namespace hstu
