/*
 * hstu.h — C ABI of the HSTU jagged pointwise-attention library (libhstu.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes is the pointwise-attention core of one HSTU layer
 * (HSTU blog "Meta HSTU: 生成式推荐系统的实践", section 3, the layer formula
 * A(X)V(X) = phi2(Q K^T + rab^{p,t}) V and O = f2(Norm(A V) * U), with phi2 =
 * SiLU per section 3.1 and the position/time biases of section 3.2), on
 * jagged batches (MTGR deep read, section 2: JaggedTensor, no padding), with:
 *
 *   s_ij = <q_i, k_j> + rab_p[min(|pos(i) - pos(j)|, n_pos - 1)]
 *                     + rab_t[min(n_tb - 1, floor(log2(max(1, |t_i - t_j|))))]
 *   a_ij = vis(i, j) ? SiLU(s_ij) / n_max : 0,   o_i = sum_j a_ij v_j
 *   y    = Norm(concat_h o^h) * u                (Norm over the D = H*d values
 *                                                 of a token: none, LayerNorm,
 *                                                 or Group LayerNorm)
 *
 * per sequence b of length L with a bidirectional prefix of P tokens and a
 * candidate tail of C tokens (E = L - C):
 *   rows i <  P : see keys j < P                      (static/history tokens)
 *   rows P<=i<E : see keys j <= i                     (causal)
 *   rows i >= E : see keys j < E and themselves       (candidates)
 * (MTGR deep read, section 2 "动态混合掩码"; fmread.com MTGR report, section
 * 三.1 "动态掩码策略"; HSTU blog section 4.2 for the candidate mask). Every
 * candidate sits at position E for rab_p. P = C = 0 is the plain causal mask.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host). Arrays are dense,
 *     row-major and token-major: Q, K, V, U are [T, H, d]; Y and O are
 *     [T, H*d]; dQ, dK, dV, dU like their inputs.
 *   - Element type of Q, K, V, U, O, Y, dY and the gradients: bf16 or fp32,
 *     one type per call (hstu_problem_t.dtype). rab tables, gamma/beta, the
 *     normalisation statistics and their gradients are fp32.
 *   - Q, K, V, U, Y, O, dY, dQ, dK, dV, dU, the K/V caches, gamma and beta
 *     must start on a 16-byte boundary (the kernels move 16-byte vectors);
 *     a misaligned pointer is rejected with HSTU_ERR_INVALID_ARG.
 *   - The caller owns every buffer. The library never allocates device
 *     memory: scratch comes from the workspace `ws` of at least
 *     hstu_workspace_size() bytes (256-byte aligned). Concurrent calls need
 *     distinct workspaces. (The one exception is the hipBLASLt handle that
 *     the full-layer entry points create per device on first use.)
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     and nothing synchronises the host, except where stated. Outputs are
 *     valid once the stream has reached the end of the call.
 *   - Outputs must not alias inputs.
 *   - Errors are returned as status codes; nothing aborts and nothing throws.
 *     Host-visible preconditions (scalars, NULL pointers, sizes) are checked
 *     before anything is enqueued. Device-data preconditions (offsets
 *     non-decreasing from 0 up to total_tokens, P + C <= L, group ids <
 *     n_groups, lengths <= max_len, timestamps of a sequence within 2^31 s
 *     of each other) are checked by the kernels: the first
 *     violation is recorded in the workspace (hstu_get_device_status), the
 *     offending sequences are treated as empty and nothing is written out of
 *     bounds; outputs of the offending sequences are then undefined.
 *   - hstu_last_error() returns a thread-local message for the last failure.
 */
#ifndef HSTU_H
#define HSTU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID_ARG = 1,  /* bad scalar, NULL required pointer, bad combination */
  HSTU_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. d not in {32, 64, 128}) */
  HSTU_ERR_WORKSPACE = 3,    /* ws NULL or smaller than hstu_workspace_size() */
  HSTU_ERR_HIP = 4           /* a HIP runtime call or launch failed */
} hstu_status_t;

typedef enum { HSTU_BF16 = 0, HSTU_F32 = 1 } hstu_dtype_t;

typedef enum { HSTU_NORM_NONE = 0, HSTU_NORM_LN = 1, HSTU_NORM_GLN = 2 } hstu_norm_t;

typedef enum { HSTU_OP_FWD = 0, HSTU_OP_BWD = 1, HSTU_OP_MFALCON = 2 } hstu_op_t;

/* Bits of the device status word (hstu_get_device_status). */
enum {
  HSTU_DEV_BAD_OFFSETS = 1,   /* offsets[0] != 0, decreasing, or offsets[B] != total_tokens */
  HSTU_DEV_BAD_SEGMENTS = 2,  /* prefix_len/cand_len negative or P + C > L */
  HSTU_DEV_BAD_GROUP = 4,     /* a token group id >= n_groups (that token uses gamma = 1, beta = 0) */
  HSTU_DEV_TOO_LONG = 8,      /* a sequence longer than max_len */
  HSTU_DEV_BAD_TIMESTAMPS = 16 /* a kernel met a timestamp 2^31 s or more away from the reference
                                  time of its tile (the tile's first row or key); this cannot
                                  happen when every sequence spans less than 2^31 s. A sequence
                                  with a larger span may or may not raise it; its rab_t terms and
                                  timestamp-filter decisions are then undefined */
};

/*
 * One jagged batch. Scalars are host values; pointers are device pointers.
 *   B            number of sequences (>= 0)
 *   H, d         heads and head width (d_qk = d_v = d, d in {32, 64, 128})
 *   dtype        hstu_dtype_t of the tensors
 *   total_tokens T = offsets[B]
 *   max_len      an upper bound of every sequence length (sizes the grids)
 *   offsets      int32 [B+1], non-decreasing, offsets[0] = 0
 *   prefix_len   int32 [B] bidirectional prefix per sequence, or NULL (0)
 *   cand_len     int32 [B] candidate tail per sequence, or NULL (0)
 *   timestamps   int64 [T] seconds, or NULL (rab_t term off)
 *   rab_p/n_pos  fp32 [n_pos] position bias shared by all heads, or NULL
 *   rab_t/n_tb   fp32 [n_tb] time-bucket bias shared by all heads, or NULL
 *   n_max        the constant N_max >= 1 of the 1/N_max scale
 *   norm, eps    hstu_norm_t and the LayerNorm epsilon (> 0)
 *   token_group  uint8 [T] group id per token (GLN only), n_groups in [1, 255]
 *   gamma, beta  fp32 [n_groups, H*d] affine of the norm, or NULL (identity);
 *                for LN only row 0 is used
 *   mask_flags   0, or HSTU_MASK_CAND_TIME_FILTER: MTGR's timestamp filter for
 *                candidates (MTGR deep read, section 2: exposure samples are
 *                filtered by timestamp to stay causal). A candidate row then
 *                sees a key of the causal segment [P, E) only if the key's
 *                timestamp is strictly earlier than the candidate's; prefix
 *                keys and the candidate's own pair are unaffected. Requires
 *                timestamps (the rab_t table may be NULL). For M-FALCON the
 *                whole history is the causal segment.
 */
enum { HSTU_MASK_CAND_TIME_FILTER = 1 };

typedef struct hstu_problem {
  int32_t B, H, d, dtype;
  int64_t total_tokens;
  int32_t max_len;
  int32_t n_max;
  const int32_t *offsets;
  const int32_t *prefix_len;
  const int32_t *cand_len;
  const int64_t *timestamps;
  const float *rab_p;
  const float *rab_t;
  int32_t n_pos, n_tb;
  int32_t norm;
  float eps;
  const uint8_t *token_group;
  int32_t n_groups;
  int32_t mask_flags;
  const float *gamma;
  const float *beta;
} hstu_problem_t;

/* Library version, e.g. "0.1.0". Host only. */
const char *hstu_version(void);

/* Thread-local text of the last error returned on this thread. Host only. */
const char *hstu_last_error(void);

/*
 * Workspace bytes needed by `op` on problem `p` (host only, touches no device
 * memory). For HSTU_OP_MFALCON, p describes the candidates (see
 * hstu_mfalcon_score), `microbatch` is the candidates-per-microbatch b_m
 * (0 = all) and `hist_max_len`, `hist_tokens` bound the cached histories;
 * the three are ignored for the other ops.
 */
hstu_status_t hstu_workspace_size(const hstu_problem_t *p, int32_t op, int32_t microbatch,
                                  int32_t hist_max_len, int64_t hist_tokens, size_t *bytes);

/*
 * Forward of the attention core (see the top of this file).
 *   Q, K, V, U   [T, H, d] inputs
 *   Y            [T, H*d] output  Norm(O) * U
 *   O            [T, H*d] output  the pre-norm attention output concat_h o^h
 *                (saved for hstu_attn_bwd)
 *   mean, rstd   fp32 [T] per-token statistics of the norm (NULL allowed when
 *                norm == NONE; then nothing is written)
 */
hstu_status_t hstu_attn_fwd(const hstu_problem_t *p, const void *Q, const void *K, const void *V,
                            const void *U, void *Y, void *O, float *mean, float *rstd, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * hstu_attn_fwd without a workspace, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation). Arguments and results as for hstu_attn_fwd; the
 * scratch it needs (the tile schedule: at most hstu_static_scratch_bytes(),
 * 4 MiB, which covers up to 8192 sequences and tens of millions of tokens)
 * lives in a static device array of the library, one per GPU, held until the
 * process ends. It calls no allocation routine. The array of the current
 * device is shared by every call on that device and keeps the last call's
 * contents (each call's scheduler rewrites all it reads): calls that overlap
 * on one GPU, e.g. on two streams, race. Returns HSTU_ERR_WORKSPACE, before
 * any GPU work, when hstu_workspace_size(p, HSTU_OP_FWD, ...) exceeds the
 * array. The stream must belong to the current device.
 */
hstu_status_t hstu_attn_fwd_static(const hstu_problem_t *p, const void *Q, const void *K, const void *V,
                                   const void *U, void *Y, void *O, float *mean, float *rstd, void *stream);

/* Bytes of the static scratch array of hstu_attn_fwd_static (host only). */
size_t hstu_static_scratch_bytes(void);

/*
 * Backward of hstu_attn_fwd given dY [T, H*d]. O, mean and rstd are the
 * forward's outputs for the same inputs. Writes dQ, dK, dV, dU (overwritten,
 * [T, H, d]), d_rab_p [n_pos] and d_rab_t [n_tb] (overwritten; required when
 * the corresponding table is given, else ignored), d_gamma and d_beta
 * ([n_groups, H*d], overwritten; NULL skips them; only produced when gamma
 * resp. beta is given). Timestamps carry no gradient. The rab, gamma and
 * beta gradients sum over all heads, tokens and sequences.
 */
hstu_status_t hstu_attn_bwd(const hstu_problem_t *p, const void *Q, const void *K, const void *V,
                            const void *U, const void *O, const float *mean, const float *rstd,
                            const void *dY, void *dQ, void *dK, void *dV, void *dU,
                            float *d_rab_p, float *d_rab_t, float *d_gamma, float *d_beta,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * M-FALCON ranking (HSTU blog, sections 4.2 "批量推理" and 4.3 "KV Caching"):
 * score the candidates of B users against each user's cached history K/V.
 * For user b the result equals the candidate rows of hstu_attn_fwd over the
 * sequence [history_b | candidates_b] with P = 0 and C = m_b: every candidate
 * sees the whole history and itself, sits at position n_b, and no candidate
 * sees another. Only candidate rows are computed.
 *   cand          describes the candidates: offsets [B+1] over Tc candidate
 *                 tokens (total_tokens = Tc, max_len = max m_b), timestamps =
 *                 candidate timestamps (or NULL), rab/norm/group/affine as in
 *                 hstu_problem_t; prefix_len and cand_len must be NULL.
 *   hist_offsets  int32 [B+1] over the cached history tokens (hist_tokens
 *                 total, hist_max_len >= every n_b), host scalars
 *   K_cache, V_cache  [Th, H, d] cached history keys and values
 *   hist_ts       int64 [Th] history timestamps (NULL iff cand->timestamps NULL)
 *   Qc, Kc, Vc, Uc    [Tc, H, d] the candidates' own projections
 *   microbatch    b_m > 0 cuts each user's candidates into microbatches of b_m
 *                 (query tiles never span two microbatches); 0 = one
 *                 microbatch. The result does not depend on b_m.
 *   Yc, Oc        [Tc, H*d] outputs (Norm(O) * U and the pre-norm O)
 *   mean, rstd    fp32 [Tc] statistics (NULL allowed when norm == NONE)
 */
hstu_status_t hstu_mfalcon_score(const hstu_problem_t *cand, const int32_t *hist_offsets,
                                 int64_t hist_tokens, int32_t hist_max_len, const void *K_cache,
                                 const void *V_cache, const int64_t *hist_ts, const void *Qc,
                                 const void *Kc, const void *Vc, const void *Uc,
                                 int32_t microbatch, void *Yc, void *Oc, float *mean, float *rstd,
                                 void *ws, size_t ws_bytes, void *stream);

/*
 * Query/key tile shape (host only) that `op` uses for `p`'s dtype and d.
 */
hstu_status_t hstu_tile_shape(const hstu_problem_t *p, int32_t op, int32_t *BM, int32_t *BN);

/*
 * Runs only the tile scheduler of `op` (HSTU_OP_FWD or HSTU_OP_MFALCON; for
 * the latter pass hist_offsets/hist_tokens/hist_max_len/microbatch as for
 * hstu_mfalcon_score, else NULL/0) on `stream`, waits for it, and copies to
 * host memory:
 *   host_qtile_off  int32 [B+1] (host) first query-tile index of each sequence
 *                   in canonical (sequence, row) order
 *   host_tiles      int32 [cap][4] (host) one record per query tile in
 *                   execution order: {b, row0, nk, nf | nrows << 16}, where
 *                   key tiles [0, nf) are FULL (no mask needed), [nf, nk)
 *                   PARTIAL, rows [row0, row0 + nrows) are local query rows
 *                   of sequence b (candidate indices for M-FALCON).
 *                   Execution order is longest first (nk descending, ties in
 *                   canonical order) when there are at most 8192 query
 *                   tiles, canonical otherwise.
 *   count           (host) number of query tiles (records beyond cap are not
 *                   copied)
 * Synchronises the stream. Intended for tests and tools.
 */
hstu_status_t hstu_schedule_export(const hstu_problem_t *p, int32_t op,
                                   const int32_t *hist_offsets, int64_t hist_tokens,
                                   int32_t hist_max_len, int32_t microbatch, void *ws,
                                   size_t ws_bytes, void *stream, int32_t *host_qtile_off,
                                   int32_t *host_tiles, int64_t cap, int64_t *count);

/*
 * Waits for `stream` and reads the device status word that the last call on
 * workspace `ws` left (0 = no violation, else HSTU_DEV_* bits) into
 * *host_code. Synchronises the stream.
 */
hstu_status_t hstu_get_device_status(const void *ws, void *stream, int32_t *host_code);

/*
 * Kernel timing for measurement tools. While enabled (process-wide), every
 * launch of a library kernel records a pair of HIP events on the stream it is
 * launched on. hstu_kernel_timing_read waits for the recorded events of one
 * kernel id, returns their summed duration in milliseconds and the number of
 * launches, and forgets them. Enabling or disabling also forgets all pending
 * records. Host only; not for concurrent use from several threads.
 */
enum {
  HSTU_KERNEL_SCHED = 0,     /* tile scheduler */
  HSTU_KERNEL_ATTN_FWD = 1,  /* attention forward (also M-FALCON scoring) */
  HSTU_KERNEL_NORM_FWD = 2,  /* Norm(O) * U */
  HSTU_KERNEL_NORM_BWD = 3,       /* backward of the norm epilogue */
  HSTU_KERNEL_ATTN_BWD_DQ = 4,    /* attention backward, query-major pass (dQ, d rab) */
  HSTU_KERNEL_AUX = 5,            /* fills */
  HSTU_KERNEL_ATTN_BWD_DKDV = 6,  /* attention backward, key-major pass (dK, dV) */
  HSTU_KERNEL_STOCHASTIC_LENGTH = 7,  /* hstu_stochastic_length (both of its kernels) */
  HSTU_KERNEL_GATHER = 8,         /* hstu_gather_rows */
  HSTU_KERNEL_BALANCE = 9,        /* hstu_balance_bins */
  HSTU_KERNEL_GEMM = 10,          /* the layer's projection GEMMs (hipBLASLt) */
  HSTU_KERNEL_LAYER_EW = 11,      /* the layer's SiLU / SiLU' / bias-gradient passes */
  HSTU_KERNEL_PROJ_SILU = 12,     /* f1 as one MFMA GEMM with the SiLU split epilogue (and W1's transpose) */
  HSTU_KERNEL_COUNT = 13          /* (launches recorded into a graph are not timed) */
};
hstu_status_t hstu_kernel_timing(int32_t enable);
hstu_status_t hstu_kernel_timing_read(int32_t kernel, double *total_ms, int64_t *launches);

/*
 * Small forwards (at most 256 sequences and 1024 work units of query tiles
 * x heads) normally skip the scheduler launch: every attention workgroup
 * validates the offsets, scans the query-tile counts and finds its own tile,
 * taking the tiles in canonical order instead of longest-first (all units
 * run at once at that size). Outputs and status bits are the same either
 * way. enable = 0 makes every forward launch the scheduler, 1 restores the
 * default. Process-wide, host only; returns the previous setting.
 */
int32_t hstu_set_inline_schedule(int32_t enable);

/*
 * Order of the scheduler's work lists (the forward's and the backward's
 * query tiles and the backward's key tiles; M-FALCON lists are always
 * longest first):
 *   HSTU_TILE_ORDER_LONGEST      longest record first (the default), which
 *                                balances the chip best;
 *   HSTU_TILE_ORDER_BY_SEQUENCE  whole sequences, longest first, each
 *                                sequence's records together and longest
 *                                first, so that its K/V (Q/dO for the key
 *                                pass) stays in one L2 while they run: far
 *                                fewer L2 refills, for a few percent more
 *                                time when the GPU has the memory system to
 *                                itself.
 * Outputs do not depend on the order (d rab and the affine gradients up to
 * the order of their atomic sums). Process-wide, host only; returns the
 * previous order, or -1 (HSTU_ERR_INVALID_ARG in hstu_last_error) for an
 * unknown one.
 */
enum { HSTU_TILE_ORDER_LONGEST = 0, HSTU_TILE_ORDER_BY_SEQUENCE = 1 };
int32_t hstu_set_tile_order(int32_t order);

/*
 * f1 of the bf16 training forward (hstu_layer_fwd with Z given; HSTU blog,
 * section 3, layer formula). By default it runs as one MFMA GEMM of the
 * library's own whose epilogue adds b1, writes Z and writes SiLU(Z) straight
 * into the U, V, Q, K blocks, after a small kernel that transposes W1 into
 * the layer workspace's GEMM area (d_model % 8 == 0, H * d % 8 == 0, and
 * 4 * H * d * d_model * 2 bytes within that 64 MiB area; other shapes, and
 * fp32, take the second form). enable = 0 selects the second form: a library
 * GEMM writing Z, then a separate SiLU split pass. Both forms round Z to bf16
 * and take the SiLU of the rounded value; they differ only in the GEMM's
 * summation order. The same setting selects the bf16 backward's form: by
 * default the norm backward and the two attention backward kernels write
 * dZ = [dU | dV | dQ | dK] * SiLU'(Z) straight into dZ's column blocks (dU
 * rounded once, dV, dQ, dK after their own bf16 rounding, as the separate
 * pass sees them) and the bias gradient is a column sum of dZ; with 0 they
 * write dU, dV, dQ, dK and a separate pass forms dZ and the column sums.
 * Process-wide, host only; returns the previous setting.
 */
int32_t hstu_set_fused_projection(int32_t enable);

/*
 * Stochastic Length (HSTU blog, section 3.4: training sequences are sampled
 * down to a length budget, 4096 -> about 776 at alpha = 1.6). Device side,
 * no host round trip. For every sequence b of the input batch (offsets [B+1],
 * device) of length L_b: if L_b <= cap all its tokens are kept, else the cap
 * tokens with the smallest (keys[t], t) are kept, in their original order (a
 * uniform random subset when keys are independent uniform random words; the
 * randomness is the caller's input, so the result is reproducible).
 *   keys         uint32 [total_tokens] device, one per input token
 *   new_offsets  int32 [B+1] device out: offsets of the kept batch
 *   gather_idx   int32 [total_tokens] device out: for r < new_offsets[B], the
 *                input index of the r-th kept token (gather rows with it)
 *   status       int32 [1] device out: 0, or HSTU_DEV_BAD_OFFSETS /
 *                HSTU_DEV_TOO_LONG (then nothing is kept: new_offsets all 0)
 * Requires cap >= 1 and max_len >= every L_b. Asynchronous on `stream`.
 */
hstu_status_t hstu_stochastic_length(const int32_t *offsets, int32_t B, int64_t total_tokens, int32_t max_len,
                                     int32_t cap, const uint32_t *keys, int32_t *new_offsets,
                                     int32_t *gather_idx, int32_t *status, void *stream);

/*
 * dst[r] = src[idx[r]] for n rows of row_bytes bytes (a multiple of 4; all
 * pointers device, rows dense). Gathers the tensors of a batch through the
 * indices hstu_stochastic_length returns. Asynchronous on `stream`.
 */
hstu_status_t hstu_gather_rows(const void *src, const int32_t *idx, int64_t n, int64_t row_bytes, void *dst,
                               void *stream);

/*
 * Work-balanced jagged batching (MTGR deep read, section 2: batch sizes are
 * adapted so that every GPU holds the same number of tokens). Sequences of a
 * batch (offsets [B+1], device) are assigned to n_bins bins (1..64), taken in
 * order of decreasing cost (ties by index), each to the bin with the smallest
 * cost so far (ties to the lowest bin). Cost: HSTU_COST_TOKENS = L, or
 * HSTU_COST_ATTENTION = L * L. Outputs (device): bin [B], bin_cost int64
 * [n_bins]. B <= 8192. Asynchronous on `stream`.
 */
enum { HSTU_COST_TOKENS = 0, HSTU_COST_ATTENTION = 1 };
hstu_status_t hstu_balance_bins(const int32_t *offsets, int32_t B, int32_t n_bins, int32_t cost_kind,
                                int32_t *bin, int64_t *bin_cost, void *stream);

/*
 * Full HSTU layer around the attention core (HSTU blog, section 3, the layer
 * formula: Q(X) = phi1(f1(X)), the pointwise attention, and
 * O(X) = f2(Norm(A V) * U)). With D = H*d and X [T, d_model]:
 *   Z          = X W1 + b1                    [T, 4D]   f1
 *   U|V|Q|K    = SiLU(Z)                      phi1 = SiLU; the four column
 *                                             blocks of width D, in this order
 *   Y, O       = hstu_attn_fwd(p, Q, K, V, U) [T, D]    the attention core
 *   Out        = Y W2 + b2                    [T, d_model]  f2
 * The pages name phi1 and the split only for Q; taking SiLU and one 4D-wide
 * projection for all four is the plainest reading. f1 and f2 run on hipBLASLt
 * (fp32 accumulation), the SiLU passes and everything else in this library's
 * kernels.
 *
 * Weights (device pointers, row-major, dense):
 *   d_model  width of X and Out, 1 <= d_model <= 65536
 *   W1       [d_model, 4D] in the problem's dtype;  b1 fp32 [4D] or NULL
 *   W2       [D, d_model] in the problem's dtype;   b2 fp32 [d_model] or NULL
 * X, Out, Z, Y, O, dOut and dX are in the problem's dtype and must be 16-byte
 * aligned, like W1 and W2.
 */
typedef struct hstu_layer_weights {
  int32_t d_model;
  const void *W1;
  const float *b1;
  const void *W2;
  const float *b2;
} hstu_layer_weights_t;

/*
 * Workspace bytes of hstu_layer_fwd (op = HSTU_OP_FWD) or hstu_layer_bwd
 * (op = HSTU_OP_BWD) for problem p and width d_model (host only). It holds
 * the attention core's workspace, the split activations (and their
 * gradients) and 64 MiB for the GEMMs.
 */
hstu_status_t hstu_layer_workspace_size(const hstu_problem_t *p, int32_t d_model, int32_t op, size_t *bytes);

/*
 * Layer forward. Writes Out [T, d_model] and, for the backward, Z [T, 4D],
 * Y and O [T, D] and mean, rstd fp32 [T] (NULL allowed when norm == NONE).
 * UVQK is optional: NULL keeps the activations U, V, Q, K in ws; else they
 * are written to UVQK [4, T, D] (U, then V, Q, K, each [T, D]) so that the
 * backward can reuse them instead of recomputing them from Z (4*T*D more
 * elements of memory for one pass less). Z may be NULL when no backward
 * follows (inference): f1 then runs as four GEMMs with the SiLU applied in
 * fp32 in their epilogue, as the serving stack does, so U, V, Q, K are
 * rounded once instead of twice and no pre-activation is written.
 * p describes the jagged batch, its masks, rab tables and norm exactly as for
 * hstu_attn_fwd. The first call on a device creates that device's hipBLASLt
 * handle, which loads hipBLASLt's kernels; apart from that handle nothing is
 * allocated (everything else lives in ws). The first call for a new GEMM
 * size class (token counts are rounded to four classes per octave) times
 * hipBLASLt's candidate algorithms on `stream` and waits for them; later
 * calls of the class do not synchronise. Under stream capture the untimed
 * first candidate is used.
 */
hstu_status_t hstu_layer_fwd(const hstu_problem_t *p, const hstu_layer_weights_t *w, const void *X, void *Out,
                             void *Z, void *UVQK, void *Y, void *O, float *mean, float *rstd, void *ws,
                             size_t ws_bytes, void *stream);

/*
 * Layer backward given dOut [T, d_model] and the forward's saved Z, UVQK
 * (or NULL: recomputed from Z), Y, O, mean, rstd for the same X and weights.
 * Writes (overwriting):
 *   dX        [T, d_model] in the problem's dtype
 *   dW1, dW2  fp32, shaped like W1 and W2 (16-byte aligned)
 *   db1, db2  fp32 [4D] and [d_model] (NULL skips each)
 *   d_rab_p, d_rab_t, d_gamma, d_beta  as in hstu_attn_bwd
 * Sums over tokens run in fp32 (the GEMMs in hipBLASLt's order, the weight
 * gradients split over token chunks whose partial sums are then added in a
 * fixed order). The GEMM algorithm choice is made as in hstu_layer_fwd.
 */
hstu_status_t hstu_layer_bwd(const hstu_problem_t *p, const hstu_layer_weights_t *w, const void *X,
                             const void *Z, const void *UVQK, const void *Y, const void *O, const float *mean,
                             const float *rstd, const void *dOut, void *dX, float *dW1, float *db1, float *dW2,
                             float *db2, float *d_rab_p, float *d_rab_t, float *d_gamma, float *d_beta, void *ws,
                             size_t ws_bytes, void *stream);

/*
 * Candidate scoring through a stack of HSTU layers with per-layer history
 * K/V caches (HSTU blog, section 4.2 "批量推理": candidates are scored in
 * microbatches against one encoding of the user's history; section 4.3
 * "KV Caching": the history's keys and values are computed once and reused).
 * The result equals running every user's sequence [history | candidates]
 * through all layers with the candidate mask (P = 0, C = m_b) and taking
 * the candidate rows: a history row never sees a candidate, so each layer's
 * history K and V are all a candidate needs.
 *
 * Each layer is described by hstu_stack_layer_t: its projections, its own
 * rab tables and norm affine (NULL = off / identity; the table sizes n_pos,
 * n_tb and the group count come from the problem), and its cache buffers
 * K_cache, V_cache [Th, H, d] (caller-owned, in the problem's dtype). All
 * layers share H, d, d_model, the norm kind and N_max, which the problem
 * passed to each call gives. Xc/X/Out are [tokens, d_model]. The serving
 * passes keep no pre-activation: f1 runs as four GEMMs (the U, V, Q, K
 * column blocks of W1) with the SiLU applied in fp32 in the GEMM epilogue,
 * so U, V, Q, K are rounded once (hstu_layer_fwd rounds Z, then SiLU(Z)).
 */
typedef struct hstu_stack_layer {
  hstu_layer_weights_t w;
  const float *rab_p;
  const float *rab_t;
  const float *gamma;
  const float *beta;
  void *K_cache;
  void *V_cache;
} hstu_stack_layer_t;

/*
 * Workspace bytes (host only) of hstu_stack_history (op = HSTU_OP_FWD; p =
 * the histories) or hstu_stack_score / hstu_stack_score_capture (op =
 * HSTU_OP_MFALCON; p = the candidates, with microbatch, hist_max_len and
 * hist_tokens as for hstu_workspace_size).
 */
hstu_status_t hstu_stack_workspace_size(const hstu_problem_t *p, int32_t d_model, int32_t op, int32_t microbatch,
                                        int32_t hist_max_len, int64_t hist_tokens, size_t *bytes);

/*
 * History pass: runs the histories (a jagged batch `hist`, any mask it
 * describes, normally causal) through the n_layers layers (1..64), writing
 * each layer's K and V into that layer's K_cache and V_cache, and the last
 * layer's output into Out [Th, d_model] (NULL skips it). The rab/gamma/beta
 * pointers of `hist` are ignored in favour of each layer's.
 */
hstu_status_t hstu_stack_history(const hstu_problem_t *hist, int32_t n_layers, const hstu_stack_layer_t *layers,
                                 const void *X, void *Out, void *ws, size_t ws_bytes, void *stream);

/*
 * Candidate pass: for each layer, the candidates' projections and
 * hstu_mfalcon_score against that layer's K_cache/V_cache (same microbatch
 * semantics; the result does not depend on microbatch), the output feeding
 * the next layer; Out [Tc, d_model] gets the last layer's output. `cand` is
 * the candidate problem as for hstu_mfalcon_score (its rab/gamma/beta
 * pointers are ignored in favour of each layer's). The caches may be reused
 * by any number of calls (new candidates of the same users) until the next
 * hstu_stack_history that writes them.
 */
hstu_status_t hstu_stack_score(const hstu_problem_t *cand, int32_t n_layers, const hstu_stack_layer_t *layers,
                               const int32_t *hist_offsets, int64_t hist_tokens, int32_t hist_max_len,
                               const int64_t *hist_ts, int32_t microbatch, const void *Xc, void *Out, void *ws,
                               size_t ws_bytes, void *stream);

/*
 * Records one hstu_stack_score call (same arguments) into an executable HIP
 * graph and returns it in *graph (host). Nothing runs until
 * hstu_graph_launch. A launch replays every kernel of the call with the
 * pointers and host scalars given here: between launches the caller may
 * change the contents of the device buffers (new candidate features, new
 * caches from a history pass of the same shapes), not their addresses or the
 * batch's sizes. Run one eager hstu_stack_score of the same sizes first so
 * that the GEMMs use timed algorithm choices (capture takes the heuristic's
 * first choice for sizes not seen before). Concurrent launches of one graph,
 * or of graphs sharing a workspace, race.
 */
hstu_status_t hstu_stack_score_capture(const hstu_problem_t *cand, int32_t n_layers,
                                       const hstu_stack_layer_t *layers, const int32_t *hist_offsets,
                                       int64_t hist_tokens, int32_t hist_max_len, const int64_t *hist_ts,
                                       int32_t microbatch, const void *Xc, void *Out, void *ws, size_t ws_bytes,
                                       void **graph);

/* Launches a graph from hstu_stack_score_capture on `stream`. */
hstu_status_t hstu_graph_launch(void *graph, void *stream);

/* Frees a graph from hstu_stack_score_capture (host; waits for nothing). */
hstu_status_t hstu_graph_destroy(void *graph);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H */
