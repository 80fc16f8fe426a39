// C-ABI of libhstu.so: host-side validation, workspace carving and the launch
// sequence of every entry point declared in include/hstu.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/hstu.h"
#include "hstu_internal.h"
#include "proj_gemm.h"

using namespace hstu;

namespace {

thread_local std::string g_err;

hstu_status_t fail(hstu_status_t st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
hstu_status_t fail(hstu_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

hstu_status_t hip_fail(hipError_t e, const char *what) {
  return fail(HSTU_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                      \
  do {                                           \
    hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// Whether small forwards build their tiles inside the attention kernel
// (hstu_set_inline_schedule).
std::atomic<int> g_inline_sched{1};
// Work-list order of the scheduler kernel (hstu_set_tile_order).
std::atomic<int> g_tile_order{kOrderLongest};
// Whether the bf16 training forward runs f1 as the fused SiLU-split GEMM
// (hstu_set_fused_projection).
std::atomic<int> g_fused_proj{1};

// Optional per-launch event timing (hstu_kernel_timing).
struct TimingRecord {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimingRecord> g_timing;

void timing_clear_locked() {
  for (auto &r : g_timing) {  // clean-up: a failure here leaves nothing to undo
    (void)hipEventSynchronize(r.stop);
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_timing.clear();
}

// Brackets one launch with events when timing is enabled.
struct Timed {
  int kernel;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  Timed(int k, hipStream_t s) : kernel(k), st(s) {
    std::lock_guard<std::mutex> g(g_timing_mu);
    if (!g_timing_on) return;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess ||
        hipEventRecord(a, st) != hipSuccess)
      drop();
  }
  ~Timed() {
    if (!a) return;
    if (hipEventRecord(b, st) != hipSuccess) {  // no record of this launch
      drop();
      return;
    }
    std::lock_guard<std::mutex> g(g_timing_mu);
    g_timing.push_back({kernel, a, b});
  }
  void drop() {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    a = b = nullptr;
  }
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
long long div_up(long long a, long long b) { return (a + b - 1) / b; }

struct Tiles {
  int BM, BN;
};

Tiles tiles_for(const hstu_problem_t *p, int op) {
  if (p->dtype == HSTU_F32) return {kF32BM, kF32BN};
  return {kFwdBM, kFwdBN};  // the backward's query-major pass uses the forward's tiles
}

// Workspace sections (byte offsets from ws).
struct Layout {
  size_t hdr, desc, qoff, tiles, total;
  long long max_tiles;
  // backward only: key-major schedule and the gradient of the pre-norm output
  size_t khdr, kdesc, kqoff, ktiles, dO;
  long long max_ktiles;
  // backward with a norm affine of at most kNormAffineLdsMax entries per
  // table: per-workgroup partials of d gamma / d beta (npart_blocks rows)
  size_t npart;
  long long npart_blocks;
  // fp32 backward: fp64 accumulators of d rab_p and d rab_t (n_pos + n_tb)
  size_t rab64;
  int norm_tpw;
};

// Tokens per wave of the norm backward when it sums d gamma / d beta per
// workgroup in LDS: at least 8, and few enough workgroups (at most 1024)
// that the partials stay small.
int norm_affine_tpw(long long T) { return (int)std::max<long long>(8, (T + 4095) / 4096); }

bool norm_affine_in_lds(const hstu_problem_t *p) {
  if (p->norm == HSTU_NORM_NONE || (!p->gamma && !p->beta)) return false;
  const long long G = p->norm == HSTU_NORM_GLN ? p->n_groups : 1;
  return G * p->H * p->d <= kNormAffineLdsMax;
}

Layout layout(const hstu_problem_t *p, int op, int microbatch, int hist_max_len) {
  Tiles t = tiles_for(p, op);
  Layout L{};
  long long nq;
  if (op == HSTU_OP_MFALCON) {
    long long bm = microbatch > 0 ? microbatch : (p->max_len > 0 ? p->max_len : 1);
    nq = div_up(p->total_tokens, t.BM) + (long long)p->B * (div_up(p->max_len, bm) + 1);
  } else {
    nq = div_up(p->total_tokens, t.BM) + p->B;
  }
  (void)hist_max_len;
  L.max_tiles = nq;
  size_t off = 0;
  L.hdr = off;   off += align256(kHdrWords * sizeof(int));
  L.desc = off;  off += align256(sizeof(SeqDesc) * (size_t)(p->B > 0 ? p->B : 1));
  L.qoff = off;  off += align256(sizeof(int) * (size_t)(p->B + 1));
  L.tiles = off; off += align256(sizeof(QTile) * (size_t)(nq > 0 ? nq : 1));
  if (op == HSTU_OP_BWD) {
    const long long nk = div_up(p->total_tokens, kBwdKBN) + p->B;
    L.max_ktiles = nk;
    L.khdr = off;   off += align256(kHdrWords * sizeof(int));
    L.kdesc = off;  off += align256(sizeof(SeqDesc) * (size_t)(p->B > 0 ? p->B : 1));
    L.kqoff = off;  off += align256(sizeof(int) * (size_t)(p->B + 1));
    L.ktiles = off; off += align256(sizeof(QTile) * (size_t)(nk > 0 ? nk : 1));
    const size_t esz = p->dtype == HSTU_BF16 ? 2 : 4;
    L.dO = off;     off += align256(esz * (size_t)p->total_tokens * p->H * p->d + 16);
    if (norm_affine_in_lds(p) && p->total_tokens > 0) {
      const long long G = p->norm == HSTU_NORM_GLN ? p->n_groups : 1;
      L.norm_tpw = norm_affine_tpw(p->total_tokens);
      L.npart_blocks = norm_bwd_blocks(p->total_tokens, L.norm_tpw);
      L.npart = off;  off += align256(sizeof(float) * 2 * (size_t)(G * p->H * p->d) * (size_t)L.npart_blocks);
    }
    if (p->dtype == HSTU_F32) {
      L.rab64 = off;  off += align256(sizeof(double) * (size_t)(std::max(p->n_pos, 0) + std::max(p->n_tb, 0) + 1));
    }
  }
  L.total = off;
  return L;
}

// The kernels move 16-byte vectors; every dense array must start on a 16-byte boundary.
bool aligned16(const void *q) { return ((uintptr_t)q & 15) == 0; }

hstu_status_t check_problem(const hstu_problem_t *p, int op) {
  if (!p) return fail(HSTU_ERR_INVALID_ARG, "problem is NULL");
  if (p->B < 0) return fail(HSTU_ERR_INVALID_ARG, "B = %d < 0", p->B);
  if (p->B > kMaxSeqs) return fail(HSTU_ERR_UNSUPPORTED, "B = %d > %d sequences per call", p->B, kMaxSeqs);
  if (p->H < 1) return fail(HSTU_ERR_INVALID_ARG, "H = %d < 1", p->H);
  if (p->d != 32 && p->d != 64 && p->d != 128)
    return fail(HSTU_ERR_UNSUPPORTED, "d = %d not in {32, 64, 128}", p->d);
  if (p->dtype != HSTU_BF16 && p->dtype != HSTU_F32)
    return fail(HSTU_ERR_INVALID_ARG, "dtype = %d", p->dtype);
  if (p->total_tokens < 0 || p->total_tokens >= (1ll << 31))
    return fail(HSTU_ERR_INVALID_ARG, "total_tokens = %lld out of [0, 2^31)", (long long)p->total_tokens);
  if (p->max_len < 0) return fail(HSTU_ERR_INVALID_ARG, "max_len = %d < 0", p->max_len);
  Tiles t = tiles_for(p, op);
  if (div_up(p->max_len, t.BN) > kMaxKeyTiles)
    return fail(HSTU_ERR_UNSUPPORTED, "max_len = %d exceeds %d key tiles", p->max_len, kMaxKeyTiles);
  if (p->n_max < 1) return fail(HSTU_ERR_INVALID_ARG, "n_max = %d < 1", p->n_max);
  if (!p->offsets) return fail(HSTU_ERR_INVALID_ARG, "offsets is NULL");
  if (p->rab_p && p->n_pos < 1) return fail(HSTU_ERR_INVALID_ARG, "rab_p given with n_pos = %d", p->n_pos);
  if (p->rab_t && p->n_tb < 1) return fail(HSTU_ERR_INVALID_ARG, "rab_t given with n_tb = %d", p->n_tb);
  if (p->norm < HSTU_NORM_NONE || p->norm > HSTU_NORM_GLN)
    return fail(HSTU_ERR_INVALID_ARG, "norm = %d", p->norm);
  if (p->norm != HSTU_NORM_NONE && !(p->eps > 0.f))
    return fail(HSTU_ERR_INVALID_ARG, "eps = %g must be > 0", (double)p->eps);
  if (p->norm == HSTU_NORM_GLN) {
    if (!p->token_group) return fail(HSTU_ERR_INVALID_ARG, "GLN needs token_group");
    if (p->n_groups < 1 || p->n_groups > 255)
      return fail(HSTU_ERR_INVALID_ARG, "n_groups = %d not in [1, 255]", p->n_groups);
  }
  if (p->mask_flags & ~HSTU_MASK_CAND_TIME_FILTER)
    return fail(HSTU_ERR_INVALID_ARG, "mask_flags = %d has unknown bits", p->mask_flags);
  if ((p->mask_flags & HSTU_MASK_CAND_TIME_FILTER) && !p->timestamps)
    return fail(HSTU_ERR_INVALID_ARG, "the candidate timestamp filter needs timestamps");
  if (!aligned16(p->gamma) || !aligned16(p->beta))
    return fail(HSTU_ERR_INVALID_ARG, "gamma/beta must be 16-byte aligned");
  const long long D = (long long)p->H * p->d;
  const long long dmax = p->dtype == HSTU_BF16 ? 4096 : 2048;
  if (D > dmax) return fail(HSTU_ERR_UNSUPPORTED, "H*d = %lld > %lld", D, dmax);
  return HSTU_OK;
}

hstu_status_t check_ws(const void *ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(HSTU_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)ws % 256) return fail(HSTU_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (ws_bytes < need) return fail(HSTU_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  return HSTU_OK;
}

template <class T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

void fill_sched(SchedArgs &s, const hstu_problem_t *p, int op, const Layout &L, void *ws,
                const int32_t *hist_offsets, int64_t hist_tokens, int hist_max_len, int microbatch) {
  Tiles t = tiles_for(p, op);
  std::memset(&s, 0, sizeof s);
  s.mode = op == HSTU_OP_MFALCON ? kSchedMFalcon : kSchedAttn;
  if (op == HSTU_OP_MFALCON) {
    s.cand_offsets = p->offsets;
    s.hist_offsets = hist_offsets;
  } else {
    s.offsets = p->offsets;
    s.prefix = p->prefix_len;
    s.cand = p->cand_len;
  }
  s.B = p->B;
  s.Tq = p->total_tokens;
  s.Tkv = op == HSTU_OP_MFALCON ? hist_tokens : p->total_tokens;
  s.max_len = p->max_len;
  s.hist_max_len = hist_max_len;
  s.BM = t.BM;
  s.BN = t.BN;
  s.microbatch = microbatch;
  s.time_filter = (p->mask_flags & HSTU_MASK_CAND_TIME_FILTER) ? 1 : 0;
  s.order = g_tile_order.load(std::memory_order_relaxed);
  s.max_tiles = (int)L.max_tiles;
  s.hdr = at<int>(ws, L.hdr);
  s.desc = at<SeqDesc>(ws, L.desc);
  s.qoff = at<int>(ws, L.qoff);
  s.tiles = at<QTile>(ws, L.tiles);
}

hstu_status_t check_mfalcon(const hstu_problem_t *cand, const int32_t *hist_offsets,
                            int64_t hist_tokens, int32_t hist_max_len, int32_t microbatch) {
  if (!cand) return fail(HSTU_ERR_INVALID_ARG, "problem is NULL");
  if (cand->prefix_len || cand->cand_len)
    return fail(HSTU_ERR_INVALID_ARG, "M-FALCON candidates take no prefix_len/cand_len");
  if (!hist_offsets) return fail(HSTU_ERR_INVALID_ARG, "hist_offsets is NULL");
  if (hist_tokens < 0 || hist_tokens >= (1ll << 31))
    return fail(HSTU_ERR_INVALID_ARG, "hist_tokens = %lld", (long long)hist_tokens);
  if (hist_max_len < 0) return fail(HSTU_ERR_INVALID_ARG, "hist_max_len < 0");
  if (microbatch < 0) return fail(HSTU_ERR_INVALID_ARG, "microbatch = %d < 0", microbatch);
  Tiles t = tiles_for(cand, HSTU_OP_MFALCON);
  if (div_up(hist_max_len, t.BN) > kMaxKeyTiles)
    return fail(HSTU_ERR_UNSUPPORTED, "hist_max_len = %d exceeds %d key tiles", hist_max_len, kMaxKeyTiles);
  if ((long long)hist_max_len + cand->max_len >= (1ll << 30))
    return fail(HSTU_ERR_INVALID_ARG, "history + candidates too long");
  return HSTU_OK;
}


// Per-call value that marks an inline-schedule forward's timestamp flag in
// the workspace header; seeded from the clock so that a fresh workspace's
// stale contents match it only by a 2^-32 chance.
unsigned next_epoch() {
  static std::atomic<unsigned> e{(unsigned)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761u};
  return e.fetch_add(1u);
}

// inl: when not NULL, the attention workgroups build their own tiles from it
// (no scheduler launch before this call).
hstu_status_t run_forward(const hstu_problem_t *p, int op, const Layout &L, void *ws,
                          hipStream_t st, const void *Q, const void *K, const void *V,
                          const void *Kself, const void *Vself, const void *U,
                          const int64_t *ts_q, const int64_t *ts_kv, void *Y, void *O,
                          float *mean, float *rstd, const SchedArgs *inl = nullptr) {
  Tiles t = tiles_for(p, op);
  FwdArgs f;
  std::memset(&f, 0, sizeof f);
  f.Q = Q; f.K = K; f.V = V; f.Kself = Kself; f.Vself = Vself; f.O = O;
  // Timestamps reach the kernel when rab_t or the candidate filter uses them.
  const bool tf = (p->mask_flags & HSTU_MASK_CAND_TIME_FILTER) != 0;
  const bool use_t = (p->rab_t || tf) && ts_q && ts_kv;
  f.ts_q = use_t ? ts_q : nullptr;
  f.ts_kv = use_t ? ts_kv : nullptr;
  f.rab_p = p->rab_p;
  f.rab_t = (use_t && p->rab_t) ? p->rab_t : nullptr;
  f.tfilt = (tf && use_t) ? 1 : 0;
  f.n_pos = p->n_pos;
  f.n_tb = p->n_tb;
  f.inv_nmax = 1.0f / (float)p->n_max;
  f.H = p->H;
  f.d = p->d;
  f.hdr = at<int>(ws, L.hdr);
  f.desc = at<SeqDesc>(ws, L.desc);
  f.tiles = at<QTile>(ws, L.tiles);
  long long units = L.max_tiles * p->H;
  if (units >= (1ll << 31)) return fail(HSTU_ERR_UNSUPPORTED, "too many work units");
  f.units = (int)units;
  (void)t;
  const unsigned epoch = next_epoch();
  if (inl) {
    f.inline_sched = 1;
    f.epoch = epoch;
    f.sched = *inl;
  }
  {
    Timed t_(HSTU_KERNEL_ATTN_FWD, st);
    HIP_TRY(p->dtype == HSTU_BF16 ? launch_attn_fwd_bf16(f, st) : launch_attn_fwd_f32(f, st),
            "attention forward launch");
  }

  NormArgs n;
  std::memset(&n, 0, sizeof n);
  n.X = O; n.U = U; n.Y = Y;
  n.mean = (mean && rstd) ? mean : nullptr;
  n.rstd = (mean && rstd) ? rstd : nullptr;
  n.group = p->norm == HSTU_NORM_GLN ? p->token_group : nullptr;
  n.gamma = p->gamma; n.beta = p->beta;
  n.n_groups = p->norm == HSTU_NORM_GLN ? p->n_groups : 1;
  n.mode = p->norm;
  n.eps = p->eps;
  n.T = p->total_tokens;
  n.D = p->H * p->d;
  n.hdr = at<int>(ws, L.hdr);
  n.merge_ts = inl && f.ts_q ? 1 : 0;
  n.epoch = epoch;
  {
    Timed t_(HSTU_KERNEL_NORM_FWD, st);
    HIP_TRY(launch_norm_fwd(n, p->dtype == HSTU_BF16, st), "norm forward launch");
  }
  return HSTU_OK;
}


// ---------------------------------------------------------------- full layer

constexpr size_t kGemmWsBytes = size_t(64) << 20;

// Layer workspace: the core's workspace first (so its status header is the
// layer's), then the split activations U|V|Q|K (reused for dZ in the
// backward), and for the backward dY and the core's gradients dU|dV|dQ|dK;
// last the GEMM workspace.
struct LayerLayout {
  size_t core_bytes, act, dy, grads, sums, wpart, gemm, total;
};

// Weight gradients W[M, N] = A^T B over T rows: split T into S equal chunks
// (a strided batch of S GEMMs into fp32 slices, then the slices summed) so
// that the few output tiles still fill the chip.
constexpr int kMaxSplits = 16;
int splits_for(long long M, long long N, long long T) {
  const long long tiles = ((M + 255) / 256) * ((N + 255) / 256);
  int S = 1;
  while (S < kMaxSplits && tiles * S * 2 <= 512 && T / (S * 2) >= 512) S *= 2;
  return S;
}

LayerLayout layer_layout(const hstu_problem_t *p, int op, int d_model) {
  LayerLayout y{};
  y.core_bytes = layout(p, op, 0, 0).total;
  const size_t esz = p->dtype == HSTU_BF16 ? 2 : 4;
  const size_t td = (size_t)p->total_tokens * p->H * p->d * esz;
  size_t off = align256(y.core_bytes);
  y.act = off;   off += align256(4 * td);
  if (op == HSTU_OP_BWD) {
    y.dy = off;    off += align256(td);
    y.grads = off; off += align256(4 * td);
    const size_t cols = std::max<size_t>((size_t)4 * p->H * p->d, (size_t)d_model);
    y.sums = off;  off += align256(sizeof(float) * kColsumGroups * cols);
    const size_t wmax = std::max<size_t>((size_t)4 * p->H * p->d * d_model, (size_t)p->H * p->d * d_model);
    y.wpart = off; off += align256(sizeof(float) * (kMaxSplits + 1) * wmax);
  }
  y.gemm = off;  off += kGemmWsBytes;
  y.total = off;
  return y;
}


hstu_status_t check_layer(const hstu_problem_t *p, const hstu_layer_weights_t *w) {
  if (!w) return fail(HSTU_ERR_INVALID_ARG, "layer weights are NULL");
  if (w->d_model < 1 || w->d_model > 65536)
    return fail(HSTU_ERR_INVALID_ARG, "d_model = %d not in [1, 65536]", w->d_model);
  if (!w->W1 || !w->W2) return fail(HSTU_ERR_INVALID_ARG, "W1/W2 must not be NULL");
  if (!aligned16(w->W1) || !aligned16(w->W2)) return fail(HSTU_ERR_INVALID_ARG, "W1/W2 must be 16-byte aligned");
  (void)p;
  return HSTU_OK;
}

hstu_status_t gemm_fail(int st, const char *what) {
  return fail(gemm_unsupported(st) ? HSTU_ERR_UNSUPPORTED : HSTU_ERR_HIP, "%s: %s (status %d)", what,
              gemm_status_text(st), st);
}

#define GEMM_RUN(g, what)                                            \
  do {                                                               \
    Timed t_(HSTU_KERNEL_GEMM, st);                                  \
    const int gs_ = gemm_rm((g), gws, kGemmWsBytes, st);           \
    if (gs_ != 0) return gemm_fail(gs_, what);                       \
  } while (0)

GemmRM gemm(bool ta, bool tb, long long M, long long N, long long K, const void *A, long long lda, const void *B,
            long long ldb, void *C, long long ldc, GemmType ab, GemmType c, const float *bias) {
  GemmRM g;
  std::memset(&g, 0, sizeof g);
  g.ta = ta; g.tb = tb; g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.ab = ab; g.c = c; g.bias = bias; g.accumulate = false;
  return g;
}

// U | V | Q | K = SiLU(X W1 + b1) split into four dense [T, D] arrays, as
// four GEMMs over the column blocks of W1 with the SiLU in their epilogue
// (no pre-activation Z is kept: the serving paths have no backward).
hstu_status_t silu_projection(const void *X, long long T, long long dm, const hstu_layer_weights_t &w, long long D,
                              GemmType et, void *U, void *V, void *Q, void *K, void *gws, hipStream_t st) {
  if (T <= 0) return HSTU_OK;
  const size_t esz = et == kGemmBF16 ? 2 : 4;
  void *out[4] = {U, V, Q, K};
  static const char *what[4] = {"f1 GEMM (U)", "f1 GEMM (V)", "f1 GEMM (Q)", "f1 GEMM (K)"};
  for (int j = 0; j < 4; ++j) {
    GemmRM g = gemm(false, false, T, D, dm, X, dm, static_cast<const char *>(w.W1) + j * D * esz, 4 * D, out[j], D,
                    et, et, w.b1 ? w.b1 + j * D : nullptr);
    g.silu = true;
    GEMM_RUN(g, what[j]);
  }
  return HSTU_OK;
}

// W (fp32 [M, N]) = A^T B for A [T, M], B [T, N] (row-major, dense, element
// type et), split over T as splits_for() says; `part` holds the slices.
hstu_status_t weight_grad(const void *A, long long M, const void *B, long long N, long long T, GemmType et, float *W,
                          float *part, void *gws, hipStream_t st, const char *what) {
  const size_t esz = et == kGemmBF16 ? 2 : 4;
  const int S = splits_for(M, N, T);
  if (S == 1) {
    GEMM_RUN(gemm(true, false, M, N, T, A, M, B, N, W, N, et, kGemmF32, nullptr), what);
    return HSTU_OK;
  }
  const long long Tc = T / S, rem = T - Tc * S;
  GemmRM g = gemm(true, false, M, N, Tc, A, M, B, N, part, N, et, kGemmF32, nullptr);
  g.batch = S;
  g.sA = Tc * M;
  g.sB = Tc * N;
  g.sC = M * N;
  GEMM_RUN(g, what);
  if (rem > 0) {
    const char *a = static_cast<const char *>(A) + (size_t)(Tc * S) * M * esz;
    const char *b = static_cast<const char *>(B) + (size_t)(Tc * S) * N * esz;
    GEMM_RUN(gemm(true, false, M, N, rem, a, M, b, N, part + (size_t)S * M * N, N, et, kGemmF32, nullptr), what);
  }
  Timed t_(HSTU_KERNEL_LAYER_EW, st);
  HIP_TRY(launch_sum_slices(part, S + (rem > 0 ? 1 : 0), M * N, W, st), "slice-sum launch");
  return HSTU_OK;
}

}  // namespace

namespace hstu {
hstu_status_t set_last_error(hstu_status_t st, const char *msg) { return fail(st, "%s", msg); }
}  // namespace hstu

extern "C" {

const char *hstu_version(void) { return "0.1.0"; }

int32_t hstu_set_inline_schedule(int32_t enable) { return g_inline_sched.exchange(enable ? 1 : 0); }

int32_t hstu_set_fused_projection(int32_t enable) { return g_fused_proj.exchange(enable ? 1 : 0); }

int32_t hstu_set_tile_order(int32_t order) {
  if (order != HSTU_TILE_ORDER_LONGEST && order != HSTU_TILE_ORDER_BY_SEQUENCE) {
    fail(HSTU_ERR_INVALID_ARG, "tile order %d", order);
    return -1;
  }
  return g_tile_order.exchange(order == HSTU_TILE_ORDER_BY_SEQUENCE ? kOrderBySequence : kOrderLongest) ==
                 kOrderBySequence
             ? HSTU_TILE_ORDER_BY_SEQUENCE
             : HSTU_TILE_ORDER_LONGEST;
}

const char *hstu_last_error(void) { return g_err.c_str(); }

hstu_status_t hstu_workspace_size(const hstu_problem_t *p, int32_t op, int32_t microbatch,
                                  int32_t hist_max_len, int64_t hist_tokens, size_t *bytes) {
  if (!bytes) return fail(HSTU_ERR_INVALID_ARG, "bytes is NULL");
  if (op != HSTU_OP_FWD && op != HSTU_OP_BWD && op != HSTU_OP_MFALCON)
    return fail(HSTU_ERR_INVALID_ARG, "op = %d", op);
  hstu_status_t st = check_problem(p, op);
  if (st) return st;
  if (op == HSTU_OP_MFALCON) {
    if (microbatch < 0) return fail(HSTU_ERR_INVALID_ARG, "microbatch = %d < 0", microbatch);
    (void)hist_tokens;
  }
  *bytes = layout(p, op, microbatch, hist_max_len).total;
  return HSTU_OK;
}

hstu_status_t hstu_tile_shape(const hstu_problem_t *p, int32_t op, int32_t *BM, int32_t *BN) {
  if (!p || !BM || !BN) return fail(HSTU_ERR_INVALID_ARG, "NULL argument");
  Tiles t = tiles_for(p, op);
  *BM = t.BM;
  *BN = t.BN;
  return HSTU_OK;
}

hstu_status_t hstu_attn_fwd(const hstu_problem_t *p, const void *Q, const void *K, const void *V,
                            const void *U, void *Y, void *O, float *mean, float *rstd, void *ws,
                            size_t ws_bytes, void *stream) {
  hstu_status_t s = check_problem(p, HSTU_OP_FWD);
  if (s) return s;
  if (p->total_tokens > 0 && (!Q || !K || !V || !U || !Y || !O))
    return fail(HSTU_ERR_INVALID_ARG, "Q/K/V/U/Y/O must not be NULL");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(U) || !aligned16(Y) || !aligned16(O))
    return fail(HSTU_ERR_INVALID_ARG, "Q/K/V/U/Y/O must be 16-byte aligned");
  if (p->norm != HSTU_NORM_NONE && p->total_tokens > 0 && (!mean || !rstd))
    return fail(HSTU_ERR_INVALID_ARG, "mean/rstd must not be NULL with a norm");
  Layout L = layout(p, HSTU_OP_FWD, 0, 0);
  s = check_ws(ws, ws_bytes, L.total);
  if (s) return s;
  hipStream_t st = (hipStream_t)stream;
  SchedArgs sa;
  fill_sched(sa, p, HSTU_OP_FWD, L, ws, nullptr, 0, 0, 0);
  // Small batches skip the scheduler launch: each attention workgroup finds
  // its own tile (one dependent launch less on a latency-bound step).
  const bool inl = g_inline_sched.load(std::memory_order_relaxed) != 0 && p->total_tokens > 0 &&
                   p->B > 0 && p->B <= kInlineSchedMaxSeqs && L.max_tiles * p->H <= kInlineSchedMaxUnits;
  if (!inl) {
    Timed t_(HSTU_KERNEL_SCHED, st);
    HIP_TRY(launch_sched(sa, st), "scheduler launch");
  }
  return run_forward(p, HSTU_OP_FWD, L, ws, st, Q, K, V, K, V, U, p->timestamps, p->timestamps,
                     Y, O, mean, rstd, inl ? &sa : nullptr);
}

hstu_status_t hstu_mfalcon_score(const hstu_problem_t *cand, const int32_t *hist_offsets,
                                 int64_t hist_tokens, int32_t hist_max_len, const void *K_cache,
                                 const void *V_cache, const int64_t *hist_ts, const void *Qc,
                                 const void *Kc, const void *Vc, const void *Uc,
                                 int32_t microbatch, void *Yc, void *Oc, float *mean, float *rstd,
                                 void *ws, size_t ws_bytes, void *stream) {
  hstu_status_t s = check_problem(cand, HSTU_OP_MFALCON);
  if (s) return s;
  s = check_mfalcon(cand, hist_offsets, hist_tokens, hist_max_len, microbatch);
  if (s) return s;
  if ((cand->timestamps == nullptr) != (hist_ts == nullptr))
    return fail(HSTU_ERR_INVALID_ARG, "give both candidate and history timestamps, or neither");
  if (cand->total_tokens > 0 && (!Qc || !Kc || !Vc || !Uc || !Yc || !Oc))
    return fail(HSTU_ERR_INVALID_ARG, "Qc/Kc/Vc/Uc/Yc/Oc must not be NULL");
  if (!aligned16(Qc) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(Uc) || !aligned16(Yc) || !aligned16(Oc) ||
      !aligned16(K_cache) || !aligned16(V_cache))
    return fail(HSTU_ERR_INVALID_ARG, "Qc/Kc/Vc/Uc/Yc/Oc/K_cache/V_cache must be 16-byte aligned");
  if (hist_tokens > 0 && (!K_cache || !V_cache))
    return fail(HSTU_ERR_INVALID_ARG, "K_cache/V_cache must not be NULL");
  if (cand->norm != HSTU_NORM_NONE && cand->total_tokens > 0 && (!mean || !rstd))
    return fail(HSTU_ERR_INVALID_ARG, "mean/rstd must not be NULL with a norm");
  Layout L = layout(cand, HSTU_OP_MFALCON, microbatch, hist_max_len);
  s = check_ws(ws, ws_bytes, L.total);
  if (s) return s;
  hipStream_t st = (hipStream_t)stream;
  SchedArgs sa;
  fill_sched(sa, cand, HSTU_OP_MFALCON, L, ws, hist_offsets, hist_tokens, hist_max_len, microbatch);
  {
    Timed t_(HSTU_KERNEL_SCHED, st);
    HIP_TRY(launch_sched(sa, st), "scheduler launch");
  }
  return run_forward(cand, HSTU_OP_MFALCON, L, ws, st, Qc, K_cache, V_cache, Kc, Vc, Uc,
                     cand->timestamps, hist_ts, Yc, Oc, mean, rstd);
}

}  // extern "C"

namespace {
// A layer's backward writes dU, dV, dQ, dK straight into the column blocks
// of its dZ [T, 4D] (row stride 4D), each times SiLU' of the same block of the
// pre-activation Z (bf16 only). dU..dK then point into dZ; z is Z itself.
struct DsiluOut {
  const void *z;
  long long ld;
};

hstu_status_t attn_bwd_impl(const hstu_problem_t *p, const void *Q, const void *K, const void *V,
                            const void *U, const void *O, const float *mean, const float *rstd,
                            const void *dY, void *dQ, void *dK, void *dV, void *dU,
                            float *d_rab_p, float *d_rab_t, float *d_gamma, float *d_beta,
                            void *ws, size_t ws_bytes, void *stream, const DsiluOut *zo) {
  hstu_status_t s = check_problem(p, HSTU_OP_BWD);
  if (s) return s;
  const long long T = p->total_tokens;
  if (T > 0 && (!Q || !K || !V || !U || !O || !dY || !dQ || !dK || !dV || !dU))
    return fail(HSTU_ERR_INVALID_ARG, "Q/K/V/U/O/dY/dQ/dK/dV/dU must not be NULL");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(U) || !aligned16(O) || !aligned16(dY) ||
      !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) || !aligned16(dU))
    return fail(HSTU_ERR_INVALID_ARG, "Q/K/V/U/O/dY/dQ/dK/dV/dU must be 16-byte aligned");
  if (p->norm != HSTU_NORM_NONE && T > 0 && (!mean || !rstd))
    return fail(HSTU_ERR_INVALID_ARG, "mean/rstd must not be NULL with a norm");
  const bool tf = (p->mask_flags & HSTU_MASK_CAND_TIME_FILTER) != 0;
  const bool use_rt = p->rab_t && p->timestamps;            // the rab_t term is on
  const bool use_t = (p->rab_t || tf) && p->timestamps;     // kernels need timestamps
  if (p->rab_p && !d_rab_p) return fail(HSTU_ERR_INVALID_ARG, "d_rab_p must not be NULL when rab_p is given");
  if (use_rt && !d_rab_t) return fail(HSTU_ERR_INVALID_ARG, "d_rab_t must not be NULL when rab_t is used");
  Layout L = layout(p, HSTU_OP_BWD, 0, 0);
  s = check_ws(ws, ws_bytes, L.total);
  if (s) return s;
  hipStream_t st = (hipStream_t)stream;
  const int D = p->H * p->d;
  const bool bf16 = p->dtype == HSTU_BF16;

  // Query-major and key-major schedules.
  SchedArgs qa;
  fill_sched(qa, p, HSTU_OP_BWD, L, ws, nullptr, 0, 0, 0);
  SchedArgs ka = qa;
  ka.mode = kSchedKeys;
  ka.BM = kBwdKBM;
  ka.BN = kBwdKBN;
  ka.max_tiles = (int)L.max_ktiles;
  ka.hdr = at<int>(ws, L.khdr);
  ka.desc = at<SeqDesc>(ws, L.kdesc);
  ka.qoff = at<int>(ws, L.kqoff);
  ka.tiles = at<QTile>(ws, L.ktiles);
  {
    Timed t_(HSTU_KERNEL_SCHED, st);
    HIP_TRY(launch_sched_pair(qa, ka, st), "scheduler launch");
  }
  const int G = p->norm == HSTU_NORM_GLN ? p->n_groups : 1;
  float *dg = (p->gamma && p->norm != HSTU_NORM_NONE) ? d_gamma : nullptr;
  float *db = (p->beta && p->norm != HSTU_NORM_NONE) ? d_beta : nullptr;
  // d gamma / d beta: per-workgroup LDS partials and a reduction when the
  // tables are small (and there are tokens), else global atomics.
  const bool aff_lds = (dg || db) && L.npart_blocks > 0;
  // fp32: d rab is summed in fp64 in the workspace and rounded once at the end
  double *rab64 = bf16 ? nullptr : at<double>(ws, L.rab64);
  {
    Timed t_(HSTU_KERNEL_AUX, st);
    if (p->rab_p) HIP_TRY(launch_fill_f32(d_rab_p, p->n_pos, 0.f, st), "fill");
    if (p->rab_t && d_rab_t) HIP_TRY(launch_fill_f32(d_rab_t, p->n_tb, 0.f, st), "fill");
    if (rab64 && (p->rab_p || (p->rab_t && d_rab_t)))
      HIP_TRY(launch_fill_f32((float *)rab64, 2ll * (p->n_pos + p->n_tb), 0.f, st), "fill");
    if (dg && !aff_lds) HIP_TRY(launch_fill_f32(dg, (long long)G * D, 0.f, st), "fill");
    if (db && !aff_lds) HIP_TRY(launch_fill_f32(db, (long long)G * D, 0.f, st), "fill");
  }
  void *dO = at<char>(ws, L.dO);
  {
    NormBwdArgs n;
    std::memset(&n, 0, sizeof n);
    n.X = O; n.U = U; n.dY = dY; n.mean = mean; n.rstd = rstd;
    n.group = p->norm == HSTU_NORM_GLN ? p->token_group : nullptr;
    n.gamma = p->gamma; n.beta = p->beta;
    n.n_groups = G;
    n.mode = p->norm;
    n.T = T;
    n.D = D;
    // One token per wave when no affine gradient is summed (as many waves as
    // tokens keep the loads in flight); with small affine tables, short runs
    // summed per workgroup in LDS; otherwise runs of 32 tokens, whose
    // dgamma / dbeta partials leave with one global atomic per column and run.
    n.tokens_per_wave = aff_lds ? L.norm_tpw : (dg || db) ? 32 : 1;
    n.dU = dU; n.dX = dO;
    n.ldu = zo ? zo->ld : D;
    n.zu = zo ? zo->z : nullptr;
    n.dgamma = dg; n.dbeta = db;
    n.partial = aff_lds ? at<float>(ws, L.npart) : nullptr;
    Timed t_(HSTU_KERNEL_NORM_BWD, st);
    HIP_TRY(launch_norm_bwd(n, bf16, st), "norm backward launch");
    if (aff_lds)
      HIP_TRY(launch_norm_affine_reduce(n.partial, L.npart_blocks, G * D, dg, db, st), "norm affine reduce launch");
  }
  BwdArgs b;
  std::memset(&b, 0, sizeof b);
  b.Q = Q; b.K = K; b.V = V; b.dO = dO;
  b.dQ = dQ; b.dK = dK; b.dV = dV;
  b.ts = use_t ? p->timestamps : nullptr;
  b.rab_p = p->rab_p;
  b.rab_t = use_rt ? p->rab_t : nullptr;
  b.tfilt = (tf && use_t) ? 1 : 0;
  b.no_cand = p->cand_len == nullptr ? 1 : 0;
  b.drab_p = d_rab_p;
  b.drab_t = d_rab_t;
  b.drab_p64 = rab64;
  b.drab_t64 = rab64 ? rab64 + p->n_pos : nullptr;
  b.n_pos = p->n_pos;
  b.n_tb = p->n_tb;
  b.inv_nmax = 1.0f / (float)p->n_max;
  b.H = p->H;
  b.d = p->d;
  b.hdr = qa.hdr;
  b.status = qa.hdr + kHdrStatus;
  b.desc = qa.desc;
  b.tiles = qa.tiles;
  b.ldo = zo ? zo->ld : D;
  if (zo) {
    const size_t blk = (size_t)D * 2;  // bytes between column blocks of a bf16 row
    b.zv = static_cast<const char *>(zo->z) + blk;
    b.zq = static_cast<const char *>(zo->z) + 2 * blk;
    b.zk = static_cast<const char *>(zo->z) + 3 * blk;
  }
  long long units = L.max_tiles * p->H;
  if (units >= (1ll << 31) || L.max_ktiles * p->H >= (1ll << 31))
    return fail(HSTU_ERR_UNSUPPORTED, "too many work units");
  b.units = (int)units;
  {
    Timed t_(HSTU_KERNEL_ATTN_BWD_DQ, st);
    HIP_TRY(bf16 ? launch_attn_bwd_dq_bf16(b, st) : launch_attn_bwd_dq_f32(b, st), "dq launch");
  }
  if (rab64 && (p->rab_p || b.rab_t)) {
    Timed t_(HSTU_KERNEL_AUX, st);
    HIP_TRY(launch_rab64_finalize(p->rab_p ? rab64 : nullptr, p->n_pos, b.rab_t ? rab64 + p->n_pos : nullptr, p->n_tb,
                                  b.inv_nmax, d_rab_p, d_rab_t, st),
            "d rab finalize launch");
  }
  b.hdr = ka.hdr;
  b.desc = ka.desc;
  b.tiles = ka.tiles;
  b.units = (int)(L.max_ktiles * p->H);
  {
    Timed t_(HSTU_KERNEL_ATTN_BWD_DKDV, st);
    HIP_TRY(bf16 ? launch_attn_bwd_dkdv_bf16(b, st) : launch_attn_bwd_dkdv_f32(b, st), "dkdv launch");
  }
  return HSTU_OK;
}
}  // namespace

extern "C" {

hstu_status_t hstu_attn_bwd(const hstu_problem_t *p, const void *Q, const void *K, const void *V,
                            const void *U, const void *O, const float *mean, const float *rstd,
                            const void *dY, void *dQ, void *dK, void *dV, void *dU,
                            float *d_rab_p, float *d_rab_t, float *d_gamma, float *d_beta,
                            void *ws, size_t ws_bytes, void *stream) {
  return attn_bwd_impl(p, Q, K, V, U, O, mean, rstd, dY, dQ, dK, dV, dU, d_rab_p, d_rab_t, d_gamma, d_beta, ws,
                       ws_bytes, stream, nullptr);
}

hstu_status_t hstu_schedule_export(const hstu_problem_t *p, int32_t op,
                                   const int32_t *hist_offsets, int64_t hist_tokens,
                                   int32_t hist_max_len, int32_t microbatch, void *ws,
                                   size_t ws_bytes, void *stream, int32_t *host_qtile_off,
                                   int32_t *host_tiles, int64_t cap, int64_t *count) {
  if (op != HSTU_OP_FWD && op != HSTU_OP_MFALCON)
    return fail(HSTU_ERR_INVALID_ARG, "schedule export supports HSTU_OP_FWD and HSTU_OP_MFALCON");
  hstu_status_t s = check_problem(p, op);
  if (s) return s;
  if (op == HSTU_OP_MFALCON) {
    s = check_mfalcon(p, hist_offsets, hist_tokens, hist_max_len, microbatch);
    if (s) return s;
  }
  if (!host_qtile_off || !count || (cap > 0 && !host_tiles))
    return fail(HSTU_ERR_INVALID_ARG, "NULL host output");
  Layout L = layout(p, op, microbatch, hist_max_len);
  s = check_ws(ws, ws_bytes, L.total);
  if (s) return s;
  hipStream_t st = (hipStream_t)stream;
  SchedArgs sa;
  fill_sched(sa, p, op, L, ws, hist_offsets, hist_tokens, hist_max_len, microbatch);
  HIP_TRY(launch_sched(sa, st), "scheduler launch");
  int hdr[kHdrWords];
  HIP_TRY(hipMemcpyAsync(hdr, at<int>(ws, L.hdr), sizeof hdr, hipMemcpyDeviceToHost, st), "copy header");
  HIP_TRY(hipMemcpyAsync(host_qtile_off, at<int>(ws, L.qoff), sizeof(int) * (p->B + 1),
                         hipMemcpyDeviceToHost, st), "copy query-tile offsets");
  HIP_TRY(hipStreamSynchronize(st), "stream synchronize");
  const long long nq = hdr[kHdrNQ];
  *count = nq;
  const long long n = nq < cap ? nq : cap;
  if (n > 0) {
    HIP_TRY(hipMemcpy(host_tiles, at<QTile>(ws, L.tiles), sizeof(QTile) * n, hipMemcpyDeviceToHost),
            "copy tiles");
  }
  return HSTU_OK;
}

hstu_status_t hstu_stochastic_length(const int32_t *offsets, int32_t B, int64_t total_tokens, int32_t max_len,
                                     int32_t cap, const uint32_t *keys, int32_t *new_offsets,
                                     int32_t *gather_idx, int32_t *status, void *stream) {
  if (B < 0) return fail(HSTU_ERR_INVALID_ARG, "B = %d < 0", B);
  if (total_tokens < 0 || total_tokens >= (1ll << 31))
    return fail(HSTU_ERR_INVALID_ARG, "total_tokens = %lld out of [0, 2^31)", (long long)total_tokens);
  if (max_len < 0) return fail(HSTU_ERR_INVALID_ARG, "max_len = %d < 0", max_len);
  if (cap < 1) return fail(HSTU_ERR_INVALID_ARG, "cap = %d < 1", cap);
  if (!offsets || !new_offsets || !status) return fail(HSTU_ERR_INVALID_ARG, "offsets/new_offsets/status NULL");
  if (total_tokens > 0 && (!keys || !gather_idx)) return fail(HSTU_ERR_INVALID_ARG, "keys/gather_idx NULL");
  Timed t_(HSTU_KERNEL_STOCHASTIC_LENGTH, (hipStream_t)stream);
  HIP_TRY(launch_stochastic_length(offsets, B, total_tokens, max_len, cap, keys, new_offsets, gather_idx, status,
                                   (hipStream_t)stream),
          "stochastic length launch");
  return HSTU_OK;
}

hstu_status_t hstu_gather_rows(const void *src, const int32_t *idx, int64_t n, int64_t row_bytes, void *dst,
                               void *stream) {
  if (n < 0) return fail(HSTU_ERR_INVALID_ARG, "n = %lld < 0", (long long)n);
  if (row_bytes <= 0 || row_bytes % 4) return fail(HSTU_ERR_INVALID_ARG, "row_bytes = %lld not a positive multiple of 4", (long long)row_bytes);
  if (n > 0 && (!src || !idx || !dst)) return fail(HSTU_ERR_INVALID_ARG, "src/idx/dst NULL");
  Timed t_(HSTU_KERNEL_GATHER, (hipStream_t)stream);
  HIP_TRY(launch_gather_rows(src, idx, n, row_bytes, dst, (hipStream_t)stream), "gather launch");
  return HSTU_OK;
}

hstu_status_t hstu_balance_bins(const int32_t *offsets, int32_t B, int32_t n_bins, int32_t cost_kind,
                                int32_t *bin, int64_t *bin_cost, void *stream) {
  if (B < 0 || B > 8192) return fail(HSTU_ERR_INVALID_ARG, "B = %d not in [0, 8192]", B);
  if (n_bins < 1 || n_bins > 64) return fail(HSTU_ERR_INVALID_ARG, "n_bins = %d not in [1, 64]", n_bins);
  if (cost_kind != HSTU_COST_TOKENS && cost_kind != HSTU_COST_ATTENTION)
    return fail(HSTU_ERR_INVALID_ARG, "cost_kind = %d", cost_kind);
  if (!offsets || !bin_cost || (B > 0 && !bin)) return fail(HSTU_ERR_INVALID_ARG, "offsets/bin/bin_cost NULL");
  Timed t_(HSTU_KERNEL_BALANCE, (hipStream_t)stream);
  HIP_TRY(launch_balance(offsets, B, n_bins, cost_kind, bin, (long long *)bin_cost, (hipStream_t)stream),
          "balance launch");
  return HSTU_OK;
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------- layer stacks

// Workspace of a stack call: the core's workspace first, then per-layer
// scratch reused by every layer (Z [T, 4D]; U, V, Q, K, Y, O [T, D]; mean,
// rstd [T]), two [T, d_model] buffers the layers alternate between, and
// the GEMM workspace.
struct StackLayout {
  size_t core_bytes, u, v, q, k, yo, o, mean, rstd, x[2], gemm, total;
};

StackLayout stack_layout(const hstu_problem_t *p, int op, int d_model, int microbatch, int hist_max_len) {
  StackLayout y{};
  y.core_bytes = layout(p, op, microbatch, hist_max_len).total;
  const size_t esz = p->dtype == HSTU_BF16 ? 2 : 4;
  const size_t T = (size_t)p->total_tokens, D = (size_t)p->H * p->d;
  size_t off = align256(y.core_bytes);
  y.u = off;    off += align256(T * D * esz);
  y.v = off;    off += align256(T * D * esz);
  y.q = off;    off += align256(T * D * esz);
  y.k = off;    off += align256(T * D * esz);
  y.yo = off;   off += align256(T * D * esz);
  y.o = off;    off += align256(T * D * esz);
  y.mean = off; off += align256(T * sizeof(float));
  y.rstd = off; off += align256(T * sizeof(float));
  y.x[0] = off; off += align256(T * d_model * esz);
  y.x[1] = off; off += align256(T * d_model * esz);
  y.gemm = off; off += kGemmWsBytes;
  y.total = off;
  return y;
}

// The problem of one layer: the caller's batch with this layer's tables and
// affine.
hstu_problem_t layer_problem(const hstu_problem_t *p, const hstu_stack_layer_t &L) {
  hstu_problem_t q = *p;
  q.rab_p = L.rab_p;
  q.rab_t = L.rab_t;
  q.gamma = L.gamma;
  q.beta = L.beta;
  return q;
}

hstu_status_t check_stack(const hstu_problem_t *p, int n_layers, const hstu_stack_layer_t *layers,
                          long long cache_tokens) {
  if (n_layers < 1 || n_layers > 64) return fail(HSTU_ERR_INVALID_ARG, "n_layers = %d not in [1, 64]", n_layers);
  if (!layers) return fail(HSTU_ERR_INVALID_ARG, "layers is NULL");
  for (int l = 0; l < n_layers; ++l) {
    const hstu_stack_layer_t &L = layers[l];
    hstu_status_t s = check_layer(p, &L.w);
    if (s) return s;
    if (L.w.d_model != layers[0].w.d_model) return fail(HSTU_ERR_INVALID_ARG, "layer %d: d_model differs", l);
    if (L.rab_p && p->n_pos < 1) return fail(HSTU_ERR_INVALID_ARG, "layer %d: rab_p given with n_pos = %d", l, p->n_pos);
    if (L.rab_t && p->n_tb < 1) return fail(HSTU_ERR_INVALID_ARG, "layer %d: rab_t given with n_tb = %d", l, p->n_tb);
    if (cache_tokens > 0 && (!L.K_cache || !L.V_cache))
      return fail(HSTU_ERR_INVALID_ARG, "layer %d: K_cache/V_cache must not be NULL", l);
    if (!aligned16(L.K_cache) || !aligned16(L.V_cache))
      return fail(HSTU_ERR_INVALID_ARG, "layer %d: K_cache/V_cache must be 16-byte aligned", l);
  }
  return HSTU_OK;
}

// One layer forward with the activations at U, V, Q, K ([T, D] each): f1
// GEMM, SiLU + split, the attention core (workspace ws_core of core_bytes),
// f2 GEMM. Arguments are checked by the callers.
hstu_status_t layer_forward(const hstu_problem_t *p, const hstu_layer_weights_t *w, const void *X, void *Out,
                            void *Z, void *U, void *V, void *Q, void *K, void *Y, void *O, float *mean, float *rstd,
                            void *ws_core, size_t core_bytes, void *gws, hipStream_t st) {
  const long long T = p->total_tokens;
  const bool bf16 = p->dtype == HSTU_BF16;
  const GemmType et = bf16 ? kGemmBF16 : kGemmF32;
  const long long D = (long long)p->H * p->d, dm = w->d_model;
  if (Z && bf16 && g_fused_proj.load() && f1_silu_gemm_supported(T, (int)dm, (int)D) &&
      f1_silu_gemm_ws_bytes((int)dm, (int)D) <= kGemmWsBytes) {
    // one GEMM writes Z and the four SiLU blocks; W1's transpose goes to gws
    Timed t_(HSTU_KERNEL_PROJ_SILU, st);
    HIP_TRY(launch_f1_silu_gemm(X, T, (int)dm, w->W1, w->b1, (int)D, gws, Z, U, V, Q, K, st), "f1 SiLU GEMM launch");
  } else if (Z) {
    if (T > 0) GEMM_RUN(gemm(false, false, T, 4 * D, dm, X, dm, w->W1, 4 * D, Z, 4 * D, et, et, w->b1), "f1 GEMM");
    Timed t_(HSTU_KERNEL_LAYER_EW, st);
    HIP_TRY(launch_silu_split(Z, T, (int)D, bf16, U, V, Q, K, st), "SiLU split launch");
  } else {
    hstu_status_t s = silu_projection(X, T, dm, *w, D, et, U, V, Q, K, gws, st);
    if (s) return s;
  }
  hstu_status_t s = hstu_attn_fwd(p, Q, K, V, U, Y, O, mean, rstd, ws_core, core_bytes, st);
  if (s) return s;
  if (T > 0) GEMM_RUN(gemm(false, false, T, dm, D, Y, D, w->W2, dm, Out, dm, et, et, w->b2), "f2 GEMM");
  return HSTU_OK;
}
}  // namespace

extern "C" {

hstu_status_t hstu_layer_workspace_size(const hstu_problem_t *p, int32_t d_model, int32_t op, size_t *bytes) {
  if (!bytes) return fail(HSTU_ERR_INVALID_ARG, "bytes is NULL");
  if (op != HSTU_OP_FWD && op != HSTU_OP_BWD) return fail(HSTU_ERR_INVALID_ARG, "op = %d", op);
  hstu_status_t s = check_problem(p, op);
  if (s) return s;
  if (d_model < 1 || d_model > 65536) return fail(HSTU_ERR_INVALID_ARG, "d_model = %d not in [1, 65536]", d_model);
  *bytes = layer_layout(p, op, d_model).total;
  return HSTU_OK;
}

hstu_status_t hstu_layer_fwd(const hstu_problem_t *p, const hstu_layer_weights_t *w, const void *X, void *Out,
                             void *Z, void *UVQK, void *Y, void *O, float *mean, float *rstd, void *ws,
                             size_t ws_bytes, void *stream) {
  hstu_status_t s = check_problem(p, HSTU_OP_FWD);
  if (s) return s;
  s = check_layer(p, w);
  if (s) return s;
  const long long T = p->total_tokens;
  if (T > 0 && (!X || !Out || !Y || !O)) return fail(HSTU_ERR_INVALID_ARG, "X/Out/Y/O must not be NULL");
  if (!aligned16(X) || !aligned16(Out) || !aligned16(Z) || !aligned16(UVQK) || !aligned16(Y) || !aligned16(O))
    return fail(HSTU_ERR_INVALID_ARG, "X/Out/Z/UVQK/Y/O must be 16-byte aligned");
  const LayerLayout y = layer_layout(p, HSTU_OP_FWD, w->d_model);
  s = check_ws(ws, ws_bytes, y.total);
  if (s) return s;
  const size_t td = (size_t)T * p->H * p->d * (p->dtype == HSTU_BF16 ? 2 : 4);
  char *act = UVQK ? static_cast<char *>(UVQK) : at<char>(ws, y.act);
  return layer_forward(p, w, X, Out, Z, act, act + td, act + 2 * td, act + 3 * td, Y, O, mean, rstd, ws,
                       y.core_bytes, at<char>(ws, y.gemm), (hipStream_t)stream);
}

hstu_status_t hstu_layer_bwd(const hstu_problem_t *p, const hstu_layer_weights_t *w, const void *X,
                             const void *Z, const void *UVQK, const void *Y, const void *O, const float *mean,
                             const float *rstd,
                             const void *dOut, void *dX, float *dW1, float *db1, float *dW2, float *db2,
                             float *d_rab_p, float *d_rab_t, float *d_gamma, float *d_beta, void *ws,
                             size_t ws_bytes, void *stream) {
  hstu_status_t s = check_problem(p, HSTU_OP_BWD);
  if (s) return s;
  s = check_layer(p, w);
  if (s) return s;
  const long long T = p->total_tokens;
  if (!dW1 || !dW2) return fail(HSTU_ERR_INVALID_ARG, "dW1/dW2 must not be NULL");
  if (T > 0 && (!X || !Z || !Y || !O || !dOut || !dX))
    return fail(HSTU_ERR_INVALID_ARG, "X/Z/Y/O/dOut/dX must not be NULL");
  if (!aligned16(X) || !aligned16(Z) || !aligned16(UVQK) || !aligned16(Y) || !aligned16(O) || !aligned16(dOut) ||
      !aligned16(dX) || !aligned16(dW1) || !aligned16(dW2))
    return fail(HSTU_ERR_INVALID_ARG, "X/Z/UVQK/Y/O/dOut/dX/dW1/dW2 must be 16-byte aligned");
  const LayerLayout y = layer_layout(p, HSTU_OP_BWD, w->d_model);
  s = check_ws(ws, ws_bytes, y.total);
  if (s) return s;
  hipStream_t st = (hipStream_t)stream;
  const bool bf16 = p->dtype == HSTU_BF16;
  const GemmType et = bf16 ? kGemmBF16 : kGemmF32;
  const long long D = (long long)p->H * p->d, dm = w->d_model;
  const size_t td = (size_t)T * D * (bf16 ? 2 : 4);
  char *act = at<char>(ws, y.act), *gr = at<char>(ws, y.grads);
  void *dY = at<char>(ws, y.dy);
  float *partial = at<float>(ws, y.sums);
  float *wpart = at<float>(ws, y.wpart);
  void *gws = at<char>(ws, y.gemm);
  // U, V, Q, K: the forward's saved activations, or recomputed from Z into ws
  const char *sv = UVQK ? static_cast<const char *>(UVQK) : act;
  const void *U = sv, *V = sv + td, *Q = sv + 2 * td, *K = sv + 3 * td;
  void *dU = gr, *dV = gr + td, *dQ = gr + 2 * td, *dK = gr + 3 * td;

  // f2: dY = dOut W2^T, dW2 = Y^T dOut, db2 = column sums of dOut
  if (T > 0) {
    GEMM_RUN(gemm(false, true, T, D, dm, dOut, dm, w->W2, dm, dY, D, et, et, nullptr), "f2 input-gradient GEMM");
    s = weight_grad(Y, D, dOut, dm, T, et, dW2, wpart, gws, st, "f2 weight-gradient GEMM");
    if (s) return s;
  }
  {
    Timed t_(HSTU_KERNEL_LAYER_EW, st);
    if (T == 0) HIP_TRY(launch_fill_f32(dW2, D * dm, 0.f, st), "fill");
    if (db2) HIP_TRY(launch_colsum(dOut, T, (int)dm, bf16, partial, db2, st), "bias-gradient launch");
    if (!UVQK)
      HIP_TRY(launch_silu_split(Z, T, (int)D, bf16, act, act + td, act + 2 * td, act + 3 * td, st),
              "SiLU split launch");
  }
  void *dZ;
  if (bf16 && g_fused_proj.load()) {
    // the attention core and the norm backward write dZ = [dU|dV|dQ|dK] *
    // SiLU'(Z) themselves, into the gradient buffer (U, V, Q, K may sit in
    // the activation buffer)
    dZ = gr;
    char *dz = gr;
    const size_t blk = (size_t)D * 2;
    const DsiluOut zo{Z, 4 * D};
    s = attn_bwd_impl(p, Q, K, V, U, O, mean, rstd, dY, dz + 2 * blk, dz + 3 * blk, dz + blk, dz, d_rab_p, d_rab_t,
                      d_gamma, d_beta, ws, y.core_bytes, stream, &zo);
    if (s) return s;
    Timed t_(HSTU_KERNEL_LAYER_EW, st);
    if (db1) HIP_TRY(launch_colsum(dZ, T, (int)(4 * D), bf16, partial, db1, st), "bias-gradient launch");
    if (T == 0) HIP_TRY(launch_fill_f32(dW1, dm * 4 * D, 0.f, st), "fill");
  } else {
    // the attention core, then phi1 and f1: dZ = [dU|dV|dQ|dK] * SiLU'(Z)
    // into the activation buffer
    s = hstu_attn_bwd(p, Q, K, V, U, O, mean, rstd, dY, dQ, dK, dV, dU, d_rab_p, d_rab_t, d_gamma, d_beta, ws,
                      y.core_bytes, stream);
    if (s) return s;
    dZ = act;
    Timed t_(HSTU_KERNEL_LAYER_EW, st);
    HIP_TRY(launch_dsilu(Z, dU, dV, dQ, dK, T, (int)D, bf16, dZ, partial, db1, st), "SiLU backward launch");
    if (T == 0) HIP_TRY(launch_fill_f32(dW1, dm * 4 * D, 0.f, st), "fill");
  }
  if (T > 0) {
    s = weight_grad(X, dm, dZ, 4 * D, T, et, dW1, wpart, gws, st, "f1 weight-gradient GEMM");
    if (s) return s;
    GEMM_RUN(gemm(false, true, T, dm, 4 * D, dZ, 4 * D, w->W1, 4 * D, dX, dm, et, et, nullptr),
             "f1 input-gradient GEMM");
  }
  return HSTU_OK;
}

hstu_status_t hstu_stack_workspace_size(const hstu_problem_t *p, int32_t d_model, int32_t op, int32_t microbatch,
                                        int32_t hist_max_len, int64_t hist_tokens, size_t *bytes) {
  if (!bytes) return fail(HSTU_ERR_INVALID_ARG, "bytes is NULL");
  if (op != HSTU_OP_FWD && op != HSTU_OP_MFALCON) return fail(HSTU_ERR_INVALID_ARG, "op = %d", op);
  hstu_status_t s = check_problem(p, op);
  if (s) return s;
  if (op == HSTU_OP_MFALCON && microbatch < 0) return fail(HSTU_ERR_INVALID_ARG, "microbatch = %d < 0", microbatch);
  if (d_model < 1 || d_model > 65536) return fail(HSTU_ERR_INVALID_ARG, "d_model = %d not in [1, 65536]", d_model);
  (void)hist_tokens;
  *bytes = stack_layout(p, op, d_model, microbatch, hist_max_len).total;
  return HSTU_OK;
}

hstu_status_t hstu_stack_history(const hstu_problem_t *hist, int32_t n_layers, const hstu_stack_layer_t *layers,
                                 const void *X, void *Out, void *ws, size_t ws_bytes, void *stream) {
  hstu_status_t s = check_problem(hist, HSTU_OP_FWD);
  if (s) return s;
  s = check_stack(hist, n_layers, layers, hist->total_tokens);
  if (s) return s;
  const long long T = hist->total_tokens;
  const int dm = layers[0].w.d_model;
  if (T > 0 && !X) return fail(HSTU_ERR_INVALID_ARG, "X must not be NULL");
  if (!aligned16(X) || !aligned16(Out)) return fail(HSTU_ERR_INVALID_ARG, "X/Out must be 16-byte aligned");
  const StackLayout y = stack_layout(hist, HSTU_OP_FWD, dm, 0, 0);
  s = check_ws(ws, ws_bytes, y.total);
  if (s) return s;
  hipStream_t st = (hipStream_t)stream;
  const GemmType et = hist->dtype == HSTU_BF16 ? kGemmBF16 : kGemmF32;
  const long long D = (long long)hist->H * hist->d;
  void *gws = at<char>(ws, y.gemm);
  for (int l = 0; l < n_layers; ++l) {
    const hstu_stack_layer_t &L = layers[l];
    hstu_problem_t q = layer_problem(hist, L);
    const void *in = l == 0 ? X : at<char>(ws, y.x[(l - 1) & 1]);
    void *out = (l == n_layers - 1 && Out) ? Out : at<char>(ws, y.x[l & 1]);
    void *U = at<char>(ws, y.u), *Q = at<char>(ws, y.q), *Yh = at<char>(ws, y.yo);
    // K and V of the history go straight into this layer's caches.
    s = silu_projection(in, T, dm, L.w, D, et, U, L.V_cache, Q, L.K_cache, gws, st);
    if (s) return s;
    s = hstu_attn_fwd(&q, Q, L.K_cache, L.V_cache, U, Yh, at<char>(ws, y.o), at<float>(ws, y.mean),
                      at<float>(ws, y.rstd), ws, y.core_bytes, st);
    if (s) return s;
    if (T > 0) GEMM_RUN(gemm(false, false, T, dm, D, Yh, D, L.w.W2, dm, out, dm, et, et, L.w.b2), "f2 GEMM");
  }
  return HSTU_OK;
}

hstu_status_t hstu_stack_score(const hstu_problem_t *cand, int32_t n_layers, const hstu_stack_layer_t *layers,
                               const int32_t *hist_offsets, int64_t hist_tokens, int32_t hist_max_len,
                               const int64_t *hist_ts, int32_t microbatch, const void *Xc, void *Out, void *ws,
                               size_t ws_bytes, void *stream) {
  hstu_status_t s = check_problem(cand, HSTU_OP_MFALCON);
  if (s) return s;
  s = check_mfalcon(cand, hist_offsets, hist_tokens, hist_max_len, microbatch);
  if (s) return s;
  s = check_stack(cand, n_layers, layers, hist_tokens);
  if (s) return s;
  const long long T = cand->total_tokens;
  if (T > 0 && (!Xc || !Out)) return fail(HSTU_ERR_INVALID_ARG, "Xc/Out must not be NULL");
  if (!aligned16(Xc) || !aligned16(Out)) return fail(HSTU_ERR_INVALID_ARG, "Xc/Out must be 16-byte aligned");
  const int dm = layers[0].w.d_model;
  const StackLayout y = stack_layout(cand, HSTU_OP_MFALCON, dm, microbatch, hist_max_len);
  s = check_ws(ws, ws_bytes, y.total);
  if (s) return s;
  hipStream_t st = (hipStream_t)stream;
  const bool bf16 = cand->dtype == HSTU_BF16;
  const GemmType et = bf16 ? kGemmBF16 : kGemmF32;
  const long long D = (long long)cand->H * cand->d;
  void *gws = at<char>(ws, y.gemm);
  for (int l = 0; l < n_layers; ++l) {
    const hstu_stack_layer_t &L = layers[l];
    hstu_problem_t q = layer_problem(cand, L);
    const void *in = l == 0 ? Xc : at<char>(ws, y.x[(l - 1) & 1]);
    void *out = l == n_layers - 1 ? Out : at<char>(ws, y.x[l & 1]);
    void *U = at<char>(ws, y.u), *V = at<char>(ws, y.v), *Q = at<char>(ws, y.q), *K = at<char>(ws, y.k),
         *Yc = at<char>(ws, y.yo);
    s = silu_projection(in, T, dm, L.w, D, et, U, V, Q, K, gws, st);
    if (s) return s;
    s = hstu_mfalcon_score(&q, hist_offsets, hist_tokens, hist_max_len, L.K_cache, L.V_cache, hist_ts, Q, K, V, U,
                           microbatch, Yc, at<char>(ws, y.o), at<float>(ws, y.mean), at<float>(ws, y.rstd), ws,
                           y.core_bytes, stream);
    if (s) return s;
    if (T > 0) GEMM_RUN(gemm(false, false, T, dm, D, Yc, D, L.w.W2, dm, out, dm, et, et, L.w.b2), "f2 GEMM");
  }
  return HSTU_OK;
}

hstu_status_t hstu_stack_score_capture(const hstu_problem_t *cand, int32_t n_layers,
                                       const hstu_stack_layer_t *layers, const int32_t *hist_offsets,
                                       int64_t hist_tokens, int32_t hist_max_len, const int64_t *hist_ts,
                                       int32_t microbatch, const void *Xc, void *Out, void *ws, size_t ws_bytes,
                                       void **graph) {
  if (!graph) return fail(HSTU_ERR_INVALID_ARG, "graph is NULL");
  *graph = nullptr;
  // host-side checks first, so that a bad argument never leaves a capture open
  hstu_status_t s = check_problem(cand, HSTU_OP_MFALCON);
  if (s) return s;
  s = check_mfalcon(cand, hist_offsets, hist_tokens, hist_max_len, microbatch);
  if (s) return s;
  s = check_stack(cand, n_layers, layers, hist_tokens);
  if (s) return s;
  if (int g = gemm_init()) return gemm_fail(g, "hipBLASLt handle");
  hipStream_t cs = nullptr;
  HIP_TRY(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking), "stream create");
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return hip_fail(e, "begin capture");
  }
  s = hstu_stack_score(cand, n_layers, layers, hist_offsets, hist_tokens, hist_max_len, hist_ts, microbatch, Xc, Out,
                       ws, ws_bytes, cs);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);
  (void)hipStreamDestroy(cs);  // clean-up of a stream of our own; its error changes nothing
  if (s) {
    if (g) (void)hipGraphDestroy(g);
    return s;
  }
  if (e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return hip_fail(e, "end capture");
  }
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) return hip_fail(e, "graph instantiate");
  *graph = ex;
  return HSTU_OK;
}

hstu_status_t hstu_graph_launch(void *graph, void *stream) {
  if (!graph) return fail(HSTU_ERR_INVALID_ARG, "graph is NULL");
  HIP_TRY(hipGraphLaunch((hipGraphExec_t)graph, (hipStream_t)stream), "graph launch");
  return HSTU_OK;
}

hstu_status_t hstu_graph_destroy(void *graph) {
  if (!graph) return fail(HSTU_ERR_INVALID_ARG, "graph is NULL");
  HIP_TRY(hipGraphExecDestroy((hipGraphExec_t)graph), "graph destroy");
  return HSTU_OK;
}

hstu_status_t hstu_get_device_status(const void *ws, void *stream, int32_t *host_code) {
  if (!ws || !host_code) return fail(HSTU_ERR_INVALID_ARG, "NULL argument");
  hipStream_t st = (hipStream_t)stream;
  int v = 0;
  HIP_TRY(hipMemcpyAsync(&v, ws, sizeof v, hipMemcpyDeviceToHost, st), "copy status");
  HIP_TRY(hipStreamSynchronize(st), "stream synchronize");
  *host_code = v;
  return HSTU_OK;
}

hstu_status_t hstu_kernel_timing(int32_t enable) {
  std::lock_guard<std::mutex> g(g_timing_mu);
  timing_clear_locked();
  g_timing_on = enable != 0;
  return HSTU_OK;
}

hstu_status_t hstu_kernel_timing_read(int32_t kernel, double *total_ms, int64_t *launches) {
  if (!total_ms || !launches) return fail(HSTU_ERR_INVALID_ARG, "NULL argument");
  if (kernel < 0 || kernel >= HSTU_KERNEL_COUNT) return fail(HSTU_ERR_INVALID_ARG, "kernel id %d", kernel);
  std::lock_guard<std::mutex> g(g_timing_mu);
  double ms = 0.0;
  int64_t n = 0;
  std::vector<TimingRecord> keep;
  for (auto &r : g_timing) {
    if (r.kernel != kernel) {
      keep.push_back(r);
      continue;
    }
    HIP_TRY(hipEventSynchronize(r.stop), "event synchronize");
    float e = 0.f;
    HIP_TRY(hipEventElapsedTime(&e, r.start, r.stop), "event elapsed time");
    ms += e;
    n++;
    (void)hipEventDestroy(r.start);  // read; a failed destroy leaves nothing to undo
    (void)hipEventDestroy(r.stop);
  }
  g_timing.swap(keep);
  *total_ms = ms;
  *launches = n;
  return HSTU_OK;
}

}  // extern "C"
