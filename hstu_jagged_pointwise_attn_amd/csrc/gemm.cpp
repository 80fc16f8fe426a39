// Row-major GEMMs of the layer's projections f1 and f2 (HSTU blog, section 3,
// the layer formula) on hipBLASLt.
//
// hipBLASLt is column-major; a row-major C[M, N] = op(A) op(B) is issued as
// the column-major C^T[N, M] = op(B)^T op(A)^T, i.e. with the operands
// swapped and each one's transpose flag kept (a row-major matrix read in
// place is its own transpose in column-major). A bias over the N columns of
// the row-major C is then a bias over the rows of the column-major result,
// which is hipBLASLt's BIAS epilogue; SiLU after it is the SWISH epilogue
// (x sigmoid(x)), applied in fp32 before C is rounded.
//
// One hipBLASLt handle per device is created on first use and kept for the
// life of the process. For a new problem (types, flags, sizes, epilogue) the
// candidates of hipBLASLt's heuristic that fit the workspace are timed on the
// caller's stream (a few runs each, then one host wait) and the fastest is
// cached; under stream capture the heuristic's first choice is taken
// untimed.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
hipblasLtHandle_t g_handle[kMaxDevices] = {};

// Algorithm cache key: device, types, transposes, epilogue, accumulate, the
// sizes rounded up to a grid of four steps per octave (a batch of jagged
// sequences changes the token count every step), whether each matrix is
// dense, the workspace size and the batch count.
using Key = std::tuple<int, int, int, int, int, int, bool, long long, long long, long long, bool, bool, bool, size_t,
                       int>;
constexpr int kCandidates = 32;
constexpr int kTuneRuns = 3;

long long bucket(long long x) {
  if (x <= 64) return x;
  int e = 63 - __builtin_clzll((unsigned long long)x);  // 2^e <= x
  const long long step = 1LL << (e - 2);
  return (x + step - 1) / step * step;
}
struct Choice {
  hipblasLtMatmulAlgo_t algo;
  size_t ws;
};
std::map<Key, Choice> g_algo;

hipDataType hip_type(GemmType t) { return t == kGemmBF16 ? HIP_R_16BF : HIP_R_32F; }

// RAII holders for the descriptors of one call.
struct Descs {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  ~Descs() {
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (c) hipblasLtMatrixLayoutDestroy(c);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
};

}  // namespace

const char *gemm_status_text(int st) {
  switch (st) {
    case HIPBLAS_STATUS_SUCCESS: return "success";
    case HIPBLAS_STATUS_NOT_INITIALIZED: return "hipBLASLt not initialised";
    case HIPBLAS_STATUS_ALLOC_FAILED: return "hipBLASLt allocation failed";
    case HIPBLAS_STATUS_INVALID_VALUE: return "hipBLASLt invalid value";
    case HIPBLAS_STATUS_ARCH_MISMATCH: return "hipBLASLt architecture mismatch";
    case HIPBLAS_STATUS_EXECUTION_FAILED: return "hipBLASLt execution failed";
    case HIPBLAS_STATUS_NOT_SUPPORTED: return "hipBLASLt: no algorithm for this problem";
    default: return "hipBLASLt error";
  }
}

bool gemm_unsupported(int st) { return st == HIPBLAS_STATUS_NOT_SUPPORTED; }

namespace {
// The current device's handle, created on first use.
int handle_for_current(hipblasLtHandle_t *h, int *dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HIPBLAS_STATUS_NOT_INITIALIZED;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_handle[dev]) {
    hipblasStatus_t st = hipblasLtCreate(&g_handle[dev]);
    if (st != HIPBLAS_STATUS_SUCCESS) {
      g_handle[dev] = nullptr;
      return st;
    }
  }
  *h = g_handle[dev];
  *dev_out = dev;
  return HIPBLAS_STATUS_SUCCESS;
}
}  // namespace

int gemm_init() {
  hipblasLtHandle_t h;
  int dev;
  return handle_for_current(&h, &dev);
}

int gemm_rm(const GemmRM &g, void *ws, size_t ws_bytes, hipStream_t stream) {
  int dev = 0;
  hipblasLtHandle_t h;
  if (int e = handle_for_current(&h, &dev)) return e;
  const hipDataType tab = hip_type(g.ab), tc = hip_type(g.c);
  // column-major problem: m = N, n = M, k = K; A' = B, B' = A
  const uint64_t m = g.N, n = g.M, k = g.K;
  const hipblasOperation_t opa = g.tb ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  const hipblasOperation_t opb = g.ta ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  Descs d;
  hipblasStatus_t st;
#define GEMM_TRY(x)                                  \
  do {                                               \
    st = (x);                                        \
    if (st != HIPBLAS_STATUS_SUCCESS) return st;     \
  } while (0)
  GEMM_TRY(hipblasLtMatmulDescCreate(&d.op, HIPBLAS_COMPUTE_32F, HIP_R_32F));
  const int32_t ta = opa, tb = opb;
  GEMM_TRY(hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta));
  GEMM_TRY(hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb));
  if (g.bias || g.silu) {
    const uint32_t epi = g.silu ? (g.bias ? HIPBLASLT_EPILOGUE_SWISH_BIAS_EXT : HIPBLASLT_EPILOGUE_SWISH_EXT)
                                : HIPBLASLT_EPILOGUE_BIAS;
    GEMM_TRY(hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof epi));
  }
  if (g.bias) {
    const int32_t bt = HIP_R_32F;
    const void *bp = g.bias;
    GEMM_TRY(hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bt, sizeof bt));
    GEMM_TRY(hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bp, sizeof bp));
  }
  // stored shapes (before op): A' is m x k (N) or k x m (T); B' is k x n or n x k
  GEMM_TRY(hipblasLtMatrixLayoutCreate(&d.a, tab, opa == HIPBLAS_OP_N ? m : k, opa == HIPBLAS_OP_N ? k : m, g.ldb));
  GEMM_TRY(hipblasLtMatrixLayoutCreate(&d.b, tab, opb == HIPBLAS_OP_N ? k : n, opb == HIPBLAS_OP_N ? n : k, g.lda));
  GEMM_TRY(hipblasLtMatrixLayoutCreate(&d.c, tc, m, n, g.ldc));
  if (g.batch > 1) {
    const int32_t bc = g.batch;
    const int64_t sa = g.sB, sb = g.sA, sc = g.sC;  // A' is B, B' is A
    GEMM_TRY(hipblasLtMatrixLayoutSetAttribute(d.a, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &bc, sizeof bc));
    GEMM_TRY(hipblasLtMatrixLayoutSetAttribute(d.b, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &bc, sizeof bc));
    GEMM_TRY(hipblasLtMatrixLayoutSetAttribute(d.c, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &bc, sizeof bc));
    GEMM_TRY(hipblasLtMatrixLayoutSetAttribute(d.a, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &sa, sizeof sa));
    GEMM_TRY(hipblasLtMatrixLayoutSetAttribute(d.b, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &sb, sizeof sb));
    GEMM_TRY(hipblasLtMatrixLayoutSetAttribute(d.c, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &sc, sizeof sc));
  }

  const Key key{dev, (int)g.ab, (int)g.c, (int)opa, (int)opb, (g.bias != nullptr) + 2 * g.silu, g.accumulate, bucket(g.M),
                bucket(g.N), bucket(g.K), g.lda == g.K || g.lda == g.M, g.ldb == g.N || g.ldb == g.K, g.ldc == g.N,
                ws_bytes, g.batch > 1 ? g.batch : 1};
  const float alpha = 1.0f, beta = g.accumulate ? 1.0f : 0.0f;
  auto run = [&](const Choice &c) {
    return hipblasLtMatmul(h, d.op, &alpha, g.B, d.a, g.A, d.b, &beta, g.C, d.c, g.C, d.c, &c.algo,
                           c.ws ? ws : nullptr, c.ws, stream);
  };
  Choice ch;
  bool have = false;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_algo.find(key);
    if (it != g_algo.end()) {
      ch = it->second;
      have = true;
    }
  }
  // A choice made for another size of the same bucket is used when
  // hipBLASLt accepts it for this size.
  if (have && run(ch) == HIPBLAS_STATUS_SUCCESS) return HIPBLAS_STATUS_SUCCESS;

  GEMM_TRY(hipblasLtMatmulPreferenceCreate(&d.pref));
  const uint64_t wsb = ws_bytes;
  GEMM_TRY(hipblasLtMatmulPreferenceSetAttribute(d.pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof wsb));
  hipblasLtMatmulHeuristicResult_t res[kCandidates];
  int count = 0;
  GEMM_TRY(hipblasLtMatmulAlgoGetHeuristic(h, d.op, d.a, d.b, d.c, d.c, d.pref, kCandidates, res, &count));
  std::vector<Choice> cands;
  for (int i = 0; i < count; ++i)
    if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= ws_bytes)
      cands.push_back({res[i].algo, res[i].workspaceSize});
  if (cands.empty()) return HIPBLAS_STATUS_NOT_SUPPORTED;
  ch = cands[0];
  // Time the candidates on this problem (not while the stream is being
  // captured, and not when accumulating into C, which repeated runs would
  // change).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  const bool tune = cands.size() > 1 && !g.accumulate && hipStreamIsCapturing(stream, &cap) == hipSuccess &&
                    cap == hipStreamCaptureStatusNone;
  if (tune) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
      float best = 1e30f;
      for (const Choice &c : cands) {
        if (run(c) != HIPBLAS_STATUS_SUCCESS) continue;  // warm-up; skip what fails
        bool timed = hipEventRecord(e0, stream) == hipSuccess;
        for (int r = 0; r < kTuneRuns; ++r) run(c);
        timed = timed && hipEventRecord(e1, stream) == hipSuccess;
        float ms = 0.f;
        if (timed && hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess &&
            ms < best) {
          best = ms;
          ch = c;
        }
      }
    }
    if (e0) (void)hipEventDestroy(e0);  // nothing to do if a destroy fails
    if (e1) (void)hipEventDestroy(e1);
  }
  GEMM_TRY(run(ch));
  std::lock_guard<std::mutex> lk(g_mu);
  g_algo[key] = ch;
#undef GEMM_TRY
  return HIPBLAS_STATUS_SUCCESS;
}

}  // namespace hstu
