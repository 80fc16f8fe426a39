// f1 of an HSTU layer with the SiLU split in its GEMM epilogue (proj_gemm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace hstu {

// Shapes the fused GEMM takes (d_model and D multiples of 8).
bool f1_silu_gemm_supported(long long T, int dm, int D);
// Bytes of the W1^T copy it needs (4 D x dm bf16).
size_t f1_silu_gemm_ws_bytes(int dm, int D);
// W1 [dm, 4D] is transposed into W1t (f1_silu_gemm_ws_bytes), then Z [T, 4D]
// = X W1 + b1 and U, V, Q, K [T, D] = the four column blocks of SiLU(Z) are
// written (bf16). b1 may be NULL. Asynchronous on `s`.
hipError_t launch_f1_silu_gemm(const void *X, long long T, int dm, const void *W1, const float *b1, int D,
                               void *W1t, void *Z, void *U, void *V, void *Q, void *K, hipStream_t s);

}  // namespace hstu
