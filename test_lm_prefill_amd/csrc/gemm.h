// MFMA GEMM for gfx950: C[m, n] = sum_k A[m, k] * B[n, k], fp32 accumulation,
// with fused epilogues.  Host-side launcher declarations.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

enum GemmEpi {
  EPI_STORE = 0,     // C (T) = acc
  EPI_STORE_F32 = 1, // Cf (fp32) = acc
  EPI_ADD_F32 = 2,   // Cf (fp32) += acc            (residual stream)
  EPI_SWIGLU = 3,    // C (T)[m, unit] = silu(gate) * up over 16-row interleaved gate/up
                     // blocks of B; C2 (T, optional) = raw gate/up pre-activations
  EPI_CE = 4,        // per-row partial (max, sum exp) over the tile's columns and the
                     // label logit -> part / zlab   (cross-entropy)
  EPI_PROBS = 5,     // C (T) = exp(acc - rowf[m]) with a per-row shift rowf; per row and
                     // 64-column slot the partial (rowf[m], sum of those exponentials in
                     // fp32) at slot col_off / 64 + local slot, and the label logit -> zlab
                     // (cross-entropy and the unnormalised softmax in one pass; C, part and
                     // zlab may each be null)
  EPI_SGD = 6,       // Cf (fp32 master) -= alpha * acc; C (T) = hi = round(c_scale * Cf) and,
                     // when C2 is set, C2 (T) = round(c_scale * Cf - hi): the working copy as
                     // hi + lo, scaled by c_scale (inner SGD); when CT is set, also
                     // CT[n][m] = round(Cf[m][n]) (the transposed working copy)
};

struct GemmArgs {
  const void *A;  // A[m, k] at A[m * lda + k] (a_kc) or A[k * lda + m] (!a_kc)
  const void *B;  // B[n, k] at B[n * ldb + k] (b_kc) or B[k * ldb + n] (!b_kc)
  long lda, ldb;
  int M, N, K;
  void *C;
  long ldc;
  float *Cf;
  long ldcf;
  void *C2;
  long ldc2;
  const float *rowf;  // per-row shift (EPI_PROBS)
  const int *rowi;    // labels: label of row m = rowi[*pos0 + m]
  const int *pos0;
  float2 *part;       // EPI_CE / EPI_PROBS partials [M][part_ld]
  int part_ld;
  float *zlab;        // EPI_CE / EPI_PROBS label logits [M]
  int *part_arg;      // EPI_CE, optional: per-tile argmax column (+ col_off) beside each partial, lowest on ties
  float alpha;
  int col_off;
  // > 0: A is [M][a_kwrap] and its reduction index is taken modulo a_kwrap, so
  // the product runs over [A | A | ...] and K may span several weight blocks
  // that multiply the same activations (a multiple of 64, or of 8 for the
  // generic kernel)
  int a_kwrap;
  // 16-bit outputs (C and C2) are written as fp16 instead of bf16 (streaming
  // kernel; the generic kernel writes its operand type)
  int c_f16;
  // EPI_SWIGLU and EPI_ADD_F32 multiply the accumulator by acc_scale first (a
  // power of two: B holds weights stored scaled by 1 / acc_scale); EPI_SGD
  // writes its 16-bit copies scaled by c_scale.  Both are 1 when unused.
  float acc_scale, c_scale;
  // EPI_SGD, optional: the updated fp32 values also written transposed and unscaled,
  // CT[n * ldct + m], in the 16-bit output type (the streaming kernel) or the operand
  // type (the generic kernel)
  void *CT;
  long ldct;
  // split-K (internal)
  int ksplit;
  float *ws;
};

// Up to GEMM_GROUP_MAX products run as one launch (gemm_group_launch).
#define GEMM_GROUP_MAX 8
struct GemmGroup {
  GemmArgs g[GEMM_GROUP_MAX];
  int beg[GEMM_GROUP_MAX];  // first block of each product (set by the launcher)
  int n;
};

// dtype (operand type): 0 = fp32, 1 = bf16, 2 = fp16.  a_kc / b_kc select the
// operand layouts.  fp16 operands need the streaming kernel's shapes (both
// k-contiguous, K and a_kwrap multiples of 64, leading dimensions multiples of 8).
// For EPI_STORE / EPI_STORE_F32 / EPI_ADD_F32 the launcher may split K over
// several work-groups into `ws` (fp32, ws_elems entries) and reduce in a fixed
// order, which keeps results deterministic.
hipError_t gemm_launch(int dtype, bool a_kc, bool b_kc, int epi, GemmArgs g, float *ws, size_t ws_elems,
                       hipStream_t st, int force_split = 0);

// Number of fp32 partial entries the launcher may need for an M x N output.
size_t gemm_ws_elems(int M, int N);

// How a product runs: the K split (fp32 partials in a workspace when > 1) and, for
// 16-bit k-contiguous operands, whether the 256 x 256 tile (wide) or the 128 x 128 tile
// computes it.  Both tiles sum every output element in the same order.
struct GemmPlan {
  int split = 1;
  bool wide = false;
};

// The same work in two launches, for callers that time them separately:
// gemm_plan returns the plan gemm_launch would use; gemm_main_launch runs the GEMM
// (partials to ws when split > 1; allow_gemv = false keeps products of a few rows on
// the tiled kernels); gemm_reduce_launch applies the epilogue to the fixed-order sum of
// the partials.
GemmPlan gemm_plan(int dtype, bool a_kc, bool b_kc, int epi, const GemmArgs &g, size_t ws_elems, int force_split = 0);
hipError_t gemm_main_launch(int dtype, bool a_kc, bool b_kc, int epi, GemmArgs g, float *ws, GemmPlan plan,
                            hipStream_t st, bool allow_gemv = true);
hipError_t gemm_reduce_launch(int dtype, int epi, GemmArgs g, float *ws, int split, hipStream_t st);

// n products with the same operand type, layouts and epilogue, each with results
// identical to its own gemm_launch: one launch of the 256 x 256 tile over all their tiles
// when every product is a 16-bit k-contiguous product that needs no K split (so that
// products too small to fill the chip share its rounds of tiles), else one launch each.
// Implemented for EPI_SWIGLU.
hipError_t gemm_group_launch(int dtype, int epi, const GemmArgs *gs, int n, float *ws, size_t ws_elems,
                             hipStream_t st);
