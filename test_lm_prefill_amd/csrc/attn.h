// Sliding-window attention over per-layer key/value rings (gfx950).
#pragma once
#include <hip/hip_runtime.h>

// Ring layouts, per layer and head h, R rows (R a multiple of 64; position j
// lives in row j mod R):
//   K  [H][R][hd]   rotated, normalised keys
//   Vt [H][hd][R]   values, transposed (slot-contiguous)
//   Kt [H][hd][R]   keys transposed     (only layers whose attention is back-propagated)
//   V  [H][R][hd]   values              (same)
struct AttnArgs {
  const void *q;     // [n][d]  rotated, normalised queries of the chunk
  const void *qt;    // [H][hd][ldt] same, transposed (backward only)
  const void *dout;  // [n][d]  gradient of the attention output (backward)
  const void *doutt; // [H][hd][ldt] same, transposed (backward)
  const void *K, *Vt, *Kt, *V;
  void *o;           // [n][d]  output (forward)
  float *lse2;       // [H][ldl] log2-sum-exp of scaled scores per query
  const float *Dq;   // [H][ldl] rowsum(dO * O) (backward)
  float *dq;         // [n][d] fp32 (backward)
  float *dk;         // [n][d] fp32, chunk keys (backward)
  float *dv;         // [n][d] fp32, chunk values (backward)
  int n, d, H, R, window, ldl, ldt;
  const int *pos0;   // absolute position of the chunk's first query (device)
  float scale;       // 1/sqrt(hd)
  float sbound;      // forward: bound of scale * q.k in log2 units (bf16 bounded kernel), 0 = none
  int fwd_f16;       // forward operands q, K, Vt are fp16 (bounded kernel only; needs sbound <= 14.5)
  int o_f16;         // forward output o (and its merge) is fp16
  // key-range split (forward and dQ): nsplit work-groups share one query tile;
  // their partial results go to ws (fp32) and are merged in a fixed order.
  int nsplit;
  float *ws;         // forward: [nsplit][n][d] outputs then [nsplit][H][ldl] log2-sum-exp; dQ: [nsplit][n][d]
};

// Work-space floats the forward / dQ passes need for `nsplit` splits.
size_t attn_ws_floats(int nsplit, int n, int d, int H, int ldl);
// Split count that gives the GPU enough work-groups for this shape (dQ pass,
// and the forward when it runs without a score bound).
int attn_pick_split(int n, int H, int window, int chunk);
// The forward's split count: the bounded kernel covers 256 queries per work-group.
int attn_fwd_split(int dtype, float sbound, int hd, int n, int H, int window, int chunk);
// Largest score bound (log2 units) the bounded forward accepts: 2^-2B must
// stay a normal fp32 number with room for sums.
constexpr float ATTN_MAX_SBOUND = 48.f;
// Whether the bounded forward can keep q, k, v and the weights in fp16: its
// weights 2^(s - B + 15) stay normal fp16 numbers while B <= 14.5.
bool attn_fwd_f16_ok(int dtype, float sbound, int hd);

hipError_t attn_fwd_launch(int dtype, int hd, const AttnArgs &a, hipStream_t st);
hipError_t attn_bwd_dq_launch(int dtype, int hd, const AttnArgs &a, hipStream_t st);
hipError_t attn_bwd_dkdv_launch(int dtype, int hd, const AttnArgs &a, hipStream_t st);
// Combines the key-range splits (no-op when nsplit == 1): forward outputs and
// log-sum-exp (dq = false) or the dQ partial sums (dq = true).
hipError_t attn_merge_launch(int dtype, int hd, bool dq, const AttnArgs &a, hipStream_t st);
bool attn_supported_hd(int hd);
