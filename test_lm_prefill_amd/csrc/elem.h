// Norm, rotary, embedding, SwiGLU-backward, cross-entropy reduction and
// small bookkeeping kernels (gfx950).  All launchers enqueue on `st`.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// h[t, :] = E[tok[*pos0 + t], :] as fp32.
hipError_t embed_launch(int dtype, const void *E, const int *tok, const int *pos0, float *h, int n, int d,
                        hipStream_t st);

// y = x * r * g, r = (mean(x^2) + eps)^-1/2 per row; optional r_out [n] and x_copy [n, d].
// g has the working dtype; y too, or fp16 when y_f16 (bf16 mode's forward GEMM operand).
// d <= 8192.  With red.ws set, x is first updated in place by a split-K residual
// product: x += red.sc * (ws[0] + ws[1] + ... + ws[red.split - 1]) with ws[s] the
// fp32 partial [n, d] at red.ws + s * n * d, summed in that order (the reduction a
// separate split-K reduce would apply), and the updated x is normalised.
struct ResidualPartials {
  const float *ws = nullptr;
  int split = 0;
  float sc = 1.f;
};
hipError_t rmsnorm_fwd_launch(int dtype, float *x, const void *g, void *y, float *r_out, float *x_copy, int n, int d,
                              float eps, hipStream_t st, bool y_f16 = false, ResidualPartials red = {});

// dh_out = dh_in + r * (g*dy) - x * r^3 * mean(x * g*dy)   (dh_in may be NULL or alias dh_out);
// also writes dh_t, the same values in the working dtype (fp16 when t_f16, bf16 mode only).
hipError_t rmsnorm_bwd_launch(int dtype, const float *dy, const float *x, const float *r, const void *g,
                              const float *dh_in, float *dh_out, void *dh_t, int n, int d, hipStream_t st,
                              bool t_f16 = false);

struct RopeArgs {
  const float *qkv;     // [n][3d] pre-norm q | k | v (fp32: the GEMM output is not rounded before the norm)
  const void *gq, *gk;  // [hd] QK-norm gains
  const float2 *cs;     // rotary table [max_pos][hd/2] of (cos, sin) pairs
  const int *pos0;
  int n, d, H, hd, R;
  float eps;
  // forward outputs
  void *qh;             // [n][d] forward type
  void *qhb;            // [n][d] working-dtype copy of qh (backward) or NULL
  void *qht;            // [H][hd][ldt] or NULL
  // ring planes: K [H][R][hd] and Vt [H][hd][R] in the forward type (fp16 when
  // fwd_f16, else the working dtype), used by the forward attention and the
  // score recomputation; Kb [H][R][hd], Kt [H][hd][R] and V [H][R][hd] in the
  // working dtype for the backward (each may be NULL)
  void *K, *Vt, *Kb, *Kt, *V;
  int fwd_f16;          // qh, K and Vt are fp16
  int ldt;
  // backward inputs / output
  const float *dqh, *dkh, *dv;  // [n][d]
  void *dqkv;           // [n][3d]
};
hipError_t qk_rope_fwd_launch(int dtype, const RopeArgs &a, hipStream_t st);
hipError_t qk_rope_bwd_launch(int dtype, const RopeArgs &a, hipStream_t st);

// Dq[h, q] = sum_i dO[q, h, i] * O[q, h, i];  dOt[h, i, q] = dO[q, h, i].
// O is fp16 when o_f16 (the forward output), else the working dtype.
hipError_t attn_bwd_pre_launch(int dtype, const void *dO, const void *O, float *Dq, void *dOt, int n, int d,
                               int H, int hd, int ldl, int ldt, hipStream_t st, bool o_f16);

// SwiGLU backward over 16-row interleaved gate/up blocks.  GU [n][ld_gu],
// dhmid [n][ld_h] (units), dGU [n][ld_gu]; `units` hidden units processed.
// All three are fp16 when f16 (bf16 mode only), else the working dtype.
hipError_t swiglu_bwd_launch(int dtype, const void *GU, const void *dhmid, void *dGU, int n, int units,
                             long ld_gu, long ld_h, hipStream_t st, bool f16 = false);

// Combines per-row partials (max, sum exp) into lse[m] and
// losses[*pos0 + m] = lse - zlab[m].
// Per-row shift of the single-pass head: shift[m] = n_f[m] . W[label] + off (one wave per
// row; f16: both operands fp16 in bf16 mode, else the working dtype).
hipError_t head_shift_launch(int dtype, bool f16, const void *nf, const void *W, const int *labs, const int *pos0,
                             float *shift, int n, int d, float off, hipStream_t st);
// dn[m] = alpha (dn[m] exp(shift[m] - lse[m]) - W[label of m]) over the d columns of each row.
hipError_t head_grad_finish_launch(int dtype, bool f16, float *dn, const float *shift, const float *lse, const void *W,
                                   const int *labs, const int *pos0, int n, int d, float alpha, hipStream_t st);
hipError_t ce_reduce_launch(const float2 *part, int P, const float *zlab, const int *pos0, float *lse,
                            float *losses, int n, hipStream_t st);

// Batched chunk of B sequences, n positions each, row r = s * n + m at position
// *pos0 + m of sequence s: ids[r] = tok[s * ld_tok + *pos0 + m], labs[r] = the
// id after it; and losses[s * ld_loss + *pos0 + m] = closs[r].
// dst[s n + t][:] = src[s (*src_n) + (*pos0 mod G) + t][:] for s < B, t < n (fp32 rows of d,
// d % 4 == 0): a chunk's residual rows from the frozen-prefix pass of its group (groups start
// at multiples of G; that pass ran *src_n rows per sequence).
hipError_t lead_rows_launch(const float *src, const int *src_n, int G, const int *pos0, float *dst, int n, int d,
                            int B, hipStream_t st);
hipError_t gather_chunk_ids_launch(const int *tok, long ld_tok, const int *pos0, int n, int B, int *ids, int *labs,
                                   hipStream_t st);
hipError_t scatter_chunk_losses_launch(const float *closs, float *losses, long ld_loss, const int *pos0, int n, int B,
                                       hipStream_t st);

// Greedy choice for the last of n rows: over the per-tile partials (max, sum
// exp) and their argmax columns, the largest logit (lowest id on ties) goes to
// tok[*pos0 + n] and lse[n-1] - max to losses[*pos0 + n - 1].
hipError_t decode_pick_launch(const float2 *part, const int *part_arg, int P, const float *lse, const int *pos0, int n,
                              int *tok, float *losses, hipStream_t st);

// Rotary table: cs[p][i] = (cos, sin)(p * theta^(-2i/hd)) evaluated in fp64.
hipError_t rope_table_launch(float2 *cs, long max_pos, int hd, double theta, hipStream_t st);

// With x = scale * src[r * ld_src + c]: dst[r * ld_dst + c] = hi = (T) x; when lo
// is given also lo[r * ld_lo + c] = (T) (x - hi), so that hi + lo carries x to
// about 16 (bf16) or 22 (fp16) significant bits.  dtype 2 writes fp16; `scale`
// (a power of two) keeps fp16's lo part out of the subnormal range.
hipError_t convert_rows_launch(int dtype, const float *src, long ld_src, void *dst, long ld_dst, int rows, int cols,
                               hipStream_t st, void *lo = nullptr, long ld_lo = 0, float scale = 1.f);
// dst (T) = src (T) copies with row strides.
hipError_t copy_rows_launch(int dtype, const void *src, long ld_src, void *dst, long ld_dst, int rows, int cols,
                            hipStream_t st);

// dst[c * ldd + r] = r < R ? src[r * lds + c] : 0 for r < Rpad, c < C.  The
// destination has the working dtype, or fp16 when dst_f16 (bf16 mode only);
// the source is fp32 (SRC_F32, always in fp32 mode), the working dtype
// (SRC_WORK) or fp16 (SRC_F16, bf16 mode).
enum { SRC_F32 = 0, SRC_WORK = 1, SRC_F16 = 2 };
hipError_t transpose_launch(int dtype, int src_kind, const void *src, long lds, void *dst, long ldd, int R, int Rpad,
                            int C, hipStream_t st, bool dst_f16 = false);
// dst (fp16) = scale * src (bf16), exact when the scaled value is in fp16's
// normal range (scale a power of two), with row strides.
hipError_t bf16_to_f16_launch(const void *src, long lds, void *dst, long ldd, int rows, int cols, hipStream_t st,
                              float scale = 1.f);
// *out = max(*out, bit pattern of max |x|) over a [rows][cols] block with row
// stride ld (dtype 0 fp32, 1 bf16); *out must start at 0.  NaN counts as largest.
// *out = max(*out, largest row norm of x [rows][cols]) as float bits (set *out to 0 first).
hipError_t rownorm_max_launch(int dtype, const void *x, long ld, int rows, int cols, unsigned *out, hipStream_t st);
hipError_t absmax_launch(int dtype, const void *x, long ld, int rows, int cols, unsigned *out, hipStream_t st);

hipError_t set_int_launch(int *p, int v, hipStream_t st);
hipError_t add_int_launch(int *p, int v, hipStream_t st);
hipError_t zero_launch(void *p, size_t bytes, hipStream_t st);
// flag |= 1 if any of x[0..n) is not finite.
hipError_t finite_check_launch(const float *x, long n, int *flag, hipStream_t st);
