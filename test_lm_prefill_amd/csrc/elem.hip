// Memory-bound kernels of the chunk step: embedding gather, RMSNorm forward /
// backward, QK-norm + rotary + ring write (and its backward), the attention
// backward pre-pass, SwiGLU backward and the cross-entropy row reduction.
// Statistics are accumulated in fp32; inputs/outputs use the working dtype.
#include "common.h"
#include "elem.h"

namespace {

template <typename T> DEVI void load4(const T *p, float *v);
template <> DEVI void load4<float>(const float *p, float *v) {
  float4 x = *reinterpret_cast<const float4 *>(p);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
template <> DEVI void load4<f16_t>(const f16_t *p, float *v) {
  uint2 x = *reinterpret_cast<const uint2 *>(p);
  v[0] = to_f(f16_t{(uint16_t)(x.x & 0xFFFF)}); v[1] = to_f(f16_t{(uint16_t)(x.x >> 16)});
  v[2] = to_f(f16_t{(uint16_t)(x.y & 0xFFFF)}); v[3] = to_f(f16_t{(uint16_t)(x.y >> 16)});
}
template <> DEVI void load4<bf16_t>(const bf16_t *p, float *v) {
  uint2 x = *reinterpret_cast<const uint2 *>(p);
  v[0] = to_f((bf16_t)(x.x & 0xFFFF)); v[1] = to_f((bf16_t)(x.x >> 16));
  v[2] = to_f((bf16_t)(x.y & 0xFFFF)); v[3] = to_f((bf16_t)(x.y >> 16));
}

// ----------------------------------------------------------------- embedding
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T *E, const int *tok, const int *pos0, float *h, int d) {
  const int t = blockIdx.x;
  const long row = tok[*pos0 + t];
  for (int i = threadIdx.x * 4; i < d; i += 1024) {
    float v[4];
    load4<T>(E + row * d + i, v);
    store4<float>(h + (long)t * d + i, v);
  }
}

// ----------------------------------------------------------------- RMSNorm
// One 256-thread block per row; the row stays in registers (NV float4 per thread,
// d <= 1024 NV) so x (and dy) are read from HBM once.  A block per row (rather than a
// wave) keeps four times as many loads in flight, which a chunk of ~1K rows needs to
// approach the HBM rate.
DEVI float block_sum4(float v, float *red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename T, typename TY, int NV>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(float *x, const T *g, TY *y, float *r_out, float *x_copy,
                                                          int n, int d, float eps, ResidualPartials rp) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const long o = (long)row * d;
  float4 v[NV];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int i = (k * 256 + threadIdx.x) * 4;
    v[k] = i < d ? *reinterpret_cast<const float4 *>(x + o + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    if (rp.ws && i < d) {  // pending split-K residual product, summed in split order
      const long st = (long)n * d;
      float4 acc = *reinterpret_cast<const float4 *>(rp.ws + o + i);
      for (int s = 1; s < rp.split; ++s) {
        const float4 p = *reinterpret_cast<const float4 *>(rp.ws + s * st + o + i);
        acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
      }
      v[k] = make_float4(v[k].x + acc.x * rp.sc, v[k].y + acc.y * rp.sc, v[k].z + acc.z * rp.sc,
                         v[k].w + acc.w * rp.sc);
      *reinterpret_cast<float4 *>(x + o + i) = v[k];
    }
    ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
  }
  ss = block_sum4(ss, red);
  const float r = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int i = (k * 256 + threadIdx.x) * 4;
    if (i < d) {
      float gv[4];
      load4<T>(g + i, gv);
      float out[4] = {v[k].x * r * gv[0], v[k].y * r * gv[1], v[k].z * r * gv[2], v[k].w * r * gv[3]};
      store4<TY>(y + o + i, out);
      if (x_copy) *reinterpret_cast<float4 *>(x_copy + o + i) = v[k];
    }
  }
  if (r_out && threadIdx.x == 0) r_out[row] = r;
}

// dx = r g dy - x r^3 mean(x g dy) (+ dh_in); written fp32 (dh_out) and in the
// working dtype (dh_t, the next GEMM's operand).
template <typename T, typename TY, int NV>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const float *dy, const float *x, const float *r,
                                                          const T *g, const float *dh_in, float *dh_out, TY *dh_t,
                                                          int n, int d) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const long o = (long)row * d;
  float4 xa[NV], gy[NV];
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int i = (k * 256 + threadIdx.x) * 4;
    if (i < d) {
      xa[k] = *reinterpret_cast<const float4 *>(x + o + i);
      const float4 b = *reinterpret_cast<const float4 *>(dy + o + i);
      float gv[4];
      load4<T>(g + i, gv);
      gy[k] = make_float4(b.x * gv[0], b.y * gv[1], b.z * gv[2], b.w * gv[3]);
    } else {
      xa[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      gy[k] = xa[k];
    }
    dot += xa[k].x * gy[k].x + xa[k].y * gy[k].y + xa[k].z * gy[k].z + xa[k].w * gy[k].w;
  }
  dot = block_sum4(dot, red);
  const float rr = r[row];
  const float c = rr * rr * rr * dot / (float)d;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int i = (k * 256 + threadIdx.x) * 4;
    if (i < d) {
      float v[4] = {rr * gy[k].x - xa[k].x * c, rr * gy[k].y - xa[k].y * c, rr * gy[k].z - xa[k].z * c,
                    rr * gy[k].w - xa[k].w * c};
      if (dh_in) {
        const float4 p = *reinterpret_cast<const float4 *>(dh_in + o + i);
        v[0] += p.x; v[1] += p.y; v[2] += p.z; v[3] += p.w;
      }
      store4<float>(dh_out + o + i, v);
      store4<TY>(dh_t + o + i, v);
    }
  }
}

// ----------------------------------------------------------------- QK-norm + rotary (+ ring write)
// grid (ceil(n/32), H): 32 tokens of one head per block.  Each wave handles 8 tokens, four at
// a time: 16-lane group g takes one token, and lane j < hd/8 of the group the elements
// 4j..4j+3 and their rotary partners 4j+hd/2.. (16-byte loads and 8-byte stores; the
// norms reduce over the group).
template <typename T, typename TF>
__global__ __launch_bounds__(256) void qk_rope_fwd_kernel(const RopeArgs a) {
  extern __shared__ float sm[];  // [3][hd][33]: Vt, Kt, Qt tiles
  const int hd = a.hd, half = hd / 2, h = blockIdx.y, t0 = blockIdx.x * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, i0 = (lane & 15) * 4;
  const int pos0 = *a.pos0;
  const float *qkv = reinterpret_cast<const float *>(a.qkv);
  float *sV = sm, *sK = sm + hd * 33, *sQ = sm + 2 * hd * 33;
  const bool act = i0 < half;
  float gq[2][4] = {}, gk[2][4] = {};
  if (act) {
    load4<T>(reinterpret_cast<const T *>(a.gq) + i0, gq[0]);
    load4<T>(reinterpret_cast<const T *>(a.gq) + i0 + half, gq[1]);
    load4<T>(reinterpret_cast<const T *>(a.gk) + i0, gk[0]);
    load4<T>(reinterpret_cast<const T *>(a.gk) + i0 + half, gk[1]);
  }
  // all loads of the wave's 8 tokens are issued first (one memory round trip)
  float4 ld[2][6];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int t = t0 + wave * 8 + it * 4 + grp;
    const bool ok = act && t < a.n;
    const float *base = qkv + (long)t * 3 * a.d + h * hd + i0;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      ld[it][2 * c] = ok ? *reinterpret_cast<const float4 *>(base + c * a.d) : make_float4(0.f, 0.f, 0.f, 0.f);
      ld[it][2 * c + 1] =
          ok ? *reinterpret_cast<const float4 *>(base + c * a.d + half) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int tl = wave * 8 + it * 4 + grp, t = t0 + tl;
    const bool ok = act && t < a.n;
    const float q[2][4] = {{ld[it][0].x, ld[it][0].y, ld[it][0].z, ld[it][0].w},
                           {ld[it][1].x, ld[it][1].y, ld[it][1].z, ld[it][1].w}};
    const float k[2][4] = {{ld[it][2].x, ld[it][2].y, ld[it][2].z, ld[it][2].w},
                           {ld[it][3].x, ld[it][3].y, ld[it][3].z, ld[it][3].w}};
    const float v[2][4] = {{ld[it][4].x, ld[it][4].y, ld[it][4].z, ld[it][4].w},
                           {ld[it][5].x, ld[it][5].y, ld[it][5].z, ld[it][5].w}};
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sq += q[x][e] * q[x][e];
        sk += k[x][e] * k[x][e];
      }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {  // within the 16-lane group
      sq += __shfl_xor(sq, o, 64);
      sk += __shfl_xor(sk, o, 64);
    }
    const float rq = 1.f / sqrtf(sq / (float)hd + a.eps), rk = 1.f / sqrtf(sk / (float)hd + a.eps);
    if (ok) {
      const int p = pos0 + t;
      const float4 *csp = reinterpret_cast<const float4 *>(a.cs + (long)p * half + i0);
      const float4 c01 = csp[0], c23 = csp[1];
      const float cs_c[4] = {c01.x, c01.z, c23.x, c23.z}, cs_s[4] = {c01.y, c01.w, c23.y, c23.w};
      float q1[4], q2[4], k1[4], k2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float qa = q[0][e] * rq * gq[0][e], qb = q[1][e] * rq * gq[1][e];
        const float ka = k[0][e] * rk * gk[0][e], kb = k[1][e] * rk * gk[1][e];
        q1[e] = qa * cs_c[e] - qb * cs_s[e];
        q2[e] = qa * cs_s[e] + qb * cs_c[e];
        k1[e] = ka * cs_c[e] - kb * cs_s[e];
        k2[e] = ka * cs_s[e] + kb * cs_c[e];
      }
      TF *qh = reinterpret_cast<TF *>(a.qh) + (long)t * a.d + h * hd + i0;
      store4<TF>(qh, q1);
      store4<TF>(qh + half, q2);
      if (a.qhb) {
        T *qb = reinterpret_cast<T *>(a.qhb) + (long)t * a.d + h * hd + i0;
        store4<T>(qb, q1);
        store4<T>(qb + half, q2);
      }
      const long slot = p % a.R;
      TF *kr = reinterpret_cast<TF *>(a.K) + ((long)h * a.R + slot) * hd + i0;
      store4<TF>(kr, k1);
      store4<TF>(kr + half, k2);
      if (a.Kb) {
        T *kb = reinterpret_cast<T *>(a.Kb) + ((long)h * a.R + slot) * hd + i0;
        store4<T>(kb, k1);
        store4<T>(kb + half, k2);
      }
      if (a.V) {
        T *vr = reinterpret_cast<T *>(a.V) + ((long)h * a.R + slot) * hd + i0;
        store4<T>(vr, v[0]);
        store4<T>(vr + half, v[1]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sV[(i0 + e) * 33 + tl] = v[0][e];
        sV[(i0 + half + e) * 33 + tl] = v[1][e];
        sK[(i0 + e) * 33 + tl] = k1[e];
        sK[(i0 + half + e) * 33 + tl] = k2[e];
        sQ[(i0 + e) * 33 + tl] = q1[e];
        sQ[(i0 + half + e) * 33 + tl] = q2[e];
      }
    }
  }
  __syncthreads();
  const int cnt = min(32, a.n - t0);
  for (int idx = threadIdx.x; idx < hd * 32; idx += 256) {
    const int dim = idx / 32, tl = idx % 32;
    if (tl >= cnt) continue;
    const int t = t0 + tl;
    const long slot = (pos0 + t) % a.R;
    reinterpret_cast<TF *>(a.Vt)[((long)h * hd + dim) * a.R + slot] = from_f<TF>(sV[dim * 33 + tl]);
    if (a.Kt) reinterpret_cast<T *>(a.Kt)[((long)h * hd + dim) * a.R + slot] = from_f<T>(sK[dim * 33 + tl]);
    if (a.qht) reinterpret_cast<T *>(a.qht)[((long)h * hd + dim) * a.ldt + t] = from_f<T>(sQ[dim * 33 + tl]);
  }
}

// grid (ceil(n/16), H): one 16-lane group per (token, head), lanes as in the forward.
template <typename T>
__global__ __launch_bounds__(256) void qk_rope_bwd_kernel(const RopeArgs a) {
  const int hd = a.hd, half = hd / 2, h = blockIdx.y;
  const int lane = threadIdx.x & 63, i0 = (lane & 15) * 4;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool ok = i0 < half && t < a.n;
  const float *qkv = reinterpret_cast<const float *>(a.qkv);
  const long base = (long)t * 3 * a.d + h * hd + i0;
  const long ob = (long)t * a.d + h * hd + i0;
  float q[2][4] = {}, k[2][4] = {}, gyq[2][4] = {}, gyk[2][4] = {};
  float sq = 0.f, sk = 0.f, dotq = 0.f, dotk = 0.f;
  if (ok) {
    float gq[2][4], gk[2][4], dqh[2][4], dkh[2][4];
    load4<float>(qkv + base, q[0]);
    load4<float>(qkv + base + half, q[1]);
    load4<float>(qkv + base + a.d, k[0]);
    load4<float>(qkv + base + a.d + half, k[1]);
    load4<float>(a.dqh + ob, dqh[0]);
    load4<float>(a.dqh + ob + half, dqh[1]);
    load4<float>(a.dkh + ob, dkh[0]);
    load4<float>(a.dkh + ob + half, dkh[1]);
    load4<T>(reinterpret_cast<const T *>(a.gq) + i0, gq[0]);
    load4<T>(reinterpret_cast<const T *>(a.gq) + i0 + half, gq[1]);
    load4<T>(reinterpret_cast<const T *>(a.gk) + i0, gk[0]);
    load4<T>(reinterpret_cast<const T *>(a.gk) + i0 + half, gk[1]);
    const float4 *csp = reinterpret_cast<const float4 *>(a.cs + (long)(*a.pos0 + t) * half + i0);
    const float4 c01 = csp[0], c23 = csp[1];
    const float cs_c[4] = {c01.x, c01.z, c23.x, c23.z}, cs_s[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // transpose of the rotation, then the gain
      gyq[0][e] = (dqh[0][e] * cs_c[e] + dqh[1][e] * cs_s[e]) * gq[0][e];
      gyq[1][e] = (-dqh[0][e] * cs_s[e] + dqh[1][e] * cs_c[e]) * gq[1][e];
      gyk[0][e] = (dkh[0][e] * cs_c[e] + dkh[1][e] * cs_s[e]) * gk[0][e];
      gyk[1][e] = (-dkh[0][e] * cs_s[e] + dkh[1][e] * cs_c[e]) * gk[1][e];
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sq += q[x][e] * q[x][e];
        sk += k[x][e] * k[x][e];
        dotq += q[x][e] * gyq[x][e];
        dotk += k[x][e] * gyk[x][e];
      }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {  // within the 16-lane group
    sq += __shfl_xor(sq, o, 64);
    sk += __shfl_xor(sk, o, 64);
    dotq += __shfl_xor(dotq, o, 64);
    dotk += __shfl_xor(dotk, o, 64);
  }
  if (ok) {
    const float rq = 1.f / sqrtf(sq / (float)hd + a.eps), rk = 1.f / sqrtf(sk / (float)hd + a.eps);
    const float cq = rq * rq * rq * dotq / (float)hd, ck = rk * rk * rk * dotk / (float)hd;
    T *o = reinterpret_cast<T *>(a.dqkv) + base;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      float oq[4], ok4[4], ov[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        oq[e] = rq * gyq[x][e] - q[x][e] * cq;
        ok4[e] = rk * gyk[x][e] - k[x][e] * ck;
      }
      load4<float>(a.dv + ob + x * half, ov);
      store4<T>(o + x * half, oq);
      store4<T>(o + a.d + x * half, ok4);
      store4<T>(o + 2 * a.d + x * half, ov);
    }
  }
}

// ----------------------------------------------------------------- attention backward pre-pass
template <typename T, typename TO>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(const T *dO, const TO *O, float *Dq, T *dOt, int n, int d,
                                                           int hd, int ldl, int ldt) {
  extern __shared__ float sm[];  // [hd][65]
  const int h = blockIdx.y, t0 = blockIdx.x * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // 16-lane group g of wave w takes tokens 16 it + 4 w + g (it = 0..3); lane j < hd/8 of the
  // group the elements 8j..8j+7
  const int grp = lane >> 4, i0 = (lane & 15) * 8;
  const bool act = i0 < hd;
  float a[4][8], o[4][8];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = t0 + it * 16 + wave * 4 + grp;
    const bool ok = act && t < n;
    const long off = (long)t * d + h * hd + i0;
    if (ok) {
      load4<T>(dO + off, a[it]);
      load4<T>(dO + off + 4, a[it] + 4);
      load4<TO>(O + off, o[it]);
      load4<TO>(O + off + 4, o[it] + 4);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[it][e] = o[it][e] = 0.f;
    }
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int tl = it * 16 + wave * 4 + grp, t = t0 + tl;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += a[it][e] * o[it][e];
#pragma unroll
    for (int m = 8; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);  // within the 16-lane group
    if (t < n) {
      if ((lane & 15) == 0) Dq[(long)h * ldl + t] = acc;
      if (act) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm[(i0 + e) * 65 + tl] = a[it][e];
      }
    }
  }
  __syncthreads();
  const int cnt = min(64, n - t0);
  for (int idx = threadIdx.x; idx < hd * 64; idx += 256) {
    const int dim = idx / 64, tl = idx % 64;
    if (tl < cnt) dOt[((long)h * hd + dim) * ldt + t0 + tl] = from_f<T>(sm[dim * 65 + tl]);
  }
}

// ----------------------------------------------------------------- SwiGLU backward
template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const T *GU, const T *dh, T *dGU, int n, int units, long ld_gu,
                                                         long ld_h) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = units / 4;
  if (idx >= (long)n * per_row) return;
  const int m = idx / per_row, u = (idx % per_row) * 4;
  const int blk = u / 16, t = u % 16;
  const long gcol = (long)m * ld_gu + blk * 32 + t, ucol = gcol + 16;
  float g[4], up[4], dy[4], dg[4], du[4];
  load4<T>(GU + gcol, g);
  load4<T>(GU + ucol, up);
  load4<T>(dh + (long)m * ld_h + u, dy);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float s = 1.f / (1.f + __expf(-g[r]));
    const float silu = g[r] * s;
    dg[r] = dy[r] * up[r] * s * (1.f + g[r] * (1.f - s));
    du[r] = dy[r] * silu;
  }
  store4<T>(dGU + gcol, dg);
  store4<T>(dGU + ucol, du);
}

// ----------------------------------------------------------------- cross-entropy reduce
// (mx, s) <- the pair for the union of the terms of (mx, s) and one partial (x, y): a sum of
// exponentials y e^x held as s e^mx.  Partials with y <= 0 hold no terms.
DEVI void ce_combine(float &mx, float &s, float x, float y) {
  if (y > 0.f) {
    if (x > mx) {
      s = s * __expf(mx - x) + y;
      mx = x;
    } else {
      s += y * __expf(x - mx);
    }
  }
}

__global__ __launch_bounds__(256) void ce_reduce_kernel(const float2 *part, int P, const float *zlab, const int *pos0,
                                                        float *lse, float *losses, int n) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= n) return;
  // one pass, two partials per 16-byte load (P is even), eight loads in flight per lane
  const float4 *pr = reinterpret_cast<const float4 *>(part + (long)m * P);
  const int P2 = P / 2;
  float mx = -INFINITY, s = 0.f;
  for (int i0 = 0; i0 < P2; i0 += 8 * 64) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 64 + lane;
      v[u] = i < P2 ? pr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      ce_combine(mx, s, v[u].x, v[u].y);
      ce_combine(mx, s, v[u].z, v[u].w);
    }
  }
  const float M = wave_max(mx);
  s = wave_sum(s > 0.f ? s * __expf(mx - M) : 0.f);
  if (lane == 0) {
    const float l = M + logf(s);
    lse[m] = l;
    losses[*pos0 + m] = l - zlab[m];
  }
}

// ----------------------------------------------------------------- head softmax shift and gradient
// shift[m] = n_f[m] . W[label of m] + off: the label's logit (in fp32, from the head's own
// operands) plus a margin, the per-row shift of the single-pass head.  One wave per row.
template <typename TA, typename TW>
__global__ __launch_bounds__(256) void head_shift_kernel(const TA *nf, const TW *W, const int *labs, const int *pos0,
                                                         float *shift, int n, int d, float off) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= n) return;
  const long lab = labs[*pos0 + m];
  float acc = 0.f;
  for (int i = lane * 4; i < d; i += 256) {
    float a[4], w[4];
    load4<TA>(nf + (long)m * d + i, a);
    load4<TW>(W + lab * d + i, w);
    acc += a[0] * w[0] + a[1] * w[1] + a[2] * w[2] + a[3] * w[3];
  }
  acc = wave_sum(acc);
  if (lane == 0) shift[m] = acc + off;
}

// dn[m] = alpha (dn[m] exp(shift[m] - lse[m]) - W[label of m]): the unnormalised softmax
// product over the vocabulary divided by its sum (sum = exp(lse - shift)), minus the
// label's row.  One work-group per row.
template <typename TW>
__global__ __launch_bounds__(256) void head_grad_finish_kernel(float *dn, const float *shift, const float *lse,
                                                               const TW *W, const int *labs, const int *pos0, int d,
                                                               float alpha) {
  const int m = blockIdx.x;
  const long lab = labs[*pos0 + m];
  const float sc = __expf(shift[m] - lse[m]);
  for (int i = threadIdx.x * 4; i < d; i += 1024) {
    float w[4];
    load4<TW>(W + lab * d + i, w);
    float4 *p = reinterpret_cast<float4 *>(dn + (long)m * d + i);
    const float4 v = *p;
    *p = make_float4(alpha * (v.x * sc - w[0]), alpha * (v.y * sc - w[1]), alpha * (v.z * sc - w[2]),
                     alpha * (v.w * sc - w[3]));
  }
}

__global__ void rope_table_kernel(float2 *cs, long max_pos, int hd, double theta) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int half = hd / 2;
  if (idx >= max_pos * half) return;
  const long p = idx / half;
  const int i = idx % half;
  const double inv = pow(theta, -2.0 * (double)i / (double)hd);
  const double ang = (double)p * inv;
  cs[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

template <typename T>
__global__ void convert_rows_kernel(const float *src, long ld_src, T *dst, long ld_dst, T *lo, long ld_lo, int rows,
                                    int cols, float scale) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)rows * cols) return;
  const int r = idx / cols, c = idx % cols;
  const float x = src[(long)r * ld_src + c] * scale;
  const T hi = from_f<T>(x);
  dst[(long)r * ld_dst + c] = hi;
  if (lo) lo[(long)r * ld_lo + c] = from_f<T>(x - to_f(hi));
}
template <typename T>
__global__ void copy_rows_kernel(const T *src, long ld_src, T *dst, long ld_dst, int rows, int cols) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)rows * cols) return;
  const int r = idx / cols, c = idx % cols;
  dst[(long)r * ld_dst + c] = src[(long)r * ld_src + c];
}

// dst[c * ldd + r] = r < R ? src[r * lds + c] : 0   for r < Rpad, c < C
// (64 x 64 tiles through LDS; both global sides coalesced).
template <typename S, typename D>
__global__ __launch_bounds__(256) void transpose_kernel(const S *src, long lds, D *dst, long ldd, int R, int Rpad,
                                                        int C) {
  __shared__ float tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? to_f(src[(long)r * lds + c]) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < Rpad) dst[(long)c * ldd + r] = from_f<D>(tile[tx][i]);
  }
}

// The same with 4-element vectors: each thread loads 4 consecutive columns of 4 rows
// and stores 4 consecutive rows of 4 columns (needs lds, ldd multiples of 4 and
// 4-element-aligned bases; partial vectors at the edges go element by element).
template <typename T> struct V4;
template <> struct V4<float> { typedef float4 t; };
template <> struct V4<f16_t> { typedef uint2 t; };
template <> struct V4<bf16_t> { typedef uint2 t; };
template <typename T> DEVI void put4(T *p, const float *v) { store4<T>(p, v); }

template <typename S, typename D>
__global__ __launch_bounds__(256) void transpose4_kernel(const S *src, long lds, D *dst, long ldd, int R, int Rpad,
                                                         int C) {
  __shared__ float tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int q = (threadIdx.x & 15) * 4, w = threadIdx.x >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = w + 16 * i, r = r0 + rl, c = c0 + q;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (r < R) {
      if (c + 3 < C) {
        load4<S>(src + (long)r * lds + c, v);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (c + j < C) v[j] = to_f(src[(long)r * lds + c + j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) tile[rl][q + j] = v[j];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cl = w + 16 * i, c = c0 + cl, r = r0 + q;
    if (c >= C) continue;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = tile[q + j][cl];
    if (r + 3 < Rpad) {
      put4<D>(dst + (long)c * ldd + r, v);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (r + j < Rpad) dst[(long)c * ldd + r + j] = from_f<D>(v[j]);
    }
  }
}

__global__ void bf16_to_f16_kernel(const bf16_t *src, long lds, f16_t *dst, long ldd, int rows, int cols,
                                   float scale) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)rows * cols) return;
  const int r = idx / cols, c = idx % cols;
  dst[(long)r * ldd + c] = from_f<f16_t>(to_f(src[(long)r * lds + c]) * scale);
}

// *out = max(*out, bits of max |x|) over x[r * ld + c], r < rows, c < cols
// (non-negative floats order like their bit patterns; a NaN compares highest).
// out = max(out, largest Euclidean norm of a row) as float bits (norms are non-negative, so
// their bit patterns order like the values; NaN rows give NaN bits, which compare above).
template <typename T>
__global__ __launch_bounds__(256) void rownorm_max_kernel(const T *x, long ld, int rows, int cols, unsigned *out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float s = 0.f;
  for (int i = lane; i < cols; i += 64) {
    const float v = to_f(x[(long)r * ld + i]);
    s += v * v;
  }
  s = wave_sum(s);
  if (lane == 0) atomicMax(out, __float_as_uint(sqrtf(s)));
}

template <typename T>
__global__ void absmax_kernel(const T *x, long ld, int rows, int cols, unsigned *out) {
  float m = 0.f;
  const long tot = (long)rows * cols;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < tot; i += (long)gridDim.x * 256) {
    const float v = fabsf(to_f(x[(i / cols) * ld + i % cols]));
    m = (v > m || v != v) ? v : m;
  }
  atomicMax(out, __float_as_uint(m));
}

__global__ void set_int_kernel(int *p, int v) { *p = v; }
__global__ void add_int_kernel(int *p, int v) { *p += v; }
__global__ void zero_kernel(uint32_t *p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256) p[i] = 0;
}
__global__ void finite_check_kernel(const float *x, long n, int *flag) {
  int bad = 0;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) bad |= !isfinite(x[i]);
  if (bad) atomicOr(flag, 1);
}

// Greedy next token of the last position: the largest logit over the vocabulary
// tiles' partials (lowest id on ties), written to tok[p + 1] with the loss
// lse - max at losses[p], p = *pos0 + n - 1.
__global__ __launch_bounds__(64) void decode_pick_kernel(const float2 *part, const int *part_arg, int P,
                                                         const float *lse, const int *pos0, int n, int *tok,
                                                         float *losses) {
  const int lane = threadIdx.x;
  const int row = n - 1;
  float mx = -INFINITY;
  int ai = 0x7fffffff;
  for (int i = lane; i < P; i += 64) {
    const float2 v = part[(long)row * P + i];
    if (!(v.y > 0.f)) continue;  // tile half with no column
    const int a = part_arg[(long)row * P + i];
    if (v.x > mx || (v.x == mx && a < ai)) {
      mx = v.x;
      ai = a;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(mx, o);
    const int a2 = __shfl_xor(ai, o);
    if (m2 > mx || (m2 == mx && a2 < ai)) {
      mx = m2;
      ai = a2;
    }
  }
  if (lane == 0) {
    const int p = *pos0 + row;
    tok[p + 1] = ai;
    losses[p] = lse[row] - mx;
  }
}

// Rows of a batched chunk: row r = s * n + m is position *pos0 + m of sequence s.
__global__ void lead_rows_kernel(const float4 *src, const int *src_n, int G, const int *pos0, float4 *dst, int n,
                                 int d4, int B) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)B * n * d4) return;
  const int c = idx % d4;
  const long r = idx / d4;
  const int s = r / n, t = r % n;
  dst[r * d4 + c] = src[((long)s * *src_n + *pos0 % G + t) * d4 + c];
}
__global__ void gather_chunk_ids_kernel(const int *tok, long ld_tok, const int *pos0, int n, int B, int *ids,
                                        int *labs) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= B * n) return;
  const int s = r / n, m = r % n;
  const long i = (long)s * ld_tok + *pos0 + m;
  ids[r] = tok[i];
  labs[r] = tok[i + 1];
}
__global__ void scatter_chunk_losses_kernel(const float *closs, float *losses, long ld_loss, const int *pos0, int n,
                                            int B) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= B * n) return;
  const int s = r / n, m = r % n;
  losses[(long)s * ld_loss + *pos0 + m] = closs[r];
}

inline unsigned blocks_for(long n, int per = 256) { return (unsigned)((n + per - 1) / per); }

}  // namespace

#define DT_DISPATCH(dtype, KERNEL, ...)                                   \
  do {                                                                    \
    if ((dtype) == 1) {                                                   \
      KERNEL(bf16_t, __VA_ARGS__);                                        \
    } else {                                                              \
      KERNEL(float, __VA_ARGS__);                                         \
    }                                                                     \
  } while (0)

hipError_t embed_launch(int dtype, const void *E, const int *tok, const int *pos0, float *h, int n, int d,
                        hipStream_t st) {
  if (n <= 0) return hipSuccess;
#define K_(T, ...) hipLaunchKernelGGL(embed_kernel<T>, dim3(n), dim3(256), 0, st, (const T *)E, tok, pos0, h, d)
  DT_DISPATCH(dtype, K_, 0);
#undef K_
  return hipGetLastError();
}

// Row width classes (float4 per thread of a 256-thread block): d <= 1024 NV.
#define NV_DISPATCH(d, CALL)                   \
  if ((d) <= 1024) { CALL(1); }                \
  else if ((d) <= 2048) { CALL(2); }           \
  else if ((d) <= 3072) { CALL(3); }           \
  else if ((d) <= 4096) { CALL(4); }           \
  else if ((d) <= 8192) { CALL(8); }           \
  else return hipErrorInvalidValue;

hipError_t rmsnorm_fwd_launch(int dtype, float *x, const void *g, void *y, float *r_out, float *x_copy, int n, int d,
                              float eps, hipStream_t st, bool y_f16, ResidualPartials red) {
  if (y_f16 && dtype != 1) return hipErrorInvalidValue;
  if (n <= 0) return hipSuccess;
#define CALL_(NV)                                                                                                  \
  if (dtype == 1 && y_f16)                                                                                         \
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<bf16_t, f16_t, NV>), dim3(n), dim3(256), 0, st, x,      \
                       (const bf16_t *)g, (f16_t *)y, r_out, x_copy, n, d, eps, red);                                   \
  else if (dtype == 1)                                                                                             \
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<bf16_t, bf16_t, NV>), dim3(n), dim3(256), 0, st, x,     \
                       (const bf16_t *)g, (bf16_t *)y, r_out, x_copy, n, d, eps, red);                                  \
  else                                                                                                             \
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<float, float, NV>), dim3(n), dim3(256), 0, st, x,       \
                       (const float *)g, (float *)y, r_out, x_copy, n, d, eps, red);
  NV_DISPATCH(d, CALL_)
#undef CALL_
  return hipGetLastError();
}

hipError_t rmsnorm_bwd_launch(int dtype, const float *dy, const float *x, const float *r, const void *g,
                              const float *dh_in, float *dh_out, void *dh_t, int n, int d, hipStream_t st,
                              bool t_f16) {
  if (n <= 0) return hipSuccess;
  if (t_f16 && dtype != 1) return hipErrorInvalidValue;
#define CALL_(NV)                                                                                                  \
  if (t_f16)                                                                                                       \
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<bf16_t, f16_t, NV>), dim3(n), dim3(256), 0, st, dy, x,  \
                       r, (const bf16_t *)g, dh_in, dh_out, (f16_t *)dh_t, n, d);                                  \
  else if (dtype == 1)                                                                                             \
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<bf16_t, bf16_t, NV>), dim3(n), dim3(256), 0, st, dy, x, \
                       r, (const bf16_t *)g, dh_in, dh_out, (bf16_t *)dh_t, n, d);                                 \
  else                                                                                                             \
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<float, float, NV>), dim3(n), dim3(256), 0, st, dy, x,   \
                       r, (const float *)g, dh_in, dh_out, (float *)dh_t, n, d);
  NV_DISPATCH(d, CALL_)
#undef CALL_
  return hipGetLastError();
}

hipError_t qk_rope_fwd_launch(int dtype, const RopeArgs &a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  size_t shm = (size_t)3 * a.hd * 33 * sizeof(float);
  dim3 grid(blocks_for(a.n, 32), a.H);
#define K_(T, ...)                                                                     \
  if (a.fwd_f16)                                                                       \
    hipLaunchKernelGGL((qk_rope_fwd_kernel<T, f16_t>), grid, dim3(256), shm, st, a);  \
  else                                                                                 \
    hipLaunchKernelGGL((qk_rope_fwd_kernel<T, T>), grid, dim3(256), shm, st, a)
  DT_DISPATCH(dtype, K_, 0);
#undef K_
  return hipGetLastError();
}

hipError_t qk_rope_bwd_launch(int dtype, const RopeArgs &a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  dim3 grid(blocks_for(a.n, 16), a.H);
#define K_(T, ...) hipLaunchKernelGGL(qk_rope_bwd_kernel<T>, grid, dim3(256), 0, st, a)
  DT_DISPATCH(dtype, K_, 0);
#undef K_
  return hipGetLastError();
}

hipError_t attn_bwd_pre_launch(int dtype, const void *dO, const void *O, float *Dq, void *dOt, int n, int d, int H,
                               int hd, int ldl, int ldt, hipStream_t st, bool o_f16) {
  if (n <= 0) return hipSuccess;
  size_t shm = (size_t)hd * 65 * sizeof(float);
  dim3 grid(blocks_for(n, 64), H);
#define K_(T, ...)                                                                                                \
  if (o_f16)                                                                                                      \
    hipLaunchKernelGGL((attn_bwd_pre_kernel<T, f16_t>), grid, dim3(256), shm, st, (const T *)dO, (const f16_t *)O, \
                       Dq, (T *)dOt, n, d, hd, ldl, ldt);                                                         \
  else                                                                                                            \
    hipLaunchKernelGGL((attn_bwd_pre_kernel<T, T>), grid, dim3(256), shm, st, (const T *)dO, (const T *)O, Dq,     \
                       (T *)dOt, n, d, hd, ldl, ldt)
  DT_DISPATCH(dtype, K_, 0);
#undef K_
  return hipGetLastError();
}

hipError_t swiglu_bwd_launch(int dtype, const void *GU, const void *dhmid, void *dGU, int n, int units, long ld_gu,
                             long ld_h, hipStream_t st, bool f16) {
  if (n <= 0) return hipSuccess;
  long tot = (long)n * (units / 4);
  if (f16) {
    if (dtype != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(swiglu_bwd_kernel<f16_t>, dim3(blocks_for(tot)), dim3(256), 0, st, (const f16_t *)GU,
                       (const f16_t *)dhmid, (f16_t *)dGU, n, units, ld_gu, ld_h);
    return hipGetLastError();
  }
#define K_(T, ...)                                                                                                  \
  hipLaunchKernelGGL(swiglu_bwd_kernel<T>, dim3(blocks_for(tot)), dim3(256), 0, st, (const T *)GU, (const T *)dhmid, \
                     (T *)dGU, n, units, ld_gu, ld_h)
  DT_DISPATCH(dtype, K_, 0);
#undef K_
  return hipGetLastError();
}

hipError_t gather_chunk_ids_launch(const int *tok, long ld_tok, const int *pos0, int n, int B, int *ids, int *labs,
                                   hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_chunk_ids_kernel, dim3(blocks_for((long)B * n)), dim3(256), 0, st, tok, ld_tok, pos0, n, B,
                     ids, labs);
  return hipGetLastError();
}
hipError_t lead_rows_launch(const float *src, const int *src_n, int G, const int *pos0, float *dst, int n, int d,
                            int B, hipStream_t st) {
  if (n <= 0 || d % 4 != 0) return n <= 0 ? hipSuccess : hipErrorInvalidValue;
  const long tot = (long)B * n * (d / 4);
  hipLaunchKernelGGL(lead_rows_kernel, dim3(blocks_for(tot)), dim3(256), 0, st, (const float4 *)src, src_n, G, pos0,
                     (float4 *)dst, n, d / 4, B);
  return hipGetLastError();
}
hipError_t scatter_chunk_losses_launch(const float *closs, float *losses, long ld_loss, const int *pos0, int n, int B,
                                       hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_chunk_losses_kernel, dim3(blocks_for((long)B * n)), dim3(256), 0, st, closs, losses,
                     ld_loss, pos0, n, B);
  return hipGetLastError();
}

hipError_t decode_pick_launch(const float2 *part, const int *part_arg, int P, const float *lse, const int *pos0, int n,
                              int *tok, float *losses, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_pick_kernel, dim3(1), dim3(64), 0, st, part, part_arg, P, lse, pos0, n, tok, losses);
  return hipGetLastError();
}

hipError_t head_shift_launch(int dtype, bool f16, const void *nf, const void *W, const int *labs, const int *pos0,
                             float *shift, int n, int d, float off, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (d % 4 != 0) return hipErrorInvalidValue;
  const dim3 grid((n + 3) / 4);
  if (f16) {
    if (dtype != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((head_shift_kernel<f16_t, f16_t>), grid, dim3(256), 0, st, (const f16_t *)nf, (const f16_t *)W,
                       labs, pos0, shift, n, d, off);
  } else if (dtype == 0) {
    hipLaunchKernelGGL((head_shift_kernel<float, float>), grid, dim3(256), 0, st, (const float *)nf, (const float *)W,
                       labs, pos0, shift, n, d, off);
  } else {
    hipLaunchKernelGGL((head_shift_kernel<bf16_t, bf16_t>), grid, dim3(256), 0, st, (const bf16_t *)nf,
                       (const bf16_t *)W, labs, pos0, shift, n, d, off);
  }
  return hipGetLastError();
}

hipError_t head_grad_finish_launch(int dtype, bool f16, float *dn, const float *shift, const float *lse, const void *W,
                                   const int *labs, const int *pos0, int n, int d, float alpha, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (d % 4 != 0) return hipErrorInvalidValue;
  if (f16) {
    if (dtype != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(head_grad_finish_kernel<f16_t>, dim3(n), dim3(256), 0, st, dn, shift, lse, (const f16_t *)W, labs,
                       pos0, d, alpha);
  } else if (dtype == 0) {
    hipLaunchKernelGGL(head_grad_finish_kernel<float>, dim3(n), dim3(256), 0, st, dn, shift, lse, (const float *)W, labs,
                       pos0, d, alpha);
  } else {
    hipLaunchKernelGGL(head_grad_finish_kernel<bf16_t>, dim3(n), dim3(256), 0, st, dn, shift, lse, (const bf16_t *)W,
                       labs, pos0, d, alpha);
  }
  return hipGetLastError();
}

hipError_t ce_reduce_launch(const float2 *part, int P, const float *zlab, const int *pos0, float *lse, float *losses,
                            int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (P % 2 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ce_reduce_kernel, dim3((n + 3) / 4), dim3(256), 0, st, part, P, zlab, pos0, lse, losses, n);
  return hipGetLastError();
}

hipError_t rope_table_launch(float2 *cs, long max_pos, int hd, double theta, hipStream_t st) {
  long tot = max_pos * (hd / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks_for(tot)), dim3(256), 0, st, cs, max_pos, hd, theta);
  return hipGetLastError();
}

hipError_t convert_rows_launch(int dtype, const float *src, long ld_src, void *dst, long ld_dst, int rows, int cols,
                               hipStream_t st, void *lo, long ld_lo, float scale) {
  long tot = (long)rows * cols;
  if (tot <= 0) return hipSuccess;
  if (dtype == 2) {
    hipLaunchKernelGGL(convert_rows_kernel<f16_t>, dim3(blocks_for(tot)), dim3(256), 0, st, src, ld_src, (f16_t *)dst,
                       ld_dst, (f16_t *)lo, ld_lo, rows, cols, scale);
    return hipGetLastError();
  }
#define K_(T, ...)                                                                                               \
  hipLaunchKernelGGL(convert_rows_kernel<T>, dim3(blocks_for(tot)), dim3(256), 0, st, src, ld_src, (T *)dst, ld_dst, \
                     (T *)lo, ld_lo, rows, cols, scale)
  DT_DISPATCH(dtype, K_, 0);
#undef K_
  return hipGetLastError();
}

hipError_t copy_rows_launch(int dtype, const void *src, long ld_src, void *dst, long ld_dst, int rows, int cols,
                            hipStream_t st) {
  long tot = (long)rows * cols;
  if (tot <= 0) return hipSuccess;
#define K_(T, ...)                                                                                                   \
  hipLaunchKernelGGL(copy_rows_kernel<T>, dim3(blocks_for(tot)), dim3(256), 0, st, (const T *)src, ld_src, (T *)dst, \
                     ld_dst, rows, cols)
  DT_DISPATCH(dtype, K_, 0);
#undef K_
  return hipGetLastError();
}

template <typename S, typename D>
static void launch_transpose(bool vec, dim3 grid, const void *src, long lds, void *dst, long ldd, int R, int Rpad,
                             int C, hipStream_t st) {
  if (vec)
    hipLaunchKernelGGL((transpose4_kernel<S, D>), grid, dim3(256), 0, st, (const S *)src, lds, (D *)dst, ldd, R,
                       Rpad, C);
  else
    hipLaunchKernelGGL((transpose_kernel<S, D>), grid, dim3(256), 0, st, (const S *)src, lds, (D *)dst, ldd, R,
                       Rpad, C);
}

hipError_t transpose_launch(int dtype, int src_kind, const void *src, long lds, void *dst, long ldd, int R, int Rpad,
                            int C, hipStream_t st, bool dst_f16) {
  if (Rpad <= 0 || C <= 0) return hipSuccess;
  dim3 grid((C + 63) / 64, (Rpad + 63) / 64);
  const size_t ssz = (src_kind == SRC_F32 || dtype == 0) ? 4 : 2, dsz = (dst_f16 || dtype == 1) ? 2 : 4;
  // 4-element vectors need row strides that keep every vector aligned
  const bool vec = lds % 4 == 0 && ldd % 4 == 0 && (uintptr_t)src % (4 * ssz) == 0 && (uintptr_t)dst % (4 * dsz) == 0;
  if (dst_f16) {
    if (dtype != 1) return hipErrorInvalidValue;
    if (src_kind == SRC_F32)
      launch_transpose<float, f16_t>(vec, grid, src, lds, dst, ldd, R, Rpad, C, st);
    else if (src_kind == SRC_F16)
      launch_transpose<f16_t, f16_t>(vec, grid, src, lds, dst, ldd, R, Rpad, C, st);
    else
      launch_transpose<bf16_t, f16_t>(vec, grid, src, lds, dst, ldd, R, Rpad, C, st);
    return hipGetLastError();
  }
  if (dtype == 1) {
    if (src_kind == SRC_F32)
      launch_transpose<float, bf16_t>(vec, grid, src, lds, dst, ldd, R, Rpad, C, st);
    else if (src_kind == SRC_F16)
      launch_transpose<f16_t, bf16_t>(vec, grid, src, lds, dst, ldd, R, Rpad, C, st);
    else
      launch_transpose<bf16_t, bf16_t>(vec, grid, src, lds, dst, ldd, R, Rpad, C, st);
  } else {
    launch_transpose<float, float>(vec, grid, src, lds, dst, ldd, R, Rpad, C, st);
  }
  return hipGetLastError();
}

hipError_t bf16_to_f16_launch(const void *src, long lds, void *dst, long ldd, int rows, int cols, hipStream_t st,
                              float scale) {
  const long tot = (long)rows * cols;
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(bf16_to_f16_kernel, dim3(blocks_for(tot)), dim3(256), 0, st, (const bf16_t *)src, lds,
                     (f16_t *)dst, ldd, rows, cols, scale);
  return hipGetLastError();
}

hipError_t rownorm_max_launch(int dtype, const void *x, long ld, int rows, int cols, unsigned *out, hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4);
#define K_(T, ...) hipLaunchKernelGGL(rownorm_max_kernel<T>, grid, dim3(256), 0, st, (const T *)x, ld, rows, cols, out)
  DT_DISPATCH(dtype, K_, 0);
#undef K_
  return hipGetLastError();
}

hipError_t absmax_launch(int dtype, const void *x, long ld, int rows, int cols, unsigned *out, hipStream_t st) {
  const long tot = (long)rows * cols;
  if (tot <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<long>((tot + 255) / 256, 1024);
#define K_(T, ...) hipLaunchKernelGGL(absmax_kernel<T>, dim3(blocks), dim3(256), 0, st, (const T *)x, ld, rows, cols, out)
  DT_DISPATCH(dtype, K_, 0);
#undef K_
  return hipGetLastError();
}

hipError_t set_int_launch(int *p, int v, hipStream_t st) {
  hipLaunchKernelGGL(set_int_kernel, dim3(1), dim3(1), 0, st, p, v);
  return hipGetLastError();
}
hipError_t add_int_launch(int *p, int v, hipStream_t st) {
  hipLaunchKernelGGL(add_int_kernel, dim3(1), dim3(1), 0, st, p, v);
  return hipGetLastError();
}
hipError_t zero_launch(void *p, size_t bytes, hipStream_t st) {
  size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  unsigned blocks = (unsigned)std::min<size_t>((words + 255) / 256, 8192);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, st, (uint32_t *)p, words);
  return hipGetLastError();
}
hipError_t finite_check_launch(const float *x, long n, int *flag, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  unsigned blocks = (unsigned)std::min<long>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(finite_check_kernel, dim3(blocks), dim3(256), 0, st, x, n, flag);
  return hipGetLastError();
}
