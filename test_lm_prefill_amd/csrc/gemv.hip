// Few-row products for gfx950 (a decode step feeds one token): C[m, n] = sum_k A[m, k] B[n, k]
// for M <= 4 (the kernel handles up to 16 rows; larger row counts stay on the tiled GEMM),
// 16-bit operands, both k-contiguous, fp32 accumulation.  A 128-row GEMM tile with one live
// row would give a d-wide product ~20 work-groups and leave most of the chip idle; here a
// work-group owns only NB output columns and its NW waves split the reduction, so the
// weights stream through hundreds of work-groups at once.
//
// Wave w takes the k range [w K/NW, (w+1) K/NW): per 32-deep step it loads one fragment of B
// per 16-column block straight from memory into registers (lane l: row l % 16,
// k 8 (l / 16) .. +7, 16 bytes) and multiplies it with the step's A fragment (rows >= M
// read as zero) on v_mfma_f32_16x16x32.  The NW partial tiles are summed in wave order
// through LDS and wave 0 applies the epilogue.  Loads go through buffer descriptors, so
// rows and columns outside the operands read as zero.
#include "common.h"
#include "gemm.h"

namespace {



// 16-bit output in the type the caller asked for (fp16 or bf16).
DEVI void put16x4(const GemmArgs &g, void *base, long off, const float *v) {
  if (g.c_f16)
    store4<f16_t>(reinterpret_cast<f16_t *>(base) + off, v);
  else
    store4<bf16_t>(reinterpret_cast<bf16_t *>(base) + off, v);
}

template <typename TI, int EPI, int NB, int NW>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(const GemmArgs g) {
  constexpr int NBB = NB / 16;              // 16-column blocks per work-group
  __shared__ float4 red[NW - 1][NBB][64];   // waves 1..NW-1: partial tiles (block, lane)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int n0 = blockIdx.x * NB;
  const int ka = g.a_kwrap > 0 ? g.a_kwrap : g.K;
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)g.B, (short)0, (uint32_t)(((long)(g.N - 1) * g.ldb + g.K) * 2), BUF_RSRC_W3);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void *)g.A, (short)0, (uint32_t)(((long)(g.M - 1) * g.lda + ka) * 2), BUF_RSRC_W3);
  // per-lane byte offsets (the k position enters through the scalar offset)
  uint32_t ob[NBB];
#pragma unroll
  for (int b = 0; b < NBB; ++b) {
    const int row = n0 + 16 * b + lr;
    ob[b] = row < g.N ? (uint32_t)(((long)row * g.ldb + 8 * lq) * 2) : BUF_OOB;
  }
  const uint32_t oa = lr < g.M ? (uint32_t)(((long)lr * g.lda + 8 * lq) * 2) : BUF_OOB;
  const int kq = g.K / NW, kbeg = wave * kq;
  f32x4_v acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  // eight 32-deep steps per batch: their loads are all in flight before the first product
  constexpr int U = 8;
  for (int k0 = kbeg; k0 < kbeg + kq; k0 += 32 * U) {
    Frag<TI> fa[U], fb[U][NBB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(k0 + 32 * u, kbeg + kq - 32);  // past the range: reload the last step (unused)
      const int kc = g.a_kwrap > 0 ? k % g.a_kwrap : k;  // a 32-deep step never straddles the wrap
      fa[u].v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, oa, kc * 2, 0));
#pragma unroll
      for (int b = 0; b < NBB; ++b)
        fb[u][b].v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, ob[b], k * 2, 0));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + 32 * u < kbeg + kq) {
#pragma unroll
        for (int b = 0; b < NBB; ++b) mma(acc[b], fb[u][b], fa[u]);
      }
  }
  if (wave > 0) {
#pragma unroll
    for (int b = 0; b < NBB; ++b) red[wave - 1][b][lane] = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < NW - 1; ++w)
#pragma unroll
    for (int b = 0; b < NBB; ++b) {
      const float4 p = red[w][b][lane];
      acc[b][0] += p.x; acc[b][1] += p.y; acc[b][2] += p.z; acc[b][3] += p.w;
    }
  // lane holds C[m = lr][n0 + 16 b + 4 lq + r], r = 0..3
  const int m = lr, g4 = 4 * lq;
  if constexpr (EPI == EPI_CE) {
    const int lab = m < g.M ? g.rowi[*g.pos0 + m] : -1;
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < NBB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n0 + 16 * b + g4 + r < g.N) mx = fmaxf(mx, acc[b][r]);
    mx = group4_max(mx);
    if (g.part_arg) {  // lowest column holding the maximum
      int ai = 0x7fffffff;
#pragma unroll
      for (int b = NBB - 1; b >= 0; --b)
#pragma unroll
        for (int r = 3; r >= 0; --r) {
          const int n = n0 + 16 * b + g4 + r;
          if (n < g.N && acc[b][r] == mx) ai = n;
        }
      ai = group4_min_int(ai);
      if (m < g.M && lq == 0) g.part_arg[(long)m * g.part_ld + blockIdx.x] = ai + g.col_off;
    }
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < NBB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 16 * b + g4 + r;
        if (n < g.N) {
          s += fast_exp2((acc[b][r] - mx) * LOG2E_F);
          if (n + g.col_off == lab) g.zlab[m] = acc[b][r];
        }
      }
    s = group4_sum(s);
    if (m < g.M && lq == 0) g.part[(long)m * g.part_ld + blockIdx.x] = make_float2(mx, s);
    return;
  }
  if (m >= g.M) return;
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int b = 0; b < NBB; b += 2) {
      const int nb = n0 + 16 * b;  // gate block start; up block is nb + 16
      if (nb >= g.N) continue;
      float hv[4], gv[4], uv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gv[r] = acc[b][r] * g.acc_scale;
        uv[r] = acc[b + 1][r] * g.acc_scale;
        hv[r] = gv[r] / (1.f + __expf(-gv[r])) * uv[r];
      }
      put16x4(g, g.C, (long)m * g.ldc + (nb >> 1) + g4, hv);
      if (g.C2) {
        put16x4(g, g.C2, (long)m * g.ldc2 + nb + g4, gv);
        put16x4(g, g.C2, (long)m * g.ldc2 + nb + 16 + g4, uv);
      }
    }
    return;
  }
#pragma unroll
  for (int b = 0; b < NBB; ++b) {
    const int n = n0 + 16 * b + g4;
    if (n >= g.N) continue;
    float4 *p = reinterpret_cast<float4 *>(g.Cf + (long)m * g.ldcf + n);
    if constexpr (EPI == EPI_STORE_F32) {
      *p = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    } else {  // EPI_ADD_F32
      const float4 o = *p;
      const float sc = g.acc_scale;
      *p = make_float4(o.x + acc[b][0] * sc, o.y + acc[b][1] * sc, o.z + acc[b][2] * sc, o.w + acc[b][3] * sc);
    }
  }
}

// Wide outputs (N >= 8192) take 64 columns and 4 waves per work-group (enough work-groups,
// longer k ranges per wave); narrow ones 16 columns (32 for SwiGLU's gate/up pairs) and 8
// waves, so that a d-wide product still spreads over ~160 work-groups.  Cross-entropy
// always works on 64-column halves of whole 128-column tiles (both halves of every tile
// are written).
template <typename TI, int EPI> hipError_t launch_e(const GemmArgs &g, hipStream_t st) {
  if (EPI == EPI_CE || g.N >= 8192) {
    const int blocks = 2 * ((g.N + 127) / 128);
    hipLaunchKernelGGL((gemv_kernel<TI, EPI, 64, 4>), dim3(blocks), dim3(256), 0, st, g);
  } else {
    constexpr int NB = EPI == EPI_SWIGLU ? 32 : 16;
    hipLaunchKernelGGL((gemv_kernel<TI, EPI, NB, 8>), dim3((g.N + NB - 1) / NB), dim3(512), 0, st, g);
  }
  return hipGetLastError();
}

template <typename TI> hipError_t launch_t(int epi, const GemmArgs &g, hipStream_t st) {
  switch (epi) {
    case EPI_STORE_F32: return launch_e<TI, EPI_STORE_F32>(g, st);
    case EPI_ADD_F32: return launch_e<TI, EPI_ADD_F32>(g, st);
    case EPI_SWIGLU: return launch_e<TI, EPI_SWIGLU>(g, st);
    case EPI_CE: return launch_e<TI, EPI_CE>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool gemv_ok(int dtype, bool a_kc, bool b_kc, int epi, const GemmArgs &g) {
  const int nw = (epi == EPI_CE || g.N >= 8192) ? 4 : 8;
  return (dtype == 1 || dtype == 2) && a_kc && b_kc && g.M >= 1 && g.M <= 4 && g.K % (32 * nw) == 0 &&
         g.lda % 8 == 0 && g.ldb % 8 == 0 && g.a_kwrap % 32 == 0 &&
         (epi == EPI_STORE_F32 || epi == EPI_ADD_F32 || epi == EPI_SWIGLU || epi == EPI_CE) &&
         (epi != EPI_SWIGLU || g.N % 32 == 0) &&
         // the vocabulary-wide product gives the tiled GEMM enough work-groups, and it
         // streams them faster
         g.N <= 32768;
}

hipError_t gemv_launch(bool f16, int epi, const GemmArgs &g, hipStream_t st) {
  return f16 ? launch_t<f16_t>(epi, g, st) : launch_t<bf16_t>(epi, g, st);
}
