// MFMA GEMM for gfx950 with fused epilogues.
//
// Tile 128 x 128 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave owns a
// 64 x 64 sub-tile computed as 4 x 4 16x16 MFMA tiles.  Operands are staged in
// LDS with the reduction dimension contiguous (an operand stored with its M/N
// dimension contiguous is transposed on the way in, 4 (bf16) or 8 (fp32)
// reduction rows at a time in registers), double-buffered with a register
// prefetch of the next tile, one barrier per 64-deep step.
//
// The MFMA "A" input is taken from B (rows n) and the "B" input from A (rows
// m), so each lane ends with 4 consecutive output columns of one output row,
// which lets epilogues store 4-wide vectors.
//
// Work-groups are mapped to tiles XCD by XCD: the hardware deals consecutive
// work-group ids round-robin to the 8 XCDs, so work-group i runs tile
// offset(i % 8) + i / 8, giving every XCD a contiguous run of tiles in
// m-fastest order; the tiles sharing one block of B (the weights) then sit on
// one XCD and share its L2.
#include <algorithm>
#include <cstring>

#include "common.h"
#include "gemm.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;

template <typename T> struct Cfg {
  static constexpr int VE = 16 / sizeof(T);               // elements per 16-byte vector
  static constexpr int PAD = sizeof(T) == 2 ? 8 : 4;
  static constexpr int LD = BK + PAD;                     // LDS row stride (elements)
  static constexpr int KC_VEC = BM * BK / VE / NT;         // vectors per thread, K-contiguous
  static constexpr int KK = BM * BK / NT / VE;             // reduction rows per thread, MN-contiguous
};

template <typename T> struct Stage {
  uint4 v[Cfg<T>::KC_VEC];  // same count for both layouts (BM*BK/VE/NT)
};

// ---- global -> registers
template <typename T, bool KC>
DEVI void load_tile(Stage<T> &st, const T *X, long ld, int rows, int K, int r0, int k0, int tid, int kwrap = 0) {
  constexpr int VE = Cfg<T>::VE;
  if constexpr (KC) {
    constexpr int VPR = BK / VE;  // vectors per row
#pragma unroll
    for (int i = 0; i < Cfg<T>::KC_VEC; ++i) {
      int v = tid + NT * i;
      int r = v / VPR, c = (v % VPR) * VE;
      int gr = r0 + r, gk = k0 + c;
      const int ck = kwrap > 0 ? gk % kwrap : gk;  // column read (a vector never straddles the wrap)
      if (gr < rows && gk < K)
        st.v[i] = *reinterpret_cast<const uint4 *>(X + (long)gr * ld + ck);
      else
        st.v[i] = make_uint4(0, 0, 0, 0);
    }
  } else {
    constexpr int MC = BM / VE;  // vectors across the tile's M/N extent
    constexpr int KK = Cfg<T>::KK;
    int mc = tid % MC, kg = tid / MC;
    int gm = r0 + mc * VE;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      int gk = k0 + kg * KK + kk;
      if (gk < K && gm < rows)
        st.v[kk] = *reinterpret_cast<const uint4 *>(X + (long)gk * ld + gm);
      else
        st.v[kk] = make_uint4(0, 0, 0, 0);
    }
  }
}

// ---- registers -> LDS ([row][k], k contiguous)
template <typename T, bool KC> DEVI void store_tile(const Stage<T> &st, T *sm, int tid);

template <> DEVI void store_tile<bf16_t, true>(const Stage<bf16_t> &st, bf16_t *sm, int tid) {
  constexpr int VPR = BK / 8;
#pragma unroll
  for (int i = 0; i < Cfg<bf16_t>::KC_VEC; ++i) {
    int v = tid + NT * i;
    int r = v / VPR, c = (v % VPR) * 8;
    *reinterpret_cast<uint4 *>(sm + r * Cfg<bf16_t>::LD + c) = st.v[i];
  }
}
template <> DEVI void store_tile<float, true>(const Stage<float> &st, float *sm, int tid) {
  constexpr int VPR = BK / 4;
#pragma unroll
  for (int i = 0; i < Cfg<float>::KC_VEC; ++i) {
    int v = tid + NT * i;
    int r = v / VPR, c = (v % VPR) * 4;
    *reinterpret_cast<uint4 *>(sm + r * Cfg<float>::LD + c) = st.v[i];
  }
}
template <> DEVI void store_tile<bf16_t, false>(const Stage<bf16_t> &st, bf16_t *sm, int tid) {
  // 4 reduction rows x 8 columns per thread -> 8 LDS rows of 4 contiguous k.
  constexpr int MC = BM / 8;
  int mc = tid % MC, kg = tid / MC;
  const uint32_t *w0 = reinterpret_cast<const uint32_t *>(&st.v[0]);
  const uint32_t *w1 = reinterpret_cast<const uint32_t *>(&st.v[1]);
  const uint32_t *w2 = reinterpret_cast<const uint32_t *>(&st.v[2]);
  const uint32_t *w3 = reinterpret_cast<const uint32_t *>(&st.v[3]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int sh = (e & 1) * 16, wi = e >> 1;
    uint32_t a = (w0[wi] >> sh) & 0xFFFF, b = (w1[wi] >> sh) & 0xFFFF;
    uint32_t c = (w2[wi] >> sh) & 0xFFFF, d = (w3[wi] >> sh) & 0xFFFF;
    uint2 out = make_uint2(a | (b << 16), c | (d << 16));
    *reinterpret_cast<uint2 *>(sm + (mc * 8 + e) * Cfg<bf16_t>::LD + kg * 4) = out;
  }
}
template <> DEVI void store_tile<float, false>(const Stage<float> &st, float *sm, int tid) {
  // 8 reduction rows x 4 columns per thread -> 4 LDS rows of 8 contiguous k.
  constexpr int MC = BM / 4;
  int mc = tid % MC, kg = tid / MC;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) x[kk] = reinterpret_cast<const float *>(&st.v[kk])[e];
    float *dst = sm + (mc * 4 + e) * Cfg<float>::LD + kg * 8;
    *reinterpret_cast<float4 *>(dst) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(dst + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
}

DEVI int remap_tile(int i, int T) {
  int q = T / 8, rem = T % 8;
  int x = i % 8, j = i / 8;
  return x * q + min(x, rem) + j;
}

// Split-K partial store marker (not a public epilogue).
constexpr int EPI_PARTIAL = 100;

template <typename T, bool AK, bool BKc, int EPI>
__global__ __launch_bounds__(NT) void gemm_kernel(const GemmArgs g) {
  constexpr int LD = Cfg<T>::LD;
  __shared__ __align__(16) T smA[2][BM * LD];
  __shared__ __align__(16) T smB[2][BN * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int mt = (g.M + BM - 1) / BM, ntl = (g.N + BN - 1) / BN;
  const int tile = remap_tile(blockIdx.x, mt * ntl);
  const int tm = tile % mt, tn = tile / mt;
  const int m0 = tm * BM, n0 = tn * BN;

  // K range of this split
  int kbeg = 0, kend = g.K;
  if constexpr (EPI == EPI_PARTIAL) {
    int per = ((g.K + g.ksplit - 1) / g.ksplit + BK - 1) / BK * BK;
    kbeg = blockIdx.z * per;
    kend = min(g.K, kbeg + per);
  }
  const T *A = reinterpret_cast<const T *>(g.A);
  const T *B = reinterpret_cast<const T *>(g.B);

  f32x4_v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  Stage<T> sa, sb;
  const int nk = (kend - kbeg + BK - 1) / BK;
  if (nk > 0) {
    load_tile<T, AK>(sa, A, g.lda, g.M, kend, m0, kbeg, tid, g.a_kwrap);
    load_tile<T, BKc>(sb, B, g.ldb, g.N, kend, n0, kbeg, tid);
    store_tile<T, AK>(sa, smA[0], tid);
    store_tile<T, BKc>(sb, smB[0], tid);
  }
  __syncthreads();

  const int lr = lane & 15, lk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_tile<T, AK>(sa, A, g.lda, g.M, kend, m0, kbeg + (kt + 1) * BK, tid, g.a_kwrap);
      load_tile<T, BKc>(sb, B, g.ldb, g.N, kend, n0, kbeg + (kt + 1) * BK, tid);
    }
    const T *pa = smA[cur];
    const T *pb = smB[cur];
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      Frag<T> fb[4], fa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) load_frag(fb[i], pb + (wn * 64 + i * 16 + lr) * LD + ks + lk);
#pragma unroll
      for (int j = 0; j < 4; ++j) load_frag(fa[j], pa + (wm * 64 + j * 16 + lr) * LD + ks + lk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma(acc[i][j], fb[i], fa[j]);
    }
    if (kt + 1 < nk) {
      store_tile<T, AK>(sa, smA[cur ^ 1], tid);
      store_tile<T, BKc>(sb, smB[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------- epilogues
  const int g4 = (lane >> 4) * 4;
  if constexpr (EPI == EPI_CE) {
    const int lab_base = *g.pos0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + j * 16 + lr;
      const int lab = (m < g.M) ? g.rowi[lab_base + m] : -1;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int n = n0 + wn * 64 + i * 16 + g4 + r;
          if (n < g.N) mx = fmaxf(mx, acc[i][j][r]);
        }
      mx = group4_max(mx);
      if (g.part_arg) {  // lowest column holding the tile's maximum (columns increase with i, r)
        int ai = 0x7fffffff;
#pragma unroll
        for (int i = 3; i >= 0; --i)
#pragma unroll
          for (int r = 3; r >= 0; --r) {
            const int n = n0 + wn * 64 + i * 16 + g4 + r;
            if (n < g.N && acc[i][j][r] == mx) ai = n;
          }
        ai = group4_min_int(ai);
        if (m < g.M && (lane >> 4) == 0) g.part_arg[(long)m * g.part_ld + tn * 2 + wn] = ai + g.col_off;
      }
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int n = n0 + wn * 64 + i * 16 + g4 + r;
          if (n < g.N) {
            s += exp2f((acc[i][j][r] - mx) * LOG2E_F);
            if (n + g.col_off == lab) g.zlab[m] = acc[i][j][r];
          }
        }
      s = group4_sum(s);
      if (m < g.M && (lane >> 4) == 0) g.part[(long)m * g.part_ld + tn * 2 + wn] = make_float2(mx, s);
    }
    return;
  }
  if constexpr (EPI == EPI_PROBS) {
    // the partial slots of EPI_CE (every 64-column half of a 128-column tile), from slot
    // col_off / 64 on; every partial of a row carries the row's shift
    const int lab_base = *g.pos0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + j * 16 + lr;
      const bool mok = m < g.M;
      const int lab = mok ? g.rowi[lab_base + m] : -1;
      const float c = mok ? g.rowf[m] : 0.f;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + wn * 64 + i * 16 + g4;
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = 0.f;
          if (n + r < g.N) {
            e[r] = exp2f((acc[i][j][r] - c) * LOG2E_F);
            s += e[r];
            if (g.zlab && n + r + g.col_off == lab) g.zlab[m] = acc[i][j][r];
          }
        }
        if (g.C && mok && n < g.N) store4<T>(reinterpret_cast<T *>(g.C) + (long)m * g.ldc + n, e);
      }
      s = group4_sum(s);
      if (g.part && mok && (lane >> 4) == 0)
        g.part[(long)m * g.part_ld + g.col_off / 64 + tn * 2 + wn] = make_float2(c, s);
    }
    return;
  }
  if constexpr (EPI == EPI_SWIGLU) {
    T *Hm = reinterpret_cast<T *>(g.C);
    T *GU = reinterpret_cast<T *>(g.C2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + j * 16 + lr;
      if (m >= g.M) continue;
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int nb = n0 + wn * 64 + i * 16;  // gate block start; up block is nb + 16
        if (nb >= g.N) continue;
        const int unit = (nb >> 1) + g4;
        float h[4], gv[4], uv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gv[r] = acc[i][j][r] * g.acc_scale;
          uv[r] = acc[i + 1][j][r] * g.acc_scale;
          h[r] = gv[r] / (1.f + __expf(-gv[r])) * uv[r];
        }
        store4<T>(Hm + (long)m * g.ldc + unit, h);
        if (GU) {
          store4<T>(GU + (long)m * g.ldc2 + nb + g4, gv);
          store4<T>(GU + (long)m * g.ldc2 + nb + 16 + g4, uv);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 64 + j * 16 + lr;
    if (m >= g.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + wn * 64 + i * 16 + g4;
      if (n >= g.N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if constexpr (EPI == EPI_STORE) {
        store4<T>(reinterpret_cast<T *>(g.C) + (long)m * g.ldc + n, v);
      } else if constexpr (EPI == EPI_STORE_F32) {
        store4<float>(g.Cf + (long)m * g.ldcf + n, v);
      } else if constexpr (EPI == EPI_ADD_F32) {
        float4 *p = reinterpret_cast<float4 *>(g.Cf + (long)m * g.ldcf + n);
        float4 o = *p;
        const float sc = g.acc_scale;
        *p = make_float4(o.x + v[0] * sc, o.y + v[1] * sc, o.z + v[2] * sc, o.w + v[3] * sc);
      } else if constexpr (EPI == EPI_PARTIAL) {
        store4<float>(g.ws + ((long)blockIdx.z * g.M + m) * g.N + n, v);
      } else if constexpr (EPI == EPI_SGD) {
        float4 *pw = reinterpret_cast<float4 *>(g.Cf + (long)m * g.ldcf + n);
        float4 w = *pw;
        float nw[4] = {w.x - g.alpha * v[0], w.y - g.alpha * v[1], w.z - g.alpha * v[2], w.w - g.alpha * v[3]};
        *pw = make_float4(nw[0], nw[1], nw[2], nw[3]);
        float sw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sw[r] = nw[r] * g.c_scale;
        store4<T>(reinterpret_cast<T *>(g.C) + (long)m * g.ldc + n, sw);
        if (g.C2) {
          float lo[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) lo[r] = sw[r] - to_f(from_f<T>(sw[r]));
          store4<T>(reinterpret_cast<T *>(g.C2) + (long)m * g.ldc2 + n, lo);
        }
        if (g.CT) {
#pragma unroll
          for (int r = 0; r < 4; ++r) reinterpret_cast<T *>(g.CT)[(long)(n + r) * g.ldct + m] = from_f<T>(nw[r]);
        }
      }
    }
  }
}

// out[m, n] (=|+=) sum_s ws[s, m, n], s in increasing order.
template <typename T, int MODE>
__global__ __launch_bounds__(256) void splitk_reduce(const float *ws, int S, int M, int N, void *out, long ld,
                                                     float sc) {
  long idx = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  long total = (long)M * N;
  if (idx >= total) return;
  int m = idx / N, n = idx % N;
  float4 acc = *reinterpret_cast<const float4 *>(ws + idx);
  for (int s = 1; s < S; ++s) {
    float4 x = *reinterpret_cast<const float4 *>(ws + (long)s * total + idx);
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  float v[4] = {acc.x, acc.y, acc.z, acc.w};
  if constexpr (MODE == EPI_STORE) {
    store4<T>(reinterpret_cast<T *>(out) + (long)m * ld + n, v);
  } else if constexpr (MODE == EPI_STORE_F32) {
    store4<float>(reinterpret_cast<float *>(out) + (long)m * ld + n, v);
  } else {
    float4 *p = reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + (long)m * ld + n);
    float4 o = *p;
    *p = make_float4(o.x + v[0] * sc, o.y + v[1] * sc, o.z + v[2] * sc, o.w + v[3] * sc);
  }
}

template <typename T, bool AK, bool BKc, int EPI>
hipError_t launch_t(const GemmArgs &g, hipStream_t st, int split) {
  int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  dim3 grid(tiles, 1, split);
  hipLaunchKernelGGL((gemm_kernel<T, AK, BKc, EPI>), grid, dim3(NT), 0, st, g);
  return hipGetLastError();
}

template <typename T, bool AK, bool BKc>
hipError_t dispatch_epi(int epi, const GemmArgs &g, hipStream_t st, int split) {
  if (split > 1) return launch_t<T, AK, BKc, EPI_PARTIAL>(g, st, split);
  switch (epi) {
    case EPI_STORE: return launch_t<T, AK, BKc, EPI_STORE>(g, st, 1);
    case EPI_STORE_F32: return launch_t<T, AK, BKc, EPI_STORE_F32>(g, st, 1);
    case EPI_ADD_F32: return launch_t<T, AK, BKc, EPI_ADD_F32>(g, st, 1);
    case EPI_SWIGLU: return launch_t<T, AK, BKc, EPI_SWIGLU>(g, st, 1);
    case EPI_CE: return launch_t<T, AK, BKc, EPI_CE>(g, st, 1);
    case EPI_PROBS: return launch_t<T, AK, BKc, EPI_PROBS>(g, st, 1);
    case EPI_SGD: return launch_t<T, AK, BKc, EPI_SGD>(g, st, 1);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t dispatch_layout(bool ak, bool bk, int epi, const GemmArgs &g, hipStream_t st, int split) {
  if (ak && bk) return dispatch_epi<T, true, true>(epi, g, st, split);
  if (ak && !bk) return dispatch_epi<T, true, false>(epi, g, st, split);
  if (!ak && !bk) return dispatch_epi<T, false, false>(epi, g, st, split);
  return dispatch_epi<T, false, true>(epi, g, st, split);
}

template <typename T>
hipError_t reduce_launch(int epi, const GemmArgs &g, int S, hipStream_t st) {
  long total = (long)g.M * g.N;
  dim3 grid((unsigned)((total / 4 + 255) / 256));
  switch (epi) {
    case EPI_STORE:
      hipLaunchKernelGGL((splitk_reduce<T, EPI_STORE>), grid, dim3(256), 0, st, g.ws, S, g.M, g.N, g.C, g.ldc, 1.f);
      break;
    case EPI_STORE_F32:
      hipLaunchKernelGGL((splitk_reduce<T, EPI_STORE_F32>), grid, dim3(256), 0, st, g.ws, S, g.M, g.N,
                         (void *)g.Cf, g.ldcf, 1.f);
      break;
    default:
      hipLaunchKernelGGL((splitk_reduce<T, EPI_ADD_F32>), grid, dim3(256), 0, st, g.ws, S, g.M, g.N,
                         (void *)g.Cf, g.ldcf, g.acc_scale);
      break;
  }
  return hipGetLastError();
}

}  // namespace

size_t gemm_ws_elems(int M, int N) { return (size_t)8 * M * N; }

hipError_t gemm_dma_launch(bool f16, int epi, const GemmArgs &g, hipStream_t st);
hipError_t gemm_dma256_launch(bool f16, int epi, const GemmArgs &g, hipStream_t st);
hipError_t gemm_dma256_group_launch(bool f16, int epi, GemmGroup &gg, hipStream_t st);
// few-row products (gemv.hip): M <= 4, 16-bit k-contiguous operands, fp32 / SwiGLU / CE epilogues
bool gemv_ok(int dtype, bool a_kc, bool b_kc, int epi, const GemmArgs &g);
hipError_t gemv_launch(bool f16, int epi, const GemmArgs &g, hipStream_t st);

static bool use_dma(int dtype, bool a_kc, bool b_kc, const GemmArgs &g) {
  return (dtype == 1 || dtype == 2) && a_kc && b_kc && g.K % 64 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
         g.a_kwrap % 64 == 0;
}

// Each split must own at least one 64-deep step.
static int round_split(int split, int K) {
  if (split < 2) return 1;
  const int per = ((K + split - 1) / split + BK - 1) / BK * BK;
  return (K + per - 1) / per;
}

GemmPlan gemm_plan(int dtype, bool a_kc, bool b_kc, int epi, const GemmArgs &g, size_t ws_elems, int force_split) {
  const bool dma = use_dma(dtype, a_kc, b_kc, g);
  GemmPlan p;
  if (force_split <= 0 && gemv_ok(dtype, a_kc, b_kc, epi, g)) return p;
  const long t256 = (long)((g.M + 255) / 256) * ((g.N + 255) / 256);
  // the 256 x 256 tile (one work-group per CU) when it has enough tiles to fill the GPU
  if (dma && force_split <= 0 && epi != EPI_SGD && t256 >= 200) {
    p.wide = true;
    return p;
  }
  if (epi == EPI_STORE || epi == EPI_STORE_F32 || epi == EPI_ADD_F32) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    int split = 1;
    if (force_split > 0) {
      split = force_split;
    } else if (dma) {
      // few tiles: split K.  The 256 x 256 tile takes about 240 work-groups (one per CU)
      // when every split keeps at least 16 steps and there are at least 4 splits;
      // otherwise the 128 x 128 tile aims for ~400 work-groups (two per CU), each split at
      // least eight steps (the fp32 partial traffic of a split costs about as much as a
      // short K range saves)
      const int s256 = std::min<long>(std::min<long>((240 + t256 - 1) / t256, g.K / (16 * BK)), 8);
      if (s256 >= 4 && (size_t)s256 * g.M * g.N <= ws_elems) {
        p.split = round_split(s256, g.K);
        p.wide = true;
        return p;
      }
      if (tiles < 256) split = std::min(std::min((400 + tiles - 1) / tiles, g.K / (8 * BK)), 4);
    } else if (tiles < 256 && g.K >= 4 * BK) {
      split = (2 * 256 + tiles - 1) / tiles;
      split = min(split, g.K / (2 * BK));
      split = min(split, 8);
    }
    split = round_split(split, g.K);
    if (split > 1 && (size_t)split * g.M * g.N > ws_elems) split = 1;
    p.split = split;
  }
  return p;
}

hipError_t gemm_main_launch(int dtype, bool a_kc, bool b_kc, int epi, GemmArgs g, float *ws, GemmPlan plan,
                            hipStream_t st, bool allow_gemv) {
  const int split = plan.split;
  g.ksplit = split;
  g.ws = ws;
  // the wrapped activation operand must be k-contiguous, whole 16-byte vectors
  if (g.a_kwrap < 0 || (g.a_kwrap > 0 && (!a_kc || g.a_kwrap % 8 != 0))) return hipErrorInvalidValue;
  if (allow_gemv && split <= 1 && gemv_ok(dtype, a_kc, b_kc, epi, g)) return gemv_launch(dtype == 2, epi, g, st);
  if (use_dma(dtype, a_kc, b_kc, g)) {
    if (plan.wide && epi != EPI_SGD) return gemm_dma256_launch(dtype == 2, epi, g, st);
    return gemm_dma_launch(dtype == 2, epi, g, st);
  }
  if (dtype == 2 || g.c_f16) return hipErrorInvalidValue;
  return dtype == 1 ? dispatch_layout<bf16_t>(a_kc, b_kc, epi, g, st, split)
                    : dispatch_layout<float>(a_kc, b_kc, epi, g, st, split);
}

hipError_t gemm_reduce_launch(int dtype, int epi, GemmArgs g, float *ws, int split, hipStream_t st) {
  if (split <= 1) return hipSuccess;
  g.ws = ws;
  if (g.c_f16) return reduce_launch<f16_t>(epi, g, split, st);
  return dtype == 0 ? reduce_launch<float>(epi, g, split, st) : reduce_launch<bf16_t>(epi, g, split, st);
}

hipError_t gemm_group_launch(int dtype, int epi, const GemmArgs *gs, int n, float *ws, size_t ws_elems,
                             hipStream_t st) {
  if (n < 0 || n > GEMM_GROUP_MAX) return hipErrorInvalidValue;
  bool one = epi == EPI_SWIGLU && n > 1;
  for (int p = 0; p < n && one; ++p)
    one = use_dma(dtype, true, true, gs[p]) && gs[p].M > 0 && gs[p].N > 0 &&
          !gemv_ok(dtype, true, true, epi, gs[p]) && (gs[p].a_kwrap == 0 || gs[p].a_kwrap % 8 == 0);
  if (!one) {
    for (int p = 0; p < n; ++p) {
      hipError_t e = gemm_launch(dtype, true, true, epi, gs[p], ws, ws_elems, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  GemmGroup gg;
  memset(&gg, 0, sizeof(gg));
  gg.n = n;
  for (int p = 0; p < n; ++p) {
    gg.g[p] = gs[p];
    gg.g[p].ksplit = 1;
    gg.g[p].ws = ws;
  }
  return gemm_dma256_group_launch(dtype == 2, epi, gg, st);
}

hipError_t gemm_launch(int dtype, bool a_kc, bool b_kc, int epi, GemmArgs g, float *ws, size_t ws_elems,
                       hipStream_t st, int force_split) {
  const GemmPlan plan = gemm_plan(dtype, a_kc, b_kc, epi, g, ws_elems, force_split);
  hipError_t e = gemm_main_launch(dtype, a_kc, b_kc, epi, g, ws, plan, st);
  if (e != hipSuccess) return e;
  return gemm_reduce_launch(dtype, epi, g, ws, plan.split, st);
}
