// bf16 MFMA GEMM for gfx950 with operands streamed straight into LDS
// (used for every bf16 GEMM whose operands are both k-contiguous).
//
// C[m, n] = sum_k A[m, k] B[n, k], both operands stored with k contiguous
// (activations A [M][lda], weights B [N][ldb]).  Work-group tile 128 (weight
// rows) x 128 (tokens) x 64 (k), 256 threads = 4 waves in a 2 x 2 grid; each
// wave owns 64 x 64 outputs as 16x16 tiles of v_mfma_f32_16x16x32_bf16.
//
// Loads: buffer_load_dwordx4 ... lds writes each lane's 16 bytes directly to
// LDS at (base + 16 * lane), so one instruction fills 1 KiB = 8 tile rows of
// 128 bytes.  The lane -> global chunk mapping applies an XOR swizzle
// (chunk ^ ((row >> 1) & 7)) so that the fragment reads (16 consecutive rows,
// one 16-byte chunk) hit 64 distinct banks.  Per-lane byte offsets are loop
// invariant; the k position enters through the scalar offset.  Rows outside
// the matrix get an offset beyond the buffer's extent, which the hardware
// returns as zeros.  Two LDS stages: while one k-step is multiplied from
// registers the next two are in flight; each thread waits on its own
// vector-memory counter for the oldest, then a barrier publishes it.
#include <type_traits>

#include "common.h"
#include "gemm.h"

namespace ttt_g2 {

constexpr int BM = 128, BK = 64, NT = 256;
constexpr uint32_t OOB = BUF_OOB;
constexpr int RSRC_W3 = BUF_RSRC_W3;

template <int BN> struct G2 {
  static constexpr int ROWS = BN + BM;        // tile rows per stage (weights then tokens)
  static constexpr int SBYTES = ROWS * 128;   // bytes per LDS stage
  static constexpr int CPT = ROWS / 32;       // 16-byte chunks each thread moves per tile
  static constexpr int WN = BN / 2;           // wave tile along n
  static constexpr int NI = WN / 16;
};

DEVI int swz(int row) { return (row >> 1) & 7; }


DEVI int remap_tile2(int i, int T) {
  int q = T / 8, rem = T % 8;
  int x = i % 8, j = i / 8;
  return x * q + min(x, rem) + j;
}

// 16-bit output in the type the caller asked for (fp16 or bf16).
DEVI void store_c4(const GemmArgs &g, void *base, long off, const float *v) {
  if (g.c_f16)
    store4<f16_t>(reinterpret_cast<f16_t *>(base) + off, v);
  else
    store4<bf16_t>(reinterpret_cast<bf16_t *>(base) + off, v);
}

// PRE: the fp32 master values of EPI_SGD were loaded ahead into `pre` (same [i][j]
// indexing as acc).
// ct_lds: 8 KiB of LDS private to this wave (EPI_SGD with CT), where the updated
// 64 x 64 tile is transposed so that CT is written in 16-byte rows.
template <int BN, int EPI, bool PRE = false, typename Acc>
DEVI void gemm2_epilogue(const GemmArgs &g, Acc &acc, int m0, int n0, int tn, int wm, int wn, int lr, int lq,
                         const float4 (&pre)[4][4], uint16_t *ct_lds = nullptr) {
  constexpr int NI = G2<BN>::NI, WN = G2<BN>::WN;
  // ------------------------------------------------------------- epilogues
  // lane holds C[m][n .. n+3] for m = m0 + wm*64 + 16 j + lr, n = n0 + wn*WN + 16 i + 4 lq
  const int g4 = lq * 4;
  if constexpr (EPI == EPI_CE) {
    // partial slots exist for both 64-column halves of every 128-column tile of N (what
    // the 128-wide kernels write); the second half of a 256-wide tile past them has none
    const bool slot = n0 + wn * WN < (g.N + 127) / 128 * 128;
    const int lab_base = *g.pos0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + j * 16 + lr;
      const int lab = (m < g.M) ? g.rowi[lab_base + m] : -1;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + wn * WN + i * 16 + g4 + r;
          if (n < g.N) mx = fmaxf(mx, acc[i][j][r]);
        }
      mx = group4_max(mx);
      if (g.part_arg) {  // lowest column holding the tile's maximum (columns increase with i, r)
        int ai = 0x7fffffff;
#pragma unroll
        for (int i = NI - 1; i >= 0; --i)
#pragma unroll
          for (int r = 3; r >= 0; --r) {
            const int n = n0 + wn * WN + i * 16 + g4 + r;
            if (n < g.N && acc[i][j][r] == mx) ai = n;
          }
        ai = group4_min_int(ai);
        if (m < g.M && lq == 0 && slot) g.part_arg[(long)m * g.part_ld + tn * 2 + wn] = ai + g.col_off;
      }
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + wn * WN + i * 16 + g4 + r;
          if (n < g.N) {
            s += fast_exp2((acc[i][j][r] - mx) * LOG2E_F);
            if (n + g.col_off == lab) g.zlab[m] = acc[i][j][r];
          }
        }
      s = group4_sum(s);
      if (m < g.M && lq == 0 && slot) g.part[(long)m * g.part_ld + tn * 2 + wn] = make_float2(mx, s);
    }
    return;
  }
  if constexpr (EPI == EPI_PROBS) {
    // same partial slots as EPI_CE (every 64-column half of a 128-column tile of N), at
    // slot col_off / 64 onwards; every partial of a row carries the row's shift
    const bool slot = n0 + wn * WN < (g.N + 127) / 128 * 128;
    const int lab_base = *g.pos0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + j * 16 + lr;
      const bool mok = m < g.M;
      const int lab = mok ? g.rowi[lab_base + m] : -1;
      const float c = mok ? g.rowf[m] : 0.f;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = n0 + wn * WN + i * 16 + g4;
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = 0.f;
          if (n + r < g.N) {
            e[r] = fast_exp2((acc[i][j][r] - c) * LOG2E_F);
            s += e[r];
            if (g.zlab && n + r + g.col_off == lab) g.zlab[m] = acc[i][j][r];
          }
        }
        if (g.C && mok && n < g.N) store_c4(g, g.C, (long)m * g.ldc + n, e);
      }
      s = group4_sum(s);
      if (g.part && mok && lq == 0 && slot)
        g.part[(long)m * g.part_ld + g.col_off / 64 + tn * 2 + wn] = make_float2(c, s);
    }
    return;
  }
  if constexpr (EPI == EPI_SWIGLU) {
    void *GU = g.C2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + j * 16 + lr;
      if (m >= g.M) continue;
#pragma unroll
      for (int i = 0; i < NI; i += 2) {
        const int nb = n0 + wn * WN + i * 16;  // gate block start; up block is nb + 16
        if (nb >= g.N) continue;
        const int unit = (nb >> 1) + g4;
        float hv[4], gv[4], uv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gv[r] = acc[i][j][r] * g.acc_scale;
          uv[r] = acc[i + 1][j][r] * g.acc_scale;
          hv[r] = gv[r] / (1.f + __expf(-gv[r])) * uv[r];
        }
        store_c4(g, g.C, (long)m * g.ldc + unit, hv);
        if (GU) {
          store_c4(g, GU, (long)m * g.ldc2 + nb + g4, gv);
          store_c4(g, GU, (long)m * g.ldc2 + nb + 16 + g4, uv);
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
    for (int i = 0; i < NI; ++i) {
      const int n = n0 + wn * WN + i * 16 + g4;
      if (n >= g.N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if constexpr (EPI == EPI_STORE) {
        store_c4(g, g.C, (long)m * g.ldc + n, v);
      } else if constexpr (EPI == EPI_STORE_F32) {
        store4<float>(g.Cf + (long)m * g.ldcf + n, v);
      } else if constexpr (EPI == EPI_ADD_F32) {
        float4 *p = reinterpret_cast<float4 *>(g.Cf + (long)m * g.ldcf + n);
        float4 o = *p;
        const float sc = g.acc_scale;
        *p = make_float4(o.x + v[0] * sc, o.y + v[1] * sc, o.z + v[2] * sc, o.w + v[3] * sc);
      } else if constexpr (EPI == 100) {  // split-K partial
        store4<float>(g.ws + ((long)blockIdx.z * g.M + m) * g.N + n, v);
      } else if constexpr (EPI == EPI_SGD) {
        float4 *pw = reinterpret_cast<float4 *>(g.Cf + (long)m * g.ldcf + n);
        float4 w;
        if constexpr (PRE)
          w = pre[i][j];
        else
          w = *pw;
        float nw[4] = {w.x - g.alpha * v[0], w.y - g.alpha * v[1], w.z - g.alpha * v[2], w.w - g.alpha * v[3]};
        *pw = make_float4(nw[0], nw[1], nw[2], nw[3]);
        float sw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sw[r] = nw[r] * g.c_scale;
        store_c4(g, g.C, (long)m * g.ldc + n, sw);
        if (g.C2) {
          float lo[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            lo[r] = sw[r] - (g.c_f16 ? to_f(from_f<f16_t>(sw[r])) : to_f(from_f<bf16_t>(sw[r])));
          store_c4(g, g.C2, (long)m * g.ldc2 + n, lo);
        }
        if (ct_lds) {  // [n][m] within the wave's 64 x 64 tile
#pragma unroll
          for (int r = 0; r < 4; ++r)
            ct_lds[(i * 16 + g4 + r) * 64 + j * 16 + lr] =
                g.c_f16 ? from_f<f16_t>(nw[r]).x : from_f<bf16_t>(nw[r]);
        }
      }
    }
  }
  if constexpr (EPI == EPI_SGD) {
    if (ct_lds) {
      // rows of 8 consecutive m: 8 lanes cover one n row of the tile (128 bytes)
      const int lane = lr + 16 * lq, mb = m0 + wm * 64, nb = n0 + wn * WN;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int idx = lane + 64 * c, nl = idx >> 3, ml = (idx & 7) * 8;
        const int n = nb + nl, m = mb + ml;
        if (n >= g.N || m >= g.M) continue;
        uint16_t *dst = reinterpret_cast<uint16_t *>(g.CT) + (long)n * g.ldct + m;
        if (m + 7 < g.M) {
          *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(ct_lds + nl * 64 + ml);
        } else {
          for (int e = 0; e < 8 && m + e < g.M; ++e) dst[e] = ct_lds[nl * 64 + ml + e];
        }
      }
    }
  }
}

// Direct-to-LDS streaming of one k-tile (both operands) by one wave.
template <int BN> struct G3Issue {
  static constexpr int CPW = G2<BN>::ROWS / 8 / 4;  // 1 KiB chunks per wave
  __amdgpu_buffer_rsrc_t rw, rx;
  uint32_t voff[CPW];
  int wave, kbeg, kwrap;
  char *sm;
  DEVI void init(const GemmArgs &g, int wave_, int lane, int n0, int m0, int kb, char *sm_) {
    const int ka = g.a_kwrap > 0 ? g.a_kwrap : g.K;  // columns of A
    const uint32_t wbytes = (uint32_t)(((long)(g.N - 1) * g.ldb + g.K) * 2);
    const uint32_t xbytes = (uint32_t)(((long)(g.M - 1) * g.lda + ka) * 2);
    rw = __builtin_amdgcn_make_buffer_rsrc((void *)g.B, (short)0, wbytes, RSRC_W3);
    rx = __builtin_amdgcn_make_buffer_rsrc((void *)g.A, (short)0, xbytes, RSRC_W3);
    wave = wave_;
    kbeg = kb;
    kwrap = g.a_kwrap;
    sm = sm_;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int j = wave * CPW + c;
      const int row = j * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ swz(row);
      if (row < BN) {
        const int gr = n0 + row;
        voff[c] = gr < g.N ? (uint32_t)(((long)gr * g.ldb + kc * 8) * 2) : OOB;
      } else {
        const int gr = m0 + row - BN;
        voff[c] = gr < g.M ? (uint32_t)(((long)gr * g.lda + kc * 8) * 2) : OOB;
      }
    }
  }
  // Streams k-step kt (64 deep) of both operands into the stage at stage_off.
  // A's column is the step's k modulo kwrap (k-steps never straddle the wrap).
  DEVI void run(int kt, int stage_off = 0) const {
    const int k = kbeg + kt * BK;
    const int soff_w = k * 2;
    const int soff_x = (kwrap > 0 ? k % kwrap : k) * 2;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int j = wave * CPW + c;
      lds_void *dst = (lds_void *)(sm + stage_off + j * 1024);
      if (j * 8 < BN)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, voff[c], soff_w, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, dst, 16, voff[c], soff_x, 0, 0);
    }
  }
};

typedef int v4i_t __attribute__((ext_vector_type(4)));

// All sixteen fragments of one 64-deep k-step of a 128 x 128 tile (4 weight
// and 4 token 16-row fragments for each 32-deep half), read in one block that
// ends by waiting for its own reads.  Written as one asm block on purpose: the
// compiler then does not treat the reads as possibly aliasing the
// direct-to-LDS writes still in flight into the other stage (it would wait for
// those before every read).  Visibility of the stage is ordered by the
// caller's explicit vector-memory wait and barrier.
template <typename TI>
DEVI void read_step_128(Frag<TI> (&fw)[2][4], Frag<TI> (&fx)[2][4], uint32_t w0, uint32_t w1, uint32_t x0,
                        uint32_t x1) {
  v4i_t a0, a1, a2, a3, b0, b1, b2, b3, c0, c1, c2, c3, d0, d1, d2, d3;
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %16 offset:2048\n"
      "ds_read_b128 %2, %16 offset:4096\n"
      "ds_read_b128 %3, %16 offset:6144\n"
      "ds_read_b128 %4, %17\n"
      "ds_read_b128 %5, %17 offset:2048\n"
      "ds_read_b128 %6, %17 offset:4096\n"
      "ds_read_b128 %7, %17 offset:6144\n"
      "ds_read_b128 %8, %18\n"
      "ds_read_b128 %9, %18 offset:2048\n"
      "ds_read_b128 %10, %18 offset:4096\n"
      "ds_read_b128 %11, %18 offset:6144\n"
      "ds_read_b128 %12, %19\n"
      "ds_read_b128 %13, %19 offset:2048\n"
      "ds_read_b128 %14, %19 offset:4096\n"
      "ds_read_b128 %15, %19 offset:6144\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3), "=&v"(c0),
        "=&v"(c1), "=&v"(c2), "=&v"(c3), "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
      : "v"(w0), "v"(w1), "v"(x0), "v"(x1)
      : "memory");
  fw[0][0].v = __builtin_bit_cast(uint4, a0);
  fw[0][1].v = __builtin_bit_cast(uint4, a1);
  fw[0][2].v = __builtin_bit_cast(uint4, a2);
  fw[0][3].v = __builtin_bit_cast(uint4, a3);
  fw[1][0].v = __builtin_bit_cast(uint4, b0);
  fw[1][1].v = __builtin_bit_cast(uint4, b1);
  fw[1][2].v = __builtin_bit_cast(uint4, b2);
  fw[1][3].v = __builtin_bit_cast(uint4, b3);
  fx[0][0].v = __builtin_bit_cast(uint4, c0);
  fx[0][1].v = __builtin_bit_cast(uint4, c1);
  fx[0][2].v = __builtin_bit_cast(uint4, c2);
  fx[0][3].v = __builtin_bit_cast(uint4, c3);
  fx[1][0].v = __builtin_bit_cast(uint4, d0);
  fx[1][1].v = __builtin_bit_cast(uint4, d1);
  fx[1][2].v = __builtin_bit_cast(uint4, d2);
  fx[1][3].v = __builtin_bit_cast(uint4, d3);
}

// Two LDS stages, 128 x 128 tile: while step kt is multiplied from registers,
// the tiles of steps kt+1 and kt+2 are in flight.  Per step: wait for this
// wave's loads of step kt, barrier, read the step's fragments, barrier (the
// stage is free), stream step kt+2 into it, MFMAs.
// EPI is a template parameter so that each epilogue is its own kernel symbol
// (profiles then separate the GEMM classes).
template <typename TI, int EPI>
__global__ __launch_bounds__(NT, 2) void gemm5_kernel(const GemmArgs g) {
  using C = G2<128>;
  constexpr int SBYTES = C::SBYTES;
  constexpr int CPW = C::ROWS / 8 / 4;  // 1 KiB chunks per wave and stage
  __shared__ __align__(1024) char sm[2 * SBYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int mt = (g.M + BM - 1) / BM, ntl = (g.N + 127) / 128;
  // Each XCD takes a contiguous run of the tile order; the order walks bands of
  // GM row tiles across all columns (rows fastest), so the 64 work-groups an XCD
  // runs at once share about 8 activation and 8 weight tiles in its L2 instead of
  // one weight tile and 64 activation tiles.  With mt <= GM it is plain
  // row-fastest order.
  constexpr int GM = 8;
  const int tile = remap_tile2(blockIdx.x, mt * ntl);
  const int band = tile / (GM * ntl), in_band = tile % (GM * ntl);
  const int bm = min(GM, mt - band * GM);
  const int tm = band * GM + in_band % bm, tn = in_band / bm;
  const int m0 = tm * BM, n0 = tn * 128;
  int kbeg = 0, kend = g.K;
  if (g.ksplit > 1) {
    const int per = ((g.K + g.ksplit - 1) / g.ksplit + BK - 1) / BK * BK;
    kbeg = blockIdx.z * per;
    kend = min(g.K, kbeg + per);
  }
  const int nk = (kend - kbeg + BK - 1) / BK;
  G3Issue<128> is;
  is.init(g, wave, lane, n0, m0, kbeg, sm);
  f32x4_v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  const int lr = lane & 15, lq = lane >> 4;
  // fragment byte offsets within a stage (rows differ by multiples of 16, which
  // keep the swizzle of the lane's first row)
  const int rw = wn * 64 + lr, rx = 128 + wm * 64 + lr;
  const uint32_t aw0 = rw * 128 + (((0 + lq) ^ swz(rw)) << 4), aw1 = rw * 128 + (((4 + lq) ^ swz(rw)) << 4);
  const uint32_t ax0 = rx * 128 + (((0 + lq) ^ swz(rx)) << 4), ax1 = rx * 128 + (((4 + lq) ^ swz(rx)) << 4);
  const uint32_t smb = (uint32_t)(uintptr_t)(lds_void *)sm;
  if (nk > 0) is.run(0, 0);
  if (nk > 1) is.run(1, SBYTES);
  // SGD: the fp32 master values this lane updates are loaded while the last steps run,
  // issued after the last tile load so that the waits on tile loads do not cover them
  // (vector-memory loads complete in issue order).
  constexpr bool PRE = EPI == EPI_SGD;
  constexpr int NPRE = PRE ? 16 : 0;
  float4 pre[4][4];
  // through a buffer descriptor: every lane issues all 16 loads (offsets outside the matrix
  // read zero), so the wave's count of outstanding loads is the same on every tile
  const __amdgpu_buffer_rsrc_t rcf = __builtin_amdgcn_make_buffer_rsrc(
      (void *)g.Cf, (short)0, PRE ? (uint32_t)(((long)(g.M - 1) * g.ldcf + g.N) * 4) : 0u, RSRC_W3);
#define GEMM5_PREFETCH                                                                                       \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) _Pragma("unroll") for (int j = 0; j < 4; ++j) {              \
    const int m = m0 + wm * 64 + j * 16 + lr, n = n0 + wn * 64 + i * 16 + lq * 4;                              \
    const uint32_t o = (m < g.M && n < g.N) ? (uint32_t)(((long)m * g.ldcf + n) * 4) : OOB;                   \
    pre[i][j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rcf, o, 0, 0));              \
  }

  if (PRE && nk <= 2) { GEMM5_PREFETCH }  // no tile load is issued inside the loop
  for (int kt = 0; kt < nk; ++kt) {
    // outstanding, oldest first: tile loads of steps kt and kt+1, then (from step nk-2 on)
    // the master values
    if (kt + 1 < nk) {
      if (PRE && nk > 2 && kt == nk - 2) wait_vm<CPW + NPRE>(); else wait_vm<CPW>();
    } else {
      if (PRE) wait_vm<NPRE>(); else wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
    const uint32_t so = smb + (kt & 1) * SBYTES;
    Frag<TI> fw[2][4], fx[2][4];
    read_step_128<TI>(fw, fx, so + aw0, so + aw1, so + ax0, so + ax1);
    __builtin_amdgcn_s_barrier();
    if (kt + 2 < nk) is.run(kt + 2, (kt & 1) * SBYTES);
    if (PRE && kt + 2 == nk - 1) { GEMM5_PREFETCH }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma(acc[i][j], fw[ks][i], fx[ks][j]);
  }
  uint16_t *ct_lds = nullptr;
  if (PRE && g.CT)  // the stage not read by the last step is free once every wave passed its barrier
    ct_lds = reinterpret_cast<uint16_t *>(sm + (nk & 1) * SBYTES + wave * 8192);
  gemm2_epilogue<128, EPI, PRE>(g, acc, m0, n0, tn, wm, wn, lr, lq, pre, ct_lds);
#undef GEMM5_PREFETCH
}

#define G5_INST(TI)                                                      \
  template __global__ void gemm5_kernel<TI, EPI_STORE>(const GemmArgs);     \
  template __global__ void gemm5_kernel<TI, EPI_STORE_F32>(const GemmArgs); \
  template __global__ void gemm5_kernel<TI, EPI_ADD_F32>(const GemmArgs);   \
  template __global__ void gemm5_kernel<TI, EPI_SWIGLU>(const GemmArgs);    \
  template __global__ void gemm5_kernel<TI, EPI_CE>(const GemmArgs);        \
  template __global__ void gemm5_kernel<TI, EPI_PROBS>(const GemmArgs);   \
  template __global__ void gemm5_kernel<TI, EPI_SGD>(const GemmArgs);       \
  template __global__ void gemm5_kernel<TI, 100>(const GemmArgs);
G5_INST(bf16_t)
G5_INST(f16_t)
#undef G5_INST

template <typename TI, int EPI> hipError_t launch5_e(const GemmArgs &g, hipStream_t st) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + 127) / 128);
  hipLaunchKernelGGL((gemm5_kernel<TI, EPI>), dim3(tiles, 1, g.ksplit), dim3(NT), 0, st, g);
  return hipGetLastError();
}

template <typename TI> hipError_t launch5(int epi, const GemmArgs &g, hipStream_t st) {
  if (g.ksplit > 1) return launch5_e<TI, 100>(g, st);
  switch (epi) {
    case EPI_STORE: return launch5_e<TI, EPI_STORE>(g, st);
    case EPI_STORE_F32: return launch5_e<TI, EPI_STORE_F32>(g, st);
    case EPI_ADD_F32: return launch5_e<TI, EPI_ADD_F32>(g, st);
    case EPI_SWIGLU: return launch5_e<TI, EPI_SWIGLU>(g, st);
    case EPI_CE: return launch5_e<TI, EPI_CE>(g, st);
    case EPI_PROBS: return launch5_e<TI, EPI_PROBS>(g, st);
    case EPI_SGD: return launch5_e<TI, EPI_SGD>(g, st);
  }
  return hipErrorInvalidValue;
}


// ====================================================================== 256 x 256 tile
// Work-group tile 256 (weight rows) x 256 (tokens) x 64 (k), 512 threads = 8 waves in a
// 2 x 4 grid (weight halves x token quarters), one work-group per CU and two waves per
// SIMD; each wave owns 128 x 64 outputs, 32 accumulator tiles of 16x16 held in AGPRs.
// Per FLOP this tile moves half the L2 -> LDS bytes of the 128 x 128 tile; while one
// wave of a SIMD waits (for a barrier, its loads or its LDS reads) the other issues
// MFMAs.
//
// LDS: two stages (one per k-step in flight), each split into two 32 KiB halves, one
// per 32-deep half of the step: 512 rows x 64 bytes (weight rows 0..255, token rows
// 256..511), 16-byte chunk c of row r stored at chunk position c ^ ((r >> 1) & 2).
// gfx950's LDS has 64 banks of 4 bytes and serves a ds_read_b128 in four passes of 16
// lanes (measured: lanes l < 32 whose 4-lane group index l / 4 has even bit parity form
// one pass, odd parity another, likewise for l >= 32); with this swizzle the 16 lanes of
// every pass of a fragment read (16 rows, one chunk per 16 lanes) hit 16 distinct 16-byte
// bank groups.  buffer_load ... lds fills a half with 4 loads per thread (1 KiB = 16 rows).
//
// Schedule of k-step t (first-half fragments of t already in registers F0):
//   barrier S (this thread waited for its loads of (t, half 1)), then
//   A: 32 MFMAs from F0; interleaved, one instruction between MFMAs: the 12 reads of
//      (t, half 1) into F1, then the 4 loads of (t+2, half 0) into the half region
//      (t, half 0), free since barrier S;
//   barrier M (loads of (t+1, half 0) waited for), then
//   B: 32 MFMAs from F1 with the reads of (t+1, half 0) into F0 and the loads of
//      (t+2, half 1) into the region (t, half 1), free since barrier M.
// A half's data is requested one and a half k-steps before it is read.  The whole loop
// is one asm statement: the accumulators stay in their AGPRs (tied "+a"; the register
// allocator moves values tied across several statements between registers), the
// fragment registers are its outputs, and every LDS read is waited for inside it.
namespace g8 {
constexpr int NT8 = 512;
constexpr int TW = 256, TX = 256, ROWS = TW + TX, HBYTES = ROWS * 64, SBYTES = 2 * HBYTES;
constexpr int LPH = HBYTES / 16 / NT8;  // loads per thread and half-step (4)
typedef int v4i __attribute__((ext_vector_type(4)));

#define G8_MF(t, F, i, j) "v_mfma_f32_16x16x32_" t " %[c" #i #j "], %[" #F "w" #i "], %[" #F "x" #j "], %[c" #i #j "]\n"
#define G8_MF4(t, F, i) G8_MF(t, F, i, 0) G8_MF(t, F, i, 1) G8_MF(t, F, i, 2) G8_MF(t, F, i, 3)
#define G8_R(N, wx, i, P, o) "ds_read_b128 %[" #N #wx #i "], %[" #P "] offset:" #o "\n"
#define G8_M0(c, MB) "s_add_u32 m0, %[" #MB "], " #c "*1024\n"
#define G8_BL(c) "buffer_load_dwordx4 %[vo" #c "], %[rsrc], %[soff] offen lds\n"
#define G8_ADV "s_add_u32 %[soff], %[soff], 64\n s_cmp_ge_u32 %[soff], %[wrap]\n s_cselect_b32 %[tmp], %[wrap], 0\n" \
               "s_sub_u32 %[soff], %[soff], %[tmp]\n"
#define G8_LDH(MB) G8_M0(0, MB) "s_nop 0\n" G8_BL(0) G8_M0(1, MB) "s_nop 0\n" G8_BL(1) G8_M0(2, MB) "s_nop 0\n"   \
  G8_BL(2) G8_M0(3, MB) "s_nop 0\n" G8_BL(3) G8_ADV
// the 4 MFMAs of weight fragment i with one other instruction (or none) after each of the first three
#define G8_ROW(t, F, i, s0, s1, s2) G8_MF(t, F, i, 0) s0 G8_MF(t, F, i, 1) s1 G8_MF(t, F, i, 2) s2 G8_MF(t, F, i, 3)
// half-step: 32 MFMAs of F; the next half's 12 reads into N during the first four rows,
// with LD the 4 loads of half region MB during rows 4..7
#define G8_HALF_X(t, F, N, PW, PX, L0, L1, L2, L3, B0, B1, B2, B3, ADV)                                    \
  G8_ROW(t, F, 0, G8_R(N, w, 0, PW, 0), G8_R(N, x, 0, PX, 0), G8_R(N, w, 1, PW, 1024))                      \
  G8_ROW(t, F, 1, G8_R(N, x, 1, PX, 1024), G8_R(N, w, 2, PW, 2048), G8_R(N, x, 2, PX, 2048))                \
  G8_ROW(t, F, 2, G8_R(N, w, 3, PW, 3072), G8_R(N, x, 3, PX, 3072), G8_R(N, w, 4, PW, 4096))                \
  G8_ROW(t, F, 3, G8_R(N, w, 5, PW, 5120), G8_R(N, w, 6, PW, 6144), G8_R(N, w, 7, PW, 7168))                \
  G8_ROW(t, F, 4, L0, B0, "") G8_ROW(t, F, 5, L1, B1, "") G8_ROW(t, F, 6, L2, B2, "") G8_ROW(t, F, 7, L3, B3, "") \
  ADV "s_waitcnt lgkmcnt(0)\n"
#define G8_HALF_RD(t, F, N, PW, PX) G8_HALF_X(t, F, N, PW, PX, "", "", "", "", "", "", "", "", "")
#define G8_HALF_RD_LD(t, F, N, PW, PX, MB)                                                                  \
  G8_HALF_X(t, F, N, PW, PX, G8_M0(0, MB), G8_M0(1, MB), G8_M0(2, MB), G8_M0(3, MB), G8_BL(0), G8_BL(1),    \
            G8_BL(2), G8_BL(3), G8_ADV)
#define G8_HALF(t, F) G8_MF4(t, F, 0) G8_MF4(t, F, 1) G8_MF4(t, F, 2) G8_MF4(t, F, 3) \
                      G8_MF4(t, F, 4) G8_MF4(t, F, 5) G8_MF4(t, F, 6) G8_MF4(t, F, 7)
#define G8_RD_ALL(N, PW, PX) G8_R(N, w, 0, PW, 0) G8_R(N, w, 1, PW, 1024) G8_R(N, w, 2, PW, 2048)          \
  G8_R(N, w, 3, PW, 3072) G8_R(N, w, 4, PW, 4096) G8_R(N, w, 5, PW, 5120) G8_R(N, w, 6, PW, 6144)          \
  G8_R(N, w, 7, PW, 7168) G8_R(N, x, 0, PX, 0) G8_R(N, x, 1, PX, 1024) G8_R(N, x, 2, PX, 2048)             \
  G8_R(N, x, 3, PX, 3072) "s_waitcnt lgkmcnt(0)\n"
#define G8_IF(D) "s_add_u32 %[tmp], %[t], " #D "\n s_cmp_lt_u32 %[tmp], %[nk]\n"
// per half region 4 loads per thread: the wait counts below are 8 (two halves) and 4
#define G8_LOOP(t)                                                                                       \
  G8_LDH(m00) G8_LDH(m01)                                                                                \
  "s_cmp_lt_u32 1, %[nk]\n s_cbranch_scc0 .Lg8one%=\n" G8_LDH(m10) G8_LDH(m11)                          \
  "s_waitcnt vmcnt(8)\n s_branch .Lg8pro%=\n"                                                          \
  ".Lg8one%=:\n s_waitcnt vmcnt(0)\n"                                                                  \
  ".Lg8pro%=:\n s_barrier\n" G8_RD_ALL(f0, a00, x00) "s_nop 4\n s_mov_b32 %[t], 0\n"                   \
  ".Lg8top%=:\n" G8_IF(1) "s_cbranch_scc0 .Lg8sa0%=\n s_waitcnt vmcnt(8)\n s_branch .Lg8sb0%=\n"       \
  ".Lg8sa0%=:\n s_waitcnt vmcnt(0)\n .Lg8sb0%=:\n s_barrier\n"                                         \
  G8_IF(2) "s_cbranch_scc0 .Lg8a0n%=\n" G8_HALF_RD_LD(t, f0, f1, a01, x01, m00) "s_branch .Lg8a0d%=\n"  \
  ".Lg8a0n%=:\n" G8_HALF_RD(t, f0, f1, a01, x01) ".Lg8a0d%=:\n"                                        \
  G8_IF(1) "s_cbranch_scc0 .Lg8last%=\n"                                                               \
  G8_IF(2) "s_cbranch_scc0 .Lg8ma0%=\n s_waitcnt vmcnt(8)\n s_branch .Lg8mb0%=\n"                      \
  ".Lg8ma0%=:\n s_waitcnt vmcnt(4)\n .Lg8mb0%=:\n s_barrier\n"                                         \
  G8_IF(2) "s_cbranch_scc0 .Lg8b0n%=\n" G8_HALF_RD_LD(t, f1, f0, a10, x10, m01) "s_branch .Lg8b0d%=\n"  \
  ".Lg8b0n%=:\n" G8_HALF_RD(t, f1, f0, a10, x10) ".Lg8b0d%=:\n"                                        \
  G8_IF(2) "s_cbranch_scc0 .Lg8sa1%=\n s_waitcnt vmcnt(8)\n s_branch .Lg8sb1%=\n"                      \
  ".Lg8sa1%=:\n s_waitcnt vmcnt(0)\n .Lg8sb1%=:\n s_barrier\n"                                         \
  G8_IF(3) "s_cbranch_scc0 .Lg8a1n%=\n" G8_HALF_RD_LD(t, f0, f1, a11, x11, m10) "s_branch .Lg8a1d%=\n"  \
  ".Lg8a1n%=:\n" G8_HALF_RD(t, f0, f1, a11, x11) ".Lg8a1d%=:\n"                                        \
  G8_IF(2) "s_cbranch_scc0 .Lg8last%=\n"                                                               \
  G8_IF(3) "s_cbranch_scc0 .Lg8ma1%=\n s_waitcnt vmcnt(8)\n s_branch .Lg8mb1%=\n"                      \
  ".Lg8ma1%=:\n s_waitcnt vmcnt(4)\n .Lg8mb1%=:\n s_barrier\n"                                         \
  G8_IF(3) "s_cbranch_scc0 .Lg8b1n%=\n" G8_HALF_RD_LD(t, f1, f0, a00, x00, m11) "s_branch .Lg8b1d%=\n"  \
  ".Lg8b1n%=:\n" G8_HALF_RD(t, f1, f0, a00, x00) ".Lg8b1d%=:\n"                                        \
  "s_add_u32 %[t], %[t], 2\n s_branch .Lg8top%=\n"                                                     \
  ".Lg8last%=:\n" G8_HALF(t, f1) "s_nop 15\n s_nop 15\n s_nop 15\n"

#define G8_C4(i) [c##i##0] "+a"(acc[i][0]), [c##i##1] "+a"(acc[i][1]), [c##i##2] "+a"(acc[i][2]), [c##i##3] "+a"(acc[i][3])
#define G8_W8(n, v) [n##0] "=&v"(v[0]), [n##1] "=&v"(v[1]), [n##2] "=&v"(v[2]), [n##3] "=&v"(v[3]), \
  [n##4] "=&v"(v[4]), [n##5] "=&v"(v[5]), [n##6] "=&v"(v[6]), [n##7] "=&v"(v[7])
#define G8_X4(n, v) [n##0] "=&v"(v[0]), [n##1] "=&v"(v[1]), [n##2] "=&v"(v[2]), [n##3] "=&v"(v[3])
#define G8_OUTS G8_C4(0), G8_C4(1), G8_C4(2), G8_C4(3), G8_C4(4), G8_C4(5), G8_C4(6), G8_C4(7), \
  G8_W8(f0w, f0w), G8_X4(f0x, f0x), G8_W8(f1w, f1w), G8_X4(f1x, f1x), [t] "=&s"(st), [tmp] "=&s"(stmp), \
  [soff] "+s"(soff)
#define G8_INS [vo0] "v"(vo[0]), [vo1] "v"(vo[1]), [vo2] "v"(vo[2]), [vo3] "v"(vo[3]),                           \
  [a00] "v"(aw[0][0]), [a01] "v"(aw[0][1]), [a10] "v"(aw[1][0]), [a11] "v"(aw[1][1]),                          \
  [x00] "v"(ax[0][0]), [x01] "v"(ax[0][1]), [x10] "v"(ax[1][0]), [x11] "v"(ax[1][1]),                          \
  [m00] "s"(mb[0][0]), [m01] "s"(mb[0][1]), [m10] "s"(mb[1][0]), [m11] "s"(mb[1][1]),                          \
  [rsrc] "s"(rsrc), [wrap] "s"(wrap), [nk] "s"(nk)

template <typename TI>
DEVI void main_loop(f32x4_v (&acc)[8][4], const uint32_t (&vo)[LPH], const uint32_t (&aw)[2][2],
                    const uint32_t (&ax)[2][2], const uint32_t (&mb)[2][2], v4i rsrc, uint32_t soff, uint32_t wrap,
                    uint32_t nk) {
  v4i f0w[8], f0x[4], f1w[8], f1x[4];
  uint32_t st, stmp;
  if constexpr (std::is_same<TI, f16_t>::value)
    asm volatile(G8_LOOP("f16") : G8_OUTS : G8_INS : "memory", "m0", "scc");
  else
    asm volatile(G8_LOOP("bf16") : G8_OUTS : G8_INS : "memory", "m0", "scc");
}
#undef G8_MF
#undef G8_MF4
#undef G8_R
#undef G8_M0
#undef G8_BL
#undef G8_ADV
#undef G8_LDH
#undef G8_ROW
#undef G8_HALF_X
#undef G8_HALF_RD
#undef G8_HALF_RD_LD
#undef G8_HALF
#undef G8_RD_ALL
#undef G8_IF
#undef G8_LOOP
#undef G8_C4
#undef G8_W8
#undef G8_X4
#undef G8_OUTS
#undef G8_INS
}  // namespace g8

// One 256 x 256 output tile of g: block bx of the product's tiles (bx < tiles).
template <typename TI, int EPI>
DEVI void gemm8_tile(const GemmArgs &g, const int bx) {
  using namespace g8;
  __shared__ __align__(1024) char sm[2 * SBYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 2, wm = wave & 3;  // weight half, token quarter
  const int mt = (g.M + TX - 1) / TX, ntl = (g.N + TW - 1) / TW;
  constexpr int GM = 8;
  const int tile = remap_tile2(bx, mt * ntl);
  const int band = tile / (GM * ntl), in_band = tile % (GM * ntl);
  const int bm = min(GM, mt - band * GM);
  const int tm = band * GM + in_band % bm, tn = in_band / bm;
  const int m0 = tm * TX, n0 = tn * TW;
  int kbeg = 0, kend = g.K;
  if (g.ksplit > 1) {
    const int per = ((g.K + g.ksplit - 1) / g.ksplit + BK - 1) / BK * BK;
    kbeg = blockIdx.z * per;
    kend = min(g.K, kbeg + per);
  }
  const int nk = (kend - kbeg + BK - 1) / BK;
  // waves 0-3 stream weight rows, waves 4-7 token rows; load c of a half covers rows
  // 16 (wave LPH + c) .. +15, lane l row + l / 4, chunk position l % 4
  const bool tok = wave >= 4;
  uint32_t vo[LPH];
#pragma unroll
  for (int c = 0; c < LPH; ++c) {
    const int row = (wave * LPH + c) * 16 + (lane >> 2);
    const int kc = (lane & 3) ^ ((row >> 1) & 2);
    if (!tok) {
      const int gr = n0 + row;
      vo[c] = gr < g.N ? (uint32_t)(((long)gr * g.ldb + kc * 8) * 2) : OOB;
    } else {
      const int gr = m0 + row - TW;
      vo[c] = gr < g.M ? (uint32_t)(((long)gr * g.lda + kc * 8) * 2) : OOB;
    }
  }
  v4i rsrc;
  uint32_t soff, wrap;
  {
    const void *base = tok ? g.A : g.B;
    const int ka = g.a_kwrap > 0 ? g.a_kwrap : g.K;
    const uint32_t bytes = tok ? (uint32_t)(((long)(g.M - 1) * g.lda + ka) * 2)
                               : (uint32_t)(((long)(g.N - 1) * g.ldb + g.K) * 2);
    const uint64_t ad = (uint64_t)(uintptr_t)base;
    rsrc = v4i{(int)(uint32_t)ad, (int)(uint32_t)(ad >> 32), (int)bytes, RSRC_W3};
    const bool wr = tok && g.a_kwrap > 0;
    wrap = wr ? (uint32_t)g.a_kwrap * 2 : 0x7fffffffu;
    soff = (uint32_t)(wr ? kbeg % g.a_kwrap : kbeg) * 2;
  }
  const uint32_t smb = (uint32_t)(uintptr_t)(lds_void *)sm;
  f32x4_v acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  const int lr = lane & 15, lq = lane >> 4;
  const uint32_t cs = (uint32_t)((lq ^ ((lr >> 1) & 2)) << 4);
  uint32_t aw[2][2], ax[2][2], mb[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t base = smb + s * SBYTES + h * HBYTES;
      aw[s][h] = base + (wn * 128 + lr) * 64 + cs;
      ax[s][h] = base + (TW + wm * 64 + lr) * 64 + cs;
      mb[s][h] = (uint32_t)__builtin_amdgcn_readfirstlane(base + wave * LPH * 1024);
    }
  if (nk > 0)
    main_loop<TI>(acc, vo, aw, ax, mb, rsrc, (uint32_t)__builtin_amdgcn_readfirstlane(soff),
                  (uint32_t)__builtin_amdgcn_readfirstlane(wrap), (uint32_t)__builtin_amdgcn_readfirstlane(nk));
  float4 pre[4][4];
#pragma unroll
  for (int qn = 0; qn < 2; ++qn) {
    f32x4_v q[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) q[i][j] = acc[qn * 4 + i][j];
    const int mq = m0 + wm * 64, nq = n0 + wn * 128 + qn * 64;
    gemm2_epilogue<128, EPI, false>(g, q, mq, nq / 128 * 128, nq / 128, 0, (nq / 64) & 1, lr, lq, pre);
  }
}

template <typename TI, int EPI>
__global__ __launch_bounds__(g8::NT8, 1) void gemm8_kernel(const GemmArgs g) {
  gemm8_tile<TI, EPI>(g, blockIdx.x);
}

// Several products with the same epilogue in one launch: problem p owns blocks
// beg[p] .. beg[p] + its tile count - 1; every beg[p] is a multiple of 8, so that a
// problem's block index modulo 8 is still the XCD that runs it (the tile remap keeps each
// XCD's tiles together); blocks between problems exit at once.
template <typename TI, int EPI>
__global__ __launch_bounds__(g8::NT8, 1) void gemm8_group_kernel(const GemmGroup gg) {
  const int bx = blockIdx.x;
  int p = 0;
  while (p + 1 < gg.n && bx >= gg.beg[p + 1]) ++p;
  const GemmArgs &g = gg.g[p];
  const int i = bx - gg.beg[p];
  if (i >= ((g.M + g8::TX - 1) / g8::TX) * ((g.N + g8::TW - 1) / g8::TW)) return;
  gemm8_tile<TI, EPI>(g, i);
}

#define G8_INST(TI)                                                      \
  template __global__ void gemm8_kernel<TI, EPI_STORE>(const GemmArgs);     \
  template __global__ void gemm8_kernel<TI, EPI_STORE_F32>(const GemmArgs); \
  template __global__ void gemm8_kernel<TI, EPI_ADD_F32>(const GemmArgs);   \
  template __global__ void gemm8_kernel<TI, EPI_SWIGLU>(const GemmArgs);    \
  template __global__ void gemm8_kernel<TI, EPI_CE>(const GemmArgs);        \
  template __global__ void gemm8_kernel<TI, EPI_PROBS>(const GemmArgs);   \
  template __global__ void gemm8_kernel<TI, 100>(const GemmArgs);
G8_INST(bf16_t)
G8_INST(f16_t)
#undef G8_INST
template __global__ void gemm8_group_kernel<f16_t, EPI_SWIGLU>(const GemmGroup);
template __global__ void gemm8_group_kernel<bf16_t, EPI_SWIGLU>(const GemmGroup);

template <typename TI, int EPI> hipError_t launch8_e(const GemmArgs &g, hipStream_t st) {
  const int tiles = ((g.M + g8::TX - 1) / g8::TX) * ((g.N + g8::TW - 1) / g8::TW);
  hipLaunchKernelGGL((gemm8_kernel<TI, EPI>), dim3(tiles, 1, g.ksplit), dim3(g8::NT8), 0, st, g);
  return hipGetLastError();
}
template <typename TI> hipError_t launch8(int epi, const GemmArgs &g, hipStream_t st) {
  if (g.ksplit > 1) return launch8_e<TI, 100>(g, st);
  switch (epi) {
    case EPI_STORE: return launch8_e<TI, EPI_STORE>(g, st);
    case EPI_STORE_F32: return launch8_e<TI, EPI_STORE_F32>(g, st);
    case EPI_ADD_F32: return launch8_e<TI, EPI_ADD_F32>(g, st);
    case EPI_SWIGLU: return launch8_e<TI, EPI_SWIGLU>(g, st);
    case EPI_CE: return launch8_e<TI, EPI_CE>(g, st);
    case EPI_PROBS: return launch8_e<TI, EPI_PROBS>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ttt_g2
using namespace ttt_g2;

// bf16, both operands k-contiguous with 16-byte aligned rows, K a multiple of
// 64.  g.ksplit > 1 writes fp32 partials to g.ws (the caller reduces them in a
// fixed order).
hipError_t gemm_dma_launch(bool f16, int epi, const GemmArgs &g, hipStream_t st) {
  return f16 ? launch5<f16_t>(epi, g, st) : launch5<bf16_t>(epi, g, st);
}

// The 256 x 256 tile (same operand conditions as gemm_dma_launch; no EPI_SGD).
hipError_t gemm_dma256_launch(bool f16, int epi, const GemmArgs &g, hipStream_t st) {
  return f16 ? launch8<f16_t>(epi, g, st) : launch8<bf16_t>(epi, g, st);
}

// Several SwiGLU products of the 256 x 256 tile in one launch (each meets the conditions
// of gemm_dma_launch and has ksplit 1); fills gg.beg.
hipError_t gemm_dma256_group_launch(bool f16, int epi, GemmGroup &gg, hipStream_t st) {
  if (epi != EPI_SWIGLU || gg.n < 1 || gg.n > GEMM_GROUP_MAX) return hipErrorInvalidValue;
  int blocks = 0;
  for (int p = 0; p < gg.n; ++p) {
    const GemmArgs &g = gg.g[p];
    if (g.ksplit > 1) return hipErrorInvalidValue;
    gg.beg[p] = blocks;
    const int tiles = ((g.M + g8::TX - 1) / g8::TX) * ((g.N + g8::TW - 1) / g8::TW);
    blocks += (tiles + 7) / 8 * 8;
  }
  if (f16)
    hipLaunchKernelGGL((gemm8_group_kernel<f16_t, EPI_SWIGLU>), dim3(blocks), dim3(g8::NT8), 0, st, gg);
  else
    hipLaunchKernelGGL((gemm8_group_kernel<bf16_t, EPI_SWIGLU>), dim3(blocks), dim3(g8::NT8), 0, st, gg);
  return hipGetLastError();
}
