// Causal sliding-window attention over key/value rings, forward and backward.
//
// Query p attends keys j with p - k < j <= p (the window of the reading
// notes, section 5 and Eq. 1).  Keys of earlier chunks come from the ring and
// are constants of the inner step; only the chunk's own keys and values get
// gradients.
//
// MFMA orientation (16x16x32 bf16 tiles, see common.h): scores are produced
// transposed, S^T = K Q^T, so each lane holds 4 keys of one query; that lane
// layout is exactly the reduction-dim fragment of the next product
// O^T = V^T P^T once the 32 keys of a step are taken in the order
// (4g..4g+3, 16+4g..16+4g+3) for lane group g, which is why V (and K for dQ)
// are read transposed from LDS.  Softmax statistics stay per lane (one query).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "attn.h"

namespace {

constexpr int NT = 256;

// Global -> registers -> LDS copy of a ROWS x COLSP tile (COLSP a multiple of
// the 16-byte vector), zero outside rows_valid x cols.
template <typename T, int ROWS, int COLSP> struct TileIO {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int VPR = COLSP / VE;
  static constexpr int TOT = ROWS * VPR;
  static constexpr int PER = (TOT + NT - 1) / NT;
  uint4 v[PER];
  DEVI void load(const T *g, long gld, int rows_valid, int cols, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int idx = tid + i * NT;
      int r = idx / VPR, c = (idx % VPR) * VE;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (idx < TOT && r < rows_valid) {
        if (c + VE <= cols) {
          x = *reinterpret_cast<const uint4 *>(g + (long)r * gld + c);
        } else if (c < cols) {
          T tmp[VE];
#pragma unroll
          for (int e = 0; e < VE; ++e) tmp[e] = (c + e < cols) ? g[(long)r * gld + c + e] : T(0);
          x = *reinterpret_cast<const uint4 *>(tmp);
        }
      }
      v[i] = x;
    }
  }
  // All ROWS rows valid and cols a multiple of VE: columns at or past cols read as zero
  // through a select, with no per-lane branches (a divergent branch around a load
  // makes the compiler wait for every earlier load at the join).
  DEVI void load_rows(const T *g, long gld, int cols, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / VPR, c = (idx % VPR) * VE;
      const bool ok = (idx < TOT) && (c < cols);
      const long o = ok ? (long)r * gld + c : 0;
      const uint4 x = *reinterpret_cast<const uint4 *>(g + o);
      v[i] = ok ? x : make_uint4(0, 0, 0, 0);
    }
  }
  DEVI void store(T *sm, int sld, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int idx = tid + i * NT;
      if (idx < TOT) {
        int r = idx / VPR, c = (idx % VPR) * VE;
        *reinterpret_cast<uint4 *>(sm + r * sld + c) = v[i];
      }
    }
  }
};

// Branch-free variant for tiles whose rows are all valid and whose valid
// columns (COLS) are known at compile time: every lane loads from an
// in-bounds address and zeroes the padding columns with a select, so the
// compiler emits straight-line loads.
template <typename T, int ROWS, int COLSP, int COLS> struct FullTile {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int VPR = COLSP / VE;
  static constexpr int TOT = ROWS * VPR;
  static constexpr int PER = (TOT + NT - 1) / NT;
  uint4 v[PER];
  DEVI void load(const T *g, long gld, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / VPR, c = (idx % VPR) * VE;
      const bool ok = (idx < TOT) && (c < COLS);
      const uint32_t o = ok ? (uint32_t)(r * (int)gld + c) : 0u;  // element offset (< 2^31)
      const uint4 x = *reinterpret_cast<const uint4 *>(g + o);
      v[i] = ok ? x : make_uint4(0, 0, 0, 0);
    }
  }
  DEVI void store(T *sm, int sld, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      if (TOT % NT == 0 || idx < TOT) {
        const int r = idx / VPR, c = (idx % VPR) * VE;
        *reinterpret_cast<uint4 *>(sm + r * sld + c) = v[i];
      }
    }
  }
};

// Ring tile loader through a buffer descriptor: per-lane byte offsets are
// computed once and the tile position enters as the scalar offset, so the
// prefetch of the next tile never waits on registers the current tile reuses.
// Columns at or past COLS (padding) read an offset beyond the extent -> 0.
template <typename T, int ROWS, int COLSP, int COLS> struct RingTile {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int VPR = COLSP / VE;
  static constexpr int TOT = ROWS * VPR;
  static constexpr int PER = (TOT + NT - 1) / NT;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff[PER];
  uint4 v[PER];
  DEVI void init(const T *plane, uint32_t plane_bytes, int gld, int tid) {
    rs = __builtin_amdgcn_make_buffer_rsrc((void *)plane, (short)0, plane_bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / VPR, c = (idx % VPR) * VE;
      voff[i] = (idx < TOT && c < COLS) ? (uint32_t)((r * gld + c) * (int)sizeof(T)) : 0x7FFFFF00u;
    }
  }
  DEVI void load(int soff_bytes) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], soff_bytes, 0));
  }
  DEVI void store(T *sm, int sld, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      if (TOT % NT == 0 || idx < TOT) {
        const int r = idx / VPR, c = (idx % VPR) * VE;
        *reinterpret_cast<uint4 *>(sm + r * sld + c) = v[i];
      }
    }
  }
};

template <int HD> struct Dims {
  static constexpr int HDP = (HD + 31) / 32 * 32;  // reduction length of q.k, zero padded
  static constexpr int NC = HDP / 32;
  static constexpr int NH = HD / 16;               // 16-wide output tiles over hd
};

template <typename T> constexpr int pad_el() { return 16 / (int)sizeof(T); }

// ======================================================================= forward
// grid (ceil(n/128), H); 4 waves x 32 queries.
template <typename T, int HD, typename TO>
__global__ __launch_bounds__(NT) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int HDP = Dims<HD>::HDP, NC = Dims<HD>::NC, NH = Dims<HD>::NH;
  constexpr int LDK = HDP + pad_el<T>(), LDV = 64 + pad_el<T>();
  __shared__ __align__(16) T smK[2][64 * LDK];
  __shared__ __align__(16) T smV[2][HD * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4, g4 = lg * 4;
  const int h = blockIdx.y, q_lo = blockIdx.x * 128;
  const int pos0 = *a.pos0;
  const int qw = q_lo + wave * 32;
  const T *Q = reinterpret_cast<const T *>(a.q);
  const T *Kr = reinterpret_cast<const T *>(a.K) + (long)h * a.R * HD;
  const T *Vr = reinterpret_cast<const T *>(a.Vt) + (long)h * HD * a.R;

  Frag<T> qf[2][NC];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      int q = qw + qs * 16 + lr, col = c * 32 + lg * 8;
      if (q < a.n && col < HD)
        load_frag(qf[qs][c], Q + (long)q * a.d + h * HD + col);
      else
        zero_frag(qf[qs][c]);
    }
  // the query fragments are complete before the tile loop, so its waits need
  // only cover the tile prefetch
  __builtin_amdgcn_s_waitcnt(0);

  const int p_first = pos0 + q_lo;
  const int p_last = pos0 + min(q_lo + 127, a.n - 1);
  const int jtw = max(0, p_first - a.window + 1) & ~63;
  const int ntw = (p_last - jtw) / 64 + 1;
  const int sp = blockIdx.z;
  const int t_lo = ntw * sp / a.nsplit, t_hi = ntw * (sp + 1) / a.nsplit;
  const int jt0 = jtw + 64 * t_lo;
  const int ntile = t_hi - t_lo;
  const int pw_min = pos0 + qw, pw_max = pos0 + qw + 31;
  const float sl2 = a.scale * LOG2E_F;

  float m_[2] = {-INFINITY, -INFINITY}, l_[2] = {0.f, 0.f};
  f32x4_v O[NH][2];
#pragma unroll
  for (int hs = 0; hs < NH; ++hs)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) O[hs][qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  const uint32_t plane = (uint32_t)((long)a.R * HD * sizeof(T));
  RingTile<T, 64, HDP, HD> kio;
  RingTile<T, HD, 64, 64> vio;
  kio.init(Kr, plane, HD, tid);
  vio.init(Vr, plane, a.R, tid);
  if (ntile > 0) {
    kio.load((jt0 % a.R) * HD * (int)sizeof(T));
    vio.load((jt0 % a.R) * (int)sizeof(T));
    kio.store(smK[0], LDK, tid);
    vio.store(smV[0], LDV, tid);
  }
  __syncthreads();

  for (int t = 0; t < ntile; ++t) {
    const int cur = t & 1;
    const int jt = jt0 + t * 64;
    if (t + 1 < ntile) {
      const int sn = (jt + 64) % a.R;
      kio.load(sn * HD * (int)sizeof(T));
      vio.load(sn * (int)sizeof(T));
    }
    const bool any = (jt <= pw_max) && (jt + 63 > pw_min - a.window);
    const bool full = (jt + 63 <= pw_min) && (jt > pw_max - a.window);
    if (any) {
      f32x4_v S[4][2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) S[ks][qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      const T *sk = smK[cur];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        Frag<T> kf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) load_frag(kf[ks], sk + (ks * 16 + lr) * LDK + c * 32 + lg * 8);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) mma(S[ks][qs], kf[ks], qf[qs][c]);
      }
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const int p = pos0 + qw + qs * 16 + lr;
        float mloc = -INFINITY;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s = S[ks][qs][r] * sl2;
            if (!full) {
              int j = jt + ks * 16 + g4 + r;
              if (j > p || j <= p - a.window) s = -INFINITY;
            }
            S[ks][qs][r] = s;
            mloc = fmaxf(mloc, s);
          }
        mloc = group4_max(mloc);
        const float mnew = fmaxf(m_[qs], mloc);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = fast_exp2(m_[qs] - muse);
        m_[qs] = mnew;
        l_[qs] *= alpha;
#pragma unroll
        for (int hs = 0; hs < NH; ++hs) O[hs][qs] *= alpha;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float pv = fast_exp2(S[ks][qs][r] - muse);
            S[ks][qs][r] = pv;
            l_[qs] += pv;
          }
      }
      const T *sv = smV[cur];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        Frag<T> pf[2];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          float x[8] = {S[2 * c2][qs][0],     S[2 * c2][qs][1],     S[2 * c2][qs][2],     S[2 * c2][qs][3],
                        S[2 * c2 + 1][qs][0], S[2 * c2 + 1][qs][1], S[2 * c2 + 1][qs][2], S[2 * c2 + 1][qs][3]};
          pack_frag(pf[qs], x);
        }
#pragma unroll
        for (int hs = 0; hs < NH; ++hs) {
          Frag<T> vf;
          const T *row = sv + (hs * 16 + lr) * LDV + c2 * 32 + g4;
          load_frag2(vf, row, row + 16);
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) mma(O[hs][qs], vf, pf[qs]);
        }
      }
    }
    if (t + 1 < ntile) {
      kio.store(smK[cur ^ 1], LDK, tid);
      vio.store(smV[cur ^ 1], LDV, tid);
    }
    __syncthreads();
  }

  TO *Out = reinterpret_cast<TO *>(a.o);
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const float lt = group4_sum(l_[qs]);
    const int q = qw + qs * 16 + lr;
    if (q < a.n) {
      // a split may see no key of this query: weight 0 in the merge
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse = lt > 0.f ? m_[qs] + log2f(lt) : -INFINITY;
      if (a.nsplit == 1) {
#pragma unroll
        for (int hs = 0; hs < NH; ++hs) {
          float v[4] = {O[hs][qs][0] * inv, O[hs][qs][1] * inv, O[hs][qs][2] * inv, O[hs][qs][3] * inv};
          store4<TO>(Out + (long)q * a.d + h * HD + hs * 16 + g4, v);
        }
        if (lg == 0) a.lse2[(long)h * a.ldl + q] = lse;
      } else {
        float *po = a.ws + (long)sp * a.n * a.d;
#pragma unroll
        for (int hs = 0; hs < NH; ++hs) {
          float v[4] = {O[hs][qs][0] * inv, O[hs][qs][1] * inv, O[hs][qs][2] * inv, O[hs][qs][3] * inv};
          store4<float>(po + (long)q * a.d + h * HD + hs * 16 + g4, v);
        }
        if (lg == 0) a.ws[(long)a.nsplit * a.n * a.d + ((long)sp * a.H + h) * a.ldl + q] = lse;
      }
    }
  }
}

// out[q, h, :] = sum_s 2^(lse_s - lse) O_s[q, h, :],  lse = log2 sum_s 2^lse_s  (fixed order in s).
// nsplit <= MERGE_MAX.  The loads of all splits are issued before they are combined (a thread
// otherwise waits for one partial after the other, which dominates when there are few rows).
constexpr int MERGE_MAX = 32;
template <typename T>
__global__ __launch_bounds__(256) void attn_fwd_merge_kernel(const AttnArgs a, int hd) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int dq4 = a.d / 4;
  if (idx >= (long)a.n * dq4) return;
  const int q = idx / dq4, col = (idx % dq4) * 4, h = col / hd;
  const float *L = a.ws + (long)a.nsplit * a.n * a.d;
  float ls[MERGE_MAX];
#pragma unroll
  for (int s = 0; s < MERGE_MAX; ++s) {
    const int sc = min(s, a.nsplit - 1);
    const float x = L[((long)sc * a.H + h) * a.ldl + q];
    ls[s] = s < a.nsplit ? x : -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < MERGE_MAX; ++s) mx = fmaxf(mx, ls[s]);
  float den = 0.f, v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < MERGE_MAX / 8; ++g) {
    if (8 * g >= a.nsplit) break;
    float4 o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sc = min(8 * g + u, a.nsplit - 1);
      o[u] = *reinterpret_cast<const float4 *>(a.ws + ((long)sc * a.n + q) * a.d + col);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (8 * g + u >= a.nsplit) break;
      const float l = ls[8 * g + u];
      const float w = (l == -INFINITY) ? 0.f : exp2f(l - mx);
      den += w;
      v[0] += w * o[u].x; v[1] += w * o[u].y; v[2] += w * o[u].z; v[3] += w * o[u].w;
    }
  }
  const float inv = 1.f / den;
  v[0] *= inv; v[1] *= inv; v[2] *= inv; v[3] *= inv;
  store4<T>(reinterpret_cast<T *>(a.o) + (long)q * a.d + col, v);
  if (col % hd == 0) a.lse2[(long)h * a.ldl + q] = mx + log2f(den);
}

// dq[q, :] = scale-free sum over splits of the partial dQ (fixed order).
__global__ __launch_bounds__(256) void attn_dq_merge_kernel(const AttnArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long tot = (long)a.n * a.d / 4;
  if (idx >= tot) return;
  float4 acc = reinterpret_cast<const float4 *>(a.ws)[idx];
  for (int s = 1; s < a.nsplit; ++s) {
    const float4 x = reinterpret_cast<const float4 *>(a.ws + (long)s * a.n * a.d)[idx];
    acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
  }
  reinterpret_cast<float4 *>(a.dq)[idx] = acc;
}

// ======================================================= forward, 16-bit, bounded
// 64 queries per wave, 4 waves (256 queries) per work-group; grid
// (ceil(n/256), H, nsplit).  Key tiles of 32 are streamed from the rings
// straight into one LDS stage (buffer_load ... lds).  Each wave reads all
// fragments of the tile into registers, a barrier frees the stage, the next
// tile is streamed into it while the MFMAs and the softmax run on registers;
// latency is covered by the second resident work-group of the CU.
//
// Softmax without a running maximum: with QK-norm every query and key has
// Euclidean norm at most max|g| * sqrt(hd), so a scaled score never exceeds
// B = max|g_q| max|g_k| sqrt(hd) (in log2 units: times log2 e), a per-layer
// constant the host derives from the gains.  p = 2^(s - B) then lies in
// (2^-2B, 1] and needs no rescaling of the output accumulators; the log2-sum-
// exp is B + log2(sum p).  The host uses this kernel only when 2B stays far
// inside the fp32 exponent range.
//
// Operand type TF: bf16, or fp16 (three more mantissa bits for q, k, v and p;
// same MFMA rate).  With fp16, p is taken as 2^(s - B + 15): at most 2^15 (the
// scores overshoot B by rounding only), and for B <= 14.5 every weight, even of
// a query whose scores all sit at -B, stays a normal fp16 number.  The output O
// is written as fp16 (the O projection's operand) or the working dtype.
//
// LDS layouts (16-byte chunks):
//   K tile  [32 keys][KCH = 4 * ceil(hd/32) chunks], chunk c of key row r at
//           position c ^ X(r); chunks at or past hd/8 read as zero (the q.k
//           reduction is padded to a multiple of 32).
//   V^T tile [hd rows][4 chunks of 8 keys], chunk c of row r at c ^ ((r>>1)&3).
// Score tiles take key rows in the order 8*(i/4) + 4*ks + i%4 (i = MFMA row,
// ks = which of the two 16-row tiles), so each lane ends up with 8
// consecutive keys of one query: exactly one 16-byte V^T fragment for the
// P V product.  With these swizzles each 16-lane phase of a fragment read
// touches every bank group twice (no conflicts).
// log2 offset of the softmax weights kept in fp16 (none for bf16)
template <typename TF> struct P16Off { static constexpr float v = 0.f; };
template <> struct P16Off<f16_t> { static constexpr float v = 15.f; };

template <int HD> struct F2 {
  static constexpr int NC = (HD + 31) / 32;   // 32-deep steps of q.k
  static constexpr int KCH = 4 * NC;          // chunks per K row in LDS
  static constexpr int RC = HD / 8;           // chunks holding data
  static constexpr int NH = HD / 16;          // 16-row output tiles over hd
  static constexpr int KB = 32 * KCH * 16;    // bytes of a K tile
  static constexpr int VB = HD * 4 * 16;      // bytes of a V^T tile
  static constexpr int KINS = KB / 1024;      // 1 KiB DMA instructions per K tile
  static constexpr int INS = (KB + VB) / 1024;
  static constexpr int IPW = (INS + 3) / 4;   // per wave
};

template <int KCH> DEVI int kswz(int row) {
  int x = ((row >> 1) & 1) | (((row >> 3) & 1) << 1);
  if (KCH % 8 == 0) x |= (row & 1) << 2;
  return x;
}

template <int HD> struct F2Issue {
  using C = F2<HD>;
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t voff[C::IPW];
  int j0;
  DEVI void init(const void *Kp, const void *Vtp, int R, int wave, int lane) {
    rk = __builtin_amdgcn_make_buffer_rsrc((void *)Kp, (short)0, (uint32_t)R * HD * 2, BUF_RSRC_W3);
    rv = __builtin_amdgcn_make_buffer_rsrc((void *)Vtp, (short)0, (uint32_t)R * HD * 2, BUF_RSRC_W3);
    j0 = wave * C::IPW;
#pragma unroll
    for (int c = 0; c < C::IPW; ++c) {
      const int j = min(j0 + c, C::INS - 1);  // the last wave repeats the last chunk (same bytes)
      if (j < C::KINS) {
        const int s = j * 64 + lane, row = s / C::KCH, ch = (s % C::KCH) ^ kswz<C::KCH>(row);
        voff[c] = ch < C::RC ? (uint32_t)(row * HD * 2 + ch * 16) : BUF_OOB;
      } else {
        const int s = (j - C::KINS) * 64 + lane, row = s / 4, ch = (s % 4) ^ ((row >> 1) & 3);
        voff[c] = (uint32_t)(row * R * 2 + ch * 16);
      }
    }
  }
  // Streams the tile whose first key sits in ring slot `slot0` into `stage`.
  DEVI void run(char *stage, int slot0) const {
#pragma unroll
    for (int c = 0; c < C::IPW; ++c) {
      const int j = min(j0 + c, C::INS - 1);
      const bool isk = j < C::KINS;  // uniform across the wave
      lds_void *dst = (lds_void *)(stage + j * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isk ? rk : rv, dst, 16, voff[c], isk ? slot0 * HD * 2 : slot0 * 2, 0, 0);
    }
  }
};

// acc + the sum of the eight 16-bit values of a fragment (v_dot2 against (1, 1)).
DEVI float sum_pairs(const Frag<f16_t> &f, float acc) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const h2_t one = {(_Float16)1.f, (_Float16)1.f};
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, f.v.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, f.v.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, f.v.z), one, acc, false);
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, f.v.w), one, acc, false);
}
DEVI float sum_pairs(const Frag<bf16_t> &f, float acc) {
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  const b2_t one = {(__bf16)1.f, (__bf16)1.f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, f.v.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, f.v.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, f.v.z), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, f.v.w), one, acc, false);
}

template <int HD, typename TF> struct F2State {
  using C = F2<HD>;
  Frag<TF> qf[4][C::NC];
  f32x4_v O[C::NH][4];
  // row sums of the 16-bit weights.  Up to hd 80: an MFMA of each P fragment against a
  // fragment of ones, so every lane holds its query's sum over all keys (4 equal values);
  // above (where registers are short): per lane over its 8 keys, v_dot2 against (1, 1)
  static constexpr bool MSUM = C::NH <= 5;
  f32x4_v ls[4];
  float lsum[4];
  int kb[2], vb;  // per-lane byte offsets of the fragment reads (kb by parity of the 32-dim step)
};

// fp16 queries are stored pre-multiplied by scale * log2(e) (rounded to fp16) in the
// forward's registers, and the score accumulators start at -B, so that the MFMA gives
// the exponent s * scale * log2(e) - B directly and each weight costs one v_exp_f32;
// bf16 keeps its queries as they are (one more bf16 rounding of q would cost precision)
template <typename TF> struct F2Pre { static constexpr bool v = false; };
template <> struct F2Pre<f16_t> { static constexpr bool v = true; };

// Tiles t0 .. t1-1 of 32 keys.  FULL tiles have every (query, key) pair of
// the work-group inside the window; otherwise each wave skips the MFMAs of a
// tile none of its queries sees and masks the rest.  Every wave takes part in
// the streaming and the barriers of every tile.
template <int HD, typename TF, bool FULL>
DEVI void fwd2_range(F2State<HD, TF> &st, const F2Issue<HD> &is, char *stage, int t0, int t1, int ntile, int jt0,
                     int pq, int lr, int lg, const AttnArgs &a) {
  using C = F2<HD>;
  const float sl2 = a.scale * LOG2E_F, B = a.sbound - P16Off<TF>::v;
  constexpr bool PRE = F2Pre<TF>::v;
  const float s_init = PRE ? -B : 0.f;
  Frag<TF> ones;
  ones.v = std::is_same<TF, f16_t>::value ? make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u)
                                          : make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
  for (int t = t0; t < t1; ++t) {
    const int jt = jt0 + 32 * t;
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    Frag<TF> kf[2][C::NC], vf[C::NH];
#pragma unroll
    for (int c = 0; c < C::NC; ++c)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        kf[ks][c].v = *reinterpret_cast<const uint4 *>(stage + st.kb[c & 1] + (4 * ks * C::KCH + 4 * c) * 16);
#pragma unroll
    for (int hs = 0; hs < C::NH; ++hs)
      vf[hs].v = *reinterpret_cast<const uint4 *>(stage + C::KB + st.vb + hs * 16 * 64);
    lds_barrier();
    if (t + 1 < ntile) is.run(stage, (jt + 32) % a.R);
    if (!FULL && !((jt <= pq + 63) && (jt + 31 > pq - a.window))) continue;
    f32x4_v S[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) S[ks][qs] = f32x4_v{s_init, s_init, s_init, s_init};
#pragma unroll
    for (int c = 0; c < C::NC; ++c)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) mma(S[ks][qs], kf[ks][c], st.qf[qs][c]);
    Frag<TF> pf[4];
#pragma unroll
    for (int qs = 0; qs < 4; ++qs) {
      const int p = pq + qs * 16 + lr;
      float x[8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float e = PRE ? fast_exp2(S[ks][qs][r]) : fast_exp2(__builtin_fmaf(S[ks][qs][r], sl2, -B));
          if (!FULL) {
            const int j = jt + 8 * lg + 4 * ks + r;
            e = (j > p || j <= p - a.window) ? 0.f : e;
          }
          x[4 * ks + r] = e;
        }
      pack_frag(pf[qs], x);
      // row sums of the packed 16-bit p (the values the PV product uses)
      if constexpr (!F2State<HD, TF>::MSUM) st.lsum[qs] = sum_pairs(pf[qs], st.lsum[qs]);
    }
#pragma unroll
    for (int hs = 0; hs < C::NH; ++hs)
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) mma(st.O[hs][qs], vf[hs], pf[qs]);
    if constexpr (F2State<HD, TF>::MSUM) {
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) mma(st.ls[qs], ones, pf[qs]);
    }
  }
}

template <int HD, typename TF, typename TO>
__global__ __launch_bounds__(NT, 2) void attn_fwd2_kernel(const AttnArgs a) {
  using C = F2<HD>;
  __shared__ __align__(1024) char stage[C::KB + C::VB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4, g4 = lg * 4;
  // Work-groups are dealt to the 8 XCDs round-robin by linear index; remap so
  // that each XCD gets a contiguous range of (head, split, query block): the
  // query blocks of one head and key range run side by side on one XCD and
  // share its L2 for the key/value tiles.
  int qb, h, sp;
  {
    const int gx = gridDim.x, total = gx * gridDim.y * gridDim.z;
    const int i = blockIdx.x + gx * (blockIdx.y + gridDim.y * blockIdx.z);
    const int q8 = total / 8, rem = total % 8, x = i % 8;
    const int m = x * q8 + min(x, rem) + i / 8;
    qb = m % gx;
    sp = (m / gx) % a.nsplit;
    h = m / (gx * a.nsplit);
  }
  const int q_lo = qb * 256;
  const int pos0 = *a.pos0;
  const int qw = q_lo + wave * 64;
  const TF *Q = reinterpret_cast<const TF *>(a.q);

  F2State<HD, TF> st;
#pragma unroll
  for (int qs = 0; qs < 4; ++qs)
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      const int q = qw + qs * 16 + lr, col = c * 32 + lg * 8;
      if (q < a.n && col < HD)
        load_frag(st.qf[qs][c], Q + (long)q * a.d + h * HD + col);
      else
        zero_frag(st.qf[qs][c]);
    }
  if constexpr (F2Pre<TF>::v) {
    // q <- fp16(q * scale * log2 e)
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    const _Float16 sc = (_Float16)(a.scale * LOG2E_F);
    const h2_t s2 = {sc, sc};
#pragma unroll
    for (int qs = 0; qs < 4; ++qs)
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        uint4 v = st.qf[qs][c].v;
        v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, v.x) * s2);
        v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, v.y) * s2);
        v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, v.z) * s2);
        v.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, v.w) * s2);
        st.qf[qs][c].v = v;
      }
  }
#pragma unroll
  for (int qs = 0; qs < 4; ++qs) {
    st.ls[qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    st.lsum[qs] = 0.f;
#pragma unroll
    for (int hs = 0; hs < C::NH; ++hs) st.O[hs][qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  }
  {
    // K row of MFMA row lr in the first 16-key tile; chunk 4c + lg of it sits
    // at 4c + (lg ^ x) + (x & 4) for even c and 4c + (lg ^ x) - (x & 4) for
    // odd c (x & 4 is nonzero only when KCH is a multiple of 8); the key rows
    // 4ks + r0 have the same x.
    const int r0 = 8 * (lr >> 2) + (lr & 3), x0 = kswz<C::KCH>(r0);
    const int base = r0 * C::KCH + (lg ^ (x0 & 3));
    st.kb[0] = (base + (x0 & 4)) * 16;
    st.kb[1] = (base - (x0 & 4)) * 16;
    st.vb = (lr * 4 + (lg ^ ((lr >> 1) & 3))) * 16;
  }
  // the query fragments are complete before the tile loop, so its waits
  // count only the tile stream
  __builtin_amdgcn_s_waitcnt(0);

  const int p_first = pos0 + q_lo;
  const int p_last = pos0 + min(q_lo + 255, a.n - 1);
  const int jtw = max(0, p_first - a.window + 1) & ~31;
  const int ntw = (p_last - jtw) / 32 + 1;
  const int t_lo = ntw * sp / a.nsplit, t_hi = ntw * (sp + 1) / a.nsplit;
  const int jt0 = jtw + 32 * t_lo;
  const int ntile = t_hi - t_lo;
  const int pq = pos0 + qw;

  F2Issue<HD> is;
  is.init(reinterpret_cast<const TF *>(a.K) + (long)h * a.R * HD, reinterpret_cast<const TF *>(a.Vt) + (long)h * HD * a.R,
          a.R, wave, lane);
  // tiles [f0, f1) are full for all four waves: every key at or before the
  // work-group's first query and inside its last query's window
  int f0, f1;
  {
    const int lo = pos0 + q_lo + 255 - a.window + 1;  // smallest key of the last query's window
    f0 = lo <= jt0 ? 0 : (lo - jt0 + 31) / 32;
    f1 = p_first - 31 < jt0 ? 0 : (p_first - 31 - jt0) / 32 + 1;
    f0 = min(f0, ntile);
    f1 = min(max(f1, f0), ntile);
  }
  if (ntile > 0) is.run(stage, jt0 % a.R);
  fwd2_range<HD, TF, false>(st, is, stage, 0, f0, ntile, jt0, pq, lr, lg, a);
  fwd2_range<HD, TF, true>(st, is, stage, f0, f1, ntile, jt0, pq, lr, lg, a);
  fwd2_range<HD, TF, false>(st, is, stage, f1, ntile, ntile, jt0, pq, lr, lg, a);

  TO *Out = reinterpret_cast<TO *>(a.o);
#pragma unroll
  for (int qs = 0; qs < 4; ++qs) {
    const float lt = F2State<HD, TF>::MSUM ? st.ls[qs][0] : group4_sum(st.lsum[qs]);
    const int q = qw + qs * 16 + lr;
    if (q < a.n) {
      // a split may see no key of this query: weight 0 in the merge
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse = lt > 0.f ? a.sbound - P16Off<TF>::v + log2f(lt) : -INFINITY;
      if (a.nsplit == 1) {
#pragma unroll
        for (int hs = 0; hs < C::NH; ++hs) {
          float v[4] = {st.O[hs][qs][0] * inv, st.O[hs][qs][1] * inv, st.O[hs][qs][2] * inv,
                        st.O[hs][qs][3] * inv};
          store4<TO>(Out + (long)q * a.d + h * HD + hs * 16 + g4, v);
        }
        if (lg == 0) a.lse2[(long)h * a.ldl + q] = lse;
      } else {
        float *po = a.ws + (long)sp * a.n * a.d;
#pragma unroll
        for (int hs = 0; hs < C::NH; ++hs) {
          float v[4] = {st.O[hs][qs][0] * inv, st.O[hs][qs][1] * inv, st.O[hs][qs][2] * inv,
                        st.O[hs][qs][3] * inv};
          store4<float>(po + (long)q * a.d + h * HD + hs * 16 + g4, v);
        }
        if (lg == 0) a.ws[(long)a.nsplit * a.n * a.d + ((long)sp * a.H + h) * a.ldl + q] = lse;
      }
    }
  }
}

// ======================================================= dQ, bf16, 32-key tiles
// 32 queries per wave, 4 waves (128 queries) per work-group; grid
// (ceil(n/128), H, nsplit), remapped so that each XCD gets whole heads.  Key
// tiles of 32 stream from the rings straight into one LDS stage: K and V
// [32 keys][KCH chunks] (rows in the same swizzled layout as the forward's K
// tile) and K^T [hd rows][4 chunks].  Every wave reads all fragments of the
// tile into registers, a barrier frees the stage, the next tile streams in
// while the MFMAs run:
//   S^T = K Q^T, dP^T = V dO^T (lane: 8 consecutive keys of one query),
//   p = 2^(s * scale * log2 e - lse2), dS = p (dP - D),
//   dQ^T += K^T dS^T.
template <int HD> struct Q2 {
  static constexpr int NC = (HD + 31) / 32;
  static constexpr int KCH = 4 * NC;
  static constexpr int RC = HD / 8;
  static constexpr int NH = HD / 16;
  static constexpr int KB = 32 * KCH * 16;  // bytes of a K (or V) tile
  static constexpr int TB = HD * 4 * 16;    // bytes of a K^T tile
  static constexpr int KINS = KB / 1024;
  static constexpr int INS = (2 * KB + TB) / 1024;
  static constexpr int IPW = (INS + 3) / 4;
};

template <int HD> struct Q2Issue {
  using C = Q2<HD>;
  __amdgpu_buffer_rsrc_t rk, rv, rt;
  uint32_t voff[C::IPW];
  int j0;
  DEVI void init(const bf16_t *Kp, const bf16_t *Vp, const bf16_t *Ktp, int R, int wave, int lane) {
    const uint32_t bytes = (uint32_t)R * HD * 2;
    rk = __builtin_amdgcn_make_buffer_rsrc((void *)Kp, (short)0, bytes, BUF_RSRC_W3);
    rv = __builtin_amdgcn_make_buffer_rsrc((void *)Vp, (short)0, bytes, BUF_RSRC_W3);
    rt = __builtin_amdgcn_make_buffer_rsrc((void *)Ktp, (short)0, bytes, BUF_RSRC_W3);
    j0 = wave * C::IPW;
#pragma unroll
    for (int c = 0; c < C::IPW; ++c) {
      const int j = min(j0 + c, C::INS - 1);  // the last wave repeats the last chunk (same bytes)
      if (j < 2 * C::KINS) {
        const int s = (j % C::KINS) * 64 + lane, row = s / C::KCH, ch = (s % C::KCH) ^ kswz<C::KCH>(row);
        voff[c] = ch < C::RC ? (uint32_t)(row * HD * 2 + ch * 16) : BUF_OOB;
      } else {
        const int s = (j - 2 * C::KINS) * 64 + lane, row = s / 4, ch = (s % 4) ^ ((row >> 1) & 3);
        voff[c] = (uint32_t)(row * R * 2 + ch * 16);
      }
    }
  }
  DEVI void run(char *stage, int slot0) const {
#pragma unroll
    for (int c = 0; c < C::IPW; ++c) {
      const int j = min(j0 + c, C::INS - 1);
      const int part = j < C::KINS ? 0 : (j < 2 * C::KINS ? 1 : 2);  // uniform across the wave
      lds_void *dst = (lds_void *)(stage + j * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(part == 0 ? rk : (part == 1 ? rv : rt), dst, 16, voff[c],
                                               part == 2 ? slot0 * 2 : slot0 * HD * 2, 0, 0);
    }
  }
};

template <int HD> struct Q2State {
  using C = Q2<HD>;
  Frag<bf16_t> qf[2][C::NC], df[2][C::NC];
  f32x4_v dQ[C::NH][2];
  float Lq[2], Dv[2];
  int kb[2], vb;
};

template <int HD, bool FULL>
DEVI void dq2_range(Q2State<HD> &st, const Q2Issue<HD> &is, char *stage, int t0, int t1, int ntile, int jt0,
                    int pq, int lr, int lg, const AttnArgs &a) {
  using C = Q2<HD>;
  const float sl2 = a.scale * LOG2E_F;
  for (int t = t0; t < t1; ++t) {
    const int jt = jt0 + 32 * t;
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    Frag<bf16_t> kf[2][C::NC], vf[2][C::NC], tf[C::NH];
#pragma unroll
    for (int c = 0; c < C::NC; ++c)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int o = st.kb[c & 1] + (4 * ks * C::KCH + 4 * c) * 16;
        kf[ks][c].v = *reinterpret_cast<const uint4 *>(stage + o);
        vf[ks][c].v = *reinterpret_cast<const uint4 *>(stage + C::KB + o);
      }
#pragma unroll
    for (int hs = 0; hs < C::NH; ++hs)
      tf[hs].v = *reinterpret_cast<const uint4 *>(stage + 2 * C::KB + st.vb + hs * 16 * 64);
    lds_barrier();
    if (t + 1 < ntile) is.run(stage, (jt + 32) % a.R);
    if (!FULL && !((jt <= pq + 31) && (jt + 31 > pq - a.window))) continue;
    f32x4_v S[2][2], P[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        S[ks][qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
        P[ks][qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int c = 0; c < C::NC; ++c)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          mma(S[ks][qs], kf[ks][c], st.qf[qs][c]);
          mma(P[ks][qs], vf[ks][c], st.df[qs][c]);
        }
    Frag<bf16_t> sf[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int p = pq + qs * 16 + lr;
      float x[8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float e = fast_exp2(__builtin_fmaf(S[ks][qs][r], sl2, -st.Lq[qs]));
          if (!FULL) {
            const int j = jt + 8 * lg + 4 * ks + r;
            e = (j > p || j <= p - a.window) ? 0.f : e;
          }
          x[4 * ks + r] = e * (P[ks][qs][r] - st.Dv[qs]);
        }
      pack_frag(sf[qs], x);
    }
#pragma unroll
    for (int hs = 0; hs < C::NH; ++hs)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) mma(st.dQ[hs][qs], tf[hs], sf[qs]);
  }
}

template <int HD>
__global__ __launch_bounds__(NT, 2) void attn_bwd_dq2_kernel(const AttnArgs a) {
  using C = Q2<HD>;
  __shared__ __align__(1024) char stage[2 * C::KB + C::TB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4, g4 = lg * 4;
  int qb, h, sp;
  {
    const int gx = gridDim.x, total = gx * gridDim.y * gridDim.z;
    const int i = blockIdx.x + gx * (blockIdx.y + gridDim.y * blockIdx.z);
    const int q8 = total / 8, rem = total % 8, x = i % 8;
    const int m = x * q8 + min(x, rem) + i / 8;
    qb = m % gx;
    sp = (m / gx) % a.nsplit;
    h = m / (gx * a.nsplit);
  }
  const int q_lo = qb * 128;
  const int pos0 = *a.pos0;
  const int qw = q_lo + wave * 32;
  const bf16_t *Q = reinterpret_cast<const bf16_t *>(a.q);
  const bf16_t *dO = reinterpret_cast<const bf16_t *>(a.dout);

  Q2State<HD> st;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int q = qw + qs * 16 + lr;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      const int col = c * 32 + lg * 8;
      if (q < a.n && col < HD) {
        load_frag(st.qf[qs][c], Q + (long)q * a.d + h * HD + col);
        load_frag(st.df[qs][c], dO + (long)q * a.d + h * HD + col);
      } else {
        zero_frag(st.qf[qs][c]);
        zero_frag(st.df[qs][c]);
      }
    }
    st.Lq[qs] = q < a.n ? a.lse2[(long)h * a.ldl + q] : 0.f;
    st.Dv[qs] = q < a.n ? a.Dq[(long)h * a.ldl + q] : 0.f;
#pragma unroll
    for (int hs = 0; hs < C::NH; ++hs) st.dQ[hs][qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  }
  {
    const int r0 = 8 * (lr >> 2) + (lr & 3), x0 = kswz<C::KCH>(r0);
    const int base = r0 * C::KCH + (lg ^ (x0 & 3));
    st.kb[0] = (base + (x0 & 4)) * 16;
    st.kb[1] = (base - (x0 & 4)) * 16;
    st.vb = (lr * 4 + (lg ^ ((lr >> 1) & 3))) * 16;
  }
  __builtin_amdgcn_s_waitcnt(0);

  const int p_first = pos0 + q_lo;
  const int p_last = pos0 + min(q_lo + 127, a.n - 1);
  const int jtw = max(0, p_first - a.window + 1) & ~31;
  const int ntw = (p_last - jtw) / 32 + 1;
  const int t_lo = ntw * sp / a.nsplit, t_hi = ntw * (sp + 1) / a.nsplit;
  const int jt0 = jtw + 32 * t_lo;
  const int ntile = t_hi - t_lo;
  const int pq = pos0 + qw;

  Q2Issue<HD> is;
  is.init(reinterpret_cast<const bf16_t *>(a.K) + (long)h * a.R * HD,
          reinterpret_cast<const bf16_t *>(a.V) + (long)h * a.R * HD,
          reinterpret_cast<const bf16_t *>(a.Kt) + (long)h * HD * a.R, a.R, wave, lane);
  int f0, f1;
  {
    const int lo = pos0 + q_lo + 127 - a.window + 1;
    f0 = lo <= jt0 ? 0 : (lo - jt0 + 31) / 32;
    f1 = p_first - 31 < jt0 ? 0 : (p_first - 31 - jt0) / 32 + 1;
    f0 = min(f0, ntile);
    f1 = min(max(f1, f0), ntile);
  }
  if (ntile > 0) is.run(stage, jt0 % a.R);
  dq2_range<HD, false>(st, is, stage, 0, f0, ntile, jt0, pq, lr, lg, a);
  dq2_range<HD, true>(st, is, stage, f0, f1, ntile, jt0, pq, lr, lg, a);
  dq2_range<HD, false>(st, is, stage, f1, ntile, ntile, jt0, pq, lr, lg, a);

#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int q = qw + qs * 16 + lr;
    if (q < a.n) {
#pragma unroll
      for (int hs = 0; hs < C::NH; ++hs) {
        float v[4] = {st.dQ[hs][qs][0] * a.scale, st.dQ[hs][qs][1] * a.scale, st.dQ[hs][qs][2] * a.scale,
                      st.dQ[hs][qs][3] * a.scale};
        float *dst = a.nsplit == 1 ? a.dq : a.ws + (long)sp * a.n * a.d;
        store4<float>(dst + (long)q * a.d + h * HD + hs * 16 + g4, v);
      }
    }
  }
}

// ======================================================================= dQ
// grid (ceil(n/128), H); 4 waves x 32 queries; loops over the window's keys.
template <typename T, int HD>
__global__ __launch_bounds__(NT) void attn_bwd_dq_kernel(const AttnArgs a) {
  constexpr int HDP = Dims<HD>::HDP, NC = Dims<HD>::NC, NH = Dims<HD>::NH;
  constexpr int LDK = HDP + pad_el<T>(), LDV = 64 + pad_el<T>();
  __shared__ __align__(16) T smK[2][64 * LDK];
  __shared__ __align__(16) T smV[2][64 * LDK];
  __shared__ __align__(16) T smKt[2][HD * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4, g4 = lg * 4;
  const int h = blockIdx.y, q_lo = blockIdx.x * 128;
  const int pos0 = *a.pos0;
  const int qw = q_lo + wave * 32;
  const T *Q = reinterpret_cast<const T *>(a.q);
  const T *dO = reinterpret_cast<const T *>(a.dout);
  const T *Kr = reinterpret_cast<const T *>(a.K) + (long)h * a.R * HD;
  const T *Vr = reinterpret_cast<const T *>(a.V) + (long)h * a.R * HD;
  const T *Ktr = reinterpret_cast<const T *>(a.Kt) + (long)h * HD * a.R;

  Frag<T> qf[2][NC], df[2][NC];
  float Lq[2], Dv[2];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int q = qw + qs * 16 + lr;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = c * 32 + lg * 8;
      if (q < a.n && col < HD) {
        load_frag(qf[qs][c], Q + (long)q * a.d + h * HD + col);
        load_frag(df[qs][c], dO + (long)q * a.d + h * HD + col);
      } else {
        zero_frag(qf[qs][c]);
        zero_frag(df[qs][c]);
      }
    }
    Lq[qs] = q < a.n ? a.lse2[(long)h * a.ldl + q] : 0.f;
    Dv[qs] = q < a.n ? a.Dq[(long)h * a.ldl + q] : 0.f;
  }
  __builtin_amdgcn_s_waitcnt(0);

  const int p_first = pos0 + q_lo;
  const int p_last = pos0 + min(q_lo + 127, a.n - 1);
  const int jtw = max(0, p_first - a.window + 1) & ~63;
  const int ntw = (p_last - jtw) / 64 + 1;
  const int sp = blockIdx.z;
  const int t_lo = ntw * sp / a.nsplit, t_hi = ntw * (sp + 1) / a.nsplit;
  const int jt0 = jtw + 64 * t_lo;
  const int ntile = t_hi - t_lo;
  const int pw_min = pos0 + qw, pw_max = pos0 + qw + 31;
  const float sl2 = a.scale * LOG2E_F;

  f32x4_v dQ[NH][2];
#pragma unroll
  for (int hs = 0; hs < NH; ++hs)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) dQ[hs][qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  const uint32_t plane = (uint32_t)((long)a.R * HD * sizeof(T));
  RingTile<T, 64, HDP, HD> kio, vio;
  RingTile<T, HD, 64, 64> ktio;
  kio.init(Kr, plane, HD, tid);
  vio.init(Vr, plane, HD, tid);
  ktio.init(Ktr, plane, a.R, tid);
  if (ntile > 0) {
    const int s0 = jt0 % a.R;
    kio.load(s0 * HD * (int)sizeof(T));
    vio.load(s0 * HD * (int)sizeof(T));
    ktio.load(s0 * (int)sizeof(T));
    kio.store(smK[0], LDK, tid);
    vio.store(smV[0], LDK, tid);
    ktio.store(smKt[0], LDV, tid);
  }
  __syncthreads();

  for (int t = 0; t < ntile; ++t) {
    const int cur = t & 1;
    const int jt = jt0 + t * 64;
    if (t + 1 < ntile) {
      const int sn = (jt + 64) % a.R;
      kio.load(sn * HD * (int)sizeof(T));
      vio.load(sn * HD * (int)sizeof(T));
      ktio.load(sn * (int)sizeof(T));
    }
    const bool any = (jt <= pw_max) && (jt + 63 > pw_min - a.window);
    const bool full = (jt + 63 <= pw_min) && (jt > pw_max - a.window);
    if (any) {
      f32x4_v S[4][2], dP[4][2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          S[ks][qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
          dP[ks][qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        Frag<T> kf[4], vf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          load_frag(kf[ks], smK[cur] + (ks * 16 + lr) * LDK + c * 32 + lg * 8);
          load_frag(vf[ks], smV[cur] + (ks * 16 + lr) * LDK + c * 32 + lg * 8);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) {
            mma(S[ks][qs], kf[ks], qf[qs][c]);
            mma(dP[ks][qs], vf[ks], df[qs][c]);
          }
      }
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const int p = pos0 + qw + qs * 16 + lr;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bool ok = true;
            if (!full) {
              int j = jt + ks * 16 + g4 + r;
              ok = (j <= p) && (j > p - a.window);
            }
            float pv = ok ? fast_exp2(S[ks][qs][r] * sl2 - Lq[qs]) : 0.f;
            S[ks][qs][r] = pv * (dP[ks][qs][r] - Dv[qs]);
          }
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        Frag<T> sf[2];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          float x[8] = {S[2 * c2][qs][0],     S[2 * c2][qs][1],     S[2 * c2][qs][2],     S[2 * c2][qs][3],
                        S[2 * c2 + 1][qs][0], S[2 * c2 + 1][qs][1], S[2 * c2 + 1][qs][2], S[2 * c2 + 1][qs][3]};
          pack_frag(sf[qs], x);
        }
#pragma unroll
        for (int hs = 0; hs < NH; ++hs) {
          Frag<T> kt;
          const T *row = smKt[cur] + (hs * 16 + lr) * LDV + c2 * 32 + g4;
          load_frag2(kt, row, row + 16);
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) mma(dQ[hs][qs], kt, sf[qs]);
        }
      }
    }
    if (t + 1 < ntile) {
      kio.store(smK[cur ^ 1], LDK, tid);
      vio.store(smV[cur ^ 1], LDK, tid);
      ktio.store(smKt[cur ^ 1], LDV, tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int q = qw + qs * 16 + lr;
    if (q < a.n) {
#pragma unroll
      for (int hs = 0; hs < NH; ++hs) {
        float v[4] = {dQ[hs][qs][0] * a.scale, dQ[hs][qs][1] * a.scale, dQ[hs][qs][2] * a.scale,
                      dQ[hs][qs][3] * a.scale};
        float *dst = a.nsplit == 1 ? a.dq : a.ws + (long)sp * a.n * a.d;
        store4<float>(dst + (long)q * a.d + h * HD + hs * 16 + g4, v);
      }
    }
  }
}

// ======================================================================= dK, dV
// grid (ceil(n/64), H); 4 waves x 16 chunk keys; loops over the chunk's
// queries at or after the key tile (all inside the window since b <= k).
template <typename T, int HD>
__global__ __launch_bounds__(NT, 2) void attn_bwd_dkdv_kernel(const AttnArgs a) {
  constexpr int HDP = Dims<HD>::HDP, NC = Dims<HD>::NC, NH = Dims<HD>::NH;
  constexpr int LDK = HDP + pad_el<T>(), LDV = 64 + pad_el<T>();
  __shared__ __align__(16) T smQ[64 * LDK];
  __shared__ __align__(16) T smdO[64 * LDK];
  __shared__ __align__(16) T smQt[HD * LDV];
  __shared__ __align__(16) T smdOt[HD * LDV];
  __shared__ float smL[64], smD[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4, g4 = lg * 4;
  // Work-groups go to the 8 XCDs round-robin by linear index; remap so that each XCD
  // gets whole heads: the key tiles of one head then re-read that head's query-side
  // tiles (q, dO and their transposes) from one L2 instead of eight.
  int h, k_lo;
  {
    const int gx = gridDim.x, total = gx * gridDim.y;
    const int i = blockIdx.x + gx * blockIdx.y;
    const int q8 = total / 8, rem = total % 8, x = i % 8;
    const int m = x * q8 + min(x, rem) + i / 8;
    k_lo = (m % gx) * 64;
    h = m / gx;
  }
  const int pos0 = *a.pos0;
  const int kw = k_lo + wave * 16;
  const int key = kw + lr;  // this lane's key (chunk-relative)
  const T *Q = reinterpret_cast<const T *>(a.q);
  const T *dO = reinterpret_cast<const T *>(a.dout);
  const T *Qt = reinterpret_cast<const T *>(a.qt) + (long)h * HD * a.ldt;
  const T *dOt = reinterpret_cast<const T *>(a.doutt) + (long)h * HD * a.ldt;

  Frag<T> kf[NC], vf[NC];
  {
    const long slot = (pos0 + key) % a.R;
    const T *kr = reinterpret_cast<const T *>(a.K) + ((long)h * a.R + slot) * HD;
    const T *vr = reinterpret_cast<const T *>(a.V) + ((long)h * a.R + slot) * HD;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = c * 32 + lg * 8;
      if (key < a.n && col < HD) {
        load_frag(kf[c], kr + col);
        load_frag(vf[c], vr + col);
      } else {
        zero_frag(kf[c]);
        zero_frag(vf[c]);
      }
    }
  }
  const float sl2 = a.scale * LOG2E_F;
  f32x4_v dK[NH], dV[NH];
#pragma unroll
  for (int hs = 0; hs < NH; ++hs) {
    dK[hs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    dV[hs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  }

  // The next query tile is loaded into registers while the current one is multiplied
  // from LDS (one tile of global-load latency per block instead of one per tile).
  TileIO<T, 64, HDP> ioq, iod;
  TileIO<T, HD, 64> ioqt, iodt;
  float nl = 0.f, nd = 0.f;
  auto fetch = [&](int qt) {
    if (qt + 64 <= a.n) {  // whole tile inside the chunk
      ioq.load_rows(Q + (long)qt * a.d + h * HD, a.d, HD, tid);
      iod.load_rows(dO + (long)qt * a.d + h * HD, a.d, HD, tid);
      ioqt.load_rows(Qt + qt, a.ldt, 64, tid);
      iodt.load_rows(dOt + qt, a.ldt, 64, tid);
    } else {
      ioq.load(Q + (long)qt * a.d + h * HD, a.d, a.n - qt, HD, tid);
      iod.load(dO + (long)qt * a.d + h * HD, a.d, a.n - qt, HD, tid);
      ioqt.load(Qt + qt, a.ldt, HD, a.n - qt, tid);
      iodt.load(dOt + qt, a.ldt, HD, a.n - qt, tid);
    }
    if (tid < 64) {
      const int q = qt + tid;
      nl = q < a.n ? a.lse2[(long)h * a.ldl + q] : 0.f;
      nd = q < a.n ? a.Dq[(long)h * a.ldl + q] : 0.f;
    }
  };
  if (k_lo < a.n) fetch(k_lo);
  for (int qt = k_lo; qt < a.n; qt += 64) {
    ioq.store(smQ, LDK, tid);
    iod.store(smdO, LDK, tid);
    ioqt.store(smQt, LDV, tid);
    iodt.store(smdOt, LDV, tid);
    if (tid < 64) {
      smL[tid] = nl;
      smD[tid] = nd;
    }
    asm volatile("" ::: "memory");
    lds_barrier();  // LDS only: the prefetch of the next tile stays in flight
    asm volatile("" ::: "memory");
    if (qt + 64 < a.n) fetch(qt + 64);
    f32x4_v S[4], dP[4];
#pragma unroll
    for (int qs = 0; qs < 4; ++qs) {
      S[qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      dP[qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) {
        Frag<T> qa, da;
        load_frag(qa, smQ + (qs * 16 + lr) * LDK + c * 32 + lg * 8);
        load_frag(da, smdO + (qs * 16 + lr) * LDK + c * 32 + lg * 8);
        mma(S[qs], qa, kf[c]);
        mma(dP[qs], da, vf[c]);
      }
    }
    // lane holds S[q = qt + 16 qs + g4 + r][key]
#pragma unroll
    for (int qs = 0; qs < 4; ++qs)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = qs * 16 + g4 + r;
        const int q = qt + qi;
        const bool ok = (q < a.n) && (key < a.n) && (q >= key) && (q - key < a.window);
        float pv = ok ? fast_exp2(S[qs][r] * sl2 - smL[qi]) : 0.f;
        S[qs][r] = pv;
        dP[qs][r] = pv * (dP[qs][r] - smD[qi]);
      }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      Frag<T> pf, sf;
      float x[8] = {S[2 * c2][0], S[2 * c2][1], S[2 * c2][2], S[2 * c2][3],
                    S[2 * c2 + 1][0], S[2 * c2 + 1][1], S[2 * c2 + 1][2], S[2 * c2 + 1][3]};
      pack_frag(pf, x);
      float y[8] = {dP[2 * c2][0], dP[2 * c2][1], dP[2 * c2][2], dP[2 * c2][3],
                    dP[2 * c2 + 1][0], dP[2 * c2 + 1][1], dP[2 * c2 + 1][2], dP[2 * c2 + 1][3]};
      pack_frag(sf, y);
#pragma unroll
      for (int hs = 0; hs < NH; ++hs) {
        Frag<T> ao, aq;
        const T *ro = smdOt + (hs * 16 + lr) * LDV + c2 * 32 + g4;
        const T *rq = smQt + (hs * 16 + lr) * LDV + c2 * 32 + g4;
        load_frag2(ao, ro, ro + 16);
        load_frag2(aq, rq, rq + 16);
        mma(dV[hs], ao, pf);
        mma(dK[hs], aq, sf);
      }
    }
    asm volatile("" ::: "memory");
    lds_barrier();  // LDS only: the prefetch of the next tile stays in flight
    asm volatile("" ::: "memory");
  }

  if (key < a.n) {
#pragma unroll
    for (int hs = 0; hs < NH; ++hs) {
      float v[4] = {dV[hs][0], dV[hs][1], dV[hs][2], dV[hs][3]};
      store4<float>(a.dv + (long)key * a.d + h * HD + hs * 16 + g4, v);
      float k4[4] = {dK[hs][0] * a.scale, dK[hs][1] * a.scale, dK[hs][2] * a.scale, dK[hs][3] * a.scale};
      store4<float>(a.dk + (long)key * a.d + h * HD + hs * 16 + g4, k4);
    }
  }
}

// ================================================================ dK, dV, 16-bit, streamed
// Gradients of the chunk's own keys and values (cached keys are constants):
//   dV[j] = sum_q P[q][j] dO[q],   dK[j] = scale * sum_q dS[q][j] q^[q],
//   P = 2^(s log2e scale - lse2[q]),   dS = P (dP - D[q]),   dP = dO v^T,
// over the chunk queries q >= j (all inside the window, since the window covers a chunk).
//
// Work: a work-group owns a pair of 64-key blocks (j, nkb-1-j), whose query tiles
// number nqt-j and j+1 (nqt = nkb tiles of 64 queries), so every work-group has nqt+1
// tiles (the middle block of an odd nkb alone); grid (ceil(nkb/2), H), remapped so that
// the work-groups of one head share an XCD and its L2 for the query-side tiles.
// 8 waves, two per SIMD: wave = (key slice kw of 16 keys) x (query half qh of the
// tile); each keeps its keys' K and V fragments in registers and accumulates dK, dV
// over its query half.  At the end of a key block the qh = 1 waves pass their sums to the
// qh = 0 waves through LDS, which add theirs and store (a fixed order).
//
// Per query tile of 64, one LDS stage holds (streamed by buffer_load ... lds three
// stages deep: tile it+2 streams while tile it is computed):
//   Q, dO   [64 rows][KCH chunks of 16 bytes] (head dims, zero past hd), chunk c of row r
//           at c ^ sq(r);
//   Q^T, dO^T [hd rows][8 chunks] (8 queries per chunk), chunk c of row d at c ^ ((d>>1)&7);
//   lse2, D [64] each (in a 1 KiB slot).
// Score rows are taken in the order 8 (i/4) + 4 qs + i%4 of the half (i = MFMA row), so
// each lane ends up with 8 consecutive queries of one key: exactly one 16-byte fragment
// of Q^T or dO^T for the dK / dV products.  The swizzles put the 16 lanes of every
// ds_read_b128 pass on 16 distinct 16-byte bank groups (measured pass grouping: lanes
// < 32 whose 4-lane group index has even bit parity form one pass, odd another, likewise
// for lanes >= 32).  A tile's reads are three asm statements that wait for their own
// reads (other stages' loads are still in flight then).
template <int HD> struct K2 {
  static constexpr int NC = (HD + 31) / 32;   // 32-deep steps over the head dims
  static constexpr int KCH = 4 * NC;          // chunks per padded Q / dO row
  static constexpr int RC = HD / 8;           // chunks holding data
  static constexpr int NH = HD / 16;          // 16-row tiles over the head dims
  static constexpr int QB = 64 * KCH * 16;    // bytes of a Q (or dO) tile
  static constexpr int TB = HD * 128;         // bytes of a Q^T (or dO^T) tile
  static constexpr int LOFF = 2 * QB + 2 * TB, DOFF = LOFF + 1024;
  static constexpr int SB = DOFF + 1024;      // bytes of a stage
  static constexpr int INS = SB / 1024;       // 1 KiB direct-to-LDS loads per stage
  static constexpr int IPW = (INS + 7) / 8;   // per wave (the last ones repeat the last load)
  static constexpr int QI = QB / 1024, TI = TB / 1024;
  static_assert(2 * NH * 4 * 64 * 16 <= SB, "a stage holds the dK / dV hand-over of the 4 key slices");
};
template <int HD> DEVI int k2sq(int r) {
  return (((r >> 3) & 1) << 1) | ((K2<HD>::KCH == 8) ? (((r >> 1) & 1) << 2) : 0);
}
typedef int k2v4 __attribute__((ext_vector_type(4)));

// ---- a tile's fragment reads, each statement waiting for its own reads
#define K2R(o, a, off) "ds_read_b128 %[" #o "], %[" #a "] offset:%[" #off "]\n"
// Q (offset 0) and dO (offset QB) fragments [qs][c] at addresses a_qs_c
template <int HD>
DEVI void k2_rd_qd(k2v4 (&q)[2][K2<HD>::NC], k2v4 (&d)[2][K2<HD>::NC], const uint32_t (&ad)[2][K2<HD>::NC]) {
  constexpr int NC = K2<HD>::NC, QB = K2<HD>::QB;
  if constexpr (NC == 1) {
    asm volatile(K2R(q0, a0, z) K2R(q1, a1, z) K2R(d0, a0, qb) K2R(d1, a1, qb) "s_waitcnt lgkmcnt(0)"
                 : [q0] "=&v"(q[0][0]), [q1] "=&v"(q[1][0]), [d0] "=&v"(d[0][0]), [d1] "=&v"(d[1][0])
                 : [a0] "v"(ad[0][0]), [a1] "v"(ad[1][0]), [z] "i"(0), [qb] "i"(QB) : "memory");
  } else if constexpr (NC == 2) {
    asm volatile(K2R(q00, a00, z) K2R(q01, a01, z) K2R(q10, a10, z) K2R(q11, a11, z)
                 K2R(d00, a00, qb) K2R(d01, a01, qb) K2R(d10, a10, qb) K2R(d11, a11, qb) "s_waitcnt lgkmcnt(0)"
                 : [q00] "=&v"(q[0][0]), [q01] "=&v"(q[0][1]), [q10] "=&v"(q[1][0]), [q11] "=&v"(q[1][1]),
                   [d00] "=&v"(d[0][0]), [d01] "=&v"(d[0][1]), [d10] "=&v"(d[1][0]), [d11] "=&v"(d[1][1])
                 : [a00] "v"(ad[0][0]), [a01] "v"(ad[0][1]), [a10] "v"(ad[1][0]), [a11] "v"(ad[1][1]), [z] "i"(0),
                   [qb] "i"(QB)
                 : "memory");
  } else {
    static_assert(NC == 3, "head dims up to 96");
    asm volatile(K2R(q00, a00, z) K2R(q01, a01, z) K2R(q02, a02, z) K2R(q10, a10, z) K2R(q11, a11, z)
                 K2R(q12, a12, z) K2R(d00, a00, qb) K2R(d01, a01, qb) K2R(d02, a02, qb) K2R(d10, a10, qb)
                 K2R(d11, a11, qb) K2R(d12, a12, qb) "s_waitcnt lgkmcnt(0)"
                 : [q00] "=&v"(q[0][0]), [q01] "=&v"(q[0][1]), [q02] "=&v"(q[0][2]), [q10] "=&v"(q[1][0]),
                   [q11] "=&v"(q[1][1]), [q12] "=&v"(q[1][2]), [d00] "=&v"(d[0][0]), [d01] "=&v"(d[0][1]),
                   [d02] "=&v"(d[0][2]), [d10] "=&v"(d[1][0]), [d11] "=&v"(d[1][1]), [d12] "=&v"(d[1][2])
                 : [a00] "v"(ad[0][0]), [a01] "v"(ad[0][1]), [a02] "v"(ad[0][2]), [a10] "v"(ad[1][0]),
                   [a11] "v"(ad[1][1]), [a12] "v"(ad[1][2]), [z] "i"(0), [qb] "i"(QB)
                 : "memory");
  }
}
// Q^T (offset 2048 hs) and dO^T (offset TB + 2048 hs) fragments from address a
#define K2T(hs) K2R(t##hs, a, ot##hs) K2R(o##hs, a, oo##hs)
#define K2TO(hs) [t##hs] "=&v"(t[hs]), [o##hs] "=&v"(o[hs])
#define K2TI(hs) [ot##hs] "i"(2048 * hs), [oo##hs] "i"(TB + 2048 * hs)
template <int HD> DEVI void k2_rd_t(k2v4 (&t)[K2<HD>::NH], k2v4 (&o)[K2<HD>::NH], uint32_t a) {
  constexpr int NH = K2<HD>::NH, TB = K2<HD>::TB;
  if constexpr (NH == 1) {
    asm volatile(K2T(0) "s_waitcnt lgkmcnt(0)" : K2TO(0) : [a] "v"(a), K2TI(0) : "memory");
  } else if constexpr (NH == 2) {
    asm volatile(K2T(0) K2T(1) "s_waitcnt lgkmcnt(0)" : K2TO(0), K2TO(1) : [a] "v"(a), K2TI(0), K2TI(1) : "memory");
  } else if constexpr (NH == 4) {
    asm volatile(K2T(0) K2T(1) K2T(2) K2T(3) "s_waitcnt lgkmcnt(0)"
                 : K2TO(0), K2TO(1), K2TO(2), K2TO(3)
                 : [a] "v"(a), K2TI(0), K2TI(1), K2TI(2), K2TI(3) : "memory");
  } else if constexpr (NH == 5) {
    asm volatile(K2T(0) K2T(1) K2T(2) K2T(3) K2T(4) "s_waitcnt lgkmcnt(0)"
                 : K2TO(0), K2TO(1), K2TO(2), K2TO(3), K2TO(4)
                 : [a] "v"(a), K2TI(0), K2TI(1), K2TI(2), K2TI(3), K2TI(4) : "memory");
  } else {
    static_assert(NH == 6, "head dims 16, 32, 64, 80, 96");
    asm volatile(K2T(0) K2T(1) K2T(2) K2T(3) K2T(4) K2T(5) "s_waitcnt lgkmcnt(0)"
                 : K2TO(0), K2TO(1), K2TO(2), K2TO(3), K2TO(4), K2TO(5)
                 : [a] "v"(a), K2TI(0), K2TI(1), K2TI(2), K2TI(3), K2TI(4), K2TI(5) : "memory");
  }
}
// lse2 and D of the lane's 8 queries from address a
template <int HD> DEVI void k2_rd_ld(k2v4 (&l)[2], k2v4 (&d)[2], uint32_t a) {
  asm volatile(K2R(l0, a, o0) K2R(l1, a, o1) K2R(d0, a, o2) K2R(d1, a, o3) "s_waitcnt lgkmcnt(0)"
               : [l0] "=&v"(l[0]), [l1] "=&v"(l[1]), [d0] "=&v"(d[0]), [d1] "=&v"(d[1])
               : [a] "v"(a), [o0] "i"(K2<HD>::LOFF), [o1] "i"(K2<HD>::LOFF + 16), [o2] "i"(K2<HD>::DOFF),
                 [o3] "i"(K2<HD>::DOFF + 16)
               : "memory");
}
#undef K2R
#undef K2T
#undef K2TO
#undef K2TI

template <int HD>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv2_kernel(const AttnArgs a) {
  using C = K2<HD>;
  constexpr int NC = C::NC, KCH = C::KCH, NH = C::NH, STG = 3;
  __shared__ __align__(1024) char sm[STG * C::SB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3, qh = wave >> 2;
  const int lr = lane & 15, lg = lane >> 4, g4 = lg * 4;
  int pr, h;
  {
    const int gx = gridDim.x, total = gx * gridDim.y;
    const int i = blockIdx.x + gx * blockIdx.y;
    const int q8 = total / 8, rem = total % 8, x = i % 8;
    const int m = x * q8 + min(x, rem) + i / 8;
    pr = m % gx;
    h = m / gx;
  }
  const int n = a.n, nkb = (n + 63) / 64;
  const int kb1 = pr, kb2 = nkb - 1 - pr;
  const int nq1 = nkb - kb1, nq2 = kb2 != kb1 ? nkb - kb2 : 0;
  const int total_it = nq1 + nq2;
  const int pos0 = *a.pos0;
  const uint32_t smb = (uint32_t)(uintptr_t)(lds_void *)sm;

  // ---- this wave's loads of a stage: load c covers stage bytes [1024 j, 1024 j + 1024)
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)a.q, (short)0, (uint32_t)n * a.d * 2, BUF_RSRC_W3);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void *)a.dout, (short)0, (uint32_t)n * a.d * 2, BUF_RSRC_W3);
  const __amdgpu_buffer_rsrc_t rqt = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.qt, (short)0, (uint32_t)a.H * HD * a.ldt * 2, BUF_RSRC_W3);
  const __amdgpu_buffer_rsrc_t rdt = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.doutt, (short)0, (uint32_t)a.H * HD * a.ldt * 2, BUF_RSRC_W3);
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void *)a.lse2, (short)0, (uint32_t)a.H * a.ldl * 4, BUF_RSRC_W3);
  const __amdgpu_buffer_rsrc_t rD = __builtin_amdgcn_make_buffer_rsrc((void *)a.Dq, (short)0, (uint32_t)a.H * a.ldl * 4, BUF_RSRC_W3);
  int srow[C::IPW], sch[C::IPW];  // per load: tile row and global chunk of this lane
#pragma unroll
  for (int c = 0; c < C::IPW; ++c) {
    const int j = min(wave * C::IPW + c, C::INS - 1);
    if (j < 2 * C::QI) {
      const int sl = (j % C::QI) * 64 + lane;
      srow[c] = sl / KCH;
      sch[c] = (sl % KCH) ^ k2sq<HD>(srow[c]);
    } else if (j < 2 * C::QI + 2 * C::TI) {
      const int sl = ((j - 2 * C::QI) % C::TI) * 64 + lane;
      srow[c] = sl / 8;
      sch[c] = (sl % 8) ^ ((srow[c] >> 1) & 7);
    } else {
      srow[c] = 0;
      sch[c] = lane;
    }
  }
  // streams the tile of 64 queries starting at qt into stage st (branches uniform per wave)
  auto issue = [=](int st, int qt) {
#pragma unroll
    for (int c = 0; c < C::IPW; ++c) {
      const int j = min(wave * C::IPW + c, C::INS - 1);
      lds_void *dst = (lds_void *)(sm + st * C::SB + j * 1024);
      if (j < 2 * C::QI) {
        const int row = srow[c], cc = sch[c];
        const uint32_t o = (cc < C::RC && qt + row < n) ? (uint32_t)(((qt + row) * a.d + h * HD + cc * 8) * 2) : BUF_OOB;
        if (j < C::QI)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, dst, 16, o, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, dst, 16, o, 0, 0, 0);
      } else if (j < 2 * C::QI + 2 * C::TI) {
        const int row = srow[c], cc = sch[c];
        const uint32_t o = qt + 8 * cc < n ? (uint32_t)(((h * HD + row) * a.ldt + qt + 8 * cc) * 2) : BUF_OOB;
        if (j < 2 * C::QI + C::TI)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rqt, dst, 16, o, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rdt, dst, 16, o, 0, 0, 0);
      } else {
        const uint32_t o = (lane < 16 && qt + 4 * lane < n) ? (uint32_t)((h * a.ldl + qt + 4 * lane) * 4) : BUF_OOB;
        if (j == C::INS - 2)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, dst, 16, o, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rD, dst, 16, o, 0, 0, 0);
      }
    }
  };
  auto qt_of = [&](int it) { return 64 * (it < nq1 ? kb1 + it : kb2 + it - nq1); };

  // ---- per-lane read offsets within a stage
  uint32_t aq[2][NC], at, al;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int row = 32 * qh + 8 * (lr >> 2) + 4 * qs + (lr & 3);
#pragma unroll
    for (int c = 0; c < NC; ++c) aq[qs][c] = row * KCH * 16 + (((4 * c + lg) ^ k2sq<HD>(row)) << 4);
  }
  at = 2 * C::QB + lr * 128 + (((4 * qh + lg) ^ ((lr >> 1) & 7)) << 4);  // row hs*16+lr at + 2048 hs
  al = (32 * qh + 8 * lg) * 4;  // this lane's 8 queries in the lse2 / D slots

  const float sl2 = a.scale * LOG2E_F;
  for (int s = 0; s < 2; ++s)
    if (s < total_it) issue(s, qt_of(s));
  // the K and V fragments of both key blocks' keys, loaded once up front: a load left in
  // flight across the loop would make every iteration wait for the tile loads behind it
  Frag<bf16_t> kf[NC], vf[NC], kf2[NC], vf2[NC];
  {
    auto load_kv = [&](Frag<bf16_t>(&kk)[NC], Frag<bf16_t>(&vv)[NC], int kbl) {
      const int ky = kbl * 64 + kw * 16 + lr;
      const long slot = (pos0 + ky) % a.R;
      const bf16_t *kr = reinterpret_cast<const bf16_t *>(a.K) + ((long)h * a.R + slot) * HD;
      const bf16_t *vr = reinterpret_cast<const bf16_t *>(a.V) + ((long)h * a.R + slot) * HD;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int col = c * 32 + lg * 8;
        if (ky < n && col < HD) {
          load_frag(kk[c], kr + col);
          load_frag(vv[c], vr + col);
        } else {
          zero_frag(kk[c]);
          zero_frag(vv[c]);
        }
      }
    };
    load_kv(kf, vf, kb1);
    load_kv(kf2, vf2, kb2);
    wait_vm<0>();
  }
  f32x4_v dK[NH], dV[NH];
  int key = 0, kb = -1, qt0 = 0;
  for (int it = 0; it < total_it; ++it) {
    const int st = it % STG;
    const int kbi = it < nq1 ? kb1 : kb2;
    const int qt = qt_of(it);
    // tile it landed for this thread: the loads of tile it+1 may stay in flight
    if (it + 1 < total_it)
      wait_vm<C::IPW>();
    else
      wait_vm<0>();
    __builtin_amdgcn_s_barrier();  // every wave's loads of tile it landed; stage (it+2) % 3 is free
    if (it + 2 < total_it) issue((it + 2) % STG, qt_of(it + 2));
    if (kbi != kb) {  // a new key block: its keys' fragments, zeroed sums
      if (kb >= 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          kf[c] = kf2[c];
          vf[c] = vf2[c];
        }
      }
      kb = kbi;
      qt0 = qt;
      key = kb * 64 + kw * 16 + lr;
#pragma unroll
      for (int hs = 0; hs < NH; ++hs) {
        dK[hs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
        dV[hs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      }
    }
    const uint32_t sb = smb + st * C::SB;
    k2v4 fq[2][NC], fd[2][NC], ft[NH], fo[NH], lv[2], dv[2];
    {
      uint32_t ad[2][NC];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int c = 0; c < NC; ++c) ad[qs][c] = sb + aq[qs][c];
      k2_rd_qd<HD>(fq, fd, ad);
    }
    // S = Q K^T, dP = dO V^T for this wave's 32 queries x 16 keys
    f32x4_v S[2], P[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      S[qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      P[qs] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        Frag<bf16_t> x, y;
        x.v = __builtin_bit_cast(uint4, fq[qs][c]);
        y.v = __builtin_bit_cast(uint4, fd[qs][c]);
        mma(S[qs], x, kf[c]);
        mma(P[qs], y, vf[c]);
      }
    }
    k2_rd_t<HD>(ft, fo, sb + at);
    k2_rd_ld<HD>(lv, dv, sb + al);
    // lane: queries qt + 32 qh + 8 lg + (4 qs + r), key `key`
    Frag<bf16_t> pf, sf;
    {
      const bool diag = qt == qt0;  // the key block's own tile: queries before a key are masked
      float x[8], y[8];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int k = 4 * qs + r, q = qt + 32 * qh + 8 * lg + k;
          const bool ok = (q < n) && (key < n) && (!diag || q >= key);
          const float L = __int_as_float(lv[qs][r]), D = __int_as_float(dv[qs][r]);
          const float pv = fast_exp2(__builtin_fmaf(S[qs][r], sl2, -L));
          x[k] = ok ? pv : 0.f;
          y[k] = ok ? pv * (P[qs][r] - D) : 0.f;
        }
      pack_frag(pf, x);
      pack_frag(sf, y);
    }
    // dV += dO^T P, dK += Q^T dS over the 32 queries
#pragma unroll
    for (int hs = 0; hs < NH; ++hs) {
      Frag<bf16_t> x, y;
      x.v = __builtin_bit_cast(uint4, fo[hs]);
      y.v = __builtin_bit_cast(uint4, ft[hs]);
      mma(dV[hs], x, pf);
      mma(dK[hs], y, sf);
    }
    const bool last = (it + 1 == total_it) || (it + 1 == nq1);
    if (last) {
      // the key block is done: the qh = 1 waves hand their sums to the qh = 0 waves
      // through this stage, which every wave has finished reading (the next load into
      // it is issued after the next iteration's barrier)
      lds_barrier();
      f32x4_v *red = reinterpret_cast<f32x4_v *>(sm + st * C::SB) + kw * 64 + lane;
      if (qh == 1) {
#pragma unroll
        for (int hs = 0; hs < NH; ++hs) {
          red[(2 * hs) * 256] = dK[hs];
          red[(2 * hs + 1) * 256] = dV[hs];
        }
      }
      lds_barrier();
      if (qh == 0 && key < n) {
        float *pk = a.dk + (long)key * a.d + h * HD + g4, *pv = a.dv + (long)key * a.d + h * HD + g4;
#pragma unroll
        for (int hs = 0; hs < NH; ++hs) {
          *reinterpret_cast<f32x4_v *>(pk + hs * 16) = (red[(2 * hs) * 256] + dK[hs]) * a.scale;
          *reinterpret_cast<f32x4_v *>(pv + hs * 16) = red[(2 * hs + 1) * 256] + dV[hs];
        }
      }
    }
  }
}

template <typename T, int HD> hipError_t fwd_t(const AttnArgs &a, hipStream_t st) {
  dim3 grid((a.n + 127) / 128, a.H, a.nsplit);
  // bf16 mode hands the O projection an fp16 operand; fp32 mode keeps fp32
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((attn_fwd_kernel<T, HD, f16_t>), grid, dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, HD, T>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}
// explicit instantiations: clang otherwise may not emit the host launch stubs
#define FWD2_INST(HD)                                                          \
  template __global__ void attn_fwd2_kernel<HD, f16_t, f16_t>(const AttnArgs); \
  template __global__ void attn_fwd2_kernel<HD, bf16_t, f16_t>(const AttnArgs);
FWD2_INST(16)
FWD2_INST(32)
FWD2_INST(64)
FWD2_INST(80)
FWD2_INST(96)
#undef FWD2_INST

template <int HD> hipError_t fwd2_t(const AttnArgs &a, hipStream_t st) {
  dim3 grid((a.n + 255) / 256, a.H, a.nsplit);
  // bf16 mode always hands the O projection an fp16 operand
  if (!a.o_f16) return hipErrorInvalidValue;
  if (a.fwd_f16)
    hipLaunchKernelGGL((attn_fwd2_kernel<HD, f16_t, f16_t>), grid, dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd2_kernel<HD, bf16_t, f16_t>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}
template <int HD> hipError_t dq2_t(const AttnArgs &a, hipStream_t st) {
  dim3 grid((a.n + 127) / 128, a.H, a.nsplit);
  hipLaunchKernelGGL((attn_bwd_dq2_kernel<HD>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}
template <typename T, int HD> hipError_t dq_t(const AttnArgs &a, hipStream_t st) {
  dim3 grid((a.n + 127) / 128, a.H, a.nsplit);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HD>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}
template <typename T, int HD> hipError_t dkdv_t(const AttnArgs &a, hipStream_t st) {
  dim3 grid((a.n + 63) / 64, a.H);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, HD>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

#define HD_SWITCH(FN, T)                          \
  switch (hd) {                                   \
    case 16: return FN<T, 16>(a, st);             \
    case 32: return FN<T, 32>(a, st);             \
    case 64: return FN<T, 64>(a, st);             \
    case 80: return FN<T, 80>(a, st);             \
    case 96: return FN<T, 96>(a, st);             \
    case 128: return FN<T, 128>(a, st);           \
  }                                               \
  return hipErrorInvalidValue;

// fp32 (the small test workloads) is compiled for head_dim <= 64 only: its
// double-buffered tiles for larger heads would not fit in 160 KiB of LDS.
#define HD_SWITCH_F32(FN)                         \
  switch (hd) {                                   \
    case 16: return FN<float, 16>(a, st);         \
    case 32: return FN<float, 32>(a, st);         \
    case 64: return FN<float, 64>(a, st);         \
  }                                               \
  return hipErrorInvalidValue;

// The bounded forward keeps 64 queries' outputs per wave in registers, which
// fits head dims up to 96.
bool bounded(int dtype, float sbound, int hd) {
  return dtype == 1 && hd <= 96 && sbound > 0.f && sbound <= ATTN_MAX_SBOUND;
}

hipError_t fwd_hd(bool bf, int hd, const AttnArgs &a, hipStream_t st) {
  if (bf && bounded(1, a.sbound, hd)) {
    switch (hd) {
      case 16: return fwd2_t<16>(a, st);
      case 32: return fwd2_t<32>(a, st);
      case 64: return fwd2_t<64>(a, st);
      case 80: return fwd2_t<80>(a, st);
      case 96: return fwd2_t<96>(a, st);
    }
    return hipErrorInvalidValue;
  }
  if (bf) { HD_SWITCH(fwd_t, bf16_t) }
  HD_SWITCH_F32(fwd_t)
}
hipError_t dq_hd(bool bf, int hd, const AttnArgs &a, hipStream_t st) {
  if (bf) {
    switch (hd) {
      case 16: return dq2_t<16>(a, st);
      case 32: return dq2_t<32>(a, st);
      case 64: return dq2_t<64>(a, st);
      case 80: return dq2_t<80>(a, st);
      case 96: return dq2_t<96>(a, st);
      case 128: return dq_t<bf16_t, 128>(a, st);  // 32 queries' dQ of hd 128 per wave exceed the registers
    }
    return hipErrorInvalidValue;
  }
  HD_SWITCH_F32(dq_t)
}
template <int HD> hipError_t dkdv2_t(const AttnArgs &a, hipStream_t st) {
  dim3 grid(((a.n + 63) / 64 + 1) / 2, a.H);
  hipLaunchKernelGGL((attn_bwd_dkdv2_kernel<HD>), grid, dim3(512), 0, st, a);
  return hipGetLastError();
}
hipError_t dkdv_hd(bool bf, int hd, const AttnArgs &a, hipStream_t st) {
  if (bf) {
    switch (hd) {
      case 16: return dkdv2_t<16>(a, st);
      case 32: return dkdv2_t<32>(a, st);
      case 64: return dkdv2_t<64>(a, st);
      case 80: return dkdv2_t<80>(a, st);
      case 96: return dkdv2_t<96>(a, st);
      case 128: return dkdv_t<bf16_t, 128>(a, st);  // its tiles would not fit two LDS stages
    }
    return hipErrorInvalidValue;
  }
  HD_SWITCH_F32(dkdv_t)
}

}  // namespace

size_t attn_ws_floats(int nsplit, int n, int d, int H, int ldl) {
  return (size_t)nsplit * n * d + (size_t)nsplit * H * ldl;
}

int attn_pick_split(int n, int H, int window, int chunk) {
  // aim for two resident work-groups per CU (256 CUs) while every split keeps
  // at least 8 key tiles of 64
  const long wg = (long)((n + 127) / 128) * H;
  int s = (int)((512 + wg - 1) / wg);
  const int tiles = (window + chunk) / 64;
  s = std::min(s, std::max(1, tiles / 8));
  return std::max(1, std::min(s, 8));
}

int attn_fwd_split(int dtype, float sbound, int hd, int n, int H, int window, int chunk) {
  if (!bounded(dtype, sbound, hd)) return attn_pick_split(n, H, window, chunk);
  const long wg = (long)((n + 255) / 256) * H;
  int s = (int)((512 + wg - 1) / wg);
  const int tiles = (window + chunk) / 32;
  s = std::min(s, std::max(1, tiles / 16));
  return std::max(1, std::min(s, 8));
}

bool attn_fwd_f16_ok(int dtype, float sbound, int hd) { return bounded(dtype, sbound, hd) && sbound <= 14.5f; }

bool attn_supported_hd(int hd) { return hd == 16 || hd == 32 || hd == 64 || hd == 80 || hd == 96 || hd == 128; }

hipError_t attn_fwd_launch(int dtype, int hd, const AttnArgs &a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  return fwd_hd(dtype == 1, hd, a, st);
}
hipError_t attn_bwd_dq_launch(int dtype, int hd, const AttnArgs &a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  return dq_hd(dtype == 1, hd, a, st);
}
hipError_t attn_merge_launch(int dtype, int hd, bool dq, const AttnArgs &a, hipStream_t st) {
  if (a.n <= 0 || a.nsplit <= 1) return hipSuccess;
  if (a.nsplit > MERGE_MAX) return hipErrorInvalidValue;
  const long tot = (long)a.n * a.d / 4;
  const dim3 grid((unsigned)((tot + 255) / 256));
  if (dq)
    hipLaunchKernelGGL(attn_dq_merge_kernel, grid, dim3(256), 0, st, a);
  else if (a.o_f16)
    hipLaunchKernelGGL((attn_fwd_merge_kernel<f16_t>), grid, dim3(256), 0, st, a, hd);
  else if (dtype == 1)
    hipLaunchKernelGGL((attn_fwd_merge_kernel<bf16_t>), grid, dim3(256), 0, st, a, hd);
  else
    hipLaunchKernelGGL((attn_fwd_merge_kernel<float>), grid, dim3(256), 0, st, a, hd);
  return hipGetLastError();
}

hipError_t attn_bwd_dkdv_launch(int dtype, int hd, const AttnArgs &a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  return dkdv_hd(dtype == 1, hd, a, st);
}
