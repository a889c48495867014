// Decode attention over the packed TurboQuant cache, for gfx950.
//
// Three launches on the caller's stream:
//   rotate_query   q' = Pi_K q once per query head (and q'' = S q' for QJL keys),
//                  scaled by a per-head power of two and split into float16
//                  hi + lo halves that together carry ~22 bits;
//   decode_scan    one wavefront per (row, KV head, context chunk): scores from
//                  the packed key codes on MFMA, online softmax in registers,
//                  values accumulated in the rotated domain on MFMA;
//   combine        fixed-order merge of the chunk partials, then o = Pi_V^T o'.
//
// Rotated-domain identity used throughout (a reading of the method on the
// ai-accelerate.xyz TurboQuant article, section "TurboQuantの仕組み": the
// rotation is orthogonal, so q . (Pi^T c) = (Pi q) . c and
// sum_t p_t Pi^T c_t = Pi^T sum_t p_t c_t).
//
// MFMA tiling of decode_scan (v_mfma_f32_16x16x32_f16, A 16x32, B 32x16):
//   QK   S^T[token][col] = sum_j Khat[token][j] * Q[col][j]. A rows are 16 of
//        the step's 32 tokens, lane (g, i) holding 8 coordinates of its token
//        unpacked from the key record; B columns are the query operand columns
//        (G <= 8: hi halves in columns 0-7, lo halves in 8-15, so one MFMA
//        produces both and a row rotate by 8 adds them; 8 < G <= 16: separate
//        hi and lo tiles). Row order is chosen so that after two MFMAs lane
//        (g, col) holds the scores of tokens 8g .. 8g+7 of the step.
//   PV   acc^T[coord][col] += sum_t Vhat^T[coord][t] * P^T[t][col]. B is the
//        probability operand, which is exactly what the QK lanes hold; A is
//        unpacked from the 8-token value blocks, lane (g, i) reading the 24-byte
//        (3-bit) slice of block g that holds coordinates 8i .. 8i+7.
//   Codes become float16 pairs through a lookup table in LDS indexed by two
//   adjacent codes (2*bits wide field), replicated once per lane so that the
//   64 lanes of a wavefront never share a bank.
#include <math.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float bf16_bits_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Select c[idx] for a runtime idx < 16 without dynamic register indexing.
__device__ inline float pick16(const float (&c)[16], int idx) {
  float r = c[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) r = (idx == i) ? c[i] : r;
  return r;
}

// ---------------------------------------------------------------- rotate q --

struct RotQArgs {
  const void* q;
  const float* rot;    // Pi_K
  const float* proj;   // S, or null
  _Float16* qop;       // [B][H_kv][1+qjl][nq][128]
  float* qcs;          // [B][H_kv][2][16]
  int q_dtype, H_q, H_kv, G, nq, qjl, wide;
  float sc1, sc2;
};

// Writes the float16 hi/lo operand columns and per-head power-of-two scales of
// vals[G][128] * sc into part `part` of the operand block of (b, kv).
__device__ void emit_query_operand(const RotQArgs& a, const float* vals, float sc, int part,
                                   int64_t bkv, float* hexp) {
  const int tid = threadIdx.x;
  if (tid < 16) {
    float mx = 0.f;
    if (tid < a.G)
      for (int i = 0; i < kD; ++i) mx = fmaxf(mx, fabsf(vals[tid * kD + i] * sc));
    // scale so that the largest entry lies in [2^13, 2^14)
    int e = (mx > 0.f) ? (__builtin_amdgcn_frexp_expf(mx) - 14) : 0;
    hexp[tid] = (float)e;
    a.qcs[(bkv * 2 + part) * 16 + tid] = ldexpf(1.0f, e);
  }
  __syncthreads();
  _Float16* dst = a.qop + (bkv * (1 + a.qjl) + part) * (int64_t)a.nq * kD;
  for (int idx = tid; idx < a.nq * kD; idx += blockDim.x) {
    const int col = idx / kD, i = idx % kD;
    const int half_cols = a.wide ? 16 : 8;
    const int h = col % half_cols;
    const bool lo = col >= half_cols;
    float v = 0.f;
    if (h < a.G) v = ldexpf(vals[h * kD + i] * sc, -(int)hexp[h]);
    const _Float16 hi = (_Float16)v;
    dst[idx] = lo ? (_Float16)(v - (float)hi) : hi;
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void rotate_query_kernel(RotQArgs a) {
  __shared__ float mat[kD * (kD + 1)];
  __shared__ float qv[16 * kD];
  __shared__ float qr[16 * kD];
  __shared__ float hexp[16];
  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t bkv = (int64_t)b * a.H_kv + kv;
  const int G = a.G;
  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    const int64_t e = ((int64_t)b * a.H_q + (int64_t)kv * G) * kD + idx;
    qv[idx] = a.q_dtype == TQ_BF16 ? bf16_bits_to_f32(((const uint16_t*)a.q)[e]) : ((const float*)a.q)[e];
  }
  for (int idx = tid; idx < kD * kD; idx += blockDim.x) mat[(idx / kD) * (kD + 1) + idx % kD] = a.rot[idx];
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    const int h = idx / kD, i = idx % kD;
    float s = 0.f;
    for (int j = 0; j < kD; ++j) s = fmaf(mat[i * (kD + 1) + j], qv[h * kD + j], s);
    qr[idx] = s;
  }
  __syncthreads();
  emit_query_operand(a, qr, a.sc1, 0, bkv, hexp);
  if (a.qjl) {
    for (int idx = tid; idx < kD * kD; idx += blockDim.x) mat[(idx / kD) * (kD + 1) + idx % kD] = a.proj[idx];
    __syncthreads();
    for (int idx = tid; idx < G * kD; idx += blockDim.x) {
      const int h = idx / kD, i = idx % kD;
      float s = 0.f;
      for (int j = 0; j < kD; ++j) s = fmaf(mat[i * (kD + 1) + j], qr[h * kD + j], s);
      qv[idx] = s;
    }
    __syncthreads();
    emit_query_operand(a, qv, a.sc2, 1, bkv, hexp);
  }
}

// ------------------------------------------------------------------- scan --

struct ScanArgs {
  const uint32_t* kcodes;
  const float* knorms;
  const uint32_t* ksigns;
  const float* kgamma;
  const uint32_t* vcodes;
  const float* vnorms;
  const _Float16* qop;
  const float* qcs;
  const int32_t* ctx_lens;
  float* ml;     // [B][H_q][n_split][2]
  float* acc;    // [B][H_q][n_split][128]
  int64_t TcK, TcV;
  int H_kv, H_q, G, T, n_split, chunk, nq;
  float inv_sqrt_d;
  float kc[16], vc[16];
};

// A operand of the QK MFMA for step KK: coordinates 32g + 8KK + 0..7 of the
// lane's token, from the lane's KB-word slice (coordinates 32g .. 32g+31).
template <int KB, int KK>
__device__ inline half8 key_operand(const uint32_t* w, const uint32_t* lut, int lane) {
  uint32_t r[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    uint32_t f;
    switch (pp) {
      case 0: f = field<2 * KB * (4 * KK + 0), 2 * KB>(w); break;
      case 1: f = field<2 * KB * (4 * KK + 1), 2 * KB>(w); break;
      case 2: f = field<2 * KB * (4 * KK + 2), 2 * KB>(w); break;
      default: f = field<2 * KB * (4 * KK + 3), 2 * KB>(w); break;
    }
    r[pp] = lut[(f << 6) | lane];
  }
  return words_to_half8(r[0], r[1], r[2], r[3]);
}

// A operand of the PV MFMA for coordinate block NB: value codes of the 8 tokens
// of the lane's block at coordinate 8i + NB (i = lane % 16), from the lane's
// 2*VB-word slice of the block record (coordinates 8i .. 8i+7).
template <int VB, int NB>
__device__ inline half8 value_operand(const uint32_t* w, const uint32_t* lut, int lane) {
  uint32_t r[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint32_t f;
    switch (s) {
      case 0: f = field<8 * VB * NB + 2 * VB * 0, 2 * VB>(w); break;
      case 1: f = field<8 * VB * NB + 2 * VB * 1, 2 * VB>(w); break;
      case 2: f = field<8 * VB * NB + 2 * VB * 2, 2 * VB>(w); break;
      default: f = field<8 * VB * NB + 2 * VB * 3, 2 * VB>(w); break;
    }
    r[s] = lut[(f << 6) | lane];
  }
  return words_to_half8(r[0], r[1], r[2], r[3]);
}

// A operand of the QJL MFMA for step KK: +-1 for coordinates 32g + 8KK + 0..7.
template <int KK>
__device__ inline half8 sign_operand(uint32_t w, const uint32_t* lut, int lane) {
  uint32_t r[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const uint32_t f = __builtin_amdgcn_ubfe(w, 8 * KK + 2 * pp, 2);
    r[pp] = lut[(f << 6) | lane];
  }
  return words_to_half8(r[0], r[1], r[2], r[3]);
}

template <int KB, int VB, int QJL, int WIDE>
__global__ __launch_bounds__(256) void decode_scan_kernel(ScanArgs a) {
  constexpr int NK = 1 << (2 * KB), NV = 1 << (2 * VB), NS = QJL ? 4 : 0;
  constexpr int KW = 4 * KB;        // words per key token
  constexpr int VBW = 32 * VB;      // words per 8-token value block
  __shared__ uint32_t lut[(NK + NV + NS) * 64];
  uint32_t* lutK = lut;
  uint32_t* lutV = lut + NK * 64;
  uint32_t* lutS = lut + (NK + NV) * 64;

  const int tid = threadIdx.x;
  for (int e = tid; e < NK * 64; e += 256) {
    const int f = e >> 6;
    lutK[e] = pack_half2(pick16(a.kc, f & ((1 << KB) - 1)), pick16(a.kc, f >> KB));
  }
  for (int e = tid; e < NV * 64; e += 256) {
    const int f = e >> 6;
    lutV[e] = pack_half2(pick16(a.vc, f & ((1 << VB) - 1)), pick16(a.vc, f >> VB));
  }
  if constexpr (QJL) {
    for (int e = tid; e < NS * 64; e += 256) {
      const int f = e >> 6;
      lutS[e] = pack_half2((f & 1) ? 1.f : -1.f, (f & 2) ? 1.f : -1.f);
    }
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int split = blockIdx.x * kWavesPerDecodeWG + wave;
  if (split >= a.n_split) return;
  const int kv = blockIdx.y, b = blockIdx.z;
  int ctx = a.ctx_lens ? a.ctx_lens[b] : a.T;
  ctx = ctx < 0 ? 0 : (ctx > a.T ? a.T : ctx);
  const int t_begin = split * a.chunk;
  const int t_end = min(t_begin + a.chunk, ctx);
  const int64_t bkv = (int64_t)b * a.H_kv + kv;

  const auto rk = make_rsrc(a.kcodes + bkv * a.TcK * KW, (uint32_t)(a.TcK * KW * 4));
  const auto rkn = make_rsrc(a.knorms + bkv * a.TcK, (uint32_t)(a.TcK * 4));
  const auto rv = make_rsrc(a.vcodes + bkv * a.TcV * 4 * VB, (uint32_t)(a.TcV * 4 * VB * 4));
  const auto rvn = make_rsrc(a.vnorms + bkv * a.TcV, (uint32_t)(a.TcV * 4));
  // QJL sketch (empty ranges when the keys carry none)
  const auto rs = make_rsrc(QJL ? (const void*)(a.ksigns + bkv * a.TcK * 4) : (const void*)a.knorms,
                            QJL ? (uint32_t)(a.TcK * 16) : 0u);
  const auto rg = make_rsrc(QJL ? (const void*)(a.kgamma + bkv * a.TcK) : (const void*)a.knorms,
                            QJL ? (uint32_t)(a.TcK * 4) : 0u);

  // query operand (B of QK) for this lane: column c, coordinates 32g + 8kk + 0..7
  const _Float16* qb = a.qop + bkv * (1 + QJL) * (int64_t)a.nq * kD;
  half8 q0[4], q1[4], r0[4], r1[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    q0[kk] = *(const half8*)(qb + c * kD + 32 * g + 8 * kk);
    if constexpr (WIDE) q1[kk] = *(const half8*)(qb + (16 + c) * kD + 32 * g + 8 * kk);
    if constexpr (QJL) {
      r0[kk] = *(const half8*)(qb + (a.nq + c) * kD + 32 * g + 8 * kk);
      if constexpr (WIDE) r1[kk] = *(const half8*)(qb + (a.nq + 16 + c) * kD + 32 * g + 8 * kk);
    }
  }
  const int hc = WIDE ? c : (c & 7);
  const float cs1 = a.qcs[(bkv * 2 + 0) * 16 + hc];
  const float cs2 = QJL ? a.qcs[(bkv * 2 + 1) * 16 + hc] : 0.f;

  float m_run = -INFINITY, l_run = 0.f;
  floatx4 acc0[8], acc1[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    acc0[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    acc1[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  for (int t0 = t_begin; t0 < t_end; t0 += kStep) {
    // ---- loads
    uint32_t kw[2][KB];
    uint32_t sw[2] = {0u, 0u};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int tk = t0 + 8 * (c >> 2) + 4 * m + (c & 3);
      bload_words<KB>(rk, (uint32_t)(tk * KW + g * KB) * 4u, kw[m]);
      if constexpr (QJL) sw[m] = bload32(rs, (uint32_t)(tk * 4 + g) * 4u);
    }
    uint32_t vw[2 * VB];
    bload_words<2 * VB>(rv, (uint32_t)((t0 / 8 + g) * VBW + c * 2 * VB) * 4u, vw);
    const int tg = t0 + 8 * g;
    float kn[8], vn[8], kg[8];
    {
      u32x4 x0 = bload128(rkn, (uint32_t)tg * 4u), x1 = bload128(rkn, (uint32_t)(tg + 4) * 4u);
      u32x4 y0 = bload128(rvn, (uint32_t)tg * 4u), y1 = bload128(rvn, (uint32_t)(tg + 4) * 4u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kn[e] = __uint_as_float(x0[e]);
        kn[4 + e] = __uint_as_float(x1[e]);
        vn[e] = __uint_as_float(y0[e]);
        vn[4 + e] = __uint_as_float(y1[e]);
      }
      if constexpr (QJL) {
        u32x4 z0 = bload128(rg, (uint32_t)tg * 4u), z1 = bload128(rg, (uint32_t)(tg + 4) * 4u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kg[e] = __uint_as_float(z0[e]);
          kg[4 + e] = __uint_as_float(z1[e]);
        }
      }
    }

    // ---- scores on MFMA
    floatx4 s0[2], s1[2], z0[2], z1[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      s0[m] = floatx4{0.f, 0.f, 0.f, 0.f};
      s1[m] = s0[m];
      z0[m] = s0[m];
      z1[m] = s0[m];
      half8 ka;
      ka = key_operand<KB, 0>(kw[m], lutK, lane);
      s0[m] = mfma16(ka, q0[0], s0[m]);
      if constexpr (WIDE) s1[m] = mfma16(ka, q1[0], s1[m]);
      ka = key_operand<KB, 1>(kw[m], lutK, lane);
      s0[m] = mfma16(ka, q0[1], s0[m]);
      if constexpr (WIDE) s1[m] = mfma16(ka, q1[1], s1[m]);
      ka = key_operand<KB, 2>(kw[m], lutK, lane);
      s0[m] = mfma16(ka, q0[2], s0[m]);
      if constexpr (WIDE) s1[m] = mfma16(ka, q1[2], s1[m]);
      ka = key_operand<KB, 3>(kw[m], lutK, lane);
      s0[m] = mfma16(ka, q0[3], s0[m]);
      if constexpr (WIDE) s1[m] = mfma16(ka, q1[3], s1[m]);
      if constexpr (QJL) {
        half8 sa;
        sa = sign_operand<0>(sw[m], lutS, lane);
        z0[m] = mfma16(sa, r0[0], z0[m]);
        if constexpr (WIDE) z1[m] = mfma16(sa, r1[0], z1[m]);
        sa = sign_operand<1>(sw[m], lutS, lane);
        z0[m] = mfma16(sa, r0[1], z0[m]);
        if constexpr (WIDE) z1[m] = mfma16(sa, r1[1], z1[m]);
        sa = sign_operand<2>(sw[m], lutS, lane);
        z0[m] = mfma16(sa, r0[2], z0[m]);
        if constexpr (WIDE) z1[m] = mfma16(sa, r1[2], z1[m]);
        sa = sign_operand<3>(sw[m], lutS, lane);
        z0[m] = mfma16(sa, r0[3], z0[m]);
        if constexpr (WIDE) z1[m] = mfma16(sa, r1[3], z1[m]);
      }
    }

    // ---- online softmax (log2 domain; the query operand already carries log2 e)
    float sc[8];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * m + r;
        float x = s0[m][r];
        x += WIDE ? s1[m][r] : dpp_ror8(x);
        float val = x * cs1;
        if constexpr (QJL) {
          float y = z0[m][r];
          y += WIDE ? z1[m][r] : dpp_ror8(y);
          val = fmaf(y * cs2, kg[e], val);
        }
        val *= kn[e];
        sc[e] = (tg + e < t_end) ? val : -INFINITY;
      }
    }
    float tmax = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, sc[e]);
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(sc[e] - m_new);
      psum += p[e];
    }
    l_run = fmaf(l_run, alpha, psum);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        acc0[nb] *= alpha;
        if constexpr (WIDE) acc1[nb] *= alpha;
      }
    }
    m_run = m_new;

    // ---- probability operand (B of PV): weight p * |v| / sqrt(d) as float16 hi or lo
    uint32_t pw0[4], pw1[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float w[2];
      _Float16 hi[2], lo[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * k + u;
        w[u] = (tg + e < t_end) ? p[e] * vn[e] * a.inv_sqrt_d : 0.f;
        hi[u] = (_Float16)w[u];
        lo[u] = (_Float16)(w[u] - (float)hi[u]);
      }
      if constexpr (WIDE) {
        pw0[k] = __builtin_bit_cast(uint32_t, half2v{hi[0], hi[1]});
        pw1[k] = __builtin_bit_cast(uint32_t, half2v{lo[0], lo[1]});
      } else {
        pw0[k] = (c < 8) ? __builtin_bit_cast(uint32_t, half2v{hi[0], hi[1]})
                         : __builtin_bit_cast(uint32_t, half2v{lo[0], lo[1]});
      }
    }
    const half8 pb0 = words_to_half8(pw0[0], pw0[1], pw0[2], pw0[3]);
    half8 pb1;
    if constexpr (WIDE) pb1 = words_to_half8(pw1[0], pw1[1], pw1[2], pw1[3]);

    // ---- values on MFMA (rotated domain)
#define TQ_PV(NB)                                                   \
    {                                                               \
      const half8 va = value_operand<VB, NB>(vw, lutV, lane);       \
      acc0[NB] = mfma16(va, pb0, acc0[NB]);                         \
      if constexpr (WIDE) acc1[NB] = mfma16(va, pb1, acc1[NB]);     \
    }
    TQ_PV(0) TQ_PV(1) TQ_PV(2) TQ_PV(3) TQ_PV(4) TQ_PV(5) TQ_PV(6) TQ_PV(7)
#undef TQ_PV
  }

  // ---- partial of this chunk: lane (g, c) holds coordinates 32g + 8r + nb of column c
  float o[8][4];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = acc0[nb][r];
      x += WIDE ? acc1[nb][r] : dpp_ror8(x);
      o[nb][r] = x;
    }
  }
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  if (c < a.G) {
    const int h = kv * a.G + c;
    const int64_t pidx = ((int64_t)b * a.H_q + h) * a.n_split + split;
    float* dst = a.acc + pidx * kD + 32 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *(floatx4*)(dst + 8 * r) = floatx4{o[0][r], o[1][r], o[2][r], o[3][r]};
      *(floatx4*)(dst + 8 * r + 4) = floatx4{o[4][r], o[5][r], o[6][r], o[7][r]};
    }
    if (g == 0) {
      a.ml[pidx * 2] = m_run;
      a.ml[pidx * 2 + 1] = l_run;
    }
  }
}

// ---------------------------------------------------------------- combine --

__global__ __launch_bounds__(128) void combine_kernel(const float* ml, const float* acc, const float* rotV,
                                                       float* out, int H_q, int n_split) {
  __shared__ float ov[kD];
  const int h = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
  const int64_t bh = (int64_t)b * H_q + h;
  const float* mlb = ml + bh * n_split * 2;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, mlb[2 * s]);
  float num = 0.f, den = 0.f;
  if (M > -INFINITY) {
    const float* ab = acc + bh * n_split * kD;
    for (int s = 0; s < n_split; ++s) {
      const float m = mlb[2 * s];
      const float w = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M);
      den = fmaf(w, mlb[2 * s + 1], den);
      num = fmaf(w, ab[(int64_t)s * kD + j], num);
    }
  }
  ov[j] = den > 0.f ? num / den : 0.f;
  __syncthreads();
  float r = 0.f;
  for (int jj = 0; jj < kD; ++jj) r = fmaf(rotV[jj * kD + j], ov[jj], r);
  out[bh * kD + j] = r;
}

template <int KB, int VB, int QJL, int WIDE>
hipError_t launch_scan(const DecodePlan& p, const ScanArgs& sa, hipStream_t stream) {
  dim3 grid((p.n_split + kWavesPerDecodeWG - 1) / kWavesPerDecodeWG, (unsigned)p.H_kv, (unsigned)p.B);
  hipLaunchKernelGGL((decode_scan_kernel<KB, VB, QJL, WIDE>), grid, dim3(256), 0, stream, sa);
  return hipGetLastError();
}

template <int KB, int VB, int QJL>
hipError_t dispatch_wide(const DecodePlan& p, const ScanArgs& sa, hipStream_t s) {
  return p.wide ? launch_scan<KB, VB, QJL, 1>(p, sa, s) : launch_scan<KB, VB, QJL, 0>(p, sa, s);
}

template <int KB, int VB>
hipError_t dispatch_qjl(const DecodePlan& p, const ScanArgs& sa, hipStream_t s) {
  return p.qjl ? dispatch_wide<KB, VB, 1>(p, sa, s) : dispatch_wide<KB, VB, 0>(p, sa, s);
}

template <int KB>
hipError_t dispatch_vb(int vb, const DecodePlan& p, const ScanArgs& sa, hipStream_t s) {
  switch (vb) {
    case 2: return dispatch_qjl<KB, 2>(p, sa, s);
    case 3: return dispatch_qjl<KB, 3>(p, sa, s);
    default: return dispatch_qjl<KB, 4>(p, sa, s);
  }
}

}  // namespace

hipError_t launch_decode(const DecodePlan& p, const tq_cache* k, const tq_cache* v, const void* q,
                         int q_dtype, const int32_t* ctx_lens, float scale, float* out, void* ws,
                         hipStream_t stream) {
  char* base = (char*)ws;
  _Float16* qop = (_Float16*)(base + p.off_qop);
  float* qcs = (float*)(base + p.off_qcs);
  float* ml = (float*)(base + p.off_ml);
  float* acc = (float*)(base + p.off_acc);

  RotQArgs ra;
  ra.q = q;
  ra.rot = k->rot;
  ra.proj = p.qjl ? k->qjl_proj : nullptr;
  ra.qop = qop;
  ra.qcs = qcs;
  ra.q_dtype = q_dtype;
  ra.H_q = (int)p.H_q;
  ra.H_kv = (int)p.H_kv;
  ra.G = p.G;
  ra.nq = p.nq;
  ra.qjl = p.qjl;
  ra.wide = p.wide;
  const float inv_sqrt_d = 1.0f / sqrtf((float)kD);
  ra.sc1 = scale * kLog2e * inv_sqrt_d;
  ra.sc2 = scale * kLog2e * sqrtf((float)M_PI / 2.0f) / (float)kD;
  hipLaunchKernelGGL(rotate_query_kernel, dim3((unsigned)p.H_kv, (unsigned)p.B), dim3(256), 0, stream, ra);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  ScanArgs sa;
  sa.kcodes = k->codes;
  sa.knorms = k->norms;
  sa.ksigns = k->qjl_signs;
  sa.kgamma = k->qjl_gamma;
  sa.vcodes = v->codes;
  sa.vnorms = v->norms;
  sa.qop = qop;
  sa.qcs = qcs;
  sa.ctx_lens = ctx_lens;
  sa.ml = ml;
  sa.acc = acc;
  sa.TcK = k->T_cap;
  sa.TcV = v->T_cap;
  sa.H_kv = (int)p.H_kv;
  sa.H_q = (int)p.H_q;
  sa.G = p.G;
  sa.T = (int)p.T;
  sa.n_split = p.n_split;
  sa.chunk = p.chunk;
  sa.nq = p.nq;
  sa.inv_sqrt_d = inv_sqrt_d;
  for (int i = 0; i < 16; ++i) {
    sa.kc[i] = i < (1 << k->bits) ? k->centroids[i] : 0.f;
    sa.vc[i] = i < (1 << v->bits) ? v->centroids[i] : 0.f;
  }
  switch (k->bits) {
    case 2: err = dispatch_vb<2>(v->bits, p, sa, stream); break;
    case 3: err = dispatch_vb<3>(v->bits, p, sa, stream); break;
    default: err = dispatch_vb<4>(v->bits, p, sa, stream); break;
  }
  if (err != hipSuccess) return err;

  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)p.H_q, (unsigned)p.B), dim3(128), 0, stream, ml, acc,
                     v->rot, out, (int)p.H_q, p.n_split);
  return hipGetLastError();
}

}  // namespace tq
