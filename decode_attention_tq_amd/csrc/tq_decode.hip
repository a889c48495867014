// Decode attention over the packed TurboQuant cache, for gfx950.
//
// Three launches on the caller's stream:
//   rotate_query   q' = Pi_K q once per query head (and q'' = S q' for QJL keys),
//                  scaled by a per-head power of two and split into float16
//                  hi + lo halves that together carry ~22 bits;
//   decode_scan    one workgroup of 4 wavefronts per (row, KV head, context
//                  chunk); each wavefront streams a quarter of the chunk: scores
//                  from the packed key codes on MFMA, online softmax in
//                  registers, values accumulated in the rotated domain on MFMA;
//                  the 4 wavefront partials are merged in LDS and written out;
//   combine        fixed-order merge of the chunk partials of each query head,
//                  then the single inverse rotation o = Pi_V^T o'.
// (Merging across workgroups inside decode_scan would need a device-scope
// release per workgroup, which on this multi-die part writes back L2; the
// kernel boundary provides that ordering once.)
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
//        weight operand, which is exactly what the QK lanes hold; A is unpacked
//        from the 8-token value blocks, lane (g, i) reading the 24-byte (3-bit)
//        slice of block g that holds coordinates 8i .. 8i+7.
//   Codes become float16 pairs through a lookup table in LDS indexed by two
//   adjacent codes (2*bits wide field), replicated kLutRep times so that lanes
//   of a wavefront read distinct banks (lane l reads replica l % kLutRep).
//
// Online softmax (log2 domain; the query operand carries log2(e) * scale / sqrt(d)):
// the reference maximum m only moves when a score exceeds it by more than
// kSlack, so the rescale of the accumulators is rare; weights are
// 2^(s - m - kShift) * |v| with kShift = kSlack + log2(sqrt(d)), which keeps
// every weight operand at or below |v| / sqrt(d) (float16 range for |v| < 7e5)
// and leaves one 1/sqrt(d) for the combine.
#include <math.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 2.0f;
constexpr float kShift = kSlack + 3.5f;   // + log2(sqrt(128))
constexpr int kLutRep = 32;              // LUT replicas (power of two)
constexpr int kLutShift = 5;             // log2(kLutRep)

__device__ inline float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

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

constexpr int kRowPad = kD + 4;   // LDS row stride of a staged matrix (16-byte aligned rows)

// Stage the d x d matrix M into LDS (row stride kRowPad) with coalesced 16-byte
// loads, all of a thread's loads in flight at once.
__device__ void stage_rows(const float* M, float* lds) {
  constexpr int PER = kD * kD / 4 / 256;
  float4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) v[k] = ((const float4*)M)[threadIdx.x + 256 * k];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int f = threadIdx.x + 256 * k;
    *(float4*)(lds + (f >> 5) * kRowPad + 4 * (f & 31)) = v[k];
  }
}

// out[h][i] = sum_j M[i][j] in[h][j] for the G heads; thread (i, hh) computes
// heads hh, hh+2, ... from the staged rows (LDS) and inputs (LDS broadcast).
__device__ void matvec_rows(const float* Ml, const float* in, float* out, int G) {
  const int i = threadIdx.x & 127, hh = threadIdx.x >> 7;
  const float4* row = (const float4*)(Ml + i * kRowPad);
  for (int h = hh; h < G; h += 2) {
    const float4* x = (const float4*)(in + h * kD);
    float acc = 0.f;
#pragma unroll 8
    for (int j4 = 0; j4 < kD / 4; ++j4) {
      const float4 r = row[j4], v = x[j4];
      acc = fmaf(r.w, v.w, fmaf(r.z, v.z, fmaf(r.y, v.y, fmaf(r.x, v.x, acc))));
    }
    out[h * kD + i] = acc;
  }
}

// Writes the float16 hi/lo operand columns and per-head power-of-two scales of
// vals[G][128] * sc into part `part` of the operand block of (b, kv).
__device__ void emit_query_operand(const RotQArgs& a, const float* vals, float sc, int part,
                                   int64_t bkv, int* hexp) {
  const int tid = threadIdx.x;
  {
    // thread (h, seg): max over 8 entries, then over the 16 segments of the head
    const int h = tid >> 4, seg = tid & 15;
    float mx = 0.f;
    if (h < a.G) {
#pragma unroll
      for (int k = 0; k < 8; ++k) mx = fmaxf(mx, fabsf(vals[h * kD + 8 * seg + k] * sc));
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    if (seg == 0) {
      // scale so that the largest entry lies in [2^13, 2^14)
      const int e = (mx > 0.f) ? (__builtin_amdgcn_frexp_expf(mx) - 14) : 0;
      hexp[h] = e;
      a.qcs[(bkv * 2 + part) * 16 + h] = ldexpf(1.0f, e);
    }
  }
  __syncthreads();
  _Float16* dst = a.qop + (bkv * (1 + a.qjl) + part) * (int64_t)a.nq * kD;
  const int half_cols = a.wide ? 16 : 8;
  for (int idx = tid; idx < a.nq * kD; idx += blockDim.x) {
    const int col = idx / kD, i = idx % kD;
    const int h = col % half_cols;
    const bool lo = col >= half_cols;
    float v = 0.f;
    if (h < a.G) v = ldexpf(vals[h * kD + i] * sc, -hexp[h]);
    const _Float16 hi = (_Float16)v;
    dst[idx] = lo ? (_Float16)(v - (float)hi) : hi;
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void rotate_query_kernel(RotQArgs a) {
  __shared__ __align__(16) float mat[kD * kRowPad];
  __shared__ __align__(16) float qv[16 * kD];
  __shared__ __align__(16) float qr[16 * kD];
  __shared__ int hexp[16];
  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t bkv = (int64_t)b * a.H_kv + kv;
  const int G = a.G;
  stage_rows(a.rot, mat);
  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    const int64_t e = ((int64_t)b * a.H_q + (int64_t)kv * G) * kD + idx;
    qv[idx] = a.q_dtype == TQ_BF16 ? bf16_bits_to_f32(((const uint16_t*)a.q)[e]) : ((const float*)a.q)[e];
  }
  __syncthreads();
  matvec_rows(mat, qv, qr, G);          // q' = Pi q
  __syncthreads();
  emit_query_operand(a, qr, a.sc1, 0, bkv, hexp);
  if (a.qjl) {
    stage_rows(a.proj, mat);
    __syncthreads();
    matvec_rows(mat, qr, qv, G);        // q'' = S q'
    __syncthreads();
    emit_query_operand(a, qv, a.sc2, 1, bkv, hexp);
  }
}

// Query operand without QJL: workgroup (kv, b, chunk) produces coordinates
// 32*chunk .. 32*chunk+31 of q' = Pi q for the G heads of KV head kv. The
// per-head power of two comes from |q| (the rotation preserves the norm, so
// every |q'_i| <= |q|), which keeps the chunks independent.
constexpr int kRotChunks = 4;

__global__ __launch_bounds__(256) void rotate_query_chunk_kernel(RotQArgs a) {
  __shared__ __align__(16) float qv[16 * kD];
  __shared__ int hexp[16];
  const int kv = blockIdx.x, b = blockIdx.y, chunk = blockIdx.z, tid = threadIdx.x;
  const int64_t bkv = (int64_t)b * a.H_kv + kv;
  const int G = a.G;
  // thread (i, hq): output coordinate 32*chunk + i, heads hq, hq + 8
  const int i = 32 * chunk + (tid & 31), hq = tid >> 5;
  const float4* rowp = (const float4*)(a.rot + i * kD);
  float4 row[kD / 4];
#pragma unroll
  for (int j4 = 0; j4 < kD / 4; ++j4) row[j4] = rowp[j4];
  for (int idx = tid; idx < G * kD; idx += 256) {
    const int64_t e = ((int64_t)b * a.H_q + (int64_t)kv * G) * kD + idx;
    qv[idx] = a.q_dtype == TQ_BF16 ? bf16_bits_to_f32(((const uint16_t*)a.q)[e]) : ((const float*)a.q)[e];
  }
  __syncthreads();
  {
    // thread (h, seg): sum of squares and largest magnitude over 8 entries,
    // then over the 16 segments of the head
    const int h = tid >> 4, seg = tid & 15;
    float ss = 0.f, mx = 0.f;
    if (h < G) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float v = qv[h * kD + 8 * seg + k];
        ss = fmaf(v, v, ss);
        mx = fmaxf(mx, fabsf(v));
      }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      ss += __shfl_xor(ss, m);
      mx = fmaxf(mx, __shfl_xor(mx, m));
    }
    if (seg == 0) {
      // |q| bounds every |q'_i|; sqrt(d) * max_j |q_j| bounds |q| and stays
      // finite where the sum of squares overflows
      const float bound = fminf(sqrtf(ss), mx * 11.3137085f) * a.sc1;
      const int e = (bound > 0.f) ? (__builtin_amdgcn_frexp_expf(bound) - 13) : 0;
      hexp[h] = e;
      if (chunk == 0) a.qcs[(bkv * 2) * 16 + h] = ldexpf(1.0f, e);
    }
  }
  __syncthreads();
  _Float16* dst = a.qop + bkv * (int64_t)a.nq * kD;
  const int half_cols = a.wide ? 16 : 8;
  for (int h = hq; h < half_cols; h += 8) {
    float acc = 0.f;
    if (h < G) {
      const float4* x = (const float4*)(qv + h * kD);
#pragma unroll
      for (int j4 = 0; j4 < kD / 4; ++j4) {
        const float4 v = x[j4];
        acc = fmaf(row[j4].w, v.w, fmaf(row[j4].z, v.z, fmaf(row[j4].y, v.y, fmaf(row[j4].x, v.x, acc))));
      }
      acc = ldexpf(acc * a.sc1, -hexp[h]);
    }
    const _Float16 hi = (_Float16)acc;
    dst[h * kD + i] = hi;
    dst[(half_cols + h) * kD + i] = (_Float16)(acc - (float)hi);
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
  int H_kv, H_q, G, T, n_split, wg_chunk, wave_chunk, nq;
  float kc[16], vc[16];
};

// A operand of the QK MFMA for step KK: coordinates 32g + 8KK + 0..7 of the
// lane's token, from the lane's KB-word slice (coordinates 32g .. 32g+31).
template <int KB, int KK>
__device__ inline half8 key_operand(const uint32_t* w, const uint32_t* lut, int lane) {
  const uint32_t r0 = lut[(field<2 * KB * (4 * KK + 0), 2 * KB>(w) << kLutShift) | lane];
  const uint32_t r1 = lut[(field<2 * KB * (4 * KK + 1), 2 * KB>(w) << kLutShift) | lane];
  const uint32_t r2 = lut[(field<2 * KB * (4 * KK + 2), 2 * KB>(w) << kLutShift) | lane];
  const uint32_t r3 = lut[(field<2 * KB * (4 * KK + 3), 2 * KB>(w) << kLutShift) | lane];
  return words_to_half8(r0, r1, r2, r3);
}

// A operand of the PV MFMA for coordinate block NB: value codes of the 8 tokens
// of the lane's block at coordinate 8i + NB (i = lane % 16), from the lane's
// 2*VB-word slice of the block record (coordinates 8i .. 8i+7).
template <int VB, int NB>
__device__ inline half8 value_operand(const uint32_t* w, const uint32_t* lut, int lane) {
  const uint32_t r0 = lut[(field<8 * VB * NB + 2 * VB * 0, 2 * VB>(w) << kLutShift) | lane];
  const uint32_t r1 = lut[(field<8 * VB * NB + 2 * VB * 1, 2 * VB>(w) << kLutShift) | lane];
  const uint32_t r2 = lut[(field<8 * VB * NB + 2 * VB * 2, 2 * VB>(w) << kLutShift) | lane];
  const uint32_t r3 = lut[(field<8 * VB * NB + 2 * VB * 3, 2 * VB>(w) << kLutShift) | lane];
  return words_to_half8(r0, r1, r2, r3);
}

// A operand of the QJL MFMA for step KK: +-1 for coordinates 32g + 8KK + 0..7.
template <int KK>
__device__ inline half8 sign_operand(uint32_t w, const uint32_t* lut, int lane) {
  uint32_t r[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) r[pp] = lut[(__builtin_amdgcn_ubfe(w, 8 * KK + 2 * pp, 2) << kLutShift) | lane];
  return words_to_half8(r[0], r[1], r[2], r[3]);
}

// Per-lane byte offsets inside the streams of one (row, KV head); a step adds a
// wave-uniform offset that travels in the scalar offset of the buffer loads.
struct LaneOffsets {
  uint32_t k[2];     // key record slice of MFMA row block m
  uint32_t s[2];     // QJL sign word of MFMA row block m
  uint32_t v;        // value block slice
  uint32_t n;        // norms (and gammas) of the lane's tokens
};

// Raw bytes of one 32-token step for one lane. Norms: for G <= 8 the two lanes
// of a hi/lo column pair split the 8 tokens of their row block (lane half hf
// takes tokens 4hf .. 4hf+3); for 8 < G <= 16 every lane takes all 8.
template <int KB, int VB, int QJL, int WIDE>
struct StepData {
  static constexpr int NT = WIDE ? 8 : 4;
  uint32_t kw[2][KB];
  uint32_t sw[2];
  uint32_t vw[2 * VB];
};

struct Streams {
  __amdgpu_buffer_rsrc_t rk, rkn, rv, rvn, rs, rg;
};

template <int N>
__device__ inline void bload_words_s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* w) {
  if constexpr (N == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (N == 3) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  } else if constexpr (N == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (N == 6) {
    bload_words_s<3>(r, voff, soff, w);
    bload_words_s<3>(r, voff + 12u, soff, w + 3);
  } else {
    static_assert(N == 8, "unsupported word count");
    bload_words_s<4>(r, voff, soff, w);
    bload_words_s<4>(r, voff + 16u, soff, w + 4);
  }
}

template <int NT>
__device__ inline void bload_floats_s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float* f) {
  uint32_t w[NT];
  bload_words_s<NT>(r, voff, soff, w);
#pragma unroll
  for (int i = 0; i < NT; ++i) f[i] = as_float(w[i]);
}

template <int KB, int VB, int QJL, int WIDE>
__device__ inline void load_step(StepData<KB, VB, QJL, WIDE>& d, const Streams& s, const LaneOffsets& lo, int t0) {
  constexpr int KW = 4 * KB, VBW = 32 * VB;
  const uint32_t st = (uint32_t)t0;   // wave-uniform
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    bload_words_s<KB>(s.rk, lo.k[m], st * (KW * 4u), d.kw[m]);
    if constexpr (QJL) d.sw[m] = __builtin_amdgcn_raw_buffer_load_b32(s.rs, lo.s[m], st * 16u, 0);
  }
  bload_words_s<2 * VB>(s.rv, lo.v, (st / 8u) * (VBW * 4u), d.vw);
}

// Norms (and QJL gammas) of the step: issued when the step starts, consumed
// after the key MFMAs.
template <int NT, int QJL>
struct StepNorms {
  float kn[NT], vn[NT], kg[NT];
};

template <int NT, int QJL>
__device__ inline void load_norms(StepNorms<NT, QJL>& n, const Streams& s, const LaneOffsets& lo, int t0) {
  const uint32_t st = (uint32_t)t0 * 4u;
  bload_floats_s<NT>(s.rkn, lo.n, st, n.kn);
  bload_floats_s<NT>(s.rvn, lo.n, st, n.vn);
  if constexpr (QJL) bload_floats_s<NT>(s.rg, lo.n, st, n.kg);
}

template <int WIDE, int QJL>
struct QOps {
  half8 q1[4], r0[4], r1[4];
  const half8* q0l;   // LDS copy of this lane's column-c operand (4 x 8 halves), shared by the workgroup
  float cs1, cs2;
  bool hf;   // G <= 8: lane holds the lo half of its query column (column >= 8)
};

// Keeps a value opaque to the optimizer inside a loop (no instruction emitted),
// so loads that depend on it are repeated instead of kept live in registers.
__device__ inline uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int WIDE>
struct SoftState {
  float m_ref, m_off, l;
  floatx4 acc0[8], acc1[8];
};

template <int KB, int VB, int QJL, int WIDE, bool MASK>
__device__ __forceinline__ void scan_step(const StepData<KB, VB, QJL, WIDE>& d, const QOps<WIDE, QJL>& q,
                                          SoftState<WIDE>& st, const uint32_t* lutK, const uint32_t* lutV,
                                          const uint32_t* lutS, int lane, int tg, int t_end,
                                          const Streams& sm, const LaneOffsets& lo, int t0) {
  constexpr int NT = StepData<KB, VB, QJL, WIDE>::NT;
  StepNorms<NT, QJL> nm;
  load_norms(nm, sm, lo, t0);
  // ---- scores on MFMA
  half8 q0[4];
  {
    const half8* ql = (const half8*)((const char*)q.q0l + opaque(0u));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) q0[kk] = ql[kk];
  }
  floatx4 s0[2], s1[2], z0[2], z1[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    s0[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    s1[m] = s0[m];
    z0[m] = s0[m];
    z1[m] = s0[m];
#define TQ_QK(KK)                                                   \
    {                                                               \
      const half8 ka = key_operand<KB, KK>(d.kw[m], lutK, lane);    \
      s0[m] = mfma16(ka, q0[KK], s0[m]);                            \
      if constexpr (WIDE) s1[m] = mfma16(ka, q.q1[KK], s1[m]);      \
    }
    TQ_QK(0) TQ_QK(1) TQ_QK(2) TQ_QK(3)
#undef TQ_QK
    if constexpr (QJL) {
#define TQ_QJ(KK)                                                   \
      {                                                             \
        const half8 sa = sign_operand<KK>(d.sw[m], lutS, lane);     \
        z0[m] = mfma16(sa, q.r0[KK], z0[m]);                        \
        if constexpr (WIDE) z1[m] = mfma16(sa, q.r1[KK], z1[m]);    \
      }
      TQ_QJ(0) TQ_QJ(1) TQ_QJ(2) TQ_QJ(3)
#undef TQ_QJ
    }
  }
  const float cs = QJL ? 1.0f : q.cs1;

  if constexpr (!WIDE) {
    // ---- G <= 8: lanes c and c+8 carry the hi and lo halves of one query
    // column. Both add the halves (row rotate by 8); then each takes 4 of the 8
    // tokens of its row block (token 4hf + r is MFMA row block m = hf) for the
    // exponentials, and the two swap their float16 weights at the end.
    float x8[8], z8[8];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = s0[m][r];
        x8[4 * m + r] = x + dpp_ror8(x);
        if constexpr (QJL) {
          const float z = z0[m][r];
          z8[4 * m + r] = z + dpp_ror8(z);
        }
      }
    }
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = q.hf ? x8[4 + r] : x8[r];
      if constexpr (QJL) {
        const float z = q.hf ? z8[4 + r] : z8[r];
        x = fmaf(z * q.cs2, nm.kg[r], x * q.cs1);
      }
      float v = x * nm.kn[r];
      if constexpr (MASK) v = (tg + 4 * (int)q.hf + r < t_end) ? v : -INFINITY;
      y[r] = v;
    }
    // the reference moves only when some score passes it by more than kSlack;
    // then the column maximum is gathered (lanes c, c^8 and the 4 row blocks)
    const float lmax = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
    if (__any(lmax * cs > st.m_ref + kSlack)) {
      float tmax = fmaxf(lmax, dpp_ror8(lmax));
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      const float m_new = fmaxf(st.m_ref, tmax * cs);
      const float alpha = __builtin_amdgcn_exp2f(st.m_ref - m_new);
      st.l *= alpha;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) st.acc0[nb] *= alpha;
      st.m_ref = m_new;
      st.m_off = m_new + kShift;
    }
    float w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(y[r], cs, -st.m_off));
      st.l += p;
      w[r] = p * nm.vn[r];
      if constexpr (MASK) w[r] = (tg + 4 * (int)q.hf + r < t_end) ? w[r] : 0.f;
    }
    // own tokens as float16 hi and lo halves (pairs of tokens per register)
    uint32_t hi2[2], lo2[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const _Float16 h0 = (_Float16)w[2 * k], h1 = (_Float16)w[2 * k + 1];
      hi2[k] = __builtin_bit_cast(uint32_t, half2v{h0, h1});
      lo2[k] = __builtin_bit_cast(uint32_t, half2v{(_Float16)(w[2 * k] - (float)h0),
                                                   (_Float16)(w[2 * k + 1] - (float)h1)});
    }
    // the hi lane keeps hi of tokens 0-3 and needs hi of tokens 4-7 from its partner;
    // the lo lane keeps lo of tokens 4-7 and needs lo of tokens 0-3
    uint32_t op[4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t send = q.hf ? hi2[k] : lo2[k];
      const uint32_t recv = __builtin_amdgcn_update_dpp(0u, send, 0x128, 0xF, 0xF, false);
      op[k] = q.hf ? recv : hi2[k];
      op[2 + k] = q.hf ? lo2[k] : recv;
    }
    const half8 pb0 = words_to_half8(op[0], op[1], op[2], op[3]);
#define TQ_PV(NB)                                                     \
    {                                                                 \
      const half8 va = value_operand<VB, NB>(d.vw, lutV, lane);       \
      st.acc0[NB] = mfma16(va, pb0, st.acc0[NB]);                     \
    }
    TQ_PV(0) TQ_PV(1) TQ_PV(2) TQ_PV(3) TQ_PV(4) TQ_PV(5) TQ_PV(6) TQ_PV(7)
#undef TQ_PV
  } else {
    // ---- 8 < G <= 16: separate hi and lo tiles; every lane holds 8 tokens
    float y[8];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * m + r;
        float x = s0[m][r] + s1[m][r];
        if constexpr (QJL) {
          const float yq = z0[m][r] + z1[m][r];
          x = fmaf(yq * q.cs2, nm.kg[e], x * q.cs1);
        }
        float v = x * nm.kn[e];
        if constexpr (MASK) v = (tg + e < t_end) ? v : -INFINITY;
        y[e] = v;
      }
    }
    const float lmax = fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])), fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
    if (__any(lmax * cs > st.m_ref + kSlack)) {
      float tmax = fmaxf(lmax, shfl_xor_f(lmax, 16));
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      const float m_new = fmaxf(st.m_ref, tmax * cs);
      const float alpha = __builtin_amdgcn_exp2f(st.m_ref - m_new);
      st.l *= alpha;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        st.acc0[nb] *= alpha;
        st.acc1[nb] *= alpha;
      }
      st.m_ref = m_new;
      st.m_off = m_new + kShift;
    }
    uint32_t pw0[4], pw1[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float w2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * k + u;
        const float p = __builtin_amdgcn_exp2f(fmaf(y[e], cs, -st.m_off));
        st.l += p;
        w2[u] = p * nm.vn[e];
        if constexpr (MASK) w2[u] = (tg + e < t_end) ? w2[u] : 0.f;
      }
      const _Float16 h0 = (_Float16)w2[0], h1 = (_Float16)w2[1];
      pw0[k] = __builtin_bit_cast(uint32_t, half2v{h0, h1});
      pw1[k] = __builtin_bit_cast(uint32_t, half2v{(_Float16)(w2[0] - (float)h0), (_Float16)(w2[1] - (float)h1)});
    }
    const half8 pb0 = words_to_half8(pw0[0], pw0[1], pw0[2], pw0[3]);
    const half8 pb1 = words_to_half8(pw1[0], pw1[1], pw1[2], pw1[3]);
#define TQ_PV(NB)                                                     \
    {                                                                 \
      const half8 va = value_operand<VB, NB>(d.vw, lutV, lane);       \
      st.acc0[NB] = mfma16(va, pb0, st.acc0[NB]);                     \
      st.acc1[NB] = mfma16(va, pb1, st.acc1[NB]);                     \
    }
    TQ_PV(0) TQ_PV(1) TQ_PV(2) TQ_PV(3) TQ_PV(4) TQ_PV(5) TQ_PV(6) TQ_PV(7)
#undef TQ_PV
  }
}


// merge buffer: [wave][column][128 + 2] floats, 8 columns (G <= 8) or 16
template <int WIDE>
constexpr int merge_cols() { return WIDE ? 16 : 8; }

// LDS: lookup tables, then the query operand of the workgroup's KV head
// (16 columns x 128 halves); the merge area reuses both after the scan.
constexpr int kQopWords = 16 * kD / 2;

template <int KB, int VB, int QJL, int WIDE>
constexpr int scan_lds_words() {
  constexpr int lut = ((1 << (2 * KB)) + (1 << (2 * VB)) + (QJL ? 4 : 0)) * kLutRep + kQopWords;
  constexpr int mrg = kWavesPerDecodeWG * merge_cols<WIDE>() * (kD + 2);
  return lut > mrg ? lut : mrg;
}

// 4 wavefronts per SIMD (<= 128 VGPRs) keeps all 4 workgroups of a compute
// unit resident for the common tiles; the QJL and G > 8 tiles carry more
// operands and run 2 per SIMD without spilling.
template <int QJL, int WIDE>
constexpr int scan_waves_per_eu() { return (QJL || WIDE) ? 2 : 4; }

template <int KB, int VB, int QJL, int WIDE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(scan_waves_per_eu<QJL, WIDE>(), 4)))
void decode_scan_kernel(ScanArgs a) {
  constexpr int NK = 1 << (2 * KB), NV = 1 << (2 * VB), NS = QJL ? 4 : 0;
  constexpr int KW = 4 * KB;
  constexpr int MC = merge_cols<WIDE>();
  __shared__ uint32_t smem[scan_lds_words<KB, VB, QJL, WIDE>()];
  uint32_t* lutK = smem;
  uint32_t* lutV = smem + NK * kLutRep;
  uint32_t* lutS = smem + (NK + NV) * kLutRep;
  uint32_t* qlds = smem + (NK + NV + NS) * kLutRep;   // 16-byte aligned (multiple of 32 words)

  const int tid = threadIdx.x;
  for (int e = tid; e < NK * kLutRep; e += 256) {
    const int f = e >> kLutShift;
    lutK[e] = pack_half2(pick16(a.kc, f & ((1 << KB) - 1)), pick16(a.kc, f >> KB));
  }
  for (int e = tid; e < NV * kLutRep; e += 256) {
    const int f = e >> kLutShift;
    lutV[e] = pack_half2(pick16(a.vc, f & ((1 << VB) - 1)), pick16(a.vc, f >> VB));
  }
  if constexpr (QJL) {
    for (int e = tid; e < NS * kLutRep; e += 256) {
      const int f = e >> kLutShift;
      lutS[e] = pack_half2((f & 1) ? 1.f : -1.f, (f & 2) ? 1.f : -1.f);
    }
  }
  {
    // query operand columns 0-15 of this (row, KV head): 4 KB, one 16-byte load per thread
    const int64_t bkv0 = (int64_t)blockIdx.z * a.H_kv + blockIdx.y;
    const u32x4* src = (const u32x4*)(a.qop + bkv0 * (1 + QJL) * (int64_t)a.nq * kD);
    ((u32x4*)qlds)[tid] = src[tid];
  }
  __syncthreads();

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const int lrep = lane & (kLutRep - 1);
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  int ctx = a.ctx_lens ? a.ctx_lens[b] : a.T;
  ctx = ctx < 0 ? 0 : (ctx > a.T ? a.T : ctx);
  const int t_begin = split * a.wg_chunk + wave * a.wave_chunk;
  const int t_end = min(t_begin + a.wave_chunk, ctx);
  const int64_t bkv = (int64_t)b * a.H_kv + kv;

  Streams s;
  s.rk = make_rsrc(a.kcodes + bkv * a.TcK * KW, (uint32_t)(a.TcK * KW * 4));
  s.rkn = make_rsrc(a.knorms + bkv * a.TcK, (uint32_t)(a.TcK * 4));
  s.rv = make_rsrc(a.vcodes + bkv * a.TcV * 4 * VB, (uint32_t)(a.TcV * 4 * VB * 4));
  s.rvn = make_rsrc(a.vnorms + bkv * a.TcV, (uint32_t)(a.TcV * 4));
  // QJL sketch (empty ranges when the keys carry none)
  s.rs = make_rsrc(QJL ? (const void*)(a.ksigns + bkv * a.TcK * 4) : (const void*)a.knorms,
                   QJL ? (uint32_t)(a.TcK * 16) : 0u);
  s.rg = make_rsrc(QJL ? (const void*)(a.kgamma + bkv * a.TcK) : (const void*)a.knorms,
                   QJL ? (uint32_t)(a.TcK * 4) : 0u);
  const bool hf = !WIDE && c >= 8;
  LaneOffsets lo;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int tk = 8 * (c >> 2) + 4 * m + (c & 3);   // MFMA row c of row block m
    lo.k[m] = (uint32_t)(tk * KW + g * KB) * 4u;
    lo.s[m] = (uint32_t)(tk * 4 + g) * 4u;
  }
  lo.v = (uint32_t)(g * 32 * VB + c * 2 * VB) * 4u;
  lo.n = (uint32_t)(8 * g + (hf ? 4 : 0)) * 4u;

  // query operand (B of QK) for this lane: column c, coordinates 32g + 8kk + 0..7
  QOps<WIDE, QJL> q;
  const _Float16* qb = a.qop + bkv * (1 + QJL) * (int64_t)a.nq * kD;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if constexpr (WIDE) q.q1[kk] = *(const half8*)(qb + (16 + c) * kD + 32 * g + 8 * kk);
    if constexpr (QJL) {
      q.r0[kk] = *(const half8*)(qb + (a.nq + c) * kD + 32 * g + 8 * kk);
      if constexpr (WIDE) q.r1[kk] = *(const half8*)(qb + (a.nq + 16 + c) * kD + 32 * g + 8 * kk);
    }
  }
  const int hc = WIDE ? c : (c & 7);
  q.cs1 = a.qcs[(bkv * 2 + 0) * 16 + hc];
  q.cs2 = QJL ? a.qcs[(bkv * 2 + 1) * 16 + hc] : 0.f;
  q.hf = hf;
  q.q0l = (const half8*)(qlds) + (c * kD + 32 * g) / 8;

  SoftState<WIDE> st;
  st.m_ref = -INFINITY;
  st.m_off = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    st.acc0[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    st.acc1[nb] = st.acc0[nb];
  }

  // ---- stream the chunk: full 32-token steps with three register buffers in
  // turn (the code words of the next two steps are in flight while the current
  // step computes), then at most one masked step for a ragged end.
  const int t_full = t_begin + (t_end > t_begin ? (t_end - t_begin) / kStep * kStep : 0);
  int t0 = t_begin;
  if (t0 < t_full) {
    StepData<KB, VB, QJL, WIDE> A, Bd, Cd;
    load_step(A, s, lo, t0);
    if (t0 + kStep < t_full) load_step(Bd, s, lo, t0 + kStep);
#define TQ_STEP(CUR, NEXT2)                                                                              \
    if (t0 + 2 * kStep < t_full) load_step(NEXT2, s, lo, t0 + 2 * kStep);                               \
    scan_step<KB, VB, QJL, WIDE, false>(CUR, q, st, lutK, lutV, lutS, lrep, t0 + 8 * g, t_end, s, lo, t0); \
    t0 += kStep;                                                                                         \
    if (t0 >= t_full) break;
    while (true) {
      TQ_STEP(A, Cd)
      TQ_STEP(Bd, A)
      TQ_STEP(Cd, Bd)
    }
#undef TQ_STEP
  }
  if (t0 < t_end) {
    StepData<KB, VB, QJL, WIDE> A;
    load_step(A, s, lo, t0);
    scan_step<KB, VB, QJL, WIDE, true>(A, q, st, lutK, lutV, lutS, lrep, t0 + 8 * g, t_end, s, lo, t0);
  }

  // ---- this wavefront's partial: lane (g, c) holds coordinates 32g + 8r + nb of column c
  float o[8][4];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = st.acc0[nb][r];
      x += WIDE ? st.acc1[nb][r] : dpp_ror8(x);
      o[nb][r] = x;
    }
  }
  float l = st.l;
  if constexpr (!WIDE) l += dpp_ror8(l);   // the hi and lo lanes each summed half of the tokens
  l += shfl_xor_f(l, 16);
  l += shfl_xor_f(l, 32);

  // ---- merge the 4 wavefront partials of this workgroup in LDS (fixed order)
  __syncthreads();   // every wavefront is done with the lookup tables
  float* mrg = (float*)smem;   // [wave][MC columns][128 + 2]
  if (c < a.G) {
    float* dst = mrg + (wave * MC + c) * (kD + 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) dst[32 * g + 8 * r + nb] = o[nb][r];
    }
    if (g == 0) {
      dst[kD] = st.m_off;
      dst[kD + 1] = l;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < a.G * kD; idx += 256) {
    const int h = idx / kD, j = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWavesPerDecodeWG; ++wv) M = fmaxf(M, mrg[(wv * MC + h) * (kD + 2) + kD]);
    float num = 0.f, den = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < kWavesPerDecodeWG; ++wv) {
        const float* src = mrg + (wv * MC + h) * (kD + 2);
        const float mw = src[kD];
        const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        num = fmaf(f, src[j], num);
        den = fmaf(f, src[kD + 1], den);
      }
    }
    const int64_t pidx = ((int64_t)b * a.H_q + kv * a.G + h) * a.n_split + split;
    a.acc[pidx * kD + j] = num;
    if (j == 0) {
      a.ml[pidx * 2] = M;
      a.ml[pidx * 2 + 1] = den;
    }
  }

}

// ---------------------------------------------------------------- combine --

// Workgroup (kv, b, chunk): merge the context-chunk partials of the G query
// heads of KV head kv in chunk order (every workgroup of the KV head merges all
// 128 coordinates; all loads are issued before use), then output coordinates
// 32*chunk .. 32*chunk+31 of o = Pi_V^T o', with those 32 columns of Pi_V
// staged in LDS.
__global__ __launch_bounds__(256) void combine_kernel(const float* ml, const float* acc, const float* rotV,
                                                       float* out, int H_q, int G, int n_split, float inv_sqrt_d) {
  __shared__ __align__(16) float colv[kD * 32];
  __shared__ __align__(16) float ov[16 * kD];
  const int kv = blockIdx.x, b = blockIdx.y, chunk = blockIdx.z, tid = threadIdx.x;
  {
    // Pi_V[j][32*chunk + 0..31] for all j: 1024 16-byte pieces, 4 per thread
    float4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int f = tid + 256 * k, j = f >> 3, c4 = f & 7;
      v[k] = *(const float4*)(rotV + j * kD + 32 * chunk + 4 * c4);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int f = tid + 256 * k;
      *(float4*)(colv + 4 * f) = v[k];
    }
  }
  for (int idx = tid; idx < G * kD; idx += 256) {
    const int h = idx / kD, j = idx % kD;
    const int64_t bh = (int64_t)b * H_q + kv * G + h;
    const float* mlb = ml + bh * n_split * 2;
    const float* ab = acc + bh * n_split * kD + j;
    // one pass in chunk order, rescaling the running sums when the maximum grows
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int sp = 0; sp < n_split; ++sp) {
      const float m = mlb[2 * sp], l = mlb[2 * sp + 1], x = ab[(int64_t)sp * kD];
      if (m == -INFINITY) continue;
      if (m > M) {
        const float f = __builtin_amdgcn_exp2f(M - m);
        num *= f;
        den *= f;
        M = m;
      }
      const float w = __builtin_amdgcn_exp2f(m - M);
      num = fmaf(w, x, num);
      den = fmaf(w, l, den);
    }
    ov[idx] = den > 0.f ? num / den * inv_sqrt_d : 0.f;
  }
  __syncthreads();
  // thread (i, hq): out[h][32*chunk + i] for heads hq, hq + 8
  const int i = tid & 31, hq = tid >> 5;
  for (int h = hq; h < G; h += 8) {
    float r = 0.f;
#pragma unroll 8
    for (int j = 0; j < kD; ++j) r = fmaf(colv[j * 32 + i], ov[h * kD + j], r);
    out[((int64_t)b * H_q + kv * G + h) * kD + 32 * chunk + i] = r;
  }
}

template <int KB, int VB, int QJL, int WIDE>
hipError_t launch_scan(const DecodePlan& p, const ScanArgs& sa, hipStream_t stream) {
  dim3 grid((unsigned)p.n_split, (unsigned)p.H_kv, (unsigned)p.B);
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
  if (p.qjl)
    hipLaunchKernelGGL(rotate_query_kernel, dim3((unsigned)p.H_kv, (unsigned)p.B), dim3(256), 0, stream, ra);
  else
    hipLaunchKernelGGL(rotate_query_chunk_kernel, dim3((unsigned)p.H_kv, (unsigned)p.B, kRotChunks), dim3(256), 0,
                       stream, ra);
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
  sa.wg_chunk = p.chunk;
  sa.wave_chunk = p.chunk / kWavesPerDecodeWG;
  sa.nq = p.nq;
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

  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)p.H_kv, (unsigned)p.B, kD / 32), dim3(256), 0, stream, ml, acc,
                     v->rot, out, (int)p.H_q, p.G, p.n_split, inv_sqrt_d);
  return hipGetLastError();
}

}  // namespace tq
