// Decode attention over the packed TurboQuant cache, for gfx950.
//
// decode_scan: one workgroup per (context chunk, KV head, row) that fills a
// compute unit (16 wavefronts; 8 for the QJL and G > 8 tiles):
//   prologue  codebook lookup tables in LDS; q' = Pi_K q for the G query heads
//             of the KV head (and q'' = S q' for QJL keys), with the rows of
//             the matrix read straight from memory in segments, scaled by a
//             power of two per head and split into float16 hi + lo halves
//             (~22 bits together); the first code words of the scan are
//             already in flight;
//   scan      each wavefront streams its share of the chunk: scores from the
//             packed key codes on MFMA, online softmax in registers, values
//             accumulated in the rotated domain on MFMA;
//   epilogue  the wavefront partials are merged in LDS in a fixed order and
//             the workgroup applies Pi_V^T: with a single chunk (the usual
//             case once B * H_kv fills the part) to o' / l, writing the output
//             itself; otherwise to the chunk's unnormalised sums, its partial.
// Paged caches: a step's token rows come from the block table (an entry read
// one step ahead); a 32-token step never crosses a block. A separate
// instantiation keeps the contiguous path free of that work.
// merge (only when the context is split into several chunks): fixed-order
// merge of the chunk partials of each query head, already in the output basis
// (the rotation is linear, so it commutes with the merge).
// (Merging chunks inside decode_scan would need a device-scope release per
// workgroup, which on this multi-die part writes back L2; the kernel boundary
// provides that ordering once.)
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
//        weight operand in float16, which is what the QK lanes hold (G <= 8:
//        the lanes of columns c and c+8 each own 4 of a block's 8 tokens and
//        zero the other 4, so the two columns are partial sums that the
//        epilogue adds); A is unpacked from the 8-token value blocks, lane
//        (g, i) reading the 24-byte (3-bit) slice of block g that holds
//        coordinates 8i .. 8i+7.
//   Precision: the query operand keeps ~22 bits (hi + lo halves), since a
//        score's error scales with the score itself and key norms reach the
//        hundreds; a weight is rounded once to float16 (relative error at most
//        2^-11, independent of the scores), which moves the output by about
//        2^-11 / sqrt(3) relative for diffuse attention and at most 2^-11 when
//        one token dominates.
//   Codes become float16 pairs through a lookup table in LDS indexed by two
//   adjacent codes (2*bits wide field), replicated kLutRep times so that lanes
//   of a wavefront read distinct banks (lane l reads replica l % kLutRep).
//
// Online softmax (log2 domain; the query operand carries log2(e) * scale / sqrt(d)):
// the reference maximum m only moves when a score exceeds it by more than
// kSlack, so the rescale of the accumulators is rare; weights are
// 2^(s - m - kShift - ev) * |v| with kShift = kSlack + log2(sqrt(d)) and 2^ev
// a per-wavefront power of two at or above the value norms of its first step,
// which keeps every weight operand at or below (|v| / 2^ev) / sqrt(d) (float16
// range while |v| < 7e5 * 2^ev, and no float16 underflow of the leading
// weights however small the norms) and leaves one 1/sqrt(d) for the end.
#include <math.h>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_append.h"
#include "tq_rotate.h"
#include "tq_scan.h"

namespace tq {

namespace {

// (shared scan pieces: tq_scan.h)

// ------------------------------------------------------ small matrix work --

constexpr int kVecWords = 16 * kD;         // [16][d] float vectors
template <int D>
constexpr int vec_words() { return 16 * D; }
// Column stride (in halves) of the float16 query operand in LDS: the 16 lanes
// that read one 16-byte piece of 16 different columns then hit distinct banks.
constexpr int kQStride = kD + 8;
template <int D>
constexpr int qstride() { return D + 8; }
// Scratch region of a decode workgroup, in 32-bit words: the lookup tables
// (scan), then the wavefront partials (merge) and the partial sums of the final
// rotation, followed by two [16][d] float vector sets.
constexpr int kRegionWords = 16896;
// A one-token append taken by the prologue: the scaled key and value, their
// rotations, their codes, sqrt(d)/|x| and |x| of each, the two codebooks'
// thresholds (in LDS: a search over registers would index a stack copy).
constexpr int kAppWords = 4 * kD + 2 * kD / 4 + 4 + 2 * 16;
// Row stride (in floats) of a wavefront partial in the merge area: 128
// coordinates, m and l, padded to a 16-byte multiple.
constexpr int kMergeStride = kD + 4;
template <int D>
constexpr int merge_stride() { return D + 4; }
template <int D>
constexpr int scratch_words() { return kRegionWords + 2 * vec_words<D>() + kAppWords; }

// Codes of a vector rotated by rotate_rows<NT, 1> (y in LDS), by the lanes
// that wrote its rows: cell of y_i * sqrt(d)/|x| (the append kernels' encode).
template <int NT, int BITS>
__device__ inline void app_encode(const float* y, float fz, const Thresholds<BITS>& th, unsigned char* cb) {
  constexpr int R = RowSegment<NT>::R;
  const int i0 = R * (threadIdx.x / 16), sg = threadIdx.x % 16;
  if (sg == 0) {
#pragma unroll
    for (int k = 0; k < R; ++k) cb[i0 + k] = (unsigned char)encode<BITS>(y[i0 + k] * fz, th);
  }
}

// Float16 operand of vals[G][d] * sc: a power of two per head puts its largest
// entry in [2^13, 2^14) (cs[h] = that power, 1 for absent heads); column h of
// dst holds the hi halves, column half_cols + h the lo halves, ~22 bits
// together (zero columns for absent heads). Needs NT >= 256; ends with the
// operand written by each thread, no barrier.
template <int NT, int D = kD>
__device__ void emit_operand(const float* vals, float sc, int G, int half_cols, _Float16* dst, float* cs,
                             int* hexp) {
  constexpr int QS = qstride<D>();
  const int tid = threadIdx.x;
  if (tid < 256) {
    // thread (h, seg): largest magnitude over D/16 entries, then over the 16 segments
    const int h = tid >> 4, seg = tid & 15;
    float mx = 0.f;
    if (h < G) {
#pragma unroll
      for (int k = 0; k < D / 16; ++k) mx = fmaxf(mx, fabsf(vals[h * D + (D / 16) * seg + k] * sc));
    }
    // maximum over the 16 lanes of the row: quads, then rotates by 4 and 8
    mx = fmaxf(mx, dpp_xor1(mx));
    mx = fmaxf(mx, dpp_xor2(mx));
    mx = fmaxf(mx, dpp_ror4(mx));
    mx = fmaxf(mx, dpp_ror8(mx));
    if (seg == 0) {
      const int e = (mx > 0.f) ? (__builtin_amdgcn_frexp_expf(mx) - 14) : 0;
      hexp[h] = e;
      cs[h] = ldexpf(1.0f, e);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < 2 * half_cols * D; idx += NT) {
    const int col = idx / D, i = idx % D;
    const int h = col % half_cols;
    float v = 0.f;
    if (h < G) v = ldexpf(vals[h * D + i] * sc, -hexp[h]);
    const _Float16 hi = (_Float16)v;
    dst[col * QS + i] = col >= half_cols ? (_Float16)(v - (float)hi) : hi;
  }
}

// out[h][i] = sum_j M[i][j] in[h][j] for the G vectors in[G][D] (LDS), D != 128
// (128 takes rotate_rows): thread (i, part) sums the part's NT/D-th of row i
// (float4 reads of M, every element read once per workgroup), the parts meet
// in `part_buf` ([NT/D][16][D] floats) in a fixed order. Ends with out
// written, after a barrier.
template <int NT, int D, int MAXG>
__device__ void rotate_generic(const float* M, const float* in, float* out, float* part_buf, int G) {
  constexpr int P = NT / D, SPAN = D / P;
  const int tid = threadIdx.x, i = tid % D, pt = tid / D;
  float acc[MAXG];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) acc[h] = 0.f;
  const float4* row = (const float4*)(M + (int64_t)i * D + pt * SPAN);
#pragma unroll 4
  for (int k = 0; k < SPAN / 4; ++k) {
    const float4 m = row[k];
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
      if (h < G) {
        const float4 x = *(const float4*)(in + h * D + pt * SPAN + 4 * k);   // (same address across the row's lanes)
        acc[h] = fmaf(m.w, x.w, fmaf(m.z, x.z, fmaf(m.y, x.y, fmaf(m.x, x.x, acc[h]))));
      }
    }
  }
#pragma unroll
  for (int h = 0; h < MAXG; ++h)
    if (h < G) part_buf[(pt * 16 + h) * D + i] = acc[h];
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D, ii = idx % D;
    float r = 0.f;
#pragma unroll
    for (int q = 0; q < P; ++q) r += part_buf[(q * 16 + h) * D + ii];
    out[h * D + ii] = r;
  }
  __syncthreads();
}

// ------------------------------------------------------------------- scan --

struct ScanArgs {
  const uint32_t* kcodes;
  const float* knorms;
  const uint32_t* ksigns;
  const float* kgamma;
  const uint32_t* vcodes;
  const float* vnorms;
  const void* q;
  const float* rotK;   // Pi_K
  const float* proj;   // S (QJL keys), or null
  const float* rotV;   // Pi_V
  const int32_t* ctx_lens;
  float* out;    // [B][H_q][d], written when n_split == 1
  float* ml;     // [B][H_q][n_split][2], partials when n_split > 1
  float* acc;    // [B][H_q][n_split][d]
  int64_t TcK, TcV;
  PageMap kpm, vpm;   // block tables of paged caches (table == nullptr: contiguous)
  int q_dtype, H_kv, H_q, G, T, n_split, wg_chunk, wave_chunk;
  int M, Mt, nqt;   // query tokens per row, per workgroup tile, tiles per row
  float sc1, sc2, inv_sqrt_d;
  float kc[16], vc[16];
  // One-token append taken by the prologue (app != 0: d = 128 keys without a
  // QJL sketch, a decode): the new key and value of each (row, KV head), x
  // [B][H_kv][d] in qk.x and qv.x, go to token clamp(ctx_len, 0, T) - 1 (T - 1
  // without context lengths) before the scan reads that token.
  int app, app_xf32;
  QuantArgs qk, qv;
};

template <int WIDE, int QJL, int D = 128>
struct QOps {
  // column c (and c + 16), coordinates (D/4)g + 8kk + 0..7
  half8 q0[Geom<D>::NKK], q1[Geom<D>::NKK], r0[Geom<D>::NKK], r1[Geom<D>::NKK];
  float cs1, cs2;
  bool hf;   // G <= 8: lane holds the lo half of its query column (column >= 8)
};

template <int WIDE, int D = 128>
struct SoftState {
  float m_ref, m_off, l;
  float ev;   // wave-uniform: log2 of the power of two that scales the value norms
  floatx4 acc0[Geom<D>::CV];
};

template <int KB, int VB, int QJL, int WIDE, bool MASK, int D>
__device__ __forceinline__ void scan_step(const StepData<KB, VB, QJL, WIDE, D>& d0, const QOps<WIDE, QJL, D>& q,
                                          SoftState<WIDE, D>& st, const char* lut, LutRegs& lr,
                                          const uint32_t* lutS, int lane, int tg, int lim) {
  constexpr int NKK = Geom<D>::NKK, CV = Geom<D>::CV;
  // a key slice that starts inside a word (d = 64, 3 bits: lane groups 1 and 3
  // at bit 16) is first aligned in registers
  StepData<KB, VB, QJL, WIDE, D> dsh;
  if constexpr (key_slice_shifted<KB, D>()) {
    dsh = d0;
    const uint32_t sh = (uint32_t)((lane >> 4) * (D / 4 * KB)) & 31u;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      dsh.kw[m][0] = __builtin_amdgcn_alignbit(dsh.kw[m][1], dsh.kw[m][0], sh);
      dsh.kw[m][1] = dsh.kw[m][1] >> sh;
    }
  }
  const StepData<KB, VB, QJL, WIDE, D>& d = key_slice_shifted<KB, D>() ? dsh : d0;
  const StepNorms<QJL>& nm = d.nm;
  // ---- scores on MFMA: coordinate block KK outer, the two row blocks inner
  // (two independent accumulation chains; one query block live at a time)
  floatx4 s0[2], s1[2], z0[2], z1[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    s0[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    s1[m] = s0[m];
    z0[m] = s0[m];
    z1[m] = s0[m];
  }
  static_for<0, NKK>([&](auto kk) {
    constexpr int KK = decltype(kk)::value;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const half8 ka = key_operand<KB, KK, D>(d.kw[m], lut, m ? lr.b : lr.a);
      s0[m] = mfma16(ka, q.q0[KK], s0[m]);
      if constexpr (WIDE) s1[m] = mfma16(ka, q.q1[KK], s1[m]);
    }
  });
  if constexpr (QJL) {
#define TQ_QJ(KK)                                                     \
    _Pragma("unroll") for (int m = 0; m < 2; ++m) {                   \
      const half8 sa = sign_operand<KK>(d.sw[m], lutS, lane);         \
      z0[m] = mfma16(sa, q.r0[KK], z0[m]);                            \
      if constexpr (WIDE) z1[m] = mfma16(sa, q.r1[KK], z1[m]);        \
    }
    TQ_QJ(0) TQ_QJ(1) TQ_QJ(2) TQ_QJ(3)
#undef TQ_QJ
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
        x = fmaf(z * q.cs2, quad_bcast(nm.kg, r), x * q.cs1);
      }
      float v = x * quad_bcast(nm.kn, r);
      if constexpr (MASK) v = (tg + 4 * (int)q.hf + r < lim) ? v : -INFINITY;
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
      // (a column with nothing accumulated yet, m_ref = -inf, may still see no
      // visible token while another column moves: its factor is 0, not NaN)
      const float alpha = st.m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m_ref - m_new);
      st.l *= alpha;
#pragma unroll
      for (int nb = 0; nb < CV; ++nb) st.acc0[nb] *= alpha;
      st.m_ref = m_new;
      st.m_off = m_new + kShift + st.ev;
    }
    float w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float p = __builtin_amdgcn_exp2f(fmaf(y[r], cs, -st.m_off));
      // (a column that has seen no visible token yet has m_off = -inf: p of a
      // masked token is then NaN, so the mask selects 0 rather than scaling)
      if constexpr (MASK) p = (tg + 4 * (int)q.hf + r < lim) ? p : 0.f;
      st.l += p;
      w[r] = p * quad_bcast(nm.vn, r);
    }
    // float16 weights of the lane's 4 tokens, two per register. The B operand
    // of lane (c, hf) holds them in k slots 4hf .. 4hf+3 of its 8-token block
    // and zeros in the other four: MFMA column c sums tokens 0-3 and column c+8
    // tokens 4-7 of every block, and the epilogue adds the two columns.
    uint32_t h2[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      // w stays a float32 value in a register (empty asm), so the conversion is a
      // plain packed convert rather than fused mixed-precision FMAs
      float a0 = w[2 * k], a1 = w[2 * k + 1];
      asm volatile("" : "+v"(a0), "+v"(a1));
      h2[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){a0, a1}, half2v));
    }
    uint32_t op[4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      op[k] = q.hf ? 0u : h2[k];
      op[2 + k] = q.hf ? h2[k] : 0u;
    }
    const half8 pb0 = words_to_half8(op[0], op[1], op[2], op[3]);
    static_for<0, CV>([&](auto nb) {
      constexpr int NB = decltype(nb)::value;
      const half8 va = value_operand<VB, NB, D>(d.vw, lut, (NB & 1) ? lr.b : lr.a);
      st.acc0[NB] = mfma16(va, pb0, st.acc0[NB]);
    });
  } else {
    // ---- 8 < G <= 16: separate hi and lo query tiles; every lane holds 8 tokens
    float y[8];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * m + r;
        float x = s0[m][r] + s1[m][r];
        if constexpr (QJL) {
          const float yq = z0[m][r] + z1[m][r];
          x = fmaf(yq * q.cs2, bcast_row(nm.kg, e), x * q.cs1);
        }
        float v = x * bcast_row(nm.kn, e);
        if constexpr (MASK) v = (tg + e < lim) ? v : -INFINITY;
        y[e] = v;
      }
    }
    const float lmax = fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])), fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
    if (__any(lmax * cs > st.m_ref + kSlack)) {
      float tmax = fmaxf(lmax, shfl_xor_f(lmax, 16));
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      const float m_new = fmaxf(st.m_ref, tmax * cs);
      // (a column with nothing accumulated yet, m_ref = -inf, may still see no
      // visible token while another column moves: its factor is 0, not NaN)
      const float alpha = st.m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m_ref - m_new);
      st.l *= alpha;
#pragma unroll
      for (int nb = 0; nb < CV; ++nb) st.acc0[nb] *= alpha;
      st.m_ref = m_new;
      st.m_off = m_new + kShift + st.ev;
    }
    uint32_t pw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float w2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * k + u;
        float p = __builtin_amdgcn_exp2f(fmaf(y[e], cs, -st.m_off));
        if constexpr (MASK) p = (tg + e < lim) ? p : 0.f;   // (NaN when no visible token yet)
        st.l += p;
        w2[u] = p * bcast_row(nm.vn, e);
      }
      pw[k] = __builtin_bit_cast(uint32_t, half2v{(_Float16)w2[0], (_Float16)w2[1]});
    }
    const half8 pb = words_to_half8(pw[0], pw[1], pw[2], pw[3]);
    static_for<0, CV>([&](auto nb) {
      constexpr int NB = decltype(nb)::value;
      const half8 va = value_operand<VB, NB, D>(d.vw, lut, (NB & 1) ? lr.b : lr.a);
      st.acc0[NB] = mfma16(va, pb, st.acc0[NB]);
    });
  }
}


// Wavefronts per workgroup: one workgroup fills a compute unit (4 wavefronts
// per SIMD, <= 128 VGPRs, for the common tiles; the QJL and G > 8 tiles carry
// more operands and run 2 per SIMD;
// d = 256 doubles the value accumulators and the key words and takes the
// 8-wavefront tile as well.)
constexpr int kCommonWaves = 16;
template <int QJL, int WIDE, int D = 128>
constexpr int scan_waves() { return (QJL || WIDE || D > 128) ? 8 : kCommonWaves; }
// Steps whose loads are in flight while a wavefront computes one (register
// buffers: ahead + 1).
constexpr int kCommonAhead = 1;
template <int QJL, int WIDE, int D = 128>
constexpr int scan_ahead() { return (QJL || WIDE || D > 128) ? 1 : kCommonAhead; }

// merge buffer: [wave][column][kMergeStride] floats, 8 columns (G <= 8) or 16
template <int WIDE>
constexpr int merge_cols() { return WIDE ? 16 : 8; }

// LDS of a decode workgroup, in 32-bit words: the float16 query operand
// ([1 + QJL][operand columns][d]), 32 column scales, 16 exponents, 32 codebook
// levels, the step counter (padded to 4 words), then the scratch region.
template <int QJL, int WIDE, int D = 128>
constexpr int scan_head_words() { return (1 + QJL) * (WIDE ? 32 : 16) * qstride<D>() / 2 + 84; }

template <int KB, int VB, int QJL, int WIDE, int D = 128>
constexpr size_t scan_lds_bytes() {
  constexpr int NW = scan_waves<QJL, WIDE, D>();
  static_assert(kLutBytes / 4 + (QJL ? 4 : 0) * kLutRep <= kRegionWords, "lookup tables exceed the scratch region");
  static_assert(NW * merge_cols<WIDE>() * merge_stride<D>() <= kRegionWords, "merge area exceeds the scratch region");
  static_assert(D != kD || NW * (WIDE ? 16 : 8) * D <= kRegionWords, "rotation partials exceed the scratch region");
  static_assert(D == kD || 64 * NW * 16 <= kRegionWords, "rotation parts exceed the scratch region");
  return (size_t)(scan_head_words<QJL, WIDE, D>() + scratch_words<D>()) * 4;
}

// One workgroup per (context chunk, KV head, row):
//   prologue  q' = Pi_K q for the G query heads (and q'' = S q' for QJL keys)
//             into the float16 operand in LDS, while the first code words are
//             already in flight;
//   scan      each wavefront streams its share of the chunk;
//   epilogue  the wavefront partials are merged in LDS in a fixed order, then
//             Pi_V^T: with one chunk the output, otherwise the chunk partial
//             for the merge kernel.
template <int KB, int VB, int QJL, int WIDE, int PAGED, int D>
__global__ __launch_bounds__((64 * scan_waves<QJL, WIDE, D>())) void decode_scan_kernel(ScanArgs a) {
  constexpr int NW = scan_waves<QJL, WIDE, D>(), NT = 64 * NW;
  constexpr int NS = QJL ? 4 : 0;
  constexpr int KW = key_record_words<KB, D>();   // words of a key record
  constexpr int VWT = D * VB / 32;                // value words per token row
  constexpr int NKK = Geom<D>::NKK, CV = Geom<D>::CV;
  constexpr int QS = qstride<D>(), MS = merge_stride<D>();
  constexpr int MC = merge_cols<WIDE>();
  constexpr int NQ = WIDE ? 32 : 16;   // operand columns per part
  constexpr int HALF = NQ / 2;
  __shared__ __align__(16) uint32_t smem[scan_lds_bytes<KB, VB, QJL, WIDE, D>() / 4];
  _Float16* qlds = (_Float16*)smem;                              // [1 + QJL][NQ][QS]
  float* qcs = (float*)(smem + (1 + QJL) * NQ * QS / 2);   // [2][16]
  int* hexp = (int*)(qcs + 32);                            // [16]
  float* cents = qcs + 48;                                 // [2][16] key, value levels
  uint32_t* steps_done = (uint32_t*)(qcs + 80);            // steps begun by the workgroup
  uint32_t* U = smem + scan_head_words<QJL, WIDE, D>();    // scratch, 16-byte aligned
  float* R = (float*)U;   // region: lookup tables, then merge area / rotation partials
  float* vA = R + kRegionWords;
  float* vB = vA + vec_words<D>();
  float* axk = vB + vec_words<D>();       // appended key: scaled vector, then its rotation
  float* ayk = axk + kD;
  float* axv = ayk + kD;                  // appended value
  float* ayv = axv + kD;
  unsigned char* acb = (unsigned char*)(ayv + kD);   // [2][d] codes
  float* afz = ayv + kD + 2 * kD / 4;     // sqrt(d)/|x|, |x| of the key, then of the value
  Thresholds<KB>* athk = (Thresholds<KB>*)(afz + 4);
  Thresholds<VB>* athv = (Thresholds<VB>*)(afz + 4 + 16);
  uint32_t* lut = U;                      // keys and values
  uint32_t* lutS = U + kLutBytes / 4;     // QJL signs

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const int lrep = lane & (kLutRep - 1);
  const int split = blockIdx.x, kv = blockIdx.y;
  const int b = blockIdx.z / a.nqt;                     // batch row
  const int i0 = (blockIdx.z - b * a.nqt) * a.Mt;       // first query token of the tile
  const int G = a.G;
  const int mq = min(a.Mt, a.M - i0);                   // query tokens of the tile
  // operand columns: (token i, head g) -> column i * G + g (the G heads of one
  // token for a decode)
  const int NC = mq * G;
  const int64_t bkv = (int64_t)b * a.H_kv + kv;

  // token range of this wavefront (before the context length clips it);
  // wave-uniform, so that every step offset travels in the scalar offset of
  // the buffer loads
  const int t_begin = split * a.wg_chunk + wave * a.wave_chunk;

  // Streams: contiguous caches start at this (row, KV head)'s first token row
  // and span its T_cap rows; paged caches span the whole arrays and a step's
  // rows come from the block table (step_row).
  // (PAGED: at least one of the two caches is paged; the contiguous-only
  // instantiation carries none of the table work)
  const bool kpg = PAGED && a.kpm.table != nullptr, vpg = PAGED && a.vpm.table != nullptr;
  const int64_t kbase = kpg ? 0 : bkv * a.TcK, vbase = vpg ? 0 : bkv * a.TcV;
  const int64_t krows = kpg ? (a.kpm.nblk * a.H_kv) << a.kpm.lg : a.TcK;
  const int64_t vrows = vpg ? (a.vpm.nblk * a.H_kv) << a.vpm.lg : a.TcV;
  Streams s;
  s.rk = make_rsrc(a.kcodes + kbase * KW, (uint32_t)(krows * KW * 4));
  s.rkn = make_rsrc(a.knorms + kbase, (uint32_t)(krows * 4));
  s.rv = make_rsrc(a.vcodes + vbase * VWT, (uint32_t)(vrows * VWT * 4));
  s.rvn = make_rsrc(a.vnorms + vbase, (uint32_t)(vrows * 4));
  // QJL sketch (empty ranges when the keys carry none)
  s.rs = make_rsrc(QJL ? (const void*)(a.ksigns + kbase * 4) : (const void*)a.knorms,
                   QJL ? (uint32_t)(krows * 16) : 0u);
  s.rg = make_rsrc(QJL ? (const void*)(a.kgamma + kbase) : (const void*)a.knorms,
                   QJL ? (uint32_t)(krows * 4) : 0u);
  // block-table rows of this batch row (range-checked reads: a block past the
  // table reads entry 0)
  const __amdgpu_buffer_rsrc_t rtk =
      make_rsrc(kpg ? (const void*)(a.kpm.table + b * a.kpm.maxblk) : (const void*)a.knorms,
                kpg ? (uint32_t)(a.kpm.maxblk * 4) : 0u);
  const __amdgpu_buffer_rsrc_t rtv =
      make_rsrc(vpg ? (const void*)(a.vpm.table + b * a.vpm.maxblk) : (const void*)a.knorms,
                vpg ? (uint32_t)(a.vpm.maxblk * 4) : 0u);
  const bool hf = !WIDE && c >= 8;
  LaneOffsets lo;
  {
    const int tk = 8 * (c >> 2) + (c & 3);   // MFMA row c of row block 0 (block 1: tk + 4)
    // lane group g's key slice starts at bit (D/4) * KB * g of the record
    lo.k = (uint32_t)(tk * KW + ((D / 4) * KB * g) / 32) * 4u;
    lo.s = (uint32_t)(tk * 4 + g) * 4u;
  }
  lo.v = (uint32_t)(g * value_block_words<VB, D>() + c * value_slice_words<VB, D>()) * 4u;
  lo.n = (uint32_t)(WIDE ? 8 * g + (c & 7) : 8 * g + (hf ? 4 : 0) + (c & 3)) * 4u;

  // ---- prologue loads, in issue order: the context length, this thread's
  // segment of the rows of Pi_K, its query elements, the appended vectors,
  // the code words of the first steps. Loads complete in issue order, so
  // waiting for the matrix and the query never waits for the code words. The
  // first steps are read before the context length is used: reads past the
  // end of the cache return zeros (buffer range check), and steps past the
  // context are never used.
  // (d = 128; the other head dimensions read the matrix rows in the rotation)
  // (the context length: unconditional, through an empty range when there are
  // none, and first: a load under a branch would make its first use wait for
  // every load issued before it)
  uint32_t ctx_word = __builtin_amdgcn_raw_buffer_load_b32(
      make_rsrc(a.ctx_lens ? (const void*)a.ctx_lens : (const void*)a.knorms, a.ctx_lens ? (uint32_t)((b + 1) * 4) : 0u),
      (uint32_t)b * 4u, 0, 0);
  RowSegment<NT> rseg;
  if constexpr (D == kD) load_row_segment<NT>(rseg, a.rotK);
  constexpr int QE = 16 * D / NT;   // query elements per thread (G <= 16)
  uint32_t qraw[QE];
  {
    // one 32-bit load per element for either dtype (a bfloat16 element is
    // taken from the word that holds it), so the loads carry no branch
    // column c's vector: token i0 + c / G, head kv * G + c % G of row b
    const bool qbf = a.q_dtype == TQ_BF16;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc((const char*)a.q + ((((int64_t)b * a.M + i0) * a.H_q + (int64_t)kv * G) * D) * (qbf ? 2 : 4),
                  (uint32_t)((((int64_t)mq - 1) * a.H_q + G) * D * (qbf ? 2 : 4)));
#pragma unroll
    for (int k = 0; k < QE; ++k) {
      const uint32_t idx = tid + k * NT;
      const uint32_t cq = idx / D;
      const uint32_t el = ((cq / (uint32_t)G) * (uint32_t)a.H_q + cq % (uint32_t)G) * D + idx % D;
      qraw[k] = __builtin_amdgcn_raw_buffer_load_b32(rq, qbf ? (el * 2u) & ~3u : el * 4u, 0, 0);
    }
  }
  // appended key (wavefront 0) and value (wavefront 1): lanes 0-31 read 4
  // coordinates each
  constexpr bool APP = D == kD && !QJL;
  float ax[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (APP) {
    if (a.app && wave < 2 && lane < 32) {
      const bool vw = wave == 1;
      const int64_t off = (int64_t)b * (vw ? a.qv.sb : a.qk.sb) + (int64_t)kv * (vw ? a.qv.sh : a.qk.sh) + 4 * lane;
      const void* xp = vw ? a.qv.x : a.qk.x;
      if (a.app_xf32) {
        const float4 f = *(const float4*)((const float*)xp + off);
        ax[0] = f.x; ax[1] = f.y; ax[2] = f.z; ax[3] = f.w;
      } else {
        const uint2 u = *(const uint2*)((const uint16_t*)xp + off);
        ax[0] = __uint_as_float(u.x << 16); ax[1] = __uint_as_float(u.x & 0xFFFF0000u);
        ax[2] = __uint_as_float(u.y << 16); ax[3] = __uint_as_float(u.y & 0xFFFF0000u);
      }
    }
  }
  constexpr int AH = scan_ahead<QJL, WIDE, D>();
  StepData<KB, VB, QJL, WIDE, D> buf[AH + 1];
  // the first AH steps of the share (a step past the caches is replaced by the
  // first step of the row: such a wavefront, or such a step, is never used,
  // and the scalar offset of a buffer load is not range checked, only the
  // per-lane offset is)
  uint32_t ek = 0u, ev = 0u;   // block-table entries of the next step to load (paged caches)
#pragma unroll
  for (int j = 0; j < AH; ++j) {
    const int tj = t_begin + (j + 1) * kStep <= min(a.TcK, a.TcV) ? t_begin + j * kStep : 0;
    if (kpg) ek = page_entry(rtk, a.kpm, tj);
    if (vpg) ev = page_entry(rtv, a.vpm, tj);
    load_step<false>(buf[j], s, lo, step_row(a.kpm, kv, a.H_kv, ek, tj), step_row(a.vpm, kv, a.H_kv, ev, tj));
  }
  {
    const int tn = t_begin + AH * kStep;
    if (kpg) ek = page_entry(rtk, a.kpm, tn);
    if (vpg) ev = page_entry(rtv, a.vpm, tn);
  }
  __builtin_amdgcn_sched_barrier(0);

  // The appended token (if any) and whether this workgroup's chunk holds it
  // (the token of a row goes where a separate append would put it).
  // The wavefront whose share holds the token stores it (and alone reads it
  // back, in its last step), so no other wavefront waits for the stores.
  int app_t = -1, app_wave = -1;
  bool appending = false;
  AppendOne<VB, TQ_VALUES> apv;   // the value block's other words (wavefront app_wave)
  if constexpr (APP) {
    if (a.app) {
      int cx = a.ctx_lens ? (int)ctx_word : a.T;
      cx = cx < 0 ? 0 : (cx > a.T ? a.T : cx);
      app_t = __builtin_amdgcn_readfirstlane(cx - 1);
      appending = app_t >= 0 && app_t >= split * a.wg_chunk && app_t < (split + 1) * a.wg_chunk;
      if (appending) app_wave = (app_t - split * a.wg_chunk) / a.wave_chunk;
    }
  }

  // ---- prologue: lookup tables, then the query operand of this (row, KV head)
  if (tid < 32) {
    // codebook levels from the kernel arguments (constant indices: scalar reads)
    float cv = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      cv = tid == i ? a.kc[i] : cv;
      cv = tid == 16 + i ? a.vc[i] : cv;
    }
    cents[tid] = cv;
  }
  if (tid == 0) *steps_done = 0u;
  __syncthreads();
  auto build_tables = [&]() {
    build_lut<KB, VB>(lut, cents, cents + 16, tid, NT);
    if constexpr (QJL) {
      for (int e = tid; e < NS * kLutRep; e += NT) {
        const int f = e >> kLutShift;
        lutS[e] = pack_half2((f & 1) ? 1.f : -1.f, (f & 2) ? 1.f : -1.f);
      }
    }
  };
  // (d = 128 builds the tables first; the other head dimensions use the
  // region for the rotation's parts first)
  if constexpr (D == kD) build_tables();
  {
    // the NC column vectors as float32 in vA ([NC][d])
#pragma unroll
    for (int k = 0; k < QE; ++k) {
      const int idx = tid + k * NT;
      if (idx < NC * D)
        vA[idx] = a.q_dtype == TQ_BF16 ? __uint_as_float(((qraw[k] >> (16 * (idx & 1))) & 0xFFFFu) << 16)
                                       : __uint_as_float(qraw[k]);
    }
    if constexpr (APP) {
      // the codebooks' thresholds, the appended vectors' scale and norm
      // (wavefronts 0 and 1), the value block's other words
      if (appending) {
        if (tid < 15) {
          if (tid < (1 << KB) - 1) athk->t[tid] = a.qk.thr[tid];
          if (tid < (1 << VB) - 1) athv->t[tid] = a.qv.thr[tid];
        }
        if (tid == 15) {
          athk->sym = a.qk.thr_sym != 0;
          athv->sym = a.qv.thr_sym != 0;
        }
        if (wave == 0) AppendOne<KB, TQ_KEYS>().begin(a.qk, bkv, app_t, lane, ax, axk, afz);
        else if (wave == 1) AppendOne<VB, TQ_VALUES>().begin(a.qv, bkv, app_t, lane, ax, axv, afz + 2);
        if (wave == app_wave) apv.load_old(a.qv, bkv, app_t, lane);
      }
    }
    __syncthreads();
    if constexpr (D == kD) {
      rotate_rows<NT, NQ / 2>(rseg, vA, vB, NC);   // q' = Pi_K q
      if constexpr (APP) {
        if (appending) {
          // the appended key on the same row segments of Pi_K (the arithmetic
          // of the append kernels), its codes by the lanes that hold the rows;
          // then Pi_V's segments, in flight while the query operand is written
          rotate_rows<NT, 1>(rseg, axk, ayk, 1);
          app_encode<NT, KB>(ayk, afz[0], *athk, acb);
          load_row_segment<NT>(rseg, a.rotV);
        }
      }
      __syncthreads();
    } else {
      rotate_generic<NT, D, NQ / 2>(a.rotK, vA, vB, R, NC);   // q' = Pi_K q
    }
    emit_operand<NT, D>(vB, a.sc1, NC, HALF, qlds, qcs, hexp);
    if constexpr (QJL) {
      static_assert(D == kD, "QJL keys take d = 128");
      load_row_segment<NT>(rseg, a.proj);
      rotate_rows<NT, NQ / 2>(rseg, vB, vA, NC);   // q'' = S q'
      __syncthreads();
      emit_operand<NT>(vA, a.sc2, NC, HALF, qlds + NQ * kQStride, qcs + 16, hexp);
    }
    if constexpr (APP) {
      if (appending) {
        // the appended value on Pi_V's row segments, its codes, then the
        // stores by the wavefront that reads the token back (after its own
        // stores have completed)
        rotate_rows<NT, 1>(rseg, axv, ayv, 1);
        app_encode<NT, VB>(ayv, afz[2], *athv, acb + kD);
        __syncthreads();
        if (wave == app_wave) {
          AppendOne<KB, TQ_KEYS>().finish(a.qk, bkv, app_t, lane, afz, acb);
          apv.finish(a.qv, bkv, app_t, lane, afz + 2, acb + kD);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
      }
    }
  }
  __syncthreads();
  if constexpr (D != kD) {
    build_tables();
    __syncthreads();
  }

  // query operand (B of QK) for this lane: column c, coordinates (D/4)g + 8kk + 0..7
  QOps<WIDE, QJL, D> q;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    q.q0[kk] = *(const half8*)(qlds + c * QS + (D / 4) * g + 8 * kk);
    if constexpr (WIDE) q.q1[kk] = *(const half8*)(qlds + (16 + c) * QS + (D / 4) * g + 8 * kk);
    if constexpr (QJL) {
      q.r0[kk] = *(const half8*)(qlds + (NQ + c) * QS + (D / 4) * g + 8 * kk);
      if constexpr (WIDE) q.r1[kk] = *(const half8*)(qlds + (NQ + 16 + c) * QS + (D / 4) * g + 8 * kk);
    }
  }
  const int hc = WIDE ? c : (c & 7);
  q.cs1 = qcs[hc];
  q.cs2 = QJL ? qcs[16 + hc] : 0.f;
  q.hf = hf;


  // the share of this wavefront, clipped by the context length
  asm volatile("" : "+v"(ctx_word));
  int ctx = a.ctx_lens ? (int)ctx_word : a.T;
  ctx = ctx < 0 ? 0 : (ctx > a.T ? a.T : ctx);
  // causal limits: token i0 + i of the tile (position ctx - M + i0 + i) sees
  // cache tokens below lim0 + i (all ctx tokens for a decode)
  const int lim0 = ctx - a.M + i0 + 1;
  const int lim_lo = max(lim0, 0), lim_hi = max(lim0 + mq - 1, 0);
  const int t_end = __builtin_amdgcn_readfirstlane(min(t_begin + a.wave_chunk, lim_hi));
  const int t_unm = min(t_end, lim_lo);   // below this every column sees every token
  int t_full =
      __builtin_amdgcn_readfirstlane(t_begin + (t_unm > t_begin ? (t_unm - t_begin) / kStep * kStep : 0));
  // the step holding a token appended by the prologue is read after it, in the
  // masked steps, past the vector L1 (the steps read ahead before the append
  // may hold the old words)
  if (appending && app_t >= t_begin && app_t < t_end)
    t_full = __builtin_amdgcn_readfirstlane(min(t_full, t_begin + (app_t - t_begin) / kStep * kStep));
  // this lane's column limit for the masked steps (columns past NC carry a zero
  // query and keep the widest limit)
  const int lcol = WIDE ? c : (c & 7);
  const int lim_lane = lcol < NC ? max(lim0 + lcol / G, 0) : lim_hi;

  LutRegs lr;
#pragma unroll
  for (int i = 0; i < 4; ++i) lr.a[i] = lr.b[i] = (uint32_t)lrep * 4u;
  SoftState<WIDE, D> st;
  st.m_ref = -INFINITY;
  st.m_off = -INFINITY;
  st.l = 0.f;
  // Value-norm scale: the weights 2^(s - m_off) * |v| are float16 operands,
  // so the wavefront divides them (and its denominator, which keeps the
  // ratio) by 2^ev, ev = the exponent of the largest value norm among the
  // tokens of its first step. The weights of those tokens then sit near the
  // top of the float16 range whatever the norms' overall scale (tiny value
  // norms would otherwise fall into float16 subnormals); ev enters through
  // m_off, which the merges already carry per wavefront.
  auto set_ev = [&](float vn) {
    float vm = fabsf(vn);
    vm = fmaxf(vm, dpp_xor1(vm));
    vm = fmaxf(vm, dpp_xor2(vm));
    vm = fmaxf(vm, dpp_ror4(vm));
    vm = fmaxf(vm, dpp_ror8(vm));
    vm = fmaxf(vm, shfl_xor_f(vm, 16));
    vm = fmaxf(vm, shfl_xor_f(vm, 32));
    int e = (vm > 0.f && vm < INFINITY) ? __builtin_amdgcn_frexp_expf(vm) : 0;
    e = e < -kNormExpClamp ? -kNormExpClamp : (e > kNormExpClamp ? kNormExpClamp : e);
    st.ev = (float)__builtin_amdgcn_readfirstlane(e);
  };
  // (from the first full step, read ahead; a share without full steps takes
  // its first masked step below)
  st.ev = 0.f;
  if (t_begin < t_full) set_ev(buf[0].nm.vn);
#pragma unroll
  for (int nb = 0; nb < CV; ++nb) st.acc0[nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---- stream the share: full 32-token steps with two register buffers in
  // turn, then at most one masked step for a ragged end. A step first waits
  // for its own loads (code words and norms, issued a step earlier, so
  // normally complete), then issues the loads of the next step, if any, and
  // computes: the next step's loads stay in flight for the whole step, and no
  // wait inside the step depends on whether they were issued.
  // Balance: the sequencer favours older wavefronts, so with equal shares the
  // younger ones would finish last and leave the compute unit a tail with few
  // wavefronts (little memory parallelism). Each step a wavefront counts
  // itself in a workgroup counter and runs at raised priority while it is more
  // than one round of steps behind the workgroup average, at lowered priority
  // while it is ahead.
  int t0 = t_begin;
  if (t0 < t_full) {
    uint32_t mine = 0;   // steps begun by this wavefront
#define TQ_STEP(CUR, NEXT)                                                                                  \
    {                                                                                                       \
      wait_step(CUR);                                                                                       \
      if (t0 + AH * kStep < t_full) {                                                                       \
        const int tl = t0 + AH * kStep, tn = tl + kStep;                                                    \
        const uint32_t rk = step_row(a.kpm, kv, a.H_kv, ek, tl);                                            \
        const uint32_t rv = step_row(a.vpm, kv, a.H_kv, ev, tl);                                            \
        /* the entry changes only where the following step starts a block */                               \
        if (kpg && (tn & ((1 << a.kpm.lg) - 1)) == 0) ek = page_entry(rtk, a.kpm, tn);                      \
        if (vpg && (tn & ((1 << a.vpm.lg) - 1)) == 0) ev = page_entry(rtv, a.vpm, tn);                      \
        load_step<false>(NEXT, s, lo, rk, rv);                                                                     \
      }                                                                                                     \
      /* count this step with an atomic add whose result (the workgroup's count */                         \
      /* before it) is first used after the step, when the step's own LDS reads */                            \
      /* have completed anyway */                                                                              \
      uint32_t prior = 0u;                                                                                  \
      if (lane == 0) prior = __hip_atomic_fetch_add(steps_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); \
      scan_step<KB, VB, QJL, WIDE, false, D>(CUR, q, st, (const char*)lut, lr, lutS, lrep, t0 + 8 * g, lim_lane);\
      const uint32_t begun = __builtin_amdgcn_readfirstlane(prior) + 1u;                                    \
      const uint32_t even = (mine + 1) * (uint32_t)NW;  /* if every wavefront kept pace */                   \
      if (begun > even + NW) __builtin_amdgcn_s_setprio(3);                                                 \
      else if (begun + NW < even) __builtin_amdgcn_s_setprio(0);                                            \
      else __builtin_amdgcn_s_setprio(1);                                                                   \
      ++mine;                                                                                               \
      t0 += kStep;                                                                                          \
      if (t0 >= t_full) break;                                                                              \
    }
    while (true) {
      if constexpr (AH == 1) {
        TQ_STEP(buf[0], buf[1])
        TQ_STEP(buf[1], buf[0])
      } else if constexpr (AH == 2) {
        TQ_STEP(buf[0], buf[2])
        TQ_STEP(buf[1], buf[0])
        TQ_STEP(buf[2], buf[1])
      } else {
        static_assert(AH == 3, "prefetch depth");
        TQ_STEP(buf[0], buf[3])
        TQ_STEP(buf[1], buf[0])
        TQ_STEP(buf[2], buf[1])
        TQ_STEP(buf[3], buf[2])
      }
    }
#undef TQ_STEP
    __builtin_amdgcn_s_setprio(0);
  }
  // masked steps: the ragged end of the share, and for several query tokens the
  // steps where their causal limits differ (at most two, limits differ by < 16)
  t0 = __builtin_amdgcn_readfirstlane(t0);   // wave-uniform (scalar buffer offsets)
  while (t0 < t_end) {
    StepData<KB, VB, QJL, WIDE, D> E;
    if (kpg) ek = page_entry(rtk, a.kpm, t0);
    if (vpg) ev = page_entry(rtv, a.vpm, t0);
    load_step<true, kFreshAux>(E, s, lo, step_row(a.kpm, kv, a.H_kv, ek, t0), step_row(a.vpm, kv, a.H_kv, ev, t0));
    if (t0 == t_begin) set_ev(E.nm.vn);
    scan_step<KB, VB, QJL, WIDE, true, D>(E, q, st, (const char*)lut, lr, lutS, lrep, t0 + 8 * g, lim_lane);
    t0 += kStep;
  }

  // ---- this wavefront's partial: lane (g, c) holds coordinates
  // (D/16)(4g + r) + nb of column c
  float o[CV][4];
#pragma unroll
  for (int nb = 0; nb < CV; ++nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = st.acc0[nb][r];
      if constexpr (!WIDE) x += dpp_ror8(x);   // columns c and c+8 hold the two token halves
      o[nb][r] = x;
    }
  }
  float l = st.l;
  if constexpr (!WIDE) l += dpp_ror8(l);   // the hi and lo lanes each summed half of the tokens
  l += shfl_xor_f(l, 16);
  l += shfl_xor_f(l, 32);

  // ---- merge the wavefront partials in LDS (fixed order)
  const bool finish = a.n_split == 1;
  // The workgroup ends with Pi_V^T applied: to o' / l with one chunk (the
  // output), to the chunk's unnormalised sums otherwise (the rotation is
  // linear, so the chunk merge can follow it). d = 128: thread (s, p) takes
  // columns 2p, 2p+1 of Pi_V over rows s*RW .. s*RW+RW-1, loaded now (a
  // wavefront reads whole rows) so that the loads are in flight while the
  // wavefront waits for the others and during the merge.
  constexpr int FSEGS = NT / 64, RW = kD / FSEGS;
  const int fp = tid & 63, fs = tid >> 6;
  float2 pv[RW];
  if constexpr (D == kD) {
    {
#pragma unroll
      for (int k = 0; k < RW; ++k) pv[k] = *(const float2*)(a.rotV + (fs * RW + k) * kD + 2 * fp);
    }
  }
  __syncthreads();   // every wavefront is done with the lookup tables
  float* mrg = R;    // [wave][MC columns][MS]: D coordinates, m, l
  if (c < NC) {
    float* dst = mrg + (wave * MC + c) * MS;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int q4 = 0; q4 < CV / 4; ++q4)
        *(float4*)(dst + CV * (4 * g + r) + 4 * q4) =
            float4{o[4 * q4][r], o[4 * q4 + 1][r], o[4 * q4 + 2][r], o[4 * q4 + 3][r]};
    }
    if (g == 0) {
      dst[D] = st.m_off;
      dst[D + 1] = l;
    }
  }
  __syncthreads();
  // weights of the wavefront partials: lane (h, w) of the first NC * 16 threads
  // (column h in a 16-lane row) takes f = 2^(m_w - M) with M the largest m_w of
  // the column, and the row sums f * l_w into the denominator
  float* fw = vA;            // [NC][16]
  float* Mh = vA + 256;      // [16]
  float* dh = vA + 272;      // [16]
  if (tid < NC * 16) {
    const int h = tid >> 4, w = tid & 15;
    float m = -INFINITY, lw = 0.f;
    if (w < NW) {
      m = mrg[(w * MC + h) * MS + D];
      lw = mrg[(w * MC + h) * MS + D + 1];
    }
    float M = fmaxf(m, dpp_xor1(m));
    M = fmaxf(M, dpp_xor2(M));
    M = fmaxf(M, dpp_ror4(M));
    M = fmaxf(M, dpp_ror8(M));
    const float f = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M);
    float den = f * lw;
    den += dpp_xor1(den);
    den += dpp_xor2(den);
    den += dpp_ror4(den);
    den += dpp_ror8(den);
    fw[h * 16 + w] = f;
    if (w == 0) {
      Mh[h] = M;
      dh[h] = den;
    }
  }
  __syncthreads();
  // column h -> query row b * M + i0 + h / G, head kv * G + h % G
  auto out_row = [&](int h) -> int64_t {
    return ((int64_t)b * a.M + i0 + h / G) * a.H_q + (int64_t)kv * G + h % G;
  };
  for (int idx = tid; idx < NC * D; idx += NT) {
    const int h = idx / D, j = idx % D;
    float num = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) num = fmaf(fw[h * 16 + wv], mrg[(wv * MC + h) * MS + j], num);
    const float den = dh[h];
    if (finish) {
      vB[idx] = den > 0.f ? num / den * a.inv_sqrt_d : 0.f;
    } else {
      vB[idx] = num;
      if (j == 0) {
        const int64_t pidx = out_row(h) * a.n_split + split;
        a.ml[pidx * 2] = Mh[h];
        a.ml[pidx * 2 + 1] = den;
      }
    }
  }
  // destination of column h's rotated vector: the output, or the chunk partial
  auto rot_dst = [&](int h) -> float* {
    return finish ? a.out + out_row(h) * D : a.acc + (out_row(h) * a.n_split + split) * D;
  };
  {
    __syncthreads();   // vB is complete; the merge area takes the partial sums
    if constexpr (D == kD) {
      float* P = R;      // [FSEGS][NC][d]
      for (int h = 0; h < NC; ++h) {
        const float4* x = (const float4*)(vB + h * kD + fs * RW);   // same address across the wavefront
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int k = 0; k < RW / 4; ++k) {
          const float4 v = x[k];
          acc0 = fmaf(pv[4 * k + 3].x, v.w, fmaf(pv[4 * k + 2].x, v.z, fmaf(pv[4 * k + 1].x, v.y, fmaf(pv[4 * k].x, v.x, acc0))));
          acc1 = fmaf(pv[4 * k + 3].y, v.w, fmaf(pv[4 * k + 2].y, v.z, fmaf(pv[4 * k + 1].y, v.y, fmaf(pv[4 * k].y, v.x, acc1))));
        }
        *(float2*)(P + (fs * NC + h) * kD + 2 * fp) = float2{acc0, acc1};
      }
      __syncthreads();
      for (int idx = tid; idx < NC * kD; idx += NT) {
        const int h = idx / kD, i = idx % kD;
        float r = 0.f;
#pragma unroll
        for (int sg = 0; sg < FSEGS; ++sg) r += P[(sg * NC + h) * kD + i];
        rot_dst(h)[i] = r;
      }
    } else {
      // thread (i, hg): coordinate i of heads hg, hg + NT/D, ... from column i
      // of Pi_V (a wavefront reads consecutive columns of one row per load)
      constexpr int HG = NT / D;
      const int i = tid % D, hg = tid / D;
      float r[16 / HG];
#pragma unroll
      for (int k = 0; k < 16 / HG; ++k) r[k] = 0.f;
#pragma unroll 8
      for (int j = 0; j < D; ++j) {
        const float pj = a.rotV[(int64_t)j * D + i];
#pragma unroll
        for (int k = 0; k < 16 / HG; ++k) {
          const int h = hg + k * HG;
          if (h < NC) r[k] = fmaf(pj, vB[h * D + j], r[k]);
        }
      }
#pragma unroll
      for (int k = 0; k < 16 / HG; ++k) {
        const int h = hg + k * HG;
        if (h < NC) rot_dst(h)[i] = r[k];
      }
    }
  }
}

// ------------------------------------------------------------------ merge --

// Fixed-order merge of the context-chunk partials of each query vector (m, l
// and the chunk's sums already in the output basis): out = sum_c 2^(m_c - M)
// acc_c / sum_c 2^(m_c - M) l_c / sqrt(d), M the largest m_c. Four consecutive
// lanes take one (vector, 4 coordinates): lane p merges chunks p, p + 4, ...,
// BATCH at a time with every load in flight together, under a running
// reference; the four parts then meet over lane exchanges (xor 1, then xor 2).
// The batch is the smallest of 1, 2, 4, 8 that covers the chunks (8 above 32
// chunks), so that with few chunks a lane does not re-read its own chunk to
// fill empty slots; up to 32 chunks a lane merges all its chunks in one batch.
template <int D, int BATCH>
__global__ __launch_bounds__(256) void merge_kernel(const float* ml, const float* acc, float* out, int64_t nvec,
                                                    int n_split, float inv_sqrt_d) {
  constexpr int Q = D / 4;   // coordinate quads of a vector
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int part = threadIdx.x & 3;
  const int64_t vq = t >> 2;   // (vector, quad)
  const bool live = vq < nvec * Q;
  const int64_t v = live ? vq / Q : 0;
  const int q4 = live ? (int)(vq % Q) : 0;
  const float* mlv = ml + v * n_split * 2;
  const float* av = acc + v * n_split * D + 4 * q4;
  float M = -INFINITY, den = 0.f;
  float4 num = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    for (int c0 = part; c0 < n_split; c0 += 4 * BATCH) {
      float mv[BATCH], lv[BATCH];
      float4 xv[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        // (chunks past n_split read chunk part again and are dropped below)
        const int c = c0 + 4 * u < n_split ? c0 + 4 * u : part;
        mv[u] = mlv[2 * c];
        lv[u] = mlv[2 * c + 1];
        xv[u] = *(const float4*)(av + (int64_t)c * D);
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        if (c0 + 4 * u >= n_split) mv[u] = -INFINITY;   // (a chunk that saw no token carries -inf too)
      float bm = M;
#pragma unroll
      for (int u = 0; u < BATCH; ++u) bm = fmaxf(bm, mv[u]);
      if (bm == -INFINITY) continue;
      const float f = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - bm);
      num.x *= f; num.y *= f; num.z *= f; num.w *= f;
      den *= f;
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const float w = mv[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[u] - bm);
        num.x = fmaf(w, xv[u].x, num.x);
        num.y = fmaf(w, xv[u].y, num.y);
        num.z = fmaf(w, xv[u].z, num.z);
        num.w = fmaf(w, xv[u].w, num.w);
        den = fmaf(w, lv[u], den);
      }
      M = bm;
    }
  }
  // the four parts of a (vector, quad), in a fixed order
#pragma unroll
  for (int x = 1; x <= 2; x <<= 1) {
    const float Mo = shfl_xor_f(M, x);
    const float Mn = fmaxf(M, Mo);
    const float fs = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    const float fo = Mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mo - Mn);
    const float4 no = {shfl_xor_f(num.x, x), shfl_xor_f(num.y, x), shfl_xor_f(num.z, x), shfl_xor_f(num.w, x)};
    const float dno = shfl_xor_f(den, x);
    // (the lower lane's part first, so both lanes of a pair compute the same sums)
    const bool low = (part & x) == 0;
    const float fa = low ? fs : fo, fb = low ? fo : fs;
    const float4 na = low ? num : no, nb = low ? no : num;
    const float da = low ? den : dno, db = low ? dno : den;
    num.x = na.x * fa + nb.x * fb;
    num.y = na.y * fa + nb.y * fb;
    num.z = na.z * fa + nb.z * fb;
    num.w = na.w * fa + nb.w * fb;
    den = da * fa + db * fb;
    M = Mn;
  }
  if (live && part == 0) {
    const float g = den > 0.f ? inv_sqrt_d / den : 0.f;
    *(float4*)(out + v * D + 4 * q4) = float4{num.x * g, num.y * g, num.z * g, num.w * g};
  }
}

template <int KB, int VB, int QJL, int WIDE, int D>
hipError_t launch_scan(const DecodePlan& p, const ScanArgs& sa, hipStream_t stream) {
  dim3 grid((unsigned)p.n_split, (unsigned)p.H_kv, (unsigned)(p.B * p.nqt));
  constexpr int NT = 64 * scan_waves<QJL, WIDE, D>();
  if (sa.kpm.table != nullptr || sa.vpm.table != nullptr)
    hipLaunchKernelGGL((decode_scan_kernel<KB, VB, QJL, WIDE, 1, D>), grid, dim3(NT), 0, stream, sa);
  else
    hipLaunchKernelGGL((decode_scan_kernel<KB, VB, QJL, WIDE, 0, D>), grid, dim3(NT), 0, stream, sa);
  return hipGetLastError();
}

template <int KB, int VB, int QJL, int D>
hipError_t dispatch_wide(const DecodePlan& p, const ScanArgs& sa, hipStream_t s) {
  // (d = 256 has no 16-column tile: the host takes such calls elsewhere)
  if constexpr (D > kD) return launch_scan<KB, VB, QJL, 0, D>(p, sa, s);
  else return p.wide ? launch_scan<KB, VB, QJL, 1, D>(p, sa, s) : launch_scan<KB, VB, QJL, 0, D>(p, sa, s);
}

template <int KB, int VB, int D>
hipError_t dispatch_qjl(const DecodePlan& p, const ScanArgs& sa, hipStream_t s) {
  // (QJL keys exist at d = 128 only)
  if constexpr (D != kD) return dispatch_wide<KB, VB, 0, D>(p, sa, s);
  else return p.qjl ? dispatch_wide<KB, VB, 1, D>(p, sa, s) : dispatch_wide<KB, VB, 0, D>(p, sa, s);
}

template <int KB, int D>
hipError_t dispatch_vb(int vb, const DecodePlan& p, const ScanArgs& sa, hipStream_t s) {
  switch (vb) {
    case 2: return dispatch_qjl<KB, 2, D>(p, sa, s);
    case 3: return dispatch_qjl<KB, 3, D>(p, sa, s);
    default: return dispatch_qjl<KB, 4, D>(p, sa, s);
  }
}

template <int D>
hipError_t dispatch_kb(int kb, int vb, const DecodePlan& p, const ScanArgs& sa, hipStream_t s) {
  switch (kb) {
    case 2: return dispatch_vb<2, D>(vb, p, sa, s);
    case 3: return dispatch_vb<3, D>(vb, p, sa, s);
    default: return dispatch_vb<4, D>(vb, p, sa, s);
  }
}

}  // namespace

hipError_t launch_decode(const DecodePlan& p, const tq_cache* k, const tq_cache* v, const void* q,
                         int q_dtype, const int32_t* ctx_lens, float scale, float* out, void* ws,
                         hipStream_t stream, const DecodeAppend* app) {
  char* base = (char*)ws;
  float* ml = (float*)(base + p.off_ml);
  float* acc = (float*)(base + p.off_acc);
  const int d = k->d;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);

  ScanArgs sa;
  sa.kcodes = k->codes;
  sa.knorms = k->norms;
  sa.ksigns = k->qjl_signs;
  sa.kgamma = k->qjl_gamma;
  sa.vcodes = v->codes;
  sa.vnorms = v->norms;
  sa.q = q;
  sa.rotK = k->rot;
  sa.proj = p.qjl ? k->qjl_proj : nullptr;
  sa.rotV = v->rot;
  sa.ctx_lens = ctx_lens;
  sa.out = out;
  sa.ml = ml;
  sa.acc = acc;
  sa.TcK = k->T_cap;
  sa.TcV = v->T_cap;
  sa.kpm = page_map(k);
  sa.vpm = page_map(v);
  sa.q_dtype = q_dtype;
  sa.H_kv = (int)p.H_kv;
  sa.H_q = (int)p.H_q;
  sa.G = p.G;
  sa.T = (int)p.T;
  sa.n_split = p.n_split;
  sa.M = (int)p.M;
  sa.Mt = p.Mt;
  sa.nqt = p.nqt;
  sa.wg_chunk = p.chunk;
  sa.wave_chunk = p.chunk / ((p.qjl || p.wide || d > kD) ? 8 : kCommonWaves);
  // the query operand carries log2(e) * scale / sqrt(d) (scores in the log2
  // domain); the QJL part log2(e) * scale * sqrt(pi/2) / d
  sa.sc1 = scale * kLog2e * inv_sqrt_d;
  sa.sc2 = scale * kLog2e * sqrtf((float)M_PI / 2.0f) / (float)kD;
  sa.inv_sqrt_d = inv_sqrt_d;
  for (int i = 0; i < 16; ++i) {
    sa.kc[i] = i < (1 << k->bits) ? k->centroids[i] : 0.f;
    sa.vc[i] = i < (1 << v->bits) ? v->centroids[i] : 0.f;
  }
  sa.app = app != nullptr ? 1 : 0;
  sa.app_xf32 = app != nullptr && app->x_dtype == TQ_F32 ? 1 : 0;
  if (app != nullptr) {
    sa.qk = make_quant_args(app->k, p.B, 1, p.H_kv, app->k_sb, 0, app->k_sh, k, p.T - 1);
    sa.qv = make_quant_args(app->v, p.B, 1, p.H_kv, app->v_sb, 0, app->v_sh, v, p.T - 1);
  } else {
    sa.qk = QuantArgs{};
    sa.qv = QuantArgs{};
  }
  hipError_t err;
  if (d == 64) err = dispatch_kb<64>(k->bits, v->bits, p, sa, stream);
  else if (d == 256) err = dispatch_kb<256>(k->bits, v->bits, p, sa, stream);
  else err = dispatch_kb<kD>(k->bits, v->bits, p, sa, stream);
  if (err != hipSuccess || p.n_split == 1) return err;
  return launch_merge(ml, acc, out, p.B * p.M * p.H_q, p.n_split, d, stream);
}

hipError_t launch_merge(const float* ml, const float* acc, float* out, int64_t nvec, int n_split, int d,
                        hipStream_t stream) {
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  const int64_t threads = nvec * (d / 4) * 4;
  const dim3 grid((unsigned)((threads + 255) / 256));
  const int nb = n_split <= 4 ? 1 : n_split <= 8 ? 2 : n_split <= 16 ? 4 : 8;
  auto go = [&](auto dt, auto bt) {
    constexpr int DD = decltype(dt)::value, NB = decltype(bt)::value;
    hipLaunchKernelGGL((merge_kernel<DD, NB>), grid, dim3(256), 0, stream, ml, acc, out, nvec, n_split, inv_sqrt_d);
  };
  auto by_batch = [&](auto dt) {
    if (nb == 1) go(dt, IntConst<1>());
    else if (nb == 2) go(dt, IntConst<2>());
    else if (nb == 4) go(dt, IntConst<4>());
    else go(dt, IntConst<8>());
  };
  if (d == 64) by_batch(IntConst<64>());
  else if (d == 256) by_batch(IntConst<256>());
  else by_batch(IntConst<kD>());
  return hipGetLastError();
}

}  // namespace tq
