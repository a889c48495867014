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
//   epilogue  the wavefront partials are merged in LDS in a fixed order; with
//             a single chunk (the usual case once B * H_kv fills the part) the
//             workgroup applies o = Pi_V^T o' and writes the output itself.
// Paged caches: a step's token rows come from the block table (an entry read
// one step ahead); a 32-token step never crosses a block. A separate
// instantiation keeps the contiguous path free of that work.
// combine (only when the context is split into several chunks): fixed-order
// merge of the chunk partials of each query head, then o = Pi_V^T o'.
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
// 2^(s - m - kShift) * |v| with kShift = kSlack + log2(sqrt(d)), which keeps
// every weight operand at or below |v| / sqrt(d) (float16 range for |v| < 7e5)
// and leaves one 1/sqrt(d) for the combine.
#include <math.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

typedef float float2v __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 2.0f;
constexpr float kShift = kSlack + 3.5f;   // + log2(sqrt(128))
constexpr int kLutRep = 32;              // LUT replicas (power of two)
constexpr int kStreamAux = 2;            // cache policy of the streamed cache reads: non-temporal
constexpr int kLutShift = 5;             // log2(kLutRep)

__device__ inline float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }


// ------------------------------------------------------ small matrix work --

constexpr int kVecWords = 16 * kD;         // [16][d] float vectors
// Column stride (in halves) of the float16 query operand in LDS: the 16 lanes
// that read one 16-byte piece of 16 different columns then hit distinct banks.
constexpr int kQStride = kD + 8;
// Scratch region of a decode workgroup, in 32-bit words: the lookup tables
// (scan), then the wavefront partials (merge) and the partial sums of the final
// rotation, followed by two [16][d] float vector sets.
constexpr int kRegionWords = 16896;
// Row stride (in floats) of a wavefront partial in the merge area: 128
// coordinates, m and l, padded to a 16-byte multiple.
constexpr int kMergeStride = kD + 4;
constexpr int kScratchWords = kRegionWords + 2 * kVecWords;

// q' = M q for the G query heads of a workgroup: out[h][i] = sum_j M[i][j]
// in[h][j] (in, out: LDS [G][d]). Thread t takes rows R*(t/16) .. R*(t/16)+R-1
// of M (R = 2048 / NT) over the 8 columns 8*(t%16) .. 8*(t%16)+7, loaded
// straight from memory (16 consecutive lanes read whole rows; each element of
// M is read once, no staging), so every query element read from LDS serves R
// rows. The 16 segments of a row group sit in the 16 lanes of a DPP row and
// are summed with DPP exchanges, for all heads at once.
template <int NT>
struct RowSegment {
  static constexpr int R = 16 * kD / NT;   // rows per thread
  float4 r[2 * R];                        // row k: r[2k], r[2k + 1]
};

template <int NT>
__device__ inline void load_row_segment(RowSegment<NT>& rs, const float* M) {
  constexpr int R = RowSegment<NT>::R;
  const int i0 = R * (threadIdx.x / 16), sg = threadIdx.x % 16;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    rs.r[2 * k] = *(const float4*)(M + (i0 + k) * kD + 8 * sg);
    rs.r[2 * k + 1] = *(const float4*)(M + (i0 + k) * kD + 8 * sg + 4);
  }
}

template <int NT, int MAXG>
__device__ void rotate_rows(const RowSegment<NT>& rs, const float* in, float* out, int G) {
  constexpr int R = RowSegment<NT>::R;
  const int i0 = R * (threadIdx.x / 16), sg = threadIdx.x % 16;
  float acc[MAXG][R];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
#pragma unroll
    for (int k = 0; k < R; ++k) acc[h][k] = 0.f;
    if (h < G) {
      const float4 a = *(const float4*)(in + h * kD + 8 * sg);
      const float4 b = *(const float4*)(in + h * kD + 8 * sg + 4);
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const float4 m0 = rs.r[2 * k], m1 = rs.r[2 * k + 1];
        const float v = fmaf(m0.x, a.x, fmaf(m0.y, a.y, fmaf(m0.z, a.z, m0.w * a.w)));
        acc[h][k] = fmaf(m1.x, b.x, fmaf(m1.y, b.y, fmaf(m1.z, b.z, fmaf(m1.w, b.w, v))));
      }
    }
  }
  // sums over the 16 lanes of the row: quads, then rotates by 4 and 8 (every
  // lane ends with the full sum)
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float v = acc[h][k] + dpp_xor1(acc[h][k]);
      v += dpp_xor2(v);
      v += dpp_ror4(v);
      v += dpp_ror8(v);
      acc[h][k] = v;
    }
  }
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    if (h < G && sg == h) {
#pragma unroll
      for (int k = 0; k < R; ++k) out[h * kD + i0 + k] = acc[h][k];
    }
  }
}

// Float16 operand of vals[G][d] * sc: a power of two per head puts its largest
// entry in [2^13, 2^14) (cs[h] = that power, 1 for absent heads); column h of
// dst holds the hi halves, column half_cols + h the lo halves, ~22 bits
// together (zero columns for absent heads). Needs NT >= 256; ends with the
// operand written by each thread, no barrier.
template <int NT>
__device__ void emit_operand(const float* vals, float sc, int G, int half_cols, _Float16* dst, float* cs,
                             int* hexp) {
  const int tid = threadIdx.x;
  if (tid < 256) {
    // thread (h, seg): largest magnitude over 8 entries, then over the 16 segments
    const int h = tid >> 4, seg = tid & 15;
    float mx = 0.f;
    if (h < G) {
#pragma unroll
      for (int k = 0; k < 8; ++k) mx = fmaxf(mx, fabsf(vals[h * kD + 8 * seg + k] * sc));
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
  for (int idx = tid; idx < 2 * half_cols * kD; idx += NT) {
    const int col = idx / kD, i = idx % kD;
    const int h = col % half_cols;
    float v = 0.f;
    if (h < G) v = ldexpf(vals[h * kD + i] * sc, -hexp[h]);
    const _Float16 hi = (_Float16)v;
    dst[col * kQStride + i] = col >= half_cols ? (_Float16)(v - (float)hi) : hi;
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
  const void* q;
  const float* rotK;   // Pi_K
  const float* proj;   // S (QJL keys), or null
  const float* rotV;   // Pi_V
  const int32_t* ctx_lens;
  float* out;    // [B][H_q][128], written when n_split == 1
  float* ml;     // [B][H_q][n_split][2], partials when n_split > 1
  float* acc;    // [B][H_q][n_split][128]
  int64_t TcK, TcV;
  PageMap kpm, vpm;   // block tables of paged caches (table == nullptr: contiguous)
  int q_dtype, H_kv, H_q, G, T, n_split, wg_chunk, wave_chunk;
  int M, Mt, nqt;   // query tokens per row, per workgroup tile, tiles per row
  float sc1, sc2, inv_sqrt_d;
  float kc[16], vc[16];
};

// Codebook lookup table in LDS, shared by keys and values: 256 slots of 256
// bytes, slot x for the 8 bits x that start at a code pair's position in the
// packed words (the pair's 2*bits wide field, then bits of the next pair, which
// the entry ignores). A slot holds the float16 levels of the key pair in
// kLutRep replicas (bytes 0-127) and of the value pair (bytes 128-255); lane l
// reads replica l % kLutRep, so the lanes of a wavefront hit distinct banks.
// The address of a lookup is a register whose byte 0 holds the lane's replica
// offset: one SDWA shift writes the 8 bits into byte 1 (x * 256) and leaves the
// rest, so a lookup costs one VALU instruction (two where a pair straddles two
// words). (Entries of 4 codes, 8 bytes, would halve the lookups, but their
// unreplicated random reads cost more LDS time than they save on this part.)
constexpr int kLutBytes = 256 * 256;

// Thread (slot, quarter) writes 8 replicas of the slot's key pair and 8 of its
// value pair (two 16-byte stores each), so each pair is formed once per thread.
template <int KB, int VB>
__device__ void build_lut(uint32_t* lut, const float* cK, const float* cV, int tid, int nt) {
  for (int e = tid; e < 256 * 4; e += nt) {
    const int x = e >> 2, qr = e & 3;
    const int fk = x & ((1 << (2 * KB)) - 1), fv = x & ((1 << (2 * VB)) - 1);
    const uint32_t pk = pack_half2(cK[fk & ((1 << KB) - 1)], cK[fk >> KB]);
    const uint32_t pv = pack_half2(cV[fv & ((1 << VB) - 1)], cV[fv >> VB]);
    uint4* dk = (uint4*)(lut + x * 64 + 8 * qr);
    uint4* dv = (uint4*)(lut + x * 64 + 32 + 8 * qr);
    dk[0] = dk[1] = uint4{pk, pk, pk, pk};
    dv[0] = dv[1] = uint4{pv, pv, pv, pv};
  }
}

// Address registers of the lookups (two sets, so that consecutive operands do
// not wait on each other's reads): byte 0 = replica offset, byte 1 = slot.
struct LutRegs {
  uint32_t a[4], b[4];
};

// Byte 1 of r = the 8 bits at bit P of the lane's N-word slice w (zeros past
// the slice); a field of W bits that straddles two words is first aligned.
template <int N, int P, int W>
__device__ inline void lut_slot(uint32_t& r, const uint32_t* w) {
  constexpr int wi = P / 32, sh = P % 32;
  if constexpr (sh + W <= 32 || wi + 1 >= N) {
    asm("v_lshrrev_b32_sdwa %0, %2, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(r) : "v"(w[wi]), "i"(sh));
  } else {
    const uint32_t t = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
    asm("v_lshrrev_b32_sdwa %0, 0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(r) : "v"(t));
  }
}

// Float16 codebook levels of the 8 codes at bit offset POS of the lane's
// N-word slice w (codes LSB first), from the key (OFF 0) or value (OFF 128)
// half of the table: an MFMA operand of 8 halves.
template <int BITS, int N, int POS, int OFF>
__device__ inline half8 levels8(const uint32_t* w, const char* lut, uint32_t (&r)[4]) {
  constexpr int W = 2 * BITS;
  lut_slot<N, POS + 0 * W, W>(r[0], w);
  lut_slot<N, POS + 1 * W, W>(r[1], w);
  lut_slot<N, POS + 2 * W, W>(r[2], w);
  lut_slot<N, POS + 3 * W, W>(r[3], w);
  const uint32_t r0 = *(const uint32_t*)(lut + r[0] + OFF);
  const uint32_t r1 = *(const uint32_t*)(lut + r[1] + OFF);
  const uint32_t r2 = *(const uint32_t*)(lut + r[2] + OFF);
  const uint32_t r3 = *(const uint32_t*)(lut + r[3] + OFF);
  return words_to_half8(r0, r1, r2, r3);
}

// A operand of the QK MFMA for step KK: coordinates 32g + 8KK + 0..7 of the
// lane's token, from the lane's KB-word slice (coordinates 32g .. 32g+31).
template <int KB, int KK>
__device__ inline half8 key_operand(const uint32_t* w, const char* lut, uint32_t (&r)[4]) {
  return levels8<KB, KB, 8 * KB * KK, 0>(w, lut, r);
}

// A operand of the PV MFMA for coordinate block NB: value codes of the 8 tokens
// of the lane's block at coordinate 8i + NB (i = lane % 16), from the lane's
// 2*VB-word slice of the block record (coordinates 8i .. 8i+7).
template <int VB, int NB>
__device__ inline half8 value_operand(const uint32_t* w, const char* lut, uint32_t (&r)[4]) {
  return levels8<VB, 2 * VB, 8 * VB * NB, 128>(w, lut, r);
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

// Norms (and QJL gammas) of one step: each lane reads one token's. For G <= 8
// the two lanes of a hi/lo column pair split the 8 tokens of their row block
// (lane half hf takes tokens 4hf .. 4hf+3) and lane (g, c) reads token
// 8g + 4hf + c % 4, so the 4 tokens a lane needs are in its quad; for
// 8 < G <= 16 every lane needs all 8 tokens of its row block and lane (g, c)
// reads token 8g + c % 8, so they are in lanes 0-7 of its row. The values
// reach the lanes that need them as DPP operands of their multiplies: one
// 4-byte read per lane and stream instead of 16 or 32 bytes.
template <int QJL>
struct StepNorms {
  float kn, vn, kg;
};

// Raw words of one 32-token step for one lane, with the step's norms.
template <int KB, int VB, int QJL, int WIDE>
struct StepData {
  uint32_t kw[2][KB];
  uint32_t sw[2];
  uint32_t vw[2 * VB];
  StepNorms<QJL> nm;
};

struct Streams {
  __amdgpu_buffer_rsrc_t rk, rkn, rv, rvn, rs, rg;
};

// Block-table entry of the block holding token t (paged caches): an
// asynchronous read through the range-checked table row rt.
__device__ inline uint32_t page_entry(__amdgpu_buffer_rsrc_t rt, const PageMap& m, int t) {
  return __builtin_amdgcn_raw_buffer_load_b32(rt, (uint32_t)(t >> m.lg) * 4u, 0, 0);
}

// Token row (relative to the stream base) of the step starting at token t: t
// itself for a contiguous cache; for a paged one, row t % 2^lg of head kv in
// physical block e (clamped into the arrays, so entries the caller left
// unset are never dereferenced out of bounds). A step never crosses a block
// (blocks are multiples of 32 tokens, steps start at multiples of 32).
__device__ inline uint32_t step_row(const PageMap& m, int kv, int H_kv, uint32_t e, int t) {
  if (m.table == nullptr) return (uint32_t)t;
  // (unsigned compare written out: a mixed-type min() resolves to the double overload)
  const uint32_t p0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)e), plast = (uint32_t)(m.nblk - 1);
  const uint32_t p = p0 < plast ? p0 : plast;
  return ((p * (uint32_t)H_kv + (uint32_t)kv) << m.lg) + ((uint32_t)t & ((1u << m.lg) - 1u));
}

template <int N>
__device__ inline void bload_words_s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* w) {
  if constexpr (N == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamAux);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (N == 3) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, kStreamAux);
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  } else if constexpr (N == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamAux);
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

// Waits until the loads of d have landed (an empty asm that reads every word:
// the compiler places the counter wait before it).
template <int KB, int VB, int QJL, int WIDE>
__device__ inline void wait_step(const StepData<KB, VB, QJL, WIDE>& d) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int k = 0; k < KB; ++k) asm volatile("" ::"v"(d.kw[m][k]));
    if constexpr (QJL) asm volatile("" ::"v"(d.sw[m]));
  }
#pragma unroll
  for (int k = 0; k < 2 * VB; ++k) asm volatile("" ::"v"(d.vw[k]));
  asm volatile("" ::"v"(d.nm.kn), "v"(d.nm.vn));
  if constexpr (QJL) asm volatile("" ::"v"(d.nm.kg));
}

// Loads one step: rk, rv are the token rows of the step's first token in the
// key and value arrays (relative to the stream bases; 32 consecutive rows).
// Full steps (CHECKED false) pass the step offset as the scalar offset, which
// the hardware does not range check: all 32 rows must lie inside the stream.
// A step that may run past the end of a stream (the ragged end of a row whose
// capacity is not a multiple of 32) adds it to the per-lane offsets instead,
// so that lanes past the end read zeros.
template <bool CHECKED, int KB, int VB, int QJL, int WIDE>
__device__ inline void load_step(StepData<KB, VB, QJL, WIDE>& d, const Streams& s, const LaneOffsets& lo,
                                 uint32_t rk, uint32_t rv) {
  constexpr int KW = 4 * KB, VBW = 32 * VB;
  // wave-uniform; readfirstlane keeps the step offsets in scalar registers
  rk = __builtin_amdgcn_readfirstlane(rk);
  rv = __builtin_amdgcn_readfirstlane(rv);
  const uint32_t ok = rk * (KW * 4u), os = rk * 16u, ov = (rv / 8u) * (VBW * 4u), onk = rk * 4u, onv = rv * 4u;
  // (TQ_OFF: the scalar offset of a load; TQ_VOF: its per-lane offset)
#define TQ_OFF(o) (CHECKED ? 0u : (o))
#define TQ_VOF(v, o) (CHECKED ? (v) + (o) : (v))
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    bload_words_s<KB>(s.rk, TQ_VOF(lo.k[m], ok), TQ_OFF(ok), d.kw[m]);
    if constexpr (QJL)
      d.sw[m] = __builtin_amdgcn_raw_buffer_load_b32(s.rs, TQ_VOF(lo.s[m], os), TQ_OFF(os), kStreamAux);
  }
  bload_words_s<2 * VB>(s.rv, TQ_VOF(lo.v, ov), TQ_OFF(ov), d.vw);
  d.nm.kn = as_float(__builtin_amdgcn_raw_buffer_load_b32(s.rkn, TQ_VOF(lo.n, onk), TQ_OFF(onk), kStreamAux));
  d.nm.vn = as_float(__builtin_amdgcn_raw_buffer_load_b32(s.rvn, TQ_VOF(lo.n, onv), TQ_OFF(onv), kStreamAux));
  if constexpr (QJL)
    d.nm.kg = as_float(__builtin_amdgcn_raw_buffer_load_b32(s.rg, TQ_VOF(lo.n, onk), TQ_OFF(onk), kStreamAux));
#undef TQ_OFF
#undef TQ_VOF
}



template <int WIDE, int QJL>
struct QOps {
  half8 q0[4], q1[4], r0[4], r1[4];   // column c (and c + 16), coordinates 32g + 8kk + 0..7
  float cs1, cs2;
  bool hf;   // G <= 8: lane holds the lo half of its query column (column >= 8)
};

template <int WIDE>
struct SoftState {
  float m_ref, m_off, l;
  floatx4 acc0[8];
};

template <int KB, int VB, int QJL, int WIDE, bool MASK>
__device__ __forceinline__ void scan_step(const StepData<KB, VB, QJL, WIDE>& d, const QOps<WIDE, QJL>& q,
                                          SoftState<WIDE>& st, const char* lut, LutRegs& lr,
                                          const uint32_t* lutS, int lane, int tg, int lim) {
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
  {
#define TQ_QK(KK)                                                     \
    {                                                                 \
      _Pragma("unroll") for (int m = 0; m < 2; ++m) {                 \
        const half8 ka = key_operand<KB, KK>(d.kw[m], lut, m ? lr.b : lr.a); \
        s0[m] = mfma16(ka, q.q0[KK], s0[m]);                          \
        if constexpr (WIDE) s1[m] = mfma16(ka, q.q1[KK], s1[m]);      \
      }                                                               \
    }
    TQ_QK(0) TQ_QK(1) TQ_QK(2) TQ_QK(3)
#undef TQ_QK
  }
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
      for (int nb = 0; nb < 8; ++nb) st.acc0[nb] *= alpha;
      st.m_ref = m_new;
      st.m_off = m_new + kShift;
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
#define TQ_PV(NB)                                                     \
    {                                                                 \
      const half8 va = value_operand<VB, NB>(d.vw, lut, (NB & 1) ? lr.b : lr.a); \
      st.acc0[NB] = mfma16(va, pb0, st.acc0[NB]);                     \
    }
    TQ_PV(0) TQ_PV(1) TQ_PV(2) TQ_PV(3) TQ_PV(4) TQ_PV(5) TQ_PV(6) TQ_PV(7)
#undef TQ_PV
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
      for (int nb = 0; nb < 8; ++nb) st.acc0[nb] *= alpha;
      st.m_ref = m_new;
      st.m_off = m_new + kShift;
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
#define TQ_PV(NB)                                                     \
    {                                                                 \
      const half8 va = value_operand<VB, NB>(d.vw, lut, (NB & 1) ? lr.b : lr.a); \
      st.acc0[NB] = mfma16(va, pb, st.acc0[NB]);                      \
    }
    TQ_PV(0) TQ_PV(1) TQ_PV(2) TQ_PV(3) TQ_PV(4) TQ_PV(5) TQ_PV(6) TQ_PV(7)
#undef TQ_PV
  }
}


// Wavefronts per workgroup: one workgroup fills a compute unit (4 wavefronts
// per SIMD, <= 128 VGPRs, for the common tiles; the QJL and G > 8 tiles carry
// more operands and run 2 per SIMD).
constexpr int kCommonWaves = 16;
template <int QJL, int WIDE>
constexpr int scan_waves() { return (QJL || WIDE) ? 8 : kCommonWaves; }
// Steps whose loads are in flight while a wavefront computes one (register
// buffers: ahead + 1).
constexpr int kCommonAhead = 1;
template <int QJL, int WIDE>
constexpr int scan_ahead() { return (QJL || WIDE) ? 1 : kCommonAhead; }

// merge buffer: [wave][column][kMergeStride] floats, 8 columns (G <= 8) or 16
template <int WIDE>
constexpr int merge_cols() { return WIDE ? 16 : 8; }

// LDS of a decode workgroup, in 32-bit words: the float16 query operand
// ([1 + QJL][operand columns][d]), 32 column scales, 16 exponents, 32 codebook
// levels, the step counter (padded to 4 words), then the scratch region.
template <int QJL, int WIDE>
constexpr int scan_head_words() { return (1 + QJL) * (WIDE ? 32 : 16) * kQStride / 2 + 84; }

template <int KB, int VB, int QJL, int WIDE>
constexpr size_t scan_lds_bytes() {
  static_assert(kLutBytes / 4 + (QJL ? 4 : 0) * kLutRep <= kRegionWords, "lookup tables exceed the scratch region");
  static_assert(scan_waves<QJL, WIDE>() * merge_cols<WIDE>() * kMergeStride <= kRegionWords,
                "merge area exceeds the scratch region");
  static_assert(scan_waves<QJL, WIDE>() * (WIDE ? 16 : 8) * kD <= kRegionWords,
                "rotation partials exceed the scratch region");
  return (size_t)(scan_head_words<QJL, WIDE>() + kScratchWords) * 4;
}

// One workgroup per (context chunk, KV head, row):
//   prologue  q' = Pi_K q for the G query heads (and q'' = S q' for QJL keys)
//             into the float16 operand in LDS, while the first code words are
//             already in flight;
//   scan      each wavefront streams its share of the chunk;
//   epilogue  the wavefront partials are merged in LDS in a fixed order; with
//             one chunk the workgroup finishes the heads (o = Pi_V^T o'),
//             otherwise it writes the chunk partial for the combine.
template <int KB, int VB, int QJL, int WIDE, int PAGED>
__global__ __launch_bounds__((64 * scan_waves<QJL, WIDE>())) void decode_scan_kernel(ScanArgs a) {
  constexpr int NW = scan_waves<QJL, WIDE>(), NT = 64 * NW;
  constexpr int NS = QJL ? 4 : 0;
  constexpr int KW = 4 * KB;
  constexpr int MC = merge_cols<WIDE>();
  constexpr int NQ = WIDE ? 32 : 16;   // operand columns per part
  constexpr int HALF = NQ / 2;
  __shared__ __align__(16) uint32_t smem[scan_lds_bytes<KB, VB, QJL, WIDE>() / 4];
  _Float16* qlds = (_Float16*)smem;                              // [1 + QJL][NQ][kQStride]
  float* qcs = (float*)(smem + (1 + QJL) * NQ * kQStride / 2);   // [2][16]
  int* hexp = (int*)(qcs + 32);                            // [16]
  float* cents = qcs + 48;                                 // [2][16] key, value levels
  uint32_t* steps_done = (uint32_t*)(qcs + 80);            // steps begun by the workgroup
  uint32_t* U = smem + scan_head_words<QJL, WIDE>();       // scratch, 16-byte aligned
  float* R = (float*)U;   // region: lookup tables, then merge area / rotation partials
  float* vA = R + kRegionWords;
  float* vB = vA + kVecWords;
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
  s.rv = make_rsrc(a.vcodes + vbase * 4 * VB, (uint32_t)(vrows * 4 * VB * 4));
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
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int tk = 8 * (c >> 2) + 4 * m + (c & 3);   // MFMA row c of row block m
    lo.k[m] = (uint32_t)(tk * KW + g * KB) * 4u;
    lo.s[m] = (uint32_t)(tk * 4 + g) * 4u;
  }
  lo.v = (uint32_t)(g * 32 * VB + c * 2 * VB) * 4u;
  lo.n = (uint32_t)(WIDE ? 8 * g + (c & 7) : 8 * g + (hf ? 4 : 0) + (c & 3)) * 4u;

  // ---- prologue loads, in issue order: this thread's segment of the rows of
  // Pi_K, its query elements, the code words of the first steps, the context
  // length. Loads complete in issue order, so waiting for the matrix and the
  // query never waits for the code words. The first steps are read before the
  // context length is known: reads past the end of the cache return zeros
  // (buffer range check), and steps past the context are never used.
  RowSegment<NT> rseg;
  load_row_segment<NT>(rseg, a.rotK);
  constexpr int QE = 16 * kD / NT;   // query elements per thread (G <= 16)
  uint32_t qraw[QE];
  {
    // one 32-bit load per element for either dtype (a bfloat16 element is
    // taken from the word that holds it), so the loads carry no branch
    // column c's vector: token i0 + c / G, head kv * G + c % G of row b
    const bool qbf = a.q_dtype == TQ_BF16;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc((const char*)a.q + ((((int64_t)b * a.M + i0) * a.H_q + (int64_t)kv * G) * kD) * (qbf ? 2 : 4),
                  (uint32_t)((((int64_t)mq - 1) * a.H_q + G) * kD * (qbf ? 2 : 4)));
#pragma unroll
    for (int k = 0; k < QE; ++k) {
      const uint32_t idx = tid + k * NT;
      const uint32_t cq = idx / kD;
      const uint32_t el = ((cq / (uint32_t)G) * (uint32_t)a.H_q + cq % (uint32_t)G) * kD + idx % kD;
      qraw[k] = __builtin_amdgcn_raw_buffer_load_b32(rq, qbf ? (el * 2u) & ~3u : el * 4u, 0, 0);
    }
  }
  constexpr int AH = scan_ahead<QJL, WIDE>();
  StepData<KB, VB, QJL, WIDE> buf[AH + 1];
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
  // (unconditional, through an empty range when there are no context lengths,
  // and first touched after the prologue: a load under a branch, or one moved
  // to a scalar register at once, would make the prologue wait for every load
  // issued before it)
  uint32_t ctx_word = __builtin_amdgcn_raw_buffer_load_b32(
      make_rsrc(a.ctx_lens ? (const void*)a.ctx_lens : (const void*)a.knorms, a.ctx_lens ? (uint32_t)((b + 1) * 4) : 0u),
      (uint32_t)b * 4u, 0, 0);
  __builtin_amdgcn_sched_barrier(0);

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
  build_lut<KB, VB>(lut, cents, cents + 16, tid, NT);
  if constexpr (QJL) {
    for (int e = tid; e < NS * kLutRep; e += NT) {
      const int f = e >> kLutShift;
      lutS[e] = pack_half2((f & 1) ? 1.f : -1.f, (f & 2) ? 1.f : -1.f);
    }
  }
  {
    // the NC column vectors as float32 in vA ([NC][d])
#pragma unroll
    for (int k = 0; k < QE; ++k) {
      const int idx = tid + k * NT;
      if (idx < NC * kD)
        vA[idx] = a.q_dtype == TQ_BF16 ? __uint_as_float(((qraw[k] >> (16 * (idx & 1))) & 0xFFFFu) << 16)
                                       : __uint_as_float(qraw[k]);
    }
    __syncthreads();
    rotate_rows<NT, NQ / 2>(rseg, vA, vB, NC);   // q' = Pi_K q
    __syncthreads();
    emit_operand<NT>(vB, a.sc1, NC, HALF, qlds, qcs, hexp);
    if constexpr (QJL) {
      load_row_segment<NT>(rseg, a.proj);
      rotate_rows<NT, NQ / 2>(rseg, vB, vA, NC);   // q'' = S q'
      __syncthreads();
      emit_operand<NT>(vA, a.sc2, NC, HALF, qlds + NQ * kQStride, qcs + 16, hexp);
    }
  }
  __syncthreads();

  // query operand (B of QK) for this lane: column c, coordinates 32g + 8kk + 0..7
  QOps<WIDE, QJL> q;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    q.q0[kk] = *(const half8*)(qlds + c * kQStride + 32 * g + 8 * kk);
    if constexpr (WIDE) q.q1[kk] = *(const half8*)(qlds + (16 + c) * kQStride + 32 * g + 8 * kk);
    if constexpr (QJL) {
      q.r0[kk] = *(const half8*)(qlds + (NQ + c) * kQStride + 32 * g + 8 * kk);
      if constexpr (WIDE) q.r1[kk] = *(const half8*)(qlds + (NQ + 16 + c) * kQStride + 32 * g + 8 * kk);
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
  const int t_full =
      __builtin_amdgcn_readfirstlane(t_begin + (t_unm > t_begin ? (t_unm - t_begin) / kStep * kStep : 0));
  // this lane's column limit for the masked steps (columns past NC carry a zero
  // query and keep the widest limit)
  const int lcol = WIDE ? c : (c & 7);
  const int lim_lane = lcol < NC ? max(lim0 + lcol / G, 0) : lim_hi;

  LutRegs lr;
#pragma unroll
  for (int i = 0; i < 4; ++i) lr.a[i] = lr.b[i] = (uint32_t)lrep * 4u;
  SoftState<WIDE> st;
  st.m_ref = -INFINITY;
  st.m_off = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) st.acc0[nb] = floatx4{0.f, 0.f, 0.f, 0.f};

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
      /* count this step (an atomic add whose result is not waited for), then */                           \
      /* read the workgroup's count after the step */                                                        \
      if (lane == 0) __hip_atomic_fetch_add(steps_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); \
      scan_step<KB, VB, QJL, WIDE, false>(CUR, q, st, (const char*)lut, lr, lutS, lrep, t0 + 8 * g, lim_lane);\
      const uint32_t begun = __builtin_amdgcn_readfirstlane(*(volatile uint32_t*)steps_done);                \
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
    StepData<KB, VB, QJL, WIDE> E;
    if (kpg) ek = page_entry(rtk, a.kpm, t0);
    if (vpg) ev = page_entry(rtv, a.vpm, t0);
    load_step<true>(E, s, lo, step_row(a.kpm, kv, a.H_kv, ek, t0), step_row(a.vpm, kv, a.H_kv, ev, t0));
    scan_step<KB, VB, QJL, WIDE, true>(E, q, st, (const char*)lut, lr, lutS, lrep, t0 + 8 * g, lim_lane);
    t0 += kStep;
  }

  // ---- this wavefront's partial: lane (g, c) holds coordinates 32g + 8r + nb of column c
  float o[8][4];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
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
  // With one chunk the workgroup finishes with o = Pi_V^T o': thread (s, p)
  // takes columns 2p, 2p+1 of Pi_V over rows s*RW .. s*RW+RW-1, loaded now (a
  // wavefront reads whole rows) so that the loads are in flight while the
  // wavefront waits for the others and during the merge.
  constexpr int FSEGS = NT / 64, RW = kD / FSEGS;
  const int fp = tid & 63, fs = tid >> 6;
  float2 pv[RW];
  if (finish) {
#pragma unroll
    for (int k = 0; k < RW; ++k) pv[k] = *(const float2*)(a.rotV + (fs * RW + k) * kD + 2 * fp);
  }
  __syncthreads();   // every wavefront is done with the lookup tables
  float* mrg = R;    // [wave][MC columns][kMergeStride]: 128 coordinates, m, l
  if (c < NC) {
    float* dst = mrg + (wave * MC + c) * kMergeStride;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *(float4*)(dst + 32 * g + 8 * r) = float4{o[0][r], o[1][r], o[2][r], o[3][r]};
      *(float4*)(dst + 32 * g + 8 * r + 4) = float4{o[4][r], o[5][r], o[6][r], o[7][r]};
    }
    if (g == 0) {
      dst[kD] = st.m_off;
      dst[kD + 1] = l;
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
      m = mrg[(w * MC + h) * kMergeStride + kD];
      lw = mrg[(w * MC + h) * kMergeStride + kD + 1];
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
  for (int idx = tid; idx < NC * kD; idx += NT) {
    const int h = idx / kD, j = idx % kD;
    float num = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) num = fmaf(fw[h * 16 + wv], mrg[(wv * MC + h) * kMergeStride + j], num);
    const float den = dh[h];
    if (finish) {
      vB[idx] = den > 0.f ? num / den * a.inv_sqrt_d : 0.f;
    } else {
      const int64_t pidx = out_row(h) * a.n_split + split;
      a.acc[pidx * kD + j] = num;
      if (j == 0) {
        a.ml[pidx * 2] = Mh[h];
        a.ml[pidx * 2 + 1] = den;
      }
    }
  }
  if (finish) {
    __syncthreads();   // o' is complete in vB; the merge area takes the partial sums
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
      a.out[out_row(h) * kD + i] = r;
    }
  }
}

// ---------------------------------------------------------------- combine --

// Workgroup (kv, b, chunk): merge the context-chunk partials of the G query
// heads of KV head kv (every workgroup of the KV head merges all 128
// coordinates), then output coordinates 32*chunk .. 32*chunk+31 of
// o = Pi_V^T o', with those 32 columns of Pi_V staged in LDS. The merge first
// takes each head's largest chunk maximum M, then sums the chunks in chunk
// order with weights 2^(m - M) kept in LDS (blocks of kCombineBlock chunks),
// so the loads of a thread's chunk partials are independent of each other.
constexpr int kCombineBlock = 256;

__global__ __launch_bounds__(256) void combine_kernel(const float* ml, const float* acc, const float* rotV,
                                                       float* out, int H_q, int G, int n_split, float inv_sqrt_d) {
  __shared__ __align__(16) float colv[kD * 32];
  __shared__ __align__(16) float ov[16 * kD];
  __shared__ float wsp[16 * kCombineBlock];
  __shared__ float Mh[16], dh[16];
  const int kv = blockIdx.x, b = blockIdx.y, chunk = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t bh0 = (int64_t)b * H_q + (int64_t)kv * G;
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
  // per-head maximum of the chunk maxima: wavefront w takes heads w, w + 4, ...
  for (int h = wave; h < G; h += 4) {
    const float* mlb = ml + (bh0 + h) * n_split * 2;
    float M = -INFINITY;
    for (int sp = lane; sp < n_split; sp += 64) M = fmaxf(M, mlb[2 * sp]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m));
    if (lane == 0) Mh[h] = M;
  }
  __syncthreads();

  constexpr int PER = 16 * kD / 256;   // (head, coordinate) pairs per thread, for G <= 16
  float num[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) num[k] = 0.f;
  float den = 0.f;   // thread h < G: denominator of head h
  for (int base = 0; base < n_split; base += kCombineBlock) {
    const int nb = min(kCombineBlock, n_split - base);
    for (int e = tid; e < G * kCombineBlock; e += 256) {
      const int h = e / kCombineBlock, sp = e % kCombineBlock;
      float w = 0.f;
      if (sp < nb) {
        const float m = ml[((bh0 + h) * n_split + base + sp) * 2];
        w = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - Mh[h]);
      }
      wsp[e] = w;
    }
    __syncthreads();
    if (tid < G) {
      const float* mlb = ml + ((bh0 + tid) * n_split + base) * 2;
#pragma unroll 8
      for (int sp = 0; sp < nb; ++sp) den = fmaf(wsp[tid * kCombineBlock + sp], mlb[2 * sp + 1], den);
      dh[tid] = den;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = tid + 256 * k;
      if (idx < G * kD) {
        const int h = idx / kD, j = idx % kD;
        const float* ab = acc + ((bh0 + h) * n_split + base) * kD + j;
        const float* wh = wsp + h * kCombineBlock;
        float x = num[k];
#pragma unroll 8
        for (int sp = 0; sp < nb; ++sp) x = fmaf(wh[sp], ab[(int64_t)sp * kD], x);
        num[k] = x;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = tid + 256 * k;
    if (idx < G * kD) {
      const float d = dh[idx / kD];
      ov[idx] = d > 0.f ? num[k] / d * inv_sqrt_d : 0.f;
    }
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
  dim3 grid((unsigned)p.n_split, (unsigned)p.H_kv, (unsigned)(p.B * p.nqt));
  if (sa.kpm.table != nullptr || sa.vpm.table != nullptr)
    hipLaunchKernelGGL((decode_scan_kernel<KB, VB, QJL, WIDE, 1>), grid, dim3(64 * scan_waves<QJL, WIDE>()), 0,
                       stream, sa);
  else
    hipLaunchKernelGGL((decode_scan_kernel<KB, VB, QJL, WIDE, 0>), grid, dim3(64 * scan_waves<QJL, WIDE>()), 0,
                       stream, sa);
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
  float* ml = (float*)(base + p.off_ml);
  float* acc = (float*)(base + p.off_acc);
  const float inv_sqrt_d = 1.0f / sqrtf((float)kD);

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
  sa.wave_chunk = p.chunk / ((p.qjl || p.wide) ? 8 : kCommonWaves);
  // the query operand carries log2(e) * scale / sqrt(d) (scores in the log2
  // domain); the QJL part log2(e) * scale * sqrt(pi/2) / d
  sa.sc1 = scale * kLog2e * inv_sqrt_d;
  sa.sc2 = scale * kLog2e * sqrtf((float)M_PI / 2.0f) / (float)kD;
  sa.inv_sqrt_d = inv_sqrt_d;
  for (int i = 0; i < 16; ++i) {
    sa.kc[i] = i < (1 << k->bits) ? k->centroids[i] : 0.f;
    sa.vc[i] = i < (1 << v->bits) ? v->centroids[i] : 0.f;
  }
  hipError_t err;
  switch (k->bits) {
    case 2: err = dispatch_vb<2>(v->bits, p, sa, stream); break;
    case 3: err = dispatch_vb<3>(v->bits, p, sa, stream); break;
    default: err = dispatch_vb<4>(v->bits, p, sa, stream); break;
  }
  if (err != hipSuccess || p.n_split == 1) return err;

  // the combine sees B * M query rows of H_q heads
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)p.H_kv, (unsigned)(p.B * p.M), kD / 32), dim3(256), 0, stream, ml, acc,
                     v->rot, out, (int)p.H_q, p.G, p.n_split, inv_sqrt_d);
  return hipGetLastError();
}

}  // namespace tq
