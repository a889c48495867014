// Shared device pieces of the kernels that scan the packed cache (decode,
// chunked and dense prefill attention): the codebook lookup table in LDS and
// the lookups that turn packed codes into float16 MFMA operands, the per-step
// loads of code words and norms through buffer resources, and the paged
// block-table addressing.
#pragma once

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
// the last step of a decode that appended its token in the prologue: device
// scope (sc1), so the read misses the compute unit's vector L1 and sees the
// words just written through it
constexpr int kFreshAux = kStreamAux | 16;
constexpr int kLutShift = 5;             // log2(kLutRep)
// Bound of the value-norm exponent (keeps the fp32 softmax denominator of a
// wavefront far from overflow: at most 2^(60 + 2 - kShift) per token).
constexpr int kNormExpClamp = 60;

__device__ inline float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

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

// A compile-time flag passed to generic lambdas.
template <int V>
struct IntConst {
  static constexpr int value = V;
};

// f(IntConst<I>()) for I = I0 .. N-1, unrolled at compile time.
template <int I0, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < N) {
    f(IntConst<I0>());
    static_for<I0 + 1, N>(f);
  }
}

// Tile geometry of head dimension D (64, 128 or 256). QK MFMA: lane group g
// (lane / 16) holds D/4 consecutive coordinates of its token (its key slice),
// D/32 MFMAs of 32 coordinates each per row block. PV MFMA: lane row i
// (lane % 16) holds D/16 consecutive coordinates of the 8 tokens of block g
// (its value slice), one MFMA per coordinate of the slice.
template <int D>
struct Geom {
  static_assert(D == 64 || D == 128 || D == 256, "head dimension");
  static constexpr int NKK = D / 32;   // QK MFMAs per row block
  static constexpr int CV = D / 16;    // PV MFMAs (coordinates per value slice)
};
// Words of a key record (one token) and of a value block record (8 tokens).
template <int KB, int D>
constexpr int key_record_words() { return D * KB / 32; }
template <int VB, int D>
constexpr int value_block_words() { return D * VB / 4; }
// Bit offset of lane group g's key slice in the record; a slice that does not
// start on a word (d = 64, 3 bits) is read as the two words that hold it and
// aligned in registers.
template <int KB, int D>
constexpr bool key_slice_shifted() { return (D / 4 * KB) % 32 != 0; }
template <int KB, int D>
constexpr int key_slice_words() { return (D / 4 * KB) / 32 + (key_slice_shifted<KB, D>() ? 1 : 0); }
template <int VB, int D>
constexpr int value_slice_words() { return D / 16 * VB / 4; }

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

// A operand of the QK MFMA for step KK: coordinates (D/4)g + 8KK + 0..7 of the
// lane's token, from the lane's key slice (coordinates (D/4)g .. (D/4)g + D/4 - 1).
template <int KB, int KK, int D = 128>
__device__ inline half8 key_operand(const uint32_t* w, const char* lut, uint32_t (&r)[4]) {
  return levels8<KB, key_slice_words<KB, D>(), 8 * KB * KK, 0>(w, lut, r);
}

// A operand of the PV MFMA for coordinate NB of the value slice: value codes
// of the 8 tokens of the lane's block at coordinate (D/16)i + NB (i = lane %
// 16), from the lane's slice of the block record (coordinates (D/16)i ..).
template <int VB, int NB, int D = 128>
__device__ inline half8 value_operand(const uint32_t* w, const char* lut, uint32_t (&r)[4]) {
  return levels8<VB, value_slice_words<VB, D>(), 8 * VB * NB, 128>(w, lut, r);
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
// (Row block m = 1 sits 4 tokens after row block 0; that distance travels in
// the scalar offset, so no second per-lane register is kept.)
struct LaneOffsets {
  uint32_t k;        // key record slice of MFMA row block 0
  uint32_t s;        // QJL sign word of MFMA row block 0
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
template <int KB, int VB, int QJL, int WIDE, int D = 128>
struct StepData {
  uint32_t kw[2][key_slice_words<KB, D>()];
  uint32_t sw[2];
  uint32_t vw[value_slice_words<VB, D>()];
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

// N words at per-lane offset voff plus scalar offset soff. A load split in two
// puts the second part's distance in the scalar offset when the per-lane
// offset needs no range check (RC false), else in the per-lane offset (the
// hardware range-checks only that one).
template <int N, bool RC = false, int AUX = kStreamAux>
__device__ inline void bload_words_s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* w) {
  if constexpr (N == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX);
  } else if constexpr (N == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (N == 3) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, AUX);
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  } else if constexpr (N == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (N == 6) {
    bload_words_s<3, false, AUX>(r, voff, soff, w);
    bload_words_s<3, false, AUX>(r, RC ? voff + 12u : voff, RC ? soff : soff + 12u, w + 3);
  } else {
    static_assert(N == 8 || N == 12 || N == 16, "unsupported word count");
    bload_words_s<4, false, AUX>(r, voff, soff, w);
    bload_words_s<N - 4, RC, AUX>(r, RC ? voff + 16u : voff, RC ? soff : soff + 16u, w + 4);
  }
}

// Waits until the loads of d have landed (an empty asm that reads every word:
// the compiler places the counter wait before it).
template <int KB, int VB, int QJL, int WIDE, int D>
__device__ inline void wait_step(const StepData<KB, VB, QJL, WIDE, D>& d) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int k = 0; k < key_slice_words<KB, D>(); ++k) asm volatile("" ::"v"(d.kw[m][k]));
    if constexpr (QJL) asm volatile("" ::"v"(d.sw[m]));
  }
#pragma unroll
  for (int k = 0; k < value_slice_words<VB, D>(); ++k) asm volatile("" ::"v"(d.vw[k]));
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
template <bool CHECKED, int AUX = kStreamAux, int KB, int VB, int QJL, int WIDE, int D>
__device__ inline void load_step(StepData<KB, VB, QJL, WIDE, D>& d, const Streams& s, const LaneOffsets& lo,
                                 uint32_t rk, uint32_t rv) {
  constexpr int KW = key_record_words<KB, D>(), VBW = value_block_words<VB, D>();
  constexpr int KSW = key_slice_words<KB, D>(), VSW = value_slice_words<VB, D>();
  // wave-uniform; readfirstlane keeps the step offsets in scalar registers
  rk = __builtin_amdgcn_readfirstlane(rk);
  rv = __builtin_amdgcn_readfirstlane(rv);
  const uint32_t ok = rk * (KW * 4u), os = rk * 16u, ov = (rv / 8u) * (VBW * 4u), onk = rk * 4u, onv = rv * 4u;
  // (TQ_OFF: the scalar offset of a load; TQ_VOF: its per-lane offset)
#define TQ_OFF(o) (CHECKED ? 0u : (o))
#define TQ_VOF(v, o) (CHECKED ? (v) + (o) : (v))
  // row block 1 is 4 tokens (4 records, 4 sign rows) after row block 0
  constexpr uint32_t dk1 = 4u * KW * 4u, ds1 = 4u * 16u;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t vk = CHECKED ? lo.k + ok + (m ? dk1 : 0u) : lo.k;
    const uint32_t sk = CHECKED ? 0u : ok + (m ? dk1 : 0u);
    bload_words_s<KSW, CHECKED, AUX>(s.rk, vk, sk, d.kw[m]);
    if constexpr (QJL) {
      const uint32_t vs = CHECKED ? lo.s + os + (m ? ds1 : 0u) : lo.s;
      const uint32_t ss = CHECKED ? 0u : os + (m ? ds1 : 0u);
      d.sw[m] = __builtin_amdgcn_raw_buffer_load_b32(s.rs, vs, ss, AUX);
    }
  }
  bload_words_s<VSW, CHECKED, AUX>(s.rv, TQ_VOF(lo.v, ov), TQ_OFF(ov), d.vw);
  d.nm.kn = as_float(__builtin_amdgcn_raw_buffer_load_b32(s.rkn, TQ_VOF(lo.n, onk), TQ_OFF(onk), AUX));
  d.nm.vn = as_float(__builtin_amdgcn_raw_buffer_load_b32(s.rvn, TQ_VOF(lo.n, onv), TQ_OFF(onv), AUX));
  if constexpr (QJL)
    d.nm.kg = as_float(__builtin_amdgcn_raw_buffer_load_b32(s.rg, TQ_VOF(lo.n, onk), TQ_OFF(onk), AUX));
#undef TQ_OFF
#undef TQ_VOF
}

}  // namespace

}  // namespace tq
