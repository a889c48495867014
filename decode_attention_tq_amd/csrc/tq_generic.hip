// Head dimensions other than 128 (64 and 256): quantize (bulk and append),
// dequantize and decode attention with the same method and the same packed
// layouts as the d = 128 kernels (ai-accelerate.xyz TurboQuant article,
// section "TurboQuantの仕組み", step 1: rotate, store the norm, Lloyd-Max code
// per coordinate; decode in the rotated domain), written generically in d.
//
// These kernels favour plainness over speed: the rotations are float32 FMAs
// with the rows of the matrices read from memory (L2-resident), and the decode
// runs one workgroup per (row, KV head) over the whole context. The d = 128
// path (MFMA rotations, codebook lookups from LDS tables, split contexts)
// stays the fast one; QJL keys and the chunked prefill exist for d = 128 only.
//
// Layouts (the same rules as d = 128, with W = d * bits / 32 words per token):
//   keys:   token row r holds code j at bits [bits*j, bits*j + bits) of words
//           codes[r*W ...], LSB first;
//   values: 8-token blocks; block b starts at the token row r0 of its first
//           token, and coordinate group g (coordinates 4g .. 4g+3) holds the
//           code of (coordinate 4g + jj, token i) at bits bits*(8jj + i) of its
//           bits words codes[r0*W + g*bits ...].
#include <math.h>

#include "tq_append.h"
#include "tq_codec.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

__device__ inline float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Code `bits` wide at bit q of a little-endian word stream.
__device__ inline uint32_t code_at(const uint32_t* w, int q, int bits) {
  const int wi = q >> 5, off = q & 31;
  uint32_t v = w[wi] >> off;
  if (off + bits > 32) v |= w[wi + 1] << (32 - off);
  return v & ((1u << bits) - 1u);
}

// Lloyd-Max cell of z: the number of thresholds (ascending, in the kernel
// arguments) that z reaches; counting keeps every threshold in a register.
template <int BITS>
__device__ inline int cell_count(float z, const float* thr) {
  int n = 0;
#pragma unroll
  for (int i = 0; i < (1 << BITS) - 1; ++i) n += z >= thr[i] ? 1 : 0;
  return n;
}

// Max (or sum) over the D threads of a workgroup, for 8 values per thread at
// once; every thread gets the 8 results.
template <int D, bool MAX>
__device__ inline void block_reduce8(float (&v)[8], float (*part)[D / 64 > 0 ? D / 64 : 1]) {
  constexpr int NW = D / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float o = __shfl_xor(v[i], m);
      v[i] = MAX ? fmaxf(v[i], o) : v[i] + o;
    }
    if (lane == 0) part[i][wv] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float r = part[i][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = MAX ? fmaxf(r, part[i][w]) : r + part[i][w];
    v[i] = r;
  }
  __syncthreads();
}

// Quantize the tokens of one 8-token block of one (row, head); thread j owns
// coordinate j. Bulk mode (ctx_lens == nullptr): workgroup blk0 + blockIdx.x =
// (row*H_kv + head, block) over the slots [t_base, t_base + nslot), input token t at
// x[b][t - t_offset][h]. Append mode: workgroup = (row*H_kv + head), the one
// token x[b][0][h] goes to token clamp(ctx_lens[b], 0, T_all) - 1 (none when
// that is -1). Tokens of the block outside the written set keep their bits.
template <int D, int BITS, int ROLE, int XF32>
__global__ __launch_bounds__(D, D == 256 ? 2 : 4) void quantize_generic_kernel(QuantArgs a, const int32_t* ctx_lens,
                                                                         int64_t T_all, int64_t blk0) {
  constexpr int W = D * BITS / 32;
  __shared__ float xs[8][D];
  __shared__ unsigned char cs[8][D];
  __shared__ float part[8][D / 64];
  const int j = threadIdx.x;
  int64_t bh, tb;
  int written = 0;   // bit i: token tb + i is written
  if (ctx_lens == nullptr) {
    const int64_t nb = a.nslot / 8, blk = blk0 + blockIdx.x;
    bh = blk / nb;
    tb = a.t_base + 8 * (blk % nb);
    for (int i = 0; i < 8; ++i) {
      const int64_t t = tb + i;
      if (t >= a.t_offset && t < a.t_offset + a.T) written |= 1 << i;
    }
  } else {
    bh = blockIdx.x;
    int64_t c = ctx_lens[bh / a.H_kv];
    c = c < 0 ? 0 : (c > T_all ? T_all : c);
    if (c == 0) return;   // (workgroup-uniform)
    tb = (c - 1) & ~(int64_t)7;
    written = 1 << (c - 1 - tb);
  }
  const int64_t b = bh / a.H_kv, h = bh % a.H_kv;

  // ---- input (zeros for tokens not written)
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = 0.f;
    if ((written >> i) & 1) {
      const int64_t tt = ctx_lens == nullptr ? tb + i - a.t_offset : 0;
      const int64_t off = b * a.sb + tt * a.st + h * a.sh + j;
      v[i] = XF32 ? ((const float*)a.x)[off] : bf16_value(((const uint16_t*)a.x)[off]);
    }
  }
  // ---- a power of two per vector puts its largest entry in [1/2, 1), so the
  // squares and the rotation neither under- nor overflow
  float mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mx[i] = fabsf(v[i]);
  block_reduce8<D, true>(mx, part);
  int sexp[8];
  float ss[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sexp[i] = mx[i] > 0.f ? -__builtin_amdgcn_frexp_expf(mx[i]) : 0;
    v[i] = ldexpf(v[i], sexp[i]);
    xs[i][j] = v[i];
    ss[i] = v[i] * v[i];
  }
  block_reduce8<D, false>(ss, part);   // (its barriers also publish xs)

  // ---- y = Pi x (row j of Pi against each token), z = y sqrt(d) / |x|, code
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = 0.f;
  const float4* prow = (const float4*)(a.rot + (int64_t)j * D);
#pragma unroll 4
  for (int k4 = 0; k4 < D / 4; ++k4) {
    const float4 p = prow[k4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y[i] = fmaf(p.x, xs[i][4 * k4], y[i]);
      y[i] = fmaf(p.y, xs[i][4 * k4 + 1], y[i]);
      y[i] = fmaf(p.z, xs[i][4 * k4 + 2], y[i]);
      y[i] = fmaf(p.w, xs[i][4 * k4 + 3], y[i]);
    }
  }
  const float sqrt_d = sqrtf((float)D);
  float ns[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ns[i] = sqrtf(ss[i]);
    const float z = ns[i] > 0.f ? y[i] * (sqrt_d / ns[i]) : 0.f;
    cs[i][j] = (unsigned char)cell_count<BITS>(z, a.thr);
  }
  __syncthreads();

  // ---- pack and store
  if constexpr (ROLE == TQ_KEYS) {
    if (j < 8 * W) {
      const int i = j / W, w = j % W;
      if ((written >> i) & 1) {
        uint32_t word = 0u;
        for (int p = 0; p < 32; ++p) {
          const int q = 32 * w + p;
          word |= (uint32_t)((cs[i][q / BITS] >> (q % BITS)) & 1) << p;
        }
        const int64_t row = tok_row(a.pm, a.H_kv, a.T_cap, bh, tb + i);
        if (row >= 0) a.codes[row * W + w] = word;
      }
    }
  } else {
    if (j < 8 * W) {
      const int g = j / BITS, ws = j % BITS;
      uint32_t word = 0u, keep = 0u;
      for (int p = 0; p < 32; ++p) {
        const int q = 32 * ws + p, code = q / BITS;
        const int jj = code >> 3, ti = code & 7;
        if ((written >> ti) & 1) word |= (uint32_t)((cs[ti][4 * g + jj] >> (q % BITS)) & 1) << p;
        else keep |= 1u << p;
      }
      const int64_t row0 = tok_row(a.pm, a.H_kv, a.T_cap, bh, tb);
      if (row0 >= 0) {
        uint32_t* dst = a.codes + row0 * W + j;
        *dst = keep == 0u ? word : ((*dst & keep) | word);
      }
    }
  }
  if (j == 0) {   // (the norms are the same in every thread)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((written >> i) & 1) {
        const int64_t row = tok_row(a.pm, a.H_kv, a.T_cap, bh, tb + i);
        if (row >= 0) a.norms[row] = ldexpf(ns[i], -sexp[i]);
      }
    }
  }
}

// ------------------------------------ bulk quantize, bfloat16 input, on MFMA --
//
// y = Pi x for 32 vectors per wavefront on v_mfma_f32_32x32x16_f16: A = the
// vector in float16 (the bfloat16 words scaled by a power of two that puts the
// largest entry in [2^13, 2^14): exact, 8 significant bits in float16's 11),
// B = a 32-row output block of Pi split into float16 hi + lo (~22 significant
// bits; the hi and lo products accumulate apart). The workgroup stages the
// output blocks in LDS in fragment order, two in turn (the next block's rows
// load while the current one is used), and packs each block's 32 coordinates
// as soon as their codes are known: a key record's words 3jb .. (bits) and a
// value block's coordinate groups 8jb .. 8jb+7 are contiguous, so the codes
// need 32 bytes per vector of LDS, not d.

typedef float gfloatx16 __attribute__((ext_vector_type(16)));

__device__ inline gfloatx16 mfma_f16_32(half8 a, half8 b, gfloatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Wavefronts per workgroup (d = 256: 4, so that two workgroups share a
// compute unit's LDS).
template <int D>
constexpr int qm_waves() { return D > 128 ? 4 : 8; }

template <int D, int BITS, int ROLE>
__global__ __launch_bounds__(64 * qm_waves<D>()) void quantize_mfma_kernel(QuantArgs a, int64_t total,
                                                                            int64_t tile0) {
  constexpr int NW = qm_waves<D>(), NT = 64 * NW, TV = 32 * NW;   // vectors of a workgroup tile
  constexpr int NKS = D / 16, NJB = D / 32;
  constexpr int W = D * BITS / 32;            // words of a key record
  constexpr int FR = 2 * NKS * 64;            // 16-byte fragments of one staged output block (hi, lo)
  constexpr int SPT = (NKS * 64 + NT - 1) / NT;   // staged (ks, lane) items per thread
  __shared__ half8 pib[2][FR];
  __shared__ unsigned char cs[2][TV][32];     // codes of one output block, two blocks in turn
  __shared__ float vscale[TV], vnorm[TV];
  __shared__ int64_t vrow[TV];                // token row of each vector (-1: not written)
  __shared__ int64_t brow[TV / 8];            // token row of each 8-token block's first token
  __shared__ uint32_t bmask[TV / 8];          // tokens of the block that are written (bit i)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t s0 = (tile0 + blockIdx.x) * TV;   // first (row * H_kv + head) * nslot + slot of the tile
  const int64_t t_hi = a.t_offset + a.T;
  auto written = [&](int64_t sl, int64_t* bh, int64_t* t) -> bool {
    if (sl >= total) return false;
    *bh = sl / a.nslot;
    *t = a.t_base + sl % a.nslot;
    return *t >= a.t_offset && *t < t_hi;
  };

  // ---- this lane's vector (i = lane % 32 of the wavefront's 32) as float16 A operands
  half8 xa[NKS];
  {
    const int v = 32 * wave + (lane & 31), kq = lane >> 5;
    int64_t bh = 0, t = 0;
    const bool wr = written(s0 + v, &bh, &t);
    const int64_t off = wr ? (bh / a.H_kv) * a.sb + (t - a.t_offset) * a.st + (bh % a.H_kv) * a.sh + 8 * kq : 0;
    const uint16_t* xp = (const uint16_t*)a.x + off;
    u32x4 raw[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) raw[ks] = wr ? *(const u32x4*)(xp + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
    float mx = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mx = fmaxf(mx, fabsf(__uint_as_float(raw[ks][q] << 16)));
        mx = fmaxf(mx, fabsf(__uint_as_float(raw[ks][q] & 0xFFFF0000u)));
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const int e = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) : 0;
    // squared norm of x * 2^-e in pairwise partial sums; the operand is x * 2^(14 - e)
    float ps[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ps[k] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = ldexpf(__uint_as_float(raw[ks][q] << 16), -e);
        const float hi = ldexpf(__uint_as_float(raw[ks][q] & 0xFFFF0000u), -e);
        ps[2 * q] = fmaf(lo, lo, ps[2 * q]);
        ps[2 * q + 1] = fmaf(hi, hi, ps[2 * q + 1]);
        xa[ks][2 * q] = (_Float16)(lo * 16384.f);
        xa[ks][2 * q + 1] = (_Float16)(hi * 16384.f);
      }
    float ss = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
    ss += __shfl_xor(ss, 32);
    if (kq == 0) {
      const float r = sqrtf(ss);
      // z = y * sqrt(d) / |x|, with y and |x| both carrying 2^(14 - e) and 2^-e
      vscale[v] = ss > 0.f ? ldexpf(sqrtf((float)D) / r, -14) : 0.f;
      vnorm[v] = ldexpf(r, e);
      vrow[v] = wr ? tok_row(a.pm, a.H_kv, a.T_cap, bh, t) : -1;
    } else if ((v & 7) == 0) {
      // (lane 32 + i of a block's first vector: the block's first row and written tokens)
      const int64_t sb0 = s0 + v;
      uint32_t m = 0;
      int64_t r0 = -1;
      if (sb0 < total) {
        const int64_t bb = sb0 / a.nslot, tb = a.t_base + sb0 % a.nslot;
        for (int i = 0; i < 8; ++i)
          if (tb + i >= a.t_offset && tb + i < t_hi) m |= 1u << i;
        r0 = tok_row(a.pm, a.H_kv, a.T_cap, bb, tb);
      }
      bmask[v >> 3] = m;
      brow[v >> 3] = r0;
    }
  }

  // ---- staging of output block jb (rows 32jb .. 32jb+31 of Pi) in fragment order
  float4 st[SPT][2];
  auto stage_load = [&](int jb) {
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int item = tid + u * NT;
      if (item < NKS * 64) {
        const int ks = item >> 6, ln = item & 63;
        const float4* src = (const float4*)(a.rot + (int64_t)(32 * jb + (ln & 31)) * D + 16 * ks + 8 * (ln >> 5));
        st[u][0] = src[0];
        st[u][1] = src[1];
      }
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int item = tid + u * NT;
      if (item < NKS * 64) {
        const float x[8] = {st[u][0].x, st[u][0].y, st[u][0].z, st[u][0].w,
                            st[u][1].x, st[u][1].y, st[u][1].z, st[u][1].w};
        half8 hi, lo;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          hi[k] = (_Float16)x[k];
          lo[k] = (_Float16)(x[k] - (float)hi[k]);
        }
        const int ks = item >> 6, ln = item & 63;
        pib[buf][(0 * NKS + ks) * 64 + ln] = hi;
        pib[buf][(1 * NKS + ks) * 64 + ln] = lo;
      }
    }
  };
  stage_load(0);
  stage_store(0);
  __syncthreads();

  // scales of the 16 vectors whose outputs this lane holds: rows 8q + 4(lane/32) + r
  float sc[16];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[4 * q + r] = vscale[32 * wave + 8 * q + 4 * (lane >> 5) + r];

  for (int jb = 0; jb < NJB; ++jb) {
    if (jb + 1 < NJB) stage_load(jb + 1);
    const half8* P = pib[jb & 1];
    gfloatx16 ah = {}, al = {};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      ah = mfma_f16_32(xa[ks], P[(0 * NKS + ks) * 64 + lane], ah);
      al = mfma_f16_32(xa[ks], P[(1 * NKS + ks) * 64 + lane], al);
    }
    // output (vector 8q + 4(lane/32) + r, coordinate 32jb + lane % 32) in element r + 4q
    unsigned char (*cb)[32] = cs[jb & 1];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float z = (ah[4 * q + r] + al[4 * q + r]) * sc[4 * q + r];
        cb[32 * wave + 8 * q + 4 * (lane >> 5) + r][lane & 31] = (unsigned char)cell_count<BITS>(z, a.thr);
      }
    if (jb + 1 < NJB) stage_store((jb + 1) & 1);
    __syncthreads();

    // ---- pack the 32 coordinates of block jb for every vector of the tile
    if constexpr (ROLE == TQ_KEYS) {
      // words BITS*jb .. BITS*jb + BITS - 1 of each key record
      for (int e = tid; e < TV * BITS; e += NT) {
        const int v = e / BITS, w = e % BITS;
        const int64_t row = vrow[v];
        if (row < 0) continue;
        const int q0 = 32 * w, c0 = q0 / BITS, c1 = (q0 + 31) / BITS;
        uint64_t acc = 0;
        for (int c = c0; c <= c1; ++c) {
          const int sh = BITS * c - q0;
          const uint64_t val = cb[v][c];
          acc |= sh >= 0 ? val << sh : val >> (-sh);
        }
        a.codes[row * W + BITS * jb + w] = (uint32_t)acc;
      }
    } else {
      // coordinate groups 8jb .. 8jb+7 of each 8-token block: group g holds the
      // code of (coordinate 4g + jj, token i) at bits BITS * (8jj + i) of its words
      for (int e = tid; e < (TV / 8) * 8 * BITS; e += NT) {
        const int blk = e / (8 * BITS), j8 = e % (8 * BITS), gl = j8 / BITS, ws = j8 % BITS;
        const uint32_t wm = bmask[blk];
        const int64_t row0 = brow[blk];
        if (wm == 0u || row0 < 0) continue;
        const int q0 = 32 * ws, c0 = q0 / BITS, c1 = (q0 + 31) / BITS;
        uint64_t acc = 0, keep = 0;
        for (int ci = c0; ci <= c1; ++ci) {
          const int sh = BITS * ci - q0, ti = ci & 7, jj = ci >> 3;
          const bool wr = (wm >> ti) & 1u;
          const uint64_t val = wr ? (uint64_t)cb[8 * blk + ti][4 * gl + jj] : 0u;
          const uint64_t m = wr ? 0u : (uint64_t)((1u << BITS) - 1u);
          acc |= sh >= 0 ? val << sh : val >> (-sh);
          keep |= sh >= 0 ? m << sh : m >> (-sh);
        }
        uint32_t* dst = a.codes + row0 * W + 8 * BITS * jb + j8;
        const uint32_t kp = (uint32_t)keep, word = (uint32_t)acc;
        *dst = kp == 0u ? word : ((*dst & kp) | word);
      }
    }
  }
  for (int v = tid; v < TV; v += NT) {
    const int64_t row = vrow[v];
    if (row >= 0) a.norms[row] = vnorm[v];
  }
}

struct GenericDequantArgs {
  const uint32_t* codes;
  const float* norms;
  const float* rot;
  float* out;   // [B][H_kv][t1 - t0][D]
  int64_t H_kv, T_cap, t0, t1;
  float cent[16];
  PageMap pm;
};

// x_hat = n Pi^T (c[code] / sqrt(d)) for 8 tokens of one (row, head); thread j
// forms coordinate j from the columns of Pi (its rows, read coalesced).
template <int D, int BITS, int ROLE>
__global__ __launch_bounds__(D, 4) void dequantize_generic_kernel(GenericDequantArgs a, int64_t blk0) {
  constexpr int W = D * BITS / 32;
  __shared__ float cv[8][D];
  const int j = threadIdx.x;
  const int64_t n = a.t1 - a.t0, nb = (n + 7) / 8, blk = blk0 + blockIdx.x;
  const int64_t bh = blk / nb, t0 = a.t0 + 8 * (blk % nb);
  const float inv_sqrt_d = 1.f / sqrtf((float)D);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = t0 + i;
    float c = 0.f;
    if (t < a.t1) {
      uint32_t code;
      if constexpr (ROLE == TQ_KEYS) {
        const int64_t row = tok_row(a.pm, a.H_kv, a.T_cap, bh, t);
        code = row >= 0 ? code_at(a.codes + row * W, BITS * j, BITS) : 0u;
        c = row >= 0 ? a.cent[code] * a.norms[row] * inv_sqrt_d : 0.f;
      } else {
        const int64_t row0 = tok_row(a.pm, a.H_kv, a.T_cap, bh, t & ~(int64_t)7);
        const int64_t row = tok_row(a.pm, a.H_kv, a.T_cap, bh, t);
        const int g = j >> 2, jj = j & 3, ti = (int)(t & 7);
        code = row0 >= 0 ? code_at(a.codes + row0 * W + g * BITS, BITS * (8 * jj + ti), BITS) : 0u;
        c = row0 >= 0 && row >= 0 ? a.cent[code] * a.norms[row] * inv_sqrt_d : 0.f;
      }
    }
    cv[i][j] = c;
  }
  __syncthreads();
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  for (int c = 0; c < D; ++c) {
    const float p = a.rot[(int64_t)c * D + j];   // Pi[c][j]
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = fmaf(p, cv[i][c], o[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = t0 + i;
    if (t < a.t1) a.out[(bh * n + (t - a.t0)) * D + j] = o[i];
  }
}

struct GenericDecodeArgs {
  const uint32_t* kcodes;
  const float* knorms;
  const float* rotK;
  const uint32_t* vcodes;
  const float* vnorms;
  const float* rotV;
  float kcent[16], vcent[16];
  PageMap kpm, vpm;
  int64_t H_kv, kT_cap, vT_cap;
  const void* q;   // [B][H_q][D]
  int q_f32;
  int64_t H_q;
  int G;
  const int32_t* ctx_lens;
  int64_t T;
  float scale;
  float* out;      // [B][H_q][D]
};

constexpr int kGenStep = 32;    // tokens per step of the generic decode
constexpr int kGenThreads = 256;
constexpr int kGenMaxG = 16;

// Decode attention of the G query heads of one (row, KV head) over its whole
// context, in the rotated domain: q' = Pi_K q once; per 32-token step the key
// levels of the step go to LDS, scores = scale * n_K / sqrt(d) * q'.c, online
// softmax per head, acc' += p * n_V / sqrt(d) * c_V (thread j: coordinate j of
// every head); at the end o = Pi_V^T (acc' / l).
template <int D, int KB, int VB>
__global__ __launch_bounds__(kGenThreads) void decode_generic_kernel(GenericDecodeArgs a) {
  constexpr int KW = D * KB / 32, VW = D * VB / 32;
  // (rows padded by one float: the score loop reads down the columns)
  __shared__ float qr[kGenMaxG][D + 1];
  __shared__ float buf[kGenStep][D + 1];
  __shared__ float sc[kGenMaxG][kGenStep];
  __shared__ float tn[kGenStep];
  __shared__ float mh[kGenMaxG], lh[kGenMaxG], al[kGenMaxG];
  const int tid = threadIdx.x, G = a.G;
  const int64_t bh = blockIdx.x, b = bh / a.H_kv, kv = bh % a.H_kv;
  int64_t ctx = a.T;
  if (a.ctx_lens != nullptr) {
    const int64_t c = a.ctx_lens[b];
    ctx = c < 0 ? 0 : (c > a.T ? a.T : c);
  }
  const float inv_sqrt_d = 1.f / sqrtf((float)D);

  // ---- q' = Pi_K q, scaled by scale / sqrt(d) (the queries staged in buf)
  for (int idx = tid; idx < G * D; idx += kGenThreads) {
    const int h = idx / D, k = idx % D;
    const int64_t e = ((b * a.H_q + kv * G + h) * D) + k;
    buf[h][k] = a.q_f32 ? ((const float*)a.q)[e] : bf16_value(((const uint16_t*)a.q)[e]);
  }
  if (tid < kGenMaxG) {
    mh[tid] = -INFINITY;
    lh[tid] = 0.f;
  }
  __syncthreads();
  for (int jq = tid; jq < D; jq += kGenThreads) {
    float acc[kGenMaxG];
#pragma unroll
    for (int h = 0; h < kGenMaxG; ++h) acc[h] = 0.f;
    const float* prow = a.rotK + (int64_t)jq * D;
    for (int k = 0; k < D; ++k) {
      const float p = prow[k];
#pragma unroll
      for (int h = 0; h < kGenMaxG; ++h)
        if (h < G) acc[h] = fmaf(p, buf[h][k], acc[h]);
    }
#pragma unroll
    for (int h = 0; h < kGenMaxG; ++h)
      if (h < G) qr[h][jq] = acc[h] * (a.scale * inv_sqrt_d);
  }
  __syncthreads();

  // thread j < D accumulates coordinate j of every head
  float oacc[kGenMaxG];
#pragma unroll
  for (int h = 0; h < kGenMaxG; ++h) oacc[h] = 0.f;
  for (int64_t t0 = 0; t0 < ctx; t0 += kGenStep) {
    const int nt = (int)(ctx - t0 < kGenStep ? ctx - t0 : kGenStep);
    // key levels of the step, and the key norms
    for (int idx = tid; idx < nt * D; idx += kGenThreads) {
      const int i = idx / D, c = idx % D;
      const int64_t row = tok_row(a.kpm, a.H_kv, a.kT_cap, bh, t0 + i);
      buf[i][c] = row >= 0 ? a.kcent[code_at(a.kcodes + row * KW, KB * c, KB)] : 0.f;
      if (c == 0) tn[i] = row >= 0 ? a.knorms[row] : 0.f;
    }
    __syncthreads();
    for (int idx = tid; idx < G * kGenStep; idx += kGenThreads) {
      const int h = idx / kGenStep, i = idx % kGenStep;
      float s = -INFINITY;
      if (i < nt) {
        float dot = 0.f;
        for (int c = 0; c < D; ++c) dot = fmaf(qr[h][c], buf[i][c], dot);
        s = tn[i] * dot;
      }
      sc[h][i] = s;
    }
    __syncthreads();
    // online softmax per head
    if (tid < G) {
      const int h = tid;
      float m = mh[h];
      for (int i = 0; i < nt; ++i) m = fmaxf(m, sc[h][i]);
      const float alpha = mh[h] == -INFINITY ? 0.f : expf(mh[h] - m);
      float l = 0.f;
      for (int i = 0; i < kGenStep; ++i) {
        const float p = i < nt ? expf(sc[h][i] - m) : 0.f;
        sc[h][i] = p;
        l += p;
      }
      lh[h] = lh[h] * alpha + l;
      mh[h] = m;
      al[h] = alpha;
    }
    __syncthreads();
    // value levels of the step, times n_V / sqrt(d)
    for (int idx = tid; idx < nt * D; idx += kGenThreads) {
      const int i = idx / D, c = idx % D;
      const int64_t t = t0 + i;
      const int64_t row0 = tok_row(a.vpm, a.H_kv, a.vT_cap, bh, t & ~(int64_t)7);
      const int64_t row = tok_row(a.vpm, a.H_kv, a.vT_cap, bh, t);
      float cv = 0.f;
      if (row0 >= 0 && row >= 0) {
        const int g = c >> 2, jj = c & 3, ti = (int)(t & 7);
        cv = a.vcent[code_at(a.vcodes + row0 * VW + g * VB, VB * (8 * jj + ti), VB)] * a.vnorms[row] * inv_sqrt_d;
      }
      buf[i][c] = cv;
    }
    __syncthreads();
    if (tid < D) {
#pragma unroll
      for (int h = 0; h < kGenMaxG; ++h) {
        if (h < G) {
          float s = oacc[h] * al[h];
          for (int i = 0; i < nt; ++i) s = fmaf(sc[h][i], buf[i][tid], s);
          oacc[h] = s;
        }
      }
    }
    __syncthreads();
  }

  // ---- o = Pi_V^T (acc' / l)
  if (tid < D) {
#pragma unroll
    for (int h = 0; h < kGenMaxG; ++h)
      if (h < G) buf[h][tid] = lh[h] > 0.f ? oacc[h] / lh[h] : 0.f;
  }
  __syncthreads();
  for (int jo = tid; jo < D; jo += kGenThreads) {
    float o[kGenMaxG];
#pragma unroll
    for (int h = 0; h < kGenMaxG; ++h) o[h] = 0.f;
    for (int c = 0; c < D; ++c) {
      const float p = a.rotV[(int64_t)c * D + jo];   // Pi_V[c][jo]
#pragma unroll
      for (int h = 0; h < kGenMaxG; ++h)
        if (h < G) o[h] = fmaf(p, buf[h][c], o[h]);
    }
#pragma unroll
    for (int h = 0; h < kGenMaxG; ++h)
      if (h < G) a.out[(b * a.H_q + kv * G + h) * D + jo] = o[h];
  }
}

// Workgroups per launch of the one-block-per-workgroup kernels (larger grids
// go out as several launches).
constexpr int64_t kGenMaxGrid = (int64_t)1 << 30;

template <int D, int BITS, int ROLE>
hipError_t launch_qg(int xf32, const QuantArgs& qa, const int32_t* ctx_lens, int64_t T_all, int64_t blocks,
                     hipStream_t s) {
  for (int64_t b0 = 0; b0 < blocks; b0 += kGenMaxGrid) {
    const unsigned n = (unsigned)(blocks - b0 < kGenMaxGrid ? blocks - b0 : kGenMaxGrid);
    if (xf32)
      hipLaunchKernelGGL((quantize_generic_kernel<D, BITS, ROLE, 1>), dim3(n), dim3(D), 0, s, qa, ctx_lens, T_all,
                         b0);
    else
      hipLaunchKernelGGL((quantize_generic_kernel<D, BITS, ROLE, 0>), dim3(n), dim3(D), 0, s, qa, ctx_lens, T_all,
                         b0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D>
hipError_t dispatch_qg(int bits, int role, int xf32, const QuantArgs& qa, const int32_t* ctx_lens, int64_t T_all,
                       int64_t blocks, hipStream_t s) {
  const bool keys = role == TQ_KEYS;
  switch (bits) {
    case 2: return keys ? launch_qg<D, 2, TQ_KEYS>(xf32, qa, ctx_lens, T_all, blocks, s)
                        : launch_qg<D, 2, TQ_VALUES>(xf32, qa, ctx_lens, T_all, blocks, s);
    case 3: return keys ? launch_qg<D, 3, TQ_KEYS>(xf32, qa, ctx_lens, T_all, blocks, s)
                        : launch_qg<D, 3, TQ_VALUES>(xf32, qa, ctx_lens, T_all, blocks, s);
    default: return keys ? launch_qg<D, 4, TQ_KEYS>(xf32, qa, ctx_lens, T_all, blocks, s)
                         : launch_qg<D, 4, TQ_VALUES>(xf32, qa, ctx_lens, T_all, blocks, s);
  }
}

template <int D, int BITS, int ROLE>
hipError_t launch_dqg(const GenericDequantArgs& da, int64_t blocks, hipStream_t s) {
  for (int64_t b0 = 0; b0 < blocks; b0 += kGenMaxGrid) {
    const unsigned n = (unsigned)(blocks - b0 < kGenMaxGrid ? blocks - b0 : kGenMaxGrid);
    hipLaunchKernelGGL((dequantize_generic_kernel<D, BITS, ROLE>), dim3(n), dim3(D), 0, s, da, b0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D>
hipError_t dispatch_dqg(int bits, int role, const GenericDequantArgs& da, int64_t blocks, hipStream_t s) {
  const bool keys = role == TQ_KEYS;
  switch (bits) {
    case 2: return keys ? launch_dqg<D, 2, TQ_KEYS>(da, blocks, s) : launch_dqg<D, 2, TQ_VALUES>(da, blocks, s);
    case 3: return keys ? launch_dqg<D, 3, TQ_KEYS>(da, blocks, s) : launch_dqg<D, 3, TQ_VALUES>(da, blocks, s);
    default: return keys ? launch_dqg<D, 4, TQ_KEYS>(da, blocks, s) : launch_dqg<D, 4, TQ_VALUES>(da, blocks, s);
  }
}

template <int D, int KB>
hipError_t dispatch_decg_v(int vbits, const GenericDecodeArgs& ga, int64_t blocks, hipStream_t s) {
  switch (vbits) {
    case 2:
      hipLaunchKernelGGL((decode_generic_kernel<D, KB, 2>), dim3((unsigned)blocks), dim3(kGenThreads), 0, s, ga);
      break;
    case 3:
      hipLaunchKernelGGL((decode_generic_kernel<D, KB, 3>), dim3((unsigned)blocks), dim3(kGenThreads), 0, s, ga);
      break;
    default:
      hipLaunchKernelGGL((decode_generic_kernel<D, KB, 4>), dim3((unsigned)blocks), dim3(kGenThreads), 0, s, ga);
      break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_decg(int kbits, int vbits, const GenericDecodeArgs& ga, int64_t blocks, hipStream_t s) {
  switch (kbits) {
    case 2: return dispatch_decg_v<D, 2>(vbits, ga, blocks, s);
    case 3: return dispatch_decg_v<D, 3>(vbits, ga, blocks, s);
    default: return dispatch_decg_v<D, 4>(vbits, ga, blocks, s);
  }
}

template <int D, int BITS, int ROLE>
hipError_t launch_qm(const QuantArgs& qa, int64_t total, hipStream_t s) {
  constexpr int TV = 32 * qm_waves<D>();
  const int64_t tiles = (total + TV - 1) / TV;
  for (int64_t t0 = 0; t0 < tiles; t0 += kGenMaxGrid) {
    const unsigned n = (unsigned)(tiles - t0 < kGenMaxGrid ? tiles - t0 : kGenMaxGrid);
    hipLaunchKernelGGL((quantize_mfma_kernel<D, BITS, ROLE>), dim3(n), dim3(64 * qm_waves<D>()), 0, s, qa, total, t0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D>
hipError_t dispatch_qm(int bits, int role, const QuantArgs& qa, int64_t total, hipStream_t s) {
  const bool keys = role == TQ_KEYS;
  switch (bits) {
    case 2: return keys ? launch_qm<D, 2, TQ_KEYS>(qa, total, s) : launch_qm<D, 2, TQ_VALUES>(qa, total, s);
    case 3: return keys ? launch_qm<D, 3, TQ_KEYS>(qa, total, s) : launch_qm<D, 3, TQ_VALUES>(qa, total, s);
    default: return keys ? launch_qm<D, 4, TQ_KEYS>(qa, total, s) : launch_qm<D, 4, TQ_VALUES>(qa, total, s);
  }
}

}  // namespace

hipError_t launch_quantize_generic(const void* x, int x_dtype, int64_t B, int64_t T, int64_t H_kv, int64_t sb,
                                   int64_t st, int64_t sh, const tq_cache* dst, int64_t t_offset,
                                   const int32_t* ctx_lens, int64_t T_all, hipStream_t stream) {
  const QuantArgs qa = make_quant_args(x, B, ctx_lens != nullptr ? 1 : T, H_kv, sb, st, sh, dst, t_offset);
  if (ctx_lens == nullptr && T > 1 && x_dtype == TQ_BF16) {
    // bulk bfloat16 input: the MFMA kernel, tiles of 32 vectors per wavefront
    const int64_t total = B * H_kv * qa.nslot;
    if (total <= 0) return hipSuccess;
    if (dst->d == 64) return dispatch_qm<64>(dst->bits, dst->role, qa, total, stream);
    return dispatch_qm<256>(dst->bits, dst->role, qa, total, stream);
  }
  const int64_t blocks = ctx_lens != nullptr ? B * H_kv : B * H_kv * (qa.nslot / kValueBlock);
  if (blocks <= 0) return hipSuccess;
  const int xf32 = x_dtype == TQ_F32;
  if (dst->d == 64) return dispatch_qg<64>(dst->bits, dst->role, xf32, qa, ctx_lens, T_all, blocks, stream);
  return dispatch_qg<256>(dst->bits, dst->role, xf32, qa, ctx_lens, T_all, blocks, stream);
}

hipError_t launch_dequantize_generic(const tq_cache* src, int64_t t0, int64_t t1, float* out, hipStream_t stream) {
  GenericDequantArgs da;
  da.codes = src->codes;
  da.norms = src->norms;
  da.rot = src->rot;
  da.out = out;
  da.H_kv = src->H_kv;
  da.T_cap = src->T_cap;
  da.t0 = t0;
  da.t1 = t1;
  da.pm = page_map(src);
  const int L = 1 << src->bits;
  for (int i = 0; i < 16; ++i) da.cent[i] = i < L ? src->centroids[i] : 0.f;
  const int64_t blocks = src->B * src->H_kv * ((t1 - t0 + 7) / 8);
  if (blocks <= 0) return hipSuccess;
  if (src->d == 64) return dispatch_dqg<64>(src->bits, src->role, da, blocks, stream);
  return dispatch_dqg<256>(src->bits, src->role, da, blocks, stream);
}

hipError_t launch_decode_generic(const tq_cache* k, const tq_cache* v, const void* q, int q_dtype, int64_t H_q,
                                 const int32_t* ctx_lens, int64_t T, float scale, float* out, hipStream_t stream) {
  GenericDecodeArgs ga;
  ga.kcodes = k->codes;
  ga.knorms = k->norms;
  ga.rotK = k->rot;
  ga.vcodes = v->codes;
  ga.vnorms = v->norms;
  ga.rotV = v->rot;
  const int LK = 1 << k->bits, LV = 1 << v->bits;
  for (int i = 0; i < 16; ++i) {
    ga.kcent[i] = i < LK ? k->centroids[i] : 0.f;
    ga.vcent[i] = i < LV ? v->centroids[i] : 0.f;
  }
  ga.kpm = page_map(k);
  ga.vpm = page_map(v);
  ga.H_kv = k->H_kv;
  ga.kT_cap = k->T_cap;
  ga.vT_cap = v->T_cap;
  ga.q = q;
  ga.q_f32 = q_dtype == TQ_F32;
  ga.H_q = H_q;
  ga.G = (int)(H_q / k->H_kv);
  ga.ctx_lens = ctx_lens;
  ga.T = T;
  ga.scale = scale;
  ga.out = out;
  const int64_t blocks = k->B * k->H_kv;
  if (k->d == 64) return dispatch_decg<64>(k->bits, v->bits, ga, blocks, stream);
  return dispatch_decg<256>(k->bits, v->bits, ga, blocks, stream);
}

}  // namespace tq
