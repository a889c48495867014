// Dense chunked-prefill attention over the packed TurboQuant cache, for gfx950.
//
// M new tokens per row attend causally to the packed cache (token i of row b
// sees cache tokens below ctx_b - M + i + 1), with the decode's rotated-domain
// computation per (token, head) column. Where the decode kernel carries the G
// heads of one query (8 or 16 MFMA columns), this kernel gives every
// wavefront 32 (token, head) columns of one KV head, so the codebook lookups
// of a cache step (the float16 key and value operands) serve 32 columns, and
// the wavefronts of a workgroup (up to 4, 128 columns) read the same cache
// chunk once from HBM. The prompt-processing cost of compressed caches is what
// the qxai.app item on Tether QVAC's TurboQuant release notes as the weak spot.
//
// Per wavefront:
//   prologue  q' = Pi_K q for its 32 columns on MFMA (Pi_K split into float16
//             hi + lo, the query scaled by a power of two into float16, float32
//             queries split as well), staged through LDS into the QK operand
//             layout with a power-of-two scale per column, float16 hi and lo
//             parts (~22 bits);
//   scan      per 32-token step: key codes -> float16 operands (LDS lookup
//             table, shared by the workgroup), QK on MFMA for 2 column blocks
//             of 16 (hi and lo parts accumulate into one result), online
//             softmax per column (log2 domain, lazy rescale), value codes ->
//             operands, PV on MFMA into 128 coordinates x 32 columns;
//   epilogue  o = Pi_V^T acc per column on MFMA (Pi_V^T staged in LDS as
//             float16 hi + lo, each column's sums split the same way under a
//             power of two); with one context chunk the normalised output is
//             written at once, else the chunk's partial (m, l, rotated sums)
//             goes to the workspace and the decode's merge_kernel combines
//             the chunks in a fixed order (the inverse rotation is linear, so it commutes
//             with the merge).
// Keys with a QJL sketch take the tiled path (tq_decode.hip).
#include <math.h>

#include "tq_scan.h"

namespace tq {

namespace {

constexpr int kDenseCB = kDenseWaveCols / 16;  // 16-column MFMA blocks per wavefront
constexpr int kDenseCols = kDenseWaveCols;     // columns per wavefront
constexpr int kStageStride = kD + 4;           // floats per staged query row (bank spread)
// halves per staged row of Pi_V^T: a 16-byte pad spreads the 16 rows that one
// operand read touches over the banks
constexpr int kPtStride = kD + 8;
constexpr int kPtBytes = 2 * kD * kPtStride * 2;   // hi and lo parts

struct DenseArgs {
  const uint32_t* kcodes;
  const float* knorms;
  const uint32_t* vcodes;
  const float* vnorms;
  const void* q;          // [B][M][H_q][d]
  const float* rotK;      // Pi_K
  const float* rotV;      // Pi_V
  const int32_t* ctx_lens;
  float* out;             // [B][M][H_q][d] (written here when n_split == 1)
  float* ml;              // [B*M*H_q][n_split][2]: m (log2 domain reference), l
  float* acc;             // [B*M*H_q][n_split][d]: unnormalised rotated-domain sums
  int64_t TcK, TcV;
  PageMap kpm, vpm;
  int q_dtype, H_kv, H_q, G, T, M, n_split, chunk, ncg, NC;
  float sc1, inv_sqrt_d;
  float kc[16], vc[16];
};

constexpr int cmax(int x, int y) { return x > y ? x : y; }

template <int NWAVE>
constexpr int dense_region_bytes() {
  return cmax(cmax(kLutBytes, NWAVE * kDenseCols * kStageStride * 4), kPtBytes);
}

// Float16 hi and lo parts of 8 floats (an MFMA operand pair).
__device__ inline void split8(const float* v, half8& hi, half8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const _Float16 h = (_Float16)v[e];
    hi[e] = h;
    lo[e] = (_Float16)(v[e] - (float)h);
  }
}

template <int KB, int VB, int NWAVE, int PAGED>
__global__ __launch_bounds__(64 * NWAVE) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_dense_kernel(DenseArgs a) {
  constexpr int NT = 64 * NWAVE;
  constexpr int KW = 4 * KB;
  constexpr int REGION = dense_region_bytes<NWAVE>();
  __shared__ __align__(16) unsigned char smem[REGION + 32 * 4 + 16];
  uint32_t* lut = (uint32_t*)smem;
  float* stage_all = (float*)smem;                 // prologue: [NWAVE][64][kStageStride]
  _Float16* pth = (_Float16*)smem;                 // epilogue: Pi_V^T hi [kD][kPtStride]
  _Float16* ptl = pth + kD * kPtStride;            //                 lo
  float* cents = (float*)(smem + REGION);          // [32] key, value levels
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int lrep = lane & (kLutRep - 1);
  const int split = blockIdx.x, kv = blockIdx.y;
  const int b = blockIdx.z / a.ncg, cgrp = blockIdx.z - b * a.ncg;
  const int G = a.G;
  const int col0 = (cgrp * NWAVE + wave) * kDenseCols;   // this wavefront's first column
  const int64_t bkv = (int64_t)b * a.H_kv + kv;

  // ---- streams (as the decode)
  const bool kpg = PAGED && a.kpm.table != nullptr, vpg = PAGED && a.vpm.table != nullptr;
  const int64_t kbase = kpg ? 0 : bkv * a.TcK, vbase = vpg ? 0 : bkv * a.TcV;
  const int64_t krows = kpg ? (a.kpm.nblk * a.H_kv) << a.kpm.lg : a.TcK;
  const int64_t vrows = vpg ? (a.vpm.nblk * a.H_kv) << a.vpm.lg : a.TcV;
  Streams s;
  s.rk = make_rsrc(a.kcodes + kbase * KW, (uint32_t)(krows * KW * 4));
  s.rkn = make_rsrc(a.knorms + kbase, (uint32_t)(krows * 4));
  s.rv = make_rsrc(a.vcodes + vbase * 4 * VB, (uint32_t)(vrows * 4 * VB * 4));
  s.rvn = make_rsrc(a.vnorms + vbase, (uint32_t)(vrows * 4));
  s.rs = make_rsrc(a.knorms, 0u);
  s.rg = make_rsrc(a.knorms, 0u);
  const __amdgpu_buffer_rsrc_t rtk =
      make_rsrc(kpg ? (const void*)(a.kpm.table + b * a.kpm.maxblk) : (const void*)a.knorms,
                kpg ? (uint32_t)(a.kpm.maxblk * 4) : 0u);
  const __amdgpu_buffer_rsrc_t rtv =
      make_rsrc(vpg ? (const void*)(a.vpm.table + b * a.vpm.maxblk) : (const void*)a.knorms,
                vpg ? (uint32_t)(a.vpm.maxblk * 4) : 0u);
  LaneOffsets lo;
  {
    const int tk = 8 * (c >> 2) + (c & 3);   // MFMA row c of row block 0 (block 1: tk + 4)
    lo.k = (uint32_t)(tk * KW + g * KB) * 4u;
    lo.s = 0u;
  }
  lo.v = (uint32_t)(g * 32 * VB + c * 2 * VB) * 4u;
  lo.n = (uint32_t)(8 * g + (c & 7)) * 4u;   // lane (g, c) reads token 8g + c % 8 (row broadcast)

  // ---- context range of this workgroup and the causal limits of the wavefront's columns
  int ctx = a.T;
  if (a.ctx_lens != nullptr) ctx = a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.T ? a.T : ctx);
  const int lim0 = ctx - a.M + 1;   // token i sees cache tokens below lim0 + i
  const int nvalid = a.NC - col0;   // columns of this wavefront that exist (may be <= 0)
  const int i_lo = col0 / G;
  const int i_hi = (col0 + (nvalid < kDenseCols ? nvalid : kDenseCols) - 1) / G;
  const int lim_lo = max(lim0 + i_lo, 0), lim_hi = max(lim0 + i_hi, 0);
  const int t_begin = split * a.chunk;
  const int t_end = __builtin_amdgcn_readfirstlane(nvalid > 0 ? min(t_begin + a.chunk, lim_hi) : t_begin);
  const int t_unm = min(t_end, lim_lo);
  const int t_full =
      __builtin_amdgcn_readfirstlane(t_begin + (t_unm > t_begin ? (t_unm - t_begin) / kStep * kStep : 0));
  // per column block: the lane's column, its token and causal limit (padding
  // columns keep the widest limit and a zero query)
  int lim_cb[kDenseCB];
#pragma unroll
  for (int cb = 0; cb < kDenseCB; ++cb) {
    const int col = col0 + 16 * cb + c;
    lim_cb[cb] = col < a.NC ? max(lim0 + col / G, 0) : lim_hi;
  }

  // ---- first step's loads in flight during the prologue
  StepData<KB, VB, 0, 1> buf[2];
  uint32_t ek = 0u, ev = 0u;
  {
    const int tj = t_begin + kStep <= min(a.TcK, a.TcV) ? t_begin : 0;
    if (kpg) ek = page_entry(rtk, a.kpm, tj);
    if (vpg) ev = page_entry(rtv, a.vpm, tj);
    load_step<false>(buf[0], s, lo, step_row(a.kpm, kv, a.H_kv, ek, tj), step_row(a.vpm, kv, a.H_kv, ev, tj));
    const int tn = t_begin + kStep;
    if (kpg) ek = page_entry(rtk, a.kpm, tn);
    if (vpg) ev = page_entry(rtv, a.vpm, tn);
  }

  // ---- prologue 1: q' = Pi_K q of the wavefront's columns on MFMA, into the
  // wavefront's LDS stage as float32 rows [column][coordinate].
  // Rotation MFMA (16x16x32): A = rows 16ob.. of Pi_K (lane (g, i): row
  // 16ob + i, coordinates 32kb + 8g + 0..7), B = the query columns (lane (g, c):
  // coordinates 32kb + 8g + 0..7 of column c), D lane (g, c) = q' coordinates
  // 16ob + 4g + 0..3 of column c.
  float* stage = stage_all + wave * kDenseCols * kStageStride;
  {
    const bool qbf = a.q_dtype == TQ_BF16;
    half8 qh[kDenseCB][4], ql[kDenseCB][4];
    float qsc[kDenseCB];   // 2^-sexp: undoes the column's power-of-two scale
#pragma unroll
    for (int cb = 0; cb < kDenseCB; ++cb) {
      const int col = col0 + 16 * cb + c;
      float v[32];
      if (col < a.NC) {
        const int i = col / G, h = col - (col / G) * G;
        const int64_t row = ((int64_t)b * a.M + i) * a.H_q + (int64_t)kv * G + h;
        if (qbf) {
          const uint16_t* p = (const uint16_t*)a.q + row * kD;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const u32x4 w = *(const u32x4*)(p + 32 * kb + 8 * g);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              v[8 * kb + 2 * u] = __uint_as_float(w[u] << 16);
              v[8 * kb + 2 * u + 1] = __uint_as_float(w[u] & 0xFFFF0000u);
            }
          }
        } else {
          const float* p = (const float*)a.q + row * kD;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const float4 x0 = *(const float4*)(p + 32 * kb + 8 * g);
            const float4 x1 = *(const float4*)(p + 32 * kb + 8 * g + 4);
            v[8 * kb + 0] = x0.x; v[8 * kb + 1] = x0.y; v[8 * kb + 2] = x0.z; v[8 * kb + 3] = x0.w;
            v[8 * kb + 4] = x1.x; v[8 * kb + 5] = x1.y; v[8 * kb + 6] = x1.z; v[8 * kb + 7] = x1.w;
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < 32; ++k) v[k] = 0.f;
      }
      // power of two per column: largest entry into [2^13, 2^14)
      float mx = 0.f;
#pragma unroll
      for (int k = 0; k < 32; ++k) mx = fmaxf(mx, fabsf(v[k]));
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const int sexp = (mx > 0.f) ? 14 - __builtin_amdgcn_frexp_expf(mx) : 0;
      qsc[cb] = ldexpf(1.0f, -sexp);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = ldexpf(v[8 * kb + e], sexp);
        split8(t, qh[cb][kb], ql[cb][kb]);
      }
    }
#pragma unroll 1
    for (int ob = 0; ob < 8; ++ob) {
      half8 ph[4], pl[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float* p = a.rotK + (16 * ob + c) * kD + 32 * kb + 8 * g;
        const float4 x0 = *(const float4*)p, x1 = *(const float4*)(p + 4);
        const float t[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        split8(t, ph[kb], pl[kb]);
      }
#pragma unroll
      for (int cb = 0; cb < kDenseCB; ++cb) {
        floatx4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          d = mfma16(ph[kb], qh[cb][kb], d);
          d = mfma16(pl[kb], qh[cb][kb], d);
          if (!qbf) d = mfma16(ph[kb], ql[cb][kb], d);
        }
        float* dst = stage + (16 * cb + c) * kStageStride + 16 * ob + 4 * g;
        *(float4*)dst = float4{d[0] * qsc[cb], d[1] * qsc[cb], d[2] * qsc[cb], d[3] * qsc[cb]};
      }
    }
  }
  // (each wavefront reads back only its own stage: LDS operations of a
  // wavefront complete in order; the fences keep the compiler's order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- prologue 2: QK operands (B of 16x16x32: lane (g, c) holds coordinates
  // 32g + 8kk + 0..7 of column c), log2(e) * scale / sqrt(d) applied, a power
  // of two per column so its largest entry lies in [2^13, 2^14), hi and lo parts
  half8 Qh[kDenseCB][4], Ql[kDenseCB][4];
  float cs[kDenseCB];
#pragma unroll
  for (int cb = 0; cb < kDenseCB; ++cb) {
    const float* src = stage + (16 * cb + c) * kStageStride + 32 * g;
    float v[32];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 x = *(const float4*)(src + 4 * k);
      v[4 * k] = x.x * a.sc1;
      v[4 * k + 1] = x.y * a.sc1;
      v[4 * k + 2] = x.z * a.sc1;
      v[4 * k + 3] = x.w * a.sc1;
    }
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) mx = fmaxf(mx, fabsf(v[k]));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const int e = (mx > 0.f) ? (__builtin_amdgcn_frexp_expf(mx) - 14) : 0;
    cs[cb] = ldexpf(1.0f, e);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = ldexpf(v[8 * kk + u], -e);
      split8(t, Qh[cb][kk], Ql[cb][kk]);
    }
  }
  __syncthreads();   // every stage has been read: the region becomes the lookup table

  // ---- lookup table (codebook levels from the kernel arguments)
  if (tid < 32) {
    float cv = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      cv = tid == i ? a.kc[i] : cv;
      cv = tid == 16 + i ? a.vc[i] : cv;
    }
    cents[tid] = cv;
  }
  __syncthreads();
  build_lut<KB, VB>(lut, cents, cents + 16, tid, NT);
  __syncthreads();

  // ---- softmax state per column block (uniform over the 4 lanes of a column
  // except l, which each lane sums over its own tokens)
  float m_ref[kDenseCB], m_off[kDenseCB], l[kDenseCB];
  floatx4 acc[kDenseCB][8];
#pragma unroll
  for (int cb = 0; cb < kDenseCB; ++cb) {
    m_ref[cb] = -INFINITY;
    m_off[cb] = -INFINITY;
    l[cb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[cb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  // value-norm scale of the wavefront (see the decode kernel)
  float evn;
  {
    float vm = fabsf(buf[0].nm.vn);
    vm = fmaxf(vm, dpp_xor1(vm));
    vm = fmaxf(vm, dpp_xor2(vm));
    vm = fmaxf(vm, dpp_ror4(vm));
    vm = fmaxf(vm, dpp_ror8(vm));
    vm = fmaxf(vm, shfl_xor_f(vm, 16));
    vm = fmaxf(vm, shfl_xor_f(vm, 32));
    int e = (vm > 0.f && vm < INFINITY) ? __builtin_amdgcn_frexp_expf(vm) : 0;
    e = e < -kNormExpClamp ? -kNormExpClamp : (e > kNormExpClamp ? kNormExpClamp : e);
    evn = (float)__builtin_amdgcn_readfirstlane(e);
  }
  LutRegs lr;
#pragma unroll
  for (int i = 0; i < 4; ++i) lr.a[i] = lr.b[i] = (uint32_t)lrep * 4u;

  // One 32-token step for the wavefront's columns. MASK: per-column causal limits.
  // The step runs in phases that the scheduler may not mix (sched_barrier):
  // every QK product (the key lookups between them), the value lookups, then
  // per column block its softmax followed by its PV products. Against the
  // compiler's own order (each block's products, then its softmax) this took
  // about 2 % off the kernel; the arithmetic is the same in either order.
  auto step = [&](const StepData<KB, VB, 0, 1>& d, int t0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value != 0;
    // scores of every column block: key operands of both row blocks (lane
    // (g, i): token 8(i/4) + 4m + i%4) against the hi and lo query parts
    floatx4 sc[kDenseCB][2];
    {
      half8 ka[2][4];
      ka[0][0] = key_operand<KB, 0>(d.kw[0], (const char*)lut, lr.a);
      ka[0][1] = key_operand<KB, 1>(d.kw[0], (const char*)lut, lr.b);
      ka[0][2] = key_operand<KB, 2>(d.kw[0], (const char*)lut, lr.a);
      ka[0][3] = key_operand<KB, 3>(d.kw[0], (const char*)lut, lr.b);
      ka[1][0] = key_operand<KB, 0>(d.kw[1], (const char*)lut, lr.a);
      ka[1][1] = key_operand<KB, 1>(d.kw[1], (const char*)lut, lr.b);
      ka[1][2] = key_operand<KB, 2>(d.kw[1], (const char*)lut, lr.a);
      ka[1][3] = key_operand<KB, 3>(d.kw[1], (const char*)lut, lr.b);
#pragma unroll
      for (int cb = 0; cb < kDenseCB; ++cb) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            x = mfma16(ka[m][kk], Qh[cb][kk], x);
            x = mfma16(ka[m][kk], Ql[cb][kk], x);
          }
          sc[cb][m] = x;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // value operands (the 8-token block layout: lane (g, c) holds 8 tokens of
    // one coordinate) and the value norms of the lane's 8 tokens
    half8 va[8];
    va[0] = value_operand<VB, 0>(d.vw, (const char*)lut, lr.a);
    va[1] = value_operand<VB, 1>(d.vw, (const char*)lut, lr.b);
    va[2] = value_operand<VB, 2>(d.vw, (const char*)lut, lr.a);
    va[3] = value_operand<VB, 3>(d.vw, (const char*)lut, lr.b);
    va[4] = value_operand<VB, 4>(d.vw, (const char*)lut, lr.a);
    va[5] = value_operand<VB, 5>(d.vw, (const char*)lut, lr.b);
    va[6] = value_operand<VB, 6>(d.vw, (const char*)lut, lr.a);
    va[7] = value_operand<VB, 7>(d.vw, (const char*)lut, lr.b);
    float vn8[8];
    vn8[0] = bcast_row_mov<0>(d.nm.vn);
    vn8[1] = bcast_row_mov<1>(d.nm.vn);
    vn8[2] = bcast_row_mov<2>(d.nm.vn);
    vn8[3] = bcast_row_mov<3>(d.nm.vn);
    vn8[4] = bcast_row_mov<4>(d.nm.vn);
    vn8[5] = bcast_row_mov<5>(d.nm.vn);
    vn8[6] = bcast_row_mov<6>(d.nm.vn);
    vn8[7] = bcast_row_mov<7>(d.nm.vn);
    __builtin_amdgcn_sched_barrier(0);
    const int tg = t0 + 8 * g;
#pragma unroll
    for (int cb = 0; cb < kDenseCB; ++cb) {
      // softmax of the block's columns (lane (g, c) holds tokens 8g + 4m + r
      // of column c) and its float16 weights, the PV operand
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = sc[cb][e >> 2][e & 3] * bcast_row(d.nm.kn, e);
        if constexpr (MASK) v = (tg + e < lim_cb[cb]) ? v : -INFINITY;
        y[e] = v;
      }
      const float lmax = fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])), fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
      if (__any(lmax * cs[cb] > m_ref[cb] + kSlack)) {
        // the reference of some column moves: column maxima over its 4 lanes
        float tmax = fmaxf(lmax, shfl_xor_f(lmax, 16));
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
        const float m_new = fmaxf(m_ref[cb], tmax * cs[cb]);
        // (a column with nothing accumulated yet, m_ref = -inf, may still see
        // no visible token while another column moves: its factor is 0, not NaN)
        const float alpha = m_ref[cb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[cb] - m_new);
        l[cb] *= alpha;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[cb][nb] *= alpha;
        m_ref[cb] = m_new;
        m_off[cb] = m_new + kShift + evn;
      }
      half8 wb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float p = __builtin_amdgcn_exp2f(fmaf(y[e], cs[cb], -m_off[cb]));
        if constexpr (MASK) p = (tg + e < lim_cb[cb]) ? p : 0.f;   // (NaN when nothing visible yet)
        l[cb] += p;
        wb[e] = (_Float16)(p * vn8[e]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) acc[cb][nb] = mfma16(va[nb], wb, acc[cb][nb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- stream the chunk: full steps with two register buffers, then the
  // masked steps (causal band, ragged end)
  int t0 = t_begin;
  if (t0 < t_full) {
    // (the two buffers in turn, with constant indices: register arrays)
    auto full_step = [&](StepData<KB, VB, 0, 1>& cur, StepData<KB, VB, 0, 1>& nxt) -> bool {
      wait_step(cur);
      if (t0 + kStep < t_full) {
        const int tl = t0 + kStep, tn = tl + kStep;
        const uint32_t rk = step_row(a.kpm, kv, a.H_kv, ek, tl);
        const uint32_t rv = step_row(a.vpm, kv, a.H_kv, ev, tl);
        if (kpg && (tn & ((1 << a.kpm.lg) - 1)) == 0) ek = page_entry(rtk, a.kpm, tn);
        if (vpg && (tn & ((1 << a.vpm.lg) - 1)) == 0) ev = page_entry(rtv, a.vpm, tn);
        load_step<false>(nxt, s, lo, rk, rv);
      }
      step(cur, t0, IntConst<0>{});
      t0 += kStep;
      return t0 < t_full;
    };
    while (full_step(buf[0], buf[1]) && full_step(buf[1], buf[0])) {
    }
  }
  t0 = __builtin_amdgcn_readfirstlane(t0);
  while (t0 < t_end) {
    StepData<KB, VB, 0, 1> E;
    if (kpg) ek = page_entry(rtk, a.kpm, t0);
    if (vpg) ev = page_entry(rtv, a.vpm, t0);
    load_step<true>(E, s, lo, step_row(a.kpm, kv, a.H_kv, ek, t0), step_row(a.vpm, kv, a.H_kv, ev, t0));
    step(E, t0, IntConst<1>{});
    t0 += kStep;
  }

  // ---- epilogue: Pi_V^T staged in LDS (the lookup tables are done with)
  __syncthreads();
  {
    // item (i, jg): rows 8jg .. 8jg+7 of column i of Pi_V (lanes take
    // consecutive columns: each load reads 256 contiguous bytes)
    constexpr int ITEMS = kD * (kD / 8), PER = ITEMS / NT;
    static_assert(ITEMS % NT == 0, "staging items");
#pragma unroll 8
    for (int u = 0; u < PER; ++u) {
      const int item = tid + u * NT, i = item % kD, jg = item / kD;
      float x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = a.rotV[(8 * jg + k) * kD + i];
      half8 hi, lo;
      split8(x, hi, lo);
      *(half8*)(pth + i * kPtStride + 8 * jg) = hi;
      *(half8*)(ptl + i * kPtStride + 8 * jg) = lo;
    }
  }
  __syncthreads();

  // ---- o = Pi_V^T acc per column (16x16x32: A = rows 16ob.. of Pi_V^T, lane
  // (g, i): entries (16ob + i, 32g + 8kb + 0..7); B = the column sums, lane
  // (g, c): coordinates 32g + 8kb + nb, nb = 0..7, which are acc[cb][nb][kb];
  // D lane (g, c): output coordinates 16ob + 4g + 0..3 of column c). l is
  // summed over the column's 4 lanes.
#pragma unroll
  for (int cb = 0; cb < kDenseCB; ++cb) {
    float lt = l[cb];
    lt += shfl_xor_f(lt, 16);
    lt += shfl_xor_f(lt, 32);
    float mx = 0.f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[cb][nb][r]));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const int e = (mx > 0.f && mx < INFINITY) ? __builtin_amdgcn_frexp_expf(mx) : 0;
    half8 bh[4], bl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float t[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) t[nb] = ldexpf(acc[cb][nb][kb], 14 - e);
      split8(t, bh[kb], bl[kb]);
    }
    const int col = col0 + 16 * cb + c;
    const bool one = a.n_split == 1;
    // one chunk: out = o / l / sqrt(d) (0 where no token is visible); else the
    // chunk's unnormalised partial
    const float f = one ? (lt > 0.f ? ldexpf(a.inv_sqrt_d / lt, e - 14) : 0.f) : ldexpf(1.0f, e - 14);
    int64_t base = 0;
    if (col < a.NC) {
      const int i = col / G, h = col - (col / G) * G;
      const int64_t row = ((int64_t)b * a.M + i) * a.H_q + (int64_t)kv * G + h;
      const int64_t pidx = row * a.n_split + split;
      base = one ? row * kD : pidx * kD;
      if (!one && g == 0) {
        a.ml[pidx * 2] = m_off[cb];
        a.ml[pidx * 2 + 1] = lt;
      }
    }
    float* dst = one ? a.out : a.acc;
#pragma unroll
    for (int ob = 0; ob < 8; ++ob) {
      floatx4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int off = (16 * ob + c) * kPtStride + 32 * g + 8 * kb;
        const half8 ah = *(const half8*)(pth + off);
        const half8 al = *(const half8*)(ptl + off);
        d = mfma16(ah, bh[kb], d);
        d = mfma16(al, bh[kb], d);
        d = mfma16(ah, bl[kb], d);
      }
      if (col < a.NC) *(float4*)(dst + base + 16 * ob + 4 * g) = float4{d[0] * f, d[1] * f, d[2] * f, d[3] * f};
    }
  }
}

template <int KB, int VB, int NWAVE>
hipError_t launch_dense3(const DensePlan& p, const DenseArgs& da, hipStream_t stream) {
  dim3 grid((unsigned)p.n_split, (unsigned)p.H_kv, (unsigned)(p.B * p.ncg));
  if (da.kpm.table != nullptr || da.vpm.table != nullptr)
    hipLaunchKernelGGL((prefill_dense_kernel<KB, VB, NWAVE, 1>), grid, dim3(64 * NWAVE), 0, stream, da);
  else
    hipLaunchKernelGGL((prefill_dense_kernel<KB, VB, NWAVE, 0>), grid, dim3(64 * NWAVE), 0, stream, da);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_dense2(const DensePlan& p, const DenseArgs& da, hipStream_t s) {
  switch (p.nwave) {
    case 1: return launch_dense3<KB, VB, 1>(p, da, s);
    case 2: return launch_dense3<KB, VB, 2>(p, da, s);
    default: return launch_dense3<KB, VB, 4>(p, da, s);
  }
}

template <int KB>
hipError_t launch_dense1(int vb, const DensePlan& p, const DenseArgs& da, hipStream_t s) {
  switch (vb) {
    case 2: return launch_dense2<KB, 2>(p, da, s);
    case 3: return launch_dense2<KB, 3>(p, da, s);
    default: return launch_dense2<KB, 4>(p, da, s);
  }
}

}  // namespace

hipError_t launch_prefill_dense(const DensePlan& p, const tq_cache* k, const tq_cache* v, const void* q, int q_dtype,
                                const int32_t* ctx_lens, float scale, float* out, void* ws, hipStream_t stream) {
  char* base = (char*)ws;
  DenseArgs da;
  da.kcodes = k->codes;
  da.knorms = k->norms;
  da.vcodes = v->codes;
  da.vnorms = v->norms;
  da.q = q;
  da.rotK = k->rot;
  da.rotV = v->rot;
  da.ctx_lens = ctx_lens;
  da.out = out;
  da.ml = (float*)(base + p.off_ml);
  da.acc = (float*)(base + p.off_acc);
  da.TcK = k->T_cap;
  da.TcV = v->T_cap;
  da.kpm = page_map(k);
  da.vpm = page_map(v);
  da.q_dtype = q_dtype;
  da.H_kv = (int)p.H_kv;
  da.H_q = (int)p.H_q;
  da.G = p.G;
  da.T = (int)p.T;
  da.M = (int)p.M;
  da.n_split = p.n_split;
  da.chunk = p.chunk;
  da.ncg = p.ncg;
  da.NC = p.NC;
  const float inv_sqrt_d = 1.0f / sqrtf((float)kD);
  da.sc1 = scale * kLog2e * inv_sqrt_d;
  da.inv_sqrt_d = inv_sqrt_d;
  for (int i = 0; i < 16; ++i) {
    da.kc[i] = i < (1 << k->bits) ? k->centroids[i] : 0.f;
    da.vc[i] = i < (1 << v->bits) ? v->centroids[i] : 0.f;
  }
  hipError_t err;
  switch (k->bits) {
    case 2: err = launch_dense1<2>(v->bits, p, da, stream); break;
    case 3: err = launch_dense1<3>(v->bits, p, da, stream); break;
    default: err = launch_dense1<4>(v->bits, p, da, stream); break;
  }
  if (err != hipSuccess || p.n_split == 1) return err;
  return launch_merge(da.ml, da.acc, out, p.B * p.M * p.H_q, p.n_split, kD, stream);
}

}  // namespace tq
