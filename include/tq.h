/*
 * tq.h — C ABI of the TurboQuant packed-KV library for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (TurboQuant as described in the ai-accelerate.xyz
 * TurboQuant article, section "TurboQuantの仕組み"):
 *   step 1  every key/value head vector x is multiplied by a seeded random
 *           orthogonal matrix Pi; each rotated coordinate is quantized on its
 *           own with the Gaussian Lloyd-Max scalar codebook at 2, 3 or 4 bits;
 *           no per-block full-precision scale is kept, only the vector norm.
 *   step 2  (optional, keys) one sign bit per coordinate of a Gaussian
 *           projection S of the quantization residual, which makes the key
 *           inner-product estimate unbiased.
 * Decode attention reads the packed cache directly: the query is rotated once,
 * scores are codebook levels times key norms, values are summed in the
 * rotated domain and one inverse rotation produces the output.
 *
 * Conventions (all functions):
 *   - return an int status (TQ_OK = 0); nothing throws; the only process-wide
 *     state is cached device attributes and kernel attributes set once, plus
 *     a per-thread record of the last HIP error (tq_last_hip_error);
 *   - argument errors are reported synchronously, before any HIP call;
 *   - device calls are asynchronous on the given hipStream_t (passed as void*,
 *     NULL = the default stream); a failed launch returns TQ_ERR_DEVICE (an
 *     error left pending on the thread by an earlier, unrelated HIP call is
 *     cleared before the launch and not reported), a fault inside a kernel
 *     surfaces at the caller's next synchronisation;
 *   - the caller owns every buffer; the library never allocates or frees device
 *     memory (its one static device array, the scratch of
 *     tq_decode_attention_noalloc, is part of its loaded code object);
 *   - head dimension d = 128, 64 or 256 (other values return
 *     TQ_ERR_UNSUPPORTED), the same packed formats at every d. Decode and
 *     chunked prefill run the same MFMA scan tiles at every d (d = 256 up to 8
 *     (query token, head) columns per KV head; a decode with G > 8 there runs
 *     a generic float32 kernel, one workgroup per (row, KV head), and a
 *     prefill with M * G > 8 returns TQ_ERR_UNSUPPORTED). Quantize, append and
 *     dequantize at d = 64 and 256 run generic kernels (float32 rotations,
 *     one workgroup per 8-token block). QJL keys take d = 128 only.
 *
 * Packed formats (one cache per tensor and layer; keys and values set their bit
 * width separately):
 *   norms   float32 [B][H_kv][T_cap]: |x| of the input vector, 0 for x = 0.
 *   codes   uint32 words, d*bits/32 words per token, [B][H_kv][T_cap*d*bits/32]:
 *             TQ_KEYS    per-token record: coordinate j's code is at bits
 *                        [bits*j, bits*j+bits) of the record's LSB-first stream
 *                        (stream bit k = bit k%32 of word k/32);
 *             TQ_VALUES  8-token blocks (tokens 8m..8m+7), one record of
 *                        8*d*bits/32 words per block: token 8m+i, coordinate j
 *                        at stream bits [bits*(8j+i), ...); T_cap % 8 == 0.
 *           code c stands for centroid c (centroids ascend; c = #{thresholds <= u*sqrt(d)}).
 *   QJL     keys only: qjl_signs uint32 [B][H_kv][T_cap][d/32], bit i = [(S r)_i >= 0];
 *           qjl_gamma float32 [B][H_kv][T_cap] = |r|, r = u - centroid/sqrt(d).
 *   Pi, S   float32 d x d row-major on the device; y = Pi x.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TQ_OK 0
#define TQ_ERR_INVALID_ARGUMENT 1   /* null pointer, bad size, inconsistent shapes */
#define TQ_ERR_UNSUPPORTED 2        /* valid but not implemented (d not 64/128/256, G > 16, ...) */
#define TQ_ERR_ALIGNMENT 3          /* a device pointer breaks its alignment rule */
#define TQ_ERR_WORKSPACE_TOO_SMALL 4
#define TQ_ERR_DEVICE 5             /* a HIP call or kernel launch failed */

/* element types of inputs */
#define TQ_F32 0
#define TQ_BF16 1

/* tq_make_rotation kinds */
#define TQ_MAT_HAAR 0       /* Pi: Haar-random orthogonal */
#define TQ_MAT_GAUSSIAN 1   /* S: i.i.d. N(0,1), not orthogonalised */
#define TQ_MAT_HADAMARD 2   /* Pi: randomized Hadamard H D / sqrt(d) (orthogonal) */

/* cache roles: decide the code layout */
#define TQ_KEYS 0
#define TQ_VALUES 1

#define TQ_MAX_LEVELS 16

/*
 * One packed cache (all heads of one layer's keys, or of its values).
 * Device pointers must be 16-byte aligned. centroids[] is held by value (host
 * memory, inside this struct): the 2^bits levels of tq_make_codebook, in
 * standard-normal units, each exactly representable in float16.
 *
 * Contiguous layout (block_table == NULL): every (row, head) owns T_cap token
 * rows, at token row (b*H_kv + h)*T_cap + t of each array.
 *
 * Paged layout (block_table != NULL): the arrays hold n_blocks physical blocks
 * of block_tokens tokens for all H_kv heads, and block_table (device int32,
 * [B][T_cap / block_tokens]) maps logical block t / block_tokens of row b to
 * a physical block p. Token t of (row b, head h) is at token row
 * (p*H_kv + h)*block_tokens + t % block_tokens of each array (for value codes,
 * its 8-token block is that row / 8). Rules: block_tokens is a power of two
 * from 32 to 65536; T_cap is a multiple of it; every entry that a call reads
 * or writes through (tokens below the context length, tokens being quantized)
 * is in [0, n_blocks) (other entries are clamped into that range when the
 * decode reads ahead, so they are never dereferenced out of bounds); a block
 * written by tq_quantize_kv is mapped by one (row, logical block) only (two
 * rows that share it would race); each array stays below 2 GiB. The layout
 * serves a runtime's per-layer cache whose blocks are allocated as sequences
 * grow (the ai-navigate-news.com post, Part 4: the serving sidecar builds one
 * TurboQuant KV cache per transformer layer; the ai-accelerate.xyz article,
 * section on what TurboQuant means for local LLM users: key and value cache
 * types are chosen separately).
 */
typedef struct tq_cache {
  int32_t role;        /* TQ_KEYS or TQ_VALUES */
  int32_t bits;        /* 2, 3 or 4 bits per coordinate (the Lloyd-Max part) */
  int32_t qjl;         /* 1: keys carry the QJL sign sketch; 0 otherwise */
  int32_t d;           /* head dimension: 128, 64 or 256 (QJL keys: 128) */
  int64_t B;           /* batch rows */
  int64_t H_kv;        /* KV heads */
  int64_t T_cap;       /* token capacity per (row, head); multiple of 8 for values */
  uint32_t* codes;     /* device, R*d*bits/32 words, R token rows (see layouts above) */
  float* norms;        /* device, R */
  uint32_t* qjl_signs; /* device, R*d/32 words, or NULL when qjl == 0 */
  float* qjl_gamma;    /* device, R, or NULL when qjl == 0 */
  const float* rot;    /* device Pi, d*d, row-major */
  const float* qjl_proj; /* device S, d*d, or NULL when qjl == 0 */
  float centroids[TQ_MAX_LEVELS];
  /* R = B*H_kv*T_cap (contiguous) or n_blocks*H_kv*block_tokens (paged) */
  const int32_t* block_table; /* device [B][T_cap/block_tokens], or NULL: contiguous */
  int64_t block_tokens;       /* paged: tokens per block; ignored when contiguous */
  int64_t n_blocks;           /* paged: physical blocks; ignored when contiguous */
} tq_cache;

/*
 * Gaussian Lloyd-Max codebook (ai-accelerate.xyz TurboQuant article, section
 * "TurboQuantの仕組み", step 1: optimal scalar quantization of near-Gaussian
 * coordinates). Lloyd's iteration for N(0,1) with 2^bits cells from
 * c_i = Phi^-1((i+1/2)/2^bits) until the largest change is below 1e-14, then
 * symmetrised and rounded to float16 (nearest even). thresholds[i] is the exact
 * midpoint of centroids[i] and centroids[i+1]; the middle one is +0.0.
 * centroids: host, 2^bits floats; thresholds: host, 2^bits - 1 floats (may be NULL).
 * The codebook is in standard units, so it is the same for every d.
 * bits in 1..4; d is 64, 128 or 256. Host only: no HIP call.
 */
int tq_make_codebook(int32_t bits, int32_t d, float* centroids, float* thresholds);

/*
 * Sphere-exact Lloyd-Max codebook (format variant of the same step 1): the
 * quantizer of the exact law of one coordinate u of a uniform unit vector in
 * d dimensions (density proportional to (1 - u^2)^((d-3)/2) on [-1, 1]; the
 * article calls the rotated coordinates near-Gaussian, and this is the law
 * they follow exactly), in the same standard units (z = u sqrt(d)) and the
 * same stored form as tq_make_codebook: Lloyd's iteration from the law's
 * quantiles (i+1/2)/2^bits to a largest change below 1e-14, symmetrised,
 * float16-rounded centroids, exact midpoint thresholds, middle one +0.0.
 * Cell probabilities use the regularized incomplete beta function. At d = 128
 * the 3-bit MSE is 0.033966 against 0.034548 for the Gaussian codebook on
 * Gaussian data. bits in 1..4; d in 3..65536 (host computation; the kernels
 * take d = 64, 128, 256). Host only: no HIP call.
 */
int tq_make_codebook_sphere(int32_t bits, int32_t d, float* centroids, float* thresholds);

/*
 * Seeded d x d matrix, row-major float32, into host memory `out`.
 * The stream is SplitMix64 (output k = finalizer(seed + k*0x9E3779B97F4A7C15),
 * k = 1, 2, ...), uniforms ((z>>11)+0.5)*2^-53, Box-Muller normals (cos then
 * sin per pair), filled row-major. TQ_MAT_HAAR: Q*diag(sign(diag R)) of the
 * Householder QR of that matrix (the random orthogonal matrix of step 1 of the
 * method); TQ_MAT_GAUSSIAN: the matrix itself (the QJL projection of step 2);
 * TQ_MAT_HADAMARD: H diag(s) / sqrt(d) with H the Sylvester-Hadamard matrix
 * (H[i][j] = (-1)^popcount(i & j)) and s_j = -1 when the top bit of stream
 * output j+1 is set, else +1 (a randomized Hadamard rotation, a cheaper
 * orthogonal alternative for step 1; stored dense like the others).
 * Computed in double precision, rounded to float32. d is 64, 128 or 256.
 * Host only: no HIP call.
 */
int tq_make_rotation(uint64_t seed, int32_t d, int32_t kind, float* out);

/*
 * Quantize T new tokens of every (row, head) into dst at token positions
 * t_offset .. t_offset+T-1 (step 1, and step 2 for QJL keys).
 * x: device, element (b, t, h, j) at x[b*stride_b + t*stride_t + h*stride_h + j]
 *    (strides in elements, j contiguous), dtype TQ_F32 or TQ_BF16, 16-byte
 *    aligned rows. Requires B == dst->B, H_kv == dst->H_kv, T >= 0,
 *    0 <= t_offset, t_offset + T <= dst->T_cap. Value blocks that the range only
 *    partly covers keep the bits of their other tokens. T == 0 is a no-op.
 */
int tq_quantize_kv(const void* x, int32_t x_dtype, int64_t B, int64_t T, int64_t H_kv,
                   int64_t stride_b, int64_t stride_t, int64_t stride_h,
                   const tq_cache* dst, int64_t t_offset, void* hip_stream);

/*
 * The key and the value of one new token per (row, head), into token position
 * t_offset of kc and vc: the same result, byte for byte, as tq_quantize_kv of
 * k into kc and of v into vc with T = 1 (step 1 of the method, and step 2 for
 * QJL keys), in one launch when the keys carry no QJL sketch (two otherwise).
 * k, v: device, element (b, h, j) at k[b*k_stride_b + h*k_stride_h + j] (and
 *   the same for v), dtype TQ_F32 or TQ_BF16, 16-byte aligned rows.
 * Requires kc->role == TQ_KEYS, vc->role == TQ_VALUES, B == kc->B == vc->B,
 * H_kv == kc->H_kv == vc->H_kv, 0 <= t_offset < min(kc->T_cap, vc->T_cap).
 * The caller owns all buffers; errors are returned before anything is launched.
 */
int tq_append_kv(const void* k, const void* v, int32_t x_dtype, int64_t B, int64_t H_kv,
                 int64_t k_stride_b, int64_t k_stride_h, int64_t v_stride_b, int64_t v_stride_h,
                 const tq_cache* kc, const tq_cache* vc, int64_t t_offset, void* hip_stream);

/*
 * Reconstruct tokens t0 .. t1-1 of every (row, head): the inverse of the two
 * steps of the method (ai-accelerate.xyz TurboQuant article, section
 * "TurboQuantの仕組み": step 1 keeps, per rotated coordinate, the Lloyd-Max
 * level of its cell, so undoing it maps the codes back to levels and applies
 * the transpose of the orthogonal rotation; step 2's sign bits add the QJL
 * estimate of the residual):
 *   x_hat = n * Pi^T (c[code]/sqrt(d) [+ gamma*sqrt(pi/2)/d * S^T sigma]),
 * sigma_i = 2*bit_i - 1 (QJL keys).
 *   src: a cache filled by tq_quantize_kv / tq_append_kv (read only)
 *   out: device float32 [B][H_kv][t1-t0][d], 16-byte aligned, owned by the caller
 * Requires 0 <= t0 <= t1 <= src->T_cap (t0 == t1 is a no-op); paged caches
 * read through their block table (entries of the range must be valid).
 * Errors: TQ_ERR_INVALID_ARGUMENT / _UNSUPPORTED / _ALIGNMENT before any
 * launch, TQ_ERR_DEVICE when the launch fails.
 */
int tq_dequantize(const tq_cache* src, int64_t t0, int64_t t1, float* out, void* hip_stream);

/*
 * Decode attention of one query per head over the packed caches:
 *   out[b][h] = sum_{t < ctx_len[b]} softmax_t(scale * q[b][h] . k_hat[b][h/G][t]) v_hat[b][h/G][t]
 * with k_hat, v_hat the reconstructions of tq_dequantize. Attention reads the
 * compressed cache itself (ai-accelerate.xyz TurboQuant article, section
 * "TurboQuantの仕組み": the rotation of step 1 is orthogonal, so a query dotted
 * with a rotated-back key equals the rotated query dotted with the stored
 * levels, and a sum of rotated-back values is one rotation of the sum; step 2's
 * sign bits give the unbiased QJL correction of each score; the thefrontairview
 * piece ties the claimed speedup to attention over the compressed keys).
 * It is computed in the rotated domain (q' = Pi_K q once; scores from key codebook
 * levels times key norms, plus the QJL term for QJL keys; values summed in the
 * rotated domain; out = Pi_V^T o'). G = H_q / H_kv query heads share KV head
 * h / G. Work is split over the context (n_split chunks per (row, KV head),
 * 0 = chosen by the library) and merged in a fixed order, so results do not
 * depend on timing.
 *   q:        device [B][H_q][d], TQ_F32 or TQ_BF16
 *   ctx_lens: device int32 [B] (each in 0..T) or NULL (= T for every row);
 *             a row with ctx_len 0 gets a zero output
 *   T:        largest context length, T <= k->T_cap and T <= v->T_cap
 *   scale:    score scale; <= 0 selects 1/sqrt(d)
 *   out:      device float32 [B][H_q][d]
 *   workspace: device, at least tq_decode_workspace_bytes(...) bytes, 256-byte aligned
 * Requires k->role == TQ_KEYS, v->role == TQ_VALUES, equal B, H_kv and d,
 * H_q % H_kv == 0 and G <= 16. At d = 256 with G > 8 the decode is one launch
 * of float32 arithmetic throughout (n_split, workspace and workspace_bytes are
 * ignored; the workspace may be NULL). On the scan tiles, value norms may have any overall scale: the
 * float16 weights of the value sum are scaled per wavefront by a power of two
 * taken from the largest value norm of its first 32 tokens, so within one
 * (row, KV head) the largest value norm must stay below 7e5 times the
 * smallest nonzero one (below 7e5 outright when 32 zero value vectors open a
 * wavefront's share of the context).
 * Errors: TQ_ERR_INVALID_ARGUMENT / _UNSUPPORTED / _ALIGNMENT /
 * _WORKSPACE_TOO_SMALL before any launch, TQ_ERR_DEVICE when a launch fails.
 * The caller owns every buffer; the workspace holds the context-chunk partials
 * and may be reused by the next call once this one has run on the stream.
 */
int tq_decode_attention(const tq_cache* k, const tq_cache* v,
                        const void* q, int32_t q_dtype, int64_t H_q,
                        const int32_t* ctx_lens, int64_t T, float scale, int32_t n_split,
                        float* out, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * tq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments (minus workspace and
 * workspace_bytes), requirements, errors and results, bit for bit, as
 * tq_decode_attention. The context-chunk partials go to a library-owned
 * static device array of TQ_NOALLOC_SCRATCH_BYTES bytes: each GPU the library
 * runs on holds its own copy until the process ends, looked up on the first
 * call on that device. Calls whose partials would exceed it return
 * TQ_ERR_WORKSPACE_TOO_SMALL before any HIP call (tq_decode_workspace_bytes
 * gives the size a call needs; a single-chunk plan needs none). The call makes
 * no allocation of any kind. Every call on one GPU shares the array: calls that
 * overlap on one GPU (different streams or threads without ordering) race and
 * give undefined results; calls ordered on one stream are safe. Nothing in the
 * array needs clearing between calls (a call writes every partial it reads).
 */
#define TQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int tq_decode_attention_noalloc(const tq_cache* k, const tq_cache* v,
                                const void* q, int32_t q_dtype, int64_t H_q,
                                const int32_t* ctx_lens, int64_t T, float scale, int32_t n_split,
                                float* out, void* hip_stream);

/*
 * One decode step in one call: for every row b with context length
 * ctx_b = clamp(ctx_lens[b], 0, T) (or T) >= 1, the new key and value of each
 * KV head are written to token ctx_b - 1 of k and v (the same bytes as
 * tq_quantize_kv / tq_append_kv at that position), then out is
 * tq_decode_attention over tokens 0 .. ctx_b - 1, which include the new one
 * (the same output, bit for bit, as tq_append_kv followed by
 * tq_decode_attention). Rows with ctx_b = 0 get no write and a zero output.
 * d = 128 keys without a QJL sketch: one launch (the decode kernel writes the
 * new token itself before reading it); otherwise an append launch, then the
 * decode launch, ordered on the stream.
 *   k_new, v_new: device, element (b, h, j) at k_new[b*k_stride_b + h*k_stride_h + j]
 *                 (and the same for v_new), dtype new_dtype (TQ_F32 or TQ_BF16),
 *                 16-byte aligned rows
 * Other arguments and requirements as tq_decode_attention. Keys with a QJL
 * sketch are appended by the tiled quantize kernel, which needs ctx_lens ==
 * NULL (TQ_ERR_UNSUPPORTED otherwise). The caller owns all buffers; argument
 * errors return before any launch.
 */
int tq_decode_attention_append(const tq_cache* k, const tq_cache* v, const void* k_new, const void* v_new,
                               int32_t new_dtype, int64_t k_stride_b, int64_t k_stride_h,
                               int64_t v_stride_b, int64_t v_stride_h, const void* q, int32_t q_dtype,
                               int64_t H_q, const int32_t* ctx_lens, int64_t T, float scale,
                               int32_t n_split, float* out, void* workspace, size_t workspace_bytes,
                               void* hip_stream);

/*
 * Chunked prefill / multi-query attention over the packed caches: M new
 * tokens per row, whose keys and values are already in the caches (appended
 * with tq_quantize_kv), attend causally to the row's context. Token i of row b
 * sits at position ctx_len[b] - M + i and attends to cache tokens
 * 0 .. ctx_len[b] - M + i, with the decode's computation per (token, head):
 *   out[b][i][h] = sum_{t <= ctx_len[b]-M+i} softmax_t(scale * q[b][i][h] . k_hat[b][h/G][t]) v_hat[b][h/G][t]
 * (a query whose position is negative gets a zero output). M = 1 is
 * tq_decode_attention. A workgroup takes a tile of tokens x the G heads of a KV
 * head as the columns of its MFMA tiles (up to 8, or 16 on the 8-wavefront
 * tile), so the codebook decode of each cache step serves every column of the
 * tile; a row with more tokens than a tile reads the cache once per tile.
 * (The prompt-processing cost of compressed caches is noted in the qxai.app
 * item on Tether QVAC's TurboQuant release.)
 *   q:        device [B][M][H_q][d], TQ_F32 or TQ_BF16
 *   out:      device float32 [B][M][H_q][d]
 *   workspace: device, at least tq_prefill_workspace_bytes(...) bytes, 256-byte aligned
 * Other arguments and requirements as tq_decode_attention; M in 1..65535 and
 * B * ceil(M / tile) <= 65535. At d = 256, M * G <= 8 (TQ_ERR_UNSUPPORTED
 * otherwise); the dense path for many columns is d = 128 only, so d = 64
 * takes the scan tiles for every M.
 */
int tq_prefill_attention(const tq_cache* k, const tq_cache* v,
                         const void* q, int32_t q_dtype, int64_t H_q, int64_t M,
                         const int32_t* ctx_lens, int64_t T, float scale, int32_t n_split,
                         float* out, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes tq_prefill_attention needs at any head dimension; 0 for invalid sizes. */
size_t tq_prefill_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t M, int64_t T,
                                  int32_t n_split, int32_t k_qjl);

/* Number of context chunks tq_decode_attention uses for these sizes (n_split 0 = auto). */
int32_t tq_decode_splits(int64_t B, int64_t H_kv, int64_t T, int32_t n_split);

/* Workspace bytes tq_decode_attention needs at any head dimension; 0 for invalid sizes. */
size_t tq_decode_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t T,
                                 int32_t n_split, int32_t k_qjl);

/*
 * Measurement helper, not a step of the method: reads `bytes` bytes of the
 * device buffer src once with a plain streaming kernel (16-byte loads, each of
 * `workgroups` 256-thread workgroups reading one contiguous slice, the
 * non-temporal cache policy of the decode's streams) and writes one XOR-folded
 * word per workgroup to sink (device uint32 [workgroups]), so that no read is
 * dead. Its rate is the pure read stream the decode's packed-cache rate is
 * compared with. src 16-byte aligned, bytes a nonzero multiple of 16,
 * workgroups in 1..65535 with slices below 2 GiB. Errors before any launch;
 * TQ_ERR_DEVICE when the launch fails.
 */
int tq_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups, void* hip_stream);

/* Static text for a status code. */
const char* tq_status_string(int status);

/* Name of the HIP error (hipGetErrorName) behind the last TQ_ERR_DEVICE that an
 * entry point returned on the calling thread; "hipSuccess" if there was none.
 * Static text, owned by the HIP runtime. */
const char* tq_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H_ */
