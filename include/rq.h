/*
 * rq.h -- C ABI of the MI355X (gfx950) KV-vector codec: RotorQuant's per-group
 * Cl(3,0) rotor codec and TurboQuant's dense-rotation codec, each optionally
 * with the 1-bit QJL residual stage, plus the q.k estimator over compressed
 * keys.
 *
 * The ABI follows the quantization map Q : R^d -> {0,1}^B and its inverse
 * Q^-1 : {0,1}^B -> R^d (hyper.ai summary of arXiv 2504.19874, section "方法").
 * A session (rq_ctx) fixes d, the bit width, the seed of the random
 * parameters and the mode; quantize / dequantize / roundtrip / score then run
 * asynchronously on a caller's HIP stream over caller-owned device buffers.
 *
 * Conventions that hold for every call below:
 *  - Pointers named x, y, q, codes, norms, signs, rnorms, scores are DEVICE
 *    pointers owned by the caller.  The library never frees or retains them.
 *    rq_host_params and rq_get_params take HOST buffers.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.  The
 *    hot calls only enqueue work; they never synchronise and never allocate.
 *  - Arguments are checked on the host before anything is enqueued.  A failed
 *    check returns a status and writes nothing; rq_last_error() then holds a
 *    message (thread-local, valid until the next failing call on the thread).
 *  - Status: RQ_OK, or RQ_EINVAL (bad argument), RQ_EUNSUPPORTED (a valid but
 *    unimplemented setting, e.g. d != 128), RQ_ENOMEM (allocation failed in
 *    rq_init), RQ_EHIP (a HIP runtime or launch error).  Nothing aborts and no
 *    C++ exception crosses the ABI.
 *  - A ctx may be used by one host thread at a time.  Calls with one ctx on
 *    different streams may run concurrently: the ctx holds only read-only
 *    parameter tables.
 *  - Identical inputs give identical output bytes.
 *
 * Record layout (structure of arrays, one row per vector; all little endian):
 *    codes [n][code_words] uint32  -- MSE codes as ONE bit stream: the code of
 *                                     coordinate i occupies bits
 *                                     [b*i, b*i + b) of the row's words, b the
 *                                     MSE bits; unused tail bits are 0.
 *    norms [n] uint16              -- ||x||_2 as an IEEE half (round to
 *                                     nearest even).
 *    signs [n][4] uint32           -- QJL only: bit j (word j/32, bit j%32)
 *                                     is 1 iff (S r)_j >= 0.
 *    rnorms [n] uint16             -- QJL only: ||r||_2 of the unit-domain
 *                                     residual, as an IEEE half.
 * Rotor sessions code 129 coordinates (43 groups of 3: the 128 inputs and a
 * zero pad; the pad's code is kept because group 42 needs it to invert);
 * dense sessions code 128.
 */
#ifndef RQ_H
#define RQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RQ_ABI_VERSION 1

/* status codes */
#define RQ_OK 0
#define RQ_EINVAL 1
#define RQ_EUNSUPPORTED 2
#define RQ_ENOMEM 3
#define RQ_EHIP 4

/* mode flags (OR-able) */
#define RQ_MSE 0   /* MSE codes only, b bits per coordinate                   */
#define RQ_QJL 1   /* b-1 MSE bits + 1-bit QJL signs of the residual + ||r||;
                      with b = 1 QJL only: no codes, signs of S x_u, gamma  */
#define RQ_DENSE 2 /* TurboQuant: dense 128x128 rotation Pi instead of rotors */
#define RQ_POLAR 4 /* PolarQuant (pq_* functions); alone, with bits = 4       */

/* element types of vector inputs / outputs */
#define RQ_F32 0
#define RQ_F16 1

/* Largest number of query rows one rq_score launch processes; larger hq is
 * processed in chunks of this many rows by the same call. */
#define RQ_SCORE_CHUNK 4096

/* Limits of rq_attend: keys per KV head and query rows per call. */
#define RQ_ATTEND_MAX_KEYS (1 << 23)
#define RQ_ATTEND_MAX_ROWS 65535

typedef struct rq_ctx rq_ctx;

/* Sizes of one session's record (see "Record layout" above). */
typedef struct {
    int32_t d;            /* vector dimension (128)                          */
    int32_t bits;         /* total bits per coordinate                       */
    int32_t mse_bits;     /* bits of the MSE codes: bits, or bits-1 with QJL */
    int32_t mode;         /* RQ_* flags                                      */
    int32_t n_coords;     /* coded coordinates: 129 rotor, 128 dense         */
    int32_t n_groups;     /* rotor groups (43) or 0                          */
    int32_t levels;       /* 2^mse_bits                                      */
    int32_t code_words;   /* ceil(n_coords * mse_bits / 32)                  */
    int32_t sign_words;   /* 4 with QJL, else 0                              */
    int32_t record_bytes; /* 4*code_words + 2 (+ 16 + 2 with QJL)            */
} rq_layout_t;

/* Host copies of a session's parameter tables.  Any member may be NULL (that
 * table is skipped).  Sizes: rotors [n_groups*4] (s, b12, b13, b23 per group:
 * the rotor [s,0,0,0,b12,b13,b23,0] of README "How RotorQuant Works");
 * rotmats [n_groups*9] row-major 3x3 M_g with grade-1((R v) R~) = M_g v;
 * centroids [levels]; boundaries [levels-1] (t_k = (c_k + c_{k+1})/2);
 * pi [d*d] row-major, y = Pi x (dense and polar); s [d*d] half bits
 * row-major, z = S r (QJL only).  RQ_POLAR sessions fill centroids [28] and
 * boundaries [24]: the codebooks of its four levels (16 + 4 + 4 + 4
 * centroids, 15 + 3 + 3 + 3 boundaries) one after another. */
typedef struct {
    float* rotors;
    float* rotmats;
    float* centroids;
    float* boundaries;
    float* pi;
    uint16_t* s;
} rq_params_host_t;

/* Fills *out with the record sizes of (d, bits, mode).  CPU only.
 * RQ_EINVAL for bits outside 1..4 (MSE) / 1..5 (QJL) or unknown mode bits.
 * bits = 1 with RQ_QJL is the QJL-only codec (blog's QJL demo with zero MSE
 * bits: the residual is the whole unit vector, gamma = 1; README "CUDA
 * Kernels" lists its 1-bit quantiser and score kernels): code_words = 0, a
 * 20-byte record, rotor and dense sessions identical (no rotation is used);
 * record code pointers may then be NULL;
 * RQ_POLAR (alone, bits = 4) is PolarQuant: n_coords 128, levels 16 (its
 * first level), code_words 16 and record_bytes 64 for the whole record (see
 * pq_quantize), no norms, signs or residual norms;
 * RQ_EUNSUPPORTED for d != 128. */
int rq_layout(int d, int bits, int mode, rq_layout_t* out);

/* Computes the parameter tables of (d, bits, seed, mode) on the host, with
 * no GPU involved, into the non-NULL buffers of *out.  These are bit-for-bit
 * the tables rq_init uploads.  Generation (float64, each table rounded once):
 *   - SplitMix64 streams per (seed, tag): rotors tag 1, Pi tag 2, S tag 3;
 *     Box-Muller normals.
 *   - rotors: exp of an N(0,1) bivector per group, normalised ("normalized
 *     random bivector exponentials"; README "How RotorQuant Works").
 *   - codebook: Lloyd-Max for the coordinate law of a uniform unit vector in
 *     R^d (blog "Beta 分布", "MSE 标量量化"; README "Codebook Calibration Fix":
 *     d_eff = d).
 *   - Pi: orthogonal factor of a QR of a Gaussian matrix with diag(R) > 0
 *     (README "How TurboQuant Works", Stage 1).
 *   - S: Gaussian, each entry rounded to IEEE half (README Stage 2).
 * Same status rules as rq_layout. */
int rq_host_params(int d, int bits, uint64_t seed, int mode, rq_params_host_t* out);

/* The 256-slot lookup table through which the rotor kernels evaluate the
 * nearest-centroid code #{k : y > t_k} and its centroid (Lloyd-Max codebook
 * of rq_host_params; README "How RotorQuant Works", quantize step).  A
 * unit-domain coordinate y falls in slot
 *   s = (bits(fp32 fma(y, 2032, *bias)) & 0xFF0) / 16,
 * and then code = table[s][0] + (y > thr), thr = bit pattern table[s][1]
 * (+inf if the slot holds no boundary), centroid = y > thr ? table[s][3]
 * : table[s][2] (fp32 bit patterns).  Host only; table is [256][4] u32.
 * Same status rules as rq_layout. */
int rq_host_quantizer(int d, int bits, int mode, float* bias, uint32_t* table);

/* Opens a session on the current HIP device: computes the tables as
 * rq_host_params does, uploads them once (synchronously) and returns the
 * ctx in *out.  On any failure *out is set to NULL and nothing is leaked. */
int rq_init(int d, int bits, uint64_t seed, int mode, rq_ctx** out);

/* Frees a session's device tables.  NULL is a no-op.  The caller must make
 * sure no enqueued work still uses the ctx. */
void rq_free(rq_ctx* ctx);

int rq_get_layout(const rq_ctx* ctx, rq_layout_t* out);
int rq_get_params(const rq_ctx* ctx, rq_params_host_t* out);

/* Q(x) for a rotor session (README "RotorQuant Fused Kernels": normalize ->
 * embed -> rotor sandwich -> quantize; with RQ_QJL also README Stage 2 and
 * hyper.ai Algorithm 2: residual r = x_u - Q_mse^-1(Q_mse(x_u)), signs of
 * S r, ||r||).
 *   x      [n][ldx] elements of x_dtype (RQ_F16 or RQ_F32), 16-byte aligned,
 *          ldx >= 128 and ldx * element size a multiple of 16 bytes and at
 *          most 2^26 bytes.
 *   n      vectors (n == 0 is a no-op returning RQ_OK).
 *   codes  [n][code_words], norms [n]; signs [n][4] and rnorms [n] must be
 *          non-NULL exactly when the session has RQ_QJL.
 * RQ_EINVAL on a dense session (use tq_quantize). */
int rq_quantize(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx,
                uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms,
                void* stream);

/* Q^-1 for a rotor session (README: inverse_sandwich -> extract -> rescale;
 * with RQ_QJL the QJL term sqrt(pi/2)/m * ||r|| * S^T sign(S r) is added
 * before rescaling, blog QJL section item 5).  Writes y [n][ldy] of y_dtype;
 * the record arrays are read.  Alignment rules as for x. */
int rq_dequantize(rq_ctx* ctx, const uint32_t* codes, const uint16_t* norms,
                  const uint32_t* signs, const uint16_t* rnorms, int64_t n,
                  void* y, int y_dtype, int64_t ldy, void* stream);

/* One launch doing rq_quantize and rq_dequantize: writes the record AND the
 * reconstruction (the README's full fused quantize -> dequantize pipeline,
 * section "Triton Kernels" / "Usage", which returns x_hat).  The
 * reconstruction is exactly what rq_dequantize returns for the written
 * record.  x and y must not overlap. */
int rq_roundtrip(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx,
                 uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms,
                 void* y, int y_dtype, int64_t ldy, void* stream);

/* q.k estimates from compressed keys (README estimator:
 *   <q,k> ~ <q,k_mse> + ||r|| sqrt(pi/2)/m <S q, sign(S r)>),
 * for grouped-query attention: query row h reads KV head h / group.
 *   q       [hq][128] fp32 queries, 16-byte aligned.
 *   group   query rows per KV head, 1 <= group <= RQ_SCORE_CHUNK; hq must be
 *           a multiple of group.
 *   codes.. records of hq/group KV heads; head j's t keys start at record
 *           row j * kv_stride (kv_stride >= t, or any value if hq == group).
 *   scores  [hq][ld_scores] fp32, t <= ld_scores <= 2^23; row h gets
 *           n^_t (<q_h, x~_mse,u(t)> + gamma^_t sqrt(pi/2)/m <S q_h, sigma_t>),
 *           raw: no 1/sqrt(d), no softmax.
 * Works for rotor and dense sessions.  The rotated queries and S q are built
 * on chip by the scoring kernel (no workspace); launches take at most
 * RQ_SCORE_CHUNK query rows each. */
int rq_score(rq_ctx* ctx, const float* q, int hq, int group,
             const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
             const uint16_t* rnorms, int64_t t, int64_t kv_stride,
             float* scores, int64_t ld_scores, void* stream);

/* Decode attention read from a compressed cache (PolarQuant article,
 * KV-cache section: attention is softmax(Q K^T / sqrt(d)) V; README, note
 * under "Triton Kernels": the q.k scores come straight from the compressed
 * keys).  For query row h, reading KV head j = h / group:
 *   out[h] = sum_t softmax_t(scale * s_ht) * v~_t
 * with s_ht the rq_score estimate of key t and v~_t what rq_dequantize
 * returns for value t; values are not decoded to vectors (the weighted sums
 * run over centroids and signs, the inverse rotation once per row).
 *   kctx, vctx   sessions of the key and value records (rotor or dense, any
 *                bits and modes; both on the current device).  kctx may also
 *                be an RQ_POLAR session: the keys are then its 16-word
 *                records in kcodes (knorms, ksigns, krnorms NULL) and s_ht is
 *                pq_score's <q_h, x~_t>.  vctx may be an RQ_POLAR session:
 *                the values are then its 16-word records in vcodes (vnorms,
 *                vsigns, vrnorms NULL) and v~_t is pq_dequantize's x~_t
 *                (the weighted sums run over the decoded y~_t, Pi^T once
 *                per row).
 *   q            [hq][128] fp32 queries, 16-byte aligned; hq <= RQ_ATTEND_MAX_ROWS.
 *   group        query rows per KV head, 1 <= group <= RQ_SCORE_CHUNK, hq % group == 0.
 *   k..., v...   records of hq/group KV heads; head j's t keys and values
 *                start at record row j * kv_stride (kv_stride >= t unless
 *                hq == group); 1 <= t <= RQ_ATTEND_MAX_KEYS.
 *   scale        multiplies every estimate before the softmax (1/sqrt(128)
 *                for standard attention); must be finite.
 *   workspace    device memory of at least rq_attend_workspace(hq, group, t)
 *                bytes, 256-byte aligned, owned by the caller; its contents
 *                are scratch (estimates, row statistics, partial sums).
 *   out          [hq][ld_out] fp32, ld_out >= 128.
 * Asynchronous on `stream` (four launches); nothing is allocated.  Errors:
 * RQ_EINVAL for any argument outside these rules (nothing is written),
 * RQ_EHIP for a launch failure.  Deterministic: fixed reduction orders. */
int64_t rq_attend_workspace(int hq, int group, int64_t t);   /* -1 if the sizes are invalid */
int rq_attend(const rq_ctx* kctx, const rq_ctx* vctx, const float* q, int hq, int group,
              const uint32_t* kcodes, const uint16_t* knorms, const uint32_t* ksigns,
              const uint16_t* krnorms, const uint32_t* vcodes, const uint16_t* vnorms,
              const uint32_t* vsigns, const uint16_t* vrnorms, int64_t t, int64_t kv_stride,
              float scale, void* workspace, int64_t workspace_bytes, float* out,
              int64_t ld_out, void* stream);

/* rq_attend for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation, arguments and rules as rq_attend, with the workspace
 * replaced by a fixed device array of RQ_ATTEND_NOALLOC_BYTES that the
 * library holds on each GPU it runs on until the process ends.  Nothing is
 * allocated and no allocating routine is called.  RQ_EINVAL (nothing is
 * enqueued) when rq_attend_workspace(hq, group, t) exceeds
 * RQ_ATTEND_NOALLOC_BYTES, besides rq_attend's own argument errors.  Every
 * call on one GPU uses that GPU's one array: calls on one stream are ordered
 * and safe, but calls that overlap in time on one GPU (other streams, other
 * host threads) race on it and give wrong results. */
#define RQ_ATTEND_NOALLOC_BYTES (64 << 20)
int rq_attend_noalloc(const rq_ctx* kctx, const rq_ctx* vctx, const float* q, int hq, int group,
                      const uint32_t* kcodes, const uint16_t* knorms, const uint32_t* ksigns,
                      const uint16_t* krnorms, const uint32_t* vcodes, const uint16_t* vnorms,
                      const uint32_t* vsigns, const uint16_t* vrnorms, int64_t t, int64_t kv_stride,
                      float scale, float* out, int64_t ld_out, void* stream);

/* Outlier-channel separation for QJL-only keys (sessions with bits = 1 and
 * RQ_QJL, rotor or dense alike).  The README's list of QJL kernels ("CUDA
 * Kernels", "QJL Kernels") gives the one-bit quantiser "outlier separation"
 * and grouped-query score kernels; the blog's random-rotation section
 * (Lemma 1) and the podcast page say LLM vectors carry very large outliers.
 * The pages fix no rule; these calls implement this one:
 *  - a head's outlier channels are the k channels of largest mean |x_j| over
 *    its keys (a tie goes to the lower channel), in increasing order, chosen
 *    once (bulk quantisation) and then fixed;
 *  - a key's values on them are stored as IEEE halves (exact for fp16
 *    input) in `outliers` [n][k];
 *  - the QJL record (norm, signs of S x_u, gamma) is that of the key with
 *    those channels set to 0;
 *  - dequantisation returns the QJL reconstruction with the outlier channels
 *    replaced by the stored values; the score is <q, x~>, i.e.
 *    n^ sqrt(pi/2)/m gamma^ <S q_in, sigma> + sum_i q_{c_i} o^_i with q_in
 *    = q with the outlier channels set to 0.
 * Layout: record row r belongs to head r / head_rows; chans [heads][k]
 * uint8 device array (every entry < 128, increasing within a head); k is
 * 0..RQ_MAX_OUTLIERS (k = 0 is the plain QJL-only codec: chans and outliers
 * may then be NULL).  outliers must be 2-byte aligned.  Other rules as for
 * rq_quantize / rq_dequantize / rq_score; RQ_EINVAL on a session that is not
 * QJL-only. */
#define RQ_MAX_OUTLIERS 16
/* chans[h][0..k) for each of `heads` heads of head_rows consecutive rows of
 * x (x rules as for rq_quantize). */
int rq_outlier_channels(const void* x, int x_dtype, int64_t heads, int64_t head_rows, int64_t ldx, int k,
                        uint8_t* chans, void* stream);
int rq_quantize_outliers(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, int64_t head_rows,
                         int k, const uint8_t* chans, uint16_t* norms, uint32_t* signs, uint16_t* rnorms,
                         uint16_t* outliers, void* stream);
int rq_dequantize_outliers(rq_ctx* ctx, const uint16_t* norms, const uint32_t* signs, const uint16_t* rnorms,
                           const uint16_t* outliers, int64_t n, int64_t head_rows, int k, const uint8_t* chans,
                           void* y, int y_dtype, int64_t ldy, void* stream);
/* Scores as rq_score (query row h reads KV head h / group, whose t keys
 * start at record row (h / group) * kv_stride and whose channel set is
 * chans[h / group]). */
int rq_score_outliers(rq_ctx* ctx, const float* q, int hq, int group, const uint16_t* norms,
                      const uint32_t* signs, const uint16_t* rnorms, const uint16_t* outliers, int k,
                      const uint8_t* chans, int64_t t, int64_t kv_stride, float* scores, int64_t ld_scores,
                      void* stream);

/* Paged compressed KV cache (README "Post-Prefill Quantization": prefill at
 * full precision, one bulk quantisation of the prefill cache, then each
 * decode step stores its new key compressed while the current token's own
 * attention uses the full-precision key; README "Project Structure" names
 * the KV-cache classes this replaces).
 *
 * A cache owns a device pool of `max_pages` pages; a page holds the records
 * of `page_tokens` consecutive tokens of one (layer, KV head), keys (kctx's
 * layout) and values (vctx's layout) alike.  A sequence reserves
 * ceil(max_tokens / page_tokens) pages per (layer, KV head) when opened and
 * gives them back when closed, so its page table is fixed and uploaded once.
 * Inputs go through a staging area of `stage_tokens` tokens per KV head.
 * Every call below runs on the caller's stream except create/free/open/close,
 * which synchronise the device (they are not on the decode path).  Errors:
 * RQ_EINVAL (arguments), RQ_EUNSUPPORTED (value sessions without an MSE
 * stage), RQ_ENOMEM (pool or device memory exhausted), RQ_EHIP. */
typedef struct rq_cache rq_cache;
int rq_cache_create(const rq_ctx* kctx, const rq_ctx* vctx, int layers, int kv_heads,
                    int page_tokens /* power of two, 64..2^20 */, int64_t max_pages,
                    int64_t stage_tokens, rq_cache** out);
void rq_cache_free(rq_cache* cache);
int rq_cache_open(rq_cache* cache, int64_t max_tokens, int* seq);
int rq_cache_close(rq_cache* cache, int seq);
/* Tokens cached for (seq, layer), or -1 for a bad argument. */
int64_t rq_cache_length(const rq_cache* cache, int seq, int layer);
int64_t rq_cache_free_pages(const rq_cache* cache);
/* Quantises n new tokens of every KV head of one layer and stores them after
 * the tokens already cached: k, v [kv_heads][n][ld] fp16 or fp32 (dtype),
 * 16-byte aligned, ld >= 128.  n = prompt length for the bulk prefill,
 * 1 per decode step. */
int rq_cache_append(rq_cache* cache, int seq, int layer, const void* k, const void* v,
                    int dtype, int64_t n, int64_t ld, void* stream);
/* Copies the cached records of one layer back into dense record arrays
 * [kv_heads][length] (which = 0 keys, 1 values); device pointers. */
int rq_cache_read(const rq_cache* cache, int seq, int layer, int which, uint32_t* codes,
                  uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* stream);
/* Workspace rq_cache_attend needs for hq query rows over t cached tokens. */
int64_t rq_cache_attend_workspace(const rq_cache* cache, int hq, int64_t t);
/* rq_attend over the cached tokens of (seq, layer) through the page table
 * (GQA: hq / kv_heads query rows per KV head), and, when k_cur and v_cur are
 * given ([kv_heads][128] fp32, the current token's exact key and value), the
 * current token folded into the same softmax at full precision:
 *   out_h = sum_{t cached} p_t v~_t + p_cur v_cur, p = softmax(scale * [s_h, q_h.k_cur]).
 * With nothing cached, k_cur/v_cur are required and out_h = v_cur. */
int rq_cache_attend(rq_cache* cache, int seq, int layer, const float* q, int hq, float scale,
                    const float* k_cur, const float* v_cur, void* workspace,
                    int64_t workspace_bytes, float* out, int64_t ld_out, void* stream);

/* A decode step over a range of layers in one call each (README "Post-Prefill
 * Quantization": every decode step appends the new token's key and value to
 * every layer's compressed cache and attends with the current token at full
 * precision).  Layers layer0 .. layer0 + nlayers - 1 must hold the same
 * number of cached tokens.  Layouts: k, v [nlayers][kv_heads][n][ld];
 * q [nlayers][hq][128] fp32; k_cur, v_cur [nlayers][kv_heads][128] fp32;
 * out [nlayers * hq][ld_out], row l * hq + h for query head h of layer
 * layer0 + l.  The results equal, bit for bit, those of the per-layer calls
 * (rq_cache_append per layer; rq_cache_attend per layer, whose key slices
 * the layered call reproduces); nlayers * hq <= RQ_ATTEND_MAX_ROWS.
 * Same errors as the per-layer calls. */
int rq_cache_append_layers(rq_cache* cache, int seq, int layer0, int nlayers, const void* k, const void* v,
                           int dtype, int64_t n, int64_t ld, void* stream);
int64_t rq_cache_attend_layers_workspace(const rq_cache* cache, int nlayers, int hq, int64_t t);
int rq_cache_attend_layers(rq_cache* cache, int seq, int layer0, int nlayers, const float* q, int hq, float scale,
                           const float* k_cur, const float* v_cur, void* workspace, int64_t workspace_bytes,
                           float* out, int64_t ld_out, void* stream);

/* TurboQuant comparison path (hyper.ai Algorithms 1 and 2; README "How
 * TurboQuant Works"): y = Pi x_u, per-coordinate Lloyd-Max codes on 128
 * coordinates, x~ = Pi^T y^ (+ the QJL stage with RQ_QJL).  Same arguments
 * and rules as the rq_ functions; the ctx must have RQ_DENSE. */
int tq_quantize(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx,
                uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms,
                void* stream);
int tq_dequantize(rq_ctx* ctx, const uint32_t* codes, const uint16_t* norms,
                  const uint32_t* signs, const uint16_t* rnorms, int64_t n,
                  void* y, int y_dtype, int64_t ldy, void* stream);
int tq_roundtrip(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx,
                 uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms,
                 void* y, int y_dtype, int64_t ldy, void* stream);

/* PolarQuant (PolarQuant article, sections on the polar transform, on the
 * algorithm in practice and on the compression ratio), for RQ_POLAR
 * sessions:
 *   y = Pi x (the session's Pi, the same as a dense session of that seed);
 *   level 1 pairs (y_2i, y_2i+1) -> angle in [0, 2 pi) coded with 4 bits and
 *   radius; levels 2..4 pair the previous radii the same way, angles in
 *   [0, pi/2] coded with 2 bits each (128 -> 64 -> 32 -> 16 -> 8 radii);
 *   codes = #{k : angle > t_k} against each level's Lloyd codebook for the
 *   article's angle law; the 8 final radii are stored as IEEE halves.
 * Record: 16 u32 words per vector, 64 bytes (the article's 496 bits plus 16
 * zero bits): words 0..11 the code bit stream, LSB first (64 level-1 codes
 * of 4 bits, then 32, 16 and 8 codes of 2 bits; bits 368..383 zero), words
 * 12..15 the radii, radius 2i in the low half of word 12 + i.
 * Dequantisation walks the levels back from the radii with the centroid
 * angles (r -> (r cos c, r sin c)) and returns x~ = Pi^T y~; pq_score
 * returns <q_h, x~_t> for every query row and key (no 1/sqrt(d)).
 * Argument rules as for the rq_ functions: x, y [n][ld] fp16 / fp32, words
 * [n][16] 4-byte aligned device memory, n == 0 a no-op; pq_score: q [hq][128]
 * fp32 16-byte aligned, hq <= 65535, query row h reads KV head h / group,
 * whose t records start at row (h / group) * kv_stride (kv_stride >= t
 * unless hq == group), scores [hq][ld_scores] with t <= ld_scores <= 2^23.
 * The rotated queries Pi q are built on chip.  RQ_EINVAL on a session
 * without RQ_POLAR; the rq_, tq_ and cache functions reject RQ_POLAR. */
int pq_quantize(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, uint32_t* words,
                void* stream);
int pq_dequantize(rq_ctx* ctx, const uint32_t* words, int64_t n, void* y, int y_dtype, int64_t ldy,
                  void* stream);
int pq_roundtrip(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, uint32_t* words,
                 void* y, int y_dtype, int64_t ldy, void* stream);
int pq_score(rq_ctx* ctx, const float* q, int hq, int group, const uint32_t* words, int64_t t,
             int64_t kv_stride, float* scores, int64_t ld_scores, void* stream);

/* Measurement reference, not part of the codec: copies `bytes` from src to
 * dst (device pointers, 16-byte aligned, bytes a multiple of 16, no overlap)
 * with the codec kernels' own global access pattern (each wave moves 16 KB
 * blocks as 16-byte non-temporal buffer loads, then 16-byte stores).  Its
 * rate is the practical HBM ceiling that kernel rates are compared with.
 * Asynchronous on `stream`; RQ_EINVAL for bad arguments (nothing is
 * enqueued), RQ_EHIP for a launch failure. */
int rq_bench_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Message of the calling thread's last failure ("" if none). */
const char* rq_last_error(void);

/* Library version string. */
const char* rq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H */
