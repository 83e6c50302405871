/*
 * qimg.h — C ABI of the shared Q8_1 activation-image library for AMD MI355X (gfx950).
 *
 * An activation producer (RMSNorm, RMSNorm x gamma, SwiGLU or GeGLU-erf) writes its f32
 * output and, in the same pass, a block-quantized Q8_1 image of that output. The image is
 * then read by any number of Q4_0-weight mat-vec projections (MMVQ): ordinary readers and
 * routed MUL_MAT_ID expert slots that process only the live rows of a padded bucket.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "Share temporary Q8_1 activation images" (llama.cpp fork, PR #117):
 *        Overview, Coverage, GLU producer evidence.
 *   [P2] "r49 - A-quantize prepass shared-A dedup: consecutive-window memoization":
 *        section 2 Principle, section 3.1 Design choices.
 *   [P3] "qwen3_5 CUDA: a captured bucket's padding rows no longer go through the routed
 *        experts" (TensorFold PR #1047): What this changes, Receipt.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership.  Every data pointer is device memory owned by the caller. The reader arrays
 *   (qimg_q4_0_reader / qimg_q4_0_expert_reader) are host memory and are copied into the
 *   kernel arguments before the call returns. The library allocates nothing, keeps no
 *   reference after return and holds no mutable global state: an image is refreshed by
 *   every call that writes it, never cached across calls ([P1] Coverage: images refresh on
 *   every execution; [P2] section 2: no cache persists across executions).
 * Execution.  Calls enqueue work on `stream` (a hipStream_t; NULL is the default stream)
 *   and return without synchronising. They never read device memory on the host, so they
 *   may be recorded into a HIP graph. The live-row count is read on the device at run time,
 *   so one recorded graph serves every live count ([P3] What this changes).
 * Errors.  A negative status means the arguments were rejected on the host and nothing was
 *   enqueued. QIMG_EHIP means a HIP launch failed; the stream state is then undefined.
 *   Errors found on the device are reported through the routed workspace error word.
 * Sizes.  K (the reduction width) must be a positive multiple of 32 (one Q8_1 block):
 *   [P1] Coverage requires whole Q8_1 blocks for output and image row widths.
 *   K <= QIMG_MAX_K. Row strides are in elements and must keep 16-byte alignment.
 *
 * Data layouts
 * ------------
 * Q8_1 image (one allocation, two planes; rows = producer rows, RB = qimg_row_blocks(K)):
 *   codes plane : int8  codes[rows][RB][32]            at byte 0
 *   ds plane    : uint32 ds[rows][RB]                  at byte rows*RB*32
 *                 low half = fp16 d (block scale amax/127), high half = fp16 s (d * sum of
 *                 the block's codes), little-endian.
 *   Blocks K/32 <= b < RB of every live row are written as zero bytes (row padding to a
 *   multiple of 16 blocks, i.e. 512 elements). Rows >= live count are never written.
 * Q4_0 weights, standard order (the input of qimg_q4_0_tile; one reader or one expert):
 *   qs plane : uint8  qs[N][K/32][16]; byte j of a block holds element j in its low nibble
 *              and element j+16 in its high nibble.
 *   d plane  : fp16   d[N][K/32]; weight = d * (nibble - 8).
 *   Routed readers stack E experts: qs[E][N][K/32][16], d[E][N][K/32].
 * Q4_0 weights, reader tiles (made once by qimg_q4_0_tile, read by the readers): rows are cut
 *   into 16-row tiles, K/32 blocks into chunks of 4 (padding rows and blocks are zero). With
 *   TL = ceil(N/16), KC = ceil(K/128) and chunk c = (e*TL + tile)*KC + s:
 *   codes : bytes [c*1024 + 16*l, +16) = block 4*s + l/16 of row 16*tile + l%16, l < 64
 *   scales: fp16 at byte E*TL*KC*1024 + 2*(c*64 + l), same (row, block)
 *   The same blocks as the standard order, reordered so that one 64-lane load moves 1 KB of
 *   contiguous weights.
 */
#ifndef QIMG_H
#define QIMG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QIMG_ABI_VERSION 12

/* status codes */
#define QIMG_OK 0
#define QIMG_EINVAL (-1)       /* null required pointer, bad size, bad op code */
#define QIMG_EALIGN (-2)       /* a plane base or stride breaks the required alignment */
#define QIMG_EALIAS (-3)       /* an output overlaps an input or another output */
#define QIMG_EUNSUPPORTED (-4) /* shape outside the supported range (e.g. K > QIMG_MAX_K) */
#define QIMG_EWORKSPACE (-5)   /* routed workspace missing or smaller than required */
#define QIMG_EHIP (-6)         /* a HIP runtime call failed */

#define QIMG_MAX_K 32768
#define QIMG_MAX_READERS 8
#define QIMG_MAX_EXPERTS 1024       /* routed readers: E */
#define QIMG_MAX_ROUTED_PAIRS 4096  /* routed readers: bucket * top_k */
#define QIMG_MAX_TOPK 64            /* qimg_moe_topk: top_k */

/* GLU producer formulas ([P1] Coverage: F32 ReGLU, GeGLU, SwiGLU, GeGLU-erf, GeGLU-quick,
 * SwiGLU-OAI and SwiGLU-clamp producers). g = gate, u = up; the last two take alpha and limit
 * (qimg_emit_glu_ex) and clamp g' = min(g, limit), u' = clamp(u, -limit, limit). */
#define QIMG_GLU_SWIGLU 0       /* y = g / (1 + exp(-g)) * u                                  */
#define QIMG_GLU_GEGLU_ERF 1    /* y = 0.5 * g * (1 + erf(g / sqrt(2))) * u                   */
#define QIMG_GLU_REGLU 2        /* y = max(g, 0) * u                                          */
#define QIMG_GLU_GEGLU 3        /* y = 0.5 * g * (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) * u */
#define QIMG_GLU_GEGLU_QUICK 4  /* y = g / (1 + exp(-1.702 g)) * u                            */
#define QIMG_GLU_SWIGLU_OAI 5   /* y = g' / (1 + exp(-alpha g')) * (u' + 1)                   */
#define QIMG_GLU_SWIGLU_CLAMP 6 /* y = g' / (1 + exp(-g')) * u'                               */

/* Routed workspace error-word bits (set on the device, read by the caller after sync). */
#define QIMG_ERR_EXPERT_RANGE 1 /* a live pair named an expert outside [0, E); it was skipped */
#define QIMG_ERR_LIVE_CLAMPED 2 /* *live_rows was above the bucket size (or negative); clamped */

/* Human-readable text for a status code. Never returns NULL. */
const char* qimg_strerror(int status);

/* QIMG_ABI_VERSION of the loaded library. */
int qimg_abi_version(void);

/* Image row blocks RB = round_up(K/32, 16); 0 when K is not a positive multiple of 32. */
int32_t qimg_row_blocks(int32_t K);

/* Bytes of an image of `rows` rows: rows * RB * 36; 0 on a bad K or rows < 0. */
int64_t qimg_image_bytes(int32_t rows, int32_t K);

/*
 * RMSNorm producer ([P1] Coverage: RMS-alone and RMS+MUL producers emit images while every
 * original F32 store remains). For each live row i (i < live, live = *live_rows clamped to
 * [0, rows], or rows when live_rows is NULL):
 *   S = sum of x[i][k]^2 in the library's fixed reduction order; r = 1/sqrt(S/K + eps)
 *   y[i][k] = (x[i][k] * r) * gamma[k]        (gamma == NULL: y = x * r)
 * and, when img != NULL, the Q8_1 image row i of y (see qimg_quantize_q8_1 for the block
 * rule). img == NULL writes y only: the separate-quantizer ("original") arm.
 *   x     : f32 [rows][ldx], 16-byte aligned, ldx % 4 == 0, ldx >= K
 *   gamma : f32 [K], 16-byte aligned, or NULL
 *   y     : f32 [rows][ldy], 16-byte aligned, ldy % 4 == 0, ldy >= K; must not overlap x,
 *           gamma or img
 *   img   : qimg_image_bytes(rows, K) bytes, 16-byte aligned, or NULL; must not overlap y or
 *           live_rows (QIMG_EALIAS). An img that overlaps the producer's inputs is declined
 *           (below).
 *   live_rows : device int32, or NULL
 * Rows >= live are not read and not written.
 *
 * Declined emission ([P1] Coverage: unsafe input/output aliases keep the original
 * preparation). Emitting while the producer runs is unsafe when img overlaps one of its inputs
 * (x, gamma, beta; gate, up for the GLU producers), since workgroups still reading an input
 * would see image bytes. Such a call is not rejected: it enqueues the original two steps on
 * `stream`, the producer writing y alone and then the separate quantizer (qimg_quantize_q8_1)
 * reading y into img, and returns QIMG_OK. The bytes of y and img are those of an emitting
 * call on non-overlapping buffers. This holds for every producer entry point below.
 */
int qimg_emit_rmsnorm(const float* x, int64_t ldx, const float* gamma, float eps, int32_t rows,
                      const int32_t* live_rows, int32_t K, float* y, int64_t ldy, void* img,
                      void* stream);

/*
 * RMS+MUL+ADD and RMS+SCALE producers ([P1] Coverage: RMS+MUL+ADD and RMS+SCALE producers
 * emit images): as qimg_emit_rmsnorm with
 *   t = x * r; t = t * gamma[k] (gamma != NULL); t = t + beta[k] (beta != NULL);
 *   y[i][k] = t * scale
 * each one f32 rounding in that order (scale = 1 and beta = NULL give qimg_emit_rmsnorm).
 *   beta  : f32 [K], 16-byte aligned, or NULL; must not overlap y or img
 *   scale : finite (QIMG_EINVAL otherwise)
 */
int qimg_emit_rmsnorm_ex(const float* x, int64_t ldx, const float* gamma, const float* beta,
                         float scale, float eps, int32_t rows, const int32_t* live_rows,
                         int32_t K, float* y, int64_t ldy, void* img, void* stream);

/*
 * GLU producer ([P1] Coverage: F32 SwiGLU and GeGLU-erf producers with separate or packed
 * inputs emit images; original F32 outputs remain). For live rows i and k < K:
 *   g = gate[i*ldg + k], u = up[i*ldu + k], y[i][k] = act(g) * u
 * with act per `op` (QIMG_GLU_*). Packed gate|up input: gate = gu, up = gu + K, ldg = ldu = 2K.
 *   gate, up : f32, 16-byte aligned, strides % 4 == 0
 *   y, img, live_rows : as for qimg_emit_rmsnorm
 */
int qimg_emit_glu(int32_t op, const float* gate, int64_t ldg, const float* up, int64_t ldu,
                  int32_t rows, const int32_t* live_rows, int32_t K, float* y, int64_t ldy,
                  void* img, void* stream);

/*
 * Every GLU producer (QIMG_GLU_* 0..6) with its parameters: as qimg_emit_glu, y = the op's
 * formula of (gate, up). alpha and limit are used by QIMG_GLU_SWIGLU_OAI and
 * QIMG_GLU_SWIGLU_CLAMP only (alpha finite, limit >= 0, else QIMG_EINVAL); qimg_emit_glu
 * rejects those two ops. Packed-swapped input (up half first): gate = gu + K, up = gu.
 */
int qimg_emit_glu_ex(int32_t op, float alpha, float limit, const float* gate, int64_t ldg,
                     const float* up, int64_t ldu, int32_t rows, const int32_t* live_rows,
                     int32_t K, float* y, int64_t ldy, void* img, void* stream);

/*
 * The separate activation quantizer: the launch the fused producers remove ([P1] Overview),
 * kept as the control arm and as the fallback when emission is declined. For each live row
 * and each 32-element block of y:
 *   amax = max |y|; d = amax / 127; id = 1/d; c = round-half-away-from-zero(y * id)
 *   d16 = fp16(d); s16 = fp16((float)(sum of c) * d)    (both round-to-nearest-even)
 * A block whose amax is 0 (or whose 1/d is not finite) is all zero bytes. Produces the same
 * bytes as the fused producers' image of the same y.
 *   y   : f32 [rows][ldy], 16-byte aligned, ldy % 4 == 0
 *   img : qimg_image_bytes(rows, K) bytes, 16-byte aligned; must not overlap y
 */
int qimg_quantize_q8_1(const float* y, int64_t ldy, int32_t rows, const int32_t* live_rows,
                       int32_t K, void* img, void* stream);

/* Bytes of the tiled weights of N rows x K (E experts; 1 for an ordinary reader); 0 on bad
 * arguments. */
int64_t qimg_q4_0_tiled_bytes(int32_t N, int32_t K, int32_t E);

/*
 * Reorder standard Q4_0 planes (qs, d; E experts of N rows) into reader tiles. A one-time
 * weight preparation, not part of the per-token path. tiled: qimg_q4_0_tiled_bytes(N, K, E)
 * bytes, 16-byte aligned, must not overlap qs or d. qs 16-byte aligned, d 2-byte aligned.
 */
int qimg_q4_0_tile(const void* qs, const void* d, int32_t N, int32_t K, int32_t E, void* tiled,
                   void* stream);

/* One ordinary Q4_0 reader of an image. */
typedef struct {
  const void* w;   /* tiled weights (qimg_q4_0_tile, E = 1), 16-byte aligned */
  int32_t N;       /* output rows (> 0) */
  int32_t reserved;
  float* out;      /* f32, out[t * ldo + n] for image row t, n < N; 4-byte aligned */
  int64_t ldo;     /* >= N */
} qimg_q4_0_reader;

/*
 * Ordinary MMVQ readers ([P1] Coverage: ordinary MUL_MAT on its MMVQ path with arbitrarily
 * many compatible readers of one image). One launch serves up to QIMG_MAX_READERS readers:
 *   out_r[t][n] = sum over blocks b of d_w[n][b] * (d16[t][b] * sumi - 8 * s16[t][b])
 *   sumi = sum_{j<16} (qs[n][b][j] & 15) * c[t][b][j] + (qs[n][b][j] >> 4) * c[t][b][j+16]
 * (qs, d_w: the reader's weights in standard order; the reader takes them tiled) for image
 * rows t < live (live as above; rows = image rows). Rows t >= live of every out are not
 * written. Outputs must not overlap each other, the image or the weights. A reader's tiled
 * code plane (N*K/2 bytes, rounded up to whole tiles and chunks; Q8_0: N*K) must stay under
 * 4 GiB (QIMG_EUNSUPPORTED otherwise).
 */
int mmvq_q4_0_q8_1(const qimg_q4_0_reader* readers, int32_t n_readers, const void* img,
                   int32_t rows, const int32_t* live_rows, int32_t K, void* stream);

/* One routed (MUL_MAT_ID) Q4_0 reader over E stacked experts. */
typedef struct {
  const void* w;   /* tiled weights of all E experts (qimg_q4_0_tile), 16-byte aligned */
  int32_t N;       /* output rows per expert (> 0) */
  int32_t reserved;
  float* out;      /* f32, out[(row * top_k + slot) * ld_pair + n] */
  int64_t ld_pair; /* >= N */
} qimg_q4_0_expert_reader;

/* Workspace bytes mmvq_id_q4_0_q8_1 needs: 16 + 4*(E + (E+1) + bucket*top_k), 256-rounded. */
size_t mmvq_id_workspace_bytes(int32_t bucket, int32_t top_k, int32_t E);

/*
 * Routed MMVQ readers ([P1] Coverage: quantized MUL_MAT_ID on its MMVQ path; the image is
 * independent of route ids and serves ID-distinct readers. [P3] What this changes: only the
 * first live rows' pairs are planned; padding rows get no picks, no plan items, no expert
 * work and no writes; launches stay sized for the bucket and read the live count at run time).
 * For every live pair p = row*top_k + slot (row < live, e = ids[p] in [0, E)):
 *   out_r[p][n] = the ordinary reader formula with expert e's weights and image row `row`.
 *   ids       : device int32 [bucket][top_k] (the whole buffer may be read); entries of padding
 *               rows are never used
 *   live_rows : device int32 (clamped to [0, bucket]), or NULL for all bucket rows
 *   img       : image with `bucket` rows
 *   workspace : device, >= mmvq_id_workspace_bytes(bucket, top_k, E), 16-byte aligned.
 *     Fully rewritten by every call (no clearing needed) with the routing plan:
 *       int32 word 0: error bits (QIMG_ERR_*), word 1: live pair count P = live*top_k,
 *       words 2..3: reserved,
 *       int32 counts[E]   : live pairs per expert
 *       int32 offsets[E+1]: exclusive prefix of counts (offsets[E] = valid live pairs)
 *       int32 members[P]  : pair ids grouped by ascending expert, ascending within an expert
 * Pair outputs are independent of which other pairs share an expert, so a live row's outputs
 * equal those of a one-row call on the same data, bit for bit ([P3] Receipt).
 */
int mmvq_id_q4_0_q8_1(const qimg_q4_0_expert_reader* readers, int32_t n_readers, int32_t E,
                      const void* img, const int32_t* ids, int32_t bucket, int32_t top_k,
                      const int32_t* live_rows, int32_t K, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Routed readers for callers that cannot allocate device memory (code recorded under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): mmvq_id_q4_0_q8_1 with the
 * same arguments minus the workspace. The routing plan is kept in a static device array of the
 * library, one per GPU, of QIMG_NOALLOC_SCRATCH_BYTES (enough for QIMG_MAX_ROUTED_PAIRS pairs and
 * QIMG_MAX_EXPERTS experts); the call allocates nothing. The array of the current device is used
 * (the stream must belong to it); its address is looked up once per device on the first call.
 * Every call on one GPU shares that array and rewrites it entirely, so calls that overlap in
 * time on one GPU (two streams, parallel graph branches) race and must not be made; calls
 * ordered on one stream are safe. Results equal those of mmvq_id_q4_0_q8_1 bit for bit.
 * Errors: as mmvq_id_q4_0_q8_1; QIMG_EUNSUPPORTED when the plan would not fit the array;
 * QIMG_EHIP when the array's address cannot be obtained.
 */
#define QIMG_NOALLOC_SCRATCH_BYTES 25600
int mmvq_id_q4_0_q8_1_noalloc(const qimg_q4_0_expert_reader* readers, int32_t n_readers, int32_t E,
                              const void* img, const int32_t* ids, int32_t bucket, int32_t top_k,
                              const int32_t* live_rows, int32_t K, void* stream);

/*
 * The rest of a routed MoE FFN after the gate and up projections ([P1] Coverage: GLU
 * producers emit images, routed MUL_MAT_ID readers on MMVQ, per-slot routed projections;
 * [P3] What this changes: padding rows get no expert work and no combine, their outputs stay
 * unwritten). Rows are (token, slot) pairs p = row*top_k + slot; the pairs of live tokens
 * (row < *live_rows, clamped to [0, bucket]) are live.
 *
 * qimg_emit_glu_per_slot: the GLU producer of qimg_emit_glu over bucket*top_k pair rows,
 *   usually gate = the gate reader's out, up = the up reader's out, ldg = ldu = ld_pair.
 *   Writes y and the image rows of live pairs only; img holds bucket*top_k rows
 *   (qimg_image_bytes(bucket*top_k, K)). Rows of a live pair whose expert was out of range
 *   hold whatever the gate/up outputs held (the routed readers skip such pairs).
 *   bucket*top_k <= QIMG_MAX_ROUTED_PAIRS.
 * mmvq_id_q4_0_q8_1_per_slot: mmvq_id_q4_0_q8_1 over a per-slot image: live pair p reads
 *   image row p (not its token's row); img has bucket*top_k rows. Same workspace, plan and
 *   errors as mmvq_id_q4_0_q8_1.
 * qimg_moe_combine: for live rows t and n < N,
 *   out[t*ldo + n] = sum over slots s = 0..top_k-1 with ids[t*top_k+s] in [0, E) of
 *                    weights[t*top_k+s] * x[(t*top_k+s)*ld_pair + n],
 *   accumulated in f32 as acc = fma(w, x, acc) from +0 in ascending slot order (the pages fix
 *   no order; this one makes the result independent of the launch shape).
 *   x: f32 [bucket*top_k][ld_pair] (the down reader's out), 16-byte aligned, ld_pair % 4 == 0;
 *   weights: f32 [bucket][top_k] routing weights; ids: int32 [bucket][top_k];
 *   out: f32 [bucket][ldo], 16-byte aligned, ldo % 4 == 0, must not overlap any input.
 *   N % 4 == 0 (QIMG_EUNSUPPORTED otherwise). Padding rows of out are not written.
 */
int qimg_emit_glu_per_slot(int32_t op, const float* gate, int64_t ldg, const float* up,
                           int64_t ldu, int32_t bucket, int32_t top_k, const int32_t* live_rows,
                           int32_t K, float* y, int64_t ldy, void* img, void* stream);
int mmvq_id_q4_0_q8_1_per_slot(const qimg_q4_0_expert_reader* readers, int32_t n_readers,
                               int32_t E, const void* img, const int32_t* ids, int32_t bucket,
                               int32_t top_k, const int32_t* live_rows, int32_t K,
                               void* workspace, size_t workspace_bytes, void* stream);
int qimg_moe_combine(const float* x, int64_t ld_pair, const float* weights, const int32_t* ids,
                     int32_t E, int32_t bucket, int32_t top_k, const int32_t* live_rows,
                     int32_t N, float* out, int64_t ldo, void* stream);

/*
 * Device router and top-k with live-row guards ([P3] What this changes: router and top-k take
 * the live count and skip padding rows, which get no picks; their outputs stay unwritten).
 *
 * qimg_moe_router: logits[t*ldl + e] = sum over k < K of x[t*ldx + k] * w[e*K + k] for live
 *   rows t (t < *live_rows clamped to [0, bucket]; all rows when live_rows is NULL), in a
 *   fixed order: leaf c = fma(x3,w3, fma(x2,w2, fma(x1,w1, x0*w0))) over elements 4c..4c+3;
 *   lane l of 64 owns leaves c = l + 64 j, j < Jp (Jp = the next power of two >= ceil(K/256),
 *   missing leaves +0) and sums them by a balanced pairwise tree over j; the 64 lane sums are
 *   then added by a balanced pairwise tree over the lanes. This is the RMS producer's sum of
 *   squares with products in place of squares, so the logits, and every pick made from them,
 *   are reproducible bit for bit whatever the launch shape.
 *   x: f32, 16-byte aligned, ldx % 4 == 0, ldx >= K (the kept f32 output of a producer is the
 *   usual input); w: f32 [E][K], 16-byte aligned; logits: f32 [bucket][ldl], ldl >= E, must not
 *   overlap x, w or live_rows. K: as for the producers.
 * qimg_moe_topk: for live rows t, ids[t*top_k + r] = the expert with the r-th largest logit
 *   (equal logits: lower id first), r < top_k, and, when weights != NULL, the softmax over the
 *   selected logits: e_r = exp(l_r - l_0) (the library's exp), s = e_0 + ... + e_{k-1} in
 *   ascending r, weights[t*top_k + r] = e_r / s. Live logits must not be NaN.
 *   1 <= top_k <= min(E, QIMG_MAX_TOPK); E <= QIMG_MAX_EXPERTS (QIMG_EUNSUPPORTED beyond).
 *   ids: int32 [bucket][top_k]; weights: f32 [bucket][top_k] or NULL; neither may overlap
 *   logits, live_rows or each other.
 */
int qimg_moe_router(const float* x, int64_t ldx, const float* w, int32_t E, int32_t bucket,
                    const int32_t* live_rows, int32_t K, float* logits, int64_t ldl, void* stream);
int qimg_moe_topk(const float* logits, int64_t ldl, int32_t E, int32_t bucket,
                  const int32_t* live_rows, int32_t top_k, int32_t* ids, float* weights,
                  void* stream);

/*
 * Extra floating reader of a producer's kept f32 output ([P1] Coverage: every original F32
 * store remains, including live outputs and extra floating readers). For live rows t (as for
 * qimg_moe_router) and n < N:
 *   out[t*ldo + n] = sum over k < K of y[t*ldy + k] * v[n*K + k]
 * in qimg_moe_router's fixed order (so the result is reproducible bit for bit); the same
 * kernel, named for a consumer that reads y in f32 beside the Q8_1 readers of its image.
 *   y: f32, 16-byte aligned, ldy % 4 == 0, ldy >= K; v: f32 [N][K], 16-byte aligned;
 *   out: f32 [rows][ldo], ldo >= N, must not overlap y, v or live_rows. K: as for the producers.
 */
int qimg_f32_reader(const float* y, int64_t ldy, const float* v, int32_t N, int32_t rows,
                    const int32_t* live_rows, int32_t K, float* out, int64_t ldo, void* stream);

/*
 * Prefill readers: Q4_0 x Q8_1 over many image rows (a prompt's tokens) on the matrix cores,
 * one product per 32-value block ([P2] section 2 Principle: the activation of the q/k/v
 * projections is quantized once and its image read by every projection). Same arguments,
 * layouts (Q4_0 reader tiles), errors and output formula as mmvq_q4_0_q8_1; the results agree
 * with it to the float rounding bound (the sums are ordered differently). mmvq_q4_0_q8_1 itself
 * takes this path when rows >= 64.
 */
int mmq_q4_0_q8_1(const qimg_q4_0_reader* readers, int32_t n_readers, const void* img,
                  int32_t rows, const int32_t* live_rows, int32_t K, void* stream);

/*
 * Other weight formats of the ordinary readers ([P1] Coverage: quantized MUL_MAT on the MMVQ
 * path reads the shared Q8_1 image; the image's half sums carry a format's block minimum).
 *   Q8_0 standard planes: qs int8 [E][N][K/32][32], d fp16 [E][N][K/32]; weight = d * q.
 *     Reader: out[t][n] = sum_b d_w d_a sum_j q_j c_j.
 *     Tiles: chunk c holds 2 KB of codes (the first 16 bytes of each lane's block, then the
 *     second 16) instead of 1 KB; fp16 scales after all codes as for Q4_0.
 *   Q4_1 standard planes: qs [E][N][K/32][16] (Q4_0's nibble order), d and m fp16;
 *     weight = d * q + m (q in 0..15).
 *     Reader: out[t][n] = sum_b (d_w d_a sum_j q_j c_j + m_w s_a), s_a the image's stored sum.
 *     Tiles: codes as Q4_0; then the 32-bit words d | m << 16 after all codes.
 * The readers take the same arguments, errors and aliasing rules as mmvq_q4_0_q8_1, with
 * qimg_reader.w pointing at tiles of the matching format; every reader of one call has that
 * format. Accuracy: as mmvq_q4_0_q8_1 (float sums of exact per-block integer dots).
 */
int64_t qimg_q8_0_tiled_bytes(int32_t N, int32_t K, int32_t E);
int64_t qimg_q4_1_tiled_bytes(int32_t N, int32_t K, int32_t E);
int qimg_q8_0_tile(const void* qs, const void* d, int32_t N, int32_t K, int32_t E, void* tiled,
                   void* stream);
int qimg_q4_1_tile(const void* qs, const void* d, const void* m, int32_t N, int32_t K, int32_t E,
                   void* tiled, void* stream);
int mmvq_q8_0_q8_1(const qimg_q4_0_reader* readers, int32_t n_readers, const void* img,
                   int32_t rows, const int32_t* live_rows, int32_t K, void* stream);
int mmvq_q4_1_q8_1(const qimg_q4_0_reader* readers, int32_t n_readers, const void* img,
                   int32_t rows, const int32_t* live_rows, int32_t K, void* stream);

/*
 * Debug export of the per-block integer dot products of one ordinary reader, computed by the
 * same device code the readers run (the matrix-core dot of each weight block with each image
 * row): sumi[t][n][b] (int32, [rows][N][K/32]) for all image rows t < rows. sumi must not
 * overlap the image or the weights.
 */
int mmvq_q4_0_q8_1_blockdots(const qimg_q4_0_reader* reader, const void* img, int32_t rows,
                             int32_t K, int32_t* sumi, void* stream);

/*
 * Check export of the producers' activation math ([P1] Coverage: F32 SwiGLU and GeGLU-erf
 * producers keep their formulas; the pages give no exp or erf, so the library fixes one f32
 * operation sequence for each and the producers inline it).
 * For i < n, out[i] = f(x_i), where x_i is the f32 whose bit pattern is first_bits + i
 * (mod 2^32), so n = 2^32 with first_bits = 0 covers every f32 input once.
 *   fn QIMG_MATH_EXP    : exp_q(x)            (e^x)
 *   fn QIMG_MATH_ERFC   : erfc_q(x)           (erfc x; the producers call it with x >= 0)
 *   fn QIMG_MATH_SWIGLU : x / (1 + exp_q(-x)) (the SwiGLU activation)
 *   fn QIMG_MATH_GEGLU  : (0.5 x) (1 + erf(x / sqrt 2)) through erfc_q (the GeGLU-erf activation)
 *   fn QIMG_MATH_RSQRT  : 1 / sqrt(x)         (the RMS scale's correctly rounded sqrt and divide)
 *   fn QIMG_MATH_QSCALE : 1 / (x / 127)       (the quantizer's d = amax/127 and 1/d)
 *   fn QIMG_MATH_QDIV   : x / 127             (the quantizer's block scale d alone)
 *   fn QIMG_MATH_F2H    : fp16 bits of x (round to nearest even) in the low half of the
 *                         output word, high half zero (the image's stored d and s)
 * out: device float[n], 4-byte aligned, owned by the caller. 0 <= n <= 2^32; n = 0 is a no-op.
 * Errors: QIMG_EINVAL for a bad fn, n out of range or a null out; QIMG_EALIGN.
 */
#define QIMG_MATH_EXP 0
#define QIMG_MATH_ERFC 1
#define QIMG_MATH_SWIGLU 2
#define QIMG_MATH_GEGLU 3
#define QIMG_MATH_RSQRT 4
#define QIMG_MATH_QSCALE 5
#define QIMG_MATH_QDIV 6
#define QIMG_MATH_F2H 7
int qimg_eval_math(int32_t fn, uint32_t first_bits, int64_t n, float* out, void* stream);

/*
 * Measurement aid, not a step of the method (no page defines it): the rate this GPU streams a
 * plain contiguous buffer at, the ceiling a reader's achieved HBM rate is set against. Reads
 * bytes of buf exactly once: 256 workgroups of 8 waves, each workgroup a contiguous run of
 * 1 KB pieces that its waves take in turn, four 16-byte nontemporal loads in flight per lane.
 * Writes one 32-bit XOR of the data per wave to sink, so that no load is dead.
 *   buf  : device, 16-byte aligned, bytes % 1024 == 0, 0 < bytes < 2^31.
 *   sink : device uint32[QIMG_CEILING_SINK_WORDS], 4-byte aligned, must not overlap buf.
 * Errors: QIMG_EINVAL (null pointer, bytes out of range), QIMG_EALIGN, QIMG_EALIAS, QIMG_EHIP.
 */
#define QIMG_CEILING_SINK_WORDS 2048
int qimg_read_ceiling(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QIMG_H */
