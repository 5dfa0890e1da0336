/*
 * lnf4.h -- C ABI of the streamed NF4 + LoRA linear for AMD Instinct MI355X (gfx950).
 *
 * The method.  Layer-streamed LoRA fine-tuning keeps the frozen base model out of
 * device memory: per-layer shards live in page-locked host RAM and are copied, one
 * decoder layer at a time, into a few preallocated device buffers by a separate
 * stream while the current layer computes (Soup deep dive, blog.123qwe.co.kr,
 * section "Core feature: how layer streaming works"; Soup 4 GB-laptop article,
 * agentlenshq.com, section "Layer streaming: technical implementation and memory
 * efficiency").  The frozen weights are 4-bit NF4 ("quantization: 4bit", 4 GB-laptop
 * article, section "Configuration and training").  Only the low-rank adapters A, B
 * are trained (20B-RLHF-on-24GB article, agentlenshq.com, section "Low-rank
 * adaptation via PEFT"); in backward the layer must be on the device again because
 * the input gradient is W^T applied to the output gradient (Soup deep dive, same
 * section).
 *
 * Conventions for every entry point.
 *  - All matrices are row-major.  A frozen weight is [out, in] (a PyTorch Linear
 *    weight).  A is [r, in], B is [out, r].  Activations are [T, features].
 *  - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 *  - Every pointer named "device" is a device address (hipMalloc / torch CUDA
 *    tensors); "host" pointers are page-locked host memory where stated.
 *  - Ownership: the caller owns every buffer, workspace and stream.  The library owns
 *    only the lnf4_stream object and the HIP events inside it.  lora_linear_* and
 *    nf4_* never allocate device memory.
 *  - Asynchrony: kernel work is enqueued on the stream argument and returns before it
 *    runs.  Faults inside kernels surface at a later call or the caller's sync.
 *  - Determinism: the same inputs and arguments give bitwise identical outputs, run
 *    to run, and streamed vs resident (no floating-point atomics anywhere).
 *  - Errors: every call returns LNF4_OK (0) or a negative LNF4_E* code and sets a
 *    thread-local message readable with lnf4_last_error().  Argument validation runs
 *    before any HIP call.  No exception crosses the ABI and the library never aborts.
 *  - Size limits: every weight matrix and every activation matrix passed to the GEMM
 *    entry points must span at most 2^31-1 bytes (ESHAPE otherwise); the kernels
 *    address each one through a 31-bit buffer range.
 *  - Not thread-safe per lnf4_stream object.
 */
#ifndef LNF4_H
#define LNF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t; /* same declaration as the HIP runtime's */

#define LNF4_OK 0
#define LNF4_EINVAL (-1) /* null pointer, value out of range (r > 64, nbuf outside 2..8, ...) */
#define LNF4_ESHAPE (-2) /* shape not supported: in % 64 != 0, blocksize != 64, buffer too small */
#define LNF4_EALIGN (-3) /* device pointer not 16-byte aligned, shard section not 256-byte aligned */
#define LNF4_EHIP (-4)   /* a HIP runtime call failed; the message names it */
#define LNF4_ESTATE (-5) /* call out of order, destroyed or finished stream context */

#define LNF4_FMT_NF4 0  /* data = packed codes uint8 [out][in/2], absmax fp32 [out*in/64] */
#define LNF4_FMT_BF16 1 /* data = bf16 [out][in], absmax unused (un-quantized streaming) */

#define LNF4_MAX_RANK 64
#define LNF4_MAX_GROUP 8

/* Message of the last failing call on this thread ("" if none).  Every call checks its
 * arguments and fails loudly rather than running a silently different computation, as
 * the Soup deep dive describes the settings schema rejecting what it cannot apply
 * ("Structure: a CLI whose settings schema is the product"). */
const char* lnf4_last_error(void);

/* Library version string (measurements are tied to a release, as the Soup deep dive ties
 * its numbers to versions: "What the published numbers say and don't say"). */
const char* lnf4_version(void);

/*
 * The 16-entry NF4 code table, fp32, ascending: T[0] = -1, T[7] = 0, T[15] = +1.
 * Levels are standard-normal quantiles: 8 positive at probabilities 1/2 + j(d-1/2)/8
 * (j = 1..8), 7 negative at minus the quantiles of 1/2 + j(d-1/2)/7 (j = 1..7) and 0,
 * all divided by the quantile of d = ((1 - 1/30) + (1 - 1/32)) / 2.  (The pages name
 * the format only; this construction is the normal-quantile NF4 reading.)
 * out: host array of 16 floats.  Runs on the host only.
 */
int lnf4_nf4_table(float out[16]);

/*
 * Decode NF4 to bf16: out[e] = bf16_rne(fp32(T[code(e)] * absmax[e / blocksize])).
 * The decode is the per-layer dequantization that the Soup deep dive ("how layer
 * streaming works") measures as the largest streaming-specific cost.
 *   codes    device, n_elems/2 bytes; byte j holds element 2j (high nibble) and 2j+1 (low)
 *   absmax   device, n_elems/blocksize fp32
 *   n_elems  number of elements, a multiple of blocksize (>= 0; 0 is a no-op)
 *   blocksize must be 64
 *   out_bf16 device, n_elems bf16
 * Bitwise equal to the definition for every code and every finite absmax.
 * Errors: EINVAL (null), ESHAPE (blocksize, n_elems % blocksize), EALIGN (16-byte), EHIP.
 */
int nf4_dequant(const uint8_t* codes, const float* absmax, int64_t n_elems, int32_t blocksize,
                uint16_t* out_bf16, hipStream_t stream);

/*
 * Quantize fp32 weights to NF4 (set-up, off the hot path: shards are built once; the
 * frozen base is stored 4-bit NF4, Soup 4 GB article, "Configuration and training").
 * Blocks of `blocksize` consecutive elements; absmax = max|w| (fp32); code = nearest
 * level to w/absmax (fp32 division and comparison, ties to the lower index); an
 * all-zero block gets code 7.  Packing as in nf4_dequant.
 *   w device fp32 [n_elems]; codes device [n_elems/2]; absmax device [n_elems/blocksize].
 * Errors: as nf4_dequant.
 */
int nf4_quantize(const float* w, int64_t n_elems, int32_t blocksize, uint8_t* codes, float* absmax,
                 hipStream_t stream);

/* A frozen weight of one projection, as it sits in a device layer buffer. */
typedef struct lnf4_weight {
  int32_t fmt;          /* LNF4_FMT_NF4 or LNF4_FMT_BF16 */
  const void* data;     /* device: NF4 codes uint8 [out][in/2] or bf16 [out][in] */
  const float* absmax;  /* device: fp32 [out*in/64] for NF4; ignored for BF16 */
  int64_t out_f, in_f;  /* out >= 1; in a positive multiple of 64 */
  int32_t blocksize;    /* 64 for NF4 (ignored for BF16) */
} lnf4_weight;

/*
 * LoRA linear forward (one projection).  The frozen linear plus the low-rank update
 * scaled by alpha / r (20B-RLHF-on-24GB article, sections "Low-rank adaptation via PEFT"
 * and "Step 2": trainable low-rank A and B beside a frozen W), run on the layer that the
 * stream has just placed on the device (Soup deep dive, "Core feature: how layer
 * streaming works"):
 *   u = x A^T (fp32, [T, r]);   y = bf16( x W'^T + scale * u B^T )
 * with W' the decoded weight (NF4 decode fused into the GEMM: W' never exists in
 * memory) and fp32 accumulation.  The forward is also the backward's recompute.
 *   W      the frozen weight
 *   x      device bf16 [T, in]
 *   T      tokens, >= 0 (0 is a no-op)
 *   A, B   device bf16 [r, in] and [out, r]; both NULL or r == 0 disables the adapter
 *          (then y is the frozen base linear exactly: the adapter-off reference pass)
 *   scale  alpha / r, computed by the caller
 *   y      device bf16 [T, out]
 *   u      device fp32 [T, r] written with x A^T; required when the adapter is on
 * Errors: EINVAL, ESHAPE (in % 64, blocksize), EALIGN, EHIP.
 */
int lora_linear_fwd(const lnf4_weight* W, const uint16_t* x, int64_t T, const uint16_t* A,
                    const uint16_t* B, int32_t r, float scale, uint16_t* y, float* u, hipStream_t stream);

/* Bytes of device workspace lora_linear_bwd needs for these sizes (0 if r == 0 and
 * the shapes need no split reduction): v = dy B and, for a split input-gradient GEMM, its
 * fp32 partial sums.  The backward it sizes is the one the Soup deep dive ("Core feature:
 * how layer streaming works") describes: W is read again for dL/dx = W^T dL/dy while only
 * the adapters receive gradients.  The caller allocates it once (fwd and bwd never
 * allocate).  Host-only; returns 0 for invalid sizes. */
size_t lora_linear_bwd_workspace(int64_t T, int64_t out_f, int64_t in_f, int32_t r);

/*
 * LoRA linear backward (one projection).  The layer is on the device a second time
 * because the input gradient needs the frozen weight again, dL/dx = W^T dL/dy, while only
 * the adapters (their gradients and optimizer state held in device memory) are trained
 * (Soup deep dive, "Core feature: how layer streaming works"); W gets no gradient:
 *   v  = dy B                                     (fp32 [T, r], in workspace)
 *   dx = bf16( dy W' + scale * v A )              (+ old dx if accumulate)
 *   dA = scale * v^T x                            (fp32 [r, in], += old if accumulate)
 *   dB = scale * dy^T u                           (fp32 [out, r], += old if accumulate)
 * u is taken from u_saved (the forward's u) or recomputed as x A^T when NULL.
 *   dx, dA, dB   device outputs; each may be NULL to skip it (dA, dB ignored when the
 *                adapter is off)
 *   workspace    device, at least lora_linear_bwd_workspace(T, out, in, r) bytes
 * Gradient reductions over T use a fixed split and a fixed-order second pass.  When the
 * dx GEMM has few output tiles and a long K (few tokens, many output features), it splits
 * K: each split's fp32 sums go to the workspace and a fixed-order pass adds them, so dx is
 * still deterministic.  The split count depends only on the shapes.
 * Errors: EINVAL, ESHAPE (in % 64, blocksize, out_f not a multiple of 8, workspace too
 * small), EALIGN, EHIP.
 */
int lora_linear_bwd(const lnf4_weight* W, const uint16_t* x, const uint16_t* dy, int64_t T,
                    const uint16_t* A, const uint16_t* B, int32_t r, float scale, const float* u_saved,
                    uint16_t* dx, float* dA, float* dB, int32_t accumulate, void* workspace,
                    size_t ws_bytes, hipStream_t stream);

/*
 * lora_linear_bwd for callers that cannot allocate device memory or take a workspace
 * argument (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and arguments minus the workspace, which is instead
 * a fixed array of LNF4_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held until
 * the process ends).  The call allocates nothing.
 *  - Limit: shapes whose workspace (v = dy B, a recomputed u and the adapter-gradient
 *    partial sums) exceeds LNF4_NOALLOC_SCRATCH_BYTES are rejected with ESHAPE.  For
 *    example a single 14336 x 4096 projection at T = 2048 with r = 16 needs about 38 MB.
 *  - The input-gradient GEMM is never split over K here (lora_linear_bwd splits it for few
 *    output tiles and a long K): dA and dB are bitwise those of lora_linear_bwd; dx is
 *    bitwise the same where lora_linear_bwd does not split, else equal up to the order of
 *    its fp32 sums.
 *  - Every call on one GPU uses that GPU's one array: calls that overlap in time on one
 *    GPU (on different streams, or from different threads) race and give wrong results.
 *    Calls ordered on one stream are safe.
 * Errors: as lora_linear_bwd (ESHAPE also for a workspace need above the limit).
 */
#define LNF4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int lora_linear_bwd_noalloc(const lnf4_weight* W, const uint16_t* x, const uint16_t* dy, int64_t T,
                            const uint16_t* A, const uint16_t* B, int32_t r, float scale, const float* u_saved,
                            uint16_t* dx, float* dA, float* dB, int32_t accumulate, hipStream_t stream);

/*
 * Projections that read the same input (q, k, v read the attention input; gate and
 * up read the MLP input) run as one grouped launch.  In the forward each projection
 * writes its own y; in backward the group's input gradient is the sum over its
 * projections: dx = sum_p ( dy_p W'_p + scale_p v_p A_p ).
 */
typedef struct lnf4_proj {
  lnf4_weight W;
  const uint16_t* A;   /* device bf16 [r, in] or NULL */
  const uint16_t* B;   /* device bf16 [out, r] or NULL */
  int32_t r;           /* 0: adapter off */
  float scale;
  uint16_t* y;         /* fwd: device bf16 [T, out] */
  float* u;            /* fwd: device fp32 [T, r] (written); bwd: saved u or NULL (recompute) */
  const uint16_t* dy;  /* bwd: device bf16 [T, out] */
  float* dA;           /* bwd: device fp32 [r, in] or NULL */
  float* dB;           /* bwd: device fp32 [out, r] or NULL */
} lnf4_proj;

/* Grouped forward: n (1..8) projections with the same in_f share x (the adapted projections
 * of the pages' configs, q and v, read the same attention input: 20B RLHF article,
 * "Low-rank adaptation via PEFT").
 *   adapters_enabled  0: base only (y = x W'^T; A, B, u ignored).  1: adapters on, u = x A^T
 *                     computed and written.  2: adapters on, u read as given: it must hold
 *                     x A^T from an earlier call with the same x and A, as in the checkpoint
 *                     recompute of the backward, which re-reads a layer for its forward on
 *                     the saved input (Soup deep dive, "Core feature: how layer streaming
 *                     works"); y is then bitwise the y of that earlier call.
 * Errors: as lora_linear_fwd; EINVAL for adapters_enabled outside 0..2. */
int lora_group_fwd(const lnf4_proj* projs, int32_t n, const uint16_t* x, int64_t T, int32_t adapters_enabled,
                   hipStream_t stream);

/* The same grouped forward with a caller-owned workspace, which lets a launch of few output
 * tiles over a long K (the SwiGLU down projection of a small model: 896 outputs over 4864
 * inputs at T = 2048) run as K splits whose fp32 sums a second launch adds in split order.
 * The operation and its results' definition are those of lora_group_fwd (20B RLHF
 * article, "Low-rank adaptation via PEFT"); a split launch sums K in another order, so y
 * may differ from lora_group_fwd's in the last bits, and it is the same for every call with
 * the same shapes (no atomics).
 *   lora_group_fwd_workspace: bytes needed for these descriptors and T (host-only; 0 when
 *   the launch is not split: bf16 weights, enough output tiles, a short K, or an out_f that
 *   is not a multiple of 4).
 *   workspace: device memory of at least that many bytes, 256-byte aligned, used only
 *   during the call (stream-ordered).  NULL with ws_bytes 0 runs the unsplit launch.
 * Errors: as lora_group_fwd; EINVAL for a NULL workspace with ws_bytes > 0 when one is
 * needed, ESHAPE for a workspace smaller than needed, EALIGN for a misaligned one. */
size_t lora_group_fwd_workspace(const lnf4_proj* projs, int32_t n, int64_t T);
int lora_group_fwd_ws(const lnf4_proj* projs, int32_t n, const uint16_t* x, int64_t T, int32_t adapters_enabled,
                      void* workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for lora_group_bwd (the grouped backward below) with these projs and T:
 * which gradients are asked
 * for (dA, dB non-NULL) and whether u is saved decide the buffers, so query with the
 * same descriptors as the call.  Host-only. */
size_t lora_group_bwd_workspace(const lnf4_proj* projs, int32_t n, int64_t T);

/* Grouped backward: dx [T, in] = sum over the group (NULL to skip), per-projection dA/dB
 * (the frozen weights are read again in the backward because dx = W^T dy: Soup deep dive,
 * "Core feature: how layer streaming works").
 * Errors: as lora_linear_bwd (every projection's out_f a multiple of 8). */
int lora_group_bwd(const lnf4_proj* projs, int32_t n, const uint16_t* x, int64_t T, uint16_t* dx,
                   int32_t accumulate, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Shard layout of one decoder layer.  The frozen base is kept as one page-locked host
 * blob per decoder layer, and a step copies whole layers (Soup deep dive, "Core feature:
 * how layer streaming works"): projections in the caller's order (q, k, v, o, gate, up,
 * down), each as [data][absmax] sections, every section starting on a 256-byte
 * boundary.  offsets[2p] = data offset, offsets[2p+1] = absmax offset (-1 for
 * BF16).  total_bytes = shard size.  Host-only.
 * Errors: EINVAL, ESHAPE (in % 64).
 */
int lnf4_shard_layout(int32_t n_proj, const int64_t* out_f, const int64_t* in_f, int32_t fmt,
                      int64_t* offsets, int64_t* total_bytes);

/* ------------------------------------------------------------------ output side
 * The vocab-sized embed_tokens and the untied lm_head take turns in one device slot
 * of the layer stream (Soup deep dive, "Core feature: how layer streaming works"): the
 * embedding lookup reads the slot at the start of a step, and the output head plus its
 * loss read it at the forward/backward turn, optionally a chunk of tokens at a time
 * (the stream_loss_chunk key, same article, "Streaming config keys").  The lm_head
 * GEMMs themselves are lora_linear_fwd / lora_linear_bwd with a BF16 weight [V, H]
 * pointing into the slot and the adapter off.
 */

/*
 * Embedding lookup: out[t][:] = table[ids[t]][:] (bf16 rows copied bitwise).
 *   table   bf16 [vocab, hidden], 16-byte aligned: either device memory (the slot holding
 *           embed_tokens) or page-locked host memory mapped for the device, whose T rows
 *           the kernel then reads over the host link (the step's rows only, instead of
 *           copying the whole table into the slot)
 *   hidden  a positive multiple of 8
 *   ids     device int32 [T]; an id outside [0, vocab) yields a zero row (device ids
 *           cannot be checked by the host)
 *   out     device bf16 [T, hidden], 16-byte aligned
 * After the argument checks the runtime is asked what kind of memory the table is.
 * Errors: EINVAL (T, NULL, a table that is neither device memory nor mapped page-locked
 * host memory), ESHAPE (vocab, hidden), EALIGN, EHIP.
 */
int lnf4_embed_gather(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* ids, int64_t T,
                      uint16_t* out, hipStream_t stream);

/*
 * Token cross-entropy on bf16 logits [T, V] from the output head:
 *   lse_t        = log sum_j exp(l[t][j])                          (fp32)
 *   logp[t]      = l[t][label_t] - lse_t
 *   dlogits[t][j] = bf16( g_t * (exp(l[t][j] - lse_t) - [j == label_t]) )
 *   g_t          = grad_scale * (seq_scale ? seq_scale[t / rows_per_scale] : 1)
 * so grad_scale = 1/T gives the gradient of the mean token loss, and a per-sequence
 * seq_scale carries a sequence-level objective (the preference loss) back to tokens.
 * A label outside [0, V) marks an ignored token: logp 0 and a zero gradient row.
 *   logits   device bf16 [T, V], V a positive multiple of 8, 16-byte aligned
 *   labels   device int32 [T]
 *   seq_scale device fp32 [ceil(T / rows_per_scale)] or NULL
 *   logp     device fp32 [T] or NULL;  dlogits device bf16 [T, V] or NULL (one of the
 *            two is required).  dlogits may alias logits (each row is read in full
 *            before it is overwritten by the same workgroup).
 * Every reduction has a fixed order: bitwise reproducible.
 * Errors: EINVAL (T, NULL, rows_per_scale < 1, non-finite grad_scale), ESHAPE (V), EALIGN, EHIP.
 */
int lnf4_cross_entropy(const uint16_t* logits, int64_t T, int64_t vocab, const int32_t* labels, float grad_scale,
                       const float* seq_scale, int64_t rows_per_scale, float* logp, uint16_t* dlogits,
                       hipStream_t stream);

/*
 * Per-sequence sums of token values (log-probs, the sequence scores of the preference
 * losses: Soup 4 GB article, "Preference optimization"): sums[i] = sum_{j < seq_len} x[i*seq_len + j],
 * fp32 in a fixed order.  x device fp32 [n_seq * seq_len]; sums device fp32 [n_seq].
 * Errors: EINVAL, EALIGN, EHIP.
 */
int lnf4_sequence_sums(const float* x, int32_t n_seq, int64_t seq_len, float* sums, hipStream_t stream);

/*
 * Sigmoid preference loss over n_pairs pairs of sequence log-prob sums, ordered
 * (chosen_0, rejected_0, chosen_1, ...).  The reference sums come from the same
 * streamed base with the adapters off (Soup 4 GB article, "Memory-free reference
 * model"; 20B-RLHF article, step 3).  The pages name the preference step but give no
 * formula; the reading taken is the standard sigmoid form with temperature beta:
 *   m_p  = beta * ((pol[2p] - ref[2p]) - (pol[2p+1] - ref[2p+1]))
 *   loss = mean_p log(1 + exp(-m_p))
 *   coef[2p] = -beta * sigmoid(-m_p) / P,  coef[2p+1] = +beta * sigmoid(-m_p) / P
 * coef is dloss / dpol, and a token's loss is minus its log-prob, so passing coef as
 * seq_scale to lnf4_cross_entropy with grad_scale = -1 and rows_per_scale = sequence
 * length gives the gradient of the preference loss with respect to the policy logits.
 *   pol_sums, ref_sums device fp32 [2 n_pairs]; loss device fp32 [1]; coef device fp32 [2 n_pairs]
 * Errors: EINVAL (n_pairs outside 1..2^20, beta not finite or <= 0, NULL), EALIGN, EHIP.
 */
int lnf4_dpo_loss(const float* pol_sums, const float* ref_sums, int32_t n_pairs, float beta, float* loss, float* coef,
                  hipStream_t stream);

/* ------------------------------------------------------------------ decoder-layer glue
 * The parts of a Llama/Qwen decoder layer between its projections: RMSNorm, rotary
 * position embedding, causal grouped-query attention, the SwiGLU MLP activation and the
 * residual adds (the layer shapes of the configs; the Soup deep dive, "Core feature: how
 * layer streaming works", names the per-layer checkpoint recompute that re-runs them in
 * backward).  The pages give no formulas; these are the standard Llama definitions.
 * All tensors are bf16 [T, width] row-major with a 16-byte aligned base; every call
 * computes in fp32 and rounds each stored value to bf16 once.
 */

/*
 * RMSNorm forward: y = bf16(x * r * g), r = 1 / sqrt(mean(x^2) + eps) per row (fp32).
 *   x, y   device bf16 [T, H], H a positive multiple of 8;  g device bf16 [H] (frozen)
 *   rstd   device fp32 [T] receiving r (NULL to skip; the backward needs it)
 * Errors: EINVAL (T, eps, NULL), ESHAPE (H), EALIGN, EHIP.
 */
int lnf4_rmsnorm_fwd(const uint16_t* x, int64_t T, int64_t H, const uint16_t* g, float eps, uint16_t* y,
                     float* rstd, hipStream_t stream);

/*
 * RMSNorm backward (g frozen: no weight gradient), with the residual gradient added:
 *   dx = bf16(dres + r g dy - x r^3 mean(x g dy))     (dres NULL: no residual term)
 *   rstd the forward's r.  Errors: as lnf4_rmsnorm_fwd.
 */
int lnf4_rmsnorm_bwd(const uint16_t* x, int64_t T, int64_t H, const uint16_t* g, const float* rstd,
                     const uint16_t* dy, const uint16_t* dres, uint16_t* dx, hipStream_t stream);

/*
 * RoPE table: table[2(p*D/2 + i)], table[2(p*D/2 + i) + 1] = cos, sin of p * base^(-2i/D)
 * for positions p < seq_len and i < D/2, computed in fp64 and rounded to fp32.
 *   table  device fp32 [seq_len * D] (8-byte aligned); D a multiple of 16; base > 1
 * Errors: EINVAL, ESHAPE, EALIGN, EHIP.
 */
int lnf4_rope_table(int64_t seq_len, int32_t head_dim, double base, float* table, hipStream_t stream);

/*
 * Rotate-half RoPE in place on x [T, n_heads * D]: for each head the pair (i, i + D/2)
 * turns by the angle of position t mod seq_len (inverse != 0: by minus that angle, the
 * backward).  Errors: EINVAL, ESHAPE, EALIGN, EHIP.
 */
int lnf4_rope(uint16_t* x, int64_t T, int32_t n_heads, int32_t head_dim, int64_t seq_len, const float* table,
              int32_t inverse, hipStream_t stream);

/* SwiGLU: s = bf16(silu(g) * u), silu(z) = z / (1 + e^-z); n elements, a multiple of 8. */
int lnf4_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* s, hipStream_t stream);

/* SwiGLU backward: dg = ds u sig (1 + g (1 - sig)), du = ds silu(g), sig = 1/(1 + e^-g). */
int lnf4_swiglu_bwd(const uint16_t* g, const uint16_t* u, const uint16_t* ds, int64_t n, uint16_t* dg,
                    uint16_t* du, hipStream_t stream);

/* Residual add: out = bf16(a + b); n elements, a multiple of 8 (out may alias a or b). */
int lnf4_add(const uint16_t* a, const uint16_t* b, int64_t n, uint16_t* out, hipStream_t stream);

/*
 * Causal grouped-query attention forward, per sequence of seq_len tokens:
 *   o = softmax(q k^T / sqrt(D) + causal mask) v, query head h reading kv head
 *   h / (n_heads / n_kv);  lse[h][t] = log sum_j exp(q_t k_j / sqrt(D)) (natural log).
 *   q, o  device bf16 [T, n_heads * D];  k, v device bf16 [T, n_kv * D]
 *   lse   device fp32 [n_heads, T]
 *   D = head_dim, 64 or 128; seq_len a positive multiple of 64 dividing T
 * fp32 accumulation on the matrix cores; probabilities (and in backward the score
 * gradients) enter their products as a bf16 hi + lo pair, about 16 significant bits.
 * Errors: EINVAL (T, NULL), ESHAPE (head_dim, heads, seq_len), EALIGN, EHIP.
 */
int lnf4_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t T, int32_t n_heads,
                  int32_t n_kv, int32_t head_dim, int64_t seq_len, uint16_t* o, float* lse, hipStream_t stream);

/*
 * Attention backward from the forward's o and lse:
 *   P = exp(q k^T / sqrt(D) - lse), dV = P^T dO, dP = dO v^T, dS = P (dP - rowsum(dO o o)),
 *   dq = dS k / sqrt(D), dk = dS^T q / sqrt(D), each kv head's dk, dv summed over its
 *   query heads.  No atomics: bitwise reproducible.
 *   dout        device bf16 [T, n_heads * D] (the output gradient)
 *   dq, dk, dv  device bf16, shaped as q, k, v
 *   workspace   device, 256-byte aligned, at least lnf4_attn_bwd_workspace(...) bytes:
 *               rowsum(dO o o) per head and token, and with grouped kv heads the fp32
 *               per-query-head shares of dk and dv (summed in head order at the end)
 * Errors: as lnf4_attn_fwd; ESHAPE also for a workspace too small.
 */
int lnf4_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o, const float* lse,
                  const uint16_t* dout, int64_t T, int32_t n_heads, int32_t n_kv, int32_t head_dim,
                  int64_t seq_len, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* workspace, size_t ws_bytes,
                  hipStream_t stream);

/* Workspace bytes lnf4_attn_bwd needs (0 for invalid sizes).  Host-only. */
size_t lnf4_attn_bwd_workspace(int64_t T, int32_t n_heads, int32_t n_kv, int32_t head_dim);

/* ------------------------------------------------------------------ layer stream */
typedef struct lnf4_stream lnf4_stream;

#define LNF4_STREAM_RING 0
#define LNF4_STREAM_RESIDENT 1
#define LNF4_STREAM_REUSE 2

#define LNF4_EV_COPY 0      /* a layer copy was issued */
#define LNF4_EV_STEP 1      /* a call made compute wait for its layer */
#define LNF4_EV_SLOT_COPY 2 /* a head-slot copy was issued */
#define LNF4_EV_SLOT_WAIT 3 /* compute was made to wait for the head slot */

typedef struct lnf4_stream_event {
  int32_t kind;   /* LNF4_EV_* */
  int32_t call;   /* stream_layer_step call index at which it happened */
  int32_t j;      /* COPY: schedule position (resident: shard); STEP: copy waited on (reuse: the
                     position whose copy filled the buffer, -1 for an earlier pass); SLOT: slot
                     load index */
  int32_t layer;  /* shard index */
  int32_t buffer; /* device buffer index (-1 for the slot) */
  int32_t wait;   /* COPY: call whose release it waited for (-1: none); STEP: copy index;
                     SLOT_COPY: previous slot load index (-1: none) */
} lnf4_stream_event;

/*
 * The stream a streamed step's kernels run on, with a hardware queue of its own, so the
 * layer copies overlap the compute (the 4 GB-laptop article, "Layer streaming: technical
 * implementation and memory efficiency": the next layer loads while the current one
 * computes; the Soup deep dive, "Core feature: how layer streaming works").  The HIP
 * runtime maps ordinary streams onto a few hardware queues shared in turn (4 by default);
 * a copy stream that lands on the compute stream's queue loses all overlap, since the
 * event wait or event record of one stream then holds back every later packet of the
 * other in that in-order queue.  This stream is created with a compute-unit mask of every
 * CU of the device, which gives it a queue no other stream uses; its kernels run on all
 * CUs at default priority.  It follows the default-flag stream rules: it orders itself
 * with the null stream (work on either waits for earlier work on the other) and not with
 * other streams.
 *   device  HIP device index
 *   out     receives the stream: created on the device's first call, the same handle on
 *           every later call, owned by the library and kept until the process ends (never
 *           destroy it)
 * Errors: EINVAL (device out of range, NULL out), EHIP.
 */
int stream_compute_stream(int32_t device, hipStream_t* out);

/*
 * The stream the layer copies run on, made the same way as the compute stream (a queue of
 * its own; the 4 GB-laptop article, "Layer streaming: technical implementation and memory
 * efficiency": the prefetch runs on a dedicated stream).  An ordinary stream shares one of
 * the runtime's few hardware queues with other streams, and where their packets sit in
 * front of the copies' event waits and records the ring loses overlap: a Llama-8B-shaped
 * decoder model whose copy stream was drawn from a process's stream pool after other
 * streams had been used ran its streamed step in 201 ms, against 182 ms on this stream.
 * It follows the default-flag stream rules (ordered with the null stream).
 *   device, out  as for stream_compute_stream (a second, distinct stream; never destroy it)
 * Errors: EINVAL (device out of range, NULL out), EHIP.
 */
int stream_copy_stream(int32_t device, hipStream_t* out);

/*
 * Create a layer stream over one pass of `schedule` (shard indices, e.g. layers
 * 0..L-1 then L-1..0 for an SFT step: forward, then recompute + backward).  The frozen
 * layers stay in page-locked host RAM and a separate stream copies them into a few
 * preallocated device buffers ahead of the compute (Soup deep dive, "Core feature: how
 * layer streaming works", and its settings table, "Streaming config keys": stream_buffers,
 * default 2, range 2..8; 4 GB-laptop article, "Layer streaming: technical implementation
 * and memory efficiency": prefetch on a dedicated stream).
 *   host_shards  n_shards page-locked host pointers (one contiguous blob per layer)
 *   shard_bytes  size of each shard, each <= buf_bytes
 *   dev_bufs     n_bufs device buffers of buf_bytes each, 256-byte aligned
 *   n_bufs       ring mode: 2..8 (2 = double buffering).  Resident mode: == n_shards.
 *   schedule     sched_len shard indices, copied by the library
 *   mode         LNF4_STREAM_RING (0): the ring below.  LNF4_STREAM_RESIDENT (1): every
 *                shard gets its own buffer and is copied once at the first call (the "H2D
 *                removed" and bit-exactness reference run).  LNF4_STREAM_REUSE (2): the ring
 *                with buffer reuse (below)
 *   copy_stream  the side stream that carries every host-to-device copy
 *   slot_buf     optional device buffer for the shared embed / lm_head slot (or NULL)
 *   slot_bytes   its size
 * Ring rule: call k uses buffer k mod n_bufs; at call k every copy j <= k+n_bufs-1 not
 * yet issued is issued into buffer j mod n_bufs after the release of call j-n_bufs;
 * call k's compute waits for copy k.
 * Reuse rule (a stream variant beyond the pages' ring, which re-copies every read): each
 * pass is planned from what the buffers hold.  A call whose shard sits intact in a
 * buffer uses it with no copy (at the forward/backward turn the last n_bufs forward
 * layers, at the next pass's start the first n_bufs layers).  Otherwise its shard is
 * copied into the least recently used buffer (lowest index on ties), issued at call
 * max(j - n_bufs + 1, u + 1) where u is that buffer's last user in the pass, after u's
 * release.  A STEP event's j is then the position whose copy filled the buffer (-1: a
 * previous pass).  SFT steady state: 2L - 2 n_bufs copies per pass instead of 2L.
 * Errors: EINVAL (also mode outside 0..2), ESHAPE, EALIGN, EHIP.
 */
int stream_create(const void* const* host_shards, const size_t* shard_bytes, int32_t n_shards,
                  void* const* dev_bufs, size_t buf_bytes, int32_t n_bufs, const int32_t* schedule,
                  int32_t sched_len, int32_t mode, hipStream_t copy_stream, void* slot_buf,
                  size_t slot_bytes, lnf4_stream** out);

/*
 * Call k of the pass (k = 0, 1, ... in order): while layer k computes, the next layer's
 * copy is already running into another buffer, and every layer is read twice in an SFT
 * step (forward, then recompute + backward) (Soup deep dive, "Core feature: how layer
 * streaming works").  Records the release of call k-1's
 * buffer on `compute`, issues the copies the ring rule allows, makes `compute` wait
 * for layer k's copy and returns its device address in *dev_ptr_out.  Every kernel
 * that reads layer k must be enqueued on `compute` before call k+1.  Resident mode: each
 * layer is copied once, and once that copy has been seen complete (a host-side event
 * query) the call enqueues nothing on `compute`: after one resident pass has finished,
 * the calls of a resident pass issue no stream work, so the caller may capture that
 * pass's kernel launches as a graph.
 * Errors: ESTATE (k out of order, pass finished, destroyed), EINVAL, EHIP.
 */
int stream_layer_step(lnf4_stream* st, int32_t k, hipStream_t compute, void** dev_ptr_out);

/*
 * Head slot: copy shard `shard` (embed_tokens or the untied lm_head, which share one
 * device slot: Soup deep dive, "how layer streaming works") into the slot on the copy
 * stream, after the compute work enqueued so far on `compute` (the previous user of
 * the slot) has finished.  Does not make compute wait; stream_slot_wait does.
 */
int stream_slot_load(lnf4_stream* st, int32_t shard, hipStream_t compute);

/*
 * The same copy issued in n_parts pieces (part = 0, 1, ..., n_parts-1, in order, on
 * successive calls), so a large slot shard can trickle over the copy stream between
 * layer copies instead of holding it for one long transfer (the prefetch stream the Soup
 * deep dive describes carries layers and the slot alike, "Core feature: how layer
 * streaming works").  Part p copies bytes
 * [p*c, min((p+1)*c, size)) with c = ceil(size/n_parts) rounded up to 4 KiB.  Part 0
 * waits for the work enqueued so far on `compute` (the slot's previous user); the load
 * counts as issued after the last part, and only then may stream_slot_wait be called.
 * Each part logs one SLOT_COPY event with buffer = -1 - part.
 * Errors: EINVAL (no slot, shard or part out of range, n_parts outside 1..1024),
 * ESHAPE (shard larger than the slot), ESTATE (part out of order, destroyed), EHIP.
 */
int stream_slot_load_part(lnf4_stream* st, int32_t shard, int32_t part, int32_t n_parts, hipStream_t compute);

/* Make `compute` wait for the last complete slot load; *slot_ptr_out = the slot (the
 * shared embed_tokens / lm_head slot: Soup deep dive, "Core feature: how layer streaming works").
 * Errors: EINVAL (no slot), ESTATE (no complete load issued, destroyed), EHIP. */
int stream_slot_wait(lnf4_stream* st, hipStream_t compute, void** slot_ptr_out);

/* Rewind a finished (or unfinished) pass so the same schedule runs again (next step: every
 * step streams the layers anew, Soup deep dive, "Core feature: how layer streaming works").
 * The first copies of the new pass wait for the release of the old pass's buffers.  On a
 * disk-tier context whose pass did not issue all its copies (a step abandoned, e.g. after
 * a failed call), the reader thread is stopped, the copies out of the staging buffers
 * already issued are waited for on the host, and the reader restarts at the first
 * position of the next pass with any read error cleared.
 * Errors: ESTATE (NULL or destroyed), EINVAL (the reader cannot restart), EHIP. */
int stream_reset(lnf4_stream* st, hipStream_t compute);

/* Copy up to cap events of the current pass to ev; *n = number copied.  The log shows,
 * per call, which copies were issued and which copy the compute waited on: the stream
 * schedule whose cost the Soup deep dive ("Core feature: how layer streaming works")
 * accounts for as compute time spent waiting on copies.
 * Errors: ESTATE (NULL or destroyed context), EINVAL (n NULL, cap < 0, ev NULL with cap > 0). */
int stream_log(const lnf4_stream* st, lnf4_stream_event* ev, int32_t cap, int32_t* n);

/* Bytes copied host-to-device by this context since creation (layers + slot): the transfer
 * whose cost the Soup deep dive measures by removing it ("Core feature: how layer streaming
 * works").
 * Errors: ESTATE (NULL or destroyed), EINVAL (bytes NULL). */
int stream_bytes_copied(const lnf4_stream* st, int64_t* bytes);

/*
 * Disk tier (Soup deep dive, "Core feature: how layer streaming works" and its table of
 * streaming settings: when host RAM is short the frozen shards are read from an NVMe
 * file, and a read-ahead depth of 1..8 layers sets how many are staged in pinned RAM
 * ahead of the copies).  A ring-mode stream (LNF4_STREAM_RING rules above) whose layer
 * copies come from `path` instead of host shards:
 *   file_offsets  n_shards byte offsets of the shards in the file (only scheduled shards
 *                 are read)
 *   drop_cache    nonzero: each shard's pages are dropped from the page cache after its
 *                 read (posix_fadvise DONTNEED), so every pass reads the device and not
 *                 host RAM.  (O_DIRECT reads cannot target HIP page-locked memory.)
 *   stage_bufs    n_stage (1..8, the read-ahead depth) page-locked staging buffers of
 *                 stage_bytes each, caller-owned
 *   host_shards   NULL, or n_shards page-locked pointers with NULL entries allowed: only
 *                 shards with a host copy can be loaded into the slot
 *   the rest      as in stream_create (ring mode)
 * A reader thread owned by the context walks the schedule positions g = 0, 1, ... (on
 * across passes) and reads position g's shard into staging buffer g mod n_stage once the
 * copy out of that buffer for position g - n_stage has completed; the copy of position g
 * is issued (inside stream_layer_step) once its read is done, so stream_layer_step may
 * block on the reader.  No GPU work waits on the host.  A failed read is reported by the
 * stream_layer_step call that needs it (EINVAL, with the errno text).  The file must stay
 * unchanged while the context lives.
 * Errors: EINVAL (NULL arguments, n_stage outside 1..8, cannot open the file, a staging
 * buffer not page-locked), ESHAPE (a shard larger than stage_bytes or past the end of the
 * file, and stream_create's), EALIGN (stream_create's), EHIP.
 */
int stream_create_disk(const char* path, const int64_t* file_offsets, int32_t drop_cache, void* const* stage_bufs,
                       size_t stage_bytes, int32_t n_stage, const void* const* host_shards, const size_t* shard_bytes,
                       int32_t n_shards, void* const* dev_bufs, size_t buf_bytes, int32_t n_bufs,
                       const int32_t* schedule, int32_t sched_len, hipStream_t copy_stream, void* slot_buf,
                       size_t slot_bytes, lnf4_stream** out);

/* Disk tier only (stream_source: disk, Soup deep dive, "Streaming config keys"): bytes read
 * from the file so far and the reader's time inside the reads (seconds), for the disk's
 * achieved rate.  Errors: EINVAL (no disk tier), ESTATE. */
int stream_disk_stats(const lnf4_stream* st, int64_t* bytes_read, double* read_seconds);

/*
 * Release a context.  A handle is checked before it is used, never trusted (the Soup deep
 * dive, "Structure: a CLI whose settings schema is the product", refuses unknown settings
 * instead of acting on them; the same strictness applies to handles):
 *  - Idempotent: NULL, or a handle already destroyed, returns LNF4_OK and does nothing.
 *  - Before it returns, every copy the context issued (layer copies, slot loads, a disk
 *    tier's staging copies) has completed and a disk tier's reader thread has ended, so
 *    the caller may then free or reuse its host shards, staging buffers, device buffers
 *    and slot.  Compute work the caller enqueued is not waited for.
 *  - Every later call on the handle returns LNF4_ESTATE.  The context's events, thread and
 *    tables are released; its small host struct is kept for the life of the process, so a
 *    later context never gets the same address and a stale handle cannot name it.
 * Errors: EHIP if waiting for a copy failed (the context is released all the same).
 */
int stream_destroy(lnf4_stream* st);

#ifdef __cplusplus
}
#endif
#endif /* LNF4_H */
