/*
 * zo.h - C-ABI of libzo: inference-native zeroth-order candidate scoring on
 * one AMD Instinct MI355X (gfx950).
 *
 * The method ("Zeroth-Order Fine-Tuning Was an Inference Workload All Along",
 * section "Why ZO Fine-Tuning Is Really Scoring"): a two-point estimator
 * evaluates the objective at theta + eps*z and theta - eps*z, forms
 * c = (L+ - L-) / (2 eps) and updates theta <- theta - eta*c*z, with z a
 * low-rank matrix per linear layer (LoZO).  The arXiv abstract of
 * "Inference-Native Zeroth-Order Optimization" describes the same process as
 * candidate-state queries planned by a ProbePlan, realised with factorized side
 * states over frozen weights, lazy updates and persistent LoRA banks.  The four
 * calls below are that query process:
 *
 *   zo_plan      ProbePlan: directions (seeds), rank r, eps, candidate list
 *   zo_score     one batched forward over every candidate state; returns the
 *                summed label log-probs S per candidate (the loss is L = -S)
 *   zo_estimate  c_d = (L_{d,+} - L_{d,-}) / (2 eps), optional explicit 1/r
 *   zo_update    lazy low-rank accumulation into the persistent bank
 *
 * plus zo_bank_fold, which commits a finished window's bank entry into the weights.
 *
 * Conventions for every function:
 *   - returns ZO_OK (0) or a negative zo_status; no exception or abort crosses
 *     the ABI; zo_last_error() gives a message for the calling thread;
 *   - all argument checks run on the host before anything is launched, except the
 *     token ids of a batch, which live in device memory: the kernels that read them
 *     flag an id outside [0, vocab) (and clamp it, so every access stays in bounds), and
 *     zo_score / zo_generate then return ZO_E_INVAL with their outputs undefined;
 *   - a plan or bank used with a model must have been made for a model of the same
 *     architecture, dtype and shapes (ZO_E_STATE otherwise, before any launch);
 *   - "device" pointers are HIP device memory of the model's device; "host"
 *     pointers are ordinary host memory;
 *   - the caller owns every buffer it passes (weights, workspace, bank memory,
 *     outputs); the library owns only the opaque objects it creates and frees
 *     them in the matching *_destroy;
 *   - stream arguments are hipStream_t; work is enqueued on that stream.
 *
 * Random numbers: every random direction is a pure function of (seed, step,
 * layer, linear kind), so factors are regenerated on the GPU, never stored.
 * Element e of the stream (seed, tag, tau) is word e % 4 of the Philox4x32-10
 * block with counter (e / 4, tag, lo32 tau, hi32 tau) and key (lo32 seed,
 * hi32 seed); a Gaussian pair comes from two words by Box-Muller evaluated with
 * binary64 +, -, *, /, sqrt only (no fused multiply-add): u = (w + 1/2) 2^-32,
 * R = sqrt(-2 ln u), ln by an exponent/mantissa split and the atanh series,
 * the angle from the other word (2-bit quadrant, half-quadrant bit, 29-bit
 * fraction times pi/4) with sin / cos by Taylor forms and an exact rotation;
 * words (0, 1) and (2, 3) of a block form the two pairs; factors are rounded
 * to fp32.
 */
#ifndef ZO_H_
#define ZO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZO_ABI_VERSION 1

typedef enum {
  ZO_OK = 0,
  ZO_E_INVAL = -1,      /* bad argument value (null pointer, out-of-range field, bad flag) */
  ZO_E_SHAPE = -2,      /* inconsistent sizes (buffer too small, length/shape mismatch) */
  ZO_E_NOMEM = -3,      /* host allocation failed, or a bank has no free slot */
  ZO_E_DEVICE = -4,     /* a HIP call or kernel launch failed */
  ZO_E_NONFINITE = -5,  /* a score passed to zo_estimate is NaN or infinite */
  ZO_E_STATE = -6,      /* object state does not allow the call (e.g. rank/target mismatch with the bank) */
  ZO_E_ABI = -7         /* descriptor written for another ABI version */
} zo_status;

enum { ZO_ARCH_OPT = 0, ZO_ARCH_QWEN3 = 1 };
/* ZO_DTYPE_FP8: the fp8-quantized model.  The layer linears (q|k|v, o, fc1 | gate|up,
   fc2 | down) are stored as OCP e4m3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
   bits, largest magnitude 448) of w * 2^11, one byte an element; the embeddings are bf16
   and the vectors fp32.  Every input of a layer linear (both norm outputs, the attention
   output, the GELU or SwiGLU output) is rounded to e4m3 (nearest even, saturating) and
   the base projections run e4m3 x e4m3 on the matrix cores; q, k, v, the residual
   stream, the final norm and the head are as in bf16 models; the side path keeps bf16
   factors.  A quantized frozen base under unquantized factorized side states is what
   "Inference-Native Zeroth-Order Optimization" has the method inherit from the runtime
   (arXiv abstract: frozen base weights; quantization among what the runtime supplies);
   the e4m3 encoding is the one of "FP8 Formats for Deep Learning", which that page's
   list of prior work names.  Requires d_model, d_ffn and n_heads * head_dim multiples
   of 128; not with
   ZO_PLAN_ACT_SPLIT or ZO_PLAN_SPLIT_*; side-input projections of at most 128 columns; zo_bank_fold
   requantizes the folded weights to e4m3. */
enum { ZO_DTYPE_F32 = 0, ZO_DTYPE_BF16 = 1, ZO_DTYPE_FP8 = 2 };
enum { ZO_ROLE_PROBE = 0, ZO_ROLE_FOREGROUND = 1 };
enum { ZO_SCORE_LAST_LABEL = 0, ZO_SCORE_ALL_NEXT = 1 };

/* Linear kinds (bit positions of a target mask). OPT: q k v o fc1 fc2.
   Qwen3: q k v o gate up down. */
enum { ZO_KIND_Q = 0, ZO_KIND_K = 1, ZO_KIND_V = 2, ZO_KIND_O = 3,
       ZO_KIND_FC1 = 4, ZO_KIND_FC2 = 5, ZO_KIND_GATE = 4, ZO_KIND_UP = 5, ZO_KIND_DOWN = 6 };

/* zo_plan flags */
#define ZO_PLAN_SCALE_INV_SQRT_R 1u  /* z = G V^T / sqrt(r) (eps_tilde = eps / sqrt(r)): MeZO-style
                                        factorized probes whose z has unit-variance entries (arXiv
                                        abstract: factorized perturbations approach dense Gaussian ZO as
                                        rank grows); zo_update then steps along the same z */
#define ZO_PLAN_ALLOW_ZERO_EPS 2u    /* permit eps == 0 (then S+ == S- exactly); testing only */
#define ZO_PLAN_ACT_SPLIT 4u         /* bf16 models: feed every projection its activations as the two-term
                                        bf16 expansion hi + lo (about 16 significant bits) against the exact
                                        bf16 weights, the side path as three-term products of split t and
                                        factors, and run attention in fp32.  Twice the MFMA work of the
                                        projections; for summed long-sequence losses and deep stacks, where
                                        bf16 activation rounding alone moves a sequence's sum by more than
                                        2e-2.  Same as all five ZO_PLAN_SPLIT_* flags below.  ZO_E_INVAL on
                                        fp32 and fp8 models. */
/* The two-term expansion at one rounding site only (bf16 models; any combination; ACT_SPLIT sets
   them all).  Each doubles the K extent of the projections that read the site (the cost is that
   projection's share of the MFMA work) and takes the site's side-input projection and side segment
   to three-term products: */
#define ZO_PLAN_SPLIT_QKV_IN 8u      /* first norm output -> packed q|k|v projection */
#define ZO_PLAN_SPLIT_ATTN 16u       /* q|k|v kept fp32, three-term attention products, attention
                                        output -> o projection */
#define ZO_PLAN_SPLIT_FC1_IN 32u     /* second norm output -> fc1 / gate-up projection */
#define ZO_PLAN_SPLIT_FC2_IN 64u     /* GELU / SwiGLU output -> fc2 / down projection */
#define ZO_PLAN_SPLIT_HEAD 128u      /* final norm output -> vocabulary head */
#define ZO_PLAN_SPLIT_SITES 248u     /* the five flags above */

/* zo_estimate flags */
#define ZO_EST_INV_RANK 1u  /* divide c by r: the explicit 1/r of LoZO's estimator, which the
                               released LoZO code omits ("Zeroth-Order Fine-Tuning Was an Inference
                               Workload All Along", section "The System Reorganization"); default off */
#define ZO_EST_MEAN 2u      /* use the mean instead of the sum of label log-probs per candidate */

/* Architecture.  OPT: pre-LayerNorm, learned positions, biases, exact-erf GELU
   FFN, LM head tied to the token embedding.  Qwen3: RMSNorm, per-head QK RMSNorm,
   rotate-half RoPE, grouped-query attention, SwiGLU FFN, untied LM head, no biases. */
typedef struct {
  int32_t abi_version;  /* ZO_ABI_VERSION */
  int32_t arch;         /* ZO_ARCH_* */
  int32_t dtype;        /* ZO_DTYPE_*: storage and GEMM operand type of the weight matrices; vectors are fp32 */
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab, max_pos;
  double norm_eps;      /* LayerNorm / RMSNorm epsilon */
  double rope_theta;    /* Qwen3 only */
} zo_model_desc;

typedef struct zo_model zo_model;
typedef struct zo_plan_s zo_plan_t;
typedef struct zo_bank zo_bank;

int zo_abi_version(void);
const char* zo_last_error(void);

/* ---- model ---------------------------------------------------------------
 * The weights live in one caller-owned device blob of zo_weights_size bytes.
 * Every logical tensor is row-major at its own 256-byte-aligned offset, with two
 * packings: per layer, q|k|v rows (and their biases) are adjacent (a packed
 * QKV matrix, as in the pages' "packed QKV updates"), and Qwen3's gate and up
 * rows are interleaved in groups of 16 ([16 gate rows | 16 up rows] ...).
 * zo_weight_locate reports where a logical tensor is.
 *   slot  = 0 for global tensors, layer + 1 for per-layer tensors
 *   param = global: 0 tok_embed [V,d], 1 pos_embed [max_pos,d] (OPT),
 *                   2 final_norm_w [d], 3 final_norm_b [d] (OPT), 4 lm_head [V,d] (Qwen3)
 *           layer:  0 ln1_w, 1 ln1_b, 2 wq, 3 bq, 4 wk, 5 bk, 6 wv, 7 bv, 8 wo, 9 bo,
 *                   10 ln2_w, 11 ln2_b, 12 w_fc1 | w_gate, 13 b_fc1, 14 w_fc2 | w_up,
 *                   15 b_fc2, 16 w_down, 17 q_norm_w, 18 k_norm_w   (absent ones -> ZO_E_INVAL)
 *   layout out: 0 plain row-major; 1 = gate rows, 2 = up rows of a 16-row interleave
 *               starting at *offset.  dtype out: ZO_DTYPE_*. */
int zo_weights_size(const zo_model_desc* desc, size_t* bytes);
int zo_weight_locate(const zo_model_desc* desc, int32_t slot, int32_t param, size_t* offset,
                     int64_t* rows, int64_t* cols, int32_t* dtype, int32_t* layout);

/* Creates a model that BORROWS weights_dev (device, zo_weights_size bytes); the library
   never frees it and never writes it except in zo_init_weights.  Allocates a small
   device RoPE table (Qwen3) freed by zo_model_destroy. */
int zo_model_create(const zo_model_desc* desc, void* weights_dev, size_t bytes, zo_model** out);
int zo_model_destroy(zo_model* m);

/* Fills the blob with the library's random initialisation: matrices and biases
   0.02*z, norm gains 1 + 0.02*z, z from the weight stream of `seed`, rounded to the
   storage type (round to nearest even).  Stand-in for pretrained checkpoints. */
int zo_init_weights(zo_model* m, uint64_t seed, void* stream);

/* ---- ProbePlan (arXiv abstract of "Inference-Native Zeroth-Order Optimization":
 *      the logical queries of one step, leaving realisation to the backend) ------ */
typedef struct {
  uint64_t step;              /* t: G factors use step t, V factors window floor(t / nu) */
  uint32_t nu;                /* lazy-sampling window (V held for nu steps), >= 1 */
  int32_t rank;               /* r >= 1 */
  double eps;                 /* > 0 and finite (0 with ZO_PLAN_ALLOW_ZERO_EPS) */
  int32_t n_dirs;             /* q directions, >= 1 */
  const uint64_t* dir_seeds;  /* host [n_dirs], distinct */
  int32_t n_cand;             /* >= 1 candidates */
  const int32_t* cand_dir;    /* host [n_cand], in [0, n_dirs) */
  const int32_t* cand_sign;   /* host [n_cand], +1 or -1 */
  uint32_t target_mask;       /* bit per ZO_KIND_* that carries the side path */
  uint32_t flags;             /* ZO_PLAN_* */
} zo_plan_desc;

/* Copies everything it needs; the plan is immutable and may be shared. */
int zo_plan(const zo_model* m, const zo_plan_desc* desc, zo_plan_t** out);
int zo_plan_destroy(zo_plan_t* p);

/* ---- bank: persistent low-rank state ("optional LoRA banks", "persistent banked
 *      state"; U accumulator of the lazy update, section "The System
 *      Reorganization": U_{t+1} = U_t - eta c_t G_t, Delta W = U_{t+1} V^T) ------
 * n_slots entries, each an fp32 U [n_out x r] per (layer, target kind), keyed by
 * (direction seed, window).  Layout of u_dev: slot-major, then layer, then kind in
 * increasing ZO_KIND order, each U row-major.  Keys live in the host object
 * (window -1 = empty slot); zo_bank_keys / zo_bank_set_keys save and restore them
 * for checkpointing together with the device memory. */
int zo_bank_size(const zo_model* m, int32_t n_slots, int32_t rank, uint32_t target_mask, size_t* bytes);
int zo_bank_create(const zo_model* m, int32_t n_slots, int32_t rank, uint32_t target_mask, void* u_dev,
                   size_t bytes, zo_bank** out);
int zo_bank_destroy(zo_bank* b);
int zo_bank_keys(const zo_bank* b, uint64_t* seeds, int64_t* windows);       /* host [n_slots] each */
int zo_bank_set_keys(zo_bank* b, const uint64_t* seeds, const int64_t* windows);
int zo_bank_entry_offset(const zo_bank* b, int32_t slot, int32_t layer, int32_t kind, size_t* offset);

/* Fold a bank entry into the weights and free its slot: for every layer and target kind,
 *   W <- round( W + sum_{k=0}^{r-1} U[:, k] V[:, k]^T )
 * with V regenerated from the entry's (seed, window) key, the sum formed in fp64 in k
 * order (products rounded, no fused multiply-add) starting from W, then rounded fp64 ->
 * fp32 -> bf16 (round to nearest even; fp32 models stop at fp32; fp8 models requantize: the
 * e4m3 code of the fp32 value times 2^11, nearest even, saturating, so that a change
 * smaller than half an e4m3 step of that weight is lost).  This is the commit of a
 * finished window's low-rank state into the dense weights (section "The System
 * Reorganization": Delta W = U V^T of the lazy update), which keeps the bank from
 * growing by one entry per window.  The only call that writes the weight blob; the
 * entry's U memory is left as is (a later zo_update on the slot zero-initialises it).
 * ws_dev: device workspace of at least zo_bank_fold_size bytes (the regenerated V
 * factors, fp32).  Synchronises `stream` before returning; ZO_E_STATE if the slot is
 * empty or the bank belongs to another model shape. */
int zo_bank_fold_size(const zo_model* m, const zo_bank* b, size_t* bytes);
int zo_bank_fold(zo_model* m, zo_bank* b, int32_t slot, void* ws_dev, size_t ws_bytes, void* stream);

/* Bank cap: every entry of a window other than the plan's is frozen (its window is over,
 * so every probe row still carries it as a rank-r side term, and the side segment of every
 * projection grows with their count).  zo_bank_cap folds the oldest frozen entries (lowest
 * window first, then lowest slot) into the weights with zo_bank_fold until at most
 * max_frozen remain; entries of the plan's window are never folded.  *n_folded (may be
 * NULL) receives the number folded.  ws_dev: as zo_bank_fold (needed only when something
 * is folded).  Synchronises `stream` when it folds. */
int zo_bank_cap(zo_model* m, zo_bank* b, const zo_plan_t* p, int32_t max_frozen, void* ws_dev, size_t ws_bytes,
                void* stream, int32_t* n_folded);

/* ---- batch and packing --------------------------------------------------------
 * Physical packing order (canonical): foreground sequences in input order, then for
 * each candidate in plan order, every probe sequence in input order.  Probe rows see
 * the candidate state W + sum_j U_j V_j^T + s*eps_tilde*G_d V_d^T (j over active bank
 * entries); foreground rows see W only (co-serving in the same physical batch,
 * arXiv abstract of "Inference-Native Zeroth-Order Optimization").
 * LAST_LABEL scores the last token from the row before it (needs length >= 2);
 * ALL_NEXT scores tokens 1..n-1 from rows 0..n-2. */
typedef struct {
  int32_t n_seq;               /* logical sequences, >= 0 */
  const int32_t* cu_seqlens;   /* host [n_seq + 1], cu[0] = 0, non-decreasing, lengths >= 1 */
  const int32_t* tokens_dev;   /* device int32 [cu_seqlens[n_seq]], ids in [0, vocab) (checked on the
                                  device: ZO_E_INVAL from zo_score / zo_generate otherwise) */
  const int32_t* role;         /* host [n_seq] ZO_ROLE_* */
  const int32_t* score_mode;   /* host [n_seq] ZO_SCORE_* */
} zo_batch;

/* Sizes of a batch under a plan: physical sequences, packed token rows, scored rows,
   and the bytes of device workspace zo_score needs (with this bank, or none). */
int zo_batch_layout(const zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b,
                    int32_t* n_phys, int64_t* n_rows, int64_t* n_scored, size_t* ws_bytes);
/* The packing itself (host arrays of n_phys): logical sequence and candidate (-1 foreground)
   of each physical sequence, and the first scored row of each (n_phys + 1 entries). */
int zo_pack(const zo_plan_t* p, const zo_batch* b, int32_t* phys_seq, int32_t* phys_cand,
            int32_t* phys_first_scored);

/* ---- zo_score ------------------------------------------------------------------
 * Direct scoring ("Zeroth-Order Fine-Tuning Was an Inference Workload All Along",
 * section "The System Reorganization": option-token losses from a direct worker
 * path): one batched forward of every physical sequence, the vocabulary-wide
 * log-softmax fused with the label gather, per-sequence sums in fp64.
 *   bank          may be NULL (no accumulated state)
 *   ws_dev        device workspace of at least the zo_batch_layout bytes
 *   seq_logp_dev  device fp64 [n_phys] or NULL: per physical sequence sum of scored log-probs
 *   tok_logp_dev  device fp32 [n_scored] or NULL: every scored log-prob in packing order
 *   S_host        host fp64 [n_cand]: S_c = sum over candidate c's sequences in packing
 *                 order (the summed label log-probs "L+/-"; loss L = -S)
 * Enqueued on `stream`; returns after synchronising that stream (S_host is valid).
 * At batches of at least one round of 256x256 tiles, the long-K projections (fc2 / down,
 * K >= 10240) run as persistent launches of one workgroup per CU whose last tiles are
 * handed between workgroups in K-slices; they expect the GPU to themselves.  Should a
 * handover wait give up (other kernels holding CUs for a long time) or cross XCDs, the
 * call fails with ZO_E_DEVICE and the model stops using them (call again); setting the
 * environment variable ZO_GEMM_SPLIT_TAIL=0 keeps every projection data-parallel (same bits). */
int zo_score(zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b, void* ws_dev,
             size_t ws_bytes, double* seq_logp_dev, float* tok_logp_dev, double* S_host, void* stream);

/* Launch amortisation: with enable != 0, zo_score captures its forward pass (embedding,
 * every layer's kernels and the head: several hundred launches) into a HIP graph on the
 * call's stream and, on later calls whose workspace, token buffer, packing sizes and side
 * geometry are the same, replays the graph instead of launching each kernel; the packing
 * tables and side factors are rewritten before every replay, so the plan's step, seeds and
 * candidates, the bank's contents and the batch's token values may change freely.  The
 * results are bitwise those of the eager launches.  Needs a stream other than the null
 * stream; per-kernel timing (zo_profile_begin) launches eagerly.  enable == 0 (the
 * default) launches eagerly and frees the graph.  One graph per model: a model shared by
 * concurrent zo_score calls must not use this. */
int zo_model_set_graphs(zo_model* m, int32_t enable);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): zo_score with the workspace taken from
 * a scratch array of ZO_NOALLOC_SCRATCH_BYTES that the library holds on each device it
 * runs on (in the code object, for the life of the process) instead of a caller buffer;
 * the caller still passes the outputs.  Allocates no device memory.  ZO_E_SHAPE if the
 * batch's workspace (zo_batch_layout) exceeds the scratch; ZO_E_DEVICE if the scratch
 * address of the model's device could not be found when the model was created.  Every
 * call on one device shares that device's scratch: calls that overlap on one device
 * (other streams or threads) race and must be serialised by the caller.  Returns after
 * synchronising `stream`, as zo_score. */
#define ZO_NOALLOC_SCRATCH_BYTES (256u << 20)
int zo_score_noalloc(zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b, double* seq_logp_dev,
                     float* tok_logp_dev, double* S_host, void* stream);

/* ---- generation queries --------------------------------------------------
 * "Inference-Native Zeroth-Order Optimization" (arXiv abstract): the candidate-state
 * formulation covers autoregressive generation as well as token scoring.  zo_generate
 * runs greedy generation of n_new tokens for every physical sequence of the packing
 * (foreground prompts under W, every probe prompt under every candidate state of the
 * plan, side path and bank as in zo_score): one prefill pass over the prompts, which also
 * fills a per-layer K/V cache in the workspace, then n_new - 1 decode steps of one row
 * per sequence attending over the cache.  Token j of a sequence is the first vocabulary
 * id holding the maximum logit at position len + j - 1 (fp32 logits).
 *   tokens_dev: device int32 [n_phys x n_new] out, the generated ids;
 *   logp_dev:   device fp32 [n_phys x n_new] out, each token's log-probability (computed
 *               in fp64 from the head's partial sums, stored fp32);
 *   S_host:     host fp64 [n_cand] out, per candidate the sum over its sequences of the
 *               generated tokens' log-probabilities (the generative objective, for
 *               zo_estimate).
 * Sequences are in zo_pack's order.  fp32, bf16 and fp8 models; not with ZO_PLAN_ACT_SPLIT or ZO_PLAN_SPLIT_*;
 * prompt length + n_new - 1 <= max_pos.  The batch's score modes are validated but not
 * used.  zo_generate_layout gives n_phys and the workspace bytes (the cache takes
 * 2 x n_layers x (sum of prompt lengths + n_phys (n_new - 1)) x n_kv_heads x head_dim
 * activation elements).  Errors as zo_score; ZO_E_INVAL for a two-term plan or
 * n_new < 1, ZO_E_SHAPE beyond max_pos. */
int zo_generate_layout(const zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b,
                       int32_t n_new, int32_t* n_phys, size_t* ws_bytes);
int zo_generate(zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b, int32_t n_new,
                void* ws_dev, size_t ws_bytes, int32_t* tokens_dev, float* logp_dev, double* S_host,
                void* stream);

/* ---- zo_estimate (host only, launches nothing) ------------------------------------
 * For each direction d with candidates (d,+1) and (d,-1):
 *   c_d = (L_{d,+} - L_{d,-}) / (2 eps),  L = -S  (or -S / n_scored with ZO_EST_MEAN)
 *   c_d /= r with ZO_EST_INV_RANK.
 * n_scored (host [n_cand]) is needed only with ZO_EST_MEAN.  Returns ZO_E_NONFINITE and
 * leaves c_out untouched if any S is NaN or infinite. */
int zo_estimate(const zo_plan_t* p, const double* S_host, const int64_t* n_scored, uint32_t flags,
                double* c_out);

/* ---- zo_update ------------------------------------------------------------------
 * Lazy low-rank update, one launch for every target linear of every layer:
 *   U_{seed_d, floor(t/nu)} <- fp32( U - (((lr / q) * c_d) * sigma) * G_d(t) )   for each direction d,
 * sigma = 1, or 1/sqrt(r) with ZO_PLAN_SCALE_INV_SQRT_R: the step theta <- theta - (lr/q) sum_d c_d z_d
 * along the directions z_d = sigma G_d V_d^T that the candidates theta +- eps z_d probed
 * ("Zeroth-Order Fine-Tuning Was an Inference Workload All Along", section "Why ZO
 * Fine-Tuning Is Really Scoring": theta <- theta - eta c z);
 * allocating (and zero-initialising) the bank entry of (seed_d, window) if absent;
 * ZO_E_NOMEM if the bank has no free slot.  W is never written. */
int zo_update(zo_model* m, const zo_plan_t* p, zo_bank* bank, const double* c_host, double lr, void* stream);

/* ---- stream access (for bit-exact checks of the random directions) -------------------
 * Tags: direction factor = (layer << 8) | (kind << 1) | factor (G = 0, V = 1);
 *       weight tensor    = (1 << 30) | (slot << 8) | param.
 * zo_philox_words: raw Philox4x32-10 blocks [first_block, first_block + n_blocks) -> device uint32 [4 n].
 * zo_normal_fill:  stream elements [first, first + n) -> device fp64 [n].
 * zo_direction:    one fp32 factor of the plan (which = 0 G [n_out x r], 1 V [n_in x r]) -> device. */
int zo_philox_words(uint64_t seed, uint32_t tag, uint64_t tau, int64_t first_block, int64_t n_blocks,
                    uint32_t* out_dev, void* stream);
int zo_normal_fill(uint64_t seed, uint32_t tag, uint64_t tau, int64_t first, int64_t n, double* out_dev,
                   void* stream);
int zo_direction(const zo_model* m, const zo_plan_t* p, int32_t dir, int32_t layer, int32_t kind, int32_t which,
                 float* out_dev, void* stream);

/* ---- per-kernel-class timing (measurement) ---------------------------------------
 * zo_profile_begin enables timing: every kernel launch of zo_score / zo_update is
 * bracketed by HIP events on the launch stream, per class below.  zo_profile_end
 * disables it, waits for the recorded events and writes, for each of the first
 * n_classes classes, the number of launches and their summed duration (ms).
 * Events come from a pool owned by the library (created on first use). */
enum { ZO_PROF_GEMM_BASE = 0,   /* shared-weight projections (qkv, o, fc1/gate-up, fc2/down) */
       ZO_PROF_GEMM_SIDE = 1,   /* side-input projections t = x [V...] */
       ZO_PROF_GEMM_HEAD = 2,   /* vocabulary head + fused log-softmax partials */
       ZO_PROF_ATTENTION = 3,
       ZO_PROF_NORM = 4,        /* embedding, LayerNorm/RMSNorm, QK-norm + RoPE */
       ZO_PROF_SIDE_PREP = 5,   /* regeneration of the G/V factors and bank packing */
       ZO_PROF_REDUCE = 6,      /* log-prob combine and per-sequence sums */
       ZO_PROF_UPDATE = 7,
       ZO_PROF_DECODE_ATTN = 8, /* generation decode steps: K/V cache append + attention over the cache */
       ZO_PROF_N_CLASSES = 9 };
int zo_profile_begin(void);
int zo_profile_end(int32_t n_classes, int64_t* counts, double* total_ms);
/* Restrict timing to the classes whose bit (1 << class) is set in class_mask (default:
   all); fewer events on the stream, e.g. only the projections while a throughput
   measurement runs. */
int zo_profile_select(uint32_t class_mask);

#ifdef __cplusplus
}
#endif
#endif /* ZO_H_ */
