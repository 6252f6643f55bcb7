/* gpt2.h -- C ABI of the MI355X (gfx950) GPT-2 training-step library.
 *
 * One training step is forward -> backward -> AdamW over a single flat device
 * arena that the caller allocates once ("1000 行 C 代码完成 GPT-2 训练的 LLM.c":
 * all memory is taken in one 1D block up front, so nothing is allocated or freed
 * while training and batches just stream through).  The model is GPT-2 as the
 * pages describe it: token + position embedding ("GPT-2 from scratch with torch",
 * token/position embedding), L pre-norm blocks x = x + attn(ln_1(x)),
 * x = x + mlp(ln_2(x)) (same page, Transformer block), causal multi-head
 * self-attention with scores scaled by 1/sqrt(head size) (same page, 自注意力;
 * "从头搭建GPT(Andrej Karpathy) 笔记", attention中为什么要做scaling), a tanh-GELU MLP
 * of width 4C (前馈网络（MLP）; the GELU formula in the comment thread of
 * "GPT-2ベースの3000バイトCで実装されたChatGPTクローン"), a final LayerNorm, logits
 * from the token-embedding matrix (tied lm_head, no bias: 3000-byte C page,
 * Transformer本体), and mean softmax cross-entropy over all B*T next-token
 * targets (CSDN notes, 计算loss).
 *
 * Conventions for every entry point
 *  - Returns a gpt2_status; nothing throws across the ABI.  On a non-OK status
 *    gpt2_last_error() returns a message (thread-local, valid until the next call
 *    on the same thread).
 *  - Device pointers are HIP device addresses; `stream` is a hipStream_t passed as
 *    void* (NULL = the null stream).  Every call only enqueues work on `stream`
 *    and never synchronises; calls on one arena must be ordered by the caller
 *    (use one stream).
 *  - The library never allocates or frees device memory.
 */
#ifndef GPT2_MI355X_H
#define GPT2_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Model hyper-parameters, named as in the llm.c run banner
 * ("1000 行 C 代码...", 快速开始吧！: max_seq_len, vocab_size, num_layers,
 * num_heads, channels). */
typedef struct gpt2_config {
    int32_t max_seq_len;
    int32_t vocab_size;
    int32_t num_layers;
    int32_t num_heads;
    int32_t channels;
} gpt2_config;

/* Arithmetic mode.
 *  GPT2_FP32: weights, activations and GEMM inputs fp32 (fp32 MFMA).
 *  GPT2_BF16: bf16 weight copy and bf16 activations as GEMM/attention inputs,
 *             fp32 accumulation, fp32 master weights, gradients, AdamW moments,
 *             LayerNorm statistics, attention log-sum-exp and losses. */
enum gpt2_dtype { GPT2_FP32 = 0, GPT2_BF16 = 1 };

enum gpt2_status {
    GPT2_OK = 0,
    GPT2_E_INVAL = -1, /* bad argument or configuration                          */
    GPT2_E_SIZE = -2,  /* device buffer smaller than gpt2_alloc_arena requires    */
    GPT2_E_ALIGN = -3, /* device buffer not 256-byte aligned                       */
    GPT2_E_STATE = -4, /* call out of order (e.g. backward without a loss forward) */
    GPT2_E_HIP = -5    /* a HIP launch or runtime call failed                      */
};

typedef struct gpt2_arena gpt2_arena; /* opaque host-side handle */

/* Lays out (and validates) an arena for `cfg` at batch B, sequence length T.
 *
 *  cfg          model shape; needs channels % num_heads == 0, channels % 8 == 0,
 *               head size (channels / num_heads) <= 128, 1 <= T <= max_seq_len,
 *               B >= 1, vocab_size >= 2.
 *  dtype        gpt2_dtype.
 *  device_base  caller-owned device memory (256-byte aligned), or NULL to only
 *               query the size.  The caller keeps ownership; it must outlive the
 *               handle and must be zero-filled before the first AdamW step (the
 *               moments start at zero).
 *  device_bytes size of device_base.
 *  required_bytes  (out, may be NULL) bytes the layout needs.
 *  out          (out) the handle, or NULL on error / size query.
 * Errors: GPT2_E_INVAL for a bad shape or dtype, GPT2_E_SIZE if device_bytes is
 * too small, GPT2_E_ALIGN if device_base is misaligned. */
int gpt2_alloc_arena(const gpt2_config* cfg, int32_t B, int32_t T, int32_t dtype,
                     void* device_base, size_t device_bytes, size_t* required_bytes,
                     gpt2_arena** out);

/* Releases the host handle only (never the device memory). NULL is a no-op. */
int gpt2_free_arena(gpt2_arena* arena);

/* Refreshes every derived copy of the fp32 master parameters (the bf16 working
 * copy in GPT2_BF16 mode; nothing in GPT2_FP32 mode).  Call after writing the
 * master parameters directly (e.g. loading weights). */
int gpt2_sync_weights(gpt2_arena* arena, void* stream);

/* Forward pass of the GPT-2 block stack ("GPT-2 from scratch with torch", 模型结构:
 * token and position embeddings, L pre-LayerNorm blocks of causal self-attention and a
 * GELU MLP, final LayerNorm, logits through the tied token embedding; the loss is the
 * mean softmax cross-entropy, "从头搭建GPT(Andrej Karpathy) 笔记", 计算loss).
 *  d_inputs   device int32 [B, T] token ids, row-major, each in [0, vocab_size).
 *  d_targets  device int32 [B, T] next-token ids (inputs shifted by one), or NULL.
 * Without targets the logits [B*T, padded_vocab] are left in GPT2_T_LOGITS.
 * With targets the fused softmax-cross-entropy writes per-position losses
 * (GPT2_T_LOSSES), their mean (GPT2_T_LOSS) and overwrites GPT2_T_LOGITS with
 * d loss / d logits, ready for gpt2_backward.  Ids are not range-checked on the
 * device: an id outside [0, vocab_size) is undefined behaviour (the Python
 * binding checks them on the host).  Both arrays must stay valid until the
 * enqueued work has run (the backward pass reads d_inputs again).  With B >= 2 (and
 * the MX format and the launch profiler off) the batch runs as two groups of
 * sequences, one of them on the arena's second stream (gpt2_set_side_stream), forked
 * from and joined back into `stream`; the results are bitwise those of one pass. */
int gpt2_forward(gpt2_arena* arena, const int32_t* d_inputs, const int32_t* d_targets, void* stream);

/* Validation loss: the mean over `num_batches` batches of the forward pass's mean loss
 * ("1000 行 C 代码完成 GPT-2 训练的 LLM.c", 快速开始吧: the trainer reports a val loss
 * averaged over a fixed number of validation batches).
 *  d_inputs, d_targets  device int32 [num_batches, B, T] token ids and next-token ids
 *  d_loss               device fp32 scalar receiving the mean (batch means added in
 *                       batch order, each times 1/num_batches)
 * No backward pass may follow (GPT2_E_STATE until the next gpt2_forward with targets).
 * Errors: GPT2_E_INVAL for NULL pointers or num_batches < 1; those of gpt2_forward. */
int gpt2_eval_loss(gpt2_arena* arena, const int32_t* d_inputs, const int32_t* d_targets, int32_t num_batches,
                   float* d_loss, void* stream);

/* Backward pass of the last forward (which must have had targets, else
 * GPT2_E_STATE): the gradient of the mean loss with respect to every parameter, by
 * the chain rule through the forward's layers in reverse ("1000 行 C 代码完成 GPT-2
 * 训练的 LLM.c": forward, backward and update, each layer's backward hand-written).
 * Overwrites every fp32 parameter gradient (GPT2_T_GRADS): one micro-batch per step,
 * no accumulation.  The parameter-gradient products run on the arena's second stream
 * (gpt2_set_side_stream) that forks from and joins back into `stream` with events, so
 * all of the pass is ordered before whatever the caller enqueues on `stream` next.
 * Results are bitwise reproducible run to run.  Two passes on the same arena must not
 * be enqueued on different streams concurrently. */
int gpt2_backward(gpt2_arena* arena, void* stream);

/* Gives the arena the second stream its forward and backward passes overlap work on
 * (a stream of the same device, other than the ones the passes are called with).  The
 * caller keeps ownership: it must outlive every pass enqueued until the next call or
 * gpt2_free_arena.  NULL (the default) lets the library create its own stream on first
 * use and destroy it in gpt2_free_arena; a stream the library created earlier is
 * synchronized and destroyed here.  Errors: GPT2_E_INVAL for a NULL arena, GPT2_E_HIP. */
int gpt2_set_side_stream(gpt2_arena* arena, void* stream);

/* AdamW over every parameter ("1000 行 C 代码...": the loop ends with an Adam
 * update; decoupled weight decay, bias correction, t counted from 1):
 *   m = beta1 m + (1-beta1) g;  v = beta2 v + (1-beta2) g^2
 *   theta -= lr * ( m/(1-beta1^t) / (sqrt(v/(1-beta2^t)) + eps) + weight_decay * theta )
 * then refreshes the bf16 copy (round to nearest even) in GPT2_BF16 mode.
 * Errors: GPT2_E_INVAL if step < 1. */
int gpt2_adamw_step(gpt2_arena* arena, float lr, float beta1, float beta2, float eps,
                    float weight_decay, int32_t step, void* stream);

/* gpt2_backward followed by gpt2_adamw_step, fused: each layer's AdamW update is
 * enqueued on the backward pass's second stream as soon as that layer's gradients are
 * complete and the pass no longer reads its weights, so it overlaps the backward pass
 * of the layers below; the embeddings and ln_f are updated last.  Gradients, moments
 * and parameters are bitwise identical to the two separate calls.  Same arguments and
 * errors as gpt2_backward and gpt2_adamw_step (GPT2_E_STATE without a preceding loss
 * forward, GPT2_E_INVAL if step < 1). */
int gpt2_backward_adamw(gpt2_arena* arena, float lr, float beta1, float beta2, float eps,
                        float weight_decay, int32_t step, void* stream);

/* Tensor ids for gpt2_tensor_info.  Model-level tensors ignore `layer`;
 * per-layer tensors need 0 <= layer < num_layers. */
enum gpt2_tensor_id {
    GPT2_T_PARAMS = 0,      /* fp32 [num_parameters] master weights                    */
    GPT2_T_GRADS = 1,       /* fp32 [num_parameters]                                   */
    GPT2_T_ADAM_M = 2,      /* fp32 [num_parameters]                                   */
    GPT2_T_ADAM_V = 3,      /* fp32 [num_parameters]                                   */
    GPT2_T_PARAMS_BF16 = 4, /* bf16 [num_parameters] working copy (GPT2_BF16 only)     */
    GPT2_T_ENCODED = 5,     /* act [B*T, C] embedding output                           */
    GPT2_T_LNF = 6,         /* act [B*T, C] final LayerNorm output                     */
    GPT2_T_LNF_STATS = 7,   /* fp32 [B*T, 2] (mean, 1/std)                             */
    GPT2_T_LOGITS = 8,      /* act [B*T, padded_vocab]: logits, or dlogits (see forward) */
    GPT2_T_LOSSES = 9,      /* fp32 [B*T]                                              */
    GPT2_T_LOSS = 10,       /* fp32 [1] mean loss                                      */
    /* per layer */
    GPT2_T_LN1 = 16,        /* act [B*T, C]                                            */
    GPT2_T_LN1_STATS = 17,  /* fp32 [B*T, 2]                                           */
    GPT2_T_QKV = 18,        /* act [B*T, 3C] columns q | k | v, head h at h*hs         */
    GPT2_T_ATTY = 19,       /* act [B*T, C] attention output, heads side by side       */
    GPT2_T_ATT_LSE = 20,    /* fp32 [B, NH, T] log-sum-exp of each scaled score row    */
    GPT2_T_RESIDUAL2 = 21,  /* act [B*T, C] x + attn                                   */
    GPT2_T_LN2 = 22,        /* act [B*T, C]                                            */
    GPT2_T_LN2_STATS = 23,  /* fp32 [B*T, 2]                                           */
    GPT2_T_FCH = 24,        /* act [B*T, 4C] pre-GELU                                  */
    GPT2_T_FCH_GELU = 25,   /* act [B*T, 4C]                                           */
    GPT2_T_RESIDUAL3 = 26   /* act [B*T, C] block output                               */
};

/* Where a tensor lives in the arena (the single up-front allocation of "1000 行 C 代码
 * 完成 GPT-2 训练的 LLM.c", laid out by gpt2_alloc_arena).  All outputs may be NULL.
 * A layer index and a two-dimensional shape with a row stride are part of the answer:
 * per-layer tensors are addressed one layer at a time, and some rows are padded
 * (the logits to a multiple of 64 columns).
 *  byte_offset  from device_base (256-byte aligned)
 *  rows, cols   logical shape; row_stride >= cols elements between rows
 *  dtype        GPT2_FP32 or GPT2_BF16 ("act" tensors follow the arena dtype)
 * Errors: GPT2_E_INVAL for an unknown id, a bad layer, or PARAMS_BF16 in fp32 mode. */
int gpt2_tensor_info(const gpt2_arena* arena, int32_t tensor_id, int32_t layer, size_t* byte_offset,
                     int64_t* rows, int64_t* cols, int64_t* row_stride, int32_t* dtype);

/* Number of parameters (equals the llm.c banner's num_parameters for GPT-2 124M). */
int64_t gpt2_num_parameters(const gpt2_config* cfg);

/* Launch profiler (process-wide, all arenas).  gpt2_profile(1) clears earlier
 * records and starts recording a pair of HIP events on the launching stream around
 * every kernel launch, tagged with the kernel name and the launch's algorithmic
 * work (flops of its contractions counting only unmasked attention pairs; bytes
 * it must read and write at least once).  gpt2_profile(0) stops recording.
 * At most 32768 launches are recorded per enable.  Timing adds a small per-launch
 * overhead, and while recording, gpt2_backward enqueues all of its work on the
 * caller's stream (normally it overlaps parameter-gradient work on an internal
 * second stream) so that each launch's duration is its own; the benchmark times
 * its headline figure with profiling off. */
typedef struct gpt2_kernel_stat {
    char name[64];
    int64_t launches;
    double total_ms;   /* sum of per-launch event durations */
    double flops;      /* sum of algorithmic flops          */
    double bytes;      /* sum of algorithmic bytes          */
} gpt2_kernel_stat;

int gpt2_profile(int enable);

/* Waits for the recorded events and writes one aggregate per kernel name (sorted
 * by name) into out[0..max_entries); *n_entries receives the number of names.
 * Errors: GPT2_E_HIP if an event cannot be read. */
int gpt2_profile_read(gpt2_kernel_stat* out, int32_t max_entries, int32_t* n_entries);

/* Order of the recorded launches: out[i] (i < max_entries) receives the index, in
 * the name-sorted array gpt2_profile_read fills, of the i-th launch recorded since
 * gpt2_profile(1); *n_entries receives the number of recorded launches.  Each
 * recorded launch is one kernel dispatch of the library, so a trace of the same
 * steps can be matched to kernel names dispatch by dispatch.  No GPU work. */
int gpt2_profile_order(int32_t* out, int32_t max_entries, int32_t* n_entries);

/* Matrix-core rate probe (measurement only).  Launches, on `stream`, a kernel in
 * which every wave of 2 per SIMD issues independent chains of one MFMA form on
 * register operands (no memory traffic), times four launches with HIP events,
 * waits for them, and writes the fastest of the last three as TFLOP/s (dense,
 * 2 flops per multiply-add) to *tflops: the rate the chip sustains at the clock
 * it holds under that load, next to which the published peak is the upper bound.
 *  kind 0: v_mfma_f32_32x32x16_bf16; 1: v_mfma_f32_16x16x32_bf16;
 *       2: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands.
 * Synchronises the stream.  Errors: GPT2_E_INVAL (NULL tflops, unknown kind),
 * GPT2_E_HIP (launch or event failure). */
int gpt2_mfma_peak(int32_t kind, double* tflops, void* stream);

/* ---------------------------------------------------------------- generation
 * Incremental next-token prediction with a key/value cache
 * ("GPT-2ベースの3000バイトCで実装されたChatGPTクローン", KVキャッシュ方式: after N tokens
 * have been run, token N+1 needs only its own row; the earlier rows' results are kept
 * where they were written instead of being recomputed).  A generation state borrows
 * an arena's parameters (bf16 arenas with head size 64) and keeps, in its own
 * caller-owned device memory, the q|k|v rows of every layer for `batch` sequences of
 * up to `max_len` tokens ([L][batch][max_len][3C] bf16) plus the decode scratch.
 * All sequences of a state advance together (one shared length). */
typedef struct gpt2_gen gpt2_gen; /* opaque host-side handle */

/* Lays out a generation state over `arena`.
 *  batch        1..16 sequences; max_len 1..cfg.max_seq_len positions.
 *  device_base  caller-owned device memory (256-byte aligned) or NULL to only query
 *               the size (*required_bytes); it must outlive the handle.  No
 *               zero-filling is needed.
 * The arena must outlive the handle.  Errors: GPT2_E_INVAL (NULL arena, fp32 arena,
 * head size other than 64, channels > 2048, batch or max_len out of range, out NULL), GPT2_E_ALIGN,
 * GPT2_E_SIZE (device_bytes too small). */
int gpt2_gen_alloc(gpt2_arena* arena, int32_t batch, int32_t max_len, void* device_base, size_t device_bytes,
                   size_t* required_bytes, gpt2_gen** out);

/* Frees the host handle only (never device memory). */
int gpt2_gen_free(gpt2_gen* gen);

/* Current length of the cached sequences (0 before the first prefill; -1 for NULL). */
int gpt2_gen_length(const gpt2_gen* gen);

/* Runs the prompt d_tokens (device int32 [batch, n], row-major) through the full
 * forward pass in the arena's activation buffers (needs batch * n <= arena B * T;
 * the arena's training activations are overwritten, so a later gpt2_backward needs
 * a new gpt2_forward with targets), copies every layer's q|k|v rows into the cache,
 * sets the length to n, and writes the next-token logits of each sequence (position
 * n - 1, the forward pass's bf16 logits widened) to d_logits (device fp32 [batch, V]).
 * Errors: GPT2_E_INVAL (NULL argument), GPT2_E_SIZE (n outside 1..max_len or too many
 * rows for the arena), GPT2_E_HIP. */
int gpt2_gen_prefill(gpt2_gen* gen, const int32_t* d_tokens, int32_t n, float* d_logits, void* stream);

/* Appends one token per sequence (d_tokens: device int32 [batch]) at position
 * length: runs that row through every layer (its q|k|v row is written into the
 * cache, attention reads cache rows 0..length), writes the next-token logits
 * (device fp32 [batch, V], fp32 accumulation, no bf16 rounding) and increments the
 * length.  Errors: GPT2_E_INVAL (NULL argument), GPT2_E_STATE (no prefill yet),
 * GPT2_E_SIZE (length == max_len), GPT2_E_HIP. */
int gpt2_gen_decode(gpt2_gen* gen, const int32_t* d_tokens, float* d_logits, void* stream);

/* Allocation-free decode step, for callers that cannot allocate device memory or
 * bring a workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, results and errors as gpt2_gen_decode (the same
 * kernels, bit-identical logits), but the step's row buffers (residual rows, attention
 * and GELU outputs, final LayerNorm rows and statistics: about 20 * batch * channels
 * bytes) live in a static device array of the library, 384 KiB on each GPU, held
 * until the process ends, instead of in the generation state's memory (its key/value
 * cache is still used).  The array is looked up on the calling thread's current
 * device, which must be the device of `g`'s memory and of `stream`; the first call on
 * a device looks up that device's copy.  Every call on one GPU shares its array:
 * calls that overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  Nothing in the array needs clearing: each step writes
 * every row it reads.  Allocates nothing (no hipMalloc / hipFree).
 * Errors: as gpt2_gen_decode; GPT2_E_SIZE when batch * channels needs more than the
 * array holds (batch * channels above about 19660), checked before any GPU call;
 * GPT2_E_HIP if the array's device address cannot be looked up. */
int gpt2_gen_decode_noalloc(gpt2_gen* g, const int32_t* d_tokens, float* d_logits, void* stream);

/* Top-k sampling on the host ("GPT-2 from scratch with torch", 生成样本: keep the k
 * highest logits, softmax over them, draw one token).  For each of `rows` rows of
 * host fp32 logits (row stride ld >= V): rank the tokens by logit (equal logits: the
 * lower id first; NaN ranks last), keep the first min(k, V), weight them
 * w_i = exp((z_i - z_max) / temperature) in double precision, and return the first
 * kept token, in rank order, whose running weight sum exceeds uniforms[r] * sum(w).
 * A leading logit that is not finite returns the leader.  uniforms: host fp32 [rows]
 * in [0, 1) (the caller's random numbers); tokens_out: host int32 [rows].
 * Errors: GPT2_E_INVAL for NULL pointers, rows < 0, V < 1, ld < V, k < 1,
 * temperature not finite and > 0, or a uniform outside [0, 1). */
int gpt2_sample_topk(const float* logits, int32_t rows, int32_t V, int64_t ld, int32_t k, float temperature,
                     const float* uniforms, int32_t* tokens_out);

/* ---------------------------------------------------------------- files (host memory only)
 * Token streams ("1000 行 C 代码完成 GPT-2 训练的 LLM.c", 快速开始吧: a .bin file is a raw
 * stream of int32 GPT-2 token ids).  Batch i of B sequences of T tokens is the B*T + 1
 * ids starting at id i*B*T: inputs are its first B*T ids, targets the same shifted by
 * one, row-major [B, T].  A stream of n ids holds n / (B*T) batches (the page's run
 * banner: 32768 ids -> 128 batches, 305260 -> 1192, at B*T = 256); if the last batch's
 * final target would lie past the end it is id 0 (the stream wraps). */

/* Number of int32 ids in the file, or a negative status (GPT2_E_INVAL: cannot open;
 * GPT2_E_SIZE: the size is not a multiple of 4 bytes). */
int64_t gpt2_tokens_count(const char* path);

/* Reads batch `batch` into host int32 inputs / targets [B*T] each.  Errors:
 * GPT2_E_INVAL (NULL argument, B or T < 1, cannot open), GPT2_E_SIZE (batch outside
 * 0 .. num_batches - 1, short read). */
int gpt2_tokens_batch(const char* path, int32_t B, int32_t T, int64_t batch, int32_t* inputs, int32_t* targets);

/* Parameter orders of a flat fp32 weight array: the arena's (layer blocks in numeric
 * order) and the order of weight files that sort their layers by name
 * ("GPT-2ベースの3000バイトCで実装されたChatGPTクローン", 重みの読み込み: the blocks of
 * layers 0, 1, 10, 11, 2, .. as the decimal indices sort as text).  Everything else -
 * wte, wpe before the layers, ln_f after them, the tensors inside a layer block - is in
 * the same place in both. */
enum gpt2_param_order { GPT2_ORDER_NUMERIC = 0, GPT2_ORDER_LEXICOGRAPHIC = 1 };

/* dst (host fp32 [gpt2_num_parameters]) = src reordered from one layer order to the
 * other.  Errors: GPT2_E_INVAL for a bad config, NULL or identical arrays, unknown order. */
int gpt2_params_permute(const gpt2_config* cfg, const float* src, float* dst, int32_t from_order, int32_t to_order);

/* Checkpoint file: a 64-byte header (int32 magic "GPT2", version 1, the five config
 * fields, has-moments flag, AdamW step, 7 zeros) followed by the fp32 parameters in the
 * arena's order and, if m and v are given, the two AdamW moment arrays.  Host arrays of
 * gpt2_num_parameters(cfg) floats; m and v both or neither.  Written to path + ".tmp"
 * and renamed.  Errors: GPT2_E_INVAL (bad arguments, cannot create), GPT2_E_SIZE (write
 * failed). */
int gpt2_checkpoint_write(const char* path, const gpt2_config* cfg, int32_t step, const float* params,
                          const float* m, const float* v);

/* Reads a checkpoint written by gpt2_checkpoint_write for the same model shape into
 * params (and m, v when both are non-NULL and the file has moments); *step and
 * *has_moments (each may be NULL) receive the header's values.  Errors: GPT2_E_INVAL
 * (bad arguments, cannot open, not a checkpoint, different model shape), GPT2_E_SIZE
 * (short read). */
int gpt2_checkpoint_read(const char* path, const gpt2_config* cfg, int32_t* step, float* params, float* m, float* v,
                         int32_t* has_moments);

/* Block types.
 *  GPT2_BLOCK_GPT2:  the GPT-2 block described at the top of this file.
 *  GPT2_BLOCK_LLAMA: a Llama-style block ("1000 行 C 代码完成 GPT-2 训练的 LLM.c" lists
 *    RoPE and the layers of Llama-2-type models as the next additions):
 *    x = x + attn(rms_1(x)), x = x + down(silu(g) * u) with (g | u) = rms_2(x) W_gu^T;
 *    RMSNorm y = x / sqrt(mean(x^2) + 1e-5) * w; no biases; the rotary position
 *    embedding (base 10000 unless set otherwise) instead of wpe; a final RMSNorm and
 *    the tied lm_head.  The MLP width is H = 8C/3 rounded up to a multiple of 64.
 *    Parameters, layer-major: wte, wpe (kept, unused, zero gradient), per layer
 *    [rms_1 w (C); qkv W (3C x C); proj W (C x C); rms_2 w (C); gate|up W (2H x C, row
 *    2j the gate of hidden unit j, row 2j+1 its up); down W (C x H)], final rms w (C).
 *    Not available with it: MX products and generation (GPT2_E_INVAL); checkpoint files
 *    describe GPT-2 arenas. */
enum gpt2_block { GPT2_BLOCK_GPT2 = 0, GPT2_BLOCK_LLAMA = 1 };

/* Parameter count of a block type (-1 for a NULL cfg or unknown block). */
int64_t gpt2_num_parameters_block(const gpt2_config* cfg, int32_t block);

/* gpt2_alloc_arena with a block type; GPT2_BLOCK_GPT2 is gpt2_alloc_arena itself.
 * Errors as gpt2_alloc_arena, and GPT2_E_INVAL for an unknown block. */
int gpt2_alloc_arena_block(const gpt2_config* cfg, int32_t block, int32_t B, int32_t T, int32_t dtype,
                           void* device_base, size_t device_bytes, size_t* required_bytes, gpt2_arena** out);

/* Position encoding of an arena's model (GPT2_BLOCK_LLAMA: always rotary).
 *  GPT2_POS_LEARNED: x = wte[token] + wpe[position] (GPT-2; the default).
 *  GPT2_POS_ROTARY:  rotary position embedding ("GPT-2 from scratch with torch", token
 *    and position embedding, names RoPE - Su et al. 2021 - as the newer alternative):
 *    x = wte[token]; after the qkv product the pair (x[2i], x[2i+1]) of every query and
 *    key head at position m is turned by the angle m * base^(-2i / head size); values
 *    are untouched.  wpe stays in the parameter array, unused, with a zero gradient.
 * Applies to gpt2_forward, gpt2_backward(_adamw) and generation.  Switching to
 * GPT2_POS_ROTARY builds the arena's cos / sin table on `stream` (float64 angles).
 * Errors: GPT2_E_INVAL (NULL arena, unknown mode, base not finite or <= 1), GPT2_E_HIP. */
enum gpt2_position_encoding { GPT2_POS_LEARNED = 0, GPT2_POS_ROTARY = 1 };
int gpt2_set_position_encoding(gpt2_arena* arena, int32_t mode, float base, void* stream);

/* ---------------------------------------------------------------------------
 * Products below 16 bits: MX FP8.  The llm.c page ("1000 行 C 代码完成 GPT-2 训练的
 * LLM.c", the paragraph on extensions after the CUDA port) names taking the trainer's
 * precision down to fp16 and below as the next step.  Below 16 bits this library uses
 * the block-scaled 8-bit format gfx950's matrix cores take natively (OCP MXFP8):
 *  - an element is an E4M3 code (sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *    subnormals at exponent 0; S.1111.111 is NaN; largest magnitude 448);
 *  - 32 consecutive values along k share one scale 2^e, stored as the byte e + 127;
 *  - e is the smallest integer with max|x| <= 448 * 2^e over the block (clamped to
 *    [-127, 127]; an all-zero block has e = -127), and each code is x / 2^e rounded
 *    to the nearest E4M3 value, ties to the even mantissa (the sign is kept: small
 *    negatives give -0).
 * Layouts: codes of a [rows, K] matrix are rows of Kp = K rounded up to 128 bytes
 * (zero codes past K) with a row stride of at least Kp; scales are
 * [Kp / 128][rows][4] bytes - byte j of row r's word in k-stage t is the scale of
 * k-block 4t + j - so that a tile of rows streams its scales in one piece.
 * --------------------------------------------------------------------------- */

/* GEMM formats of an arena's products. */
enum gpt2_gemm_format {
    GPT2_GEMM_BF16 = 0,     /* the arena's dtype (default)                                   */
    GPT2_GEMM_MXFP8 = 1,    /* the block (qkv, attention projection, fc, fc projection) and
                               lm_head products of gpt2_forward / gpt2_gen_prefill run on MX
                               codes; everything else, and the backward pass, unchanged */
    GPT2_GEMM_MXFP8_DX = 2, /* as GPT2_GEMM_MXFP8, and the backward pass's input-gradient
                               products of the same five layers (dX = dY W) run on MX codes
                               of dY's rows and of W's columns (the rows of W^T, blocks of 32
                               along the layer's outputs); the weight gradients stay bf16 */
};

/* Gives a bf16 arena the device memory the MX formats need: codes and scales of the
 * forward weights and of their transposes (made from the bf16 weight copy at the first
 * MX forward after any change of the weights: gpt2_sync_weights, gpt2_adamw_step,
 * gpt2_backward_adamw; the transposes only under GPT2_GEMM_MXFP8_DX), buffers for the
 * quantized input of the product at hand and for the upstream gradient of an
 * input-gradient product (up to B*T x vocab).  device_base NULL: only
 * *required_bytes is set.  The memory stays the caller's; it must outlive the arena's
 * use of the MX format.  Errors: GPT2_E_INVAL (NULL arena, not GPT2_BF16),
 * GPT2_E_ALIGN (not 256-byte aligned), GPT2_E_SIZE (too small). */
int gpt2_mx_attach(gpt2_arena* arena, void* device_base, size_t device_bytes, size_t* required_bytes);

/* Selects the format of the products.  Errors: GPT2_E_INVAL (unknown format, an MX
 * format for a Llama-style arena), GPT2_E_STATE (an MX format before gpt2_mx_attach). */
int gpt2_set_gemm_format(gpt2_arena* arena, int32_t format);

/* Codes and scales of forward weight `index` (0 <= index <= 4 L: 4 l + 0..3 are layer l's
 * qkv, attention projection, fc and fc projection weights, 4 L the tied token
 * embedding), as byte offsets into the memory given to gpt2_mx_attach: with
 * transposed = 0 the codes of W [rows = outputs, ld = inputs rounded up to 128], with
 * transposed = 1 those of W^T [rows = inputs, ld = outputs rounded up to 128] (made only
 * under GPT2_GEMM_MXFP8_DX).  Valid after a forward pass in the format.  Errors:
 * GPT2_E_INVAL, GPT2_E_STATE (no MX memory). */
int gpt2_mx_weight_codes(const gpt2_arena* arena, int32_t index, int32_t transposed, size_t* codes_offset,
                         size_t* scales_offset, int64_t* rows, int64_t* ld);

/* The arena's MX input buffers, as byte offsets into the memory given to
 * gpt2_mx_attach: codes [rows, ld] and scales [ld / 128][rows][4] of
 *  GPT2_MX_BUF_INPUT - the C-wide product inputs (LayerNorm outputs, attention
 *                      output); after a forward pass: ln_f's output,
 *  GPT2_MX_BUF_GELU  - the 4C-wide GELU output; after a forward pass: the last layer's,
 *  GPT2_MX_BUF_DY    - under GPT2_GEMM_MXFP8_DX, the upstream gradient of the input-gradient
 *                      product at hand; after a forward pass with targets: the codes of the
 *                      logits' gradient (ld = the vocabulary rounded up to 128), which the
 *                      softmax-CE kernel writes beside the gradient itself.
 * rows = B*T.  Errors: GPT2_E_INVAL, GPT2_E_STATE (no MX memory). */
enum gpt2_mx_buffer_id { GPT2_MX_BUF_INPUT = 0, GPT2_MX_BUF_GELU = 1, GPT2_MX_BUF_DY = 2 };
int gpt2_mx_buffer(const gpt2_arena* arena, int32_t which, size_t* codes_offset, size_t* scales_offset,
                   int64_t* rows, int64_t* ld);

/* MX quantization: device bf16 x [rows, K] (row stride ldx elements) -> device codes
 * [rows, Kp] (row stride ldq bytes) and scales [Kp / 128][rows][4] bytes, as defined
 * above.  Needs K % 8 == 0, ldx >= K (a multiple of 8), ldq >= Kp (a multiple of 16);
 * inputs finite.  Errors: GPT2_E_INVAL, GPT2_E_HIP. */
int gpt2_mx_quantize(const void* d_x, int64_t ldx, int32_t rows, int32_t K, void* d_codes, int64_t ldq,
                     void* d_scales, void* stream);

/* Epilogues of gpt2_mx_gemm (bias may be NULL for none). */
enum gpt2_mx_epilogue {
    GPT2_EPI_BIAS = 0,      /* C = A B^T + bias                                    */
    GPT2_EPI_BIAS_RES = 1,  /* C = residual + A B^T + bias (residual [M, ldc])     */
    GPT2_EPI_BIAS_GELU = 2, /* C = A B^T + bias, C2 = GELU(C) (C2 [M, ldc])         */
    GPT2_EPI_GELU_BWD = 3,  /* C = (A B^T) * GELU'(residual) (no bias): the GELU
                               input's gradient, residual = the GELU input [M, ldc] */
};

/* The block-scaled product C = A B^T on MX operands, fp32 accumulation, bf16 output:
 * A codes [M, K] (row stride lda bytes) with scales d_sa [K / 128][M][4], B codes
 * [N, K] (ldb) with scales d_sb [K / 128][N][4]; K a multiple of 128 (pad with zero
 * codes), lda / ldb multiples of 16, ldc (elements) >= N and a multiple of 8; bias
 * fp32 [N].  Errors: GPT2_E_INVAL, GPT2_E_SIZE (operands over 4 GiB), GPT2_E_HIP. */
int gpt2_mx_gemm(const void* d_qa, const void* d_sa, int64_t lda, const void* d_qb, const void* d_sb, int64_t ldb,
                 void* d_c, int64_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue, const float* d_bias,
                 const void* d_residual, void* d_c2, void* stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char* gpt2_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_MI355X_H */
