/*
 * nc.h -- C ABI of the gfx950 (MI355X) forward pass of nanochat's GPT:
 * batched prefill and KV-cache incremental decode.
 *
 * The model computed (sources: yelogs.com nanochat launch write-up, section on technical
 * details and the author's Q&A, architecture answer; apidog.com/th "How to train your own
 * ChatGPT for $50", section "How nanochat works", parts 1 (GPT model), 3 (precision) and
 * 6 (inference engine); geoz.com.cn summary, development-tricks section):
 *
 *   x      = norm(wte[token])                                  (fp32 residual stream)
 *   per layer l:
 *     h    = norm(x)
 *     q    = norm(rope(h Wq^T, pos)) per head,  k = norm(rope(h Wk^T, pos)),  v = h Wv^T
 *     y_h  = softmax(q_h k_g^T / sqrt(hd) + causal mask) v_g,  g = h / (n_head / n_kv_head)
 *            (n_kv_head K/V heads, each shared by a group of query heads: n_kv_head == 1
 *            is multi-query attention, n_kv_head == n_head plain multi-head attention)
 *     x   += concat_h(y_h) Wo^T
 *     x   += relu(norm(x) Wfc^T)^2 Wproj^T
 *   logits = cap * tanh(norm(x) Wlm^T / cap)                   (fp32)
 *
 * norm(z) = z / sqrt(mean(z^2) + eps) has no parameters.  RoPE rotates the pair
 * (i, i + hd/2) by pos * base^(-2i/hd).  Linear layers have no bias; weights are stored
 * [out, in] as in torch.nn.Linear.  Matrix products take dtype operands (bf16 or fp32)
 * with fp32 accumulation; the residual stream, norms, softmax and logits are fp32.  With
 * bf16, the inputs of the MLP products and of the LM head are carried as two bf16 parts
 * (a = hi + lo) and multiplied part by part, so their operand rounding error is about
 * 2^-17 instead of 2^-9; the KV cache and the other operands are bf16.
 *
 * Conventions for every call:
 *  - Every pointer named *_dev is device memory on the current HIP device; pointers named
 *    *_host are host memory.  Device buffers must be 16-byte aligned.
 *  - Calls that take a `stream` (a hipStream_t passed as void*, NULL = default stream) only
 *    enqueue work and return; the caller keeps inputs alive and reads outputs after the
 *    stream reaches that point.  One nc_kv must not be used on two streams at once.
 *  - Every call returns NC_OK (0) or a negative nc_status.  On error nothing is enqueued
 *    and no state changes; nc_last_error() returns a message for the calling thread.
 *    Faults of already-enqueued kernels surface as NC_ERR_DEVICE from a later call.
 *  - No C++ exception and no abort crosses this boundary.
 */
#ifndef NC_H
#define NC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t nc_status;

#define NC_OK 0
#define NC_ERR_INVALID_ARG (-1) /* null pointer, bad size or shape, mismatched batch     */
#define NC_ERR_UNSUPPORTED (-2) /* valid but not supported (head_dim, n_kv_head, device) */
#define NC_ERR_OOM (-3)         /* device allocation failed                               */
#define NC_ERR_CAPACITY (-4)    /* a row would exceed the cache's max_seq                 */
#define NC_ERR_STATE (-5)       /* call not allowed in the object's state                 */
#define NC_ERR_DEVICE (-6)      /* no usable GPU, or a HIP runtime error                  */

#define NC_F32 0
#define NC_BF16 1

#define NC_ABI_VERSION 1

/* Model shape.  Requirements: d_model == n_head * head_dim; n_kv_head >= 1 divides n_head
 * (NC_ERR_INVALID_ARG otherwise) with at most 16 query heads per K/V head
 * (NC_ERR_UNSUPPORTED otherwise); head_dim in {64, 128}; d_model <= 4096; d_model, d_ff
 * multiples of 64; vocab >= 1; max_seq >= 1 (longest position the RoPE table covers);
 * softcap > 0; norm_eps >= 0. */
typedef struct nc_config {
    int32_t n_layer;
    int32_t d_model;
    int32_t n_head;
    int32_t n_kv_head;
    int32_t head_dim;
    int32_t d_ff;
    int32_t vocab;
    int32_t max_seq;
    float rope_base;
    float softcap;
    float norm_eps;
    int32_t dtype; /* NC_F32 or NC_BF16: storage type of weights, matmul operands, KV cache */
} nc_config;

typedef struct nc_model nc_model; /* weights + RoPE table, owned by the library          */
typedef struct nc_kv nc_kv;       /* KV cache + per-row lengths + workspace, library-owned */

/* Build a model from 6*n_layer + 2 device tensors of cfg->dtype elements, row-major
 * [out, in], in canonical order:
 *   wte [vocab, d_model],
 *   per layer: Wq [n_head*hd, d], Wk [n_kv_head*hd, d], Wv [n_kv_head*hd, d],
 *              Wo [d, n_head*hd],
 *              Wfc [d_ff, d], Wproj [d, d_ff],
 *   lm_head [vocab, d_model].
 * The library copies (and repacks) them into memory it owns, synchronously; the caller may
 * free its tensors when this returns.  Fails with NC_ERR_DEVICE if no gfx950 GPU is
 * current, NC_ERR_UNSUPPORTED / NC_ERR_INVALID_ARG for a bad cfg. */
nc_status nc_model_create(const nc_config* cfg, const void* const* weights_dev,
                          nc_model** out);
void nc_model_free(nc_model* m); /* NULL is a no-op; all kv objects must be freed first */

/* Sliding-window attention per layer (the later version's configurable pattern of short
 * and long windows, apidog.com/th guide, part 1 architecture features; the window size
 * argument of the attention call, part 5).  windows_host: n_layer int32 values; for
 * w >= 0 a query at position p of that layer attends to keys p - w .. p only, w < 0 to
 * the whole causal context 0..p (the default of a new model).  Allowed only while the
 * model has no nc_kv object (NC_ERR_STATE otherwise); copies the values. */
nc_status nc_model_set_windows(nc_model* m, const int32_t* windows_host);

/* The later version's learned blocks (apidog.com/th guide, part 1: value embeddings on some
 * layers with an input-dependent gate, per-layer residual scaling against x0, smear and
 * backout; the pages give their update rules only, so these are the readings):
 *   e_t    = norm(wte[token_t]);  smear: x_t = e_t + smear_lambda sigmoid(e_t[:Cs] . g) e_{t-1}
 *            (e_{t-1} the row's previous token's; none at position 0); x0 = x;
 *   layer l starts with x <- resid_lambda[l] x + x0_lambda[l] x0;
 *   layers with a value embedding: value head j gains
 *            3 sigmoid(h[:Cv] . ve_gate[l][j]) ve[l][token][j hd .. (j+1) hd), h = norm(x)
 *            the attention input;
 *   backout: xb = x at the start of layer backout_layer; after the last layer
 *            x <- x - backout_lambda xb, before the final norm.
 * Tables are device memory of cfg.dtype, copied by the library; scalars are host values.
 * ex == NULL switches every block off (the default).  Allowed only while the model has no
 * nc_kv object (NC_ERR_STATE); NC_ERR_INVALID_ARG for channels outside [1, min(64, d_model)],
 * a backout layer outside [-1, n_layer) or tables that are not device memory. */
typedef struct nc_extras {
    const float* resid_lambda_host;   /* n_layer values, or NULL: all 1 */
    const float* x0_lambda_host;      /* n_layer values, or NULL: all 0 */
    const void* smear_gate_dev;       /* [smear_channels], or NULL: no smear */
    int32_t smear_channels;
    float smear_lambda;
    int32_t backout_layer;            /* -1: no backout */
    float backout_lambda;
    const void* const* ve_dev;        /* n_layer pointers (NULL entries: no value embedding in
                                         that layer) to [vocab][n_kv_head * head_dim], or NULL */
    const void* const* ve_gate_dev;   /* n_layer pointers to [n_kv_head][ve_channels] */
    int32_t ve_channels;
} nc_extras;
nc_status nc_model_set_extras(nc_model* m, const nc_extras* ex);

/* KV cache for `batch` rows of up to `max_seq` positions (max_seq <= cfg.max_seq, and at
 * most 32768: NC_ERR_UNSUPPORTED otherwise).  The cache of the pages' inference engine:
 * keys and values of every processed position kept per layer so that each new token
 * attends to them without recomputation (szyisi.cn launch article, section on the base
 * model's evaluation: an Engine class with a KV cache and the two inference stages,
 * prefill and decode; apidog.com/th guide, part 6: the prompt's cache filled once, then
 * read by flash_attn_with_kvcache).
 * Layout (library-private): K [L][batch][n_kv_head][max_seq][hd], V transposed
 * [L][batch][n_kv_head][hd][max_seq],
 * both cfg.dtype; keys are stored after RoPE and QK-norm.  All lengths start at 0. */
nc_status nc_kv_create(nc_model* m, int32_t batch, int32_t max_seq, nc_kv** out);
void nc_kv_free(nc_kv* kv); /* NULL is a no-op; synchronises the device first */

/* Shrink row lengths (lens_host[b] <= current length; 0 empties a row).  Keys past the new
 * length are ignored from then on: truncation equals a shorter prefill (causality).
 * Synchronous with respect to the device. */
nc_status nc_kv_set_lens(nc_kv* kv, const int32_t* lens_host);
/* Current row lengths as the host sees them once enqueued work completes. */
nc_status nc_kv_get_lens(const nc_kv* kv, int32_t* lens_host);

/* Copy layer `layer` of the cache out in plain layout: k_dev and v_dev are
 * [batch][n_kv_head][max_seq][hd] of cfg.dtype (positions past each length hold stale
 * values). */
nc_status nc_kv_export(nc_kv* kv, int32_t layer, void* k_dev, void* v_dev, void* stream);

/* Copy cache rows: for i < n, row dst_rows_host[i] of dst takes the keys and values (every
 * layer) and the length of row src_rows_host[i] of src, as src holds them once its
 * enqueued work completes.  This is the batch generation of the pages' inference engine
 * (apidog.com/th guide, part 6: the KV cache cloned for parallel sampling): a prompt is
 * prefilled once and its row copied to the rows that then sample independently.  src and
 * dst belong to the same model and may be the same object; destination rows must be
 * distinct and, within one cache, disjoint from the source rows (NC_ERR_INVALID_ARG); a
 * source length above dst's max_seq gives NC_ERR_CAPACITY.  n == 0 is a no-op.  Enqueued
 * on `stream` (both caches are then in use on that stream). */
nc_status nc_kv_copy_rows(nc_kv* dst, const int32_t* dst_rows_host, nc_kv* src,
                          const int32_t* src_rows_host, int32_t n, void* stream);

/* Prefill, the engine's first inference stage (szyisi.cn launch article, base-model
 * evaluation section: prefill then decode over a KV cache; apidog.com/th guide, part 5: the
 * causal attention call over a whole sequence, part 6: the prompt's cache filled once).
 * Computes the forward pass above for T tokens per row in one batched pass and stores
 * their keys and values.
 * tokens_dev int32 [B, T]; row b's tokens go to positions lens[b] .. lens[b]+T-1
 * and attend to the row's cached positions as well (0..lens[b]-1): on an empty cache this
 * is the prompt prefill, on a filled one it appends a chunk (a long prompt in pieces, or
 * forced tokens in the middle of a generation), with the same results as a single prefill
 * of the whole sequence or as T decode steps.  Requires B == batch of kv, T >= 1
 * (NC_ERR_INVALID_ARG) and lens[b] + T <= max_seq for every row (NC_ERR_CAPACITY).
 * logits_dev: fp32 [B, T, vocab] for every new position, or NULL to fill the cache only.
 * On success every length grows by T.
 * Token ids outside [0, vocab) are clamped (memory-safe; their outputs are meaningless). */
nc_status nc_prefill(nc_model* m, const int32_t* tokens_dev, int32_t B, int32_t T,
                     nc_kv* kv, float* logits_dev, void* stream);

/* One decode step, the engine's second inference stage (szyisi.cn launch article,
 * base-model evaluation section; apidog.com/th guide, part 6: one new token per row whose
 * query attends to the cached keys and values, flash_attn_with_kvcache).  Computes the
 * forward pass above for one token per row and appends its key and value to the cache.
 * Row b takes token tokens_dev[b] at position lens[b] and attends to
 * cache positions 0..lens[b].  Requires B == batch of kv, B <= 128 (NC_ERR_UNSUPPORTED
 * otherwise) and lens[b] + 1 <= max_seq for every row (NC_ERR_CAPACITY otherwise).
 * logits_dev: fp32 [B, vocab] (not NULL).  On success every length grows by one.
 * The step's kernels are captured once per (tokens_dev, logits_dev) pair into a HIP graph
 * owned by the kv object and replayed on later calls (set NC_DECODE_GRAPH=0 in the
 * environment before nc_kv_create to launch them one by one instead). */
nc_status nc_decode_step(nc_model* m, const int32_t* tokens_dev, int32_t B, nc_kv* kv,
                         float* logits_dev, void* stream);

/* Allocation-free decode step, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same step as
 * nc_decode_step, with the same arguments, requirements, results (bitwise) and errors, but
 * its workspace (residual stream, activations, raw QKV product, attention partial states
 * and ready flags, split-K partial sums and arrival counters, the QKV finish's per-head
 * arrival counters) lives in a file-scope device
 * array of NC_STATIC_SCRATCH_BYTES that every GPU the library runs on holds until the
 * process ends, not in memory of the kv object; kernels are launched one by one (no graph
 * is captured).  The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine) and clears the array's flags and counters with a kernel before the step.
 * Errors beyond nc_decode_step's: NC_ERR_CAPACITY when the step's workspace for this
 * (model, kv) exceeds the array (the message gives the bytes needed); NC_ERR_UNSUPPORTED
 * for a model with the later version's blocks (nc_model_set_extras).  Every call on a GPU
 * uses the same array, which keeps the last call's contents: calls that overlap on one GPU
 * (other streams or threads) race and give wrong results. */
#define NC_STATIC_SCRATCH_BYTES 67108864 /* 64 MiB */
nc_status nc_decode_step_static(nc_model* m, const int32_t* tokens_dev, int32_t B, nc_kv* kv,
                                float* logits_dev, void* stream);

/* Greedy decode step, the engine's generation loop with argmax picks (apidog.com/th guide,
 * part 6): nc_decode_step followed by nc_argmax of its logits into next_dev (int32 [B]),
 * both in one captured graph: one call per generated token.  next_dev may be
 * tokens_dev itself (the step reads its tokens before it writes the picks).  Same
 * requirements and errors as nc_decode_step; next_dev must not be NULL.  The graph is
 * keyed by (tokens_dev, logits_dev, next_dev). */
nc_status nc_decode_greedy(nc_model* m, const int32_t* tokens_dev, int32_t B, nc_kv* kv,
                           float* logits_dev, int32_t* next_dev, void* stream);

/* Greedy pick, the deterministic choice of the engine's generation loop (the pages show
 * base-model completions of prompts, szyisi.cn launch article, base-model evaluation
 * section, and give no sampling formula for them; the greedy reading takes the most
 * likely token): out_dev[b] = argmax_v logits_dev[b, v] over fp32 [B, V] (row-major,
 * caller-owned device memory; out_dev int32 [B]); ties go to the lowest index; NaN compares
 * below every number.  NC_ERR_INVALID_ARG for NULL pointers or B, V < 1. */
nc_status nc_argmax(const float* logits_dev, int32_t B, int32_t V, int32_t* out_dev,
                    void* stream);

/* Sampled pick, the engine's parallel sampling (apidog.com/th guide, part 6; the pages give
 * no formula, so this is the plain temperature / top-k reading): over the logits of row b
 * at or above its top_k-th largest value (every logit when top_k <= 0 or top_k >= V; ties
 * with that value are all kept), probabilities proportional to exp(logit / temperature);
 * out_dev[b] = the smallest token index whose cumulative probability, in token order,
 * exceeds u_dev[b].  u_dev: fp32 [B] uniform numbers in [0, 1) drawn by the caller (values
 * outside are clamped into it), so a draw is reproducible.  NaN logits have probability 0;
 * logits must not be +inf.  temperature <= 0 (or NaN) is the greedy pick of nc_argmax and
 * u_dev may then be NULL.  fp32 arithmetic: where u_dev[b] lies within about 1e-5 of a
 * boundary of the cumulative distribution, the neighbouring token may be returned. */
nc_status nc_sample(const float* logits_dev, int32_t B, int32_t V, float temperature,
                    int32_t top_k, const float* u_dev, int32_t* out_dev, void* stream);

/* Kernel timing, for diagnostics and roofline reports.  When a kernel class is enabled,
 * every kernel of that class is launched with a pair of HIP events that the dispatch itself
 * stamps with the kernel's start and end (hipExtLaunchKernel), on the launch stream; decode
 * steps then launch their kernels one by one instead of replaying their captured graphs
 * (which stay cached for when timing is switched off).  nc_timing_read synchronises the
 * device and adds the operations recorded since the last read to running totals: their
 * number, their summed kernel time, and their algorithmic bytes and flops.
 * nc_timing_enable resets the totals.  Process-wide, not thread-safe.  Returns
 * NC_ERR_INVALID_ARG for an unknown class. */
#define NC_KC_NONE 0
#define NC_KC_DECODE_GEMM 1  /* decode projections: QKV (with its finish), O, FC, PROJ, LM head */
#define NC_KC_PREFILL_GEMM 2 /* prefill projections                                       */
#define NC_KC_PREFILL_ATTN 3 /* prefill attention                                         */
#define NC_KC_DECODE_ATTN 4  /* decode attention                                          */
typedef struct nc_timing {
    int64_t launches; /* timed operations (one decode attention = its two kernels)       */
    double ms;    /* summed kernel time of the launches (start/stop of each kernel)        */
    double bytes; /* algorithmic bytes: weights, activations and outputs, each moved once */
    double flops; /* algorithmic flops: 2 M N K per product, 4 hd per visible score pair  */
                  /* (decode attention bytes: K and V rows 0..lens_b of every row, once)  */
} nc_timing;
nc_status nc_timing_enable(int32_t kernel_class);
nc_status nc_timing_read(nc_timing* out);

/* Diagnostics (measurement context, not part of the forward): what the current GPU
 * sustains with plain kernels, synchronous, about a second each.
 * nc_diag_mfma_rate: dense bf16 32x32x16 MFMA throughput in TFLOP/s, with operands that
 *   keep toggling (random_operands != 0) or stay fixed; the matrix cores' power draw, and
 *   so the clock they hold, depends on the data.
 * nc_diag_hbm_read_rate: a 1 GiB device-memory read stream in TB/s.
 * NC_ERR_INVALID_ARG for a NULL output, NC_ERR_DEVICE on a HIP error. */
nc_status nc_diag_mfma_rate(int32_t random_operands, double* tflops_out);
nc_status nc_diag_hbm_read_rate(double* tbps_out);

/* Message of the last error on the calling thread ("" if none). */
const char* nc_last_error(void);
int32_t nc_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NC_H */
