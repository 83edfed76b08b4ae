/*
 * dec.h — C ABI of the MI355X (gfx950) decoder-only transformer forward.
 *
 * The library runs the forward of a Llama-family decoder (RMSNorm, q/k/v
 * projections with optional biases, adjacent-pair RoPE, a K/V cache write,
 * causal grouped-query attention, output projection and residual, RMSNorm,
 * SwiGLU FFN or top-k MoE FFN, final norm, LM head) as single-pass prefill and
 * as batched one-token decode, entirely in HIP kernels on one GPU.
 *
 * Memory: the library allocates NO device memory.  Weights are borrowed
 * device pointers (they must outlive the handle); the workspace (KV cache and
 * activations) is one caller-allocated device buffer of dec_workspace_bytes().
 * All work is enqueued on the caller's HIP stream given at dec_create; calls
 * return before the GPU finishes.  One host thread per handle.
 *
 * Errors: every function returns DEC_OK (0) or a negative status.  All argument
 * checks run on the host before anything is enqueued, and on error nothing has
 * changed: no KV length or content, no output.  (rml "The decoder", section
 * "One forward pass", step 1: invalid input and a full cache are reported
 * before any state changes; Pantheon "Llama Forward Pass", section "Batched
 * Multi-Sequence Decode": an unsupported batch returns without mutating state.)
 * A device fault is reported as DEC_ERR_DEVICE by the next call that synchronises.
 *
 * Structs have one fixed layout in every build; no field depends on a build
 * flag (Pantheon "Llama Forward Pass", section "ABI note").
 */
#ifndef DEC_H
#define DEC_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define DEC_API __attribute__((visibility("default")))
#else
#define DEC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DEC_OK = 0,
    DEC_ERR_INVALID = -1,      /* bad argument, bad config, wrong struct_size, null pointer */
    DEC_ERR_RANGE = -2,        /* the request does not fit the KV capacity or max sizes */
    DEC_ERR_NOMEM = -3,        /* workspace smaller than dec_workspace_bytes() */
    DEC_ERR_DEVICE = -4,       /* a HIP call or kernel failed */
    DEC_ERR_UNSUPPORTED = -5   /* a shape the library's kernels do not handle */
};

enum { DEC_WEIGHT_BF16 = 0, DEC_WEIGHT_F32 = 1 };
enum { DEC_ROPE_ADJACENT = 0, DEC_ROPE_HALF = 1 };
enum { DEC_ROPE_PLAIN = 0, DEC_ROPE_LLAMA3 = 1 };
enum { DEC_KV_F32 = 0, DEC_KV_BF16 = 1, DEC_KV_F24 = 2 };
enum { DEC_PREFILL_BF16_PAIR = 0, DEC_PREFILL_F16_F8 = 1 };

/*
 * Model configuration: the base recipe plus switches (rml "The decoder",
 * section "The model config").  Validation at dec_create follows that page's
 * ValidateConfig: sizes > 0, n_heads % n_kv_heads == 0, head_dim even,
 * rms_eps > 0, rope_theta > 0, 1 <= top_k <= n_experts when n_experts > 0.
 * head_dim is explicit, never derived from hidden / n_heads (sipllm
 * "Transformer forward pass", section "Tradeoffs").
 *
 * sliding_window > 0 makes the KV cache a ring of max_seq slots, written at
 * pos % max_seq, with min(pos+1, max_seq) positions readable, max_seq <=
 * sliding_window (Pantheon, section "Sliding Window (Mistral)").  With
 * sliding_window == 0 a sequence holds at most max_seq positions.
 */
typedef struct dec_config {
    uint32_t struct_size;      /* sizeof(dec_config) */
    int32_t n_layers;
    int32_t hidden;            /* d */
    int32_t n_heads;           /* query heads */
    int32_t n_kv_heads;        /* key/value heads; query head h reads kv head h*n_kv/n_heads */
    int32_t head_dim;
    int32_t ffn_dim;           /* SwiGLU inner size (per expert for MoE) */
    int32_t vocab;
    int32_t n_experts;         /* 0 = dense FFN */
    int32_t top_k;             /* experts per token (MoE) */
    int32_t qkv_bias;          /* 1 = q/k/v projections add fp32 biases */
    int32_t tied_embedding;    /* 1 = LM head is the embedding matrix */
    int32_t sliding_window;    /* 0 = full causal range */
    int32_t max_seq;           /* KV positions per sequence slot */
    int32_t max_batch;         /* sequence slots == largest decode batch (<= 64) */
    int32_t max_prefill;       /* largest n of one dec_prefill call */
    int32_t weight_dtype;      /* DEC_WEIGHT_BF16 or DEC_WEIGHT_F32 */
    double rms_eps;
    double rope_theta;
    /* RoPE variants (rml "The decoder", section "Rotary embeddings"):
       rope_pairing DEC_ROPE_ADJACENT rotates elements (2i, 2i+1) of a head,
       DEC_ROPE_HALF rotates (i, i + head_dim/2); rope_scaling DEC_ROPE_LLAMA3
       applies llama3 frequency scaling: pairs whose wavelength 2*pi/f is under
       orig_ctx/high_freq_factor keep f, those over orig_ctx/low_freq_factor use
       f/factor, and between them s = (orig_ctx/wavelength - low)/(high - low)
       gives (1 - s) f/factor + s f. */
    int32_t rope_pairing;
    int32_t rope_scaling;
    int32_t rope_orig_ctx;
    /* Element type of the K/V cache (rml "The decoder", section "Attend": the
       cache has a choice of element type and attention widens each row to fp32
       as it reads it).  DEC_KV_F32: fp32.  DEC_KV_BF16: each rotated key and
       each value element is rounded to the nearest-even bf16 when stored,
       halving the cache's bytes and its bytes read per decode step; every
       later read (decode and prefill) sees the rounded value.  DEC_KV_F24:
       each element is rounded to nearest even at 16 significant bits (fp32's
       sign and exponent, 15 stored mantissa bits) and stored as 3 bytes: a
       cache row of head_dim elements is head_dim 16-bit words (the upper half
       of the rounded fp32 word) followed by head_dim bytes (the third bytes,
       by blocks of 8 elements: block b at byte 16 (b % L) + 8 (b / L) of that
       part, L = head_dim / 16).
       Three quarters of the fp32 cache's bytes; readers rebuild the fp32
       word exactly.  Arithmetic stays fp32. */
    int32_t kv_dtype;
    double rope_factor;
    double rope_low_freq_factor;
    double rope_high_freq_factor;
    /* Operands of the prefill projections (calls of more than 64 rows, bf16
       weights): an arithmetic choice of this library, not a step of the
       forward.  Both forms compute y = W a with a split a = hi + lo, so that
       the product keeps near-fp32 accuracy against the exact weights.
       DEC_PREFILL_BF16_PAIR: hi = bf16(a), lo = bf16(a - hi), two bf16 MFMA
       passes against the caller's weights.
       DEC_PREFILL_F16_F8: hi = fp16(a) against an fp16 copy of the weights,
       plus lo = a - hi as fp8 e4m3 with a power-of-two scale per 32 inputs
       against an fp8 copy of the weights (same scaling) on the fp8 MFMA, which
       runs at twice the bf16 rate.  It covers the q|k|v projection and, for a
       dense FFN whose fused gate|up grid fills the device, gate|up; the other
       projections and MoE experts keep the pair, and so does a config whose
       max_prefill is 64 or less.  The converted weights live in the
       workspace (dec_workspace_bytes grows by about 3 bytes per q|k|v and
       gate|up weight) and are written by dec_create on its stream from the
       caller's weights, which must hold their values by then.  |a| above 65504 (the
       fp16 maximum) keeps only fp8 accuracy for that element.  */
    int32_t prefill_operands;
} dec_config;

/*
 * Weights of one layer: device pointers, row-major [out][in], each 16-byte
 * aligned (the kernels read them in 16-byte words; dec_create returns
 * DEC_ERR_INVALID otherwise).  Matrices are bf16 (or fp32 when weight_dtype ==
 * DEC_WEIGHT_F32); norm gains and biases are always fp32.  Dense:  w_gate, w_up [ffn][d], w_down [d][ffn].
 * MoE: router [E][d]; w_gate, w_up [E][ffn][d]; w_down [E][d][ffn], expert e
 * being the e-th slice (Pantheon, section "Mixture of Experts (Mixtral)",
 * merged expert tensors).  bq/bk/bv only with qkv_bias; router only with MoE.
 */
typedef struct dec_layer_weights {
    const float *attn_norm;    /* [d] */
    const void *wq;            /* [n_heads*head_dim][d] */
    const void *wk;            /* [n_kv_heads*head_dim][d] */
    const void *wv;            /* [n_kv_heads*head_dim][d] */
    const float *bq, *bk, *bv; /* [q_dim], [kv_dim], [kv_dim] */
    const void *wo;            /* [d][n_heads*head_dim] */
    const float *ffn_norm;     /* [d] */
    const void *w_gate;
    const void *w_up;
    const void *w_down;
    const void *router;
} dec_layer_weights;

typedef struct dec_weights {
    uint32_t struct_size;                  /* sizeof(dec_weights) */
    const void *embed;                     /* [vocab][d] */
    const float *out_norm;                 /* [d] */
    const void *lm_head;                   /* [vocab][d]; ignored when tied */
    const dec_layer_weights *layers;       /* host array of n_layers entries (copied) */
} dec_weights;

typedef struct dec_model *dec_handle;

/* Device bytes the workspace must hold for this config; 0 if cfg is invalid.
   Pure host function. */
DEC_API size_t dec_workspace_bytes(const dec_config *cfg);

/* Validate cfg and weights and bind them to a handle.  workspace: device
   buffer of at least dec_workspace_bytes(cfg) bytes, 256-byte aligned, owned by
   the caller.  hip_stream: a hipStream_t (NULL = the null stream).  All KV
   slots start empty. */
DEC_API int dec_create(const dec_config *cfg, const dec_weights *w, void *workspace, size_t ws_bytes,
               void *hip_stream, dec_handle *out);

/*
 * dec_create for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, checks and handle as dec_create, but the workspace is the
 * library's own file-scope device array of DEC_NOALLOC_WORKSPACE_BYTES (64 MiB;
 * one copy per GPU, held until the process ends) instead of a caller buffer.
 * Nothing is allocated on the device.  The handle's stream must belong to the
 * current device (DEC_ERR_INVALID otherwise).
 *   DEC_ERR_NOMEM:   dec_workspace_bytes(cfg) exceeds DEC_NOALLOC_WORKSPACE_BYTES
 *                    (the tiny shapes fit, a SmolLM2-135M shape with up to 4
 *                    slots of 256 positions and 128-token prefills fits).
 *   DEC_ERR_INVALID: also when another handle made by this call is still alive
 *                    on the same device: the array holds one handle's KV cache
 *                    and activations, and two would overwrite each other.
 * The array keeps whatever the last handle left in it; nothing in the library
 * reads workspace memory before writing it (KV slots are read only below their
 * committed length), so nothing needs clearing.  Calls that overlap on one
 * GPU's array race.  dec_destroy frees the device's array for the next handle.
 */
#define DEC_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
DEC_API int dec_create_noalloc(const dec_config *cfg, const dec_weights *w, void *hip_stream, dec_handle *out);

DEC_API void dec_destroy(dec_handle h);

/*
 * Single-pass prefill of n tokens into sequence slot `seq` (sipllm
 * "Transformer forward pass", section "Single-pass prefill"): every layer
 * processes all n positions once, positions ascending, and only the last
 * position's logits are produced.  start_pos must equal the slot's committed
 * length: 0 starts a sequence, > 0 appends to it (zLLM "The Algorithm Layer",
 * section 5: NewPrefill / AppendPrefill).
 *   tokens: host int32[n], each in [0, vocab).   1 <= n <= max_prefill.
 *   logits: device float[vocab], the last position's logits.
 * Without a window, start_pos + n <= max_seq (else DEC_ERR_RANGE).  With a
 * window, a call whose positions would overwrite slots still needed by its own
 * earlier positions (start_pos + n > max_seq) runs position by position.
 * On success the slot's length becomes start_pos + n.
 */
DEC_API int dec_prefill(dec_handle h, int seq, const int32_t *tokens, int n, int start_pos, float *logits);

/*
 * dec_prefill with a choice of which rows get logits (rml "The decoder",
 * section "One forward pass", step 7: only the rows that need logits get the
 * final norm and the output product, the last row or, with all_logits, every
 * row).  all_logits = 0: as dec_prefill.  all_logits = 1: logits is device
 * float[n][vocab], row t the logits after position start_pos + t.  Any other
 * value is DEC_ERR_INVALID.  Errors and state changes as dec_prefill.
 */
DEC_API int dec_prefill_ex(dec_handle h, int seq, const int32_t *tokens, int n, int start_pos, float *logits,
                           int all_logits);

/*
 * One decode step of B independent sequences (Pantheon, section "Batched
 * Multi-Sequence Decode"): row b uses slot b, reads token tokens[b] at
 * position pos[b] == slot b's committed length, and writes logits row b.
 *   tokens, pos: host int32[B].   1 <= B <= max_batch.
 *   logits: device float[B][vocab] row-major.
 * On success each slot b < B has length pos[b] + 1.
 */
DEC_API int dec_decode(dec_handle h, int B, const int32_t *tokens, const int32_t *pos, float *logits);

/*
 * `steps` greedy decode steps of B sequences with the tokens kept on the GPU
 * (Pantheon, section "Optional GPU Paths": a GPU-resident decode runs the whole
 * layer chain on the device with one synchronisation per step; here there is
 * none inside the loop).  Step 0 reads tokens[b] (host int32[B]) for row b at
 * position slot b's committed length; every later step reads the greedy
 * choice of the step before it (largest logit, lowest id on ties, as
 * dec_greedy), chosen on the device.  Each step is one captured graph replay.
 *   tokens_out: device int32[steps][B]: row s holds the choices made from
 *               step s's logits (the input of step s + 1).
 *   logits:     device float[B][vocab], scratch for every step; it holds the
 *               last step's logits when the call's work completes.
 * Capacity is checked for all steps before anything is enqueued (a full
 * cache is DEC_ERR_RANGE, bad ids or sizes DEC_ERR_INVALID; nothing changes).
 * On success each slot b < B has length += steps.  Asynchronous on the
 * handle's stream.
 */
DEC_API int dec_decode_greedy(dec_handle h, int B, const int32_t *tokens, int steps, int32_t *tokens_out,
                              float *logits);

/* Set slot `seq`'s committed length to 0 (seq = -1: every slot).  No memory is
   cleared: only min(pos+1, max_seq) positions are ever read. */
DEC_API int dec_kv_reset(dec_handle h, int seq);

/* Committed length of slot `seq`, or a negative status. */
DEC_API int dec_kv_length(dec_handle h, int seq);

/* Greedy choice for B rows of device logits [B][vocab]: the largest logit, the
   lowest token id on ties.  Writes host int32[B]; synchronises the stream. */
DEC_API int dec_greedy(dec_handle h, const float *logits, int B, int32_t *tokens_out);

/* Wait for the handle's stream; DEC_ERR_DEVICE if any enqueued work failed. */
DEC_API int dec_sync(dec_handle h);

/*
 * Test capture.  Non-null device pointers make every following call write
 *   hidden:      the residual stream after the embedding and after each layer,
 *                float[(n_layers+1)][rows][d];
 *   expert_ids:  the chosen experts, int32[n_layers][rows][top_k] (MoE only);
 *   router:      the router logits, float[n_layers][rows][n_experts] (MoE only);
 * with rows = n (prefill) or B (decode).  NULL turns a capture off.  The
 * buffers must hold the largest call made while capture is on.
 */
DEC_API int dec_set_capture(dec_handle h, float *hidden, int32_t *expert_ids, float *router);

/* Kernel classes for dec_timing_*. */
enum {
    DEC_K_GEMV = 0,            /* decode projections (weights streamed once per step) */
    DEC_K_ATTN_DECODE = 1,     /* split-KV decode attention (+ its merge) */
    DEC_K_GEMM = 2,            /* prefill projections (MFMA) */
    DEC_K_ATTN_PREFILL = 3,    /* causal prefill attention */
    DEC_K_COUNT = 4
};

/* Live per-kernel timing with HIP events on the handle's stream: while enabled,
   every launch of the class is bracketed by an event pair.  dec_timing_read
   synchronises, returns the summed duration (ms) and launch count since the
   last enable, and the algorithmic bytes and flops of those launches. */
DEC_API int dec_timing_enable(dec_handle h, int kernel_class, int on);
DEC_API int dec_timing_read(dec_handle h, int kernel_class, double *total_ms, int64_t *launches,
                    double *bytes, double *flops);

/* Number of captured decode-step graphs the handle holds.  A decode call runs
   its first call of a given shape (batch, attention split count, logits buffer)
   eagerly and captures the second; later calls of that shape replay the graph
   on an internal stream ordered after, and before, the caller's stream.
   Results are identical either way.  A handle keeps at most 16 graphs: a new
   capture beyond that drops the least recently replayed one.  A shape whose
   capture fails stays eager.  While a test capture or per-kernel timing is on,
   decode runs eagerly. */
DEC_API int dec_graph_count(dec_handle h);

/* Text of a status code. */
DEC_API const char *dec_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* DEC_H */
