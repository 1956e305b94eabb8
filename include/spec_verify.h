/*
 * spec_verify.h -- C ABI of the speculative-decoding verification step on
 * AMD Instinct MI355X (gfx950).
 *
 * The step (one target iteration of speculative decoding):
 *   1. one forward of the target over all B*(K+1) drafted positions, reading
 *      the target weights once for all of them (onlylabs/Cohere "Hardware
 *      Aware Dynamic Speculative Decoding", section "Hardware-aware dynamic
 *      SD": the target processes BS x (K+1) tokens; publishertech "Speculative
 *      Decoding in Large Language Models", section 1 "The Speculative Cycle");
 *   2. modified rejection sampling per request: accept draft token x with
 *      probability min(1, p(x)/q(x)); at the first rejection discard it and all
 *      later drafts and emit one token from max(0, p - q) normalised; if all K
 *      drafts are accepted emit a bonus token from the next target
 *      distribution (publishertech section 2 "Modified Rejection Sampling";
 *      mohashari "Speculative Decoding in Production", section "Speculative
 *      Decoding Mechanics"; NVIDIA co-design post, section "What is
 *      speculative decoding?": the acceptance length AL lies in [1, 1 + K]).
 *
 * The synthetic target: n_layers pre-norm residual MLP blocks
 *     a = bf16(rmsnorm(h) * g_l);  s = bf16(silu(a W_up_l^T));  h += s W_down_l^T
 * then a_f = bf16(rmsnorm(h) * g_L) and logits = a_f W_head^T (fp32).  With
 * fp32 weights nothing is rounded to bf16.  rmsnorm(h) = h / sqrt(mean(h^2)
 * + eps).  Accumulation is fp32.
 *
 * Layout: every matrix is row-major; weights are [out, in].  Row r = b*(K+1)+j
 * of the hidden states and of the target logits belongs to request b, position
 * j (0 <= j <= K); row j scores draft token j, row K is the bonus row.
 *
 * Memory and streams: every pointer argument is a DEVICE pointer unless its
 * comment says "host".  The caller owns all memory (weights, inputs, outputs
 * and workspace).  The library never allocates or frees device memory, never
 * synchronises, and never reads device data on the host, so a whole call can
 * be captured into a HIP graph.  Work is enqueued on `stream` (a hipStream_t
 * passed as void*; NULL means the default stream) and completes
 * asynchronously; results are valid once the caller synchronises the stream.
 *
 * Errors: every function that can fail returns an int: 0 (SV_OK) or a
 * negative sv_status.  All argument checks run on the host before anything is
 * enqueued, so on an error nothing has been launched; spec_verify_last_error()
 * then returns a message for the calling thread.  A failed launch returns
 * SV_ERR_HIP.  Device faults surface at the caller's next synchronisation.
 * No C++ exception crosses this interface.
 *
 * Thread safety: an sv_model is immutable after creation; concurrent calls on
 * different streams are safe if each uses its own workspace and outputs.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 1

typedef enum {
    SV_OK = 0,
    SV_ERR_INVALID_ARG = -1,   /* null pointer, bad size, bad temperature     */
    SV_ERR_UNSUPPORTED = -2,   /* shape or dtype this build does not handle   */
    SV_ERR_WORKSPACE = -3,     /* workspace pointer missing or too small      */
    SV_ERR_HIP = -4            /* a HIP launch or runtime call failed         */
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Storage order of the weight matrices.
 *   SV_LAYOUT_ROW_MAJOR  [out, in] row-major.
 *   SV_LAYOUT_TILED      bf16 only: each [rows, cols] matrix as produced by
 *                        spec_verify_pack_weights -- 16 x 32 blocks of 1 KiB,
 *                        each stored in the lane order of the gfx950 matrix-core
 *                        operand, rows padded with zeros to a multiple of 16.
 *                        Block (rt, s), rt < ceil(rows/16), s < cols/32, starts
 *                        at element (rt * cols/32 + s) * 512, and its element
 *                        l*8 + e (lane l = r + 16 q, r < 16, q < 4, e < 8) is
 *                        W[rt*16 + r][s*32 + 8q + e].  Streaming the weights
 *                        then reads one contiguous KiB per wave load. */
typedef enum { SV_LAYOUT_ROW_MAJOR = 0, SV_LAYOUT_TILED = 1 } sv_layout;

/* Target model description (host struct; the weight pointers are device
 * pointers that the model only borrows: keep them alive and unchanged until
 * sv_model_destroy).  d and ffn must be positive multiples of 64, d <= 32768;
 * vocab >= 1; n_layers >= 0.  Weight pointers must be 16-byte aligned.  With
 * SV_LAYOUT_TILED the three matrices are in the tiled layout (w_up: n_layers
 * consecutive tiled [ffn, d] matrices; w_down: tiled [d, ffn]; w_head: tiled
 * [vocab, d], spec_verify_packed_elems(vocab, d) elements). */
typedef struct {
    int32_t d;            /* model width                                      */
    int32_t ffn;          /* MLP width                                        */
    int32_t n_layers;     /* number of MLP blocks                             */
    int32_t vocab;        /* V                                                */
    int32_t wdtype;       /* sv_dtype of w_up, w_down, w_head                 */
    int32_t layout;       /* sv_layout of w_up, w_down, w_head                */
    float rms_eps;        /* RMSNorm epsilon (>= 0)                           */
    const void* w_up;     /* [n_layers, ffn, d]                               */
    const void* w_down;   /* [n_layers, d, ffn]                               */
    const float* gain;    /* [n_layers + 1, d] fp32; last row = final norm    */
    const void* w_head;   /* [vocab, d]                                       */
} sv_model_desc;

/* Elements of the tiled copy of one bf16 [rows, cols] matrix
 * (ceil(rows/16) * 16 * cols); 0 if rows < 1 or cols is not a positive
 * multiple of 32. */
size_t spec_verify_packed_elems(int32_t rows, int32_t cols);

/* Packs `count` consecutive row-major bf16 [rows, cols] matrices at `src` into
 * the tiled layout at `dst` (count * spec_verify_packed_elems(rows, cols)
 * elements, caller-owned, must not overlap src).  Device pointers, 16-byte
 * aligned; cols a positive multiple of 32.  A one-time preparation step done
 * when the weights are loaded, not part of the verification step. */
int spec_verify_pack_weights(const void* src, void* dst, int32_t rows, int32_t cols,
                             int32_t count, void* stream);

typedef struct sv_model sv_model;

/* Version of this interface (SV_ABI_VERSION of the built library). */
int32_t spec_verify_abi_version(void);

/* Validates `desc` (host only; touches no device memory) and creates a model
 * handle in *out (host pointer).  Returns SV_ERR_INVALID_ARG / UNSUPPORTED. */
int sv_model_create(const sv_model_desc* desc, sv_model** out);
void sv_model_destroy(sv_model* m);

/* Workspace bytes needed by spec_verify_forward for M rows, by
 * spec_verify_accept for (B, K, V), and by spec_verify_step for (B, K)
 * (= forward(B*(K+1)) + accept(B, K, vocab)).  Return 0 for invalid
 * arguments. */
size_t spec_verify_forward_workspace_bytes(const sv_model* m, int32_t M);
size_t spec_verify_accept_workspace_bytes(int32_t B, int32_t K, int32_t V);
size_t spec_verify_workspace_bytes(const sv_model* m, int32_t B, int32_t K);

/* Target forward over M rows (the verification forward, step 1 above).
 *   hidden  [M, d] fp32 input hidden states (read only)
 *   logits  [M, vocab] fp32 output
 *   ws      workspace of ws_bytes >= spec_verify_forward_workspace_bytes(m, M),
 *           256-byte aligned; contents on entry are ignored.
 * M == 0 is a no-op.  Returns SV_OK or an error as above. */
int spec_verify_forward(const sv_model* m, const float* hidden, int32_t M, float* logits,
                        void* ws, size_t ws_bytes, void* stream);

/* Modified rejection sampling for B requests with K drafts each (step 2).
 *   target_logits [B, K+1, V] fp32; draft_logits [B, K, V] fp32 (may be NULL
 *   when temperature == 0 or K == 0); draft_tokens [B, K] int32 (may be NULL
 *   when K == 0).
 *   temperature  T > 0: p = softmax(z_target / T), q = softmax(z_draft / T).
 *                T == 0: greedy -- accept while the draft equals the target's
 *                argmax (lowest id on ties), then emit the target's argmax.
 *                T must be finite and either 0 or >= FLT_MIN.
 *   seed, step   key and last counter word of the Philox4x32-10 stream; the
 *                uniform for the accept test of draft position j (1-based) of
 *                request b is U_acc = ((w >> 8) + 1) / 2^24 with w = word 0 of
 *                Philox((b, j, 0, step), seed); the uniform of the replacement
 *                or bonus token emitted at position j is U_res = (w >> 8) / 2^24
 *                with w from counter (b, j, 1, step).  Accept iff U_acc <= p/q;
 *                the emitted token is the smallest id y whose running sum of
 *                weights exceeds U_res times their total.
 *   out_tokens   [B, K+1] int32: emitted tokens, -1 after the first AL slots.
 *   accept_len   [B] int32: AL in [1, K+1] (tokens emitted = accepted + 1);
 *                0 (with all out_tokens -1) if any draft token of the request
 *                lies outside [0, V).
 *   p_at_draft, q_at_draft  optional [B, K] fp32 outputs (NULL to skip):
 *                p_j(x_j) and q_j(x_j) for every draft (1 / 0 at T == 0).
 *   ws           >= spec_verify_accept_workspace_bytes(B, K, V) bytes, 256-byte
 *                aligned.
 * B == 0 is a no-op.  K >= 0 (K == 0: plain sampling from the one row). */
int spec_verify_accept(const float* target_logits, const float* draft_logits,
                       const int32_t* draft_tokens, int32_t B, int32_t K, int32_t V,
                       float temperature, uint64_t seed, uint32_t step,
                       int32_t* out_tokens, int32_t* accept_len,
                       float* p_at_draft, float* q_at_draft,
                       void* ws, size_t ws_bytes, void* stream);

/* spec_verify_accept for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results without the workspace.  Its
 * scratch is one static device array of SV_ACCEPT_STATIC_SCRATCH_BYTES per
 * GPU, held until the process ends.
 *   - Sizes with spec_verify_accept_workspace_bytes(B, K, V) above that
 *     limit return SV_ERR_WORKSPACE with nothing launched (4 MiB covers, for
 *     instance, B = 1024, K = 8 at V = 128256: 2.9 MB).
 *   - The first call on each device resolves the array's address
 *     (hipGetSymbolAddress, with that device current) and keeps it; later
 *     calls on that device reuse it.  The current device is the one used.
 *   - Every call on a GPU shares that GPU's array: calls that overlap on one
 *     GPU (two streams, or two threads) race, and the caller must order them.
 *     Nothing in the array needs to start at zero.
 *   - No device memory is allocated or freed; argument errors are reported as
 *     for spec_verify_accept. */
#define SV_ACCEPT_STATIC_SCRATCH_BYTES ((size_t)4 << 20)
int spec_verify_accept_noalloc(const float* target_logits, const float* draft_logits,
                               const int32_t* draft_tokens, int32_t B, int32_t K, int32_t V,
                               float temperature, uint64_t seed, uint32_t step,
                               int32_t* out_tokens, int32_t* accept_len,
                               float* p_at_draft, float* q_at_draft, void* stream);

/* The whole step: spec_verify_forward on hidden [B*(K+1), d] into
 * logits_out [B*(K+1), V], then spec_verify_accept on those logits with the
 * model's vocab.  ws >= spec_verify_workspace_bytes(m, B, K). */
int spec_verify_step(const sv_model* m, const float* hidden, const float* draft_logits,
                     const int32_t* draft_tokens, int32_t B, int32_t K, float temperature,
                     uint64_t seed, uint32_t step, float* logits_out,
                     int32_t* out_tokens, int32_t* accept_len,
                     float* p_at_draft, float* q_at_draft,
                     void* ws, size_t ws_bytes, void* stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* spec_verify_last_error(void);

/* ---- Per-kernel timing (tracing) -------------------------------------------
 * Between spec_verify_profile_begin() and spec_verify_profile_end(), every
 * kernel the library launches (from any thread) is bracketed by a pair of HIP
 * events on its stream; at most `max_launches` launches are recorded, later
 * ones run untimed.  profile_end synchronises on the recorded events and
 * fills `out` (host array of `cap` entries) with one entry per kernel name,
 * returning the number of entries in *n_out.  Events add a small gap between
 * launches, so time a workload without profiling for throughput.  These two
 * calls create and destroy HIP events (host-side objects) and are not meant
 * for graph capture. */
typedef struct {
    char name[64];        /* kernel name (the launch site's label)           */
    int32_t launches;     /* launches recorded                               */
    double total_ms;      /* summed event-to-event time                      */
    double bytes;         /* algorithmic bytes summed over those launches    */
    double flops;         /* algorithmic flops summed over those launches    */
} sv_kernel_time;

int spec_verify_profile_begin(int32_t max_launches);
int spec_verify_profile_end(sv_kernel_time* out, int32_t cap, int32_t* n_out);

/* Between profile_begin and profile_end: paused != 0 stops recording (later
 * launches run untimed and take no slot), 0 resumes it.  A launch with events
 * costs the host more than a short kernel takes to run, so a caller can queue
 * untimed work ahead of each timed step and keep the GPU from waiting on the
 * host inside the timed launches.  SV_ERR_INVALID_ARG when profiling is off. */
int spec_verify_profile_pause(int32_t paused);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
