/*
 * sscan.h -- C ABI of libsscan, the selective state-space scan for AMD MI355X (gfx950).
 *
 * The scan (sources by page title and section):
 *   "Mamba" (nnterp guide, architectures), opening paragraph and section
 *   "The values": per channel of the mixer's inner width, a state of state_dim
 *   numbers updated for each token as
 *       h = exp(dt * A) * h + dt * B * x,      y = C . h + D * x,
 *   with the step dt = softplus(dt_raw + dt_bias) per token and channel, A per
 *   channel and state dimension, B and C from one group shared by every channel,
 *   state_input None (zeros) on a prompt and state_output the state after the
 *   call's last token. "Mamba" (tokentrails lineage), section "Code":
 *   A = -exp(A_log), and the mixer's output is y * silu(z).
 *   "Falcon-Mamba" (nnterp encyclopedia), section "Where the norms sit":
 *   B and C pass a weightless RMS norm over state_dim before the scan.
 *   "Mamba-2" (nnterp encyclopedia), sections "The mixer's values" and
 *   "The block, in order": the same recurrence with one scalar decay per head
 *   and token (decays = softplus(dt + dt_bias) * A) and a state matrix per head;
 *   y = ssd(...) + D * x, then the gate.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer (hipMalloc / torch CUDA tensors)
 *     to a contiguous, row-major, tokens-first array. Host pointers are rejected
 *     with SSCAN_ERR_NOT_DEVICE (the pages' prior-art kernels also refuse CPU
 *     tensors).
 *   - Every tensor pointer must be 16-byte aligned (SSCAN_ERR_ALIGN).
 *   - "act" tensors (x, dt_raw, z, B, C, y) are float32 or bfloat16 as the
 *     descriptor says; dt_bias, A_log, D and every state are float32.
 *   - The caller owns every buffer, including the workspace (size it with the
 *     *_workspace_size query). The library allocates nothing and never
 *     synchronizes: work is queued on `stream` (a hipStream_t; NULL is the null
 *     stream) and the call returns at once.
 *   - Validation happens before anything is launched. A nonzero status means
 *     nothing was launched (except SSCAN_ERR_HIP, which reports a failed
 *     launch). Faults inside a kernel surface at the caller's next sync.
 *   - Outputs must not overlap inputs (SSCAN_ERR_ALIAS), except that
 *     sscan_step and sscan_ssd_step may update the state in place
 *     (state_output == state_input).
 *   - Thread-safe: the only global state is a thread-local error string and the
 *     process-wide switches of sscan_set_pointer_checks and sscan_set_tuning
 *     (atomics).
 */
#ifndef SSCAN_H
#define SSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSCAN_ABI_VERSION 3

typedef enum { SSCAN_F32 = 0, SSCAN_BF16 = 1 } sscan_dtype;

typedef enum {
  SSCAN_OK = 0,
  SSCAN_ERR_NULL = 1,        /* a required pointer (or the descriptor) is NULL      */
  SSCAN_ERR_SHAPE = 2,       /* a size is negative/zero where it must be positive, or inconsistent */
  SSCAN_ERR_DTYPE = 3,       /* act is not SSCAN_F32 / SSCAN_BF16                   */
  SSCAN_ERR_UNSUPPORTED = 4, /* valid, but not a variant this build implements      */
  SSCAN_ERR_NOT_DEVICE = 5,  /* a tensor pointer is not device memory               */
  SSCAN_ERR_ALIGN = 6,       /* a tensor pointer is not 16-byte aligned             */
  SSCAN_ERR_ALIAS = 7,       /* an output overlaps an input                         */
  SSCAN_ERR_WORKSPACE = 8,   /* workspace NULL or smaller than the query returned   */
  SSCAN_ERR_HIP = 9          /* the HIP runtime reported an error                   */
} sscan_status;

/* Mamba-1 problem. channels is the mixer's inner width (d_inner). ngroups must
 * divide channels; channel c reads group c / (channels / ngroups). When
 * ngroups > 1, channels / ngroups must be a multiple of 64. state_dim in 1..256:
 * 16, 32 or 64 with channels a multiple of 4 take the prompt kernel with a
 * 16-lane row per channel; other state_dim up to 64 the one with 1, 2 or 4 lanes
 * per channel; 65..256 the token loop with 16 lanes per channel.
 * bc_rms_eps > 0 applies the weightless RMS norm b / sqrt(mean(b^2) + eps) to
 * every [state_dim] vector of B and of C before the scan ("Falcon-Mamba",
 * section "Where the norms sit"); <= 0 reads B and C as given. */
typedef struct sscan_mamba1_desc {
  int64_t batch, seqlen, channels, state_dim, ngroups;
  int32_t act;        /* sscan_dtype of x, dt_raw, z, B, C and y */
  float bc_rms_eps;
} sscan_mamba1_desc;

/* Mamba-2 (SSD) problem. nheads heads of head_dim channels each, a
 * [head_dim, state_dim] state per head; head h reads group h / (nheads / ngroups).
 * chunk is the interval at which a chunked scan keeps boundary states ("Mamba-2",
 * section "The state": 256 on the pages' kernel). It does not change the result
 * beyond rounding; 0 lets the library choose, otherwise a power of two in 16..256. */
typedef struct sscan_ssd_desc {
  int64_t batch, seqlen, nheads, head_dim, state_dim, ngroups, chunk;
  int32_t act;
  int32_t reserved;   /* must be 0 */
} sscan_ssd_desc;

/* Bytes of workspace sscan_mamba1_fwd needs for this problem (0 if none). */
size_t sscan_mamba1_workspace_size(const sscan_mamba1_desc* desc);

/* Mamba-1 selective scan over a prompt ("Mamba", opening paragraph and section
 * "The values"; "Falcon-Mamba", section "Where the norms sit").
 *   x, dt_raw     [batch, seqlen, channels]  act
 *   dt_bias       [channels]                 f32
 *   A_log         [channels, state_dim]      f32   (A = -exp(A_log))
 *   B, C          [batch, seqlen, ngroups, state_dim] act
 *   D             [channels]                 f32
 *   z             [batch, seqlen, channels]  act, or NULL: no gate; else y *= silu(z)
 *   state_input   [batch, channels, state_dim] f32, or NULL: start from zeros
 *   y             [batch, seqlen, channels]  act  (out)
 *   state_output  [batch, channels, state_dim] f32 (out): the state after the last token
 *   states        [batch, seqlen, channels, state_dim] f32 (out) or NULL: the state after
 *                 every token; states[:, -1] equals state_output bit for bit.
 *   workspace     device buffer of workspace_bytes >= sscan_mamba1_workspace_size()
 * seqlen may be 0: then state_output = state_input (or zeros) and y is untouched. */
sscan_status sscan_mamba1_fwd(const sscan_mamba1_desc* desc, const void* x, const void* dt_raw,
                              const float* dt_bias, const float* A_log, const void* B, const void* C,
                              const float* D, const void* z, const float* state_input, void* y,
                              float* state_output, float* states, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Mamba-1 one-token decode step ("Mamba", section "The state": the state is
 * handed from state_output to the next step's state_input, and the step updates
 * the state before it reads y). desc->seqlen must be 1. Shapes as
 * sscan_mamba1_fwd with seqlen 1; state_input is required and state_output may
 * equal it (update in place). */
sscan_status sscan_step(const sscan_mamba1_desc* desc, const float* state_input, float* state_output,
                        const void* x, const void* dt_raw, const float* dt_bias, const float* A_log,
                        const void* B, const void* C, const float* D, const void* z, void* y,
                        void* stream);

/* Bytes of workspace sscan_ssd_fwd needs for this problem (0 if none). */
size_t sscan_ssd_workspace_size(const sscan_ssd_desc* desc);

/* Byte offset, in the workspace of an sscan_ssd_fwd call that takes the MFMA
 * chunk path (head_dim 64, 128, 256, ..., state_dim 64..128, states NULL; act
 * bf16, or f32 unless SSCAN_TUNE_SSD_F32_TOKEN_LOOP is set), of a 32-bit
 * word that is 0 after the call unless a state hand-off between two segments of
 * a head's sequence gave up waiting (see sscan_ssd_fwd). */
#define SSCAN_SSD_GIVEUP_WORD_OFFSET 512

/* Mamba-2 SSD scan over a prompt ("Mamba-2", sections "The mixer's values",
 * "The block, in order", "The hidden attention" and "The state").
 *   x, z          [batch, seqlen, nheads, head_dim] act (z NULL: no gate)
 *   dt_raw        [batch, seqlen, nheads]   act
 *   dt_bias, A_log, D [nheads]              f32
 *   B, C          [batch, seqlen, ngroups, state_dim] act
 *   state_input   [batch, nheads, head_dim, state_dim] f32 or NULL (zeros)
 *   y             [batch, seqlen, nheads, head_dim] act (out): ssd(...) + D*x, gated if z
 *   state_output  [batch, nheads, head_dim, state_dim] f32 (out)
 *   states        [batch, seqlen, nheads, head_dim, state_dim] f32 (out) or NULL
 * The state is stored value side (head_dim) first and state_dim innermost: entry
 * [b, h, p, n] is the pages' [b, h, key n, value p]. state_dim in 1..128.
 * head_dim 64 times a power of two (64, 128, 256, ...) with state_dim 64..128 and
 * no per-token states takes the MFMA chunk path: bf16 MFMA for bf16 activations,
 * fp32 MFMA (fp32 products and sums) for fp32 ones. A head of 64 m columns runs as m
 * heads of 64 columns that share its step, decay and D (its columns are
 * independent given those), so its results are those of that split, bit for bit.
 * state_dim below 128 runs on B, C and states padded with zero states in the
 * workspace (the padded entries stay exactly zero), with the results of that
 * padding, bit for bit. Other shapes take the token loop (fp32 arithmetic).
 * The MFMA chunk path cuts a head's sequence into segments that different
 * workgroups scan. In one pass each segment hands its final state to the next
 * through the workspace. The kernel's own scheduling guarantees every hand-off
 * wait ends; its bound exists only so that the kernel always terminates. A wait
 * that gives up sets the word at SSCAN_SSD_GIVEUP_WORD_OFFSET and starts its
 * segment from a NaN state, so every output that depends on the missing hand-off
 * (the rest of that head's y, and its state_output) is NaN, never silently wrong.
 * With fewer heads x batch rows than the GPU has compute units the path takes two
 * passes instead (SSCAN_TUNE_SSD_TWO_PASS): every segment but the last is first
 * scanned from a zero state, then every segment runs at once from its entering
 * state, folded from those (S_in of the next segment = 2^(segment's sum of dt*A,
 * exp2 domain) S_in + the segment's state from zero); nothing waits. */
sscan_status sscan_ssd_fwd(const sscan_ssd_desc* desc, const void* x, const void* dt_raw,
                           const float* dt_bias, const float* A_log, const void* B, const void* C,
                           const float* D, const void* z, const float* state_input, void* y,
                           float* state_output, float* states, void* workspace, size_t workspace_bytes,
                           void* stream);

/* sscan_ssd_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, and the same kernels and results. What the
 * workspace would hold (the chunk path's work queues, give-up word, state
 * hand-offs and C.B^T tiles, or the token loop's slice carries) lives in the library's static
 * device scratch of SSCAN_NOALLOC_SCRATCH_BYTES, which every GPU the library runs
 * on holds from the first call until the process ends. A problem that needs more
 * returns SSCAN_ERR_UNSUPPORTED before any launch (sscan_ssd_workspace_size
 * gives the need). The call allocates nothing and frees nothing. Every call on
 * one GPU shares that GPU's scratch, and the kernels clear what must start at
 * zero, so calls that overlap in time on one GPU (several streams or threads)
 * race and give wrong results; calls in sequence on one stream are safe. The
 * give-up word (SSCAN_SSD_GIVEUP_WORD_OFFSET) is in the scratch, not visible to
 * the caller; a give-up still turns the dependent outputs to NaN. */
#define SSCAN_NOALLOC_SCRATCH_BYTES (16u << 20)
sscan_status sscan_ssd_fwd_noalloc(const sscan_ssd_desc* desc, const void* x, const void* dt_raw,
                                   const float* dt_bias, const float* A_log, const void* B, const void* C,
                                   const float* D, const void* z, const float* state_input, void* y,
                                   float* state_output, float* states, void* stream);

/* Mamba-2 one-token decode step: sscan_ssd_fwd with seqlen 1, state_input
 * required, state_output may equal state_input ("Mamba-2", section "The state":
 * on a decode step the update comes before the read). */
sscan_status sscan_ssd_step(const sscan_ssd_desc* desc, const float* state_input, float* state_output,
                            const void* x, const void* dt_raw, const float* dt_bias, const float* A_log,
                            const void* B, const void* C, const float* D, const void* z, void* y,
                            void* stream);

/* The SSD scan's hidden attention map, an optional output for inspection
 * ("Mamba-2", section "The hidden attention"): per head the scan is the causal
 * linear map y_t = sum_s alpha[t, s] x_s + D x_t (before the gate), with
 *     alpha[b, t, s, h] = (C_t . B_s) * exp(decays_{s+1} + ... + decays_t) * betas_s  for s <= t,
 * and 0 for s > t; betas = softplus(dt_raw + dt_bias), decays = betas * A,
 * A = -exp(A_log) ("The mixer's values"); head h reads group h / (nheads / ngroups).
 * desc as for sscan_ssd_fwd (head_dim and chunk are not used).
 *   dt_raw        [batch, seqlen, nheads]   act
 *   dt_bias, A_log [nheads]                 f32
 *   B, C          [batch, seqlen, ngroups, state_dim] act
 *   alpha         [batch, seqlen (query t), seqlen (key s), nheads] f32 (out),
 *                 batch * seqlen^2 * nheads * 4 bytes: meant for modest lengths.
 *   workspace     device buffer of workspace_bytes >= sscan_ssd_attention_workspace_size()
 *                 (batch * seqlen * nheads * 12 bytes: the running decay sums in fp64
 *                 and the betas); contents on entry do not matter; must not overlap
 *                 the other buffers (SSCAN_ERR_WORKSPACE when too small or NULL).
 * Every entry is written (zeros above the diagonal). SSCAN_ERR_UNSUPPORTED when the
 * map has 2^31 or more tiles of 32 query x 32 key tokens x up to 128 heads. */
size_t sscan_ssd_attention_workspace_size(const sscan_ssd_desc* desc);
sscan_status sscan_ssd_attention(const sscan_ssd_desc* desc, const void* dt_raw, const float* dt_bias,
                                 const float* A_log, const void* B, const void* C, float* alpha,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Causal depthwise conv1d + silu, the step in front of the scan ("Mamba-2",
 * section "The block, in order": x, B, C = silu(conv1d(xBC)), causal, width 4;
 * "Mamba", tokentrails lineage, section "Code": depthwise, width 4).
 * Output token t of channel c is
 *     out[b, t, c] = silu(bias[c] + sum_{k=0}^{W-1} weight[c, k] * xx[t - W + 1 + k])
 * where xx is x preceded by the W-1 inputs of conv_state_in (oldest first), or
 * by zeros when conv_state_in is NULL.
 *   x, out          [batch, seqlen, channels]  act
 *   weight          [channels, width]          f32
 *   bias            [channels] f32 or NULL
 *   conv_state_in   [batch, channels, width-1] f32 or NULL
 *   conv_state_out  [batch, channels, width-1] f32 or NULL: the last width-1 inputs
 *                   (for the next call); may not alias conv_state_in.
 * width in 1..8. seqlen may be 0 (the state passes through). */
typedef struct sscan_conv_desc {
  int64_t batch, seqlen, channels, width;
  int32_t act;
  int32_t reserved;   /* must be 0 */
} sscan_conv_desc;

sscan_status sscan_conv1d_silu(const sscan_conv_desc* desc, const void* x, const float* weight, const float* bias,
                               const float* conv_state_in, void* out, float* conv_state_out, void* stream);

/* Gated RMS norm after the SSD ("Mamba-2", section "The block, in order" and
 * the note under it): g = y * silu(z), then
 *     out = g / sqrt(mean(g^2) + eps) * weight
 * with the mean over the whole width of a row (all heads), in fp32.
 *   y, z, out  [rows, width] act;  weight [width] f32;  eps > 0. */
sscan_status sscan_gated_rmsnorm(int64_t rows, int64_t width, int32_t act, const void* y, const void* z,
                                 const float* weight, float eps, void* out, void* stream);

/* Text of a status code (static storage). */
const char* sscan_status_string(int status);
/* Detail of the last failing call on this thread (thread-local storage). */
const char* sscan_last_error(void);
/* SSCAN_ABI_VERSION of the library. */
int sscan_abi_version(void);
/* 1 (default): check that tensor pointers are device memory on every call
 * (hipPointerGetAttributes); 0: skip that check (shape, alignment and alias
 * checks still run). Process-wide; returns the previous setting. */
int sscan_set_pointer_checks(int enabled);

/* Tuning and test overrides of the launch plans. Process-wide (atomics), read
 * when a call plans its launch; value 0 restores the library's own choice.
 * Returns the previous value, or -1 (and changes nothing) for an unknown knob or
 * a negative value. A knob changed between a *_workspace_size query and the
 * call it sizes can change the workspace the call needs: the call then returns
 * SSCAN_ERR_WORKSPACE instead of launching. */
typedef enum {
  SSCAN_TUNE_M1_LANES = 1,          /* lanes per channel of the Mamba-1 prompt kernels: 1, 2, 4 or 16
                                       (others, and shapes the kernel cannot take, are ignored) */
  SSCAN_TUNE_SSD_SEGMENT_CHUNKS = 2, /* chunks per segment of the SSD chunk path */
  SSCAN_TUNE_SSD_WORKGROUPS = 3,    /* workgroups of the SSD chunk path */
  SSCAN_TUNE_SSD_GIVE_UP = 4,       /* nonzero: every state hand-off wait of the SSD chunk path gives
                                       up at once (for testing what a wait that gives up does) */
  SSCAN_TUNE_SSD_HEADS_PER_WORKGROUP = 5, /* 2: two neighbouring heads of a group share a workgroup of
                                       the SSD chunk path, with B, C and C.B^T staged once (by
                                       default one head per workgroup; same results; bf16 only) */
  SSCAN_TUNE_SSD_F32_TOKEN_LOOP = 6, /* nonzero: fp32 activations of sscan_ssd_fwd take the token loop
                                       instead of the fp32 MFMA chunk path */
  SSCAN_TUNE_SSD_TWO_PASS = 7,      /* the SSD chunk path's form: 1 one pass (a head's segments hand
                                       their states on in turn), 2 two passes (every segment but the
                                       last from a zero state, then all segments at once from states
                                       folded from those); 0 the library's choice (two passes when a
                                       problem has too few heads x batch rows to fill the GPU) */
  SSCAN_TUNE_SSD_SPLIT_STATE = 8    /* nonzero: the bf16 SSD chunk path carries the state as C reads
                                       it and the weighted inputs w x that update it as two bf16 parts
                                       each (hi, and the rounding hi leaves out), about 16 significant
                                       bits instead of 8: closer results for heads whose slow decays
                                       make the state sum thousands of tokens, at twice the MFMA work of
                                       those two products (one head per workgroup) */
} sscan_tune_knob;
int64_t sscan_set_tuning(int knob, int64_t value);

#ifdef __cplusplus
}
#endif
#endif /* SSCAN_H */
