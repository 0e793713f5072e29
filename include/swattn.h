/*
 * swattn.h -- C ABI of the banded sliding-window attention library for AMD
 * MI355X (gfx950).
 *
 * The operation is Longformer-style self-attention as the Longformer summary
 * page (velog.io/@lainshower/Longformer) describes it in section 3-1
 * "Attention Pattern":
 *   - "Sliding Window": token i attends to w/2 tokens on each side;
 *   - "Dilated Sliding Window": the window keeps its w+1 keys, spaced by a
 *     per-head dilation, so its span grows to w*dilation;
 *   - "Global Attention": a small set G of tokens attends to every token and
 *     is attended by every token;
 *   - "Linear Projections for Global Attention": the rows of G are computed
 *     from separate projections Qg, Kg, Vg;
 * and section 7 "Longformer-Encoder-Decoder" for the optional left-only
 * (causal) mask.
 *
 * Precisely, for head h with window w_h (even) and dilation d_h, and the
 * softmax scale s = 1/sqrt(d):
 *   band(i,j)  <=>  j = i + k*d_h  for an integer k in [-w_h/2, R_h],
 *                   R_h = 0 when causal, w_h/2 otherwise;
 *   row i not in G:  keys A(i) = band(i) U {g in G : (not causal) or g <= i},
 *                    each key counted once, projections Q, K, V;
 *   row g in G:      keys {j : (not causal) or j <= g}, projections Qg, Kg, Vg;
 *   O_i   = sum_{j in A(i)} softmax_j(s q_i.k_j) v_j,
 *   LSE_i = ln sum_{j in A(i)} exp(s q_i.k_j)   (natural log, fp32).
 *
 * Threading: a plan may be used from any host thread, but not by two
 * in-flight forwards at once (they share the plan's device workspace).
 * No C++ exception crosses this interface.
 */
#ifndef SWATTN_H
#define SWATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define SWATTN_OK 0
#define SWATTN_ERR_INVALID_ARG 1 /* a parameter is out of its documented range */
#define SWATTN_ERR_UNSUPPORTED 2 /* valid, but not implemented (e.g. d != 64) */
#define SWATTN_ERR_HIP 3         /* the HIP runtime reported an error */
#define SWATTN_ERR_ALIGNMENT 4   /* a device pointer is not 16-byte aligned */

/* Element types of Q, K, V, Qg, Kg, Vg and O. */
#define SWATTN_BF16 0 /* bfloat16 in and out, fp32 accumulation */
#define SWATTN_FP32 1 /* fp32 in and out, fp32 accumulation */

typedef struct swattn_params {
  int32_t batch;               /* B >= 1 */
  int32_t heads;               /* H >= 1 */
  int32_t n;                   /* sequence length, 1 <= n <= 2^24 */
  int32_t d;                   /* head dimension; only 64 is supported */
  const int32_t* window;       /* host [H]: w_h, even, 0 <= w_h (any size; clipped at the ends) */
  const int32_t* dilation;     /* host [H]: d_h >= 1 */
  int32_t causal;              /* 0 or 1: left-only mask on band, global rows and global columns */
  const int32_t* global_idx;   /* host [n_global]: positions of G, each in [0, n), no repeats, any order */
  int32_t n_global;            /* 0 <= |G| <= n; global_idx may be NULL when 0 */
  int32_t dtype;               /* SWATTN_BF16 or SWATTN_FP32 */
  const int32_t* global_offsets; /* host [batch+1] or NULL. NULL: global_idx is one set G
                                    shared by every batch item. Otherwise batch item b has
                                    its own set global_idx[global_offsets[b] ..
                                    global_offsets[b+1]) (each in [0, n), no repeats within
                                    an item, any order, at most n per item; offsets start
                                    at 0, never decrease and end at n_global <= batch*n):
                                    the QA setting of section 3-1, where each example's
                                    question tokens are its global tokens. */
  int32_t key_split;           /* 0: the library decides; 1: never; 2..16: the band keys of
                                  every 128-row tile are shared out over this many
                                  workgroups, whose partial results a merge kernel
                                  combines (for problems too small to fill the GPU; the
                                  result is the same up to fp32 rounding). Zero-initialising
                                  the struct selects 0. */
} swattn_params;

typedef struct swattn_plan swattn_plan;

/*
 * Validate the parameters and build a plan for the attention pattern of
 * section 3-1 of the Longformer summary page: the per-head window ("Sliding
 * Window") and dilation ("Dilated Sliding Window"), the global set ("Global
 * Attention") and the left-only mask of section 7. The plan holds the
 * per-head (left, right, dilation) table, the residue-class tile schedule of
 * the band and its key split, the
 * sorted device copy of G (per item with global_offsets), and one device
 * allocation for every workspace the forward and backward use (global-row
 * partials, key-split partials, the backward's per-row statistics). Every
 * host array is copied; the caller may free them when this returns. Uses the
 * current HIP device; the plan may only be used with streams of that device.
 * On success *out receives the plan; on failure *out is untouched.
 * Errors: INVALID_ARG (null pointers, ranges, odd window, dilation < 1,
 * repeated or out-of-range global index, bad global_offsets, key_split
 * outside [0, 16]), UNSUPPORTED (d != 64, unknown dtype, sizes beyond the
 * 32-bit grid limits or a key-split workspace above 1 GiB), HIP (device
 * allocation or copy failed; see swattn_last_error()).
 */
int swattn_create(const swattn_params* p, swattn_plan** out);

/*
 * Enqueue one forward pass on `stream` (a hipStream_t; NULL = the default
 * stream) and return without waiting: O and LSE as defined at the top of this
 * file (section 3-1 of the Longformer summary page, its four bullets, and
 * section 7 for the causal mask), the band and the global columns from
 * Q, K, V, the rows of G from Qg, Kg, Vg ("Linear Projections for Global
 * Attention").
 *   q, k, v     device, [B, H, n, d] contiguous (d fastest), plan dtype;
 *   qg, kg, vg  device, same shape and dtype: the separate global projections
 *               (only rows G of qg are read; kg, vg are read in full). They
 *               must be NULL exactly when n_global == 0;
 *   o           device, [B, H, n, d] plan dtype, written in full; must not
 *               overlap any input;
 *   lse         device fp32 [B, H, n] or NULL to skip.
 * All device pointers must be 16-byte aligned (else ALIGNMENT) and stay
 * valid until the stream reaches the enqueued work. The caller owns every
 * buffer; forward allocates nothing. Forwards on one plan share its
 * workspace (the global rows' partial records and, with one global token
 * per item, their arrival counters), so they must not run concurrently:
 * enqueue them on one stream, or synchronise between them. The current HIP
 * device must be the plan's. Errors: INVALID_ARG (null plan or tensor, NULL-ness of qg/kg/vg
 * not matching n_global, o overlapping an input, another current device),
 * ALIGNMENT, HIP (launch failure; see swattn_last_error()).
 */
int swattn_forward(swattn_plan* plan, const void* q, const void* k,
                   const void* v, const void* qg, const void* kg,
                   const void* vg, void* o, float* lse, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward pass as swattn_create + swattn_forward + swattn_destroy, in one
 * call that allocates nothing. The parameters are those of swattn_create and
 * are validated the same way; the tensors are those of swattn_forward, with
 * the same rules. The schedule tables and the partial results exchanged
 * between the kernels live in a 32 MiB array in device memory that the
 * library reserves statically (each GPU it runs on holds one copy until the
 * process ends) instead of in a plan; the tables reach it through the
 * arguments of small copy kernels enqueued on `stream`, so no host buffer
 * must outlive the call. Nothing in the array has to start at zero: every
 * entry a kernel reads was written earlier in the same call. Every call on
 * one GPU uses that GPU's array, so two calls whose work overlaps in time
 * on one GPU (different streams, or host threads) race and may return wrong
 * results: serialise them. Enqueues work and returns without waiting.
 * Errors: as swattn_create and swattn_forward; UNSUPPORTED also when the
 * problem needs more than 32 MiB of that array (its global-row partials,
 * B*H*|G|*ceil(n/256)*264 bytes, plus its key-split partials, B*H*n*parts*
 * 272 bytes, plus the tables), or the device index is above 63.
 */
int swattn_forward_noalloc(const swattn_params* p, const void* q, const void* k,
                           const void* v, const void* qg, const void* kg,
                           const void* vg, void* o, float* lse, void* stream);

/*
 * Enqueue the backward pass of one forward on `stream` and return without
 * waiting: the gradients of Q, K, V (and of Qg, Kg, Vg) for a cotangent dout
 * of O. With P_ij = exp(s q_i.k_j - LSE_i) on the key set A(i) of the
 * forward (section 3-1 of the Longformer summary page, as above):
 *   D_i = dout_i . O_i,  dS_ij = P_ij (dout_i.v_j - D_i),
 *   dq_i = s sum_j dS_ij k_j,  dk_j = s sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i,
 * and the same with Qg, Kg, Vg for the rows of G (which take nothing from
 * Q, K, V: dq is zero on them).
 *   q .. vg   the forward's inputs (same rules as swattn_forward);
 *   o, lse    the forward's outputs for those inputs (lse is required);
 *   dout      device [B, H, n, d] plan dtype;
 *   dq, dk, dv        device [B, H, n, d] plan dtype, written in full;
 *   dqg, dkg, dvg     the same for the global projections; NULL exactly
 *                     when n_global == 0.
 * Gradients must not overlap each other or any input. The plan's workspace
 * holds per-row statistics, so a plan runs one backward (or forward) at a
 * time. bf16 plans run on the matrix cores (P and dS enter their products
 * in bf16); fp32 plans run an fp32 path on the vector ALUs, one wavefront
 * per row for dq, dqg and one per key position for dk, dv, dkg, dvg, for
 * correctness rather than speed. Tensors have the plan's dtype; the
 * current HIP device must be the plan's.
 * Errors: INVALID_ARG, ALIGNMENT, HIP.
 */
int swattn_backward(swattn_plan* plan, const void* q, const void* k, const void* v,
                    const void* qg, const void* kg, const void* vg, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* dqg, void* dkg, void* dvg, void* stream);

/*
 * Enqueue the projections in front of the attention on `stream` (a
 * hipStream_t; NULL = the default stream): the linear maps that produce Q, K,
 * V from a layer's input and, for global tokens, the separate Qg, Kg, Vg
 * (section 3-1 of the Longformer summary page, "Linear Projections for Global
 * Attention"). Needs no plan. For projection p < nproj, head h, token i of
 * batch item b and feature e < 64:
 *   out[p][b][h][i][e] = sum_c x[b][i][c] * w[(p*heads + h)*64 + e][c]
 *                        + bias[(p*heads + h)*64 + e]
 * accumulated in fp32 and, for bf16, rounded once to bf16. x, w, bias and
 * out all have the type `dtype` (SWATTN_BF16: the matrix cores; SWATTN_FP32:
 * the vector ALUs, a plain fp32 dot product in input-feature order).
 *   x     device [batch, n, d_model] contiguous;
 *   w     device [nproj*heads*64, d_model]: one output feature per row,
 *         the layout of a linear layer's weight; the rows of projection p
 *         are the block p*heads*64 .. (p+1)*heads*64-1, head-major;
 *   bias  device [nproj*heads*64] or NULL (no bias);
 *   out   device [nproj, batch, heads, n, 64], written in full: out + p*
 *         batch*heads*n*64 elements is projection p in the [B, H, n, d]
 *         layout swattn_forward reads (order q, k, v, then qg, kg, vg);
 *         must not overlap an input.
 * d_model must be a multiple of 32 and x, w each smaller than 2 GiB; every
 * device pointer 16-byte aligned. The caller owns every buffer; nothing is
 * allocated. Errors: INVALID_ARG (NULL pointer, size < 1, out overlapping an
 * input), UNSUPPORTED (unknown dtype, d_model, sizes),
 * ALIGNMENT, HIP (launch failure).
 */
int swattn_project(const void* x, const void* w, const void* bias, void* out,
                   int batch, int n, int d_model, int heads, int nproj, int dtype,
                   void* stream);

/*
 * Free the plan (the pattern tables of section 3-1 that swattn_create built,
 * and its workspaces) and its device memory. NULL is a no-op. The caller must
 * make sure no enqueued forward still uses the plan (e.g. synchronise its
 * stream).
 */
int swattn_destroy(swattn_plan* plan);

/*
 * Measurement hooks (not part of the computation). With timing enabled, each
 * forward records HIP events on its stream around its kernels, in two
 * phases: the forward kernel (band rows, global columns and the global rows'
 * partials), and the merges after it (the key-part merge with a key split,
 * the global-row merge with global tokens unless the kernel folds the
 * global row itself, as it does in bf16 with at most one global token per
 * item and no key split; from before the first one to after the last one,
 * 0 when there are none). An interval covers the
 * kernels' dispatch and completion, including the cache write-back at a
 * kernel's end; up to 4096 forwards are kept.
 * swattn_kernel_times() waits for the recorded events, returns the average
 * duration in milliseconds of each phase over the recorded forwards and the
 * number of forwards averaged, then clears the record. Enabling creates the
 * events (host objects); disabling destroys them. Errors: INVALID_ARG (NULL
 * plan or outputs), HIP.
 */
int swattn_set_timing(swattn_plan* plan, int enable);
int swattn_kernel_times(swattn_plan* plan, float* band_ms, float* global_ms, int* count);

/* Static, human-readable name of a status code. */
const char* swattn_status_string(int status);

/* Message of the last error raised on this host thread ("" when none):
 * the HIP runtime's error text for SWATTN_ERR_HIP, else the failed check. */
const char* swattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SWATTN_H */
