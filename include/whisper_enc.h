/*
 * whisper_enc.h - C ABI of the MI355X (gfx950) Whisper-style encoder block library.
 *
 * The library computes the forward pass of the pre-LayerNorm transformer block of the Whisper
 * audio encoder over 30 s windows (t = 1500 positions), for one block or a stack of blocks
 * ending in an optional final LayerNorm:
 *
 *   a  = LN1(x)                               LayerNorm, eps 1e-5, biased variance
 *   q  = a Wq^T + bq,  k = a Wk^T,  v = a Wv^T + bv          (K has no bias)
 *   o  = softmax(q_h k_h^T / sqrt(64)) v_h  per head h, bidirectional, per window
 *   x1 = x + o Wo^T + bo
 *   y  = x1 + gelu(LN2(x1) W1^T + b1) W2^T + b2              gelu(z) = z/2 (1 + erf(z/sqrt 2))
 *
 * Sources: inferencelayer 0.2.4 "whisper_gpu.rs" (VANILLA_ATTN and LN_SRC shaders,
 * WhisperEncoderGpu::forward), turbospark-runtime 0.3.0 "src/whisper/metal.rs" (module doc,
 * EncLayerGpu, encode_layer, encode_partial), oxinfer "src/whisper/model.rs" (WhisperConfig,
 * Precision, WhisperModel::encode).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers (memory of the current HIP device) unless marked "host".
 *     The caller owns every buffer; the library never allocates, frees or synchronises, keeps
 *     no mutable global state (apart from the static scratch of
 *     whisper_enc_stack_forward_noalloc), and enqueues all work on `stream` (a hipStream_t;
 *     NULL = the default stream).  Results are ready when the stream's work completes.
 *   - Matrices are row-major.  Activations x, y are [batch, t, d_model] fp32; weights are in
 *     PyTorch layout [n_out, n_in].
 *   - Every argument is validated before anything is enqueued; a call that returns an error
 *     has enqueued nothing.  A launch failure reported by HIP returns WENC_ERR_HIP; faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - Calls with zero rows (batch * t == 0) enqueue nothing and return WENC_OK; their data
 *     pointers may then be NULL.
 *   - Calls on one stream run in order; concurrent calls on different streams need separate
 *     workspaces and outputs.
 */
#ifndef WHISPER_ENC_H
#define WHISPER_ENC_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define WENC_OK 0
#define WENC_ERR_ARG 1         /* NULL pointer, misaligned pointer, bad size or enum value   */
#define WENC_ERR_UNSUPPORTED 2 /* valid shape the kernels do not implement: hd != 64, or one  */
                               /* window's QKV rows (t * 3 d_model elements) >= 2 GiB        */
#define WENC_ERR_WORKSPACE 3   /* workspace_bytes below whisper_enc_workspace_bytes()       */
#define WENC_ERR_HIP 4         /* HIP reported an error for a launch                         */
#define WENC_ERR_SCRATCH 5     /* whisper_enc_stack_forward_noalloc: the shape needs more     */
                               /* workspace than its static scratch holds                    */

/* Arithmetic paths: the type of every matrix-multiply operand.  Accumulation, LayerNorm
 * statistics, softmax state and the residual stream are fp32 on every path.
 *   BF16 - bfloat16 MFMA operands (weights rounded to nearest even when packed);
 *   BF16X2 - layer and stack calls only: bfloat16 weights and MFMA operands, with the LayerNorm
 *     and GELU outputs (the QKV, fc1 and fc2 activations) carried as two bfloat16 numbers,
 *     hi = bf16(v) and lo = bf16(v - hi), both multiplied by the same bf16 weight row, so those
 *     projections see v to ~2^-17 instead of bf16's 2^-9 (twice the MFMA work on them); Q, K, V,
 *     the probabilities and the attention output stay single bfloat16.  For bf16-valued weights;
 *   BF16X3 - as BF16X2, with every weight also packed as a bf16 hi / lo pair (twice the blob):
 *     the projections compute x_hi w_hi + x_lo w_hi + x_hi w_lo (dropping x_lo w_lo, ~2^-18;
 *     three times the MFMA work; the out-projection x w_hi + x w_lo), for fp32 weights that bf16
 *     storage would round;
 *   FP32 - fp32 operands and intermediates (fp32 MFMA), the fallback path;
 *   FP16 - IEEE half MFMA operands, same MFMA rate as BF16 with 3 more mantissa bits;
 *   Q8, Q4 - layer and stack calls only (every other entry point rejects them): the packed
 *     weight matrices are stored as int8 (Q8) or int4 (Q4) codes in blocks of 32 consecutive
 *     input columns with one fp16 scale per block, quantised from the matrices rounded to bf16
 *     (oxinfer whisper/model.rs, Precision and make_lin: q8 / q4 blocks of 32 from bf16).  The
 *     encodings follow the q8_0 / q4_0 block formats:
 *       Q8: d = amax / 127, code = round-half-away(x / d) in [-127, 127], value = code * d;
 *       Q4: m = first element of largest magnitude, d = m / -8,
 *           code = min(15, floor(x / d + 8.5)) in [0, 15], value = (code - 8) * d;
 *     (fp32 arithmetic, x times the correctly rounded fp32 1 / d; d stored as fp16).  Each block
 *     call expands its layer's matrices to fp16 in the workspace and runs the FP16 path;
 *   MXFP8 - gfx950's block-scaled fp8 arithmetic for oxinfer's blocks of 32 (Precision,
 *     make_lin): the QKV, fc1 and fc2 projections run on MXFP8 operands (OCP Microscaling
 *     Formats v1.0: E4M3 values, one power-of-two E8M0 scale 2^X per 32 consecutive input
 *     columns of a row, X the smallest integer with amax <= 448 * 2^X, values rounded to nearest
 *     even) with fp32 accumulation: their weights are quantised when packed, and their
 *     activations (the two LayerNorm outputs and the GELU output) by the kernels that produce
 *     them.  Attention and the out-projection stay FP16.  A different numerical method: the
 *     operands carry 4 significant bits, so outputs differ from the fp32 model by about 1 % of
 *     their RMS per block; it is not held to the FP16 path's error bounds.  Layer and stack
 *     calls, whisper_enc_linear and whisper_enc_layernorm (WENC_DTYPE_MXFP8) accept it; the
 *     attention, front-end and cross K/V calls do not. */
#define WENC_PATH_BF16 0
#define WENC_PATH_FP32 1
#define WENC_PATH_FP16 2
#define WENC_PATH_Q8 3
#define WENC_PATH_Q4 4
#define WENC_PATH_BF16X2 5
#define WENC_PATH_BF16X3 6
#define WENC_PATH_MXFP8 7

/* Element types of step-level outputs. */
#define WENC_DTYPE_F32 0
#define WENC_DTYPE_BF16 1
#define WENC_DTYPE_F16 2
#define WENC_DTYPE_MXFP8 3 /* an MXFP8 matrix, laid out as whisper_enc_mx_quantize writes it */

/* Projection epilogues (whisper_enc_linear). */
#define WENC_EPI_BIAS 0          /* c = a w^T + bias                        (path dtype) */
#define WENC_EPI_BIAS_GELU 1     /* c = gelu_erf(a w^T + bias)              (path dtype) */
#define WENC_EPI_BIAS_RESIDUAL 2 /* c = residual + a w^T + bias              (fp32)      */
#define WENC_EPI_BIAS_GELU_RESIDUAL 3 /* c = residual + gelu_erf(a w^T + bias) (fp32)      */

/* Limits checked by every entry point. */
#define WENC_HEAD_DIM 64
#define WENC_MAX_D_MODEL 4096
#define WENC_MAX_FFN_DIM 65536
#define WENC_MAX_ROWS (1 << 24)
#define WENC_MAX_DEC_LAYERS 64
#define WENC_MAX_MELS 1024

/* Human-readable text of a status code (static storage; never NULL).  The pages report
 * errors as text (inferencelayer WhisperEncoderGpu::forward returns Result with ensure!
 * messages; turbospark-runtime encode returns Result<(), String>); a C ABI returns the code and
 * offers its text here. */
const char* whisper_enc_strerror(int code);

/*
 * Size in bytes of one packed layer blob (256-byte aligned sections), 0 if the arguments are
 * invalid.  The blob holds LN1/LN2 gamma and beta, the QKV bias with a zero K slot, the out,
 * fc1 and fc2 biases (all fp32), and Wqkv [3d, d] (Q, K, V row blocks), Wo [d, d],
 * W1 [ffn, d], W2 [d, ffn] in the path's operand type (oxinfer Precision: norms and biases
 * always stay f32; turbospark-runtime DecLayerGpu: packed [3d, d] QKV with a zero K bias);
 * on WENC_PATH_Q8 / WENC_PATH_Q4 the matrices are held as codes plus fp16 block scales
 * (1 + 1/16 or 1/2 + 1/16 bytes per weight).  The blob is opaque: only whisper_enc_pack_layer
 * writes it.
 */
size_t whisper_enc_layer_bytes(int d_model, int ffn_dim, int path);

/*
 * Pack one block's parameters into `dst_layer` (device, layer_bytes(), 256-byte aligned).
 * Sources are device fp32 arrays in PyTorch layout: ln*_g/ln*_b [d]; wq, wk, wv, wo [d, d];
 * w1 [ffn, d]; w2 [d, ffn]; bq, bv, bo, b2 [d]; b1 [ffn].  `bk` may be NULL (Whisper's K
 * projection has no bias), which packs zeros.  Matrices are rounded to the path's operand type
 * (round to nearest even), fp32 on WENC_PATH_FP32.  Runs asynchronously on `stream`; the sources
 * must stay valid until it completes.
 */
int whisper_enc_pack_layer(const float* ln1_g, const float* ln1_b, const float* wq,
                           const float* bq, const float* wk, const float* bk, const float* wv,
                           const float* bv, const float* wo, const float* bo,
                           const float* ln2_g, const float* ln2_b, const float* w1,
                           const float* b1, const float* w2, const float* b2, int d_model,
                           int ffn_dim, int path, void* dst_layer, void* stream);

/*
 * The intermediate buffers of one call (inferencelayer WhisperEncoderGpu::forward allocates
 * them on every call; turbospark-runtime WhisperMetalEngine::new allocates the scratch for a full
 * window once), here owned by the caller and sized by this call.
 * Workspace bytes a block/stack call needs for `batch` windows of `t` positions: the LN
 * output / attention output [batch*t, d] and the QKV / FFN hidden activations
 * [batch*t, max(3d, ffn)], in the path's operand type; on the Q8 / Q4 paths room for one
 * layer's matrices expanded to fp16 (2 (4d^2 + 2 d ffn) bytes); and, when batch*t is too small
 * for the out-projection and fc2 to fill the GPU (one window), fp32 partial sums of those
 * split-k products (up to 8 x batch*t x d floats, added in a fixed order: results stay
 * deterministic), a region that also holds the two key halves' partial attention state
 * (2 x batch*t x heads x 66 floats) when too few query blocks would run to fill the GPU.
 * The size depends only on the arguments.  0 if the arguments are invalid.
 */
size_t whisper_enc_workspace_bytes(int batch, int t, int d_model, int heads, int ffn_dim,
                                   int path);

/*
 * One pre-LN encoder block (inferencelayer WhisperEncoderGpu::forward, block loop;
 * turbospark-runtime encode_layer; oxinfer WhisperModel::encode, layer loop):
 *   y = x1 + FFN(LN2(x1)),  x1 = x + Attn(LN1(x)).
 * x, y: [batch, t, d_model] fp32, 16-byte aligned; y == x (in place) is allowed, partial
 * overlap is not.  layer: a blob from whisper_enc_pack_layer with the same d_model, ffn_dim and
 * path.  heads must give head_dim d_model/heads == 64 (else WENC_ERR_UNSUPPORTED).  Attention
 * never crosses windows.  workspace: device, 256-byte aligned, >= workspace_bytes().
 */
int whisper_enc_block_forward(const float* x, float* y, const void* layer, int batch, int t,
                              int d_model, int heads, int ffn_dim, int path, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * n_layers blocks in order, then the final LayerNorm y = LN(y; ln_post_g, ln_post_b) when
 * ln_post_g is non-NULL (inferencelayer forward, ln_post, optional: "absent when the host
 * model replaced it with Identity"; oxinfer encode, enc_ln).  layers: n_layers blobs packed
 * back to back, blob i at (char*)layers + i * whisper_enc_layer_bytes(...).  n_layers >= 0
 * (0 applies only the final LayerNorm, or copies x to y).  ln_post_b must be non-NULL when
 * ln_post_g is.  Other arguments as for whisper_enc_block_forward.  The result is bit-identical
 * to one whisper_enc_block_forward call per layer followed by whisper_enc_layernorm (where the
 * residual products split k, the LayerNorm that reads a block's output runs inside their final
 * pass, with the same rounding).
 */
int whisper_enc_stack_forward(const float* x, float* y, const void* layers, int n_layers,
                              const float* ln_post_g, const float* ln_post_b, int batch, int t,
                              int d_model, int heads, int ffn_dim, int path, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * whisper_enc_stack_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The workspace is a static device array of WENC_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the first call on that GPU until the process ends; the call itself allocates
 * nothing.  64 MiB hold the workspace of one 1500-position window of every Whisper encoder size
 * on the BF16, FP16 and FP32 paths (large-v3: 47.6 MiB on the 16-bit paths, 36.6 MiB on fp32);
 * larger ones (more windows; large-v3 on Q8 / Q4 with the fp16 copy of its weights, 85.1 MiB, or
 * on BF16X2 / X3 with hi / lo activations) are rejected.  A shape whose whisper_enc_workspace_bytes() exceeds it returns WENC_ERR_SCRATCH
 * (having enqueued nothing).  The array of the current device is used (the stream must belong to
 * it), so calls that overlap on one GPU (other threads, or other streams) race on it: serialise
 * them.  Other arguments and the result are exactly those of whisper_enc_stack_forward.  The
 * first call on a device looks the array's address up (a HIP query, no allocation).
 */
#define WENC_NOALLOC_SCRATCH_BYTES (64 << 20)
int whisper_enc_stack_forward_noalloc(const float* x, float* y, const void* layers, int n_layers,
                                      const float* ln_post_g, const float* ln_post_b, int batch,
                                      int t, int d_model, int heads, int ffn_dim, int path,
                                      void* stream);

/* ---- Step-level entry points: one step of the block each, for tests and profiling. ---- */

/*
 * y[rows, d] = (x - mean) / sqrt(var + 1e-5) * gamma + beta per row, two-pass biased variance
 * (inferencelayer LN_SRC).  x fp32; y in out_dtype (WENC_DTYPE_*); d % 64 == 0, 64 <= d <= 4096.
 * y may equal x for WENC_DTYPE_F32 and must not otherwise overlap it.  WENC_DTYPE_MXFP8 writes
 * whisper_enc_mx_bytes(rows, d) bytes at y, each block of 32 columns scaled as
 * whisper_enc_mx_quantize does.
 */
int whisper_enc_layernorm(const float* x, const float* gamma, const float* beta, void* y,
                          int rows, int d, int out_dtype, void* stream);

/*
 * One projection c = epilogue(a w^T + bias): a [m, k] and w [n, k] in the path's operand type
 * (fp32 on WENC_PATH_FP32), bias [n] fp32.  WENC_EPI_BIAS / WENC_EPI_BIAS_GELU write c [m, n]
 * in the operand type; WENC_EPI_BIAS_RESIDUAL writes fp32 c = residual + a w^T + bias and
 * WENC_EPI_BIAS_GELU_RESIDUAL fp32 c = residual + gelu_erf(a w^T + bias) (the conv front end's
 * second convolution plus positions), with residual [m, n] fp32 (c == residual allowed).
 * n % 64 == 0, k % 64 == 0.  WENC_PATH_MXFP8: a and w are MXFP8 matrices of m and n rows of k
 * (whisper_enc_mx_quantize layout; m * k and n * k below 2^31, else WENC_ERR_UNSUPPORTED);
 * WENC_EPI_BIAS writes fp16 c [m, n], WENC_EPI_BIAS_GELU an MXFP8 matrix of m rows of n
 * (whisper_enc_mx_bytes(m, n) bytes at c).
 */
int whisper_enc_linear(const void* a, const void* w, const float* bias, const float* residual,
                       void* c, int m, int n, int k, int path, int epilogue, void* stream);

/*
 * Bidirectional attention with head_dim 64 for `batch` windows of t rows (inferencelayer
 * VANILLA_ATTN): row i of window b is at ptr + (b*t + i) * ld; head h occupies columns
 * 64h .. 64h+63.  q, k, v use row stride ld_qkv, o uses ld_o (elements, multiples of 8, at least
 * 64*heads); all in the path's operand type.  o = softmax(q k^T / 8) v per (window, head).
 * t * ld_qkv elements of one window must span less than 2 GiB (else WENC_ERR_UNSUPPORTED).
 */
int whisper_enc_attention(const void* q, const void* k, const void* v, void* o, int batch, int t,
                          int heads, int ld_qkv, int ld_o, int path, void* stream);

/* ---- Low-precision weights, one matrix at a time (what the Q8 / Q4 layer paths use). ---- */

/*
 * Quantise w [n, k] (device fp32, k % 32 == 0) into codes and fp16 scales [n, k / 32] (device,
 * scales 2-byte aligned) with the WENC_PATH_Q8 (bits 8: int8 codes [n, k]) or WENC_PATH_Q4
 * (bits 4: codes [n, k / 2] bytes, column 2i in the low nibble of byte i, 2i + 1 in the high one)
 * encoding.  Asynchronous on `stream`.
 */
int whisper_enc_quantize_matrix(const float* w, void* codes, void* scales, int n, int k, int bits,
                                void* stream);

/*
 * Expand codes + scales (as written by whisper_enc_quantize_matrix; codes and dst 16-byte
 * aligned) to fp16 dst [n, k]: value code * scale (Q4: (code - 8) * scale) rounded once to fp16;
 * n * k / 8 >= 2^31 gives WENC_ERR_UNSUPPORTED.
 */
int whisper_enc_dequantize_matrix(const void* codes, const void* scales, void* dst, int n, int k,
                                  int bits, void* stream);

/*
 * MXFP8 matrices (WENC_PATH_MXFP8).  A matrix of `rows` rows of k values (k % 32 == 0) is
 * rows * k E4M3 codes (row-major, one byte each: sign, 4 exponent bits with bias 7, 3 fraction
 * bits) followed, at byte offset rows * k rounded up to a multiple of 256, by k / 32 planes of
 * rows rounded up to a multiple of 16 bytes: byte r of plane j is X + 127 for block j (columns
 * 32 j .. 32 j + 31) of row r, whose values are code * 2^X.  whisper_enc_mx_bytes gives the total
 * (0 for invalid sizes).  whisper_enc_mx_quantize writes the MXFP8 form of src [rows, k] (device
 * fp32, 16-byte aligned, values finite) to dst (device, 16-byte aligned, whisper_enc_mx_bytes
 * bytes, not overlapping src): X is the smallest integer with the block's largest magnitude
 * <= 448 * 2^X (-127 for an all-zero block), and each code the E4M3 value nearest to v * 2^-X,
 * ties to even; no value saturates.  Asynchronous on `stream`.
 */
size_t whisper_enc_mx_bytes(int rows, int k);
int whisper_enc_mx_quantize(const float* src, void* dst, int rows, int k, void* stream);

/* ---- Ragged batches: windows of different lengths packed back to back. ---- */

/*
 * The pages encode one window of t <= max_t rows at a time (inferencelayer
 * WhisperEncoderGpu::forward checks t against max_t), or pad every window to 30 s
 * (turbospark-runtime module doc, buffering).  Here `batch` windows of different lengths share
 * one call without padding: window b is rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1 of a packed
 * [total_rows, ...] array, and attends only within itself.
 *
 * cu_seqlens: DEVICE int32 [batch + 1], read by the kernels on `stream` (not by the host), with
 * cu_seqlens[0] = 0, non-decreasing, cu_seqlens[batch] = total_rows and every window at most
 * max_t rows.  The kernels skip a window whose entries break 0 <= cu[b] <= cu[b + 1] <=
 * total_rows or cu[b + 1] - cu[b] <= max_t, and never address rows outside [0, total_rows); the
 * output rows of a skipped window, and rows that no window covers, are unspecified.  The host
 * checks total_rows <= batch * max_t.  Zero-length windows are allowed.
 *
 * whisper_enc_varlen_workspace_bytes: workspace for whisper_enc_stack_forward_varlen (the dense
 * call's, for total_rows rows), 0 if the shape is invalid.
 */
size_t whisper_enc_varlen_workspace_bytes(int batch, int total_rows, int max_t, int d_model,
                                          int heads, int ffn_dim, int path);

/*
 * whisper_enc_stack_forward over a ragged batch: x, y [total_rows, d_model] fp32; other arguments
 * as for whisper_enc_stack_forward, with max_t in place of t for the per-window limits.
 */
int whisper_enc_stack_forward_varlen(const float* x, float* y, const void* layers, int n_layers,
                                     const float* ln_post_g, const float* ln_post_b,
                                     const int* cu_seqlens, int batch, int total_rows, int max_t,
                                     int d_model, int heads, int ffn_dim, int path,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * whisper_enc_attention over a ragged batch: row i of window b at ptr + (cu_seqlens[b] + i) * ld.
 * max_t * ld_qkv elements must span less than 2 GiB (else WENC_ERR_UNSUPPORTED).
 */
int whisper_enc_attention_varlen(const void* q, const void* k, const void* v, void* o,
                                 const int* cu_seqlens, int batch, int total_rows, int max_t,
                                 int heads, int ld_qkv, int ld_o, int path, void* stream);


/* ---- Conv front end (the step before the first block). ---- */

/*
 * Whisper's convolutional front end over mel frames (oxinfer whisper/model.rs,
 * WhisperModel::encode and conv_weight; turbospark-runtime whisper/metal.rs, encode_partial):
 *   h = gelu(conv1(mel)),  kernel 3, stride 1, padding 1      [t_mel, d]
 *   x = gelu(conv2(h)) + pos,  kernel 3, stride 2, padding 1    [ceil(t_mel / 2), d]
 * with frames as rows (a 30 s window is 3000 frames -> 1500 positions).
 *
 * whisper_enc_stem_bytes: size of the packed front end (conv weights rearranged to [cout][k][cin]
 * in the path's operand type, biases and n_pos positional rows fp32), 0 if invalid.
 */
size_t whisper_enc_stem_bytes(int n_mels, int d_model, int n_pos, int path);

/*
 * Pack it from device fp32 arrays in PyTorch layout: conv1_w [d, n_mels, 3], conv1_b [d],
 * conv2_w [d, d, 3], conv2_b [d], pos [n_pos, d].  dst: device, whisper_enc_stem_bytes() bytes,
 * 256-byte aligned.  Asynchronous on `stream`; sources must stay valid until it completes.
 */
int whisper_enc_pack_stem(const float* conv1_w, const float* conv1_b, const float* conv2_w,
                          const float* conv2_b, const float* pos, int n_mels, int d_model,
                          int n_pos, int path, void* dst, void* stream);

/* Workspace for whisper_enc_stem_forward: both unfolded inputs and h, in the operand type. */
size_t whisper_enc_stem_workspace_bytes(int batch, int t_mel, int n_mels, int d_model, int path);

/*
 * mel: [batch, t_mel, n_mels] fp32 (16-byte aligned); x: [batch, ceil(t_mel / 2), d_model] fp32,
 * distinct from mel; needs ceil(t_mel / 2) <= n_pos.  stem: from whisper_enc_pack_stem with the
 * same n_mels, d_model, n_pos and path.  workspace: device, 256-byte aligned,
 * >= whisper_enc_stem_workspace_bytes().
 */
int whisper_enc_stem_forward(const float* mel, float* x, const void* stem, int batch, int t_mel,
                             int n_mels, int d_model, int n_pos, int path, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---- Cross-attention keys and values for the decoder (the step after the encoder). ---- */

/*
 * The decoder's cross-attention projects the encoder output once per window through every
 * decoder layer's K and V weights (turbospark-runtime whisper/metal.rs, build_cross_caches;
 * oxinfer whisper/model.rs, cross_kv): for decoder layer l,
 *   K_l = y Wk_l^T   (no bias),   V_l = y Wv_l^T + bv_l,
 * stored head-major as in oxinfer's Kv ([heads][n][dh], each head's rows contiguous).
 *
 * whisper_enc_cross_kv_bytes: size of the packed weights for n_dec_layers (1..64) layers,
 * 0 if invalid.  Layout: fp32 biases [2L][d] (K rows zero) then W [2L d, d] in the path's
 * operand type, row block 2l = Wk_l, 2l + 1 = Wv_l.
 */
size_t whisper_enc_cross_kv_bytes(int d_model, int n_dec_layers, int path);

/*
 * Pack the cross K/V weights: wk, wv, bv are HOST arrays of n_dec_layers DEVICE pointers to
 * fp32 Wk_l [d, d], Wv_l [d, d] (PyTorch [n_out, n_in]) and bv_l [d].  dst: device,
 * whisper_enc_cross_kv_bytes() bytes, 256-byte aligned.  Matrices are rounded to the path's
 * operand type (nearest even).  Asynchronous on `stream`; sources must stay valid until done.
 */
int whisper_enc_pack_cross_kv(const float* const* wk, const float* const* wv,
                              const float* const* bv, int n_dec_layers, int d_model, int path,
                              void* dst, void* stream);

/* Workspace for whisper_enc_cross_kv: the 16-bit copy of y (256 bytes on the fp32 path). */
size_t whisper_enc_cross_kv_workspace_bytes(int batch, int t, int d_model, int path);

/*
 * y: [batch, t, d_model] fp32 encoder output (16-byte aligned).  kv: output, element
 * [b][l][j][h][i][e] = (j == 0 ? K_l : V_l)[b, i, 64 h + e] with b < batch, l < n_dec_layers,
 * j in {0, 1}, h < heads, i < t, e < 64, in the path's operand type (fp32 on WENC_PATH_FP32);
 * batch * n_dec_layers * 2 * t * d_model elements.  wkv: from whisper_enc_pack_cross_kv with the
 * same d_model, n_dec_layers and path.  d_model / heads must be 64.  workspace: device,
 * 256-byte aligned, >= whisper_enc_cross_kv_workspace_bytes().
 */
int whisper_enc_cross_kv(const float* y, void* kv, const void* wkv, int n_dec_layers, int batch,
                         int t, int d_model, int heads, int path, void* workspace,
                         size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WHISPER_ENC_H */
