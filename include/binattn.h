/*
 * binattn.h -- C ABI of the MI355X (gfx950) BinaryAttention forward library
 * (libbinattn.so).
 *
 * The method is the one described by the gist.science summaries of
 * "BinaryAttention: One-Bit QK-Attention for Vision and Diffusion
 * Transformers".  Queries and keys are reduced to a per-token scale times a
 * sign ("Representaciones Binarias Escaladas", technical summary section 2):
 * s_i = mu_q sign(q_i), t_j = mu_k sign(k_j).  Their similarity is an
 * XNOR/popcount count of sign agreements.  A learnable position-sensitive bias
 * b_ij is added ("Mejora mediante Sesgo").  Softmax and the product with V
 * follow inside one tiled kernel in the FlashAttention2 manner
 * ("Implementacion en Hardware").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense and row-major (ba_attention_fwd_strided and the
 *   dense-bias entries also take strided views, as they state):
 *   Q, K, V and O are bf16 [B, H, N, d].  The bias table is bf16
 *   [H, 2*gh-1, 2*gw-1].  Packed sign words are uint32 [B, H, N, W] with
 *   W = ceil(d/32).  Scales are float32 [B, H, N].
 * - All pointers are device pointers (hipMalloc'ed or equivalent) aligned to
 *   16 bytes.  The caller owns every buffer.  The library allocates no device
 *   memory at run time, frees nothing and does not synchronise, with two
 *   stated exceptions: ba_attention_bwd creates one side stream and two
 *   events per device on its first call there (see that entry), and
 *   ba_attention_fwd_static uses a fixed scratch array the library's code
 *   object carries (see that entry).
 * - stream is a hipStream_t passed as void*; NULL means the default stream.
 *   All work is enqueued on it, and the call returns before it completes.
 *   Buffers must stay valid until the stream has passed the work.
 * - Arguments are validated before anything is enqueued.  On a validation
 *   error nothing is launched and outputs are untouched.  Launch errors are
 *   reported as BA_ERR_HIP.  Faults inside kernels surface at the caller's
 *   next synchronisation, as for any HIP work.
 * - ba_last_error() returns a thread-local message for the last failing call
 *   on the calling thread.
 * - Supported head dims: 8 <= d <= 256 with d % 8 == 0.  Any other d gives
 *   BA_ERR_UNSUPPORTED.  N >= 1, B >= 1, H >= 1, and B*H*N must stay below
 *   2^31 tokens.
 *
 * Packed-sign layout (fixed; ba_pack_signs writes it and ba_qk_int_dot
 * reads it): channel c goes to word c/32, bit c%32, least significant bit
 * first.  A bit is 1 iff the channel value compares < 0, so +0.0 and -0.0
 * both give 0 (sign +1).  Bits for channels >= d are 0.
 */
#ifndef BINATTN_H
#define BINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BA_VERSION 1

/* Size of the per-device scratch of ba_attention_fwd_static, in MiB. */
#define BA_STATIC_SCRATCH_MIB 64

typedef enum ba_status {
  BA_OK = 0,
  BA_ERR_NULL = 1,        /* a required pointer is NULL                     */
  BA_ERR_SHAPE = 2,       /* inconsistent or non-positive sizes             */
  BA_ERR_UNSUPPORTED = 3, /* valid request outside what the library handles */
  BA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned               */
  BA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required     */
  BA_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed     */
} ba_status;

/* Library version (BA_VERSION of the build). */
int ba_version(void);

/* Human-readable name of a status code (static string). */
const char* ba_status_string(ba_status s);

/* Thread-local message describing the last failing call on this thread
 * (empty string if none).  Valid until the next failing call on the thread. */
const char* ba_last_error(void);

/* Number of 32-bit sign words per token, W = ceil(d/32); 0 if d < 1. */
int ba_pack_words(int d);

/* ba_pack_signs -- scaled 1-bit representation of one tensor.
 * Reduces each token x[b,h,n,:] to its scale and its signs: the scale is
 * alpha = mean over the d channels of |x| (the mu of s_i = mu sign(q_i) in
 * "Representaciones Binarias Escaladas") and the signs go into the packed
 * layout above.
 *   x      bf16  [B,H,N,d]   input (read only)
 *   bits   uint32 [B,H,N,W]  output, every word written
 *   alpha  float [B,H,N]     output; the fp32 sum over d is taken in a fixed
 *                            order, so results are deterministic (within
 *                            1e-6 relative of the exact mean for d <= 256)
 * Errors: BA_ERR_NULL, BA_ERR_SHAPE, BA_ERR_UNSUPPORTED, BA_ERR_ALIGN,
 *         BA_ERR_HIP. */
ba_status ba_pack_signs(const void* x, int64_t B, int64_t H, int64_t N, int d,
                        uint32_t* bits, float* alpha, void* stream);

/* Workspace bytes that ba_attention_fwd needs for this problem: the K signs
 * as fp4 +/-1 matrix operands (32 bytes per token and 64 channels), the K
 * scales and their maximum per 64 tokens, a key-major V^T section (per
 * head, N padded to a multiple of 128), for a bias grid with gw % 32 == 0 the
 * table rows in float32, where the prepared forward runs the pipelined
 * kernel (see ba_attention_fwd) a copy of V in its own layout [B,H,Npad,d],
 * and, for shapes the pipelined kernel takes, each K scale as three bf16
 * terms laid out as a matrix operand (12 bytes per token), and for a grid
 * whose table is written out as a dense bias (see ba_attention_fwd) that
 * bias, bf16 [H, Npad, Npad].  The queries are
 * packed inside the fused kernel.  Pass gh = gw = 0 for a
 * call without bias table.  Returns 0 for sizes the library rejects
 * (including gh*gw != N when a grid is given). */
size_t ba_workspace_bytes(int64_t B, int64_t H, int64_t N, int d, int gh, int gw);

/* ba_attention_fwd -- BinaryAttention forward.
 *   O[b,h,i,:] = sum_j P_ij V[b,h,j,:],  P = row softmax of
 *   S_ij = scale * alpha_q,i * alpha_k,j * D_ij + bias(h,i,j),
 *   D_ij = <sign q_i, sign k_j> = d - 2 popcount(qbits_i XOR kbits_j)
 * (XNOR/popcount similarity, "Representaciones Binarias Escaladas"; added
 * bias, "Mejora mediante Sesgo").  There is no masking (bidirectional
 * attention).
 *   q, k, v    bf16 [B,H,N,d]
 *   bias       bf16 [H, 2*gh-1, 2*gw-1] or NULL.  Tokens lie row-major on a
 *              gh x gw grid (token i at (i/gw, i%gw)), and
 *              bias(h,i,j) = bias[h, yi-yj+gh-1, xi-xj+gw-1], shared over b.
 *              With a table, gh*gw must equal N; without one, gh and gw are
 *              ignored.
 *   scale      softmax scale; pass 1/sqrt(d) for the standard scaling.  It
 *              must be finite and >= 0.
 *   o          bf16 [B,H,N,d] output (must not alias the inputs)
 *   workspace  device buffer of at least ba_workspace_bytes(B,H,N,d,gh,gw)
 *              bytes (gh = gw = 0 there when bias is NULL),
 *              256-byte aligned.  Its contents on entry do not matter, and it
 *              must not be shared by calls that may overlap on the GPU.
 * Two kernels are enqueued: the sign/scale pack of K (with the bias rows),
 * then the fused attention kernel, which packs Q.  For d in {32, 64, 72, 128}
 * with the table rows (gw % 32 == 0, window small enough) or no bias, the
 * fused kernel is the pipelined one, which reads V where it lies; otherwise
 * the prologue also writes V^T into the workspace for it.  For N <= 256,
 * d in {32, 64} and no table rows, one kernel does everything.  A table on
 * a grid that neither the table-row reads (gw % 32 == 0) nor the whole-table
 * reads (table <= 48 KB) take is written out by the prologue as a dense bias
 * bf16 [H, Npad, Npad] in the workspace, which the dense-bias kernel reads
 * (N up to 46336; beyond that such a table gives BA_ERR_UNSUPPORTED).
 * Errors: BA_ERR_NULL, BA_ERR_SHAPE, BA_ERR_UNSUPPORTED, BA_ERR_ALIGN,
 *         BA_ERR_WORKSPACE, BA_ERR_HIP. */
ba_status ba_attention_fwd(const void* q, const void* k, const void* v,
                           const void* bias, int gh, int gw,
                           int64_t B, int64_t H, int64_t N, int d, float scale,
                           void* o, void* workspace, size_t ws_bytes,
                           void* stream);

/* ba_attention_fwd_strided -- ba_attention_fwd on strided views, e.g. the
 * [B,N,H,d] tensors a QKV projection writes, or q, k and v as three slices
 * of one [B,N,3,H,d] tensor, without a transpose first.
 *   strides    host array of 12 int64 element strides: the (batch, head,
 *              token) strides of q, then k, then v, then o.  Row (b,h,n) of
 *              a view starts at ptr + b*sb + h*sh + n*sn elements and holds
 *              d contiguous bf16 channels.  ba_attention_fwd is this call
 *              with (H*N*d, N*d, d) for all four.
 * Every stride must be a multiple of 8 (rows stay 16-byte aligned) in
 * [0, 2^40]; a view may span at most 2^50 elements.  Input views may repeat
 * rows (stride 0 broadcasts); o's strides must keep its rows apart (taken
 * in order of increasing stride, each stride at least the extent the
 * smaller ones reach), and o's span must not overlap the spans of q, k, v or
 * the workspace.  The strides are read before the call returns.  Other
 * arguments, the workspace size and the errors are those of
 * ba_attention_fwd (BA_ERR_NULL also for strides == NULL, BA_ERR_SHAPE for
 * strides that break the rules above). */
ba_status ba_attention_fwd_strided(const void* q, const void* k, const void* v,
                                   const void* bias, int gh, int gw,
                                   int64_t B, int64_t H, int64_t N, int d, float scale,
                                   void* o, const int64_t* strides,
                                   void* workspace, size_t ws_bytes, void* stream);

/* ba_attention_fwd_dense_bias -- the forward with a dense bias: one learnable
 * value per query, key and head ("Mejora mediante Sesgo": besides the
 * position-sensitive form, the bias may be dense), in place of the
 * relative-position table:
 *   S_ij = scale * alpha_q,i * alpha_k,j * D_ij + bias(b,h,i,j)
 *   bias       bf16, bias(b,h,i,j) at bias + b*bias_sb + h*bias_sh +
 *              i*bias_ld + j elements.  bias_sb = 0 shares one [H,N,N] bias
 *              over the batch; a contiguous [B,H,N,N] tensor has
 *              (H*N*N, N*N, N).  All three strides must be multiples of 8 in
 *              [0, 2^40] (rows 16-byte aligned: pad the rows when N % 8 != 0),
 *              and (N rounded up to 128) * (bias_ld + 1) * 2 must stay below
 *              2^32 bytes.  Entries must be finite or -inf (-inf masks the
 *              key; a row whose entries are all -inf gives NaN, as softmax
 *              does).
 *   strides    as for ba_attention_fwd_strided, or NULL for contiguous
 *              [B,H,N,d] q, k, v and o.
 *   workspace  ba_workspace_bytes(B,H,N,d,0,0) bytes (no table section).
 * A dense bias has no cheap bound on its values, so the fused kernel always
 * runs the exact online softmax (running row maximum).  Two kernels are
 * enqueued, as for ba_attention_fwd.  o must not overlap the bias.
 * Errors: as ba_attention_fwd; BA_ERR_UNSUPPORTED when the bias of one head
 * spans 4 GiB or more. */
ba_status ba_attention_fwd_dense_bias(const void* q, const void* k, const void* v,
                                      const void* bias, int64_t bias_sb, int64_t bias_sh,
                                      int64_t bias_ld,
                                      int64_t B, int64_t H, int64_t N, int d, float scale,
                                      void* o, const int64_t* strides,
                                      void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes of ba_attention_fwd_int8pv: as ba_workspace_bytes, with
 * int8 value-code tiles, per-tile channel maxima, channel scales and code
 * column sums in place of the bf16 V^T copy.  0 for sizes that entry point
 * rejects (also d > 128 or N > 65536). */
size_t ba_workspace_bytes_int8pv(int64_t B, int64_t H, int64_t N, int d, int gh, int gw);

/* ba_attention_fwd_int8pv -- the forward with the pages' hybrid 8-bit P.V
 * ("Cuantizacion Hibrida": the attention coefficients, in [0, 1], take a
 * static unsigned 8-bit quantization and the values a per-channel 8-bit
 * one, with Q and K in 1 bit as in ba_attention_fwd):
 *   code_ij = round-half-even(255 exp(S_ij - max_j S_ij))   in [0, 255]
 *   s_c     = max_j |V_jc| / 127 per (b, h, channel c)
 *   vq_jc   = round-half-even(V_jc * (127 / max_j |V_jc|))  in [-127, 127]
 *   O_ic    = s_c * sum_j code_ij vq_jc / sum_j code_ij
 * S as in ba_attention_fwd.  The products and sums of codes are exact
 * (int32 on the int8 matrix cores); the coefficient codes come from a
 * float32 exp2, so one may differ by one from a float64 evaluation where
 * 255 exp(.) lies within rounding of a half-integer.
 * Arguments, layouts and errors are those of ba_attention_fwd, with
 * workspace >= ba_workspace_bytes_int8pv(B,H,N,d,gh,gw) bytes, and
 * BA_ERR_UNSUPPORTED for d > 128 or N > 65536.  Three kernels are enqueued:
 * per-tile channel maxima of |V| (with the bias rows), the K signs/scales
 * with the value codes, then the fused kernel (a pass for the row maxima,
 * then the 8-bit pass). */
ba_status ba_attention_fwd_int8pv(const void* q, const void* k, const void* v,
                                  const void* bias, int gh, int gw,
                                  int64_t B, int64_t H, int64_t N, int d, float scale,
                                  void* o, void* workspace, size_t ws_bytes,
                                  void* stream);

/* The two halves of ba_attention_fwd, for callers that time or schedule the
 * two kernels separately, or serve several queries from one K and V.
 *
 * ba_attention_prepare -- enqueues the prologue kernel: the signs and scales
 * of K ("Representaciones Binarias Escaladas"), the key-major V^T copy, a
 * copy of V in its own layout where the prepared forward runs the pipelined
 * kernel together with the K scales as its matrix operands, and, for
 * gw % 32 == 0, the float32 bias rows, all written into
 * `workspace`.  Same arguments and errors as ba_attention_fwd, without q,
 * scale and o.
 *
 * ba_attention_fwd_prepared -- enqueues only the fused kernel, which packs
 * the queries itself and reads a workspace that ba_attention_prepare filled
 * with the same bias, gh, gw, B, H, N and d (stream order must put the
 * prepare first).  The bias table is read again here when gw % 32 != 0.
 * Same arguments and errors as ba_attention_fwd, without k and v.
 *
 * The pair gives ba_attention_fwd's O bit for bit (for contiguous inputs:
 * the kernels and their arithmetic are the same; where ba_attention_fwd
 * runs one kernel for short sequences, the pair runs the two-kernel path
 * with the same arithmetic). */
ba_status ba_attention_prepare(const void* k, const void* v,
                               const void* bias, int gh, int gw,
                               int64_t B, int64_t H, int64_t N, int d,
                               void* workspace, size_t ws_bytes, void* stream);

ba_status ba_attention_fwd_prepared(const void* q, const void* bias, int gh, int gw,
                                    int64_t B, int64_t H, int64_t N, int d,
                                    float scale, void* o,
                                    const void* workspace, size_t ws_bytes,
                                    void* stream);

/* ba_attention_fwd_dense_bias_prepared -- the fused kernel of
 * ba_attention_fwd_dense_bias alone, on a workspace that
 * ba_attention_prepare(k, v, NULL, 0, 0, B, H, N, d, ...) filled (stream
 * order must put the prepare first): a prepared K/V can serve several
 * queries or biases.  q and o are contiguous [B,H,N,d]; the bias arguments,
 * the rules on them and the errors are those of ba_attention_fwd_dense_bias.
 * ba_attention_prepare followed by this call on one stream gives the same O
 * as ba_attention_fwd_dense_bias, bit for bit. */
ba_status ba_attention_fwd_dense_bias_prepared(const void* q, const void* bias,
                                               int64_t bias_sb, int64_t bias_sh, int64_t bias_ld,
                                               int64_t B, int64_t H, int64_t N, int d,
                                               float scale, void* o,
                                               const void* workspace, size_t ws_bytes,
                                               void* stream);

/* ba_attention_fwd_static -- ba_attention_fwd for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses
 * that forbid device allocation.  It takes no workspace: the library keeps
 * one scratch array of BA_STATIC_SCRATCH_MIB MiB in device memory of each
 * GPU it runs on (placed when the library's code is loaded there, held
 * until the process ends) and runs ba_attention_fwd on it.  Nothing is
 * allocated or freed by the call; its device address is looked up once per
 * device, on the first call there, with the device current.
 *   q, k, v, bias, gh, gw, B, H, N, d, scale, o, stream: as ba_attention_fwd
 *   (contiguous [B,H,N,d] tensors).
 * The scratch holds the K signs and scales and the bias rows (no V^T where
 * the pipelined kernel runs), at most BA_STATIC_SCRATCH_MIB MiB: larger
 * problems get BA_ERR_WORKSPACE before anything is enqueued.  Every call on
 * one GPU shares that GPU's scratch, so calls that may overlap on one GPU
 * (two streams, two host threads) race on it; calls in one stream do not.
 * Nothing in the scratch needs to start at zero.  O is bit for bit
 * ba_attention_fwd's.  Errors: as ba_attention_fwd, with BA_ERR_WORKSPACE
 * for problems beyond the scratch and BA_ERR_HIP if the address lookup
 * fails. */
ba_status ba_attention_fwd_static(const void* q, const void* k, const void* v,
                                  const void* bias, int gh, int gw,
                                  int64_t B, int64_t H, int64_t N, int d, float scale,
                                  void* o, void* stream);

/* Workspace bytes of ba_attention_bwd (0 for sizes it rejects; d must be
 * 32, 64 or 128). */
size_t ba_workspace_bytes_bwd(int64_t B, int64_t H, int64_t N, int d, int gh, int gw);

/* ba_attention_bwd -- gradients of ba_attention_fwd for an output gradient
 * dout (the loss L with dL/dO = dout).  The pages train BinaryAttention with
 * quantization-aware training and self-distillation ("Entrenamiento y
 * Optimizacion") but give no gradient for sign; here alpha = mean |x| takes
 * its exact derivative sign(x)/d and sign the clipped straight-through
 * estimator (derivative 1 where |x| <= 1, else 0):
 *   dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),
 *   dq~ = scale dS (alpha_k sign k),  dk~ = scale dS^T (alpha_q sign q),
 *   dx = sign(x) <sign(x), dx~> / d + alpha_x 1{|x| <= 1} dx~   (x = q, k),
 *   dtable[h, dy, dx] = sum over b and all (i, j) at that grid offset of dS.
 *   q, k, v, dout  bf16 [B,H,N,d], contiguous; d in {32, 64, 128}
 *   bias, gh, gw   as for ba_attention_fwd
 *   dq, dk, dv     float32 [B,H,N,d] outputs
 *   dtable         float32 [H, 2gh-1, 2gw-1] output, or NULL (it must be
 *                  NULL without a bias table)
 *   workspace      >= ba_workspace_bytes_bwd(B,H,N,d,gh,gw) bytes, 256-byte
 *                  aligned
 * The forward is recomputed inside (its O and row log2-sum-exp2 are kept in
 * the workspace): five kernels are enqueued, six with dtable.  With dtable
 * and N >= 1024 the key-role kernel (dk, dv) goes to a second stream that
 * the library owns on the current device (default priority, created on the
 * first such call): an event recorded on `stream` after the second prologue
 * forks it, and `stream` waits for an event recorded after it, so all of the
 * call's work still comes before later work on `stream`.  `stream` must then
 * be on the current device, else everything stays on `stream`.  dtable is
 * reduced from per-workgroup shares in a fixed order (no atomics), so it is
 * the same from run to run.  Errors: as ba_attention_fwd;
 * BA_ERR_UNSUPPORTED for other d; BA_ERR_SHAPE if dtable overlaps dq, dk, dv,
 * the inputs or the table. */
ba_status ba_attention_bwd(const void* q, const void* k, const void* v,
                           const void* bias, int gh, int gw,
                           int64_t B, int64_t H, int64_t N, int d, float scale,
                           const void* dout, float* dq, float* dk, float* dv, float* dtable,
                           void* workspace, size_t ws_bytes, void* stream);

/* ba_attention_fwd_train -- ba_attention_fwd that also writes each query
 * row's log-sum-exp, the quantity a training step keeps for the backward:
 *   lse  float32 [B,H,N] output, lse[b,h,i] = ln sum_j exp(S_ij), S as in
 *        ba_attention_fwd (natural-log units; the kernel forms it as
 *        (m_i + log2 l_i) ln 2 from its base-2 row maximum and the row sum of
 *        the bf16 P it multiplies V with, so it carries that P's rounding,
 *        about 2^-9 of l_i)
 * o is bit for bit the output of ba_attention_fwd on the same arguments.
 * lse must be 4-byte aligned and must not overlap q, k, v, o or the
 * workspace.  Other arguments and errors as ba_attention_fwd. */
ba_status ba_attention_fwd_train(const void* q, const void* k, const void* v,
                                 const void* bias, int gh, int gw,
                                 int64_t B, int64_t H, int64_t N, int d, float scale,
                                 void* o, float* lse, void* workspace, size_t ws_bytes, void* stream);

/* ba_attention_bwd_saved -- ba_attention_bwd without the recomputed forward:
 * o (bf16 [B,H,N,d], contiguous, 16-byte aligned) and lse (float32 [B,H,N],
 * 4-byte aligned) are the outputs of ba_attention_fwd_train on the same q,
 * k, v, bias and scale.  Four kernels are enqueued (five with dtable); the
 * gradients equal ba_attention_bwd's up to the rounding of lse's change of
 * units.  o and lse must not overlap the gradients or the workspace.  Other
 * arguments, the workspace (ba_workspace_bytes_bwd) and errors as
 * ba_attention_bwd. */
ba_status ba_attention_bwd_saved(const void* q, const void* k, const void* v,
                                 const void* bias, int gh, int gw,
                                 int64_t B, int64_t H, int64_t N, int d, float scale,
                                 const void* o, const float* lse,
                                 const void* dout, float* dq, float* dk, float* dv, float* dtable,
                                 void* workspace, size_t ws_bytes, void* stream);

/* QK integer-dot routes for ba_qk_int_dot. */
#define BA_ROUTE_MFMA_FP4 0 /* +/-1 in fp4 (e2m1) on the scaled f8f6f4 MFMA;
                               the route the fused kernel uses */
#define BA_ROUTE_VALU_POPCOUNT 1 /* v_xor + v_bcnt on the packed words */
#define BA_ROUTE_MFMA_INT8 2 /* +/-1 in int8 on v_mfma_i32_32x32x32_i8 */
/* OR'ed into the route: row sums instead of the N x N matrix (see below). */
#define BA_QK_ROWSUM 0x100

/* ba_qk_int_dot -- the integer similarities D_ij = <sign q_i, sign k_j> for
 * all pairs, from packed signs ("XNOR y popcount", "Representaciones
 * Binarias Escaladas").  It exists to check the fused kernel's QK step bit
 * for bit (route BA_ROUTE_MFMA_FP4 runs the same device code the fused kernel
 * uses) and to time the three ways of taking these dots against each other.
 *   qbits, kbits  uint32 [B,H,N,W] in the packed layout
 *   route         BA_ROUTE_*, optionally | BA_QK_ROWSUM
 *   dots          int32 [B,H,N,N] output, dots[b,h,i,j] = D_ij; with
 *                 BA_QK_ROWSUM int32 [B,H,N], dots[b,h,i] = sum_j D_ij (each
 *                 workgroup shares 64-key tiles in LDS across 128 queries, as
 *                 the fused kernel does, so the time is the route's arithmetic)
 * Errors: BA_ERR_NULL, BA_ERR_SHAPE (also if B*H*N*N overflows int64 or
 *         exceeds 2^40 elements without BA_QK_ROWSUM), BA_ERR_UNSUPPORTED
 *         (unknown route or d), BA_ERR_ALIGN, BA_ERR_HIP. */
ba_status ba_qk_int_dot(const uint32_t* qbits, const uint32_t* kbits,
                        int64_t B, int64_t H, int64_t N, int d, int route,
                        int32_t* dots, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BINATTN_H */
